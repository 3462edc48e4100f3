// lmhead_api.hip — host side of the C ABI declared in include/lmhead.h:
// argument validation, the workspace plan and the launch sequence of each
// entry. Host-checkable errors return before anything is enqueued; nothing
// here allocates device memory or synchronises (except
// lmhead_read_device_error).
#include <limits.h>
#include <string.h>

#include <atomic>
#include <functional>
#include <mutex>
#include <queue>
#include <vector>

#include <hip/hip_runtime.h>

#include "lmhead.h"
#include "lmhead_kernels.h"

namespace {

using namespace lmhead;

constexpr int64_t kMaxRows = int64_t(1) << 30;
constexpr int64_t kMaxVocab = int64_t(1) << 30;
constexpr int64_t kMaxHidden = 65536;
// Widest padded chunk, round_up(min(chunk, vocab), 256): dL/dz is the K-major
// operand of the dH contraction with a row pitch of that width, and a tile's
// buffer range (256 rows of it, in bytes) must stay below 2^31.
constexpr int64_t kMaxChunkPad = (int64_t(1) << 22) - 256;
constexpr int64_t kMaxWorkItems = 0xffffffffLL;   // work-items in one launch
// Most K slices of a chunk's dH contraction (bounds the fp32 partials)
constexpr int kMaxDhSlices = 16;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

// Per-tile candidate buckets of the dense support entry (hit_count_kernel):
// one set in the forward's regions and one in the backward's.
struct HitRegions {
    size_t counts, cursor, offsets, tsum, tprefix, list, sort_tmp, large, n_large;
};

struct Layout {
    int64_t n, n_pad, hidden, vocab, chunk, w_pad, tiles_v, k;
    HitRegions hit_fwd, hit_bwd;
    // forward regions (hfrag_fwd: H in MFMA fragment order, n_pad rows)
    size_t hdr, lse, part, zg, rows, hfrag_fwd;
    size_t hfrag_bwd;                 // the backward's own copy (workspace contents do not survive calls)
    size_t htfrag;                    // backward: H^T in fragment order, [n_pad / 32][hid_pad / 16] blocks
    int64_t hfrag_bytes, htfrag_bytes, hid_pad;
    int64_t group;    // chunks per recompute launch (grad_group)
    int64_t g_cols;   // columns of the dL/dz region (grad_cols, or a dH pass's columns)
    bool dh_pass;     // kDhPass consecutive chunks share one dH pass (shared_dh_pass)
    // backward regions
    size_t coef_a, coef_c, G, dh_acc;
    size_t dh_part;   // fp32 partial dH tiles of the K-split (few row tiles only)
    int64_t dh_part_bytes;
    // backward of the KL-only entry: inverse index of the candidate ids
    size_t counts, offsets, cursor, list, sort_tmp, tsum, tprefix, large, n_large, pieces, piece_off, partial;
    size_t fwd_total, bwd_total;
};

bool is_support(int entry) { return entry == LMHEAD_ENTRY_SUPPORT || entry == LMHEAD_ENTRY_SUPPORT_KL; }

int validate_problem(const lmhead_problem* p, int entry) {
    if (p == nullptr) return LMHEAD_ERR_ARG;
    if (entry < LMHEAD_ENTRY_CE_MEAN || entry > LMHEAD_ENTRY_SUPPORT_KL) return LMHEAD_ERR_ARG;
    if ((p->flags & ~LMHEAD_FLAG_PADDED_IDS) != 0 || p->reserved != 0) return LMHEAD_ERR_ARG;
    if ((p->flags & LMHEAD_FLAG_PADDED_IDS) && !is_support(entry)) return LMHEAD_ERR_ARG;
    // scalar temperature: 0 (off) or positive and finite
    if (!(p->temperature >= 0.0f && p->temperature <= 3.402823466e38f)) return LMHEAD_ERR_ARG;
    if (p->n < 0 || p->n > kMaxRows) return LMHEAD_ERR_SHAPE;
    if (p->hidden < 64 || p->hidden > kMaxHidden || p->hidden % 64 != 0) return LMHEAD_ERR_SHAPE;
    if (p->vocab < 1 || p->vocab > kMaxVocab) return LMHEAD_ERR_SHAPE;
    if (p->chunk < 256 || p->chunk % 256 != 0 || p->chunk > kMaxVocab + 256) return LMHEAD_ERR_SHAPE;
    if (p->num_valid < -1) return LMHEAD_ERR_SHAPE;
    if (is_support(entry) && (p->k < 1 || p->k > kMaxCandidates)) return LMHEAD_ERR_SHAPE;
    // both support entries index (row, candidate) entries with int32: the
    // KL-only entry's inverse index, the dense entry's per-tile buckets and
    // their offset scans
    if (is_support(entry) && p->n * (int64_t)p->k > INT_MAX) return LMHEAD_ERR_SHAPE;
    // every entry with a vocabulary-wide pass: the backward's chunk width
    if (entry != LMHEAD_ENTRY_SUPPORT_KL &&
        round_up(p->chunk < p->vocab ? p->chunk : p->vocab, kTile) > kMaxChunkPad)
        return LMHEAD_ERR_SHAPE;
    // A launch holds at most 2^32 - 1 work-items (the dispatch's grid size is
    // a 32-bit count). The support entries' per-row kernels run 64 threads per
    // row (n_pad rows), the other entries' at most 8; the KL-only entry's dW
    // pass runs 64 per vocabulary id; every other entry runs one 256-thread
    // workgroup per 256 x 256 tile of rows x vocabulary (forward, recompute)
    // and of rows x hidden (dH). The other launches have capped grids.
    const int64_t n_pad = round_up(p->n, kTile);
    if ((is_support(entry) ? 64 : 8) * n_pad > kMaxWorkItems) return LMHEAD_ERR_SHAPE;
    if (entry == LMHEAD_ENTRY_SUPPORT_KL) {
        if (64 * round_up(p->vocab, 4) > kMaxWorkItems) return LMHEAD_ERR_SHAPE;
    } else {
        const int64_t tv = cdiv(p->vocab, kTile), th = cdiv(p->hidden, kTile);
        if (cdiv(p->n, kTile) * (tv > th ? tv : th) * kThreads > kMaxWorkItems) return LMHEAD_ERR_SHAPE;
    }
    return LMHEAD_OK;
}

constexpr int kComputeUnits = 256;
int dh_slices(int64_t n, int64_t n_pad, int64_t hidden, int64_t w_pad);
int64_t dh_units(int64_t n_pad, int64_t hidden);
struct DhGroupPlan {
    int64_t slices, batch;
};
DhGroupPlan dh_group_plan(int64_t n_pad, int64_t hidden, int64_t w_pad, int64_t group);

// Columns of the dL/dz region: one chunk, or, when the chunks are narrower,
// the compute units' worth of 256 x 256 tiles (2^24 / n_pad columns) but no
// more than the whole vocabulary. It never shrinks as the chunk widens, so
// the workspace grows with the chunk and the 256-column chunk needs least.
int64_t grad_cols(int64_t n_pad, int64_t w_pad, int64_t vocab) {
    const int64_t all = round_up(vocab, kTile);
    const int64_t units = (int64_t)kComputeUnits * kTile * kTile / n_pad;
    const int64_t c = all < units ? all : units;
    return c > w_pad ? c : w_pad;
}

// Chunks whose dL/dz one recompute launch writes. A chunk of few 256 x 256
// tiles (small batches) leaves most compute units idle, so consecutive
// chunks share a launch, up to one workgroup per compute unit, each into a
// slot of its own within the grad_cols columns; dW and dH then take the
// group's chunks in order and sum each output element exactly as they would
// one chunk at a time.
int64_t grad_group(int64_t n_pad, int64_t w_pad, int64_t vocab, int64_t chunk) {
    const int64_t tiles = (n_pad / kTile) * (w_pad / kTile);
    int64_t g = tiles >= kComputeUnits ? 1 : kComputeUnits / tiles;
    const int64_t fit = grad_cols(n_pad, w_pad, vocab) / w_pad;
    const int64_t nchunks = cdiv(vocab, chunk);
    g = g < fit ? g : fit;
    g = g < nchunks ? g : nchunks;
    return g > 1 ? g : 1;
}

// Four consecutive chunks share one dH pass when each chunk has enough dH
// tiles to fill the compute units by itself (no K-split): chunks 4p .. 4p + 3
// keep their dL/dz side by side in one region of the pass's columns, each
// chunk's dW runs after its recompute as usual, and after the pass's last
// recompute one dH contraction runs over all of the pass's columns (W rows
// v0 .. v0 + 4 chunk are contiguous, and an accepted chunk is a multiple of
// 256 columns, so the region's columns are the W rows in order). The fp32
// running sum of dH is then read and written once per pass instead of once
// per chunk; the vocabulary's last pass may hold fewer chunks. A pass's dH
// sum is one K loop over ascending columns, i.e. what a chunk four times as
// wide would sum; forward outputs and dW are unchanged.
// dh_pass_cols: the region a pass needs, min(4 padded chunks, V, the widest
// accepted chunk), sized whenever the dH tiles alone fill the units (also for
// a chunk too wide to share a pass), so that the workspace never shrinks as
// the chunk widens. Both depend on the shape alone.
constexpr int64_t kDhPass = 4;   // chunks per dH pass where they share one
bool dh_fills_units(int64_t n_pad, int64_t hidden) {
    return (n_pad / kTile) * cdiv(hidden, kTile) >= kComputeUnits;
}
int64_t dh_pass_cols(int64_t n_pad, int64_t hidden, int64_t vocab, int64_t w_pad) {
    if (!dh_fills_units(n_pad, hidden)) return 0;
    int64_t c = kDhPass * w_pad;
    const int64_t all = round_up(vocab, kTile);
    c = c < all ? c : all;
    return c < kMaxChunkPad ? c : kMaxChunkPad;
}
bool shared_dh_pass(int64_t n_pad, int64_t hidden, int64_t vocab, int64_t chunk, int64_t group) {
    return group == 1 && dh_fills_units(n_pad, hidden) && chunk < vocab && kDhPass * chunk <= kMaxChunkPad;
}

Layout plan(const lmhead_problem& p, int entry) {
    Layout L{};
    L.n = p.n;
    L.n_pad = round_up(p.n > 0 ? p.n : 1, kTile);
    L.hidden = p.hidden;
    L.vocab = p.vocab;
    L.chunk = p.chunk;
    L.w_pad = round_up(p.chunk < p.vocab ? p.chunk : p.vocab, kTile);
    L.tiles_v = cdiv(p.vocab, kTile);
    L.k = is_support(entry) ? p.k : 1;
    size_t off = 0;
    auto take = [&off](int64_t bytes) {
        const size_t o = off;
        off += (size_t)round_up(bytes > 0 ? bytes : 0, 256);
        return o;
    };
    L.hdr = take(256);
    const size_t after_hdr = off;
    if (entry == LMHEAD_ENTRY_SUPPORT_KL) {
        // no vocabulary-wide pass: the forward needs only the header
        L.fwd_total = off;
        L.coef_a = take(4 * L.n_pad);
        L.coef_c = take(4 * L.n * L.k);
        L.counts = take(4 * L.vocab);
        L.offsets = take(4 * (L.vocab + 1));
        L.cursor = take(4 * L.vocab);
        L.list = take(4 * L.n * L.k);
        L.sort_tmp = take(4 * L.n * L.k);
        L.tsum = take(4 * cdiv(L.vocab, kScanTile));
        L.tprefix = take(4 * (cdiv(L.vocab, kScanTile) + 1));
        L.large = take(4 * L.vocab);
        L.n_large = take(4);
        // split pieces of large dW buckets: at most 2 N k / kDwSplitEntries of them
        L.pieces = take(4 * L.vocab);
        L.piece_off = take(4 * (L.vocab + 1));
        L.partial = take(4 * (2 * L.n * L.k / kDwSplitEntries + 1) * L.hidden);
        L.bwd_total = off;
        return L;
    }
    const bool buckets = entry == LMHEAD_ENTRY_SUPPORT;
    const int64_t nb = (L.n_pad / kTile) * L.tiles_v;
    auto take_hits = [&](HitRegions& R) {
        R.counts = take(4 * nb);
        R.cursor = take(4 * nb);
        R.offsets = take(4 * (nb + 1));
        R.tsum = take(4 * cdiv(nb, kScanTile));
        R.tprefix = take(4 * (cdiv(nb, kScanTile) + 1));
        R.list = take(4 * L.n * L.k);
        R.sort_tmp = take(4 * L.n * L.k);
        R.large = take(4 * nb);
        R.n_large = take(4);
    };
    L.hfrag_bytes = 2 * L.n_pad * L.hidden;
    L.hfrag_fwd = take(L.hfrag_bytes);
    L.lse = take(4 * L.n);
    L.part = take(8 * L.tiles_v * L.n);
    L.zg = take(4 * L.n * L.k);
    L.rows = take(4 * L.n);
    if (buckets) take_hits(L.hit_fwd);
    L.fwd_total = off;
    off = after_hdr;
    L.hfrag_bwd = take(L.hfrag_bytes);
    L.hid_pad = round_up(L.hidden, kTile);
    L.htfrag_bytes = 2 * L.n_pad * L.hid_pad;
    L.htfrag = take(L.htfrag_bytes);
    L.coef_a = take(4 * L.n_pad);
    L.coef_c = take(4 * L.n * L.k);
    L.group = grad_group(L.n_pad, L.w_pad, L.vocab, L.chunk);
    L.g_cols = grad_cols(L.n_pad, L.w_pad, L.vocab);
    L.dh_pass = shared_dh_pass(L.n_pad, L.hidden, L.vocab, L.chunk, L.group);
    {
        const int64_t pc = dh_pass_cols(L.n_pad, L.hidden, L.vocab, L.w_pad);
        L.g_cols = pc > L.g_cols ? pc : L.g_cols;
    }
    L.G = take(2 * L.n_pad * L.g_cols);
    L.dh_acc = take(4 * L.n * L.hidden);
    {
        // the K-split's partials, whatever the chunk: every split (one chunk's
        // slices, or a group's chunks x slices) takes at most dh_units planes
        const int64_t units = L.n > 0 ? dh_units(L.n_pad, L.hidden) : 0;
        L.dh_part_bytes = units > 1 ? 4 * units * L.n * L.hidden : 0;
        L.dh_part = take(L.dh_part_bytes);
    }
    if (buckets) take_hits(L.hit_bwd);
    L.bwd_total = off > L.fwd_total ? off : L.fwd_total;
    return L;
}

bool aligned(const void* ptr, uintptr_t a) { return ((uintptr_t)ptr % a) == 0; }

Temperature temperature_of(const lmhead_problem& p) {
    Temperature T;
    T.t = p.temperature == 0.0f ? 1.0f : p.temperature;
    T.row = p.row_temperature;
    return T;
}

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return LMHEAD_ERR_DEVICE;
    // 0 unknown, 1 gfx950, 2 other; atomic so that threads calling at once on
    // different devices (or the same one) neither race nor tear
    static std::atomic<int> cache[256];
    if (dev < 256) {
        const int known = cache[dev].load(std::memory_order_relaxed);
        if (known != 0) return known == 1 ? LMHEAD_OK : LMHEAD_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return LMHEAD_ERR_DEVICE;
    const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 256) cache[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? LMHEAD_OK : LMHEAD_ERR_DEVICE;
}

int launched() { return hipGetLastError() == hipSuccess ? LMHEAD_OK : LMHEAD_ERR_HIP; }

// The dW and dH contractions of a chunk run as two launches, or as one when
// that finishes sooner: a launch whose last round of 256 x 256 tiles leaves
// compute units idle can lend them to the other kind. Estimated in units of
// one K step of one tile, with one workgroup per compute unit and workgroups
// starting in launch order on the first free unit (the MI355X has 256
// compute units; the choice changes only the schedule, never a result).
// workgroups of bucket_sort_block_kernel (each loops over the listed large buckets)
constexpr int kSortBlocks = 512;
// workgroups of the split dW kernels (each loops over its share of the pieces / buckets)
constexpr int kSplitBlocks = 1024;

int64_t rounds_time(int64_t tiles, int64_t steps) { return cdiv(tiles, kComputeUnits) * steps; }

int64_t list_time(int64_t n1, int64_t s1, int64_t n2, int64_t s2) {
    // finish times of the units, kept sorted: n1 tiles of s1 steps, then n2 of s2
    std::vector<int64_t> free_at((size_t)kComputeUnits, 0);
    std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>> q(free_at.begin(), free_at.end());
    int64_t end = 0;
    auto run = [&](int64_t n, int64_t steps) {
        for (int64_t i = 0; i < n; ++i) {
            const int64_t t = q.top() + steps;
            q.pop();
            q.push(t);
            end = t > end ? t : end;
        }
    };
    run(n1, s1);
    run(n2, s2);
    return end;
}

// 1: one launch with the dH tiles first, 0: one launch with the dW tiles
// first, -1: two launches. One launch unless the estimate makes it longer:
// at a tie (both kinds filling whole rounds) it still saves a launch
// boundary, and the second kind's tiles start on the units the first kind's
// last round frees.
int dwdh_plan(int64_t n_dw, int64_t k_dw, int64_t n_dh, int64_t k_dh) {
    // with many rounds the last one's idle units matter little: keep two launches
    if (n_dw == 0 || n_dh == 0 || n_dw + n_dh > 16 * kComputeUnits) return -1;
    const int64_t apart = rounds_time(n_dw, k_dw) + rounds_time(n_dh, k_dh);
    const bool dh_first = k_dh >= k_dw;   // longer tiles first
    const int64_t together = dh_first ? list_time(n_dh, k_dh, n_dw, k_dw) : list_time(n_dw, k_dw, n_dh, k_dh);
    return together <= apart ? (dh_first ? 1 : 0) : -1;
}

// fp32 partial dH planes of the K-split (below 2: no split): one per (chunk,
// slice) unit a launch computes, at most 16 and at most one workgroup per
// compute unit over all of them (units x dH tiles <= 256), so the partials
// never exceed 256 tiles of 256 x 256 fp32 (64 MiB). Depends on n and hidden
// alone.
int64_t dh_units(int64_t n_pad, int64_t hidden) {
    const int64_t n_dh = (n_pad / kTile) * cdiv(hidden, kTile);
    const int64_t u = kComputeUnits / n_dh;
    return u < kMaxDhSlices ? u : kMaxDhSlices;
}

// The grouped dH K-split (several chunks per recompute launch): each chunk
// of the group is cut into `slices` equal K ranges (a power of two dividing
// a full chunk's K steps, at least 8 steps each) and `batch` chunks go to
// one launch, so that slices x chunks fills the units (dh_units) and each
// workgroup runs as many K steps as that allows. slices = 0: no split (one
// dH launch per chunk). Depends on the shape and the group alone.
DhGroupPlan dh_group_plan(int64_t n_pad, int64_t hidden, int64_t w_pad, int64_t group) {
    const int64_t units = dh_units(n_pad, hidden);
    if (units < 2) return {0, 0};
    const int64_t kt = w_pad / kTileK;
    int64_t sl = 1;
    while (2 * sl * group <= units && kt % (2 * sl) == 0 && kt / (2 * sl) >= 8) sl *= 2;
    return {sl, units / sl};
}

// K slices of a chunk's dH contraction (1: no split). With few dH tiles
// (small batches) each one runs all of the chunk's K steps while most compute
// units idle; cutting the chunk's columns into S equal slices (S a power of
// two dividing the K steps, at least 8 steps each, S <= dh_units) gives S times the tiles,
// whose fp32 partials dh_join_kernel adds in slice order. Chosen from the
// same estimate as dwdh_plan, plus two steps per tile for the prologue and
// the partial's store and the join's HBM traffic at 8 MB per step (one K step
// of one tile is about 1.7 us), only where it saves at least 5 %. It depends
// on the shape alone (dW wanted or not), so one shape always sums in one order.
int dh_slices(int64_t n, int64_t n_pad, int64_t hidden, int64_t w_pad) {
    const int64_t n_dh = (n_pad / kTile) * cdiv(hidden, kTile);
    const int64_t units = dh_units(n_pad, hidden);
    if (n <= 0 || units < 2) return 1;
    const int64_t n_dw = (w_pad / kTile) * cdiv(hidden, kTile), k_dw = n_pad / kTileK;
    const int64_t kt = w_pad / kTileK;
    const int one = dwdh_plan(n_dw, k_dw, n_dh, kt);
    const int64_t base = one < 0 ? rounds_time(n_dw, k_dw) + rounds_time(n_dh, kt)
                                 : (one == 1 ? list_time(n_dh, kt, n_dw, k_dw) : list_time(n_dw, k_dw, n_dh, kt));
    int best = 1;
    int64_t best_t = base;
    for (int64_t sl = 2; sl <= units && kt % sl == 0 && kt / sl >= 8; sl *= 2) {
        const int64_t join = cdiv((sl + 2) * n * hidden * 4, (int64_t)8 << 20);
        const int64_t t = rounds_time(n_dw, k_dw) + rounds_time(n_dh * sl, kt / sl + 2) + join;
        if (t * 20 <= base * 19 && t < best_t) {
            best = (int)sl;
            best_t = t;
        }
    }
    return best;
}

int grid_1d(int64_t items, int per_block, int cap) {
    int64_t g = cdiv(items, per_block);
    if (g < 1) g = 1;
    return (int)(g < cap ? g : cap);
}

void fill_u32(void* p, int64_t count, uint32_t value, hipStream_t s) {
    if (count <= 0) return;
    fill_u32_kernel<<<grid_1d(count, kThreads, 4096), kThreads, 0, s>>>((uint32_t*)p, count, value);
}

// The dense support entry's per-tile candidate buckets: bucket (row tile,
// vocabulary tile) lists its (row, column, slot) hits in ascending order.
// Counting uses integer atomics only; the scan and the per-bucket sort make
// the result independent of their order.
void build_hits(const Layout& L, const HitRegions& R, char* w, const int32_t* ids, hipStream_t s,
                const int32_t** offsets_out, const int32_t** list_out) {
    const int64_t nb = (L.n_pad / kTile) * L.tiles_v;
    int32_t* counts = (int32_t*)(w + R.counts);
    int32_t* cursor = (int32_t*)(w + R.cursor);
    int32_t* offsets = (int32_t*)(w + R.offsets);
    int32_t* tsum = (int32_t*)(w + R.tsum);
    int32_t* tprefix = (int32_t*)(w + R.tprefix);
    int32_t* list = (int32_t*)(w + R.list);
    fill_u32(counts, nb, 0u, s);
    fill_u32(cursor, nb, 0u, s);
    const int64_t nk = L.n * L.k;
    hit_count_kernel<<<grid_1d(nk, kThreads, 4096), kThreads, 0, s>>>(ids, L.n, (int)L.k, L.vocab, L.tiles_v,
                                                                      counts);
    const int64_t tiles = cdiv(nb, kScanTile);
    tile_sums_kernel<<<(unsigned)tiles, 256, 0, s>>>(counts, nb, tsum);
    exclusive_scan_kernel<<<1, 1024, 0, s>>>(tsum, tiles, tprefix);
    scan_tiles_kernel<<<(unsigned)tiles, 256, 0, s>>>(counts, nb, tprefix, tiles, offsets);
    hit_fill_kernel<<<grid_1d(nk, kThreads, 4096), kThreads, 0, s>>>(ids, L.n, (int)L.k, L.vocab, L.tiles_v,
                                                                     offsets, cursor, list);
    int32_t* large = (int32_t*)(w + R.large);
    int32_t* n_large = (int32_t*)(w + R.n_large);
    fill_u32(n_large, 1, 0u, s);
    bucket_sort_wave_kernel<<<(unsigned)cdiv(nb, kThreads / 64), kThreads, 0, s>>>(offsets, nb, list, large,
                                                                                  n_large);
    bucket_sort_block_kernel<<<kSortBlocks, 1024, 0, s>>>(offsets, list, (int32_t*)(w + R.sort_tmp), large,
                                                          n_large);
    *offsets_out = offsets;
    *list_out = list;
}

// Validation shared by the three forward entries.
int forward(const lmhead_problem* p, int entry, const void* H, const void* W, const int32_t* ids,
            const float* ref_logq, float* row_out, float* kl, float* lse_out, float* loss,
            void* ws, size_t ws_bytes, void* stream) {
    int st = validate_problem(p, entry);
    if (st != LMHEAD_OK) return st;
    const bool ce = entry == LMHEAD_ENTRY_CE_MEAN || entry == LMHEAD_ENTRY_CE_SUM;
    if (ws == nullptr) return LMHEAD_ERR_ARG;
    if (ce && loss == nullptr) return LMHEAD_ERR_ARG;
    if (p->n > 0) {
        if (H == nullptr || W == nullptr || ids == nullptr) return LMHEAD_ERR_ARG;
        if (!ce && row_out == nullptr) return LMHEAD_ERR_ARG;
    }
    if (kl != nullptr && ref_logq == nullptr) return LMHEAD_ERR_ARG;
    if (!aligned(H, 16) || !aligned(W, 16) || !aligned(ws, 256) || !aligned(p->row_temperature, 4))
        return LMHEAD_ERR_ALIGN;
    const Layout L = plan(*p, entry);
    if (ws_bytes < L.fwd_total) return LMHEAD_ERR_WORKSPACE;
    const Temperature T = temperature_of(*p);
    st = check_device();
    if (st != LMHEAD_OK) return st;

    hipStream_t s = (hipStream_t)stream;
    char* w = (char*)ws;
    int32_t* hdr = (int32_t*)(w + L.hdr);
    init_header_kernel<<<1, 64, 0, s>>>(hdr);
    if (L.n == 0) {
        if (loss) fill_u32(loss, 1, 0u, s);
        return launched();
    }
    const int padded = (p->flags & LMHEAD_FLAG_PADDED_IDS) ? 1 : 0;
    const int mode = entry == LMHEAD_ENTRY_SUPPORT ? 1 + padded : 0;
    scan_labels_kernel<<<grid_1d(L.n, kThreads, 1024), kThreads, 0, s>>>(ids, L.n, (int)L.k, L.vocab,
                                                                          mode, T, hdr);
    frag_pack_kernel<<<grid_1d(L.n_pad * L.hidden / 8, kThreads, 8192), kThreads, 0, s>>>(
        (const bf16_bits*)H, L.n, L.hidden, L.n_pad, (bf16_bits*)(w + L.hfrag_fwd));
    FwdTilesArgs fa;
    fa.T = T;
    fa.Hf = (const bf16_bits*)(w + L.hfrag_fwd);
    fa.W = (const bf16_bits*)W;
    fa.n = L.n;
    fa.hidden = L.hidden;
    fa.vocab = L.vocab;
    fa.tiles_m = cdiv(L.n, kTile);
    fa.tiles_n = L.tiles_v;
    fa.ids = ids;
    fa.k = (int)L.k;
    fa.part = (float2*)(w + L.part);
    fa.zg = (float*)(w + L.zg);
    fa.hit_offsets = nullptr;
    fa.hit_list = nullptr;
    if (entry == LMHEAD_ENTRY_SUPPORT) build_hits(L, L.hit_fwd, w, ids, s, &fa.hit_offsets, &fa.hit_list);
    fwd_tiles_kernel<<<(unsigned)(fa.tiles_m * fa.tiles_n), kThreads, 0, s>>>(fa);

    FinalizeArgs fin;
    fin.T = T;
    fin.part = fa.part;
    fin.n = L.n;
    fin.tiles_n = L.tiles_v;
    fin.vocab = L.vocab;
    fin.ids = ids;
    fin.k = (int)L.k;
    fin.entry = entry;
    fin.zg = fa.zg;
    fin.ref_logq = ref_logq;
    fin.lse = lse_out != nullptr ? lse_out : (float*)(w + L.lse);
    fin.row_out = ce ? (float*)(w + L.rows) : row_out;
    fin.kl = kl;
    fin.padded = padded;
    finalize_rows_kernel<<<grid_1d(L.n * 8, kThreads, INT_MAX), kThreads, 0, s>>>(fin);   // 8 lanes per row
    if (ce)
        ce_reduce_kernel<<<1, kThreads, 0, s>>>(fin.row_out, L.n, hdr, p->num_valid,
                                                entry == LMHEAD_ENTRY_CE_MEAN ? 1 : 0, loss);
    return launched();
}

// The backward of both entry points. dH_acc / dW_acc: the caller's fp32
// accumulators (null for the plain backward, where dH / dW are the results).
int backward(const lmhead_problem* p, int entry, const void* H, const void* W, const int32_t* ids,
             const float* ref_logq, const float* lse, const float* saved_lp, const float* grad,
             const float* grad_kl, void* dH, void* dW, float* dH_acc, float* dW_acc, void* workspace,
             size_t workspace_bytes, void* stream) {
    int st = validate_problem(p, entry);
    if (st != LMHEAD_OK) return st;
    const bool support = is_support(entry);
    const bool kl_only = entry == LMHEAD_ENTRY_SUPPORT_KL;
    if (workspace == nullptr) return LMHEAD_ERR_ARG;
    if (kl_only && grad != nullptr) return LMHEAD_ERR_ARG;   // the KL-only entry has no lp output
    if (p->n > 0) {
        if (H == nullptr || W == nullptr || ids == nullptr) return LMHEAD_ERR_ARG;
        if (!kl_only && lse == nullptr) return LMHEAD_ERR_ARG;
        if (!support && grad == nullptr) return LMHEAD_ERR_ARG;
        if (support && grad_kl != nullptr && (ref_logq == nullptr || saved_lp == nullptr))
            return LMHEAD_ERR_ARG;
    }
    if (!aligned(H, 16) || !aligned(W, 16) || !aligned(dH, 16) || !aligned(dW, 16) ||
        !aligned(dH_acc, 16) || !aligned(dW_acc, 16) || !aligned(workspace, 256) ||
        !aligned(p->row_temperature, 4))
        return LMHEAD_ERR_ALIGN;
    const Layout L = plan(*p, entry);
    if (workspace_bytes < L.bwd_total) return LMHEAD_ERR_WORKSPACE;
    const Temperature T = temperature_of(*p);
    st = check_device();
    if (st != LMHEAD_OK) return st;
    const bool want_dh = dH != nullptr || dH_acc != nullptr;
    const bool want_dw = dW != nullptr || dW_acc != nullptr;
    if (!want_dh && !want_dw) return LMHEAD_OK;

    hipStream_t s = (hipStream_t)stream;
    char* w = (char*)workspace;
    int32_t* hdr = (int32_t*)(w + L.hdr);
    init_header_kernel<<<1, 64, 0, s>>>(hdr);
    if (L.n == 0) {
        // dL/dW = 0: the plain result is zero, an accumulator is unchanged
        if (dW != nullptr && dW_acc == nullptr) fill_u32(dW, L.vocab * L.hidden / 2, 0u, s);
        if (dW != nullptr && dW_acc != nullptr)
            f32_to_bf16_kernel<<<grid_1d(L.vocab * L.hidden / 2, kThreads, 4096), kThreads, 0, s>>>(
                dW_acc, L.vocab * L.hidden, (bf16_bits*)dW);
        return launched();
    }
    const int padded = (p->flags & LMHEAD_FLAG_PADDED_IDS) ? 1 : 0;
    scan_labels_kernel<<<grid_1d(L.n, kThreads, 1024), kThreads, 0, s>>>(ids, L.n, (int)L.k, L.vocab,
                                                                          support ? 1 + padded : 0, T, hdr);
    CoeffArgs ca;
    ca.T = T;
    ca.entry = support ? LMHEAD_ENTRY_SUPPORT : entry;
    ca.padded = padded;
    ca.n = L.n;
    ca.n_pad = L.n_pad;
    ca.vocab = L.vocab;
    ca.k = (int)L.k;
    ca.ids = ids;
    ca.ref_logq = ref_logq;
    ca.saved_lp = saved_lp;
    ca.grad = grad;
    ca.grad_kl = (support && ref_logq != nullptr && saved_lp != nullptr) ? grad_kl : nullptr;
    ca.hdr = hdr;
    ca.num_valid = p->num_valid;
    ca.coef_a = (float*)(w + L.coef_a);
    ca.coef_c = (float*)(w + L.coef_c);
    if (support)
        coeffs_support_kernel<<<(unsigned)cdiv(L.n_pad, kThreads / 64), kThreads, 0, s>>>(ca);
    else
        coeffs_kernel<<<grid_1d(L.n_pad, kThreads, INT_MAX), kThreads, 0, s>>>(ca);
    if (kl_only) {
        // dL/dz is nonzero only at the candidates: gathers instead of contractions
        CandBwdArgs cb;
        cb.H = (const bf16_bits*)H;
        cb.W = (const bf16_bits*)W;
        cb.n = L.n;
        cb.hidden = L.hidden;
        cb.vocab = L.vocab;
        cb.k = (int)L.k;
        cb.ids = ids;
        cb.coef_c = ca.coef_c;
        cb.dH = (bf16_bits*)dH;
        cb.dH_acc = dH_acc;
        cb.dW = (bf16_bits*)dW;
        cb.dW_acc = dW_acc;
        int32_t* counts = (int32_t*)(w + L.counts);
        int32_t* offsets = (int32_t*)(w + L.offsets);
        int32_t* cursor = (int32_t*)(w + L.cursor);
        int32_t* list = (int32_t*)(w + L.list);
        cb.offsets = offsets;
        cb.list = list;
        const unsigned row_blocks = (unsigned)cdiv(L.n, kThreads / 64);
        if (want_dh) cand_dh_kernel<<<row_blocks, kThreads, 0, s>>>(cb);
        if (want_dw) {
            const int64_t nk = L.n * L.k;
            fill_u32(counts, L.vocab, 0u, s);
            fill_u32(cursor, L.vocab, 0u, s);
            cand_count_kernel<<<grid_1d(nk, kThreads, 4096), kThreads, 0, s>>>(ids, nk, L.vocab, counts);
            const int64_t tiles = cdiv(L.vocab, kScanTile);
            int32_t* tsum = (int32_t*)(w + L.tsum);
            int32_t* tprefix = (int32_t*)(w + L.tprefix);
            tile_sums_kernel<<<(unsigned)tiles, 256, 0, s>>>(counts, L.vocab, tsum);
            exclusive_scan_kernel<<<1, 1024, 0, s>>>(tsum, tiles, tprefix);
            scan_tiles_kernel<<<(unsigned)tiles, 256, 0, s>>>(counts, L.vocab, tprefix, tiles, offsets);
            cand_fill_kernel<<<grid_1d(nk, kThreads, 4096), kThreads, 0, s>>>(ids, nk, L.vocab, offsets,
                                                                              cursor, list);
            int32_t* large = (int32_t*)(w + L.large);
            int32_t* n_large = (int32_t*)(w + L.n_large);
            fill_u32(n_large, 1, 0u, s);
            bucket_sort_kernel<<<grid_1d(L.vocab, kThreads, 4096), kThreads, 0, s>>>(offsets, L.vocab, list,
                                                                                     large, n_large);
            bucket_sort_block_kernel<<<kSortBlocks, 1024, 0, s>>>(offsets, list, (int32_t*)(w + L.sort_tmp), large,
                                                                  n_large);
            cand_dw_kernel<<<(unsigned)cdiv(L.vocab, kThreads / 64), kThreads, 0, s>>>(cb);
            cand_dw_mid_kernel<<<kSplitBlocks, kThreads, 0, s>>>(cb, large, n_large);
            // buckets above kDwSplitEntries entries: pieces, their offsets, partial rows, join
            int32_t* pieces = (int32_t*)(w + L.pieces);
            int32_t* piece_off = (int32_t*)(w + L.piece_off);
            float* partial = (float*)(w + L.partial);
            cand_split_counts_kernel<<<grid_1d(L.vocab, kThreads, 4096), kThreads, 0, s>>>(offsets, large, n_large,
                                                                                           L.vocab, pieces);
            tile_sums_kernel<<<(unsigned)tiles, 256, 0, s>>>(pieces, L.vocab, tsum);
            exclusive_scan_kernel<<<1, 1024, 0, s>>>(tsum, tiles, tprefix);
            scan_tiles_kernel<<<(unsigned)tiles, 256, 0, s>>>(pieces, L.vocab, tprefix, tiles, piece_off);
            cand_dw_split_kernel<<<kSplitBlocks, kThreads, 0, s>>>(cb, large, n_large, piece_off, partial);
            cand_dw_join_kernel<<<kSplitBlocks, kThreads, 0, s>>>(cb, large, n_large, piece_off, partial);
        }
        return launched();
    }

    bf16_bits* G = (bf16_bits*)(w + L.G);
    const bf16_bits* Hf = (const bf16_bits*)(w + L.hfrag_bwd);
    frag_pack_kernel<<<grid_1d(L.n_pad * L.hidden / 8, kThreads, 8192), kThreads, 0, s>>>(
        (const bf16_bits*)H, L.n, L.hidden, L.n_pad, (bf16_bits*)Hf);
    const bf16_bits* HTf = (const bf16_bits*)(w + L.htfrag);
    if (want_dw)
        ht_pack_kernel<<<dim3((unsigned)(L.n_pad / 32), (unsigned)(L.hid_pad / kTile)), 256, 0, s>>>(
            (const bf16_bits*)H, L.n, L.hidden, L.hid_pad, (bf16_bits*)HTf);
    const int32_t* hit_offsets = nullptr;
    const int32_t* hit_list = nullptr;
    if (entry == LMHEAD_ENTRY_SUPPORT) build_hits(L, L.hit_bwd, w, ids, s, &hit_offsets, &hit_list);
    const int64_t nchunks = cdiv(L.vocab, L.chunk);
    const int64_t tiles_rows = L.n_pad / kTile;
    const int64_t tiles_hidden = cdiv(L.hidden, kTile);
    const int64_t g_stride = L.n_pad * L.w_pad;
    const int64_t g_pitch = L.dh_pass ? L.g_cols : 0;   // columns per block row of the region (0: per chunk)
    const float* part_in = (const float*)(w + L.dh_part);
    float* part = (float*)(w + L.dh_part);
    float* dh_sum = dH_acc != nullptr ? dH_acc : (float*)(w + L.dh_acc);
    // argument blocks of chunk c (dW: `group` chunks from c on; slot: its dL/dz)
    auto dw_args = [&](int64_t c, int64_t group, const bf16_bits* slot) {
        const int64_t v0 = c * L.chunk;
        const int64_t width = (L.vocab - v0) < L.chunk ? (L.vocab - v0) : L.chunk;
        DwArgs da{};
        da.G = slot;
        da.HTf = HTf;
        da.n = L.n;
        da.n_pad = L.n_pad;
        da.hidden = L.hidden;
        da.hid_pad = L.hid_pad;
        da.vocab = L.vocab;
        da.v0 = v0;
        da.chunk = L.chunk;
        da.group = group;
        da.g_stride = g_stride;
        da.tiles_m = L.hid_pad / kTile;
        da.tiles_n = round_up(width, kTile) / kTile;
        da.g_pitch = g_pitch;
        da.dW = (bf16_bits*)dW;
        da.dw_acc = dW_acc;
        return da;
    };
    // dH of chunks c .. last: the running sum starts at c and ends at last
    auto dh_args = [&](int64_t c, int64_t last, const bf16_bits* slot) {
        const int64_t v0 = c * L.chunk;
        DhArgs ha{};
        ha.G = slot;
        ha.Wc = (const bf16_bits*)W + v0 * L.hidden;
        ha.width = (L.vocab - v0) < L.chunk ? (L.vocab - v0) : L.chunk;
        ha.n = L.n;
        ha.n_pad = L.n_pad;
        ha.hidden = L.hidden;
        ha.w_pad = round_up(ha.width, kTile);
        ha.tiles_m = tiles_rows;
        ha.tiles_n = tiles_hidden;
        ha.first = c == 0 && dH_acc == nullptr;
        ha.last = last == nchunks - 1;
        ha.keep_acc = dH_acc != nullptr;
        ha.dh_acc = dh_sum;
        ha.dH = (bf16_bits*)dH;
        ha.g_pitch = g_pitch;
        return ha;
    };
    auto split_of = [&](int64_t c, int64_t chunks, int64_t slices, int64_t w_pad) {
        DhSplit q;
        q.W = (const bf16_bits*)W;
        q.v0 = c * L.chunk;
        q.chunk = L.chunk;
        q.vocab = L.vocab;
        q.chunks = chunks;
        q.slices = slices;
        q.ks = w_pad / slices;
        q.g_stride = g_stride;
        return q;
    };
    const unsigned join_grid = grid_1d(L.n * L.hidden / 4, kThreads, 4096);
    const int64_t n_dh = want_dh ? tiles_rows * tiles_hidden : 0;
    for (int64_t c = 0; c < nchunks; c += L.group) {
        const int64_t ng = (nchunks - c) < L.group ? (nchunks - c) : L.group;
        // position of chunk c in its dH pass: its dL/dz goes pos x C_pad
        // columns into the region (C_pad / 32 blocks of 512 elements each)
        const int64_t pos = L.dh_pass ? c % kDhPass : 0;
        bf16_bits* const slot = G + pos * 16 * L.w_pad;
        {
            // dL/dz of chunks c .. c + ng - 1, one launch
            LogitGradArgs ga;
            ga.T = T;
            ga.Hf = Hf;
            ga.W = (const bf16_bits*)W;
            ga.n = L.n;
            ga.n_pad = L.n_pad;
            ga.hidden = L.hidden;
            ga.vocab = L.vocab;
            ga.v0 = c * L.chunk;
            ga.chunk = L.chunk;
            ga.group = ng;
            ga.tiles_m = tiles_rows;
            ga.tiles_n = round_up((L.vocab - ga.v0) < L.chunk ? (L.vocab - ga.v0) : L.chunk, kTile) / kTile;
            ga.coef_a = ca.coef_a;
            ga.coef_c = ca.coef_c;
            ga.ids = ids;
            ga.k = (int)L.k;
            ga.lse = lse;
            ga.G = slot;
            ga.g_stride = g_stride;
            ga.g_pitch = g_pitch;
            ga.tiles_v = L.tiles_v;
            ga.hit_offsets = hit_offsets;
            ga.hit_list = hit_list;
            bwd_logit_grad_kernel<<<(unsigned)(ga.tiles_m * ga.tiles_n * ga.group), kThreads, 0, s>>>(ga);
        }
        if (L.group > 1) {
            // small batches: dW of the whole group in one launch; dH of the
            // group's chunks K-split in batches, each joined chunk by chunk
            if (want_dw) {
                const DwArgs da = dw_args(c, ng, G);
                bwd_dw_kernel<<<(unsigned)(da.tiles_m * da.tiles_n * ng), kThreads, 0, s>>>(da);
            }
            if (!want_dh) continue;
            const DhGroupPlan dp = dh_group_plan(L.n_pad, L.hidden, L.w_pad, ng);
            if (dp.slices == 0) {
                for (int64_t g = 0; g < ng; ++g)
                    bwd_dh_kernel<<<(unsigned)n_dh, kThreads, 0, s>>>(dh_args(c + g, c + g, G + g * g_stride));
                continue;
            }
            for (int64_t b0 = 0; b0 < ng; b0 += dp.batch) {
                const int64_t nb = (ng - b0) < dp.batch ? (ng - b0) : dp.batch;
                const DhArgs ha = dh_args(c + b0, c + b0 + nb - 1, G + b0 * g_stride);
                const DhSplit q = split_of(c + b0, nb, dp.slices, L.w_pad);
                bwd_dh_split_kernel<<<(unsigned)(n_dh * nb * dp.slices), kThreads, 0, s>>>(ha, q, part);
                dh_join_kernel<<<join_grid, kThreads, 0, s>>>(ha, q, part_in);
            }
            continue;
        }
        // one chunk per group
        const int64_t v0 = c * L.chunk;
        const int64_t width = (L.vocab - v0) < L.chunk ? (L.vocab - v0) : L.chunk;
        const int64_t w_pad = round_up(width, kTile);
        const DwArgs da = dw_args(c, 1, slot);
        const int64_t n_dw = want_dw ? da.tiles_m * da.tiles_n : 0;
        if (L.dh_pass) {
            // a chunk before the last of its pass: its dW now, its dH with the pass
            if (pos + 1 < kDhPass && c + 1 < nchunks) {
                if (want_dw) bwd_dw_kernel<<<(unsigned)n_dw, kThreads, 0, s>>>(da);
                continue;
            }
            // dH over the pass's chunks (the last pass may hold fewer) from the region's first column
            DhArgs ha = dh_args(c - pos, c, G);
            ha.width = pos * L.chunk + width;
            ha.w_pad = pos * L.w_pad + w_pad;
            const int plan_one = dwdh_plan(n_dw, L.n_pad / kTileK, n_dh, ha.w_pad / kTileK);
            if (plan_one >= 0) {
                bwd_dwdh_kernel<<<(unsigned)(n_dw + n_dh), kThreads, 0, s>>>(da, ha, plan_one);
            } else {
                if (want_dw) bwd_dw_kernel<<<(unsigned)n_dw, kThreads, 0, s>>>(da);
                if (want_dh) bwd_dh_kernel<<<(unsigned)n_dh, kThreads, 0, s>>>(ha);
            }
            continue;
        }
        const DhArgs ha = dh_args(c, c, G);
        const int slices = dh_slices(L.n, L.n_pad, L.hidden, w_pad);
        if (want_dh && slices > 1) {
            if (want_dw) bwd_dw_kernel<<<(unsigned)n_dw, kThreads, 0, s>>>(da);
            const DhSplit q = split_of(c, 1, slices, w_pad);
            bwd_dh_split_kernel<<<(unsigned)(n_dh * slices), kThreads, 0, s>>>(ha, q, part);
            dh_join_kernel<<<join_grid, kThreads, 0, s>>>(ha, q, part_in);
            continue;
        }
        const int plan_one = dwdh_plan(n_dw, L.n_pad / kTileK, n_dh, w_pad / kTileK);
        if (plan_one >= 0) {
            bwd_dwdh_kernel<<<(unsigned)(n_dw + n_dh), kThreads, 0, s>>>(da, ha, plan_one);
        } else {
            if (want_dw) bwd_dw_kernel<<<(unsigned)n_dw, kThreads, 0, s>>>(da);
            if (want_dh) bwd_dh_kernel<<<(unsigned)n_dh, kThreads, 0, s>>>(ha);
        }
    }
    return launched();
}


// The allocation-free forward's workspace: a file-scope device array, one
// copy per device, held until the process ends. Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the
// symbol); it uses the device address hipGetSymbolAddress returns, fetched
// once per device with that device current.
constexpr size_t kScratchBytes = LMHEAD_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[256];

int scratch_base(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) return LMHEAD_ERR_DEVICE;
    void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (ptr == nullptr) {
            if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
                return LMHEAD_ERR_HIP;
            g_scratch_ptr[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = ptr;
    return LMHEAD_OK;
}

}  // namespace

extern "C" {

int lmhead_loss_fwd_noalloc(const lmhead_problem* p, int entry, const void* H, const void* W,
                            const int32_t* targets, float* loss, float* lse, void* stream) {
    if (entry != LMHEAD_ENTRY_CE_MEAN && entry != LMHEAD_ENTRY_CE_SUM) return LMHEAD_ERR_ARG;
    int st = validate_problem(p, entry);
    if (st != LMHEAD_OK) return st;
    if (plan(*p, entry).fwd_total > kScratchBytes) return LMHEAD_ERR_SCRATCH;
    st = check_device();
    if (st != LMHEAD_OK) return st;
    void* ws = nullptr;
    st = scratch_base(&ws);
    if (st != LMHEAD_OK) return st;
    // the header words that must start at zero are cleared by the forward's
    // first kernel; every other region is written before it is read
    return forward(p, entry, H, W, targets, nullptr, nullptr, nullptr, lse, loss, ws, kScratchBytes,
                   stream);
}

size_t lmhead_workspace_size(const lmhead_problem* p, int entry, int with_backward) {
    if (validate_problem(p, entry) != LMHEAD_OK) return 0;
    const Layout L = plan(*p, entry);
    return with_backward ? L.bwd_total : L.fwd_total;
}

int lmhead_memory_report(const lmhead_problem* p, int entry, int with_backward,
                         lmhead_memory_figures* out) {
    if (out == nullptr) return LMHEAD_ERR_ARG;
    const int st = validate_problem(p, entry);
    if (st != LMHEAD_OK) return st;
    const Layout L = plan(*p, entry);
    lmhead_memory_figures r{};
    r.chunk = L.chunk;
    r.chunks = cdiv(L.vocab, L.chunk);
    r.workspace_bytes = with_backward ? L.bwd_total : L.fwd_total;
    r.forward_bytes = L.fwd_total;
    const bool kl_only = entry == LMHEAD_ENTRY_SUPPORT_KL;
    r.partials_bytes = kl_only ? 0 : (size_t)(8 * L.tiles_v * L.n);
    if (!kl_only) r.operand_copy_bytes = (size_t)L.hfrag_bytes + (with_backward ? (size_t)L.htfrag_bytes : 0);
    if (with_backward && !kl_only) {
        r.dz_chunk_bytes = (size_t)(2 * L.n_pad * L.g_cols);
        r.dz_group = L.group;
        r.dh_acc_bytes = (size_t)(4 * L.n * L.hidden);
        r.dh_split_bytes = (size_t)L.dh_part_bytes;
    }
    // fp32 outputs: lse [n] plus loss [1] / logp [n] / lp [n, k] and kl [n]
    size_t outs = (size_t)(4 * L.n);
    if (entry == LMHEAD_ENTRY_CE_MEAN || entry == LMHEAD_ENTRY_CE_SUM) outs += 4;
    else if (entry == LMHEAD_ENTRY_LOGPROB) outs += (size_t)(4 * L.n);
    else outs += (size_t)(4 * L.n * L.k + 4 * L.n);   // lp or log p_hat [n, k], kl [n]
    if (kl_only) outs -= (size_t)(4 * L.n);            // no lse
    if (with_backward) outs += (size_t)(2 * L.n * L.hidden + 2 * L.vocab * L.hidden);
    r.caller_output_bytes = outs;
    *out = r;
    return LMHEAD_OK;
}

int lmhead_plan_chunk(const lmhead_problem* p, int entry, size_t budget_bytes, int64_t* chunk) {
    if (p == nullptr || chunk == nullptr) return LMHEAD_ERR_ARG;
    lmhead_problem q = *p;
    q.chunk = 256;
    const int st = validate_problem(&q, entry);
    if (st != LMHEAD_OK) return st;
    auto fits = [&](int64_t c) {
        q.chunk = c;
        return plan(q, entry).bwd_total <= budget_bytes;
    };
    if (!fits(256)) return LMHEAD_ERR_WORKSPACE;
    // largest fitting chunk by bisection over multiples of 256 (the workspace
    // never shrinks as the chunk widens: the dL/dz region is sized by
    // grad_cols and the dH partials by the shape alone)
    int64_t lo = 1, hi = cdiv(q.vocab, 256);
    if (entry != LMHEAD_ENTRY_SUPPORT_KL && hi > kMaxChunkPad / 256) hi = kMaxChunkPad / 256;
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo + 1) / 2;
        if (fits(mid * 256)) lo = mid;
        else hi = mid - 1;
    }
    const int64_t passes = cdiv(q.vocab, lo * 256);
    const int64_t even = round_up(cdiv(q.vocab, passes), 256);
    // the even split of the same passes: no wider than the bisection's
    // chunk, so it fits as well (checked all the same)
    *chunk = fits(even) ? even : lo * 256;
    return LMHEAD_OK;
}

int lmhead_loss_fwd(const lmhead_problem* p, int entry, const void* H, const void* W,
                    const int32_t* targets, float* loss, float* lse, void* workspace,
                    size_t workspace_bytes, void* stream) {
    if (entry != LMHEAD_ENTRY_CE_MEAN && entry != LMHEAD_ENTRY_CE_SUM) return LMHEAD_ERR_ARG;
    return forward(p, entry, H, W, targets, nullptr, nullptr, nullptr, lse, loss, workspace,
                   workspace_bytes, stream);
}

int lmhead_logprob(const lmhead_problem* p, const void* H, const void* W, const int32_t* targets,
                   float* logp, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
    return forward(p, LMHEAD_ENTRY_LOGPROB, H, W, targets, nullptr, logp, nullptr, lse, nullptr,
                   workspace, workspace_bytes, stream);
}

int lmhead_support_logprob_kl(const lmhead_problem* p, const void* H, const void* W,
                              const int32_t* ids, const float* ref_logq, float* lp, float* kl,
                              float* lse, void* workspace, size_t workspace_bytes, void* stream) {
    return forward(p, LMHEAD_ENTRY_SUPPORT, H, W, ids, ref_logq, lp, kl, lse, nullptr, workspace,
                   workspace_bytes, stream);
}


int lmhead_support_logprob(const lmhead_problem* p, const void* H, const void* W,
                           const int32_t* ids, float* lp, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream) {
    return forward(p, LMHEAD_ENTRY_SUPPORT, H, W, ids, nullptr, lp, nullptr, lse, nullptr, workspace,
                   workspace_bytes, stream);
}

int lmhead_support_kl(const lmhead_problem* p, const void* H, const void* W, const int32_t* ids,
                      const float* ref_logq, float* kl, float* logp_hat, void* workspace,
                      size_t workspace_bytes, void* stream) {
    int st = validate_problem(p, LMHEAD_ENTRY_SUPPORT_KL);
    if (st != LMHEAD_OK) return st;
    if (workspace == nullptr) return LMHEAD_ERR_ARG;
    if (p->n > 0 && (H == nullptr || W == nullptr || ids == nullptr || ref_logq == nullptr ||
                     kl == nullptr))
        return LMHEAD_ERR_ARG;
    if (!aligned(H, 16) || !aligned(W, 16) || !aligned(workspace, 256) ||
        !aligned(p->row_temperature, 4))
        return LMHEAD_ERR_ALIGN;
    const Layout L = plan(*p, LMHEAD_ENTRY_SUPPORT_KL);
    if (workspace_bytes < L.fwd_total) return LMHEAD_ERR_WORKSPACE;
    const Temperature T = temperature_of(*p);
    st = check_device();
    if (st != LMHEAD_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    int32_t* hdr = (int32_t*)((char*)workspace + L.hdr);
    init_header_kernel<<<1, 64, 0, s>>>(hdr);
    if (L.n == 0) return launched();
    const int padded = (p->flags & LMHEAD_FLAG_PADDED_IDS) ? 1 : 0;
    scan_labels_kernel<<<grid_1d(L.n, kThreads, 1024), kThreads, 0, s>>>(ids, L.n, (int)L.k, L.vocab,
                                                                          1 + padded, T, hdr);
    CandFwdArgs ca;
    ca.H = (const bf16_bits*)H;
    ca.W = (const bf16_bits*)W;
    ca.n = L.n;
    ca.hidden = L.hidden;
    ca.vocab = L.vocab;
    ca.k = (int)L.k;
    ca.padded = padded;
    ca.ids = ids;
    ca.ref_logq = ref_logq;
    ca.kl = kl;
    ca.logp_hat = logp_hat;
    ca.T = T;
    cand_kl_fwd_kernel<<<(unsigned)cdiv(L.n, kThreads / 64), kThreads, 0, s>>>(ca);
    return launched();
}

int lmhead_loss_bwd(const lmhead_problem* p, int entry, const void* H, const void* W,
                    const int32_t* ids, const float* ref_logq, const float* lse,
                    const float* saved_lp, const float* grad, const float* grad_kl, void* dH,
                    void* dW, void* workspace, size_t workspace_bytes, void* stream) {
    return backward(p, entry, H, W, ids, ref_logq, lse, saved_lp, grad, grad_kl, dH, dW, nullptr,
                    nullptr, workspace, workspace_bytes, stream);
}

int lmhead_loss_bwd_accumulate(const lmhead_problem* p, int entry, const void* H, const void* W,
                               const int32_t* ids, const float* ref_logq, const float* lse,
                               const float* saved_lp, const float* grad, const float* grad_kl,
                               float* dH_acc, float* dW_acc, void* dH, void* dW, void* workspace,
                               size_t workspace_bytes, void* stream) {
    // a bf16 output is the cast of its accumulator, so it needs one
    if ((dH != nullptr && dH_acc == nullptr) || (dW != nullptr && dW_acc == nullptr))
        return LMHEAD_ERR_ARG;
    return backward(p, entry, H, W, ids, ref_logq, lse, saved_lp, grad, grad_kl, dH, dW, dH_acc,
                    dW_acc, workspace, workspace_bytes, stream);
}

const char* lmhead_status_string(int status) {
    switch (status) {
        case LMHEAD_OK: return "ok";
        case LMHEAD_ERR_ARG: return "invalid argument (NULL pointer, unknown entry or nonzero flags)";
        case LMHEAD_ERR_SHAPE: return "unsupported problem size";
        case LMHEAD_ERR_ALIGN: return "misaligned pointer (16 bytes; workspace 256 bytes)";
        case LMHEAD_ERR_WORKSPACE: return "workspace too small";
        case LMHEAD_ERR_DEVICE: return "no gfx950 (MI355X) device is current";
        case LMHEAD_ERR_HIP: return "HIP runtime error";
        case LMHEAD_ERR_SCRATCH:
            return "forward workspace larger than the static scratch buffer (LMHEAD_STATIC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

int lmhead_read_device_error(const void* workspace, void* stream, int32_t* code, int64_t* row) {
    if (workspace == nullptr || code == nullptr || row == nullptr) return LMHEAD_ERR_ARG;
    if (!aligned(workspace, 256)) return LMHEAD_ERR_ALIGN;
    int st = check_device();
    if (st != LMHEAD_OK) return st;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return LMHEAD_ERR_HIP;
    int32_t h[3];
    if (hipMemcpy(h, workspace, sizeof h, hipMemcpyDeviceToHost) != hipSuccess) return LMHEAD_ERR_HIP;
    *code = h[kHdrErrCode];
    *row = h[kHdrErrRow] == INT_MAX ? -1 : (int64_t)h[kHdrErrRow];
    return LMHEAD_OK;
}

}  // extern "C"
