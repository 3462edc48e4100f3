// lmhead_candidates.hip — the KL-only support entry, which needs the logits of
// the listed candidates only: KL(q || p_hat) renormalises the model over the
// K candidates of a row, so neither it nor its gradient touches the other
// V - K logits (FlashInfer PR #8059 lists support_logprob and support_kl as
// separate entries). Every kernel is a gather over rows of W or H; there is
// no vocabulary-wide contraction.
//
// Determinism: each dot product accumulates in a fixed lane order and is
// reduced by a fixed xor-butterfly; the dW rows sum their (row, candidate)
// entries in ascending order after a counting sort whose buckets are sorted,
// so atomics only ever count (integers) and never order a floating-point sum.
#include <climits>

#include "lmhead_kernels.h"

namespace lmhead {

namespace {

constexpr int kWaves = kThreads / 64;   // rows (or vocabulary rows) per workgroup
constexpr int kSeg = 512;               // hidden elements one wave covers per step (8 per lane)
constexpr int kHoldSeg = 8;             // segments of an H row the KL forward keeps in registers

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ void fma8(float (&acc)[8], float c, const uint4& v) {
    acc[0] = __builtin_fmaf(c, bf16_lo(v.x), acc[0]);
    acc[1] = __builtin_fmaf(c, bf16_hi(v.x), acc[1]);
    acc[2] = __builtin_fmaf(c, bf16_lo(v.y), acc[2]);
    acc[3] = __builtin_fmaf(c, bf16_hi(v.y), acc[3]);
    acc[4] = __builtin_fmaf(c, bf16_lo(v.z), acc[4]);
    acc[5] = __builtin_fmaf(c, bf16_hi(v.z), acc[5]);
    acc[6] = __builtin_fmaf(c, bf16_lo(v.w), acc[6]);
    acc[7] = __builtin_fmaf(c, bf16_hi(v.w), acc[7]);
}

__device__ __forceinline__ float dot8(const uint4& a, const uint4& b, float acc) {
    acc = __builtin_fmaf(bf16_lo(a.x), bf16_lo(b.x), acc);
    acc = __builtin_fmaf(bf16_hi(a.x), bf16_hi(b.x), acc);
    acc = __builtin_fmaf(bf16_lo(a.y), bf16_lo(b.y), acc);
    acc = __builtin_fmaf(bf16_hi(a.y), bf16_hi(b.y), acc);
    acc = __builtin_fmaf(bf16_lo(a.z), bf16_lo(b.z), acc);
    acc = __builtin_fmaf(bf16_hi(a.z), bf16_hi(b.z), acc);
    acc = __builtin_fmaf(bf16_lo(a.w), bf16_lo(b.w), acc);
    acc = __builtin_fmaf(bf16_hi(a.w), bf16_hi(b.w), acc);
    return acc;
}

// xor-butterfly over the 64 lanes: every lane ends with the same value, and the
// association order is fixed
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float quiet_nan_f() { return __builtin_nanf(""); }
__device__ __forceinline__ float neg_inf_f() { return -__builtin_huge_valf(); }

// Store 8 fp32 values as bf16 (RNE) and / or add them to an fp32 accumulator.
__device__ __forceinline__ void store_row8(float (&acc)[8], float* acc_row, bf16_bits* out_row) {
    if (acc_row != nullptr) {
        float4* p = reinterpret_cast<float4*>(acc_row);
        const float4 a0 = p[0], a1 = p[1];
        acc[0] = a0.x + acc[0];
        acc[1] = a0.y + acc[1];
        acc[2] = a0.z + acc[2];
        acc[3] = a0.w + acc[3];
        acc[4] = a1.x + acc[4];
        acc[5] = a1.y + acc[5];
        acc[6] = a1.z + acc[6];
        acc[7] = a1.w + acc[7];
        p[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        p[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
    if (out_row != nullptr)
        *reinterpret_cast<uint4*>(out_row) =
            make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                       pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
}

// W rows of candidates k0 .. k0 + 3 of a row. A padding slot (or one past k)
// reads row 0 and its z is never used (every use checks the id), so the loads
// of a segment are unconditional and in flight together instead of each
// waiting behind a branch join.
__device__ __forceinline__ void cand_rows4(const CandFwdArgs& a, const int32_t* idr, int k0,
                                           const bf16_bits* (&wr)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int32_t id = k0 + c < a.k ? idr[k0 + c] : -1;
        wr[c] = a.W + (int64_t)(id >= 0 ? id : 0) * a.hidden;
    }
}

// z_k = (wave sum of the lanes' partial dot products) / tau for the real
// slots among k0 .. k0 + 3, written by lane 0
__device__ __forceinline__ void store_z4(float* z, const float (&part)[4], int k0, int k,
                                         float inv_tau, int lane) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const float zc = wave_sum(part[c]) * inv_tau;
        if (lane == 0 && k0 + c < k) z[k0 + c] = zc;
    }
}

}  // namespace

// One wave per row: the K candidate logits z_k = H[n] . W[id_k] / tau_n
// (fp32 sums of bf16 products), then log p_hat_k = z_k - log sum_j exp z_j
// over the row's real candidates and KL = sum_k q_k (r_k - log p_hat_k).
__global__ __launch_bounds__(kThreads) void cand_kl_fwd_kernel(CandFwdArgs a) {
    __shared__ float zs[kWaves][kMaxCandidates];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t row = (int64_t)blockIdx.x * kWaves + wave;
    if (row >= a.n) return;   // whole waves only; nothing below synchronises the workgroup
    const int k = a.k;
    const int32_t* idr = a.ids + row * k;
    const float tau = row_tau(a.T, row);
    bool bad = a.T.row != nullptr && !tau_ok(tau);
    for (int kk = 0; kk < k; ++kk) {
        const int64_t id = idr[kk];
        bad = bad || id >= a.vocab || (id < 0 && !a.padded);
    }
    if (bad) {
        if (lane == 0) a.kl[row] = quiet_nan_f();
        if (a.logp_hat != nullptr)
            for (int kk = lane; kk < k; kk += 64) a.logp_hat[row * k + kk] = quiet_nan_f();
        return;
    }
    const float inv_tau = 1.0f / tau;
    const bf16_bits* hrow = a.H + row * a.hidden;
    float* z = zs[wave];
    if (a.hidden % (2 * kSeg) == 0 && a.hidden <= kHoldSeg * kSeg) {
        // the row of H stays in registers (at most 8 segments, 32 registers
        // per lane), so each group of candidates loads only its W rows:
        // re-reading H for every group added a quarter to the bytes moved
        const int nseg = a.hidden / kSeg;
        uint4 hv[kHoldSeg];
#pragma unroll
        for (int s = 0; s < kHoldSeg; ++s)
            hv[s] = s < nseg ? *reinterpret_cast<const uint4*>(hrow + lane * 8 + s * kSeg)
                             : make_uint4(0, 0, 0, 0);
        for (int k0 = 0; k0 < k; k0 += 4) {
            const bf16_bits* wr[4];
            cand_rows4(a, idr, k0, wr);
            float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            // two segments' eight W loads at a time, then their products in
            // ascending segment order
#pragma unroll
            for (int s = 0; s < kHoldSeg; s += 2) {
                if (s < nseg) {
                    uint4 w0[4], w1[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        w0[c] = *reinterpret_cast<const uint4*>(wr[c] + lane * 8 + s * kSeg);
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        w1[c] = *reinterpret_cast<const uint4*>(wr[c] + lane * 8 + (s + 1) * kSeg);
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        part[c] = dot8(hv[s + 1], w1[c], dot8(hv[s], w0[c], part[c]));
                }
            }
            store_z4(z, part, k0, k, inv_tau, lane);
        }
    } else {
        for (int k0 = 0; k0 < k; k0 += 4) {
            const bf16_bits* wr[4];
            cand_rows4(a, idr, k0, wr);
            float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            // two segments' ten loads (H and four W rows each) at a time, then
            // their products in ascending segment order: per lane the same sums,
            // in the same order, as the path above
            int64_t h = lane * 8;
            for (; h + kSeg < a.hidden; h += 2 * kSeg) {
                const uint4 hv0 = *reinterpret_cast<const uint4*>(hrow + h);
                const uint4 hv1 = *reinterpret_cast<const uint4*>(hrow + h + kSeg);
                uint4 w0[4], w1[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) w0[c] = *reinterpret_cast<const uint4*>(wr[c] + h);
#pragma unroll
                for (int c = 0; c < 4; ++c) w1[c] = *reinterpret_cast<const uint4*>(wr[c] + h + kSeg);
#pragma unroll
                for (int c = 0; c < 4; ++c) part[c] = dot8(hv1, w1[c], dot8(hv0, w0[c], part[c]));
            }
            if (h < a.hidden) {
                const uint4 hv = *reinterpret_cast<const uint4*>(hrow + h);
                uint4 wv[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) wv[c] = *reinterpret_cast<const uint4*>(wr[c] + h);
#pragma unroll
                for (int c = 0; c < 4; ++c) part[c] = dot8(hv, wv[c], part[c]);
            }
            store_z4(z, part, k0, k, inv_tau, lane);
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float mx = neg_inf_f();
    for (int kk = lane; kk < k; kk += 64)
        if (idr[kk] >= 0) mx = fmaxf(mx, z[kk]);
    mx = wave_max(mx);
    float se = 0.0f;
    for (int kk = lane; kk < k; kk += 64)
        if (idr[kk] >= 0) se += expf(z[kk] - mx);
    se = wave_sum(se);
    const float ls = mx + logf(se);
    const float* r = a.ref_logq + row * k;
    float kl = 0.0f;
    for (int kk = lane; kk < k; kk += 64) {
        const bool real = idr[kk] >= 0;
        const float lph = real ? z[kk] - ls : 0.0f;
        if (a.logp_hat != nullptr) a.logp_hat[row * k + kk] = lph;
        const float q = expf(r[kk]);
        if (real && q > 0.0f) kl += q * (r[kk] - lph);
    }
    kl = wave_sum(kl);
    if (lane == 0) a.kl[row] = kl;
}

// dH[n] = sum_k c_nk W[id_nk] (ascending k), one wave per row.
__global__ __launch_bounds__(kThreads) void cand_dh_kernel(CandBwdArgs a) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t row = (int64_t)blockIdx.x * kWaves + wave;
    if (row >= a.n) return;
    const int32_t* idr = a.ids + row * a.k;
    const float* cr = a.coef_c + row * a.k;
    for (int64_t h = lane * 8; h < a.hidden; h += kSeg) {
        float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
        // four candidates at a time: their W rows are loaded together and
        // unconditionally (a padding slot or a past-k one reads row 0), and
        // only the products are skipped, so the sum keeps its terms and order
        for (int k0 = 0; k0 < a.k; k0 += 4) {
            int32_t id[4];
            float c[4];
            uint4 wv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int kk = k0 + u < a.k ? k0 + u : a.k - 1;
                id[u] = k0 + u < a.k ? idr[kk] : -1;
                c[u] = cr[kk];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t r = id[u] >= 0 && id[u] < a.vocab ? id[u] : 0;
                wv[u] = *reinterpret_cast<const uint4*>(a.W + r * a.hidden + h);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (id[u] >= 0 && id[u] < a.vocab && c[u] != 0.0f) fma8(acc, c[u], wv[u]);
        }
        store_row8(acc, a.dH_acc != nullptr ? a.dH_acc + row * a.hidden + h : nullptr,
                   a.dH != nullptr ? a.dH + row * a.hidden + h : nullptr);
    }
}

// counts[v] = number of (row, candidate) entries with id v.
__global__ void cand_count_kernel(const int32_t* ids, int64_t nk, int64_t vocab, int32_t* counts) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nk;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int32_t id = ids[i];
        if (id >= 0 && id < vocab) atomicAdd(counts + id, 1);
    }
}

// offsets[v] = sum_{u < v} counts[u] for v = 0..vocab (one workgroup).
__global__ __launch_bounds__(1024) void exclusive_scan_kernel(const int32_t* counts, int64_t vocab,
                                                              int32_t* offsets) {
    __shared__ int32_t part[1024];
    const int t = threadIdx.x;
    const int64_t per = (vocab + 1023) / 1024;
    const int64_t b = t * per, e = (b + per) < vocab ? (b + per) : vocab;
    int32_t s = 0;
    for (int64_t v = b; v < e; ++v) s += counts[v];
    part[t] = s;
    __syncthreads();
    // inclusive Hillis-Steele scan of the 1024 partial sums
    for (int o = 1; o < 1024; o <<= 1) {
        const int32_t add = t >= o ? part[t - o] : 0;
        __syncthreads();
        part[t] += add;
        __syncthreads();
    }
    int32_t run = t > 0 ? part[t - 1] : 0;
    for (int64_t v = b; v < e; ++v) {
        offsets[v] = run;
        run += counts[v];
    }
    if (t == 1023) offsets[vocab] = part[1023];
}

// The bucket offsets over the whole vocabulary, in three launches: the sum of
// each 1024-count tile, an exclusive scan of those sums (exclusive_scan_kernel
// on the tile sums, one workgroup, ceil(V / 1024) values), then each tile's
// own exclusive scan plus its prefix. Integer sums are exact, so the result
// is the plain exclusive scan whatever the grouping.
__global__ __launch_bounds__(256) void tile_sums_kernel(const int32_t* counts, int64_t vocab, int32_t* sums) {
    __shared__ int32_t wsum[4];
    const int64_t base = (int64_t)blockIdx.x * kScanTile;
    const int t = threadIdx.x;
    int32_t s = 0;
#pragma unroll
    for (int i = 0; i < kScanTile / 256; ++i) {
        const int64_t v = base + i * 256 + t;
        if (v < vocab) s += counts[v];
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) s += __shfl_xor(s, o);
    if ((t & 63) == 0) wsum[t >> 6] = s;
    __syncthreads();
    if (t == 0) sums[blockIdx.x] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
}

// offsets[v] for v in one tile: prefix[tile] plus the exclusive scan of the
// tile's counts (thread t holds counts 4 t .. 4 t + 3); the first tile also
// writes offsets[vocab] = prefix[tiles].
__global__ __launch_bounds__(256) void scan_tiles_kernel(const int32_t* counts, int64_t vocab,
                                                         const int32_t* prefix, int64_t tiles,
                                                         int32_t* offsets) {
    __shared__ int32_t wtot[4];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int64_t v0 = (int64_t)blockIdx.x * kScanTile + 4 * t;
    int32_t c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = v0 + i < vocab ? counts[v0 + i] : 0;
    const int32_t own = c[0] + c[1] + c[2] + c[3];
    int32_t inc = own;   // inclusive scan over the wave's lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t u = __shfl_up(inc, o);
        if (lane >= o) inc += u;
    }
    if (lane == 63) wtot[w] = inc;
    __syncthreads();
    int32_t run = prefix[blockIdx.x] + inc - own;
    for (int i = 0; i < w; ++i) run += wtot[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (v0 + i < vocab) offsets[v0 + i] = run;
        run += c[i];
    }
    if (blockIdx.x == 0 && t == 0) offsets[vocab] = prefix[tiles];
}

// list[offsets[id] + slot] = entry index i = row * k + candidate; the slot
// order inside a bucket is arbitrary here and fixed by bucket_sort_kernel.
__global__ void cand_fill_kernel(const int32_t* ids, int64_t nk, int64_t vocab, const int32_t* offsets,
                                 int32_t* cursor, int32_t* list) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nk;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int32_t id = ids[i];
        if (id >= 0 && id < vocab) list[offsets[id] + atomicAdd(cursor + id, 1)] = (int32_t)i;
    }
}

// Sorting the buckets ascending (entries are distinct, so the ascending order
// is unique and the result does not depend on how it is reached). Small
// buckets are sorted where they are found; larger ones are appended to a list
// (an integer atomic fixes only the list's order, not the result) and sorted
// by bucket_sort_block_kernel, one workgroup per bucket.
constexpr int kSortLdsMax = 32768;   // entries a workgroup sorts in LDS (128 KB)
// A vocabulary bucket above this many entries is listed as large: sorted by
// the workgroup sort and, in the KL-only dW, summed by the mid / split kernels.
constexpr int kSmallBucket = 16;

// One thread per bucket: insertion sort for up to kSmallBucket entries, the vocabulary
// buckets of the KL-only entry holding N·K / V (a few) on average.
__global__ void bucket_sort_kernel(const int32_t* offsets, int64_t buckets, int32_t* list, int32_t* large,
                                   int32_t* n_large) {
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < buckets;
         v += (int64_t)gridDim.x * blockDim.x) {
        const int32_t b = offsets[v], e = offsets[v + 1];
        if (e - b > kSmallBucket) {
            large[atomicAdd(n_large, 1)] = (int32_t)v;
            continue;
        }
        for (int32_t i = b + 1; i < e; ++i) {
            const int32_t x = list[i];
            int32_t j = i - 1;
            while (j >= b && list[j] > x) {
                list[j + 1] = list[j];
                --j;
            }
            list[j + 1] = x;
        }
    }
}

// One wave per bucket: up to 64 entries sorted across the lanes by a bitonic
// network (lanes past the bucket hold INT_MAX, above every entry): the
// per-tile hit buckets, which hold tens of entries.
__global__ __launch_bounds__(256) void bucket_sort_wave_kernel(const int32_t* offsets, int64_t buckets,
                                                               int32_t* list, int32_t* large,
                                                               int32_t* n_large) {
    const int lane = threadIdx.x & 63;
    const int64_t v = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
    if (v >= buckets) return;   // the whole wave
    const int32_t b = offsets[v], e = offsets[v + 1];
    const int32_t cnt = e - b;
    if (cnt <= 1) return;
    if (cnt > 64) {
        if (lane == 0) large[atomicAdd(n_large, 1)] = (int32_t)v;
        return;
    }
    int32_t x = lane < cnt ? list[b + lane] : INT_MAX;
#pragma unroll
    for (int k = 2; k <= 64; k <<= 1)
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const int32_t y = __shfl_xor(x, j);
            const bool up = (lane & k) == 0;      // this pair's sequence sorts ascending
            const bool lower = (lane & j) == 0;   // the pair's lower lane
            x = (lower == up) ? (x < y ? x : y) : (x < y ? y : x);
        }
    if (lane < cnt) list[b + lane] = x;
}

// The listed large buckets, one workgroup of 1024 threads per bucket. Runs
// of up to kSortLdsMax entries are sorted in LDS by a bitonic network over
// the run padded with INT_MAX to a power of two; a bucket with more entries
// (only a heavily skewed candidate list makes one) then merges its sorted
// runs pairwise, doubling the run length each pass, between the list and the
// bucket's own range of tmp (merge path: each thread finds by binary search
// where its share of the output starts in each run, then merges that share),
// so a bucket of m entries takes O(m log m) work spread over the workgroup.
__device__ void sort_run_lds(int32_t* sh, int32_t* p, int32_t m) {
    const int t = threadIdx.x;
    int32_t P = 64;
    while (P < m) P <<= 1;
    for (int32_t i = t; i < P; i += 1024) sh[i] = i < m ? p[i] : INT_MAX;
    __syncthreads();
    for (int32_t k = 2; k <= P; k <<= 1)
        for (int32_t j = k >> 1; j > 0; j >>= 1) {
            for (int32_t i = t; i < P; i += 1024) {
                const int32_t l = i ^ j;
                if (l > i) {
                    const int32_t x = sh[i], y = sh[l];
                    const bool up = (i & k) == 0;
                    if ((x > y) == up) {
                        sh[i] = y;
                        sh[l] = x;
                    }
                }
            }
            __syncthreads();
        }
    for (int32_t i = t; i < m; i += 1024) p[i] = sh[i];
    __syncthreads();
}

// Entries of a (sorted, distinct) taken among the first d of the merge of a
// and b.
__device__ __forceinline__ int64_t merge_split(const int32_t* a, int64_t na, const int32_t* b, int64_t nb, int64_t d) {
    int64_t lo = d > nb ? d - nb : 0, hi = d < na ? d : na;
    while (lo < hi) {
        const int64_t mid = (lo + hi) / 2;
        if (a[mid] < b[d - mid - 1]) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

// out[0, na + nb) = the merge of the sorted runs a and b, by the workgroup.
__device__ void merge_runs(const int32_t* a, int64_t na, const int32_t* b, int64_t nb, int32_t* out) {
    const int64_t L = na + nb;
    const int64_t t = threadIdx.x;
    const int64_t d0 = L * t / 1024, d1 = L * (t + 1) / 1024;
    int64_t i = merge_split(a, na, b, nb, d0), j = d0 - i;
    for (int64_t d = d0; d < d1; ++d) {
        const bool take_a = j >= nb || (i < na && a[i] < b[j]);
        out[d] = take_a ? a[i++] : b[j++];
    }
}

__global__ __launch_bounds__(1024) void bucket_sort_block_kernel(const int32_t* offsets, int32_t* list, int32_t* tmp,
                                                                 const int32_t* large, const int32_t* n_large) {
    __shared__ int32_t sh[kSortLdsMax];
    const int t = threadIdx.x;
    const int32_t count = *n_large;
    for (int32_t q = blockIdx.x; q < count; q += gridDim.x) {
        const int32_t v = large[q];
        const int64_t b = offsets[v], e = offsets[v + 1];
        const int64_t m = e - b;
        for (int64_t r0 = 0; r0 < m; r0 += kSortLdsMax)
            sort_run_lds(sh, list + b + r0, (int32_t)(m - r0 < kSortLdsMax ? m - r0 : kSortLdsMax));
        if (m <= kSortLdsMax) continue;
        int32_t* src = list + b;
        int32_t* dst = tmp + b;
        for (int64_t w = kSortLdsMax; w < m; w *= 2) {
            for (int64_t p0 = 0; p0 < m; p0 += 2 * w) {
                const int64_t na = m - p0 < w ? m - p0 : w;
                const int64_t rest = m - p0 - na;
                const int64_t nb = rest < w ? rest : w;
                merge_runs(src + p0, na, src + p0 + na, nb, dst + p0);
            }
            __syncthreads();
            int32_t* x = src;
            src = dst;
            dst = x;
        }
        if (src != list + b)
            for (int64_t i = t; i < m; i += 1024) list[b + i] = src[i];
        __syncthreads();
    }
}

// Hit lists for the tile epilogues of the support entries: count, then fill
// (positions within a bucket come from an atomic cursor, so the order is
// arbitrary until bucket_sort_kernel sorts each bucket's packed values).
__global__ void hit_count_kernel(const int32_t* ids, int64_t n, int k, int64_t vocab, int64_t tiles_v,
                                 int32_t* counts) {
    const int64_t nk = n * k;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nk;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int32_t id = ids[i];
        if (id >= 0 && id < vocab) atomicAdd(counts + (i / k >> 8) * tiles_v + (id >> 8), 1);
    }
}

__global__ void hit_fill_kernel(const int32_t* ids, int64_t n, int k, int64_t vocab, int64_t tiles_v,
                                const int32_t* offsets, int32_t* cursor, int32_t* list) {
    const int64_t nk = n * k;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nk;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int32_t id = ids[i];
        if (id < 0 || id >= vocab) continue;
        const int64_t row = i / k;
        const int kk = (int)(i - row * k);
        const int64_t b = (row >> 8) * tiles_v + (id >> 8);
        list[offsets[b] + atomicAdd(cursor + b, 1)] =
            (int32_t)(((row & 255) << kHitRowShift) | ((id & 255) << kHitColShift) | kk);
    }
}

// dW[v] = sum over the entries (n, k) with id_nk = v, in ascending (n, k)
// order, of c_nk H[n]; rows no candidate lists get 0.
//
// dw_sum adds the entries [j0, j1) of a bucket into acc for the hidden
// positions h0 + 512 s + 8 lane (s < kDwPass): four entries' list, coefficient
// and H loads are issued together, and every element still takes its products
// in ascending entry order.
constexpr int kDwPass = 4;      // 512-wide hidden segments per pass over the entries
constexpr int kDwSplit = kDwSplitEntries;   // a bucket with more entries is summed by several waves

__device__ __forceinline__ void dw_sum(const CandBwdArgs& a, int32_t j0, int32_t j1, int64_t h0, int lane,
                                       float (&acc)[kDwPass][8]) {
#pragma unroll
    for (int s = 0; s < kDwPass; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[s][e] = 0.0f;
    int32_t j = j0;
    for (; j + 4 <= j1; j += 4) {
        int32_t ii[4];
        float cc[4];
        uint4 hv[4][kDwPass];
#pragma unroll
        for (int u = 0; u < 4; ++u) ii[u] = a.list[j + u];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            cc[u] = a.coef_c[ii[u]];
            const bf16_bits* hr = a.H + (int64_t)(ii[u] / a.k) * a.hidden;
#pragma unroll
            for (int s = 0; s < kDwPass; ++s) {
                const int64_t h = h0 + s * kSeg + lane * 8;
                hv[u][s] = h < a.hidden ? *reinterpret_cast<const uint4*>(hr + h) : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (cc[u] != 0.0f)
#pragma unroll
                for (int s = 0; s < kDwPass; ++s) fma8(acc[s], cc[u], hv[u][s]);
    }
    for (; j < j1; ++j) {
        const int32_t i = a.list[j];
        const float c = a.coef_c[i];
        if (c == 0.0f) continue;
        const bf16_bits* hr = a.H + (int64_t)(i / a.k) * a.hidden;
#pragma unroll
        for (int s = 0; s < kDwPass; ++s) {
            const int64_t h = h0 + s * kSeg + lane * 8;
            if (h < a.hidden) fma8(acc[s], c, *reinterpret_cast<const uint4*>(hr + h));
        }
    }
}

// One wave per vocabulary row whose bucket holds at most kSmallBucket entries (the
// common case: N·K / V entries per row on average), with few registers so that
// many waves hide the gather latency. Larger buckets are in the sort's list
// of large buckets and are summed by cand_dw_mid_kernel (up to kDwSplit
// entries) or split (above it).
__global__ __launch_bounds__(kThreads) void cand_dw_kernel(CandBwdArgs a) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t v = (int64_t)blockIdx.x * kWaves + wave;
    if (v >= a.vocab) return;
    const int32_t b = a.offsets[v], e = a.offsets[v + 1];
    if (e - b > kSmallBucket) return;
    for (int64_t h = lane * 8; h < a.hidden; h += kSeg) {
        float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
        // four entries at a time, their loads together (entries past the
        // bucket repeat its last one and are not added), products in order
        for (int32_t j0 = b; j0 < e; j0 += 4) {
            int32_t i[4];
            float c[4];
            uint4 hv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) i[u] = a.list[j0 + u < e ? j0 + u : e - 1];
#pragma unroll
            for (int u = 0; u < 4; ++u) c[u] = a.coef_c[i[u]];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                hv[u] = *reinterpret_cast<const uint4*>(a.H + (int64_t)(i[u] / a.k) * a.hidden + h);
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (j0 + u < e && c[u] != 0.0f) fma8(acc, c[u], hv[u]);
        }
        store_row8(acc, a.dW_acc != nullptr ? a.dW_acc + v * a.hidden + h : nullptr,
                   a.dW != nullptr ? a.dW + v * a.hidden + h : nullptr);
    }
}

// One wave per listed large bucket of kSmallBucket + 1 .. kDwSplit entries.
__global__ __launch_bounds__(kThreads) void cand_dw_mid_kernel(CandBwdArgs a, const int32_t* large,
                                                               const int32_t* n_large) {
    const int lane = threadIdx.x & 63;
    const int32_t count = *n_large;
    for (int64_t q = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); q < count;
         q += (int64_t)gridDim.x * kWaves) {
        const int64_t v = large[q];
        const int32_t b = a.offsets[v], e = a.offsets[v + 1];
        if (e - b > kDwSplit) continue;
        for (int64_t h0 = 0; h0 < a.hidden; h0 += kDwPass * kSeg) {
            float acc[kDwPass][8];
            dw_sum(a, b, e, h0, lane, acc);
#pragma unroll
            for (int s = 0; s < kDwPass; ++s) {
                const int64_t h = h0 + s * kSeg + lane * 8;
                if (h < a.hidden)
                    store_row8(acc[s], a.dW_acc != nullptr ? a.dW_acc + v * a.hidden + h : nullptr,
                               a.dW != nullptr ? a.dW + v * a.hidden + h : nullptr);
            }
        }
    }
}

// Large buckets (a common id listed by many rows) are split into pieces of
// kDwSplit entries so that no single wave sums thousands of rows: piece
// counts per listed large bucket (zero for the listed ones not above
// kDwSplit), their exclusive scan (the multi-block scan), one wave per piece
// writing its fp32 partial row, and one wave per bucket adding the partials
// in piece order. The split depends only on the bucket sizes, so the result
// is deterministic; a split bucket's sum is associated piece by piece.
__global__ void cand_split_counts_kernel(const int32_t* offsets, const int32_t* large, const int32_t* n_large,
                                         int64_t cap, int32_t* pieces) {
    const int32_t count = *n_large;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < cap;
         q += (int64_t)gridDim.x * blockDim.x) {
        int32_t p = 0;
        if (q < count) {
            const int32_t v = large[q];
            const int32_t m = offsets[v + 1] - offsets[v];
            p = m > kDwSplit ? (m + kDwSplit - 1) / kDwSplit : 0;
        }
        pieces[q] = p;
    }
}

__global__ __launch_bounds__(kThreads) void cand_dw_split_kernel(CandBwdArgs a, const int32_t* large,
                                                                 const int32_t* n_large, const int32_t* piece_off,
                                                                 float* partial) {
    const int lane = threadIdx.x & 63;
    const int32_t count = *n_large;
    if (count == 0) return;
    const int32_t total = piece_off[count];
    for (int64_t g = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); g < total;
         g += (int64_t)gridDim.x * kWaves) {
        // the listed bucket q with piece_off[q] <= g < piece_off[q + 1]
        int32_t lo = 0, hi = count - 1;
        while (lo < hi) {
            const int32_t mid = (lo + hi + 1) >> 1;
            if (piece_off[mid] <= g) lo = mid;
            else hi = mid - 1;
        }
        const int32_t v = large[lo];
        const int32_t b = a.offsets[v], e = a.offsets[v + 1];
        const int32_t j0 = b + (int32_t)(g - piece_off[lo]) * kDwSplit;
        const int32_t j1 = j0 + kDwSplit < e ? j0 + kDwSplit : e;
        for (int64_t h0 = 0; h0 < a.hidden; h0 += kDwPass * kSeg) {
            float acc[kDwPass][8];
            dw_sum(a, j0, j1, h0, lane, acc);
#pragma unroll
            for (int s = 0; s < kDwPass; ++s) {
                const int64_t h = h0 + s * kSeg + lane * 8;
                if (h < a.hidden) {
                    float4* o = reinterpret_cast<float4*>(partial + g * a.hidden + h);
                    o[0] = make_float4(acc[s][0], acc[s][1], acc[s][2], acc[s][3]);
                    o[1] = make_float4(acc[s][4], acc[s][5], acc[s][6], acc[s][7]);
                }
            }
        }
    }
}

__global__ __launch_bounds__(kThreads) void cand_dw_join_kernel(CandBwdArgs a, const int32_t* large,
                                                                const int32_t* n_large, const int32_t* piece_off,
                                                                const float* partial) {
    const int lane = threadIdx.x & 63;
    const int32_t count = *n_large;
    for (int64_t q = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); q < count;
         q += (int64_t)gridDim.x * kWaves) {
        const int32_t p0 = piece_off[q], p1 = piece_off[q + 1];
        if (p1 == p0) continue;   // not split: cand_dw_kernel wrote it
        const int64_t v = large[q];
        for (int64_t h = lane * 8; h < a.hidden; h += kSeg) {
            float acc[8];
            const float4* f = reinterpret_cast<const float4*>(partial + (int64_t)p0 * a.hidden + h);
            acc[0] = f[0].x; acc[1] = f[0].y; acc[2] = f[0].z; acc[3] = f[0].w;
            acc[4] = f[1].x; acc[5] = f[1].y; acc[6] = f[1].z; acc[7] = f[1].w;
            for (int32_t g = p0 + 1; g < p1; ++g) {
                const float4* x = reinterpret_cast<const float4*>(partial + (int64_t)g * a.hidden + h);
                acc[0] += x[0].x; acc[1] += x[0].y; acc[2] += x[0].z; acc[3] += x[0].w;
                acc[4] += x[1].x; acc[5] += x[1].y; acc[6] += x[1].z; acc[7] += x[1].w;
            }
            store_row8(acc, a.dW_acc != nullptr ? a.dW_acc + v * a.hidden + h : nullptr,
                       a.dW != nullptr ? a.dW + v * a.hidden + h : nullptr);
        }
    }
}

}  // namespace lmhead
