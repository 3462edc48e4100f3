// gemm_core.h — bf16 MFMA tile core for gfx950 (CDNA4), shared by every
// contraction of the chunked LM-head path.
//
// One workgroup = 256 threads = 4 wave64s computes a 256 x 256 fp32 tile
// acc[m][n] = sum_k A[m, k] B[n, k]. Waves are laid out 2 x 2; each wave owns
// a 128 x 128 sub-tile, i.e. 8 x 8 blocks of v_mfma_f32_16x16x32_bf16 (256
// fp32 accumulators per lane, in AGPRs). K advances 64 at a time. A goes
// from memory straight into the MFMA fragment registers, read from a copy in
// fragment order; B is staged in LDS by buffer loads that write LDS directly
// (gemm_mainloop_da below). The four contractions of the path:
//   logits (forward and the backward recompute): A = H, B = W (or a chunk);
//   dH: A = dL/dz of the chunk, B = the W chunk read MN-major;
//   dW: computed transposed, A = H^T, B = dL/dz read MN-major.
// MN-major B fragments come from gfx950's transposing LDS reads, so no
// operand is ever transposed in HBM beyond the small H^T copy.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmhead {

typedef uint16_t bf16_bits;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTile = 256;                   // output tile edge (M and N)
constexpr int kTileK = 64;                   // K step per LDS stage
constexpr int kEpiStride = kTile + 4;               // fp32 staging: floats per column
constexpr int kEpiLdsBytes = 128 * kEpiStride * 4;  // one 128-column half, [col][row]
constexpr int kRowStride = 128 + 4;                 // fp32 staging: floats per row, [row][col]
constexpr int kRowLdsBytes = kTile * kRowStride * 4;   // one 128-column half, [row][col]
constexpr int kDaStages = 4;                        // B stages of the K loop
constexpr int kRowBlock = 1024 + 32;                // MN-major B block: two k rows plus a 32-byte bank shift
constexpr int kDaStageMax = 32 * kRowBlock;         // largest B stage (33 KB)
constexpr int kLdsRowConsts = 3 * kTile * 4;        // the dL/dz epilogue's per-row constants, past the staging
constexpr int kMax2(int a, int b) { return a > b ? a : b; }
constexpr int kLdsBytes =
    kMax2(kMax2(kDaStages * kDaStageMax, kEpiLdsBytes + kLdsRowConsts), kRowLdsBytes);
constexpr int kGroupM = 8;                   // row tiles per group in the tile order

// Workgroups are dispatched round-robin over the 8 XCDs, so id i runs on XCD
// i % 8. xcd_order gives each XCD a contiguous range of a logical tile order
// (a bijection of [0, total) that depends only on total); group_tile walks
// that order kGroupM row tiles per column tile, so the workgroups resident on
// one XCD at a time share A and B tiles in that XCD's L2.
__device__ __forceinline__ int64_t xcd_order(int64_t bid, int64_t total) {
    const int64_t q = total / 8, r = total % 8;
    const int64_t x = bid % 8, j = bid / 8;
    return x * q + (x < r ? x : r) + j;
}

__device__ __forceinline__ void group_tile(int64_t L, int64_t tiles_m, int64_t tiles_n, int64_t& tm,
                                           int64_t& tn) {
    const int64_t group = (int64_t)kGroupM * tiles_n;
    const int64_t g = L / group;
    const int64_t first_m = g * kGroupM;
    const int64_t gm = (tiles_m - first_m) < kGroupM ? (tiles_m - first_m) : kGroupM;
    const int64_t in = L - g * group;
    tm = first_m + in % gm;
    tn = in / gm;
}

// Workgroup id -> (row tile, column tile) of one GEMM.
__device__ __forceinline__ void map_tile(int64_t bid, int64_t tiles_m, int64_t tiles_n,
                                         int64_t& tm, int64_t& tn) {
    group_tile(xcd_order(bid, tiles_m * tiles_n), tiles_m, tiles_n, tm, tn);
}

// LDS tile layout: a tile row is 64 bf16 = 128 B = eight 16-byte chunks. The
// LDS has 64 four-byte banks and serves a 16-byte-per-lane read 16 lanes at a
// time, so the 16 rows one quarter-wave reads must land in distinct 16-byte
// bank slots: chunk q of row r is stored at position q ^ ((r >> 1) & 7).
__device__ __forceinline__ int swizzle(int row) { return (row >> 1) & 7; }


// The accumulators: each wave's 128 x 128 sub-tile as 8 x 8 blocks of
// v_mfma_f32_16x16x32_bf16 (block (i, j) covers rows wr*128 + 16 i .. +16 and
// columns wc*128 + 16 j .. +16; lane l, register e holds row 4*(l/16) + e and
// column l%16 of its block). 256 fp32 per lane, in AGPRs. The 16x16x32 form
// moves half as many accumulator bytes per flop as 32x32x16 and sustains a
// higher clock under the board's power limit.
typedef floatx4 AccTile[8][8];

// acc += a * b in place. Issued from inline assembly because the compiler,
// given 64 separate accumulator quads, otherwise copies them between AGPRs
// around every MFMA. The compiler's hazard recognizer does not see these
// MFMAs, so the schedule itself keeps the gfx950 dependency rules for them:
//   - an MFMA whose srcC is an earlier MFMA's vdst needs that MFMA's result:
//     each accumulator is reused only 64 MFMAs later (about a thousand
//     cycles), far past the latency of one 8-pass MFMA;
//   - a VALU read or write of an accumulator needs the MFMA writing it to
//     have finished: mma_drain() puts 48 wait states (three s_nop 15)
//     between the last MFMA and the epilogue's first accumulator access,
//     more than one MFMA's latency, and nothing else touches the
//     accumulators inside the loop;
//   - srcA / srcB registers may be overwritten once the MFMA has read them
//     (its first pass): they are overwritten only by LDS reads and buffer
//     loads issued after it, whose data returns tens to hundreds of cycles
//     later, never by VALU instructions in the loop.
__device__ __forceinline__ void mma16(floatx4& acc, const bf16x8& a, const bf16x8& b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mma_drain() { asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory"); }

// Fragment of 16 rows x 32 k for substep s of a stage: lane l reads row
// rb + l % 16, 16-byte chunk 4 s + l / 16.
__device__ __forceinline__ bf16x8 frag16(const char* base, int rb, int s, int lane) {
    const int row = rb + (lane & 15);
    const int q = 4 * s + (lane >> 4);
    return *reinterpret_cast<const bf16x8*>(base + row * 128 + ((q ^ swizzle(row)) << 4));
}

// MN-major B fragments come from ds_read_b64_tr_b16: within a 16-lane group
// lane i receives element i % 4 of the 8-byte piece addressed by lane
// 4 j + i / 4, as its element j. So lane p of the group addresses k row
// base + p / 4 at mn rb + 4 (p % 4) (four consecutive mn values), lane i
// ends up with k rows base .. base + 3 of mn rb + i, and a second read 4 k
// rows further gives k + 4..7: the 8 k of one MFMA operand per lane.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// ------------------------------------------------------------------------
// The direct-A K loop. A goes from memory straight into the MFMA fragment
// registers; only B is staged in LDS, and it gets there without registers,
// by buffer loads that write LDS directly. Against the staged core above this
// halves the LDS traffic per K step against staging both operands (B only:
// 32 KB written and 64 KB read per workgroup instead of 64 and 128) and
// drops every LDS store instruction from the loop: with A and B both staged
// through registers and LDS stores the loop held the MFMAs at 0.72 busy, with
// this one at 0.80, at the same clock (8192 x 151,936 x 4096 logits GEMM).
//
// A is read from a copy in MFMA fragment order: 16-row x 32-k blocks of
// 1 KB, lane l's 16 bytes (row l % 16, k 8 (l / 16) .. + 8: exactly the
// lane's A operand of one v_mfma_f32_16x16x32_bf16) in one 16-byte slot of
// the block. One fragment load is one fully used 1 KB block (eight 128-byte
// lines); reading the same fragments from a row-major operand touches 16
// rows per 16 lanes and ran at 0.40 MFMA busy, limited by the vector cache's
// line rate. Block orders (rows past the operand are stored as zeros):
//   kATile: block (m / 16, k / 32) at ((m / 16) (K / 32) + k / 32) KB, one
//           descriptor per tile (256 rows x K x 2 bytes < 2^31 by the shape
//           limits). With `perm`, lane l sits in slot pslot(l) (dL/dz, so
//           that the dW contraction's transposing reads of the same blocks
//           are conflict-free).
//   kAStep: block (k / 32, m / 16) at ((k / 32) (M / 16) + m / 16) KB, one
//           descriptor per K step, so any K fits 32-bit offsets (H^T in dW,
//           where K is the row count).
// Register ring: fragments of K steps kt and kt + 1 (2 x 2 substeps x 8
// blocks x 4 registers = 128 VGPRs); the fragment of step kt is reloaded
// with step kt + 2's right after its last MFMA, so each load has two K steps
// to land.
//
// B stage layouts (one K step: 64 k x 256 mn), four stages in a ring; during
// step kt each wave issues eight 1 KB loads of step kt + 3 into the stage
// step kt - 1 released:
//   kBK:    K-major [mn][k] operand (W, a chunk of W): 256 rows of 128 bytes,
//           16-byte chunk q of row r at q ^ ((r >> 1) & 7) (the staged
//           core's layout); 32 KB.
//   kBRow:  MN-major row-major [k][mn] operand (a chunk of W in dH): blocks
//           of two 512-byte k rows, block b = 8 (r / 16) + (r % 4) + 4 ((r / 8)
//           % 2) holding rows r (first half) and r + 4 (second half) for
//           r % 8 < 4, at b x 1056 bytes; 33 KB. A 32-lane transposing read
//           takes k rows {0..3, 8..11} (or {4..7, 12..15}) + 16 q: eight
//           distinct blocks, 32 bytes apart modulo 256, so its 32-byte pieces
//           fill the 64 banks once; every fragment address is one per-lane
//           base plus immediates.
//   kBFrag: MN-major operand stored as fragment blocks (dL/dz as B of dW:
//           mn = chunk column, k = row): the step's 4 x 8 blocks copied
//           verbatim (slot 8 (k / 16) + mn / 32, 32 KB); pslot makes the
//           transposing reads of a block conflict-free.
//
// The stage barrier (mid-step, between the passes of the second substep)
// waits only for this wave's loads of step kt + 1: 48 loads were issued
// after them (the rest of step kt - 2, all of step kt - 1 and step kt up to
// the barrier, 24 per step), so vmcnt(48) leaves the later ones in flight
// (40 in steps 0 and 1, which follow the prologue); the compiler's own
// barrier fence would wait for every load, since it counts the LDS-writing
// loads as LDS stores. The prologue issues B steps 0, 1, 2 and A steps 0, 1
// and waits only for step 0 (vmcnt(32)) before the first MFMA.
constexpr int kATile = 0, kAStep = 1;
constexpr int kBK = 0, kBRow = 1, kBFrag = 2;
static_assert(kDaStages * kDaStageMax <= kLdsBytes, "B ring must fit the LDS");

__host__ __device__ constexpr int da_stage_bytes(int bl) { return bl == kBRow ? 32 * kRowBlock : 32 * 1024; }

// Fragment-order slot of lane l in a dL/dz block: bit 2 flipped when bit 4
// is set (an involution). A dW transposing read takes rows {0..3, 8..11}
// (+ 4) of a block at two consecutive 8-column groups g, g + 1 (lanes
// n + 16 g); flipping bit 2 for odd g puts those 16 lanes' slots in 16
// distinct positions modulo 256 bytes.
__host__ __device__ constexpr int pslot(int l) { return l ^ (((l >> 4) & 1) << 2); }

typedef __attribute__((address_space(3))) void lds_void_t;

// The four B stages of the ring, as four LDS pointers. The MN-major layouts
// (kBRow, kBFrag) are loaded with the LDS-writing buffer-load builtin into
// four separate LDS arrays: the compiler then proves that a transposing read
// of stage ST (an intrinsic) does not touch the stages the loads in flight
// write, instead of draining every load before each read, and it counts
// those loads in its own waits for the A fragments (loads it cannot see would
// make those waits stricter than the schedule needs). kBK kernels pass one
// buffer cut into four stages; their plain LDS reads never needed this.
struct StageSet {
    char* p[4];
};

struct DaA {
    const char* base;   // kATile: the tile's first block; kAStep: the tile's first block of K step 0
    int64_t kblk;       // kATile: bytes per 16-row block (K / 32 KB); kAStep: bytes per K block (M / 16 KB)
    int64_t koff;       // kATile: byte offset of the first K block (K slices)
    int perm;           // kATile: lanes in pslot order
};

struct DaB {
    const char* base;   // kBK: the tile's first row; kBRow: k row 0; kBFrag: block (0, tile's first mn block)
    int64_t ld;         // kBK / kBRow: elements per row; kBFrag: bytes per 16-row block row (mn extent / 32 KB)
    int64_t rows;       // kBK: mn rows in the tile (rest read zero); kBRow: k rows that exist
    int64_t n0;         // kBRow: the tile's first mn column
};

struct DaCtx {
    DaA A;
    DaB B;
    __amdgpu_buffer_rsrc_t ra;    // kATile only
    uint32_t va;                  // lane offset in A
    __amdgpu_buffer_rsrc_t rb;    // kBK only
    uint32_t vb[2];               // lane offsets in B (kBK: even / odd chunk u)
    int64_t KT;
    StageSet st;
    int wave, lane;
};

template <int AM>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t da_a_rsrc(const DaCtx& c, int64_t kt) {
    if (AM == kATile) return c.ra;
    const int64_t ktc = kt < c.KT ? kt : c.KT - 1;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(c.A.base + 2 * ktc * c.A.kblk), 0, (int)(2 * c.A.kblk),
                                             0x00020000);
}

// Fragment (substep s, block i) of K step kt (clamped to the last step).
template <int AM>
__device__ __forceinline__ bf16x8 da_a(const DaCtx& c, __amdgpu_buffer_rsrc_t r, int64_t kt, int s, int i) {
    const int64_t ktc = kt < c.KT ? kt : c.KT - 1;
    const uint32_t soff = AM == kATile ? (uint32_t)(i * c.A.kblk + c.A.koff + ktc * 2048 + s * 1024)
                                       : (uint32_t)(s * c.A.kblk + i * 1024);
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, c.va, soff, 0));
}

// B load u (0..7) of a wave for K step kt into stage ST.
template <int BL, int ST>
__device__ __forceinline__ void da_b(const DaCtx& c, int64_t kt, int u) {
    const int64_t ktc = kt < c.KT ? kt : c.KT - 1;
    char* stage = c.st.p[ST];
    if (BL == kBK) {
        // LDS rows 64 w + 8 u .. + 8 in lane order; lane p loads the chunk that
        // belongs at its position
        char* dst = stage + (c.wave * 64 + u * 8) * 128;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rb, (lds_void_t*)dst, 16, c.vb[u & 1],
                                                 (uint32_t)(u * 8 * c.B.ld * 2 + ktc * 128), 0, 0);
    } else if (BL == kBRow) {
        // block 8 w + u: k rows r1 = 16 w + u % 4 + 8 (u / 4) (lanes 0-31) and
        // r1 + 4 (lanes 32-63), 512 bytes each from the tile's first column;
        // k rows past the operand read as zero
        const int64_t k0 = ktc * kTileK;
        int64_t left = c.B.rows - k0;
        left = left < 0 ? 0 : (left > kTileK ? kTileK : left);
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(c.B.base + k0 * c.B.ld * 2), 0, (int)(left * c.B.ld * 2), 0x00020000);
        const int r1 = c.wave * 16 + (u & 3) + 8 * (u >> 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(stage + (c.wave * 8 + u) * kRowBlock), 16,
                                                 c.vb[0], (uint32_t)(r1 * c.B.ld * 2), 0, 0);
    } else {
        // block (4 kt + w, u) of the tile's columns, 1 KB verbatim
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(c.B.base + 4 * ktc * c.B.ld), 0, (int)(4 * c.B.ld), 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(stage + (c.wave * 8 + u) * 1024), 16, c.vb[0],
                                                 (uint32_t)(c.wave * c.B.ld + u * 1024), 0, 0);
    }
}

// B fragment (block j: mn br + 16 j .. + 16, substep s) from a stage.
template <int BL>
__device__ __forceinline__ bf16x8 da_bfrag(const char* stage, const DaCtx& c, uint32_t lo, uint32_t hi, int br,
                                           int j, int s) {
    if (BL == kBK) return frag16(stage, br + 16 * j, s, c.lane);
    const int imm = BL == kBRow ? s * 16 * kRowBlock + 32 * j : s * 16384 + (j >> 1) * 1024 + (j & 1) * 512;
    const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(stage + lo + imm));
    const i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(stage + hi + imm));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
}

// K step kt, reading B stage ST = kt % 4: two 32-deep substeps of 64 MFMAs,
// each in two passes (column blocks 0-3, then 4-7). B fragments are single
// buffered: early in pass 1 the substep's blocks 4-7 are read; early in pass
// 2 the next substep's blocks 0-3 (after the stage barrier, from the next
// stage). Each A fragment is reloaded with step kt + 2's right after its last
// MFMA (in pass 2). B loads of step kt + 3 go out every 12 MFMAs from the
// first. sched_barrier pins this order.
template <int AM, int BL, int ST>
__device__ __forceinline__ void da_step(const DaCtx& c, int64_t kt, AccTile& acc, bf16x8 (&fa)[2][2][8],
                                        bf16x8 (&fb)[8], uint32_t blo, uint32_t bhi) {
    constexpr int P = ST & 1;
    const char* cur = c.st.p[ST];
    const char* nxt = c.st.p[(ST + 1) & 3];
    const int br = (c.wave & 1) * 128;
    const __amdgpu_buffer_rsrc_t ra2 = da_a_rsrc<AM>(c, kt + 2);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int t = 0; t < 32; ++t) {
            const int bi = t >> 2, bj = t & 3;
            mma16(acc[bi][bj], fa[P][s][bi], fb[bj]);
            if ((t & 1) && t < 8) fb[4 + (t >> 1)] = da_bfrag<BL>(cur, c, blo, bhi, br, 4 + (t >> 1), s);
            const int pos = s * 64 + t;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (u * 12 == pos) da_b<BL, (ST + 3) & 3>(c, kt + 3, u);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (s == 1) {
            // steps 0 and 1 follow the prologue, after whose loads of steps
            // 1 and 2 only 40 loads were issued
            if (kt < 2) asm volatile("s_waitcnt vmcnt(40) lgkmcnt(0)\n\ts_barrier" ::: "memory");
            else asm volatile("s_waitcnt vmcnt(48) lgkmcnt(0)\n\ts_barrier" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        }
        const char* src = s == 0 ? cur : nxt;
        const int s2 = s == 0 ? 1 : 0;
#pragma unroll
        for (int t = 0; t < 32; ++t) {
            const int bi = t >> 2, bj = 4 + (t & 3);
            mma16(acc[bi][bj], fa[P][s][bi], fb[bj]);
            if ((t & 3) == 3) fa[P][s][bi] = da_a<AM>(c, ra2, kt + 2, s, bi);
            if ((t & 1) && t < 8) fb[t >> 1] = da_bfrag<BL>(src, c, blo, bhi, br, t >> 1, s2);
            const int pos = s * 64 + 32 + t;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (u * 12 == pos) da_b<BL, (ST + 3) & 3>(c, kt + 3, u);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// acc = sum over K of A(m, k) B(n, k) for one 256 x 256 tile: A in fragment
// order (AM), B in layout BL (see above). K: a multiple of 64. Whatever the
// layouts, lane l of block (i, j) gets k = 32 s + 8 (l / 16) .. + 8 of each
// substep in the same MFMA slot, so each output element is one fixed-order
// sum over ascending K.
template <int AM, int BL>
__device__ __forceinline__ void gemm_mainloop_da(const DaA& A, const DaB& B, int64_t K, const StageSet& st,
                                                 AccTile& acc) {
    const int tid = threadIdx.x;
    DaCtx c;
    c.A = A;
    c.B = B;
    c.KT = K / kTileK;
    c.st = st;
    c.lane = tid & 63;
    c.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = c.wave >> 1;
    if (AM == kATile) {
        c.ra = __builtin_amdgcn_make_buffer_rsrc((void*)A.base, 0, (int)(16 * A.kblk), 0x00020000);
        c.va = (uint32_t)(wr * 8 * A.kblk + (A.perm ? pslot(c.lane) : c.lane) * 16);
    } else {
        c.ra = c.rb;   // unused
        c.va = (uint32_t)((wr * 8 + 0) * 1024 + c.lane * 16);
    }
    uint32_t blo = 0, bhi = 0;
    const int p = c.lane & 15, G = c.lane >> 4;
    if (BL == kBK) {
        c.rb = __builtin_amdgcn_make_buffer_rsrc((void*)B.base, 0, (int)(B.rows * B.ld * 2), 0x00020000);
        // row r + 8 u has swizzle(r) ^ 4 for odd u
        const int r = c.wave * 64 + (c.lane >> 3);
        const int q = (c.lane & 7) ^ swizzle(r);
        c.vb[0] = (uint32_t)((r * B.ld + q * 8) * 2);
        c.vb[1] = (uint32_t)((r * B.ld + (q ^ 4) * 8) * 2);
    } else if (BL == kBRow) {
        c.rb = c.ra;
        c.vb[0] = (uint32_t)(((c.lane >> 5) * 4 * B.ld + B.n0) * 2 + (c.lane & 31) * 16);
        c.vb[1] = c.vb[0];
        // k row 32 s + 8 G + p / 4 of the group's 16-lane half: block
        // 8 (G / 2) + 4 (G % 2) + p / 4 (+ 16 s), first half; + 4 rows: second half
        const int br = (c.wave & 1) * 128;
        blo = (uint32_t)(((G >> 1) * 8 + 4 * (G & 1) + (p >> 2)) * kRowBlock + (br + 4 * (p & 3)) * 2);
        bhi = blo + 512;
    } else {
        c.rb = c.ra;
        c.vb[0] = (uint32_t)(c.lane * 16);
        c.vb[1] = c.vb[0];
        // rows n = 8 (G % 2) + p / 4 of k block G / 2, columns 4 (p % 4) .. + 4 of
        // the 16-column group: lane slot pslot(n + 16 g), g = 2 (j % 2) + (p % 4) / 2
        const int br = (c.wave & 1) * 128;
        const int n = 8 * (G & 1) + (p >> 2), gb = (p & 3) >> 1;
        const int slot_lo = pslot(n + 16 * gb), slot_hi = pslot(n + 4 + 16 * gb);
        const uint32_t base = (uint32_t)((G >> 1) * 8192 + (br / 32) * 1024 + 8 * (p & 1));
        blo = base + (uint32_t)slot_lo * 16;
        bhi = base + (uint32_t)slot_hi * 16;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.0f;
    bf16x8 fa[2][2][8];
    // prologue: B steps 0, 1, 2 into stages 0, 1, 2; A steps 0 and 1 into the ring
    const __amdgpu_buffer_rsrc_t r0 = da_a_rsrc<AM>(c, 0), r1 = da_a_rsrc<AM>(c, 1);
#pragma unroll
    for (int u = 0; u < 8; ++u) da_b<BL, 0>(c, 0, u);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) fa[0][s][i] = da_a<AM>(c, r0, 0, s, i);
#pragma unroll
    for (int u = 0; u < 8; ++u) da_b<BL, 1>(c, 1, u);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) fa[1][s][i] = da_a<AM>(c, r1, 1, s, i);
#pragma unroll
    for (int u = 0; u < 8; ++u) da_b<BL, 2>(c, 2, u);
    // the first MFMAs need only step 0: B step 0 of every wave (32 loads were
    // issued after this wave's) and this wave's A step 0
    asm volatile("s_waitcnt vmcnt(32)\n\ts_barrier" ::: "memory");
    bf16x8 fb[8];
    const int br = (c.wave & 1) * 128;
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = da_bfrag<BL>(c.st.p[0], c, blo, bhi, br, j, 0);
    int64_t kt = 0;
    for (; kt + 3 < c.KT; kt += 4) {
        da_step<AM, BL, 0>(c, kt, acc, fa, fb, blo, bhi);
        da_step<AM, BL, 1>(c, kt + 1, acc, fa, fb, blo, bhi);
        da_step<AM, BL, 2>(c, kt + 2, acc, fa, fb, blo, bhi);
        da_step<AM, BL, 3>(c, kt + 3, acc, fa, fb, blo, bhi);
    }
    if (kt < c.KT) da_step<AM, BL, 0>(c, kt, acc, fa, fb, blo, bhi);
    if (kt + 1 < c.KT) da_step<AM, BL, 1>(c, kt + 1, acc, fa, fb, blo, bhi);
    if (kt + 2 < c.KT) da_step<AM, BL, 2>(c, kt + 2, acc, fa, fb, blo, bhi);
    mma_drain();
    // every load (the clamped ones past the last step included) has landed
    // before the epilogue reuses the LDS
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The same with the four stages cut from one LDS buffer (the K-major layout).
template <int AM, int BL>
__device__ __forceinline__ void gemm_mainloop_da(const DaA& A, const DaB& B, int64_t K, char* smem, AccTile& acc) {
    static_assert(BL == kBK, "the MN-major layouts take four separate stage arrays");
    constexpr int SB = da_stage_bytes(BL);
    const StageSet st{{smem, smem + SB, smem + 2 * SB, smem + 3 * SB}};
    gemm_mainloop_da<AM, BL>(A, B, K, st, acc);
}

// Write the accumulators of the waves whose column half is `half` into the
// fp32 staging area S laid out [column 0..127][row 0..255] (stride kEpiStride):
// afterwards thread t can walk row t of that half with conflict-free reads.
__device__ __forceinline__ void stage_half(float* S, const AccTile& acc, int wr, int lane) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int col = j * 16 + (lane & 15);
            const int row = wr * 128 + i * 16 + 4 * (lane >> 4);
            *reinterpret_cast<floatx4*>(S + col * kEpiStride + row) = acc[i][j];
        }
}

// The same half tile laid out [row 0..255][column 0..127] with a row stride of
// kRowStride floats (4 mod 64 banks: the four row groups one 32-bit store
// instruction writes, 4 rows apart, fall 16 banks apart). Afterwards 32 lanes
// can read one row's 128 values as float4s, conflict-free, for coalesced
// row-major global traffic. The rows are spread over the four stage arrays of
// the K loop, 64 rows each (64 x kRowStride x 4 bytes = one kBRow stage):
// rows 64 q .. 64 q + 63 in array q, so wave w later reads its own rows
// 64 w .. + 63 from array w alone.
static_assert(64 * kRowStride * 4 <= kDaStageMax, "64 staged rows must fit one stage array");
__device__ __forceinline__ float* stage_rows(const StageSet& st, int q) {
    return reinterpret_cast<float*>(q == 0 ? st.p[0] : q == 1 ? st.p[1] : q == 2 ? st.p[2] : st.p[3]);
}
__device__ __forceinline__ void stage_half_rows(const StageSet& st, const AccTile& acc, int wr, int lane) {
    float* const lo = stage_rows(st, 2 * wr);       // rows wr * 128 + 0 .. 63
    float* const hi = stage_rows(st, 2 * wr + 1);   // rows wr * 128 + 64 .. 127
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = (i & 3) * 16 + 4 * (lane >> 4) + e;   // within its 64-row array
                const int col = j * 16 + (lane & 15);
                (i < 4 ? lo : hi)[row * kRowStride + col] = acc[i][j][e];
            }
}

// fp32 -> bf16, round to nearest even: the conversion lowers to gfx950's
// v_cvt_pk_bf16_f32, two values per instruction, packed low | high << 16.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

}  // namespace lmhead
