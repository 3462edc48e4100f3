// gemm_core.h — bf16 MFMA tile core for gfx950 (CDNA4), shared by every
// contraction of the chunked LM-head path.
//
// One workgroup = 256 threads = 4 wave64s computes a 256 x 256 fp32 tile
// C[m0:m0+256, n0:n0+256] = A[m0:, :] * B[n0:, :]^T where both operands are
// row-major with the contraction dimension K contiguous ("NT" form). The
// logits GEMM (z = H W^T) is natively NT; the two backward contractions are
// brought to NT form by giving them operands stored contraction-contiguous
// (the host-side plan transposes H and the W chunk once, and the dL/dz tile
// is written in both layouts).
//
// Waves are laid out 2 x 2; each wave owns a 128 x 128 sub-tile, i.e. 8 x 8
// blocks of v_mfma_f32_16x16x32_bf16 (256 fp32 accumulators per lane, in
// AGPRs). K advances 64 at a time through two LDS stages of 64 KB (A and B
// tiles of 256 x 64 bf16 each). Global data reaches LDS through registers:
// each wave holds two more K steps in flight in VGPRs (2 x 64 registers), so
// a load has about one and a half K steps to return before it is needed —
// with only two 64 KB LDS stages, loads straight into LDS could be issued at
// most one step ahead, and the waves then spent about a third of their time
// waiting for them.
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
constexpr int kOperandBytes = kTile * kTileK * 2;   // 32 KB
constexpr int kStageBytes = 2 * kOperandBytes;      // 64 KB
constexpr int kMainLdsBytes = 2 * kStageBytes;      // 128 KB
constexpr int kEpiStride = kTile + 4;               // fp32 staging: floats per column
constexpr int kEpiLdsBytes = 128 * kEpiStride * 4;  // one 128-column half, [col][row]
constexpr int kRowStride = 128 + 4;                 // fp32 staging: floats per row, [row][col]
constexpr int kRowLdsBytes = kTile * kRowStride * 4;   // one 128-column half, [row][col]
constexpr int kLdsBytes0 = kMainLdsBytes > kEpiLdsBytes ? kMainLdsBytes : kEpiLdsBytes;
constexpr int kLdsBytes = kLdsBytes0 > kRowLdsBytes ? kLdsBytes0 : kRowLdsBytes;
constexpr int kGroupM = 8;                   // row tiles per group in the tile order

// Row-major bf16 operand with K contiguous; rows at or beyond `rows` read as
// zero (their products land in masked output rows / columns).
struct Operand {
    const bf16_bits* ptr;
    int64_t ld;
    int64_t rows;
};

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

__device__ __forceinline__ bf16x8 lds_fragment(const char* base, int row, int q) {
    return *reinterpret_cast<const bf16x8*>(base + row * 128 + ((q ^ swizzle(row)) << 4));
}

// ------------------------------------------------------------------------
// The K loop.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Buffer load of one 16-byte chunk per lane. The descriptor starts at the
// tile's first row and ends at the operand's last row, so rows past the end
// read as zero (no clamping). voff: the lane's byte offset within an 8-row
// group; soff: the group's byte offset plus the K offset (uniform).
__device__ __forceinline__ u32x4_t stage_fetch_b(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, soff, 0));
}

// Staging chunk u of a wave (u = 0..7: eight rows of A, 8..15: of B; wave w
// owns rows [64 w, 64 w + 64)) into its swizzled LDS position.
__device__ __forceinline__ void stage_put(char* stage, int wave, int lane, int u, const u32x4_t& v) {
    char* base = stage + (u < 8 ? 0 : kOperandBytes);
    const int r = wave * 64 + (u & 7) * 8 + (lane >> 3);
    const int q = (lane & 7) ^ swizzle(r);
    *reinterpret_cast<u32x4_t*>(base + r * 128 + (q << 4)) = v;
}

struct PgCtx {
    __amdgpu_buffer_rsrc_t ra, rb;
    uint32_t voff_a, voff_b;     // lane offsets (bytes) within an 8-row group, wave's rows included
    uint32_t step_a, step_b;     // bytes per 8 rows
    int64_t KT;
    char* smem;
    int wave, lane;
};

__device__ __forceinline__ u32x4_t pg_fetch(const PgCtx& c, int64_t k0, int u) {
    const uint32_t kb = (uint32_t)(k0 * 2);
    if (u < 8) return stage_fetch_b(c.ra, c.voff_a, (uint32_t)(u & 7) * c.step_a + kb);
    return stage_fetch_b(c.rb, c.voff_b, (uint32_t)(u & 7) * c.step_b + kb);
}

// The accumulators: each wave's 128 x 128 sub-tile as 8 x 8 blocks of
// v_mfma_f32_16x16x32_bf16 (block (i, j) covers rows wr*128 + 16 i .. +16 and
// columns wc*128 + 16 j .. +16; lane l, register e holds row 4*(l/16) + e and
// column l%16 of its block). 256 fp32 per lane, in AGPRs. The 16x16x32 form
// moves half as many accumulator bytes per flop as 32x32x16 and sustains a
// higher clock under the board's power limit.
typedef floatx4 AccTile[8][8];

// acc += a * b in place. Issued from inline assembly because the compiler,
// given 64 separate accumulator quads, otherwise copies them between AGPRs
// around every MFMA. The hazard recognizer does not see these MFMAs: each
// accumulator is reused only 64 MFMAs later, A / B registers are overwritten
// only by LDS reads (whose data returns long after the MFMA has read its
// operands), and mma_drain() separates the last MFMA from any read of acc.
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

// One 64-wide K step kt of parity P: two 32-wide substeps of 64 MFMAs, each
// in two passes (columns blocks 0-3, then 4-7). Fragments are single
// buffered: early in pass 1 the substep's B blocks 4-7 are read; early in pass
// 2 the next substep's B blocks 0-3, and each A block for the next substep
// right after its last use. Register set [1 - P] holds step kt+1 and set [P] step kt+2
// (loads in flight): over the first 96 MFMAs, chunk u of step kt+1 is stored
// to the LDS buffer that step kt-1 released and its registers are at once
// reloaded with chunk u of step kt+3 (16 evenly spaced store / load pairs, two
// full K steps of latency cover per chunk; the compiler's vmcnt wait before
// each store is per register). The stage barrier sits between the passes of
// the second substep; the reads after it fetch step kt+1's first fragments.
// sched_barrier pins the order.
template <int P>
__device__ __forceinline__ void pg_step(const PgCtx& c, int64_t kt, AccTile& acc, bf16x8 (&fa)[8], bf16x8 (&fb)[8],
                                        u32x4_t (&s0)[16], u32x4_t (&s1)[16]) {
    u32x4_t (&sn)[16] = P ? s0 : s1;    // step kt+1, then kt+3
    const char* cur = c.smem + P * kStageBytes;
    char* nxt = c.smem + (1 - P) * kStageBytes;
    const int64_t k3 = (kt + 3 < c.KT ? kt + 3 : c.KT - 1) * kTileK;
    const int ar = (c.wave >> 1) * 128, br = (c.wave & 1) * 128;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int t = 0; t < 32; ++t) {
            const int bi = t >> 2, bj = t & 3;
            mma16(acc[bi][bj], fa[bi], fb[bj]);
            if ((t & 1) && t < 8) fb[4 + (t >> 1)] = frag16(cur + kOperandBytes, br + 16 * (4 + (t >> 1)), s, c.lane);
            const int pos = s * 64 + t;
#pragma unroll
            for (int u = 0; u < 16; ++u)
                if (u * 6 == pos) {
                    stage_put(nxt, c.wave, c.lane, u, sn[u]);
                    sn[u] = pg_fetch(c, k3, u);
                }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (s == 1) {
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
        }
        const char* src = s == 0 ? cur : nxt;
        const int s2 = s == 0 ? 1 : 0;
#pragma unroll
        for (int t = 0; t < 32; ++t) {
            const int bi = t >> 2, bj = 4 + (t & 3);
            mma16(acc[bi][bj], fa[bi], fb[bj]);
            if ((t & 3) == 3) fa[bi] = frag16(src, ar + 16 * bi, s2, c.lane);
            if ((t & 1) && t < 8) fb[t >> 1] = frag16(src + kOperandBytes, br + 16 * (t >> 1), s2, c.lane);
            const int pos = s * 64 + 32 + t;
#pragma unroll
            for (int u = 0; u < 16; ++u)
                if (u * 6 == pos) {
                    stage_put(nxt, c.wave, c.lane, u, sn[u]);
                    sn[u] = pg_fetch(c, k3, u);
                }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// C[m0.., n0..] = A[m0.., :K] B[n0.., :K]^T for one 256 x 256 tile. K must
// be a multiple of 64.
__device__ __forceinline__ void gemm_mainloop(const Operand& A, int64_t m0, const Operand& B, int64_t n0,
                                              int64_t K, char* smem, AccTile& acc) {
    const int tid = threadIdx.x;
    PgCtx c;
    c.KT = K / kTileK;
    c.smem = smem;
    c.lane = tid & 63;
    c.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    {
        const int64_t ra_rows = A.rows - m0 < kTile ? A.rows - m0 : kTile;
        const int64_t rb_rows = B.rows - n0 < kTile ? B.rows - n0 : kTile;
        c.ra = __builtin_amdgcn_make_buffer_rsrc((void*)(A.ptr + m0 * A.ld), 0, (int)(ra_rows * A.ld * 2), 0x00020000);
        c.rb = __builtin_amdgcn_make_buffer_rsrc((void*)(B.ptr + n0 * B.ld), 0, (int)(rb_rows * B.ld * 2), 0x00020000);
        const int r = c.wave * 64 + (c.lane >> 3);
        c.voff_a = (uint32_t)((r * A.ld + (c.lane & 7) * 8) * 2);
        c.voff_b = (uint32_t)((r * B.ld + (c.lane & 7) * 8) * 2);
        c.step_a = (uint32_t)(8 * A.ld * 2);
        c.step_b = (uint32_t)(8 * B.ld * 2);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.0f;
    auto kof = [&](int64_t s) { return (s < c.KT ? s : c.KT - 1) * kTileK; };
    u32x4_t s0[16], s1[16];
    // prologue: step 0 -> set 0 -> LDS buffer 0; step 1 -> set 1 (stored during step 0); step 2 -> set 0
#pragma unroll
    for (int u = 0; u < 16; ++u) s0[u] = pg_fetch(c, kof(0), u);
#pragma unroll
    for (int u = 0; u < 16; ++u) s1[u] = pg_fetch(c, kof(1), u);
#pragma unroll
    for (int u = 0; u < 16; ++u) stage_put(smem, c.wave, c.lane, u, s0[u]);
#pragma unroll
    for (int u = 0; u < 16; ++u) s0[u] = pg_fetch(c, kof(2), u);
    __syncthreads();
    bf16x8 fa[8], fb[8];
    const int ar = (c.wave >> 1) * 128, br = (c.wave & 1) * 128;
#pragma unroll
    for (int i = 0; i < 8; ++i) fa[i] = frag16(smem, ar + 16 * i, 0, c.lane);
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = frag16(smem + kOperandBytes, br + 16 * j, 0, c.lane);
    int64_t kt = 0;
    for (; kt + 1 < c.KT; kt += 2) {
        pg_step<0>(c, kt, acc, fa, fb, s0, s1);
        pg_step<1>(c, kt + 1, acc, fa, fb, s0, s1);
    }
    if (kt < c.KT) pg_step<0>(c, kt, acc, fa, fb, s0, s1);
    mma_drain();
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
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
// row-major global traffic.
__device__ __forceinline__ void stage_half_rows(float* S, const AccTile& acc, int wr, int lane) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = wr * 128 + i * 16 + 4 * (lane >> 4) + e;
                const int col = j * 16 + (lane & 15);
                S[row * kRowStride + col] = acc[i][j][e];
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
