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
// Waves are laid out 2 x 2; each wave owns a 128 x 128 sub-tile, i.e. 4 x 4
// blocks of v_mfma_f32_32x32x16_bf16 (256 fp32 accumulators per lane).
// K advances 64 at a time through two LDS stages of 64 KB (A and B tiles of
// 256 x 64 bf16 each), filled by direct global -> LDS loads (no VGPR staging).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmhead {

typedef uint16_t bf16_bits;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTile = 256;                   // output tile edge (M and N)
constexpr int kTileK = 64;                   // K step per LDS stage
constexpr int kOperandBytes = kTile * kTileK * 2;   // 32 KB
constexpr int kStageBytes = 2 * kOperandBytes;      // 64 KB
constexpr int kMainLdsBytes = 2 * kStageBytes;      // 128 KB
constexpr int kEpiStride = kTile + 4;               // fp32 staging: floats per column
constexpr int kEpiLdsBytes = 128 * kEpiStride * 4;  // one 128-column half, [col][row]
constexpr int kLdsBytes = kMainLdsBytes > kEpiLdsBytes ? kMainLdsBytes : kEpiLdsBytes;
constexpr int kGroupM = 8;                   // row tiles per group in the tile order

// Row-major bf16 operand with K contiguous; rows beyond `rows` are clamped to
// the last row (their products land in masked output rows / columns).
struct Operand {
    const bf16_bits* ptr;
    int64_t ld;
    int64_t rows;
};

// Workgroup id -> (row tile, column tile). Workgroups are dispatched
// round-robin over the 8 XCDs, so id i runs on XCD i % 8. Each XCD is given a
// contiguous range of the logical tile order, and that order walks kGroupM row
// tiles for each column tile: the workgroups resident on one XCD at a time
// share A and B tiles in that XCD's L2. The mapping is a bijection that
// depends only on the grid shape.
__device__ __forceinline__ void map_tile(int64_t bid, int64_t tiles_m, int64_t tiles_n,
                                         int64_t& tm, int64_t& tn) {
    const int64_t total = tiles_m * tiles_n;
    const int64_t q = total / 8, r = total % 8;
    const int64_t x = bid % 8, j = bid / 8;
    const int64_t L = x * q + (x < r ? x : r) + j;
    const int64_t group = (int64_t)kGroupM * tiles_n;
    const int64_t g = L / group;
    const int64_t first_m = g * kGroupM;
    const int64_t gm = (tiles_m - first_m) < kGroupM ? (tiles_m - first_m) : kGroupM;
    const int64_t in = L - g * group;
    tm = first_m + in % gm;
    tn = in / gm;
}

// LDS tile layout: a tile row is 64 bf16 = 128 B = eight 16-byte chunks. The
// LDS has 64 four-byte banks and serves a 16-byte-per-lane read 16 lanes at a
// time, so the 16 rows one quarter-wave reads must land in distinct 16-byte
// bank slots: chunk q of row r is stored at position q ^ ((r >> 1) & 7).
__device__ __forceinline__ int swizzle(int row) { return (row >> 1) & 7; }

__device__ __forceinline__ bf16x8 lds_fragment(const char* base, int row, int q) {
    return *reinterpret_cast<const bf16x8*>(base + row * 128 + ((q ^ swizzle(row)) << 4));
}

// One direct global -> LDS load (16 bytes per lane, 1 KB per wave) of stage
// data: u = 0..7 load eight rows of A, u = 8..15 eight rows of B. Wave w owns
// rows [64 w, 64 w + 64) of both operands. The lanes of one instruction write
// 1 KB of LDS contiguously (lane l at offset 16 l), so lane l fetches the
// global chunk that belongs at that swizzled position.
__device__ __forceinline__ void stage_load(const Operand& A, int64_t m0, const Operand& B, int64_t n0,
                                           int64_t k0, char* stage, int wave, int lane, int u) {
    const Operand& op = u < 8 ? A : B;
    const int64_t row0 = u < 8 ? m0 : n0;
    char* base = stage + (u < 8 ? 0 : kOperandBytes);
    const int i = u & 7;
    const int r = wave * 64 + i * 8 + (lane >> 3);
    const int q = (lane & 7) ^ swizzle(r);
    int64_t row = row0 + r;
    row = row < op.rows ? row : op.rows - 1;
    const bf16_bits* g = op.ptr + row * op.ld + k0 + q * 8;
    __builtin_amdgcn_global_load_lds((const void*)g,
                                     (__attribute__((address_space(3))) void*)(base + (wave * 64 + i * 8) * 128),
                                     16, 0, 0);
}

// acc[i][j] covers rows wr*128 + 32 i .. +32 and columns wc*128 + 32 j .. +32 of
// the tile. Lane l, register e of a 32x32 block holds row 8*(e/4) + 4*(l/32) +
// e%4 and column l%32.
//
// Schedule of one 64-wide K step (four 16-wide substeps of 16 MFMAs each):
// every other MFMA is followed by one fragment read for the next substep and
// every fourth by one stage load for step kt+1, so LDS reads and the global ->
// LDS traffic run under the MFMAs. The stage barrier sits in the middle of the
// last substep: after it, step kt+1's fragments are read and step kt+2's loads
// start into the buffer step kt just finished with, which gives every load a
// full step of latency cover. sched_barrier pins this order.
__device__ __forceinline__ void gemm_mainloop(const Operand& A, int64_t m0, const Operand& B,
                                              int64_t n0, int64_t K, char* smem,
                                              floatx16 (&acc)[4][4]) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave >> 1, wc = wave & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    const int64_t KT = K / kTileK;
    const int arow = wr * 128 + (lane & 31);
    const int brow = wc * 128 + (lane & 31);
    const int qh = lane >> 5;

    // prologue: step 0 resident, the first quarter of step 1 in flight, step 0's first fragments
#pragma unroll
    for (int u = 0; u < 16; ++u) stage_load(A, m0, B, n0, 0, smem, wave, lane, u);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int64_t k1 = (KT > 1 ? 1 : 0) * kTileK;
#pragma unroll
    for (int u = 0; u < 4; ++u) stage_load(A, m0, B, n0, k1, smem + kStageBytes, wave, lane, u);
    bf16x8 fa[2][4], fb[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        fa[0][i] = lds_fragment(smem, arow + 32 * i, qh);
        fb[0][i] = lds_fragment(smem + kOperandBytes, brow + 32 * i, qh);
    }

    for (int64_t kt = 0; kt < KT; ++kt) {
        const char* cur = smem + (kt & 1) * kStageBytes;
        char* nxt = smem + ((kt + 1) & 1) * kStageBytes;    // step kt+1
        char* nxt2 = smem + (kt & 1) * kStageBytes;         // step kt+2, after the barrier
        // past the end, loads repeat the last step into the idle buffer (never read)
        const int64_t kn1 = (kt + 1 < KT ? kt + 1 : KT - 1) * kTileK;
        const int64_t kn2 = (kt + 2 < KT ? kt + 2 : KT - 1) * kTileK;
#pragma unroll
        for (int ks = 0; ks < 3; ++ks) {
            const int c = ks & 1;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const int i = t >> 2, j = t & 3;
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[c][i], fb[c][j], acc[i][j], 0, 0, 0);
                if ((t & 3) == 0) stage_load(A, m0, B, n0, kn1, nxt, wave, lane, 4 + ks * 4 + (t >> 2));
                if (t & 1) {
                    const int r = t >> 1;   // fa0 fb0 fa1 fb1 ...
                    if (r & 1)
                        fb[c ^ 1][r >> 1] = lds_fragment(cur + kOperandBytes, brow + 32 * (r >> 1), (ks + 1) * 2 + qh);
                    else
                        fa[c ^ 1][r >> 1] = lds_fragment(cur, arow + 32 * (r >> 1), (ks + 1) * 2 + qh);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int i = t >> 2, j = t & 3;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[1][i], fb[1][j], acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 8; t < 16; ++t) {
            const int i = t >> 2, j = t & 3;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[1][i], fb[1][j], acc[i][j], 0, 0, 0);
            const int r = t - 8;
            if (r & 1)
                fb[0][r >> 1] = lds_fragment(nxt + kOperandBytes, brow + 32 * (r >> 1), qh);
            else
                fa[0][r >> 1] = lds_fragment(nxt, arow + 32 * (r >> 1), qh);
            if ((t & 1) == 0) stage_load(A, m0, B, n0, kn2, nxt2, wave, lane, (t - 8) >> 1);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // the trailing loads land before the epilogue reuses the LDS
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
}

// Write the accumulators of the waves whose column half is `half` into the
// fp32 staging area S laid out [column 0..127][row 0..255] (stride kEpiStride):
// afterwards thread t can walk row t of that half with conflict-free reads.
__device__ __forceinline__ void stage_half(float* S, const floatx16 (&acc)[4][4], int wr, int lane) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = j * 32 + (lane & 31);
                const int row = wr * 128 + i * 32 + 8 * g + 4 * (lane >> 5);
                floatx4 v;
                v[0] = acc[i][j][4 * g + 0];
                v[1] = acc[i][j][4 * g + 1];
                v[2] = acc[i][j][4 * g + 2];
                v[3] = acc[i][j][4 * g + 3];
                *reinterpret_cast<floatx4*>(S + col * kEpiStride + row) = v;
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
