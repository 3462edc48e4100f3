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
// 256 x 64 bf16 each). Global loads for stage k+1 are issued before the MFMAs
// of stage k, so HBM/L2 latency hides behind 64 MFMAs per wave.
//
// LDS layout: a tile row is 64 bf16 = 128 B = eight 16-byte chunks; chunk q of
// row r is stored at chunk position q ^ (r & 7), so the 32 rows one MFMA
// fragment read touches spread over all banks.
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

// The 8 x 16 bytes one thread moves per operand and stage are held in one
// 32-wide vector value (not an array) so they stay in VGPRs between the
// global load and the LDS store.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x32 __attribute__((ext_vector_type(32)));

__device__ __forceinline__ u32x32 global_tile_load(const Operand& op, int64_t row0, int64_t k0, int tid) {
    const int q = tid & 7;
    u32x32 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int64_t row = row0 + (tid >> 3) + 32 * i;
        row = row < op.rows ? row : op.rows - 1;
        const u32x4 x = *reinterpret_cast<const u32x4*>(op.ptr + row * op.ld + k0 + q * 8);
        r[4 * i + 0] = x[0];
        r[4 * i + 1] = x[1];
        r[4 * i + 2] = x[2];
        r[4 * i + 3] = x[3];
    }
    return r;
}

__device__ __forceinline__ void lds_tile_store(char* base, int tid, const u32x32& r) {
    const int q = tid & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = (tid >> 3) + 32 * i;
        u32x4 x;
        x[0] = r[4 * i + 0];
        x[1] = r[4 * i + 1];
        x[2] = r[4 * i + 2];
        x[3] = r[4 * i + 3];
        *reinterpret_cast<u32x4*>(base + row * 128 + ((q ^ (row & 7)) << 4)) = x;
    }
}

__device__ __forceinline__ bf16x8 lds_fragment(const char* base, int row, int q) {
    return *reinterpret_cast<const bf16x8*>(base + row * 128 + ((q ^ (row & 7)) << 4));
}

// acc[i][j] covers rows wr*128 + 32 i .. +32 and columns wc*128 + 32 j .. +32 of
// the tile. Lane l, register e of a 32x32 block holds row 8*(e/4) + 4*(l/32) +
// e%4 and column l%32.
__device__ __forceinline__ void gemm_mainloop(const Operand& A, int64_t m0, const Operand& B,
                                              int64_t n0, int64_t K, char* smem,
                                              floatx16 (&acc)[4][4]) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    u32x32 ra = global_tile_load(A, m0, 0, tid);
    u32x32 rb = global_tile_load(B, n0, 0, tid);
    lds_tile_store(smem, tid, ra);
    lds_tile_store(smem + kOperandBytes, tid, rb);
    __syncthreads();

    const int64_t KT = K / kTileK;
    const int arow = wr * 128 + (lane & 31);
    const int brow = wc * 128 + (lane & 31);
    const int qh = lane >> 5;
    for (int64_t kt = 0; kt < KT; ++kt) {
        const char* cur = smem + (kt & 1) * kStageBytes;
        const bool more = kt + 1 < KT;
        if (more) {
            ra = global_tile_load(A, m0, (kt + 1) * kTileK, tid);
            rb = global_tile_load(B, n0, (kt + 1) * kTileK, tid);
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bf16x8 fa[4], fb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                fa[i] = lds_fragment(cur, arow + 32 * i, ks * 2 + qh);
                fb[i] = lds_fragment(cur + kOperandBytes, brow + 32 * i, ks * 2 + qh);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        if (more) {
            char* nxt = smem + ((kt + 1) & 1) * kStageBytes;
            lds_tile_store(nxt, tid, ra);
            lds_tile_store(nxt + kOperandBytes, tid, rb);
        }
        __syncthreads();
    }
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

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ bf16_bits to_bf16(float x) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_bits)((u >> 16) | 0x40u);
    const uint32_t rounding = 0x7fffu + ((u >> 16) & 1u);
    return (bf16_bits)((u + rounding) >> 16);
}

}  // namespace lmhead
