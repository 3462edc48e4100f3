// gemm_core.h — bf16 MFMA tile core for gfx950 (CDNA4), shared by every
// contraction of the chunked LM-head path.
//
// One workgroup = 256 threads = 4 wave64s computes a 256 x 256 fp32 tile
// C[m0:m0+256, n0:n0+256] = sum_k A[m, k] B[n, k]. Each operand is stored
// either K-major (row-major [mn][k], the contraction contiguous) or MN-major
// (row-major [k][mn]). The logits GEMM (z = H W^T) has both operands K-major;
// dW = G^T H reads G and H MN-major, and dH = G W_c reads W_c MN-major, so no
// operand is ever transposed in HBM: an MN-major tile is staged in LDS as
// [k][mn] and its MFMA fragments come from gfx950's transposing LDS reads.
//
// Waves are laid out 2 x 2; each wave owns a 128 x 128 sub-tile, i.e. 8 x 8
// blocks of v_mfma_f32_16x16x32_bf16 (256 fp32 accumulators per lane, in
// AGPRs). K advances 64 at a time through two LDS stages (A and B tiles of
// 256 x 64 bf16 each, in 34 KB slots). Global data reaches LDS through
// registers: each wave holds two more K steps in flight in VGPRs (2 x 64
// registers), so a load has two K steps to return before it is stored —
// with only two LDS stages, loads straight into LDS could be issued at most
// one step ahead, and the waves then spent about a third of their time
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
constexpr int kTPitch = 2 * kTile + 32;             // MN-major LDS tile: bytes per k row (512 + pad)
constexpr int kOperandBytes = kTileK * kTPitch;     // 34 KB slot (a K-major tile uses 32 KB of it)
constexpr int kStageBytes = 2 * kOperandBytes;      // 68 KB
constexpr int kMainLdsBytes = 2 * kStageBytes;      // 136 KB
constexpr int kEpiStride = kTile + 4;               // fp32 staging: floats per column
constexpr int kEpiLdsBytes = 128 * kEpiStride * 4;  // one 128-column half, [col][row]
constexpr int kRowStride = 128 + 4;                 // fp32 staging: floats per row, [row][col]
constexpr int kRowLdsBytes = kTile * kRowStride * 4;   // one 128-column half, [row][col]
constexpr int kLdsBytes0 = kMainLdsBytes > kEpiLdsBytes ? kMainLdsBytes : kEpiLdsBytes;
constexpr int kLdsBytes = kLdsBytes0 > kRowLdsBytes ? kLdsBytes0 : kRowLdsBytes;
constexpr int kGroupM = 8;                   // row tiles per group in the tile order

// Row-major bf16 operand. K-major: element (mn, k) at ptr[mn * ld + k], and
// rows (mn) at or beyond `rows` read as zero (their products land in masked
// output rows / columns). MN-major: element (mn, k) at ptr[k * ld + mn], and
// K rows at or beyond `rows` read as zero; columns past the operand's MN
// extent read the next row's first elements (zero after the last row; never
// memory beyond the operand) and only reach output rows / columns that are
// masked.
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

// Buffer load of one 16-byte chunk per lane. The descriptor's range ends at
// the operand's last row, so rows past the end read as zero (no clamping).
// voff: the lane's byte offset within an 8-row group; soff: the group's byte
// offset (plus, K-major, the K offset), uniform.
__device__ __forceinline__ u32x4_t stage_fetch_b(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, soff, 0));
}

// Staging chunk u of a wave (u = 0..7: eight rows of A, 8..15: of B; wave w
// owns rows [64 w, 64 w + 64)) into its swizzled LDS position: the K-major
// form, a tile row being 64 k of one mn.
__device__ __forceinline__ void stage_put(char* base, int wave, int lane, int u, const u32x4_t& v) {
    const int r = wave * 64 + (u & 7) * 8 + (lane >> 3);
    const int q = (lane & 7) ^ swizzle(r);
    *reinterpret_cast<u32x4_t*>(base + r * 128 + (q << 4)) = v;
}

// MN-major LDS tile: 64 k rows of 256 mn (512 B) at a pitch of kTPitch =
// 17 x 32 bytes, k row r stored as LDS row trow(r) (bits 2 and 3 of r
// swapped). A transposing fragment read takes four consecutive k rows per
// 16-lane group (k = 8 g + 0..3, or + 4..7, for group g) and 32 lanes are
// served together: the swap makes their eight k rows eight consecutive LDS
// rows, whose 32-byte pieces at one column then fall in eight distinct bank
// groups (17 r mod 8). No XOR: every fragment address is one per-lane base
// plus an immediate offset. Stores (16 lanes, 256 contiguous bytes of one
// row) are conflict-free.
__device__ __forceinline__ int trow(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Staging chunk u of a wave for an MN-major tile: k row 8 (u & 7) + 2 w +
// lane / 32, bytes 16 (lane % 32) .. + 16 of the row.
__device__ __forceinline__ void stage_put_t(char* base, int wave, int lane, int u, const u32x4_t& v) {
    const int r = (u & 7) * 8 + wave * 2 + (lane >> 5);
    *reinterpret_cast<u32x4_t*>(base + trow(r) * kTPitch + ((lane & 31) << 4)) = v;
}

// One operand's K stream. K-major: a descriptor over the tile's 256 rows (the
// K offset goes into the scalar offset). MN-major: the descriptor is rebuilt
// for each K step over that step's 64 k rows, so offsets stay small and k rows
// past `krows` read as zero.
struct OpStream {
    __amdgpu_buffer_rsrc_t rsrc;  // K-major only
    const char* base;             // MN-major: address of k row 0 (mn = 0)
    int64_t ld_bytes;             // MN-major: bytes per k row
    int64_t krows;                // MN-major: k rows that exist
    uint32_t voff;                // lane offset (bytes) within an 8-row group, wave's rows included
    uint32_t step;                // bytes per 8 rows (K-major) or 8 k rows (MN-major)
};

template <bool T>
__device__ __forceinline__ OpStream make_stream(const Operand& X, int64_t mn0, int wave, int lane) {
    OpStream o;
    if (!T) {
        const int64_t rows = X.rows - mn0 < kTile ? X.rows - mn0 : kTile;
        o.rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(X.ptr + mn0 * X.ld), 0, (int)(rows * X.ld * 2),
                                                   0x00020000);
        o.base = nullptr;
        o.ld_bytes = 0;
        o.krows = 0;
        const int r = wave * 64 + (lane >> 3);
        o.voff = (uint32_t)((r * X.ld + (lane & 7) * 8) * 2);
        o.step = (uint32_t)(8 * X.ld * 2);
    } else {
        o.rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)X.ptr, 0, 0, 0x00020000);
        // the tile's column offset goes into the lane offset, not the base:
        // the range of a step's descriptor then ends with its last k row, and
        // the columns a tile reads past the end of that row read zero
        o.base = reinterpret_cast<const char*>(X.ptr);
        o.ld_bytes = X.ld * 2;
        o.krows = X.rows;
        o.voff = (uint32_t)((wave * 2 + (lane >> 5)) * o.ld_bytes + mn0 * 2 + (lane & 31) * 16);
        o.step = (uint32_t)(8 * o.ld_bytes);
    }
    return o;
}

// The descriptor for K step kt (k0 = 64 kt): k rows k0 .. k0 + 63, cut at
// the operand's last k row (rows past it read zero).
template <bool T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t step_rsrc(const OpStream& o, int64_t k0) {
    if (!T) return o.rsrc;
    int64_t rows = o.krows - k0;
    rows = rows < 0 ? 0 : (rows > kTileK ? kTileK : rows);
    return __builtin_amdgcn_make_buffer_rsrc((void*)(o.base + k0 * o.ld_bytes), 0, (int)(rows * o.ld_bytes),
                                             0x00020000);
}

template <bool T>
__device__ __forceinline__ u32x4_t op_fetch(const OpStream& o, __amdgpu_buffer_rsrc_t r, int64_t k0, int u) {
    if (!T) return stage_fetch_b(r, o.voff, (uint32_t)(u & 7) * o.step + (uint32_t)(k0 * 2));
    return stage_fetch_b(r, o.voff, (uint32_t)(u & 7) * o.step);
}

template <bool T>
__device__ __forceinline__ void op_put(char* base, int wave, int lane, int u, const u32x4_t& v) {
    if (!T) stage_put(base, wave, lane, u, v);
    else stage_put_t(base, wave, lane, u, v);
}

struct PgCtx {
    OpStream a, b;
    int64_t KT;
    char* smem;
    int wave, lane;
};

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

// The same fragment from an MN-major tile: lane l needs mn = rb + l % 16 and
// k = 32 s + 8 (l / 16) + 0..7. ds_read_b64_tr_b16 hands lane i of each
// 16-lane group element i % 4 of the 8-byte piece addressed by lane
// 4 j + i / 4, as its element j; so lane p of the group addresses k row
// 32 s + 8 g + p / 4 at mn rb + 4 (p % 4), and a second read 4 k rows further
// (8 LDS rows on) gives k + 4..7.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
__device__ __forceinline__ bf16x8 frag16_t(const char* base, int rb, int s, int lane) {
    const int p = lane & 15;
    const int r = 32 * s + 8 * (lane >> 4) + (p >> 2);
    const char* a = base + trow(r) * kTPitch + rb * 2 + ((p & 3) << 3);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a + 8 * kTPitch));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <bool T>
__device__ __forceinline__ bf16x8 op_frag(const char* base, int rb, int s, int lane) {
    if (!T) return frag16(base, rb, s, lane);
    return frag16_t(base, rb, s, lane);
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
template <bool TA, bool TB, int P>
__device__ __forceinline__ void pg_step(const PgCtx& c, int64_t kt, AccTile& acc, bf16x8 (&fa)[8], bf16x8 (&fb)[8],
                                        u32x4_t (&s0)[16], u32x4_t (&s1)[16]) {
    u32x4_t (&sn)[16] = P ? s0 : s1;    // step kt+1, then kt+3
    const char* cur = c.smem + P * kStageBytes;
    char* nxt = c.smem + (1 - P) * kStageBytes;
    const int64_t k3 = (kt + 3 < c.KT ? kt + 3 : c.KT - 1) * kTileK;
    const __amdgpu_buffer_rsrc_t ra3 = step_rsrc<TA>(c.a, k3);
    const __amdgpu_buffer_rsrc_t rb3 = step_rsrc<TB>(c.b, k3);
    const int ar = (c.wave >> 1) * 128, br = (c.wave & 1) * 128;
    auto put_fetch = [&](int u) {
        if (u < 8) {
            op_put<TA>(nxt, c.wave, c.lane, u, sn[u]);
            sn[u] = op_fetch<TA>(c.a, ra3, k3, u);
        } else {
            op_put<TB>(nxt + kOperandBytes, c.wave, c.lane, u, sn[u]);
            sn[u] = op_fetch<TB>(c.b, rb3, k3, u);
        }
    };
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int t = 0; t < 32; ++t) {
            const int bi = t >> 2, bj = t & 3;
            mma16(acc[bi][bj], fa[bi], fb[bj]);
            if ((t & 1) && t < 8)
                fb[4 + (t >> 1)] = op_frag<TB>(cur + kOperandBytes, br + 16 * (4 + (t >> 1)), s, c.lane);
            const int pos = s * 64 + t;
#pragma unroll
            for (int u = 0; u < 16; ++u)
                if (u * 6 == pos) put_fetch(u);
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
            if ((t & 3) == 3) fa[bi] = op_frag<TA>(src, ar + 16 * bi, s2, c.lane);
            if ((t & 1) && t < 8) fb[t >> 1] = op_frag<TB>(src + kOperandBytes, br + 16 * (t >> 1), s2, c.lane);
            const int pos = s * 64 + 32 + t;
#pragma unroll
            for (int u = 0; u < 16; ++u)
                if (u * 6 == pos) put_fetch(u);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// C[m0.., n0..] = sum_k A(m, k) B(n, k) for one 256 x 256 tile; TA / TB
// select the MN-major form of an operand. K must be a multiple of 64.
template <bool TA, bool TB>
__device__ __forceinline__ void gemm_mainloop(const Operand& A, int64_t m0, const Operand& B, int64_t n0,
                                              int64_t K, char* smem, AccTile& acc) {
    const int tid = threadIdx.x;
    PgCtx c;
    c.KT = K / kTileK;
    c.smem = smem;
    c.lane = tid & 63;
    c.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    c.a = make_stream<TA>(A, m0, c.wave, c.lane);
    c.b = make_stream<TB>(B, n0, c.wave, c.lane);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.0f;
    auto kof = [&](int64_t s) { return (s < c.KT ? s : c.KT - 1) * kTileK; };
    auto fetch = [&](int64_t k0, int u) {
        return u < 8 ? op_fetch<TA>(c.a, step_rsrc<TA>(c.a, k0), k0, u)
                     : op_fetch<TB>(c.b, step_rsrc<TB>(c.b, k0), k0, u);
    };
    u32x4_t s0[16], s1[16];
    // prologue: step 0 -> set 0 -> LDS buffer 0; step 1 -> set 1 (stored during step 0); step 2 -> set 0
#pragma unroll
    for (int u = 0; u < 16; ++u) s0[u] = fetch(kof(0), u);
#pragma unroll
    for (int u = 0; u < 16; ++u) s1[u] = fetch(kof(1), u);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        if (u < 8) op_put<TA>(smem, c.wave, c.lane, u, s0[u]);
        else op_put<TB>(smem + kOperandBytes, c.wave, c.lane, u, s0[u]);
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) s0[u] = fetch(kof(2), u);
    __syncthreads();
    bf16x8 fa[8], fb[8];
    const int ar = (c.wave >> 1) * 128, br = (c.wave & 1) * 128;
#pragma unroll
    for (int i = 0; i < 8; ++i) fa[i] = op_frag<TA>(smem, ar + 16 * i, 0, c.lane);
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = op_frag<TB>(smem + kOperandBytes, br + 16 * j, 0, c.lane);
    int64_t kt = 0;
    for (; kt + 1 < c.KT; kt += 2) {
        pg_step<TA, TB, 0>(c, kt, acc, fa, fb, s0, s1);
        pg_step<TA, TB, 1>(c, kt + 1, acc, fa, fb, s0, s1);
    }
    if (kt < c.KT) pg_step<TA, TB, 0>(c, kt, acc, fa, fb, s0, s1);
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
