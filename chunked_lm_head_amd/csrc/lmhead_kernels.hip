// lmhead_kernels.hip — HIP kernels of the deterministic chunked LM-head + loss
// path for gfx950.
//
// Method (FlashInfer PR #8059, "feat(cake_lm_head_det_loss): det names for the
// chunked LM-head + loss backend", PR description and CodeRabbit summary): the
// hidden states are projected through the vocabulary matrix a vocabulary block
// at a time, each row keeps what logsumexp and the requested logits need, the
// n x V logits are never stored, and the backward recomputes each chunk's
// logits to form dL/dz for the dH and dW contractions. Determinism (same PR,
// description): every output element and every partial has exactly one writer,
// merges run in a fixed order, and no floating-point atomic is used; integer
// atomics (valid-row count, lowest error row) are order-independent.
#include "lmhead_kernels.h"

#include <limits.h>

namespace lmhead {

namespace {
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }
__device__ __forceinline__ float quiet_nan() { return __builtin_nanf(""); }
}  // namespace

// ---------------------------------------------------------------- header words

__global__ void init_header_kernel(int32_t* hdr) {
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        hdr[kHdrErrCode] = 0;
        hdr[kHdrErrRow] = INT_MAX;
        hdr[kHdrCount] = 0;
    }
}

// Count valid rows (0 <= t < V) and record data errors. Labels: any negative
// value is an ignored row, t >= V is an error (miles-ext-kernels PR #14, the
// commit declaring the lm_head op). Candidate ids (support = 1) must lie in
// [0, V); in padded lists (support = 2) a negative id is a padding slot.
__global__ void scan_labels_kernel(const int32_t* ids, int64_t n, int k, int64_t vocab,
                                   int support, Temperature T, int32_t* hdr) {
    __shared__ int32_t s_count, s_row, s_code;
    if (threadIdx.x == 0) { s_count = 0; s_row = INT_MAX; s_code = 0; }
    __syncthreads();
    int32_t count = 0, row_min = INT_MAX, code = 0;
    for (int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; row < n;
         row += (int64_t)gridDim.x * blockDim.x) {
        if (T.row != nullptr && !tau_ok(row_tau(T, row))) {
            code |= kDevErrTemperature;
            row_min = row_min < row ? row_min : (int32_t)row;
        }
        if (!support) {
            const int64_t t = ids[row];
            if (t >= vocab) { code |= kDevErrLabel; row_min = row_min < row ? row_min : (int32_t)row; }
            else if (t >= 0) ++count;
        } else {
            const int32_t* r = ids + row * k;
            for (int kk = 0; kk < k; ++kk) {
                const int64_t id = r[kk];
                if (id >= vocab || (id < 0 && support != 2)) {
                    code |= kDevErrCandidate;
                    row_min = row_min < row ? row_min : (int32_t)row;
                }
            }
        }
    }
    if (count) atomicAdd(&s_count, count);
    if (code) { atomicOr(&s_code, code); atomicMin(&s_row, row_min); }
    __syncthreads();
    if (threadIdx.x == 0) {
        if (s_count) atomicAdd(hdr + kHdrCount, s_count);
        if (s_code) { atomicOr(hdr + kHdrErrCode, s_code); atomicMin(hdr + kHdrErrRow, s_row); }
    }
}

__global__ void fill_u32_kernel(uint32_t* p, int64_t count, uint32_t value) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = value;
}

// A row's label against a tile's columns [col0, col0 + ncol) (k = 1: each
// thread checks its own row's id). The difference is taken modulo 2^32: with
// 0 <= col0 < 2^30 an id lands in [0, ncol) exactly when id - col0 does over
// the integers. For k > 1 the tiles read their hits from per-tile buckets
// built before the launch (hit_count_kernel, hit_fill_kernel): a row has about
// k * 256 / V hits per tile, so scanning every id in every tile cost more
// than the hits themselves.
__device__ __forceinline__ bool id_in_tile(const int32_t* idr, uint32_t col0, int ncol, int& j) {
    const uint32_t d = (uint32_t)idr[0] - col0;
    j = (int)d;
    return d < (uint32_t)ncol;
}

// ------------------------------------------------------------- forward tiles

// One 256-row x 256-column logits tile: z = H W^T on MFMA, then per row the
// tile's max and sum of exp(z - max) over the columns below V, and the logits
// at the row's ids that fall inside the tile. Every (row, tile) partial and
// every gathered logit has exactly one writer.
__global__ __launch_bounds__(kThreads, 1) void fwd_tiles_kernel(FwdTilesArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
    int64_t tm, tn;
    map_tile(blockIdx.x, a.tiles_m, a.tiles_n, tm, tn);
    const int64_t m0 = tm * kTile, n0 = tn * kTile;

    AccTile acc;
    gemm_mainloop<false, false>(Operand{a.H, a.hidden, a.n}, m0, Operand{a.W, a.hidden, a.vocab}, n0, a.hidden,
                  smem, acc);

    float* S = reinterpret_cast<float*>(smem);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    const int64_t row = m0 + tid;
    const bool row_ok = row < a.n;
    // logits / tau_n (the scale is exactly 1 without a temperature)
    const float inv_tau = row_ok ? 1.0f / row_tau(a.T, row) : 1.0f;
    float* Sr = S + tid;
    float run_m = neg_inf(), run_s = 0.0f;
#pragma unroll 1
    for (int half = 0; half < 2; ++half) {
        if (wc == half) stage_half(S, acc, wr, lane);
        __syncthreads();
        const int64_t col0 = n0 + half * 128;
        const int64_t rem = a.vocab - col0;
        const int ncol = rem <= 0 ? 0 : (rem >= 128 ? 128 : (int)rem);
        // the row's 128 values in registers: one pass of reads, all in flight
        // (one wave per SIMD hides no LDS latency). Columns at or past ncol
        // read as -inf: they leave the max alone and add exp2(-inf) = +0 to
        // the sum (a half with ncol = 0 is never merged).
        float x[128];
#pragma unroll
        for (int c = 0; c < 128; ++c) x[c] = Sr[c * kEpiStride] * inv_tau;
        if (ncol < 128) {
#pragma unroll
            for (int c = 0; c < 128; ++c) x[c] = c < ncol ? x[c] : neg_inf();
        }
        float m = neg_inf();
#pragma unroll
        for (int c = 0; c < 128; ++c) m = fmaxf(m, x[c]);
        const float mb = m * kLog2e;
        float s = 0.0f;
#pragma unroll
        for (int c = 0; c < 128; ++c) s += exp2_fast(__builtin_fmaf(x[c], kLog2e, -mb));
        if (half == 0) {
            run_m = m;
            run_s = s;
        } else if (ncol > 0) {
            const float M = fmaxf(run_m, m);
            run_s = run_s * exp2_fast((run_m - M) * kLog2e) + s * exp2_fast((m - M) * kLog2e);
            run_m = M;
        }
        if (a.k == 1) {
            int j;
            if (row_ok && id_in_tile(a.ids + row, (uint32_t)col0, ncol, j))
                a.zg[row] = Sr[j * kEpiStride] * inv_tau;
        } else {
            // the tile's hits from its bucket, one thread per entry: every
            // (row, slot) has one entry, so each zg element has one writer
            const int64_t b = tm * a.tiles_n + tn;
            const int32_t e1 = a.hit_offsets[b + 1];
            for (int32_t i = a.hit_offsets[b] + tid; i < e1; i += kThreads) {
                const int32_t e = a.hit_list[i];
                const int c = (e >> kHitColShift) & 255;
                if ((c >> 7) != half) continue;
                const int r = e >> kHitRowShift;
                const int64_t rw = m0 + r;
                a.zg[rw * a.k + (e & 1023)] = S[(c & 127) * kEpiStride + r] * (1.0f / row_tau(a.T, rw));
            }
        }
        __syncthreads();
    }
    if (row_ok) a.part[tn * a.n + row] = make_float2(run_m, run_s);
}

// Per row: merge the tiles' (max, sum) pairs into lse = M + log(sum_t s_t
// exp(m_t - M)). Eight lanes share a row: lane `sub` takes tiles t = sub,
// sub + 8, ... in ascending order, and the eight partial results are combined
// by xor-shuffles with a fixed pairing (1, 2, 4), so the association order is
// a function of the tile count only. Lane 0 of each group then writes the
// entry's per-row outputs.
constexpr int kFinLanes = 8;

__device__ __forceinline__ float group_max8(float v) {
    v = fmaxf(v, __shfl_xor(v, 1));
    v = fmaxf(v, __shfl_xor(v, 2));
    v = fmaxf(v, __shfl_xor(v, 4));
    return v;
}
__device__ __forceinline__ float group_sum8(float v) {
    v = v + __shfl_xor(v, 1);
    v = v + __shfl_xor(v, 2);
    v = v + __shfl_xor(v, 4);
    return v;
}

__global__ void finalize_rows_kernel(FinalizeArgs a) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t row = gid / kFinLanes;
    const int sub = (int)(gid % kFinLanes);
    const bool live = row < a.n;                 // whole groups share `live`
    const float2* p = a.part + (live ? row : 0);
    // unrolled so that eight loads are in flight at once (the loop is
    // latency-bound otherwise); the per-lane order of the additions is unchanged
    float M = neg_inf();
    if (live)
#pragma unroll 8
        for (int64_t t = sub; t < a.tiles_n; t += kFinLanes) M = fmaxf(M, p[t * a.n].x);
    M = group_max8(M);
    const float Mb = M * kLog2e;
    float S = 0.0f;
    if (live)
#pragma unroll 8
        for (int64_t t = sub; t < a.tiles_n; t += kFinLanes) {
            const float2 v = p[t * a.n];
            S += v.y * exp2_fast(__builtin_fmaf(v.x, kLog2e, -Mb));
        }
    S = group_sum8(S);
    if (!live) return;
    const float lse = M + logf(S);   // every lane of the group holds the same M and S
    const bool bad_tau = a.T.row != nullptr && !tau_ok(row_tau(a.T, row));
    if (a.entry == kEntryCeMean || a.entry == kEntryCeSum || a.entry == kEntryLogprob) {
        if (sub != 0) return;
        a.lse[row] = lse;
        const int64_t t = a.ids[row];
        const bool bad = t >= a.vocab || bad_tau;
        const bool valid = t >= 0 && !bad;
        const float zt = valid ? a.zg[row] : 0.0f;
        float out;
        if (a.entry == kEntryLogprob) out = valid ? zt - lse : 0.0f;
        else out = valid ? lse - zt : 0.0f;
        a.row_out[row] = bad ? quiet_nan() : out;
        return;
    }
    // support entry; in padded lists a negative id is a padding slot (lp = 0,
    // no part in p_hat or the KL). The group's eight lanes share the row's k
    // slots (lane sub takes kk = sub, sub + 8, ... in ascending order) and
    // combine their partial max / sums with the fixed xor pairing above.
    if (sub == 0) a.lse[row] = lse;
    const int k = a.k;
    const int32_t* idr = a.ids + row * k;
    const float* zc = a.zg + row * k;
    bool bad_own = false;
    for (int kk = sub; kk < k; kk += kFinLanes) {
        const int64_t id = idr[kk];
        bad_own = bad_own || id >= a.vocab || (id < 0 && !a.padded);
    }
    const bool bad = bad_tau || group_max8(bad_own ? 1.0f : 0.0f) != 0.0f;
    float* lp = a.row_out + row * k;
    for (int kk = sub; kk < k; kk += kFinLanes)
        lp[kk] = bad ? quiet_nan() : (idr[kk] < 0 ? 0.0f : zc[kk] - lse);
    if (a.kl != nullptr) {
        if (bad) {
            if (sub == 0) a.kl[row] = quiet_nan();
            return;
        }
        // log p_hat_k = z_k - log sum_j exp z_j over the listed candidates
        float mx = neg_inf();
        for (int kk = sub; kk < k; kk += kFinLanes)
            if (idr[kk] >= 0) mx = fmaxf(mx, zc[kk]);
        mx = group_max8(mx);
        float se = 0.0f;
        for (int kk = sub; kk < k; kk += kFinLanes)
            if (idr[kk] >= 0) se += expf(zc[kk] - mx);
        se = group_sum8(se);
        const float ls = mx + logf(se);
        const float* r = a.ref_logq + row * k;
        float kl = 0.0f;
        for (int kk = sub; kk < k; kk += kFinLanes) {
            const float q = expf(r[kk]);
            if (idr[kk] >= 0 && q > 0.0f) kl += q * (r[kk] - (zc[kk] - ls));
        }
        kl = group_sum8(kl);
        if (sub == 0) a.kl[row] = kl;
    }
}

// loss = sum of the per-row losses (fixed strided order per thread, then a
// fixed LDS tree), divided by the valid count for the mean.
__global__ void ce_reduce_kernel(const float* rows, int64_t n, const int32_t* hdr,
                                 int64_t num_valid, int mean, float* loss) {
    __shared__ float red[kThreads];
    const int tid = threadIdx.x;
    float s = 0.0f;
    for (int64_t i = tid; i < n; i += kThreads) s += rows[i];
    red[tid] = s;
    __syncthreads();
    for (int w = kThreads / 2; w > 0; w >>= 1) {
        if (tid < w) red[tid] += red[tid + w];
        __syncthreads();
    }
    if (tid == 0) {
        const float total = red[0];
        if (!mean) {
            loss[0] = total;
        } else {
            const int64_t cnt = num_valid >= 0 ? num_valid : (int64_t)hdr[kHdrCount];
            loss[0] = cnt > 0 ? total / (float)cnt : (total != total ? total : 0.0f);
        }
    }
}

// --------------------------------------------------------------- backward

// Per-row coefficients of dL/dz = a_n softmax(z_n) + sum_k c_nk onehot(id_nk).
//   CE mean:  a = valid g / count,  c = -a (at the label)
//   CE sum:   a = valid g,          c = -a
//   logprob:  a = -valid gamma_n,   c = valid gamma_n
//   support:  a = -sum_k gamma_nk,  c_k = gamma_nk + beta_n (Q p_hat_k - q_k), Q = sum q
// Rows past n (tile padding) and rows with a data error get a = c = 0.
// coeffs_kernel (one thread per row) serves the single-id entries,
// coeffs_support_kernel (one wave per row) the support entries.
__global__ void coeffs_kernel(CoeffArgs a) {
    const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= a.n_pad) return;
    if (row >= a.n) {
        a.coef_a[row] = 0.0f;
        return;
    }
    const int k = a.k;
    // chain rule through z / tau_n: every coefficient carries 1 / tau_n
    const float tau = row_tau(a.T, row);
    const bool good_tau = a.T.row == nullptr || tau_ok(tau);
    const float inv_tau = good_tau ? 1.0f / tau : 0.0f;
    {
        const int64_t t = a.ids[row];
        const bool valid = t >= 0 && t < a.vocab && good_tau;
        float ca = 0.0f, cc = 0.0f;
        if (a.entry == kEntryCeMean) {
            const int64_t cnt = a.num_valid >= 0 ? a.num_valid : (int64_t)a.hdr[kHdrCount];
            ca = (valid && cnt > 0) ? a.grad[0] / (float)cnt : 0.0f;
            cc = -ca;
        } else if (a.entry == kEntryCeSum) {
            ca = valid ? a.grad[0] : 0.0f;
            cc = -ca;
        } else {
            const float g = (a.grad != nullptr && valid) ? a.grad[row] : 0.0f;
            ca = -g;
            cc = g;
        }
        a.coef_a[row] = ca * inv_tau;
        a.coef_c[row] = cc * inv_tau;
    }
}

// Support entries, one wave per row: lane l takes the slots l, l + 64, ...
// in ascending order, and each row sum (of gamma, of exp(lp - max), of q) is
// the lanes' partial sums combined by a fixed xor butterfly, so the
// association order depends on k only. A row with a bad id (or a bad
// per-row temperature) gets a = c = 0, like a row past n.
__device__ __forceinline__ float wave_sum64(float v) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ __forceinline__ float wave_max64(float v) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__global__ __launch_bounds__(256) void coeffs_support_kernel(CoeffArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
    if (row >= a.n_pad) return;
    if (row >= a.n) {
        if (lane == 0) a.coef_a[row] = 0.0f;
        return;
    }
    const int k = a.k;
    const float tau = row_tau(a.T, row);
    const bool good_tau = a.T.row == nullptr || tau_ok(tau);
    const float inv_tau = good_tau ? 1.0f / tau : 0.0f;
    const int32_t* idr = a.ids + row * k;
    float* c = a.coef_c + row * k;
    bool bad_l = false;
    for (int kk = lane; kk < k; kk += 64) {
        const int32_t id = idr[kk];
        bad_l = bad_l || id >= a.vocab || (id < 0 && !a.padded);
    }
    if (!good_tau || __any(bad_l)) {
        for (int kk = lane; kk < k; kk += 64) c[kk] = 0.0f;
        if (lane == 0) a.coef_a[row] = 0.0f;
        return;
    }
    const float* g = a.grad != nullptr ? a.grad + row * k : nullptr;
    float gs = 0.0f;
    for (int kk = lane; kk < k; kk += 64) {
        const float gk = (g != nullptr && idr[kk] >= 0) ? g[kk] : 0.0f;
        gs += gk;
        c[kk] = gk;
    }
    const float gsum = wave_sum64(gs);
    if (lane == 0) a.coef_a[row] = -gsum * inv_tau;
    if (a.grad_kl != nullptr) {
        const float beta = a.grad_kl[row];
        const float* lp = a.saved_lp + row * k;
        const float* r = a.ref_logq + row * k;
        float mx = neg_inf();
        for (int kk = lane; kk < k; kk += 64)
            if (idr[kk] >= 0) mx = fmaxf(mx, lp[kk]);
        mx = wave_max64(mx);
        float se = 0.0f, Q = 0.0f;
        for (int kk = lane; kk < k; kk += 64) {
            if (idr[kk] < 0) continue;
            se += expf(lp[kk] - mx);
            Q += expf(r[kk]);
        }
        se = wave_sum64(se);
        Q = wave_sum64(Q);
        const float inv = 1.0f / se;
        for (int kk = lane; kk < k; kk += 64) {
            if (idr[kk] < 0) continue;
            const float phat = expf(lp[kk] - mx) * inv;
            c[kk] += beta * (Q * phat - expf(r[kk]));
        }
    }
    for (int kk = lane; kk < k; kk += 64) c[kk] *= inv_tau;
}

// Recompute one chunk's logits tile and write dL/dz in bf16: G[n, j] = a_n
// exp(z - lse_n) for chunk columns j < width, plus c_nk where v0 + j = id_nk;
// zero elsewhere. G is written row-major [n_pad, w_pad]; it is the K-major
// operand of dH and the MN-major operand of dW.
__global__ __launch_bounds__(kThreads, 1) void bwd_logit_grad_kernel(LogitGradArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
    int64_t tm, tn;
    map_tile(blockIdx.x, a.tiles_m, a.tiles_n, tm, tn);
    const int64_t m0 = tm * kTile, n0 = tn * kTile;

    AccTile acc;
    gemm_mainloop<false, false>(Operand{a.H, a.hidden, a.n}, m0, Operand{a.Wc, a.hidden, a.width}, n0, a.hidden,
                  smem, acc);

    float* S = reinterpret_cast<float*>(smem);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    const int64_t row = m0 + tid;   // < n_pad
    const bool row_ok = row < a.n;
    const float ca = row_ok ? a.coef_a[row] : 0.0f;
    const float lb = row_ok ? a.lse[row] * kLog2e : 0.0f;
    const float xs = row_ok ? kLog2e / row_tau(a.T, row) : kLog2e;   // log2(e) / tau_n
    // a_n exp(z - lse_n) in the accumulators, by all four waves at once: each
    // lane holds 32 rows (4 per block row), whose constants thread t, row t,
    // shares through the LDS past the staging area (the K loop is done with it)
    static_assert(kEpiLdsBytes + 3 * kTile * 4 <= kLdsBytes, "row constants must fit past the staging area");
    {
        float* K3 = S + 128 * kEpiStride;
        K3[tid] = ca;
        K3[kTile + tid] = lb;
        K3[2 * kTile + tid] = xs;
        __syncthreads();
        const int64_t cb = n0 + wc * 128 + (lane & 15);   // chunk-local column of block 0
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r0 = wr * 128 + i * 16 + 4 * (lane >> 4);
            const floatx4 ca4 = *reinterpret_cast<const floatx4*>(K3 + r0);
            const floatx4 lb4 = *reinterpret_cast<const floatx4*>(K3 + kTile + r0);
            const floatx4 xs4 = *reinterpret_cast<const floatx4*>(K3 + 2 * kTile + r0);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const bool col_ok = cb + 16 * j < a.width;
                floatx4 v = acc[i][j];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float g = ca4[e] * exp2_fast(__builtin_fmaf(v[e], xs4[e], -lb4[e]));
                    v[e] = (ca4[e] != 0.0f && col_ok) ? g : 0.0f;
                }
                acc[i][j] = v;
            }
        }
    }
    float* Sr = S + tid;
#pragma unroll 1
    for (int half = 0; half < 2; ++half) {
        if (wc == half) stage_half(S, acc, wr, lane);
        __syncthreads();
        const int64_t col0 = n0 + half * 128;   // chunk-local column
        const int64_t rem = a.width - col0;
        const int ncol = rem <= 0 ? 0 : (rem >= 128 ? 128 : (int)rem);
        // c_nk at the row's ids in the tile, in ascending k
        if (a.k == 1) {
            int j;
            if (row_ok && id_in_tile(a.ids + row, (uint32_t)(a.v0 + col0), ncol, j))
                Sr[j * kEpiStride] += a.coef_c[row];
        } else {
            // the tile's bucket lists its hits by row, column, slot: the first
            // entry of each (row, column) run adds the run's c_nk in ascending
            // slot order, so every element has one writer and a fixed order
            const int64_t b = tm * a.tiles_v + (a.v0 >> 8) + tn;
            const int32_t e0 = a.hit_offsets[b], e1 = a.hit_offsets[b + 1];
            for (int32_t i = e0 + tid; i < e1; i += kThreads) {
                const int32_t key = a.hit_list[i] >> kHitColShift;   // row << 8 | column
                if (i > e0 && (a.hit_list[i - 1] >> kHitColShift) == key) continue;
                const int c = key & 255;
                if ((c >> 7) != half) continue;
                const int r = key >> 8;
                float* dst = S + (c & 127) * kEpiStride + r;
                float v = *dst;
                for (int32_t i2 = i; i2 < e1; ++i2) {
                    const int32_t e = a.hit_list[i2];
                    if ((e >> kHitColShift) != key) break;
                    v += a.coef_c[(m0 + r) * a.k + (e & 1023)];
                }
                *dst = v;
            }
        }
        __syncthreads();
        if (a.G != nullptr) {
            // row-major copy, 64 columns at a time: each thread packs its row's
            // values to bf16 in registers, the rows go back to LDS as [row][64]
            // (16-byte chunk q of row r at q ^ ((r >> 1) & 7), over columns
            // 0..31 of S, which are consumed), and 8 lanes then store one row's
            // 128 contiguous bytes
            uint16_t* Gl = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                uint32_t w[32];
#pragma unroll
                for (int i = 0; i < 32; ++i)
                    w[i] = pack_bf16x2(Sr[(q * 64 + 2 * i) * kEpiStride], Sr[(q * 64 + 2 * i + 1) * kEpiStride]);
                __syncthreads();
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    *reinterpret_cast<uint4*>(Gl + tid * 64 + ((j ^ swizzle(tid)) << 3)) =
                        make_uint4(w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]);
                __syncthreads();
                for (int it = 0; it < 8; ++it) {
                    const int r = wave * 64 + it * 8 + (lane >> 3);
                    const int ch = lane & 7;
                    const uint4 v = *reinterpret_cast<const uint4*>(Gl + r * 64 + ((ch ^ swizzle(r)) << 3));
                    *reinterpret_cast<uint4*>(a.G + (m0 + r) * a.w_pad + col0 + q * 64 + ch * 8) = v;
                }
            }
        }
        __syncthreads();
    }
}

// dW rows of one chunk: dW[v0 + i, h] = sum_n G[n, i] H[n, h], a single
// K-loop over every row n in ascending order; bf16 store of the fp32 sum.
// With a caller accumulator the fp32 sum is first added to it (dw_acc +=),
// and the bf16 output, if any, is the cast of the updated accumulator.
__device__ __forceinline__ void dw_tile(const DwArgs& a, int64_t bid, char* smem) {
    int64_t tm, tn;
    map_tile(bid, a.tiles_m, a.tiles_n, tm, tn);
    const int64_t m0 = tm * kTile, n0 = tn * kTile;
    AccTile acc;
    // both operands MN-major: G [n_pad, w_pad] and H [n, hidden], k = n
    gemm_mainloop<true, true>(Operand{a.G, a.w_pad, a.n_pad}, m0, Operand{a.H, a.hidden, a.n}, n0, a.n_pad,
                              smem, acc);
    float* S = reinterpret_cast<float*>(smem);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    // 32 lanes per dW row (4 columns each), two rows per wave and step: coalesced
#pragma unroll 1
    for (int half = 0; half < 2; ++half) {
        if (wc == half) stage_half_rows(S, acc, wr, lane);
        __syncthreads();
        const int c = 4 * (lane & 31);
        const int64_t h = n0 + half * 128 + c;
        const bool hok = h < a.hidden;
        // 16 rows at a time; with a caller accumulator all 16 of its values
        // are loaded (unconditionally, from in-bounds places for masked
        // elements) before the first is used
        const int64_t hc = hok ? h : 0;
#pragma unroll 1
        for (int i0 = 0; i0 < 32; i0 += 16) {
            float4 p[16];
            if (a.dw_acc != nullptr) {
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const int64_t v = m0 + wave * 64 + (i0 + u) * 2 + (lane >> 5);
                    const int64_t vc = v < a.width ? v : a.width - 1;
                    p[u] = *reinterpret_cast<const float4*>(a.dw_acc + (a.v0 + vc) * a.hidden + hc);
                }
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int r = wave * 64 + (i0 + u) * 2 + (lane >> 5);
                const int64_t v = m0 + r;   // chunk-local vocabulary row
                if (v >= a.width || !hok) continue;
                const float4 x = *reinterpret_cast<const float4*>(S + r * kRowStride + c);
                const int64_t o = (a.v0 + v) * a.hidden + h;
                if (a.dw_acc == nullptr) {
                    *reinterpret_cast<uint2*>(a.dW + o) = make_uint2(pack_bf16x2(x.x, x.y), pack_bf16x2(x.z, x.w));
                } else {
                    float4 y;
                    y.x = p[u].x + x.x;
                    y.y = p[u].y + x.y;
                    y.z = p[u].z + x.z;
                    y.w = p[u].w + x.w;
                    *reinterpret_cast<float4*>(a.dw_acc + o) = y;
                    if (a.dW != nullptr)
                        *reinterpret_cast<uint2*>(a.dW + o) = make_uint2(pack_bf16x2(y.x, y.y), pack_bf16x2(y.z, y.w));
                }
            }
        }
        __syncthreads();
    }
}

// dH contribution of one chunk: acc = sum_j G[n, j] W[v0 + j, h] over the
// chunk's columns; the fp32 running sum over chunks (chunk order) lives in
// dh_acc and the last chunk writes the bf16 result. A caller accumulator is
// dh_acc itself: read from chunk 0 on and stored after the last chunk too.
__device__ __forceinline__ void dh_tile(const DhArgs& a, int64_t bid, char* smem) {
    int64_t tm, tn;
    map_tile(bid, a.tiles_m, a.tiles_n, tm, tn);
    const int64_t m0 = tm * kTile, n0 = tn * kTile;
    AccTile acc;
    // B = the chunk of W, MN-major [width, hidden], k = chunk column
    gemm_mainloop<false, true>(Operand{a.G, a.w_pad, a.n_pad}, m0, Operand{a.Wc, a.hidden, a.width}, n0, a.w_pad,
                               smem, acc);
    float* S = reinterpret_cast<float*>(smem);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    // 32 lanes per row (4 columns each), two rows per wave and step: the fp32
    // read-modify-write of dh_acc is coalesced
#pragma unroll 1
    for (int half = 0; half < 2; ++half) {
        if (wc == half) stage_half_rows(S, acc, wr, lane);
        __syncthreads();
        const int c = 4 * (lane & 31);
        const int64_t h = n0 + half * 128 + c;
        const bool hok = h < a.hidden;
        // 16 rows at a time: the running sums of all 16 are loaded before the
        // first is used (one wave per SIMD hides no memory latency). The loads
        // are unconditional, from an in-bounds row and column for lanes whose
        // element is masked, so the compiler can count them and wait for each
        // one alone rather than for every earlier load and store.
        const int64_t hc = hok ? h : 0;
#pragma unroll 1
        for (int i0 = 0; i0 < 32; i0 += 16) {
            float4 p[16];
            if (!a.first) {
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const int64_t row = m0 + wave * 64 + (i0 + u) * 2 + (lane >> 5);
                    const int64_t rc = row < a.n ? row : a.n - 1;
                    p[u] = *reinterpret_cast<const float4*>(a.dh_acc + rc * a.hidden + hc);
                }
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int r = wave * 64 + (i0 + u) * 2 + (lane >> 5);
                const int64_t row = m0 + r;
                if (row >= a.n || !hok) continue;
                float4 v = *reinterpret_cast<const float4*>(S + r * kRowStride + c);
                const int64_t o = row * a.hidden + h;
                if (!a.first) {
                    v.x = p[u].x + v.x;
                    v.y = p[u].y + v.y;
                    v.z = p[u].z + v.z;
                    v.w = p[u].w + v.w;
                }
                if (a.last && a.dH != nullptr)
                    *reinterpret_cast<uint2*>(a.dH + o) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
                if (!a.last || a.keep_acc) *reinterpret_cast<float4*>(a.dh_acc + o) = v;
            }
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(kThreads, 1) void bwd_dw_kernel(DwArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
    dw_tile(a, blockIdx.x, smem);
}

__global__ __launch_bounds__(kThreads, 1) void bwd_dh_kernel(DhArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
    dh_tile(a, blockIdx.x, smem);
}

// The dW and dH tiles of one chunk in one launch: the first `first_count`
// workgroups take the kind named by dh_first, the rest the other kind. Each
// tile is computed exactly as in its own kernel (same code, same K order), so
// the results do not depend on which launch runs it; the host picks this form
// when one launch leaves compute units idle that the other kind can fill.
__global__ __launch_bounds__(kThreads, 1) void bwd_dwdh_kernel(DwArgs dw, DhArgs dh, int dh_first) {
    __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
    const int64_t bid = blockIdx.x;
    const int64_t n_first = dh_first ? dh.tiles_m * dh.tiles_n : dw.tiles_m * dw.tiles_n;
    const bool take_dh = dh_first ? bid < n_first : bid >= n_first;
    const int64_t local = bid < n_first ? bid : bid - n_first;
    if (take_dh) dh_tile(dh, local, smem);
    else dw_tile(dw, local, smem);
}

// Few row tiles (small batches): a chunk's dH tiles are split along the
// chunk's columns into `slices` equal K ranges (multiples of 64), one
// workgroup per (slice, tile), each writing its fp32 partial tile to
// partial[slice, n, hidden]; dh_join_kernel then adds the partials in slice
// order to the running sum. The split depends only on the problem's shape.
__global__ __launch_bounds__(kThreads, 1) void bwd_dh_split_kernel(DhArgs a, int slices, float* partial) {
    __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
    const int64_t tiles = a.tiles_m * a.tiles_n;
    const int64_t sl = blockIdx.x / tiles;
    int64_t tm, tn;
    map_tile(blockIdx.x - sl * tiles, a.tiles_m, a.tiles_n, tm, tn);
    const int64_t m0 = tm * kTile, n0 = tn * kTile;
    const int64_t ks = a.w_pad / slices, k0 = sl * ks;
    const int64_t krows = a.width - k0;   // rows of W_c from k0 on (<= 0: the slice is all padding)
    AccTile acc;
    gemm_mainloop<false, true>(Operand{a.G + k0, a.w_pad, a.n_pad}, m0,
                               Operand{a.Wc + (krows > 0 ? k0 : 0) * a.hidden, a.hidden, krows > 0 ? krows : 0},
                               n0, ks, smem, acc);
    float* S = reinterpret_cast<float*>(smem);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    float* out = partial + sl * a.n * a.hidden;
#pragma unroll 1
    for (int half = 0; half < 2; ++half) {
        if (wc == half) stage_half_rows(S, acc, wr, lane);
        __syncthreads();
        const int c = 4 * (lane & 31);
        const int64_t h = n0 + half * 128 + c;
        if (h < a.hidden) {
#pragma unroll 4
            for (int u = 0; u < 32; ++u) {
                const int r = wave * 64 + u * 2 + (lane >> 5);
                const int64_t row = m0 + r;
                if (row < a.n)
                    *reinterpret_cast<float4*>(out + row * a.hidden + h) =
                        *reinterpret_cast<const float4*>(S + r * kRowStride + c);
            }
        }
        __syncthreads();
    }
}

// dh_acc (+)= partial[0] + partial[1] + ... in slice order, four elements per
// thread; the last chunk writes the bf16 dH and, for a caller accumulator,
// the fp32 sum, exactly as bwd_dh_kernel's epilogue does.
__global__ void dh_join_kernel(DhArgs a, int slices, const float* partial) {
    const int64_t count = a.n * a.hidden / 4;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < count;
         q += (int64_t)gridDim.x * blockDim.x) {
        const int64_t o = q * 4;
        float4 p = *reinterpret_cast<const float4*>(partial + o);
        for (int sl = 1; sl < slices; ++sl) {
            const float4 x = *reinterpret_cast<const float4*>(partial + sl * a.n * a.hidden + o);
            p.x += x.x;
            p.y += x.y;
            p.z += x.z;
            p.w += x.w;
        }
        float4 v = p;
        if (!a.first) {
            const float4 d = *reinterpret_cast<const float4*>(a.dh_acc + o);
            v.x = d.x + p.x;
            v.y = d.y + p.y;
            v.z = d.z + p.z;
            v.w = d.w + p.w;
        }
        if (a.last && a.dH != nullptr)
            *reinterpret_cast<uint2*>(a.dH + o) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
        if (!a.last || a.keep_acc) *reinterpret_cast<float4*>(a.dh_acc + o) = v;
    }
}

// out[i] = bf16 (round to nearest even) of in[i]; count is a multiple of 2.
__global__ void f32_to_bf16_kernel(const float* in, int64_t count, bf16_bits* out) {
    for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 2; i < count;
         i += (int64_t)gridDim.x * blockDim.x * 2) {
        const float2 v = *reinterpret_cast<const float2*>(in + i);
        *reinterpret_cast<uint32_t*>(out + i) = pack_bf16x2(v.x, v.y);
    }
}

}  // namespace lmhead
