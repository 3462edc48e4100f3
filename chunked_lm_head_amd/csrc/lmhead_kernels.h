// lmhead_kernels.h — kernel argument blocks and launch declarations shared by
// the kernels and the host-side plan (lmhead_api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_core.h"

namespace lmhead {

// entry kinds (same values as enum lmhead_entry)
constexpr int kEntryCeMean = 0;
constexpr int kEntryCeSum = 1;
constexpr int kEntryLogprob = 2;
constexpr int kEntrySupport = 3;
constexpr int kEntrySupportKl = 4;

constexpr int kMaxCandidates = 1024;   // candidates per row, support entries

// int32 words at the start of every workspace
constexpr int kHdrErrCode = 0;
constexpr int kHdrErrRow = 1;
constexpr int kHdrCount = 2;
constexpr int kDevErrLabel = 1;
constexpr int kDevErrCandidate = 2;
constexpr int kDevErrTemperature = 4;

// Temperature: tau_n = t * r_n (r_n = 1 without a per-row array). Kernels use
// 1 / tau_n; tau_n = 1 gives exactly 1, so that route is bit-identical to no
// temperature.
struct Temperature {
    float t;            // scalar, already resolved (1 when off)
    const float* row;   // [n] or null
};

__device__ __forceinline__ float row_tau(const Temperature& T, int64_t row) {
    return T.row != nullptr ? T.t * T.row[row] : T.t;
}
__device__ __forceinline__ bool tau_ok(float tau) { return tau > 0.0f && tau <= 3.402823466e38f; }

struct FwdTilesArgs {
    const bf16_bits* Hf;   // H in MFMA fragment order (frag_pack_kernel), n_pad rows
    const bf16_bits* W;
    int64_t n, hidden, vocab;
    int64_t tiles_m, tiles_n;
    const int32_t* ids;   // labels [n] (k = 1) or candidate ids [n, k]
    int k;
    float2* part;         // [tiles_n, n] (max, sum) per (tile, row)
    float* zg;            // [n, k] logits at the ids
    Temperature T;
    // k > 1: the candidate ids bucketed by (row tile, vocabulary tile), see
    // hit_count_kernel; bucket b's entries are hit_list[hit_offsets[b] ..
    // hit_offsets[b + 1])
    const int32_t* hit_offsets;
    const int32_t* hit_list;
};

struct FinalizeArgs {
    const float2* part;
    int64_t n, tiles_n, vocab;
    const int32_t* ids;
    int k;
    int entry;
    const float* zg;
    const float* ref_logq;  // support KL only
    float* lse;             // [n]
    float* row_out;         // CE: loss rows; logprob: logp [n]; support: lp [n, k]
    float* kl;              // support: [n] or null
    int padded;             // support: a negative id is a padding slot
    Temperature T;
};

struct CoeffArgs {
    int entry;
    int64_t n, n_pad, vocab;
    int k;
    const int32_t* ids;
    const float* ref_logq;
    const float* saved_lp;
    const float* grad;
    const float* grad_kl;
    const int32_t* hdr;
    int64_t num_valid;
    float* coef_a;   // [n_pad]
    float* coef_c;   // [n, k]
    int padded;      // support: a negative id is a padding slot
    Temperature T;
};

// One launch recomputes dL/dz for `group` consecutive chunks (several when a
// chunk has fewer 256 x 256 tiles than the chip has compute units): chunk g
// of the group starts at column v0 + g * chunk, spans min(chunk, vocab -
// its first column) columns and writes its own slot G + g * g_stride.
struct LogitGradArgs {
    const bf16_bits* Hf;   // H in MFMA fragment order (frag_pack_kernel), n_pad rows
    const bf16_bits* W;    // [vocab, hidden]
    int64_t n, n_pad, hidden, vocab;
    int64_t v0, chunk, group;   // first column of the group, columns per chunk, chunks
    int64_t tiles_m, tiles_n;   // row tiles, column tiles of a full chunk
    const float* coef_a;
    const float* coef_c;
    const int32_t* ids;
    int k;
    const float* lse;
    bf16_bits* G;          // slot g: chunk g's dL/dz, fragment order [n_pad / 16][w_pad / 32]
    int64_t g_stride;      // elements between slots (n_pad x a full chunk's w_pad)
    int64_t g_pitch;       // columns per block row of the dL/dz region (0: the chunk's own w_pad)
    Temperature T;
    int64_t tiles_v;       // vocabulary tiles of the whole vocabulary (bucket index)
    const int32_t* hit_offsets;   // k > 1: as in FwdTilesArgs
    const int32_t* hit_list;
};

// dW of `group` consecutive chunks in one launch (one, unless the dL/dz of
// several was recomputed together): chunk g starts at column v0 + g * chunk,
// is min(chunk, vocab - its first column) wide and reads slot G + g * g_stride.
struct DwArgs {
    const bf16_bits* G;    // slot 0: dL/dz in fragment order [n_pad / 16][w_pad / 32] (pslot lanes)
    const bf16_bits* HTf;  // H^T in fragment order [n_pad / 32][hid_pad / 16] (ht_pack_kernel)
    int64_t n, n_pad, hidden, hid_pad, vocab;
    int64_t v0, chunk, group, g_stride;
    int64_t g_pitch;            // as in LogitGradArgs
    int64_t tiles_m, tiles_n;   // hidden tiles x column tiles of the first chunk
    bf16_bits* dW;         // [vocab, hidden] or null
    float* dw_acc;         // caller's fp32 [vocab, hidden] (+=) or null
};

struct DhArgs {
    const bf16_bits* G;    // dL/dz of the chunk in fragment order [n_pad / 16][w_pad / 32] (pslot lanes)
    const bf16_bits* Wc;   // first row of the chunk: [width, hidden]
    int64_t n, n_pad, hidden, width, w_pad;   // a pair of chunks: both chunks' columns, W rows contiguous
    int64_t g_pitch;       // as in LogitGradArgs
    int64_t tiles_m, tiles_n;
    int first;             // chunk 0 of a fresh sum: dh_acc is written, not read
    int last;              // last chunk: the bf16 dH is written (if dH is set)
    int keep_acc;          // the last chunk also stores the fp32 sum (caller's accumulator)
    float* dh_acc;         // [n, hidden]
    bf16_bits* dH;         // [n, hidden] or null
};

// The K-split dH of `chunks` consecutive chunks (DhArgs::G is the first
// one's dL/dz slot, DhArgs::first / last refer to the first / last of them):
// each chunk's columns are cut into `slices` ranges of ks columns (the last
// ones of a narrower chunk shorter or empty), one fp32 partial per (chunk,
// slice), which dh_join_kernel adds to the running sum chunk by chunk.
struct DhSplit {
    const bf16_bits* W;    // [vocab, hidden]
    int64_t v0, chunk, vocab;   // first column of the first chunk, columns per chunk
    int64_t chunks, slices, ks; // ks: a multiple of 64
    int64_t g_stride;      // elements between dL/dz slots
};

// KL-only support entry (candidate gathers, lmhead_candidates.hip)
struct CandFwdArgs {
    const bf16_bits* H;
    const bf16_bits* W;
    int64_t n, hidden, vocab;
    int k;
    int padded;              // a negative id is a padding slot
    const int32_t* ids;      // [n, k]
    const float* ref_logq;   // [n, k]
    float* kl;               // [n]
    float* logp_hat;         // [n, k] or null
    Temperature T;
};

struct CandBwdArgs {
    const bf16_bits* H;
    const bf16_bits* W;
    int64_t n, hidden, vocab;
    int k;
    const int32_t* ids;      // [n, k]
    const float* coef_c;     // [n, k]: dL/dz at the candidates (0 for padding and bad rows)
    bf16_bits* dH;           // [n, hidden] or null
    float* dH_acc;           // caller's fp32 [n, hidden] (+=) or null
    bf16_bits* dW;           // [vocab, hidden] or null
    float* dW_acc;           // caller's fp32 [vocab, hidden] (+=) or null
    const int32_t* offsets;  // [vocab + 1]: bucket v is list[offsets[v] .. offsets[v + 1])
    const int32_t* list;     // entries i = row * k + candidate, ascending in each bucket
};

__global__ void init_header_kernel(int32_t* hdr);
__global__ void scan_labels_kernel(const int32_t* ids, int64_t n, int k, int64_t vocab, int support,
                                   Temperature T, int32_t* hdr);
__global__ void fill_u32_kernel(uint32_t* p, int64_t count, uint32_t value);
__global__ void frag_pack_kernel(const bf16_bits* H, int64_t n, int64_t hidden, int64_t n_pad, bf16_bits* Hf);
__global__ void ht_pack_kernel(const bf16_bits* H, int64_t n, int64_t hidden, int64_t hid_pad, bf16_bits* HTf);
__global__ void fwd_tiles_kernel(FwdTilesArgs a);
__global__ void finalize_rows_kernel(FinalizeArgs a);
__global__ void ce_reduce_kernel(const float* rows, int64_t n, const int32_t* hdr, int64_t num_valid,
                                 int mean, float* loss);
__global__ void coeffs_kernel(CoeffArgs a);
__global__ void coeffs_support_kernel(CoeffArgs a);
__global__ void bwd_logit_grad_kernel(LogitGradArgs a);
__global__ void bwd_dw_kernel(DwArgs a);
__global__ void bwd_dh_kernel(DhArgs a);
__global__ void bwd_dwdh_kernel(DwArgs dw, DhArgs dh, int dh_first);
__global__ void bwd_dh_split_kernel(DhArgs a, DhSplit q, float* partial);
__global__ void dh_join_kernel(DhArgs a, DhSplit q, const float* partial);
__global__ void cand_kl_fwd_kernel(CandFwdArgs a);
__global__ void cand_dh_kernel(CandBwdArgs a);
__global__ void cand_count_kernel(const int32_t* ids, int64_t nk, int64_t vocab, int32_t* counts);
__global__ void exclusive_scan_kernel(const int32_t* counts, int64_t vocab, int32_t* offsets);
constexpr int kScanTile = 1024;   // counts per workgroup of the multi-block scan
__global__ void tile_sums_kernel(const int32_t* counts, int64_t vocab, int32_t* sums);
__global__ void scan_tiles_kernel(const int32_t* counts, int64_t vocab, const int32_t* prefix, int64_t tiles,
                                  int32_t* offsets);
__global__ void cand_fill_kernel(const int32_t* ids, int64_t nk, int64_t vocab, const int32_t* offsets,
                                 int32_t* cursor, int32_t* list);
__global__ void bucket_sort_kernel(const int32_t* offsets, int64_t buckets, int32_t* list, int32_t* large,
                                   int32_t* n_large);
__global__ void bucket_sort_wave_kernel(const int32_t* offsets, int64_t buckets, int32_t* list, int32_t* large,
                                        int32_t* n_large);
__global__ void bucket_sort_block_kernel(const int32_t* offsets, int32_t* list, int32_t* tmp, const int32_t* large,
                                         const int32_t* n_large);
__global__ void cand_dw_mid_kernel(CandBwdArgs a, const int32_t* large, const int32_t* n_large);
__global__ void cand_split_counts_kernel(const int32_t* offsets, const int32_t* large, const int32_t* n_large,
                                         int64_t cap, int32_t* pieces);
__global__ void cand_dw_split_kernel(CandBwdArgs a, const int32_t* large, const int32_t* n_large,
                                     const int32_t* piece_off, float* partial);
__global__ void cand_dw_join_kernel(CandBwdArgs a, const int32_t* large, const int32_t* n_large,
                                    const int32_t* piece_off, const float* partial);
constexpr int kDwSplitEntries = 256;   // bucket entries per split piece (must match the kernels)

// Per-tile hit lists of the support entries. Entry (n, kk) with a valid id
// goes to bucket (n / 256) * tiles_v + id / 256 as the packed value
// (n % 256) << 18 | (id % 256) << 10 | kk, so a bucket sorted ascending lists
// its hits by row, then column, then slot.
constexpr int kHitRowShift = 18;
constexpr int kHitColShift = 10;
__global__ void hit_count_kernel(const int32_t* ids, int64_t n, int k, int64_t vocab, int64_t tiles_v,
                                 int32_t* counts);
__global__ void hit_fill_kernel(const int32_t* ids, int64_t n, int k, int64_t vocab, int64_t tiles_v,
                                const int32_t* offsets, int32_t* cursor, int32_t* list);
__global__ void cand_dw_kernel(CandBwdArgs a);
__global__ void f32_to_bf16_kernel(const float* in, int64_t count, bf16_bits* out);

}  // namespace lmhead
