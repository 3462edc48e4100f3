/*
 * lmhead.h — C ABI of the deterministic chunked LM-head + loss library for
 * AMD Instinct MI355X (gfx950).
 *
 * The library projects bf16 hidden states H[n, hidden] through the bf16
 * vocabulary matrix W[vocab, hidden] without ever holding the n x vocab
 * logits: each 256-wide vocabulary tile is reduced to a per-row (max, sum of
 * exponentials) pair and the logits at the requested ids, and the pairs are
 * merged in a fixed order into logsumexp. The backward pass recomputes the
 * logits one vocabulary chunk at a time, forms dL/dz in registers and feeds
 * the two contractions dH = dZ W and dW = dZ^T H.
 *
 * Passages that define the operations (cited below by short name):
 *   [PR8059]  FlashInfer pull request #8059, "feat(cake_lm_head_det_loss):
 *             det names for the chunked LM-head + loss backend" — the PR
 *             description (deterministic forward and backward for fixed
 *             inputs, hardware, chunk plan and initial accumulation buffers;
 *             BF16 only; CE and policy losses, the log-probability entry and
 *             the support-set log-probability and KL entries) and the
 *             CodeRabbit summary (candidate-restricted log-probabilities and
 *             forward KL; valid-row controls; workspace reporting).
 *   [PR8059-review]  the same PR's CodeRabbit review comment on cache-miss
 *             bindings (FP32 dx / dw accumulators plus BF16 outputs).
 *   [PR14-op] miles-ext-kernels pull request #14, "[Cake 13/13] mok", the
 *             commit declaring the lm_head op (every negative label marks an
 *             ignored row; a label >= V must not give a plausible value; dW
 *             is BF16, the cast of an FP32 [V, H] accumulator).
 *   [PR14-tests] the same PR's commit adding tests/cake/lm_head/ (empty
 *             calls, frozen inputs, given counts, zero-gradient rows,
 *             negative labels, geometry and device errors).
 *
 * Conventions for every entry point:
 *   - Pointers named as device pointers are device memory on the current
 *     HIP device; `p` and `code`/`row` out-parameters are host memory.
 *   - The caller owns and allocates every buffer, including the workspace;
 *     the library never allocates device memory and never synchronises
 *     (except lmhead_read_device_error). All work is enqueued on `stream`
 *     (a hipStream_t; NULL = the null stream).
 *   - Host-checkable errors (NULL required pointers, bad sizes, misaligned
 *     pointers, a small workspace, a device that is not gfx950) return a
 *     status before anything is enqueued.
 *   - Data errors found on the device (a label >= vocab, a candidate id
 *     outside [0, vocab), a per-row temperature that is not positive and
 *     finite) never trap: the row's outputs become NaN (forward) or the row
 *     gets zero gradient (backward), and the workspace's error word records
 *     the lowest offending row (lmhead_read_device_error).
 *   - Results are a function of (inputs, problem incl. chunk, library build,
 *     device model): no floating-point atomics, every reduction runs in a
 *     fixed order, and the work decomposition does not depend on the number
 *     of compute units. Two calls with the same arguments give the same bits.
 *   - A workspace may not be shared by two calls in flight. Its contents are
 *     undefined between calls; the state the backward needs (lse, and lp
 *     for the support KL) is passed explicitly.
 */
#ifndef LMHEAD_H
#define LMHEAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
enum lmhead_status {
    LMHEAD_OK = 0,
    LMHEAD_ERR_ARG = 1,        /* NULL required pointer, unknown entry, nonzero flags */
    LMHEAD_ERR_SHAPE = 2,      /* sizes outside the supported ranges */
    LMHEAD_ERR_ALIGN = 3,      /* a device pointer not 16-byte aligned (workspace: 256) */
    LMHEAD_ERR_WORKSPACE = 4,  /* workspace_bytes < lmhead_workspace_size(...) */
    LMHEAD_ERR_DEVICE = 5,     /* current device is not gfx950 or no device */
    LMHEAD_ERR_HIP = 6,        /* a HIP launch or runtime call failed */
    LMHEAD_ERR_SCRATCH = 7     /* lmhead_loss_fwd_noalloc: the problem's forward workspace
                                  exceeds LMHEAD_STATIC_SCRATCH_BYTES */
};

/* Loss entries ([PR8059]: CE loss, log-probability entry, support-set entries). */
enum lmhead_entry {
    LMHEAD_ENTRY_CE_MEAN = 0,  /* mean cross-entropy over valid rows */
    LMHEAD_ENTRY_CE_SUM = 1,   /* summed cross-entropy over valid rows */
    LMHEAD_ENTRY_LOGPROB = 2,  /* per-token log-probability of the label */
    LMHEAD_ENTRY_SUPPORT = 3,  /* log-probabilities of K candidates (+ KL) */
    LMHEAD_ENTRY_SUPPORT_KL = 4 /* KL over the K candidates only (no vocabulary-wide pass) */
};

/* Problem flags. */
enum lmhead_flags {
    /* Support entries: candidate lists are padded; a negative id marks a padding
     * slot, which has lp = log p_hat = 0 and takes no part in the
     * renormalisation, the KL or the gradients. Without it a negative id is a
     * data error. */
    LMHEAD_FLAG_PADDED_IDS = 1
};

/* Device error codes recorded in the workspace's error word (bits). */
enum lmhead_device_error {
    LMHEAD_DEVERR_NONE = 0,
    LMHEAD_DEVERR_LABEL = 1,     /* a label >= vocab ([PR14-op]) */
    LMHEAD_DEVERR_CANDIDATE = 2, /* a candidate id >= vocab, or < 0 in unpadded lists */
    LMHEAD_DEVERR_TEMPERATURE = 4 /* a per-row temperature that is not positive and finite */
};

/*
 * Problem description (host memory).
 *   n          rows (tokens), 0 <= n <= 2^30. n = 0 is a valid, empty call.
 *   hidden     hidden size, a multiple of 64, 64 <= hidden <= 65536.
 *   vocab      vocabulary size, 1 <= vocab <= 2^30. Any value: the last
 *              256-wide tile is masked, so results equal the definition over
 *              exactly `vocab` columns (no padding of W).
 *   chunk      vocabulary chunk of the backward pass: a multiple of 256,
 *              >= 256. The backward materialises dL/dz for one chunk
 *              ([n x chunk] bf16) at a time, or for a few consecutive
 *              chunks when one chunk has fewer 256 x 256 tiles than the
 *              chip's 256 compute units (at most 256 tiles together; the
 *              gradients are the same either way); the forward's result
 *              does not depend on it. Every entry but the KL-only one also needs
 *              round_up(min(chunk, vocab), 256) <= 4,194,048 (2^22 - 256:
 *              dL/dz is read with that row pitch, 256 rows per buffer
 *              range of at most 2^31 - 1 bytes); vocabularies above that
 *              take a smaller chunk.
 *   num_valid  -1: count valid rows (0 <= label < vocab) on the device,
 *              with no host synchronisation; >= 0: use this value verbatim as
 *              the CE mean's denominator ("given counts", [PR14-tests]).
 *   k          candidates per row for the support entries (1..1024, and
 *              n * k <= 2^31 - 1: both support entries index their (row,
 *              candidate) entries with int32); ignored by the others.
 *   Launch sizes: one launch holds at most 2^32 - 1 work-items, so with
 *              n_pad = round_up(n, 256): 8 * n_pad <= 2^32 - 1 (n <=
 *              536,870,656), and 64 * n_pad <= 2^32 - 1 for the support
 *              entries (n <= 67,108,608); every entry but the KL-only one
 *              also needs ceil(n / 256) * max(ceil(vocab / 256),
 *              ceil(hidden / 256)) <= 16,777,215 (one 256-thread workgroup
 *              per 256 x 256 tile; at vocab = 151,936: n <= 7,230,464), and
 *              the KL-only entry 64 * round_up(vocab, 4) <= 2^32 - 1 (vocab
 *              <= 67,108,860). Larger problems are a shape error; split
 *              the rows over several calls.
 *   flags      0, or LMHEAD_FLAG_PADDED_IDS with a support entry.
 *   temperature     scalar temperature t applied to every row; 0 = off
 *                   (t = 1). Must be finite and >= 0.
 *   reserved        must be 0.
 *   row_temperature device fp32 [n] per-row temperatures r_n, or NULL.
 *              Every entry then works on the logits z / tau_n with
 *              tau_n = t * r_n (temperature routes off, scalar, per-row and
 *              1.0: [PR14-tests]); tau_n = 1 gives bit-identical results to
 *              no temperature. A tau_n that is not positive and finite is a
 *              data error (LMHEAD_DEVERR_TEMPERATURE) handled like a bad label.
 */
typedef struct lmhead_problem {
    int64_t n;
    int64_t hidden;
    int64_t vocab;
    int64_t chunk;
    int64_t num_valid;
    int32_t k;
    int32_t flags;
    float temperature;
    int32_t reserved;
    const float* row_temperature;
} lmhead_problem;

/*
 * Bytes of device workspace an entry needs ("workspace reporting",
 * [PR8059]). Pure host function: no device is touched. `with_backward`
 * != 0 sizes the workspace for lmhead_loss_bwd (which needs more: dL/dz
 * of one chunk, of four when n and hidden give at least 256 dH tiles of
 * 256 x 256, or of a few at small n, and the fp32 dH accumulator).
 * Returns 0 for an invalid problem or entry.
 */
size_t lmhead_workspace_size(const lmhead_problem* p, int entry, int with_backward);

/*
 * Memory report ("workspace reporting", "memory-budgeted backend options",
 * [PR8059]; the memory of a multi-chunk plan, [PR8059-review]). Pure host
 * function. Every figure is in bytes for the problem as given (its chunk).
 */
typedef struct lmhead_memory_figures {
    int64_t chunk;               /* vocabulary chunk of the backward */
    int64_t chunks;              /* number of chunks, ceil(vocab / chunk) */
    size_t workspace_bytes;      /* = lmhead_workspace_size(p, entry, with_backward) */
    size_t forward_bytes;        /* workspace the forward uses */
    size_t partials_bytes;       /* forward: (max, sum-exp) per 256-column tile and row */
    size_t dz_chunk_bytes;       /* backward: dL/dz of the chunks one recompute launch
                                    covers (dz_group of them), or of the four chunks
                                    that share a dH pass (at least 256 dH tiles:
                                    min(4 chunks, vocab) columns), bf16 */
    size_t dh_acc_bytes;         /* backward: fp32 running sum of dH over the chunks */
    size_t caller_output_bytes;  /* buffers the caller allocates: the entry's fp32 outputs
                                    (loss / logp / lp, kl, lse), plus bf16 dH and dW
                                    with the backward */
    size_t dh_split_bytes;       /* backward, few row tiles only (else 0): fp32 partial
                                    dH of the (chunk, K slice) units of the dH
                                    contraction, joined in order; sized by n and hidden
                                    alone (at most 16 planes of n x hidden) */
    size_t operand_copy_bytes;   /* (not the KL-only entry) H in MFMA fragment order,
                                    bf16 [n rounded up to 256, hidden]; the backward adds
                                    H^T in fragment order, [n, hidden rounded up to 256] */
    int64_t dz_group;            /* backward: chunks one recompute launch covers (1 unless
                                    a chunk has fewer than 256 tiles of 256 x 256) */
} lmhead_memory_figures;

/* Fills *out. Returns LMHEAD_ERR_ARG / LMHEAD_ERR_SHAPE for an invalid
 * problem or entry (then *out is untouched). */
int lmhead_memory_report(const lmhead_problem* p, int entry, int with_backward,
                         lmhead_memory_figures* out);

/*
 * Memory-budgeted chunk planner ([PR8059]). Pure host function; p->chunk is
 * ignored. Chooses the chunk for lmhead_loss_bwd whose workspace fits in
 * `budget_bytes` with the fewest vocabulary chunks (the fewest passes) and,
 * among those, the smallest chunk (a multiple of 256), which spreads the
 * vocabulary evenly over the passes. Writes it to *chunk. Returns
 * LMHEAD_ERR_WORKSPACE if even a 256-wide chunk does not fit. The chunk
 * returned always fits. The backward workspace never shrinks as the chunk
 * widens (the dL/dz region grows with it; the small-batch dH partials are
 * sized by n and hidden alone), so a 256-wide chunk is the floor and the
 * search over chunk widths is exact.
 */
int lmhead_plan_chunk(const lmhead_problem* p, int entry, size_t budget_bytes, int64_t* chunk);

/*
 * Cross-entropy forward ([PR8059]; ignore rule [PR14-op]).
 *   entry      LMHEAD_ENTRY_CE_MEAN or LMHEAD_ENTRY_CE_SUM.
 *   H          device, bf16 [n, hidden], row-major, 16-byte aligned.
 *   W          device, bf16 [vocab, hidden], row-major, 16-byte aligned.
 *   targets    device, int32 [n]. Every negative value marks an ignored row
 *              (loss 0, not counted); a value >= vocab is a data error.
 *   loss       device, fp32 [1]: sum over valid rows of (lse - z[t]) divided
 *              by the valid count (MEAN; 0 when the count is 0) or not (SUM).
 *   lse        device, fp32 [n] or NULL: per-row logsumexp of the logits,
 *              the state the backward needs.
 *   workspace  device, >= lmhead_workspace_size(p, entry, 0) bytes,
 *              256-byte aligned.
 */
int lmhead_loss_fwd(const lmhead_problem* p, int entry,
                    const void* H, const void* W, const int32_t* targets,
                    float* loss, float* lse,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Allocation-free variant of lmhead_loss_fwd, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. Same arguments (minus the workspace),
 * results and bits as lmhead_loss_fwd. Its workspace is a static device
 * buffer inside this library, LMHEAD_STATIC_SCRATCH_BYTES (64 MiB) per
 * device, held until the process ends; the call allocates nothing.
 *   Returns LMHEAD_ERR_SCRATCH, before anything is enqueued, when the
 *   problem's forward workspace (lmhead_workspace_size(p, entry, 0)) is
 *   larger than that buffer; host errors as lmhead_loss_fwd otherwise.
 *   Every call on one device shares that device's buffer, which keeps the
 *   last call's contents: calls that overlap on one device (two streams or
 *   two host threads without ordering between them) race, so serialise them.
 *   The device error word lives in that buffer and cannot be read with
 *   lmhead_read_device_error; a label >= vocab shows as a NaN loss.
 */
#define LMHEAD_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int lmhead_loss_fwd_noalloc(const lmhead_problem* p, int entry,
                            const void* H, const void* W, const int32_t* targets,
                            float* loss, float* lse, void* stream);

/*
 * Per-token log-probability ([PR8059] "the log-probability entry"; the RL
 * policy-loss input).
 *   logp       device, fp32 [n]: z[n, t_n] - lse[n]; 0 on ignored rows.
 *   lse        device, fp32 [n] or NULL.
 * Other arguments as lmhead_loss_fwd.
 */
int lmhead_logprob(const lmhead_problem* p,
                   const void* H, const void* W, const int32_t* targets,
                   float* logp, float* lse,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Support-set log-probabilities and KL ([PR8059] "support-set
 * log-probability and KL entries", "candidate-restricted
 * log-probabilities", "forward-KL").
 *   ids        device, int32 [n, k]: candidate vocabulary ids per row
 *              (duplicates allowed, each counts separately); an id outside
 *              [0, vocab) is a data error.
 *   ref_logq   device, fp32 [n, k] or NULL: reference log-probabilities
 *              over the k candidates. NULL: no KL.
 *   lp         device, fp32 [n, k]: full-vocabulary log-probability
 *              z[n, id] - lse[n] of each candidate.
 *   kl         device, fp32 [n] or NULL (must be NULL when ref_logq is):
 *              KL(q || p_hat) = sum_k q_k (ref_logq_k - log p_hat_k), q =
 *              exp(ref_logq), p_hat = the model's softmax renormalised over
 *              the k listed candidates; terms with q = 0 contribute 0.
 *   lse        device, fp32 [n] or NULL.
 */
int lmhead_support_logprob_kl(const lmhead_problem* p,
                              const void* H, const void* W, const int32_t* ids,
                              const float* ref_logq, float* lp, float* kl, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Support-set log-probabilities without the KL ([PR8059]: the entries
 * support_logprob and support_kl are separate): lmhead_support_logprob_kl
 * with ref_logq = kl = NULL. Backward: lmhead_loss_bwd with
 * LMHEAD_ENTRY_SUPPORT, grad_kl = NULL.
 */
int lmhead_support_logprob(const lmhead_problem* p,
                           const void* H, const void* W, const int32_t* ids,
                           float* lp, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * KL-only support entry ([PR8059] support_kl; "forward KL",
 * "candidate-restricted"): KL(q || p_hat) per row, where p_hat renormalises
 * the model over the row's k candidates. Neither the KL nor its gradient
 * depends on logits outside the candidates, so this entry computes only the
 * n * k candidate logits z = H[n] . W[id] (fp32 sums of bf16 products, in a
 * fixed order) and never makes a vocabulary-wide pass.
 *   p->k, ids, ref_logq  as for lmhead_support_logprob_kl (ref_logq required).
 *   kl         device, fp32 [n].
 *   logp_hat   device, fp32 [n, k] or NULL: log p_hat (0 at padding slots),
 *              the state lmhead_loss_bwd needs (as saved_lp).
 *   workspace  >= lmhead_workspace_size(p, LMHEAD_ENTRY_SUPPORT_KL, 0) bytes.
 * Backward: lmhead_loss_bwd / lmhead_loss_bwd_accumulate with
 * LMHEAD_ENTRY_SUPPORT_KL, saved_lp = logp_hat, grad = NULL, lse unused
 * (may be NULL), grad_kl = dL/dKL [n]; dH and dW are gathers over the
 * candidates (dW: each vocabulary row sums its (row, candidate) entries in
 * ascending order; rows no list names get 0).
 */
int lmhead_support_kl(const lmhead_problem* p,
                      const void* H, const void* W, const int32_t* ids,
                      const float* ref_logq, float* kl, float* logp_hat,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of any entry: recompute each vocabulary chunk's logits, form
 * dL/dz = a_n softmax(z)_n + sum_k c_nk onehot(id_nk) in registers, round it
 * to bf16 and contract: dH = dZ W, dW = dZ^T H ([PR8059]; FP32 accumulators
 * with BF16 outputs, [PR8059-review], [PR14-op]).
 *   entry           the forward's entry.
 *   targets_or_ids  device, int32 [n] (CE, LOGPROB) or [n, k] (SUPPORT).
 *   ref_logq        device, fp32 [n, k] (SUPPORT with a KL gradient) or NULL.
 *   lse             device, fp32 [n]: the forward's lse output.
 *   saved_lp        device, fp32 [n, k]: the forward's lp output (SUPPORT
 *                   with grad_kl only; else NULL).
 *   grad            device, fp32: CE: [1] dL/dloss; LOGPROB: [n] dL/dlogp;
 *                   SUPPORT: [n, k] dL/dlp or NULL (= 0).
 *   grad_kl         device, fp32 [n] dL/dKL (SUPPORT) or NULL (= 0).
 *   dH              device, bf16 [n, hidden] or NULL (frozen H: skipped).
 *   dW              device, bf16 [vocab, hidden] or NULL (frozen W: skipped).
 *   workspace       >= lmhead_workspace_size(p, entry, 1) bytes.
 * Ignored rows, rows with zero upstream gradient and rows with a data error
 * get exactly zero gradient. n = 0 writes zeros to dW.
 * dH sums each element in fp32 in a fixed order: a K loop over a dH pass's
 * columns in ascending order, added to the running sum pass by pass. A pass
 * is one chunk, or four consecutive chunks (0-3, 4-7, ...; the last pass may
 * hold fewer) when the chunk is narrower than vocab and n and hidden give at
 * least 256 dH tiles; at small n a chunk's columns are
 * split into K slices joined in slice order. The pass plan depends on the
 * shape alone. dW sums over all n rows in one K loop, whatever the chunk.
 */
int lmhead_loss_bwd(const lmhead_problem* p, int entry,
                    const void* H, const void* W, const int32_t* targets_or_ids,
                    const float* ref_logq, const float* lse, const float* saved_lp,
                    const float* grad, const float* grad_kl,
                    void* dH, void* dW,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward into caller-owned FP32 accumulators: the same computation as
 * lmhead_loss_bwd, but dL/dH and dL/dW (before any bf16 rounding) are added
 * to dH_acc and dW_acc, so that gradients of several calls (micro-batches,
 * or several losses of one batch) are summed in FP32 ("initial accumulation
 * buffers" are part of the determinism contract, [PR8059]; FP32 dx / dw
 * accumulators plus BF16 outputs, [PR8059-review]; dW as the BF16 cast of
 * the FP32 accumulator, [PR14-tests]). For a CE mean over several
 * micro-batches, pass the global valid-row count as p->num_valid.
 *   dH_acc   device, fp32 [n, hidden] or NULL: dH_acc += dL/dH. Within a
 *            call the chunks are added in ascending order, starting from the
 *            caller's values.
 *   dW_acc   device, fp32 [vocab, hidden] or NULL: dW_acc += dL/dW (each
 *            element gets one fp32 sum over the rows, then one addition).
 *   dH, dW   device, bf16, or NULL: the RNE bf16 cast of the updated
 *            accumulator. Each needs its accumulator (else LMHEAD_ERR_ARG).
 *   The other arguments are those of lmhead_loss_bwd. NULL accumulators
 *   (frozen H / W) skip that side; with n = 0 the accumulators are unchanged
 *   and dH / dW receive their casts. Bits depend on the accumulators'
 *   initial values as well as on the inputs. With zero-initialised
 *   accumulators, dH and dW equal lmhead_loss_bwd's outputs bit for bit.
 */
int lmhead_loss_bwd_accumulate(const lmhead_problem* p, int entry,
                               const void* H, const void* W, const int32_t* targets_or_ids,
                               const float* ref_logq, const float* lse, const float* saved_lp,
                               const float* grad, const float* grad_kl,
                               float* dH_acc, float* dW_acc, void* dH, void* dW,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Static, human-readable text for a status code. */
const char* lmhead_status_string(int status);

/*
 * Reads the device error word the last call on `workspace` left behind.
 * Synchronises `stream` (tests and debugging only). code: an
 * lmhead_device_error bit set; row: the lowest offending row, or -1.
 */
int lmhead_read_device_error(const void* workspace, void* stream, int32_t* code, int64_t* row);

#ifdef __cplusplus
}
#endif

#endif /* LMHEAD_H */
