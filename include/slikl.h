/*
 * slikl.h -- C ABI of the sparse lightning-indexer KL-loss backward for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is the one defined on the operator page
 * "aclnnSparseLightningIndexerKLLossGrad" (CANN API reference,
 * ops-transformer), 计算公式 / formula section: for every query token t and
 * key head g, gather the top-k key rows named by sparseIndices, form
 * S = q_t K_topk^T per indexer head, I = sum_h w_h ReLU(S_h), write
 * y = Softmax(I) to softmaxOut, form dI = y - p (p = attnSoftmaxL1Norm),
 * dW = dI ReLU(S)^T, dS = w (x) dI masked by S > 0, dq = dS K_topk and
 * scatter-add dK_topk = dS^T q into the key rows; -1 slots take no part.
 * The page's two-phase call (workspace query, then execute) and its
 * constraints section (dtypes, BSND/TND layouts, cuSeqLens for TND, -1
 * padding, batch-relative indices) fix the interface below.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers, contiguous, non-aliasing, owned
 *    by the caller.  The library never allocates, frees or synchronises.
 *    q, k, dq and dk must be 16-byte aligned and the workspace 256-byte
 *    aligned (PARAM_INVALID / WORKSPACE otherwise); every tensor must hold
 *    fewer than 2^31 elements (PARAM_INVALID otherwise).
 *  - Work is only enqueued on `stream` (a hipStream_t passed as void*, NULL =
 *    the default stream); the caller keeps buffers alive until it completes.
 *  - A non-OK status is returned from host-side validation only, and then
 *    nothing has been enqueued.  Device-side contract violations (an index
 *    outside [0, key length of its batch) other than -1, cuSeqLens that do not
 *    start at 0, decrease or miss the total) are not reported through the
 *    status: such slots are treated as -1 and the metadata error word is set.
 *  - The library is stateless and thread-safe.
 *
 * Tensor shapes (BSND | TND):
 *    q            [B,S1,N1,D] | [T1,N1,D]      fp16 or bf16
 *    k            [B,S2,N2,D] | [T2,N2,D]      same dtype as q
 *    w            [B,S1,N1]   | [T1,N1]        fp32
 *    sparse_indices, attn_softmax_l1norm, softmax_out
 *                 [B,S1,N2,topk] | [T1,N2,topk]  int32 / fp32 / fp32
 *    dq, dk, dw   like q, k, w.
 * Query head h belongs to key head h / (N1/N2).  Indices are relative to
 * their batch's key sequence.  Outputs are fully overwritten: softmax_out is
 * 0 at -1 slots, dk is 0 for keys no slot names.
 */
#ifndef SLIKL_H
#define SLIKL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  NULLPTR mirrors the page family's null-pointer errors,
 * PARAM_INVALID its parameter errors (dtype, layout, shape, range, missing
 * cuSeqLens for TND). */
typedef enum slikl_status {
    SLIKL_OK = 0,
    SLIKL_ERR_NULLPTR = 1,        /* a required pointer is NULL                 */
    SLIKL_ERR_PARAM_INVALID = 2,  /* a descriptor field is out of its range     */
    SLIKL_ERR_UNSUPPORTED = 3,    /* valid per the page, not built here          */
    SLIKL_ERR_WORKSPACE = 4,      /* workspace missing or smaller than required */
    SLIKL_ERR_LAUNCH = 5,         /* a HIP launch or device query failed        */
} slikl_status;

enum { SLIKL_LAYOUT_BSND = 0, SLIKL_LAYOUT_TND = 1 };
enum { SLIKL_DTYPE_F16 = 0, SLIKL_DTYPE_BF16 = 1 };
/* Metadata split modes: WEIGHTED balances (valid slots + overhead) per unit;
 * ROWS is the even row split of the metadata pre-pass prior art. */
enum { SLIKL_SPLIT_WEIGHTED = 0, SLIKL_SPLIT_ROWS = 1 };
/* dK strategies.  SCATTER adds each slot's dK part into the key rows with
 * atomics (fp32, or int64 fixed point when deterministic).  DENSE (BSND, or TND
 * with the maxima max_seqlen_q / max_seqlen_k given) writes per (query row, key)
 * records and runs a key-major kernel that sums over query rows in registers: no
 * atomics, bitwise reproducible; it pays off when the top-k lists cover a fair
 * share of each batch's keys.  SORTED (T1*N2*topk < 2^31 - 65536, and with head
 * groups N1/N2 up to 64 N2*D*2 < 16384 bytes, else UNSUPPORTED) writes each valid slot's dK part once
 * (fp32) into a buffer (workspace: about D*4 + 16 bytes per (unit, slot) more) and
 * sums each key's parts through a key-sorted list of them: no atomics on hot keys
 * (global atomics only where a key's run is split between two waves); deterministic
 * mode sums in int64 fixed point, so its result is bitwise reproducible.  With L the
 * key length per batch (S2, or max_seqlen_k for TND), AUTO picks DENSE when
 * L <= 16 topk (L <= 32 topk when deterministic), there are at least 2048 units and
 * the records fit in 8 GiB; else SORTED when it is supported, there are at least 2048
 * units and its parts fit in 8 GiB; else SCATTER. */
enum { SLIKL_DK_AUTO = 0, SLIKL_DK_SCATTER = 1, SLIKL_DK_DENSE = 2, SLIKL_DK_SORTED = 3 };

/* Metadata array (int32, SLIKL_METADATA_INTS entries).  A "unit" is one
 * (query row, key head) pair, u = row * N2 + g.
 *   [0] total units          [1] former size (ROWS)   [2] remain size (ROWS)
 *   [3] remain count (ROWS)  [4] used parts           [5] max key length
 *   [6] parts P              [7] split mode           [8] error word
 *   [9] per-unit overhead    [10..15] 0
 *   [16 + i], i = 0..P: first unit of part i (part i = [b_i, b_{i+1})).
 * Error word bits: 1 = bad cuSeqLensQ, 2 = bad cuSeqLensK, 4 = an index out
 * of its batch's key range (WEIGHTED mode only; ROWS reads no indices), 8 = a TND
 * sequence longer than the max_seqlen_q / max_seqlen_k given for its side. */
#define SLIKL_METADATA_HEADER 16
#define SLIKL_MAX_PARTS 2048
#define SLIKL_METADATA_INTS 2080
/* Fixed cost of one unit in valid-slot equivalents for the WEIGHTED split
 * (loads, compaction, softmax and epilogue latency of a unit vs the per-slot
 * cost of the two key passes, measured on MI355X): SLIKL_UNIT_OVERHEAD for the
 * SCATTER dK strategy, SLIKL_UNIT_OVERHEAD_DENSE for DENSE and SORTED, whose fused
 * kernels' per-slot key passes are cheaper relative to their per-unit work. */
#define SLIKL_UNIT_OVERHEAD 512
#define SLIKL_UNIT_OVERHEAD_DENSE 1024

typedef struct slikl_desc {
    int32_t layout_q;        /* SLIKL_LAYOUT_*                                        */
    int32_t layout_k;        /* SLIKL_LAYOUT_*                                        */
    int32_t dtype;           /* SLIKL_DTYPE_* of q, k, dq, dk                         */
    int32_t deterministic;   /* 0: fp32 atomic dK (run-to-run order may vary);
                                1: bitwise reproducible dK (fixed-point integer sum)  */
    int64_t batch;           /* B (> 0).  TND: number of sequences, cuSeqLens hold B+1 */
    int64_t s1;              /* BSND q: S1 (> 0); TND q: T1 (>= 0, total rows)         */
    int64_t s2;              /* BSND k: S2 (> 0); TND k: T2 (>= 0, total rows)         */
    int64_t n1;              /* query (indexer) heads, 1..128                          */
    int64_t n2;              /* key heads, >= 1, divides n1                            */
    int64_t d;               /* head dim: 32, 64 or 128                                */
    int64_t topk;            /* 1..2048                                                */
    const int32_t *cu_seqlens_q; /* device, B+1 entries starting at 0; required iff TND q */
    const int32_t *cu_seqlens_k; /* device, B+1 entries starting at 0; required iff TND k */
    int32_t num_parts;       /* metadata parts; 0 = library default (CUs x blocks/CU)  */
    int32_t split_mode;      /* SLIKL_SPLIT_*                                         */
    int32_t dk_mode;         /* SLIKL_DK_*; DENSE with a TND side needs its maximum   */
    /* TND sides only (ignored for BSND): the longest sequence of the side, 0 = not
     * given.  The DENSE dK strategy sizes its per-(query row, key) records by them, so
     * with a TND side it needs both given (else DENSE -> UNSUPPORTED, AUTO -> SCATTER).
     * A sequence longer than its given maximum violates the contract: in the DENSE
     * strategy its keys past the maximum are treated as -1 slots and its rows past the
     * maximum add nothing to dk, and the metadata pre-pass sets error bit 8. */
    int64_t max_seqlen_q;
    int64_t max_seqlen_k;
    /* Optional output (device, fp32 [T1, N2], NULL = not computed): per (query row,
     * key head) unit, the term of the formula section's loss L = sum_t KL(p_t ||
     * Softmax(I_t)), i.e. sum over the unit's valid slots with p > 0 of
     * p (log p - log softmaxOut) (0 log 0 = 0, duplicate slots count separately,
     * 0 for a unit without a valid slot).  Computed in the softmax step of the same
     * call, in fp32.  Sum it for L. */
    float *kl_loss;
    /* TND sides only (ignored for BSND), optional (device int32 [B], NULL = whole
     * sequences): the seqUsedQ / seqUsedK inputs of the constraints section, read as
     * each batch's used length (values clamped to [0, the sequence's length]; a batch
     * given 0 takes no part).  Query rows past seq_used_q[b] take no part: their dq,
     * dw, softmaxOut (and kl_loss) are 0 and their indices are not read for errors.
     * The batch's key range is cut to seq_used_k[b]: an index at or past it is out of
     * range (skipped, error bit 4). */
    const int32_t *seq_used_q;
    const int32_t *seq_used_k;
} slikl_desc;

/* First phase (the page's "GetWorkspaceSize" step): validate `desc` and return
 * the workspace bytes slikl_grad and slikl_grad_metadata need.  Host only: no
 * device access.  Errors: NULLPTR (desc or bytes NULL, or a TND side without
 * its cuSeqLens pointer), PARAM_INVALID (any field out of range). */
slikl_status slikl_grad_workspace_size(const slikl_desc *desc, size_t *bytes);

/* Number of metadata parts the library uses for `desc` (num_parts, or the
 * default derived from the current device).  Queries the current HIP device
 * when num_parts == 0 (LAUNCH if that fails). */
slikl_status slikl_grad_parts(const slikl_desc *desc, int32_t *parts);

/* Per-unit overhead (valid-slot equivalents) the WEIGHTED split uses for
 * `desc`: SLIKL_UNIT_OVERHEAD_DENSE when the resolved dK strategy is DENSE or
 * SORTED (which runs the dense strategy's 64-head fused kernel), else
 * SLIKL_UNIT_OVERHEAD.  Host only.  PARAM_INVALID / UNSUPPORTED as
 * slikl_grad_workspace_size; NULLPTR for a null argument. */
slikl_status slikl_grad_unit_overhead(const slikl_desc *desc, int32_t *overhead);

/* The dK strategy a call with `desc` runs: SLIKL_DK_SCATTER, SLIKL_DK_DENSE or
 * SLIKL_DK_SORTED (AUTO resolved as described at SLIKL_DK_*).  Host only.
 * PARAM_INVALID / UNSUPPORTED as slikl_grad_workspace_size; NULLPTR for a null
 * argument. */
slikl_status slikl_grad_dk_strategy(const slikl_desc *desc, int32_t *strategy);

/* Load-balancing metadata pre-pass (prior art: the metadata article's
 * 功能定位 and Metadata 输出布局 sections describe an AICPU pre-operator
 * that splits the merged B*S1 rows over cores into a fixed int32 array).
 * Enqueues device kernels that write SLIKL_METADATA_INTS int32 values to
 * `metadata` (device).  WEIGHTED mode reads `sparse_indices` (device, required
 * then); ROWS mode ignores it (may be NULL).  `workspace` is the same buffer
 * slikl_grad takes (at least slikl_grad_workspace_size bytes).  The result
 * depends only on desc, the indices and the parts count. */
slikl_status slikl_grad_metadata(const slikl_desc *desc, const int32_t *sparse_indices,
                                 int32_t *metadata, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* Second phase (the page's execute step): enqueue the backward pass.
 * `metadata` may be NULL (the library then runs the metadata pre-pass into
 * the workspace first) or an array written by slikl_grad_metadata for the
 * same desc and indices.  Results do not depend on the metadata: dq, dw and
 * softmax_out are bitwise identical for any split; dk is bitwise identical
 * too in deterministic mode, and equal up to fp32 summation order otherwise.
 * Errors: NULLPTR (a required pointer NULL), PARAM_INVALID, WORKSPACE
 * (workspace NULL or workspace_bytes too small), LAUNCH. */
slikl_status slikl_grad(const slikl_desc *desc, const void *q, const void *k,
                        const float *w, const int32_t *sparse_indices,
                        const float *attn_softmax_l1norm, const int32_t *metadata,
                        void *dq, void *dk, float *dw, float *softmax_out,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Phases of one slikl_grad call, for slikl_grad_profiled. */
enum {
    SLIKL_PHASE_METADATA = 0,  /* metadata pre-pass (only when metadata == NULL)       */
    SLIKL_PHASE_FILL = 1,      /* zero fills of accumulators / records               */
    SLIKL_PHASE_KEY_COPY = 2,  /* fp16 copy of bf16 keys with its power-of-two scale  */
    SLIKL_PHASE_DET_SCALE = 3, /* fixed-point scale of the deterministic scatter      */
    SLIKL_PHASE_FUSED = 4,     /* the fused S / softmax / dI / dW / dq kernel          */
    SLIKL_PHASE_DK = 5,        /* the main dK kernel: key-major sums (DENSE) or the
                                  slot parts (SORTED)                                 */
    SLIKL_PHASE_DK_FINAL = 6,  /* dK finalisation (rounding / fixed-order reduce)     */
    SLIKL_PHASE_DK_PREP = 7,   /* dK task table (DENSE) or key bucket sort (SORTED)   */
    SLIKL_PHASE_DK_REDUCE = 8, /* per-key sums of the sorted parts (SORTED)           */
    SLIKL_PHASES = 9
};

/* Same work and results as slikl_grad, for measurement: records HIP events on
 * `stream` around each phase, waits for the last one, and writes the elapsed
 * milliseconds of every phase to phase_ms[0 .. SLIKL_PHASES) (0 for a phase
 * the call did not run).  Unlike slikl_grad it blocks the host until the
 * stream reaches the end of the call.  phase_ms is host memory owned by the
 * caller.  Errors as slikl_grad; NULLPTR also when phase_ms is NULL; LAUNCH
 * when an event cannot be created or read. */
slikl_status slikl_grad_profiled(const slikl_desc *desc, const void *q, const void *k,
                                 const float *w, const int32_t *sparse_indices,
                                 const float *attn_softmax_l1norm, const int32_t *metadata,
                                 void *dq, void *dk, float *dw, float *softmax_out,
                                 void *workspace, size_t workspace_bytes, void *stream,
                                 float *phase_ms);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): slikl_grad with the
 * workspace taken from a fixed array inside this library instead of the caller.
 * The array holds SLIKL_STATIC_SCRATCH_BYTES bytes per GPU, kept from the first
 * call on that GPU until the process ends; its device address is looked up once
 * per device (the call's current device).  The call allocates and frees nothing.
 * It runs the dK strategy of `desc` when that strategy's workspace fits the array;
 * with dk_mode AUTO it otherwise runs SCATTER (the least workspace: the dK
 * accumulator, T2*N2*D*4 bytes, 8 when deterministic, plus the fp16 key copy for
 * bf16 and the split prefix); slikl_grad_noalloc_strategy names the strategy.
 * Errors as slikl_grad; WORKSPACE when no strategy allowed by `desc` fits the
 * array (nothing is launched).  Every call on one GPU uses that GPU's one array,
 * which keeps the last call's contents (each call clears what must start at zero):
 * calls that overlap on one GPU (concurrent streams or host threads) race and give
 * wrong results; serialize them. */
#define SLIKL_STATIC_SCRATCH_BYTES (64u << 20)
slikl_status slikl_grad_noalloc(const slikl_desc *desc, const void *q, const void *k,
                                const float *w, const int32_t *sparse_indices,
                                const float *attn_softmax_l1norm, const int32_t *metadata,
                                void *dq, void *dk, float *dw, float *softmax_out, void *stream);

/* The dK strategy slikl_grad_noalloc runs for `desc` (as slikl_grad_dk_strategy);
 * WORKSPACE when none fits its fixed array.  Host only. */
slikl_status slikl_grad_noalloc_strategy(const slikl_desc *desc, int32_t *strategy);

/* ---------------------------------------------------------------------------
 * The target distribution p = attnSoftmaxL1Norm from the main attention.
 * The operator page's function section (接口功能) and the note after its softmax
 * equation (计算公式) describe p as the main attention's score summed over heads
 * and L1-normalised, computed by the main attention branch beforehand (the older
 * fused operator formed it in its kernel).  Per (query row, key head g) unit and
 * valid slot s of the unit's index list (key rows as for slikl_grad):
 *    z[h, s] = scale * q_main[h] . k_main[key of s, g]   for the Hm = heads / n2
 *              main-attention heads h of key head g (h = g*Hm .. g*Hm + Hm - 1),
 *    P[h, s] = exp(z[h, s] - lse[h]),
 *    p[s]    = sum_h P[h, s] / sum over the unit's valid slots of sum_h P[h, .],
 * p = 0 at -1 slots (and at indices outside their batch's key range, which are
 * skipped as in slikl_grad); a unit without a valid slot gets p = 0.  lse[h] is
 * the natural log-sum-exp of z[h, .] over the keys the main attention normalised
 * over: the caller's (its forward keeps it), or when lse is NULL the log-sum-exp
 * over the unit's valid slots, computed here (one more pass over the keys).
 *
 * Shapes (BSND | TND): q_main [B,S1,Nm,Dm] | [T1,Nm,Dm] and k_main [B,S2,N2,Dm] |
 * [T2,N2,Dm], fp16 or bf16 (one dtype); sparse_indices and p [B,S1,N2,topk] |
 * [T1,N2,topk] (int32 / fp32); lse [B,S1,Nm] | [T1,Nm] fp32.  Device pointers,
 * caller-owned, contiguous; q_main and k_main 16-byte aligned.  No workspace; the
 * call only enqueues on `stream`.  fp32 arithmetic with MFMA dot products; every
 * sum has a fixed order, so p is bitwise reproducible.
 * Errors: NULLPTR (desc, or a tensor pointer NULL while T1 > 0 / T2 > 0, or a TND
 * side without cuSeqLens), PARAM_INVALID (a field out of range, heads / n2 outside
 * 1..128, d not one of 64, 128, 256, 512, 576, n2 * d * 2 >= 16384, scale not
 * finite, misaligned q_main / k_main), LAUNCH. */
typedef struct slikl_attn_p_desc {
    int32_t layout_q;        /* SLIKL_LAYOUT_* of q_main                              */
    int32_t layout_k;        /* SLIKL_LAYOUT_* of k_main                              */
    int32_t dtype;           /* SLIKL_DTYPE_* of q_main and k_main                    */
    int32_t reserved;        /* 0                                                     */
    int64_t batch;           /* B (> 0); TND: number of sequences                     */
    int64_t s1;              /* BSND: S1 (> 0); TND: T1 (>= 0)                        */
    int64_t s2;              /* BSND: S2 (> 0); TND: T2 (>= 0)                        */
    int64_t heads;           /* Nm, main-attention query heads; heads / n2 in 1..128  */
    int64_t n2;              /* key heads (index lists), divides heads                 */
    int64_t d;               /* Dm: 64, 128, 256, 512 or 576                          */
    int64_t topk;            /* 1..2048                                               */
    float scale;             /* softmax scale of the main attention                   */
    const int32_t *cu_seqlens_q; /* device, B+1 entries starting at 0; required iff TND */
    const int32_t *cu_seqlens_k;
} slikl_attn_p_desc;

slikl_status slikl_attn_softmax_l1norm(const slikl_attn_p_desc *desc, const void *q_main,
                                       const void *k_main, const int32_t *sparse_indices,
                                       const float *lse, float *p, void *stream);

/* ---------------------------------------------------------------------------
 * The dense sibling operator (DenseLightningIndexerKLLossGrad).  The metadata
 * article (DenseLightningIndexerKLLossGradMetadata: 导读, 功能定位, 约束说明 Mask)
 * names it and fixes its mask modes: 0 = no mask, 3 = rightDownCausal (the lower
 * triangle cornered at the bottom-right vertex: row t of a batch with S1_b rows and
 * S2_b keys sees keys j <= t + S2_b - S1_b).  Its formulas are the sparse operator's
 * with the top-k set replaced by the keys the mask shows; p (attnSoftmaxL1Norm) and
 * softmax_out are dense over the key positions, [B,S1,N2,L] | [T1,N2,L] with
 * L = S2 (BSND k) or max_seqlen_k (TND k); positions a row does not see get
 * softmax_out 0 and their p is ignored.  q, k, w, dq, dk, dw as for slikl_grad.
 * `base` is a slikl_desc read as for slikl_grad except that base.topk is ignored
 * (the dense axis is L) and seq_used_q / seq_used_k must be NULL.  Limits: L in
 * 1..2048 (the fused kernel holds a row's keys in LDS; UNSUPPORTED above), and
 * cmp_ratio must be 1 (key compression is named on the page but not defined:
 * cmp_ratio in 2..128 gives UNSUPPORTED, outside 1..128 PARAM_INVALID).  The work
 * runs through slikl_grad's kernels on index lists of the visible keys that the
 * call writes into its workspace (T1*N2*L*4 bytes beyond slikl_grad's), so the dK
 * strategies, determinism, metadata and loss output behave as there.
 * Errors as slikl_grad, plus the limits above. */
typedef struct slikl_dense_desc {
    slikl_desc base;
    int32_t mask_mode;       /* 0 or 3                                                */
    int32_t cmp_ratio;       /* 1                                                     */
} slikl_dense_desc;

slikl_status slikl_dense_grad_workspace_size(const slikl_dense_desc *desc, size_t *bytes);

/* The load-balancing pre-pass of the dense operator (the metadata article's own
 * subject): writes the index lists into the workspace and splits the rows by their
 * visible keys (base.split_mode) into `metadata` (SLIKL_METADATA_INTS int32). */
slikl_status slikl_dense_grad_metadata(const slikl_dense_desc *desc, int32_t *metadata, void *workspace,
                                       size_t workspace_bytes, void *stream);

slikl_status slikl_dense_grad(const slikl_dense_desc *desc, const void *q, const void *k, const float *w,
                              const float *attn_softmax_l1norm, const int32_t *metadata, void *dq,
                              void *dk, float *dw, float *softmax_out, void *workspace,
                              size_t workspace_bytes, void *stream);

/* slikl_dense_grad with the per-phase times of slikl_grad_profiled (the index-list
 * fill is counted in SLIKL_PHASE_FILL); blocks until the call has run. */
slikl_status slikl_dense_grad_profiled(const slikl_dense_desc *desc, const void *q, const void *k,
                                       const float *w, const float *attn_softmax_l1norm,
                                       const int32_t *metadata, void *dq, void *dk, float *dw,
                                       float *softmax_out, void *workspace, size_t workspace_bytes,
                                       void *stream, float *phase_ms);

/* Static description of a status code. */
const char *slikl_status_string(slikl_status s);

#ifdef __cplusplus
}
#endif

#endif /* SLIKL_H */
