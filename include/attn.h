/*
 * libattn: fused multi-head attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI. Every tensor argument is a plain device pointer to caller-owned
 * memory; sizes travel in attn_problem. Nothing in these signatures depends
 * on a framework.
 *
 * What the calls compute (sources, by page title and section):
 *
 *  - attn_fwd: "fused multi-head attention operator" write-up on the
 *    Ascend CANN ops-nn path (zwxr.cn), section 3.1: inputs Q, K, V of
 *    shape [batch, head, seq_len, head_dim] and an optional mask, output of
 *    the same shape, each query's dot products with all keys times a scale,
 *    a softmax over the keys, then the probability-weighted sum of V rows.
 *    Section 3.2-3.3: computed tile by tile with a running maximum and sum
 *    (online softmax), so the seq_len x seq_len score matrix is never stored.
 *    Section 3.3: a mask entry of 0 sends the score to -infinity.
 *  - attn_bwd: the Xingchen-Cup report on operator optimisation (smzdm.com),
 *    section 03: the backward of (sparse) FlashAttention produces the three
 *    gradients dQ, dK, dV, recomputing the attention probabilities tile by
 *    tile because the forward kept only per-row statistics; skipped blocks
 *    of a sparse mask are never visited.
 *
 * Conventions shared by every call:
 *  - Layout: Q, O, dO, dQ are [batch, heads_q, seq_q, head_dim]; K, V, dK, dV
 *    are [batch, heads_kv, seq_k, head_dim]; all contiguous, row-major, in the
 *    problem's dtype. LSE is float32 [batch, heads_q, seq_q].
 *  - Grouped-query attention: query head h reads key/value head
 *    h / (heads_q / heads_kv).
 *  - LSE is the natural logarithm of the softmax denominator of the scaled,
 *    masked scores. A query row with no visible key gets O = 0 and
 *    LSE = -infinity (and zero gradient rows).
 *  - Execution: calls enqueue work on `stream` (a hipStream_t; NULL means the
 *    default stream) and return without synchronising. Outputs are valid once
 *    the stream reaches that point; inputs must stay unchanged until then.
 *    No host<->device copies happen inside a call.
 *  - Ownership: the library never allocates or frees device memory. Scratch
 *    space is the caller-provided `workspace`, sized by the matching
 *    *_workspace_bytes query (the planner's item list lives there); the one
 *    exception, attn_bwd_noalloc, uses a fixed array inside the library.
 *  - Errors: all argument checks run on the host before any launch or memory
 *    access (the only HIP calls before them are device-attribute queries);
 *    on an error nothing is launched and nothing is written. Device-resident
 *    mask data cannot be checked on the host: padding lengths are clamped to
 *    [0, seq] by the kernels. A failed launch returns ATTN_ERR_HIP.
 *  - Device: calls run on the calling thread's current HIP device. Its
 *    compute-unit and XCD counts are queried once and select the split-KV
 *    choice and the per-XCD order of work items.
 *  - Thread safety: calls may be issued from several host threads; the state
 *    is the set of loaded kernels, the per-device counts above and the
 *    scratch array of attn_bwd_noalloc (whose calls must not overlap on one
 *    device).
 */
#ifndef LIBATTN_ATTN_H
#define LIBATTN_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL */
  ATTN_ERR_SHAPE = 2,       /* a size is < 1, heads_q % heads_kv != 0, or seq_q != seq_k where required */
  ATTN_ERR_ALIGN = 3,       /* a tensor base pointer is not 16-byte aligned */
  ATTN_ERR_DTYPE = 4,       /* unknown dtype */
  ATTN_ERR_MASK = 5,        /* unknown mask kind, missing mask data, or block size != 64 */
  ATTN_ERR_WORKSPACE = 6,   /* workspace smaller than the *_workspace_bytes query, or NULL when non-zero is needed */
  ATTN_ERR_ALIAS = 7,       /* an output range overlaps an input range or another output */
  ATTN_ERR_UNSUPPORTED = 8, /* valid but not implemented: head_dim other than 64/128, or an unsupported combination */
  ATTN_ERR_HIP = 9,         /* the HIP runtime reported an error when launching */
  ATTN_ERR_TOO_LARGE = 10   /* attn_bwd_noalloc: the problem needs more scratch than its fixed array holds */
} attn_status;

/* Element types. ATTN_FP8_E4M3 (OCP e4m3, 1 byte) is a forward input type: Q, K, V are fp8,
 * O is written in bf16 and LSE in fp32; a per-tensor dequantisation of the inputs folds into the
 * arguments (scale *= q_scale * k_scale; multiply O by v_scale afterwards). */
typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1, ATTN_FP8_E4M3 = 2 } attn_dtype;

typedef enum {
  ATTN_MASK_NONE = 0,    /* every key visible */
  ATTN_MASK_CAUSAL = 1,  /* key j hidden from query i when j > i; needs seq_q == seq_k */
  ATTN_MASK_PADDING = 2, /* per batch element b: (i, j) visible iff i < len[b] and j < len[b] */
  ATTN_MASK_BLOCK = 3,   /* block_q x block_k tiles kept where the layout byte is non-zero */
  ATTN_MASK_DENSE = 4    /* (i, j) visible iff the dense mask byte is non-zero */
} attn_mask_kind;

/* Sizes of one attention problem. dtype is an attn_dtype value. */
typedef struct {
  int32_t batch, heads_q, heads_kv, seq_q, seq_k, head_dim;
  int32_t dtype;
} attn_problem;

/*
 * Mask descriptor. kind is an attn_mask_kind value.
 *  lengths      PADDING: device int32[batch], the valid length of both queries
 *               and keys of each batch element (clamped to [0, seq]).
 *  block_layout BLOCK: device uint8, one [nb_q][nb_k] row-major matrix per
 *               (b, h) at element offset b*layout_stride_b + h*layout_stride_h,
 *               nb_q = ceil(seq_q / block_q), nb_k = ceil(seq_k / block_k);
 *               0 = skip the tile, non-zero = keep it. Strides of 0 share one
 *               layout across batch elements and/or heads. A tile on a ragged
 *               edge covers only the rows/columns that exist.
 *  block_q, block_k  BLOCK: tile sizes; the library supports 64 x 64.
 *  dense        DENSE: device uint8, one [seq_q][seq_k] row-major matrix per
 *               (b, h) at element offset b*dense_stride_b + h*dense_stride_h
 *               (h = query head); 0 = the score becomes -infinity, non-zero =
 *               visible. This is the generic mask[i][j] of the fused
 *               multi-head attention operator write-up (zwxr.cn), section 3.3.
 *               Strides of 0 share one mask across batch elements and/or heads.
 *               Each call packs it once to bits and a 64x64 block layout in
 *               the workspace, so blocks it hides entirely are never visited.
 * Pointers a kind does not use are ignored and may be NULL.
 */
typedef struct {
  int32_t kind;
  const int32_t *lengths;
  const uint8_t *block_layout;
  int64_t layout_stride_b, layout_stride_h;
  int32_t block_q, block_k;
  const uint8_t *dense;
  int64_t dense_stride_b, dense_stride_h;
} attn_mask;

/* Bytes of workspace attn_fwd needs for this problem and mask (0 if none). Equal to
 * attn_fwd_ex_workspace_bytes(problem, mask, 0). */
size_t attn_fwd_workspace_bytes(const attn_problem *problem, const attn_mask *mask);

/*
 * Forward: O = softmax(scale * Q K^T + mask) V and LSE per query row.
 * Q, K, V: inputs (see layout above). O: output in the problem dtype.
 * LSE: float32 output [batch, heads_q, seq_q]. workspace: device scratch of
 * at least attn_fwd_workspace_bytes() bytes (may be NULL if that is 0).
 * Supported: dtype F32, BF16 or FP8_E4M3 (O in bf16 for fp8 inputs); head_dim 64 or 128; every mask kind;
 * heads_q a multiple of heads_kv.
 */
attn_status attn_fwd(const attn_problem *problem, const void *Q, const void *K, const void *V,
                     const attn_mask *mask, float scale, void *O, float *LSE,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * Forward with a split of every work item's key range (split-KV), following the core split
 * along the sequence direction of the fused multi-head attention operator write-up (zwxr.cn),
 * section 4.2 (split by head first, then by sequence, to keep every core busy).
 * kv_splits workgroups share the key tiles of one (batch, head, query tile) item in equal runs;
 * each writes its partial O (normalised over its keys, fp32) and the log of its partial
 * denominator to the workspace. A merge kernel then writes LSE = log sum_s exp(LSE_s) and
 * O = sum_s exp(LSE_s - LSE) O_s. The result equals attn_fwd's up to rounding.
 * kv_splits: 0 = automatic (split only when there are fewer items than the GPU has compute
 * units, with at least 8 key tiles per split), 1 = never split, 2..32 = that many splits (at most one per
 * 64-key tile). A value outside 0..32 returns ATTN_ERR_SHAPE; more than 1 with F32 returns
 * ATTN_ERR_UNSUPPORTED. Other arguments and errors are as for attn_fwd; the workspace must hold
 * attn_fwd_ex_workspace_bytes(problem, mask, kv_splits) bytes.
 */
attn_status attn_fwd_ex(const attn_problem *problem, const void *Q, const void *K, const void *V,
                        const attn_mask *mask, float scale, void *O, float *LSE,
                        void *workspace, size_t workspace_bytes, int32_t kv_splits, void *stream);

/* Workspace bytes of attn_fwd_ex with this kv_splits (0 for an invalid problem). */
size_t attn_fwd_ex_workspace_bytes(const attn_problem *problem, const attn_mask *mask, int32_t kv_splits);

/* Number of splits attn_fwd_ex would use for this kv_splits (0 for an invalid problem). */
int32_t attn_fwd_kv_splits(const attn_problem *problem, const attn_mask *mask, int32_t kv_splits);

/* Bytes of workspace attn_bwd needs (the planner lists, D = rowsum(dO * O) and LSE * log2(e)).
 * Equal to attn_bwd_ex_workspace_bytes(problem, mask, 0). */
size_t attn_bwd_workspace_bytes(const attn_problem *problem, const attn_mask *mask);

/*
 * Backward: dQ, dK, dV of L = sum(dO * O) for the forward above, given the
 * forward's O and LSE and the same mask and scale (the scale is needed to
 * recompute the probabilities and to scale dQ and dK).
 * Q, K, V, O, dO: inputs in the problem dtype; LSE: float32 from attn_fwd.
 * dQ, dK, dV: outputs in the problem dtype. For grouped-query attention dK
 * and dV sum over the query heads sharing a key/value head.
 * Supported: dtype BF16; head_dim 128 or 64; every mask kind.
 */
attn_status attn_bwd(const attn_problem *problem, const void *Q, const void *K, const void *V,
                     const void *O, const void *dO, const float *LSE, const attn_mask *mask,
                     float scale, void *dQ, void *dK, void *dV, void *workspace,
                     size_t workspace_bytes, void *stream);

/* Flags of attn_bwd_ex. */
enum {
  /* Single pass: the report on the sparse FlashAttention backward (Xingchen-Cup, smzdm.com),
   * section 03, names two ways to resolve the conflicting accumulation directions of the three
   * gradients: two loops, or many cores adding into the same place with write conflicts resolved.
   * attn_bwd takes the two loops (a dK/dV pass and a dQ pass, deterministic). With this flag the
   * dK/dV pass also adds each block's dQ contribution (dS K) into an fp32 accumulator in the
   * workspace with hardware float atomics, and a convert kernel writes dQ = scale * accumulator
   * in bf16: no second recomputation of S and dP, but dQ depends on the order of the atomic
   * additions (not bitwise reproducible from run to run; dK and dV still are). */
  ATTN_BWD_ATOMIC_DQ = 1,
  /* The workspace already holds the backward's two work lists, written by
   * attn_fwd_with_bwd_plan (below) for the same problem and mask, with the mask's data unchanged
   * since and no other use of the workspace in between: the call launches no planner. The
   * library cannot check the lists' contents; a list from another problem only makes its
   * out-of-range items do nothing (wrong results, no out-of-bounds access). Not combinable with
   * ATTN_BWD_ATOMIC_DQ (ATTN_ERR_UNSUPPORTED). */
  ATTN_BWD_PLANNED = 2
};

/*
 * Backward with options (flags: 0, ATTN_BWD_ATOMIC_DQ or ATTN_BWD_PLANNED). Arguments, outputs
 * and errors as for attn_bwd; an unknown flag returns ATTN_ERR_SHAPE; the workspace must hold
 * attn_bwd_ex_workspace_bytes(problem, mask, flags) bytes (with ATTN_BWD_ATOMIC_DQ it includes
 * a float32 [batch, heads_q, seq_q, head_dim] accumulator).
 */
attn_status attn_bwd_ex(const attn_problem *problem, const void *Q, const void *K, const void *V,
                        const void *O, const void *dO, const float *LSE, const attn_mask *mask,
                        float scale, void *dQ, void *dK, void *dV, void *workspace,
                        size_t workspace_bytes, int32_t flags, void *stream);

/* Workspace bytes of attn_bwd_ex with these flags (0 for an invalid problem or flag). */
size_t attn_bwd_ex_workspace_bytes(const attn_problem *problem, const attn_mask *mask, int32_t flags);

/*
 * Forward that also plans the backward which follows it. The report on the sparse FlashAttention
 * operator (Xingchen-Cup, smzdm.com) opens with a slow statistics prologue that cost more than it
 * saved, and its section 03 asks for the uneven sparse blocks to be spread evenly over the cores;
 * the planner that orders the work items longest first is that spreading, and this entry point
 * runs it once per forward/backward pair instead of once per call: one planner launch writes the
 * forward's list into `workspace` and the backward's two lists into `bwd_workspace`. The forward
 * is attn_fwd's (the library chooses the key-range split). A later attn_bwd_ex with
 * ATTN_BWD_PLANNED on `bwd_workspace` then launches no planner.
 * bwd_workspace: device memory of attn_bwd_workspace_bytes(problem, mask) bytes, 16-byte aligned,
 *   owned by the caller, overlapping no input, output, mask or `workspace`.
 * Errors: as attn_fwd, and ATTN_ERR_NULL (bwd_workspace null), ATTN_ERR_WORKSPACE (too small),
 * ATTN_ERR_ALIGN, ATTN_ERR_ALIAS, ATTN_ERR_UNSUPPORTED (a problem attn_bwd does not support,
 * such as an F32 or F8 dtype), all checked before any launch.
 */
attn_status attn_fwd_with_bwd_plan(const attn_problem *problem, const void *Q, const void *K, const void *V,
                                   const attn_mask *mask, float scale, void *O, float *LSE, void *workspace,
                                   size_t workspace_bytes, void *bwd_workspace, size_t bwd_workspace_bytes,
                                   void *stream);

/*
 * Backward that allocates nothing, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation. Same arguments, outputs and
 * kernels as attn_bwd (two passes, deterministic, results bitwise equal to attn_bwd's) minus the
 * workspace: the scratch lives in a fixed device array of attn_bwd_noalloc_scratch_bytes() bytes
 * (32 MiB) inside the library, one copy per device, held until the process ends. A problem whose
 * attn_bwd_workspace_bytes() exceeds that returns ATTN_ERR_TOO_LARGE before any GPU call; other
 * errors are as for attn_bwd. Calls on one device share its array, so calls that overlap in time
 * on one device (other streams or host threads) race; calls ordered on one stream are safe. The
 * array's address on a device is looked up on the first call on that device (a symbol query, no
 * allocation); no call allocates or frees memory.
 */
attn_status attn_bwd_noalloc(const attn_problem *problem, const void *Q, const void *K, const void *V,
                             const void *O, const void *dO, const float *LSE, const attn_mask *mask, float scale,
                             void *dQ, void *dK, void *dV, void *stream);

/* Size in bytes of the fixed scratch array attn_bwd_noalloc uses on each device. */
size_t attn_bwd_noalloc_scratch_bytes(void);

/*
 * Kernel timing hook, for profiling tools. Kernel classes: */
typedef enum {
  ATTN_KERNEL_PLAN = 0,     /* tile-list scheduler */
  ATTN_KERNEL_FWD = 1,      /* fused forward */
  ATTN_KERNEL_BWD_PRE = 2,  /* backward preprocess, Delta = rowsum(dO * O) (single-pass mode only;
                               the two-pass dQ pass computes it for its own rows) */
  ATTN_KERNEL_BWD_DKDV = 3, /* backward dK/dV pass */
  ATTN_KERNEL_BWD_DQ = 4,   /* backward dQ pass */
  ATTN_KERNEL_FWD_MERGE = 5, /* split-KV merge of the forward */
  ATTN_KERNEL_BWD_DQ_CONVERT = 6, /* single-pass backward: dQ accumulator to bf16 */
  ATTN_KERNEL_MASK_PACK = 7, /* dense mask to bits and a block layout */
  ATTN_KERNEL_CLASSES = 8
} attn_kernel_class;
/*
 * While set for a class, each launch of that class records start_events[i] before it and
 * stop_events[i] after it (hipEventRecord on the call's stream), i = *count, then increments
 * *count; launches beyond `capacity` are not bracketed. The events (hipEvent_t, created by the
 * caller with timing enabled) and `count` are caller-owned and must outlive the setting. Pass
 * capacity 0 (or NULL arrays) to clear. Not thread-safe: set it while no other thread calls the
 * library. Returns ATTN_ERR_SHAPE for an unknown class, ATTN_ERR_NULL for a missing count.
 */
attn_status attn_set_timing_events(int32_t kernel_class, void *const *start_events, void *const *stop_events,
                                   int32_t capacity, int32_t *count);

/* Static English description of a status code (never NULL). */
const char *attn_status_string(attn_status status);

/* Library version as major*10000 + minor*100 + patch. */
int32_t attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBATTN_ATTN_H */
