/*
 * ffa.h -- C ABI of the MI355X (gfx950) flexible-mask flash attention (forward,
 *          backward and total attention).
 *
 * The operation (MagiAttention quickstart, section "Single-GPU
 * Flex-Flash-Attention"; FlagAttention user guide, section "FlashAttention"):
 *
 *   q [total_q, Hq, D], k and v [total_k, Hkv, D], head_dim D contiguous.
 *   A mask is a list of S slices (q_range, k_range, type) with half-open
 *   ranges.  Query row i of slice s (qs <= i < qe) sees
 *     FULL      (type 0): keys [ks, ke)
 *     CAUSAL    (type 1): keys [ks, ke - (qe - 1 - i))             -- bottom-right aligned
 *     INVCAUSAL (type 2): keys [ks + (i - qs), ke)                 -- top-left aligned
 *     BICAUSAL  (type 3): keys [ks + (i - qs), ke - (qe - 1 - i))  -- a band (sliding window)
 *   (the kv-interval formula of the MagiAttention blog page "Calculate KV
 *   Interval Boundaries for Mask Types", bits 0 / 1 of the type).
 *   Query head h uses kv head h / (Hq / Hkv); Hq % Hkv == 0 is required.
 *   With s_ij = softmax_scale * q_i . k_j over the visible keys V(i):
 *     lse[i,h] = ln sum_{j in V(i)} exp(s_ij)           (-inf if V(i) is empty)
 *     out[i,h] = sum_{j in V(i)} exp(s_ij - lse[i,h]) v_j  (0 if V(i) is empty)
 *   q, k, v and out are bfloat16 (or IEEE half with ffa_attn_extras.dtype),
 *   rounded to nearest even; lse is float32; the kernels accumulate in float32
 *   (the quickstart states fp32 reduction).  head_dim is 16, 32, 64 or 128.
 *
 * Calls:
 *   ffa_plan        validate the slices and build the work plan on the host
 *   ffa_plan_info_get  sizes and statistics of a plan
 *   ffa_plan_sizes  the metadata and workspace sizes alone
 *   ffa_plan_upload copy the plan's metadata to a caller-owned device buffer
 *   ffa_plan_export copy the same metadata to host memory (inspection, tests)
 *   ffa_fwd         run the forward on a stream (main kernel, then the split
 *                   combine when the plan has split rows)
 *   ffa_combine     the split combine alone, over partials ffa_fwd left
 *   ffa_bwd         gradients dq, dk, dv from the forward's out and lse and the
 *                   upstream gradient dout (plan built with FFA_PLAN_BACKWARD)
 *   ffa_total_attention  attention probabilities summed over the queries, per key
 *   ffa_plan_destroy, ffa_status_string, ffa_last_error, ffa_abi_version
 *
 * Ownership.  The library owns only the host plan.  All device memory (meta,
 * workspace, q/k/v/out/lse) belongs to the caller.  The library never allocates
 * or frees device memory and never synchronises a stream; ffa_fwd only enqueues
 * kernels, so a device fault surfaces at the caller's next synchronisation.
 * ffa_fwd, ffa_combine, ffa_bwd and ffa_total_attention enqueue kernels only (no
 * copies, no memory clears), so they may be captured into a HIP graph once the
 * plan's metadata has been uploaded (ffa_plan_upload copies from host memory and
 * belongs outside the capture).
 *
 * Errors.  Every call returns an ffa_status.  Arguments are validated before
 * anything is enqueued, so a non-OK return means nothing was written.
 * ffa_last_error() returns a thread-local message for the last failure in the
 * calling thread (offending slice, stride, size...).  Nothing throws across the ABI.
 */
#ifndef FFA_H
#define FFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FFA_ABI_VERSION 3

#define FFA_MASK_FULL 0
#define FFA_MASK_CAUSAL 1
#define FFA_MASK_INVCAUSAL 2
#define FFA_MASK_BICAUSAL 3

#define FFA_DTYPE_BF16 0
#define FFA_DTYPE_F16 1

#define FFA_PLAN_NATURAL_ORDER 1u
#define FFA_PLAN_BACKWARD 2u

typedef enum {
  FFA_OK = 0,
  FFA_ERR_NULL = 1,        /* a required pointer is NULL                                   */
  FFA_ERR_SHAPE = 2,       /* total_q/total_k outside [0, 2^30 - 2], heads <= 0,
                              head_dim not 16/32/64/128                                    */
  FFA_ERR_GQA = 3,         /* heads_q % heads_kv != 0                                      */
  FFA_ERR_RANGE = 4,       /* a range leaves [0, total] or has start > end                 */
  FFA_ERR_MASK_TYPE = 5,   /* a type outside 0..3 (FULL, CAUSAL, INVCAUSAL, BICAUSAL)      */
  FFA_ERR_OVERLAP = 6,     /* two slices make some (q, k) pair visible twice               */
  FFA_ERR_WORKSPACE = 7,   /* meta or workspace buffer missing or too small                */
  FFA_ERR_HIP = 8,         /* a HIP runtime call failed (message in ffa_last_error)        */
  FFA_ERR_HOST_OOM = 9,    /* host allocation failed while planning                        */
  FFA_ERR_ALIGN = 10,      /* a tensor base or stride is not a multiple of 8 elements      */
  FFA_ERR_ARG = 11         /* any other invalid argument (batch, scale, plan state)        */
} ffa_status;

/*
 * Optional arguments of ffa_fwd / ffa_bwd (pass NULL for none; zero fields are
 * "off").  MagiAttention quickstart, "Single-GPU Flex-Flash-Attention": the FFA
 * call takes an optional fp32 `sink` of [S_sink, Hq] logits (or [Tq, S_sink, Hq]
 * per row in the extension functions' "ssh" layout) and a `softcap` (0 = off).
 * Readings (the pages name them without formulas):
 *   sink    each logit adds exp(sink) to the row's softmax denominator and
 *           carries no value; it is neither scaled nor capped.  lse includes
 *           it; a row that sees no key gets out = 0 and lse = ln sum exp(sink).
 *   softcap score s = softmax_scale q.k becomes softcap * tanh(s / softcap).
 * sink element (b, row, s, h) is at sink[b*sink_sb + row*sink_st + s*sink_ss +
 * h*sink_sh] (sink_st = 0: the same logits for every row).  ffa_bwd writes
 * d sink to dsink with the same strides when dsink is not NULL (summed over
 * rows when sink_st == 0, in a fixed order).
 * flags: 0 or FFA_EXTRAS_ROUNDED_NORM (any other bit: FFA_ERR_ARG).  With it the
 * forward divides each row's output by the sum of the 16-bit rounded weights
 * that its P.V product multiplies, instead of the sum of their fp32 values (lse
 * still comes from the fp32 sum): out is then a convex combination of value rows
 * up to fp32 accumulation, which keeps a row dominated by one key met past the
 * row's first key tile within the output's own rounding (default: within that
 * plus up to 2^-9 of the value row).  About 6-9% slower.  ffa_bwd ignores it.
 */
#define FFA_EXTRAS_ROUNDED_NORM 1
typedef struct {
  const float* sink;
  float* dsink;
  int64_t sink_sb, sink_st, sink_ss, sink_sh;
  int32_t n_sink;   /* sink logits per (row, head); 0: no sink; at most 65536 */
  float softcap;    /* 0: off; must be finite and >= 0 */
  int32_t dtype;    /* element type of q, k, v, out, dout and the gradients:
                       FFA_DTYPE_BF16 (0, also when extras is NULL) or FFA_DTYPE_F16 */
  int32_t flags;    /* 0 or FFA_EXTRAS_ROUNDED_NORM (forward only) */
} ffa_attn_extras;

/* Opaque host plan; immutable after ffa_plan, safe to share between threads. */
typedef struct ffa_plan_s* ffa_plan_t;

/* Planner options.  Pass NULL for defaults; zero fields also mean "default". */
typedef struct {
  /* Split-K control.  0: automatic (split only when the work cannot fill the
   * device: long rows and few items).  > 0: split every item whose key-tile
   * count exceeds this value into chunks of about this many tiles.  < 0: never
   * split.  Split items write float32 partial (out, lse) to the workspace and a
   * second kernel merges them with a global logsumexp (FlagAttention user
   * guide, "Split-KV and paged attention"). */
  int32_t split_tiles;
  /* Upper bound on chunks per split item (0: 64). */
  int32_t max_splits;
  /* Compute units to plan for (0: query the current HIP device). */
  int32_t num_cus;
  /* Bit 0 (FFA_PLAN_NATURAL_ORDER): keep items in natural order (no
   * longest-first ordering).  Bit 1 (FFA_PLAN_BACKWARD): also plan the
   * backward worklists that ffa_bwd needs. */
  uint32_t flags;
} ffa_plan_opts;

/* Plan statistics.  Byte sizes are what ffa_plan_upload / ffa_fwd require. */
typedef struct {
  int64_t meta_bytes;        /* device metadata buffer size (ffa_plan_upload)             */
  int64_t workspace_bytes;   /* split-K workspace per batch element (0: no split rows)     */
  int64_t visible_pairs;     /* unmasked (q, k) pairs per head: FLOPs = 4 * D * Hq * this  */
  int64_t computed_pairs;    /* (row, key) pairs the kernels evaluate per head, incl. waste */
  int32_t num_items;         /* workgroups of the main kernel per batch element            */
  int32_t num_runs;          /* (item, slice) key runs                                     */
  int32_t num_combine;       /* combine entries (split row blocks)                         */
  int32_t num_split_items;   /* main-kernel items that write partials                      */
  int32_t heads_per_item;    /* query heads one workgroup covers (GQA group share)          */
  int32_t rows_per_item;     /* query rows one workgroup covers                             */
  int32_t block_n;           /* keys per tile                                               */
  int32_t max_item_tiles;    /* longest item, in key tiles                                  */
  int64_t total_tiles;       /* key tiles over all items                                    */
  /* backward (zero unless the plan was built with FFA_PLAN_BACKWARD) */
  int64_t bwd_workspace_bytes; /* ffa_bwd workspace per batch element: 2 * 4 * Hq * total_q  */
  int64_t dq_tiles;          /* key tiles of the dQ kernel over all its items                 */
  int64_t kv_tiles;          /* query tiles of the dK/dV kernel, counted once per query head  */
  int32_t num_dq_items;      /* workgroups of the dQ kernel per batch element                 */
  int32_t num_kv_items;      /* workgroups of the dK/dV kernel per batch element              */
} ffa_plan_info;

/*
 * Build a plan.  q_ranges, k_ranges: HOST int32 [num_slices][2] (start, end);
 * mask_types: HOST int32 [num_slices].  num_slices may be 0 (every row empty).
 * The slices must be pairwise disjoint in the (q, k) plane (FFA_ERR_OVERLAP
 * otherwise); empty ranges (start == end) are valid no-ops.  head_dim must be
 * 16, 32, 64 or 128 (the FlagAttention user guide, "FlashAttention").  On success *plan_out receives a plan the caller must destroy.
 */
ffa_status ffa_plan(const int32_t* q_ranges, const int32_t* k_ranges, const int32_t* mask_types,
                    int32_t num_slices, int32_t total_q, int32_t total_k, int32_t heads_q,
                    int32_t heads_kv, int32_t head_dim, const ffa_plan_opts* opts,
                    ffa_plan_t* plan_out);

/* All statistics of a plan (sizes, the visible-pair count behind the FLOP
 * metric, item counts).  FFA_ERR_NULL when plan or info is NULL. */
ffa_status ffa_plan_info_get(ffa_plan_t plan, ffa_plan_info* info);

/* The two buffer sizes a caller must provide, without the rest of the
 * statistics: *meta_bytes for ffa_plan_upload, *workspace_bytes for ffa_fwd
 * per batch element (0 when the plan splits no row).  Either output pointer
 * may be NULL (that size is not returned); FFA_ERR_NULL when plan is NULL. */
ffa_status ffa_plan_sizes(ffa_plan_t plan, size_t* meta_bytes, size_t* workspace_bytes);

/* Copy the plan metadata (info.meta_bytes) into d_meta, a device buffer of
 * meta_bytes >= info.meta_bytes, with hipMemcpyAsync on `stream` (a hipStream_t;
 * NULL = the null stream).  The copy is ordered before later work on the stream. */
ffa_status ffa_plan_upload(ffa_plan_t plan, void* d_meta, size_t meta_bytes, void* stream);

/* Copy the same metadata to host memory h_meta (>= info.meta_bytes bytes).
 * Layout: int32 header[16], then items[num_items][16] (8 item fields followed
 * by a copy of the item's first run), runs[num_runs][8],
 * combine[num_combine][8]; with FFA_PLAN_BACKWARD, header[14] is the int32
 * offset of the backward section: a header[8], then the dQ items and runs and
 * the dK/dV items and runs in the same formats.  See the planner source for
 * the field order. */
ffa_status ffa_plan_export(ffa_plan_t plan, void* h_meta, size_t meta_bytes);

/*
 * Forward: out and lse of the operation at the top of this header for every
 * query row and head (MagiAttention quickstart, "Single-GPU
 * Flex-Flash-Attention": flex_flash_attn_func returns out and meta.lse;
 * FlagAttention user guide, "FlashAttention": the log-normalizer lse).  Plans
 * that split long rows run a second kernel that merges float32 partial (out,
 * lse) pairs with a global logsumexp (FlagAttention user guide, "Split-KV and
 * paged attention").  All tensor pointers are DEVICE pointers; strides are in elements.
 *   batch >= 1 independent problems share the plan; element b of every tensor
 *   starts at base + b * stride_b.
 *   q:   bf16, element (b, t, h, d) at q[b*q_sb + t*q_st + h*q_sh + d]
 *   k,v: bf16, (b, t, hkv, d) likewise with their own strides
 *   out: bf16, like q (written for every row and head)
 *   lse: fp32, (b, t, h) at lse[b*l_sb + t*l_st + h*l_sh]
 * q, k, v, out bases and their strides must be multiples of 8 elements (16 B);
 * the token strides of k and v must be in [0, 2^24) elements (FFA_ERR_ARG).
 * softmax_scale must be finite and > 0 (callers resolve "None" to 1/sqrt(D)).
 * extras: sink / softcap (see ffa_attn_extras), NULL for plain attention.
 * d_meta: the buffer filled by ffa_plan_upload.  d_workspace: workspace_bytes
 * >= batch * info.workspace_bytes, may be NULL when that is 0.
 * Kernels are enqueued on `stream` (a hipStream_t); the call does not block.
 * Results are bitwise reproducible run to run for a given plan.
 */
ffa_status ffa_fwd(ffa_plan_t plan, const void* d_meta, int32_t batch,
                   const void* q, int64_t q_sb, int64_t q_st, int64_t q_sh,
                   const void* k, int64_t k_sb, int64_t k_st, int64_t k_sh,
                   const void* v, int64_t v_sb, int64_t v_st, int64_t v_sh,
                   void* out, int64_t o_sb, int64_t o_st, int64_t o_sh,
                   float* lse, int64_t l_sb, int64_t l_st, int64_t l_sh,
                   float softmax_scale, const ffa_attn_extras* extras,
                   void* d_workspace, size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): ffa_fwd with
 * the same arguments and results, except that a plan's split-K partials go to
 * a library-owned device array of FFA_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU
 * instead of a caller workspace.  Nothing is allocated: the array is part of
 * the library's device image, held from its load until the process ends, and
 * its address is looked up once per device (hipGetSymbolAddress) on the first
 * call that needs it, with the stream's device current.  A plan whose
 * batch * info.workspace_bytes exceeds the array is rejected with
 * FFA_ERR_WORKSPACE before anything is enqueued.  Every call on one GPU shares
 * that GPU's array and the array keeps the last call's contents (every slot a
 * call reads is written by the same call first, so nothing needs clearing);
 * calls that overlap in time on one GPU (other streams, other threads) race on
 * it and must be serialised by the caller.
 */
#define FFA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
ffa_status ffa_fwd_noalloc(ffa_plan_t plan, const void* d_meta, int32_t batch,
                           const void* q, int64_t q_sb, int64_t q_st, int64_t q_sh,
                           const void* k, int64_t k_sb, int64_t k_st, int64_t k_sh,
                           const void* v, int64_t v_sb, int64_t v_st, int64_t v_sh,
                           void* out, int64_t o_sb, int64_t o_st, int64_t o_sh,
                           float* lse, int64_t l_sb, int64_t l_st, int64_t l_sh,
                           float softmax_scale, const ffa_attn_extras* extras, void* stream);

/*
 * The merge step of a split plan on its own (FlagAttention user guide,
 * "Split-KV and paged attention": a second kernel merges the partial results
 * with a global logsumexp): for every split (row, head),
 *   lse = ln sum_c exp(lse_c),  out = sum_c exp(lse_c - lse) out_c
 * over the float32 partials (out_c, lse_c) that the main kernel of ffa_fwd left
 * in d_workspace, in a fixed chunk order; sink logits in extras join the sum as
 * terms without a value.  ffa_fwd already runs this step; calling ffa_combine
 * after it on the same workspace rewrites the split rows' out and lse with the
 * same values (this is how the merge is timed alone).  Only split rows are
 * written; a plan without split rows enqueues nothing.  Arguments, strides and
 * error rules are those of ffa_fwd (d_workspace must hold the partials of an
 * ffa_fwd call with the same plan, batch and sink logits).
 */
ffa_status ffa_combine(ffa_plan_t plan, const void* d_meta, int32_t batch,
                       void* out, int64_t o_sb, int64_t o_st, int64_t o_sh,
                       float* lse, int64_t l_sb, int64_t l_st, int64_t l_sh,
                       const ffa_attn_extras* extras, const void* d_workspace, size_t workspace_bytes,
                       void* stream);

/*
 * Backward.  The derivative of the operation above for a loss L with
 * dout = dL/dout (the softmax Jacobian; both pages present the forward as a
 * differentiable training operator: MagiAttention quickstart, "Single-GPU
 * Flex-Flash-Attention"; FlagAttention user guide, "FlashAttention"): with
 * P[i,h,j] = exp(s_ij - lse[i,h]) on visible pairs (0 elsewhere),
 *   dv[j,g] = sum_{h in g} sum_i P dout[i,h]
 *   dS      = P * (dout[i,h] . v[j,g] - sum_d dout[i,h,d] out[i,h,d])
 *   dq[i,h] = softmax_scale * sum_j dS k[j,g]
 *   dk[j,g] = softmax_scale * sum_{h in g} sum_i dS q[i,h]
 * q, k, v, out, lse are the forward's inputs and outputs (out bf16, lse fp32
 * as ffa_fwd wrote them, -inf for rows that see nothing); dout, dq, dk, dv are
 * bf16 with the layout and stride rules of q (dout, dq) and k (dk, dv).
 * Every element of dq, dk and dv is written (zero where nothing is visible).
 * Accumulation is fp32; results are bitwise reproducible (no atomics).
 * d_workspace: >= batch * info.bwd_workspace_bytes bytes of device memory
 * (fp32 per head and row: the lse in the kernels' own scaling and -rowsum(dout * out);
 * its contents are scratch between the call's kernels, not a result).  The plan must
 * have been built with FFA_PLAN_BACKWARD (FFA_ERR_ARG otherwise); token
 * strides of q, k, v and dout must be below 2^24 elements.  extras: the same
 * sink / softcap as the forward call (dS is multiplied by 1 - tanh^2 under a
 * softcap; d sink = -sum_i exp(sink - lse) * rowsum(dout * out)).
 */
ffa_status ffa_bwd(ffa_plan_t plan, const void* d_meta, int32_t batch,
                   const void* q, int64_t q_sb, int64_t q_st, int64_t q_sh,
                   const void* k, int64_t k_sb, int64_t k_st, int64_t k_sh,
                   const void* v, int64_t v_sb, int64_t v_st, int64_t v_sh,
                   const void* out, int64_t o_sb, int64_t o_st, int64_t o_sh,
                   const float* lse, int64_t l_sb, int64_t l_st, int64_t l_sh,
                   const void* dout, int64_t d_sb, int64_t d_st, int64_t d_sh,
                   void* dq, int64_t dq_sb, int64_t dq_st, int64_t dq_sh,
                   void* dk, int64_t dk_sb, int64_t dk_st, int64_t dk_sh,
                   void* dv, int64_t dv_sb, int64_t dv_st, int64_t dv_sh,
                   float softmax_scale, const ffa_attn_extras* extras,
                   void* d_workspace, size_t workspace_bytes, void* stream);

/*
 * FlagAttention's total attention (user guide, "FlashAttention": `total`
 * [B, Hq, N], the attention probabilities summed over the query axis):
 *   total[b, j, h] = sum_i P[i, h, j],  P = exp(s_ij - lse[i,h]) on visible pairs
 * from q, k and the forward's lse (and the same extras: softcap changes s, sinks
 * only enter through lse).  fp32, element (b, key j, head h) at
 * total[b*t_sb + j*t_st + h*t_sh]; every element is written (0 for keys no
 * query sees).  Needs a plan with FFA_PLAN_BACKWARD (it walks the key-major
 * worklist) and the backward's workspace (>= batch * info.bwd_workspace_bytes).
 */
ffa_status ffa_total_attention(ffa_plan_t plan, const void* d_meta, int32_t batch,
                               const void* q, int64_t q_sb, int64_t q_st, int64_t q_sh,
                               const void* k, int64_t k_sb, int64_t k_st, int64_t k_sh,
                               const float* lse, int64_t l_sb, int64_t l_st, int64_t l_sh,
                               float* total, int64_t t_sb, int64_t t_st, int64_t t_sh,
                               float softmax_scale, const ffa_attn_extras* extras,
                               void* d_workspace, size_t workspace_bytes, void* stream);

void ffa_plan_destroy(ffa_plan_t plan);
const char* ffa_status_string(ffa_status status);
const char* ffa_last_error(void);
int32_t ffa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FFA_H */
