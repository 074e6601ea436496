/*
 * jfa.h — C ABI of the MI355X (gfx950) jagged flash attention library.
 *
 * The library computes attention directly on jagged tensors: packed values plus offsets, no
 * padding (vibekk.com GEM page, FAQ entry on jagged tensors; aihot.vn GEM page, section "Jagged
 * Sequence Flash Attention", which asks for custom attention bias, asymmetric query vs key/value
 * lengths and an efficient backward pass). The score activation is either online softmax
 * (FlashAttention) or a pointwise SiLU / GELU-tanh with the result divided by the sequence's key
 * count (aihot.vn GEM page, section "Generalized Dot-Product Attention (GDPA)": two matrix
 * products with a pointwise activation between them in place of softmax). Masking excludes
 * pairs exactly; on the device it is done by subtracting infinity from the score (kerneldigest.dev
 * page, section "Arquitectura del Sistema").
 *
 * For sequence b with Lq = q_off[b+1]-q_off[b] queries and Lkv = kv_off[b+1]-kv_off[b] keys, head h,
 * query i < Lq, key j < Lkv:
 *   s_ij = scale * <q_i, k_j> + beta_h(i, j),  beta = 0 | c_h | T[h][bucket(|i - j|)]
 *   visible(i, j) = base && window && block
 *     base   = (mask == NONE) || (j <= i)     (causal with Lq > Lkv: rows i >= Lkv see every key)
 *     window = (W == 0) || (i - j < W && (mask == CAUSAL || j - i < W))
 *     block  = (Bk == 0) || (i / Bk == j / Bk)
 *   softmax: out_i = sum_j P_ij v_j with P the softmax of s_i over visible j; lse_i = ln sum exp
 *            (a row with no visible key gives out_i = 0 and lse_i = -inf)
 *   GDPA:    out_i = (1 / Lkv) * sum_{visible j} act(s_ij) v_j,  act = SiLU | GELU (tanh form)
 *   bucket(d) = d for d < 16, else min(63, 16 + 4 (e - 4) + ((d >> (e - 2)) & 3)), e = floor(log2 d)
 *
 * Layouts (all row-major, contiguous, device memory unless named *_host):
 *   q, out, dout, dq : [Tq,  H, D]   Tq  = q_off[B]
 *   k, v, dk, dv     : [Tkv, H, D]   Tkv = kv_off[B]
 *   element type bf16; out may be fp32 (out_dtype), dq/dk/dv may be fp32 (grad_dtype)
 *   lse              : [H, Tq] fp32 (natural log)
 *   bias             : fp32 [H] (HEAD_SCALAR) or [H, 64] (REL_BUCKET64)
 *   offsets          : int32 [B+1], offsets[0] == 0, non-decreasing; empty sequences are legal
 *   Every tensor pointer must be 16-byte aligned (JFA_ERR_MISALIGNED otherwise).
 *
 * Ownership: the caller owns every tensor, both copies of the offsets and the workspace. A plan
 * owns its host schedule and its device copy of the work lists and returns them in
 * jfa_plan_destroy. A plan is immutable after jfa_plan and may be used on several streams at
 * once when each call gets its own workspace. jfa_forward / jfa_backward allocate nothing, never
 * synchronise the stream, and only enqueue kernels on the stream they are given.
 *
 * Limits: a (sequence, head) slice is addressed with 32-bit offsets, so (L + 128) * H * D must not
 * exceed 2^30 for every sequence, L = max(Lq, Lkv) (JFA_ERR_BAD_SHAPE otherwise; e.g. H = 8,
 * D = 128 allows L up to 1,048,448). The scale must be finite and >= 0.
 *
 * Errors: every call returns a jfa_status; nothing aborts and no exception crosses the ABI. All
 * argument checks run before the first launch, so on error no output has been touched.
 * jfa_last_error() gives a thread-local description of the last failure. A launch failure is
 * JFA_ERR_HIP; a device fault shows at the caller's next synchronisation.
 */
#ifndef JFA_H
#define JFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* jfa_stream_t; /* a hipStream_t; NULL is the default stream */
typedef struct jfa_plan_s* jfa_plan_t;     /* opaque; created by jfa_plan, freed by jfa_plan_destroy */

typedef enum {
  JFA_OK = 0,
  JFA_ERR_NULL_ARG = 1,     /* a required pointer is NULL */
  JFA_ERR_BAD_OFFSETS = 2,  /* offsets[0] != 0, decreasing offsets, or a total beyond int32 */
  JFA_ERR_BAD_SHAPE = 3,    /* B < 1, H < 1, D not 64/128, causal with some Lq < Lkv, shared
                               queries with unequal Lq,
                               window or block < 0, a sequence beyond the 32-bit slice limit */
  JFA_ERR_UNSUPPORTED = 4,  /* enum out of range, negative or non-finite scale, or a feature this
                               build does not provide */
  JFA_ERR_MISALIGNED = 5,   /* a tensor pointer is not 16-byte aligned */
  JFA_ERR_WORKSPACE = 6,    /* workspace smaller than jfa_workspace_bytes reports */
  JFA_ERR_HIP = 7,          /* a HIP runtime call or launch failed */
  JFA_ERR_HOST_ONLY = 8     /* the plan was built with JFA_PLAN_HOST_ONLY and cannot launch */
} jfa_status;

typedef enum { JFA_MASK_NONE = 0, JFA_MASK_CAUSAL = 1 } jfa_mask;
typedef enum { JFA_ACT_SOFTMAX = 0, JFA_ACT_SILU = 1, JFA_ACT_GELU_TANH = 2 } jfa_act;
typedef enum { JFA_BIAS_NONE = 0, JFA_BIAS_HEAD_SCALAR = 1, JFA_BIAS_REL_BUCKET64 = 2 } jfa_bias;
typedef enum { JFA_BF16 = 0, JFA_F32 = 1 } jfa_dtype;

/* jfa_problem.flags */
#define JFA_PLAN_HOST_ONLY 0x1u /* build the schedule on the host only: no HIP call, no launches */
#define JFA_PLAN_NO_SPLIT 0x2u  /* never split a work item into key (or query) ranges */
/* Shared queries: one set of Ls query rows serves every sequence, as the learned seed queries of
 * pooling by multihead attention (PMA), which the pages list beside self- and cross-attention as
 * the same two-product structure (aihot.vn GEM page, "Generalized Dot-Product Attention (GDPA)").
 * Every Lq_b must equal Ls (q_offsets_host = b * Ls); q and dq are [Ls, H, D] and are read (resp.
 * written) once for all sequences, with no copy per sequence; out, lse and dout stay per sequence
 * ([B * Ls, H, D], [H, B * Ls]). dq is the sum over sequences of each sequence's query gradient,
 * taken in a fixed order (deterministic). */
#define JFA_PLAN_SHARED_Q 0x4u
/* MXFP8 forward pass (kerneldigest.dev page, "Arquitectura del Sistema": attention in MXFP8 with
 * block quantisation and online conversion of P). jfa_forward quantises Q and K (blocks of 32
 * features of a row), V (blocks of 32 consecutive keys of a feature, from the sequence's first key)
 * into the forward workspace and computes both products on FP8 E4M3 values with E8M0 block scales
 * (scale 2^(floor(log2 amax) - 8), elements rounded to nearest even, saturated at 448), fp32
 * accumulation. P is quantised the same way per row in blocks of 32 consecutive keys, taken
 * against an integer running maximum (in log2 units) so that rescaling commutes with the
 * quantisation: out_i = sum_j P^_ij V^_j / sum_j P~_ij with P~ = 2^(s log2(e) - M_i); lse is the
 * log-sum-exp of the scores from the quantised Q and K. Softmax, head dim 128, no shared queries;
 * forward only (jfa_backward refuses the plan with JFA_ERR_UNSUPPORTED). The inputs and outputs
 * keep their bf16 / fp32 layouts. */
#define JFA_PLAN_MXFP8 0x8u

typedef struct {
  int32_t num_seqs;               /* B >= 1 */
  int32_t num_heads;              /* H >= 1 */
  int32_t head_dim;               /* D in {64, 128} */
  const int32_t* q_offsets_host;  /* [B+1] host array, read during jfa_plan only */
  const int32_t* kv_offsets_host; /* [B+1] host array, read during jfa_plan only */
  int32_t mask;                   /* jfa_mask; causal requires Lq >= Lkv for every sequence: rows
                                     i >= Lkv are target rows that see every key (fused self + target
                                     pass, itsolotime.com IKBO page, table of contents section 3.3) */
  int32_t act;                    /* jfa_act */
  int32_t bias;                   /* jfa_bias */
  float scale;                    /* score scale; 0 means 1/sqrt(D) */
  int32_t out_dtype;              /* jfa_dtype of out */
  int32_t grad_dtype;             /* jfa_dtype of dq, dk, dv */
  int32_t num_slots;              /* concurrent workgroups the split rule balances for; 0: from the device
                                     (CUs x resident workgroups), or 512 for a host-only plan */
  uint32_t flags;                 /* JFA_PLAN_* */
  /* Optional long-sequence limits on visibility, 0 = off (aihot.vn GEM page, "BlockAttention":
   * sliding-window attention restricted to neighbouring events, whose kernel skips the tiles
   * outside the window; vibekk.com GEM page, section on moving from padding to jagged kernels,
   * and kerneldigest.dev page, "Arquitectura del Sistema": block attention over fixed blocks).
   * window W: a query sees keys fewer than W positions before it (and, without the causal mask,
   * fewer than W after it). block Bk: a query sees only keys of its own block of Bk positions,
   * with the base mask kept inside the block. The work lists hold only the tiles that contain a
   * visible pair. GDPA still divides by the sequence's full key count. */
  int32_t window;                 /* W >= 0 */
  int32_t block;                  /* Bk >= 0 */
} jfa_problem;

/* Validate the problem, build the longest-first work lists (jagged tile scheduler) and, unless
 * JFA_PLAN_HOST_ONLY, upload them to device memory with an asynchronous copy on `stream`.
 * The pages place the cost that remains once padding is gone in tile scheduling and load balance
 * (vibekk.com GEM page, section on moving from padding to jagged kernels; aihot.vn GEM page,
 * "Jagged Sequence Flash Attention": compute units idle when short sequences finish early), and
 * offsets change with every batch, so planning never waits for the device: the records are written
 * into pinned host memory and copied asynchronously, and the pinned and device buffers come from
 * a process-wide cache that hands a buffer out again only after the device has finished with it
 * (the upload and the last pass on every stream that used the plan). The host offsets are read
 * during this call only. On error *plan_out is NULL and nothing was enqueued. */
jfa_status jfa_plan(const jfa_problem* problem, jfa_stream_t stream, jfa_plan_t* plan_out);

/* Device bytes of workspace each pass needs (0 when nothing is split and no scratch is used).
 * At head dim 128 the backward workspace always holds the dK/dV kernel's work-queue counters
 * (256 bytes): that kernel keeps as many workgroups as the GPU holds at once and hands them the
 * work items through per-XCD queues; the backward pass zeroes the counters itself before the
 * kernel runs. Either pointer may be NULL. */
jfa_status jfa_workspace_bytes(jfa_plan_t plan, size_t* fwd_bytes, size_t* bwd_bytes);

/* Forward pass: out (and lse for softmax) of the attention defined above, computed straight on
 * the jagged values with no padded tensor (aihot.vn GEM page, "Jagged Sequence Flash Attention";
 * "Generalized Dot-Product Attention (GDPA)" for the pointwise activations). `bias` may be NULL
 * only without bias; `lse` may be NULL only for GDPA (it is not defined there). `q_offsets` /
 * `kv_offsets` are optional device copies of the offsets given to jfa_plan (NULL allowed): the
 * kernels take every sequence's offsets from the plan's work records, and with JFA_DEBUG=1 in the
 * environment the copies are read back and compared with the plan (JFA_ERR_BAD_OFFSETS on a
 * mismatch; a synchronising check). `workspace` may be NULL when its size is 0. */
jfa_status jfa_forward(jfa_plan_t plan, const void* q, const void* k, const void* v,
                       const int32_t* q_offsets, const int32_t* kv_offsets, const float* bias,
                       void* out, float* lse, void* workspace, size_t workspace_bytes,
                       jfa_stream_t stream);

/* Backward pass: gradients of <out, dout> with respect to q, k and v, and optionally the bias.
 * `out` and `lse` are the forward results (softmax only; they may be NULL for GDPA). The optional
 * device offsets are treated as in jfa_forward.
 * `dbias` is NULL (no bias gradient) or a device fp32 array of the bias shape, [H] for
 * JFA_BIAS_HEAD_SCALAR and [H][64] for JFA_BIAS_REL_BUCKET64 (16-byte aligned), that receives
 * dL/dbias: for the table, entry (h, u) is the sum of dS over the visible scores of head h whose
 * relative distance |i - j| falls in bucket u; for the scalar, the sum of dS over all visible
 * scores of head h (exactly 0 under softmax, which is invariant to a per-row shift). It is
 * overwritten, not accumulated, and does not depend on launch timing (fixed-point sums).
 * Requesting it without a bias returns JFA_ERR_UNSUPPORTED. The pages ask for custom attention
 * bias together with an efficient backward pass (aihot.vn GEM page, section "Jagged Sequence
 * Flash Attention"); a learned bias needs this gradient to train. */
jfa_status jfa_backward(jfa_plan_t plan, const void* q, const void* k, const void* v,
                        const int32_t* q_offsets, const int32_t* kv_offsets, const float* bias,
                        const void* out, const float* lse, const void* dout, void* dq, void* dk,
                        void* dv, float* dbias, void* workspace, size_t workspace_bytes,
                        jfa_stream_t stream);

/* Allocation-free backward pass, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation. Same arguments and results
 * as jfa_backward without the workspace: the library uses a static device array of
 * JFA_NOALLOC_SCRATCH_BYTES per GPU (held until the process ends) instead, and calls no allocating
 * routine. A plan whose backward workspace (jfa_workspace_bytes) exceeds that size is refused with
 * JFA_ERR_WORKSPACE before any launch. All calls on one GPU share its array: calls that overlap in
 * time (several streams or threads) race and must be ordered by the caller. No per-kernel timing
 * is recorded, and the plan must stay alive until the work this call enqueued has finished (the
 * call records no event for the plan's buffer cache). */
#define JFA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
jfa_status jfa_backward_noalloc(jfa_plan_t plan, const void* q, const void* k, const void* v,
                                const int32_t* q_offsets, const int32_t* kv_offsets, const float* bias,
                                const void* out, const float* lse, const void* dout, void* dq, void* dk,
                                void* dv, float* dbias, jfa_stream_t stream);

/* Work lists, for inspection and tests. `which`: 0 forward items, 1 forward split groups,
 * 2 dQ items, 3 dQ split groups, 4 dK/dV items, 5 dK/dV split groups (longest first), and
 * 6 forward, 7 dQ, 8 dK/dV items in dispatch order: the order in which the kernels' workgroups
 * take them. Workgroup p runs on XCD p % 8, so the dispatch order keeps all items of a
 * (sequence, head) group on one XCD's L2 (groups assigned longest first to the least-loaded XCD;
 * each XCD takes its groups longest first, a group's items together in list order). Items are 6
 * int32 each (b, h, tile, lo, hi, slot): query-tile lists own query tile `tile` and cover key
 * tiles [lo, hi); the dK/dV list owns key tile `tile` and covers query tiles [lo, hi); slot is
 * the partial-result slot of a split piece or -1. Groups are 5 int32 each (b, h, tile, slot0,
 * R). The pages place the post-padding bottleneck in tile scheduling and load balance (vibekk.com
 * GEM page, section on moving from padding to jagged kernels). Writes min(count, cap) records
 * and sets *count to the total number of records. */
jfa_status jfa_plan_schedule(jfa_plan_t plan, int32_t which, int32_t* out, size_t cap, size_t* count);

/* Tile geometry and slot counts the plan used: writes up to `n` of
 * {fwd BM, fwd BN, dq BM, dq BN, dkdv BM, dkdv BN, fwd slots, dq slots, dkdv slots, fused backward}
 * (the last is 1 when the backward runs as one fused pass over the dQ items: every sequence has at
 * most 64 queries, head_dim 128, no window or block limit, and every sequence with keys has
 * queries). */
jfa_status jfa_plan_info(jfa_plan_t plan, int32_t* info, size_t n);

/* Per-kernel timing with HIP events recorded around every launch of this plan (for
 * measurement; adds two event records per launch while on). Kernel ids: 0 forward,
 * 1 forward combine, 3 dK/dV, 4 dQ (which also computes rowsum(dO * O) for dK/dV), 5 backward
 * partial reduce, 6 bias-gradient clear and finish, 7 MXFP8 quantisation, 8 fused backward of
 * short query sets (2 is not used).
 * jfa_timing_read waits for the recorded events and returns their summed time and count;
 * jfa_timing_enable(plan, 1) also clears previous records and reuses the plan's events, which are
 * created on first use and record without a system-scope memory fence (timing only). Not thread
 * safe. */
jfa_status jfa_timing_enable(jfa_plan_t plan, int32_t enable);
jfa_status jfa_timing_read(jfa_plan_t plan, int32_t kernel, float* total_ms, int32_t* launches);

void jfa_plan_destroy(jfa_plan_t plan);
const char* jfa_status_string(jfa_status status);
const char* jfa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* JFA_H */
