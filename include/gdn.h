/*
 * gdn.h -- C ABI of the MI355X (gfx950) Gated DeltaNet layer core.
 *
 * The layer core, in order ("System Design" (project_6 SYSTEM_DESIGN.md),
 * sections "Runtime Data Flow" and "GDN Kernel Dispatch Detail"):
 *   1. a depthwise causal conv1d over the projected q|k|v channels, each sequence
 *      continuing from its own conv state;
 *   2. L2 normalisation of every q and k head vector;
 *   3. the gated delta rule over a fixed-size fp32 state per sequence and v-head,
 *        S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t,
 *      run either as a chunked prefill over packed ragged sequences (the chunked
 *      prefill kernel of that section takes (q, k, v, g, beta, state) and updates the
 *      temporal state) or as a batched single-token decode.
 * The decode batches over m slots, each reached through a device array of u64
 * per-slot state pointers with the slot index on the grid ("serve: Qwen3.5 on CUDA
 * never batches concurrent requests", aprender #5279, comment "Phase plan", phase
 * P5); conv and delta-rule kernels carry a sequence dimension with per-sequence
 * conv and SSM state (same issue, comment "Where concurrency is lost", item 3).
 *
 * Conventions for every entry point
 *  - Every pointer argument except `dims`, `bytes` and `stream` is a DEVICE pointer
 *    (HIP global memory) owned by the caller. The library allocates nothing, keeps
 *    no device state, and never reads device memory from the host.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream). Calls on different streams are thread-safe.
 *  - Argument checks are host-only and O(1); a failed check returns a status,
 *    launches nothing and sets the thread-local text of gdn_last_error(). A failed
 *    launch returns GDN_ERR_HIP with the HIP error text.
 *  - Strides are in ELEMENTS of the pointed-to type.
 *  - Unchecked preconditions (undefined behaviour when violated): device pointers
 *    are valid for the stated extents; per-slot pointers within one call are
 *    distinct; outputs alias no input; g <= 0 and finite; beta in [0, 1];
 *    cu_seqlens is non-decreasing from 0 to total_tokens.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 6

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_NULL = 1,        /* a required pointer is NULL */
  GDN_ERR_SHAPE = 2,       /* a count, size or stride is out of range or inconsistent */
  GDN_ERR_DTYPE = 3,       /* an enumerated field holds an unknown value (dtype, activation,
                              precision policy, prefill form, or a 0/1 switch) */
  GDN_ERR_ALIGN = 4,       /* a pointer or stride breaks the 16-byte alignment rule */
  GDN_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than gdn_prefill_workspace_size */
  GDN_ERR_UNSUPPORTED = 6, /* valid but not built: head dim, chunk size or conv width */
  GDN_ERR_HIP = 7          /* the HIP runtime failed the launch */
} gdn_status;

typedef enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* Activation applied to the conv output. The pages name the conv only as a depthwise
 * causal Conv1d, so the default is the identity; SiLU is offered as an option. */
typedef enum gdn_activation { GDN_ACT_NONE = 0, GDN_ACT_SILU = 1 } gdn_activation;

/* Matrix-core precision of the prefill contractions (decode is plain fp32 FMA).
 *  AUTO   : FP32 when in_dtype is F32, BF16X3 when in_dtype is BF16.
 *  FP32   : v_mfma_f32_16x16x4_f32, fp32 operands.
 *  BF16X3 : every fp32 operand split as hi + lo (two bf16 values); each product is
 *           hi*hi + hi*lo + lo*hi on v_mfma_f32_16x16x32_bf16 with fp32 accumulation
 *           ("bf16x3", Henry, Tang & Heinecke, ARITH 2019). */
typedef enum gdn_mma { GDN_MMA_AUTO = 0, GDN_MMA_FP32 = 1, GDN_MMA_BF16X3 = 2 } gdn_mma;

/* How gdn_prefill_chunked walks a sequence's chunks.
 *  WHOLE    : one pass over every sequence's chunks in order, the state slice resident.
 *  SEGMENTS : chunk-parallel: a sequence of 8 or more chunks is cut into segments (their
 *             length set by the sequence's own chunk count n: the largest k with
 *             k^2 <= n, within [2, 32]); each segment's affine state map S -> S M + B
 *             is computed in parallel, a scan gives every segment's start state, then all
 *             segments produce their outputs in parallel. More arithmetic, a much shorter
 *             sequential chain: for launches too small to fill the GPU.
 *  AUTO     : SEGMENTS when (d / 16) * Hv * num_seqs is below 256 (fewer state-row
 *             workgroups than MI355X CUs), else WHOLE.
 * The two forms agree to rounding; within one form a sequence's result does not depend
 * on what else is packed with it. */
typedef enum gdn_prefill_form { GDN_PREFILL_AUTO = 0, GDN_PREFILL_WHOLE = 1, GDN_PREFILL_SEGMENTS = 2 } gdn_prefill_form;

/* Layer dimensions and options, passed by pointer. struct_size must be
 * sizeof(gdn_dims) as compiled by the caller (lets the struct grow later).
 * Every enumerated field and switch reads 0 as its default, so a zero-filled struct
 * (plus struct_size and the sizes) asks for the layer as defined: identity activation,
 * fp32 input, the automatic precision policy and prefill form, fp32 output and the q/k
 * L2 norm on. Only `scale` has no usable zero (it would zero every output) and is
 * rejected there; gdn_dims_init() fills every field with its default. */
typedef struct gdn_dims {
  int32_t struct_size;
  int32_t num_k_heads; /* Hk >= 1 (q and k heads) */
  int32_t num_v_heads; /* Hv >= 1 with Hv % Hk == 0; v-head j reads k-head j / (Hv / Hk) */
  int32_t head_dim;    /* d = d_k = d_v; built for 32, 64 and 128 */
  int32_t conv_width;  /* K; built for 2, 3 and 4 */
  int32_t chunk_size;  /* prefill chunk length; built for 16, 32 and 64 */
  int32_t activation;  /* gdn_activation */
  int32_t in_dtype;    /* gdn_dtype of x, conv weight, conv bias and conv state */
  int32_t mma;         /* gdn_mma */
  float l2_eps;        /* k^ = k / sqrt(|k|^2 + l2_eps); q^ likewise, then times scale; >= 0 */
  float scale;         /* multiplies q^ (1.0 = no scaling); finite and nonzero */
  int32_t prefill_form; /* gdn_prefill_form */
  int32_t out_dtype;    /* gdn_dtype of o: GDN_F32, or GDN_BF16 = the fp32 result rounded to
                           nearest even (the conv output y is fp32 either way) */
  int32_t qk_l2norm_off; /* 0 (default): q and k L2-normalised in the kernels (the layer's
                            step 2); 1: used as the conv gives them (q still times scale) */
} gdn_dims;

/* ---------------------------------------------------------------------------------
 * gdn_dims_init -- fill *dims with the given head counts and head dim and every other
 * field at its default: struct_size = sizeof(gdn_dims), conv_width 4, chunk_size 64,
 * GDN_ACT_NONE, in_dtype GDN_F32, GDN_MMA_AUTO, l2_eps 1e-6, scale 1.0,
 * GDN_PREFILL_AUTO, out_dtype GDN_F32, qk_l2norm_off 0 (the enumerated fields as a
 * zero-filled struct has them). Host only; checks nothing but dims != NULL (the entry
 * points check the values).
 */
gdn_status gdn_dims_init(gdn_dims* dims, int32_t num_k_heads, int32_t num_v_heads, int32_t head_dim);

/* Conv channel count C = 2*Hk*d + Hv*d, channels ordered [q heads | k heads | v heads]. */

/* ---------------------------------------------------------------------------------
 * gdn_conv_update -- depthwise causal conv1d + conv-state update (both modes).
 *
 * For one sequence with conv state cs (K-1 rows, oldest first) and tokens x_0..x_{L-1},
 * let z = [cs_0 .. cs_{K-2}, x_0 .. x_{L-1}]. Then per channel c
 *     y_t[c] = act( b[c] + sum_{j<K} w[c][j] * z_{t+j}[c] ),     t = 0 .. L-1
 * (w[c][K-1] multiplies the current token) and the new conv state is the last K-1
 * rows of z. ("System Design", "GDN Kernel Dispatch Detail": Conv1d before the L2
 * norm in prefill; conv state update first in the decode branch.)
 *
 *  x          [total_tokens][C] in_dtype, row stride x_stride (>= C).
 *  y          [total_tokens][C] fp32 output, row stride y_stride (>= C). Feed q/k/v
 *             views of y to gdn_prefill_chunked / gdn_decode_batched.
 *  conv_w     [C][K] in_dtype, contiguous.   conv_b: [C] in_dtype, or NULL for no bias.
 *  cu_seqlens prefill mode: device int32 [n+1], sequence s owns tokens
 *             [cu_seqlens[s], cu_seqlens[s+1]); a zero-length sequence keeps its state.
 *             NULL selects decode mode: token i belongs to slot i and total_tokens == n.
 *  conv_state_ptrs  device u64 [n]; entry s points at sequence/slot s's conv state,
 *             [K-1][C] in_dtype contiguous, 16-byte aligned, read and updated in place.
 *             Decode mode only: an entry of 0 marks an inactive slot (its y row is left
 *             untouched and nothing is read for it).
 *  Prefill mode launches two kernels in stream order (outputs, then state commit), so
 *  the in-place state update never races with a read of the old state.
 *  Alignment: x, y 16-byte aligned; x_stride * elt_size and y_stride * 4 multiples of 16.
 */
gdn_status gdn_conv_update(const gdn_dims* dims, const void* x, int64_t x_stride, float* y,
                           int64_t y_stride, const void* conv_w, const void* conv_b,
                           const int32_t* cu_seqlens, const uint64_t* conv_state_ptrs, int32_t n,
                           int32_t total_tokens, void* stream);

/* ---------------------------------------------------------------------------------
 * gdn_prefill_workspace_size -- bytes of device workspace gdn_prefill_chunked needs
 * for at most num_seqs sequences and total_tokens tokens (written to *bytes).
 */
gdn_status gdn_prefill_workspace_size(const gdn_dims* dims, int32_t num_seqs, int32_t total_tokens,
                                      size_t* bytes);

/* ---------------------------------------------------------------------------------
 * gdn_prefill_chunked -- L2 norm + gated delta rule over packed ragged sequences,
 * chunked ("System Design", "GDN Kernel Dispatch Detail": the prefill branch runs a
 * chunked gated-delta-rule kernel on (q, k, v, g, beta, state), then updates the
 * temporal state).
 *
 * Chunks of chunk_size tokens start at each sequence's own first token, so within one
 * dims->prefill_form the arithmetic of a sequence does not depend on what else is packed
 * with it (AUTO picks the form from Hv, d and num_seqs: see gdn_prefill_form).
 *
 *  q, k       [total_tokens][Hk*d] fp32 (raw conv output; normalised inside), row
 *             strides q_stride, k_stride.   v: [total_tokens][Hv*d] fp32, stride v_stride.
 *  g, beta    [total_tokens][Hv] fp32 contiguous: log-decay (<= 0) and write strength.
 *  o          [total_tokens][Hv][d] contiguous output in dims->out_dtype.
 *  cu_seqlens device int32 [num_seqs+1].
 *  state_ptrs device u64 [num_seqs]; entry s points at sequence s's state, fp32
 *             [Hv][d_v][d_k] (d_k contiguous), 16-byte aligned; read as the initial
 *             state and overwritten with the final state. Zero-length sequences keep it.
 *  workspace  device scratch of at least gdn_prefill_workspace_size(dims, num_seqs,
 *             total_tokens) bytes, 256-byte aligned; contents on entry are ignored.
 *  Alignment: q, k, v 16-byte aligned, strides multiples of 4 elements.
 */
gdn_status gdn_prefill_chunked(const gdn_dims* dims, const float* q, int64_t q_stride, const float* k,
                               int64_t k_stride, const float* v, int64_t v_stride, const float* g,
                               const float* beta, void* o, const int32_t* cu_seqlens, int32_t num_seqs,
                               int32_t total_tokens, const uint64_t* state_ptrs, void* workspace,
                               size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * gdn_prefill_fused_workspace_size -- bytes of device workspace gdn_prefill_fused needs
 * for at most num_seqs sequences and total_tokens tokens (written to *bytes): the
 * gdn_prefill_chunked workspace plus the v part of the conv output (total_tokens x Hv*d
 * fp32).
 */
gdn_status gdn_prefill_fused_workspace_size(const gdn_dims* dims, int32_t num_seqs, int32_t total_tokens,
                                            size_t* bytes);

/* ---------------------------------------------------------------------------------
 * gdn_prefill_fused -- the prefill of a layer in one call: gdn_conv_update in prefill
 * mode followed by gdn_prefill_chunked on the q/k/v views of its output ("System
 * Design", "GDN Kernel Dispatch Detail": conv with the per-sequence conv state, then the
 * chunked gated delta rule and the state update), without writing the conv output to
 * memory: the intra-chunk kernel convolves its chunk's q and k channels from x itself, and
 * the inter-chunk kernel the v channels it needs (the same per-channel arithmetic as the
 * conv kernel); with the chunk-parallel form or chunks other than 64 tokens the v part of
 * the conv output goes through the workspace instead. o, the recurrent states and the conv
 * states come out bit-identical to those two calls in sequence.
 *
 *  x          [total_tokens][C] in dims->in_dtype, row stride x_stride (C = (2 Hk + Hv) d,
 *             channels ordered q | k | v as for gdn_conv_update).
 *  conv_w     [C][conv_width], conv_b [C] or NULL, in dims->in_dtype.
 *  g, beta, o, cu_seqlens, num_seqs, total_tokens, state_ptrs: as for gdn_prefill_chunked.
 *  conv_state_ptrs device u64 [num_seqs]; entry s points at sequence s's conv state,
 *             [conv_width-1][C] in dims->in_dtype: read before, and replaced by, the last
 *             conv_width-1 rows of the sequence's conv input (as gdn_conv_update).
 *  workspace  device scratch of at least gdn_prefill_fused_workspace_size(dims, num_seqs,
 *             total_tokens) bytes, 256-byte aligned; contents on entry are ignored.
 *  Alignment: x, conv_w, conv_b 16-byte aligned, x_stride a multiple of 16 bytes.
 *  Errors: as the two calls (GDN_ERR_NULL, _SHAPE, _ALIGN, _WORKSPACE); nothing is
 *  launched unless every check passes.
 */
gdn_status gdn_prefill_fused(const gdn_dims* dims, const void* x, int64_t x_stride, const void* conv_w,
                             const void* conv_b, const float* g, const float* beta, void* o,
                             const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                             const uint64_t* state_ptrs, const uint64_t* conv_state_ptrs, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * gdn_prefill_fused_static -- gdn_prefill_fused with no workspace argument, for callers
 * that cannot allocate device memory (code being captured into a HIP graph, serving loops
 * that may not call hipMalloc, harnesses that forbid it). The workspace is the library's
 * own file-scope device array of 64 MiB (GDN_STATIC_SCRATCH_BYTES), one per GPU it runs on,
 * held until the process ends; this entry point itself allocates nothing. The same
 * kernels run on the same bits as gdn_prefill_fused.
 *
 *  Arguments as gdn_prefill_fused, without workspace and workspace_bytes.
 *  Limit: gdn_prefill_fused_workspace_size(dims, num_seqs, total_tokens) must not exceed
 *  GDN_STATIC_SCRATCH_BYTES (about 1280 tokens of a 16 q/k-head, 32 v-head, d = 128
 *  layer); above it the call returns GDN_ERR_WORKSPACE and launches nothing.
 *  Every call on one GPU uses that GPU's single array: calls on one GPU must not overlap
 *  in time (one stream, or streams ordered by events); overlapping calls race. Nothing
 *  in the array needs clearing between calls. The GPU is the one `stream` belongs to
 *  (the current device for the null stream).
 */
#define GDN_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
gdn_status gdn_prefill_fused_static(const gdn_dims* dims, const void* x, int64_t x_stride, const void* conv_w,
                                    const void* conv_b, const float* g, const float* beta, void* o,
                                    const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                                    const uint64_t* state_ptrs, const uint64_t* conv_state_ptrs, void* stream);

/* ---------------------------------------------------------------------------------
 * gdn_decode_batched -- one token for each of m slots: L2 norm + one step of the gated
 * delta rule on each slot's state, in place ("System Design", "GDN Kernel Dispatch
 * Detail", decode branch: decay the temporal state and write the delta, then
 * multiply the query by the state; aprender #5279, "Phase plan", phase P5: the
 * slot index on the launch grid, one 64-bit state address per slot in a device array).
 *
 * Each slot's result is the same bits whatever m is and whatever other slots are in
 * the call: no reduction crosses slots and every reduction has a fixed order.
 *
 *  q, k       [m][Hk*d] fp32, row strides q_stride, k_stride (raw; normalised inside).
 *  v          [m][Hv*d] fp32, row stride v_stride.
 *  g, beta    [m][Hv] fp32 contiguous.
 *  o          [m][Hv][d] contiguous output in dims->out_dtype.
 *  state_ptrs device u64 [m]; entry i points at slot i's fp32 [Hv][d_v][d_k] state
 *             (16-byte aligned), updated in place. An entry of 0 marks an inactive
 *             slot: nothing is read or written for it (its o rows are left untouched).
 *  Alignment: q, k, v 16-byte aligned, strides multiples of 4 elements.
 */
gdn_status gdn_decode_batched(const gdn_dims* dims, const float* q, int64_t q_stride, const float* k,
                              int64_t k_stride, const float* v, int64_t v_stride, const float* g,
                              const float* beta, void* o, const uint64_t* state_ptrs, int32_t m,
                              void* stream);

/* ---------------------------------------------------------------------------------
 * gdn_decode_fused -- the whole decode step of a layer in one launch: the conv of
 * gdn_conv_update in decode mode (token i <-> slot i), its conv-state commit, then
 * gdn_decode_batched on the conv output, which never leaves the chip. o, the states
 * and the conv states come out bit-identical to those two calls in sequence. (The same
 * passages as gdn_conv_update and gdn_decode_batched: "System Design", "GDN Kernel
 * Dispatch Detail", decode branch: conv state update, then the decay and delta write,
 * then the query against the state.)
 *
 *  x, x_stride, conv_w, conv_b   as gdn_conv_update (x: [m][C] in_dtype).
 *  g, beta, o                    as gdn_decode_batched.
 *  state_ptrs, conv_state_ptrs   device u64 [m]: slot i's recurrent state (updated in
 *             place) and its conv state ([K-1][C] in_dtype, read).
 *  conv_state_out_ptrs  device u64 [m]: where slot i's new conv state goes. NULL, or the
 *             same array as conv_state_ptrs, updates the conv states in place. Any other
 *             array names separate buffers (e.g. a second conv pool the caller alternates
 *             with the first from step to step): the old state is then only read and stays
 *             as it was. Unchecked precondition for that case: no output buffer overlaps a
 *             conv state the call reads, and the outputs are distinct from one another.
 *             Separate buffers let the launch run without cross-workgroup ordering: it is
 *             the faster form; in place, one workgroup per (slot, k-head) reads and
 *             rewrites every conv-state value of its channels itself.
 *  Slot i is inactive (nothing read or written, o rows untouched) when its state pointer,
 *  its conv-state pointer or its output conv-state pointer is 0.
 *  No workspace. Errors: as the two calls; GDN_ERR_UNSUPPORTED when (2 + Hv/Hk) *
 *  head_dim * 4 bytes of conv output exceed 64 KiB.
 *  Alignment: x, conv_w, conv_b 16-byte aligned, x_stride a multiple of 16 bytes.
 */
gdn_status gdn_decode_fused(const gdn_dims* dims, const void* x, int64_t x_stride, const void* conv_w,
                            const void* conv_b, const float* g, const float* beta, void* o,
                            const uint64_t* state_ptrs, const uint64_t* conv_state_ptrs,
                            const uint64_t* conv_state_out_ptrs, int32_t m, void* stream);

/* ---------------------------------------------------------------------------------
 * gdn_slot_pointers -- build a device u64 pointer array from slot indices, on the
 * device: out_ptrs[i] = pool_base + slot_idx[i] * slot_bytes, or 0 when slot_idx[i]
 * is outside [0, pool_slots) (an inactive slot). The slot pool is one caller-owned
 * allocation of pool_slots equal-sized blocks (the "qLLM" page, section "What this is",
 * holds the linear-attention layers' recurrent and conv state in a pool of slots;
 * aprender #5279, "Phase plan", phase P5, gives each layer's kernels one address per
 * slot in a device array).
 *
 *  pool_base  device address of slot 0 (16-byte aligned); slot_bytes: multiple of 16.
 *  slot_idx   device int32 [m].   out_ptrs: device u64 [m].
 */
gdn_status gdn_slot_pointers(uint64_t pool_base, int64_t slot_bytes, int32_t pool_slots,
                             const int32_t* slot_idx, int32_t m, uint64_t* out_ptrs, void* stream);

/* ---------------------------------------------------------------------------------
 * gdn_slot_copy -- snapshot / fork of slots: for i < n, copy the recurrent state at
 * src_state_ptrs[i] to dst_state_ptrs[i] (Hv*d*d fp32 each) and the conv state at
 * src_conv_ptrs[i] to dst_conv_ptrs[i] ((K-1)*C in_dtype each), in one launch per kind.
 * A sequence prefix run once can then seed any number of slots, and a slot can be
 * checkpointed and restored, since the fixed-size state is all the history the layer
 * keeps ("qLLM", "What's still open": prefix caching is off because recurrent state
 * cannot be rebuilt from a cached prefix; aprender #5279, "Where concurrency is lost",
 * item 6, and "Phase plan", P7: per-slot prefix reuse and checkpoints).
 *
 *  src_state_ptrs, dst_state_ptrs  device u64 [n], or both NULL (no state copied).
 *  src_conv_ptrs,  dst_conv_ptrs   device u64 [n], or both NULL (no conv state copied).
 *  An entry whose source or destination is 0 is skipped. All addresses 16-byte aligned.
 *  Unchecked precondition: destination slots are distinct from one another and from
 *  every source (one source may feed several destinations).
 */
gdn_status gdn_slot_copy(const gdn_dims* dims, const uint64_t* src_state_ptrs, const uint64_t* dst_state_ptrs,
                         const uint64_t* src_conv_ptrs, const uint64_t* dst_conv_ptrs, int32_t n, void* stream);

/* Thread-local text describing the last non-OK status returned on this thread. */
const char* gdn_last_error(void);

/* GDN_ABI_VERSION of the built library. */
int32_t gdn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
