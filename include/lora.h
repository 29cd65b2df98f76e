/*
 * lora.h -- C ABI of liblora: the LoRA-linear training hot path on one
 * MI355X (gfx950) GPU.
 *
 * The adapted linear, its backward and its optimizer step follow
 *   - "8. LoRA Fundamentals: The Math and the Architecture Support Matrix"
 *     (Juno documentation), sections "How it works", "The training loop" and
 *     "Training decisions";
 *   - "4.3. Training Guide" (Juno documentation), sections "Gradient
 *     accumulation", "Optimizer", "Schedules", "Dropout", "Gradient clipping";
 *   - "Backward Bug Hunts and Vulkan Tiled GEMM: Pi-Train LoRA SFT
 *     Hardening", section "Bug #1" (the frozen weight is read in its native
 *     layout; no transposed copy is ever made);
 *   - "Multi-LoRA Training Example (fully-async)", section "Design (decoupled
 *     per-adapter optimizers)" (one independent optimizer state per slot).
 *
 * Conventions for every entry point
 *   - Layout is row-major and contiguous: X [T,K], W [N,K] (out x in, the
 *     native layout), A [r,K], B [N,r], U = X~ A^T [T,r], Y, Z, dY [T,N],
 *     dX [T,K].  T = tokens of one chunk, K = in_dim, N = out_dim, r = rank.
 *   - Every pointer except those documented as host pointers is a device
 *     pointer, 16-byte aligned, owned by the caller.  The library never
 *     allocates or frees memory; scratch comes from a caller workspace.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *     enqueued; the one host synchronisation in the library is in
 *     lora_grad_prepare when `h_norm` is not NULL.
 *   - Every argument is validated before anything is enqueued.  On a negative
 *     status no buffer has been touched.  HIP launch failures return
 *     LORA_E_HIP.  No exceptions cross the ABI.  The compute entry points
 *     keep no mutable state between calls, so calls on different streams may
 *     run concurrently as long as their buffers do not overlap.  The launch
 *     profiler is the exception: lora_profile_begin / lora_profile_end keep
 *     one process-wide profile that every launch of the library records
 *     into while it is open (not thread-safe; meant for benchmarks).
 *   - Results are deterministic: every reduction runs in a fixed order (no
 *     floating-point atomics), so equal inputs give bitwise equal outputs.
 */
#ifndef LORA_H
#define LORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lora_status {
  LORA_OK = 0,
  LORA_E_INVALID = -1,    /* NULL pointer, bad enum, out-of-range scalar   */
  LORA_E_SHAPE = -2,      /* non-positive dim, rank > min(K,N) or > 128     */
  LORA_E_DTYPE = -3,      /* unsupported frozen-weight dtype                */
  LORA_E_ALIGN = -4,      /* pointer not 16-byte aligned, or K/N/r/segment
                             sizes not multiples of 4 (K/N of 8 for bf16)  */
  LORA_E_WORKSPACE = -5,  /* workspace NULL or smaller than required        */
  LORA_E_NONFINITE = -6,  /* NaN/Inf gradient: the update is vetoed         */
  LORA_E_HIP = -7         /* a HIP runtime call failed                      */
} lora_status;

/* Frozen-weight (and merge output) element types.  The block-quantized
 * formats hold W for a quantized base model ("8. LoRA Fundamentals", opening
 * paragraph and "Training decisions"; "Backward Bug Hunts and Vulkan Tiled
 * GEMM", "The fix", for the pages' Q4_0, Q4_K and Q6_K frozen paths).  Their
 * arithmetic is that of the GGUF block types of the same names; their
 * storage is planar, one array per field, in one buffer (see
 * lora_qweight_layout):
 *   LORA_Q8_0  qs int8 [N,K]; d fp16 [N,K/32]                 w = d*q
 *   LORA_Q4_0  qs u4 [N,K]; d fp16 [N,K/32]                   w = d*(q-8)
 *   LORA_Q4_K  qs u4 [N,K]; sm u8 [N,K/32][2] = (sc, mn), each < 64;
 *              dm fp16 [N,K/256][2] = (d, dmin)               w = d*sc*q - dmin*mn
 *   LORA_Q6_K  ql u4 [N,K]; qh u2 [N,K]; sc int8 [N,K/16]; d fp16 [N,K/256]
 *                                              w = d*sc*(q-32), q = ql | qh<<4
 * u4 planes hold element 2j in the low nibble of byte j and element 2j+1 in
 * the high nibble; the u2 plane holds element 4j+i in bits 2i..2i+1 of
 * byte j.  K must be a multiple of 32 (Q8_0, Q4_0) or 256 (Q4_K, Q6_K). */
typedef enum lora_dtype {
  LORA_F32 = 0,
  LORA_BF16 = 1,
  LORA_Q8_0 = 2,
  LORA_Q4_0 = 3,
  LORA_Q4_K = 4,
  LORA_Q6_K = 5
} lora_dtype;

/* Train-only inverted dropout on the LoRA-branch input ("4.3. Training
 * Guide", "Dropout"): a stateless hash of (seed, optimizer step,
 * accumulation ordinal, layer, projection, token row, feature column).
 * Element (t,k) is kept when the top 24 bits of the hash are
 * >= round(p * 2^24); kept values are multiplied by float(1/(1-p)).
 * The hash is SplitMix64's output function chained over the keys in the
 * order seed, step, ordinal, layer, proj, t, k.  p == 0 (or a NULL
 * descriptor) turns dropout off.  Requires 0 <= p < 1. */
typedef struct lora_dropout {
  uint64_t seed;
  int64_t step;      /* 0-based index of the optimizer update being built  */
  int32_t ordinal;   /* accumulation chunk index within the update         */
  int32_t layer;
  int32_t proj;      /* projection ordinal: wq..wdown = 0..6               */
  float p;
} lora_dropout;

/* One adapted linear ("8. LoRA Fundamentals", "How it works"):
 *   Y = X W^T + scale * (X~ A^T) B^T,   X~ = X masked by dropout.
 * DoRA (same section): when dora_mag and dora_norm are both non-NULL, the
 * output column n is multiplied by dora_mag[n] / dora_norm[n]; the norm is a
 * detached input (see lora_dora_row_norms).
 * Constraints: tokens, in_dim, out_dim > 0; in_dim and out_dim multiples of 4
 * (of 8 for bf16 W); rank a multiple of 4 with rank <= min(in_dim, out_dim,
 * 128).  W is float32, bf16 or block-quantized (lora_dtype; the quantized
 * products run in bf16 on the decoded weights).  Any T is accepted (ragged
 * tails are masked).  Every pointer, dora_mag and dora_norm included, is
 * 16-byte aligned (LORA_E_ALIGN otherwise).  bf16 and quantized W also need
 * in_dim*out_dim, tokens*in_dim and tokens*out_dim below 2^30 (their operands
 * are addressed with 32-bit byte offsets; LORA_E_SHAPE otherwise), and
 * quantized W an in_dim that is a whole number of its blocks (LORA_E_SHAPE). */
typedef struct lora_linear {
  int64_t tokens, in_dim, out_dim, rank;
  int32_t w_dtype;          /* lora_dtype                                  */
  float scale;              /* alpha/rank or alpha/sqrt(rank)              */
  const void* W;            /* [N,K] float32 or bf16, or the planes of a
                               quantized W laid out by lora_qweight_layout */
  const float* A;           /* [r,K]                                       */
  const float* B;           /* [N,r]                                       */
  const float* dora_mag;    /* [N] or NULL                                 */
  const float* dora_norm;   /* [N] or NULL                                 */
  int32_t dora_from_y;      /* DoRA only, else 0: the backward's Z argument
                               is the forward's Y (below); every dora_mag
                               entry must then be nonzero                   */
} lora_linear;

/* Layout of a block-quantized W [out_dim, in_dim] in one buffer: the planes
 * of the format (table at lora_dtype) in that order, each starting at a
 * multiple of 256 bytes from the buffer's start.  Writes the byte offset of
 * each plane to offsets[0..3] (formats with fewer planes get the total for
 * the missing ones) and returns the total size in bytes; returns 0, writing
 * nothing, for a format that is not block-quantized, non-positive sizes or
 * an in_dim that is not a whole number of blocks.  offsets may be NULL. */
size_t lora_qweight_layout(int32_t w_dtype, int64_t out_dim, int64_t in_dim, size_t* offsets);

/* A run of parameters in the optimizer arena. kind 0 = LoRA A (decayed,
 * rate lr), 1 = LoRA B (never decayed, rate lr * plus_ratio), 2 = DoRA
 * magnitude (never decayed, rate lr). */
typedef struct lora_segment {
  int64_t offset, count;
  int32_t kind;
} lora_segment;

/* AdamW hyper-parameters of one update ("4.3. Training Guide", "Optimizer").
 * lr is the already-scheduled rate of this update; t is the 1-based count of
 * applied updates of the slot including this one.  Host doubles: the derived
 * constants (1-beta, bias corrections, rates) are formed in double and
 * rounded once to float for the kernel. */
typedef struct lora_adamw_hparams {
  double lr, beta1, beta2, eps, weight_decay, plus_ratio;
  int64_t t;
} lora_adamw_hparams;

/* Bytes of workspace that lora_forward and lora_backward need for `lin`
 * (split-contraction partials).  Returns 0 when `lin` is invalid. */
size_t lora_workspace_bytes(const lora_linear* lin);

/* Forward of one chunk ("8. LoRA Fundamentals", "How it works"):
 *   U = X~ A^T  [T,r]  (saved for the backward)
 *   Z = X W^T + scale * U B^T  [T,N]
 *   Y = Z, or Y = (dora_mag/dora_norm) * Z per column for DoRA.
 * Z may be NULL.  A DoRA backward needs Z, or, with lin->dora_from_y set,
 * Y in its place, in which case the forward need not write Z (half of a DoRA
 * forward's output traffic).  Y and U are overwritten.  `drop` may be NULL.
 * ws must hold lora_workspace_bytes(lin). */
int lora_forward(const lora_linear* lin, const float* X, float* Y, float* U,
                 float* Z, const lora_dropout* drop, void* ws, size_t ws_bytes,
                 void* stream);

/* Backward of one chunk ("8. LoRA Fundamentals", "Training decisions" and
 * "The training loop"; "Backward Bug Hunts ...", "Bug #1").  With g = dY, or
 * for DoRA g = dY * dora_mag/dora_norm (the norm is detached):
 *   V   = g B                                   [T,r]
 *   dX  = g W + scale * (V A) * mask * keep     [T,K]  overwritten
 *   dB (+)= scale * g^T U                       [N,r]
 *   dA (+)= scale * V^T X~                      [r,K]
 *   dMag (+)= sum_t dY * Z / dora_norm          [N]    (DoRA, may be NULL)
 * accumulate != 0 adds into dA/dB/dMag (gradient accumulation over the
 * chunks of one update); accumulate == 0 overwrites them (first chunk).
 * W is read in its native [N,K] layout.  dX may be NULL (not computed).
 * U is the forward's U of the same chunk; Z is required when dMag is given:
 * the forward's Z, or with lin->dora_from_y its Y, from which
 *   dMag (+)= sum_t dY * Y / dora_mag   (the same sum: Y = Z dora_mag/dora_norm).
 * The mask is recomputed from `drop`, which must equal the forward's. */
int lora_backward(const lora_linear* lin, const float* X, const float* dY,
                  const float* U, const float* Z, float* dX, float* dA,
                  float* dB, float* dMag, int accumulate,
                  const lora_dropout* drop, void* ws, size_t ws_bytes,
                  void* stream);

/* Linears that read one X (the projections of one layer that share their
 * input, e.g. wq and wv; "8. LoRA Fundamentals", "How it works", target
 * list) may run as a group: the same results, bitwise, as calling
 * lora_forward / lora_backward on each in turn, with the group's launches
 * shared where the kernels allow (short chunks with fp32 W).  All linears of
 * a group must have equal tokens and in_dim (else LORA_E_SHAPE); their W
 * types may differ (a quantized base mixes formats); 1 <= n <= LORA_MAX_GROUP.  Array arguments hold one entry
 * per linear, in the order of `lins`; Z, dX, dMag and drops may be NULL as a
 * whole (meaning NULL for every linear) or hold NULL entries.  The group
 * workspace is the per-linear workspaces laid end to end (each rounded up to
 * 256 bytes).  Validation of every linear precedes any launch. */
#define LORA_MAX_GROUP 4
#define LORA_MAX_SLOTS 4
size_t lora_group_workspace_bytes(int n, const lora_linear* lins);
int lora_forward_group(int n, const lora_linear* lins, const float* X, float* const* Y,
                       float* const* U, float* const* Z, const lora_dropout* drops, void* ws,
                       size_t ws_bytes, void* stream);
int lora_backward_group(int n, const lora_linear* lins, const float* X, const float* const* dY,
                        const float* const* U, const float* const* Z, float* const* dX,
                        float* const* dA, float* const* dB, float* const* dMag, int accumulate,
                        const lora_dropout* drops, void* ws, size_t ws_bytes, void* stream);

/* Adapter slots over one frozen W ("Multi-LoRA Training Example
 * (fully-async)", "Design (decoupled per-adapter optimizers)": adapters
 * share the base model, each with its own data, factors and optimizer).
 * The same work as n separate lora_forward / lora_backward calls, slot i
 * with lins[i], X[i], Y[i] ... and drops[i] (drops may be NULL).  When W is
 * bf16, n > 1, every slot's token count is a multiple of 256 and n*tokens
 * times in_dim and out_dim stay below 2^30, each frozen product runs once
 * over the slots' stacked rows (one pass over W for all slots); otherwise the
 * slots run one after another.  Results equal the separate calls up to the
 * summation order of the frozen products.  lins[i] must share W, tokens,
 * in_dim, out_dim, rank and w_dtype, and all or none be DoRA (LORA_E_SHAPE /
 * LORA_E_DTYPE / LORA_E_INVALID otherwise); 1 <= n <= LORA_MAX_SLOTS.
 * dX is NULL, or an array whose entries are all NULL or all set.  The
 * workspace (lora_slots_workspace_bytes) holds every slot's share and the
 * stacked bf16 operands and partials; its contents between calls do not
 * matter. */
size_t lora_slots_workspace_bytes(int n, const lora_linear* lins);
int lora_forward_slots(int n, const lora_linear* lins, const float* const* X, float* const* Y,
                       float* const* U, float* const* Z, const lora_dropout* drops, void* ws,
                       size_t ws_bytes, void* stream);
int lora_backward_slots(int n, const lora_linear* lins, const float* const* X,
                        const float* const* dY, const float* const* U, const float* const* Z,
                        float* const* dX, float* const* dA, float* const* dB, float* const* dMag,
                        int accumulate, const lora_dropout* drops, void* ws, size_t ws_bytes,
                        void* stream);

/* Workspace bytes lora_grad_prepare needs for n gradient elements. */
size_t lora_grad_prepare_workspace_bytes(int64_t n);

/* Prepare the summed gradients of one slot ("4.3. Training Guide",
 * "Gradient clipping" and "Gradient accumulation").  Pass 1: sum of squares
 * in double and a non-finite flag, per block.  Pass 2 (one block, fixed
 * order): norm = sqrt(ss)/n_pred_tokens; clip = max_norm/norm when
 * max_norm > 0 and norm > max_norm, else 1; writes the combined scale
 * *d_scale = float(clip/n_pred_tokens), or NaN when any gradient is
 * non-finite.  `grads` is not modified (the scale is applied on load by
 * lora_adamw_step).  If h_norm (host) is not NULL the call waits for the
 * stream, stores the norm (NaN on veto) and returns LORA_E_NONFINITE on a
 * veto; with h_norm NULL nothing waits and the veto travels in *d_scale.
 * d_stats (device, may be NULL) receives {norm, clip} as doubles. */
int lora_grad_prepare(const float* grads, int64_t n, int64_t n_pred_tokens,
                      float max_norm, float* d_scale, double* d_stats,
                      double* h_norm, void* ws, size_t ws_bytes, void* stream);

/* Allocation-free lora_grad_prepare, for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  The same two passes and
 * results as lora_grad_prepare (bitwise: the same kernels over the same
 * partition), with its partials, flags and {norm, clip} pair in a static
 * device scratch array of 16,640 bytes per GPU (held until the process
 * ends; its device address is looked up once per device, on the first call
 * on that device).  That size holds the passes' scratch for any n; a size
 * it could not hold would be refused with LORA_E_WORKSPACE.  Allocates
 * nothing and calls no allocating routine.  Every call on one GPU uses that
 * GPU's one array, which keeps the last call's contents (each call writes
 * every word it reads before reading it): calls that overlap on one GPU
 * (concurrent streams or host threads) race and must be serialised by the
 * caller.  h_norm != NULL synchronises the stream, as in lora_grad_prepare.
 * Returns LORA_E_HIP if the scratch's address cannot be obtained. */
int lora_grad_prepare_noalloc(const float* grads, int64_t n, int64_t n_pred_tokens,
                              float max_norm, float* d_scale, double* d_stats, double* h_norm,
                              void* stream);

/* Decoupled AdamW over the arena segments ("4.3. Training Guide",
 * "Optimizer"; "8. LoRA Fundamentals", "The training loop"):
 *   g' = grads * (*d_scale)
 *   m = b1 m + (1-b1) g';  v = b2 v + (1-b2) g'^2
 *   p -= rate * (m/(1-b1^t)) / (sqrt(v/(1-b2^t)) + eps)
 *   A only: p -= lr * weight_decay * p_old
 * rate = lr (A, magnitude) or lr * plus_ratio (B).  When *d_scale is not
 * finite (a vetoed update) no element is changed.  `segs` is a host array
 * of n_seg (1..64) non-overlapping segments. */
int lora_adamw_step(float* params, const float* grads, float* m, float* v,
                    const lora_segment* segs, int n_seg,
                    const lora_adamw_hparams* hp, const float* d_scale,
                    void* stream);

/* Writes the dropout keep mask [tokens, in_dim] (1 = keep) of `drop`: the
 * same decisions lora_forward and lora_backward take inline. */
int lora_dropout_mask(const lora_dropout* drop, int64_t tokens, int64_t in_dim,
                      uint8_t* mask, void* stream);

/* DoRA row norms ("8. LoRA Fundamentals", "How it works"):
 * out_norm[i] = || W_i + scale * (B A)_i ||_2 over the K inputs.  With
 * lin->A == lin->B == NULL it gives ||W_i|| (the magnitude initialisation).
 * lin->tokens and lin->dora_* are ignored; any out_dim > 0, 0 < in_dim <=
 * 2^22 and 0 < rank <= 128 are accepted (LORA_E_SHAPE otherwise; unaligned
 * rows take element loads).  A block-quantized W (the DoRA of a quantized
 * base) is decoded to float32 (exactly, but for one rounding of Q4_K's sum);
 * it needs in_dim a whole number of its blocks and in_dim * out_dim < 2^30.
 * The contraction is split over column ranges whose double partials go to
 * `workspace` (device, lora_dora_row_norms_workspace_bytes(lin) bytes, 0 for
 * small K: then it may be NULL) and are summed per row in a fixed order by a
 * second launch; with workspace == NULL one block covers all columns of its
 * rows (fewer blocks, same result up to rounding order).  A non-NULL
 * workspace smaller than required gives LORA_E_WORKSPACE.  out_norm is a
 * device float[out_dim]. */
size_t lora_dora_row_norms_workspace_bytes(const lora_linear* lin);
int lora_dora_row_norms(const lora_linear* lin, float* out_norm, void* workspace,
                        size_t workspace_bytes, void* stream);

/* The DoRA row norms of n linears (the refresh after an update; "8. LoRA
 * Fundamentals", "How it works"), out_norms[i] for lins[i], each accepted as
 * by lora_dora_row_norms (the first invalid one's status is returned before
 * any launch).  Linears with bf16 W whose rows are 16-byte aligned (in_dim a
 * multiple of 8), LoRA factors and rank <= 64 expand the square:
 *   n_i^2 = ||W_i||^2 + 2 scale sum_j B_ij (W A^T)_ij
 *           + scale^2 sum_jl B_ij (A A^T)_jl B_il,
 * with A split exactly into three bf16 parts so that the products over the
 * inputs are exact bf16 products summed in float32, and the three terms
 * combined in double; adjacent such linears with the same W, out_dim, in_dim
 * and rank (adapter slots over one base, up to 4) share one pass over W.
 * The expansion matches the direct form to float32 rounding relative to
 * ||W_i||^2 + |2 scale <W_i,(B A)_i>| + scale^2 ||(B A)_i||^2, so rows whose
 * adapted norm is far below ||W_i|| lose relative accuracy; use
 * lora_dora_row_norms for such rows.  The other linears run as
 * lora_dora_row_norms, one after another.  workspace: device,
 * lora_dora_row_norms_batch_workspace_bytes(n, lins) bytes (0 only when no
 * linear needs any), 16-byte aligned (LORA_E_WORKSPACE / LORA_E_ALIGN
 * otherwise); its contents between calls do not matter.  The results equal
 * lora_dora_row_norms up to rounding. */
size_t lora_dora_row_norms_batch_workspace_bytes(int n, const lora_linear* lins);
int lora_dora_row_norms_batch(int n, const lora_linear* lins, float* const* out_norms,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Merge for export ("8. LoRA Fundamentals": "How it works" for the
 * effective weight W + scale*B*A merged in F32 and DoRA's row rescale;
 * "Profiling with --jfr" for the RMSE a merge reports):
 *   W_out[i][k] = c_i * (W[i][k] + scale * (B A)[i][k]),
 *   c_i = dora_mag[i] / dora_norm[i] when both are set (DoRA), else 1.
 * out_dtype LORA_F32 stores the float32 values; LORA_BF16 rounds them to
 * bfloat16, to nearest with ties to even.  W_out is a device [out_dim,
 * in_dim] array of that type, caller-owned.  When rmse (device double[1]) is
 * non-NULL it receives sqrt(mean((W_out - merged float32)^2)) over all
 * elements: 0 for LORA_F32 output; for LORA_BF16 the per-wave sums go to
 * `workspace` (lora_merge_workspace_bytes(lin) bytes, else LORA_E_WORKSPACE)
 * and are added in a fixed order.  lin->A == lin->B == NULL merges W alone
 * (a conversion).  Shapes as for lora_dora_row_norms. */
size_t lora_merge_workspace_bytes(const lora_linear* lin);
int lora_merge(const lora_linear* lin, void* W_out, int out_dtype, double* rmse, void* workspace,
               size_t workspace_bytes, void* stream);

/* Diagnostics: launch timing.  lora_profile_begin opens a profile that can
 * hold max_launches launches (it creates that many HIP event pairs once and
 * keeps them); until lora_profile_end, each kernel launch of the library is
 * bracketed by two events recorded on its own stream.  lora_profile_end waits
 * for the device, writes up to max_entries aggregates (one per kernel name and
 * shape, in first-launch order) and returns their count, or a negative status.
 * `kernel` points to a static string.  flops and bytes are the algorithmic
 * work of one launch (bytes: each operand read once, each result written
 * once).  Not thread-safe; meant for benchmarks, not production paths. */
typedef struct lora_profile_entry {
  const char* kernel;
  int64_t M, N, K;        /* shape the kernel name documents                  */
  int64_t launches;
  double total_ms;        /* summed event-to-event time over the launches      */
  double flops, bytes;    /* algorithmic work of one launch                    */
} lora_profile_entry;
int lora_profile_begin(int max_launches);
int lora_profile_end(lora_profile_entry* out, int max_entries);

/* Tile configuration of the bf16-W frozen products (a tuning and testing
 * control; "8. LoRA Fundamentals", "How it works", is the product itself).
 * cfg -1 (the default) lets the planner choose per product; cfg 0-5 makes
 * every bf16 product the configuration can run use it (with the planner's
 * contraction split), others keep the planner's choice.  Configuration 5
 * loads the activation operand straight into registers from a fragment-tiled
 * copy and needs plain bf16 W, tokens a multiple of 32 and a contraction a
 * multiple of 64.  Process-wide; workspace sizes follow the setting, so set
 * it before sizing workspaces and while no call is being planned.  Returns
 * LORA_OK, or LORA_E_INVALID for cfg outside -1..5. */
int lora_set_bf16_config(int cfg);

/* Host helpers. */
/* alpha/rank, or alpha/sqrt(rank) when rslora != 0 ("How it works"). */
double lora_scaling(double alpha, int64_t rank, int rslora);
/* Learning rate of the 0-based update k ("4.3. Training Guide",
 * "Schedules"): schedule 0 = constant lr; 1 = warmup-cosine: lr*(k+1)/warmup
 * for k < warmup, then lr_min + (lr-lr_min)(1+cos(pi*min(1,(k-warmup)/
 * max(1,total-warmup))))/2. */
double lora_lr_at(int64_t k, double lr, int schedule, int64_t warmup,
                  int64_t total, double lr_min);
/* Static message for a status code. */
const char* lora_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* LORA_H */
