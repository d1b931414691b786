/*
 * moe.h -- C ABI of the MI355X (gfx950) DeepSeek-V3-style MoE layer forward.
 *
 * The layer, as the pages state it:
 *   - gate: sigmoid scores of a linear map of the token, a per-expert bias
 *     that only takes part in choosing experts, a per-group sum of the two
 *     largest choice scores, the topk_group best groups, the top_k best
 *     experts inside them, weights from the unbiased scores normalised over
 *     the chosen experts (top_k > 1) and multiplied by routed_scaling_factor
 *     ("从 1024 块 GPU 到 558 万美元：拆解 DeepSeek-V3 的算法-系统协同设计",
 *     section 2.2, the MoEGate module);
 *   - dispatch: per-expert token counts and the tokens sorted by expert id
 *     (same page, section 2.3, the dispatch skeleton);
 *   - experts: 256 fine-grained routed experts of FFN width 2048 and one
 *     always-active shared expert (same page, section 2.2; "深入理解
 *     DeepSeek-V3：大规模缩放挑战与对 AI 架构硬件的反思（中文精读）", section 3.1:
 *     8 routed + 1 shared per token); each a SwiGLU FFN (mqxn.cn/news/19449,
 *     section 3.1);
 *   - combine: the expert outputs collected back to their tokens (first page,
 *     section 2.3), summed with the gate weights, plus the shared expert;
 *   - FP8 variant: activations quantised per 1x128 tile and weights per
 *     128x128 block, fp32 accumulation ("深入理解 DeepSeek-V3…", section 3.2).
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers, owned by the caller.  The
 *     library allocates no device memory; scratch space comes from the
 *     caller's workspace (ws, ws_bytes; see moe_workspace_bytes).
 *   - All work is enqueued asynchronously on `stream` (a hipStream_t; NULL is
 *     the default stream).  No entry point synchronises the host with the
 *     device except moe_get_device_error.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     failed validation returns an error code and enqueues nothing.  No C++
 *     exception crosses the ABI.  moe_last_error() gives a thread-local text
 *     for the last failing call on the calling thread.
 *   - Layouts are row-major.  Weight matrices are stored "output rows x
 *     input columns" with the input dimension contiguous.
 *   - T == 0 is a no-op returning MOE_OK.
 *   - Global state: the kernel timer below (off by default), the gate mode
 *     (moe_set_gate_mode, split by default), kernel attributes set once per
 *     process on first use, the two fork/join events of moe_forward_overlap (per device and host
 *     thread), and the static workspace of moe_forward_noalloc (one per
 *     device).  Calls on
 *     different streams with different workspaces may run concurrently.
 *   - Results are deterministic: no floating-point atomics anywhere, so two
 *     runs on the same inputs give bitwise-identical outputs.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,   /* null pointer, bad shape, inconsistent config   */
    MOE_ERR_UNSUPPORTED = 2,   /* valid for the method, not handled by kernels   */
    MOE_ERR_WORKSPACE = 3,     /* ws null or ws_bytes below the required size    */
    MOE_ERR_HIP = 4,           /* a HIP runtime call or kernel launch failed     */
    MOE_ERR_DEVICE_CHECK = 5   /* a kernel saw an out-of-range expert index      */
} moe_status;

typedef enum {
    MOE_F32 = 0,       /* IEEE binary32                                        */
    MOE_BF16 = 1,      /* bfloat16                                             */
    MOE_FP8_E4M3 = 2,  /* OCP e4m3fn + fp32 scale per 128x128 block (weights)  */
    MOE_FP8_E4M3_E8M0 = 3  /* OCP e4m3fn + power-of-two fp32 scale per 128x128
                              block (weights); the activations get
                              power-of-two 1x128 scales too, and the matrix
                              cores apply the scales (packed weights only)  */
} moe_dtype;

/* Layer shape: the MoEGate constructor arguments of the first page's
 * section 2.2 plus the expert FFN widths. */
typedef struct {
    int32_t hidden_size;              /* H                                         */
    int32_t n_routed_experts;         /* E   (2 <= E <= 512)                        */
    int32_t n_group;                  /* G   (E % G == 0, E / G >= 2, G <= 64)      */
    int32_t topk_group;               /* TG  (1 <= TG <= G)                         */
    int32_t num_experts_per_tok;      /* K   (1 <= K <= min(E, 64))                 */
    int32_t moe_intermediate_size;    /* I   routed expert FFN width                */
    int32_t shared_intermediate_size; /* Is  shared expert FFN width, 0 = none      */
    float routed_scaling_factor;      /* rho (finite, > 0)                          */
    moe_dtype act_dtype;              /* x, expert outputs and layer output:
                                         MOE_F32 or MOE_BF16                        */
    moe_dtype weight_dtype;           /* expert and shared weights: MOE_F32 (with
                                         act F32), MOE_BF16 or MOE_FP8_E4M3 (with
                                         act BF16)                                  */
} moe_config;

/* Layer weights.  The gate weight and the selection bias are always fp32.
 * w13 stacks each expert's gate projection (rows 0..I-1) over its up
 * projection (rows I..2I-1).  For MOE_FP8_E4M3 the *_scale arrays hold one
 * fp32 per 128x128 block, row-major over (row block, column block); for
 * MOE_FP8_E4M3_E8M0 every scale must be a power of two (the kernels read its
 * exponent field); the scales are ignored (may be NULL) otherwise.  ws13/ws2 (+scales) may be NULL iff Is == 0.
 * packed = 0: w13, w2, ws13, ws2 are row-major as shown; packed = 1: all four
 * were rearranged by moe_pack_weight (bf16 or e4m3 weights; scales unchanged). */
typedef struct {
    const float* gate_w;     /* [E, H]                                           */
    const float* bias;       /* [E]  e_score_correction_bias                     */
    const void* w13;         /* [E, 2I, H]                                       */
    const float* w13_scale;  /* [E, 2I/128, H/128]                               */
    const void* w2;          /* [E, H, I]                                        */
    const float* w2_scale;   /* [E, H/128, I/128]                                */
    const void* ws13;        /* [2Is, H]                                         */
    const float* ws13_scale; /* [2Is/128, H/128]                                 */
    const void* ws2;         /* [H, Is]                                          */
    const float* ws2_scale;  /* [H/128, Is/128]                                  */
    int32_t packed;          /* 0 = row-major, 1 = moe_pack_weight layout         */
} moe_weights;

/* Which expert weight matrix a pack call converts. */
typedef enum { MOE_W13 = 0, MOE_W2 = 1, MOE_WS13 = 2, MOE_WS2 = 3 } moe_weight_id;

/* Bytes of workspace that every entry point below needs for T tokens (the
 * maximum over them, so one buffer serves all).  Returns 0 if cfg is invalid
 * or unsupported. */
size_t moe_workspace_bytes(const moe_config* cfg, int64_t T);

/* Gate and selection (first page, section 2.2).
 *   x       [T, H] act_dtype
 *   gate_w  [E, H] fp32,  bias [E] fp32
 *   logits  [T, E] fp32 out, may be NULL: then they are not kept (the
 *           workspace holds per-k-range partial sums only), so a caller that
 *           needs them later (moe_backward does) passes this array.  The
 *           gate product is computed to fp32 accuracy: x is exact in bf16 and
 *           the fp32 gate weight is split into three bf16 parts whose
 *           products with x are exact, accumulated in fp32 on MFMA.
 *   topk_idx [T, K] int32 out: chosen experts, in descending order of masked
 *           choice score, ties to the lower expert id.
 *   topk_w  [T, K] fp32 out: routed weights.
 * Selection arithmetic (bit-reproducible from the fp32 logits): score =
 * fp32 rounding of the double-precision sigmoid; choice = score + bias (fp32
 * add); group score = fp32 sum of the group's two largest choices; groups and
 * experts chosen by exact fp32 comparison, ties to the lower index; experts
 * outside the kept groups compete with choice 0.0f. */
moe_status moe_gate(const moe_config* cfg, int64_t T, const void* x, const float* gate_w,
                    const float* bias, float* logits, int32_t* topk_idx, float* topk_w,
                    void* ws, size_t ws_bytes, void* stream);

/* How moe_gate and moe_forward run the gate and the selection of bf16 tokens
 * (the same layer step as moe_gate above; the routing is the same function
 * of the fp32 logits either way, the logits may differ in the last bits
 * because the k sums are ordered differently):
 *   MOE_GATE_SPLIT (default): the gate GEMM writes k-split partial logits
 *     to the workspace and a second kernel sums them and selects;
 *   MOE_GATE_FUSED: one kernel per 64 tokens computes all E logits over
 *     the whole hidden size, keeps them in LDS and selects in its epilogue
 *     (nothing but the outputs goes to memory); taken only for shapes it
 *     supports (E a multiple of 32 up to 256, n_group dividing E with either
 *     whole groups per eighth of E or a group spanning 2, 4 or 8 eighths,
 *     n_group <= 32, top_k <= 16, hidden_size a multiple of 64), else SPLIT.
 *     On an MI355X it is slower than SPLIT at every batch size measured
 *     (T = 16384: about 0.28 against 0.26 ms): a workgroup holding every
 *     expert of its tokens holds only 64 tokens, so each weight byte read
 *     from L2 feeds half as many MFMAs.
 * Process-wide; decode batches (T <= 32) of moe_forward keep their own
 * routing schedule.  Returns MOE_ERR_INVALID_ARG for other values. */
typedef enum { MOE_GATE_SPLIT = 0, MOE_GATE_FUSED = 1 } moe_gate_mode;
moe_status moe_set_gate_mode(int mode);

/* Dispatch order (first page, section 2.3).
 *   topk_idx [T, K] int32 in (values in [0, E); others set the device error
 *           flag in ws, see moe_get_device_error, and are skipped)
 *   counts  [E] int32 out: tokens per expert
 *   offsets [E+1] int32 out: exclusive prefix sum, offsets[E] = T*K
 *   perm    [T*K] int32 out: flat indices f = t*K + k sorted by expert id,
 *           stable (ascending f inside an expert)
 *   pos     [T*K] int32 out: inverse of perm (pos[perm[j]] = j) */
moe_status moe_permute(const moe_config* cfg, int64_t T, const int32_t* topk_idx,
                       int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pos,
                       void* ws, size_t ws_bytes, void* stream);

/* Routed and shared expert FFNs (SwiGLU: W2 (silu(W_gate x) * (W_up x))).
 *   x       [T, H] act_dtype
 *   perm, offsets from moe_permute (device)
 *   y       [T*K, H] act_dtype out: row j = expert e's output on token
 *           perm[j] / K, where offsets[e] <= j < offsets[e+1]
 *   y_shared [T, H] act_dtype out (NULL iff Is == 0)
 * bf16 weights: bf16 MFMA, fp32 accumulation, SiLU*up fused, h kept in bf16.
 * fp8 weights: x and h quantised per 1x128 tile to e4m3 (see
 * moe_quantize_act), e4m3 MFMA, per-128-block scales applied to fp32 partial
 * sums.  fp8 weights with power-of-two scales (MOE_FP8_E4M3_E8M0, packed):
 * x and h quantised with power-of-two 1x128 scales, and the scaled e4m3
 * MFMA applies both scales inside the matrix core over the whole k loop
 * (its accumulation carries about 13 fraction bits per instruction, below
 * the bf16 rounding of the outputs).  f32: fp32 arithmetic throughout. */
moe_status moe_expert_ffn(const moe_config* cfg, int64_t T, const void* x, const int32_t* perm,
                          const int32_t* offsets, const moe_weights* w, void* y, void* y_shared,
                          void* ws, size_t ws_bytes, void* stream);

/* Combine: out[t] = y_shared[t] + sum_k topk_w[t,k] * y[pos[t*K+k]], fp32
 * accumulation in k order, rounded once to act_dtype.
 *   y [T*K, H], y_shared [T, H] (NULL iff Is == 0), pos [T*K], topk_w [T, K],
 *   out [T, H] act_dtype. */
moe_status moe_combine(const moe_config* cfg, int64_t T, const void* y, const void* y_shared,
                       const int32_t* pos, const float* topk_w, void* out, void* stream);

/* The whole layer: gate, permute, expert FFNs, combine, enqueued in that
 * order.  out [T, H] act_dtype.  logits [T,E], topk_idx/topk_w [T,K],
 * counts [E] and perm [T*K] are optional copies of the intermediate results
 * (NULL: kept in the workspace only).
 * Decode batches (1 <= T <= 32) take a shorter schedule of the same steps:
 * the gate straight from the fp32 gate weight over a few k ranges (bf16
 * activations: bf16 MFMA over the weight's exact bf16 split, made in
 * registers; fp32 activations: fp32 dot products), the same selection
 * kernel, then one workgroup that permutes and lays out the GEMM tiles.  The
 * logits then differ from moe_gate's in rounding only (both are fp32
 * accumulations of the exact products); the choice is made from the logits
 * written. */
moe_status moe_forward(const moe_config* cfg, int64_t T, const void* x, const moe_weights* w,
                       void* out, float* logits, int32_t* topk_idx, float* topk_w,
                       int32_t* counts, int32_t* perm, void* ws, size_t ws_bytes, void* stream);

/* moe_forward of a decode batch as ONE kernel launch ("深入理解 DeepSeek-V3…",
 * section 3.1: batches of about 32 tokens, the always-active shared expert
 * overlapped with the routed path): gate, selection, permutation, the routed
 * and shared expert GEMMs and the combine run as roles of one grid whose
 * workgroups signal each other through completion flags in ws, so that the
 * shared expert streams its weights during the routing and an expert's down
 * projection starts when its own gate/up projection is done.  Same
 * arguments, workspace and results as moe_forward, bit for bit.
 *   Takes 1 <= T <= 32 bf16 tokens with packed bf16 weights; anything else
 *   returns MOE_ERR_UNSUPPORTED and enqueues nothing.
 *   Under HIP graph capture it enqueues two launches: a one-thread kernel
 *   that advances a call counter kept in ws, then the layer, so that every
 *   replay uses fresh completion flags.
 *   Every wait inside the kernel is bounded; a wait that gives up sets bit 2
 *   of the device error flag (moe_get_device_error) and that call's outputs
 *   are unreliable.  Calls that overlap on one workspace race.
 *   Measured on MI355X it is slower than moe_forward's multi-launch decode
 *   schedule at the V3 shape (agent-scope fences and polls under the
 *   weight stream cost more than the launch gaps they remove), so
 *   moe_forward does not use it. */
moe_status moe_forward_decode_fused(const moe_config* cfg, int64_t T, const void* x,
                                    const moe_weights* w, void* out, float* logits,
                                    int32_t* topk_idx, float* topk_w, int32_t* counts,
                                    int32_t* perm, void* ws, size_t ws_bytes, void* stream);

/* moe_forward with the shared expert on a second stream, the single-GPU
 * part of the dual micro-batch overlap ("深入理解 DeepSeek-V3…", section 3.1):
 * the always-active shared expert ("从 1024 块 GPU 到 558 万美元：拆解 DeepSeek-V3
 * 的算法-系统协同设计", section 2.2) does not depend on the routing, so its GEMMs
 * start on shared_stream at once and run beside the gate, the permutation
 * and the routed experts on stream; stream waits for them before the
 * combine.  Same arguments and outputs as moe_forward, bit for bit (the
 * shared expert's tiles are the same kernels with the same arithmetic).
 *   shared_stream: a stream of the same device, not stream.  Work enqueued on
 *   it before the call runs before the shared expert; when the call returns,
 *   every output is ordered on stream (shared_stream is not needed again).
 * fp32 weights (and configs without a shared expert) run wholly on stream.
 * The library keeps two HIP events per device and host thread for the fork
 * and the join (created on first use).  The call may be captured into a
 * HIP graph on stream.
 * Errors: MOE_ERR_INVALID_ARG if shared_stream is NULL or equals stream; the
 * rest as moe_forward. */
moe_status moe_forward_overlap(const moe_config* cfg, int64_t T, const void* x,
                               const moe_weights* w, void* out, float* logits, int32_t* topk_idx,
                               float* topk_w, int32_t* counts, int32_t* perm, void* ws,
                               size_t ws_bytes, void* stream, void* shared_stream);

/* moe_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments and outputs as moe_forward, bit for bit (the same
 * kernels), without ws / ws_bytes: the workspace is a static device array
 * of MOE_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU, held
 * from the library's first use on that GPU until the process ends.  The
 * call allocates nothing (no hipMalloc, no allocating library routine).
 *   Limit: moe_workspace_bytes(cfg, T) <= MOE_NOALLOC_SCRATCH_BYTES (at the
 *   V3 shape, H 7168, 256 experts, top-8, bf16, FFN width 2048, that is
 *   T <= 288);
 *   larger batches return MOE_ERR_UNSUPPORTED and enqueue nothing.
 *   Every call on one GPU shares that GPU's array, which keeps the last
 *   call's contents; each call writes every part it reads before reading
 *   it, so nothing needs clearing.  Calls that overlap on one GPU (other
 *   streams, other threads) race on the array: the caller orders them.
 *   The error flag of moe_get_device_error lives in that array too; the
 *   forward's own selection always yields ids in [0, E).  The first call on
 *   a device looks the array's address up (hipGetSymbolAddress, which loads
 *   it): make that first call outside graph capture. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_forward_noalloc(const moe_config* cfg, int64_t T, const void* x,
                               const moe_weights* w, void* out, float* logits, int32_t* topk_idx,
                               float* topk_w, int32_t* counts, int32_t* perm, void* stream);

/* FP8 activation quantiser ("深入理解 DeepSeek-V3…", section 3.2: 1x128
 * activation tiles).  For each row of x [rows, H] (bf16, H % 128 == 0) and
 * each tile of 128 columns: a = max |v|; scale = a / 448 and inv = 448 / a,
 * each computed in double and rounded to fp32 (scale 1, inv 0 for a == 0);
 * code = nearest e4m3fn value of the fp32 product v * inv, ties to even,
 * saturated at +-448.  With weight_dtype MOE_FP8_E4M3_E8M0 the scale is
 * instead the smallest power of two 2^e >= a / 448 (e in [-126, 127]) and
 * inv = 2^-e, so v * inv is exact.
 *   xq [rows, H] uint8 out, xs [rows, H/128] fp32 out. */
moe_status moe_quantize_act(const moe_config* cfg, int64_t rows, const void* x, uint8_t* xq,
                            float* xs, void* stream);

/* Backward of the grouped SwiGLU expert FFN, for training.  The experts are
 * SwiGLU FFNs (mqxn.cn/news/19449, section 3.1) over the routed rows and the
 * always-active shared expert ("从 1024 块 GPU 到 558 万美元：拆解 DeepSeek-V3 的
 * 算法-系统协同设计", section 2.2); this computes their exact derivatives.  With
 * [g; u] = W13 x_row, h = silu(g) u, y_row = W2 h and the output gradient
 * dy_row of each row:
 *   dh = dy W2;  dg = dh u silu'(g);  du = dh silu(g);  dx_row = [dg du] W13;
 *   dW2 = sum over the expert's rows of dy^T h;  dW13 = sum of [dg du]^T x_row.
 * [g; u] is recomputed from x (fp32 accumulation); [dg du] and h are rounded
 * to bf16 before the GEMMs that consume them; every GEMM accumulates in fp32.
 *   x [T, H] bf16; perm [T*K] and offsets [E+1] as written by moe_permute.
 *   w: row-major bf16 weights (packed = 0): w13 [E, 2I, H], w2 [E, H, I],
 *      ws13 [2Is, H], ws2 [H, Is].
 *   dy [T*K, H] bf16: gradient of the routed expert outputs in the sorted row
 *      order of moe_expert_ffn's y (for the layer output: row pos[t*K+k] is
 *      topk_w[t,k] * dOut[t]); dy_shared [T, H]: gradient of y_shared.
 *   dx [T*K, H], dx_shared [T, H] out bf16 (nullable, both or neither):
 *      gradient of each row's input (sum the rows of a token for dx_t).
 *   dw13 [E, 2I, H], dw2 [E, H, I], dws13, dws2 out bf16: weight gradients
 *      (zero for an expert without rows).
 * e4m3 weights (MOE_FP8_E4M3 or MOE_FP8_E4M3_E8M0, row-major, with their
 * 128x128 block scales): the FP8 backward ("深入理解 DeepSeek-V3…", section
 * 3.2: operands in tiles of 128, fp32 accumulation).  [g; u] is recomputed
 * from x quantised per 1x128 tile (the FP8 forward); dy and [dg du] are
 * quantised per 1x128 tile along the dgrad GEMMs' contraction; for the
 * weight gradients dy, h, [dg du] and x are quantised per column in tiles of
 * 128 of the expert's rows (from its first row; the last tile shorter); the
 * weights keep their blocks; every GEMM accumulates in fp32 and the outputs
 * are bf16.  Scales as the forward's quantiser (a / 448, or powers of two
 * for MOE_FP8_E4M3_E8M0).
 * Workspace: moe_expert_ffn_backward_workspace_bytes(cfg, T) bytes (0 for a
 * configuration it does not handle), 256-byte aligned.  bf16 activations
 * with bf16 or e4m3 weights (MOE_ERR_UNSUPPORTED otherwise, or for packed
 * weights). */
size_t moe_expert_ffn_backward_workspace_bytes(const moe_config* cfg, int64_t T);
moe_status moe_expert_ffn_backward(const moe_config* cfg, int64_t T, const void* x,
                                   const int32_t* perm, const int32_t* offsets,
                                   const moe_weights* w, const void* dy, const void* dy_shared,
                                   void* dx, void* dx_shared, void* dw13, void* dw2,
                                   void* dws13, void* dws2, void* ws, size_t ws_bytes,
                                   void* stream);

/* Backward of the whole layer, for training, with the routing held at the
 * forward's choice (the top-k selection is piecewise constant: the gradient
 * reaches the gate through the chosen experts' weights only, and the
 * selection-only bias gets none).  The forward is that of moe_forward
 * ("从 1024 块 GPU 到 558 万美元：拆解 DeepSeek-V3 的算法-系统协同设计", section 2.2,
 * MoEGate, and the combine of section 2.3): out_t = shared(x_t) +
 * sum_k w_tk y_tk with w_k = rho s_k / (sum_j s_j + 1e-20) (top_k > 1) or
 * rho s_k, s = sigmoid(logits) of the chosen experts, logits = x Wg^T.
 * Given dout [T, H], with D = sum_j s_j + 1e-20:
 *   dy_tk = w_tk dout_t (the routed rows' gradients, rounded to bf16),
 *   dw_tk = <dout_t, y_tk>,  ds_k = rho (dw_k / D - sum_j dw_j s_j / D^2)
 *   (rho dw_k for top-1),  dlogit_tk = ds_k s_k (1 - s_k),
 *   dgate_w[e] = sum over the rows routed to e of dlogit x_t (fp32),
 *   dx_t = sum_k dlogit_tk Wg[idx_tk] + the experts' input gradients
 *   (moe_expert_ffn_backward, with the shared expert's output gradient dout;
 *   with e4m3 weights that is the FP8 expert backward, its operands
 *   quantised per 128 along each GEMM's contraction, "深入理解 DeepSeek-V3…",
 *   section 3.2).
 *   x [T, H] bf16; w: gate_w [E, H] fp32 and row-major bf16 or e4m3 expert
 *      weights with their block scales (packed = 0) as in
 *      moe_expert_ffn_backward;
 *   logits [T, E] fp32, topk_idx / topk_w [T, K], perm [T*K], offsets [E+1],
 *      pos [T*K]: the forward's (moe_gate, moe_permute);
 *   y [T*K, H] bf16: the routed expert outputs of the forward in sorted row
 *      order (moe_expert_ffn's y);
 *   dout [T, H] bf16: the gradient of the layer output.
 *   Outputs (written whole): dx [T, H] bf16, dgate_w [E, H] fp32, dw13,
 *   dw2 (and dws13, dws2 with a shared expert) bf16 as in
 *   moe_expert_ffn_backward.
 * Workspace: moe_backward_workspace_bytes(cfg, T) bytes (0 for a config the
 * backward does not take), 256-byte aligned.
 * Errors: MOE_ERR_UNSUPPORTED for fp32 activations or weights, or packed
 * weights; MOE_ERR_INVALID_ARG for a missing array (the block scales too,
 * with e4m3 weights); MOE_ERR_WORKSPACE. */
size_t moe_backward_workspace_bytes(const moe_config* cfg, int64_t T);
moe_status moe_backward(const moe_config* cfg, int64_t T, const void* x, const moe_weights* w,
                        const float* logits, const int32_t* topk_idx, const float* topk_w,
                        const int32_t* perm, const int32_t* offsets, const int32_t* pos,
                        const void* y, const void* dout, void* dx, float* dgate_w, void* dw13,
                        void* dw2, void* dws13, void* dws2, void* ws, size_t ws_bytes,
                        void* stream);

/* Load-balancing update of the selection bias.  The bias takes part only in
 * choosing experts and is steered by the experts' observed load instead of
 * a gradient ("从 1024 块 GPU 到 558 万美元：拆解 DeepSeek-V3 的算法-系统协同设计",
 * section 2.2, where the bias is a buffer updated from load statistics; the
 * page gives no formula).  Rule: with mean = sum(counts) / E, each expert's
 * bias becomes bias + gamma if counts[e] < mean, bias - gamma if
 * counts[e] > mean, and stays bit-identical otherwise; one fp32 add,
 * round-to-nearest-even.  The comparison with the mean is exact.
 *   counts [E] int32 in (device): rows per expert, e.g. the counts written
 *          by moe_permute or moe_forward, or their sum over several batches;
 *          a negative entry leaves the whole bias unchanged.
 *   bias   [E] fp32 in/out (device): updated in place; stream-ordered with
 *          the gate calls that read it.
 *   gamma  step, finite and >= 0 (MOE_ERR_INVALID_ARG otherwise).
 * Enqueues one small kernel; no workspace. */
moe_status moe_bias_update(const moe_config* cfg, const int32_t* counts, float gamma,
                           float* bias, void* stream);

/* Weight streaming layout for the expert GEMMs.  The grouped GEMM reads
 * each weight matrix once per call; in row-major order that is one short
 * piece per weight row per k step, rows a whole row length apart.  The packed
 * layout stores, for every (expert, output tile, k step), the MFMA operand
 * fragments of the tile's 256 weight rows as one contiguous 32 KiB block in
 * the order the kernel consumes them, so the weights stream sequentially
 * from HBM into registers.  Output tiles are 128 h columns (gate and up rows
 * together) for w13/ws13 and 256 output rows for w2/ws2.
 *   bf16: k steps of 64; block = [wave 4][col block 2][k slice 4][lane 64]
 *         x 16 bytes, lane l holding 8 values at k = 64 step + 32 (l / 32)
 *         + 8 slice.
 *   e4m3: k steps of 128 (one scale block); block = [wave 4][col block 2]
 *         [k half 2][16-byte half 2][lane 64] x 16 bytes, lane l holding 16
 *         codes at k = 128 step + 64 half_k + 32 (l / 32) + 16 half_16.
 *   Row of (wave w, col block cb, lane l) in tile t: w13/ws13 gate row
 *   128 t + 32 w + l % 32 (cb = 0) or the up row I + 128 t + 32 w + l % 32
 *   (cb = 1); w2/ws2 row 256 t + 64 w + 32 cb + l % 32.  Rows past the
 *   matrix are zero.  The fp8 block scales keep their row-major layout.
 * Pack once when the weights are loaded.
 *   moe_packed_bytes: size of the packed copy of matrix `which` (0 for an
 *     invalid or fp32 config, or for MOE_WS13/MOE_WS2 when Is == 0).
 *   moe_pack_weight: src is the row-major matrix (w13 [E,2I,H], w2 [E,H,I],
 *     ws13 [2Is,H] or ws2 [H,Is], bf16 or e4m3), dst a device buffer of
 *     moe_packed_bytes(cfg, which) bytes (tile padding is zero-filled). */
size_t moe_packed_bytes(const moe_config* cfg, moe_weight_id which);
moe_status moe_pack_weight(const moe_config* cfg, moe_weight_id which, const void* src,
                           void* dst, void* stream);

/* Reads the device error flag in ws, which each moe_permute / moe_forward
 * call rewrites; synchronises `stream`.  Returns MOE_OK, MOE_ERR_DEVICE_CHECK
 * if the last permutation on this workspace saw an expert index outside
 * [0, E) (flag bit 1) or if a completion wait inside moe_forward_decode_fused gave up after its bound
 * (bit 2: the outputs of that call are unreliable), or MOE_ERR_HIP. */
moe_status moe_get_device_error(void* ws, size_t ws_bytes, void* stream);

/* Kernel timer, for measurement.  While enabled, every kernel launch of the
 * library is bracketed by two HIP events recorded on the stream the kernel
 * runs on; `only` (NULL = all) restricts this to the kernels of that name
 * (names are those listed by moe_kernel_timer_read, e.g.
 * "grouped_gemm_bf16_packed<true>").  Enabling or disabling keeps what was
 * recorded so far.  The timer is process-wide and its calls are serialised
 * by a lock. */
moe_status moe_kernel_timer_enable(int on, const char* only);

/* Waits for every recorded event pair, sums durations per kernel name and
 * clears the record.  Returns the number n of distinct names; fills
 * names[i] (valid until the next read), total_ms[i] (summed event time) and
 * launches[i] for i < min(n, cap).  Any output pointer may be NULL. */
int moe_kernel_timer_read(int cap, const char** names, double* total_ms, int64_t* launches);

/* Static text for a status code. */
const char* moe_strerror(moe_status s);

/* Thread-local detail of the last failing call on this thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
