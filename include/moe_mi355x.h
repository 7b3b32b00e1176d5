/*
 * moe_mi355x.h - C ABI of the MoE expert-FFN layer hot path for MI355X (gfx950).
 *
 * One GPU's share of an expert-parallel mixture-of-experts layer: router top-k, routing
 * metadata computed on the device, a rowwise permute into contiguous expert buffers, a
 * device-scheduled grouped GEMM running the SwiGLU expert FFN (bf16 or MXFP8), a weighted
 * unpermute-combine, and the matching backward.
 *
 * The method is the MoE layer of the Olmo-core 3 training stack:
 *   [news] "Ai2 rebuilds Olmo's training stack for trillion-parameter MoEs"
 *          - lead paragraphs: a router sends each token to a small selection of FFN experts;
 *          - "Routing work stays on the GPU": rows are written straight into expert input
 *            buffers, routing metadata stays on the device so the CPU never waits for a copy
 *            back, and a grouped GEMM runs the many small expert products together;
 *          - "MXFP8 reduces compute and memory costs": 8-bit floats with one scale per small
 *            block of values.
 *   [card] "Supercharging Olmo-core for Efficient and Scalable MoE Training", "Summary":
 *          rowwise EP, GPU-resident routing metadata, device-scheduled grouped GEMMs, MXFP8.
 * The pages give no arithmetic; this library computes: softmax over all E experts, top-k
 * (descending logit, ties to the lower expert id), gates renormalised over the k chosen;
 * SwiGLU experts  A = silu(X W_gate^T) * (X W_up^T),  Yexp = A W_down^T  (no biases);
 * y[t] = sum_j gate[t,j] * Yexp[dest[t,j]]; MXFP8 = E4M3 elements + one E8M0 scale per 32
 * consecutive elements along each GEMM's contraction dimension.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller, row-major, contiguous,
 *     16-byte aligned.  They must stay valid until the enqueued work has completed.
 *   - bf16 tensors are passed as uint16_t bit patterns; E4M3 elements and E8M0 scales as
 *     uint8_t.  Indices are int32_t.  Floating-point accumulation is fp32; bf16 results are
 *     rounded to nearest-even once, when stored.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only enqueues work on
 *     it: no allocation, no synchronisation, no device-to-host copy.
 *   - Outputs are written, never accumulated into.  Results are deterministic: the same
 *     inputs give bit-identical outputs (no floating-point atomics anywhere).
 *   - Errors: a nonzero moe_status_t.  Every check on host-visible arguments happens before
 *     anything is enqueued.  Device-side contents are trusted (e.g. `dest` must come from
 *     moe_route_topk with the same T, k).  A failed kernel launch returns MOE_ERR_HIP; its
 *     text is in moe_last_error_string() (per calling thread).  Asynchronous faults surface
 *     at the caller's next synchronisation.
 *   - Shapes: 1 <= E <= 256, 1 <= k <= min(E, 16), T >= 1, T*k < 2^31; d and f multiples of
 *     64 for bf16, of 128 for the MXFP8 grouped GEMMs (their K steps are 128 elements, four
 *     E8M0 blocks); MXFP8 row tensors need their blocked dimension a multiple of 32.  Anything
 *     else: MOE_ERR_UNSUPPORTED.
 *
 * Layouts (n = T*k routed rows):
 *   x [T,d] bf16; router weight w_r [d,E] fp32; logits [T,E] fp32;
 *   w_gate, w_up [E,f,d] bf16; w_down [E,d,f] bf16 (output features first);
 *   xp, yexp, dyexp, dxp [n,d] bf16; g, u, a, dg, du [n,f] bf16;
 *   topk_idx, dest [T,k] int32; topk_gate, d_gate [T,k] fp32; counts [E]; offsets [E+1].
 *   GEMM scale layout: the E8M0 scales of an MXFP8 operand of the forward and dgrad grouped
 *   GEMMs -- a matrix of R rows quantised along K, one scale per row and 32-element block b --
 *   are stored as [K/(32G)][R][G]: the byte of row r, block b at ((b / G) * R + r) * G + b % G,
 *   G = 16 when K is a multiple of 512, 4 when of 128, else 1 (R * K/32 bytes either way;
 *   batched matrices each laid out alone).  A product's K step then reads the scales of its
 *   256-row tile as one contiguous run.  mxfp8_scales_to_gemm converts row-major scales.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_MI355X_ABI_VERSION 2

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* null pointer, negative size, misaligned pointer */
  MOE_ERR_UNSUPPORTED = 2,  /* a shape or mode outside the supported set */
  MOE_ERR_WORKSPACE = 3,    /* workspace missing or smaller than the *_workspace_bytes value */
  MOE_ERR_HIP = 4           /* a HIP launch failed; see moe_last_error_string() */
} moe_status_t;

enum { MOE_BF16 = 0, MOE_MXFP8 = 1 };

/* Version of this ABI (MOE_MI355X_ABI_VERSION of the built library). */
int moe_abi_version(void);
/* Static text for a status code. */
const char* moe_status_string(int status);
/* Text of the last MOE_ERR_* returned on the calling thread ("" if none). */
const char* moe_last_error_string(void);

/* ---------------------------------------------------------------- router */

/* logits[T,E] = x[T,d] (bf16) @ w_r[d,E] (fp32), fp32 accumulation.
 * The router's projection that scores every expert for every token ([news] lead paragraphs).
 * Used where the router weight is part of the layer (the router-driven workloads); callers that
 * already hold logits skip it.  Computed on the bf16 matrix cores from an exact three-part bf16
 * split of each fp32 value (fp32 accuracy; the summation order is the hardware's, not a
 * sequential dot product).  d must be a multiple of 8 and x 16-byte aligned (MOE_ERR_UNSUPPORTED
 * / MOE_ERR_INVALID_ARG otherwise); any E in [1, 256]. */
int moe_router_project(const uint16_t* x, const float* w_r, int T, int d, int E, float* logits,
                       void* stream);

/* Workspace for moe_router_project_bwd: the three bf16 parts of d_logits and of w_r (expert axis
 * zero-padded to a multiple of 64) and the split-K partial sums of dw_r. */
size_t moe_router_bwd_workspace_bytes(int T, int d, int E);

/* Backward of moe_router_project ([news] lead paragraphs: the stack trains the model, router
 * included, so the projection that scores the experts has a gradient):
 * dx_router[T,d] = d_logits @ w_r^T (fp32: the six products of the operands' bf16 parts that keep
 *                  fp32 accuracy),
 * dw_r[d,E] = x^T @ d_logits (fp32: x exact times the three parts of d_logits; summed over
 *             2048-token chunks in a fixed order, so repeated calls give identical bits).
 * Either output may be NULL to skip it; ws (>= moe_router_bwd_workspace_bytes) is needed whenever
 * one is requested (MOE_ERR_WORKSPACE otherwise); dx_router must be 16-byte aligned.  Argument
 * limits as moe_router_project. */
int moe_router_project_bwd(const uint16_t* x, const float* w_r, const float* d_logits, int T, int d,
                           int E, float* dx_router_or_null, float* dw_r_or_null, void* ws,
                           size_t ws_bytes, void* stream);

/* Workspace for moe_route_topk, from host scalars only. */
size_t moe_route_workspace_bytes(int T, int E, int k);

/* Router top-k and the device-resident routing metadata ([news] "Routing work stays on the GPU";
 * [card] "Summary": GPU-resident routing metadata).
 *   in   logits [T,E] fp32
 *   out  topk_idx [T,k]: the k largest logits per token, descending, ties to the lower expert id;
 *        topk_gate [T,k]: softmax over the chosen logits (= full softmax renormalised over them);
 *        probs [T,E] (optional): full softmax;
 *        counts [E]: rows per expert; offsets [E+1]: exclusive prefix sum (offsets[E] = T*k);
 *        offsets_pad [E+1] (optional): prefix sum of counts rounded up to `pad` (pad >= 1; the
 *        MXFP8 token-block layout takes 32, 64 or 128, and 128 is the fast choice: each
 *        128-token K step of the weight gradients then starts on a cache line);
 *        dest [T,k]: row of (t, j) in the expert-major buffer, rows ordered by expert, then token;
 *        row_token [T*k] (optional): the token of each row.
 *   ws   at least moe_route_workspace_bytes(T,E,k) bytes of device memory (contents ignored). */
int moe_route_topk(const float* logits, int T, int E, int k, int32_t* topk_idx, float* topk_gate,
                   float* probs_or_null, int32_t* counts, int32_t* offsets,
                   int32_t* offsets_pad_or_null, int pad, int32_t* dest, int32_t* row_token_or_null,
                   void* ws, size_t ws_bytes, void* stream);

/* moe_route_topk for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments (minus the workspace)
 * and bit-identical outputs; the per-block expert counts live instead in a fixed scratch array
 * that the library holds on every GPU it runs on (MOE_ROUTE_NOALLOC_SCRATCH_BYTES per GPU, kept
 * until the process ends; its device address is looked up on the first call on each device).
 * The call allocates nothing, clears nothing (every scratch entry it reads it has first written
 * in the same call) and needs ceil(T/64) * E * 4 <= MOE_ROUTE_NOALLOC_SCRATCH_BYTES (e.g.
 * T <= 262144 at E = 256), else MOE_ERR_UNSUPPORTED before anything is enqueued.
 * All calls on one GPU share its scratch: calls that can overlap on the device (other streams,
 * other host threads) race and give undefined results; serialise them on one stream. */
#define MOE_ROUTE_NOALLOC_SCRATCH_BYTES (4u << 20)
int moe_route_topk_noalloc(const float* logits, int T, int E, int k, int32_t* topk_idx,
                           float* topk_gate, float* probs_or_null, int32_t* counts, int32_t* offsets,
                           int32_t* offsets_pad_or_null, int pad, int32_t* dest,
                           int32_t* row_token_or_null, void* stream);

/* Backward of the renormalised gates with the selection held fixed ([news] lead paragraphs: the
 * router sends each token to a small selection of experts; training differentiates the gates
 * of that selection, not the discrete choice):
 * d_logits[t, idx[t,j]] = g_j * (dg_j - sum_i g_i dg_i), 0 for experts not chosen.  [T,E] fp32. */
int moe_route_topk_bwd(const float* topk_gate, const int32_t* topk_idx, const float* d_gate, int T,
                       int E, int k, float* d_logits, void* stream);

/* Router load-balancing score and balance statistics of the actual load ([news] "Four failure
 * modes from the report": a routing-balance score can improve while the workload grows less
 * balanced, "token gerrymandering"; the pages give no formula, this is the usual auxiliary
 * load-balancing loss of top-k routers):
 *   f_e = counts[e] / (T k),  P_e = mean over tokens of probs[t, e]
 *   out  p_mean [E] fp32 = P;  stats [4] fp32 = { aux = E sum_e f_e P_e, load_max = E max_e f_e,
 *        prob_max = E max_e P_e, load_cv = std_e(f) / mean_e(f) }
 *   in   probs [T,E] fp32 (moe_route_topk's full softmax), counts [E] int32 (its counts)
 *   ws   at least moe_route_balance_workspace_bytes(T, E) bytes (contents ignored).
 * Sums run in a fixed order: results are bit-reproducible. */
size_t moe_route_balance_workspace_bytes(int T, int E);
int moe_route_balance(const float* probs, const int32_t* counts, int T, int E, int k, float* p_mean,
                      float* stats, void* ws, size_t ws_bytes, void* stream);

/* moe_route_topk_bwd plus the gradient of weight * aux (moe_route_balance), counts held fixed:
 * d_logits[t,e] += p[t,e] (c_e - sum_e' p[t,e'] c_e'), c_e = weight E f_e / T.  Written, not
 * accumulated (the whole d_logits [T,E] is produced).  weight must be finite. */
int moe_route_topk_bwd_balance(const float* topk_gate, const int32_t* topk_idx, const float* d_gate,
                               const float* probs, const int32_t* counts, float weight, int T, int E,
                               int k, float* d_logits, void* stream);

/* ---------------------------------------------------------------- rows */

/* Rowwise permute: xp[dest[t,j], :] = x[t, :] for every slot j, a bit copy
 * ([news] "Routing work stays on the GPU": routed rows go straight into expert input buffers).
 *   dtype MOE_BF16:  x [T,d] bf16 -> xp [n,d] bf16; the scale pointers must be NULL.
 *   dtype MOE_MXFP8: x [T,d] E4M3 + x_scale [T,d/32] E8M0 -> xp [n,d] + xp_scale [n,d/32]. */
int moe_permute(int dtype, const void* x, const uint8_t* x_scale_or_null, const int32_t* dest,
                int T, int d, int k, void* xp, uint8_t* xp_scale_or_null, void* stream);

/* MXFP8 permute straight from bf16 x ([news] "Routing work stays on the GPU" and "MXFP8 reduces
 * compute and memory costs": routed rows go straight into the expert buffers, here already as
 * 8-bit codes with a scale per 32-element block): xpq[dest[t,j]] are the E4M3 row blocks of x[t]
 * and xps their scales in the GEMM scale layout (R = n, K = d), ready for the gate/up product --
 * the codes byte-identical to mxfp8_quantize(x, axis 0, scale_mode 0) followed by
 * moe_permute(MOE_MXFP8, ...), the scales the same bytes rearranged, without the token-major
 * quantised copy.
 *   in  x [T,d] bf16, dest [T,k] int32;  out xpq [n,d] E4M3, xps (n*d/32 bytes) E8M0 (n = T*k).
 * Same shape rules and errors as moe_permute (d a positive multiple of 64, 1 <= k <= 16);
 * x and xpq 16-byte aligned. */
int moe_permute_quant_mx(const uint16_t* x, const int32_t* dest, int T, int d, int k, uint8_t* xpq, uint8_t* xps,
                         void* stream);

/* Weighted unpermute-combine, the return path of the rowwise exchange ([news] "Routing work stays
 * on the GPU": routed rows live in expert buffers; the lead paragraphs: each token's output is
 * its chosen experts' outputs weighted by the router):
 * y[t] = sum_j topk_gate[t,j] * yexp[dest[t,j]], fp32 in slot order, bf16 out. */
int moe_unpermute_combine(const uint16_t* yexp, const float* topk_gate, const int32_t* dest, int T,
                          int d, int k, uint16_t* y, void* stream);

/* Backward of the combine (the gradient flows back along the same rowwise path, [news] "Routing
 * work stays on the GPU"): dyexp[dest[t,j]] = bf16(gate[t,j] * dy[t]);
 * d_gate[t,j] = <dy[t], yexp[dest[t,j]]> (fp32). */
int moe_unpermute_combine_bwd(const uint16_t* dy, const uint16_t* yexp, const float* topk_gate,
                              const int32_t* dest, int T, int d, int k, uint16_t* dyexp,
                              float* d_gate, void* stream);

/* The combine backward for MXFP8 backward products (fused producer): the rows of dyexp,
 * bf16(gate[t,j] * dy[t]), are formed in registers and leave only as MXFP8 row blocks along d,
 * byte-identical to mxfp8_quantize(dyexp, axis 0) of the bf16 rows, which are never written
 * (the scales in the GEMM scale layout, R = n, K = d, for the down dgrad).
 *   out  dyexp_q [n,d] E4M3, dyexp_scale (n*d/32 bytes) E8M0, row_gate [n] fp32 (row_gate[dest[t,j]] =
 *        gate[t,j], for mxfp8_quantize_grouped_gated), d_gate [T,k] fp32 as
 *        moe_unpermute_combine_bwd.  Shapes and alignment as moe_unpermute_combine_bwd. */
int moe_unpermute_combine_bwd_mx(const uint16_t* dy, const uint16_t* yexp, const float* topk_gate,
                                 const int32_t* dest, int T, int d, int k, uint8_t* dyexp_q,
                                 uint8_t* dyexp_scale, float* row_gate, float* d_gate, void* stream);

/* Backward of the permute: each token gathers the gradients of its k expert rows back from the
 * expert buffers ([news] "Routing work stays on the GPU", the rowwise write run in reverse):
 * dx[t] = sum_j dxp[dest[t,j]] (+ dx_addend[t] if given, the fp32 router-path term), fp32
 * accumulation, bf16 out. */
int moe_permute_bwd(const uint16_t* dxp, const int32_t* dest, int T, int d, int k,
                    const float* dx_addend_or_null, uint16_t* dx, void* stream);

/* The permute backward of a layer that owns its router, with the router's dx term computed in
 * the same kernel ([news] lead paragraphs: the router is trained with the layer, so x receives
 * the router path's gradient beside the experts'; "Routing work stays on the GPU"):
 *   dx[t] = bf16( dx_router[t] + dxp[dest[t,0]] + ... + dxp[dest[t,k-1]] ),
 * dx_router = d_logits @ w_r^T as moe_router_project_bwd computes it, summed in fp32 in that
 * order: byte-identical to moe_router_project_bwd (dx only) followed by moe_permute_bwd with its
 * dx_router as the addend, without the fp32 term going to memory and back (4*T*d bytes each way).
 *   dxp [T*k, d] bf16, dest [T,k], w_r [d,E] fp32, d_logits [T,E] fp32; dx [T,d] bf16 out.
 * ws: moe_router_bwd_workspace_bytes(T, d, E) bytes (MOE_ERR_WORKSPACE otherwise).  Limits:
 * T >= 1, 1 <= k <= 16, d a positive multiple of 64, 1 <= E <= 256, T*k < 2^31; dxp, dx and ws
 * 16-byte aligned. */
int moe_permute_bwd_router(const uint16_t* dxp, const int32_t* dest, int T, int d, int k, const float* w_r,
                           const float* d_logits, int E, uint16_t* dx, void* ws, size_t ws_bytes,
                           void* stream);

/* ---------------------------------------------------------------- MXFP8 quantisation */

/* MXFP8 block quantisation of a bf16 tensor in[batch][rows][cols]
 * ([news] "MXFP8 reduces compute and memory costs").  Per block of 32 bf16 values:
 * amax = max|v|; scale byte s = clamp(e - 8, -127, 127) + 127 (s = 0 when amax = 0), with
 *   scale_mode 0: e = floor(log2 amax) (the MX definition's rule; every other entry point of
 *                 this library quantises this way);
 *   scale_mode 1: e = floor(log2 amax) + 1 when amax's significand exceeds 1.75, else as mode 0:
 *                 the smallest power-of-two scale with amax / scale <= 448, so nothing saturates;
 * q = E4M3(v / 2^(s-127)) with round-to-nearest-even, magnitudes above 448 saturate to 448,
 * signs (and -0) kept.  Any other scale_mode: MOE_ERR_INVALID_ARG.
 *   axis 0: blocks along cols (the contiguous dim): q [batch][rows][cols], scale [batch][rows][cols/32]
 *           (cols % 32 == 0)
 *   axis 1: blocks along rows (the strided dim), output transposed:
 *           q [batch][cols][rows], scale [batch][cols][rows/32]   (rows % 32 == 0) */
int mxfp8_quantize(const uint16_t* in, int batch, int rows, int cols, int axis, int scale_mode,
                   uint8_t* q, uint8_t* scale, void* stream);

/* Both mxfp8_quantize layouts of one input from a single read of it: q as axis 0 and qT as axis 1,
 * bit-identical to the two separate calls, with the scales in the GEMM scale layout of each
 * matrix (scale: R = rows, K = cols; scaleT: R = cols, K = rows; the same bytes as the separate
 * calls' scales, rearranged).  For the expert weights, which the forward and the dgrad products
 * need quantised along each of their two dims ([news] "MXFP8 reduces compute and memory costs").
 * rows % 32 == 0 and cols % 64 == 0 (MOE_ERR_UNSUPPORTED otherwise); in, q, qT 16-byte aligned. */
int mxfp8_quantize_both(const uint16_t* in, int batch, int rows, int cols, uint8_t* q, uint8_t* scale,
                        uint8_t* qT, uint8_t* scaleT, void* stream);

/* Token-axis MXFP8 blocks restarting at each expert group: the weight-gradient operands, whose
 * product contracts over each expert's tokens ([news] "MXFP8 reduces compute and memory costs":
 * one scale per small block of values, here blocks of 32 tokens of one expert).
 * Row r of the grouped tensor is in[r] (row_token NULL; in is [n,C]) or in[row_token[r]]
 * (in is the token-major source [T,C]).  Expert e's rows [offsets[e], offsets[e+1]) go to
 * positions [offsets_pad[e], offsets_pad[e] + count_e) of a padded token axis; padding
 * positions up to offsets_pad[e+1] hold zeros, and so does everything from offsets_pad[E] to
 * n_pad_cap.  offsets_pad must be the padded prefix sum from moe_route_topk with pad 32, 64 or
 * 128 (scale blocks of 32 never straddle two experts, and offsets_pad[E] <= n_pad_cap).
 *   out qT [C, n_pad_cap] E4M3, n_pad_cap = n + 128*E rounded up to a multiple of 128
 *   (moe_mx_pad_cap); scaleT [n_pad_cap/32, C] E8M0, block-major: the scale of channel c and
 *   position block b is scaleT[b * C + c] (one weight-gradient K step of consecutive channels
 *   reads contiguous bytes). */
int mxfp8_quantize_grouped(const uint16_t* in, const int32_t* row_token_or_null,
                           const int32_t* offsets, const int32_t* offsets_pad, int E, int n, int C,
                           uint8_t* qT, uint8_t* scaleT, void* stream);

/* As mxfp8_quantize_grouped with row_token (required) and a per-row gate: grouped row r is
 * bf16(row_gate[r] * in[row_token[r]]) (fp32 product, round to nearest even) -- with `in` = dy and
 * row_gate from moe_unpermute_combine_bwd_mx, exactly the bf16 dyexp rows that call never
 * writes, so the output equals mxfp8_quantize_grouped(dyexp) byte for byte. */
int mxfp8_quantize_grouped_gated(const uint16_t* in, const int32_t* row_token, const float* row_gate,
                                 const int32_t* offsets, const int32_t* offsets_pad, int E, int n,
                                 int C, uint8_t* qT, uint8_t* scaleT, void* stream);

/* Both MXFP8 layouts of a grouped [n, C] bf16 tensor from one read ([news] "MXFP8 reduces compute
 * and memory costs": the expert products run on 8-bit operands with a scale per small block; the
 * backward's dG and dU feed one product contracting over C and one contracting over tokens):
 *   q_rows [n, C] E4M3 + s_rows (n*C/32 bytes) E8M0: row blocks as
 *     mxfp8_quantize(in, 1, n, C, axis 0, scale_mode 0), the scales in the GEMM scale layout
 *     (R = n, K = C);
 *   qT, scaleT: the grouped token blocks, byte-identical to mxfp8_quantize_grouped(in, NULL, ...).
 * Same requirements and errors as mxfp8_quantize_grouped (C a multiple of 64, 1 <= E <= 256),
 * plus q_rows and s_rows non-NULL and q_rows 16-byte aligned. */
int mxfp8_quantize_rows_grouped(const uint16_t* in, const int32_t* offsets, const int32_t* offsets_pad, int E,
                                int n, int C, uint8_t* q_rows, uint8_t* s_rows, uint8_t* qT, uint8_t* scaleT,
                                void* stream);

/* Row blocks of in [batch][rows][cols] as mxfp8_quantize axis 0 (scale_mode 0), the scales in the
 * GEMM scale layout of each matrix (R = rows, K = cols): an operand of the MXFP8 forward and dgrad
 * grouped GEMMs ([news] "MXFP8 reduces compute and memory costs").  cols % 32 == 0
 * (MOE_ERR_UNSUPPORTED otherwise); in and q 16-byte aligned. */
int mxfp8_quantize_gemm(const uint16_t* in, int batch, int rows, int cols, uint8_t* q, uint8_t* scale,
                        void* stream);

/* Row-major E8M0 scales in [batch][rows][K/32] (mxfp8_quantize axis 0, or axis 1 with rows and K
 * the transposed output's) rearranged into the GEMM scale layout; for callers that quantise with
 * mxfp8_quantize or permute with moe_permute and then call the MXFP8 grouped GEMMs.  K % 32 == 0
 * (MOE_ERR_UNSUPPORTED otherwise); in and out must not alias. */
int mxfp8_scales_to_gemm(const uint8_t* in, int batch, int rows, int K, uint8_t* out, void* stream);

/* Length of the padded token axis used by mxfp8_quantize_grouped and the MXFP8 backward:
 * n + 128*E rounded up to a multiple of 128 (room for any pad up to 128); -1 past 2^31 - 1. */
int moe_mx_pad_cap(int n, int E);

/* ---------------------------------------------------------------- grouped GEMMs */

/* Workspace for moe_grouped_gemm_swiglu / _bwd, from host scalars only. */
size_t moe_gg_workspace_bytes(int dtype, int E, int n, int d, int f);

/* Expert SwiGLU FFN as device-scheduled grouped GEMMs over the expert-major rows
 * ([news] "Routing work stays on the GPU": grouped GEMM; [card] "Summary": device-scheduled).
 * The per-expert row ranges are read from `offsets` on the device; the host never sees them.
 * For expert e, rows r in [offsets[e], offsets[e+1]):
 *   g = xp W_gate[e]^T, u = xp W_up[e]^T, a = silu(g) * u  (stored bf16; a from fp32 g, u),
 *   yexp = a W_down[e]^T.
 * dtype MOE_BF16:  xp, w_* bf16; all *_scale NULL.
 * dtype MOE_MXFP8: xp [n,d] E4M3 + xp_scale; w_gate, w_up [E,f,d] E4M3 + scales; w_down [E,d,f]
 *   E4M3 + scale (all blocks along the contraction dim; every scale in the GEMM scale layout:
 *   xp_scale R = n, K = d; each expert's w_gate / w_up scales R = f, K = d, w_down's R = d,
 *   K = f, as mxfp8_quantize_both writes them).
 *   a is quantised (rows, blocks along f) into the workspace before the second product.
 * Outputs g, u, a [n,f], yexp [n,d] bf16. */
int moe_grouped_gemm_swiglu(int dtype, int E, int n, int d, int f, const int32_t* offsets,
                            const void* xp, const uint8_t* xp_scale, const void* w_gate,
                            const uint8_t* w_gate_scale, const void* w_up,
                            const uint8_t* w_up_scale, const void* w_down,
                            const uint8_t* w_down_scale, uint16_t* g, uint16_t* u, uint16_t* a,
                            uint16_t* yexp, void* ws, size_t ws_bytes, void* stream);

/* The two products of moe_grouped_gemm_swiglu as separate calls (same arguments, same results):
 * gate_up runs the first grouped product with the SwiGLU epilogue (g, u, a); down runs the second
 * (yexp) from a bf16 `a` (for MOE_MXFP8 it first quantises a along f into the workspace, so it
 * needs moe_gg_workspace_bytes; gate_up needs none).  One kernel each for bf16. */
int moe_grouped_gemm_gate_up(int dtype, int E, int n, int d, int f, const int32_t* offsets,
                             const void* xp, const uint8_t* xp_scale, const void* w_gate,
                             const uint8_t* w_gate_scale, const void* w_up,
                             const uint8_t* w_up_scale, uint16_t* g, uint16_t* u, uint16_t* a,
                             void* stream);
int moe_grouped_gemm_down(int dtype, int E, int n, int d, int f, const int32_t* offsets,
                          const uint16_t* a, const void* w_down, const uint8_t* w_down_scale,
                          uint16_t* yexp, void* ws, size_t ws_bytes, void* stream);

/* The MXFP8 down product on an already quantised a ([news] "MXFP8 reduces compute and memory
 * costs": the expert products run on 8-bit operands with a scale per block of 32): yexp [n,d] bf16
 * = a W_down[e]^T per expert, with a_q [n,f] E4M3 and a_scale its row blocks in the GEMM scale
 * layout (R = n, K = f) -- mxfp8_quantize_rows_grouped's q_rows / s_rows, which also give a's
 * grouped token blocks for the down weight gradient from the same read -- and w_down [E,d,f]
 * E4M3 + scale as for moe_grouped_gemm_down.  Equals moe_grouped_gemm_down(MOE_MXFP8) on the bf16
 * a byte for byte; needs no workspace.  Shapes and errors as moe_grouped_gemm_down (MXFP8: d, f
 * multiples of 128); a_q, w_down, yexp and both scales 16-byte aligned. */
int moe_grouped_gemm_down_mx(int E, int n, int d, int f, const int32_t* offsets, const uint8_t* a_q,
                             const uint8_t* a_scale, const uint8_t* w_down, const uint8_t* w_down_scale,
                             uint16_t* yexp, void* stream);

/* Backward of moe_grouped_gemm_swiglu: the dgrad and wgrad grouped GEMMs that training the
 * experts needs ([news] "Routing work stays on the GPU": grouped GEMM; [card] "Summary":
 * device-scheduled grouped GEMMs in the training stack; "MXFP8 reduces compute and memory
 * costs" for the MXFP8 form).
 *   da = dyexp W_down[e];  dg = da * u * s * (1 + g (1 - s)),  du = da * g * s,  s = sigmoid(g)
 *   dxp = dg W_gate[e] + du W_up[e]
 *   dw_down[e] = dyexp_e^T a_e,  dw_gate[e] = dg_e^T xp_e,  dw_up[e] = du_e^T xp_e
 * Weight gradients of experts with no rows are written as zeros.
 * dtype MOE_BF16: x_rows = xp [n,d] bf16 (row_token NULL); w_* are the forward weights (bf16).
 * dtype MOE_MXFP8: x_rows = x [T,d] bf16 read through row_token (the token of each row);
 *   w_gate_t, w_up_t [E,d,f] and w_down_t [E,f,d] are the weights quantised along the dgrad
 *   contraction (mxfp8_quantize_both's qT per expert), with their scales in the GEMM scale
 *   layout (R = d, K = f; R = f, K = d); dyexp, dg|du are quantised along rows (GEMM-layout
 *   scales), and xp, a, dyexp, dg, du along grouped tokens (offsets_pad: pad 32, 64 or 128), into the
 *   workspace.
 * Outputs dg, du [n,f], dxp [n,d], dw_gate, dw_up [E,f,d], dw_down [E,d,f], all bf16. */
int moe_grouped_gemm_swiglu_bwd(int dtype, int E, int n, int d, int f, const int32_t* offsets,
                                const int32_t* offsets_pad_or_null,
                                const int32_t* row_token_or_null, const uint16_t* x_rows,
                                const uint16_t* g, const uint16_t* u, const uint16_t* a,
                                const uint16_t* dyexp, const void* w_gate,
                                const uint8_t* w_gate_scale, const void* w_up,
                                const uint8_t* w_up_scale, const void* w_down,
                                const uint8_t* w_down_scale, uint16_t* dg, uint16_t* du,
                                uint16_t* dxp, uint16_t* dw_gate, uint16_t* dw_up,
                                uint16_t* dw_down, void* ws, size_t ws_bytes, void* stream);

/* The four products of moe_grouped_gemm_swiglu_bwd as separate calls, one grouped GEMM kernel
 * each, on operands the caller has already put in the form the kernel reads (same results as the
 * composite, which is built from them; none needs a workspace).
 *
 * dgrad_down:    dg, du [n,f] from dyexp and the SwiGLU backward of (g, u) as above.
 *   bf16: dyexp [n,d], w_down_t = the forward W_down [E,d,f]; scales NULL.
 *   MXFP8: dyexp [n,d] E4M3 + dyexp_scale (row blocks along d; GEMM scale layout, R = n, K = d);
 *   w_down_t [E,f,d] E4M3 + scale (W_down quantised along d: mxfp8_quantize_both's qT / scaleT).
 * wgrad_down:    dw_down [E,d,f] = dyexp_e^T a_e.
 * dgrad_gate_up: dxp [n,d] = dg W_gate[e] + du W_up[e].
 *   bf16: dg, du [n,f]; w_gate_t, w_up_t = the forward weights [E,f,d]; scales NULL.
 *   MXFP8: dg, du [n,f] E4M3 + scales (GEMM scale layout, R = n, K = f); w_gate_t, w_up_t
 *   [E,d,f] E4M3 + scales (GEMM scale layout per expert, R = d, K = f).
 * wgrad_gate_up: dw_gate, dw_up [E,f,d] = dg_e^T xp_e, du_e^T xp_e.
 *   The wgrad operands ("*_t") are token-major:
 *   bf16: the row tensors themselves (dyexp [n,d], a [n,f], dg, du [n,f], xp [n,d]);
 *     offsets_pad and all scales NULL.
 *   MXFP8: mxfp8_quantize_grouped outputs, [C, P] E4M3 + block-major scales [P/32, C], with
 *     P = moe_mx_pad_cap(n, E) and offsets_pad the route's padded offsets (pad 32, 64 or 128).
 * Weight gradients of experts with no rows are written as zeros. */
int moe_grouped_gemm_dgrad_down(int dtype, int E, int n, int d, int f, const int32_t* offsets,
                                const void* dyexp, const uint8_t* dyexp_scale, const void* w_down_t,
                                const uint8_t* w_down_t_scale, const uint16_t* g,
                                const uint16_t* u, uint16_t* dg, uint16_t* du, void* stream);
int moe_grouped_gemm_wgrad_down(int dtype, int E, int n, int d, int f, const int32_t* offsets,
                                const int32_t* offsets_pad_or_null, const void* dyexp_t,
                                const uint8_t* dyexp_t_scale, const void* a_t,
                                const uint8_t* a_t_scale, uint16_t* dw_down, void* stream);
int moe_grouped_gemm_dgrad_gate_up(int dtype, int E, int n, int d, int f, const int32_t* offsets,
                                   const void* dg, const uint8_t* dg_scale, const void* du,
                                   const uint8_t* du_scale, const void* w_gate_t,
                                   const uint8_t* w_gate_t_scale, const void* w_up_t,
                                   const uint8_t* w_up_t_scale, uint16_t* dxp, void* stream);
int moe_grouped_gemm_wgrad_gate_up(int dtype, int E, int n, int d, int f, const int32_t* offsets,
                                   const int32_t* offsets_pad_or_null, const void* dg_t,
                                   const uint8_t* dg_t_scale, const void* du_t,
                                   const uint8_t* du_t_scale, const void* xp_t,
                                   const uint8_t* xp_t_scale, uint16_t* dw_gate, uint16_t* dw_up,
                                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
