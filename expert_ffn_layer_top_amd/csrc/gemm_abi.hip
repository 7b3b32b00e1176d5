// C ABI of the grouped GEMMs: argument checks, workspace sizing, dispatch to the bf16 or MXFP8
// kernels.  Everything here is host code; the work itself is enqueued on the caller's stream.
#include <initializer_list>

#include "common.h"

namespace moe {

int gg_bf16_gate_up(int E, int n, int d, int f, const int32_t* offsets, const uint16_t* xp, const uint16_t* wg,
                    const uint16_t* wu, uint16_t* g, uint16_t* u, uint16_t* a, hipStream_t s);
int gg_bf16_down(int E, int n, int d, int f, const int32_t* offsets, const uint16_t* a, const uint16_t* wd,
                 uint16_t* yexp, hipStream_t s);
int gg_bf16_backward(int E, int n, int d, int f, const int32_t* offsets, const uint16_t* xp, const uint16_t* g,
                     const uint16_t* u, const uint16_t* a, const uint16_t* dyexp, const uint16_t* wg,
                     const uint16_t* wu, const uint16_t* wd, uint16_t* dg, uint16_t* du, uint16_t* dxp,
                     uint16_t* dwg, uint16_t* dwu, uint16_t* dwd, hipStream_t s);
int gg_mx_gate_up(int E, int n, int d, int f, const int32_t* offsets, const uint8_t* xq, const uint8_t* xs,
                  const uint8_t* wgq, const uint8_t* wgs, const uint8_t* wuq, const uint8_t* wus, uint16_t* g,
                  uint16_t* u, uint16_t* a, hipStream_t s);
int gg_mx_down(int E, int n, int d, int f, const int32_t* offsets, const uint16_t* a, const uint8_t* wdq,
               const uint8_t* wds, uint16_t* yexp, uint8_t* ws, hipStream_t s);
int gg_mx_down_q(int E, int n, int d, int f, const int32_t* offsets, const uint8_t* aq, const uint8_t* as,
                 const uint8_t* wdq, const uint8_t* wds, uint16_t* yexp, hipStream_t s);
int gg_bf16_dgrad_down(int E, int n, int d, int f, const int32_t* offsets, const uint16_t* dyexp,
                       const uint16_t* wd, const uint16_t* g, const uint16_t* u, uint16_t* dg, uint16_t* du,
                       hipStream_t s);
int gg_bf16_wgrad_down(int E, int n, int d, int f, const int32_t* offsets, const uint16_t* dyexp,
                       const uint16_t* a, uint16_t* dwd, hipStream_t s);
int gg_bf16_dgrad_gate_up(int E, int n, int d, int f, const int32_t* offsets, const uint16_t* dg,
                          const uint16_t* du, const uint16_t* wg, const uint16_t* wu, uint16_t* dxp,
                          hipStream_t s);
int gg_bf16_wgrad_gate_up(int E, int n, int d, int f, const int32_t* offsets, const uint16_t* dg,
                          const uint16_t* du, const uint16_t* xp, uint16_t* dwg, uint16_t* dwu, hipStream_t s);
int gg_mx_dgrad_down(int E, int n, int d, int f, const int32_t* offsets, const uint8_t* dyq, const uint8_t* dys,
                     const uint8_t* wdtq, const uint8_t* wdts, const uint16_t* g, const uint16_t* u, uint16_t* dg,
                     uint16_t* du, hipStream_t s);
int gg_mx_wgrad_down(int E, int n, int d, int f, const int32_t* offsets, const int32_t* offsets_pad,
                     const uint8_t* dyT, const uint8_t* dyTs, const uint8_t* aT, const uint8_t* aTs, uint16_t* dwd,
                     hipStream_t s);
int gg_mx_dgrad_gate_up(int E, int n, int d, int f, const int32_t* offsets, const uint8_t* dgq, const uint8_t* dgs,
                        const uint8_t* duq, const uint8_t* dus, const uint8_t* wgtq, const uint8_t* wgts,
                        const uint8_t* wutq, const uint8_t* wuts, uint16_t* dxp, hipStream_t s);
int gg_mx_wgrad_gate_up(int E, int n, int d, int f, const int32_t* offsets, const int32_t* offsets_pad,
                        const uint8_t* dgT, const uint8_t* dgTs, const uint8_t* duT, const uint8_t* duTs,
                        const uint8_t* xT, const uint8_t* xTs, uint16_t* dwg, uint16_t* dwu, hipStream_t s);
size_t gg_mx_forward_ws(int n, int f);
size_t gg_mx_backward_ws(int E, int n, int d, int f);
int gg_mx_backward(int E, int n, int d, int f, const int32_t* offsets, const int32_t* offsets_pad,
                   const int32_t* row_token, const uint16_t* x, const uint16_t* g, const uint16_t* u,
                   const uint16_t* a, const uint16_t* dyexp, const uint8_t* wgtq, const uint8_t* wgts,
                   const uint8_t* wutq, const uint8_t* wuts, const uint8_t* wdtq, const uint8_t* wdts, uint16_t* dg,
                   uint16_t* du, uint16_t* dxp, uint16_t* dwg, uint16_t* dwu, uint16_t* dwd, uint8_t* ws,
                   hipStream_t s);

namespace {

int check_gg_shape(int dtype, int E, int n, int d, int f) {
  MOE_REQUIRE(dtype == MOE_BF16 || dtype == MOE_MXFP8, MOE_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  MOE_REQUIRE(E >= 1 && E <= 256, MOE_ERR_UNSUPPORTED, "E must be in [1, 256]");
  MOE_REQUIRE(n >= 1, MOE_ERR_UNSUPPORTED, "n must be >= 1");
  const int q = dtype == MOE_MXFP8 ? 128 : 64;
  MOE_REQUIRE(d >= q && d % q == 0 && f >= q && f % q == 0, MOE_ERR_UNSUPPORTED,
              "d and f must be positive multiples of %d for this dtype", q);
  // Everything the kernels of any call (the composite ones included) check at launch, checked
  // here first, so that an unsupported size is reported before anything is enqueued: buffer
  // offsets below 2^31 bytes for every operand, and tile counts below 2^31.
  const long long eb = dtype == MOE_MXFP8 ? 1 : 2;
  const long long dmax = d > f ? d : f;
  MOE_REQUIRE(static_cast<long long>(n) * dmax * eb < 0x7fffffffLL && static_cast<long long>(d) * f * eb < 0x7fffffffLL,
              MOE_ERR_UNSUPPORTED, "grouped GEMM: an operand exceeds 2 GiB");
  if (dtype == MOE_MXFP8) {
    const int P = moe_mx_pad_cap(n, E);
    MOE_REQUIRE(P > 0 && static_cast<long long>(P) * dmax < 0x7fffffffLL, MOE_ERR_UNSUPPORTED,
                "grouped GEMM: the padded token axis of the weight-gradient operands exceeds 2 GiB");
  }
  const long long mtiles = static_cast<long long>(n) / 256 + E;
  MOE_REQUIRE(mtiles * ((dmax + 127) / 128) < (1LL << 31) &&
                  static_cast<long long>(E) * 2 * ((f + 255) / 256) * ((d + 255) / 256) < (1LL << 31),
              MOE_ERR_UNSUPPORTED, "grouped GEMM: too many tiles");
  return MOE_OK;
}

// bf16 takes no scales; MXFP8 needs every one of them (non-null, 16-byte aligned).
int check_scales(int dtype, std::initializer_list<const void*> scales) {
  for (const void* p : scales) {
    if (dtype == MOE_BF16) {
      MOE_REQUIRE(p == nullptr, MOE_ERR_INVALID_ARG, "bf16 grouped GEMM takes no scales");
    } else {
      MOE_REQUIRE(p != nullptr, MOE_ERR_INVALID_ARG, "MXFP8 grouped GEMM: a scale pointer is NULL");
      MOE_REQUIRE((reinterpret_cast<uintptr_t>(p) & 15u) == 0, MOE_ERR_INVALID_ARG,
                  "MXFP8 grouped GEMM: a scale pointer is not 16-byte aligned");
    }
  }
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_gg_workspace_bytes(int dtype, int E, int n, int d, int f) {
  if (check_gg_shape(dtype, E, n, d, f) != MOE_OK) return 0;
  if (dtype == MOE_BF16) return 0;
  const size_t fw = gg_mx_forward_ws(n, f);
  const size_t bw = gg_mx_backward_ws(E, n, d, f);
  return fw > bw ? fw : bw;
}

extern "C" int moe_grouped_gemm_gate_up(int dtype, int E, int n, int d, int f, const int32_t* offsets,
                                        const void* xp, const uint8_t* xp_scale, const void* w_gate,
                                        const uint8_t* w_gate_scale, const void* w_up, const uint8_t* w_up_scale,
                                        uint16_t* g, uint16_t* u, uint16_t* a, void* stream) {
  if (int st = check_gg_shape(dtype, E, n, d, f)) return st;
  MOE_CHECK_PTR(offsets); MOE_CHECK_PTR(xp); MOE_CHECK_PTR(w_gate); MOE_CHECK_PTR(w_up);
  MOE_CHECK_PTR(g); MOE_CHECK_PTR(u); MOE_CHECK_PTR(a);
  MOE_CHECK_ALIGN(xp); MOE_CHECK_ALIGN(w_gate); MOE_CHECK_ALIGN(w_up);
  MOE_CHECK_ALIGN(g); MOE_CHECK_ALIGN(u); MOE_CHECK_ALIGN(a);
  hipStream_t s = as_stream(stream);
  if (dtype == MOE_BF16) {
    MOE_REQUIRE(!xp_scale && !w_gate_scale && !w_up_scale, MOE_ERR_INVALID_ARG, "bf16 grouped GEMM takes no scales");
    return gg_bf16_gate_up(E, n, d, f, offsets, static_cast<const uint16_t*>(xp), static_cast<const uint16_t*>(w_gate),
                           static_cast<const uint16_t*>(w_up), g, u, a, s);
  }
  MOE_CHECK_PTR(xp_scale); MOE_CHECK_PTR(w_gate_scale); MOE_CHECK_PTR(w_up_scale);
  MOE_CHECK_ALIGN(xp_scale); MOE_CHECK_ALIGN(w_gate_scale); MOE_CHECK_ALIGN(w_up_scale);
  return gg_mx_gate_up(E, n, d, f, offsets, static_cast<const uint8_t*>(xp), xp_scale,
                       static_cast<const uint8_t*>(w_gate), w_gate_scale, static_cast<const uint8_t*>(w_up),
                       w_up_scale, g, u, a, s);
}

extern "C" int moe_grouped_gemm_down(int dtype, int E, int n, int d, int f, const int32_t* offsets,
                                     const uint16_t* a, const void* w_down, const uint8_t* w_down_scale,
                                     uint16_t* yexp, void* ws, size_t ws_bytes, void* stream) {
  if (int st = check_gg_shape(dtype, E, n, d, f)) return st;
  MOE_CHECK_PTR(offsets); MOE_CHECK_PTR(a); MOE_CHECK_PTR(w_down); MOE_CHECK_PTR(yexp);
  MOE_CHECK_ALIGN(a); MOE_CHECK_ALIGN(w_down); MOE_CHECK_ALIGN(yexp);
  hipStream_t s = as_stream(stream);
  if (dtype == MOE_BF16) {
    MOE_REQUIRE(!w_down_scale, MOE_ERR_INVALID_ARG, "bf16 grouped GEMM takes no scales");
    return gg_bf16_down(E, n, d, f, offsets, a, static_cast<const uint16_t*>(w_down), yexp, s);
  }
  MOE_CHECK_PTR(w_down_scale);
  MOE_CHECK_ALIGN(w_down_scale);
  const size_t need = moe_gg_workspace_bytes(dtype, E, n, d, f);
  MOE_REQUIRE(ws != nullptr && ws_bytes >= need, MOE_ERR_WORKSPACE, "grouped GEMM workspace: need %zu bytes", need);
  MOE_CHECK_ALIGN(ws);
  return gg_mx_down(E, n, d, f, offsets, a, static_cast<const uint8_t*>(w_down), w_down_scale, yexp,
                    static_cast<uint8_t*>(ws), s);
}

extern "C" int moe_grouped_gemm_down_mx(int E, int n, int d, int f, const int32_t* offsets, const uint8_t* a_q,
                                        const uint8_t* a_scale, const uint8_t* w_down, const uint8_t* w_down_scale,
                                        uint16_t* yexp, void* stream) {
  if (int st = check_gg_shape(MOE_MXFP8, E, n, d, f)) return st;
  MOE_CHECK_PTR(offsets); MOE_CHECK_PTR(a_q); MOE_CHECK_PTR(w_down); MOE_CHECK_PTR(yexp);
  MOE_CHECK_ALIGN(a_q); MOE_CHECK_ALIGN(w_down); MOE_CHECK_ALIGN(yexp);
  if (int st = check_scales(MOE_MXFP8, {a_scale, w_down_scale})) return st;
  return gg_mx_down_q(E, n, d, f, offsets, a_q, a_scale, w_down, w_down_scale, yexp, as_stream(stream));
}

extern "C" int moe_grouped_gemm_swiglu(int dtype, int E, int n, int d, int f, const int32_t* offsets,
                                       const void* xp, const uint8_t* xp_scale, const void* w_gate,
                                       const uint8_t* w_gate_scale, const void* w_up, const uint8_t* w_up_scale,
                                       const void* w_down, const uint8_t* w_down_scale, uint16_t* g, uint16_t* u,
                                       uint16_t* a, uint16_t* yexp, void* ws, size_t ws_bytes, void* stream) {
  // argument checks of both halves happen before either enqueues anything
  if (int st = check_gg_shape(dtype, E, n, d, f)) return st;
  MOE_CHECK_PTR(w_down); MOE_CHECK_PTR(yexp);
  MOE_CHECK_ALIGN(w_down); MOE_CHECK_ALIGN(yexp);
  if (dtype == MOE_BF16) {
    MOE_REQUIRE(!w_down_scale, MOE_ERR_INVALID_ARG, "bf16 grouped GEMM takes no scales");
  } else {
    MOE_CHECK_PTR(w_down_scale);
    MOE_CHECK_ALIGN(w_down_scale);
    const size_t need = moe_gg_workspace_bytes(dtype, E, n, d, f);
    MOE_REQUIRE(ws != nullptr && ws_bytes >= need, MOE_ERR_WORKSPACE, "grouped GEMM workspace: need %zu bytes", need);
    MOE_CHECK_ALIGN(ws);
  }
  if (int st = moe_grouped_gemm_gate_up(dtype, E, n, d, f, offsets, xp, xp_scale, w_gate, w_gate_scale, w_up,
                                        w_up_scale, g, u, a, stream))
    return st;
  return moe_grouped_gemm_down(dtype, E, n, d, f, offsets, a, w_down, w_down_scale, yexp, ws, ws_bytes, stream);
}

extern "C" int moe_grouped_gemm_swiglu_bwd(int dtype, int E, int n, int d, int f, const int32_t* offsets,
                                           const int32_t* offsets_pad, const int32_t* row_token,
                                           const uint16_t* x_rows, const uint16_t* g, const uint16_t* u,
                                           const uint16_t* a, const uint16_t* dyexp, const void* w_gate,
                                           const uint8_t* w_gate_scale, const void* w_up, const uint8_t* w_up_scale,
                                           const void* w_down, const uint8_t* w_down_scale, uint16_t* dg, uint16_t* du,
                                           uint16_t* dxp, uint16_t* dw_gate, uint16_t* dw_up, uint16_t* dw_down,
                                           void* ws, size_t ws_bytes, void* stream) {
  if (int st = check_gg_shape(dtype, E, n, d, f)) return st;
  MOE_CHECK_PTR(offsets); MOE_CHECK_PTR(x_rows); MOE_CHECK_PTR(g); MOE_CHECK_PTR(u); MOE_CHECK_PTR(a);
  MOE_CHECK_PTR(dyexp); MOE_CHECK_PTR(w_gate); MOE_CHECK_PTR(w_up); MOE_CHECK_PTR(w_down);
  MOE_CHECK_PTR(dg); MOE_CHECK_PTR(du); MOE_CHECK_PTR(dxp); MOE_CHECK_PTR(dw_gate); MOE_CHECK_PTR(dw_up);
  MOE_CHECK_PTR(dw_down);
  MOE_CHECK_ALIGN(x_rows); MOE_CHECK_ALIGN(g); MOE_CHECK_ALIGN(u); MOE_CHECK_ALIGN(a); MOE_CHECK_ALIGN(dyexp);
  MOE_CHECK_ALIGN(w_gate); MOE_CHECK_ALIGN(w_up); MOE_CHECK_ALIGN(w_down); MOE_CHECK_ALIGN(dg); MOE_CHECK_ALIGN(du);
  MOE_CHECK_ALIGN(dxp); MOE_CHECK_ALIGN(dw_gate); MOE_CHECK_ALIGN(dw_up); MOE_CHECK_ALIGN(dw_down);
  hipStream_t s = as_stream(stream);
  if (dtype == MOE_BF16) {
    MOE_REQUIRE(!w_gate_scale && !w_up_scale && !w_down_scale, MOE_ERR_INVALID_ARG, "bf16 grouped GEMM takes no scales");
    MOE_REQUIRE(row_token == nullptr, MOE_ERR_INVALID_ARG, "bf16 backward reads xp directly (row_token must be NULL)");
    return gg_bf16_backward(E, n, d, f, offsets, x_rows, g, u, a, dyexp, static_cast<const uint16_t*>(w_gate),
                            static_cast<const uint16_t*>(w_up), static_cast<const uint16_t*>(w_down), dg, du, dxp,
                            dw_gate, dw_up, dw_down, s);
  }
  MOE_CHECK_PTR(offsets_pad); MOE_CHECK_PTR(row_token);
  MOE_CHECK_PTR(w_gate_scale); MOE_CHECK_PTR(w_up_scale); MOE_CHECK_PTR(w_down_scale);
  MOE_CHECK_ALIGN(w_gate_scale); MOE_CHECK_ALIGN(w_up_scale); MOE_CHECK_ALIGN(w_down_scale);
  MOE_REQUIRE(moe_mx_pad_cap(n, E) > 0, MOE_ERR_UNSUPPORTED, "padded token axis too long");
  const size_t need = moe_gg_workspace_bytes(dtype, E, n, d, f);
  MOE_REQUIRE(ws != nullptr && ws_bytes >= need, MOE_ERR_WORKSPACE, "grouped GEMM workspace: need %zu bytes", need);
  MOE_CHECK_ALIGN(ws);
  return gg_mx_backward(E, n, d, f, offsets, offsets_pad, row_token, x_rows, g, u, a, dyexp,
                        static_cast<const uint8_t*>(w_gate), w_gate_scale, static_cast<const uint8_t*>(w_up), w_up_scale,
                        static_cast<const uint8_t*>(w_down), w_down_scale, dg, du, dxp, dw_gate, dw_up, dw_down,
                        static_cast<uint8_t*>(ws), s);
}

extern "C" int moe_grouped_gemm_dgrad_down(int dtype, int E, int n, int d, int f, const int32_t* offsets,
                                           const void* dyexp, const uint8_t* dyexp_scale, const void* w_down_t,
                                           const uint8_t* w_down_t_scale, const uint16_t* g, const uint16_t* u,
                                           uint16_t* dg, uint16_t* du, void* stream) {
  if (int st = check_gg_shape(dtype, E, n, d, f)) return st;
  MOE_CHECK_PTR(offsets); MOE_CHECK_PTR(dyexp); MOE_CHECK_PTR(w_down_t); MOE_CHECK_PTR(g); MOE_CHECK_PTR(u);
  MOE_CHECK_PTR(dg); MOE_CHECK_PTR(du);
  MOE_CHECK_ALIGN(dyexp); MOE_CHECK_ALIGN(w_down_t); MOE_CHECK_ALIGN(g); MOE_CHECK_ALIGN(u);
  MOE_CHECK_ALIGN(dg); MOE_CHECK_ALIGN(du);
  if (int st = check_scales(dtype, {dyexp_scale, w_down_t_scale})) return st;
  hipStream_t s = as_stream(stream);
  if (dtype == MOE_BF16)
    return gg_bf16_dgrad_down(E, n, d, f, offsets, static_cast<const uint16_t*>(dyexp),
                              static_cast<const uint16_t*>(w_down_t), g, u, dg, du, s);
  return gg_mx_dgrad_down(E, n, d, f, offsets, static_cast<const uint8_t*>(dyexp), dyexp_scale,
                          static_cast<const uint8_t*>(w_down_t), w_down_t_scale, g, u, dg, du, s);
}

extern "C" int moe_grouped_gemm_wgrad_down(int dtype, int E, int n, int d, int f, const int32_t* offsets,
                                           const int32_t* offsets_pad, const void* dyexp_t,
                                           const uint8_t* dyexp_t_scale, const void* a_t, const uint8_t* a_t_scale,
                                           uint16_t* dw_down, void* stream) {
  if (int st = check_gg_shape(dtype, E, n, d, f)) return st;
  MOE_CHECK_PTR(offsets); MOE_CHECK_PTR(dyexp_t); MOE_CHECK_PTR(a_t); MOE_CHECK_PTR(dw_down);
  MOE_CHECK_ALIGN(dyexp_t); MOE_CHECK_ALIGN(a_t); MOE_CHECK_ALIGN(dw_down);
  if (int st = check_scales(dtype, {dyexp_t_scale, a_t_scale})) return st;
  hipStream_t s = as_stream(stream);
  if (dtype == MOE_BF16) {
    MOE_REQUIRE(offsets_pad == nullptr, MOE_ERR_INVALID_ARG, "bf16 wgrad reads unpadded rows (offsets_pad NULL)");
    return gg_bf16_wgrad_down(E, n, d, f, offsets, static_cast<const uint16_t*>(dyexp_t),
                              static_cast<const uint16_t*>(a_t), dw_down, s);
  }
  MOE_CHECK_PTR(offsets_pad);
  MOE_REQUIRE(moe_mx_pad_cap(n, E) > 0, MOE_ERR_UNSUPPORTED, "padded token axis too long");
  return gg_mx_wgrad_down(E, n, d, f, offsets, offsets_pad, static_cast<const uint8_t*>(dyexp_t), dyexp_t_scale,
                          static_cast<const uint8_t*>(a_t), a_t_scale, dw_down, s);
}

extern "C" int moe_grouped_gemm_dgrad_gate_up(int dtype, int E, int n, int d, int f, const int32_t* offsets,
                                              const void* dg, const uint8_t* dg_scale, const void* du,
                                              const uint8_t* du_scale, const void* w_gate_t,
                                              const uint8_t* w_gate_t_scale, const void* w_up_t,
                                              const uint8_t* w_up_t_scale, uint16_t* dxp, void* stream) {
  if (int st = check_gg_shape(dtype, E, n, d, f)) return st;
  MOE_CHECK_PTR(offsets); MOE_CHECK_PTR(dg); MOE_CHECK_PTR(du); MOE_CHECK_PTR(w_gate_t); MOE_CHECK_PTR(w_up_t);
  MOE_CHECK_PTR(dxp);
  MOE_CHECK_ALIGN(dg); MOE_CHECK_ALIGN(du); MOE_CHECK_ALIGN(w_gate_t); MOE_CHECK_ALIGN(w_up_t); MOE_CHECK_ALIGN(dxp);
  if (int st = check_scales(dtype, {dg_scale, du_scale, w_gate_t_scale, w_up_t_scale})) return st;
  hipStream_t s = as_stream(stream);
  if (dtype == MOE_BF16)
    return gg_bf16_dgrad_gate_up(E, n, d, f, offsets, static_cast<const uint16_t*>(dg),
                                 static_cast<const uint16_t*>(du), static_cast<const uint16_t*>(w_gate_t),
                                 static_cast<const uint16_t*>(w_up_t), dxp, s);
  return gg_mx_dgrad_gate_up(E, n, d, f, offsets, static_cast<const uint8_t*>(dg), dg_scale,
                             static_cast<const uint8_t*>(du), du_scale, static_cast<const uint8_t*>(w_gate_t),
                             w_gate_t_scale, static_cast<const uint8_t*>(w_up_t), w_up_t_scale, dxp, s);
}

extern "C" int moe_grouped_gemm_wgrad_gate_up(int dtype, int E, int n, int d, int f, const int32_t* offsets,
                                              const int32_t* offsets_pad, const void* dg_t,
                                              const uint8_t* dg_t_scale, const void* du_t,
                                              const uint8_t* du_t_scale, const void* xp_t,
                                              const uint8_t* xp_t_scale, uint16_t* dw_gate, uint16_t* dw_up,
                                              void* stream) {
  if (int st = check_gg_shape(dtype, E, n, d, f)) return st;
  MOE_CHECK_PTR(offsets); MOE_CHECK_PTR(dg_t); MOE_CHECK_PTR(du_t); MOE_CHECK_PTR(xp_t);
  MOE_CHECK_PTR(dw_gate); MOE_CHECK_PTR(dw_up);
  MOE_CHECK_ALIGN(dg_t); MOE_CHECK_ALIGN(du_t); MOE_CHECK_ALIGN(xp_t); MOE_CHECK_ALIGN(dw_gate);
  MOE_CHECK_ALIGN(dw_up);
  if (int st = check_scales(dtype, {dg_t_scale, du_t_scale, xp_t_scale})) return st;
  hipStream_t s = as_stream(stream);
  if (dtype == MOE_BF16) {
    MOE_REQUIRE(offsets_pad == nullptr, MOE_ERR_INVALID_ARG, "bf16 wgrad reads unpadded rows (offsets_pad NULL)");
    return gg_bf16_wgrad_gate_up(E, n, d, f, offsets, static_cast<const uint16_t*>(dg_t),
                                 static_cast<const uint16_t*>(du_t), static_cast<const uint16_t*>(xp_t), dw_gate,
                                 dw_up, s);
  }
  MOE_CHECK_PTR(offsets_pad);
  MOE_REQUIRE(moe_mx_pad_cap(n, E) > 0, MOE_ERR_UNSUPPORTED, "padded token axis too long");
  return gg_mx_wgrad_gate_up(E, n, d, f, offsets, offsets_pad, static_cast<const uint8_t*>(dg_t), dg_t_scale,
                             static_cast<const uint8_t*>(du_t), du_t_scale, static_cast<const uint8_t*>(xp_t),
                             xp_t_scale, dw_gate, dw_up, s);
}
