// Router projection and its backward, in fp32 ([news] "Ai2 rebuilds Olmo's training stack for
// trillion-parameter MoEs", lead paragraphs: the router scores the experts for every token).
//   forward   logits[T,E]    = x[T,d] @ w_r[d,E]
//   backward  dx_router[T,d] = d_logits[T,E] @ w_r^T
//             dw_r[d,E]      = x^T @ d_logits      (K = T: split over token chunks, partial sums
//                                                   reduced in a fixed order -> deterministic)
// These products have one small dimension (E <= 256) and stay in fp32, so they run on the vector
// ALUs: 64 x 64 output tiles, 256 threads with 4 x 4 outputs each, K steps of 32 staged in LDS
// with the next step's global loads issued before the current step's FMAs.
#include "common.h"

namespace moe {
namespace {

constexpr int TM = 64, TN = 64, TK = 32;

// C[M,N] (+)= sum_{k in [k_lo, k_hi)} A(m,k) B(k,n); A element (m,k) at A[m*a_sm + k*a_sk]
// (bf16 bits when A_BF16), B element (k,n) at B[k*b_sk + n*b_sn] (fp32).  C row-major, pitch N.
template <bool A_BF16, bool A_KFAST, bool B_KFAST>
__global__ __launch_bounds__(256) void small_gemm(const void* __restrict__ Av, long long a_sm, long long a_sk,
                                                  const float* __restrict__ B, long long b_sk, long long b_sn, int M,
                                                  int N, int K, int k_chunk, float* __restrict__ C,
                                                  long long c_split_stride) {
  __shared__ float As[TK][TM + 1];
  __shared__ float Bs[TK][TN + 1];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.x * TM, n0 = blockIdx.y * TN;
  const int k_lo = blockIdx.z * k_chunk;
  const int k_hi = min(K, k_lo + k_chunk);
  float* Cz = C + blockIdx.z * c_split_stride;
  const int tm = (tid & 15) * 4, tn = (tid >> 4) * 4;
  float acc[4][4] = {};

  // each thread stages 8 elements of A and 8 of B per K step: element e = tid + 256*i of the
  // TK x 64 tile, with consecutive threads walking the operand's unit-stride dimension
  float ra[8], rb[8];
  auto load = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = tid + 256 * i;
      const int ka = A_KFAST ? (e & 31) : (e >> 6), ma = A_KFAST ? (e >> 5) : (e & 63);
      const int kbb = B_KFAST ? (e & 31) : (e >> 6), nb = B_KFAST ? (e >> 5) : (e & 63);
      float av = 0.f, bv = 0.f;
      if (kb + ka < k_hi && m0 + ma < M) {
        const long long off = static_cast<long long>(m0 + ma) * a_sm + static_cast<long long>(kb + ka) * a_sk;
        av = A_BF16 ? bf16_to_f32(static_cast<const uint16_t*>(Av)[off]) : static_cast<const float*>(Av)[off];
      }
      if (kb + kbb < k_hi && n0 + nb < N)
        bv = B[static_cast<long long>(kb + kbb) * b_sk + static_cast<long long>(n0 + nb) * b_sn];
      ra[i] = av;
      rb[i] = bv;
    }
  };
  load(k_lo);
  for (int kb = k_lo; kb < k_hi; kb += TK) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = tid + 256 * i;
      if (A_KFAST) As[e & 31][e >> 5] = ra[i]; else As[e >> 6][e & 63] = ra[i];
      if (B_KFAST) Bs[e & 31][e >> 5] = rb[i]; else Bs[e >> 6][e & 63] = rb[i];
    }
    __syncthreads();
    if (kb + TK < k_hi) load(kb + TK);
#pragma unroll 8
    for (int kk = 0; kk < TK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = As[kk][tm + i]; b[i] = Bs[kk][tn + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + tm + i, n = n0 + tn + j;
      if (m < M && n < N) Cz[static_cast<long long>(m) * N + n] = acc[i][j];
    }
}

// out[i] = sum_s part[s][i], s ascending (fixed order)
__global__ __launch_bounds__(256) void reduce_splits(const float* __restrict__ part, int S, long long count,
                                                     float* __restrict__ out) {
  const long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= count) return;
  float s = 0.f;
  for (int z = 0; z < S; ++z) s += part[z * count + i];
  out[i] = s;
}

constexpr int kSplitTokens = 1024;   // tokens per split of the dw_r reduction

int n_splits(int T) { return (T + kSplitTokens - 1) / kSplitTokens; }

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_router_project(const uint16_t* x, const float* w_r, int T, int d, int E, float* logits,
                                  void* stream) {
  MOE_CHECK_PTR(x); MOE_CHECK_PTR(w_r); MOE_CHECK_PTR(logits);
  MOE_REQUIRE(T >= 1 && d >= 1 && E >= 1 && E <= 256, MOE_ERR_UNSUPPORTED, "need T, d >= 1 and 1 <= E <= 256");
  dim3 grid((T + TM - 1) / TM, (E + TN - 1) / TN, 1);
  small_gemm<true, true, false><<<grid, 256, 0, as_stream(stream)>>>(x, d, 1, w_r, E, 1, T, E, d, d, logits, 0);
  return check_launch("router_project");
}

extern "C" size_t moe_router_bwd_workspace_bytes(int T, int d, int E) {
  if (T < 1 || d < 1 || E < 1) return 0;
  return static_cast<size_t>(n_splits(T)) * d * E * sizeof(float);
}

extern "C" int moe_router_project_bwd(const uint16_t* x, const float* w_r, const float* d_logits, int T, int d,
                                      int E, float* dx_router, float* dw_r, void* ws, size_t ws_bytes,
                                      void* stream) {
  MOE_CHECK_PTR(x); MOE_CHECK_PTR(w_r); MOE_CHECK_PTR(d_logits);
  MOE_REQUIRE(T >= 1 && d >= 1 && E >= 1 && E <= 256, MOE_ERR_UNSUPPORTED, "need T, d >= 1 and 1 <= E <= 256");
  hipStream_t s = as_stream(stream);
  if (dw_r != nullptr) {
    const size_t need = moe_router_bwd_workspace_bytes(T, d, E);
    MOE_REQUIRE(ws != nullptr && ws_bytes >= need, MOE_ERR_WORKSPACE, "router bwd workspace: need %zu bytes", need);
  }
  if (dx_router != nullptr) {
    // dx[t, c] = sum_e dl[t, e] * w_r[c, e]
    dim3 grid((T + TM - 1) / TM, (d + TN - 1) / TN, 1);
    small_gemm<false, true, true><<<grid, 256, 0, s>>>(d_logits, E, 1, w_r, 1, E, T, d, E, E, dx_router, 0);
    if (int st = check_launch("router_project_bwd dx")) return st;
  }
  if (dw_r != nullptr) {
    // dw_r[c, e] = sum_t x[t, c] * dl[t, e], split over token chunks
    const int S = n_splits(T);
    float* part = static_cast<float*>(ws);
    dim3 grid((d + TM - 1) / TM, (E + TN - 1) / TN, S);
    small_gemm<true, false, false><<<grid, 256, 0, s>>>(x, 1, d, d_logits, E, 1, d, E, T, kSplitTokens, part,
                                          static_cast<long long>(d) * E);
    if (int st = check_launch("router_project_bwd dw partial")) return st;
    const long long count = static_cast<long long>(d) * E;
    reduce_splits<<<static_cast<unsigned>((count + 255) / 256), 256, 0, s>>>(part, S, count, dw_r);
    if (int st = check_launch("router_project_bwd dw reduce")) return st;
  }
  return MOE_OK;
}
