// Router top-k with renormalised gates, and the device-resident routing metadata.
//
// [news] "Ai2 rebuilds Olmo's training stack for trillion-parameter MoEs", lead paragraphs
// (a router picks a small set of experts per token) and "Routing work stays on the GPU"
// (routing metadata stays on the device, so the host never waits for a copy back).
//
// Three kernels, all sized from host scalars (no host sync):
//   route_topk_local   one wave per token: k rounds of a wave-wide arg-max over packed
//                      (order-preserving logit bits, inverted expert id) keys, gates, probs;
//                      then, per block of 256 tokens, a stable rank of every (token, slot)
//                      among the block's rows of the same expert (ballot-based match on the
//                      expert-id bits + popcount under the lane mask) and the block's
//                      per-expert histogram.
//   route_scan         one block: per-expert exclusive scan over blocks (in place), counts,
//                      offsets, padded offsets.
//   route_finalize     dest = offsets[e] + rows of e in earlier blocks + rank in block;
//                      row_token[dest] = token.
#include <cmath>

#include "common.h"

namespace moe {
namespace {

constexpr int kRouteBlock = 256;   // tokens (and threads) per block
constexpr int kMaxK = 16;

// Order-preserving map of a float to uint32 (larger float -> larger key); -0 is folded to +0
// so that equal logits compare equal.
__device__ __forceinline__ uint32_t float_key(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7fffffffu) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_float(uint32_t key) {
  uint32_t u = (key & 0x80000000u) ? (key & 0x7fffffffu) : ~key;
  return __uint_as_float(u);
}

__global__ __launch_bounds__(kRouteBlock) void route_topk_local(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_gate, float* __restrict__ probs, int32_t* __restrict__ local_rank,
    int32_t* __restrict__ hist) {
  __shared__ int s_idx[kRouteBlock][kMaxK];
  __shared__ int s_cnt[kRouteBlock / 64][256];

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const long long t0 = static_cast<long long>(blockIdx.x) * kRouteBlock;

  for (int i = tid; i < (kRouteBlock / 64) * 256; i += kRouteBlock) (&s_cnt[0][0])[i] = 0;

  // ---- phase 1: top-k per token, one wave per token
  for (int i = 0; i < 64; ++i) {
    const int tl = w * 64 + i;
    const long long t = t0 + tl;
    if (t >= T) break;
    const float* row = logits + t * E;
    float v[4];
    unsigned long long key[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      v[q] = (e < E) ? row[e] : 0.f;
      key[q] = (e < E) ? ((static_cast<unsigned long long>(float_key(v[q])) << 32) | (255u - e)) : 0ull;
    }
    int my_e = 0;
    float my_l = 0.f;
    float l0 = 0.f;
    for (int j = 0; j < k; ++j) {
      unsigned long long best = key[0];
#pragma unroll
      for (int q = 1; q < 4; ++q) best = key[q] > best ? key[q] : best;
      best = wave_max_u64(best);
      const int e = 255 - static_cast<int>(best & 0xffu);
      const float lv = key_float(static_cast<uint32_t>(best >> 32));
      if (j == 0) l0 = lv;
      if (lane == j) { my_e = e; my_l = lv; }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (lane + 64 * q == e) key[q] = 0ull;
    }
    // gates: softmax over the chosen logits (the full-softmax denominator cancels)
    const float ex = (lane < k) ? expf(my_l - l0) : 0.f;
    const float den = wave_sum(ex);
    if (lane < k) {
      topk_idx[t * k + lane] = my_e;
      topk_gate[t * k + lane] = ex / den;
      s_idx[tl][lane] = my_e;
    }
    if (probs != nullptr) {
      float p[4];
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        p[q] = (lane + 64 * q < E) ? expf(v[q] - l0) : 0.f;
        s += p[q];
      }
      s = wave_sum(s);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (lane + 64 * q < E) probs[t * E + lane + 64 * q] = p[q] / s;
    }
  }
  __syncthreads();

  // ---- phase 2: stable rank within each 64-token group (wave), per expert
  const int tl = tid;
  const bool valid = (t0 + tl) < T;
  int my_exp[kMaxK], rank[kMaxK], total[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    my_exp[j] = (j < k && valid) ? s_idx[tl][j] : 256;
    rank[j] = 0;
    total[j] = 0;
  }
  const unsigned long long lt = __lanemask_lt();
#pragma unroll
  for (int jp = 0; jp < kMaxK; ++jp) {
    if (jp < k) {
    const int ej = my_exp[jp];
    unsigned long long b[9];
#pragma unroll
    for (int bit = 0; bit < 9; ++bit) b[bit] = __ballot((ej >> bit) & 1);
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      unsigned long long m = ~0ull;
#pragma unroll
      for (int bit = 0; bit < 9; ++bit) m &= ((my_exp[j] >> bit) & 1) ? b[bit] : ~b[bit];
      rank[j] += __popcll(m & lt);
      total[j] += __popcll(m);
    }
    }
  }
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j < k && valid && rank[j] == total[j] - 1) s_cnt[w][my_exp[j]] = total[j];
  __syncthreads();

  // ---- phase 3: rank within the block, and the block's histogram
  if (valid) {
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j >= k) continue;
      int base = 0;
      for (int wp = 0; wp < w; ++wp) base += s_cnt[wp][my_exp[j]];
      local_rank[(t0 + tl) * k + j] = base + rank[j];
    }
  }
  for (int e = tid; e < E; e += kRouteBlock) {
    int s = 0;
#pragma unroll
    for (int wp = 0; wp < kRouteBlock / 64; ++wp) s += s_cnt[wp][e];
    hist[static_cast<long long>(blockIdx.x) * E + e] = s;
  }
}

// Single block.  hist[b][e] becomes the exclusive prefix over blocks b' < b for expert e.
__global__ __launch_bounds__(256) void route_scan(int32_t* __restrict__ hist, int nb, int E,
                                                  int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ offsets_pad, int pad) {
  __shared__ int s_a[256];
  __shared__ int s_b[256];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int b = 0; b < nb; ++b) {
      const int v = hist[static_cast<long long>(b) * E + e];
      hist[static_cast<long long>(b) * E + e] = run;
      run += v;
    }
    counts[e] = run;
  }
  const int padded = (e < E) ? (run + pad - 1) / pad * pad : 0;
  s_a[e] = (e < E) ? run : 0;
  s_b[e] = padded;
  __syncthreads();
  // inclusive Hillis-Steele scan over 256 entries (two arrays at once)
  for (int o = 1; o < 256; o <<= 1) {
    const int a = (e >= o) ? s_a[e - o] : 0;
    const int b = (e >= o) ? s_b[e - o] : 0;
    __syncthreads();
    s_a[e] += a;
    s_b[e] += b;
    __syncthreads();
  }
  if (e < E) {
    offsets[e + 1] = s_a[e];
    if (offsets_pad != nullptr) offsets_pad[e + 1] = s_b[e];
  }
  if (e == 0) {
    offsets[0] = 0;
    if (offsets_pad != nullptr) offsets_pad[0] = 0;
  }
}

__global__ __launch_bounds__(256) void route_finalize(const int32_t* __restrict__ topk_idx,
                                                      int32_t* __restrict__ dest,
                                                      const int32_t* __restrict__ hist,
                                                      const int32_t* __restrict__ offsets, int T, int k,
                                                      int E, int32_t* __restrict__ row_token) {
  const long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<long long>(T) * k) return;
  const long long t = i / k;
  const int e = topk_idx[i];
  const long long b = t / kRouteBlock;
  const int r = offsets[e] + hist[b * E + e] + dest[i];
  dest[i] = r;
  if (row_token != nullptr) row_token[r] = static_cast<int32_t>(t);
}

__global__ __launch_bounds__(256) void route_topk_bwd_kernel(const float* __restrict__ gate,
                                                             const int32_t* __restrict__ idx,
                                                             const float* __restrict__ dgate, int T,
                                                             int E, int k, float* __restrict__ dlogits) {
  const long long t = static_cast<long long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  const float g_l = (lane < k) ? gate[t * k + lane] : 0.f;
  const float dg_l = (lane < k) ? dgate[t * k + lane] : 0.f;
  const int e_l = (lane < k) ? idx[t * k + lane] : -1;
  const float inner = wave_sum(g_l * dg_l);
  const float val_l = g_l * (dg_l - inner);
  // broadcast the k (expert, value) pairs to every lane while all lanes are active
  int ej[kMaxK];
  float vj[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    ej[j] = __shfl(e_l, j, 64);
    vj[j] = __shfl(val_l, j, 64);
  }
  for (int e = lane; e < E; e += 64) {
    float v = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < k && ej[j] == e) v = vj[j];
    dlogits[t * E + e] = v;
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_route_workspace_bytes(int T, int E, int k) {
  (void)k;
  if (T < 1 || E < 1) return 0;
  const size_t nb = (static_cast<size_t>(T) + kRouteBlock - 1) / kRouteBlock;
  return nb * static_cast<size_t>(E) * sizeof(int32_t);
}

extern "C" int moe_route_topk(const float* logits, int T, int E, int k, int32_t* topk_idx,
                              float* topk_gate, float* probs, int32_t* counts, int32_t* offsets,
                              int32_t* offsets_pad, int pad, int32_t* dest, int32_t* row_token,
                              void* ws, size_t ws_bytes, void* stream) {
  if (int st = check_layer_shape(T, E, k)) return st;
  MOE_CHECK_PTR(logits); MOE_CHECK_PTR(topk_idx); MOE_CHECK_PTR(topk_gate);
  MOE_CHECK_PTR(counts); MOE_CHECK_PTR(offsets); MOE_CHECK_PTR(dest);
  MOE_CHECK_ALIGN(logits); MOE_CHECK_ALIGN(topk_idx); MOE_CHECK_ALIGN(topk_gate);
  MOE_CHECK_ALIGN(counts); MOE_CHECK_ALIGN(offsets); MOE_CHECK_ALIGN(dest);
  if (probs) MOE_CHECK_ALIGN(probs);
  if (offsets_pad) { MOE_CHECK_ALIGN(offsets_pad); MOE_REQUIRE(pad >= 1, MOE_ERR_INVALID_ARG, "pad must be >= 1"); }
  if (row_token) MOE_CHECK_ALIGN(row_token);
  const size_t need = moe_route_workspace_bytes(T, E, k);
  MOE_REQUIRE(ws != nullptr && ws_bytes >= need, MOE_ERR_WORKSPACE, "route workspace: need %zu bytes", need);
  MOE_CHECK_ALIGN(ws);
  hipStream_t s = as_stream(stream);
  const int nb = (T + kRouteBlock - 1) / kRouteBlock;
  int32_t* hist = static_cast<int32_t*>(ws);
  route_topk_local<<<nb, kRouteBlock, 0, s>>>(logits, T, E, k, topk_idx, topk_gate, probs, dest, hist);
  if (int st = check_launch("route_topk_local")) return st;
  route_scan<<<1, 256, 0, s>>>(hist, nb, E, counts, offsets, offsets_pad, offsets_pad ? pad : 1);
  if (int st = check_launch("route_scan")) return st;
  const long long n = static_cast<long long>(T) * k;
  route_finalize<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(topk_idx, dest, hist, offsets, T, k, E, row_token);
  return check_launch("route_finalize");
}

extern "C" int moe_route_topk_bwd(const float* topk_gate, const int32_t* topk_idx, const float* d_gate,
                                  int T, int E, int k, float* d_logits, void* stream) {
  if (int st = check_layer_shape(T, E, k)) return st;
  MOE_CHECK_PTR(topk_gate); MOE_CHECK_PTR(topk_idx); MOE_CHECK_PTR(d_gate); MOE_CHECK_PTR(d_logits);
  route_topk_bwd_kernel<<<(T + 3) / 4, 256, 0, as_stream(stream)>>>(topk_gate, topk_idx, d_gate, T, E, k, d_logits);
  return check_launch("route_topk_bwd");
}
