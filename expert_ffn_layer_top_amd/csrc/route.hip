// Router top-k with renormalised gates, and the device-resident routing metadata.
//
// [news] "Ai2 rebuilds Olmo's training stack for trillion-parameter MoEs", lead paragraphs
// (a router picks a small set of experts per token) and "Routing work stays on the GPU"
// (routing metadata stays on the device, so the host never waits for a copy back).
//
// Three kernels, all sized from host scalars (no host sync):
//   route_topk_local   16 lanes per token, 64 tokens per 1024-thread block: k rounds of a
//                      16-lane arg-max over packed (order-preserving
//                      logit bits, inverted expert id) keys, the gates and the optional probs.
//                      Each (token, slot) then sets its token's bit in a per-expert 64-bit LDS
//                      mask (atomic OR, order-free), so the stable rank of a row among the
//                      block's rows of the same expert is a popcount of the lower bits, and
//                      the block's per-expert count is the mask's popcount.
//   route_scan         one block: per-expert exclusive scan over blocks (in place; 1024 / E'
//                      partial chains per expert, E' = E rounded up to a power of two),
//                      counts, offsets, padded offsets.
//   route_finalize     dest = offsets[e] + rows of e in earlier blocks + rank in block;
//                      row_token[dest] = token.
#include <cmath>
#include <mutex>

#include "common.h"

namespace moe {
namespace {

constexpr int kRouteBlock = 64;    // tokens per block (one bit each in a 64-bit mask)
constexpr int kGroup = 16;         // lanes per token
constexpr int kMaxK = 16;
constexpr int kMaxE = 256;
constexpr int kScanBatch = 16;   // hist loads in flight per scan thread

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

template <class T>
__device__ __forceinline__ T group_max(T v) {
#pragma unroll
  for (int o = kGroup / 2; o > 0; o >>= 1) {
    const T w = __shfl_xor(v, o, kGroup);
    v = w > v ? w : v;
  }
  return v;
}

__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = kGroup / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kGroup);
  return v;
}

// 16 lanes per token; lane g of a token holds experts g, g + 16, ... (NQ = ceil(E / 16) slots).
template <int NQ>
__device__ __forceinline__ void topk_token(const float* __restrict__ row, int E, int k, int g, int& my_e,
                                           float& my_gate, float* __restrict__ prow) {
  float v[NQ];
  unsigned long long key[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int e = g + kGroup * q;
    v[q] = (e < E) ? row[e] : 0.f;
    key[q] = (e < E) ? ((static_cast<unsigned long long>(float_key(v[q])) << 32) | (255u - e)) : 0ull;
  }
  my_e = 0;
  float my_l = 0.f, l0 = 0.f;
  for (int j = 0; j < k; ++j) {
    unsigned long long best = key[0];
#pragma unroll
    for (int q = 1; q < NQ; ++q) best = key[q] > best ? key[q] : best;
    best = group_max(best);
    const int e = 255 - static_cast<int>(best & 0xffu);
    const float lv = key_float(static_cast<uint32_t>(best >> 32));
    if (j == 0) l0 = lv;
    if (g == j) { my_e = e; my_l = lv; }
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      if (g + kGroup * q == e) key[q] = 0ull;
  }
  // gates: softmax over the chosen logits (the full-softmax denominator cancels)
  const float ex = (g < k) ? expf(my_l - l0) : 0.f;
  const float den = group_sum(ex);
  my_gate = ex / den;
  if (prow != nullptr) {
    float pe[NQ];
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      pe[q] = (g + kGroup * q < E) ? expf(v[q] - l0) : 0.f;
      s += pe[q];
    }
    s = group_sum(s);
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      if (g + kGroup * q < E) prow[g + kGroup * q] = pe[q] / s;
  }
}

template <int NQ>
__global__ __launch_bounds__(1024) void route_topk_local(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_gate, float* __restrict__ probs, int32_t* __restrict__ local_rank,
    int32_t* __restrict__ hist) {
  __shared__ unsigned long long s_mask[kMaxE];
  __shared__ int s_e[kRouteBlock][kMaxK];
  const int tid = threadIdx.x;
  const int g = tid & (kGroup - 1);
  const long long t0 = static_cast<long long>(blockIdx.x) * kRouteBlock;
  for (int e = tid; e < E; e += 1024) s_mask[e] = 0ull;
  __syncthreads();

  // ---- top-k, one token per 16 lanes
  {
    const int tl = tid >> 4;
    const long long t = t0 + tl;
    if (t < T) {   // uniform across the token's 16 lanes
      int my_e;
      float my_gate;
      topk_token<NQ>(logits + t * E, E, k, g, my_e, my_gate, probs != nullptr ? probs + t * E : nullptr);
      if (g < k) {
        topk_idx[t * k + g] = my_e;
        topk_gate[t * k + g] = my_gate;
        s_e[tl][g] = my_e;
        atomicOr(&s_mask[my_e], 1ull << tl);
      }
    }
  }
  __syncthreads();

  // ---- stable rank within the block: rows of the same expert from earlier tokens
  for (int i = tid; i < kRouteBlock * k; i += 1024) {
    const int tl = i / k, j = i - tl * k;
    const long long t = t0 + tl;
    if (t < T) {
      const int e = s_e[tl][j];
      local_rank[t * k + j] = __popcll(s_mask[e] & ((1ull << tl) - 1ull));
    }
  }
  for (int e = tid; e < E; e += 1024) hist[static_cast<long long>(blockIdx.x) * E + e] = __popcll(s_mask[e]);
}

// Single block of 1024 threads.  hist[b][e] becomes the exclusive prefix over blocks b' < b for
// expert e.  Thread (part, e) owns a contiguous run of blocks; the runs' sums are scanned
// through LDS, then every run rewrites its entries as prefixes.
__global__ __launch_bounds__(1024) void route_scan(int32_t* __restrict__ hist, int nb, int E, int ep_log2,
                                                   int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ offsets_pad, int pad) {
  __shared__ int s_part[1024];
  __shared__ int s_a[kMaxE];
  __shared__ int s_b[kMaxE];
  const int ep = 1 << ep_log2;                 // E rounded up to a power of two
  const int e = threadIdx.x & (ep - 1);
  const int part = threadIdx.x >> ep_log2;
  const int nparts = 1024 >> ep_log2;
  const int per = (nb + nparts - 1) / nparts;
  const int b0 = min(nb, part * per);
  const int b1 = min(nb, b0 + per);
  // the run's entries are read in batches of kScanBatch independent loads; a run that fits one
  // batch stays in registers for the rewrite
  int vals[kScanBatch];
  int sum = 0;
  for (int c0 = b0; c0 < b1; c0 += kScanBatch) {
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i)
      vals[i] = (e < E && c0 + i < b1) ? hist[static_cast<long long>(c0 + i) * E + e] : 0;
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i) sum += vals[i];
  }
  s_part[threadIdx.x] = sum;
  __syncthreads();
  int run = 0;
  for (int q = 0; q < part; ++q) run += s_part[(q << ep_log2) + e];
  if (e < E) {
    for (int c0 = b0; c0 < b1; c0 += kScanBatch) {
      if (b1 - b0 > kScanBatch) {
#pragma unroll
        for (int i = 0; i < kScanBatch; ++i)
          vals[i] = c0 + i < b1 ? hist[static_cast<long long>(c0 + i) * E + e] : 0;
      }
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) {
        if (c0 + i < b1) {
          hist[static_cast<long long>(c0 + i) * E + e] = run;
          run += vals[i];
        }
      }
    }
  }
  if (threadIdx.x < kMaxE) {
    const int ee = threadIdx.x;
    int total = 0;
    if (ee < E)
      for (int q = 0; q < nparts; ++q) total += s_part[(q << ep_log2) + ee];
    if (ee < E) counts[ee] = total;
    s_a[ee] = (ee < E) ? total : 0;
    s_b[ee] = (ee < E) ? (total + pad - 1) / pad * pad : 0;
  }
  __syncthreads();
  // inclusive Hillis-Steele scan over 256 entries (two arrays at once) by the first 256 threads
  const bool lead = threadIdx.x < kMaxE;
  const int ee = threadIdx.x;
  for (int o = 1; o < kMaxE; o <<= 1) {
    int a = 0, b = 0;
    if (lead && ee >= o) { a = s_a[ee - o]; b = s_b[ee - o]; }
    __syncthreads();
    if (lead) { s_a[ee] += a; s_b[ee] += b; }
    __syncthreads();
  }
  if (lead) {
    if (ee < E) {
      offsets[ee + 1] = s_a[ee];
      if (offsets_pad != nullptr) offsets_pad[ee + 1] = s_b[ee];
    }
    if (ee == 0) {
      offsets[0] = 0;
      if (offsets_pad != nullptr) offsets_pad[0] = 0;
    }
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

// One wave per token.  With `probs` given, the gradient of the balance score (weighted) is added:
// c_e = cscale * counts[e] (cscale = weight E / (T^2 k)) and the term p[t,e] (c_e - sum_e' p c).
__global__ __launch_bounds__(256) void route_topk_bwd_kernel(const float* __restrict__ gate,
                                                             const int32_t* __restrict__ idx,
                                                             const float* __restrict__ dgate, int T,
                                                             int E, int k, const float* __restrict__ probs,
                                                             const int32_t* __restrict__ counts, float cscale,
                                                             float* __restrict__ dlogits) {
  const long long t = static_cast<long long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  // balance term: this lane's experts e = lane + 64 i (E <= 256)
  float pb[kMaxE / 64], cb[kMaxE / 64];
  float pc = 0.f;
  if (probs != nullptr) {
#pragma unroll
    for (int i = 0; i < kMaxE / 64; ++i) {
      const int e = lane + 64 * i;
      pb[i] = e < E ? probs[t * E + e] : 0.f;
      cb[i] = e < E ? cscale * static_cast<float>(counts[e]) : 0.f;
      pc += pb[i] * cb[i];
    }
    pc = wave_sum(pc);
  }
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
#pragma unroll
  for (int i = 0; i < kMaxE / 64; ++i) {
    const int e = lane + 64 * i;
    if (e >= E) break;
    float v = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < k && ej[j] == e) v = vj[j];
    if (probs != nullptr) v += pb[i] * (cb[i] - pc);
    dlogits[t * E + e] = v;
  }
}

// ---- balance score: P_e = mean_t probs[t,e] by a fixed-order two-pass sum, then the statistics
constexpr int kBalTokens = 256;   // tokens per first-pass block

// part[b][e] = sum of probs[t][e] over block b's tokens (thread e sums column e; E <= 256).
__global__ __launch_bounds__(256) void balance_partial(const float* __restrict__ probs, int T, int E,
                                                       float* __restrict__ part) {
  const int e = threadIdx.x;
  if (e >= E) return;
  const long long t0 = static_cast<long long>(blockIdx.x) * kBalTokens;
  const long long t1 = min(static_cast<long long>(T), t0 + kBalTokens);
  float s = 0.f;
  for (long long t = t0; t < t1; ++t) s += probs[t * E + e];
  part[static_cast<long long>(blockIdx.x) * E + e] = s;
}

// One block: P_e, then aux = E sum f_e P_e, load_max = E max f, prob_max = E max P,
// load_cv = std(f) / mean(f), with f_e = counts[e] / (T k).
__global__ __launch_bounds__(256) void balance_finish(const float* __restrict__ part, int nb, int T, int E, int k,
                                                      const int32_t* __restrict__ counts, float* __restrict__ p_mean,
                                                      float* __restrict__ stats) {
  __shared__ float red[3][256];
  const int e = threadIdx.x;
  float P = 0.f, f = 0.f;
  if (e < E) {
    for (int b = 0; b < nb; ++b) P += part[static_cast<long long>(b) * E + e];
    P /= static_cast<float>(T);
    f = static_cast<float>(counts[e]) / (static_cast<float>(T) * static_cast<float>(k));
    p_mean[e] = P;
  }
  red[0][e] = f * P;
  red[1][e] = f;
  red[2][e] = P;
  __syncthreads();
  if (e == 0) {
    float fp = 0.f, fmax = 0.f, pmax = 0.f, fs = 0.f;
    for (int i = 0; i < E; ++i) {   // fixed order
      fp += red[0][i];
      fmax = fmaxf(fmax, red[1][i]);
      pmax = fmaxf(pmax, red[2][i]);
      fs += red[1][i];
    }
    const float mean = fs / E;
    float ss = 0.f;                 // squared deviations (no cancellation when the load is even)
    for (int i = 0; i < E; ++i) ss += (red[1][i] - mean) * (red[1][i] - mean);
    const float var = ss / E;
    stats[0] = E * fp;
    stats[1] = E * fmax;
    stats[2] = E * pmax;
    stats[3] = mean > 0.f ? sqrtf(var) / mean : 0.f;
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

namespace moe {
namespace {

// Host-visible checks of the route's arguments, shared by its entry points (everything but the
// workspace).
int check_route_args(const float* logits, int T, int E, int k, const int32_t* topk_idx, const float* topk_gate,
                     const float* probs, const int32_t* counts, const int32_t* offsets, const int32_t* offsets_pad,
                     int pad, const int32_t* dest, const int32_t* row_token) {
  if (int st = check_layer_shape(T, E, k)) return st;
  MOE_CHECK_PTR(logits); MOE_CHECK_PTR(topk_idx); MOE_CHECK_PTR(topk_gate);
  MOE_CHECK_PTR(counts); MOE_CHECK_PTR(offsets); MOE_CHECK_PTR(dest);
  MOE_CHECK_ALIGN(logits); MOE_CHECK_ALIGN(topk_idx); MOE_CHECK_ALIGN(topk_gate);
  MOE_CHECK_ALIGN(counts); MOE_CHECK_ALIGN(offsets); MOE_CHECK_ALIGN(dest);
  if (probs) MOE_CHECK_ALIGN(probs);
  if (offsets_pad) { MOE_CHECK_ALIGN(offsets_pad); MOE_REQUIRE(pad >= 1, MOE_ERR_INVALID_ARG, "pad must be >= 1"); }
  if (row_token) MOE_CHECK_ALIGN(row_token);
  return MOE_OK;
}

// The three kernels of the route, with `hist` (moe_route_workspace_bytes bytes of device memory)
// as the per-block expert counts.  route_topk_local writes every entry before route_scan reads
// it, so the buffer needs no clearing.
int enqueue_route(const float* logits, int T, int E, int k, int32_t* topk_idx, float* topk_gate, float* probs,
                  int32_t* counts, int32_t* offsets, int32_t* offsets_pad, int pad, int32_t* dest,
                  int32_t* row_token, int32_t* hist, hipStream_t s) {
  const int nb = (T + kRouteBlock - 1) / kRouteBlock;
  const int nq = (E + kGroup - 1) / kGroup;
  if (nq <= 1) route_topk_local<1><<<nb, 1024, 0, s>>>(logits, T, E, k, topk_idx, topk_gate, probs, dest, hist);
  else if (nq <= 2) route_topk_local<2><<<nb, 1024, 0, s>>>(logits, T, E, k, topk_idx, topk_gate, probs, dest, hist);
  else if (nq <= 4) route_topk_local<4><<<nb, 1024, 0, s>>>(logits, T, E, k, topk_idx, topk_gate, probs, dest, hist);
  else if (nq <= 8) route_topk_local<8><<<nb, 1024, 0, s>>>(logits, T, E, k, topk_idx, topk_gate, probs, dest, hist);
  else route_topk_local<16><<<nb, 1024, 0, s>>>(logits, T, E, k, topk_idx, topk_gate, probs, dest, hist);
  if (int st = check_launch("route_topk_local")) return st;
  int ep_log2 = 0;
  while ((1 << ep_log2) < E) ++ep_log2;
  route_scan<<<1, 1024, 0, s>>>(hist, nb, E, ep_log2, counts, offsets, offsets_pad, offsets_pad ? pad : 1);
  if (int st = check_launch("route_scan")) return st;
  const long long n = static_cast<long long>(T) * k;
  route_finalize<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(topk_idx, dest, hist, offsets, T, k, E, row_token);
  return check_launch("route_finalize");
}

// ---- the no-allocation variant's scratch: the per-block counts in a file-scope device array.
// Every GPU the library runs on holds its own copy until the process ends.  Host code never
// uses the array's name as an address (on the host it is only a stand-in for the symbol): the
// device address comes from hipGetSymbolAddress, looked up once per device with that device
// current, and every launch takes that pointer.
__device__ __align__(256) int32_t scratch[MOE_ROUTE_NOALLOC_SCRATCH_BYTES / sizeof(int32_t)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device.
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(MOE_ERR_HIP, "route (no-alloc): hipGetDevice: %s", hipGetErrorString(e));
  MOE_REQUIRE(dev >= 0 && dev < kMaxDevices, MOE_ERR_UNSUPPORTED, "route (no-alloc): device id %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return set_error(MOE_ERR_HIP, "route (no-alloc): hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" int moe_route_topk(const float* logits, int T, int E, int k, int32_t* topk_idx,
                              float* topk_gate, float* probs, int32_t* counts, int32_t* offsets,
                              int32_t* offsets_pad, int pad, int32_t* dest, int32_t* row_token,
                              void* ws, size_t ws_bytes, void* stream) {
  if (int st = check_route_args(logits, T, E, k, topk_idx, topk_gate, probs, counts, offsets, offsets_pad, pad, dest,
                                row_token))
    return st;
  const size_t need = moe_route_workspace_bytes(T, E, k);
  MOE_REQUIRE(ws != nullptr && ws_bytes >= need, MOE_ERR_WORKSPACE, "route workspace: need %zu bytes", need);
  MOE_CHECK_ALIGN(ws);
  return enqueue_route(logits, T, E, k, topk_idx, topk_gate, probs, counts, offsets, offsets_pad, pad, dest, row_token,
                       static_cast<int32_t*>(ws), as_stream(stream));
}

extern "C" int moe_route_topk_noalloc(const float* logits, int T, int E, int k, int32_t* topk_idx,
                                      float* topk_gate, float* probs, int32_t* counts, int32_t* offsets,
                                      int32_t* offsets_pad, int pad, int32_t* dest, int32_t* row_token,
                                      void* stream) {
  if (int st = check_route_args(logits, T, E, k, topk_idx, topk_gate, probs, counts, offsets, offsets_pad, pad, dest,
                                row_token))
    return st;
  const size_t need = moe_route_workspace_bytes(T, E, k);
  MOE_REQUIRE(need <= MOE_ROUTE_NOALLOC_SCRATCH_BYTES, MOE_ERR_UNSUPPORTED,
              "route (no-alloc): T=%d, E=%d needs %zu bytes of scratch, above the built-in %zu "
              "(ceil(T/64) * E * 4 must not exceed it); use moe_route_topk with a workspace",
              T, E, need, static_cast<size_t>(MOE_ROUTE_NOALLOC_SCRATCH_BYTES));
  void* ptr = nullptr;
  if (int st = scratch_address(&ptr)) return st;
  return enqueue_route(logits, T, E, k, topk_idx, topk_gate, probs, counts, offsets, offsets_pad, pad, dest, row_token,
                       static_cast<int32_t*>(ptr), as_stream(stream));
}

extern "C" int moe_route_topk_bwd(const float* topk_gate, const int32_t* topk_idx, const float* d_gate,
                                  int T, int E, int k, float* d_logits, void* stream) {
  if (int st = check_layer_shape(T, E, k)) return st;
  MOE_CHECK_PTR(topk_gate); MOE_CHECK_PTR(topk_idx); MOE_CHECK_PTR(d_gate); MOE_CHECK_PTR(d_logits);
  route_topk_bwd_kernel<<<(T + 3) / 4, 256, 0, as_stream(stream)>>>(topk_gate, topk_idx, d_gate, T, E, k, nullptr,
                                                                    nullptr, 0.f, d_logits);
  return check_launch("route_topk_bwd");
}

extern "C" int moe_route_topk_bwd_balance(const float* topk_gate, const int32_t* topk_idx, const float* d_gate,
                                          const float* probs, const int32_t* counts, float weight, int T, int E,
                                          int k, float* d_logits, void* stream) {
  if (int st = check_layer_shape(T, E, k)) return st;
  MOE_CHECK_PTR(topk_gate); MOE_CHECK_PTR(topk_idx); MOE_CHECK_PTR(d_gate); MOE_CHECK_PTR(d_logits);
  MOE_CHECK_PTR(probs); MOE_CHECK_PTR(counts);
  MOE_REQUIRE(std::isfinite(weight), MOE_ERR_INVALID_ARG, "balance weight must be finite");
  const double cscale = static_cast<double>(weight) * E / (static_cast<double>(T) * T * k);
  route_topk_bwd_kernel<<<(T + 3) / 4, 256, 0, as_stream(stream)>>>(topk_gate, topk_idx, d_gate, T, E, k, probs,
                                                                    counts, static_cast<float>(cscale), d_logits);
  return check_launch("route_topk_bwd_balance");
}

extern "C" size_t moe_route_balance_workspace_bytes(int T, int E) {
  if (T < 1 || E < 1) return 0;
  return static_cast<size_t>((T + kBalTokens - 1) / kBalTokens) * E * sizeof(float);
}

extern "C" int moe_route_balance(const float* probs, const int32_t* counts, int T, int E, int k, float* p_mean,
                                 float* stats, void* ws, size_t ws_bytes, void* stream) {
  if (int st = check_layer_shape(T, E, k)) return st;
  MOE_CHECK_PTR(probs); MOE_CHECK_PTR(counts); MOE_CHECK_PTR(p_mean); MOE_CHECK_PTR(stats);
  const size_t need = moe_route_balance_workspace_bytes(T, E);
  MOE_REQUIRE(ws != nullptr && ws_bytes >= need, MOE_ERR_WORKSPACE, "route balance workspace: need %zu bytes", need);
  const int nb = (T + kBalTokens - 1) / kBalTokens;
  hipStream_t s = as_stream(stream);
  balance_partial<<<nb, 256, 0, s>>>(probs, T, E, static_cast<float*>(ws));
  if (int st = check_launch("route_balance partial")) return st;
  balance_finish<<<1, 256, 0, s>>>(static_cast<const float*>(ws), nb, T, E, k, counts, p_mean, stats);
  return check_launch("route_balance finish");
}
