// Row-moving kernels of the layer: rowwise permute into the expert-major buffer, weighted
// unpermute-combine, and their backward.  All are HBM-bound row gathers/scatters.
//
// [news] "Ai2 rebuilds Olmo's training stack for trillion-parameter MoEs", "Routing work stays
// on the GPU": routed token rows are written straight into the experts' input buffers; the
// combine returns each token the gate-weighted sum of its experts' outputs.
//
// Layout of the work: one wave per token.  The wave reads the token's k destination rows once
// (lanes j < k load dest[t, j], then every lane gets all k by shuffles), then streams the row
// in 16-byte chunks (lane c handles chunks c, c + 64, ...), so every global access is a fully
// coalesced 1 KiB wave transaction.  Accumulation is fp32 in slot order j = 0..k-1.
#include "common.h"

namespace moe {
namespace {

constexpr int kMaxK = 16;
constexpr int kWaves = 4;   // tokens per 256-thread block

__device__ __forceinline__ void load_dest(const int32_t* __restrict__ dest, long long t, int k, int lane,
                                          long long (&rows)[kMaxK]) {
  const int mine = (lane < k) ? dest[t * k + lane] : 0;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) rows[j] = __shfl(mine, j, 64);
}

// Chunks per lane per batch: every lane issues all loads of a batch before using any, so each
// wave keeps several 1 KiB transactions per row in flight.  The two backward kernels gain from
// it; permute and combine keep one chunk per batch, where the higher occupancy serves better.
constexpr int kUFwd = 1;
constexpr int kUBwd = 4;

__global__ __launch_bounds__(256) void permute_kernel(const uint8_t* __restrict__ x, const uint8_t* __restrict__ xs,
                                                      const int32_t* __restrict__ dest, int T, int k,
                                                      long long pitch, long long spitch, uint8_t* __restrict__ xp,
                                                      uint8_t* __restrict__ xps) {
  const long long t = static_cast<long long>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  long long rows[kMaxK];
  load_dest(dest, t, k, lane, rows);
  const int chunks = static_cast<int>(pitch / 16);
  const uint4* src = reinterpret_cast<const uint4*>(x + t * pitch);
  for (int c0 = lane; c0 < chunks; c0 += 64 * kUFwd) {
    uint4 v[kUFwd];
#pragma unroll
    for (int u = 0; u < kUFwd; ++u)
      if (c0 + 64 * u < chunks) v[u] = src[c0 + 64 * u];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < k) {
        uint4* dst = reinterpret_cast<uint4*>(xp + rows[j] * pitch);
#pragma unroll
        for (int u = 0; u < kUFwd; ++u)
          if (c0 + 64 * u < chunks) dst[c0 + 64 * u] = v[u];
      }
    }
  }
  if (xs != nullptr) {
    // scale rows: d/32 bytes, an even count; copied in 2-byte units
    const uint16_t* sc = reinterpret_cast<const uint16_t*>(xs + t * spitch);
    for (int c = lane; c < spitch / 2; c += 64) {
      const uint16_t v = sc[c];
#pragma unroll
      for (int j = 0; j < kMaxK; ++j)
        if (j < k) reinterpret_cast<uint16_t*>(xps + rows[j] * spitch)[c] = v;
    }
  }
}

__device__ __forceinline__ void unpack8(const uint4& v, float (&f)[8]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                    pack_bf16x2(f[6], f[7]));
}

// y[t] = sum_j gate[t,j] * yexp[dest[t,j]]   (bf16 rows of d elements), fp32 in slot order
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ yexp, const float* __restrict__ gate,
                                                      const int32_t* __restrict__ dest, int T, int d, int k,
                                                      uint16_t* __restrict__ y) {
  const long long t = static_cast<long long>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  long long rows[kMaxK];
  load_dest(dest, t, k, lane, rows);
  const float gmine = (lane < k) ? gate[t * k + lane] : 0.f;
  float g[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) g[j] = __shfl(gmine, j, 64);
  const int chunks = d / 8;
  for (int c0 = lane; c0 < chunks; c0 += 64 * kUFwd) {
    float acc[kUFwd][8];
#pragma unroll
    for (int u = 0; u < kUFwd; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[u][i] = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < k) {
        const uint4* row = reinterpret_cast<const uint4*>(yexp + rows[j] * d);
        uint4 v[kUFwd];
#pragma unroll
        for (int u = 0; u < kUFwd; ++u)
          if (c0 + 64 * u < chunks) v[u] = row[c0 + 64 * u];
#pragma unroll
        for (int u = 0; u < kUFwd; ++u) {
          if (c0 + 64 * u < chunks) {
            float f[8];
            unpack8(v[u], f);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[u][i] = fmaf(g[j], f[i], acc[u][i]);
          }
        }
      }
    }
    uint4* out = reinterpret_cast<uint4*>(y + t * d);
#pragma unroll
    for (int u = 0; u < kUFwd; ++u)
      if (c0 + 64 * u < chunks) out[c0 + 64 * u] = pack8(acc[u]);
  }
}

// dyexp[dest[t,j]] = bf16(gate[t,j] * dy[t]);  d_gate[t,j] = <dy[t], yexp[dest[t,j]]>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const uint16_t* __restrict__ dy, const uint16_t* __restrict__ yexp,
                                                          const float* __restrict__ gate, const int32_t* __restrict__ dest,
                                                          int T, int d, int k, uint16_t* __restrict__ dyexp,
                                                          float* __restrict__ dgate) {
  const long long t = static_cast<long long>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  long long rows[kMaxK];
  load_dest(dest, t, k, lane, rows);
  const float gmine = (lane < k) ? gate[t * k + lane] : 0.f;
  float g[kMaxK], dot[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    g[j] = __shfl(gmine, j, 64);
    dot[j] = 0.f;
  }
  const int chunks = d / 8;
  const uint4* dyrow = reinterpret_cast<const uint4*>(dy + t * d);
  for (int c0 = lane; c0 < chunks; c0 += 64 * kUBwd) {
    uint4 vdy[kUBwd];
#pragma unroll
    for (int u = 0; u < kUBwd; ++u)
      if (c0 + 64 * u < chunks) vdy[u] = dyrow[c0 + 64 * u];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < k) {
        const uint4* yrow = reinterpret_cast<const uint4*>(yexp + rows[j] * d);
        uint4* orow = reinterpret_cast<uint4*>(dyexp + rows[j] * d);
        uint4 vy[kUBwd];
#pragma unroll
        for (int u = 0; u < kUBwd; ++u)
          if (c0 + 64 * u < chunks) vy[u] = yrow[c0 + 64 * u];
#pragma unroll
        for (int u = 0; u < kUBwd; ++u) {
          if (c0 + 64 * u < chunks) {
            float fdy[8], fy[8], o[8];
            unpack8(vdy[u], fdy);
            unpack8(vy[u], fy);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              dot[j] = fmaf(fdy[i], fy[i], dot[j]);
              o[i] = g[j] * fdy[i];
            }
            orow[c0 + 64 * u] = pack8(o);
          }
        }
      }
    }
  }
  float mine = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    const float s = wave_sum(dot[j]);   // every lane takes part, also for j >= k (zeros)
    if (lane == j) mine = s;
  }
  if (lane < k) dgate[t * k + lane] = mine;
}

// dx[t] = sum_j dxp[dest[t,j]] (+ addend[t])
__global__ __launch_bounds__(256) void permute_bwd_kernel(const uint16_t* __restrict__ dxp, const int32_t* __restrict__ dest,
                                                          int T, int d, int k, const float* __restrict__ addend,
                                                          uint16_t* __restrict__ dx) {
  const long long t = static_cast<long long>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  long long rows[kMaxK];
  load_dest(dest, t, k, lane, rows);
  const int chunks = d / 8;
  for (int c0 = lane; c0 < chunks; c0 += 64 * kUBwd) {
    float acc[kUBwd][8];
#pragma unroll
    for (int u = 0; u < kUBwd; ++u) {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[u][i] = 0.f;
      if (addend != nullptr && c0 + 64 * u < chunks) {
        const float4* a = reinterpret_cast<const float4*>(addend + t * d + 8 * (c0 + 64 * u));
        const float4 a0 = a[0], a1 = a[1];
        acc[u][0] = a0.x; acc[u][1] = a0.y; acc[u][2] = a0.z; acc[u][3] = a0.w;
        acc[u][4] = a1.x; acc[u][5] = a1.y; acc[u][6] = a1.z; acc[u][7] = a1.w;
      }
    }
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < k) {
        const uint4* row = reinterpret_cast<const uint4*>(dxp + rows[j] * d);
        uint4 v[kUBwd];
#pragma unroll
        for (int u = 0; u < kUBwd; ++u)
          if (c0 + 64 * u < chunks) v[u] = row[c0 + 64 * u];
#pragma unroll
        for (int u = 0; u < kUBwd; ++u) {
          if (c0 + 64 * u < chunks) {
            float f[8];
            unpack8(v[u], f);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[u][i] += f[i];
          }
        }
      }
    }
    uint4* out = reinterpret_cast<uint4*>(dx + t * d);
#pragma unroll
    for (int u = 0; u < kUBwd; ++u)
      if (c0 + 64 * u < chunks) out[c0 + 64 * u] = pack8(acc[u]);
  }
}

int check_rows(int T, int d, int k) {
  MOE_REQUIRE(T >= 1, MOE_ERR_UNSUPPORTED, "T must be >= 1");
  MOE_REQUIRE(k >= 1 && k <= kMaxK, MOE_ERR_UNSUPPORTED, "k must be in [1, 16]");
  MOE_REQUIRE(d >= 64 && d % 64 == 0, MOE_ERR_UNSUPPORTED, "d must be a positive multiple of 64");
  MOE_REQUIRE(static_cast<long long>(T) * k < (1LL << 31), MOE_ERR_UNSUPPORTED, "T*k must be < 2^31");
  return MOE_OK;
}

unsigned grid_for(int T) { return static_cast<unsigned>((T + kWaves - 1) / kWaves); }

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_permute(int dtype, const void* x, const uint8_t* x_scale, const int32_t* dest, int T, int d,
                           int k, void* xp, uint8_t* xp_scale, void* stream) {
  if (int st = check_rows(T, d, k)) return st;
  MOE_CHECK_PTR(x); MOE_CHECK_PTR(dest); MOE_CHECK_PTR(xp);
  MOE_CHECK_ALIGN(x); MOE_CHECK_ALIGN(xp);
  long long pitch, spitch = 0;
  if (dtype == MOE_BF16) {
    MOE_REQUIRE(x_scale == nullptr && xp_scale == nullptr, MOE_ERR_INVALID_ARG, "bf16 permute takes no scales");
    pitch = 2LL * d;
  } else if (dtype == MOE_MXFP8) {
    MOE_CHECK_PTR(x_scale); MOE_CHECK_PTR(xp_scale);
    MOE_REQUIRE((reinterpret_cast<uintptr_t>(x_scale) & 1u) == 0 && (reinterpret_cast<uintptr_t>(xp_scale) & 1u) == 0,
                MOE_ERR_INVALID_ARG, "scale pointers must be 2-byte aligned");
    pitch = d;
    spitch = d / 32;
  } else {
    return set_error(MOE_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  }
  permute_kernel<<<grid_for(T), 256, 0, as_stream(stream)>>>(
      static_cast<const uint8_t*>(x), x_scale, dest, T, k, pitch, spitch, static_cast<uint8_t*>(xp), xp_scale);
  return check_launch("permute");
}

extern "C" int moe_unpermute_combine(const uint16_t* yexp, const float* gate, const int32_t* dest, int T, int d,
                                     int k, uint16_t* y, void* stream) {
  if (int st = check_rows(T, d, k)) return st;
  MOE_CHECK_PTR(yexp); MOE_CHECK_PTR(gate); MOE_CHECK_PTR(dest); MOE_CHECK_PTR(y);
  MOE_CHECK_ALIGN(yexp); MOE_CHECK_ALIGN(y);
  combine_kernel<<<grid_for(T), 256, 0, as_stream(stream)>>>(yexp, gate, dest, T, d, k, y);
  return check_launch("combine");
}

extern "C" int moe_unpermute_combine_bwd(const uint16_t* dy, const uint16_t* yexp, const float* gate,
                                         const int32_t* dest, int T, int d, int k, uint16_t* dyexp, float* dgate,
                                         void* stream) {
  if (int st = check_rows(T, d, k)) return st;
  MOE_CHECK_PTR(dy); MOE_CHECK_PTR(yexp); MOE_CHECK_PTR(gate); MOE_CHECK_PTR(dest);
  MOE_CHECK_PTR(dyexp); MOE_CHECK_PTR(dgate);
  MOE_CHECK_ALIGN(dy); MOE_CHECK_ALIGN(yexp); MOE_CHECK_ALIGN(dyexp);
  combine_bwd_kernel<<<grid_for(T), 256, 0, as_stream(stream)>>>(dy, yexp, gate, dest, T, d, k, dyexp, dgate);
  return check_launch("combine_bwd");
}

extern "C" int moe_permute_bwd(const uint16_t* dxp, const int32_t* dest, int T, int d, int k,
                               const float* addend, uint16_t* dx, void* stream) {
  if (int st = check_rows(T, d, k)) return st;
  MOE_CHECK_PTR(dxp); MOE_CHECK_PTR(dest); MOE_CHECK_PTR(dx);
  MOE_CHECK_ALIGN(dxp); MOE_CHECK_ALIGN(dx);
  if (addend) MOE_CHECK_ALIGN(addend);
  permute_bwd_kernel<<<grid_for(T), 256, 0, as_stream(stream)>>>(dxp, dest, T, d, k, addend, dx);
  return check_launch("permute_bwd");
}
