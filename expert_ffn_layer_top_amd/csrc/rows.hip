// Row-moving kernels of the layer: rowwise permute into the expert-major buffer, weighted
// unpermute-combine, and their backward.  All are HBM-bound row gathers/scatters.
//
// [news] "Ai2 rebuilds Olmo's training stack for trillion-parameter MoEs", "Routing work stays
// on the GPU": routed token rows are written straight into the experts' input buffers; the
// combine returns each token the gate-weighted sum of its experts' outputs.
//
// Layout of the work: the permute, the combine and the permute backward give each wave one
// 1 KiB segment of one token's row (lane c moves 16-byte chunk c of it), so every global access
// is a fully coalesced 1 KiB wave transaction, each lane has its k row accesses in flight at once,
// and the many small work items keep a launch's last round short.  The token's k destination
// rows (and gates) are read once per wave (lanes j < k load dest[t, j]) and kept in scalar
// registers.  The combine backward, which also reduces whole rows to dot products, gives each
// wave one token.  Accumulation is fp32 in slot order j = 0..k-1.
#include "mx_common.h"

namespace moe {
namespace {

constexpr int kMaxK = 16;
constexpr int kWaves = 4;   // tokens per 256-thread block

// Chunks per lane per batch in the combine backward (one wave per token, for its row dot
// products): every lane issues all loads of a batch before using any, so each wave keeps several
// 1 KiB transactions per row in flight.
constexpr int kUBwd = 4;

// Work items of the permute, the combine and the permute backward: one 1 KiB segment (64 lanes
// x 16 bytes) of one token's row per wave, four waves to a 256-thread block, the segments of a
// token on consecutive waves.  Small items keep the last round of a launch short; each lane keeps
// its k row loads in flight together.
constexpr int kSegChunks = 64;   // 16-byte chunks per segment

struct SegItem {
  long long t;   // token (wave-uniform)
  int c;         // this lane's 16-byte chunk within the row
};

__device__ __forceinline__ SegItem seg_item(int nseg) {
  const long long i = static_cast<long long>(blockIdx.x) * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  SegItem it;
  it.t = i / nseg;
  it.c = static_cast<int>(i - it.t * nseg) * kSegChunks + (threadIdx.x & 63);
  return it;
}

// The token's k destination rows (and optionally its k gates), as wave-uniform scalars.
template <int KM>
__device__ __forceinline__ void dest_rows(const int32_t* __restrict__ dest, long long t, int k, int (&rows)[KM]) {
  const int lane = threadIdx.x & 63;
  const int mine = (lane < k) ? dest[t * k + lane] : 0;
#pragma unroll
  for (int j = 0; j < KM; ++j) rows[j] = __builtin_amdgcn_readlane(mine, j);
}

template <int KM>
__device__ __forceinline__ void gates_of(const float* __restrict__ gate, long long t, int k, float (&g)[KM]) {
  const int lane = threadIdx.x & 63;
  const float mine = (lane < k) ? gate[t * k + lane] : 0.f;
#pragma unroll
  for (int j = 0; j < KM; ++j) g[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), j));
}

// xp[dest[t,j]] = x[t] for rows of `pitch` bytes (bf16, or E4M3 bytes plus a scale row of
// `spitch` bytes, copied by the token's first segment).
template <int KM>
__global__ __launch_bounds__(256) void permute_kernel(const uint8_t* __restrict__ x, const uint8_t* __restrict__ xs,
                                                      const int32_t* __restrict__ dest, int T, int k, int nseg,
                                                      long long pitch, long long spitch, uint8_t* __restrict__ xp,
                                                      uint8_t* __restrict__ xps) {
  const SegItem it = seg_item(nseg);
  if (it.t >= T) return;
  int rows[KM];
  dest_rows<KM>(dest, it.t, k, rows);
  const int chunks = static_cast<int>(pitch / 16);
  if (it.c < chunks) {
    const uint4 v = reinterpret_cast<const uint4*>(x + it.t * pitch)[it.c];
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (j < k) reinterpret_cast<uint4*>(xp + rows[j] * pitch)[it.c] = v;
  }
  if (xs != nullptr && it.c < kSegChunks) {
    // scale rows: d/32 bytes, an even count; copied in 2-byte units
    const uint16_t* sc = reinterpret_cast<const uint16_t*>(xs + it.t * spitch);
    for (int c = it.c; c < spitch / 2; c += 64) {
      const uint16_t v = sc[c];
#pragma unroll
      for (int j = 0; j < KM; ++j)
        if (j < k) reinterpret_cast<uint16_t*>(xps + rows[j] * spitch)[c] = v;
    }
  }
}

// MXFP8 permute straight from bf16 x: xpq[dest[t,j]] = the E4M3 row blocks of x[t], their E8M0
// scales into xps in the GEMM layout (mx_gemm_scale_index, R = T k), so the quantised rows go into
// the expert buffers, ready for the gate/up product, without a token-major quantised copy.  A 32-element block is 4 adjacent
// lanes of the wave's 1 KiB segment (amax by two shuffles); each lane writes 8 codes per
// destination and the block's first lane its scale byte.  d a multiple of 32.
template <int KM>
__global__ __launch_bounds__(256) void permute_mx_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ dest,
                                                         int T, int d, int k, int nseg, uint8_t* __restrict__ xpq,
                                                         uint8_t* __restrict__ xps) {
  const SegItem it = seg_item(nseg);
  if (it.t >= T) return;
  int rows[KM];
  dest_rows<KM>(dest, it.t, k, rows);
  const int e0 = 8 * it.c;                      // first element of this lane's chunk
  const bool live = e0 < d;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (live) v = *reinterpret_cast<const uint4*>(x + it.t * d + e0);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t amax = 0;
#pragma unroll
  for (int h = 0; h < 4; ++h) amax = max(amax, max(w[h] & 0x7fffu, (w[h] >> 16) & 0x7fffu));
  amax = max(amax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(amax), 1, 64)));
  amax = max(amax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(amax), 2, 64)));
  if (!live) return;
  const int sh = mx_shared_exp(amax);
  const uint2 o = make_uint2(mx_encode4(w[0] & 0xffffu, w[0] >> 16, w[1] & 0xffffu, w[1] >> 16, sh),
                             mx_encode4(w[2] & 0xffffu, w[2] >> 16, w[3] & 0xffffu, w[3] >> 16, sh));
  const uint8_t sb = static_cast<uint8_t>(sh + 127);
  const long long n = static_cast<long long>(T) * k;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    if (j < k) {
      *reinterpret_cast<uint2*>(xpq + static_cast<long long>(rows[j]) * d + e0) = o;
      if ((it.c & 3) == 0) xps[mx_gemm_scale_index(rows[j], e0 / 32, n, d)] = sb;
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
template <int KM>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ yexp, const float* __restrict__ gate,
                                                      const int32_t* __restrict__ dest, int T, int d, int k, int nseg,
                                                      uint16_t* __restrict__ y) {
  const SegItem it = seg_item(nseg);
  if (it.t >= T) return;
  int rows[KM];
  float g[KM];
  dest_rows<KM>(dest, it.t, k, rows);
  gates_of<KM>(gate, it.t, k, g);
  const int chunks = d / 8;
  if (it.c >= chunks) return;
  uint4 v[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j)
    if (j < k) v[j] = reinterpret_cast<const uint4*>(yexp + static_cast<long long>(rows[j]) * d)[it.c];
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    if (j < k) {
      float f[8];
      unpack8(v[j], f);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(g[j], f[i], acc[i]);
    }
  }
  reinterpret_cast<uint4*>(y + it.t * d)[it.c] = pack8(acc);
}

// dyexp[dest[t,j]] = bf16(gate[t,j] * dy[t]);  d_gate[t,j] = <dy[t], yexp[dest[t,j]]>
template <int KM>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const uint16_t* __restrict__ dy, const uint16_t* __restrict__ yexp,
                                                          const float* __restrict__ gate, const int32_t* __restrict__ dest,
                                                          int T, int d, int k, uint16_t* __restrict__ dyexp,
                                                          float* __restrict__ dgate) {
  const long long t = static_cast<long long>(blockIdx.x) * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  int rows[KM];
  float g[KM], dot[KM];
  dest_rows<KM>(dest, t, k, rows);
  gates_of<KM>(gate, t, k, g);
#pragma unroll
  for (int j = 0; j < KM; ++j) dot[j] = 0.f;
  const int chunks = d / 8;
  const uint4* dyrow = reinterpret_cast<const uint4*>(dy + t * d);
  for (int c0 = lane; c0 < chunks; c0 += 64 * kUBwd) {
    uint4 vdy[kUBwd];
#pragma unroll
    for (int u = 0; u < kUBwd; ++u)
      if (c0 + 64 * u < chunks) vdy[u] = dyrow[c0 + 64 * u];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j < k) {
        const uint4* yrow = reinterpret_cast<const uint4*>(yexp + static_cast<long long>(rows[j]) * d);
        uint4* orow = reinterpret_cast<uint4*>(dyexp + static_cast<long long>(rows[j]) * d);
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
  for (int j = 0; j < KM; ++j) {
    const float s = wave_sum(dot[j]);   // every lane takes part, also for j >= k (zeros)
    if (lane == j) mine = s;
  }
  if (lane < k) dgate[t * k + lane] = mine;
}

// The same with dyexp leaving as MXFP8 row blocks: the bf16 values bf16(gate[t,j] * dy[t]) are
// formed in registers and quantised there (32-element blocks = 4 lanes, amax by shuffles), so
// dyq holds exactly what mxfp8_quantize gives for the bf16 rows, which are never written, and dys
// the same scales in the GEMM layout (mx_gemm_scale_index, R = T k) the down dgrad reads.
// row_gate[dest[t,j]] = gate[t,j] lets the grouped quantiser rebuild the same rows from dy.
template <int KM>
__global__ __launch_bounds__(256) void combine_bwd_mx_kernel(const uint16_t* __restrict__ dy,
                                                             const uint16_t* __restrict__ yexp,
                                                             const float* __restrict__ gate,
                                                             const int32_t* __restrict__ dest, int T, int d, int k,
                                                             uint8_t* __restrict__ dyq, uint8_t* __restrict__ dys,
                                                             float* __restrict__ row_gate, float* __restrict__ dgate) {
  const long long t = static_cast<long long>(blockIdx.x) * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  int rows[KM];
  float g[KM], dot[KM];
  dest_rows<KM>(dest, t, k, rows);
  gates_of<KM>(gate, t, k, g);
  const long long nrows = static_cast<long long>(T) * k;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    dot[j] = 0.f;
    if (j < k && lane == j) row_gate[rows[j]] = g[j];
  }
  const int chunks = d / 8;   // a multiple of 8: a 4-lane block group is all in range or all out
  const uint4* dyrow = reinterpret_cast<const uint4*>(dy + t * d);
  for (int c0 = lane; c0 < chunks; c0 += 64 * kUBwd) {
    uint4 vdy[kUBwd];
#pragma unroll
    for (int u = 0; u < kUBwd; ++u)
      if (c0 + 64 * u < chunks) vdy[u] = dyrow[c0 + 64 * u];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j < k) {
        const uint4* yrow = reinterpret_cast<const uint4*>(yexp + static_cast<long long>(rows[j]) * d);
        uint4 vy[kUBwd];
#pragma unroll
        for (int u = 0; u < kUBwd; ++u)
          if (c0 + 64 * u < chunks) vy[u] = yrow[c0 + 64 * u];
#pragma unroll
        for (int u = 0; u < kUBwd; ++u) {
          const int c = c0 + 64 * u;
          if (c < chunks) {
            float fdy[8], fy[8], o[8];
            unpack8(vdy[u], fdy);
            unpack8(vy[u], fy);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              dot[j] = fmaf(fdy[i], fy[i], dot[j]);
              o[i] = g[j] * fdy[i];
            }
            const uint4 b = pack8(o);   // the bf16 dyexp values
            const uint32_t w[4] = {b.x, b.y, b.z, b.w};
            uint32_t amax = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) amax = max(amax, max(w[i] & 0x7fffu, (w[i] >> 16) & 0x7fffu));
            amax = max(amax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(amax), 1, 64)));
            amax = max(amax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(amax), 2, 64)));
            const int sh = mx_shared_exp(amax);
            const uint32_t lo = mx_encode4(w[0] & 0xffffu, w[0] >> 16, w[1] & 0xffffu, w[1] >> 16, sh);
            const uint32_t hi = mx_encode4(w[2] & 0xffffu, w[2] >> 16, w[3] & 0xffffu, w[3] >> 16, sh);
            const long long r = rows[j];
            *reinterpret_cast<uint2*>(dyq + r * d + 8 * c) = make_uint2(lo, hi);
            if ((lane & 3) == 0) dys[mx_gemm_scale_index(r, c / 4, nrows, d)] = static_cast<uint8_t>(sh + 127);
          }
        }
      }
    }
  }
  float mine = 0.f;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    const float s = wave_sum(dot[j]);
    if (lane == j) mine = s;
  }
  if (lane < k) dgate[t * k + lane] = mine;
}

// dx[t] = sum_j dxp[dest[t,j]] (+ addend[t]), fp32 in slot order after the addend
template <int KM>
__global__ __launch_bounds__(256) void permute_bwd_kernel(const uint16_t* __restrict__ dxp, const int32_t* __restrict__ dest,
                                                          int T, int d, int k, int nseg, const float* __restrict__ addend,
                                                          uint16_t* __restrict__ dx) {
  const SegItem it = seg_item(nseg);
  if (it.t >= T) return;
  int rows[KM];
  dest_rows<KM>(dest, it.t, k, rows);
  const int chunks = d / 8;
  if (it.c >= chunks) return;
  uint4 v[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j)
    if (j < k) v[j] = reinterpret_cast<const uint4*>(dxp + static_cast<long long>(rows[j]) * d)[it.c];
  float acc[8];
  if (addend != nullptr) {
    const float4* a = reinterpret_cast<const float4*>(addend + it.t * d + 8 * it.c);
    const float4 a0 = a[0], a1 = a[1];
    acc[0] = a0.x; acc[1] = a0.y; acc[2] = a0.z; acc[3] = a0.w;
    acc[4] = a1.x; acc[5] = a1.y; acc[6] = a1.z; acc[7] = a1.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    if (j < k) {
      float f[8];
      unpack8(v[j], f);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += f[i];
    }
  }
  reinterpret_cast<uint4*>(dx + it.t * d)[it.c] = pack8(acc);
}

int check_rows(int T, int d, int k) {
  MOE_REQUIRE(T >= 1, MOE_ERR_UNSUPPORTED, "T must be >= 1");
  MOE_REQUIRE(k >= 1 && k <= kMaxK, MOE_ERR_UNSUPPORTED, "k must be in [1, 16]");
  MOE_REQUIRE(d >= 64 && d % 64 == 0, MOE_ERR_UNSUPPORTED, "d must be a positive multiple of 64");
  MOE_REQUIRE(static_cast<long long>(T) * k < (1LL << 31), MOE_ERR_UNSUPPORTED, "T*k must be < 2^31");
  return MOE_OK;
}

unsigned grid_for(int T) { return static_cast<unsigned>((T + kWaves - 1) / kWaves); }

// Segments per row of `chunks` 16-byte chunks, and the launch grid for T tokens of them.
int segs_of(long long chunks) { return static_cast<int>((chunks + kSegChunks - 1) / kSegChunks); }
unsigned seg_grid(int T, int nseg) {
  return static_cast<unsigned>((static_cast<long long>(T) * nseg + kWaves - 1) / kWaves);
}

// Instantiation for k: the smallest of 4, 8, 16 that holds it (fewer registers for small k).
#define MOE_SEG_LAUNCH(KERNEL, GRID, STREAM, K, ...)                              \
  do {                                                                           \
    if ((K) <= 4) KERNEL<4><<<(GRID), 256, 0, (STREAM)>>>(__VA_ARGS__);         \
    else if ((K) <= 8) KERNEL<8><<<(GRID), 256, 0, (STREAM)>>>(__VA_ARGS__);    \
    else KERNEL<16><<<(GRID), 256, 0, (STREAM)>>>(__VA_ARGS__);                 \
  } while (0)

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
  const int nseg = segs_of(pitch / 16);
  MOE_REQUIRE(static_cast<long long>(T) * nseg * 64 < (1LL << 32), MOE_ERR_UNSUPPORTED, "too many row segments");
  MOE_SEG_LAUNCH(permute_kernel, seg_grid(T, nseg), as_stream(stream), k, static_cast<const uint8_t*>(x), x_scale, dest,
                 T, k, nseg, pitch, spitch, static_cast<uint8_t*>(xp), xp_scale);
  return check_launch("permute");
}

extern "C" int moe_permute_quant_mx(const uint16_t* x, const int32_t* dest, int T, int d, int k, uint8_t* xpq,
                                    uint8_t* xps, void* stream) {
  if (int st = check_rows(T, d, k)) return st;
  MOE_CHECK_PTR(x); MOE_CHECK_PTR(dest); MOE_CHECK_PTR(xpq); MOE_CHECK_PTR(xps);
  MOE_CHECK_ALIGN(x); MOE_CHECK_ALIGN(xpq);
  const int nseg = segs_of(d / 8);
  MOE_REQUIRE(static_cast<long long>(T) * nseg * 64 < (1LL << 32), MOE_ERR_UNSUPPORTED, "too many row segments");
  MOE_SEG_LAUNCH(permute_mx_kernel, seg_grid(T, nseg), as_stream(stream), k, x, dest, T, d, k, nseg, xpq, xps);
  return check_launch("permute_quant_mx");
}

extern "C" int moe_unpermute_combine(const uint16_t* yexp, const float* gate, const int32_t* dest, int T, int d,
                                     int k, uint16_t* y, void* stream) {
  if (int st = check_rows(T, d, k)) return st;
  MOE_CHECK_PTR(yexp); MOE_CHECK_PTR(gate); MOE_CHECK_PTR(dest); MOE_CHECK_PTR(y);
  MOE_CHECK_ALIGN(yexp); MOE_CHECK_ALIGN(y);
  const int nseg = segs_of(d / 8);
  MOE_REQUIRE(static_cast<long long>(T) * nseg * 64 < (1LL << 32), MOE_ERR_UNSUPPORTED, "too many row segments");
  MOE_SEG_LAUNCH(combine_kernel, seg_grid(T, nseg), as_stream(stream), k, yexp, gate, dest, T, d, k, nseg, y);
  return check_launch("combine");
}

extern "C" int moe_unpermute_combine_bwd(const uint16_t* dy, const uint16_t* yexp, const float* gate,
                                         const int32_t* dest, int T, int d, int k, uint16_t* dyexp, float* dgate,
                                         void* stream) {
  if (int st = check_rows(T, d, k)) return st;
  MOE_CHECK_PTR(dy); MOE_CHECK_PTR(yexp); MOE_CHECK_PTR(gate); MOE_CHECK_PTR(dest);
  MOE_CHECK_PTR(dyexp); MOE_CHECK_PTR(dgate);
  MOE_CHECK_ALIGN(dy); MOE_CHECK_ALIGN(yexp); MOE_CHECK_ALIGN(dyexp);
  MOE_SEG_LAUNCH(combine_bwd_kernel, grid_for(T), as_stream(stream), k, dy, yexp, gate, dest, T, d, k, dyexp, dgate);
  return check_launch("combine_bwd");
}

extern "C" int moe_unpermute_combine_bwd_mx(const uint16_t* dy, const uint16_t* yexp, const float* gate,
                                            const int32_t* dest, int T, int d, int k, uint8_t* dyexp_q,
                                            uint8_t* dyexp_scale, float* row_gate, float* dgate, void* stream) {
  if (int st = check_rows(T, d, k)) return st;
  MOE_CHECK_PTR(dy); MOE_CHECK_PTR(yexp); MOE_CHECK_PTR(gate); MOE_CHECK_PTR(dest);
  MOE_CHECK_PTR(dyexp_q); MOE_CHECK_PTR(dyexp_scale); MOE_CHECK_PTR(row_gate); MOE_CHECK_PTR(dgate);
  MOE_CHECK_ALIGN(dy); MOE_CHECK_ALIGN(yexp); MOE_CHECK_ALIGN(dyexp_q);
  MOE_SEG_LAUNCH(combine_bwd_mx_kernel, grid_for(T), as_stream(stream), k, dy, yexp, gate, dest, T, d, k, dyexp_q,
                 dyexp_scale, row_gate, dgate);
  return check_launch("combine_bwd_mx");
}

extern "C" int moe_permute_bwd(const uint16_t* dxp, const int32_t* dest, int T, int d, int k,
                               const float* addend, uint16_t* dx, void* stream) {
  if (int st = check_rows(T, d, k)) return st;
  MOE_CHECK_PTR(dxp); MOE_CHECK_PTR(dest); MOE_CHECK_PTR(dx);
  MOE_CHECK_ALIGN(dxp); MOE_CHECK_ALIGN(dx);
  if (addend) MOE_CHECK_ALIGN(addend);
  const int nseg = segs_of(d / 8);
  MOE_REQUIRE(static_cast<long long>(T) * nseg * 64 < (1LL << 32), MOE_ERR_UNSUPPORTED, "too many row segments");
  MOE_SEG_LAUNCH(permute_bwd_kernel, seg_grid(T, nseg), as_stream(stream), k, dxp, dest, T, d, k, nseg, addend, dx);
  return check_launch("permute_bwd");
}
