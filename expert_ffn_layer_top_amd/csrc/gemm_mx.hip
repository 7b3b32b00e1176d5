// Device-scheduled grouped GEMMs of the SwiGLU expert FFN in MXFP8 (E4M3 operands, one E8M0
// scale per 32 elements along K, fp32 accumulation, bf16 outputs), forward and backward, on
// CDNA4's block-scaled matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4).
//
// [news] "Ai2 rebuilds Olmo's training stack for trillion-parameter MoEs", "MXFP8 reduces compute
// and memory costs": 8-bit floats with a separate scale per small block, used for the expert
// FFN products; "Routing work stays on the GPU" / [card] "Summary": grouped, device-scheduled.
//
// Every operand arrives quantised along its product's contraction dimension, so all six
// products read both operands K-contiguous:
//   FWD1   xp_q [n][d]          x  W_gate_q[e], W_up_q[e] [f][d]      -> G, U, A = silu(G) U
//   FWD2   a_q [n][f]           x  W_down_q[e] [d][f]                 -> Yexp
//   DGRAD1 dyexp_q [n][d]       x  W_down^T_q[e] [f][d]               -> dG, dU (SwiGLU backward)
//   DGRAD2 dg_q | du_q [n][f]   x  W_gate^T_q[e] | W_up^T_q[e] [d][f] -> dXp        (K = 2f)
//   WGRAD_DOWN  dyexp^T_q [d][P]  x  a^T_q [f][P]                     -> dW_down[e]
//   WGRAD_GU    dg^T_q | du^T_q [f][P]  x  xp^T_q [d][P]              -> dW_gate[e], dW_up[e]
// where P is the padded token axis: expert e owns positions [offsets_pad[e], offsets_pad[e+1]).
//
// Tile geometry matches the bf16 kernels: 256 x 256 outputs per workgroup, four waves of
// 128 x 128, K step 128 elements = one 128-byte LDS row per operand row (same XOR swizzle), two
// stages.  Each K step also stages 4 scale bytes per row (one 32-bit word) in LDS.  The MFMA
// lane layout (checked on the device): lane l holds row l % 16, K bytes 16*(l/16) .. +15 and
// 64 + 16*(l/16) .. +15 of the 128-wide step, and supplies the scale of row l % 16, K block l/16.
#include <type_traits>

#include "common.h"

namespace moe {
namespace gmx {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 128;                           // fp8 elements (bytes) per K step
constexpr int NTH = 256;
constexpr int ROW_BYTES = BK;
constexpr int TILE_BYTES = BM * ROW_BYTES;        // 32 KiB
constexpr int SCALE_BYTES = BM * 4;               // 1 KiB per operand per stage
constexpr int STAGE_BYTES = 2 * TILE_BYTES + 2 * SCALE_BYTES;
constexpr int LDS_BYTES = 2 * STAGE_BYTES;        // 130 KiB

enum Mode { FWD1 = 0, FWD2 = 1, DGRAD1 = 2, DGRAD2 = 3, WGRAD_DOWN = 4, WGRAD_GU = 5 };

struct Params {
  const int32_t* offsets;
  const int32_t* offsets_pad;   // WGRAD: padded token offsets
  int E, n, d, f;
  int P;                        // WGRAD: length of the padded token axis
  const uint8_t* a0; const uint8_t* a0s;
  const uint8_t* a1; const uint8_t* a1s;
  const uint8_t* b0; const uint8_t* b0s;
  const uint8_t* b1; const uint8_t* b1s;
  const uint16_t* g;
  const uint16_t* u;
  uint16_t* o0;
  uint16_t* o1;
  uint16_t* o2;
};

template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int r, int chunk) { return r * ROW_BYTES + ((chunk ^ swz(r)) << 4); }
__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

template <int MODE>
struct Traits {
  static constexpr bool WGRAD = (MODE >= WGRAD_DOWN);
};

struct Tile {
  int e, m0, m_end, n0, half;
  int k_begin;   // WGRAD: first padded token position of the expert
  int k_len;     // K extent
};

template <int MODE>
__device__ __forceinline__ int n_total(const Params& p) {
  if (MODE == FWD1 || MODE == DGRAD1 || MODE == WGRAD_DOWN) return p.f;
  return p.d;
}
template <int MODE>
__device__ __forceinline__ int n_tile_width() { return MODE == FWD1 ? BN / 2 : BN; }
template <int MODE>
__device__ __forceinline__ int k_total(const Params& p) {
  if (MODE == FWD1 || MODE == DGRAD1) return p.d;
  if (MODE == FWD2) return p.f;
  if (MODE == DGRAD2) return 2 * p.f;
  return 0;
}

// Loads one K step of the A side (M rows) into registers: 8 data chunks + 1 scale word.
template <int MODE>
__device__ __forceinline__ void load_a(const Params& p, const Tile& t, int kt, uint4 (&reg)[8], uint32_t& sreg) {
  const int tid = threadIdx.x;
  const int ch = tid & 7;
  if constexpr (!Traits<MODE>::WGRAD) {
    const int K = (MODE == DGRAD2) ? p.f : k_total<MODE>(p);
    int k0 = kt * BK;
    const uint8_t* base = p.a0;
    const uint8_t* sbase = p.a0s;
    if (MODE == DGRAD2 && k0 >= p.f) { base = p.a1; sbase = p.a1s; k0 -= p.f; }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int r = t.m0 + (tid >> 3) + 32 * i;
      r = r < p.n ? r : p.n - 1;
      reg[i] = ld16(base + static_cast<long long>(r) * K + k0 + 16 * ch);
    }
    int r = t.m0 + tid;
    r = r < p.n ? r : p.n - 1;
    sreg = *reinterpret_cast<const uint32_t*>(sbase + static_cast<long long>(r) * (K / 32) + k0 / 32);
  } else {
    const int Mtot = (MODE == WGRAD_DOWN) ? p.d : p.f;
    const uint8_t* base = (MODE == WGRAD_GU && t.half) ? p.a1 : p.a0;
    const uint8_t* sbase = (MODE == WGRAD_GU && t.half) ? p.a1s : p.a0s;
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int m = t.m0 + (tid >> 3) + 32 * i;
      m = m < Mtot ? m : Mtot - 1;
      const int k = k0 + 16 * ch;
      reg[i] = (k < t.k_len) ? ld16(base + static_cast<long long>(m) * p.P + t.k_begin + k) : make_uint4(0, 0, 0, 0);
    }
    int m = t.m0 + tid;
    m = m < Mtot ? m : Mtot - 1;
    const uint8_t* sp = sbase + static_cast<long long>(m) * (p.P / 32) + (t.k_begin + k0) / 32;
    uint32_t w = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      if (k0 + 32 * b < t.k_len) w |= static_cast<uint32_t>(sp[b]) << (8 * b);
    sreg = w;
  }
}

// Loads one K step of the B side (N rows).
template <int MODE>
__device__ __forceinline__ void load_b(const Params& p, const Tile& t, int kt, uint4 (&reg)[8], uint32_t& sreg) {
  const int tid = threadIdx.x;
  const int ch = tid & 7;
  const int k0 = kt * BK;
  if constexpr (MODE == FWD1) {
    // LDS rows 0..127: W_gate_q[e] rows n0 + r; rows 128..255: W_up_q[e] rows n0 + r - 128
    const long long eoff = static_cast<long long>(t.e) * p.f * p.d;
    const long long esoff = static_cast<long long>(t.e) * p.f * (p.d / 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = (tid >> 3) + 32 * i;
      int c = t.n0 + (r & 127);
      c = c < p.f ? c : p.f - 1;
      reg[i] = ld16(((r < 128) ? p.b0 : p.b1) + eoff + static_cast<long long>(c) * p.d + k0 + 16 * ch);
    }
    int c = t.n0 + (tid & 127);
    c = c < p.f ? c : p.f - 1;
    sreg = *reinterpret_cast<const uint32_t*>(((tid < 128) ? p.b0s : p.b1s) + esoff +
                                              static_cast<long long>(c) * (p.d / 32) + k0 / 32);
  } else if constexpr (!Traits<MODE>::WGRAD) {
    // weights [E][Ntot][K'] quantised along K' (K' = K, or f per half for DGRAD2)
    const int Ntot = n_total<MODE>(p);
    int K = k_total<MODE>(p);
    int kk = k0;
    const uint8_t* base = p.b0;
    const uint8_t* sbase = p.b0s;
    if constexpr (MODE == DGRAD2) {
      K = p.f;
      if (kk >= p.f) { base = p.b1; sbase = p.b1s; kk -= p.f; }
    }
    const long long eoff = static_cast<long long>(t.e) * Ntot * K;
    const long long esoff = static_cast<long long>(t.e) * Ntot * (K / 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int c = t.n0 + (tid >> 3) + 32 * i;
      c = c < Ntot ? c : Ntot - 1;
      reg[i] = ld16(base + eoff + static_cast<long long>(c) * K + kk + 16 * ch);
    }
    int c = t.n0 + tid;
    c = c < Ntot ? c : Ntot - 1;
    sreg = *reinterpret_cast<const uint32_t*>(sbase + esoff + static_cast<long long>(c) * (K / 32) + kk / 32);
  } else {
    const int Ntot = n_total<MODE>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int c = t.n0 + (tid >> 3) + 32 * i;
      c = c < Ntot ? c : Ntot - 1;
      const int k = k0 + 16 * ch;
      reg[i] = (k < t.k_len) ? ld16(p.b0 + static_cast<long long>(c) * p.P + t.k_begin + k) : make_uint4(0, 0, 0, 0);
    }
    int c = t.n0 + tid;
    c = c < Ntot ? c : Ntot - 1;
    const uint8_t* sp = p.b0s + static_cast<long long>(c) * (p.P / 32) + (t.k_begin + k0) / 32;
    uint32_t w = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      if (k0 + 32 * b < t.k_len) w |= static_cast<uint32_t>(sp[b]) << (8 * b);
    sreg = w;
  }
}

__device__ __forceinline__ void store_stage(uint8_t* tile, uint32_t* scales, const uint4 (&reg)[8], uint32_t sreg) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<uint4*>(tile + lds_off((tid >> 3) + 32 * i, tid & 7)) = reg[i];
  scales[tid] = sreg;
}

__device__ __forceinline__ void st4(uint16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}
__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

template <int MODE>
__global__ __launch_bounds__(NTH, 1) void mx_grouped_gemm_kernel(Params p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int s_pre[257];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const int NTW = n_tile_width<MODE>();
  const int ntiles_n = (n_total<MODE>(p) + NTW - 1) / NTW;
  int total_tiles;
  if constexpr (!Traits<MODE>::WGRAD) {
    if (tid == 0) s_pre[0] = 0;
    for (int e = tid; e < p.E; e += NTH) s_pre[e + 1] = (p.offsets[e + 1] - p.offsets[e] + BM - 1) / BM;
    __syncthreads();
    if (tid == 0)
      for (int e = 0; e < p.E; ++e) s_pre[e + 1] += s_pre[e];
    __syncthreads();
    total_tiles = s_pre[p.E] * ntiles_n;
  } else {
    const int Mtot = (MODE == WGRAD_DOWN) ? p.d : p.f;
    total_tiles = p.E * ((Mtot + BM - 1) / BM) * (MODE == WGRAD_GU ? 2 : 1) * ntiles_n;
  }
  const int tot8 = (total_tiles + 7) & ~7;
  const int bid = blockIdx.x;
  if (bid >= tot8) return;
  const int lid = (bid & 7) * (tot8 >> 3) + (bid >> 3);
  if (lid >= total_tiles) return;

  Tile t;
  if constexpr (!Traits<MODE>::WGRAD) {
    const int mt_glob = lid / ntiles_n;
    const int nt = lid - mt_glob * ntiles_n;
    int lo = 0, hi = p.E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pre[mid] <= mt_glob) lo = mid; else hi = mid - 1;
    }
    t.e = lo;
    t.m0 = p.offsets[lo] + (mt_glob - s_pre[lo]) * BM;
    t.m_end = p.offsets[lo + 1];
    t.n0 = nt * NTW;
    t.half = 0;
    t.k_begin = 0;
    t.k_len = k_total<MODE>(p);
  } else {
    const int Mtot = (MODE == WGRAD_DOWN) ? p.d : p.f;
    const int mt = (Mtot + BM - 1) / BM;
    const int per_e = mt * (MODE == WGRAD_GU ? 2 : 1) * ntiles_n;
    t.e = lid / per_e;
    const int rem = lid - t.e * per_e;
    const int mi = rem / ntiles_n;
    const int nt = rem - mi * ntiles_n;
    t.half = mi >= mt ? 1 : 0;
    t.m0 = (mi - t.half * mt) * BM;
    t.m_end = Mtot;
    t.n0 = nt * BN;
    t.k_begin = p.offsets_pad[t.e];
    t.k_len = p.offsets_pad[t.e + 1] - t.k_begin;
  }
  const int nk = (t.k_len + BK - 1) / BK;

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto brow = [&](int i) -> int {
    if constexpr (MODE == FWD1) return (i < 4) ? (64 * wn + 16 * i) : (128 + 64 * wn + 16 * (i - 4));
    return 128 * wn + 16 * i;
  };

  uint4 ra[8], rb[8];
  uint32_t sa_reg = 0, sb_reg = 0;
  auto stage_ptrs = [&](int st, uint8_t*& ta, uint8_t*& tb, uint32_t*& sa, uint32_t*& sb) {
    uint8_t* base = lds + st * STAGE_BYTES;
    ta = base;
    tb = base + TILE_BYTES;
    sa = reinterpret_cast<uint32_t*>(base + 2 * TILE_BYTES);
    sb = reinterpret_cast<uint32_t*>(base + 2 * TILE_BYTES + SCALE_BYTES);
  };
  if (nk > 0) {
    load_a<MODE>(p, t, 0, ra, sa_reg);
    load_b<MODE>(p, t, 0, rb, sb_reg);
    uint8_t *ta, *tb;
    uint32_t *sa, *sb;
    stage_ptrs(0, ta, tb, sa, sb);
    store_stage(ta, sa, ra, sa_reg);
    store_stage(tb, sb, rb, sb_reg);
  }
  __syncthreads();

  const int sel = lane >> 4;
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) {
      load_a<MODE>(p, t, kt + 1, ra, sa_reg);
      load_b<MODE>(p, t, kt + 1, rb, sb_reg);
    }
    uint8_t *ta, *tb;
    uint32_t *sa, *sb;
    stage_ptrs(kt & 1, ta, tb, sa, sb);
    i32x8 fa[8], fb[8];
    int xa[8], xb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = 128 * wm + 16 * j + (lane & 15);
      const uint4 lo = *reinterpret_cast<const uint4*>(ta + lds_off(r, sel));
      const uint4 hi = *reinterpret_cast<const uint4*>(ta + lds_off(r, 4 + sel));
      fa[j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      xa[j] = (sa[r] >> (8 * sel)) & 0xff;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = brow(i) + (lane & 15);
      const uint4 lo = *reinterpret_cast<const uint4*>(tb + lds_off(r, sel));
      const uint4 hi = *reinterpret_cast<const uint4*>(tb + lds_off(r, 4 + sel));
      fb[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      xb[i] = (sb[r] >> (8 * sel)) & 0xff;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb[i], fa[j], acc[i][j], 0, 0, 0, xb[i], 0,
                                                                     xa[j]);
    if (more) {
      stage_ptrs((kt + 1) & 1, ta, tb, sa, sb);
      store_stage(ta, sa, ra, sa_reg);
      store_stage(tb, sb, rb, sb_reg);
    }
    __syncthreads();
  }

  const int rl = lane & 15;
  const int cq = 4 * (lane >> 4);
  if constexpr (MODE == FWD1) {
    static_for<0, 8>([&](auto j) {
      const int row = t.m0 + 128 * wm + 16 * j + rl;
      if (row >= t.m_end) return;
      static_for<0, 4>([&](auto i) {
        const int col = t.n0 + 64 * wn + 16 * i + cq;
        if (col >= p.f) return;
        const f32x4 gv = acc[i][j], uv = acc[i + 4][j];
        float av[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) av[q] = gv[q] * sigmoidf_(gv[q]) * uv[q];
        const long long o = static_cast<long long>(row) * p.f + col;
        st4(p.o0 + o, gv[0], gv[1], gv[2], gv[3]);
        st4(p.o1 + o, uv[0], uv[1], uv[2], uv[3]);
        st4(p.o2 + o, av[0], av[1], av[2], av[3]);
      });
    });
  } else if constexpr (MODE == DGRAD1) {
    static_for<0, 8>([&](auto j) {
      const int row = t.m0 + 128 * wm + 16 * j + rl;
      if (row >= t.m_end) return;
      static_for<0, 8>([&](auto i) {
        const int col = t.n0 + 128 * wn + 16 * i + cq;
        if (col >= p.f) return;
        const long long o = static_cast<long long>(row) * p.f + col;
        const uint2 gw = *reinterpret_cast<const uint2*>(p.g + o);
        const uint2 uw = *reinterpret_cast<const uint2*>(p.u + o);
        const float gv[4] = {bf16_lo(gw.x), bf16_hi(gw.x), bf16_lo(gw.y), bf16_hi(gw.y)};
        const float uv[4] = {bf16_lo(uw.x), bf16_hi(uw.x), bf16_lo(uw.y), bf16_hi(uw.y)};
        const f32x4 dav = acc[i][j];
        float dg[4], du[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float sg = sigmoidf_(gv[q]);
          dg[q] = dav[q] * uv[q] * sg * (1.0f + gv[q] * (1.0f - sg));
          du[q] = dav[q] * gv[q] * sg;
        }
        st4(p.o0 + o, dg[0], dg[1], dg[2], dg[3]);
        st4(p.o1 + o, du[0], du[1], du[2], du[3]);
      });
    });
  } else {
    const int Ntot = n_total<MODE>(p);
    uint16_t* out = p.o0;
    if constexpr (Traits<MODE>::WGRAD) {
      const int Mtot = (MODE == WGRAD_DOWN) ? p.d : p.f;
      out = (MODE == WGRAD_GU && t.half ? p.o1 : p.o0) + static_cast<long long>(t.e) * Mtot * Ntot;
    }
    static_for<0, 8>([&](auto j) {
      const int row = t.m0 + 128 * wm + 16 * j + rl;
      if (row >= t.m_end) return;
      static_for<0, 8>([&](auto i) {
        const int col = t.n0 + 128 * wn + 16 * i + cq;
        if (col >= Ntot) return;
        const f32x4 v = acc[i][j];
        st4(out + static_cast<long long>(row) * Ntot + col, v[0], v[1], v[2], v[3]);
      });
    });
  }
}

inline long long grid_upper(int mode, int E, int n, int d, int f) {
  switch (mode) {
    case FWD1: return (static_cast<long long>(n / BM) + E) * ((f + 127) / 128);
    case FWD2: return (static_cast<long long>(n / BM) + E) * ((d + BN - 1) / BN);
    case DGRAD1: return (static_cast<long long>(n / BM) + E) * ((f + BN - 1) / BN);
    case DGRAD2: return (static_cast<long long>(n / BM) + E) * ((d + BN - 1) / BN);
    case WGRAD_DOWN: return static_cast<long long>(E) * ((d + BM - 1) / BM) * ((f + BN - 1) / BN);
    default: return static_cast<long long>(E) * 2 * ((f + BM - 1) / BM) * ((d + BN - 1) / BN);
  }
}

template <int MODE>
int launch(const Params& p, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    // Raises the dynamic-LDS limit for this kernel.  Advisory: where the runtime does not take the
    // attribute, the launch below reports any real problem, so its status is cleared, not returned.
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&mx_grouped_gemm_kernel<MODE>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    (void)hipGetLastError();
    attr_set = true;
  }
  const long long g = (grid_upper(MODE, p.E, p.n, p.d, p.f) + 7) / 8 * 8;
  MOE_REQUIRE(g < (1LL << 31), MOE_ERR_UNSUPPORTED, "too many tiles");
  mx_grouped_gemm_kernel<MODE><<<static_cast<unsigned>(g), NTH, LDS_BYTES, s>>>(p);
  return check_launch("grouped_gemm_mxfp8");
}

}  // namespace gmx

// ------------------------------------------------------------------ host-side composition

// Forward, first product: FWD1 (G, U, A bf16).
int gg_mx_gate_up(int E, int n, int d, int f, const int32_t* offsets, const uint8_t* xq, const uint8_t* xs,
                  const uint8_t* wgq, const uint8_t* wgs, const uint8_t* wuq, const uint8_t* wus, uint16_t* g,
                  uint16_t* u, uint16_t* a, hipStream_t s) {
  gmx::Params p{};
  p.offsets = offsets; p.E = E; p.n = n; p.d = d; p.f = f;
  p.a0 = xq; p.a0s = xs; p.b0 = wgq; p.b0s = wgs; p.b1 = wuq; p.b1s = wus;
  p.o0 = g; p.o1 = u; p.o2 = a;
  return gmx::launch<gmx::FWD1>(p, s);
}

// Forward, second product: quantise A along f into ws, then FWD2 (Yexp).
int gg_mx_down(int E, int n, int d, int f, const int32_t* offsets, const uint16_t* a, const uint8_t* wdq,
               const uint8_t* wds, uint16_t* yexp, uint8_t* ws, hipStream_t s) {
  uint8_t* aq = ws;
  uint8_t* as = ws + static_cast<size_t>(n) * f;
  if (int st = mxfp8_quantize(a, 1, n, f, 0, aq, as, s)) return st;
  gmx::Params q{};
  q.offsets = offsets; q.E = E; q.n = n; q.d = d; q.f = f;
  q.a0 = aq; q.a0s = as; q.b0 = wdq; q.b0s = wds; q.o0 = yexp;
  return gmx::launch<gmx::FWD2>(q, s);
}

size_t gg_mx_forward_ws(int n, int f) { return static_cast<size_t>(n) * f + static_cast<size_t>(n) * f / 32; }

// Workspace layout of the MXFP8 backward (byte offsets), from host scalars.
struct MxBwdLayout {
  size_t dyq, dys, dgq, dgs, duq, dus;             // row-quantised (blocks along K of the dgrads)
  size_t dyT, dyTs, aT, aTs, dgT, dgTs, duT, duTs, xT, xTs;   // grouped-token (wgrad) operands
  size_t total;
  MxBwdLayout(int E, int n, int d, int f) {
    const size_t P = static_cast<size_t>(moe_mx_pad_cap(n, E));
    size_t o = 0;
    auto take = [&](size_t bytes) { const size_t at = o; o += (bytes + 255) / 256 * 256; return at; };
    dyq = take(static_cast<size_t>(n) * d);  dys = take(static_cast<size_t>(n) * d / 32);
    dgq = take(static_cast<size_t>(n) * f);  dgs = take(static_cast<size_t>(n) * f / 32);
    duq = take(static_cast<size_t>(n) * f);  dus = take(static_cast<size_t>(n) * f / 32);
    dyT = take(d * P); dyTs = take(d * P / 32);
    aT = take(f * P);  aTs = take(f * P / 32);
    dgT = take(f * P); dgTs = take(f * P / 32);
    duT = take(f * P); duTs = take(f * P / 32);
    xT = take(d * P);  xTs = take(d * P / 32);
    total = o;
  }
};

size_t gg_mx_backward_ws(int E, int n, int d, int f) { return MxBwdLayout(E, n, d, f).total; }

int gg_mx_backward(int E, int n, int d, int f, const int32_t* offsets, const int32_t* offsets_pad,
                   const int32_t* row_token, const uint16_t* x, const uint16_t* g, const uint16_t* u,
                   const uint16_t* a, const uint16_t* dyexp, const uint8_t* wgtq, const uint8_t* wgts,
                   const uint8_t* wutq, const uint8_t* wuts, const uint8_t* wdtq, const uint8_t* wdts, uint16_t* dg,
                   uint16_t* du, uint16_t* dxp, uint16_t* dwg, uint16_t* dwu, uint16_t* dwd, uint8_t* ws,
                   hipStream_t s) {
  const MxBwdLayout L(E, n, d, f);
  const int P = moe_mx_pad_cap(n, E);
  // dgrad through W_down: dYexp quantised along d
  if (int st = mxfp8_quantize(dyexp, 1, n, d, 0, ws + L.dyq, ws + L.dys, s)) return st;
  gmx::Params p{};
  p.offsets = offsets; p.E = E; p.n = n; p.d = d; p.f = f;
  p.a0 = ws + L.dyq; p.a0s = ws + L.dys; p.b0 = wdtq; p.b0s = wdts; p.g = g; p.u = u; p.o0 = dg; p.o1 = du;
  if (int st = gmx::launch<gmx::DGRAD1>(p, s)) return st;
  // wgrad operands along grouped tokens
  if (int st = mxfp8_quantize_grouped(dyexp, nullptr, offsets, offsets_pad, E, n, d, ws + L.dyT, ws + L.dyTs, s)) return st;
  if (int st = mxfp8_quantize_grouped(a, nullptr, offsets, offsets_pad, E, n, f, ws + L.aT, ws + L.aTs, s)) return st;
  gmx::Params w{};
  w.offsets = offsets; w.offsets_pad = offsets_pad; w.E = E; w.n = n; w.d = d; w.f = f; w.P = P;
  w.a0 = ws + L.dyT; w.a0s = ws + L.dyTs; w.b0 = ws + L.aT; w.b0s = ws + L.aTs; w.o0 = dwd;
  if (int st = gmx::launch<gmx::WGRAD_DOWN>(w, s)) return st;
  // dgrad through W_gate, W_up: dG, dU quantised along f
  if (int st = mxfp8_quantize(dg, 1, n, f, 0, ws + L.dgq, ws + L.dgs, s)) return st;
  if (int st = mxfp8_quantize(du, 1, n, f, 0, ws + L.duq, ws + L.dus, s)) return st;
  gmx::Params q{};
  q.offsets = offsets; q.E = E; q.n = n; q.d = d; q.f = f;
  q.a0 = ws + L.dgq; q.a0s = ws + L.dgs; q.a1 = ws + L.duq; q.a1s = ws + L.dus;
  q.b0 = wgtq; q.b0s = wgts; q.b1 = wutq; q.b1s = wuts; q.o0 = dxp;
  if (int st = gmx::launch<gmx::DGRAD2>(q, s)) return st;
  // wgrad of W_gate, W_up
  if (int st = mxfp8_quantize_grouped(dg, nullptr, offsets, offsets_pad, E, n, f, ws + L.dgT, ws + L.dgTs, s)) return st;
  if (int st = mxfp8_quantize_grouped(du, nullptr, offsets, offsets_pad, E, n, f, ws + L.duT, ws + L.duTs, s)) return st;
  if (int st = mxfp8_quantize_grouped(x, row_token, offsets, offsets_pad, E, n, d, ws + L.xT, ws + L.xTs, s)) return st;
  gmx::Params r{};
  r.offsets = offsets; r.offsets_pad = offsets_pad; r.E = E; r.n = n; r.d = d; r.f = f; r.P = P;
  r.a0 = ws + L.dgT; r.a0s = ws + L.dgTs; r.a1 = ws + L.duT; r.a1s = ws + L.duTs;
  r.b0 = ws + L.xT; r.b0s = ws + L.xTs; r.o0 = dwg; r.o1 = dwu;
  return gmx::launch<gmx::WGRAD_GU>(r, s);
}

}  // namespace moe
