// Device-scheduled grouped GEMMs of the SwiGLU expert FFN in bf16 with fp32 accumulation,
// forward and backward, on CDNA4 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// [news] "Ai2 rebuilds Olmo's training stack for trillion-parameter MoEs", "Routing work stays on
// the GPU": the many small per-expert products run as one grouped operation; [card]
// "Supercharging Olmo-core ...", "Summary": the grouped GEMMs are device-scheduled.  Here the
// per-expert row counts exist only on the device: every workgroup reads `offsets`, builds the
// per-expert tile prefix in LDS and maps its own id to (expert, m-tile, n-tile).  The host
// launches an upper bound of tiles computed from T*k alone; surplus workgroups exit at once.
//
// Products (rows r of expert e are offsets[e] .. offsets[e+1]-1):
//   FWD1   [G | U] = Xp W_gate^T | Xp W_up^T, epilogue G, U, A = silu(G) * U        (K = d)
//   FWD2   Yexp = A W_down^T                                                      (K = f)
//   DGRAD1 dA = dYexp W_down, epilogue dG = dA U s (1 + G (1 - s)), dU = dA G s    (K = d)
//   DGRAD2 dXp = dG W_gate + dU W_up                                               (K = 2f)
//   WGRAD_DOWN  dW_down[e] = dYexp_e^T A_e                                         (K = rows of e)
//   WGRAD_GU    dW_gate[e] = dG_e^T Xp_e,  dW_up[e] = dU_e^T Xp_e                   (K = rows of e)
//
// Tiling: 256 x 256 output tile per 256-thread workgroup, K step 64, four waves in a 2 x 2
// grid, each wave owning 128 x 128 outputs as 8 x 8 MFMA 16x16 tiles (256 fp32 accumulators
// per lane).  Operands are staged in LDS as [row][64 k] bf16 with a 16-byte-chunk XOR swizzle
// (chunk ^ ((row ^ row >> 3) & 7)) so that both the MFMA fragment reads (16 consecutive rows,
// one chunk) and the transposed writes (rows 8 apart) spread over all banks; two LDS stages
// (128 KiB) double-buffer the K loop.  Operands stored K-contiguous are copied with 16-byte
// loads; operands stored K-strided (the weights in the dgrad products, the token-major
// activations in the wgrad products) are read as 8 rows x 16 bytes per lane and transposed
// 8 x 8 in registers before the LDS store.  The MFMA computes the transposed tile
// (weights / N side as the first operand), so each lane ends with 4 consecutive output
// columns of one row and stores 8 bytes.
#include <type_traits>

#include "common.h"

namespace moe {
namespace gg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int NTH = 256;
constexpr int ROW_BYTES = BK * 2;                 // 128 bytes per LDS row
constexpr int TILE_BYTES = BM * ROW_BYTES;        // 32 KiB per operand per stage
constexpr int STAGE_BYTES = 2 * TILE_BYTES;
constexpr int LDS_BYTES = 2 * STAGE_BYTES;        // 128 KiB

enum Mode { FWD1 = 0, FWD2 = 1, DGRAD1 = 2, DGRAD2 = 3, WGRAD_DOWN = 4, WGRAD_GU = 5 };

struct Params {
  const int32_t* offsets;
  int E, n, d, f;
  const uint16_t* a0;   // token-side operand (or M-side operand in wgrad)
  const uint16_t* a1;   // second half (DGRAD2: dU; WGRAD_GU: dU)
  const uint16_t* b0;   // weight-side operand (or N-side operand in wgrad)
  const uint16_t* b1;   // second half (FWD1: W_up; DGRAD2: W_up)
  const uint16_t* g;    // DGRAD1 epilogue inputs
  const uint16_t* u;
  uint16_t* o0;
  uint16_t* o1;
  uint16_t* o2;
};

// Compile-time loop: f(std::integral_constant<int, I>{}) for I = B .. E-1, so that indices into
// the accumulator array stay static (a dynamically indexed accumulator array would be demoted
// to scratch memory).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int r, int chunk) { return r * ROW_BYTES + ((chunk ^ swz(r)) << 4); }

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

// 8 x 8 transpose of bf16: in[i] holds k = i, columns 0..7; out[j] holds column j, k = 0..7.
__device__ __forceinline__ void transpose8(const uint4 (&in)[8], uint4 (&out)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint4& lo = in[2 * p];
      const uint4& hi = in[2 * p + 1];
      const uint32_t a = (j >> 1) == 0 ? lo.x : (j >> 1) == 1 ? lo.y : (j >> 1) == 2 ? lo.z : lo.w;
      const uint32_t b = (j >> 1) == 0 ? hi.x : (j >> 1) == 1 ? hi.y : (j >> 1) == 2 ? hi.z : hi.w;
      w[p] = (j & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
    out[j] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <int MODE>
struct Traits {
  static constexpr bool A_KCONTIG = (MODE <= DGRAD2);
  static constexpr bool B_KCONTIG = (MODE <= FWD2);
  static constexpr bool WGRAD = (MODE >= WGRAD_DOWN);
};

// Tile -> work mapping (computed per workgroup from device-resident offsets).
struct Tile {
  int e;
  int m0;          // FWD/DGRAD: first row (absolute); WGRAD: first output row of dW
  int m_end;       // FWD/DGRAD: end of the expert's rows; WGRAD: rows of dW
  int n0;          // first output column (FWD1: first f column of the gate/up pair)
  int half;        // WGRAD_GU: 0 = gate, 1 = up
  int k_begin;     // WGRAD: first token row of the expert
  int k_len;       // K extent (tokens for WGRAD)
};

template <int MODE>
__device__ __forceinline__ int n_total(const Params& p) {
  if (MODE == FWD1 || MODE == DGRAD1) return p.f;
  if (MODE == WGRAD_DOWN) return p.f;
  return p.d;   // FWD2, DGRAD2, WGRAD_GU
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

// ---------------------------------------------------------------- operand loaders

// A side (rows of the output; the second MFMA operand).
template <int MODE>
__device__ __forceinline__ void load_a(const Params& p, const Tile& t, int kt, uint4 (&reg)[8]) {
  const int tid = threadIdx.x;
  if constexpr (Traits<MODE>::A_KCONTIG) {
    const int K = (MODE == DGRAD2) ? p.f : k_total<MODE>(p);
    int k0 = kt * BK;
    const uint16_t* base = p.a0;
    if (MODE == DGRAD2 && k0 >= p.f) { base = p.a1; k0 -= p.f; }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int r = t.m0 + (tid >> 3) + 32 * i;
      r = r < p.n ? r : p.n - 1;                       // rows past n: clamped, never stored
      reg[i] = ld16(base + static_cast<long long>(r) * K + k0 + 8 * (tid & 7));
    }
  } else {
    // WGRAD: M side is a token-major activation [n][Mtot], read K(token)-strided
    const int Mtot = (MODE == WGRAD_DOWN) ? p.d : p.f;
    const uint16_t* base = (MODE == WGRAD_GU && t.half) ? p.a1 : p.a0;
    const int m = t.m0 + 8 * (tid & 31);
    const int kk = kt * BK + 8 * (tid >> 5);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = kk + i;
      if (m < Mtot && k < t.k_len)
        reg[i] = ld16(base + static_cast<long long>(t.k_begin + k) * Mtot + m);
      else
        reg[i] = make_uint4(0, 0, 0, 0);
    }
  }
}

// B side (columns of the output; the first MFMA operand).
template <int MODE>
__device__ __forceinline__ void load_b(const Params& p, const Tile& t, int kt, uint4 (&reg)[8]) {
  const int tid = threadIdx.x;
  if constexpr (MODE == FWD1) {
    // LDS rows 0..127: W_gate[e] rows n0 + r; rows 128..255: W_up[e] rows n0 + r - 128
    const long long eoff = static_cast<long long>(t.e) * p.f * p.d;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = (tid >> 3) + 32 * i;
      const uint16_t* base = (r < 128) ? p.b0 : p.b1;
      int c = t.n0 + (r & 127);
      c = c < p.f ? c : p.f - 1;
      reg[i] = ld16(base + eoff + static_cast<long long>(c) * p.d + kt * BK + 8 * (tid & 7));
    }
  } else if constexpr (MODE == FWD2) {
    const long long eoff = static_cast<long long>(t.e) * p.d * p.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int c = t.n0 + (tid >> 3) + 32 * i;
      c = c < p.d ? c : p.d - 1;
      reg[i] = ld16(p.b0 + eoff + static_cast<long long>(c) * p.f + kt * BK + 8 * (tid & 7));
    }
  } else {
    // K-strided: element (k, n) at base + k * ld + n, 8 k-rows x 8 n per lane
    const int n = t.n0 + 8 * (tid & 31);
    const int kk = kt * BK + 8 * (tid >> 5);
    if constexpr (MODE == DGRAD1) {
      const uint16_t* base = p.b0 + static_cast<long long>(t.e) * p.d * p.f;   // W_down[e] [d][f]
#pragma unroll
      for (int i = 0; i < 8; ++i)
        reg[i] = (n < p.f) ? ld16(base + static_cast<long long>(kk + i) * p.f + n) : make_uint4(0, 0, 0, 0);
    } else if constexpr (MODE == DGRAD2) {
      // k < f: W_gate[e] [f][d] row k; k >= f: W_up[e] row k - f (a 64-block never straddles)
      const bool up = kk >= p.f;
      const uint16_t* base = (up ? p.b1 : p.b0) + static_cast<long long>(t.e) * p.f * p.d;
      const int k0 = up ? kk - p.f : kk;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        reg[i] = (n < p.d) ? ld16(base + static_cast<long long>(k0 + i) * p.d + n) : make_uint4(0, 0, 0, 0);
    } else {
      // WGRAD: N side is a token-major activation [n][Ntot]
      const int Ntot = n_total<MODE>(p);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int k = kk + i;
        if (n < Ntot && k < t.k_len)
          reg[i] = ld16(p.b0 + static_cast<long long>(t.k_begin + k) * Ntot + n);
        else
          reg[i] = make_uint4(0, 0, 0, 0);
      }
    }
  }
}

template <bool KCONTIG>
__device__ __forceinline__ void store_tile(uint8_t* lds, const uint4 (&reg)[8]) {
  const int tid = threadIdx.x;
  if constexpr (KCONTIG) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<uint4*>(lds + lds_off((tid >> 3) + 32 * i, tid & 7)) = reg[i];
  } else {
    uint4 tr[8];
    transpose8(reg, tr);
    const int rb = tid & 31, kb = tid >> 5;
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<uint4*>(lds + lds_off(8 * rb + j, kb)) = tr[j];
  }
}

// ---------------------------------------------------------------- epilogue helpers

__device__ __forceinline__ void st4(uint16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

// ---------------------------------------------------------------- the kernel

template <int MODE>
__global__ __launch_bounds__(NTH, 1) void grouped_gemm_kernel(Params p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int s_pre[257];     // FWD/DGRAD: prefix of m-tiles per expert
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- device-side schedule: count tiles, remap the block id XCD-major, find the tile
  const int NTW = n_tile_width<MODE>();
  const int ntiles_n = (n_total<MODE>(p) + NTW - 1) / NTW;
  int total_tiles;
  if constexpr (!Traits<MODE>::WGRAD) {
    if (tid == 0) s_pre[0] = 0;
    for (int e = tid; e < p.E; e += NTH) {
      const int cnt = p.offsets[e + 1] - p.offsets[e];
      s_pre[e + 1] = (cnt + BM - 1) / BM;
    }
    __syncthreads();
    if (tid == 0)
      for (int e = 0; e < p.E; ++e) s_pre[e + 1] += s_pre[e];
    __syncthreads();
    total_tiles = s_pre[p.E] * ntiles_n;
  } else {
    const int Mtot = (MODE == WGRAD_DOWN) ? p.d : p.f;
    const int mt = (Mtot + BM - 1) / BM;
    total_tiles = p.E * mt * (MODE == WGRAD_GU ? 2 : 1) * ntiles_n;
  }
  const int tot8 = (total_tiles + 7) & ~7;
  const int bid = blockIdx.x;
  if (bid >= tot8) return;
  const int lid = (bid & 7) * (tot8 >> 3) + (bid >> 3);
  if (lid >= total_tiles) return;

  Tile t;
  int nk;
  if constexpr (!Traits<MODE>::WGRAD) {
    const int mt_glob = lid / ntiles_n;
    const int nt = lid - mt_glob * ntiles_n;
    int lo = 0, hi = p.E - 1;                     // last e with s_pre[e] <= mt_glob
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
    nk = t.k_len / BK;
  } else {
    const int Mtot = (MODE == WGRAD_DOWN) ? p.d : p.f;
    const int mt = (Mtot + BM - 1) / BM;
    const int mtt = mt * (MODE == WGRAD_GU ? 2 : 1);
    const int per_e = mtt * ntiles_n;
    t.e = lid / per_e;
    const int rem = lid - t.e * per_e;
    const int mi = rem / ntiles_n;
    const int nt = rem - mi * ntiles_n;
    t.half = mi >= mt ? 1 : 0;
    t.m0 = (mi - t.half * mt) * BM;
    t.m_end = Mtot;
    t.n0 = nt * BN;
    t.k_begin = p.offsets[t.e];
    t.k_len = p.offsets[t.e + 1] - t.k_begin;
    nk = (t.k_len + BK - 1) / BK;
  }

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // LDS B rows owned by this wave for MFMA tile i (FWD1 pairs gate rows with up rows)
  auto brow = [&](int i) -> int {
    if constexpr (MODE == FWD1) return (i < 4) ? (64 * wn + 16 * i) : (128 + 64 * wn + 16 * (i - 4));
    return 128 * wn + 16 * i;
  };

  uint4 ra[8], rb[8];
  if (nk > 0) {
    load_a<MODE>(p, t, 0, ra);
    load_b<MODE>(p, t, 0, rb);
    store_tile<Traits<MODE>::A_KCONTIG>(lds, ra);
    store_tile<Traits<MODE>::B_KCONTIG>(lds + TILE_BYTES, rb);
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    uint8_t* cur = lds + (kt & 1) * STAGE_BYTES;
    const bool more = kt + 1 < nk;
    if (more) {
      load_a<MODE>(p, t, kt + 1, ra);
      load_b<MODE>(p, t, kt + 1, rb);
    }
    const uint8_t* sa = cur;
    const uint8_t* sb = cur + TILE_BYTES;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int chunk = 4 * s + (lane >> 4);
      bf16x8 fa[8], fb[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        fa[j] = *reinterpret_cast<const bf16x8*>(sa + lds_off(128 * wm + 16 * j + (lane & 15), chunk));
#pragma unroll
      for (int i = 0; i < 8; ++i)
        fb[i] = *reinterpret_cast<const bf16x8*>(sb + lds_off(brow(i) + (lane & 15), chunk));
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[i], fa[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      uint8_t* nxt = lds + ((kt + 1) & 1) * STAGE_BYTES;
      store_tile<Traits<MODE>::A_KCONTIG>(nxt, ra);
      store_tile<Traits<MODE>::B_KCONTIG>(nxt + TILE_BYTES, rb);
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds, for MFMA tile (i, j), output row 16j + lane%16 of the wave's
  // rows and 4 consecutive columns 4*(lane/16) .. +3 of the wave's 16-column group i.
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
    // plain stores: FWD2 -> yexp [n][d]; DGRAD2 -> dxp [n][d]; WGRAD -> dW[e] [Mtot][Ntot]
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

// Upper bound of tiles for a launch, from host scalars only.
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
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&grouped_gemm_kernel<MODE>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    (void)hipGetLastError();
    attr_set = true;
  }
  const long long g = (grid_upper(MODE, p.E, p.n, p.d, p.f) + 7) / 8 * 8;
  MOE_REQUIRE(g < (1LL << 31), MOE_ERR_UNSUPPORTED, "too many tiles");
  grouped_gemm_kernel<MODE><<<static_cast<unsigned>(g), NTH, LDS_BYTES, s>>>(p);
  return check_launch("grouped_gemm_bf16");
}

}  // namespace gg

int gg_bf16_gate_up(int E, int n, int d, int f, const int32_t* offsets, const uint16_t* xp, const uint16_t* wg,
                    const uint16_t* wu, uint16_t* g, uint16_t* u, uint16_t* a, hipStream_t s) {
  gg::Params p{};
  p.offsets = offsets; p.E = E; p.n = n; p.d = d; p.f = f;
  p.a0 = xp; p.b0 = wg; p.b1 = wu; p.o0 = g; p.o1 = u; p.o2 = a;
  return gg::launch<gg::FWD1>(p, s);
}

int gg_bf16_down(int E, int n, int d, int f, const int32_t* offsets, const uint16_t* a, const uint16_t* wd,
                 uint16_t* yexp, hipStream_t s) {
  gg::Params q{};
  q.offsets = offsets; q.E = E; q.n = n; q.d = d; q.f = f;
  q.a0 = a; q.b0 = wd; q.o0 = yexp;
  return gg::launch<gg::FWD2>(q, s);
}

int gg_bf16_backward(int E, int n, int d, int f, const int32_t* offsets, const uint16_t* xp, const uint16_t* g,
                     const uint16_t* u, const uint16_t* a, const uint16_t* dyexp, const uint16_t* wg,
                     const uint16_t* wu, const uint16_t* wd, uint16_t* dg, uint16_t* du, uint16_t* dxp,
                     uint16_t* dwg, uint16_t* dwu, uint16_t* dwd, hipStream_t s) {
  gg::Params p{};
  p.offsets = offsets; p.E = E; p.n = n; p.d = d; p.f = f;
  // dgrad through W_down with the SwiGLU backward epilogue
  p.a0 = dyexp; p.b0 = wd; p.g = g; p.u = u; p.o0 = dg; p.o1 = du;
  if (int st = gg::launch<gg::DGRAD1>(p, s)) return st;
  // wgrad of W_down
  gg::Params w{};
  w.offsets = offsets; w.E = E; w.n = n; w.d = d; w.f = f;
  w.a0 = dyexp; w.b0 = a; w.o0 = dwd;
  if (int st = gg::launch<gg::WGRAD_DOWN>(w, s)) return st;
  // dgrad through W_gate and W_up
  gg::Params q{};
  q.offsets = offsets; q.E = E; q.n = n; q.d = d; q.f = f;
  q.a0 = dg; q.a1 = du; q.b0 = wg; q.b1 = wu; q.o0 = dxp;
  if (int st = gg::launch<gg::DGRAD2>(q, s)) return st;
  // wgrad of W_gate and W_up
  gg::Params r{};
  r.offsets = offsets; r.E = E; r.n = n; r.d = d; r.f = f;
  r.a0 = dg; r.a1 = du; r.b0 = xp; r.o0 = dwg; r.o1 = dwu;
  return gg::launch<gg::WGRAD_GU>(r, s);
}

}  // namespace moe
