// Router projection and its backward, in fp32 ([news] "Ai2 rebuilds Olmo's training stack for
// trillion-parameter MoEs", lead paragraphs: the router scores the experts for every token).
//   forward   logits[T,E]    = x[T,d] @ w_r[d,E]
//   backward  dx_router[T,d] = d_logits[T,E] @ w_r^T
//             dw_r[d,E]      = x^T @ d_logits      (K = T: split over token chunks, partial sums
//                                                   reduced in a fixed order -> deterministic)
//
// fp32 products on the bf16 matrix cores.  Every fp32 operand value v is split exactly into three
// bf16 parts, v = hi + mid + lo: hi = bf16(v) (round to nearest even), mid = bf16(v - hi),
// lo = v - hi - mid.  Each subtraction is exact (its operands lie within a factor of two of each
// other), and what remains after hi and mid spans at most 8 significant bits, so lo is exact too.
// A product of two bf16 parts is exact in fp32, and v_mfma_f32_16x16x32_bf16 accumulates in fp32,
// so the result keeps fp32 accuracy:
//   x (bf16, exact) times an fp32 operand:  x*hi + x*mid + x*lo                 (3 products)
//   fp32 times fp32:  hi*hi + hi*mid + mid*hi + hi*lo + lo*hi + mid*mid  (6; the rest are below
//                     2^-24 of the product)
// MFMA lane layout (as in the grouped GEMMs): an operand lane l holds row (or column) l % 16 and
// K elements 8 (l / 16) .. + 7; the result lane l holds column l % 16 and rows 4 (l / 16) .. + 3.
// Kernels: router_fwd_kernel (forward); split_parts, router_dx_kernel, router_dw_kernel and
// reduce_splits (backward), each described where it is defined.
#include "common.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// v = hi + mid + lo exactly (see the file comment).
__device__ __forceinline__ void split3(const float (&v)[8], bf16x8& hi, bf16x8& mid, bf16x8& lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const __bf16 h = static_cast<__bf16>(v[i]);
    const float r = v[i] - static_cast<float>(h);
    const __bf16 m = static_cast<__bf16>(r);
    hi[i] = h;
    mid[i] = m;
    lo[i] = static_cast<__bf16>(r - static_cast<float>(m));
  }
}

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---- forward: logits = x @ w_r, read-bound on x.  A workgroup takes 128 tokens (four waves of
// 32) x 64 experts.  Per K chunk of 64, the chunk of w_r is split once (hi, mid, lo) into LDS as
// bf16 [part][expert][k] (double-buffered: chunk c + 1 is split while chunk c's products run);
// both the w_r chunks and each wave's x fragments (straight from global memory into registers,
// in the MFMA layout) are loaded FDEPTH chunks ahead, so the token stream keeps enough loads in
// flight without staging x in LDS.  Per accumulator the products run in a fixed order (chunks of
// 64, K halves of 32, then lo, mid, hi).
constexpr int FT = 128, FE = 64, FK = 64;
constexpr int FPITCH = FK + 8;   // bf16 per LDS row (144 bytes: a fragment read spreads over all banks)
constexpr int FDEPTH = 4;        // x chunks in flight per wave


__global__ __launch_bounds__(256) void router_fwd_kernel(const uint16_t* __restrict__ x, const float* __restrict__ w_r,
                                                         int T, int d, int E, float* __restrict__ logits) {
  __shared__ __attribute__((aligned(16))) __bf16 Bs[2][3][FE][FPITCH];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = blockIdx.x * FT + 32 * wave, n0 = blockIdx.y * FE;
  // chunks, padded to a multiple of FDEPTH: the chunks past d read zeros (their products add
  // +0), so every load of the loop is unconditional
  const int nk = ((d + FK - 1) / FK + FDEPTH - 1) / FDEPTH * FDEPTH;
  // All loads are unconditional buffer loads (a lane outside the matrix gets an offset past the
  // buffer and reads zero): without branches around them the compiler counts them exactly and
  // keeps FDEPTH chunks in flight.  x's descriptor starts at the workgroup's first token.
  constexpr uint32_t OOB = 0x80000000u;
  const int tw = blockIdx.x * FT;
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x + static_cast<long long>(tw) * d), 0, min(T - tw, FT) * d * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t wr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(w_r), 0, static_cast<int>(static_cast<long long>(d) * E * 4),
                                        0x00020000);
  // x fragment (row tile i, K half kk) of chunk c: lane row l % 16, K 8 (l / 16) .. + 7.  The
  // lane's part of the offset is fixed; the chunk's is a scalar offset.  A piece at or past d
  // reads zero: its offset is pushed past the buffer (the lane part when the piece straddles d's
  // last 32-wide K block, which only happens when d is not a multiple of 32).
  uint32_t va[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) va[i] = static_cast<uint32_t>(((32 * wave + 16 * i + (lane & 15)) * d + 8 * (lane >> 4)) * 2);
  const int klane = 8 * (lane >> 4);
  auto load_a = [&](int c, bf16x8 (&a)[2][2]) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int kb = c * FK + 32 * kk;
      const int soff = kb < d ? 2 * kb : 0x40000000;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t v = kb + klane < d ? va[i] : OOB;
        a[i][kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(xr, static_cast<int>(v), soff, 0));
      }
    }
  };
  // w_r chunk: thread -> expert n0 + lane, rows k0 + 16 wave .. + 15 (coalesced across lanes);
  // row validity is uniform (a scalar offset past the buffer), expert validity the lane's
  const int be = n0 + lane;
  const uint32_t vb = be < E ? static_cast<uint32_t>((16 * wave * E + be) * 4) : OOB;
  auto load_b = [&](int c, float (&b)[16]) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int k = c * FK + 16 * wave + r;
      const int soff = k < d ? (c * FK + r) * E * 4 : 0x40000000;
      b[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(wr, static_cast<int>(vb), soff, 0));
    }
  };
  auto store_b = [&](int buf, const float (&b)[16]) {
    bf16x8 hi[2], mid[2], lo[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = b[8 * h + i];
      split3(v, hi[h], mid[h], lo[h]);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *reinterpret_cast<bf16x8*>(&Bs[buf][0][lane][16 * wave + 8 * h]) = hi[h];
      *reinterpret_cast<bf16x8*>(&Bs[buf][1][lane][16 * wave + 8 * h]) = mid[h];
      *reinterpret_cast<bf16x8*>(&Bs[buf][2][lane][16 * wave + 8 * h]) = lo[h];
    }
  };

  f32x4 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 ar[FDEPTH][2][2];
  float br[FDEPTH][16];
#pragma unroll
  for (int s = 0; s < FDEPTH; ++s) {
    load_a(s, ar[s]);
    load_b(s, br[s]);
  }
  store_b(0, br[0]);
  load_b(FDEPTH, br[0]);
  __syncthreads();
  // chunk c: its products from Bs[c % 2], and in the same stretch of code (no barrier between,
  // so the split's VALU work overlaps the matrix cores) the split of chunk c + 1 into the other
  // buffer, whose last readers finished before the barrier that closed chunk c - 1
  for (int c0 = 0; c0 < nk; c0 += FDEPTH) {
#pragma unroll
    for (int s = 0; s < FDEPTH; ++s) {
      const int c = c0 + s;
      {
        const int buf = c & 1;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          bf16x8 bp[3][4];
#pragma unroll
          for (int p = 0; p < 3; ++p)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              bp[p][j] = *reinterpret_cast<const bf16x8*>(&Bs[buf][p][16 * j + (lane & 15)][32 * kk + 8 * (lane >> 4)]);
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              f32x4 cc = acc[i][j];
              cc = mfma(ar[s][i][kk], bp[2][j], cc);
              cc = mfma(ar[s][i][kk], bp[1][j], cc);
              cc = mfma(ar[s][i][kk], bp[0][j], cc);
              acc[i][j] = cc;
            }
        }
        const int sn = (s + 1) % FDEPTH;
        store_b(buf ^ 1, br[sn]);
        load_b(c + 1 + FDEPTH, br[sn]);
        load_a(c + FDEPTH, ar[s]);
        __syncthreads();
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = n0 + 16 * j + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + 16 * i + 4 * (lane >> 4) + r;
        if (t < T && e < E) logits[static_cast<long long>(t) * E + e] = acc[i][j][r];
      }
    }
}

// ---- backward.  Both products run on bf16 parts of the fp32 operands, split once per call into
// the workspace (zero-padded to EP = E rounded up to 64 experts, so every fragment load is a whole
// 16-byte piece): d_logits -> dl parts [3][T][EP], w_r -> w parts [3][d][EP].

constexpr int kSplitTokens = 2048;   // tokens per split of the dw_r reduction

int n_splits(int T) { return (T + kSplitTokens - 1) / kSplitTokens; }
int padded_experts(int E) { return (E + 63) / 64 * 64; }

// Workspace layout (byte offsets): dw_r partials [S][d][EP] fp32, dl parts, w parts.
struct BwdWs {
  size_t dls, wps, total;
  BwdWs(int T, int d, int E) {
    auto al = [](size_t b) { return (b + 255) / 256 * 256; };
    const size_t EP = static_cast<size_t>(padded_experts(E));
    dls = al(static_cast<size_t>(n_splits(T)) * d * EP * 4);
    wps = dls + al(3 * static_cast<size_t>(T) * EP * 2);
    total = wps + al(3 * static_cast<size_t>(d) * EP * 2);
  }
};

// rows x E fp32 -> 3 x rows x EP bf16 parts (hi, mid, lo; zero past E).  One thread per output
// element of a part.
__global__ __launch_bounds__(256) void split_parts(const float* __restrict__ src, long long rows, int E, int EP,
                                                   __bf16* __restrict__ dst) {
  const long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  const long long count = rows * EP;
  if (i >= count) return;
  const long long r = i / EP;
  const int e = static_cast<int>(i - r * EP);
  const float v = e < E ? src[r * E + e] : 0.f;
  const __bf16 h = static_cast<__bf16>(v);
  const float rem = v - static_cast<float>(h);
  const __bf16 m = static_cast<__bf16>(rem);
  dst[i] = h;
  dst[count + i] = m;
  dst[2 * count + i] = static_cast<__bf16>(rem - static_cast<float>(m));
}

// dx_router[t][c] = sum_e dl[t][e] w_r[c][e] over the six products of parts whose sum keeps fp32
// accuracy, smallest first: (mid, mid), (lo, hi), (hi, lo), (mid, hi), (hi, mid), (hi, hi)
// (dl part, w part), per 32-expert K half in order.  A workgroup takes 16 NI channels x 64 NJ
// tokens (four waves of 16 NI x 16 NJ); per 64-expert chunk the w parts go to LDS (shared by the
// waves) and each wave's dl fragments come straight from global memory.  The MFMA computes
// D[channel][token], so each lane ends with 4 consecutive channels of one token.  Every output
// element gets the same MFMA sequence whatever NI and NJ, so the tile shape does not change a bit.
// Unfused (128 x 256): the fp32 term is stored.  FUSED (64 x 128, so the small register and LDS
// footprint lets five workgroups (k <= 4; four above) share a compute unit and keep many row loads
// in flight): the permute backward in place of the fp32 store -- dxb[t][c] = bf16(dx_router[t][c]
// + dxp[dest[t][0]][c] + ... + dxp[dest[t][k-1]][c]), summed in fp32 in that order (the router
// term first, then the slots), which is moe_permute_bwd's sum with dx_router as its addend: the
// same bytes as the two calls, without writing and re-reading the fp32 term (4 T d bytes each
// way).  KM: the slot count rounded up to 4, 8 or 16 (unfused: unused).
constexpr int XPITCH = 64 + 8;   // bf16 per LDS row of a w part (144 bytes)

template <int NI, int NJ>
struct DxTile {
  static constexpr int XC = 16 * NI, XT = 64 * NJ;    // workgroup: channels, tokens
  static constexpr int OPITCH = XC + 4;               // fp32 per output staging row
  static constexpr int TPR = 256 / XC;                // threads per channel row of the w fill
  static constexpr int WPT = 64 / TPR / 8;            // 16-byte pieces per part per thread
  static_assert(4 * 16 * OPITCH * 4 <= 3 * XC * XPITCH * 2, "output staging fits the w area");
};

template <bool FUSED, int NI, int NJ, int KM>
__global__ __launch_bounds__(256, FUSED ? (KM <= 4 ? 5 : 4) : 2) void router_dx_kernel(const __bf16* __restrict__ dlp,
                                                                    const __bf16* __restrict__ wp, int T, int d, int EP,
                                                                    float* __restrict__ dx,
                                                                    const uint16_t* __restrict__ dxp,
                                                                    const int32_t* __restrict__ dest, int k,
                                                                    uint16_t* __restrict__ dxb) {
  using Tl = DxTile<NI, NJ>;
  constexpr int XC = Tl::XC, XT = Tl::XT, OPITCH = Tl::OPITCH;
  __shared__ __attribute__((aligned(16))) __bf16 Ws[3][XC][XPITCH];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c0 = blockIdx.x * XC, tw = blockIdx.y * XT + 16 * NJ * wave;
  constexpr uint32_t OOB = 0x80000000u;
  const long long pd = static_cast<long long>(d) * EP, pt = static_cast<long long>(T) * EP;
  // the workgroup's channel rows of each w part, and the wave's token rows of each dl part
  const int crows = min(XC, d - c0);
  const int trows = max(0, min(16 * NJ, T - tw));
  __amdgpu_buffer_rsrc_t wr[3], dr[3];
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    wr[q] = __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(wp + q * pd + static_cast<long long>(c0) * EP), 0,
                                              crows * EP * 2, 0x00020000);
    dr[q] = __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(dlp + q * pt + static_cast<long long>(max(tw, 0)) * EP),
                                              0, trows * EP * 2, 0x00020000);
  }
  f32x4 acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // w chunk loads: thread -> channel row tid / TPR, experts 8 WPT (tid % TPR) .. of each part
  const int wrow = tid / Tl::TPR, wcol = 8 * Tl::WPT * (tid % Tl::TPR);
  for (int e0 = 0; e0 < EP; e0 += 64) {
    uint4 wv[3][Tl::WPT];
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
      for (int u = 0; u < Tl::WPT; ++u)
        wv[q][u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 wr[q], static_cast<int>((wrow * EP + e0 + wcol + 8 * u) * 2), 0, 0));
    if (e0 > 0) __syncthreads();   // the previous chunk's readers are done
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
      for (int u = 0; u < Tl::WPT; ++u) *reinterpret_cast<uint4*>(&Ws[q][wrow][wcol + 8 * u]) = wv[q][u];
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      // the wave's dl fragments of this K half: token tile j, part p (lane row l % 16, experts
      // 8 (l / 16) .. + 7)
      bf16x8 df[3][NJ];
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int r = 16 * j + (lane & 15);
          const uint32_t off = r < trows ? static_cast<uint32_t>((r * EP + e0 + 32 * ks + 8 * (lane >> 4)) * 2) : OOB;
          df[p][j] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(dr[p], static_cast<int>(off), 0, 0));
        }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        bf16x8 wf[3];
#pragma unroll
        for (int q = 0; q < 3; ++q)
          wf[q] = *reinterpret_cast<const bf16x8*>(&Ws[q][16 * i + (lane & 15)][32 * ks + 8 * (lane >> 4)]);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          f32x4 c = acc[i][j];
          c = mfma(wf[1], df[1][j], c);   // (mid, mid)
          c = mfma(wf[0], df[2][j], c);   // (lo, hi)
          c = mfma(wf[2], df[0][j], c);   // (hi, lo)
          c = mfma(wf[0], df[1][j], c);   // (mid, hi)
          c = mfma(wf[1], df[0][j], c);   // (hi, mid)
          c = mfma(wf[0], df[0][j], c);   // (hi, hi)
          acc[i][j] = c;
        }
      }
    }
  }
  // Output through LDS (the w area, free once every wave is past its products): per round, one
  // token tile (16 tokens x the wave's XC channels) goes in as each lane's 4-channel pieces.
  __syncthreads();
  float* stg = reinterpret_cast<float*>(&Ws[0][0][0]) + wave * (16 * OPITCH);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    if constexpr (FUSED) {
      // out as 8-channel pieces (XC / 8 lanes per token); each lane adds its token's k permuted
      // rows (16 bytes of bf16 each), the loads of UG tokens per lane in flight together: 64
      // registers of rows whatever KM
      constexpr int LPT = XC / 8;            // lanes per token
      constexpr int TPI = 64 / LPT;          // tokens per instruction
      constexpr int NU = 16 / TPI;           // instructions per tile
      constexpr int UG = (16 / KM) < NU ? (16 / KM) : NU;
      static_assert(UG >= 1 && NU % UG == 0, "load groups");
      const int c = c0 + 8 * (lane % LPT);
#pragma unroll
      for (int ug = 0; ug < NU; ug += UG) {
        uint4 pv[UG][KM];
        int tv[UG];
#pragma unroll
        for (int u = 0; u < UG; ++u) {
          const int t = tw + 16 * j + TPI * (ug + u) + lane / LPT;
          tv[u] = t < T && c < d ? t : -1;
#pragma unroll
          for (int jj = 0; jj < KM; ++jj) {
            pv[u][jj] = make_uint4(0, 0, 0, 0);
            if (tv[u] >= 0 && jj < k) {
              const long long row = dest[static_cast<long long>(t) * k + jj];
              pv[u][jj] = *reinterpret_cast<const uint4*>(dxp + row * d + c);
            }
          }
        }
        if (ug == 0) {
#pragma unroll
          for (int i = 0; i < NI; ++i)
            *reinterpret_cast<float4*>(stg + (lane & 15) * OPITCH + 16 * i + 4 * (lane >> 4)) =
                make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        }
#pragma unroll
        for (int u = 0; u < UG; ++u) {
          const float* sp = stg + (TPI * (ug + u) + lane / LPT) * OPITCH + 8 * (lane % LPT);
          const float4 a0 = *reinterpret_cast<const float4*>(sp), a1 = *reinterpret_cast<const float4*>(sp + 4);
          float f[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
          for (int jj = 0; jj < KM; ++jj) {
            if (jj < k) {
              const uint4 w = pv[u][jj];
              f[0] += bf16_lo(w.x); f[1] += bf16_hi(w.x); f[2] += bf16_lo(w.y); f[3] += bf16_hi(w.y);
              f[4] += bf16_lo(w.z); f[5] += bf16_hi(w.z); f[6] += bf16_lo(w.w); f[7] += bf16_hi(w.w);
            }
          }
          if (tv[u] >= 0)
            *reinterpret_cast<uint4*>(dxb + static_cast<long long>(tv[u]) * d + c) =
                make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                           pack_bf16x2(f[6], f[7]));
        }
      }
    } else {
      // out as 16-byte pieces of whole row spans, 2 rows per store instruction (XC = 128)
      static_assert(FUSED || XC == 128, "the fp32 store takes 128-channel tiles");
#pragma unroll
      for (int i = 0; i < NI; ++i)
        *reinterpret_cast<float4*>(stg + (lane & 15) * OPITCH + 16 * i + 4 * (lane >> 4)) =
            make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const float4*>(stg + (2 * u + (lane >> 5)) * OPITCH + 4 * (lane & 31));
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int t = tw + 16 * j + 2 * u + (lane >> 5);
        const int cc = c0 + 4 * (lane & 31);
        if (t < T && cc < d) *reinterpret_cast<float4*>(dx + static_cast<long long>(t) * d + cc) = v[u];
      }
    }
  }
}

// dw_r partial of token split z: part[z][c][e] = sum over the split's tokens t of dl[t][e] x[t][c]
// (x exact in bf16: three products, lo, mid, hi).  A workgroup takes 256 channels x 64 experts
// (four waves of 64 channels); per step of 32 tokens, the x rows and the dl parts' rows go to
// LDS in their source layout (token-major), and both MFMA operands come from transposing reads
// (ds_read_b64_tr_b16: 4 x 4 blocks of 16-bit elements across each group of 16 lanes), the
// token axis being the contraction.  Loads run one step ahead in registers.  D[expert][channel]
// per MFMA: each lane ends with 4 consecutive experts of one channel.
constexpr int WC = 256, WSTEP = 32;
constexpr int XSP = WC + 16;   // bf16 per x row in LDS (544 bytes)
constexpr int DSP = 64 + 16;   // bf16 per dl row in LDS (160 bytes)

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Two transposing reads (K rows 8 g + 0..3 and 8 g + 4..7 of the lane's column); the caller
// waits (lgkm_all) before using the halves.
__device__ __forceinline__ void tr_read(s16x4 (&h)[2], uint32_t a0, uint32_t a1) {
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(h[0]) : "v"(a0));
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(h[1]) : "v"(a1));
}
__device__ __forceinline__ bf16x8 tr_join(const s16x4 (&h)[2]) {
  return __builtin_shufflevector(__builtin_bit_cast(bf16x4, h[0]), __builtin_bit_cast(bf16x4, h[1]), 0, 1, 2, 3, 4, 5, 6,
                                 7);
}
// Waits for this wave's LDS reads and ties the 16 fragments read for a step.
__device__ __forceinline__ void lgkm_all(s16x4 (&xh)[4][2], s16x4 (&dh)[4][3][2]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(xh[0][0]), "+v"(xh[0][1]), "+v"(xh[1][0]), "+v"(xh[1][1]), "+v"(xh[2][0]), "+v"(xh[2][1]),
                 "+v"(xh[3][0]), "+v"(xh[3][1]));
#pragma unroll
  for (int a = 0; a < 4; ++a)
    asm volatile("" : "+v"(dh[a][0][0]), "+v"(dh[a][0][1]), "+v"(dh[a][1][0]), "+v"(dh[a][1][1]), "+v"(dh[a][2][0]),
                 "+v"(dh[a][2][1]));
}

__global__ __launch_bounds__(256) void router_dw_kernel(const uint16_t* __restrict__ x, const __bf16* __restrict__ dlp,
                                                        int T, int d, int EP, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) __bf16 Xs[2][WSTEP][XSP];
  __shared__ __attribute__((aligned(16))) __bf16 Ds[2][3][WSTEP][DSP];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c0 = blockIdx.x * WC, e0 = blockIdx.y * 64, z = blockIdx.z;
  const int ts = z * kSplitTokens, te = min(T, ts + kSplitTokens);
  const int nrows = te - ts;
  constexpr uint32_t OOB = 0x80000000u;
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x + static_cast<long long>(ts) * d), 0, nrows * d * 2, 0x00020000);
  const long long pt = static_cast<long long>(T) * EP;
  __amdgpu_buffer_rsrc_t dr[3];
#pragma unroll
  for (int p = 0; p < 3; ++p)
    dr[p] = __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(dlp + p * pt + static_cast<long long>(ts) * EP), 0,
                                              nrows * EP * 2, 0x00020000);
  // step loads: x row tid / 8, channels 32 (tid % 8) .. + 31 (4 pieces); dl part u: token row
  // tid / 8, experts 8 (tid % 8) .. + 7
  const int xrow = tid >> 3, xcol = 32 * (tid & 7);
  auto load = [&](int step, uint4 (&xv)[4], uint4 (&dv)[3]) {
    const int r = step * WSTEP + xrow;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + xcol + 8 * u;
      const uint32_t off = (r < nrows && c < d) ? static_cast<uint32_t>((r * d + c) * 2) : OOB;
      xv[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, static_cast<int>(off), 0, 0));
    }
    const int tr = step * WSTEP + xrow;
    const uint32_t doff = tr < nrows ? static_cast<uint32_t>((tr * EP + e0 + 8 * (tid & 7)) * 2) : OOB;
#pragma unroll
    for (int u = 0; u < 3; ++u)
      dv[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(dr[u], static_cast<int>(doff), 0, 0));
  };
  auto store = [&](int buf, const uint4 (&xv)[4], const uint4 (&dv)[3]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) *reinterpret_cast<uint4*>(&Xs[buf][xrow][xcol + 8 * u]) = xv[u];
#pragma unroll
    for (int u = 0; u < 3; ++u) *reinterpret_cast<uint4*>(&Ds[buf][u][xrow][8 * (tid & 7)]) = dv[u];
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  // transposing-read lane addresses: lane (g, i) reads row 8 g + 4 h + i / 4, columns 4 (i % 4)
  const int g = lane >> 4, i = lane & 15;
  const uint32_t xs0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)&Xs[0][0][0]));
  const uint32_t ds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)&Ds[0][0][0][0]));
  uint32_t xo[2], dof[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = 8 * g + 4 * h + (i >> 2), col = 4 * (i & 3);
    xo[h] = static_cast<uint32_t>((row * XSP + 64 * wave + col) * 2);
    dof[h] = static_cast<uint32_t>((row * DSP + col) * 2);
  }
  const int nsteps = (nrows + WSTEP - 1) / WSTEP;
  uint4 xv[4], dv[3];
  load(0, xv, dv);
  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    store(buf, xv, dv);
    if (step + 1 < nsteps) load(step + 1, xv, dv);
    __syncthreads();
    const uint32_t xb = xs0 + buf * (WSTEP * XSP * 2), db = ds0 + buf * (3 * WSTEP * DSP * 2);
    s16x4 xh[4][2], dh[4][3][2];
#pragma unroll
    for (int b = 0; b < 4; ++b) tr_read(xh[b], xb + xo[0] + 32 * b, xb + xo[1] + 32 * b);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int p = 0; p < 3; ++p)
        tr_read(dh[a][p], db + p * (WSTEP * DSP * 2) + dof[0] + 32 * a, db + p * (WSTEP * DSP * 2) + dof[1] + 32 * a);
    lgkm_all(xh, dh);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const bf16x8 xf = tr_join(xh[b]);
        f32x4 c = acc[a][b];
        c = mfma(tr_join(dh[a][2]), xf, c);
        c = mfma(tr_join(dh[a][1]), xf, c);
        c = mfma(tr_join(dh[a][0]), xf, c);
        acc[a][b] = c;
      }
    }
  }
  // part[z][c][e .. e + 3]
  float* pz = part + static_cast<long long>(z) * d * EP;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int c = c0 + 64 * wave + 16 * b + (lane & 15);
      const int e = e0 + 16 * a + 4 * (lane >> 4);
      if (c < d)
        *reinterpret_cast<float4*>(pz + static_cast<long long>(c) * EP + e) =
            make_float4(acc[a][b][0], acc[a][b][1], acc[a][b][2], acc[a][b][3]);
    }
}

// dw_r[c][e] = sum_z part[z][c][e], z ascending (fixed order)
__global__ __launch_bounds__(256) void reduce_splits(const float* __restrict__ part, int S, int d, int E, int EP,
                                                     float* __restrict__ dw) {
  const long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<long long>(d) * E) return;
  const long long c = i / E;
  const int e = static_cast<int>(i - c * E);
  float s = 0.f;
  for (int z = 0; z < S; ++z) s += part[(static_cast<long long>(z) * d + c) * EP + e];
  dw[i] = s;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_router_project(const uint16_t* x, const float* w_r, int T, int d, int E, float* logits,
                                  void* stream) {
  MOE_CHECK_PTR(x); MOE_CHECK_PTR(w_r); MOE_CHECK_PTR(logits);
  MOE_REQUIRE(T >= 1 && d >= 1 && E >= 1 && E <= 256, MOE_ERR_UNSUPPORTED, "need T, d >= 1 and 1 <= E <= 256");
  MOE_REQUIRE(d % 8 == 0, MOE_ERR_UNSUPPORTED, "router: d must be a multiple of 8");
  MOE_CHECK_ALIGN(x);
  // the kernel's buffer offsets (a 128-token slice of x, all of w_r) stay below 2^31 bytes
  MOE_REQUIRE(static_cast<long long>(FT) * d * 2 < 0x7fffffffLL && static_cast<long long>(d) * E * 4 < 0x7fffffffLL,
              MOE_ERR_UNSUPPORTED, "router: d too large");
  dim3 grid((T + FT - 1) / FT, (E + FE - 1) / FE, 1);
  router_fwd_kernel<<<grid, 256, 0, as_stream(stream)>>>(x, w_r, T, d, E, logits);
  return check_launch("router_project");
}

extern "C" size_t moe_router_bwd_workspace_bytes(int T, int d, int E) {
  if (T < 1 || d < 1 || E < 1) return 0;
  return BwdWs(T, d, E).total;
}

extern "C" int moe_router_project_bwd(const uint16_t* x, const float* w_r, const float* d_logits, int T, int d,
                                      int E, float* dx_router, float* dw_r, void* ws, size_t ws_bytes,
                                      void* stream) {
  MOE_CHECK_PTR(x); MOE_CHECK_PTR(w_r); MOE_CHECK_PTR(d_logits);
  MOE_REQUIRE(T >= 1 && d >= 1 && E >= 1 && E <= 256, MOE_ERR_UNSUPPORTED, "need T, d >= 1 and 1 <= E <= 256");
  MOE_REQUIRE(d % 8 == 0, MOE_ERR_UNSUPPORTED, "router: d must be a multiple of 8");
  MOE_CHECK_ALIGN(x);
  if (dx_router == nullptr && dw_r == nullptr) return MOE_OK;
  const int EP = padded_experts(E);
  // the kernels' buffer offsets stay below 2^31 bytes
  MOE_REQUIRE(static_cast<long long>(kSplitTokens) * d * 2 < 0x7fffffffLL &&
                  static_cast<long long>(DxTile<8, 4>::XC) * EP * 2 < 0x7fffffffLL,
              MOE_ERR_UNSUPPORTED, "router: d too large");
  if (dx_router != nullptr) MOE_CHECK_ALIGN(dx_router);
  const BwdWs L(T, d, E);
  MOE_REQUIRE(ws != nullptr && ws_bytes >= L.total, MOE_ERR_WORKSPACE, "router bwd workspace: need %zu bytes", L.total);
  MOE_CHECK_ALIGN(ws);
  hipStream_t s = as_stream(stream);
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  __bf16* dlp = reinterpret_cast<__bf16*>(w8 + L.dls);
  __bf16* wp = reinterpret_cast<__bf16*>(w8 + L.wps);
  {
    const long long n1 = static_cast<long long>(T) * EP;
    split_parts<<<static_cast<unsigned>((n1 + 255) / 256), 256, 0, s>>>(d_logits, T, E, EP, dlp);
    if (int st = check_launch("router_project_bwd split dl")) return st;
  }
  if (dx_router != nullptr) {
    const long long n2 = static_cast<long long>(d) * EP;
    split_parts<<<static_cast<unsigned>((n2 + 255) / 256), 256, 0, s>>>(w_r, d, E, EP, wp);
    if (int st = check_launch("router_project_bwd split w")) return st;
    using Tl = DxTile<8, 4>;
    dim3 grid((d + Tl::XC - 1) / Tl::XC, (T + Tl::XT - 1) / Tl::XT, 1);
    router_dx_kernel<false, 8, 4, 1><<<grid, 256, 0, s>>>(dlp, wp, T, d, EP, dx_router, nullptr, nullptr, 0, nullptr);
    if (int st = check_launch("router_project_bwd dx")) return st;
  }
  if (dw_r != nullptr) {
    const int S = n_splits(T);
    float* part = reinterpret_cast<float*>(w8);
    dim3 grid((d + WC - 1) / WC, EP / 64, S);
    router_dw_kernel<<<grid, 256, 0, s>>>(x, dlp, T, d, EP, part);
    if (int st = check_launch("router_project_bwd dw partial")) return st;
    const long long count = static_cast<long long>(d) * E;
    reduce_splits<<<static_cast<unsigned>((count + 255) / 256), 256, 0, s>>>(part, S, d, E, EP, dw_r);
    if (int st = check_launch("router_project_bwd dw reduce")) return st;
  }
  return MOE_OK;
}

extern "C" int moe_permute_bwd_router(const uint16_t* dxp, const int32_t* dest, int T, int d, int k,
                                      const float* w_r, const float* d_logits, int E, uint16_t* dx, void* ws,
                                      size_t ws_bytes, void* stream) {
  MOE_CHECK_PTR(dxp); MOE_CHECK_PTR(dest); MOE_CHECK_PTR(w_r); MOE_CHECK_PTR(d_logits); MOE_CHECK_PTR(dx);
  MOE_REQUIRE(T >= 1 && E >= 1 && E <= 256, MOE_ERR_UNSUPPORTED, "need T >= 1 and 1 <= E <= 256");
  MOE_REQUIRE(k >= 1 && k <= 16, MOE_ERR_UNSUPPORTED, "k must be in [1, 16]");
  MOE_REQUIRE(d >= 64 && d % 64 == 0, MOE_ERR_UNSUPPORTED, "d must be a positive multiple of 64");
  MOE_REQUIRE(static_cast<long long>(T) * k < (1LL << 31), MOE_ERR_UNSUPPORTED, "T*k must be < 2^31");
  MOE_CHECK_ALIGN(dxp); MOE_CHECK_ALIGN(dx);
  const int EP = padded_experts(E);
  const BwdWs L(T, d, E);
  MOE_REQUIRE(ws != nullptr && ws_bytes >= L.total, MOE_ERR_WORKSPACE, "router bwd workspace: need %zu bytes", L.total);
  MOE_CHECK_ALIGN(ws);
  hipStream_t s = as_stream(stream);
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  __bf16* dlp = reinterpret_cast<__bf16*>(w8 + L.dls);
  __bf16* wp = reinterpret_cast<__bf16*>(w8 + L.wps);
  const long long n1 = static_cast<long long>(T) * EP, n2 = static_cast<long long>(d) * EP;
  split_parts<<<static_cast<unsigned>((n1 + 255) / 256), 256, 0, s>>>(d_logits, T, E, EP, dlp);
  if (int st = check_launch("permute_bwd_router split dl")) return st;
  split_parts<<<static_cast<unsigned>((n2 + 255) / 256), 256, 0, s>>>(w_r, d, E, EP, wp);
  if (int st = check_launch("permute_bwd_router split w")) return st;
  using Tl = DxTile<4, 2>;
  dim3 grid((d + Tl::XC - 1) / Tl::XC, (T + Tl::XT - 1) / Tl::XT, 1);
  if (k <= 4) router_dx_kernel<true, 4, 2, 4><<<grid, 256, 0, s>>>(dlp, wp, T, d, EP, nullptr, dxp, dest, k, dx);
  else if (k <= 8) router_dx_kernel<true, 4, 2, 8><<<grid, 256, 0, s>>>(dlp, wp, T, d, EP, nullptr, dxp, dest, k, dx);
  else router_dx_kernel<true, 4, 2, 16><<<grid, 256, 0, s>>>(dlp, wp, T, d, EP, nullptr, dxp, dest, k, dx);
  return check_launch("permute_bwd_router");
}
