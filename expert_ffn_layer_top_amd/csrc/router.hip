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
// Tiles: 64 x 64 outputs per 256-thread workgroup (four waves of 32 x 32 = 2 x 2 MFMA tiles), K
// chunks of 64 staged in LDS as fp32 with K contiguous for both operands; the next chunk's global
// loads are issued before the current chunk's products.  MFMA lane layout (as in the grouped
// GEMMs): an operand lane l holds row (or column) l % 16 and K elements 8 (l / 16) .. + 7; the
// result lane l holds column l % 16 and rows 4 (l / 16) .. + 3.
#include "common.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int TM = 64, TN = 64, TK = 64;
constexpr int LDK = TK + 4;   // LDS row pitch (floats): rows of a fragment read fall on distinct banks

// Operand sources.  A is [M][K]; B is [K][N].
enum Src {
  A_X_KC = 0,    // A = x [M=T][K=d] bf16, K contiguous              (forward)
  A_F_KC = 1,    // A = d_logits [M=T][K=E] fp32, K contiguous       (dx)
  A_X_MC = 2,    // A[m][k] = x[k][m], x [K=T][M=d] bf16             (dw)
  B_F_NC = 3,    // B = [K][N] fp32, N contiguous (w_r for forward, d_logits for dw)
  B_F_KC = 4,    // B[k][n] = w_r[n][k], w_r [N=d][K=E] fp32          (dx)
};

// NE consecutive elements (row, col .. col + NE - 1) of a row-major matrix with `pitch` elements
// per row; elements of rows at or past row_lim or columns at or past col_lim read 0.  One vector
// load when the piece is whole and `vec` says fp32 rows are 16-byte aligned.
template <int NE, bool BF16>
__device__ __forceinline__ void piece(const void* __restrict__ base, long long pitch, int row, int row_lim, int col,
                                      int col_lim, bool vec, float* v) {
  if (row >= row_lim) {
#pragma unroll
    for (int i = 0; i < NE; ++i) v[i] = 0.f;
    return;
  }
  const long long off = static_cast<long long>(row) * pitch + col;
  if constexpr (BF16) {
    static_assert(NE == 8, "bf16 pieces are 16 bytes");
    const uint16_t* p = static_cast<const uint16_t*>(base) + off;
    if (col + 8 <= col_lim) {
      const uint4 t = *reinterpret_cast<const uint4*>(p);
      const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) { v[2 * i] = bf16_lo(w[i]); v[2 * i + 1] = bf16_hi(w[i]); }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = col + i < col_lim ? bf16_to_f32(p[i]) : 0.f;
    }
  } else {
    static_assert(NE == 4, "fp32 pieces are 16 bytes");
    const float* p = static_cast<const float*>(base) + off;
    if (vec && col + 4 <= col_lim) {
      const float4 t = *reinterpret_cast<const float4*>(p);
      v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = col + i < col_lim ? p[i] : 0.f;
    }
  }
}

// One workgroup's share of a chunk: 16 values per thread for each operand (64 x 64 = 4096).
struct Chunk {
  float a[16], b[16];
};

// Piece p of a chunk: bf16 sources in 8-element pieces (8 per 64-element row), fp32 sources in
// 4-element pieces (16 per row); "row" is the source's row (m, or k for x^T), "col" its
// contiguous index.
template <int SA>
__device__ __forceinline__ void load_a(const void* __restrict__ A, int M, int K, int k_hi, int m0, int k0, int tid,
                                       bool vec, float (&a)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (SA == A_X_KC) {          // x [T][d]: row m, col k
      if (i < 2) {
        const int p = tid + 256 * i;
        piece<8, true>(A, K, m0 + (p >> 3), M, k0 + (p & 7) * 8, k_hi, vec, a + 8 * i);
      }
    } else if constexpr (SA == A_X_MC) {   // x [T][d]: row k, col m
      if (i < 2) {
        const int p = tid + 256 * i;
        piece<8, true>(A, M, k0 + (p >> 3), k_hi, m0 + (p & 7) * 8, M, vec, a + 8 * i);
      }
    } else {                               // d_logits [T][E]: row m, col k
      const int p = tid + 256 * i;
      piece<4, false>(A, K, m0 + (p >> 4), M, k0 + (p & 15) * 4, k_hi, vec, a + 4 * i);
    }
  }
}

template <int SB>
__device__ __forceinline__ void load_b(const float* __restrict__ B, int N, int K, int k_hi, int n0, int k0, int tid,
                                       bool vec, float (&b)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = tid + 256 * i;
    if constexpr (SB == B_F_NC) piece<4, false>(B, N, k0 + (p >> 4), k_hi, n0 + (p & 15) * 4, N, vec, b + 4 * i);
    else piece<4, false>(B, K, n0 + (p >> 4), N, k0 + (p & 15) * 4, k_hi, vec, b + 4 * i);   // w_r [d][E]
  }
}

// Chunk registers -> LDS, both operands as [row][k] fp32.
template <int SA, int SB>
__device__ __forceinline__ void store_chunk(const Chunk& ch, float (*As)[LDK], float (*Bs)[LDK], int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = tid + 256 * i;
    if constexpr (SA == A_X_KC) {
      if (i < 2) {
#pragma unroll
        for (int j = 0; j < 8; ++j) As[p >> 3][(p & 7) * 8 + j] = ch.a[8 * i + j];
      }
    } else if constexpr (SA == A_X_MC) {
      if (i < 2) {
#pragma unroll
        for (int j = 0; j < 8; ++j) As[(p & 7) * 8 + j][p >> 3] = ch.a[8 * i + j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) As[p >> 4][(p & 15) * 4 + j] = ch.a[4 * i + j];
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = tid + 256 * i;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (SB == B_F_NC) Bs[(p & 15) * 4 + j][p >> 4] = ch.b[4 * i + j];
      else Bs[p >> 4][(p & 15) * 4 + j] = ch.b[4 * i + j];
    }
  }
}

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

__device__ __forceinline__ void frag(const float (*S)[LDK], int row, int k, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(&S[row][k]);
  const float4 b = *reinterpret_cast<const float4*>(&S[row][k + 4]);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// C[M][N] (row pitch N; + blockIdx.z * c_split for split-K partials) over K range
// [blockIdx.z * k_chunk, + k_chunk).  `vec`: fp32 rows are 16-byte aligned (their length is a
// multiple of 4), so fp32 pieces load as float4.
template <int SA, int SB>
__global__ __launch_bounds__(256) void router_gemm(const void* __restrict__ A, const float* __restrict__ B, int M,
                                                   int N, int K, int k_chunk, int vec, float* __restrict__ C,
                                                   long long c_split) {
  constexpr bool A_EXACT = SA != A_F_KC;   // bf16 source: one part
  __shared__ __attribute__((aligned(16))) float As[TM][LDK];
  __shared__ __attribute__((aligned(16))) float Bs[TN][LDK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.x * TM, n0 = blockIdx.y * TN;
  const int k_lo = blockIdx.z * k_chunk;
  const int k_hi = min(K, k_lo + k_chunk);   // loads past k_hi read zero
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  Chunk ch;
  auto fetch = [&](int k0) {
    load_a<SA>(A, M, K, k_hi, m0, k0, tid, vec, ch.a);
    load_b<SB>(B, N, K, k_hi, n0, k0, tid, vec, ch.b);
  };
  fetch(k_lo);
  for (int k0 = k_lo; k0 < k_hi; k0 += TK) {
    __syncthreads();
    store_chunk<SA, SB>(ch, As, Bs, tid);
    __syncthreads();
    if (k0 + TK < k_hi) fetch(k0 + TK);
#pragma unroll
    for (int kk = 0; kk < TK; kk += 32) {
      const int kf = kk + 8 * (lane >> 4);
      bf16x8 ah[2], am[2], al[2], bh[2], bm[2], bl[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float v[8];
        frag(As, 32 * wm + 16 * t + (lane & 15), kf, v);
        split3(v, ah[t], am[t], al[t]);
        frag(Bs, 32 * wn + 16 * t + (lane & 15), kf, v);
        split3(v, bh[t], bm[t], bl[t]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          f32x4 c = acc[i][j];
          if constexpr (A_EXACT) {
            c = mfma(ah[i], bl[j], c);
            c = mfma(ah[i], bm[j], c);
            c = mfma(ah[i], bh[j], c);
          } else {
            c = mfma(am[i], bm[j], c);
            c = mfma(al[i], bh[j], c);
            c = mfma(ah[i], bl[j], c);
            c = mfma(am[i], bh[j], c);
            c = mfma(ah[i], bm[j], c);
            c = mfma(ah[i], bh[j], c);
          }
          acc[i][j] = c;
        }
    }
  }
  float* Cz = C + blockIdx.z * c_split;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + 32 * wn + 16 * j + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 32 * wm + 16 * i + 4 * (lane >> 4) + r;
        if (m < M && n < N) Cz[static_cast<long long>(m) * N + n] = acc[i][j][r];
      }
    }
}

// ---- forward: logits = x @ w_r, read-bound on x.  A workgroup takes 128 tokens (four waves of
// 32) x 64 experts.  Per K chunk of 64, the chunk of w_r is split once (hi, mid, lo) into LDS as
// bf16 [part][expert][k] (double-buffered: chunk c + 1 is split while chunk c's products run);
// both the w_r chunks and each wave's x fragments (straight from global memory into registers,
// in the MFMA layout) are loaded FDEPTH chunks ahead, so the token stream keeps enough loads in
// flight without staging x in LDS.  The
// products and their order per accumulator (chunks of 64, K halves of 32, then lo, mid, hi) are
// those of router_gemm, so the logits are the same bits.
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

// fp32 rows of E elements load as float4 when E is a multiple of 4 and both bases are 16-byte aligned.
int f32_rows_aligned(int E, const void* p, const void* q) {
  return E % 4 == 0 && (reinterpret_cast<uintptr_t>(p) & 15u) == 0 && (reinterpret_cast<uintptr_t>(q) & 15u) == 0;
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
  return static_cast<size_t>(n_splits(T)) * d * E * sizeof(float);
}

extern "C" int moe_router_project_bwd(const uint16_t* x, const float* w_r, const float* d_logits, int T, int d,
                                      int E, float* dx_router, float* dw_r, void* ws, size_t ws_bytes,
                                      void* stream) {
  MOE_CHECK_PTR(x); MOE_CHECK_PTR(w_r); MOE_CHECK_PTR(d_logits);
  MOE_REQUIRE(T >= 1 && d >= 1 && E >= 1 && E <= 256, MOE_ERR_UNSUPPORTED, "need T, d >= 1 and 1 <= E <= 256");
  MOE_REQUIRE(d % 8 == 0, MOE_ERR_UNSUPPORTED, "router: d must be a multiple of 8");
  MOE_CHECK_ALIGN(x);
  const int vec = f32_rows_aligned(E, w_r, d_logits);
  hipStream_t s = as_stream(stream);
  if (dw_r != nullptr) {
    const size_t need = moe_router_bwd_workspace_bytes(T, d, E);
    MOE_REQUIRE(ws != nullptr && ws_bytes >= need, MOE_ERR_WORKSPACE, "router bwd workspace: need %zu bytes", need);
  }
  if (dx_router != nullptr) {
    // dx[t, c] = sum_e dl[t, e] * w_r[c, e]
    dim3 grid((T + TM - 1) / TM, (d + TN - 1) / TN, 1);
    router_gemm<A_F_KC, B_F_KC><<<grid, 256, 0, s>>>(d_logits, w_r, T, d, E, E, vec, dx_router, 0);
    if (int st = check_launch("router_project_bwd dx")) return st;
  }
  if (dw_r != nullptr) {
    // dw_r[c, e] = sum_t x[t, c] * dl[t, e], split over token chunks
    const int S = n_splits(T);
    float* part = static_cast<float*>(ws);
    dim3 grid((d + TM - 1) / TM, (E + TN - 1) / TN, S);
    router_gemm<A_X_MC, B_F_NC><<<grid, 256, 0, s>>>(x, d_logits, d, E, T, kSplitTokens, vec, part,
                                                     static_cast<long long>(d) * E);
    if (int st = check_launch("router_project_bwd dw partial")) return st;
    const long long count = static_cast<long long>(d) * E;
    reduce_splits<<<static_cast<unsigned>((count + 255) / 256), 256, 0, s>>>(part, S, count, dw_r);
    if (int st = check_launch("router_project_bwd dw reduce")) return st;
  }
  return MOE_OK;
}
