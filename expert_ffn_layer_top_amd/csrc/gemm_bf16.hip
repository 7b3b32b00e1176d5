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
// Tiling: 256 x 256 outputs per 256-thread workgroup, four waves in a 2 x 2 grid, each wave
// owning 128 x 128 outputs as 8 x 8 MFMA 16x16 tiles (256 fp32 accumulators per lane).  K steps
// of 32 run through a four-deep ring of LDS stages (4 x 32 KiB).
//
// Operand staging.  Every operand tile goes from HBM/L2 to LDS by the LDS-DMA form of the
// buffer load (16 bytes per lane, written to a wave-contiguous 1 KiB LDS span), so no operand
// passes through VGPRs and no wave spends VALU time on copies.  Two LDS layouts:
//   KC  operand stored K-contiguous (rows x K): LDS [256 rows][32 k] (64 B rows); MFMA fragments
//       are one ds_read_b128 per lane.
//   KS  operand stored K-strided (K x columns: the weights in the dgrad products, the
//       token-major activations in the wgrad products): LDS [32 k][256 columns] (512 B rows),
//       kept in the source layout; fragments come from two ds_read_b64_tr_b16 per lane, which
//       transpose 4 x 4 blocks of 16-bit elements across each group of 16 lanes.
// Both layouts XOR-swizzle 16-byte chunks within a row (the DMA source address of each lane is
// permuted to match), so fragment reads spread over all LDS banks.  Buffer descriptors bound
// every operand to its valid extent: rows past an expert's last row (wgrad K tails) and past
// the tensor end read as zeros.
//
// Pipeline.  Three K steps are in flight in a four-stage ring.  In the middle of step kt (after
// its fourth MFMA row) every wave waits for its own DMA of tile kt+1 and joins a barrier; past it,
// all of tile kt+1 is in LDS and every wave has finished reading tile kt-1, so the DMA of tile
// kt+3 goes into that stage.  Fragment reads run one MFMA row ahead of their use.  The MFMA
// computes the transposed tile (weights / N side as the first operand), so each lane ends with 4
// consecutive output columns of one row.
#include <type_traits>

#include "common.h"

namespace moe {
namespace gg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 32;
constexpr int NTH = 256;
constexpr int OP_BYTES = BM * BK * 2;             // 16 KiB per operand per stage
constexpr uint32_t RSRC_WORD3 = 0x00020000u;      // raw buffer, 32-bit data format (gfx9 family)

// Four stages of each operand as eight distinct LDS objects: the compiler tracks outstanding
// LDS-DMA per object, so a fragment read of one stage never waits for the DMA into another.  The
// A stages fill the first 64 KiB and the B stages the next, so every fragment address is one
// per-lane base plus a 16-bit immediate.
__shared__ __attribute__((aligned(1024))) uint8_t lds_a0[OP_BYTES];
__shared__ __attribute__((aligned(1024))) uint8_t lds_a1[OP_BYTES];
__shared__ __attribute__((aligned(1024))) uint8_t lds_a2[OP_BYTES];
__shared__ __attribute__((aligned(1024))) uint8_t lds_a3[OP_BYTES];
__shared__ __attribute__((aligned(1024))) uint8_t lds_b0[OP_BYTES];
__shared__ __attribute__((aligned(1024))) uint8_t lds_b1[OP_BYTES];
__shared__ __attribute__((aligned(1024))) uint8_t lds_b2[OP_BYTES];
__shared__ __attribute__((aligned(1024))) uint8_t lds_b3[OP_BYTES];

template <int S>
__device__ __forceinline__ uint8_t* stage_a() {
  if constexpr (S == 0) return lds_a0;
  else if constexpr (S == 1) return lds_a1;
  else if constexpr (S == 2) return lds_a2;
  else return lds_a3;
}

template <int S>
__device__ __forceinline__ uint8_t* stage_b() {
  if constexpr (S == 0) return lds_b0;
  else if constexpr (S == 1) return lds_b1;
  else if constexpr (S == 2) return lds_b2;
  else return lds_b3;
}

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
// the accumulator and fragment arrays stay static (dynamic indexing would demote them to scratch).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

template <int MODE>
struct Traits {
  static constexpr bool A_KC = (MODE <= DGRAD2);   // M side K-contiguous
  static constexpr bool B_KC = (MODE <= FWD2);     // N side K-contiguous
  static constexpr bool WGRAD = (MODE >= WGRAD_DOWN);
};

// ---------------------------------------------------------------- LDS layouts

// KC: row r (64 bytes = 4 chunks), chunk c stored at chunk position c ^ ((r >> 2) & 3).
__device__ __forceinline__ int kc_off(int r, int c) { return r * 64 + ((c ^ ((r >> 2) & 3)) << 4); }
// KS: row k (512 bytes = 32 chunks), chunk c stored at chunk position c ^ ks_swz(k); the XOR
// value is even, so the two chunks of an aligned 32-byte pair stay adjacent.
__device__ __forceinline__ int ks_swz(int k) { return ((k & 3) | (((k >> 3) & 1) << 2)) << 1; }
__device__ __forceinline__ int ks_off(int k, int c) { return k * 512 + ((c ^ ks_swz(k)) << 4); }

// ---------------------------------------------------------------- buffer descriptors / DMA

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, long long bytes) {
  const int nrec = bytes <= 0 ? 0 : (bytes >= 0x7fffffffLL ? 0x7fffffff : static_cast<int>(bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, nrec, RSRC_WORD3);
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds), 16, voff, soff, 0, 0);
}

// Waits for this wave's LDS reads and all but the newest N of its vector-memory operations,
// then joins the workgroup barrier.  The memory clobber keeps the compiler from moving LDS
// accesses across it.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// ---------------------------------------------------------------- tile -> work

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
__device__ __forceinline__ int m_total_wgrad(const Params& p) { return MODE == WGRAD_DOWN ? p.d : p.f; }

template <int MODE>
__device__ __forceinline__ int n_tile_width() { return MODE == FWD1 ? BN / 2 : BN; }

template <int MODE>
__device__ __forceinline__ int k_total(const Params& p) {
  if (MODE == FWD1 || MODE == DGRAD1) return p.d;
  if (MODE == FWD2) return p.f;
  if (MODE == DGRAD2) return 2 * p.f;
  return 0;
}

// Per-lane DMA offsets of one operand (4 instructions per lane per stage) and the descriptors.
struct OpLoad {
  __amdgpu_buffer_rsrc_t r0, r1;   // r1: second tensor (FWD1 B: W_up; DGRAD2: dU / W_up)
  int vo[4];
  int step;                        // bytes to advance per K step (KC: 64; KS: 32 rows)
};

// KC operand, rows [row0, row0 + 256) of a row-major tensor with `ldb` bytes per row.
// Wave w fills LDS rows 64w .. 64w + 63 with 4 instructions of 16 rows each.
__device__ __forceinline__ void kc_offsets(int ldb, int (&vo)[4]) {
  const int L = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = (L & 3) ^ ((L >> 4) & 3);
#pragma unroll
  for (int i = 0; i < 4; ++i) vo[i] = (64 * w + 16 * i + (L >> 2)) * ldb + 16 * c;
}

// KS operand, 32 K-rows x 256 columns; wave w fills LDS rows 8w .. 8w + 7, 2 rows per instruction.
__device__ __forceinline__ void ks_offsets(int ldb, int (&vo)[4]) {
  const int L = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kr = 8 * w + 2 * i + (L >> 5);
    vo[i] = kr * ldb + 16 * ((L & 31) ^ ks_swz(kr));
  }
}

// Issues the DMA of K step kt into stage S.  Steps past the last one (kt >= nk) read through an
// empty descriptor, so the stage fills with zeros and its MFMAs add nothing.
template <int MODE, int S>
__device__ __forceinline__ void issue_stage(const Params& p, const OpLoad& la, const OpLoad& lb, int kt, int nk) {
  const int w = threadIdx.x >> 6;
  const bool valid = kt < nk;
  uint8_t* da = stage_a<S>() + w * 4096;
  uint8_t* db = stage_b<S>() + w * 4096;
  // ---- A (M side)
  {
    __amdgpu_buffer_rsrc_t r = la.r0;
    int soff = kt * la.step;
    if constexpr (MODE == DGRAD2) {
      const int kf = p.f / BK;   // K steps per half
      if (kt >= kf) { r = la.r1; soff = (kt - kf) * la.step; }
    }
    if (!valid) { r = make_rsrc(p.a0, 0); soff = 0; }
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(r, da + i * 1024, la.vo[i], soff);
  }
  // ---- B (N side)
  {
    __amdgpu_buffer_rsrc_t r = lb.r0;
    int soff = kt * lb.step;
    if constexpr (MODE == FWD1) {
      if (w >= 2) r = lb.r1;
    } else if constexpr (MODE == DGRAD2) {
      const int kf = p.f / BK;
      if (kt >= kf) { r = lb.r1; soff = (kt - kf) * lb.step; }
    }
    if (!valid) { r = make_rsrc(p.b0, 0); soff = 0; }
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(r, db + i * 1024, lb.vo[i], soff);
  }
}

// ---------------------------------------------------------------- fragments

// Per-lane fragment addresses, computed once.
//   KC: fragment q (rows 16q .. 16q + 15 of the stage) of lane l sits at kc + 1024 q: the chunk
//       swizzle (r >> 2) & 3 of row r = 16q + l % 16 does not depend on q.
//   KS: fragment q (columns 16q .. 16q + 15) of lane l, half h (K = 8 (l / 16) + 4h .. + 3), is
//       read at ks[h] ^ (q << 5): row k = 8 (l / 16) + 4h + (l % 16) / 4 and columns
//       16q + 4 (l % 4) .. + 3; the row's swizzle only flips bits 5..7 of the byte address, the
//       same bits q selects.
struct FragAddr {
  int a_kc, b_kc;
  int a_ks[2], b_ks[2];
};

__device__ __forceinline__ int kc_lane() {
  const int l = threadIdx.x & 63;
  return kc_off(l & 15, l >> 4);
}

__device__ __forceinline__ int ks_lane(int h) {
  const int l = threadIdx.x & 63;
  const int g = l >> 4, i = l & 15;
  const int k = 8 * g + 4 * h + (i >> 2);
  const int col = 4 * (i & 3);                   // fragment 0
  return ks_off(k, col >> 3) + ((col & 7) << 1);
}

template <int MODE>
__device__ __forceinline__ FragAddr frag_addr() {
  FragAddr fa;
  fa.a_kc = fa.b_kc = kc_lane();
  fa.a_ks[0] = fa.b_ks[0] = ks_lane(0);
  fa.a_ks[1] = fa.b_ks[1] = ks_lane(1);
  return fa;
}

__device__ __forceinline__ bf16x8 read_kc(const uint8_t* stage, int lane_off, int q) {
  return *reinterpret_cast<const bf16x8*>(stage + lane_off + 1024 * q);
}

__device__ __forceinline__ bf16x8 read_ks(const uint8_t* stage, const int (&ks)[2], int q) {
  bf16x4 h[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const uint8_t* pa = stage + (ks[hh] ^ (q << 5));
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(pa));
    h[hh] = __builtin_bit_cast(bf16x4, v);
  }
  return bf16x8{h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
}

// Fragment q of the LDS B tile for MFMA tile i (FWD1 pairs gate rows with up rows), in units of
// 16 rows (KC) or 16 columns (KS).
template <int MODE>
__device__ __forceinline__ int bfrag(int wn, int i) {
  if constexpr (MODE == FWD1) return (i < 4) ? (4 * wn + i) : (8 + 4 * wn + (i - 4));
  return 8 * wn + i;
}

// The transposing read takes no immediate offset, so every (stage, fragment, half) address is a
// VGPR.  The KS bases are laundered once per K step so the compiler forms those addresses next to
// their reads instead of keeping all of them live across the loop.
// acc += x * y on the matrix core, accumulating in place in AGPRs.  Written as inline asm so the
// accumulator is tied to one register quad for the whole loop: the builtin's untied form made the
// register allocator rotate all 256 accumulators through copies every K step.  Callers cover the
// hazards the compiler cannot see: wait states between the accumulator initialisation and the
// first MFMA, and between the last MFMA and any VALU read of the accumulators.
__device__ __forceinline__ void mfma_acc(f32x4& c, const bf16x8& x, const bf16x8& y) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(x), "v"(y));
}

// Orders the (zero) initialisation of one accumulator row before later volatile asm.
__device__ __forceinline__ void pin_acc_row(f32x4 (&r)[8]) {
  asm volatile("" : "+a"(r[0]), "+a"(r[1]), "+a"(r[2]), "+a"(r[3]), "+a"(r[4]), "+a"(r[5]), "+a"(r[6]),
               "+a"(r[7]));
}

template <int MODE, int S>
__device__ __forceinline__ bf16x8 read_a(const FragAddr& fa, int q) {
  if constexpr (Traits<MODE>::A_KC) return read_kc(stage_a<S>(), fa.a_kc, q);
  else return read_ks(stage_a<S>(), fa.a_ks, q);
}

template <int MODE, int S>
__device__ __forceinline__ bf16x8 read_b(const FragAddr& fa, int q) {
  if constexpr (Traits<MODE>::B_KC) return read_kc(stage_b<S>(), fa.b_kc, q);
  else return read_ks(stage_b<S>(), fa.b_ks, q);
}

// One K step of tile kt (stage S), as 8 rows of 8 MFMAs; row i multiplies B fragment i by the
// 8 A fragments.  Fragment reads run one row ahead of their use, from two small register sets:
//   a[8]      A fragments of tile kt (read during the previous step), an[8] those of tile kt+1;
//   b[2]      ping-pong: B fragment i+1 is read while row i runs.
// The barrier before row 4 opens tile kt+1: each wave first waits for its own DMA of that tile
// (one newer tile, 8 DMA instructions, stays in flight), and past the barrier every wave has
// also finished reading tile kt-1, whose stage then receives the DMA of tile kt+3.  Rows 4..7
// read the A fragments of tile kt+1 (two per row) and row 7 its first B fragment.
template <int MODE, int S>
__device__ __forceinline__ void k_step(const Params& p, const OpLoad& la, const OpLoad& lb, const FragAddr& fa_in,
                                       int kt, int nk, bf16x8 (&a)[8], bf16x8 (&an)[8], bf16x8 (&b)[2],
                                       f32x4 (&acc)[8][8]) {
  constexpr int SN = (S + 1) & 3;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qa = 8 * (wave >> 1), wn = wave & 1;
  FragAddr fa = fa_in;
  if constexpr (!Traits<MODE>::A_KC) asm volatile("" : "+v"(fa.a_ks[0]), "+v"(fa.a_ks[1]));
  if constexpr (!Traits<MODE>::B_KC) asm volatile("" : "+v"(fa.b_ks[0]), "+v"(fa.b_ks[1]));
  constexpr int RB = Traits<MODE>::B_KC ? 1 : 2;   // LDS reads per B fragment
  constexpr int RA = Traits<MODE>::A_KC ? 1 : 2;
  static_for<0, 8>([&](auto i) {
    if constexpr (i == 4) {
      wait_barrier<8>();
      issue_stage<MODE, (S + 3) & 3>(p, la, lb, kt + 3, nk);
    }
    if constexpr (i < 7) b[(i + 1) & 1] = read_b<MODE, S>(fa, bfrag<MODE>(wn, i + 1));
    else b[0] = read_b<MODE, SN>(fa, bfrag<MODE>(wn, 0));
    if constexpr (i >= 4) {
      an[2 * (i - 4)] = read_a<MODE, SN>(fa, qa + 2 * (i - 4));
      an[2 * (i - 4) + 1] = read_a<MODE, SN>(fa, qa + 2 * (i - 4) + 1);
    }
    static_for<0, 8>([&](auto j) {
      mfma_acc(acc[i][j], b[i & 1], a[j]);
    });
    // keep this row's reads ahead of its MFMAs (the DMA of row 4 goes first)
    if constexpr (i == 4) __builtin_amdgcn_sched_group_barrier(0x020, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, RB + (i >= 4 ? 2 * RA : 0), 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  });
}

// ---------------------------------------------------------------- epilogue helpers

__device__ __forceinline__ void st4(uint16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

// ---------------------------------------------------------------- the kernel

template <int MODE>
__global__ __launch_bounds__(NTH, 1) void grouped_gemm_kernel(Params p) {
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
    const int mt = (m_total_wgrad<MODE>(p) + BM - 1) / BM;
    total_tiles = p.E * mt * (MODE == WGRAD_GU ? 2 : 1) * ntiles_n;
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
  } else {
    const int Mtot = m_total_wgrad<MODE>(p);
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
  }
  const int nk = (t.k_len + BK - 1) / BK;

  // ---- operand descriptors, bounded to each operand's valid extent
  OpLoad la, lb;
  if constexpr (MODE == FWD1 || MODE == FWD2 || MODE == DGRAD1) {
    const int K = k_total<MODE>(p);
    const long long rem_rows = static_cast<long long>(p.n) - t.m0;
    la.r0 = make_rsrc(p.a0 + static_cast<long long>(t.m0) * K, rem_rows * K * 2);
    la.r1 = la.r0;
    la.step = BK * 2;
    kc_offsets(K * 2, la.vo);
  } else if constexpr (MODE == DGRAD2) {
    const long long rem_rows = static_cast<long long>(p.n) - t.m0;
    la.r0 = make_rsrc(p.a0 + static_cast<long long>(t.m0) * p.f, rem_rows * p.f * 2);
    la.r1 = make_rsrc(p.a1 + static_cast<long long>(t.m0) * p.f, rem_rows * p.f * 2);
    la.step = BK * 2;
    kc_offsets(p.f * 2, la.vo);
  } else {
    // WGRAD: M side is a token-major activation [n][Mtot], rows k_begin .. k_begin + k_len
    const int Mtot = m_total_wgrad<MODE>(p);
    const uint16_t* base = (MODE == WGRAD_GU && t.half) ? p.a1 : p.a0;
    la.r0 = make_rsrc(base + static_cast<long long>(t.k_begin) * Mtot + t.m0,
                      static_cast<long long>(t.k_len) * Mtot * 2 - t.m0 * 2);
    la.r1 = la.r0;
    la.step = BK * Mtot * 2;
    ks_offsets(Mtot * 2, la.vo);
  }
  if constexpr (MODE == FWD1) {
    // rows 0..127 of the B tile: W_gate[e] rows n0 ..; rows 128..255: W_up[e] rows n0 ..
    const long long eoff = static_cast<long long>(t.e) * p.f * p.d;
    const long long bytes = static_cast<long long>(p.f - t.n0) * p.d * 2;
    lb.r0 = make_rsrc(p.b0 + eoff + static_cast<long long>(t.n0) * p.d, bytes);
    lb.r1 = make_rsrc(p.b1 + eoff + static_cast<long long>(t.n0) * p.d, bytes);
    lb.step = BK * 2;
    // wave w fills rows 64w..: waves 2, 3 start again at row 0 of W_up
    const int L = tid & 63;
    const int c = (L & 3) ^ ((L >> 4) & 3);
#pragma unroll
    for (int i = 0; i < 4; ++i) lb.vo[i] = (64 * (wave & 1) + 16 * i + (L >> 2)) * p.d * 2 + 16 * c;
  } else if constexpr (MODE == FWD2) {
    // W_down[e] [d][f], rows n0 .. (K = f contiguous)
    const long long eoff = static_cast<long long>(t.e) * p.d * p.f;
    lb.r0 = make_rsrc(p.b0 + eoff + static_cast<long long>(t.n0) * p.f, static_cast<long long>(p.d - t.n0) * p.f * 2);
    lb.r1 = lb.r0;
    lb.step = BK * 2;
    kc_offsets(p.f * 2, lb.vo);
  } else if constexpr (MODE == DGRAD1) {
    // W_down[e] [d][f]: element (k = d index, n = f index), rows k, columns n0 ..
    const long long eoff = static_cast<long long>(t.e) * p.d * p.f;
    lb.r0 = make_rsrc(p.b0 + eoff + t.n0, static_cast<long long>(p.d) * p.f * 2 - t.n0 * 2);
    lb.r1 = lb.r0;
    lb.step = BK * p.f * 2;
    ks_offsets(p.f * 2, lb.vo);
  } else if constexpr (MODE == DGRAD2) {
    // W_gate[e] / W_up[e] [f][d]: element (k = f index, n = d index)
    const long long eoff = static_cast<long long>(t.e) * p.f * p.d;
    const long long bytes = static_cast<long long>(p.f) * p.d * 2 - t.n0 * 2;
    lb.r0 = make_rsrc(p.b0 + eoff + t.n0, bytes);
    lb.r1 = make_rsrc(p.b1 + eoff + t.n0, bytes);
    lb.step = BK * p.d * 2;
    ks_offsets(p.d * 2, lb.vo);
  } else {
    // WGRAD: N side is a token-major activation [n][Ntot]
    const int Ntot = n_total<MODE>(p);
    lb.r0 = make_rsrc(p.b0 + static_cast<long long>(t.k_begin) * Ntot + t.n0,
                      static_cast<long long>(t.k_len) * Ntot * 2 - t.n0 * 2);
    lb.r1 = lb.r0;
    lb.step = BK * Ntot * 2;
    ks_offsets(Ntot * 2, lb.vo);
  }

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (nk > 0) {
    // ---- prologue: tiles 0..2 in flight, fragments of tile 0 read
    // accumulator initialisation -> first MFMA: pin the zeroed registers ahead of the wait states
#pragma unroll
    for (int i = 0; i < 8; ++i) pin_acc_row(acc[i]);
    asm volatile("s_nop 7" ::: "memory");
    issue_stage<MODE, 0>(p, la, lb, 0, nk);
    issue_stage<MODE, 1>(p, la, lb, 1, nk);
    issue_stage<MODE, 2>(p, la, lb, 2, nk);
    const FragAddr fa = frag_addr<MODE>();
    wait_barrier<16>();
    const int qa = 8 * (wave >> 1);
    bf16x8 fa0[8], fa1[8], fb[2];
#pragma unroll
    for (int j = 0; j < 8; ++j) fa0[j] = read_a<MODE, 0>(fa, qa + j);
    fb[0] = read_b<MODE, 0>(fa, bfrag<MODE>(wn, 0));
    for (int kt = 0; kt < nk; kt += 4) {
      k_step<MODE, 0>(p, la, lb, fa, kt, nk, fa0, fa1, fb, acc);
      k_step<MODE, 1>(p, la, lb, fa, kt + 1, nk, fa1, fa0, fb, acc);
      k_step<MODE, 2>(p, la, lb, fa, kt + 2, nk, fa0, fa1, fb, acc);
      k_step<MODE, 3>(p, la, lb, fa, kt + 3, nk, fa1, fa0, fb, acc);
    }
    // no LDS-DMA may still be writing when the workgroup ends; the last MFMA results settle
    // before the epilogue's VALU reads them
    asm volatile("s_waitcnt vmcnt(0)\n\ts_nop 15\n\ts_nop 15" ::: "memory");
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
      const int Mtot = m_total_wgrad<MODE>(p);
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
  const long long g = (grid_upper(MODE, p.E, p.n, p.d, p.f) + 7) / 8 * 8;
  MOE_REQUIRE(g < (1LL << 31), MOE_ERR_UNSUPPORTED, "too many tiles");
  // every buffer offset the kernel forms stays below 2^31 bytes
  MOE_REQUIRE(static_cast<long long>(p.n) * (p.d > p.f ? p.d : p.f) * 2 < 0x7fffffffLL &&
                  static_cast<long long>(p.d) * p.f * 2 < 0x7fffffffLL,
              MOE_ERR_UNSUPPORTED, "bf16 grouped GEMM: an operand exceeds 2 GiB");
  grouped_gemm_kernel<MODE><<<static_cast<unsigned>(g), NTH, 0, s>>>(p);
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
