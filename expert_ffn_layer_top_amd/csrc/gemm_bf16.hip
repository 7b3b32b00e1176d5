// Device-scheduled grouped GEMMs of the SwiGLU expert FFN in bf16 with fp32 accumulation,
// forward and backward, on CDNA4 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// [news] "Ai2 rebuilds Olmo's training stack for trillion-parameter MoEs", "Routing work stays on
// the GPU": the many small per-expert products run as one grouped operation; [card]
// "Supercharging Olmo-core ...", "Summary": the grouped GEMMs are device-scheduled.  Here the
// per-expert row counts exist only on the device: every workgroup reads `offsets`, builds the
// per-expert tile prefix and walks its own list of (expert, m-tile, n-tile) tiles.  The host
// launches at most one workgroup per compute unit (persistent); the tile list follows from the
// device-side counts alone.
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
// owning 128 x 128 outputs as 8 x 8 MFMA 16x16 tiles (256 fp32 accumulators per lane, AGPRs).  K
// steps of 64 (two 32-deep MFMA sub-steps) run through two LDS rings of 32 KiB stages: two
// stages for the M-side operand and three for the N-side one (the whole 160 KiB LDS).
//
// Operand staging.  Every operand tile goes from HBM/L2 to LDS by the LDS-DMA form of the
// buffer load (16 bytes per lane, written to a wave-contiguous 1 KiB LDS span), so no operand
// passes through VGPRs and no wave spends VALU time on copies.  Two LDS layouts:
//   KC  operand stored K-contiguous (rows x K): LDS [256 rows][64 k] (128 B rows: each row one
//       whole 128-byte line of the source); MFMA fragments are one ds_read_b128 per lane.
//   KS  operand stored K-strided (K x columns: the weights in the dgrad products, the
//       token-major activations in the wgrad products): LDS [64 k][256 columns] (512 B rows),
//       kept in the source layout; fragments come from two ds_read_b64_tr_b16 per lane, which
//       transpose 4 x 4 blocks of 16-bit elements across each group of 16 lanes.
// Both layouts XOR-swizzle 16-byte chunks within a row (the DMA source address of each lane is
// permuted to match), so fragment reads spread over all LDS banks.  Buffer descriptors bound
// every operand to its valid extent: rows past an expert's last row (wgrad K tails) and past
// the tensor end read as zeros, and so do K steps past the last one.
//
// Pipeline.  Each wave streams one operand (waves 0, 1 the N side, waves 2, 3 the M side, half a
// stage each).  Half-way through step g (before its second sub-step) every wave waits for its own
// DMA of step g+1 and joins a barrier; past it all of step g+1 is in LDS, every wave has finished
// reading the M-side stage of step g and the N-side stage of step g-1, so the DMA of step g+2
// goes into those stages.  Steps run on across a workgroup's tiles: the DMA of the next tile's
// first steps overlaps the current tile's last steps and its epilogue.  B fragment reads run two
// MFMA rows ahead of their use, A fragments a sub-step ahead.  They are inline asm with explicit lgkmcnt waits: the stage is a
// runtime index, and the compiler, which cannot tell which stage a read touches, would otherwise
// wait for every outstanding DMA before each read.  The MFMA computes the transposed tile
// (weights / N side as the first operand), so each lane ends with 4 consecutive output columns
// of one row.
#include <type_traits>

#include "common.h"
#include "gemm_epilogue.h"
#include "gemm_sched.h"

namespace moe {
namespace gg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;                            // K per stage (two 32-deep MFMA sub-steps)
constexpr int NTH = 256;
constexpr int OP_BYTES = BM * BK * 2;             // 32 KiB per operand per stage
// Stage counts of the two operand rings (A = M side, B = N side), 160 KiB in all.  The N side
// (the weights in the forward and dgrad products) mostly misses L2, so its ring is deeper.
constexpr int NA = 2;
constexpr int NB = 3;
constexpr int A_RING = 0;
constexpr int B_RING = NA * OP_BYTES;
constexpr int DMA_ROWS = 8;                       // MFMA rows a stage's DMA issue is spread over
constexpr uint32_t RSRC_WORD3 = 0x00020000u;      // raw buffer, 32-bit data format (gfx9 family)

__shared__ __attribute__((aligned(1024))) uint8_t lds_ring[(NA + NB) * OP_BYTES];

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// LDS byte address of a generic pointer into lds_ring.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_u8*)(p)));
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
  int cm, cn;           // tile cell shape (set by launch)
  int cell_mt;          // cells apply to experts of at most this many m-tiles
  int cell_deal;        // weight gradients: cells apply under the round-robin deal too
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

// KC: row r (128 bytes = 8 chunks), chunk c stored at chunk position c ^ ((r >> 1) & 7).
__device__ __forceinline__ int kc_swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int kc_off(int r, int c) { return r * 128 + ((c ^ kc_swz(r)) << 4); }
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

// The experts with rows (empty = false) or without (empty = true), as four 64-bit ballots (bit l
// of m[r]: expert 64 r + l), wave-uniform so that they stay in scalar registers.
struct ExpertSet {
  unsigned long long m[4];
  int total;
};

__device__ __forceinline__ ExpertSet expert_set(const int32_t* __restrict__ offsets, int E, bool empty) {
  const int lane = threadIdx.x & 63;
  ExpertSet s;
  s.total = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int ex = 64 * r + lane;
    const bool in = ex < E && ((offsets[ex + 1] - offsets[ex]) == 0) == empty;
    s.m[r] = __ballot(in);
    s.total += __popcll(s.m[r]);
  }
  return s;
}

// The j-th expert of the set (j < s.total).
__device__ __forceinline__ int expert_set_nth(const ExpertSet& s, int j) {
  int r = 0;
  unsigned long long m = s.m[0];
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    const int c = __popcll(m);
    if (j >= c) {
      j -= c;
      m = s.m[q + 1];
      r = q + 1;
    }
  }
  int pos = 0;
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) {
    const int c = __popcll(m & ((1ull << w) - 1));
    if (j >= c) {
      j -= c;
      m >>= w;
      pos += w;
    }
  }
  return 64 * r + pos;
}

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

// DMA roles: waves 0 and 1 stream the N-side operand (B), waves 2 and 3 the M-side operand (A);
// each wave fills one half of its operand's stage (8 instructions of 1 KiB).  Splitting by
// operand gives each ring its own depth: a wave's vmcnt counts only its own loads, and vector
// loads complete in order, so one deep ring shared with a shallow one would wait at the
// shallow one's pace.
struct OpLoad {
  int vo[16];                      // per-lane byte offsets of the 16 DMA instructions (tile-independent)
  int step;                        // bytes to advance per K step (KC: 128; KS: 64 rows)
};

// One tile's DMA sources for this wave: its operand bounded to the tile's valid extent.
struct TileSrc {
  __amdgpu_buffer_rsrc_t r0, r1;   // r1: second tensor (FWD1 B half 1: W_up; DGRAD2 K >= f)
  int nreal;                       // K steps holding data
  int nk;                          // K steps run: at least 2 (see the kernel's pipeline notes)
};

// KC operand: LDS rows 128h .. 128h + 127 of a [256 rows][64 k] stage, 8 rows per instruction;
// `row0` is the first tensor row of this half (relative to the descriptor base), `ldb` the
// tensor's bytes per row.  Each row is one whole 128-byte line.
__device__ __forceinline__ void kc_offsets(int row0, int ldb, int (&vo)[16]) {
  const int L = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 8 * i + (L >> 3);              // LDS row within the half (128h is a multiple of 16)
    vo[i] = (row0 + r) * ldb + 16 * ((L & 7) ^ kc_swz(r));
  }
}

// KS operand: K-rows 32h .. 32h + 31 of a [64 k][256 columns] stage, 2 rows per instruction.
__device__ __forceinline__ void ks_offsets(int h, int ldb, int (&vo)[16]) {
  const int L = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int kr = 32 * h + 2 * i + (L >> 5);
    vo[i] = kr * ldb + 16 * ((L & 31) ^ ks_swz(kr));
  }
}

// Where this wave's DMA of K step k of the tile `src` reads and writes (stage `st` of its
// operand's ring).  Steps past the tile's data (k >= nreal) read through an empty descriptor,
// so the stage fills with zeros and its MFMAs add nothing.
struct StageIssue {
  __amdgpu_buffer_rsrc_t r;
  int soff;
  uint8_t* dst;
};

template <int MODE>
__device__ __forceinline__ StageIssue stage_issue(const Params& p, const OpLoad& ld, const TileSrc& src, bool role_b,
                                                  int h, int k, int st) {
  StageIssue si;
  si.r = src.r0;
  si.soff = k * ld.step;
  if constexpr (MODE == FWD1) {
    if (role_b && h) si.r = src.r1;
  } else if constexpr (MODE == DGRAD2) {
    const int kf = p.f / BK;   // K steps per half
    if (k >= kf) { si.r = src.r1; si.soff = (k - kf) * ld.step; }
  }
  if (k >= src.nreal) { si.r = make_rsrc(p.a0, 0); si.soff = 0; }
  si.dst = lds_ring + (role_b ? B_RING : A_RING) + st * OP_BYTES + h * (OP_BYTES / 2);
  return si;
}

// DMA instructions FIRST .. FIRST + COUNT - 1 (of 16, 1 KiB each) of a stage.
template <int FIRST, int COUNT>
__device__ __forceinline__ void issue_part(const OpLoad& ld, const StageIssue& si) {
#pragma unroll
  for (int i = FIRST; i < FIRST + COUNT; ++i) dma16(si.r, si.dst + i * 1024, ld.vo[i], si.soff);
}

template <int MODE>
__device__ __forceinline__ void issue_stage(const Params& p, const OpLoad& ld, const TileSrc& src, bool role_b, int h,
                                            int k, int st) {
  issue_part<0, 16>(ld, stage_issue<MODE>(p, ld, src, role_b, h, k, st));
}

// ---------------------------------------------------------------- fragments

// Per-lane fragment addresses within a stage, computed once.
//   KC: fragment q (rows 16q .. 16q + 15 of the stage) of lane l, sub-step s, sits at
//       kc[s] + 2048 q: the chunk swizzle (r >> 1) & 7 of row r = 16q + l % 16 does not depend
//       on q.
//   KS: fragment q (columns 16q .. 16q + 15) of lane l, half h (K = 32s + 8 (l / 16) + 4h .. + 3),
//       is read at (ks[h] ^ (q << 5)) + 16384 s: row k = 32s + 8 (l / 16) + 4h + (l % 16) / 4 and
//       columns 16q + 4 (l % 4) .. + 3; the row's swizzle only flips bits 5..7 of the byte
//       address, the same bits q selects, and does not depend on s.
struct FragAddr {
  uint32_t kc[2];     // per 32-deep sub-step
  uint32_t ks[2];     // per half; sub-step 1 is 32 rows (16 KiB) further
};

__device__ __forceinline__ FragAddr frag_addr() {
  const int l = threadIdx.x & 63;
  FragAddr fa;
  fa.kc[0] = kc_off(l & 15, l >> 4);
  fa.kc[1] = kc_off(l & 15, 4 + (l >> 4));
  const int g = l >> 4, i = l & 15;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int k = 8 * g + 4 * h + (i >> 2);
    const int col = 4 * (i & 3);                 // fragment 0
    fa.ks[h] = ks_off(k, col >> 3) + ((col & 7) << 1);
  }
  return fa;
}

// LDS reads as asm: the compiler neither reorders them across the barrier asm nor inserts DMA
// waits before them; callers wait with lgkm_wait before using the results.
template <int OFF>
__device__ __forceinline__ void ds_b128(bf16x8& v, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
}

template <int OFF>
__device__ __forceinline__ void ds_tr(s16x4& v, uint32_t addr) {
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
}

// Fragment q of sub-step S of the operand whose stage starts at LDS address `base`.
template <bool KC, int S, int Q>
__device__ __forceinline__ void read_frag(bf16x8& v, uint32_t base, const FragAddr& fa, int qoff) {
  if constexpr (KC) {
    ds_b128<2048 * Q>(v, base + fa.kc[S] + 2048 * qoff);
  } else {
    s16x4 h0, h1;
    const uint32_t q = static_cast<uint32_t>(Q + qoff) << 5;
    ds_tr<16384 * S>(h0, base + (fa.ks[0] ^ q));
    ds_tr<16384 * S>(h1, base + (fa.ks[1] ^ q));
    v = __builtin_shufflevector(__builtin_bit_cast(bf16x4, h0), __builtin_bit_cast(bf16x4, h1), 0, 1, 2, 3, 4, 5,
                                6, 7);
  }
}

// Waits until at most N LDS reads are outstanding; ties the fragments the next MFMAs use, so
// those MFMAs cannot be scheduled above the wait.
template <int N>
__device__ __forceinline__ void lgkm_wait(bf16x8& b, bf16x8 (&a)[8]) {
  asm volatile("s_waitcnt lgkmcnt(%9)"
               : "+v"(b), "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]),
                 "+v"(a[7])
               : "n"(N));
}

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

// Fragment index (units of 16 rows/columns) of B fragment i for wave column wn (FWD1 pairs gate
// rows with up rows).
template <int MODE, int I>
__device__ __forceinline__ constexpr int bfrag_c() {
  if constexpr (MODE == FWD1) return (I < 4) ? I : 8 + (I - 4);
  return I;
}

template <int MODE>
__device__ __forceinline__ int bfrag_base(int wn) {
  return MODE == FWD1 ? 4 * wn : 8 * wn;
}

// LDS reads a row of MFMAs may still leave outstanding when it waits for its B fragment (see
// sub_step), capped at the counter's 4-bit range (a lower count only waits for more).
template <int I, int RA, int RB>
__device__ __forceinline__ constexpr int row_wait() {
  constexpr int n = 2 * RB + RA * (I == 0 || I == 5 ? 2 : I == 1 || I == 4 ? 4 : I == 2 || I == 3 ? 6 : 0);
  return n < 15 ? n : 15;
}

// Waits until at most N LDS reads are outstanding and ties every fragment register, so no MFMA
// can be scheduled above the wait (used before the epilogue with N = 0).
template <int N>
__device__ __forceinline__ void lgkm_wait_all(bf16x8 (&b)[4], bf16x8 (&a)[8]) {
  asm volatile("s_waitcnt lgkmcnt(%12)"
               : "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]), "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]),
                 "+v"(a[4]), "+v"(a[5]), "+v"(a[6]), "+v"(a[7])
               : "n"(N));
}

// One 32-deep sub-step S of a K step, as 8 rows of 8 MFMAs; row i multiplies B fragment i by the
// 8 A fragments.  Registers: a[8] the A fragments of this sub-step, an[8] the next sub-step's
// (read two per row in rows 0..3), b[4] the B fragments, read two rows ahead of their use (row i
// reads row i + 2's; rows 6 and 7 read the next sub-step's rows 0 and 1).  Each row waits only
// for its own B fragment (row_wait counts the reads issued after it).
// Sub-step 0 reads the A fragments of sub-step 1 from the same stages.  Sub-step 1 opens K step
// g+1 (g = this step in the workgroup's stream of steps over its tiles) before its row 0: each
// wave waits for its own DMA of that step and joins a barrier; past it all of step g+1 is in
// LDS and every wave has finished reading the M-side stage of step g (its A fragments are all in
// registers) and the N-side stage of step g-1, so the DMA of step g+2 (step `ik` of tile `isrc`)
// goes into those stages.  Rows 0..3 then read step g+1's first A fragments, and rows 6, 7 its
// first two B fragments.
template <int MODE, int S>
__device__ __forceinline__ void sub_step(const Params& p, const OpLoad& ld, bool role_b, int h, const FragAddr& fa,
                                         const TileSrc& isrc, int ik, int sa, int sb, bf16x8 (&a)[8], bf16x8 (&an)[8],
                                         bf16x8 (&b)[4], f32x4 (&acc)[8][8]) {
  constexpr bool AKC = Traits<MODE>::A_KC, BKC = Traits<MODE>::B_KC;
  constexpr int RA = AKC ? 1 : 2;   // LDS reads per A fragment
  constexpr int RB = BKC ? 1 : 2;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qa = 8 * (wave >> 1);
  const int qb = bfrag_base<MODE>(wave & 1);
  const int san = sa + 1 == NA ? 0 : sa + 1;
  const int sbn = sb + 1 == NB ? 0 : sb + 1, sbp = sb == 0 ? NB - 1 : sb - 1;
  const uint32_t ring = lds_addr(lds_ring);
  const uint32_t a_cur = ring + A_RING + sa * OP_BYTES, a_nxt = ring + A_RING + san * OP_BYTES;
  const uint32_t b_cur = ring + B_RING + sb * OP_BYTES, b_nxt = ring + B_RING + sbn * OP_BYTES;
  StageIssue si{};
  static_for<0, 8>([&](auto i) {
    if constexpr (S == 1) {
      if constexpr (i == 0) {
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        si = stage_issue<MODE>(p, ld, isrc, role_b, h, ik, role_b ? sbp : sa);
      }
      // the stage's 16 DMA instructions, spread over the rows so the wave keeps issuing MFMAs
      // while the texture addresser works through them
      if constexpr (i < DMA_ROWS) issue_part<i * (16 / DMA_ROWS), 16 / DMA_ROWS>(ld, si);
    }
    if constexpr (i < 6) read_frag<BKC, S, bfrag_c<MODE, i + 2>()>(b[(i + 2) & 3], b_cur, fa, qb);
    else if constexpr (S == 0) read_frag<BKC, 1, bfrag_c<MODE, i - 6>()>(b[(i + 2) & 3], b_cur, fa, qb);
    else read_frag<BKC, 0, bfrag_c<MODE, i - 6>()>(b[(i + 2) & 3], b_nxt, fa, qb);
    if constexpr (i < 4) {
      constexpr int SN = S ^ 1;
      const uint32_t src = S == 0 ? a_cur : a_nxt;
      read_frag<AKC, SN, 2 * i>(an[2 * i], src, fa, qa);
      read_frag<AKC, SN, 2 * i + 1>(an[2 * i + 1], src, fa, qa);
    }
    lgkm_wait<row_wait<i, RA, RB>()>(b[i & 3], a);
    static_for<0, 8>([&](auto j) { mfma_acc(acc[i][j], b[i & 3], a[j]); });
  });
}

// ---------------------------------------------------------------- epilogue

// The LDS each wave stages its epilogue through: 8 KiB of the N-side stage of the tile's last K
// step, which every wave has finished reading (the stream's next DMA into it comes a step later).
constexpr int STG_BYTES = 8192;

// ---------------------------------------------------------------- the kernel

using gsched::MTiles;

// Writes the tile's results from the accumulators (helpers in gemm_epilogue.h): SwiGLU on the
// gate/up product, its backward on the down dgrad, plain stores otherwise.
template <int MODE>
__device__ __forceinline__ void epilogue(const Params& p, const Tile& t, f32x4 (&acc)[8][8], int wm, int wn,
                                         int lane, uint32_t stg) {
  const int row0 = t.m0 + 128 * wm;
  const int rows_valid = t.m_end - row0;
  if constexpr (MODE == FWD1) {
    gep::epi_gate_up<2>(acc, p.o0, p.o1, p.o2, p.n, p.f, row0, rows_valid, t.n0 + 64 * wn, stg, lane);
  } else if constexpr (MODE == DGRAD1) {
    // 16 rows per round: the dgrad epilogue holds G, U and dA values at once, so its rounds are
    // half the plain ones' to stay within the registers the K loop leaves
    gep::epi_swiglu_bwd<1>(acc, p.g, p.u, p.o0, p.o1, p.n, p.f, row0, rows_valid, t.n0 + 128 * wn, stg, lane);
  } else {
    // FWD2 -> yexp [n][d]; DGRAD2 -> dxp [n][d]; WGRAD -> dW[e] [Mtot][Ntot]
    const int Ntot = n_total<MODE>(p);
    uint16_t* out = p.o0;
    long long rows = p.n;
    if constexpr (Traits<MODE>::WGRAD) {
      const int Mtot = m_total_wgrad<MODE>(p);
      out = (MODE == WGRAD_GU && t.half ? p.o1 : p.o0) + static_cast<long long>(t.e) * Mtot * Ntot;
      rows = Mtot;
    }
    gep::epi_plain<2>(acc, out, rows, Ntot, row0, rows_valid, t.n0 + 128 * wn, stg, lane);
  }
}

// The tile with linear id `lid` (< the launch's tile count).  Each expert owns a contiguous run
// of ids (experts in order); inside it, tiles follow cell_order in cells of cm x cn (plain
// n-fastest for experts of more than cell_mt m-tiles), so the tiles running at once on one XCD
// share their operand slices in its L2.
template <int MODE>
__device__ __forceinline__ Tile tile_at(const Params& p, const MTiles& mts, const ExpertSet& nz, int ntiles_n, int cm,
                                        int cn, int lid) {
  Tile t;
  if constexpr (!Traits<MODE>::WGRAD) {
    const int mt_glob = lid / ntiles_n;
    int e, first;
    gsched::mtile_find(mts, mt_glob, e, first);
    e = __builtin_amdgcn_readfirstlane(e);
    first = __builtin_amdgcn_readfirstlane(first);
    const int mt_e = (p.offsets[e + 1] - p.offsets[e] + BM - 1) / BM;
    const bool cells = mt_e <= p.cell_mt;
    int mi, nt;
    gsched::cell_order(lid - first * ntiles_n, mt_e, ntiles_n, cells ? cm : 1, cells ? cn : 1 << 20, mi, nt);
    t.e = e;
    t.m0 = p.offsets[e] + mi * BM;
    t.m_end = p.offsets[e + 1];
    t.n0 = nt * n_tile_width<MODE>();
    t.half = 0;
    t.k_begin = 0;
    t.k_len = k_total<MODE>(p);
  } else {
    const int Mtot = m_total_wgrad<MODE>(p);
    const int mt = (Mtot + BM - 1) / BM;
    const int per_e = mt * (MODE == WGRAD_GU ? 2 : 1) * ntiles_n;
    // ids run over the experts with rows only (the kernel writes the others' zero tiles first)
    const int j = lid / per_e;
    t.e = expert_set_nth(nz, j);
    const int rem = lid - j * per_e;
    int mi, nt;
    gsched::cell_order(rem, mt * (MODE == WGRAD_GU ? 2 : 1), ntiles_n, cm, cn, mi, nt);
    t.half = mi >= mt ? 1 : 0;
    t.m0 = (mi - t.half * mt) * BM;
    t.m_end = Mtot;
    t.n0 = nt * BN;
    t.k_begin = p.offsets[t.e];
    t.k_len = p.offsets[t.e + 1] - t.k_begin;
  }
  // The tile is uniform across the workgroup, but it was derived through shuffles and loads the
  // compiler treats as per-lane; without this, every buffer descriptor built from it would be
  // "divergent" and each DMA instruction wrapped in a readfirstlane waterfall loop.
  t.e = __builtin_amdgcn_readfirstlane(t.e);
  t.m0 = __builtin_amdgcn_readfirstlane(t.m0);
  t.m_end = __builtin_amdgcn_readfirstlane(t.m_end);
  t.n0 = __builtin_amdgcn_readfirstlane(t.n0);
  t.half = __builtin_amdgcn_readfirstlane(t.half);
  t.k_begin = __builtin_amdgcn_readfirstlane(t.k_begin);
  t.k_len = __builtin_amdgcn_readfirstlane(t.k_len);
  return t;
}

// A source that supplies only zeros (the step after a workgroup's last tile).
__device__ __forceinline__ TileSrc empty_src(const Params& p) {
  TileSrc s;
  s.r0 = make_rsrc(p.a0, 0);
  s.r1 = s.r0;
  s.nreal = 0;
  s.nk = 2;
  return s;
}

// This wave's DMA operand for tile t, bounded to its valid extent (role: waves 0, 1 -> B;
// 2, 3 -> A; h = which half of the stage the wave fills).
template <int MODE>
__device__ __forceinline__ TileSrc tile_src(const Params& p, const Tile& t, bool role_b, int h) {
  TileSrc s;
  s.nreal = (t.k_len + BK - 1) / BK;
  s.nk = s.nreal < 2 ? 2 : s.nreal;
  if (!role_b) {
    if constexpr (MODE == FWD1 || MODE == FWD2 || MODE == DGRAD1) {
      const int K = k_total<MODE>(p);
      const long long rem_rows = static_cast<long long>(p.n) - t.m0;
      s.r0 = make_rsrc(p.a0 + static_cast<long long>(t.m0) * K, rem_rows * K * 2);
      s.r1 = s.r0;
    } else if constexpr (MODE == DGRAD2) {
      const long long rem_rows = static_cast<long long>(p.n) - t.m0;
      s.r0 = make_rsrc(p.a0 + static_cast<long long>(t.m0) * p.f, rem_rows * p.f * 2);
      s.r1 = make_rsrc(p.a1 + static_cast<long long>(t.m0) * p.f, rem_rows * p.f * 2);
    } else {
      // WGRAD: M side is a token-major activation [n][Mtot], rows k_begin .. k_begin + k_len
      const int Mtot = m_total_wgrad<MODE>(p);
      const uint16_t* base = (MODE == WGRAD_GU && t.half) ? p.a1 : p.a0;
      s.r0 = make_rsrc(base + static_cast<long long>(t.k_begin) * Mtot + t.m0,
                       static_cast<long long>(t.k_len) * Mtot * 2 - t.m0 * 2);
      s.r1 = s.r0;
    }
  } else {
    if constexpr (MODE == FWD1) {
      // B half 0: W_gate[e] rows n0 .. n0 + 127; half 1: W_up[e] rows n0 .. n0 + 127
      const long long eoff = static_cast<long long>(t.e) * p.f * p.d;
      const long long bytes = static_cast<long long>(p.f - t.n0) * p.d * 2;
      s.r0 = make_rsrc(p.b0 + eoff + static_cast<long long>(t.n0) * p.d, bytes);
      s.r1 = make_rsrc(p.b1 + eoff + static_cast<long long>(t.n0) * p.d, bytes);
    } else if constexpr (MODE == FWD2) {
      // W_down[e] [d][f], rows n0 .. (K = f contiguous)
      const long long eoff = static_cast<long long>(t.e) * p.d * p.f;
      s.r0 = make_rsrc(p.b0 + eoff + static_cast<long long>(t.n0) * p.f,
                       static_cast<long long>(p.d - t.n0) * p.f * 2);
      s.r1 = s.r0;
    } else if constexpr (MODE == DGRAD1) {
      // W_down[e] [d][f]: element (k = d index, n = f index), rows k, columns n0 ..
      const long long eoff = static_cast<long long>(t.e) * p.d * p.f;
      s.r0 = make_rsrc(p.b0 + eoff + t.n0, static_cast<long long>(p.d) * p.f * 2 - t.n0 * 2);
      s.r1 = s.r0;
    } else if constexpr (MODE == DGRAD2) {
      // W_gate[e] / W_up[e] [f][d]: element (k = f index, n = d index)
      const long long eoff = static_cast<long long>(t.e) * p.f * p.d;
      const long long bytes = static_cast<long long>(p.f) * p.d * 2 - t.n0 * 2;
      s.r0 = make_rsrc(p.b0 + eoff + t.n0, bytes);
      s.r1 = make_rsrc(p.b1 + eoff + t.n0, bytes);
    } else {
      // WGRAD: N side is a token-major activation [n][Ntot]
      const int Ntot = n_total<MODE>(p);
      s.r0 = make_rsrc(p.b0 + static_cast<long long>(t.k_begin) * Ntot + t.n0,
                       static_cast<long long>(t.k_len) * Ntot * 2 - t.n0 * 2);
      s.r1 = s.r0;
    }
  }
  return s;
}

// This wave's per-lane DMA offsets and K-step stride; they depend on the launch, not the tile.
template <int MODE>
__device__ __forceinline__ OpLoad op_load(const Params& p, bool role_b, int h) {
  OpLoad ld;
  if (!role_b) {
    if constexpr (MODE == FWD1 || MODE == FWD2 || MODE == DGRAD1) {
      ld.step = BK * 2;
      kc_offsets(128 * h, k_total<MODE>(p) * 2, ld.vo);
    } else if constexpr (MODE == DGRAD2) {
      ld.step = BK * 2;
      kc_offsets(128 * h, p.f * 2, ld.vo);
    } else {
      const int Mtot = m_total_wgrad<MODE>(p);
      ld.step = BK * Mtot * 2;
      ks_offsets(h, Mtot * 2, ld.vo);
    }
  } else {
    if constexpr (MODE == FWD1) {
      ld.step = BK * 2;
      kc_offsets(0, p.d * 2, ld.vo);
    } else if constexpr (MODE == FWD2) {
      ld.step = BK * 2;
      kc_offsets(128 * h, p.f * 2, ld.vo);
    } else if constexpr (MODE == DGRAD1) {
      ld.step = BK * p.f * 2;
      ks_offsets(h, p.f * 2, ld.vo);
    } else if constexpr (MODE == DGRAD2) {
      ld.step = BK * p.d * 2;
      ks_offsets(h, p.d * 2, ld.vo);
    } else {
      const int Ntot = n_total<MODE>(p);
      ld.step = BK * Ntot * 2;
      ks_offsets(h, Ntot * 2, ld.vo);
    }
  }
  return ld;
}

__device__ __forceinline__ void zero_acc(f32x4 (&acc)[8][8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // initialisation -> first MFMA: pin the zeroed registers ahead of the wait states
#pragma unroll
  for (int i = 0; i < 8; ++i) pin_acc_row(acc[i]);
  asm volatile("s_nop 7" ::: "memory");
}

// Persistent: the host launches at most one workgroup per compute unit, and each workgroup runs
// a list of tiles.  Schedule: every workgroup counts the tiles from `offsets` once.  Balanced
// launches give XCD x (block ids b with b % 8 == x) the contiguous run of tiles
// [x * per, (x + 1) * per), per = ceil(tiles / 8), which its workgroups take in strides of the
// number of workgroups on the XCD, so the tiles that run at once on one XCD share operand rows in
// its L2.  Weight gradients whose largest expert holds more than twice the mean rows deal tiles
// round-robin over all workgroups instead (snake order: odd rounds run the workgroups backwards),
// so the hot experts' (long) tiles spread over the chip and do not pile up on the same ones.
// The K steps of a workgroup's tiles form one stream through the LDS rings: the DMA of the next
// tile's first two steps is issued during the current tile's last two, so it lands while the
// current tile's epilogue runs.  Each tile runs at least two K steps (zero-filled past its data),
// so the step two ahead always belongs to the current or the next tile.
template <int MODE>
__global__ __launch_bounds__(NTH, 1) void grouped_gemm_kernel(Params p) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // ---- device-side schedule
  const int NTW = n_tile_width<MODE>();
  const int ntiles_n = (n_total<MODE>(p) + NTW - 1) / NTW;
  MTiles mts{};
  ExpertSet nz{};
  int total;
  bool deal = false;
  if constexpr (!Traits<MODE>::WGRAD) {
    mts = gsched::mtile_scan<BM>(p.offsets, p.E);
    total = mts.total * ntiles_n;
  } else {
    const int mt = (m_total_wgrad<MODE>(p) + BM - 1) / BM;
    nz = expert_set(p.offsets, p.E, false);
    total = nz.total * mt * (MODE == WGRAD_GU ? 2 : 1) * ntiles_n;
    deal = gsched::wgrad_skewed(p.offsets, p.E, p.n);
  }
  const int cm = deal && !p.cell_deal ? 1 : p.cm;
  const int cn = deal && !p.cell_deal ? 1 << 20 : p.cn;
  const int G = gridDim.x;     // a multiple of 8
  const int bid = blockIdx.x;
  int lid, lstep, lend;
  if (deal) {
    lid = bid;
    lstep = G;
    lend = total;
  } else {
    const int per = (total + 7) >> 3;
    const int x = bid & 7;
    lid = x * per + (bid >> 3);
    lstep = G >> 3;
    lend = (x + 1) * per < total ? (x + 1) * per : total;
  }
  lid = __builtin_amdgcn_readfirstlane(lid);
  lstep = __builtin_amdgcn_readfirstlane(lstep);
  lend = __builtin_amdgcn_readfirstlane(lend);

  // Weight gradients of experts without rows are zero.  Their tiles stay out of the K-step
  // stream (which runs at least two steps per tile): before its own tiles each workgroup writes
  // its round-robin share of them with the epilogue on zeroed accumulators, staged in the first
  // operand stage (the epilogue synchronises only within a wave; a barrier then hands the LDS to
  // the stream).
  if constexpr (Traits<MODE>::WGRAD) {
    f32x4 acc[8][8];
    const uint32_t stg = lds_addr(lds_ring) + B_RING + wave * STG_BYTES;
    const int Mtot = m_total_wgrad<MODE>(p);
    const int mt = (Mtot + BM - 1) / BM;
    const int per_e = mt * (MODE == WGRAD_GU ? 2 : 1) * ntiles_n;
    const ExpertSet ez = expert_set(p.offsets, p.E, true);
    const int total_z = ez.total * per_e;
    for (int z = bid; z < total_z; z += G) {
      const int j = z / per_e;
      const int rem = z - j * per_e;
      const int mi = rem / ntiles_n;
      Tile tz;
      tz.e = expert_set_nth(ez, j);
      tz.half = mi >= mt ? 1 : 0;
      tz.m0 = (mi - tz.half * mt) * BM;
      tz.m_end = Mtot;
      tz.n0 = (rem - mi * ntiles_n) * BN;
      tz.k_begin = 0;
      tz.k_len = 0;
      zero_acc(acc);
      epilogue<MODE>(p, tz, acc, wm, wn, lane, stg);
    }
    // the stores done (the prologue's vmcnt waits count only its own DMA) and every wave's
    // staging reads done before the stream writes that stage
    if (total_z > 0) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  if (lid >= lend) return;

  const bool role_b = wave < 2;
  const int h = wave & 1;
  const OpLoad ld = op_load<MODE>(p, role_b, h);
  Tile t = tile_at<MODE>(p, mts, nz, ntiles_n, cm, cn, lid);
  TileSrc cur = tile_src<MODE>(p, t, role_b, h);
  // round-robin deal in snake order: round r gives workgroup b tile r G + b (r even) or
  // r G + G - 1 - b (r odd), so the workgroups holding the first (hottest, lowest-id) experts'
  // tiles take the lightest of the next round's
  int rn = 1;
  auto deal_lid = [&](int r) { return r * G + ((r & 1) ? (G - 1 - bid) : bid); };
  int lid_n = deal ? deal_lid(1) : lid + lstep;
  Tile tn = t;
  TileSrc nxt = empty_src(p);
  if (lid_n < lend) {
    tn = tile_at<MODE>(p, mts, nz, ntiles_n, cm, cn, lid_n);
    nxt = tile_src<MODE>(p, tn, role_b, h);
  }

  f32x4 acc[8][8];
  zero_acc(acc);
  // ---- prologue: steps 0 and 1 in flight, then step 0 everywhere
  issue_stage<MODE>(p, ld, cur, role_b, h, 0, 0);
  issue_stage<MODE>(p, ld, cur, role_b, h, 1, 1);
  asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
  const FragAddr fa = frag_addr();
  const uint32_t a0 = lds_addr(lds_ring) + A_RING, b0 = lds_addr(lds_ring) + B_RING;
  const int qa = 8 * wm, qb = bfrag_base<MODE>(wn);
  bf16x8 fa0[8], fa1[8], fb[4];
  static_for<0, 8>([&](auto j) { read_frag<Traits<MODE>::A_KC, 0, j>(fa0[j], a0, fa, qa); });
  read_frag<Traits<MODE>::B_KC, 0, bfrag_c<MODE, 0>()>(fb[0], b0, fa, qb);
  read_frag<Traits<MODE>::B_KC, 0, bfrag_c<MODE, 1>()>(fb[1], b0, fa, qb);
  int sa = 0, sb = 0, kt = 0;
  for (;;) {
    sub_step<MODE, 0>(p, ld, role_b, h, fa, cur, 0, sa, sb, fa0, fa1, fb, acc);
    {
      const bool here = kt + 2 < cur.nk;
      TileSrc is;
      is.r0 = here ? cur.r0 : nxt.r0;
      is.r1 = here ? cur.r1 : nxt.r1;
      is.nreal = here ? cur.nreal : nxt.nreal;
      is.nk = 0;
      sub_step<MODE, 1>(p, ld, role_b, h, fa, is, here ? kt + 2 : kt + 2 - cur.nk, sa, sb, fa1, fa0, fb, acc);
    }
    sa = sa + 1 == NA ? 0 : sa + 1;
    sb = sb + 1 == NB ? 0 : sb + 1;
    if (++kt < cur.nk) continue;
    // ---- tile done.  The next tile's first fragments (fa0, fb[0], fb[1]) are complete before
    // the epilogue, and the last MFMA results settle before its VALU reads them.
    lgkm_wait_all<0>(fb, fa0);
    asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
    // every wave is done with the N-side stage of the last step: it stages the epilogue
    asm volatile("s_barrier" ::: "memory");
    const uint32_t stg = lds_addr(lds_ring) + B_RING + (sb == 0 ? NB - 1 : sb - 1) * OP_BYTES + wave * STG_BYTES;
    epilogue<MODE>(p, t, acc, wm, wn, lane, stg);
    if (lid_n >= lend) break;
    zero_acc(acc);
    t = tn;
    cur = nxt;
    kt = 0;
    lid_n = deal ? deal_lid(++rn) : lid_n + lstep;
    if (lid_n < lend) {
      tn = tile_at<MODE>(p, mts, nz, ntiles_n, cm, cn, lid_n);
      nxt = tile_src<MODE>(p, tn, role_b, h);
    } else {
      nxt = empty_src(p);
    }
  }
  // no LDS-DMA may still be writing when the workgroup ends
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
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

// Tile cells per product, measured on the bf16 workloads (balanced E 64; sweep d 4096, f 1536 at
// E 8, 32, 128; skewed zipf routing, E 128, top-8) against plain n-fastest order:
//  - down product 4 x 4: 8-10% faster at E 8 and skewed, 2-3% elsewhere;
//  - gate/up dgrad 4 x 4: 4-6% faster at E 128 and skewed, level elsewhere;
//  - down weight gradient 4 x 8: 2-3% faster at E 128 and skewed;
//  - gate/up product 8 x 2 on experts of at most 16 m-tiles: 4% faster at E 128 and 2% at E 32;
//    on the skewed workload's hot experts (64 m-tiles) every cell shape ran 2-5% slower;
//  - gate/up weight gradient 4 x 4 except under the round-robin deal: 2.5-6% faster at E 32 and
//    128; the skewed workload (dealt) ran 3% slower in cells;
//  - down dgrad: n-fastest (no shape was outside the run-to-run spread of about 1.5%).
template <int MODE>
void tile_cells(Params& p) {
  p.cm = 1;
  p.cn = 1 << 20;
  p.cell_mt = 1 << 20;
  p.cell_deal = 1;
  if (MODE == FWD1) { p.cm = 8; p.cn = 2; p.cell_mt = 16; }
  if (MODE == FWD2 || MODE == DGRAD2) { p.cm = 4; p.cn = 4; }
  if (MODE == WGRAD_DOWN) { p.cm = 4; p.cn = 8; }
  if (MODE == WGRAD_GU) { p.cm = 4; p.cn = 4; p.cell_deal = 0; }
}

template <int MODE>
int launch(const Params& p0, hipStream_t s) {
  Params p = p0;
  tile_cells<MODE>(p);
  const long long upper = grid_upper(MODE, p.E, p.n, p.d, p.f);
  MOE_REQUIRE(upper < (1LL << 31), MOE_ERR_UNSUPPORTED, "too many tiles");
  const int g = gemm_workgroups(upper);
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

int gg_bf16_dgrad_down(int E, int n, int d, int f, const int32_t* offsets, const uint16_t* dyexp,
                       const uint16_t* wd, const uint16_t* g, const uint16_t* u, uint16_t* dg, uint16_t* du,
                       hipStream_t s) {
  // dgrad through W_down with the SwiGLU backward epilogue
  gg::Params p{};
  p.offsets = offsets; p.E = E; p.n = n; p.d = d; p.f = f;
  p.a0 = dyexp; p.b0 = wd; p.g = g; p.u = u; p.o0 = dg; p.o1 = du;
  return gg::launch<gg::DGRAD1>(p, s);
}

int gg_bf16_wgrad_down(int E, int n, int d, int f, const int32_t* offsets, const uint16_t* dyexp,
                       const uint16_t* a, uint16_t* dwd, hipStream_t s) {
  gg::Params w{};
  w.offsets = offsets; w.E = E; w.n = n; w.d = d; w.f = f;
  w.a0 = dyexp; w.b0 = a; w.o0 = dwd;
  return gg::launch<gg::WGRAD_DOWN>(w, s);
}

int gg_bf16_dgrad_gate_up(int E, int n, int d, int f, const int32_t* offsets, const uint16_t* dg,
                          const uint16_t* du, const uint16_t* wg, const uint16_t* wu, uint16_t* dxp,
                          hipStream_t s) {
  gg::Params q{};
  q.offsets = offsets; q.E = E; q.n = n; q.d = d; q.f = f;
  q.a0 = dg; q.a1 = du; q.b0 = wg; q.b1 = wu; q.o0 = dxp;
  return gg::launch<gg::DGRAD2>(q, s);
}

int gg_bf16_wgrad_gate_up(int E, int n, int d, int f, const int32_t* offsets, const uint16_t* dg,
                          const uint16_t* du, const uint16_t* xp, uint16_t* dwg, uint16_t* dwu, hipStream_t s) {
  gg::Params r{};
  r.offsets = offsets; r.E = E; r.n = n; r.d = d; r.f = f;
  r.a0 = dg; r.a1 = du; r.b0 = xp; r.o0 = dwg; r.o1 = dwu;
  return gg::launch<gg::WGRAD_GU>(r, s);
}

int gg_bf16_backward(int E, int n, int d, int f, const int32_t* offsets, const uint16_t* xp, const uint16_t* g,
                     const uint16_t* u, const uint16_t* a, const uint16_t* dyexp, const uint16_t* wg,
                     const uint16_t* wu, const uint16_t* wd, uint16_t* dg, uint16_t* du, uint16_t* dxp,
                     uint16_t* dwg, uint16_t* dwu, uint16_t* dwd, hipStream_t s) {
  if (int st = gg_bf16_dgrad_down(E, n, d, f, offsets, dyexp, wd, g, u, dg, du, s)) return st;
  if (int st = gg_bf16_wgrad_down(E, n, d, f, offsets, dyexp, a, dwd, s)) return st;
  if (int st = gg_bf16_dgrad_gate_up(E, n, d, f, offsets, dg, du, wg, wu, dxp, s)) return st;
  return gg_bf16_wgrad_gate_up(E, n, d, f, offsets, dg, du, xp, dwg, dwu, s);
}

}  // namespace moe
