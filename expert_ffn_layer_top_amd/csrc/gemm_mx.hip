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
// Tile geometry and staging follow the bf16 kernels: 256 x 256 outputs per workgroup, four
// waves of 128 x 128 (256 fp32 accumulators per lane in AGPRs), K stages of 128 elements = one
// 128-byte row per operand row, XOR-swizzled 16-byte chunks, LDS-DMA buffer loads.  Waves 0-1
// stream the N-side operand and waves 2-3 the M-side one, two stages each; every K step needs the
// 4 scale bytes of each row too, loaded by the same waves as the cache lines allow (see OpLoad:
// per step, in four-step groups, or block-major for the weight gradients).  The barrier opening
// K step g sits at its start: past
// it every wave has finished step g-1, so the DMA of step g+1 goes into that step's stages while
// step g is consumed.  The MFMA lane layout (checked on the
// device): lane l holds row l % 16, K bytes 16*(l/16) .. +15 and 64 + 16*(l/16) .. +15 of the
// 128-wide step, and supplies the scale of row l % 16, K block l/16.
//
// Weight-gradient K tails: an expert's padded token range is a multiple of 32, not of 128, so a
// stage can run into the next expert's positions.  Those K blocks get scale byte 0 on both
// operands (2^-127 each): their products fall below the smallest fp32 subnormal and add exactly
// zero.
#include <type_traits>

#include "common.h"
#include "gemm_epilogue.h"
#include "mx_common.h"
#include "gemm_sched.h"

namespace moe {
namespace gmx {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 128;                           // fp8 elements (bytes) per K step
constexpr int NTH = 256;
constexpr int OP_BYTES = BM * BK;                 // 32 KiB per operand per stage
constexpr int SC_BYTES = BM * 16;                 // scales: 16 bytes per row (see OpLoad)
constexpr int NSTG = 2;                           // stages per operand ring
constexpr int A_RING = 0;
constexpr int B_RING = NSTG * OP_BYTES;
constexpr int SA_RING = 2 * NSTG * OP_BYTES;
constexpr int SB_RING = SA_RING + NSTG * SC_BYTES;
constexpr int STG_RING = SB_RING + NSTG * SC_BYTES;    // epilogue staging, 4 KiB per wave
constexpr int STG_BYTES = 4096;
constexpr int LDS_TOTAL = STG_RING + 4 * STG_BYTES;    // 160 KiB
constexpr uint32_t RSRC_WORD3 = 0x00020000u;      // raw buffer, 32-bit data format (gfx9 family)

__shared__ __attribute__((aligned(1024))) uint8_t lds_ring[LDS_TOTAL];

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_u8*)(p)));
}

enum Mode { FWD1 = 0, FWD2 = 1, DGRAD1 = 2, DGRAD2 = 3, WGRAD_DOWN = 4, WGRAD_GU = 5 };

struct Params {
  int cm, cn;                   // tile order: cells of cm m-tiles x cn n-tiles (see tile_at)
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

template <int MODE>
struct Traits {
  static constexpr bool WGRAD = (MODE >= WGRAD_DOWN);
};

// row r (128 bytes = 8 chunks), chunk c stored at chunk position c ^ ((r >> 1) & 7)
__device__ __forceinline__ int kc_swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int kc_off(int r, int c) { return r * 128 + ((c ^ kc_swz(r)) << 4); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, long long bytes) {
  const int nrec = bytes <= 0 ? 0 : (bytes >= 0x7fffffffLL ? 0x7fffffff : static_cast<int>(bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, nrec, RSRC_WORD3);
}

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

using gsched::MTiles;

// One wave's share of an operand stage: 128 rows x 128 bytes of data (16 DMA instructions of
// 16 bytes per lane) and the rows' scale bytes, one lane per row and dword (2 dword instructions,
// 4 for the weight gradients).  The offsets depend on the launch, not the tile.
//
// A K step needs 4 scale bytes per row (4 blocks of 32).
// - Forward and dgrad operands (row-major scales [rows][K/32], K a multiple of 128): the 4 bytes
//   are one aligned dword of the row; two dword loads per wave (lane = row) put row R of the
//   stage at 4 R (the dword form of the LDS-DMA load writes lane l's dword at its base + 4 l).
//   Each such load touches a separate cache line per row, as many lines as the step's data.
//   When K is a multiple of 512, scale groups replace them: every fourth K step loads the 16
//   scale bytes of four steps per row (one 16-byte load per row, into one of two group
//   buffers: row R at 16 R), a quarter of the lines.
// - Weight-gradient operands (block-major scales [P/32][C]): a step's 4 block rows of the
//   wave's 128 channels are 4 runs of 128 contiguous bytes; one 16-byte load per lane (lane l:
//   block l / 8, channels 16 (l % 8) ..) takes them and the next step's 4 (unused), stored
//   [block][128 channels] per wave half.
struct OpLoad {
  int vo[16];
  int so[2];    // scale instructions (lane offsets)
  int sstep;    // scale bytes per K step
};

// Rows row0 .. row0 + 127 of a row-major byte tensor with `ldb` bytes per row, and their scale
// dwords (`lds_` scale bytes per row, a multiple of 4): instruction i covers rows 64 i + lane.
__device__ __forceinline__ void op_offsets(int row0, int ldb, int lds_, OpLoad& ld) {
  const int L = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 8 * i + (L >> 3);
    ld.vo[i] = (row0 + r) * ldb + 16 * ((L & 7) ^ kc_swz(r));
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) ld.so[i] = (row0 + 64 * i + L) * lds_;
  ld.sstep = BK / 32;
}

// Scale group load J (rows 64 J + lane of the wave's half; the half adds 2048).
template <int J>
__device__ __forceinline__ void issue_sgrp(const OpLoad& ld, __amdgpu_buffer_rsrc_t rs, int ssoff, uint8_t* gdst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(gdst + 1024 * J), 16, ld.so[J], ssoff, 0, 0);
}

// Block-major scale load of a weight-gradient step (the wave half's slot: [8 blocks][128]).
__device__ __forceinline__ void issue_sblk(const OpLoad& ld, __amdgpu_buffer_rsrc_t rs, int ssoff, uint8_t* sdst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)sdst, 16, ld.so[0], ssoff, 0, 0);
}

// One tile's DMA sources for this wave: data and scale descriptors bounded to the tile's valid
// extent (r1, s1: the second tensor of FWD1's B half 1 and of DGRAD2's second K half).
struct TileSrc {
  __amdgpu_buffer_rsrc_t r0, r1, s0, s1;
  int nk;   // K steps
};

// Where K step k of tile `src` is read from; steps past the tile read zeros.
struct StepSrc {
  __amdgpu_buffer_rsrc_t r, rs;
  int soff, ssoff;
};

template <int MODE>
__device__ __forceinline__ StepSrc step_src(const Params& p, int sstep, const TileSrc& src, bool role_b, int h,
                                            int k) {
  StepSrc ss{src.r0, src.s0, k * BK, k * sstep};
  if constexpr (MODE == FWD1) {
    if (role_b && h) { ss.r = src.r1; ss.rs = src.s1; }
  } else if constexpr (MODE == DGRAD2) {
    const int kf = p.f / BK;
    if (k >= kf) { ss.r = src.r1; ss.rs = src.s1; ss.soff = (k - kf) * BK; ss.ssoff = (k - kf) * sstep; }
  }
  if (k >= src.nk) { ss.r = make_rsrc(p.a0, 0); ss.rs = ss.r; ss.soff = 0; ss.ssoff = 0; }
  return ss;
}

// DMA instructions of a stage: data pieces [D0, D0 + ND) and per-row scale dwords [S0, S0 + NS).
template <int D0, int ND, int S0, int NS>
__device__ __forceinline__ void issue_part(const OpLoad& ld, const StepSrc& ss, uint8_t* dst, uint8_t* sdst) {
#pragma unroll
  for (int i = D0; i < D0 + ND; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ss.r, (lds_void*)(dst + i * 1024), 16, ld.vo[i], ss.soff, 0, 0);
#pragma unroll
  for (int i = S0; i < S0 + NS; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ss.rs, (lds_void*)(sdst + 256 * i), 4, ld.so[i], ss.ssoff, 0, 0);
}

// acc += x * y (scaled fp8), accumulating in place in AGPRs (tied inline asm; callers cover the
// accumulator-initialisation and epilogue wait states).
__device__ __forceinline__ void mfma_acc(f32x4& c, const i32x8& x, const i32x8& y, int sx, int sy) {
  asm("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
      : "+a"(c)
      : "v"(x), "v"(y), "v"(sx), "v"(sy));
}

__device__ __forceinline__ void pin_acc_row(f32x4 (&r)[8]) {
  asm volatile("" : "+a"(r[0]), "+a"(r[1]), "+a"(r[2]), "+a"(r[3]), "+a"(r[4]), "+a"(r[5]), "+a"(r[6]),
               "+a"(r[7]));
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

// Fragment q (16 rows) of a stage: lane l reads row 16q + l % 16, chunks l/16 and 4 + l/16, and
// the scale byte of that row and K block l/16 (`sq`: the lane's scale byte in fragment 0).
template <int OFF>
__device__ __forceinline__ void ds_b128(i32x4& v, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void ds_u8(int& v, uint32_t addr) {
  asm volatile("ds_read_u8 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
}

// SST: bytes of scale slots per 16 rows (64 for dword slots, 256 for scale groups, 16 for the
// block-major weight-gradient slots); `sq`: this lane's scale byte in fragment 0 of its operand
// (the fragment offset qoff included).
template <int Q, int SST>
__device__ __forceinline__ void read_frag(i32x8& v, int& sw, uint32_t base, uint32_t sbase, uint32_t kc0,
                                          uint32_t kc1, uint32_t sq, int qoff) {
  i32x4 lo, hi;
  ds_b128<2048 * Q>(lo, base + kc0 + 2048 * qoff);
  ds_b128<2048 * Q>(hi, base + kc1 + 2048 * qoff);
  ds_u8<SST * Q>(sw, sbase + sq);
  v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int N>
__device__ __forceinline__ void lgkm_wait(i32x8& b, int& sb, i32x8 (&a)[8], int (&sa)[8]) {
  asm volatile("s_waitcnt lgkmcnt(%18)"
               : "+v"(b), "+v"(sb), "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]),
                 "+v"(a[6]), "+v"(a[7]), "+v"(sa[0]), "+v"(sa[1]), "+v"(sa[2]), "+v"(sa[3]), "+v"(sa[4]),
                 "+v"(sa[5]), "+v"(sa[6]), "+v"(sa[7])
               : "n"(N));
}

template <int MODE, int I>
__device__ __forceinline__ constexpr int bfrag_c() {
  if constexpr (MODE == FWD1) return (I < 4) ? I : 8 + (I - 4);
  return I;
}
template <int MODE>
__device__ __forceinline__ int bfrag_base(int wn) {
  return MODE == FWD1 ? 4 * wn : 8 * wn;
}

// The tile with linear id `lid` (< the launch's tile count).  Each expert owns a contiguous run
// of ids (experts in order); inside it, tiles follow cell_order with the launch's cell shape, so
// the tiles running at once on one XCD (consecutive ids) share their operand slices in its L2.
template <int MODE>
__device__ __forceinline__ Tile tile_at(const Params& p, const MTiles& mts, int ntiles_n, int lid) {
  Tile t;
  if constexpr (!Traits<MODE>::WGRAD) {
    const int mt_glob = lid / ntiles_n;
    int e, first;
    gsched::mtile_find(mts, mt_glob, e, first);
    e = __builtin_amdgcn_readfirstlane(e);
    first = __builtin_amdgcn_readfirstlane(first);
    const int mt_e = (p.offsets[e + 1] - p.offsets[e] + BM - 1) / BM;
    int mi, nt;
    gsched::cell_order(lid - first * ntiles_n, mt_e, ntiles_n, p.cm, p.cn, mi, nt);
    t.e = e;
    t.m0 = p.offsets[e] + mi * BM;
    t.m_end = p.offsets[e + 1];
    t.n0 = nt * n_tile_width<MODE>();
    t.half = 0;
    t.k_begin = 0;
    t.k_len = k_total<MODE>(p);
  } else {
    const int Mtot = (MODE == WGRAD_DOWN) ? p.d : p.f;
    const int mt = (Mtot + BM - 1) / BM;
    const int per_e = mt * (MODE == WGRAD_GU ? 2 : 1) * ntiles_n;
    t.e = lid / per_e;
    const int rem = lid - t.e * per_e;
    int mi, nt;
    gsched::cell_order(rem, mt * (MODE == WGRAD_GU ? 2 : 1), ntiles_n, p.cm, p.cn, mi, nt);
    t.half = mi >= mt ? 1 : 0;
    t.m0 = (mi - t.half * mt) * BM;
    t.m_end = Mtot;
    t.n0 = nt * BN;
    t.k_begin = p.offsets_pad[t.e];
    t.k_len = p.offsets_pad[t.e + 1] - t.k_begin;
  }
  // the tile is uniform; without this the descriptors built from it would look divergent
  t.e = __builtin_amdgcn_readfirstlane(t.e);
  t.m0 = __builtin_amdgcn_readfirstlane(t.m0);
  t.m_end = __builtin_amdgcn_readfirstlane(t.m_end);
  t.n0 = __builtin_amdgcn_readfirstlane(t.n0);
  t.half = __builtin_amdgcn_readfirstlane(t.half);
  t.k_begin = __builtin_amdgcn_readfirstlane(t.k_begin);
  t.k_len = __builtin_amdgcn_readfirstlane(t.k_len);
  return t;
}

__device__ __forceinline__ TileSrc empty_src(const Params& p) {
  TileSrc s;
  s.r0 = make_rsrc(p.a0, 0);
  s.r1 = s.r0;
  s.s0 = s.r0;
  s.s1 = s.r0;
  s.nk = 0;
  return s;
}

// This wave's DMA sources for tile t (waves 0, 1 -> B; 2, 3 -> A), bounded to its valid extent.
template <int MODE>
__device__ __forceinline__ TileSrc tile_src(const Params& p, const Tile& t, bool role_b) {
  TileSrc s;
  s.nk = (t.k_len + BK - 1) / BK;
  if (!role_b) {
    if constexpr (!Traits<MODE>::WGRAD) {
      const int K = (MODE == DGRAD2) ? p.f : k_total<MODE>(p);
      const int G = mx_gemm_group(K);
      const long long rem_rows = static_cast<long long>(p.n) - t.m0;
      const long long sbeg = static_cast<long long>(t.m0) * G, send = static_cast<long long>(p.n) * (K / 32);
      s.r0 = make_rsrc(p.a0 + static_cast<long long>(t.m0) * K, rem_rows * K);
      s.s0 = make_rsrc(p.a0s + sbeg, send - sbeg);
      s.r1 = s.r0;
      s.s1 = s.s0;
      if constexpr (MODE == DGRAD2) {
        s.r1 = make_rsrc(p.a1 + static_cast<long long>(t.m0) * K, rem_rows * K);
        s.s1 = make_rsrc(p.a1s + sbeg, send - sbeg);
      }
    } else {
      // [Mtot][P]: rows m0 .., columns from the expert's first padded position
      const int Mtot = (MODE == WGRAD_DOWN) ? p.d : p.f;
      const uint8_t* base = (MODE == WGRAD_GU && t.half) ? p.a1 : p.a0;
      const uint8_t* sbase = (MODE == WGRAD_GU && t.half) ? p.a1s : p.a0s;
      const long long rem_rows = static_cast<long long>(Mtot) - t.m0;
      s.r0 = make_rsrc(base + static_cast<long long>(t.m0) * p.P + t.k_begin, rem_rows * p.P - t.k_begin);
      // block-major scales [P/32][Mtot]: block rows from the expert's first, channels from m0
      const long long sb0 = static_cast<long long>(t.k_begin / 32) * Mtot + t.m0;
      s.s0 = make_rsrc(sbase + sb0, static_cast<long long>(p.P / 32) * Mtot - sb0);
      s.r1 = s.r0;
      s.s1 = s.s0;
    }
  } else {
    if constexpr (MODE == FWD1) {
      const long long eoff = static_cast<long long>(t.e) * p.f * p.d;
      const long long esoff = static_cast<long long>(t.e) * p.f * (p.d / 32);
      const long long rows = p.f - t.n0;
      const int G = mx_gemm_group(p.d);
      const long long sbeg = static_cast<long long>(t.n0) * G, send = static_cast<long long>(p.f) * (p.d / 32);
      s.r0 = make_rsrc(p.b0 + eoff + static_cast<long long>(t.n0) * p.d, rows * p.d);
      s.r1 = make_rsrc(p.b1 + eoff + static_cast<long long>(t.n0) * p.d, rows * p.d);
      s.s0 = make_rsrc(p.b0s + esoff + sbeg, send - sbeg);
      s.s1 = make_rsrc(p.b1s + esoff + sbeg, send - sbeg);
    } else if constexpr (!Traits<MODE>::WGRAD) {
      // weights [E][Ntot][K'] quantised along K' (K' = K, or f per half for DGRAD2)
      const int Ntot = n_total<MODE>(p);
      const int K = (MODE == DGRAD2) ? p.f : k_total<MODE>(p);
      const long long eoff = static_cast<long long>(t.e) * Ntot * K;
      const long long esoff = static_cast<long long>(t.e) * Ntot * (K / 32);
      const long long rows = Ntot - t.n0;
      const int G = mx_gemm_group(K);
      const long long sbeg = static_cast<long long>(t.n0) * G, send = static_cast<long long>(Ntot) * (K / 32);
      s.r0 = make_rsrc(p.b0 + eoff + static_cast<long long>(t.n0) * K, rows * K);
      s.s0 = make_rsrc(p.b0s + esoff + sbeg, send - sbeg);
      s.r1 = s.r0;
      s.s1 = s.s0;
      if constexpr (MODE == DGRAD2) {
        s.r1 = make_rsrc(p.b1 + eoff + static_cast<long long>(t.n0) * K, rows * K);
        s.s1 = make_rsrc(p.b1s + esoff + sbeg, send - sbeg);
      }
    } else {
      const int Ntot = n_total<MODE>(p);
      const long long rem_rows = static_cast<long long>(Ntot) - t.n0;
      s.r0 = make_rsrc(p.b0 + static_cast<long long>(t.n0) * p.P + t.k_begin, rem_rows * p.P - t.k_begin);
      const long long sb0 = static_cast<long long>(t.k_begin / 32) * Ntot + t.n0;
      s.s0 = make_rsrc(p.b0s + sb0, static_cast<long long>(p.P / 32) * Ntot - sb0);
      s.r1 = s.r0;
      s.s1 = s.s0;
    }
  }
  return s;
}

template <int MODE>
__device__ __forceinline__ OpLoad op_load(const Params& p, bool role_b, int h) {
  OpLoad ld;
  if constexpr (Traits<MODE>::WGRAD) {
    op_offsets(128 * h, p.P, p.P / 32, ld);
    // block-major scales of a [C][P] operand: lane l reads block l / 8, channels 16 (l % 8) ..
    const int C = role_b ? n_total<MODE>(p) : (MODE == WGRAD_DOWN ? p.d : p.f);
    const int L = threadIdx.x & 63;
    ld.so[0] = (L >> 3) * C + 128 * h + 16 * (L & 7);
    ld.sstep = (BK / 32) * C;
  } else {
    const int K = (MODE == DGRAD2) ? p.f : k_total<MODE>(p);
    const int G = mx_gemm_group(K);
    op_offsets(role_b && MODE == FWD1 ? 0 : 128 * h, K, G, ld);
    const int R = role_b ? (MODE == FWD1 ? p.f : n_total<MODE>(p)) : p.n;
    ld.sstep = (BK / 32) * R;
  }
  return ld;
}

// Writes the tile's results from the accumulators (helpers in gemm_epilogue.h), staged through
// this wave's 4 KiB of the staging area.
template <int MODE>
__device__ __forceinline__ void epilogue(const Params& p, const Tile& t, f32x4 (&acc)[8][8], int wm, int wn,
                                         int lane, uint32_t stg) {
  const int row0 = t.m0 + 128 * wm;
  const int rows_valid = t.m_end - row0;
  if constexpr (MODE == FWD1) {
    gep::epi_gate_up<1>(acc, p.o0, p.o1, p.o2, p.n, p.f, row0, rows_valid, t.n0 + 64 * wn, stg, lane);
  } else if constexpr (MODE == DGRAD1) {
    gep::epi_swiglu_bwd<1, true>(acc, p.g, p.u, p.o0, p.o1, p.n, p.f, row0, rows_valid, t.n0 + 128 * wn, stg, lane);
  } else {
    const int Ntot = n_total<MODE>(p);
    uint16_t* out = p.o0;
    long long rows = p.n;
    if constexpr (Traits<MODE>::WGRAD) {
      const int Mtot = (MODE == WGRAD_DOWN) ? p.d : p.f;
      out = (MODE == WGRAD_GU && t.half ? p.o1 : p.o0) + static_cast<long long>(t.e) * Mtot * Ntot;
      rows = Mtot;
    }
    gep::epi_plain<1>(acc, out, rows, Ntot, row0, rows_valid, t.n0 + 128 * wn, stg, lane);
  }
}

// Persistent, as the bf16 kernels: at most one workgroup per compute unit, each running a list of
// tiles (XCD-contiguous runs, or round-robin for weight gradients with a hot expert).  The K
// steps of a workgroup's tiles form one stream through the two-stage rings: the barrier opening
// step g waits for its DMA, and the DMA of step g+1 (in this tile or the next one) then goes into
// the stages step g-1 used, spread over the first MFMA rows so the wave keeps issuing MFMAs.
template <int MODE, bool SGRP>
__global__ __launch_bounds__(NTH, 1) void mx_grouped_gemm_kernel(Params p) {
  static_assert(!(SGRP && Traits<MODE>::WGRAD), "scale groups serve the forward and dgrad products");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // ---- device-side schedule
  const int NTW = n_tile_width<MODE>();
  const int ntiles_n = (n_total<MODE>(p) + NTW - 1) / NTW;
  MTiles mts{};
  int total;
  bool deal = false;
  if constexpr (!Traits<MODE>::WGRAD) {
    mts = gsched::mtile_scan<BM>(p.offsets, p.E);
    total = mts.total * ntiles_n;
  } else {
    const int Mtot = (MODE == WGRAD_DOWN) ? p.d : p.f;
    total = p.E * ((Mtot + BM - 1) / BM) * (MODE == WGRAD_GU ? 2 : 1) * ntiles_n;
    deal = gsched::wgrad_skewed(p.offsets, p.E, p.n);
  }
  const int G = gridDim.x;   // a multiple of 8
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
  if (lid >= lend) return;

  const bool role_b = wave < 2;
  const int h = wave & 1;
  const OpLoad ld = op_load<MODE>(p, role_b, h);
  constexpr bool WG = Traits<MODE>::WGRAD;
  constexpr int NSC = (SGRP || WG) ? 0 : 2;   // per-step, per-row scale dword instructions
  constexpr int SST = SGRP ? 256 : (WG ? 16 : 64);
  Tile t = tile_at<MODE>(p, mts, ntiles_n, lid);
  TileSrc cur = tile_src<MODE>(p, t, role_b);
  // round-robin deal in snake order: round r gives workgroup b tile r G + b (r even) or
  // r G + G - 1 - b (r odd), so the workgroups holding the first (hottest, lowest-id) experts'
  // tiles take the lightest of the next round's
  int rn = 1;
  auto deal_lid = [&](int r) { return r * G + ((r & 1) ? (G - 1 - bid) : bid); };
  int lid_n = deal ? deal_lid(1) : lid + lstep;
  Tile tn = t;
  TileSrc nxt = empty_src(p);
  if (lid_n < lend) {
    tn = tile_at<MODE>(p, mts, ntiles_n, lid_n);
    nxt = tile_src<MODE>(p, tn, role_b);
  }

  const uint32_t ring = lds_addr(lds_ring);
  const uint32_t stg = ring + STG_RING + wave * STG_BYTES;
  // per-lane fragment addresses: row l % 16 of each 16-row fragment, chunks l/16 and 4 + l/16
  const uint32_t kc0 = kc_off(lane & 15, lane >> 4), kc1 = kc_off(lane & 15, 4 + (lane >> 4));
  const int qa = 8 * wm, qb = bfrag_base<MODE>(wn);
  // scale byte of (row l % 16, K block l/16) in fragment 0 of each operand (scale groups add
  // 4 (step % 4) per step; weight gradients: fragments 8.. are the second wave half's slot)
  auto sq_of = [&](int qoff) -> uint32_t {
    if constexpr (SGRP) return 16 * (lane & 15) + (lane >> 4) + 256 * qoff;
    if constexpr (WG) return (qoff >> 3) * 1024 + 128 * (lane >> 4) + (lane & 15);
    return 4 * (lane & 15) + (lane >> 4) + 64 * qoff;
  };
  const uint32_t sqa = sq_of(qa), sqb = sq_of(qb);
  uint8_t* const dst0 = lds_ring + (role_b ? B_RING : A_RING) + h * (OP_BYTES / 2);
  uint8_t* const sdst0 = lds_ring + (role_b ? SB_RING : SA_RING) + h * (SGRP ? 2048 : (WG ? 1024 : 512));
  // scale groups: ig = buffer the next group load goes to, rg = buffer of the current step's group
  int ig = 0, rg = 1;

  f32x4 acc[8][8];
  zero_acc(acc);
  // `ready`: step 0 of the current tile has been issued into stage st.  An expert without rows
  // (weight gradients) has an all-zero tile and no steps: nothing of it is streamed, and the
  // step 0 of the tile after it is issued when that tile becomes current.
  int st = 0, kt = 0;
  bool ready = false;
  for (;;) {
    if (!ready && cur.nk > 0) {
      const StepSrc s0 = step_src<MODE>(p, ld.sstep, cur, role_b, h, 0);
      issue_part<0, 16, 0, NSC>(ld, s0, dst0 + st * OP_BYTES, sdst0 + st * SC_BYTES);
      if constexpr (WG) issue_sblk(ld, s0.rs, s0.ssoff, sdst0 + st * SC_BYTES);
      if constexpr (SGRP) {
        issue_sgrp<0>(ld, s0.rs, s0.ssoff, sdst0 + ig * SC_BYTES);
        issue_sgrp<1>(ld, s0.rs, s0.ssoff, sdst0 + ig * SC_BYTES);
        ig ^= 1;
      }
      ready = true;
    }
    bool next_ready = false;
    while (kt < cur.nk) {
      // step kt in LDS everywhere; every wave is done with step kt-1, whose stages take the next
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      const bool here = kt + 1 < cur.nk;
      next_ready = !here && nxt.nk > 0;
      const StepSrc ns = here ? step_src<MODE>(p, ld.sstep, cur, role_b, h, kt + 1) : step_src<MODE>(p, ld.sstep, nxt, role_b, h, 0);
      uint8_t* const dst = dst0 + (st ^ 1) * OP_BYTES;
      uint8_t* const sdst = sdst0 + (st ^ 1) * SC_BYTES;
      const uint32_t a_base = ring + A_RING + st * OP_BYTES, b_base = ring + B_RING + st * OP_BYTES;
      if constexpr (SGRP) rg ^= (kt & 3) == 0 ? 1 : 0;
      const uint32_t sc_off = SGRP ? rg * SC_BYTES + 4 * (kt & 3) : st * SC_BYTES;
      const uint32_t sa_base = ring + SA_RING + sc_off, sb_base = ring + SB_RING + sc_off;
      // scale groups: the step issued below starts a group (steps per tile are a multiple of 4)
      const bool gnew = SGRP && (((here ? kt + 1 : 0) & 3) == 0);
      uint8_t* const gdst = sdst0 + ig * SC_BYTES;
      i32x8 fa[8], fb[2];
      int xa[8], xb[2];
      static_for<0, 8>([&](auto j) { read_frag<j, SST>(fa[j], xa[j], a_base, sa_base, kc0, kc1, sqa, qa); });
      read_frag<bfrag_c<MODE, 0>(), SST>(fb[0], xb[0], b_base, sb_base, kc0, kc1, sqb, qb);
      // K blocks past the expert's padded range (wgrad only): scale 0 on both sides -> exact zero
      int live = 0xff;
      if constexpr (Traits<MODE>::WGRAD) live = (kt * BK + 32 * (lane >> 4) < t.k_len) ? 0xff : 0;
      static_for<0, 8>([&](auto i) {
        // the next step's DMA: 4 data instructions in each of the first four rows, one scale
        // instruction in each of the first NSC (or a scale group load in each of the first two
        // when the next step starts a group)
        if constexpr (i < 4) issue_part<4 * i, 4, i, (i < NSC ? 1 : 0)>(ld, ns, dst, sdst);
        if constexpr (SGRP && i < 2) {
          if (gnew) issue_sgrp<i>(ld, ns.rs, ns.ssoff, gdst);
        }
        if constexpr (WG && i == 0) issue_sblk(ld, ns.rs, ns.ssoff, sdst);
        if constexpr (i < 7)
          read_frag<bfrag_c<MODE, i + 1>(), SST>(fb[(i + 1) & 1], xb[(i + 1) & 1], b_base, sb_base, kc0, kc1, sqb, qb);
        lgkm_wait<i < 7 ? 3 : 0>(fb[i & 1], xb[i & 1], fa, xa);
        const int sbv = xb[i & 1] & live;
        static_for<0, 8>([&](auto j) { mfma_acc(acc[i][j], fb[i & 1], fa[j], sbv, xa[j] & live); });
      });
      if (gnew) ig ^= 1;
      st ^= 1;
      ++kt;
    }
    // ---- tile done (or empty): the last MFMA results settle before the epilogue reads them
    asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
    epilogue<MODE>(p, t, acc, wm, wn, lane, stg);
    if (lid_n >= lend) break;
    zero_acc(acc);
    ready = next_ready;
    t = tn;
    cur = nxt;
    kt = 0;
    lid_n = deal ? deal_lid(++rn) : lid_n + lstep;
    if (lid_n < lend) {
      tn = tile_at<MODE>(p, mts, ntiles_n, lid_n);
      nxt = tile_src<MODE>(p, tn, role_b);
    } else {
      nxt = empty_src(p);
    }
  }
  // no LDS-DMA may still be writing when the workgroup ends
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
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

// Tile cells per product, measured at the MXFP8 workload (2048 rows per expert, d 7168, f 2048;
// time and FETCH_SIZE per product for several shapes): cells of 8 m-tiles x 2 n-tiles for the
// gate/up product and the gate/up dgrad (fetch beyond L2 1.5-2.5x lower, 7-9% faster than
// n-fastest), 8 x 4 for the down weight gradient (7% faster, same fetch; n-fastest, 4 x 8 and
// 16 x 2 slower); n-fastest for the down dgrad, which was no faster in cells, for the down product
// (5% faster than its 2 x 16 cells, 4 x 8 slower still) and for the gate/up weight gradient: its
// cells cut the fetch (16 x 2: 16 -> 8.9 GB per call) but ran 10-15% slower in the layer step.
template <int MODE>
void tile_cells(Params& p) {
  p.cm = 1;
  p.cn = 1 << 20;
  if (MODE == FWD1 || MODE == DGRAD2) { p.cm = 8; p.cn = 2; }
  if (MODE == WGRAD_DOWN) { p.cm = 8; p.cn = 4; }
}

template <int MODE>
int launch(const Params& p0, hipStream_t s) {
  Params p = p0;
  tile_cells<MODE>(p);
  const long long upper = grid_upper(MODE, p.E, p.n, p.d, p.f);
  MOE_REQUIRE(upper < (1LL << 31), MOE_ERR_UNSUPPORTED, "too many tiles");
  const int g = gemm_workgroups(upper);
  // every buffer offset the kernel forms stays below 2^31 bytes
  const long long big = static_cast<long long>(p.n) * (p.d > p.f ? p.d : p.f);
  const long long wbig = static_cast<long long>(p.d) * p.f;
  const long long pbig = static_cast<long long>(p.P) * (p.d > p.f ? p.d : p.f);
  MOE_REQUIRE(big < 0x7fffffffLL && wbig < 0x7fffffffLL && pbig < 0x7fffffffLL, MOE_ERR_UNSUPPORTED,
              "MXFP8 grouped GEMM: an operand exceeds 2 GiB");
  // scale groups when every operand row's scale bytes are a multiple of 16 (K per tensor a
  // multiple of 512: steps per tile and per DGRAD2 half then come in fours)
  const int kh = MODE == DGRAD2 ? p.f : (MODE == FWD1 || MODE == DGRAD1 ? p.d : p.f);
  if (!Traits<MODE>::WGRAD && kh % 512 == 0)
    mx_grouped_gemm_kernel<MODE, !Traits<MODE>::WGRAD><<<static_cast<unsigned>(g), NTH, 0, s>>>(p);
  else
    mx_grouped_gemm_kernel<MODE, false><<<static_cast<unsigned>(g), NTH, 0, s>>>(p);
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
int gg_mx_down_q(int E, int n, int d, int f, const int32_t* offsets, const uint8_t* aq, const uint8_t* as,
                 const uint8_t* wdq, const uint8_t* wds, uint16_t* yexp, hipStream_t s) {
  gmx::Params q{};
  q.offsets = offsets; q.E = E; q.n = n; q.d = d; q.f = f;
  q.a0 = aq; q.a0s = as; q.b0 = wdq; q.b0s = wds; q.o0 = yexp;
  return gmx::launch<gmx::FWD2>(q, s);
}

int gg_mx_down(int E, int n, int d, int f, const int32_t* offsets, const uint16_t* a, const uint8_t* wdq,
               const uint8_t* wds, uint16_t* yexp, uint8_t* ws, hipStream_t s) {
  uint8_t* aq = ws;
  uint8_t* as = ws + static_cast<size_t>(n) * f;
  if (int st = mxfp8_quantize_gemm(a, 1, n, f, aq, as, s)) return st;
  return gg_mx_down_q(E, n, d, f, offsets, aq, as, wdq, wds, yexp, s);
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

int gg_mx_dgrad_down(int E, int n, int d, int f, const int32_t* offsets, const uint8_t* dyq, const uint8_t* dys,
                     const uint8_t* wdtq, const uint8_t* wdts, const uint16_t* g, const uint16_t* u, uint16_t* dg,
                     uint16_t* du, hipStream_t s) {
  gmx::Params p{};
  p.offsets = offsets; p.E = E; p.n = n; p.d = d; p.f = f;
  p.a0 = dyq; p.a0s = dys; p.b0 = wdtq; p.b0s = wdts; p.g = g; p.u = u; p.o0 = dg; p.o1 = du;
  return gmx::launch<gmx::DGRAD1>(p, s);
}

int gg_mx_wgrad_down(int E, int n, int d, int f, const int32_t* offsets, const int32_t* offsets_pad,
                     const uint8_t* dyT, const uint8_t* dyTs, const uint8_t* aT, const uint8_t* aTs, uint16_t* dwd,
                     hipStream_t s) {
  gmx::Params w{};
  w.offsets = offsets; w.offsets_pad = offsets_pad; w.E = E; w.n = n; w.d = d; w.f = f;
  w.P = moe_mx_pad_cap(n, E);
  w.a0 = dyT; w.a0s = dyTs; w.b0 = aT; w.b0s = aTs; w.o0 = dwd;
  return gmx::launch<gmx::WGRAD_DOWN>(w, s);
}

int gg_mx_dgrad_gate_up(int E, int n, int d, int f, const int32_t* offsets, const uint8_t* dgq, const uint8_t* dgs,
                        const uint8_t* duq, const uint8_t* dus, const uint8_t* wgtq, const uint8_t* wgts,
                        const uint8_t* wutq, const uint8_t* wuts, uint16_t* dxp, hipStream_t s) {
  gmx::Params q{};
  q.offsets = offsets; q.E = E; q.n = n; q.d = d; q.f = f;
  q.a0 = dgq; q.a0s = dgs; q.a1 = duq; q.a1s = dus;
  q.b0 = wgtq; q.b0s = wgts; q.b1 = wutq; q.b1s = wuts; q.o0 = dxp;
  return gmx::launch<gmx::DGRAD2>(q, s);
}

int gg_mx_wgrad_gate_up(int E, int n, int d, int f, const int32_t* offsets, const int32_t* offsets_pad,
                        const uint8_t* dgT, const uint8_t* dgTs, const uint8_t* duT, const uint8_t* duTs,
                        const uint8_t* xT, const uint8_t* xTs, uint16_t* dwg, uint16_t* dwu, hipStream_t s) {
  gmx::Params r{};
  r.offsets = offsets; r.offsets_pad = offsets_pad; r.E = E; r.n = n; r.d = d; r.f = f;
  r.P = moe_mx_pad_cap(n, E);
  r.a0 = dgT; r.a0s = dgTs; r.a1 = duT; r.a1s = duTs;
  r.b0 = xT; r.b0s = xTs; r.o0 = dwg; r.o1 = dwu;
  return gmx::launch<gmx::WGRAD_GU>(r, s);
}

int gg_mx_backward(int E, int n, int d, int f, const int32_t* offsets, const int32_t* offsets_pad,
                   const int32_t* row_token, const uint16_t* x, const uint16_t* g, const uint16_t* u,
                   const uint16_t* a, const uint16_t* dyexp, const uint8_t* wgtq, const uint8_t* wgts,
                   const uint8_t* wutq, const uint8_t* wuts, const uint8_t* wdtq, const uint8_t* wdts, uint16_t* dg,
                   uint16_t* du, uint16_t* dxp, uint16_t* dwg, uint16_t* dwu, uint16_t* dwd, uint8_t* ws,
                   hipStream_t s) {
  const MxBwdLayout L(E, n, d, f);
  // dgrad through W_down: dYexp quantised along d
  if (int st = mxfp8_quantize_gemm(dyexp, 1, n, d, ws + L.dyq, ws + L.dys, s)) return st;
  if (int st = gg_mx_dgrad_down(E, n, d, f, offsets, ws + L.dyq, ws + L.dys, wdtq, wdts, g, u, dg, du, s)) return st;
  // wgrad of W_down: operands along grouped tokens
  if (int st = mxfp8_quantize_grouped(dyexp, nullptr, offsets, offsets_pad, E, n, d, ws + L.dyT, ws + L.dyTs, s)) return st;
  if (int st = mxfp8_quantize_grouped(a, nullptr, offsets, offsets_pad, E, n, f, ws + L.aT, ws + L.aTs, s)) return st;
  if (int st = gg_mx_wgrad_down(E, n, d, f, offsets, offsets_pad, ws + L.dyT, ws + L.dyTs, ws + L.aT, ws + L.aTs, dwd, s))
    return st;
  // dgrad through W_gate, W_up: dG, dU quantised along f
  if (int st = mxfp8_quantize_gemm(dg, 1, n, f, ws + L.dgq, ws + L.dgs, s)) return st;
  if (int st = mxfp8_quantize_gemm(du, 1, n, f, ws + L.duq, ws + L.dus, s)) return st;
  if (int st = gg_mx_dgrad_gate_up(E, n, d, f, offsets, ws + L.dgq, ws + L.dgs, ws + L.duq, ws + L.dus, wgtq, wgts,
                                   wutq, wuts, dxp, s))
    return st;
  // wgrad of W_gate, W_up
  if (int st = mxfp8_quantize_grouped(dg, nullptr, offsets, offsets_pad, E, n, f, ws + L.dgT, ws + L.dgTs, s)) return st;
  if (int st = mxfp8_quantize_grouped(du, nullptr, offsets, offsets_pad, E, n, f, ws + L.duT, ws + L.duTs, s)) return st;
  if (int st = mxfp8_quantize_grouped(x, row_token, offsets, offsets_pad, E, n, d, ws + L.xT, ws + L.xTs, s)) return st;
  return gg_mx_wgrad_gate_up(E, n, d, f, offsets, offsets_pad, ws + L.dgT, ws + L.dgTs, ws + L.duT, ws + L.duTs,
                             ws + L.xT, ws + L.xTs, dwg, dwu, s);
}

}  // namespace moe
