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
// stream the N-side operand and waves 2-3 the M-side one, two stages each; each stage also
// carries the 4 scale bytes of every row.  The barrier opening tile
// kt sits at the start of step kt: past it every wave has finished tile kt-1, so the DMA of tile
// kt+1 goes into its stages while tile kt is consumed.  The MFMA lane layout (checked on the
// device): lane l holds row l % 16, K bytes 16*(l/16) .. +15 and 64 + 16*(l/16) .. +15 of the
// 128-wide step, and supplies the scale of row l % 16, K block l/16.
//
// Weight-gradient K tails: an expert's padded token range is a multiple of 32, not of 128, so a
// stage can run into the next expert's positions.  Those K blocks get scale byte 0 on both
// operands (2^-127 each): their products fall below the smallest fp32 subnormal and add exactly
// zero.
#include <type_traits>

#include "common.h"

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
constexpr int SC_BYTES = BM * 4 * 4;              // scales: one dword slot per (row, K block)
constexpr int NSTG = 2;                           // stages per operand ring
constexpr int A_RING = 0;
constexpr int B_RING = NSTG * OP_BYTES;
constexpr int SA_RING = 2 * NSTG * OP_BYTES;
constexpr int SB_RING = SA_RING + NSTG * SC_BYTES;
constexpr int LDS_TOTAL = SB_RING + NSTG * SC_BYTES;   // 144 KiB
constexpr uint32_t RSRC_WORD3 = 0x00020000u;      // raw buffer, 32-bit data format (gfx9 family)

__shared__ __attribute__((aligned(1024))) uint8_t lds_ring[LDS_TOTAL];

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_u8*)(p)));
}

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

// m-tile prefix over experts from one round of loads (lane l holds experts l + 64 r).
struct MTiles {
  int tiles[4], excl[4];
  int total;
};

__device__ __forceinline__ MTiles mtile_scan(const int32_t* __restrict__ offsets, int E) {
  const int lane = threadIdx.x & 63;
  MTiles m;
  int lo[4], hi[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int ex = 64 * r + lane;
    lo[r] = ex < E ? offsets[ex] : 0;
    hi[r] = ex < E ? offsets[ex + 1] : 0;
  }
  int carry = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int tiles = (hi[r] - lo[r] + BM - 1) / BM;
    int incl = tiles;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    m.tiles[r] = tiles;
    m.excl[r] = carry + incl - tiles;
    carry += __shfl(incl, 63, 64);
  }
  m.total = __builtin_amdgcn_readfirstlane(carry);
  return m;
}

// True when some expert's row count exceeds twice the mean (n / E, rounded up).
__device__ __forceinline__ bool wgrad_skewed(const int32_t* __restrict__ offsets, int E, int n) {
  const int lane = threadIdx.x & 63;
  int cmax = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int ex = 64 * r + lane;
    const int c = ex < E ? offsets[ex + 1] - offsets[ex] : 0;
    cmax = c > cmax ? c : cmax;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const int v = __shfl_xor(cmax, o, 64);
    cmax = v > cmax ? v : cmax;
  }
  cmax = __builtin_amdgcn_readfirstlane(cmax);
  return cmax > 2 * ((n + E - 1) / E);
}

__device__ __forceinline__ void mtile_find(const MTiles& m, int mt, int& e, int& first) {
  const int lane = threadIdx.x & 63;
  e = 0;
  first = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const unsigned long long hit = __ballot(m.tiles[r] > 0 && m.excl[r] <= mt && mt < m.excl[r] + m.tiles[r]);
    if (hit) {
      const int src = __ffsll(static_cast<long long>(hit)) - 1;
      e = 64 * r + src;
      first = __shfl(m.excl[r], src, 64);
    }
  }
}

// One wave's share of an operand stage: 128 rows x 128 bytes of data (16 DMA instructions) and
// the rows' 4-byte scale words (2 dword DMA instructions).
struct OpLoad {
  __amdgpu_buffer_rsrc_t r0, r1, s0, s1;   // data / scale descriptors (r1, s1: second tensor)
  int vo[16];
  int so[8];
  int step, sstep;                         // bytes per K step (data, scales)
};

// Rows row0 .. row0 + 127 of a row-major byte tensor with `ldb` bytes per row, and their scale
// bytes (`lds_` bytes per row).  The byte form of the LDS-DMA load puts each lane's byte in a
// dword slot of its own (checked on the device), so a stage keeps one dword per (row, K block):
// 8 instructions of 16 rows x 4 blocks.  Bytes also serve the weight-gradient operands, whose
// scales start at an expert's padded position / 32 and need not be 4-byte aligned.
__device__ __forceinline__ void op_offsets(int row0, int ldb, int lds_, OpLoad& ld) {
  const int L = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 8 * i + (L >> 3);
    ld.vo[i] = (row0 + r) * ldb + 16 * ((L & 7) ^ kc_swz(r));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) ld.so[i] = (row0 + 16 * i + (L >> 2)) * lds_ + (L & 3);
}

template <int MODE>
__device__ __forceinline__ void issue_stage(const Params& p, const OpLoad& ld, bool role_b, int h, int kt, int nk,
                                            int st) {
  __amdgpu_buffer_rsrc_t r = ld.r0, rs = ld.s0;
  int soff = kt * ld.step, ssoff = kt * ld.sstep;
  if constexpr (MODE == FWD1) {
    if (role_b && h) { r = ld.r1; rs = ld.s1; }
  } else if constexpr (MODE == DGRAD2) {
    const int kf = p.f / BK;
    if (kt >= kf) { r = ld.r1; rs = ld.s1; soff = (kt - kf) * ld.step; ssoff = (kt - kf) * ld.sstep; }
  }
  if (kt >= nk) { r = make_rsrc(p.a0, 0); rs = r; soff = 0; ssoff = 0; }
  uint8_t* dst = lds_ring + (role_b ? B_RING : A_RING) + st * OP_BYTES + h * (OP_BYTES / 2);
#pragma unroll
  for (int i = 0; i < 16; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + i * 1024), 16, ld.vo[i], soff, 0, 0);
  uint8_t* sdst = lds_ring + (role_b ? SB_RING : SA_RING) + st * SC_BYTES + h * (SC_BYTES / 2);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(sdst + i * 256), 1, ld.so[i], ssoff, 0, 0);
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

// Fragment q (16 rows) of a stage: lane l reads row 16q + l % 16, chunks l/16 and 4 + l/16, and
// the scale slot of that row and K block l/16.
template <int OFF>
__device__ __forceinline__ void ds_b128(i32x4& v, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void ds_b32(int& v, uint32_t addr) {
  asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
}

template <int Q>
__device__ __forceinline__ void read_frag(i32x8& v, int& sw, uint32_t base, uint32_t sbase, uint32_t kc0,
                                          uint32_t kc1, uint32_t srow, int qoff) {
  i32x4 lo, hi;
  ds_b128<2048 * Q>(lo, base + kc0 + 2048 * qoff);
  ds_b128<2048 * Q>(hi, base + kc1 + 2048 * qoff);
  ds_b32<256 * Q>(sw, sbase + srow + 256 * qoff);
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

__device__ __forceinline__ void st4(uint16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}
__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

template <int MODE>
__global__ __launch_bounds__(NTH, 1) void mx_grouped_gemm_kernel(Params p) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // ---- device-side schedule (as in the bf16 kernels)
  const int NTW = n_tile_width<MODE>();
  const int ntiles_n = (n_total<MODE>(p) + NTW - 1) / NTW;
  const int bid = blockIdx.x;
  Tile t;
  if constexpr (!Traits<MODE>::WGRAD) {
    const MTiles mts = mtile_scan(p.offsets, p.E);
    const int total_tiles = mts.total * ntiles_n;
    const int tot8 = (total_tiles + 7) & ~7;
    if (bid >= tot8) return;
    const int lid = (bid & 7) * (tot8 >> 3) + (bid >> 3);
    if (lid >= total_tiles) return;
    const int mt_glob = lid / ntiles_n;
    const int nt = lid - mt_glob * ntiles_n;
    int e, first;
    mtile_find(mts, mt_glob, e, first);
    t.e = e;
    t.m0 = p.offsets[e] + (mt_glob - first) * BM;
    t.m_end = p.offsets[e + 1];
    t.n0 = nt * NTW;
    t.half = 0;
    t.k_begin = 0;
    t.k_len = k_total<MODE>(p);
  } else {
    const int Mtot = (MODE == WGRAD_DOWN) ? p.d : p.f;
    const int mt = (Mtot + BM - 1) / BM;
    const int mtt = mt * (MODE == WGRAD_GU ? 2 : 1);
    const int total_tiles = p.E * mtt * ntiles_n;
    const int tot8 = (total_tiles + 7) & ~7;
    if (bid >= tot8) return;
    // Weight-gradient tiles cost in proportion to their expert's rows.  With balanced experts,
    // keep each XCD on a contiguous run of tiles (experts' operand rows shared in its L2); when
    // one expert holds more than twice the mean, deal tiles round-robin over the XCDs instead
    // (block ids go to XCDs round-robin), so a hot expert's tiles run on every XCD at once.
    const int lid = wgrad_skewed(p.offsets, p.E, p.n) ? bid : (bid & 7) * (tot8 >> 3) + (bid >> 3);
    if (lid >= total_tiles) return;
    const int per_e = mtt * ntiles_n;
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
  // the tile is uniform; without this the descriptors below would look divergent
  t.e = __builtin_amdgcn_readfirstlane(t.e);
  t.m0 = __builtin_amdgcn_readfirstlane(t.m0);
  t.m_end = __builtin_amdgcn_readfirstlane(t.m_end);
  t.n0 = __builtin_amdgcn_readfirstlane(t.n0);
  t.half = __builtin_amdgcn_readfirstlane(t.half);
  t.k_begin = __builtin_amdgcn_readfirstlane(t.k_begin);
  t.k_len = __builtin_amdgcn_readfirstlane(t.k_len);
  const int nk = (t.k_len + BK - 1) / BK;

  // ---- this wave's DMA operand (waves 0, 1 -> B; 2, 3 -> A), bounded to its valid extent
  const bool role_b = wave < 2;
  const int h = wave & 1;
  OpLoad ld;
  if (!role_b) {
    if constexpr (!Traits<MODE>::WGRAD) {
      const int K = (MODE == DGRAD2) ? p.f : k_total<MODE>(p);
      const long long rem_rows = static_cast<long long>(p.n) - t.m0;
      ld.r0 = make_rsrc(p.a0 + static_cast<long long>(t.m0) * K, rem_rows * K);
      ld.s0 = make_rsrc(p.a0s + static_cast<long long>(t.m0) * (K / 32), rem_rows * (K / 32));
      ld.r1 = ld.r0;
      ld.s1 = ld.s0;
      if constexpr (MODE == DGRAD2) {
        ld.r1 = make_rsrc(p.a1 + static_cast<long long>(t.m0) * K, rem_rows * K);
        ld.s1 = make_rsrc(p.a1s + static_cast<long long>(t.m0) * (K / 32), rem_rows * (K / 32));
      }
      ld.step = BK;
      ld.sstep = BK / 32;
      op_offsets(128 * h, K, K / 32, ld);
    } else {
      // [Mtot][P]: rows m0 .., columns from the expert's first padded position
      const int Mtot = (MODE == WGRAD_DOWN) ? p.d : p.f;
      const uint8_t* base = (MODE == WGRAD_GU && t.half) ? p.a1 : p.a0;
      const uint8_t* sbase = (MODE == WGRAD_GU && t.half) ? p.a1s : p.a0s;
      const long long rem_rows = static_cast<long long>(Mtot) - t.m0;
      ld.r0 = make_rsrc(base + static_cast<long long>(t.m0) * p.P + t.k_begin, rem_rows * p.P - t.k_begin);
      ld.s0 = make_rsrc(sbase + static_cast<long long>(t.m0) * (p.P / 32) + t.k_begin / 32,
                        rem_rows * (p.P / 32) - t.k_begin / 32);
      ld.r1 = ld.r0;
      ld.s1 = ld.s0;
      ld.step = BK;
      ld.sstep = BK / 32;
      op_offsets(128 * h, p.P, p.P / 32, ld);
    }
  } else {
    if constexpr (MODE == FWD1) {
      const long long eoff = static_cast<long long>(t.e) * p.f * p.d;
      const long long esoff = static_cast<long long>(t.e) * p.f * (p.d / 32);
      const long long rows = p.f - t.n0;
      ld.r0 = make_rsrc(p.b0 + eoff + static_cast<long long>(t.n0) * p.d, rows * p.d);
      ld.r1 = make_rsrc(p.b1 + eoff + static_cast<long long>(t.n0) * p.d, rows * p.d);
      ld.s0 = make_rsrc(p.b0s + esoff + static_cast<long long>(t.n0) * (p.d / 32), rows * (p.d / 32));
      ld.s1 = make_rsrc(p.b1s + esoff + static_cast<long long>(t.n0) * (p.d / 32), rows * (p.d / 32));
      ld.step = BK;
      ld.sstep = BK / 32;
      op_offsets(0, p.d, p.d / 32, ld);
    } else if constexpr (!Traits<MODE>::WGRAD) {
      // weights [E][Ntot][K'] quantised along K' (K' = K, or f per half for DGRAD2)
      const int Ntot = n_total<MODE>(p);
      const int K = (MODE == DGRAD2) ? p.f : k_total<MODE>(p);
      const long long eoff = static_cast<long long>(t.e) * Ntot * K;
      const long long esoff = static_cast<long long>(t.e) * Ntot * (K / 32);
      const long long rows = Ntot - t.n0;
      ld.r0 = make_rsrc(p.b0 + eoff + static_cast<long long>(t.n0) * K, rows * K);
      ld.s0 = make_rsrc(p.b0s + esoff + static_cast<long long>(t.n0) * (K / 32), rows * (K / 32));
      ld.r1 = ld.r0;
      ld.s1 = ld.s0;
      if constexpr (MODE == DGRAD2) {
        ld.r1 = make_rsrc(p.b1 + eoff + static_cast<long long>(t.n0) * K, rows * K);
        ld.s1 = make_rsrc(p.b1s + esoff + static_cast<long long>(t.n0) * (K / 32), rows * (K / 32));
      }
      ld.step = BK;
      ld.sstep = BK / 32;
      op_offsets(128 * h, K, K / 32, ld);
    } else {
      const int Ntot = n_total<MODE>(p);
      const long long rem_rows = static_cast<long long>(Ntot) - t.n0;
      ld.r0 = make_rsrc(p.b0 + static_cast<long long>(t.n0) * p.P + t.k_begin, rem_rows * p.P - t.k_begin);
      ld.s0 = make_rsrc(p.b0s + static_cast<long long>(t.n0) * (p.P / 32) + t.k_begin / 32,
                        rem_rows * (p.P / 32) - t.k_begin / 32);
      ld.r1 = ld.r0;
      ld.s1 = ld.s0;
      ld.step = BK;
      ld.sstep = BK / 32;
      op_offsets(128 * h, p.P, p.P / 32, ld);
    }
  }

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (nk > 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) pin_acc_row(acc[i]);
    asm volatile("s_nop 7" ::: "memory");
    // per-lane fragment addresses: row l % 16 of each 16-row fragment, chunks l/16 and 4 + l/16
    const uint32_t kc0 = kc_off(lane & 15, lane >> 4), kc1 = kc_off(lane & 15, 4 + (lane >> 4));
    const uint32_t srow = 16 * (lane & 15) + 4 * (lane >> 4);   // dword slot (row, K block l/16)
    const int qa = 8 * wm, qb = bfrag_base<MODE>(wn);
    const uint32_t ring = lds_addr(lds_ring);
    issue_stage<MODE>(p, ld, role_b, h, 0, nk, 0);
    for (int kt = 0; kt < nk; ++kt) {
      const int st = kt & 1;
      // tile kt in LDS everywhere; every wave is done with tile kt-1, whose stages take tile kt+1
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      issue_stage<MODE>(p, ld, role_b, h, kt + 1, nk, st ^ 1);
      const uint32_t a_base = ring + A_RING + st * OP_BYTES, b_base = ring + B_RING + st * OP_BYTES;
      const uint32_t sa_base = ring + SA_RING + st * SC_BYTES, sb_base = ring + SB_RING + st * SC_BYTES;
      i32x8 fa[8], fb[2];
      int xa[8], xb[2];
      static_for<0, 8>([&](auto j) { read_frag<j>(fa[j], xa[j], a_base, sa_base, kc0, kc1, srow, qa); });
      read_frag<bfrag_c<MODE, 0>()>(fb[0], xb[0], b_base, sb_base, kc0, kc1, srow, qb);
      // K blocks past the expert's padded range (wgrad only): scale 0 on both sides -> exact zero
      int live = 0xff;
      if constexpr (Traits<MODE>::WGRAD) live = (kt * BK + 32 * (lane >> 4) < t.k_len) ? 0xff : 0;
      static_for<0, 8>([&](auto i) {
        if constexpr (i < 7) read_frag<bfrag_c<MODE, i + 1>()>(fb[(i + 1) & 1], xb[(i + 1) & 1], b_base, sb_base, kc0, kc1, srow, qb);
        lgkm_wait<i < 7 ? 3 : 0>(fb[i & 1], xb[i & 1], fa, xa);
        const int sbv = xb[i & 1] & live;
        static_for<0, 8>([&](auto j) { mfma_acc(acc[i][j], fb[i & 1], fa[j], sbv, xa[j] & live); });
      });
    }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_nop 15\n\ts_nop 15" ::: "memory");
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
  const long long g = (grid_upper(MODE, p.E, p.n, p.d, p.f) + 7) / 8 * 8;
  MOE_REQUIRE(g < (1LL << 31), MOE_ERR_UNSUPPORTED, "too many tiles");
  // every buffer offset the kernel forms stays below 2^31 bytes
  const long long big = static_cast<long long>(p.n) * (p.d > p.f ? p.d : p.f);
  const long long wbig = static_cast<long long>(p.d) * p.f;
  const long long pbig = static_cast<long long>(p.P) * (p.d > p.f ? p.d : p.f);
  MOE_REQUIRE(big < 0x7fffffffLL && wbig < 0x7fffffffLL && pbig < 0x7fffffffLL, MOE_ERR_UNSUPPORTED,
              "MXFP8 grouped GEMM: an operand exceeds 2 GiB");
  mx_grouped_gemm_kernel<MODE><<<static_cast<unsigned>(g), NTH, 0, s>>>(p);
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
  if (int st = mxfp8_quantize(dyexp, 1, n, d, 0, ws + L.dyq, ws + L.dys, s)) return st;
  if (int st = gg_mx_dgrad_down(E, n, d, f, offsets, ws + L.dyq, ws + L.dys, wdtq, wdts, g, u, dg, du, s)) return st;
  // wgrad of W_down: operands along grouped tokens
  if (int st = mxfp8_quantize_grouped(dyexp, nullptr, offsets, offsets_pad, E, n, d, ws + L.dyT, ws + L.dyTs, s)) return st;
  if (int st = mxfp8_quantize_grouped(a, nullptr, offsets, offsets_pad, E, n, f, ws + L.aT, ws + L.aTs, s)) return st;
  if (int st = gg_mx_wgrad_down(E, n, d, f, offsets, offsets_pad, ws + L.dyT, ws + L.dyTs, ws + L.aT, ws + L.aTs, dwd, s))
    return st;
  // dgrad through W_gate, W_up: dG, dU quantised along f
  if (int st = mxfp8_quantize(dg, 1, n, f, 0, ws + L.dgq, ws + L.dgs, s)) return st;
  if (int st = mxfp8_quantize(du, 1, n, f, 0, ws + L.duq, ws + L.dus, s)) return st;
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
