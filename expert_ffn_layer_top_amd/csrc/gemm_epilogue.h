// Epilogue helpers shared by the bf16 and MXFP8 grouped GEMMs: writing a wave's 128-row block of
// fp32 accumulators (MFMA layout) to a row-major bf16 output through LDS, and reading row-major
// bf16 inputs into the MFMA layout the same way.
//
// The MFMA layout gives each lane 4 consecutive columns (8 bytes) of one row per 16 x 16 tile, so
// a store straight from it writes 32-byte pieces of 16 rows per instruction, which the memory
// system absorbs several times slower than whole lines.  Staged through LDS, the values go in as
// 8-byte pieces and come out as 16-byte pieces of whole rows; every store then covers full
// 128-byte lines.  16-byte chunks are XOR-swizzled by row so both access patterns spread over the
// LDS banks.  All global accesses go through buffer descriptors: an element a lane must not touch
// (a row past the expert's or the matrix's end, a column past the matrix) gets a byte offset past
// any buffer, so the hardware drops the store and a load there reads zero; no lane-dependent
// branches, so the compiler schedules the epilogue as straight-line code.
#pragma once

#include <type_traits>

#include "common.h"

namespace moe {
namespace gep {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t OOB = 0x80000000u;
constexpr uint32_t RSRC_WORD3 = 0x00020000u;   // raw buffer, 32-bit data format (gfx9 family)

template <int B, int E, class F>
__device__ __forceinline__ void sfor(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    sfor<B + 1, E>(f);
  }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, long long bytes) {
  const int nrec = bytes <= 0 ? 0 : (bytes >= 0x7fffffffLL ? 0x7fffffff : static_cast<int>(bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, nrec, RSRC_WORD3);
}

// Descriptor over a row-major [rows][ld] bf16 tensor from element (row0, col0) to its end.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(const uint16_t* base, long long rows, int ld, int row0,
                                                         int col0) {
  const long long start = static_cast<long long>(row0) * ld + col0;
  return rsrc(base + start, (rows * ld - start) * 2);
}

// Keeps column J of the accumulators (acc[0..7][J]) in AGPRs up to this point: the epilogue pins
// each column just before it reads it, so the compiler copies the accumulators out a column at a
// time rather than all 256 at once.
template <int J>
__device__ __forceinline__ void pin_acc_col(f32x4 (&acc)[8][8]) {
  asm volatile("" : "+a"(acc[0][J]), "+a"(acc[1][J]), "+a"(acc[2][J]), "+a"(acc[3][J]), "+a"(acc[4][J]),
               "+a"(acc[5][J]), "+a"(acc[6][J]), "+a"(acc[7][J]));
}

__device__ __forceinline__ u32x2 pack4(const f32x4& v) { return u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])}; }

// Logistic function with the hardware reciprocal (v_rcp_f32, about 1 ulp): far below the bf16
// rounding the results get.  Saturates to 0 / 1 for large |x|.
__device__ __forceinline__ float sigmoid(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// LDS accesses as asm, like the GEMM main loops' fragment reads, so the compiler neither orders
// them against LDS traffic it cannot see nor inserts waits of its own; callers wait explicitly.
__device__ __forceinline__ void ds_w64(uint32_t addr, const u32x2& v) {
  asm volatile("ds_write_b64 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ void ds_w128(uint32_t addr, const u32x4& v) {
  asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ void ds_r64(u32x2& v, uint32_t addr) {
  asm volatile("ds_read_b64 %0, %1" : "=v"(v) : "v"(addr) : "memory");
}
__device__ __forceinline__ void ds_r128(u32x4& v, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr) : "memory");
}

// Waits for every LDS operation of the wave and ties the N registers read, so their uses cannot
// move above the wait.
template <int N>
__device__ __forceinline__ void lgkm_tie(u32x4 (&v)[N]) {
  if constexpr (N == 4) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3])::"memory");
  } else {
    static_assert(N == 8, "4 or 8 pieces");
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])::"memory");
  }
}
__device__ __forceinline__ void lgkm_tie_row(u32x2 (&v)[8]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])::"memory");
}
__device__ __forceinline__ void lgkm_tie(u32x2 (&v)[1][8]) { lgkm_tie_row(v[0]); }
__device__ __forceinline__ void lgkm_tie(u32x2 (&v)[2][8]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(v[0][0]), "+v"(v[0][1]), "+v"(v[0][2]), "+v"(v[0][3]), "+v"(v[0][4]), "+v"(v[0][5]),
                 "+v"(v[0][6]), "+v"(v[0][7]), "+v"(v[1][0]), "+v"(v[1][1]), "+v"(v[1][2]), "+v"(v[1][3]),
                 "+v"(v[1][4]), "+v"(v[1][5]), "+v"(v[1][6]), "+v"(v[1][7])::"memory");
}

// One staged round of a wave's output: rows 16 JR q .. 16 JR (q + 1) - 1 of its 128 rows by
// 16 NI columns (16 JR rows of 32 NI bytes at `stg`).  v[jj][i] holds this lane's 4 packed
// values of MFMA tile (i, JR q + jj): row 16 (JR q + jj) + lane % 16, columns 16 i + 4 (lane / 16)
// .. + 3.  `r` is based at the wave's first output element of a row-major output of pitch `ld`;
// rows at or past `rows_valid` and columns at or past `cols_valid` (relative to the wave) are
// dropped.
template <int NI, int JR>
__device__ __forceinline__ void stage_out_round(const u32x2 (&v)[JR][NI], int q, __amdgpu_buffer_rsrc_t r,
                                                int rows_valid, int cols_valid, int ld, uint32_t stg, int lane) {
  constexpr int CH = 2 * NI;            // 16-byte chunks per row
  constexpr int RB = 32 * NI;           // bytes per row
  constexpr int RPI = 64 / CH;          // rows per 16-byte read instruction
  constexpr int NR = JR * NI / 2;       // 16-byte reads (and stores) per lane
  const int rl = lane & 15, g = lane >> 4;
  const int lr = lane / CH, lc = lane % CH;
  sfor<0, JR>([&](auto jj) {
    const int row = 16 * jj + rl;
    const uint32_t rowb = stg + row * RB + ((g & 1) << 3);
    sfor<0, NI>([&](auto i) { ds_w64(rowb + ((((2 * i) | (g >> 1)) ^ (row & (CH - 1))) << 4), v[jj][i]); });
  });
  u32x4 rd[NR];
  sfor<0, NR>([&](auto k) {
    const int row = RPI * k + lr;   // row within the round
    ds_r128(rd[k], stg + row * RB + ((lc ^ (row & (CH - 1))) << 4));
  });
  lgkm_tie(rd);
  sfor<0, NR>([&](auto k) {
    const int rr = 16 * JR * q + RPI * k + lr;   // row within the wave
    const int cb = 8 * lc;                       // column within the wave
    const uint32_t off = rr < rows_valid && cb < cols_valid ? static_cast<uint32_t>((rr * ld + cb) * 2) : OOB;
    __builtin_amdgcn_raw_buffer_store_b128(rd[k], r, static_cast<int>(off), 0, 0);
  });
}

// Stores a wave's 128 x 16 NI bf16 outputs in rounds of 16 JR rows; val(i, j) gives this lane's
// packed values of MFMA tile (i, j).  Other arguments as for stage_out_round.
template <int NI, int JR, class Val>
__device__ __forceinline__ void store_staged(Val&& val, __amdgpu_buffer_rsrc_t r, int rows_valid, int cols_valid,
                                             int ld, uint32_t stg, int lane) {
  sfor<0, 8 / JR>([&](auto q) {
    u32x2 v[JR][NI];
    sfor<0, JR>([&](auto jj) {
      sfor<0, NI>([&](auto i) { v[jj][i] = val(i, std::integral_constant<int, JR * q + jj>{}); });
    });
    stage_out_round<NI, JR>(v, q, r, rows_valid, cols_valid, ld, stg, lane);
    __builtin_amdgcn_sched_barrier(0);
  });
}

// The reverse for a 128-column wave: 16 JR rows of a row-major bf16 input, held as whole-row
// pieces (`in`: 4 JR pieces of 16 bytes per lane, piece k = row 4k + lane / 16, columns
// 8 (lane % 16) .. + 7), go through LDS into the MFMA layout v[jj][i] (as stage_out_round).
template <int JR>
__device__ __forceinline__ void stage_in_round(const u32x4 (&in)[4 * JR], u32x2 (&v)[JR][8], uint32_t stg, int lane) {
  const int rl = lane & 15, g = lane >> 4;
  sfor<0, 4 * JR>([&](auto k) {
    const int row = 4 * k + g;
    ds_w128(stg + row * 256 + ((rl ^ (row & 15)) << 4), in[k]);
  });
  sfor<0, JR>([&](auto jj) {
    const int row = 16 * jj + rl;
    const uint32_t rowb = stg + row * 256 + ((g & 1) << 3);
    sfor<0, 8>([&](auto i) { ds_r64(v[jj][i], rowb + ((((2 * i) | (g >> 1)) ^ (row & 15)) << 4)); });
  });
  lgkm_tie(v);
}

// Loads 16 JR rows (round q) of a row-major [.][ld] bf16 input as whole-row pieces for
// stage_in_round; rows and columns outside the valid extent read zero.
template <int JR>
__device__ __forceinline__ void load_rows(__amdgpu_buffer_rsrc_t r, int q, int rows_valid, int cols_valid, int ld,
                                          int lane, u32x4 (&dst)[4 * JR]) {
  const int lr = lane >> 4, lc = lane & 15;
  sfor<0, 4 * JR>([&](auto k) {
    const int rr = 16 * JR * q + 4 * k + lr, cb = 8 * lc;
    const int off = rr < rows_valid && cb < cols_valid ? (rr * ld + cb) * 2 : static_cast<int>(OOB);
    dst[k] = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  });
}

// The three epilogues of the SwiGLU expert FFN products, for a wave whose outputs start at row
// row0 (rows_valid rows left in its expert / matrix) and column col0.
//   gate/up: accumulators i < 4 are G, i + 4 are U (same 64 columns); writes G, U, A = silu(G) U.
//   SwiGLU backward: accumulators are dA (128 columns); reads G, U, writes dG, dU.
//   plain: accumulators (128 columns) written as they are.
// A round moves 16 JR rows of a 128-column output: `stg` holds 4096 JR bytes for the wave.
template <int JR>
__device__ __forceinline__ void epi_gate_up(f32x4 (&acc)[8][8], uint16_t* g, uint16_t* u, uint16_t* a, long long n,
                                            int f, int row0, int rows_valid, int col0, uint32_t stg, int lane) {
  const int cv = f - col0;
  auto gval = [&](auto i, auto j) -> u32x2 {
    pin_acc_col<j>(acc);
    return pack4(acc[i][j]);
  };
  auto uval = [&](auto i, auto j) -> u32x2 {
    pin_acc_col<j>(acc);
    return pack4(acc[i + 4][j]);
  };
  auto aval = [&](auto i, auto j) -> u32x2 {
    pin_acc_col<j>(acc);
    const f32x4 gv = acc[i][j], uv = acc[i + 4][j];
    f32x4 av;
#pragma unroll
    for (int q = 0; q < 4; ++q) av[q] = gv[q] * sigmoid(gv[q]) * uv[q];
    return pack4(av);
  };
  // 64-column outputs: twice the rows per round in the same staging bytes
  store_staged<4, 2 * JR>(gval, out_rsrc(g, n, f, row0, col0), rows_valid, cv, f, stg, lane);
  store_staged<4, 2 * JR>(uval, out_rsrc(u, n, f, row0, col0), rows_valid, cv, f, stg, lane);
  store_staged<4, 2 * JR>(aval, out_rsrc(a, n, f, row0, col0), rows_valid, cv, f, stg, lane);
}

// PF: load G and U of round q + 1 while round q is processed (two register buffers), so only the
// first round waits a whole memory latency -- for kernels with the registers to spare.
template <int JR, bool PF = false>
__device__ __forceinline__ void epi_swiglu_bwd(f32x4 (&acc)[8][8], const uint16_t* g, const uint16_t* u,
                                               uint16_t* dg, uint16_t* du, long long n, int f, int row0,
                                               int rows_valid, int col0, uint32_t stg, int lane) {
  const int cv = f - col0;
  const auto rgi = out_rsrc(g, n, f, row0, col0);
  const auto rui = out_rsrc(u, n, f, row0, col0);
  const auto rdg = out_rsrc(dg, n, f, row0, col0);
  const auto rdu = out_rsrc(du, n, f, row0, col0);
  // (separate code for the two forms, so the kernels that do not prefetch keep their registers)
  [[maybe_unused]] u32x4 pgl[PF ? 2 : 1][4 * JR], pul[PF ? 2 : 1][4 * JR];
  if constexpr (PF) {
    load_rows<JR>(rgi, 0, rows_valid, cv, f, lane, pgl[0]);
    load_rows<JR>(rui, 0, rows_valid, cv, f, lane, pul[0]);
  }
  sfor<0, 8 / JR>([&](auto q) {
    u32x2 gm[JR][8], um[JR][8];
    if constexpr (PF) {
      constexpr int b = q & 1;
      if constexpr (q + 1 < 8 / JR) {
        load_rows<JR>(rgi, q + 1, rows_valid, cv, f, lane, pgl[b ^ 1]);
        load_rows<JR>(rui, q + 1, rows_valid, cv, f, lane, pul[b ^ 1]);
      }
      stage_in_round<JR>(pgl[b], gm, stg, lane);
      stage_in_round<JR>(pul[b], um, stg, lane);
    } else {
      u32x4 gl[4 * JR], ul[4 * JR];
      load_rows<JR>(rgi, q, rows_valid, cv, f, lane, gl);
      load_rows<JR>(rui, q, rows_valid, cv, f, lane, ul);
      stage_in_round<JR>(gl, gm, stg, lane);
      stage_in_round<JR>(ul, um, stg, lane);
    }
    sfor<0, JR>([&](auto jj) { pin_acc_col<JR * q + jj>(acc); });
    // dG, dU replace G, U in place (fewer live registers)
    sfor<0, JR>([&](auto jj) {
      constexpr int j = JR * q + jj;
      sfor<0, 8>([&](auto i) {
        const u32x2 g2 = gm[jj][i], u2 = um[jj][i];
        const float gv[4] = {bf16_lo(g2.x), bf16_hi(g2.x), bf16_lo(g2.y), bf16_hi(g2.y)};
        const float uv[4] = {bf16_lo(u2.x), bf16_hi(u2.x), bf16_lo(u2.y), bf16_hi(u2.y)};
        const f32x4 dav = acc[i][j];
        float dgv[4], duv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float sg = sigmoid(gv[e]);
          dgv[e] = dav[e] * uv[e] * sg * (1.0f + gv[e] * (1.0f - sg));
          duv[e] = dav[e] * gv[e] * sg;
        }
        gm[jj][i] = u32x2{pack_bf16x2(dgv[0], dgv[1]), pack_bf16x2(dgv[2], dgv[3])};
        um[jj][i] = u32x2{pack_bf16x2(duv[0], duv[1]), pack_bf16x2(duv[2], duv[3])};
      });
    });
    stage_out_round<8, JR>(gm, q, rdg, rows_valid, cv, f, stg, lane);
    stage_out_round<8, JR>(um, q, rdu, rows_valid, cv, f, stg, lane);
    __builtin_amdgcn_sched_barrier(0);
  });
}

template <int JR>
__device__ __forceinline__ void epi_plain(f32x4 (&acc)[8][8], uint16_t* out, long long rows, int ld, int row0,
                                          int rows_valid, int col0, uint32_t stg, int lane) {
  auto val = [&](auto i, auto j) -> u32x2 {
    pin_acc_col<j>(acc);
    return pack4(acc[i][j]);
  };
  store_staged<8, JR>(val, out_rsrc(out, rows, ld, row0, col0), rows_valid, ld - col0, ld, stg, lane);
}

}  // namespace gep
}  // namespace moe
