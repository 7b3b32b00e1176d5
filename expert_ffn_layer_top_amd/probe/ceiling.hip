// Ceiling probes: what this chip sustains on the two resources the layer's kernels are bound by,
// measured with self-written kernels so that every roofline fraction can be set beside a
// measured ceiling as well as the published peak.  Not part of the layer's ABI
// (libmoe_probe.so is a separate library used by the benchmark only).
//
//   probe_mfma_bf16   matrix cores only: each wave issues independent v_mfma_f32_16x16x32_bf16
//                     on register operands (16 accumulators in rotation, so no MFMA waits for
//                     another's result); no memory traffic in the loop.
//   probe_mfma_fp8    the same with the block-scaled v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3
//                     operands, unit scales): the MXFP8 grouped GEMMs' instruction.
//   probe_copy        HBM copy: 16 bytes per lane read and written, grid-stride over the buffer.
//   probe_read        HBM read: 16 bytes per lane read and summed; one word per block written.
//   probe_dma_stream  the grouped GEMMs' operand stream alone: one workgroup per compute unit
//                     moves 256-row A and B panels into LDS with LDS-DMA buffer loads (16 bytes
//                     per lane, 8 rows x 128 bytes per instruction), 128 bytes of every row per K
//                     step, two 64 KiB stages, one barrier per step; no MFMAs, nothing read back.
//                     Shared mode: every workgroup streams the same two panels (L2-resident after
//                     the first pass).  Fresh mode: the 32 workgroups of an XCD form a cell of 8
//                     A panels x 4 B panels, a new cell per round, drawn from buffers larger than
//                     the last-level cache (the products' tile order, on data arriving from HBM).
//   probe_kstep       the MX products' K step without scales or epilogue: the LDS-DMA stream
//                     above (cells from HBM) feeding ds_read_b128 fragments and block-scaled
//                     16x16x128 fp8 MFMAs on a 256 x 256 tile, K = 7168.  Variants: 0 four
//                     waves of 128 x 128 (the kernels' layout), 1 eight waves of 64 x 128 (two per
//                     SIMD), 2 variant 0 without the DMA after the first step, 3 variant 0 with the
//                     fragments read once (no LDS reads in the K loop).
// Each result is written so the compiler keeps the work; the host times the launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kAcc = 16;   // independent accumulators per wave

// acc += x * y accumulating in place (tied asm: the accumulator stays in one register quad;
// the builtin's untied form lets the register allocator copy accumulators every iteration).
__device__ __forceinline__ void mfma_bf16(f32x4& c, const bf16x8& x, const bf16x8& y) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(x), "v"(y));
}
__device__ __forceinline__ void mfma_fp8(f32x4& c, const i32x8& x, const i32x8& y, int s) {
  asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]"
               : "+a"(c) : "v"(x), "v"(y), "v"(s));
}

// Orders every accumulator's current value against the volatile asm around it (the wait states
// between accumulator writes and the MFMAs, and between the MFMAs and the reads).
__device__ __forceinline__ void pin(f32x4 (&acc)[kAcc]) {
#pragma unroll
  for (int j = 0; j < kAcc; ++j) asm volatile("" : "+a"(acc[j]));
}

__global__ __launch_bounds__(256) void mfma_bf16_loop(int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(1.0f / (1 + ((lane + i) & 7)));
    b[i] = static_cast<__bf16>(1.0f / (2 + ((lane * 3 + i) & 7)));
  }
  f32x4 acc[kAcc];
#pragma unroll
  for (int j = 0; j < kAcc; ++j) acc[j] = f32x4{1.f * j, 0.f, 0.f, 0.f};   // distinct: no two chains merge
  pin(acc);
  asm volatile("s_nop 7" ::: "memory");          // accumulator writes -> first MFMA
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kAcc; ++j) mfma_bf16(acc[j], a, b);
  }
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");  // last MFMA -> reads of the accumulators
  pin(acc);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kAcc; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void mfma_fp8_loop(int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  i32x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // E4M3 codes of small positive values (0x30 .. 0x37: 0.5 .. 0.9375)
    const int ca = 0x30 + ((lane + i) & 7), cb = 0x30 + ((lane * 5 + i) & 7);
    a[i] = ca * 0x01010101;
    b[i] = cb * 0x01010101;
  }
  f32x4 acc[kAcc];
#pragma unroll
  for (int j = 0; j < kAcc; ++j) acc[j] = f32x4{1.f * j, 0.f, 0.f, 0.f};   // distinct: no two chains merge
  const int unit = 127;                          // E8M0 scale 2^0
  pin(acc);
  asm volatile("s_nop 7" ::: "memory");
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kAcc; ++j) mfma_fp8(acc[j], a, b, unit);
  }
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
  pin(acc);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kAcc; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

typedef __attribute__((address_space(3))) void lds_void;
constexpr int kStage = 65536;    // one K step of both panels: 2 x 256 rows x 128 bytes

__global__ __launch_bounds__(256, 1) void dma_stream_kernel(const uint8_t* __restrict__ a, const uint8_t* __restrict__ b,
                                                            int kbytes, int rounds, int npanels, int shared) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[2 * kStage];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int row = 128 * (wave & 1) + (lane >> 3);          // first row of this lane, 8 rows per load
  const int voff = row * kbytes + 16 * (lane & 7);
  const int steps = kbytes / 128;
  int g = 0;
  for (int r = 0; r < rounds; ++r) {
    const int pa = shared ? 0 : ((xcd * rounds + r) * 8 + (j & 7)) % npanels;
    const int pb = shared ? 0 : ((xcd * rounds + r) * 4 + (j >> 3)) % npanels;
    const uint8_t* base = wave < 2 ? b + static_cast<long long>(pb) * 256 * kbytes
                                   : a + static_cast<long long>(pa) * 256 * kbytes;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, 256 * kbytes, 0x00020000);
    for (int k = 0; k < steps; ++k, ++g) {
      uint8_t* dst = ring + kStage * (g & 1) + 16384 * wave;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + 1024 * i), 16, voff + 8 * i * kbytes, 128 * k, 0, 0);
      asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");   // the previous step has landed
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

template <int B, int E, class F>
__device__ __forceinline__ void sfor(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    sfor<B + 1, E>(f);
  }
}

// ---- probe_kstep.  Stage layout as in the MX products: 256 A rows then 256 B rows of 128 bytes,
// each row's eight 16-byte chunks XOR-swizzled by (row / 2) % 8.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

template <int OFF>
__device__ __forceinline__ void ds_b128(i32x4& v, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
}
// fragment q of an operand stage: lane l reads row 16 q + l % 16, chunks l / 16 and 4 + l / 16
template <int Q>
__device__ __forceinline__ void frag(i32x8& v, uint32_t base, uint32_t kc0, uint32_t kc1) {
  i32x4 lo, hi;
  ds_b128<2048 * Q>(lo, base + kc0);
  ds_b128<2048 * Q>(hi, base + kc1);
  v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void mfma(f32x4& c, const i32x8& x, const i32x8& y, int s) {
  asm("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]" : "+a"(c) : "v"(x), "v"(y), "v"(s));
}
template <int N, int NA>
__device__ __forceinline__ void wait_lgkm(i32x8& b, i32x8 (&a)[NA]) {
  if constexpr (NA == 8)
    asm volatile("s_waitcnt lgkmcnt(%9)" : "+v"(b), "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]),
                 "+v"(a[5]), "+v"(a[6]), "+v"(a[7]) : "n"(N));
  else
    asm volatile("s_waitcnt lgkmcnt(%5)" : "+v"(b), "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]) : "n"(N));
}

// NW waves, each with NAF A fragments (16 NAF rows) and NBF B fragments (16 NBF columns) of the
// 256 x 256 tile; ABL 1 drops the DMA after the first step, ABL 2 the fragment reads in the K loop.
template <int NW, int NAF, int NBF, int ABL = 0>
__global__ __launch_bounds__(NW * 64, 1) void kstep_kernel(const uint8_t* __restrict__ a, const uint8_t* __restrict__ b,
                                                           int kbytes, int rounds, int npanels, float* __restrict__ out) {
  constexpr int WM = 256 / (16 * NAF);        // waves along M
  constexpr int PER = 64 / NW;                // DMA instructions per wave per step
  __shared__ __attribute__((aligned(1024))) uint8_t ring[2 * kStage];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave % WM, wn = wave / WM;
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  // DMA: group g of 64 (8 rows x 128 bytes each): g < 32 A rows 8 g.., else B rows 8 (g - 32)..
  int vo[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int g = wave * PER + i;
    const int row = 8 * (g & 31) + (lane >> 3);
    vo[i] = row * kbytes + 16 * ((lane & 7) ^ swz(row));
  }
  const bool is_a = wave * PER < 32;   // PER divides 32: a wave's groups are all A or all B
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ring));
  const uint32_t kc0 = (lane & 15) * 128 + (((lane >> 4) ^ swz(lane & 15)) << 4);
  const uint32_t kc1 = (lane & 15) * 128 + (((4 + (lane >> 4)) ^ swz(lane & 15)) << 4);
  const int unit = 127;
  f32x4 acc[NBF][NAF];
#pragma unroll
  for (int i = 0; i < NBF; ++i)
#pragma unroll
    for (int q = 0; q < NAF; ++q) acc[i][q] = f32x4{0.f, 0.f, 0.f, 0.f};
  asm volatile("s_nop 7" ::: "memory");
  const int steps = kbytes / 128;
  int g = 0;
  __amdgpu_buffer_rsrc_t rs;
  auto set_panel = [&](int r) {
    const int pa = ((xcd * rounds + r) * 8 + (j & 7)) % npanels;
    const int pb = ((xcd * rounds + r) * 4 + (j >> 3)) % npanels;
    const uint8_t* base = is_a ? a + static_cast<long long>(pa) * 256 * kbytes : b + static_cast<long long>(pb) * 256 * kbytes;
    rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, 256 * kbytes, 0x00020000);
  };
  auto issue = [&](auto i0, auto n, int stage, int k) {
    uint8_t* dst = ring + kStage * stage + 1024 * (wave * PER);
    sfor<decltype(i0)::value, decltype(i0)::value + decltype(n)::value>([&](auto i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + 1024 * i), 16, vo[i], 128 * k, 0, 0);
    });
  };
  // prologue: step 0
  set_panel(0);
  issue(std::integral_constant<int, 0>{}, std::integral_constant<int, PER>{}, 0, 0);
  i32x8 ga[NAF], gb[2];   // ABL 2: fragments read once, reused every step
  if constexpr (ABL == 2) {
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    const uint32_t abase = lds0 + 2048 * NAF * wm, bbase = lds0 + 32768 + 2048 * NBF * wn;
    sfor<0, NAF>([&](auto q) { frag<q>(ga[q], abase, kc0, kc1); });
    frag<0>(gb[0], bbase, kc0, kc1);
    frag<1>(gb[1], bbase, kc0, kc1);
    wait_lgkm<0>(gb[0], ga);
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(gb[1]));
  }
  for (int r = 0; r < rounds; ++r) {
    for (int k = 0; k < steps; ++k, ++g) {
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      const int st = g & 1;
      const bool last = k + 1 == steps;
      if (last && r + 1 < rounds) set_panel(r + 1);
      const int kn = last ? 0 : k + 1;
      const bool more = !(last && r + 1 == rounds);
      const uint32_t abase = lds0 + kStage * st + 2048 * NAF * wm;
      const uint32_t bbase = lds0 + kStage * st + 32768 + 2048 * NBF * wn;
      if constexpr (ABL == 2) {
        sfor<0, NBF>([&](auto i) {
          if constexpr (i < 4) {
            if (more) issue(std::integral_constant<int, i * PER / 4>{}, std::integral_constant<int, PER / 4>{}, st ^ 1, kn);
          }
          sfor<0, NAF>([&](auto q) { mfma(acc[i][q], gb[i & 1], ga[q], unit); });
        });
      } else {
        i32x8 fa[NAF], fb[2];
        sfor<0, NAF>([&](auto q) { frag<q>(fa[q], abase, kc0, kc1); });
        frag<0>(fb[0], bbase, kc0, kc1);
        sfor<0, NBF>([&](auto i) {
          if constexpr (i < 4 && ABL != 1) {
            if (more) issue(std::integral_constant<int, i * PER / 4>{}, std::integral_constant<int, PER / 4>{}, st ^ 1, kn);
          }
          if constexpr (i + 1 < NBF) frag<i + 1>(fb[(i + 1) & 1], bbase, kc0, kc1);
          wait_lgkm<(i + 1 < NBF) ? 2 : 0>(fb[i & 1], fa);
          sfor<0, NAF>([&](auto q) { mfma(acc[i][q], fb[i & 1], fa[q], unit); });
        });
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)\n\ts_nop 15\n\ts_nop 15" ::: "memory");
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NBF; ++i)
#pragma unroll
    for (int q = 0; q < NAF; ++q) s += acc[i][q][0] + acc[i][q][1] + acc[i][q][2] + acc[i][q][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}


__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                   long long n16) {
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  for (long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
    dst[i] = src[i];
}

__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ src, long long n16,
                                                   unsigned* __restrict__ out) {
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  unsigned s = 0;
  for (long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const uint4 v = src[i];
    s ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ unsigned red[256];
  red[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned t = 0;
    for (int i = 0; i < 256; ++i) t ^= red[i];
    out[blockIdx.x] = t;
  }
}

}  // namespace

// Flop per launch of the two MFMA probes: blocks * 4 waves * iters * kAcc * (16 * 16 * K * 2).
extern "C" double probe_mfma_flop(int fp8, int blocks, int iters) {
  const double per = fp8 ? 16.0 * 16 * 128 * 2 : 16.0 * 16 * 32 * 2;
  return static_cast<double>(blocks) * 4 * iters * kAcc * per;
}

// out: blocks * 256 floats.  Returns 0 or the HIP error code.
extern "C" int probe_mfma(int fp8, int blocks, int iters, float* out, void* stream) {
  if (blocks < 1 || iters < 1 || out == nullptr) return -1;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (fp8) mfma_fp8_loop<<<blocks, 256, 0, s>>>(iters, out);
  else mfma_bf16_loop<<<blocks, 256, 0, s>>>(iters, out);
  return static_cast<int>(hipGetLastError());
}

// Copies `bytes` (a multiple of 16) from src to dst, 16-byte aligned buffers.
extern "C" int probe_copy(const void* src, void* dst, long long bytes, int blocks, void* stream) {
  if (bytes % 16 || src == nullptr || dst == nullptr || blocks < 1) return -1;
  copy_kernel<<<blocks, 256, 0, reinterpret_cast<hipStream_t>(stream)>>>(static_cast<const uint4*>(src),
                                                                          static_cast<uint4*>(dst), bytes / 16);
  return static_cast<int>(hipGetLastError());
}

// Reads `bytes` (a multiple of 16) of src; out: `blocks` words.
extern "C" int probe_read(const void* src, long long bytes, unsigned* out, int blocks, void* stream) {
  if (bytes % 16 || src == nullptr || out == nullptr || blocks < 1) return -1;
  read_kernel<<<blocks, 256, 0, reinterpret_cast<hipStream_t>(stream)>>>(static_cast<const uint4*>(src),
                                                                          bytes / 16, out);
  return static_cast<int>(hipGetLastError());
}

// Bytes one probe_dma_stream launch moves into LDS.
extern "C" double probe_dma_bytes(int blocks, int kbytes, int rounds) {
  return static_cast<double>(blocks) * rounds * (kbytes / 128) * kStage;
}

// a and b: npanels panels of 256 rows x kbytes each (kbytes a multiple of 128, 256 * kbytes
// < 2^31), 16-byte aligned.  One workgroup per compute unit: `blocks` = the CU count (a multiple
// of 8, 32 per XCD for the fresh mode's cells).
extern "C" int probe_dma_stream(const void* a, const void* b, int kbytes, int npanels, int rounds, int shared,
                                int blocks, void* stream) {
  if (a == nullptr || b == nullptr || kbytes < 128 || kbytes % 128 || 256LL * kbytes >= (1LL << 31) || npanels < 1 ||
      rounds < 1 || blocks < 8 || blocks % 8)
    return -1;
  dma_stream_kernel<<<blocks, 256, 0, reinterpret_cast<hipStream_t>(stream)>>>(
      static_cast<const uint8_t*>(a), static_cast<const uint8_t*>(b), kbytes, rounds, npanels, shared);
  return static_cast<int>(hipGetLastError());
}

// Flop per probe_kstep launch.
extern "C" double probe_kstep_flop(int blocks, int kbytes, int rounds) {
  return static_cast<double>(blocks) * rounds * 256.0 * 256.0 * kbytes * 2.0;
}

// a, b as for probe_dma_stream; out: blocks * 512 floats.
extern "C" int probe_kstep(int variant, const void* a, const void* b, int kbytes, int npanels, int rounds, int blocks,
                           float* out, void* stream) {
  if (a == nullptr || b == nullptr || out == nullptr || kbytes < 128 || kbytes % 128 || 256LL * kbytes >= (1LL << 31) ||
      npanels < 1 || rounds < 1 || blocks < 8 || blocks % 8)
    return -1;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const uint8_t* A = static_cast<const uint8_t*>(a);
  const uint8_t* B = static_cast<const uint8_t*>(b);
  if (variant == 0) kstep_kernel<4, 8, 8><<<blocks, 256, 0, s>>>(A, B, kbytes, rounds, npanels, out);
  else if (variant == 1) kstep_kernel<8, 4, 8><<<blocks, 512, 0, s>>>(A, B, kbytes, rounds, npanels, out);
  else if (variant == 2) kstep_kernel<4, 8, 8, 1><<<blocks, 256, 0, s>>>(A, B, kbytes, rounds, npanels, out);
  else if (variant == 3) kstep_kernel<4, 8, 8, 2><<<blocks, 256, 0, s>>>(A, B, kbytes, rounds, npanels, out);
  else return -1;
  return static_cast<int>(hipGetLastError());
}
