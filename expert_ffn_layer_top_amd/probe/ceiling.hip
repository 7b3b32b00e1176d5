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
// Each result is written so the compiler keeps the work; the host times the launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

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
