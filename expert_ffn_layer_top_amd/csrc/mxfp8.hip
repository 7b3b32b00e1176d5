// MXFP8 block quantisation of bf16 tensors ([news] "MXFP8 reduces compute and memory costs":
// 8-bit floats with a separate scale per small block of values).  Three layouts, each with one
// E8M0 scale per 32 elements along a GEMM's contraction dimension:
//   rows     blocks along the contiguous dim, output in the input's layout;
//   cols     blocks along the strided dim, output transposed (each block contiguous again);
//   grouped  token-axis blocks restarting at each expert group (padded to 32, 64 or 128 rows), output
//            transposed to [C, padded tokens]: the weight-gradient operands.  Their scales are
//            stored block-major, [padded tokens / 32, C], so the scales of one K step of the
//            weight-gradient products (4 blocks) for consecutive channels are contiguous.
// rows and cols also come together from one read of the input (the weights, which the products
// need quantised along each of their two dims).  All are HBM-bound: 2 bytes read, 1 + 1/32
// bytes written per element and output.
#include "mx_common.h"

namespace moe {
namespace {

// ---- rows: 4 lanes per 32-element block, 8 elements (16 bytes) per lane
// gemm_rows > 0: the input is [batch][gemm_rows][cols] and the scales go out in the GEMM layout
// (mx_gemm_scale_index) of each matrix; else row-major [.][cols/32].
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ in, long long total,
                                                         uint8_t* __restrict__ q, uint8_t* __restrict__ scale,
                                                         int mode, int gemm_rows, int cols) {
  const long long g = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  const long long e0 = g * 8;
  const bool live = e0 < total;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (live) v = *reinterpret_cast<const uint4*>(in + e0);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = w[i] & 0x7fffu, hi = (w[i] >> 16) & 0x7fffu;
    amax = lo > amax ? lo : amax;
    amax = hi > amax ? hi : amax;
  }
  // reduce over the 4 lanes of the block (lanes 4m..4m+3 of the wave)
  amax = max(amax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(amax), 1, 64)));
  amax = max(amax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(amax), 2, 64)));
  if (!live) return;
  const int sh = mx_shared_exp(amax, mode);
  const uint32_t o0 = mx_encode4(w[0] & 0xffffu, w[0] >> 16, w[1] & 0xffffu, w[1] >> 16, sh);
  const uint32_t o1 = mx_encode4(w[2] & 0xffffu, w[2] >> 16, w[3] & 0xffffu, w[3] >> 16, sh);
  *reinterpret_cast<uint2*>(q + e0) = make_uint2(o0, o1);
  if ((threadIdx.x & 3) == 0) {
    long long si = e0 / 32;
    if (gemm_rows > 0) {
      const long long plane = static_cast<long long>(gemm_rows) * cols;
      const long long bi = e0 / plane, rem = e0 - bi * plane;
      const long long r = rem / cols;
      si = bi * (plane / 32) + mx_gemm_scale_index(r, (rem - r * cols) / 32, gemm_rows, cols);
    }
    scale[si] = static_cast<uint8_t>(sh + 127);
  }
}

// ---- transposed layouts: a tile of 128 (strided-dim) positions x 64 columns staged in LDS.
constexpr int kTP = 128;       // positions per tile (4 blocks of 32)
constexpr int kTC = 64;        // columns per tile
constexpr int kPitch = kTC + 2;  // LDS row pitch in bf16 (33 words: column reads hit distinct banks)

// Each of the 256 threads quantises one (column, 32-position block) of the staged tile and
// writes 32 bytes of q and one scale byte.  Lanes 4c..4c+3 take the 4 blocks of column c, so
// they write 128 contiguous bytes.  The scale of (column c, block b) goes to
// scale[c * s_col + b * s_blk] (b counted from position 0; `scale` based at the tile's column 0).
// With gemm_R > 0 the scales go out in the GEMM layout instead: `scale` based at the matrix, the
// byte of column gemm_c0 + c and block b (of the strided dim's gemm_K positions) at
// mx_gemm_scale_index(gemm_c0 + c, b, gemm_R, gemm_K).
__device__ __forceinline__ void quant_tile_columns(const uint16_t (*tile)[kPitch], int ncols, long long pos0,
                                                   long long out_pitch, uint8_t* __restrict__ q,
                                                   uint8_t* __restrict__ scale, long long s_col, long long s_blk,
                                                   int mode = 0, long long gemm_R = 0, long long gemm_K = 0,
                                                   long long gemm_c0 = 0) {
  const int c = threadIdx.x >> 2;
  const int blk = threadIdx.x & 3;
  if (c >= ncols) return;
  uint32_t vals[32];
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    vals[i] = tile[blk * 32 + i][c];
    const uint32_t m = vals[i] & 0x7fffu;
    amax = m > amax ? m : amax;
  }
  const int sh = mx_shared_exp(amax, mode);
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    o[i] = mx_encode4(vals[4 * i], vals[4 * i + 1], vals[4 * i + 2], vals[4 * i + 3], sh);
  }
  uint8_t* dst = q + c * out_pitch + pos0 + blk * 32;
  reinterpret_cast<uint4*>(dst)[0] = make_uint4(o[0], o[1], o[2], o[3]);
  reinterpret_cast<uint4*>(dst)[1] = make_uint4(o[4], o[5], o[6], o[7]);
  const long long si = gemm_R > 0 ? mx_gemm_scale_index(gemm_c0 + c, pos0 / 32 + blk, gemm_R, gemm_K)
                                  : c * s_col + (pos0 / 32 + blk) * s_blk;
  scale[si] = static_cast<uint8_t>(sh + 127);
}

// in [batch][rows][cols] -> q [batch][cols][rows], scale [batch][cols][rows/32]
// grid: (ceil(rows/128), ceil(cols/64), batch); rows % 32 == 0, cols % 64 == 0.
__global__ __launch_bounds__(256) void quant_cols_kernel(const uint16_t* __restrict__ in, int rows, int cols,
                                                         uint8_t* __restrict__ q, uint8_t* __restrict__ scale,
                                                         int mode) {
  __shared__ uint16_t tile[kTP][kPitch];
  const long long b = blockIdx.z;
  const int r0 = blockIdx.x * kTP;
  const int c0 = blockIdx.y * kTC;
  const uint16_t* src = in + b * rows * static_cast<long long>(cols);
  // load 128 x 64 bf16: thread t takes column chunk t%8 of rows t/8 + 32i
  const int cc = threadIdx.x & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (threadIdx.x >> 3) + 32 * i;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r0 + r < rows) v = *reinterpret_cast<const uint4*>(src + static_cast<long long>(r0 + r) * cols + c0 + 8 * cc);
    uint32_t* t = reinterpret_cast<uint32_t*>(&tile[r][8 * cc]);
    t[0] = v.x; t[1] = v.y; t[2] = v.z; t[3] = v.w;
  }
  __syncthreads();
  // positions beyond `rows` in the last tile form whole 32-blocks (rows % 32 == 0): skip them
  const int blk = threadIdx.x & 3;
  if (r0 + blk * 32 >= rows) return;
  quant_tile_columns(tile, kTC, r0, rows, q + b * cols * static_cast<long long>(rows) + static_cast<long long>(c0) * rows,
                     scale + b * cols * static_cast<long long>(rows / 32) + static_cast<long long>(c0) * (rows / 32),
                     rows / 32, 1, mode);
}

// ---- both layouts from one read (the weights, quantised along each of their two dims every
// step): the 128 x 64 tile of the column quantiser, staged in LDS once, also gives its 128 x 2
// row blocks (one per thread; output in the input's layout).  A workgroup walks kBothTiles
// column tiles of one 128-row band, loading the next tile into registers while it quantises the
// current one, so each compute unit keeps more of the input in flight.
// in [batch][rows][cols] -> q [batch][rows][cols] + scale [batch][rows][cols/32] and
// qT [batch][cols][rows] + scaleT [batch][cols][rows/32].  rows % 32 == 0, cols % 64 == 0.
// 1-D grid of cgroups * bands * batch blocks, work items ordered column groups fastest, then bands,
// then matrices, dealt to the XCDs in contiguous runs (xcd_run_item).
constexpr int kBothTiles = 4;

// Work item of block `id` when XCD x (block ids = x mod 8, each XCD with its own L2) takes the
// contiguous run of items [start(x), start(x + 1)): the workgroups that fill one scale line (the
// column groups of a band) then run side by side on one XCD, whose L2 merges their bytes before
// the line is written back (dealt round-robin, a line's pieces sat in up to eight L2s).
__device__ __forceinline__ long long xcd_run_item(long long id, long long total) {
  const long long per = total >> 3, extra = total & 7;
  const long long x = id & 7, j = id >> 3;
  return x * per + (x < extra ? x : extra) + j;
}

__device__ __forceinline__ void load_tile_regs(const uint16_t* __restrict__ src, int rows, int cols, int r0, int c0,
                                               uint4 (&v)[4]) {
  const int cc = threadIdx.x & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (threadIdx.x >> 3) + 32 * i;
    v[i] = make_uint4(0, 0, 0, 0);
    if (r0 + r < rows && c0 < cols)
      v[i] = *reinterpret_cast<const uint4*>(src + static_cast<long long>(r0 + r) * cols + c0 + 8 * cc);
  }
}

// At most two waves per SIMD (two workgroups per compute unit): measured 8-10% faster than the
// six the registers would allow, and faster than one, three or four (each workgroup's 128 source
// rows are read as 128-byte pieces, and fewer bands in flight at once keep the DRAM and L2 traffic
// of the two output layouts more local).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void quant_both_kernel(const uint16_t* __restrict__ in, int rows, int cols,
                                                         uint8_t* __restrict__ q, uint8_t* __restrict__ scale,
                                                         uint8_t* __restrict__ qT, uint8_t* __restrict__ scaleT,
                                                         int cgroups, int bands, long long total) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kTP][kPitch];
  const long long item = xcd_run_item(blockIdx.x, total);
  const long long b = item / (static_cast<long long>(cgroups) * bands);
  const int rest = static_cast<int>(item - b * cgroups * bands);
  const int r0 = (rest / cgroups) * kTP;
  const long long plane = static_cast<long long>(rows) * cols;
  const uint16_t* src = in + b * plane;
  const int cc = threadIdx.x & 7;
  int c0 = (rest % cgroups) * kTC * kBothTiles;
  uint4 v[4];
  load_tile_regs(src, rows, cols, r0, c0, v);
  for (int it = 0; it < kBothTiles && c0 < cols; ++it, c0 += kTC) {
    __syncthreads();   // the previous tile's readers are done with the LDS tile
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t* t = reinterpret_cast<uint32_t*>(&tile[(threadIdx.x >> 3) + 32 * i][8 * cc]);
      t[0] = v[i].x; t[1] = v[i].y; t[2] = v[i].z; t[3] = v[i].w;
    }
    __syncthreads();
    if (it + 1 < kBothTiles) load_tile_regs(src, rows, cols, r0, c0 + kTC, v);
    // row blocks: row t/2, columns 32 (t%2) .. + 31 of the tile
    {
      const int r = threadIdx.x >> 1, blk = threadIdx.x & 1;
      if (r0 + r < rows) {
        uint32_t vals[32];
        const uint32_t* w = reinterpret_cast<const uint32_t*>(&tile[r][32 * blk]);
        uint32_t amax = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t x = w[i];
          vals[2 * i] = x & 0xffffu;
          vals[2 * i + 1] = x >> 16;
          amax = max(amax, max(x & 0x7fffu, (x >> 16) & 0x7fffu));
        }
        const int sh = mx_shared_exp(amax);
        uint32_t o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = mx_encode4(vals[4 * i], vals[4 * i + 1], vals[4 * i + 2], vals[4 * i + 3], sh);
        const long long row = r0 + r;
        uint8_t* dst = q + b * plane + row * cols + c0 + 32 * blk;
        reinterpret_cast<uint4*>(dst)[0] = make_uint4(o[0], o[1], o[2], o[3]);
        reinterpret_cast<uint4*>(dst)[1] = make_uint4(o[4], o[5], o[6], o[7]);
        scale[b * (plane / 32) + mx_gemm_scale_index(row, c0 / 32 + blk, rows, cols)] =
            static_cast<uint8_t>(sh + 127);
      }
    }
    // column blocks, as the column quantiser
    if (r0 + (threadIdx.x & 3) * 32 < rows)
      quant_tile_columns(tile, kTC, r0, rows, qT + b * plane + static_cast<long long>(c0) * rows,
                         scaleT + b * (plane / 32), 0, 0, 0, cols, rows, c0);
  }
}

// Column tiles a grouped-quantiser workgroup walks along one band.
constexpr int kGroupTiles = 4;

// Grouped token-axis blocks.  Padded position p in [offsets_pad[e], offsets_pad[e+1]) holds
// grouped row r = offsets[e] + (p - offsets_pad[e]) if r < offsets[e+1], else zero; positions
// from offsets_pad[E] to n_pad_cap hold zeros.  Row r's data is in[row_token ? row_token[r] : r].
// With row_gate, grouped row r is bf16(row_gate[r] * in[row_token[r]]) (fp32 product, round to
// nearest even): the rows the fused MXFP8 combine backward never writes in bf16.
// q [C][n_pad_cap], scale [n_pad_cap/32][C].  With ROWS (contiguous rows, no gather, no gate), the
// same tiles also give the real rows' row blocks: qr [n][C] and their scales sr in the GEMM layout
// (mx_gemm_scale_index, R = n), so a tensor both products need (dG, dU) is read once for its two
// layouts.
// A workgroup takes a 128-position band and walks
// kGroupTiles column tiles of it (the rows' adjacent 128-byte pieces, read close together in time,
// with the next tile's loads in flight while the current one is quantised); the band's source
// rows are looked up once.  Without a gather (contiguous rows), the column groups of one band
// have adjacent block ids, so the workgroups reading the rest of the same source rows run
// alongside (whole rows stream from DRAM together: 25% faster at the MXFP8 workload); with a
// gather through row_token the bands come first (measured slightly faster), as they do whenever
// there are more than 65535 bands.  grid: (ceil(C / (64 kGroupTiles)), n_pad_cap/128), or
// transposed (bands in x).
template <bool ROWS>
__device__ __forceinline__ void quant_grouped_body(const uint16_t* __restrict__ in,
                                                            const int32_t* __restrict__ row_token,
                                                            const float* __restrict__ row_gate,
                                                            const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ offsets_pad, int E, int C,
                                                            long long n_pad_cap, uint8_t* __restrict__ q,
                                                            uint8_t* __restrict__ scale, int band, int cgroup,
                                                            uint8_t* __restrict__ qr, uint8_t* __restrict__ sr,
                                                            long long nrows) {
  __shared__ uint16_t tile[kTP][kPitch];
  __shared__ int s_off[257];
  __shared__ int s_offp[257];
  __shared__ long long s_src[kTP];
  __shared__ float s_gate[kTP];
  for (int i = threadIdx.x; i <= E; i += 256) {
    s_off[i] = offsets[i];
    s_offp[i] = offsets_pad[i];
  }
  __syncthreads();
  const long long p0 = static_cast<long long>(band) * kTP;
  if (threadIdx.x < kTP) {
    const long long p = p0 + threadIdx.x;
    long long src = -1;
    if (p < s_offp[E]) {
      int lo = 0, hi = E - 1;                 // last e with offsets_pad[e] <= p
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_offp[mid] <= p) lo = mid; else hi = mid - 1;
      }
      const long long r = s_off[lo] + (p - s_offp[lo]);
      if (r < s_off[lo + 1]) {
        src = row_token ? row_token[r] : r;
        if (row_gate) s_gate[threadIdx.x] = row_gate[r];
      }
    }
    s_src[threadIdx.x] = src;
  }
  __syncthreads();
  const int cc = threadIdx.x & 7;
  long long src[4];
  float gt[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    src[i] = s_src[(threadIdx.x >> 3) + 32 * i];
    gt[i] = (row_gate && src[i] >= 0) ? s_gate[(threadIdx.x >> 3) + 32 * i] : 1.f;
  }
  auto load = [&](int c0, uint4 (&v)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = make_uint4(0, 0, 0, 0);
      if (src[i] >= 0 && c0 < C) v[i] = *reinterpret_cast<const uint4*>(in + src[i] * C + c0 + 8 * cc);
    }
  };
  // the gated rows, formed once the loads have landed (just before the tile goes to LDS)
  auto gated = [&](uint4 (&v)[4]) {
    if (!row_gate) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
      uint32_t o[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) o[h] = pack_bf16x2(gt[i] * bf16_lo(w[h]), gt[i] * bf16_hi(w[h]));
      v[i] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  };
  int c0 = cgroup * kTC * kGroupTiles;
  uint4 v[4];
  load(c0, v);
  for (int it = 0; it < kGroupTiles && c0 < C; ++it, c0 += kTC) {
    gated(v);
    if constexpr (ROWS) {
      // row blocks from the registers: v[i] is columns c0 + 8 (t % 8) .. + 7 of row src[i], so a
      // 32-column block is 4 adjacent lanes (amax by two shuffles), each writing 8 codes
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        uint32_t amax = 0;
#pragma unroll
        for (int h = 0; h < 4; ++h) amax = max(amax, max(w[h] & 0x7fffu, (w[h] >> 16) & 0x7fffu));
        amax = max(amax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(amax), 1, 64)));
        amax = max(amax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(amax), 2, 64)));
        if (src[i] >= 0 && c0 < C) {
          const int sh = mx_shared_exp(amax);
          const uint32_t o0 = mx_encode4(w[0] & 0xffffu, w[0] >> 16, w[1] & 0xffffu, w[1] >> 16, sh);
          const uint32_t o1 = mx_encode4(w[2] & 0xffffu, w[2] >> 16, w[3] & 0xffffu, w[3] >> 16, sh);
          const int col = c0 + 8 * cc;
          *reinterpret_cast<uint2*>(qr + src[i] * C + col) = make_uint2(o0, o1);
          if ((cc & 3) == 0) sr[mx_gemm_scale_index(src[i], col / 32, nrows, C)] = static_cast<uint8_t>(sh + 127);
        }
      }
    }
    __syncthreads();   // the previous tile's readers are done with the LDS tile
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t* t = reinterpret_cast<uint32_t*>(&tile[(threadIdx.x >> 3) + 32 * i][8 * cc]);
      t[0] = v[i].x; t[1] = v[i].y; t[2] = v[i].z; t[3] = v[i].w;
    }
    __syncthreads();
    if (it + 1 < kGroupTiles) load(c0 + kTC, v);
    quant_tile_columns(tile, kTC, p0, n_pad_cap, q + static_cast<long long>(c0) * n_pad_cap, scale + c0, 1, C);
  }
}

__global__ __launch_bounds__(256) void quant_grouped_kernel(const uint16_t* __restrict__ in,
                                                            const int32_t* __restrict__ row_token,
                                                            const float* __restrict__ row_gate,
                                                            const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ offsets_pad, int E, int C,
                                                            long long n_pad_cap, uint8_t* __restrict__ q,
                                                            uint8_t* __restrict__ scale, int bands_in_x) {
  quant_grouped_body<false>(in, row_token, row_gate, offsets, offsets_pad, E, C, n_pad_cap, q, scale,
                            bands_in_x ? blockIdx.x : blockIdx.y, bands_in_x ? blockIdx.y : blockIdx.x, nullptr,
                            nullptr, 0);
}

// The rows + grouped form runs at most two waves per SIMD (8% faster than the four its registers
// allow, and than five or three, at the MXFP8 workload's dG), on a 1-D grid of bands * cgroups
// blocks dealt to the XCDs in contiguous runs (column groups fastest), so the column groups that
// fill one row's scale line run on one XCD and its L2 merges the pieces (as the weight quantiser).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void quant_rows_grouped_kernel(
    const uint16_t* __restrict__ in, const int32_t* __restrict__ offsets, const int32_t* __restrict__ offsets_pad,
    int E, int C, long long n_pad_cap, uint8_t* __restrict__ q, uint8_t* __restrict__ scale, int cgroups,
    long long total, uint8_t* __restrict__ qr, uint8_t* __restrict__ sr, long long nrows) {
  const long long item = xcd_run_item(blockIdx.x, total);
  quant_grouped_body<true>(in, nullptr, nullptr, offsets, offsets_pad, E, C, n_pad_cap, q, scale,
                           static_cast<int>(item / cgroups), static_cast<int>(item % cgroups), qr, sr, nrows);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_mx_pad_cap(int n, int E) {
  const long long cap = (static_cast<long long>(n) + 128LL * E + 127) / 128 * 128;
  return cap < (1LL << 31) ? static_cast<int>(cap) : -1;
}

extern "C" int mxfp8_quantize(const uint16_t* in, int batch, int rows, int cols, int axis, int scale_mode,
                              uint8_t* q, uint8_t* scale, void* stream) {
  MOE_CHECK_PTR(in); MOE_CHECK_PTR(q); MOE_CHECK_PTR(scale);
  MOE_CHECK_ALIGN(in); MOE_CHECK_ALIGN(q);
  MOE_REQUIRE(batch >= 1 && rows >= 1 && cols >= 1, MOE_ERR_INVALID_ARG, "sizes must be positive");
  MOE_REQUIRE(scale_mode == 0 || scale_mode == 1, MOE_ERR_INVALID_ARG, "scale_mode must be 0 or 1");
  hipStream_t s = as_stream(stream);
  if (axis == 0) {
    MOE_REQUIRE(cols % 32 == 0, MOE_ERR_UNSUPPORTED, "axis 0 needs cols %% 32 == 0");
    const long long total = static_cast<long long>(batch) * rows * cols;
    quant_rows_kernel<<<static_cast<unsigned>((total / 8 + 255) / 256), 256, 0, s>>>(in, total, q, scale,
                                                                                    scale_mode, 0, cols);
    return check_launch("mxfp8_quantize rows");
  }
  MOE_REQUIRE(axis == 1, MOE_ERR_INVALID_ARG, "axis must be 0 or 1");
  MOE_REQUIRE(rows % 32 == 0 && cols % 64 == 0, MOE_ERR_UNSUPPORTED, "axis 1 needs rows %% 32 == 0, cols %% 64 == 0");
  MOE_REQUIRE(batch <= 65535, MOE_ERR_UNSUPPORTED, "batch too large");
  dim3 grid((rows + kTP - 1) / kTP, cols / kTC, batch);
  quant_cols_kernel<<<grid, 256, 0, s>>>(in, rows, cols, q, scale, scale_mode);
  return check_launch("mxfp8_quantize cols");
}

extern "C" int mxfp8_quantize_both(const uint16_t* in, int batch, int rows, int cols, uint8_t* q, uint8_t* scale,
                                   uint8_t* qT, uint8_t* scaleT, void* stream) {
  MOE_CHECK_PTR(in); MOE_CHECK_PTR(q); MOE_CHECK_PTR(scale); MOE_CHECK_PTR(qT); MOE_CHECK_PTR(scaleT);
  MOE_CHECK_ALIGN(in); MOE_CHECK_ALIGN(q); MOE_CHECK_ALIGN(qT);
  MOE_REQUIRE(batch >= 1 && rows >= 1 && cols >= 1, MOE_ERR_INVALID_ARG, "sizes must be positive");
  MOE_REQUIRE(rows % 32 == 0 && cols % 64 == 0, MOE_ERR_UNSUPPORTED, "need rows %% 32 == 0, cols %% 64 == 0");
  const int cgroups = (cols / kTC + kBothTiles - 1) / kBothTiles, bands = (rows + kTP - 1) / kTP;
  const long long total = static_cast<long long>(cgroups) * bands * batch;
  MOE_REQUIRE(total <= 0x7fffffffLL, MOE_ERR_UNSUPPORTED, "too many tiles");
  quant_both_kernel<<<static_cast<unsigned>(total), 256, 0, as_stream(stream)>>>(in, rows, cols, q, scale, qT, scaleT,
                                                                                 cgroups, bands, total);
  return check_launch("mxfp8_quantize_both");
}

static int quantize_grouped(const uint16_t* in, const int32_t* row_token, const float* row_gate,
                            const int32_t* offsets, const int32_t* offsets_pad, int E, int n, int C, uint8_t* qT,
                            uint8_t* scaleT, void* stream, uint8_t* q_rows = nullptr, uint8_t* s_rows = nullptr) {
  MOE_CHECK_PTR(in); MOE_CHECK_PTR(offsets); MOE_CHECK_PTR(offsets_pad); MOE_CHECK_PTR(qT); MOE_CHECK_PTR(scaleT);
  MOE_CHECK_ALIGN(in); MOE_CHECK_ALIGN(qT);
  MOE_REQUIRE(E >= 1 && E <= 256, MOE_ERR_UNSUPPORTED, "E must be in [1, 256]");
  MOE_REQUIRE(n >= 1 && C >= 64 && C % 64 == 0, MOE_ERR_UNSUPPORTED, "need n >= 1 and C a multiple of 64");
  const int cap = moe_mx_pad_cap(n, E);
  MOE_REQUIRE(cap > 0, MOE_ERR_UNSUPPORTED, "padded token axis too long");
  const int bands = cap / kTP, cgroups = (C / kTC + kGroupTiles - 1) / kGroupTiles;
  const int bands_in_x = (bands > 65535 || row_token != nullptr) ? 1 : 0;
  dim3 grid(bands_in_x ? bands : cgroups, bands_in_x ? cgroups : bands);
  if (q_rows != nullptr) {
    const long long total = static_cast<long long>(bands) * cgroups;
    MOE_REQUIRE(total <= 0x7fffffffLL, MOE_ERR_UNSUPPORTED, "too many tiles");
    quant_rows_grouped_kernel<<<static_cast<unsigned>(total), 256, 0, as_stream(stream)>>>(
        in, offsets, offsets_pad, E, C, cap, qT, scaleT, cgroups, total, q_rows, s_rows, n);
  } else
    quant_grouped_kernel<<<grid, 256, 0, as_stream(stream)>>>(in, row_token, row_gate, offsets, offsets_pad, E, C, cap,
                                                               qT, scaleT, bands_in_x);
  return check_launch("mxfp8_quantize_grouped");
}

extern "C" int mxfp8_quantize_grouped(const uint16_t* in, const int32_t* row_token, const int32_t* offsets,
                                      const int32_t* offsets_pad, int E, int n, int C, uint8_t* qT, uint8_t* scaleT,
                                      void* stream) {
  return quantize_grouped(in, row_token, nullptr, offsets, offsets_pad, E, n, C, qT, scaleT, stream);
}

extern "C" int mxfp8_quantize_grouped_gated(const uint16_t* in, const int32_t* row_token, const float* row_gate,
                                            const int32_t* offsets, const int32_t* offsets_pad, int E, int n, int C,
                                            uint8_t* qT, uint8_t* scaleT, void* stream) {
  MOE_CHECK_PTR(row_token); MOE_CHECK_PTR(row_gate);
  return quantize_grouped(in, row_token, row_gate, offsets, offsets_pad, E, n, C, qT, scaleT, stream);
}

extern "C" int mxfp8_quantize_rows_grouped(const uint16_t* in, const int32_t* offsets, const int32_t* offsets_pad,
                                           int E, int n, int C, uint8_t* q_rows, uint8_t* s_rows, uint8_t* qT,
                                           uint8_t* scaleT, void* stream) {
  MOE_CHECK_PTR(q_rows); MOE_CHECK_PTR(s_rows);
  MOE_CHECK_ALIGN(q_rows);
  return quantize_grouped(in, nullptr, nullptr, offsets, offsets_pad, E, n, C, qT, scaleT, stream, q_rows, s_rows);
}

extern "C" int mxfp8_quantize_gemm(const uint16_t* in, int batch, int rows, int cols, uint8_t* q, uint8_t* scale,
                                   void* stream) {
  MOE_CHECK_PTR(in); MOE_CHECK_PTR(q); MOE_CHECK_PTR(scale);
  MOE_CHECK_ALIGN(in); MOE_CHECK_ALIGN(q);
  MOE_REQUIRE(batch >= 1 && rows >= 1 && cols >= 1, MOE_ERR_INVALID_ARG, "sizes must be positive");
  MOE_REQUIRE(cols % 32 == 0, MOE_ERR_UNSUPPORTED, "need cols %% 32 == 0");
  const long long total = static_cast<long long>(batch) * rows * cols;
  MOE_REQUIRE(total / 8 / 256 < 0x7fffffffLL, MOE_ERR_UNSUPPORTED, "tensor too large");
  quant_rows_kernel<<<static_cast<unsigned>((total / 8 + 255) / 256), 256, 0, as_stream(stream)>>>(in, total, q, scale,
                                                                                                 0, rows, cols);
  return check_launch("mxfp8_quantize_gemm");
}

namespace moe {
namespace {
// out[matrix][mx_gemm_scale_index(r, b, rows, K)] = in[matrix][r][b], one byte per thread.
__global__ __launch_bounds__(256) void scales_to_gemm_kernel(const uint8_t* __restrict__ in, long long total, int rows,
                                                             int K, uint8_t* __restrict__ out) {
  const long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= total) return;
  const long long per = static_cast<long long>(rows) * (K / 32);
  const long long m = i / per, rem = i - m * per;
  const long long r = rem / (K / 32), b = rem - r * (K / 32);
  out[m * per + mx_gemm_scale_index(r, b, rows, K)] = in[i];
}
}  // namespace
}  // namespace moe

extern "C" int mxfp8_scales_to_gemm(const uint8_t* in, int batch, int rows, int K, uint8_t* out, void* stream) {
  MOE_CHECK_PTR(in); MOE_CHECK_PTR(out);
  MOE_REQUIRE(batch >= 1 && rows >= 1 && K >= 32, MOE_ERR_INVALID_ARG, "sizes must be positive");
  MOE_REQUIRE(K % 32 == 0, MOE_ERR_UNSUPPORTED, "need K %% 32 == 0");
  MOE_REQUIRE(in != out, MOE_ERR_INVALID_ARG, "in and out must not alias");
  const long long total = static_cast<long long>(batch) * rows * (K / 32);
  MOE_REQUIRE(total / 256 < 0x7fffffffLL, MOE_ERR_UNSUPPORTED, "tensor too large");
  scales_to_gemm_kernel<<<static_cast<unsigned>((total + 255) / 256), 256, 0, as_stream(stream)>>>(in, total, rows, K,
                                                                                                  out);
  return check_launch("mxfp8_scales_to_gemm");
}
