// Tile schedule of the persistent grouped GEMMs (bf16 and MXFP8): how many m-tiles each expert's
// rows make and which expert owns a global m-tile, computed by every wave from one round of loads
// (no LDS: the operand rings fill it), and the order of an expert's tiles.  Lane l of group r holds expert 64 r + l (at most 256).
#pragma once

#include "common.h"

namespace moe {
namespace gsched {

struct MTiles {
  int tiles[4], excl[4];   // m-tiles of the lane's expert, and m-tiles before it
  int total;
};

// m-tile prefix over experts (tiles of BM rows; an expert's last tile may be partial).
template <int BM>
__device__ __forceinline__ MTiles mtile_scan(const int32_t* __restrict__ offsets, int E) {
  const int lane = threadIdx.x & 63;
  MTiles m;
  int carry = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int ex = 64 * r + lane;
    const int tiles = ex < E ? (offsets[ex + 1] - offsets[ex] + BM - 1) / BM : 0;
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

// True when some expert's row count exceeds twice the mean (n / E, rounded up): weight gradients
// then deal tiles round-robin rather than in XCD-contiguous runs.
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

// The expert owning global m-tile mt (< total) and that expert's first m-tile.
__device__ __forceinline__ void mtile_find(const MTiles& m, int mt, int& e, int& first) {
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

// Local tile l of an expert's MT x NT tiles -> (m-tile, n-tile), in cells of CM m-tiles x CN
// n-tiles taken m-fastest inside a cell, cells n-group by n-group within each group of CM
// m-tiles (partial cells at the edges, no holes).  CM = 1, CN >= NT is plain n-fastest order.
__device__ __forceinline__ void cell_order(int l, int MT, int NT, int CM, int CN, int& m, int& n) {
  const int mg = l / (CM * NT);
  const int r = l - mg * CM * NT;
  const int cm = min(CM, MT - mg * CM);
  const int ng = r / (cm * CN);
  const int r2 = r - ng * cm * CN;
  m = mg * CM + r2 % cm;
  n = ng * CN + r2 / cm;
}

}  // namespace gsched
}  // namespace moe
