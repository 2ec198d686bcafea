// Tile schedule shared by the grouped GEMMs: row-tile prefix sums over the groups
// (built on the device from the permute offsets, so no host synchronisation), tile
// decode, and the cost-balanced split of the tile list over the XCDs.
//
// Group g has mt_g = ceil(m_g / BM) row tiles; a GEMM with nt column tiles has
// mt_start[NG]*nt tiles, ordered (group, column tile, row tile) so the row tiles that
// share one weight tile, and the column tiles that share one activation tile, are
// neighbours.  The grid is persistent and XCD-aware: workgroup w runs on XCD w%8
// (dispatch is round-robin over the 8 XCDs) and each XCD takes one contiguous range of
// the list, so neighbouring tiles share that XCD's L2.
#pragma once
#include "common.h"

namespace moe {
namespace sched {

constexpr int kMaxGroups = 513;
constexpr int kSchedPer = 9;  // groups per lane of wave 0 (64 * 9 >= kMaxGroups)

// Row-tile prefix sums of the groups into LDS: s_mt[g] = sum_{g' < g} ceil(m_g'/BM),
// s_mt[NG] = total.  Wave 0 scans; the whole workgroup waits.
__device__ __forceinline__ void build_schedule(const int32_t* __restrict__ offsets, int NG, int BM,
                                               int* s_mt) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    int loc[kSchedPer];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kSchedPer; ++i) {
      const int g = lane * kSchedPer + i;
      loc[i] = (g < NG) ? (offsets[g + 1] - offsets[g] + BM - 1) / BM : 0;
      sum += loc[i];
    }
    int incl = sum;
#pragma unroll
    for (int dd = 1; dd < kWave; dd <<= 1) {
      const int o = __shfl_up(incl, dd);
      if (lane >= dd) incl += o;
    }
    int run = incl - sum;
#pragma unroll
    for (int i = 0; i < kSchedPer; ++i) {
      const int g = lane * kSchedPer + i;
      if (g < NG) s_mt[g] = run;
      run += loc[i];
    }
    if (lane == kWave - 1) s_mt[NG] = incl;
  }
  __syncthreads();
}

// Tile decode: group by binary search over mt_start * nt.
struct Tile {
  int g, m_idx, n_idx;
};
__device__ __forceinline__ Tile decode_tile(int tile, const int32_t* mt_start, int NG, int nt) {
  int lo = 0, hi = NG;  // find g with mt_start[g]*nt <= tile < mt_start[g+1]*nt
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (mt_start[mid] * nt <= tile) lo = mid;
    else hi = mid;
  }
  const int g = lo;
  const int mt = mt_start[g + 1] - mt_start[g];
  const int local = tile - mt_start[g] * nt;
  Tile r;
  r.g = g;
  r.n_idx = local / mt;
  r.m_idx = local % mt;
  return r;
}

// Cost-balanced XCD split.  A tile's cost is taken as BM + its rows (weight stream plus
// activation rows); s_cost[g] = sum over groups g' < g of nt * (BM * mt_g' + m_g').  XCD x
// takes the tiles whose cumulative cost starts in [x, x+1) * total / 8, cut at column-
// block granularity, so a group's neighbouring tiles stay on one XCD and its L2 while
// heavy groups (the shared expert's full row tiles) do not pile up on one XCD.
__device__ __forceinline__ void build_costs(const int32_t* __restrict__ offsets, const int* s_mt,
                                            int NG, int BM, int nt, long long* s_cost) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    long long loc[kSchedPer];
    long long sum = 0;
#pragma unroll
    for (int i = 0; i < kSchedPer; ++i) {
      const int g = lane * kSchedPer + i;
      loc[i] = (g < NG) ? (long long)nt * ((long long)BM * (s_mt[g + 1] - s_mt[g]) +
                                           (offsets[g + 1] - offsets[g]))
                        : 0;
      sum += loc[i];
    }
    long long incl = sum;
#pragma unroll
    for (int dd = 1; dd < kWave; dd <<= 1) {
      const long long o = __shfl_up(incl, dd);
      if (lane >= dd) incl += o;
    }
    long long run = incl - sum;
#pragma unroll
    for (int i = 0; i < kSchedPer; ++i) {
      const int g = lane * kSchedPer + i;
      if (g < NG) s_cost[g] = run;
      run += loc[i];
    }
    if (lane == kWave - 1) s_cost[NG] = incl;
  }
  __syncthreads();
}

// First tile of XCD x (x = 0..8) under the cost split.
__device__ __forceinline__ int xcd_boundary(int x, const int32_t* __restrict__ offsets,
                                            const int* s_mt, const long long* s_cost, int NG,
                                            int BM, int nt) {
  if (x <= 0) return 0;
  if (x >= kXcds) return s_mt[NG] * nt;
  const long long target = s_cost[NG] * x / kXcds;
  int lo = 0, hi = NG;  // last g with s_cost[g] <= target
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_cost[mid] <= target) lo = mid;
    else hi = mid;
  }
  const int mt = s_mt[lo + 1] - s_mt[lo];
  const long long blk = (long long)BM * mt + (offsets[lo + 1] - offsets[lo]);
  const int n = blk > 0 ? (int)min((target - s_cost[lo]) / blk, (long long)nt) : 0;
  return s_mt[lo] * nt + n * mt;
}

}  // namespace sched
}  // namespace moe
