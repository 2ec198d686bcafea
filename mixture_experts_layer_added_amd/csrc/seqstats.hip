// Sequence-wise load statistic (DeepSeek-V3 report summary on mpbf.cn, section 2.2:
// besides the bias rule, a sequence-level balance term with a very small weight keeps
// any single sequence from extreme imbalance).  The pages give that term no formula,
// so this computes only the loads it is built from: per (sequence, expert) counts of
// the chosen experts, and per sequence the largest and smallest count, the number of
// experts left without a token and max / mean (the mean being the uniform share L*K/E
// of the sequence's L tokens).
//   k_seq_zero:  clears the counts (a fill kernel, so the call can be captured in a
//                graph);
//   k_seq_hist:  one workgroup per 256 tokens; a block inside one sequence adds an LDS
//                histogram of its K*256 choices to that sequence's counts once per
//                expert, a block that straddles sequences adds pair by pair (integer
//                atomics, so the result does not depend on their order);
//   k_seq_stats: one wave per sequence reduces its E counts.
// Tokens are assigned to sequences by binary search over the caller's offsets, clamped
// to [0, n_seq), and indices outside [0, E) are skipped, so every write stays inside
// the outputs whatever the inputs hold.
#include "common.h"

namespace moe {
namespace {

constexpr int kSeqBlock = 256;
constexpr int kSeqMaxE = 512;

__global__ __launch_bounds__(256) void k_seq_zero(int32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0;
}

// last s in [0, n_seq) with off[s] <= t: the sequence holding token t
__device__ __forceinline__ int seq_of(const int32_t* __restrict__ off, int n_seq, int64_t t) {
  int lo = 0, hi = n_seq;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= t) lo = mid;
    else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(256) void k_seq_hist(const int32_t* __restrict__ idx,
                                                  const int32_t* __restrict__ off, int n_seq,
                                                  int64_t T, int E, int K,
                                                  int32_t* __restrict__ counts) {
  __shared__ int hist[kSeqMaxE];
  __shared__ int s_lo, s_hi;
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * kSeqBlock;
  const int64_t t = t0 + tid;
  const int64_t t_last = min(t0 + kSeqBlock, T) - 1;
  if (tid == 0) s_lo = seq_of(off, n_seq, t0);
  if (tid == 1) s_hi = seq_of(off, n_seq, t_last);
  for (int e = tid; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const bool one = s_lo == s_hi;
  if (t <= t_last) {
    const int s = one ? s_lo : seq_of(off, n_seq, t);
    for (int k = 0; k < K; ++k) {
      const int e = idx[t * K + k];
      if (e < 0 || e >= E) continue;
      if (one) atomicAdd(&hist[e], 1);
      else atomicAdd(&counts[(int64_t)s * E + e], 1);
    }
  }
  if (!one) return;
  __syncthreads();
  for (int e = tid; e < E; e += 256)
    if (hist[e]) atomicAdd(&counts[(int64_t)s_lo * E + e], hist[e]);
}

// One wave per sequence: max, min and zero count over its E counts, and
// max / (L*K/E) = (float)(max*E) / (float)(L*K) (0 for an empty sequence).
__global__ __launch_bounds__(256) void k_seq_stats(const int32_t* __restrict__ counts,
                                                   const int32_t* __restrict__ off, int n_seq,
                                                   int E, int K, int32_t* __restrict__ stats,
                                                   float* __restrict__ ratio) {
  const int s = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (s >= n_seq) return;
  const int32_t* c = counts + (int64_t)s * E;
  int mx = INT32_MIN, mn = INT32_MAX, zeros = 0;
  for (int e = lane; e < E; e += kWave) {
    const int v = c[e];
    mx = max(mx, v);
    mn = min(mn, v);
    zeros += v == 0;
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    mx = max(mx, __shfl_xor(mx, d));
    mn = min(mn, __shfl_xor(mn, d));
    zeros += __shfl_xor(zeros, d);
  }
  if (lane == 0) {
    stats[s * 3 + 0] = mx;
    stats[s * 3 + 1] = mn;
    stats[s * 3 + 2] = zeros;
    const int64_t L = (int64_t)off[s + 1] - off[s];
    ratio[s] = L > 0 ? (float)((int64_t)mx * E) / (float)(L * K) : 0.0f;
  }
}

}  // namespace

hipError_t launch_seq_load_stats(const Dims& d, const int32_t* idx, const int32_t* seq_off,
                                 int n_seq, int32_t* counts, int32_t* stats, float* ratio,
                                 hipStream_t st) {
  const int64_t n = (int64_t)n_seq * d.E;
  const int64_t zb = min((n + 255) / 256, (int64_t)4096);
  hipLaunchKernelGGL(k_seq_zero, dim3((unsigned)zb), dim3(256), 0, st, counts, n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nb = (d.T + kSeqBlock - 1) / kSeqBlock;
  hipLaunchKernelGGL(k_seq_hist, dim3((unsigned)nb), dim3(256), 0, st, idx, seq_off, n_seq, d.T,
                     d.E, d.K, counts);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_seq_stats, dim3((unsigned)((n_seq + 3) / 4)), dim3(256), 0, st, counts,
                     seq_off, n_seq, d.E, d.K, stats, ratio);
  return hipGetLastError();
}

}  // namespace moe
