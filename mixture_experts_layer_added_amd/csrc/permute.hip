// Permute: the single-GPU form of the token dispatch (DeepSeek-V3 report summary on
// mpbf.cn, section 3.2: a transformer block runs attention, dispatch, the expert MLP,
// combine).  Every (token, chosen expert) pair gets one row of x_sorted; rows are
// grouped by expert in index order with tokens ascending inside an expert, and the
// shared expert's T rows follow.  The order is unique, so no atomics decide it:
//   1. k_perm_hist:    per 256-token block, a 64-bit token mask per (wave, expert)
//                      gives each pair its rank inside the block and the block's
//                      per-expert counts;
//   2. k_perm_scan:    per expert, an exclusive scan over blocks; over experts, the
//                      exclusive scan that gives the group offsets;
//   3. k_perm_scatter: one workgroup per token writes its rows, the index maps and
//                      the K+S copies of the token (FP8: quantised once per
//                      128-column tile, scale = amax/448, RNE-saturating E4M3);
//      k_perm_index:   the index maps alone, when the expert GEMM gathers its rows
//                      from x itself (then FP8 quantises each token once, in
//                      k_quant_act).
#include <mutex>

#include "common.h"

namespace moe {

// Scratch of moe_permute_noalloc: the per-pair ranks and the per-block expert counts and
// offsets that moe_permute keeps in the caller's workspace, in a fixed device array
// instead (one copy per GPU, held until the process ends).  Host code never passes
// `scratch` itself to a kernel: its device address comes from hipGetSymbolAddress,
// taken once per device with that device current.
constexpr size_t kPermuteScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) char scratch[kPermuteScratchBytes];

namespace {

constexpr int kBlockTok = 256;  // tokens per histogram block (4 waves)
typedef uint32_t pu32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t pu32x2 __attribute__((ext_vector_type(2)));
constexpr int kMaxE = 512;

__global__ __launch_bounds__(256) void k_perm_hist(const int32_t* __restrict__ idx,
                                                   int32_t* __restrict__ lrank,
                                                   int32_t* __restrict__ bcount, int T, int E, int K) {
  __shared__ unsigned long long mask[4][kMaxE];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  for (int i = tid; i < 4 * E; i += 256) mask[i / E][i % E] = 0ull;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kBlockTok + tid;
  const bool live = t < T;
  if (live)
    for (int k = 0; k < K; ++k) {
      const int e = idx[t * K + k];
      if (e >= 0 && e < E) atomicOr(&mask[wv][e], 1ull << lane);
    }
  __syncthreads();
  if (live) {
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int k = 0; k < K; ++k) {
      const int e = idx[t * K + k];
      int r = -1;
      if (e >= 0 && e < E) {
        r = __popcll(mask[wv][e] & below);
        for (int w = 0; w < wv; ++w) r += __popcll(mask[w][e]);
      }
      lrank[t * K + k] = r;
    }
  }
  for (int e = tid; e < E; e += 256) {
    int c = 0;
    for (int w = 0; w < 4; ++w) c += __popcll(mask[w][e]);
    bcount[(int64_t)blockIdx.x * E + e] = c;
  }
}

// One workgroup of 512 threads: thread e scans its expert over the blocks, then the
// workgroup scans the expert totals.
__global__ __launch_bounds__(512) void k_perm_scan(const int32_t* __restrict__ bcount,
                                                   int32_t* __restrict__ boff,
                                                   int32_t* __restrict__ offsets, int nb, int E,
                                                   int S, int T) {
  __shared__ int tot[kMaxE];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E)
    for (int b = 0; b < nb; ++b) {
      const int v = bcount[(int64_t)b * E + e];
      boff[(int64_t)b * E + e] = run;
      run += v;
    }
  tot[e] = (e < E) ? run : 0;
  __syncthreads();
  // Hillis-Steele inclusive scan over 512 entries
  for (int d = 1; d < kMaxE; d <<= 1) {
    const int v = (e >= d) ? tot[e - d] : 0;
    __syncthreads();
    tot[e] += v;
    __syncthreads();
  }
  if (e < E) offsets[e + 1] = tot[e];
  if (e == 0) offsets[0] = 0;
  if (e == 0 && S) offsets[E + 1] = tot[E - 1] + T;
}

template <bool kFp8, typename XT>
__global__ __launch_bounds__(256) void k_perm_scatter(
    const XT* __restrict__ x, const int32_t* __restrict__ idx, const int32_t* __restrict__ lrank,
    const int32_t* __restrict__ boff, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_token, int32_t* __restrict__ inv_perm, void* __restrict__ xs,
    float* __restrict__ xs_scale, int T, int H, int E, int K, int S) {
  __shared__ int rows[17];
  const int tid = threadIdx.x;
  const int t = blockIdx.x;
  if (tid < K) {
    const int e = idx[(int64_t)t * K + tid];
    int row = -1;
    if (e >= 0 && e < E) {
      row = offsets[e] + boff[(int64_t)(t / kBlockTok) * E + e] + lrank[(int64_t)t * K + tid];
      sorted_token[row] = t;
    }
    inv_perm[(int64_t)t * K + tid] = row;
    rows[tid] = row;
  } else if (tid == K && S) {
    const int row = offsets[E] + t;
    sorted_token[row] = t;
    rows[K] = row;
  }
  __syncthreads();
  const int nd = K + (S ? 1 : 0);
  if constexpr (!kFp8) {
    // 16-byte chunks of the row, copied to every destination row.  The copies are
    // stored non-temporally: the GEMM reads them much later, and cached they would only
    // push other lines out of the L2 (0.132 -> 0.118 ms at the V3 shape).
    const int nchunk = H * (int)sizeof(XT) / 16;
    const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)t * H);
    pu32x4* dst = reinterpret_cast<pu32x4*>(xs);
    for (int c = tid; c < nchunk; c += 256) {
      const uint4 u = src[c];
      const pu32x4 v = {u.x, u.y, u.z, u.w};
      for (int d = 0; d < nd; ++d) {
        const int r = rows[d];
        if (r >= 0) __builtin_nontemporal_store(v, dst + (int64_t)r * nchunk + c);
      }
    }
  } else {
    // bf16 in: chunk = 8 values; 16 consecutive lanes hold one 128-wide tile
    const int nchunk = H / 8, ntile = H / 128;
    const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)t * H);
    pu32x2* dst = reinterpret_cast<pu32x2*>(xs);
    for (int c0 = 0; c0 < nchunk; c0 += 256) {
      const int c = c0 + tid;
      const bool in = c < nchunk;  // nchunk is a multiple of 16: whole tiles per 16 lanes
      float v[8];
      float amax = 0.0f;
      if (in) {
        const uint4 u = src[c];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = __uint_as_float(w[i] << 16);
          v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
      }
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, off));
      if (in) {
        const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
        const pu32x2 q = {pack4_e4m3(v[0] / sc, v[1] / sc, v[2] / sc, v[3] / sc),
                          pack4_e4m3(v[4] / sc, v[5] / sc, v[6] / sc, v[7] / sc)};
        for (int d = 0; d < nd; ++d) {
          const int r = rows[d];
          if (r < 0) continue;
          __builtin_nontemporal_store(q, dst + (int64_t)r * nchunk + c);
          if ((c & 15) == 0) xs_scale[(int64_t)r * ntile + (c >> 4)] = sc;
        }
      }
    }
  }
}

// Index maps only: one thread per (token, k) pair and per shared row.
__global__ __launch_bounds__(256) void k_perm_index(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ lrank,
    const int32_t* __restrict__ boff, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_token, int32_t* __restrict__ inv_perm, int T, int E, int K,
    int S) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nroute = (int64_t)T * K;
  if (q < nroute) {
    const int t = (int)(q / K);
    const int e = idx[q];
    int row = -1;
    if (e >= 0 && e < E) {
      row = offsets[e] + boff[(int64_t)(t / kBlockTok) * E + e] + lrank[q];
      sorted_token[row] = t;
    }
    inv_perm[q] = row;
  } else if (S && q < nroute + T) {
    const int t = (int)(q - nroute);
    sorted_token[offsets[E] + t] = t;
  }
}

// Per-token activation quantisation (the FP8 path's x, once per token): 16 lanes per
// 128-column tile, scale = amax/448 (1 if the tile is all zeros), RNE-saturating E4M3.
__global__ __launch_bounds__(256) void k_quant_act(const uint16_t* __restrict__ x,
                                                   uint8_t* __restrict__ xq,
                                                   float* __restrict__ x_scale, int64_t nchunk) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;  // chunk of 8 values
  const bool in = c < nchunk;  // nchunk is a multiple of 16: whole tiles per 16 lanes
  float v[8];
  float amax = 0.0f;
  if (in) {
    const uint4 u = reinterpret_cast<const uint4*>(x)[c];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, off));
  if (in) {
    const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
    uint2 q;
    q.x = pack4_e4m3(v[0] / sc, v[1] / sc, v[2] / sc, v[3] / sc);
    q.y = pack4_e4m3(v[4] / sc, v[5] / sc, v[6] / sc, v[7] / sc);
    reinterpret_cast<uint2*>(xq)[c] = q;
    if ((c & 15) == 0) x_scale[c >> 4] = sc;
  }
}

}  // namespace

hipError_t launch_quantize_act(const Dims& d, const uint16_t* x, uint8_t* xq, float* x_scale,
                               hipStream_t st) {
  const int64_t nchunk = d.T * (int64_t)d.H / 8;
  hipLaunchKernelGGL(k_quant_act, dim3((unsigned)((nchunk + 255) / 256)), dim3(256), 0, st, x, xq,
                     x_scale, nchunk);
  return hipGetLastError();
}

size_t permute_ws_bytes(const Dims& d) {
  const int64_t nb = (d.T + kBlockTok - 1) / kBlockTok;
  return sizeof(int32_t) * (size_t)(d.T * d.K + 2 * nb * d.E) + 256;
}

size_t permute_scratch_capacity() { return kPermuteScratchBytes; }

namespace {
constexpr int kMaxScratchDevices = 64;
std::once_flag g_scratch_once[kMaxScratchDevices];
void* g_scratch_ptr[kMaxScratchDevices];
hipError_t g_scratch_err[kMaxScratchDevices];
}  // namespace

hipError_t permute_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

namespace {

__global__ void k_zero_i32(int32_t* __restrict__ p) { *p = 0; }

// Pairs outside [0,E): each wave counts its lanes' with a ballot and adds the wave's
// count once (grid-stride over the T*K pairs).
__global__ __launch_bounds__(256) void k_count_invalid(const int32_t* __restrict__ idx,
                                                       int64_t n, int E,
                                                       int32_t* __restrict__ n_invalid) {
  int cnt = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int e = idx[i];
    cnt += (e < 0 || e >= E) ? 1 : 0;
  }
  // wave sum by shuffles, then one atomic per wave
  for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off);
  if ((threadIdx.x & 63) == 0 && cnt) atomicAdd(n_invalid, cnt);
}

}  // namespace

hipError_t launch_count_invalid(const Dims& d, const int32_t* idx, int32_t* n_invalid,
                                hipStream_t st) {
  const int64_t n = d.T * d.K;
  // the clear is a kernel, not a memset, so the pair can sit in a captured graph
  hipLaunchKernelGGL(k_zero_i32, dim3(1), dim3(1), 0, st, n_invalid);
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4 * device_cu_count());
  hipLaunchKernelGGL(k_count_invalid, dim3((unsigned)blocks), dim3(256), 0, st, idx, n, d.E,
                     n_invalid);
  return hipGetLastError();
}

hipError_t launch_permute(const Dims& d, const void* x, const int32_t* idx, int32_t* offsets,
                          int32_t* sorted_token, int32_t* inv_perm, void* x_sorted,
                          float* x_scale, void* ws, hipStream_t st) {
  const int T = static_cast<int>(d.T);
  const int nb = (T + kBlockTok - 1) / kBlockTok;
  int32_t* lrank = static_cast<int32_t*>(ws);
  int32_t* bcount = lrank + (int64_t)T * d.K;
  int32_t* boff = bcount + (int64_t)nb * d.E;
  hipLaunchKernelGGL(k_perm_hist, dim3(nb), dim3(256), 0, st, idx, lrank, bcount, T, d.E, d.K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_perm_scan, dim3(1), dim3(512), 0, st, bcount, boff, offsets, nb, d.E, d.S,
                     T);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!x_sorted) {
    const int64_t n = (int64_t)T * d.K + (d.S ? T : 0);
    hipLaunchKernelGGL(k_perm_index, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, idx,
                       lrank, boff, offsets, sorted_token, inv_perm, T, d.E, d.K, d.S);
  } else if (d.expert == MOE_FP8_E4M3)
    hipLaunchKernelGGL((k_perm_scatter<true, uint16_t>), dim3(T), dim3(256), 0, st,
                       static_cast<const uint16_t*>(x), idx, lrank, boff, offsets, sorted_token,
                       inv_perm, x_sorted, x_scale, T, d.H, d.E, d.K, d.S);
  else if (d.act == MOE_BF16)
    hipLaunchKernelGGL((k_perm_scatter<false, uint16_t>), dim3(T), dim3(256), 0, st,
                       static_cast<const uint16_t*>(x), idx, lrank, boff, offsets, sorted_token,
                       inv_perm, x_sorted, x_scale, T, d.H, d.E, d.K, d.S);
  else
    hipLaunchKernelGGL((k_perm_scatter<false, float>), dim3(T), dim3(256), 0, st,
                       static_cast<const float*>(x), idx, lrank, boff, offsets, sorted_token,
                       inv_perm, x_sorted, x_scale, T, d.H, d.E, d.K, d.S);
  return hipGetLastError();
}

}  // namespace moe
