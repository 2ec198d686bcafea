// Router: logits, sigmoid affinities, bias-steered group-limited top-K, gates and
// per-expert counts (DeepSeek-V3 report summary on mpbf.cn, section 2.2: sigmoid
// gating renormalised over the chosen experts; a per-expert bias that only steers
// the choice; node-limited routing by the summed affinity of each node's experts;
// whole-batch expert loads).
//
// Numerics are fixed so the result is reproducible bit for bit:
//   z[t,e]  = sequential fused multiply-add over h = 0..H-1, starting from +0
//             (fp32 VALU, compiled without contraction; MFMA is not used because
//             its internal summation order is not a sequential chain)
//   s       = 1 / (1 + exp(-clamp(z, -80, 80)))   with exp by Cody-Waite
//             reduction and a degree-7 Taylor polynomial (Horner, fused)
//   key     = s + bias[e]
//   group   = fp32 sum from 0 of the J largest keys of the group
//   ranking = (value descending, index ascending) for groups and experts
//   gate    = s / (s_0 + s_1 + ... + s_{K-1}) in rank order, IEEE division
#include "common.h"

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// Logits: lanes are tokens, experts are wave-uniform.  A workgroup takes 64 tokens x
// 8*kRE experts; its 8 waves share the tokens' hidden chunk (64 h at a time, in LDS as
// fp32, one padded row per token) and each wave owns kRE experts, whose router-weight
// rows it reads with scalar loads, so each fused multiply-add takes its weight operand
// from a scalar register and its x operand from the lane's own row.  Every
// accumulator sees h in increasing order.  kRE = 4 when there are enough tokens to fill
// the GPU (fewer weight loads per multiply-add); up to 3072 tokens kRE = 1, which gives
// four times as many waves to hide the latency of the chunk loads (T=128: 0.22 ->
// 0.10 ms, T=2048: 0.31 -> 0.26 ms; logits unchanged bit for bit).
// ---------------------------------------------------------------------------
constexpr int RT = 64, RWV = 8, RH = 64, RROW = RH + 4;

template <typename XT, int RE>
__global__ __launch_bounds__(RWV * kWave) void k_router_logits(const XT* __restrict__ x,
                                                               const float* __restrict__ w,
                                                               float* __restrict__ z,
                                                               int32_t* __restrict__ counts,
                                                               int T, int H, int E) {
  __shared__ __attribute__((aligned(16))) float xs[2][RT * RROW];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = blockIdx.x * RT;
  const int eb = blockIdx.y * (RE * RWV) + wv * RE;
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int e = tid; e < E; e += RWV * kWave) counts[e] = 0;  // zeroed before the select kernel

  // loader: token row tid/8, 8 consecutive h at (tid%8)*8
  const int lr = tid >> 3, lh = (tid & 7) * 8;
  const XT* xp = x + (int64_t)min(t0 + lr, T - 1) * H + lh;
  const float* wr[RE];
#pragma unroll
  for (int e = 0; e < RE; ++e) wr[e] = w + (int64_t)min(eb + e, E - 1) * H;

  float xr[8];
  auto gload = [&](int h0) {
    if constexpr (sizeof(XT) == 2) {
      const uint4 v = *reinterpret_cast<const uint4*>(xp + h0);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xr[2 * i] = __uint_as_float(u[i] << 16);
        xr[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
      }
    } else {
      const float4 a = *reinterpret_cast<const float4*>(xp + h0);
      const float4 b = *reinterpret_cast<const float4*>(xp + h0 + 4);
      xr[0] = a.x; xr[1] = a.y; xr[2] = a.z; xr[3] = a.w;
      xr[4] = b.x; xr[5] = b.y; xr[6] = b.z; xr[7] = b.w;
    }
  };
  auto lstore = [&](int buf) {
    float* d = &xs[buf][lr * RROW + lh];
    *reinterpret_cast<float4*>(d) = make_float4(xr[0], xr[1], xr[2], xr[3]);
    *reinterpret_cast<float4*>(d + 4) = make_float4(xr[4], xr[5], xr[6], xr[7]);
  };

  float acc[RE];
#pragma unroll
  for (int e = 0; e < RE; ++e) acc[e] = 0.0f;
  const int nchunk = H / RH;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int c = 0; c < nchunk; ++c) {
    const int buf = c & 1;
    if (c + 1 < nchunk) gload((c + 1) * RH);
    const float* xrow = &xs[buf][lane * RROW];
    const int hc = c * RH;
    // register double buffer: the loads of step hh+8 (x from LDS, weights with scalar
    // loads) are issued before the multiply-adds of step hh, which use the values
    // loaded one step earlier
    float xc[8], wc[RE][8];
    {
      const float4 xa = *reinterpret_cast<const float4*>(xrow);
      const float4 xb = *reinterpret_cast<const float4*>(xrow + 4);
      xc[0] = xa.x; xc[1] = xa.y; xc[2] = xa.z; xc[3] = xa.w;
      xc[4] = xb.x; xc[5] = xb.y; xc[6] = xb.z; xc[7] = xb.w;
#pragma unroll
      for (int e = 0; e < RE; ++e)
#pragma unroll
        for (int j = 0; j < 8; ++j) wc[e][j] = wr[e][hc + j];
    }
#pragma unroll
    for (int hh = 0; hh < RH; hh += 8) {
      float xn[8], wn[RE][8];
      if (hh + 8 < RH) {
        const float4 xa = *reinterpret_cast<const float4*>(xrow + hh + 8);
        const float4 xb = *reinterpret_cast<const float4*>(xrow + hh + 12);
        xn[0] = xa.x; xn[1] = xa.y; xn[2] = xa.z; xn[3] = xa.w;
        xn[4] = xb.x; xn[5] = xb.y; xn[6] = xb.z; xn[7] = xb.w;
#pragma unroll
        for (int e = 0; e < RE; ++e)
#pragma unroll
          for (int j = 0; j < 8; ++j) wn[e][j] = wr[e][hc + hh + 8 + j];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < RE; ++e) acc[e] = __builtin_fmaf(xc[j], wc[e][j], acc[e]);
      if (hh + 8 < RH) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          xc[j] = xn[j];
#pragma unroll
          for (int e = 0; e < RE; ++e) wc[e][j] = wn[e][j];
        }
      }
    }
    if (c + 1 < nchunk) lstore(buf ^ 1);
    __syncthreads();
  }
  const int t = t0 + lane;
  if (t < T)
#pragma unroll
    for (int e = 0; e < RE; ++e)
      if (eb + e < E) z[(int64_t)t * E + eb + e] = acc[e];
}

// (value, index) ordering: larger value first, then the lower index.
__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// ---------------------------------------------------------------------------
// Selection: one wave per token, 4 tokens per workgroup.  Lane l holds experts
// l, l+64, ... (at most 8).  Keys and affinities go to LDS; lane g < G ranks the
// keys of group g and sums its J best; lane g then ranks its group among all G;
// K rounds of a wave-wide (key, index) argmax over the kept groups pick the experts
// in rank order.  Expert counts go to an LDS histogram per workgroup, added to the
// global counts once at the end (at large batches the per-token global atomics on 256
// addresses were the kernel's main cost).
// ---------------------------------------------------------------------------
constexpr int kMaxE = 512, kMaxPer = kMaxE / kWave, kMaxG = 64;

template <int kJ>
__global__ __launch_bounds__(256) void k_router_select(const float* __restrict__ z,
                                                       const float* __restrict__ bias,
                                                       int32_t* __restrict__ idx, float* __restrict__ gate,
                                                       int32_t* __restrict__ counts, int T, int E, int G,
                                                       int M, int K) {
  __shared__ float s_key[4][kMaxE];
  __shared__ float s_aff[4][kMaxE];
  __shared__ float s_gscore[4][kMaxG];
  __shared__ int s_kept[4][kMaxG];
  __shared__ int s_cnt[kMaxE];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int gs = E / G;
  const int per = (E + kWave - 1) / kWave;
  for (int e = threadIdx.x; e < E; e += 256) s_cnt[e] = 0;
  // grid-stride over groups of 4 tokens (one per wave); the bounds are uniform over
  // the workgroup, so every wave takes part in every barrier
  for (int base = blockIdx.x * 4; base < T; base += gridDim.x * 4) {
    const int t_raw = base + wv;
    const bool live = t_raw < T;
    const int t = live ? t_raw : T - 1;
    __syncthreads();  // the previous token's LDS rows are no longer read

    float key[kMaxPer];
  #pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      key[i] = 0.0f;
      const int e = lane + kWave * i;
      if (i < per && e < E) {
        const float s = affinity(z[(int64_t)t * E + e]);
        key[i] = s + bias[e];
        s_key[wv][e] = key[i];
        s_aff[wv][e] = s;
      }
    }
    __syncthreads();

    if (lane < G) {
      // ordered list of the best keys so far, kept by carrying each new key down the
      // list and swapping where it ranks first (static indices: stays in registers)
      float top[kJ];
      int topi[kJ];
  #pragma unroll
      for (int q = 0; q < kJ; ++q) {
        top[q] = -__builtin_inff();
        topi[q] = 0x7FFFFFFF;
      }
      for (int e = lane * gs; e < (lane + 1) * gs; ++e) {
        float v = s_key[wv][e];
        int vi = e;
  #pragma unroll
        for (int q = 0; q < kJ; ++q) {
          if (ranks_before(v, vi, top[q], topi[q])) {
            const float tv = top[q];
            const int ti = topi[q];
            top[q] = v;
            topi[q] = vi;
            v = tv;
            vi = ti;
          }
        }
      }
      float sc = 0.0f;
  #pragma unroll
      for (int q = 0; q < kJ; ++q) sc = sc + top[q];
      s_gscore[wv][lane] = sc;
    }
    __syncthreads();
    if (lane < G) {
      const float mine = s_gscore[wv][lane];
      int rank = 0;
      for (int g = 0; g < G; ++g)
        rank += ranks_before(s_gscore[wv][g], g, mine, lane) ? 1 : 0;
      s_kept[wv][lane] = rank < M;
    }
    __syncthreads();

    bool avail[kMaxPer];
  #pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      const int e = lane + kWave * i;
      avail[i] = (i < per) && (e < E) && s_kept[wv][e / gs];
    }
    int my_e = 0;
    float my_s = 0.0f;
    for (int r = 0; r < K; ++r) {
      float bv = -__builtin_inff();
      int bi = 0x7FFFFFFF;
  #pragma unroll
      for (int i = 0; i < kMaxPer; ++i) {
        const int e = lane + kWave * i;
        if (avail[i] && ranks_before(key[i], e, bv, bi)) {
          bv = key[i];
          bi = e;
        }
      }
  #pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (ranks_before(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if (bi >= E) bi = 0;  // unreachable: K <= M*E/G candidates always exist
  #pragma unroll
      for (int i = 0; i < kMaxPer; ++i)
        if (bi == lane + kWave * i) avail[i] = false;
      if (lane == r) {
        my_e = bi;
        my_s = s_aff[wv][bi];
      }
    }
    float sum = 0.0f;
    for (int r = 0; r < K; ++r) sum = sum + __shfl(my_s, r);
    if (live && lane < K) {
      idx[(int64_t)t * K + lane] = my_e;
      gate[(int64_t)t * K + lane] = my_s / sum;
      atomicAdd(&s_cnt[my_e], 1);
    }
  }
  // one global addition per expert and workgroup (integer sums: order-free)
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256)
    if (s_cnt[e]) atomicAdd(&counts[e], s_cnt[e]);
}

}  // namespace

hipError_t launch_route(const Dims& d, const void* x, const float* w_router, const float* bias,
                        int32_t* idx, float* gate, int32_t* counts, float* logits,
                        hipStream_t st) {
  const int T = static_cast<int>(d.T);
  const bool few = T <= 3072;
  const int re = few ? 1 : 4;
  dim3 g1((T + RT - 1) / RT, (d.E + re * RWV - 1) / (re * RWV));
  if (d.act == MOE_BF16) {
    if (few)
      hipLaunchKernelGGL((k_router_logits<uint16_t, 1>), g1, dim3(RWV * kWave), 0, st,
                         static_cast<const uint16_t*>(x), w_router, logits, counts, T, d.H, d.E);
    else
      hipLaunchKernelGGL((k_router_logits<uint16_t, 4>), g1, dim3(RWV * kWave), 0, st,
                         static_cast<const uint16_t*>(x), w_router, logits, counts, T, d.H, d.E);
  } else {
    if (few)
      hipLaunchKernelGGL((k_router_logits<float, 1>), g1, dim3(RWV * kWave), 0, st,
                         static_cast<const float*>(x), w_router, logits, counts, T, d.H, d.E);
    else
      hipLaunchKernelGGL((k_router_logits<float, 4>), g1, dim3(RWV * kWave), 0, st,
                         static_cast<const float*>(x), w_router, logits, counts, T, d.H, d.E);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the group lists have exactly J entries (J <= 8); at most 16 workgroups per CU, each
  // then looping over its tokens, so the per-workgroup count histograms stay few
  const int sel_wg = std::min((T + 3) / 4, 16 * device_cu_count());
#define MOE_SELECT(J_)                                                                  \
  case J_:                                                                              \
    hipLaunchKernelGGL(k_router_select<J_>, dim3(sel_wg), dim3(256), 0, st, logits, bias, \
                       idx, gate, counts, T, d.E, d.G, d.M, d.K);                       \
    break;
  switch (d.J) {
    MOE_SELECT(1) MOE_SELECT(2) MOE_SELECT(3) MOE_SELECT(4)
    MOE_SELECT(5) MOE_SELECT(6) MOE_SELECT(7) MOE_SELECT(8)
    default: return hipErrorInvalidValue;
  }
#undef MOE_SELECT
  return hipGetLastError();
}

}  // namespace moe
