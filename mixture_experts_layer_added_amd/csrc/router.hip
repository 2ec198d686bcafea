// Router: logits, sigmoid affinities, bias-steered group-limited top-K, gates and
// per-expert counts (DeepSeek-V3 report summary on mpbf.cn, section 2.2: sigmoid
// gating renormalised over the chosen experts; a per-expert bias that only steers
// the choice; node-limited routing by the summed affinity of each node's experts;
// whole-batch expert loads).
//
// Numerics are fixed so the result is reproducible bit for bit:
//   z[t,e]  = sequential fused multiply-add over h = 0..H-1, starting from +0
//             (fp32, compiled without contraction: on the VALU, or on the matrix
//             cores with the k=1 fp32 MFMA, which adds one product to each
//             accumulator per instruction with a single rounding, i.e. an fma)
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
// Logits on the VALU (small batches; larger ones use the matrix-core kernel below):
// lanes are tokens, experts are wave-uniform.  A workgroup takes 64 tokens x 8*RE
// experts; its 8 waves share the tokens' hidden chunk (64 h at a time, in LDS as fp32,
// one padded row per token) and each wave owns RE experts, whose router-weight rows it
// reads with scalar loads, so each fused multiply-add takes its weight operand from a
// scalar register and its x operand from the lane's own row.  Every accumulator sees h
// in increasing order.  It runs with RE = 1: four times as many waves as RE = 4 hide
// the latency of the chunk loads at these batch sizes (T=128: 0.22 -> 0.10 ms, T=2048:
// 0.31 -> 0.26 ms; logits unchanged bit for bit).
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

// ---------------------------------------------------------------------------
// Logits on the matrix cores.  v_mfma_f32_16x16x1_4b_f32 adds one product a_i * b_j
// to each of its 4 x 16 x 16 accumulators and rounds once, exactly like a fused
// multiply-add (checked bit for bit against IEEE fma on gfx950, including products
// whose rounding before the addition would change the sum, and subnormal ones), so a
// chain of them over h = 0, 1, 2, ... is the sequential fma chain of the VALU kernel.
// A workgroup of 4 waves takes 64 tokens x 64 experts and wave w the 32 x 32 block of
// tokens 32(w&1).. and experts 32(w>>1)..; instruction block b covers tokens 16(b&1)..
// and experts 16(b>>1).., so A lane l carries token l%32 and B lane l expert
// 16(l/32) + l%16, and accumulator r of lane l is token 16(b&1) + 4(l/16) + r%4,
// expert 16(b>>1) + l%16 with b = r/4.
// x (as fp32) and W_r pass through three LDS buffers of 64 h, one padded row per token
// or expert.  Chunk j is loaded from memory while chunk j-3 is multiplied, written to
// LDS (buffer j%3) while chunk j-2 is, and published by that chunk's closing barrier,
// so the operand reads (two 16-byte reads per 4 h, two groups of 4 h ahead) run on
// across chunk boundaries and the waves never drain.  While a chained MFMA waits for
// its predecessor the wave issues nothing else, so the reads and the LDS writes are
// placed after the first MFMA of each group of four.
// ---------------------------------------------------------------------------
constexpr int MT = 64, ME = 64, MH = 64, MROW = MH + 4, MG = MH / 4;
// from this many tokens the logits run on the matrix cores (one 32 x 32 block per
// wave; with fewer, too few waves fill the SIMDs: the route call at T=1024 took 0.20 ms
// here against 0.14 ms on the VALU, at T=2048 0.21 against 0.26 ms)
constexpr int kMfmaLogitsMinTokens = 2048;

template <typename XT>
__global__ __launch_bounds__(256) void k_router_logits_mfma(const XT* __restrict__ x,
                                                            const float* __restrict__ w,
                                                            float* __restrict__ z,
                                                            int32_t* __restrict__ counts,
                                                            int T, int H, int E) {
  __shared__ __attribute__((aligned(16))) float xs[3][MT * MROW];
  __shared__ __attribute__((aligned(16))) float ws[3][ME * MROW];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = blockIdx.x * MT, e0 = blockIdx.y * ME;
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int e = tid; e < E; e += 256) counts[e] = 0;  // zeroed before the select kernel

  // loader: row tid/4 of the tile, h (tid%4)*16 .. +15 of the chunk (rows past T or E
  // repeat the last one and are never stored)
  const int lr = tid >> 2, lh = (tid & 3) * 16;
  const XT* xp = x + (int64_t)min(t0 + lr, T - 1) * H + lh;
  const float* wp = w + (int64_t)min(e0 + lr, E - 1) * H + lh;
  constexpr int XV = sizeof(XT) * 16 / 16;  // 16-byte loads of the x segment
  constexpr int NW = XV * (sizeof(XT) == 2 ? 2 : 1) + 4;  // LDS writes per chunk
  u32x4 xr[2][XV], wr[2][4];
  const int nchunk = H / MH;  // even: H is a multiple of 128
  // past the last chunk: loads re-read the last one, and their LDS writes go to a
  // buffer whose chunk every wave has finished (the reads of it are never used)
  auto gload = [&](int j, int set) {
    j = min(j, nchunk - 1);
#pragma unroll
    for (int i = 0; i < XV; ++i)
      xr[set][i] = *reinterpret_cast<const u32x4*>(xp + j * MH + i * 16 / sizeof(XT));
#pragma unroll
    for (int i = 0; i < 4; ++i) wr[set][i] = *reinterpret_cast<const u32x4*>(wp + j * MH + 4 * i);
  };
  // LDS write q (0 .. NW-1) of chunk j from register set `set`
  auto lwrite = [&](int j, int set, int q) {
    const int buf = j % 3;
    if (q < NW - 4) {
      float* dx = &xs[buf][lr * MROW + lh];
      if constexpr (sizeof(XT) == 2) {
        const u32x4 u = xr[set][q >> 1];
        const int o = 2 * (q & 1);
        f32x4 f;
        f[0] = __uint_as_float(u[o] << 16);
        f[1] = __uint_as_float(u[o] & 0xFFFF0000u);
        f[2] = __uint_as_float(u[o + 1] << 16);
        f[3] = __uint_as_float(u[o + 1] & 0xFFFF0000u);
        *reinterpret_cast<f32x4*>(dx + 4 * q) = f;
      } else {
        *reinterpret_cast<u32x4*>(dx + 4 * q) = xr[set][q];
      }
    } else {
      const int i = q - (NW - 4);
      *reinterpret_cast<u32x4*>(&ws[buf][lr * MROW + lh + 4 * i]) = wr[set][i];
    }
  };

  const int ta = 32 * (wv & 1) + (lane & 31);
  const int eb = 32 * (wv >> 1) + 16 * (lane >> 5) + (lane & 15);
  // operand reads of group g (4 h) of chunk j
  auto aread = [&](int j, int g) {
    return *reinterpret_cast<const f32x4*>(&xs[j % 3][ta * MROW + 4 * g]);
  };
  auto bread = [&](int j, int g) {
    return *reinterpret_cast<const f32x4*>(&ws[j % 3][eb * MROW + 4 * g]);
  };
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

  // chunks 0 and 1 in LDS, chunk 2 in registers, operand reads of groups 0, 1 issued
  gload(0, 0);
  gload(1, 1);
#pragma unroll
  for (int q = 0; q < NW; ++q) lwrite(0, 0, q);
#pragma unroll
  for (int q = 0; q < NW; ++q) lwrite(1, 1, q);
  gload(2, 0);
  __syncthreads();
  f32x4 a[4], b[4];
  a[0] = aread(0, 0);
  b[0] = bread(0, 0);
  a[1] = aread(0, 1);
  b[1] = bread(0, 1);

  // chunk c: loads of chunk c+3 into set (c+1)%2, writes of chunk c+2 from set c%2
  auto chunk = [&](int c, int lset, int wset) {
    gload(c + 3, lset);
#pragma unroll
    for (int g = 0; g < MG; ++g) {
      acc = __builtin_amdgcn_mfma_f32_16x16x1f32(a[g % 4][0], b[g % 4][0], acc, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      const int gn = g + 2;
      a[gn % 4] = gn < MG ? aread(c, gn) : aread(c + 1, gn - MG);
      b[gn % 4] = gn < MG ? bread(c, gn) : bread(c + 1, gn - MG);
      if (g < NW) lwrite(c + 2, wset, g);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 1; k < 4; ++k)
        acc = __builtin_amdgcn_mfma_f32_16x16x1f32(a[g % 4][k], b[g % 4][k], acc, 0, 0, 0);
    }
    __syncthreads();
  };
  for (int c = 0; c < nchunk; c += 2) {
    chunk(c, 1, 0);
    chunk(c + 1, 0, 1);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int bk = r >> 2;
    const int t = t0 + 32 * (wv & 1) + 16 * (bk & 1) + 4 * (lane >> 4) + (r & 3);
    const int e = e0 + 32 * (wv >> 1) + 16 * (bk >> 1) + (lane & 15);
    if (t < T && e < E) z[(int64_t)t * E + e] = acc[r];
  }
}

// (value, index) ordering: larger value first, then the lower index.
__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// ---------------------------------------------------------------------------
// Selection for the shapes the group-per-lane kernel below does not take (one group,
// G not a power of two, E/G not a multiple of 4 or above 32): one wave per token,
// 4 tokens per workgroup.  Lane l holds experts
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

// ---------------------------------------------------------------------------
// Selection with one lane per expert group (G a power of two from 2 to 64, E/G a
// multiple of 4 and at most 32): a token takes G adjacent lanes, 64/G tokens per wave.
// Lane g of a token reads its group's E/G logits (one contiguous run) and, in
// ascending expert order, forms each key and keeps the group's best kList keys as a
// list in rank order.  A new key is placed behind every entry with a key >= its own
// (equal keys in the list have lower indices, which rank first), so the list equals
// the group's keys ordered by (key desc, index asc), and its first J entries give the
// group score summed from 0 as above.  A group's rank among the token's groups comes
// from the other lanes' scores by in-segment shuffles; the K rounds then take the
// largest (key, index) over the heads of the kept lanes' lists with a butterfly of DPP
// moves inside the segment, and the winner's lane drops its head.  Round r is kept by lane
// r mod G, which re-reads z of its chosen expert for the unbiased affinity; the gate
// denominator adds the K affinities in rank order.  The one-wave-per-token kernel
// issued a whole wave's instructions for each token and was bound by that issue; here
// a wave serves 64/G tokens (V3 shape, T = 262,144: 0.26 instead of 0.74 ms; T = 4096:
// 19 instead of 33 us; same bits).
// ---------------------------------------------------------------------------
constexpr int kLaneMaxGs = 32, kLaneWg = 128;

// DPP lane moves (gfx9 dpp_ctrl codes): quad_perm [1,0,3,2] and [2,3,0,1] (partner at
// distance 1 and 2 inside a quad), row_half_mirror (lane i of an 8-lane half-row takes
// lane 7-i) and row_mirror (lane i of a 16-lane row takes lane 15-i)
constexpr int kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E, kDppHalfMirror = 0x141,
              kDppMirror = 0x140;
template <int kCtrl>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xF, 0xF, false);
}
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(dpp_i<kCtrl>(__float_as_int(v)));
}

template <int kJ, int kList>
__global__ __launch_bounds__(kLaneWg) void k_router_select_lanes(
    const float* __restrict__ z, const float* __restrict__ bias, int32_t* __restrict__ idx,
    float* __restrict__ gate, int32_t* __restrict__ counts, int T, int E, int G, int M,
    int K) {
  constexpr int kSlots = 8;  // rounds kept per lane: K <= 16, G >= 2
  __shared__ int s_cnt[kMaxE];
  const int L = G, gs = E / G;
  const int q = threadIdx.x & (L - 1);
  const int tpw = kLaneWg / L;  // tokens per workgroup pass
  const int e0 = q * gs;
  for (int e = threadIdx.x; e < E; e += kLaneWg) s_cnt[e] = 0;
  // the group's biases: the same for every token this lane takes
  // (the scan below has no branches: slots past the group re-read its last chunk and
  // carry a bias of -inf, so their keys are -inf and never enter the list)
  float b[kLaneMaxGs];
#pragma unroll
  for (int c = 0; c < kLaneMaxGs / 4; ++c) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(bias + e0 + min(4 * c, gs - 4));
#pragma unroll
    for (int i = 0; i < 4; ++i) b[4 * c + i] = 4 * c + i < gs ? v[i] : -__builtin_inff();
  }
  __syncthreads();
  for (int64_t base = (int64_t)blockIdx.x * tpw; base < T; base += (int64_t)gridDim.x * tpw) {
    const int64_t t_raw = base + threadIdx.x / L;
    const bool live = t_raw < T;
    const int64_t t = live ? t_raw : T - 1;
    const float* zr = z + t * E;
    float zv[kLaneMaxGs];
#pragma unroll
    for (int c = 0; c < kLaneMaxGs / 4; ++c) {
      // (cached loads: the lanes that keep the K rounds re-read z of their chosen experts
      // below; streamed past the L2, those re-reads fetched 1.7x the logits' bytes)
      const f32x4 v = *reinterpret_cast<const f32x4*>(zr + e0 + min(4 * c, gs - 4));
      zv[4 * c] = v[0], zv[4 * c + 1] = v[1], zv[4 * c + 2] = v[2], zv[4 * c + 3] = v[3];
    }
    // list entries: key bits in the low half, expert index in the high half, so an
    // entry moves with one select per half under one comparison
    auto entry = [](float v, int e) {
      return (static_cast<uint64_t>(static_cast<uint32_t>(e)) << 32) | __float_as_uint(v);
    };
    auto key_of = [](uint64_t x) { return __uint_as_float(static_cast<uint32_t>(x)); };
    auto idx_of = [](uint64_t x) { return static_cast<int>(x >> 32); };
    uint64_t lst[kList];
#pragma unroll
    for (int p = 0; p < kList; ++p) lst[p] = entry(-__builtin_inff(), 0x7FFFFFFF);
#pragma unroll
    for (int j = 0; j < kLaneMaxGs; ++j) {
      const float v = affinity(zv[j]) + b[j];
      const uint64_t nv = entry(v, e0 + j);
      // selects, not branches: entry p takes v where v ranks first at p alone, the
      // entry above it where v ranks first there too, else keeps its own
      bool c[kList];
#pragma unroll
      for (int p = 0; p < kList; ++p) c[p] = v > key_of(lst[p]);
#pragma unroll
      for (int p = kList - 1; p >= 1; --p) lst[p] = c[p] ? (c[p - 1] ? lst[p - 1] : nv) : lst[p];
      lst[0] = c[0] ? nv : lst[0];
      // one key at a time, its index selects included: hoisting the sigmoids of later
      // keys, or sinking the index selects below the scan, made the compiler keep a
      // flag pair per select in scalar registers (spills)
#pragma unroll
      for (int p = 0; p < kList; ++p) asm volatile("" ::"v"(lst[p]));
      __builtin_amdgcn_sched_barrier(0);
    }
    float sc = 0.0f;
#pragma unroll
    for (int p = 0; p < kJ; ++p) sc = sc + key_of(lst[p]);
    int rank = 0;
    for (int dg = 1; dg < L; ++dg) {
      const int og = (q + dg) & (L - 1);
      const float os = __shfl(sc, og, L);
      rank += ranks_before(os, og, sc, q) ? 1 : 0;
    }
    const bool kept = rank < M;
    int my_e[kSlots];
#pragma unroll
    for (int s = 0; s < kSlots; ++s) my_e[s] = 0;
    for (int r = 0; r < K; ++r) {
      float bv = kept ? key_of(lst[0]) : -__builtin_inff();
      int bi = kept ? idx_of(lst[0]) : 0x7FFFFFFF;
      // the segment's largest (key, index): within 16 lanes by DPP moves (partner in the
      // quad at distance 1 and 2, then the mirrored lane of the 8- and 16-lane row part),
      // beyond that by shuffles; any pairing that covers the segment gives every lane
      // the same maximum of this total order
      auto take = [&](float ov, int oi) {
        if (ranks_before(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      };
      take(dpp_f<kDppQuadXor1>(bv), dpp_i<kDppQuadXor1>(bi));
      if (L >= 4) take(dpp_f<kDppQuadXor2>(bv), dpp_i<kDppQuadXor2>(bi));
      if (L >= 8) take(dpp_f<kDppHalfMirror>(bv), dpp_i<kDppHalfMirror>(bi));
      if (L >= 16) take(dpp_f<kDppMirror>(bv), dpp_i<kDppMirror>(bi));
      for (int off = 16; off < L; off <<= 1) take(__shfl_xor(bv, off, L), __shfl_xor(bi, off, L));
      const bool won = kept && idx_of(lst[0]) == bi;
#pragma unroll
      for (int p = 0; p + 1 < kList; ++p) lst[p] = won ? lst[p + 1] : lst[p];
      lst[kList - 1] = won ? entry(-__builtin_inff(), 0x7FFFFFFF) : lst[kList - 1];
    const int e_r = bi < E ? bi : 0;  // bi < E: K <= M*E/G candidates always exist
#pragma unroll
      for (int s = 0; s < kSlots; ++s) my_e[s] = r == q + s * L ? e_r : my_e[s];
    }
    float my_s[kSlots];
#pragma unroll
    for (int s = 0; s < kSlots; ++s)
      my_s[s] = q + s * L < K ? affinity(zr[my_e[s]]) : 0.0f;
    float sum = 0.0f;
#pragma unroll
    for (int s = 0; s < kSlots; ++s)
      for (int qq = 0; qq < L; ++qq)
        if (qq + s * L < K) sum = sum + __shfl(my_s[s], qq, L);
#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
      const int r = q + s * L;
      if (live && r < K) {
        idx[t * K + r] = my_e[s];
        gate[t * K + r] = my_s[s] / sum;
        atomicAdd(&s_cnt[my_e[s]], 1);
      }
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kLaneWg)
    if (s_cnt[e]) atomicAdd(&counts[e], s_cnt[e]);
}

bool select_by_lanes(const Dims& d) {
  const int gs = d.E / d.G;
  return d.G >= 2 && d.G <= kWave && (d.G & (d.G - 1)) == 0 && gs % 4 == 0 &&
         gs <= kLaneMaxGs && d.K <= 16;
}

hipError_t launch_select(const Dims& d, const float* logits, const float* bias, int32_t* idx,
                         float* gate, int32_t* counts, hipStream_t st) {
  const int T = static_cast<int>(d.T);
  if (select_by_lanes(d)) {
    const int tpw = kLaneWg / d.G;
    const int wg = static_cast<int>(std::min<int64_t>((d.T + tpw - 1) / tpw,
                                                       4 * device_cu_count()));
#define MOE_SELECT_LANES(J_)                                                              \
  case J_:                                                                                \
    if (d.K <= 8)                                                                         \
      hipLaunchKernelGGL((k_router_select_lanes<J_, 8>), dim3(wg), dim3(kLaneWg), 0, st,  \
                         logits, bias, idx, gate, counts, T, d.E, d.G, d.M, d.K);         \
    else                                                                                  \
      hipLaunchKernelGGL((k_router_select_lanes<J_, 16>), dim3(wg), dim3(kLaneWg), 0, st, \
                         logits, bias, idx, gate, counts, T, d.E, d.G, d.M, d.K);         \
    break;
    switch (d.J) {
      MOE_SELECT_LANES(1) MOE_SELECT_LANES(2) MOE_SELECT_LANES(3) MOE_SELECT_LANES(4)
      MOE_SELECT_LANES(5) MOE_SELECT_LANES(6) MOE_SELECT_LANES(7) MOE_SELECT_LANES(8)
      default: return hipErrorInvalidValue;
    }
#undef MOE_SELECT_LANES
    return hipGetLastError();
  }
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

}  // namespace

hipError_t launch_route(const Dims& d, const void* x, const float* w_router, const float* bias,
                        int32_t* idx, float* gate, int32_t* counts, float* logits,
                        hipStream_t st) {
  const int T = static_cast<int>(d.T);
  if (T >= kMfmaLogitsMinTokens) {
    const dim3 gm((T + MT - 1) / MT, (d.E + ME - 1) / ME);
    if (d.act == MOE_BF16)
      hipLaunchKernelGGL(k_router_logits_mfma<uint16_t>, gm, dim3(256), 0, st,
                         static_cast<const uint16_t*>(x), w_router, logits, counts, T, d.H, d.E);
    else
      hipLaunchKernelGGL(k_router_logits_mfma<float>, gm, dim3(256), 0, st,
                         static_cast<const float*>(x), w_router, logits, counts, T, d.H, d.E);
  } else {
    const dim3 g1((T + RT - 1) / RT, (d.E + RWV - 1) / RWV);
    if (d.act == MOE_BF16)
      hipLaunchKernelGGL((k_router_logits<uint16_t, 1>), g1, dim3(RWV * kWave), 0, st,
                         static_cast<const uint16_t*>(x), w_router, logits, counts, T, d.H, d.E);
    else
      hipLaunchKernelGGL((k_router_logits<float, 1>), g1, dim3(RWV * kWave), 0, st,
                         static_cast<const float*>(x), w_router, logits, counts, T, d.H, d.E);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_select(d, logits, bias, idx, gate, counts, st);
}

}  // namespace moe
