// Combine, bias update and the offline FP8 weight quantiser.
//
// Combine (blog.resmic.cn, "DeepSeek-V3架构深度解析", section 核心架构二: the layer
// output is the shared expert's output plus the gate-weighted routed outputs):
//   acc = 0; for k in rank order: acc = fma(gate[t,k], Y[inv_perm[t,k]], acc);
//   acc = Y[T*K + t] + acc (shared expert); y[t] = acc rounded to the output dtype.
// Bias update (mpbf.cn DeepSeek-V3 report summary, sections 2.2 and 6.2): compare
// each expert's batch load with the uniform share, exactly in integers, and move its
// bias by gamma against the imbalance.
// Weight quantiser (same summary, section 4.3: scaling per block, not one global
// scale): one E4M3 scale per 128x128 block, scale = amax/448.
#include "common.h"

namespace moe {
namespace {

constexpr int kMaxK = 16;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld_nt(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_nt(void* p, const uint4& o) {
  const u32x4 v = {o.x, o.y, o.z, o.w};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

template <typename T>
__device__ __forceinline__ void widen(const uint4& u, float* v) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y);
    v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
  }
}

// One workgroup of 128 threads per (token, 128 chunks of 16 bytes); each thread owns 16
// bytes of the row.  All K+1 rows are loaded before the first multiply-add (the loads are
// independent, so they are all in flight together), then summed in rank order.  Y is
// read once and y is not read again here: both go non-temporal.  The grid is linear and
// token-major (the workgroups of one token are neighbours), so the pieces of each 14 KB
// row are read at about the same time: DRAM pages are opened once per row, not once per
// piece (0.110 -> 0.095 ms at the V3 shape).  The grid strides over (token, slice) items.
template <typename T>
__global__ __launch_bounds__(128) void k_combine(const T* __restrict__ ys,
                                                 const int32_t* __restrict__ inv_perm,
                                                 const float* __restrict__ gate, T* __restrict__ y,
                                                 int Tn, int H, int K, int S) {
  constexpr int V = 16 / sizeof(T);
  const int nblk = (H / V + 127) / 128;
  const int64_t work = (int64_t)Tn * nblk;
  for (int64_t b = blockIdx.x; b < work; b += gridDim.x) {
    const int t = (int)(b / nblk);
    const int c = (int)(b % nblk) * 128 + threadIdx.x;
    if (c * V >= H) continue;
    uint4 u[kMaxK];
    int row[kMaxK];
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
      row[k] = k < K ? inv_perm[(int64_t)t * K + k] : -1;
      if (row[k] >= 0)
        u[k] = ld_nt(ys + (int64_t)row[k] * H + c * V);
    }
    uint4 us = make_uint4(0, 0, 0, 0);
    if (S) us = ld_nt(ys + ((int64_t)Tn * K + t) * H + c * V);
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
      if (row[k] < 0) continue;
      const float g = gate[(int64_t)t * K + k];
      float v[V];
      widen<T>(u[k], v);
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] = __builtin_fmaf(g, v[i], acc[i]);
    }
    if (S) {
      float v[V];
      widen<T>(us, v);
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] = v[i] + acc[i];
    }
    uint4 o;
    if constexpr (sizeof(T) == 2) {
      o.x = f32_to_bf16_bits(acc[0]) | (uint32_t)f32_to_bf16_bits(acc[1]) << 16;
      o.y = f32_to_bf16_bits(acc[2]) | (uint32_t)f32_to_bf16_bits(acc[3]) << 16;
      o.z = f32_to_bf16_bits(acc[4]) | (uint32_t)f32_to_bf16_bits(acc[5]) << 16;
      o.w = f32_to_bf16_bits(acc[6]) | (uint32_t)f32_to_bf16_bits(acc[7]) << 16;
    } else {
      o.x = __float_as_uint(acc[0]);
      o.y = __float_as_uint(acc[1]);
      o.z = __float_as_uint(acc[2]);
      o.w = __float_as_uint(acc[3]);
    }
    st_nt(y + (int64_t)t * H + c * V, o);
  }
}

__global__ void k_bias_update(const int32_t* __restrict__ counts, float* __restrict__ bias,
                              float gamma, int E, int64_t target) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const int64_t load = (int64_t)counts[e] * E;
  if (load > target) bias[e] = bias[e] - gamma;
  else if (load < target) bias[e] = bias[e] + gamma;
}

// One workgroup per 128x128 block; thread i owns row i/2, columns (i%2)*64 .. +63.
__global__ __launch_bounds__(256) void k_quant_weight(const uint16_t* __restrict__ w,
                                                      uint8_t* __restrict__ q,
                                                      float* __restrict__ scale, int rows, int cols) {
  __shared__ float red[4];
  const int nbc = cols / 128, nbr = rows / 128;
  const int64_t mat = blockIdx.x / (nbr * nbc);
  const int blk = blockIdx.x % (nbr * nbc);
  const int br = blk / nbc, bc = blk % nbc;
  const int r = br * 128 + (threadIdx.x >> 1);
  const int c0 = bc * 128 + (threadIdx.x & 1) * 64;
  const uint16_t* src = w + (mat * rows + r) * (int64_t)cols + c0;
  float v[64];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 u = reinterpret_cast<const uint4*>(src)[i];
    const uint32_t ww[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = __uint_as_float(ww[j] << 16);
      v[8 * i + 2 * j + 1] = __uint_as_float(ww[j] & 0xFFFF0000u);
    }
  }
#pragma unroll
  for (int i = 0; i < 64; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
  const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
  if (threadIdx.x == 0) scale[mat * nbr * nbc + blk] = sc;
  uint4* dst = reinterpret_cast<uint4*>(q + (mat * rows + r) * (int64_t)cols + c0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint4 o;
    o.x = pack4_e4m3(v[16 * i + 0] / sc, v[16 * i + 1] / sc, v[16 * i + 2] / sc, v[16 * i + 3] / sc);
    o.y = pack4_e4m3(v[16 * i + 4] / sc, v[16 * i + 5] / sc, v[16 * i + 6] / sc, v[16 * i + 7] / sc);
    o.z = pack4_e4m3(v[16 * i + 8] / sc, v[16 * i + 9] / sc, v[16 * i + 10] / sc, v[16 * i + 11] / sc);
    o.w = pack4_e4m3(v[16 * i + 12] / sc, v[16 * i + 13] / sc, v[16 * i + 14] / sc, v[16 * i + 15] / sc);
    dst[i] = o;
  }
}

}  // namespace

hipError_t launch_combine(const Dims& d, const void* ys, const int32_t* inv_perm,
                          const float* gate, void* y, hipStream_t st) {
  const int T = static_cast<int>(d.T);
  if (d.act == MOE_BF16) {
    dim3 grid((unsigned)std::min<int64_t>((int64_t)T * ((d.H / 8 + 127) / 128), 1 << 20));
    hipLaunchKernelGGL(k_combine<uint16_t>, grid, dim3(128), 0, st,
                       static_cast<const uint16_t*>(ys), inv_perm, gate,
                       static_cast<uint16_t*>(y), T, d.H, d.K, d.S);
  } else {
    dim3 grid((unsigned)std::min<int64_t>((int64_t)T * ((d.H / 4 + 127) / 128), 1 << 20));
    hipLaunchKernelGGL(k_combine<float>, grid, dim3(128), 0, st, static_cast<const float*>(ys),
                       inv_perm, gate, static_cast<float*>(y), T, d.H, d.K, d.S);
  }
  return hipGetLastError();
}

hipError_t launch_bias_update(const Dims& d, const int32_t* counts, float gamma, float* bias,
                              hipStream_t st) {
  hipLaunchKernelGGL(k_bias_update, dim3((d.E + 255) / 256), dim3(256), 0, st, counts, bias,
                     gamma, d.E, d.T * (int64_t)d.K);
  return hipGetLastError();
}

hipError_t launch_quantize_weights(const uint16_t* w, uint8_t* q, float* scale, int64_t batch,
                                   int rows, int cols, hipStream_t st) {
  const int64_t nblk = batch * (rows / 128) * (cols / 128);
  hipLaunchKernelGGL(k_quant_weight, dim3((unsigned)nblk), dim3(256), 0, st, w, q, scale, rows,
                     cols);
  return hipGetLastError();
}

}  // namespace moe
