// Backward of the layer, apart from the expert GEMMs (gemm_bwd.hip): the derivative of
// the forward.  The pages fix only that the routing bias takes no part in
// back-propagation (blog.resmic.cn, "DeepSeek-V3架构深度解析", section 核心架构三) and
// that gradients accumulate at high precision (joto.ai item 3: FP32 accumulation), so
// every reduction here is in fp32 and the routing bias does not appear.
//
//   combine:  y[t] = Y[T*K+t] + sum_k g[t,k] Y[row(t,k)]
//             -> dY[row(t,k)] = g[t,k] dy[t], dY[T*K+t] = dy[t], dg[t,k] = <dy[t], Y[row]>
//   gates:    g_k = s_k / S, S = sum of the chosen s (mpbf.cn section 2.2: the selected
//             scores are renormalised), s = sigmoid(clamp(z, +-80))
//             -> ds_j = (dg_j - sum_k g_k dg_k) / S, dz_j = ds_j s_j (1 - s_j), 0 when
//                |z| > 80 (the clamp is flat there)
//   router:   z = x W_r^T -> dx_r[t] = sum_j dz_j W_r[e_j], dW_r[e] = sum over the rows
//             of expert e of dz x[token]
//   input:    dx[t] = dx_r[t] + sum_k dx_sorted[row(t,k)] + dx_sorted[T*K+t]
#include "common.h"

namespace moe {
namespace {

constexpr int kMaxK = 16;

__device__ __forceinline__ void load8(const uint16_t* p, float* v) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float* v) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void store8(uint16_t* p, const float* v) {
  uint4 o;
  o.x = f32_to_bf16_bits(v[0]) | (uint32_t)f32_to_bf16_bits(v[1]) << 16;
  o.y = f32_to_bf16_bits(v[2]) | (uint32_t)f32_to_bf16_bits(v[3]) << 16;
  o.z = f32_to_bf16_bits(v[4]) | (uint32_t)f32_to_bf16_bits(v[5]) << 16;
  o.w = f32_to_bf16_bits(v[6]) | (uint32_t)f32_to_bf16_bits(v[7]) << 16;
  *reinterpret_cast<uint4*>(p) = o;
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// Combine backward: one workgroup per token; thread c owns 8-element chunks c, c+256, ...
template <typename T>
__global__ __launch_bounds__(256) void k_combine_bwd(const T* __restrict__ dy,
                                                     const T* __restrict__ ys,
                                                     const int32_t* __restrict__ inv_perm,
                                                     const float* __restrict__ gate,
                                                     T* __restrict__ dys, float* __restrict__ dgate,
                                                     int Tn, int H, int K, int S) {
  __shared__ float red[4][kMaxK];
  const int t = blockIdx.x, tid = threadIdx.x;
  int rows[kMaxK];
  float g[kMaxK], dot[kMaxK];
#pragma unroll
  for (int k = 0; k < kMaxK; ++k) {
    rows[k] = k < K ? inv_perm[(int64_t)t * K + k] : -1;
    g[k] = k < K ? gate[(int64_t)t * K + k] : 0.0f;
    dot[k] = 0.0f;
  }
  for (int c = tid * 8; c < H; c += 256 * 8) {
    float d[8];
    load8(dy + (int64_t)t * H + c, d);
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
      if (rows[k] < 0) continue;
      float v[8], o[8];
      load8(ys + (int64_t)rows[k] * H + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        dot[k] = __builtin_fmaf(d[i], v[i], dot[k]);
        o[i] = g[k] * d[i];
      }
      store8(dys + (int64_t)rows[k] * H + c, o);
    }
    if (S) store8(dys + ((int64_t)Tn * K + t) * H + c, d);
  }
  const int lane = tid & 63, wv = tid >> 6;
#pragma unroll
  for (int k = 0; k < kMaxK; ++k) {
    float v = dot[k];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0) red[wv][k] = v;
  }
  __syncthreads();
  if (tid < K)
    dgate[(int64_t)t * K + tid] =
        rows[tid] < 0 ? 0.0f : (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
}

// Gate + router-input backward: one wave per token (4 per workgroup).  Lane k < K
// forms dz for its choice; then the wave walks the hidden dimension for dx_r.
__global__ __launch_bounds__(256) void k_router_bwd(
    const float* __restrict__ w, const float* __restrict__ z, const int32_t* __restrict__ idx,
    const float* __restrict__ gate, const float* __restrict__ dgate, float* __restrict__ dz,
    float* __restrict__ dxr, int T, int H, int E, int K) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float s = 0.0f, gdg = 0.0f;
  int e = 0;
  float zz = 0.0f;
  if (lane < K) {
    e = idx[(int64_t)t * K + lane];
    zz = z[(int64_t)t * E + e];
    s = affinity(zz);
    gdg = gate[(int64_t)t * K + lane] * dgate[(int64_t)t * K + lane];
  }
  float S = s, GD = gdg;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    S += __shfl_xor(S, off);
    GD += __shfl_xor(GD, off);
  }
  float d = 0.0f;
  if (lane < K) {
    const float ds = (dgate[(int64_t)t * K + lane] - GD) / S;
    d = (zz > 80.0f || zz < -80.0f) ? 0.0f : ds * s * (1.0f - s);
    dz[(int64_t)t * K + lane] = d;
  }
  float dk[kMaxK];
  int ek[kMaxK];
#pragma unroll
  for (int k = 0; k < kMaxK; ++k) {
    dk[k] = __shfl(d, k);
    ek[k] = __shfl(e, k);
  }
  for (int h = lane * 4; h < H; h += 256) {
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
      if (k >= K) break;
      const float4 wv = *reinterpret_cast<const float4*>(w + (int64_t)ek[k] * H + h);
      acc[0] = __builtin_fmaf(dk[k], wv.x, acc[0]);
      acc[1] = __builtin_fmaf(dk[k], wv.y, acc[1]);
      acc[2] = __builtin_fmaf(dk[k], wv.z, acc[2]);
      acc[3] = __builtin_fmaf(dk[k], wv.w, acc[3]);
    }
    *reinterpret_cast<float4*>(dxr + (int64_t)t * H + h) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  }
}

// Router weight gradient: workgroup (expert e, 2048-wide column slice); thread c owns
// 8 columns and walks the expert's rows in order (tokens ascending), so the sum order
// is fixed.
template <typename T>
__global__ __launch_bounds__(256) void k_router_wgrad(const T* __restrict__ x,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ sorted_token,
                                                      const int32_t* __restrict__ idx,
                                                      const float* __restrict__ dz,
                                                      float* __restrict__ dw, int H, int K) {
  const int e = blockIdx.x;
  const int c = (blockIdx.y * 256 + threadIdx.x) * 8;
  if (c >= H) return;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  const int r0 = offsets[e], r1 = offsets[e + 1];
  for (int r = r0; r < r1; ++r) {
    const int t = sorted_token[r];
    float d = 0.0f;
    for (int k = 0; k < K; ++k)
      if (idx[(int64_t)t * K + k] == e) d = dz[(int64_t)t * K + k];
    float v[8];
    load8(x + (int64_t)t * H + c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(d, v[i], acc[i]);
  }
  store8(dw + (int64_t)e * H + c, acc);
}

// Input gradient: one workgroup of 128 threads per (token, 1024-column slice), in a
// linear token-major grid (the slices of one token are neighbours, so the pieces of each
// row are read together; the grid strides over (token, slice) items).  dx = the
// router's part + the token's rows in rank order.
template <typename T>
__global__ __launch_bounds__(128) void k_unpermute_sum(const T* __restrict__ dxs,
                                                       const int32_t* __restrict__ inv_perm,
                                                       const float* __restrict__ dxr,
                                                       T* __restrict__ dx, int Tn, int H, int K,
                                                       int S) {
  const int nblk = (H / 8 + 127) / 128;
  const int64_t work = (int64_t)Tn * nblk;
  for (int64_t b = blockIdx.x; b < work; b += gridDim.x) {
    const int t = (int)(b / nblk);
    const int c = ((int)(b % nblk) * 128 + threadIdx.x) * 8;
    if (c >= H) continue;
    float acc[8];
    if (dxr) {
      load8(dxr + (int64_t)t * H + c, acc);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    }
    for (int k = 0; k < K; ++k) {
      const int row = inv_perm[(int64_t)t * K + k];
      if (row < 0) continue;
      float v[8];
      load8(dxs + (int64_t)row * H + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    if (S) {
      float v[8];
      load8(dxs + ((int64_t)Tn * K + t) * H + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    store8(dx + (int64_t)t * H + c, acc);
  }
}

}  // namespace

hipError_t launch_combine_bwd(const Dims& d, const void* dy, const void* ys,
                              const int32_t* inv_perm, const float* gate, void* dys, float* dgate,
                              hipStream_t st) {
  const int T = static_cast<int>(d.T);
  if (d.act == MOE_BF16)
    hipLaunchKernelGGL(k_combine_bwd<uint16_t>, dim3(T), dim3(256), 0, st,
                       static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(ys),
                       inv_perm, gate, static_cast<uint16_t*>(dys), dgate, T, d.H, d.K, d.S);
  else
    hipLaunchKernelGGL(k_combine_bwd<float>, dim3(T), dim3(256), 0, st,
                       static_cast<const float*>(dy), static_cast<const float*>(ys), inv_perm,
                       gate, static_cast<float*>(dys), dgate, T, d.H, d.K, d.S);
  return hipGetLastError();
}

hipError_t launch_router_bwd(const Dims& d, const void* x, const float* w, const float* z,
                             const int32_t* idx, const float* gate, const float* dgate,
                             const int32_t* offsets, const int32_t* sorted_token, float* dz,
                             float* dxr, float* dw, hipStream_t st) {
  const int T = static_cast<int>(d.T);
  hipLaunchKernelGGL(k_router_bwd, dim3((T + 3) / 4), dim3(256), 0, st, w, z, idx, gate, dgate,
                     dz, dxr, T, d.H, d.E, d.K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 g(d.E, (d.H + 2047) / 2048);
  if (d.act == MOE_BF16)
    hipLaunchKernelGGL(k_router_wgrad<uint16_t>, g, dim3(256), 0, st,
                       static_cast<const uint16_t*>(x), offsets, sorted_token, idx, dz, dw, d.H,
                       d.K);
  else
    hipLaunchKernelGGL(k_router_wgrad<float>, g, dim3(256), 0, st, static_cast<const float*>(x),
                       offsets, sorted_token, idx, dz, dw, d.H, d.K);
  return hipGetLastError();
}

hipError_t launch_unpermute_sum(const Dims& d, const void* dxs, const int32_t* inv_perm,
                                const float* dxr, void* dx, hipStream_t st) {
  const int T = static_cast<int>(d.T);
  const dim3 g((unsigned)std::min<int64_t>((int64_t)T * ((d.H / 8 + 127) / 128), 1 << 20));
  if (d.act == MOE_BF16)
    hipLaunchKernelGGL(k_unpermute_sum<uint16_t>, g, dim3(128), 0, st,
                       static_cast<const uint16_t*>(dxs), inv_perm, dxr,
                       static_cast<uint16_t*>(dx), T, d.H, d.K, d.S);
  else
    hipLaunchKernelGGL(k_unpermute_sum<float>, g, dim3(128), 0, st,
                       static_cast<const float*>(dxs), inv_perm, dxr, static_cast<float*>(dx),
                       T, d.H, d.K, d.S);
  return hipGetLastError();
}

}  // namespace moe
