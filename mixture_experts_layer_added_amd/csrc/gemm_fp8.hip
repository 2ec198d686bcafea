// FP8 (E4M3) expert FFN: the grouped GEMM pair with tile-wise scaling and
// higher-precision accumulation (DeepSeek-V3 report summary on mpbf.cn, section 3.1:
// scaling factors per small tile and online accumulation for matmul precision;
// section 4.3: block-wise rather than global scales; joto.ai item 3: FP8 inputs and
// weights, FP32 accumulation).
//
// Operands: activations carry one fp32 scale per (row, 128 columns), weights one per
// 128x128 block.  For every 128-deep block of the reduction the MFMA forms the block's
// partial sum of code products in fp32 (two v_mfma_scale_f32_32x32x64_f8f6f4 with
// neutral E8M0 scales: the fp32 scales are not powers of two, so they cannot ride in
// the instruction's scale operands), and the partial is promoted into the fp32
// accumulator as acc += partial * (s_a * s_w).
//
// Tile: 64 rows x BN weight rows, 64-deep k steps double-buffered in LDS, four waves
// side by side along N, each wave 2 (rows) x NSUB (columns) MFMA tiles of 32x32.
//   up   (kSwiglu, NSUB=2): BN = 256 = 128 gate rows + the matching 128 up rows; each
//        wave holds gate and up of the same h element, applies SwiGLU, and the tile's
//        128 h columns are exactly one quantisation tile of h: amax per row across the
//        four waves, scale = amax/448, RNE-saturating E4M3 codes.
//   down (NSUB=1): BN = 128 output columns, bf16 output.
// Operand layout (32x32x64 f8): lane l supplies row l%32 and k = 32*(l/32)..+31 of A,
// column l%32 and the same k of B; result element i of lane l is row
// 8*(i/4) + 4*(l/32) + i%4, column l%32.
#include "common.h"

namespace moe {
namespace {

constexpr int kMaxGroups = 513;
constexpr int kSchedPer = 9;
constexpr int FBM = 64, FBK = 64, FLD = FBK + 16;  // LDS row stride in bytes

__device__ __forceinline__ void fp8_schedule(const int32_t* __restrict__ offsets, int NG, int BM,
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

__device__ __forceinline__ float silu(float a) { return a / (1.0f + __expf(-a)); }

template <bool kSwiglu, int NSUB>
__global__ __launch_bounds__(256, 2) void k_gemm_fp8(
    const uint8_t* __restrict__ A, const float* __restrict__ A_scale,
    const uint8_t* __restrict__ B, const float* __restrict__ B_scale, void* __restrict__ C,
    float* __restrict__ C_scale, const int32_t* __restrict__ offsets, int NG, int Kd, int Nrows,
    int Nout, int half) {
  constexpr int BN = 128 * NSUB;
  constexpr int BCH = BN * FBK / 16 / 256;  // 16-byte B chunks per thread per k step
  __shared__ __attribute__((aligned(16))) uint8_t As[2][FBM * FLD];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BN * FLD];
  __shared__ float s_sa[2][FBM];
  __shared__ float s_red[4][FBM];
  __shared__ int mt_start[kMaxGroups + 1];
  fp8_schedule(offsets, NG, FBM, mt_start);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nt = kSwiglu ? half / 128 : Nout / 128;
  const int ntiles = mt_start[NG] * nt;
  const int nkb = Kd / 128;   // scale blocks along k
  const int nk = Kd / FBK;    // k steps
  const int nbr = Nrows / 128;

  const int P = gridDim.x, per_xcd = P / kXcds;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int chunk = (ntiles + kXcds - 1) / kXcds;
  const int end = min(ntiles, (xcd + 1) * chunk);
  for (int tile = xcd * chunk + slot; tile < end; tile += per_xcd) {
    // decode (group, column tile, row tile)
    int lo = 0, hi = NG;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (mt_start[mid] * nt <= tile) lo = mid;
      else hi = mid;
    }
    const int g = lo;
    const int mt = mt_start[g + 1] - mt_start[g];
    const int local = tile - mt_start[g] * nt;
    const int n_idx = local / mt, m_idx = local % mt;
    const int row0 = offsets[g];
    const int m_g = offsets[g + 1] - row0;
    const int m0 = m_idx * FBM;

    // loaders: A one 16-byte chunk per thread (row tid/4), B BCH chunks
    const int arow = tid >> 2, akc = (tid & 3) * 16;
    const int64_t a_off = (int64_t)(row0 + min(m0 + arow, m_g - 1)) * Kd + akc;
    // B chunk i of this thread: row tid/4 + 64*i, the same 16 bytes of k as A
    auto brow_of = [&](int r) {
      if (kSwiglu) return r < 128 ? n_idx * 128 + r : half + n_idx * 128 + (r - 128);
      return n_idx * 128 + r;
    };
    const int64_t bg = (int64_t)g * Nrows;
    const int64_t b_off0 = (bg + brow_of(arow)) * Kd + akc;
    const int64_t b_off1 = (bg + brow_of(arow + 64)) * Kd + akc;
    const int64_t b_off2 = BCH > 2 ? (bg + brow_of(arow + 128)) * Kd + akc : 0;
    const int64_t b_off3 = BCH > 2 ? (bg + brow_of(arow + 192)) * Kd + akc : 0;
    const int64_t sa_row = (int64_t)(row0 + min(m0 + (tid & 63), m_g - 1)) * nkb;
    // weight-scale block rows of this wave's column tiles
    const int wblk0 = n_idx;                              // gate rows / output columns
    const int wblk1 = kSwiglu ? half / 128 + n_idx : n_idx;  // up rows
    const float* bsc = B_scale + (int64_t)g * nbr * nkb;

    uint4 ra, rb0, rb1, rb2, rb3;
    float rsa = 0.0f;
#define FP8_GLOAD(kt_)                                                                        \
  {                                                                                           \
    ra = *reinterpret_cast<const uint4*>(A + a_off + (kt_) * FBK);                            \
    rb0 = *reinterpret_cast<const uint4*>(B + b_off0 + (kt_) * FBK);                          \
    rb1 = *reinterpret_cast<const uint4*>(B + b_off1 + (kt_) * FBK);                          \
    if (BCH > 2) {                                                                            \
      rb2 = *reinterpret_cast<const uint4*>(B + b_off2 + (kt_) * FBK);                        \
      rb3 = *reinterpret_cast<const uint4*>(B + b_off3 + (kt_) * FBK);                        \
    }                                                                                         \
    if ((((kt_) & 1) == 0) && tid < FBM) rsa = A_scale[sa_row + ((kt_) >> 1)];                \
  }
#define FP8_LSTORE(kt_, buf_)                                                                 \
  {                                                                                           \
    *reinterpret_cast<uint4*>(&As[buf_][arow * FLD + akc]) = ra;                              \
    *reinterpret_cast<uint4*>(&Bs[buf_][(tid >> 2) * FLD + akc]) = rb0;                       \
    *reinterpret_cast<uint4*>(&Bs[buf_][((tid >> 2) + 64) * FLD + akc]) = rb1;                \
    if (BCH > 2) {                                                                            \
      *reinterpret_cast<uint4*>(&Bs[buf_][((tid >> 2) + 128) * FLD + akc]) = rb2;             \
      *reinterpret_cast<uint4*>(&Bs[buf_][((tid >> 2) + 192) * FLD + akc]) = rb3;             \
    }                                                                                         \
    if ((((kt_) & 1) == 0) && tid < FBM) s_sa[((kt_) >> 1) & 1][tid] = rsa;                   \
  }

    f32x16 acc[2][NSUB], tmp[2][NSUB];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int s = 0; s < NSUB; ++s)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mi][s][i] = 0.0f;

    const int kq = (lane >> 5) * 32;
    FP8_GLOAD(0)
    FP8_LSTORE(0, 0)
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nk) FP8_GLOAD(kt + 1)
      i32x8 af[2], bfr[NSUB];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const uint8_t* p = &As[buf][(32 * mi + (lane & 31)) * FLD + kq];
        const uint4 u0 = *reinterpret_cast<const uint4*>(p);
        const uint4 u1 = *reinterpret_cast<const uint4*>(p + 16);
        af[mi][0] = u0.x; af[mi][1] = u0.y; af[mi][2] = u0.z; af[mi][3] = u0.w;
        af[mi][4] = u1.x; af[mi][5] = u1.y; af[mi][6] = u1.z; af[mi][7] = u1.w;
      }
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        const uint8_t* p = &Bs[buf][(32 * wv + 128 * s + (lane & 31)) * FLD + kq];
        const uint4 u0 = *reinterpret_cast<const uint4*>(p);
        const uint4 u1 = *reinterpret_cast<const uint4*>(p + 16);
        bfr[s][0] = u0.x; bfr[s][1] = u0.y; bfr[s][2] = u0.z; bfr[s][3] = u0.w;
        bfr[s][4] = u1.x; bfr[s][5] = u1.y; bfr[s][6] = u1.z; bfr[s][7] = u1.w;
      }
      const bool first_half = (kt & 1) == 0;
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
          if (first_half) {
            f32x16 z;
#pragma unroll
            for (int i = 0; i < 16; ++i) z[i] = 0.0f;
            tmp[mi][s] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[mi], bfr[s], z, 0, 0, 0,
                                                                         127, 0, 127);
          } else {
            tmp[mi][s] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[mi], bfr[s], tmp[mi][s],
                                                                         0, 0, 0, 127, 0, 127);
          }
        }
      if (!first_half) {
        // promote the finished 128-deep block: acc += partial * (s_a[row] * s_w)
        const int kb = kt >> 1;
        float sw[NSUB];
#pragma unroll
        for (int s = 0; s < NSUB; ++s) sw[s] = bsc[(int64_t)(s == 0 ? wblk0 : wblk1) * nkb + kb];
        const float* sa = s_sa[kb & 1];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 a4 = *reinterpret_cast<const float4*>(&sa[32 * mi + 8 * q + 4 * (lane >> 5)]);
            const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int s = 0; s < NSUB; ++s)
                acc[mi][s][4 * q + j] =
                    __builtin_fmaf(tmp[mi][s][4 * q + j], av[j] * sw[s], acc[mi][s][4 * q + j]);
          }
      }
      if (kt + 1 < nk) FP8_LSTORE(kt + 1, buf ^ 1)
      __syncthreads();
    }
#undef FP8_GLOAD
#undef FP8_LSTORE

    if constexpr (kSwiglu) {
      // h = silu(gate) * up; per-row amax over the tile's 128 columns (4 waves x 32)
      float hv[2][16];
      float rmax[2][16];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          hv[mi][i] = silu(acc[mi][0][i]) * acc[mi][1][i];
          float m = __builtin_fabsf(hv[mi][i]);
#pragma unroll
          for (int off = 1; off < 32; off <<= 1) m = __builtin_fmaxf(m, __shfl_xor(m, off));
          rmax[mi][i] = m;
        }
      if ((lane & 31) == 0)
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            s_red[wv][32 * mi + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3)] = rmax[mi][i];
      __syncthreads();
      uint8_t* hq = static_cast<uint8_t*>(C);
      const int ncb = Nout / 128;
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 32 * mi + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
          const float amax = __builtin_fmaxf(__builtin_fmaxf(s_red[0][r], s_red[1][r]),
                                             __builtin_fmaxf(s_red[2][r], s_red[3][r]));
          const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
          const int m = m0 + r;
          if (m < m_g) {
            hq[(int64_t)(row0 + m) * Nout + n_idx * 128 + 32 * wv + (lane & 31)] =
                static_cast<uint8_t>(f32_to_e4m3_bits(hv[mi][i] / sc));
            if (wv == 0 && (lane & 31) == 0) C_scale[(int64_t)(row0 + m) * ncb + n_idx] = sc;
          }
        }
      __syncthreads();  // s_red is reused by the next tile
    } else {
      uint16_t* y = static_cast<uint16_t*>(C);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int m = m0 + 32 * mi + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
          if (m < m_g)
            y[(int64_t)(row0 + m) * Nout + n_idx * 128 + 32 * wv + (lane & 31)] =
                f32_to_bf16_bits(acc[mi][0][i]);
        }
    }
  }
}

int fp8_grid(int cus) {
  const int p = (cus * 2 / kXcds) * kXcds;
  return p < kXcds ? kXcds : p;
}

}  // namespace

hipError_t launch_fp8_up(const Dims& d, const void* xs, const float* xs_scale,
                         const int32_t* offsets, const void* w13, const float* w13_scale, void* h,
                         float* h_scale, hipStream_t st) {
  hipLaunchKernelGGL((k_gemm_fp8<true, 2>), dim3(fp8_grid(device_cu_count())), dim3(256), 0, st,
                     static_cast<const uint8_t*>(xs), xs_scale, static_cast<const uint8_t*>(w13),
                     w13_scale, h, h_scale, offsets, d.E + d.S, d.H, 2 * d.I, d.I, d.I);
  return hipGetLastError();
}

hipError_t launch_fp8_down(const Dims& d, const void* h, const float* h_scale,
                           const int32_t* offsets, const void* w2, const float* w2_scale, void* ys,
                           hipStream_t st) {
  hipLaunchKernelGGL((k_gemm_fp8<false, 1>), dim3(fp8_grid(device_cu_count())), dim3(256), 0, st,
                     static_cast<const uint8_t*>(h), h_scale, static_cast<const uint8_t*>(w2),
                     w2_scale, ys, nullptr, offsets, d.E + d.S, d.I, d.H, d.H, 0);
  return hipGetLastError();
}

}  // namespace moe
