// Expert FFNs as grouped GEMMs over the permuted rows (one group per routed expert,
// plus the shared expert as the last group):
//   GEMM1 + SwiGLU:  h = silu(x W13[g][0:I]^T) * (x W13[g][I:2I]^T)
//   GEMM2:           Y = h W2[g]^T
// Each expert's weights stream from HBM once per (row tile); the tile schedule is
// built on the device from the permute offsets, so no host synchronisation happens.
//
// Schedule: group g has mt_g = ceil(m_g / BM) row tiles; mt_start is their prefix
// sum.  A GEMM with nt column tiles has mt_start[NG]*nt tiles, ordered (group,
// column tile, row tile) so the row tiles that share one weight tile run side by
// side.  The grid is persistent (a fixed number of workgroups per CU) and XCD-aware:
// workgroup w runs on XCD w%8 (dispatch is round-robin over the 8 XCDs), and each
// XCD takes one contiguous eighth of the tile list, so the workgroups of one XCD work
// on neighbouring tiles of the same expert and share its rows through their L2.
#include "common.h"

namespace moe {
namespace {

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

// XCD-aware persistent iteration: calls body(tile) for this workgroup's tiles.
template <typename F>
__device__ __forceinline__ void for_each_tile(int ntiles, F&& body) {
  const int P = gridDim.x;
  const int per_xcd = P / kXcds;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int chunk = (ntiles + kXcds - 1) / kXcds;
  const int end = min(ntiles, (xcd + 1) * chunk);
  for (int tile = xcd * chunk + slot; tile < end; tile += per_xcd) body(tile);
}

__device__ __forceinline__ float silu(float a) { return a / (1.0f + __expf(-a)); }

// ---------------------------------------------------------------------------
// fp32 path: LDS-tiled SIMT GEMM, 64x64 tile, 16-deep k steps, 4x4 per thread.
// kSwiglu: the 64 output columns are 32 gate + the matching 32 up columns.
// ---------------------------------------------------------------------------
template <bool kSwiglu>
__global__ __launch_bounds__(256) void k_gemm_f32(const float* __restrict__ A,
                                                  const float* __restrict__ B, float* __restrict__ C,
                                                  const int32_t* __restrict__ offsets, int NG,
                                                  int Kd, int Nrows, int Nout, int half) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ __attribute__((aligned(16))) float As[BK][BM];
  __shared__ __attribute__((aligned(16))) float Bs[BK][BN];
  __shared__ int mt_start[kMaxGroups + 1];
  build_schedule(offsets, NG, BM, mt_start);
  const int nt = kSwiglu ? half / 32 : Nout / BN;
  const int ntiles = mt_start[NG] * nt;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  for_each_tile(ntiles, [&](int tile) {
    const Tile tl = decode_tile(tile, mt_start, NG, nt);
    const int row0 = offsets[tl.g];
    const int m_g = offsets[tl.g + 1] - row0;
    const int m0 = tl.m_idx * BM;
    // loader: thread -> (row tid/4, k (tid%4)*4)
    const int lr = tid >> 2, lk = (tid & 3) * 4;
    const float* ap = A + (int64_t)(row0 + min(m0 + lr, m_g - 1)) * Kd + lk;
    int brow;
    if (kSwiglu) brow = lr < 32 ? tl.n_idx * 32 + lr : half + tl.n_idx * 32 + (lr - 32);
    else brow = tl.n_idx * BN + lr;
    const float* bp = B + ((int64_t)tl.g * Nrows + brow) * Kd + lk;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < Kd; k0 += BK) {
      const float4 av = *reinterpret_cast<const float4*>(ap + k0);
      const float4 bv = *reinterpret_cast<const float4*>(bp + k0);
      __syncthreads();
      As[lk + 0][lr] = av.x; As[lk + 1][lr] = av.y; As[lk + 2][lr] = av.z; As[lk + 3][lr] = av.w;
      Bs[lk + 0][lr] = bv.x; Bs[lk + 1][lr] = bv.y; Bs[lk + 2][lr] = bv.z; Bs[lk + 3][lr] = bv.w;
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < BK; ++kk) {
        const float4 a4 = *reinterpret_cast<const float4*>(&As[kk][ty * 4]);
        const float a[4] = {a4.x, a4.y, a4.z, a4.w};
        if (kSwiglu) {
          // columns tx*2, tx*2+1 of the gate half and the same of the up half
          const float b[4] = {Bs[kk][tx * 2], Bs[kk][tx * 2 + 1], Bs[kk][32 + tx * 2],
                              Bs[kk][32 + tx * 2 + 1]};
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        } else {
          const float4 b4 = *reinterpret_cast<const float4*>(&Bs[kk][tx * 4]);
          const float b[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + ty * 4 + i;
      if (m >= m_g) continue;
      float* cp = C + (int64_t)(row0 + m) * Nout;
      if (kSwiglu) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
          cp[tl.n_idx * 32 + tx * 2 + j] = silu(acc[i][j]) * acc[i][2 + j];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) cp[tl.n_idx * BN + tx * 4 + j] = acc[i][j];
      }
    }
    __syncthreads();
  });
}

// ---------------------------------------------------------------------------
// bf16 path: MFMA 32x32x16 (bf16 in, fp32 accumulate), 128x128 tile, 64-deep k
// steps double-buffered in LDS with the next step's global loads in flight during
// the current step's MFMAs.  Four waves in a 2x2 arrangement, each 2x2 MFMA tiles.
//   kSwiglu: the tile's 128 weight rows are 64 gate rows and the matching 64 up
//   rows; wave (wm, wn) takes gate rows 32wn.. and up rows 64+32wn.., so each lane
//   holds the gate and up value of the same h element and applies SwiGLU in
//   registers.
// Operand layout (32x32x16): lane l supplies row (l%32), k = 8*(l/32)..+7 of A and
// column (l%32), the same k of B; result element i of lane l is row
// 8*(i/4) + 4*(l/32) + i%4, column l%32.
// ---------------------------------------------------------------------------
constexpr int BM = 128, BN = 128, BK = 64, LDA = BK + 8;

template <bool kSwiglu>
__device__ __forceinline__ void gemm_bf16_tile(const uint16_t* __restrict__ A,
                                               const uint16_t* __restrict__ B,
                                               uint16_t* __restrict__ C, uint16_t* As, uint16_t* Bs,
                                               const Tile& tl, int row0, int m_g, int Kd,
                                               int Nrows, int Nout, int half) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int nk = Kd / BK;
  const int m0 = tl.m_idx * BM;

  // loader: chunk c = tid + 256*i -> row c/8, 8 bf16 at k (c%8)*8
  int64_t aoff[4], boff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    const int r = c >> 3, kc = (c & 7) * 8;
    aoff[i] = (int64_t)(row0 + min(m0 + r, m_g - 1)) * Kd + kc;
    int brow;
    if (kSwiglu) brow = r < 64 ? tl.n_idx * 64 + r : half + tl.n_idx * 64 + (r - 64);
    else brow = tl.n_idx * BN + r;
    boff[i] = ((int64_t)tl.g * Nrows + brow) * Kd + kc;
  }
  const int soff = (tid >> 3) * LDA + (tid & 7) * 8;  // + 32*LDA per i
  uint4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
#define GEMM_GLOAD(k0)                                                  \
  ra0 = *reinterpret_cast<const uint4*>(A + aoff[0] + (k0));            \
  ra1 = *reinterpret_cast<const uint4*>(A + aoff[1] + (k0));            \
  ra2 = *reinterpret_cast<const uint4*>(A + aoff[2] + (k0));            \
  ra3 = *reinterpret_cast<const uint4*>(A + aoff[3] + (k0));            \
  rb0 = *reinterpret_cast<const uint4*>(B + boff[0] + (k0));            \
  rb1 = *reinterpret_cast<const uint4*>(B + boff[1] + (k0));            \
  rb2 = *reinterpret_cast<const uint4*>(B + boff[2] + (k0));            \
  rb3 = *reinterpret_cast<const uint4*>(B + boff[3] + (k0));
#define GEMM_LSTORE(buf)                                                          \
  *reinterpret_cast<uint4*>(As + (buf) * BM * LDA + soff) = ra0;                  \
  *reinterpret_cast<uint4*>(As + (buf) * BM * LDA + soff + 32 * LDA) = ra1;       \
  *reinterpret_cast<uint4*>(As + (buf) * BM * LDA + soff + 64 * LDA) = ra2;       \
  *reinterpret_cast<uint4*>(As + (buf) * BM * LDA + soff + 96 * LDA) = ra3;       \
  *reinterpret_cast<uint4*>(Bs + (buf) * BN * LDA + soff) = rb0;                  \
  *reinterpret_cast<uint4*>(Bs + (buf) * BN * LDA + soff + 32 * LDA) = rb1;       \
  *reinterpret_cast<uint4*>(Bs + (buf) * BN * LDA + soff + 64 * LDA) = rb2;       \
  *reinterpret_cast<uint4*>(Bs + (buf) * BN * LDA + soff + 96 * LDA) = rb3;

  f32x16 acc00, acc01, acc10, acc11;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    acc00[i] = 0.0f; acc01[i] = 0.0f; acc10[i] = 0.0f; acc11[i] = 0.0f;
  }
  const int a_row = 64 * wm + (lane & 31);
  const int b_row0 = kSwiglu ? 32 * wn + (lane & 31) : 64 * wn + (lane & 31);
  const int b_row1 = b_row0 + (kSwiglu ? 64 : 32);
  const int kq = (lane >> 5) * 8;

  GEMM_GLOAD(0)
  GEMM_LSTORE(0)
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) {
      GEMM_GLOAD((kt + 1) * BK)
    }
    const uint16_t* as = As + buf * BM * LDA;
    const uint16_t* bs = Bs + buf * BN * LDA;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(as + a_row * LDA + 16 * s + kq);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(as + (a_row + 32) * LDA + 16 * s + kq);
      const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(bs + b_row0 * LDA + 16 * s + kq);
      const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(bs + b_row1 * LDA + 16 * s + kq);
      acc00 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc00, 0, 0, 0);
      acc01 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc01, 0, 0, 0);
      acc10 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc10, 0, 0, 0);
      acc11 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc11, 0, 0, 0);
    }
    if (kt + 1 < nk) {
      GEMM_LSTORE(buf ^ 1)
    }
    __syncthreads();
  }
#undef GEMM_GLOAD
#undef GEMM_LSTORE

  // epilogue: rows 64wm + 32mi + 8(i/4) + 4(l/32) + i%4, column l%32 of the sub-tile
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    const f32x16& c0 = mi ? acc10 : acc00;
    const f32x16& c1 = mi ? acc11 : acc01;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = m0 + 64 * wm + 32 * mi + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      if (m >= m_g) continue;
      uint16_t* cp = C + (int64_t)(row0 + m) * Nout;
      if (kSwiglu) {
        cp[tl.n_idx * 64 + 32 * wn + (lane & 31)] = f32_to_bf16_bits(silu(c0[i]) * c1[i]);
      } else {
        cp[tl.n_idx * BN + 64 * wn + (lane & 31)] = f32_to_bf16_bits(c0[i]);
        cp[tl.n_idx * BN + 64 * wn + 32 + (lane & 31)] = f32_to_bf16_bits(c1[i]);
      }
    }
  }
}

template <bool kSwiglu>
__global__ __launch_bounds__(256, 2) void k_gemm_bf16(const uint16_t* __restrict__ A,
                                                      const uint16_t* __restrict__ B,
                                                      uint16_t* __restrict__ C,
                                                      const int32_t* __restrict__ offsets,
                                                      int NG, int Kd, int Nrows, int Nout,
                                                      int half) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2 * BM * LDA];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2 * BN * LDA];
  __shared__ int mt_start[kMaxGroups + 1];
  build_schedule(offsets, NG, BM, mt_start);
  const int nt = kSwiglu ? half / 64 : Nout / BN;
  const int ntiles = mt_start[NG] * nt;
  const int P = gridDim.x;
  const int per_xcd = P / kXcds;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int chunk = (ntiles + kXcds - 1) / kXcds;
  const int end = min(ntiles, (xcd + 1) * chunk);
  for (int tile = xcd * chunk + slot; tile < end; tile += per_xcd) {
    const Tile tl = decode_tile(tile, mt_start, NG, nt);
    const int row0 = offsets[tl.g];
    const int m_g = offsets[tl.g + 1] - row0;
    gemm_bf16_tile<kSwiglu>(A, B, C, As, Bs, tl, row0, m_g, Kd, Nrows, Nout, half);
  }
}

}  // namespace

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Workgroups of a persistent launch: occupancy per CU times the CUs, rounded down to
// a multiple of the XCD count so every XCD gets the same number of slots.
static int persistent_grid(int cus, int per_cu) {
  const int p = (cus * per_cu / kXcds) * kXcds;
  return p < kXcds ? kXcds : p;
}

size_t ffn_ws_bytes(const Dims& d) {
  if (d.expert == MOE_FP8_E4M3)
    return align256((size_t)d.R() * d.I) + align256((size_t)d.R() * (d.I / 128) * sizeof(float));
  return align256((size_t)d.R() * d.I * (d.expert == MOE_F32 ? 4 : 2));
}

float* ffn_ws_h_scale(const Dims& d, void* ws) {
  return reinterpret_cast<float*>(static_cast<char*>(ws) + align256((size_t)d.R() * d.I));
}

hipError_t launch_ffn_up(const Dims& d, const void* xs, const float* xs_scale,
                         const int32_t* offsets, const void* w13, const float* w13_scale, void* h,
                         float* h_scale, hipStream_t st) {
  const int NG = d.E + d.S;
  const int cus = device_cu_count();
  if (d.expert == MOE_F32) {
    hipLaunchKernelGGL(k_gemm_f32<true>, dim3(persistent_grid(cus, 4)), dim3(256), 0, st,
                       static_cast<const float*>(xs), static_cast<const float*>(w13),
                       static_cast<float*>(h), offsets, NG, d.H, 2 * d.I, d.I, d.I);
    return hipGetLastError();
  }
  if (d.expert == MOE_BF16) {
    hipLaunchKernelGGL(k_gemm_bf16<true>, dim3(persistent_grid(cus, 2)), dim3(256), 0, st,
                       static_cast<const uint16_t*>(xs), static_cast<const uint16_t*>(w13),
                       static_cast<uint16_t*>(h), offsets, NG, d.H, 2 * d.I, d.I, d.I);
    return hipGetLastError();
  }
  return launch_fp8_up(d, xs, xs_scale, offsets, w13, w13_scale, h, h_scale, st);
}

hipError_t launch_ffn_down(const Dims& d, const void* h, const float* h_scale,
                           const int32_t* offsets, const void* w2, const float* w2_scale, void* ys,
                           hipStream_t st) {
  const int NG = d.E + d.S;
  const int cus = device_cu_count();
  if (d.expert == MOE_F32) {
    hipLaunchKernelGGL(k_gemm_f32<false>, dim3(persistent_grid(cus, 4)), dim3(256), 0, st,
                       static_cast<const float*>(h), static_cast<const float*>(w2),
                       static_cast<float*>(ys), offsets, NG, d.I, d.H, d.H, 0);
    return hipGetLastError();
  }
  if (d.expert == MOE_BF16) {
    hipLaunchKernelGGL(k_gemm_bf16<false>, dim3(persistent_grid(cus, 2)), dim3(256), 0, st,
                       static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(w2),
                       static_cast<uint16_t*>(ys), offsets, NG, d.I, d.H, d.H, 0);
    return hipGetLastError();
  }
  return launch_fp8_down(d, h, h_scale, offsets, w2, w2_scale, ys, st);
}

}  // namespace moe
