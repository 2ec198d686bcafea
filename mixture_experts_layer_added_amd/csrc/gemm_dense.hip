// The shared expert's gate/up GEMM + SwiGLU as a dense GEMM (bf16 in, fp32 accumulate,
// bf16 out):  h = silu(x Wg^T) * (x Wu^T)  over all T tokens.
//
// Every token passes through the shared expert, so at a few thousand tokens this GEMM
// is dense (T x 2I x H, both operands re-read by many tiles from the L2) and bound by
// the matrix cores rather than by HBM.  Inside the grouped launch, whose ring is shaped
// for streaming routed weights, its full-height tiles get one k step in flight and
// stall on the L2; here it gets a ring shaped for reuse:
//   - 256 x 256 tiles (128 gate columns + the same 128 up columns), 8 waves each
//     owning 64 rows x 128 columns (2 x 4 MFMA 32x32x16), all eight multiplying;
//   - 32-deep k steps (64 bytes per row), four LDS stages of 32 KiB, three in flight
//     while one is multiplied; all fragment reads of a step are issued before its
//     first multiply;
//   - tiles ordered in bands of four row tiles, column-major inside a band, and each
//     XCD (workgroup b runs on XCD b % 8) takes one contiguous range of that order, so
//     the workgroups sharing an L2 share their activation and weight rows.
// The MFMAs of a tile run over k in the same order as in the grouped kernel, so both
// produce the same fp32 sums.  (The shared expert's down GEMM stays in the grouped
// launch: there a dense launch measured no faster.)
#include "common.h"

namespace moe {
namespace {

constexpr int DB = 256;                 // tile rows and columns
constexpr int DK = 32;                  // k per stage
constexpr int kDRow = DK * 2;           // bytes of one row of one stage
constexpr int kDOp = DB * kDRow;        // one operand of one stage: 16 KiB
constexpr int kDStage = 2 * kDOp;       // A then B: 32 KiB
constexpr int kDRing = 4;               // stages
constexpr int kDBand = 4;               // row tiles per band of the tile order
constexpr int kDPerStage = 4;           // DMA loads per thread per stage

// byte offset of (row r, 16-byte k-chunk c) inside an operand stage: rows of 64 B,
// chunk slots xor-swizzled by (r >> 2) & 3, so the 16 rows read at one chunk by a
// group of 16 lanes fall in 16 distinct 16-byte bank groups
__device__ __forceinline__ int dswz(int r, int c) { return r * kDRow + ((c ^ (r >> 2)) & 3) * 16; }

__device__ __forceinline__ float dsilu(float a) { return a / (1.0f + __expf(-a)); }

// The MFMAs of one stage for one wave (2 32-row sub-tiles x 4 32-column sub-tiles):
// every fragment of the stage is read from LDS before the first multiply.
// Operand layout (32x32x16): lane l supplies row l%32, k = 8(l/32) .. +7 of the
// sub-step, for A and for B alike.
__device__ __forceinline__ void stage_mfma(f32x16 (&acc)[2][4], const char* as, const char* bs,
                                           const int (&brow)[4], int arow0, int kq) {
  constexpr int S = DK / 16;
  bf16x8 b[S][4], a[S][2];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int c = 2 * s + kq;
#pragma unroll
    for (int n = 0; n < 4; ++n) b[s][n] = *reinterpret_cast<const bf16x8*>(bs + dswz(brow[n], c));
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
      a[s][mi] = *reinterpret_cast<const bf16x8*>(as + dswz(arow0 + 32 * mi, c));
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the multiplies
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int n = 0; n < 4; ++n)
        acc[mi][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s][mi], b[s][n], acc[mi][n], 0, 0, 0);
}

// A [M, Kd] (token order), B [2*half, Kd] (gate rows, then up rows), h [M, half];
// au [M, 2*half] (optional): the gate and up pre-activations.  Column tile n holds gate
// rows 128n .. +127 of B and the matching up rows half + 128n .. +127.
__global__ __launch_bounds__(512, 1) void k_gemm_dense_swiglu_bf16(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, uint16_t* __restrict__ h,
    uint16_t* __restrict__ au, int M, int Kd, int half, int mt, int nt) {
  __shared__ __attribute__((aligned(1024))) char smem[kDRing * kDStage];
  const int total = mt * nt;
  const int per = (total + kXcds - 1) / kXcds;
  const int tile = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (tile >= total) return;
  // band of kDBand row tiles, column-major inside the band
  const int band = tile / (kDBand * nt), within = tile % (kDBand * nt);
  const int rb = min(kDBand, mt - band * kDBand);
  const int n_idx = within / rb, m_idx = band * kDBand + within % rb;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv >> 1, wn = wv & 1;
  const int nk = Kd / DK;
  const int m0 = m_idx * DB;
  const int m_rows = min(DB, M - m0);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_offset(smem));

  // loader: instruction j of wave wv fills rows 32wv + 16j .. +15 of an operand stage;
  // lane l writes row 32wv + 16j + (l >> 2), slot l & 3, which holds k-chunk
  // (l & 3) ^ ((row >> 2) & 3) = (l & 3) ^ ((l >> 4) & 3)
  const int lchunk = (lane & 3) ^ ((lane >> 4) & 3);
  // A rows past M read as zeros (range check)
  const i32x4 arsrc = buffer_rsrc(A + (int64_t)m0 * Kd, (uint32_t)m_rows * Kd * 2);
  const i32x4 brsrc = buffer_rsrc(B, (uint32_t)(2 * half) * Kd * 2);
  uint32_t aoff[2], boff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 32 * wv + 16 * j + (lane >> 2);
    aoff[j] = (uint32_t)(r * Kd + lchunk * 8) * 2;
    const int br = r < 128 ? n_idx * 128 + r : half + n_idx * 128 + (r - 128);
    boff[j] = (uint32_t)(br * Kd + lchunk * 8) * 2;
  }
  const uint32_t ldsw = lds0 + 32 * wv * kDRow;

#define DSTAGE_LOAD(kt, st)                                          \
  {                                                                  \
    const uint32_t sa_ = ldsw + (st) * kDStage;                      \
    const uint32_t ko_ = (uint32_t)(kt) * kDRow;                     \
    load16_to_lds(arsrc, sa_, aoff[0] + ko_);                        \
    load16_to_lds(arsrc, sa_ + 16 * kDRow, aoff[1] + ko_);           \
    load16_to_lds(brsrc, sa_ + kDOp, boff[0] + ko_);                 \
    load16_to_lds(brsrc, sa_ + kDOp + 16 * kDRow, boff[1] + ko_);    \
  }

  f32x16 acc[2][4];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mi][n][i] = 0.0f;
  // sub-tile n of wave column wn: gate (n even) or up (n odd) columns 64wn + 32(n/2) ..
  int brow[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) brow[n] = (n & 1) * 128 + 64 * wn + 32 * (n >> 1) + (lane & 31);
  const int arow0 = 64 * wm + (lane & 31);
  const int kq = lane >> 5;

#pragma unroll
  for (int s = 0; s < kDRing - 1; ++s)
    if (s < nk) DSTAGE_LOAD(s, s)
  int st = 0;
  for (int kt = 0; kt < nk; ++kt) {
    // stages issued beyond kt: min(kDRing - 2, nk - 1 - kt)
    wait_vmcnt(min(kDRing - 2, nk - 1 - kt) * kDPerStage);
    __syncthreads();
    if (kt + kDRing - 1 < nk) {
      int sn = st + kDRing - 1;
      if (sn >= kDRing) sn -= kDRing;
      DSTAGE_LOAD(kt + kDRing - 1, sn)
    }
    // every wave multiplies (rows past M hold zeros and are not stored), so the loop
    // body is one straight-line block
    const char* as = smem + st * kDStage;
    stage_mfma(acc, as, as + kDOp, brow, arow0, kq);
    if (++st == kDRing) st = 0;
  }
#undef DSTAGE_LOAD

  if (64 * wm >= m_rows) return;
  // result element i of lane l: row 8(i/4) + 4(l/32) + i%4, column l%32 of its 32x32 tile
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = 64 * wm + 32 * mi + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      if (m >= m_rows) continue;
      uint16_t* hp = h + (int64_t)(m0 + m) * half;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int col = n_idx * 128 + 64 * wn + 32 * t + (lane & 31);
        __builtin_nontemporal_store(
            f32_to_bf16_bits(dsilu(acc[mi][2 * t][i]) * acc[mi][2 * t + 1][i]), hp + col);
        if (au) {  // gate and up pre-activations, kept for the backward
          uint16_t* ap = au + (int64_t)(m0 + m) * 2 * half;
          ap[col] = f32_to_bf16_bits(acc[mi][2 * t][i]);
          ap[half + col] = f32_to_bf16_bits(acc[mi][2 * t + 1][i]);
        }
      }
    }
}

}  // namespace

bool dense_shared(const Dims& d) {
  // one workgroup per tile (tiles of at least 128 rows x 128 h columns): beyond 2^22
  // tiles the dispatch would exceed 2^31 work-items, and the grouped launch (persistent)
  // keeps the shared expert instead
  const int64_t max_tiles = ((d.T + 127) / 128) * (int64_t)(d.I / 128);
  return d.S == 1 && (d.expert == MOE_BF16 || d.expert == MOE_FP8_E4M3) &&
         d.T >= kDenseSharedMinRows && max_tiles <= ((int64_t)1 << 22);
}

hipError_t launch_dense_swiglu_bf16(const uint16_t* x, const uint16_t* w13, uint16_t* h,
                                    uint16_t* au, int M, int Kd, int half, hipStream_t st) {
  const int mt = (M + DB - 1) / DB;
  const int nt = half / 128;
  const int per = (mt * nt + kXcds - 1) / kXcds;
  hipLaunchKernelGGL(k_gemm_dense_swiglu_bf16, dim3(per * kXcds), dim3(512), 0, st, x, w13, h, au,
                     M, Kd, half, mt, nt);
  return hipGetLastError();
}

}  // namespace moe
