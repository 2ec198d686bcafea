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
// Tile: 256 rows (one tile holds all rows of an expert, so its weights stream from
// HBM once) x 256 weight rows x one 128-deep scale block per k step; a row of a step
// is one full 128-byte line.  Operands and the activation scales of a step go from
// memory straight into LDS (buffer loads with the LDS destination bit); the ring holds
// three steps when the A stage (ceil(rows/64)*64 rows) is at most 128 rows, else two.
// Activation rows past the expert's end arrive as zeros (range-checked descriptor).
// Eight waves, wave w owns rows 32w..32w+31 and all 256 columns (8 MFMA tiles of
// 32x32); waves past the expert's rows skip their MFMAs.
//   up   (kSwiglu): the 256 weight rows are 128 gate rows + the matching 128 up rows;
//        tile n even is gate, n+1 the matching up, so each lane holds gate and up of
//        the same h element.  The tile's 128 h columns are one quantisation tile of h
//        and lie in one wave: per-row amax by lane shuffles, scale = amax/448,
//        RNE-saturating E4M3 codes.
//   down: 256 output columns, bf16 output.
// Operand layout (32x32x64 f8): lane l supplies row l%32 and k = 32*(l/32)..+31 of A,
// column l%32 and the same k of B; result element i of lane l is row
// 8*(i/4) + 4*(l/32) + i%4, column l%32.
#include "common.h"
#include "schedule.h"

namespace moe {
namespace {

using sched::build_costs;
using sched::build_schedule;
using sched::decode_tile;
using sched::kMaxGroups;
using sched::Tile;
using sched::xcd_boundary;

constexpr int FBM = 256, FBN = 256, FBK = 128;   // FBK bytes = one 128-B line per row
constexpr int kFB = FBN * FBK;                    // B stage: 32 KiB
constexpr int kFRing = 3 * (128 * FBK + kFB);     // 144 KiB

__device__ __forceinline__ float silu(float a) { return a / (1.0f + __expf(-a)); }

// byte offset of (row, 16-byte chunk c) inside an operand stage: 128-B rows, chunk
// slots xor-swizzled by (row >> 1) & 7 (16 consecutive rows at one chunk hit 16
// distinct bank groups)
__device__ __forceinline__ int fswz(int r, int c) { return r * FBK + ((c ^ (r >> 1)) & 7) * 16; }

__device__ __forceinline__ i32x8 frag32(const char* p0, const char* p1) {
  const uint4 u0 = *reinterpret_cast<const uint4*>(p0);
  const uint4 u1 = *reinterpret_cast<const uint4*>(p1);
  i32x8 f;
  f[0] = u0.x; f[1] = u0.y; f[2] = u0.z; f[3] = u0.w;
  f[4] = u1.x; f[5] = u1.y; f[6] = u1.z; f[7] = u1.w;
  return f;
}

// gather != nullptr: row r of the permuted order is row gather[r] of A and A_scale
// (a_rows rows), so the activation rows are read from the unpermuted input.
template <bool kSwiglu>
__global__ __launch_bounds__(512, 1) void k_gemm_fp8(
    const uint8_t* __restrict__ A, const float* __restrict__ A_scale,
    const uint8_t* __restrict__ B, const float* __restrict__ B_scale, void* __restrict__ C,
    float* __restrict__ C_scale, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ gather, int a_rows, int NG, int Kd, int Nrows, int Nout,
    int half) {
  __shared__ __attribute__((aligned(1024))) char smem[kFRing];
  __shared__ __attribute__((aligned(16))) float s_sa[3][FBM];
  __shared__ int mt_start[kMaxGroups + 1];
  __shared__ long long s_cost[kMaxGroups + 1];
  build_schedule(offsets, NG, FBM, mt_start);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nt = kSwiglu ? half / 128 : (Nout + FBN - 1) / FBN;
  build_costs(offsets, mt_start, NG, FBM, nt, s_cost);
  const int nk = Kd / FBK;     // k steps = scale blocks along k
  const int nbr = Nrows / 128;  // weight-scale block rows
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_offset(smem));
  const uint32_t lds_sa = __builtin_amdgcn_readfirstlane(lds_offset(&s_sa[0][0]));
  // loader: instruction i of wave wv fills rows 64i + 8wv .. +7 of an operand stage;
  // lane l writes row 64i + 8wv + (l>>3), slot l&7 = k-chunk (l&7) ^ ((row>>1)&7)
  const int lrow = lane >> 3;
  const int lchunk = (lane & 7) ^ ((4 * (wv & 1) + (lane >> 4)) & 7);
  const int kq = lane >> 5;

  const int P = gridDim.x, per_xcd = P / kXcds;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int begin = xcd_boundary(xcd, offsets, mt_start, s_cost, NG, FBM, nt);
  const int end = xcd_boundary(xcd + 1, offsets, mt_start, s_cost, NG, FBM, nt);
  for (int tile = begin + slot; tile < end; tile += per_xcd) {
    const Tile tl = decode_tile(tile, mt_start, NG, nt);
    const int g = __builtin_amdgcn_readfirstlane(tl.g);
    const int n_idx = __builtin_amdgcn_readfirstlane(tl.n_idx);
    const int m_idx = __builtin_amdgcn_readfirstlane(tl.m_idx);
    const int row0 = offsets[g];
    const int m_g = offsets[g + 1] - row0;
    const int m0 = m_idx * FBM;
    const int m_rows = min(FBM, m_g - m0);
    const bool w_on = 32 * wv < m_rows;
    const int nA = (m_rows + 63) >> 6;
    const int sA = nA * 64 * FBK;
    const int sStage = sA + kFB;
    const int nst = (3 * sStage <= kFRing) ? 3 : 2;
    const bool ld_sa = wv < nA;  // waves 0..nA-1 bring 64 activation scales each
    const int per_stage = nA + 4 + (ld_sa ? 1 : 0);

    const i32x4 arsrc = gather ? buffer_rsrc(A, (uint32_t)a_rows * Kd)
                               : buffer_rsrc(A + (int64_t)(row0 + m0) * Kd, (uint32_t)m_rows * Kd);
    const i32x4 brsrc = buffer_rsrc(B + (int64_t)g * Nrows * Kd, (uint32_t)Nrows * Kd);
    const i32x4 srsrc =
        gather ? buffer_rsrc(A_scale, (uint32_t)a_rows * nk * 4)
               : buffer_rsrc(A_scale + (int64_t)(row0 + m0) * nk, (uint32_t)m_rows * nk * 4);
    uint32_t aoff[4], boff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 64 * i + 8 * wv + lrow;
      if (gather)
        aoff[i] = r < m_rows ? (uint32_t)(gather[row0 + m0 + r] * Kd + lchunk * 16) : 0x7ffffff0u;
      else
        aoff[i] = (uint32_t)(r * Kd + lchunk * 16);
      int br;
      if (kSwiglu) br = r < 128 ? n_idx * 128 + r : half + n_idx * 128 + (r - 128);
      else br = n_idx * FBN + r;
      boff[i] = br < Nrows ? (uint32_t)(br * Kd + lchunk * 16) : 0x7ffffff0u;
    }
    const int srow = 64 * wv + lane;  // activation-scale row this lane brings
    uint32_t soff;
    if (gather)
      soff = srow < m_rows ? (uint32_t)(gather[row0 + m0 + srow] * nk) * 4 : 0x7ffffff0u;
    else
      soff = (uint32_t)(srow * nk) * 4;
    const uint32_t ldsw = lds0 + 8 * wv * FBK;
    const uint32_t ldss = lds_sa + 64 * wv * 4;
    // weight-scale block rows: up: gate block n_idx (tiles n even), up block
    // half/128 + n_idx (n odd); down: blocks 2 n_idx (n < 4) and 2 n_idx + 1 (n >= 4)
    const float* bsc = B_scale + (int64_t)g * nbr * nk;
    const int wb0 = kSwiglu ? n_idx : min(2 * n_idx, nbr - 1);
    const int wb1 = kSwiglu ? half / 128 + n_idx : min(2 * n_idx + 1, nbr - 1);

#define FSTAGE_LOAD(kt, st)                                                           \
  {                                                                                   \
    const uint32_t sa_ = ldsw + (st) * sStage;                                        \
    const uint32_t ko_ = (uint32_t)(kt) * FBK;                                        \
    load16_to_lds(arsrc, sa_, aoff[0] + ko_);                                         \
    if (nA > 1) load16_to_lds(arsrc, sa_ + 64 * FBK, aoff[1] + ko_);                  \
    if (nA > 2) load16_to_lds(arsrc, sa_ + 128 * FBK, aoff[2] + ko_);                 \
    if (nA > 3) load16_to_lds(arsrc, sa_ + 192 * FBK, aoff[3] + ko_);                 \
    load16_to_lds_nt(brsrc, sa_ + sA, boff[0] + ko_);                                    \
    load16_to_lds_nt(brsrc, sa_ + sA + 64 * FBK, boff[1] + ko_);                         \
    load16_to_lds_nt(brsrc, sa_ + sA + 128 * FBK, boff[2] + ko_);                        \
    load16_to_lds_nt(brsrc, sa_ + sA + 192 * FBK, boff[3] + ko_);                        \
    if (ld_sa) load4_to_lds(srsrc, ldss + (st) * (FBM * 4), soff + (uint32_t)(kt) * 4); \
  }

    f32x16 acc[8];
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[n][i] = 0.0f;
    const int arow = 32 * wv + (lane & 31);

    __syncthreads();  // previous tile's LDS reads are done before the ring is refilled
    FSTAGE_LOAD(0, 0)
    if (nst == 3 && nk > 1) FSTAGE_LOAD(1, 1)
    int st = 0;
    for (int kt = 0; kt < nk; ++kt) {
      const float sw0 = bsc[(int64_t)wb0 * nk + kt];
      const float sw1 = bsc[(int64_t)wb1 * nk + kt];
      wait_vmcnt(min(nst - 2, nk - 1 - kt) * per_stage);
      __syncthreads();
      if (kt + nst - 1 < nk) {
        int sn = st + nst - 1;
        if (sn >= nst) sn -= nst;
        FSTAGE_LOAD(kt + nst - 1, sn)
      }
      if (w_on) {
        const char* as = smem + st * sStage;
        const char* bs = as + sA;
        // A fragments of both 64-deep halves: chunks 2*kq, 2*kq+1 and 4 + the same
        const i32x8 a0 = frag32(as + fswz(arow, 2 * kq), as + fswz(arow, 2 * kq + 1));
        const i32x8 a1 = frag32(as + fswz(arow, 4 + 2 * kq), as + fswz(arow, 5 + 2 * kq));
        float sa[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 v = *reinterpret_cast<const float4*>(&s_sa[st][32 * wv + 8 * q + 4 * kq]);
          sa[4 * q + 0] = v.x; sa[4 * q + 1] = v.y; sa[4 * q + 2] = v.z; sa[4 * q + 3] = v.w;
        }
#pragma unroll
        for (int n = 0; n < 8; n += 2) {
          f32x16 t[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int nn = n + u;
            const int brow = (kSwiglu ? ((nn & 1) * 128 + 32 * (nn >> 1)) : 32 * nn) + (lane & 31);
            const i32x8 b0 = frag32(bs + fswz(brow, 2 * kq), bs + fswz(brow, 2 * kq + 1));
            f32x16 z;
#pragma unroll
            for (int i = 0; i < 16; ++i) z[i] = 0.0f;
            t[u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, b0, z, 0, 0, 0, 127, 0, 127);
          }
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int nn = n + u;
            const int brow = (kSwiglu ? ((nn & 1) * 128 + 32 * (nn >> 1)) : 32 * nn) + (lane & 31);
            const i32x8 b1 = frag32(bs + fswz(brow, 4 + 2 * kq), bs + fswz(brow, 5 + 2 * kq));
            t[u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, b1, t[u], 0, 0, 0, 127, 0,
                                                                    127);
          }
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int nn = n + u;
            const float sw = kSwiglu ? ((nn & 1) ? sw1 : sw0) : (nn < 4 ? sw0 : sw1);
#pragma unroll
            for (int i = 0; i < 16; ++i)
              acc[nn][i] = __builtin_fmaf(t[u][i], sa[i] * sw, acc[nn][i]);
          }
        }
      }
      if (++st == nst) st = 0;
    }
#undef FSTAGE_LOAD

    if (!w_on) continue;
    if constexpr (kSwiglu) {
      // h = silu(gate) * up; the row's 128 h columns are the 4 gate/up pairs x 32 lanes
      float hv[4][16];
      uint8_t* hq = static_cast<uint8_t*>(C);
      const int ncb = Nout / 128;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float m = 0.0f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          hv[t][i] = silu(acc[2 * t][i]) * acc[2 * t + 1][i];
          m = __builtin_fmaxf(m, __builtin_fabsf(hv[t][i]));
        }
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) m = __builtin_fmaxf(m, __shfl_xor(m, off));
        const float sc = m > 0.0f ? m / 448.0f : 1.0f;
        const int r = 32 * wv + 8 * (i >> 2) + 4 * kq + (i & 3);
        if (r < m_rows) {
          uint8_t* hp = hq + (int64_t)(row0 + m0 + r) * Nout + n_idx * 128 + (lane & 31);
#pragma unroll
          for (int t = 0; t < 4; ++t)
            __builtin_nontemporal_store(static_cast<uint8_t>(f32_to_e4m3_bits(hv[t][i] / sc)),
                                        hp + 32 * t);
          if ((lane & 31) == 0) C_scale[(int64_t)(row0 + m0 + r) * ncb + n_idx] = sc;
        }
      }
    } else {
      uint16_t* y = static_cast<uint16_t*>(C);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 32 * wv + 8 * (i >> 2) + 4 * kq + (i & 3);
        if (r >= m_rows) continue;
        uint16_t* yp = y + (int64_t)(row0 + m0 + r) * Nout + n_idx * FBN + (lane & 31);
#pragma unroll
        for (int n = 0; n < 8; ++n)
          if (n_idx * FBN + 32 * n < Nout)  // non-temporal, as the weight loads
            __builtin_nontemporal_store(f32_to_bf16_bits(acc[n][i]), yp + 32 * n);
      }
    }
  }
}

// The shared expert's gate/up as a dense FP8 GEMM (at T >= kDenseSharedMinRows; the
// grouped launch then covers the routed experts).  Its full-height tiles in the grouped
// launch get one 64 KiB step in flight and stall on the L2; here tiles are 128 rows x
// 256 weight rows, so a step (16 KiB of codes + 32 KiB of weights + 512 B of scales)
// fits three times in LDS, two in flight, and all eight waves multiply: wave (wm, wn)
// owns rows 32wm .. +31 and the sub-tiles 4wn .. 4wn+3 of [g0 u0 g1 u1 g2 u2 g3 u3]
// (32 columns each), i.e. h columns 64wn .. +63 of the tile's 128.  The per-block
// promotion acc += partial * (s_a * s_w) is the grouped kernel's; an h row's 128-column
// quantisation tile spans the two waves wn = 0, 1, so its amax is combined through LDS.
// Tiles in bands of eight row tiles, column-major inside a band, one contiguous range
// of that order per XCD.
constexpr int QBM = 128, QBand = 8;
constexpr int kQA = QBM * FBK;        // A stage: 16 KiB
constexpr int kQStage = kQA + kFB;    // 48 KiB
constexpr int kQRing = 3;

__global__ __launch_bounds__(512, 1) void k_gemm_dense_swiglu_fp8(
    const uint8_t* __restrict__ A, const float* __restrict__ A_scale,
    const uint8_t* __restrict__ B, const float* __restrict__ B_scale, uint8_t* __restrict__ h,
    float* __restrict__ h_scale, int M, int Kd, int half, int mt, int nt) {
  __shared__ __attribute__((aligned(1024))) char smem[kQRing * kQStage];
  __shared__ __attribute__((aligned(16))) float s_sa[kQRing][QBM];
  __shared__ float s_amax[2][QBM];
  const int total = mt * nt;
  const int per = (total + kXcds - 1) / kXcds;
  const int tile = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (tile >= total) return;
  const int band = tile / (QBand * nt), within = tile % (QBand * nt);
  const int rb = min(QBand, mt - band * QBand);
  const int n_idx = within / rb, m_idx = band * QBand + within % rb;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv >> 1, wn = wv & 1;
  const int nk = Kd / FBK;      // k steps = scale blocks along k
  const int m0 = m_idx * QBM;
  const int m_rows = min(QBM, M - m0);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_offset(smem));
  const uint32_t lds_sa = __builtin_amdgcn_readfirstlane(lds_offset(&s_sa[0][0]));
  // loader: instruction i of wave wv fills rows 64i + 8wv .. +7 of an operand stage;
  // lane l writes row 64i + 8wv + (l>>3), slot l&7 (chunk (l&7) ^ ((row>>1)&7))
  const int lrow = lane >> 3;
  const int lchunk = (lane & 7) ^ ((4 * (wv & 1) + (lane >> 4)) & 7);
  const int kq = lane >> 5;
  // codes and scales of rows past M read as zeros (range check)
  const i32x4 arsrc = buffer_rsrc(A + (int64_t)m0 * Kd, (uint32_t)m_rows * Kd);
  const i32x4 brsrc = buffer_rsrc(B, (uint32_t)(2 * half) * Kd);
  const i32x4 srsrc = buffer_rsrc(A_scale + (int64_t)m0 * nk, (uint32_t)m_rows * nk * 4);
  uint32_t aoff[2], boff[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) aoff[i] = (uint32_t)((64 * i + 8 * wv + lrow) * Kd + lchunk * 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 64 * i + 8 * wv + lrow;
    const int br = r < 128 ? n_idx * 128 + r : half + n_idx * 128 + (r - 128);
    boff[i] = (uint32_t)(br * Kd + lchunk * 16);
  }
  const bool ld_sa = wv < 2;  // waves 0, 1 bring 64 activation scales each
  const uint32_t soff = (uint32_t)((64 * wv + lane) * nk) * 4;
  const uint32_t ldsw = lds0 + 8 * wv * FBK;
  const uint32_t ldss = lds_sa + 64 * wv * 4;
  const int per_stage = 6 + (ld_sa ? 1 : 0);
  const float* bsc0 = B_scale + (int64_t)n_idx * nk;                  // gate block row
  const float* bsc1 = B_scale + (int64_t)(half / 128 + n_idx) * nk;   // up block row

#define QSTAGE_LOAD(kt, st)                                                           \
  {                                                                                   \
    const uint32_t sa_ = ldsw + (st) * kQStage;                                       \
    const uint32_t ko_ = (uint32_t)(kt) * FBK;                                        \
    load16_to_lds(arsrc, sa_, aoff[0] + ko_);                                         \
    load16_to_lds(arsrc, sa_ + 64 * FBK, aoff[1] + ko_);                              \
    load16_to_lds(brsrc, sa_ + kQA, boff[0] + ko_);                                   \
    load16_to_lds(brsrc, sa_ + kQA + 64 * FBK, boff[1] + ko_);                        \
    load16_to_lds(brsrc, sa_ + kQA + 128 * FBK, boff[2] + ko_);                       \
    load16_to_lds(brsrc, sa_ + kQA + 192 * FBK, boff[3] + ko_);                       \
    if (ld_sa) load4_to_lds(srsrc, ldss + (st) * (QBM * 4), soff + (uint32_t)(kt) * 4); \
  }

  f32x16 acc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[n][i] = 0.0f;
  const int arow = 32 * wm + (lane & 31);

  QSTAGE_LOAD(0, 0)
  if (nk > 1) QSTAGE_LOAD(1, 1)
  int st = 0;
  for (int kt = 0; kt < nk; ++kt) {
    const float sw0 = bsc0[kt];
    const float sw1 = bsc1[kt];
    wait_vmcnt(min(kQRing - 2, nk - 1 - kt) * per_stage);
    __syncthreads();
    if (kt + kQRing - 1 < nk) {
      int sn = st + kQRing - 1;
      if (sn >= kQRing) sn -= kQRing;
      QSTAGE_LOAD(kt + kQRing - 1, sn)
    }
    const char* as = smem + st * kQStage;
    const char* bs = as + kQA;
    // A fragments of both 64-deep halves: chunks 2*kq, 2*kq+1 and 4 + the same
    const i32x8 a0 = frag32(as + fswz(arow, 2 * kq), as + fswz(arow, 2 * kq + 1));
    const i32x8 a1 = frag32(as + fswz(arow, 4 + 2 * kq), as + fswz(arow, 5 + 2 * kq));
    float sa[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = *reinterpret_cast<const float4*>(&s_sa[st][32 * wm + 8 * q + 4 * kq]);
      sa[4 * q + 0] = v.x; sa[4 * q + 1] = v.y; sa[4 * q + 2] = v.z; sa[4 * q + 3] = v.w;
    }
#pragma unroll
    for (int n = 0; n < 4; n += 2) {
      f32x16 t[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int nn = 4 * wn + n + u;
        const int brow = (nn & 1) * 128 + 32 * (nn >> 1) + (lane & 31);
        const i32x8 b0 = frag32(bs + fswz(brow, 2 * kq), bs + fswz(brow, 2 * kq + 1));
        f32x16 z;
#pragma unroll
        for (int i = 0; i < 16; ++i) z[i] = 0.0f;
        t[u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, b0, z, 0, 0, 0, 127, 0, 127);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int nn = 4 * wn + n + u;
        const int brow = (nn & 1) * 128 + 32 * (nn >> 1) + (lane & 31);
        const i32x8 b1 = frag32(bs + fswz(brow, 4 + 2 * kq), bs + fswz(brow, 5 + 2 * kq));
        t[u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, b1, t[u], 0, 0, 0, 127, 0, 127);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float sw = (u & 1) ? sw1 : sw0;  // sub-tile parity: gate even, up odd
#pragma unroll
        for (int i = 0; i < 16; ++i)
          acc[n + u][i] = __builtin_fmaf(t[u][i], sa[i] * sw, acc[n + u][i]);
      }
    }
    if (++st == kQRing) st = 0;
  }
#undef QSTAGE_LOAD

  // h = silu(gate) * up; this wave holds 64 of the row's 128 quantisation columns
  float hv[2][16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float m = 0.0f;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      hv[t][i] = silu(acc[2 * t][i]) * acc[2 * t + 1][i];
      m = __builtin_fmaxf(m, __builtin_fabsf(hv[t][i]));
    }
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) m = __builtin_fmaxf(m, __shfl_xor(m, off));
    if ((lane & 31) == 0) s_amax[wn][32 * wm + 8 * (i >> 2) + 4 * kq + (i & 3)] = m;
  }
  __syncthreads();
  const int ncb = half / 128;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 32 * wm + 8 * (i >> 2) + 4 * kq + (i & 3);
    if (r >= m_rows) continue;
    const float m = __builtin_fmaxf(s_amax[0][r], s_amax[1][r]);
    const float sc = m > 0.0f ? m / 448.0f : 1.0f;
    uint8_t* hp = h + (int64_t)(m0 + r) * half + n_idx * 128 + 64 * wn + (lane & 31);
#pragma unroll
    for (int t = 0; t < 2; ++t)
      __builtin_nontemporal_store(static_cast<uint8_t>(f32_to_e4m3_bits(hv[t][i] / sc)),
                                  hp + 32 * t);
    if (wn == 0 && (lane & 31) == 0) h_scale[(int64_t)(m0 + r) * ncb + n_idx] = sc;
  }
}

// The same dense FP8 gate/up over 256-row tiles, for batches that give every CU a
// tile: 256 rows x 256 weight rows per tile, wave (wm, wn) owning rows 64wm .. +63 (two
// 32-row sub-tiles) and the sub-tiles 4wn .. 4wn+3 of the gate/up interleave.  Each
// wave multiplies 16 MFMAs per 128-deep step for 24 KiB of LDS fragment reads (the
// 128-row kernel: 8 MFMAs for 20 KiB; its LDS reads, not its MFMAs, bound it).  The
// weight fragment is the MFMA's first operand, as in the packed kernels, so a lane's
// accumulators belong to one activation row and the per-block promotion takes a single
// scale per lane: acc += partial * (s_a * s_w), the same products in the same order,
// so the codes equal the 128-row kernel's bit for bit.  Two 64 KiB stages in LDS: step
// kt's loads go out right after the barrier that frees their buffer, one step ahead.
// h codes are staged per row in LDS (16-byte chunks swizzled by the row) and written
// back as whole 128-byte lines.
constexpr int WBM = 256;
constexpr int kWA = WBM * FBK;          // A stage: 32 KiB
constexpr int kWStage = kWA + kFB;      // 64 KiB

__global__ __launch_bounds__(512, 1) void k_gemm_dense_swiglu_fp8_w(
    const uint8_t* __restrict__ A, const float* __restrict__ A_scale,
    const uint8_t* __restrict__ B, const float* __restrict__ B_scale, uint8_t* __restrict__ h,
    float* __restrict__ h_scale, int M, int Kd, int half, int mt, int nt) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * kWStage];
  __shared__ __attribute__((aligned(16))) float s_sa[2][WBM];
  __shared__ float s_amax[2][WBM];
  const int total = mt * nt;
  const int per = (total + kXcds - 1) / kXcds;
  const int tile = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (tile >= total) return;
  constexpr int band_h = 4;  // row tiles per band; column-major inside a band
  const int band = tile / (band_h * nt), within = tile % (band_h * nt);
  const int rb = min(band_h, mt - band * band_h);
  const int n_idx = within / rb, m_idx = band * band_h + within % rb;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv >> 1, wn = wv & 1;
  const int nk = Kd / FBK;
  const int m0 = m_idx * WBM;
  const int m_rows = min(WBM, M - m0);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_offset(smem));
  const uint32_t lds_sa = __builtin_amdgcn_readfirstlane(lds_offset(&s_sa[0][0]));
  // loader: instruction i of wave wv fills rows 64i + 8wv .. +7 of an operand stage;
  // lane l writes row 64i + 8wv + (l>>3), slot l&7 (chunk (l&7) ^ ((row>>1)&7))
  const int lrow = lane >> 3;
  const int lchunk = (lane & 7) ^ ((4 * (wv & 1) + (lane >> 4)) & 7);
  const int kq = lane >> 5, fr = lane & 31;
  const i32x4 arsrc = buffer_rsrc(A + (int64_t)m0 * Kd, (uint32_t)m_rows * Kd);
  const i32x4 brsrc = buffer_rsrc(B, (uint32_t)(2 * half) * Kd);
  const i32x4 srsrc = buffer_rsrc(A_scale + (int64_t)m0 * nk, (uint32_t)m_rows * nk * 4);
  uint32_t aoff[4], boff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 64 * i + 8 * wv + lrow;
    aoff[i] = (uint32_t)(r * Kd + lchunk * 16);
    const int br = r < 128 ? n_idx * 128 + r : half + n_idx * 128 + (r - 128);
    boff[i] = (uint32_t)(br * Kd + lchunk * 16);
  }
  const bool ld_sa = wv < 4;  // waves 0..3 bring 64 activation scales each
  const uint32_t soff = (uint32_t)((64 * wv + lane) * nk) * 4;
  const uint32_t ldsw = lds0 + 8 * wv * FBK;
  const uint32_t ldss = lds_sa + 64 * wv * 4;
  const float* bsc0 = B_scale + (int64_t)n_idx * nk;                  // gate block row
  const float* bsc1 = B_scale + (int64_t)(half / 128 + n_idx) * nk;   // up block row
  auto stage_load = [&](int kt, int st) {
    const uint32_t sa_ = ldsw + st * kWStage;
    const uint32_t ko = (uint32_t)kt * FBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) load16_to_lds(arsrc, sa_ + i * 64 * FBK, aoff[i] + ko);
#pragma unroll
    for (int i = 0; i < 4; ++i) load16_to_lds(brsrc, sa_ + kWA + i * 64 * FBK, boff[i] + ko);
    if (ld_sa) load4_to_lds(srsrc, ldss + st * (WBM * 4), soff + (uint32_t)kt * 4);
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][n][i] = 0.0f;

  stage_load(0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    const float sw0 = bsc0[kt];
    const float sw1 = bsc1[kt];
    wait_vm<0>();     // step kt's stage is in
    __syncthreads();  // ... for every wave, and step kt-1's buffer is free
    if (kt + 1 < nk) stage_load(kt + 1, st ^ 1);
    const char* as = smem + st * kWStage;
    const char* bs = as + kWA;
    i32x8 a0[2], a1[2];
    float sa[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int arow = 64 * wm + 32 * m + fr;
      a0[m] = frag32(as + fswz(arow, 2 * kq), as + fswz(arow, 2 * kq + 1));
      a1[m] = frag32(as + fswz(arow, 4 + 2 * kq), as + fswz(arow, 5 + 2 * kq));
      sa[m] = s_sa[st][arow];
    }
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int nn = 4 * wn + n;
      const int brow = (nn & 1) * 128 + 32 * (nn >> 1) + fr;
      const i32x8 b0 = frag32(bs + fswz(brow, 2 * kq), bs + fswz(brow, 2 * kq + 1));
      const i32x8 b1 = frag32(bs + fswz(brow, 4 + 2 * kq), bs + fswz(brow, 5 + 2 * kq));
      const float sw = (n & 1) ? sw1 : sw0;  // sub-tile parity: gate even, up odd
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        f32x16 t;
#pragma unroll
        for (int i = 0; i < 16; ++i) t[i] = 0.0f;
        t = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b0, a0[m], t, 0, 0, 0, 127, 0, 127);
        t = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b1, a1[m], t, 0, 0, 0, 127, 0, 127);
        const float sc = sa[m] * sw;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[m][n][i] = __builtin_fmaf(t[i], sc, acc[m][n][i]);
      }
    }
  }
  __syncthreads();  // every wave is done with the stages, which now stage the codes

  // lane: activation row 64wm + 32m + l%32; h columns (of the tile's 128)
  // 64wn + 32p + 8q + 4(l/32) + t for accumulator element 4q + t of pair p
  float hv[2][2][16];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    float am = 0.0f;
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        hv[m][p][i] = silu(acc[m][2 * p][i]) * acc[m][2 * p + 1][i];
        am = __builtin_fmaxf(am, __builtin_fabsf(hv[m][p][i]));
      }
    am = __builtin_fmaxf(am, __shfl_xor(am, 32));
    if (kq == 0) s_amax[wn][64 * wm + 32 * m + fr] = am;
  }
  __syncthreads();
  char* hst = smem;  // [256 rows][128 bytes] of codes, chunk slot c ^ (row & 7)
  const int ncb = half / 128;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int r = 64 * wm + 32 * m + fr;
    const float am = __builtin_fmaxf(s_amax[0][r], s_amax[1][r]);
    const float sc = am > 0.0f ? am / 448.0f : 1.0f;
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t w = pack4_e4m3(hv[m][p][4 * q] / sc, hv[m][p][4 * q + 1] / sc,
                                      hv[m][p][4 * q + 2] / sc, hv[m][p][4 * q + 3] / sc);
        const int ch = 4 * wn + 2 * p + (q >> 1);
        *reinterpret_cast<uint32_t*>(hst + r * 128 + ((ch ^ (r & 7)) << 4) + 8 * (q & 1) +
                                     4 * kq) = w;
      }
    if (wn == 0 && kq == 0 && r < m_rows) h_scale[(int64_t)(m0 + r) * ncb + n_idx] = sc;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // 256 rows x 8 chunks, 4 per thread
    const int row = 64 * i + (tid >> 3), ch = tid & 7;
    const u32x4 v = *reinterpret_cast<const u32x4*>(hst + row * 128 + ((ch ^ (row & 7)) << 4));
    if (row < m_rows)
      __builtin_nontemporal_store(
          v, reinterpret_cast<u32x4*>(h + (int64_t)(m0 + row) * half + n_idx * 128 + 16 * ch));
  }
}

int fp8_grid(int cus) {
  const int p = (cus / kXcds) * kXcds;
  return p < kXcds ? kXcds : p;
}

}  // namespace

hipError_t launch_dense_swiglu_fp8_shared(const Dims& d, const void* xs, const float* xs_scale,
                                          const int32_t* gather, const void* w13,
                                          const float* w13_scale, void* h, float* h_scale,
                                          hipStream_t st) {
  const int64_t r0 = d.T * d.K;
  const int nkb = d.H / 128;
  const uint8_t* xa = static_cast<const uint8_t*>(xs) + (gather ? 0 : r0 * d.H);
  const float* xsa = xs_scale + (gather ? 0 : r0 * nkb);
  const int nt = d.I / 128;
  const int mtw = (int)((d.T + WBM - 1) / WBM);
  if (mtw * nt >= device_cu_count()) {  // every CU gets a 256-row tile
    const int perw = (mtw * nt + kXcds - 1) / kXcds;
    hipLaunchKernelGGL(k_gemm_dense_swiglu_fp8_w, dim3(perw * kXcds), dim3(512), 0, st, xa, xsa,
                       static_cast<const uint8_t*>(w13) + (int64_t)d.E * 2 * d.I * d.H,
                       w13_scale + (int64_t)d.E * (2 * d.I / 128) * nkb,
                       static_cast<uint8_t*>(h) + r0 * d.I, h_scale + r0 * (d.I / 128),
                       (int)d.T, d.H, d.I, mtw, nt);
    return hipGetLastError();
  }
  const int mt = (int)((d.T + QBM - 1) / QBM);
  const int per = (mt * nt + kXcds - 1) / kXcds;
  hipLaunchKernelGGL(k_gemm_dense_swiglu_fp8, dim3(per * kXcds), dim3(512), 0, st, xa, xsa,
                     static_cast<const uint8_t*>(w13) + (int64_t)d.E * 2 * d.I * d.H,
                     w13_scale + (int64_t)d.E * (2 * d.I / 128) * nkb,
                     static_cast<uint8_t*>(h) + r0 * d.I, h_scale + r0 * (d.I / 128), (int)d.T,
                     d.H, d.I, mt, nt);
  return hipGetLastError();
}

hipError_t launch_fp8_up(const Dims& d, const void* xs, const float* xs_scale,
                         const int32_t* offsets, const int32_t* gather, const void* w13,
                         const float* w13_scale, void* h, float* h_scale, hipStream_t st) {
  int ng = d.E + d.S;
  if (dense_shared(d)) {  // the shared expert's rows T*K .. T*K+T-1, token order
    ng = d.E;
    const hipError_t e =
        launch_dense_swiglu_fp8_shared(d, xs, xs_scale, gather, w13, w13_scale, h, h_scale, st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_gemm_fp8<true>), dim3(fp8_grid(device_cu_count())), dim3(512), 0, st,
                     static_cast<const uint8_t*>(xs), xs_scale, static_cast<const uint8_t*>(w13),
                     w13_scale, h, h_scale, offsets, gather, (int)d.T, ng, d.H, 2 * d.I,
                     d.I, d.I);
  return hipGetLastError();
}

hipError_t launch_fp8_down(const Dims& d, const void* h, const float* h_scale,
                           const int32_t* offsets, const void* w2, const float* w2_scale, void* ys,
                           hipStream_t st) {
  hipLaunchKernelGGL((k_gemm_fp8<false>), dim3(fp8_grid(device_cu_count())), dim3(512), 0, st,
                     static_cast<const uint8_t*>(h), h_scale, static_cast<const uint8_t*>(w2),
                     w2_scale, ys, nullptr, offsets, nullptr, 0, d.E + d.S, d.I, d.H, d.H, 0);
  return hipGetLastError();
}

}  // namespace moe
