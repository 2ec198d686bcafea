// Expert FFN backward as grouped GEMMs (the derivative of the forward in gemm.hip;
// gradients accumulate in fp32 -- joto.ai item 3, FP32 accumulation; weight
// gradients are stored in fp32):
//   dh          = dY W2[g]                       (reduction over H)
//   [da|du]     = dh u silu'(a) | dh silu(a)     (epilogue of dh; a, u saved by the
//                                                 forward's gate/up GEMM)
//   dx_sorted   = [da|du] W13[g]                 (reduction over 2I)
//   dW2[g]      = dY^T h,   dW13[g] = [da|du]^T x  (reductions over the group's rows)
// The dgrad products contract over a dimension that is the OUTER one of the stored
// weights (W2 is [H, I], W13 is [2I, H]), and the weight-gradient products contract
// over rows of both operands, so those operands are "K-outer".  They go to LDS
// unchanged (64 k-rows of 256 columns per stage, 512-byte rows, loaded straight into
// LDS in full lines) and the MFMA fragments are read with ds_read_b64_tr_b16, which
// transposes 16-bit elements across each group of 16 lanes: source lane a + 4i points
// at k-row kbase + i, columns nbase + 4a .. +3, and lane 4a + b receives column
// nbase + 4a + b at k-rows kbase .. kbase + 3.  Two such reads give a lane the 8
// consecutive k of its column -- the operand layout of v_mfma_f32_32x32x16_bf16.
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

typedef short v4i16 __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kARow = BK * 2;         // K-inner operand: 128-byte rows
constexpr int kORow = BN * 2;         // K-outer operand: 512-byte rows (64 k-rows)
constexpr int kOStage = BK * kORow;   // 32 KiB
constexpr int kRing = 3 * (128 * kARow + kOStage);  // 144 KiB

__device__ __forceinline__ float silu_f(float a) { return a / (1.0f + __expf(-a)); }

// K-inner operand (rows of 128 B): chunk slots xor-swizzled by (row >> 1) & 7.
__device__ __forceinline__ int swz_a(int r, int c) { return r * kARow + ((c ^ (r >> 1)) & 7) * 16; }

// K-outer operand (k-rows of 512 B = 32 chunks): chunk c of k-row r sits in slot
// c ^ (2 (r & 3)), so the 4 k-rows x 2 chunks a 16-lane transposed read touches land
// in 8 distinct bank groups.
__device__ __forceinline__ int swz_o(int r, int c) { return r * kORow + ((c ^ (2 * (r & 3))) << 4); }

// Lane part of the LDS byte offset of a K-outer fragment read, for fragment columns
// nb with (nb / 32) & 1 == par.  In each 16-lane group g, source lane j reads k-row
// 8 (g >> 1) + j / 4 and 4 columns starting at 16 (g & 1) + 4 (j & 3); the chunk swizzle
// stays inside an aligned group of 8 chunks (64 columns), so the fragment at columns
// nb, k-step s (16 k-rows), upper half (k + 4) sits at
//   kouter_lane_off(lane, par) + (nb / 64) * 128 + s * 8192 + hi * 2048,
// constants the compiler folds into the read's offset field.
__device__ __forceinline__ uint32_t kouter_lane_off(int lane, int par) {
  const int g = lane >> 4, j = lane & 15, i = j >> 2;
  const int row = 8 * (g >> 1) + i;
  const int c = 4 * par + 2 * (g & 1) + ((j & 3) >> 1);
  return (uint32_t)(row * kORow + ((c ^ (2 * i)) << 4) + (j & 1) * 8);
}

// 8 consecutive k of one column per lane (the v_mfma_f32_32x32x16_bf16 operand layout)
// from a K-outer stage: `addr` is the LDS byte address of the lower read.
__device__ __forceinline__ bf16x8 frag_ko(uint32_t addr) {
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(uintptr_t)addr);
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(uintptr_t)(addr + 4 * kORow));
  bf16x8 f;
  const v4i16 both[2] = {lo, hi};
  __builtin_memcpy(&f, both, 16);
  return f;
}

// One k-stage of a K-outer operand: k-rows k0 .. k0+63 (those >= krows read as zeros)
// of columns col0 .. col0+255 (those >= ncols read as zeros) of a row-major matrix
// with `ld` elements per row.  Wave wv, instruction j fills k-rows 2(4wv+j), +1.
// gather != nullptr: k-row q is matrix row gather[q].
struct KOuterLoader {
  i32x4 rsrc;
  uint32_t off[4];  // byte offset of this lane's 16 bytes for instruction j, k0 = 0
  bool row_ok[4];
  int krow[4];
};

__device__ __forceinline__ void kouter_setup(KOuterLoader& L, const void* base, int64_t nrows,
                                             int ld, int col0, int ncols, int lane, int wv) {
  L.rsrc = buffer_rsrc(base, (uint32_t)(nrows * ld * 2));
  const int slot = lane & 31;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 2 * (4 * wv + j) + (lane >> 5);
    const int c = slot ^ (2 * (r & 3));
    L.krow[j] = r;
    L.row_ok[j] = col0 + 8 * c < ncols;
    L.off[j] = (uint32_t)((col0 + 8 * c) * 2);
  }
}

// issue the 4 loads of stage k0 (k-rows k0..k0+63; rows >= krows -> zeros)
__device__ __forceinline__ void kouter_issue(const KOuterLoader& L, uint32_t lds_stage, int wv,
                                             int k0, int krows, int ld, int rowbase,
                                             const int32_t* __restrict__ gather) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int kr = k0 + L.krow[j];
    uint32_t voff = 0x7ffffff0u;
    if (kr < krows && L.row_ok[j]) {
      const int grow = gather ? gather[rowbase + kr] : rowbase + kr;
      voff = (uint32_t)grow * (uint32_t)ld * 2u + L.off[j];
    }
    load16_to_lds(L.rsrc, lds_stage + (4 * wv + j) * 1024, voff);
  }
}

// The same stage in two halves: the matrix row of each of this lane's 4 loads (-1:
// outside, read as zeros), then the loads.  Fetching the gather indices ahead lets the
// loads themselves be issued without waiting on index reads.
__device__ __forceinline__ void kouter_rows(const KOuterLoader& L, int k0, int krows, int rowbase,
                                            const int32_t* __restrict__ gather, int rows[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int kr = k0 + L.krow[j];
    rows[j] = -1;
    if (kr < krows && L.row_ok[j]) rows[j] = gather ? gather[rowbase + kr] : rowbase + kr;
  }
}

__device__ __forceinline__ void kouter_issue_rows(const KOuterLoader& L, uint32_t lds_stage,
                                                  int wv, int ld, const int rows[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t voff =
        rows[j] >= 0 ? (uint32_t)rows[j] * (uint32_t)ld * 2u + L.off[j] : 0x7ffffff0u;
    load16_to_lds(L.rsrc, lds_stage + (4 * wv + j) * 1024, voff);
  }
}

// ---------------------------------------------------------------------------
// dgrad:  C[r, n] = sum_k A[r, k] B[g][k, n] over the rows r of group g.
//   A: [R, Kd] activations (K-inner, bf16); B: [NG, Kd, N] weights (K-outer);
//   kSwigluBwd: C columns are h columns n < I; the epilogue turns dh into
//   da = dh u silu'(a) and du = dh silu(a) with a = au[r][n], u = au[r][I + n] and
//   writes both into C ([R, 2I]); else C[r, n] = dh rounded ([R, N]).
// Tile, ring, schedule and wave layout as the forward bf16 GEMM.
// ---------------------------------------------------------------------------
template <bool kSwigluBwd>
__global__ __launch_bounds__(512, 1) void k_gemm_nn_bf16(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, uint16_t* __restrict__ C,
    const uint16_t* __restrict__ au, const int32_t* __restrict__ offsets, int NG, int Kd, int N,
    int I) {
  __shared__ __attribute__((aligned(1024))) char smem[kRing];
  __shared__ int mt_start[kMaxGroups + 1];
  __shared__ long long s_cost[kMaxGroups + 1];
  build_schedule(offsets, NG, BM, mt_start);
  const int nt = (N + BN - 1) / BN;
  build_costs(offsets, mt_start, NG, BM, nt, s_cost);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv >> 1, wn = wv & 1;
  const int nk = Kd / BK;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_offset(smem));
  const int lrow = lane >> 3;
  const int lchunk = (lane & 7) ^ ((4 * (wv & 1) + (lane >> 4)) & 7);
  const int kq = lane >> 5;

  const int P = gridDim.x, per_xcd = P / kXcds;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int begin = xcd_boundary(xcd, offsets, mt_start, s_cost, NG, BM, nt);
  const int end = xcd_boundary(xcd + 1, offsets, mt_start, s_cost, NG, BM, nt);
  for (int tile = begin + slot; tile < end; tile += per_xcd) {
    Tile tl = decode_tile(tile, mt_start, NG, nt);
    tl.g = __builtin_amdgcn_readfirstlane(tl.g);
    tl.n_idx = __builtin_amdgcn_readfirstlane(tl.n_idx);
    tl.m_idx = __builtin_amdgcn_readfirstlane(tl.m_idx);
    const int row0 = offsets[tl.g];
    const int m_g = offsets[tl.g + 1] - row0;
    const int m0 = tl.m_idx * BM;
    const int m_rows = min(BM, m_g - m0);
    const int n0 = tl.n_idx * BN;
    const bool w_on = 64 * wm < m_rows && n0 + 128 * wn < N;
    const bool w_sub1 = 64 * wm + 32 < m_rows;
    const int nA = (m_rows + 63) >> 6;
    const int sA = nA * 64 * kARow;
    const int sStage = sA + kOStage;
    const int nst = (3 * sStage <= kRing) ? 3 : 2;
    const int per_stage = nA + 4;

    const i32x4 arsrc = buffer_rsrc(A + (int64_t)(row0 + m0) * Kd, (uint32_t)m_rows * Kd * 2);
    uint32_t aoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) aoff[i] = (uint32_t)((64 * i + 8 * wv + lrow) * Kd + lchunk * 8) * 2;
    KOuterLoader bl;
    kouter_setup(bl, B + (int64_t)tl.g * Kd * N, Kd, N, n0, N, lane, wv);
    const uint32_t ldsw = lds0 + 8 * wv * kARow;
    const uint32_t lo_b[2] = {lds0 + kouter_lane_off(lane, 0), lds0 + kouter_lane_off(lane, 1)};

#define NN_STAGE_LOAD(kt, st)                                                         \
  {                                                                                   \
    const uint32_t sa_ = ldsw + (st) * sStage;                                        \
    const uint32_t ko_ = (uint32_t)(kt) * kARow;                                      \
    load16_to_lds(arsrc, sa_, aoff[0] + ko_);                                         \
    if (nA > 1) load16_to_lds(arsrc, sa_ + 64 * kARow, aoff[1] + ko_);                \
    if (nA > 2) load16_to_lds(arsrc, sa_ + 128 * kARow, aoff[2] + ko_);               \
    if (nA > 3) load16_to_lds(arsrc, sa_ + 192 * kARow, aoff[3] + ko_);               \
    kouter_issue(bl, lds0 + (st) * sStage + sA, wv, (kt) * BK, Kd, N, 0, nullptr);    \
  }

    f32x16 acc[2][4];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mi][n][i] = 0.0f;
    const int arow0 = 64 * wm + (lane & 31), arow1 = arow0 + 32;

    __syncthreads();
    NN_STAGE_LOAD(0, 0)
    if (nst == 3 && nk > 1) NN_STAGE_LOAD(1, 1)
    int st = 0;
    for (int kt = 0; kt < nk; ++kt) {
      wait_vmcnt(min(nst - 2, nk - 1 - kt) * per_stage);
      __syncthreads();
      if (kt + nst - 1 < nk) {
        int sn = st + nst - 1;
        if (sn >= nst) sn -= nst;
        NN_STAGE_LOAD(kt + nst - 1, sn)
      }
      if (w_on) {
        const char* as = smem + st * sStage;
        const uint32_t boff = st * sStage + sA + 2 * wn * 128;
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
          const int c = 2 * s + kq;
          bf16x8 b[4];
#pragma unroll
          for (int n = 0; n < 4; ++n)
            b[n] = frag_ko(lo_b[n & 1] + boff + (n >> 1) * 128 + s * 16 * kORow);
          const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(as + swz_a(arow0, c));
#pragma unroll
          for (int n = 0; n < 4; ++n)
            acc[0][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b[n], acc[0][n], 0, 0, 0);
          if (w_sub1) {
            const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(as + swz_a(arow1, c));
#pragma unroll
            for (int n = 0; n < 4; ++n)
              acc[1][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b[n], acc[1][n], 0, 0, 0);
          }
        }
      }
      if (++st == nst) st = 0;
    }
#undef NN_STAGE_LOAD

    if (w_on) {
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int m = 64 * wm + 32 * mi + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
          if (m >= m_rows) continue;
          const int64_t r = row0 + m0 + m;
#pragma unroll
          for (int n = 0; n < 4; ++n) {
            const int col = n0 + 128 * wn + 32 * n + (lane & 31);
            if (col >= N) continue;
            const float dh = acc[mi][n][i];
            if (kSwigluBwd) {
              const float a = bf16_bits_to_f32(au[r * 2 * I + col]);
              const float u = bf16_bits_to_f32(au[r * 2 * I + I + col]);
              const float sg = 1.0f / (1.0f + __expf(-a));
              C[r * 2 * I + col] = f32_to_bf16_bits(dh * u * (sg * (1.0f + a * (1.0f - sg))));
              C[r * 2 * I + I + col] = f32_to_bf16_bits(dh * (a * sg));
            } else {
              C[r * N + col] = f32_to_bf16_bits(dh);
            }
          }
        }
    }
  }
}

// ---------------------------------------------------------------------------
// wgrad:  Cw[g][i, n] = sum over the rows r of group g of A[r, i] B[r, n]  (fp32 out)
//   A: [R, M] rows; B: [R, N] rows (or, with gather, [T, N] rows gather[r]).
// Tiles (group, i-tile, n-tile), 256 x 256, k steps of 64 rows; both operands K-outer
// (two 32 KiB stages of each, double-buffered).  Groups without rows write zeros.
//
// With ~128 rows per expert a tile is 2 k-steps of MFMA work and 256 KiB of fp32
// output, so the kernel is bound by HBM writes.  Two choices keep the write stream
// going:
//  * the MFMA takes the B fragment as its first operand, so a lane's accumulator holds
//    4 consecutive n of one output row: each lane writes 16 bytes per store, 32 stores
//    per tile, every one issued (lanes outside the matrix point past the end of the
//    buffer and are dropped), so the count is exact;
//  * the first two k-stages of the NEXT tile are issued before this tile's stores.
//    Vector memory operations complete in issue order, so the wait for those stages
//    leaves this tile's 32 stores outstanding (vmcnt <= 32 (+8 for the second stage))
//    and the stores drain while the next tile computes.
// ---------------------------------------------------------------------------
constexpr int kTnStores = 32;  // 16-byte stores per lane per tile

// K-outer stage loader of the wgrad kernel: the column (within the matrix) of this
// lane's 16 bytes for each of its 4 load instructions; k-rows as in kouter_setup.
struct TnLoader {
  i32x4 rsrc;
  int col[4];
};

__device__ __forceinline__ int tn_krow(int wv, int j, int lane) {
  return 2 * (4 * wv + j) + (lane >> 5);
}

__device__ __forceinline__ void tn_setup(TnLoader& L, const void* base, int64_t nrows, int ld,
                                         int col0, int lane) {
  L.rsrc = buffer_rsrc(base, (uint32_t)(nrows * ld * 2));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 2 * j + (lane >> 5);  // k-row mod 4 (the 8 wv term drops out)
    L.col[j] = col0 + 8 * ((lane & 31) ^ (2 * (r & 3)));
  }
}

// matrix rows of stage k0 for this lane's 4 loads (-1: outside, read as zeros)
__device__ __forceinline__ void tn_rows(int wv, int lane, int k0, int m_g, int row0,
                                        const int32_t* __restrict__ gather, int rows[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int kr = k0 + tn_krow(wv, j, lane);
    rows[j] = -1;
    if (kr < m_g) rows[j] = gather ? gather[row0 + kr] : row0 + kr;
  }
}

__device__ __forceinline__ void tn_issue(const TnLoader& L, uint32_t lds_stage, int wv, int ld,
                                         const int rows[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t voff = (rows[j] >= 0 && L.col[j] < ld)
                              ? ((uint32_t)rows[j] * (uint32_t)ld + (uint32_t)L.col[j]) * 2u
                              : 0x7ffffff0u;
    load16_to_lds(L.rsrc, lds_stage + (4 * wv + j) * 1024, voff);
  }
}

struct TnTile {
  int g, i0, n0, row0, m_g, nk;
};

__device__ __forceinline__ TnTile tn_tile(int tile, int mtn, int ntn,
                                          const int32_t* __restrict__ offsets) {
  TnTile t;
  t.g = __builtin_amdgcn_readfirstlane(tile / (mtn * ntn));
  const int rem = tile - t.g * mtn * ntn;
  t.i0 = __builtin_amdgcn_readfirstlane(rem / ntn) * BM;
  t.n0 = __builtin_amdgcn_readfirstlane(rem % ntn) * BN;
  t.row0 = __builtin_amdgcn_readfirstlane(offsets[t.g]);
  t.m_g = __builtin_amdgcn_readfirstlane(offsets[t.g + 1]) - t.row0;
  t.nk = (t.m_g + BK - 1) / BK;
  return t;
}

// Stages 0 and 1 of tile t into the two LDS buffers; every index read (stages 0-2) is
// made before the first load is issued, so issuing never waits on memory.
__device__ __forceinline__ void tn_prefetch(const TnTile& t, const TnLoader& al,
                                            const TnLoader& bl, int wv, int lane, uint32_t lds0,
                                            int M, int N, const int32_t* __restrict__ gather,
                                            int rB2[4]) {
  int ra0[4], ra1[4], rb0[4], rb1[4];
  tn_rows(wv, lane, 0, t.m_g, t.row0, gather, rb0);
  tn_rows(wv, lane, BK, t.m_g, t.row0, gather, rb1);
  tn_rows(wv, lane, 2 * BK, t.m_g, t.row0, gather, rB2);
  tn_rows(wv, lane, 0, t.m_g, t.row0, nullptr, ra0);
  tn_rows(wv, lane, BK, t.m_g, t.row0, nullptr, ra1);
  // the index reads are the youngest memory operations here: wait for them before
  // the loads, so no wait for an index lands between loads (it would also wait for
  // the loads issued before it)
  wait_vm<0>();
  if (t.nk > 0) {
    tn_issue(al, lds0, wv, M, ra0);
    tn_issue(bl, lds0 + kOStage, wv, N, rb0);
  }
  if (t.nk > 1) {
    tn_issue(al, lds0 + 2 * kOStage, wv, M, ra1);
    tn_issue(bl, lds0 + 3 * kOStage, wv, N, rb1);
  }
}

__global__ __launch_bounds__(512, 1) void k_gemm_tn_bf16(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
    const int32_t* __restrict__ gather, int64_t b_rows, float* __restrict__ Cw,
    const int32_t* __restrict__ offsets, int NG, int M, int N) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * 2 * kOStage];  // 128 KiB
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv >> 1, wn = wv & 1;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_offset(smem));
  const int mtn = (M + BM - 1) / BM, ntn = (N + BN - 1) / BN;
  const int ntiles = NG * mtn * ntn;
  const int64_t R = offsets[NG];
  const int64_t brows = gather ? b_rows : R;
  const uint32_t out_bytes = (uint32_t)M * (uint32_t)N * 4u;  // <= 2^31 (checked on the host)

  const int P = gridDim.x, per_xcd = P / kXcds;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int chunk = (ntiles + kXcds - 1) / kXcds;
  const int end = min(ntiles, (xcd + 1) * chunk);
  int tile = xcd * chunk + slot;
  if (tile >= end) return;

  // Vector memory operations complete in issue order.  Every tile's first two k-stages
  // are issued before the previous tile's 32 stores, so waiting until at most 32
  // operations are outstanding leaves those stores draining while the tile computes.
  // The first tile follows 32 stores that point past the end of the output (dropped),
  // so the count is the same for every tile.
  const __amdgpu_buffer_rsrc_t out0 =
      __builtin_amdgcn_make_buffer_rsrc(Cw, (short)0, (int)out_bytes, 0x00020000);
  const uint32_t lo_f[2] = {lds0 + kouter_lane_off(lane, 0), lds0 + kouter_lane_off(lane, 1)};
  const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};

  TnTile t = tn_tile(tile, mtn, ntn, offsets);
  TnLoader al, bl;
  tn_setup(al, A, R, M, t.i0, lane);
  tn_setup(bl, B, brows, N, t.n0, lane);
  int rB2[4];  // B rows of stage 2 (gather indices fetched ahead)
  tn_prefetch(t, al, bl, wv, lane, lds0, M, N, gather, rB2);
#pragma unroll
  for (int q = 0; q < kTnStores; ++q)  // distinct addresses, so none is merged away
    __builtin_amdgcn_raw_buffer_store_b128(zero4, out0, out_bytes + 16u * q, 0, 0);

  for (;;) {
    f32x16 acc[2][4];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mi][n][i] = 0.0f;

    for (int kt = 0; kt < t.nk; ++kt) {
      if (kt < 2) wait_vm<kTnStores>();
      else wait_vm<0>();
      __syncthreads();
      if (kt >= 1 && kt + 1 < t.nk) {  // stage kt+1 >= 2 into the buffer stage kt-1 used
        const uint32_t sb = lds0 + ((kt + 1) & 1) * 2 * kOStage;
        int ra[4], rb[4];
        tn_rows(wv, lane, (kt + 1) * BK, t.m_g, t.row0, nullptr, ra);
        if (kt == 1) {
#pragma unroll
          for (int j = 0; j < 4; ++j) rb[j] = rB2[j];
        } else {
          tn_rows(wv, lane, (kt + 1) * BK, t.m_g, t.row0, gather, rb);
          wait_vm<0>();  // only these index reads are outstanding here
        }
        tn_issue(al, sb, wv, M, ra);
        tn_issue(bl, sb + kOStage, wv, N, rb);
      }
      const uint32_t aoff = (kt & 1) * 2 * kOStage + wm * 128;
      const uint32_t boff = (kt & 1) * 2 * kOStage + kOStage + 2 * wn * 128;
#pragma unroll
      for (int s = 0; s < BK / 16; ++s) {
        bf16x8 b[4];
#pragma unroll
        for (int n = 0; n < 4; ++n)
          b[n] = frag_ko(lo_f[n & 1] + boff + (n >> 1) * 128 + s * 16 * kORow);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
          const bf16x8 a = frag_ko(lo_f[mi] + aoff + s * 16 * kORow);
#pragma unroll
          for (int n = 0; n < 4; ++n)  // output row = A column, 4 consecutive n per lane
            acc[mi][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[n], a, acc[mi][n], 0, 0, 0);
        }
      }
    }

    // the next tile: its rows, then (LDS free) its first two stages
    const int next = tile + per_xcd;
    const bool has_next = next < end;
    const TnTile cur = t;
    __syncthreads();  // every wave is done with this tile's LDS
    if (has_next) {
      t = tn_tile(next, mtn, ntn, offsets);
      tn_setup(al, A, R, M, t.i0, lane);
      tn_setup(bl, B, brows, N, t.n0, lane);
      tn_prefetch(t, al, bl, wv, lane, lds0, M, N, gather, rB2);
    }

    // this tile's stores: lane holds output row i (its MFMA column) and 4 consecutive n
    const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
        Cw + (int64_t)cur.g * M * N, (short)0, (int)out_bytes, 0x00020000);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
      const int row = cur.i0 + 64 * wm + 32 * mi + (lane & 31);
#pragma unroll
      for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = cur.n0 + 128 * wn + 32 * n + 8 * j + 4 * (lane >> 5);
          const uint32_t off = (row < M && col < N)
                                   ? ((uint32_t)row * (uint32_t)N + (uint32_t)col) * 4u
                                   : out_bytes;  // past the end: dropped
          const f32x4 v = {acc[mi][n][4 * j], acc[mi][n][4 * j + 1], acc[mi][n][4 * j + 2],
                           acc[mi][n][4 * j + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(v, crs, off, 0, 0);
        }
    }
    if (!has_next) break;
    tile = next;
  }
}

// ---------------------------------------------------------------------------
// fp32 path (small problems): one thread per output element.
// ---------------------------------------------------------------------------
// dgrad; group of row r found by binary search over offsets
__global__ void k_nn_f32(const float* __restrict__ A, const float* __restrict__ B,
                         float* __restrict__ C, const float* __restrict__ au,
                         const int32_t* __restrict__ offsets, int NG, int Kd, int N, int I,
                         int swiglu_bwd, int64_t R) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= R * N) return;
  const int64_t r = q / N;
  const int n = (int)(q % N);
  int lo = 0, hi = NG;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= r) lo = mid;
    else hi = mid;
  }
  const float* b = B + (int64_t)lo * Kd * N;
  float acc = 0.0f;
  for (int k = 0; k < Kd; ++k) acc = __builtin_fmaf(A[r * Kd + k], b[(int64_t)k * N + n], acc);
  if (swiglu_bwd) {
    const float a = au[r * 2 * I + n], u = au[r * 2 * I + I + n];
    const float sg = 1.0f / (1.0f + __expf(-a));
    C[r * 2 * I + n] = acc * u * (sg * (1.0f + a * (1.0f - sg)));
    C[r * 2 * I + I + n] = acc * (a * sg);
  } else {
    C[r * N + n] = acc;
  }
}

// wgrad
__global__ void k_tn_f32(const float* __restrict__ A, const float* __restrict__ B,
                         const int32_t* __restrict__ gather, float* __restrict__ Cw,
                         const int32_t* __restrict__ offsets, int NG, int M, int N) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= (int64_t)NG * M * N) return;
  const int g = (int)(q / ((int64_t)M * N));
  const int64_t rem = q % ((int64_t)M * N);
  const int i = (int)(rem / N), n = (int)(rem % N);
  float acc = 0.0f;
  for (int r = offsets[g]; r < offsets[g + 1]; ++r) {
    const int64_t br = gather ? gather[r] : r;
    acc = __builtin_fmaf(A[(int64_t)r * M + i], B[br * N + n], acc);
  }
  Cw[q] = acc;
}

int bwd_grid(int cus) {
  const int p = (cus / kXcds) * kXcds;
  return p < kXcds ? kXcds : p;
}

}  // namespace

hipError_t launch_ffn_bwd_input(const Dims& d, const int32_t* offsets, const void* w13,
                                const void* w2, const void* au, const void* dys, void* dau,
                                void* dxs, hipStream_t st) {
  const int NG = d.E + d.S;
  const int64_t R = d.R();
  const int H = d.H, I = d.I;
  if (d.expert == MOE_BF16) {
    const int grid = bwd_grid(device_cu_count());
    // dh -> [da|du]
    hipLaunchKernelGGL(k_gemm_nn_bf16<true>, dim3(grid), dim3(512), 0, st,
                       static_cast<const uint16_t*>(dys), static_cast<const uint16_t*>(w2),
                       static_cast<uint16_t*>(dau), static_cast<const uint16_t*>(au), offsets,
                       NG, H, I, I);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // dx_sorted = [da|du] W13
    hipLaunchKernelGGL(k_gemm_nn_bf16<false>, dim3(grid), dim3(512), 0, st,
                       static_cast<const uint16_t*>(dau), static_cast<const uint16_t*>(w13),
                       static_cast<uint16_t*>(dxs), nullptr, offsets, NG, 2 * I, H, I);
    return hipGetLastError();
  }
  if (d.expert == MOE_F32) {
    auto blocks = [](int64_t n) { return dim3((unsigned)((n + 255) / 256)); };
    hipLaunchKernelGGL(k_nn_f32, blocks(R * I), dim3(256), 0, st,
                       static_cast<const float*>(dys), static_cast<const float*>(w2),
                       static_cast<float*>(dau), static_cast<const float*>(au), offsets, NG, H, I,
                       I, 1, R);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_nn_f32, blocks(R * H), dim3(256), 0, st,
                       static_cast<const float*>(dau), static_cast<const float*>(w13),
                       static_cast<float*>(dxs), nullptr, offsets, NG, 2 * I, H, I, 0, R);
    return hipGetLastError();
  }
  return hipErrorNotSupported;
}

hipError_t launch_ffn_bwd_weight(const Dims& d, const void* x, const int32_t* gather,
                                 const int32_t* offsets, const void* h, const void* dys,
                                 const void* dau, float* dw13, float* dw2, hipStream_t st) {
  const int NG = d.E + d.S;
  const int64_t R = d.R();
  const int H = d.H, I = d.I;
  if (d.expert == MOE_BF16) {
    const int grid = bwd_grid(device_cu_count());
    // dW2 = dY^T h
    hipLaunchKernelGGL(k_gemm_tn_bf16, dim3(grid), dim3(512), 0, st,
                       static_cast<const uint16_t*>(dys), static_cast<const uint16_t*>(h),
                       nullptr, R, dw2, offsets, NG, H, I);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // dW13 = [da|du]^T x
    hipLaunchKernelGGL(k_gemm_tn_bf16, dim3(grid), dim3(512), 0, st,
                       static_cast<const uint16_t*>(dau), static_cast<const uint16_t*>(x),
                       gather, gather ? d.T : R, dw13, offsets, NG, 2 * I, H);
    return hipGetLastError();
  }
  if (d.expert == MOE_F32) {
    auto blocks = [](int64_t n) { return dim3((unsigned)((n + 255) / 256)); };
    hipLaunchKernelGGL(k_tn_f32, blocks((int64_t)NG * H * I), dim3(256), 0, st,
                       static_cast<const float*>(dys), static_cast<const float*>(h), nullptr,
                       dw2, offsets, NG, H, I);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_tn_f32, blocks((int64_t)NG * 2 * I * H), dim3(256), 0, st,
                       static_cast<const float*>(dau), static_cast<const float*>(x), gather, dw13,
                       offsets, NG, 2 * I, H);
    return hipGetLastError();
  }
  return hipErrorNotSupported;
}

}  // namespace moe
