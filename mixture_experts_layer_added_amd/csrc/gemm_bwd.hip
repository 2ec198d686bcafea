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
constexpr int kRing = 3 * (160 * kARow + kOStage);  // 156 KiB: 3 stages up to 160 A rows

__device__ __forceinline__ float silu_f(float a) { return a / (1.0f + __expf(-a)); }

// K-inner operand (rows of 128 B): chunk slots xor-swizzled by (row >> 1) & 7.
__device__ __forceinline__ int swz_a(int r, int c) { return r * kARow + ((c ^ (r >> 1)) & 7) * 16; }

// K-outer stages keep k-rows of 512 bytes (256 columns) with 16-byte chunk c of k-row r
// at slot c ^ 4 (r & 3).  In each 16-lane group g of a fragment read
// (ds_read_b64_tr_b16), source lane j reads k-row 8 (g >> 1) + j / 4 and 4 columns
// from 16 (g & 1) + 4 (j & 3), so a half-wave touches 4 k-rows x 4 chunks = 16 distinct
// slots of a 256-byte bank window.  For fragment columns nb with (nb / 32) & 3 == p the
// read of k-step s (16 k-rows), half hi (k + 4) sits at
//   tn_lane_off(lane, p) + (nb / 128) * 256 + s * 8192 + hi * 2048,
// constants the compiler folds into the read's offset field.
__device__ __forceinline__ uint32_t tn_lane_off(int lane, int p) {
  const int g = lane >> 4, j = lane & 15, i = j >> 2;
  const int row = 8 * (g >> 1) + i;
  const int c = 4 * p + 2 * (g & 1) + ((j & 3) >> 1);
  return (uint32_t)(row * kORow + ((c ^ (4 * i)) << 4) + (j & 1) * 8);
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

// One k-stage of a K-outer operand (the weights of the dgrad GEMMs, loaded
// non-temporally: each weight tile is streamed once): k-rows k0 .. k0+63 (those >=
// krows read as zeros) of columns col0 .. col0+255 (those >= ncols read as zeros) of a row-major matrix
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
    const int c = slot ^ (4 * (r & 3));
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
    load16_to_lds_nt(L.rsrc, lds_stage + (4 * wv + j) * 1024, voff);  // weights: streamed
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
  // the cost prefix is only needed for the XCD split, before the first tile's loads
  // overwrite the ring (they follow a barrier), so it borrows the ring's memory
  long long* s_cost = reinterpret_cast<long long*>(smem);
  static_assert(sizeof(long long) * (kMaxGroups + 1) <= kRing, "cost prefix fits the ring");
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
    // three stages when an A stage of the rows rounded up to 16 fits three times
    // (up to 160 rows), else two of nA*64 rows; A rows past the expert's end that are not
    // loaded only feed output rows that are not stored
    const int nA = (m_rows + 63) >> 6;
    const int rA16 = (m_rows + 15) & ~15;
    const bool three = 3 * (rA16 * kARow + kOStage) <= kRing;
    const int rowsA = three ? rA16 : nA * 64;
    const int sA = rowsA * kARow;
    const int sStage = sA + kOStage;
    const int nst = three ? 3 : 2;
    const int nAw = __builtin_amdgcn_readfirstlane((rowsA - 8 * wv + 63) >> 6);
    const int per_stage = nAw + 4;

    const i32x4 arsrc = buffer_rsrc(A + (int64_t)(row0 + m0) * Kd, (uint32_t)m_rows * Kd * 2);
    uint32_t aoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) aoff[i] = (uint32_t)((64 * i + 8 * wv + lrow) * Kd + lchunk * 8) * 2;
    KOuterLoader bl;
    kouter_setup(bl, B + (int64_t)tl.g * Kd * N, Kd, N, n0, N, lane, wv);
    const uint32_t ldsw = lds0 + 8 * wv * kARow;
    uint32_t lo_b[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) lo_b[p] = lds0 + tn_lane_off(lane, p);

#define NN_STAGE_LOAD(kt, st)                                                         \
  {                                                                                   \
    const uint32_t sa_ = ldsw + (st) * sStage;                                        \
    const uint32_t ko_ = (uint32_t)(kt) * kARow;                                      \
    if (nAw > 0) load16_to_lds(arsrc, sa_, aoff[0] + ko_);                            \
    if (nAw > 1) load16_to_lds(arsrc, sa_ + 64 * kARow, aoff[1] + ko_);               \
    if (nAw > 2) load16_to_lds(arsrc, sa_ + 128 * kARow, aoff[2] + ko_);              \
    if (nAw > 3) load16_to_lds(arsrc, sa_ + 192 * kARow, aoff[3] + ko_);              \
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
        const uint32_t boff = st * sStage + sA + wn * 256;
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
          const int c = 2 * s + kq;
          bf16x8 b[4];
#pragma unroll
          for (int n = 0; n < 4; ++n)
            b[n] = frag_ko(lo_b[n] + boff + s * 16 * kORow);
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
              __builtin_nontemporal_store(
                  f32_to_bf16_bits(dh * u * (sg * (1.0f + a * (1.0f - sg)))), C + r * 2 * I + col);
              __builtin_nontemporal_store(f32_to_bf16_bits(dh * (a * sg)), C + r * 2 * I + I + col);
            } else {
              __builtin_nontemporal_store(f32_to_bf16_bits(dh), C + r * N + col);
            }
          }
        }
    }
  }
}

// ---------------------------------------------------------------------------
// wgrad:  Cw[g][i, n] = sum over the rows r of group g of A[r, i] B[r, n]  (fp32 out)
//   A: [R, M] rows; B: [R, N] rows (or, with gather, [T, N] rows gather[r]).
// Tiles (group, i-tile, n-tile) of 256 x 256; both operands K-outer.  Groups without
// rows write zeros.
//
// With ~128 rows per expert a tile is little MFMA work and 256 KiB of fp32 output, so
// the kernel is bound by HBM writes, and the loads must not wait behind the stores.
//  * Stage k-rows are 512 bytes (256 columns) with 16-byte chunk c of k-row r at slot
//    c ^ 4 (r & 3): the 32 lanes of a half-wave fragment read (4 k-rows x 4 chunks)
//    touch 16 distinct slots of a 256-byte bank window.
//  * The k-stages (32 rows of both operands, 32 KiB) of all the workgroup's tiles form
//    one stream: stage q is loaded kTAhead steps before it is computed, into LDS buffer
//    q % kTRing, across tile boundaries.  With gather, the 32 row indices of stage q
//    are themselves loaded into LDS kTAhead steps before the stage.
//  * Vector memory operations complete in issue order, and every step issues the same
//    number of loads (dummy ones past the end of the stream), so the wait for stage q
//    is "at most (kTAhead-1) steps of loads plus the stores issued since are
//    outstanding"; stores of a finished tile drain while later stages load.
//  * The MFMA takes the row operand second, so a lane holds 4 consecutive outputs of
//    one row; the tile goes out through the LDS buffer of its last stage as 32 stores
//    of 16 bytes per lane that each cover 8 whole 128-byte rows (partial-line writes
//    make the L2 fetch the rest of the line first), every one issued (lanes outside
//    the matrix write past the end of the buffer, which drops them).
// ---------------------------------------------------------------------------
constexpr int kTK = 32;                // rows of each operand per stage
constexpr int kTOp = kTK * kORow;      // 16 KiB: one operand of one stage
constexpr int kTRing = 4;              // stages held in LDS
constexpr int kTAhead = 3;             // stages in flight ahead of the one computed
constexpr int kTIdx = 8;               // gather-index slots of 64 ints (> kTAhead)
constexpr int kTStores = 32;           // 16-byte stores per lane per tile
constexpr int kCpolNT = 2;             // cache-policy bit of a buffer store: non-temporal
static_assert(kTAhead < kTRing, "the buffer refilled at a step was computed the step before");

struct TnCursor {
  int q;                         // position in the stage stream
  int tile;                      // >= end: past the end of the stream
  int kt, nk, g, i0, n0, row0, m_g;
};

__device__ __forceinline__ void tn_tile_params(TnCursor& c, int tile, int mtn, int ntn,
                                               const int* s_off) {
  c.tile = tile;
  c.kt = 0;
  c.g = __builtin_amdgcn_readfirstlane(tile / (mtn * ntn));
  const int rem = tile - c.g * mtn * ntn;
  c.i0 = __builtin_amdgcn_readfirstlane(rem / ntn) * BM;
  c.n0 = __builtin_amdgcn_readfirstlane(rem % ntn) * BN;
  c.row0 = __builtin_amdgcn_readfirstlane(s_off[c.g]);
  c.m_g = __builtin_amdgcn_readfirstlane(s_off[c.g + 1]) - c.row0;
  c.nk = (c.m_g + kTK - 1) / kTK;
}

// first stage at or after tile `from` (tiles without rows are skipped)
__device__ __forceinline__ void tn_seek(TnCursor& c, int from, int end, int step, int mtn,
                                        int ntn, const int* s_off) {
  for (int t = from; t < end; t += step) {
    tn_tile_params(c, t, mtn, ntn, s_off);
    if (c.nk > 0) return;
  }
  c.tile = end;
}

__device__ __forceinline__ void tn_advance(TnCursor& c, int end, int step, int mtn, int ntn,
                                           const int* s_off) {
  ++c.q;
  if (c.tile >= end) return;
  if (++c.kt < c.nk) return;
  tn_seek(c, c.tile + step, end, step, mtn, ntn, s_off);
}

// LDS column offset (bytes within a 512-byte k-row) and matrix column of this lane's
// 16 bytes for load instruction j; k-row of instruction j is 2 (2 wv + j) + lane / 32.
__device__ __forceinline__ int tn_chunk(int j, int lane) {
  const int r = 2 * j + (lane >> 5);  // k-row mod 4
  return (lane & 31) ^ (4 * (r & 3));
}


// the 32 gather indices of stage x into its 256-byte slot (lanes 32-63 fill the upper
// half of the slot with zeros)
template <bool kGather>
__device__ __forceinline__ void tn_issue_index(const TnCursor& x, bool live, i32x4 grs,
                                               uint32_t lds_idx, int lane) {
  if (!kGather) return;
  uint32_t voff = 0x7ffffff0u;
  const int kr = x.kt * kTK + lane;
  if (live && lane < kTK && kr < x.m_g) voff = (uint32_t)(x.row0 + kr) * 4u;
  load4_to_lds(grs, __builtin_amdgcn_readfirstlane(lds_idx + (x.q % kTIdx) * 256), voff);
}

template <bool kGather>
__device__ __forceinline__ void tn_issue_stage(const TnCursor& d, bool live, i32x4 ars, i32x4 brs,
                                               uint32_t lds0, const int* s_idx, int wv, int lane,
                                               int M, int N) {
  const uint32_t buf = __builtin_amdgcn_readfirstlane(lds0 + (d.q % kTRing) * 2 * kTOp);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int kr = d.kt * kTK + 2 * (2 * wv + j) + (lane >> 5);
    const bool row_ok = live && kr < d.m_g;
    const int c8 = 8 * tn_chunk(j, lane);
    uint32_t va = 0x7ffffff0u, vb = 0x7ffffff0u;
    if (row_ok && d.i0 + c8 < M) va = ((uint32_t)(d.row0 + kr) * (uint32_t)M + d.i0 + c8) * 2u;
    if (row_ok && d.n0 + c8 < N) {
      const int brow = kGather ? s_idx[(d.q % kTIdx) * 64 + kr - d.kt * kTK] : d.row0 + kr;
      vb = ((uint32_t)brow * (uint32_t)N + d.n0 + c8) * 2u;
    }
    load16_to_lds(ars, buf + (2 * wv + j) * 1024, va);
    load16_to_lds(brs, buf + kTOp + (2 * wv + j) * 1024, vb);
  }
}

template <bool kGather>
__device__ __forceinline__ void tn_wait(int b) {
  constexpr int base = (kTAhead - 1) * (4 + (kGather ? 1 : 0));
  if (b == 0) wait_vm<base>();
  else wait_vm<base + kTStores>();  // two or more batches: waits for more than it needs
}

// Output of one tile.  Each wave's 64 x 128 block goes out as 8 sub-blocks of 32 x 32:
// the accumulators (lane = output row, 4 consecutive columns) are written to the wave's
// 4 KiB of `stage` (a free LDS buffer) and read back as 8 rows x 8 chunks of 16 bytes,
// so every store writes 8 whole 128-byte rows.  Chunk c of row r sits at slot
// c ^ (r & 7).  32 stores per lane; lanes outside the matrix write past its end
// (dropped).  zero: store zeros without staging (tiles of groups without rows).
__device__ __forceinline__ void tn_store(float* __restrict__ Cw, const f32x16 (&acc)[2][4],
                                         int g, int i0, int n0, int M, int N, int wm, int wn,
                                         int lane, char* stage, int wv, bool zero) {
  const uint32_t out_bytes = (uint32_t)M * (uint32_t)N * 4u;
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      Cw + (int64_t)g * M * N, (short)0, (int)out_bytes, 0x00020000);
  char* mine = stage + wv * 4096;
  const int wr = lane & 31;                  // row this lane writes
  const int rr = lane >> 3, rc = lane & 7;   // row (within 8) and chunk this lane reads
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      if (!zero) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = 2 * j + (lane >> 5);
          const f32x4 v = {acc[mi][n][4 * j], acc[mi][n][4 * j + 1], acc[mi][n][4 * j + 2],
                           acc[mi][n][4 * j + 3]};
          *reinterpret_cast<f32x4*>(mine + wr * 128 + ((c ^ (wr & 7)) << 4)) = v;
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 8 * q + rr;
        f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
        if (!zero) v = *reinterpret_cast<const f32x4*>(mine + r * 128 + ((rc ^ (r & 7)) << 4));
        const int row = i0 + 64 * wm + 32 * mi + r;
        const int col = n0 + 128 * wn + 32 * n + 4 * rc;
        const uint32_t off = (row < M && col < N)
                                 ? ((uint32_t)row * (uint32_t)N + (uint32_t)col) * 4u
                                 : out_bytes;  // past the end: dropped
        // non-temporal: the gradient is not read again here, and keeping it out of the
        // L2 keeps the operand rows there
        __builtin_amdgcn_raw_buffer_store_b128(v, crs, off, 0, kCpolNT);
      }
    }
}

template <bool kGather>
__global__ __launch_bounds__(512, 1) void k_gemm_tn_bf16(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
    const int32_t* __restrict__ gather, int64_t b_rows, float* __restrict__ Cw,
    const int32_t* __restrict__ offsets, int NG, int M, int N) {
  __shared__ __attribute__((aligned(1024))) char smem[kTRing * 2 * kTOp];  // 128 KiB
  __shared__ __attribute__((aligned(256))) int s_idx[kTIdx * 64];
  __shared__ int s_off[kMaxGroups + 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv >> 1, wn = wv & 1;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_offset(smem));
  const uint32_t lds_idx = __builtin_amdgcn_readfirstlane(lds_offset(s_idx));
  for (int i = tid; i <= NG; i += 512) s_off[i] = offsets[i];
  __syncthreads();
  const int mtn = (M + BM - 1) / BM, ntn = (N + BN - 1) / BN;
  const int ntiles = NG * mtn * ntn;
  const int64_t R = __builtin_amdgcn_readfirstlane(s_off[NG]);
  const i32x4 ars = buffer_rsrc(A, (uint32_t)(R * M * 2));
  const i32x4 brs = buffer_rsrc(B, (uint32_t)((kGather ? b_rows : R) * N * 2));
  const i32x4 grs = buffer_rsrc(gather, (uint32_t)(R * 4));

  const int P = gridDim.x, step = P / kXcds;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int chunk = (ntiles + kXcds - 1) / kXcds;
  const int end = min(ntiles, (xcd + 1) * chunk);
  const int begin = xcd * chunk + slot;
  if (begin >= end) return;

  uint32_t lo4[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) lo4[p] = lds0 + tn_lane_off(lane, p);
  const uint32_t la0 = ((wm & 1) ? lo4[2] : lo4[0]) + (wm >> 1) * 256;
  const uint32_t la1 = ((wm & 1) ? lo4[3] : lo4[1]) + (wm >> 1) * 256;
  f32x16 acc[2][4];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mi][n][i] = 0.0f;

  // tiles of groups without rows before the first stage: zeros, before any load
  TnCursor c;
  c.q = 0;
  for (int t = begin; t < end; t += step) {
    tn_tile_params(c, t, mtn, ntn, s_off);
    if (c.nk > 0) break;
    tn_store(Cw, acc, c.g, c.i0, c.n0, M, N, wm, wn, lane, smem, wv, true);
    c.tile = end;
  }
  if (c.tile >= end || c.nk == 0) return;
  TnCursor d = c, x = c;

  // prologue: indices of the first kTAhead stages, then kTAhead steps of loads
  if (kGather) {
    for (int k = 0; k < kTAhead; ++k) {
      tn_issue_index<kGather>(x, x.tile < end, grs, lds_idx, lane);
      tn_advance(x, end, step, mtn, ntn, s_off);
    }
    wait_vm<0>();
    __syncthreads();
  }
  for (int k = 0; k < kTAhead; ++k) {
    tn_issue_index<kGather>(x, x.tile < end, grs, lds_idx, lane);
    tn_advance(x, end, step, mtn, ntn, s_off);
    tn_issue_stage<kGather>(d, d.tile < end, ars, brs, lds0, s_idx, wv, lane, M, N);
    tn_advance(d, end, step, mtn, ntn, s_off);
  }

  int h0 = 0, h1 = 0, h2 = 0;  // store batches issued at the ends of the last 3 steps
  for (;;) {
    tn_wait<kGather>(h0 + h1 + h2);
    __syncthreads();
    // refill the buffer computed at the previous step
    tn_issue_index<kGather>(x, x.tile < end, grs, lds_idx, lane);
    tn_advance(x, end, step, mtn, ntn, s_off);
    tn_issue_stage<kGather>(d, d.tile < end, ars, brs, lds0, s_idx, wv, lane, M, N);
    tn_advance(d, end, step, mtn, ntn, s_off);

    const uint32_t aoff = (c.q % kTRing) * 2 * kTOp;
    const uint32_t boff = (c.q % kTRing) * 2 * kTOp + kTOp + wn * 256;
#pragma unroll
    for (int s = 0; s < kTK / 16; ++s) {
      bf16x8 b[4];
#pragma unroll
      for (int n = 0; n < 4; ++n) b[n] = frag_ko(lo4[n] + boff + s * 16 * kORow);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const bf16x8 a = frag_ko((mi ? la1 : la0) + aoff + s * 16 * kORow);
#pragma unroll
        for (int n = 0; n < 4; ++n)  // output row = A column, 4 consecutive n per lane
          acc[mi][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[n], a, acc[mi][n], 0, 0, 0);
      }
    }

    int batches = 0;
    if (c.kt + 1 == c.nk) {  // last stage of the tile
      // its buffer is free once every wave has computed it (it is refilled only after
      // the next step's barrier): stage the output through it
      __syncthreads();
      tn_store(Cw, acc, c.g, c.i0, c.n0, M, N, wm, wn, lane,
               smem + (c.q % kTRing) * 2 * kTOp, wv, false);
      ++batches;
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int n = 0; n < 4; ++n)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[mi][n][i] = 0.0f;
      // following tiles of groups without rows: zeros
      int t = c.tile + step;
      for (; t < end; t += step) {
        tn_tile_params(c, t, mtn, ntn, s_off);
        if (c.nk > 0) break;
        tn_store(Cw, acc, c.g, c.i0, c.n0, M, N, wm, wn, lane, smem, wv, true);
        ++batches;
      }
      if (t >= end) {
        wait_vm<0>();  // no load into LDS may outlive the workgroup
        break;
      }
      ++c.q;
    } else {
      ++c.q;
      ++c.kt;
    }
    h2 = h1;
    h1 = h0;
    h0 = batches;
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
    hipLaunchKernelGGL(k_gemm_tn_bf16<false>, dim3(grid), dim3(512), 0, st,
                       static_cast<const uint16_t*>(dys), static_cast<const uint16_t*>(h),
                       nullptr, R, dw2, offsets, NG, H, I);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // dW13 = [da|du]^T x
    if (gather)
      hipLaunchKernelGGL(k_gemm_tn_bf16<true>, dim3(grid), dim3(512), 0, st,
                         static_cast<const uint16_t*>(dau), static_cast<const uint16_t*>(x),
                         gather, d.T, dw13, offsets, NG, 2 * I, H);
    else
      hipLaunchKernelGGL(k_gemm_tn_bf16<false>, dim3(grid), dim3(512), 0, st,
                         static_cast<const uint16_t*>(dau), static_cast<const uint16_t*>(x),
                         nullptr, R, dw13, offsets, NG, 2 * I, H);
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
