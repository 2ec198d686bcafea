// Expert FFNs as grouped GEMMs over the permuted rows (one group per routed expert,
// plus the shared expert as the last group):
//   GEMM1 + SwiGLU:  h = silu(x W13[g][0:I]^T) * (x W13[g][I:2I]^T)
//   GEMM2:           Y = h W2[g]^T
// Each expert's weights stream from HBM once per row tile; the tile schedule (built on
// the device from the permute offsets, split over the XCDs by cost) is in schedule.h.
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
                                                  const int32_t* __restrict__ offsets,
                                                  const int32_t* __restrict__ gather,
                                                  float* __restrict__ au, int NG,
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
    const int arow = row0 + min(m0 + lr, m_g - 1);
    const float* ap = A + (int64_t)(gather ? gather[arow] : arow) * Kd + lk;
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
        for (int j = 0; j < 2; ++j) {
          const int col = tl.n_idx * 32 + tx * 2 + j;
          cp[col] = silu(acc[i][j]) * acc[i][2 + j];
          if (au) {  // gate and up pre-activations, kept for the backward
            au[(int64_t)(row0 + m) * 2 * half + col] = acc[i][j];
            au[(int64_t)(row0 + m) * 2 * half + half + col] = acc[i][2 + j];
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) cp[tl.n_idx * BN + tx * 4 + j] = acc[i][j];
      }
    }
    __syncthreads();
  });
}

// ---------------------------------------------------------------------------
// bf16 path: MFMA 32x32x16 (bf16 in, fp32 accumulate).
//
// Every weight byte comes from HBM once, while an expert's activation tile is re-read
// (from L2) by each of its column tiles.  The tile is shaped for that:
//   - 256 rows: one tile holds all rows of an expert (73..193 at the V3 shape), so
//     the weights never stream twice;
//   - 256 weight rows (GEMM1: 128 gate + the matching 128 up rows): one activation
//     read serves 256 weight rows;
//   - 64-deep k steps: every row of a step is one full 128-byte line (narrower row
//     segments cost far more memory-pipeline time per byte on this GPU).
// Operands go from memory straight into LDS (buffer loads with the LDS destination
// bit, no register staging).  Weight loads and output stores are non-temporal: a
// weight tile is read only by the few workgroups working on it at the same moment and
// outputs are not read again here, so the L2 is left to the activation rows that
// every column tile of an expert re-reads.  The LDS ring is shaped per tile: experts of
// up to 160 rows get three stages (A part = rows rounded up to 16), so two steps are in
// flight while one is multiplied; larger ones two stages of ceil(rows/64)*64 A rows.
// Activation rows past the expert's end are read through a buffer descriptor sized
// to the expert's rows, so they arrive as zeros with no memory traffic.
// One workgroup of 8 waves per CU: wave w owns rows 64*(w/2) .. +63 and columns
// 128*(w%2) .. +127 (2 x 4 MFMA tiles), so the waves with rows sit on all four SIMDs;
// MFMAs of 32-row sub-tiles past the expert's rows are skipped (wave-uniform).
//   kSwiglu: wave column wn owns gate rows 64wn..64wn+63 of the tile and the matching
//   up rows, so each lane holds the gate and up value of the same h element and
//   applies SwiGLU in registers.
// Operand layout (32x32x16): lane l supplies row (l%32), k = 8*(l/32)..+7 of the first
// operand and column (l%32), the same k of the second; result element i of lane l is
// row 8*(i/4) + 4*(l/32) + i%4, column l%32.  The gate/up kernel passes the activation
// fragment first (a lane's results: one output column, 16 rows); the down kernel passes
// the weight fragment first, so a lane's results are one activation row (l%32) and four
// consecutive output columns per group of four elements.  The down kernel's epilogue
// stages each wave's 64 x 128 block of Y in the ring (16 KiB per wave, once every wave is
// done with it) and stores it back with 16-byte lanes, so every store instruction writes
// whole 128-byte lines.
// ---------------------------------------------------------------------------
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kRowBytes = BK * 2;               // one row of one stage: a full 128-B line
constexpr int kBStage = BN * kRowBytes;         // 32 KiB
constexpr int kRing = 3 * (160 * kRowBytes + kBStage);  // 156 KiB: 3 stages up to 160 A rows

// byte offset of (row, 16-byte k-chunk c) inside an operand stage: rows of 128 B,
// chunk slots xor-swizzled by (row >> 1) & 7 so 16 consecutive rows at one chunk hit
// 16 distinct bank groups
__device__ __forceinline__ int swz(int r, int c) { return r * kRowBytes + ((c ^ (r >> 1)) & 7) * 16; }

constexpr int kStgBytes = 64 * 256;  // one wave's staged outputs: 64 rows x 256 bytes
static_assert(8 * kStgBytes <= kRing, "the eight waves' staging areas fit the ring");

// gather != nullptr: row r of the permuted order is row gather[r] of A (a_rows rows),
// so the activation rows are read from the unpermuted input.
template <bool kSwiglu>
__global__ __launch_bounds__(512, 1) void k_gemm_bf16(const uint16_t* __restrict__ A,
                                                      const uint16_t* __restrict__ B,
                                                      uint16_t* __restrict__ C,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ gather,
                                                      uint16_t* __restrict__ au,
                                                      int a_rows, int NG, int Kd, int Nrows,
                                                      int Nout, int half) {
  __shared__ __attribute__((aligned(1024))) char smem[kRing];
  __shared__ int mt_start[kMaxGroups + 1];
  // the cost prefix is only needed for the XCD split below, before the first tile's
  // loads overwrite the ring (they follow a barrier), so it borrows the ring's memory
  long long* s_cost = reinterpret_cast<long long*>(smem);
  static_assert(sizeof(long long) * (kMaxGroups + 1) <= kRing, "cost prefix fits the ring");
  build_schedule(offsets, NG, BM, mt_start);
  const int nt = kSwiglu ? half / 128 : (Nout + BN - 1) / BN;
  build_costs(offsets, mt_start, NG, BM, nt, s_cost);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv >> 1, wn = wv & 1;
  const int nk = Kd / BK;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_offset(smem));
  // loader: instruction i of wave wv fills rows 64i + 8wv .. +7 of an operand stage;
  // lane l writes row 64i + 8wv + (l>>3), slot l&7, which holds k-chunk
  // (l&7) ^ ((row>>1)&7); (row>>1)&7 = (4*(wv&1) + (l>>4)) & 7
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
    const bool w_on = 64 * wm < m_rows && (kSwiglu || tl.n_idx * BN + 128 * wn < Nout);
    const bool w_sub1 = 64 * wm + 32 < m_rows;
    // ring shape of this tile: three stages when an A stage of the rows rounded up to 16
    // fits three times (experts of up to 160 rows), else two stages of nA*64 rows.  A
    // rows past the expert's end that are not loaded hold stale data: their products
    // land in output rows that are not stored.
    const int nA = (m_rows + 63) >> 6;
    const int rA16 = (m_rows + 15) & ~15;
    const bool three = 3 * (rA16 * kRowBytes + kBStage) <= kRing;
    const int rowsA = three ? rA16 : nA * 64;
    const int sA = rowsA * kRowBytes;
    const int sStage = sA + kBStage;
    const int nst = three ? 3 : 2;
    // A load instructions of this wave (instruction i covers rows 64i + 8wv .. +7)
    const int nAw = __builtin_amdgcn_readfirstlane((rowsA - 8 * wv + 63) >> 6);
    const int per_stage = nAw + 4;  // loads per thread per stage

    // A rows past the expert's end and B rows past Nout read as zeros (range check)
    const i32x4 arsrc =
        gather ? buffer_rsrc(A, (uint32_t)a_rows * Kd * 2)
               : buffer_rsrc(A + (int64_t)(row0 + m0) * Kd, (uint32_t)m_rows * Kd * 2);
    const i32x4 brsrc = buffer_rsrc(B + (int64_t)tl.g * Nrows * Kd, (uint32_t)Nrows * Kd * 2);
    uint32_t aoff[4], boff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 64 * i + 8 * wv + lrow;
      if (gather)
        aoff[i] = r < m_rows ? (uint32_t)(gather[row0 + m0 + r] * Kd + lchunk * 8) * 2 : 0x7ffffff0u;
      else
        aoff[i] = (uint32_t)(r * Kd + lchunk * 8) * 2;
      int br;
      if (kSwiglu) br = r < 128 ? tl.n_idx * 128 + r : half + tl.n_idx * 128 + (r - 128);
      else br = tl.n_idx * BN + r;
      boff[i] = br < Nrows ? (uint32_t)(br * Kd + lchunk * 8) * 2 : 0x7ffffff0u;
    }
    const uint32_t ldsw = lds0 + 8 * wv * kRowBytes;

#define STAGE_LOAD(kt, st)                                                            \
  {                                                                                   \
    const uint32_t sa_ = ldsw + (st) * sStage;                                        \
    const uint32_t ko_ = (uint32_t)(kt) * kRowBytes;                                  \
    if (nAw > 0) load16_to_lds(arsrc, sa_, aoff[0] + ko_);                              \
    if (nAw > 1) load16_to_lds(arsrc, sa_ + 64 * kRowBytes, aoff[1] + ko_);             \
    if (nAw > 2) load16_to_lds(arsrc, sa_ + 128 * kRowBytes, aoff[2] + ko_);            \
    if (nAw > 3) load16_to_lds(arsrc, sa_ + 192 * kRowBytes, aoff[3] + ko_);            \
    load16_to_lds_nt(brsrc, sa_ + sA, boff[0] + ko_);                                      \
    load16_to_lds_nt(brsrc, sa_ + sA + 64 * kRowBytes, boff[1] + ko_);                     \
    load16_to_lds_nt(brsrc, sa_ + sA + 128 * kRowBytes, boff[2] + ko_);                    \
    load16_to_lds_nt(brsrc, sa_ + sA + 192 * kRowBytes, boff[3] + ko_);                    \
  }

    f32x16 acc[2][4];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mi][n][i] = 0.0f;
    // LDS rows read by this lane: A rows 64wm + 32mi + lane%32; B rows per sub-tile n
    int brow[4];
#pragma unroll
    for (int n = 0; n < 4; ++n)
      brow[n] = (kSwiglu ? ((n & 1) * 128 + 64 * wn + 32 * (n >> 1)) : (128 * wn + 32 * n)) +
                (lane & 31);
    const int arow0 = 64 * wm + (lane & 31), arow1 = arow0 + 32;

    __syncthreads();  // previous tile's LDS reads are done before the ring is refilled
    STAGE_LOAD(0, 0)
    if (nst == 3 && nk > 1) STAGE_LOAD(1, 1)
    int st = 0;
    for (int kt = 0; kt < nk; ++kt) {
      // stages issued beyond kt: nst-2 (all but the tail)
      wait_vmcnt(min(nst - 2, nk - 1 - kt) * per_stage);
      __syncthreads();
      if (kt + nst - 1 < nk) {
        int sn = st + nst - 1;
        if (sn >= nst) sn -= nst;
        STAGE_LOAD(kt + nst - 1, sn)
      }
      if (w_on) {
        const char* as = smem + st * sStage;
        const char* bs = as + sA;
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
          const int c = 2 * s + kq;
          bf16x8 b[4];
#pragma unroll
          for (int n = 0; n < 4; ++n)
            b[n] = *reinterpret_cast<const bf16x8*>(bs + swz(brow[n], c));
          const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(as + swz(arow0, c));
#pragma unroll
          for (int n = 0; n < 4; ++n)
            acc[0][n] = kSwiglu
                            ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b[n], acc[0][n], 0, 0, 0)
                            : __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[n], a0, acc[0][n], 0, 0, 0);
          if (w_sub1) {
            const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(as + swz(arow1, c));
#pragma unroll
            for (int n = 0; n < 4; ++n)
              acc[1][n] = kSwiglu
                              ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b[n], acc[1][n], 0, 0, 0)
                              : __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[n], a1, acc[1][n], 0, 0, 0);
          }
        }
      }
      if (++st == nst) st = 0;
    }
#undef STAGE_LOAD

    if (kSwiglu) {
      // gate/up: h (and a, u) stored straight from the accumulators, 32 lanes writing
      // 64 contiguous bytes of a row per instruction (staging these through LDS measured
      // 0.6% slower for this launch)
      if (w_on) {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int m = 64 * wm + 32 * mi + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
            if (m >= m_rows) continue;
            uint16_t* cp = C + (int64_t)(row0 + m0 + m) * Nout;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const int col = tl.n_idx * 128 + 64 * wn + 32 * t + (lane & 31);
              __builtin_nontemporal_store(
                  f32_to_bf16_bits(silu(acc[mi][2 * t][i]) * acc[mi][2 * t + 1][i]), cp + col);
              if (au) {  // gate and up pre-activations, kept for the backward
                uint16_t* ap = au + (int64_t)(row0 + m0 + m) * 2 * half;
                ap[col] = f32_to_bf16_bits(acc[mi][2 * t][i]);
                ap[half + col] = f32_to_bf16_bits(acc[mi][2 * t + 1][i]);
              }
            }
          }
      }
    } else {
      // down: every wave is done with the ring's stages, whose memory then stages each
      // wave's 64 x 128 block of Y (16 KiB per wave) for whole-line stores.  Lane
      // columns 128wn + 32n + 8ig + 4(lane/32) .. +3 of the tile go to chunk 4n + ig.
      __syncthreads();
      if (w_on) {
        char* stg = smem + wv * kStgBytes;
        const int nrows = min(64, m_rows - 64 * wm);  // rows of this wave's block (>= 1)
        const int64_t orow = (int64_t)row0 + m0 + 64 * wm;
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int n = 0; n < 4; ++n)
#pragma unroll
            for (int ig = 0; ig < 4; ++ig) {
              const f32x16& v = acc[mi][n];
              stg256_put(stg, 32 * mi + (lane & 31), 4 * n + ig, lane >> 5,
                         pack4_bf16(v[4 * ig], v[4 * ig + 1], v[4 * ig + 2], v[4 * ig + 3]));
            }
        stg256_flush(stg, lane, nrows,
                     reinterpret_cast<char*>(C + orow * Nout + tl.n_idx * BN + 128 * wn),
                     (int64_t)Nout * 2);
      }
    }
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
                         const int32_t* offsets, const int32_t* gather, const void* w13,
                         const float* w13_scale, void* h, float* h_scale, hipStream_t st,
                         void* au) {
  const int NG = d.E + d.S;
  const int cus = device_cu_count();
  if (d.expert == MOE_F32) {
    hipLaunchKernelGGL(k_gemm_f32<true>, dim3(persistent_grid(cus, 4)), dim3(256), 0, st,
                       static_cast<const float*>(xs), static_cast<const float*>(w13),
                       static_cast<float*>(h), offsets, gather, static_cast<float*>(au), NG, d.H,
                       2 * d.I, d.I, d.I);
    return hipGetLastError();
  }
  if (d.expert == MOE_BF16) {
    int ng = NG;
    if (dense_shared(d)) {  // the shared expert's rows T*K .. T*K+T-1, token order
      ng = d.E;
      const int64_t r0 = d.T * d.K;
      const uint16_t* xa = static_cast<const uint16_t*>(xs) + (gather ? 0 : r0 * d.H);
      uint16_t* aua = au ? static_cast<uint16_t*>(au) + r0 * 2 * d.I : nullptr;
      const hipError_t e = launch_dense_swiglu_bf16(
          xa, static_cast<const uint16_t*>(w13) + (int64_t)d.E * 2 * d.I * d.H,
          static_cast<uint16_t*>(h) + r0 * d.I, aua, (int)d.T, d.H, d.I, st);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_gemm_bf16<true>, dim3(persistent_grid(cus, 1)), dim3(512), 0, st,
                       static_cast<const uint16_t*>(xs), static_cast<const uint16_t*>(w13),
                       static_cast<uint16_t*>(h), offsets, gather, static_cast<uint16_t*>(au),
                       (int)d.T, ng, d.H, 2 * d.I, d.I, d.I);
    return hipGetLastError();
  }
  return launch_fp8_up(d, xs, xs_scale, offsets, gather, w13, w13_scale, h, h_scale, st);
}

hipError_t launch_ffn_down(const Dims& d, const void* h, const float* h_scale,
                           const int32_t* offsets, const void* w2, const float* w2_scale, void* ys,
                           hipStream_t st) {
  const int NG = d.E + d.S;
  const int cus = device_cu_count();
  if (d.expert == MOE_F32) {
    hipLaunchKernelGGL(k_gemm_f32<false>, dim3(persistent_grid(cus, 4)), dim3(256), 0, st,
                       static_cast<const float*>(h), static_cast<const float*>(w2),
                       static_cast<float*>(ys), offsets, nullptr, nullptr, NG, d.I, d.H, d.H, 0);
    return hipGetLastError();
  }
  if (d.expert == MOE_BF16) {
    hipLaunchKernelGGL(k_gemm_bf16<false>, dim3(persistent_grid(cus, 1)), dim3(512), 0, st,
                       static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(w2),
                       static_cast<uint16_t*>(ys), offsets, nullptr, nullptr, 0, NG, d.I, d.H, d.H,
                       0);
    return hipGetLastError();
  }
  return launch_fp8_down(d, h, h_scale, offsets, w2, w2_scale, ys, st);
}

}  // namespace moe
