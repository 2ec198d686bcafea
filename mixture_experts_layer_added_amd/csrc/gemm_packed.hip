// Expert FFN grouped GEMMs (bf16) over expert weights stored in a pre-arranged
// ("packed") layout, so that each weight load instruction reads 1 KiB of contiguous
// memory straight into the registers the matrix instruction consumes:
//   GEMM1 + SwiGLU:  h = silu(x W13[g][0:I]^T) * (x W13[g][I:2I]^T)
//   GEMM2:           Y = h W2[g]^T
// (DeepSeek-V3 report summary on mpbf.cn, section 2.2: every expert an FFN over the
// tokens routed to it; the SwiGLU form of the expert FFN.)
//
// Packed layout.  A group's weight matrix (rows x Kd, row-major in the natural layout)
// is cut into blocks of 64 rows; block b holds the rows r(b, n, c), n in {0, 1},
// c in 0..31:
//   gate/up (W13, 2I rows): r = n*I + 32b + c   (32 gate rows and the matching up rows)
//   down    (W2, H rows):   r = 64b + 32n + c
// Per (group, block, 64-deep k step kt) come 4096 elements: 8 load instructions of 64
// lanes x 8 bf16, where instruction i = 4n + s and lane l = 32h + c hold
// W[r(b, n, c)][64kt + 16s + 8h .. +7] -- the 32x32x16 MFMA operand of column c, k
// half h, sub-step s.  Blocks follow each other per group, k steps per block.
//
// Kernel.  One workgroup of 4 waves per CU (one wave per SIMD, 512 registers per lane
// for it), persistent over the same XCD-aware, cost-balanced tile list as the LDS-ring
// kernels (schedule.h).  A tile is up to 192 rows of one group x 4 blocks (gate/up: 128
// h columns; down: 256 output columns); wave w owns block 4*n_tile + w and every row of
// the tile, so the four SIMDs do equal work at any row count.  Each wave streams its
// block's weights into registers (non-temporal; one or three k steps ahead); the
// activation rows, which all four waves need, go by direct-to-LDS loads into a three-
// slot ring, two steps ahead, issued after the step's multiplies.  One barrier per step.
// Activation rows past the group's end read as zeros (out-of-range buffer offsets).
#include <type_traits>

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

constexpr int PBM = 192;            // rows per tile (up to 6 subtiles of 32)
constexpr int PBK = 64;             // k per step: one 128-byte line per activation row
constexpr int kPkStep = 4096;       // elements of one (block, k step)
constexpr int kASlot = PBM * 128;   // bytes of one activation step at 192 rows
constexpr int kPRing = 3 * kASlot;  // 72 KiB
constexpr int kPStg = 32 * 128;     // down epilogue staging per wave: 32 rows x 128 bytes

__device__ __forceinline__ float silu(float a) { return a / (1.0f + __expf(-a)); }

// ---------------------------------------------------------------------------
// pack: one thread per 16-byte chunk of the packed output
// ---------------------------------------------------------------------------
__global__ void k_pack_bf16(const uint4* __restrict__ w, uint4* __restrict__ p, int64_t chunks,
                            int nblk, int nk, int Kd, int I, int swiglu) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < chunks; q += stride) {
    const int l = (int)(q & 63);
    const int i = (int)((q >> 6) & 7);
    const int64_t rest = q >> 9;  // (g * nblk + b) * nk + kt
    const int kt = (int)(rest % nk);
    const int64_t gb = rest / nk;
    const int b = (int)(gb % nblk);
    const int64_t g = gb / nblk;
    const int n = i >> 2, s = i & 3, c = l & 31, h = l >> 5;
    const int rows = swiglu ? 2 * I : nblk * 64;
    const int r = swiglu ? n * I + 32 * b + c : 64 * b + 32 * n + c;
    const int k = 64 * kt + 16 * s + 8 * h;
    p[q] = w[((g * rows + r) * Kd + k) >> 3];
  }
}

// The backward input part contracts over the OUTER dimension of the stored weights
// (dh = dY W2[g] over H, dx = [da|du] W13[g] over 2I), so it gets packed copies of the
// transposed matrices: B = W[g]^T, with W[g] stored [Kd rows][Nout columns], in the down
// layout (Nout rows in blocks of 64, k steps of 64 over Kd).  One thread per 16-byte
// chunk; its 8 elements are W[g][k .. k+7][r], and the 32 lanes of a half-wave take 32
// consecutive r.
__global__ void k_pack_bf16_t(const uint16_t* __restrict__ w, uint4* __restrict__ p,
                              int64_t chunks, int nblk, int nk, int Kd, int Nout) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < chunks; q += stride) {
    const int l = (int)(q & 63);
    const int i = (int)((q >> 6) & 7);
    const int64_t rest = q >> 9;  // (g * nblk + b) * nk + kt
    const int kt = (int)(rest % nk);
    const int64_t gb = rest / nk;
    const int b = (int)(gb % nblk);
    const int64_t g = gb / nblk;
    const int n = i >> 2, s = i & 3, c = l & 31, h = l >> 5;
    const int r = 64 * b + 32 * n + c;
    const int k = 64 * kt + 16 * s + 8 * h;
    const uint16_t* src = w + (g * Kd + k) * Nout + r;
    uint32_t u[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      u[e] = (uint32_t)src[(int64_t)(2 * e) * Nout] |
             ((uint32_t)src[(int64_t)(2 * e + 1) * Nout] << 16);
    p[q] = make_uint4(u[0], u[1], u[2], u[3]);
  }
}

// ---------------------------------------------------------------------------
// one tile, MS subtiles of 32 rows, D weight steps in flight
// ---------------------------------------------------------------------------
// Mode 0: gate/up + SwiGLU (C = h; au: the pre-activations kept for the backward, or
// NULL).  Mode 1: down (C = Y [rows, Nout]).  Mode 2: the backward's dh, a down-form
// product over packed W2^T, whose epilogue turns dh into da = dh u silu'(a) and
// du = dh silu(a) with a = au[r][c], u = au[r][I + c] (I = Nout) and writes both into
// C = [da|du] [rows, 2I].
template <int Mode, int MS, int D>
__device__ __forceinline__ void pk_tile(const uint16_t* __restrict__ A,
                                        const int32_t* __restrict__ gather, int a_rows,
                                        const uint16_t* __restrict__ Bw, bool w_on,
                                        uint16_t* __restrict__ C, uint16_t* __restrict__ au,
                                        int Kd, int Nout, int col0, int64_t grow0, int m_rows,
                                        char* smem, uint32_t lds0, char* stg) {
  constexpr bool kSwiglu = Mode == 0;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nk = Kd / PBK;
  constexpr int SL = MS * 32 * 128;  // bytes of one activation slot
  // activation loads: instruction i of wave wv fills rows 32i + 8wv + lane/8; lane l
  // writes slot l&7 of its row, which holds k-chunk (l&7) ^ ((row>>1)&7)
  const int lrow = lane >> 3;
  const int lchunk = (lane & 7) ^ ((4 * wv + (lane >> 4)) & 7);
  const i32x4 arsrc = gather ? buffer_rsrc(A, (uint32_t)a_rows * Kd * 2)
                             : buffer_rsrc(A + grow0 * Kd, (uint32_t)m_rows * Kd * 2);
  uint32_t aoff[MS];
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    const int r = 32 * i + 8 * wv + lrow;
    if (r >= m_rows) aoff[i] = 0x7ffffff0u;
    else if (gather) aoff[i] = (uint32_t)(gather[grow0 + r] * Kd + lchunk * 8) * 2;
    else aoff[i] = (uint32_t)(r * Kd + lchunk * 8) * 2;
  }
  const uint32_t ldsw = lds0 + 8 * wv * 128;
  auto aload = [&](int kt, int slot) {
#pragma unroll
    for (int i = 0; i < MS; ++i)
      load16_to_lds(arsrc, ldsw + slot * SL + i * 32 * 128, aoff[i] + (uint32_t)kt * 128);
  };
  u32x4 br[D + 1][8];
  auto bload = [&](int kt, int buf) {
    const uint16_t* p = Bw + (int64_t)kt * kPkStep;
    // full-height down tiles load their weights through the L2 normally: the shared
    // expert at a few thousand tokens has many such tiles per weight block, run at
    // about the same time on one XCD, and the later ones find the block there
    constexpr bool kTemporal = Mode == 1 && MS == PBM / 32;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (kTemporal) br[buf][i] = *reinterpret_cast<const u32x4*>(p + i * 512);
      else br[buf][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + i * 512));
    }
  };
  f32x16 acc[MS][2];
#pragma unroll
  for (int m = 0; m < MS; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[m][n][e] = 0.0f;

  // LDS row r of a slot: chunk c at slot (c ^ (r>>1)) & 7; (r>>1)&7 does not depend
  // on the subtile, so a lane's fragment offset is one value per k half-step
  const int frow = lane & 31;
  auto afrag = [&](const char* as, int m, int s) {
    const int c = 2 * s + (lane >> 5);
    return *reinterpret_cast<const bf16x8*>(as + (32 * m + frow) * 128 +
                                            ((c ^ (frow >> 1)) & 7) * 16);
  };

  // the loads below are issued in a fixed pattern: after A(kk) a wave issues B(kk-1+D)
  // (8 loads) and A(kk+1) (MS loads), so all but the last MS + 8 loads are complete when
  // A(kk) is.  The last D + 1 steps are peeled: they issue no loads past the tile's end,
  // and their counts shrink accordingly (compile-time, as j is)
  __syncthreads();  // the previous tile's LDS reads are done before the ring is refilled
  aload(0, 0);
  bload(0, 0);
  aload(min(1, nk - 1), 1);
#pragma unroll
  for (int j = 1; j < D; ++j) bload(min(j, nk - 1), j);

  auto step = [&](int kk, auto jc, auto lc) {
    constexpr int j = decltype(jc)::value;
    constexpr bool last = decltype(lc)::value;
    if constexpr (!last) wait_vm<MS + 8>();
    else wait_vm<(j < 2 ? 8 : 0) + (j < D ? MS : 0)>();
    __syncthreads();
    if constexpr (!last || j == 0) bload(kk + D, (j + D) % (D + 1));
    __builtin_amdgcn_sched_barrier(0);
    const int cs = kk % 3;
    if (w_on) {
      const char* as = smem + cs * SL;
      // fragments of the next half-step are read while this one multiplies
      bf16x8 af[2][MS];
#pragma unroll
      for (int m = 0; m < MS; ++m) af[0][m] = afrag(as, m, 0);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (s < 3) {
#pragma unroll
          for (int m = 0; m < MS; ++m) af[(s + 1) & 1][m] = afrag(as, m, s + 1);
        }
        const bf16x8 b0 = __builtin_bit_cast(bf16x8, br[j][s]);
        const bf16x8 b1 = __builtin_bit_cast(bf16x8, br[j][4 + s]);
#pragma unroll
        for (int m = 0; m < MS; ++m) {
          if (kSwiglu) {
            acc[m][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s & 1][m], b0, acc[m][0], 0, 0, 0);
            acc[m][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s & 1][m], b1, acc[m][1], 0, 0, 0);
          } else {
            acc[m][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0, af[s & 1][m], acc[m][0], 0, 0, 0);
            acc[m][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b1, af[s & 1][m], acc[m][1], 0, 0, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (!last || j < D - 1) aload(kk + 2, (kk + 2) % 3);
  };
  using std::integral_constant;
  const int kl = nk - (D + 1);  // first of the peeled steps
  for (int kt = 0; kt < kl; kt += D + 1) {
    step(kt, integral_constant<int, 0>(), std::false_type());
    step(kt + 1, integral_constant<int, 1>(), std::false_type());
    if constexpr (D == 3) {
      step(kt + 2, integral_constant<int, 2>(), std::false_type());
      step(kt + 3, integral_constant<int, 3>(), std::false_type());
    }
  }
  step(kl, integral_constant<int, 0>(), std::true_type());
  step(kl + 1, integral_constant<int, 1>(), std::true_type());
  if constexpr (D == 3) {
    step(kl + 2, integral_constant<int, 2>(), std::true_type());
    step(kl + 3, integral_constant<int, 3>(), std::true_type());
  }
  wait_vm<0>();  // no load of this tile lands in the ring after the next tile's barrier

  if (!w_on) return;
  if (kSwiglu) {
    // lane: h column col0 + (l%32); rows 32m + 8(e/4) + 4(l/32) + e%4.  32 lanes write
    // 64 contiguous bytes of a row per instruction.
    const int half = Nout;
    const int rl = 4 * (lane >> 5);
    uint16_t* cp = C + (grow0 + rl) * half + col0 + (lane & 31);
    uint16_t* ap = au ? au + (grow0 + rl) * 2 * half + col0 + (lane & 31) : nullptr;
#pragma unroll
    for (int m = 0; m < MS; ++m) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = 32 * m + 8 * (e >> 2) + (e & 3);  // + rl
        if (row + rl >= m_rows) continue;
        __builtin_nontemporal_store(f32_to_bf16_bits(silu(acc[m][0][e]) * acc[m][1][e]),
                                    cp + (int64_t)row * half);
        if (ap) {  // gate and up pre-activations, kept for the backward
          __builtin_nontemporal_store(f32_to_bf16_bits(acc[m][0][e]), ap + (int64_t)row * 2 * half);
          __builtin_nontemporal_store(f32_to_bf16_bits(acc[m][1][e]),
                                      ap + (int64_t)row * 2 * half + half);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  } else if constexpr (Mode == 2) {
    // as the down epilogue below, twice per subtile: the da columns, then the du columns
    const int r = lane & 31;
    const int I = Nout;
#pragma unroll
    for (int m = 0; m < MS; ++m) {
      const bool live = 32 * m + r < m_rows;
      const uint16_t* ar = au + (grow0 + 32 * m + r) * 2 * I + col0 + 4 * (lane >> 5);
      float da[2][16], du[2][16];
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint2 av = make_uint2(0u, 0u), uv = make_uint2(0u, 0u);
          if (live) {
            av = *reinterpret_cast<const uint2*>(ar + 32 * n + 8 * q);
            uv = *reinterpret_cast<const uint2*>(ar + I + 32 * n + 8 * q);
          }
          const uint32_t aw[2] = {av.x, av.y}, uw[2] = {uv.x, uv.y};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t ab = (t & 1) ? (aw[t >> 1] & 0xFFFF0000u) : (aw[t >> 1] << 16);
            const uint32_t ub = (t & 1) ? (uw[t >> 1] & 0xFFFF0000u) : (uw[t >> 1] << 16);
            const float a = __uint_as_float(ab), u = __uint_as_float(ub);
            const float dh = acc[m][n][4 * q + t];
            const float sg = 1.0f / (1.0f + __expf(-a));
            da[n][4 * q + t] = dh * u * (sg * (1.0f + a * (1.0f - sg)));
            du[n][4 * q + t] = dh * (a * sg);
          }
        }
      const int nrows = min(32, m_rows - 32 * m);
#pragma unroll
      for (int part = 0; part < 2; ++part) {
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float* v4 = part ? &du[n][4 * q] : &da[n][4 * q];
            const int j = 4 * n + q;
            *reinterpret_cast<uint2*>(stg + r * 128 + ((j ^ (r & 7)) << 4) + (lane >> 5) * 8) =
                pack4_bf16(v4[0], v4[1], v4[2], v4[3]);
          }
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int fr = 8 * p + (lane >> 3), j = lane & 7;
          const u32x4 v = *reinterpret_cast<const u32x4*>(stg + fr * 128 + ((j ^ (fr & 7)) << 4));
          if (fr < nrows)
            __builtin_nontemporal_store(
                v, reinterpret_cast<u32x4*>(C + (grow0 + 32 * m + fr) * 2 * I + part * I + col0 +
                                            8 * j));
        }
      }
    }
  } else {
    // lane: row 32m + l%32, columns col0 + 32n + 8q + 4(l/32) .. +3 (4 per group q of
    // four elements).  Each 32-row subtile is staged in the wave's own 4 KiB of LDS
    // (rows of 128 bytes, 16-byte chunk j at slot j ^ (row & 7)) and written back with
    // 16-byte lanes, 8 lanes per row: every store instruction writes 8 whole lines.
    const int r = lane & 31;
#pragma unroll
    for (int m = 0; m < MS; ++m) {
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = 4 * n + q;
          const uint2 v = pack4_bf16(acc[m][n][4 * q], acc[m][n][4 * q + 1],
                                     acc[m][n][4 * q + 2], acc[m][n][4 * q + 3]);
          *reinterpret_cast<uint2*>(stg + r * 128 + ((j ^ (r & 7)) << 4) + (lane >> 5) * 8) = v;
        }
      const int nrows = min(32, m_rows - 32 * m);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int fr = 8 * p + (lane >> 3), j = lane & 7;
        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + fr * 128 + ((j ^ (fr & 7)) << 4));
        if (fr < nrows)
          __builtin_nontemporal_store(
              v, reinterpret_cast<u32x4*>(C + (grow0 + 32 * m + fr) * Nout + col0 + 8 * j));
      }
    }
  }
}

// gather != nullptr: row r of the permuted order is row gather[r] of A (a_rows rows).
// Mode 0: Nout = I (h columns), Bp = packed W13.  Mode 1: Nout = H, Bp = packed W2.
// Mode 2: Nout = I, Bp = packed W2^T, A = dY, au the saved pre-activations (read).
template <int Mode>
__global__ __launch_bounds__(256, 1) void k_gemm_packed(const uint16_t* __restrict__ A,
                                                        const uint16_t* __restrict__ Bp,
                                                        uint16_t* __restrict__ C,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ gather,
                                                        uint16_t* __restrict__ au, int a_rows,
                                                        int NG, int Kd, int Nout) {
  constexpr bool kSwiglu = Mode == 0;
  __shared__ __attribute__((aligned(1024))) char smem[kPRing + 4 * kPStg];
  __shared__ int mt_start[kMaxGroups + 1];
  // the cost prefix is only needed for the XCD split below, before the first tile's
  // loads overwrite the ring (they follow a barrier), so it borrows the ring's memory
  long long* s_cost = reinterpret_cast<long long*>(smem);
  static_assert(sizeof(long long) * (kMaxGroups + 1) <= kPRing, "cost prefix fits the ring");
  build_schedule(offsets, NG, PBM, mt_start);
  const int nblk = kSwiglu ? Nout / 32 : Nout / 64;
  const int nt = (nblk + 3) / 4;
  build_costs(offsets, mt_start, NG, PBM, nt, s_cost);
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nk = Kd / PBK;
  // three weight steps in flight need nk % 4 == 0, and their registers fit beside the
  // accumulators of up to 4 sub-tiles in the SwiGLU and dh epilogues, of all 6 in down
  const bool deep = (nk & 3) == 0;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_offset(smem));
  char* stg = smem + kPRing + wv * kPStg;

  const int P = gridDim.x, per_xcd = P / kXcds;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int begin = xcd_boundary(xcd, offsets, mt_start, s_cost, NG, PBM, nt);
  const int end = xcd_boundary(xcd + 1, offsets, mt_start, s_cost, NG, PBM, nt);
  for (int tile = begin + slot; tile < end; tile += per_xcd) {
    Tile tl = decode_tile(tile, mt_start, NG, nt);
    const int g = __builtin_amdgcn_readfirstlane(tl.g);
    const int n_idx = __builtin_amdgcn_readfirstlane(tl.n_idx);
    const int m_idx = __builtin_amdgcn_readfirstlane(tl.m_idx);
    const int row0 = offsets[g];
    const int m_g = offsets[g + 1] - row0;
    const int m0 = m_idx * PBM;
    const int m_rows = min(PBM, m_g - m0);
    const int b = 4 * n_idx + wv;
    const bool w_on = b < nblk;
    // a wave without a block streams the tile's first block (the same load count keeps
    // every wave's waits exact) and skips its multiplies and stores
    const int bb = w_on ? b : 4 * n_idx;
    const uint16_t* Bw = Bp + ((int64_t)g * nblk + bb) * nk * kPkStep + lane * 8;
    const int col0 = kSwiglu ? 32 * b : 64 * b;
    const int64_t grow0 = (int64_t)row0 + m0;
    const int ms = (m_rows + 31) >> 5;
#define PK_CASE(MSV)                                                                      \
  case MSV:                                                                               \
    if (deep && (MSV <= 4 || Mode == 1))                                                 \
      pk_tile<Mode, MSV, 3>(A, gather, a_rows, Bw, w_on, C, au, Kd, Nout, col0, grow0,    \
                               m_rows, smem, lds0, stg);                                  \
    else                                                                                  \
      pk_tile<Mode, MSV, 1>(A, gather, a_rows, Bw, w_on, C, au, Kd, Nout, col0, grow0,    \
                               m_rows, smem, lds0, stg);                                  \
    break;
    switch (ms) {
      PK_CASE(1)
      PK_CASE(2)
      PK_CASE(3)
      PK_CASE(4)
      PK_CASE(5)
      PK_CASE(6)
      default: break;
    }
#undef PK_CASE
  }
}

int pk_grid() {
  const int p = (device_cu_count() / kXcds) * kXcds;
  return p < kXcds ? kXcds : p;
}

}  // namespace

bool packed_supported(const Dims& d) {
  return d.act == MOE_BF16 && (d.expert == MOE_BF16 || d.expert == MOE_FP8_E4M3);
}

size_t packed_w13_elems(const Dims& d) { return (size_t)(d.E + d.S) * 2 * d.I * d.H; }
size_t packed_w2_elems(const Dims& d) { return (size_t)(d.E + d.S) * d.H * d.I; }

hipError_t launch_pack_weights(const Dims& d, const void* w13, const void* w2, void* p13,
                               void* p2, hipStream_t st) {
  const int NG = d.E + d.S;
  if (w13) {
    const int64_t chunks = (int64_t)packed_w13_elems(d) / 8;
    hipLaunchKernelGGL(k_pack_bf16, dim3(4096), dim3(256), 0, st,
                       static_cast<const uint4*>(w13), static_cast<uint4*>(p13), chunks,
                       d.I / 32, d.H / PBK, d.H, d.I, 1);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (w2) {
    const int64_t chunks = (int64_t)packed_w2_elems(d) / 8;
    hipLaunchKernelGGL(k_pack_bf16, dim3(4096), dim3(256), 0, st,
                       static_cast<const uint4*>(w2), static_cast<uint4*>(p2), chunks, d.H / 64,
                       d.I / PBK, d.I, d.I, 0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  (void)NG;
  return hipSuccess;
}

hipError_t launch_ffn_up_packed(const Dims& d, const void* xs, const int32_t* offsets,
                                const int32_t* gather, const void* w13, const void* p13, void* h,
                                void* au, hipStream_t st) {
  int ng = d.E + d.S;
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
  hipLaunchKernelGGL(k_gemm_packed<0>, dim3(pk_grid()), dim3(256), 0, st,
                     static_cast<const uint16_t*>(xs), static_cast<const uint16_t*>(p13),
                     static_cast<uint16_t*>(h), offsets, gather, static_cast<uint16_t*>(au),
                     (int)d.T, ng, d.H, d.I);
  return hipGetLastError();
}

hipError_t launch_ffn_down_packed(const Dims& d, const void* h, const int32_t* offsets,
                                  const void* p2, void* ys, hipStream_t st) {
  hipLaunchKernelGGL(k_gemm_packed<1>, dim3(pk_grid()), dim3(256), 0, st,
                     static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(p2),
                     static_cast<uint16_t*>(ys), offsets, nullptr, nullptr, 0, d.E + d.S, d.I,
                     d.H);
  return hipGetLastError();
}

hipError_t launch_pack_weights_t(const Dims& d, const void* w13, const void* w2, void* p13t,
                                 void* p2t, hipStream_t st) {
  const int NG = d.E + d.S;
  if (w2) {  // W2[g] is [H, I]: its transpose packed as I rows over k = H
    const int64_t chunks = (int64_t)NG * d.I * d.H / 8;
    hipLaunchKernelGGL(k_pack_bf16_t, dim3(4096), dim3(256), 0, st,
                       static_cast<const uint16_t*>(w2), static_cast<uint4*>(p2t), chunks,
                       d.I / 64, d.H / PBK, d.H, d.I);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (w13) {  // W13[g] is [2I, H]: its transpose packed as H rows over k = 2I
    const int64_t chunks = (int64_t)NG * 2 * d.I * d.H / 8;
    hipLaunchKernelGGL(k_pack_bf16_t, dim3(4096), dim3(256), 0, st,
                       static_cast<const uint16_t*>(w13), static_cast<uint4*>(p13t), chunks,
                       d.H / 64, 2 * d.I / PBK, 2 * d.I, d.H);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_ffn_bwd_input_packed(const Dims& d, const int32_t* offsets, const void* p13t,
                                       const void* p2t, const void* au, const void* dys,
                                       void* dau, void* dxs, hipStream_t st) {
  const int NG = d.E + d.S;
  // dh = dY W2 (k over H) -> [da|du]
  hipLaunchKernelGGL(k_gemm_packed<2>, dim3(pk_grid()), dim3(256), 0, st,
                     static_cast<const uint16_t*>(dys), static_cast<const uint16_t*>(p2t),
                     static_cast<uint16_t*>(dau), offsets, nullptr,
                     const_cast<uint16_t*>(static_cast<const uint16_t*>(au)), 0, NG, d.H, d.I);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dx_sorted = [da|du] W13 (k over 2I)
  hipLaunchKernelGGL(k_gemm_packed<1>, dim3(pk_grid()), dim3(256), 0, st,
                     static_cast<const uint16_t*>(dau), static_cast<const uint16_t*>(p13t),
                     static_cast<uint16_t*>(dxs), offsets, nullptr, nullptr, 0, NG, 2 * d.I,
                     d.H);
  return hipGetLastError();
}

}  // namespace moe
