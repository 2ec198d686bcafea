// FP8 (E4M3) expert FFN grouped GEMMs over packed weight codes: the block-scaled GEMM
// pair of gemm_fp8.hip (DeepSeek-V3 report summary on mpbf.cn, section 3.1: scaling
// per small tile and fp32 promotion of the partial sums; section 4.3: block-wise
// scales) with the weight stream of gemm_packed.hip (each weight load instruction
// reads 1 KiB of contiguous memory straight into the matrix-core operand registers).
//
// Packed layout.  A group's code matrix (rows x Kd bytes, row-major in the natural
// layout) is cut into blocks of 64 rows, as the bf16 layout (gate/up: 32 gate rows and
// the matching 32 up rows; down: 64 consecutive rows); per (group, block, 128-deep k
// step kt) come 8192 bytes: 8 load instructions of 64 lanes x 16 bytes, where
// instruction i = 4n + 2u + v and lane l = 32h + c hold
// W[r(b, n, c)][128kt + 64u + 32h + 16v .. +15] -- half v of the 32x32x64 MFMA operand
// of weight row c of half n, k half u, lane half h.  Instructions 4n .. 4n+3 (4 KiB)
// are half n of the block.  The 128x128 weight scales keep their natural layout.
//
// Kernel.  One workgroup of 8 waves per CU (two per SIMD); a tile is up to 192 rows of
// one group x 4 blocks; waves 2p and 2p+1 own halves 0 and 1 of block 4*n_tile + p and
// every row of the tile.  Per 128-deep step a wave multiplies each 32-row sub-tile
// twice (k halves) with its weight half as the first operand, so a lane's 16 results
// are one activation row and 16 weight rows; the block's partial sum is promoted as
// acc += partial * (s_a[row] * s_w), with one activation scale per lane and sub-tile
// and one weight scale per wave and step.  Activation codes and their scales go by
// direct-to-LDS loads into a three-slot ring two steps ahead, weights into registers
// one or three steps ahead; one barrier per step.
//   up: per 32-row sub-tile the gate half's wave and the up half's wave of a block hand
//       each other half of their values through LDS and each forms h = silu(gate) * up
//       for half of the block's columns; the row's 128-column amax is combined over the
//       tile's eight waves in LDS, and the E4M3 codes are staged so that whole 128-byte
//       rows are stored.
//   down: each 32-row sub-tile of a block (64 bf16 columns, one 128-byte line per row)
//       is staged in LDS and stored as whole lines.
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

constexpr int QPM = 192;               // rows per tile (up to 6 sub-tiles of 32)
constexpr int QPK = 128;               // k per step: one 128-byte line per activation row
constexpr int kQPStep = 8192;          // bytes of one (block, k step)
constexpr int kQPSlot = QPM * 128;     // activation slot at 192 rows: 24 KiB
constexpr int kQPRing = 3 * kQPSlot;   // 72 KiB
constexpr int kQPSa = QPM;             // activation scales per slot

__device__ __forceinline__ float silu(float a) { return a / (1.0f + __expf(-a)); }

// byte offset of (row, 16-byte chunk c) in an activation slot: 128-byte rows, chunk
// slots xor-swizzled by (row >> 1) & 7
__device__ __forceinline__ int qswz(int r, int c) { return r * 128 + ((c ^ (r >> 1)) & 7) * 16; }

__device__ __forceinline__ i32x8 frag32(const char* p0, const char* p1) {
  const uint4 u0 = *reinterpret_cast<const uint4*>(p0);
  const uint4 u1 = *reinterpret_cast<const uint4*>(p1);
  i32x8 f;
  f[0] = u0.x; f[1] = u0.y; f[2] = u0.z; f[3] = u0.w;
  f[4] = u1.x; f[5] = u1.y; f[6] = u1.z; f[7] = u1.w;
  return f;
}

__device__ __forceinline__ i32x8 join(u32x4 a, u32x4 b) {
  i32x8 f;
  f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
  f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
  return f;
}

// pack: one thread per 16-byte chunk of the packed output
__global__ void k_pack_fp8(const uint4* __restrict__ w, uint4* __restrict__ p, int64_t chunks,
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
    const int n = i >> 2, u = (i >> 1) & 1, v = i & 1, c = l & 31, h = l >> 5;
    const int rows = swiglu ? 2 * I : nblk * 64;
    const int r = swiglu ? n * I + 32 * b + c : 64 * b + 32 * n + c;
    const int k = 128 * kt + 64 * u + 32 * h + 16 * v;
    p[q] = w[((g * rows + r) * Kd + k) >> 4];
  }
}

// one tile: MS sub-tiles of 32 rows, D weight steps in flight
template <bool kSwiglu, int MS, int D>
__device__ __forceinline__ void pk8_tile(const uint8_t* __restrict__ A,
                                         const float* __restrict__ A_scale,
                                         const int32_t* __restrict__ gather, int a_rows,
                                         const uint8_t* __restrict__ Bw,
                                         const float* __restrict__ bsc, bool w_on,
                                         void* __restrict__ C, float* __restrict__ C_scale,
                                         int Kd, int Nout, int n_idx, int64_t grow0,
                                         int m_rows, char* smem, float* s_sa, uint32_t lds0,
                                         uint32_t lds_sa) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pair = wv >> 1, half = wv & 1;
  const int nk = Kd / QPK;
  constexpr int NAI = (MS + 1) / 2;          // activation load instructions per wave
  constexpr int SL = NAI * 64 * 128;         // bytes of one activation slot
  // activation codes: instruction i of wave wv fills rows 64i + 8wv + lane/8; lane l
  // writes slot l&7 of its row, which holds chunk (l&7) ^ ((row>>1)&7)
  const int lrow = lane >> 3;
  const int lchunk = (lane & 7) ^ ((4 * (wv & 1) + (lane >> 4)) & 7);
  const int nkb = nk;  // scale columns per activation row
  const i32x4 arsrc = gather ? buffer_rsrc(A, (uint32_t)a_rows * Kd)
                             : buffer_rsrc(A + grow0 * Kd, (uint32_t)m_rows * Kd);
  const i32x4 srsrc = gather ? buffer_rsrc(A_scale, (uint32_t)a_rows * nkb * 4)
                             : buffer_rsrc(A_scale + grow0 * nkb, (uint32_t)m_rows * nkb * 4);
  uint32_t aoff[NAI];
#pragma unroll
  for (int i = 0; i < NAI; ++i) {
    const int r = 64 * i + 8 * wv + lrow;
    if (r >= m_rows) aoff[i] = 0x7ffffff0u;
    else if (gather) aoff[i] = (uint32_t)(gather[grow0 + r] * Kd + lchunk * 16);
    else aoff[i] = (uint32_t)(r * Kd + lchunk * 16);
  }
  // activation scales: lanes 0..23 of wave wv bring rows 24wv + lane
  const int srow = 24 * wv + lane;
  uint32_t soff = 0x7ffffff0u;
  if (lane < 24 && srow < m_rows)
    soff = (uint32_t)((gather ? gather[grow0 + srow] : srow) * nkb) * 4;
  const uint32_t ldsw = lds0 + 8 * wv * 128;
  const uint32_t ldss = lds_sa + 24 * wv * 4;
  auto aload = [&](int kt, int slot) {
#pragma unroll
    for (int i = 0; i < NAI; ++i)
      load16_to_lds(arsrc, ldsw + slot * SL + i * 64 * 128, aoff[i] + (uint32_t)kt * QPK);
    if (lane < 24) load4_to_lds(srsrc, ldss + slot * (kQPSa * 4), soff + (uint32_t)kt * 4);
  };
  u32x4 br[D + 1][4];
  auto bload = [&](int kt, int buf) {
    const uint8_t* p = Bw + (int64_t)kt * kQPStep;
    // full-height down tiles load their weights through the L2 normally: the shared
    // expert at a few thousand tokens has many such tiles per weight block, run at
    // about the same time on one XCD, and the later ones find the block there
    constexpr bool kTemporal = !kSwiglu && MS == QPM / 32;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (kTemporal) br[buf][i] = *reinterpret_cast<const u32x4*>(p + i * 1024);
      else br[buf][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + i * 1024));
    }
  };
  f32x16 acc[MS];
#pragma unroll
  for (int m = 0; m < MS; ++m)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[m][e] = 0.0f;
  const int frow = lane & 31, kq = lane >> 5;

  // fixed load pattern: after A(kt) (NAI codes + 1 scale load) a wave issues B(kt-1+D)
  // (4 loads) and A(kt+1), so NAI + 5 loads are behind it at every step
  __syncthreads();  // the previous tile's LDS use is over before the ring is refilled
  aload(0, 0);
  bload(0, 0);
  aload(min(1, nk - 1), 1);
#pragma unroll
  for (int j = 1; j < D; ++j) bload(min(j, nk - 1), j);

  for (int kt = 0; kt < nk; kt += D + 1) {
#pragma unroll
    for (int j = 0; j <= D; ++j) {
      const int kk = kt + j;
      if (kk >= nk) break;
      wait_vm<NAI + 5>();
      __syncthreads();
      bload(min(kk + D, nk - 1), (j + D) % (D + 1));
      __builtin_amdgcn_sched_barrier(0);
      const int cs = kk % 3;
      if (w_on) {
        const float sw = bsc[kk];
        const char* as = smem + cs * SL;
        const float* sas = s_sa + cs * kQPSa;
        const i32x8 b0 = join(br[j][0], br[j][1]);
        const i32x8 b1 = join(br[j][2], br[j][3]);
#pragma unroll
        for (int m = 0; m < MS; ++m) {
          const int r = 32 * m + frow;
          const i32x8 a0 = frag32(as + qswz(r, 2 * kq), as + qswz(r, 2 * kq + 1));
          const i32x8 a1 = frag32(as + qswz(r, 4 + 2 * kq), as + qswz(r, 5 + 2 * kq));
          f32x16 t;
#pragma unroll
          for (int e = 0; e < 16; ++e) t[e] = 0.0f;
          t = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b0, a0, t, 0, 0, 0, 127, 0, 127);
          t = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b1, a1, t, 0, 0, 0, 127, 0, 127);
          const float s = sas[r] * sw;
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[m][e] = __builtin_fmaf(t[e], s, acc[m][e]);
        }
      }
      aload(min(kk + 2, nk - 1), (kk + 2) % 3);
    }
  }
  wait_vm<0>();
  __syncthreads();  // every wave is done with the ring, which now stages the outputs

  // lane: activation row 32m + l%32; weight rows 8q + 4(l/32) + 0..3 of the wave's
  // 32-row half (q = element / 4)
  const int rr = frow;
  if constexpr (kSwiglu) {
    // the pair's two waves split the h elements: the gate wave forms those of q = 0, 1
    // (columns 8q + 4h ..), the up wave those of q = 2, 3; each first hands the other
    // its values of the other's columns (float4 slot 2qq + h, swizzled by row & 3)
    float* exg = reinterpret_cast<float*>(smem);   // [4 blocks][32 rows][16] gate, q = 2, 3
    float* exu = exg + 4 * 32 * 16;                // [4 blocks][32 rows][16] up, q = 0, 1
    float* amx = exu + 4 * 32 * 16;                // [8 waves][32 rows]
    char* hst = reinterpret_cast<char*>(amx + 8 * 32);  // [32 rows][128 bytes] codes
    uint8_t* h = static_cast<uint8_t*>(C);
    const int ncb = Nout / 128;
    const int qb = half ? 2 : 0;                   // this wave's q range: qb, qb + 1
    float* mine = (half ? exu : exg) + (pair * 32 + rr) * 16;
    const float* theirs = (half ? exg : exu) + (pair * 32 + rr) * 16;
#pragma unroll
    for (int m = 0; m < MS; ++m) {
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const int q = (half ? 0 : 2) + qq;  // the partner's columns
        const int f = (2 * qq + kq) ^ (rr & 3);
        *reinterpret_cast<float4*>(mine + 4 * f) =
            make_float4(acc[m][4 * q], acc[m][4 * q + 1], acc[m][4 * q + 2], acc[m][4 * q + 3]);
      }
      __syncthreads();
      float hv[8];
      float am = 0.0f;
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const int q = qb + qq;
        const int f = (2 * qq + kq) ^ (rr & 3);
        const float4 o = *reinterpret_cast<const float4*>(theirs + 4 * f);
        const float other[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float g = half ? other[t] : acc[m][4 * q + t];
          const float u = half ? acc[m][4 * q + t] : other[t];
          hv[4 * qq + t] = silu(g) * u;
          am = __builtin_fmaxf(am, __builtin_fabsf(hv[4 * qq + t]));
        }
      }
      am = __builtin_fmaxf(am, __shfl_xor(am, 32));
      if (kq == 0) amx[wv * 32 + rr] = am;
      __syncthreads();
#pragma unroll
      for (int w = 0; w < 8; ++w) am = __builtin_fmaxf(am, amx[w * 32 + rr]);
      const float sc = am > 0.0f ? am / 448.0f : 1.0f;
      // codes of columns 32 pair + 8q + 4h .. +3: 4 bytes at byte 8(q&1) + 4h of chunk
      // 2 pair + q/2 (16-byte chunks of the 128-byte row, slot chunk ^ (r & 7))
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const int q = qb + qq;
        const uint32_t w = pack4_e4m3(hv[4 * qq] / sc, hv[4 * qq + 1] / sc, hv[4 * qq + 2] / sc,
                                      hv[4 * qq + 3] / sc);
        const int ch = 2 * pair + (q >> 1);
        *reinterpret_cast<uint32_t*>(hst + rr * 128 + ((ch ^ (rr & 7)) << 4) + 8 * (q & 1) +
                                     4 * kq) = w;
      }
      if (wv == 0 && kq == 0 && 32 * m + rr < m_rows)
        C_scale[(grow0 + 32 * m + rr) * ncb + n_idx] = sc;
      __syncthreads();
      if (wv < 4) {  // 32 rows x 8 chunks: waves 0..3, 8 rows each
        const int fr = 8 * wv + (lane >> 3), ch = lane & 7;
        const u32x4 v = *reinterpret_cast<const u32x4*>(hst + fr * 128 + ((ch ^ (fr & 7)) << 4));
        if (32 * m + fr < m_rows)
          __builtin_nontemporal_store(
              v, reinterpret_cast<u32x4*>(h + (grow0 + 32 * m + fr) * Nout + n_idx * 128 + 16 * ch));
      }
    }
  } else {
    // block p's sub-tile: 32 rows x 64 bf16 columns = one 128-byte line per row; the
    // wave of half n writes chunks 4n + q (columns 32n + 8q .. +7), lane half h the
    // second 8 bytes of a chunk; chunk slot j ^ (r & 7)
    char* stg = smem + pair * 4096;
    uint16_t* y = static_cast<uint16_t*>(C);
#pragma unroll
    for (int m = 0; m < MS; ++m) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int jj = 4 * half + q;
        *reinterpret_cast<uint2*>(stg + rr * 128 + ((jj ^ (rr & 7)) << 4) + kq * 8) =
            pack4_bf16(acc[m][4 * q], acc[m][4 * q + 1], acc[m][4 * q + 2], acc[m][4 * q + 3]);
      }
      __syncthreads();
      if (w_on) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int fr = 16 * half + 8 * i + (lane >> 3), ch = lane & 7;
          const u32x4 v = *reinterpret_cast<const u32x4*>(stg + fr * 128 + ((ch ^ (fr & 7)) << 4));
          if (32 * m + fr < m_rows)
            __builtin_nontemporal_store(
                v, reinterpret_cast<u32x4*>(y + (grow0 + 32 * m + fr) * Nout +
                                            (4 * n_idx + pair) * 64 + 8 * ch));
        }
      }
      __syncthreads();
    }
  }
}

// gather != nullptr: row r of the permuted order is row gather[r] of A and A_scale.
// kSwiglu: Nout = I (h columns), Bp = packed W13 codes; else Nout = H, Bp = packed W2.
template <bool kSwiglu>
__global__ __launch_bounds__(512, 1) void k_gemm_packed_fp8(
    const uint8_t* __restrict__ A, const float* __restrict__ A_scale,
    const uint8_t* __restrict__ Bp, const float* __restrict__ B_scale, void* __restrict__ C,
    float* __restrict__ C_scale, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ gather, int a_rows, int NG, int Kd, int Nout) {
  __shared__ __attribute__((aligned(1024))) char smem[kQPRing];
  __shared__ __attribute__((aligned(16))) float s_sa[3 * kQPSa];
  __shared__ int mt_start[kMaxGroups + 1];
  // the cost prefix is only needed for the XCD split below, before the first tile's
  // loads overwrite the ring (they follow a barrier), so it borrows the ring's memory
  long long* s_cost = reinterpret_cast<long long*>(smem);
  static_assert(sizeof(long long) * (kMaxGroups + 1) <= kQPRing, "cost prefix fits the ring");
  build_schedule(offsets, NG, QPM, mt_start);
  const int nblk = kSwiglu ? Nout / 32 : Nout / 64;
  const int nt = (nblk + 3) / 4;
  build_costs(offsets, mt_start, NG, QPM, nt, s_cost);
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pair = wv >> 1, half = wv & 1;
  const int nk = Kd / QPK;
  const int nbr = kSwiglu ? 2 * Nout / 128 : Nout / 128;  // weight-scale block rows
  const bool deep = (nk & 3) == 0;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_offset(smem));
  const uint32_t lds_sa = __builtin_amdgcn_readfirstlane(lds_offset(s_sa));

  const int P = gridDim.x, per_xcd = P / kXcds;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int begin = xcd_boundary(xcd, offsets, mt_start, s_cost, NG, QPM, nt);
  const int end = xcd_boundary(xcd + 1, offsets, mt_start, s_cost, NG, QPM, nt);
  for (int tile = begin + slot; tile < end; tile += per_xcd) {
    Tile tl = decode_tile(tile, mt_start, NG, nt);
    const int g = __builtin_amdgcn_readfirstlane(tl.g);
    const int n_idx = __builtin_amdgcn_readfirstlane(tl.n_idx);
    const int m_idx = __builtin_amdgcn_readfirstlane(tl.m_idx);
    const int row0 = offsets[g];
    const int m_g = offsets[g + 1] - row0;
    const int m0 = m_idx * QPM;
    const int m_rows = min(QPM, m_g - m0);
    const int b = 4 * n_idx + pair;
    const bool w_on = b < nblk;
    // a wave without a block streams the tile's first block (same load count, so the
    // waits stay exact) and skips its multiplies and stores
    const int bb = w_on ? b : 4 * n_idx;
    const uint8_t* Bw = Bp + ((int64_t)g * nblk + bb) * nk * kQPStep + half * 4096 + lane * 16;
    // weight-scale row of this wave's 32 rows: up: gate rows 32b.. (row b/4), up rows
    // I + 32b.. (I/128 + b/4); down: rows 64b + 32 half .. (row b/2)
    const int srow = kSwiglu ? (half ? Nout / 128 : 0) + (bb >> 2) : (bb >> 1);
    const float* bsc = B_scale + ((int64_t)g * nbr + srow) * nk;
    const int64_t grow0 = (int64_t)row0 + m0;
    const int ms = (m_rows + 31) >> 5;
#define PK8_CASE(MSV)                                                                        \
  case MSV:                                                                                  \
    if (deep && MSV <= 4)                                                                    \
      pk8_tile<kSwiglu, MSV, 3>(A, A_scale, gather, a_rows, Bw, bsc, w_on, C, C_scale, Kd,   \
                                Nout, n_idx, grow0, m_rows, smem, s_sa, lds0, lds_sa);       \
    else                                                                                     \
      pk8_tile<kSwiglu, MSV, 1>(A, A_scale, gather, a_rows, Bw, bsc, w_on, C, C_scale, Kd,   \
                                Nout, n_idx, grow0, m_rows, smem, s_sa, lds0, lds_sa);       \
    break;
    switch (ms) {
      PK8_CASE(1)
      PK8_CASE(2)
      PK8_CASE(3)
      PK8_CASE(4)
      PK8_CASE(5)
      PK8_CASE(6)
      default: break;
    }
#undef PK8_CASE
  }
}

int pk8_grid() {
  const int p = (device_cu_count() / kXcds) * kXcds;
  return p < kXcds ? kXcds : p;
}

}  // namespace

hipError_t launch_pack_weights_fp8(const Dims& d, const void* w13, const void* w2, void* p13,
                                   void* p2, hipStream_t st) {
  const int NG = d.E + d.S;
  if (w13) {
    const int64_t chunks = (int64_t)NG * 2 * d.I * d.H / 16;
    hipLaunchKernelGGL(k_pack_fp8, dim3(4096), dim3(256), 0, st, static_cast<const uint4*>(w13),
                       static_cast<uint4*>(p13), chunks, d.I / 32, d.H / QPK, d.H, d.I, 1);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (w2) {
    const int64_t chunks = (int64_t)NG * d.H * d.I / 16;
    hipLaunchKernelGGL(k_pack_fp8, dim3(4096), dim3(256), 0, st, static_cast<const uint4*>(w2),
                       static_cast<uint4*>(p2), chunks, d.H / 64, d.I / QPK, d.I, d.I, 0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_ffn_up_packed_fp8(const Dims& d, const void* xs, const float* xs_scale,
                                    const int32_t* offsets, const int32_t* gather,
                                    const void* w13, const void* p13, const float* w13_scale,
                                    void* h, float* h_scale, hipStream_t st) {
  int ng = d.E + d.S;
  if (dense_shared(d)) {
    ng = d.E;
    const hipError_t e =
        launch_dense_swiglu_fp8_shared(d, xs, xs_scale, gather, w13, w13_scale, h, h_scale, st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_gemm_packed_fp8<true>, dim3(pk8_grid()), dim3(512), 0, st,
                     static_cast<const uint8_t*>(xs), xs_scale, static_cast<const uint8_t*>(p13),
                     w13_scale, h, h_scale, offsets, gather, (int)d.T, ng, d.H, d.I);
  return hipGetLastError();
}

hipError_t launch_ffn_down_packed_fp8(const Dims& d, const void* h, const float* h_scale,
                                      const int32_t* offsets, const void* p2,
                                      const float* w2_scale, void* ys, hipStream_t st) {
  hipLaunchKernelGGL(k_gemm_packed_fp8<false>, dim3(pk8_grid()), dim3(512), 0, st,
                     static_cast<const uint8_t*>(h), h_scale, static_cast<const uint8_t*>(p2),
                     w2_scale, ys, nullptr, offsets, nullptr, 0, d.E + d.S, d.I, d.H);
  return hipGetLastError();
}

}  // namespace moe
