// Internal declarations shared by the HIP kernels and the C ABI of libmoe.
// gfx950 only: wave64, MFMA, 160 KB LDS per CU, 8 XCDs of 32 CUs.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kXcds = 8;

// Buffer descriptor for raw loads from p: byte offsets at or past `bytes` read as zero
// without touching memory (per-dword range check, stride 0).
__device__ __forceinline__ i32x4 buffer_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  i32x4 r;
  r.x = (int)(uint32_t)a;
  r.y = (int)((uint32_t)(a >> 32) & 0xffffu);
  r.z = (int)bytes;
  r.w = 0x00020000;
  return r;
}

// Byte address of a __shared__ object in the workgroup's LDS.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Buffer loads whose data goes to LDS instead of registers: lane l writes its 16 (or
// 4) bytes at LDS byte address lds + 16*l (4*l).  `lds` must be wave-uniform.  The
// compiler does not see these loads: the caller waits for them with wait_vmcnt and
// a barrier before reading the LDS they fill.
__device__ __forceinline__ void load16_to_lds(i32x4 rsrc, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               ::"s"(lds), "v"(voff), "s"(rsrc) : "memory");
}
// Same, non-temporal: for data read once (expert weights streamed through a GEMM),
// so it does not push reused rows out of the L2.
__device__ __forceinline__ void load16_to_lds_nt(i32x4 rsrc, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               ::"s"(lds), "v"(voff), "s"(rsrc) : "memory");
}
__device__ __forceinline__ void load4_to_lds(i32x4 rsrc, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               ::"s"(lds), "v"(voff), "s"(rsrc) : "memory");
}

// Wait until at most n (0..15) vector-memory operations of this wave are outstanding;
// other n wait for all.
// s_waitcnt vmcnt(N) for a compile-time N in [0, 63] (6-bit counter: bits 3:0 and
// 15:14 of the immediate); expcnt and lgkmcnt left unconstrained.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
#define MOE_VMCNT_CASE(k) \
  case k: __builtin_amdgcn_s_waitcnt(0x0F70 | k); break;
    MOE_VMCNT_CASE(1) MOE_VMCNT_CASE(2) MOE_VMCNT_CASE(3) MOE_VMCNT_CASE(4)
    MOE_VMCNT_CASE(5) MOE_VMCNT_CASE(6) MOE_VMCNT_CASE(7) MOE_VMCNT_CASE(8)
    MOE_VMCNT_CASE(9) MOE_VMCNT_CASE(10) MOE_VMCNT_CASE(11) MOE_VMCNT_CASE(12)
    MOE_VMCNT_CASE(13) MOE_VMCNT_CASE(14) MOE_VMCNT_CASE(15)
#undef MOE_VMCNT_CASE
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
  }
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bf16 bits (inputs are finite on every path here).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// E4M3 (OCP) code of v with round-to-nearest-even and saturation at +-448: the
// hardware conversion rounds to nearest even but maps |v| >= 464 to NaN, so the
// input is clamped first.
__device__ __forceinline__ uint32_t f32_to_e4m3_bits(float v) {
  v = __builtin_fminf(__builtin_fmaxf(v, -448.0f), 448.0f);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false)) & 0xFFu;
}

// Pack four E4M3 codes (little-endian byte order) from four floats.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  a = __builtin_fminf(__builtin_fmaxf(a, -448.0f), 448.0f);
  b = __builtin_fminf(__builtin_fmaxf(b, -448.0f), 448.0f);
  c = __builtin_fminf(__builtin_fmaxf(c, -448.0f), 448.0f);
  d = __builtin_fminf(__builtin_fmaxf(d, -448.0f), 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

// ---- output staging through LDS (GEMM epilogues) ----
// A wave stages a block of rows of 256 bytes in LDS and stores it back with 16-byte
// lanes, 16 lanes per row, so every store instruction writes whole 128-byte lines.
// The 16-byte chunk slots of a row are xor-swizzled by the row, so 32 lanes writing
// 8 bytes at one chunk position of 32 consecutive rows, and lanes reading whole rows,
// spread over the banks.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int stg256_off(int r, int c) { return r * 256 + ((c ^ (r & 15)) << 4); }

__device__ __forceinline__ uint2 pack4_bf16(float a, float b, float c, float d) {
  return make_uint2((uint32_t)f32_to_bf16_bits(a) | ((uint32_t)f32_to_bf16_bits(b) << 16),
                    (uint32_t)f32_to_bf16_bits(c) | ((uint32_t)f32_to_bf16_bits(d) << 16));
}

// 8 bytes at byte 16*c + 8*half of staged row r
__device__ __forceinline__ void stg256_put(char* stg, int r, int c, int half, uint2 v) {
  *reinterpret_cast<uint2*>(stg + stg256_off(r, c) + 8 * half) = v;
}

// Staged rows 0 .. nrows-1 to out (row stride ld_bytes), non-temporally.  Waits for the
// wave's own staging writes first and for its reads at the end, so the area can be
// written again by the same wave; other waves must be kept off it by the caller.
__device__ __forceinline__ void stg256_flush(const char* stg, int lane, int nrows, char* out,
                                             int64_t ld_bytes) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  const int c = lane & 15;
  for (int r = lane >> 4; r < nrows; r += 4) {
    const uint4 u = *reinterpret_cast<const uint4*>(stg + stg256_off(r, c));
    const u32x4 v = {u.x, u.y, u.z, u.w};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(out + r * ld_bytes + 16 * c));
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// ---------------------------------------------------------------------------
// exp and sigmoid of the router (shared by the routing and its backward).  ln 2 is split for Cody-Waite reduction: the high part is ln 2
// rounded to 16 significant bits (45426/65536) so k*LN2_HI is exact for |k| < 256;
// the low part is the float nearest ln 2 - LN2_HI.  The polynomial is the Taylor
// series of exp to degree 7 with coefficients rounded to float (1/n!).  |a| <= 80
// keeps k within [-116, 116] and 2^k a normal float, so the final scaling is exact.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float exp_cw7(float a) {
  constexpr float kInvLn2 = 0x1.715476p+0f;
  constexpr float kLn2Hi = 0x1.62e4p-1f;
  constexpr float kLn2Lo = 0x1.7f7d1cp-20f;
  const float k = __builtin_rintf(a * kInvLn2);
  float r = __builtin_fmaf(-k, kLn2Hi, a);
  r = __builtin_fmaf(-k, kLn2Lo, r);
  float p = 0x1.a01a02p-13f;
  p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);
  p = __builtin_fmaf(p, r, 0x1.111112p-7f);
  p = __builtin_fmaf(p, r, 0x1.555556p-5f);
  p = __builtin_fmaf(p, r, 0x1.555556p-3f);
  p = __builtin_fmaf(p, r, 0.5f);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  return p * __uint_as_float(static_cast<uint32_t>(static_cast<int>(k) + 127) << 23);
}

__device__ __forceinline__ float affinity(float z) {
  const float zc = __builtin_fminf(__builtin_fmaxf(z, -80.0f), 80.0f);
  return 1.0f / (1.0f + exp_cw7(-zc));
}

// ---- launchers (each returns hipGetLastError() of its launch) ----
struct Dims {
  int64_t T;
  int H, E, G, M, K, J, I, S;
  int act, expert;  // moe_dtype codes
  int64_t R() const { return T * K + (S ? T : 0); }
};

hipError_t launch_route(const Dims& d, const void* x, const float* w_router, const float* bias,
                        int32_t* idx, float* gate, int32_t* counts, float* logits,
                        hipStream_t st);

size_t permute_ws_bytes(const Dims& d);
// The permute's device-resident scratch (moe_permute_noalloc): its size, and its device
// address on the current device (looked up once per device).
size_t permute_scratch_capacity();
hipError_t permute_scratch(void** ptr);
// pairs of idx [T,K] outside [0,E), counted into *n_invalid (cleared first)
hipError_t launch_count_invalid(const Dims& d, const int32_t* idx, int32_t* n_invalid,
                                hipStream_t st);
// x_sorted == nullptr: only offsets, sorted_token and inv_perm are written
hipError_t launch_permute(const Dims& d, const void* x, const int32_t* idx, int32_t* offsets,
                          int32_t* sorted_token, int32_t* inv_perm, void* x_sorted,
                          float* x_scale, void* ws, hipStream_t st);

size_t ffn_ws_bytes(const Dims& d);
float* ffn_ws_h_scale(const Dims& d, void* ws);
// gather: nullptr (xs is the permuted x_sorted) or sorted_token (xs is the unpermuted
// input, [T, H], and row r of the permuted order is xs row gather[r])
// au != nullptr (bf16 / fp32 paths): the gate and up pre-activations, [R, 2I] at the
// activation dtype, are written as well (for the backward)
hipError_t launch_ffn_up(const Dims& d, const void* xs, const float* xs_scale,
                         const int32_t* offsets, const int32_t* gather, const void* w13,
                         const float* w13_scale, void* h, float* h_scale, hipStream_t st,
                         void* au = nullptr);
hipError_t launch_ffn_down(const Dims& d, const void* h, const float* h_scale,
                           const int32_t* offsets, const void* w2, const float* w2_scale, void* ys,
                           hipStream_t st);
// The shared expert's gate/up GEMM + SwiGLU as a dense launch (bf16: gemm_dense.hip,
// FP8: gemm_fp8.hip), used when it has at least kDenseSharedMinRows rows (T); the
// grouped gate/up launch then covers the routed experts only.  x [M, Kd] in token order, w13 [2*half, Kd]
// (gate rows, then up rows), h [M, half], au [M, 2*half] optional.
constexpr int64_t kDenseSharedMinRows = 2048;
bool dense_shared(const Dims& d);
hipError_t launch_dense_swiglu_bf16(const uint16_t* x, const uint16_t* w13, uint16_t* h,
                                    uint16_t* au, int M, int Kd, int half, hipStream_t st);
// the shared expert's FP8 gate/up as its dense launch (rows T*K .. T*K+T-1 of the
// permuted order; gather != nullptr: xs is x itself, in token order)
hipError_t launch_dense_swiglu_fp8_shared(const Dims& d, const void* xs, const float* xs_scale,
                                          const int32_t* gather, const void* w13,
                                          const float* w13_scale, void* h, float* h_scale,
                                          hipStream_t st);
hipError_t launch_fp8_up(const Dims& d, const void* xs, const float* xs_scale,
                         const int32_t* offsets, const int32_t* gather, const void* w13,
                         const float* w13_scale, void* h, float* h_scale, hipStream_t st);
hipError_t launch_quantize_act(const Dims& d, const uint16_t* x, uint8_t* xq, float* x_scale,
                               hipStream_t st);
hipError_t launch_fp8_down(const Dims& d, const void* h, const float* h_scale,
                           const int32_t* offsets, const void* w2, const float* w2_scale, void* ys,
                           hipStream_t st);

// bf16 expert GEMMs over packed weights (gemm_packed.hip): the layout, its sizes
// (elements, equal to the natural layout's) and the pack; the gate/up launch takes the
// natural w13 as well, for the shared expert's dense launch (dense_shared)
bool packed_supported(const Dims& d);
size_t packed_w13_elems(const Dims& d);
size_t packed_w2_elems(const Dims& d);
hipError_t launch_pack_weights(const Dims& d, const void* w13, const void* w2, void* p13,
                               void* p2, hipStream_t st);
hipError_t launch_ffn_up_packed(const Dims& d, const void* xs, const int32_t* offsets,
                                const int32_t* gather, const void* w13, const void* p13, void* h,
                                void* au, hipStream_t st);
hipError_t launch_ffn_down_packed(const Dims& d, const void* h, const int32_t* offsets,
                                  const void* p2, void* ys, hipStream_t st);
// the backward input part over packed transposed weights (bf16): W2^T and W13^T in the
// down layout, dh -> [da|du] and dx_sorted = [da|du] W13
hipError_t launch_pack_weights_t(const Dims& d, const void* w13, const void* w2, void* p13t,
                                 void* p2t, hipStream_t st);
hipError_t launch_ffn_bwd_input_packed(const Dims& d, const int32_t* offsets, const void* p13t,
                                       const void* p2t, const void* au, const void* dys,
                                       void* dau, void* dxs, hipStream_t st);
// FP8 expert GEMMs over packed weight codes (gemm_packed_fp8.hip)
hipError_t launch_pack_weights_fp8(const Dims& d, const void* w13, const void* w2, void* p13,
                                   void* p2, hipStream_t st);
hipError_t launch_ffn_up_packed_fp8(const Dims& d, const void* xs, const float* xs_scale,
                                    const int32_t* offsets, const int32_t* gather,
                                    const void* w13, const void* p13, const float* w13_scale,
                                    void* h, float* h_scale, hipStream_t st);
hipError_t launch_ffn_down_packed_fp8(const Dims& d, const void* h, const float* h_scale,
                                      const int32_t* offsets, const void* p2,
                                      const float* w2_scale, void* ys, hipStream_t st);

hipError_t launch_combine(const Dims& d, const void* ys, const int32_t* inv_perm,
                          const float* gate, void* y, hipStream_t st);

hipError_t launch_bias_update(const Dims& d, const int32_t* counts, float gamma, float* bias,
                              hipStream_t st);

// sequence-wise loads (seqstats.hip): counts [n_seq, E], stats [n_seq, 3], ratio [n_seq]
hipError_t launch_seq_load_stats(const Dims& d, const int32_t* idx, const int32_t* seq_off,
                                 int n_seq, int32_t* counts, int32_t* stats, float* ratio,
                                 hipStream_t st);

hipError_t launch_quantize_weights(const uint16_t* w, uint8_t* q, float* scale, int64_t batch,
                                   int rows, int cols, hipStream_t st);

// backward (backward.hip, gemm_bwd.hip)
hipError_t launch_combine_bwd(const Dims& d, const void* dy, const void* ys,
                              const int32_t* inv_perm, const float* gate, void* dys, float* dgate,
                              hipStream_t st);
hipError_t launch_router_bwd(const Dims& d, const void* x, const float* w, const float* z,
                             const int32_t* idx, const float* gate, const float* dgate,
                             const int32_t* offsets, const int32_t* sorted_token, float* dz,
                             float* dxr, float* dw, hipStream_t st);
hipError_t launch_unpermute_sum(const Dims& d, const void* dxs, const int32_t* inv_perm,
                                const float* dxr, void* dx, hipStream_t st);
// expert backward, input part: dys -> dau -> dxs
hipError_t launch_ffn_bwd_input(const Dims& d, const int32_t* offsets, const void* w13,
                                const void* w2, const void* au, const void* dys, void* dau,
                                void* dxs, hipStream_t st);
// expert backward, weight part; x: x_sorted (gather == nullptr) or x [T, H] read
// through gather = sorted_token
hipError_t launch_ffn_bwd_weight(const Dims& d, const void* x, const int32_t* gather,
                                 const int32_t* offsets, const void* h, const void* dys,
                                 const void* dau, float* dw13, float* dw2, hipStream_t st);

int device_cu_count();

}  // namespace moe
