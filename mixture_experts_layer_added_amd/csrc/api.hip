// C ABI of libmoe: argument validation, workspace layout and launches.
// Every call validates first and enqueues nothing when it returns an error.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "common.h"

namespace moe {

namespace {
thread_local char g_err[512] = "";

moe_status fail(moe_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status fail(moe_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

moe_status hip_fail(hipError_t e, const char* what) {
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
int g_dev_cus[kMaxDevices];
bool g_dev_ok[kMaxDevices];

// Device checks are cached per device: gfx950 and its CU count.
moe_status check_device(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d out of range", dev);
  std::call_once(g_dev_once[dev], [dev] {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess) {
      g_dev_ok[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
      g_dev_cus[dev] = prop.multiProcessorCount;
    }
  });
  if (!g_dev_ok[dev]) return fail(MOE_ERR_UNSUPPORTED, "device %d is not gfx950 (MI355X)", dev);
  if (cus) *cus = g_dev_cus[dev];
  return MOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

moe_status validate(const moe_problem* p, Dims* d) {
  if (!p) return fail(MOE_ERR_INVALID_ARG, "problem is NULL");
  if (p->T < 1) return fail(MOE_ERR_INVALID_ARG, "T=%lld must be >= 1", (long long)p->T);
  if (p->K < 1 || p->K > 16) return fail(MOE_ERR_INVALID_ARG, "K=%d must be in [1,16]", p->K);
  if (p->T * (int64_t)(p->K + 1) >= (int64_t)1 << 31)
    return fail(MOE_ERR_INVALID_ARG, "T*(K+1) must be < 2^31");
  if (p->H < 128 || p->H > 65536 || p->H % 128)
    return fail(MOE_ERR_INVALID_ARG, "H=%d must be a multiple of 128 in [128,65536]", p->H);
  if (p->I < 128 || p->I > 32768 || p->I % 128)
    return fail(MOE_ERR_INVALID_ARG, "I=%d must be a multiple of 128 in [128,32768]", p->I);
  if ((int64_t)p->H * p->I > ((int64_t)1 << 28))
    return fail(MOE_ERR_INVALID_ARG, "H*I=%lld must be <= 2^28 (32-bit buffer offsets)",
                (long long)p->H * p->I);
  if (p->E < 1 || p->E > 512) return fail(MOE_ERR_INVALID_ARG, "E=%d must be in [1,512]", p->E);
  if (p->G < 1 || p->G > 64 || p->E % p->G)
    return fail(MOE_ERR_INVALID_ARG, "G=%d must divide E=%d and be in [1,64]", p->G, p->E);
  const int gs = p->E / p->G;
  if (p->M < 1 || p->M > p->G) return fail(MOE_ERR_INVALID_ARG, "M=%d must be in [1,G]", p->M);
  if (p->J < 1 || p->J > gs || p->J > 8)
    return fail(MOE_ERR_INVALID_ARG, "J=%d must be in [1,min(E/G,8)]", p->J);
  if (p->K > p->M * gs) return fail(MOE_ERR_INVALID_ARG, "K=%d exceeds M*E/G=%d", p->K, p->M * gs);
  if (p->S != 0 && p->S != 1) return fail(MOE_ERR_INVALID_ARG, "S=%d must be 0 or 1", p->S);
  const bool ok_dtypes = (p->act_dtype == MOE_F32 && p->expert_dtype == MOE_F32) ||
                         (p->act_dtype == MOE_BF16 &&
                          (p->expert_dtype == MOE_BF16 || p->expert_dtype == MOE_FP8_E4M3));
  if (!ok_dtypes)
    return fail(MOE_ERR_INVALID_ARG, "dtypes act=%d expert=%d not supported", p->act_dtype,
                p->expert_dtype);
  d->T = p->T; d->H = p->H; d->E = p->E; d->G = p->G; d->M = p->M; d->K = p->K;
  d->J = p->J; d->I = p->I; d->S = p->S; d->act = p->act_dtype; d->expert = p->expert_dtype;
  return MOE_OK;
}

size_t route_ws_bytes(const Dims& d) { return sizeof(float) * (size_t)d.T * d.E; }

#define REQUIRE_PTR(ptr)                                                   \
  do {                                                                     \
    if (!(ptr)) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", #ptr);      \
    if (!aligned16(ptr)) return fail(MOE_ERR_INVALID_ARG, "%s is not 16-byte aligned", #ptr); \
  } while (0)

}  // namespace

int device_cu_count() {
  int cus = 0;
  if (check_device(&cus) != MOE_OK || cus <= 0) return 256;
  return cus;
}

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* moe_last_error(void) { return g_err; }

size_t moe_workspace_bytes(const moe_problem* p, int32_t which_call) {
  Dims d;
  if (validate(p, &d) != MOE_OK) return 0;
  switch (which_call) {
    case MOE_CALL_ROUTE: return route_ws_bytes(d);
    case MOE_CALL_PERMUTE: return permute_ws_bytes(d);
    case MOE_CALL_EXPERT_FFN: return ffn_ws_bytes(d);
  }
  fail(MOE_ERR_INVALID_ARG, "unknown call id %d", which_call);
  return 0;
}

moe_status moe_route(const moe_problem* p, const void* x, const float* w_router,
                     const float* bias, int32_t* topk_idx, float* topk_gate,
                     int32_t* expert_counts, float* logits_out, void* ws, size_t ws_bytes,
                     void* stream) {
  Dims d;
  moe_status s = validate(p, &d);
  if (s != MOE_OK) return s;
  REQUIRE_PTR(x);
  REQUIRE_PTR(w_router);
  if (!bias || !topk_idx || !topk_gate || !expert_counts)
    return fail(MOE_ERR_INVALID_ARG, "bias, topk_idx, topk_gate and expert_counts are required");
  float* z = logits_out;
  if (!z) {
    if (!ws || ws_bytes < route_ws_bytes(d))
      return fail(MOE_ERR_WORKSPACE, "route needs %zu workspace bytes, got %zu",
                  route_ws_bytes(d), ws ? ws_bytes : (size_t)0);
    z = static_cast<float*>(ws);
  }
  if ((s = check_device(nullptr)) != MOE_OK) return s;
  hipError_t e = launch_route(d, x, w_router, bias, topk_idx, topk_gate, expert_counts, z,
                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_route launch");
}

moe_status moe_permute(const moe_problem* p, const void* x, const int32_t* topk_idx,
                       int32_t* offsets, int32_t* sorted_token, int32_t* inv_perm,
                       void* x_sorted, float* x_sorted_scale, void* ws, size_t ws_bytes,
                       void* stream) {
  Dims d;
  moe_status s = validate(p, &d);
  if (s != MOE_OK) return s;
  if (!topk_idx || !offsets || !sorted_token || !inv_perm)
    return fail(MOE_ERR_INVALID_ARG, "topk_idx, offsets, sorted_token and inv_perm are required");
  if (x_sorted) {  // NULL: index maps only
    REQUIRE_PTR(x);
    REQUIRE_PTR(x_sorted);
    if (d.expert == MOE_FP8_E4M3 && !x_sorted_scale)
      return fail(MOE_ERR_INVALID_ARG, "x_sorted_scale is required for the FP8 path");
  }
  if (!ws || ws_bytes < permute_ws_bytes(d))
    return fail(MOE_ERR_WORKSPACE, "permute needs %zu workspace bytes, got %zu",
                permute_ws_bytes(d), ws ? ws_bytes : (size_t)0);
  if ((s = check_device(nullptr)) != MOE_OK) return s;
  hipError_t e = launch_permute(d, x, topk_idx, offsets, sorted_token, inv_perm, x_sorted,
                                x_sorted_scale, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_permute launch");
}

moe_status moe_count_invalid_ids(const moe_problem* p, const int32_t* topk_idx,
                                 int32_t* n_invalid, void* stream) {
  Dims d;
  moe_status s = validate(p, &d);
  if (s != MOE_OK) return s;
  REQUIRE_PTR(topk_idx);
  REQUIRE_PTR(n_invalid);
  if ((s = check_device(nullptr)) != MOE_OK) return s;
  const hipError_t e = launch_count_invalid(d, topk_idx, n_invalid, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_count_invalid_ids launch");
}

moe_status moe_permute_noalloc(const moe_problem* p, const void* x, const int32_t* topk_idx,
                               int32_t* offsets, int32_t* sorted_token, int32_t* inv_perm,
                               void* x_sorted, float* x_sorted_scale, void* stream) {
  Dims d;
  moe_status s = validate(p, &d);
  if (s != MOE_OK) return s;
  if (!topk_idx || !offsets || !sorted_token || !inv_perm)
    return fail(MOE_ERR_INVALID_ARG, "topk_idx, offsets, sorted_token and inv_perm are required");
  if (x_sorted) {  // NULL: index maps only
    REQUIRE_PTR(x);
    REQUIRE_PTR(x_sorted);
    if (d.expert == MOE_FP8_E4M3 && !x_sorted_scale)
      return fail(MOE_ERR_INVALID_ARG, "x_sorted_scale is required for the FP8 path");
  }
  if (permute_ws_bytes(d) > permute_scratch_capacity())
    return fail(MOE_ERR_WORKSPACE,
                "moe_permute_noalloc: this problem needs %zu scratch bytes, the library holds "
                "%zu (T*K + 2*ceil(T/256)*E must be at most %zu); use moe_permute",
                permute_ws_bytes(d), permute_scratch_capacity(),
                (permute_scratch_capacity() - 256) / sizeof(int32_t));
  if ((s = check_device(nullptr)) != MOE_OK) return s;
  void* ws = nullptr;
  hipError_t e = permute_scratch(&ws);
  if (e != hipSuccess) return hip_fail(e, "moe_permute_noalloc: device address of the scratch");
  e = launch_permute(d, x, topk_idx, offsets, sorted_token, inv_perm, x_sorted, x_sorted_scale,
                     ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_permute_noalloc launch");
}

moe_status moe_expert_ffn_up(const moe_problem* p, const void* x_sorted,
                             const float* x_sorted_scale, const int32_t* offsets,
                             const void* w13, const float* w13_scale, void* h, float* h_scale,
                             void* stream) {
  Dims d;
  moe_status s = validate(p, &d);
  if (s != MOE_OK) return s;
  REQUIRE_PTR(x_sorted);
  REQUIRE_PTR(w13);
  REQUIRE_PTR(h);
  if (!offsets) return fail(MOE_ERR_INVALID_ARG, "offsets is NULL");
  if (d.expert == MOE_FP8_E4M3 && (!x_sorted_scale || !w13_scale || !h_scale))
    return fail(MOE_ERR_INVALID_ARG, "the FP8 path needs x_sorted_scale, w13_scale, h_scale");
  if ((s = check_device(nullptr)) != MOE_OK) return s;
  hipError_t e = launch_ffn_up(d, x_sorted, x_sorted_scale, offsets, nullptr, w13, w13_scale, h,
                               h_scale, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported)
    return fail(MOE_ERR_UNSUPPORTED, "no expert FFN kernel for expert dtype %d", d.expert);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_expert_ffn_up launch");
}

moe_status moe_expert_ffn_up_gather(const moe_problem* p, const void* x, const float* x_scale,
                                    const int32_t* sorted_token, const int32_t* offsets,
                                    const void* w13, const float* w13_scale, void* h,
                                    float* h_scale, void* stream) {
  Dims d;
  moe_status s = validate(p, &d);
  if (s != MOE_OK) return s;
  REQUIRE_PTR(x);
  REQUIRE_PTR(w13);
  REQUIRE_PTR(h);
  if (!offsets || !sorted_token)
    return fail(MOE_ERR_INVALID_ARG, "offsets and sorted_token are required");
  if (d.expert == MOE_FP8_E4M3 && (!x_scale || !w13_scale || !h_scale))
    return fail(MOE_ERR_INVALID_ARG, "the FP8 path needs x_scale, w13_scale, h_scale");
  const int es = d.expert == MOE_FP8_E4M3 ? 1 : (d.expert == MOE_F32 ? 4 : 2);
  if (d.T * (int64_t)d.H * es >= ((int64_t)1 << 31) - 16)
    return fail(MOE_ERR_INVALID_ARG, "T*H*%d must be < 2^31 - 16 (32-bit row offsets)", es);
  if ((s = check_device(nullptr)) != MOE_OK) return s;
  hipError_t e = launch_ffn_up(d, x, x_scale, offsets, sorted_token, w13, w13_scale, h, h_scale,
                               static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported)
    return fail(MOE_ERR_UNSUPPORTED, "no expert FFN kernel for expert dtype %d", d.expert);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_expert_ffn_up_gather launch");
}

moe_status moe_quantize_act_fp8(const moe_problem* p, const void* x, void* x_q, float* x_scale,
                                void* stream) {
  Dims d;
  moe_status s = validate(p, &d);
  if (s != MOE_OK) return s;
  if (d.expert != MOE_FP8_E4M3 || d.act != MOE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "moe_quantize_act_fp8 needs act BF16 and expert FP8_E4M3");
  REQUIRE_PTR(x);
  REQUIRE_PTR(x_q);
  if (!x_scale) return fail(MOE_ERR_INVALID_ARG, "x_scale is NULL");
  if ((s = check_device(nullptr)) != MOE_OK) return s;
  hipError_t e = launch_quantize_act(d, static_cast<const uint16_t*>(x), static_cast<uint8_t*>(x_q),
                                     x_scale, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_quantize_act_fp8 launch");
}

moe_status moe_expert_ffn_down(const moe_problem* p, const void* h, const float* h_scale,
                               const int32_t* offsets, const void* w2, const float* w2_scale,
                               void* y_sorted, void* stream) {
  Dims d;
  moe_status s = validate(p, &d);
  if (s != MOE_OK) return s;
  REQUIRE_PTR(h);
  REQUIRE_PTR(w2);
  REQUIRE_PTR(y_sorted);
  if (!offsets) return fail(MOE_ERR_INVALID_ARG, "offsets is NULL");
  if (d.expert == MOE_FP8_E4M3 && (!h_scale || !w2_scale))
    return fail(MOE_ERR_INVALID_ARG, "the FP8 path needs h_scale and w2_scale");
  if ((s = check_device(nullptr)) != MOE_OK) return s;
  hipError_t e = launch_ffn_down(d, h, h_scale, offsets, w2, w2_scale, y_sorted,
                                 static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported)
    return fail(MOE_ERR_UNSUPPORTED, "no expert FFN kernel for expert dtype %d", d.expert);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_expert_ffn_down launch");
}

moe_status moe_expert_ffn(const moe_problem* p, const void* x_sorted,
                          const float* x_sorted_scale, const int32_t* offsets,
                          const void* w13, const float* w13_scale, const void* w2,
                          const float* w2_scale, void* y_sorted, void* ws, size_t ws_bytes,
                          void* stream) {
  Dims d;
  moe_status s = validate(p, &d);
  if (s != MOE_OK) return s;
  REQUIRE_PTR(x_sorted);
  REQUIRE_PTR(w13);
  REQUIRE_PTR(w2);
  REQUIRE_PTR(y_sorted);
  if (!offsets) return fail(MOE_ERR_INVALID_ARG, "offsets is NULL");
  if (d.expert == MOE_FP8_E4M3 && (!x_sorted_scale || !w13_scale || !w2_scale))
    return fail(MOE_ERR_INVALID_ARG, "the FP8 path needs x_sorted_scale, w13_scale, w2_scale");
  if (!ws || ws_bytes < ffn_ws_bytes(d) || !aligned16(ws))
    return fail(MOE_ERR_WORKSPACE, "expert_ffn needs %zu aligned workspace bytes, got %zu",
                ffn_ws_bytes(d), ws ? ws_bytes : (size_t)0);
  float* h_scale = d.expert == MOE_FP8_E4M3 ? ffn_ws_h_scale(d, ws) : nullptr;
  s = moe_expert_ffn_up(p, x_sorted, x_sorted_scale, offsets, w13, w13_scale, ws, h_scale, stream);
  if (s != MOE_OK) return s;
  return moe_expert_ffn_down(p, ws, h_scale, offsets, w2, w2_scale, y_sorted, stream);
}

moe_status moe_combine(const moe_problem* p, const void* y_sorted, const int32_t* inv_perm,
                       const float* topk_gate, void* y, void* stream) {
  Dims d;
  moe_status s = validate(p, &d);
  if (s != MOE_OK) return s;
  REQUIRE_PTR(y_sorted);
  REQUIRE_PTR(y);
  if (!inv_perm || !topk_gate)
    return fail(MOE_ERR_INVALID_ARG, "inv_perm and topk_gate are required");
  if ((s = check_device(nullptr)) != MOE_OK) return s;
  hipError_t e = launch_combine(d, y_sorted, inv_perm, topk_gate, y,
                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_combine launch");
}

moe_status moe_bias_update(const moe_problem* p, const int32_t* expert_counts, float gamma,
                           float* bias, void* stream) {
  Dims d;
  moe_status s = validate(p, &d);
  if (s != MOE_OK) return s;
  if (!expert_counts || !bias)
    return fail(MOE_ERR_INVALID_ARG, "expert_counts and bias are required");
  if (!(gamma >= 0.0f) || gamma > 1e30f)
    return fail(MOE_ERR_INVALID_ARG, "gamma must be finite and >= 0");
  if ((s = check_device(nullptr)) != MOE_OK) return s;
  hipError_t e = launch_bias_update(d, expert_counts, gamma, bias,
                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_bias_update launch");
}

moe_status moe_seq_load_stats(const moe_problem* p, const int32_t* topk_idx,
                              const int32_t* seq_offsets, int32_t n_seq, int32_t* seq_counts,
                              int32_t* seq_stats, float* seq_ratio, void* stream) {
  Dims d;
  moe_status s = validate(p, &d);
  if (s != MOE_OK) return s;
  if (!topk_idx || !seq_offsets || !seq_counts || !seq_stats || !seq_ratio)
    return fail(MOE_ERR_INVALID_ARG,
                "topk_idx, seq_offsets, seq_counts, seq_stats and seq_ratio are required");
  if (n_seq < 1 || n_seq > (1 << 24) || (int64_t)n_seq * d.E >= ((int64_t)1 << 31))
    return fail(MOE_ERR_INVALID_ARG, "n_seq=%d must be in [1, 2^24] with n_seq*E < 2^31", n_seq);
  if ((s = check_device(nullptr)) != MOE_OK) return s;
  hipError_t e = launch_seq_load_stats(d, topk_idx, seq_offsets, n_seq, seq_counts, seq_stats,
                                       seq_ratio, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_seq_load_stats launch");
}

static moe_status require_no_fp8(const Dims& d, const char* call) {
  if (d.expert == MOE_FP8_E4M3)
    return fail(MOE_ERR_UNSUPPORTED, "%s: the backward is built for the bf16 and fp32 paths", call);
  return MOE_OK;
}

moe_status moe_combine_backward(const moe_problem* p, const void* dy, const void* y_sorted,
                                const int32_t* inv_perm, const float* topk_gate, void* dy_sorted,
                                float* dgate, void* stream) {
  Dims d;
  moe_status s = validate(p, &d);
  if (s != MOE_OK) return s;
  if ((s = require_no_fp8(d, "moe_combine_backward")) != MOE_OK) return s;
  REQUIRE_PTR(dy);
  REQUIRE_PTR(y_sorted);
  REQUIRE_PTR(dy_sorted);
  if (!inv_perm || !topk_gate || !dgate)
    return fail(MOE_ERR_INVALID_ARG, "inv_perm, topk_gate and dgate are required");
  if ((s = check_device(nullptr)) != MOE_OK) return s;
  hipError_t e = launch_combine_bwd(d, dy, y_sorted, inv_perm, topk_gate, dy_sorted, dgate,
                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_combine_backward launch");
}

moe_status moe_router_backward(const moe_problem* p, const void* x, const float* w_router,
                               const float* logits, const int32_t* topk_idx,
                               const float* topk_gate, const float* dgate,
                               const int32_t* offsets, const int32_t* sorted_token, float* dz,
                               float* dx_router, float* dw_router, void* stream) {
  Dims d;
  moe_status s = validate(p, &d);
  if (s != MOE_OK) return s;
  if ((s = require_no_fp8(d, "moe_router_backward")) != MOE_OK) return s;
  REQUIRE_PTR(x);
  REQUIRE_PTR(w_router);
  REQUIRE_PTR(dx_router);
  REQUIRE_PTR(dw_router);
  if (!logits || !topk_idx || !topk_gate || !dgate || !offsets || !sorted_token || !dz)
    return fail(MOE_ERR_INVALID_ARG,
                "logits, topk_idx, topk_gate, dgate, offsets, sorted_token and dz are required");
  if ((s = check_device(nullptr)) != MOE_OK) return s;
  hipError_t e = launch_router_bwd(d, x, w_router, logits, topk_idx, topk_gate, dgate, offsets,
                                   sorted_token, dz, dx_router, dw_router,
                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_router_backward launch");
}

moe_status moe_unpermute_sum(const moe_problem* p, const void* dx_sorted,
                             const int32_t* inv_perm, const float* dx_router, void* dx,
                             void* stream) {
  Dims d;
  moe_status s = validate(p, &d);
  if (s != MOE_OK) return s;
  if ((s = require_no_fp8(d, "moe_unpermute_sum")) != MOE_OK) return s;
  REQUIRE_PTR(dx_sorted);
  REQUIRE_PTR(dx);
  if (dx_router && !aligned16(dx_router))
    return fail(MOE_ERR_INVALID_ARG, "dx_router is not 16-byte aligned");
  if (!inv_perm) return fail(MOE_ERR_INVALID_ARG, "inv_perm is NULL");
  if ((s = check_device(nullptr)) != MOE_OK) return s;
  hipError_t e = launch_unpermute_sum(d, dx_sorted, inv_perm, dx_router, dx,
                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_unpermute_sum launch");
}

moe_status moe_expert_ffn_up_save(const moe_problem* p, const void* x,
                                  const int32_t* sorted_token, const int32_t* offsets,
                                  const void* w13, void* h, void* au, void* stream) {
  Dims d;
  moe_status s = validate(p, &d);
  if (s != MOE_OK) return s;
  if ((s = require_no_fp8(d, "moe_expert_ffn_up_save")) != MOE_OK) return s;
  REQUIRE_PTR(x);
  REQUIRE_PTR(w13);
  REQUIRE_PTR(h);
  REQUIRE_PTR(au);
  if (!offsets) return fail(MOE_ERR_INVALID_ARG, "offsets is NULL");
  const int es = d.expert == MOE_F32 ? 4 : 2;
  if (sorted_token && d.T * (int64_t)d.H * es >= ((int64_t)1 << 31) - 16)
    return fail(MOE_ERR_INVALID_ARG, "T*H*%d must be < 2^31 - 16 (32-bit row offsets)", es);
  if ((s = check_device(nullptr)) != MOE_OK) return s;
  hipError_t e = launch_ffn_up(d, x, nullptr, offsets, sorted_token, w13, nullptr, h, nullptr,
                               static_cast<hipStream_t>(stream), au);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_expert_ffn_up_save launch");
}

static moe_status check_bwd_rows(const Dims& d) {
  const int es = d.expert == MOE_F32 ? 4 : 2;
  const int64_t widest = d.H > 2 * d.I ? d.H : 2 * d.I;
  if (d.R() * widest * es >= ((int64_t)1 << 31) - 16)
    return fail(MOE_ERR_INVALID_ARG,
                "R*max(H,2I)*%d must be < 2^31 - 16 (32-bit row offsets in the backward)", es);
  return MOE_OK;
}

moe_status moe_expert_ffn_backward_input(const moe_problem* p, const int32_t* offsets,
                                         const void* w13, const void* w2, const void* au,
                                         const void* dy_sorted, void* dau, void* dx_sorted,
                                         void* stream) {
  Dims d;
  moe_status s = validate(p, &d);
  if (s != MOE_OK) return s;
  if ((s = require_no_fp8(d, "moe_expert_ffn_backward_input")) != MOE_OK) return s;
  REQUIRE_PTR(w13);
  REQUIRE_PTR(w2);
  REQUIRE_PTR(au);
  REQUIRE_PTR(dy_sorted);
  REQUIRE_PTR(dau);
  REQUIRE_PTR(dx_sorted);
  if (!offsets) return fail(MOE_ERR_INVALID_ARG, "offsets is NULL");
  if ((s = check_bwd_rows(d)) != MOE_OK) return s;
  if ((s = check_device(nullptr)) != MOE_OK) return s;
  hipError_t e = launch_ffn_bwd_input(d, offsets, w13, w2, au, dy_sorted, dau, dx_sorted,
                                      static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported)
    return fail(MOE_ERR_UNSUPPORTED, "no backward kernel for expert dtype %d", d.expert);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_expert_ffn_backward_input launch");
}

moe_status moe_expert_ffn_backward_weight(const moe_problem* p, const void* x,
                                          const int32_t* sorted_token, const int32_t* offsets,
                                          const void* h, const void* dy_sorted, const void* dau,
                                          float* dw13, float* dw2, void* stream) {
  Dims d;
  moe_status s = validate(p, &d);
  if (s != MOE_OK) return s;
  if ((s = require_no_fp8(d, "moe_expert_ffn_backward_weight")) != MOE_OK) return s;
  REQUIRE_PTR(x);
  REQUIRE_PTR(h);
  REQUIRE_PTR(dy_sorted);
  REQUIRE_PTR(dau);
  REQUIRE_PTR(dw13);
  REQUIRE_PTR(dw2);
  if (!offsets) return fail(MOE_ERR_INVALID_ARG, "offsets is NULL");
  if ((s = check_bwd_rows(d)) != MOE_OK) return s;
  if ((s = check_device(nullptr)) != MOE_OK) return s;
  hipError_t e = launch_ffn_bwd_weight(d, x, sorted_token, offsets, h, dy_sorted, dau, dw13, dw2,
                                       static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported)
    return fail(MOE_ERR_UNSUPPORTED, "no backward kernel for expert dtype %d", d.expert);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_expert_ffn_backward_weight launch");
}

static moe_status require_packed(const Dims& d, const char* call) {
  if (!packed_supported(d))
    return fail(MOE_ERR_UNSUPPORTED,
                "%s: packed weights are built for act dtype BF16 with expert dtype BF16 or FP8",
                call);
  return MOE_OK;
}

moe_status moe_pack_expert_weights(const moe_problem* p, const void* w13, const void* w2,
                                   void* w13_packed, void* w2_packed, void* stream) {
  Dims d;
  moe_status s = validate(p, &d);
  if (s != MOE_OK) return s;
  if ((s = require_packed(d, "moe_pack_expert_weights")) != MOE_OK) return s;
  if (!w13 && !w2) return fail(MOE_ERR_INVALID_ARG, "w13 and w2 are both NULL");
  if ((w13 && !w13_packed) || (w2 && !w2_packed))
    return fail(MOE_ERR_INVALID_ARG, "a packed output is NULL for a given input");
  if ((w13 && w13 == w13_packed) || (w2 && w2 == w2_packed))
    return fail(MOE_ERR_INVALID_ARG, "packing cannot run in place");
  if ((s = check_device(nullptr)) != MOE_OK) return s;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = d.expert == MOE_FP8_E4M3
                     ? launch_pack_weights_fp8(d, w13, w2, w13_packed, w2_packed, st)
                     : launch_pack_weights(d, w13, w2, w13_packed, w2_packed, st);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_pack_expert_weights launch");
}

static moe_status require_bf16_pair(const Dims& d, const char* call) {
  if (d.act != MOE_BF16 || d.expert != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "%s: built for act and expert dtype BF16", call);
  return MOE_OK;
}

moe_status moe_pack_expert_weights_transposed(const moe_problem* p, const void* w13,
                                              const void* w2, void* w13t_packed,
                                              void* w2t_packed, void* stream) {
  Dims d;
  moe_status s = validate(p, &d);
  if (s != MOE_OK) return s;
  if ((s = require_bf16_pair(d, "moe_pack_expert_weights_transposed")) != MOE_OK) return s;
  if (!w13 && !w2) return fail(MOE_ERR_INVALID_ARG, "w13 and w2 are both NULL");
  if ((w13 && !w13t_packed) || (w2 && !w2t_packed))
    return fail(MOE_ERR_INVALID_ARG, "a packed output is NULL for a given input");
  if ((w13 && w13 == w13t_packed) || (w2 && w2 == w2t_packed))
    return fail(MOE_ERR_INVALID_ARG, "packing cannot run in place");
  if ((s = check_device(nullptr)) != MOE_OK) return s;
  const hipError_t e =
      launch_pack_weights_t(d, w13, w2, w13t_packed, w2t_packed, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_pack_expert_weights_transposed launch");
}

moe_status moe_expert_ffn_backward_input_packed(const moe_problem* p, const int32_t* offsets,
                                                const void* w13t_packed,
                                                const void* w2t_packed, const void* au,
                                                const void* dy_sorted, void* dau,
                                                void* dx_sorted, void* stream) {
  Dims d;
  moe_status s = validate(p, &d);
  if (s != MOE_OK) return s;
  if ((s = require_bf16_pair(d, "moe_expert_ffn_backward_input_packed")) != MOE_OK) return s;
  REQUIRE_PTR(w13t_packed);
  REQUIRE_PTR(w2t_packed);
  REQUIRE_PTR(au);
  REQUIRE_PTR(dy_sorted);
  REQUIRE_PTR(dau);
  REQUIRE_PTR(dx_sorted);
  if (!offsets) return fail(MOE_ERR_INVALID_ARG, "offsets is NULL");
  if ((s = check_bwd_rows(d)) != MOE_OK) return s;
  if ((s = check_device(nullptr)) != MOE_OK) return s;
  const hipError_t e = launch_ffn_bwd_input_packed(d, offsets, w13t_packed, w2t_packed, au,
                                                   dy_sorted, dau, dx_sorted,
                                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_expert_ffn_backward_input_packed launch");
}

moe_status moe_expert_ffn_up_packed(const moe_problem* p, const void* x, const float* x_scale,
                                    const int32_t* sorted_token, const int32_t* offsets,
                                    const void* w13, const void* w13_packed,
                                    const float* w13_scale, void* h, float* h_scale, void* au,
                                    void* stream) {
  Dims d;
  moe_status s = validate(p, &d);
  if (s != MOE_OK) return s;
  if ((s = require_packed(d, "moe_expert_ffn_up_packed")) != MOE_OK) return s;
  REQUIRE_PTR(x);
  REQUIRE_PTR(w13);
  REQUIRE_PTR(w13_packed);
  REQUIRE_PTR(h);
  if (!offsets) return fail(MOE_ERR_INVALID_ARG, "offsets is NULL");
  const bool fp8 = d.expert == MOE_FP8_E4M3;
  if (fp8 && (!x_scale || !w13_scale || !h_scale))
    return fail(MOE_ERR_INVALID_ARG, "the FP8 path needs x_scale, w13_scale, h_scale");
  if (fp8 && au)
    return fail(MOE_ERR_INVALID_ARG, "au (the pre-activations) is kept by the bf16 path only");
  const int es = fp8 ? 1 : 2;
  if (sorted_token && d.T * (int64_t)d.H * es >= ((int64_t)1 << 31) - 16)
    return fail(MOE_ERR_INVALID_ARG, "T*H*%d must be < 2^31 - 16 (32-bit row offsets)", es);
  if ((s = check_device(nullptr)) != MOE_OK) return s;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = fp8 ? launch_ffn_up_packed_fp8(d, x, x_scale, offsets, sorted_token, w13,
                                                w13_packed, w13_scale, h, h_scale, st)
                     : launch_ffn_up_packed(d, x, offsets, sorted_token, w13, w13_packed, h, au,
                                            st);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_expert_ffn_up_packed launch");
}

moe_status moe_expert_ffn_down_packed(const moe_problem* p, const void* h, const float* h_scale,
                                      const int32_t* offsets, const void* w2_packed,
                                      const float* w2_scale, void* y_sorted, void* stream) {
  Dims d;
  moe_status s = validate(p, &d);
  if (s != MOE_OK) return s;
  if ((s = require_packed(d, "moe_expert_ffn_down_packed")) != MOE_OK) return s;
  REQUIRE_PTR(h);
  REQUIRE_PTR(w2_packed);
  REQUIRE_PTR(y_sorted);
  if (!offsets) return fail(MOE_ERR_INVALID_ARG, "offsets is NULL");
  const bool fp8 = d.expert == MOE_FP8_E4M3;
  if (fp8 && (!h_scale || !w2_scale))
    return fail(MOE_ERR_INVALID_ARG, "the FP8 path needs h_scale and w2_scale");
  if ((s = check_device(nullptr)) != MOE_OK) return s;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = fp8 ? launch_ffn_down_packed_fp8(d, h, h_scale, offsets, w2_packed, w2_scale,
                                                  y_sorted, st)
                     : launch_ffn_down_packed(d, h, offsets, w2_packed, y_sorted, st);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_expert_ffn_down_packed launch");
}

moe_status moe_quantize_weights_fp8(const void* w_bf16, void* w_fp8, float* scale,
                                    int64_t batch, int32_t rows, int32_t cols, void* stream) {
  if (batch < 1 || rows < 128 || cols < 128 || rows % 128 || cols % 128)
    return fail(MOE_ERR_INVALID_ARG, "batch >= 1 and rows, cols multiples of 128 are required");
  if (batch * (rows / 128) * (int64_t)(cols / 128) >= ((int64_t)1 << 31))
    return fail(MOE_ERR_INVALID_ARG, "too many 128x128 blocks");
  REQUIRE_PTR(w_bf16);
  REQUIRE_PTR(w_fp8);
  if (!scale) return fail(MOE_ERR_INVALID_ARG, "scale is NULL");
  moe_status s = check_device(nullptr);
  if (s != MOE_OK) return s;
  hipError_t e = launch_quantize_weights(static_cast<const uint16_t*>(w_bf16),
                                         static_cast<uint8_t*>(w_fp8), scale, batch, rows, cols,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_quantize_weights_fp8 launch");
}

}  // extern "C"
