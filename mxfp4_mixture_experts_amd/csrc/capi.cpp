// C ABI of the MXFP4 mixture-of-experts library: argument checks, the gfx950
// device check, path selection and kernel dispatch.  Declarations and the
// contract of each entry point are in include/mxfp4_moe.h.
//
// Every host-checkable precondition is tested before any HIP call, so a
// rejected call enqueues nothing and the checks work on a host without a GPU
// (the gpt-oss-20b files page, README "Loading", validates names, shapes and
// dtypes up front in the same way).

#include "mxfp4_moe.h"

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "kernels.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(MXFP4_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// gfx950 check of the current device, cached per device ordinal.
constexpr int kMaxDevices = 64;
int g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
std::mutex g_dev_mutex;

int check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MXFP4_ERR_UNSUPPORTED_DEVICE, "device ordinal %d out of range", dev);
  {
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    if (g_dev_state[dev] == 0) {
      hipDeviceProp_t prop;
      e = hipGetDeviceProperties(&prop, dev);
      if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
      g_dev_state[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
      if (g_dev_state[dev] == 2)
        return fail(MXFP4_ERR_UNSUPPORTED_DEVICE, "device %d is %s, this library runs on gfx950 only", dev,
                    prop.gcnArchName);
    }
    if (g_dev_state[dev] != 1) return fail(MXFP4_ERR_UNSUPPORTED_DEVICE, "device %d is not gfx950", dev);
  }
  return MXFP4_OK;
}

// The GEMV streams each used expert's weights once per 16 routed rows; the
// grouped GEMM pays a quantization pass but runs at the MX-FP4 MFMA rate.  The
// GEMV wins while the routed rows per expert stay around 16 or fewer.
int resolve_path(int path, int T, int k, int E) {
  if (path != MXFP4_PATH_AUTO) return path;
  const long long R = (long long)T * k;
  const long long used = R < E ? R : E;
  return R <= 16 * used ? MXFP4_PATH_GEMV : MXFP4_PATH_GEMM;
}

bool gemv_fits(int T, int K) { return mxfp4::gemv_lds_bytes(T, K) <= 160 * 1024 - 1024; }  // = kGemvMaxDynLds

// The routed projection; exactly one of out (f32 [T, k, N]) and act (bf16
// [T, k, N / 2], the gated activation) is written.
static_assert(mxfp4::kGemmStaticScratchBytes == MXFP4_NOALLOC_SCRATCH_BYTES, "one size for the static scratch");

// noalloc: the grouped GEMM's scratch is the library's static device array
// (workspace and workspace_bytes are ignored).  y != NULL: out, then y [T, N]
// = the gate-weighted combine of each token's routed slots (ids, gates [T, k]),
// fused into the grouped GEMM; on the GEMV path in the same launch while T * k
// <= E, else after the projection.
int expert_proj_impl(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias, int E, int N, int K,
                     const uint16_t* x, int x_per_slot, int T, int k, const int32_t* expert_offsets,
                     const int32_t* sorted_rows, float* out, uint16_t* act, int path, void* workspace,
                     size_t workspace_bytes, void* stream, bool noalloc = false, const int32_t* ids = nullptr,
                     const float* gates = nullptr, float* y = nullptr) {
  g_last_error[0] = '\0';
  if (E < 1 || E > MXFP4_MAX_EXPERTS) return fail(MXFP4_ERR_INVALID_ARG, "E = %d must be in [1, %d]", E, MXFP4_MAX_EXPERTS);
  if (N < 1) return fail(MXFP4_ERR_INVALID_ARG, "N = %d must be >= 1", N);
  if (act && N % 2 != 0) return fail(MXFP4_ERR_INVALID_ARG, "N = %d must be even (gate and up rows in pairs)", N);
  if (K < 32 || K % 32 != 0) return fail(MXFP4_ERR_INVALID_ARG, "K = %d must be a positive multiple of 32", K);
  if (T < 0) return fail(MXFP4_ERR_INVALID_ARG, "T = %d must be >= 0", T);
  if (k < 1 || k > E || k > MXFP4_MAX_TOPK)
    return fail(MXFP4_ERR_INVALID_ARG, "k = %d must be in [1, min(E = %d, %d)]", k, E, MXFP4_MAX_TOPK);
  if ((long long)T * k > 0x7fffffffLL) return fail(MXFP4_ERR_INVALID_ARG, "T * k overflows int32");
  if ((long long)E * N > 0x7fffffffLL) return fail(MXFP4_ERR_INVALID_ARG, "E * N overflows int32");
  if (path < MXFP4_PATH_AUTO || path > MXFP4_PATH_GEMM) return fail(MXFP4_ERR_INVALID_ARG, "path = %d unknown", path);
  if (T == 0) return MXFP4_OK;
  if (!blocks || !scales || !x || !expert_offsets || !sorted_rows || (!out && !act))
    return fail(MXFP4_ERR_INVALID_ARG, "a required pointer is NULL");
  if (y && (!out || !ids || !gates)) return fail(MXFP4_ERR_INVALID_ARG, "a required pointer is NULL");
  if (y && (size_t)T * k * N * 4 > 0xFFFFFFFFull)
    return fail(MXFP4_ERR_INVALID_ARG, "out [T, k, N] f32 must stay under 4 GiB for the fused combine");
  if (!aligned16(blocks) || !aligned16(x)) return fail(MXFP4_ERR_INVALID_ARG, "blocks and x must be 16-byte aligned");
  const int p = resolve_path(path, T, k, E);
  if (p == MXFP4_PATH_GEMV && !gemv_fits(T, K))
    return fail(MXFP4_ERR_INVALID_ARG, "K = %d too large for the GEMV path's LDS staging", K);
  if (p == MXFP4_PATH_GEMM && K > MXFP4_GEMM_MAX_K)
    return fail(MXFP4_ERR_INVALID_ARG, "K = %d above the grouped GEMM's limit %d", K, MXFP4_GEMM_MAX_K);
  if ((size_t)N * (size_t)(K / 32) * 16 > 0xFFFFFFFFull)  // one buffer resource per expert, either path
    return fail(MXFP4_ERR_INVALID_ARG, "N * K / 2 = %zu bytes per expert exceeds 4 GiB", (size_t)N * (K / 32) * 16);
  if (p == MXFP4_PATH_GEMM) {
    const size_t need = mxfp4::gemm_workspace_bytes(E, N, T, k, K, x_per_slot);
    if (noalloc) {
      if (need > MXFP4_NOALLOC_SCRATCH_BYTES)
        return fail(MXFP4_ERR_WORKSPACE, "the grouped GEMM needs %zu bytes of scratch, the static scratch holds %zu",
                    need, (size_t)MXFP4_NOALLOC_SCRATCH_BYTES);
    } else {
      if (!workspace || workspace_bytes < need)
        return fail(MXFP4_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0,
                    need);
      if (!aligned16(workspace)) return fail(MXFP4_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    }
  }
  int st = check_device();
  if (st != MXFP4_OK) return st;
  if (noalloc && p == MXFP4_PATH_GEMM) {
    const hipError_t se = mxfp4::gemm_static_scratch(&workspace);
    if (se != hipSuccess) return hip_fail(se, "static scratch address");
  }
  hipError_t e;
  if (p == MXFP4_PATH_GEMV && y) {
    e = mxfp4::launch_expert_gemv_combine(blocks, scales, bias, E, N, K, x, x_per_slot, T, k, expert_offsets,
                                          sorted_rows, ids, gates, out, y, static_cast<hipStream_t>(stream));
  } else if (p == MXFP4_PATH_GEMV) {
    e = mxfp4::launch_expert_gemv(blocks, scales, bias, E, N, K, x, x_per_slot, T, k, expert_offsets, sorted_rows,
                                  out, act, static_cast<hipStream_t>(stream));
  } else {
    e = mxfp4::launch_expert_gemm(blocks, scales, bias, E, N, K, x, x_per_slot, T, k, expert_offsets, sorted_rows,
                                  out, act, workspace, static_cast<hipStream_t>(stream), ids, gates, y);
  }
  if (e != hipSuccess) return hip_fail(e, "expert_proj launch");
  return MXFP4_OK;
}

}  // namespace

extern "C" {

const char* mxfp4_status_string(int status) {
  switch (status) {
    case MXFP4_OK: return "ok";
    case MXFP4_ERR_INVALID_ARG: return "invalid argument";
    case MXFP4_ERR_WORKSPACE: return "workspace missing or too small";
    case MXFP4_ERR_UNSUPPORTED_DEVICE: return "unsupported device (gfx950 required)";
    case MXFP4_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* mxfp4_last_error(void) { return g_last_error; }

int mxfp4_moe_route_group(const uint16_t* logits, const int32_t* ids_in, int T, int E, int k, int32_t* topk_ids,
                          float* gates, int32_t* expert_offsets, int32_t* sorted_rows, int32_t* error_word,
                          void* stream) {
  g_last_error[0] = '\0';
  if (T < 0) return fail(MXFP4_ERR_INVALID_ARG, "T = %d must be >= 0", T);
  if (E < 1 || E > MXFP4_MAX_EXPERTS) return fail(MXFP4_ERR_INVALID_ARG, "E = %d must be in [1, %d]", E, MXFP4_MAX_EXPERTS);
  if (k < 1 || k > E || k > MXFP4_MAX_TOPK)
    return fail(MXFP4_ERR_INVALID_ARG, "k = %d must be in [1, min(E = %d, %d)]", k, E, MXFP4_MAX_TOPK);
  if ((long long)T * k > 0x7fffffffLL) return fail(MXFP4_ERR_INVALID_ARG, "T * k overflows int32");
  if (T > 0 && !logits && !ids_in) return fail(MXFP4_ERR_INVALID_ARG, "one of logits / ids_in must be given");
  if (!expert_offsets) return fail(MXFP4_ERR_INVALID_ARG, "expert_offsets is NULL");
  if (T > 0 && (!topk_ids || !sorted_rows)) return fail(MXFP4_ERR_INVALID_ARG, "topk_ids / sorted_rows is NULL");
  int st = check_device();
  if (st != MXFP4_OK) return st;
  hipError_t e = mxfp4::launch_route_group(logits, ids_in, T, E, k, topk_ids, gates, expert_offsets, sorted_rows,
                                           error_word, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "route_group launch");
  return MXFP4_OK;
}

int mxfp4_moe_dense_route(const uint16_t* logits, int T, int E, int k, float* probs, void* stream) {
  g_last_error[0] = '\0';
  if (T < 0) return fail(MXFP4_ERR_INVALID_ARG, "T = %d must be >= 0", T);
  if (E < 1 || E > MXFP4_MAX_EXPERTS) return fail(MXFP4_ERR_INVALID_ARG, "E = %d must be in [1, %d]", E, MXFP4_MAX_EXPERTS);
  if (k < 1 || k > E) return fail(MXFP4_ERR_INVALID_ARG, "k = %d must be in [1, E = %d]", k, E);
  if (T == 0) return MXFP4_OK;
  if (!logits || !probs) return fail(MXFP4_ERR_INVALID_ARG, "a required pointer is NULL");
  int st = check_device();
  if (st != MXFP4_OK) return st;
  hipError_t e = mxfp4::launch_dense_route(logits, T, E, k, probs, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "dense_route launch");
  return MXFP4_OK;
}

int mxfp4_moe_router(const uint16_t* x, const uint16_t* w, const uint16_t* bias, int T, int H, int E,
                     uint16_t* logits, void* stream) {
  g_last_error[0] = '\0';
  if (T < 0) return fail(MXFP4_ERR_INVALID_ARG, "T = %d must be >= 0", T);
  if (H < 32 || H % 32 != 0) return fail(MXFP4_ERR_INVALID_ARG, "H = %d must be a positive multiple of 32", H);
  if (E < 1 || E > MXFP4_MAX_EXPERTS) return fail(MXFP4_ERR_INVALID_ARG, "E = %d must be in [1, %d]", E, MXFP4_MAX_EXPERTS);
  if (T == 0) return MXFP4_OK;
  if (!x || !w || !logits) return fail(MXFP4_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(x) || !aligned16(w)) return fail(MXFP4_ERR_INVALID_ARG, "x and w must be 16-byte aligned");
  int st = check_device();
  if (st != MXFP4_OK) return st;
  hipError_t e = mxfp4::launch_router(x, w, bias, T, H, E, logits, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "router launch");
  return MXFP4_OK;
}

size_t mxfp4_expert_proj_workspace_size(int E, int N, int T, int k, int K, int x_per_slot, int path) {
  if (E < 1 || E > MXFP4_MAX_EXPERTS || N < 1 || T < 0 || k < 1 || K < 32 || K % 32 != 0) return (size_t)-1;
  if (path < MXFP4_PATH_AUTO || path > MXFP4_PATH_GEMM) return (size_t)-1;
  if (T == 0) return 0;
  if (resolve_path(path, T, k, E) != MXFP4_PATH_GEMM) return 0;
  return mxfp4::gemm_workspace_bytes(E, N, T, k, K, x_per_slot);
}

int mxfp4_expert_proj(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias, int E, int N, int K,
                      const uint16_t* x, int x_per_slot, int T, int k, const int32_t* expert_offsets,
                      const int32_t* sorted_rows, float* out, int path, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (T > 0 && !out) return fail(MXFP4_ERR_INVALID_ARG, "out is NULL");
  return expert_proj_impl(blocks, scales, bias, E, N, K, x, x_per_slot, T, k, expert_offsets, sorted_rows, out,
                          nullptr, path, workspace, workspace_bytes, stream);
}

int mxfp4_expert_proj_noalloc(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias, int E, int N, int K,
                              const uint16_t* x, int x_per_slot, int T, int k, const int32_t* expert_offsets,
                              const int32_t* sorted_rows, float* out, int path, void* stream) {
  if (T > 0 && !out) {
    g_last_error[0] = '\0';
    return fail(MXFP4_ERR_INVALID_ARG, "out is NULL");
  }
  return expert_proj_impl(blocks, scales, bias, E, N, K, x, x_per_slot, T, k, expert_offsets, sorted_rows, out,
                          nullptr, path, nullptr, 0, stream, true);
}

int mxfp4_expert_proj_swiglu(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias, int E, int N,
                             int K, const uint16_t* x, int x_per_slot, int T, int k, const int32_t* expert_offsets,
                             const int32_t* sorted_rows, uint16_t* act, int path, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (T > 0 && !act) return fail(MXFP4_ERR_INVALID_ARG, "act is NULL");
  return expert_proj_impl(blocks, scales, bias, E, N, K, x, x_per_slot, T, k, expert_offsets, sorted_rows, nullptr,
                          act, path, workspace, workspace_bytes, stream);
}

namespace {
int moe_decode_impl(const uint16_t* logits, int E, int k, const uint8_t* blocks, const uint8_t* scales,
                    const uint16_t* bias, int N, int K, const uint16_t* x, int x_per_slot, int32_t* topk_ids,
                    float* gates, int32_t* expert_offsets, int32_t* sorted_rows, int32_t* error_word, float* out,
                    uint16_t* act, void* stream) {
  g_last_error[0] = '\0';
  if (E < 1 || E > MXFP4_DECODE_MAX_EXPERTS)
    return fail(MXFP4_ERR_INVALID_ARG, "E = %d must be in [1, %d]", E, MXFP4_DECODE_MAX_EXPERTS);
  if (k < 1 || k > E || k > MXFP4_MAX_TOPK)
    return fail(MXFP4_ERR_INVALID_ARG, "k = %d must be in [1, min(E = %d, %d)]", k, E, MXFP4_MAX_TOPK);
  if (N < 1) return fail(MXFP4_ERR_INVALID_ARG, "N = %d must be >= 1", N);
  if (act && N % 2 != 0) return fail(MXFP4_ERR_INVALID_ARG, "N = %d must be even (gate/up row pairs)", N);
  if (K < 32 || K % 32 != 0 || K > MXFP4_DECODE_MAX_K)
    return fail(MXFP4_ERR_INVALID_ARG, "K = %d must be a positive multiple of 32 up to %d", K, MXFP4_DECODE_MAX_K);
  if ((long long)E * N > 0x7fffffffLL) return fail(MXFP4_ERR_INVALID_ARG, "E * N overflows int32");
  if (!logits || !blocks || !scales || !x || !topk_ids || !expert_offsets || !sorted_rows || (!out && !act))
    return fail(MXFP4_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(blocks) || !aligned16(x)) return fail(MXFP4_ERR_INVALID_ARG, "blocks and x must be 16-byte aligned");
  int st = check_device();
  if (st != MXFP4_OK) return st;
  hipError_t e = mxfp4::launch_moe_decode_t1(logits, E, k, blocks, scales, bias, N, K, x, x_per_slot, topk_ids, gates,
                                             expert_offsets, sorted_rows, error_word, out, act,
                                             static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "moe_decode launch");
  return MXFP4_OK;
}
int moe_decode_batch_impl(const uint16_t* logits, int T, int E, int k, const uint8_t* blocks, const uint8_t* scales,
                          const uint16_t* bias, int N, int K, const uint16_t* x, int x_per_slot, int32_t* topk_ids,
                          float* gates, int32_t* expert_offsets, int32_t* sorted_rows, int32_t* error_word,
                          float* out, uint16_t* act, void* stream) {
  g_last_error[0] = '\0';
  if (T < 1 || T > MXFP4_DECODE_MAX_T)
    return fail(MXFP4_ERR_INVALID_ARG, "T = %d must be in [1, %d]", T, MXFP4_DECODE_MAX_T);
  if (E < 1 || E > MXFP4_DECODE_MAX_EXPERTS)
    return fail(MXFP4_ERR_INVALID_ARG, "E = %d must be in [1, %d]", E, MXFP4_DECODE_MAX_EXPERTS);
  if (k < 1 || k > E || k > MXFP4_MAX_TOPK)
    return fail(MXFP4_ERR_INVALID_ARG, "k = %d must be in [1, min(E = %d, %d)]", k, E, MXFP4_MAX_TOPK);
  if (N < 1) return fail(MXFP4_ERR_INVALID_ARG, "N = %d must be >= 1", N);
  if (act && N % 2 != 0) return fail(MXFP4_ERR_INVALID_ARG, "N = %d must be even (gate/up row pairs)", N);
  if (K < 32 || K % 32 != 0 || K > MXFP4_DECODE_MAX_K)
    return fail(MXFP4_ERR_INVALID_ARG, "K = %d must be a positive multiple of 32 up to %d", K, MXFP4_DECODE_MAX_K);
  if ((long long)E * N > 0x7fffffffLL) return fail(MXFP4_ERR_INVALID_ARG, "E * N overflows int32");
  if ((long long)T * k * N > 0x7fffffffLL) return fail(MXFP4_ERR_INVALID_ARG, "T * k * N overflows int32");
  if (!logits || !blocks || !scales || !x || !topk_ids || !expert_offsets || !sorted_rows || (!out && !act))
    return fail(MXFP4_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(blocks) || !aligned16(x)) return fail(MXFP4_ERR_INVALID_ARG, "blocks and x must be 16-byte aligned");
  if (!gemv_fits(T, K)) return fail(MXFP4_ERR_INVALID_ARG, "K = %d needs more LDS than a workgroup has", K);
  if ((size_t)N * (size_t)(K / 32) * 16 > 0xFFFFFFFFull)
    return fail(MXFP4_ERR_INVALID_ARG, "N * K / 2 = %zu bytes per expert exceeds 4 GiB", (size_t)N * (K / 32) * 16);
  int st = check_device();
  if (st != MXFP4_OK) return st;
  hipError_t e = mxfp4::launch_moe_decode_batch(logits, T, E, k, blocks, scales, bias, N, K, x, x_per_slot, topk_ids,
                                                gates, expert_offsets, sorted_rows, error_word, out, act,
                                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "moe_decode_batch launch");
  return MXFP4_OK;
}
}  // namespace

int mxfp4_moe_decode(const uint16_t* logits, int E, int k, const uint8_t* blocks, const uint8_t* scales,
                     const uint16_t* bias, int N, int K, const uint16_t* x, int x_per_slot, int32_t* topk_ids,
                     float* gates, int32_t* expert_offsets, int32_t* sorted_rows, int32_t* error_word, float* out,
                     void* stream) {
  if (!out) {
    g_last_error[0] = '\0';
    return fail(MXFP4_ERR_INVALID_ARG, "a required pointer is NULL");
  }
  return moe_decode_impl(logits, E, k, blocks, scales, bias, N, K, x, x_per_slot, topk_ids, gates, expert_offsets,
                         sorted_rows, error_word, out, nullptr, stream);
}

int mxfp4_moe_decode_swiglu(const uint16_t* logits, int E, int k, const uint8_t* blocks, const uint8_t* scales,
                            const uint16_t* bias, int N, int K, const uint16_t* x, int32_t* topk_ids, float* gates,
                            int32_t* expert_offsets, int32_t* sorted_rows, int32_t* error_word, uint16_t* act,
                            void* stream) {
  if (!act) {
    g_last_error[0] = '\0';
    return fail(MXFP4_ERR_INVALID_ARG, "a required pointer is NULL");
  }
  return moe_decode_impl(logits, E, k, blocks, scales, bias, N, K, x, 0, topk_ids, gates, expert_offsets,
                         sorted_rows, error_word, nullptr, act, stream);
}

int mxfp4_moe_decode_batch(const uint16_t* logits, int T, int E, int k, const uint8_t* blocks,
                           const uint8_t* scales, const uint16_t* bias, int N, int K, const uint16_t* x,
                           int x_per_slot, int32_t* topk_ids, float* gates, int32_t* expert_offsets,
                           int32_t* sorted_rows, int32_t* error_word, float* out, void* stream) {
  if (!out) {
    g_last_error[0] = '\0';
    return fail(MXFP4_ERR_INVALID_ARG, "a required pointer is NULL");
  }
  return moe_decode_batch_impl(logits, T, E, k, blocks, scales, bias, N, K, x, x_per_slot, topk_ids, gates,
                               expert_offsets, sorted_rows, error_word, out, nullptr, stream);
}

int mxfp4_moe_decode_batch_swiglu(const uint16_t* logits, int T, int E, int k, const uint8_t* blocks,
                                  const uint8_t* scales, const uint16_t* bias, int N, int K, const uint16_t* x,
                                  int32_t* topk_ids, float* gates, int32_t* expert_offsets, int32_t* sorted_rows,
                                  int32_t* error_word, uint16_t* act, void* stream) {
  if (!act) {
    g_last_error[0] = '\0';
    return fail(MXFP4_ERR_INVALID_ARG, "a required pointer is NULL");
  }
  return moe_decode_batch_impl(logits, T, E, k, blocks, scales, bias, N, K, x, 0, topk_ids, gates, expert_offsets,
                               sorted_rows, error_word, nullptr, act, stream);
}

int mxfp4_expert_proj_combine(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias, int E, int N,
                              int K, const uint16_t* x, int x_per_slot, int k, const int32_t* topk_ids,
                              const float* gates, float* out, float* y, void* stream) {
  g_last_error[0] = '\0';
  if (E < 1 || E > MXFP4_MAX_EXPERTS) return fail(MXFP4_ERR_INVALID_ARG, "E = %d must be in [1, %d]", E, MXFP4_MAX_EXPERTS);
  if (k < 1 || k > E || k > MXFP4_MAX_TOPK)
    return fail(MXFP4_ERR_INVALID_ARG, "k = %d must be in [1, min(E = %d, %d)]", k, E, MXFP4_MAX_TOPK);
  if (N < 1) return fail(MXFP4_ERR_INVALID_ARG, "N = %d must be >= 1", N);
  if (K < 32 || K % 32 != 0 || K > MXFP4_DECODE_MAX_K)
    return fail(MXFP4_ERR_INVALID_ARG, "K = %d must be a positive multiple of 32 up to %d", K, MXFP4_DECODE_MAX_K);
  if ((long long)E * N > 0x7fffffffLL) return fail(MXFP4_ERR_INVALID_ARG, "E * N overflows int32");
  if (!blocks || !scales || !x || !topk_ids || !gates || !y) return fail(MXFP4_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(blocks) || !aligned16(x)) return fail(MXFP4_ERR_INVALID_ARG, "blocks and x must be 16-byte aligned");
  int st = check_device();
  if (st != MXFP4_OK) return st;
  hipError_t e = mxfp4::launch_proj_combine_t1(blocks, scales, bias, E, N, K, x, x_per_slot, k, topk_ids, gates, out,
                                               y, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "expert_proj_combine launch");
  return MXFP4_OK;
}

int mxfp4_expert_proj_combine_routed(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias, int E,
                                     int N, int K, const uint16_t* x, int x_per_slot, int T, int k,
                                     const int32_t* topk_ids, const float* gates, const int32_t* expert_offsets,
                                     const int32_t* sorted_rows, float* out, float* y, int path, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (T > 0 && (!topk_ids || !gates || !out || !y)) {
    g_last_error[0] = '\0';
    return fail(MXFP4_ERR_INVALID_ARG, "a required pointer is NULL");
  }
  return expert_proj_impl(blocks, scales, bias, E, N, K, x, x_per_slot, T, k, expert_offsets, sorted_rows, out,
                          nullptr, path, workspace, workspace_bytes, stream, false, topk_ids, gates, y);
}

int mxfp4_dequantize(const uint8_t* blocks, const uint8_t* scales, long long rows, int K, uint16_t* out,
                     void* stream) {
  g_last_error[0] = '\0';
  if (rows < 0) return fail(MXFP4_ERR_INVALID_ARG, "rows = %lld must be >= 0", rows);
  if (K < 32 || K % 32 != 0) return fail(MXFP4_ERR_INVALID_ARG, "K = %d must be a positive multiple of 32", K);
  if (rows == 0) return MXFP4_OK;
  if (!blocks || !scales || !out) return fail(MXFP4_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(blocks) || !aligned16(out)) return fail(MXFP4_ERR_INVALID_ARG, "blocks and out must be 16-byte aligned");
  int st = check_device();
  if (st != MXFP4_OK) return st;
  hipError_t e = mxfp4::launch_dequantize(blocks, scales, (size_t)rows * (size_t)(K / 32), out,
                                          static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "dequantize launch");
  return MXFP4_OK;
}

int moe_combine(const float* proj, const float* gates, int T, int k, int N, float* y, void* stream) {
  g_last_error[0] = '\0';
  if (T < 0) return fail(MXFP4_ERR_INVALID_ARG, "T = %d must be >= 0", T);
  if (k < 1) return fail(MXFP4_ERR_INVALID_ARG, "k = %d must be >= 1", k);
  if (N < 1) return fail(MXFP4_ERR_INVALID_ARG, "N = %d must be >= 1", N);
  if (T == 0) return MXFP4_OK;
  if (!proj || !gates || !y) return fail(MXFP4_ERR_INVALID_ARG, "a required pointer is NULL");
  int st = check_device();
  if (st != MXFP4_OK) return st;
  hipError_t e = mxfp4::launch_combine(proj, gates, T, k, N, y, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return MXFP4_OK;
}

}  // extern "C"
