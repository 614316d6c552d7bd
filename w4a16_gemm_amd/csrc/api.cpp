// C ABI of the W4A16 / W4A8 linear layer library (declarations and the contract of
// every entry point are in include/w4a16.h).  This file only validates arguments,
// checks the device, picks a kernel and enqueues it on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "../../include/w4a16.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxDim = int64_t(1) << 30;

// Shape rules shared by the entry points.  K must be a positive multiple of 128 (the
// group size of the packed layout); M and N may be zero (no-op).
int check_mnk(const char* fn, int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0) return fail(W4_ERR_INVALID_ARG, "%s: negative size (M=%lld N=%lld K=%lld)", fn,
                                           (long long)M, (long long)N, (long long)K);
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim)
    return fail(W4_ERR_UNSUPPORTED, "%s: size above 2^30 (M=%lld N=%lld K=%lld)", fn, (long long)M, (long long)N,
                (long long)K);
  if (K == 0 || K % 128 != 0)
    return fail(W4_ERR_INVALID_ARG, "%s: K=%lld must be a positive multiple of 128", fn, (long long)K);
  if (N * (K / 8) > (int64_t(1) << 40))
    return fail(W4_ERR_UNSUPPORTED, "%s: N*K too large", fn);
  return W4_OK;
}

// int8 MFMA GEMMs accumulate in int32: |xq w| <= 127 * 128 per term (W4A8 per-channel
// enters as 16 q), so K <= 2^17 keeps every sum below 2^31.
constexpr int64_t kMaxKInt8 = int64_t(1) << 17;

int check_k_int8(const char* fn, int64_t K) {
  if (K > kMaxKInt8)
    return fail(W4_ERR_UNSUPPORTED, "%s: K=%lld above 131072 (int32 accumulator range)", fn, (long long)K);
  return W4_OK;
}

// W4A16 group sizes: 128, 64, 32, or -1 for per-channel (one group over K).
bool group_ok_w4a16(int32_t group_size) {
  return group_size == 128 || group_size == 64 || group_size == 32 || group_size == -1;
}

int check_group_w4a16(const char* fn, int32_t group_size) {
  if (!group_ok_w4a16(group_size))
    return fail(W4_ERR_UNSUPPORTED, "%s: group_size=%d (128, 64, 32 or -1 are implemented)", fn, group_size);
  return W4_OK;
}

// M <= 32: the skinny kernels; above, the MFMA GEMM (faster from M = 48 on the
// Llama-2-13B projection shapes, equal at 33..47 within a few percent).
bool use_skinny(int64_t M) { return M <= 32; }

int check_ptrs(const char* fn, std::initializer_list<std::pair<const char*, const void*>> ptrs) {
  for (auto& p : ptrs) {
    if (p.second == nullptr) return fail(W4_ERR_INVALID_ARG, "%s: %s is NULL", fn, p.first);
    if (!aligned16(p.second)) return fail(W4_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, p.first);
  }
  return W4_OK;
}

// 0 = unknown, 1 = gfx950, 2 = other
std::atomic<int> g_dev_ok[64];

int check_device(const char* fn) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(W4_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(W4_ERR_DEVICE, "%s: device index %d out of range", fn, dev);
  int st = g_dev_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(W4_ERR_HIP, "%s: hipGetDeviceProperties: %s", fn, hipGetErrorString(e));
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_dev_ok[dev].store(st, std::memory_order_relaxed);
    if (st == 2) return fail(W4_ERR_DEVICE, "%s: device %d is %s, this library is built for gfx950 only", fn, dev,
                             prop.gcnArchName);
  }
  if (st == 2) return fail(W4_ERR_DEVICE, "%s: device %d is not gfx950", fn, dev);
  return W4_OK;
}

int launched(const char* fn, hipError_t e) {
  if (e != hipSuccess) return fail(W4_ERR_HIP, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
  return W4_OK;
}

// The kernel choice and tile plan of one W4A16 call (computed once per call).
struct AwqPlan {
  bool skinny;
  w4::SkinnyPlan sp;
  w4::GemmPlan gp;
};

AwqPlan awq_plan(int64_t M, int64_t N, int64_t K, int32_t group_size) {
  AwqPlan p{};
  p.skinny = use_skinny(M);
  if (p.skinny) p.sp = w4::skinny_plan((int)M, (int)N, (int)K, group_size);
  else p.gp = w4::gemm_plan((int)M, (int)N, (int)K);
  return p;
}

size_t awq_ws(const AwqPlan& p, int64_t M, int64_t N) {
  if (M <= 0 || N <= 0) return 0;
  return p.skinny ? w4::skinny_workspace_bytes(p.sp, (int)M, (int)N) : w4::gemm_workspace_bytes(p.gp, (int)M, (int)N);
}

#define W4_TRY(expr)          \
  do {                        \
    const int rc_ = (expr);   \
    if (rc_ != W4_OK) return rc_; \
  } while (0)

}  // namespace

namespace w4 {
int env_int(const char* name, int dflt) {
  static const bool tuning = [] {
    const char* t = std::getenv("W4_TUNING");
    return t != nullptr && std::strcmp(t, "1") == 0;
  }();
  if (!tuning) return dflt;
  const char* v = std::getenv(name);
  if (v == nullptr || *v == 0) return dflt;
  char* end = nullptr;
  const long x = std::strtol(v, &end, 10);
  return (end && *end == 0 && x >= 0 && x < (1L << 30)) ? (int)x : dflt;
}
}  // namespace w4

extern "C" {

static int pack_w4a16(const char* fn, bool symmetric, const void* w, int32_t* qweight, void* scales,
                      int32_t* qzeros, int64_t M, int64_t N, int64_t K, int32_t group_size, void* stream) {
  g_last_error.clear();
  W4_TRY(check_group_w4a16(fn, group_size));
  W4_TRY(check_mnk(fn, M, N, K));
  if (N == 0) return W4_OK;
  W4_TRY(check_ptrs(fn, {{"w", w}, {"qweight", qweight}, {"scales", scales}, {"qzeros", qzeros}}));
  W4_TRY(check_device(fn));
  return launched(fn, w4::launch_awq_pack(w, qweight, scales, qzeros, (int)N, (int)K, group_size, symmetric,
                                          (hipStream_t)stream));
}

int awq_pack(const void* w, int32_t* qweight, void* scales, int32_t* qzeros, int64_t M, int64_t N, int64_t K,
             int32_t group_size, void* stream) {
  return pack_w4a16("awq_pack", false, w, qweight, scales, qzeros, M, N, K, group_size, stream);
}

int awq_pack_sym(const void* w, int32_t* qweight, void* scales, int32_t* qzeros, int64_t M, int64_t N, int64_t K,
                 int32_t group_size, void* stream) {
  return pack_w4a16("awq_pack_sym", true, w, qweight, scales, qzeros, M, N, K, group_size, stream);
}

int awq_unpack_dequant(const int32_t* qweight, const void* scales, const int32_t* qzeros, void* w_out, int64_t N,
                       int64_t K, int32_t group_size, void* stream) {
  const char* fn = "awq_unpack_dequant";
  g_last_error.clear();
  W4_TRY(check_group_w4a16(fn, group_size));
  W4_TRY(check_mnk(fn, 0, N, K));
  if (N == 0) return W4_OK;
  W4_TRY(check_ptrs(fn, {{"qweight", qweight}, {"scales", scales}, {"qzeros", qzeros}, {"w_out", w_out}}));
  W4_TRY(check_device(fn));
  return launched(fn, w4::launch_awq_unpack_dequant(qweight, scales, qzeros, w_out, (int)N, (int)K, group_size,
                                                    (hipStream_t)stream));
}

int w4_pack_codes(const uint8_t* codes, int32_t* out, int64_t R, int64_t C, void* stream) {
  const char* fn = "w4_pack_codes";
  g_last_error.clear();
  if (R < 0 || C < 0) return fail(W4_ERR_INVALID_ARG, "%s: negative size (R=%lld C=%lld)", fn, (long long)R, (long long)C);
  if (R > kMaxDim || C > kMaxDim || R * ((C + 7) / 8) > (int64_t(1) << 40))
    return fail(W4_ERR_UNSUPPORTED, "%s: size too large (R=%lld C=%lld)", fn, (long long)R, (long long)C);
  if (R == 0 || C == 0) return W4_OK;
  if (codes == nullptr) return fail(W4_ERR_INVALID_ARG, "%s: codes is NULL", fn);
  W4_TRY(check_ptrs(fn, {{"out", out}}));
  W4_TRY(check_device(fn));
  return launched(fn, w4::launch_pack_codes(codes, out, R, C, (hipStream_t)stream));
}

static int import_common(const char* fn, int64_t N, int64_t K, int32_t layout) {
  W4_TRY(check_mnk(fn, 0, N, K));
  if (layout != W4_LAYOUT_ROWS && layout != W4_LAYOUT_COLS)
    return fail(W4_ERR_INVALID_ARG, "%s: layout=%d (W4_LAYOUT_ROWS 0 or W4_LAYOUT_COLS 1)", fn, layout);
  return W4_OK;
}

int awq_import_plain(const int32_t* qweight_plain, const void* scales_plain, const int32_t* qzeros_plain,
                     int32_t* qweight, void* scales, int32_t* qzeros, int64_t N, int64_t K, int32_t group_size,
                     int32_t layout, void* stream) {
  const char* fn = "awq_import_plain";
  g_last_error.clear();
  W4_TRY(check_group_w4a16(fn, group_size));
  W4_TRY(import_common(fn, N, K, layout));
  if (N == 0) return W4_OK;
  W4_TRY(check_ptrs(fn, {{"qweight_plain", qweight_plain}, {"scales_plain", scales_plain},
                         {"qzeros_plain", qzeros_plain}, {"qweight", qweight}, {"scales", scales}, {"qzeros", qzeros}}));
  W4_TRY(check_device(fn));
  const int ng = group_size == -1 ? 1 : (int)(K / group_size);
  return launched(fn, w4::launch_import_plain(qweight_plain, scales_plain, qzeros_plain, nullptr, qweight, scales,
                                              qzeros, nullptr, (int)N, (int)K, ng, layout, 0u, 1,
                                              (hipStream_t)stream));
}

int w4a8_import_plain(const int32_t* qweight_plain, const int8_t* gscale_plain, int32_t* qweight, int8_t* gscale,
                      int64_t N, int64_t K, int32_t group_size, int32_t layout, void* stream) {
  const char* fn = "w4a8_import_plain";
  g_last_error.clear();
  if (group_size != 128 && group_size != -1)
    return fail(W4_ERR_UNSUPPORTED, "%s: group_size=%d (128 or -1)", fn, group_size);
  W4_TRY(import_common(fn, N, K, layout));
  if (N == 0) return W4_OK;
  W4_TRY(check_ptrs(fn, {{"qweight_plain", qweight_plain}, {"qweight", qweight}}));
  if (group_size == 128) {
    W4_TRY(check_ptrs(fn, {{"gscale_plain", gscale_plain}, {"gscale", gscale}}));
  } else if (gscale_plain != nullptr || gscale != nullptr) {
    return fail(W4_ERR_INVALID_ARG, "%s: gscale_plain and gscale must be NULL for group_size=-1", fn);
  }
  W4_TRY(check_device(fn));
  return launched(fn, w4::launch_import_plain(qweight_plain, nullptr, nullptr, gscale_plain, qweight, nullptr, nullptr,
                                              gscale, (int)N, (int)K, (int)(K / 128), layout, 0x88888888u, 2,
                                              (hipStream_t)stream));
}

size_t awq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group_size) {
  if (!group_ok_w4a16(group_size) || M < 0 || N < 0 || K <= 0 || K % 128 || M > kMaxDim || N > kMaxDim ||
      K > kMaxDim)
    return 0;
  if (M == 0 || N == 0) return 0;
  return awq_ws(awq_plan(M, N, K, group_size), M, N);
}

int awq_gemm(const void* x, const int32_t* qweight, const void* scales, const int32_t* qzeros, void* y,
             void* workspace, size_t workspace_bytes, int64_t M, int64_t N, int64_t K, int32_t group_size,
             void* stream) {
  const char* fn = "awq_gemm";
  g_last_error.clear();
  W4_TRY(check_group_w4a16(fn, group_size));
  W4_TRY(check_mnk(fn, M, N, K));
  if (M == 0 || N == 0) return W4_OK;
  W4_TRY(check_ptrs(fn, {{"x", x}, {"qweight", qweight}, {"scales", scales}, {"qzeros", qzeros}, {"y", y}}));
  const AwqPlan plan = awq_plan(M, N, K, group_size);
  const size_t need = awq_ws(plan, M, N);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need)
      return fail(W4_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(W4_ERR_INVALID_ARG, "%s: workspace is not 16-byte aligned", fn);
  }
  W4_TRY(check_device(fn));
  hipError_t e;
  if (plan.skinny)
    e = w4::launch_skinny(plan.sp, x, qweight, scales, qzeros, y, workspace, (int)M, (int)N, (int)K, group_size,
                          (hipStream_t)stream);
  else
    e = w4::launch_gemm(plan.gp, x, qweight, scales, qzeros, y, workspace, (int)M, (int)N, (int)K, group_size,
                        (hipStream_t)stream);
  return launched(fn, e);
}

int awq_gemm_noalloc(const void* x, const int32_t* qweight, const void* scales, const int32_t* qzeros, void* y,
                     int64_t M, int64_t N, int64_t K, int32_t group_size, void* stream) {
  static_assert(W4_NOALLOC_SCRATCH_BYTES == w4::kNoAllocScratchBytes, "scratch size");
  const char* fn = "awq_gemm_noalloc";
  g_last_error.clear();
  W4_TRY(check_group_w4a16(fn, group_size));
  W4_TRY(check_mnk(fn, M, N, K));
  if (M == 0 || N == 0) return W4_OK;
  W4_TRY(check_ptrs(fn, {{"x", x}, {"qweight", qweight}, {"scales", scales}, {"qzeros", qzeros}, {"y", y}}));
  const AwqPlan plan = awq_plan(M, N, K, group_size);
  const size_t need = awq_ws(plan, M, N);
  if (need > w4::kNoAllocScratchBytes)
    return fail(W4_ERR_WORKSPACE, "%s: this shape needs %zu bytes of workspace, above the static %zu", fn, need,
                w4::kNoAllocScratchBytes);
  W4_TRY(check_device(fn));
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = w4::noalloc_scratch(&ws, (hipStream_t)stream);
    if (e != hipSuccess) return fail(W4_ERR_HIP, "%s: static workspace: %s", fn, hipGetErrorString(e));
  }
  hipError_t e;
  if (plan.skinny)
    e = w4::launch_skinny(plan.sp, x, qweight, scales, qzeros, y, ws, (int)M, (int)N, (int)K, group_size,
                          (hipStream_t)stream);
  else
    e = w4::launch_gemm(plan.gp, x, qweight, scales, qzeros, y, ws, (int)M, (int)N, (int)K, group_size,
                        (hipStream_t)stream);
  return launched(fn, e);
}

int w4a8_pack(const void* w, int32_t* qweight, int8_t* gscale, void* cscale, int64_t M, int64_t N, int64_t K,
              int32_t group_size, void* stream) {
  const char* fn = "w4a8_pack";
  g_last_error.clear();
  if (group_size != 128 && group_size != -1)
    return fail(W4_ERR_UNSUPPORTED, "%s: group_size=%d (128 or -1)", fn, group_size);
  W4_TRY(check_mnk(fn, M, N, K));
  if (N == 0) return W4_OK;
  W4_TRY(check_ptrs(fn, {{"w", w}, {"qweight", qweight}, {"cscale", cscale}}));
  if (group_size == -1 && gscale != nullptr) return fail(W4_ERR_INVALID_ARG, "%s: gscale must be NULL for group_size=-1", fn);
  if (group_size == 128 && gscale == nullptr) return fail(W4_ERR_INVALID_ARG, "%s: gscale is NULL", fn);
  W4_TRY(check_device(fn));
  return launched(fn, w4::launch_w4a8_pack(w, qweight, gscale, cscale, (int)N, (int)K, group_size == 128 ? 1 : 0,
                                           (hipStream_t)stream));
}

int w4a8_quant_act(const void* x, const void* gamma, float eps, int8_t* xq, float* s_a, int64_t M, int64_t N,
                   int64_t K, int32_t group_size, void* stream) {
  const char* fn = "w4a8_quant_act";
  (void)group_size;
  g_last_error.clear();
  if (M < 0 || N < 0 || K < 0) return fail(W4_ERR_INVALID_ARG, "%s: negative size", fn);
  if (K == 0 || K % 8 != 0) return fail(W4_ERR_INVALID_ARG, "%s: K=%lld must be a positive multiple of 8", fn, (long long)K);
  if (M > kMaxDim || K > kMaxDim) return fail(W4_ERR_UNSUPPORTED, "%s: size above 2^30", fn);
  if (!(eps >= 0.0f)) return fail(W4_ERR_INVALID_ARG, "%s: eps must be >= 0", fn);
  if (M == 0) return W4_OK;
  W4_TRY(check_ptrs(fn, {{"x", x}, {"xq", xq}, {"s_a", s_a}}));
  if (gamma != nullptr && !aligned16(gamma)) return fail(W4_ERR_INVALID_ARG, "%s: gamma is not 16-byte aligned", fn);
  W4_TRY(check_device(fn));
  return launched(fn, w4::launch_w4a8_quant_act(x, gamma, eps, xq, s_a, (int)M, (int)K, (hipStream_t)stream));
}

int w4a8_silu_mul_quant(const void* gate_up, int8_t* xq, float* s_a, int64_t M, int64_t N, int64_t K,
                        int32_t group_size, void* stream) {
  const char* fn = "w4a8_silu_mul_quant";
  (void)group_size;
  g_last_error.clear();
  if (M < 0 || N < 0 || K < 0) return fail(W4_ERR_INVALID_ARG, "%s: negative size", fn);
  if (K == 0 || K % 8 != 0) return fail(W4_ERR_INVALID_ARG, "%s: K=%lld must be a positive multiple of 8", fn, (long long)K);
  if (M > kMaxDim || K > kMaxDim / 2) return fail(W4_ERR_UNSUPPORTED, "%s: size above the limit (M <= 2^30, K <= 2^29)", fn);
  if (M == 0) return W4_OK;
  W4_TRY(check_ptrs(fn, {{"gate_up", gate_up}, {"xq", xq}, {"s_a", s_a}}));
  W4_TRY(check_device(fn));
  return launched(fn, w4::launch_w4a8_silu_mul_quant(gate_up, xq, s_a, (int)M, (int)K, (hipStream_t)stream));
}

int w8a8_pack(const void* w, int8_t* qweight, void* cscale, int64_t M, int64_t N, int64_t K, int32_t group_size,
              void* stream) {
  const char* fn = "w8a8_pack";
  g_last_error.clear();
  if (group_size != -1) return fail(W4_ERR_UNSUPPORTED, "%s: group_size=%d (only -1, per-channel)", fn, group_size);
  W4_TRY(check_mnk(fn, M, N, K));
  if (N == 0) return W4_OK;
  W4_TRY(check_ptrs(fn, {{"w", w}, {"qweight", qweight}, {"cscale", cscale}}));
  W4_TRY(check_device(fn));
  return launched(fn, w4::launch_w8a8_pack(w, qweight, cscale, (int)N, (int)K, (hipStream_t)stream));
}

size_t w8a8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group_size) {
  if (group_size != -1 || M <= 0 || N <= 0 || K <= 0 || K % 128 || M > kMaxDim || N > kMaxDim || K > kMaxKInt8)
    return 0;
  return w4::w4a8_workspace_bytes(w4::w4a8_plan((int)M, (int)N, (int)K, 0), (int)M, (int)N);
}

static int w8a8_common(const char* fn, const int8_t* xq, const float* s_a, const int8_t* qweight,
                       const void* cscale, void* y, int32_t* acc, void* workspace, size_t workspace_bytes, int64_t M,
                       int64_t N, int64_t K, int32_t group_size, void* stream) {
  g_last_error.clear();
  if (group_size != -1) return fail(W4_ERR_UNSUPPORTED, "%s: group_size=%d (only -1, per-channel)", fn, group_size);
  W4_TRY(check_mnk(fn, M, N, K));
  W4_TRY(check_k_int8(fn, K));
  if (M == 0 || N == 0) return W4_OK;
  if (acc) {
    W4_TRY(check_ptrs(fn, {{"xq", xq}, {"qweight", qweight}, {"acc", acc}}));
  } else {
    W4_TRY(check_ptrs(fn, {{"xq", xq}, {"s_a", s_a}, {"qweight", qweight}, {"cscale", cscale}, {"y", y}}));
  }
  const w4::W4A8Plan plan = w4::w4a8_plan((int)M, (int)N, (int)K, 0);
  const size_t need = w4::w4a8_workspace_bytes(plan, (int)M, (int)N);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need)
      return fail(W4_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(W4_ERR_INVALID_ARG, "%s: workspace is not 16-byte aligned", fn);
  }
  W4_TRY(check_device(fn));
  return launched(fn, w4::launch_w8a8_gemm(plan, xq, s_a, qweight, cscale, y, acc, workspace, (int)M, (int)N,
                                           (int)K, (hipStream_t)stream));
}

int w8a8_gemm(const int8_t* xq, const float* s_a, const int8_t* qweight, const void* cscale, void* y,
              void* workspace, size_t workspace_bytes, int64_t M, int64_t N, int64_t K, int32_t group_size,
              void* stream) {
  return w8a8_common("w8a8_gemm", xq, s_a, qweight, cscale, y, nullptr, workspace, workspace_bytes, M, N, K,
                     group_size, stream);
}

int w8a8_gemm_i32(const int8_t* xq, const int8_t* qweight, int32_t* acc, void* workspace, size_t workspace_bytes,
                  int64_t M, int64_t N, int64_t K, int32_t group_size, void* stream) {
  return w8a8_common("w8a8_gemm_i32", xq, nullptr, qweight, nullptr, nullptr, acc, workspace, workspace_bytes, M, N,
                     K, group_size, stream);
}

size_t w4a8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group_size) {
  if ((group_size != 128 && group_size != -1) || M <= 0 || N <= 0 || K <= 0 || K % 128 || M > kMaxDim ||
      N > kMaxDim || K > kMaxKInt8)
    return 0;
  return w4::w4a8_workspace_bytes(w4::w4a8_plan((int)M, (int)N, (int)K, group_size), (int)M, (int)N);
}

static int w4a8_common(const char* fn, const int8_t* xq, const float* s_a, const int32_t* qweight,
                       const int8_t* gscale, const void* cscale, void* y, int32_t* acc, void* workspace,
                       size_t workspace_bytes, int64_t M, int64_t N, int64_t K, int32_t group_size, void* stream) {
  g_last_error.clear();
  if (group_size != 128 && group_size != -1)
    return fail(W4_ERR_UNSUPPORTED, "%s: group_size=%d (128 or -1)", fn, group_size);
  W4_TRY(check_mnk(fn, M, N, K));
  W4_TRY(check_k_int8(fn, K));
  if (M == 0 || N == 0) return W4_OK;
  if (acc) {
    W4_TRY(check_ptrs(fn, {{"xq", xq}, {"qweight", qweight}, {"acc", acc}}));
  } else {
    W4_TRY(check_ptrs(fn, {{"xq", xq}, {"s_a", s_a}, {"qweight", qweight}, {"cscale", cscale}, {"y", y}}));
  }
  if (group_size == 128 && gscale == nullptr) return fail(W4_ERR_INVALID_ARG, "%s: gscale is NULL", fn);
  if (group_size == -1 && gscale != nullptr) return fail(W4_ERR_INVALID_ARG, "%s: gscale must be NULL for group_size=-1", fn);
  const w4::W4A8Plan plan = w4::w4a8_plan((int)M, (int)N, (int)K, group_size);
  const size_t need = w4::w4a8_workspace_bytes(plan, (int)M, (int)N);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need)
      return fail(W4_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(W4_ERR_INVALID_ARG, "%s: workspace is not 16-byte aligned", fn);
  }
  W4_TRY(check_device(fn));
  return launched(fn, w4::launch_w4a8_gemm(plan, xq, s_a, qweight, gscale, cscale, y, acc, workspace, (int)M,
                                           (int)N, (int)K, group_size, (hipStream_t)stream));
}

int w4a8_gemm(const int8_t* xq, const float* s_a, const int32_t* qweight, const int8_t* gscale, const void* cscale,
              void* y, void* workspace, size_t workspace_bytes, int64_t M, int64_t N, int64_t K, int32_t group_size,
              void* stream) {
  return w4a8_common("w4a8_gemm", xq, s_a, qweight, gscale, cscale, y, nullptr, workspace, workspace_bytes, M, N, K,
                     group_size, stream);
}

int w4a8_gemm_i32(const int8_t* xq, const int32_t* qweight, const int8_t* gscale, int32_t* acc, void* workspace,
                  size_t workspace_bytes, int64_t M, int64_t N, int64_t K, int32_t group_size, void* stream) {
  return w4a8_common("w4a8_gemm_i32", xq, nullptr, qweight, gscale, nullptr, nullptr, acc, workspace,
                     workspace_bytes, M, N, K, group_size, stream);
}

int w4_ceiling_read(const void* buf, int64_t bytes, uint32_t* sink, int32_t blocks, int32_t unroll, void* stream) {
  const char* fn = "w4_ceiling_read";
  g_last_error.clear();
  if (bytes <= 0 || bytes % 16 != 0) return fail(W4_ERR_INVALID_ARG, "%s: bytes=%lld must be a positive multiple of 16",
                                                 fn, (long long)bytes);
  if (blocks < 1 || blocks > 65536) return fail(W4_ERR_INVALID_ARG, "%s: blocks=%d (1..65536)", fn, blocks);
  if (unroll != 4 && unroll != 8) return fail(W4_ERR_UNSUPPORTED, "%s: unroll=%d (4 or 8)", fn, unroll);
  W4_TRY(check_ptrs(fn, {{"buf", buf}, {"sink", sink}}));
  W4_TRY(check_device(fn));
  return launched(fn, w4::launch_ceiling_read(buf, bytes, sink, blocks, unroll, (hipStream_t)stream));
}

int w4_ceiling_mfma(const void* operands, int64_t operand_bytes, int32_t kind, int32_t iters, float* out,
                    int32_t blocks, void* stream) {
  const char* fn = "w4_ceiling_mfma";
  g_last_error.clear();
  if (kind != 0 && kind != 1) return fail(W4_ERR_UNSUPPORTED, "%s: kind=%d (0 fp16, 1 int8)", fn, kind);
  if (operand_bytes < 16 || operand_bytes % 16 != 0)
    return fail(W4_ERR_INVALID_ARG, "%s: operand_bytes=%lld must be a positive multiple of 16", fn,
                (long long)operand_bytes);
  if (iters < 1) return fail(W4_ERR_INVALID_ARG, "%s: iters=%d must be >= 1", fn, iters);
  if (blocks < 1 || blocks > 65536) return fail(W4_ERR_INVALID_ARG, "%s: blocks=%d (1..65536)", fn, blocks);
  W4_TRY(check_ptrs(fn, {{"operands", operands}, {"out", out}}));
  W4_TRY(check_device(fn));
  return launched(fn, w4::launch_ceiling_mfma(operands, operand_bytes, kind, iters, out, blocks, (hipStream_t)stream));
}

const char* w4_status_string(int status) {
  switch (status) {
    case W4_OK: return "W4_OK";
    case W4_ERR_INVALID_ARG: return "W4_ERR_INVALID_ARG";
    case W4_ERR_UNSUPPORTED: return "W4_ERR_UNSUPPORTED";
    case W4_ERR_WORKSPACE: return "W4_ERR_WORKSPACE";
    case W4_ERR_DEVICE: return "W4_ERR_DEVICE";
    case W4_ERR_HIP: return "W4_ERR_HIP";
    default: return "W4_ERR_UNKNOWN";
  }
}

const char* w4_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
