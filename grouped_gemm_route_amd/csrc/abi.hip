// Host side of the C ABI declared in include/moe_route.h: argument checks,
// workspace sizing and the launches.  Every check runs before any HIP call,
// so a rejected call enqueues nothing.
#include "moe_route.h"
#include "moe_internal.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_status(hipError_t err, const char* what) {
  if (err == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

int elem_size(int32_t dtype) {
  if (dtype == MOE_DTYPE_F32) return 4;
  if (dtype == MOE_DTYPE_BF16) return 2;
  return 0;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

int64_t moe_capacity(double C, int64_t N, int32_t K, int32_t E) {
  if (!(std::isfinite(C) && C > 0.0) || N < 0 || K < 1 || E < 1) return -2;
  const unsigned __int128 nk = (unsigned __int128)N * (unsigned __int128)K;
  if (nk >> 62) return -2;
  // C = m * 2^ex exactly, with m an odd integer below 2^53.
  int ex = 0;
  const double fr = std::frexp(C, &ex);
  int64_t m = (int64_t)std::ldexp(fr, 53);
  ex -= 53;
  while ((m & 1) == 0) {
    m >>= 1;
    ++ex;
  }
  unsigned __int128 num = (unsigned __int128)m * nk;  // < 2^115
  if (ex >= 0) {
    // num * 2^ex must stay far from overflow; any result above INT64_MAX fails.
    if (num != 0 && ex > 126 - 115) {
      int bits = 0;
      for (unsigned __int128 v = num; v; v >>= 1) ++bits;
      if (bits + ex > 126) return -2;
    }
    num <<= ex;
  } else {
    // ceil(num / (E * 2^s)) = ceil(ceil(num / 2^s) / E)
    const int s = -ex;
    if (s >= 120) {
      num = num != 0 ? 1 : 0;
    } else {
      const unsigned __int128 one = 1;
      num = (num + (one << s) - 1) >> s;
    }
  }
  const unsigned __int128 q = (num + (unsigned)E - 1) / (unsigned)E;
  if (q > (unsigned __int128)INT64_MAX) return -2;
  return (int64_t)q;
}

namespace {

int route_checks(const char* fn, const float* logits, int32_t N, int32_t E, int32_t K,
                 const void* a, const void* b) {
  if (!logits || !a || !b) return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (N < 0 || E < 1 || K < 1 || K > E)
    return fail(MOE_ERR_INVALID_ARG, "%s: need N >= 0 and 1 <= K <= E (N=%d E=%d K=%d)", fn,
                N, E, K);
  if (E > MOE_MAX_EXPERTS || K > MOE_MAX_TOPK)
    return fail(MOE_ERR_UNSUPPORTED, "%s: E <= %d and K <= %d supported", fn, MOE_MAX_EXPERTS,
                MOE_MAX_TOPK);
  if ((int64_t)N * E >= ((int64_t)1 << 31) * 4 || (int64_t)N * K >= ((int64_t)1 << 31))
    return fail(MOE_ERR_UNSUPPORTED, "%s: N too large", fn);
  return MOE_OK;
}

}  // namespace

int moe_route_topk(const float* logits, int32_t N, int32_t E, int32_t K,
                   int32_t renormalize, int32_t* topk_idx, float* topk_w,
                   void* stream) {
  return moe_route_topk_gated(logits, N, E, K, MOE_GATE_SOFTMAX, renormalize, topk_idx,
                              topk_w, stream);
}

int moe_route_topk_gated(const float* logits, int32_t N, int32_t E, int32_t K, int32_t gate,
                         int32_t renormalize, int32_t* topk_idx, float* topk_w, void* stream) {
  const int st = route_checks("moe_route_topk", logits, N, E, K, topk_idx, topk_w);
  if (st != MOE_OK) return st;
  if (gate != MOE_GATE_SOFTMAX && gate != MOE_GATE_SIGMOID)
    return fail(MOE_ERR_INVALID_ARG, "moe_route_topk: gate %d is not a moe_gate_t", gate);
  return hip_status(moe::launch_route_topk(logits, N, E, K, gate == MOE_GATE_SIGMOID,
                                           renormalize, topk_idx, topk_w, as_stream(stream)),
                    "moe_route_topk");
}

size_t moe_reroute_workspace_bytes(int32_t N, int32_t E, int32_t K) {
  if (N < 1 || E < 1 || K < 1) return 0;
  return moe::reroute_workspace_bytes(N, E, K);
}

int moe_reroute_overflow(const float* logits, int32_t N, int32_t E, int32_t K, int32_t gate,
                         int32_t renormalize, int64_t capacity, int32_t* topk_idx,
                         float* topk_w, int32_t* rerouted, void* workspace,
                         size_t workspace_bytes, void* stream) {
  const int st = route_checks("moe_reroute_overflow", logits, N, E, K, topk_idx, topk_w);
  if (st != MOE_OK) return st;
  if (N < 1 || capacity < -1)
    return fail(MOE_ERR_INVALID_ARG, "moe_reroute_overflow: need N >= 1 and capacity >= -1 "
                "(N=%d capacity=%lld)", N, (long long)capacity);
  if (gate != MOE_GATE_SOFTMAX && gate != MOE_GATE_SIGMOID)
    return fail(MOE_ERR_INVALID_ARG, "moe_reroute_overflow: gate %d is not a moe_gate_t", gate);
  const size_t need = moe::reroute_workspace_bytes(N, E, K);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_reroute_overflow: workspace needs %zu bytes", need);
  return hip_status(moe::launch_reroute(logits, N, E, K, gate == MOE_GATE_SIGMOID, renormalize,
                                        capacity, topk_idx, topk_w, rerouted, workspace,
                                        as_stream(stream)),
                    "moe_reroute_overflow");
}

size_t moe_dispatch_workspace_bytes(int32_t N, int32_t E, int32_t K) {
  if (N < 1 || E < 1 || K < 1) return 0;
  return moe::dispatch_workspace_bytes(N, E, K);
}

namespace {

// The per-block count table [ceil(N / tokens) + 64, E] of int32 addressed
// with 32-bit byte offsets (its scan reads up to 32 rows past a range).
bool table_fits(int32_t N, int32_t E, int tokens) {
  const int64_t B = ((int64_t)N + tokens - 1) / tokens;
  return (B + 64) * E * (int64_t)sizeof(int32_t) < ((int64_t)1 << 31);
}

// Checks shared by moe_dispatch and moe_dispatch_fp8 (es: bytes per element).
int dispatch_checks(const char* fn, const void* x, int es, int32_t N, int32_t d,
                    const int32_t* topk_idx, int32_t E, int32_t K, int32_t W, int64_t capacity,
                    const void* x_perm, const int32_t* perm_token, const int32_t* dest,
                    const int32_t* demand, const int32_t* counts, const int32_t* offsets,
                    const int32_t* rank_offsets, const void* workspace, size_t workspace_bytes) {
  if (!x || !topk_idx || !x_perm || !perm_token || !dest || !demand || !counts || !offsets ||
      !rank_offsets)
    return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (N < 1 || d < 1 || K < 1 || K > E || W < 1 || E % W != 0 || capacity < -1)
    return fail(MOE_ERR_INVALID_ARG,
                "%s: need N >= 1, d >= 1, 1 <= K <= E, W >= 1, E %% W == 0, "
                "capacity >= -1 (N=%d d=%d E=%d K=%d W=%d capacity=%lld)",
                fn, N, d, E, K, W, (long long)capacity);
  if (((int64_t)d * es) % 16 != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: row bytes d*%d must be a multiple of 16", fn, es);
  if ((int64_t)N * K >= ((int64_t)1 << 31))
    return fail(MOE_ERR_INVALID_ARG, "%s: N*K must be below 2^31", fn);
  if (E > MOE_MAX_EXPERTS || K > MOE_MAX_TOPK)
    return fail(MOE_ERR_UNSUPPORTED, "%s: E <= %d and K <= %d supported", fn, MOE_MAX_EXPERTS,
                MOE_MAX_TOPK);
  if (!table_fits(N, E, moe::kRankBlockTokens))
    return fail(MOE_ERR_UNSUPPORTED, "%s: N*E too large", fn);
  const size_t need = moe::dispatch_workspace_bytes(N, E, K);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, need);
  return MOE_OK;
}

int fp8_row_checks(const char* fn, int32_t d) {
  if (d < 1 || d % 128 != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: d must be a positive multiple of 128 (d=%d)", fn, d);
  return MOE_OK;
}

}  // namespace

int moe_dispatch(const void* x, int32_t dtype, int32_t N, int32_t d,
                 const int32_t* topk_idx, int32_t E, int32_t K, int32_t W,
                 int64_t capacity, void* x_perm, int32_t* perm_token,
                 int32_t* dest, int32_t* demand, int32_t* counts,
                 int32_t* offsets, int32_t* rank_offsets, void* workspace,
                 size_t workspace_bytes, void* stream) {
  const int es = elem_size(dtype);
  if (x && es == 0) return fail(MOE_ERR_UNSUPPORTED, "moe_dispatch: dtype %d", dtype);
  const int st = dispatch_checks("moe_dispatch", x, es ? es : 1, N, d, topk_idx, E, K, W,
                                 capacity, x_perm, perm_token, dest, demand, counts, offsets,
                                 rank_offsets, workspace, workspace_bytes);
  if (st != MOE_OK) return st;
  const moe::DispatchWorkspace ws = moe::dispatch_workspace(workspace, N, E, K);
  return hip_status(
      moe::launch_dispatch(x, (size_t)d * es, N, topk_idx, E, K, W, capacity,
                           x_perm, nullptr, perm_token, dest, demand, counts, offsets,
                           rank_offsets, ws, as_stream(stream)),
      "moe_dispatch");
}

size_t moe_route_plan_bytes(int32_t N, int32_t E, int32_t K) {
  if (N < 1 || E < 1 || K < 1) return 0;
  return moe::route_plan_bytes(N, E, K);
}

int moe_route_plan(const float* logits, int32_t N, int32_t E, int32_t K, int32_t gate,
                   int32_t renormalize, int32_t W, int64_t capacity, int32_t* topk_idx,
                   float* topk_w, int32_t* demand, int32_t* counts, int32_t* offsets,
                   int32_t* rank_offsets, void* plan, size_t plan_bytes, void* stream) {
  const char* fn = "moe_route_plan";
  const int st = route_checks(fn, logits, N, E, K, topk_idx, topk_w);
  if (st != MOE_OK) return st;
  if (!demand || !counts || !offsets || !rank_offsets)
    return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (N < 1 || W < 1 || E % W != 0 || capacity < -1)
    return fail(MOE_ERR_INVALID_ARG,
                "%s: need N >= 1, W >= 1, E %% W == 0, capacity >= -1 (N=%d E=%d W=%d "
                "capacity=%lld)", fn, N, E, W, (long long)capacity);
  if (gate != MOE_GATE_SOFTMAX && gate != MOE_GATE_SIGMOID)
    return fail(MOE_ERR_INVALID_ARG, "%s: gate %d is not a moe_gate_t", fn, gate);
  if (!table_fits(N, E, moe::route_plan_tokens(E)))
    return fail(MOE_ERR_UNSUPPORTED, "%s: N*E too large", fn);
  const size_t need = moe::route_plan_bytes(N, E, K);
  if (!plan || plan_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "%s: plan needs %zu bytes", fn, need);
  return hip_status(
      moe::launch_route_plan(logits, N, E, K, gate == MOE_GATE_SIGMOID, renormalize, W,
                             capacity, topk_idx, topk_w, demand, counts, offsets, rank_offsets,
                             moe::route_plan(plan, N, E, K), as_stream(stream)),
      fn);
}

int moe_dispatch_planned(const void* x, int32_t dtype, int32_t N, int32_t d,
                         const int32_t* topk_idx, int32_t E, int32_t K, int32_t W,
                         int64_t capacity, void* plan, size_t plan_bytes, void* x_perm,
                         float* x_scale, int32_t* perm_token, int32_t* dest, int32_t* demand,
                         int32_t* counts, int32_t* offsets, int32_t* rank_offsets,
                         void* stream) {
  const char* fn = "moe_dispatch_planned";
  const int es = elem_size(dtype);
  if (x && es == 0) return fail(MOE_ERR_UNSUPPORTED, "%s: dtype %d", fn, dtype);
  if (!x || !topk_idx || !x_perm || !perm_token || !dest || !demand || !counts || !offsets ||
      !rank_offsets)
    return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (N < 1 || d < 1 || K < 1 || K > E || W < 1 || E % W != 0 || capacity < -1)
    return fail(MOE_ERR_INVALID_ARG,
                "%s: need N >= 1, d >= 1, 1 <= K <= E, W >= 1, E %% W == 0, "
                "capacity >= -1 (N=%d d=%d E=%d K=%d W=%d capacity=%lld)",
                fn, N, d, E, K, W, (long long)capacity);
  if (((int64_t)d * es) % 16 != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: row bytes d*%d must be a multiple of 16", fn, es);
  if ((int64_t)N * K >= ((int64_t)1 << 31))
    return fail(MOE_ERR_INVALID_ARG, "%s: N*K must be below 2^31", fn);
  if (E > MOE_MAX_EXPERTS || K > MOE_MAX_TOPK)
    return fail(MOE_ERR_UNSUPPORTED, "%s: E <= %d and K <= %d supported", fn, MOE_MAX_EXPERTS,
                MOE_MAX_TOPK);
  if (!table_fits(N, E, moe::route_plan_tokens(E)))
    return fail(MOE_ERR_UNSUPPORTED, "%s: N*E too large", fn);
  if (x_scale) {
    if (dtype != MOE_DTYPE_BF16)
      return fail(MOE_ERR_INVALID_ARG, "%s: the fp8 payload needs bf16 rows", fn);
    const int st = fp8_row_checks(fn, d);
    if (st != MOE_OK) return st;
  }
  const size_t need = moe::route_plan_bytes(N, E, K);
  if (!plan || plan_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "%s: plan needs %zu bytes", fn, need);
  return hip_status(
      moe::launch_dispatch_planned(x, (size_t)d * es, N, topk_idx, E, K, W, capacity,
                                   moe::route_plan(plan, N, E, K), x_perm, x_scale, perm_token,
                                   dest, demand, counts, offsets, rank_offsets,
                                   as_stream(stream)),
      fn);
}

}  // extern "C"

namespace {

// Scratch of moe_dispatch_noalloc: a fixed array in device memory, one copy
// per GPU (each device that loads the library holds its own, until the
// process ends), zero when the library is loaded.  In host code its name is
// a host-side stand-in, never a device address: the device address comes
// from hipGetSymbolAddress, looked up once per device with that device
// current, and only that address is handed to kernels.
__device__ __align__(256) unsigned char scratch[MOE_DISPATCH_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of the current device's scratch (looked up on first use).
int scratch_address(const char* fn, void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return hip_status(err, fn);
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(MOE_ERR_UNSUPPORTED, "%s: device %d beyond the %d this call supports", fn, dev,
                kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return hip_status(err, fn);
    if (p == nullptr) return fail(MOE_ERR_HIP, "%s: no device address for the scratch", fn);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_dispatch_noalloc(const void* x, int32_t dtype, int32_t N, int32_t d,
                         const int32_t* topk_idx, int32_t E, int32_t K, int32_t W,
                         int64_t capacity, void* x_perm, int32_t* perm_token, int32_t* dest,
                         int32_t* demand, int32_t* counts, int32_t* offsets,
                         int32_t* rank_offsets, void* stream) {
  static const char* fn = "moe_dispatch_noalloc";
  const int es = elem_size(dtype);
  if (x && es == 0) return fail(MOE_ERR_UNSUPPORTED, "%s: dtype %d", fn, dtype);
  // the usual checks, with the scratch standing in for the workspace (a
  // non-null placeholder: the size is checked just below)
  const size_t need = (N >= 1 && E >= 1 && K >= 1) ? moe::dispatch_workspace_bytes(N, E, K) : 0;
  int st = dispatch_checks(fn, x, es ? es : 1, N, d, topk_idx, E, K, W, capacity, x_perm,
                           perm_token, dest, demand, counts, offsets, rank_offsets,
                           reinterpret_cast<const void*>(1), need);
  if (st != MOE_OK) return st;
  if (need > (size_t)MOE_DISPATCH_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_UNSUPPORTED,
                "%s: these sizes need %zu bytes of scratch, above the %zu this call holds "
                "(N=%d E=%d K=%d); use moe_dispatch with a workspace",
                fn, need, (size_t)MOE_DISPATCH_NOALLOC_SCRATCH_BYTES, N, E, K);
  void* ws_ptr = nullptr;
  st = scratch_address(fn, &ws_ptr);
  if (st != MOE_OK) return st;
  // Nothing in the scratch needs to start at zero: the rank kernel writes
  // every per-block count and local rank, the scan every exclusive base.
  const moe::DispatchWorkspace ws = moe::dispatch_workspace(ws_ptr, N, E, K);
  return hip_status(
      moe::launch_dispatch(x, (size_t)d * es, N, topk_idx, E, K, W, capacity, x_perm, nullptr,
                           perm_token, dest, demand, counts, offsets, rank_offsets, ws,
                           as_stream(stream)),
      fn);
}

int moe_dispatch_fp8(const void* x, int32_t N, int32_t d, const int32_t* topk_idx, int32_t E,
                     int32_t K, int32_t W, int64_t capacity, uint8_t* x8, float* x_scale,
                     int32_t* perm_token, int32_t* dest, int32_t* demand, int32_t* counts,
                     int32_t* offsets, int32_t* rank_offsets, void* workspace,
                     size_t workspace_bytes, void* stream) {
  int st = dispatch_checks("moe_dispatch_fp8", x, 2, N, d, topk_idx, E, K, W, capacity, x8,
                           perm_token, dest, demand, counts, offsets, rank_offsets, workspace,
                           workspace_bytes);
  if (st != MOE_OK) return st;
  if (!x_scale) return fail(MOE_ERR_INVALID_ARG, "moe_dispatch_fp8: null pointer");
  st = fp8_row_checks("moe_dispatch_fp8", d);
  if (st != MOE_OK) return st;
  const moe::DispatchWorkspace ws = moe::dispatch_workspace(workspace, N, E, K);
  return hip_status(
      moe::launch_dispatch(x, (size_t)d * 2, N, topk_idx, E, K, W, capacity, x8, x_scale,
                           perm_token, dest, demand, counts, offsets, rank_offsets, ws,
                           as_stream(stream)),
      "moe_dispatch_fp8");
}

int moe_combine_fp8(const uint8_t* y8, const float* y_scale, int32_t N, int32_t d, int32_t K,
                    const int32_t* dest, const float* topk_w, void* out, void* stream) {
  if (!y8 || !y_scale || !dest || !topk_w || !out)
    return fail(MOE_ERR_INVALID_ARG, "moe_combine_fp8: null pointer");
  if (N < 1 || K < 1) return fail(MOE_ERR_INVALID_ARG, "moe_combine_fp8: need N, K >= 1");
  const int st = fp8_row_checks("moe_combine_fp8", d);
  if (st != MOE_OK) return st;
  if (K > MOE_MAX_TOPK)
    return fail(MOE_ERR_UNSUPPORTED, "moe_combine_fp8: K <= %d supported", MOE_MAX_TOPK);
  return hip_status(moe::launch_combine_fp8(y8, y_scale, N, d, K, dest, topk_w, out,
                                            as_stream(stream)),
                    "moe_combine_fp8");
}

int moe_fp8_quantize_rows(const void* src, const int32_t* n_rows, int64_t max_rows, int32_t d,
                          uint8_t* q, float* scale, void* stream) {
  if (!src || !n_rows || !q || !scale)
    return fail(MOE_ERR_INVALID_ARG, "moe_fp8_quantize_rows: null pointer");
  if (max_rows < 0 || max_rows >= ((int64_t)1 << 31))
    return fail(MOE_ERR_INVALID_ARG, "moe_fp8_quantize_rows: need 0 <= max_rows < 2^31");
  const int st = fp8_row_checks("moe_fp8_quantize_rows", d);
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_fp8_quantize_rows(src, n_rows, (int)max_rows, d, q, scale,
                                                  as_stream(stream)),
                    "moe_fp8_quantize_rows");
}

int moe_fp8_dequantize_rows(const uint8_t* q, const float* scale, const int32_t* n_rows,
                            int64_t max_rows, int32_t d, void* dst, void* stream) {
  if (!q || !scale || !n_rows || !dst)
    return fail(MOE_ERR_INVALID_ARG, "moe_fp8_dequantize_rows: null pointer");
  if (max_rows < 0 || max_rows >= ((int64_t)1 << 31))
    return fail(MOE_ERR_INVALID_ARG, "moe_fp8_dequantize_rows: need 0 <= max_rows < 2^31");
  const int st = fp8_row_checks("moe_fp8_dequantize_rows", d);
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_fp8_dequantize_rows(q, scale, n_rows, (int)max_rows, d, dst,
                                                    as_stream(stream)),
                    "moe_fp8_dequantize_rows");
}

size_t moe_grouped_ffn_workspace_bytes(int64_t max_rows, int32_t E,
                                       int32_t dtype) {
  if (max_rows < 0 || E < 1 || elem_size(dtype) == 0) return 0;
  return moe::grouped_ffn_workspace_bytes(max_rows, E, dtype == MOE_DTYPE_BF16);
}

int moe_grouped_ffn(const void* x_perm, int32_t dtype, int32_t d, int32_t ffn,
                    int32_t E, const int32_t* offsets, int64_t max_rows,
                    const void* w_gate, const void* w_up, const void* w_down,
                    void* h, void* y_perm, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (!x_perm || !offsets || !w_gate || !w_up || !w_down || !h || !y_perm)
    return fail(MOE_ERR_INVALID_ARG, "moe_grouped_ffn: null pointer");
  const int es = elem_size(dtype);
  if (es == 0) return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_ffn: dtype %d", dtype);
  if (d < 1 || ffn < 1 || E < 1 || max_rows < 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_grouped_ffn: need d, ffn, E >= 1 and max_rows >= 0");
  if (E > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_ffn: E <= %d supported", MOE_MAX_EXPERTS);
  if (max_rows >= ((int64_t)1 << 31))
    return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_ffn: max_rows must be below 2^31");
  if (dtype == MOE_DTYPE_BF16 && (d % 64 != 0 || ffn % 64 != 0))
    return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_ffn: bf16 needs d and ffn multiples of 64 (d=%d ffn=%d)", d, ffn);
  if (dtype == MOE_DTYPE_F32 && (d % 8 != 0 || ffn % 8 != 0))
    return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_ffn: fp32 needs d and ffn multiples of 8 (d=%d ffn=%d)", d, ffn);
  if ((int64_t)d * ffn * es >= ((int64_t)1 << 31))
    return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_ffn: one expert's weight matrix must stay below 2 GiB (d=%d ffn=%d)", d, ffn);
  if (max_rows == 0) return MOE_OK;
  const size_t need = moe::grouped_ffn_workspace_bytes(max_rows, E, dtype == MOE_DTYPE_BF16);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_grouped_ffn: workspace needs %zu bytes", need);
  return hip_status(
      moe::launch_grouped_ffn(x_perm, dtype == MOE_DTYPE_BF16, d, ffn, E,
                              offsets, max_rows, w_gate, w_up, w_down, h,
                              y_perm, workspace, as_stream(stream)),
      "moe_grouped_ffn");
}

// Size checks shared by the packed-weight entry points: the packed matrices
// of one expert (plus the 3 panels a block's last waves may point past them)
// must stay below 2 GiB, the kernel's 32-bit per-lane offsets.
static int packed_shape_checks(const char* fn, int32_t E, int32_t d, int32_t ffn) {
  if (E < 1 || d < 1 || ffn < 1)
    return fail(MOE_ERR_INVALID_ARG, "%s: need E, d, ffn >= 1", fn);
  if (E > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_UNSUPPORTED, "%s: E <= %d supported", fn, MOE_MAX_EXPERTS);
  if (d % 64 != 0 || ffn % 64 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "%s: d and ffn must be multiples of 64 (d=%d ffn=%d)", fn,
                d, ffn);
  const int64_t up = (int64_t)(moe::packed_panels(d, ffn, true) + 3) * (d / 16) * 4096;
  const int64_t dn = (int64_t)(moe::packed_panels(d, ffn, false) + 3) * (ffn / 16) * 4096;
  if (up >= ((int64_t)1 << 31) || dn >= ((int64_t)1 << 31))
    return fail(MOE_ERR_UNSUPPORTED, "%s: one expert's packed weights must stay below 2 GiB (d=%d ffn=%d)",
                fn, d, ffn);
  return MOE_OK;
}

size_t moe_packed_ffn_weight_bytes(int32_t E, int32_t d, int32_t ffn, int32_t part) {
  if (E < 1 || d < 1 || ffn < 1 || d % 64 != 0 || ffn % 64 != 0) return 0;
  if (part != MOE_FFN_GATE_UP && part != MOE_FFN_DOWN) return 0;
  return moe::packed_ffn_weight_bytes(E, d, ffn, part == MOE_FFN_GATE_UP);
}

int moe_pack_ffn_weights(const void* w_gate, const void* w_up, const void* w_down,
                         int32_t E, int32_t d, int32_t ffn, void* packed_up,
                         void* packed_down, void* stream) {
  if (!w_gate || !w_up || !w_down || !packed_up || !packed_down)
    return fail(MOE_ERR_INVALID_ARG, "moe_pack_ffn_weights: null pointer");
  const int rc = packed_shape_checks("moe_pack_ffn_weights", E, d, ffn);
  if (rc != MOE_OK) return rc;
  return hip_status(moe::launch_pack_ffn_weights(w_gate, w_up, w_down, E, d, ffn, packed_up,
                                                 packed_down, as_stream(stream)),
                    "moe_pack_ffn_weights");
}

int moe_grouped_ffn_packed(const void* x_perm, int32_t d, int32_t ffn, int32_t E,
                           const int32_t* offsets, int64_t max_rows, const void* packed_up,
                           const void* packed_down, void* h, void* y_perm, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (!x_perm || !offsets || !packed_up || !packed_down || !h || !y_perm)
    return fail(MOE_ERR_INVALID_ARG, "moe_grouped_ffn_packed: null pointer");
  if (max_rows < 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_grouped_ffn_packed: need max_rows >= 0");
  const int rc = packed_shape_checks("moe_grouped_ffn_packed", E, d, ffn);
  if (rc != MOE_OK) return rc;
  if (max_rows >= ((int64_t)1 << 31))
    return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_ffn_packed: max_rows must be below 2^31");
  if (max_rows == 0) return MOE_OK;
  const size_t need = moe::grouped_ffn_workspace_bytes(max_rows, E, true);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_grouped_ffn_packed: workspace needs %zu bytes", need);
  return hip_status(moe::launch_grouped_ffn_packed(x_perm, d, ffn, E, offsets, max_rows,
                                                   packed_up, packed_down, h, y_perm,
                                                   workspace, as_stream(stream)),
                    "moe_grouped_ffn_packed");
}

namespace {
int combine_checks(const char* name, const void* y_perm, int32_t dtype, int32_t N, int32_t d,
                   int32_t K, const int32_t* dest, const float* topk_w, const void* out) {
  if (!y_perm || !dest || !topk_w || !out)
    return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", name);
  const int es = elem_size(dtype);
  if (es == 0) return fail(MOE_ERR_UNSUPPORTED, "%s: dtype %d", name, dtype);
  if (N < 1 || d < 1 || K < 1)
    return fail(MOE_ERR_INVALID_ARG, "%s: need N, d, K >= 1", name);
  if (((int64_t)d * es) % 16 != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: row bytes d*%d must be a multiple of 16", name, es);
  if (K > MOE_MAX_TOPK)
    return fail(MOE_ERR_UNSUPPORTED, "%s: K <= %d supported", name, MOE_MAX_TOPK);
  return MOE_OK;
}
}  // namespace

int moe_combine(const void* y_perm, int32_t dtype, int32_t N, int32_t d,
                int32_t K, const int32_t* dest, const float* topk_w, void* out,
                void* stream) {
  const int rc = combine_checks("moe_combine", y_perm, dtype, N, d, K, dest, topk_w, out);
  if (rc != MOE_OK) return rc;
  return hip_status(moe::launch_combine(y_perm, dtype == MOE_DTYPE_BF16, N, d,
                                        K, dest, topk_w, nullptr, out, as_stream(stream)),
                    "moe_combine");
}

int moe_combine_residual(const void* y_perm, int32_t dtype, int32_t N, int32_t d, int32_t K,
                         const int32_t* dest, const float* topk_w, const void* shared,
                         void* out, void* stream) {
  const int rc =
      combine_checks("moe_combine_residual", y_perm, dtype, N, d, K, dest, topk_w, out);
  if (rc != MOE_OK) return rc;
  if (!shared) return fail(MOE_ERR_INVALID_ARG, "moe_combine_residual: null pointer");
  return hip_status(moe::launch_combine(y_perm, dtype == MOE_DTYPE_BF16, N, d, K, dest,
                                        topk_w, shared, out, as_stream(stream)),
                    "moe_combine_residual");
}

int moe_router_logits(const void* x, int32_t dtype, int32_t N, int32_t d,
                      const void* w_router, int32_t E, float* logits, void* stream) {
  if (!x || !w_router || !logits)
    return fail(MOE_ERR_INVALID_ARG, "moe_router_logits: null pointer");
  const int es = elem_size(dtype);
  if (es == 0) return fail(MOE_ERR_UNSUPPORTED, "moe_router_logits: dtype %d", dtype);
  if (N < 1 || d < 1 || E < 1)
    return fail(MOE_ERR_INVALID_ARG, "moe_router_logits: need N, d, E >= 1");
  if (E > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_UNSUPPORTED, "moe_router_logits: E <= %d supported", MOE_MAX_EXPERTS);
  if (d % 8 != 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_router_logits: d must be a multiple of 8 (d=%d)", d);
  if ((int64_t)N * E >= ((int64_t)1 << 31) || (int64_t)256 * d * es >= ((int64_t)1 << 31))
    return fail(MOE_ERR_UNSUPPORTED, "moe_router_logits: sizes too large");
  return hip_status(moe::launch_router_logits(x, dtype == MOE_DTYPE_BF16, N, d, w_router, E,
                                              logits, as_stream(stream)),
                    "moe_router_logits");
}

size_t moe_exchange_workspace_bytes(int32_t E, int32_t W) {
  if (E < 1 || W < 1) return 0;
  return moe::exchange_workspace_bytes(E, W);
}

int moe_exchange_plan(const int32_t* topk_idx, const int32_t* dest,
                      const int32_t* perm_token, const int32_t* offsets, int32_t N,
                      int32_t E, int32_t K, int32_t W, int64_t max_rows,
                      int32_t* src_counts, int32_t* traffic, int32_t* send_row,
                      int32_t* send_token, int32_t* a2a_src, int32_t* regroup_src,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!topk_idx || !dest || !perm_token || !offsets || !src_counts || !traffic || !send_row ||
      !send_token || !a2a_src || !regroup_src)
    return fail(MOE_ERR_INVALID_ARG, "moe_exchange_plan: null pointer");
  if (N < 1 || K < 1 || K > E || W < 1 || E % W != 0 || max_rows < 0)
    return fail(MOE_ERR_INVALID_ARG,
                "moe_exchange_plan: need N >= 1, 1 <= K <= E, W >= 1, E %% W == 0, max_rows >= 0 "
                "(N=%d E=%d K=%d W=%d)", N, E, K, W);
  if ((int64_t)N * K >= ((int64_t)1 << 31) || max_rows >= ((int64_t)1 << 31))
    return fail(MOE_ERR_INVALID_ARG, "moe_exchange_plan: N*K and max_rows must be below 2^31");
  if (E > MOE_MAX_EXPERTS || K > MOE_MAX_TOPK || W > MOE_MAX_RANKS)
    return fail(MOE_ERR_UNSUPPORTED, "moe_exchange_plan: E <= %d, K <= %d, W <= %d supported",
                MOE_MAX_EXPERTS, MOE_MAX_TOPK, MOE_MAX_RANKS);
  const size_t need = moe::exchange_workspace_bytes(E, W);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_exchange_plan: workspace needs %zu bytes", need);
  return hip_status(moe::launch_exchange_plan(topk_idx, dest, perm_token, offsets, N, E, K, W,
                                              (int)max_rows, src_counts, traffic, send_row,
                                              send_token, a2a_src, regroup_src, workspace,
                                              as_stream(stream)),
                    "moe_exchange_plan");
}

int moe_rows_permute(const void* src, void* dst, const int32_t* map, const int32_t* n_rows,
                     int64_t max_rows, int32_t row_bytes, int32_t scatter, void* stream) {
  if (!src || !dst || !map || !n_rows)
    return fail(MOE_ERR_INVALID_ARG, "moe_rows_permute: null pointer");
  if (max_rows < 0 || row_bytes < 16 || row_bytes % 16 != 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_rows_permute: need max_rows >= 0 and row_bytes a positive multiple of 16");
  if (max_rows >= ((int64_t)1 << 31))
    return fail(MOE_ERR_INVALID_ARG, "moe_rows_permute: max_rows must be below 2^31");
  if (src == dst)
    return fail(MOE_ERR_INVALID_ARG, "moe_rows_permute: src and dst must not be the same buffer");
  return hip_status(moe::launch_rows_permute(src, dst, map, n_rows, (int)max_rows, row_bytes,
                                             scatter != 0, as_stream(stream)),
                    "moe_rows_permute");
}

}  // extern "C"
