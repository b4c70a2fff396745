// abi.cpp -- the extern "C" entry points declared in include/lin_gemm.h.
//
// lin_gemm_run plays the part of the custom-op wrapper in the
// TorchInductor-integration section of "Совместная работа Helion и
// TorchInductor: слияние операторов" (check the inner dimension, pick the
// launch shape, launch one kernel), with the per-shape variant choice of
// "helion-vllm-linear-backend" (sections "Одно ядро вместо трёх вариантов"
// and "Гибридный диспатч").  Argument checks happen here, on the host, before
// anything is enqueued; kernels never see a shape they were not built for.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <mutex>
#include <sstream>
#include <string>
#include <vector>

#include "../../include/lin_gemm.h"
#include "dispatch.hpp"
#include "launch.hpp"

struct lin_gemm_ctx {
  std::vector<lg::TableEntry> table;
  bool forced = false;
  lg::Variant force;
  std::string last_error;
  void* ws = nullptr;         // split-K workspace
  size_t ws_bytes = 0;
  int* counters = nullptr;    // per-16-row-group arrival counters (kept at zero between calls)
  size_t counters_n = 0;
  void* dq = nullptr;         // staging of lin_gemm_run_dynamic: codes, then scales
  size_t dq_bytes = 0;
  // Buffers replaced by bigger ones.  They stay allocated until the handle
  // is destroyed: a graph captured before the growth still holds their
  // addresses and may be replayed.
  std::vector<void*> retired;
};

namespace {

int fail(lin_gemm_t h, int status, const std::string& msg) {
  if (h) h->last_error = msg;
  return status;
}

int hip_fail(lin_gemm_t h, hipError_t e, const char* what) {
  return fail(h, LIN_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Sizes of handle-owned buffers grow in powers of two (at least 1 MiB), so
// the retired ones add up to less than the live one.
size_t grow_size(size_t need) {
  size_t b = (size_t)1 << 20;
  while (b < need) b <<= 1;
  return b;
}

// Bytes per element of A (bf16 activations in the MXFP4 mode).
int esize(int quant) {
  return (quant == LIN_Q_BF16 || quant == LIN_Q_FP16 || quant == LIN_Q_MXFP4) ? 2 : 1;
}

int qkind(int quant) {
  switch (quant) {
    case LIN_Q_BF16: return lg::QK_BF16;
    case LIN_Q_FP16: return lg::QK_FP16;
    case LIN_Q_FP8_DYNAMIC: return lg::QK_FP8;
    case LIN_Q_W8A8_INT8: return lg::QK_I8;
    case LIN_Q_BLOCK_FP8: return lg::QK_FP8_BLOCK;
    case LIN_Q_MXFP4: return lg::QK_MXFP4;
  }
  return -1;
}

// Bytes of one row of B (the weight): K elements, or K/2 for 4-bit codes.
int64_t b_row_bytes(int quant, int64_t K) {
  return quant == LIN_Q_MXFP4 ? K / 2 : K * esize(quant);
}

bool misaligned(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15) != 0; }

// Shape / pointer checks shared by the fused and unfused entry points.
int check_shape(lin_gemm_t h, int quant, int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0) return fail(h, LIN_ERR_INVALID_ARG, "negative size");
  if (quant < LIN_Q_BF16 || quant > LIN_Q_MXFP4)
    return fail(h, LIN_ERR_INVALID_ARG, "unknown quant mode " + std::to_string(quant));
  if (M == 0) return LIN_OK;
  if (N < 1 || K < 1) return fail(h, LIN_ERR_UNSUPPORTED, "N and K must be >= 1");
  if ((K * esize(quant)) % 16 != 0)
    return fail(h, LIN_ERR_UNSUPPORTED, "rows of A and B must be a multiple of 16 bytes "
                                        "(K % 8 for bf16/fp16, K % 16 for e4m3/int8)");
  if (quant == LIN_Q_BLOCK_FP8 && (K % 128 != 0 || N % 128 != 0))
    return fail(h, LIN_ERR_UNSUPPORTED, "block FP8 needs K % 128 == 0 and N % 128 == 0");
  if (quant == LIN_Q_MXFP4 && K % 256 != 0)
    return fail(h, LIN_ERR_UNSUPPORTED, "MXFP4 weights need K % 256 == 0");
  if (quant == LIN_Q_W8A8_INT8 && K > 131071)
    return fail(h, LIN_ERR_UNSUPPORTED, "int8 needs K <= 131071 (int32 accumulator range)");
  if (M > (int64_t)1 << 31 || N > (int64_t)1 << 31 || K > (int64_t)1 << 31)
    return fail(h, LIN_ERR_UNSUPPORTED, "sizes beyond 2^31");
  // Tile kernels address a 256-row operand panel with 32-bit buffer offsets.
  if (K * esize(quant) > ((int64_t)1 << 31) / 256 - 256)
    return fail(h, LIN_ERR_UNSUPPORTED, "operand rows longer than 8 MiB");
  return LIN_OK;
}

int select_variant(lin_gemm_t h, int quant, int64_t M, int64_t N, int64_t K, lg::Variant* v) {
  if (h->forced) {
    *v = h->force;
  } else if (!lg::lookup(h->table, quant, M, N, K, v)) {
    // No entry: the built-in rule.
    lg::Variant d;
    if (M <= 32) { d.kind = lg::V_DECODE; }
    else { d.kind = lg::V_TILE; d.bm = 128; d.bn = 128; d.wm = 2; d.wn = 2; }
    *v = d;
  }
  if (quant == LIN_Q_MXFP4 && M <= 32 && !lg::decode_mx_supported(*v)) {
    if (h->forced) return fail(h, LIN_ERR_UNSUPPORTED, "variant not compiled for MXFP4 weights");
    *v = lg::Variant();
    v->kind = lg::V_DECODE;
    v->waves = 8; v->unroll = 2; v->rows = 16; v->split = 1;
  }
  if (v->kind == lg::V_DECODE && M > 32) {
    if (h->forced) return fail(h, LIN_ERR_UNSUPPORTED, "decode variants need M <= 32");
    v->kind = lg::V_TILE; v->bm = 128; v->bn = 128; v->wm = 2; v->wn = 2;
  }
  // The ping-pong family covers bf16 / fp16 / int8 and block FP8; split-K
  // only for block FP8.
  if (v->kind == lg::V_PP) {
    const bool ok = lg::pp_supported(qkind(quant)) &&
                    (quant == LIN_Q_BLOCK_FP8 || v->split <= 1);
    if (!ok) {
      if (h->forced)
        return fail(h, LIN_ERR_UNSUPPORTED,
                    "pp variants cover bf16, fp16, int8 and block FP8 (split-K for block FP8 only)");
      v->kind = lg::V_TILE; v->bm = 128; v->bn = 128; v->wm = 2; v->wn = 2;
    }
  }
  // 4-bit weights take the tile shapes whose weight loads split evenly (32
  // rows of 32 bytes per load instruction).
  if (v->kind == lg::V_TILE && !lg::tile_supported(qkind(quant), v->bm, v->bn, v->wm, v->wn)) {
    if (h->forced) return fail(h, LIN_ERR_UNSUPPORTED, "tile shape not compiled for this mode");
    v->bm = 128; v->bn = 128; v->wm = 2; v->wn = 2;
  }
  if (v->kind == lg::V_TILE && v->sk > 0 &&
      !lg::tile_sk_supported(qkind(quant), v->bm, v->bn, v->wm, v->wn)) {
    if (h->forced) return fail(h, LIN_ERR_UNSUPPORTED, "tile shape not compiled in stream-K form");
    v->sk = 0;
  }
  // Block scales are uniform over a decode workgroup's rows only when the
  // rows sit inside one 128-row scale block.
  if (v->kind == lg::V_DECODE && quant == LIN_Q_BLOCK_FP8 && 128 % v->rows != 0) {
    if (h->forced)
      return fail(h, LIN_ERR_UNSUPPORTED, "block FP8 decode needs rows dividing 128");
    v->rows = 16;
  }
  return LIN_OK;
}

int resolve_split(const lg::Variant& v, const lg::Call& c) {
  if (v.kind == lg::V_PP) {
    int split = v.split > 0 ? v.split : lg::pp_auto_split(c);
    const int64_t blocks = c.KB / 128;
    while (split > 1 && split > blocks) split >>= 1;  // at least one scale block per slice
    return c.qk == lg::QK_FP8_BLOCK ? split : 1;
  }
  if (v.kind == lg::V_TILE) {
    if (v.sk > 0) return 1;
    int split = v.split > 0 ? v.split : lg::tile_auto_split(v, c);
    return std::min(split, 16);
  }
  if (v.kind != lg::V_DECODE) return 1;
  int split = v.split > 0 ? v.split : lg::decode_auto_split(c, v);
  const int64_t steps = (c.KB + 127) / 128;
  while (split > 1 && split > steps) split >>= 1;  // at least one 128-byte step per slice
  return split;
}

// Make sure the workspace and counters cover this call.
int ensure_workspace(lin_gemm_t h, const lg::Variant& v, const lg::Call& c, int split,
                     hipStream_t s) {
  const bool pp = v.kind == lg::V_PP;
  const bool dec = v.kind == lg::V_DECODE;
  const size_t need = pp ? lg::pp_ws_bytes(c, split)
                         : (dec ? lg::decode_ws_bytes(v, c, split) : lg::tile_ws_bytes(v, c, split));
  const size_t ncnt = (size_t)((c.N + v.rows - 1) / v.rows);  // one per row group
  const bool grow_ws = need > h->ws_bytes;
  const bool grow_cnt = dec && split > 1 && ncnt > h->counters_n;
  if (grow_ws || grow_cnt) {
    hipError_t e = hipStreamSynchronize(s);  // in-flight calls may still use the old buffers
    if (e != hipSuccess) return hip_fail(h, e, "hipStreamSynchronize");
  }
  if (grow_ws) {
    if (h->ws) h->retired.push_back(h->ws);
    h->ws = nullptr;
    h->ws_bytes = 0;
    size_t bytes = grow_size(need);
    if (hipMalloc(&h->ws, bytes) != hipSuccess) {
      h->ws = nullptr;
      return fail(h, LIN_ERR_OOM, "split-K workspace allocation of " + std::to_string(bytes) + " bytes failed");
    }
    h->ws_bytes = bytes;
  }
  if (grow_cnt) {
    if (h->counters) h->retired.push_back(h->counters);
    h->counters = nullptr;
    h->counters_n = 0;
    size_t n = grow_size(ncnt * sizeof(int)) / sizeof(int);
    if (hipMalloc(&h->counters, n * sizeof(int)) != hipSuccess) {
      h->counters = nullptr;
      return fail(h, LIN_ERR_OOM, "split-K counter allocation failed");
    }
    h->counters_n = n;
    hipError_t e = lg::launch_fill_zero(h->counters, n * sizeof(int), s);
    if (e != hipSuccess) return hip_fail(h, e, "counter zero fill");
  }
  if (split > 1 && dec && v.reduce == lg::R_ATOMIC) {
    // The atomic reduction needs a zero accumulator.  Its last arrival
    // re-zeroes what it used, but other split-K forms (and other shapes)
    // leave partials in the same workspace, and a graph captured now must
    // not depend on what eager calls do between its replays: the fill is
    // enqueued with every atomic call.
    hipError_t e = lg::launch_fill_zero(h->ws, need, s);
    if (e != hipSuccess) return hip_fail(h, e, "workspace zero fill");
  }
  return LIN_OK;
}

lg::Epi make_epi(const lin_scales_t* scales, const void* bias, const void* residual, void* C,
                 int64_t M, int64_t N, int quant, int act) {
  lg::Epi e;
  e.sa = scales ? scales->a : nullptr;
  e.sb = scales ? scales->b : nullptr;
  e.bias = (const uint16_t*)bias;
  e.residual = (const uint16_t*)residual;
  e.C = C;
  e.alpha = scales ? scales->alpha : 1.0f;
  e.raw = act == LIN_ACT_RAW_ACC;
  e.act = e.raw ? 0 : act;
  e.scale_mode = (quant == LIN_Q_FP8_DYNAMIC || quant == LIN_Q_W8A8_INT8) && !e.raw ? 1 : 0;
  e.M = M;
  e.N = N;
  return e;
}

// ------------------------------------------------ static scratch (no-alloc)
//
// lin_gemm_run_noalloc keeps its split-K partials and arrival counters in
// this array instead of handle buffers, for callers that cannot allocate.
// Each device that loads the library holds its own copy until the process
// ends.  In host code `scratch` only names the symbol: its device address
// comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address is handed to kernels and fill launches.
constexpr size_t kScratchCounterBytes = (size_t)256 << 10;  // arrival counters
constexpr size_t kScratchWsBytes = (size_t)64 << 20;        // split-K partials
static __device__ __align__(256) unsigned char scratch[kScratchCounterBytes + kScratchWsBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_base(lin_gemm_t h, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(h, e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(h, LIN_ERR_UNSUPPORTED, "device index beyond " + std::to_string(kMaxDevices));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(h, e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(h, LIN_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LIN_OK;
}

// Point c.ws / c.counters into the device's scratch array and clear what
// the kernels expect to find at zero: the arrival counters of a cross-
// workgroup decode split (kept at zero by each finishing call, cleared
// again here because the array is shared by every call and handle on the
// device) and the accumulator of the atomic reduction.  The other split-K
// forms overwrite their slices.  Clearing uses a fill kernel, so a caller
// may capture the call into a graph.
int scratch_workspace(lin_gemm_t h, const lg::Variant& v, lg::Call& c, int split,
                      hipStream_t s) {
  const bool pp = v.kind == lg::V_PP;
  const bool dec = v.kind == lg::V_DECODE;
  const size_t need = pp ? lg::pp_ws_bytes(c, split)
                         : (dec ? lg::decode_ws_bytes(v, c, split) : lg::tile_ws_bytes(v, c, split));
  const size_t ncnt = dec && split > 1 ? (size_t)((c.N + v.rows - 1) / v.rows) : 0;
  if (need > kScratchWsBytes || ncnt * sizeof(int) > kScratchCounterBytes)
    return fail(h, LIN_ERR_UNSUPPORTED,
                "lin_gemm_run_noalloc: this call's split-K partials need " +
                    std::to_string(need) + " bytes and " + std::to_string(ncnt) +
                    " counters; the static scratch holds " + std::to_string(kScratchWsBytes) +
                    " bytes and " + std::to_string(kScratchCounterBytes / sizeof(int)) +
                    " counters");
  void* base = nullptr;
  if (need > 0 || ncnt > 0) {
    int rc = scratch_base(h, &base);
    if (rc != LIN_OK) return rc;
  }
  c.counters = base ? (int*)base : nullptr;
  c.ws = base ? (void*)((char*)base + kScratchCounterBytes) : nullptr;
  if (ncnt > 0) {
    hipError_t e = lg::launch_fill_zero(c.counters, ncnt * sizeof(int), s);
    if (e != hipSuccess) return hip_fail(h, e, "scratch counter clear");
  }
  if (dec && split > 1 && v.reduce == lg::R_ATOMIC) {
    hipError_t e = lg::launch_fill_zero(c.ws, need, s);
    if (e != hipSuccess) return hip_fail(h, e, "scratch accumulator clear");
  }
  return LIN_OK;
}

// lin_gemm_run and lin_gemm_run_noalloc: the same checks, variant choice
// and kernels.  noalloc == false: split-K partials and arrival counters live
// in handle-owned buffers (grown on demand).  noalloc == true: they live in
// the device's static scratch array; a call that needs more than it holds
// is rejected before anything is enqueued.
int run_impl(lin_gemm_t h, const void* A, const void* B, const lin_scales_t* scales,
             const void* bias, const void* residual, void* C, int64_t M, int64_t N, int64_t K,
             int quant_mode, int activation, void* stream, bool noalloc) {
  if (!h) return LIN_ERR_INVALID_ARG;
  h->last_error.clear();
  int rc = check_shape(h, quant_mode, M, N, K);
  if (rc != LIN_OK || M == 0) return rc;
  if (!A || !B || !C) return fail(h, LIN_ERR_INVALID_ARG, "A, B and C must be non-null");
  if (!(activation >= LIN_ACT_NONE && activation <= LIN_ACT_SILU) && activation != LIN_ACT_RAW_ACC)
    return fail(h, LIN_ERR_INVALID_ARG, "unknown activation " + std::to_string(activation));
  const bool quantised = quant_mode >= LIN_Q_FP8_DYNAMIC && quant_mode != LIN_Q_MXFP4;
  if (quantised && (!scales || !scales->a || !scales->b))
    return fail(h, LIN_ERR_INVALID_ARG, "quantised modes need scales->a and scales->b");
  if (quant_mode == LIN_Q_MXFP4 && (!scales || !scales->b))
    return fail(h, LIN_ERR_INVALID_ARG, "MXFP4 weights need scales->b (E8M0 bytes)");
  if (misaligned(A) || misaligned(B) || misaligned(C) || misaligned(bias) || misaligned(residual))
    return fail(h, LIN_ERR_UNSUPPORTED, "A, B, C, bias and residual must be 16-byte aligned");
  if (scales && (misaligned(scales->a) || misaligned(scales->b)))
    return fail(h, LIN_ERR_UNSUPPORTED, "scale arrays must be 16-byte aligned");

  hipStream_t s = (hipStream_t)stream;
  lg::Call c{};
  c.A = A; c.B = B; c.M = M; c.N = N; c.K = K;
  c.KB = b_row_bytes(quant_mode, K);
  c.qk = qkind(quant_mode);
  c.epi = make_epi(scales, bias, residual, C, M, N, quant_mode, activation);

  lg::Variant v;
  rc = select_variant(h, quant_mode, M, N, K, &v);
  if (rc != LIN_OK) return rc;
  if (v.kind == lg::V_DECODE && !lg::decode_plain_supported(v.swap, v.waves, v.unroll, v.rows) &&
      !(v.xs == 2 && lg::decode_wd_supported(v, c, resolve_split(v, c))) &&
      !(v.xs && lg::decode_xs_supported(v, c)))
    return fail(h, LIN_ERR_UNSUPPORTED,
                "decode shape compiled only with staged activations, which do not apply to this call");
  hipError_t e;
  const int split = resolve_split(v, c);
  if (noalloc) {
    rc = scratch_workspace(h, v, c, split, s);
  } else {
    rc = ensure_workspace(h, v, c, split, s);
    c.ws = h->ws;
    c.counters = h->counters;
  }
  if (rc != LIN_OK) return rc;
  if (v.kind == lg::V_TILE) {
    e = lg::launch_tile(v, c, split, s);
  } else if (v.kind == lg::V_PP) {
    e = lg::launch_pp(v, c, split, s);
  } else {
    if (v.xs == 2 && lg::decode_wd_supported(v, c, split)) e = lg::launch_decode_wd(v, c, split, s);
    else if (v.xs && lg::decode_xs_supported(v, c)) e = lg::launch_decode_xs(v, c, split, s);
    else e = lg::launch_decode(v, c, split, s);
  }
  if (e != hipSuccess) return hip_fail(h, e, "kernel launch");
  if (std::getenv("LIN_GEMM_LOG")) {
    lg::Call cc = c;
    std::fprintf(stderr, "lin_gemm: quant=%d M=%lld N=%lld K=%lld -> %s\n", quant_mode,
                 (long long)M, (long long)N, (long long)K,
                 lg::format_variant(v, resolve_split(v, cc)).c_str());
  }
  return LIN_OK;
}


}  // namespace

extern "C" {

int lin_gemm_create(lin_gemm_t* out, const char* config_path) {
  if (!out) return LIN_ERR_INVALID_ARG;
  *out = nullptr;
  lin_gemm_ctx* h = new (std::nothrow) lin_gemm_ctx();
  if (!h) return LIN_ERR_OOM;
  std::string text = lg::builtin_table();
  const char* path = config_path;
  if (!path) path = std::getenv("LIN_GEMM_CONFIG");
  if (path && *path) {
    std::ifstream f(path);
    if (!f) { delete h; return LIN_ERR_CONFIG; }
    std::stringstream ss;
    ss << f.rdbuf();
    text = ss.str();
  }
  std::string err;
  if (!lg::parse_table(text, &h->table, &err)) {
    std::fprintf(stderr, "lin_gemm: variant table: %s\n", err.c_str());
    delete h;
    return LIN_ERR_CONFIG;
  }
  *out = h;
  return LIN_OK;
}

int lin_gemm_destroy(lin_gemm_t h) {
  if (!h) return LIN_OK;
  if (h->ws) hipFree(h->ws);
  if (h->counters) hipFree(h->counters);
  if (h->dq) hipFree(h->dq);
  for (void* p : h->retired) hipFree(p);
  delete h;
  return LIN_OK;
}

const char* lin_gemm_strerror(int status) {
  switch (status) {
    case LIN_OK: return "ok";
    case LIN_ERR_INVALID_ARG: return "invalid argument";
    case LIN_ERR_UNSUPPORTED: return "unsupported shape or mode";
    case LIN_ERR_HIP: return "HIP runtime error";
    case LIN_ERR_OOM: return "out of device memory";
    case LIN_ERR_CONFIG: return "bad variant table or spec";
  }
  return "unknown status";
}

const char* lin_gemm_last_error(lin_gemm_t h) { return h ? h->last_error.c_str() : ""; }

int lin_gemm_set_force(lin_gemm_t h, const char* spec) {
  if (!h) return LIN_ERR_INVALID_ARG;
  if (!spec || !*spec) { h->forced = false; return LIN_OK; }
  lg::Variant v;
  std::string err;
  if (!lg::parse_variant(spec, &v, &err)) return fail(h, LIN_ERR_CONFIG, err);
  h->force = v;
  h->forced = true;
  return LIN_OK;
}

int lin_gemm_describe(lin_gemm_t h, int quant_mode, int64_t M, int64_t N, int64_t K, char* buf,
                      int buflen) {
  if (!h || !buf || buflen < 1) return LIN_ERR_INVALID_ARG;
  int rc = check_shape(h, quant_mode, M, N, K);
  if (rc != LIN_OK) return rc;
  lg::Variant v;
  rc = select_variant(h, quant_mode, M, N, K, &v);
  if (rc != LIN_OK) return rc;
  lg::Call c{};
  c.M = M; c.N = N; c.K = K; c.KB = b_row_bytes(quant_mode, K);
  c.qk = qkind(quant_mode);
  // Report staged / widened activations only where lin_gemm_run would use
  // them (the widened form falls back to staging, then to neither).
  const int split = resolve_split(v, c);
  if (v.xs == 2 && !lg::decode_wd_supported(v, c, split)) v.xs = 1;
  if (v.xs == 1 && !lg::decode_xs_supported(v, c)) v.xs = 0;
  std::string s = lg::format_variant(v, split);
  std::snprintf(buf, (size_t)buflen, "%s", s.c_str());
  return LIN_OK;
}

int lin_gemm_run(lin_gemm_t h, const void* A, const void* B, const lin_scales_t* scales,
                 const void* bias, const void* residual, void* C, int64_t M, int64_t N, int64_t K,
                 int quant_mode, int activation, void* stream) {
  return run_impl(h, A, B, scales, bias, residual, C, M, N, K, quant_mode, activation, stream,
                  false);
}

int lin_gemm_run_noalloc(lin_gemm_t h, const void* A, const void* B, const lin_scales_t* scales,
                         const void* bias, const void* residual, void* C, int64_t M, int64_t N,
                         int64_t K, int quant_mode, int activation, void* stream) {
  return run_impl(h, A, B, scales, bias, residual, C, M, N, K, quant_mode, activation, stream,
                  true);
}

int lin_gemm_run_unfused(lin_gemm_t h, const void* A, const void* B, const void* bias,
                         const void* residual, void* C, void* T, void* U, int64_t M, int64_t N,
                         int64_t K, float alpha, int quant_mode, int activation, void* stream) {
  if (!h) return LIN_ERR_INVALID_ARG;
  h->last_error.clear();
  if (quant_mode != LIN_Q_BF16 && quant_mode != LIN_Q_FP16)
    return fail(h, LIN_ERR_UNSUPPORTED, "the unfused path is bf16 / fp16 only");
  int rc = check_shape(h, quant_mode, M, N, K);
  if (rc != LIN_OK || M == 0) return rc;
  if (!A || !B || !C || !T || !U) return fail(h, LIN_ERR_INVALID_ARG, "null pointer");
  if (activation < LIN_ACT_NONE || activation > LIN_ACT_SILU)
    return fail(h, LIN_ERR_INVALID_ARG, "unknown activation " + std::to_string(activation));
  if (misaligned(A) || misaligned(B) || misaligned(C) || misaligned(T) || misaligned(U) ||
      misaligned(bias) || misaligned(residual))
    return fail(h, LIN_ERR_UNSUPPORTED, "buffers must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  const bool f16 = quant_mode == LIN_Q_FP16;
  lg::Call c{};
  c.A = A; c.B = B; c.M = M; c.N = N; c.K = K;
  c.KB = K * 2;
  c.qk = qkind(quant_mode);
  c.epi = make_epi(nullptr, nullptr, nullptr, T, M, N, quant_mode, LIN_ACT_NONE);
  lg::Variant v;
  rc = select_variant(h, quant_mode, M, N, K, &v);
  if (rc != LIN_OK) return rc;
  hipError_t e;
  if (v.kind == lg::V_PP) {
    e = lg::launch_pp(v, c, 1, s);
  } else {
    if (v.kind != lg::V_TILE) { v = lg::Variant(); v.kind = lg::V_TILE; }
    e = lg::launch_tile(v, c, 1, s);
  }
  if (e != hipSuccess) return hip_fail(h, e, "GEMM launch");
  e = lg::launch_bias_act(T, bias, U, M, N, activation, f16, s);
  if (e != hipSuccess) return hip_fail(h, e, "bias+activation launch");
  e = lg::launch_scale_residual(U, residual, C, M, N, alpha, f16, s);
  if (e != hipSuccess) return hip_fail(h, e, "scale+residual launch");
  return LIN_OK;
}

int lin_gemm_stream_read(lin_gemm_t h, const void* src, int64_t bytes, int grid, int unroll,
                         int* sink, void* stream) {
  if (!h) return LIN_ERR_INVALID_ARG;
  h->last_error.clear();
  if (bytes < 0) return fail(h, LIN_ERR_INVALID_ARG, "negative size");
  if (bytes == 0) return LIN_OK;
  if (!src || !sink) return fail(h, LIN_ERR_INVALID_ARG, "src and sink must be non-null");
  if (bytes % 16 != 0 || misaligned(src) || (reinterpret_cast<uintptr_t>(sink) & 3))
    return fail(h, LIN_ERR_UNSUPPORTED, "bytes % 16 == 0, src 16-byte and sink 4-byte aligned");
  if (grid == 0) grid = 1024;
  if (grid < 1 || grid > (1 << 20))
    return fail(h, LIN_ERR_INVALID_ARG, "grid must be in 1 .. 2^20 (0 = 1024)");
  if (unroll != 4 && unroll != 8 && unroll != 16)
    return fail(h, LIN_ERR_INVALID_ARG, "unroll must be 4, 8 or 16");
  hipError_t e = lg::launch_stream_read(src, bytes, grid, unroll, sink, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(h, e, "stream read launch");
  return LIN_OK;
}

int lin_gemm_quantize(lin_gemm_t h, const void* X, int x_dtype, int64_t M, int64_t K, int kind,
                      void* Q, float* scales, void* stream) {
  if (!h) return LIN_ERR_INVALID_ARG;
  h->last_error.clear();
  if (M < 0 || K < 0) return fail(h, LIN_ERR_INVALID_ARG, "negative size");
  if (x_dtype != LIN_Q_BF16 && x_dtype != LIN_Q_FP16)
    return fail(h, LIN_ERR_INVALID_ARG, "x_dtype must be LIN_Q_BF16 or LIN_Q_FP16");
  if (kind < LIN_DQ_FP8_TOKEN || kind > LIN_DQ_FP8_BLOCK)
    return fail(h, LIN_ERR_INVALID_ARG, "unknown quantization kind " + std::to_string(kind));
  if (M == 0) return LIN_OK;
  if (!X || !Q || !scales) return fail(h, LIN_ERR_INVALID_ARG, "X, Q and scales must be non-null");
  if (K < 16 || K % 16 != 0)
    return fail(h, LIN_ERR_UNSUPPORTED, "K must be a positive multiple of 16");
  if (kind == LIN_DQ_FP8_BLOCK && K % 128 != 0)
    return fail(h, LIN_ERR_UNSUPPORTED, "1x128 blocks need K % 128 == 0");
  if (M >= ((int64_t)1 << 31) || K > ((int64_t)1 << 31) || M * K >= ((int64_t)1 << 40))
    return fail(h, LIN_ERR_UNSUPPORTED, "sizes beyond 2^31 rows / 2^40 values");
  if (misaligned(X) || misaligned(Q) || misaligned(scales))
    return fail(h, LIN_ERR_UNSUPPORTED, "X, Q and scales must be 16-byte aligned");
  hipError_t e = lg::launch_dynamic_quant(kind, x_dtype == LIN_Q_FP16, X, M, K, Q, scales,
                                          (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(h, e, "quantization launch");
  return LIN_OK;
}

int lin_gemm_run_dynamic(lin_gemm_t h, const void* X, int x_dtype, const void* B,
                         const float* sb, float alpha, const void* bias, const void* residual,
                         void* C, int64_t M, int64_t N, int64_t K, int quant_mode, int activation,
                         void* stream) {
  if (!h) return LIN_ERR_INVALID_ARG;
  h->last_error.clear();
  int kind;
  switch (quant_mode) {
    case LIN_Q_FP8_DYNAMIC: kind = LIN_DQ_FP8_TOKEN; break;
    case LIN_Q_W8A8_INT8: kind = LIN_DQ_INT8_TOKEN; break;
    case LIN_Q_BLOCK_FP8: kind = LIN_DQ_FP8_BLOCK; break;
    default:
      return fail(h, LIN_ERR_INVALID_ARG, "run_dynamic needs a quantised mode (2, 3 or 4)");
  }
  int rc = check_shape(h, quant_mode, M, N, K);
  if (rc != LIN_OK || M == 0) return rc;
  if (!X || !B || !C || !sb) return fail(h, LIN_ERR_INVALID_ARG, "X, B, sb and C must be non-null");
  hipStream_t s = (hipStream_t)stream;
  // Decode shapes: quantize in the kernel's prologue when the chosen variant
  // has one (bf16 activations).
  if (x_dtype == LIN_Q_BF16 && M <= 16) {
    if (activation < LIN_ACT_NONE || (activation > LIN_ACT_SILU && activation != LIN_ACT_RAW_ACC))
      return fail(h, LIN_ERR_INVALID_ARG, "unknown activation " + std::to_string(activation));
    if (misaligned(X) || misaligned(B) || misaligned(C) || misaligned(bias) ||
        misaligned(residual) || misaligned(sb))
      return fail(h, LIN_ERR_UNSUPPORTED, "X, B, C, sb, bias and residual must be 16-byte aligned");
    lg::Variant v;
    rc = select_variant(h, quant_mode, M, N, K, &v);
    if (rc != LIN_OK) return rc;
    lg::Call c{};
    c.A = X; c.B = B; c.M = M; c.N = N; c.K = K;
    c.KB = K;
    c.qk = qkind(quant_mode);
    lin_scales_t sc{nullptr, sb, alpha};
    c.epi = make_epi(&sc, bias, residual, C, M, N, quant_mode, activation);
    const int split = resolve_split(v, c);
    if (v.dq && lg::decode_dq_supported(v, c, split)) {
      hipError_t e = lg::launch_decode_dq(v, c, s);
      if (e != hipSuccess) return hip_fail(h, e, "kernel launch");
      if (std::getenv("LIN_GEMM_LOG"))
        std::fprintf(stderr, "lin_gemm: dynamic quant=%d M=%lld N=%lld K=%lld -> %s (prologue)\n",
                     quant_mode, (long long)M, (long long)N, (long long)K,
                     lg::format_variant(v, split).c_str());
      return LIN_OK;
    }
  }
  // Otherwise: the quantization kernel into staging, then the layer.
  // Staging: the codes [M][K], then the scales (256-byte aligned).
  const size_t qbytes = ((size_t)M * (size_t)K + 255) & ~(size_t)255;
  const size_t nscale = kind == LIN_DQ_FP8_BLOCK ? (size_t)M * (size_t)(K / 128) : (size_t)M;
  const size_t need = qbytes + nscale * sizeof(float);
  if (need > h->dq_bytes) {
    hipError_t e = hipStreamSynchronize(s);  // in-flight calls may still read the old staging
    if (e != hipSuccess) return hip_fail(h, e, "hipStreamSynchronize");
    if (h->dq) h->retired.push_back(h->dq);
    h->dq = nullptr;
    h->dq_bytes = 0;
    const size_t bytes = grow_size(need);
    if (hipMalloc(&h->dq, bytes) != hipSuccess) {
      h->dq = nullptr;
      return fail(h, LIN_ERR_OOM, "staging allocation of " + std::to_string(bytes) + " bytes failed");
    }
    h->dq_bytes = bytes;
  }
  float* sa = (float*)((char*)h->dq + qbytes);
  rc = lin_gemm_quantize(h, X, x_dtype, M, K, kind, h->dq, sa, stream);
  if (rc != LIN_OK) return rc;
  lin_scales_t sc{sa, sb, alpha};
  return lin_gemm_run(h, h->dq, B, &sc, bias, residual, C, M, N, K, quant_mode, activation, stream);
}

int lin_gemm_run_grouped(lin_gemm_t h, const void* A, const void* B, const lin_scales_t* scales,
                         const void* bias, const void* residual, void* C, const int32_t* offsets,
                         int64_t E, int64_t M, int64_t N, int64_t K, int64_t max_rows,
                         int quant_mode, int activation, void* stream) {
  if (!h) return LIN_ERR_INVALID_ARG;
  h->last_error.clear();
  if (E < 0 || M < 0 || max_rows < 0) return fail(h, LIN_ERR_INVALID_ARG, "negative size");
  // Each token chunk is a decode-shaped call of up to 32 rows: the shape rules
  // of lin_gemm_run apply to it.
  int rc = check_shape(h, quant_mode, M == 0 ? 0 : 1, N, K);
  if (rc != LIN_OK || M == 0 || E == 0) return rc;
  if (M >= ((int64_t)1 << 31)) return fail(h, LIN_ERR_UNSUPPORTED, "M beyond 2^31");
  if (E > 65535) return fail(h, LIN_ERR_UNSUPPORTED, "more than 65535 experts");
  if (!A || !B || !C || !offsets)
    return fail(h, LIN_ERR_INVALID_ARG, "A, B, C and offsets must be non-null");
  if (!(activation >= LIN_ACT_NONE && activation <= LIN_ACT_SILU) && activation != LIN_ACT_RAW_ACC)
    return fail(h, LIN_ERR_INVALID_ARG, "unknown activation " + std::to_string(activation));
  const bool quantised = quant_mode >= LIN_Q_FP8_DYNAMIC && quant_mode != LIN_Q_MXFP4;
  if (quantised && (!scales || !scales->a || !scales->b))
    return fail(h, LIN_ERR_INVALID_ARG, "quantised modes need scales->a and scales->b");
  if (quant_mode == LIN_Q_MXFP4 && (!scales || !scales->b))
    return fail(h, LIN_ERR_INVALID_ARG, "MXFP4 weights need scales->b (E8M0 bytes)");
  if (misaligned(A) || misaligned(B) || misaligned(C) || misaligned(bias) || misaligned(residual))
    return fail(h, LIN_ERR_UNSUPPORTED, "A, B, C, bias and residual must be 16-byte aligned");
  if (scales && (misaligned(scales->a) || misaligned(scales->b)))
    return fail(h, LIN_ERR_UNSUPPORTED, "scale arrays must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(offsets) & 3)
    return fail(h, LIN_ERR_UNSUPPORTED, "offsets must be 4-byte aligned");

  lg::Call c{};
  c.A = A; c.B = B; c.M = M; c.N = N; c.K = K;
  c.KB = b_row_bytes(quant_mode, K);
  c.qk = qkind(quant_mode);
  c.epi = make_epi(scales, bias, residual, C, M, N, quant_mode, activation);
  // The typical segment: the mean rows per expert (M / E) capped by the
  // caller's bound.  Beyond 4 rows (or with a forced tile variant) the tile
  // kernels take every BM-row tile of every segment; otherwise the decode
  // kernels take 16- or 32-token chunks.  (Measured on a 128-expert layer,
  // N = 1536, K = 2048: decode 75.5 against tile 78.3 us at 4 rows per
  // expert, 83.3 against 80.8 at 8.)
  const int64_t bound = (max_rows == 0 || max_rows > M) ? M : max_rows;
  const int64_t mean = std::min(bound, (M + E - 1) / E);
  if ((h->forced && h->force.kind == lg::V_TILE) || (!h->forced && mean > 4)) {
    lg::Variant t;
    t.kind = lg::V_TILE;
    if (h->forced) {
      t = h->force;
      if (!lg::grouped_tile_supported(t.bm, t.bn, t.wm, t.wn) ||
          !lg::tile_supported(c.qk, t.bm, t.bn, t.wm, t.wn))
        return fail(h, LIN_ERR_UNSUPPORTED, "tile shape not compiled for grouped calls");
    } else if (mean <= 256) {
      t.bm = 64; t.bn = 128; t.wm = 1; t.wn = 4;
    } else {
      t.bm = 256; t.bn = 256; t.wm = 2; t.wn = 4;
    }
    if ((M + t.bm - 1) / t.bm + std::min<int64_t>(E, M) > 65535)
      return fail(h, LIN_ERR_UNSUPPORTED, "too many row tiles for one grouped launch");
    hipError_t e = lg::launch_grouped_tile(t, c, offsets, E, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(h, e, "grouped kernel launch");
    return LIN_OK;
  }
  const int ntt = mean <= 16 ? 1 : 2;
  const int chunks = (int)std::min<int64_t>((mean + 16 * ntt - 1) / (16 * ntt), 65535);
  // A forced decode variant picks the grouped variant: its waves, unroll
  // and rows where that grouped variant is compiled, else the default with
  // its staging choice (staging dropped where the mode has none).
  // Unforced: the default of the mode, every lane loading its own
  // activations (staging measured no faster on decode-sized segments).
  lg::Variant v;
  v.waves = 0;
  v.xs = 0;
  if (h->forced) {
    if (h->force.kind != lg::V_DECODE || h->force.swap != 1)
      return fail(h, LIN_ERR_UNSUPPORTED, "grouped calls use swap-orientation decode variants");
    v = h->force;
    if (!lg::grouped_supported(v, c.qk, ntt, c.KB)) v.waves = 0;
  }
  if (!lg::grouped_supported(v, c.qk, ntt, c.KB)) {
    v.waves = 0;
    v.xs = 0;
  }
  hipError_t e = lg::launch_grouped(v, c, offsets, E, ntt, chunks, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(h, e, "grouped kernel launch");
  return LIN_OK;
}

}  // extern "C"
