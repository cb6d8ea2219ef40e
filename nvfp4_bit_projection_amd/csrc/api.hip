// api.hip -- the C ABI (include/flint_moe.h): argument validation, workspace
// carving and kernel launches.  Every check runs on the host before anything
// is enqueued, so a failing call leaves all buffers untouched.
#include <atomic>
#include <mutex>
#include <string.h>

#include "flint_common.h"
#include "flint_internal.h"

using namespace flint;

namespace {

std::atomic<int32_t> g_last_hip_error{0};
std::atomic<int32_t> g_device_ok[64];  // 0 unknown, 1 gfx950, -1 other

int32_t hip_fail(hipError_t e) {
  g_last_hip_error.store((int32_t)e);
  return FLINT_E_HIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

int32_t check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= 64) return FLINT_E_DEVICE;
  int st = g_device_ok[dev].load();
  if (st == 0) {
    hipDeviceProp_t p;
    e = hipGetDeviceProperties(&p, dev);
    if (e != hipSuccess) return hip_fail(e);
    st = (strncmp(p.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    g_device_ok[dev].store(st);
  }
  return st == 1 ? FLINT_OK : FLINT_E_DEVICE;
}

int32_t check_dims(const flint_moe_dims* d) {
  if (!d) return FLINT_E_NULL;
  if (d->hidden < 32 || d->hidden % 32 || d->top_k < 1 || d->top_k > kMaxTopK || d->n_experts < d->top_k ||
      d->n_experts > kMaxExperts || d->expert_width < 32 || d->expert_width % 32 || d->expert_width > 2048 ||
      d->shared_width < 32 || d->shared_width % 32 || d->shared_width > 2048)
    return FLINT_E_DIMS;
  if (d->hidden != kHidden) return FLINT_E_UNSUPPORTED;
  if (d->top_k * d->expert_width + d->shared_width > kMaxKdown) return FLINT_E_UNSUPPORTED;
  return FLINT_OK;
}

int32_t check_nvfp4(const flint_nvfp4* q) {
  if (!q || !q->codes || !q->scales || !q->tscale) return FLINT_E_NULL;
  if (!aligned16(q->codes) || !aligned4(q->scales) || !aligned4(q->tscale)) return FLINT_E_ALIGN;
  return FLINT_OK;
}

int32_t check_layer(const flint_moe_layer* L) {
  if (!L) return FLINT_E_NULL;
  if (!L->router || !L->gate_codes || !L->gate_scales || !L->up_codes || !L->up_scales || !L->down_codes ||
      !L->down_scales || !L->expert_tscales)
    return FLINT_E_NULL;
  if (!aligned16(L->router) || !aligned16(L->gate_codes) || !aligned16(L->up_codes) || !aligned16(L->down_codes) ||
      !aligned4(L->gate_scales) || !aligned4(L->up_scales) || !aligned4(L->down_scales) || !aligned4(L->expert_tscales))
    return FLINT_E_ALIGN;
  int32_t st;
  if ((st = check_nvfp4(&L->shared_gate)) || (st = check_nvfp4(&L->shared_up)) || (st = check_nvfp4(&L->shared_down)))
    return st;
  return FLINT_OK;
}

template <typename T>
T* carve(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

}  // namespace

int32_t flint::api_hip_fail(hipError_t e) { return hip_fail(e); }
int32_t flint::api_check_device() { return check_device(); }

extern "C" {

const char* flint_status_str(int32_t s) {
  switch (s) {
    case FLINT_OK: return "ok";
    case FLINT_E_NULL: return "a required pointer is NULL";
    case FLINT_E_DIMS: return "a size is out of range";
    case FLINT_E_ALIGN: return "a pointer is not 16-byte aligned";
    case FLINT_E_WORKSPACE: return "workspace or table buffer too small";
    case FLINT_E_DEVICE: return "current device is not gfx950";
    case FLINT_E_HIP: return "a HIP call failed";
    case FLINT_E_INTERNAL: return "a device-side wait gave up in an earlier call";
    case FLINT_E_UNSUPPORTED: return "sizes not supported by this build";
    default: return "unknown status";
  }
}

int32_t flint_last_hip_error(void) { return g_last_hip_error.load(); }

size_t flint_workspace_bytes(int32_t op, const flint_moe_dims* dims, int32_t B, int32_t vocab, int32_t L) {
  (void)L;
  if (B < 1) return 0;
  switch (op) {
    case FLINT_OP_ROUTE:
      if (check_dims(dims) != FLINT_OK) return 0;
      return RouteWs(dims->n_experts, B).total;
    case FLINT_OP_DECODE:
      if (check_dims(dims) != FLINT_OK) return 0;
      return DecodeWs(*dims, B).total;
    case FLINT_OP_LMHEAD:
      if (vocab < 1) return 0;
      return HeadWs(B).total;
    case FLINT_OP_STACK:
      if (check_dims(dims) != FLINT_OK || vocab < 1) return 0;
      return StackWs(*dims, vocab).total;
    case FLINT_OP_QUANTIZE:  // B = number of matrices
      return align_up(4 * (size_t)B, 256);
    case FLINT_OP_STACK_BATCH:
      if (check_dims(dims) != FLINT_OK || vocab < 1 || !batch_supported(*dims, B)) return 0;
      return BatchWs(*dims, B, vocab).total;
    default:
      return 0;
  }
}

int32_t flint_moe_route(const flint_moe_dims* dims, const float* router, const float* x, int32_t B, int32_t* topk_idx,
                        float* topk_w, float* logits_opt, void* ws, size_t ws_bytes, void* stream) {
  int32_t st;
  if ((st = check_dims(dims))) return st;
  if (!router || !x || !topk_idx || !topk_w || !ws) return FLINT_E_NULL;
  if (B < 1) return FLINT_E_DIMS;
  if (!aligned16(router) || !aligned16(x) || !aligned4(topk_idx) || !aligned4(topk_w) || !aligned16(ws) ||
      (logits_opt && !aligned4(logits_opt)))
    return FLINT_E_ALIGN;
  RouteWs rw(dims->n_experts, B);
  if (ws_bytes < rw.total) return FLINT_E_WORKSPACE;
  if ((st = check_device())) return st;
  hipStream_t s = (hipStream_t)stream;
  float* logits = logits_opt ? logits_opt : carve<float>(ws, rw.logits);
  hipError_t e = launch_route(*dims, router, x, B, -1.0f, logits, topk_idx, topk_w, s);
  return e == hipSuccess ? FLINT_OK : hip_fail(e);
}

int32_t flint_moe_route_ex(const flint_moe_dims* dims, const void* router, int32_t router_dtype, int32_t scoring,
                           const float* x, int32_t B, int32_t* topk_idx, float* topk_w, float* logits_opt, void* ws,
                           size_t ws_bytes, void* stream) {
  int32_t st;
  if ((st = check_dims(dims))) return st;
  if (!router || !x || !topk_idx || !topk_w || !ws) return FLINT_E_NULL;
  if (B < 1) return FLINT_E_DIMS;
  if ((router_dtype != FLINT_ROUTER_F32 && router_dtype != FLINT_ROUTER_BF16) ||
      (scoring != FLINT_SCORE_SOFTMAX && scoring != FLINT_SCORE_SIGMOID))
    return FLINT_E_DIMS;
  if (!aligned16(router) || !aligned16(x) || !aligned4(topk_idx) || !aligned4(topk_w) || !aligned16(ws) ||
      (logits_opt && !aligned4(logits_opt)))
    return FLINT_E_ALIGN;
  RouteWs rw(dims->n_experts, B);
  if (ws_bytes < rw.total) return FLINT_E_WORKSPACE;
  if ((st = check_device())) return st;
  hipStream_t s = (hipStream_t)stream;
  float* logits = logits_opt ? logits_opt : carve<float>(ws, rw.logits);
  hipError_t e = launch_route_ex(*dims, router, router_dtype == FLINT_ROUTER_BF16, scoring == FLINT_SCORE_SIGMOID, x,
                                 B, logits, topk_idx, topk_w, s);
  return e == hipSuccess ? FLINT_OK : hip_fail(e);
}

static int32_t decode_impl(const flint_moe_dims& d, const flint_moe_layer& L, const float* x, int B, float norm_eps,
                           float* y, bool add_to_y, int32_t* idx, float* w, void* ws, hipStream_t s) {
  DecodeWs dw(d, B);
  RouteWs rw(d.n_experts, B);
  char* base = static_cast<char*>(ws);
  float* logits = carve<float>(base + dw.route, rw.logits);
  float* hact = carve<float>(ws, dw.hact);
  hipError_t e = launch_route(d, L.router, x, B, norm_eps, logits, idx, w, s);
  if (e == hipSuccess) e = launch_gateup(d, L, x, B, norm_eps, idx, hact, s);
  if (e == hipSuccess) e = launch_down(d, L, idx, w, hact, B, y, add_to_y, s);
  return e == hipSuccess ? FLINT_OK : hip_fail(e);
}

}  // extern "C"

int32_t flint::api_moe_check(const flint_moe_dims* d, const flint_moe_layer* L) {
  int32_t st;
  if ((st = check_dims(d))) return st;
  return check_layer(L);
}
size_t flint::api_moe_ws_bytes(const flint_moe_dims& d) { return DecodeWs(d, 1).total; }
hipError_t flint::api_moe_run(const flint_moe_dims& d, const flint_moe_layer& L, const float* x, float norm_eps,
                              float* y, bool add, void* ws, hipStream_t s) {
  const DecodeWs dw(d, 1);
  const RouteWs rw(d.n_experts, 1);
  char* base = static_cast<char*>(ws);
  int32_t* idx = carve<int32_t>(ws, dw.idx);
  float* w = carve<float>(ws, dw.wts);
  hipError_t e = launch_route(d, L.router, x, 1, norm_eps, carve<float>(base + dw.route, rw.logits), idx, w, s);
  if (e == hipSuccess) e = launch_gateup(d, L, x, 1, norm_eps, idx, carve<float>(ws, dw.hact), s);
  if (e == hipSuccess) e = launch_down(d, L, idx, w, carve<float>(ws, dw.hact), 1, y, add, s);
  return e;
}

extern "C" {

int32_t flint_moe_decode(const flint_moe_dims* dims, const flint_moe_layer* layer, const float* x, int32_t B, float* y,
                         int32_t* topk_idx_opt, float* topk_w_opt, void* ws, size_t ws_bytes, void* stream) {
  int32_t st;
  if ((st = check_dims(dims))) return st;
  if ((st = check_layer(layer))) return st;
  if (!x || !y || !ws) return FLINT_E_NULL;
  if (B < 1) return FLINT_E_DIMS;
  if (!aligned16(x) || !aligned16(y) || !aligned16(ws) || (topk_idx_opt && !aligned4(topk_idx_opt)) ||
      (topk_w_opt && !aligned4(topk_w_opt)))
    return FLINT_E_ALIGN;
  DecodeWs dw(*dims, B);
  if (ws_bytes < dw.total) return FLINT_E_WORKSPACE;
  if ((st = check_device())) return st;
  int32_t* idx = topk_idx_opt ? topk_idx_opt : carve<int32_t>(ws, dw.idx);
  float* w = topk_w_opt ? topk_w_opt : carve<float>(ws, dw.wts);
  return decode_impl(*dims, *layer, x, B, -1.0f, y, false, idx, w, ws, (hipStream_t)stream);
}

}  // extern "C"

// Scratch of flint_moe_decode_noalloc: a fixed device array, one copy per
// GPU, held until the process ends.  Host code never passes `scratch` itself
// to a kernel (on the host that name is only a stand-in); it takes the
// array's device address from hipGetSymbolAddress once per device and uses
// that address everywhere.
constexpr size_t kNoAllocScratchBytes = 1179648;  // 1.125 MiB
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];  // device address of `scratch` per device (null until set up)

int32_t noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= 64) return FLINT_E_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {  // first call on this device, with it current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (!p) return FLINT_E_INTERNAL;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FLINT_OK;
}
}  // namespace

extern "C" {

int32_t flint_moe_decode_noalloc(const flint_moe_dims* dims, const flint_moe_layer* layer, const float* x, int32_t B,
                                 float* y, int32_t* topk_idx_opt, float* topk_w_opt, void* stream) {
  int32_t st;
  if ((st = check_dims(dims))) return st;
  if ((st = check_layer(layer))) return st;
  if (!x || !y) return FLINT_E_NULL;
  if (B < 1) return FLINT_E_DIMS;
  if (!aligned16(x) || !aligned16(y) || (topk_idx_opt && !aligned4(topk_idx_opt)) ||
      (topk_w_opt && !aligned4(topk_w_opt)))
    return FLINT_E_ALIGN;
  const DecodeWs dw(*dims, B);
  if (dw.total > kNoAllocScratchBytes) return FLINT_E_WORKSPACE;
  if ((st = check_device())) return st;
  void* ws = nullptr;
  if ((st = noalloc_scratch(&ws))) return st;
  // the same kernels as flint_moe_decode on the same scratch layout; every
  // scratch byte a kernel reads was written earlier in this call, so nothing
  // has to be cleared
  int32_t* idx = topk_idx_opt ? topk_idx_opt : carve<int32_t>(ws, dw.idx);
  float* w = topk_w_opt ? topk_w_opt : carve<float>(ws, dw.wts);
  return decode_impl(*dims, *layer, x, B, -1.0f, y, false, idx, w, ws, (hipStream_t)stream);
}

int32_t flint_lmhead_gemv(const flint_nvfp4* head, int32_t vocab, int32_t hidden, const float* x, int32_t B,
                          float* logits, int32_t* argmax, void* ws, size_t ws_bytes, void* stream) {
  int32_t st;
  if ((st = check_nvfp4(head))) return st;
  if (!x || !logits || !argmax || !ws) return FLINT_E_NULL;
  if (vocab < 1 || B < 1 || hidden < 32 || hidden % 32) return FLINT_E_DIMS;
  if (hidden != kHidden) return FLINT_E_UNSUPPORTED;
  if (!aligned16(x) || !aligned4(logits) || !aligned4(argmax) || !aligned16(ws)) return FLINT_E_ALIGN;
  HeadWs hw(B);
  if (ws_bytes < hw.total) return FLINT_E_WORKSPACE;
  if ((st = check_device())) return st;
  hipError_t e = launch_lmhead(*head, vocab, x, B, -1.0f, logits, argmax, carve<HeadPartial>(ws, hw.partials),
                               (hipStream_t)stream);
  return e == hipSuccess ? FLINT_OK : hip_fail(e);
}

size_t flint_stack_table_bytes(int32_t L) { return L < 1 ? 0 : stack_table_bytes(L); }

size_t flint_stack_packed_bytes(const flint_moe_dims* dims, int32_t L) {
  if (check_dims(dims) || !stack_persistent_supported(*dims, L)) return 0;
  return PackedDown(*dims).total * (size_t)L;
}

int32_t flint_stack_prepare(const flint_moe_dims* dims, const flint_moe_layer* layers, int32_t L,
                            const flint_nvfp4* head, int32_t vocab, void* table, size_t table_bytes, void* packed,
                            size_t packed_bytes, flint_stack_plan* plan, void* stream) {
  int32_t st;
  if ((st = check_dims(dims))) return st;
  if (!layers || !head || !table || !plan) return FLINT_E_NULL;
  if (L < 1 || vocab < 1) return FLINT_E_DIMS;
  for (int l = 0; l < L; ++l)
    if ((st = check_layer(&layers[l]))) return st;
  if ((st = check_nvfp4(head))) return st;
  if (!aligned16(table)) return FLINT_E_ALIGN;
  if (table_bytes < stack_table_bytes(L)) return FLINT_E_WORKSPACE;
  if (packed) {
    if (!stack_persistent_supported(*dims, L)) return FLINT_E_UNSUPPORTED;
    if (!aligned16(packed)) return FLINT_E_ALIGN;
    if (packed_bytes < PackedDown(*dims).total * (size_t)L) return FLINT_E_WORKSPACE;
  }
  if ((st = check_device())) return st;
  hipStream_t s = (hipStream_t)stream;
  // build the table on the host, then one copy; the copy completes before
  // this call returns, so the host buffer may be freed right after.  With a
  // packed buffer, the table's down-projection pointers refer to the packed
  // (column-sliced) copies.
  const size_t nb = stack_table_bytes(L);
  char* host = new char[nb];
  StackTable* t = reinterpret_cast<StackTable*>(host);
  t->head = *head;
  memcpy(t->layers, layers, sizeof(flint_moe_layer) * (size_t)L);
  hipError_t e = hipSuccess;
  if (packed) {
    const PackedDown pd(*dims);
    const int H = dims->hidden, E = dims->n_experts, I = dims->expert_width, Is = dims->shared_width;
    for (int l = 0; l < L && e == hipSuccess; ++l) {
      uint8_t* base = static_cast<uint8_t*>(packed) + pd.total * (size_t)l;
      const flint_moe_layer& src = layers[l];
      flint_moe_layer& dst = t->layers[l];
      e = launch_slice_cols(src.down_codes, base + pd.codes, E, H, I / 2, kStackGroups, s);
      if (e == hipSuccess) e = launch_slice_cols(src.down_scales, base + pd.scales, E, H, I / 16, kStackGroups, s);
      if (e == hipSuccess)
        e = launch_slice_cols(src.shared_down.codes, base + pd.shared_codes, 1, H, Is / 2, kStackGroups, s);
      if (e == hipSuccess)
        e = launch_slice_cols(src.shared_down.scales, base + pd.shared_scales, 1, H, Is / 16, kStackGroups, s);
      dst.down_codes = base + pd.codes;
      dst.down_scales = base + pd.scales;
      dst.shared_down.codes = base + pd.shared_codes;
      dst.shared_down.scales = base + pd.shared_scales;
    }
  }
  if (e == hipSuccess) e = hipMemcpyAsync(table, host, nb, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  delete[] host;
  if (e != hipSuccess) return hip_fail(e);
  plan->dims = *dims;
  plan->n_layers = L;
  plan->vocab = vocab;
  plan->head = *head;
  plan->layers = layers;
  plan->table = table;
  plan->schedule = FLINT_SCHEDULE_AUTO;
  plan->packed = packed;
  return FLINT_OK;
}

static int32_t stack_decode_impl(const flint_stack_plan* plan, const float* x, int32_t T, float eps, float* logits,
                                 int32_t* argmax, int32_t* routes_opt, void* ws, size_t ws_bytes, int64_t* trace,
                                 void* stream) {
  int32_t st;
  if (!plan || !x || !argmax || !ws) return FLINT_E_NULL;
  if ((st = check_dims(&plan->dims))) return st;
  if (!plan->layers || !plan->table) return FLINT_E_NULL;
  if (T < 1 || plan->n_layers < 1 || plan->vocab < 1 || !(eps > 0.0f) || plan->schedule < 0 || plan->schedule > 2)
    return FLINT_E_DIMS;
  if (!aligned16(x) || !aligned16(ws) || !aligned4(argmax) || (logits && !aligned4(logits)) ||
      (routes_opt && !aligned4(routes_opt)))
    return FLINT_E_ALIGN;
  const flint_moe_dims& d = plan->dims;
  StackWs sw(d, plan->vocab);
  if (ws_bytes < sw.total) return FLINT_E_WORKSPACE;
  const bool persistent_ok = plan->packed && stack_persistent_supported(d, plan->n_layers);
  if (plan->schedule == FLINT_SCHEDULE_PERSISTENT && !persistent_ok) return FLINT_E_UNSUPPORTED;
  if ((st = check_device())) return st;
  hipStream_t s = (hipStream_t)stream;
  if (persistent_ok && plan->schedule != FLINT_SCHEDULE_KERNELS) {
    hipError_t e = launch_stack_persistent(d, plan->n_layers, plan->vocab, plan->table, x, T, eps, logits, argmax,
                                           routes_opt, static_cast<char*>(ws) + sw.persist, trace, s);
    return e == hipSuccess ? FLINT_OK : hip_fail(e);
  }
  char* base = static_cast<char*>(ws);
  float* h = carve<float>(ws, sw.h);
  void* dws = base + sw.decode;
  DecodeWs dw(d, 1);
  HeadWs hw(1);
  const int L = plan->n_layers, k = d.top_k;
  for (int t = 0; t < T; ++t) {
    hipError_t e = launch_copy_f32(x + (size_t)t * kHidden, h, kHidden, s);
    if (e != hipSuccess) return hip_fail(e);
    for (int l = 0; l < L; ++l) {
      int32_t* idx = routes_opt ? routes_opt + ((size_t)t * L + l) * k : carve<int32_t>(dws, dw.idx);
      st = decode_impl(d, plan->layers[l], h, 1, eps, h, true, idx, carve<float>(dws, dw.wts), dws, s);
      if (st) return st;
    }
    e = launch_lmhead(plan->head, plan->vocab, h, 1, eps, logits ? logits + (size_t)t * plan->vocab : nullptr,
                      argmax + t, carve<HeadPartial>(base + sw.head, hw.partials), s);
    if (e != hipSuccess) return hip_fail(e);
  }
  return FLINT_OK;
}

int32_t flint_stack_decode(const flint_stack_plan* plan, const float* x, int32_t T, float eps, float* logits,
                           int32_t* argmax, int32_t* routes_opt, void* ws, size_t ws_bytes, void* stream) {
  return stack_decode_impl(plan, x, T, eps, logits, argmax, routes_opt, ws, ws_bytes, nullptr, stream);
}

int32_t flint_stack_decode_traced(const flint_stack_plan* plan, const float* x, int32_t T, float eps, float* logits,
                                  int32_t* argmax, int32_t* routes_opt, void* ws, size_t ws_bytes, int64_t* trace,
                                  void* stream) {
  if (!trace) return FLINT_E_NULL;
  if (!aligned16(trace)) return FLINT_E_ALIGN;
  if (plan && plan->schedule == FLINT_SCHEDULE_KERNELS) return FLINT_E_UNSUPPORTED;
  if (plan && (!plan->packed || !stack_persistent_supported(plan->dims, plan->n_layers))) return FLINT_E_UNSUPPORTED;
  return stack_decode_impl(plan, x, T, eps, logits, argmax, routes_opt, ws, ws_bytes, trace, stream);
}

int32_t flint_stack_decode_layers(const flint_stack_plan* plan, int32_t l0, int32_t n, const float* x, float eps,
                                  float* h_out, int32_t* routes_opt, void* ws, size_t ws_bytes, void* stream) {
  int32_t st;
  if (!plan || !x || !h_out || !ws) return FLINT_E_NULL;
  if ((st = check_dims(&plan->dims))) return st;
  if (!plan->layers || !plan->table) return FLINT_E_NULL;
  if (plan->n_layers < 1 || l0 < 0 || n < 1 || l0 + n > plan->n_layers || !(eps > 0.0f)) return FLINT_E_DIMS;
  if (!plan->packed || !stack_persistent_supported(plan->dims, plan->n_layers)) return FLINT_E_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(h_out) || !aligned16(ws) || (routes_opt && !aligned4(routes_opt)))
    return FLINT_E_ALIGN;
  StackWs sw(plan->dims, plan->vocab > 0 ? plan->vocab : 1);
  if (ws_bytes < sw.total) return FLINT_E_WORKSPACE;
  if ((st = check_device())) return st;
  hipError_t e = launch_stack_persistent(plan->dims, n, 0, plan->table, x, 1, eps, nullptr, nullptr, routes_opt,
                                         static_cast<char*>(ws) + sw.persist, nullptr, (hipStream_t)stream, l0, h_out);
  return e == hipSuccess ? FLINT_OK : hip_fail(e);
}

int32_t flint_stack_decode_stress(const flint_stack_plan* plan, const float* x, int32_t T, float eps, float* logits,
                                  int32_t* argmax, int32_t* routes_opt, void* ws, size_t ws_bytes, uint32_t seed,
                                  uint32_t spin_limit, void* stream) {
  int32_t st;
  if (!plan || !x || !argmax || !ws) return FLINT_E_NULL;
  if ((st = check_dims(&plan->dims))) return st;
  if (!plan->layers || !plan->table) return FLINT_E_NULL;
  if (T < 1 || plan->n_layers < 1 || plan->vocab < 1 || !(eps > 0.0f) || spin_limit < 1) return FLINT_E_DIMS;
  if (!plan->packed || !stack_persistent_supported(plan->dims, plan->n_layers)) return FLINT_E_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(ws) || !aligned4(argmax) || (logits && !aligned4(logits)) ||
      (routes_opt && !aligned4(routes_opt)))
    return FLINT_E_ALIGN;
  StackWs sw(plan->dims, plan->vocab);
  if (ws_bytes < sw.total) return FLINT_E_WORKSPACE;
  if ((st = check_device())) return st;
  hipError_t e = launch_stack_persistent(plan->dims, plan->n_layers, plan->vocab, plan->table, x, T, eps, logits,
                                         argmax, routes_opt, static_cast<char*>(ws) + sw.persist, nullptr,
                                         (hipStream_t)stream, 0, nullptr, nullptr, seed, spin_limit);
  return e == hipSuccess ? FLINT_OK : hip_fail(e);
}

int32_t flint_stack_decode_batch(const flint_stack_plan* plan, const float* x, int32_t B, float eps, float* logits,
                                 int32_t* argmax, int32_t* routes_opt, void* ws, size_t ws_bytes, void* stream) {
  int32_t st;
  if (!plan || !x || !argmax || !ws) return FLINT_E_NULL;
  if (!plan->layers || !plan->table) return FLINT_E_NULL;
  const flint_moe_dims& d = plan->dims;
  if ((st = check_dims(&d))) return st;
  if (B < 1 || B > kMaxBatch || !(eps >= 0.0f)) return FLINT_E_DIMS;
  if (!batch_supported(d, B)) return FLINT_E_UNSUPPORTED;
  if (!aligned16(x) || (logits && !aligned4(logits)) || !aligned4(argmax) || (routes_opt && !aligned4(routes_opt)) ||
      !aligned16(ws))
    return FLINT_E_ALIGN;
  if (ws_bytes < BatchWs(d, B, plan->vocab).total) return FLINT_E_WORKSPACE;
  if ((st = check_device())) return st;
  hipError_t e = launch_batch_step(d, plan->layers, plan->n_layers, plan->head, plan->vocab, x, B, eps, logits, argmax,
                                   routes_opt, ws, (hipStream_t)stream);
  return e == hipSuccess ? FLINT_OK : hip_fail(e);
}

size_t flint_stack_batch_tiles_bytes(const flint_moe_dims* dims, int32_t L) {
  if (check_dims(dims) != FLINT_OK || L < 1 || !batch_supported(*dims, 1)) return 0;
  return (size_t)L * batch_tiles_layer_bytes(*dims);
}

int32_t flint_stack_batch_tiles(const flint_stack_plan* plan, void* tiles, size_t tiles_bytes, void* stream) {
  if (!plan || !tiles || !plan->layers) return FLINT_E_NULL;
  int32_t st;
  if ((st = check_dims(&plan->dims))) return st;
  const size_t need = flint_stack_batch_tiles_bytes(&plan->dims, plan->n_layers);
  if (need == 0) return FLINT_E_UNSUPPORTED;
  if (!aligned16(tiles)) return FLINT_E_ALIGN;
  if (tiles_bytes < need) return FLINT_E_WORKSPACE;
  for (int l = 0; l < plan->n_layers; ++l)
    if ((st = check_layer(&plan->layers[l]))) return st;
  if ((st = check_device())) return st;
  hipError_t e = launch_batch_tiles(plan->dims, plan->layers, plan->n_layers, static_cast<uint8_t*>(tiles),
                                    (hipStream_t)stream);
  return e == hipSuccess ? FLINT_OK : hip_fail(e);
}

int32_t flint_stack_decode_batch_tiled(const flint_stack_plan* plan, const void* tiles, const float* x, int32_t B,
                                       float eps, float* logits, int32_t* argmax, int32_t* routes_opt, void* ws,
                                       size_t ws_bytes, void* stream) {
  int32_t st;
  if (!plan || !tiles || !x || !argmax || !ws) return FLINT_E_NULL;
  if (!plan->layers || !plan->table) return FLINT_E_NULL;
  const flint_moe_dims& d = plan->dims;
  if ((st = check_dims(&d))) return st;
  if (B < 1 || B > kMaxBatch || !(eps >= 0.0f)) return FLINT_E_DIMS;
  if (!batch_supported(d, B)) return FLINT_E_UNSUPPORTED;
  if (!aligned16(tiles) || !aligned16(x) || (logits && !aligned4(logits)) || !aligned4(argmax) ||
      (routes_opt && !aligned4(routes_opt)) || !aligned16(ws))
    return FLINT_E_ALIGN;
  if (ws_bytes < BatchWs(d, B, plan->vocab).total) return FLINT_E_WORKSPACE;
  if ((st = check_device())) return st;
  hipError_t e = launch_batch_step_tiled(d, plan->layers, plan->n_layers, plan->head, plan->vocab, x, B, eps, logits,
                                         argmax, routes_opt, ws, (hipStream_t)stream,
                                         static_cast<const uint8_t*>(tiles));
  return e == hipSuccess ? FLINT_OK : hip_fail(e);
}

int32_t flint_stack_error(const void* ws, size_t ws_bytes, int32_t* error) {
  if (!ws || !error) return FLINT_E_NULL;
  if (ws_bytes < 256) return FLINT_E_WORKSPACE;
  hipError_t e = read_stack_error(ws, error);
  return e == hipSuccess ? FLINT_OK : hip_fail(e);
}

int32_t flint_nvfp4_quantize(const float* w, int64_t n_mats, int64_t rows, int64_t cols, uint8_t* codes,
                             uint8_t* scales, float* tscales, void* ws, size_t ws_bytes, void* stream) {
  if (!w || !codes || !scales || !tscales || !ws) return FLINT_E_NULL;
  if (n_mats < 1 || rows < 1 || cols < 32 || cols % 32) return FLINT_E_DIMS;
  if (!aligned16(w) || !aligned16(codes) || !aligned4(scales) || !aligned4(tscales) || !aligned16(ws))
    return FLINT_E_ALIGN;
  if (n_mats > (int64_t)1 << 30 || ws_bytes < align_up(4 * (size_t)n_mats, 256)) return FLINT_E_WORKSPACE;
  int32_t st;
  if ((st = check_device())) return st;
  hipError_t e = launch_quantize(w, n_mats, rows, cols, codes, scales, tscales, carve<uint32_t>(ws, 0),
                                 (hipStream_t)stream);
  return e == hipSuccess ? FLINT_OK : hip_fail(e);
}

int32_t flint_nvfp4_dequantize(const flint_nvfp4* q, int64_t rows, int64_t cols, float* out, void* stream) {
  int32_t st;
  if ((st = check_nvfp4(q))) return st;
  if (!out) return FLINT_E_NULL;
  if (rows < 1 || cols < 32 || cols % 32) return FLINT_E_DIMS;
  if (!aligned16(out)) return FLINT_E_ALIGN;
  if ((st = check_device())) return st;
  hipError_t e = launch_dequantize(*q, rows, cols, out, (hipStream_t)stream);
  return e == hipSuccess ? FLINT_OK : hip_fail(e);
}

}  // extern "C"
