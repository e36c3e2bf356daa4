// C ABI and host runtime of the MoE layer: configuration checks, packed-weight
// and workspace layouts, the per-call launch plan, and error reporting.
// Nothing here allocates device memory or synchronises the host.
#include "../../include/moe_layer.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cfloat>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>

#include "moe_kernels.hpp"

namespace {

thread_local std::string g_last_error;

moe_status_t fail(moe_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

moe_status_t ok() {
  g_last_error.clear();
  return MOE_OK;
}

constexpr int kMaxTokens = 1 << 18;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

struct moe_layer {
  moe_layer_config_t cfg;
  int device;
  size_t expert_bytes;   // one routed expert, packed
  size_t shared_bytes;   // the shared expert, packed
  // second stream (default priority, non-blocking) for the hot experts'
  // LDS-tiled GEMMs, which then overlap the streaming GEMMs; created with the
  // handle when its configuration can take that path, else null.  The fork
  // and join events are created with it; aux_mu keeps one forward's fork
  // record and the second stream's wait on it together (another forward's
  // record in between would otherwise be the one waited for).
  hipStream_t aux = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  std::mutex aux_mu;
};

namespace {

size_t packed_group_bytes(const moe_layer_config_t& c, int width) {
  const size_t wh = (size_t)width * c.hidden;
  if (c.weight_dtype == MOE_INT4_G32) return wh + wh / 8 + wh / 2 + wh / 16;
  return 3 * wh * 2;
}

moe_status_t check_config(const moe_layer_config_t* c) {
  if (!c) return fail(MOE_ERR_NULL, "config is NULL");
  if (c->act_dtype != MOE_BF16 && c->act_dtype != MOE_F32)
    return fail(MOE_ERR_DTYPE, "act_dtype must be MOE_BF16 or MOE_F32 (got %d)", c->act_dtype);
  if (c->weight_dtype != MOE_BF16 && c->weight_dtype != MOE_INT4_G32)
    return fail(MOE_ERR_DTYPE, "weight_dtype must be MOE_BF16 or MOE_INT4_G32 (got %d)",
                c->weight_dtype);
  if (c->score != MOE_SCORE_SOFTMAX && c->score != MOE_SCORE_SIGMOID)
    return fail(MOE_ERR_DTYPE, "score must be MOE_SCORE_SOFTMAX or MOE_SCORE_SIGMOID");
  if (c->bias_mode != MOE_BIAS_LOGIT && c->bias_mode != MOE_BIAS_SELECT)
    return fail(MOE_ERR_DTYPE, "bias_mode must be MOE_BIAS_LOGIT or MOE_BIAS_SELECT");
  if (!(c->routed_scale == c->routed_scale) || c->routed_scale <= 0.f)
    return fail(MOE_ERR_SHAPE, "routed_scale must be a positive number");
  if (!(c->swiglu_limit >= 0.f && c->swiglu_limit <= FLT_MAX) ||
      !(c->swiglu_limit_shared >= 0.f && c->swiglu_limit_shared <= FLT_MAX))
    return fail(MOE_ERR_SHAPE, "SwiGLU limits must be finite and >= 0 (got %g, %g)",
                (double)c->swiglu_limit, (double)c->swiglu_limit_shared);
  if (c->num_experts < 1 || c->num_experts > 512)
    return fail(MOE_ERR_SHAPE, "num_experts must be in [1, 512] (got %d)", c->num_experts);
  if (c->top_k < 1 || c->top_k > 16 || c->top_k > c->num_experts)
    return fail(MOE_ERR_SHAPE, "top_k must be in [1, min(num_experts, 16)] (got %d)", c->top_k);
  if (c->hidden < 64 || c->hidden % 64)
    return fail(MOE_ERR_SHAPE, "hidden must be a positive multiple of 64 (got %d)", c->hidden);
  if (c->inter < 32 || c->inter % 32)
    return fail(MOE_ERR_SHAPE, "inter must be a positive multiple of 32 (got %d)", c->inter);
  if (c->shared_inter < 0 || c->shared_inter % 32)
    return fail(MOE_ERR_SHAPE, "shared_inter must be 0 or a multiple of 32 (got %d)",
                c->shared_inter);
  if (c->max_tokens < 1 || c->max_tokens > kMaxTokens)
    return fail(MOE_ERR_SHAPE, "max_tokens must be in [1, %d] (got %d)", kMaxTokens,
                c->max_tokens);
  if (c->weight_dtype == MOE_INT4_G32 &&
      (c->hidden % 128 || c->inter % 128 || c->shared_inter % 128))
    return fail(MOE_ERR_SHAPE, "INT4 weights need hidden, inter and shared_inter %% 128 == 0");
  return MOE_OK;
}

// Per-call plan and workspace layout.
struct Plan {
  int T, P, ks, tg, max_tiles, has_shared, hstride, tiled;
  // hybrid: streaming GEMMs for most groups, LDS-tiled ones (tg2, list 2) for
  // the groups with `hot` rows or more
  int hybrid, hot, tg2, max_tiles2;
  // the LDS-tiled down GEMM's K split (Y then holds ksplit partial-sum planes)
  // and the gate/up's (partial gate/up planes in gu_part, reduced into h)
  int ksplit, ksplit_gu;
  // bf16 activations and no K split: the down GEMMs weight the routed rows of
  // Y by their gate weights (row_w, written by the dispatch) and store them in
  // bf16 at the pairs' rows (yb = y), the shared rows in fp32 (ys)
  int y_bf16;
  size_t ys, row_w;
  size_t gu_part;
  size_t part, idx, w, gap, counts, offsets, perm, inv, row_tok, tiles, ntiles, tiles2, ntiles2,
      done, dbg, blk_hist, h, h_lo, h2, y, total;
  int large_dispatch;
};

// Rows from which a group leaves the streaming GEMMs for the LDS-tiled ones
// in a load-imbalanced batch, and the smallest batch that does so.
constexpr int kHotRows = 32;
constexpr int kHybridMinTokens = 256;

Plan make_plan(const moe_layer& L, int T) {
  const moe_layer_config_t& c = L.cfg;
  Plan p{};
  p.T = T;
  p.P = T * c.top_k;
  p.has_shared = c.shared_inter > 0;
  // router: split H so that small batches still spread over the CUs
  const int wgs = moe::router_blocks(c.act_dtype == MOE_F32, T, c.num_experts);
  p.ks = 1;
  while (wgs * p.ks < 256 && p.ks < 8 && (c.hidden / 32) % (2 * p.ks) == 0) p.ks *= 2;
  // expert GEMM tile rows: 16 when experts see about one row (decode), 32 or
  // 64 when denser
  const double rows_per_expert = (double)p.P / c.num_experts;
  p.tg = rows_per_expert < 2.0 ? 1 : (rows_per_expert < 24.0 ? 2 : 4);
  if (c.weight_dtype == MOE_INT4_G32 && p.tg > 2) p.tg = 2;  // register budget
  // LDS-staged tiles with bf16 h (bf16 weights and activations only) from 16
  // rows per expert on: measured even at 16 rows and ahead from ~20 (4% at
  // 21-28 rows, 10-28% at 36-57 rows, where the streaming kernels with
  // 64-row groups run at two waves per SIMD)
  p.tiled = rows_per_expert >= 16.0 && c.weight_dtype == MOE_BF16 && c.act_dtype == MOE_BF16;
  // 256-row tiles (one 8-wave workgroup per CU) from 128 rows per expert:
  // fewer bytes pulled per flop, the bound of these GEMMs (9-11% ahead at
  // 142-178 rows), but a tile that is mostly padding below that (96-114
  // rows: 128-row tiles 10% ahead)
  if (p.tiled) p.tg = rows_per_expert >= 128.0 ? 16 : 8;
  // A tiled batch with few tiles (one expert or a handful, e.g. a dense FFN
  // as one expert at a decode batch) would run its down GEMM -- K = the
  // expert width, up to thousands -- on a few dozen workgroups: K is split
  // into up to 16 parts, each writing its own partial-sum plane of Y, until
  // the launch has ~512 workgroups (the bound below counts every tile the
  // dispatch could write, so real batches use fewer).
  // The gate/up GEMM of such a batch splits K (H) the same way, up to 8
  // parts of an even number of k-steps; its parts write fp32 partial sums of
  // gate and up, and a reduction applies the SwiGLU.
  p.ksplit = 1;
  p.ksplit_gu = 1;
  if (p.tiled) {
    const int nz0 = c.num_experts < p.P ? c.num_experts : p.P;
    const long tiles = (long)nz0 + p.P / (16 * p.tg) + (p.has_shared ? T / (16 * p.tg) + 1 : 0) + 1;
    const long bound = tiles * ((c.hidden + 255) / 256);
    while (bound * p.ksplit < 512 && p.ksplit < 16 && (c.inter / 32) % (2 * p.ksplit) == 0 &&
           (c.shared_inter / 32) % (2 * p.ksplit) == 0)
      p.ksplit *= 2;
    const int wmax = c.inter > c.shared_inter ? c.inter : c.shared_inter;
    const long bound_gu = tiles * ((2 * wmax + 255) / 256);
    while (bound_gu * p.ksplit_gu < 512 && p.ksplit_gu < 8 &&
           (c.hidden / 32) % (4 * p.ksplit_gu) == 0)
      p.ksplit_gu *= 2;
  }
  // one workgroup dispatches small batches; larger ones use per-block counts
  p.large_dispatch = T > 1024;
  // Streaming batches whose routing is uneven (a Zipf-popular expert can
  // take most of the tokens) would stream a hot expert's weights once per
  // 16-32-row tile: routed experts with kHotRows rows or more go to 128-row
  // LDS tiles instead, launched on the handle's second stream beside the
  // streaming GEMMs (see forward_impl).  The shared expert stays with the
  // streaming GEMMs (a launch of its tiles alone would occupy a handful of
  // CUs).  From 256 tokens: with Zipf-popular experts, as a launch after the
  // streaming one, measured 6% faster at 256 tokens and 12% at 512 but 5%
  // slower at 128, where the hot experts' few tiles leave that launch mostly
  // idle; neutral on uniform routing.
  p.hybrid = !p.tiled && !p.large_dispatch && c.weight_dtype == MOE_BF16 &&
             c.act_dtype == MOE_BF16 && T >= kHybridMinTokens;
  p.hot = p.hybrid ? kHotRows : 0;
  p.tg2 = 8;
  const int bm = 16 * p.tg;
  const int nz = c.num_experts < p.P ? c.num_experts : p.P;
  p.max_tiles = nz + p.P / bm + (p.has_shared ? (T + bm - 1) / bm : 0) + 1;
  // list 2: at most P / kHotRows routed groups, ceil(rows / 128) tiles each
  p.max_tiles2 = p.hybrid ? p.P / (16 * p.tg2) + p.P / kHotRows + 1 : 0;
  const int rows = p.P + (p.has_shared ? T : 0);
  p.hstride = c.inter > c.shared_inter ? c.inter : c.shared_inter;
  const int E = c.num_experts;

  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  p.part = take((size_t)p.ks * T * E * 4);
  p.idx = take((size_t)p.P * 4);
  p.w = take((size_t)p.P * 4);
  p.gap = take((size_t)T * 4);
  p.counts = take((size_t)(E + 1) * 4);
  p.offsets = take((size_t)(E + 2) * 4);
  p.perm = take((size_t)p.P * 4);
  p.inv = take((size_t)p.P * 4);
  p.row_tok = take((size_t)rows * 4);
  p.tiles = take((size_t)p.max_tiles * 4);
  p.ntiles = take(4);
  p.tiles2 = take((size_t)p.max_tiles2 * 4);
  p.ntiles2 = take(p.hybrid ? 4 : 0);
  p.done = take(4);
  p.dbg = take(8);  // debug word pair: code and value of the first out-of-range index
  p.blk_hist = take(p.large_dispatch ? (size_t)moe::dispatch_blocks(T) * E * 4 : 0);
  // h: rows of hstride on the streaming paths -- fp32 for fp32 activations
  // with bf16 weights (it enters the down MFMA as hi + lo), bf16 otherwise;
  // bf16 in packed fragment order, with a 16-row gap per group and a tile of
  // slack, on the tiled path
  const size_t h_rows_tiled = moe::tiled_h_rows(rows, E);
  const size_t h_elem = (c.act_dtype == MOE_F32 && c.weight_dtype == MOE_BF16) ? 4 : 2;
  p.h = take(p.tiled ? h_rows_tiled * p.hstride * 2 : (size_t)rows * p.hstride * h_elem);
  // bf16 remainder of the shared expert's h: bf16 weights and activations
  const bool lo_plane = p.has_shared && c.weight_dtype == MOE_BF16 && c.act_dtype == MOE_BF16;
  p.h_lo = take(!lo_plane ? 0
                : p.tiled ? moe::tiled_h_rows(T, 0) * p.hstride * 2
                          : (size_t)T * p.hstride * 2);
  // the hybrid's LDS-tiled groups (routed only): packed h of their own
  p.h2 = take(p.hybrid ? h_rows_tiled * p.hstride * 2 : 0);
  // Y: fp32 rows (ksplit partial-sum planes of them for a split K), or, with
  // bf16 activations and no split, the routed rows as bf16 of w * Y at the
  // pairs' rows -- half the bytes the down GEMM writes and the combine reads,
  // whose loads then need no index; the rounding of w * Y is about 1/8 of a
  // rounding of Y -- and the shared expert's rows, which enter unweighted, in
  // fp32
  p.y_bf16 = c.act_dtype == MOE_BF16 && p.ksplit == 1;
  p.row_w = take(p.y_bf16 ? (size_t)p.P * 4 : 0);
  if (p.y_bf16) {
    p.y = take((size_t)p.P * c.hidden * 2);
    p.ys = take(p.has_shared ? (size_t)T * c.hidden * 4 : 0);
  } else {
    p.y = take((size_t)p.ksplit * rows * c.hidden * 4);
  }
  p.gu_part = take(p.ksplit_gu > 1 ? (size_t)p.ksplit_gu * rows * 2 * p.hstride * 4 : 0);
  p.total = o;
  return p;
}

struct DeviceGuard {
  int prev = -1;
  bool changed = false;
  hipError_t err = hipSuccess;
  explicit DeviceGuard(int dev) {
    err = hipGetDevice(&prev);
    if (err == hipSuccess && prev != dev) {
      err = hipSetDevice(dev);
      changed = err == hipSuccess;
    }
  }
  ~DeviceGuard() {
    if (changed) (void)hipSetDevice(prev);
  }
};

// ---- scratch of the allocation-free entry point -----------------------------
// One static device array per GPU the library runs on (the code object's
// copy on that device), held until the process ends.  In host code `scratch`
// only stands in for the symbol: its device address on each GPU comes from
// hipGetSymbolAddress, taken once per device while that device is current
// (moe_layer_create, the library's set-up call) and kept in g_scratch.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The calling thread's current device must be `device`.
void scratch_setup(int device) {
  if (device < 0 || device >= kMaxDevices) return;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch[device]) return;
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  g_scratch_err[device] = e;
  if (e == hipSuccess) g_scratch[device] = ptr;
  else (void)hipGetLastError();  // a later launch check must not report this failure
}

void* scratch_of(int device, hipError_t* err) {
  if (device < 0 || device >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  *err = g_scratch_err[device];
  return g_scratch[device];
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

int moe_debug_checks(void) { return MOE_DEBUG ? 1 : 0; }

const char* moe_status_str(moe_status_t s) {
  // a C caller may pass any int; reading the enum parameter as such a value
  // would be undefined in C++, so its bytes are read as an int
  static_assert(sizeof(moe_status_t) == sizeof(int), "moe_status_t is int-sized");
  int v;
  memcpy(&v, &s, sizeof v);
  switch (v) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL: return "MOE_ERR_NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE";
    case MOE_ERR_DTYPE: return "MOE_ERR_DTYPE";
    case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

moe_status_t moe_layer_create(const moe_layer_config_t* cfg, int device, moe_layer_t* out) {
  if (!out) return fail(MOE_ERR_NULL, "out handle pointer is NULL");
  *out = nullptr;
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  int n = 0;
  hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess || n == 0)
    return fail(MOE_ERR_DEVICE, "no HIP device available (%s)",
                e != hipSuccess ? hipGetErrorString(e) : "0 devices");
  if (device < 0 || device >= n)
    return fail(MOE_ERR_DEVICE, "device %d out of range (%d devices)", device, n);
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, device);
  if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(MOE_ERR_DEVICE, "device %d is %s; this library is built for gfx950 only", device,
                prop.gcnArchName);
  moe_layer* L = new (std::nothrow) moe_layer;
  if (!L) return fail(MOE_ERR_DEVICE, "out of host memory");
  L->cfg = *cfg;
  L->device = device;
  L->expert_bytes = packed_group_bytes(*cfg, cfg->inter);
  L->shared_bytes = cfg->shared_inter ? packed_group_bytes(*cfg, cfg->shared_inter) : 0;
  DeviceGuard dg(device);
  if (dg.err != hipSuccess) {
    delete L;
    return fail(MOE_ERR_DEVICE, "hipSetDevice: %s", hipGetErrorString(dg.err));
  }
  if (cfg->weight_dtype == MOE_BF16 && cfg->act_dtype == MOE_BF16 &&
      cfg->max_tokens >= kHybridMinTokens) {
    e = hipStreamCreateWithFlags(&L->aux, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&L->fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&L->join, hipEventDisableTiming);
    if (e != hipSuccess) {
      moe_layer_destroy(L);
      return fail(MOE_ERR_DEVICE, "second stream or its events: %s", hipGetErrorString(e));
    }
  }
  scratch_setup(device);
  *out = L;
  return ok();
}

void moe_layer_destroy(moe_layer_t layer) {
  if (!layer) return;
  if (layer->aux || layer->fork || layer->join) {
    // the stream's pending work completes before its resources are released
    DeviceGuard dg(layer->device);
    if (layer->aux) (void)hipStreamDestroy(layer->aux);
    if (layer->fork) (void)hipEventDestroy(layer->fork);
    if (layer->join) (void)hipEventDestroy(layer->join);
  }
  delete layer;
}

size_t moe_layer_packed_bytes(moe_layer_t L) {
  if (!L) return 0;
  return L->expert_bytes * (size_t)L->cfg.num_experts + L->shared_bytes;
}

size_t moe_layer_workspace_bytes(moe_layer_t L, int32_t num_tokens) {
  if (!L || num_tokens <= 0 || num_tokens > L->cfg.max_tokens) return 0;
  return make_plan(*L, num_tokens).total;
}

moe_status_t moe_layer_pack_weights(moe_layer_t L, const moe_weights_t* w, void* packed,
                                    hipStream_t stream) {
  if (!L) return fail(MOE_ERR_NULL, "layer is NULL");
  if (!w || !packed) return fail(MOE_ERR_NULL, "weights or packed buffer is NULL");
  const moe_layer_config_t& c = L->cfg;
  const bool int4 = c.weight_dtype == MOE_INT4_G32;
  const bool sh = c.shared_inter > 0;
  if (!w->w_gate || !w->w_up || !w->w_down || (sh && (!w->s_gate || !w->s_up || !w->s_down)))
    return fail(MOE_ERR_NULL, "a weight pointer is NULL");
  if (int4 && (!w->sc_gate || !w->sc_up || !w->sc_down ||
               (sh && (!w->sc_s_gate || !w->sc_s_up || !w->sc_s_down))))
    return fail(MOE_ERR_NULL, "an INT4 scale pointer is NULL");
  const void* ptrs[] = {w->w_gate, w->w_up, w->w_down, packed};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(MOE_ERR_ALIGN, "weight pointers must be 16-byte aligned");
  DeviceGuard dg(L->device);
  if (dg.err != hipSuccess) return fail(MOE_ERR_DEVICE, "hipSetDevice: %s", hipGetErrorString(dg.err));

  const int H = c.hidden, I = c.inter, Is = c.shared_inter, E = c.num_experts;
  uint8_t* dst = static_cast<uint8_t*>(packed);
  hipError_t e = hipSuccess;
  auto pack_group = [&](const void* g, const void* u, const void* d, const void* sg,
                        const void* su, const void* sd, int width, int batch, uint8_t* base,
                        size_t group_bytes) -> hipError_t {
    hipError_t r;
    const size_t wh = (size_t)width * H;
    if (!int4) {
      r = moe::launch_pack_bf16((const uint16_t*)g, (const uint16_t*)u, 2, 2, width, H, batch, wh,
                                base, group_bytes, stream);
      if (r != hipSuccess) return r;
      return moe::launch_pack_bf16((const uint16_t*)d, (const uint16_t*)d, 1, 4, H, width, batch,
                                   wh, base + 2 * wh * 2, group_bytes, stream);
    }
    r = moe::launch_pack_int4((const uint8_t*)g, (const uint8_t*)u, (const uint16_t*)sg,
                              (const uint16_t*)su, 2, 2, width, H, batch, wh / 2, wh / 32, base,
                              base + wh, group_bytes, stream);
    if (r != hipSuccess) return r;
    uint8_t* dbase = base + wh + wh / 8;
    return moe::launch_pack_int4((const uint8_t*)d, (const uint8_t*)d, (const uint16_t*)sd,
                                 (const uint16_t*)sd, 1, 4, H, width, batch, wh / 2, wh / 32,
                                 dbase, dbase + wh / 2, group_bytes, stream);
  };
  e = pack_group(w->w_gate, w->w_up, w->w_down, w->sc_gate, w->sc_up, w->sc_down, I, E, dst,
                 L->expert_bytes);
  if (e == hipSuccess && sh)
    e = pack_group(w->s_gate, w->s_up, w->s_down, w->sc_s_gate, w->sc_s_up, w->sc_s_down, Is, 1,
                   dst + L->expert_bytes * E, L->shared_bytes);
  if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "pack launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

namespace {

moe_status_t forward_impl(moe_layer_t L, int32_t T, const void* x, const void* router_w,
                          const float* router_bias, const void* packed, void* out,
                          void* workspace, size_t workspace_bytes, moe_route_t* route,
                          hipStream_t stream, hipEvent_t* ev) {
  if (!L) return fail(MOE_ERR_NULL, "layer is NULL");
  const moe_layer_config_t& c = L->cfg;
  if (T < 0 || T > c.max_tokens)
    return fail(MOE_ERR_SHAPE, "num_tokens %d outside [0, max_tokens=%d]", T, c.max_tokens);
  if (T == 0) {
    if (route) memset(route, 0, sizeof *route);
    return ok();
  }
  if (!x || !router_w || !packed || !out || !workspace)
    return fail(MOE_ERR_NULL, "x, router_w, packed, out and workspace must be non-NULL");
  const void* al[] = {x, router_w, packed, out, workspace};
  for (const void* p : al)
    if (!aligned16(p)) return fail(MOE_ERR_ALIGN, "device pointers must be 16-byte aligned");
  if (router_bias && (reinterpret_cast<uintptr_t>(router_bias) & 3u))
    return fail(MOE_ERR_ALIGN, "router_bias must be 4-byte aligned");
  if (out == x) return fail(MOE_ERR_SHAPE, "out may not alias x");
  const Plan p = make_plan(*L, T);
  if (workspace_bytes < p.total)
    return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, p.total);
  DeviceGuard dg(L->device);
  if (dg.err != hipSuccess) return fail(MOE_ERR_DEVICE, "hipSetDevice: %s", hipGetErrorString(dg.err));

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* part = reinterpret_cast<float*>(ws + p.part);
  int32_t* idx = reinterpret_cast<int32_t*>(ws + p.idx);
  float* wts = reinterpret_cast<float*>(ws + p.w);
  float* gap = reinterpret_cast<float*>(ws + p.gap);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + p.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + p.offsets);
  int32_t* perm = reinterpret_cast<int32_t*>(ws + p.perm);
  int32_t* inv = reinterpret_cast<int32_t*>(ws + p.inv);
  int32_t* row_tok = reinterpret_cast<int32_t*>(ws + p.row_tok);
  int32_t* tiles = reinterpret_cast<int32_t*>(ws + p.tiles);
  int32_t* ntiles = reinterpret_cast<int32_t*>(ws + p.ntiles);
  float* h = reinterpret_cast<float*>(ws + p.h);
  float* y = reinterpret_cast<float*>(ws + p.y);
  float* row_w = p.y_bf16 ? reinterpret_cast<float*>(ws + p.row_w) : nullptr;
  const bool f32 = c.act_dtype == MOE_F32;
  const bool int4 = c.weight_dtype == MOE_INT4_G32;
  const int E = c.num_experts, H = c.hidden, k = c.top_k;

  // stage boundary i (a NULL entry of the caller's array: not recorded)
  auto mark = [&](int i) -> hipError_t {
    return ev && ev[i] ? hipEventRecord(ev[i], stream) : hipSuccess;
  };
  // up to 1024 tokens, top-k and dispatch run as one launch (the router stage
  // then ends after the logits); larger batches use the multi-workgroup
  // dispatch after a separate top-k
  int32_t* done = reinterpret_cast<int32_t*>(ws + p.done);
  int32_t* dbg = reinterpret_cast<int32_t*>(ws + p.dbg);
  hipError_t e = mark(0);
  if (e == hipSuccess)
    e = moe::launch_router_logits(f32, x, static_cast<const uint16_t*>(router_w), part, T, H, E,
                                  p.ks, p.large_dispatch ? nullptr : done, dbg, stream);
  if (p.large_dispatch) {
    if (e == hipSuccess)
      e = moe::launch_router_topk(part, p.ks, router_bias, c.bias_mode, T, E, k, c.score,
                                  c.renormalize, c.routed_scale, idx, wts, gap, stream);
    if (e == hipSuccess) e = mark(1);
    if (e == hipSuccess)
      e = moe::launch_dispatch_large(idx, T, k, E, p.has_shared, 16 * p.tg,
                                     reinterpret_cast<int32_t*>(ws + p.blk_hist), counts, offsets,
                                     perm, inv, row_tok, tiles, ntiles, wts, row_w, dbg, stream);
  } else {
    if (e == hipSuccess) e = mark(1);
    const moe::TileLists tl{16 * p.tg, p.hot, 16 * p.tg2, tiles, ntiles,
                            p.hybrid ? reinterpret_cast<int32_t*>(ws + p.tiles2) : nullptr,
                            p.hybrid ? reinterpret_cast<int32_t*>(ws + p.ntiles2) : nullptr};
    if (e == hipSuccess)
      e = moe::launch_topk_dispatch(part, p.ks, router_bias, c.bias_mode, T, E, k, c.score,
                                    c.renormalize, c.routed_scale, idx, wts, gap, done,
                                    p.has_shared, tl, counts, offsets, perm, inv, row_tok, row_w,
                                    dbg, stream);
  }
  if (e == hipSuccess) e = mark(2);
  moe::GemmGeom g{};
  g.H = H;
  g.I = c.inter;
  g.Is = c.shared_inter;
  g.E = E;
  g.T = T;
  g.expert_bytes = L->expert_bytes;
  g.packed = static_cast<const uint8_t*>(packed);
  g.tiles = tiles;
  g.ntiles = ntiles;
  g.offsets = offsets;
  g.counts = counts;
  g.max_tiles = p.max_tiles;
  g.tg = p.tg;
  // the shared group's tiles close list 1
  g.shared_tiles = p.has_shared ? (T + 16 * p.tg - 1) / (16 * p.tg) : 0;
  g.limit = c.swiglu_limit;
  g.limit_shared = c.swiglu_limit_shared;
  g.ksplit = p.ksplit;
  g.y_plane = (size_t)(p.P + (p.has_shared ? T : 0)) * H;
  g.ksplit_gu = p.ksplit_gu;
  g.gu_part = p.ksplit_gu > 1 ? reinterpret_cast<float*>(ws + p.gu_part) : nullptr;
  g.gu_plane = (size_t)(p.P + (p.has_shared ? T : 0)) * 2 * p.hstride;
  g.dbg = dbg;
  g.y_bf16 = p.y_bf16;
  g.yb = p.y_bf16 ? reinterpret_cast<uint16_t*>(ws + p.y) : nullptr;
  g.ys = p.y_bf16 && p.has_shared ? reinterpret_cast<float*>(ws + p.ys) : nullptr;
  g.row_w = row_w;
  g.perm = perm;
  moe::GemmGeom g2 = g;  // the hybrid's LDS-tiled groups
  g2.tiles = reinterpret_cast<int32_t*>(ws + p.tiles2);
  g2.ntiles = reinterpret_cast<int32_t*>(ws + p.ntiles2);
  g2.max_tiles = p.max_tiles2;
  g2.tg = p.tg2;
  g2.shared_tiles = 0;
  if (p.tiled) {
    uint16_t* hb = reinterpret_cast<uint16_t*>(h);
    uint16_t* hl = reinterpret_cast<uint16_t*>(ws + p.h_lo);
    if (e == hipSuccess)
      e = moe::launch_gateup_tiled(g, static_cast<const uint16_t*>(x), row_tok, hb, hl,
                                   p.hstride, stream);
    if (e == hipSuccess && p.ksplit_gu > 1)
      e = moe::launch_gateup_reduce(g, p.P + (p.has_shared ? T : 0), hb, hl, p.hstride, stream);
    if (e == hipSuccess) e = mark(3);
    if (e == hipSuccess) e = moe::launch_down_tiled(g, hb, hl, p.hstride, y, stream);
  } else {
    uint16_t* hl = reinterpret_cast<uint16_t*>(ws + p.h_lo);
    uint16_t* h2 = reinterpret_cast<uint16_t*>(ws + p.h2);
    // The hot experts' LDS-tiled gate/up and down -- few, long-running
    // workgroups -- go to the handle's second stream, forked after the
    // dispatch and joined before the combine, where they overlap the
    // streaming GEMMs on the caller's stream (they write h2 and their own rows
    // of Y only).  The fork record, the second stream's wait on it, the
    // launches there and the join record are enqueued under the handle's
    // lock, so a concurrent forward's record cannot come between them; the
    // caller's stream then waits on the join event (if another forward has
    // recorded it since, that record is later on the in-order second stream,
    // so the wait still covers this call's work).
    const bool fork_join = p.hybrid && L->aux;
    bool joined = false;  // this call recorded the join event
    if (e == hipSuccess && p.hybrid) {
      std::unique_lock<std::mutex> lk(L->aux_mu, std::defer_lock);
      hipStream_t s2 = stream;
      if (fork_join) {
        lk.lock();
        e = hipEventRecord(L->fork, stream);
        if (e == hipSuccess) e = hipStreamWaitEvent(L->aux, L->fork, 0);
        s2 = L->aux;
      }
      if (e == hipSuccess)
        e = moe::launch_gateup_tiled(g2, static_cast<const uint16_t*>(x), row_tok, h2, nullptr,
                                     p.hstride, s2);
      if (e == hipSuccess) e = moe::launch_down_tiled(g2, h2, nullptr, p.hstride, y, s2);
      if (fork_join) {  // also after a failed launch: the caller's stream must not run ahead
        hipError_t r = hipEventRecord(L->join, s2);
        joined = r == hipSuccess;
        if (e == hipSuccess) e = r;
      }
    }
    if (e == hipSuccess)
      e = moe::launch_gateup(g, int4, f32, x, row_tok, h, hl, p.hstride, stream);
    if (e == hipSuccess) e = mark(3);
    if (e == hipSuccess) e = moe::launch_down(g, int4, f32, h, hl, p.hstride, y, stream);
    if (joined) {
      hipError_t r = hipStreamWaitEvent(stream, L->join, 0);
      if (e == hipSuccess) e = r;
    }
  }
  if (e == hipSuccess) e = mark(4);
  if (e == hipSuccess)
    e = moe::launch_combine(f32, y, H, inv, wts, k, p.P, p.has_shared, out, T, p.ksplit,
                            g.y_plane, g.yb, g.ys, dbg, stream);
  if (e == hipSuccess) e = mark(5);
  if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
  if (route) {
    route->topk_idx = idx;
    route->topk_w = wts;
    route->topk_gap = gap;
    route->expert_counts = counts;
    route->expert_offsets = offsets;
    route->perm = perm;
    route->inv = inv;
    route->debug_flag = MOE_DEBUG ? dbg : nullptr;
  }
  return ok();
}

}  // namespace

extern "C" {

moe_status_t moe_layer_forward(moe_layer_t L, int32_t T, const void* x, const void* router_w,
                               const float* router_bias, const void* packed, void* out,
                               void* workspace, size_t workspace_bytes, moe_route_t* route,
                               hipStream_t stream) {
  return forward_impl(L, T, x, router_w, router_bias, packed, out, workspace, workspace_bytes,
                      route, stream, nullptr);
}

moe_status_t moe_layer_forward_noalloc(moe_layer_t L, int32_t T, const void* x,
                                       const void* router_w, const float* router_bias,
                                       const void* packed, void* out, moe_route_t* route,
                                       hipStream_t stream) {
  if (!L) return fail(MOE_ERR_NULL, "layer is NULL");
  if (T > 0 && T <= L->cfg.max_tokens) {
    const size_t need = make_plan(*L, T).total;
    if (need > MOE_NOALLOC_SCRATCH_BYTES)
      return fail(MOE_ERR_WORKSPACE,
                  "num_tokens %d needs %zu bytes of scratch; the allocation-free entry point has "
                  "%zu per device (call moe_layer_forward with a workspace instead)",
                  T, need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  }
  hipError_t err = hipSuccess;
  void* ws = scratch_of(L->device, &err);
  if (!ws)
    return fail(MOE_ERR_DEVICE, "no scratch address for device %d: %s", L->device,
                hipGetErrorString(err));
  return forward_impl(L, T, x, router_w, router_bias, packed, out, ws,
                      MOE_NOALLOC_SCRATCH_BYTES, route, stream, nullptr);
}

moe_status_t moe_layer_forward_timed(moe_layer_t L, int32_t T, const void* x,
                                     const void* router_w, const float* router_bias,
                                     const void* packed, void* out, void* workspace,
                                     size_t workspace_bytes, moe_route_t* route,
                                     hipStream_t stream, hipEvent_t* stage_events) {
  if (!stage_events) return fail(MOE_ERR_NULL, "stage_events is NULL");
  return forward_impl(L, T, x, router_w, router_bias, packed, out, workspace, workspace_bytes,
                      route, stream, stage_events);
}

}  // extern "C"
