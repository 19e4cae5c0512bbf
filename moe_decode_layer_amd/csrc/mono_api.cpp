/*
 * libmonolayer host side: the C ABI of include/mono.h.
 *
 * Every call checks its arguments on the host and, on any failure, enqueues
 * nothing and lists every failed check (the refusal style of the SGLang mono
 * page, "Modifications": unsupported deployments are refused with every reason
 * listed, never silently degraded). The calls only enqueue kernels on the
 * caller's stream: no synchronisation and no allocation on the hot path (the
 * vLLM GLM-5 page, "Validation": no host syncs in the forward path).
 */
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>
#include <utility>
#include <unordered_map>
#include <mutex>
#include <atomic>

#include "mono_internal.h"

namespace mono {
int launch_debug(uint32_t* ctl, uint32_t spin, uint32_t fwg, uint32_t fph, void* stream);
int launch_trace(uint32_t* ctl, uint32_t on, void* stream);
int launch_head(int act, int rows, int H, float eps_hc, float eps_norm, const void* state,
                const float* w_head, const float* head_scale, const float* head_base,
                const void* w_norm, float* pre, void* x, void* norm, void* stream);
}

namespace {
thread_local std::string g_error;
}  // namespace

void mono::set_last_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
}

using namespace mono;

namespace {

struct Check {
  std::string msg;
  int code = MONO_OK;
  void fail(int c, const char* fmt, ...) {
    char buf[256];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    if (!msg.empty()) msg += "; ";
    msg += buf;
    if (code == MONO_OK || c == MONO_E_INVAL) code = c;
  }
  void req(bool ok, const char* what) {
    if (!ok) fail(MONO_E_INVAL, "%s", what);
  }
  void ptr(const void* p, const char* name, size_t align = 4) {
    if (!p)
      fail(MONO_E_INVAL, "%s is NULL", name);
    else if (reinterpret_cast<uintptr_t>(p) % align)
      fail(MONO_E_INVAL, "%s is not %zu-byte aligned", name, align);
  }
  mono_status done() {
    g_error = msg;
    return (mono_status)code;
  }
};

bool act_ok(int a) { return a == MONO_F32 || a == MONO_BF16; }
bool fmt_ok(int f) { return f >= MONO_F32 && f <= MONO_MXFP4; }

void check_shape(Check& c, const mono_shape* s) {
  if (!s) {
    c.fail(MONO_E_INVAL, "shape is NULL");
    return;
  }
  if (s->rows < 0 || s->rows > kMaxRows) c.fail(MONO_E_INVAL, "rows=%d not in [0, %d]", s->rows, kMaxRows);
  if (s->n_streams != 4) c.fail(MONO_E_INVAL, "n_streams=%d (must be 4)", s->n_streams);
  if (s->hidden <= 0 || s->hidden % 64) c.fail(MONO_E_INVAL, "hidden=%d (must be a positive multiple of 64)", s->hidden);
  if (s->inter <= 0 || s->inter % 32) c.fail(MONO_E_INVAL, "inter=%d (must be a positive multiple of 32)", s->inter);
  if (s->shared_inter < 0 || s->shared_inter % 32)
    c.fail(MONO_E_INVAL, "shared_inter=%d (must be a non-negative multiple of 32)", s->shared_inter);
  if (s->top_k < 1 || s->top_k > kMaxTopK) c.fail(MONO_E_INVAL, "top_k=%d not in [1, %d]", s->top_k, kMaxTopK);
  if (s->n_experts < s->top_k || s->n_experts > kMaxExperts)
    c.fail(MONO_E_INVAL, "n_experts=%d not in [top_k, %d]", s->n_experts, kMaxExperts);
  if (!act_ok(s->act)) c.fail(MONO_E_INVAL, "act=%d (must be MONO_F32 or MONO_BF16)", (int)s->act);
  if (s->sinkhorn_iters < 0 || s->sinkhorn_iters > 1000)
    c.fail(MONO_E_INVAL, "sinkhorn_iters=%d not in [0, 1000]", s->sinkhorn_iters);
  if (!std::isfinite(s->routed_scale)) c.fail(MONO_E_INVAL, "routed_scale is not finite");
  if (!(s->eps_hc >= 0.0f) || !(s->eps_norm >= 0.0f)) c.fail(MONO_E_INVAL, "eps_hc / eps_norm must be >= 0");
  if (s->act_quant != MONO_AQ_NONE && s->act_quant != MONO_AQ_MXFP8)
    c.fail(MONO_E_INVAL, "act_quant=%d (must be MONO_AQ_NONE or MONO_AQ_MXFP8)", s->act_quant);
  if (act_ok(s->act) && s->rows > 0 && s->hidden > 0) {
    const size_t ab = s->act == MONO_F32 ? 4 : 2;
    const size_t wide = (size_t)(s->inter > s->shared_inter ? s->inter : s->shared_inter);
    if ((size_t)s->rows * wide * ab > (size_t)kLdsHidBytes)
      c.fail(MONO_E_UNSUPPORTED, "rows*max(inter, shared_inter)*%zu exceeds the %d-byte hidden-row buffer",
             ab, kLdsHidBytes);
    if (wide * ab > 16384)
      c.fail(MONO_E_UNSUPPORTED, "max(inter, shared_inter)*%zu exceeds 16384 bytes per hidden row", ab);
    if ((size_t)(s->rows + 1) * s->hidden * ab > (size_t)kLdsActBytes)
      c.fail(MONO_E_UNSUPPORTED, "(rows + 1)*hidden*%zu exceeds the %d-byte activation buffer", ab,
             kLdsActBytes);
  }
}

void check_formats(Check& c, const mono_shape* s, const mono_layer* L, bool routed, bool shared) {
  if (!s || !L || !act_ok(s->act)) return;
  auto one = [&](const mono_experts& x, const char* name) {
    if (!fmt_ok(x.fmt)) {
      c.fail(MONO_E_INVAL, "%s.fmt=%d unknown", name, (int)x.fmt);
      return;
    }
    if (s->act == MONO_F32 && x.fmt != MONO_F32)
      c.fail(MONO_E_UNSUPPORTED, "%s.fmt must be MONO_F32 when act is MONO_F32", name);
    if (s->act == MONO_BF16 && x.fmt == MONO_F32)
      c.fail(MONO_E_UNSUPPORTED, "%s.fmt MONO_F32 with bf16 activations is not supported", name);
  };
  if (routed) one(L->routed, "routed");
  if (shared && s->shared_inter > 0) one(L->shared, "shared");
  if (routed && s->act_quant == MONO_AQ_MXFP8 && L->routed.fmt != MONO_MXFP4)
    c.fail(MONO_E_UNSUPPORTED, "act_quant MONO_AQ_MXFP8 needs routed.fmt MONO_MXFP4 (routed.fmt=%d)",
           (int)L->routed.fmt);
}

void check_experts(Check& c, const mono_shape* s, const mono_experts& x, const char* name,
                   bool gateup, bool down) {
  char b[64];
  const bool q = x.fmt == MONO_Q8_0 || x.fmt == MONO_MXFP4;
  if (gateup) {
    snprintf(b, sizeof b, "%s.gate", name); c.ptr(x.gate, b, 16);
    snprintf(b, sizeof b, "%s.up", name); c.ptr(x.up, b, 16);
    if (q) {
      snprintf(b, sizeof b, "%s.gate_s", name); c.ptr(x.gate_s, b, x.fmt == MONO_Q8_0 ? 2 : 1);
      snprintf(b, sizeof b, "%s.up_s", name); c.ptr(x.up_s, b, x.fmt == MONO_Q8_0 ? 2 : 1);
    }
  }
  if (down) {
    snprintf(b, sizeof b, "%s.down", name); c.ptr(x.down, b, 16);
    if (q) { snprintf(b, sizeof b, "%s.down_s", name); c.ptr(x.down_s, b, x.fmt == MONO_Q8_0 ? 2 : 1); }
  }
  (void)s;
}

size_t act_align(const mono_shape* s) { return 16; }

/* Device-dependent limits: the persistent grid and the down-phase slice buffer. */
int device_grid(Check& c, const mono_shape* s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    c.fail(MONO_E_DEVICE, "no HIP device");
    return 0;
  }
  static int cached[64] = {0};
  int g = dev < 64 ? cached[dev] : 0;
  if (!g) {
    g = grid_size_for_device(dev);
    if (dev < 64) cached[dev] = g;
  }
  if (g <= 0) {
    c.fail(MONO_E_DEVICE, "cannot read the compute-unit count of device %d", dev);
    return 0;
  }
  const int hs = (s->hidden + g - 1) / g;
  const size_t need = (size_t)hs * s->rows * (s->top_k + 2) * 4 + (size_t)hs * s->rows * 4 * 4 +
                      (size_t)hs * s->rows * kNCarry * 4;
  if (need > (size_t)(kLdsActBytes - kLdsHidBytes))
    c.fail(MONO_E_UNSUPPORTED, "hidden slice of %d rows x %d rows needs %zu bytes of LDS (max %d)",
           hs, s->rows, need, kLdsActBytes - kLdsHidBytes);
  return g;
}

/* The fused launch exchanges values between all of its workgroups, so all of them must be
 * resident at once: one per compute unit needs an occupancy of at least one (its LDS and
 * registers), read once per device and kernel instantiation. */
void check_resident(Check& c, const mono_shape* s, int rf, int sf) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return; /* reported by device_grid */
  static int cached[64][2][4][4][2]; /* occupancy + 1; 0 = not read yet */
  const int a = s->act == MONO_F32 ? 0 : 1, m = s->rows > 1 ? 1 : 0;
  int occ;
  if (dev < 64 && rf >= 0 && rf < 4 && sf >= 0 && sf < 4 && cached[dev][a][rf][sf][m] != 0) {
    occ = cached[dev][a][rf][sf][m] - 1;
  } else {
    occ = max_active_persistent(s->act, rf, sf, s->rows);
    if (dev < 64 && rf >= 0 && rf < 4 && sf >= 0 && sf < 4) cached[dev][a][rf][sf][m] = occ + 1;
  }
  if (occ < 1)
    c.fail(MONO_E_UNSUPPORTED,
           "the fused launch needs one resident workgroup per compute unit, device %d holds %d",
           dev, occ);
}

Params base_params(const mono_shape* s, const mono_layer* L, void* ws, int grid) {
  Params p = {};
  p.R = s->rows; p.H = s->hidden; p.E = s->n_experts; p.K = s->top_k; p.I = s->inter;
  p.Is = s->shared_inter; p.iters = s->sinkhorn_iters; p.nslice = grid;
  p.rho = s->routed_scale; p.eps_hc = s->eps_hc; p.eps_norm = s->eps_norm;
  p.aq8 = s->act_quant == MONO_AQ_MXFP8 ? 1 : 0;
  if (L) {
    p.w_mix = L->w_mix; p.hc_scale = L->hc_scale; p.hc_base = L->hc_base; p.w_norm = L->w_norm;
    p.w_router = L->w_router; p.bias = L->bias;
    auto m = [](const mono_experts& x) {
      Mat r;
      r.fmt = x.fmt;
      r.gate = static_cast<const uint8_t*>(x.gate);
      r.up = static_cast<const uint8_t*>(x.up);
      r.down = static_cast<const uint8_t*>(x.down);
      r.gate_s = static_cast<const uint8_t*>(x.gate_s);
      r.up_s = static_cast<const uint8_t*>(x.up_s);
      r.down_s = static_cast<const uint8_t*>(x.down_s);
      return r;
    };
    p.routed = m(L->routed);
    p.shared = m(L->shared);
  }
  const WsLayout W = ws_layout(*s);
  uint8_t* b = static_cast<uint8_t*>(ws);
  p.ctl = reinterpret_cast<uint32_t*>(b + W.ctl);
  p.mix_part = reinterpret_cast<uint64_t*>(b + W.mix_part);
  p.carry_part = reinterpret_cast<float*>(b + W.carry_part);
  p.pre_done = reinterpret_cast<uint64_t*>(b + W.pre_done);
  p.y_part = reinterpret_cast<uint64_t*>(b + W.y_part);
  p.lgp = reinterpret_cast<uint64_t*>(b + W.lgp);
  p.trace = reinterpret_cast<uint64_t*>(b + W.trace);
  p.h_routed = b + W.h_routed;
  p.h_shared = b + W.h_shared;
  return p;
}

int sfmt_of(const mono_shape* s, const mono_layer* L) {
  return (s->shared_inter > 0) ? (int)L->shared.fmt : (int)L->routed.fmt;
}

mono_status enqueue(Kernel k, const Params& p, const mono_shape* s, int rfmt, int sfmt, int grid,
                    void* stream, const char* what) {
  const int rc = launch(k, p, s->act, rfmt, sfmt, grid, stream);
  if (rc != 0) {
    g_error = std::string(what) + ": " + hipGetErrorString((hipError_t)rc);
    return MONO_E_DEVICE;
  }
  return MONO_OK;
}

}  // namespace

extern "C" {

const char* mono_last_error(void) { return g_error.c_str(); }

int mono_grid_size(void) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  return grid_size_for_device(dev);
}

size_t mono_workspace_bytes(const mono_shape* shape) {
  Check c;
  check_shape(c, shape);
  if (c.code != MONO_OK) {
    c.done();
    return 0;
  }
  g_error.clear();
  return ws_layout(*shape).total;
}

/* Race-shaker settings per workspace (host side; read by every fused launch on it). */
static std::mutex g_jitter_mu;
static std::unordered_map<const void*, std::pair<uint32_t, uint32_t>> g_jitter;
static std::atomic<int> g_jitter_n{0};

static void jitter_of(const void* ws, uint32_t& max_ticks, uint32_t& seed) {
  max_ticks = seed = 0;
  if (g_jitter_n.load(std::memory_order_relaxed) == 0) return;
  std::lock_guard<std::mutex> lk(g_jitter_mu);
  const auto it = g_jitter.find(ws);
  if (it != g_jitter.end()) {
    max_ticks = it->second.first;
    seed = it->second.second;
  }
}

static void jitter_set(const void* ws, uint32_t max_ticks, uint32_t seed) {
  std::lock_guard<std::mutex> lk(g_jitter_mu);
  if (max_ticks)
    g_jitter[ws] = std::make_pair(max_ticks, seed);
  else
    g_jitter.erase(ws);
  g_jitter_n.store((int)g_jitter.size(), std::memory_order_relaxed);
}

mono_status mono_workspace_init(void* ws, const mono_shape* shape, void* stream) {
  Check c;
  check_shape(c, shape);
  c.ptr(ws, "ws", 256);
  if (c.code != MONO_OK) return c.done();
  Params p = base_params(shape, nullptr, ws, 1);
  {
    const WsLayout W = ws_layout(*shape);
    p.tag_words = (W.lgp_end - W.carry_part) / 8;
  }
  jitter_set(ws, 0, 0);
  const int rc = launch(K_WS_INIT, p, shape->act, 0, 0, 1, stream);
  if (rc != 0) {
    g_error = std::string("workspace init: ") + hipGetErrorString((hipError_t)rc);
    return MONO_E_DEVICE;
  }
  g_error.clear();
  return MONO_OK;
}

mono_status mono_workspace_set_debug(void* ws, uint32_t spin_limit_ticks, int32_t fault_wg,
                                     int32_t fault_phase, void* stream) {
  Check c;
  c.ptr(ws, "ws", 256);
  if (c.code != MONO_OK) return c.done();
  const int rc = launch_debug(static_cast<uint32_t*>(ws), spin_limit_ticks, (uint32_t)fault_wg,
                              (uint32_t)fault_phase, stream);
  if (rc != 0) {
    g_error = std::string("set_debug: ") + hipGetErrorString((hipError_t)rc);
    return MONO_E_DEVICE;
  }
  g_error.clear();
  return MONO_OK;
}

mono_status mono_workspace_set_trace(void* ws, int enable, void* stream) {
  Check c;
  c.ptr(ws, "ws", 256);
  if (c.code != MONO_OK) return c.done();
  const int rc = launch_trace(static_cast<uint32_t*>(ws), enable ? 1u : 0u, stream);
  if (rc != 0) {
    g_error = std::string("set_trace: ") + hipGetErrorString((hipError_t)rc);
    return MONO_E_DEVICE;
  }
  g_error.clear();
  return MONO_OK;
}

mono_status mono_workspace_set_jitter(void* ws, uint32_t max_ticks, uint32_t seed) {
  Check c;
  c.ptr(ws, "ws", 256);
  if (max_ticks > MONO_JITTER_MAX_TICKS)
    c.fail(MONO_E_INVAL, "set_jitter: max_ticks %u exceeds MONO_JITTER_MAX_TICKS (%u)", max_ticks,
           (unsigned)MONO_JITTER_MAX_TICKS);
  if (c.code != MONO_OK) return c.done();
  jitter_set(ws, max_ticks, seed);
  g_error.clear();
  return MONO_OK;
}

mono_status mono_workspace_poll(const void* ws, uint32_t err[4], void* stream) {
  Check c;
  c.ptr(ws, "ws", 256);
  c.ptr(err, "err");
  if (c.code != MONO_OK) return c.done();
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e == hipSuccess)
    e = hipMemcpy(err, static_cast<const uint32_t*>(ws) + CTL_ERR, 16, hipMemcpyDeviceToHost);
  if (e != hipSuccess) {
    g_error = std::string("poll: ") + hipGetErrorString(e);
    return MONO_E_DEVICE;
  }
  g_error.clear();
  return err[0] ? MONO_E_TIMEOUT : MONO_OK;
}

mono_status mono_workspace_tensor(const mono_shape* shape, void* ws, mono_tensor which, void** ptr,
                                  size_t* bytes) {
  Check c;
  check_shape(c, shape);
  c.ptr(ws, "ws", 256);
  c.ptr(ptr, "ptr", 1);
  if (c.code != MONO_OK) return c.done();
  const WsLayout W = ws_layout(*shape);
  const size_t R = shape->rows, H = shape->hidden, ab = shape->act == MONO_F32 ? 4 : 2;
  size_t off = 0, n = 0;
  switch (which) {
    case MONO_T_MIXES: off = W.mixes; n = R * kNMix * 4; break;
    case MONO_T_PRE: off = W.pre; n = R * 16; break;
    case MONO_T_POST: off = W.post; n = R * 16; break;
    case MONO_T_COMB: off = W.comb; n = R * 64; break;
    case MONO_T_X: off = W.x; n = R * H * ab; break;
    case MONO_T_NORM: off = W.norm; n = R * H * ab; break;
    case MONO_T_LOGITS: off = W.logits; n = R * shape->n_experts * 4; break;
    case MONO_T_IDX: off = W.idx; n = R * shape->top_k * 4; break;
    case MONO_T_WEIGHTS: off = W.weights; n = R * shape->top_k * 4; break;
    case MONO_T_H_ROUTED: off = W.h_routed; n = R * shape->top_k * shape->inter * ab * 2; break;
    case MONO_T_H_SHARED: off = W.h_shared; n = R * shape->shared_inter * ab * 2; break;
    case MONO_T_SHARED: off = W.shared; n = R * H * ab; break;
    case MONO_T_ROUTED: off = W.routed; n = R * H * 4; break;
    case MONO_T_BLOCK: off = W.block; n = R * H * ab; break;
    case MONO_T_CARRY: off = W.carry; n = R * kNCarry * 4; break;
    case MONO_T_TRACE: off = W.trace; n = (size_t)kMaxGrid * kTraceSlots * 8; break;
    default:
      c.fail(MONO_E_INVAL, "unknown tensor %d", (int)which);
      return c.done();
  }
  *ptr = static_cast<uint8_t*>(ws) + off;
  if (bytes) *bytes = n;
  g_error.clear();
  return MONO_OK;
}

mono_status mono_hc_mix_collapse(const mono_shape* shape, const void* state,
                                 const mono_layer* layer, const float* carry_in, float* mixes,
                                 float* pre, float* post, float* comb, void* x, void* norm,
                                 void* ws, void* stream) {
  Check c;
  check_shape(c, shape);
  c.req(layer != nullptr, "layer is NULL");
  if (c.code == MONO_OK) {
    c.ptr(state, "state", 16);
    if (!carry_in) c.ptr(layer->w_mix, "layer.w_mix", 16);
    else c.ptr(carry_in, "carry_in");
    c.ptr(layer->hc_scale, "layer.hc_scale");
    c.ptr(layer->hc_base, "layer.hc_base");
    c.ptr(layer->w_norm, "layer.w_norm", 16);
    c.ptr(pre, "pre"); c.ptr(post, "post"); c.ptr(comb, "comb"); c.ptr(norm, "norm", 16);
    if (mixes) c.ptr(mixes, "mixes");
    if (x) c.ptr(x, "x", 16);
  }
  c.ptr(ws, "ws", 256);
  if (c.code != MONO_OK || shape->rows == 0) return c.done();
  const int grid = device_grid(c, shape);
  if (c.code != MONO_OK) return c.done();
  Params p = base_params(shape, layer, ws, grid);
  p.state = state; p.carry_in = carry_in;
  p.mixes = mixes; p.pre = pre; p.post = post; p.comb = comb; p.x = x; p.norm = norm;
  mono_status st = MONO_OK;
  if (!carry_in) st = enqueue(K_MIX_PARTIALS, p, shape, 0, 0, grid, stream, "mix partials");
  if (st == MONO_OK) st = enqueue(K_HC_PRE, p, shape, 0, 0, 1, stream, "hc pre");
  if (st == MONO_OK) g_error.clear();
  return st;
}

mono_status mono_router_select(const mono_shape* shape, const void* norm,
                               const mono_layer* layer, float* logits, int32_t* idx,
                               float* weights, void* ws, void* stream) {
  Check c;
  check_shape(c, shape);
  c.req(layer != nullptr, "layer is NULL");
  if (c.code == MONO_OK) {
    c.ptr(norm, "norm", 16);
    c.ptr(layer->w_router, "layer.w_router", 16);
    c.ptr(layer->bias, "layer.bias");
    c.ptr(idx, "idx"); c.ptr(weights, "weights");
    if (logits) c.ptr(logits, "logits");
  }
  c.ptr(ws, "ws", 256);
  if (c.code != MONO_OK || shape->rows == 0) return c.done();
  const int grid = device_grid(c, shape);
  if (c.code != MONO_OK) return c.done();
  Params p = base_params(shape, layer, ws, grid);
  const WsLayout W = ws_layout(*shape);
  p.norm_in = norm;
  p.logits = logits ? logits : reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + W.logits);
  p.idx = idx; p.weights = weights;
  mono_status st = enqueue(K_ROUTER_LOGITS, p, shape, 0, 0, grid, stream, "router logits");
  if (st == MONO_OK) st = enqueue(K_SELECT, p, shape, 0, 0, 1, stream, "select");
  if (st == MONO_OK) g_error.clear();
  return st;
}

mono_status mono_moe_experts(const mono_shape* shape, const void* norm, const int32_t* idx,
                             const float* weights, const mono_layer* layer, void* shared_out,
                             float* routed_out, void* block, void* ws, void* stream) {
  Check c;
  check_shape(c, shape);
  c.req(layer != nullptr, "layer is NULL");
  if (c.code == MONO_OK) {
    check_formats(c, shape, layer, true, true);
    c.ptr(norm, "norm", 16); c.ptr(idx, "idx"); c.ptr(weights, "weights"); c.ptr(block, "block", 4);
    check_experts(c, shape, layer->routed, "routed", true, true);
    if (shape->shared_inter > 0) check_experts(c, shape, layer->shared, "shared", true, true);
    if (shared_out) c.ptr(shared_out, "shared_out", 4);
    if (routed_out) c.ptr(routed_out, "routed_out");
  }
  c.ptr(ws, "ws", 256);
  if (c.code != MONO_OK || shape->rows == 0) return c.done();
  const int grid = device_grid(c, shape);
  if (c.code != MONO_OK) return c.done();
  Params p = base_params(shape, layer, ws, grid);
  const WsLayout W = ws_layout(*shape);
  uint8_t* b = static_cast<uint8_t*>(ws);
  p.norm_in = norm; p.idx_in = idx; p.w_in = weights;
  p.shared_out = shared_out ? shared_out : b + W.shared;
  p.routed_out = routed_out ? routed_out : reinterpret_cast<float*>(b + W.routed);
  p.block = block;
  const int rf = layer->routed.fmt, sf = sfmt_of(shape, layer);
  mono_status st = enqueue(K_GATEUP, p, shape, rf, sf, grid, stream, "experts gate/up");
  if (st == MONO_OK) st = enqueue(K_DOWN, p, shape, rf, sf, grid, stream, "experts down");
  if (st == MONO_OK) g_error.clear();
  return st;
}

mono_status mono_hc_head(const mono_shape* shape, const void* state, const mono_head* head,
                         float* pre, void* x, void* norm, void* stream) {
  Check c;
  check_shape(c, shape);
  c.req(head != nullptr, "head is NULL");
  if (c.code == MONO_OK) {
    c.ptr(state, "state", 16);
    c.ptr(head->w_head, "head.w_head", 16);
    c.ptr(head->head_scale, "head.head_scale");
    c.ptr(head->head_base, "head.head_base");
    c.ptr(head->w_norm, "head.w_norm", 16);
    c.ptr(norm, "norm", 16);
    if (pre) c.ptr(pre, "pre");
    if (x) c.ptr(x, "x", 16);
  }
  if (c.code != MONO_OK || shape->rows == 0) return c.done();
  const int rc = launch_head(shape->act, shape->rows, shape->hidden, shape->eps_hc,
                             shape->eps_norm, state, head->w_head, head->head_scale,
                             head->head_base, head->w_norm, pre, x, norm, stream);
  if (rc != 0) {
    g_error = std::string("hc head: ") + hipGetErrorString((hipError_t)rc);
    return MONO_E_DEVICE;
  }
  g_error.clear();
  return MONO_OK;
}

mono_status mono_hc_expand(const mono_shape* shape, const void* state, const void* block,
                           const float* post, const float* comb, const float* w_mix_next,
                           void* new_state, float* carry_out, void* ws, void* stream) {
  Check c;
  check_shape(c, shape);
  if (c.code == MONO_OK) {
    c.ptr(state, "state", 16); c.ptr(block, "block", 4); c.ptr(post, "post"); c.ptr(comb, "comb");
    c.ptr(new_state, "new_state", 16);
    if (w_mix_next) {
      c.ptr(w_mix_next, "w_mix_next", 4);
      c.ptr(carry_out, "carry_out");
    }
    if (state && new_state && state == new_state) c.fail(MONO_E_INVAL, "new_state aliases state");
  }
  c.ptr(ws, "ws", 256);
  if (c.code != MONO_OK || shape->rows == 0) return c.done();
  const int grid = device_grid(c, shape);
  if (c.code != MONO_OK) return c.done();
  Params p = base_params(shape, nullptr, ws, grid);
  const WsLayout W = ws_layout(*shape);
  p.state = state; p.block_in = block; p.post_in = post; p.comb_in = comb;
  p.w_mix_next = w_mix_next; p.state_out = new_state; p.carry_out = carry_out;
  p.carry_ws = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + W.carry);
  mono_status st = enqueue(K_EXPAND, p, shape, 0, 0, grid, stream, "expand");
  if (st == MONO_OK) g_error.clear();
  return st;
}

mono_status mono_ffn_layer(const mono_shape* shape, const mono_layer* layer,
                           const float* w_mix_next, const void* state_in, const float* carry_in,
                           void* state_out, float* carry_out, void* ws, void* stream) {
  Check c;
  check_shape(c, shape);
  c.req(layer != nullptr, "layer is NULL");
  if (c.code == MONO_OK) {
    check_formats(c, shape, layer, true, true);
    c.ptr(state_in, "state_in", 16);
    c.ptr(state_out, "state_out", 16);
    if (!carry_in) c.ptr(layer->w_mix, "layer.w_mix", 16);
    else c.ptr(carry_in, "carry_in");
    c.ptr(layer->hc_scale, "layer.hc_scale");
    c.ptr(layer->hc_base, "layer.hc_base");
    c.ptr(layer->w_norm, "layer.w_norm", 16);
    c.ptr(layer->w_router, "layer.w_router", 16);
    c.ptr(layer->bias, "layer.bias");
    check_experts(c, shape, layer->routed, "routed", true, true);
    if (shape->shared_inter > 0) check_experts(c, shape, layer->shared, "shared", true, true);
    if (w_mix_next) {
      c.ptr(w_mix_next, "w_mix_next", 4);
      c.ptr(carry_out, "carry_out");
    }
  }
  c.ptr(ws, "ws", 256);
  if (c.code != MONO_OK || shape->rows == 0) return c.done();
  const int grid = device_grid(c, shape);
  const int rf = layer->routed.fmt, sf = sfmt_of(shape, layer);
  if (c.code == MONO_OK) check_resident(c, shape, rf, sf);
  if (c.code != MONO_OK) return c.done();
  Params p = base_params(shape, layer, ws, grid);
  jitter_of(ws, p.jitter, p.jseed);
  const WsLayout W = ws_layout(*shape);
  uint8_t* b = static_cast<uint8_t*>(ws);
  p.state = state_in; p.carry_in = carry_in; p.w_mix_next = w_mix_next;
  p.state_out = state_out; p.carry_out = carry_out;
  p.carry_ws = reinterpret_cast<float*>(b + W.carry);
  p.mixes = reinterpret_cast<float*>(b + W.mixes);
  p.pre = reinterpret_cast<float*>(b + W.pre);
  p.post = reinterpret_cast<float*>(b + W.post);
  p.comb = reinterpret_cast<float*>(b + W.comb);
  p.x = b + W.x; p.norm = b + W.norm;
  p.logits = reinterpret_cast<float*>(b + W.logits);
  p.idx = reinterpret_cast<int32_t*>(b + W.idx);
  p.weights = reinterpret_cast<float*>(b + W.weights);
  p.shared_out = b + W.shared;
  p.routed_out = reinterpret_cast<float*>(b + W.routed);
  p.block = b + W.block;
  mono_status st = enqueue(K_FFN_LAYER, p, shape, rf, sf, grid, stream, "ffn layer");
  if (st == MONO_OK) g_error.clear();
  return st;
}

}  // extern "C"
