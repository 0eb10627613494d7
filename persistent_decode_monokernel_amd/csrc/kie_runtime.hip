// Host runtime behind include/kie.h: validation, device memory owned by a
// handle, and the launches of the persistent decode kernel (or of the staged
// per-kernel fallback).  No C++ exception crosses the C ABI.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "kie.h"
#include "kie_params.h"

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

#define KIE_HIP(expr)                                                                   \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess)                                                               \
      return fail(KIE_ERR_HIP, std::string(#expr) + " failed: " + hipGetErrorString(e_)); \
  } while (0)

bool is_mult(long long v, long long m) { return v > 0 && v % m == 0; }

// Checks that [p, p + bytes) lies inside one device allocation and that p is
// 16-byte aligned (the kernels read weights with 128-bit loads).
int check_device_range(const void* p, size_t bytes, const char* what) {
  if (!p) return fail(KIE_ERR_INVALID_ARG, std::string(what) + " is NULL");
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
    return fail(KIE_ERR_INVALID_ARG, std::string(what) + " is not 16-byte aligned");
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return fail(KIE_ERR_INVALID_ARG, std::string(what) + " is not a HIP device pointer");
  }
  if (attr.type != hipMemoryTypeDevice)
    return fail(KIE_ERR_INVALID_ARG, std::string(what) + " is not in device memory");
  void* base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, const_cast<void*>(p)) != hipSuccess) {
    (void)hipGetLastError();
    return fail(KIE_ERR_INVALID_ARG, std::string(what) + ": cannot query its allocation");
  }
  const char* b = static_cast<const char*>(base);
  const char* q = static_cast<const char*>(p);
  if (q < b || (size_t)(q - b) + bytes > size)
    return fail(KIE_ERR_INVALID_ARG, std::string(what) + " is smaller than its shape needs");
  return KIE_OK;
}

kie::Params shape_params(const kie_config& c) {
  kie::Params p;
  std::memset(&p, 0, sizeof(p));
  p.L = c.n_layers;
  p.d = c.d_model;
  p.H = c.n_heads;
  p.nkv = c.n_kv_heads;
  p.hd = c.head_dim;
  p.F = c.n_experts ? 0 : c.ffn_hidden;
  p.Vin = c.vocab_in;
  p.Vout = c.vocab_out;
  p.cap = c.max_seq;
  p.E = c.n_experts;
  p.topk = c.n_experts ? c.top_k : 0;
  p.moe_renorm = (c.flags & KIE_MOE_RENORM) ? 1 : 0;
  p.nshared = c.n_experts ? c.n_shared_experts : 0;
  p.Fe = c.n_experts ? c.expert_hidden : 0;
  p.eps = c.rms_eps;
  return p;
}

constexpr size_t kMaxLdsBytes = 160 * 1024;

}  // namespace

namespace {
constexpr int kPrefillChunk = 2048;                // positions per batched prefill chunk, at most
size_t moe_max_tiles(size_t rows, int E);
int scratch_setup(int dev);
}  // namespace

struct kie_handle {
  kie_config cfg{};
  kie::Params base{};            // shapes, weights and owned buffers (per-call fields unset)
  hipStream_t stream = nullptr;
  int device = 0;
  size_t lds = 0;
  long long ticks_per_ms = 100000;
  std::vector<void*> allocs;     // every hipMalloc of this handle
  kie::LayerPtrs* d_layers = nullptr;
  std::vector<kie::LayerPtrs> layers;   // host copy of the layer weight pointers
  int* d_prompt = nullptr;
  kie::Params* d_params = nullptr;   // device copy of the launch's parameter block
  kie::Params call{};                // host source of that copy (outlives the async copy)
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  float last_ms = 0.f;
  int pos = 0;
  bool pending = false;
  bool broken = false;
  int last_decode_steps = 0;
  int trace_events = 0;          // events per workgroup recorded by the last decode
  unsigned epoch_next = 1;       // first activation epoch of the next launch
  unsigned dbg_epoch0 = 0;       // kie_debug_stage: epochs of the open stage-by-stage step (0: none)
  void* pf_ws = nullptr;         // batched prefill workspace (grown on demand, freed with the handle)
  size_t pf_ws_bytes = 0;
  // MoE batched prefill: host copies of one chunk's routing and grouping,
  // sized at creation for the largest chunk
};

namespace {

int dev_alloc(kie_handle* h, size_t bytes, void** out) {
  void* p = nullptr;
  hipError_t e = hipMalloc(&p, bytes < 256 ? 256 : bytes);
  if (e != hipSuccess)
    return fail(KIE_ERR_HIP, std::string("hipMalloc(") + std::to_string(bytes) +
                                 ") failed: " + hipGetErrorString(e));
  h->allocs.push_back(p);
  *out = p;
  return KIE_OK;
}

void free_handle(kie_handle* h) {
  if (!h) return;
  (void)hipStreamSynchronize(h->stream);
  for (void* p : h->allocs) (void)hipFree(p);
  if (h->pf_ws) (void)hipFree(h->pf_ws);
  if (h->ev0) (void)hipEventDestroy(h->ev0);
  if (h->ev1) (void)hipEventDestroy(h->ev1);
  delete h;
}

// Clears barrier/argmax/error words before a launch (outside any capture).
int reset_sync_words(kie_handle* h) {
  const kie::Params& b = h->base;
  KIE_HIP(hipMemsetAsync(b.bar, 0, sizeof(unsigned) * kie::kBarrierWords, h->stream));
  KIE_HIP(hipMemsetAsync(b.amax, 0, 2 * sizeof(unsigned long long), h->stream));
  KIE_HIP(hipMemsetAsync(b.err, 0, sizeof(int), h->stream));
  KIE_HIP(hipMemsetAsync(b.state + 1, 0, sizeof(int), h->stream));
  return KIE_OK;
}

int finish_launch(kie_handle* h) {
  KIE_HIP(hipEventRecord(h->ev1, h->stream));
  KIE_HIP(hipStreamSynchronize(h->stream));
  int err = 0;
  KIE_HIP(hipMemcpy(&err, h->base.err, sizeof(int), hipMemcpyDeviceToHost));
  KIE_HIP(hipEventElapsedTime(&h->last_ms, h->ev0, h->ev1));
  if (err != 0) {
    h->broken = true;
    if (err == kie::kErrTimeout)
      return fail(KIE_ERR_TIMEOUT, "a grid barrier wait timed out; the handle needs kie_reset");
    return fail(KIE_ERR_HIP, "device reported error " + std::to_string(err));
  }
  return KIE_OK;
}

// Gives the launch a fresh range of activation epochs: every stage of every
// step of this launch stamps its outputs with an epoch no earlier launch
// used, so stale arena words never satisfy a wait.  When the 32-bit range
// would run out, the arena is cleared and numbering restarts.
int assign_epochs(kie_handle* h, kie::Params& p) {
  const unsigned long long need = (unsigned long long)(p.n_steps + 1) * p.L * 8ull + 8ull;
  if ((unsigned long long)h->epoch_next + need >= 0xFFFFFF00ull) {
    KIE_HIP(hipMemsetAsync(h->base.act, 0, sizeof(unsigned long long) * h->base.act_words, h->stream));
    h->epoch_next = 1;
  }
  p.epoch0 = h->epoch_next;
  h->epoch_next += (unsigned)need;
  return KIE_OK;
}

// Runs p.n_steps steps (prefill or decode) in the handle's mode.
int run_steps(kie_handle* h, kie::Params& p) {
  h->dbg_epoch0 = 0;
  int rc = reset_sync_words(h);
  if (rc) return rc;
  if ((rc = assign_epochs(h, p))) return rc;
  const bool staged = (h->cfg.flags & KIE_MODE_GRAPH) != 0;
  if (!staged) {
    h->call = p;
    KIE_HIP(hipMemcpyAsync(h->d_params, &h->call, sizeof(kie::Params), hipMemcpyHostToDevice,
                           h->stream));
    KIE_HIP(hipEventRecord(h->ev0, h->stream));
    KIE_HIP(kie::launch_mono(p, h->d_params, h->lds, (h->cfg.flags & KIE_PLAIN_LAUNCH) != 0,
                             h->stream));
    return finish_launch(h);
  }
  // Staged mode.  Decode: one step's kernels are captured into a hipGraph
  // once per call and replayed n_steps times; the step counter and pending
  // token live in device memory, so every replay is the same graph.
  // Prefill runs the same per-stage kernels without a graph.
  if (p.mode == kie::kPrefill || p.n_steps == 0) {
    KIE_HIP(hipEventRecord(h->ev0, h->stream));
    for (int i = 0; i < p.n_steps; ++i) KIE_HIP(kie::launch_staged_step(p, h->lds, h->stream));
    if (p.n_steps == 0 && p.mode == kie::kPrefill)
      KIE_HIP(hipMemcpyAsync(h->base.state, p.prompt, sizeof(int), hipMemcpyDeviceToDevice,
                             h->stream));
    return finish_launch(h);
  }
  hipStream_t cap_stream = nullptr;
  KIE_HIP(hipStreamCreateWithFlags(&cap_stream, hipStreamNonBlocking));
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  hipError_t e = hipStreamBeginCapture(cap_stream, hipStreamCaptureModeThreadLocal);
  if (e == hipSuccess) {
    hipError_t le = kie::launch_staged_step(p, h->lds, cap_stream);
    e = hipStreamEndCapture(cap_stream, &graph);
    if (e == hipSuccess) e = le;
  }
  if (e == hipSuccess) e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (e == hipSuccess) e = hipEventRecord(h->ev0, h->stream);
  for (int i = 0; e == hipSuccess && i < p.n_steps; ++i) e = hipGraphLaunch(exec, h->stream);
  if (e == hipSuccess) {
    rc = finish_launch(h);                 // synchronises before the graph is freed
  } else {
    (void)hipStreamSynchronize(h->stream);
    rc = fail(KIE_ERR_HIP, std::string("staged decode graph failed: ") + hipGetErrorString(e));
  }
  if (exec) (void)hipGraphExecDestroy(exec);
  if (graph) (void)hipGraphDestroy(graph);
  (void)hipStreamDestroy(cap_stream);
  return rc;
}

}  // namespace

extern "C" {

const char* kie_last_error(void) { return g_err.c_str(); }

int kie_config_check(const kie_config* c) {
  g_err.clear();
  if (!c) return fail(KIE_ERR_INVALID_ARG, "config is NULL");
  if (c->n_layers < 1 || c->n_layers > 2048) return fail(KIE_ERR_INVALID_ARG, "n_layers out of range (1..2048)");
  if (!is_mult(c->d_model, 8) || c->d_model > 32768)
    return fail(KIE_ERR_INVALID_ARG, "d_model must be a positive multiple of 8, at most 32768");
  if (c->n_heads < 1 || c->n_kv_heads < 1 || c->n_heads % c->n_kv_heads != 0)
    return fail(KIE_ERR_INVALID_ARG, "n_heads must be a positive multiple of n_kv_heads");
  const int G = c->n_heads / c->n_kv_heads;
  if (G != 1 && G != 2 && G != 4)
    return fail(KIE_ERR_UNSUPPORTED, "n_heads / n_kv_heads must be 1, 2 or 4");
  if (!is_mult(c->head_dim, 8) || c->head_dim > kie::kMaxHeadDim)
    return fail(KIE_ERR_UNSUPPORTED, "head_dim must be a multiple of 8 and at most 128");
  if ((long long)c->n_heads * c->head_dim > 32768)
    return fail(KIE_ERR_INVALID_ARG, "n_heads * head_dim too large");
  if (c->n_experts == 0) {
    if (!is_mult(c->ffn_hidden, 8) || c->ffn_hidden > 65536)
      return fail(KIE_ERR_INVALID_ARG, "ffn_hidden must be a positive multiple of 8");
  } else {
    if (c->n_experts < 1 || c->n_experts > 1024) return fail(KIE_ERR_INVALID_ARG, "n_experts out of range");
    if (c->top_k < 1 || c->top_k > c->n_experts) return fail(KIE_ERR_INVALID_ARG, "top_k out of range");
    if (c->n_shared_experts < 0) return fail(KIE_ERR_INVALID_ARG, "n_shared_experts < 0");
    if (c->top_k + c->n_shared_experts > kie::kMaxActiveExperts)
      return fail(KIE_ERR_UNSUPPORTED, "top_k + n_shared_experts must be at most 16");
    if (!is_mult(c->expert_hidden, 8)) return fail(KIE_ERR_INVALID_ARG, "expert_hidden must be a positive multiple of 8");
  }
  if (c->vocab_in < 1 || c->vocab_out < 1 || c->vocab_out > c->vocab_in)
    return fail(KIE_ERR_INVALID_ARG, "need 1 <= vocab_out <= vocab_in");
  if (c->max_seq < 1 || c->max_seq > (1 << 20)) return fail(KIE_ERR_INVALID_ARG, "max_seq out of range");
  if (!(c->rms_eps >= 0.f) || !std::isfinite(c->rms_eps)) return fail(KIE_ERR_INVALID_ARG, "rms_eps must be >= 0");
  if (!(c->rope_base > 1.f) || !std::isfinite(c->rope_base)) return fail(KIE_ERR_INVALID_ARG, "rope_base must be > 1");
  if (c->flags & ~(KIE_MODE_GRAPH | KIE_TRACE | KIE_PLAIN_LAUNCH | KIE_MOE_RENORM))
    return fail(KIE_ERR_INVALID_ARG, "unknown flag bits");
  if (c->n_workgroups < 0 || c->n_workgroups > 4096) return fail(KIE_ERR_INVALID_ARG, "n_workgroups out of range");
  if (c->timeout_ms < 0) return fail(KIE_ERR_INVALID_ARG, "timeout_ms < 0");
  kie::Params p = shape_params(*c);
  // the LDS need grows with the attention splits, i.e. with the grid: check
  // the configured grid, or 256 workgroups (one per MI355X compute unit)
  p.n_wg = c->n_workgroups > 0 ? c->n_workgroups : 256;
  p.splits = std::max(1, p.n_wg / p.nkv);
  const kie::LdsLayout L = kie::lds_layout(p);
  if ((size_t)L.total * sizeof(float) > kMaxLdsBytes)
    return fail(KIE_ERR_UNSUPPORTED, "shape needs more LDS than a compute unit has");
  return KIE_OK;
}

int kie_create(const kie_config* cfg, const kie_weights* w, void* hip_stream, kie_handle** out) {
  int rc = kie_config_check(cfg);
  if (rc) return rc;
  if (!w || !out) return fail(KIE_ERR_INVALID_ARG, "weights or out is NULL");
  if (!w->layers) return fail(KIE_ERR_INVALID_ARG, "weights->layers is NULL");
  const kie_config& c = *cfg;
  const size_t d = c.d_model, qd = (size_t)c.n_heads * c.head_dim,
               kd = (size_t)c.n_kv_heads * c.head_dim, hb = sizeof(__half);
  // ---- weight pointers: device memory, aligned, large enough
  if ((rc = check_device_range(w->tok_emb, (size_t)c.vocab_in * d * hb, "tok_emb"))) return rc;
  if ((rc = check_device_range(w->final_norm, d * hb, "final_norm"))) return rc;
  if ((rc = check_device_range(w->lm_head, (size_t)c.vocab_out * d * hb, "lm_head"))) return rc;
  for (int l = 0; l < c.n_layers; ++l) {
    const kie_layer_weights& lw = w->layers[l];
    const std::string pre = "layers[" + std::to_string(l) + "].";
    struct Need { const void* p; size_t bytes; const char* name; };
    std::vector<Need> need = {{lw.attn_norm, d * hb, "attn_norm"}, {lw.wq, qd * d * hb, "wq"},
                              {lw.wk, kd * d * hb, "wk"},          {lw.wv, kd * d * hb, "wv"},
                              {lw.wo, d * qd * hb, "wo"},          {lw.ffn_norm, d * hb, "ffn_norm"}};
    if (c.n_experts == 0) {
      const size_t F = c.ffn_hidden;
      need.push_back({lw.w_gate, F * d * hb, "w_gate"});
      need.push_back({lw.w_up, F * d * hb, "w_up"});
      need.push_back({lw.w_down, d * F * hb, "w_down"});
    } else {
      const size_t ne = (size_t)c.n_experts + c.n_shared_experts, fe = c.expert_hidden;
      need.push_back({lw.router, (size_t)c.n_experts * d * hb, "router"});
      need.push_back({lw.e_gate, ne * fe * d * hb, "e_gate"});
      need.push_back({lw.e_up, ne * fe * d * hb, "e_up"});
      need.push_back({lw.e_down, ne * d * fe * hb, "e_down"});
    }
    for (const Need& n : need)
      if ((rc = check_device_range(n.p, n.bytes, (pre + n.name).c_str()))) return rc;
  }

  kie_handle* h = new (std::nothrow) kie_handle();
  if (!h) return fail(KIE_ERR_INVALID_ARG, "out of host memory");
  h->cfg = c;
  h->stream = static_cast<hipStream_t>(hip_stream);
  auto bail = [&](int code) {
    free_handle(h);
    return code;
  };
  if (hipGetDevice(&h->device) != hipSuccess) return bail(fail(KIE_ERR_HIP, "hipGetDevice failed"));
  int n_cu = 0, clk_khz = 0;
  if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, h->device) != hipSuccess ||
      hipDeviceGetAttribute(&clk_khz, hipDeviceAttributeWallClockRate, h->device) != hipSuccess)
    return bail(fail(KIE_ERR_HIP, "device attribute query failed"));
  if (clk_khz > 0) h->ticks_per_ms = clk_khz;

  kie::Params& p = h->base;
  p = shape_params(c);
  p.n_wg = c.n_workgroups > 0 ? c.n_workgroups : n_cu;
  p.splits = std::max(1, p.n_wg / p.nkv);
  if ((c.d_model + p.n_wg - 1) / p.n_wg > kie::kPartCap)
    return bail(fail(KIE_ERR_UNSUPPORTED, "d_model / n_workgroups must be at most " +
                                              std::to_string(kie::kPartCap)));
  const kie::LdsLayout L = kie::lds_layout(p);
  h->lds = (size_t)L.total * sizeof(float);
  if (h->lds > kMaxLdsBytes)
    return bail(fail(KIE_ERR_UNSUPPORTED, "shape needs more LDS than a compute unit has"));
  const int per_cu = kie::max_blocks_per_cu(c.n_heads / c.n_kv_heads, c.n_experts != 0, h->lds);
  if (per_cu < 1 || (long long)per_cu * n_cu < p.n_wg)
    return bail(fail(KIE_ERR_OCCUPANCY, "grid of " + std::to_string(p.n_wg) +
                                            " workgroups cannot be co-resident (" +
                                            std::to_string(per_cu) + " per CU x " +
                                            std::to_string(n_cu) + " CUs)"));
  p.tok_emb = static_cast<const __half*>(w->tok_emb);
  p.final_norm = static_cast<const __half*>(w->final_norm);
  p.lm_head = static_cast<const __half*>(w->lm_head);

  // ---- owned buffers
  const size_t cap = c.max_seq, hd = c.head_dim;
  const size_t kv_elems = (size_t)c.n_layers * c.n_kv_heads * cap * hd;
  void* ptr = nullptr;
#define KIE_ALLOC(field, type, count)                                   \
  do {                                                                  \
    if ((rc = dev_alloc(h, sizeof(type) * (size_t)(count), &ptr))) return bail(rc); \
    p.field = static_cast<type*>(ptr);                                  \
  } while (0)
  KIE_ALLOC(kc, __half, kv_elems);
  KIE_ALLOC(vc, __half, kv_elems);
  float* rc_tab = nullptr;
  if ((rc = dev_alloc(h, sizeof(float) * cap * hd, &ptr))) return bail(rc);
  rc_tab = static_cast<float*>(ptr);
  p.rope_cos = rc_tab;
  p.rope_sin = rc_tab + cap * (hd / 2);
  // activation arena (64-bit flag-in-data words), one region per buffer
  const size_t ucount = c.n_experts ? (size_t)(c.top_k + c.n_shared_experts) * c.expert_hidden
                                    : (size_t)c.ffn_hidden;
  {
    size_t off = 0;
    auto region = [&](int& field, size_t words) {
      field = (int)off;
      off += (words + 1) & ~(size_t)1;     // keep regions 16-byte aligned
    };
    region(p.off_x, d);
    region(p.off_xh, d / 2);
    region(p.off_qkv, qd + 2 * kd);
    region(p.off_o, qd / 2);
    region(p.off_u, ucount / 2);
    region(p.off_router, std::max(1, c.n_experts));
    region(p.off_part, (size_t)c.n_heads * p.splits * (hd + 2));
    if (off * 8 >= 0xFFFFFF00ull) return bail(fail(KIE_ERR_UNSUPPORTED, "activation arena too large"));
    p.act_words = (int)off;
    KIE_ALLOC(act, unsigned long long, off);
  }
  KIE_ALLOC(bar, unsigned, kie::kBarrierWords);
  KIE_ALLOC(amax, unsigned long long, 2);
  KIE_ALLOC(err, int, 1);
  KIE_ALLOC(state, int, 4);
  KIE_ALLOC(zbuf, float, c.vocab_out);
  KIE_ALLOC(expert_log, int, c.n_experts ? cap * c.n_layers * c.top_k : 1);
  if (c.flags & KIE_TRACE) {
    KIE_ALLOC(trace, unsigned long long, (size_t)p.n_wg * kie::kTraceEvents);
  }
#undef KIE_ALLOC
  if ((rc = dev_alloc(h, sizeof(int) * cap, &ptr))) return bail(rc);
  h->d_prompt = static_cast<int*>(ptr);
  if ((rc = dev_alloc(h, sizeof(kie::Params), &ptr))) return bail(rc);
  h->d_params = static_cast<kie::Params*>(ptr);
  if ((rc = dev_alloc(h, sizeof(kie::LayerPtrs) * c.n_layers, &ptr))) return bail(rc);
  h->d_layers = static_cast<kie::LayerPtrs*>(ptr);
  p.layers = h->d_layers;

  std::vector<kie::LayerPtrs> lp(c.n_layers);
  for (int l = 0; l < c.n_layers; ++l) {
    const kie_layer_weights& s = w->layers[l];
    kie::LayerPtrs& t = lp[l];
    auto hp = [](const void* v) { return static_cast<const __half*>(v); };
    t.attn_norm = hp(s.attn_norm); t.wq = hp(s.wq); t.wk = hp(s.wk); t.wv = hp(s.wv);
    t.wo = hp(s.wo); t.ffn_norm = hp(s.ffn_norm);
    t.w_gate = hp(s.w_gate); t.w_up = hp(s.w_up); t.w_down = hp(s.w_down);
    t.router = hp(s.router); t.e_gate = hp(s.e_gate); t.e_up = hp(s.e_up); t.e_down = hp(s.e_down);
  }
  // RoPE table: angle p * base^(-2j/hd) in float64, cos/sin rounded once to fp32.
  std::vector<float> tab(cap * hd);
  const size_t half = hd / 2;
  for (size_t j = 0; j < half; ++j) {
    const double theta = std::pow((double)c.rope_base, -2.0 * (double)j / (double)hd);
    for (size_t q = 0; q < cap; ++q) {
      const double a = (double)q * theta;
      tab[q * half + j] = (float)std::cos(a);
      tab[cap * half + q * half + j] = (float)std::sin(a);
    }
  }
  h->layers = lp;
  if (hipMemcpy(h->d_layers, lp.data(), sizeof(kie::LayerPtrs) * c.n_layers, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(rc_tab, tab.data(), sizeof(float) * tab.size(), hipMemcpyHostToDevice) != hipSuccess ||
      hipMemset(p.state, 0, 4 * sizeof(int)) != hipSuccess ||
      hipMemset(p.act, 0, sizeof(unsigned long long) * (size_t)p.act_words) != hipSuccess ||
      hipEventCreate(&h->ev0) != hipSuccess || hipEventCreate(&h->ev1) != hipSuccess)
    return bail(fail(KIE_ERR_HIP, "initialising handle buffers failed"));
  const int tmo = c.timeout_ms > 0 ? c.timeout_ms : 20000;
  p.timeout_ticks = (long long)tmo * h->ticks_per_ms;
  if ((rc = scratch_setup(h->device))) return bail(rc);
  *out = h;
  g_err.clear();
  return KIE_OK;
}

int kie_prefill(kie_handle* h, const int32_t* tokens, int32_t n) {
  g_err.clear();
  if (!h || !tokens) return fail(KIE_ERR_INVALID_ARG, "handle or tokens is NULL");
  if (h->broken) return fail(KIE_ERR_BAD_STATE, "handle is broken; call kie_reset");
  if (h->pos != 0 || h->pending) return fail(KIE_ERR_BAD_STATE, "prefill needs a fresh or reset handle");
  if (n < 1) return fail(KIE_ERR_INVALID_ARG, "n_tokens must be >= 1");
  if (n > h->cfg.max_seq) return fail(KIE_ERR_CONTEXT_OVERFLOW, "prompt longer than max_seq");
  for (int i = 0; i < n; ++i)
    if (tokens[i] < 0 || tokens[i] >= h->cfg.vocab_in)
      return fail(KIE_ERR_TOKEN_RANGE, "prompt token " + std::to_string(i) + " out of range");
  KIE_HIP(hipMemcpyAsync(h->d_prompt, tokens, sizeof(int) * n, hipMemcpyHostToDevice, h->stream));
  kie::Params p = h->base;
  p.trace = nullptr;
  p.mode = kie::kPrefill;
  p.n_steps = n - 1;
  p.pos0 = 0;
  p.prompt = h->d_prompt;
  int rc = run_steps(h, p);
  if (rc) return rc;
  h->pos = n - 1;
  h->pending = true;
  return KIE_OK;
}

namespace {
static int decode_steps(kie_handle* h, int32_t n, int32_t* out_tokens, float* out_logits, int sample,
                        float temperature, uint64_t seed, int top_k = 0, float top_p = 1.f);

// Batched prefill of positions 0 .. n - 2 in chunks of kPrefillChunk positions.
// Per chunk and layer: RMSNorm -> Q/K/V products -> RoPE + fp16 K/V rows into
// the cache -> causal attention over the cache -> O product + residual ->
// RMSNorm -> gate/up products -> SwiGLU -> down product + residual.

// Mixture-of-experts FFN of one chunk and layer (hi/lo hold the normed
// input): router product, routing per position, positions grouped by expert
// on the device, the routed experts' products over their grouped rows as one
// grouped launch per product, shared experts over all rows, and the weighted
// expert outputs summed back in rank order.
struct MoeWs {
  float *R, *wts, *Gc, *Uc, *Yc;
  int *ids, *perm, *inv, *tiles;
  __half *ch, *cl, *sh, *sl;
  int* fill;                                             // int[E]
};

// Row tiles of the grouped products: at most rows / 64 + E of them.
size_t moe_max_tiles(size_t rows, int E) { return rows / 64 + (size_t)E + 1; }

static int moe_ffn_batched(kie_handle* h, const kie::LayerPtrs& w, int l, int c0, int Tn, const __half* hi,
                    const __half* lo, float* X, MoeWs& m) {
  const kie::Params& p = h->base;
  hipStream_t s = h->stream;
  const int d = p.d, E = p.E, k = p.topk, Fe = p.Fe, rows = Tn * k;
  auto ok = [&](hipError_t err) {
    return err == hipSuccess ? KIE_OK : fail(KIE_ERR_HIP, std::string("prefill launch failed: ") + hipGetErrorString(err));
  };
  int rc;
  if ((rc = ok(kie::launch_gemm(hi, lo, d, w.router, d, m.R, E, Tn, E, d, false, s)))) return rc;
  if ((rc = ok(kie::launch_route(m.R, E, k, p.moe_renorm, m.ids, m.wts, p.expert_log, p.L, l, c0, Tn, s)))) return rc;
  const int mt = (int)moe_max_tiles((size_t)rows, E);
  if ((rc = ok(kie::launch_moe_group(m.ids, rows, E, m.fill, m.tiles, mt, m.perm, m.inv, s)))) return rc;
  if ((rc = ok(kie::launch_gather_rows(hi, lo, d, m.perm, k, m.ch, m.cl, rows, s)))) return rc;
  const size_t gate_e = (size_t)Fe * d, down_e = (size_t)d * Fe;
  if ((rc = ok(kie::launch_gemm_grouped(m.ch, m.cl, d, w.e_gate, gate_e, d, m.Gc, Fe, m.tiles, mt, Fe, d, s))) ||
      (rc = ok(kie::launch_gemm_grouped(m.ch, m.cl, d, w.e_up, gate_e, d, m.Uc, Fe, m.tiles, mt, Fe, d, s))) ||
      (rc = ok(kie::launch_swiglu_w_split(m.Gc, m.Uc, Fe, rows, m.perm, m.wts, m.sh, m.sl, s))) ||
      (rc = ok(kie::launch_gemm_grouped(m.sh, m.sl, Fe, w.e_down, down_e, Fe, m.Yc, d, m.tiles, mt, d, Fe, s))))
    return rc;
  for (int a = 0; a < p.nshared; ++a) {
    const size_t es = (size_t)(E + a);
    if ((rc = ok(kie::launch_gemm(hi, lo, d, w.e_gate + es * gate_e, d, m.Gc, Fe, Tn, Fe, d, false, s))) ||
        (rc = ok(kie::launch_gemm(hi, lo, d, w.e_up + es * gate_e, d, m.Uc, Fe, Tn, Fe, d, false, s))) ||
        (rc = ok(kie::launch_swiglu_w_split(m.Gc, m.Uc, Fe, Tn, nullptr, nullptr, m.sh, m.sl, s))) ||
        (rc = ok(kie::launch_gemm(m.sh, m.sl, Fe, w.e_down + es * down_e, Fe, X, d, Tn, d, Fe, true, s))))
      return rc;
  }
  return ok(kie::launch_combine(X, d, m.Yc, m.inv, k, Tn, s));
}

// The batched prefill's device workspace for chunks of T positions: the
// chunk's activations (fp32), the hi/lo fp16 split of the widest product
// input and, for MoE, the routing and grouped-row buffers.  Returns its size
// in bytes; with a base address, also carves it (regions 256-byte aligned).
struct PfWs {
  float *X, *QKV, *O, *G, *U;
  __half *hi, *lo;
  MoeWs m;
};

static size_t prefill_ws(const kie::Params& p, int T, char* base, PfWs* w) {
  const bool moe = p.E != 0;
  const int d = p.d, qd = p.H * p.hd, kd = p.nkv * p.hd, F = moe ? 0 : p.F, qkv = qd + 2 * kd;
  const int wide = std::max(std::max(d, qd), F);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) & ~(size_t)255;
    return base ? base + at : nullptr;
  };
  const size_t t = (size_t)T;
  char* X = take(sizeof(float) * t * d);
  char* QKV = take(sizeof(float) * t * qkv);
  char* O = take(sizeof(float) * t * qd);
  char* G = take(sizeof(float) * t * F);
  char* U = take(sizeof(float) * t * F);
  char* hi = take(sizeof(__half) * t * wide);
  char* lo = take(sizeof(__half) * t * wide);
  if (w) {
    w->X = reinterpret_cast<float*>(X);
    w->QKV = reinterpret_cast<float*>(QKV);
    w->O = reinterpret_cast<float*>(O);
    w->G = reinterpret_cast<float*>(G);
    w->U = reinterpret_cast<float*>(U);
    w->hi = reinterpret_cast<__half*>(hi);
    w->lo = reinterpret_cast<__half*>(lo);
  }
  if (moe) {
    // router logits, routing, compact rows (T * top_k of them), row tiles
    const size_t rk = t * p.topk, rx = std::max(rk, t), Fe = p.Fe, rows_d = rk * d;
    char* R = take(sizeof(float) * t * p.E);
    char* wts = take(sizeof(float) * rk);
    char* Gc = take(sizeof(float) * rx * Fe);
    char* Uc = take(sizeof(float) * rx * Fe);
    char* Yc = take(sizeof(float) * rows_d);
    char* ids = take(sizeof(int) * rk);
    char* perm = take(sizeof(int) * rk);
    char* inv = take(sizeof(int) * rk);
    char* tiles = take(sizeof(int) * 3 * moe_max_tiles(rk, p.E));
    char* fill = take(sizeof(int) * p.E);
    char* ch = take(sizeof(__half) * rows_d);
    char* cl = take(sizeof(__half) * rows_d);
    char* sh = take(sizeof(__half) * rx * Fe);
    char* sl = take(sizeof(__half) * rx * Fe);
    if (w) {
      MoeWs& m = w->m;
      m.R = reinterpret_cast<float*>(R);
      m.wts = reinterpret_cast<float*>(wts);
      m.Gc = reinterpret_cast<float*>(Gc);
      m.Uc = reinterpret_cast<float*>(Uc);
      m.Yc = reinterpret_cast<float*>(Yc);
      m.ids = reinterpret_cast<int*>(ids);
      m.perm = reinterpret_cast<int*>(perm);
      m.inv = reinterpret_cast<int*>(inv);
      m.tiles = reinterpret_cast<int*>(tiles);
      m.fill = reinterpret_cast<int*>(fill);
      m.ch = reinterpret_cast<__half*>(ch);
      m.cl = reinterpret_cast<__half*>(cl);
      m.sh = reinterpret_cast<__half*>(sh);
      m.sl = reinterpret_cast<__half*>(sl);
    }
  }
  return off;
}

// Prefill of positions 0 .. n - 2 in chunks of T positions, with the
// workspace `ws` carved for T (prefill_ws).  No allocation.
static int prefill_batched(kie_handle* h, int n, int T, char* ws) {
  const kie::Params& p = h->base;
  const bool moe = p.E != 0;
  const int d = p.d, qd = p.H * p.hd, kd = p.nkv * p.hd, F = moe ? 0 : p.F, qkv = qd + 2 * kd;
  PfWs W{};
  (void)prefill_ws(p, T, ws, &W);
  MoeWs& mw = W.m;
  float* X = W.X;
  float* QKV = W.QKV;
  float* O = W.O;
  float* G = W.G;
  float* U = W.U;
  __half* hi = W.hi;
  __half* lo = W.lo;
  hipStream_t s = h->stream;
  const size_t layer_kv = (size_t)p.nkv * p.cap * p.hd;
  int rc = KIE_OK;
  auto ok = [&](hipError_t err) {
    if (err != hipSuccess && rc == KIE_OK)
      rc = fail(KIE_ERR_HIP, std::string("prefill launch failed: ") + hipGetErrorString(err));
    return rc == KIE_OK;
  };
  for (int c0 = 0; c0 < n - 1 && rc == KIE_OK; c0 += T) {
    const int Tn = std::min(T, n - 1 - c0);
    if (!ok(kie::launch_embed(p.tok_emb, h->d_prompt + c0, d, X, Tn, s))) break;
    for (int l = 0; l < p.L && rc == KIE_OK; ++l) {
      const kie::LayerPtrs& w = h->layers[l];
      __half* kc = p.kc + (size_t)l * layer_kv;
      __half* vc = p.vc + (size_t)l * layer_kv;
      ok(kie::launch_rmsnorm_split(X, w.attn_norm, d, p.eps, hi, lo, Tn, s)) &&
          ok(kie::launch_gemm(hi, lo, d, w.wq, d, QKV, qkv, Tn, qd, d, false, s)) &&
          ok(kie::launch_gemm(hi, lo, d, w.wk, d, QKV + qd, qkv, Tn, kd, d, false, s)) &&
          ok(kie::launch_gemm(hi, lo, d, w.wv, d, QKV + qd + kd, qkv, Tn, kd, d, false, s)) &&
          ok(kie::launch_rope_kv(QKV, qkv, p.H, p.nkv, p.hd, c0, p.rope_cos, p.rope_sin, kc, vc, p.cap, Tn, s)) &&
          ok(kie::launch_attn_prefill(QKV, qkv, kc, vc, p.cap, p.H, p.nkv, p.hd, c0, O, Tn, s)) &&
          ok(kie::launch_split(O, qd, hi, lo, Tn, qd, s)) &&
          ok(kie::launch_gemm(hi, lo, qd, w.wo, qd, X, d, Tn, d, qd, true, s)) &&
          ok(kie::launch_rmsnorm_split(X, w.ffn_norm, d, p.eps, hi, lo, Tn, s));
      if (rc != KIE_OK) break;
      if (moe) {
        rc = moe_ffn_batched(h, w, l, c0, Tn, hi, lo, X, mw);
      } else {
        ok(kie::launch_gemm(hi, lo, d, w.w_gate, d, G, F, Tn, F, d, false, s)) &&
            ok(kie::launch_gemm(hi, lo, d, w.w_up, d, U, F, Tn, F, d, false, s)) &&
            ok(kie::launch_swiglu_split(G, U, (size_t)Tn * F, hi, lo, s)) &&
            ok(kie::launch_gemm(hi, lo, F, w.w_down, F, X, d, Tn, d, F, true, s));
      }
    }
  }
  const hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess && rc == KIE_OK)
    rc = fail(KIE_ERR_HIP, std::string("prefill failed: ") + hipGetErrorString(e));
  return rc;
}

// Validation shared by both batched prefill entries (nothing launched).
static int prefill_batched_check(kie_handle* h, const int32_t* tokens, int32_t n) {
  if (!h || !tokens) return fail(KIE_ERR_INVALID_ARG, "handle or tokens is NULL");
  if (h->broken) return fail(KIE_ERR_BAD_STATE, "handle is broken; call kie_reset");
  if (h->pos != 0 || h->pending) return fail(KIE_ERR_BAD_STATE, "prefill needs a fresh or reset handle");
  if (n < 1) return fail(KIE_ERR_INVALID_ARG, "n_tokens must be >= 1");
  if (n > h->cfg.max_seq) return fail(KIE_ERR_CONTEXT_OVERFLOW, "prompt longer than max_seq");
  const kie::Params& p = h->base;
  if (p.d % 32 != 0 || (p.H * p.hd) % 32 != 0 || (p.E ? p.Fe : p.F) % 32 != 0 || p.hd % 16 != 0)
    return fail(KIE_ERR_UNSUPPORTED, "batched prefill needs d_model, n_heads*head_dim and ffn_hidden "
                                     "to be multiples of 32 and head_dim of 16; use kie_prefill");
  for (int i = 0; i < n; ++i)
    if (tokens[i] < 0 || tokens[i] >= h->cfg.vocab_in)
      return fail(KIE_ERR_TOKEN_RANGE, "prompt token " + std::to_string(i) + " out of range");
  return KIE_OK;
}

// Runs a validated batched prefill with chunks of T positions in workspace
// `ws` and makes the last prompt token pending.
static int prefill_batched_run(kie_handle* h, const int32_t* tokens, int32_t n, int T, char* ws) {
  KIE_HIP(hipMemcpyAsync(h->d_prompt, tokens, sizeof(int) * n, hipMemcpyHostToDevice, h->stream));
  KIE_HIP(hipEventRecord(h->ev0, h->stream));
  int rc = prefill_batched(h, n, T, ws);
  if (rc) {
    h->broken = true;
    return rc;
  }
  // the pending token, where the decode kernel reads it
  KIE_HIP(hipMemcpyAsync(h->base.state, h->d_prompt + (n - 1), sizeof(int), hipMemcpyDeviceToDevice,
                         h->stream));
  KIE_HIP(hipEventRecord(h->ev1, h->stream));
  KIE_HIP(hipStreamSynchronize(h->stream));
  KIE_HIP(hipEventElapsedTime(&h->last_ms, h->ev0, h->ev1));
  h->pos = n - 1;
  h->pending = true;
  return KIE_OK;
}

// ---- the no-allocation prefill's workspace: one static array per GPU
constexpr size_t kScratchBytes = (size_t)KIE_PREFILL_SCRATCH_MIB << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// Device memory of the no-allocation prefill.  In host code this name is a
// stand-in, not a device address: kernels get the address that
// hipGetSymbolAddress returns for the current device (scratch_setup).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
// Looks up, once per device and with that device current, the device
// address of `scratch`.
int scratch_setup(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return fail(KIE_ERR_UNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev]) return KIE_OK;
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr)
    return fail(KIE_ERR_HIP, std::string("hipGetSymbolAddress(scratch) failed: ") + hipGetErrorString(e));
  g_scratch_ptr[dev] = ptr;
  return KIE_OK;
}

static void* scratch_of(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch_ptr[dev];
}
}  // namespace

int kie_prefill_batched(kie_handle* h, const int32_t* tokens, int32_t n) {
  g_err.clear();
  int rc = prefill_batched_check(h, tokens, n);
  if (rc) return rc;
  const int T = std::max(1, std::min(kPrefillChunk, n - 1));   // positions per chunk (workspace rows)
  const size_t need = prefill_ws(h->base, T, nullptr, nullptr);
  if (need > h->pf_ws_bytes) {
    // grow the handle's workspace; the stream is idle between calls
    KIE_HIP(hipStreamSynchronize(h->stream));
    if (h->pf_ws) (void)hipFree(h->pf_ws);
    h->pf_ws = nullptr;
    h->pf_ws_bytes = 0;
    void* ws = nullptr;
    const hipError_t e = hipMalloc(&ws, need);
    if (e != hipSuccess)
      return fail(KIE_ERR_HIP, std::string("prefill workspace hipMalloc failed: ") + hipGetErrorString(e));
    h->pf_ws = ws;
    h->pf_ws_bytes = need;
  }
  return prefill_batched_run(h, tokens, n, T, static_cast<char*>(h->pf_ws));
}

int kie_prefill_batched_noalloc(kie_handle* h, const int32_t* tokens, int32_t n) {
  g_err.clear();
  int rc = prefill_batched_check(h, tokens, n);
  if (rc) return rc;
  char* ws = static_cast<char*>(scratch_of(h->device));
  if (!ws) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || cur != h->device)
      return fail(KIE_ERR_BAD_STATE, "the handle's device is not current");
    if ((rc = scratch_setup(h->device))) return rc;
    ws = static_cast<char*>(scratch_of(h->device));
  }
  // the largest chunk, up to the usual one, whose workspace fits the array
  int T = std::max(1, std::min(kPrefillChunk, n - 1));
  if (prefill_ws(h->base, 1, nullptr, nullptr) > kScratchBytes)
    return fail(KIE_ERR_UNSUPPORTED, "one position's prefill workspace exceeds the " +
                                         std::to_string(KIE_PREFILL_SCRATCH_MIB) +
                                         " MiB static scratch; use kie_prefill_batched");
  if (prefill_ws(h->base, T, nullptr, nullptr) > kScratchBytes) {
    int lo = 1, hi = T;                       // lo fits, hi does not
    while (hi - lo > 1) {
      const int mid = lo + (hi - lo) / 2;
      (prefill_ws(h->base, mid, nullptr, nullptr) <= kScratchBytes ? lo : hi) = mid;
    }
    T = lo;
  }
  return prefill_batched_run(h, tokens, n, T, ws);
}

int kie_debug_gemm(const void* w, const float* a, float* c, int32_t m, int32_t n, int32_t k,
                   int32_t accumulate, void* hip_stream) {
  g_err.clear();
  if (m < 1 || n < 1 || k < 32 || k % 32 != 0 || m > 65536 || n > 65536 || k > 65536)
    return fail(KIE_ERR_INVALID_ARG, "need m, n >= 1 and k a positive multiple of 32 (all <= 65536)");
  // the product kernel addresses each operand with 32-bit byte offsets
  if ((size_t)n * k * sizeof(__half) >= ((size_t)1 << 31) || (size_t)m * k * sizeof(__half) >= ((size_t)1 << 31))
    return fail(KIE_ERR_INVALID_ARG, "w (n x k) and the split a (m x k) must each be under 2 GiB of fp16");
  int rc;
  if ((rc = check_device_range(w, (size_t)n * k * sizeof(__half), "w"))) return rc;
  if ((rc = check_device_range(a, (size_t)m * k * sizeof(float), "a"))) return rc;
  if ((rc = check_device_range(c, (size_t)m * n * sizeof(float), "c"))) return rc;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  void* ws = nullptr;
  KIE_HIP(hipMalloc(&ws, sizeof(__half) * (size_t)m * k * 2));
  __half* hi = static_cast<__half*>(ws);
  __half* lo = hi + (size_t)m * k;
  hipError_t e = kie::launch_split(a, k, hi, lo, m, k, s);
  if (e == hipSuccess)
    e = kie::launch_gemm(hi, lo, k, static_cast<const __half*>(w), k, c, n, m, n, k, accumulate != 0, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  (void)hipFree(ws);
  if (e != hipSuccess) return fail(KIE_ERR_HIP, std::string("gemm failed: ") + hipGetErrorString(e));
  return KIE_OK;
}

int kie_decode(kie_handle* h, int32_t n, int32_t* out_tokens, float* out_logits) {
  g_err.clear();
  return decode_steps(h, n, out_tokens, out_logits, 0, 0.f, 0ull);
}

int kie_decode_sampled(kie_handle* h, int32_t n, uint64_t seed, float temperature, int32_t* out_tokens,
                       float* out_logits) {
  g_err.clear();
  if (!(temperature >= 0.f) || !std::isfinite(temperature))
    return fail(KIE_ERR_INVALID_ARG, "temperature must be finite and >= 0");
  return decode_steps(h, n, out_tokens, out_logits, temperature > 0.f ? 1 : 0, temperature, seed);
}

int kie_decode_sampled_topkp(kie_handle* h, int32_t n, uint64_t seed, float temperature, int32_t top_k,
                             float top_p, int32_t* out_tokens, float* out_logits) {
  g_err.clear();
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(KIE_ERR_INVALID_ARG, "temperature must be finite and > 0");
  if (top_k < 0 || top_k > kie::kMaxTopK)
    return fail(KIE_ERR_INVALID_ARG, "top_k must be in [0, " + std::to_string(kie::kMaxTopK) + "]");
  if (!(top_p > 0.f && top_p <= 1.f)) return fail(KIE_ERR_INVALID_ARG, "top_p must be in (0, 1]");
  if (top_k == 0 && top_p == 1.f)      // nothing restricts the draw: plain temperature sampling
    return decode_steps(h, n, out_tokens, out_logits, 1, temperature, seed);
  if (h && (h->cfg.flags & KIE_MODE_GRAPH))
    return fail(KIE_ERR_UNSUPPORTED, "top-k / top-p sampling runs in the persistent mode only");
  return decode_steps(h, n, out_tokens, out_logits, 2, temperature, seed, top_k, top_p);
}

namespace {
static int decode_steps(kie_handle* h, int32_t n, int32_t* out_tokens, float* out_logits, int sample,
                 float temperature, uint64_t seed, int top_k, float top_p) {
  if (!h) return fail(KIE_ERR_INVALID_ARG, "handle is NULL");
  if (h->broken) return fail(KIE_ERR_BAD_STATE, "handle is broken; call kie_reset");
  if (n < 0) return fail(KIE_ERR_INVALID_ARG, "n_steps < 0");
  if (n == 0) return KIE_OK;
  if (!h->pending) return fail(KIE_ERR_BAD_STATE, "decode needs a prompt (kie_prefill)");
  if ((long long)h->pos + n > h->cfg.max_seq)
    return fail(KIE_ERR_CONTEXT_OVERFLOW, "position + n_steps exceeds max_seq");
  int rc = check_device_range(out_tokens, sizeof(int32_t) * (size_t)n, "out_tokens");
  if (rc) return rc;
  if (out_logits &&
      (rc = check_device_range(out_logits, sizeof(float) * (size_t)n * h->cfg.vocab_out, "out_logits")))
    return rc;
  kie::Params p = h->base;
  p.mode = kie::kDecode;
  p.n_steps = n;
  p.pos0 = h->pos;
  p.out_tokens = out_tokens;
  p.out_logits = out_logits;
  p.trace_step = n > 1 ? 1 : 0;
  p.sample = sample;
  p.temperature = sample ? temperature : 0.f;
  p.seed = sample ? (unsigned long long)seed : 0ull;
  p.top_k = sample == 2 ? top_k : 0;
  p.top_p = sample == 2 ? top_p : 1.f;
  rc = run_steps(h, p);
  if (rc) return rc;
  h->pos += n;
  h->last_decode_steps = n;
  if (p.trace) {
    const int per_layer = h->cfg.n_experts ? 6 : 5;
    // step start; for every stage (per_layer per layer, then lm_head) the
    // moment its inputs were complete, the moment its main loop started and
    // the moment it finished (the previous step's argmax barrier is waited
    // for inside the first stage)
    h->trace_events = std::min(kie::kTraceEvents, 1 + 3 * (h->cfg.n_layers * per_layer + 1));
  }
  return KIE_OK;
}
}  // namespace

int kie_reset(kie_handle* h) {
  g_err.clear();
  if (!h) return fail(KIE_ERR_INVALID_ARG, "handle is NULL");
  KIE_HIP(hipStreamSynchronize(h->stream));
  h->pos = 0;
  h->pending = false;
  h->broken = false;
  h->last_decode_steps = 0;
  h->dbg_epoch0 = 0;
  return KIE_OK;
}

int kie_get_position(const kie_handle* h, int32_t* pos) {
  if (!h || !pos) return fail(KIE_ERR_INVALID_ARG, "handle or pos is NULL");
  *pos = h->pos;
  return KIE_OK;
}

int kie_last_elapsed_ms(const kie_handle* h, float* ms) {
  if (!h || !ms) return fail(KIE_ERR_INVALID_ARG, "handle or ms is NULL");
  *ms = h->last_ms;
  return KIE_OK;
}

void kie_destroy(kie_handle* h) { free_handle(h); }

int kie_debug_read_kv(const kie_handle* h, int32_t layer, int32_t pos0, int32_t pos1, void* k_host,
                      void* v_host) {
  g_err.clear();
  if (!h) return fail(KIE_ERR_INVALID_ARG, "handle is NULL");
  const kie_config& c = h->cfg;
  if (layer < 0 || layer >= c.n_layers || pos0 < 0 || pos1 < pos0 || pos1 > c.max_seq)
    return fail(KIE_ERR_INVALID_ARG, "layer or position range out of bounds");
  KIE_HIP(hipStreamSynchronize(h->stream));
  const size_t hd = c.head_dim, cap = c.max_seq, rows = (size_t)(pos1 - pos0);
  const size_t row_bytes = hd * sizeof(__half);
  for (int g = 0; g < c.n_kv_heads; ++g) {
    const size_t src = (((size_t)layer * c.n_kv_heads + g) * cap + pos0) * hd;
    const size_t dst = (size_t)g * rows * hd;
    if (k_host && rows)
      KIE_HIP(hipMemcpy(static_cast<__half*>(k_host) + dst, h->base.kc + src, rows * row_bytes,
                        hipMemcpyDeviceToHost));
    if (v_host && rows)
      KIE_HIP(hipMemcpy(static_cast<__half*>(v_host) + dst, h->base.vc + src, rows * row_bytes,
                        hipMemcpyDeviceToHost));
  }
  return KIE_OK;
}

int kie_debug_expert_ids(const kie_handle* h, int32_t pos0, int32_t pos1, int32_t* ids_host) {
  g_err.clear();
  if (!h || !ids_host) return fail(KIE_ERR_INVALID_ARG, "handle or ids is NULL");
  const kie_config& c = h->cfg;
  if (c.n_experts == 0) return fail(KIE_ERR_INVALID_ARG, "not a MoE model");
  if (pos0 < 0 || pos1 < pos0 || pos1 > h->pos)
    return fail(KIE_ERR_INVALID_ARG, "position range is not inside the processed positions");
  KIE_HIP(hipStreamSynchronize(h->stream));
  const size_t row = (size_t)c.n_layers * c.top_k;
  if (pos1 > pos0)
    KIE_HIP(hipMemcpy(ids_host, h->base.expert_log + (size_t)pos0 * row,
                      sizeof(int) * (size_t)(pos1 - pos0) * row, hipMemcpyDeviceToHost));
  return KIE_OK;
}

int kie_debug_read_trace(const kie_handle* h, uint64_t* out, int32_t max_events, int32_t* n_events,
                         int32_t* n_workgroups) {
  g_err.clear();
  if (!h || !out || !n_events) return fail(KIE_ERR_INVALID_ARG, "handle, out or n_events is NULL");
  if (!h->base.trace || h->trace_events == 0)
    return fail(KIE_ERR_BAD_STATE, "no trace: create with KIE_TRACE and call kie_decode first");
  if (max_events < h->trace_events) return fail(KIE_ERR_INVALID_ARG, "max_events too small");
  KIE_HIP(hipStreamSynchronize(h->stream));
  const int nwg = h->base.n_wg, ne = h->trace_events;
  std::vector<unsigned long long> buf((size_t)nwg * kie::kTraceEvents);
  KIE_HIP(hipMemcpy(buf.data(), h->base.trace, sizeof(unsigned long long) * buf.size(),
                    hipMemcpyDeviceToHost));
  for (int w = 0; w < nwg; ++w)
    for (int e = 0; e < ne; ++e) out[(size_t)w * max_events + e] = buf[(size_t)w * kie::kTraceEvents + e];
  *n_events = ne;
  if (n_workgroups) *n_workgroups = nwg;
  return KIE_OK;
}

int kie_debug_gemv(const void* w, const float* x, float* y, int32_t rows, int32_t cols,
                   int32_t n_wg, void* hip_stream) {
  g_err.clear();
  if (rows < 1 || !is_mult(cols, 8) || cols > 16384)
    return fail(KIE_ERR_INVALID_ARG, "need rows >= 1 and cols a multiple of 8, at most 16384");
  int rc;
  if ((rc = check_device_range(w, (size_t)rows * cols * sizeof(__half), "w"))) return rc;
  if ((rc = check_device_range(x, (size_t)cols * sizeof(float), "x"))) return rc;
  if ((rc = check_device_range(y, (size_t)rows * sizeof(float), "y"))) return rc;
  int dev = 0, n_cu = 0;
  KIE_HIP(hipGetDevice(&dev));
  KIE_HIP(hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev));
  if (n_wg < 0 || n_wg > 65536) return fail(KIE_ERR_INVALID_ARG, "n_workgroups out of range");
  const int grid = n_wg > 0 ? n_wg : n_cu;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  KIE_HIP(kie::launch_gemv(static_cast<const __half*>(w), x, y, rows, cols, grid, s));
  KIE_HIP(hipStreamSynchronize(s));
  return KIE_OK;
}

int kie_debug_barrier(int32_t n_wg, int32_t rounds, int32_t spin_limit, int32_t* violations,
                      float* ms_per_barrier, void* hip_stream) {
  g_err.clear();
  if (!violations || rounds < 1 || rounds > 1000000 || spin_limit < 0)
    return fail(KIE_ERR_INVALID_ARG, "bad barrier test arguments");
  int dev = 0, n_cu = 0, clk = 0;
  KIE_HIP(hipGetDevice(&dev));
  KIE_HIP(hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev));
  KIE_HIP(hipDeviceGetAttribute(&clk, hipDeviceAttributeWallClockRate, dev));
  const int grid = n_wg > 0 ? n_wg : n_cu;
  if (grid > n_cu) return fail(KIE_ERR_OCCUPANCY, "barrier test runs one workgroup per CU at most");
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  void* mem = nullptr;
  const size_t bar_bytes = sizeof(unsigned) * kie::kBarrierWords;
  const size_t bytes = bar_bytes + 256 + sizeof(unsigned) * (size_t)grid;
  KIE_HIP(hipMalloc(&mem, bytes));
  int rc = KIE_OK;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  unsigned* bar = static_cast<unsigned*>(mem);
  int* viol = reinterpret_cast<int*>(static_cast<char*>(mem) + bar_bytes);
  int* err = reinterpret_cast<int*>(static_cast<char*>(mem) + bar_bytes + 128);
  unsigned* slots = reinterpret_cast<unsigned*>(static_cast<char*>(mem) + bar_bytes + 256);
  do {
    if (hipMemsetAsync(mem, 0, bytes, s) != hipSuccess || hipEventCreate(&e0) != hipSuccess ||
        hipEventCreate(&e1) != hipSuccess || hipEventRecord(e0, s) != hipSuccess) {
      rc = fail(KIE_ERR_HIP, "barrier test setup failed");
      break;
    }
    const long long ticks = 5000LL * (clk > 0 ? clk : 100000);
    hipError_t e = kie::launch_barrier_test(bar, slots, viol, err, grid, rounds, ticks, spin_limit, s);
    if (e != hipSuccess) {
      rc = fail(KIE_ERR_HIP, std::string("barrier test launch: ") + hipGetErrorString(e));
      break;
    }
    int host[2] = {0, 0};
    float ms = 0.f;
    if (hipEventRecord(e1, s) != hipSuccess || hipStreamSynchronize(s) != hipSuccess ||
        hipMemcpy(&host[0], viol, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(&host[1], err, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess ||
        hipEventElapsedTime(&ms, e0, e1) != hipSuccess) {
      rc = fail(KIE_ERR_HIP, "barrier test readback failed");
      break;
    }
    *violations = host[0];
    if (ms_per_barrier) *ms_per_barrier = ms / (2.0f * rounds);
    if (host[1] == kie::kErrTimeout) rc = fail(KIE_ERR_TIMEOUT, "barrier wait timed out");
  } while (0);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  (void)hipFree(mem);
  return rc;
}

int kie_debug_stream(const void* src, void* dst, size_t bytes, int32_t n_wg, int32_t reps,
                     float* ms_per_launch, void* hip_stream) {
  return kie_debug_stream_ex(src, dst, bytes, n_wg, 8, 0, reps, ms_per_launch, hip_stream);
}

int kie_debug_stream_ex(const void* src, void* dst, size_t bytes, int32_t n_wg, int32_t depth,
                        int32_t kind, int32_t reps, float* ms_per_launch, void* hip_stream) {
  g_err.clear();
  if (bytes == 0 || bytes % 16 != 0 || reps < 1 || reps > 10000 || n_wg < 0 || n_wg > 65536)
    return fail(KIE_ERR_INVALID_ARG, "need bytes a positive multiple of 16, 1 <= reps <= 10000");
  if (depth != 1 && depth != 2 && depth != 4 && depth != 8 && depth != 16)
    return fail(KIE_ERR_INVALID_ARG, "depth must be 1, 2, 4, 8 or 16");
  if (kind < 0 || kind > 2) return fail(KIE_ERR_INVALID_ARG, "kind must be 0, 1 or 2");
  if (kind == 2 && bytes >= (size_t(1) << 32))
    return fail(KIE_ERR_INVALID_ARG, "buffer loads (kind 2) address less than 4 GiB");
  int rc;
  if ((rc = check_device_range(src, bytes, "src"))) return rc;
  if (dst && (rc = check_device_range(dst, bytes, "dst"))) return rc;
  int dev = 0, n_cu = 0;
  KIE_HIP(hipGetDevice(&dev));
  KIE_HIP(hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev));
  const int grid = n_wg > 0 ? n_wg : 4 * n_cu;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  void* sink = nullptr;
  KIE_HIP(hipMalloc(&sink, 256));
  hipEvent_t e0 = nullptr, e1 = nullptr;
  do {
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess ||
        hipEventRecord(e0, s) != hipSuccess) {
      rc = fail(KIE_ERR_HIP, "stream probe setup failed");
      break;
    }
    hipError_t e = hipSuccess;
    for (int r = 0; r < reps && e == hipSuccess; ++r)
      e = kie::launch_stream(src, dst, bytes, grid, depth, kind, static_cast<unsigned*>(sink), s);
    float ms = 0.f;
    if (e != hipSuccess || hipEventRecord(e1, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess || hipEventElapsedTime(&ms, e0, e1) != hipSuccess) {
      rc = fail(KIE_ERR_HIP, "stream probe launch failed");
      break;
    }
    if (ms_per_launch) *ms_per_launch = ms / (float)reps;
  } while (0);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  (void)hipFree(sink);
  return rc;
}

// ---- one decode stage at a time (test-only)
namespace {
// kie.h's KIE_STAGE_* in the staged mode's stage numbering
constexpr int kStageMap[] = {0, 1, 3, 4, 5, 6, 7, 8, 9};
constexpr int kNumStages = (int)(sizeof(kStageMap) / sizeof(kStageMap[0]));
constexpr int kSlotQkv = 0, kSlotO = 2, kSlotXO = 3, kSlotRouter = 4, kSlotU = 5, kSlotXDown = 6;

static kie::Params debug_params(const kie_handle* h) {
  kie::Params p = h->base;
  p.trace = nullptr;
  p.mode = kie::kDecode;
  p.n_steps = 1;
  p.pos0 = h->pos;
  p.epoch0 = h->dbg_epoch0;
  p.out_tokens = nullptr;
  p.out_logits = h->base.zbuf;      // the LM-head stage's logits, for kie_debug_read_act
  p.sample = 0;
  return p;
}
}  // namespace

int kie_debug_stage(kie_handle* h, int32_t stage, int32_t layer) {
  g_err.clear();
  if (!h) return fail(KIE_ERR_INVALID_ARG, "handle is NULL");
  if (h->broken) return fail(KIE_ERR_BAD_STATE, "handle is broken; call kie_reset");
  if (!h->pending) return fail(KIE_ERR_BAD_STATE, "no pending token: call kie_prefill first");
  if (stage < 0 || stage >= kNumStages) return fail(KIE_ERR_INVALID_ARG, "unknown stage");
  const bool moe = h->cfg.n_experts != 0;
  const bool ffn_stage = stage == KIE_STAGE_GATEUP || stage == KIE_STAGE_DOWN;
  const bool moe_stage = stage == KIE_STAGE_ROUTER || stage == KIE_STAGE_MOE_GATEUP || stage == KIE_STAGE_MOE_DOWN;
  if ((moe && ffn_stage) || (!moe && moe_stage))
    return fail(KIE_ERR_INVALID_ARG, moe ? "a MoE model has no dense FFN stage" : "a dense model has no MoE stage");
  if (stage == KIE_STAGE_LM_HEAD ? layer != 0 : (layer < 0 || layer >= h->cfg.n_layers))
    return fail(KIE_ERR_INVALID_ARG, "layer out of range (0 for the LM head)");
  if ((long long)h->pos + 1 > h->cfg.max_seq) return fail(KIE_ERR_CONTEXT_OVERFLOW, "no room for a decode step");
  if (stage == KIE_STAGE_QKV && layer == 0) {
    // opens a step: fresh epochs, cleared argmax slot, step counter 0
    kie::Params p = debug_params(h);
    int rc = reset_sync_words(h);
    if (rc) return rc;
    if ((rc = assign_epochs(h, p))) return rc;
    h->dbg_epoch0 = p.epoch0;
  } else if (h->dbg_epoch0 == 0) {
    return fail(KIE_ERR_BAD_STATE, "open a step with KIE_STAGE_QKV at layer 0 first");
  }
  const kie::Params p = debug_params(h);
  KIE_HIP(kie::launch_stage(p, h->lds, kStageMap[stage], layer, h->stream));
  KIE_HIP(hipStreamSynchronize(h->stream));
  int err = 0;
  KIE_HIP(hipMemcpy(&err, h->base.err, sizeof(int), hipMemcpyDeviceToHost));
  if (err != 0) {
    h->broken = true;
    return fail(KIE_ERR_HIP, "device reported error " + std::to_string(err));
  }
  return KIE_OK;
}

int kie_debug_read_act(const kie_handle* h, int32_t what, int32_t layer, void* out_host, int32_t n) {
  g_err.clear();
  if (!h || !out_host) return fail(KIE_ERR_INVALID_ARG, "handle or out is NULL");
  if (h->dbg_epoch0 == 0) return fail(KIE_ERR_BAD_STATE, "no step open (kie_debug_stage)");
  const kie::Params& b = h->base;
  const kie_config& c = h->cfg;
  const int qd = c.n_heads * c.head_dim, kd = c.n_kv_heads * c.head_dim;
  const int ucount = c.n_experts ? (c.top_k + c.n_shared_experts) * c.expert_hidden : c.ffn_hidden;
  if (layer < 0 || layer >= c.n_layers) return fail(KIE_ERR_INVALID_ARG, "layer out of range");
  auto flag = [&](int slot) { return h->dbg_epoch0 + (unsigned)layer * 8u + (unsigned)slot; };
  if (what == KIE_ACT_LOGITS || what == KIE_ACT_TOKEN) {
    const int need = what == KIE_ACT_LOGITS ? c.vocab_out : 1;
    if (n < need) return fail(KIE_ERR_INVALID_ARG, "out too small");
    if (what == KIE_ACT_LOGITS) {
      KIE_HIP(hipMemcpy(out_host, b.zbuf, sizeof(float) * c.vocab_out, hipMemcpyDeviceToHost));
    } else {
      unsigned long long key = 0;
      KIE_HIP(hipMemcpy(&key, b.amax, sizeof(key), hipMemcpyDeviceToHost));
      if (key == 0) return fail(KIE_ERR_BAD_STATE, "the LM-head stage has not run");
      *static_cast<int32_t*>(out_host) = (int32_t)(0xFFFFFFFFu - (unsigned)(key & 0xFFFFFFFFull));
    }
    return KIE_OK;
  }
  int off = 0, count = 0, slot = 0;
  bool pair = false;
  switch (what) {
    case KIE_ACT_X_ATTN: off = b.off_x; count = c.d_model; slot = kSlotXO; break;
    case KIE_ACT_X: off = b.off_x; count = c.d_model; slot = kSlotXDown; break;
    case KIE_ACT_QKV: off = b.off_qkv; count = qd + 2 * kd; slot = kSlotQkv; break;
    case KIE_ACT_O: off = b.off_o; count = qd; slot = kSlotO; pair = true; break;
    case KIE_ACT_U: off = b.off_u; count = ucount; slot = kSlotU; pair = true; break;
    case KIE_ACT_ROUTER:
      if (!c.n_experts) return fail(KIE_ERR_INVALID_ARG, "a dense model has no router");
      off = b.off_router; count = c.n_experts; slot = kSlotRouter; break;
    default: return fail(KIE_ERR_INVALID_ARG, "unknown activation");
  }
  if (n < count) return fail(KIE_ERR_INVALID_ARG, "out too small");
  const int words = pair ? count / 2 : count;
  std::vector<unsigned long long> w(words);
  KIE_HIP(hipMemcpy(w.data(), b.act + off, sizeof(unsigned long long) * words, hipMemcpyDeviceToHost));
  float* out = static_cast<float*>(out_host);
  const unsigned f = flag(slot);
  for (int i = 0; i < words; ++i) {
    const unsigned lo = (unsigned)w[i], hi = (unsigned)(w[i] >> 32);
    if (pair) {
      if ((hi >> 16) != f % 65535u + 1u)
        return fail(KIE_ERR_BAD_STATE, "activation word " + std::to_string(i) + " is not from that stage");
      const unsigned a = lo & 0xFFFFFFu, bb = (lo >> 24) | ((hi & 0xFFFFu) << 8);
      unsigned ua = a << 8, ub = bb << 8;
      std::memcpy(&out[2 * i], &ua, 4);
      std::memcpy(&out[2 * i + 1], &ub, 4);
    } else {
      if (hi != f) return fail(KIE_ERR_BAD_STATE, "activation word " + std::to_string(i) + " is not from that stage");
      std::memcpy(&out[i], &lo, 4);
    }
  }
  return KIE_OK;
}

}  // extern "C"
