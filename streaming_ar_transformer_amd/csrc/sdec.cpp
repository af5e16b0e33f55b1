// Host side of the sdec C ABI: argument checks, device buffers, the per-token launch sequence
// and its hipGraph.  Page names in citations: [talker] inferencelayer 0.2.8 src/qwen3tts_gpu.rs,
// [mimi] 0.2.1 src/mimi_gpu.rs, [pocket] 0.2.4 src/pocket_tts_gpu.rs.

#include "sdec.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"

using namespace sdec;

namespace {

// How a step's attention runs (one recorded graph each): items over chunks of the compacted
// legal slots, or (few legal slots) inside the o-projection launch.
enum StepForm { FORM_LIST = 0, FORM_SHORT = 1 };

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define HIP_TRY(expr)                                                                      \
  do {                                                                                     \
    hipError_t e_ = (expr);                                                                \
    if (e_ != hipSuccess)                                                                  \
      return fail(SDEC_E_HIP, "%s failed: %s", #expr, hipGetErrorString(e_));              \
  } while (0)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

struct sdec_handle {
  sdec_config cfg{};
  std::vector<sdec_layer_weights> layers;
  sdec_final_weights fin{};
  uint32_t ring = 0;
  uint32_t rows = 0;          // scratch rows: max(m, max_prefill)
  uint32_t n_chunks = 0;
  uint32_t chunk = 0;
  int device = 0;

  // library-owned device memory
  float* k_rings = nullptr;   // [m][L][R][Hkv][hd]
  float* v_rings = nullptr;
  uint32_t* pos_rings = nullptr;  // [m][R]
  uint32_t* legal = nullptr;      // [m][R] slots this step attends, the pushed slot first
  uint32_t* n_legal = nullptr;    // [m]
  float* xres = nullptr;      // [m][d]
  float* qkv = nullptr;       // [m][(Hq+2Hkv)hd]
  float* attn_out = nullptr;  // [m][Hq hd], or [L][m][Hq hd] with taps
  float* act = nullptr;       // [m][d_ff]
  float* part = nullptr;      // [m][Hq][n_chunks][hd] outputs, then [m][Hq][n_chunks][2] (max, sum)
  uint32_t* counters = nullptr;  // [m][Hkv]
  float* cs = nullptr;        // [hd]
  DevState* st = nullptr;
  float* tap_attn_proj = nullptr;  // [L][m][d]
  float* tap_ffn_proj = nullptr;   // [L][m][d]

  uint64_t ring_stream_stride = 0;  // floats between streams in k_rings / v_rings
  uint64_t ring_layer_stride = 0;   // floats between layers of one stream

  std::vector<GemvLaunch> plan_qkv, plan_o, plan_up, plan_down;
  // one stream, at most kShortSlots legal slots: the attention runs inside the o-projection launch
  // (no attention launch); a second graph records that plan
  bool short_ok = false;
  GemvLaunch plan_o_short{};
  int short_early_rows = 0;  // tuning override SDEC_SHORT_EARLY
  // one stream: the attention launch leaves its chunk partials and the o projection combines them
  bool attn_fused = false;
  // several streams: attention items split each stream's legal slots evenly (n_chunks per kv head)
  bool attn_split = false;
  // one stream: the step begin runs in layer 0's q/k/v launch (k_qkv_begin), which therefore sits
  // outside the recorded graphs (tuning override SDEC_BEGIN_IN_QKV)
  bool begin_in_qkv = false;
  // no final norm, one stream: the last down projection writes the caller's rows itself (no end
  // launch; tuning override SDEC_END_IN_DOWN)
  bool end_in_down = false;
  // the same for prefill blocks (any block width)
  bool prefill_end_in_down = false;

  hipStream_t cap_stream = nullptr;
  hipGraphExec_t exec[2] = {nullptr, nullptr};  // one recorded graph per StepForm
  bool graph_ready = false;
  uint32_t last_form = 0;

  bool has_next = false;
  uint32_t next_pos = 0;
  // first position of the stream's history when known (every legal position lies in
  // [hist_start, pos]); kNoHistory: set by the next step; hist_known false after an import
  bool hist_known = true;
  uint32_t hist_start = 0xFFFFFFFFu;
};

namespace {

struct Alloc {
  std::vector<void*> ptrs;
  int code = SDEC_OK;
  template <class T>
  T* get(size_t count) {
    if (code != SDEC_OK) return nullptr;
    void* p = nullptr;
    size_t bytes = count * sizeof(T);
    if (bytes == 0) bytes = 16;
    hipError_t e = hipMalloc(&p, bytes);
    if (e != hipSuccess) {
      code = fail(SDEC_E_NOMEM, "hipMalloc of %zu bytes failed: %s", bytes, hipGetErrorString(e));
      return nullptr;
    }
    ptrs.push_back(p);
    return static_cast<T*>(p);
  }
};

void free_handle_memory(sdec_handle* h) {
  void* ps[] = {h->k_rings, h->v_rings, h->pos_rings, h->legal, h->n_legal, h->xres, h->qkv, h->attn_out,
                h->act, h->part, h->counters, h->cs, h->st, h->tap_attn_proj, h->tap_ffn_proj};
  for (void* p : ps)
    if (p) (void)hipFree(p);
}

int validate_config(const sdec_config* c, uint32_t ring) {
  if (c->n_layers < 1) return fail(SDEC_E_ARG, "n_layers must be >= 1");
  if (c->d_model == 0 || c->d_model % 4) return fail(SDEC_E_ARG, "d_model must be a positive multiple of 4");
  if (c->d_ff == 0 || c->d_ff % 4) return fail(SDEC_E_ARG, "d_ff must be a positive multiple of 4");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(SDEC_E_ARG, "head_dim %u unsupported (64 or 128)", c->head_dim);
  if (c->n_kv_heads == 0 || c->n_q_heads == 0 || c->n_q_heads % c->n_kv_heads)
    return fail(SDEC_E_ARG, "n_q_heads must be a positive multiple of n_kv_heads");
  const uint32_t group = c->n_q_heads / c->n_kv_heads;
  if (group != 1 && group != 2 && group != 4)
    return fail(SDEC_E_ARG, "GQA group %u unsupported (1, 2 or 4)", group);
  if (c->m < 1 || c->m > kMaxM) return fail(SDEC_E_ARG, "m must be in [1, %d]", kMaxM);
  if (c->max_prefill > static_cast<uint32_t>(kMaxPrefill))
    return fail(SDEC_E_ARG, "max_prefill must be in [0, %d]", kMaxPrefill);
  if (c->max_prefill > 1 && c->m != 1)
    return fail(SDEC_E_ARG, "a stack with max_prefill > 1 must have one stream (m == 1)");
  if (c->norm > SDEC_NORM_LAYER) return fail(SDEC_E_ARG, "bad norm kind");
  if (c->rope > SDEC_ROPE_INTERLEAVED) return fail(SDEC_E_ARG, "bad rope kind");
  if (c->ffn > SDEC_FFN_GELU_ERF) return fail(SDEC_E_ARG, "bad ffn kind");
  if (!(c->rope_theta > 0.0)) return fail(SDEC_E_ARG, "rope_theta must be positive");
  if (ring < 1) return fail(SDEC_E_ARG, "ring_slots must be >= 1");
  if (c->window < 1 || c->window > ring)
    return fail(SDEC_E_ARG, "window %u must be in [1, ring_slots=%u]", c->window, ring);
  if (c->unbounded && c->window != ring)
    return fail(SDEC_E_ARG, "an unbounded stack needs window == ring_slots");
  const uint32_t rows = c->m > c->max_prefill ? c->m : c->max_prefill;
  const uint32_t mp = rows <= 1 ? 1 : rows <= 2 ? 2 : rows <= 4 ? 4 : rows <= 8 ? 8 : 16;
  if (static_cast<uint64_t>(mp) * c->d_model * sizeof(float) > 65536)
    return fail(SDEC_E_ARG, "%u rows of d_model=%u exceed the 64 KiB staging tile", rows,
                c->d_model);
  return SDEC_OK;
}

int check_vec(const float* p, const char* name, uint32_t layer) {
  if (p == nullptr) return fail(SDEC_E_ARG, "layer %u: %s is NULL", layer, name);
  if (!aligned16(p)) return fail(SDEC_E_ARG, "layer %u: %s is not 16-byte aligned", layer, name);
  return SDEC_OK;
}

int validate_weights(const sdec_config* c, const sdec_layer_weights* L,
                     const sdec_final_weights* fw) {
  for (uint32_t l = 0; l < c->n_layers; ++l) {
    const sdec_layer_weights& w = L[l];
    int r;
#define REQ(field) \
  if ((r = check_vec(w.field, #field, l)) != SDEC_OK) return r;
    REQ(attn_norm_w) REQ(wq) REQ(wk) REQ(wv) REQ(wo) REQ(ffn_norm_w) REQ(w_up) REQ(w_down)
    if (c->norm == SDEC_NORM_LAYER) { REQ(attn_norm_b) REQ(ffn_norm_b) }
    if (c->qk_norm) { REQ(q_norm) REQ(k_norm) }
    if (c->layer_scale) { REQ(ls1) REQ(ls2) }
    if (c->ffn == SDEC_FFN_SWIGLU) { REQ(w_gate) }
#undef REQ
  }
  if (c->final_norm) {
    if (!fw || !fw->norm_w || !aligned16(fw->norm_w))
      return fail(SDEC_E_ARG, "final_norm needs a 16-byte aligned norm_w");
    if (c->norm == SDEC_NORM_LAYER && (!fw->norm_b || !aligned16(fw->norm_b)))
      return fail(SDEC_E_ARG, "final LayerNorm needs a 16-byte aligned norm_b");
  }
  return SDEC_OK;
}

// Device pointer of stream s, layer l in a ring array.
inline float* ring_at(const sdec_handle* h, float* base, uint32_t s, uint32_t l) {
  return base + s * h->ring_stream_stride + l * h->ring_layer_stride;
}

// Which launch of the per-layer sequence is about to be enqueued (for per-kernel timing).
struct Hooks {
  hipEvent_t* ev = nullptr;  // pairs
  int* kinds = nullptr;
  int n = 0;
  int cap = 0;
};

// The events of a profiled launch are stamped by the launch itself, around the kernel's execution.
int hook_pre(Hooks* k, hipStream_t s) {
  (void)s;
  if (!k) return SDEC_OK;
  if (k->n >= k->cap) return fail(SDEC_E_ARG, "profile event buffer too small");
  set_launch_events(k->ev[2 * k->n], k->ev[2 * k->n + 1]);
  return SDEC_OK;
}
int hook_post(Hooks* k, hipStream_t s, int kind) {
  (void)s;
  if (!k) return SDEC_OK;
  set_launch_events(nullptr, nullptr);
  k->kinds[k->n++] = kind;
  return SDEC_OK;
}

#define LAUNCH(hooks, stream, kind, call)                                               \
  do {                                                                                  \
    int r_ = hook_pre(hooks, stream);                                                   \
    if (r_ != SDEC_OK) return r_;                                                       \
    hipError_t e_ = (call);                                                             \
    if (e_ != hipSuccess) {                                                             \
      set_launch_events(nullptr, nullptr);                                              \
      return fail(SDEC_E_HIP, "launch of %s failed: %s", #kind, hipGetErrorString(e_)); \
    }                                                                                   \
    r_ = hook_post(hooks, stream, kind);                                                \
    if (r_ != SDEC_OK) return r_;                                                       \
  } while (0)

// The per-token launch sequence of every layer ([talker] build_step_plan; [mimi]
// Builder::transformer_shaped), on `s`.  Position-dependent values come from h->st.
// The normed q/k/v projection of layer l, reading the residual stream.
GemvArgs qkv_args(sdec_handle* h, uint32_t l) {
  const sdec_config& c = h->cfg;
  const sdec_layer_weights& w = h->layers[l];
  const uint32_t qw = c.n_q_heads * c.head_dim, kw = c.n_kv_heads * c.head_dim;
  const uint32_t nqkv = qw + 2 * kw;
  GemvArgs g{};
  g.w[0] = w.wq; g.w[1] = w.wk; g.w[2] = w.wv;
  g.seg_end[0] = qw; g.seg_end[1] = qw + kw; g.seg_end[2] = nqkv;
  g.n_rows = nqkv; g.k = c.d_model; g.m = c.m;
  g.x = h->xres; g.x_stride = c.d_model;
  g.norm_w = w.attn_norm_w; g.norm_b = w.attn_norm_b; g.eps = c.norm_eps;
  g.y = h->qkv; g.y_stride = nqkv;
  return g;
}

// first_qkv false: layer 0's q/k/v projection already ran (with the step begin, k_qkv_begin).
int enqueue_layers(sdec_handle* h, hipStream_t s, Hooks* hk, StepForm form = FORM_LIST,
                   bool first_qkv = true) {
  const bool short_attn = form == FORM_SHORT;
  const sdec_config& c = h->cfg;
  const uint32_t hd = c.head_dim, hq = c.n_q_heads, hkv = c.n_kv_heads;
  const uint32_t qw = hq * hd, kw = hkv * hd, nqkv = qw + 2 * kw;
  const bool taps = (c.flags & SDEC_FLAG_TAPS) != 0;
  const int pro = c.norm == SDEC_NORM_RMS ? PRO_RMS : PRO_LN;
  for (uint32_t l = 0; l < c.n_layers; ++l) {
    const sdec_layer_weights& w = h->layers[l];
    // attention norm + q/k/v projections
    if (l > 0 || first_qkv) {
      const GemvArgs g = qkv_args(h, l);
      LAUNCH(hk, s, SDEC_K_QKV, launch_gemv(g, h->plan_qkv[l], s));
    }
    float* att = taps ? h->attn_out + static_cast<size_t>(l) * c.m * qw : h->attn_out;
    if (short_attn) {
      // attention (qk-norm, rope, push, softmax over the few legal slots) inside the o launch
      GemvArgs o{};
      o.w[0] = o.w[1] = o.w[2] = w.wo;
      o.seg_end[0] = o.seg_end[1] = o.seg_end[2] = c.d_model;
      o.n_rows = c.d_model; o.k = qw; o.m = 1;
      o.x_tap = taps ? att : nullptr;
      o.res = h->xres; o.res_stride = c.d_model; o.ls = c.layer_scale ? w.ls1 : nullptr;
      o.tap = taps ? h->tap_attn_proj + static_cast<size_t>(l) * c.d_model : nullptr;
      o.tap_stride = c.d_model;
      ShortAttnArgs& sa = o.sa;
      sa.qkv = h->qkv;
      sa.q_norm = c.qk_norm ? w.q_norm : nullptr; sa.k_norm = c.qk_norm ? w.k_norm : nullptr;
      sa.eps = c.qk_norm_eps; sa.rope_style = c.rope == SDEC_ROPE_HALF ? 0 : 1; sa.cs = h->cs;
      sa.k_ring = ring_at(h, h->k_rings, 0, l); sa.v_ring = ring_at(h, h->v_rings, 0, l);
      sa.legal = h->legal; sa.n_legal = h->n_legal; sa.st = h->st;
      sa.n_q_heads = hq; sa.n_kv_heads = hkv; sa.ring = h->ring;
      sa.early_rows = h->short_early_rows;
      LAUNCH(hk, s, SDEC_K_O, launch_gemv(o, h->plan_o_short, s));
    } else {
    // ring attention; it also finishes this step's q/k (qk-norm, rope) and pushes k/v
    AttnArgs aa{};
    aa.qkv = h->qkv; aa.qkv_stride = nqkv;
    aa.q_norm = c.qk_norm ? w.q_norm : nullptr; aa.k_norm = c.qk_norm ? w.k_norm : nullptr;
    aa.eps = c.qk_norm_eps; aa.rope_style = c.rope == SDEC_ROPE_HALF ? 0 : 1; aa.cs = h->cs;
    aa.push = 1;
    aa.k_ring = ring_at(h, h->k_rings, 0, l); aa.v_ring = ring_at(h, h->v_rings, 0, l);
    aa.ring_stream_stride = h->ring_stream_stride;
    aa.legal = h->legal; aa.n_legal = h->n_legal;
    aa.out = att; aa.part = h->part; aa.counters = h->counters;
    aa.m = c.m; aa.n_q_heads = hq; aa.n_kv_heads = hkv; aa.head_dim = hd; aa.ring = h->ring;
    aa.chunk = h->chunk; aa.n_chunks = h->n_chunks; aa.st = h->st;
    aa.partials_only = h->attn_fused ? 1 : 0;
    aa.split = h->attn_split ? 1 : 0;
    LAUNCH(hk, s, SDEC_K_ATTENTION, launch_attention(aa, s));
    // o projection + (LayerScale) residual; with the fused combine its prologue finishes the
    // attention output from the chunk partials (and copies it to the tap)
    GemvArgs o{};
    o.w[0] = o.w[1] = o.w[2] = w.wo;
    o.seg_end[0] = o.seg_end[1] = o.seg_end[2] = c.d_model;
    o.n_rows = c.d_model; o.k = qw; o.m = c.m; o.x = att; o.x_stride = qw;
    if (h->attn_fused) {  // x (= att) still carries a single chunk's output
      o.part = h->part; o.n_legal = h->n_legal;
      o.chunk = h->chunk; o.n_chunks = h->n_chunks; o.head_dim = hd;
      o.x_tap = taps ? att : nullptr;
    }
    o.res = h->xres; o.res_stride = c.d_model; o.ls = c.layer_scale ? w.ls1 : nullptr;
    o.tap = taps ? h->tap_attn_proj + static_cast<size_t>(l) * c.m * c.d_model : nullptr;
    o.tap_stride = c.d_model;
    LAUNCH(hk, s, SDEC_K_O, launch_gemv(o, h->plan_o[l], s));
    }
    // FFN norm + up projection(s) + activation
    GemvArgs u{};
    if (c.ffn == SDEC_FFN_SWIGLU) {
      u.w[0] = w.w_gate; u.w[1] = w.w_up; u.w[2] = w.w_up;
    } else {
      u.w[0] = u.w[1] = u.w[2] = w.w_up;
    }
    u.seg_end[0] = u.seg_end[1] = u.seg_end[2] = c.d_ff;
    u.n_rows = c.d_ff; u.k = c.d_model; u.m = c.m; u.x = h->xres; u.x_stride = c.d_model;
    u.norm_w = w.ffn_norm_w; u.norm_b = w.ffn_norm_b; u.eps = c.norm_eps;
    u.y = h->act; u.y_stride = c.d_ff;
    (void)pro;
    LAUNCH(hk, s, SDEC_K_FFN_UP, launch_gemv(u, h->plan_up[l], s));
    // down projection + (LayerScale) residual
    GemvArgs dn{};
    dn.w[0] = dn.w[1] = dn.w[2] = w.w_down;
    dn.seg_end[0] = dn.seg_end[1] = dn.seg_end[2] = c.d_model;
    dn.n_rows = c.d_model; dn.k = c.d_ff; dn.m = c.m; dn.x = h->act; dn.x_stride = c.d_ff;
    dn.res = h->xres; dn.res_stride = c.d_model; dn.ls = c.layer_scale ? w.ls2 : nullptr;
    dn.tap = taps ? h->tap_ffn_proj + static_cast<size_t>(l) * c.m * c.d_model : nullptr;
    dn.tap_stride = c.d_model;
    if (h->end_in_down && l + 1 == c.n_layers) {  // no final norm: the caller's rows directly
      dn.res_in = h->xres;
      dn.res_st = h->st;
    }
    LAUNCH(hk, s, SDEC_K_FFN_DOWN, launch_gemv(dn, h->plan_down[l], s));
  }
  return SDEC_OK;
}

// The attention form of this step, from a bound on its legal slots: the legal positions are
// distinct and lie in (pos - window, pos], in the stream's history [hist_start, pos] when it is
// known (else [0, pos]), and in the R ring slots.  At most kShortSlots: the short form, else the
// legal-list form.  Also records where the stream's history starts.
StepForm step_form(sdec_handle* h, uint32_t pos, uint32_t first) {
  if (first || (h->hist_known && h->hist_start == 0xFFFFFFFFu)) {
    h->hist_known = true;
    h->hist_start = pos;
  }
  const uint64_t span = h->hist_known ? static_cast<uint64_t>(pos) - h->hist_start + 1
                                      : static_cast<uint64_t>(pos) + 1;
  uint64_t bound = span < h->cfg.window ? span : h->cfg.window;
  if (bound > h->ring) bound = h->ring;
  if (h->short_ok && bound <= kShortSlots) return FORM_SHORT;
  return FORM_LIST;
}

int check_step(sdec_handle* h, const float* x, uint32_t pos, uint32_t first) {
  if (!h) return fail(SDEC_E_ARG, "null handle");
  if (!x || !aligned16(x)) return fail(SDEC_E_ARG, "x must be a 16-byte aligned device pointer");
  if (pos == kInvalidPos) return fail(SDEC_E_ARG, "pos 0xFFFFFFFF is the empty-slot marker");
  if (!first && h->has_next && pos != h->next_pos)
    return fail(SDEC_E_POS, "step pos %u != next position %u (positions must be contiguous)",
                pos, h->next_pos);
  if (h->cfg.unbounded && pos >= h->ring)
    return fail(SDEC_E_CAPACITY, "position %u exceeds the %u-slot ring of an unbounded stack",
                pos, h->ring);
  return SDEC_OK;
}

int enqueue_begin(sdec_handle* h, float* x, uint32_t pos, uint32_t first, hipStream_t s,
                  Hooks* hk) {
  const sdec_config& c = h->cfg;
  BeginArgs b{};
  b.x_in = x; b.xres = h->xres; b.d = c.d_model; b.pos_rings = h->pos_rings;
  b.legal = h->legal; b.n_legal = h->n_legal;
  b.m = c.m; b.ring = h->ring; b.window = c.window; b.pos = pos; b.first = first ? 1u : 0u;
  b.cs = h->cs; b.x_out = x;
  b.head_dim = c.head_dim; b.theta = c.rope_theta; b.st = h->st;
  LAUNCH(hk, s, SDEC_K_BEGIN, launch_begin(b, s));
  return SDEC_OK;
}

// The step begin together with layer 0's q/k/v projection, which reads the caller's row.
int enqueue_qkv_begin(sdec_handle* h, float* x, uint32_t pos, uint32_t first, hipStream_t s,
                      Hooks* hk) {
  const sdec_config& c = h->cfg;
  QkvBeginArgs a{};
  BeginArgs& b = a.b;
  b.x_in = x; b.xres = h->xres; b.d = c.d_model; b.pos_rings = h->pos_rings;
  b.legal = h->legal; b.n_legal = h->n_legal;
  b.m = c.m; b.ring = h->ring; b.window = c.window; b.pos = pos; b.first = first ? 1u : 0u;
  b.cs = h->cs; b.x_out = x;
  b.head_dim = c.head_dim; b.theta = c.rope_theta; b.st = h->st;
  a.g = qkv_args(h, 0);
  a.g.x = x;
  a.gemv_wgs = h->plan_qkv[0].grid;
  LAUNCH(hk, s, SDEC_K_QKV, launch_qkv_begin(a, h->plan_qkv[0], s));
  return SDEC_OK;
}

int enqueue_step_begin(sdec_handle* h, float* x, uint32_t pos, uint32_t first, hipStream_t s,
                       Hooks* hk) {
  return h->begin_in_qkv ? enqueue_qkv_begin(h, x, pos, first, s, hk)
                         : enqueue_begin(h, x, pos, first, s, hk);
}

// x null: the output rows the step begin recorded in the device state (so the launch can sit in
// the recorded graph)
int enqueue_end(sdec_handle* h, float* x, hipStream_t s, Hooks* hk) {
  const sdec_config& c = h->cfg;
  EndArgs e{};
  e.xres = h->xres; e.x_out = x; e.st = h->st; e.m = c.m; e.d = c.d_model;
  e.norm = c.final_norm ? (c.norm == SDEC_NORM_RMS ? PRO_RMS : PRO_LN) : -1;
  e.w = h->fin.norm_w; e.b = h->fin.norm_b; e.eps = c.norm_eps;
  LAUNCH(hk, s, SDEC_K_END, launch_end(e, s));
  return SDEC_OK;
}

// A prefill block of t rows at positions pos .. pos+t-1 of stream 0 ([talker] TalkerGpu::prefill
// → forward_rows): the rows share stream 0's rings, every row's K/V is pushed before attention,
// and the attention launch treats the rows as t streams with their own legal lists and rope
// tables over one ring.
int enqueue_prefill(sdec_handle* h, float* x, uint32_t pos, uint32_t t, uint32_t first,
                    hipStream_t s, Hooks* hk) {
  const sdec_config& c = h->cfg;
  const uint32_t hd = c.head_dim, hq = c.n_q_heads, hkv = c.n_kv_heads;
  const uint32_t qw = hq * hd, kw = hkv * hd, nqkv = qw + 2 * kw;
  const int pro = c.norm == SDEC_NORM_RMS ? PRO_RMS : PRO_LN;
  BeginArgs b{};
  b.x_in = x; b.xres = h->xres; b.d = c.d_model; b.pos_rings = h->pos_rings;
  b.legal = h->legal; b.n_legal = h->n_legal;
  b.m = t; b.ring = h->ring; b.window = c.window; b.pos = pos; b.first = first ? 1u : 0u;
  b.cs = h->cs; b.head_dim = hd; b.theta = c.rope_theta; b.st = h->st;
  LAUNCH(hk, s, SDEC_K_BEGIN, launch_begin_rows(b, s));
  const GemvLaunch p_qkv = plan_gemv(pro, EPI_STORE, nqkv, c.d_model, t);
  const GemvLaunch p_o = plan_gemv(PRO_NONE, EPI_RESIDUAL, c.d_model, qw, t);
  const GemvLaunch p_up = plan_gemv(pro, c.ffn == SDEC_FFN_SWIGLU ? EPI_SWIGLU : EPI_GELU, c.d_ff,
                                    c.d_model, t);
  const GemvLaunch p_down = plan_gemv(PRO_NONE, EPI_RESIDUAL, c.d_model, c.d_ff, t);
  for (uint32_t l = 0; l < c.n_layers; ++l) {
    const sdec_layer_weights& w = h->layers[l];
    GemvArgs g{};
    g.w[0] = w.wq; g.w[1] = w.wk; g.w[2] = w.wv;
    g.seg_end[0] = qw; g.seg_end[1] = qw + kw; g.seg_end[2] = nqkv;
    g.n_rows = nqkv; g.k = c.d_model; g.m = t;
    g.x = h->xres; g.x_stride = c.d_model;
    g.norm_w = w.attn_norm_w; g.norm_b = w.attn_norm_b; g.eps = c.norm_eps;
    g.y = h->qkv; g.y_stride = nqkv;
    LAUNCH(hk, s, SDEC_K_QKV, launch_gemv(g, p_qkv, s));
    PushArgs pa{};
    pa.qkv = h->qkv; pa.qkv_stride = nqkv;
    pa.k_norm = c.qk_norm ? w.k_norm : nullptr; pa.eps = c.qk_norm_eps;
    pa.rope_style = c.rope == SDEC_ROPE_HALF ? 0 : 1; pa.cs = h->cs;
    pa.k_ring = ring_at(h, h->k_rings, 0, l); pa.v_ring = ring_at(h, h->v_rings, 0, l);
    pa.m = t; pa.n_q_heads = hq; pa.n_kv_heads = hkv; pa.head_dim = hd; pa.ring = h->ring;
    pa.pos = pos;
    LAUNCH(hk, s, SDEC_K_ATTENTION, launch_push(pa, s));
    AttnArgs aa{};
    aa.qkv = h->qkv; aa.qkv_stride = nqkv;
    aa.q_norm = c.qk_norm ? w.q_norm : nullptr; aa.k_norm = nullptr;
    aa.eps = c.qk_norm_eps; aa.rope_style = pa.rope_style; aa.cs = h->cs; aa.cs_stride = hd;
    aa.push = 0;
    aa.k_ring = pa.k_ring; aa.v_ring = pa.v_ring;
    aa.ring_stream_stride = 0;  // every row reads stream 0's rings
    aa.legal = h->legal; aa.n_legal = h->n_legal;
    aa.out = h->attn_out; aa.part = h->part; aa.counters = h->counters;
    aa.m = t; aa.n_q_heads = hq; aa.n_kv_heads = hkv; aa.head_dim = hd; aa.ring = h->ring;
    aa.chunk = h->chunk; aa.n_chunks = h->n_chunks; aa.st = nullptr; aa.partials_only = 0;
    {
      // a block's rows attend with 256-slot chunks: half the items of the step's 128 and no merge
      // below 256 legal slots (blocks of 8 on the talker: 1.84 vs 2.10 ms from position 0, 2.16 vs
      // 2.54 ms from 1792).  At most one slot per thread in the item's list, and never more items
      // than the partial buffers hold (they are sized for the step's chunks).  Tuning override:
      // SDEC_PREFILL_CHUNK.
      const char* ev = std::getenv("SDEC_PREFILL_CHUNK");
      const uint32_t pc = ev && *ev ? static_cast<uint32_t>(atoi(ev)) : 256u;
      if (pc >= h->chunk && pc <= 256 && pc % 64 == 0) {
        aa.chunk = pc;
        aa.n_chunks = (h->ring + pc - 1) / pc;
      }
    }
    LAUNCH(hk, s, SDEC_K_ATTENTION, launch_attention(aa, s));
    GemvArgs o{};
    o.w[0] = o.w[1] = o.w[2] = w.wo;
    o.seg_end[0] = o.seg_end[1] = o.seg_end[2] = c.d_model;
    o.n_rows = c.d_model; o.k = qw; o.m = t; o.x = h->attn_out; o.x_stride = qw;
    o.res = h->xres; o.res_stride = c.d_model; o.ls = c.layer_scale ? w.ls1 : nullptr;
    LAUNCH(hk, s, SDEC_K_O, launch_gemv(o, p_o, s));
    GemvArgs u{};
    if (c.ffn == SDEC_FFN_SWIGLU) {
      u.w[0] = w.w_gate; u.w[1] = w.w_up; u.w[2] = w.w_up;
    } else {
      u.w[0] = u.w[1] = u.w[2] = w.w_up;
    }
    u.seg_end[0] = u.seg_end[1] = u.seg_end[2] = c.d_ff;
    u.n_rows = c.d_ff; u.k = c.d_model; u.m = t; u.x = h->xres; u.x_stride = c.d_model;
    u.norm_w = w.ffn_norm_w; u.norm_b = w.ffn_norm_b; u.eps = c.norm_eps;
    u.y = h->act; u.y_stride = c.d_ff;
    LAUNCH(hk, s, SDEC_K_FFN_UP, launch_gemv(u, p_up, s));
    GemvArgs dn{};
    dn.w[0] = dn.w[1] = dn.w[2] = w.w_down;
    dn.seg_end[0] = dn.seg_end[1] = dn.seg_end[2] = c.d_model;
    dn.n_rows = c.d_model; dn.k = c.d_ff; dn.m = t; dn.x = h->act; dn.x_stride = c.d_ff;
    dn.res = h->xres; dn.res_stride = c.d_model; dn.ls = c.layer_scale ? w.ls2 : nullptr;
    if (h->prefill_end_in_down && l + 1 == c.n_layers) {  // no final norm: the caller's rows
      dn.res_in = h->xres;
      dn.res = x;
    }
    LAUNCH(hk, s, SDEC_K_FFN_DOWN, launch_gemv(dn, p_down, s));
  }
  if (h->prefill_end_in_down) return SDEC_OK;
  EndArgs e{};
  e.xres = h->xres; e.x_out = x; e.m = t; e.d = c.d_model;
  e.norm = c.final_norm ? (c.norm == SDEC_NORM_RMS ? PRO_RMS : PRO_LN) : -1;
  e.w = h->fin.norm_w; e.b = h->fin.norm_b; e.eps = c.norm_eps;
  LAUNCH(hk, s, SDEC_K_END, launch_end(e, s));
  return SDEC_OK;
}

int clear_state(sdec_handle* h, hipStream_t s) {
  const sdec_config& c = h->cfg;
  const uint64_t nkv = static_cast<uint64_t>(c.m) * c.n_layers * h->ring * c.n_kv_heads * c.head_dim;
  HIP_TRY(launch_fill_f32(h->k_rings, 0.f, nkv, s));
  HIP_TRY(launch_fill_f32(h->v_rings, 0.f, nkv, s));
  HIP_TRY(launch_fill_u32(h->pos_rings, kInvalidPos, static_cast<uint64_t>(c.m) * h->ring, s));
  HIP_TRY(launch_fill_u32(h->counters, 0u, static_cast<uint64_t>(h->rows) * c.n_kv_heads, s));
  return SDEC_OK;
}

// One-shot ring attention (sdec_ring_attention and its variant without allocation): argument
// checks, the scratch each call needs, and the launches.
int check_ring_attention(const float* q, const float* k_ring, const float* v_ring,
                         const uint32_t* pos_ring, const float* out, uint32_t m,
                         uint32_t n_q_heads, uint32_t n_kv_heads, uint32_t head_dim,
                         uint32_t ring_slots, uint32_t window) {
  if (!q || !k_ring || !v_ring || !pos_ring || !out) return fail(SDEC_E_ARG, "null pointer");
  if (!aligned16(q) || !aligned16(k_ring) || !aligned16(v_ring))
    return fail(SDEC_E_ARG, "q and the rings must be 16-byte aligned");
  if (head_dim != 64 && head_dim != 128) return fail(SDEC_E_ARG, "head_dim must be 64 or 128");
  if (!n_kv_heads || !n_q_heads || n_q_heads % n_kv_heads) return fail(SDEC_E_ARG, "bad heads");
  const uint32_t group = n_q_heads / n_kv_heads;
  if (group != 1 && group != 2 && group != 4) return fail(SDEC_E_ARG, "GQA group must be 1, 2 or 4");
  if (m < 1 || m > static_cast<uint32_t>(kMaxM) || ring_slots < 1 || window < 1)
    return fail(SDEC_E_ARG, "bad m, ring_slots or window");
  return SDEC_OK;
}

struct OneShotSizes {
  uint32_t chunk, n_chunks;
  size_t part;      // floats: chunk partials [m][Hq][n_chunks][hd + 2]
  size_t counters;  // words: [m][Hkv]
  size_t legal;     // words: legal-slot lists [m][R], then the counts [m]
};

OneShotSizes one_shot_sizes(uint32_t m, uint32_t n_q_heads, uint32_t n_kv_heads,
                            uint32_t head_dim, uint32_t ring_slots) {
  OneShotSizes z;
  z.chunk = attention_chunk(head_dim);
  z.n_chunks = (ring_slots + z.chunk - 1) / z.chunk;
  z.part = static_cast<size_t>(m) * n_q_heads * z.n_chunks * (head_dim + 2);
  z.counters = static_cast<size_t>(m) * n_kv_heads;
  z.legal = static_cast<size_t>(m) * ring_slots + m;
  return z;
}

// Needs counters [m][Hkv] at zero; leaves them at zero.
int enqueue_ring_attention(const float* q, const float* k_ring, const float* v_ring,
                           const uint32_t* pos_ring, float* out, uint32_t m, uint32_t n_q_heads,
                           uint32_t n_kv_heads, uint32_t head_dim, uint32_t ring_slots,
                           uint32_t window, uint32_t pos, float* part, uint32_t* counters,
                           uint32_t* legal, hipStream_t s) {
  const OneShotSizes z = one_shot_sizes(m, n_q_heads, n_kv_heads, head_dim, ring_slots);
  uint32_t* n_legal = legal + static_cast<size_t>(m) * ring_slots;
  HIP_TRY(launch_compact_legal(pos_ring, m, ring_slots, pos, window, legal, n_legal, s));
  AttnArgs a{};
  a.qkv = q; a.qkv_stride = n_q_heads * head_dim;
  a.q_norm = a.k_norm = nullptr; a.cs = nullptr; a.push = 0;
  a.k_ring = const_cast<float*>(k_ring); a.v_ring = const_cast<float*>(v_ring);
  a.ring_stream_stride = static_cast<uint64_t>(ring_slots) * n_kv_heads * head_dim;
  a.legal = legal; a.n_legal = n_legal; a.out = out; a.part = part;
  a.counters = counters; a.m = m; a.n_q_heads = n_q_heads; a.n_kv_heads = n_kv_heads;
  a.head_dim = head_dim; a.ring = ring_slots; a.chunk = z.chunk;
  a.n_chunks = z.n_chunks; a.st = nullptr;
  // a head with no legal slot gets zeros: the attention kernel skips items past the legal count
  HIP_TRY(launch_fill_f32(out, 0.f, static_cast<uint64_t>(m) * n_q_heads * head_dim, s));
  HIP_TRY(launch_attention(a, s));
  return SDEC_OK;
}

// Scratch of the one-shot attention variant that allocates nothing: a fixed array in device
// memory (each device the library runs on holds its own copy until the process ends).  Host code
// never uses the array's name as an address: the device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and kept here.
constexpr size_t kStaticScratchBytes = size_t(4) << 20;
constexpr int kStaticMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kStaticMaxDevices] = {};

int static_scratch(void** out) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kStaticMaxDevices)
    return fail(SDEC_E_ARG, "device %d: the static scratch serves devices 0..%d", dev,
                kStaticMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (p == nullptr) return fail(SDEC_E_HIP, "hipGetSymbolAddress(scratch) returned null");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SDEC_OK;
}

size_t align256(size_t bytes) { return (bytes + 255) / 256 * 256; }

}  // namespace

extern "C" {

const char* sdec_last_error(void) { return g_err.c_str(); }

int sdec_create(const sdec_config* cfg, const sdec_layer_weights* layers,
                const sdec_final_weights* final_weights, uint32_t ring_slots,
                sdec_handle** out) {
  g_err.clear();
  if (!cfg || !layers || !out) return fail(SDEC_E_ARG, "null argument");
  int r = validate_config(cfg, ring_slots);
  if (r != SDEC_OK) return r;
  r = validate_weights(cfg, layers, final_weights);
  if (r != SDEC_OK) return r;

  int device = 0;
  HIP_TRY(hipGetDevice(&device));
  sdec_handle* h = new sdec_handle();
  h->device = device;
  h->cfg = *cfg;
  h->layers.assign(layers, layers + cfg->n_layers);
  if (final_weights) h->fin = *final_weights;
  h->ring = ring_slots;
  const sdec_config& c = h->cfg;
  const uint32_t hd = c.head_dim, hq = c.n_q_heads, hkv = c.n_kv_heads;
  const uint32_t qw = hq * hd, kw = hkv * hd;
  h->chunk = attention_chunk(hd);
  h->n_chunks = (ring_slots + h->chunk - 1) / h->chunk;
  if (c.m > 1) {
    // several streams, each attending its own ring: the split form, a fixed number of items per
    // (stream, kv head) whatever the context length (tuning override SDEC_ATTN_ITEMS)
    const char* ev = std::getenv("SDEC_ATTN_ITEMS");
    uint32_t items = ev && *ev ? static_cast<uint32_t>(atoi(ev)) : 8u;
    const uint32_t least = (ring_slots + kAttnSplitList - 1) / kAttnSplitList;
    if (items < least) items = least;
    if (items > ring_slots) items = ring_slots;
    h->attn_split = true;
    h->n_chunks = items;
  }
  h->ring_layer_stride = static_cast<uint64_t>(ring_slots) * kw;
  h->ring_stream_stride = h->ring_layer_stride * c.n_layers;
  const bool taps = (c.flags & SDEC_FLAG_TAPS) != 0;

  // per-row scratch serves m streams of a step or the rows of a prefill block
  h->rows = c.m > c.max_prefill ? c.m : c.max_prefill;
  const size_t rows = h->rows;
  Alloc A;
  h->k_rings = A.get<float>(h->ring_stream_stride * c.m);
  h->v_rings = A.get<float>(h->ring_stream_stride * c.m);
  h->pos_rings = A.get<uint32_t>(static_cast<size_t>(c.m) * ring_slots);
  h->legal = A.get<uint32_t>(rows * ring_slots);
  h->n_legal = A.get<uint32_t>(rows);
  h->xres = A.get<float>(rows * c.d_model);
  h->qkv = A.get<float>(rows * (qw + 2 * kw));
  const size_t att_rows = taps && static_cast<size_t>(c.m) * c.n_layers > rows
                              ? static_cast<size_t>(c.m) * c.n_layers : rows;
  h->attn_out = A.get<float>(att_rows * qw);
  h->act = A.get<float>(rows * c.d_ff);
  h->part = A.get<float>(rows * hq * h->n_chunks * (hd + 2));
  h->counters = A.get<uint32_t>(rows * hkv);
  h->cs = A.get<float>(rows * hd);
  h->st = A.get<DevState>(1);
  if (taps) {
    h->tap_attn_proj = A.get<float>(static_cast<size_t>(c.n_layers) * c.m * c.d_model);
    h->tap_ffn_proj = A.get<float>(static_cast<size_t>(c.n_layers) * c.m * c.d_model);
  }
  if (A.code != SDEC_OK) {
    for (void* p : A.ptrs) (void)hipFree(p);
    delete h;
    return A.code;
  }

  // the o prologue forms chunk weights for at most kAttnMaxChunks chunks per head; longer rings
  // merge their chunks in the attention launch instead
  if (c.m == 1 && hq <= kAttnMaxHeads && h->n_chunks <= kAttnMaxChunks &&
      static_cast<size_t>(hq) * h->n_chunks <= kAttnMaxPartials) {
    const GemvLaunch fused = plan_gemv(PRO_ATTN, EPI_RESIDUAL, c.d_model, qw, c.m);
    const char* fe = std::getenv("SDEC_ATTN_COMBINE_IN_O");  // tuning override: "0" = combine in attention
    h->attn_fused = gemv_supported(fused, qw, c.m) && !(fe != nullptr && fe[0] == '0');
  }
  const char* se = std::getenv("SDEC_SHORT_ATTN");  // tuning override: "0" keeps the attention launch
  if (c.m == 1 && !(se != nullptr && se[0] == '0')) {
    h->plan_o_short = plan_attn_short_o(c.d_model, qw, hd, hq, hkv);
    h->short_ok = gemv_supported(h->plan_o_short, qw, 1);
    const char* ee = std::getenv("SDEC_SHORT_EARLY");
    h->short_early_rows = ee && *ee ? atoi(ee) : 0;
  }

  for (uint32_t l = 0; l < c.n_layers; ++l) {
    h->plan_qkv.push_back(plan_gemv(c.norm == SDEC_NORM_RMS ? PRO_RMS : PRO_LN, EPI_STORE,
                                    qw + 2 * kw, c.d_model, c.m));
    h->plan_o.push_back(plan_gemv(h->attn_fused ? PRO_ATTN : PRO_NONE, EPI_RESIDUAL, c.d_model, qw,
                                  c.m));
    h->plan_up.push_back(plan_gemv(c.norm == SDEC_NORM_RMS ? PRO_RMS : PRO_LN,
                                   c.ffn == SDEC_FFN_SWIGLU ? EPI_SWIGLU : EPI_GELU, c.d_ff,
                                   c.d_model, c.m));
    h->plan_down.push_back(plan_gemv(PRO_NONE, EPI_RESIDUAL, c.d_model, c.d_ff, c.m));
  }
  {
    const GemvLaunch& ld = h->plan_down.back();
    const char* ed = std::getenv("SDEC_END_IN_DOWN");
    h->end_in_down = c.m == 1 && !c.final_norm && !ld.stream && ld.ks == 0 &&
                     !(ed != nullptr && ed[0] == '0');
    h->prefill_end_in_down = !c.final_norm && !(ed != nullptr && ed[0] == '0');
  }
  {
    const char* bq = std::getenv("SDEC_BEGIN_IN_QKV");  // tuning override: "0" = separate begin
    h->begin_in_qkv = c.m == 1 && qkv_begin_supported(h->plan_qkv[0]) &&
                      !(bq != nullptr && bq[0] == '0');
  }


  auto bail = [&](int code) {
    if (h->cap_stream) (void)hipStreamDestroy(h->cap_stream);
    free_handle_memory(h);
    delete h;
    return code;
  };
  hipError_t e = hipStreamCreateWithFlags(&h->cap_stream, hipStreamNonBlocking);
  if (e != hipSuccess) return bail(fail(SDEC_E_HIP, "hipStreamCreate: %s", hipGetErrorString(e)));
  r = clear_state(h, h->cap_stream);
  if (r != SDEC_OK) return bail(r);
  e = hipStreamSynchronize(h->cap_stream);
  if (e != hipSuccess) return bail(fail(SDEC_E_HIP, "init: %s", hipGetErrorString(e)));

  if (!(c.flags & SDEC_FLAG_EAGER)) {
    // record the layer launches once per attention form the handle can take
    for (int pass = 0; pass < 2; ++pass) {
      if (pass == FORM_SHORT && !h->short_ok) continue;
      e = hipStreamBeginCapture(h->cap_stream, hipStreamCaptureModeThreadLocal);
      if (e != hipSuccess) return bail(fail(SDEC_E_HIP, "begin capture: %s", hipGetErrorString(e)));
      r = enqueue_layers(h, h->cap_stream, nullptr, static_cast<StepForm>(pass), !h->begin_in_qkv);
      if (r == SDEC_OK && !h->end_in_down)
        r = enqueue_end(h, nullptr, h->cap_stream, nullptr);  // the last node
      hipGraph_t graph = nullptr;
      e = hipStreamEndCapture(h->cap_stream, &graph);
      if (r != SDEC_OK) {
        if (graph) (void)hipGraphDestroy(graph);
        return bail(r);
      }
      if (e != hipSuccess) return bail(fail(SDEC_E_HIP, "end capture: %s", hipGetErrorString(e)));
      e = hipGraphInstantiate(&h->exec[pass], graph, nullptr, nullptr, 0);
      (void)hipGraphDestroy(graph);
      if (e != hipSuccess) return bail(fail(SDEC_E_HIP, "graph instantiate: %s", hipGetErrorString(e)));
    }
    h->graph_ready = true;
  }
  *out = h;
  return SDEC_OK;
}

int sdec_step(sdec_handle* h, float* x, uint32_t pos, uint32_t first, void* stream) {
  int r = check_step(h, x, pos, first);
  if (r != SDEC_OK) return r;
  hipStream_t s = static_cast<hipStream_t>(stream);
  r = enqueue_step_begin(h, x, pos, first, s, nullptr);
  if (r != SDEC_OK) return r;
  const StepForm form = step_form(h, pos, first);
  if (h->graph_ready) {  // the graph ends with the end launch
    HIP_TRY(hipGraphLaunch(h->exec[form], s));
  } else {
    r = enqueue_layers(h, s, nullptr, form, !h->begin_in_qkv);
    if (r != SDEC_OK) return r;
    if (!h->end_in_down) r = enqueue_end(h, x, s, nullptr);
    if (r != SDEC_OK) return r;
  }
  h->has_next = true;
  h->next_pos = pos + 1;
  h->last_form = form;
  return SDEC_OK;
}

int sdec_prefill(sdec_handle* h, float* x, uint32_t pos, uint32_t t, uint32_t first,
                 void* stream) {
  if (!h) return fail(SDEC_E_ARG, "null handle");
  const sdec_config& c = h->cfg;
  if (c.m != 1) return fail(SDEC_E_ARG, "prefill needs a single-stream stack (m == 1)");
  const uint32_t cap = c.max_prefill > 1 ? c.max_prefill : 1;
  if (t < 1 || t > cap) return fail(SDEC_E_ARG, "t=%u must be in [1, max_prefill=%u]", t, cap);
  int r = check_step(h, x, pos, first);
  if (r != SDEC_OK) return r;
  if (static_cast<uint64_t>(pos) + t - 1 >= kInvalidPos)
    return fail(SDEC_E_ARG, "positions up to %u + %u overflow the position ring", pos, t);
  // an append evicts position p - R; row r of the block still attends positions > pos + r - W
  if (static_cast<uint64_t>(pos) + t > h->ring &&
      static_cast<uint64_t>(h->ring) + 1 < static_cast<uint64_t>(c.window) + t)
    return fail(SDEC_E_CAPACITY,
                "a %u-row block past the first ring turn needs ring_slots >= window + %u = %u "
                "(ring_slots = %u)", t, t - 1, c.window + t - 1, h->ring);
  if (c.unbounded && static_cast<uint64_t>(pos) + t > h->ring)
    return fail(SDEC_E_CAPACITY, "positions up to %u exceed the %u-slot ring of an unbounded stack",
                pos + t - 1, h->ring);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)step_form(h, pos, first);  // records where the stream's history starts
  r = enqueue_prefill(h, x, pos, t, first, s, nullptr);
  if (r != SDEC_OK) return r;
  h->has_next = true;
  h->next_pos = pos + t;
  return SDEC_OK;
}

int sdec_step_profile(sdec_handle* h, float* x, uint32_t pos, uint32_t first, void* stream,
                      double* ms, uint32_t* calls) {
  int r = check_step(h, x, pos, first);
  if (r != SDEC_OK) return r;
  if (!ms || !calls) return fail(SDEC_E_ARG, "null timing arrays");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int cap = 2 + 5 * static_cast<int>(h->cfg.n_layers);
  std::vector<hipEvent_t> ev(2 * cap, nullptr);
  std::vector<int> kinds(cap, 0);
  for (auto& e : ev) HIP_TRY(hipEventCreate(&e));
  Hooks hk;
  hk.ev = ev.data(); hk.kinds = kinds.data(); hk.cap = cap;
  const StepForm form = step_form(h, pos, first);
  r = enqueue_step_begin(h, x, pos, first, s, &hk);
  if (r == SDEC_OK) r = enqueue_layers(h, s, &hk, form, !h->begin_in_qkv);
  if (r == SDEC_OK && !h->end_in_down) r = enqueue_end(h, x, s, &hk);
  hipError_t e = hipStreamSynchronize(s);
  if (r == SDEC_OK && e != hipSuccess) r = fail(SDEC_E_HIP, "sync: %s", hipGetErrorString(e));
  if (r == SDEC_OK) {
    for (int i = 0; i < hk.n; ++i) {
      float t = 0.f;
      e = hipEventElapsedTime(&t, ev[2 * i], ev[2 * i + 1]);
      if (e != hipSuccess) {
        r = fail(SDEC_E_HIP, "event time: %s", hipGetErrorString(e));
        break;
      }
      ms[kinds[i]] += t;
      calls[kinds[i]] += 1;
    }
    h->has_next = true;
    h->next_pos = pos + 1;
    h->last_form = form;
  }
  for (auto& ev1 : ev) (void)hipEventDestroy(ev1);
  return r;
}

int sdec_reset(sdec_handle* h, void* stream) {
  if (!h) return fail(SDEC_E_ARG, "null handle");
  int r = clear_state(h, static_cast<hipStream_t>(stream));
  if (r != SDEC_OK) return r;
  h->has_next = false;
  h->next_pos = 0;
  h->hist_known = true;
  h->hist_start = 0xFFFFFFFFu;
  return SDEC_OK;
}

int sdec_status(sdec_handle* h, uint32_t* path, uint32_t* attention) {
  if (!h) return fail(SDEC_E_ARG, "null handle");
  if (path) *path = h->graph_ready ? 0u : 1u;
  if (attention) *attention = h->attn_split ? 2u : h->last_form;
  return SDEC_OK;
}

void sdec_destroy(sdec_handle* h) {
  if (!h) return;
  (void)hipDeviceSynchronize();
  for (hipGraphExec_t g : h->exec)
    if (g) (void)hipGraphExecDestroy(g);
  if (h->cap_stream) (void)hipStreamDestroy(h->cap_stream);
  free_handle_memory(h);
  delete h;
}

int sdec_kv_view(sdec_handle* h, uint32_t stream_idx, uint32_t layer, float** k, float** v,
                 uint32_t** pos_ring) {
  if (!h) return fail(SDEC_E_ARG, "null handle");
  if (stream_idx >= h->cfg.m || layer >= h->cfg.n_layers)
    return fail(SDEC_E_ARG, "stream %u / layer %u out of range", stream_idx, layer);
  if (k) *k = ring_at(h, h->k_rings, stream_idx, layer);
  if (v) *v = ring_at(h, h->v_rings, stream_idx, layer);
  if (pos_ring) *pos_ring = h->pos_rings + static_cast<size_t>(stream_idx) * h->ring;
  return SDEC_OK;
}

int sdec_set_next_position(sdec_handle* h, uint32_t next_pos) {
  if (!h) return fail(SDEC_E_ARG, "null handle");
  if (next_pos == kInvalidPos) return fail(SDEC_E_ARG, "bad position");
  h->has_next = true;
  h->next_pos = next_pos;
  h->hist_known = false;  // the imported history may hold any positions below next_pos
  return SDEC_OK;
}

int sdec_tap_view(sdec_handle* h, uint32_t layer, uint32_t which, float** ptr) {
  if (!h || !ptr) return fail(SDEC_E_ARG, "null argument");
  if (!(h->cfg.flags & SDEC_FLAG_TAPS)) return fail(SDEC_E_ARG, "handle built without SDEC_FLAG_TAPS");
  if (layer >= h->cfg.n_layers || which > 2) return fail(SDEC_E_ARG, "tap out of range");
  const size_t md = static_cast<size_t>(h->cfg.m) * h->cfg.d_model;
  const size_t mq = static_cast<size_t>(h->cfg.m) * h->cfg.n_q_heads * h->cfg.head_dim;
  if (which == 0) *ptr = h->attn_out + layer * mq;
  else if (which == 1) *ptr = h->tap_attn_proj + layer * md;
  else *ptr = h->tap_ffn_proj + layer * md;
  return SDEC_OK;
}

int sdec_gemv(const float* w, const float* x, float* y, uint32_t n, uint32_t k, uint32_t m,
              void* stream) {
  if (!w || !x || !y) return fail(SDEC_E_ARG, "null pointer");
  if (!aligned16(w) || !aligned16(x)) return fail(SDEC_E_ARG, "w and x must be 16-byte aligned");
  if (n == 0 || k == 0 || k % 4) return fail(SDEC_E_ARG, "need n > 0 and k a positive multiple of 4");
  if (m < 1 || m > static_cast<uint32_t>(kMaxM)) return fail(SDEC_E_ARG, "m must be in [1, %d]", kMaxM);
  GemvArgs g{};
  g.w[0] = g.w[1] = g.w[2] = w;
  g.seg_end[0] = g.seg_end[1] = g.seg_end[2] = n;
  g.n_rows = n; g.k = k; g.m = m; g.x = x; g.x_stride = k; g.y = y; g.y_stride = n;
  const GemvLaunch l = plan_gemv(PRO_NONE, EPI_STORE, n, k, m);
  HIP_TRY(launch_gemv(g, l, static_cast<hipStream_t>(stream)));
  return SDEC_OK;
}

int sdec_ring_attention(const float* q, const float* k_ring, const float* v_ring,
                        const uint32_t* pos_ring, float* out, uint32_t m, uint32_t n_q_heads,
                        uint32_t n_kv_heads, uint32_t head_dim, uint32_t ring_slots,
                        uint32_t window, uint32_t pos, void* stream) {
  int r = check_ring_attention(q, k_ring, v_ring, pos_ring, out, m, n_q_heads, n_kv_heads,
                               head_dim, ring_slots, window);
  if (r != SDEC_OK) return r;
  // The chunk partials, counters and legal-slot lists live in buffers kept for the life of the
  // process and grown on demand; the counters are returned to zero by each launch.
  static float* part = nullptr;
  static size_t part_cap = 0;
  static uint32_t* counters = nullptr;
  static size_t cnt_cap = 0;
  static uint32_t* legal = nullptr;
  static size_t legal_cap = 0;
  const OneShotSizes z = one_shot_sizes(m, n_q_heads, n_kv_heads, head_dim, ring_slots);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (z.part > part_cap) {
    HIP_TRY(hipDeviceSynchronize());
    if (part) HIP_TRY(hipFree(part));
    part = nullptr;
    part_cap = 0;
    HIP_TRY(hipMalloc(&part, z.part * sizeof(float)));
    part_cap = z.part;
  }
  if (z.counters > cnt_cap) {
    HIP_TRY(hipDeviceSynchronize());
    if (counters) HIP_TRY(hipFree(counters));
    counters = nullptr;
    cnt_cap = 0;
    const size_t alloc = z.counters > 64 ? z.counters : 64;
    HIP_TRY(hipMalloc(&counters, alloc * sizeof(uint32_t)));
    cnt_cap = alloc;
    HIP_TRY(launch_fill_u32(counters, 0u, cnt_cap, s));
  }
  if (z.legal > legal_cap) {
    HIP_TRY(hipDeviceSynchronize());
    if (legal) HIP_TRY(hipFree(legal));
    legal = nullptr;
    legal_cap = 0;
    HIP_TRY(hipMalloc(&legal, z.legal * sizeof(uint32_t)));
    legal_cap = z.legal;
  }
  return enqueue_ring_attention(q, k_ring, v_ring, pos_ring, out, m, n_q_heads, n_kv_heads,
                                head_dim, ring_slots, window, pos, part, counters, legal, s);
}

int sdec_ring_attention_static(const float* q, const float* k_ring, const float* v_ring,
                               const uint32_t* pos_ring, float* out, uint32_t m,
                               uint32_t n_q_heads, uint32_t n_kv_heads, uint32_t head_dim,
                               uint32_t ring_slots, uint32_t window, uint32_t pos,
                               void* stream) {
  int r = check_ring_attention(q, k_ring, v_ring, pos_ring, out, m, n_q_heads, n_kv_heads,
                               head_dim, ring_slots, window);
  if (r != SDEC_OK) return r;
  const OneShotSizes z = one_shot_sizes(m, n_q_heads, n_kv_heads, head_dim, ring_slots);
  const size_t off_legal = align256(z.counters * sizeof(uint32_t));
  const size_t off_part = off_legal + align256(z.legal * sizeof(uint32_t));
  const size_t need = off_part + z.part * sizeof(float);
  if (need > kStaticScratchBytes)
    return fail(SDEC_E_ARG,
                "m=%u, %u query heads of %u over %u slots need %zu bytes of scratch, more than "
                "the %zu-byte static scratch", m, n_q_heads, head_dim, ring_slots, need,
                kStaticScratchBytes);
  void* base = nullptr;
  r = static_scratch(&base);
  if (r != SDEC_OK) return r;
  unsigned char* b = static_cast<unsigned char*>(base);
  uint32_t* counters = reinterpret_cast<uint32_t*>(b);
  uint32_t* legal = reinterpret_cast<uint32_t*>(b + off_legal);
  float* part = reinterpret_cast<float*>(b + off_part);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the array keeps whatever the last call on this device left: the counters start at zero
  HIP_TRY(launch_fill_u32(counters, 0u, z.counters, s));
  return enqueue_ring_attention(q, k_ring, v_ring, pos_ring, out, m, n_q_heads, n_kv_heads,
                                head_dim, ring_slots, window, pos, part, counters, legal, s);
}

}  // extern "C"

// ------------------------------------------------------------------------------------------------
// Split RVQ ([mimi] NEAREST, SUB_EMB, EMB_SUM; MimiGpu's encode and decode plans).
// ------------------------------------------------------------------------------------------------
struct sdec_rvq {
  sdec_rvq_config cfg{};
  sdec_rvq_weights w{};
  uint32_t groups = 0;
  float* cbT = nullptr;       // [nq][vq][bins]: level 0 = first, 1.. = rest
  float* proj = nullptr;      // [max_frames][2 vq]
  float* res = nullptr;       // [2][max_frames][vq] running residual (ping-pong)
  float* cand_d = nullptr;    // [nq][max_frames][groups]
  uint32_t* cand_i = nullptr;
  float* acc = nullptr;       // [max_frames][2 vq]
};

namespace {

void rvq_free(sdec_rvq* q) {
  void* ps[] = {q->cbT, q->proj, q->res, q->cand_d, q->cand_i, q->acc};
  for (void* p : ps)
    if (p) (void)hipFree(p);
}

int rvq_check_frames(const sdec_rvq* q, uint32_t frames) {
  if (!q) return fail(SDEC_E_ARG, "null rvq handle");
  if (frames < 1 || frames > q->cfg.max_frames)
    return fail(SDEC_E_ARG, "frames=%u must be in [1, max_frames=%u]", frames, q->cfg.max_frames);
  return SDEC_OK;
}

// GEMV rows in blocks of at most kMaxM frames.
template <class F>
int rvq_row_blocks(uint32_t frames, F body) {
  for (uint32_t f0 = 0; f0 < frames; f0 += static_cast<uint32_t>(kMaxM)) {
    const uint32_t n = frames - f0 < static_cast<uint32_t>(kMaxM) ? frames - f0 : kMaxM;
    int r = body(f0, n);
    if (r != SDEC_OK) return r;
  }
  return SDEC_OK;
}

int rvq_quantise_levels(sdec_rvq* q, const float* r_first, uint32_t sf, const float* r_rest,
                        uint32_t sr, uint32_t frames, uint32_t* codes, hipStream_t s) {
  const sdec_rvq_config& c = q->cfg;
  const size_t level_cb = static_cast<size_t>(c.vq) * c.bins;
  const size_t level_cand = static_cast<size_t>(c.max_frames) * q->groups;
  const size_t res_half = static_cast<size_t>(c.max_frames) * c.vq;
  for (uint32_t l = 0; l < c.nq; ++l) {
    RvqLevelArgs a{};
    a.cbT = q->cbT + l * level_cb;
    a.cand_d = q->cand_d + l * level_cand;
    a.cand_i = q->cand_i + l * level_cand;
    a.codes = codes; a.nq = c.nq; a.bins = c.bins; a.vq = c.vq; a.groups = q->groups;
    if (l == 0) {
      a.r_in = r_first; a.r_stride = sf;
    } else {
      a.prev_cand_d = q->cand_d + (l - 1) * level_cand;
      a.prev_cand_i = q->cand_i + (l - 1) * level_cand;
      a.prev_level = l - 1;
      a.r_out = q->res + (l % 2) * res_half;
      if (l == 1) {  // the rest chain starts from the second projection
        a.r_in = r_rest; a.r_stride = sr;
      } else {       // SUB_EMB of the previous rest level's code
        a.r_in = q->res + ((l - 1) % 2) * res_half; a.r_stride = c.vq;
        a.prev_cb = q->w.cb_rest + static_cast<size_t>(l - 2) * c.bins * c.vq;
      }
    }
    HIP_TRY(launch_rvq_level(a, frames, s));
  }
  RvqLevelArgs fin{};
  fin.prev_cand_d = q->cand_d + (c.nq - 1) * level_cand;
  fin.prev_cand_i = q->cand_i + (c.nq - 1) * level_cand;
  fin.prev_level = c.nq - 1; fin.codes = codes; fin.nq = c.nq; fin.groups = q->groups;
  HIP_TRY(launch_rvq_final(fin, frames, s));
  return SDEC_OK;
}

}  // namespace

extern "C" {

int sdec_rvq_create(const sdec_rvq_config* cfg, const sdec_rvq_weights* w, sdec_rvq** out) {
  g_err.clear();
  if (!cfg || !w || !out) return fail(SDEC_E_ARG, "null argument");
  const sdec_rvq_config c = *cfg;
  if (c.dim == 0 || c.dim % 4) return fail(SDEC_E_ARG, "dim must be a positive multiple of 4");
  if (c.vq == 0 || c.vq % 64 || c.vq > static_cast<uint32_t>(kRvqMaxVq))
    return fail(SDEC_E_ARG, "vq must be a multiple of 64 in [64, %d]", kRvqMaxVq);
  if (c.bins < 64 || c.bins % 64 || c.bins / 64 > 65535)
    return fail(SDEC_E_ARG, "bins must be a multiple of 64, at least 64");
  if (c.nq < 2) return fail(SDEC_E_ARG, "nq must be at least 2 (one first and one rest codebook)");
  if (c.max_frames < 1 || c.max_frames > 65535)
    return fail(SDEC_E_ARG, "max_frames must be in [1, 65535]");
  const float* ptrs[] = {w->in_first, w->in_rest, w->out_first, w->out_rest, w->cb_first, w->cb_rest};
  const char* names[] = {"in_first", "in_rest", "out_first", "out_rest", "cb_first", "cb_rest"};
  for (int i = 0; i < 6; ++i)
    if (!ptrs[i] || !aligned16(ptrs[i]))
      return fail(SDEC_E_ARG, "%s must be a 16-byte aligned device pointer", names[i]);
  sdec_rvq* q = new sdec_rvq();
  q->cfg = c; q->w = *w; q->groups = c.bins / 64;
  Alloc A;
  const size_t level_cb = static_cast<size_t>(c.vq) * c.bins;
  q->cbT = A.get<float>(level_cb * c.nq);
  q->proj = A.get<float>(static_cast<size_t>(c.max_frames) * 2 * c.vq);
  q->res = A.get<float>(static_cast<size_t>(2) * c.max_frames * c.vq);
  q->cand_d = A.get<float>(static_cast<size_t>(c.nq) * c.max_frames * q->groups);
  q->cand_i = A.get<uint32_t>(static_cast<size_t>(c.nq) * c.max_frames * q->groups);
  q->acc = A.get<float>(static_cast<size_t>(c.max_frames) * 2 * c.vq);
  if (A.code != SDEC_OK) {
    for (void* p : A.ptrs) (void)hipFree(p);
    delete q;
    return A.code;
  }
  hipError_t e = launch_transpose(w->cb_first, q->cbT, 1, c.bins, c.vq, nullptr);
  if (e == hipSuccess)
    e = launch_transpose(w->cb_rest, q->cbT + level_cb, c.nq - 1, c.bins, c.vq, nullptr);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    rvq_free(q);
    delete q;
    return fail(SDEC_E_HIP, "codebook transpose: %s", hipGetErrorString(e));
  }
  *out = q;
  return SDEC_OK;
}

int sdec_rvq_quantise(sdec_rvq* q, const float* r_first, const float* r_rest, uint32_t frames,
                      uint32_t* codes, void* stream) {
  int r = rvq_check_frames(q, frames);
  if (r != SDEC_OK) return r;
  if (!r_first || !r_rest || !codes) return fail(SDEC_E_ARG, "null device pointer");
  return rvq_quantise_levels(q, r_first, q->cfg.vq, r_rest, q->cfg.vq, frames, codes,
                             static_cast<hipStream_t>(stream));
}

int sdec_rvq_encode(sdec_rvq* q, const float* latent, uint32_t frames, uint32_t* codes,
                    void* stream) {
  int r = rvq_check_frames(q, frames);
  if (r != SDEC_OK) return r;
  if (!latent || !aligned16(latent) || !codes)
    return fail(SDEC_E_ARG, "latent (16-byte aligned) and codes must be device pointers");
  const sdec_rvq_config& c = q->cfg;
  hipStream_t s = static_cast<hipStream_t>(stream);
  r = rvq_row_blocks(frames, [&](uint32_t f0, uint32_t n) -> int {
    GemvArgs g{};
    g.w[0] = q->w.in_first; g.w[1] = q->w.in_rest; g.w[2] = q->w.in_rest;
    g.seg_end[0] = c.vq; g.seg_end[1] = 2 * c.vq; g.seg_end[2] = 2 * c.vq;
    g.n_rows = 2 * c.vq; g.k = c.dim; g.m = n;
    g.x = latent + static_cast<size_t>(f0) * c.dim; g.x_stride = c.dim;
    g.y = q->proj + static_cast<size_t>(f0) * 2 * c.vq; g.y_stride = 2 * c.vq;
    HIP_TRY(launch_gemv(g, plan_gemv(PRO_NONE, EPI_STORE, 2 * c.vq, c.dim, n), s));
    return SDEC_OK;
  });
  if (r != SDEC_OK) return r;
  return rvq_quantise_levels(q, q->proj, 2 * c.vq, q->proj + c.vq, 2 * c.vq, frames, codes, s);
}

int sdec_rvq_decode(sdec_rvq* q, const uint32_t* codes, uint32_t frames, float* latent,
                    void* stream) {
  int r = rvq_check_frames(q, frames);
  if (r != SDEC_OK) return r;
  if (!latent || !aligned16(latent) || !codes)
    return fail(SDEC_E_ARG, "codes and latent (16-byte aligned) must be device pointers");
  const sdec_rvq_config& c = q->cfg;
  hipStream_t s = static_cast<hipStream_t>(stream);
  RvqEmbArgs e{};
  e.codes = codes; e.cb_first = q->w.cb_first; e.cb_rest = q->w.cb_rest; e.acc = q->acc;
  e.nq = c.nq; e.bins = c.bins; e.vq = c.vq;
  HIP_TRY(launch_rvq_emb_sum(e, frames, s));
  return rvq_row_blocks(frames, [&](uint32_t f0, uint32_t n) -> int {
    float* y = latent + static_cast<size_t>(f0) * c.dim;
    const float* acc = q->acc + static_cast<size_t>(f0) * 2 * c.vq;
    GemvArgs g{};
    g.w[0] = g.w[1] = g.w[2] = q->w.out_first;
    g.seg_end[0] = g.seg_end[1] = g.seg_end[2] = c.dim;
    g.n_rows = c.dim; g.k = c.vq; g.m = n; g.x = acc; g.x_stride = 2 * c.vq;
    g.y = y; g.y_stride = c.dim;
    HIP_TRY(launch_gemv(g, plan_gemv(PRO_NONE, EPI_STORE, c.dim, c.vq, n), s));
    GemvArgs h{};  // the second projection accumulates into the first ([mimi] decode plan)
    h.w[0] = h.w[1] = h.w[2] = q->w.out_rest;
    h.seg_end[0] = h.seg_end[1] = h.seg_end[2] = c.dim;
    h.n_rows = c.dim; h.k = c.vq; h.m = n; h.x = acc + c.vq; h.x_stride = 2 * c.vq;
    h.res = y; h.res_stride = c.dim;
    HIP_TRY(launch_gemv(h, plan_gemv(PRO_NONE, EPI_RESIDUAL, c.dim, c.vq, n), s));
    return SDEC_OK;
  });
}

void sdec_rvq_destroy(sdec_rvq* q) {
  if (!q) return;
  (void)hipDeviceSynchronize();
  rvq_free(q);
  delete q;
}

}  // extern "C"

// ------------------------------------------------------------------------------------------------
// Streaming codec convolutions ([mimi] CONV1D, convtr_src and their carries).
// ------------------------------------------------------------------------------------------------
struct sdec_conv {
  sdec_conv_config cfg{};
  const float* w = nullptr;
  const float* b = nullptr;
  float* state[2] = {nullptr, nullptr};  // prefix [in_ch][k - s] or tail [out_ch][k - s]
  float* part = nullptr;                 // split-k partial sums (groups == 1)
  uint64_t part_cap = 0;
  uint32_t* counters = nullptr;          // per output tile: splits finished
  uint32_t counter_cap = 0;
  int cur = 0;
  bool started = false;
};

extern "C" {

int sdec_conv_create(const sdec_conv_config* cfg, const float* w, const float* b, sdec_conv** out) {
  g_err.clear();
  if (!cfg || !out) return fail(SDEC_E_ARG, "null argument");
  const sdec_conv_config c = *cfg;
  if (!w || !b) return fail(SDEC_E_ARG, "w and b must be device pointers");
  if (c.in_ch < 1 || c.out_ch < 1 || c.out_ch > 65535)
    return fail(SDEC_E_ARG, "channels must be in [1, 65535]");
  if (c.stride < 1 || c.kernel < c.stride) return fail(SDEC_E_ARG, "need kernel >= stride >= 1");
  if (!(c.groups == 1 || (c.groups == c.in_ch && c.in_ch == c.out_ch)))
    return fail(SDEC_E_ARG, "groups must be 1 or in_ch == out_ch (channel-wise)");
  if (c.max_t_in < 1) return fail(SDEC_E_ARG, "max_t_in must be >= 1");
  if (c.transposed && (c.replicate_first || c.accumulate))
    return fail(SDEC_E_ARG, "replicate_first and accumulate apply to the forward conv only");
  sdec_conv* h = new sdec_conv();
  h->cfg = c; h->w = w; h->b = b;
  const size_t n = static_cast<size_t>(c.transposed ? c.out_ch : c.in_ch) * (c.kernel - c.stride);
  Alloc A;
  h->state[0] = A.get<float>(n);
  h->state[1] = A.get<float>(n);
  if (c.groups == 1) {
    // partial sums of up to kConvMaxSplits input-channel splits of the largest frame
    const uint64_t cols = c.transposed
                              ? static_cast<uint64_t>(c.max_t_in) * c.stride + (c.kernel - c.stride)
                              : c.max_t_in / c.stride;
    uint64_t splits = (c.in_ch + 31) / 32;
    if (splits > kConvMaxSplits) splits = kConvMaxSplits;
    if (splits > 1) {
      h->part_cap = splits * c.out_ch * cols;
      h->part = A.get<float>(h->part_cap);
      // output tiles are at least 16 columns x 4 channels
      h->counter_cap = static_cast<uint32_t>(((cols + 15) / 16) * ((c.out_ch + 3) / 4));
      h->counters = A.get<uint32_t>(h->counter_cap);
      if (h->counters && hipMemset(h->counters, 0, sizeof(uint32_t) * h->counter_cap) != hipSuccess)
        A.code = fail(SDEC_E_HIP, "clearing the conv tile counters failed");
    }
  }
  if (A.code != SDEC_OK) {
    for (void* p : A.ptrs) (void)hipFree(p);
    delete h;
    return A.code;
  }
  *out = h;
  return SDEC_OK;
}

int sdec_conv_step(sdec_conv* h, const float* x, uint32_t t_in, float* y, uint32_t first,
                   void* stream) {
  if (!h) return fail(SDEC_E_ARG, "null conv handle");
  const sdec_conv_config& c = h->cfg;
  if (!x || !y) return fail(SDEC_E_ARG, "x and y must be device pointers");
  if (t_in < 1 || t_in > c.max_t_in)
    return fail(SDEC_E_ARG, "t_in=%u must be in [1, max_t_in=%u]", t_in, c.max_t_in);
  if (!first && !h->started) return fail(SDEC_E_POS, "the first frame of a stream needs first != 0");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint32_t carry = c.kernel - c.stride;
  if (c.transposed) {
    SConvTrArgs a{};
    a.w = h->w; a.b = h->b; a.x = x; a.tail = h->state[h->cur]; a.tail_out = h->state[h->cur ^ 1];
    a.y = y; a.c_in = c.in_ch; a.c_out = c.out_ch; a.k = c.kernel; a.stride = c.stride;
    a.groups = c.groups; a.t_in = t_in; a.tl = carry; a.pre_elu = c.pre_elu ? 1 : 0;
    a.first = first ? 1 : 0;
    a.part = h->part; a.part_cap = h->part_cap;
    a.counters = h->counters; a.counter_cap = h->counter_cap;
    HIP_TRY(launch_sconvtr(a, s));
  } else {
    if (t_in % c.stride) return fail(SDEC_E_ARG, "t_in=%u is not a multiple of stride %u", t_in, c.stride);
    SConvArgs a{};
    a.w = h->w; a.b = h->b; a.x = x; a.prefix = h->state[h->cur]; a.prefix_out = h->state[h->cur ^ 1];
    a.y = y; a.c_in = c.in_ch; a.c_out = c.out_ch; a.k = c.kernel; a.stride = c.stride;
    a.groups = c.groups; a.t_in = t_in; a.pad = carry; a.pre_elu = c.pre_elu ? 1 : 0;
    a.replicate_first = c.replicate_first ? 1 : 0; a.first = first ? 1 : 0;
    a.accumulate = c.accumulate ? 1 : 0;
    a.part = h->part; a.part_cap = h->part_cap;
    a.counters = h->counters; a.counter_cap = h->counter_cap;
    HIP_TRY(launch_sconv(a, s));
  }
  h->cur ^= 1;
  h->started = true;
  return SDEC_OK;
}

int sdec_transpose(const float* x, uint32_t rows, uint32_t cols, float* y, void* stream) {
  if (!x || !y) return fail(SDEC_E_ARG, "x and y must be device pointers");
  if (rows == 0 || cols == 0) return fail(SDEC_E_ARG, "rows=%u cols=%u must be nonzero", rows, cols);
  if ((cols + 31u) / 32u > 65535u) return fail(SDEC_E_ARG, "cols=%u exceeds the grid's limit", cols);
  const uintptr_t bytes = static_cast<uintptr_t>(rows) * cols * sizeof(float);
  const uintptr_t xa = reinterpret_cast<uintptr_t>(x), ya = reinterpret_cast<uintptr_t>(y);
  if (xa < ya + bytes && ya < xa + bytes) return fail(SDEC_E_ARG, "x and y overlap");
  HIP_TRY(launch_transpose(x, y, 1, rows, cols, static_cast<hipStream_t>(stream)));
  return SDEC_OK;
}

void sdec_conv_destroy(sdec_conv* h) {
  if (!h) return;
  (void)hipDeviceSynchronize();
  for (float* p : h->state)
    if (p) (void)hipFree(p);
  if (h->part) (void)hipFree(h->part);
  if (h->counters) (void)hipFree(h->counters);
  delete h;
}

}  // extern "C"
