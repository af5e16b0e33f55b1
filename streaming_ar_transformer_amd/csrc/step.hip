// Persistent step kernel: one cooperative launch runs a whole decode step of one stream.
//
// Page names in citations: [talker] inferencelayer 0.2.8 src/qwen3tts_gpu.rs, [mimi] 0.2.1
// src/mimi_gpu.rs.
//
// The pages replay a recorded pass list of small dispatches per token ([talker] StepPlan /
// build_step_plan: 19 dispatches per layer; [mimi] Builder::transformer_shaped: 9).  On MI355X a
// kernel boundary costs about 1.7 us of idle HBM, which at m=1 is a large share of a 25 us layer.
// Here every CU holds one workgroup for the whole step and the phases of the pass list are
// separated by device-wide barriers instead of launches:
//
//   begin | per layer: norm+QKV GEMV | qk-norm+rope+push+ring attention | O GEMV+residual |
//         norm+FFN up GEMV+activation | down GEMV+residual | end (final norm)
//
// Before a wave waits at a barrier it issues the weight loads of its first tile of the next GEMV
// phase (weights never depend on activations), so HBM keeps streaming while the barrier settles.
// Activations handed between phases go through per-layer buffers that are written exactly once per
// launch with device-coherent stores, so their consumers may use ordinary cached loads without any
// cache-wide writeback or invalidate.

#include "dev.h"
#include "kernels.h"

namespace sdec {
namespace {

using namespace dev;

constexpr int kStepThreads = 256;  // one wave per SIMD: 512 registers per lane for the pipelines
constexpr int kStepWaves = kStepThreads / kWave;
constexpr int kMaxK4 = 6144 / 4;  // widest GEMV input row staged in LDS (float4)
constexpr uint32_t kSpinLimit = 1u << 20;

template <int HD, int G>
union StepSmem {
  AttnSmem<HD, G, kStepThreads> attn;
  struct {
    float4 raw[kMaxK4];
    float4 norm[kMaxK4];
  } gemv;
};

// Device-wide barrier on a monotonic 64-bit arrival counter: barrier number `idx` of this launch
// is complete when the counter reaches base + (idx + 1) * gridDim.x.  A bounded wait: past the
// spin limit the flag `err` is set and every later barrier of the launch returns at once, so a
// broken launch drains instead of hanging.
// With a.trace set, workgroup 0 stamps the constant-rate device clock when it arrives at barrier
// idx (trace[2*idx]) and when the barrier releases it (trace[2*idx + 1]).
__device__ __forceinline__ void grid_sync(const StepArgs& a, uint32_t idx) {
  wait_stores();  // this thread's coherent stores are complete
  __syncthreads();
  if (threadIdx.x == 0) {
    if (a.trace && blockIdx.x == 0) a.trace[2 * idx] = wall_clock64();
    const uint64_t target = a.bar_base + static_cast<uint64_t>(idx + 1) * gridDim.x;
    __hip_atomic_fetch_add(a.bar, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t spins = 0;
    while (__hip_atomic_load(a.bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (__hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) break;
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit) {
        __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
    if (a.trace && blockIdx.x == 0) a.trace[2 * idx + 1] = wall_clock64();
  }
  __syncthreads();
}

// A wave's weight pipeline in a GEMV phase: the phase's tiles are cut into units of SB float4 per
// lane of each of the tile's R rows (8 float4 per lane per unit, 8 KiB per wave); two units are in
// flight while the one before them is reduced.
template <int R, int KB>
struct Pipe {
  static constexpr int SB = KB < 8 / R ? KB : 8 / R;  // float4 per lane per row per unit
  static constexpr int NB = KB / SB;          // units per tile
  float4 cur[SB][R];
  float4 nxt[SB][R];
};

template <int R, int EPI, int KB>
__device__ __forceinline__ void load_unit(const GemvArgs& g, uint32_t t, int b,
                                          float4 (&w)[Pipe<R, KB>::SB][R]) {
  constexpr int SB = Pipe<R, KB>::SB;
  const float4* wr[R];
  tile_rows<R, EPI>(g, t, wr);
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int j = 0; j < SB; ++j)
#pragma unroll
    for (int r = 0; r < R; ++r) w[j][r] = ldw(wr[r] + lane + kWave * (b * SB + j));
}

// The first two units of this wave in a GEMV phase (the same balanced split gemv_phase uses).
template <int R, int EPI, int KB>
__device__ __forceinline__ void prefetch_pipe(const GemvArgs& g, Pipe<R, KB>& p) {
  constexpr int RH = EPI == EPI_SWIGLU ? R / 2 : R;
  constexpr int NB = Pipe<R, KB>::NB;
  uint32_t t, t_end;
  wave_tiles((g.n_rows + RH - 1) / RH, t, t_end);
  const uint32_t n_units = (t_end - t) * NB;
  if (n_units > 0) load_unit<R, EPI, KB>(g, t, 0, p.cur);
  if (n_units > 1) load_unit<R, EPI, KB>(g, t + 1 / NB, 1 % NB, p.nxt);
}

// One GEMV phase for a single input row: stage the row in LDS (normalised if PRO), then every
// wave reduces its tiles.  `p` holds the wave's first two units, loaded before the preceding
// barrier.
template <int R, int EPI, int PRO, int KB>
__device__ __forceinline__ void gemv_phase(const GemvArgs& g, float4* raw, float4* nrm,
                                           Pipe<R, KB>& p) {
  constexpr int K4 = KB * kWave;
  constexpr int RH = EPI == EPI_SWIGLU ? R / 2 : R;
  constexpr int SB = Pipe<R, KB>::SB, NB = Pipe<R, KB>::NB;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const float4* x4 = reinterpret_cast<const float4*>(g.x);
  for (int i = tid; i < K4; i += kStepThreads) raw[i] = x4[i];
  __syncthreads();
  const float4* xs = raw;
  if (PRO != PRO_NONE) {
    // every wave forms the same statistics, in the same order, from the staged row
    const float kf = static_cast<float>(g.k);
    float mean = 0.f, inv;
    if (PRO == PRO_RMS) {
      float ss = 0.f;
      for (int c = lane; c < K4; c += kWave) ss = dot4(raw[c], raw[c], ss);
      inv = 1.0f / sqrtf(wave_sum(ss) / kf + g.eps);
    } else {
      float sm = 0.f;
      for (int c = lane; c < K4; c += kWave) sm += (raw[c].x + raw[c].y) + (raw[c].z + raw[c].w);
      mean = wave_sum(sm) / kf;
      float ss = 0.f;
      for (int c = lane; c < K4; c += kWave) {
        float4 d = raw[c];
        d.x -= mean; d.y -= mean; d.z -= mean; d.w -= mean;
        ss = dot4(d, d, ss);
      }
      inv = 1.0f / sqrtf(wave_sum(ss) / kf + g.eps);
    }
    const float4* g4 = reinterpret_cast<const float4*>(g.norm_w);
    const float4* b4 = reinterpret_cast<const float4*>(g.norm_b);
    for (int i = tid; i < K4; i += kStepThreads) {
      float4 v = raw[i];
      const float4 gg = g4[i];
      if (PRO == PRO_RMS) {
        v.x = (v.x * inv) * gg.x; v.y = (v.y * inv) * gg.y;
        v.z = (v.z * inv) * gg.z; v.w = (v.w * inv) * gg.w;
      } else {
        const float4 b = b4[i];
        v.x = ((v.x - mean) * inv) * gg.x + b.x; v.y = ((v.y - mean) * inv) * gg.y + b.y;
        v.z = ((v.z - mean) * inv) * gg.z + b.z; v.w = ((v.w - mean) * inv) * gg.w + b.w;
      }
      nrm[i] = v;
    }
    __syncthreads();
    xs = nrm;
  }
  uint32_t t0, t_end;
  wave_tiles((g.n_rows + RH - 1) / RH, t0, t_end);
  const uint32_t n_units = (t_end - t0) * NB;
  float acc[R];
  for (uint32_t i = 0; i < n_units; ++i) {
    const uint32_t t = t0 + i / NB;
    const int b = static_cast<int>(i % NB);
    if (b == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      const float4 xv = xs[lane + kWave * (b * SB + j)];
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = dot4(p.cur[j][r], xv, acc[r]);
    }
#pragma unroll
    for (int j = 0; j < SB; ++j)
#pragma unroll
      for (int r = 0; r < R; ++r) p.cur[j][r] = p.nxt[j][r];
    if (i + 2 < n_units) load_unit<R, EPI, KB>(g, t0 + (i + 2) / NB, static_cast<int>((i + 2) % NB), p.nxt);
    if (b == NB - 1) gemv_epilogue<1, R, EPI, true>(g, t, acc, lane);
  }
}

template <int HD, int G, int KBQ, int KBD, int PRO, int FFN>
__global__ __launch_bounds__(kStepThreads) void k_step(StepArgs a) {
  __shared__ StepSmem<HD, G> sm;
  constexpr int RU = 2;  // FFN up tile: a gate row and its up row (SwiGLU), or two W1 rows
  const int tid = threadIdx.x;
  const uint32_t d = a.d, hq = a.hq, hkv = a.hkv, nqkv = a.nqkv;
  uint32_t bar = 0;
  const uint32_t n_bar = 1 + 5 * a.n_layers;
  if (a.trace && blockIdx.x == 0 && tid == 0) a.trace[2 * n_bar] = wall_clock64();

  // ---- begin: input row, position ring, rope cos/sin ([mimi] rope_push_src; [talker] load)
  const uint32_t slot = a.pos % a.ring;
  if (blockIdx.x == 0) {
    for (uint32_t i = tid; i < d; i += kStepThreads) st_dev(a.x0 + i, a.x_in[i]);
    if (a.first) {
      for (uint32_t i = tid; i < a.ring; i += kStepThreads) a.pos_ring[i] = i == slot ? a.pos : kInvalidPos;
    } else if (tid == 0) {
      a.pos_ring[slot] = a.pos;
    }
    __syncthreads();
    compact_legal<kStepThreads, true>(a.pos_ring, a.ring, a.pos, a.window, static_cast<int>(slot),
                                      a.legal, a.n_legal, reinterpret_cast<uint32_t*>(sm.gemv.raw));
    const uint32_t half = HD / 2;
    if (static_cast<uint32_t>(tid) < half) {
      const double inv_freq = pow(a.theta, -2.0 * static_cast<double>(tid) / static_cast<double>(HD));
      const double ang = static_cast<double>(a.pos) * inv_freq;
      st_dev(a.cs + tid, static_cast<float>(cos(ang)));
      st_dev(a.cs + half + tid, static_cast<float>(sin(ang)));
    }
    if (tid == 0) {
      __hip_atomic_store(&a.st->pos, a.pos, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.st->slot, slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  Pipe<1, KBQ> wq;  // carried from one layer's down phase to the next layer's QKV phase

  auto qkv_args = [&](const StepLayer& L) {
    GemvArgs g{};
    g.w[0] = L.wq; g.w[1] = L.wk; g.w[2] = L.wv;
    g.seg_end[0] = hq * HD; g.seg_end[1] = (hq + hkv) * HD; g.seg_end[2] = nqkv;
    g.n_rows = nqkv; g.k = d; g.m = 1; g.x = L.x_in; g.x_stride = d;
    g.norm_w = L.attn_norm_w; g.norm_b = L.attn_norm_b; g.eps = a.eps;
    g.y = L.qkv; g.y_stride = nqkv;
    return g;
  };
  auto o_args = [&](const StepLayer& L) {
    GemvArgs g{};
    g.w[0] = g.w[1] = g.w[2] = L.wo;
    g.seg_end[0] = g.seg_end[1] = g.seg_end[2] = d;
    g.n_rows = d; g.k = hq * HD; g.m = 1; g.x = L.attn_out; g.x_stride = hq * HD;
    g.res = L.x_attn; g.res_in = L.x_in; g.res_stride = d; g.ls = a.layer_scale ? L.ls1 : nullptr;
    return g;
  };
  auto up_args = [&](const StepLayer& L) {
    GemvArgs g{};
    if (FFN == EPI_SWIGLU) {
      g.w[0] = L.w_gate; g.w[1] = L.w_up; g.w[2] = L.w_up;
    } else {
      g.w[0] = g.w[1] = g.w[2] = L.w_up;
    }
    g.seg_end[0] = g.seg_end[1] = g.seg_end[2] = a.d_ff;
    g.n_rows = a.d_ff; g.k = d; g.m = 1; g.x = L.x_attn; g.x_stride = d;
    g.norm_w = L.ffn_norm_w; g.norm_b = L.ffn_norm_b; g.eps = a.eps;
    g.y = L.act; g.y_stride = a.d_ff;
    return g;
  };
  auto down_args = [&](const StepLayer& L) {
    GemvArgs g{};
    g.w[0] = g.w[1] = g.w[2] = L.w_down;
    g.seg_end[0] = g.seg_end[1] = g.seg_end[2] = d;
    g.n_rows = d; g.k = a.d_ff; g.m = 1; g.x = L.act; g.x_stride = a.d_ff;
    g.res = L.x_ffn; g.res_in = L.x_attn; g.res_stride = d; g.ls = a.layer_scale ? L.ls2 : nullptr;
    return g;
  };

  prefetch_pipe<1, EPI_STORE, KBQ>(qkv_args(a.layers[0]), wq);
  grid_sync(a, bar++);

  for (uint32_t l = 0; l < a.n_layers; ++l) {
    const StepLayer& L = a.layers[l];
    // ---- norm + q/k/v projections ([talker] RMSNORM_SRC + MATVEC_SRC; [mimi] LN + MATVEC)
    gemv_phase<1, EPI_STORE, PRO, KBQ>(qkv_args(L), sm.gemv.raw, sm.gemv.norm, wq);
    Pipe<1, KBQ> wo;
    prefetch_pipe<1, EPI_RESIDUAL, KBQ>(o_args(L), wo);
    grid_sync(a, bar++);
    // ---- qk-norm + rope + ring push + ring attention ([talker] QK_NORM_SRC, ROPE_SRC,
    //      APPEND_SRC, GQA_ATTN_SRC; [mimi] rope_push_src, attn_src)
    {
      AttnArgs aa{};
      aa.qkv = L.qkv; aa.qkv_stride = nqkv;
      aa.q_norm = L.q_norm; aa.k_norm = L.k_norm; aa.eps = a.qk_eps;
      aa.rope_style = a.rope_style; aa.cs = a.cs; aa.push = 1;
      aa.k_ring = L.k_ring; aa.v_ring = L.v_ring; aa.ring_stream_stride = 0;
      aa.legal = a.legal; aa.n_legal = a.n_legal;
      aa.out = L.attn_out; aa.part = L.part; aa.counters = L.counters;
      aa.m = 1; aa.n_q_heads = hq; aa.n_kv_heads = hkv; aa.head_dim = HD; aa.ring = a.ring;
      aa.chunk = a.chunk; aa.n_chunks = a.n_chunks; aa.st = a.st;
      const uint32_t items = a.n_chunks * hkv;
      for (uint32_t it = blockIdx.x; it < items; it += gridDim.x)
        attention_item<HD, G, kStepThreads, true, 2, 4>(aa, it % a.n_chunks, it / a.n_chunks, 0u, sm.attn);
    }
    grid_sync(a, bar++);
    // ---- o projection + (LayerScale) residual ([talker] o GEMV + ADD; [mimi] MV_LS)
    gemv_phase<1, EPI_RESIDUAL, PRO_NONE, KBQ>(o_args(L), sm.gemv.raw, sm.gemv.norm, wo);
    Pipe<RU, KBQ> wu;
    prefetch_pipe<RU, FFN, KBQ>(up_args(L), wu);
    grid_sync(a, bar++);
    // ---- norm + FFN up + activation ([talker] SWIGLU_SRC; [mimi] lin1 + GELU_ERF)
    gemv_phase<RU, FFN, PRO, KBQ>(up_args(L), sm.gemv.raw, sm.gemv.norm, wu);
    Pipe<1, KBD> wd;
    prefetch_pipe<1, EPI_RESIDUAL, KBD>(down_args(L), wd);
    grid_sync(a, bar++);
    // ---- down projection + (LayerScale) residual
    gemv_phase<1, EPI_RESIDUAL, PRO_NONE, KBD>(down_args(L), sm.gemv.raw, sm.gemv.norm, wd);
    if (l + 1 < a.n_layers) {
      prefetch_pipe<1, EPI_STORE, KBQ>(qkv_args(a.layers[l + 1]), wq);
    } else {
      wq = Pipe<1, KBQ>{};  // no next layer: the carried units are dead
    }
    grid_sync(a, bar++);
  }

  // ---- end: final norm ([talker] build_step_plan's closing RMSNorm) or the residual stream
  if (blockIdx.x == 0) {
    if (a.trace && tid == 0) a.trace[2 * n_bar + 1] = wall_clock64();
    const float* x = a.layers[a.n_layers - 1].x_ffn;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    if (!a.final_norm) {
      for (uint32_t i = tid; i < d; i += kStepThreads) a.x_out[i] = x[i];
      return;
    }
    float* red = reinterpret_cast<float*>(sm.gemv.raw);
    const float df = static_cast<float>(d);
    float mean = 0.f;
    if (PRO == PRO_LN) {
      float s = 0.f;
      for (uint32_t i = tid; i < d; i += kStepThreads) s += x[i];
      s = wave_sum(s);
      if (lane == 0) red[wave] = s;
      __syncthreads();
      float t = 0.f;
      for (int w = 0; w < kStepWaves; ++w) t += red[w];
      mean = t / df;
      __syncthreads();
    }
    float ss = 0.f;
    for (uint32_t i = tid; i < d; i += kStepThreads) {
      const float v = x[i] - mean;
      ss = fmaf(v, v, ss);
    }
    ss = wave_sum(ss);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    float t = 0.f;
    for (int w = 0; w < kStepWaves; ++w) t += red[w];
    const float inv = 1.0f / sqrtf(t / df + a.eps);
    for (uint32_t i = tid; i < d; i += kStepThreads) {
      if (PRO == PRO_LN) a.x_out[i] = ((x[i] - mean) * inv) * a.fin_w[i] + a.fin_b[i];
      else a.x_out[i] = (x[i] * inv) * a.fin_w[i];
    }
  }
}

template <int HD, int G, int KBQ, int KBD, int PRO, int FFN>
const void* step_fn() {
  return reinterpret_cast<const void*>(&k_step<HD, G, KBQ, KBD, PRO, FFN>);
}

// The geometries the persistent kernel is built for: the talker family (hd 128, GQA group 2,
// hidden 2048, FFN 6144, RMSNorm, SwiGLU) and the codec family (hd 64, MHA, hidden 512, FFN
// 2048, LayerNorm, GELU).
const void* pick_step(uint32_t hd, uint32_t group, uint32_t kbq, uint32_t kbd, int pro, int ffn) {
  if (hd == 128 && group == 2 && kbq == 8 && kbd == 24 && pro == PRO_RMS && ffn == EPI_SWIGLU)
    return step_fn<128, 2, 8, 24, PRO_RMS, EPI_SWIGLU>();
  if (hd == 64 && group == 1 && kbq == 2 && kbd == 8 && pro == PRO_LN && ffn == EPI_GELU)
    return step_fn<64, 1, 2, 8, PRO_LN, EPI_GELU>();
  return nullptr;
}

}  // namespace

uint32_t step_barriers(uint32_t n_layers) { return 1 + 5 * n_layers; }

hipError_t plan_step(uint32_t head_dim, uint32_t group, uint32_t d_model, uint32_t d_ff,
                     uint32_t q_width, int norm, int ffn, uint32_t* grid) {
  if (q_width != d_model || d_model % 256 || d_ff % 256) return hipErrorInvalidValue;
  const void* fn = pick_step(head_dim, group, d_model / 256, d_ff / 256, norm, ffn);
  if (fn == nullptr) return hipErrorInvalidValue;
  int dev = 0, cus = 0, occ = 0, coop = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
    return e;
  if ((e = hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev)) != hipSuccess)
    return e;
  if (!coop) return hipErrorNotSupported;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, kStepThreads, 0)) != hipSuccess)
    return e;
  if (occ < 1) return hipErrorNotSupported;
  *grid = static_cast<uint32_t>(cus);  // one resident workgroup per CU
  return hipSuccess;
}

hipError_t launch_step(const StepArgs& a, uint32_t grid, uint32_t group, hipStream_t s) {
  const void* fn = pick_step(a.hd, group, a.d / 256, a.d_ff / 256, a.norm, a.ffn);
  if (fn == nullptr) return hipErrorInvalidValue;
  StepArgs args = a;
  void* params[] = {&args};
  return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kStepThreads), params, 0, s);
}

}  // namespace sdec
