// HIP kernels of the streaming decode step, written for CDNA4 (gfx950, wave64).
//
// Page names used in citations (docs.rs inferencelayer source pages):
//   [talker] 0.2.8 src/qwen3tts_gpu.rs   [mimi] 0.2.1 src/mimi_gpu.rs
//   [pocket] 0.2.4 src/pocket_tts_gpu.rs [parakeet] 0.2.10 src/parakeet_gpu.rs
//
// The step is HBM-bound weight streaming at m <= 8 rows (0.5 .. 4 flop/byte in float32), so
// nothing here is shaped for the matrix cores: the GEMV streams each weight row once with
// 128-bit loads, reduces k inside one wave with cross-lane shuffles, and fuses the neighbouring
// elementwise work (norm prologue, SwiGLU / GELU / LayerScale-residual epilogues) into itself.

#include <math.h>
#include <stdlib.h>

#include <type_traits>

#include <hip/hip_ext.h>

#include "dev.h"
#include "kernels.h"

namespace sdec {

namespace {

using namespace dev;

// ------------------------------------------------------------------------------------------------
// GEMV prologue: stage the m input rows in LDS, normalised ([talker] RMSNORM_SRC; [mimi] ln_src).
// ------------------------------------------------------------------------------------------------
template <int M, int PRO>
__device__ __forceinline__ void stage_x(const GemvArgs& a, float4* xs, uint32_t K4) {
  const float4* x4 = reinterpret_cast<const float4*>(a.x);
  const uint32_t xstride4 = a.x_stride >> 2;
  for (uint32_t i = threadIdx.x; i < M * K4; i += blockDim.x) {
    const uint32_t m = i / K4, c = i - m * K4;
    xs[i] = m < a.m ? x4[m * xstride4 + c] : f4zero();
  }
  __syncthreads();
  // Wave w normalises rows w, w + nw, ...: its statistics never leave its registers.
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  const float kf = static_cast<float>(a.k);
  const float4* g4 = reinterpret_cast<const float4*>(a.norm_w);
  const float4* b4 = reinterpret_cast<const float4*>(a.norm_b);
  for (int m = wave; m < static_cast<int>(a.m) && m < M; m += nw) {
    float4* row = xs + m * K4;
    float mean = 0.f, inv;
    if (PRO == PRO_RMS) {
      float ss = 0.f;
      for (uint32_t c = lane; c < K4; c += kWave) {
        const float4 t = row[c];
        ss = dot4(t, t, ss);
      }
      inv = rsqrtf(wave_sum(ss) * (1.0f / kf) + a.eps);
    } else {
      float s = 0.f;
      for (uint32_t c = lane; c < K4; c += kWave) {
        const float4 t = row[c];
        s += (t.x + t.y) + (t.z + t.w);
      }
      mean = wave_sum(s) * (1.0f / kf);
      float ss = 0.f;
      for (uint32_t c = lane; c < K4; c += kWave) {
        float4 t = row[c];
        t.x -= mean; t.y -= mean; t.z -= mean; t.w -= mean;
        ss = dot4(t, t, ss);
      }
      inv = rsqrtf(wave_sum(ss) * (1.0f / kf) + a.eps);
    }
    for (uint32_t c = lane; c < K4; c += kWave) {
      float4 t = row[c];
      const float4 g = g4[c];
      if (PRO == PRO_RMS) {
        t.x = (t.x * inv) * g.x; t.y = (t.y * inv) * g.y;
        t.z = (t.z * inv) * g.z; t.w = (t.w * inv) * g.w;
      } else {
        const float4 b = b4[c];
        t.x = ((t.x - mean) * inv) * g.x + b.x; t.y = ((t.y - mean) * inv) * g.y + b.y;
        t.z = ((t.z - mean) * inv) * g.z + b.z; t.w = ((t.w - mean) * inv) * g.w + b.w;
      }
      row[c] = t;
    }
  }
  __syncthreads();
}

// ------------------------------------------------------------------------------------------------
// Weight-streaming GEMV: y[m][n] = sum_k x[m][k] W[n][k], W row-major [n][k] read exactly once
// ([talker] MATVEC_SRC; [mimi] MATVEC, MV_LS).  One wave owns R rows at a time (a "tile") for all
// M input rows; lane l reads float4 columns l, l+64, ... of each row, so one load instruction of a
// wave covers 1 KiB of a row.  Each wave owns a contiguous, balanced range of tiles, and the first
// tile's weights are requested before anything that depends on x, so the HBM latency overlaps
// the input prologue.
// ------------------------------------------------------------------------------------------------
// Register-resident variant: k == 256*KB, and each lane keeps its KB float4 of every input row in
// registers, normalised by the wave itself (no LDS, no workgroup barrier).
// PRO_ATTN input row: this step's attention output.  With one chunk of legal slots the attention
// launch wrote it to x; otherwise it is combined here from the chunk partials (the attention's
// softmax, finished here): for each head, with M the largest chunk maximum,
// out = sum_c e^(M_c - M) O_c / sum_c e^(M_c - M) L_c ([talker] GQA_ATTN_SRC; [mimi] attn_src).
// Run by the whole workgroup.  The legal-slot count comes through the scalar cache; then the row,
// or every partial of up to IB chunks, is requested before `issue_weights` streams the weights, so
// the combine overlaps them.  Every load here is unconditional (indices are clamped to valid
// entries and unused values are never read): with no branches around them the compiler waits for
// the partials alone, not for the weights requested after them.
template <int KB>
struct CombineSmem {
  float4 xsh[KB * kWave];
  float msh[kAttnMaxPartials];
};

template <int KB, int IB, typename F>
__device__ __forceinline__ void attn_combine(const GemvArgs& a, uint32_t n_items, float4 (&xr)[KB],
                                             F issue_weights, CombineSmem<KB>& sm) {
  constexpr int K4 = KB * kWave;
  constexpr int PER = (K4 + kWgThreads - 1) / kWgThreads;  // row float4 per thread
  float4* xsh = sm.xsh;
  float* msh = sm.msh;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const uint32_t HD = a.head_dim, hq = a.k / HD, nc = a.n_chunks;
  const float* ml = a.part + static_cast<size_t>(hq) * nc * HD;
  float4 o[PER][IB];
  auto load_batch = [&](uint32_t i0) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const uint32_t c4 = min(static_cast<uint32_t>(tid + p * kWgThreads), static_cast<uint32_t>(K4 - 1));
      const uint32_t h = 4 * c4 / HD, d = 4 * c4 % HD;
#pragma unroll
      for (int i = 0; i < IB; ++i) {
        const uint32_t c = min(i0 + i, n_items - 1);
        o[p][i] = *reinterpret_cast<const float4*>(a.part + (static_cast<size_t>(h) * nc + c) * HD + d);
      }
    }
  };
  load_batch(0);
  // chunk weights e^(M_c - M) / L: 16 lanes per head (one DPP row), lane j of the row takes chunks
  // j, j + 16, ...; every head's (max, sum) pairs are requested before the weights, in straight
  // code (a load in a loop would make the wait for them cover the weights as well)
  constexpr int CPL = kAttnMaxChunks / 16;
  static_assert(kWgThreads / 16 == kAttnMaxHeads, "one DPP row per head");
  const uint32_t sub = lane & 15;
  const uint32_t h = tid / 16;  // rows past the last head work on a clamped copy, write nothing
  float mv[CPL], lv[CPL];
  {
    const uint32_t hc = min(h, hq - 1);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const uint32_t i = min(sub + 16u * j, n_items - 1);
      mv[j] = ml[(static_cast<size_t>(hc) * nc + i) * 2];
      lv[j] = ml[(static_cast<size_t>(hc) * nc + i) * 2 + 1];
    }
  }
  issue_weights();
  {
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < CPL; ++j)
      if (sub + 16u * j < n_items) mx = fmaxf(mx, mv[j]);
    mx = group_max<16>(mx);
    float l = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j)
      if (sub + 16u * j < n_items && mv[j] != -INFINITY) l = fmaf(__builtin_amdgcn_exp2f(mv[j] - mx), lv[j], l);
    l = group_sum<16>(l);
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    if (h < hq) {
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const uint32_t i = sub + 16u * j;
        if (i < n_items) msh[h * n_items + i] = mv[j] != -INFINITY ? __builtin_amdgcn_exp2f(mv[j] - mx) * inv : 0.f;
      }
    }
  }
  __syncthreads();
  float4 acc[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) acc[p] = f4zero();
  auto accumulate = [&](uint32_t i0) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const uint32_t c4 = min(static_cast<uint32_t>(tid + p * kWgThreads), static_cast<uint32_t>(K4 - 1));
      const uint32_t h = 4 * c4 / HD;
#pragma unroll
      for (int i = 0; i < IB; ++i) {
        const float w = i0 + i < n_items ? msh[h * n_items + i0 + i] : 0.f;
        acc[p].x = fmaf(w, o[p][i].x, acc[p].x); acc[p].y = fmaf(w, o[p][i].y, acc[p].y);
        acc[p].z = fmaf(w, o[p][i].z, acc[p].z); acc[p].w = fmaf(w, o[p][i].w, acc[p].w);
      }
    }
  };
  accumulate(0);  // the first batch outside the loop: its wait does not cover the weights
  for (uint32_t i0 = IB; i0 < n_items; i0 += IB) {
    load_batch(i0);  // more than IB chunks: these wait behind the weights
    accumulate(i0);
  }
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const uint32_t c4 = tid + p * kWgThreads;
    if (c4 < static_cast<uint32_t>(K4)) xsh[c4] = acc[p];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < KB; ++j) xr[j] = xsh[lane + kWave * j];
  if (a.x_tap != nullptr && blockIdx.x == 0)
    for (uint32_t c4 = tid; c4 < static_cast<uint32_t>(K4); c4 += kWgThreads)
      reinterpret_cast<float4*>(a.x_tap)[c4] = xsh[c4];
}

template <int KB, typename F>
__device__ __forceinline__ void attn_input(const GemvArgs& a, float4 (&xr)[KB], F issue_weights) {
  __shared__ CombineSmem<KB> sm;
  typedef const __attribute__((address_space(4))) uint32_t ConstU32;
  const uint32_t nl = *((ConstU32*)a.n_legal);
  const uint32_t n_items = min((nl + a.chunk - 1) / a.chunk, a.n_chunks);
  if (n_items <= 1) {
    const float4* x4 = reinterpret_cast<const float4*>(a.x);
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int j = 0; j < KB; ++j) xr[j] = x4[lane + kWave * j];
    issue_weights();
    if (a.x_tap != nullptr && blockIdx.x == 0)
      for (uint32_t c4 = threadIdx.x; c4 < static_cast<uint32_t>(KB * kWave); c4 += kWgThreads)
        reinterpret_cast<float4*>(a.x_tap)[c4] = x4[c4];
  } else if (n_items <= 4) {
    attn_combine<KB, 4>(a, n_items, xr, issue_weights, sm);
  } else if (n_items <= 8) {
    attn_combine<KB, 8>(a, n_items, xr, issue_weights, sm);
  } else {
    attn_combine<KB, 16>(a, n_items, xr, issue_weights, sm);
  }
}

// Workgroup blk of nblk (kWgThreads threads each).
template <int M, int R, int PRO, int EPI, int KB>
__device__ __forceinline__ void gemv_rx_body(const GemvArgs& a, uint32_t blk, uint32_t nblk) {
  constexpr int V = R * M;
  static_assert(V <= 64, "tile too large for one wave");
  constexpr int RH = EPI == EPI_SWIGLU ? R / 2 : R;
  const int lane = threadIdx.x & (kWave - 1);
  // Wave w owns tiles w, w + W, w + 2W, ... (W waves in the grid): at any moment the waves stream
  // neighbouring rows, which the DRAM pages serve better than far-apart contiguous ranges.
  const uint32_t n_tiles = (a.n_rows + RH - 1) / RH;
  const uint32_t ts = nblk * (kWgThreads / kWave);
  // wave-uniform, and known to be: the row and segment arithmetic stays scalar, so the weight
  // pointer is never fetched by a vector load (whose wait would also cover every tile in flight)
  uint32_t t = blk * (kWgThreads / kWave) +
               __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const uint32_t t_end = n_tiles;

  // Two of the wave's tiles of weight rows in flight: the one after next is requested as soon as a
  // tile is reduced.  The attention-combine variant keeps one (its registers hold the chunk
  // partials instead), and so do the 6144-wide rows: with one 24 KiB row per wave in flight the
  // rows reach DRAM in a more orderly stream (measured 10.3 vs 10.7 us for 2048 x 6144).
  constexpr bool kTwo = PRO != PRO_ATTN && KB != 24;
  float4 w0[KB][R], w1[kTwo ? KB : 1][R];
  ResPre p0, p1;
  auto load_tile = [&](uint32_t tt, float4 (&w)[KB][R], ResPre& p) {
    const float4* wr[R];
    tile_rows<R, EPI>(a, tt, wr);
#pragma unroll
    for (int j = 0; j < KB; ++j)
#pragma unroll
      for (int r = 0; r < R; ++r) w[j][r] = ldw(wr[r] + lane + kWave * j);
    p = residual_prefetch<M, R, EPI>(a, tt, lane);
  };
  auto load_first = [&]() {
    if constexpr (kTwo) {
      if (t < t_end) load_tile(t, w0, p0);
      if (t + ts < t_end) load_tile(t + ts, w1, p1);
    } else {
      // unconditional (a wave without a tile loads the last one and never uses it): no branch
      // here, so waits for loads issued before it need not cover these
      load_tile(t < t_end ? t : n_tiles - 1, w0, p0);
    }
  };

  float4 xr[M][KB];
  if constexpr (PRO == PRO_ATTN) {
    static_assert(M == 1, "the attention combine serves one stream");
    attn_input<KB>(a, xr[0], load_first);  // the whole workgroup takes part
    if (t >= t_end) return;
  } else {
    if (t >= t_end) return;
    // The small input row (and the norm gain and bias) are requested first: loads return in
    // order, so the norm arithmetic runs while the weight rows are still streaming in.
    const float4* x4 = reinterpret_cast<const float4*>(a.x);
    const uint32_t xs4 = a.x_stride >> 2;
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int j = 0; j < KB; ++j)
        xr[m][j] = m == 0 || m < static_cast<int>(a.m) ? x4[m * xs4 + lane + kWave * j] : f4zero();
  }
  float4 gr[PRO == PRO_RMS || PRO == PRO_LN ? KB : 1], br[PRO == PRO_LN ? KB : 1];
  if (PRO == PRO_RMS || PRO == PRO_LN) {
    const float4* g4 = reinterpret_cast<const float4*>(a.norm_w);
#pragma unroll
    for (int j = 0; j < KB; ++j) gr[j] = g4[lane + kWave * j];
  }
  if (PRO == PRO_LN) {
    const float4* b4 = reinterpret_cast<const float4*>(a.norm_b);
#pragma unroll
    for (int j = 0; j < KB; ++j) br[j] = b4[lane + kWave * j];
  }
  // Loads complete in issue order: keep the weight loads after the row and gain loads, so the norm
  // arithmetic does not wait for the first tile of weights.
  asm volatile("" ::: "memory");
  if constexpr (PRO != PRO_ATTN) load_first();

  if (PRO == PRO_RMS || PRO == PRO_LN) {
    const float kf = static_cast<float>(a.k);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float mean = 0.f, inv;
      if (PRO == PRO_RMS) {
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < KB; ++j) ss = dot4(xr[m][j], xr[m][j], ss);
        inv = rsqrtf(wave_sum(ss) * (1.0f / kf) + a.eps);
      } else {
        float sm = 0.f;
#pragma unroll
        for (int j = 0; j < KB; ++j) sm += (xr[m][j].x + xr[m][j].y) + (xr[m][j].z + xr[m][j].w);
        mean = wave_sum(sm) * (1.0f / kf);
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < KB; ++j) {
          float4 d = xr[m][j];
          d.x -= mean; d.y -= mean; d.z -= mean; d.w -= mean;
          ss = dot4(d, d, ss);
        }
        inv = rsqrtf(wave_sum(ss) * (1.0f / kf) + a.eps);
      }
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        const float4 g = gr[j];
        float4 v = xr[m][j];
        if (PRO == PRO_RMS) {
          v.x = (v.x * inv) * g.x; v.y = (v.y * inv) * g.y;
          v.z = (v.z * inv) * g.z; v.w = (v.w * inv) * g.w;
        } else {
          const float4 b = br[j];
          v.x = ((v.x - mean) * inv) * g.x + b.x; v.y = ((v.y - mean) * inv) * g.y + b.y;
          v.z = ((v.z - mean) * inv) * g.z + b.z; v.w = ((v.w - mean) * inv) * g.w + b.w;
        }
        xr[m][j] = m < static_cast<int>(a.m) ? v : f4zero();
      }
    }
  }

  auto reduce_tile = [&](uint32_t tt, const float4 (&w)[KB][R], const ResPre& p) {
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < KB; ++j)
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r * M + m] = dot4(w[j][r], xr[m][j], acc[r * M + m]);
    gemv_epilogue<M, R, EPI>(a, tt, acc, lane, &p);
  };
  if constexpr (kTwo) {
    // ping-pong between the two register buffers (unrolled: registers cannot be indexed)
    while (true) {
      reduce_tile(t, w0, p0);
      if (t + 2 * ts < t_end) load_tile(t + 2 * ts, w0, p0);
      if ((t += ts) >= t_end) break;
      reduce_tile(t, w1, p1);
      if (t + 2 * ts < t_end) load_tile(t + 2 * ts, w1, p1);
      if ((t += ts) >= t_end) break;
    }
  } else {
    while (true) {
      reduce_tile(t, w0, p0);
      if ((t += ts) >= t_end) break;
      load_tile(t, w0, p0);
    }
  }
}

template <int M, int R, int PRO, int EPI, int KB>
__global__ __launch_bounds__(kWgThreads) void k_gemv_rx(GemvArgs a) {
  gemv_rx_body<M, R, PRO, EPI, KB>(a, blockIdx.x, gridDim.x);
}

// ------------------------------------------------------------------------------------------------
// Short-context attention + o projection for one stream (at most kShortSlots legal slots): the
// attention of every head is computed inside the o-projection launch, so no attention launch sits
// between the q/k/v projection and this one.  A workgroup has 4 GEMV waves and NAW attention
// waves.  Attention wave a takes kv heads a*HPW .. a*HPW + HPW - 1 and their G query heads each
// ([talker] QK_NORM_SRC, ROPE_SRC, GQA_ATTN_SRC; [mimi] rope_push_src, attn_src): lane (group,
// sub) holds elements 8 sub .. 8 sub + 7 of a head row, so the raw q/k/v rows, the slot list and
// the ring rows arrive in two round trips and every cross-lane step is a DPP or permlane move:
// the qk-RMSNorm sums and the scores over the hd/8 lanes of a slot group, the rope partner
// (rotate_half: the lane hd/16 away), and the merge of the slot groups' online softmax states.
// The pushed slot is scored from registers by group 0.  The GEMV waves (k_gemv_rx's tile loop, R
// rows per wave) request their weights once the attention waves' ring rows have arrived, so those
// requests are not queued behind the weight stream; every workgroup computes the whole
// attention row (its ring rows come from L2), and workgroup 0 pushes this step's key and value.
// ------------------------------------------------------------------------------------------------

template <int HD, int G, int HPW>
__device__ __forceinline__ void short_attention_wave(const GemvArgs& a, int aw, float* out) {
  constexpr int LPS = HD / 8;            // lanes per slot row, 8 floats each
  constexpr int GPW = kWave / LPS;       // slot groups per wave
  constexpr int SPG = (static_cast<int>(kShortSlots) - 1 + GPW - 1) / GPW;  // older slots per group
  constexpr int HALF = HD / 2;
  const ShortAttnArgs& sa = a.sa;
  const int lane = threadIdx.x & (kWave - 1);
  const int grp = lane / LPS, sub = lane % LPS;
  const uint32_t hq = sa.n_q_heads, hkv = sa.n_kv_heads;
  const uint32_t g0 = static_cast<uint32_t>(aw) * HPW;
  // round trip 1: the slot count, this group's list entries (entry 0 is the pushed slot; group grp
  // takes entries 1 + grp + GPW j), this lane's 8 elements of the raw q, k, v rows, the norm gains
  // and the rope cos/sin of those elements
  const uint32_t nl = *sa.n_legal;
  const uint32_t push_slot = sa.st->slot;
  uint32_t slot[SPG];
#pragma unroll
  for (int j = 0; j < SPG; ++j)  // entries past the count hold anything: clamp the slot too
    slot[j] = min(sa.legal[min(1u + grp + GPW * j, sa.ring - 1)], sa.ring - 1);
  auto ld8 = [&](const float* p, float (&d)[8]) {
    const float4 u = reinterpret_cast<const float4*>(p)[0], v = reinterpret_cast<const float4*>(p)[1];
    d[0] = u.x; d[1] = u.y; d[2] = u.z; d[3] = u.w; d[4] = v.x; d[5] = v.y; d[6] = v.z; d[7] = v.w;
  };
  float q8[HPW][G][8], k8[HPW][8], v8[HPW][8], gq[8], gk[8], cv[8], sv[8];
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
#pragma unroll
    for (int q = 0; q < G; ++q) ld8(sa.qkv + static_cast<size_t>((g0 + h) * G + q) * HD + 8 * sub, q8[h][q]);
    ld8(sa.qkv + static_cast<size_t>(hq + g0 + h) * HD + 8 * sub, k8[h]);
    ld8(sa.qkv + static_cast<size_t>(hq + hkv + g0 + h) * HD + 8 * sub, v8[h]);
  }
  // round trip 2 starts as soon as the list is in: every older slot's key and value rows, then
  // the norm gains and the rope cos/sin (not needed before the rows arrive)
  float4 K[HPW][SPG][2], V[HPW][SPG][2];
  const size_t row = static_cast<size_t>(hkv) * HD;
#pragma unroll
  for (int h = 0; h < HPW; ++h)
#pragma unroll
    for (int j = 0; j < SPG; ++j) {
      const float4* kp = reinterpret_cast<const float4*>(sa.k_ring + slot[j] * row + (g0 + h) * HD + 8 * sub);
      const float4* vp = reinterpret_cast<const float4*>(sa.v_ring + slot[j] * row + (g0 + h) * HD + 8 * sub);
      K[h][j][0] = kp[0]; K[h][j][1] = kp[1];
      V[h][j][0] = vp[0]; V[h][j][1] = vp[1];
    }
  if (sa.q_norm) { ld8(sa.q_norm + 8 * sub, gq); ld8(sa.k_norm + 8 * sub, gk); }
  if (sa.rope_style == 0) {  // element d takes frequency d mod hd/2: 8 consecutive ones
    ld8(sa.cs + (8 * sub) % HALF, cv);
    ld8(sa.cs + HALF + (8 * sub) % HALF, sv);
  } else {                   // element d takes frequency d / 2: 4 consecutive ones, twice each
    const float4 c4 = reinterpret_cast<const float4*>(sa.cs + 4 * sub)[0];
    const float4 s4 = reinterpret_cast<const float4*>(sa.cs + HALF + 4 * sub)[0];
    cv[0] = cv[1] = c4.x; cv[2] = cv[3] = c4.y; cv[4] = cv[5] = c4.z; cv[6] = cv[7] = c4.w;
    sv[0] = sv[1] = s4.x; sv[2] = sv[3] = s4.y; sv[4] = sv[5] = s4.z; sv[6] = sv[7] = s4.w;
  }
  // (1) the ring rows are in: only now do the GEMV waves start their weight stream, so these
  // requests were not queued behind it; the math below overlaps the stream
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // rotate_half pairs element d with d + hd/2 (lower half: x c - x' s) and d - hd/2 (upper half:
  // x c + x' s): the sign goes into the sine once
  if (sa.rope_style == 0 && 8 * sub < HALF) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sv[e] = -sv[e];
  }
  // qk-RMSNorm over the hd/8 lanes of a group (the G queries and the key of a kv head at once,
  // so their reduction chains interleave), then rope
  auto rope = [&](float (&x)[8]) {
    float r[8];
    if (sa.rope_style == 0) {  // rotate_half: the partner element is hd/16 lanes away
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pr = lane_xor<HALF / 8>(x[e], lane);
        r[e] = fmaf(pr, sv[e], x[e] * cv[e]);
      }
    } else {  // interleaved: pairs (2i, 2i + 1) inside the lane
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float xa = x[2 * i], xb = x[2 * i + 1];
        r[2 * i] = xa * cv[2 * i] - xb * sv[2 * i];
        r[2 * i + 1] = xa * sv[2 * i] + xb * cv[2 * i];
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = r[e];
  };
  // scores in log2 units: exponentials are single exp2 instructions; with the qk-norm the scale
  // rides on the query's normalisation, otherwise it multiplies each score
  const float scale = 1.4426950408889634f / sqrtf(static_cast<float>(HD));
  const float sscale = sa.q_norm ? 1.0f : scale;
  constexpr int NS = 1 + SPG;  // the pushed slot, then this group's older slots
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    const uint32_t g = g0 + h;
    if (sa.q_norm) {
      float ss[G + 1];
#pragma unroll
      for (int q = 0; q <= G; ++q) {
        const float* x = q < G ? q8[h][q] : k8[h];
        float t = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) t = fmaf(x[e], x[e], t);
        ss[q] = t;
      }
#pragma unroll
      for (int q = 0; q <= G; ++q) ss[q] = group_sum<LPS>(ss[q]);
#pragma unroll
      for (int q = 0; q <= G; ++q) {
        const float inv = rsqrtf(ss[q] / static_cast<float>(HD) + sa.eps) * (q < G ? scale : 1.0f);
        float* x = q < G ? q8[h][q] : k8[h];
        const float* gn = q < G ? gq : gk;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (x[e] * inv) * gn[e];
      }
    }
#pragma unroll
    for (int q = 0; q < G; ++q) rope(q8[h][q]);
    rope(k8[h]);
    // every score of the group first (independent dot products and reductions), then the
    // group's max, the exponentials and the sums: slot 0 is the pushed one (group 0 only)
    float sc[NS][G];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      float kf[8];
      if (j == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) kf[e] = k8[h][e];
      } else {
        const float4 k0 = K[h][j - 1][0], k1 = K[h][j - 1][1];
        kf[0] = k0.x; kf[1] = k0.y; kf[2] = k0.z; kf[3] = k0.w;
        kf[4] = k1.x; kf[5] = k1.y; kf[6] = k1.z; kf[7] = k1.w;
      }
#pragma unroll
      for (int q = 0; q < G; ++q) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d = fmaf(q8[h][q][e], kf[e], d);
        sc[j][q] = d;
      }
    }
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
      for (int q = 0; q < G; ++q) sc[j][q] = group_sum<LPS>(sc[j][q]);
    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int q = 0; q < G; ++q) {
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const uint32_t ent = j == 0 ? 0u : 1u + grp + GPW * (j - 1);
        const bool live = j == 0 ? grp == 0 : (ent < nl && ent < kShortSlots);
        sc[j][q] = live ? sc[j][q] * sscale : -INFINITY;
        mx = fmaxf(mx, sc[j][q]);
      }
      m[q] = mx;
      l[q] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[q][e] = 0.f;
      if (mx != -INFINITY) {
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          const float p = __builtin_amdgcn_exp2f(sc[j][q] - mx);  // 0 for a masked slot
          l[q] += p;
          if (j == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[q][e] = fmaf(p, v8[h][e], acc[q][e]);
          } else {
            const float4 v0 = V[h][j - 1][0], v1 = V[h][j - 1][1];
            acc[q][0] = fmaf(p, v0.x, acc[q][0]); acc[q][1] = fmaf(p, v0.y, acc[q][1]);
            acc[q][2] = fmaf(p, v0.z, acc[q][2]); acc[q][3] = fmaf(p, v0.w, acc[q][3]);
            acc[q][4] = fmaf(p, v1.x, acc[q][4]); acc[q][5] = fmaf(p, v1.y, acc[q][5]);
            acc[q][6] = fmaf(p, v1.z, acc[q][6]); acc[q][7] = fmaf(p, v1.w, acc[q][7]);
          }
        }
      }
    }
    // merge the slot groups: first every group's (max, sum) with its partners LPS, 2 LPS, ... lanes
    // apart, so each group knows the overall max and can rescale its sums; then reduce-scatter the
    // G x 8 rescaled output sums, halving the values per step, so each element ends in one group
    float M[G];
#pragma unroll
    for (int q = 0; q < G; ++q) M[q] = m[q];
#pragma unroll
    for (int off = LPS; off < kWave; off <<= 1)
#pragma unroll
      for (int q = 0; q < G; ++q) {
        if (off == 8) M[q] = fmaxf(M[q], lane_xor<8>(M[q], lane));
        else if (off == 16) M[q] = pair_max<16>(M[q]);
        else M[q] = pair_max<32>(M[q]);
      }
    float vals[G * 8 + G];  // rescaled output sums, then the rescaled denominators
#pragma unroll
    for (int q = 0; q < G; ++q) {
      const float c = m[q] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[q] - M[q]);
#pragma unroll
      for (int e = 0; e < 8; ++e) vals[q * 8 + e] = acc[q][e] * c;
      vals[G * 8 + q] = l[q] * c;
    }
    // the denominators are summed in full (every group needs them); the outputs reduce-scatter
#pragma unroll
    for (int q = 0; q < G; ++q) {
      float t = vals[G * 8 + q];
      if constexpr (LPS <= 8) t += lane_xor<8>(t, lane);
      if constexpr (LPS <= 16) t = pair_sum<16>(t);
      t = pair_sum<32>(t);
      vals[G * 8 + q] = t;
    }
    constexpr int NV = G * 8;
    static_assert(NV == 8 || NV == 16, "reduce-scatter of 8 or 16 values");
    float* r = vals;
    // step over 32 lanes: the lower half keeps values [0, NV/2), the upper half [NV/2, NV)
    {
#pragma unroll
      for (int i = 0; i < NV / 2; ++i) r[i] = halves_sum(r[i], r[i + NV / 2]);
    }
    int nv = NV / 2;
    // step over 16 lanes (when groups are 16 lanes or narrower)
    if constexpr (LPS <= 16) {
#pragma unroll
      for (int i = 0; i < NV / 4; ++i) r[i] = rows16_sum(r[i], r[i + NV / 4]);
      nv = NV / 4;
    }
    if constexpr (LPS <= 8) {  // and over 8 lanes: rows of 16 hold two groups of 8
#pragma unroll
      for (int i = 0; i < NV / 8; ++i) {
        const bool upper = (lane & 8) != 0;
        const float send = upper ? r[i] : r[i + NV / 8];
        const float keep = upper ? r[i + NV / 8] : r[i];
        r[i] = keep + lane_xor<8>(send, lane);
      }
      nv = NV / 8;
    }
    // group k (of GPW) now holds values [k nv, (k + 1) nv) of the G x 8 sums: the value index of
    // r[i] follows the halving order -- upper half of 32 lanes took the upper half of the values,
    // odd rows of 16 the upper half of the rest, upper 8 lanes the upper half after that
    {
      const int hi32 = (lane & 32) ? 1 : 0, hi16 = (lane & 16) ? 1 : 0, hi8 = (lane & 8) ? 1 : 0;
      int base = hi32 * (NV / 2);
      if constexpr (LPS <= 16) base += hi16 * (NV / 4);
      if constexpr (LPS <= 8) base += hi8 * (NV / 8);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        if (i < nv) {
          const int v = base + i;            // value index: query v / 8, element v % 8
          const int q = v / 8, e = v % 8;
          const float den = vals[G * 8 + q];
          out[static_cast<size_t>(g * G + q) * HD + 8 * sub + e] = r[i] * __builtin_amdgcn_rcpf(den);
        }
      }
    }
  }
  // workgroup 0 pushes this step's roped keys and values into ring slot pos mod R, after its
  // attention row is out (nothing in this launch reads them back)
  __syncthreads();  // (2) the attention row is in LDS
  if (blockIdx.x == 0 && grp == 0) {
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
      const size_t roff = (static_cast<size_t>(push_slot) * hkv + g0 + h) * HD + 8 * sub;
      float4* kd = reinterpret_cast<float4*>(sa.k_ring + roff);
      float4* vd = reinterpret_cast<float4*>(sa.v_ring + roff);
      kd[0] = make_float4(k8[h][0], k8[h][1], k8[h][2], k8[h][3]);
      kd[1] = make_float4(k8[h][4], k8[h][5], k8[h][6], k8[h][7]);
      vd[0] = make_float4(v8[h][0], v8[h][1], v8[h][2], v8[h][3]);
      vd[1] = make_float4(v8[h][4], v8[h][5], v8[h][6], v8[h][7]);
    }
  }
}

// Rows per GEMV tile of k_attn_short_o for an input row of 256 KB floats (every SIMD of a
// 256-CU device gets a tile at the workloads' widths).
constexpr int short_o_rows(int kb) { return kb == 2 ? 4 : kb == 4 ? 1 : 2; }

template <int HD, int G, int HPW, int NAW, int KB>
__global__ __launch_bounds__(kWgThreads + NAW * kWave) void k_attn_short_o(GemvArgs a) {
  constexpr int M = 1, EPI = EPI_RESIDUAL, R = short_o_rows(KB);
  constexpr int NGW = kWgThreads / kWave;  // GEMV waves; the attention waves follow them
  static_assert(R * M <= kWave, "tile too large for one wave");
  __shared__ float4 xsh[KB * kWave];       // this step's attention output row
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if (wave >= NGW) {
    short_attention_wave<HD, G, HPW>(a, wave - NGW, reinterpret_cast<float*>(xsh));
    return;  // it has passed barrier (2)
  }
  const uint32_t n_tiles = (a.n_rows + R - 1) / R;
  const uint32_t ts = gridDim.x * NGW;
  uint32_t t = blockIdx.x * NGW + wave;
  float4 w0[KB][R];
  ResPre p0;
  // rows [r0, r1) of a tile (then the old residual): the first tile's rows below
  // sa.early_rows are requested before the attention waves' ring rows are in, the rest after
  auto load_tile = [&](uint32_t tt, int r0, int r1) {
    const float4* wr[R];
    tile_rows<R, EPI>(a, tt, wr);
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r >= r0 && r < r1) {
#pragma unroll
        for (int j = 0; j < KB; ++j) w0[j][r] = ldw(wr[r] + lane + kWave * j);
      }
    if (r1 == R) p0 = residual_prefetch<M, R, EPI>(a, tt, lane);
  };
  // unconditional (a wave without a tile loads the last one and never uses it)
  const uint32_t t0 = t < n_tiles ? t : n_tiles - 1;
  const int early = a.sa.early_rows < R ? a.sa.early_rows : R;
  load_tile(t0, 0, early);
  __syncthreads();  // (1) the attention waves' ring rows have arrived
  load_tile(t0, early, R);
  __syncthreads();  // (2) the attention waves have left the attention row in LDS
  float4 xr[KB];
#pragma unroll
  for (int j = 0; j < KB; ++j) xr[j] = xsh[lane + kWave * j];
  if (a.x_tap != nullptr && blockIdx.x == 0)
    for (uint32_t c4 = threadIdx.x; c4 < static_cast<uint32_t>(KB * kWave); c4 += kWgThreads)
      reinterpret_cast<float4*>(a.x_tap)[c4] = xsh[c4];
  while (t < n_tiles) {
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;
#pragma unroll
    for (int j = 0; j < KB; ++j)
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = dot4(w0[j][r], xr[j], acc[r]);
    gemv_epilogue<M, R, EPI>(a, t, acc, lane, &p0);
    if ((t += ts) >= n_tiles) break;
    load_tile(t, 0, R);
  }
}

// Generic variant: any k (multiple of 4).  With a norm prologue the input rows are staged in LDS;
// without one they are read from global memory (they stay in L1/L2).
template <int M, int R, int PRO, int EPI>
__global__ __launch_bounds__(kWgThreads) void k_gemv(GemvArgs a) {
  extern __shared__ float4 xs[];
  constexpr int U = M <= 2 ? 8 : (M <= 4 ? 4 : 2);
  constexpr int V = R * M;
  static_assert(V <= 64, "tile too large for one wave");
  constexpr int RH = EPI == EPI_SWIGLU ? R / 2 : R;
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t K4 = a.k >> 2;
  const uint32_t n_iter = (K4 + kWave * U - 1) / (kWave * U);
  uint32_t t, t_end;
  wave_tiles((a.n_rows + RH - 1) / RH, t, t_end);

  const float4* wr[R];
  float4 wv[U][R];
  auto load_chunk = [&](uint32_t it) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t c = lane + kWave * (U * it + u);
#pragma unroll
      for (int r = 0; r < R; ++r) wv[u][r] = c < K4 ? ldw(wr[r] + c) : f4zero();
    }
  };
  bool prefetched = false;
  if (t < t_end) {
    tile_rows<R, EPI>(a, t, wr);
    load_chunk(0);
    prefetched = true;
  }
  if (PRO != PRO_NONE) stage_x<M, PRO>(a, xs, K4);  // every wave reaches the barriers inside
  const float4* x4 = reinterpret_cast<const float4*>(a.x);
  const uint32_t xstride4 = a.x_stride >> 2;

  for (; t < t_end; ++t) {
    if (!prefetched) tile_rows<R, EPI>(a, t, wr);
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    for (uint32_t it = 0; it < n_iter; ++it) {
      if (!prefetched) load_chunk(it);
      prefetched = false;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t c = lane + kWave * (U * it + u);
        if (c < K4) {
#pragma unroll
          for (int m = 0; m < M; ++m) {
            float4 xv;
            if (PRO != PRO_NONE) xv = xs[m * K4 + c];
            else xv = m < static_cast<int>(a.m) ? x4[m * xstride4 + c] : f4zero();
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r * M + m] = dot4(wv[u][r], xv, acc[r * M + m]);
          }
        }
      }
    }
    gemv_epilogue<M, R, EPI>(a, t, acc, lane);
  }
}

// ------------------------------------------------------------------------------------------------
// Ring attention, split over slot chunks ([mimi] attn_src: legality from the position ring, a
// masked slot weighs nothing; [talker] GQA_ATTN_SRC: kv head = q head / group, scale 1/sqrt(hd)).
// Grid (chunk, kv head, stream).  Each workgroup first finishes this step's queries of its GQA
// group (qk-norm + rope, in LDS); the workgroup whose chunk holds slot pos mod R also finishes
// this step's key and pushes it, roped, with the raw value into the rings ([talker] APPEND_SRC;
// [mimi] rope_push_src).  The chunk's legal slots are compacted, so masked slots cost no K/V
// traffic.  Slot groups of hd/8 lanes (8 dims per lane) walk the legal slots with an online
// softmax for all G query heads, so each K/V row is read once for the whole GQA group.  Groups
// merge in LDS; chunks merge in the last workgroup to finish, in ascending chunk order.
// ------------------------------------------------------------------------------------------------
template <int HD, int G>
__global__ __launch_bounds__(kWgThreads) void k_attention(AttnArgs a) {
  __shared__ AttnSmem<HD, G, kWgThreads> sm;
  // one pass over a default-size chunk: all of a group's key and value rows in flight at once
  constexpr int UNR = HD >= 128 ? 8 : 4;
  attention_item<HD, G, kWgThreads, false, UNR>(a, blockIdx.x, blockIdx.y, blockIdx.z, sm);
}

// Split form for streams with long rings: grid (item, kv head, stream), n_chunks items per
// (stream, kv head) sharing its legal slots evenly, two passes of keys and values in flight.
template <int HD, int G>
__global__ __launch_bounds__(kWgThreads) void k_attention_split(AttnArgs a) {
  __shared__ AttnSmem<HD, G, kWgThreads, kAttnSplitList> sm;
  attention_item<HD, G, kWgThreads, false, 4, 0, true, kAttnSplitList>(a, blockIdx.x, blockIdx.y,
                                                                       blockIdx.z, sm);
}

// ------------------------------------------------------------------------------------------------
// Row-stream GEMV for one stream: each wave holds one weight row (KB float4 per lane) in flight and
// walks rows t, t + W, t + 2W, ... (W waves in the grid), so at any moment the device streams a
// dense band of whole rows, one row per wave ([talker] build_step_plan; [mimi] MV_LS).  For
// SwiGLU the walk covers the gate rows and then the up rows (n_rows must be a multiple of W); a
// wave's gate sums wait in lane k of one register until its up row k arrives.
// ------------------------------------------------------------------------------------------------
template <int KB, int PRO, int EPI>
__device__ __forceinline__ void gemv_rows_body(const GemvArgs& a, uint32_t blk, uint32_t nblk) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t W = nblk * (kWgThreads / kWave);
  const uint32_t t = blk * (kWgThreads / kWave) +
                     __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const uint32_t n = a.n_rows;
  const uint32_t total = EPI == EPI_SWIGLU ? 2 * n : n;
  if (t >= total) return;
  auto row_ptr = [&](uint32_t r) {
    const float* base = a.w[0];
    if (EPI == EPI_SWIGLU) {
      if (r >= n) {
        base = a.w[1];
        r -= n;
      }
    } else if (r >= a.seg_end[1]) {
      base = a.w[2];
      r -= a.seg_end[1];
    } else if (r >= a.seg_end[0]) {
      base = a.w[1];
      r -= a.seg_end[0];
    }
    return reinterpret_cast<const float4*>(base + static_cast<size_t>(r) * a.k) + lane;
  };
  const float4* x4 = reinterpret_cast<const float4*>(a.x);
  float4 xr[KB], gr[PRO == PRO_NONE ? 1 : KB], br[PRO == PRO_LN ? KB : 1];
#pragma unroll
  for (int j = 0; j < KB; ++j) xr[j] = x4[lane + kWave * j];
  if (PRO != PRO_NONE) {
#pragma unroll
    for (int j = 0; j < KB; ++j) gr[j] = reinterpret_cast<const float4*>(a.norm_w)[lane + kWave * j];
  }
  if (PRO == PRO_LN) {
#pragma unroll
    for (int j = 0; j < KB; ++j) br[j] = reinterpret_cast<const float4*>(a.norm_b)[lane + kWave * j];
  }
  asm volatile("" ::: "memory");  // the input row (and gains) are requested before the weights
  float4 w[KB];
  float res_old = 0.f, ls_v = 1.f;
  auto load = [&](uint32_t r) {
    const float4* wr = row_ptr(r);
#pragma unroll
    for (int j = 0; j < KB; ++j) w[j] = ldw(wr + kWave * j);
    if (EPI == EPI_RESIDUAL) {
      res_old = (a.res_in ? a.res_in : a.res)[r];
      if (a.ls) ls_v = a.ls[r];
    }
  };
  load(t);
  __builtin_amdgcn_sched_barrier(0);  // and they are requested before the norm arithmetic waits

  if (PRO != PRO_NONE) {
    const float kf = static_cast<float>(a.k);
    float mean = 0.f;
    if (PRO == PRO_LN) {
      float sm = 0.f;
#pragma unroll
      for (int j = 0; j < KB; ++j) sm += (xr[j].x + xr[j].y) + (xr[j].z + xr[j].w);
      mean = wave_sum(sm) * (1.0f / kf);
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      float4 d = xr[j];
      d.x -= mean; d.y -= mean; d.z -= mean; d.w -= mean;
      ss = dot4(d, d, ss);
    }
    const float inv = rsqrtf(wave_sum(ss) * (1.0f / kf) + a.eps);
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      float4 v = xr[j];
      const float4 g = gr[j];
      if (PRO == PRO_RMS) {
        v.x = (v.x * inv) * g.x; v.y = (v.y * inv) * g.y;
        v.z = (v.z * inv) * g.z; v.w = (v.w * inv) * g.w;
      } else {
        const float4 b = br[j];
        v.x = ((v.x - mean) * inv) * g.x + b.x; v.y = ((v.y - mean) * inv) * g.y + b.y;
        v.z = ((v.z - mean) * inv) * g.z + b.z; v.w = ((v.w - mean) * inv) * g.w + b.w;
      }
      xr[j] = v;
    }
  }

  const uint32_t K = n / W;  // SwiGLU: gate rows per wave
  float gates = 0.f;          // SwiGLU: lane k holds the wave's k-th gate sum
  uint32_t k = 0;
  for (uint32_t r = t;; r += W, ++k) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < KB; ++j) acc = dot4(w[j], xr[j], acc);
    const float v = wave_sum(acc);
    const float res_here = res_old, ls_here = ls_v;
    const bool more = r + W < total;
    if (more) load(r + W);  // the next row streams while this one's result is written
    if (EPI == EPI_SWIGLU) {
      if (k < K) {
        if (static_cast<uint32_t>(lane) == k) gates = v;
      } else {
        const float g = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gates), k - K));
        if (lane == 0) a.y[r - n] = silu(g) * v;
      }
    } else if (lane == 0) {
      if (EPI == EPI_STORE) {
        a.y[r] = v;
      } else if (EPI == EPI_GELU) {
        a.y[r] = gelu_erf(v);
      } else {
        if (a.tap) a.tap[r] = v;
        a.res[r] = res_here + (a.ls ? ls_here * v : v);
      }
    }
    if (!more) return;
  }
}

template <int KB, int PRO, int EPI>
__global__ __launch_bounds__(kWgThreads) void k_gemv_rows(GemvArgs a) {
  gemv_rows_body<KB, PRO, EPI>(a, blockIdx.x, gridDim.x);
}


// ------------------------------------------------------------------------------------------------
// Split-k GEMV for M input rows (m streams, or the rows of a prefill block), k = NW*256*KW: the
// workgroup's NW waves take the NW slices of k, so a wave keeps only its slice of all M input
// rows in registers (M*KW float4 per lane) and every weight float4 it loads meets all M rows
// there: the M-row step reads each weight once ([talker] MATVEC_SRC loops the m rows per weight
// read; [mimi] MV_LS).  Row slot rr of workgroup b is unit b + (rr mod U) * G as in k_gemv_ks; the
// slice sums and the per-row norm statistics meet in LDS.
// ------------------------------------------------------------------------------------------------
template <int M, int NW, int KW, int RB, int PRO, int EPI>
__global__ __launch_bounds__(NW * kWave) void k_gemv_ksm(GemvArgs a) {
  constexpr int U = EPI == EPI_SWIGLU ? RB / 2 : RB;
  constexpr int V = RB * M;
  static_assert(V <= kWave && kWave % V == 0 && (EPI != EPI_SWIGLU || RB % 2 == 0), "tile");
  __shared__ float part[NW][V];
  __shared__ float stat[2][M][NW];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const uint32_t n = a.n_rows, G = gridDim.x, mv = a.m;
  const uint32_t off = static_cast<uint32_t>(wave) * (KW * kWave) + lane;  // float4 in the row
  const float4* x4 = reinterpret_cast<const float4*>(a.x);
  const uint32_t xs4 = a.x_stride >> 2;
  float4 xr[M][KW], gr[PRO == PRO_NONE ? 1 : KW], br[PRO == PRO_LN ? KW : 1];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int j = 0; j < KW; ++j) xr[m][j] = x4[min(static_cast<uint32_t>(m), mv - 1) * xs4 + off + kWave * j];
  if (PRO != PRO_NONE) {
#pragma unroll
    for (int j = 0; j < KW; ++j) gr[j] = reinterpret_cast<const float4*>(a.norm_w)[off + kWave * j];
  }
  if (PRO == PRO_LN) {
#pragma unroll
    for (int j = 0; j < KW; ++j) br[j] = reinterpret_cast<const float4*>(a.norm_b)[off + kWave * j];
  }
  float4 w[RB][KW];
  auto row_base = [&](uint32_t u, int rr) {
    const float* base = a.w[0];
    uint32_t row = u;
    if (EPI == EPI_SWIGLU) {
      base = rr < U ? a.w[0] : a.w[1];
    } else if (row >= a.seg_end[1]) {
      base = a.w[2];
      row -= a.seg_end[1];
    } else if (row >= a.seg_end[0]) {
      base = a.w[1];
      row -= a.seg_end[0];
    }
    return reinterpret_cast<const float4*>(base + static_cast<size_t>(row) * a.k) + off;
  };
  // thread tid writes output (unit slot tid / M, row tid % M) when tid < U*M; every thread requests
  // the old residual and LayerScale of slot tid % (U*M) (unconditional, duplicates unused)
  const uint32_t es = static_cast<uint32_t>(tid) % (U * M);
  const uint32_t e_u = es / M, e_m = es % M;
  float res_old = 0.f, ls_v = 1.f;
  auto load = [&](uint32_t u0) {
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      const float4* wr = row_base(min(u0 + (rr % U) * G, n - 1), rr);
#pragma unroll
      for (int j = 0; j < KW; ++j) w[rr][j] = ldw(wr + kWave * j);
    }
    if (EPI == EPI_RESIDUAL) {
      const uint32_t u = min(u0 + e_u * G, n - 1);
      res_old = (a.res_in ? a.res_in : a.res)[min(e_m, mv - 1) * a.res_stride + u];
      if (a.ls) ls_v = a.ls[u];
    }
  };
  asm volatile("" ::: "memory");  // the input slices (and gains) are requested before the rows
  uint32_t u0 = blockIdx.x;
  load(u0);
  __builtin_amdgcn_sched_barrier(0);

  // RMSNorm: the products use g * x and the epilogue scales each row's sums by that row's 1/rms,
  // so no workgroup barrier stands between the input rows' arrival and the first products (the
  // slices' sums of squares go to LDS here and are read after the first tile's barrier)
  constexpr bool LATE_RMS = PRO == PRO_RMS;
  const float rk_late = 1.0f / static_cast<float>(a.k);
  if constexpr (LATE_RMS) {
    float st[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < KW; ++j) ss = dot4(xr[m][j], xr[m][j], ss);
      st[m] = ss;
    }
#pragma unroll
    for (int m = 0; m < M; ++m) st[m] = wave_sum(st[m]);
    if (lane == 0) {
#pragma unroll
      for (int m = 0; m < M; ++m) stat[1][m][wave] = st[m];
    }
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int j = 0; j < KW; ++j) {
        float4 v = xr[m][j];
        const float4 g = gr[j];
        v.x *= g.x; v.y *= g.y; v.z *= g.z; v.w *= g.w;
        xr[m][j] = v;
      }
  } else if (PRO != PRO_NONE) {  // per input row: statistics of the whole row from the NW slices
    // Each phase runs over all M rows before the next (the sums, then the cross-lane reductions,
    // then one guarded LDS write per row), so the M independent reduction chains interleave
    // instead of running one after another between exec-mask switches.
    const float kf = static_cast<float>(a.k), rk = 1.0f / kf;
    float mean[M], st[M];
#pragma unroll
    for (int m = 0; m < M; ++m) mean[m] = 0.f;
    if (PRO == PRO_LN) {
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float sm = 0.f;
#pragma unroll
        for (int j = 0; j < KW; ++j) sm += (xr[m][j].x + xr[m][j].y) + (xr[m][j].z + xr[m][j].w);
        st[m] = sm;
      }
#pragma unroll
      for (int m = 0; m < M; ++m) st[m] = wave_sum(st[m]);
      if (lane == 0) {
#pragma unroll
        for (int m = 0; m < M; ++m) stat[0][m][wave] = st[m];
      }
      __syncthreads();
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float tot = 0.f;
#pragma unroll
        for (int q = 0; q < NW; ++q) tot += stat[0][m][q];
        mean[m] = tot * rk;
      }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < KW; ++j) {
        float4 d = xr[m][j];
        d.x -= mean[m]; d.y -= mean[m]; d.z -= mean[m]; d.w -= mean[m];
        ss = dot4(d, d, ss);
      }
      st[m] = ss;
    }
#pragma unroll
    for (int m = 0; m < M; ++m) st[m] = wave_sum(st[m]);
    if (lane == 0) {
#pragma unroll
      for (int m = 0; m < M; ++m) stat[1][m][wave] = st[m];
    }
    __syncthreads();
    float invs[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float tot = 0.f;
#pragma unroll
      for (int q = 0; q < NW; ++q) tot += stat[1][m][q];
      // one reciprocal square root instruction (within 1 ulp of 1 / sqrt) and a product by
      // 1 / k: 8 rows of correctly rounded divisions and square roots cost about 1.1 us per launch
      invs[m] = rsqrtf(tot * rk + a.eps);
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float inv = invs[m];
#pragma unroll
      for (int j = 0; j < KW; ++j) {
        float4 v = xr[m][j];
        const float4 g = gr[j];
        if (PRO == PRO_RMS) {
          v.x = (v.x * inv) * g.x; v.y = (v.y * inv) * g.y;
          v.z = (v.z * inv) * g.z; v.w = (v.w * inv) * g.w;
        } else {
          const float4 b = br[j];
          v.x = ((v.x - mean[m]) * inv) * g.x + b.x; v.y = ((v.y - mean[m]) * inv) * g.y + b.y;
          v.z = ((v.z - mean[m]) * inv) * g.z + b.z; v.w = ((v.w - mean[m]) * inv) * g.w + b.w;
        }
        xr[m][j] = v;
      }
    }
  }
#pragma unroll
  for (int m = 0; m < M; ++m)  // rows past the valid ones contribute nothing
#pragma unroll
    for (int j = 0; j < KW; ++j) xr[m][j] = static_cast<uint32_t>(m) < mv ? xr[m][j] : f4zero();

  for (;;) {
    float acc[V];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr)
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float d = 0.f;
#pragma unroll
        for (int j = 0; j < KW; ++j) d = dot4(w[rr][j], xr[m][j], d);
        acc[rr * M + m] = d;
      }
    ReduceScatter<V, 32>::run(acc, lane);  // lane (64/V)*i holds value i's slice sum
    if (lane % (kWave / V) == 0) part[wave][lane / (kWave / V)] = acc[0];
    __syncthreads();
    const uint32_t base = u0;
    const float res_here = res_old, ls_here = ls_v;
    u0 += G * U;
    if (u0 < n) load(u0);  // the next rows stream while this tile's results are written
    if (static_cast<uint32_t>(tid) < U * M) {
      const uint32_t u = base + e_u * G;
      if (u < n && e_m < mv) {
        float v = 0.f;
#pragma unroll
        for (int q = 0; q < NW; ++q) v += part[q][e_u * M + e_m];
        float rs = 1.f;  // LATE_RMS: 1/rms of input row e_m
        if constexpr (LATE_RMS) {
          float tot = 0.f;
#pragma unroll
          for (int q = 0; q < NW; ++q) tot += stat[1][e_m][q];
          rs = rsqrtf(tot * rk_late + a.eps);
          v *= rs;
        }
        if (EPI == EPI_SWIGLU) {
          float up = 0.f;
#pragma unroll
          for (int q = 0; q < NW; ++q) up += part[q][(e_u + U) * M + e_m];
          a.y[e_m * a.y_stride + u] = silu(v) * (up * rs);
        } else if (EPI == EPI_STORE) {
          a.y[e_m * a.y_stride + u] = v;
        } else if (EPI == EPI_GELU) {
          a.y[e_m * a.y_stride + u] = gelu_erf(v);
        } else {
          if (a.tap) a.tap[e_m * a.tap_stride + u] = v;
          a.res[e_m * a.res_stride + u] = res_here + (a.ls ? ls_here * v : v);
        }
      }
    }
    if (u0 >= n) return;
    __syncthreads();  // part is rewritten by the next tile
  }
}

// ------------------------------------------------------------------------------------------------
// Split-k GEMV for one stream (k = 1024*KW), with the norm prologues and every epilogue of the
// register GEMV ([talker] build_step_plan; [mimi] MV_LS).  The workgroup's four waves take the
// four quarters of each of its RB rows, so a wave keeps only its quarter of the (normalised) input
// in registers and the rows of all workgroups are in flight at once; the quarter sums, and the
// norm statistics, meet in LDS.  Row slot rr of workgroup b is unit b + (rr mod U) * G (G
// workgroups; a unit is a row, or for SwiGLU a gate row and its up row, U units per workgroup):
// at any moment the device streams a dense band of whole rows.
// ------------------------------------------------------------------------------------------------
template <int KW, int RB, int PRO, int EPI>
__global__ __launch_bounds__(kWgThreads) void k_gemv_ks(GemvArgs a) {
  constexpr int NW = kWgThreads / kWave;
  constexpr int U = EPI == EPI_SWIGLU ? RB / 2 : RB;
  static_assert(NW == 4 && RB <= kWave && (EPI != EPI_SWIGLU || RB % 2 == 0), "tile shape");
  __shared__ float part[NW][RB];
  __shared__ float stat[2][NW];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const uint32_t n = a.n_rows, G = gridDim.x;
  const uint32_t off = static_cast<uint32_t>(wave) * (KW * kWave) + lane;  // float4 in the row
  const float4* x4 = reinterpret_cast<const float4*>(a.x);
  float4 xr[KW], gr[PRO == PRO_NONE ? 1 : KW], br[PRO == PRO_LN ? KW : 1];
#pragma unroll
  for (int j = 0; j < KW; ++j) xr[j] = x4[off + kWave * j];
  if (PRO != PRO_NONE) {
#pragma unroll
    for (int j = 0; j < KW; ++j) gr[j] = reinterpret_cast<const float4*>(a.norm_w)[off + kWave * j];
  }
  if (PRO == PRO_LN) {
#pragma unroll
    for (int j = 0; j < KW; ++j) br[j] = reinterpret_cast<const float4*>(a.norm_b)[off + kWave * j];
  }
  float4 w[RB][KW];
  auto row_base = [&](uint32_t u, int rr) {
    const float* base = a.w[0];
    uint32_t row = u;
    if (EPI == EPI_SWIGLU) {
      base = rr < U ? a.w[0] : a.w[1];
    } else if (row >= a.seg_end[1]) {
      base = a.w[2];
      row -= a.seg_end[1];
    } else if (row >= a.seg_end[0]) {
      base = a.w[1];
      row -= a.seg_end[0];
    }
    return reinterpret_cast<const float4*>(base + static_cast<size_t>(row) * a.k) + off;
  };
  // every thread requests the old residual and LayerScale of unit slot tid % U (unconditional
  // loads: threads past U fetch duplicates that are never used)
  float res_old = 0.f, ls_v = 1.f;
  auto load = [&](uint32_t u0) {
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      const float4* wr = row_base(min(u0 + (rr % U) * G, n - 1), rr);
#pragma unroll
      for (int j = 0; j < KW; ++j) w[rr][j] = ldw(wr + kWave * j);
    }
    if (EPI == EPI_RESIDUAL) {
      const uint32_t u = min(u0 + (tid % U) * G, n - 1);
      res_old = (a.res_in ? a.res_in : a.res)[u];
      if (a.ls) ls_v = a.ls[u];
    }
  };
  asm volatile("" ::: "memory");  // the input quarter (and gains) are requested before the rows
  uint32_t u0 = blockIdx.x;
  load(u0);
  __builtin_amdgcn_sched_barrier(0);  // the rows are requested before the norm arithmetic waits

  if (PRO != PRO_NONE) {  // the norm statistics of the whole row, from the four quarters
    const float kf = static_cast<float>(a.k);
    float mean = 0.f;
    if (PRO == PRO_LN) {
      float sm = 0.f;
#pragma unroll
      for (int j = 0; j < KW; ++j) sm += (xr[j].x + xr[j].y) + (xr[j].z + xr[j].w);
      sm = wave_sum(sm);
      if (lane == 0) stat[0][wave] = sm;
      __syncthreads();
      mean = ((stat[0][0] + stat[0][1]) + (stat[0][2] + stat[0][3])) * (1.0f / kf);
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < KW; ++j) {
      float4 d = xr[j];
      d.x -= mean; d.y -= mean; d.z -= mean; d.w -= mean;
      ss = dot4(d, d, ss);
    }
    ss = wave_sum(ss);
    if (lane == 0) stat[1][wave] = ss;
    __syncthreads();
    const float inv = rsqrtf(((stat[1][0] + stat[1][1]) + (stat[1][2] + stat[1][3])) * (1.0f / kf) + a.eps);
#pragma unroll
    for (int j = 0; j < KW; ++j) {
      float4 v = xr[j];
      const float4 g = gr[j];
      if (PRO == PRO_RMS) {
        v.x = (v.x * inv) * g.x; v.y = (v.y * inv) * g.y;
        v.z = (v.z * inv) * g.z; v.w = (v.w * inv) * g.w;
      } else {
        const float4 b = br[j];
        v.x = ((v.x - mean) * inv) * g.x + b.x; v.y = ((v.y - mean) * inv) * g.y + b.y;
        v.z = ((v.z - mean) * inv) * g.z + b.z; v.w = ((v.w - mean) * inv) * g.w + b.w;
      }
      xr[j] = v;
    }
  }

  for (;;) {
    float acc[RB];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      acc[rr] = 0.f;
#pragma unroll
      for (int j = 0; j < KW; ++j) acc[rr] = dot4(w[rr][j], xr[j], acc[rr]);
    }
    ReduceScatter<RB, 32>::run(acc, lane);  // lane (64/RB)*rr holds row slot rr's quarter sum
    if (lane % (kWave / RB) == 0) part[wave][lane / (kWave / RB)] = acc[0];
    __syncthreads();
    const uint32_t base = u0;
    const float res_here = res_old, ls_here = ls_v;
    u0 += G * U;
    if (u0 < n) load(u0);  // the next rows stream while this tile's results are written
    if (tid < U) {
      const uint32_t u = base + tid * G;
      if (u < n) {
        const float v = (part[0][tid] + part[1][tid]) + (part[2][tid] + part[3][tid]);
        if (EPI == EPI_SWIGLU) {
          const float up = (part[0][tid + U] + part[1][tid + U]) + (part[2][tid + U] + part[3][tid + U]);
          a.y[u] = silu(v) * up;
        } else if (EPI == EPI_STORE) {
          a.y[u] = v;
        } else if (EPI == EPI_GELU) {
          a.y[u] = gelu_erf(v);
        } else {
          if (a.tap) a.tap[u] = v;
          a.res[u] = res_here + (a.ls ? ls_here * v : v);
        }
      }
    }
    if (u0 >= n) return;
    __syncthreads();  // part is rewritten by the next tile
  }
}

// ------------------------------------------------------------------------------------------------
// Step begin: copy the caller's rows into the residual stream, start fresh streams (every
// position-ring slot empty), stamp pos into slot pos mod R of each stream's position ring
// ([mimi] rope_push_src: pr[slot] = pos), and form this position's rope cos/sin in float64
// ([talker] TalkerGpu::load builds its tables on the CPU; rounding once to float32).
// ------------------------------------------------------------------------------------------------
// Legal-slot lists of the step begin are formed from per-wave 64-slot ballots kept in LDS: rings of
// up to 64 * kBeginMaxChunks slots (larger rings take the scan of compact_legal).
constexpr uint32_t kBeginMaxChunks = 1024;

struct BeginSmem {
  unsigned long long masks[kBeginMaxChunks];
  uint32_t wcount[kWgThreads / kWave];
  uint32_t scan[kWgThreads];
};

// Workgroup s of the step begin: s < m takes stream s, s == m the rope table and the state.
__device__ __forceinline__ void begin_body(const BeginArgs& a, uint32_t s, BeginSmem& sm) {
  unsigned long long* masks = sm.masks;
  uint32_t* wcount = sm.wcount;
  uint32_t* scan = sm.scan;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const uint32_t slot = a.pos % a.ring;
  if (s == a.m) {  // workgroup-uniform: the float64 trig runs beside the streams' compaction
    const uint32_t half = a.head_dim >> 1;
    if (static_cast<uint32_t>(tid) < half) {
      const double inv_freq = pow(a.theta, -2.0 * static_cast<double>(tid) /
                                               static_cast<double>(a.head_dim));
      const double ang = static_cast<double>(a.pos) * inv_freq;
      a.cs[tid] = static_cast<float>(cos(ang));
      a.cs[half + tid] = static_cast<float>(sin(ang));
    }
    if (tid == 0) {
      a.st->pos = a.pos;
      a.st->slot = slot;
      a.st->x_out = a.x_out;
    }
    return;
  }
  // the caller's row is requested together with the position ring (one round trip)
  const float4* src = reinterpret_cast<const float4*>(a.x_in + static_cast<size_t>(s) * a.d);
  float4* dst = reinterpret_cast<float4*>(a.xres + static_cast<size_t>(s) * a.d);
  const uint32_t d4 = a.d >> 2;
  float4 xv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t i = tid + u * kWgThreads;
    xv[u] = i < d4 ? src[i] : f4zero();
  }
  uint32_t* P = a.pos_rings + static_cast<size_t>(s) * a.ring;
  uint32_t* out = a.legal + static_cast<size_t>(s) * a.ring;
  const uint32_t R = a.ring;
  const uint32_t nch = (R + kWave - 1) / kWave;  // 64-slot chunks
  if (nch > kBeginMaxChunks) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t i = tid + u * kWgThreads;
      if (i < d4) dst[i] = xv[u];
    }
    for (uint32_t i = tid + 4 * kWgThreads; i < d4; i += kWgThreads) dst[i] = src[i];
    if (a.first) {
      for (uint32_t i = tid; i < R; i += kWgThreads) P[i] = i == slot ? a.pos : kInvalidPos;
    } else if (tid == 0) {
      P[slot] = a.pos;
    }
    __syncthreads();
    compact_legal<kWgThreads, false>(P, R, a.pos, a.window, static_cast<int>(slot), out,
                                     a.n_legal + s, scan);
    return;
  }
  // Wave w takes chunks [w cpw, (w + 1) cpw); lane l of a chunk c tests slot 64 c + l.  The slot
  // pushed now is listed first and left out of the ballots, so the stamp below never matters to
  // them; a fresh stream (first) has no other legal slot.  The ring words of a batch of 8 chunks
  // are requested together ([mimi] attn_src: legal iff P != INVALID, P <= pos, pos - P < window).
  const uint32_t cpw = (nch + kWgThreads / kWave - 1) / (kWgThreads / kWave);
  const uint32_t c0 = min(static_cast<uint32_t>(wave) * cpw, nch), c1 = min(c0 + cpw, nch);
  uint32_t cnt = 0;
  if (!a.first) {
    for (uint32_t cb = c0; cb < c1; cb += 8) {
      uint32_t pv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) pv[j] = P[min((cb + j) * kWave + lane, R - 1)];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t c = cb + j, sl = c * kWave + lane;
        const uint32_t p = pv[j];
        const bool legal = c < c1 && sl < R && sl != slot && p != kInvalidPos && p <= a.pos &&
                           a.pos - p < a.window;
        const unsigned long long m = __ballot(legal);
        if (c < c1 && lane == 0) masks[c] = m;
        cnt += c < c1 ? static_cast<uint32_t>(__popcll(m)) : 0u;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t i = tid + u * kWgThreads;
    if (i < d4) dst[i] = xv[u];
  }
  for (uint32_t i = tid + 4 * kWgThreads; i < d4; i += kWgThreads) dst[i] = src[i];
  if (a.first) {
    for (uint32_t i = tid; i < R; i += kWgThreads) P[i] = i == slot ? a.pos : kInvalidPos;
  } else if (tid == 0) {
    P[slot] = a.pos;
  }
  if (lane == 0) wcount[wave] = cnt;
  __syncthreads();
  uint32_t o = 1, total = 1;
  for (int w = 0; w < kWgThreads / kWave; ++w) {
    o += w < wave ? wcount[w] : 0u;
    total += wcount[w];
  }
  if (!a.first) {
    const unsigned long long below = lane ? (~0ull >> (kWave - lane)) : 0ull;
    for (uint32_t c = c0; c < c1; ++c) {
      const unsigned long long m = masks[c];
      if ((m >> lane) & 1ull) out[o + __popcll(m & below)] = c * kWave + lane;
      o += static_cast<uint32_t>(__popcll(m));
    }
  }
  if (tid == 0) {
    out[0] = slot;
    a.n_legal[s] = total;
  }
}

__global__ __launch_bounds__(kWgThreads) void k_begin(BeginArgs a) {
  __shared__ BeginSmem sm;
  begin_body(a, blockIdx.x, sm);
}

// The first layer's normed q/k/v projection and the step begin in one launch: workgroups
// [0, gemv_wgs) stream the q/k/v rows from the caller's row (which the begin workgroups copy into
// the residual stream for the later layers), the m + 1 after them do the step begin.
template <int KB, int PRO>
__global__ __launch_bounds__(kWgThreads) void k_qkv_begin(QkvBeginArgs a) {
  __shared__ BeginSmem sm;
  if (blockIdx.x < a.gemv_wgs) gemv_rows_body<KB, PRO, EPI_STORE>(a.g, blockIdx.x, a.gemv_wgs);
  else begin_body(a.b, blockIdx.x - a.gemv_wgs, sm);
}
// The same with the register GEMV (tiles of R rows; the codec and FlowLM widths).
template <int R, int PRO, int KB>
__global__ __launch_bounds__(kWgThreads) void k_qkv_begin_rx(QkvBeginArgs a) {
  __shared__ BeginSmem sm;
  if (blockIdx.x < a.gemv_wgs) gemv_rx_body<1, R, PRO, EPI_STORE, KB>(a.g, blockIdx.x, a.gemv_wgs);
  else begin_body(a.b, blockIdx.x - a.gemv_wgs, sm);
}

// Multi-position begin ([talker] TalkerGpu::prefill → forward_rows): the m rows are positions
// pos .. pos+m-1 of one stream.  Every row's slot is stamped before any row's legal list is formed;
// with pos + m <= R or R >= window + m - 1 no stamp removes a position an earlier row of the
// block may attend, so row r's list is exactly the one a single step at pos + r would form.
//
// Workgroup r < m forms row r's list; workgroup m writes every row's rope table and the state.
// A row's workgroup reads the ring as it stands after the whole block's stamps without waiting for
// them: a slot of the block holds pos + (its distance from the block's first slot), any other
// slot is empty after `first` and otherwise unchanged, so the one value the stamps would change
// is computed, not read.  The list is the lead slot then the other legal slots in ascending
// order, as the single-workgroup form below builds it.
__global__ __launch_bounds__(kWgThreads) void k_begin_rows_wg(BeginArgs a) {
  __shared__ BeginSmem sm;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const uint32_t r = blockIdx.x, rows = a.m, R = a.ring;
  const uint32_t base = a.pos % R;
  if (r == rows) {
    const uint32_t half = a.head_dim >> 1;
    for (uint32_t i = tid; i < rows * half; i += kWgThreads) {
      const uint32_t rr = i / half, j = i % half;
      const double inv_freq = pow(a.theta, -2.0 * static_cast<double>(j) /
                                               static_cast<double>(a.head_dim));
      const double ang = static_cast<double>(a.pos + rr) * inv_freq;
      a.cs[static_cast<size_t>(rr) * a.head_dim + j] = static_cast<float>(cos(ang));
      a.cs[static_cast<size_t>(rr) * a.head_dim + half + j] = static_cast<float>(sin(ang));
    }
    if (tid == 0 && a.st != nullptr) {
      a.st->pos = a.pos + rows - 1;
      a.st->slot = (base + rows - 1) % R;
    }
    return;
  }
  const uint32_t pos_r = a.pos + r, slot_r = (base + r) % R;
  uint32_t* P = a.pos_rings;
  // the ring after the block's stamps
  auto stamped = [&](uint32_t j, uint32_t old) {
    const uint32_t k = j >= base ? j - base : j + R - base;
    return k < rows ? a.pos + k : (a.first ? kInvalidPos : old);
  };
  const uint32_t nch = (R + kWave - 1) / kWave;
  const uint32_t cpw = (nch + kWgThreads / kWave - 1) / (kWgThreads / kWave);
  const uint32_t c0 = min(static_cast<uint32_t>(wave) * cpw, nch), c1 = min(c0 + cpw, nch);
  uint32_t cnt = 0;
  for (uint32_t cb = c0; cb < c1; cb += 8) {
    uint32_t pv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) pv[j] = a.first ? kInvalidPos : P[min((cb + j) * kWave + lane, R - 1)];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t c = cb + j, sl = c * kWave + lane;
      const uint32_t p = stamped(min(sl, R - 1), pv[j]);
      const bool legal = c < c1 && sl < R && sl != slot_r && p != kInvalidPos && p <= pos_r &&
                         pos_r - p < a.window;
      const unsigned long long m = __ballot(legal);
      if (c < c1 && lane == 0) sm.masks[c] = m;
      cnt += c < c1 ? static_cast<uint32_t>(__popcll(m)) : 0u;
    }
  }
  const float4* src = reinterpret_cast<const float4*>(a.x_in + static_cast<size_t>(r) * a.d);
  float4* dst = reinterpret_cast<float4*>(a.xres + static_cast<size_t>(r) * a.d);
  for (uint32_t i = tid; i < (a.d >> 2); i += kWgThreads) dst[i] = src[i];
  if (a.first) {
    for (uint32_t j = r * kWgThreads + tid; j < R; j += rows * kWgThreads) P[j] = stamped(j, 0u);
  } else if (tid == 0) {
    P[slot_r] = pos_r;
  }
  if (lane == 0) sm.wcount[wave] = cnt;
  __syncthreads();
  uint32_t o = 1, total = 1;
  for (int w = 0; w < kWgThreads / kWave; ++w) {
    o += w < wave ? sm.wcount[w] : 0u;
    total += sm.wcount[w];
  }
  uint32_t* out = a.legal + static_cast<size_t>(r) * R;
  const unsigned long long below = lane ? (~0ull >> (kWave - lane)) : 0ull;
  for (uint32_t c = c0; c < c1; ++c) {
    const unsigned long long m = sm.masks[c];
    if ((m >> lane) & 1ull) out[o + __popcll(m & below)] = c * kWave + lane;
    o += static_cast<uint32_t>(__popcll(m));
  }
  if (tid == 0) {
    out[0] = slot_r;
    a.n_legal[r] = total;
  }
}

// The same in one workgroup, rows one after another (rings of more than kBeginMaxChunks * 64
// slots).
__global__ __launch_bounds__(kWgThreads) void k_begin_rows(BeginArgs a) {
  __shared__ uint32_t scan[kWgThreads];
  const int tid = threadIdx.x;
  const uint32_t rows = a.m;
  const float4* src = reinterpret_cast<const float4*>(a.x_in);
  float4* dst = reinterpret_cast<float4*>(a.xres);
  for (uint32_t i = tid; i < rows * (a.d >> 2); i += kWgThreads) dst[i] = src[i];
  uint32_t* P = a.pos_rings;
  const uint32_t base_slot = a.pos % a.ring;
  if (a.first) {
    for (uint32_t j = tid; j < a.ring; j += kWgThreads) {
      const uint32_t r = (j + a.ring - base_slot) % a.ring;  // the row whose slot j is, if any
      P[j] = r < rows ? a.pos + r : kInvalidPos;
    }
  } else {
    for (uint32_t r = tid; r < rows; r += kWgThreads) P[(base_slot + r) % a.ring] = a.pos + r;
  }
  __syncthreads();
  for (uint32_t r = 0; r < rows; ++r) {
    compact_legal<kWgThreads, false>(P, a.ring, a.pos + r, a.window,
                                     static_cast<int>((base_slot + r) % a.ring),
                                     a.legal + static_cast<size_t>(r) * a.ring, a.n_legal + r, scan);
    __syncthreads();  // the scan buffer is reused by the next row
  }
  const uint32_t half = a.head_dim >> 1;
  for (uint32_t i = tid; i < rows * half; i += kWgThreads) {
    const uint32_t r = i / half, j = i % half;
    const double inv_freq = pow(a.theta, -2.0 * static_cast<double>(j) /
                                             static_cast<double>(a.head_dim));
    const double ang = static_cast<double>(a.pos + r) * inv_freq;
    a.cs[static_cast<size_t>(r) * a.head_dim + j] = static_cast<float>(cos(ang));
    a.cs[static_cast<size_t>(r) * a.head_dim + half + j] = static_cast<float>(sin(ang));
  }
  if (tid == 0 && a.st != nullptr) {
    a.st->pos = a.pos + rows - 1;
    a.st->slot = (base_slot + rows - 1) % a.ring;
  }
}

// Key/value push of a block of rows: one wave per (row, kv head); lane j owns rope pair j, as in
// the attention item that pushes a single step's key ([talker] QK_NORM_SRC, ROPE_SRC, append).
template <int HD>
__global__ __launch_bounds__(kWave) void k_push(PushArgs a) {
  constexpr int HALF = HD / 2;
  const uint32_t r = blockIdx.x, g = blockIdx.y;
  const int lane = threadIdx.x;
  const float* row = a.qkv + static_cast<size_t>(r) * a.qkv_stride;
  const float* k = row + static_cast<size_t>(a.n_q_heads + g) * HD;
  const float* v = row + static_cast<size_t>(a.n_q_heads + a.n_kv_heads + g) * HD;
  const int ia = a.rope_style == 0 ? lane : 2 * lane;
  const int ib = a.rope_style == 0 ? lane + HALF : 2 * lane + 1;
  float va = lane < HALF ? k[ia] : 0.f, vb = lane < HALF ? k[ib] : 0.f;
  norm_rope_pair<HD>(va, vb, lane, a.k_norm, a.eps, a.cs + static_cast<size_t>(r) * HD,
                     a.rope_style);
  const uint32_t slot = (a.pos % a.ring + r) % a.ring;
  const size_t roff = (static_cast<size_t>(slot) * a.n_kv_heads + g) * HD;
  if (lane < HALF) {
    a.k_ring[roff + ia] = va;
    a.k_ring[roff + ib] = vb;
  }
  for (int d = lane; d < HD; d += kWave) a.v_ring[roff + d] = v[d];
}

// The legal-slot lists of m streams (one workgroup per stream) for the one-shot attention call.
__global__ __launch_bounds__(kWgThreads) void k_compact_legal(const uint32_t* pos_rings,
                                                              uint32_t ring, uint32_t pos,
                                                              uint32_t window, uint32_t* legal,
                                                              uint32_t* n_legal) {
  __shared__ uint32_t scan[kWgThreads];
  const uint32_t s = blockIdx.x;
  compact_legal<kWgThreads, false>(pos_rings + static_cast<size_t>(s) * ring, ring, pos, window,
                                   -1, legal + static_cast<size_t>(s) * ring, n_legal + s, scan);
}

// Step end: the output rows -- the final norm of the residual stream ([talker] build_step_plan's
// closing RMSNorm) or the residual stream itself ([mimi] transformer_shaped works in place).
// Rows of up to 4096 floats: the row, the gain and the bias are requested in one round trip and
// held in registers (16 floats per thread); the statistics meet in LDS.
__global__ __launch_bounds__(kWgThreads) void k_end(EndArgs a) {
  __shared__ float red[2][kWgThreads / kWave];
  const uint32_t r = blockIdx.x;
  const float* x = a.xres + static_cast<size_t>(r) * a.d;
  float* y = (a.x_out != nullptr ? a.x_out : a.st->x_out) + static_cast<size_t>(r) * a.d;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const uint32_t d4 = a.d >> 2;
  if (a.norm < 0 || d4 > 4 * kWgThreads) {  // a copy, or a row wider than the register tile
    if (a.norm < 0) {
      for (uint32_t i = tid; i < a.d; i += blockDim.x) y[i] = x[i];
      return;
    }
    const float df = static_cast<float>(a.d);
    float s = 0.f;
    for (uint32_t i = tid; i < a.d; i += blockDim.x) s += x[i];
    s = wave_sum(s);
    if (lane == 0) red[0][wave] = s;
    __syncthreads();
    const float mean = a.norm == PRO_LN ? ((red[0][0] + red[0][1]) + (red[0][2] + red[0][3])) * (1.0f / df) : 0.f;
    float ss = 0.f;
    for (uint32_t i = tid; i < a.d; i += blockDim.x) {
      const float v = x[i] - mean;
      ss = fmaf(v, v, ss);
    }
    ss = wave_sum(ss);
    if (lane == 0) red[1][wave] = ss;
    __syncthreads();
    const float inv = rsqrtf(((red[1][0] + red[1][1]) + (red[1][2] + red[1][3])) * (1.0f / df) + a.eps);
    for (uint32_t i = tid; i < a.d; i += blockDim.x) {
      if (a.norm == PRO_LN) y[i] = ((x[i] - mean) * inv) * a.w[i] + a.b[i];
      else y[i] = (x[i] * inv) * a.w[i];
    }
    return;
  }
  static_assert(kWgThreads / kWave == 4, "four partial sums");
  const float4* x4 = reinterpret_cast<const float4*>(x);
  const float4* w4 = reinterpret_cast<const float4*>(a.w);
  const float4* b4 = reinterpret_cast<const float4*>(a.b);
  float4 xv[4], wv[4], bv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t i = min(tid + u * kWgThreads, d4 - 1);  // clamped; lanes past the row add 0
    xv[u] = x4[i];
    wv[u] = w4[i];
    bv[u] = a.norm == PRO_LN ? b4[i] : f4zero();
  }
  const float df = static_cast<float>(a.d);
  float mean = 0.f;
  if (a.norm == PRO_LN) {
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (tid + u * kWgThreads < d4) s += (xv[u].x + xv[u].y) + (xv[u].z + xv[u].w);
    s = wave_sum(s);
    if (lane == 0) red[0][wave] = s;
    __syncthreads();
    mean = ((red[0][0] + red[0][1]) + (red[0][2] + red[0][3])) * (1.0f / df);
  }
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (tid + u * kWgThreads < d4) {
      float4 v = xv[u];
      v.x -= mean; v.y -= mean; v.z -= mean; v.w -= mean;
      ss = dot4(v, v, ss);
    }
  }
  ss = wave_sum(ss);
  if (lane == 0) red[1][wave] = ss;
  __syncthreads();
  const float inv = rsqrtf(((red[1][0] + red[1][1]) + (red[1][2] + red[1][3])) * (1.0f / df) + a.eps);
  float4* y4 = reinterpret_cast<float4*>(y);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t i = tid + u * kWgThreads;
    if (i < d4) {
      const float4 v = xv[u], g = wv[u], bb = bv[u];
      float4 o;
      if (a.norm == PRO_LN) {
        o.x = ((v.x - mean) * inv) * g.x + bb.x; o.y = ((v.y - mean) * inv) * g.y + bb.y;
        o.z = ((v.z - mean) * inv) * g.z + bb.z; o.w = ((v.w - mean) * inv) * g.w + bb.w;
      } else {
        o.x = (v.x * inv) * g.x; o.y = (v.y * inv) * g.y;
        o.z = (v.z * inv) * g.z; o.w = (v.w * inv) * g.w;
      }
      y4[i] = o;
    }
  }
}

__global__ void k_fill_u32(uint32_t* p, uint32_t v, uint64_t n) {
  for (uint64_t i = blockIdx.x * static_cast<uint64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<uint64_t>(gridDim.x) * blockDim.x)
    p[i] = v;
}
__global__ void k_fill_f32(float* p, float v, uint64_t n) {
  for (uint64_t i = blockIdx.x * static_cast<uint64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<uint64_t>(gridDim.x) * blockDim.x)
    p[i] = v;
}

// The kernel a launch plan names, and its dynamic LDS.
struct GemvKernel {
  const void* fn;
  size_t lds;
};

template <int M, int R, int PRO, int EPI>
GemvKernel gemv_generic(uint32_t k) {
  return {reinterpret_cast<const void*>(&k_gemv<M, R, PRO, EPI>),
          PRO == PRO_NONE ? 0 : static_cast<size_t>(M) * k * sizeof(float)};
}

template <int M, int R, int PRO, int EPI>
GemvKernel gemv_rx(int kb) {
  switch (kb) {
    case 2: return {reinterpret_cast<const void*>(&k_gemv_rx<M, R, PRO, EPI, 2>), 0};
    case 8: return {reinterpret_cast<const void*>(&k_gemv_rx<M, R, PRO, EPI, 8>), 0};
    case 4:  // k = 1024 (the FlowLM backbone)
      if constexpr (M == 1) return {reinterpret_cast<const void*>(&k_gemv_rx<M, R, PRO, EPI, 4>), 0};
      break;
    case 16:  // k = 4096 (the FlowLM FFN down projection)
      if constexpr (M == 1 && R == 1)
        return {reinterpret_cast<const void*>(&k_gemv_rx<M, R, PRO, EPI, 16>), 0};
      break;
    case 24:
      if constexpr (M == 1 && R == 1)
        return {reinterpret_cast<const void*>(&k_gemv_rx<M, R, PRO, EPI, 24>), 0};
      break;
    default: break;
  }
  return {nullptr, 0};
}

template <int M, int PRO, int EPI>
GemvKernel gemv_pick_r(const GemvLaunch& l, uint32_t k) {
  if (l.kb > 0) {
    if constexpr (M <= 2) {
      switch (l.rows_per_wave) {
        case 1:
          if constexpr (EPI != EPI_SWIGLU) return gemv_rx<M, 1, PRO, EPI>(l.kb);
          break;
        case 2: return gemv_rx<M, 2, PRO, EPI>(l.kb);
        case 4:
          if constexpr (M == 1) return gemv_rx<M, 4, PRO, EPI>(l.kb);
          break;
        default: break;
      }
    }
    return {nullptr, 0};
  }
  switch (l.rows_per_wave) {
    case 1:
      if constexpr (EPI != EPI_SWIGLU) return gemv_generic<M, 1, PRO, EPI>(k);
      break;
    case 2: return gemv_generic<M, 2, PRO, EPI>(k);
    case 4: return gemv_generic<M, 4, PRO, EPI>(k);
    default: break;
  }
  return {nullptr, 0};
}

// The attention-combine prologue: one stream, register-resident input rows of 512 or 2048.
template <int R>
GemvKernel gemv_rx_attn(int kb) {
  if (kb == 2) return {reinterpret_cast<const void*>(&k_gemv_rx<1, R, PRO_ATTN, EPI_RESIDUAL, 2>), 0};
  if (kb == 8) return {reinterpret_cast<const void*>(&k_gemv_rx<1, R, PRO_ATTN, EPI_RESIDUAL, 8>), 0};
  if (kb == 4) return {reinterpret_cast<const void*>(&k_gemv_rx<1, R, PRO_ATTN, EPI_RESIDUAL, 4>), 0};
  return {nullptr, 0};
}

// The multi-row split-k kernels: ks = KW (float4 per lane per row slice), waves_per_wg = NW,
// rows_per_wave = rows per workgroup tile.
template <int M, int NW, int KW, int RB>
GemvKernel gemv_ksm_kind(const GemvLaunch& l) {
#define SDEC_KSM(P, E) \
  if (l.prologue == P && l.epilogue == E) \
    return {reinterpret_cast<const void*>(&k_gemv_ksm<M, NW, KW, RB, P, E>), 0};
  SDEC_KSM(PRO_NONE, EPI_STORE)
  SDEC_KSM(PRO_NONE, EPI_RESIDUAL)
  SDEC_KSM(PRO_RMS, EPI_STORE)
  SDEC_KSM(PRO_LN, EPI_STORE)
  SDEC_KSM(PRO_RMS, EPI_SWIGLU)
  SDEC_KSM(PRO_RMS, EPI_GELU)
  SDEC_KSM(PRO_LN, EPI_SWIGLU)
  SDEC_KSM(PRO_LN, EPI_GELU)
#undef SDEC_KSM
  return {nullptr, 0};
}
template <int M>
GemvKernel gemv_ksm(const GemvLaunch& l) {
  if constexpr (M == 16) {
    // sixteen rows (prefill blocks past eight): one float4 per lane and row, k = 256 * waves
    if (l.ks != 1) return {nullptr, 0};
    if (l.waves_per_wg == 2 && l.rows_per_wave == 4) return gemv_ksm_kind<M, 2, 1, 4>(l);
    if (l.waves_per_wg == 2 && l.rows_per_wave == 2) return gemv_ksm_kind<M, 2, 1, 2>(l);
    if (l.waves_per_wg == 4 && l.rows_per_wave == 4) return gemv_ksm_kind<M, 4, 1, 4>(l);
    if (l.waves_per_wg == 4 && l.rows_per_wave == 2) return gemv_ksm_kind<M, 4, 1, 2>(l);
    if (l.waves_per_wg == 8 && l.rows_per_wave == 4) return gemv_ksm_kind<M, 8, 1, 4>(l);
    if (l.waves_per_wg == 8 && l.rows_per_wave == 2) return gemv_ksm_kind<M, 8, 1, 2>(l);
    return {nullptr, 0};
  }
  if (l.waves_per_wg == 4 && l.ks == 2 && l.rows_per_wave == 4) return gemv_ksm_kind<M, 4, 2, 4>(l);
  if (l.waves_per_wg == 8 && l.ks == 3 && l.rows_per_wave == 2) return gemv_ksm_kind<M, 8, 3, 2>(l);
  // k = 512 and 1024 (the codec and FlowLM widths): one float4 per lane and row in each slice
  if (l.waves_per_wg == 2 && l.ks == 1 && l.rows_per_wave == 4) return gemv_ksm_kind<M, 2, 1, 4>(l);
  if (l.waves_per_wg == 2 && l.ks == 1 && l.rows_per_wave == 2) return gemv_ksm_kind<M, 2, 1, 2>(l);
  if (l.waves_per_wg == 4 && l.ks == 1 && l.rows_per_wave == 4) return gemv_ksm_kind<M, 4, 1, 4>(l);
  if (l.waves_per_wg == 4 && l.ks == 1 && l.rows_per_wave == 2) return gemv_ksm_kind<M, 4, 1, 2>(l);
  if constexpr (M == 8) {  // taller tiles: every tile of the launch in flight in one round
    if (l.waves_per_wg == 4 && l.ks == 2 && l.rows_per_wave == 8) return gemv_ksm_kind<M, 4, 2, 8>(l);
    if (l.waves_per_wg == 8 && l.ks == 3 && l.rows_per_wave == 4) return gemv_ksm_kind<M, 8, 3, 4>(l);
  }
  return {nullptr, 0};
}

// The row-stream kernels: k = 256*kb.
template <int KB>
GemvKernel gemv_stream_kb(const GemvLaunch& l) {
#define SDEC_RS(P, E) \
  if (l.prologue == P && l.epilogue == E) return {reinterpret_cast<const void*>(&k_gemv_rows<KB, P, E>), 0};
  SDEC_RS(PRO_NONE, EPI_STORE)
  SDEC_RS(PRO_NONE, EPI_RESIDUAL)
  SDEC_RS(PRO_RMS, EPI_STORE)
  SDEC_RS(PRO_LN, EPI_STORE)
  SDEC_RS(PRO_RMS, EPI_SWIGLU)
  SDEC_RS(PRO_RMS, EPI_GELU)
  SDEC_RS(PRO_LN, EPI_SWIGLU)
  SDEC_RS(PRO_LN, EPI_GELU)
#undef SDEC_RS
  return {nullptr, 0};
}
GemvKernel gemv_stream(const GemvLaunch& l) {
  if (l.kb == 8) return gemv_stream_kb<8>(l);
  return {nullptr, 0};
}

// The split-k kernel the planner picks: the down projection at one stream (k = 6144, four-row
// tiles, residual epilogue).  Quarter-row split-k for the k = 2048 projections measured slower
// than the row stream and is not instantiated.
GemvKernel gemv_ks(const GemvLaunch& l) {
  if (l.ks == 6 && l.rows_per_wave == 4 && l.prologue == PRO_NONE && l.epilogue == EPI_RESIDUAL)
    return {reinterpret_cast<const void*>(&k_gemv_ks<6, 4, PRO_NONE, EPI_RESIDUAL>), 0};
  return {nullptr, 0};
}

// The short-context attention + o kernels: (head_dim, group, kv heads per attention wave,
// attention waves) of the workloads, input row of 256 * kb floats.
template <int HD, int G, int HPW, int NAW>
GemvKernel gemv_short_kb(int kb) {
  switch (kb) {
    case 2: return {reinterpret_cast<const void*>(&k_attn_short_o<HD, G, HPW, NAW, 2>), 0};
    case 4: return {reinterpret_cast<const void*>(&k_attn_short_o<HD, G, HPW, NAW, 4>), 0};
    case 8: return {reinterpret_cast<const void*>(&k_attn_short_o<HD, G, HPW, NAW, 8>), 0};
    default: return {nullptr, 0};
  }
}
GemvKernel gemv_short(const GemvLaunch& l) {
  if (l.epilogue != EPI_RESIDUAL || l.rows_per_wave != short_o_rows(l.kb)) return {nullptr, 0};
  const int naw = l.waves_per_wg - kWgThreads / kWave;
  if (l.attn_hd == 128 && l.attn_g == 2 && l.attn_hpw == 1 && naw == 8) return gemv_short_kb<128, 2, 1, 8>(l.kb);
  if (l.attn_hd == 128 && l.attn_g == 2 && l.attn_hpw == 1 && naw == 4) return gemv_short_kb<128, 2, 1, 4>(l.kb);
  if (l.attn_hd == 64 && l.attn_g == 1 && l.attn_hpw == 1 && naw == 8) return gemv_short_kb<64, 1, 1, 8>(l.kb);
  return {nullptr, 0};
}

template <int M>
GemvKernel gemv_pick_m(const GemvLaunch& l, uint32_t k) {
  if (l.prologue == PRO_ATTN_SHORT) {
    if constexpr (M == 1) return gemv_short(l);
    return {nullptr, 0};
  }
  if (l.prologue == PRO_ATTN) {
    if constexpr (M == 1) {
      if (l.epilogue != EPI_RESIDUAL) return {nullptr, 0};
      switch (l.rows_per_wave) {
        case 1: return gemv_rx_attn<1>(l.kb);
        case 2: return gemv_rx_attn<2>(l.kb);
        case 4: return gemv_rx_attn<4>(l.kb);
        default: return {nullptr, 0};
      }
    }
    return {nullptr, 0};
  }
  if constexpr (M == 1) {
    if (l.ks > 0) return gemv_ks(l);
    if (l.stream) return gemv_stream(l);
  } else {
    if (l.ks > 0) return gemv_ksm<M>(l);
  }
#define SDEC_KIND(P, E) \
  if (l.prologue == P && l.epilogue == E) return gemv_pick_r<M, P, E>(l, k);
  SDEC_KIND(PRO_NONE, EPI_STORE)
  SDEC_KIND(PRO_NONE, EPI_RESIDUAL)
  SDEC_KIND(PRO_RMS, EPI_STORE)
  SDEC_KIND(PRO_LN, EPI_STORE)
  SDEC_KIND(PRO_RMS, EPI_SWIGLU)
  SDEC_KIND(PRO_RMS, EPI_GELU)
  SDEC_KIND(PRO_LN, EPI_SWIGLU)
  SDEC_KIND(PRO_LN, EPI_GELU)
#undef SDEC_KIND
  return {nullptr, 0};
}

// Timing of the next step-kernel launch of this thread (per-kernel profiles): with a pair set,
// the launch goes through hipExtLaunchKernel, which stamps both events around the kernel's own
// execution, so the interval excludes the launch gap.
thread_local hipEvent_t t_ev_start = nullptr, t_ev_stop = nullptr;

hipError_t launch_timed(const void* fn, dim3 grid, dim3 block, void** params, size_t lds,
                        hipStream_t s) {
  if (t_ev_start != nullptr)
    return hipExtLaunchKernel(fn, grid, block, params, lds, s, t_ev_start, t_ev_stop, 0);
  return hipLaunchKernel(fn, grid, block, params, lds, s);
}

template <int HD>
hipError_t launch_attention_hd(const AttnArgs& a, hipStream_t s) {
  const dim3 grid(a.n_chunks, a.n_kv_heads, a.m);
  const void* fn = nullptr;
  switch (a.n_q_heads / a.n_kv_heads) {
    case 1: fn = a.split ? reinterpret_cast<const void*>(&k_attention_split<HD, 1>)
                         : reinterpret_cast<const void*>(&k_attention<HD, 1>); break;
    case 2: fn = a.split ? reinterpret_cast<const void*>(&k_attention_split<HD, 2>)
                         : reinterpret_cast<const void*>(&k_attention<HD, 2>); break;
    case 4: fn = a.split ? reinterpret_cast<const void*>(&k_attention_split<HD, 4>)
                         : reinterpret_cast<const void*>(&k_attention<HD, 4>); break;
    default: return hipErrorInvalidValue;
  }
  if (a.split && (a.n_chunks == 0 || (a.ring + a.n_chunks - 1) / a.n_chunks > kAttnSplitList))
    return hipErrorInvalidValue;
  AttnArgs args = a;
  void* params[] = {&args};
  return launch_timed(fn, grid, dim3(kWgThreads), params, 0, s);
}

}  // namespace

// Rows m are processed as M = next power of two (unused rows read zeros, write nothing).
static int round_m(uint32_t m) { return m <= 1 ? 1 : m <= 2 ? 2 : m <= 4 ? 4 : m <= 8 ? 8 : 16; }

static int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return v && *v ? atoi(v) : dflt;
}

static GemvKernel gemv_pick(const GemvLaunch& l, uint32_t k, uint32_t m) {
  switch (round_m(m)) {
    case 1: return gemv_pick_m<1>(l, k);
    case 2: return gemv_pick_m<2>(l, k);
    case 4: return gemv_pick_m<4>(l, k);
    case 8: return gemv_pick_m<8>(l, k);
    default: return gemv_pick_m<16>(l, k);
  }
}

GemvLaunch plan_gemv(int prologue, int epilogue, uint32_t n_rows, uint32_t k, uint32_t m) {
  GemvLaunch l{};
  l.prologue = prologue;
  l.epilogue = epilogue;
  const int M = round_m(m);
  const uint32_t kb = k % 256 == 0 ? k / 256 : 0;
  l.kb = 0;
  l.ks = 0;
  l.stream = 0;
  if (M <= 2 && (kb == 2 || kb == 8)) l.kb = static_cast<int>(kb);
  if (M == 1 && (kb == 4 || (kb == 16 && epilogue != EPI_SWIGLU)) && env_int("SDEC_GEMV_RX_1K", 1) != 0)
    l.kb = static_cast<int>(kb);
  if (M == 1 && kb == 24 && epilogue != EPI_SWIGLU) l.kb = 24;
  int dev = 0, cus = 256, occ = 1;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (M == 1 && k == 6144 && prologue == PRO_NONE && epilogue == EPI_RESIDUAL &&
      env_int("SDEC_GEMV_SPLITK", 1) != 0) {
    // four quarter-row waves per workgroup, four rows per workgroup, every row in flight at once
    l.ks = 6;
    l.kb = 0;
    l.rows_per_wave = 4;
    l.waves_per_wg = kWgThreads / kWave;
    int occ_ks = 1;
    const GemvKernel kern = gemv_pick(l, k, m);
    if (kern.fn == nullptr ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ_ks, kern.fn, kWgThreads, 0) != hipSuccess ||
        occ_ks < 1)
      occ_ks = 1;
    const uint32_t need = (n_rows + 3) / 4;
    const uint32_t max_wgs = static_cast<uint32_t>(cus * occ_ks);
    l.grid = need < max_wgs ? need : max_wgs;
    if (l.grid < 1) l.grid = 1;
    return l;
  }
  // one float4 per lane and row in each slice: k = 512 and 1024 at any row count, and k = 2048 at
  // sixteen rows (eight waves), where two float4 per row would not fit the registers
  const bool narrow_k = ((k == 512 || k == 1024) && env_int("SDEC_KSM_NARROW", 1) != 0) ||
                        (M == 16 && k == 2048);
  if (M >= 2 && (((k == 2048 || k == 6144) && M < 16) || narrow_k) && prologue != PRO_ATTN &&
      env_int("SDEC_GEMV_SPLITK", 1) != 0) {
    // the NW waves of a workgroup take the NW slices of k; all M input rows of a slice in registers
    l.ks = narrow_k ? 1 : k == 2048 ? 2 : 3;
    l.kb = 0;
    l.waves_per_wg = narrow_k ? static_cast<int>(k / 256) : k == 2048 ? 4 : 8;
    l.rows_per_wave = narrow_k ? 4 : k == 2048 ? 4 : 2;
    // narrow rows: 4-row tiles while they give every CU a workgroup, else 2-row tiles
    if (narrow_k && n_rows / 4 < static_cast<uint32_t>(cus)) l.rows_per_wave = 2;
    if (M == 8) {
      // taller tiles where measured faster at 8 streams: the q/k/v projection (8 rows per tile,
      // 10.7 vs 12.8 us) and the down projection (4 rows, 12.6 vs 13.1 us); the o and gate/up
      // projections keep theirs.  Tuning overrides: SDEC_KSM_RB2048, SDEC_KSM_RB6144.
      const int dflt = k == 2048 ? (epilogue == EPI_STORE ? 8 : 4) : 4;
      const int rb = env_int(k == 2048 ? "SDEC_KSM_RB2048" : "SDEC_KSM_RB6144", dflt);
      if ((k == 2048 && (rb == 4 || rb == 8)) || (k == 6144 && (rb == 2 || rb == 4)))
        l.rows_per_wave = rb;
    }
    const int units_per_wg = epilogue == EPI_SWIGLU ? l.rows_per_wave / 2 : l.rows_per_wave;
    int occ_m = 1;
    const GemvKernel kern = gemv_pick(l, k, m);
    if (kern.fn == nullptr ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ_m, kern.fn, l.waves_per_wg * kWave, 0) !=
            hipSuccess || occ_m < 1)
      occ_m = 1;
    const uint32_t need = (n_rows + units_per_wg - 1) / units_per_wg;
    const uint32_t max_wgs = static_cast<uint32_t>(cus * occ_m);
    l.grid = need < max_wgs ? need : max_wgs;
    if (l.grid < 1) l.grid = 1;
    if (kern.fn != nullptr) return l;
    l.ks = 0;  // no such kernel: the register GEMV below
  }
  if (M == 1 && l.kb == 8 &&
      (epilogue == EPI_SWIGLU ||
       (epilogue == EPI_STORE && prologue != PRO_NONE && env_int("SDEC_GEMV_STREAM_QKV", 1) != 0)) &&
      env_int("SDEC_GEMV_STREAM", 1) != 0 &&
      n_rows % (4u * static_cast<uint32_t>(cus)) == 0 && n_rows / (4u * static_cast<uint32_t>(cus)) <= 64) {
    // one row per wave in flight, one workgroup per CU: the gate rows and then the up rows stream
    // as a dense band (16.8 vs 17.2 us for 2 x 6144 x 2048); the normed q/k/v projection streams
    // its 4096 rows the same way (6.9 vs 7.0 us; tuning override SDEC_GEMV_STREAM_QKV=0)
    l.stream = 1;
    l.rows_per_wave = 1;
    l.waves_per_wg = kWgThreads / kWave;
    l.grid = static_cast<uint32_t>(cus);
    return l;
  }
  if (l.kb > 0) {
    // rows in flight per wave: enough 16-byte loads per lane to cover the HBM latency
    if (epilogue == EPI_SWIGLU) {
      l.rows_per_wave = 2;
    } else if (l.kb == 2) {
      l.rows_per_wave = M == 1 ? 4 : 2;
    } else if ((l.kb == 8 || l.kb == 4) && M == 1) {
      // the widest tile that still gives every SIMD of the device a tile of its own
      const uint32_t waves = 4u * static_cast<uint32_t>(cus);
      l.rows_per_wave = n_rows / 4 >= waves ? 4 : n_rows / 2 >= waves ? 2 : 1;
    } else {
      l.rows_per_wave = 1;
    }
  } else {
    l.rows_per_wave = M == 1 ? (epilogue == EPI_SWIGLU ? 2 : 1) : (M == 2 ? 2 : 4);
  }
  l.waves_per_wg = kWgThreads / kWave;
  const int rh = epilogue == EPI_SWIGLU ? l.rows_per_wave / 2 : l.rows_per_wave;
  const uint32_t tiles = (n_rows + rh - 1) / rh;
  // Resident waves only: every wave owns a contiguous range of tiles, so a grid larger than what
  // the device holds at once would leave a second, serial round of workgroups.
  const GemvKernel kern = gemv_pick(l, k, m);
  if (kern.fn == nullptr ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern.fn, kWgThreads, kern.lds) !=
          hipSuccess || occ < 1)
    occ = 1;
  // workgroups per CU: at most 4, and 1 for the 6144-wide rows (see k_gemv_rx)
  const int cap = l.kb == 24 ? 1 : env_int("SDEC_GEMV_WGS_PER_CU", 4);
  if (occ > cap) occ = cap;
  const uint32_t max_wgs = static_cast<uint32_t>(cus * occ);
  uint32_t wgs = (tiles + l.waves_per_wg - 1) / l.waves_per_wg;
  if (wgs > max_wgs) wgs = max_wgs;
  l.grid = wgs < 1 ? 1 : wgs;
  return l;
}

GemvLaunch plan_attn_short_o(uint32_t n_rows, uint32_t k, uint32_t head_dim, uint32_t n_q_heads,
                             uint32_t n_kv_heads) {
  GemvLaunch l{};
  l.prologue = PRO_ATTN_SHORT;
  l.epilogue = EPI_RESIDUAL;
  l.kb = k % 256 == 0 ? static_cast<int>(k / 256) : 0;
  l.rows_per_wave = short_o_rows(l.kb);
  // one attention wave per kv head (up to eight)
  const uint32_t naw = n_kv_heads <= 8 ? n_kv_heads : 0;
  l.waves_per_wg = static_cast<int>(kWgThreads / kWave + naw);
  l.attn_hd = static_cast<int>(head_dim);
  l.attn_g = n_kv_heads ? static_cast<int>(n_q_heads / n_kv_heads) : 0;
  l.attn_hpw = naw ? static_cast<int>(n_kv_heads / naw) : 0;
  if (naw == 0 || n_kv_heads % naw != 0 || n_q_heads != static_cast<uint32_t>(l.attn_g) * n_kv_heads ||
      k != n_q_heads * head_dim) {
    l.kb = 0;  // no such kernel
  }
  const uint32_t tiles = (n_rows + l.rows_per_wave - 1) / l.rows_per_wave;
  const uint32_t gemv_waves = kWgThreads / kWave;
  l.grid = (tiles + gemv_waves - 1) / gemv_waves;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (l.grid > static_cast<uint32_t>(cus)) l.grid = static_cast<uint32_t>(cus);
  if (l.grid < 1) l.grid = 1;
  return l;
}

bool gemv_supported(const GemvLaunch& l, uint32_t k, uint32_t m) {
  return gemv_pick(l, k, m).fn != nullptr;
}

hipError_t launch_gemv(const GemvArgs& a, const GemvLaunch& l, hipStream_t s) {
  const GemvKernel kern = gemv_pick(l, a.k, a.m);
  if (kern.fn == nullptr) return hipErrorInvalidValue;
  GemvArgs args = a;
  void* params[] = {&args};
  return launch_timed(kern.fn, dim3(l.grid), dim3(l.waves_per_wg * kWave), params, kern.lds, s);
}

uint32_t attention_chunk(uint32_t head_dim) {
  (void)head_dim;
  // legal slots per workgroup; a tuning override may pick 64 or 256 (at most the workgroup size)
  const int c = env_int("SDEC_ATTN_CHUNK", 128);
  return c == 64 || c == 256 ? static_cast<uint32_t>(c) : 128u;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.head_dim == 128) return launch_attention_hd<128>(a, s);
  if (a.head_dim == 64) return launch_attention_hd<64>(a, s);
  return hipErrorInvalidValue;
}

namespace {
const void* qkv_begin_kernel(const GemvLaunch& l) {
  if (l.epilogue != EPI_STORE || (l.prologue != PRO_RMS && l.prologue != PRO_LN) ||
      l.waves_per_wg * kWave != kWgThreads || l.ks > 0)
    return nullptr;
  const bool rms = l.prologue == PRO_RMS;
  if (l.stream) {
    if (l.kb != 8) return nullptr;
    return rms ? reinterpret_cast<const void*>(&k_qkv_begin<8, PRO_RMS>)
               : reinterpret_cast<const void*>(&k_qkv_begin<8, PRO_LN>);
  }
  // the register shapes of the codec (R 4, k 512) and FlowLM (R 2, k 1024) projections
  if (l.rows_per_wave == 4 && l.kb == 2)
    return rms ? reinterpret_cast<const void*>(&k_qkv_begin_rx<4, PRO_RMS, 2>)
               : reinterpret_cast<const void*>(&k_qkv_begin_rx<4, PRO_LN, 2>);
  if (l.rows_per_wave == 2 && l.kb == 4)
    return rms ? reinterpret_cast<const void*>(&k_qkv_begin_rx<2, PRO_RMS, 4>)
               : reinterpret_cast<const void*>(&k_qkv_begin_rx<2, PRO_LN, 4>);
  return nullptr;
}
}  // namespace

bool qkv_begin_supported(const GemvLaunch& l) { return qkv_begin_kernel(l) != nullptr; }

hipError_t launch_qkv_begin(const QkvBeginArgs& a, const GemvLaunch& l, hipStream_t s) {
  const void* fn = qkv_begin_kernel(l);
  if (fn == nullptr || a.gemv_wgs != l.grid || a.g.m != 1 || a.b.m != 1)
    return hipErrorInvalidValue;
  QkvBeginArgs args = a;
  void* params[] = {&args};
  return launch_timed(fn, dim3(l.grid + a.b.m + 1), dim3(kWgThreads), params, 0, s);
}

hipError_t launch_begin(const BeginArgs& a, hipStream_t s) {
  BeginArgs args = a;
  void* params[] = {&args};
  return launch_timed(reinterpret_cast<const void*>(&k_begin), dim3(a.m + 1), dim3(kWgThreads), params, 0, s);
}

hipError_t launch_begin_rows(const BeginArgs& a, hipStream_t s) {
  BeginArgs args = a;
  void* params[] = {&args};
  if ((a.ring + kWave - 1) / kWave <= kBeginMaxChunks)
    return launch_timed(reinterpret_cast<const void*>(&k_begin_rows_wg), dim3(a.m + 1),
                        dim3(kWgThreads), params, 0, s);
  return launch_timed(reinterpret_cast<const void*>(&k_begin_rows), dim3(1), dim3(kWgThreads), params, 0, s);
}

hipError_t launch_push(const PushArgs& a, hipStream_t s) {
  const void* fn = a.head_dim == 128 ? reinterpret_cast<const void*>(&k_push<128>)
                   : a.head_dim == 64 ? reinterpret_cast<const void*>(&k_push<64>)
                                      : nullptr;
  if (fn == nullptr || a.m == 0 || a.n_kv_heads == 0) return hipErrorInvalidValue;
  PushArgs args = a;
  void* params[] = {&args};
  return launch_timed(fn, dim3(a.m, a.n_kv_heads), dim3(kWave), params, 0, s);
}

hipError_t launch_compact_legal(const uint32_t* pos_rings, uint32_t m, uint32_t ring, uint32_t pos,
                                uint32_t window, uint32_t* legal, uint32_t* n_legal, hipStream_t s) {
  hipLaunchKernelGGL(k_compact_legal, dim3(m), dim3(kWgThreads), 0, s, pos_rings, ring, pos, window,
                     legal, n_legal);
  return hipGetLastError();
}

hipError_t launch_end(const EndArgs& a, hipStream_t s) {
  EndArgs args = a;
  void* params[] = {&args};
  return launch_timed(reinterpret_cast<const void*>(&k_end), dim3(a.m), dim3(kWgThreads), params, 0, s);
}

void set_launch_events(hipEvent_t start, hipEvent_t stop) {
  t_ev_start = start;
  t_ev_stop = stop;
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t value, uint64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  uint64_t g = (n + kWgThreads - 1) / kWgThreads;
  hipLaunchKernelGGL(k_fill_u32, dim3(g > 4096 ? 4096 : static_cast<uint32_t>(g)),
                     dim3(kWgThreads), 0, s, p, value, n);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, float value, uint64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  uint64_t g = (n + kWgThreads - 1) / kWgThreads;
  hipLaunchKernelGGL(k_fill_f32, dim3(g > 4096 ? 4096 : static_cast<uint32_t>(g)),
                     dim3(kWgThreads), 0, s, p, value, n);
  return hipGetLastError();
}

}  // namespace sdec
