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

#include "kernels.h"

namespace sdec {

namespace {

constexpr int kWave = 64;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ float4 f4zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }

__device__ __forceinline__ float dot4(float4 w, float4 x, float acc) {
  acc = fmaf(w.x, x.x, acc);
  acc = fmaf(w.y, x.y, acc);
  acc = fmaf(w.z, x.z, acc);
  return fmaf(w.w, x.w, acc);
}

// Butterfly reduce-scatter of V per-lane partial sums across the wave.  Each halving step swaps
// half of the values with the lane `off` away, so after log2(V) steps lane l holds the wave total
// of value index l / (64 / V); the remaining offsets finish the sum inside each lane group.
template <int V, int OFF>
struct ReduceScatter {
  static __device__ __forceinline__ void run(float* v, int lane) {
    constexpr int H = V / 2;
    const bool upper = (lane & OFF) != 0;
#pragma unroll
    for (int i = 0; i < H; ++i) {
      const float send = upper ? v[i] : v[i + H];
      const float keep = upper ? v[i + H] : v[i];
      v[i] = keep + __shfl_xor(send, OFF, kWave);
    }
    ReduceScatter<H, OFF / 2>::run(v, lane);
  }
};
template <int OFF>
struct ReduceScatter<1, OFF> {
  static __device__ __forceinline__ void run(float* v, int) {
#pragma unroll
    for (int off = OFF; off > 0; off >>= 1) v[0] += __shfl_xor(v[0], off, kWave);
  }
};

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }
__device__ __forceinline__ float gelu_erf(float v) {
  return 0.5f * v * (1.0f + erff(v * 0.70710678118654752440f));
}

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
      inv = 1.0f / sqrtf(wave_sum(ss) / kf + a.eps);
    } else {
      float s = 0.f;
      for (uint32_t c = lane; c < K4; c += kWave) {
        const float4 t = row[c];
        s += (t.x + t.y) + (t.z + t.w);
      }
      mean = wave_sum(s) / kf;
      float ss = 0.f;
      for (uint32_t c = lane; c < K4; c += kWave) {
        float4 t = row[c];
        t.x -= mean; t.y -= mean; t.z -= mean; t.w -= mean;
        ss = dot4(t, t, ss);
      }
      inv = 1.0f / sqrtf(wave_sum(ss) / kf + a.eps);
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
// ([talker] MATVEC_SRC; [mimi] MATVEC, MV_LS).  One wave owns R rows (a "tile") for all M input
// rows; lane l reads float4 column l, l+64, ... of each row, so a wave's loads cover 1 KiB of a
// row per instruction.  U float4 per row are issued before any use to keep bytes in flight.
// ------------------------------------------------------------------------------------------------
template <int M, int R, int PRO, int EPI>
__global__ __launch_bounds__(kWgThreads) void k_gemv(GemvArgs a) {
  extern __shared__ float4 xs[];
  constexpr int U = M <= 2 ? 8 : (M <= 4 ? 4 : 2);
  constexpr int V = R * M;
  static_assert(V <= 64, "tile too large for one wave");
  constexpr int S = kWave / V;  // lanes per reduced value
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  const uint32_t K4 = a.k >> 2;
  if (PRO != PRO_NONE) stage_x<M, PRO>(a, xs, K4);

  constexpr int RH = EPI == EPI_SWIGLU ? R / 2 : R;  // output indices per tile
  const uint32_t n_tiles = (a.n_rows + RH - 1) / RH;
  const float4* x4 = reinterpret_cast<const float4*>(a.x);
  const uint32_t xstride4 = a.x_stride >> 2;

  for (uint32_t t = blockIdx.x * nw + wave; t < n_tiles; t += gridDim.x * nw) {
    const float4* wr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      uint32_t row;
      const float* base;
      if (EPI == EPI_SWIGLU) {
        row = min(t * RH + (r % RH), a.n_rows - 1);
        base = r < RH ? a.w[0] : a.w[1];
      } else {
        row = min(t * RH + r, a.n_rows - 1);
        if (row < a.seg_end[0]) {
          base = a.w[0];
        } else if (row < a.seg_end[1]) {
          base = a.w[1];
          row -= a.seg_end[0];
        } else {
          base = a.w[2];
          row -= a.seg_end[1];
        }
      }
      wr[r] = reinterpret_cast<const float4*>(base + static_cast<size_t>(row) * a.k);
    }

    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;

    for (uint32_t c0 = lane; c0 < K4; c0 += kWave * U) {
      float4 wv[U][R];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t c = c0 + u * kWave;
#pragma unroll
        for (int r = 0; r < R; ++r) wv[u][r] = c < K4 ? wr[r][c] : f4zero();
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t c = c0 + u * kWave;
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

    ReduceScatter<V, 32>::run(acc, lane);
    const float val = acc[0];
    const int idx = lane / S;
    const bool owner = (lane % S) == 0;
    const int r = idx / M, m = idx % M;
    if (EPI == EPI_SWIGLU) {
      const float up = __shfl_xor(val, 32, kWave);  // row r + R/2 lives 32 lanes away
      const uint32_t i = t * RH + r;
      if (owner && lane < 32 && i < a.n_rows && m < static_cast<int>(a.m))
        a.y[m * a.y_stride + i] = silu(val) * up;
    } else {
      const uint32_t row = t * RH + r;
      if (owner && row < a.n_rows && m < static_cast<int>(a.m)) {
        if (EPI == EPI_STORE) {
          a.y[m * a.y_stride + row] = val;
        } else if (EPI == EPI_GELU) {
          a.y[m * a.y_stride + row] = gelu_erf(val);
        } else {
          if (a.tap) a.tap[m * a.tap_stride + row] = val;
          float* dst = a.res + m * a.res_stride + row;
          *dst = *dst + (a.ls ? a.ls[row] * val : val);
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------------------
// Per-head qk-RMSNorm + rope + KV ring push ([talker] QK_NORM_SRC, ROPE_SRC, APPEND_SRC;
// [mimi] rope_push_src).  One wave per (head, stream); lane j owns rope pair j, which is
// (j, j+hd/2) for rotate_half and (2j, 2j+1) for the interleaved form, so both forms are the same
// rotation (a, b) -> (a c - b s, a s + b c).  Query heads land in q_out; key heads are written,
// already roped, into ring slot pos mod R, and the value head is copied beside them.
// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kWave) void k_qk_rope_push(QkRopeArgs a) {
  const uint32_t h = blockIdx.x, s = blockIdx.y, j = threadIdx.x;
  const uint32_t hd = a.head_dim, half = hd >> 1;
  const bool act = j < half;
  const bool is_q = h < a.n_q_heads;
  const float* src = a.qkv + static_cast<size_t>(s) * a.qkv_stride + h * hd;
  const uint32_t ia = a.rope_style == 0 ? j : 2 * j;
  const uint32_t ib = a.rope_style == 0 ? j + half : 2 * j + 1;
  float va = act ? src[ia] : 0.f;
  float vb = act ? src[ib] : 0.f;
  const float* g = is_q ? a.q_norm : a.k_norm;
  if (g != nullptr) {
    const float ss = wave_sum(va * va + vb * vb);
    const float inv = 1.0f / sqrtf(ss / static_cast<float>(hd) + a.eps);
    if (act) {
      va = (va * inv) * g[ia];
      vb = (vb * inv) * g[ib];
    }
  }
  if (!act) return;
  const float c = a.cs[j], sn = a.cs[half + j];
  const float ra = va * c - vb * sn;
  const float rb = va * sn + vb * c;
  if (is_q) {
    float* d = a.q_out + static_cast<size_t>(s) * a.n_q_heads * hd + h * hd;
    d[ia] = ra;
    d[ib] = rb;
  } else {
    const uint32_t kvh = h - a.n_q_heads;
    const size_t off = static_cast<size_t>(s) * a.ring_stream_stride +
                       (static_cast<size_t>(a.st->slot) * a.n_kv_heads + kvh) * hd;
    a.k_ring[off + ia] = ra;
    a.k_ring[off + ib] = rb;
    const float* vsrc = a.qkv + static_cast<size_t>(s) * a.qkv_stride +
                        (a.n_q_heads + a.n_kv_heads + kvh) * hd;
    a.v_ring[off + ia] = vsrc[ia];
    a.v_ring[off + ib] = vsrc[ib];
  }
}

// ------------------------------------------------------------------------------------------------
// Ring attention, split over slot chunks ([mimi] attn_src: legality from the position ring, a
// masked slot weighs nothing; [talker] GQA_ATTN_SRC: kv head = q head / group, scale 1/sqrt(hd)).
// Grid (chunk, kv head, stream).  The chunk's legal slots are compacted first, so masked slots
// cost no K/V traffic.  Slot groups of hd/8 lanes (8 dims per lane) walk the legal slots with an
// online softmax for all G query heads of the kv head, so each K/V row is read once for the whole
// GQA group.  Groups merge in LDS; chunks merge in the last workgroup to finish (integer counter),
// in ascending chunk order, so the result does not depend on which workgroup finishes last.
// ------------------------------------------------------------------------------------------------
template <int HD, int G>
__global__ __launch_bounds__(kWgThreads) void k_attention(AttnArgs a) {
  constexpr int LPS = HD / 8;
  constexpr int GPW = kWave / LPS;
  constexpr int NWV = kWgThreads / kWave;
  constexpr int NG = NWV * GPW;
  constexpr int UNR = 4;
  __shared__ uint32_t list[kWgThreads];
  __shared__ uint32_t wave_cnt[NWV];
  __shared__ float sm_m[NG][G], sm_l[NG][G];
  __shared__ float sm_acc[NG][G][HD];
  __shared__ uint32_t is_last;

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int grp = wave * GPW + lane / LPS;
  const int sub = lane % LPS;
  const uint32_t chunk = blockIdx.x, kvh = blockIdx.y, s = blockIdx.z;
  const uint32_t pos = a.st ? a.st->pos : a.pos;
  const uint32_t c0 = chunk * a.chunk;
  const uint32_t c1 = min(c0 + a.chunk, a.ring);

  // 1. legal slots of the chunk, in slot order
  const uint32_t slot = c0 + tid;
  bool ok = false;
  if (slot < c1) {
    const uint32_t p = a.pos_ring[static_cast<size_t>(s) * a.pos_stream_stride + slot];
    ok = p != kInvalidPos && p <= pos && pos - p < a.window;
  }
  const unsigned long long mask = __ballot(ok);
  const uint32_t before = __popcll(mask & ((1ull << lane) - 1ull));
  if (lane == 0) wave_cnt[wave] = __popcll(mask);
  __syncthreads();
  uint32_t off = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    off += w < wave ? wave_cnt[w] : 0u;
    total += wave_cnt[w];
  }
  if (ok) list[off + before] = slot;
  __syncthreads();

  // 2. online softmax over this group's share of the legal slots
  const uint32_t hq = a.n_q_heads, hkv = a.n_kv_heads;
  const uint32_t h0 = kvh * G;
  float q[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float4* qp = reinterpret_cast<const float4*>(
        a.q + static_cast<size_t>(s) * hq * HD + (h0 + g) * HD + 8 * sub);
    const float4 q0 = qp[0], q1 = qp[1];
    q[g][0] = q0.x; q[g][1] = q0.y; q[g][2] = q0.z; q[g][3] = q0.w;
    q[g][4] = q1.x; q[g][5] = q1.y; q[g][6] = q1.z; q[g][7] = q1.w;
  }
  const float scale = 1.0f / sqrtf(static_cast<float>(HD));
  float mrun[G], lrun[G], acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    mrun[g] = -INFINITY;
    lrun[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
  }
  const size_t row = static_cast<size_t>(hkv) * HD;
  const float* kb = a.k_ring + static_cast<size_t>(s) * a.ring_stream_stride + kvh * HD + 8 * sub;
  const float* vb = a.v_ring + static_cast<size_t>(s) * a.ring_stream_stride + kvh * HD + 8 * sub;
  for (uint32_t i0 = grp; i0 < total; i0 += NG * UNR) {
    float4 kk[UNR][2], vv[UNR][2];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const uint32_t i = i0 + u * NG;
      if (i < total) {
        const size_t sl = list[i];
        const float4* kp = reinterpret_cast<const float4*>(kb + sl * row);
        const float4* vp = reinterpret_cast<const float4*>(vb + sl * row);
        kk[u][0] = kp[0]; kk[u][1] = kp[1];
        vv[u][0] = vp[0]; vv[u][1] = vp[1];
      } else {
        kk[u][0] = kk[u][1] = vv[u][0] = vv[u][1] = f4zero();
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      if (i0 + u * NG < total) {
        const float kf[8] = {kk[u][0].x, kk[u][0].y, kk[u][0].z, kk[u][0].w,
                             kk[u][1].x, kk[u][1].y, kk[u][1].z, kk[u][1].w};
        const float vf[8] = {vv[u][0].x, vv[u][0].y, vv[u][0].z, vv[u][0].w,
                             vv[u][1].x, vv[u][1].y, vv[u][1].z, vv[u][1].w};
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) d = fmaf(q[g][e], kf[e], d);
#pragma unroll
          for (int o = LPS / 2; o > 0; o >>= 1) d += __shfl_xor(d, o, kWave);
          const float sc = d * scale;
          const float mnew = fmaxf(mrun[g], sc);
          const float corr = expf(mrun[g] - mnew);
          const float p = expf(sc - mnew);
          lrun[g] = lrun[g] * corr + p;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[g][e] = acc[g][e] * corr + p * vf[e];
          mrun[g] = mnew;
        }
      }
    }
  }

  // 3. merge the slot groups of this workgroup
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (sub == 0) {
      sm_m[grp][g] = mrun[g];
      sm_l[grp][g] = lrun[g];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) sm_acc[grp][g][8 * sub + e] = acc[g][e];
  }
  __syncthreads();
  const bool single = a.n_chunks == 1;
  for (int t = tid; t < G * HD; t += kWgThreads) {
    const int g = t / HD, d = t % HD;
    float M = -INFINITY;
    for (int k = 0; k < NG; ++k) M = fmaxf(M, sm_m[k][g]);
    float L = 0.f, O = 0.f;
    for (int k = 0; k < NG; ++k) {
      const float mk = sm_m[k][g];
      if (mk != -INFINITY) {
        const float w = expf(mk - M);
        L = fmaf(w, sm_l[k][g], L);
        O = fmaf(w, sm_acc[k][g][d], O);
      }
    }
    if (single) {
      a.out[static_cast<size_t>(s) * hq * HD + (h0 + g) * HD + d] = L > 0.f ? O / L : 0.f;
    } else {
      float* pp = a.part + ((static_cast<size_t>(s) * hq + h0 + g) * a.n_chunks + chunk) * (HD + 2);
      pp[d] = O;
      if (d == 0) {
        pp[HD] = M;
        pp[HD + 1] = L;
      }
    }
  }
  if (single) return;

  // 4. the last chunk of this (stream, kv head) to finish merges all chunks
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = atomicAdd(&a.counters[s * hkv + kvh], 1u);
    is_last = prev == a.n_chunks - 1 ? 1u : 0u;
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  for (int t = tid; t < G * HD; t += kWgThreads) {
    const int g = t / HD, d = t % HD;
    const float* base = a.part + (static_cast<size_t>(s) * hq + h0 + g) * a.n_chunks * (HD + 2);
    float M = -INFINITY;
    for (uint32_t c = 0; c < a.n_chunks; ++c) M = fmaxf(M, base[c * (HD + 2) + HD]);
    float L = 0.f, O = 0.f;
    for (uint32_t c = 0; c < a.n_chunks; ++c) {
      const float mc = base[c * (HD + 2) + HD];
      if (mc != -INFINITY) {
        const float w = expf(mc - M);
        L = fmaf(w, base[c * (HD + 2) + HD + 1], L);
        O = fmaf(w, base[c * (HD + 2) + d], O);
      }
    }
    a.out[static_cast<size_t>(s) * hq * HD + (h0 + g) * HD + d] = L > 0.f ? O / L : 0.f;
  }
  if (tid == 0) a.counters[s * hkv + kvh] = 0u;
}

// ------------------------------------------------------------------------------------------------
// Step begin: copy the caller's rows into the residual stream, start fresh streams (every
// position-ring slot empty), stamp pos into slot pos mod R of each stream's position ring
// ([mimi] rope_push_src: pr[slot] = pos), and form this position's rope cos/sin in float64
// ([talker] TalkerGpu::load builds its tables on the CPU; rounding once to float32).
// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kWgThreads) void k_begin(BeginArgs a) {
  const uint32_t tid = blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t nth = gridDim.x * blockDim.x;
  const uint32_t slot = a.pos % a.ring;
  const float4* src = reinterpret_cast<const float4*>(a.x_in);
  float4* dst = reinterpret_cast<float4*>(a.xres);
  for (uint32_t i = tid; i < (a.md >> 2); i += nth) dst[i] = src[i];
  if (a.first) {
    for (uint32_t i = tid; i < a.m * a.ring; i += nth)
      a.pos_rings[i] = (i % a.ring) == slot ? a.pos : kInvalidPos;
  } else {
    for (uint32_t i = tid; i < a.m; i += nth) a.pos_rings[i * a.ring + slot] = a.pos;
  }
  const uint32_t half = a.head_dim >> 1;
  if (tid < half) {
    const double inv_freq = pow(a.theta, -2.0 * static_cast<double>(tid) /
                                             static_cast<double>(a.head_dim));
    const double ang = static_cast<double>(a.pos) * inv_freq;
    a.cs[tid] = static_cast<float>(cos(ang));
    a.cs[half + tid] = static_cast<float>(sin(ang));
  }
  if (tid == 0) {
    a.st->pos = a.pos;
    a.st->slot = slot;
  }
}

// Step end: the output rows -- the final norm of the residual stream ([talker] build_step_plan's
// closing RMSNorm) or the residual stream itself ([mimi] transformer_shaped works in place).
__global__ __launch_bounds__(kWgThreads) void k_end(EndArgs a) {
  __shared__ float red[kWgThreads / kWave];
  __shared__ float2 st;
  const uint32_t r = blockIdx.x;
  const float* x = a.xres + static_cast<size_t>(r) * a.d;
  float* y = a.x_out + static_cast<size_t>(r) * a.d;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  if (a.norm < 0) {
    for (uint32_t i = tid; i < a.d; i += blockDim.x) y[i] = x[i];
    return;
  }
  const float df = static_cast<float>(a.d);
  float mean = 0.f;
  if (a.norm == PRO_LN) {
    float s = 0.f;
    for (uint32_t i = tid; i < a.d; i += blockDim.x) s += x[i];
    s = wave_sum(s);
    if (lane == 0) red[wave] = s;
    __syncthreads();
    if (tid == 0) {
      float t = 0.f;
      for (int w = 0; w < kWgThreads / kWave; ++w) t += red[w];
      st.x = t / df;
    }
    __syncthreads();
    mean = st.x;
  }
  float ss = 0.f;
  for (uint32_t i = tid; i < a.d; i += blockDim.x) {
    const float v = x[i] - mean;
    ss = fmaf(v, v, ss);
  }
  ss = wave_sum(ss);
  __syncthreads();
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  if (tid == 0) {
    float t = 0.f;
    for (int w = 0; w < kWgThreads / kWave; ++w) t += red[w];
    st.y = 1.0f / sqrtf(t / df + a.eps);
  }
  __syncthreads();
  const float inv = st.y;
  for (uint32_t i = tid; i < a.d; i += blockDim.x) {
    if (a.norm == PRO_LN) y[i] = ((x[i] - mean) * inv) * a.w[i] + a.b[i];
    else y[i] = (x[i] * inv) * a.w[i];
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

template <int M, int R, int PRO, int EPI>
hipError_t launch_gemv_t(const GemvArgs& a, const GemvLaunch& l, hipStream_t s) {
  const size_t lds = PRO == PRO_NONE ? 0 : static_cast<size_t>(M) * a.k * sizeof(float);
  hipLaunchKernelGGL((k_gemv<M, R, PRO, EPI>), dim3(l.grid), dim3(l.waves_per_wg * kWave), lds,
                     s, a);
  return hipGetLastError();
}

template <int M, int PRO, int EPI>
hipError_t launch_gemv_r(const GemvArgs& a, const GemvLaunch& l, hipStream_t s) {
  switch (l.rows_per_wave) {
    case 1:
      if constexpr (EPI != EPI_SWIGLU) return launch_gemv_t<M, 1, PRO, EPI>(a, l, s);
      break;
    case 2: return launch_gemv_t<M, 2, PRO, EPI>(a, l, s);
    case 4: return launch_gemv_t<M, 4, PRO, EPI>(a, l, s);
    default: break;
  }
  return hipErrorInvalidValue;
}

template <int M>
hipError_t launch_gemv_m(const GemvArgs& a, const GemvLaunch& l, hipStream_t s) {
#define SDEC_KIND(P, E) \
  if (l.prologue == P && l.epilogue == E) return launch_gemv_r<M, P, E>(a, l, s);
  SDEC_KIND(PRO_NONE, EPI_STORE)
  SDEC_KIND(PRO_NONE, EPI_RESIDUAL)
  SDEC_KIND(PRO_RMS, EPI_STORE)
  SDEC_KIND(PRO_LN, EPI_STORE)
  SDEC_KIND(PRO_RMS, EPI_SWIGLU)
  SDEC_KIND(PRO_RMS, EPI_GELU)
  SDEC_KIND(PRO_LN, EPI_SWIGLU)
  SDEC_KIND(PRO_LN, EPI_GELU)
#undef SDEC_KIND
  return hipErrorInvalidValue;
}

template <int HD>
hipError_t launch_attention_hd(const AttnArgs& a, hipStream_t s) {
  const dim3 grid(a.n_chunks, a.n_kv_heads, a.m);
  switch (a.n_q_heads / a.n_kv_heads) {
    case 1: hipLaunchKernelGGL((k_attention<HD, 1>), grid, dim3(kWgThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_attention<HD, 2>), grid, dim3(kWgThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_attention<HD, 4>), grid, dim3(kWgThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// Rows m are processed as M = next power of two (unused rows read zeros, write nothing).
static int round_m(uint32_t m) { return m <= 1 ? 1 : m <= 2 ? 2 : m <= 4 ? 4 : 8; }

GemvLaunch plan_gemv(int prologue, int epilogue, uint32_t n_rows, uint32_t k, uint32_t m) {
  (void)k;
  GemvLaunch l;
  l.prologue = prologue;
  l.epilogue = epilogue;
  const int M = round_m(m);
  l.rows_per_wave = M == 1 ? (epilogue == EPI_SWIGLU ? 2 : 1) : (M == 2 ? 2 : 4);
  if (epilogue == EPI_SWIGLU && l.rows_per_wave < 2) l.rows_per_wave = 2;
  l.waves_per_wg = kWgThreads / kWave;
  const int rh = epilogue == EPI_SWIGLU ? l.rows_per_wave / 2 : l.rows_per_wave;
  const uint32_t tiles = (n_rows + rh - 1) / rh;
  const uint32_t wgs = (tiles + l.waves_per_wg - 1) / l.waves_per_wg;
  l.grid = wgs < 1 ? 1 : wgs;
  return l;
}

hipError_t launch_gemv(const GemvArgs& a, const GemvLaunch& l, hipStream_t s) {
  switch (round_m(a.m)) {
    case 1: return launch_gemv_m<1>(a, l, s);
    case 2: return launch_gemv_m<2>(a, l, s);
    case 4: return launch_gemv_m<4>(a, l, s);
    default: return launch_gemv_m<8>(a, l, s);
  }
}

hipError_t launch_qk_rope_push(const QkRopeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_qk_rope_push, dim3(a.n_q_heads + a.n_kv_heads, a.m), dim3(kWave), 0, s,
                     a);
  return hipGetLastError();
}

uint32_t attention_chunk(uint32_t head_dim) { return head_dim == 128 ? 64u : 64u; }

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.head_dim == 128) return launch_attention_hd<128>(a, s);
  if (a.head_dim == 64) return launch_attention_hd<64>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_begin(const BeginArgs& a, hipStream_t s) {
  uint64_t work = a.md / 4;
  if (a.first && static_cast<uint64_t>(a.m) * a.ring > work) work = static_cast<uint64_t>(a.m) * a.ring;
  uint32_t grid = static_cast<uint32_t>((work + kWgThreads - 1) / kWgThreads);
  grid = grid < 1 ? 1 : (grid > 64 ? 64 : grid);
  hipLaunchKernelGGL(k_begin, dim3(grid), dim3(kWgThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_end(const EndArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_end, dim3(a.m), dim3(kWgThreads), 0, s, a);
  return hipGetLastError();
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
