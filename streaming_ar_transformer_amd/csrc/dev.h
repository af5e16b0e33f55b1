// Device helpers of the step kernels (kernels.hip).  Page names in citations: [talker] inferencelayer 0.2.8 src/qwen3tts_gpu.rs,
// [mimi] 0.2.1 src/mimi_gpu.rs.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"

namespace sdec {
namespace dev {

constexpr int kWave = 64;

// Cross-lane moves without LDS traffic.  DPP reaches lanes inside a 16-lane row (swap neighbours,
// swap pairs, mirror halves of 8, mirror the row); gfx950's permlane swaps exchange whole rows
// between two registers: permlane16 swaps the odd rows of the first with the even rows of the
// second, permlane32 the upper half of the first with the lower half of the second.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
// Over the row pairs (0,1) and (2,3): the even row of each pair gets a[even] + a[odd], the odd
// row b[even] + b[odd] (lane by lane).
__device__ __forceinline__ float rows16_sum(float a, float b) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
// Over the two halves of the wave: the lower half gets a[lo] + a[hi], the upper b[lo] + b[hi].
__device__ __forceinline__ float halves_sum(float a, float b) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
// The value of lane l ^ 32.
__device__ __forceinline__ float partner32(float x, int lane) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((lane & 32) ? p[0] : p[1]);
}

// The value of lane l ^ OFF (OFF = 8: a DPP row rotation by 8 inside a 16-lane row).
template <int OFF>
__device__ __forceinline__ float lane_xor(float x, int lane) {
  if constexpr (OFF == 32) return partner32(x, lane);
  else if constexpr (OFF == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((lane & 16) ? p[0] : p[1]);
  } else if constexpr (OFF == 8) {
    return dpp_mov<0x128>(x);  // row_ror:8 -- lane i of a 16-lane row reads lane i ^ 8
  } else {
    return __shfl_xor(x, OFF);
  }
}

// max / sum of a value and the lane l ^ 16 or l ^ 32 one: the swap returns both in some order, so
// no lane select is needed (as there is for lane_xor).
template <int OFF>
__device__ __forceinline__ float pair_max(float x) {
  static_assert(OFF == 16 || OFF == 32, "row or half swaps");
  const auto p = OFF == 16
      ? __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false)
      : __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
template <int OFF>
__device__ __forceinline__ float pair_sum(float x) {
  static_assert(OFF == 16 || OFF == 32, "row or half swaps");
  return OFF == 16 ? rows16_sum(x, x) : halves_sum(x, x);
}

// Sum over the whole wave, left in every lane.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_mov<kDppXor1>(v);
  v += dpp_mov<kDppXor2>(v);
  v += dpp_mov<kDppHalfMirror>(v);
  v += dpp_mov<kDppMirror>(v);
  v = rows16_sum(v, v);
  return halves_sum(v, v);
}

__device__ __forceinline__ float4 f4zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }

// Weights are streamed once per step: load them non-temporally so they do not displace the
// small, reused activations from the caches.
typedef float f4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ldw(const float4* p) {
  const f4v v = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

// Device-coherent (agent-scope) stores and loads: they bypass the per-XCD cache state, so data
// handed between workgroups needs no cache-wide writeback or invalidate -- only completion of the
// stores before the hand-off counter is bumped.
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0); }
// A store that is coherent across the device when COH (a hand-off to other workgroups of the
// same launch), or an ordinary store.
template <bool COH>
__device__ __forceinline__ void put(float* p, float v) {
  if (COH) st_dev(p, v);
  else *p = v;
}

__device__ __forceinline__ float dot4(float4 w, float4 x, float acc) {
  acc = fmaf(w.x, x.x, acc);
  acc = fmaf(w.y, x.y, acc);
  acc = fmaf(w.z, x.z, acc);
  return fmaf(w.w, x.w, acc);
}

// Butterfly reduce-scatter of V per-lane partial sums across the wave.  Each halving step pairs
// every lane with one in the other half of its OFF-block and keeps half of the values, so after
// log2(V) steps lane l holds the wave total of value index l / (64 / V); the remaining steps
// finish the sum inside each lane group.  Steps across 32 and 16 lanes use the permlane swaps,
// the rest DPP moves (partners: the mirror lane within 16, within 8, then the quad swaps).
template <int OFF>
__device__ __forceinline__ float dpp_partner(float x) {
  static_assert(OFF == 8 || OFF == 4 || OFF == 2 || OFF == 1, "inside a 16-lane row");
  if constexpr (OFF == 8) return dpp_mov<kDppMirror>(x);
  else if constexpr (OFF == 4) return dpp_mov<kDppHalfMirror>(x);
  else if constexpr (OFF == 2) return dpp_mov<kDppXor2>(x);
  else return dpp_mov<kDppXor1>(x);
}
template <int V, int OFF>
struct ReduceScatter {
  static __device__ __forceinline__ void run(float* v, int lane) {
    constexpr int H = V / 2;
#pragma unroll
    for (int i = 0; i < H; ++i) {
      if constexpr (OFF == 32) {
        v[i] = halves_sum(v[i], v[i + H]);
      } else if constexpr (OFF == 16) {
        v[i] = rows16_sum(v[i], v[i + H]);
      } else {
        const bool upper = (lane & OFF) != 0;
        const float send = upper ? v[i] : v[i + H];
        const float keep = upper ? v[i + H] : v[i];
        v[i] = keep + dpp_partner<OFF>(send);
      }
    }
    ReduceScatter<H, OFF / 2>::run(v, lane);
  }
};
template <int OFF>
struct ReduceScatter<1, OFF> {  // full sums over aligned blocks of 2 * OFF lanes
  static __device__ __forceinline__ void run(float* v, int) {
    float x = v[0];
    if constexpr (OFF >= 8) x += dpp_partner<8>(x);
    if constexpr (OFF >= 4) x += dpp_partner<4>(x);
    if constexpr (OFF >= 2) x += dpp_partner<2>(x);
    if constexpr (OFF >= 1) x += dpp_partner<1>(x);
    if constexpr (OFF >= 16) x = rows16_sum(x, x);
    if constexpr (OFF >= 32) x = halves_sum(x, x);
    v[0] = x;
  }
};

// Sum over aligned groups of N lanes (N = 8 or 16), left in every lane of the group.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 8 || N == 16, "DPP rows hold 16 lanes");
  v += dpp_mov<kDppXor1>(v);
  v += dpp_mov<kDppXor2>(v);
  v += dpp_mov<kDppHalfMirror>(v);
  if (N == 16) v += dpp_mov<kDppMirror>(v);
  return v;
}

template <int N>
__device__ __forceinline__ float group_max(float v) {
  static_assert(N == 8 || N == 16, "DPP rows hold 16 lanes");
  v = fmaxf(v, dpp_mov<kDppXor1>(v));
  v = fmaxf(v, dpp_mov<kDppXor2>(v));
  v = fmaxf(v, dpp_mov<kDppHalfMirror>(v));
  if (N == 16) v = fmaxf(v, dpp_mov<kDppMirror>(v));
  return v;
}

// g / (1 + e^-g) with the reciprocal instruction (within 1 ulp) in place of a correctly rounded
// division; e^-g overflowing to infinity gives -0 for very negative g, as the division does.
__device__ __forceinline__ float silu(float g) { return g * __builtin_amdgcn_rcpf(1.0f + expf(-g)); }
__device__ __forceinline__ float gelu_erf(float v) {
  return 0.5f * v * (1.0f + erff(v * 0.70710678118654752440f));
}

// ------------------------------------------------------------------------------------------------
// qk-RMSNorm + rope of one head pair ([talker] QK_NORM_SRC then ROPE_SRC; [mimi] rope_push_src).
// Lane j owns rope pair j: (j, j + hd/2) for rotate_half, (2j, 2j + 1) for the interleaved form;
// both are the rotation (a, b) -> (a c - b s, a s + b c).  Called by a whole wave.
// ------------------------------------------------------------------------------------------------
template <int HD>
__device__ __forceinline__ void norm_rope_pair(float& va, float& vb, int j, const float* gnorm,
                                               float eps, const float* cs, int style) {
  constexpr int HALF = HD / 2;
  const bool act = j < HALF;
  if (gnorm != nullptr) {
    const float ss = wave_sum(act ? va * va + vb * vb : 0.f);
    const float inv = rsqrtf(ss * (1.0f / static_cast<float>(HD)) + eps);
    if (act) {
      const int ia = style == 0 ? j : 2 * j, ib = style == 0 ? j + HALF : 2 * j + 1;
      va = (va * inv) * gnorm[ia];
      vb = (vb * inv) * gnorm[ib];
    }
  }
  if (cs != nullptr && act) {
    const float c = cs[j], sn = cs[HALF + j];
    const float ra = va * c - vb * sn;
    const float rb = va * sn + vb * c;
    va = ra;
    vb = rb;
  }
}

template <int R, int EPI>
__device__ __forceinline__ void tile_rows(const GemvArgs& a, uint32_t t, const float4* (&wr)[R]) {
  constexpr int RH = EPI == EPI_SWIGLU ? R / 2 : R;
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
}

// Reduce the tile's R*M lane partials and apply the epilogue: store, GELU, SwiGLU (gate row r and
// up row r + R/2 of the same FFN index sit 32 lanes apart after the reduce-scatter), or the
// (LayerScale) residual add ([mimi] MV_LS: y += ls * (W x)).
// The old residual value (and LayerScale) that this lane's output of tile t needs: requested
// together with the tile's weights, so the residual epilogue does not start a dependent load.
struct ResPre {
  float res = 0.f, ls = 1.f;
};
template <int M, int R, int EPI>
__device__ __forceinline__ ResPre residual_prefetch(const GemvArgs& a, uint32_t t, int lane) {
  ResPre p;
  if constexpr (EPI == EPI_RESIDUAL) {
    constexpr int V = R * M;
    constexpr int S = kWave / V;
    const int idx = lane / S;
    const uint32_t r = idx / M, m = min(static_cast<uint32_t>(idx % M), a.m - 1);
    const uint32_t row = min(t * R + r, a.n_rows - 1);
    p.res = ((a.res_in ? a.res_in : a.res) + m * a.res_stride)[row];
    if (a.ls) p.ls = a.ls[row];
  }
  return p;
}

template <int M, int R, int EPI, bool COH = false>
__device__ __forceinline__ void gemv_epilogue(const GemvArgs& a, uint32_t t, float* acc, int lane,
                                              const ResPre* pre = nullptr) {
  constexpr int V = R * M;
  constexpr int S = kWave / V;
  constexpr int RH = EPI == EPI_SWIGLU ? R / 2 : R;
  ReduceScatter<V, 32>::run(acc, lane);
  const float val = acc[0];
  const int idx = lane / S;
  const bool owner = (lane % S) == 0;
  const int r = idx / M, m = idx % M;
  if (EPI == EPI_SWIGLU) {
    const float up = partner32(val, lane);
    const uint32_t i = t * RH + r;
    if (owner && lane < 32 && i < a.n_rows && m < static_cast<int>(a.m))
      put<COH>(a.y + m * a.y_stride + i, silu(val) * up);
  } else {
    const uint32_t row = t * RH + r;
    if (owner && row < a.n_rows && m < static_cast<int>(a.m)) {
      if (EPI == EPI_STORE) {
        put<COH>(a.y + m * a.y_stride + row, val);
      } else if (EPI == EPI_GELU) {
        put<COH>(a.y + m * a.y_stride + row, gelu_erf(val));
      } else {
        if (a.tap) a.tap[m * a.tap_stride + row] = val;
        float* dst = a.res_st != nullptr ? a.res_st->x_out : a.res;
        if (pre) {
          put<COH>(dst + m * a.res_stride + row, pre->res + (a.ls ? pre->ls * val : val));
        } else {
          const float* src = (a.res_in ? a.res_in : a.res) + m * a.res_stride + row;
          put<COH>(dst + m * a.res_stride + row, *src + (a.ls ? a.ls[row] * val : val));
        }
      }
    }
  }
}

__device__ __forceinline__ void wave_tiles(uint32_t n_tiles, uint32_t& t, uint32_t& t_end) {
  const uint32_t nw = blockDim.x / kWave;
  const uint32_t gw = blockIdx.x * nw + threadIdx.x / kWave;
  const uint64_t nwaves = static_cast<uint64_t>(gridDim.x) * nw;
  t = static_cast<uint32_t>(gw * static_cast<uint64_t>(n_tiles) / nwaves);
  t_end = static_cast<uint32_t>((gw + 1) * static_cast<uint64_t>(n_tiles) / nwaves);
}

// The slots a query at `pos` may attend, from one stream's position ring ([mimi] attn_src: slot
// j is legal iff P[j] != INVALID, P[j] <= pos and pos - P[j] < window), written to `out` in
// ascending slot order -- after `lead` when lead >= 0 (the slot this step pushes, legal by
// construction).  Legality depends only on the ring and pos, so one list serves every layer of
// the step.  Called by a whole workgroup of NT threads; `scan` is NT words of LDS.
template <int NT, bool COH>
__device__ __forceinline__ void compact_legal(const uint32_t* P, uint32_t R, uint32_t pos,
                                              uint32_t window, int lead, uint32_t* out,
                                              uint32_t* n_out, uint32_t* scan) {
  const int tid = threadIdx.x;
  const uint32_t per = (R + NT - 1) / NT;
  const uint32_t b = min(static_cast<uint32_t>(tid) * per, R), e = min(b + per, R);
  auto is_legal = [&](uint32_t j) {
    const uint32_t p = P[j];
    return static_cast<int>(j) != lead && p != kInvalidPos && p <= pos && pos - p < window;
  };
  uint32_t cnt = 0;
  for (uint32_t j = b; j < e; ++j) cnt += is_legal(j) ? 1u : 0u;
  scan[tid] = cnt;
  __syncthreads();
  for (int off = 1; off < NT; off <<= 1) {  // inclusive scan
    const uint32_t v = tid >= off ? scan[tid - off] : 0u;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  const uint32_t base = lead >= 0 ? 1u : 0u;
  uint32_t o = base + scan[tid] - cnt;
  for (uint32_t j = b; j < e; ++j) {
    if (is_legal(j)) {
      if (COH) __hip_atomic_store(out + o, j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else out[o] = j;
      ++o;
    }
  }
  if (tid == 0) {
    const uint32_t n = base + scan[NT - 1];
    if (COH) {
      if (lead >= 0)
        __hip_atomic_store(out, static_cast<uint32_t>(lead), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(n_out, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      if (lead >= 0) out[0] = static_cast<uint32_t>(lead);
      *n_out = n;
    }
  }
}

template <int HD, int G, int NT, int LIST = NT>
struct AttnSmem {
  static constexpr int LPS = HD / 8;
  static constexpr int NG = (NT / kWave) * (kWave / LPS);
  uint32_t list[LIST];
  float qs[G][HD];
  float ks[HD], vs[HD];  // this step's key (normed, roped) and value, for the item that pushes
  float sm_m[NG][G], sm_l[NG][G];
  float sm_acc[NG][G][HD];
  uint32_t is_last;
};

// One (slot chunk, kv head, stream) work item, run by a whole workgroup of NT threads.  COH: the
// output is handed to other workgroups of the same launch.  UNR: slots per lane group whose keys
// and values are in flight together.  CG: partials each thread requests together in the chunk
// combine (0: a whole batch at once).
//
// The memory round trips are kept few: the slot list and this head group's raw q/k/v are fetched
// together; then every key and value row of the item is requested at once, and the query and key
// normalisation and rope run while those loads are in flight.  The slot this step pushes (always
// the first of item 0) is scored from LDS, so no load waits for the push.
//
// SPLIT (streams that each attend a long ring): instead of fixed-size chunks, the legal slots of a
// (stream, kv head) are dealt round-robin to its n_chunks items, up to LIST slots each, so all
// items of a step run in one round however long the context; an item walks its share in passes
// of NG * UNR slots with two passes' keys and values in flight, the next pass requested before
// the current one is scored.
template <int HD, int G, int NT, bool COH, int UNR = 4, int CG = 0, bool SPLIT = false,
          int LIST = NT>
__device__ __forceinline__ void attention_item(const AttnArgs& a, uint32_t chunk, uint32_t kvh,
                                               uint32_t s, AttnSmem<HD, G, NT, LIST>& sm) {
  constexpr int LPS = HD / 8;
  constexpr int GPW = kWave / LPS;
  constexpr int NWV = NT / kWave;
  constexpr int NG = NWV * GPW;
  constexpr int HALF = HD / 2;
  constexpr int CB = 16;  // chunks merged per batch by the last workgroup
  static_assert(CB <= NG, "combine staging reuses the group buffers");
  static_assert(G <= NWV, "one wave per query head of the group");
  uint32_t* list = sm.list;
  auto& qs = sm.qs;
  auto& sm_m = sm.sm_m;
  auto& sm_l = sm.sm_l;
  auto& sm_acc = sm.sm_acc;
  uint32_t& is_last = sm.is_last;
  __syncthreads();  // the previous item of this workgroup is done with the LDS

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int grp = wave * GPW + lane / LPS;
  const int sub = lane % LPS;
  const uint32_t hq = a.n_q_heads, hkv = a.n_kv_heads;
  const uint32_t h0 = kvh * G;
  const float* qkv = a.qkv + static_cast<size_t>(s) * a.qkv_stride;
  const float* cs = a.cs ? a.cs + static_cast<size_t>(s) * a.cs_stride : nullptr;

  // 1. this item's share of the step's legal slots; this step's raw queries (and, for the item
  //    that pushes, the raw key and value).  All of them are requested together with the slot
  //    count, before it is known which are needed: indices are clamped into the buffers and
  //    values that turn out unused are dropped, so the item waits for one round trip, not two.
  static_assert(NT >= 2 * HD, "one thread per raw key or value element");
  constexpr int QPT = (G * HD + NT - 1) / NT;
  const uint32_t nl = a.n_legal[s];
  // this item's slot entries are requested with the count (clamped indices).  Fixed chunks: entry
  // chunk * chunk_size + tid.  SPLIT: the item takes every n_chunks-th legal slot from `chunk`
  // (entries chunk, chunk + n, chunk + 2n, ...), whose indices do not depend on the count.
  constexpr int LPT = SPLIT ? (LIST + NT - 1) / NT : 1;
  uint32_t slot_of[LPT];
  const uint32_t* lg = a.legal + static_cast<size_t>(s) * a.ring;
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const uint32_t e = SPLIT ? chunk + (tid + j * NT) * a.n_chunks : chunk * a.chunk + tid;
    slot_of[j] = lg[min(e, a.ring - 1)];
  }
  float qv[QPT];
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const int t = min(tid + j * NT, G * HD - 1);
    qv[j] = qkv[(h0 + t / HD) * HD + t % HD];
  }
  const int kt = tid % (2 * HD);  // raw key element kt, or value element kt - HD
  const float kvraw = qkv[(kt < HD ? hq + kvh : hq + hkv + kvh) * HD + kt % HD];
  // keep the compiler from sinking these loads below the early exit, which waits for the count
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  // items holding at least one legal slot, and this item's slot count
  const uint32_t n_items = SPLIT ? min(nl, a.n_chunks) : (nl + a.chunk - 1) / a.chunk;
  if (chunk >= n_items) return;  // no legal slot falls in this item
  const uint32_t total = SPLIT ? min((nl - 1 - chunk) / a.n_chunks + 1, static_cast<uint32_t>(LIST))
                               : min(a.chunk, nl - chunk * a.chunk);
  const bool lead = a.push && a.st != nullptr && chunk == 0;  // list[0] is the slot pushed now
#pragma unroll
  for (int j = 0; j < LPT; ++j)
    if (static_cast<uint32_t>(tid + j * NT) < total) list[tid + j * NT] = slot_of[j];
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const int t = tid + j * NT;
    if (t < G * HD) qs[t / HD][t % HD] = qv[j];
  }
  if (lead && tid < 2 * HD) (kt < HD ? sm.ks : sm.vs)[kt % HD] = kvraw;
  __syncthreads();

  // 2. request this group's first pass of key and value rows
  const size_t row = static_cast<size_t>(hkv) * HD;
  const float* kb = a.k_ring + static_cast<size_t>(s) * a.ring_stream_stride + kvh * HD + 8 * sub;
  const float* vb = a.v_ring + static_cast<size_t>(s) * a.ring_stream_stride + kvh * HD + 8 * sub;
  float4 kk[UNR][2], vv[UNR][2];
  float4 kk2[SPLIT ? UNR : 1][2], vv2[SPLIT ? UNR : 1][2];  // SPLIT: the pass after kk, vv
  auto load_pass = [&](auto& K, auto& V, uint32_t i0) {
    uint32_t slots[UNR];  // every slot index of the pass read from LDS before any load waits
#pragma unroll
    for (int u = 0; u < UNR; ++u) slots[u] = list[min(i0 + u * NG, total - 1)];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const uint32_t i = i0 + u * NG;
      // SPLIT requests every row unconditionally (indices clamped into the item, rows past its
      // end weigh nothing), so the waits of consecutive passes stay ordered and narrow
      if (SPLIT || (i < total && !(lead && i == 0))) {
        const size_t sl = slots[u];
        const float4* kp = reinterpret_cast<const float4*>(kb + sl * row);
        const float4* vp = reinterpret_cast<const float4*>(vb + sl * row);
        K[u][0] = kp[0]; K[u][1] = kp[1];
        V[u][0] = vp[0]; V[u][1] = vp[1];
      } else {
        K[u][0] = K[u][1] = V[u][0] = V[u][1] = f4zero();
      }
    }
  };
  constexpr uint32_t PASS = NG * UNR;
  load_pass(kk, vv, grp);
  if constexpr (SPLIT) load_pass(kk2, vv2, grp + PASS);

  // 3. queries: qk-norm + rope, one wave per head; the pushing item's last wave also normalises and
  //    ropes this step's key and writes key and value into the ring slot pos mod R
  const bool prep = a.q_norm != nullptr || a.cs != nullptr;
  const int ia = a.rope_style == 0 ? lane : 2 * lane;
  const int ib = a.rope_style == 0 ? lane + HALF : 2 * lane + 1;
  if (prep) {
    for (int g = wave; g < G; g += NWV) {
      float va = lane < HALF ? qs[g][ia] : 0.f, vb2 = lane < HALF ? qs[g][ib] : 0.f;
      norm_rope_pair<HD>(va, vb2, lane, a.q_norm, a.eps, cs, a.rope_style);
      if (lane < HALF) {
        qs[g][ia] = va;
        qs[g][ib] = vb2;
      }
    }
  }
  if (lead && wave == NWV - 1) {
    float va = lane < HALF ? sm.ks[ia] : 0.f, vb2 = lane < HALF ? sm.ks[ib] : 0.f;
    norm_rope_pair<HD>(va, vb2, lane, a.k_norm, a.eps, cs, a.rope_style);
    const uint32_t ps = a.st->slot;
    const size_t roff = static_cast<size_t>(s) * a.ring_stream_stride +
                        (static_cast<size_t>(ps) * hkv + kvh) * HD;
    if (lane < HALF) {
      sm.ks[ia] = va;
      sm.ks[ib] = vb2;
      a.k_ring[roff + ia] = va;
      a.k_ring[roff + ib] = vb2;
    }
    for (int d = lane; d < HD; d += kWave) a.v_ring[roff + d] = sm.vs[d];
  }
  __syncthreads();  // queries and this step's key are in LDS

  // 4. online softmax over this group's share of the legal slots.  Scores are kept in log2 units
  //    (q.k log2(e) / sqrt(hd)), so every exponential is one exp2 instruction; the chunk maxima
  //    left in the partials are in the same units.
  float q[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) q[g][e] = qs[g][8 * sub + e];
  const float scale = 1.4426950408889634f / sqrtf(static_cast<float>(HD));
  float mrun[G], lrun[G], acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    mrun[g] = -INFINITY;
    lrun[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
  }
  auto score_pass = [&](auto& K, auto& V, uint32_t i0) {
    // all UNR scores of the pass first (independent chains), then one softmax update per head
    float sc[UNR][G];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const uint32_t i = i0 + u * NG;
      float kf[8] = {K[u][0].x, K[u][0].y, K[u][0].z, K[u][0].w,
                     K[u][1].x, K[u][1].y, K[u][1].z, K[u][1].w};
      if (lead && i == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) kf[e] = sm.ks[8 * sub + e];
        V[u][0] = make_float4(sm.vs[8 * sub], sm.vs[8 * sub + 1], sm.vs[8 * sub + 2], sm.vs[8 * sub + 3]);
        V[u][1] = make_float4(sm.vs[8 * sub + 4], sm.vs[8 * sub + 5], sm.vs[8 * sub + 6], sm.vs[8 * sub + 7]);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d = fmaf(q[g][e], kf[e], d);
        d = group_sum<LPS>(d);
        sc[u][g] = i < total ? d * scale : -INFINITY;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mb = sc[0][g];
#pragma unroll
      for (int u = 1; u < UNR; ++u) mb = fmaxf(mb, sc[u][g]);
      const float mnew = fmaxf(mrun[g], mb);
      if (mnew != -INFINITY) {
        const float corr = __builtin_amdgcn_exp2f(mrun[g] - mnew);  // 0 while mrun is -inf
        lrun[g] *= corr;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] *= corr;
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const float p = __builtin_amdgcn_exp2f(sc[u][g] - mnew);  // 0 for a masked slot
          const float vf[8] = {V[u][0].x, V[u][0].y, V[u][0].z, V[u][0].w,
                               V[u][1].x, V[u][1].y, V[u][1].z, V[u][1].w};
          lrun[g] += p;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(p, vf[e], acc[g][e]);
        }
        mrun[g] = mnew;
      }
    }
  };
  if constexpr (SPLIT) {
    for (uint32_t i0 = grp; i0 < total;) {
      score_pass(kk, vv, i0);
      load_pass(kk, vv, i0 + 2 * PASS);  // clamped: past the end it re-reads the last slot
      i0 += PASS;
      if (i0 >= total) break;
      score_pass(kk2, vv2, i0);
      load_pass(kk2, vv2, i0 + 2 * PASS);
      i0 += PASS;
    }
  } else {
    for (uint32_t i0 = grp; i0 < total;) {  // a group past the item's end has nothing to score
      score_pass(kk, vv, i0);
      i0 += PASS;
      if (i0 >= total) break;
      load_pass(kk, vv, i0);
    }
  }

  // 5. merge the slot groups into the chunk's (max, sum, output): first the GPW groups of each
  //    wave (lanes LPS, 2 LPS, ... apart hold the same elements) with cross-lane moves, then the
  //    waves through LDS
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float M = mrun[g];
#pragma unroll
    for (int off = LPS; off < kWave; off <<= 1)
      M = off == 8 ? fmaxf(M, lane_xor<8>(M, lane)) : off == 16 ? pair_max<16>(M) : pair_max<32>(M);
    const float c = mrun[g] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrun[g] - M);
    float v[9];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = acc[g][e] * c;
    v[8] = lrun[g] * c;
#pragma unroll
    for (int off = LPS; off < kWave; off <<= 1)
#pragma unroll
      for (int e = 0; e < 9; ++e)
        v[e] = off == 8 ? v[e] + lane_xor<8>(v[e], lane) : off == 16 ? pair_sum<16>(v[e]) : pair_sum<32>(v[e]);
    if (lane < LPS) {  // the wave's first group writes the wave's merge
      if (sub == 0) {
        sm_m[wave][g] = M;
        sm_l[wave][g] = v[8];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) sm_acc[wave][g][8 * sub + e] = v[e];
    }
  }
  __syncthreads();
  const bool single = n_items == 1;
  for (int t = tid; t < G * HD; t += NT) {
    const int g = t / HD, d = t % HD;
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < NWV; ++k) M = fmaxf(M, sm_m[k][g]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int k = 0; k < NWV; ++k) {
      const float mk = sm_m[k][g];
      if (mk != -INFINITY) {
        const float w = __builtin_amdgcn_exp2f(mk - M);
        L = fmaf(w, sm_l[k][g], L);
        O = fmaf(w, sm_acc[k][g][d], O);
      }
    }
    if (single) {
      put<COH>(a.out + static_cast<size_t>(s) * hq * HD + (h0 + g) * HD + d, L > 0.f ? O / L : 0.f);
    } else {
      // chunk partials: unnormalised output rows, then (max, sum) pairs after all of them
      const size_t pi = (static_cast<size_t>(s) * hq + h0 + g) * a.n_chunks + chunk;
      float* po = a.part + pi * HD + d;
      float* pml = a.part + static_cast<size_t>(a.m) * hq * a.n_chunks * HD + pi * 2;
      if (a.partials_only) {
        *po = O;
        if (d == 0) {
          pml[0] = M;
          pml[1] = L;
        }
      } else {
        st_dev(po, O);
        if (d == 0) {
          st_dev(pml, M);
          st_dev(pml + 1, L);
        }
      }
    }
  }
  if (single || a.partials_only) return;

  // 6. the last chunk of this (stream, kv head) to finish merges all chunks.  The partials went
  // out with agent-scope stores (written through to the device's point of coherence); every wave
  // waits for their acknowledgement before the barrier, the count is an agent-scope RMW at that
  // point, and the merging workgroup reads with agent-scope loads issued after its RMW returned.
  // (Release and acquire fences instead compile to an L2 writeback per wave and an L2 invalidate:
  // measured on the eight-stream talker step, 3.05 -> 5.61 ms.)
  wait_stores();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&a.counters[s * hkv + kvh], 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    is_last = prev == n_items - 1 ? 1u : 0u;
  }
  __syncthreads();
  if (!is_last) return;
  float* stage = &sm_acc[0][0][0];  // [CB][G][HD]
  float Mr[(G * HD + NT - 1) / NT], Lr[(G * HD + NT - 1) / NT];
  float Or[(G * HD + NT - 1) / NT];
#pragma unroll
  for (int i = 0; i < (G * HD + NT - 1) / NT; ++i) {
    Mr[i] = -INFINITY;
    Lr[i] = 0.f;
    Or[i] = 0.f;
  }
  // A batch's partials are requested CG per thread at a time before any is used (one memory round
  // trip per batch when CG covers it).
  constexpr int PER = (CB * G * (HD + 2) + NT - 1) / NT;
  constexpr int GRP = CG > 0 && CG < PER ? CG : PER;
  for (uint32_t b0 = 0; b0 < n_items; b0 += CB) {
    const uint32_t nb = min(static_cast<uint32_t>(CB), n_items - b0);
    const uint32_t n_e = nb * G * (HD + 2);
    __syncthreads();  // the previous batch is consumed
    for (int k0 = 0; k0 < PER; k0 += GRP) {
      float pv[GRP];
#pragma unroll
      for (int k = 0; k < GRP; ++k) {
        const uint32_t e = tid + (k0 + k) * NT;
        const uint32_t c = e / (G * (HD + 2)), rem = e % (G * (HD + 2));
        const uint32_t g = rem / (HD + 2), d = rem % (HD + 2);
        const size_t pi = (static_cast<size_t>(s) * hq + h0 + g) * a.n_chunks + b0 + c;
        const float* src = d < HD ? a.part + pi * HD + d
                                  : a.part + static_cast<size_t>(a.m) * hq * a.n_chunks * HD + pi * 2 +
                                        (d - HD);
        pv[k] = e < n_e ? ld_dev(src) : 0.f;
      }
#pragma unroll
      for (int k = 0; k < GRP; ++k) {
        const uint32_t e = tid + (k0 + k) * NT;
        const uint32_t c = e / (G * (HD + 2)), rem = e % (G * (HD + 2));
        const uint32_t g = rem / (HD + 2), d = rem % (HD + 2);
        if (e < n_e) {
          if (d < HD) stage[(c * G + g) * HD + d] = pv[k];
          else if (d == HD) sm_m[c][g] = pv[k];
          else sm_l[c][g] = pv[k];
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < (G * HD + NT - 1) / NT; ++i) {
      const int t = tid + i * NT;
      if (t < G * HD) {
        const int g = t / HD, d = t % HD;
        float Mb = Mr[i];
        for (uint32_t c = 0; c < nb; ++c) Mb = fmaxf(Mb, sm_m[c][g]);
        if (Mb != -INFINITY) {
          const float corr = Mr[i] != -INFINITY ? __builtin_amdgcn_exp2f(Mr[i] - Mb) : 0.f;
          float L = Lr[i] * corr, O = Or[i] * corr;
          for (uint32_t c = 0; c < nb; ++c) {
            const float mc = sm_m[c][g];
            if (mc != -INFINITY) {
              const float w = __builtin_amdgcn_exp2f(mc - Mb);
              L = fmaf(w, sm_l[c][g], L);
              O = fmaf(w, stage[(c * G + g) * HD + d], O);
            }
          }
          Mr[i] = Mb;
          Lr[i] = L;
          Or[i] = O;
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < (G * HD + NT - 1) / NT; ++i) {
    const int t = tid + i * NT;
    if (t < G * HD) {
      const int g = t / HD, d = t % HD;
      put<COH>(a.out + static_cast<size_t>(s) * hq * HD + (h0 + g) * HD + d,
               Lr[i] > 0.f ? Or[i] / Lr[i] : 0.f);
    }
  }
  if (tid == 0)
    __hip_atomic_store(&a.counters[s * hkv + kvh], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace dev
}  // namespace sdec
