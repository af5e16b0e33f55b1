// Streaming codec convolutions on CDNA4 ([mimi] inferencelayer 0.2.1, src/mimi_gpu.rs: CONV1D with
// the carried input prefix of WRITE_XA / CARRY / REPLICATE, the gather-form transposed conv of
// convtr_src with its overlap tail carried bias-subtracted by TRP_ADD / TR_OUT / TR_CARRY, and
// the ELU of ELU_IP folded into the reads).  Frames arrive one at a time; the state between them
// is the last K - S input columns of a conv and the K - S pending output columns of a transposed
// conv, kept in ping-pong buffers so no kernel reads what another thread of it rewrites.

#include <hip/hip_runtime.h>
#include <math.h>

#include "dev.h"
#include "kernels.h"

namespace sdec {

namespace {

__device__ __forceinline__ float elu_f(float v) { return v > 0.f ? v : expf(v) - 1.0f; }

// Column j of the padded input stream of this frame: the carried prefix, then the frame.  On the
// first frame the prefix is zeros or copies of the frame's first column.
__device__ __forceinline__ float sconv_sample(const SConvArgs& a, uint32_t ic, uint32_t j) {
  if (j >= a.pad) return a.x[static_cast<size_t>(ic) * a.t_in + (j - a.pad)];
  if (a.first) return a.replicate_first ? a.x[static_cast<size_t>(ic) * a.t_in] : 0.f;
  return a.prefix[static_cast<size_t>(ic) * a.pad + j];
}

// One thread per (output channel, output column); grid (ceil(t_out / 64), c_out).
__global__ __launch_bounds__(64) void k_sconv(SConvArgs a) {
  const uint32_t oc = blockIdx.y;
  const uint32_t ot = blockIdx.x * 64 + threadIdx.x;
  const uint32_t t_out = a.t_in / a.stride;
  if (ot >= t_out) return;
  const uint32_t ipg = a.c_in / a.groups, opg = a.c_out / a.groups;
  const uint32_t ic0 = (oc / opg) * ipg;
  float acc = a.b[oc];
  for (uint32_t i = 0; i < ipg; ++i) {
    const float* w = a.w + (static_cast<size_t>(oc) * ipg + i) * a.k;
    for (uint32_t k = 0; k < a.k; ++k) {
      float v = sconv_sample(a, ic0 + i, ot * a.stride + k);
      if (a.pre_elu) v = elu_f(v);
      acc = fmaf(w[k], v, acc);
    }
  }
  float* y = a.y + static_cast<size_t>(oc) * t_out + ot;
  *y = a.accumulate ? *y + acc : acc;
}

// The next frame's prefix: the last pad columns of this frame's padded stream.
__global__ __launch_bounds__(256) void k_sconv_carry(SConvArgs a) {
  const uint32_t e = blockIdx.x * 256 + threadIdx.x;
  if (e >= a.c_in * a.pad) return;
  const uint32_t ic = e / a.pad, i = e % a.pad;
  a.prefix_out[e] = sconv_sample(a, ic, a.t_in + i);
}

// Transposed conv, gather form: one thread per (output channel, column i of this frame's full
// output, i < t_in*S + K - S); grid (ceil(len / 64), c_out).  Columns below t_in*S are emitted
// with the carried tail added; the rest become the next tail, bias subtracted.
__global__ __launch_bounds__(64) void k_sconvtr(SConvTrArgs a) {
  const uint32_t oc = blockIdx.y;
  const uint32_t i = blockIdx.x * 64 + threadIdx.x;
  const uint32_t emit = a.t_in * a.stride, len = emit + a.tl;
  if (i >= len) return;
  const uint32_t ipg = a.c_in / a.groups, opg = a.c_out / a.groups;
  const uint32_t g = oc / opg, oo = oc % opg;
  float acc = a.b[oc];
  // the input columns whose taps reach column i, tap k = i - ti * stride ascending (ti from the
  // largest with ti * stride <= i down), one division per thread
  const uint32_t ti_hi = min(i / a.stride, a.t_in - 1);
  for (int32_t ti = static_cast<int32_t>(ti_hi); ti >= 0; --ti) {
    const uint32_t k = i - static_cast<uint32_t>(ti) * a.stride;
    if (k >= a.k) break;
    for (uint32_t ii = 0; ii < ipg; ++ii) {
      const uint32_t ic = g * ipg + ii;
      float v = a.x[static_cast<size_t>(ic) * a.t_in + ti];
      if (a.pre_elu) v = elu_f(v);
      acc = fmaf(a.w[(static_cast<size_t>(ic) * opg + oo) * a.k + k], v, acc);
    }
  }
  const float old = (!a.first && i < a.tl) ? a.tail[static_cast<size_t>(oc) * a.tl + i] : 0.f;
  if (i < emit) {
    a.y[static_cast<size_t>(oc) * emit + i] = acc + old;
  } else {
    a.tail_out[static_cast<size_t>(oc) * a.tl + (i - emit)] = (acc - a.b[oc]) + old;
  }
}

// Tiled forms for groups == 1: a workgroup of 256 threads owns oc_t output channels x t_t output
// columns (oc_t * t_t == 256, one output per thread) and walks the input channels in blocks of
// icb, staging the block's input window (ELU applied once per sample) and weights in LDS, so the
// inner loop reads only LDS.  Per output the sum runs over input channels, then taps, as in the
// one-thread-per-output kernels above.
constexpr uint32_t kConvTileThreads = 256;
constexpr int kConvStageBatch = 8;

// Quotient and remainder by a divisor fixed for the launch, for dividends below 2^24: the float
// estimate e * (1/d) is within one of the quotient (both operands exact in float32, the product
// off by under 2 ulp of a value below 2^24), and one remainder test corrects it.  A few
// instructions instead of the ~30 of an integer division, which dominated the staging loops.
struct FastDiv {
  uint32_t d;
  float inv;
  __device__ explicit FastDiv(uint32_t dv) : d(dv), inv(1.0f / static_cast<float>(dv)) {}
  __device__ __forceinline__ uint32_t div(uint32_t e, uint32_t& rem) const {
    uint32_t q = static_cast<uint32_t>(static_cast<float>(e) * inv);
    int32_t r = static_cast<int32_t>(e) - static_cast<int32_t>(q * d);
    if (r < 0) {
      --q;
      r += static_cast<int32_t>(d);
    } else if (r >= static_cast<int32_t>(d)) {
      ++q;
      r -= static_cast<int32_t>(d);
    }
    rem = static_cast<uint32_t>(r);
    return q;
  }
};

// Split-k hand-off: every split of an output tile leaves its partial sum with a device-coherent
// store and counts itself in the tile's counter; the last one to arrive (nothing waits) reads
// the others' partials back with device-coherent loads and finishes the tile.  Returns whether
// this workgroup is that last one; it also resets the counter for the next launch.
// Ordering, on the hardware: the partial goes out as an agent-scope store (written through to the
// device's point of coherence), every wave waits for its stores to be acknowledged before the
// workgroup barrier, the count is an agent-scope RMW performed at that point, and the finisher
// reads with agent-scope loads issued after its RMW returned, which bypass the non-coherent
// caches.  The language-level form (release before the count, acquire after it) compiles to an
// L2 writeback and an L2 invalidate per wave; measured on the SEANet-style frame it costs 151 ->
// 443 us per frame, so the hand-off keeps the relaxed agent-scope operations.
__device__ __forceinline__ bool conv_split_arrive(uint32_t* counter, uint32_t splits, bool live,
                                                  float* slot, float acc) {
  __shared__ uint32_t last;
  if (live) dev::st_dev(slot, acc);
  dev::wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = prev == splits - 1 ? 1u : 0u;
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return last != 0;
}

// acc plus the splits' partial sums of one output, added in split order: every partial is
// requested before the first is added (a loop of load, wait, add paid one device-coherent round
// trip per split; the indices are clamped, so the loads need no branch).
__device__ __forceinline__ float conv_split_sum(float acc, const float* p, size_t plane,
                                                uint32_t splits) {
  float v[kConvMaxSplits];
#pragma unroll
  for (uint32_t z = 0; z < kConvMaxSplits; ++z) v[z] = dev::ld_dev(p + min(z, splits - 1) * plane);
#pragma unroll
  for (uint32_t z = 0; z < kConvMaxSplits; ++z)
    if (z < splits) acc += v[z];
  return acc;
}

// Fills n LDS elements, kConvStageBatch per thread per batch: the batch's global loads are all
// issued before any result is used (indices clamped into [0, n), so no branch guards a load), so
// a thread waits about one memory round trip per batch instead of one per element.
template <typename Load, typename Store>
__device__ __forceinline__ void conv_stage(uint32_t n, Load load, Store store) {
  for (uint32_t e0 = threadIdx.x; e0 < n; e0 += kConvStageBatch * kConvTileThreads) {
    float v[kConvStageBatch];
#pragma unroll
    for (int u = 0; u < kConvStageBatch; ++u) v[u] = load(min(e0 + u * kConvTileThreads, n - 1));
#pragma unroll
    for (int u = 0; u < kConvStageBatch; ++u) {
      const uint32_t e = e0 + u * kConvTileThreads;
      if (e < n) store(e, v[u]);
    }
  }
}

// A block of `rows` rows of rw floats (rw a multiple of 4): row r from global src + r * gs (16-byte
// aligned) into LDS dst + r * ds (ds a multiple of 4), rows at or past `valid` (1 <= valid) filled
// with zeros.
// One 16-byte load per four floats, a batch of four per thread issued before any is stored: a
// quarter of the load instructions of the element-wise staging, which is what a weight tile's
// staging time tracked.
__device__ __forceinline__ void conv_stage_rows4(float* dst, uint32_t ds, const float* src, size_t gs,
                                                 uint32_t rows, uint32_t valid, uint32_t rw) {
  constexpr int B = 4;
  const uint32_t q = rw >> 2, n = rows * q;
  const FastDiv dq(q);
  for (uint32_t e0 = threadIdx.x; e0 < n; e0 += B * kConvTileThreads) {
    float4 v[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      uint32_t c;
      const uint32_t r = dq.div(min(e0 + u * kConvTileThreads, n - 1), c);
      // rows past `valid` read the last valid row (in bounds) and store zeros
      v[u] = *reinterpret_cast<const float4*>(src + min(r, valid - 1) * gs + 4 * c);
      if (r >= valid) v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const uint32_t e = e0 + u * kConvTileThreads;
      if (e < n) {
        uint32_t c;
        const uint32_t r = dq.div(e, c);
        *reinterpret_cast<float4*>(dst + r * ds + 4 * c) = v[u];
      }
    }
  }
}

// With gridDim.z > 1 the input channels are split: workgroup z sums channels [z * ics, (z+1) * ics)
// without the bias into part[z], and k_sconv_sum adds the splits in order.
// KT: the kernel size when it is one of the unrolled ones (1, 3, 7), else 0 (a.k at run time).
// Unrolled, the LDS reads of several input channels are issued before their products are summed,
// instead of one LDS round trip per product.
template <int KT>
__global__ __launch_bounds__(kConvTileThreads) void k_sconv_tiled(SConvArgs a, uint32_t oc_t,
                                                                  uint32_t t_t, uint32_t icb,
                                                                  uint32_t ics) {
  extern __shared__ float lds[];
  const uint32_t t_out = a.t_in / a.stride;
  const bool split = gridDim.z > 1;
  const uint32_t ic_begin = blockIdx.z * ics, ic_end = min(a.c_in, ic_begin + ics);
  const uint32_t oc0 = blockIdx.y * oc_t, col0 = blockIdx.x * t_t;
  const uint32_t xw = t_t * a.stride + a.pad;  // padded-stream columns the tile reads
  float* X = lds;
  float* W = lds + icb * xw;
  // W rows (one per output channel) padded by 4 floats: the channel groups of a wave (64 / t_t of
  // them, each reading one row in lockstep) then fall in different LDS banks
  const uint32_t wst = icb * a.k + 4;
  const uint32_t tid = threadIdx.x;
  const uint32_t ocl = tid / t_t, otl = tid % t_t;
  const uint32_t oc = oc0 + ocl, ot = col0 + otl;
  const bool live = oc < a.c_out && ot < t_out;
  float acc = live && !split ? a.b[oc] : 0.f;
  if (blockIdx.z == 0 && a.pad > 0) {
    // the next frame's prefix (the last pad columns of this frame's padded stream), spread over
    // the workgroups of the first split: it depends on the inputs only, so it needs no launch of
    // its own
    const uint32_t n_carry = a.c_in * a.pad;
    const uint32_t step = gridDim.x * gridDim.y * kConvTileThreads;
    for (uint32_t e = (blockIdx.y * gridDim.x + blockIdx.x) * kConvTileThreads + tid; e < n_carry;
         e += step)
      a.prefix_out[e] = sconv_sample(a, e / a.pad, a.t_in + e % a.pad);
  }
  for (uint32_t ic0 = ic_begin; ic0 < ic_end; ic0 += icb) {
    const uint32_t nb = min(icb, ic_end - ic0);
    __syncthreads();  // the previous block is consumed
    // X[i][j]: padded-stream column col0 * stride + j of input channel ic0 + i.  The tile's
    // first n_pre columns lie in the carried prefix (only tiles that start inside it have
    // any); the rest come from this frame, zero past its end.  Each region is staged with one
    // unconditional load per element.
    const uint32_t c_lo = col0 * a.stride;
    const uint32_t n_pre = c_lo < a.pad ? min(a.pad - c_lo, xw) : 0u, wx = xw - n_pre;
    const FastDiv dwx(wx);
    conv_stage(
        nb * wx,
        [&](uint32_t e) {
          uint32_t j;
          const uint32_t i = dwx.div(e, j);
          const uint32_t col = c_lo + n_pre + j;
          const float v = a.x[static_cast<size_t>(ic0 + i) * a.t_in + min(col - a.pad, a.t_in - 1)];
          return col < a.t_in + a.pad ? v : 0.f;
        },
        [&](uint32_t e, float v) {
          uint32_t j;
          const uint32_t i = dwx.div(e, j);
          X[i * xw + n_pre + j] = a.pre_elu ? elu_f(v) : v;
        });
    if (n_pre) {
      // the prefix, or on the first frame zeros or copies of the frame's first column
      const bool from_x = a.first && a.replicate_first;
      conv_stage(
          nb * n_pre,
          [&](uint32_t e) {
            const size_t row = static_cast<size_t>(ic0 + e / n_pre);
            return from_x ? a.x[row * a.t_in] : a.prefix[row * a.pad + c_lo + e % n_pre];
          },
          [&](uint32_t e, float v) {
            if (a.first && !a.replicate_first) v = 0.f;
            X[(e / n_pre) * xw + e % n_pre] = a.pre_elu ? elu_f(v) : v;
          });
    }
    // W[o][i][k] for output channel oc0 + o (zero past c_out): row o of the tile is nb * k
    // consecutive floats of the weights
    if (((nb * a.k) & 3u) == 0 && ((a.c_in * a.k) & 3u) == 0 && ((ic0 * a.k) & 3u) == 0 &&
        (reinterpret_cast<uintptr_t>(a.w) & 15u) == 0) {
      const uint32_t valid = a.c_out > oc0 ? min(oc_t, a.c_out - oc0) : 0u;
      conv_stage_rows4(W, wst,
                       a.w + (static_cast<size_t>(min(oc0, a.c_out - 1)) * a.c_in + ic0) * a.k,
                       static_cast<size_t>(a.c_in) * a.k, valid > 0 ? oc_t : 0u, valid, nb * a.k);
    } else {
      const FastDiv dnk(nb * a.k);
      conv_stage(
          oc_t * nb * a.k,
          [&](uint32_t e) {
            uint32_t r;
            const uint32_t o = dnk.div(e, r);
            return a.w[(static_cast<size_t>(min(oc0 + o, a.c_out - 1)) * a.c_in + ic0) * a.k + r];
          },
          [&](uint32_t e, float v) {
            uint32_t r;
            const uint32_t o = dnk.div(e, r);
            W[o * wst + r] = oc0 + o < a.c_out ? v : 0.f;
          });
    }
    __syncthreads();
    if (live) {
      const float* wr = W + ocl * wst;
      if constexpr (KT > 0) {
#pragma unroll 4
        for (uint32_t i = 0; i < nb; ++i) {
          const float* xr = X + i * xw + otl * a.stride;
#pragma unroll
          for (int k = 0; k < KT; ++k) acc = fmaf(wr[i * KT + k], xr[k], acc);
        }
      } else {
        for (uint32_t i = 0; i < nb; ++i) {
          const float* xr = X + i * xw + otl * a.stride;
          for (uint32_t k = 0; k < a.k; ++k) acc = fmaf(wr[i * a.k + k], xr[k], acc);
        }
      }
    }
  }
  if (split) {
    const size_t plane = static_cast<size_t>(a.c_out) * t_out, e = static_cast<size_t>(oc) * t_out + ot;
    if (a.counters == nullptr) {  // k_sconv_sum finishes the tiles
      if (live) a.part[blockIdx.z * plane + e] = acc;
      return;
    }
    float* mine = a.part + blockIdx.z * plane + e;
    if (!conv_split_arrive(a.counters + blockIdx.y * gridDim.x + blockIdx.x, gridDim.z, live, mine,
                           acc))
      return;
    if (!live) return;
    acc = a.b[oc];  // the bias, then the splits in order
    acc = conv_split_sum(acc, a.part + e, plane, gridDim.z);
  }
  if (live) {
    float* y = a.y + static_cast<size_t>(oc) * t_out + ot;
    *y = a.accumulate ? *y + acc : acc;
  }
}

// The splits of a split-k conv: bias, then the partial sums in split order.
__global__ __launch_bounds__(256) void k_sconv_sum(SConvArgs a, uint32_t splits) {
  const uint32_t t_out = a.t_in / a.stride;
  const uint32_t e = blockIdx.x * 256 + threadIdx.x;
  if (e >= a.c_out * t_out) return;
  const uint32_t oc = e / t_out;
  float acc = a.b[oc];
  for (uint32_t z = 0; z < splits; ++z) acc += a.part[static_cast<size_t>(z) * a.c_out * t_out + e];
  a.y[e] = a.accumulate ? a.y[e] + acc : acc;
}

// Column i of this frame's full transposed-conv output (bias included in acc): below t_in * S it
// is emitted with the carried tail added; the rest becomes the next tail, bias subtracted.
__device__ __forceinline__ void sconvtr_emit(const SConvTrArgs& a, uint32_t oc, uint32_t i, float acc) {
  const uint32_t emit = a.t_in * a.stride;
  const float old = (!a.first && i < a.tl) ? a.tail[static_cast<size_t>(oc) * a.tl + i] : 0.f;
  if (i < emit) {
    a.y[static_cast<size_t>(oc) * emit + i] = acc + old;
  } else {
    a.tail_out[static_cast<size_t>(oc) * a.tl + (i - emit)] = (acc - a.b[oc]) + old;
  }
}

// Split input channels as in k_sconv_tiled; k_sconvtr_sum adds the splits and emits.
__global__ __launch_bounds__(kConvTileThreads) void k_sconvtr_tiled(SConvTrArgs a, uint32_t oc_t,
                                                                    uint32_t t_t, uint32_t icb,
                                                                    uint32_t ics) {
  extern __shared__ float lds[];
  const uint32_t emit = a.t_in * a.stride, len = emit + a.tl;
  const bool split = gridDim.z > 1;
  const uint32_t ic_begin = blockIdx.z * ics, ic_end = min(a.c_in, ic_begin + ics);
  const uint32_t i0 = blockIdx.x * t_t, oc0 = blockIdx.y * oc_t;
  // input columns that reach output columns [i0, i0 + t_t)
  const uint32_t lo = i0 + 1 > a.k ? (i0 + 1 - a.k + a.stride - 1) / a.stride : 0;
  const uint32_t hi = min(a.t_in - 1, (i0 + t_t - 1) / a.stride);
  const uint32_t xw = hi >= lo ? hi - lo + 1 : 0;
  const uint32_t xcap = t_t / a.stride + a.k / a.stride + 2;  // LDS columns per channel
  float* X = lds;
  float* W = lds + icb * xcap;
  const uint32_t tid = threadIdx.x;
  const uint32_t ocl = tid / t_t, il = tid % t_t;
  const uint32_t oc = oc0 + ocl, i = i0 + il;
  const bool live = oc < a.c_out && i < len;
  float acc = live && !split ? a.b[oc] : 0.f;
  const FastDiv dxw(xw > 0 ? xw : 1u), dok(oc_t * a.k), dk(a.k);
  for (uint32_t ic0 = ic_begin; ic0 < ic_end; ic0 += icb) {
    const uint32_t nb = min(icb, ic_end - ic0);
    __syncthreads();
    conv_stage(
        nb * xw,
        [&](uint32_t e) {
          uint32_t j;
          const uint32_t c = dxw.div(e, j);
          return a.x[static_cast<size_t>(ic0 + c) * a.t_in + lo + j];
        },
        [&](uint32_t e, float v) {
          uint32_t j;
          const uint32_t c = dxw.div(e, j);
          X[c * xcap + j] = a.pre_elu ? elu_f(v) : v;
        });
    if (oc0 + oc_t <= a.c_out && ((oc_t * a.k) & 3u) == 0 && ((a.c_out * a.k) & 3u) == 0 &&
        (reinterpret_cast<uintptr_t>(a.w) & 15u) == 0) {
      // W[c][o][k]: row c of the tile is the oc_t * k consecutive floats of input channel ic0 + c
      conv_stage_rows4(W, oc_t * a.k, a.w + (static_cast<size_t>(ic0) * a.c_out + oc0) * a.k,
                       static_cast<size_t>(a.c_out) * a.k, nb, nb, oc_t * a.k);
    } else {
      conv_stage(
          nb * oc_t * a.k,
          [&](uint32_t e) {
            uint32_t r, k;
            const uint32_t c = dok.div(e, r), o = dk.div(r, k);
            return a.w[(static_cast<size_t>(ic0 + c) * a.c_out + min(oc0 + o, a.c_out - 1)) * a.k + k];
          },
          [&](uint32_t e, float v) {
            uint32_t r, k;
            dok.div(e, r);
            const uint32_t o = dk.div(r, k);
            W[e] = oc0 + o < a.c_out ? v : 0.f;
          });
    }
    __syncthreads();
    if (live) {
      for (uint32_t k = i % a.stride; k < a.k && k <= i; k += a.stride) {
        const uint32_t ti = (i - k) / a.stride;
        if (ti >= a.t_in) continue;
        const float* xr = X + (ti - lo);
        const float* wr = W + ocl * a.k + k;
#pragma unroll 8
        for (uint32_t c = 0; c < nb; ++c) acc = fmaf(wr[c * oc_t * a.k], xr[c * xcap], acc);
      }
    }
  }
  if (split) {
    const size_t plane = static_cast<size_t>(a.c_out) * len, e = static_cast<size_t>(oc) * len + i;
    if (a.counters == nullptr) {  // k_sconvtr_sum finishes the tiles
      if (live) a.part[blockIdx.z * plane + e] = acc;
      return;
    }
    float* mine = a.part + blockIdx.z * plane + e;
    if (!conv_split_arrive(a.counters + blockIdx.y * gridDim.x + blockIdx.x, gridDim.z, live, mine,
                           acc))
      return;
    if (!live) return;
    acc = a.b[oc];  // the bias, then the splits in order
    acc = conv_split_sum(acc, a.part + e, plane, gridDim.z);
  }
  if (!live) return;
  sconvtr_emit(a, oc, i, acc);
}

__global__ __launch_bounds__(256) void k_sconvtr_sum(SConvTrArgs a, uint32_t splits) {
  const uint32_t len = a.t_in * a.stride + a.tl;
  const uint32_t e = blockIdx.x * 256 + threadIdx.x;
  if (e >= a.c_out * len) return;
  const uint32_t oc = e / len, i = e % len;
  float acc = a.b[oc];
  for (uint32_t z = 0; z < splits; ++z) acc += a.part[static_cast<size_t>(z) * a.c_out * len + e];
  sconvtr_emit(a, oc, i, acc);
}

// Output tile: t_t columns (a power of two, 16..64, covering short frames) x 256/t_t channels.
void conv_tile(uint32_t cols, uint32_t& oc_t, uint32_t& t_t) {
  t_t = cols <= 16 ? 16 : cols <= 32 ? 32 : 64;
  oc_t = kConvTileThreads / t_t;
}
constexpr uint32_t kConvIcb = 32;

// Input-channel splits for a tiled launch of `grid` workgroups: enough to give the device about
// four workgroups per CU (SEANet frame 182 us vs 193 us at two), whole blocks of kConvIcb channels
// per split, and within the scratch.
uint32_t conv_splits(uint32_t grid, uint32_t c_in, uint64_t outs, uint64_t cap, uint32_t* ics) {
  const uint32_t blocks = (c_in + kConvIcb - 1) / kConvIcb;
  uint32_t s = (1024 + grid - 1) / grid;
  if (s > blocks) s = blocks;
  if (s > kConvMaxSplits) s = kConvMaxSplits;
  while (s > 1 && static_cast<uint64_t>(s) * outs > cap) --s;
  if (s <= 1) {
    *ics = c_in;
    return 1;
  }
  const uint32_t bps = (blocks + s - 1) / s;  // blocks per split
  *ics = bps * kConvIcb;
  return (c_in + *ics - 1) / *ics;
}

}  // namespace

hipError_t launch_sconv(const SConvArgs& a, hipStream_t s) {
  const uint32_t t_out = a.t_in / a.stride;
  if (t_out == 0 || a.c_out == 0 || a.c_out > 65535) return hipErrorInvalidValue;
  if (a.groups == 1) {
    uint32_t oc_t, t_t;
    conv_tile(t_out, oc_t, t_t);
    const uint32_t xw = t_t * a.stride + a.pad;
    const size_t lds = (static_cast<size_t>(kConvIcb) * xw + static_cast<size_t>(oc_t) * (kConvIcb * a.k + 4)) * sizeof(float);
    if (lds > 64 * 1024) return hipErrorInvalidValue;
    const dim3 g((t_out + t_t - 1) / t_t, (a.c_out + oc_t - 1) / oc_t);
    uint32_t ics = a.c_in;
    const uint32_t splits = a.part ? conv_splits(g.x * g.y, a.c_in,
                                                 static_cast<uint64_t>(a.c_out) * t_out, a.part_cap, &ics)
                                   : 1u;
    const void* fn = a.k == 1   ? reinterpret_cast<const void*>(&k_sconv_tiled<1>)
                     : a.k == 3 ? reinterpret_cast<const void*>(&k_sconv_tiled<3>)
                     : a.k == 7 ? reinterpret_cast<const void*>(&k_sconv_tiled<7>)
                                : reinterpret_cast<const void*>(&k_sconv_tiled<0>);
    SConvArgs args = a;
    if (splits <= 1 || static_cast<uint64_t>(g.x) * g.y > a.counter_cap) args.counters = nullptr;
    uint32_t p_oc = oc_t, p_t = t_t, p_icb = kConvIcb, p_ics = ics;
    void* params[] = {&args, &p_oc, &p_t, &p_icb, &p_ics};
    hipError_t le = hipLaunchKernel(fn, dim3(g.x, g.y, splits), dim3(kConvTileThreads), params, lds, s);
    if (le != hipSuccess) return le;
    if (splits > 1 && args.counters == nullptr)
      hipLaunchKernelGGL(k_sconv_sum, dim3((a.c_out * t_out + 255) / 256), dim3(256), 0, s, a, splits);
    return hipGetLastError();  // the tiled kernel also writes the next prefix
  } else {
    hipLaunchKernelGGL(k_sconv, dim3((t_out + 63) / 64, a.c_out), dim3(64), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.pad == 0) return e;
  hipLaunchKernelGGL(k_sconv_carry, dim3((a.c_in * a.pad + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sconvtr(const SConvTrArgs& a, hipStream_t s) {
  const uint32_t len = a.t_in * a.stride + a.tl;
  if (a.t_in == 0 || a.c_out == 0 || a.c_out > 65535) return hipErrorInvalidValue;
  if (a.groups == 1) {
    uint32_t oc_t, t_t;
    conv_tile(len, oc_t, t_t);
    const uint32_t xcap = t_t / a.stride + a.k / a.stride + 2;
    const size_t lds = (static_cast<size_t>(kConvIcb) * xcap + static_cast<size_t>(kConvIcb) * oc_t * a.k) * sizeof(float);
    if (lds > 64 * 1024) return hipErrorInvalidValue;
    const dim3 g((len + t_t - 1) / t_t, (a.c_out + oc_t - 1) / oc_t);
    uint32_t ics = a.c_in;
    const uint32_t splits = a.part ? conv_splits(g.x * g.y, a.c_in,
                                                 static_cast<uint64_t>(a.c_out) * len, a.part_cap, &ics)
                                   : 1u;
    SConvTrArgs args = a;
    if (splits <= 1 || static_cast<uint64_t>(g.x) * g.y > a.counter_cap) args.counters = nullptr;
    hipLaunchKernelGGL(k_sconvtr_tiled, dim3(g.x, g.y, splits), dim3(kConvTileThreads), lds, s, args,
                       oc_t, t_t, kConvIcb, ics);
    if (splits > 1 && args.counters == nullptr) {
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(k_sconvtr_sum, dim3((a.c_out * len + 255) / 256), dim3(256), 0, s, a, splits);
    }
  } else {
    hipLaunchKernelGGL(k_sconvtr, dim3((len + 63) / 64, a.c_out), dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace sdec
