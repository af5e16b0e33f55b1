// Streaming codec convolutions on CDNA4 ([mimi] inferencelayer 0.2.1, src/mimi_gpu.rs: CONV1D with
// the carried input prefix of WRITE_XA / CARRY / REPLICATE, the gather-form transposed conv of
// convtr_src with its overlap tail carried bias-subtracted by TRP_ADD / TR_OUT / TR_CARRY, and
// the ELU of ELU_IP folded into the reads).  Frames arrive one at a time; the state between them
// is the last K - S input columns of a conv and the K - S pending output columns of a transposed
// conv, kept in ping-pong buffers so no kernel reads what another thread of it rewrites.

#include <hip/hip_runtime.h>
#include <math.h>

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
  for (uint32_t k = 0; k < a.k && k <= i; ++k) {
    const uint32_t d = i - k;
    if (d % a.stride != 0) continue;
    const uint32_t ti = d / a.stride;
    if (ti >= a.t_in) continue;
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

}  // namespace

hipError_t launch_sconv(const SConvArgs& a, hipStream_t s) {
  const uint32_t t_out = a.t_in / a.stride;
  if (t_out == 0 || a.c_out == 0 || a.c_out > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_sconv, dim3((t_out + 63) / 64, a.c_out), dim3(64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.pad == 0) return e;
  hipLaunchKernelGGL(k_sconv_carry, dim3((a.c_in * a.pad + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sconvtr(const SConvTrArgs& a, hipStream_t s) {
  const uint32_t len = a.t_in * a.stride + a.tl;
  if (a.t_in == 0 || a.c_out == 0 || a.c_out > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_sconvtr, dim3((len + 63) / 64, a.c_out), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace sdec
