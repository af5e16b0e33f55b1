// Split residual vector quantisation on CDNA4 ([mimi] inferencelayer 0.2.1, src/mimi_gpu.rs:
// NEAREST, SUB_EMB, EMB_SUM and MimiGpu's encode / decode plans).
//
// A code is an integer decided by float32 arithmetic, so the distance is computed exactly as the
// pages define it: one lane per bin sums (cb - r)^2 over the dimensions in ascending order, the
// difference, the square and each partial sum rounded separately (no fused multiply-add), and
// the smallest distance wins with ties going to the lower bin.  Codebooks are read through a
// transposed copy ([level][dim][bin]) so the 64 lanes of a wave (64 consecutive bins) read one
// contiguous 256-byte run per dimension.

#include <hip/hip_runtime.h>

#include "kernels.h"

namespace sdec {

namespace {

constexpr int kRvqLanes = 64;

// (d, bin) order of the first-wins argmin: smaller distance, then lower bin.
__device__ __forceinline__ bool rvq_better(float d, uint32_t i, float bd, uint32_t bi) {
  return d < bd || (d == bd && i < bi);
}

// First-wins argmin over the wave; every lane ends with the winner.
__device__ __forceinline__ void rvq_wave_argmin(float& d, uint32_t& i) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float od = __shfl_xor(d, off, kRvqLanes);
    const uint32_t oi = static_cast<uint32_t>(__shfl_xor(static_cast<int>(i), off, kRvqLanes));
    if (rvq_better(od, oi, d, i)) {
      d = od;
      i = oi;
    }
  }
}

// [levels][bins][vq] -> [levels][vq][bins], 32 x 32 tiles through LDS (the 33-float rows keep
// the column reads free of bank conflicts).  Also the codec frame's channel-major <-> time-major
// layout change (one level).
__global__ __launch_bounds__(256) void k_transpose(const float* src, float* dst, uint32_t bins,
                                                   uint32_t vq) {
  __shared__ float tile[32][33];
  const uint32_t l = blockIdx.z;
  const uint32_t b0 = blockIdx.x * 32, c0 = blockIdx.y * 32;
  const float* s = src + static_cast<size_t>(l) * bins * vq;
  float* d = dst + static_cast<size_t>(l) * bins * vq;
  for (uint32_t y = threadIdx.y; y < 32; y += 8) {
    const uint32_t b = b0 + y, c = c0 + threadIdx.x;
    if (b < bins && c < vq) tile[y][threadIdx.x] = s[static_cast<size_t>(b) * vq + c];
  }
  __syncthreads();
  for (uint32_t y = threadIdx.y; y < 32; y += 8) {
    const uint32_t c = c0 + y, b = b0 + threadIdx.x;
    if (b < bins && c < vq) d[static_cast<size_t>(c) * bins + b] = tile[threadIdx.x][y];
  }
}

// One quantiser level for every frame: grid (bins / 64, frames), one wave per 64 bins.
__global__ __launch_bounds__(kRvqLanes) void k_rvq_level(RvqLevelArgs a) {
  __shared__ float r[kRvqMaxVq];
  const uint32_t f = blockIdx.y, wg = blockIdx.x;
  const int lane = threadIdx.x;
  const float* rin = a.r_in + static_cast<size_t>(f) * a.r_stride;
  if (a.prev_cand_d != nullptr) {
    // the previous level's code, from its per-wave candidates (the same first-wins order)
    float d = INFINITY;
    uint32_t i = 0xFFFFFFFFu;
    for (uint32_t g = lane; g < a.groups; g += kRvqLanes) {
      const float cd = a.prev_cand_d[static_cast<size_t>(f) * a.groups + g];
      const uint32_t ci = a.prev_cand_i[static_cast<size_t>(f) * a.groups + g];
      if (rvq_better(cd, ci, d, i)) {
        d = cd;
        i = ci;
      }
    }
    rvq_wave_argmin(d, i);
    const uint32_t code = i;
    if (wg == 0 && lane == 0) a.codes[static_cast<size_t>(f) * a.nq + a.prev_level] = code;
    if (a.prev_cb != nullptr) {  // SUB_EMB: the running residual loses the chosen code vector
      const float* e = a.prev_cb + static_cast<size_t>(code) * a.vq;
      for (uint32_t c = lane; c < a.vq; c += kRvqLanes) {
        const float v = rin[c] - e[c];
        r[c] = v;
        if (wg == 0) a.r_out[static_cast<size_t>(f) * a.vq + c] = v;
      }
    } else {
      for (uint32_t c = lane; c < a.vq; c += kRvqLanes) {
        r[c] = rin[c];
        if (wg == 0 && a.r_out != nullptr) a.r_out[static_cast<size_t>(f) * a.vq + c] = rin[c];
      }
    }
  } else {
    for (uint32_t c = lane; c < a.vq; c += kRvqLanes) {
      r[c] = rin[c];
      if (wg == 0 && a.r_out != nullptr) a.r_out[static_cast<size_t>(f) * a.vq + c] = rin[c];
    }
  }
  __syncthreads();
  const uint32_t b = wg * kRvqLanes + lane;  // bins is a multiple of 64
  const float* col = a.cbT + b;
  float d = 0.f;
  {
#pragma clang fp contract(off)
    // 16 codebook words requested per round trip (the sum itself stays in dimension order)
#pragma unroll 16
    for (uint32_t c = 0; c < a.vq; ++c) {
      const float df = col[static_cast<size_t>(c) * a.bins] - r[c];
      const float sq = df * df;  // rounded on its own: no fused multiply-add
      d = d + sq;
    }
  }
  uint32_t i = b;
  rvq_wave_argmin(d, i);
  if (lane == 0) {
    a.cand_d[static_cast<size_t>(f) * a.groups + wg] = d;
    a.cand_i[static_cast<size_t>(f) * a.groups + wg] = i;
  }
}

// The last level's code from its candidates; grid (frames), one wave.
__global__ __launch_bounds__(kRvqLanes) void k_rvq_final(RvqLevelArgs a) {
  const uint32_t f = blockIdx.x;
  const int lane = threadIdx.x;
  float d = INFINITY;
  uint32_t i = 0xFFFFFFFFu;
  for (uint32_t g = lane; g < a.groups; g += kRvqLanes) {
    const float cd = a.prev_cand_d[static_cast<size_t>(f) * a.groups + g];
    const uint32_t ci = a.prev_cand_i[static_cast<size_t>(f) * a.groups + g];
    if (rvq_better(cd, ci, d, i)) {
      d = cd;
      i = ci;
    }
  }
  rvq_wave_argmin(d, i);
  if (lane == 0) a.codes[static_cast<size_t>(f) * a.nq + a.prev_level] = i;
}

// EMB_SUM for both groups: acc_first = cb_first[code0], acc_rest = sum over rest levels in order;
// grid (frames), 256 threads over the vq dimensions.  Codes past the codebook read its last bin.
__global__ __launch_bounds__(256) void k_rvq_emb_sum(RvqEmbArgs a) {
  const uint32_t f = blockIdx.x;
  const uint32_t* codes = a.codes + static_cast<size_t>(f) * a.nq;
  for (uint32_t c = threadIdx.x; c < a.vq; c += 256) {
    const uint32_t c0 = min(codes[0], a.bins - 1);
    a.acc[static_cast<size_t>(f) * 2 * a.vq + c] = a.cb_first[static_cast<size_t>(c0) * a.vq + c];
    float s = 0.f;
    for (uint32_t l = 1; l < a.nq; ++l) {
      const uint32_t cl = min(codes[l], a.bins - 1);
      s = s + a.cb_rest[(static_cast<size_t>(l - 1) * a.bins + cl) * a.vq + c];
    }
    a.acc[static_cast<size_t>(f) * 2 * a.vq + a.vq + c] = s;
  }
}

}  // namespace

hipError_t launch_transpose(const float* src, float* dst, uint32_t levels, uint32_t bins,
                            uint32_t vq, hipStream_t s) {
  hipLaunchKernelGGL(k_transpose, dim3((bins + 31) / 32, (vq + 31) / 32, levels), dim3(32, 8),
                     0, s, src, dst, bins, vq);
  return hipGetLastError();
}

hipError_t launch_rvq_level(const RvqLevelArgs& a, uint32_t frames, hipStream_t s) {
  if (a.vq > static_cast<uint32_t>(kRvqMaxVq) || a.bins % kRvqLanes != 0 ||
      a.groups != a.bins / kRvqLanes || frames == 0)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_rvq_level, dim3(a.groups, frames), dim3(kRvqLanes), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rvq_final(const RvqLevelArgs& a, uint32_t frames, hipStream_t s) {
  if (frames == 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_rvq_final, dim3(frames), dim3(kRvqLanes), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rvq_emb_sum(const RvqEmbArgs& a, uint32_t frames, hipStream_t s) {
  if (frames == 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_rvq_emb_sum, dim3(frames), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace sdec
