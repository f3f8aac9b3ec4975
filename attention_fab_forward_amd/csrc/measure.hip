// Rate probe of the softmax's per-element transcendental work, a secondary
// bound of the attention kernels next to the MFMA rate: every lane runs kChains
// independent chains of exp2(fma(x, a, b)) (the form each probability takes:
// the scale folded into the exponent), so issue rate, not latency, bounds the
// run.  Only measurement uses it.
#include "fab_device.h"
#include "fab_internal.h"

namespace fab {
namespace {

constexpr int kChains = 8;

__global__ __launch_bounds__(256) void exp_rate_kernel(int iters, float* sink) {
  float x[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) x[c] = 0.25f + 0.03125f * c + 1e-6f * (threadIdx.x & 7);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) x[c] = fast_exp2(fmaf(x[c], -1.f, -0.5f));  // stays in (0, 1)
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += x[c];
  sink[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

int exp_probe_chains() { return kChains; }

hipError_t launch_exp_probe(int blocks, int iters, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(exp_rate_kernel, dim3((unsigned)blocks), dim3(256), 0, s, iters, sink);
  return hipGetLastError();
}

}  // namespace fab
