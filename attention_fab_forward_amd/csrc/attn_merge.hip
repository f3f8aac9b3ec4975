// Merge of two softmax attention results over disjoint key sets of the same
// queries: LSE = log(e^LSE_a + e^LSE_b), O = w_a O_a + w_b O_b with
// w_x = e^(LSE_x - LSE).  This is the result over the union of the key sets,
// the step that combines key-range shards (ring / key-sharded attention:
// "Ulysses Sequence Parallelism", Analyse; FITEE abstract, B and C exchanged
// in sub-blocks) or the splits of a split-key launch.  Memory bound: one
// pass over O_a, O_b and the two LSE vectors.
#include "fab_device.h"
#include "fab_internal.h"

namespace fab {
namespace {

// One query row (b, i, h) per LPR lanes, each lane 16 bytes of the row; rows
// are taken in O's [b, m, hq] order, so for the packed layout a workgroup
// streams one contiguous stretch of O (the LSE reads, 4 bytes per row, are
// the scattered ones).  The lanes of a row sit in one wave, so an in-place
// merge (O_out = O_a, lse_out = lse_a) reads every input before any lane
// writes.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeArgs a) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int EPL = 16 / ES;  // elements per lane
  constexpr int LPR = D / EPL;
  constexpr int RPB = 256 / LPR;
  static_assert(64 % LPR == 0, "a row's lanes must share a wave");
  const int tid = threadIdx.x;
  const int64_t orow = (int64_t)blockIdx.x * RPB + tid / LPR;  // O order [b, m, hq]
  const int part = tid % LPR;
  const int64_t total = (int64_t)a.b * a.hq * a.m;
  if (orow >= total) return;
  int64_t i, h, bi;
  if (a.small) {  // every index below 2^31: division by multiplication
    const uint32_t r32 = (uint32_t)orow;
    const uint32_t bm = (__umulhi(r32, a.div_hq.m) + r32) >> a.div_hq.s;
    h = r32 - bm * (uint32_t)a.hq;
    bi = (__umulhi(bm, a.div_m.m) + bm) >> a.div_m.s;
    i = bm - (uint32_t)bi * (uint32_t)a.m;
  } else {
    const int64_t bm = orow / a.hq;
    h = orow - bm * a.hq;
    bi = bm / a.m;
    i = bm - bi * a.m;
  }
  const int64_t row = (bi * a.hq + h) * a.m + i;  // LSE order [b, hq, m]
  const float la = a.la[row], lb = a.lb[row];
  const float mx = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f, lse = -INFINITY;
  if (mx != -INFINITY) {
    // base-2 hardware exponential and logarithm and one reciprocal (each
    // within a few ulp, far inside the bf16 rounding of O and the fp32 LSE
    // bound; the library functions' range handling cost 3 % of the kernel)
    const float ea = fast_exp2((la - mx) * kLog2e), eb = fast_exp2((lb - mx) * kLog2e);
    const float sum = ea + eb;
    const float inv = __builtin_amdgcn_rcpf(sum);
    wa = ea * inv;
    wb = eb * inv;
    lse = mx + __builtin_amdgcn_logf(sum) * kLn2;
  }
  const int64_t off = bi * a.o_sb + h * a.o_sh + i * a.o_sr + part * EPL;
  if constexpr (BF16) {
    const u32x4 x = ldg16(static_cast<const uint16_t*>(a.oa) + off);
    const u32x4 y = ldg16(static_cast<const uint16_t*>(a.ob) + off);
    u32x4 r;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      r[w] = pack_bf16(wa * bf16_lo(x[w]) + wb * bf16_lo(y[w]), wa * bf16_hi(x[w]) + wb * bf16_hi(y[w]));
    stg16(static_cast<uint16_t*>(a.oo) + off, r);
  } else {
    const f32x4 x = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.oa) + off);
    const f32x4 y = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.ob) + off);
    f32x4 r;
#pragma unroll
    for (int w = 0; w < 4; ++w) r[w] = wa * x[w] + wb * y[w];
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.oo) + off) = r;
  }
  if (part == 0) a.lo[row] = lse;
}

template <int D, bool BF16>
hipError_t merge_d(const MergeArgs& a, hipStream_t s) {
  constexpr int RPB = 256 / (D * (BF16 ? 2 : 4) / 16);
  const int64_t rows = (int64_t)a.b * a.hq * a.m;
  const dim3 grid((unsigned)((rows + RPB - 1) / RPB)), block(256);
  FAB_TIMED("attn_merge", s, hipLaunchKernelGGL((attn_merge_kernel<D, BF16>), grid, block, 0, s, a));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_merge(const MergeArgs& a, int d, bool bf16, hipStream_t s) {
  if (d == 128) return bf16 ? merge_d<128, true>(a, s) : merge_d<128, false>(a, s);
  if (d == 64) return bf16 ? merge_d<64, true>(a, s) : merge_d<64, false>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace fab
