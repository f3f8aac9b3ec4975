// Softmax attention in fp32 (forward and backward), plus the backward
// preprocessing kernel (D = rowsum(dO * O)) used by the bf16 path.
//
// The fp32 path keeps every operation in fp32 FMA arithmetic (no reduced
// precision step anywhere), as the fp32 workload asks.  Its intended sizes are
// small and latency-bound, so it uses plain VALU FMA: T = D/32 lanes share one
// row (query or key), each owning 32 of its D columns, and dot products are
// finished with lane exchanges.  Key/value (or query/dO) tiles are staged in
// LDS and read by broadcast.
//
// Definitions follow the softmax attention block O = softmax(scale Q K^T) V
// (the block O = f(A B) C of the "Memory-efficient tensor parallelism"
// abstract; tiling per "Ulysses Sequence Parallelism", "Contexte Technique";
// causal index mask per "AutoSP" 2.A) and its derivative:
//   dP = dO V^T, D_i = sum_j P_ij dP_ij = rowsum(dO * O), dS = P (dP - D),
//   dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO.
// The backward recomputes P from the saved log-sum-exp instead of storing it
// ("AutoSP" 2.B).
#include "fab_device.h"
#include "fab_internal.h"

namespace fab {
namespace {

constexpr int kTile = 32;  // rows of a staged tile

template <int T>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (T >= 2) v += __shfl_xor(v, 1, 64);
  if constexpr (T >= 4) v += __shfl_xor(v, 2, 64);
  return v;
}

// Stage rows [r0, r0 + kTile) of a [rows, D] fp32 matrix (row stride sr) into
// LDS (packed rows of D floats); rows >= nrows are zero.
template <int D>
__device__ __forceinline__ void stage_f32(float* dst, const float* src, int64_t sr, int r0,
                                          int nrows, int tid, int nthreads) {
  constexpr int V4 = D / 4;
  for (int i = tid; i < kTile * V4; i += nthreads) {
    const int r = i / V4, c = i % V4;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (r0 + r < nrows) v = *reinterpret_cast<const f32x4*>(src + (int64_t)(r0 + r) * sr + 4 * c);
    *reinterpret_cast<f32x4*>(dst + r * D + 4 * c) = v;
  }
}

// ---------------------------------------------------------------------------
// forward: one row group of T lanes per query, 256 threads = 256/T queries
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(AttnArgs a) {
  constexpr int T = D / 32, QPB = 256 / T;
  __shared__ float ks[kTile * D];
  __shared__ float vs[kTile * D];
  const int tid = threadIdx.x;
  const int part = tid % T;
  const int nqb = (a.m + QPB - 1) / QPB;
  int id = blockIdx.x;
  const int h = id % a.hq;
  id /= a.hq;
  const int bi = id % a.b;
  id /= a.b;
  const int qb = CAUSAL ? nqb - 1 - id : id;
  const int g = h / a.group;
  const int q = qb * QPB + tid / T;
  const float* qbase = static_cast<const float*>(a.q) + bi * a.q_sb + h * a.q_sh;
  const float* kbase = static_cast<const float*>(a.k) + bi * a.k_sb + g * a.k_sh;
  const float* vbase = static_cast<const float*>(a.v) + bi * a.v_sb + g * a.v_sh;

  float qr[32], o[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    qr[i] = q < a.m ? qbase[(int64_t)q * a.q_sr + part * 32 + i] : 0.f;
    o[i] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  const float cs = a.scale_log2;
  const int kend = CAUSAL ? min(a.n, max(0, qb * QPB + QPB + a.diag)) : a.n;
  for (int k0 = 0; k0 < kend; k0 += kTile) {
    __syncthreads();
    stage_f32<D>(ks, kbase, a.k_sr, k0, a.n, tid, 256);
    stage_f32<D>(vs, vbase, a.v_sr, k0, a.n, tid, 256);
    __syncthreads();
    float s[kTile];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) acc = fmaf(qr[i], ks[j * D + part * 32 + i], acc);
      acc = group_sum<T>(acc);
      const int key = k0 + j;
      const bool dead = key >= a.n || (CAUSAL && key > q + a.diag);
      s[j] = dead ? -INFINITY : acc * cs;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) o[i] *= alpha;
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      const float p = s[j] == -INFINITY ? 0.f : exp2f(s[j] - m_new);
      lsum += p;
#pragma unroll
      for (int i = 0; i < 32; ++i) o[i] = fmaf(p, vs[j * D + part * 32 + i], o[i]);
    }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
  }
  if (q >= a.m) return;
  // a row that saw no key (offset causal masks): O = 0, LSE = -inf
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  float* orow = static_cast<float*>(a.o_out) + bi * a.o_sb + h * a.o_sh + (int64_t)q * a.o_sr +
                part * 32;
#pragma unroll
  for (int i = 0; i < 32; i += 4) {
    f32x4 v = {o[i] * inv, o[i + 1] * inv, o[i + 2] * inv, o[i + 3] * inv};
    *reinterpret_cast<f32x4*>(orow + i) = v;
  }
  if (part == 0)
    a.lse[((int64_t)bi * a.hq + h) * a.m + q] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// dQ: one row group per query, loop over keys
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_dq_f32_kernel(AttnArgs a) {
  constexpr int T = D / 32, QPB = 256 / T;
  __shared__ float ks[kTile * D];
  __shared__ float vs[kTile * D];
  const int tid = threadIdx.x;
  const int part = tid % T;
  const int nqb = (a.m + QPB - 1) / QPB;
  int id = blockIdx.x;
  const int h = id % a.hq;
  id /= a.hq;
  const int bi = id % a.b;
  id /= a.b;
  const int qb = CAUSAL ? nqb - 1 - id : id;
  const int g = h / a.group;
  const int q = qb * QPB + tid / T;
  const int64_t qoff = bi * a.q_sb + h * a.q_sh + (int64_t)q * a.q_sr + part * 32;
  const int64_t ooff = bi * a.o_sb + h * a.o_sh + (int64_t)q * a.o_sr + part * 32;
  const float* kbase = static_cast<const float*>(a.k) + bi * a.k_sb + g * a.k_sh;
  const float* vbase = static_cast<const float*>(a.v) + bi * a.v_sb + g * a.v_sh;
  float qr[32], dor[32], dq[32];
  const bool live = q < a.m;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    qr[i] = live ? static_cast<const float*>(a.q)[qoff + i] : 0.f;
    dor[i] = live ? static_cast<const float*>(a.dout)[ooff + i] : 0.f;
    dq[i] = 0.f;
  }
  const int64_t ridx = ((int64_t)bi * a.hq + h) * a.m + q;
  const float lse2 = live ? a.lse_in[ridx] * kLog2e : 0.f;
  // D = rowsum(dO * O), accumulated in the same lane split and order as the
  // dP dot products below, so that a row whose exact dS vanishes (a query that
  // sees a single key) gets dP - D = 0 exactly.  Written for the dK/dV kernel.
  float dlt = 0.f;
  {
    const float* orow = static_cast<const float*>(a.o) + ooff;
#pragma unroll
    for (int i = 0; i < 32; ++i) dlt = fmaf(dor[i], live ? orow[i] : 0.f, dlt);
    dlt = group_sum<T>(dlt);
    if (live && part == 0) a.delta[ridx] = dlt;
  }
  const float cs = a.scale_log2;
  const int kend = CAUSAL ? min(a.n, max(0, qb * QPB + QPB + a.diag)) : a.n;
  for (int k0 = 0; k0 < kend; k0 += kTile) {
    __syncthreads();
    stage_f32<D>(ks, kbase, a.k_sr, k0, a.n, tid, 256);
    stage_f32<D>(vs, vbase, a.v_sr, k0, a.n, tid, 256);
    __syncthreads();
#pragma unroll 4
    for (int j = 0; j < kTile; ++j) {
      float sacc = 0.f, dpacc = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        sacc = fmaf(qr[i], ks[j * D + part * 32 + i], sacc);
        dpacc = fmaf(dor[i], vs[j * D + part * 32 + i], dpacc);
      }
      sacc = group_sum<T>(sacc);
      dpacc = group_sum<T>(dpacc);
      const int key = k0 + j;
      const bool dead = !live || key >= a.n || (CAUSAL && key > q + a.diag);
      const float p = dead ? 0.f : exp2f(sacc * cs - lse2);
      const float ds = p * (dpacc - dlt);
#pragma unroll
      for (int i = 0; i < 32; ++i) dq[i] = fmaf(ds, ks[j * D + part * 32 + i], dq[i]);
    }
  }
  if (!live) return;
  float* out = static_cast<float*>(a.dq) + qoff;
#pragma unroll
  for (int i = 0; i < 32; i += 4) {
    f32x4 v = {dq[i] * a.scale, dq[i + 1] * a.scale, dq[i + 2] * a.scale, dq[i + 3] * a.scale};
    *reinterpret_cast<f32x4*>(out + i) = v;
  }
}

// ---------------------------------------------------------------------------
// dK, dV: one row group per key, loop over the group's query heads and rows
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_dkdv_f32_kernel(AttnArgs a) {
  constexpr int T = D / 32, KPB = 256 / T;
  __shared__ float qs[kTile * D];
  __shared__ float dos[kTile * D];
  __shared__ float lses[kTile];
  __shared__ float dls[kTile];
  const int tid = threadIdx.x;
  const int part = tid % T;
  const int nkb = (a.n + KPB - 1) / KPB;
  int id = blockIdx.x;
  const int g = id % a.hkv;
  id /= a.hkv;
  const int bi = id % a.b;
  id /= a.b;
  const int kblk = CAUSAL ? id : nkb - 1 - id;  // causal: early keys see most queries
  const int key = kblk * KPB + tid / T;
  const bool live = key < a.n;
  const int64_t koff = bi * a.k_sb + g * a.k_sh + (int64_t)key * a.k_sr + part * 32;
  const int64_t voff = bi * a.v_sb + g * a.v_sh + (int64_t)key * a.v_sr + part * 32;
  float kr[32], vr[32], dk[32], dv[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    kr[i] = live ? static_cast<const float*>(a.k)[koff + i] : 0.f;
    vr[i] = live ? static_cast<const float*>(a.v)[voff + i] : 0.f;
    dk[i] = 0.f;
    dv[i] = 0.f;
  }
  const float cs = a.scale_log2;
  // first query tile holding a query that sees the block's first key
  const int qstart = CAUSAL ? (max(0, kblk * KPB - a.diag) / kTile) * kTile : 0;
  for (int hh = 0; hh < a.group; ++hh) {
    const int h = g * a.group + hh;
    const float* qbase = static_cast<const float*>(a.q) + bi * a.q_sb + h * a.q_sh;
    const float* dobase = static_cast<const float*>(a.dout) + bi * a.o_sb + h * a.o_sh;
    const int64_t rbase = ((int64_t)bi * a.hq + h) * a.m;
    for (int q0 = qstart; q0 < a.m; q0 += kTile) {
      __syncthreads();
      stage_f32<D>(qs, qbase, a.q_sr, q0, a.m, tid, 256);
      stage_f32<D>(dos, dobase, a.o_sr, q0, a.m, tid, 256);
      if (tid < kTile) {
        const bool ok = q0 + tid < a.m;
        lses[tid] = ok ? a.lse_in[rbase + q0 + tid] * kLog2e : 0.f;
        dls[tid] = ok ? a.delta[rbase + q0 + tid] : 0.f;
      }
      __syncthreads();
#pragma unroll 4
      for (int j = 0; j < kTile; ++j) {
        float sacc = 0.f, dpacc = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          sacc = fmaf(kr[i], qs[j * D + part * 32 + i], sacc);
          dpacc = fmaf(vr[i], dos[j * D + part * 32 + i], dpacc);
        }
        sacc = group_sum<T>(sacc);
        dpacc = group_sum<T>(dpacc);
        const int qi = q0 + j;
        const bool dead = !live || qi >= a.m || (CAUSAL && key > qi + a.diag);
        const float p = dead ? 0.f : exp2f(sacc * cs - lses[j]);
        const float ds = p * (dpacc - dls[j]);
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          dv[i] = fmaf(p, dos[j * D + part * 32 + i], dv[i]);
          dk[i] = fmaf(ds, qs[j * D + part * 32 + i], dk[i]);
        }
      }
    }
  }
  if (!live) return;
  float* dko = static_cast<float*>(a.dk) + koff;
  float* dvo = static_cast<float*>(a.dv) + voff;
#pragma unroll
  for (int i = 0; i < 32; i += 4) {
    f32x4 x = {dk[i] * a.scale, dk[i + 1] * a.scale, dk[i + 2] * a.scale, dk[i + 3] * a.scale};
    f32x4 y = {dv[i], dv[i + 1], dv[i + 2], dv[i + 3]};
    *reinterpret_cast<f32x4*>(dko + i) = x;
    *reinterpret_cast<f32x4*>(dvo + i) = y;
  }
}

template <int D>
hipError_t fwd_d(const AttnArgs& a, hipStream_t s) {
  constexpr int QPB = 256 / (D / 32);
  const dim3 grid((unsigned)((a.m + QPB - 1) / QPB) * a.hq * a.b), block(256);
  if (a.causal)
    FAB_TIMED("attn_fwd_f32", s, hipLaunchKernelGGL((attn_fwd_f32_kernel<D, true>), grid, block, 0, s, a));
  else
    FAB_TIMED("attn_fwd_f32", s, hipLaunchKernelGGL((attn_fwd_f32_kernel<D, false>), grid, block, 0, s, a));
  return hipGetLastError();
}

template <int D>
hipError_t bwd_d(const AttnArgs& a, hipStream_t s) {
  constexpr int T = D / 32, RPB = 256 / T;
  const dim3 block(256);
  const dim3 gq((unsigned)((a.m + RPB - 1) / RPB) * a.hq * a.b);
  const dim3 gk((unsigned)((a.n + RPB - 1) / RPB) * a.hkv * a.b);
  if (a.causal) {
    FAB_TIMED("attn_bwd_dq_f32", s, hipLaunchKernelGGL((attn_dq_f32_kernel<D, true>), gq, block, 0, s, a));
    FAB_TIMED("attn_bwd_dkdv_f32", s, hipLaunchKernelGGL((attn_dkdv_f32_kernel<D, true>), gk, block, 0, s, a));
  } else {
    FAB_TIMED("attn_bwd_dq_f32", s, hipLaunchKernelGGL((attn_dq_f32_kernel<D, false>), gq, block, 0, s, a));
    FAB_TIMED("attn_bwd_dkdv_f32", s, hipLaunchKernelGGL((attn_dkdv_f32_kernel<D, false>), gk, block, 0, s, a));
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_f32(const AttnArgs& a, int d, hipStream_t s) {
  if (d == 128) return fwd_d<128>(a, s);
  if (d == 64) return fwd_d<64>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_bwd_f32(const AttnArgs& a, int d, hipStream_t s) {
  if (d == 128) return bwd_d<128>(a, s);
  if (d == 64) return bwd_d<64>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace fab
