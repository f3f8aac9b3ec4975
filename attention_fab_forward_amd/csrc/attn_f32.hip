// Softmax attention in fp32: one forward kernel and one backward launch (dQ
// and dK/dV workgroups side by side).
//
// The fp32 path keeps every operation in fp32 FMA arithmetic (no reduced
// precision step anywhere), as the fp32 workload asks.  Its intended sizes are
// small and latency-bound, so it uses plain VALU FMA: T = D/8 lanes share one
// row (query or key), each owning 8 of its D columns, and dot products are
// finished with lane exchanges.  Key/value (or query/dO) rows are staged in
// LDS and read by broadcast; the loop over them is split across the waves of
// a workgroup (see below), which keeps the serial chain per lane short.
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

// Lane layout: T = D / kCols lanes share one row (query, or key in the dK/dV
// kernel), each owning kCols (= KC) of its D columns; a wave holds RW = 64 / T rows and
// a workgroup is one wave-width of rows served by NW waves.  The loop over the
// other side (keys, or queries) runs in stages of SUP = NW * KS rows staged
// in LDS by the whole workgroup (KS = 32 at d = 64, 16 at d = 128: a stage
// fills about 130 KiB); wave w takes rows w KS .. w KS + KS - 1 of each
// stage, so the serial work per lane is 1 / NW of the loop.  The waves'
// partial results are combined through LDS at the end (softmax states merged
// by their maxima, gradients summed).
// KC, the columns of a row per lane, is 8, or 4 at d = 64 for launches that
// would otherwise leave CUs idle (twice the workgroups, each with half the
// rows; 16 lanes a row either way: 32 would need an exchange across DPP rows).
constexpr int kCUs = 256;
constexpr int kWaves = 8;   // NW

// Rows of a stage per wave (KS) and per workgroup (SUP).
template <int D>
struct F32Stage {
  static constexpr int SLICE = D == 64 ? 32 : 16;
  static constexpr int ROWS = kWaves * SLICE;
};

// Stage rows [r0, r0 + SUP) of two [rows, D] fp32 matrices (row strides sx,
// sy) into LDS as packed rows of D floats; rows >= nrows are zero.  Each
// thread issues all its global loads before its first LDS store, so a stage
// pays the global latency about once instead of once per 16-byte piece.
template <int D>
__device__ __forceinline__ void stage2_f32(float* dx, const float* x, int64_t sx, float* dy,
                                           const float* y, int64_t sy, int r0, int nrows, int tid) {
  constexpr int V4 = D / 4, kStage = F32Stage<D>::ROWS;
  constexpr int N = kStage * V4 / (64 * kWaves);  // pieces per thread and matrix
  static_assert(N * 64 * kWaves == kStage * V4, "a stage splits evenly over the threads");
  f32x4 vx[N], vy[N];
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const int i = tid + u * 64 * kWaves;
    const int r = i / V4, c = i % V4;
    const bool live = r0 + r < nrows;
    vx[u] = live ? *reinterpret_cast<const f32x4*>(x + (int64_t)(r0 + r) * sx + 4 * c)
                 : f32x4{0.f, 0.f, 0.f, 0.f};
    vy[u] = live ? *reinterpret_cast<const f32x4*>(y + (int64_t)(r0 + r) * sy + 4 * c)
                 : f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const int i = tid + u * 64 * kWaves;
    const int r = i / V4, c = i % V4;
    *reinterpret_cast<f32x4*>(dx + r * D + 4 * c) = vx[u];
    *reinterpret_cast<f32x4*>(dy + r * D + 4 * c) = vy[u];
  }
}

// LDS floats: a stage of two [kStage, D] matrices (+ two kStage vectors), or
// the cross-wave combination area (NW x RW x D partial rows + 2 NW RW scalars).
template <int D, int KC>
struct F32Lds {
  static constexpr int T = D / KC;
  static constexpr int RW = 64 / T;
  static constexpr int CHUNKS = RW * D / 4;  // float4 chunks of an RW x D block
  static constexpr int STAGE = 2 * F32Stage<D>::ROWS * D + 2 * F32Stage<D>::ROWS;
  static constexpr int PART = kWaves * RW * D;
  static constexpr int FLOATS = STAGE > PART + 2 * kWaves * RW ? STAGE : PART + 2 * kWaves * RW;
};

// Sum of the NW waves' partial rows part[w][r][:] (r < RW) for float4 chunk
// `tid` (< CHUNKS) of the RW x D block: returns the chunk, row r = tid / (D / 4).
template <int D, int KC>
__device__ __forceinline__ f32x4 sum_parts(const float* part, int tid) {
  constexpr int RW = F32Lds<D, KC>::RW;
  const int r = tid / (D / 4), c = tid % (D / 4);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < kWaves; ++w) acc += *reinterpret_cast<const f32x4*>(part + (w * RW + r) * D + 4 * c);
  return acc;
}

// Writes this lane's NC partial columns of row `row` (0..RW-1) for wave w.
template <int NC>
__device__ __forceinline__ void put_part(float* part, int D, int RW, int w, int row, int col0,
                                         const float (&x)[NC]) {
  static_assert(NC % 4 == 0, "columns are written as whole float4 chunks");
  float* dst = part + (w * RW + row) * D + col0;
#pragma unroll
  for (int i = 0; i < NC; i += 4)
    *reinterpret_cast<f32x4*>(dst + i) = f32x4{x[i], x[i + 1], x[i + 2], x[i + 3]};
}

// ---------------------------------------------------------------------------
// forward: workgroup = RW queries of one head, keys split over the waves
// ---------------------------------------------------------------------------
template <int D, int KC, bool CAUSAL>
__global__ __launch_bounds__(64 * kWaves) void attn_fwd_f32_kernel(AttnArgs a) {
  constexpr int kCols = KC;
  constexpr int T = F32Lds<D, KC>::T, RW = F32Lds<D, KC>::RW;
  constexpr int kSlice = F32Stage<D>::SLICE, kStage = F32Stage<D>::ROWS;
  static_assert(F32Lds<D, KC>::CHUNKS <= 64 * kWaves, "one float4 of the output block per thread");
  __shared__ __attribute__((aligned(16))) float sm[F32Lds<D, KC>::FLOATS];
  float* ks = sm;
  float* vs = sm + kStage * D;
  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, part = lane % T;
  const int nqb = (a.m + RW - 1) / RW;
  int id = blockIdx.x;
  const int h = id % a.hq;
  id /= a.hq;
  const int bi = id % a.b;
  id /= a.b;
  const int qb = CAUSAL ? nqb - 1 - id : id;  // causal: longest blocks first
  const int g = h / a.group;
  const int q = qb * RW + lane / T;
  const float* qbase = static_cast<const float*>(a.q) + bi * a.q_sb + h * a.q_sh;
  const float* kbase = static_cast<const float*>(a.k) + bi * a.k_sb + g * a.k_sh;
  const float* vbase = static_cast<const float*>(a.v) + bi * a.v_sb + g * a.v_sh;

  float qr[kCols], o[kCols];
#pragma unroll
  for (int i = 0; i < kCols; ++i) {
    qr[i] = q < a.m ? qbase[(int64_t)q * a.q_sr + part * kCols + i] : 0.f;
    o[i] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;  // scores in scale * log2(e) units
  const float cs = a.scale_log2;
  const int kend = CAUSAL ? min(a.n, max(0, qb * RW + RW + a.diag)) : a.n;
  for (int k0 = 0; k0 < kend; k0 += kStage) {
    __syncthreads();
    stage2_f32<D>(ks, kbase, a.k_sr, vs, vbase, a.v_sr, k0, a.n, tid);
    __syncthreads();
    const int kw = k0 + wave * kSlice;
    if (kw >= kend) continue;  // wave-uniform
    const float* kt = ks + wave * kSlice * D + part * kCols;
    const float* vt = vs + wave * kSlice * D + part * kCols;
    float s[kSlice];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kSlice; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < kCols; ++i) acc = fmaf(qr[i], kt[j * D + i], acc);
      acc = lane_group_sum<T>(acc);
      const int key = kw + j;
      const bool dead = key >= a.n || (CAUSAL && key > q + a.diag);
      s[j] = dead ? -INFINITY : acc * cs;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < kCols; ++i) o[i] *= alpha;
#pragma unroll
    for (int j = 0; j < kSlice; ++j) {
      const float p = s[j] == -INFINITY ? 0.f : fast_exp2(s[j] - m_new);
      lsum += p;
#pragma unroll
      for (int i = 0; i < kCols; ++i) o[i] = fmaf(p, vt[j * D + i], o[i]);
    }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
  }

  // merge the waves' states: M = max_w m_w, L = sum_w l_w 2^(m_w - M),
  // O = sum_w o_w 2^(m_w - M) / L
  __syncthreads();
  float* po = sm;
  float* pm = sm + F32Lds<D, KC>::PART;
  float* pl = pm + kWaves * RW;
  put_part(po, D, RW, wave, lane / T, part * kCols, o);
  if (part == 0) {
    pm[wave * RW + lane / T] = m_run;
    pl[wave * RW + lane / T] = l_run;
  }
  __syncthreads();
  const int r = tid / (D / 4), c = tid % (D / 4);
  const int qo = qb * RW + r;
  if (tid >= F32Lds<D, KC>::CHUNKS || qo >= a.m) return;
  float mm = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, pm[w * RW + r]);
  float ll = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (mm != -INFINITY) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float e = fast_exp2(pm[w * RW + r] - mm);  // 0 for a wave that saw no key
      ll = fmaf(pl[w * RW + r], e, ll);
      acc += e * *reinterpret_cast<const f32x4*>(po + (w * RW + r) * D + 4 * c);
    }
  }
  // a row that saw no key (offset causal masks): O = 0, LSE = -inf
  const float inv = ll > 0.f ? 1.f / ll : 0.f;
  float* orow = static_cast<float*>(a.o_out) + bi * a.o_sb + h * a.o_sh + (int64_t)qo * a.o_sr;
  *reinterpret_cast<f32x4*>(orow + 4 * c) = acc * inv;
  if (c == 0)
    a.lse[((int64_t)bi * a.hq + h) * a.m + qo] = ll > 0.f ? (mm + log2f(ll)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// Backward: one launch holds the dQ workgroups and the dK/dV workgroups (they
// are independent), so the two run side by side.
// dQ: workgroup = RW queries of one head, keys split over the waves
// ---------------------------------------------------------------------------
template <int D, int KC, bool CAUSAL>
__device__ __forceinline__ void dq_f32_body(const AttnArgs& a, int id, float* sm) {
  constexpr int kCols = KC;
  constexpr int T = F32Lds<D, KC>::T, RW = F32Lds<D, KC>::RW;
  constexpr int kSlice = F32Stage<D>::SLICE, kStage = F32Stage<D>::ROWS;
  float* ks = sm;
  float* vs = sm + kStage * D;
  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, part = lane % T;
  const int nqb = (a.m + RW - 1) / RW;
  const int h = id % a.hq;
  id /= a.hq;
  const int bi = id % a.b;
  id /= a.b;
  const int qb = CAUSAL ? nqb - 1 - id : id;
  const int g = h / a.group;
  const int q = qb * RW + lane / T;
  const int64_t qoff = bi * a.q_sb + h * a.q_sh + (int64_t)q * a.q_sr + part * kCols;
  const int64_t ooff = bi * a.o_sb + h * a.o_sh + (int64_t)q * a.o_sr + part * kCols;
  const float* kbase = static_cast<const float*>(a.k) + bi * a.k_sb + g * a.k_sh;
  const float* vbase = static_cast<const float*>(a.v) + bi * a.v_sb + g * a.v_sh;
  float qr[kCols], dor[kCols], dq[kCols];
  const bool live = q < a.m;
#pragma unroll
  for (int i = 0; i < kCols; ++i) {
    qr[i] = live ? static_cast<const float*>(a.q)[qoff + i] : 0.f;
    dor[i] = live ? static_cast<const float*>(a.dout)[ooff + i] : 0.f;
    dq[i] = 0.f;
  }
  const int64_t ridx = ((int64_t)bi * a.hq + h) * a.m + q;
  const float lse2 = live ? a.lse_in[ridx] * kLog2e : 0.f;
  // D = rowsum(dO * O), accumulated in the same lane split and order as the
  // dP dot products below, so that a row whose exact dS vanishes (a query that
  // sees a single key) gets dP - D = 0 exactly.  The dK/dV workgroups form the
  // same value the same way.
  float dlt = 0.f;
  {
    const float* orow = static_cast<const float*>(a.o) + ooff;
#pragma unroll
    for (int i = 0; i < kCols; ++i) dlt = fmaf(dor[i], live ? orow[i] : 0.f, dlt);
    dlt = lane_group_sum<T>(dlt);
  }
  const float cs = a.scale_log2;
  const int kend = CAUSAL ? min(a.n, max(0, qb * RW + RW + a.diag)) : a.n;
  for (int k0 = 0; k0 < kend; k0 += kStage) {
    __syncthreads();
    stage2_f32<D>(ks, kbase, a.k_sr, vs, vbase, a.v_sr, k0, a.n, tid);
    __syncthreads();
    const int kw = k0 + wave * kSlice;
    if (kw >= kend) continue;  // wave-uniform
    const float* kt = ks + wave * kSlice * D + part * kCols;
    const float* vt = vs + wave * kSlice * D + part * kCols;
#pragma unroll 4
    for (int j = 0; j < kSlice; ++j) {
      float sacc = 0.f, dpacc = 0.f;
#pragma unroll
      for (int i = 0; i < kCols; ++i) {
        sacc = fmaf(qr[i], kt[j * D + i], sacc);
        dpacc = fmaf(dor[i], vt[j * D + i], dpacc);
      }
      sacc = lane_group_sum<T>(sacc);
      dpacc = lane_group_sum<T>(dpacc);
      const int key = kw + j;
      const bool dead = !live || key >= a.n || (CAUSAL && key > q + a.diag);
      const float p = dead ? 0.f : fast_exp2(sacc * cs - lse2);
      const float ds = p * (dpacc - dlt);
#pragma unroll
      for (int i = 0; i < kCols; ++i) dq[i] = fmaf(ds, kt[j * D + i], dq[i]);
    }
  }
  __syncthreads();
  put_part(sm, D, RW, wave, lane / T, part * kCols, dq);
  __syncthreads();
  const int r = tid / (D / 4), c = tid % (D / 4);
  const int qo = qb * RW + r;
  if (tid >= F32Lds<D, KC>::CHUNKS || qo >= a.m) return;
  const f32x4 x = sum_parts<D, KC>(sm, tid) * a.scale;
  *reinterpret_cast<f32x4*>(static_cast<float*>(a.dq) + bi * a.q_sb + h * a.q_sh +
                            (int64_t)qo * a.q_sr + 4 * c) = x;
}

// ---------------------------------------------------------------------------
// dK, dV: workgroup = RW keys of one kv head; the group's query heads and rows
// split over the waves
// ---------------------------------------------------------------------------
template <int D, int KC, bool CAUSAL>
__device__ __forceinline__ void dkdv_f32_body(const AttnArgs& a, int id, float* sm) {
  constexpr int kCols = KC;
  constexpr int T = F32Lds<D, KC>::T, RW = F32Lds<D, KC>::RW;
  constexpr int kSlice = F32Stage<D>::SLICE, kStage = F32Stage<D>::ROWS;
  float* qs = sm;
  float* dos = sm + kStage * D;
  float* lses = sm + 2 * kStage * D;
  float* dls = lses + kStage;
  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, part = lane % T;
  const int nkb = (a.n + RW - 1) / RW;
  const int g = id % a.hkv;
  id /= a.hkv;
  const int bi = id % a.b;
  id /= a.b;
  const int kblk = CAUSAL ? id : nkb - 1 - id;  // causal: early keys see most queries
  const int key = kblk * RW + lane / T;
  const bool live = key < a.n;
  const int64_t koff = bi * a.k_sb + g * a.k_sh + (int64_t)key * a.k_sr + part * kCols;
  const int64_t voff = bi * a.v_sb + g * a.v_sh + (int64_t)key * a.v_sr + part * kCols;
  float kr[kCols], vr[kCols], dk[kCols], dv[kCols];
#pragma unroll
  for (int i = 0; i < kCols; ++i) {
    kr[i] = live ? static_cast<const float*>(a.k)[koff + i] : 0.f;
    vr[i] = live ? static_cast<const float*>(a.v)[voff + i] : 0.f;
    dk[i] = 0.f;
    dv[i] = 0.f;
  }
  const float cs = a.scale_log2;
  // first query that sees the block's first key
  const int qstart = CAUSAL ? max(0, kblk * RW - a.diag) : 0;
  for (int hh = 0; hh < a.group; ++hh) {
    const int h = g * a.group + hh;
    const float* qbase = static_cast<const float*>(a.q) + bi * a.q_sb + h * a.q_sh;
    const float* dobase = static_cast<const float*>(a.dout) + bi * a.o_sb + h * a.o_sh;
    const float* obase = static_cast<const float*>(a.o) + bi * a.o_sb + h * a.o_sh;
    const int64_t rbase = ((int64_t)bi * a.hq + h) * a.m;
    for (int q0 = qstart; q0 < a.m; q0 += kStage) {
      __syncthreads();
      stage2_f32<D>(qs, qbase, a.q_sr, dos, dobase, a.o_sr, q0, a.m, tid);
      if (tid < kStage) {
        const bool ok = q0 + tid < a.m;
        lses[tid] = ok ? a.lse_in[rbase + q0 + tid] * kLog2e : 0.f;
      }
      __syncthreads();
      // D of the staged rows: T lanes per row, each summing dO * O over its
      // kCols columns in order, then the lane exchange -- the dQ workgroups'
      // split and order, so both get the same value
#pragma unroll
      for (int r0 = 0; r0 < kStage; r0 += 64 * kWaves / T) {
        const int r = r0 + tid / T;
        const bool ok = q0 + r < a.m;
        const float* drow = dos + r * D + part * kCols;
        const float* orow = obase + (int64_t)(q0 + r) * a.o_sr + part * kCols;
        float dl = 0.f;
#pragma unroll
        for (int i = 0; i < kCols; ++i) dl = fmaf(drow[i], ok ? orow[i] : 0.f, dl);
        dl = lane_group_sum<T>(dl);
        if (part == 0) dls[r] = dl;
      }
      __syncthreads();
      const int qw = q0 + wave * kSlice;
      if (qw >= a.m) continue;  // wave-uniform
      const float* qt = qs + wave * kSlice * D + part * kCols;
      const float* dt = dos + wave * kSlice * D + part * kCols;
#pragma unroll 1
      for (int j = 0; j < kSlice; ++j) {
        float sacc = 0.f, dpacc = 0.f;
#pragma unroll
        for (int i = 0; i < kCols; ++i) {
          sacc = fmaf(kr[i], qt[j * D + i], sacc);
          dpacc = fmaf(vr[i], dt[j * D + i], dpacc);
        }
        sacc = lane_group_sum<T>(sacc);
        dpacc = lane_group_sum<T>(dpacc);
        const int qi = qw + j;
        const bool dead = !live || qi >= a.m || (CAUSAL && key > qi + a.diag);
        const int js = wave * kSlice + j;
        const float p = dead ? 0.f : fast_exp2(sacc * cs - lses[js]);
        const float ds = p * (dpacc - dls[js]);
#pragma unroll
        for (int i = 0; i < kCols; ++i) {
          dv[i] = fmaf(p, dt[j * D + i], dv[i]);
          dk[i] = fmaf(ds, qt[j * D + i], dk[i]);
        }
      }
    }
  }
  const int r = tid / (D / 4), c = tid % (D / 4);
  const int ko = kblk * RW + r;
  const bool out_ok = tid < F32Lds<D, KC>::CHUNKS && ko < a.n;
  __syncthreads();
  put_part(sm, D, RW, wave, lane / T, part * kCols, dk);
  __syncthreads();
  if (out_ok) {
    const f32x4 x = sum_parts<D, KC>(sm, tid) * a.scale;
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.dk) + bi * a.k_sb + g * a.k_sh +
                              (int64_t)ko * a.k_sr + 4 * c) = x;
  }
  __syncthreads();
  put_part(sm, D, RW, wave, lane / T, part * kCols, dv);
  __syncthreads();
  if (out_ok) {
    const f32x4 y = sum_parts<D, KC>(sm, tid);
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.dv) + bi * a.v_sb + g * a.v_sh +
                              (int64_t)ko * a.v_sr + 4 * c) = y;
  }
}

template <int D, int KC>
hipError_t fwd_dk(const AttnArgs& a, hipStream_t s) {
  constexpr int RW = F32Lds<D, KC>::RW;
  const dim3 grid((unsigned)((a.m + RW - 1) / RW) * a.hq * a.b), block(64 * kWaves);
  if (a.causal)
    FAB_TIMED("attn_fwd_f32", s, hipLaunchKernelGGL((attn_fwd_f32_kernel<D, KC, true>), grid, block, 0, s, a));
  else
    FAB_TIMED("attn_fwd_f32", s, hipLaunchKernelGGL((attn_fwd_f32_kernel<D, KC, false>), grid, block, 0, s, a));
  return hipGetLastError();
}

template <int D>
hipError_t fwd_d(const AttnArgs& a, hipStream_t s) {
  constexpr int RW8 = F32Lds<D, 8>::RW;
  const int64_t wgs = (a.m + RW8 - 1) / RW8 * (int64_t)a.hq * a.b;
  if constexpr (D == 64) {
    if (wgs < kCUs) return fwd_dk<D, 4>(a, s);
  }
  return fwd_dk<D, 8>(a, s);
}

template <int D, int KC, bool CAUSAL>
__global__ __launch_bounds__(64 * kWaves) void attn_bwd_f32_kernel(AttnArgs a, int nq) {
  __shared__ __attribute__((aligned(16))) float sm[F32Lds<D, KC>::FLOATS];
  if ((int)blockIdx.x < nq)
    dq_f32_body<D, KC, CAUSAL>(a, (int)blockIdx.x, sm);
  else
    dkdv_f32_body<D, KC, CAUSAL>(a, (int)blockIdx.x - nq, sm);
}

template <int D, int KC>
hipError_t bwd_dk(const AttnArgs& a, hipStream_t s) {
  constexpr int RW = F32Lds<D, KC>::RW;
  const dim3 block(64 * kWaves);
  const int nq = (a.m + RW - 1) / RW * a.hq * a.b;
  const int nk = (a.n + RW - 1) / RW * a.hkv * a.b;
  const dim3 grid((unsigned)(nq + nk));
  if (a.causal)
    FAB_TIMED("attn_bwd_f32", s, hipLaunchKernelGGL((attn_bwd_f32_kernel<D, KC, true>), grid, block, 0, s, a, nq));
  else
    FAB_TIMED("attn_bwd_f32", s, hipLaunchKernelGGL((attn_bwd_f32_kernel<D, KC, false>), grid, block, 0, s, a, nq));
  return hipGetLastError();
}

template <int D>
hipError_t bwd_d(const AttnArgs& a, hipStream_t s) {
  constexpr int RW8 = F32Lds<D, 8>::RW;
  const int64_t wgs = (a.m + RW8 - 1) / RW8 * (int64_t)a.hq * a.b +
                      (a.n + RW8 - 1) / RW8 * (int64_t)a.hkv * a.b;
  if constexpr (D == 64) {
    if (wgs < kCUs) return bwd_dk<D, 4>(a, s);
  }
  return bwd_dk<D, 8>(a, s);
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
