// Softmax attention backward, bf16 in / fp32 accumulate, on gfx950 MFMA.
//
// Gradients of L = <dO, O> for O = softmax(scale Q K^T [+ causal]) V, with the
// probabilities recomputed from the saved log-sum-exp instead of being stored
// (rematerialisation over storage: "AutoSP", section 2.B):
//   P = exp(scale Q K^T - LSE), dP = dO V^T, D_i = rowsum(dO_i * O_i),
//   dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO.
//
// Deterministic two-kernel schedule (no atomics):
//  * attn_dkdv_bf16_kernel: one workgroup per 128 keys (4 waves x 32 keys)
//    of one kv head.  K and V stay in registers; query blocks of 64 (and all
//    query heads of the group) stream through a double-buffered LDS in both
//    natural and transposed layouts.  dK^T and dV^T accumulate in registers.
//  * attn_dq_bf16_kernel: one workgroup per 128 queries (4 waves x 32) of one
//    query head.  Q, dO, LSE and D stay in registers; key blocks of 64 stream
//    through LDS (K and V natural, K transposed).  dQ^T accumulates in
//    registers.  S and dP are recomputed here rather than exchanged.
// MFMA layout conventions are those of the forward kernel (perm_row order
// makes accumulator slots contiguous along the lane's row).
#include "fab_device.h"
#include "fab_internal.h"

namespace fab {
namespace {

template <int D>
struct BwdCfg {
  static constexpr int CPR = D / 8;         // 16-byte chunks per row
  static constexpr int NP = D * 2 + 16;     // natural tile row pitch (bytes)
  static constexpr int TILE = 64;           // rows of a streamed tile
  static constexpr int TP = TILE * 2 + 16;  // transposed tile row pitch (bytes)
  static constexpr int NBYTES = TILE * NP;
  static constexpr int TBYTES = D * TP;
  static constexpr int RPT = TILE * CPR / 256;  // rows per thread (transposing staging)
  static constexpr int RQ = TILE / RPT;         // row groups in transposing staging
  static constexpr int NLOADS = TILE * CPR / 256;
  static constexpr int DT = D / 32;
  static constexpr int DC = D / 16;
};

// Rows [r0, r0 + 64) of a [rows, D] bf16 matrix, loaded so that each thread
// holds RPT consecutive rows of one 16-byte column chunk (ready for both a
// natural and a transposed LDS write).  Rows >= nrows read as zero.
template <int D>
struct TTile {
  u32x4 v[BwdCfg<D>::RPT];
};

template <int D>
__device__ __forceinline__ void ttile_fetch(TTile<D>& t, const uint16_t* base, int64_t sr,
                                            int r0, int nrows, int tid) {
  using C = BwdCfg<D>;
  const int wave = tid >> 6, lane = tid & 63;
  const int rq = lane % C::RQ;
  const int dc = (64 / C::RQ) * wave + lane / C::RQ;
#pragma unroll
  for (int u = 0; u < C::RPT; ++u) {
    const int r = r0 + C::RPT * rq + u;
    t.v[u] = r < nrows ? ldg16(base + (int64_t)r * sr + dc * 8) : u32x4{0, 0, 0, 0};
  }
}

// Natural layout: LDS row perm_row_inv(r) holds tile row r (per 32-row group).
template <int D>
__device__ __forceinline__ void ttile_store_natural(const TTile<D>& t, char* dst, int tid) {
  using C = BwdCfg<D>;
  const int wave = tid >> 6, lane = tid & 63;
  const int rq = lane % C::RQ;
  const int dc = (64 / C::RQ) * wave + lane / C::RQ;
#pragma unroll
  for (int u = 0; u < C::RPT; ++u) {
    const int r = C::RPT * rq + u;
    const int pos = perm_row_inv(r & 31) + (r & ~31);
    sts16(dst + pos * C::NP + dc * 16, t.v[u]);
  }
}

// Transposed layout: LDS row (perm order of d) holds the 64 tile rows of one
// column d, contiguous.
template <int D>
__device__ __forceinline__ void ttile_store_transposed(const TTile<D>& t, char* dst, int tid) {
  using C = BwdCfg<D>;
  const int wave = tid >> 6, lane = tid & 63;
  const int rq = lane % C::RQ;
  const int dc = (64 / C::RQ) * wave + lane / C::RQ;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int d = dc * 8 + i;
    const int row = perm_row_inv(d & 31) + (d & ~31);
    char* p = dst + row * C::TP + C::RPT * rq * 2;
    const int w = i >> 1;
    if constexpr (C::RPT == 4) {
      u32x2 val;
      if (i & 1) {
        val[0] = pick_hi(t.v[0][w], t.v[1][w]);
        val[1] = pick_hi(t.v[2][w], t.v[3][w]);
      } else {
        val[0] = pick_lo(t.v[0][w], t.v[1][w]);
        val[1] = pick_lo(t.v[2][w], t.v[3][w]);
      }
      sts8(p, val);
    } else {
      sts4(p, (i & 1) ? pick_hi(t.v[0][w], t.v[1][w]) : pick_lo(t.v[0][w], t.v[1][w]));
    }
  }
}

// Plain natural tile: thread t loads chunk t % CPR of rows t / CPR + k*(256/CPR).
template <int D>
struct NTile {
  u32x4 v[BwdCfg<D>::NLOADS];
};

template <int D>
__device__ __forceinline__ void ntile_fetch(NTile<D>& t, const uint16_t* base, int64_t sr,
                                            int r0, int nrows, int tid) {
  using C = BwdCfg<D>;
  const int c = tid % C::CPR;
#pragma unroll
  for (int u = 0; u < C::NLOADS; ++u) {
    const int r = r0 + tid / C::CPR + (256 / C::CPR) * u;
    t.v[u] = r < nrows ? ldg16(base + (int64_t)r * sr + c * 8) : u32x4{0, 0, 0, 0};
  }
}

template <int D>
__device__ __forceinline__ void ntile_store(const NTile<D>& t, char* dst, int tid) {
  using C = BwdCfg<D>;
  const int c = tid % C::CPR;
#pragma unroll
  for (int u = 0; u < C::NLOADS; ++u) {
    const int r = tid / C::CPR + (256 / C::CPR) * u;
    const int pos = perm_row_inv(r & 31) + (r & ~31);
    sts16(dst + pos * C::NP + c * 16, t.v[u]);
  }
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
template <int D>
struct DkdvStage {
  static constexpr int Q = 0;
  static constexpr int DO = BwdCfg<D>::NBYTES;
  static constexpr int QT = 2 * BwdCfg<D>::NBYTES;
  static constexpr int DOT = QT + BwdCfg<D>::TBYTES;
  static constexpr int LSE = DOT + BwdCfg<D>::TBYTES;
  static constexpr int DLT = LSE + 64 * 4;
  static constexpr int BYTES = DLT + 64 * 4;
};

template <int D>
struct DkdvPrefetch {
  TTile<D> q, dout;
  float lse2, dlt;
};

template <int D>
__device__ __forceinline__ void dkdv_fetch(DkdvPrefetch<D>& pf, const AttnArgs& a, int bi, int h,
                                           int q0, int tid) {
  const uint16_t* qb = static_cast<const uint16_t*>(a.q) + bi * a.q_sb + h * a.q_sh;
  const uint16_t* ob = static_cast<const uint16_t*>(a.dout) + bi * a.o_sb + h * a.o_sh;
  ttile_fetch<D>(pf.q, qb, a.q_sr, q0, a.m, tid);
  ttile_fetch<D>(pf.dout, ob, a.o_sr, q0, a.m, tid);
  if (tid < 64) {
    const int q = q0 + tid;
    const int64_t r = ((int64_t)bi * a.hq + h) * a.m + q;
    pf.lse2 = q < a.m ? a.lse_in[r] * kLog2e : INFINITY;
    pf.dlt = q < a.m ? a.delta[r] : 0.f;
  }
}

template <int D>
__device__ __forceinline__ void dkdv_store(const DkdvPrefetch<D>& pf, char* st, int tid) {
  using S = DkdvStage<D>;
  ttile_store_natural<D>(pf.q, st + S::Q, tid);
  ttile_store_natural<D>(pf.dout, st + S::DO, tid);
  ttile_store_transposed<D>(pf.q, st + S::QT, tid);
  ttile_store_transposed<D>(pf.dout, st + S::DOT, tid);
  if (tid < 64) {
    reinterpret_cast<float*>(st + S::LSE)[tid] = pf.lse2;
    reinterpret_cast<float*>(st + S::DLT)[tid] = pf.dlt;
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void attn_dkdv_bf16_kernel(AttnArgs a) {
  using C = BwdCfg<D>;
  using S = DkdvStage<D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * S::BYTES];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int lq = lane & 31, lg = lane >> 5;

  int id = blockIdx.x;
  const int g = id % a.hkv;
  id /= a.hkv;
  const int bi = id % a.b;
  id /= a.b;
  const int kblk = id;  // causal: low key blocks see the most queries, so they go first
  const int k0w = kblk * kAttnBwdKB + wave * 32;
  const int mykey = k0w + lq;

  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + bi * a.k_sb + g * a.k_sh;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + bi * a.v_sb + g * a.v_sh;
  u32x4 kf[C::DC], vf[C::DC];
#pragma unroll
  for (int c = 0; c < C::DC; ++c) {
    const bool ok = mykey < a.n;
    kf[c] = ok ? ldg16(kbase + (int64_t)mykey * a.k_sr + 16 * c + 8 * lg) : u32x4{0, 0, 0, 0};
    vf[c] = ok ? ldg16(vbase + (int64_t)mykey * a.v_sr + 16 * c + 8 * lg) : u32x4{0, 0, 0, 0};
  }
  f32x16 dk[C::DT], dv[C::DT];
#pragma unroll
  for (int t = 0; t < C::DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[t][r] = dv[t][r] = 0.f;

  const float cs = a.scale_log2;
  const int qb_first = CAUSAL ? (kblk * kAttnBwdKB) / C::TILE : 0;
  const int nqb = (a.m + C::TILE - 1) / C::TILE;
  const int steps_per_head = nqb - qb_first;
  const int steps = steps_per_head * a.group;
  const bool wave_live = k0w < a.n;

  DkdvPrefetch<D> pf;
  if (steps > 0) {
    dkdv_fetch<D>(pf, a, bi, g * a.group, qb_first * C::TILE, tid);
    dkdv_store<D>(pf, smem, tid);
  }
  __syncthreads();

  for (int step = 0; step < steps; ++step) {
    const bool more = step + 1 < steps;
    if (more) {
      const int nh = (step + 1) / steps_per_head, nq = (step + 1) % steps_per_head;
      dkdv_fetch<D>(pf, a, bi, g * a.group + nh, (qb_first + nq) * C::TILE, tid);
    }
    const int q0 = (qb_first + step % steps_per_head) * C::TILE;
    const char* st = smem + (step & 1) * S::BYTES;
    // A wave skips a query block when every query precedes all its keys.
    const bool wave_work = wave_live && (!CAUSAL || q0 + C::TILE - 1 >= k0w);
    if (wave_work) {
      const bool need_mask = CAUSAL && q0 < k0w + 31;
#pragma unroll
      for (int sq = 0; sq < 2; ++sq) {
        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
        const char* qrow = st + S::Q + (32 * sq + lq) * C::NP + lg * 16;
        const char* orow = st + S::DO + (32 * sq + lq) * C::NP + lg * 16;
#pragma unroll
        for (int c = 0; c < C::DC; ++c) {
          s = mfma32(lds16(qrow + c * 32), kf[c], s);
          dp = mfma32(lds16(orow + c * 32), vf[c], dp);
        }
        // accumulator slot r holds query q0 + 32 sq + 16 lg + r for key `mykey`
        const float* lse2 = reinterpret_cast<const float*>(st + S::LSE) + 32 * sq + 16 * lg;
        const float* dlt = reinterpret_cast<const float*>(st + S::DLT) + 32 * sq + 16 * lg;
        float p[16], ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pr = fast_exp2(s[r] * cs - lse2[r]);
          if (need_mask && q0 + 32 * sq + 16 * lg + r < mykey) pr = 0.f;
          p[r] = pr;
          ds[r] = pr * (dp[r] - dlt[r]);
        }
        u32x4 pb[2], db[2];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            pb[c][w] = pack_bf16(p[8 * c + 2 * w], p[8 * c + 2 * w + 1]);
            db[c][w] = pack_bf16(ds[8 * c + 2 * w], ds[8 * c + 2 * w + 1]);
          }
#pragma unroll
        for (int t = 0; t < C::DT; ++t) {
          const char* trow_o = st + S::DOT + (32 * t + lq) * C::TP + lg * 32 + 64 * sq;
          const char* trow_q = st + S::QT + (32 * t + lq) * C::TP + lg * 32 + 64 * sq;
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            dv[t] = mfma32(lds16(trow_o + 16 * c), pb[c], dv[t]);
            dk[t] = mfma32(lds16(trow_q + 16 * c), db[c], dk[t]);
          }
        }
      }
    }
    if (more) dkdv_store<D>(pf, smem + ((step + 1) & 1) * S::BYTES, tid);
    __syncthreads();
  }

  if (!wave_live || mykey >= a.n) return;
  uint16_t* dkrow = static_cast<uint16_t*>(a.dk) + bi * a.k_sb + g * a.k_sh +
                    (int64_t)mykey * a.k_sr + 16 * lg;
  uint16_t* dvrow = static_cast<uint16_t*>(a.dv) + bi * a.v_sb + g * a.v_sh +
                    (int64_t)mykey * a.v_sr + 16 * lg;
#pragma unroll
  for (int t = 0; t < C::DT; ++t) {
    u32x4 k0, k1, v0, v1;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      k0[w] = pack_bf16(dk[t][2 * w] * a.scale, dk[t][2 * w + 1] * a.scale);
      k1[w] = pack_bf16(dk[t][8 + 2 * w] * a.scale, dk[t][8 + 2 * w + 1] * a.scale);
      v0[w] = pack_bf16(dv[t][2 * w], dv[t][2 * w + 1]);
      v1[w] = pack_bf16(dv[t][8 + 2 * w], dv[t][8 + 2 * w + 1]);
    }
    stg16(dkrow + 32 * t, k0);
    stg16(dkrow + 32 * t + 8, k1);
    stg16(dvrow + 32 * t, v0);
    stg16(dvrow + 32 * t + 8, v1);
  }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <int D>
struct DqStage {
  static constexpr int K = 0;
  static constexpr int V = BwdCfg<D>::NBYTES;
  static constexpr int KT = 2 * BwdCfg<D>::NBYTES;
  static constexpr int BYTES = KT + BwdCfg<D>::TBYTES;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void attn_dq_bf16_kernel(AttnArgs a) {
  using C = BwdCfg<D>;
  using S = DqStage<D>;
  __shared__ __attribute__((aligned(16))) char smem[S::BYTES];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int lq = lane & 31, lg = lane >> 5;

  const int nqb = (a.m + kAttnBwdBM - 1) / kAttnBwdBM;
  int id = blockIdx.x;
  const int h = id % a.hq;
  id /= a.hq;
  const int bi = id % a.b;
  id /= a.b;
  const int qb = CAUSAL ? (nqb - 1 - id) : id;
  const int g = h / a.group;

  const int q0 = qb * kAttnBwdBM + wave * 32;
  const int myq = q0 + lq;
  const bool live = myq < a.m;
  const bool wave_live = q0 < a.m;

  const uint16_t* qbase = static_cast<const uint16_t*>(a.q) + bi * a.q_sb + h * a.q_sh;
  const uint16_t* obase = static_cast<const uint16_t*>(a.dout) + bi * a.o_sb + h * a.o_sh;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + bi * a.k_sb + g * a.k_sh;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + bi * a.v_sb + g * a.v_sh;

  u32x4 qf[C::DC], df[C::DC];
#pragma unroll
  for (int c = 0; c < C::DC; ++c) {
    qf[c] = live ? ldg16(qbase + (int64_t)myq * a.q_sr + 16 * c + 8 * lg) : u32x4{0, 0, 0, 0};
    df[c] = live ? ldg16(obase + (int64_t)myq * a.o_sr + 16 * c + 8 * lg) : u32x4{0, 0, 0, 0};
  }
  const int64_t ridx = ((int64_t)bi * a.hq + h) * a.m + myq;
  const float lse2 = live ? a.lse_in[ridx] * kLog2e : INFINITY;
  const float dlt = live ? a.delta[ridx] : 0.f;

  f32x16 dq[C::DT];
#pragma unroll
  for (int t = 0; t < C::DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[t][r] = 0.f;
  const float cs = a.scale_log2;

  const int kend = CAUSAL ? min(a.n, qb * kAttnBwdBM + kAttnBwdBM) : a.n;
  const int nkb = (kend + C::TILE - 1) / C::TILE;

  TTile<D> kpre;
  NTile<D> vpre;
  ttile_fetch<D>(kpre, kbase, a.k_sr, 0, a.n, tid);
  ntile_fetch<D>(vpre, vbase, a.v_sr, 0, a.n, tid);

  for (int kb = 0; kb < nkb; ++kb) {
    __syncthreads();
    ttile_store_natural<D>(kpre, smem + S::K, tid);
    ttile_store_transposed<D>(kpre, smem + S::KT, tid);
    ntile_store<D>(vpre, smem + S::V, tid);
    __syncthreads();
    if (kb + 1 < nkb) {
      ttile_fetch<D>(kpre, kbase, a.k_sr, (kb + 1) * C::TILE, a.n, tid);
      ntile_fetch<D>(vpre, vbase, a.v_sr, (kb + 1) * C::TILE, a.n, tid);
    }
    const int key0 = kb * C::TILE;
    const bool wave_work = wave_live && (!CAUSAL || key0 <= q0 + 31);
    if (!wave_work) continue;
    const bool need_mask = (CAUSAL && key0 + C::TILE - 1 > q0) || (key0 + C::TILE > a.n);
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
      const char* krow = smem + S::K + (32 * sb + lq) * C::NP + lg * 16;
      const char* vrow = smem + S::V + (32 * sb + lq) * C::NP + lg * 16;
#pragma unroll
      for (int c = 0; c < C::DC; ++c) {
        s = mfma32(lds16(krow + c * 32), qf[c], s);
        dp = mfma32(lds16(vrow + c * 32), df[c], dp);
      }
      // accumulator slot r holds key key0 + 32 sb + 16 lg + r for query `myq`
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = fast_exp2(s[r] * cs - lse2);
        if (need_mask) {
          const int key = key0 + 32 * sb + 16 * lg + r;
          if ((CAUSAL && key > myq) || key >= a.n) p = 0.f;
        }
        ds[r] = p * (dp[r] - dlt);
      }
      u32x4 db[2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int w = 0; w < 4; ++w) db[c][w] = pack_bf16(ds[8 * c + 2 * w], ds[8 * c + 2 * w + 1]);
#pragma unroll
      for (int t = 0; t < C::DT; ++t) {
        const char* trow = smem + S::KT + (32 * t + lq) * C::TP + lg * 32 + 64 * sb;
#pragma unroll
        for (int c = 0; c < 2; ++c) dq[t] = mfma32(lds16(trow + 16 * c), db[c], dq[t]);
      }
    }
  }

  if (!live) return;
  uint16_t* out = static_cast<uint16_t*>(a.dq) + bi * a.q_sb + h * a.q_sh +
                  (int64_t)myq * a.q_sr + 16 * lg;
#pragma unroll
  for (int t = 0; t < C::DT; ++t) {
    u32x4 lo, hi;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      lo[w] = pack_bf16(dq[t][2 * w] * a.scale, dq[t][2 * w + 1] * a.scale);
      hi[w] = pack_bf16(dq[t][8 + 2 * w] * a.scale, dq[t][8 + 2 * w + 1] * a.scale);
    }
    stg16(out + 32 * t, lo);
    stg16(out + 32 * t + 8, hi);
  }
}

template <int D>
hipError_t bwd_d(const AttnArgs& a, hipStream_t s) {
  hipError_t e = launch_attn_delta(a, D, true, s);
  if (e != hipSuccess) return e;
  const dim3 block(256);
  const int nkb = (a.n + kAttnBwdKB - 1) / kAttnBwdKB;
  const int nqb = (a.m + kAttnBwdBM - 1) / kAttnBwdBM;
  const dim3 gk((unsigned)nkb * a.hkv * a.b), gq((unsigned)nqb * a.hq * a.b);
  if (a.causal) {
    FAB_TIMED("attn_bwd_dkdv_bf16", s, hipLaunchKernelGGL((attn_dkdv_bf16_kernel<D, true>), gk, block, 0, s, a));
    FAB_TIMED("attn_bwd_dq_bf16", s, hipLaunchKernelGGL((attn_dq_bf16_kernel<D, true>), gq, block, 0, s, a));
  } else {
    FAB_TIMED("attn_bwd_dkdv_bf16", s, hipLaunchKernelGGL((attn_dkdv_bf16_kernel<D, false>), gk, block, 0, s, a));
    FAB_TIMED("attn_bwd_dq_bf16", s, hipLaunchKernelGGL((attn_dq_bf16_kernel<D, false>), gq, block, 0, s, a));
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd_bf16(const AttnArgs& a, int d, hipStream_t s) {
  if (d == 128) return bwd_d<128>(a, s);
  if (d == 64) return bwd_d<64>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace fab
