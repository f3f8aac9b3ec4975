// Softmax attention forward, bf16 in / fp32 accumulate, on gfx950 MFMA.
//
// Computes O = softmax(scale * Q K^T [+ causal mask]) V and the per-row
// log-sum-exp, one query block per workgroup, streaming key/value blocks
// through LDS so the n x n score matrix is never stored (FlashAttention-style
// tiling: "Ulysses Sequence Parallelism", section "Contexte Technique"; causal
// masks defined from indices: "AutoSP", section 2.A).  The running row
// maximum and sum follow the usual online-softmax rescaling, which leaves the
// result equal to the plain definition.
//
// Layout choices (per wave of 64 lanes, 32 queries):
//  * S^T = K Q^T is formed with v_mfma_f32_32x32x16_bf16, K as the A operand
//    (from LDS) and Q^T as the B operand (held in registers for the whole
//    kernel).  Lane l then owns query l%32, so row max / row sum are in-lane
//    reductions plus one exchange with lane l^32.
//  * K rows are stored in LDS in perm_row order, which makes accumulator slot
//    s of lane l hold key 16*(l/32)+s: each lane's probabilities for 8
//    consecutive keys become directly the B operand of the P.V product.
//  * O^T = V^T P^T uses V^T (d x keys) as the A operand; V is transposed while
//    being staged into LDS, with d rows also in perm_row order so each lane
//    ends up owning 16 consecutive output columns.
//  * Two LDS stages: tile j+1 is fetched into registers while tile j is
//    computed, then written to the other stage; one barrier per step.
//  * Causal blocks are visited longest-first; blocks above the diagonal are
//    never loaded, and a wave skips blocks that are fully masked for it.
#include "fab_device.h"
#include "fab_internal.h"

namespace fab {
namespace {

template <int D>
struct FwdCfg {
  static constexpr int BM = kAttnFwdBM;
  static constexpr int BN = kAttnFwdBN;
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int KP = D * 2 + 16;         // K row pitch in LDS (bytes)
  static constexpr int VP = BN * 2 + 16;        // V^T row pitch (bytes), one row per d
  static constexpr int KBYTES = BN * KP;
  static constexpr int STAGE = KBYTES + D * VP;
  static constexpr int KLOADS = BN * CPR / 256; // K chunks per thread per tile
  static constexpr int KPT = BN * CPR / 256;    // keys per thread in V staging
  static constexpr int KQ = BN / KPT;           // key groups in V staging
  static constexpr int DT = D / 32;             // 32-wide output tiles
  static constexpr int DC = D / 16;             // 16-deep contraction chunks
};

template <int D>
struct Stage {
  u32x4 k[FwdCfg<D>::KLOADS];
  u32x4 v[FwdCfg<D>::KPT];
};

template <int D>
__device__ __forceinline__ void fetch_tile(Stage<D>& st, const uint16_t* kbase,
                                           const uint16_t* vbase, int64_t k_sr,
                                           int64_t v_sr, int key0, int n, int tid) {
  using C = FwdCfg<D>;
  const int c = tid % C::CPR;
#pragma unroll
  for (int u = 0; u < C::KLOADS; ++u) {
    const int r = tid / C::CPR + (256 / C::CPR) * u;
    const int key = key0 + r;
    st.k[u] = key < n ? ldg16(kbase + (int64_t)key * k_sr + c * 8) : u32x4{0, 0, 0, 0};
  }
  const int wave = tid >> 6, lane = tid & 63;
  const int kq = lane % C::KQ;
  const int dc = (64 / C::KQ) * wave + lane / C::KQ;
#pragma unroll
  for (int u = 0; u < C::KPT; ++u) {
    const int key = key0 + C::KPT * kq + u;
    st.v[u] = key < n ? ldg16(vbase + (int64_t)key * v_sr + dc * 8) : u32x4{0, 0, 0, 0};
  }
}

template <int D>
__device__ __forceinline__ void store_tile(const Stage<D>& st, char* stage, int tid) {
  using C = FwdCfg<D>;
  const int c = tid % C::CPR;
#pragma unroll
  for (int u = 0; u < C::KLOADS; ++u) {
    const int r = tid / C::CPR + (256 / C::CPR) * u;
    const int pos = perm_row_inv(r & 31) + (r & ~31);
    sts16(stage + pos * C::KP + c * 16, st.k[u]);
  }
  char* vt = stage + C::KBYTES;
  const int wave = tid >> 6, lane = tid & 63;
  const int kq = lane % C::KQ;
  const int dc = (64 / C::KQ) * wave + lane / C::KQ;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int d = dc * 8 + i;
    const int row = perm_row_inv(d & 31) + (d & ~31);
    char* dst = vt + row * C::VP + C::KPT * kq * 2;
    const int w = i >> 1;
    if constexpr (C::KPT == 4) {
      u32x2 val;
      if (i & 1) {
        val[0] = pick_hi(st.v[0][w], st.v[1][w]);
        val[1] = pick_hi(st.v[2][w], st.v[3][w]);
      } else {
        val[0] = pick_lo(st.v[0][w], st.v[1][w]);
        val[1] = pick_lo(st.v[2][w], st.v[3][w]);
      }
      sts8(dst, val);
    } else {
      const uint32_t val = (i & 1) ? pick_hi(st.v[0][w], st.v[1][w])
                                   : pick_lo(st.v[0][w], st.v[1][w]);
      sts4(dst, val);
    }
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(AttnArgs a) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int lq = lane & 31, lg = lane >> 5;

  const int nqb = (a.m + C::BM - 1) / C::BM;
  int id = blockIdx.x;
  const int h = id % a.hq;
  id /= a.hq;
  const int bi = id % a.b;
  id /= a.b;
  const int qb = CAUSAL ? (nqb - 1 - id) : id;
  const int g = h / a.group;

  const uint16_t* qbase = static_cast<const uint16_t*>(a.q) + bi * a.q_sb + h * a.q_sh;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + bi * a.k_sb + g * a.k_sh;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + bi * a.v_sb + g * a.v_sh;

  const int q0 = qb * C::BM + wave * 32;
  const int myq = q0 + lq;
  const bool wave_live = q0 < a.m;

  // Q^T fragments: lane holds Q[myq][16c + 8lg .. +7] for every chunk c.
  u32x4 qf[C::DC];
#pragma unroll
  for (int c = 0; c < C::DC; ++c)
    qf[c] = myq < a.m ? ldg16(qbase + (int64_t)myq * a.q_sr + 16 * c + 8 * lg)
                      : u32x4{0, 0, 0, 0};

  const int kend = CAUSAL ? min(a.n, qb * C::BM + C::BM) : a.n;
  const int nkb = (kend + C::BN - 1) / C::BN;

  f32x16 o[C::DT];
#pragma unroll
  for (int t = 0; t < C::DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float cs = a.scale_log2;

  Stage<D> pre;
  fetch_tile<D>(pre, kbase, vbase, a.k_sr, a.v_sr, 0, a.n, tid);
  store_tile<D>(pre, smem, tid);
  __syncthreads();

  for (int kb = 0; kb < nkb; ++kb) {
    const bool more = kb + 1 < nkb;
    if (more) fetch_tile<D>(pre, kbase, vbase, a.k_sr, a.v_sr, (kb + 1) * C::BN, a.n, tid);

    const int key0 = kb * C::BN;
    const char* kbuf = smem + (kb & 1) * C::STAGE;
    const char* vbuf = kbuf + C::KBYTES;
    const bool wave_work = wave_live && (!CAUSAL || key0 <= q0 + 31);
    if (wave_work) {
      f32x16 s[2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[sb][r] = 0.f;
        const char* krow = kbuf + (32 * sb + lq) * C::KP + lg * 16;
#pragma unroll
        for (int c = 0; c < C::DC; ++c) s[sb] = mfma32(lds16(krow + c * 32), qf[c], s[sb]);
      }
      const bool need_mask = (CAUSAL && key0 + C::BN - 1 > q0) || (key0 + C::BN > a.n);
      if (need_mask) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + 32 * sb + 16 * lg + r;
            if ((CAUSAL && key > myq) || key >= a.n) s[sb][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sb][r]);
      mx = fmaxf(mx, wave_xor32(mx));
      const float m_new = fmaxf(m_run, mx * cs);
      const float alpha = fast_exp2(m_run - m_new);
      float lsum = 0.f;
      u32x4 pb[2][2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = fast_exp2(s[sb][r] * cs - m_new);
          lsum += p[r];
        }
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int w = 0; w < 4; ++w) pb[sb][c][w] = pack_bf16(p[8 * c + 2 * w], p[8 * c + 2 * w + 1]);
      }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int t = 0; t < C::DT; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
      }
#pragma unroll
      for (int t = 0; t < C::DT; ++t) {
        const char* vrow = vbuf + (32 * t + lq) * C::VP + lg * 32;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int c = 0; c < 2; ++c) o[t] = mfma32(lds16(vrow + (32 * sb + 8 * c) * 2), pb[sb][c], o[t]);
      }
    }
    if (more) store_tile<D>(pre, smem + ((kb + 1) & 1) * C::STAGE, tid);
    __syncthreads();
  }

  if (!wave_live) return;
  const float l_tot = l_run + wave_xor32(l_run);
  if (myq < a.m) {
    const float inv = 1.f / l_tot;
    uint16_t* orow = static_cast<uint16_t*>(a.o_out) + bi * a.o_sb + h * a.o_sh +
                     (int64_t)myq * a.o_sr + 16 * lg;
#pragma unroll
    for (int t = 0; t < C::DT; ++t) {
      u32x4 lo, hi;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        lo[w] = pack_bf16(o[t][2 * w] * inv, o[t][2 * w + 1] * inv);
        hi[w] = pack_bf16(o[t][8 + 2 * w] * inv, o[t][8 + 2 * w + 1] * inv);
      }
      stg16(orow + 32 * t, lo);
      stg16(orow + 32 * t + 8, hi);
    }
    if (lg == 0)
      a.lse[((int64_t)bi * a.hq + h) * a.m + myq] = (m_run + fast_log2(l_tot)) * kLn2;
  }
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t s) {
  const int nqb = (a.m + kAttnFwdBM - 1) / kAttnFwdBM;
  const dim3 grid((unsigned)nqb * a.hq * a.b), block(256);
  if (a.causal)
    FAB_TIMED("attn_fwd_bf16", s, hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, true>), grid, block, 0, s, a));
  else
    FAB_TIMED("attn_fwd_bf16", s, hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, false>), grid, block, 0, s, a));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const AttnArgs& a, int d, hipStream_t s) {
  if (d == 128) return launch_d<128>(a, s);
  if (d == 64) return launch_d<64>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace fab
