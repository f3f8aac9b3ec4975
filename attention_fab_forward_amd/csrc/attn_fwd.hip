// Softmax attention forward, bf16 in / fp32 accumulate, on gfx950 MFMA.
//
// Computes O = softmax(scale * Q K^T [+ causal mask]) V and the per-row
// log-sum-exp, one block of query rows per workgroup, streaming key/value
// blocks through LDS so the n x n score matrix is never stored
// (FlashAttention-style tiling: "Ulysses Sequence Parallelism", section
// "Contexte Technique"; causal masks defined from indices: "AutoSP", section
// 2.A).  The running row maximum and sum are the usual online-softmax
// rescaling, which leaves the result equal to the plain definition.
//
// Layout choices (workgroup = NW waves, 8 by default so that the 256 queries
// of a workgroup share every K / V tile copied into LDS; each wave takes 32 QT
// queries, and with QT = 2 the two 32-query MFMA tiles share every LDS
// fragment read):
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: K is the A operand (from LDS),
//    Q^T the B operand (registers, whole kernel).  Lane l owns query l%32 of
//    each tile, so row max / row sum are in-lane plus one exchange with lane
//    l^32, and an output rescale is one scalar per lane.
//  * K rows sit in LDS in perm_row order, so accumulator slot s of lane l holds
//    key 16*(l/32)+s and the lane's 8 consecutive probabilities are directly
//    the B operand of O^T = V^T P^T.
//  * V stays in its natural [key][d] layout in LDS; the V^T A operand is read
//    with the transposing ds_read_b64_tr_b16, the source lanes addressing the
//    d columns in perm_row order so every lane owns 16 consecutive outputs.
//  * K and V tiles are copied global -> LDS asynchronously
//    (global_load_lds_dwordx4, no register staging) into two stages, each
//    wave group issuing one tile during its softmax phase; each LDS row is
//    16-byte-chunk XOR-swizzled so the MFMA operand reads are free of bank
//    conflicts, the swizzle being applied on the global address side.
//  * A block's exponentials are taken against the running reference m (a row
//    maximum of earlier blocks) without forming the block's own row maximum.
//    Only a block that would carry some row's probabilities past a sum of
//    2^32, or a row with no reference yet, takes its row maximum; the
//    reference then moves when that maximum exceeds it by more than 2^8 (one
//    accumulator rescale).  fp32 and bf16 keep their relative precision at
//    any scale, and per row O and l stay below (keys / 64) 2^32 max|V|, far
//    inside fp32's range, so the result is that of the plain definition.
//  * Causal blocks are dispatched longest-first; blocks above the diagonal
//    are never loaded; a wave skips key blocks fully masked for it.
#include "fab_device.h"
#include "fab_internal.h"

namespace fab {
namespace {

template <int D>
struct FwdCfg {
  static constexpr int BN = kAttnFwdBN;     // keys per step
  static constexpr int QT = kAttnFwdQT;     // 32-query tiles per wave
  static constexpr int NW = kAttnFwdWaves;  // waves per workgroup
  static constexpr int BM = 32 * NW * QT;   // queries per workgroup
  static constexpr int CPR = D / 8;         // 16-byte chunks per row
  static constexpr int RB = D * 2;          // row bytes (no padding)
  static constexpr int TILE = BN * RB;      // bytes of one K or V tile
  static constexpr int STAGE = 2 * TILE;
  static constexpr int RPI = 1024 / RB;     // rows per 1 KiB async copy
  static constexpr int DT = D / 32;         // 32-wide output tiles
  static constexpr int DC = D / 16;         // 16-deep contraction chunks
};

// Physical 16-byte chunk of logical chunk c in row r.
template <int D>
__device__ __forceinline__ int k_swz(int r, int c) { return c ^ (r & (FwdCfg<D>::CPR - 1)); }
template <int D>
__device__ __forceinline__ int v_swz(int r, int c) {
  return c ^ ((4 * (r & 3)) & (FwdCfg<D>::CPR - 1));
}

// Async copies of one key block of K and V into an LDS stage, by NWC copying
// waves.  Copying wave w fills 1 KiB blocks [w * CPW, (w+1) * CPW) of each
// tile; lane j of copy i writes
// LDS row r = (w * CPW + i) * RPI + j / CPR, physical chunk j % CPR.  The
// per-lane element offsets inside a block are fixed for the whole kernel, so
// they are computed once; each step only advances the wave-uniform base.
template <int D, int NWC>
struct TileOffsets {
  static constexpr int CPW = FwdCfg<D>::TILE / 1024 / NWC;  // copies per copying wave per tile
  static_assert(CPW * NWC * 1024 == FwdCfg<D>::TILE, "tile copies must split evenly");
  uint32_t k[CPW], v[CPW];  // byte offsets within a block
};

// LDS row written by lane `lane` of copying wave `wave` in copy i; K holds
// tile key perm_row(r) there, V tile key r.
template <int D, int NWC>
__device__ __forceinline__ int copy_row(int wave, int lane, int i) {
  using C = FwdCfg<D>;
  return (wave * TileOffsets<D, NWC>::CPW + i) * C::RPI + lane / C::CPR;
}

template <int D, int NWC>
__device__ __forceinline__ TileOffsets<D, NWC> tile_offsets(int64_t k_sr, int64_t v_sr, int wave,
                                                            int lane) {
  using C = FwdCfg<D>;
  TileOffsets<D, NWC> t;
#pragma unroll
  for (int i = 0; i < TileOffsets<D, NWC>::CPW; ++i) {
    const int r = copy_row<D, NWC>(wave, lane, i);
    const int pc = lane % C::CPR;
    const int kr = perm_row(r & 31) + (r & ~31);
    t.k[i] = (uint32_t)(2 * (kr * k_sr + 8 * k_swz<D>(r, pc)));
    t.v[i] = (uint32_t)(2 * (r * v_sr + 8 * v_swz<D>(r, pc)));
  }
  return t;
}

// Async copy of key block [key0, key0 + BN) of K (perm_row row order) or V
// (natural order) into an LDS tile.  Rows past n (only in a ragged last block)
// are clamped to row n - 1: their scores are masked, so their probabilities
// are zero.
template <int D, bool IS_K, int NWC>
__device__ __forceinline__ void issue_kv(const TileOffsets<D, NWC>& t, const uint16_t* base,
                                         int64_t sr, int key0, int n, char* tile, int wave,
                                         int lane) {
  using C = FwdCfg<D>;
  constexpr int CPW = TileOffsets<D, NWC>::CPW;
  const char* src = reinterpret_cast<const char*>(base + (int64_t)key0 * sr);
  char* dst = tile + wave * CPW * 1024;
  if (key0 + C::BN <= n) {
#pragma unroll
    for (int i = 0; i < CPW; ++i) dma16(src, IS_K ? t.k[i] : t.v[i], dst + i * 1024);
  } else {
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int r = copy_row<D, NWC>(wave, lane, i);
      const int kr = IS_K ? perm_row(r & 31) + (r & ~31) : r;
      const int64_t shift = min(kr, n - 1 - key0) - kr;  // row shift for clamping
      dma16_at(src + (IS_K ? t.k[i] : t.v[i]) + 2 * shift * sr, dst + i * 1024);
    }
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * FwdCfg<D>::NW, 8 / FwdCfg<D>::NW) void
attn_fwd_bf16_kernel(AttnArgs a) {
  using C = FwdCfg<D>;
  static_assert(C::QT == 1, "the pipelined forward takes one 32-query tile per wave");
  __shared__ __attribute__((aligned(1024))) char smem[4 * C::TILE];
  auto kbuf = [&](int i) { return smem + (i & 1) * C::TILE; };        // K tile buffers
  auto vbuf = [&](int i) { return smem + (2 + (i & 1)) * C::TILE; };  // V tile buffers

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lq = lane & 31, lg = lane >> 5;
  const int l16 = lane & 15, g16 = lane >> 4;

  const int nqb = (a.m + C::BM - 1) / C::BM;
  // longest query blocks of a head first, XCD-aware (see xcd_map)
  int bh, qi;
  xcd_map(blockIdx.x, a.b * a.hq, nqb, bh, qi);
  const int h = bh % a.hq, bi = bh / a.hq;
  const int qb = CAUSAL ? (nqb - 1 - qi) : qi;
  const int g = h / a.group;

  const uint16_t* qbase = static_cast<const uint16_t*>(a.q) + bi * a.q_sb + h * a.q_sh;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + bi * a.k_sb + g * a.k_sh;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + bi * a.v_sb + g * a.v_sh;

  const int q0 = qb * C::BM + wave * 32;  // first query of this wave
  const int myq = q0 + lq;

  // keys up to the last one visible to the workgroup's last query
  const int kend = CAUSAL ? min(a.n, max(0, qb * C::BM + C::BM + a.diag)) : a.n;
  const int nkb = (kend + C::BN - 1) / C::BN;  // key blocks of the workgroup
  // key blocks this wave computes (causal: up to the one holding the last key
  // its last query sees)
  const int nkw = q0 >= a.m ? 0
                  : CAUSAL ? (q0 + 31 + a.diag < 0 ? 0 : min(nkb, (q0 + 31 + a.diag) / C::BN + 1))
                           : nkb;
  // Copies go out at the L2 -> CU rate and hold up the wave that issues
  // them, so each wave group issues one tile in its softmax phase: the second
  // group K (at the start of an iteration), the first group V (after the
  // first barrier); the group running its products issues none.
  constexpr int NWC = C::NW / 2;
  const int cw = wave % NWC;
  const TileOffsets<D, NWC> toff = tile_offsets<D, NWC>(a.k_sr, a.v_sr, cw, lane);
  auto copy_k = [&](int kb) {
    issue_kv<D, true, NWC>(toff, kbase, a.k_sr, kb * C::BN, a.n, kbuf(kb), cw, lane);
  };
  auto copy_v = [&](int kb) {
    issue_kv<D, false, NWC>(toff, vbase, a.v_sr, kb * C::BN, a.n, vbuf(kb), cw, lane);
  };
  if (wave >= NWC) copy_k(0);

  // Q^T fragments: lane holds Q[myq][16c + 8lg .. +7] for every chunk c.
  u32x4 qf[C::DC];
#pragma unroll
  for (int c = 0; c < C::DC; ++c)
    qf[c] = myq < a.m ? ldg16(qbase + (int64_t)myq * a.q_sr + 16 * c + 8 * lg) : u32x4{0, 0, 0, 0};

  f32x16 o[C::DT];
#pragma unroll
  for (int t = 0; t < C::DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float cs = a.scale_log2;

  // Transposed V^T reads (ds_read_b64_tr_b16): this lane, as source lane
  // s = l16 of its 16-lane group, addresses key row s/4 of a 4-key group and
  // the 4 d columns starting at D_u = 16(u%2) + 8(g%2) + 4(u/2), u = s%4,
  // which hands lane l the d column perm_row(l%32) of the 32-wide tile.
  const int u = l16 & 3;
  const int tr_d = 16 * (u & 1) + 8 * (g16 & 1) + 4 * (u >> 1);  // + 32 t
  const int tr_row = l16 >> 2;

  // S^T of one key block: s[sb] holds keys 32 sb + 16 lg + r (slot r) of query
  // myq.  Operand i: d chunk c = i / 2 of key sub-block sb = i % 2.
  auto compute_s = [&](f32x16 (&s)[2], const char* kt) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[sb][r] = 0.f;
    lds_mfma_pipeline<2 * C::DC, 6>(
        [&](int i) {
          const int row = 32 * (i % 2) + lq;
          return lds16(kt + row * C::RB + 16 * k_swz<D>(row, 2 * (i / 2) + lg));
        },
        [&](int i, const u32x4& x) { s[i % 2] = mfma32(x, qf[i / 2], s[i % 2]); });
  };

  // Online softmax of block j on the VALU: mask, P_j (bf16, packed as the
  // next MFMA's B operand) and its row sum; the row maximum and the O rescale
  // only when the reference has to move.
  f32x16 s[2];
  u32x4 pb[2][2];
  auto softmax = [&](int j) {
    const int key0 = j * C::BN;
    if ((CAUSAL && key0 + C::BN - 1 > q0 + a.diag) || key0 + C::BN > a.n) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * sb + 16 * lg + r;
          if ((CAUSAL && key > myq + a.diag) || key >= a.n) s[sb][r] = -INFINITY;
        }
    }
    // P_j against the running reference m (a row maximum of earlier blocks,
    // in log2 units): only a block whose probabilities for some row would sum
    // to 2^32 or more, or a row with no reference yet (its first keys: the
    // exponent is then +inf or NaN), takes the row maximum of S_j and may move
    // the reference.  fp32 and bf16 keep their relative precision at any
    // scale, so how far p sits above 1 changes no result.
    auto exponentials = [&](float ref) {
      float sum = 0.f;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = fast_exp2(fmaf(s[sb][r], cs, -ref));
          sum += p[r];
        }
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int w = 0; w < 4; ++w) pb[sb][c][w] = pack_bf16(p[8 * c + 2 * w], p[8 * c + 2 * w + 1]);
      }
      return sum;
    };
    float lsum = exponentials(m_run);
    if (__ballot(!(lsum < 0x1p32f))) {
      float mx = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sb][r]);
      mx = pair_max(mx) * cs;
      // move the reference maximum only when p would otherwise exceed 2^8
      const float m_new = mx > m_run + 8.f ? mx : m_run;
      // a row that has seen no key yet (offset causal masks) keeps m = -inf and
      // takes 0 as the exponent reference: its probabilities are exactly 0
      const float m_ref = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_ref);
      const bool rescale = m_new != m_run;
      lsum = exponentials(m_ref);
      l_run *= alpha;
      m_run = m_new;
      if (__ballot(rescale)) {
#pragma unroll
        for (int t = 0; t < C::DT; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
      }
    }
    l_run += lsum;
  };
  // O^T += V_j^T P_j^T.  Operand i: output tile t = i % DT, keys
  // 32 sb + 16 lg + 8 c + e with (sb, c) = (i / DT / 2, i / DT % 2), read as
  // two 4-key groups.
  auto pv = [&](int j) {
    const char* vt = vbuf(j);
    // raised wave priority while issuing PV: the group that has finished its
    // softmax gets the MFMA pipe before the other group's S products
    __builtin_amdgcn_s_setprio(2);
    lds_mfma_pipeline<4 * C::DT, 6>(
        [&](int i) {
          const int t = i % C::DT, sb = i / C::DT / 2, c = (i / C::DT) % 2;
          const int dcol = 32 * t + tr_d;    // first of the 4 d columns this lane addresses
          const int cbyte = 2 * (dcol & 7);  // byte offset inside its 16-byte chunk
          const int r0 = 32 * sb + 16 * (g16 >> 1) + 8 * c + tr_row;
          const int r1 = r0 + 4;
          const u32x2 lo = lds_tr8(vt + r0 * C::RB + 16 * v_swz<D>(r0, dcol >> 3) + cbyte);
          const u32x2 hi = lds_tr8(vt + r1 * C::RB + 16 * v_swz<D>(r1, dcol >> 3) + cbyte);
          return u32x4{lo[0], lo[1], hi[0], hi[1]};
        },
        [&](int i, const u32x4& x) {
          const int t = i % C::DT, sb = i / C::DT / 2, c = (i / C::DT) % 2;
          o[t] = mfma32(x, pb[sb][c], o[t]);
        });
    __builtin_amdgcn_s_setprio(0);
  };
  // copies issued in iteration j: K[j + 1] and V[j] (their buffers held
  // K[j - 1] and V[j - 2], read by both groups before the previous barrier);
  // V[j] is first read in iteration j + 1

  wait_vmem();
  lds_barrier();
  // Two wave groups in ping-pong: waves 0-3 and 4-7 (one of each per SIMD).
  // Iteration j has two phases separated by barriers; a wave's MFMA phase
  // (S_j = K_j Q^T and O += V_{j-1} P_{j-1}) overlaps the other group's VALU
  // phase (softmax of its S) on the same SIMD:
  //   group 0:  [copies j, MFMA j]  |  [softmax j]      then wait for copies
  //   group 1:  [copies j, softmax j-1]  |  [MFMA j]    then wait for copies
  // Both groups run j = 0 .. nkb with two barriers per iteration.
  if (wave < 4) {
    int j = 0;
    for (; j <= nkb; ++j) {
      if (j < nkw) compute_s(s, kbuf(j));
      if (j >= 1 && j <= nkw) pv(j - 1);
      lds_barrier();
      if (j < nkb) copy_v(j);
      if (j < nkw) softmax(j);
      wait_vmem();
      lds_barrier();
    }
  } else {
    for (int j = 0; j <= nkb; ++j) {
      if (j + 1 < nkb) copy_k(j + 1);
      if (j >= 1 && j <= nkw) softmax(j - 1);
      lds_barrier();
      if (j < nkw) compute_s(s, kbuf(j));
      if (j >= 1 && j <= nkw) pv(j - 1);
      wait_vmem();
      lds_barrier();
    }
  }

  // rows that saw no key (offset causal masks): O = 0, LSE = -inf
  const float l_tot = pair_sum(l_run);
  if (myq < a.m) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
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
      a.lse[((int64_t)bi * a.hq + h) * a.m + myq] =
          l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t s) {
  const int nqb = (a.m + FwdCfg<D>::BM - 1) / FwdCfg<D>::BM;
  const dim3 grid((unsigned)nqb * a.hq * a.b), block(64 * FwdCfg<D>::NW);
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
