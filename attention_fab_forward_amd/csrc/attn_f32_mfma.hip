// Softmax attention in fp32 on the gfx950 fp32 matrix cores
// (v_mfma_f32_32x32x2_f32): forward, and a backward of three launches
// (per-row constants, dK/dV, dQ).  For fp32 problems large enough to fill the
// chip; the plain-FMA kernels of attn_f32.hip serve the small, latency-bound
// ones.  Every operation stays in fp32 (products, sums, exponentials).
//
// Definitions as in the other attention kernels: O = softmax(scale Q K^T
// [+ causal mask]) V, the block O = f(A B) C of the "Memory-efficient tensor
// parallelism" abstract, tiled so the score matrix is never stored ("Ulysses
// Sequence Parallelism", "Contexte Technique"; causal index mask per "AutoSP"
// 2.A), and its derivative with P recomputed from the saved log-sum-exp
// ("AutoSP" 2.B):
//   dP = dO V^T, D_i = rowsum(dO_i * O_i), dS = P (dP - D),
//   dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO.
//
// Layout of one 32 x 32 x 2 product: lane l supplies A[l % 32][l / 32] and
// B[l / 32][l % 32] and holds D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32] in
// accumulator slot r.  A contraction over 8 g + 4 h + e (h = l / 32, e = 0..3)
// in product 4 g + e therefore reads each lane's operand as 4 consecutive
// values, and the contraction index of product j over a 32-row accumulator
// (8 (j / 4) + 4 h + j % 4) is exactly slot j of that accumulator: S (or dS)
// slots are the B operands of the products that follow, with no exchange.
//  * forward: S^T = K Q^T (K rows from LDS, Q in registers), lanes own
//    queries; O^T += V^T P^T.
//  * dK/dV: S = Q K^T, dP = dO V^T (Q, dO rows from LDS, K, V in registers),
//    lanes own keys; dV^T += dO^T P, dK^T += Q^T dS.
//  * dQ: S^T = K Q^T, dP^T = V dO^T, lanes own queries; dQ^T += K^T dS^T.
// Tiles of 32 rows are copied global -> LDS asynchronously (double
// buffered); 16-byte chunk c of row r sits at chunk c ^ (r mod 16), which
// keeps the 16-byte row reads of 16 lanes on distinct banks.
#include "fab_device.h"
#include "fab_internal.h"

namespace fab {
namespace {

__device__ __forceinline__ f32x16 mfma32f(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

constexpr int kMfmaF32Waves = 4;  // waves per workgroup, 32 rows each
// Workgroups per CU of the forward and dQ kernels: at d = 128 a wave's
// operands and accumulators take more than the 256 registers two waves per
// SIMD leave, so it runs one wave per SIMD with the whole register file.
template <int D>
constexpr int f32_mfma_occupancy() { return D == 128 ? 1 : 2; }

template <int D>
struct F32T {
  static constexpr int RB = D * 4;          // row bytes
  static constexpr int ROWS = 32;           // rows of a tile
  static constexpr int BYTES = ROWS * RB;   // 8 or 16 KiB
  static constexpr int G = D / 8;           // contraction groups (4 values per half-wave)
  static constexpr int DT = D / 32;         // 32-wide output tiles
};

__device__ __forceinline__ int fswz(int r, int c) { return c ^ (r & 15); }

// 16 bytes (4 floats, logical chunk c) of row r of a tile.
template <int D>
__device__ __forceinline__ f32x4 tile_row4(const char* tile, int r, int c) {
  return *reinterpret_cast<const f32x4*>(tile + r * F32T<D>::RB + 16 * fswz(r, c));
}
// Element (r, col) of a tile.
template <int D>
__device__ __forceinline__ float tile_at(const char* tile, int r, int col) {
  return *reinterpret_cast<const float*>(tile + r * F32T<D>::RB + 16 * fswz(r, col >> 2) +
                                         4 * (col & 3));
}

// Per-lane sources of the asynchronous copies of a 32-row tile shared by NWC
// waves: lane j of copying wave w's copy i lands at tile byte (w CPW + i)
// 1 KiB + 16 j, i.e. row `row[i]`, physical chunk p, and fetches logical
// chunk p ^ (row mod 16).
template <int D, int NWC = kMfmaF32Waves>
struct F32Copy {
  static constexpr int CPW = F32T<D>::BYTES / 1024 / NWC;  // 1 KiB copies per wave per tile
  static_assert(CPW * 1024 * NWC == F32T<D>::BYTES, "tile copies split evenly over the waves");
  uint32_t off[CPW];  // byte offset from the tile's first source row
  int row[CPW];
};

template <int D, int NWC = kMfmaF32Waves>
__device__ __forceinline__ F32Copy<D, NWC> f32_copy_offsets(int64_t sr, int wave, int lane) {
  using T = F32T<D>;
  using Cp = F32Copy<D, NWC>;
  Cp t;
#pragma unroll
  for (int i = 0; i < Cp::CPW; ++i) {
    const int byte = (wave * Cp::CPW + i) * 1024 + 16 * lane;
    const int r = byte / T::RB, pc = (byte % T::RB) / 16;
    t.row[i] = r;
    t.off[i] = (uint32_t)(4 * (r * sr + 4 * fswz(r, pc)));
  }
  return t;
}

// Copy rows [r0, r0 + 32) of a [rows, D] fp32 matrix into a tile; rows at or
// past nrows (ragged last tile only, r0 < nrows) repeat row nrows - 1, whose
// contributions the callers mask.
template <int D, int NWC>
__device__ __forceinline__ void f32_issue(const F32Copy<D, NWC>& t, const float* base, int64_t sr,
                                          int r0, int nrows, char* tile, int wave) {
  constexpr int CPW = F32Copy<D, NWC>::CPW;
  const char* src = reinterpret_cast<const char*>(base + (int64_t)r0 * sr);
  char* dst = tile + wave * CPW * 1024;
  if (r0 + 32 <= nrows) {
#pragma unroll
    for (int i = 0; i < CPW; ++i) dma16(src, t.off[i], dst + i * 1024);
  } else {
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int64_t shift = min(t.row[i], nrows - 1 - r0) - t.row[i];
      dma16_at(src + t.off[i] + 4 * shift * sr, dst + i * 1024);
    }
  }
}

// Values of a 32-row tile's per-row constants (LSE log2 e, -D) for
// accumulator slot r: row 8 (r / 4) + 4 h + r % 4.
__device__ __forceinline__ void slot_consts(const float* v, int h, float (&out)[16]) {
  const f32x4* p = reinterpret_cast<const f32x4*>(v) + h;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 x = p[2 * q];
#pragma unroll
    for (int e = 0; e < 4; ++e) out[4 * q + e] = x[e];
  }
}

// Stores one 32 x 32 transposed accumulator tile (slot r: column
// 8 (r / 4) + 4 h + r % 4 of the lane's row) times `mul`.
__device__ __forceinline__ void store_row_tile(float* row, const f32x16& v, int h, float mul) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<f32x4*>(row + 8 * q + 4 * h) =
        f32x4{v[4 * q] * mul, v[4 * q + 1] * mul, v[4 * q + 2] * mul, v[4 * q + 3] * mul};
}

// Sum of the contraction over d of a row operand read from a tile (row lq)
// against this lane's register operand x (4 values per group), in two
// interleaved accumulators so consecutive products do not depend on each
// other.
// With AHEAD > 0 the tile reads run AHEAD groups ahead of the products that
// take them (one wave per SIMD at d = 128 leaves no other wave to cover LDS
// latency); AHEAD = 0 leaves the order to the compiler, for the kernel whose
// live registers leave no room for the read-ahead buffers (dK/dV).
template <int D, int AHEAD>
__device__ __forceinline__ f32x16 row_product(const char* tile, int lq, int h,
                                              const f32x4 (&x)[F32T<D>::G]) {
  f32x16 acc[2] = {};
  if constexpr (AHEAD > 0) {
    lds_mfma_pipeline<F32T<D>::G, AHEAD>(
        [&](int g) { return __builtin_bit_cast(u32x4, tile_row4<D>(tile, lq, 2 * g + h)); },
        [&](int g, const u32x4& yv) {
          const f32x4 y = __builtin_bit_cast(f32x4, yv);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e & 1] = mfma32f(y[e], x[g][e], acc[e & 1]);
        });
  } else {
#pragma unroll
    for (int g = 0; g < F32T<D>::G; ++g) {
      const f32x4 y = tile_row4<D>(tile, lq, 2 * g + h);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e & 1] = mfma32f(y[e], x[g][e], acc[e & 1]);
    }
  }
  return acc[0] + acc[1];
}

// out^T += tile^T S^T over the tile's 32 rows: product j takes tile row
// 8 (j / 4) + 4 h + j % 4 (the row of slot j) and column 32 t + lq.
template <int D, int AHEAD>
__device__ __forceinline__ void col_product(const char* tile, int lq, int h, const float (&s)[16],
                                            f32x16 (&out)[F32T<D>::DT]) {
  constexpr int DT = F32T<D>::DT;
  static_assert(DT <= 4, "one read group holds a row's DT values");
  if constexpr (AHEAD > 0) {
    lds_mfma_pipeline<16, AHEAD>(
        [&](int j) {
          const int r = 8 * (j >> 2) + 4 * h + (j & 3);
          u32x4 v = {0, 0, 0, 0};
#pragma unroll
          for (int t = 0; t < DT; ++t) v[t] = __float_as_uint(tile_at<D>(tile, r, 32 * t + lq));
          return v;
        },
        [&](int j, const u32x4& v) {
#pragma unroll
          for (int t = 0; t < DT; ++t) out[t] = mfma32f(__uint_as_float(v[t]), s[j], out[t]);
        });
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = 8 * (j >> 2) + 4 * h + (j & 3);
#pragma unroll
      for (int t = 0; t < DT; ++t) out[t] = mfma32f(tile_at<D>(tile, r, 32 * t + lq), s[j], out[t]);
    }
  }
}

// ---------------------------------------------------------------------------
// forward: workgroup = 64 queries of one head (two 32-query tiles) x the two
// halves of their key range, one wave per (tile, half); key blocks of 32.
// Splitting the key range halves the serial work of the longest rows, whose
// workgroups (the last query blocks under a causal mask) otherwise set the
// kernel's time when there are about as many workgroups as CUs.  Each half
// streams its own K / V blocks through two LDS stages; at the end the halves'
// running states (unnormalised O, row maximum, partial sums) are combined
// through LDS with the usual rescaling to the larger maximum.
// ---------------------------------------------------------------------------
constexpr int kF32FwdBM = 64;  // queries per forward workgroup

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kMfmaF32Waves, f32_mfma_occupancy<D>()) void attn_fwd_f32_mfma_kernel(AttnArgs a) {
  using T = F32T<D>;
  constexpr int BM = kF32FwdBM, BN = 32;
  static_assert(kMfmaF32Waves == 4 && BM == 64, "two query tiles x two key halves");
  __shared__ __attribute__((aligned(1024))) char smem[8 * T::BYTES];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lq = lane & 31, h = lane >> 5;
  const int half = wave >> 1, qt = wave & 1;  // key half, query tile
  char* const hs = smem + half * 4 * T::BYTES;
  auto ktile = [&](int i) { return hs + (i & 1) * T::BYTES; };
  auto vtile = [&](int i) { return hs + (2 + (i & 1)) * T::BYTES; };
  const int nqb = (a.m + BM - 1) / BM;
  int bh, qi;
  xcd_map(blockIdx.x, a.b * a.hq, nqb, bh, qi);
  const int hh = bh % a.hq, bi = bh / a.hq;
  const int qb = CAUSAL ? (nqb - 1 - qi) : qi;
  const int g = hh / a.group;
  const float* qbase = static_cast<const float*>(a.q) + bi * a.q_sb + hh * a.q_sh;
  const float* kbase = static_cast<const float*>(a.k) + bi * a.k_sb + g * a.k_sh;
  const float* vbase = static_cast<const float*>(a.v) + bi * a.v_sb + g * a.v_sh;

  const int q0 = qb * BM + qt * 32;
  const int myq = q0 + lq;
  const int kend = CAUSAL ? min(a.n, max(0, qb * BM + BM + a.diag)) : a.n;
  const int nkb = (kend + BN - 1) / BN;
  // half 0: key blocks [0, nkb / 2), half 1: [nkb / 2, nkb); every wave runs
  // the longer half's iteration count (the same barriers)
  const int nkb0 = nkb / 2;
  const int kb_begin = half ? nkb0 : 0, kb_end = half ? nkb : nkb0;
  const int nloop = nkb - nkb0;
  // blocks past this tile's last live key are skipped
  const int nkw = q0 >= a.m ? 0
                  : CAUSAL ? (q0 + 31 + a.diag < 0 ? 0 : min(nkb, (q0 + 31 + a.diag) / BN + 1))
                           : nkb;
  const F32Copy<D, 2> ck = f32_copy_offsets<D, 2>(a.k_sr, qt, lane);
  const F32Copy<D, 2> cv = f32_copy_offsets<D, 2>(a.v_sr, qt, lane);
  // block kb of this half into stage i
  auto copy = [&](int kb, int i) {
    f32_issue<D, 2>(ck, kbase, a.k_sr, kb * BN, a.n, ktile(i), qt);
    f32_issue<D, 2>(cv, vbase, a.v_sr, kb * BN, a.n, vtile(i), qt);
  };
  if (kb_begin < kb_end) copy(kb_begin, 0);

  f32x4 qf[T::G];  // Q[myq][8 g + 4 h .. + 3]
#pragma unroll
  for (int gi = 0; gi < T::G; ++gi)
    qf[gi] = myq < a.m ? *reinterpret_cast<const f32x4*>(qbase + (int64_t)myq * a.q_sr + 8 * gi + 4 * h)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
  f32x16 o[T::DT] = {};
  float m_run = -INFINITY, l_run = 0.f;
  const float cs = a.scale_log2;
  wait_vmem();
  lds_barrier();

  for (int it = 0; it < nloop; ++it) {
    const int kb = kb_begin + it;
    if (kb + 1 < kb_end) copy(kb + 1, it + 1);
    if (kb < kb_end && kb < nkw) {
      // slot r: key kb BN + 8 (r / 4) + 4 h + r % 4 of query myq
      const f32x16 sacc = row_product<D, 4>(ktile(it), lq, h, qf);
      float s[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = sacc[r];
      const int key0 = kb * BN;
      if ((CAUSAL && key0 + BN - 1 > q0 + a.diag) || key0 + BN > a.n) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 8 * (r >> 2) + 4 * h + (r & 3);
          if ((CAUSAL && key > myq + a.diag) || key >= a.n) s[r] = -INFINITY;
        }
      }
      // exponentials against the running reference m (a row maximum of
      // earlier blocks); only a block whose probabilities for some row would
      // sum to 2^32 or more, or a row with no reference yet (the exponent is
      // then +inf or NaN), takes the row maximum and may move m.  fp32 keeps
      // its relative precision at any scale, so the result is unchanged.
      float p[16], lsum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = fast_exp2(fmaf(s[r], cs, -m_run));
        lsum += p[r];
      }
      if (__ballot(!(lsum < 0x1p32f))) {
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
        mx = pair_max(mx) * cs;
        // the reference moves only when a probability would exceed 2^8
        const float m_new = mx > m_run + 8.f ? mx : m_run;
        const float m_ref = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_ref);
        const bool rescale = m_new != m_run;
        lsum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = fast_exp2(fmaf(s[r], cs, -m_ref));
          lsum += p[r];
        }
        l_run *= alpha;
        m_run = m_new;
        if (__ballot(rescale)) {
#pragma unroll
          for (int t = 0; t < T::DT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
        }
      }
      l_run += lsum;
      col_product<D, 4>(vtile(it), lq, h, p, o);
    }
    wait_vmem();
    lds_barrier();
  }

  // half 1 hands its state to half 0 through the (now free) stages:
  // per query tile, 16 DT accumulator values, the maximum and the partial sum
  // of each lane, lane-minor
  float* xs = reinterpret_cast<float*>(smem) + qt * (16 * T::DT + 2) * 64;
  if (half == 1) {
#pragma unroll
    for (int t = 0; t < T::DT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) xs[(16 * t + r) * 64 + lane] = o[t][r];
    xs[16 * T::DT * 64 + lane] = m_run;
    xs[(16 * T::DT + 1) * 64 + lane] = l_run;
  }
  lds_barrier();
  if (half == 1) return;
  {
    const float m1 = xs[16 * T::DT * 64 + lane], l1 = xs[(16 * T::DT + 1) * 64 + lane];
    const float mm = fmaxf(m_run, m1);
    // a half that saw no key contributes nothing (its maximum is -inf)
    const float f0 = m_run == -INFINITY ? 0.f : fast_exp2(m_run - mm);
    const float f1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - mm);
#pragma unroll
    for (int t = 0; t < T::DT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[t][r] = fmaf(o[t][r], f0, xs[(16 * t + r) * 64 + lane] * f1);
    l_run = fmaf(l_run, f0, l1 * f1);
    m_run = mm;
  }

  // rows that saw no key (offset causal masks): O = 0, LSE = -inf
  const float l_tot = pair_sum(l_run);
  if (myq < a.m) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* orow = static_cast<float*>(a.o_out) + bi * a.o_sb + hh * a.o_sh + (int64_t)myq * a.o_sr;
#pragma unroll
    for (int t = 0; t < T::DT; ++t) store_row_tile(orow + 32 * t, o[t], h, inv);
    if (h == 0)
      a.lse[((int64_t)bi * a.hq + hh) * a.m + myq] =
          l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// backward per-row constants: delta = -rowsum(dO * O), lse2 = LSE log2(e)
// (+inf for a row without keys, so its probabilities are exactly 0)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_prep_f32_kernel(AttnArgs a) {
  constexpr int LPR = D / 4;  // lanes per row, 4 floats each
  constexpr int RPB = 256 / LPR;
  const int tid = threadIdx.x;
  const int64_t orow = (int64_t)blockIdx.x * RPB + tid / LPR;  // rows in O's [b, m, hq] order
  const int part = tid % LPR;
  const int64_t total = (int64_t)a.b * a.hq * a.m;
  float acc = 0.f;
  int64_t row = 0;
  if (orow < total) {
    const int64_t bm = orow / a.hq;
    const int64_t hh = orow - bm * a.hq;
    const int64_t bi = bm / a.m;
    const int64_t i = bm - bi * a.m;
    row = (bi * a.hq + hh) * a.m + i;
    const int64_t off = bi * a.o_sb + hh * a.o_sh + i * a.o_sr + 4 * part;
    const f32x4 x = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.o) + off);
    const f32x4 y = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.dout) + off);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = fmaf(x[e], y[e], acc);
  }
  acc = lane_group_sum<LPR>(acc);
  if (orow < total && part == 0) {
    a.delta[row] = -acc;
    const float l = a.lse_in[row];
    a.lse2[row] = l == -INFINITY ? INFINITY : l * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dK, dV: workgroup = 64 keys of one kv head (two 32-key tiles) x the two
// halves of their steps (query blocks of 32, of every query head of the
// group), one wave per (tile, half); each half streams its own Q / dO blocks
// through two LDS stages, and half 0 adds half 1's partial dK, dV at the end
// (the split halves the serial work of the first key blocks, which see every
// query under a causal mask).
// ---------------------------------------------------------------------------
template <int D>
struct F32DkdvLds {
  static constexpr int Q = 0;
  static constexpr int DO = F32T<D>::BYTES;
  static constexpr int LSE = 2 * F32T<D>::BYTES;  // 64 floats (rows 32.. unused)
  static constexpr int DLT = LSE + 256;
  static constexpr int STAGE = DLT + 256;
};
constexpr int kF32BwdB = 64;  // keys (dK, dV) or queries (dQ) per backward workgroup

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kMfmaF32Waves, 1) void attn_dkdv_f32_mfma_kernel(AttnArgs a) {
  using T = F32T<D>;
  using L = F32DkdvLds<D>;
  constexpr int KB = kF32BwdB, QB = 32;
  static_assert(kMfmaF32Waves == 4 && KB == 64, "two key tiles x two step halves");
  constexpr int kDkdvAhead = D == 128 ? 0 : 4;  // at d = 128 the read-ahead buffers would spill
  __shared__ __attribute__((aligned(1024))) char smem[4 * L::STAGE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lq = lane & 31, h = lane >> 5;
  const int half = wave >> 1, kt = wave & 1;  // step half, key tile
  char* const hs = smem + half * 2 * L::STAGE;
  const int nkb = (a.n + KB - 1) / KB;
  int gh, kblk;
  xcd_map(blockIdx.x, a.b * a.hkv, nkb, gh, kblk);  // low key blocks (most queries) first
  const int g = gh % a.hkv, bi = gh / a.hkv;
  const int k0w = kblk * KB + kt * 32;
  const int mykey = k0w + lq;
  const bool live = k0w < a.n;
  const float cs = a.scale_log2;
  const int qb_first = CAUSAL ? max(0, kblk * KB - a.diag) / QB : 0;
  const int nqb = (a.m + QB - 1) / QB;
  const int steps_per_head = max(0, nqb - qb_first);
  const int steps = steps_per_head * a.group;
  // half 0: steps [0, steps / 2), half 1: [steps / 2, steps); every wave runs
  // the longer half's iteration count (the same barriers)
  const int s0 = steps / 2;
  const int st_begin = half ? s0 : 0, st_end = half ? steps : s0;
  const int nloop = steps - s0;

  const F32Copy<D, 2> cq = f32_copy_offsets<D, 2>(a.q_sr, kt, lane);
  const F32Copy<D, 2> co = f32_copy_offsets<D, 2>(a.o_sr, kt, lane);
  auto copy = [&](int hq_idx, int q0, char* st) {
    const float* qb = static_cast<const float*>(a.q) + bi * a.q_sb + hq_idx * a.q_sh;
    const float* ob = static_cast<const float*>(a.dout) + bi * a.o_sb + hq_idx * a.o_sh;
    f32_issue<D, 2>(cq, qb, a.q_sr, q0, a.m, st + L::Q, kt);
    f32_issue<D, 2>(co, ob, a.o_sr, q0, a.m, st + L::DO, kt);
    const int64_t r = ((int64_t)bi * a.hq + hq_idx) * a.m;
    const int i = min(q0 + lane, a.m - 1);  // lanes past the block copy a valid row, unused
    if (kt == 0) dma4_at(a.lse2 + r + i, st + L::LSE);
    else dma4_at(a.delta + r + i, st + L::DLT);
  };
  // (head, block) of this half's first step
  int hc = steps_per_head > 0 ? st_begin / steps_per_head : 0;
  int qc = st_begin - hc * steps_per_head;
  if (st_begin < st_end) copy(g * a.group + hc, (qb_first + qc) * QB, hs);

  f32x4 kf[T::G], vf[T::G];  // K, V rows of this lane's key
  {
    const float* kr = static_cast<const float*>(a.k) + bi * a.k_sb + g * a.k_sh + (int64_t)mykey * a.k_sr;
    const float* vr = static_cast<const float*>(a.v) + bi * a.v_sb + g * a.v_sh + (int64_t)mykey * a.v_sr;
#pragma unroll
    for (int gi = 0; gi < T::G; ++gi) {
      kf[gi] = mykey < a.n ? *reinterpret_cast<const f32x4*>(kr + 8 * gi + 4 * h) : f32x4{0.f, 0.f, 0.f, 0.f};
      vf[gi] = mykey < a.n ? *reinterpret_cast<const f32x4*>(vr + 8 * gi + 4 * h) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  f32x16 dk[T::DT] = {}, dv[T::DT] = {};
  wait_vmem();
  lds_barrier();

  for (int it = 0; it < nloop; ++it) {
    const int step = st_begin + it;
    int hn = hc, qn = qc;
    if (++qn == steps_per_head) {
      qn = 0;
      ++hn;
    }
    if (step + 1 < st_end) copy(g * a.group + hn, (qb_first + qn) * QB, hs + ((it + 1) & 1) * L::STAGE);
    const int q0 = (qb_first + qc) * QB;
    hc = hn, qc = qn;
    const char* st = hs + (it & 1) * L::STAGE;
    if (step < st_end && live && (!CAUSAL || q0 + QB - 1 + a.diag >= k0w)) {
      // slot r: query q0 + 8 (r / 4) + 4 h + r % 4 of key mykey
      const f32x16 sacc = row_product<D, kDkdvAhead>(st + L::Q, lq, h, kf);
      float lse2[16], ndl[16], p[16];
      slot_consts(reinterpret_cast<const float*>(st + L::LSE), h, lse2);
      slot_consts(reinterpret_cast<const float*>(st + L::DLT), h, ndl);
      const bool need_mask = (CAUSAL && q0 + a.diag < k0w + 31) || q0 + QB > a.m;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = fast_exp2(fmaf(sacc[r], cs, -lse2[r]));
        if (need_mask) {
          const int q = q0 + 8 * (r >> 2) + 4 * h + (r & 3);
          if ((CAUSAL && q + a.diag < mykey) || q >= a.m) p[r] = 0.f;
        }
      }
      col_product<D, kDkdvAhead>(st + L::DO, lq, h, p, dv);  // dV^T += dO^T P
      const f32x16 dpacc = row_product<D, kDkdvAhead>(st + L::DO, lq, h, vf);
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) ds[r] = p[r] * (dpacc[r] + ndl[r]);
      col_product<D, kDkdvAhead>(st + L::Q, lq, h, ds, dk);  // dK^T += Q^T dS
    }
    wait_vmem();
    lds_barrier();
  }

  // half 1's partial dK, dV to half 0 through the (now free) stages, lane-minor
  float* xs = reinterpret_cast<float*>(smem) + kt * (32 * T::DT) * 64;
  if (half == 1) {
#pragma unroll
    for (int t = 0; t < T::DT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        xs[(16 * t + r) * 64 + lane] = dk[t][r];
        xs[(16 * (T::DT + t) + r) * 64 + lane] = dv[t][r];
      }
  }
  lds_barrier();
  if (half == 1 || !live || mykey >= a.n) return;
#pragma unroll
  for (int t = 0; t < T::DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[t][r] += xs[(16 * t + r) * 64 + lane];
      dv[t][r] += xs[(16 * (T::DT + t) + r) * 64 + lane];
    }
  float* dvrow = static_cast<float*>(a.dv) + bi * a.v_sb + g * a.v_sh + (int64_t)mykey * a.v_sr;
  float* dkrow = static_cast<float*>(a.dk) + bi * a.k_sb + g * a.k_sh + (int64_t)mykey * a.k_sr;
#pragma unroll
  for (int t = 0; t < T::DT; ++t) {
    store_row_tile(dvrow + 32 * t, dv[t], h, 1.f);
    store_row_tile(dkrow + 32 * t, dk[t], h, a.scale);
  }
}

// ---------------------------------------------------------------------------
// dQ: workgroup = 64 queries of one query head (two 32-query tiles) x the two
// halves of their key range, one wave per (tile, half), key blocks of 32;
// half 0 adds half 1's partial dQ at the end.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kMfmaF32Waves, f32_mfma_occupancy<D>()) void attn_dq_f32_mfma_kernel(AttnArgs a) {
  using T = F32T<D>;
  constexpr int BM = kF32BwdB, BN = 32;
  static_assert(kMfmaF32Waves == 4 && BM == 64, "two query tiles x two key halves");
  constexpr int kDqAhead = D == 128 ? 4 : 2;  // two waves per SIMD at d = 64: 256 registers
  __shared__ __attribute__((aligned(1024))) char smem[8 * T::BYTES];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lq = lane & 31, h = lane >> 5;
  const int half = wave >> 1, qt = wave & 1;  // key half, query tile
  char* const hs = smem + half * 4 * T::BYTES;
  auto ktile = [&](int i) { return hs + (i & 1) * T::BYTES; };
  auto vtile = [&](int i) { return hs + (2 + (i & 1)) * T::BYTES; };
  const int nqb = (a.m + BM - 1) / BM;
  int bh, qi;
  xcd_map(blockIdx.x, a.b * a.hq, nqb, bh, qi);
  const int hh = bh % a.hq, bi = bh / a.hq;
  const int qb = CAUSAL ? (nqb - 1 - qi) : qi;
  const int g = hh / a.group;
  const float* kbase = static_cast<const float*>(a.k) + bi * a.k_sb + g * a.k_sh;
  const float* vbase = static_cast<const float*>(a.v) + bi * a.v_sb + g * a.v_sh;

  const int q0 = qb * BM + qt * 32;
  const int myq = q0 + lq;
  const bool qlive = myq < a.m;
  const int kend = CAUSAL ? min(a.n, max(0, qb * BM + BM + a.diag)) : a.n;
  const int nkb = (kend + BN - 1) / BN;
  const int nkb0 = nkb / 2;
  const int kb_begin = half ? nkb0 : 0, kb_end = half ? nkb : nkb0;
  const int nloop = nkb - nkb0;
  const F32Copy<D, 2> ck = f32_copy_offsets<D, 2>(a.k_sr, qt, lane);
  const F32Copy<D, 2> cv = f32_copy_offsets<D, 2>(a.v_sr, qt, lane);
  auto copy = [&](int kb, int i) {
    f32_issue<D, 2>(ck, kbase, a.k_sr, kb * BN, a.n, ktile(i), qt);
    f32_issue<D, 2>(cv, vbase, a.v_sr, kb * BN, a.n, vtile(i), qt);
  };
  if (kb_begin < kb_end) copy(kb_begin, 0);

  f32x4 qf[T::G], df[T::G];  // Q, dO rows of this lane's query
  {
    const float* qr = static_cast<const float*>(a.q) + bi * a.q_sb + hh * a.q_sh + (int64_t)myq * a.q_sr;
    const float* dr = static_cast<const float*>(a.dout) + bi * a.o_sb + hh * a.o_sh + (int64_t)myq * a.o_sr;
#pragma unroll
    for (int gi = 0; gi < T::G; ++gi) {
      qf[gi] = qlive ? *reinterpret_cast<const f32x4*>(qr + 8 * gi + 4 * h) : f32x4{0.f, 0.f, 0.f, 0.f};
      df[gi] = qlive ? *reinterpret_cast<const f32x4*>(dr + 8 * gi + 4 * h) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  const int64_t ridx = ((int64_t)bi * a.hq + hh) * a.m + myq;
  const float lse2 = qlive ? a.lse2[ridx] : INFINITY;
  const float ndl = qlive ? a.delta[ridx] : 0.f;
  f32x16 dq[T::DT] = {};
  const float cs = a.scale_log2;
  wait_vmem();
  lds_barrier();

  for (int it = 0; it < nloop; ++it) {
    const int kb = kb_begin + it;
    if (kb + 1 < kb_end) copy(kb + 1, it + 1);
    const int key0 = kb * BN;
    if (kb < kb_end && q0 < a.m && (!CAUSAL || key0 <= q0 + 31 + a.diag)) {
      // slot r: key key0 + 8 (r / 4) + 4 h + r % 4 of query myq
      const f32x16 sacc = row_product<D, kDqAhead>(ktile(it), lq, h, qf);
      const f32x16 dpacc = row_product<D, kDqAhead>(vtile(it), lq, h, df);
      const bool need_mask = (CAUSAL && key0 + BN - 1 > q0 + a.diag) || key0 + BN > a.n;
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = fast_exp2(fmaf(sacc[r], cs, -lse2));
        if (need_mask) {
          const int key = key0 + 8 * (r >> 2) + 4 * h + (r & 3);
          if ((CAUSAL && key > myq + a.diag) || key >= a.n) p = 0.f;
        }
        ds[r] = p * (dpacc[r] + ndl);
      }
      col_product<D, kDqAhead>(ktile(it), lq, h, ds, dq);  // dQ^T += K^T dS^T
    }
    wait_vmem();
    lds_barrier();
  }

  // half 1's partial dQ to half 0 through the (now free) stages, lane-minor
  float* xs = reinterpret_cast<float*>(smem) + qt * (16 * T::DT) * 64;
  if (half == 1) {
#pragma unroll
    for (int t = 0; t < T::DT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) xs[(16 * t + r) * 64 + lane] = dq[t][r];
  }
  lds_barrier();
  if (half == 1 || !qlive) return;
#pragma unroll
  for (int t = 0; t < T::DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[t][r] += xs[(16 * t + r) * 64 + lane];
  float* out = static_cast<float*>(a.dq) + bi * a.q_sb + hh * a.q_sh + (int64_t)myq * a.q_sr;
#pragma unroll
  for (int t = 0; t < T::DT; ++t) store_row_tile(out + 32 * t, dq[t], h, a.scale);
}

template <int D>
hipError_t fwd_d(const AttnArgs& a, hipStream_t s) {
  const int nqb = (a.m + kF32FwdBM - 1) / kF32FwdBM;
  const dim3 grid((unsigned)nqb * a.hq * a.b), block(64 * kMfmaF32Waves);
  if (a.causal)
    FAB_TIMED("attn_fwd_f32_mfma", s, hipLaunchKernelGGL((attn_fwd_f32_mfma_kernel<D, true>), grid, block, 0, s, a));
  else
    FAB_TIMED("attn_fwd_f32_mfma", s, hipLaunchKernelGGL((attn_fwd_f32_mfma_kernel<D, false>), grid, block, 0, s, a));
  return hipGetLastError();
}

template <int D>
hipError_t bwd_d(const AttnArgs& a, hipStream_t s) {
  {
    constexpr int rpb = 256 / (D / 4);
    const int64_t rows = (int64_t)a.b * a.hq * a.m;
    const dim3 gp((unsigned)((rows + rpb - 1) / rpb)), block(256);
    FAB_TIMED("attn_bwd_prep_f32", s, hipLaunchKernelGGL((attn_bwd_prep_f32_kernel<D>), gp, block, 0, s, a));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int kb = kF32BwdB;
  const dim3 gk((unsigned)((a.n + kb - 1) / kb) * a.hkv * a.b);
  const dim3 gq((unsigned)((a.m + kb - 1) / kb) * a.hq * a.b);
  const dim3 block(64 * kMfmaF32Waves);
  if (a.causal) {
    FAB_TIMED("attn_bwd_dkdv_f32_mfma", s, hipLaunchKernelGGL((attn_dkdv_f32_mfma_kernel<D, true>), gk, block, 0, s, a));
    FAB_TIMED("attn_bwd_dq_f32_mfma", s, hipLaunchKernelGGL((attn_dq_f32_mfma_kernel<D, true>), gq, block, 0, s, a));
  } else {
    FAB_TIMED("attn_bwd_dkdv_f32_mfma", s, hipLaunchKernelGGL((attn_dkdv_f32_mfma_kernel<D, false>), gk, block, 0, s, a));
    FAB_TIMED("attn_bwd_dq_f32_mfma", s, hipLaunchKernelGGL((attn_dq_f32_mfma_kernel<D, false>), gq, block, 0, s, a));
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_f32_mfma(const AttnArgs& a, int d, hipStream_t s) {
  if (d == 128) return fwd_d<128>(a, s);
  if (d == 64) return fwd_d<64>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_bwd_f32_mfma(const AttnArgs& a, int d, hipStream_t s) {
  if (d == 128) return bwd_d<128>(a, s);
  if (d == 64) return bwd_d<64>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace fab
