// Softmax attention backward, bf16 in / fp32 accumulate, on gfx950 MFMA.
//
// Gradients of L = <dO, O> for O = softmax(scale Q K^T [+ causal]) V, with the
// probabilities recomputed from the saved log-sum-exp instead of being stored
// (rematerialisation over storage: "AutoSP", section 2.B):
//   P = exp(scale Q K^T - LSE), dP = dO V^T, D_i = rowsum(dO_i * O_i),
//   dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO.
//
// Deterministic two-kernel schedule (no atomics):
//  * attn_dkdv_bf16_kernel: one workgroup per 128 keys of one kv head, in four
//    32-key groups each served by a pair of waves with split roles (P / dV and
//    dP / dS / dK).  K and V stay in registers; query blocks of 64 (and all
//    query heads of the group) stream through a three-stage LDS ring, copied
//    two steps ahead.  dK^T and dV^T accumulate in registers.
//  * attn_dq_bf16_kernel: one workgroup per 32 x NW queries (NW waves, 8 by
//    default) of one query head.  Q, dO, LSE and D stay in registers; key
//    blocks of 64 stream through LDS (K and V natural, K read transposed).
//    dQ^T accumulates in registers.  S and dP are recomputed here rather than
//    exchanged.
// MFMA layout conventions are those of the forward kernel (perm_row order
// makes accumulator slots contiguous along the lane's row).
#include "fab_device.h"
#include "fab_internal.h"

namespace fab {
namespace {

template <int D>
struct BwdCfg {
  static constexpr int CPR = D / 8;          // 16-byte chunks per row
  static constexpr int RB = D * 2;           // row bytes (no padding)
  static constexpr int TILE = 64;            // rows of a streamed tile
  static constexpr int TBYTES = TILE * RB;   // bytes of one tile
  static constexpr int RPI = 1024 / RB;      // rows per 1 KiB async copy
  static constexpr int DT = D / 32;
  static constexpr int DC = D / 16;
};

// Streamed 64-row tiles live in LDS with tile row x at LDS row
// perm_row_inv(x % 32) + 32 (x / 32) (so MFMA row r of a 32-row group reads
// tile row perm_row(r)), and logical 16-byte chunk c of LDS row r = 4a + b
// (b = r % 4, a = (r / 4) % 4) at physical chunk c ^ (4 b + a).  The XOR value
// differs across any 16 aligned rows (conflict-free 16-byte row reads) and its
// upper two bits differ across 4 aligned rows (conflict-free transposing reads
// of 4 rows x 64 bytes).
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  return c ^ ((((r & 3) << 2) | ((r >> 2) & 3)) & (BwdCfg<D>::CPR - 1));
}
__device__ __forceinline__ int lds_row_of(int x) { return perm_row_inv(x & 31) + (x & ~31); }

// Async copy of rows [r0, r0 + 64) of a [rows, D] matrix (row stride sr) into
// a tile as above, shared by NW waves: each does CPW = TBYTES / 1 KiB / NW
// 1 KiB copies.  Lane j of wave copy i writes LDS row
// r = (w * CPW + i) * RPI + j / CPR, physical chunk j % CPR; its byte offset
// inside the source block is fixed for the whole kernel and precomputed.
template <int D, int NW>
struct TileOffsets {
  static constexpr int CPW = BwdCfg<D>::TBYTES / 1024 / NW;
  static_assert(CPW * NW * 1024 == BwdCfg<D>::TBYTES, "tile copies must split evenly");
  uint32_t off[CPW];  // byte offset of this lane's 16 bytes within a block
};

// Tile row copied by lane `lane` of wave `wave` in copy i.
template <int D, int NW>
__device__ __forceinline__ int tile_row_of_copy(int wave, int lane, int i) {
  using C = BwdCfg<D>;
  const int r = (wave * TileOffsets<D, NW>::CPW + i) * C::RPI + lane / C::CPR;
  return perm_row(r & 31) + (r & ~31);
}

template <int D, int NW>
__device__ __forceinline__ TileOffsets<D, NW> tile_offsets(int64_t sr, int wave, int lane) {
  using C = BwdCfg<D>;
  using T = TileOffsets<D, NW>;
  T t;
#pragma unroll
  for (int i = 0; i < T::CPW; ++i) {
    const int r = (wave * T::CPW + i) * C::RPI + lane / C::CPR;
    t.off[i] = (uint32_t)(2 * (tile_row_of_copy<D, NW>(wave, lane, i) * sr +
                               8 * swz<D>(r, lane % C::CPR)));
  }
  return t;
}

// Rows at or past nrows (ragged last tile only) are clamped to nrows - 1;
// callers mask them.
template <int D, int NW>
__device__ __forceinline__ void issue_tile(const TileOffsets<D, NW>& t, const uint16_t* base,
                                           int64_t sr, int r0, int nrows, char* dst, int wave,
                                           int lane) {
  using C = BwdCfg<D>;
  using T = TileOffsets<D, NW>;
  const char* b = reinterpret_cast<const char*>(base + (int64_t)r0 * sr);
  char* d = dst + wave * T::CPW * 1024;
  if (r0 + C::TILE <= nrows) {
#pragma unroll
    for (int i = 0; i < T::CPW; ++i) dma16(b, t.off[i], d + i * 1024);
  } else {
#pragma unroll
    for (int i = 0; i < T::CPW; ++i) {
      const int x = tile_row_of_copy<D, NW>(wave, lane, i);
      const int64_t shift = min(x, nrows - 1 - r0) - x;
      dma16_at(b + t.off[i] + 2 * shift * sr, d + i * 1024);
    }
  }
}

// MFMA operand with rows = tile rows (32 sb + perm_row(l % 32)) and k = the
// 16 columns 16 c .. 16 c + 15 (this lane: columns 16 c + 8 (l / 32) + 0..7).
template <int D>
__device__ __forceinline__ u32x4 read_nat(const char* tile, int sb, int c, int lq, int lg) {
  const int r = 32 * sb + lq;
  return lds16(tile + r * BwdCfg<D>::RB + 16 * swz<D>(r, 2 * c + lg));
}

// Transposed MFMA operand: rows = columns d = 32 t + perm_row(l % 32), k = tile
// rows 32 sb + 16 (l / 32) + 8 c + e, e = 0..7, read with ds_read_b64_tr_b16
// (within a 16-lane group, lane i gets element i % 4 of the 8 bytes that lane
// 4 j + i / 4 addresses, for j = 0..3).  tr_d / tr_row: this lane's column
// offset D_u = 16 (u%2) + 8 (g%2) + 4 (u/2), u = (l%16) % 4, and row (l%16)/4.
template <int D>
__device__ __forceinline__ u32x4 read_tr(const char* tile, int t, int sb, int c, int lg,
                                         int tr_d, int tr_row) {
  using C = BwdCfg<D>;
  const int dcol = 32 * t + tr_d;
  const int cbyte = 2 * (dcol & 7);
  const int x0 = 32 * sb + 16 * lg + 8 * c + tr_row;
  const int r0 = lds_row_of(x0), r1 = lds_row_of(x0 + 4);
  const u32x2 lo = lds_tr8(tile + r0 * C::RB + 16 * swz<D>(r0, dcol >> 3) + cbyte);
  const u32x2 hi = lds_tr8(tile + r1 * C::RB + 16 * swz<D>(r1, dcol >> 3) + cbyte);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// 64 consecutive fp32 values (clamped at `count`) into LDS, one wave.
__device__ __forceinline__ void issue_vec64(const float* src, int i0, int count, char* dst,
                                            int lane) {
  const int i = min(i0 + lane, count - 1);
  dma4_at(src + i, dst);
}

// ---------------------------------------------------------------------------
// dK, dV: workgroup = 128 keys of one kv head in 4 groups of 32, each group
// served by a pair of waves with split roles, so that each wave's registers
// (one 32-key accumulator, one operand set) leave room for two waves per SIMD:
//  * P wave (waves 0-3): holds K; S = Q K^T, P = exp2(S scale log2e - LSE
//    log2e); hands P (bf16, as its dV products take it) to its partner
//    through LDS; dV^T += dO^T P.
//  * dS wave (waves 4-7): holds V; dP - D = dO V^T - D; dS = P (dP - D) with
//    the bf16 P; dK^T += Q^T dS.
// Query blocks of 64 (all query heads of the group) stream through three LDS
// stages, copied two steps ahead (Q by the P waves, dO and the row constants by
// the dS waves); each step has two barriers: P written -> P read, and end of
// step (stage and P buffer released).
// ---------------------------------------------------------------------------
constexpr int kDkdvWaves = 8;

template <int D>
struct DkdvLds {
  static constexpr int Q = 0;                          // per stage
  static constexpr int DO = BwdCfg<D>::TBYTES;
  static constexpr int LSE = 2 * BwdCfg<D>::TBYTES;    // LSE * log2(e), 64 floats
  static constexpr int DLT = LSE + 256;                // -D, 64 floats
  static constexpr int STAGE = DLT + 256;
  static constexpr int STAGES = 3;                     // steps s, s + 1, s + 2 in flight
  static constexpr int PX = STAGES * STAGE;            // P exchange: [group][sq][c][lane] 8 x bf16
  static constexpr int PX_GROUP = 2 * 2 * 64 * 16;     // 4 KiB per 32-key group
  static constexpr int BYTES = PX + 4 * PX_GROUP;
};

// The Q tile of one step (copied by the P waves, NW of them) ...
template <int D, int NW>
__device__ __forceinline__ void dkdv_issue_q(const AttnArgs& a, const TileOffsets<D, NW>& tq,
                                             int bi, int h, int q0, char* st, int wave, int lane) {
  using L = DkdvLds<D>;
  const uint16_t* qb = static_cast<const uint16_t*>(a.q) + bi * a.q_sb + h * a.q_sh;
  issue_tile<D, NW>(tq, qb, a.q_sr, q0, a.m, st + L::Q, wave, lane);
}
// ... and its dO tile, LSE log2(e) and -D rows (by the dS waves: copying waves
// 0 and 1 issue one vector copy more than the others).
template <int D, int NW>
__device__ __forceinline__ void dkdv_issue_o(const AttnArgs& a, const TileOffsets<D, NW>& to,
                                             int bi, int h, int q0, char* st, int wave, int lane) {
  using L = DkdvLds<D>;
  const uint16_t* ob = static_cast<const uint16_t*>(a.dout) + bi * a.o_sb + h * a.o_sh;
  issue_tile<D, NW>(to, ob, a.o_sr, q0, a.m, st + L::DO, wave, lane);
  const int64_t r = ((int64_t)bi * a.hq + h) * a.m;
  if (wave == 0) issue_vec64(a.lse2 + r, q0, a.m, st + L::LSE, lane);
  if (wave == 1) issue_vec64(a.delta + r, q0, a.m, st + L::DLT, lane);
}

// Accumulator slot r of the S / dP tiles of query sub-block sq holds query
// q0 + 32 sq + 16 (l / 32) + r for the lane's key k0 + l % 32.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void attn_dkdv_bf16_kernel(AttnArgs a) {
  using C = BwdCfg<D>;
  using L = DkdvLds<D>;
  // Copies go out at the L2 -> CU rate and hold up the wave that issues them,
  // and an LDS write waits while copies are going out.  Three stages hold
  // steps s, s + 1 and s + 2: the P waves copy the Q tile of step s + 2 after
  // their dV products (in the slack before the second barrier, their P writes
  // long done), the dS waves copy its dO tile and row constants at the start
  // of step s; each wave then waits only for its copies of step s + 1.
  constexpr int CW = kDkdvWaves / 2;
  using TO = TileOffsets<D, CW>;
  constexpr int kCopiesP = TO::CPW;  // Q tile copies per P wave and step
  __shared__ __attribute__((aligned(1024))) char smem[L::BYTES];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lq = lane & 31, lg = lane >> 5;
  const int l16 = lane & 15, g16 = lane >> 4;
  const int tr_d = 16 * (l16 & 1) + 8 * (g16 & 1) + 4 * ((l16 >> 1) & 1);
  const int tr_row = l16 >> 2;
  const bool p_role = wave < 4;
  const int kg = wave & 3;  // 32-key group

  // causal: low key blocks see the most queries, so they go first (see
  // xcd_map for the XCD-aware order)
  const int nkb = (a.n + kAttnBwdKB - 1) / kAttnBwdKB;
  int gh, kblk;
  xcd_map(blockIdx.x, a.b * a.hkv, nkb, gh, kblk);
  const int g = gh % a.hkv, bi = gh / a.hkv;
  const int k0w = kblk * kAttnBwdKB + kg * 32;
  const int mykey = k0w + lq;

  const float cs = a.scale_log2;
  // first query block holding a query that sees the workgroup's first key
  const int qb_first = CAUSAL ? max(0, kblk * kAttnBwdKB - a.diag) / C::TILE : 0;
  const int nqb = (a.m + C::TILE - 1) / C::TILE;
  const int steps_per_head = max(0, nqb - qb_first);
  const int steps = steps_per_head * a.group;
  const bool group_live = k0w < a.n;
  const int cw = wave % CW;  // copy index within the role
  const TO tofs = tile_offsets<D, CW>(p_role ? a.q_sr : a.o_sr, cw, lane);
  // steps 0 and 1 up front
  auto issue_step = [&](int hh, int qq, int stage) {
    char* st = smem + stage * L::STAGE;
    if (p_role) dkdv_issue_q<D, CW>(a, tofs, bi, g * a.group + hh, (qb_first + qq) * C::TILE, st, cw, lane);
    else dkdv_issue_o<D, CW>(a, tofs, bi, g * a.group + hh, (qb_first + qq) * C::TILE, st, cw, lane);
  };
  if (steps > 0) issue_step(0, 0, 0);
  if (steps > 1) issue_step(steps_per_head > 1 ? 0 : 1, steps_per_head > 1 ? 1 : 0, 1);

  // this wave's operand: K (P wave) or V (dS wave) rows of its 32 keys
  u32x4 kv[C::DC];
  {
    const uint16_t* base =
        p_role ? static_cast<const uint16_t*>(a.k) + bi * a.k_sb + g * a.k_sh + (int64_t)mykey * a.k_sr
               : static_cast<const uint16_t*>(a.v) + bi * a.v_sb + g * a.v_sh + (int64_t)mykey * a.v_sr;
#pragma unroll
    for (int c = 0; c < C::DC; ++c)
      kv[c] = mykey < a.n ? ldg16(base + 16 * c + 8 * lg) : u32x4{0, 0, 0, 0};
  }
  f32x16 acc[C::DT];  // dV^T (P wave) or dK^T (dS wave), unscaled
#pragma unroll
  for (int t = 0; t < C::DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  u32x4* px = reinterpret_cast<u32x4*>(smem + L::PX + kg * L::PX_GROUP) + lane;
  wait_vmem();
  lds_barrier();

  // The two roles run separate copies of the step loop (same barriers per
  // step), so each loop keeps only its own role's invariants in registers.
  // Step s covers query block qb_first + s % steps_per_head of query head
  // g * group + s / steps_per_head; the loops advance (head, block) counters
  // instead of dividing, for this step and for step s + 2.
  auto advance = [&](int& hh, int& qq) {
    if (++qq == steps_per_head) {
      qq = 0;
      ++hh;
    }
  };
  int h2 = 0, q2 = 0;  // (head, block) of step + 2
  advance(h2, q2);
  advance(h2, q2);
  if (p_role) {
    int hc = 0, qc = 0;  // (head, block) of this step
    int sc = 0;          // stage of this step
    for (int step = 0; step < steps; ++step) {
      const int q0 = (qb_first + qc) * C::TILE;
      const char* st = smem + sc * L::STAGE;
      const int s2 = sc == 0 ? 2 : sc - 1;  // stage of step + 2
      // A key group skips a query block when every query precedes all its keys.
      const bool work = group_live && (!CAUSAL || q0 + C::TILE - 1 + a.diag >= k0w);
      u32x4 pb[2][2];
      if (work) {
        const bool need_mask = (CAUSAL && q0 + a.diag < k0w + 31) || q0 + C::TILE > a.m;
        // S of both query sub-blocks at raised wave priority, so the P wave
        // gets the MFMA pipe ahead of its partner's dP products; one
        // straight-line phase per mask case (and the LSE read up front), so the
        // first sub-block's exponentials can be scheduled between the second
        // sub-block's S products
        auto phase1 = [&]<bool MASK>() {
          f32x16 s[2];
#pragma unroll
          for (int sq = 0; sq < 2; ++sq)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[sq][r] = 0.f;
          // LSE of both halves first: the exponentials then wait on nothing but S
          f32x4 lse[2][4];
#pragma unroll
          for (int sq = 0; sq < 2; ++sq)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              lse[sq][j] = reinterpret_cast<const f32x4*>(st + L::LSE)[8 * sq + 4 * lg + j];
          __builtin_amdgcn_s_setprio(2);
          lds_mfma_pipeline<C::DC, 3>(
              [&](int i) { return read_nat<D>(st + L::Q, 0, i, lq, lg); },
              [&](int i, const u32x4& x) { s[0] = mfma32(x, kv[i], s[0]); });
          lds_mfma_pipeline<C::DC, 3>(
              [&](int i) { return read_nat<D>(st + L::Q, 1, i, lq, lg); },
              [&](int i, const u32x4& x) { s[1] = mfma32(x, kv[i], s[1]); });
#pragma unroll
          for (int sq = 0; sq < 2; ++sq) {
            if constexpr (MASK) {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int q = q0 + 32 * sq + 16 * lg + r;
                if ((CAUSAL && q + a.diag < mykey) || q >= a.m) s[sq][r] = -INFINITY;
              }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const f32x4 lse2 = lse[sq][j];
              f32x4 p;
#pragma unroll
              for (int e = 0; e < 4; ++e) p[e] = fast_exp2(fmaf(s[sq][4 * j + e], cs, -lse2[e]));
              pb[sq][j >> 1][2 * (j & 1)] = pack_bf16(p[0], p[1]);
              pb[sq][j >> 1][2 * (j & 1) + 1] = pack_bf16(p[2], p[3]);
            }
            // P goes to the partner in the bf16 form the dV products use
            px[(2 * sq) * 64] = pb[sq][0];
            px[(2 * sq + 1) * 64] = pb[sq][1];
          }
          __builtin_amdgcn_s_setprio(0);
        };
        if (need_mask) phase1.template operator()<true>();
        else phase1.template operator()<false>();
      }
      lds_barrier();  // P visible to the dS waves
      if (work) {
        // operand i: query sub-block i / (2 DT), output tile (i / 2) % DT, chunk i % 2
        lds_mfma_pipeline<4 * C::DT, 6>(
            [&](int i) {
              return read_tr<D>(st + L::DO, (i / 2) % C::DT, i / (2 * C::DT), i % 2, lg, tr_d, tr_row);
            },
            [&](int i, const u32x4& x) {
              acc[(i / 2) % C::DT] = mfma32(x, pb[i / (2 * C::DT)][i % 2], acc[(i / 2) % C::DT]);
            });
      }
      if (step + 2 < steps) {
        issue_step(h2, q2, s2);
        wait_copies<kCopiesP>();  // step + 1's Q tile; step + 2's stays in flight
      } else {
        wait_copies<0>();
      }
      lds_barrier();
      advance(hc, qc);
      advance(h2, q2);
      sc = sc == 2 ? 0 : sc + 1;
    }
  } else {
    int hc = 0, qc = 0;  // (head, block) of this step
    int sc = 0;          // stage of this step
    for (int step = 0; step < steps; ++step) {
      const int q0 = (qb_first + qc) * C::TILE;
      const char* st = smem + sc * L::STAGE;
      const bool pf = step + 2 < steps;
      if (pf) issue_step(h2, q2, sc == 0 ? 2 : sc - 1);
      const bool work = group_live && (!CAUSAL || q0 + C::TILE - 1 + a.diag >= k0w);
      f32x16 dp[2];
      if (work) {
#pragma unroll
        for (int sq = 0; sq < 2; ++sq) {
          const f32x4* nd = reinterpret_cast<const f32x4*>(st + L::DLT) + 8 * sq + 4 * lg;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x4 x = nd[j];
#pragma unroll
            for (int e = 0; e < 4; ++e) dp[sq][4 * j + e] = x[e];
          }
          lds_mfma_pipeline<C::DC, 4>(
              [&](int c) { return read_nat<D>(st + L::DO, sq, c, lq, lg); },
              [&](int c, const u32x4& x) { dp[sq] = mfma32(x, kv[c], dp[sq]); });
        }
      }
      lds_barrier();  // P from the partner wave
      if (work) {
#pragma unroll
        for (int sq = 0; sq < 2; ++sq) {
          // dS = P (dP - D) with the partner's bf16 P; slot pair (8 c + 2 w,
          // 8 c + 2 w + 1) in word w of chunk c
          u32x4 db[2];
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const u32x4 pv = px[(2 * sq + c) * 64];
#pragma unroll
            for (int w = 0; w < 4; ++w)
              db[c][w] = pack_bf16(bf16_lo(pv[w]) * dp[sq][8 * c + 2 * w],
                                   bf16_hi(pv[w]) * dp[sq][8 * c + 2 * w + 1]);
          }
          // raised priority while issuing dK, as for dQ (the dS wave has just
          // finished its VALU work; its partner's dV products wait)
          __builtin_amdgcn_s_setprio(2);
          lds_mfma_pipeline<2 * C::DT, 3>(
              [&](int i) { return read_tr<D>(st + L::Q, i / 2, sq, i % 2, lg, tr_d, tr_row); },
              [&](int i, const u32x4& x) { acc[i / 2] = mfma32(x, db[i % 2], acc[i / 2]); });
          __builtin_amdgcn_s_setprio(0);
        }
      }
      // step + 1's dO tile and row constants; step + 2's stay in flight
      if (!pf) wait_copies<0>();
      else if (cw < 2) wait_copies<kCopiesP + 1>();
      else wait_copies<kCopiesP>();
      lds_barrier();
      advance(hc, qc);
      advance(h2, q2);
      sc = sc == 2 ? 0 : sc + 1;
    }
  }

  if (!group_live || mykey >= a.n) return;
  const float osc = p_role ? 1.f : a.scale;
  uint16_t* row = p_role ? static_cast<uint16_t*>(a.dv) + bi * a.v_sb + g * a.v_sh + (int64_t)mykey * a.v_sr
                         : static_cast<uint16_t*>(a.dk) + bi * a.k_sb + g * a.k_sh + (int64_t)mykey * a.k_sr;
  row += 16 * lg;
#pragma unroll
  for (int t = 0; t < C::DT; ++t) {
    u32x4 lo, hi;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      lo[w] = pack_bf16(acc[t][2 * w] * osc, acc[t][2 * w + 1] * osc);
      hi[w] = pack_bf16(acc[t][8 + 2 * w] * osc, acc[t][8 + 2 * w + 1] * osc);
    }
    stg16(row + 32 * t, lo);
    stg16(row + 32 * t + 8, hi);
  }
}

// ---------------------------------------------------------------------------
// dQ: workgroup = NW waves x 32 QT queries of one query head; key blocks of 64
// stream through two LDS stages (K and V tiles; K^T is read transposed).
// ---------------------------------------------------------------------------
template <int D>
struct DqStage {
  static constexpr int K = 0;
  static constexpr int V = BwdCfg<D>::TBYTES;
  static constexpr int BYTES = 2 * BwdCfg<D>::TBYTES;
};

// One 64-key block against this wave's 32 QT queries.  Accumulator slot r of
// the S / dP tiles holds key key0 + 32 sb + 16 (l / 32) + r for query myq[qt].
// need_mask (wave-uniform; diagonal or ragged blocks): masked scores are set
// to -inf in one uniform branch, so full blocks pay nothing for masking.
// ndt[qt]: -D of query myq[qt] in all 16 slots; the dP products start from
// that tile, so dP - D comes out of the MFMAs (one add per element fewer).
template <int D, bool CAUSAL, int QT>
__device__ __forceinline__ void dq_block(const char* st, const u32x4 (&qf)[QT][BwdCfg<D>::DC],
                                         const u32x4 (&df)[QT][BwdCfg<D>::DC],
                                         f32x16 (&dq)[QT][BwdCfg<D>::DT], const int (&myq)[QT],
                                         const float (&lse2)[QT], const f32x16 (&ndt)[QT],
                                         bool need_mask, int key0, int n, int diag, float cs, int lq,
                                         int lg, int tr_d, int tr_row) {
  using C = BwdCfg<D>;
  using S = DqStage<D>;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    f32x16 s[QT], dp[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[qt][r] = 0.f;
      dp[qt] = ndt[qt];
    }
    // operand i: d chunk c = i / 2 of K (i even, for S) or V (i odd, for dP)
    auto kv_read = [&](int i) { return read_nat<D>(st + (i % 2 ? S::V : S::K), sb, i / 2, lq, lg); };
    if constexpr (QT == 1) {
      lds_mfma_pipeline<2 * C::DC, 3>(kv_read, [&](int i, const u32x4& x) {
        if (i % 2) dp[0] = mfma32(x, df[0][i / 2], dp[0]);
        else s[0] = mfma32(x, qf[0][i / 2], s[0]);
      });
    } else {
#pragma unroll
      for (int i = 0; i < 2 * C::DC; ++i) {
        const u32x4 x = kv_read(i);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          if (i % 2) dp[qt] = mfma32(x, df[qt][i / 2], dp[qt]);
          else s[qt] = mfma32(x, qf[qt][i / 2], s[qt]);
        }
      }
    }
    if (need_mask) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * sb + 16 * lg + r;
          if ((CAUSAL && key > myq[qt] + diag) || key >= n) s[qt][r] = -INFINITY;
        }
    }
    u32x4 db[QT][2];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(s[qt][r], cs, -lse2[qt]));
        ds[r] = p * dp[qt][r];
      }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int w = 0; w < 4; ++w) db[qt][c][w] = pack_bf16(ds[8 * c + 2 * w], ds[8 * c + 2 * w + 1]);
    }
    // operand i: output tile t = i % DT, key chunk c = i / DT
    auto kt_read = [&](int i) { return read_tr<D>(st + S::K, i % C::DT, sb, i / C::DT, lg, tr_d, tr_row); };
    if constexpr (QT == 1) {
      // raised wave priority while issuing dQ: the wave that has finished its
      // dS gets the MFMA pipe first, so the two waves of a SIMD drift out of
      // phase and one's dS work overlaps the other's products
      __builtin_amdgcn_s_setprio(2);
      lds_mfma_pipeline<2 * C::DT, 3>(kt_read, [&](int i, const u32x4& x) {
        dq[0][i % C::DT] = mfma32(x, db[0][i / C::DT], dq[0][i % C::DT]);
      });
      __builtin_amdgcn_s_setprio(0);
    } else {
#pragma unroll
      for (int i = 0; i < 2 * C::DT; ++i) {
        const u32x4 x = kt_read(i);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) dq[qt][i % C::DT] = mfma32(x, db[qt][i / C::DT], dq[qt][i % C::DT]);
      }
    }
  }
}

// SAME: K and V have equal row strides, so one set of copy offsets serves both.
template <int D, bool CAUSAL, int QT, bool SAME>
__global__ __launch_bounds__(64 * kAttnDqWaves, QT == 1 ? 8 / kAttnDqWaves : 1) void
attn_dq_bf16_kernel(AttnArgs a) {
  using C = BwdCfg<D>;
  using S = DqStage<D>;
  constexpr int NW = kAttnDqWaves;
  constexpr int BM = 32 * NW * QT;
  __shared__ __attribute__((aligned(1024))) char smem[2 * S::BYTES];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lq = lane & 31, lg = lane >> 5;
  const int l16 = lane & 15, g16 = lane >> 4;
  const int tr_d = 16 * (l16 & 1) + 8 * (g16 & 1) + 4 * ((l16 >> 1) & 1);
  const int tr_row = l16 >> 2;

  const int nqb = (a.m + BM - 1) / BM;
  int bh, qi;
  xcd_map(blockIdx.x, a.b * a.hq, nqb, bh, qi);
  const int h = bh % a.hq, bi = bh / a.hq;
  const int qb = CAUSAL ? (nqb - 1 - qi) : qi;
  const int g = h / a.group;

  const int q0 = qb * BM + wave * 32 * QT;
  const bool wave_live = q0 < a.m;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + bi * a.k_sb + g * a.k_sh;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + bi * a.v_sb + g * a.v_sh;
  const int kend = CAUSAL ? min(a.n, max(0, qb * BM + BM + a.diag)) : a.n;
  const int nkb = (kend + C::TILE - 1) / C::TILE;
  const TileOffsets<D, NW> tk = tile_offsets<D, NW>(a.k_sr, wave, lane);
  const TileOffsets<D, NW> tv = SAME ? tk : tile_offsets<D, NW>(a.v_sr, wave, lane);
  issue_tile<D, NW>(tk, kbase, a.k_sr, 0, a.n, smem + S::K, wave, lane);
  issue_tile<D, NW>(tv, vbase, a.v_sr, 0, a.n, smem + S::V, wave, lane);

  const uint16_t* qbase = static_cast<const uint16_t*>(a.q) + bi * a.q_sb + h * a.q_sh;
  const uint16_t* obase = static_cast<const uint16_t*>(a.dout) + bi * a.o_sb + h * a.o_sh;
  int myq[QT];
  u32x4 qf[QT][C::DC], df[QT][C::DC];
  float lse2[QT];   // LSE * log2(e) of the lane's query
  f32x16 ndt[QT];  // its -D, in every slot
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    myq[qt] = q0 + 32 * qt + lq;
    const bool live = myq[qt] < a.m;
#pragma unroll
    for (int c = 0; c < C::DC; ++c) {
      qf[qt][c] = live ? ldg16(qbase + (int64_t)myq[qt] * a.q_sr + 16 * c + 8 * lg)
                       : u32x4{0, 0, 0, 0};
      df[qt][c] = live ? ldg16(obase + (int64_t)myq[qt] * a.o_sr + 16 * c + 8 * lg)
                       : u32x4{0, 0, 0, 0};
    }
    const int64_t ridx = ((int64_t)bi * a.hq + h) * a.m + myq[qt];
    lse2[qt] = live ? a.lse2[ridx] : INFINITY;
    const float ndl = live ? a.delta[ridx] : 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) ndt[qt][r] = ndl;
  }
  f32x16 dq[QT][C::DT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int t = 0; t < C::DT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) dq[qt][t][r] = 0.f;
  const float cs = a.scale_log2;
  wait_vmem();
  lds_barrier();

  for (int kb = 0; kb < nkb; ++kb) {
    if (kb + 1 < nkb) {
      char* nst = smem + ((kb + 1) & 1) * S::BYTES;
      issue_tile<D, NW>(tk, kbase, a.k_sr, (kb + 1) * C::TILE, a.n, nst + S::K, wave, lane);
      issue_tile<D, NW>(tv, vbase, a.v_sr, (kb + 1) * C::TILE, a.n, nst + S::V, wave, lane);
    }
    const char* st = smem + (kb & 1) * S::BYTES;
    const int key0 = kb * C::TILE;
    const bool wave_work = wave_live && (!CAUSAL || key0 <= q0 + 32 * QT - 1 + a.diag);
    if (wave_work) {
      const bool need_mask = (CAUSAL && key0 + C::TILE - 1 > q0 + a.diag) || key0 + C::TILE > a.n;
      dq_block<D, CAUSAL, QT>(st, qf, df, dq, myq, lse2, ndt, need_mask, key0, a.n, a.diag, cs,
                              lq, lg, tr_d, tr_row);
    }
    wait_vmem();
    lds_barrier();
  }

#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    if (myq[qt] >= a.m) continue;
    uint16_t* out = static_cast<uint16_t*>(a.dq) + bi * a.q_sb + h * a.q_sh +
                    (int64_t)myq[qt] * a.q_sr + 16 * lg;
#pragma unroll
    for (int t = 0; t < C::DT; ++t) {
      u32x4 lo, hi;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        lo[w] = pack_bf16(dq[qt][t][2 * w] * a.scale, dq[qt][t][2 * w + 1] * a.scale);
        hi[w] = pack_bf16(dq[qt][t][8 + 2 * w] * a.scale, dq[qt][t][8 + 2 * w + 1] * a.scale);
      }
      stg16(out + 32 * t, lo);
      stg16(out + 32 * t + 8, hi);
    }
  }
}

// ---------------------------------------------------------------------------
// Preprocessing, one row per LPR lanes (16 bytes of dO and O each):
// delta[row] = -rowsum(dO * O) (fp32, from the bf16 values) and
// lse2[row] = LSE * log2(e), the two per-query constants both kernels use.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_prep_bf16_kernel(AttnArgs a) {
  constexpr int LPR = D * 2 / 16;
  constexpr int RPB = 256 / LPR;
  const int tid = threadIdx.x;
  // rows taken in O's [b, m, hq] order, so a workgroup streams contiguous O
  // and dO (the 4-byte results, in [b, hq, m] order, are the scattered part)
  const int64_t orow = (int64_t)blockIdx.x * RPB + tid / LPR;
  const int part = tid % LPR;
  const int64_t total = (int64_t)a.b * a.hq * a.m;
  float acc = 0.f;
  int64_t row = 0;  // [b, hq, m] index of the result
  if (orow < total) {
    int64_t i, h, bi;
    if (a.rows_small) {
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
    row = (bi * a.hq + h) * a.m + i;
    const int64_t off = bi * a.o_sb + h * a.o_sh + i * a.o_sr + part * 8;
    const u32x4 x = ldg16(static_cast<const uint16_t*>(a.o) + off);
    const u32x4 y = ldg16(static_cast<const uint16_t*>(a.dout) + off);
#pragma unroll
    for (int w = 0; w < 4; ++w)
      acc += bf16_lo(x[w]) * bf16_lo(y[w]) + bf16_hi(x[w]) * bf16_hi(y[w]);
  }
  acc = lane_group_sum<LPR>(acc);
  if (orow < total && part == 0) {
    a.delta[row] = -acc;
    // a row without keys (LSE = -inf) gets +inf, so its P = exp2(S - inf) = 0
    const float l = a.lse_in[row];
    a.lse2[row] = l == -INFINITY ? INFINITY : l * kLog2e;
  }
}

template <int D>
hipError_t bwd_d(const AttnArgs& a, hipStream_t s) {
  const dim3 block(256);
  {
    constexpr int rpb = 256 / (D * 2 / 16);
    const int64_t rows = (int64_t)a.b * a.hq * a.m;
    const dim3 gp((unsigned)((rows + rpb - 1) / rpb));
    FAB_TIMED("attn_bwd_prep", s, hipLaunchKernelGGL((attn_bwd_prep_bf16_kernel<D>), gp, block, 0, s, a));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  constexpr int QT = kAttnBwdQT;
  const int nkb = (a.n + kAttnBwdKB - 1) / kAttnBwdKB;
  const int nqb = (a.m + kAttnBwdBM - 1) / kAttnBwdBM;
  const dim3 gk((unsigned)nkb * a.hkv * a.b), gq((unsigned)nqb * a.hq * a.b);
  const bool same_kv = a.k_sr == a.v_sr;
#define FAB_DKDV(C) FAB_TIMED("attn_bwd_dkdv_bf16", s, hipLaunchKernelGGL((attn_dkdv_bf16_kernel<D, C>), gk, dim3(64 * kDkdvWaves), 0, s, a))
#define FAB_DQ(C, S) FAB_TIMED("attn_bwd_dq_bf16", s, hipLaunchKernelGGL((attn_dq_bf16_kernel<D, C, QT, S>), gq, dim3(64 * kAttnDqWaves), 0, s, a))
  if (a.causal) {
    FAB_DKDV(true);
    if (same_kv) FAB_DQ(true, true); else FAB_DQ(true, false);
  } else {
    FAB_DKDV(false);
    if (same_kv) FAB_DQ(false, true); else FAB_DQ(false, false);
  }
#undef FAB_DKDV
#undef FAB_DQ
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd_bf16(const AttnArgs& a, int d, hipStream_t s) {
  if (d == 128) return bwd_d<128>(a, s);
  if (d == 64) return bwd_d<64>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace fab
