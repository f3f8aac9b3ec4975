// GeLU MLP block O = GeLU(scale * A Bt^T) C and its backward, bf16 in / fp32
// accumulate, on gfx950 MFMA.
//
// The block is the unit O = f(A B) C with f = GeLU (erf form) applied
// elementwise ("Memory-efficient tensor parallelism" abstract; the MLP block of
// "AutoSP" 2.A).  The m x n intermediate H = scale A Bt^T is formed one 32 x 32
// tile at a time in registers, passed through GeLU and consumed by the second
// product at once; it is never written to device memory.  The backward
// recomputes H (and dG = dO C^T) per tile instead of storing activations
// ("AutoSP" 2.B):
//   dH = dG * GeLU'(H), dA = scale dH Bt, dBt = scale dH^T A, dC = GeLU(H)^T dO.
//
// Two kernels, each used twice through the symmetry of H = scale A Bt^T in
// (A, Bt):
//  * mlp_fwd_kernel (64-row blocks): O[i] = sum_j GeLU(H_ij) C_j, and with the
//    roles of (A, Bt, C) taken by (Bt, A, dO), dC[j] = sum_i GeLU(H_ij) dO_i;
//  * mlp_bwd_da_kernel (32-row blocks): dA[i] = scale sum_j dH_ij Bt_j, and
//    with (A, dO, Bt, C) taken by (Bt, C, A, dO), dBt[j] = scale sum_i dH_ij A_i.
// Lanes own rows as in the attention kernels.  The long contractions of the
// first products (k, p <= 1024) are split across the waves, each keeping its
// slice of the resident operand in registers; the partial 32 x 32 tiles are
// summed through LDS and each wave finishes a share of every lane's tile
// entries (GeLU or GeLU'), so each erf is evaluated once; each wave then owns
// a slice of the output columns for the second product.  Streamed operands are
// read from copies of the inputs (never of the intermediate) that small
// kernels pack into the workspace first, in MFMA operand order, so each load
// or async copy reads 1 KiB of contiguous memory (see the packing kernels
// below).  The streamed loop is split across workgroups; the fp32 partial
// sums are added by a final elementwise kernel.  The second products put the
// register operand (G, dH) on the MFMA's row side, so an accumulator tile holds
// output rows by slot and output columns by lane: each partial-sum store of a
// wave then writes whole 128-byte lines (one per row and half-wave) instead
// of 32 bytes of each of 32 lines, which at the end of a kernel, when every
// workgroup stores at once, is four times fewer L2 writes.
#include "fab_device.h"
#include "fab_internal.h"

namespace fab {
namespace {

constexpr int kPad = 64;        // padding of the packed copies' row count

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// GeLU = x Phi(x) and GeLU' = Phi(x) + x phi(x) take Phi from erf by
// Abramowitz and Stegun, Handbook of Mathematical Functions, formula 7.1.26
// (absolute error below 1.5e-7, far inside the bf16 rounding G and dH receive
// next); its factor exp(-x^2 / 2) is also the density phi up to 1 / sqrt(2 pi).
// The formula has no branches (the library erf switches between two
// polynomials with a divergent branch), so its instructions can be scheduled
// between the matrix products.
struct NormalParts {
  float cdf;  // Phi(x)
  float e;    // exp(-x^2 / 2)
};
__device__ __forceinline__ NormalParts normal_parts(float x) {
  const float z = fabsf(x) * 0.7071067811865476f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.f));  // v_rcp_f32, 1 ulp
  float poly = fmaf(1.061405429f, t, -1.453152027f);
  poly = fmaf(poly, t, 1.421413741f);
  poly = fmaf(poly, t, -0.284496736f);
  poly = fmaf(poly, t, 0.254829592f);
  poly *= t;
  const float e = __expf(-z * z);
  const float erf_abs = fmaf(-poly, e, 1.f);
  const float erf = x < 0.f ? -erf_abs : erf_abs;
  return {fmaf(0.5f, erf, 0.5f), e};
}
__device__ __forceinline__ float gelu_f(float x) { return x * normal_parts(x).cdf; }
__device__ __forceinline__ float gelu_grad_f(float x) {
  const NormalParts n = normal_parts(x);
  return fmaf(x * 0.3989422804014327f, n.e, n.cdf);
}

// Operands are streamed from copies packed in MFMA operand order, so that
// every load (or async copy) of a wave reads 1 KiB of contiguous memory: a
// fragment is the 64 lanes x 16 bytes one MFMA takes as its A operand, lane
// l holding 8 consecutive values of row perm_row(l % 32) of a 32-row tile.
//  * "row" fragments (first-product operands, X [rows][cols] as stored):
//    fragment (R, j), j = cols / 16 chunk, lane l: X[32 R + perm_row(l % 32)]
//    [16 j + 8 (l / 32) + e]; stored at ((R * cols / 16) + j) * 512.
//  * "column" fragments (second-product operands, X transposed): fragment
//    (R, T, c), R over cols / 32, T over rows_pad / 32, c in {0, 1}, lane l:
//    X[32 T + 16 (l / 32) + 8 c + e][32 R + perm_row(l % 32)]; stored at
//    ((T * cols / 32 + R) * 2 + c) * 512, so the fragments of one 32-row step
//    T are contiguous (a step's copies spread over every L2 channel instead of
//    landing 64 rows_pad bytes apart, on one channel).
// The fragments cover cols_pad columns (the kernels' compiled width, a power
// of two from 128); rows of X at or past `rows` and columns at or past `cols`
// read as zero.  rows_pad % 64 == 0, cols % 64 == 0, cols <= cols_pad.
// One pack job: row fragments (cols_kind 0) or column fragments (1) of
// X [rows][cols], zero-padded to rows_pad x cols_pad, on workgroups
// [block0, block0 + blocks) of a batched launch.
struct PackJob {
  const uint16_t* x;
  uint16_t* out;
  int64_t ld, rows_pad;
  int rows, cols, cols_pad, cols_kind, block0;
};
// Up to seven jobs per launch (the backward packs seven operand copies).
struct PackJobs {
  PackJob j[7];
  int n;
};

// Row fragments, workgroup b: 256 consecutive 16-byte pieces.
__device__ __forceinline__ void pack_rows_block(const PackJob& J, int b) {
  const int64_t pieces = J.rows_pad * J.cols_pad / 8;
  const int64_t i = (int64_t)b * 256 + threadIdx.x;  // one 16-byte piece
  if (i >= pieces) return;
  const int l = (int)(i & 63);
  const int64_t f = i >> 6;
  const int nj = J.cols_pad / 16;
  const int j = (int)(f % nj);
  const int64_t R = f / nj;
  const int64_t row = 32 * R + perm_row(l & 31);
  const int col = 16 * j + 8 * (l >> 5);
  const u32x4 v = row < J.rows && col < J.cols ? ldg16(J.x + row * J.ld + col) : u32x4{0, 0, 0, 0};
  stg16(J.out + i * 8, v);
}

// Column fragments, workgroup b: one 64 x 64 block of X through LDS.
__device__ __forceinline__ void pack_cols_block(const PackJob& J, int b, uint16_t (*tile)[64 + 2]) {
  const int gx = (int)(J.rows_pad / 64);
  const int r0 = (b % gx) * 64, c0 = (b / gx) * 64;
  const int tid = threadIdx.x;
  // load 64 x 64 of X: 512 chunks of 8 elements, 2 per thread
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = tid + 256 * u;
    const int r = i / 8, ch = i % 8;
    const int gr = r0 + r, gc = c0 + ch * 8;
    u32x4 v = {0, 0, 0, 0};
    if (gr < J.rows && gc < J.cols) v = ldg16(J.x + (int64_t)gr * J.ld + gc);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      tile[r][ch * 8 + 2 * w] = (uint16_t)(v[w] & 0xffff);
      tile[r][ch * 8 + 2 * w + 1] = (uint16_t)(v[w] >> 16);
    }
  }
  __syncthreads();
  // write the 2 (R) x 2 (T) x 2 (c) fragments of this 64 x 64 block
  const int nr = J.cols_pad / 32;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int piece = tid + 256 * u;
    const int l = piece & 63, c = (piece >> 6) & 1, tl = (piece >> 7) & 1, rl = piece >> 8;
    const int xc = 32 * rl + perm_row(l & 31);
    const int xr = 32 * tl + 16 * (l >> 5) + 8 * c;
    u32x4 v;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      v[w] = (uint32_t)tile[xr + 2 * w][xc] | ((uint32_t)tile[xr + 2 * w + 1][xc] << 16);
    const int64_t frag = ((int64_t)(r0 / 32 + tl) * nr + (c0 / 32 + rl)) * 2 + c;
    stg16(J.out + frag * 512 + l * 8, v);
  }
}

// Every pack job of a pass in one launch (jobs in block0 order); a
// workgroup finds its job by a uniform scan of at most seven entries.
__global__ __launch_bounds__(256) void pack_kernel(PackJobs jobs) {
  __shared__ uint16_t tile[64][64 + 2];
  const int b = blockIdx.x;
  int k = 0;
  while (k + 1 < jobs.n && b >= jobs.j[k + 1].block0) ++k;
  const PackJob& J = jobs.j[k];
  if (J.cols_kind) pack_cols_block(J, b - J.block0, tile);
  else pack_rows_block(J, b - J.block0);
}

// One reduction job: out[r][c] = bf16(scale * sum_s part[s][r][c]), part
// packed [splits][rows][cols], on workgroups [block0, block0 + blocks).
struct ReduceJob {
  const float* part;
  uint16_t* out;
  int64_t ld_out;
  float scale;
  int splits, rows, cols, block0;
};
struct ReduceJobs {
  ReduceJob j[3];
  int n;
};

__global__ __launch_bounds__(256) void reduce_parts_kernel(ReduceJobs jobs) {
  const int b = blockIdx.x;
  int k = 0;
  while (k + 1 < jobs.n && b >= jobs.j[k + 1].block0) ++k;
  const ReduceJob& J = jobs.j[k];
  const int64_t i = ((int64_t)(b - J.block0) * 256 + threadIdx.x) * 8;
  const int64_t total = (int64_t)J.rows * J.cols;
  if (i >= total) return;
  const int64_t r = i / J.cols, c = i % J.cols;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int s = 0; s < J.splits; ++s) {
    const f32x4* src = reinterpret_cast<const f32x4*>(J.part + (int64_t)s * total + i);
    const f32x4 x = src[0], y = src[1];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc[w] += x[w];
      acc[4 + w] += y[w];
    }
  }
  u32x4 v;
#pragma unroll
  for (int w = 0; w < 4; ++w) v[w] = pack_bf16(acc[2 * w] * J.scale, acc[2 * w + 1] * J.scale);
  stg16(J.out + r * J.ld_out + c, v);
}

// Partial tiles live in LDS as float pairs, slot-pair major: pair q (slots
// 2q, 2q + 1) of wave w's partial for lane l at float2 index (8 w + q) 64 + l,
// so every 8-byte write or read of a wave covers 512 contiguous bytes (no bank
// conflicts; a lane-major layout puts a wave's reads 64 bytes apart).
//
// finish_tile sums the NW partial tiles of H and of dG and writes
// dH = dG * GeLU'(scale H) as bf16 pairs to gsh; wave w takes slots
// [16 w / NW, 16 (w + 1) / NW) of every lane, so each erf is evaluated once.
// Caller: barrier before (partials written) and after (gsh complete).
template <int NW>
__device__ __forceinline__ void finish_tile(const float* red_h, const float* red_g, uint32_t* gsh,
                                            int wave, int lane, float scale) {
  constexpr int SPW = 16 / NW;
  static_assert(SPW % 2 == 0, "slots are packed in pairs");
  float h[SPW], g[SPW];
#pragma unroll
  for (int j = 0; j < SPW; ++j) h[j] = g[j] = 0.f;
  const f32x2* rh = reinterpret_cast<const f32x2*>(red_h);
  const f32x2* rg = reinterpret_cast<const f32x2*>(red_g);
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int j = 0; j < SPW; j += 2) {
      const int idx = (8 * w + (wave * SPW + j) / 2) * 64 + lane;
      const f32x2 x = rh[idx];
      h[j] += x[0];
      h[j + 1] += x[1];
      const f32x2 y = rg[idx];
      g[j] += y[0];
      g[j + 1] += y[1];
    }
  float x[SPW];
#pragma unroll
  for (int j = 0; j < SPW; ++j) x[j] = g[j] * gelu_grad_f(scale * h[j]);
#pragma unroll
  for (int j = 0; j < SPW; j += 2) gsh[lane * 8 + (wave * SPW + j) / 2] = pack_bf16(x[j], x[j + 1]);
}

__device__ __forceinline__ void stash_tile(float* red, int wave, int lane, const f32x16& v) {
  f32x2* mine = reinterpret_cast<f32x2*>(red) + wave * 8 * 64 + lane;
#pragma unroll
  for (int q = 0; q < 8; ++q) mine[q * 64] = f32x2{v[2 * q], v[2 * q + 1]};
}

// The backward kernels stage their transposed second-product operand in LDS
// with asynchronous global -> LDS copies (each lane reads back exactly the 16
// byte pieces it copied, so only a wave-local wait is needed).  The copies are
// issued right before the next tile's row loads, and vector memory operations
// complete in issue order, so waiting until only those N loads remain
// outstanding (wait_copies<N>) waits for exactly the copies.

__device__ __forceinline__ void wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Waits until at most N LDS (and scalar memory) operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_lds_reads_but() {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
}
// Inside step i of lds_mfma_pipeline<N, DEPTH>: waits until operand i's LDS
// read has completed.  At that point at most min(DEPTH - 1, N - 1 - i) reads
// were issued after it, and LDS operations complete in order (the counter
// also counts scalar memory loads, which do not; the loops that use this
// issue none: their kernel arguments are loaded before the loop); i is a
// constant once the pipeline is unrolled, so the branches fold away.
template <int N, int DEPTH>
__device__ __forceinline__ void wait_operand_read(int i) {
  static_assert(DEPTH >= 1 && DEPTH <= 4, "pipeline depth");
  const int newer = N - 1 - i < DEPTH - 1 ? N - 1 - i : DEPTH - 1;
  if (newer >= 3) wait_lds_reads_but<3>();
  else if (newer == 2) wait_lds_reads_but<2>();
  else if (newer == 1) wait_lds_reads_but<1>();
  else wait_lds_reads_but<0>();
}

// ---------------------------------------------------------------------------
// forward: workgroup = 64 rows of A (two 32-row tiles), one split of the n
// tiles, four waves with the whole register file each.
//
// The output block O [64 rows, p] stays in registers for the whole n loop
// (wave w owns columns [w p / 4, (w + 1) p / 4) of both row tiles), so every
// Bt and C^T fragment a wave stages serves 64 rows: twice the operand reuse
// of 32-row blocks, which halves the L2 -> CU bytes per MFMA.  The first
// product's contraction k is split over the waves (wave w: [w k / 4,
// (w + 1) k / 4)); each wave keeps its A slice of both row tiles in registers
// and forms partial H^T tiles for both.  Each wave then finishes a quarter of
// the 64 x 32 chunk (tile w / 2, slots 8 (w % 2) .. + 7 of every lane): it
// sums its own partials with the three the other waves left in LDS, applies
// GeLU once per element and publishes bf16 G.  Per n chunk j:
//   H^T(j) partials (MFMA) -> stash, read G(j - 1) -> barrier ->
//   finish(j) (sums, GeLU) and O += G(j - 1) C(j - 1) (MFMA)
//   -> publish G(j) -> barrier
// (the GeLU of chunk j and the second product of chunk j - 1 are independent,
// so the scheduler may interleave their instructions).  The Bt and C^T fragments of a wave are private to it (contraction slice,
// output slice): they are copied global -> LDS asynchronously into per-wave
// regions and need only wave-local waits.  Each 1 KiB slot is refilled with
// the next chunk's fragment as soon as the product reading it has its operand
// in registers (Bt(j + 1) during H(j), C^T(j) during the second product of
// chunk j - 1), so every copy has about a chunk's time to land.  The
// workspace holds Bt and C^T packed in MFMA operand order, one chunk's
// fragments contiguous.
// ---------------------------------------------------------------------------
constexpr int kFwdWaves = 4;

template <int K, int P>
struct FwdShape {
  static constexpr int kq = K / kFwdWaves, kc = kq / 16;  // k slice, 16-deep steps
  static constexpr int pq = P / kFwdWaves, pt = pq / 32;  // p slice, 32-wide tiles
  static_assert(kc >= 1 && pt >= 1, "k >= 64 and p >= 128");
  static constexpr int BT = kc * 1024;        // Bt fragments of one wave, one chunk
  static constexpr int CT = pt * 2 * 1024;    // C^T fragments of one wave, one chunk
  static constexpr int RED = 4 * 3 * 2048;    // partial H: 8 values per lane per (wave, other wave)
  static constexpr int GSH = 2 * 2 * 1024;    // G of the chunk: 2 row tiles x 2 halves
  static constexpr int LDS = kFwdWaves * (BT + CT) + RED + GSH;
  static_assert(LDS <= 160 * 1024, "LDS");
};

template <int K, int P>
__device__ __forceinline__ void mlp_fwd_body(MlpArgs a, const uint16_t* btr, const uint16_t* ctf,
                                             int mb, int splits, int tiles_per_split, float* part) {
  using S = FwdShape<K, P>;
  constexpr int kc = S::kc, pt = S::pt;
  __shared__ __attribute__((aligned(1024))) char lds[S::LDS];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lq = lane & 31;
  char* const bsh = lds + wave * S::BT;
  char* const csh = lds + kFwdWaves * S::BT + wave * S::CT;
  char* const red = lds + kFwdWaves * (S::BT + S::CT);
  char* const gsh = red + S::RED;

  // workgroup i runs on XCD i % 8: give each XCD whole runs of one split, so
  // the workgroups sharing an L2 stream the same n range of Bt and C
  int lid = blockIdx.x;
  const int total = mb * splits;
  if (total % 8 == 0) lid = (lid % 8) * (total / 8) + lid / 8;
  const int split = lid / mb, rb = lid % mb;
  const int ntiles = (a.n + 31) / 32;
  const int j0 = split * tiles_per_split;
  const int j1 = min(ntiles, j0 + tiles_per_split);

  // A slices of both row tiles: B operands of H^T = Bt A^T
  const uint16_t* A = static_cast<const uint16_t*>(a.a);
  u32x4 af[2][kc];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row = rb * 64 + 32 * rt + lq;
#pragma unroll
    for (int c = 0; c < kc; ++c) {
      const int col = wave * S::kq + 16 * c + 8 * (lane >> 5);  // zero past k (padded width)
      af[rt][c] = row < a.m && col < a.k ? ldg16(A + (int64_t)row * a.a_sr + col) : u32x4{0, 0, 0, 0};
    }
  }
  f32x16 o[pt][2];
#pragma unroll
  for (int t = 0; t < pt; ++t)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[t][rt][r] = 0.f;

  // Fragment c of Bt chunk j: row fragment (j, wave kc + c), 1 KiB; fragment
  // i = 2 t + c of C^T chunk j: column fragment (wave pt + t, j, c).  Slot i of
  // a wave's region is refilled with the next chunk's fragment i as soon as
  // the product that reads it has its operand in registers, so each copy has a
  // whole chunk period to land.
  auto bt_src = [&](int j) { return btr + ((int64_t)j * (K / 16) + wave * kc) * 512; };
  auto c_src = [&](int j, int i) {
    return ctf + (((int64_t)j * (P / 32) + wave * pt + i / 2) * 2 + i % 2) * 512;
  };
  auto copy_c = [&](int j) {
#pragma unroll
    for (int i = 0; i < 2 * pt; ++i) dma16(c_src(j, i), 16 * lane, csh + i * 1024);
  };
  // O += G C over one chunk, G from registers (g[rt][half], the A operands;
  // a C^T fragment read as the B operand is C); with REFILL, slot i then
  // receives fragment i of chunk jn
  constexpr int kDepth2 = 2;
  auto second_product = [&]<bool REFILL>(const u32x4 (&g)[2][2], int jn) {
    lds_mfma_pipeline<2 * pt, kDepth2>(
        [&](int i) { return lds16(csh + i * 1024 + 16 * lane); },
        [&](int i, const u32x4& x) {
          o[i / 2][0] = mfma32(g[0][i % 2], x, o[i / 2][0]);
          o[i / 2][1] = mfma32(g[1][i % 2], x, o[i / 2][1]);
          if constexpr (REFILL) {
            wait_operand_read<2 * pt, kDepth2>(i);  // slot i's read is complete
            dma16(c_src(jn, i), 16 * lane, csh + i * 1024);
          }
        });
  };

  // this wave's quarter of the chunk: row tile wave / 2, slots 8 (wave % 2) .. + 7
  const int mine_rt = wave >> 1, mine_h = wave & 1;
  // G of the previous chunk (bf16, the second product's A operands); read
  // from gsh before the barrier after which the waves overwrite it
  u32x4 g[2][2];
  auto read_g = [&]() {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) g[rt][hh] = lds16(gsh + (rt * 2 + hh) * 1024 + 16 * lane);
  };
  // one n chunk; PREV: the previous chunk's second product runs alongside
  // this chunk's GeLU (false only for the first chunk)
  constexpr int kDepth1 = 3;
  auto chunk = [&]<bool PREV>(int j) {
    // this chunk's Bt (the C^T copies issued after it may still be in flight)
    if (PREV) wait_copies<2 * pt>();
    else wait_copies<0>();
    f32x16 hp[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) hp[0][r] = hp[1][r] = 0.f;
    // the last chunk copies itself again (its slots are read before each copy):
    // keeps the copy count, and so the waits, the same for every chunk
    const uint16_t* next = bt_src(min(j + 1, j1 - 1));
    lds_mfma_pipeline<kc, kDepth1>(
        [&](int c) { return lds16(bsh + c * 1024 + 16 * lane); },
        [&](int c, const u32x4& x) {
          hp[0] = mfma32(x, af[0][c], hp[0]);
          hp[1] = mfma32(x, af[1][c], hp[1]);
          wait_operand_read<kc, kDepth1>(c);  // slot c's read is complete
          dma16(next + c * 512, 16 * lane, bsh + c * 1024);
        });
    // stash the quarters the other waves finish: 8 values per lane each, at
    // red + ((owner * 3 + k) * 2 + half) * 1024, k = this wave's rank among
    // the owner's three sources
#pragma unroll
    for (int u = 0; u < kFwdWaves; ++u) {
      if (u == wave) continue;
      const int k = wave < u ? wave : wave - 1;
      char* dst = red + ((u * 3 + k) * 2) * 1024 + 16 * lane;
      const f32x16& h = hp[u >> 1];
      const int s0 = 8 * (u & 1);
      *reinterpret_cast<f32x4*>(dst) = f32x4{h[s0], h[s0 + 1], h[s0 + 2], h[s0 + 3]};
      *reinterpret_cast<f32x4*>(dst + 1024) = f32x4{h[s0 + 4], h[s0 + 5], h[s0 + 6], h[s0 + 7]};
    }
    float own[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x0 = mine_rt ? hp[1][e] : hp[0][e];
      const float x1 = mine_rt ? hp[1][8 + e] : hp[0][8 + e];
      own[e] = mine_h ? x1 : x0;
    }
    if constexpr (PREV) read_g();
    lds_barrier();
    if (PREV) wait_copies<kc>();  // C^T(j - 1); the next chunk's Bt stays in flight
    // finish this wave's quarter of chunk j while the previous chunk's second
    // product runs
#pragma unroll
    for (int k = 0; k < 3; ++k)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(red + ((wave * 3 + k) * 2 + hh) * 1024 + 16 * lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) own[4 * hh + e] += x[e];
      }
    if constexpr (PREV) second_product.template operator()<true>(g, j);
    u32x4 gv;
#pragma unroll
    for (int e = 0; e < 4; ++e) gv[e] = pack_bf16(gelu_f(a.scale * own[2 * e]), gelu_f(a.scale * own[2 * e + 1]));
    sts16(gsh + (mine_rt * 2 + mine_h) * 1024 + 16 * lane, gv);
    if constexpr (!PREV) copy_c(j);
    lds_barrier();
  };
  if (j0 < j1) {
#pragma unroll
    for (int c = 0; c < kc; ++c) dma16(bt_src(j0) + c * 512, 16 * lane, bsh + c * 1024);
    chunk.template operator()<false>(j0);
  }
  for (int j = j0 + 1; j < j1; ++j) chunk.template operator()<true>(j);
  if (j0 < j1) {
    read_g();
    wait_copies<0>();
    second_product.template operator()<false>(g, 0);
  }
  wait_copies<0>();
  // o[t][rt] holds O rows rb 64 + 32 rt + 8 (r / 4) + 4 (lane / 32) + r % 4,
  // column wave pq + 32 t + perm_row(lane % 32): lanes 0..31 (and 32..63)
  // of one store fill one 128-byte line of a row
  const int col0 = wave * S::pq + perm_row(lq);
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int t = 0; t < pt; ++t) {
      if (wave * S::pq + 32 * t >= a.p) continue;  // p <= padded width, p % 32 == 0
      float* dst = part + ((int64_t)split * a.m + rb * 64 + 32 * rt + 4 * (lane >> 5)) * a.p + col0 + 32 * t;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int dr = 8 * (r >> 2) + (r & 3);
        if (rb * 64 + 32 * rt + 4 * (lane >> 5) + dr < a.m) dst[(int64_t)dr * a.p] = o[t][rt][r];
      }
    }
}

// ---------------------------------------------------------------------------
// backward: dA (and, with the roles swapped, dBt).  The kernel recomputes one
// 32 x 32 tile of H and of dG per step, split over NW waves along the
// contractions, finishes dH with finish_tile and feeds it to the second
// product.  After this tile's first-product MFMAs, the tile's transposed
// second-product operand is copied asynchronously into LDS and the rows of
// the next tile's first-product operands are loaded into registers, so both
// overlap the barriers and GeLU', and the second operand holds no registers
// while the partial tiles do.
// ---------------------------------------------------------------------------

// Copies this wave's kt x 2 column fragments (R = r0 + t of the transposed
// operand's nr, step T, halves c) into its LDS region: fragment (t, c) lands
// at region + (2 t + c) * 1024, lane l's 16 bytes at + 16 l, which is where
// that lane reads them back.  The 2 kt fragments are 2 kt KiB of contiguous
// memory.
template <int kt, int nr>
__device__ __forceinline__ void copy_second_operand(const uint16_t* xf, int r0, int T, int lane,
                                                    char* region) {
#pragma unroll
  for (int t = 0; t < kt; ++t)
#pragma unroll
    for (int c = 0; c < 2; ++c)
      dma16(xf + (((int64_t)T * nr + r0 + t) * 2 + c) * 512, 16 * lane, region + (2 * t + c) * 1024);
}

// Wave count of a backward kernel whose first product contracts over K (and P
// for dG) and whose output has OUT columns: each wave needs a 16-deep slice
// of each contraction and 32 output columns.
template <int K, int P, int OUT>
constexpr int mlp_bwd_waves() { return (K >= 128 && P >= 128 && OUT >= 256) ? 8 : 4; }

// dA: workgroup = 32 rows of A, one split of the n tiles.
template <int K, int P>
__device__ __forceinline__ void mlp_bwd_da_body(MlpArgs a, const uint16_t* btr, const uint16_t* cr,
                                                const uint16_t* btc, int tiles_per_split,
                                                float* part) {
  constexpr int NW = mlp_bwd_waves<K, P, K>();
  __shared__ __attribute__((aligned(16))) float red[2 * NW * 64 * 16];  // partial H, dG tiles
  constexpr int kq = K / NW, kc = kq / 16, kt = kq / 32;
  __shared__ __attribute__((aligned(16))) uint32_t gsh[64 * 8];         // dH tile, bf16 pairs
  __shared__ __attribute__((aligned(16))) char tsh[NW * kt * 2048];     // Bt^T pieces, per wave
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lq = lane & 31, lg = lane >> 5;
  const int row = blockIdx.x * 32 + lq;
  const bool rlive = row < a.m;
  char* const tmine = tsh + wave * kt * 2048;
  constexpr int pq = P / NW, pc = pq / 16;
  static_assert(kt >= 1 && pc >= 1, "each wave needs 32 columns of k and a 16-deep slice of p");
  const uint16_t* A = static_cast<const uint16_t*>(a.a);
    const uint16_t* dO = static_cast<const uint16_t*>(a.dout);

  // columns past k (or p) read as zero: the compiled widths K, P may exceed them
  u32x4 af[kc], df[pc];
#pragma unroll
  for (int c = 0; c < kc; ++c) {
    const int ck = wave * kq + 16 * c + 8 * lg;
    af[c] = rlive && ck < a.k ? ldg16(A + (int64_t)row * a.a_sr + ck) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int c = 0; c < pc; ++c) {
    const int cp = wave * pq + 16 * c + 8 * lg;
    df[c] = rlive && cp < a.p ? ldg16(dO + (int64_t)row * a.o_sr + cp) : u32x4{0, 0, 0, 0};
  }
  f32x16 acc[kt];
#pragma unroll
  for (int t = 0; t < kt; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;

  const int ntiles = (a.n + 31) / 32;
  const int jt0 = blockIdx.y * tiles_per_split;
  const int jt1 = min(ntiles, jt0 + tiles_per_split);
  u32x4 bfr[kc], cfr[pc];
  // row fragments (jt, wave kc + c) of Bt and (jt, wave pc + c) of C
  auto load_rows = [&](int jt) {
    const uint16_t* bp = btr + ((int64_t)jt * (K / 16) + wave * kc) * 512 + lane * 8;
    const uint16_t* cp = cr + ((int64_t)jt * (P / 16) + wave * pc) * 512 + lane * 8;
#pragma unroll
    for (int c = 0; c < kc; ++c) bfr[c] = ldg16(bp + c * 512);
#pragma unroll
    for (int c = 0; c < pc; ++c) cfr[c] = ldg16(cp + c * 512);
  };
  if (jt0 < jt1) load_rows(jt0);
  for (int jt = jt0; jt < jt1; ++jt) {
    f32x16 hp, gp;
#pragma unroll
    for (int r = 0; r < 16; ++r) hp[r] = gp[r] = 0.f;
#pragma unroll
    for (int c = 0; c < kc; ++c) hp = mfma32(bfr[c], af[c], hp);
#pragma unroll
    for (int c = 0; c < pc; ++c) gp = mfma32(cfr[c], df[c], gp);
    wait_lds_reads();  // the previous tile's reads of tmine are done
    copy_second_operand<kt, K / 32>(btc, wave * kq / 32, jt, lane, tmine);
    load_rows(min(jt + 1, jt1 - 1));  // unconditional: a branch here costs register copies
    stash_tile(red, wave, lane, hp);
    stash_tile(red + NW * 64 * 16, wave, lane, gp);
    __syncthreads();
    // slot r of lane l: row `row`, column 32 jt + 16 lg + r
    finish_tile<NW>(red, red + NW * 64 * 16, gsh, wave, lane, a.scale);
    __syncthreads();
    u32x4 db[2];
    db[0] = *reinterpret_cast<const u32x4*>(gsh + lane * 8);
    db[1] = *reinterpret_cast<const u32x4*>(gsh + lane * 8 + 4);
    wait_copies<kc + pc>();  // the next tile's row loads stay in flight
#pragma unroll
    for (int t = 0; t < kt; ++t) {
      acc[t] = mfma32(db[0], lds16(tmine + (2 * t) * 1024 + 16 * lane), acc[t]);
      acc[t] = mfma32(db[1], lds16(tmine + (2 * t + 1) * 1024 + 16 * lane), acc[t]);
    }
  }
  // acc[t] holds dA rows 32 blockIdx.x + 8 (r / 4) + 4 lg + r % 4, column
  // wave kq + 32 t + perm_row(lane % 32): each store fills one 128-byte line
  // of two rows
  const int r0 = blockIdx.x * 32 + 4 * lg;
  float* dst = part + ((int64_t)blockIdx.y * a.m + r0) * a.k + wave * kq + perm_row(lq);
#pragma unroll
  for (int t = 0; t < kt; ++t) {
    if (wave * kq + 32 * t >= a.k) continue;  // k <= padded width, k % 32 == 0
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int dr = 8 * (r >> 2) + (r & 3);
      if (r0 + dr < a.m) dst[(int64_t)dr * a.k + 32 * t] = acc[t][r];
    }
  }
}

// The two bodies each back two kernels (same code, names of their own so
// profiles tell the launches apart): the forward and dC; dA and dBt.
template <int K, int P>
__global__ __launch_bounds__(64 * kFwdWaves, 1) void mlp_fwd_kernel(
    MlpArgs a, const uint16_t* btr, const uint16_t* ctf, int mb, int splits, int per, float* part) {
  mlp_fwd_body<K, P>(a, btr, ctf, mb, splits, per, part);
}
template <int K, int P>
__global__ __launch_bounds__(64 * kFwdWaves, 1) void mlp_bwd_dc_kernel(
    MlpArgs a, const uint16_t* btr, const uint16_t* ctf, int mb, int splits, int per, float* part) {
  mlp_fwd_body<K, P>(a, btr, ctf, mb, splits, per, part);
}
template <int K, int P>
__global__ __launch_bounds__((64 * mlp_bwd_waves<K, P, K>())) void mlp_bwd_da_kernel(
    MlpArgs a, const uint16_t* btr, const uint16_t* cr, const uint16_t* btc, int per, float* part) {
  mlp_bwd_da_body<K, P>(a, btr, cr, btc, per, part);
}
template <int K, int P>
__global__ __launch_bounds__((64 * mlp_bwd_waves<K, P, K>())) void mlp_bwd_dbt_kernel(
    MlpArgs a, const uint16_t* btr, const uint16_t* cr, const uint16_t* btc, int per, float* part) {
  mlp_bwd_da_body<K, P>(a, btr, cr, btc, per, part);
}

struct MlpLayout {
  int split_fwd;    // splits of the n loop for the forward (64-row blocks)
  int split_rows;   // splits of the n loop for the row-block backward kernel
  int split_cols;   // splits of the m loop for the dBt kernel
  int split_dc;     // splits of the m loop for dC (the forward kernel, 64-column blocks)
  int64_t m_pad, n_pad;
  size_t fwd_btr, fwd_ct, fwd_part, fwd_total;
  // row fragments of Bt, C, A, dO; column fragments of Bt, A, dO; partials
  size_t bwd_btr, bwd_cr, bwd_ar, bwd_dor, bwd_btc, bwd_ac, bwd_doc, bwd_pa, bwd_pb, bwd_pc, bwd_total;
};

int pick_splits(int blocks, int tiles) {
  int s = (256 + blocks - 1) / blocks;
  if (s > tiles) s = tiles;
  return s < 1 ? 1 : s;
}

// The width the kernels are compiled for that holds x (a multiple of 64 up to
// 1024): operands are zero-padded to it in the packed copies.
int padded_width(int x) { return x <= 128 ? 128 : x <= 256 ? 256 : x <= 512 ? 512 : 1024; }

MlpLayout layout(int m, int n, int k, int p) {
  MlpLayout L{};
  const int kw = padded_width(k), pw = padded_width(p);
  const int mb = (m + 31) / 32, nb = (n + 31) / 32;
  L.split_fwd = pick_splits((m + 63) / 64, nb);
  L.split_rows = pick_splits(mb, nb);
  L.split_cols = pick_splits(nb, mb);
  L.split_dc = pick_splits((n + 63) / 64, mb);
  L.m_pad = (int64_t)round_up(m, kPad);
  L.n_pad = (int64_t)round_up(n, kPad);
  size_t off = 0;
  L.fwd_btr = off;
  off = round_up(off + (size_t)kw * L.n_pad * 2, 256);
  L.fwd_ct = off;
  off = round_up(off + (size_t)pw * L.n_pad * 2, 256);
  L.fwd_part = off;
  off = round_up(off + (size_t)L.split_fwd * m * p * 4, 256);
  L.fwd_total = off;
  off = 0;
  for (size_t* slot : {&L.bwd_btr, &L.bwd_btc}) {
    *slot = off;
    off = round_up(off + (size_t)kw * L.n_pad * 2, 256);
  }
  L.bwd_cr = off;
  off = round_up(off + (size_t)pw * L.n_pad * 2, 256);
  for (size_t* slot : {&L.bwd_ar, &L.bwd_ac}) {
    *slot = off;
    off = round_up(off + (size_t)kw * L.m_pad * 2, 256);
  }
  for (size_t* slot : {&L.bwd_dor, &L.bwd_doc}) {
    *slot = off;
    off = round_up(off + (size_t)pw * L.m_pad * 2, 256);
  }
  L.bwd_pa = off;
  off = round_up(off + (size_t)L.split_rows * m * k * 4, 256);
  L.bwd_pb = off;
  off = round_up(off + (size_t)L.split_cols * n * k * 4, 256);
  L.bwd_pc = off;
  off = round_up(off + (size_t)L.split_dc * n * p * 4, 256);
  L.bwd_total = off;
  return L;
}

// Pack jobs of one pass, launched together by run().
struct Packer {
  PackJobs jobs{};
  int blocks = 0;
  // Row fragments of X [rows][cols], zero-padded to rows_pad x cols_pad.
  void rows(const void* x, int64_t ld, int rows, int cols, int cols_pad, int64_t rows_pad, void* out) {
    add(x, ld, rows, cols, cols_pad, rows_pad, out, 0,
        (int)((rows_pad * cols_pad / 8 + 255) / 256));
  }
  // Column fragments of X [rows][cols] (row fragments of X^T).
  void cols(const void* x, int64_t ld, int rows, int cols, int cols_pad, int64_t rows_pad, void* out) {
    add(x, ld, rows, cols, cols_pad, rows_pad, out, 1, (int)(rows_pad / 64) * (cols_pad / 64));
  }
  void add(const void* x, int64_t ld, int rows, int cols, int cols_pad, int64_t rows_pad, void* out,
           int kind, int nblocks) {
    PackJob& J = jobs.j[jobs.n++];
    J = {static_cast<const uint16_t*>(x), static_cast<uint16_t*>(out), ld, rows_pad, rows, cols,
         cols_pad, kind, blocks};
    blocks += nblocks;
  }
  hipError_t run(hipStream_t s) {
    FAB_TIMED("mlp_pack", s, hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, jobs));
    return hipGetLastError();
  }
};

// Split-sum reductions of one pass, launched together by run().
struct Reducer {
  ReduceJobs jobs{};
  int blocks = 0;
  void add(const float* part, int splits, int rows, int cols, float scale, void* out, int64_t ld_out) {
    ReduceJob& J = jobs.j[jobs.n++];
    J = {part, static_cast<uint16_t*>(out), ld_out, scale, splits, rows, cols, blocks};
    blocks += (int)(((int64_t)rows * cols / 8 + 255) / 256);
  }
  hipError_t run(hipStream_t s) {
    FAB_TIMED("mlp_reduce", s, hipLaunchKernelGGL(reduce_parts_kernel, dim3((unsigned)blocks), dim3(256), 0, s, jobs));
    return hipGetLastError();
  }
};

}  // namespace

size_t mlp_fwd_workspace(int m, int n, int k, int p, int* splits) {
  const MlpLayout L = layout(m, n, k, p);
  *splits = L.split_fwd;
  return L.fwd_total;
}

size_t mlp_bwd_workspace(int m, int n, int k, int p) { return layout(m, n, k, p).bwd_total; }

namespace {

// The forward kernel: for every row i of a.a, sum over the streamed rows j of
// GeLU(scale a.a_i . X_j) Y_j, with X's row fragments in btr and Y's column
// fragments in ctf.  It also computes dC (a.a = Bt, X = A, Y = dO).
template <int K, int P, bool DC>
hipError_t fwd_kp(const MlpArgs& a, int splits, const uint16_t* btr, const uint16_t* ctf,
                  float* part, hipStream_t s) {
  const int ntiles = (a.n + 31) / 32, mb = (a.m + 63) / 64;
  const int per = (ntiles + splits - 1) / splits;
  const dim3 grid((unsigned)(mb * splits)), block(64 * kFwdWaves);
  if (DC)
    FAB_TIMED("mlp_bwd_dc", s, hipLaunchKernelGGL((mlp_bwd_dc_kernel<K, P>), grid, block, 0, s, a, btr,
                                                  ctf, mb, splits, per, part));
  else
    FAB_TIMED("mlp_fwd", s, hipLaunchKernelGGL((mlp_fwd_kernel<K, P>), grid, block, 0, s, a, btr, ctf,
                                               mb, splits, per, part));
  return hipGetLastError();
}

template <int K, int P>
hipError_t bwd_kp(const MlpArgs& a, const MlpLayout& L, const char* ws, float* pa, float* pb,
                  float* pc, hipStream_t s) {
  auto frag = [&](size_t off) { return reinterpret_cast<const uint16_t*>(ws + off); };
  const int ntiles = (a.n + 31) / 32, mtiles = (a.m + 31) / 32;
  const int per_n = (ntiles + L.split_rows - 1) / L.split_rows;
  const int per_m = (mtiles + L.split_cols - 1) / L.split_cols;
  FAB_TIMED("mlp_bwd_da", s, hipLaunchKernelGGL((mlp_bwd_da_kernel<K, P>), dim3((unsigned)mtiles, (unsigned)L.split_rows),
                     dim3(64 * mlp_bwd_waves<K, P, K>()), 0, s, a, frag(L.bwd_btr), frag(L.bwd_cr),
                     frag(L.bwd_btc), per_n, pa));
  // dBt[j] = scale sum_i (C_j . dO_i) GeLU'(scale Bt_j . A_i) A_i: the dA
  // kernel with the roles of (A, dO, Bt, C) taken by (Bt, C, A, dO)
  MlpArgs u = a;
  u.a = a.bt;
  u.a_sr = a.bt_sr;
  u.dout = a.c;
  u.o_sr = a.c_sr;
  u.m = a.n;
  u.n = a.m;
  FAB_TIMED("mlp_bwd_dbt", s, hipLaunchKernelGGL((mlp_bwd_dbt_kernel<K, P>), dim3((unsigned)ntiles, (unsigned)L.split_cols),
                     dim3(64 * mlp_bwd_waves<K, P, K>()), 0, s, u, frag(L.bwd_ar), frag(L.bwd_dor),
                     frag(L.bwd_ac), per_m, pb));
  if (const hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  // dC[j] = sum_i GeLU(scale Bt_j . A_i) dO_i: the forward with the roles of
  // (A, Bt, C) taken by (Bt, A, dO), on 64-column blocks of n
  MlpArgs t = a;
  t.a = a.bt;
  t.a_sr = a.bt_sr;
  t.m = a.n;
  t.n = a.m;
  return fwd_kp<K, P, true>(t, L.split_dc, frag(L.bwd_ar), frag(L.bwd_doc), pc, s);
}

// Calls fn.template operator()<K, P>() for the supported sizes.
template <typename F>
hipError_t dispatch_kp(int k, int p, F&& fn) {
#define FAB_MLP_P(K)                                  \
  switch (p) {                                        \
    case 128: return fn.template operator()<K, 128>(); \
    case 256: return fn.template operator()<K, 256>(); \
    case 512: return fn.template operator()<K, 512>(); \
    case 1024: return fn.template operator()<K, 1024>(); \
  }                                                   \
  return hipErrorInvalidValue;
  switch (k) {
    case 128: { FAB_MLP_P(128) }
    case 256: { FAB_MLP_P(256) }
    case 512: { FAB_MLP_P(512) }
    case 1024: { FAB_MLP_P(1024) }
  }
#undef FAB_MLP_P
  return hipErrorInvalidValue;
}

}  // namespace

bool mlp_shape_supported(int k, int p) {
  auto ok = [](int x) { return x >= 64 && x <= 1024 && x % 64 == 0; };
  return ok(k) && ok(p);
}

hipError_t launch_mlp_fwd_bf16(const MlpArgs& a, hipStream_t s) {
  if (!mlp_shape_supported(a.k, a.p)) return hipErrorInvalidValue;
  const MlpLayout L = layout(a.m, a.n, a.k, a.p);
  const int kw = padded_width(a.k), pw = padded_width(a.p);
  char* ws = reinterpret_cast<char*>(a.ws);
  uint16_t* btr = reinterpret_cast<uint16_t*>(ws + L.fwd_btr);
  uint16_t* ctf = reinterpret_cast<uint16_t*>(ws + L.fwd_ct);
  float* part = reinterpret_cast<float*>(ws + L.fwd_part);
  Packer pk;
  pk.rows(a.bt, a.bt_sr, a.n, a.k, kw, L.n_pad, btr);
  pk.cols(a.c, a.c_sr, a.n, a.p, pw, L.n_pad, ctf);
  hipError_t e = pk.run(s);
  if (e != hipSuccess) return e;
  e = dispatch_kp(kw, pw, [&]<int K, int P>() {
    return fwd_kp<K, P, false>(a, L.split_fwd, btr, ctf, part, s);
  });
  if (e != hipSuccess) return e;
  Reducer rd;
  rd.add(part, L.split_fwd, a.m, a.p, 1.f, a.o, a.o_sr);
  return rd.run(s);
}

hipError_t launch_mlp_bwd_bf16(const MlpArgs& a, hipStream_t s) {
  if (!mlp_shape_supported(a.k, a.p)) return hipErrorInvalidValue;
  const MlpLayout L = layout(a.m, a.n, a.k, a.p);
  const int kw = padded_width(a.k), pw = padded_width(a.p);
  char* ws = reinterpret_cast<char*>(a.ws);
  float* pa = reinterpret_cast<float*>(ws + L.bwd_pa);
  float* pb = reinterpret_cast<float*>(ws + L.bwd_pb);
  float* pc = reinterpret_cast<float*>(ws + L.bwd_pc);
  Packer pk;
  pk.rows(a.bt, a.bt_sr, a.n, a.k, kw, L.n_pad, ws + L.bwd_btr);
  pk.rows(a.c, a.c_sr, a.n, a.p, pw, L.n_pad, ws + L.bwd_cr);
  pk.rows(a.a, a.a_sr, a.m, a.k, kw, L.m_pad, ws + L.bwd_ar);
  pk.rows(a.dout, a.o_sr, a.m, a.p, pw, L.m_pad, ws + L.bwd_dor);
  pk.cols(a.bt, a.bt_sr, a.n, a.k, kw, L.n_pad, ws + L.bwd_btc);
  pk.cols(a.a, a.a_sr, a.m, a.k, kw, L.m_pad, ws + L.bwd_ac);
  pk.cols(a.dout, a.o_sr, a.m, a.p, pw, L.m_pad, ws + L.bwd_doc);
  hipError_t e = pk.run(s);
  if (e != hipSuccess) return e;
  e = dispatch_kp(kw, pw, [&]<int K, int P>() { return bwd_kp<K, P>(a, L, ws, pa, pb, pc, s); });
  if (e != hipSuccess) return e;
  Reducer rd;
  rd.add(pa, L.split_rows, a.m, a.k, a.scale, a.da, a.a_sr);
  rd.add(pb, L.split_cols, a.n, a.k, a.scale, a.dbt, a.bt_sr);
  rd.add(pc, L.split_dc, a.n, a.p, 1.f, a.dc, a.c_sr);
  return rd.run(s);
}

}  // namespace fab
