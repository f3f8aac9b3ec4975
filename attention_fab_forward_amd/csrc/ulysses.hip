// Local layout steps around the all-to-all exchanges of Ulysses sequence
// parallelism ("Ulysses Sequence Parallelism", sections "Contexte Technique"
// and "Analyse"; "AutoSP" section 2, communication inserted at the attention
// boundaries).  Before the first exchange each of the p ranks holds n_local
// consecutive tokens of all H heads; after it, every rank holds all
// n = p * n_local tokens of its own Hl = H / p heads.  The second exchange,
// after attention, goes back.
//
// Exchange buffer (what one rank sends, and what it receives): [p][n_local]
// [b][Hl][d], one contiguous [n_local][b][Hl][d] block per peer, so an
// all-to-all with equal splits moves block j of rank s to block s of rank j.
// On the receiving side the p blocks of n_local tokens follow each other in
// sequence order, i.e. the buffer is [n][b][Hl][d]: the attention kernels read
// it in place (batch stride Hl d, head stride d, row stride b Hl d) and write
// their output in the same layout, which is the send buffer of the return
// exchange.  Only two reorderings therefore touch memory:
//   pack:   send[j][t][bi][hl] = x[bi][t][head0(j) + hl]
//   unpack: x[bi][t][h] = sum over the ranks j that hold head h of
//           recv[j][t][bi][h - head0(j)],
// with head0(j) = floor(j H / p).  When H < p (grouped-query key/value heads)
// Hl = 1 and head h goes to the p / H consecutive ranks whose query heads
// read it; unpacking gradients then sums those ranks' contributions (fp32,
// in rank order, rounded once).
//
// Both kernels are pure data movement (HBM bound): each thread moves one 16
// byte chunk, threads in index order of the written tensor so stores are
// coalesced, reads are runs of Hl (pack) or one head (unpack) rows.
#include "fab_device.h"
#include "fab_internal.h"

namespace fab {
namespace {

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
  return (__umulhi(n, f.m) + n) >> f.s;
}

__device__ __forceinline__ void add_chunk(f32x4 (&acc)[2], const u32x4& v, bool bf16) {
  if (bf16) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc[w / 2][2 * (w % 2)] += bf16_lo(v[w]);
      acc[w / 2][2 * (w % 2) + 1] += bf16_hi(v[w]);
    }
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) acc[0][w] += __uint_as_float(v[w]);
  }
}

// send [p][n_local][b][Hl][d] <- x; one 16-byte chunk per thread.
__global__ __launch_bounds__(256) void ulysses_pack_kernel(UlyssesArgs a) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i >= a.total) return;
  const uint32_t row = fdiv(i, a.div_cpr), k = i - row * a.cpr;    // row of send, chunk
  const uint32_t r1 = fdiv(row, a.div_hl), hl = row - r1 * a.hl;  // (tok, bi), head slot
  const uint32_t tok = fdiv(r1, a.div_b), bi = r1 - tok * a.b;    // j n_local + t, batch
  const uint32_t j = fdiv(tok, a.div_nl), t = tok - j * a.n_local;
  const uint32_t head = fdiv(j * a.heads, a.div_p) + hl;
  const char* src = static_cast<const char*>(a.src) +
                    ((int64_t)bi * a.x_sb + (int64_t)t * a.x_sr + (int64_t)head * a.x_sh) * a.esize +
                    16 * k;
  stg16(static_cast<char*>(a.dst) + (int64_t)i * 16, ldg16(src));
}

// x <- recv [p][n_local][b][Hl][d], summing the replicas of a head.
__global__ __launch_bounds__(256) void ulysses_unpack_kernel(UlyssesArgs a) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i >= a.total) return;
  const uint32_t row = fdiv(i, a.div_cpr), k = i - row * a.cpr;    // row of x in [b][t][h]
  const uint32_t r1 = fdiv(row, a.div_h), h = row - r1 * a.heads;
  const uint32_t bi = fdiv(r1, a.div_nl), t = r1 - bi * a.n_local;
  const uint32_t j0 = fdiv(h * a.p, a.div_h);                     // first rank holding h
  const uint32_t hl = h - fdiv(j0 * a.heads, a.div_p);
  const int64_t rank_stride = (int64_t)a.n_local * a.b * a.hl;   // rows per peer block
  const int64_t rrow = ((int64_t)t * a.b + bi) * a.hl + hl;
  const char* src = static_cast<const char*>(a.src) + ((int64_t)j0 * rank_stride + rrow) * a.row_bytes + 16 * k;
  char* dst = static_cast<char*>(a.dst) +
              ((int64_t)bi * a.x_sb + (int64_t)t * a.x_sr + (int64_t)h * a.x_sh) * a.esize + 16 * k;
  if (a.replicas == 1) {
    stg16(dst, ldg16(src));
    return;
  }
  const bool bf16 = a.esize == 2;
  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  for (uint32_t r = 0; r < a.replicas; ++r)
    add_chunk(acc, ldg16(src + r * rank_stride * a.row_bytes), bf16);
  u32x4 v;
  if (bf16) {
#pragma unroll
    for (int w = 0; w < 4; ++w) v[w] = pack_bf16(acc[w / 2][2 * (w % 2)], acc[w / 2][2 * (w % 2) + 1]);
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) v[w] = __float_as_uint(acc[0][w]);
  }
  stg16(dst, v);
}

}  // namespace

FastDiv make_fastdiv(uint32_t d) {
  // Division by an invariant integer through a round-up multiplier
  // (Granlund and Montgomery, PLDI 1994): with s = ceil(log2 d) and
  // m = floor(2^32 (2^s - d) / d) + 1, n / d = (umulhi(n, m) + n) >> s for
  // every n < 2^31 (the sum cannot overflow 32 bits there).
  FastDiv f{};
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  f.s = s;
  f.m = (uint32_t)((((1ull << s) - d) << 32) / d + 1);
  return f;
}

hipError_t launch_ulysses(const UlyssesArgs& a, bool pack, hipStream_t s) {
  if (a.total == 0) return hipSuccess;
  const dim3 grid((a.total + 255) / 256), block(256);
  if (pack)
    hipLaunchKernelGGL(ulysses_pack_kernel, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(ulysses_unpack_kernel, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace fab
