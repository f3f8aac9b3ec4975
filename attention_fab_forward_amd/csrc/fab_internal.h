// Host/device argument blocks and kernel launchers of the fused f(A.B).C
// library.  Host code in fab_api.cpp validates a problem, fills these blocks
// and calls the launchers; each launcher enqueues its kernels on the given
// stream and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fab {

// Quotient by a divisor fixed at launch: (umulhi(n, m) + n) >> s, n < 2^31.
struct FastDiv {
  uint32_t m, s;
};
FastDiv make_fastdiv(uint32_t d);

// Softmax attention: A = Q [b, m, hq, d], Bt = K [b, n, hkv, d], C = V [b, n, hkv, d].
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;      // forward output (read by the backward)
  void* o_out;        // forward output (written by the forward)
  float* lse;         // [b, hq, m] natural log
  const float* lse_in;
  const void* dout;   // dO, layout of O
  void* dq;           // layout of Q
  void* dk;           // layout of K
  void* dv;           // layout of V
  float* delta;       // workspace [b, hq, m]: rowsum(dO * O); negated on the bf16 path
  float* lse2;        // workspace [b, hq, m] (bf16 path): LSE * log2(e)
  int64_t q_sb, q_sh, q_sr;
  int64_t k_sb, k_sh, k_sr;
  int64_t v_sb, v_sh, v_sr;
  int64_t o_sb, o_sh, o_sr;
  int32_t b, hq, hkv, m, n;
  int32_t group;      // hq / hkv
  float scale;        // softmax scale
  float scale_log2;   // scale * log2(e)
  int32_t causal;
  // causal: key j is visible to query i iff j <= i + diag (diag = global
  // query offset - key offset, clamped to [-m - 1, n]: beyond that range every
  // row sees all keys or none)
  int32_t diag;
  // row index splits of [b, m, hq] by multiplication (when b hq m < 2^31)
  int32_t rows_small;
  FastDiv div_hq, div_m;
};

// Merge of two partial softmax results (fab_merge): packed LSE [b, hq, m].
struct MergeArgs {
  const void* oa;
  const void* ob;
  void* oo;
  const float* la;
  const float* lb;
  float* lo;
  int64_t o_sb, o_sh, o_sr;
  int32_t b, hq, m;
  int32_t small;          // b * hq * m < 2^31: the divisions below apply
  FastDiv div_hq, div_m;
};

// Ulysses exchange layout (fab_ulysses_pack / _unpack).  x [b, n_local, H, d]
// with element strides; exchange buffer [p][n_local][b][Hl][d] packed.
// pack: src = x, dst = buffer; unpack: src = buffer, dst = x.
struct UlyssesArgs {
  const void* src;
  void* dst;
  uint32_t total;      // 16-byte chunks written
  uint32_t cpr;        // chunks per head row (d * esize / 16)
  uint32_t hl, b, n_local, heads, p, replicas, esize;
  int64_t row_bytes;   // d * esize
  int64_t x_sb, x_sr, x_sh;
  FastDiv div_cpr, div_hl, div_b, div_nl, div_p, div_h;
};

// GeLU MLP: A [m, k], Bt [n, k], C [n, p], O [m, p] (row strides in elements).
struct MlpArgs {
  const void* a;
  const void* bt;
  const void* c;
  void* o;
  const void* dout;
  void* da;
  void* dbt;
  void* dc;
  float* ws;          // fp32 workspace
  int64_t a_sr, bt_sr, c_sr, o_sr;
  int32_t m, n, k, p;
  int32_t splits;     // n-splits of the forward partial sums
  float scale;
};

constexpr float kLog2eHost = 1.4426950408889634f;

// Optional per-kernel timing of one call (see fab_plan_set_timing): launchers
// bracket every kernel they enqueue with these; both are no-ops unless the
// calling thread is inside a timed fab_forward / fab_backward.
void timer_begin(const char* kernel, hipStream_t s);
void timer_end(hipStream_t s);

// Bracket a kernel launch: FAB_TIMED("name", stream, hipLaunchKernelGGL(...)).
#define FAB_TIMED(name, stream, ...) \
  do {                               \
    ::fab::timer_begin(name, stream); \
    __VA_ARGS__;                     \
    ::fab::timer_end(stream);        \
  } while (0)

// Forward attention tile shapes (bf16 MFMA path).
#ifndef FAB_FWD_QT
#define FAB_FWD_QT 1
#endif
#ifndef FAB_FWD_WAVES
#define FAB_FWD_WAVES 8
#endif
constexpr int kAttnFwdQT = FAB_FWD_QT;        // 32-query MFMA tiles per wave
constexpr int kAttnFwdWaves = FAB_FWD_WAVES;  // waves per workgroup
constexpr int kAttnFwdBM = 32 * kAttnFwdWaves * kAttnFwdQT;  // queries per workgroup
constexpr int kAttnFwdBN = 64;    // keys per inner step
#ifndef FAB_BWD_QT
#define FAB_BWD_QT 1
#endif
#ifndef FAB_DQ_WAVES
#define FAB_DQ_WAVES 8
#endif
constexpr int kAttnBwdQT = FAB_BWD_QT;        // dQ kernel: 32-query tiles per wave
constexpr int kAttnDqWaves = FAB_DQ_WAVES;    // dQ kernel: waves per workgroup
constexpr int kAttnBwdBM = 32 * kAttnDqWaves * kAttnBwdQT;  // dQ kernel: queries per workgroup
constexpr int kAttnBwdKB = 128;   // dK/dV kernel: keys per workgroup (4 waves x 32)
constexpr int kAttnBwdQB = 64;    // dK/dV kernel: queries per inner step

hipError_t launch_attn_fwd_bf16(const AttnArgs& a, int d, hipStream_t s);
hipError_t launch_attn_merge(const MergeArgs& a, int d, bool bf16, hipStream_t s);
hipError_t launch_attn_bwd_bf16(const AttnArgs& a, int d, hipStream_t s);
hipError_t launch_attn_fwd_f32(const AttnArgs& a, int d, hipStream_t s);
hipError_t launch_attn_bwd_f32(const AttnArgs& a, int d, hipStream_t s);
hipError_t launch_attn_fwd_f32_mfma(const AttnArgs& a, int d, hipStream_t s);
hipError_t launch_attn_bwd_f32_mfma(const AttnArgs& a, int d, hipStream_t s);

hipError_t launch_ulysses(const UlyssesArgs& a, bool pack, hipStream_t s);

int exp_probe_chains();
hipError_t launch_exp_probe(int blocks, int iters, float* sink, hipStream_t s);

// k, p pairs the GeLU MLP kernels are built for
bool mlp_shape_supported(int k, int p);
size_t mlp_fwd_workspace(int m, int n, int k, int p, int* splits);
size_t mlp_bwd_workspace(int m, int n, int k, int p);
hipError_t launch_mlp_fwd_bf16(const MlpArgs& a, hipStream_t s);
hipError_t launch_mlp_bwd_bf16(const MlpArgs& a, hipStream_t s);

}  // namespace fab
