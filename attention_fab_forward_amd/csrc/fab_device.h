// Device-side helpers shared by the HIP kernels of the fused f(A.B).C block:
// MFMA wrappers for gfx950, bf16 packing, 16-byte global/LDS moves and the
// lane permutation used to keep MFMA accumulator slots on contiguous indices.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fab {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D = A (32x16) * B (16x32) + C, bf16 inputs, fp32 accumulate.
// Lane l supplies A[l%32][8*(l/32)+e] and B[8*(l/32)+e][l%32], e = 0..7, and
// holds D[8*(r/4) + 4*(l/32) + r%4][l%32] in accumulator slot r = 0..15.
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// MFMA row index r (0..31) of a 32-row operand -> the tile row it carries.
// Chosen so that accumulator slot s of lane l corresponds to tile row
// 16*(l/32) + s: rows of one lane become contiguous.
__device__ __forceinline__ int perm_row(int r) {
  return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
}
// Inverse of perm_row: tile row -> MFMA row that must carry it.
__device__ __forceinline__ int perm_row_inv(int t) {
  const int g = t >> 4, i = t & 15;
  return 8 * (i >> 2) + 4 * g + (i & 3);
}

// fp32 -> bf16 pair, round to nearest even (gfx950 hardware conversion).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 b = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Combine the low (sel=0) or high (sel=1) 16-bit halves of two words.
__device__ __forceinline__ uint32_t pick_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pick_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ u32x4 ldg16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void stg16(void* p, const u32x4& v) {
  *reinterpret_cast<u32x4*>(p) = v;
}
__device__ __forceinline__ u32x4 lds16(const char* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void sts16(char* p, const u32x4& v) {
  *reinterpret_cast<u32x4*>(p) = v;
}
__device__ __forceinline__ void sts8(char* p, const u32x2& v) {
  *reinterpret_cast<u32x2*>(p) = v;
}
__device__ __forceinline__ void sts4(char* p, uint32_t v) {
  *reinterpret_cast<uint32_t*>(p) = v;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane i receives element j = element (i % 4) of the 8-byte value
// addressed by lane 4 j + i / 4 of the same group.
__device__ __forceinline__ u32x2 lds_tr8(const char* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Asynchronous 16-byte global -> LDS copy (global_load_lds_dwordx4): lane i of
// the wave writes LDS bytes [lds_base + 16 i, lds_base + 16 i + 16).  lds_base
// must be wave-uniform.  Completion is tracked by the vector-memory counter.
// Asynchronous global -> LDS copies (gfx950 global_load_lds): lane i's bytes
// land at LDS byte address lds + size * i, lds wave-uniform (passed in M0).
// They are issued as inline assembly so the compiler does not track them: its
// own tracking waits for every copy in flight before any transposing LDS
// read, which would serialise the prefetch with the compute.  Callers wait
// for their copies (wait_vmem) before the barrier that publishes them, and no
// compiler-generated code here keeps a value in M0.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane from base + voff (base wave-uniform, voff per lane, >= 0).
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, const char* lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_addr(lds)), "v"(voff), "s"(base)
               : "memory", "m0");
}
// 16 bytes per lane from a per-lane 64-bit address.
__device__ __forceinline__ void dma16_at(const void* addr, const char* lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds_addr(lds)), "v"(addr)
               : "memory", "m0");
}
// 4 bytes per lane from a per-lane 64-bit address.
__device__ __forceinline__ void dma4_at(const void* addr, const char* lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :
               : "s"(lds_addr(lds)), "v"(addr)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Software-pipelined run of N MFMAs whose A operands come from LDS:
// read(i) issues the LDS reads of operand i, mma(i, x) consumes it.  Operands
// are requested DEPTH MFMAs ahead through a ring of DEPTH registers sets, and
// scheduling barriers (VALU, SALU and transcendental work may still move
// across them) keep the compiler from sinking the reads next to their uses.
template <int N, int DEPTH, class Read, class Mma>
__device__ __forceinline__ void lds_mfma_pipeline(Read read, Mma mma) {
  u32x4 buf[DEPTH];
#pragma unroll
  for (int i = 0; i < DEPTH && i < N; ++i) buf[i] = read(i);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    mma(i, buf[i % DEPTH]);
    if (i + DEPTH < N) buf[i % DEPTH] = read(i + DEPTH);
    __builtin_amdgcn_sched_barrier(0x0406);
  }
}

// Workgroup barrier ordering LDS accesses only: unlike __syncthreads it does
// not wait for outstanding global memory operations (the copies in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// s_waitcnt vmcnt(0) with the export and LDS counters left unconstrained
// (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// Waits until at most N of this wave's vector memory operations are
// outstanding; they complete in issue order, so this waits for all but the
// last N issued (a copy pipeline keeps its newest tiles in flight).  Assembly
// with a memory clobber, so LDS accesses stay on their side of it.
template <int N>
__device__ __forceinline__ void wait_copies() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Sum over aligned groups of T consecutive lanes (T a power of two up to 64),
// returned in every lane of the group: DPP moves folded into the adds inside
// each 16-lane DPP row (neighbour and pair swaps within quads, after which
// each quad holds its sum in every lane, then the half-row and row mirrors,
// which pair the quads and the 8-lane halves), a lane exchange beyond.  The
// additions are those of an xor butterfly, so the sum is the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}
template <int T>
__device__ __forceinline__ float lane_group_sum(float v) {
  static_assert(T >= 1 && T <= 64 && (T & (T - 1)) == 0, "a power of two up to 64 lanes");
  if constexpr (T >= 2) v += dpp_move<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  if constexpr (T >= 4) v += dpp_move<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  if constexpr (T >= 8) v += dpp_move<0x141>(v);  // row_half_mirror
  if constexpr (T >= 16) v += dpp_move<0x140>(v); // row_mirror
  if constexpr (T >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (T >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

// Combine each lane's value with that of lane l ^ 32 (v_permlane32_swap:
// afterwards one register holds x[l % 32], the other x[l % 32 + 32] in every
// lane).
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}


// Workgroup i runs on XCD i % 8 (8 XCDs, each with its own L2).  Maps i to
// (head slot, block) for H head slots of nb blocks each, block 0 being the
// longest (causal work varies along the blocks), so that the workgroups an XCD
// runs together share one head's K / V in its L2 and every XCD gets the same
// mix of long and short blocks:
//  * H a multiple of 8: XCD x takes whole heads [x H / 8, (x + 1) H / 8), head
//    by head, blocks in order;
//  * 8 a multiple of H (and s = 8 / H dividing nb): head x / s is spread over s
//    XCDs, XCD x taking its blocks x % s, x % s + s, ... in order;
//  * otherwise plain head-major order.
// Bijective on [0, H nb) in every case.
__device__ __forceinline__ void xcd_map(int i, int H, int nb, int& head, int& blk) {
  if (H % 8 == 0) {
    const int per = H / 8 * nb;
    const int lid = (i % 8) * per + i / 8;
    head = lid / nb;
    blk = lid % nb;
  } else if (8 % H == 0 && nb % (8 / H) == 0) {
    const int s = 8 / H, x = i % 8;
    head = x / s;
    blk = x % s + s * (i / 8);
  } else {
    head = i / nb;
    blk = i % nb;
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace fab
