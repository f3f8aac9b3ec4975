/*
 * fab.h -- C ABI of the fused two-matmul block  O = f(A . B) . C  on MI355X.
 *
 * The unit: two consecutive matrix products with a function between them
 * ("Memory-efficient tensor parallelism", FITEE 10.1631/FITEE.2400602,
 * abstract).  f is either
 *   - a scaled row softmax over the n axis, optionally under a causal index
 *     mask (attention; "Ulysses Sequence Parallelism", section "Contexte
 *     Technique"; causal masks as index tensors: "AutoSP", section 2.A), or
 *   - GeLU in its erf form, applied elementwise (the MLP block; "AutoSP",
 *     sections 2.A and 2.B).
 * The m x n intermediate f(A.B) is computed tile by tile on chip and never
 * written to device memory; the backward pass recomputes it from the saved
 * per-row log-sum-exp (softmax) or from A and B (GeLU) instead of storing it
 * ("AutoSP", section 2.B: rematerialise rather than keep activations).
 *
 * Shapes (per batch entry and head):
 *   A  : m x k      (attention: Q, one query head)
 *   Bt : n x k      (B transposed; attention: K.  MLP: nn.Linear weight layout)
 *   C  : n x p      (attention: V)
 *   O  : m x p
 * softmax: O_i = sum_j P_ij C_j, P_ij = exp(S_ij - LSE_i),
 *          S = scale * A Bt^T, masked S_ij = -inf when causal and key j lies
 *          after query i (global positions: k_offset + j > q_offset + i),
 *          LSE_i = log sum_j exp(S_ij) (natural log).  A row that sees no key
 *          gets O_i = 0 and LSE_i = -inf.
 * GeLU:    O = GeLU(scale * A Bt^T) C, GeLU(x) = x * Phi(x).
 *
 * Layout: every matrix has a contiguous last dimension.  Attention tensors are
 * addressed as base + b*stride_batch + h*stride_head + row*stride_row + col
 * (elements); leaving all three strides 0 selects the packed
 * [batch, rows, heads, cols] layout.  Query head h reads key/value head
 * h / (heads_a / heads_bc) (consecutive query heads share a kv head).
 * Gradients use the strides of their primal tensor (dA like A, dO like O, ...).
 * LSE is packed [batch, heads_a, m] float32.
 *
 * Ownership: the caller owns every device buffer.  The library allocates no
 * device memory (its one static array, the 32 MiB scratch of
 * fab_backward_noalloc, is reserved by the HIP runtime when it loads the
 * library's device code on a GPU) and never synchronises: all work is
 * enqueued on the caller's stream.  Temporary device memory is passed in as `workspace`, whose size
 * fab_plan reports.  Outputs are overwritten, not accumulated.  A plan is an
 * immutable host object; one plan may serve concurrent calls that use
 * distinct workspaces.
 *
 * Errors: every entry point returns a fab_status synchronously and never
 * throws or aborts.  FAB_ERR_HIP reports a launch error; a fault inside a
 * kernel surfaces at the caller's next synchronisation.  fab_last_error()
 * returns a thread-local description of the last failure on this thread.
 */
#ifndef FAB_H
#define FAB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FAB_ABI_VERSION 3

typedef enum {
  FAB_OK = 0,
  FAB_ERR_NULL_ARG = 1,             /* a required pointer is NULL            */
  FAB_ERR_BAD_SHAPE = 2,            /* sizes < 1, heads_a % heads_bc != 0, ... */
  FAB_ERR_UNSUPPORTED = 3,          /* valid problem this build does not run */
  FAB_ERR_ALIGNMENT = 4,            /* base not 16-byte aligned / bad stride  */
  FAB_ERR_WORKSPACE_TOO_SMALL = 5,  /* workspace_bytes below the plan's need */
  FAB_ERR_ABI_VERSION = 6,          /* prob->abi_version != FAB_ABI_VERSION  */
  FAB_ERR_HIP = 7                   /* the HIP runtime reported an error     */
} fab_status;

typedef enum { FAB_F_SOFTMAX = 0, FAB_F_GELU_ERF = 1 } fab_function;
typedef enum { FAB_MASK_NONE = 0, FAB_MASK_CAUSAL = 1 } fab_mask;
typedef enum { FAB_BF16 = 0, FAB_F32 = 1 } fab_dtype;
/* Kernel family of an fp32 softmax problem (any other problem takes 0):
 * FAB_VARIANT_F32_FMA, plain fp32 FMA kernels (for small problems, where
 * launch latency dominates); FAB_VARIANT_F32_MFMA, the fp32 matrix cores
 * (v_mfma_f32_32x32x2_f32).  Both compute in fp32 throughout; 0 chooses by
 * size (the matrix cores once batch * heads_a * ceil(m / 64) >= 32 at
 * k = 128, or >= 64 at k = 64, and there are 2^22 or more unmasked (query,
 * key) pairs). */
typedef enum { FAB_VARIANT_AUTO = 0, FAB_VARIANT_F32_FMA = 1, FAB_VARIANT_F32_MFMA = 2 } fab_variant;

/* Full description of one problem.  Zero-initialise, then fill in. */
typedef struct {
  int32_t abi_version; /* must be FAB_ABI_VERSION                             */
  int32_t f;           /* fab_function                                        */
  int32_t mask;        /* fab_mask; GeLU requires FAB_MASK_NONE               */
  int32_t dtype;       /* fab_dtype of A, Bt, C, O, dO and all gradients       */
  int64_t batch;       /* >= 1                                                */
  int64_t heads_a;     /* heads of A and O (query heads); >= 1                */
  int64_t heads_bc;    /* heads of Bt and C (kv heads); divides heads_a       */
  int64_t m, n, k, p;  /* matrix sizes above                                  */
  float scale;         /* f is applied to scale * (A Bt^T)                    */
  int32_t variant;     /* fab_variant: 0 lets the library choose             */
  /* element strides {batch, head, row}; all-zero = packed [b, rows, h, cols] */
  int64_t a_stride[3];
  int64_t bt_stride[3];
  int64_t c_stride[3];
  int64_t o_stride[3];
  /* Causal mask positions: query row i sits at global position q_offset + i,
   * key row j at k_offset + j (a rank or a split holding a slice of the
   * sequence; "Ulysses Sequence Parallelism", Analyse: ring attention passes
   * key blocks between ranks).  Only the difference matters; both 0 for the
   * plain causal mask over one full sequence.  Must be 0 for GeLU. */
  int64_t q_offset;
  int64_t k_offset;
} fab_problem;

typedef struct fab_plan_s fab_plan_t;

/* Validate `prob` and build a reusable plan.  Host only: touches no device.
 * Supported in this build:
 *   softmax, bf16: k == p, k in {64, 128}; any m, n >= 1; causal with any
 *                  offsets.
 *   softmax, f32:  k == p, k in {64, 128}; same rules.
 *   GeLU, bf16:    batch == heads_a == heads_bc == 1, each of k and p a
 *                  multiple of 64 from 64 to 1024, any m, n >= 1, mask NONE
 *                  (the kernels run at the next width of 128, 256, 512 or
 *                  1024, with the operands zero-padded in the workspace).
 * Row strides must be multiples of 8 elements (bf16) or 4 (f32), and so must
 * the head and batch strides; softmax row strides stay below 2^24 elements.  O's strides must give every output element its
 * own address (no zero or overlapping batch / head strides): FAB_ERR_BAD_SHAPE
 * otherwise.  A, Bt and C may be broadcast (say a zero head stride) for the
 * forward; fab_backward refuses such a plan, since each gradient takes its
 * primal's layout.  On success *plan_out receives a plan that the
 * caller releases with fab_plan_destroy, and the two sizes receive the bytes
 * of device workspace fab_forward / fab_backward need (either size pointer
 * may be NULL).  On failure *plan_out is set to NULL. */
fab_status fab_plan(const fab_problem* prob, fab_plan_t** plan_out,
                    size_t* fwd_workspace_bytes, size_t* bwd_workspace_bytes);

/* Forward pass: O = f(scale * A Bt^T) C, and for softmax the fp32 LSE rows.
 * A, Bt, C, O: device pointers in the plan's dtype and strides.
 * lse: device float32 [batch, heads_a, m] for softmax (required), NULL for GeLU.
 * workspace: device memory of at least the plan's forward size (may be NULL if
 * that size is 0).  Enqueued on `stream` (a hipStream_t; NULL = default). */
fab_status fab_forward(const fab_plan_t* plan, const void* A, const void* Bt,
                       const void* C, void* O, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Backward pass of L = <dO, O>: dA, dBt, dC (attention: dQ, dK, dV).
 * O and lse must be what fab_forward returned for the same inputs (softmax;
 * pass NULL for both with GeLU).  dO has O's layout; dA, dBt, dC have the
 * layouts of A, Bt, C and are overwritten (FAB_ERR_BAD_SHAPE if one of those
 * layouts maps two elements to one address).  workspace: at least the plan's
 * backward size.  Enqueued on `stream`. */
fab_status fab_backward(const fab_plan_t* plan, const void* A, const void* Bt,
                        const void* C, const void* O, const float* lse,
                        const void* dO, void* dA, void* dBt, void* dC,
                        void* workspace, size_t workspace_bytes, void* stream);

/* fab_backward for callers that cannot allocate device memory at all (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same kernels and results, with the workspace taken from a
 * scratch array of 32 MiB that the library holds statically on each GPU it
 * runs on (from when its device code is loaded there until the process
 * ends).  The
 * caller passes inputs and outputs only; nothing is allocated or freed.
 * A plan whose backward workspace exceeds 32 MiB is refused with
 * FAB_ERR_WORKSPACE_TOO_SMALL (the attention backward needs 8 bytes per
 * query row and head, so up to 4 Mi (row, head) pairs fit).  All calls on one
 * GPU share that array: calls that overlap in time on one GPU (say on two
 * streams) race on it and must be ordered by the caller.  Arguments,
 * layouts and errors are as for fab_backward; FAB_ERR_HIP also reports a
 * failed lookup of the array's device address. */
fab_status fab_backward_noalloc(const fab_plan_t* plan, const void* A, const void* Bt,
                                const void* C, const void* O, const float* lse,
                                const void* dO, void* dA, void* dBt, void* dC, void* stream);

/* Merge two softmax results over disjoint key sets of the same queries (for
 * instance two key ranges computed by fab_forward with k_offset set): with
 * weights w_x = exp(LSE_x - LSE),
 *   LSE = log(exp(LSE_a) + exp(LSE_b)),  O = w_a O_a + w_b O_b,
 * which is the result over the union of the key sets (the ring / key-sharded
 * attention step: "Ulysses Sequence Parallelism", Analyse; FITEE abstract,
 * B and C exchanged in sub-blocks).  Applied pairwise it merges any number of
 * parts in any order.
 * plan: a softmax plan; O_a, O_b, O_out: device pointers with the plan's O
 * layout and dtype; lse_a, lse_b, lse_out: device float32 [batch, heads_a, m].
 * O_out / lse_out may be O_a / lse_a (in-place accumulation) but must not
 * partially overlap any input.  A row whose two LSE are both -inf gets O = 0,
 * LSE = -inf.  Computed in fp32, O rounded to the dtype.  Enqueued on stream.
 * Backward over key ranges: pass the merged O and LSE to fab_backward for
 * each range; dK, dV are that range's, and dA is its contribution to dQ (the
 * caller sums the ranges' dA). */
fab_status fab_merge(const fab_plan_t* plan, const void* O_a, const float* lse_a,
                     const void* O_b, const float* lse_b, void* O_out, float* lse_out,
                     void* stream);

/* ---------------------------------------------------------------------------
 * Layout steps around the two all-to-all exchanges of Ulysses sequence
 * parallelism ("Ulysses Sequence Parallelism", sections "Contexte Technique"
 * and "Analyse"; "AutoSP" section 2: exchanges inserted at the attention
 * boundaries, attention on the full sequence for a subset of heads).  Before
 * the first exchange each of the p ranks holds n_local consecutive tokens of
 * all H heads (x [b, n_local, H, d], rank j's tokens being j n_local ..
 * j n_local + n_local - 1); afterwards each rank holds all n = p n_local
 * tokens of Hl heads.  The exchanges themselves are the caller's (one
 * all-to-all with equal splits of a buffer of fab_ulysses_sizes' elements).
 *
 * Exchange buffer: [p][n_local][b][Hl][d], packed.  Block j of a rank's send
 * buffer goes to rank j; block s of its receive buffer came from rank s.  A
 * receive buffer therefore reads as [n][b][Hl][d]: pass it to fab_plan /
 * fab_forward directly with element strides {batch Hl d, head d, row b Hl d},
 * and give O (and dQ, dK, dV) the same strides: that output is the send
 * buffer of the return exchange, whose receive buffer fab_ulysses_unpack
 * turns back into x's layout.
 *
 * Heads: with head0(j) = floor(j H / p), rank j receives heads head0(j) ..
 * head0(j) + Hl - 1.  H % p == 0 gives Hl = H / p (disjoint head groups).
 * p % H == 0 (fewer key/value heads than ranks under grouped-query attention)
 * gives Hl = 1: head h goes to the p / H consecutive ranks whose query heads
 * read it, and fab_ulysses_unpack sums what those ranks return (the gradient
 * of a replicated head), in fp32, in rank order, rounded once to the dtype.
 * Any other H, p pair is FAB_ERR_BAD_SHAPE.
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t abi_version; /* must be FAB_ABI_VERSION                               */
  int32_t dtype;       /* fab_dtype of x and of the exchange buffer              */
  int64_t batch;       /* b >= 1                                                */
  int64_t n_local;     /* tokens per rank before the exchange, >= 1             */
  int64_t heads;       /* H, heads of x, >= 1                                   */
  int64_t head_dim;    /* d; d * element size must be a multiple of 16 bytes    */
  int64_t ranks;       /* p >= 1                                                */
  /* element strides {batch, head, row} of x; all-zero = packed [b, n_local, H, d];
   * multiples of 16 bytes, last dimension contiguous */
  int64_t x_stride[3];
} fab_ulysses_layout;

/* Validates the layout; *heads_per_rank receives Hl and *buffer_elems the
 * elements of one exchange buffer (p n_local b Hl d).  Either output may be
 * NULL.  Host only. */
fab_status fab_ulysses_sizes(const fab_ulysses_layout* layout, int64_t* heads_per_rank,
                             int64_t* buffer_elems);

/* send[j][t][bi][hl][:] = x[bi][t][head0(j) + hl][:] for every rank j (a
 * pure copy, bit-exact).  x: device, the layout's strides; send: device,
 * buffer_elems elements, must not overlap x.  Both 16-byte aligned.  Enqueued
 * on `stream` (a hipStream_t; NULL = default). */
fab_status fab_ulysses_pack(const fab_ulysses_layout* layout, const void* x, void* send,
                            void* stream);

/* x[bi][t][h][:] = sum over the ranks j holding head h of
 * recv[j][t][bi][h - head0(j)][:]; one term (a bit-exact copy) unless H < p.
 * recv: device, buffer_elems elements; x: device, the layout's strides,
 * overwritten, must not overlap recv.  Both 16-byte aligned.  Enqueued on
 * `stream`. */
fab_status fab_ulysses_unpack(const fab_ulysses_layout* layout, const void* recv, void* x,
                              void* stream);

/* Release a plan (NULL is ignored). */
void fab_plan_destroy(fab_plan_t* plan);

/* Static English name of a status code. */
const char* fab_status_string(fab_status s);

/* Thread-local description of the last failure on the calling thread ("" if
 * none).  Valid until the next library call on this thread. */
const char* fab_last_error(void);

/* FAB_ABI_VERSION of the loaded library. */
int32_t fab_abi_version(void);

/* sizeof(fab_problem) as compiled into the library (binding layout check). */
size_t fab_problem_size(void);

/* Writes a one-line description of the plan's kernel variant, tiles and
 * grids into buf (truncated to len, always NUL-terminated when len > 0).
 * Returns the number of characters the full description needs. */
size_t fab_plan_describe(const fab_plan_t* plan, char* buf, size_t len);

/* Per-kernel timing, for measurement.  While enabled on a plan, every
 * fab_forward / fab_backward made with it records a HIP event on the caller's
 * stream before and after each kernel it enqueues (host-side event objects;
 * no device memory).  Calls on a plan with timing enabled must not overlap
 * across threads.  enable = 0 releases the events. */
fab_status fab_plan_set_timing(fab_plan_t* plan, int enable);

/* Waits for the recorded events, adds their durations into per-kernel totals
 * and writes up to `capacity` entries: kernel name (static string valid until
 * the next reset or fab_plan_set_timing), number of timed launches and total
 * milliseconds.  Any output pointer may be NULL.  Returns the number of
 * distinct kernels (0 if timing is off), or -1 on a HIP error. */
int fab_plan_kernel_times(fab_plan_t* plan, const char** names, int* counts,
                          double* total_ms, int capacity);

/* Waits for pending events and clears the per-kernel totals. */
fab_status fab_plan_reset_kernel_times(fab_plan_t* plan);

/* Rate probe of the softmax's per-element transcendental work (a secondary
 * bound of the attention kernels beside the MFMA rate): enqueues `blocks`
 * workgroups of 256 lanes, each lane running `iters` steps of 8 independent
 * chains x <- exp2(fma(x, a, b)) -- the form every probability takes -- and
 * writing one float to sink[lane index] (sink: device, blocks * 256 floats).
 * *exp_count receives the number of exponentials enqueued (may be NULL).
 * With sink NULL nothing is launched (count only).  The caller times the
 * stream; blocks in [1, 2^20], iters in [1, 2^24]. */
fab_status fab_exp_probe(int blocks, int iters, float* sink, int64_t* exp_count, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FAB_H */
