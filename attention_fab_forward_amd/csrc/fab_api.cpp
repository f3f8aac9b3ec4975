// C ABI of the fused f(A.B).C library: problem validation, plans, dispatch.
//
// Host-only code.  fab_plan checks a problem without touching the device;
// fab_forward / fab_backward check their pointers and workspace, then enqueue
// the kernels of the selected variant on the caller's stream.  No call
// allocates device memory or synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "fab.h"
#include "fab_internal.h"

namespace {

// Event-pair recorder behind fab_plan_set_timing.  Events are created once and
// reused; each record brackets one kernel on the stream it was launched on.
struct KernelTimer {
  struct Rec {
    const char* name;
    hipEvent_t start, stop;
  };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> free_events;
  std::map<std::string, std::pair<int, double>> totals;
  const char* pending = nullptr;
  hipEvent_t pending_start = nullptr;
  bool failed = false;

  hipEvent_t get() {
    if (!free_events.empty()) {
      hipEvent_t e = free_events.back();
      free_events.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) {
      failed = true;
      return nullptr;
    }
    return e;
  }
  void begin(const char* name, hipStream_t s) {
    pending = name;
    pending_start = get();
    if (pending_start && hipEventRecord(pending_start, s) != hipSuccess) {
      failed = true;
      free_events.push_back(pending_start);
      pending_start = nullptr;
    }
  }
  void end(hipStream_t s) {
    if (pending_start) {
      hipEvent_t stop = get();
      if (stop && hipEventRecord(stop, s) == hipSuccess) {
        recs.push_back({pending, pending_start, stop});
      } else {
        failed = true;
        free_events.push_back(pending_start);
        if (stop) free_events.push_back(stop);
      }
    }
    pending = nullptr;
    pending_start = nullptr;
  }
  // Waits for every recorded pair and folds it into the totals.
  void drain() {
    for (Rec& r : recs) {
      float ms = 0.f;
      if (hipEventSynchronize(r.stop) == hipSuccess && hipEventElapsedTime(&ms, r.start, r.stop) == hipSuccess) {
        auto& t = totals[r.name];
        t.first += 1;
        t.second += ms;
      } else {
        failed = true;
      }
      free_events.push_back(r.start);
      free_events.push_back(r.stop);
    }
    recs.clear();
  }
  ~KernelTimer() {
    for (Rec& r : recs) {
      (void)hipEventSynchronize(r.stop);
      free_events.push_back(r.start);
      free_events.push_back(r.stop);
    }
    for (hipEvent_t e : free_events) (void)hipEventDestroy(e);
  }
};

thread_local KernelTimer* t_active_timer = nullptr;

// Makes `timer` the target of timer_begin / timer_end for one library call.
struct TimerScope {
  explicit TimerScope(KernelTimer* timer) { t_active_timer = timer; }
  ~TimerScope() { t_active_timer = nullptr; }
};

}  // namespace

namespace fab {
void timer_begin(const char* kernel, hipStream_t s) {
  if (t_active_timer) t_active_timer->begin(kernel, s);
}
void timer_end(hipStream_t s) {
  if (t_active_timer) t_active_timer->end(s);
}
}  // namespace fab

struct fab_plan_s {
  std::mutex timer_mu;
  KernelTimer* timer = nullptr;  // owned; non-null while timing is enabled
  ~fab_plan_s() { delete timer; }
  fab_problem prob;
  int64_t as[3], bs[3], cs[3], os[3];  // resolved {batch, head, row} strides
  // no two (batch, head, row, col) indices of A / Bt / C share an address, so
  // their gradients (which take these layouts) can be written
  bool a_distinct, bt_distinct, c_distinct;
  size_t fwd_ws;
  size_t bwd_ws;
  int mlp_splits;
  bool f32_mfma;  // fp32 softmax on the matrix cores
  char desc[256];
};

namespace {

thread_local std::string g_last_error;

fab_status fail(fab_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

fab_status ok() {
  g_last_error.clear();
  return FAB_OK;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Resolve strides: all-zero means packed [batch, rows, heads, cols].
void resolve(const int64_t in[3], int64_t rows, int64_t heads, int64_t cols, int64_t out[3]) {
  if (in[0] == 0 && in[1] == 0 && in[2] == 0) {
    out[0] = rows * heads * cols;
    out[1] = cols;
    out[2] = heads * cols;
  } else {
    out[0] = in[0];
    out[1] = in[1];
    out[2] = in[2];
  }
}

fab_status check_strides(const char* name, const int64_t s[3], int64_t cols, int64_t unit) {
  for (int i = 0; i < 3; ++i) {
    if (s[i] < 0) return fail(FAB_ERR_BAD_SHAPE, "%s stride %d is negative", name, i);
    if (s[i] % unit)
      return fail(FAB_ERR_ALIGNMENT, "%s stride %d (%lld) is not a multiple of %lld elements",
                  name, i, (long long)s[i], (long long)unit);
  }
  if (s[2] < cols)
    return fail(FAB_ERR_BAD_SHAPE, "%s row stride %lld is smaller than its row length %lld", name,
                (long long)s[2], (long long)cols);
  return FAB_OK;
}

// True when the map (batch, head, row, col) -> element offset of a tensor of
// these sizes and strides is one-to-one, by the sufficient test that, with
// the dimensions of size > 1 sorted by stride, each stride reaches past the
// whole span of the smaller ones.  A zero batch or head stride (a tensor
// broadcast over heads) fails it.
bool distinct_layout(const int64_t s[3], int64_t batch, int64_t heads, int64_t rows,
                     int64_t cols) {
  struct Dim {
    int64_t size, stride;
  } d[4] = {{cols, 1}, {rows, s[2]}, {heads, s[1]}, {batch, s[0]}};
  std::sort(d, d + 4, [](const Dim& x, const Dim& y) { return x.stride < y.stride; });
  int64_t span = 0;  // largest offset reached by the dimensions seen so far
  for (const Dim& x : d) {
    if (x.size <= 1) continue;
    if (x.stride <= span) return false;
    span += (x.size - 1) * x.stride;
  }
  return true;
}

constexpr int64_t kMaxRows = (int64_t)1 << 30;

fab::AttnArgs attn_args(const fab_plan_s* p) {
  fab::AttnArgs a{};
  const fab_problem& q = p->prob;
  a.q_sb = p->as[0], a.q_sh = p->as[1], a.q_sr = p->as[2];
  a.k_sb = p->bs[0], a.k_sh = p->bs[1], a.k_sr = p->bs[2];
  a.v_sb = p->cs[0], a.v_sh = p->cs[1], a.v_sr = p->cs[2];
  a.o_sb = p->os[0], a.o_sh = p->os[1], a.o_sr = p->os[2];
  a.b = (int32_t)q.batch;
  a.hq = (int32_t)q.heads_a;
  a.hkv = (int32_t)q.heads_bc;
  a.m = (int32_t)q.m;
  a.n = (int32_t)q.n;
  a.group = (int32_t)(q.heads_a / q.heads_bc);
  a.scale = q.scale;
  a.scale_log2 = q.scale * fab::kLog2eHost;
  a.causal = q.mask == FAB_MASK_CAUSAL;
  const int64_t diag = q.q_offset - q.k_offset;
  a.diag = (int32_t)std::min<int64_t>(std::max<int64_t>(diag, -q.m - 1), q.n);
  a.rows_small = q.batch * q.heads_a * q.m < ((int64_t)1 << 31);
  a.div_hq = fab::make_fastdiv((uint32_t)q.heads_a);
  a.div_m = fab::make_fastdiv((uint32_t)q.m);
  return a;
}


// Validates a Ulysses exchange layout and fills the launch sizes; *hl and
// *elems receive the heads per rank and the exchange buffer's elements.
fab_status ulysses_setup(const fab_ulysses_layout* l, const char* who, bool pack,
                         fab::UlyssesArgs* a, int64_t* hl, int64_t* elems) {
  if (!l) return fail(FAB_ERR_NULL_ARG, "%s: layout is NULL", who);
  if (l->abi_version != FAB_ABI_VERSION)
    return fail(FAB_ERR_ABI_VERSION, "%s: abi_version %d, library has %d", who, l->abi_version,
                FAB_ABI_VERSION);
  if (l->dtype != FAB_BF16 && l->dtype != FAB_F32)
    return fail(FAB_ERR_UNSUPPORTED, "%s: unknown dtype %d", who, l->dtype);
  if (l->batch < 1 || l->n_local < 1 || l->heads < 1 || l->head_dim < 1 || l->ranks < 1)
    return fail(FAB_ERR_BAD_SHAPE, "%s: sizes must be >= 1 (batch %lld n_local %lld heads %lld "
                "head_dim %lld ranks %lld)", who, (long long)l->batch, (long long)l->n_local,
                (long long)l->heads, (long long)l->head_dim, (long long)l->ranks);
  if (l->heads % l->ranks != 0 && l->ranks % l->heads != 0)
    return fail(FAB_ERR_BAD_SHAPE, "%s: heads %lld and ranks %lld: one must divide the other", who,
                (long long)l->heads, (long long)l->ranks);
  const int64_t esize = l->dtype == FAB_BF16 ? 2 : 4;
  if ((l->head_dim * esize) % 16 != 0)
    return fail(FAB_ERR_ALIGNMENT, "%s: a head row (%lld elements) must be a multiple of 16 bytes",
                who, (long long)l->head_dim);
  int64_t xs[3];
  resolve(l->x_stride, l->n_local, l->heads, l->head_dim, xs);
  const fab_status st = check_strides("x", xs, l->head_dim, 16 / esize);
  if (st != FAB_OK) return st;
  const int64_t h_loc = l->heads >= l->ranks ? l->heads / l->ranks : 1;
  const int64_t cpr = l->head_dim * esize / 16;
  const int64_t rows_buf = l->ranks * l->n_local * l->batch * h_loc;
  const int64_t rows_x = l->batch * l->n_local * l->heads;
  const int64_t limit = (int64_t)1 << 31;
  if (l->ranks * l->heads >= limit || rows_buf > limit / cpr || rows_x > limit / cpr)
    return fail(FAB_ERR_UNSUPPORTED, "%s: more than 2^31 16-byte chunks (or heads * ranks >= "
                "2^31) is beyond this build's limits", who);
  *hl = h_loc;
  *elems = rows_buf * l->head_dim;
  a->total = (uint32_t)((pack ? rows_buf : rows_x) * cpr);
  a->cpr = (uint32_t)cpr;
  a->hl = (uint32_t)h_loc;
  a->b = (uint32_t)l->batch;
  a->n_local = (uint32_t)l->n_local;
  a->heads = (uint32_t)l->heads;
  a->p = (uint32_t)l->ranks;
  a->replicas = (uint32_t)(l->ranks > l->heads ? l->ranks / l->heads : 1);
  a->esize = (uint32_t)esize;
  a->row_bytes = l->head_dim * esize;
  a->x_sb = xs[0], a->x_sh = xs[1], a->x_sr = xs[2];
  a->div_cpr = fab::make_fastdiv(a->cpr);
  a->div_hl = fab::make_fastdiv(a->hl);
  a->div_b = fab::make_fastdiv(a->b);
  a->div_nl = fab::make_fastdiv(a->n_local);
  a->div_p = fab::make_fastdiv(a->p);
  a->div_h = fab::make_fastdiv(a->heads);
  return FAB_OK;
}

}  // namespace

extern "C" {

int32_t fab_abi_version(void) { return FAB_ABI_VERSION; }

size_t fab_problem_size(void) { return sizeof(fab_problem); }

const char* fab_status_string(fab_status s) {
  switch (s) {
    case FAB_OK: return "ok";
    case FAB_ERR_NULL_ARG: return "null argument";
    case FAB_ERR_BAD_SHAPE: return "bad shape";
    case FAB_ERR_UNSUPPORTED: return "unsupported problem";
    case FAB_ERR_ALIGNMENT: return "misaligned pointer or stride";
    case FAB_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case FAB_ERR_ABI_VERSION: return "ABI version mismatch";
    case FAB_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* fab_last_error(void) { return g_last_error.c_str(); }

fab_status fab_plan(const fab_problem* prob, fab_plan_t** plan_out, size_t* fwd_ws,
                    size_t* bwd_ws) {
  if (plan_out) *plan_out = nullptr;
  if (!prob || !plan_out) return fail(FAB_ERR_NULL_ARG, "fab_plan: prob and plan_out are required");
  const fab_problem& q = *prob;
  if (q.abi_version != FAB_ABI_VERSION)
    return fail(FAB_ERR_ABI_VERSION, "abi_version %d, library has %d", q.abi_version,
                FAB_ABI_VERSION);
  if (q.f != FAB_F_SOFTMAX && q.f != FAB_F_GELU_ERF)
    return fail(FAB_ERR_UNSUPPORTED, "unknown function %d", q.f);
  if (q.mask != FAB_MASK_NONE && q.mask != FAB_MASK_CAUSAL)
    return fail(FAB_ERR_UNSUPPORTED, "unknown mask %d", q.mask);
  if (q.dtype != FAB_BF16 && q.dtype != FAB_F32)
    return fail(FAB_ERR_UNSUPPORTED, "unknown dtype %d", q.dtype);
  if (q.variant < FAB_VARIANT_AUTO || q.variant > FAB_VARIANT_F32_MFMA)
    return fail(FAB_ERR_BAD_SHAPE, "unknown variant %d", q.variant);
  if (q.variant != FAB_VARIANT_AUTO && !(q.f == FAB_F_SOFTMAX && q.dtype == FAB_F32))
    return fail(FAB_ERR_UNSUPPORTED, "variant %d applies to fp32 softmax problems only", q.variant);
  if (q.batch < 1 || q.heads_a < 1 || q.heads_bc < 1 || q.m < 1 || q.n < 1 || q.k < 1 || q.p < 1)
    return fail(FAB_ERR_BAD_SHAPE, "sizes must be >= 1 (batch %lld heads %lld/%lld m %lld n %lld "
                "k %lld p %lld)", (long long)q.batch, (long long)q.heads_a,
                (long long)q.heads_bc, (long long)q.m, (long long)q.n, (long long)q.k,
                (long long)q.p);
  if (q.heads_a % q.heads_bc)
    return fail(FAB_ERR_BAD_SHAPE, "heads_a %lld is not a multiple of heads_bc %lld",
                (long long)q.heads_a, (long long)q.heads_bc);
  if (q.m > kMaxRows || q.n > kMaxRows || q.batch * q.heads_a > (1 << 20))
    return fail(FAB_ERR_UNSUPPORTED, "sizes beyond this build's limits (rows <= 2^30, "
                "batch*heads <= 2^20)");
  if (q.f == FAB_F_SOFTMAX) {
    // the largest grids (fp32 kernels: 4 rows per workgroup at d = 128;
    // per-row kernels: 16 rows per workgroup) stay below 2^31 workgroups
    const int64_t rows = std::max(q.m, q.n);
    if (rows > ((((int64_t)1 << 33) - 1) / (q.batch * q.heads_a)))
      return fail(FAB_ERR_UNSUPPORTED, "batch * heads_a * max(m, n) = %lld * %lld * %lld is beyond "
                  "this build's limit of 2^33 rows (kernel grids would exceed 2^31 workgroups)",
                  (long long)q.batch, (long long)q.heads_a, (long long)rows);
  }
  if (!std::isfinite(q.scale)) return fail(FAB_ERR_BAD_SHAPE, "scale must be finite");
  if (q.q_offset < -((int64_t)1 << 40) || q.q_offset > ((int64_t)1 << 40) ||
      q.k_offset < -((int64_t)1 << 40) || q.k_offset > ((int64_t)1 << 40))
    return fail(FAB_ERR_BAD_SHAPE, "mask offsets beyond +-2^40");

  const int64_t unit = q.dtype == FAB_BF16 ? 8 : 4;
  fab_plan_s tmp;
  tmp.prob = q;
  tmp.f32_mfma = false;
  tmp.mlp_splits = 0;
  resolve(q.a_stride, q.m, q.heads_a, q.k, tmp.as);
  resolve(q.bt_stride, q.n, q.heads_bc, q.k, tmp.bs);
  resolve(q.c_stride, q.n, q.heads_bc, q.p, tmp.cs);
  resolve(q.o_stride, q.m, q.heads_a, q.p, tmp.os);
  fab_status st;
  if ((st = check_strides("A", tmp.as, q.k, unit)) != FAB_OK) return st;
  if ((st = check_strides("Bt", tmp.bs, q.k, unit)) != FAB_OK) return st;
  if ((st = check_strides("C", tmp.cs, q.p, unit)) != FAB_OK) return st;
  if ((st = check_strides("O", tmp.os, q.p, unit)) != FAB_OK) return st;
  if (!distinct_layout(tmp.os, q.batch, q.heads_a, q.m, q.p))
    return fail(FAB_ERR_BAD_SHAPE, "O strides {%lld, %lld, %lld} map two output elements to one "
                "address (zero or overlapping batch / head / row strides)", (long long)tmp.os[0],
                (long long)tmp.os[1], (long long)tmp.os[2]);
  tmp.a_distinct = distinct_layout(tmp.as, q.batch, q.heads_a, q.m, q.k);
  tmp.bt_distinct = distinct_layout(tmp.bs, q.batch, q.heads_bc, q.n, q.k);
  tmp.c_distinct = distinct_layout(tmp.cs, q.batch, q.heads_bc, q.n, q.p);

  const char* dt = q.dtype == FAB_BF16 ? "bf16" : "f32";
  if (q.f == FAB_F_SOFTMAX) {
    if (q.k != q.p) return fail(FAB_ERR_UNSUPPORTED, "softmax needs k == p (got %lld, %lld)",
                                (long long)q.k, (long long)q.p);
    if (q.k != 64 && q.k != 128)
      return fail(FAB_ERR_UNSUPPORTED, "softmax head dim %lld not in {64, 128}", (long long)q.k);
    if (!(q.scale > 0.f)) return fail(FAB_ERR_UNSUPPORTED, "softmax scale must be > 0");
    // the kernels' per-lane copy offsets are 32-bit byte offsets within a
    // tile of up to 64 rows
    for (const int64_t* sr : {&tmp.as[2], &tmp.bs[2], &tmp.cs[2], &tmp.os[2]})
      if (*sr >= ((int64_t)1 << 24))
        return fail(FAB_ERR_UNSUPPORTED, "row stride %lld is beyond this build's limit of 2^24 "
                    "elements", (long long)*sr);
    tmp.fwd_ws = 0;
    // fp32: the matrix-core kernels (or when asked) once the problem has at
    // least 32 blocks of 64 queries at d = 128 (64 at d = 64, where the
    // plain-FMA kernels are cheaper per pair) and 2^22 unmasked (query, key)
    // pairs; below that their few workgroups leave most of the chip idle and
    // the plain-FMA kernels, with 4-16 rows per workgroup, finish first
    const double pairs = (double)q.batch * q.heads_a * q.m * q.n *
                         (q.mask == FAB_MASK_CAUSAL ? 0.5 : 1.0);
    const int64_t qblocks = q.batch * q.heads_a * ((q.m + 63) / 64);
    tmp.f32_mfma = q.dtype == FAB_F32 &&
                   (q.variant == FAB_VARIANT_F32_MFMA ||
                    (q.variant == FAB_VARIANT_AUTO && qblocks >= (q.k == 128 ? 32 : 64) &&
                     pairs >= (double)((int64_t)1 << 22)));
    // bf16 and fp32 matrix-core backward: -D and LSE * log2(e) per query row;
    // the plain-FMA fp32 backward forms D inside its kernel (no workspace)
    const size_t rows = (size_t)q.batch * q.heads_a * q.m;
    tmp.bwd_ws = (q.dtype == FAB_BF16 || tmp.f32_mfma) ? round_up(rows * sizeof(float) * 2, 256) : 0;
    if (q.dtype == FAB_BF16)
      snprintf(tmp.desc, sizeof tmp.desc,
               "attention %s d=%lld %s group=%lld fwd[BM=%d BN=%d grid=%lld] "
               "bwd[dq BM=%d, dkdv KB=%d QB=%d]", dt, (long long)q.k,
               q.mask == FAB_MASK_CAUSAL ? "causal" : "full", (long long)(q.heads_a / q.heads_bc),
               fab::kAttnFwdBM, fab::kAttnFwdBN,
               (long long)((q.m + fab::kAttnFwdBM - 1) / fab::kAttnFwdBM * q.heads_a * q.batch),
               fab::kAttnBwdBM, fab::kAttnBwdKB, fab::kAttnBwdQB);
    else
      snprintf(tmp.desc, sizeof tmp.desc, "attention %s d=%lld %s group=%lld (%s)", dt,
               (long long)q.k, q.mask == FAB_MASK_CAUSAL ? "causal" : "full",
               (long long)(q.heads_a / q.heads_bc), tmp.f32_mfma ? "fp32 MFMA" : "fp32 FMA");
  } else {
    if (q.mask != FAB_MASK_NONE) return fail(FAB_ERR_UNSUPPORTED, "GeLU takes no mask");
    if (q.q_offset || q.k_offset) return fail(FAB_ERR_UNSUPPORTED, "GeLU takes no mask offsets");
    if (q.dtype != FAB_BF16) return fail(FAB_ERR_UNSUPPORTED, "GeLU MLP runs in bf16 only");
    if (q.batch != 1 || q.heads_a != 1 || q.heads_bc != 1)
      return fail(FAB_ERR_UNSUPPORTED, "GeLU MLP needs batch == heads == 1");
    if (q.k > 1024 || q.p > 1024 || !fab::mlp_shape_supported((int)q.k, (int)q.p))
      return fail(FAB_ERR_UNSUPPORTED, "GeLU MLP: k = %lld, p = %lld is not a width pair this "
                  "build runs (each of k and p a multiple of 64 from 64 to 1024)", (long long)q.k,
                  (long long)q.p);
    int splits = 1;
    tmp.fwd_ws = round_up(fab::mlp_fwd_workspace((int)q.m, (int)q.n, (int)q.k, (int)q.p, &splits), 256);
    tmp.bwd_ws = round_up(fab::mlp_bwd_workspace((int)q.m, (int)q.n, (int)q.k, (int)q.p), 256);
    tmp.mlp_splits = splits;
    snprintf(tmp.desc, sizeof tmp.desc, "gelu-mlp bf16 m=%lld k=%lld n=%lld p=%lld splits=%d",
             (long long)q.m, (long long)q.k, (long long)q.n, (long long)q.p, splits);
  }
  fab_plan_s* plan = new (std::nothrow) fab_plan_s;
  if (!plan) return fail(FAB_ERR_UNSUPPORTED, "out of host memory");
  plan->prob = tmp.prob;
  memcpy(plan->as, tmp.as, sizeof tmp.as);
  memcpy(plan->bs, tmp.bs, sizeof tmp.bs);
  memcpy(plan->cs, tmp.cs, sizeof tmp.cs);
  memcpy(plan->os, tmp.os, sizeof tmp.os);
  plan->fwd_ws = tmp.fwd_ws;
  plan->bwd_ws = tmp.bwd_ws;
  plan->mlp_splits = tmp.mlp_splits;
  plan->f32_mfma = tmp.f32_mfma;
  plan->a_distinct = tmp.a_distinct;
  plan->bt_distinct = tmp.bt_distinct;
  plan->c_distinct = tmp.c_distinct;
  memcpy(plan->desc, tmp.desc, sizeof tmp.desc);
  *plan_out = plan;
  if (fwd_ws) *fwd_ws = plan->fwd_ws;
  if (bwd_ws) *bwd_ws = plan->bwd_ws;
  return ok();
}

void fab_plan_destroy(fab_plan_t* plan) { delete plan; }

fab_status fab_plan_set_timing(fab_plan_t* plan, int enable) {
  if (!plan) return fail(FAB_ERR_NULL_ARG, "fab_plan_set_timing: plan is NULL");
  std::lock_guard<std::mutex> lock(plan->timer_mu);
  if (enable && !plan->timer) {
    plan->timer = new (std::nothrow) KernelTimer;
    if (!plan->timer) return fail(FAB_ERR_UNSUPPORTED, "out of host memory");
  } else if (!enable && plan->timer) {
    delete plan->timer;
    plan->timer = nullptr;
  }
  return ok();
}

int fab_plan_kernel_times(fab_plan_t* plan, const char** names, int* counts, double* total_ms,
                          int capacity) {
  if (!plan) return -1;
  std::lock_guard<std::mutex> lock(plan->timer_mu);
  if (!plan->timer) return 0;
  plan->timer->drain();
  if (plan->timer->failed) {
    fail(FAB_ERR_HIP, "fab_plan_kernel_times: a HIP event call failed");
    return -1;
  }
  int i = 0;
  for (auto& kv : plan->timer->totals) {
    if (i < capacity) {
      // names point at the static strings the launchers pass
      if (names) names[i] = kv.first.c_str();
      if (counts) counts[i] = kv.second.first;
      if (total_ms) total_ms[i] = kv.second.second;
    }
    ++i;
  }
  return i;
}

fab_status fab_plan_reset_kernel_times(fab_plan_t* plan) {
  if (!plan) return fail(FAB_ERR_NULL_ARG, "fab_plan_reset_kernel_times: plan is NULL");
  std::lock_guard<std::mutex> lock(plan->timer_mu);
  if (plan->timer) {
    plan->timer->drain();
    plan->timer->totals.clear();
  }
  return ok();
}

size_t fab_plan_describe(const fab_plan_t* plan, char* buf, size_t len) {
  if (!plan) return 0;
  const size_t need = strlen(plan->desc);
  if (buf && len) {
    const size_t nc = need < len - 1 ? need : len - 1;
    memcpy(buf, plan->desc, nc);
    buf[nc] = 0;
  }
  return need;
}

fab_status fab_forward(const fab_plan_t* plan, const void* A, const void* Bt, const void* C,
                       void* O, float* lse, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (!plan || !A || !Bt || !C || !O) return fail(FAB_ERR_NULL_ARG, "fab_forward: null argument");
  const fab_problem& q = plan->prob;
  if (!aligned16(A) || !aligned16(Bt) || !aligned16(C) || !aligned16(O))
    return fail(FAB_ERR_ALIGNMENT, "fab_forward: tensor base pointers must be 16-byte aligned");
  if (workspace_bytes < plan->fwd_ws)
    return fail(FAB_ERR_WORKSPACE_TOO_SMALL, "fab_forward: workspace %zu < %zu bytes",
                workspace_bytes, plan->fwd_ws);
  if (plan->fwd_ws && !workspace) return fail(FAB_ERR_NULL_ARG, "fab_forward: workspace is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  TimerScope scope(plan->timer);
  if (q.f == FAB_F_SOFTMAX) {
    if (!lse) return fail(FAB_ERR_NULL_ARG, "fab_forward: softmax needs lse");
    if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
      return fail(FAB_ERR_ALIGNMENT, "fab_forward: lse must be 4-byte aligned");
    fab::AttnArgs a = attn_args(plan);
    a.q = A, a.k = Bt, a.v = C, a.o_out = O, a.lse = lse;
    e = q.dtype == FAB_BF16 ? fab::launch_attn_fwd_bf16(a, (int)q.k, s)
        : plan->f32_mfma    ? fab::launch_attn_fwd_f32_mfma(a, (int)q.k, s)
                            : fab::launch_attn_fwd_f32(a, (int)q.k, s);
  } else {
    if (lse) return fail(FAB_ERR_UNSUPPORTED, "fab_forward: GeLU takes no lse");
    if (plan->fwd_ws && !aligned16(workspace))
      return fail(FAB_ERR_ALIGNMENT, "fab_forward: workspace must be 16-byte aligned");
    fab::MlpArgs a{};
    a.a = A, a.bt = Bt, a.c = C, a.o = O, a.ws = static_cast<float*>(workspace);
    a.a_sr = plan->as[2], a.bt_sr = plan->bs[2], a.c_sr = plan->cs[2], a.o_sr = plan->os[2];
    a.m = (int)q.m, a.n = (int)q.n, a.k = (int)q.k, a.p = (int)q.p;
    a.splits = plan->mlp_splits;
    a.scale = q.scale;
    e = fab::launch_mlp_fwd_bf16(a, s);
  }
  if (e != hipSuccess) return fail(FAB_ERR_HIP, "fab_forward: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

namespace {

// Checks of fab_backward's tensor arguments (everything but the workspace).
fab_status check_backward_args(const char* who, const fab_plan_t* plan, const void* A,
                               const void* Bt, const void* C, const void* O, const float* lse,
                               const void* dO, const void* dA, const void* dBt, const void* dC) {
  if (!plan || !A || !Bt || !C || !dO || !dA || !dBt || !dC)
    return fail(FAB_ERR_NULL_ARG, "%s: null argument", who);
  const fab_problem& q = plan->prob;
  if (!aligned16(A) || !aligned16(Bt) || !aligned16(C) || !aligned16(dO) || !aligned16(dA) ||
      !aligned16(dBt) || !aligned16(dC))
    return fail(FAB_ERR_ALIGNMENT, "%s: tensor base pointers must be 16-byte aligned", who);
  if (!plan->a_distinct || !plan->bt_distinct || !plan->c_distinct)
    return fail(FAB_ERR_BAD_SHAPE, "%s: the strides of %s map two elements to one address, so "
                "its gradient cannot be written in that layout (pass a packed copy)", who,
                !plan->a_distinct ? "A" : !plan->bt_distinct ? "Bt" : "C");
  if (q.f == FAB_F_SOFTMAX) {
    if (!O || !lse) return fail(FAB_ERR_NULL_ARG, "%s: softmax needs O and lse", who);
    if (!aligned16(O)) return fail(FAB_ERR_ALIGNMENT, "%s: O must be 16-byte aligned", who);
    if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
      return fail(FAB_ERR_ALIGNMENT, "%s: lse must be 4-byte aligned", who);
  } else if (O || lse) {
    return fail(FAB_ERR_UNSUPPORTED, "%s: GeLU takes no O / lse", who);
  }
  return FAB_OK;
}

// Enqueues the backward kernels; arguments already checked.
fab_status backward_launch(const char* who, const fab_plan_t* plan, const void* A, const void* Bt,
                           const void* C, const void* O, const float* lse, const void* dO,
                           void* dA, void* dBt, void* dC, void* workspace, void* stream) {
  const fab_problem& q = plan->prob;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  TimerScope scope(plan->timer);
  if (q.f == FAB_F_SOFTMAX) {
    fab::AttnArgs a = attn_args(plan);
    a.q = A, a.k = Bt, a.v = C, a.o = O, a.lse_in = lse, a.dout = dO;
    a.dq = dA, a.dk = dBt, a.dv = dC;
    if (q.dtype == FAB_BF16 || plan->f32_mfma) {  // the fp32 FMA path uses no workspace
      a.delta = static_cast<float*>(workspace);
      a.lse2 = a.delta + (size_t)q.batch * q.heads_a * q.m;
    }
    e = q.dtype == FAB_BF16 ? fab::launch_attn_bwd_bf16(a, (int)q.k, s)
        : plan->f32_mfma    ? fab::launch_attn_bwd_f32_mfma(a, (int)q.k, s)
                            : fab::launch_attn_bwd_f32(a, (int)q.k, s);
  } else {
    fab::MlpArgs a{};
    a.a = A, a.bt = Bt, a.c = C, a.dout = dO, a.da = dA, a.dbt = dBt, a.dc = dC;
    a.ws = static_cast<float*>(workspace);
    a.a_sr = plan->as[2], a.bt_sr = plan->bs[2], a.c_sr = plan->cs[2], a.o_sr = plan->os[2];
    a.m = (int)q.m, a.n = (int)q.n, a.k = (int)q.k, a.p = (int)q.p;
    a.splits = plan->mlp_splits;
    a.scale = q.scale;
    e = fab::launch_mlp_bwd_bf16(a, s);
  }
  if (e != hipSuccess) return fail(FAB_ERR_HIP, "%s: %s", who, hipGetErrorString(e));
  return ok();
}

// Device scratch of fab_backward_noalloc: one copy per GPU, held until the
// process ends.  Host code never uses this name as an address (on the host it
// is a stand-in, not device memory); it uses the per-device address that
// hipGetSymbolAddress returns.
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // device address of `scratch`, by device ordinal

// The current device's copy of `scratch`, looked up once per device.
fab_status static_scratch(const char* who, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0)
    return fail(FAB_ERR_HIP, "%s: hipGetDevice: %s", who, hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(FAB_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", who, dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FAB_OK;
}

}  // namespace

extern "C" {

fab_status fab_backward(const fab_plan_t* plan, const void* A, const void* Bt, const void* C,
                        const void* O, const float* lse, const void* dO, void* dA, void* dBt,
                        void* dC, void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "fab_backward";
  fab_status st = check_backward_args(who, plan, A, Bt, C, O, lse, dO, dA, dBt, dC);
  if (st != FAB_OK) return st;
  if (workspace_bytes < plan->bwd_ws)
    return fail(FAB_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu < %zu bytes", who,
                workspace_bytes, plan->bwd_ws);
  if (plan->bwd_ws && !workspace) return fail(FAB_ERR_NULL_ARG, "%s: workspace is NULL", who);
  if (plan->bwd_ws && !aligned16(workspace))
    return fail(FAB_ERR_ALIGNMENT, "%s: workspace must be 16-byte aligned", who);
  return backward_launch(who, plan, A, Bt, C, O, lse, dO, dA, dBt, dC, workspace, stream);
}

fab_status fab_backward_noalloc(const fab_plan_t* plan, const void* A, const void* Bt,
                                const void* C, const void* O, const float* lse, const void* dO,
                                void* dA, void* dBt, void* dC, void* stream) {
  const char* who = "fab_backward_noalloc";
  fab_status st = check_backward_args(who, plan, A, Bt, C, O, lse, dO, dA, dBt, dC);
  if (st != FAB_OK) return st;
  if (plan->bwd_ws > kStaticScratchBytes)
    return fail(FAB_ERR_WORKSPACE_TOO_SMALL, "%s: this problem needs %zu bytes of scratch; the "
                "library's static scratch holds %zu (use fab_backward with a workspace)", who,
                plan->bwd_ws, kStaticScratchBytes);
  void* ws = nullptr;
  if (plan->bwd_ws && (st = static_scratch(who, &ws)) != FAB_OK) return st;
  return backward_launch(who, plan, A, Bt, C, O, lse, dO, dA, dBt, dC, ws, stream);
}

fab_status fab_merge(const fab_plan_t* plan, const void* O_a, const float* lse_a,
                     const void* O_b, const float* lse_b, void* O_out, float* lse_out,
                     void* stream) {
  if (!plan || !O_a || !lse_a || !O_b || !lse_b || !O_out || !lse_out)
    return fail(FAB_ERR_NULL_ARG, "fab_merge: null argument");
  const fab_problem& q = plan->prob;
  if (q.f != FAB_F_SOFTMAX) return fail(FAB_ERR_UNSUPPORTED, "fab_merge: needs a softmax plan");
  if (!aligned16(O_a) || !aligned16(O_b) || !aligned16(O_out))
    return fail(FAB_ERR_ALIGNMENT, "fab_merge: O pointers must be 16-byte aligned");
  const uintptr_t lmask = reinterpret_cast<uintptr_t>(lse_a) | reinterpret_cast<uintptr_t>(lse_b) |
                          reinterpret_cast<uintptr_t>(lse_out);
  if (lmask & 3u) return fail(FAB_ERR_ALIGNMENT, "fab_merge: lse pointers must be 4-byte aligned");
  fab::MergeArgs a{};
  a.oa = O_a, a.ob = O_b, a.oo = O_out, a.la = lse_a, a.lb = lse_b, a.lo = lse_out;
  a.o_sb = plan->os[0], a.o_sh = plan->os[1], a.o_sr = plan->os[2];
  a.b = (int32_t)q.batch, a.hq = (int32_t)q.heads_a, a.m = (int32_t)q.m;
  a.small = q.batch * q.heads_a * q.m < ((int64_t)1 << 31);
  a.div_hq = fab::make_fastdiv((uint32_t)q.heads_a);
  a.div_m = fab::make_fastdiv((uint32_t)q.m);
  hipStream_t s = static_cast<hipStream_t>(stream);
  TimerScope scope(plan->timer);
  const hipError_t e = fab::launch_attn_merge(a, (int)q.p, q.dtype == FAB_BF16, s);
  if (e != hipSuccess) return fail(FAB_ERR_HIP, "fab_merge: %s", hipGetErrorString(e));
  return ok();
}

fab_status fab_ulysses_sizes(const fab_ulysses_layout* l, int64_t* heads_per_rank,
                             int64_t* buffer_elems) {
  fab::UlyssesArgs a{};
  int64_t hl = 0, elems = 0;
  const fab_status st = ulysses_setup(l, "fab_ulysses_sizes", true, &a, &hl, &elems);
  if (st != FAB_OK) return st;
  if (heads_per_rank) *heads_per_rank = hl;
  if (buffer_elems) *buffer_elems = elems;
  return ok();
}

fab_status fab_ulysses_pack(const fab_ulysses_layout* l, const void* x, void* send, void* stream) {
  if (!x || !send) return fail(FAB_ERR_NULL_ARG, "fab_ulysses_pack: null argument");
  if (!aligned16(x) || !aligned16(send))
    return fail(FAB_ERR_ALIGNMENT, "fab_ulysses_pack: pointers must be 16-byte aligned");
  fab::UlyssesArgs a{};
  int64_t hl = 0, elems = 0;
  const fab_status st = ulysses_setup(l, "fab_ulysses_pack", true, &a, &hl, &elems);
  if (st != FAB_OK) return st;
  a.src = x;
  a.dst = send;
  const hipError_t e = fab::launch_ulysses(a, true, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FAB_ERR_HIP, "fab_ulysses_pack: %s", hipGetErrorString(e));
  return ok();
}

fab_status fab_ulysses_unpack(const fab_ulysses_layout* l, const void* recv, void* x,
                              void* stream) {
  if (!recv || !x) return fail(FAB_ERR_NULL_ARG, "fab_ulysses_unpack: null argument");
  if (!aligned16(recv) || !aligned16(x))
    return fail(FAB_ERR_ALIGNMENT, "fab_ulysses_unpack: pointers must be 16-byte aligned");
  fab::UlyssesArgs a{};
  int64_t hl = 0, elems = 0;
  const fab_status st = ulysses_setup(l, "fab_ulysses_unpack", false, &a, &hl, &elems);
  if (st != FAB_OK) return st;
  a.src = recv;
  a.dst = x;
  const hipError_t e = fab::launch_ulysses(a, false, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FAB_ERR_HIP, "fab_ulysses_unpack: %s", hipGetErrorString(e));
  return ok();
}

fab_status fab_exp_probe(int blocks, int iters, float* sink, int64_t* exp_count, void* stream) {
  if (blocks < 1 || iters < 1 || blocks > (1 << 20) || iters > (1 << 24))
    return fail(FAB_ERR_BAD_SHAPE, "fab_exp_probe: blocks in [1, 2^20], iters in [1, 2^24]");
  if (exp_count) *exp_count = (int64_t)blocks * 256 * iters * fab::exp_probe_chains();
  if (!sink) return ok();  // count only
  if (reinterpret_cast<uintptr_t>(sink) & 3u)
    return fail(FAB_ERR_ALIGNMENT, "fab_exp_probe: sink must be 4-byte aligned");
  const hipError_t e = fab::launch_exp_probe(blocks, iters, sink, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FAB_ERR_HIP, "fab_exp_probe: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
