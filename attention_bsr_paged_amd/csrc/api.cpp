// C ABI of libabp: validation, plan upload and kernel launches.
//
// Every entry point returns an abp_status and records a message in a
// thread-local string; no C++ exception crosses the boundary. Nothing here
// allocates device or pinned memory: the caller owns all buffers.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "../../include/abp.h"
#include "kernels.h"
#include "plan.h"

namespace {

thread_local std::string g_err;

int fail(int status, const std::string& msg) {
  g_err = msg;
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  g_err = std::string(what) + ": " + hipGetErrorString(e);
  return ABP_ERR_HIP;
}

std::mutex g_cu_mutex;
int32_t g_cu_count[64] = {0};

int num_cus(int device, int32_t* out) {
  if (device < 0 || device >= 64) return fail(ABP_ERR_INVALID_ARG, "device out of range");
  std::lock_guard<std::mutex> lock(g_cu_mutex);
  if (g_cu_count[device] == 0) {
    int v = 0;
    hipError_t e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    g_cu_count[device] = v;
  }
  *out = g_cu_count[device];
  return ABP_OK;
}

// One worker per resident workgroup slot of the current device: compute units
// times the workgroups of the chosen kernel that fit on one compute unit.
int default_workers(const abp::Config& cfg, int32_t* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  int32_t cus = 0;
  int st = num_cus(dev, &cus);
  if (st != ABP_OK) return st;
  int per_cu = cfg.kind == ABP_KIND_DECODE ? abp::decode_blocks_per_cu(cfg)
                                           : abp::append_blocks_per_cu(cfg);
  *out = cus * (per_cu > 0 ? per_cu : 1);
  return ABP_OK;
}

// Layout of a plan from its capacity fields (what *_run can reconstruct).
int layout_of_plan(const abp::Config& cfg, const abp_plan* plan, abp::Layout* L, std::string* err) {
  int st = abp::make_layout_caps(cfg, plan->max_tiles, plan->num_workers, L, err);
  if (st != ABP_OK) return st;
  if (L->max_segs != plan->max_segments || L->max_partials != plan->max_partials) {
    *err = "plan capacities are inconsistent";
    return ABP_ERR_PLAN_MISMATCH;
  }
  return ABP_OK;
}

int resolve_layout(int kind, const abp_params* params, int32_t max_batch, int32_t max_qo,
                   int32_t workers, abp::Config* cfg, abp::Layout* L) {
  std::string err;
  int st = abp::check_params(kind, params, cfg, &err);
  if (st != ABP_OK) return fail(st, err);
  if (kind == ABP_KIND_DECODE && cfg->group > 8)
    return fail(ABP_ERR_UNSUPPORTED, "decode supports group sizes 1, 2, 4 and 8");
  if (workers == ABP_WORKERS_PER_TILE) {
    // one worker per tile: as many workers as the capacities allow tiles
    st = abp::make_layout(*cfg, max_batch, max_qo, 1, L, &err);
    if (st != ABP_OK) return fail(st, err);
    st = abp::make_layout(*cfg, max_batch, max_qo, std::max<int32_t>(1, L->max_tiles), L, &err);
    if (st != ABP_OK) return fail(st, err);
    L->no_split = true;
    return ABP_OK;
  }
  if (workers <= 0) {
    st = default_workers(*cfg, &workers);
    if (st != ABP_OK) return st;
  }
  st = abp::make_layout(*cfg, max_batch, max_qo, workers, L, &err);
  if (st != ABP_OK) return fail(st, err);
  return ABP_OK;
}

int do_plan(int kind, const abp_params* params, int32_t batch, const int32_t* qo_indptr_h,
            const int32_t* kv_indptr_h, const int32_t* lpl_h, int32_t max_batch, int32_t max_qo,
            int32_t workers, void* host_ws, size_t host_bytes, abp_plan* plan,
            abp::Config* cfg_out, abp::Layout* lay_out) {
  if (!plan) return fail(ABP_ERR_INVALID_ARG, "plan is NULL");
  if (!host_ws) return fail(ABP_ERR_INVALID_ARG, "host workspace is NULL");
  if (batch > max_batch) return fail(ABP_ERR_WORKSPACE_TOO_SMALL, "batch > max_batch");
  abp::Config cfg;
  abp::Layout L;
  int st = resolve_layout(kind, params, max_batch, max_qo, workers, &cfg, &L);
  if (st != ABP_OK) return st;
  if (host_bytes < L.plan_bytes)
    return fail(ABP_ERR_WORKSPACE_TOO_SMALL, "host workspace smaller than abp_workspace_size");
  if (kind == ABP_KIND_APPEND && qo_indptr_h && batch >= 0 && qo_indptr_h[batch] > max_qo)
    return fail(ABP_ERR_WORKSPACE_TOO_SMALL, "total query tokens > max_qo_tokens");
  std::string err;
  st = abp::plan_compute(cfg, L, batch, qo_indptr_h, kv_indptr_h, lpl_h,
                         static_cast<int32_t*>(host_ws), plan, &err);
  if (st != ABP_OK) return fail(st, err);
  if (cfg_out) *cfg_out = cfg;
  if (lay_out) *lay_out = L;
  return ABP_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Grid of the merge launch after decode: one wave per (tile, row) at the
// plan's capacity (4 waves per workgroup), at least one workgroup per worker.
// It depends only on capacities, so a captured run stays valid after a
// re-plan. Measured on the batch decode run: 98.4 us against 99.8 us with one
// workgroup per worker (two rows per wave).
int32_t decode_merge_grid(const abp_plan& plan) {
  const int64_t waves = int64_t(plan.max_tiles) * plan.rows_per_tile;
  return int32_t(std::min<int64_t>(std::max<int64_t>(plan.num_workers, (waves + 3) / 4), 4096));
}

int prepare_run(int kind, const abp_plan* plan, const abp_params* params, void* dev_ws,
                size_t dev_bytes, abp::Config* cfg, abp::Layout* L) {
  if (!plan || !params) return fail(ABP_ERR_INVALID_ARG, "plan or params is NULL");
  if (plan->kind != kind) return fail(ABP_ERR_PLAN_MISMATCH, "plan was made for the other kind");
  std::string err;
  int st = abp::check_params(kind, params, cfg, &err);
  if (st != ABP_OK) return fail(st, err);
  if (kind == ABP_KIND_DECODE && cfg->group > 8)
    return fail(ABP_ERR_UNSUPPORTED, "decode supports group sizes 1, 2, 4 and 8");
  if (plan->num_workers < 1) return fail(ABP_ERR_PLAN_MISMATCH, "plan has no workers");
  st = layout_of_plan(*cfg, plan, L, &err);
  if (st != ABP_OK) return fail(st, err);
  if (abp::fingerprint(*cfg, *L) != plan->fingerprint)
    return fail(ABP_ERR_PLAN_MISMATCH, "params or capacities differ from the planned ones");
  if (!dev_ws) return fail(ABP_ERR_INVALID_ARG, "device workspace is NULL");
  if (dev_bytes < L->dev_bytes)
    return fail(ABP_ERR_WORKSPACE_TOO_SMALL, "device workspace smaller than abp_workspace_size");
  if (!aligned16(dev_ws)) return fail(ABP_ERR_INVALID_ARG, "device workspace must be 16-byte aligned");
  return ABP_OK;
}

void fill_args(const abp::Config& cfg, const abp::Layout& L, const abp_plan* plan, void* dev_ws,
               abp::AttnArgs* a) {
  a->num_qo_heads = cfg.hq;
  a->num_kv_heads = cfg.hkv;
  a->page_size = cfg.page_size;
  int shift = -1;
  if ((cfg.page_size & (cfg.page_size - 1)) == 0) {
    shift = 0;
    while ((1 << shift) < cfg.page_size) ++shift;
  }
  a->page_shift = shift;
  a->token_stride = cfg.hkv * cfg.head_dim;
  a->page_stride = int64_t(cfg.page_size) * a->token_stride;
  a->out_dtype = cfg.out_dtype;
  // fp8 keys are k_scale times their codes: the logit scale absorbs k_scale
  const float qk_scale = cfg.kv_fp8 ? cfg.sm_scale * cfg.k_scale : cfg.sm_scale;
  a->sm_scale = qk_scale;
  a->sm_scale_log2 = qk_scale * 1.4426950408889634f;
  a->v_scale = cfg.kv_fp8 ? cfg.v_scale : 1.f;
  a->workers = plan->num_workers;
  char* ws = static_cast<char*>(dev_ws);
  a->plan = reinterpret_cast<const int32_t*>(ws);
  a->o_part = reinterpret_cast<float*>(ws + L.partial_offset);
  a->lse_part = a->o_part + int64_t(L.max_partials) * L.rows * cfg.head_dim;
}

}  // namespace

namespace abp {

int default_decode_workers(const abp_params* params, int32_t* out) {
  Config cfg;
  std::string err;
  int st = check_params(ABP_KIND_DECODE, params, &cfg, &err);
  if (st != ABP_OK) return fail(st, err);
  return default_workers(cfg, out);
}

int set_error(int status, const char* msg) { return fail(status, msg); }

}  // namespace abp

// Mixed decode + append batches: worker split and the two sub-plans.
namespace {

// Decode bandwidth of the matrix-core decode kernel against the compute units
// it runs on (one 4-wave worker each), measured on MI355X with the batch decode
// workload (64 requests, GQA 32/8, page 16, bf16): 2.65, 4.23, 5.14 and 5.20
// TB/s on 64, 128, 192 and 256 compute units.
double pod_decode_bw(double cus) {
  static const double x[] = {0.0, 64.0, 128.0, 192.0, 256.0};
  static const double y[] = {0.0, 2.65e12, 4.23e12, 5.14e12, 5.20e12};
  if (cus >= x[4]) return y[4];
  int i = 0;
  while (cus > x[i + 1]) ++i;
  return y[i] + (y[i + 1] - y[i]) * (cus - x[i]) / (x[i + 1] - x[i]);
}
// append kernel throughput per compute unit (ragged causal append, bf16)
constexpr double kPodAppendFlopPerCu = 3.0e12;
// Decode beside a running append is slower than on the same compute units
// alone: the append's K/V traffic competes for the memory system. Measured on
// the mixed benchmark batch (64 decode requests, 4 x 512-token prefill
// chunks), the launch took 1.08 to 1.24 times the slower part's time alone.
constexpr double kPodDecodeSlowdown = 1.2;

int64_t pod_kv_len(const int32_t* indptr, const int32_t* lpl, int32_t b, int32_t page) {
  const int64_t n = int64_t(indptr[b + 1]) - indptr[b];
  return n > 0 ? (n - 1) * page + lpl[b] : 0;
}

// Decode workgroups of a launch of `groups` workgroups.
int32_t pod_split(const abp::Config& cfg, int32_t groups, int32_t decode_batch,
                  const int32_t* d_indptr, const int32_t* d_lpl, int32_t append_batch,
                  const int32_t* qo, const int32_t* a_indptr, const int32_t* a_lpl,
                  int32_t decode_groups) {
  const bool has_d = decode_batch > 0, has_a = append_batch > 0;
  if (!has_d) return 0;
  if (!has_a) return groups;
  if (decode_groups > 0) return std::min(std::max(decode_groups, 1), groups - 1);
  double bytes = 0.0;  // decode K/V bytes
  for (int32_t b = 0; b < decode_batch; ++b)
    bytes += double(pod_kv_len(d_indptr, d_lpl, b, cfg.page_size)) * cfg.hkv * cfg.head_dim * 4.0;
  double pairs = 0.0;  // visible (query, key) pairs of the append part
  for (int32_t b = 0; b < append_batch; ++b) {
    const double q = std::max(0, qo[b + 1] - qo[b]);
    const double k = double(pod_kv_len(a_indptr, a_lpl, b, cfg.page_size));
    pairs += cfg.causal ? q * std::max(0.0, k - q) + q * (q + 1) / 2 : q * k;
  }
  const double flop = 4.0 * cfg.head_dim * cfg.hq * pairs;
  // whole XCD rows (8 workgroups) when the launch is large enough
  const int32_t step = groups >= 16 ? 8 : 1;
  int32_t best = step, lo = step, hi = groups - step;
  double best_t = 1e300;
  for (int32_t g = lo; g <= hi; g += step) {
    const double t = std::max(kPodDecodeSlowdown * bytes / pod_decode_bw(g),
                              flop / (kPodAppendFlopPerCu * (groups - g)));
    if (t < best_t) {
      best_t = t;
      best = g;
    }
  }
  return best;
}

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

struct PodLayout {
  abp_params pd, pa;  // decode part (causal off) and append part
  abp::Config cd, ca;
  abp::Layout ld, la;
  size_t d_host = 0, a_host = 0, d_dev = 0, a_dev = 0;  // region sizes
  int32_t groups = 0;
};

int pod_layout(const abp_params* params, int32_t max_d, int32_t max_a, int32_t max_qo,
               int32_t groups, PodLayout* P) {
  if (!params) return fail(ABP_ERR_INVALID_ARG, "params is NULL");
  if (max_d < 0 || max_a < 0) return fail(ABP_ERR_INVALID_ARG, "negative maximum batch");
  if (groups <= 0) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    int st = num_cus(dev, &groups);
    if (st != ABP_OK) return st;
  }
  if (groups < 2) return fail(ABP_ERR_INVALID_ARG, "a mixed launch needs at least 2 workgroups");
  P->groups = groups;
  P->pd = *params;
  P->pd.causal = 0;
  P->pa = *params;
  std::string err;
  int st = abp::check_params(ABP_KIND_APPEND, &P->pa, &P->ca, &err);
  if (st != ABP_OK) return fail(st, err);
  st = abp::check_params(ABP_KIND_DECODE, &P->pd, &P->cd, &err);
  if (st != ABP_OK) return fail(st, err);
  if (!abp::pod_applies(P->cd))
    return fail(ABP_ERR_UNSUPPORTED,
                "mixed batches need 16-bit K/V, no RoPE, power-of-two pages >= 16, kv heads a "
                "multiple of 4 and group 4 or 8");
  if (max_d > 0) {
    st = resolve_layout(ABP_KIND_DECODE, &P->pd, max_d, 0, groups, &P->cd, &P->ld);
    if (st != ABP_OK) return st;
    P->d_host = round256(P->ld.plan_bytes);
    P->d_dev = round256(P->ld.dev_bytes);
  }
  if (max_a > 0) {
    st = resolve_layout(ABP_KIND_APPEND, &P->pa, max_a, max_qo, groups, &P->ca, &P->la);
    if (st != ABP_OK) return st;
    P->a_host = round256(P->la.plan_bytes);
    P->a_dev = round256(P->la.dev_bytes);
  }
  return ABP_OK;
}

int pod_plan_host(const abp_params* params, int32_t decode_batch, const int32_t* d_indptr,
                  const int32_t* d_lpl, int32_t append_batch, const int32_t* qo,
                  const int32_t* a_indptr, const int32_t* a_lpl, int32_t max_d, int32_t max_a,
                  int32_t max_qo, int32_t groups, int32_t decode_groups, void* host_ws,
                  size_t host_bytes, abp_pod_plan_t* plan, PodLayout* P) {
  if (!plan) return fail(ABP_ERR_INVALID_ARG, "plan is NULL");
  if (!host_ws) return fail(ABP_ERR_INVALID_ARG, "host workspace is NULL");
  if (decode_batch < 0 || append_batch < 0) return fail(ABP_ERR_INVALID_ARG, "negative batch");
  if (decode_batch > max_d) return fail(ABP_ERR_WORKSPACE_TOO_SMALL, "decode_batch > max_decode_batch");
  if (append_batch > max_a) return fail(ABP_ERR_WORKSPACE_TOO_SMALL, "append_batch > max_append_batch");
  if ((decode_batch > 0 && (!d_indptr || !d_lpl)) ||
      (append_batch > 0 && (!qo || !a_indptr || !a_lpl)))
    return fail(ABP_ERR_INVALID_ARG, "NULL index array");
  int st = pod_layout(params, max_d, max_a, max_qo, groups, P);
  if (st != ABP_OK) return st;
  if (host_bytes < P->d_host + P->a_host)
    return fail(ABP_ERR_WORKSPACE_TOO_SMALL, "host workspace smaller than abp_pod_workspace_size");
  memset(plan, 0, sizeof(*plan));
  plan->num_groups = P->groups;
  plan->decode_host_offset = 0;
  plan->append_host_offset = P->d_host;
  plan->decode_dev_offset = 0;
  plan->append_dev_offset = P->d_dev;
  plan->decode_dev_bytes = P->d_dev;
  plan->append_dev_bytes = P->a_dev;
  const int32_t wd = pod_split(P->ca, P->groups, decode_batch, d_indptr, d_lpl, append_batch, qo,
                               a_indptr, a_lpl, decode_groups);
  const int32_t wa = append_batch > 0 ? P->groups - wd : 0;
  char* hw = static_cast<char*>(host_ws);
  if (wd > 0) {
    st = do_plan(ABP_KIND_DECODE, &P->pd, decode_batch, nullptr, d_indptr, d_lpl, max_d, 0, wd,
                 hw + plan->decode_host_offset, P->d_host, &plan->decode, &P->cd, &P->ld);
    if (st != ABP_OK) return st;
  }
  if (wa > 0) {
    st = do_plan(ABP_KIND_APPEND, &P->pa, append_batch, qo, a_indptr, a_lpl, max_a, max_qo, wa,
                 hw + plan->append_host_offset, P->a_host, &plan->append, &P->ca, &P->la);
    if (st != ABP_OK) return st;
  }
  return ABP_OK;
}

}  // namespace

extern "C" {

const char* abp_status_string(int status) {
  switch (status) {
    case ABP_OK: return "ok";
    case ABP_ERR_INVALID_ARG: return "invalid argument";
    case ABP_ERR_UNSUPPORTED: return "unsupported configuration";
    case ABP_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case ABP_ERR_PLAN_MISMATCH: return "plan does not match the run arguments";
    case ABP_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* abp_last_error(void) { return g_err.c_str(); }

int abp_device_num_cus(int device, int32_t* out) {
  try {
    if (!out) return fail(ABP_ERR_INVALID_ARG, "num_cus is NULL");
    return num_cus(device, out);
  } catch (...) {
    return fail(ABP_ERR_HIP, "exception");
  }
}

int abp_workspace_size(int kind, const abp_params* params, int32_t max_batch,
                       int32_t max_qo_tokens, int32_t num_workers, size_t* host_bytes,
                       size_t* dev_bytes) {
  try {
    if (!host_bytes || !dev_bytes) return fail(ABP_ERR_INVALID_ARG, "NULL size pointer");
    abp::Config cfg;
    abp::Layout L;
    int st = resolve_layout(kind, params, max_batch, max_qo_tokens, num_workers, &cfg, &L);
    if (st != ABP_OK) return st;
    *host_bytes = L.plan_bytes;
    *dev_bytes = L.dev_bytes;
    return ABP_OK;
  } catch (...) {
    return fail(ABP_ERR_INVALID_ARG, "exception");
  }
}

int abp_plan_host(int kind, const abp_params* params, int32_t batch, const int32_t* qo_indptr_h,
                  const int32_t* kv_indptr_h, const int32_t* kv_last_page_len_h,
                  int32_t max_batch, int32_t max_qo_tokens, int32_t num_workers, void* host_ws,
                  size_t host_bytes, abp_plan* plan) {
  try {
    if (num_workers <= 0 && num_workers != ABP_WORKERS_PER_TILE)
      return fail(ABP_ERR_INVALID_ARG, "abp_plan_host needs num_workers > 0 or ABP_WORKERS_PER_TILE");
    if (kind == ABP_KIND_BSR)
      return fail(ABP_ERR_INVALID_ARG, "block-sparse plans are made by abp_bsr_plan_host");
    return do_plan(kind, params, batch, qo_indptr_h, kv_indptr_h, kv_last_page_len_h, max_batch,
                   max_qo_tokens, num_workers, host_ws, host_bytes, plan, nullptr, nullptr);
  } catch (...) {
    return fail(ABP_ERR_INVALID_ARG, "exception");
  }
}

// True when `p` is pinned host memory that the GPU addresses at the same
// virtual address (hipHostMalloc memory), 16-byte aligned, so a kernel may read
// it. Pageable or unknown memory gives false (and leaves no sticky HIP error).
static bool mapped_pinned(const void* p, uint64_t bytes) {
  if ((reinterpret_cast<uintptr_t>(p) & 15) || (bytes & 3)) return false;
  hipPointerAttribute_t attr{};
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return attr.type == hipMemoryTypeHost && !attr.isManaged && attr.devicePointer == p;
}

// Block-sparse plan on the host: the BSR pattern becomes append requests (one
// per row block) whose query ranges and page counts the planner writes into
// the blob's aux region.
static int do_bsr_plan(const abp_params* params, int32_t M, int32_t N, int32_t R,
                       const int32_t* indptr_h, int32_t max_rb, int32_t max_M, int32_t workers,
                       void* host_ws, size_t host_bytes, abp_plan* plan, abp::Layout* lay_out) {
  if (!plan) return fail(ABP_ERR_INVALID_ARG, "plan is NULL");
  if (!host_ws) return fail(ABP_ERR_INVALID_ARG, "host workspace is NULL");
  if (M > max_M) return fail(ABP_ERR_WORKSPACE_TOO_SMALL, "M > max_M");
  if (R >= 1 && M >= 0 && (int64_t(M) + R - 1) / R > max_rb)
    return fail(ABP_ERR_WORKSPACE_TOO_SMALL, "ceil(M / R) > max_row_blocks");
  abp::Config cfg;
  abp::Layout L;
  int st = resolve_layout(ABP_KIND_BSR, params, max_rb, max_M, workers, &cfg, &L);
  if (st != ABP_OK) return st;
  if (host_bytes < L.plan_bytes)
    return fail(ABP_ERR_WORKSPACE_TOO_SMALL, "host workspace smaller than abp_workspace_size");
  std::string err;
  st = abp::bsr_plan_compute(cfg, L, M, N, R, indptr_h, static_cast<int32_t*>(host_ws), plan,
                             &err);
  if (st != ABP_OK) return fail(st, err);
  if (lay_out) *lay_out = L;
  return ABP_OK;
}

static int upload_plan(const abp::Layout& L, void* host_ws, void* dev_ws, size_t dev_bytes,
                       abp_stream_t stream, abp_plan* plan);

static int plan_and_upload(int kind, const abp_params* params, int32_t batch,
                           const int32_t* qo_indptr_h, const int32_t* kv_indptr_h,
                           const int32_t* lpl_h, int32_t max_batch, int32_t max_qo,
                           int32_t workers, void* host_ws, size_t host_bytes, void* dev_ws,
                           size_t dev_bytes, abp_stream_t stream, abp_plan* plan) {
  abp::Config cfg;
  abp::Layout L;
  int st = do_plan(kind, params, batch, qo_indptr_h, kv_indptr_h, lpl_h, max_batch, max_qo,
                   workers, host_ws, host_bytes, plan, &cfg, &L);
  if (st != ABP_OK) return st;
  return upload_plan(L, host_ws, dev_ws, dev_bytes, stream, plan);
}

// Copy the plan blob to the start of dev_ws on `stream`.
static int upload_plan(const abp::Layout& L, void* host_ws, void* dev_ws, size_t dev_bytes,
                       abp_stream_t stream, abp_plan* plan) {
  if (!dev_ws) return fail(ABP_ERR_INVALID_ARG, "device workspace is NULL");
  if (dev_bytes < L.dev_bytes)
    return fail(ABP_ERR_WORKSPACE_TOO_SMALL, "device workspace smaller than abp_workspace_size");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (mapped_pinned(host_ws, L.plan_bytes)) {
    // pinned host memory: a small kernel on the same queue reads it directly
    hipError_t e = abp::launch_upload(dev_ws, host_ws, L.plan_bytes, s);
    if (e != hipSuccess) return hip_fail(e, "plan upload kernel");
    plan->upload_path = 1;
  } else {
    hipError_t e = hipMemcpyAsync(dev_ws, host_ws, L.plan_bytes, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(plan)");
    plan->upload_path = 0;
  }
  return ABP_OK;
}

int abp_decode_plan(const abp_params* params, int32_t batch, const int32_t* kv_indptr_h,
                    const int32_t* kv_last_page_len_h, int32_t max_batch, int32_t num_workers,
                    void* host_ws, size_t host_bytes, void* dev_ws, size_t dev_bytes,
                    abp_stream_t stream, abp_plan* plan) {
  try {
    return plan_and_upload(ABP_KIND_DECODE, params, batch, nullptr, kv_indptr_h,
                           kv_last_page_len_h, max_batch, 0, num_workers, host_ws, host_bytes,
                           dev_ws, dev_bytes, stream, plan);
  } catch (...) {
    return fail(ABP_ERR_INVALID_ARG, "exception");
  }
}

int abp_append_plan(const abp_params* params, int32_t batch, const int32_t* qo_indptr_h,
                    const int32_t* kv_indptr_h, const int32_t* kv_last_page_len_h,
                    int32_t max_batch, int32_t max_qo_tokens, int32_t num_workers,
                    void* host_ws, size_t host_bytes, void* dev_ws, size_t dev_bytes,
                    abp_stream_t stream, abp_plan* plan) {
  try {
    if (!qo_indptr_h) return fail(ABP_ERR_INVALID_ARG, "qo_indptr is NULL");
    return plan_and_upload(ABP_KIND_APPEND, params, batch, qo_indptr_h, kv_indptr_h,
                           kv_last_page_len_h, max_batch, max_qo_tokens, num_workers, host_ws,
                           host_bytes, dev_ws, dev_bytes, stream, plan);
  } catch (...) {
    return fail(ABP_ERR_INVALID_ARG, "exception");
  }
}

int abp_decode_run(const abp_plan* plan, const abp_params* params, const void* q,
                   const void* k_pages, const void* v_pages, const int32_t* kv_indptr_d,
                   const int32_t* kv_indices_d, const int32_t* kv_last_page_len_d,
                   const int32_t* q_pos_d, const int32_t* kv_pos_offset_d, void* o, float* lse,
                   void* dev_ws, size_t dev_bytes, abp_stream_t stream) {
  try {
    abp::Config cfg;
    abp::Layout L;
    int st = prepare_run(ABP_KIND_DECODE, plan, params, dev_ws, dev_bytes, &cfg, &L);
    if (st != ABP_OK) return st;
    if (plan->num_tiles > 0 && (!q || !k_pages || !v_pages || !kv_indptr_d || !kv_indices_d ||
                            !kv_last_page_len_d || !o))
      return fail(ABP_ERR_INVALID_ARG, "NULL tensor pointer");
    if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o))
      return fail(ABP_ERR_INVALID_ARG, "q, k_pages, v_pages and o must be 16-byte aligned");
    abp::AttnArgs a = {};
    a.q = q;
    a.k_pages = k_pages;
    a.v_pages = v_pages;
    a.kv_indptr = kv_indptr_d;
    a.kv_indices = kv_indices_d;
    a.kv_last_page_len = kv_last_page_len_d;
    a.q_pos = q_pos_d;
    a.kv_pos_offset = kv_pos_offset_d;
    a.o = o;
    a.lse = lse;
    fill_args(cfg, L, plan, dev_ws, &a);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = abp::launch_decode(cfg, a, s);
    if (e != hipSuccess) return hip_fail(e, "decode kernel launch");
    // decode tiles are split often and are cheap: a second launch merges them
    // (append merges its few split tiles inside the kernel)
    e = abp::launch_plan_merge(cfg, a, decode_merge_grid(*plan), s);
    if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
    return ABP_OK;
  } catch (...) {
    return fail(ABP_ERR_HIP, "exception");
  }
}

int abp_append_run(const abp_plan* plan, const abp_params* params, const void* q,
                   const void* k_pages, const void* v_pages, const int32_t* qo_indptr_d,
                   const int32_t* kv_indptr_d, const int32_t* kv_indices_d,
                   const int32_t* kv_last_page_len_d, const int32_t* q_pos_d,
                   const int32_t* kv_pos_offset_d, void* o, float* lse, void* dev_ws,
                   size_t dev_bytes, abp_stream_t stream) {
  try {
    abp::Config cfg;
    abp::Layout L;
    int st = prepare_run(ABP_KIND_APPEND, plan, params, dev_ws, dev_bytes, &cfg, &L);
    if (st != ABP_OK) return st;
    if (plan->num_tiles > 0 && (!q || !k_pages || !v_pages || !qo_indptr_d || !kv_indptr_d ||
                            !kv_indices_d || !kv_last_page_len_d || !o))
      return fail(ABP_ERR_INVALID_ARG, "NULL tensor pointer");
    if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o))
      return fail(ABP_ERR_INVALID_ARG, "q, k_pages, v_pages and o must be 16-byte aligned");
    abp::AttnArgs a = {};
    a.q = q;
    a.k_pages = k_pages;
    a.v_pages = v_pages;
    a.qo_indptr = qo_indptr_d;
    a.kv_indptr = kv_indptr_d;
    a.kv_indices = kv_indices_d;
    a.kv_last_page_len = kv_last_page_len_d;
    a.q_pos = q_pos_d;
    a.kv_pos_offset = kv_pos_offset_d;
    a.o = o;
    a.lse = lse;
    fill_args(cfg, L, plan, dev_ws, &a);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = abp::launch_append(cfg, a, s);
    if (e != hipSuccess) return hip_fail(e, "append kernel launch");
    // tiles split into many partials are merged across all CUs (the plan says
    // which; the kernel returns at once otherwise, so the launch sequence does
    // not depend on the plan)
    e = abp::launch_plan_merge(cfg, a, plan->num_workers, s);
    if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
    return ABP_OK;
  } catch (...) {
    return fail(ABP_ERR_HIP, "exception");
  }
}

int abp_bsr_plan_host(const abp_params* params, int32_t M, int32_t N, int32_t R,
                      const int32_t* indptr_h, int32_t max_row_blocks, int32_t max_M,
                      int32_t num_workers, void* host_ws, size_t host_bytes, abp_plan* plan) {
  try {
    if (num_workers <= 0)
      return fail(ABP_ERR_INVALID_ARG, "abp_bsr_plan_host needs num_workers > 0");
    return do_bsr_plan(params, M, N, R, indptr_h, max_row_blocks, max_M, num_workers, host_ws,
                       host_bytes, plan, nullptr);
  } catch (...) {
    return fail(ABP_ERR_INVALID_ARG, "exception");
  }
}

int abp_bsr_plan(const abp_params* params, int32_t M, int32_t N, int32_t R,
                 const int32_t* indptr_h, int32_t max_row_blocks, int32_t max_M,
                 int32_t num_workers, void* host_ws, size_t host_bytes, void* dev_ws,
                 size_t dev_bytes, abp_stream_t stream, abp_plan* plan) {
  try {
    abp::Layout L;
    int st = do_bsr_plan(params, M, N, R, indptr_h, max_row_blocks, max_M, num_workers, host_ws,
                         host_bytes, plan, &L);
    if (st != ABP_OK) return st;
    return upload_plan(L, host_ws, dev_ws, dev_bytes, stream, plan);
  } catch (...) {
    return fail(ABP_ERR_INVALID_ARG, "exception");
  }
}

int abp_bsr_run(const abp_plan* plan, const abp_params* params, const void* q, const void* k,
                const void* v, const int32_t* indptr_d, const int32_t* indices_d, void* o,
                float* lse, void* dev_ws, size_t dev_bytes, abp_stream_t stream) {
  try {
    abp::Config cfg;
    abp::Layout L;
    int st = prepare_run(ABP_KIND_BSR, plan, params, dev_ws, dev_bytes, &cfg, &L);
    if (st != ABP_OK) return st;
    if (plan->num_tiles > 0 && (!q || !k || !v || !indptr_d || !indices_d || !o))
      return fail(ABP_ERR_INVALID_ARG, "NULL tensor pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
      return fail(ABP_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
    // row block i is append request i; its query range and page count come
    // from the aux region the planner filled (k / v viewed as [N / C, C, Hkv, d])
    const int32_t* aux = reinterpret_cast<const int32_t*>(dev_ws) + L.off_aux;
    abp::AttnArgs a = {};
    a.q = q;
    a.k_pages = k;
    a.v_pages = v;
    a.qo_indptr = aux;
    a.kv_indptr = indptr_d;
    a.kv_indices = indices_d;
    a.kv_last_page_len = aux + ((int64_t(L.aux_cap) + 1 + 3) & ~int64_t(3));
    a.o = o;
    a.lse = lse;
    fill_args(cfg, L, plan, dev_ws, &a);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = abp::launch_append(cfg, a, s);
    if (e != hipSuccess) return hip_fail(e, "append kernel launch (block-sparse)");
    e = abp::launch_plan_merge(cfg, a, plan->num_workers, s);
    if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
    return ABP_OK;
  } catch (...) {
    return fail(ABP_ERR_HIP, "exception");
  }
}

int abp_append_paged_kv(const abp_params* params, int32_t batch, int64_t nnz, const void* k_new,
                        const void* v_new, const int32_t* append_indptr_d, void* k_pages,
                        void* v_pages, const int32_t* kv_indptr_d, const int32_t* kv_indices_d,
                        const int32_t* kv_last_page_len_d, abp_stream_t stream) {
  try {
    if (!params) return fail(ABP_ERR_INVALID_ARG, "params is NULL");
    if (params->head_dim != 128) return fail(ABP_ERR_UNSUPPORTED, "only head_dim 128 is built");
    if (params->num_kv_heads < 1 || params->page_size < 1)
      return fail(ABP_ERR_INVALID_ARG, "num_kv_heads and page_size must be >= 1");
    if (params->qkv_dtype != ABP_F16 && params->qkv_dtype != ABP_BF16)
      return fail(ABP_ERR_UNSUPPORTED, "qkv_dtype must be ABP_F16 or ABP_BF16");
    if (params->kv_fp8 != 0 && params->kv_fp8 != 1)
      return fail(ABP_ERR_INVALID_ARG, "kv_fp8 must be 0 or 1");
    if (batch < 0 || nnz < 0) return fail(ABP_ERR_INVALID_ARG, "batch and nnz must be >= 0");
    if (nnz == 0 || batch == 0) return ABP_OK;
    if (nnz > (int64_t(1) << 31) - 1) return fail(ABP_ERR_INVALID_ARG, "nnz must be < 2^31");
    if (!k_new || !v_new || !append_indptr_d || !k_pages || !v_pages || !kv_indptr_d ||
        !kv_indices_d || !kv_last_page_len_d)
      return fail(ABP_ERR_INVALID_ARG, "NULL pointer");
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pages) || !aligned16(v_pages))
      return fail(ABP_ERR_INVALID_ARG, "K/V pointers must be 16-byte aligned");
    hipError_t e = abp::launch_page_append(
        k_new, v_new, append_indptr_d, k_pages, v_pages, kv_indptr_d, kv_indices_d,
        kv_last_page_len_d, batch, nnz, params->num_kv_heads * 128 * (params->kv_fp8 ? 1 : 2),
        params->page_size,
        reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "page append launch");
    return ABP_OK;
  } catch (...) {
    return fail(ABP_ERR_HIP, "exception");
  }
}

// ---------------------------------------------------------------------------
// Mixed decode + append batches (one launch, workgroups split by role)

int abp_pod_workspace_size(const abp_params* params, int32_t max_decode_batch,
                           int32_t max_append_batch, int32_t max_qo_tokens, int32_t num_groups,
                           size_t* host_bytes, size_t* dev_bytes) {
  try {
    if (!host_bytes || !dev_bytes) return fail(ABP_ERR_INVALID_ARG, "NULL output");
    PodLayout P;
    int st = pod_layout(params, max_decode_batch, max_append_batch, max_qo_tokens, num_groups, &P);
    if (st != ABP_OK) return st;
    *host_bytes = P.d_host + P.a_host;
    *dev_bytes = P.d_dev + P.a_dev;
    return ABP_OK;
  } catch (...) {
    return fail(ABP_ERR_INVALID_ARG, "exception");
  }
}

int abp_pod_plan_host(const abp_params* params, int32_t decode_batch,
                      const int32_t* d_kv_indptr_h, const int32_t* d_kv_last_page_len_h,
                      int32_t append_batch, const int32_t* qo_indptr_h,
                      const int32_t* a_kv_indptr_h, const int32_t* a_kv_last_page_len_h,
                      int32_t max_decode_batch, int32_t max_append_batch, int32_t max_qo_tokens,
                      int32_t num_groups, int32_t decode_groups, void* host_ws,
                      size_t host_bytes, abp_pod_plan_t* plan) {
  try {
    PodLayout P;
    return pod_plan_host(params, decode_batch, d_kv_indptr_h, d_kv_last_page_len_h, append_batch,
                         qo_indptr_h, a_kv_indptr_h, a_kv_last_page_len_h, max_decode_batch,
                         max_append_batch, max_qo_tokens, num_groups, decode_groups, host_ws,
                         host_bytes, plan, &P);
  } catch (...) {
    return fail(ABP_ERR_INVALID_ARG, "exception");
  }
}

int abp_pod_plan(const abp_params* params, int32_t decode_batch, const int32_t* d_kv_indptr_h,
                 const int32_t* d_kv_last_page_len_h, int32_t append_batch,
                 const int32_t* qo_indptr_h, const int32_t* a_kv_indptr_h,
                 const int32_t* a_kv_last_page_len_h, int32_t max_decode_batch,
                 int32_t max_append_batch, int32_t max_qo_tokens, int32_t num_groups,
                 int32_t decode_groups, void* host_ws, size_t host_bytes, void* dev_ws,
                 size_t dev_bytes, abp_stream_t stream, abp_pod_plan_t* plan) {
  try {
    PodLayout P;
    int st = pod_plan_host(params, decode_batch, d_kv_indptr_h, d_kv_last_page_len_h,
                           append_batch, qo_indptr_h, a_kv_indptr_h, a_kv_last_page_len_h,
                           max_decode_batch, max_append_batch, max_qo_tokens, num_groups,
                           decode_groups, host_ws, host_bytes, plan, &P);
    if (st != ABP_OK) return st;
    if (!dev_ws) return fail(ABP_ERR_INVALID_ARG, "device workspace is NULL");
    if (dev_bytes < P.d_dev + P.a_dev)
      return fail(ABP_ERR_WORKSPACE_TOO_SMALL, "device workspace smaller than abp_pod_workspace_size");
    char* hw = static_cast<char*>(host_ws);
    char* dw = static_cast<char*>(dev_ws);
    if (plan->decode.num_workers > 0) {
      st = upload_plan(P.ld, hw + plan->decode_host_offset, dw + plan->decode_dev_offset,
                       P.d_dev, stream, &plan->decode);
      if (st != ABP_OK) return st;
    }
    if (plan->append.num_workers > 0) {
      st = upload_plan(P.la, hw + plan->append_host_offset, dw + plan->append_dev_offset,
                       P.a_dev, stream, &plan->append);
      if (st != ABP_OK) return st;
    }
    return ABP_OK;
  } catch (...) {
    return fail(ABP_ERR_INVALID_ARG, "exception");
  }
}

int abp_pod_run(const abp_pod_plan_t* plan, const abp_params* params, const void* q_decode,
                const void* q_append, const void* k_pages, const void* v_pages,
                const int32_t* d_kv_indptr_d, const int32_t* d_kv_indices_d,
                const int32_t* d_kv_last_page_len_d, const int32_t* qo_indptr_d,
                const int32_t* a_kv_indptr_d, const int32_t* a_kv_indices_d,
                const int32_t* a_kv_last_page_len_d, void* o_decode, float* lse_decode,
                void* o_append, float* lse_append, void* dev_ws, size_t dev_bytes,
                abp_stream_t stream) {
  try {
    if (!plan || !params) return fail(ABP_ERR_INVALID_ARG, "plan or params is NULL");
    if (!dev_ws) return fail(ABP_ERR_INVALID_ARG, "device workspace is NULL");
    if (dev_bytes < plan->decode_dev_bytes + plan->append_dev_bytes ||
        plan->append_dev_offset < plan->decode_dev_bytes)
      return fail(ABP_ERR_WORKSPACE_TOO_SMALL, "device workspace smaller than the plan's regions");
    const int32_t wd = plan->decode.num_workers, wa = plan->append.num_workers;
    if (wd < 0 || wa < 0 || wd + wa > plan->num_groups)
      return fail(ABP_ERR_PLAN_MISMATCH, "inconsistent worker split");
    abp_params pd = *params;
    pd.causal = 0;
    char* dw = static_cast<char*>(dev_ws);
    abp::Config cd, ca;
    abp::Layout ld, la;
    abp::AttnArgs dec = {}, app = {};
    if (wd > 0) {
      int st = prepare_run(ABP_KIND_DECODE, &plan->decode, &pd, dw + plan->decode_dev_offset,
                           plan->decode_dev_bytes, &cd, &ld);
      if (st != ABP_OK) return st;
      if (!abp::pod_applies(cd)) return fail(ABP_ERR_UNSUPPORTED, "params not supported for mixed batches");
      if (plan->decode.num_tiles > 0 && (!q_decode || !k_pages || !v_pages || !d_kv_indptr_d ||
                                         !d_kv_indices_d || !d_kv_last_page_len_d || !o_decode))
        return fail(ABP_ERR_INVALID_ARG, "NULL decode tensor pointer");
      if (!aligned16(q_decode) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o_decode))
        return fail(ABP_ERR_INVALID_ARG, "q, k_pages, v_pages and o must be 16-byte aligned");
      dec.q = q_decode;
      dec.k_pages = k_pages;
      dec.v_pages = v_pages;
      dec.kv_indptr = d_kv_indptr_d;
      dec.kv_indices = d_kv_indices_d;
      dec.kv_last_page_len = d_kv_last_page_len_d;
      dec.o = o_decode;
      dec.lse = lse_decode;
      fill_args(cd, ld, &plan->decode, dw + plan->decode_dev_offset, &dec);
    }
    if (wa > 0) {
      int st = prepare_run(ABP_KIND_APPEND, &plan->append, params, dw + plan->append_dev_offset,
                           plan->append_dev_bytes, &ca, &la);
      if (st != ABP_OK) return st;
      if (!abp::pod_applies(ca)) return fail(ABP_ERR_UNSUPPORTED, "params not supported for mixed batches");
      if (plan->append.num_tiles > 0 && (!q_append || !k_pages || !v_pages || !qo_indptr_d ||
                                         !a_kv_indptr_d || !a_kv_indices_d ||
                                         !a_kv_last_page_len_d || !o_append))
        return fail(ABP_ERR_INVALID_ARG, "NULL append tensor pointer");
      if (!aligned16(q_append) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o_append))
        return fail(ABP_ERR_INVALID_ARG, "q, k_pages, v_pages and o must be 16-byte aligned");
      app.q = q_append;
      app.k_pages = k_pages;
      app.v_pages = v_pages;
      app.qo_indptr = qo_indptr_d;
      app.kv_indptr = a_kv_indptr_d;
      app.kv_indices = a_kv_indices_d;
      app.kv_last_page_len = a_kv_last_page_len_d;
      app.o = o_append;
      app.lse = lse_append;
      fill_args(ca, la, &plan->append, dw + plan->append_dev_offset, &app);
    }
    if (wd + wa == 0) return ABP_OK;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = abp::launch_pod(wa > 0 ? ca : cd, app, dec, s);
    if (e != hipSuccess) return hip_fail(e, "mixed kernel launch");
    if (wd > 0) {
      e = abp::launch_plan_merge(cd, dec, decode_merge_grid(plan->decode), s);
      if (e != hipSuccess) return hip_fail(e, "decode merge kernel launch");
    }
    if (wa > 0) {
      e = abp::launch_plan_merge(ca, app, wa, s);
      if (e != hipSuccess) return hip_fail(e, "append merge kernel launch");
    }
    return ABP_OK;
  } catch (...) {
    return fail(ABP_ERR_HIP, "exception");
  }
}

int abp_cascade_run(const abp_plan* prefix_plan, const abp_params* prefix_params,
                    void* prefix_dev_ws, size_t prefix_dev_bytes, const abp_plan* suffix_plan,
                    const abp_params* suffix_params, void* suffix_dev_ws, size_t suffix_dev_bytes,
                    const void* q, const void* prefix_k_pages, const void* prefix_v_pages,
                    const int32_t* prefix_qo_indptr_d, const int32_t* prefix_kv_indptr_d,
                    const int32_t* prefix_kv_indices_d, const int32_t* prefix_kv_last_page_len_d,
                    const void* k_pages, const void* v_pages, const int32_t* kv_indptr_d,
                    const int32_t* kv_indices_d, const int32_t* kv_last_page_len_d,
                    const int32_t* q_pos_d, const int32_t* kv_pos_offset_d, float* o_prefix,
                    float* lse_prefix, float* o_suffix, float* lse_suffix, void* o, float* lse,
                    int32_t out_dtype, abp_stream_t stream) {
  try {
    abp::Config cp, cs;
    abp::Layout lp, ls;
    int st = prepare_run(ABP_KIND_APPEND, prefix_plan, prefix_params, prefix_dev_ws,
                         prefix_dev_bytes, &cp, &lp);
    if (st != ABP_OK) return st;
    st = prepare_run(ABP_KIND_DECODE, suffix_plan, suffix_params, suffix_dev_ws, suffix_dev_bytes,
                     &cs, &ls);
    if (st != ABP_OK) return st;
    if (cp.out_dtype != ABP_F32 || cs.out_dtype != ABP_F32)
      return fail(ABP_ERR_UNSUPPORTED, "cascade levels must write fp32 states (out_dtype ABP_F32)");
    if (cp.hq != cs.hq || cp.hkv != cs.hkv || cp.qkv_dtype != cs.qkv_dtype || cp.causal)
      return fail(ABP_ERR_PLAN_MISMATCH,
                  "cascade levels need the same heads and q dtype, and a non-causal prefix");
    if (out_dtype < ABP_F16 || out_dtype > ABP_F32)
      return fail(ABP_ERR_UNSUPPORTED, "out_dtype must be ABP_F16, ABP_BF16 or ABP_F32");
    const int32_t B = suffix_plan->batch;
    // the prefix is one request whose query tokens are the suffix level's B
    // queries: its tiles are (kv-head group, query tile), one head per tile
    const int32_t tq = prefix_plan->tile_q;
    const int64_t want_tiles = int64_t(cp.hkv) * ((B + tq - 1) / tq);
    if (prefix_plan->batch != 1 || lp.tile_heads != 1 || prefix_plan->num_tiles != want_tiles)
      return fail(ABP_ERR_PLAN_MISMATCH,
                  "prefix plan must be one request with the suffix batch's queries");
    if (B > 0 && (!q || !prefix_k_pages || !prefix_v_pages || !prefix_qo_indptr_d ||
                  !prefix_kv_indptr_d || !prefix_kv_indices_d || !prefix_kv_last_page_len_d ||
                  !k_pages || !v_pages || !kv_indptr_d || !kv_indices_d || !kv_last_page_len_d ||
                  !o_prefix || !lse_prefix || !o_suffix || !lse_suffix || !o))
      return fail(ABP_ERR_INVALID_ARG, "NULL tensor pointer");
    if (!aligned16(q) || !aligned16(prefix_k_pages) || !aligned16(prefix_v_pages) ||
        !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o_prefix) ||
        !aligned16(o_suffix) || !aligned16(o))
      return fail(ABP_ERR_INVALID_ARG, "q, pages and o buffers must be 16-byte aligned");
    abp::AttnArgs ap = {};
    ap.q = q;
    ap.k_pages = prefix_k_pages;
    ap.v_pages = prefix_v_pages;
    ap.qo_indptr = prefix_qo_indptr_d;
    ap.kv_indptr = prefix_kv_indptr_d;
    ap.kv_indices = prefix_kv_indices_d;
    ap.kv_last_page_len = prefix_kv_last_page_len_d;
    ap.q_pos = q_pos_d;
    ap.kv_pos_offset = nullptr;  // prefix keys sit at 0 .. prefix length - 1
    ap.o = o_prefix;
    ap.lse = lse_prefix;
    fill_args(cp, lp, prefix_plan, prefix_dev_ws, &ap);
    abp::AttnArgs as = {};
    as.q = q;
    as.k_pages = k_pages;
    as.v_pages = v_pages;
    as.kv_indptr = kv_indptr_d;
    as.kv_indices = kv_indices_d;
    as.kv_last_page_len = kv_last_page_len_d;
    as.q_pos = q_pos_d;
    as.kv_pos_offset = kv_pos_offset_d;
    as.o = o_suffix;
    as.lse = lse_suffix;
    fill_args(cs, ls, suffix_plan, suffix_dev_ws, &as);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = abp::launch_append(cp, ap, s);
    if (e != hipSuccess) return hip_fail(e, "prefix append kernel launch");
    e = abp::launch_decode(cs, as, s);
    if (e != hipSuccess) return hip_fail(e, "suffix decode kernel launch");
    e = abp::launch_cascade_merge(ap, as, B, o, lse, out_dtype, s);
    if (e != hipSuccess) return hip_fail(e, "cascade merge kernel launch");
    return ABP_OK;
  } catch (...) {
    return fail(ABP_ERR_HIP, "exception");
  }
}

int abp_merge_state(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                    void* o_out, float* lse_out, int64_t num_rows, int32_t head_dim,
                    int in_dtype, int out_dtype, abp_stream_t stream) {
  try {
    if (head_dim != 128) return fail(ABP_ERR_UNSUPPORTED, "only head_dim 128 is built");
    if (num_rows < 0) return fail(ABP_ERR_INVALID_ARG, "num_rows < 0");
    if (in_dtype < ABP_F16 || in_dtype > ABP_F32 || out_dtype < ABP_F16 || out_dtype > ABP_F32)
      return fail(ABP_ERR_UNSUPPORTED, "dtype must be ABP_F16, ABP_BF16 or ABP_F32");
    if (num_rows > 0 && (!o_a || !lse_a || !o_b || !lse_b || !o_out))
      return fail(ABP_ERR_INVALID_ARG, "NULL pointer");
    if (!aligned16(o_a) || !aligned16(o_b) || !aligned16(o_out))
      return fail(ABP_ERR_INVALID_ARG, "o pointers must be 16-byte aligned");
    hipError_t e = abp::launch_merge_two(o_a, lse_a, o_b, lse_b, o_out, lse_out, num_rows,
                                         in_dtype, out_dtype, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "merge_state launch");
    return ABP_OK;
  } catch (...) {
    return fail(ABP_ERR_HIP, "exception");
  }
}

int abp_merge_states(const void* o_in, const float* lse_in, int32_t num_states, int64_t num_rows,
                     int32_t head_dim, int in_dtype, int out_dtype, void* o_out, float* lse_out,
                     abp_stream_t stream) {
  try {
    if (head_dim != 128) return fail(ABP_ERR_UNSUPPORTED, "only head_dim 128 is built");
    if (num_rows < 0 || num_states < 0) return fail(ABP_ERR_INVALID_ARG, "negative size");
    if (in_dtype < ABP_F16 || in_dtype > ABP_F32 || out_dtype < ABP_F16 || out_dtype > ABP_F32)
      return fail(ABP_ERR_UNSUPPORTED, "dtype must be ABP_F16, ABP_BF16 or ABP_F32");
    if (num_rows > 0 && (!o_out || (num_states > 0 && (!o_in || !lse_in))))
      return fail(ABP_ERR_INVALID_ARG, "NULL pointer");
    if (!aligned16(o_in) || !aligned16(o_out))
      return fail(ABP_ERR_INVALID_ARG, "o pointers must be 16-byte aligned");
    hipError_t e = abp::launch_merge_states(o_in, lse_in, num_states, num_rows, in_dtype,
                                            out_dtype, o_out, lse_out,
                                            reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "merge_states launch");
    return ABP_OK;
  } catch (...) {
    return fail(ABP_ERR_HIP, "exception");
  }
}

}  // extern "C"
