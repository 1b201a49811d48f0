// Mixed decode + append batches in one persistent launch on gfx950.
//
// Batches that hold both prefill (append) requests and decode requests are
// the case the POD attention kernels of the README target (gittoolsai.com,
// section 核心功能 / 注意力机制内核): decode is bound by HBM bandwidth and
// append by the matrix cores, so running them at the same time uses both.
// On this chip the append workgroup fills a compute unit's registers, so the
// two cannot share a compute unit: the launch gives each workgroup (one per
// compute unit) one role instead. Workgroups 0 .. Wa - 1 run the append
// plan's workers (the append kernel's body); workgroups Wa .. Wa + Wd - 1 run
// the decode plan's workers (the matrix-core decode body) on their first four
// waves. The planner picks Wd from a measured model of decode bandwidth
// against compute units, so that both parts end at about the same time: a
// few compute units already draw a large share of the HBM bandwidth, and the
// rest keep their matrix throughput for the append.
//
// Each part's outputs, partial states and merges are those of its own kernel,
// so the results are the same as those of the two runs made one after the
// other (split tiles of both parts are merged by the plan-merge launches that
// follow).
#include "append_impl.h"
#include "decode_mfma_impl.h"

namespace abp {

namespace {

// LDS: the decode role's arrays (K and V rings of 32 KB each, q rows); the
// append role borrows the four rings as its K and V stages (16 KB each), so
// one workgroup fits per compute unit.
template <typename T, int G, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void pod_kernel(AttnArgs app, AttnArgs dec) {
  static_assert(appi::append_waves<false>() == 8, "append workers are 512-thread workgroups");
  static_assert(4 * dmi::kC * dmi::kD >= appi::kTk * appi::kD, "append stages fit the rings");
  ABP_DECODE_LDS(dlds, G, false);
  __shared__ int app_last;
  const int b = blockIdx.x;
  if (b < app.workers) {
    const appi::PipeLds alds = {dlds.k0, dlds.k1, dlds.q, dlds.v0, dlds.v1, dlds.q, &app_last};
    appi::append_worker<T, G, CAUSAL, false, true, false, 2>(app, b, alds);
  } else if (threadIdx.x < 256) {
    // ordinary loads: few CUs
    dmi::decode_mfma_worker<T, G, false, false, false>(dec, b - app.workers, dlds);
  }
}

template <typename T, int G>
hipError_t launch_g(bool causal, const AttnArgs& app, const AttnArgs& dec, hipStream_t s) {
  const unsigned grid = unsigned(app.workers + dec.workers);
  if (causal)
    pod_kernel<T, G, true><<<grid, 512, 0, s>>>(app, dec);
  else
    pod_kernel<T, G, false><<<grid, 512, 0, s>>>(app, dec);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const Config& cfg, const AttnArgs& app, const AttnArgs& dec, hipStream_t s) {
  switch (cfg.group) {
    case 4: return launch_g<T, 4>(cfg.causal, app, dec, s);
    case 8: return launch_g<T, 8>(cfg.causal, app, dec, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool pod_applies(const Config& cfg) {
  return !cfg.kv_fp8 && !cfg.rope && decode_mfma_applies(cfg);
}

hipError_t launch_pod(const Config& cfg, const AttnArgs& app, const AttnArgs& dec, hipStream_t s) {
  if (app.workers < 0 || dec.workers < 0) return hipErrorInvalidValue;
  if (app.workers + dec.workers == 0) return hipSuccess;
  if (cfg.qkv_dtype == ABP_BF16) return launch_t<BF16>(cfg, app, dec, s);
  return launch_t<F16>(cfg, app, dec, s);
}

}  // namespace abp
