// Append / prefill attention with LLaMA RoPE fused into the q and k loads, on
// gfx950 matrix cores: the append kernel's computation (append.hip) with q and
// every key rotated by its position before the score products (the RoPE
// fusion of the paper summary, "图谱动态｜学苑周刊 NO.266", section
// 可定制的注意力模板).
//
// The worker (append_worker_rope in append_impl.h) runs 8 waves of 16 rows
// over 128-row tiles; its rotated operands are carried as 16-bit hi and lo
// parts. This translation unit is built with the matrix products in VGPR form
// (-mllvm -amdgpu-mfma-vgpr-form): the O and S accumulators stay in VGPRs,
// where the softmax and the rare rescale use them directly. In the default
// form the compiler kept O in AGPRs and copied the accumulators to VGPRs on
// every block for the rescale branch.
#include "append_impl.h"

namespace abp {

namespace {

using appi::append_waves;

template <typename T, int G, bool CAUSAL, bool FASTPAGE, bool RIL>
__global__ __launch_bounds__(64 * append_waves<true>(), 1) void append_rope_kernel(AttnArgs a) {
  appi::append_worker_rope<T, G, CAUSAL, FASTPAGE, RIL>(a, blockIdx.x);
}

template <typename T, int G, bool CAUSAL, bool RIL>
hipError_t launch_f(const AttnArgs& a, hipStream_t s) {
  if (a.page_shift >= 4)
    append_rope_kernel<T, G, CAUSAL, true, RIL><<<a.workers, 64 * append_waves<true>(), 0, s>>>(a);
  else
    append_rope_kernel<T, G, CAUSAL, false, RIL><<<a.workers, 64 * append_waves<true>(), 0, s>>>(a);
  return hipGetLastError();
}

template <typename T, int G>
hipError_t launch_g(const Config& cfg, const AttnArgs& a, hipStream_t s) {
  if (cfg.causal)
    return cfg.rope_interleave ? launch_f<T, G, true, true>(a, s) : launch_f<T, G, true, false>(a, s);
  return cfg.rope_interleave ? launch_f<T, G, false, true>(a, s) : launch_f<T, G, false, false>(a, s);
}

template <typename T>
hipError_t launch_t(const Config& cfg, const AttnArgs& a, hipStream_t s) {
  switch (cfg.group) {
    case 1: return launch_g<T, 1>(cfg, a, s);
    case 2: return launch_g<T, 2>(cfg, a, s);
    case 4: return launch_g<T, 4>(cfg, a, s);
    case 8: return launch_g<T, 8>(cfg, a, s);
    case 16: return launch_g<T, 16>(cfg, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_append_rope(const Config& cfg, const AttnArgs& a, hipStream_t s) {
  if (cfg.qkv_dtype == ABP_BF16) return launch_t<BF16>(cfg, a, s);
  return launch_t<F16>(cfg, a, s);
}

int append_rope_blocks_per_cu() {
  int n = 0;
  // the tile shape is shared by all variants, each built for one per CU
  const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &n, append_rope_kernel<BF16, 4, true, true, false>, 64 * append_waves<true>(), 0);
  return e == hipSuccess && n > 0 ? n : 1;
}

}  // namespace abp
