// Batch decode on gfx950 matrix cores (paged block-sparse-row KV cache).
//
// Same work split, plan and outputs as decode_kernel (paper summary
// "图谱动态｜学苑周刊 NO.266", sections 统一的 KV 缓存存储格式 and
// 动态负载均衡调度): a 256-thread workgroup is one worker, a tile is 4
// consecutive kv heads of one request and each wave owns one head. What
// changes is where the arithmetic runs. The vector-unit kernel spends most of
// its instructions on per-lane dot products, 16-lane reductions and one
// exponential per (token, row) in every lane; here both products run on the
// matrix cores and the vector unit does only the softmax of each score once:
//
//   S^T = K Q^T   v_mfma_f32_16x16x32: A = 16 token rows of K (lane: token
//                 l % 16, 16 bytes of head dims 32 kc + 8 (l / 16) ..), B = q
//                 of the G rows padded to 16. A 32-token chunk is two 16-token
//                 tiles x 4 head-dim windows = 8 products. With RoPE, q and K
//                 are rotated in fp32 and the products are fp32 ones
//                 (v_mfma_f32_16x16x4_f32, 32 per tile).
//   softmax       fp32, base 2, lazy rescale; a lane holds 8 scores of one row
//                 (l % 16); the row maximum is a 4-lane-group exchange.
//   O^T += V^T P^T  8 products (16 head dims each): B = P^T taken from the S^T
//                 registers in the order S holds the keys; A = V^T read from
//                 LDS with transpose reads.
//
// K, V and q go from global memory straight into per-wave LDS rings
// (memory-to-LDS loads, 16-byte pieces of a row XOR-swizzled by row), so no
// wave waits on another and every wait counts loads of one kind; a worker's
// chunks stream across its segments, the next segment's first chunk loading
// while the current segment ends. LDS: 136 or 144 KB (group 4 or 8), 154 KB
// with RoPE at group 8; one workgroup per compute unit.
//
// Scope (the dispatcher falls back to decode_kernel otherwise): 16-bit K/V
// with or without RoPE, or fp8 (e4m3, in decode_mfma_fp8_kernel below,
// without RoPE), power-of-two page size >= 16 (a 16-token tile never
// straddles a page), kv head count a multiple of 4, group size 4 or 8 (rows
// padded to 16).
//
// Built with the matrix products in VGPR form (-mllvm -amdgpu-mfma-vgpr-form):
// in the default form the compiler kept accumulators and loaded codes in
// AGPRs and moved them to VGPRs around the vector work (376 moves in the
// plain kernel, 864 in the fp8 one, 457 with RoPE; 0, 0 and 116 in VGPR form).
#include "decode_mfma_impl.h"

namespace abp {

namespace {

template <typename T, int G>
__global__ __launch_bounds__(256, 1) void decode_mfma_kernel(AttnArgs a) {
  ABP_DECODE_LDS(lds, G, false);
  dmi::decode_mfma_worker<T, G, true, false, false>(a, blockIdx.x, lds);
}

template <typename T, int G>
__global__ __launch_bounds__(256, 1) void decode_mfma_fp8_kernel(AttnArgs a) {
  dmi::decode_mfma_fp8_worker<T, G>(a, blockIdx.x);
}

template <typename T, int G, bool RIL>
__global__ __launch_bounds__(256, 1) void decode_mfma_rope_kernel(AttnArgs a) {
  ABP_DECODE_LDS(lds, G, true);
  dmi::decode_mfma_worker<T, G, true, true, RIL>(a, blockIdx.x, lds);
}

template <typename T>
hipError_t launch_t(const Config& cfg, const AttnArgs& a, hipStream_t s) {
  if (cfg.rope) {
    const bool il = cfg.rope_interleave != 0;
    switch (cfg.group) {
      case 4:
        if (il) decode_mfma_rope_kernel<T, 4, true><<<a.workers, 256, 0, s>>>(a);
        else decode_mfma_rope_kernel<T, 4, false><<<a.workers, 256, 0, s>>>(a);
        break;
      case 8:
        if (il) decode_mfma_rope_kernel<T, 8, true><<<a.workers, 256, 0, s>>>(a);
        else decode_mfma_rope_kernel<T, 8, false><<<a.workers, 256, 0, s>>>(a);
        break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (cfg.kv_fp8) {
    switch (cfg.group) {
      case 4: decode_mfma_fp8_kernel<T, 4><<<a.workers, 256, 0, s>>>(a); break;
      case 8: decode_mfma_fp8_kernel<T, 8><<<a.workers, 256, 0, s>>>(a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (cfg.group) {
    case 4: decode_mfma_kernel<T, 4><<<a.workers, 256, 0, s>>>(a); break;
    case 8: decode_mfma_kernel<T, 8><<<a.workers, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool decode_mfma_applies(const Config& cfg) {
  const bool pow2 = (cfg.page_size & (cfg.page_size - 1)) == 0;
  return !(cfg.rope && cfg.kv_fp8) && pow2 && cfg.page_size >= 16 && cfg.hkv % 4 == 0 &&
         (cfg.group == 4 || cfg.group == 8);
}

hipError_t launch_decode_mfma(const Config& cfg, const AttnArgs& a, hipStream_t s) {
  if (cfg.qkv_dtype == ABP_BF16) return launch_t<BF16>(cfg, a, s);
  return launch_t<F16>(cfg, a, s);
}

// Default workers per compute unit: fewer than fit. With non-temporal K/V
// loads, one 16-bit worker per compute unit beat two on the batch decode
// (99.8 against 102.2 us; skewed lengths 89.9 against 92.7 us). The fp8
// worker needs a compute unit's registers for its four chunk stages (one
// workgroup per compute unit: 61.0 us against 62.2 for two with two stages).
int decode_mfma_blocks_per_cu(const Config& cfg) {
  int n = 0;
  if (cfg.rope) {
    const hipError_t e = cfg.qkv_dtype == ABP_BF16
        ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_mfma_rope_kernel<BF16, 4, false>, 256, 0)
        : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_mfma_rope_kernel<F16, 4, false>, 256, 0);
    return e == hipSuccess ? (n < 1 ? n : 1) : 0;
  }
  if (cfg.kv_fp8) {
    const hipError_t e = cfg.qkv_dtype == ABP_BF16
        ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_mfma_fp8_kernel<BF16, 4>, 256, 0)
        : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_mfma_fp8_kernel<F16, 4>, 256, 0);
    return e == hipSuccess ? (n < 1 ? n : 1) : 0;
  }
  const hipError_t e = cfg.qkv_dtype == ABP_BF16
      ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_mfma_kernel<BF16, 4>, 256, 0)
      : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_mfma_kernel<F16, 4>, 256, 0);
  return e == hipSuccess ? (n < 1 ? n : 1) : 0;
}

}  // namespace abp
