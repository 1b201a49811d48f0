// Merge of a split tile by the last worker to finish one of its segments.
//
// A tile cut over several workers writes one fp32 partial state (o normalised,
// lse) per segment. The states are combined in slot order (key order) with the
// natural-log sum of exponentials:
//   M = max lse_i,  lse = M + ln sum_i exp(lse_i - M),  o = sum_i exp(lse_i - lse) o_i,
// and all-(-inf) inputs give (0, -inf) (paper summary "图谱动态｜学苑周刊
// NO.266", section 动态负载均衡调度: work units of one attention computation
// spread over the compute units and recombined).
//
// Arrival is counted with an agent-scope atomic per tile; partial stores are
// released before it and the merging worker acquires before reading them. The
// merging worker resets the counter, so the plan stays valid for repeated runs
// (graph replays); every plan upload also writes the counters as zero. There is
// no waiting on other workers, and the merge order does not depend on which
// worker merges, so results are bit-reproducible.
#pragma once
#include "common.h"
#include "kernels.h"
#include "layout.h"

namespace abp {

__device__ __forceinline__ void store8_out(void* base, int64_t off, const float v[8], int dt) {
  if (dt == ABP_F32) store8<ABP_F32>(base, off, v);
  else if (dt == ABP_BF16) store8<ABP_BF16>(base, off, v);
  else store8<ABP_F16>(base, off, v);
}

// Call with every thread of the workgroup after this worker stored its partial
// of `tile`. `row_out(r, &orow)` maps tile row r to an output row and returns
// false for rows past the end of the request. head_dim is 128.
template <typename RowOut>
__device__ __forceinline__ void merge_if_last(const AttnArgs& a, int tile, int rows,
                                              int* s_last, RowOut row_out) {
  const int32_t* plan = a.plan;
  const int np = plan[plan[H_OFF_NTILE] + tile];
  const int first = plan[plan[H_OFF_TILE] + 4 * tile + 3];
  int* cnt = const_cast<int*>(plan) + plan[H_OFF_CNT] + tile;
  // The barrier orders every wave's partial stores (completed to L2) before
  // thread 0's agent-scope release, which writes them back for other XCDs;
  // thread 0's acquire invalidates this CU's caches before the barrier that
  // lets the workgroup read the other workers' partials.
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    *s_last = prev == np - 1;
  }
  __syncthreads();
  if (*s_last) {
    for (int item = threadIdx.x; item < rows * 16; item += blockDim.x) {
      const int r = item >> 4;
      const int e0 = (item & 15) * 8;
      int64_t orow;
      if (!row_out(r, &orow)) continue;
      float M = kNegInf;
      for (int i = 0; i < np; ++i)
        M = __builtin_fmaxf(M, a.lse_part[int64_t(first + i) * rows + r]);
      float out[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = 0.f;
      float lse = kNegInf;
      if (M != kNegInf) {
        float tot = 0.f;
        for (int i = 0; i < np; ++i)
          tot += fast_exp2((a.lse_part[int64_t(first + i) * rows + r] - M) * kLog2e);
        lse = M + fast_log2(tot) * kLn2;
        for (int i = 0; i < np; ++i) {
          const int64_t sr = int64_t(first + i) * rows + r;
          const float w = fast_exp2((a.lse_part[sr] - lse) * kLog2e);
          float v[8];
          load8<ABP_F32>(a.o_part, sr * 128 + e0, v);
#pragma unroll
          for (int e = 0; e < 8; ++e) out[e] = __builtin_fmaf(w, v[e], out[e]);
        }
      }
      store8_out(a.o, orow * 128 + e0, out, a.out_dtype);
      if (a.lse && e0 == 0) a.lse[orow] = lse;
    }
    if (threadIdx.x == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace abp
