// Merge of a split tile by the last worker to finish one of its segments.
//
// A tile cut over several workers writes one fp32 partial state (o normalised,
// lse) per segment. The states are combined in slot order (key order) with the
// natural-log sum of exponentials:
//   M = max lse_i,  lse = M + ln sum_i exp(lse_i - M),  o = sum_i exp(lse_i - lse) o_i,
// evaluated as a running fold over i (running max, rescaled sums),
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
// of `tile`. ROWS tile rows of head_dim 128 are merged by NT threads, each
// owning ROWS * 16 / NT items of 8 elements. `row_out(r, &orow)` maps tile row
// r to an output row and returns false for rows past the end of the request.
//
// The partials are folded in slot order with a running maximum (the same
// natural-log sum of exponentials, evaluated incrementally), so each step
// issues all loads of one partial for every item of the thread at once.
template <int ROWS, int NT, typename RowOut>
__device__ __forceinline__ void merge_if_last(const AttnArgs& a, int tile, int* s_last,
                                              RowOut row_out) {
  static_assert((ROWS * 16) % NT == 0, "items must divide evenly");
  constexpr int K = ROWS * 16 / NT;
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
  if (!*s_last) return;

  const int tid = threadIdx.x;
  constexpr int KC = K < 8 ? K : 8;  // items per pass (bounds the registers)
  for (int k0 = 0; k0 < K; k0 += KC) {
    float M[KC], tot[KC], acc[KC][8];
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      M[k] = kNegInf;
      tot[k] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[k][e] = 0.f;
    }
    for (int i = 0; i < np; ++i) {
      const int64_t slot_row = int64_t(first + i) * ROWS;
      float l[KC];
      float4 v[KC][2];
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        const int item = tid + (k0 + k) * NT;
        const int64_t sr = slot_row + (item >> 4);
        l[k] = a.lse_part[sr];
        const float4* src =
            reinterpret_cast<const float4*>(a.o_part + sr * 128 + (item & 15) * 8);
        v[k][0] = src[0];
        v[k][1] = src[1];
      }
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        const float nm = __builtin_fmaxf(M[k], l[k]);
        // rescale of the running sums; no change (and no -inf - -inf) when M holds
        const float sc = nm == M[k] ? 1.f : fast_exp2((M[k] - nm) * kLog2e);
        const float wt = l[k] == kNegInf ? 0.f : fast_exp2((l[k] - nm) * kLog2e);
        M[k] = nm;
        tot[k] = __builtin_fmaf(tot[k], sc, wt);
        const float x[8] = {v[k][0].x, v[k][0].y, v[k][0].z, v[k][0].w,
                            v[k][1].x, v[k][1].y, v[k][1].z, v[k][1].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[k][e] = __builtin_fmaf(acc[k][e], sc, wt * x[e]);
      }
    }
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      const int item = tid + (k0 + k) * NT;
      int64_t orow;
      if (!row_out(item >> 4, &orow)) continue;
      float out[8];
      float lse = kNegInf;
      if (M[k] != kNegInf) {
        const float inv = 1.f / tot[k];
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] = acc[k][e] * inv;
        lse = M[k] + fast_log2(tot[k]) * kLn2;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] = 0.f;
      }
      store8_out(a.o, orow * 128 + (item & 15) * 8, out, a.out_dtype);
      if (a.lse && (item & 15) == 0) a.lse[orow] = lse;
    }
  }
  if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace abp
