// Merging of attention states (o, lse) computed over disjoint key sets.
//
// Attention split over key ranges is recombined exactly through the natural-log
// sum of exponentials of the scaled logits: with M = max_i lse_i,
//   lse = M + ln sum_i exp(lse_i - M),   o = sum_i exp(lse_i - lse) o_i,
// and all-(-inf) inputs give (0, -inf). This is what lets the planner cut one
// request's keys over several workers (paper summary "图谱动态｜学苑周刊 NO.266",
// section 动态负载均衡调度) and what combines a shared prefix with per-request
// suffixes (section 统一的 KV 缓存存储格式: several formats in one attention).
//
// Layout: 16 lanes per row of 128, 8 consecutive elements per lane (one
// 16-byte load of bf16/fp16, two of fp32); 16 rows per 256-thread block. The
// merge order is fixed (slot 0, 1, ...), so results are bit-reproducible.
#include "common.h"
#include "kernels.h"
#include "layout.h"

namespace abp {

namespace {

template <int IN_DT, int OUT_DT>
__global__ __launch_bounds__(256) void merge_states_kernel(const void* o_in, const float* lse_in,
                                                           int32_t n, int64_t rows, void* o_out,
                                                           float* lse_out) {
  const int64_t row = int64_t(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int e0 = (threadIdx.x & 15) * 8;
  if (row >= rows) return;
  float M = kNegInf;
  for (int i = 0; i < n; ++i) M = __builtin_fmaxf(M, lse_in[int64_t(i) * rows + row]);
  float out[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = 0.f;
  float lse = kNegInf;
  if (M != kNegInf) {
    float tot = 0.f;
    for (int i = 0; i < n; ++i) tot += fast_exp2((lse_in[int64_t(i) * rows + row] - M) * kLog2e);
    lse = M + fast_log2(tot) * kLn2;
    for (int i = 0; i < n; ++i) {
      const int64_t sr = int64_t(i) * rows + row;
      const float w = fast_exp2((lse_in[sr] - lse) * kLog2e);
      float v[8];
      load8<IN_DT>(o_in, sr * 128 + e0, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = __builtin_fmaf(w, v[e], out[e]);
    }
  }
  store8<OUT_DT>(o_out, row * 128 + e0, out);
  if (lse_out && e0 == 0) lse_out[row] = lse;
}

template <int IN_DT, int OUT_DT>
__global__ __launch_bounds__(256) void merge_two_kernel(const void* o_a, const float* lse_a,
                                                        const void* o_b, const float* lse_b,
                                                        int64_t rows, void* o_out,
                                                        float* lse_out) {
  const int64_t row = int64_t(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int e0 = (threadIdx.x & 15) * 8;
  if (row >= rows) return;
  const float la = lse_a[row], lb = lse_b[row];
  const float M = __builtin_fmaxf(la, lb);
  float out[8];
  float lse = kNegInf;
  if (M == kNegInf) {
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = 0.f;
  } else {
    const float ea = fast_exp2((la - M) * kLog2e), eb = fast_exp2((lb - M) * kLog2e);
    lse = M + fast_log2(ea + eb) * kLn2;
    const float wa = fast_exp2((la - lse) * kLog2e), wb = fast_exp2((lb - lse) * kLog2e);
    float va[8], vb[8];
    load8<IN_DT>(o_a, row * 128 + e0, va);
    load8<IN_DT>(o_b, row * 128 + e0, vb);
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = __builtin_fmaf(wa, va[e], wb * vb[e]);
  }
  store8<OUT_DT>(o_out, row * 128 + e0, out);
  if (lse_out && e0 == 0) lse_out[row] = lse;
}

// Merge the split tiles of a plan after its main kernel (the kernel boundary
// orders the partial stores before these loads); a no-op when the append
// kernel merged them itself. Grid is fixed; counts come from the plan header
// at run time. One wave takes one (merge entry, tile row): its 4 groups of 16
// lanes fold every 4th partial (8 head-dim elements per lane) with a running
// maximum, loading 4 partials per group at a time, so 16 partials are in
// flight per round trip; the groups' states are then combined by lane
// exchange. Rows with many partials (a long request split over many workers)
// thus take few dependent memory round trips.
template <int OUT_DT>
__global__ __launch_bounds__(256) void plan_merge_kernel(AttnArgs a) {
  const ABP_CONST_AS int32_t* plan = const_as(a.plan);
  if (plan[H_MERGE_KERNEL] == 0) return;  // merged inside the append kernel
  const int kind = plan[H_KIND];
  const int rows = plan[H_ROWS];
  const int G = plan[H_GROUP];
  const int Tq = plan[H_TILE_Q];
  const int num_merges = plan[H_NUM_MERGES];
  const ABP_CONST_AS int32_t* tiles = plan + plan[H_OFF_TILE];
  const ABP_CONST_AS int32_t* merges = plan + plan[H_OFF_MERGE];
  const int total = num_merges * rows;
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4;  // lane group: partials q, q + 4, q + 8, ...
  const int e0 = (lane & 15) * 8;
  const int nwaves = gridDim.x * 4;
  for (int ri = blockIdx.x * 4 + (threadIdx.x >> 6); ri < total; ri += nwaves) {
    const int m = ri / rows;
    const int r = ri - m * rows;
    const int mtile = merges[4 * m], mfirst = merges[4 * m + 1], n = merges[4 * m + 2];
    const int tb = tiles[4 * mtile], th = tiles[4 * mtile + 1], tq = tiles[4 * mtile + 2];
    int64_t token;
    int head;
    if (kind == ABP_KIND_DECODE) {
      token = tb;
      head = th * G + r;
    } else {
      const int q0 = a.qo_indptr[tb];
      const int qo_len = a.qo_indptr[tb + 1] - q0;
      const int tloc = tq * Tq + r / G;
      if (tloc >= qo_len) continue;  // uniform over the wave
      token = q0 + tloc;
      head = th * G + (r % G);
    }
    float M = kNegInf, tot = 0.f;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int i0 = q; i0 < n; i0 += 16) {
      float l[4], v[4][8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (i0 + 4 * j < n) {
          const int64_t sr = int64_t(mfirst + i0 + 4 * j) * rows + r;
          l[j] = a.lse_part[sr];
          load8<ABP_F32>(a.o_part, sr * 128 + e0, v[j]);
        } else {
          l[j] = kNegInf;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[j][e] = 0.f;
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float nm = __builtin_fmaxf(M, l[j]);
        const float sc = nm == M ? 1.f : fast_exp2((M - nm) * kLog2e);
        const float wt = l[j] == kNegInf ? 0.f : fast_exp2((l[j] - nm) * kLog2e);
        M = nm;
        tot = __builtin_fmaf(tot, sc, wt);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(acc[e], sc, wt * v[j][e]);
      }
    }
    // combine the 4 lane groups (lanes xor 16, xor 32)
    float Mall = __builtin_fmaxf(M, __shfl_xor(M, 16));
    Mall = __builtin_fmaxf(Mall, __shfl_xor(Mall, 32));
    const float f = M == kNegInf ? 0.f : fast_exp2((M - Mall) * kLog2e);
    tot *= f;
    tot += __shfl_xor(tot, 16);
    tot += __shfl_xor(tot, 32);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = acc[e] * f;
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      acc[e] = x;
    }
    if (q != 0) continue;
    float out[8];
    float lse = kNegInf;
    if (Mall != kNegInf) {
      const float inv = 1.f / tot;
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = acc[e] * inv;
      lse = Mall + fast_log2(tot) * kLn2;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = 0.f;
    }
    const int64_t orow = token * a.num_qo_heads + head;
    store8<OUT_DT>(a.o, orow * 128 + e0, out);
    if (a.lse && e0 == 0) a.lse[orow] = lse;
  }
}

// Cascade: the final state of every output row from both levels' states in
// one pass (paper summary "图谱动态｜学苑周刊 NO.266", section 统一的 KV 缓存存储格式:
// a shared-prefix level and a per-request level recombined by their attention
// states). Per level, row (b, head) has either one state in the level's output
// (fp32; an unsplit tile, or a tile the append kernel merged itself) or the
// partial slots of its split tile; all of them are folded with a running
// maximum in the level order of the partial slots, prefix first. One wave per
// row: its 4 groups of 16 lanes fold every 4th state (8 head dims per lane),
// then combine by lane exchange.
struct LevelRow {
  const float* o;    // first state's row (128 floats)
  const float* lse;  // first state's lse
  int64_t so, sl;    // strides between states (floats)
  int n;             // number of states
};

__device__ __forceinline__ LevelRow level_row(const AttnArgs& a, int tile, int r, int64_t orow) {
  const ABP_CONST_AS int32_t* plan = const_as(a.plan);
  const int np = plan[plan[H_OFF_NTILE] + tile];
  LevelRow L;
  if (np == 0 || plan[H_MERGE_KERNEL] == 0) {
    L.o = static_cast<const float*>(a.o) + orow * 128;
    L.lse = a.lse + orow;
    L.so = 0;
    L.sl = 0;
    L.n = 1;
  } else {
    const int rows = plan[H_ROWS];
    const int64_t first = plan[plan[H_OFF_TILE] + 4 * tile + 3];
    L.o = a.o_part + (first * rows + r) * 128;
    L.lse = a.lse_part + first * rows + r;
    L.so = int64_t(rows) * 128;
    L.sl = rows;
    L.n = np;
  }
  return L;
}

template <int OUT_DT>
__global__ __launch_bounds__(256) void cascade_merge_kernel(AttnArgs pre, AttnArgs suf, int batch,
                                                            void* o, float* lse) {
  const ABP_CONST_AS int32_t* pplan = const_as(pre.plan);
  const ABP_CONST_AS int32_t* splan = const_as(suf.plan);
  const int hq = suf.num_qo_heads;
  const int G = splan[H_GROUP];
  const int hkv = hq / G;
  const int hpt_s = splan[H_TILE_HEADS], hpt_p = pplan[H_TILE_HEADS];
  const int tq = pplan[H_TILE_Q];
  const int nqt = (batch + tq - 1) / tq;
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4;
  const int e0 = (lane & 15) * 8;
  const int total = batch * hq;
  const int nwaves = gridDim.x * 4;
  for (int row = blockIdx.x * 4 + (threadIdx.x >> 6); row < total; row += nwaves) {
    const int b = row / hq, head = row - b * hq;
    const int hk = head / G, g = head - hk * G;
    // prefix: one request whose query tokens are the batch's queries; tiles
    // in kv-head-group order, then query tiles. suffix: tiles in request order,
    // then kv-head groups.
    const LevelRow P = level_row(pre, (hk / hpt_p) * nqt + b / tq,
                                 ((b % tq) * hpt_p + hk % hpt_p) * G + g, row);
    const LevelRow S = level_row(suf, b * (hkv / hpt_s) + hk / hpt_s, (hk % hpt_s) * G + g, row);
    const int n = P.n + S.n;
    float M = kNegInf, tot = 0.f;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int i0 = q; i0 < n; i0 += 16) {
      float l[4], v[4][8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = i0 + 4 * j;
        if (i < n) {
          const bool pi = i < P.n;
          const int k = pi ? i : i - P.n;
          const LevelRow& X = pi ? P : S;
          l[j] = X.lse[k * X.sl];
          load8<ABP_F32>(X.o, k * X.so + e0, v[j]);
        } else {
          l[j] = kNegInf;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[j][e] = 0.f;
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float nm = __builtin_fmaxf(M, l[j]);
        const float sc = nm == M ? 1.f : fast_exp2((M - nm) * kLog2e);
        const float wt = l[j] == kNegInf ? 0.f : fast_exp2((l[j] - nm) * kLog2e);
        M = nm;
        tot = __builtin_fmaf(tot, sc, wt);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(acc[e], sc, wt * v[j][e]);
      }
    }
    float Mall = __builtin_fmaxf(M, __shfl_xor(M, 16));
    Mall = __builtin_fmaxf(Mall, __shfl_xor(Mall, 32));
    const float f = M == kNegInf ? 0.f : fast_exp2((M - Mall) * kLog2e);
    tot *= f;
    tot += __shfl_xor(tot, 16);
    tot += __shfl_xor(tot, 32);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = acc[e] * f;
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      acc[e] = x;
    }
    if (q != 0) continue;
    float out[8];
    float lse_r = kNegInf;
    if (Mall != kNegInf) {
      const float inv = 1.f / tot;
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = acc[e] * inv;
      lse_r = Mall + fast_log2(tot) * kLn2;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = 0.f;
    }
    store8<OUT_DT>(o, int64_t(row) * 128 + e0, out);
    if (lse && e0 == 0) lse[row] = lse_r;
  }
}

template <int IN_DT>
hipError_t merge_two_out(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                         void* o_out, float* lse_out, int64_t rows, int out_dtype,
                         hipStream_t s) {
  const dim3 grid((unsigned)((rows + 15) / 16));
  if (out_dtype == ABP_F32)
    merge_two_kernel<IN_DT, ABP_F32><<<grid, 256, 0, s>>>(o_a, lse_a, o_b, lse_b, rows, o_out, lse_out);
  else if (out_dtype == ABP_BF16)
    merge_two_kernel<IN_DT, ABP_BF16><<<grid, 256, 0, s>>>(o_a, lse_a, o_b, lse_b, rows, o_out, lse_out);
  else
    merge_two_kernel<IN_DT, ABP_F16><<<grid, 256, 0, s>>>(o_a, lse_a, o_b, lse_b, rows, o_out, lse_out);
  return hipGetLastError();
}

template <int IN_DT>
hipError_t merge_states_out(const void* o_in, const float* lse_in, int32_t n, int64_t rows,
                            int out_dtype, void* o_out, float* lse_out, hipStream_t s) {
  const dim3 grid((unsigned)((rows + 15) / 16));
  if (out_dtype == ABP_F32)
    merge_states_kernel<IN_DT, ABP_F32><<<grid, 256, 0, s>>>(o_in, lse_in, n, rows, o_out, lse_out);
  else if (out_dtype == ABP_BF16)
    merge_states_kernel<IN_DT, ABP_BF16><<<grid, 256, 0, s>>>(o_in, lse_in, n, rows, o_out, lse_out);
  else
    merge_states_kernel<IN_DT, ABP_F16><<<grid, 256, 0, s>>>(o_in, lse_in, n, rows, o_out, lse_out);
  return hipGetLastError();
}

}  // namespace


hipError_t launch_merge_two(const void* o_a, const float* lse_a, const void* o_b,
                            const float* lse_b, void* o_out, float* lse_out, int64_t rows,
                            int in_dtype, int out_dtype, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (in_dtype == ABP_F32)
    return merge_two_out<ABP_F32>(o_a, lse_a, o_b, lse_b, o_out, lse_out, rows, out_dtype, s);
  if (in_dtype == ABP_BF16)
    return merge_two_out<ABP_BF16>(o_a, lse_a, o_b, lse_b, o_out, lse_out, rows, out_dtype, s);
  return merge_two_out<ABP_F16>(o_a, lse_a, o_b, lse_b, o_out, lse_out, rows, out_dtype, s);
}

hipError_t launch_merge_states(const void* o_in, const float* lse_in, int32_t n, int64_t rows,
                               int in_dtype, int out_dtype, void* o_out, float* lse_out,
                               hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (in_dtype == ABP_F32)
    return merge_states_out<ABP_F32>(o_in, lse_in, n, rows, out_dtype, o_out, lse_out, s);
  if (in_dtype == ABP_BF16)
    return merge_states_out<ABP_BF16>(o_in, lse_in, n, rows, out_dtype, o_out, lse_out, s);
  return merge_states_out<ABP_F16>(o_in, lse_in, n, rows, out_dtype, o_out, lse_out, s);
}

hipError_t launch_cascade_merge(const AttnArgs& pre, const AttnArgs& suf, int32_t batch,
                                void* o, float* lse, int out_dtype, hipStream_t s) {
  const int64_t rows = int64_t(batch) * suf.num_qo_heads;
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (out_dtype == ABP_F32)
    cascade_merge_kernel<ABP_F32><<<grid, 256, 0, s>>>(pre, suf, batch, o, lse);
  else if (out_dtype == ABP_BF16)
    cascade_merge_kernel<ABP_BF16><<<grid, 256, 0, s>>>(pre, suf, batch, o, lse);
  else
    cascade_merge_kernel<ABP_F16><<<grid, 256, 0, s>>>(pre, suf, batch, o, lse);
  return hipGetLastError();
}

hipError_t launch_plan_merge(const Config& cfg, const AttnArgs& a, int32_t grid, hipStream_t s) {
  if (cfg.out_dtype == ABP_F32)
    plan_merge_kernel<ABP_F32><<<grid, 256, 0, s>>>(a);
  else if (cfg.out_dtype == ABP_BF16)
    plan_merge_kernel<ABP_BF16><<<grid, 256, 0, s>>>(a);
  else
    plan_merge_kernel<ABP_F16><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace abp
