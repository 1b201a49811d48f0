// Persistent batch decode over a paged block-sparse-row KV cache (gfx950).
//
// What it computes: for each request b and qo head, exact softmax attention of
// the one query token over the request's keys, read through its page table
// (paper summary "图谱动态｜学苑周刊 NO.266", section 统一的 KV 缓存存储格式;
// single and batch decode kernels of "FlashInfer 源码级解读"). Decode reads
// every K/V byte once and does ~4 flop per byte at a GQA group of 4, so it is
// bound by HBM bandwidth; the design goal is to keep enough bytes in flight.
//
// Work split: the host planner cuts the (request, kv head) tiles into segments
// of whole 64-key blocks spread evenly over a fixed grid of workers (section
// 动态负载均衡调度); one 256-thread workgroup is one worker and walks its
// segments in order.
//
// Inside a segment the 4 waves take 16-token chunks round-robin. In a chunk,
// lane (grp = lane / 16, sub = lane % 16) holds head-dim elements
// [8 sub, 8 sub + 8) of tokens c + 4 i + grp for i = 0..3: each load
// instruction reads 4 contiguous 256-byte head rows (coalesced 128-bit
// lanes). All G query rows of the kv head (the GQA group) are kept in every
// lane, so one K/V read serves the whole group:
//   * q.k uses dot2 (bf16/fp16 pairs, fp32 accumulate) and a 16-lane DPP sum;
//   * online softmax in fp32 with base-2 exponentials, one running max per
//     (row, token group);
//   * p.v uses dot2 over token pairs: p of tokens (i, i+1) packed as a pair
//     against V elements of the same two tokens repacked with v_perm.
// Chunks are double-buffered in registers so the next chunk's loads are in
// flight while the current one is computed. At the end of a segment the
// states of the 4 token groups and 4 waves are merged, and the tile's rows
// are written either as the final o / lse or as an fp32 partial state.
#include "common.h"
#include "kernels.h"
#include "layout.h"

namespace abp {

namespace {

constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kChunk = 16;           // tokens per wave step
constexpr int kStep = kWaves * kChunk;

struct KVRegs {
  uint4 k[4];
  uint4 v[4];
};

__device__ __forceinline__ uint32_t word(const uint4& u, int j) {
  return j == 0 ? u.x : j == 1 ? u.y : j == 2 ? u.z : u.w;
}
__device__ __forceinline__ void set_word(uint4& u, int j, uint32_t v) {
  if (j == 0) u.x = v;
  else if (j == 1) u.y = v;
  else if (j == 2) u.z = v;
  else u.w = v;
}

// Rotate this lane's 8 elements (pairs (j, j + 64) split across lanes sub and
// sub ^ 8) at position `pos`. All lanes of the wave must call it together.
template <typename T>
__device__ __forceinline__ void rope_rotate8(uint4& u, float pos, const float* fhi,
                                             const float* flo, bool hi_half) {
  uint32_t w[4], pw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    w[j] = word(u, j);
    pw[j] = dpp_u<kDppRor8>(w[j]);
  }
  float out[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float own = (e & 1) ? hi_f32<T>(w[e >> 1]) : lo_f32<T>(w[e >> 1]);
    const float par = (e & 1) ? hi_f32<T>(pw[e >> 1]) : lo_f32<T>(pw[e >> 1]);
    float sn, cs;
    rope_sincos(pos, fhi[e], flo[e], &sn, &cs);
    out[e] = __builtin_fmaf(par, hi_half ? sn : -sn, own * cs);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) set_word(u, j, pack2<T>(out[2 * j], out[2 * j + 1]));
}

__device__ __forceinline__ void store8_dt(void* base, int64_t off, const float v[8], int dt) {
  if (dt == ABP_F32) store8<ABP_F32>(base, off, v);
  else if (dt == ABP_BF16) store8<ABP_BF16>(base, off, v);
  else store8<ABP_F16>(base, off, v);
}

template <typename T, int G, bool ROPE>
__global__ __launch_bounds__(256, 2) void decode_kernel(AttnArgs a) {
  const int32_t* plan = a.plan;
  const int32_t* wseg = plan + plan[H_OFF_WSEG];
  const int4* segs = reinterpret_cast<const int4*>(plan + plan[H_OFF_SEG]);
  const int4* tiles = reinterpret_cast<const int4*>(plan + plan[H_OFF_TILE]);
  const int s_begin = wseg[blockIdx.x], s_end = wseg[blockIdx.x + 1];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int grp = lane >> 4;
  const int sub = lane & 15;
  const bool hi_half = sub >= 8;
  const float cl2 = a.sm_scale_log2;

  const uint16_t* __restrict__ kp = static_cast<const uint16_t*>(a.k_pages);
  const uint16_t* __restrict__ vp = static_cast<const uint16_t*>(a.v_pages);
  const int P = a.page_size;
  const int shift = a.page_shift;

  __shared__ float s_o[kWaves][G][kD];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];

  float fhi[8], flo[8];
  if constexpr (ROPE) {
    const float* rope = reinterpret_cast<const float*>(plan + plan[H_OFF_ROPE]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = (sub & 7) * 8 + e;
      fhi[e] = rope[2 * j];
      flo[e] = rope[2 * j + 1];
    }
  }

  for (int s = s_begin; s < s_end; ++s) {
    const int4 sg = segs[s];
    const int4 tl = tiles[sg.x];
    const int b = tl.x, h = tl.y;
    const int kv_begin = sg.y, kv_end = sg.z, slot = sg.w;
    const int ip0 = a.kv_indptr[b];
    const int64_t head_off = int64_t(h) * kD + sub * 8;

    // ---- q of the G rows of this kv head: words of elements [8 sub, 8 sub + 8)
    uint4 qv[G];
    {
      const uint16_t* qb = static_cast<const uint16_t*>(a.q) +
                           (int64_t(b) * a.num_qo_heads + int64_t(h) * G) * kD + sub * 8;
#pragma unroll
      for (int g = 0; g < G; ++g) qv[g] = *reinterpret_cast<const uint4*>(qb + g * kD);
    }
    float kv_pos0 = 0.f;
    if constexpr (ROPE) {
      const int n = a.kv_indptr[b + 1] - ip0;
      const int kv_len = n > 0 ? (n - 1) * P + a.kv_last_page_len[b] : 0;
      const int qpos = a.q_pos ? a.q_pos[b] : kv_len - 1;
      kv_pos0 = a.kv_pos_offset ? (float)a.kv_pos_offset[b] : 0.f;
#pragma unroll
      for (int g = 0; g < G; ++g) rope_rotate8<T>(qv[g], (float)qpos, fhi, flo, hi_half);
    }

    float m[G], l[G], o[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = kNegInf;
      l[g] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[g][e] = 0.f;
    }

    auto load_chunk = [&](KVRegs& X, int c) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = min(c + 4 * i + grp, kv_end - 1);
        int page, off;
        if (shift >= 0) {
          page = tok >> shift;
          off = tok & (P - 1);
        } else {
          page = tok / P;
          off = tok - page * P;
        }
        const int64_t pid = a.kv_indices[ip0 + page];
        const int64_t base = pid * a.page_stride + int64_t(off) * a.token_stride + head_off;
        X.k[i] = *reinterpret_cast<const uint4*>(kp + base);
        X.v[i] = *reinterpret_cast<const uint4*>(vp + base);
      }
    };

    auto compute_chunk = [&](KVRegs& X, int c) {
      if constexpr (ROPE) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          rope_rotate8<T>(X.k[i], kv_pos0 + (float)(c + 4 * i + grp), fhi, flo, hi_half);
      }
      // scores of 4 tokens x G rows, summed over the 16 lanes of the token's row
      float sc[4][G];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float acc = dot2<T>(qv[g].x, X.k[i].x, 0.f);
          acc = dot2<T>(qv[g].y, X.k[i].y, acc);
          acc = dot2<T>(qv[g].z, X.k[i].z, acc);
          acc = dot2<T>(qv[g].w, X.k[i].w, acc);
          sc[i][g] = row16_sum(acc);
        }
        if (c + 4 * i + grp >= kv_end) {
#pragma unroll
          for (int g = 0; g < G; ++g) sc[i][g] = kNegInf;
        }
      }
      // online softmax (per row, per token group) and p packed as token pairs
      uint32_t pp[2][G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float mx = __builtin_fmaxf(__builtin_fmaxf(sc[0][g], sc[1][g]),
                                         __builtin_fmaxf(sc[2][g], sc[3][g]));
        const float mn = __builtin_fmaxf(m[g], mx);
        const float mu = mn == kNegInf ? 0.f : mn;
        const float alpha = fast_exp2((m[g] - mu) * cl2);
        const float mc = mu * cl2;
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = fast_exp2(__builtin_fmaf(sc[i][g], cl2, -mc));
        l[g] = __builtin_fmaf(l[g], alpha, (p[0] + p[1]) + (p[2] + p[3]));
        m[g] = mn;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[g][e] *= alpha;
        pp[0][g] = pack2<T>(p[0], p[1]);
        pp[1][g] = pack2<T>(p[2], p[3]);
      }
      // o += p . v over token pairs (0, 1) and (2, 3)
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t va = word(X.v[2 * pr], j), vb = word(X.v[2 * pr + 1], j);
          const uint32_t vlo = pair_lo(va, vb);  // element 2j of both tokens
          const uint32_t vhi = pair_hi(va, vb);  // element 2j + 1
#pragma unroll
          for (int g = 0; g < G; ++g) {
            o[g][2 * j] = dot2<T>(pp[pr][g], vlo, o[g][2 * j]);
            o[g][2 * j + 1] = dot2<T>(pp[pr][g], vhi, o[g][2 * j + 1]);
          }
        }
      }
    };

    // ---- main loop: double-buffered chunks, this wave's chunks every kStep keys
    {
      KVRegs A, B;
      int c = kv_begin + wave * kChunk;
      if (c < kv_end) load_chunk(A, c);
      while (c < kv_end) {
        if (c + kStep < kv_end) load_chunk(B, c + kStep);
        compute_chunk(A, c);
        c += kStep;
        if (c >= kv_end) break;
        if (c + kStep < kv_end) load_chunk(A, c + kStep);
        compute_chunk(B, c);
        c += kStep;
      }
    }

    // ---- merge the 4 token groups of this wave (lanes xor 16, xor 32)
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float M = __builtin_fmaxf(m[g], __shfl_xor(m[g], 16));
      M = __builtin_fmaxf(M, __shfl_xor(M, 32));
      const float Mu = M == kNegInf ? 0.f : M;
      const float f = fast_exp2((m[g] - Mu) * cl2);
      float lg = l[g] * f;
      lg += __shfl_xor(lg, 16);
      lg += __shfl_xor(lg, 32);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = o[g][e] * f;
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        o[g][e] = v;
      }
      m[g] = M;
      l[g] = lg;
    }
    if (grp == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int e = 0; e < 8; ++e) s_o[wave][g][sub * 8 + e] = o[g][e];
        if (sub == 0) {
          s_m[wave][g] = m[g];
          s_l[wave][g] = l[g];
        }
      }
    }
    __syncthreads();

    // ---- merge the 4 waves and write the tile's G rows
    if (threadIdx.x < G * 16) {
      const int g = threadIdx.x >> 4;
      const int e0 = (threadIdx.x & 15) * 8;
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = __builtin_fmaxf(M, s_m[w][g]);
      float out[8];
      float lse = kNegInf;
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = 0.f;
      if (M != kNegInf) {
        float L = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float f = fast_exp2((s_m[w][g] - M) * cl2);
          L = __builtin_fmaf(f, s_l[w][g], L);
#pragma unroll
          for (int e = 0; e < 8; ++e) out[e] = __builtin_fmaf(f, s_o[w][g][e0 + e], out[e]);
        }
        const float inv = 1.f / L;
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] *= inv;
        lse = M * a.sm_scale + fast_log2(L) * kLn2;
      }
      if (slot < 0) {
        const int64_t row = int64_t(b) * a.num_qo_heads + int64_t(h) * G + g;
        store8_dt(a.o, row * kD + e0, out, a.out_dtype);
        if (a.lse && e0 == 0) a.lse[row] = lse;
      } else {
        const int64_t row = int64_t(slot) * G + g;
        store8<ABP_F32>(a.o_part, row * kD + e0, out);
        if (e0 == 0) a.lse_part[row] = lse;
      }
    }
    __syncthreads();
  }
}

template <typename T, int G>
hipError_t launch_g(const Config& cfg, const AttnArgs& a, hipStream_t s) {
  if (cfg.rope)
    decode_kernel<T, G, true><<<a.workers, 256, 0, s>>>(a);
  else
    decode_kernel<T, G, false><<<a.workers, 256, 0, s>>>(a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const Config& cfg, const AttnArgs& a, hipStream_t s) {
  switch (cfg.group) {
    case 1: return launch_g<T, 1>(cfg, a, s);
    case 2: return launch_g<T, 2>(cfg, a, s);
    case 4: return launch_g<T, 4>(cfg, a, s);
    case 8: return launch_g<T, 8>(cfg, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const Config& cfg, const AttnArgs& a, hipStream_t s) {
  if (cfg.qkv_dtype == ABP_BF16) return launch_t<BF16>(cfg, a, s);
  return launch_t<F16>(cfg, a, s);
}

}  // namespace abp
