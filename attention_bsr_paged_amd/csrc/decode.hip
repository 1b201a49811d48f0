// Persistent batch decode over a paged block-sparse-row KV cache (gfx950).
//
// What it computes: for each request b and qo head, exact softmax attention of
// the one query token over the request's keys, read through its page table
// (paper summary "图谱动态｜学苑周刊 NO.266", section 统一的 KV 缓存存储格式;
// single and batch decode kernels of "FlashInfer 源码级解读"). Decode reads
// every K/V byte once and does ~4 flop per byte at a GQA group of 4, so it is
// bound by HBM bandwidth; the design goal is to keep enough bytes in flight
// while spending few instructions per byte.
//
// Work split: the host planner cuts the (request, kv-head group) tiles into
// segments of whole 64-key blocks spread evenly over a fixed grid of workers
// (section 动态负载均衡调度); one 256-thread workgroup is one worker and walks
// its segments in order. When the kv head count is a multiple of 4, a tile
// holds 4 consecutive kv heads and each wave takes one of them: the workgroup
// then reads 1 KB runs of every token row together (4 heads x 256 bytes), which
// the HBM serves faster than 256-byte pieces at the token stride, and each
// wave owns its head's state, so no workgroup barrier is needed. Otherwise a
// tile is one head and the 4 waves take its 16-token chunks round-robin.
//
// In a chunk,
// lane (grp = lane / 16, sub = lane % 16) holds head-dim elements
// [8 sub, 8 sub + 8) of tokens c + 4 i + grp for i = 0..3: each load
// instruction reads 4 whole 256-byte head rows (coalesced 128-bit lanes). All
// G query rows of the kv head (the GQA group) are kept in every lane, so one
// K/V read serves the whole group:
//   * q.k uses dot2 (bf16/fp16 pairs, fp32 accumulate) and 16-lane DPP sums,
//     done step by step over all 4 G values so no DPP hazard stalls remain;
//   * online softmax in fp32 with base-2 exponentials, one running max per
//     (row, token group), rescaled lazily: the reference max only moves when a
//     score exceeds it by more than 2^8 in probability, so most chunks skip the
//     rescale of o (exact: the final normalisation uses the same reference);
//   * p.v uses dot2 over token pairs: p of tokens (i, i+1) packed as a pair
//     against V elements of the same two tokens repacked with v_perm.
// When the page size is a power of two and a multiple of 16, a 16-token chunk
// never straddles a page: its page id is one scalar load (issued a chunk
// ahead) and all K/V addresses are a uniform page base plus fixed per-lane
// offsets. Other page sizes translate every token.
// With an fp8 (OCP e4m3) KV cache a lane loads the same 8 elements as 8 bytes
// and turns each byte pair into the 16-bit pair layout above with one gfx950
// conversion (exact: every e4m3 value is a bf16 and an fp16 value), so the
// arithmetic is the 16-bit path's; k_scale is folded into the logit scale and
// v_scale into the final normalisation.
// Chunks are double-buffered in registers. At the end of a segment the states
// of the 4 token groups (and of the waves sharing a head) are merged, and the
// tile's rows are written either as the final o / lse or as an fp32 partial
// state.
#include "common.h"
#include "kernels.h"
#include "layout.h"

namespace abp {

namespace {

constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kSub = 16;             // tokens per sub-chunk (4 load instructions)
constexpr float kRescaleLog2 = 8.f;  // lazy rescale threshold (log2 of the max p)

template <int S, bool KV8>
struct KVRegs {  // S sub-chunks of 16 tokens; 8 elements per lane and row
  using W = typename std::conditional<KV8, uint2, uint4>::type;
  W k[4 * S];
  W v[4 * S];
};

// two e4m3 codes (byte pair HI of w) as a 16-bit pair of the query's type
template <typename T, bool HI>
__device__ __forceinline__ uint32_t fp8x2(uint32_t w);
template <>
__device__ __forceinline__ uint32_t fp8x2<BF16, false>(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, false));
}
template <>
__device__ __forceinline__ uint32_t fp8x2<BF16, true>(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, true));
}
template <>
__device__ __forceinline__ uint32_t fp8x2<F16, false>(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.f, false));
}
template <>
__device__ __forceinline__ uint32_t fp8x2<F16, true>(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.f, true));
}

// 8 elements of a row as 4 words of 16-bit pairs
template <typename T>
__device__ __forceinline__ uint4 widen8(const uint4& u) {
  return u;
}
template <typename T>
__device__ __forceinline__ uint4 widen8(const uint2& u) {
  return make_uint4(fp8x2<T, false>(u.x), fp8x2<T, true>(u.x), fp8x2<T, false>(u.y),
                    fp8x2<T, true>(u.y));
}

__device__ __forceinline__ uint32_t word(const uint4& u, int j) {
  return j == 0 ? u.x : j == 1 ? u.y : j == 2 ? u.z : u.w;
}
__device__ __forceinline__ void set_word(uint4& u, int j, uint32_t v) {
  if (j == 0) u.x = v;
  else if (j == 1) u.y = v;
  else if (j == 2) u.z = v;
  else u.w = v;
}

// RoPE (rotate-half): element j pairs with j + 64. With RoPE on, a lane's K
// (and q) register holds elements [4 sub, 4 sub + 4) in words 0-1 and
// [64 + 4 sub, 64 + 4 sub + 4) in words 2-3, so both halves of its 4 pairs are
// local and each angle is needed by one lane only. Rotate them by the angles
// whose cosines and sines are cs / sn, into fp32: rounding the rotated values
// back to 16 bits would put ~1e-3 of noise on every logit, which short key
// ranges do not average out.
template <typename T>
__device__ __forceinline__ void rope_rotate_pairs(const uint4& u, const float cs[4],
                                                  const float sn[4], float out[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t wl = (e < 2) ? u.x : u.y;
    const uint32_t wh = (e < 2) ? u.z : u.w;
    const float x = (e & 1) ? hi_f32<T>(wl) : lo_f32<T>(wl);
    const float y = (e & 1) ? hi_f32<T>(wh) : lo_f32<T>(wh);
    out[e] = __builtin_fmaf(-y, sn[e], x * cs[e]);
    out[4 + e] = __builtin_fmaf(x, sn[e], y * cs[e]);
  }
}

// Interleaved RoPE: word w of the lane's 8 elements is the adjacent pair
// (2w, 2w + 1) of its 4 pairs; rotate each by cs[w] / sn[w] into fp32.
template <typename T>
__device__ __forceinline__ void rope_rotate_adjacent(const uint4& u, const float cs[4],
                                                     const float sn[4], float out[8]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t wd = w == 0 ? u.x : w == 1 ? u.y : w == 2 ? u.z : u.w;
    const float x = lo_f32<T>(wd), y = hi_f32<T>(wd);
    out[2 * w] = __builtin_fmaf(-y, sn[w], x * cs[w]);
    out[2 * w + 1] = __builtin_fmaf(x, sn[w], y * cs[w]);
  }
}

template <typename T, bool RIL>
__device__ __forceinline__ void rope_rot(const uint4& u, const float cs[4], const float sn[4],
                                         float out[8]) {
  if constexpr (RIL) rope_rotate_adjacent<T>(u, cs, sn, out);
  else rope_rotate_pairs<T>(u, cs, sn, out);
}

__device__ __forceinline__ void store8_dt(void* base, int64_t off, const float v[8], int dt) {
  if (dt == ABP_F32) store8<ABP_F32>(base, off, v);
  else if (dt == ABP_BF16) store8<ABP_BF16>(base, off, v);
  else store8<ABP_F16>(base, off, v);
}

template <int N>
__device__ __forceinline__ void row16_sum_all(float* x) {
#pragma unroll
  for (int n = 0; n < N; ++n) x[n] += dpp<kDppXor1>(x[n]);
#pragma unroll
  for (int n = 0; n < N; ++n) x[n] += dpp<kDppXor2>(x[n]);
#pragma unroll
  for (int n = 0; n < N; ++n) x[n] += dpp<kDppHalfMirror>(x[n]);
#pragma unroll
  for (int n = 0; n < N; ++n) x[n] += dpp<kDppMirror>(x[n]);
}

template <typename T, int G, bool ROPE, bool FASTPAGE, int S, int HT, bool KV8, bool RIL>
__global__ __launch_bounds__(256, 2) void decode_kernel(AttnArgs a) {
  static_assert(!(KV8 && ROPE), "fp8 KV pages are read without RoPE");
  static_assert(ROPE || !RIL, "interleaving is a RoPE layout");
  using KE = typename std::conditional<KV8, uint8_t, uint16_t>::type;  // K/V element
  using KW = typename KVRegs<1, KV8>::W;  // 8 elements of a K/V row
  constexpr uint32_t kEsz = sizeof(KE);
  constexpr int TW = kWaves / HT;     // waves per kv head (they split its keys)
  constexpr int kChunk = kSub * S;    // tokens per wave per buffered chunk
  constexpr int kStep = TW * kChunk;  // tokens per step of one head
  const ABP_CONST_AS int32_t* plan = const_as(a.plan);
  const ABP_CONST_AS int32_t* wseg = plan + plan[H_OFF_WSEG];
  const ABP_CONST_AS int32_t* segs = plan + plan[H_OFF_SEG];    // 4 ints per record
  const ABP_CONST_AS int32_t* tiles = plan + plan[H_OFF_TILE];
  const ABP_CONST_AS int32_t* kv_indptr = const_as(a.kv_indptr);
  const ABP_CONST_AS int32_t* kv_indices = const_as(a.kv_indices);
  const int s_begin = wseg[blockIdx.x], s_end = wseg[blockIdx.x + 1];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane >> 4;
  const int sub = lane & 15;
  const int hw = wave % HT;  // this wave's kv head within the tile
  const int tw = wave / HT;  // this wave's share of the head's keys
  const float cl2 = a.sm_scale_log2;
  const float thr = kRescaleLog2 / cl2;  // threshold in raw score units

  const KE* __restrict__ kp = static_cast<const KE*>(a.k_pages);
  const KE* __restrict__ vp = static_cast<const KE*>(a.v_pages);
  const int P = a.page_size;
  const int shift = a.page_shift;
  const int tstride = a.token_stride;

  // cross-wave merge of a head's key shares (only when TW > 1)
  __shared__ float s_o[TW > 1 ? kWaves : 1][G][kD];
  __shared__ float s_m[TW > 1 ? kWaves : 1][G];
  __shared__ float s_l[TW > 1 ? kWaves : 1][G];

  // RoPE: frequencies (revolutions per position, split hi + lo) of this lane's
  // 4 pairs j = 4 sub + e (rotate-half: elements 4 sub + e and 64 + 4 sub + e;
  // interleaved: elements 8 sub + 2e and 8 sub + 2e + 1, the lane's plain 8), and the rotation by 4 positions (c4, s4): a lane's
  // tokens in a sub-chunk are 4 apart, so only the first one's angles are
  // evaluated and the next three follow by angle addition
  float fhi[ROPE ? 4 : 1], flo[ROPE ? 4 : 1], c4[ROPE ? 4 : 1], s4[ROPE ? 4 : 1];
  if constexpr (ROPE) {
    const ABP_CONST_AS float* rope = (const ABP_CONST_AS float*)(plan + plan[H_OFF_ROPE]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = 4 * sub + e;
      fhi[e] = rope[2 * j];
      flo[e] = rope[2 * j + 1];
      rope_sincos(4.f, fhi[e], flo[e], &s4[e], &c4[e]);
    }
  }
  // byte offset of this lane's K words from its V words (RoPE layout above)
  const uint32_t kdel = (ROPE && !RIL) ? 8u * sub : 0u;
  auto load_k = [&](const char* p) -> KW {
    if constexpr (ROPE && !RIL) {
      const uint2 lo = load_once(reinterpret_cast<const uint2*>(p));
      const uint2 hi = load_once(reinterpret_cast<const uint2*>(p + 128));
      return make_uint4(lo.x, lo.y, hi.x, hi.y);
    } else {
      return load_once(reinterpret_cast<const KW*>(p));
    }
  };

  // Chunk buffers, page ids and q live across segments: on the page-aligned
  // path the end of a segment's chunk loop issues the loads of the next
  // segment (q, page ids, first chunk), so they are in flight while the
  // segment's states are merged and written.
  KVRegs<S, KV8> A, B;
  int pidA[S] = {}, pidB[S] = {};
  uint4 qn[G];
  bool pre = false;  // the loads of segment s were issued by segment s - 1
  auto load_q = [&](int b, int h, uint4* q) {
    const uint16_t* qb = static_cast<const uint16_t*>(a.q) +
                         (int64_t(b) * a.num_qo_heads + int64_t(h) * G) * kD + sub * 8;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if constexpr (ROPE) q[g] = load_k(reinterpret_cast<const char*>(qb + g * kD) - kdel);
      else q[g] = *reinterpret_cast<const uint4*>(qb + g * kD);
    }
  };

  for (int s = s_begin; s < s_end; ++s) {
    const int tile = segs[4 * s];
    const int kv_begin = segs[4 * s + 1], kv_end = segs[4 * s + 2], slot = segs[4 * s + 3];
    const int b = tiles[4 * tile], h = tiles[4 * tile + 1] + hw;
    const int ip0 = kv_indptr[b];
    const int head_off = h * kD + sub * 8;

    // ---- q of the G rows of this kv head: words of elements [8 sub, 8 sub + 8)
    uint4 qv[G];
    if (pre) {
#pragma unroll
      for (int g = 0; g < G; ++g) qv[g] = qn[g];
    } else {
      load_q(b, h, qv);
    }
    // Consume q here so its load is waited for before the chunk loop; else the
    // loop's first use of q waits for every load in flight (the next chunk too).
#pragma unroll
    for (int g = 0; g < G; ++g)
      asm volatile("" : "+v"(qv[g].x), "+v"(qv[g].y), "+v"(qv[g].z), "+v"(qv[g].w));
    float kv_pos0 = 0.f;
    float qr[ROPE ? G : 1][8];  // rotated q in fp32 (RoPE only)
    if constexpr (ROPE) {
      const int n = kv_indptr[b + 1] - ip0;
      const int kv_len = n > 0 ? (n - 1) * P + a.kv_last_page_len[b] : 0;
      const int qpos = a.q_pos ? a.q_pos[b] : kv_len - 1;
      kv_pos0 = a.kv_pos_offset ? (float)a.kv_pos_offset[b] : 0.f;
      float cs[4], sn[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) rope_sincos((float)qpos, fhi[e], flo[e], &sn[e], &cs[e]);
#pragma unroll
      for (int g = 0; g < G; ++g) rope_rot<T, RIL>(qv[g], cs, sn, qr[g]);
    }

    float m[G], l[G], o[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = kNegInf;
      l[g] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[g][e] = 0.f;
    }

    // per-lane byte offsets of the 4 token rows of a sub-chunk (fast path)
    uint32_t lane_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) lane_off[i] = uint32_t((4 * i + grp) * tstride + head_off) * kEsz;

    // fast path: one scalar page-table load per sub-chunk, issued a chunk ahead
    // of its use. A sub-chunk that starts past kv_end re-reads the chunk's
    // first sub-chunk (in bounds, cached, fully masked).
    auto chunk_pids = [&](int c, int* pid) {
#pragma unroll
      for (int u = 0; u < S; ++u) {
        const int cu = c + kSub * u < kv_end ? c + kSub * u : c;
        pid[u] = kv_indices[ip0 + (cu >> shift)];
      }
    };

    auto load_chunk = [&](KVRegs<S, KV8>& X, int c, const int* pid) {
#pragma unroll
      for (int u = 0; u < S; ++u) {
        if constexpr (FASTPAGE) {
          const int cu = c + kSub * u < kv_end ? c + kSub * u : c;
          const int64_t base = int64_t(pid[u]) * a.page_stride + int64_t(cu & (P - 1)) * tstride;
          const char* kb = reinterpret_cast<const char*>(kp + base);
          const char* vb = reinterpret_cast<const char*>(vp + base);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            X.k[4 * u + i] = load_k(kb + lane_off[i] - kdel);
            X.v[4 * u + i] = load_once(reinterpret_cast<const KW*>(vb + lane_off[i]));
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tok = min(c + kSub * u + 4 * i + grp, kv_end - 1);
            int page, off;
            if (shift >= 0) {
              page = tok >> shift;
              off = tok & (P - 1);
            } else {
              page = tok / P;
              off = tok - page * P;
            }
            const int64_t pg = a.kv_indices[ip0 + page];  // per-lane (vector) load
            const int64_t at = pg * a.page_stride + int64_t(off) * tstride + head_off;
            X.k[4 * u + i] = load_k(reinterpret_cast<const char*>(kp + at) - kdel);
            X.v[4 * u + i] = load_once(reinterpret_cast<const KW*>(vp + at));
          }
        }
      }
    };

    // one 16-token sub-chunk starting at token c (registers k4[4], v4[4])
    auto compute_sub = [&](const KW* k4w, const KW* v4w, int c) {
      // 16-bit pairs of the 4 K and V rows (fp8 pages are widened here)
      uint4 k4[4], v4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        k4[i] = widen8<T>(k4w[i]);
        v4[i] = widen8<T>(v4w[i]);
      }
      // tokens at or past kv_end were read from slots that may hold no token
      // (NaN or inf bits); their p is 0, but 0 * NaN is not, so their values
      // are zeroed (their scores are masked below)
      if (c + kSub > kv_end) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (c + 4 * i + grp >= kv_end) v4[i] = make_uint4(0u, 0u, 0u, 0u);
      }
      // scores of 4 tokens x G rows, summed over the 16 lanes of the token's row
      float sc[4 * G];
      float cs[ROPE ? 4 : 1], sn[ROPE ? 4 : 1];
      if constexpr (ROPE) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          rope_sincos(kv_pos0 + (float)(c + grp), fhi[e], flo[e], &sn[e], &cs[e]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (ROPE) {
          if (i > 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float cn = __builtin_fmaf(-sn[e], s4[e], cs[e] * c4[e]);
              sn[e] = __builtin_fmaf(cs[e], s4[e], sn[e] * c4[e]);
              cs[e] = cn;
            }
          }
          float kr[8];
          rope_rot<T, RIL>(k4[i], cs, sn, kr);
#pragma unroll
          for (int g = 0; g < G; ++g) {
            float acc = qr[g][0] * kr[0];
#pragma unroll
            for (int e = 1; e < 8; ++e) acc = __builtin_fmaf(qr[g][e], kr[e], acc);
            sc[i * G + g] = acc;
          }
        } else {
#pragma unroll
          for (int g = 0; g < G; ++g) {
            float acc = dot2<T>(qv[g].x, k4[i].x, 0.f);
            acc = dot2<T>(qv[g].y, k4[i].y, acc);
            acc = dot2<T>(qv[g].z, k4[i].z, acc);
            sc[i * G + g] = dot2<T>(qv[g].w, k4[i].w, acc);
          }
        }
      }
      row16_sum_all<4 * G>(sc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (c + 4 * i + grp >= kv_end) {
#pragma unroll
          for (int g = 0; g < G; ++g) sc[i * G + g] = kNegInf;
        }
      }
      // lazy online softmax: move the reference max only when it is exceeded by thr
      float mx[G];
      bool need = false;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        mx[g] = __builtin_fmaxf(__builtin_fmaxf(sc[g], sc[G + g]),
                                __builtin_fmaxf(sc[2 * G + g], sc[3 * G + g]));
        need |= mx[g] > m[g] + thr;
      }
      if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float mn = __builtin_fmaxf(m[g], mx[g]);
          const float alpha = mn == kNegInf ? 1.f : fast_exp2((m[g] - mn) * cl2);
          l[g] *= alpha;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[g][e] *= alpha;
          m[g] = mn;
        }
      }
      uint32_t pp[2][G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float mc = (m[g] == kNegInf ? 0.f : m[g]) * cl2;
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = fast_exp2(__builtin_fmaf(sc[i * G + g], cl2, -mc));
        l[g] += (p[0] + p[1]) + (p[2] + p[3]);
        pp[0][g] = pack2<T>(p[0], p[1]);
        pp[1][g] = pack2<T>(p[2], p[3]);
      }
      // o += p . v over token pairs (0, 1) and (2, 3)
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t va = word(v4[2 * pr], j), vb = word(v4[2 * pr + 1], j);
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

    auto compute_chunk = [&](KVRegs<S, KV8>& X, int c) {
#pragma unroll
      for (int u = 0; u < S; ++u) {
        if (u == 0 || c + kSub * u < kv_end) compute_sub(&X.k[4 * u], &X.v[4 * u], c + kSub * u);
      }
    };

    // ---- main loop: double-buffered chunks, this wave's chunks every kStep keys.
    // The steady-state body issues its loads unconditionally (the last one or
    // two chunks are peeled), so each compute waits only for its own chunk.
    {
      const int c0 = kv_begin + tw * kChunk;
      const int n = c0 < kv_end ? (kv_end - c0 + kStep - 1) / kStep : 0;
      auto cpos = [&](int i) { return c0 + i * kStep; };
      if (n > 0) {
        if (!pre) {
          if constexpr (FASTPAGE) {
            chunk_pids(cpos(0), pidA);
            if (n > 1) chunk_pids(cpos(1), pidB);
          }
          load_chunk(A, cpos(0), pidA);
        }
        int i = 0;
        for (; i + 2 < n; i += 2) {
          load_chunk(B, cpos(i + 1), pidB);
          if constexpr (FASTPAGE) chunk_pids(cpos(i + 2), pidA);
          compute_chunk(A, cpos(i));
          load_chunk(A, cpos(i + 2), pidA);
          if constexpr (FASTPAGE) {
            if (i + 3 < n) chunk_pids(cpos(i + 3), pidB);
          }
          compute_chunk(B, cpos(i + 1));
        }
        if (i + 1 < n) {
          load_chunk(B, cpos(i + 1), pidB);
          compute_chunk(A, cpos(i));
          compute_chunk(B, cpos(i + 1));
        } else {
          compute_chunk(A, cpos(i));
        }
      }
    }
    // ---- issue the next segment's loads (page-aligned path); both chunk
    // buffers are free here
    pre = false;
    if constexpr (FASTPAGE) {
      if (s + 1 < s_end) {
        const int nt = segs[4 * (s + 1)];
        const int nbeg = segs[4 * (s + 1) + 1], nend = segs[4 * (s + 1) + 2];
        const int nb_ = tiles[4 * nt], nh = tiles[4 * nt + 1] + hw;
        const int nip0 = kv_indptr[nb_];
        load_q(nb_, nh, qn);
        const int nc0 = nbeg + tw * kChunk;
        const int nn = nc0 < nend ? (nend - nc0 + kStep - 1) / kStep : 0;
        if (nn > 0) {
          // the same page ids and addresses as chunk_pids / load_chunk compute
          // for that segment
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            if (c == 1 && nn < 2) break;
#pragma unroll
            for (int u = 0; u < S; ++u) {
              const int cc = nc0 + c * kStep;
              const int cu = cc + kSub * u < nend ? cc + kSub * u : cc;
              (c == 0 ? pidA : pidB)[u] = kv_indices[nip0 + (cu >> shift)];
            }
          }
          const uint32_t nhead = uint32_t(nh * kD + sub * 8);
#pragma unroll
          for (int u = 0; u < S; ++u) {
            const int cu = nc0 + kSub * u < nend ? nc0 + kSub * u : nc0;
            const int64_t base = int64_t(pidA[u]) * a.page_stride + int64_t(cu & (P - 1)) * tstride;
            const char* kb = reinterpret_cast<const char*>(kp + base);
            const char* vb = reinterpret_cast<const char*>(vp + base);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t off = uint32_t((4 * i + grp) * tstride + nhead) * kEsz;
              A.k[4 * u + i] = load_k(kb + off - kdel);
              A.v[4 * u + i] = *reinterpret_cast<const KW*>(vb + off);
            }
          }
        }
        pre = true;
      }
    }

    // ---- merge the 4 token groups of this wave (lanes xor 16, xor 32)
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float M = __builtin_fmaxf(m[g], __shfl_xor(m[g], 16));
      M = __builtin_fmaxf(M, __shfl_xor(M, 32));
      const float f = M == kNegInf ? 0.f : fast_exp2((m[g] - M) * cl2);
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
    if constexpr (TW == 1) {
      // the wave holds its head's whole state: lanes of token group g % 4
      // write row g (16 lanes x 8 elements), no workgroup barrier
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if ((g & 3) != grp) continue;
        float out[8];
        float lse = kNegInf;
        if (m[g] != kNegInf) {
          // fp8: the values are v_scale times their codes
          const float inv = KV8 ? a.v_scale / l[g] : 1.f / l[g];
#pragma unroll
          for (int e = 0; e < 8; ++e) out[e] = o[g][e] * inv;
          lse = m[g] * a.sm_scale + fast_log2(l[g]) * kLn2;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) out[e] = 0.f;
        }
        if (slot < 0) {
          const int64_t row = int64_t(b) * a.num_qo_heads + int64_t(h) * G + g;
          store8_dt(a.o, row * kD + sub * 8, out, a.out_dtype);
          if (a.lse && sub == 0) a.lse[row] = lse;
        } else {
          const int64_t row = int64_t(slot) * (HT * G) + hw * G + g;
          store8<ABP_F32>(a.o_part, row * kD + sub * 8, out);
          if (sub == 0) a.lse_part[row] = lse;
        }
      }
    } else {
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

      // ---- merge the TW waves of each head and write the tile's HT * G rows
      if (threadIdx.x < HT * G * 16) {
        const int rr = threadIdx.x >> 4;  // row within the tile
        const int hr = rr / G, g = rr - hr * G;
        const int e0 = (threadIdx.x & 15) * 8;
        float M = kNegInf;
#pragma unroll
        for (int j = 0; j < TW; ++j) M = __builtin_fmaxf(M, s_m[hr + HT * j][g]);
        float out[8];
        float lse = kNegInf;
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] = 0.f;
        if (M != kNegInf) {
          float L = 0.f;
#pragma unroll
          for (int j = 0; j < TW; ++j) {
            const int w = hr + HT * j;
            const float f = s_m[w][g] == kNegInf ? 0.f : fast_exp2((s_m[w][g] - M) * cl2);
            L = __builtin_fmaf(f, s_l[w][g], L);
#pragma unroll
            for (int e = 0; e < 8; ++e) out[e] = __builtin_fmaf(f, s_o[w][g][e0 + e], out[e]);
          }
          const float inv = KV8 ? a.v_scale / L : 1.f / L;
#pragma unroll
          for (int e = 0; e < 8; ++e) out[e] *= inv;
          lse = M * a.sm_scale + fast_log2(L) * kLn2;
        }
        if (slot < 0) {
          const int64_t row =
              int64_t(b) * a.num_qo_heads + int64_t(tiles[4 * tile + 1] + hr) * G + g;
          store8_dt(a.o, row * kD + e0, out, a.out_dtype);
          if (a.lse && e0 == 0) a.lse[row] = lse;
        } else {
          const int64_t row = int64_t(slot) * (HT * G) + rr;
          store8<ABP_F32>(a.o_part, row * kD + e0, out);
          if (e0 == 0) a.lse_part[row] = lse;
        }
      }
      __syncthreads();
    }
  }
}

// Sub-chunks per buffered chunk on the page-aligned path: 2 (32 tokens, 16 KB
// of K/V in flight per wave) where the registers allow it (G <= 4, no RoPE),
// else 1. The per-token path always uses 1.
template <int G, bool ROPE>
constexpr int sub_fast() {
  return (G <= 4 && !ROPE) ? 2 : 1;
}

template <typename T, int G, bool ROPE, int HT, bool KV8, bool RIL>
hipError_t launch_r(const AttnArgs& a, hipStream_t s) {
  const bool fast = a.page_shift >= 4;  // power of two and a multiple of 16
  if (fast)
    decode_kernel<T, G, ROPE, true, sub_fast<G, ROPE>(), HT, KV8, RIL>
        <<<a.workers, 256, 0, s>>>(a);
  else
    decode_kernel<T, G, ROPE, false, 1, HT, KV8, RIL><<<a.workers, 256, 0, s>>>(a);
  return hipGetLastError();
}

template <typename T, int G, int HT>
hipError_t launch_h(const Config& cfg, const AttnArgs& a, hipStream_t s) {
  if (cfg.kv_fp8) return launch_r<T, G, false, HT, true, false>(a, s);
  if (!cfg.rope) return launch_r<T, G, false, HT, false, false>(a, s);
  return cfg.rope_interleave ? launch_r<T, G, true, HT, false, true>(a, s)
                             : launch_r<T, G, true, HT, false, false>(a, s);
}

template <typename T, int G>
hipError_t launch_g(const Config& cfg, const AttnArgs& a, hipStream_t s) {
  static_assert(decode_tile_heads(4) == 4 && decode_tile_heads(2) == 1, "tile heads are 4 or 1");
  return decode_tile_heads(cfg.hkv) == 4 ? launch_h<T, G, 4>(cfg, a, s)
                                          : launch_h<T, G, 1>(cfg, a, s);
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

template <typename T, int G, int HT>
int occupancy_h(const Config& cfg, bool fast) {
  int n = 0;
  hipError_t e;
  if (cfg.kv_fp8)
    e = fast ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                   &n, decode_kernel<T, G, false, true, sub_fast<G, false>(), HT, true, false>, 256, 0)
             : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                   &n, decode_kernel<T, G, false, false, 1, HT, true, false>, 256, 0);
  else if (cfg.rope)
    e = fast ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                   &n, decode_kernel<T, G, true, true, sub_fast<G, true>(), HT, false, false>, 256, 0)
             : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                   &n, decode_kernel<T, G, true, false, 1, HT, false, false>, 256, 0);
  else
    e = fast ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                   &n, decode_kernel<T, G, false, true, sub_fast<G, false>(), HT, false, false>, 256, 0)
             : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                   &n, decode_kernel<T, G, false, false, 1, HT, false, false>, 256, 0);
  return e == hipSuccess ? n : 0;
}

template <typename T, int G>
int occupancy_g(const Config& cfg, bool fast) {
  return decode_tile_heads(cfg.hkv) == 4 ? occupancy_h<T, G, 4>(cfg, fast)
                                          : occupancy_h<T, G, 1>(cfg, fast);
}

template <typename T>
int occupancy_t(const Config& cfg, bool fast) {
  switch (cfg.group) {
    case 1: return occupancy_g<T, 1>(cfg, fast);
    case 2: return occupancy_g<T, 2>(cfg, fast);
    case 4: return occupancy_g<T, 4>(cfg, fast);
    case 8: return occupancy_g<T, 8>(cfg, fast);
    default: return 0;
  }
}

}  // namespace

hipError_t launch_decode(const Config& cfg, const AttnArgs& a, hipStream_t s) {
  if (decode_mfma_applies(cfg)) return launch_decode_mfma(cfg, a, s);
  if (cfg.qkv_dtype == ABP_BF16) return launch_t<BF16>(cfg, a, s);
  return launch_t<F16>(cfg, a, s);
}

int decode_blocks_per_cu(const Config& cfg) {
  if (decode_mfma_applies(cfg)) return decode_mfma_blocks_per_cu(cfg);
  const bool pow2 = (cfg.page_size & (cfg.page_size - 1)) == 0;
  const bool fast = pow2 && cfg.page_size >= 16;
  return cfg.qkv_dtype == ABP_BF16 ? occupancy_t<BF16>(cfg, fast) : occupancy_t<F16>(cfg, fast);
}

}  // namespace abp
