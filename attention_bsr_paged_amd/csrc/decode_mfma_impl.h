// Bodies of the matrix-core decode kernels, as device functions of one worker,
// so that a kernel can run them beside other work (the mixed decode + append
// launch). The kernels themselves, and what they compute, are in
// decode_mfma.hip.
#pragma once
#include "common.h"
#include "kernels.h"
#include "layout.h"

namespace abp {
namespace {
namespace dmi {

constexpr int kD = 128;
constexpr int kC = 32;               // tokens per chunk
constexpr float kRescaleLog2 = 8.f;  // lazy rescale threshold (log2 of the max p)

template <typename T>
__device__ __forceinline__ f32x4_t mfma16(const uint4& a, const uint4& b, f32x4_t c);
template <>
__device__ __forceinline__ f32x4_t mfma16<BF16>(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4_t mfma16<F16>(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// maximum over the 4 lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48)
__device__ __forceinline__ float max4groups(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto h = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = __builtin_fmaxf(__builtin_bit_cast(float, h[0]), __builtin_bit_cast(float, h[1]));
  const uint32_t w = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return __builtin_fmaxf(__builtin_bit_cast(float, r[0]), __builtin_bit_cast(float, r[1]));
}

__device__ __forceinline__ void store4_dt(void* base, int64_t off, const f32x4_t& v, int dt) {
  if (dt == ABP_F32) {
    *reinterpret_cast<float4*>(static_cast<float*>(base) + off) = make_float4(v[0], v[1], v[2], v[3]);
  } else if (dt == ABP_BF16) {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + off) =
        make_uint2(pack2<BF16>(v[0], v[1]), pack2<BF16>(v[2], v[3]));
  } else {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + off) =
        make_uint2(pack2<F16>(v[0], v[1]), pack2<F16>(v[2], v[3]));
  }
}

// two e4m3 codes (byte pair HI of w) as a 16-bit pair of the query's type;
// exact: every e4m3 value is a bf16 and an fp16 value
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
// 8 codes (two words) as 8 16-bit elements (four words), in order
template <typename T>
__device__ __forceinline__ uint4 widen8(uint32_t w0, uint32_t w1) {
  return make_uint4(fp8x2<T, false>(w0), fp8x2<T, true>(w0), fp8x2<T, false>(w1),
                    fp8x2<T, true>(w1));
}

// one plan segment of a decode worker's wave (uniform over the wave)
struct DecSeg {
  int b, h, ip0, kv_begin, kv_end, slot;
};

__device__ __forceinline__ uint32_t word_of(const uint4& u, int j) {
  return j == 0 ? u.x : j == 1 ? u.y : j == 2 ? u.z : u.w;
}

// Element e (0..7) of 8 16-bit values as fp32
template <typename T>
__device__ __forceinline__ float elem(const uint4& u, int e) {
  const uint32_t w = word_of(u, e >> 1);
  return (e & 1) ? hi_f32<T>(w) : lo_f32<T>(w);
}

// 8 fp32 values as 16-bit hi parts and the 16-bit rounding of the remainders
// (hi + lo carries ~16 significant bits), for products that keep fp32-level
// accuracy with three 16-bit matrix products
template <typename T>
__device__ __forceinline__ void split_hilo(const float (&v)[8], uint4& hi, uint4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    h[w] = pack2<T>(v[2 * w], v[2 * w + 1]);
    l[w] = pack2<T>(v[2 * w] - lo_f32<T>(h[w]), v[2 * w + 1] - hi_f32<T>(h[w]));
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// The rotary pairs a lane holds for one row in the operand layout of the
// matrix products (windows kc = 0..3, head dims 32 kc + 8 g16 + e):
// rotate-half pairs (j, j + 64) are elements e of windows kc and kc + 2,
// i = 8 kc + e for kc < 2 (j = 32 kc + 8 g16 + e); adjacent pairs (2j, 2j + 1)
// are word w of window kc, i = 4 kc + w (j = 16 kc + 4 g16 + w). Rotates the
// 16 pairs by the angles whose cosines and sines are cs / sn, in fp32.
template <typename T, bool RIL>
__device__ __forceinline__ void rope_rotate(const uint4 (&k)[4], const float (&cs)[16],
                                            const float (&sn)[16], float (&r)[4][8]) {
  if constexpr (RIL) {
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int i = 4 * kc + w;
        const float x = elem<T>(k[kc], 2 * w), y = elem<T>(k[kc], 2 * w + 1);
        r[kc][2 * w] = __builtin_fmaf(-y, sn[i], x * cs[i]);
        r[kc][2 * w + 1] = __builtin_fmaf(x, sn[i], y * cs[i]);
      }
  } else {
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 8 * kc + e;
        const float x = elem<T>(k[kc], e), y = elem<T>(k[kc + 2], e);
        r[kc][e] = __builtin_fmaf(-y, sn[i], x * cs[i]);
        r[kc + 2][e] = __builtin_fmaf(x, sn[i], y * cs[i]);
      }
  }
}

// LDS of a decode workgroup: one slice per wave of each array. The kernel
// declares the arrays separately (ABP_DECODE_LDS), so the compiler sees every
// stage as its own object and does not order a stage's reads behind loads
// into another.
struct DecodeLds {
  uint16_t* k0;  // [4][kC * kD] K ring, stage 0 (rows XOR-swizzled by 16-byte piece)
  uint16_t* k1;  // stage 1
  uint16_t* v0;  // [4][kC * kD] V ring, stage 0
  uint16_t* v1;  // stage 1
  uint16_t* q;   // [4][2][G * kD] raw q rows of the current and the next segment
                 // ([4][G * kD] with RoPE: a segment's rows are consumed when it opens)
};

#define ABP_DECODE_LDS(name, G, ROPE)                                                    \
  __shared__ __align__(16) uint16_t name##_k0[4 * dmi::kC * dmi::kD];                    \
  __shared__ __align__(16) uint16_t name##_k1[4 * dmi::kC * dmi::kD];                    \
  __shared__ __align__(16) uint16_t name##_v0[4 * dmi::kC * dmi::kD];                    \
  __shared__ __align__(16) uint16_t name##_v1[4 * dmi::kC * dmi::kD];                    \
  __shared__ __align__(16) uint16_t name##_q[((ROPE) ? 4 : 8) * (G) * dmi::kD];          \
  const dmi::DecodeLds name = {name##_k0, name##_k1, name##_v0, name##_v1, name##_q}

constexpr int kAnchorTiles = 32;  // even: anchors fall on chunk boundaries

// The work of one decode worker (a 256-thread workgroup, or the first four
// waves of a larger one): segments wseg[worker] .. wseg[worker + 1] of the
// plan, each wave taking one kv head of the segment's tile.
//
// Data movement. K, V and q reach LDS by memory-to-LDS loads only, so that
// every load a wait counts is of one kind: loads into registers and loads
// into LDS are not retired in order with each other, and a count over a mix
// of both does not prove that a given earlier load has landed. K and V go
// through per-wave rings of two 32-row stages (16-byte pieces of a row
// XOR-swizzled by the row, so the row reads of K and the transpose reads of V
// are free of bank conflicts); a segment's q rows arrive with the chunk that
// opens the segment.
//
// The worker's chunks form one stream over its segments (c = kv_begin +
// 32 n within each): the next chunk of the stream, also when it opens the
// next segment, is loaded while the current one is computed, so a segment
// boundary costs no memory round trip. The current chunk's 16 loads were
// issued before the 16 of the next chunk (and its segment's NQ q loads), so
// vmcnt(16) or vmcnt(16 + NQ) covers them (vmcnt(0) when nothing follows);
// output stores are never younger than a wait's younger loads. A stage is
// refilled only after the reads of its previous chunk have completed
// (lgkmcnt(0)). Segments without keys (requests of length 0) write their
// empty state when reached.
//
// Products. S^T = K Q^T: A = 16 token rows of K (lane: token l % 16, 16 bytes
// of head dims 32 kc + 8 (l / 16) .. + 7), B = q of the G rows padded to 16
// (lanes of rows >= G take row G - 1: those rows of S, P and O repeat it and
// are never written). Softmax in fp32, base 2, lazy rescale; a lane holds 8
// scores of one row. O^T += V^T P^T: B = P^T straight from the S^T registers,
// A = V^T by transpose reads.
//
// RoPE (ROPE, pair layout RIL): q (at its position) and every K row (key t at
// kv_pos_offset + t) are rotated in fp32 and enter S^T as 16-bit hi and lo
// parts, S^T = Kh Qh + Kh Ql + Kl Qh (12 products per 16-token tile), so the
// scores keep fp32-level accuracy: rounding the rotated operands to 16 bits
// moves lse by up to ~1e-2. A segment's q is rotated once, when it opens, and
// its hi / lo parts stay in registers. A lane's 16 pairs keep the cosine and
// sine of their angle at the lane's token of the next 16-token tile; each tile
// steps them by 16 positions (angle addition), and every kAnchorTiles tiles
// (at a chunk boundary) they are evaluated exactly again, so the stepping
// error stays below ~1e-5 rad. V is not rotated. (Scores as fp32 products,
// v_mfma_f32_16x16x4_f32 with 32 per tile, measured slower: 104 against
// 101 us for the whole cascade.)
//
// NT: non-temporal K/V loads. They pay when decode holds the whole chip and
// HBM is the limit; on a few compute units beside other work (the mixed
// launch) ordinary loads are faster.
template <typename T, int G, bool NT, bool ROPE, bool RIL>
__device__ __forceinline__ void decode_mfma_worker(const AttnArgs& a, int worker,
                                                   const DecodeLds& lds) {
  static_assert(G == 4 || G == 8, "rows of one kv head fill at most one 16-row tile");
  constexpr int HT = 4;      // kv heads per tile = waves per worker
  constexpr int NQ = G / 4;  // memory-to-LDS loads of a segment's q rows (1 KB each)
  constexpr int AUX = NT ? 2 : 0;

  const ABP_CONST_AS int32_t* plan = const_as(a.plan);
  const ABP_CONST_AS int32_t* wseg = plan + plan[H_OFF_WSEG];
  const ABP_CONST_AS int32_t* segs = plan + plan[H_OFF_SEG];
  const ABP_CONST_AS int32_t* tiles = plan + plan[H_OFF_TILE];
  const ABP_CONST_AS int32_t* kv_indptr = const_as(a.kv_indptr);
  const ABP_CONST_AS int32_t* kv_indices = const_as(a.kv_indices);
  const int s_begin = wseg[worker], s_end = wseg[worker + 1];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g16 = lane >> 4;
  const int l16 = lane & 15;
  const int qrow = l16 < G ? l16 : G - 1;  // q row of this lane's B-operand column
  const float cl2 = a.sm_scale_log2;
  const float thr = kRescaleLog2 / cl2;
  const int P = a.page_size;
  const int shift = a.page_shift;
  const int tstride = a.token_stride;
  uint16_t* const myK0 = lds.k0 + wave * (kC * kD);
  uint16_t* const myK1 = lds.k1 + wave * (kC * kD);
  uint16_t* const myV0 = lds.v0 + wave * (kC * kD);
  uint16_t* const myV1 = lds.v1 + wave * (kC * kD);
  // q row buffers: two, alternating by segment (RoPE: one)
  constexpr int NQB = ROPE ? 1 : 2;
  uint16_t* const myQ = lds.q + wave * (NQB * G * kD);
  int qsel = 0;  // buffer of the current segment's q rows

  auto seg_at = [&](int s) {
    DecSeg g;
    const int tile = segs[4 * s];
    g.kv_begin = segs[4 * s + 1];
    g.kv_end = segs[4 * s + 2];
    g.slot = segs[4 * s + 3];
    g.b = tiles[4 * tile];
    g.h = tiles[4 * tile + 1] + wave;
    g.ip0 = kv_indptr[g.b];
    return g;
  };
  // element offset of token t (< the tile's page end) of head g.h
  auto row_base = [&](const DecSeg& g, int t) -> int64_t {
    return int64_t(kv_indices[g.ip0 + (t >> shift)]) * a.page_stride +
           int64_t(t & (P - 1)) * tstride + int64_t(g.h) * kD;
  };

  // Memory-to-LDS loads address a row as a uniform base (the tile's first row,
  // in bytes) plus a 32-bit lane offset. For instruction i of a tile, lane l
  // takes row 4 i + l / 16 and writes LDS position l % 16 of it; the lane
  // offsets repeat every 4 (K) or 2 (V) instructions, so few stay in registers.
  const uint32_t lrow = uint32_t(lane >> 4) * uint32_t(tstride) * 2u;
  uint32_t koff[4], voff[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) koff[i] = lrow + (uint32_t((lane & 15) ^ (4 * i + (lane >> 4))) << 4);
#pragma unroll
  for (int i = 0; i < 2; ++i)
    voff[i] = lrow + (uint32_t((lane & 15) ^ (2 * (4 * i + (lane >> 4)))) << 4);
  const char* const kbytes = static_cast<const char*>(a.k_pages);
  const char* const vbytes = static_cast<const char*>(a.v_pages);

  // q rows of the segment into buffer sel (row-major [G][128]): load k moves
  // rows 4 k .. 4 k + 3, position l % 16 of row r holding piece (l % 16) ^ (r % 4)
  auto load_q = [&](const DecSeg& g, int sel) {
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
      const int r = 4 * k + g16;
      const uint16_t* src = static_cast<const uint16_t*>(a.q) +
                            (int64_t(g.b) * a.num_qo_heads + int64_t(g.h) * G + r) * kD +
                            8 * (l16 ^ (r & 3));
      __builtin_amdgcn_global_load_lds(src, (ABP_LDS void*)(myQ + sel * (G * kD) + 4 * k * kD),
                                       16, 0, 0);
    }
  };
  // K of chunk c: row r of the stage = token c + r (a tile past kv_end re-reads
  // tile 0, in bounds and masked); position p of row r holds piece p ^ (r % 16)
  auto load_k = [&](const DecSeg& g, int c, uint16_t* dst) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int t0 = (c + 16 * mb < g.kv_end) ? c + 16 * mb : c;
      const char* tb = kbytes + row_base(g, t0) * 2;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_global_load_lds(tb + int64_t(4 * i) * tstride * 2 + koff[i],
                                         (ABP_LDS void*)(dst + (16 * mb + 4 * i) * kD), 16, 0,
                                         AUX);
    }
  };
  // V of chunk c: position p of row r holds piece p ^ (2 (r % 8)), the swizzle
  // of the transpose reads. A row at or past kv_end takes the last key's
  // values instead: slots past a request's last valid token hold undefined
  // bits (possibly NaN or inf), and although their p is 0, 0 * NaN would
  // still reach o.
  auto load_v = [&](const DecSeg& g, int c, uint16_t* dst) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int t0 = (c + 16 * mb < g.kv_end) ? c + 16 * mb : c;
      const char* tb = vbytes + row_base(g, t0) * 2;
      if (t0 + 16 <= g.kv_end) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          __builtin_amdgcn_global_load_lds(tb + int64_t(4 * i) * tstride * 2 + voff[i & 1],
                                           (ABP_LDS void*)(dst + (16 * mb + 4 * i) * kD), 16, 0,
                                           AUX);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * i + (lane >> 4);
          const int rs = min(r, g.kv_end - 1 - t0);
          const uint32_t off = uint32_t(rs) * uint32_t(tstride) * 2u +
                               (uint32_t((lane & 15) ^ (2 * (r & 7))) << 4);
          __builtin_amdgcn_global_load_lds(tb + off, (ABP_LDS void*)(dst + (16 * mb + 4 * i) * kD),
                                           16, 0, AUX);
        }
      }
    }
  };
  // 16-byte window kc (head dims 32 kc + 8 g16 ..) of this lane's K row in tile mb
  auto k_window = [&](const uint16_t* sk, int mb, int kc) {
    return *reinterpret_cast<const uint4*>(sk + (16 * mb + l16) * kD + (((4 * kc + g16) ^ l16) << 3));
  };
  // the same window of this lane's q row (current segment)
  auto q_window = [&](int kc) {
    return *reinterpret_cast<const uint4*>(myQ + qsel * (G * kD) + qrow * kD +
                                           (((4 * kc + g16) ^ (qrow & 3)) << 3));
  };

  // ---- RoPE state
  const float* rope = ROPE ? reinterpret_cast<const float*>(a.plan + plan[H_OFF_ROPE]) : nullptr;
  // pair i of this lane: rotate-half j = 32 (i / 8) + 8 g16 + i % 8,
  // interleaved j = 16 (i / 4) + 4 g16 + i % 4
  auto pair_j = [&](int i) {
    return RIL ? 16 * (i >> 2) + 4 * g16 + (i & 3) : 32 * (i >> 3) + 8 * g16 + (i & 7);
  };
  // exact cosines and sines of the lane's 16 pairs at position pos
  auto anchor = [&](float pos, float (&cs)[16], float (&sn)[16]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = pair_j(i);
      rope_sincos(pos, rope[2 * j], rope[2 * j + 1], &sn[i], &cs[i]);
    }
  };
  float c16[16], s16[16];  // RoPE: the rotation by 16 positions of the lane's pairs
  if constexpr (ROPE) anchor(16.f, c16, s16);
  float cs[16], sn[16];    // RoPE: angles at the lane's token of the next tile
  uint4 qh[4], ql[4];      // RoPE: the segment's rotated q as 16-bit hi / lo parts
  int tcount = 0;          // RoPE: tiles of the segment so far
  float kpos0 = 0.f;       // RoPE: position of the segment's key 0

  float m = kNegInf, lsum = 0.f;
  f32x4_t O[8];
#pragma unroll
  for (int md = 0; md < 8; ++md) O[md] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // A segment opens: its q rows have landed in LDS (only the 16 loads of the
  // next chunk are younger). RoPE: rotate them at the query position into
  // the fp32 q of the segment.
  auto open = [&](const DecSeg& g) {
    __builtin_amdgcn_s_waitcnt(0x4f70);  // vmcnt(16)
    if constexpr (ROPE) {
      const int npg = kv_indptr[g.b + 1] - g.ip0;
      const int kv_len = npg > 0 ? (npg - 1) * P + a.kv_last_page_len[g.b] : 0;
      const float qpos = a.q_pos ? (float)a.q_pos[g.b] : (float)(kv_len - 1);
      kpos0 = a.kv_pos_offset ? (float)a.kv_pos_offset[g.b] : 0.f;
      tcount = 0;
      uint4 qf[4];
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) qf[kc] = q_window(kc);
      float rq[4][8];
      {
        float qc[16], qs[16];
        anchor(qpos, qc, qs);
        rope_rotate<T, RIL>(qf, qc, qs, rq);
      }
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) split_hilo<T>(rq[kc], qh[kc], ql[kc]);
    }
  };

  // S^T of chunk c (both 16-token tiles): S[mb] holds keys c + 16 mb + 4 g16 + j of row l16
  auto scores = [&](int c, const uint16_t* sk, f32x4_t (&S)[2]) __attribute__((always_inline)) {
    if constexpr (!ROPE) {
      uint4 qf[4];
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) qf[kc] = q_window(kc);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        S[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) S[mb] = mfma16<T>(k_window(sk, mb, kc), qf[kc], S[mb]);
      }
    } else {
      if (tcount % kAnchorTiles == 0) anchor(kpos0 + (float)(c + l16), cs, sn);
      tcount += 2;
      uint4 kw[2][4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) kw[mb][kc] = k_window(sk, mb, kc);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        uint4 kh[4], kl[4];
        {
          float r[4][8];
          rope_rotate<T, RIL>(kw[mb], cs, sn, r);
#pragma unroll
          for (int kc = 0; kc < 4; ++kc) split_hilo<T>(r[kc], kh[kc], kl[kc]);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {  // to the next tile: 16 positions further
          const float cn = __builtin_fmaf(-sn[i], s16[i], cs[i] * c16[i]);
          sn[i] = __builtin_fmaf(cs[i], s16[i], sn[i] * c16[i]);
          cs[i] = cn;
        }
        S[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          S[mb] = mfma16<T>(kh[kc], qh[kc], S[mb]);
          S[mb] = mfma16<T>(kh[kc], ql[kc], S[mb]);
          S[mb] = mfma16<T>(kl[kc], qh[kc], S[mb]);
        }
      }
    }
  };

  auto compute = [&](const DecSeg& g, int c, const uint16_t* sk, const uint16_t* sv)
                     __attribute__((always_inline)) {
    f32x4_t S[2];
    scores(c, sk, S);
    if (c + kC > g.kv_end) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (c + 16 * mb + 4 * g16 + j >= g.kv_end) S[mb][j] = kNegInf;
    }
    float mx = __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(S[0][0], S[0][1]),
                                               __builtin_fmaxf(S[0][2], S[0][3])),
                               __builtin_fmaxf(__builtin_fmaxf(S[1][0], S[1][1]),
                                               __builtin_fmaxf(S[1][2], S[1][3])));
    mx = max4groups(mx);
    if (__builtin_amdgcn_ballot_w64(mx > m + thr)) {
      const float mn = __builtin_fmaxf(m, mx);
      const float alpha = mn == kNegInf ? 1.f : fast_exp2((m - mn) * cl2);
      m = mn;
      lsum *= alpha;
#pragma unroll
      for (int md = 0; md < 8; ++md) O[md] *= alpha;
    }
    const float mc = (m == kNegInf ? 0.f : m) * cl2;
    float p[2][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) p[mb][j] = fast_exp2(__builtin_fmaf(S[mb][j], cl2, -mc));
    lsum += ((p[0][0] + p[0][1]) + (p[0][2] + p[0][3])) +
            ((p[1][0] + p[1][1]) + (p[1][2] + p[1][3]));
    // P^T: K-slots of lane group g16 are keys 4 g16 .. + 3 and 16 + 4 g16 .. + 3
    const uint4 pB = make_uint4(pack2<T>(p[0][0], p[0][1]), pack2<T>(p[0][2], p[0][3]),
                                pack2<T>(p[1][0], p[1][1]), pack2<T>(p[1][2], p[1][3]));
    // O^T += V^T P^T: lane c of a 16-lane group points at V[key 4 g16 + c / 4
    // (+ 16)][d 16 md + 4 (c % 4)] and receives V[4 keys][d 16 md + c]
    const int kA = 4 * g16 + (l16 >> 2);
    const int kB = kA + 16;
#pragma unroll
    for (int md = 0; md < 8; ++md) {
      const int d0 = md * 16 + 4 * (l16 & 3);
      const int offA = kA * kD + (((d0 >> 3) ^ (2 * (kA & 7))) * 8) + (d0 & 7);
      const int offB = kB * kD + (((d0 >> 3) ^ (2 * (kB & 7))) * 8) + (d0 & 7);
      const v4i16_t a4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ABP_LDS v4i16_t*)(sv + offA));
      const v4i16_t b4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ABP_LDS v4i16_t*)(sv + offB));
      const uint2 av = __builtin_bit_cast(uint2, a4), bv = __builtin_bit_cast(uint2, b4);
      O[md] = mfma16<T>(make_uint4(av.x, av.y, bv.x, bv.y), pB, O[md]);
    }
  };

  // ---- rows: o = O / L, lse = m * scale + ln L (L summed over the lane groups)
  auto finish = [&](const DecSeg& g) {
    float L = lsum;
    L += __shfl_xor(L, 16);
    L += __shfl_xor(L, 32);
    const bool empty = !(L > 0.f);
    const float inv = empty ? 0.f : 1.f / L;
    const float lse = empty ? kNegInf : m * a.sm_scale + fast_log2(L) * kLn2;
    if (l16 < G) {
      if (g.slot < 0) {
        const int64_t row = int64_t(g.b) * a.num_qo_heads + int64_t(g.h) * G + l16;
#pragma unroll
        for (int md = 0; md < 8; ++md) store4_dt(a.o, row * kD + md * 16 + 4 * g16, O[md] * inv,
                                                 a.out_dtype);
        if (a.lse && g16 == 0) a.lse[row] = lse;
      } else {
        const int64_t row = int64_t(g.slot) * (HT * G) + int64_t(wave) * G + l16;
#pragma unroll
        for (int md = 0; md < 8; ++md) {
          const f32x4_t v = O[md] * inv;
          *reinterpret_cast<float4*>(a.o_part + row * kD + md * 16 + 4 * g16) =
              make_float4(v[0], v[1], v[2], v[3]);
        }
        if (g16 == 0) a.lse_part[row] = lse;
      }
    }
    m = kNegInf;
    lsum = 0.f;
#pragma unroll
    for (int md = 0; md < 8; ++md) O[md] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  };
  // empty state (o = 0, lse = -inf) of a segment without keys
  auto finish_empty = [&](const DecSeg& g) {
    if (l16 < G) {
      if (g.slot < 0) {
        const int64_t row = int64_t(g.b) * a.num_qo_heads + int64_t(g.h) * G + l16;
#pragma unroll
        for (int md = 0; md < 8; ++md)
          store4_dt(a.o, row * kD + md * 16 + 4 * g16, f32x4_t{0.f, 0.f, 0.f, 0.f}, a.out_dtype);
        if (a.lse && g16 == 0) a.lse[row] = kNegInf;
      } else {
        const int64_t row = int64_t(g.slot) * (HT * G) + int64_t(wave) * G + l16;
#pragma unroll
        for (int md = 0; md < 8; ++md)
          *reinterpret_cast<float4*>(a.o_part + row * kD + md * 16 + 4 * g16) =
              make_float4(0.f, 0.f, 0.f, 0.f);
        if (g16 == 0) a.lse_part[row] = kNegInf;
      }
    }
  };

  int s = s_begin;
  if (s >= s_end) return;
  DecSeg g = seg_at(s);
  while (g.kv_begin >= g.kv_end) {
    finish_empty(g);
    if (++s >= s_end) return;
    g = seg_at(s);
  }
  int c = g.kv_begin;
  load_q(g, qsel);
  load_v(g, c, myV0);
  load_k(g, c, myK0);
  open(g);

  // one chunk of the stream on stage (Kc, Vc); the next goes to (Kn, Vn).
  // Returns false when the stream has ended.
  auto step = [&](const uint16_t* Kc, const uint16_t* Vc, uint16_t* Kn, uint16_t* Vn)
                  __attribute__((always_inline)) -> bool {
    int c2 = c + kC, s2 = s;
    DecSeg g2 = g;
    const bool newseg = c2 >= g.kv_end;
    if (newseg) {
      for (;;) {
        if (++s2 >= s_end) break;
        g2 = seg_at(s2);
        if (g2.kv_begin < g2.kv_end) break;
        finish_empty(g2);
      }
      c2 = g2.kv_begin;
    }
    const bool more = s2 < s_end;
    if (more) {
      // previous reads of stages Kn, Vn (and of the q buffer the next
      // segment takes) have completed
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      if (newseg) load_q(g2, qsel ^ (NQB - 1));
      load_v(g2, c2, Vn);
      load_k(g2, c2, Kn);
      if (newseg)
        __builtin_amdgcn_s_waitcnt(NQ == 1 ? 0x4f71 : 0x4f72);  // vmcnt(16 + NQ)
      else
        __builtin_amdgcn_s_waitcnt(0x4f70);  // vmcnt(16)
    } else {
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    }
    compute(g, c, Kc, Vc);
    if (newseg) {
      finish(g);
      if (!more) return false;
      g = g2;
      s = s2;
      qsel ^= NQB - 1;
      open(g);
    }
    c = c2;
    return true;
  };
  for (;;) {
    if (!step(myK0, myV0, myK1, myV1)) break;
    if (!step(myK1, myV1, myK0, myV0)) break;
  }
}

// The same decode for an fp8 (OCP e4m3) KV cache. K and V rows are half as
// wide, so each lane's share is loaded into registers as codes and widened
// to the query's 16-bit type on the way to the matrix cores:
//   * K: lane group g16 holds head dims [16 g16, 16 g16 + 16) and
//     [64 + 16 g16, 64 + 16 g16 + 16) of its token (two 16-byte loads per
//     16-token tile, each covering a contiguous 64-byte half of every row);
//     product kc takes dims 64 (kc / 2) + 16 g16 + 8 (kc % 2) .. + 7 as the
//     lane's 8 K-slots, and q is loaded with the same head-dim map (any map
//     serves a dot product if q and K share it);
//   * V: lane l loads 16 codes of row 8 i + l / 8 (four loads per chunk),
//     widens them to two 16-byte chunks and writes them into its wave's LDS
//     slice in the layout the transpose reads of the 16-bit kernel expect.
// k_scale is folded into the logit scale on the host; v_scale multiplies the
// final normalisation. K and V codes take 32 VGPRs per chunk; with one
// 4-wave workgroup per compute unit (512 registers a wave) four register sets
// fit, so three chunks stay in flight per wave and every wait is a register
// dependency.
template <typename T, int G>
__device__ __forceinline__ void decode_mfma_fp8_worker(const AttnArgs& a, int worker) {
  static_assert(G == 4 || G == 8, "rows of one kv head fill at most one 16-row tile");
  constexpr int HT = 4;
  __shared__ __align__(16) uint16_t sV[HT][kC * kD];  // widened V of a wave's chunk

  const ABP_CONST_AS int32_t* plan = const_as(a.plan);
  const ABP_CONST_AS int32_t* wseg = plan + plan[H_OFF_WSEG];
  const ABP_CONST_AS int32_t* segs = plan + plan[H_OFF_SEG];
  const ABP_CONST_AS int32_t* tiles = plan + plan[H_OFF_TILE];
  const ABP_CONST_AS int32_t* kv_indptr = const_as(a.kv_indptr);
  const ABP_CONST_AS int32_t* kv_indices = const_as(a.kv_indices);
  const int s_begin = wseg[worker], s_end = wseg[worker + 1];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g16 = lane >> 4;
  const int l16 = lane & 15;
  const float cl2 = a.sm_scale_log2;
  const float thr = kRescaleLog2 / cl2;
  const uint8_t* __restrict__ kp = static_cast<const uint8_t*>(a.k_pages);
  const uint8_t* __restrict__ vp = static_cast<const uint8_t*>(a.v_pages);
  const int P = a.page_size;
  const int shift = a.page_shift;
  const int tstride = a.token_stride;  // elements = bytes
  uint16_t* const sv = sV[wave];

  for (int s = s_begin; s < s_end; ++s) {
    const int tile = segs[4 * s];
    const int kv_begin = segs[4 * s + 1], kv_end = segs[4 * s + 2], slot = segs[4 * s + 3];
    const int b = tiles[4 * tile], h = tiles[4 * tile + 1] + wave;
    const int ip0 = kv_indptr[b];

    // q of row l16 (< G), head dims dim0(kc) .. + 7 for product kc, the K map
    uint4 qf[4];
    {
      const int qr = l16 < G ? l16 : G - 1;
      const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                             (int64_t(b) * a.num_qo_heads + int64_t(h) * G + qr) * kD;
      const uint32_t keep = l16 < G ? 0xffffffffu : 0u;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const uint4 v = *reinterpret_cast<const uint4*>(qrow + 64 * (kc >> 1) + 16 * g16 + 8 * (kc & 1));
        qf[kc] = make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep);
      }
    }

    float m = kNegInf, lsum = 0.f;
    f32x4_t O[8];
#pragma unroll
    for (int md = 0; md < 8; ++md) O[md] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto row_base = [&](int t) -> int64_t {
      return int64_t(kv_indices[ip0 + (t >> shift)]) * a.page_stride +
             int64_t(t & (P - 1)) * tstride + int64_t(h) * kD;
    };
    // K codes of chunk c: tile mb (a tile past kv_end re-reads tile 0, in
    // bounds and masked); lane: token l16, bytes 16 g16 .. + 15 and 64 + 16 g16
    // .. + 15, so that each load covers a contiguous 64-byte half of every row
    auto load_k = [&](int c, uint4 (&kr)[2][2]) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int t0 = (c + 16 * mb < kv_end) ? c + 16 * mb : c;
        const uint8_t* rp = kp + row_base(t0) + int64_t(l16) * tstride + 16 * g16;
        kr[mb][0] = load_once(reinterpret_cast<const uint4*>(rp));
        kr[mb][1] = load_once(reinterpret_cast<const uint4*>(rp + 64));
      }
    };
    // V codes of chunk c: piece i is row 8 i + l / 8, bytes 16 (l % 8) .. + 15;
    // a row at or past kv_end takes the last key's codes (unwritten slots may
    // hold NaN codes, and p = 0 does not cancel them)
    auto load_v = [&](int c, uint4 (&vr)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 8 * i + (lane >> 3);
        const int t0 = (c + 16 * (r >> 4) < kv_end) ? c + 16 * (r >> 4) : c;
        const int rs = min(r & 15, kv_end - 1 - t0);
        vr[i] = load_once(reinterpret_cast<const uint4*>(vp + row_base(t0) +
                                                         int64_t(rs) * tstride +
                                                         16 * (lane & 7)));
      }
    };

    auto compute = [&](int c, const uint4 (&kr)[2][2], const uint4 (&vr)[4])
                       __attribute__((always_inline)) {
      // widened V into the wave's LDS slice: the 16 codes of a lane are the
      // row's logical 16-byte chunks q0 = 2 (l % 8) and q0 + 1, held at
      // positions q0 ^ (2 (row & 7)) and the one after (the swizzle is even)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 8 * i + (lane >> 3);
        const int p0 = (2 * (lane & 7)) ^ (2 * (r & 7));
        uint16_t* dst = sv + r * kD + p0 * 8;
        *reinterpret_cast<uint4*>(dst) = widen8<T>(vr[i].x, vr[i].y);
        *reinterpret_cast<uint4*>(dst + 8) = widen8<T>(vr[i].z, vr[i].w);
      }
      f32x4_t S[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        S[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        S[mb] = mfma16<T>(widen8<T>(kr[mb][0].x, kr[mb][0].y), qf[0], S[mb]);
        S[mb] = mfma16<T>(widen8<T>(kr[mb][0].z, kr[mb][0].w), qf[1], S[mb]);
        S[mb] = mfma16<T>(widen8<T>(kr[mb][1].x, kr[mb][1].y), qf[2], S[mb]);
        S[mb] = mfma16<T>(widen8<T>(kr[mb][1].z, kr[mb][1].w), qf[3], S[mb]);
      }
      if (c + kC > kv_end) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (c + 16 * mb + 4 * g16 + j >= kv_end) S[mb][j] = kNegInf;
      }
      float mx = __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(S[0][0], S[0][1]),
                                                 __builtin_fmaxf(S[0][2], S[0][3])),
                                 __builtin_fmaxf(__builtin_fmaxf(S[1][0], S[1][1]),
                                                 __builtin_fmaxf(S[1][2], S[1][3])));
      mx = max4groups(mx);
      if (__builtin_amdgcn_ballot_w64(mx > m + thr)) {
        const float mn = __builtin_fmaxf(m, mx);
        const float alpha = mn == kNegInf ? 1.f : fast_exp2((m - mn) * cl2);
        m = mn;
        lsum *= alpha;
#pragma unroll
        for (int md = 0; md < 8; ++md) O[md] *= alpha;
      }
      const float mc = (m == kNegInf ? 0.f : m) * cl2;
      float p[2][4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) p[mb][j] = fast_exp2(__builtin_fmaf(S[mb][j], cl2, -mc));
      lsum += ((p[0][0] + p[0][1]) + (p[0][2] + p[0][3])) +
              ((p[1][0] + p[1][1]) + (p[1][2] + p[1][3]));
      const uint4 pB = make_uint4(pack2<T>(p[0][0], p[0][1]), pack2<T>(p[0][2], p[0][3]),
                                  pack2<T>(p[1][0], p[1][1]), pack2<T>(p[1][2], p[1][3]));
      const int kA = 4 * g16 + (l16 >> 2);
      const int kB = kA + 16;
#pragma unroll
      for (int md = 0; md < 8; ++md) {
        const int d0 = md * 16 + 4 * (l16 & 3);
        const int offA = kA * kD + (((d0 >> 3) ^ (2 * (kA & 7))) * 8) + (d0 & 7);
        const int offB = kB * kD + (((d0 >> 3) ^ (2 * (kB & 7))) * 8) + (d0 & 7);
        const v4i16_t a4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ABP_LDS v4i16_t*)(sv + offA));
        const v4i16_t b4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ABP_LDS v4i16_t*)(sv + offB));
        const uint2 av = __builtin_bit_cast(uint2, a4), bv = __builtin_bit_cast(uint2, b4);
        O[md] = mfma16<T>(make_uint4(av.x, av.y, bv.x, bv.y), pB, O[md]);
      }
    };

    // Four register sets: chunk n is computed while chunks n + 1 .. n + 3 are
    // in flight. The first three loads are issued unconditionally (a chunk
    // past the segment's last re-reads it), so every wait in the steady loop,
    // where all loads are real chunks, is the same register dependency; the
    // last chunks (fewer than seven) run in a tail with conditional loads.
    constexpr int NS = 4;
    const int nch = kv_begin < kv_end ? (kv_end - kv_begin + kC - 1) / kC : 0;
    uint4 Kr[NS][2][2], Vr[NS][4];
    auto ch = [&](int n) { return kv_begin + min(n, nch - 1) * kC; };
    if (nch > 0) {
#pragma unroll
      for (int i = 0; i < NS - 1; ++i) {
        load_k(ch(i), Kr[i]);
        load_v(ch(i), Vr[i]);
      }
      int n = 0;
      for (; n + 2 * NS - 1 <= nch; n += NS) {
#pragma unroll
        for (int u = 0; u < NS; ++u) {
          load_k(kv_begin + (n + u + NS - 1) * kC, Kr[(u + NS - 1) % NS]);
          load_v(kv_begin + (n + u + NS - 1) * kC, Vr[(u + NS - 1) % NS]);
          compute(kv_begin + (n + u) * kC, Kr[u], Vr[u]);
        }
      }
      for (; n < nch; n += NS) {
#pragma unroll
        for (int u = 0; u < NS; ++u) {
          if (n + u + NS - 1 < nch) {
            load_k(kv_begin + (n + u + NS - 1) * kC, Kr[(u + NS - 1) % NS]);
            load_v(kv_begin + (n + u + NS - 1) * kC, Vr[(u + NS - 1) % NS]);
          }
          if (n + u < nch) compute(kv_begin + (n + u) * kC, Kr[u], Vr[u]);
        }
      }
    }

    float L = lsum;
    L += __shfl_xor(L, 16);
    L += __shfl_xor(L, 32);
    const bool empty = !(L > 0.f);
    const float inv = empty ? 0.f : a.v_scale / L;  // the values are v_scale times their codes
    const float lse = empty ? kNegInf : m * a.sm_scale + fast_log2(L) * kLn2;
    if (l16 < G) {
      if (slot < 0) {
        const int64_t row = int64_t(b) * a.num_qo_heads + int64_t(h) * G + l16;
#pragma unroll
        for (int md = 0; md < 8; ++md) store4_dt(a.o, row * kD + md * 16 + 4 * g16, O[md] * inv,
                                                 a.out_dtype);
        if (a.lse && g16 == 0) a.lse[row] = lse;
      } else {
        const int64_t row = int64_t(slot) * (HT * G) + int64_t(wave) * G + l16;
#pragma unroll
        for (int md = 0; md < 8; ++md) {
          const f32x4_t v = O[md] * inv;
          *reinterpret_cast<float4*>(a.o_part + row * kD + md * 16 + 4 * g16) =
              make_float4(v[0], v[1], v[2], v[3]);
        }
        if (g16 == 0) a.lse_part[row] = lse;
      }
    }
  }
}

}  // namespace dmi
}  // namespace
}  // namespace abp
