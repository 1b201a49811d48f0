// Body of the append kernel, as a device function of one worker, so that a
// kernel can run it beside other work (the mixed decode + append launch). The
// kernel itself, and what it computes, are in append.hip.
#pragma once
#include "common.h"
#include "kernels.h"
#include "layout.h"
#include "tile_merge.h"

namespace abp {
namespace {
namespace appi {

constexpr int kD = 128;
constexpr int kTk = kAppendTileKv;   // 64
constexpr int kKStride = 136;        // sK row stride (uint16): 128 + 8 pad
constexpr int kVStride = 68;         // sVt row stride (uint16): 64 + 4 pad
constexpr float kRescaleLog2 = 8.f;  // lazy rescale threshold (log2 of the max p)


template <typename T>
__device__ __forceinline__ f32x4_t mfma(const uint4& a, const uint4& b, f32x4_t c);
template <>
__device__ __forceinline__ f32x4_t mfma<BF16>(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4_t mfma<F16>(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t word(const uint4& u, int j) {
  return j == 0 ? u.x : j == 1 ? u.y : j == 2 ? u.z : u.w;
}

// Split fp32 values into a 16-bit high part and the 16-bit rounding of the
// remainder, so that hi + lo carries ~16 significant bits: products of rotated
// operands keep fp32-level accuracy with three 16-bit matrix products.
template <typename T>
__device__ __forceinline__ void split8(const float v[8], uint4& hi, uint4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    h[w] = pack2<T>(v[2 * w], v[2 * w + 1]);
    l[w] = pack2<T>(v[2 * w] - lo_f32<T>(h[w]), v[2 * w + 1] - hi_f32<T>(h[w]));
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// Rotate q: `lo` holds elements j0..j0+7 (j0 < 64) and `hi` their partners
// j0+64..; results are split into (hi, lo) 16-bit parts for both halves.
template <typename T>
__device__ __forceinline__ void rope_pair(uint4& lo, uint4& hi, uint4& lo_r, uint4& hi_r,
                                          float pos, int j0, const ABP_CONST_AS float* rope) {
  float a[8], b[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    a[2 * w] = lo_f32<T>(word(lo, w));
    a[2 * w + 1] = hi_f32<T>(word(lo, w));
    b[2 * w] = lo_f32<T>(word(hi, w));
    b[2 * w + 1] = hi_f32<T>(word(hi, w));
  }
  float ra[8], rb[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float sn, cs;
    rope_sincos(pos, rope[2 * (j0 + e)], rope[2 * (j0 + e) + 1], &sn, &cs);
    ra[e] = __builtin_fmaf(a[e], cs, -b[e] * sn);
    rb[e] = __builtin_fmaf(b[e], cs, a[e] * sn);
  }
  split8<T>(ra, lo, lo_r);
  split8<T>(rb, hi, hi_r);
}

// Interleaved RoPE for q: `u` holds elements 2 j0 .. 2 j0 + 7, the adjacent
// pairs j0 .. j0 + 3; rotated in place into (hi, lo) 16-bit parts.
template <typename T>
__device__ __forceinline__ void rope_adjacent8(uint4& u, uint4& u_lo, float pos, int j0,
                                               const ABP_CONST_AS float* rope) {
  float r[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float x = lo_f32<T>(word(u, w)), y = hi_f32<T>(word(u, w));
    float sn, cs;
    rope_sincos(pos, rope[2 * (j0 + w)], rope[2 * (j0 + w) + 1], &sn, &cs);
    r[2 * w] = __builtin_fmaf(x, cs, -y * sn);
    r[2 * w + 1] = __builtin_fmaf(y, cs, x * sn);
  }
  split8<T>(r, u, u_lo);
}

// Interleaved RoPE for a K row: word w of u is the adjacent pair w of the
// lane's 4 pairs; out is in element order.
template <typename T>
__device__ __forceinline__ void rope_k_adjacent(const uint4& u, const float (&cs)[4],
                                                const float (&sn)[4], float out[8]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float x = lo_f32<T>(word(u, w)), y = hi_f32<T>(word(u, w));
    out[2 * w] = __builtin_fmaf(-y, sn[w], x * cs[w]);
    out[2 * w + 1] = __builtin_fmaf(x, sn[w], y * cs[w]);
  }
}

// Rotate the 4 rotary pairs a lane holds for one K row: u has elements
// 4c..4c+3 in words 0-1 and their partners 64+4c.. in words 2-3; cs / sn are
// the cosines and sines of the pairs' angles. out[e] / out[4 + e] are the
// rotated elements 4c + e and 64 + 4c + e.
template <typename T>
__device__ __forceinline__ void rope_k_pairs(const uint4& u, const float (&cs)[4],
                                             const float (&sn)[4], float out[8]) {
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

// Maximum over the 4 lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48) without
// LDS: each swap exchanges halves (32 lanes) or rows (16 lanes) between two
// copies of x, so the two results hold both partners of every lane.
__device__ __forceinline__ float max_over_groups(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto h = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = __builtin_fmaxf(__builtin_bit_cast(float, h[0]), __builtin_bit_cast(float, h[1]));
  const uint32_t w = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return __builtin_fmaxf(__builtin_bit_cast(float, r[0]), __builtin_bit_cast(float, r[1]));
}

// Waves per workgroup: 8 for both workers (one workgroup per CU). The
// pipelined worker's waves own 32 rows each (256-row tiles), the RoPE worker's
// 16 (128-row tiles: its q operands are hi and lo parts).
template <bool ROPE>
constexpr int append_waves() {
  return 8;
}

// The append worker with RoPE: 8 waves, 128 rows (tile_q tokens x G heads),
// wave w owning rows 16 w .. 16 w + 15, against 64-key blocks.
//
// K must be rotated by its position before the score products, so it comes
// into registers, is rotated there and is split into hi and lo 16-bit parts
// (S = Kh Qh + Kh Ql + Kl Qh keeps fp32-level accuracy); V is transposed on
// the way to LDS. Every thread stages 2 K rows (32 keys apart) and 4 V rows
// (4 head dims) of each block.
//
// Staging runs one block ahead of the products and its loads two blocks
// ahead: while block j's products read LDS stage j & 1, block j + 1's
// rotation (registers loaded during block j - 1) is interleaved with them and
// stored into stage (j + 1) & 1, and block j + 2's loads are issued into the
// registers block j came in. One barrier per block: it ends block j's reads of
// stage j & 1 and publishes stage (j + 1) & 1. The score products are written
// as fenced slots of 2 products and one small piece of the staging work; with
// two waves per SIMD the other wave's vector work fills the rest.
template <typename T, int G, bool CAUSAL, bool FASTPAGE, bool RIL>
__device__ __forceinline__ void append_worker_rope(const AttnArgs& a, int bid) {
  // K elements a staging thread reads per row: rotate-half RoPE takes 4 + 4
  // (both halves of its 4 pairs), interleaved RoPE 8 consecutive ones
  constexpr int kKPiece = RIL ? 8 : 4;
  constexpr int NW = append_waves<true>();
  constexpr int NT = 64 * NW;
  constexpr int kRows = 16 * NW;
  constexpr int TQ = kRows / G;
  constexpr int KSTEP = NT / 16;           // keys between a thread's K rows
  constexpr int KI = kTk / KSTEP;          // K rows a thread stages per block
  static_assert(KI == 2 && NW == 8, "staging map: 2 K rows of 32 keys apart, 8 V keys a wave");
  // a stage: rotated K as hi and lo parts [64][kKStride] each, then V^T
  // [128][kVStride]; one array per stage, each named at compile time where
  // used, so the compiler sees that stores into one stage never alias reads
  // of the other
  constexpr int kKElems = kTk * kKStride;
  constexpr int kVElems = kD * kVStride;
  __shared__ __align__(16) uint16_t ldsK0[2 * kKElems];
  __shared__ __align__(16) uint16_t ldsK1[2 * kKElems];
  __shared__ __align__(16) uint16_t ldsV0[kVElems];
  __shared__ __align__(16) uint16_t ldsV1[kVElems];
  __shared__ int s_last;
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  auto sK_of = [&](auto st) -> uint16_t* {
    if constexpr (decltype(st)::value == 0) return ldsK0;
    else return ldsK1;
  };
  auto sV_of = [&](auto st) -> uint16_t* {
    if constexpr (decltype(st)::value == 0) return ldsV0;
    else return ldsV1;
  };

  const ABP_CONST_AS int32_t* plan = const_as(a.plan);
  const ABP_CONST_AS int32_t* wseg = plan + plan[H_OFF_WSEG];
  const ABP_CONST_AS int32_t* segs = plan + plan[H_OFF_SEG];
  const ABP_CONST_AS int32_t* tiles = plan + plan[H_OFF_TILE];
  const ABP_CONST_AS float* rope = (const ABP_CONST_AS float*)(plan + plan[H_OFF_ROPE]);
  const ABP_CONST_AS int32_t* kv_indices = const_as(a.kv_indices);
  const ABP_CONST_AS int32_t* qo_indptr = const_as(a.qo_indptr);

  // XCD-major worker id: workgroup i runs on XCD i % 8
  const int W = a.workers;
  const int worker = (W % 8 == 0) ? (bid % 8) * (W / 8) + bid / 8 : bid;
  const int s_begin = wseg[worker], s_end = wseg[worker + 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g16 = lane >> 4;   // lane group 0..3
  const int l16 = lane & 15;
  const float cl2 = a.sm_scale_log2;
  const int P = a.page_size;
  const int shift = a.page_shift;
  const int tstride = a.token_stride;
  const uint16_t* __restrict__ kp = static_cast<const uint16_t*>(a.k_pages);
  const uint16_t* __restrict__ vp = static_cast<const uint16_t*>(a.v_pages);

  const float thr = kRescaleLog2 / cl2;  // lazy rescale threshold, raw score units
  // staging: K rows k_row + 32 i (i < 2), 16-byte chunk kc_chunk. A thread
  // stages both elements of the rotary pairs j = 4 kc_chunk + e (e < 4) of
  // its K rows (rotate-half: elements j and j + 64; interleaved: 2j and
  // 2j + 1, its plain 8 elements), so each angle is computed once; its second
  // row follows by angle addition with the rotation by 32 positions.
  // V: wave w stages keys 8 w + 4 v_kg + i (i < 4), head dims 4 v_q .. + 3.
  const int kc_chunk = tid & 15;
  const int k_row = tid >> 4;
  const int k_grp = k_row & ~15;  // 16-key group of the row (uniform over the wave)
  float kfhi[4], kflo[4], cst[4], sst[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int j = 4 * kc_chunk + e;
    kfhi[e] = rope[2 * j];
    kflo[e] = rope[2 * j + 1];
    rope_sincos((float)KSTEP, kfhi[e], kflo[e], &sst[e], &cst[e]);
  }
  const int v_kg = lane & 1;
  const int v_q = lane >> 1;

  // registers of one staged block
  struct Regs {
    uint4 k[KI];
    uint2 v[4];
  };
  Regs R0, R1;

  for (int s = s_begin; s < s_end; ++s) {
    const int tile = segs[4 * s];
    const int kv_begin = segs[4 * s + 1], kv_end = segs[4 * s + 2], slot = segs[4 * s + 3];
    const int b = tiles[4 * tile], h = tiles[4 * tile + 1], qt = tiles[4 * tile + 2];
    const int q0 = qo_indptr[b];
    const int qo_len = qo_indptr[b + 1] - q0;
    const int ip0 = a.kv_indptr[b];
    const int npg = a.kv_indptr[b + 1] - ip0;
    const int kv_len = npg > 0 ? (npg - 1) * P + a.kv_last_page_len[b] : 0;
    const int kv_pos0 = a.kv_pos_offset ? a.kv_pos_offset[b] : 0;
    // elements; the first piece of the lane's pairs (see above)
    const int koff_lane = (k_row & 15) * tstride + h * kD + kc_chunk * kKPiece;

    // ---- staging: global -> registers. Any kb is in bounds: groups past
    // the segment end re-read its last valid rows (masked, or never read).
    auto kload = [&](const uint16_t* p) -> uint4 {
      if constexpr (!RIL) {
        const uint2 lo = *reinterpret_cast<const uint2*>(p);
        const uint2 hi = *reinterpret_cast<const uint2*>(p + 64);
        return make_uint4(lo.x, lo.y, hi.x, hi.y);
      } else {
        return *reinterpret_cast<const uint4*>(p);
      }
    };
    auto gload = [&](int kb, Regs& R) __attribute__((always_inline)) {
      if constexpr (FASTPAGE) {
        // one page id per 16-key group (uniform over the wave), on the scalar
        // unit; the page ids are read first, so their scalar loads overlap
        const int last16 = (kv_end - 1) & ~15;
        int kk[KI], pid[KI];
#pragma unroll
        for (int i = 0; i < KI; ++i) {
          kk[i] = min(kb + k_grp + KSTEP * i, last16);
          pid[i] = kv_indices[ip0 + (kk[i] >> shift)];
        }
        const int kkv = min(kb + 16 * (wave >> 1), last16);
        const int pidv = kv_indices[ip0 + (kkv >> shift)];
#pragma unroll
        for (int i = 0; i < KI; ++i) {
          const int64_t base = (int64_t)pid[i] * a.page_stride + (int64_t)(kk[i] & (P - 1)) * tstride;
          R.k[i] = kload(kp + base + koff_lane);
        }
        const int64_t vb = (int64_t)pidv * a.page_stride + (int64_t)(kkv & (P - 1)) * tstride;
        // a key at or past kv_end takes the last key's values: slots past a
        // request's last token may hold NaN / inf bits, which p = 0 does not
        // cancel in P.V (K rows there only reach masked scores)
        const int rmax = kv_end - 1 - kkv;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          R.v[i] = *reinterpret_cast<const uint2*>(
              vp + vb + min(8 * (wave & 1) + 4 * v_kg + i, rmax) * tstride + h * kD + 4 * v_q);
      } else {
        auto row_of = [&](int key) -> int64_t {
          int page, off;
          if (shift >= 0) {
            page = key >> shift;
            off = key & (P - 1);
          } else {
            page = key / P;
            off = key - page * P;
          }
          return (int64_t)a.kv_indices[ip0 + page] * a.page_stride + (int64_t)off * tstride;
        };
#pragma unroll
        for (int i = 0; i < KI; ++i) {
          const int key = min(kb + k_row + KSTEP * i, kv_end - 1);
          R.k[i] = kload(kp + row_of(key) + h * kD + kc_chunk * kKPiece);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = min(kb + 8 * wave + 4 * v_kg + i, kv_end - 1);
          R.v[i] = *reinterpret_cast<const uint2*>(vp + row_of(key) + h * kD + 4 * v_q);
        }
      }
    };
    // ---- staging: registers -> LDS, cut into small pieces that the score
    // products are interleaved with: st_begin sets up the angles of K row
    // k_row, st_step moves them on by 32 positions, st_rot rotates one pair,
    // st_split splits one word of the rotated row into hi and lo parts,
    // st_store_k stores a K row, st_store_v two head dims of the V^T rows
    float cs[4], sn[4];
    float kr[8];
    uint32_t hw[4], lw[4];
    auto st_begin = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        rope_sincos((float)(kv_pos0 + kb + k_row), kfhi[e], kflo[e], &sn[e], &cs[e]);
    };
    auto st_step = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float cn = __builtin_fmaf(-sn[e], sst[e], cs[e] * cst[e]);
        sn[e] = __builtin_fmaf(cs[e], sst[e], sn[e] * cst[e]);
        cs[e] = cn;
      }
    };
    // pair e of K row i: rotate-half holds elements 4c + e (words 0-1) and
    // 64 + 4c + e (words 2-3), giving kr[e] and kr[4 + e]; interleaved holds
    // the pair in word e, giving kr[2e] and kr[2e + 1]
    auto st_rot = [&](const Regs& R, int i, int e) __attribute__((always_inline)) {
      const uint4& u = R.k[i];
      if constexpr (RIL) {
        const float x = lo_f32<T>(word(u, e)), y = hi_f32<T>(word(u, e));
        kr[2 * e] = __builtin_fmaf(-y, sn[e], x * cs[e]);
        kr[2 * e + 1] = __builtin_fmaf(x, sn[e], y * cs[e]);
      } else {
        const uint32_t wl = (e < 2) ? u.x : u.y;
        const uint32_t wh = (e < 2) ? u.z : u.w;
        const float x = (e & 1) ? hi_f32<T>(wl) : lo_f32<T>(wl);
        const float y = (e & 1) ? hi_f32<T>(wh) : lo_f32<T>(wh);
        kr[e] = __builtin_fmaf(-y, sn[e], x * cs[e]);
        kr[4 + e] = __builtin_fmaf(x, sn[e], y * cs[e]);
      }
    };
    auto st_split = [&](int w) __attribute__((always_inline)) {
      hw[w] = pack2<T>(kr[2 * w], kr[2 * w + 1]);
      lw[w] = pack2<T>(kr[2 * w] - lo_f32<T>(hw[w]), kr[2 * w + 1] - hi_f32<T>(hw[w]));
    };
    auto st_store_k = [&](int i, auto stage) __attribute__((always_inline)) {
      uint16_t* sK = sK_of(stage);
      uint16_t* sKlo = sK + kKElems;
      if constexpr (RIL) {
        // 8 consecutive elements, stored in place as one 16-byte piece
        const int at = (k_row + KSTEP * i) * kKStride + kc_chunk * 8;
        *reinterpret_cast<uint4*>(&sK[at]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        *reinterpret_cast<uint4*>(&sKlo[at]) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      } else {
        const int at = (k_row + KSTEP * i) * kKStride + kc_chunk * 4;
        *reinterpret_cast<uint2*>(&sK[at]) = make_uint2(hw[0], hw[1]);
        *reinterpret_cast<uint2*>(&sK[at + 64]) = make_uint2(hw[2], hw[3]);
        *reinterpret_cast<uint2*>(&sKlo[at]) = make_uint2(lw[0], lw[1]);
        *reinterpret_cast<uint2*>(&sKlo[at + 64]) = make_uint2(lw[2], lw[3]);
      }
    };
    // V^T: head dims 4 v_q + 2 j, + 1 of the 4 keys 8 wave + 4 v_kg + 0..3 as
    // one 8-byte piece each
    auto st_store_v = [&](const Regs& R, int j, auto stage) __attribute__((always_inline)) {
      uint16_t* V = sV_of(stage) + 8 * wave + 4 * v_kg;
      const uint32_t w0 = j ? R.v[0].y : R.v[0].x, w1 = j ? R.v[1].y : R.v[1].x;
      const uint32_t w2 = j ? R.v[2].y : R.v[2].x, w3 = j ? R.v[3].y : R.v[3].x;
      const int d = 4 * v_q + 2 * j;
      *reinterpret_cast<uint2*>(&V[d * kVStride]) = make_uint2(pair_lo(w0, w1), pair_lo(w2, w3));
      *reinterpret_cast<uint2*>(&V[(d + 1) * kVStride]) =
          make_uint2(pair_hi(w0, w1), pair_hi(w2, w3));
    };
    // staging piece p of a block (p = 0 is st_begin, placed by the caller):
    // K row i takes pieces 1 + 10 i .. 10 + 10 i (the step to it, 4 pair
    // rotations, 4 splits, the store), then the two V^T pieces
    constexpr int kPieces = 1 + 10 * KI + 2;
    auto st_piece = [&](const Regs& R, int p, auto stage) __attribute__((always_inline)) {
      if (p >= 1 && p <= 10 * KI) {
        const int i = (p - 1) / 10, r = (p - 1) % 10;
        if (r == 0) {
          if (i > 0) st_step();
        } else if (r <= 4) {
          st_rot(R, i, r - 1);
        } else if (r <= 8) {
          st_split(r - 5);
        } else {
          st_store_k(i, stage);
        }
      } else if (p > 10 * KI && p < kPieces) {
        st_store_v(R, p - 1 - 10 * KI, stage);
      }
    };
    auto st_all = [&](const Regs& R, auto stage) __attribute__((always_inline)) {
#pragma unroll
      for (int p = 1; p < kPieces; ++p) st_piece(R, p, stage);
    };

    const int nblk = kv_end > kv_begin ? (kv_end - kv_begin + kTk - 1) / kTk : 0;

    // ---- Q fragment (B operand of S^T = K Q^T) for this wave's 16 rows,
    // rotated and split into hi (qf) and lo (qfl) parts. The q loads go out
    // first and the first two blocks' K/V loads next, so that the q rotation
    // waits for q alone and the blocks' latency overlaps it.
    uint4 qf[4], qfl[4];
    const int r_row = wave * 16 + l16;
    const int tloc_r = qt * TQ + r_row / G;
    int lim;
    float qpos;
    {
      const int tl = min(tloc_r, qo_len - 1);
      lim = kv_len - qo_len + tl;
      const uint16_t* qptr = static_cast<const uint16_t*>(a.q) +
                             ((int64_t)(q0 + tl) * a.num_qo_heads + h * G + (r_row % G)) * kD +
                             g16 * 8;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) qf[kc] = *reinterpret_cast<const uint4*>(qptr + kc * 32);
      qpos = a.q_pos ? (float)a.q_pos[q0 + tl] : (float)lim;
    }
    if (nblk > 0) {
      gload(kv_begin, R0);
      gload(kv_begin + kTk, R1);
    }
    if constexpr (RIL) {
      // chunk kc holds elements g16 * 8 + 32 kc .. + 7: pairs 4 g16 + 16 kc ..
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
        rope_adjacent8<T>(qf[kc], qfl[kc], qpos, 4 * g16 + 16 * kc, rope);
    } else {
      rope_pair<T>(qf[0], qf[2], qfl[0], qfl[2], qpos, g16 * 8, rope);
      rope_pair<T>(qf[1], qf[3], qfl[1], qfl[3], qpos, 32 + g16 * 8, rope);
    }
    // first row of the tile sees the fewest keys
    const int tile_min_lim = kv_len - qo_len + qt * TQ;

    float m = kNegInf;
    float lsum = 0.f;
    f32x4_t O[8];
#pragma unroll
    for (int md = 0; md < 8; ++md) O[md] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    if (nblk > 0) {
      st_begin(kv_begin);
      st_all(R0, S0{});
    }
    __syncthreads();

    // one block on stage `st`: R holds block j + 1 (rotated and stored into
    // the other stage beside the score products), Rn takes block j + 2
    auto block = [&](auto st, int kb, Regs& R, Regs& Rn) __attribute__((always_inline)) {
      using Other = std::integral_constant<int, 1 - decltype(st)::value>;
      // always issued (past the end it re-reads the last rows), so the wait
      // for R below is the same count on every block
      gload(kb + 2 * kTk, Rn);
      const uint16_t* sK = sK_of(st);
      const uint16_t* sKlo = sK + kKElems;
      const uint16_t* sVt = sV_of(st);
      // S^T = K Q^T: S[mb] holds keys kb + 16 mb + 4 g16 + j of row l16. Piece
      // (mb, kc) is 3 products (hi/lo parts); its operands are read one piece
      // ahead. Each fenced slot issues 2 products and one staging piece of
      // the next block (past the last block it fills the idle stage with
      // values nobody reads).
      f32x4_t S[4];
      uint4 kh[2], kl[2];
      auto rd = [&](int mb, int kc, int buf) __attribute__((always_inline)) {
        const int at = (mb * 16 + l16) * kKStride + kc * 32 + g16 * 8;
        kh[buf] = *reinterpret_cast<const uint4*>(&sK[at]);
        kl[buf] = *reinterpret_cast<const uint4*>(&sKlo[at]);
      };
      rd(0, 0, 0);
#pragma unroll
      for (int u = 0; u < 48; ++u) {
        const int pc = u / 3, t = u % 3;  // piece (mb, kc) = (pc / 4, pc % 4)
        const int mb = pc >> 2, kc = pc & 3, buf = pc & 1;
        if (t == 0) {
          if (kc == 0) S[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          if (pc < 15) rd((pc + 1) >> 2, (pc + 1) & 3, buf ^ 1);
        }
        const uint4& ka = t < 2 ? kh[buf] : kl[buf];
        const uint4& qb = t == 1 ? qfl[kc] : qf[kc];
        S[mb] = mfma<T>(ka, qb, S[mb]);
        if (u & 1) {
          const int sl = u >> 1;
          if (sl == 0) st_begin(kb + kTk);
          else st_piece(R, sl, Other{});
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // ---- online softmax over the block's 64 keys: masks (keys past the
      // segment end, causal limit), one reference check per row with a lazy
      // rescale, then the exponentials of each 32-key half, P packed as the
      // PV B operand (K-slots of lane group g16 are keys 4 g16..+3 and
      // 16 + 4 g16..+3 of the half)
      const bool edge = (kb + kTk > kv_end) || (CAUSAL && kb + kTk - 1 > tile_min_lim);
      if (edge) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int key = kb + mb * 16 + g16 * 4 + j;
            const bool dead = key >= kv_end || (CAUSAL && key > lim);
            if (dead) S[mb][j] = kNegInf;
          }
      }
      {
        float x = kNegInf;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          x = __builtin_fmaxf(x, __builtin_fmaxf(__builtin_fmaxf(S[mb][0], S[mb][1]),
                                                 __builtin_fmaxf(S[mb][2], S[mb][3])));
        const float mx = max_over_groups(x);
        // the reference max moves only when a score exceeds it by more than thr
        if (__builtin_amdgcn_ballot_w64(mx > m + thr)) {
          const float mn = __builtin_fmaxf(m, mx);
          const float alpha = mn == kNegInf ? 1.f : fast_exp2((m - mn) * cl2);
          m = mn;
          lsum *= alpha;
#pragma unroll
          for (int md = 0; md < 8; ++md) O[md] *= alpha;
        }
      }
      const float mc = (m == kNegInf ? 0.f : m) * cl2;
      uint4 pB[2];
      float p[2][4];  // [16-key group of the half][key]
      // piece i (0..1) of half hh's exponentials: 16-key group i; the row sum
      // and the packing follow with the second. The row sum is taken in fp32
      // of the unrounded p: lse must not carry P's 16-bit rounding.
      auto exps = [&](int hh, int i) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) p[i][j] = fast_exp2(__builtin_fmaf(S[2 * hh + i][j], cl2, -mc));
        if (i == 1) {
          lsum += ((p[0][0] + p[0][1]) + (p[0][2] + p[0][3])) +
                  ((p[1][0] + p[1][1]) + (p[1][2] + p[1][3]));
          pB[hh] = make_uint4(pack2<T>(p[0][0], p[0][1]), pack2<T>(p[0][2], p[0][3]),
                              pack2<T>(p[1][0], p[1][1]), pack2<T>(p[1][2], p[1][3]));
        }
      };
      // O^T += V^T P^T over half hh, 16 dims (md) at a time; the V^T operand
      // of each md is read one slot ahead, and the first half's slots carry
      // the second half's exponentials
      uint4 va[2];
      auto rdv = [&](int hh, int md, int buf) __attribute__((always_inline)) {
        const uint16_t* vrow = &sVt[(md * 16 + l16) * kVStride + hh * 32 + g16 * 4];
        const uint2 v0 = *reinterpret_cast<const uint2*>(vrow);
        const uint2 v1 = *reinterpret_cast<const uint2*>(vrow + 16);
        va[buf] = make_uint4(v0.x, v0.y, v1.x, v1.y);
      };
      rdv(0, 0, 0);
      exps(0, 0);
      exps(0, 1);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int md = 0; md < 8; ++md) {
          const int buf = md & 1;
          if (md < 7) rdv(hh, md + 1, buf ^ 1);
          else if (hh == 0) rdv(1, 0, buf ^ 1);
          O[md] = mfma<T>(va[buf], pB[hh], O[md]);
          if (hh == 0 && md < 2) exps(1, md);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // ends every wave's reads of this stage and publishes the other
      __syncthreads();
    };
    for (int kb = kv_begin; kb < kv_end; kb += 2 * kTk) {
      block(S0{}, kb, R1, R0);
      if (kb + kTk < kv_end) block(S1{}, kb + kTk, R0, R1);
    }

    // ---- finalize rows: o = O / l, lse = m * scale + ln l
    {
      float L = lsum;
      L += __shfl_xor(L, 16);
      L += __shfl_xor(L, 32);
      const bool valid = tloc_r < qo_len;
      const bool empty = !(L > 0.f);
      const float inv = empty ? 0.f : 1.f / L;
      const float lse = empty ? kNegInf : m * a.sm_scale + fast_log2(L) * kLn2;
      if (valid) {
        if (slot < 0) {
          const int64_t orow = (int64_t)(q0 + tloc_r) * a.num_qo_heads + h * G + (r_row % G);
#pragma unroll
          for (int md = 0; md < 8; ++md) {
            const int64_t off = orow * kD + md * 16 + g16 * 4;
            const f32x4_t v = O[md] * inv;
            if (a.out_dtype == ABP_F32) {
              *reinterpret_cast<float4*>(static_cast<float*>(a.o) + off) =
                  make_float4(v[0], v[1], v[2], v[3]);
            } else if (a.out_dtype == ABP_BF16) {
              *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.o) + off) =
                  make_uint2(pack2<BF16>(v[0], v[1]), pack2<BF16>(v[2], v[3]));
            } else {
              *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.o) + off) =
                  make_uint2(pack2<F16>(v[0], v[1]), pack2<F16>(v[2], v[3]));
            }
          }
          if (a.lse && g16 == 0) a.lse[orow] = lse;
        } else {
          const int64_t prow = (int64_t)slot * kRows + r_row;
#pragma unroll
          for (int md = 0; md < 8; ++md) {
            const f32x4_t v = O[md] * inv;
            *reinterpret_cast<float4*>(a.o_part + prow * kD + md * 16 + g16 * 4) =
                make_float4(v[0], v[1], v[2], v[3]);
          }
          if (g16 == 0) a.lse_part[prow] = lse;
        }
      }
    }
    if (slot >= 0 && plan[H_MERGE_KERNEL] == 0) {
      merge_if_last<kRows, NT>(a, tile, &s_last, [&](int r, int64_t* orow) {
        const int tloc = qt * TQ + r / G;
        if (tloc >= qo_len) return false;
        *orow = (int64_t)(q0 + tloc) * a.num_qo_heads + h * G + (r % G);
        return true;
      });
    }
  }
}

// Softmax reference of the pipelined worker. A row keeps its reference max m
// while every p = 2^(s * scale * log2 e - m) of the row stays at or below
// 2^kSumCheckLog2: a lane's partial row sum bounds each of its p, so one
// comparison per row and step replaces the row maximum; when it fails the step
// takes the exact maximum instead. fp32 keeps full relative precision over
// that range, and O and l stay far below overflow (at most
// 2^(kSumCheckLog2 + 32) for 2^32 keys of unit size). Before its first key a
// row's reference is kNoRef, finite and far below any score, so the first p
// overflows the check and the exact maximum is taken.
constexpr float kSumCheckLog2 = 16.f;
constexpr float kNoRef = -1.0e30f;

// LDS of the pipelined append worker: K and V stages of kTk * kD elements
// each (the third ones only with three stages) and the merge flag, declared by
// the kernel as separate arrays (ABP_APPEND_PIPE_LDS), so the compiler sees
// every stage as its own object; a kernel with other roles may lend it larger
// arrays of its own.
struct PipeLds {
  uint16_t *k0, *k1, *k2, *v0, *v1, *v2;
  int* last;
};

#define ABP_APPEND_PIPE_LDS(name, NS)                                                      \
  __shared__ __align__(16) uint16_t name##_k0[appi::kTk * appi::kD];                      \
  __shared__ __align__(16) uint16_t name##_k1[appi::kTk * appi::kD];                      \
  __shared__ __align__(16) uint16_t name##_k2[(NS) > 2 ? appi::kTk * appi::kD : 8];       \
  __shared__ __align__(16) uint16_t name##_v0[appi::kTk * appi::kD];                      \
  __shared__ __align__(16) uint16_t name##_v1[appi::kTk * appi::kD];                      \
  __shared__ __align__(16) uint16_t name##_v2[(NS) > 2 ? appi::kTk * appi::kD : 8];       \
  __shared__ int name##_last;                                                             \
  const appi::PipeLds name = {name##_k0, name##_k1, name##_k2, name##_v0,                \
                              name##_v1, name##_v2, &name##_last}

// The work of one append worker without RoPE: 8 waves, 256 rows (tile_q tokens
// x G heads), wave w owning rows 32 w .. 32 w + 31, against 64-key blocks.
//
// Software pipeline over 32-key half blocks t: step t issues the S products
// of half t + 1 and the P.V products of half t - 1 on the matrix cores while
// the vector unit runs the softmax of half t. A step is written as 8 slots,
// each holding 4 products, the exponentials of 2 of the lane's 16 scores and
// the operand reads of the slot two ahead, with scheduling fences between the
// slots, so every wave keeps both units busy and each LDS read has two slots
// of products to land. S is double-buffered in registers; P of each half
// waits one step in registers for its P.V products.
//
// Staging: K and V blocks go straight from global memory into LDS (global-to-
// LDS loads, rows of 256 bytes whose 16-byte chunks are XOR-swizzled by row:
// K chunk q of row r at q ^ (r & 15), V at q ^ 2 (r & 7); K operands are
// 16-byte reads, V^T operands transpose reads, both free of bank conflicts).
// K and V have two stages each, V one block behind K: during block j's steps
// the LDS holds K(j), K(j + 1), V(j - 1) and V(j). After the first step of
// block j, once every wave is past it (barrier), K(j + 2) and V(j + 1) are
// loaded into the stages of K(j) and V(j - 1); they have two steps to land.
template <typename T, int G, bool CAUSAL, bool FASTPAGE, int NS>
__device__ __forceinline__ void append_worker_pipe(const AttnArgs& a, int bid,
                                                   const PipeLds& lds) {
  static_assert(NS == 2 || NS == 3, "two or three K/V stages");
  constexpr int NW = 8;
  constexpr int kRows = 32 * NW;
  constexpr int TQ = kRows / G;
  uint16_t* const ldsK0 = lds.k0;
  uint16_t* const ldsK1 = lds.k1;
  uint16_t* const ldsK2 = lds.k2;
  uint16_t* const ldsV0 = lds.v0;
  uint16_t* const ldsV1 = lds.v1;
  uint16_t* const ldsV2 = lds.v2;
  int& s_last = *lds.last;
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  auto sK_of = [&](auto st) -> uint16_t* {
    if constexpr (decltype(st)::value == 0) return ldsK0;
    else if constexpr (decltype(st)::value == 1) return ldsK1;
    else return ldsK2;
  };
  auto sV_of = [&](auto st) -> uint16_t* {
    if constexpr (decltype(st)::value == 0) return ldsV0;
    else if constexpr (decltype(st)::value == 1) return ldsV1;
    else return ldsV2;
  };

  const ABP_CONST_AS int32_t* plan = const_as(a.plan);
  const ABP_CONST_AS int32_t* wseg = plan + plan[H_OFF_WSEG];
  const ABP_CONST_AS int32_t* segs = plan + plan[H_OFF_SEG];
  const ABP_CONST_AS int32_t* tiles = plan + plan[H_OFF_TILE];
  const ABP_CONST_AS int32_t* kv_indptr = const_as(a.kv_indptr);
  const ABP_CONST_AS int32_t* kv_indices = const_as(a.kv_indices);
  const ABP_CONST_AS int32_t* qo_indptr = const_as(a.qo_indptr);

  // XCD-major worker id: workgroup i runs on XCD i % 8
  const int W = a.workers;
  const int worker = (W % 8 == 0) ? (bid % 8) * (W / 8) + bid / 8 : bid;
  const int s_begin = wseg[worker], s_end = wseg[worker + 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g16 = lane >> 4;   // lane group 0..3
  const int l16 = lane & 15;
  const float cl2 = a.sm_scale_log2;
  const int P = a.page_size;
  const int shift = a.page_shift;
  const int tstride = a.token_stride;
  const uint16_t* __restrict__ kp = static_cast<const uint16_t*>(a.k_pages);
  const uint16_t* __restrict__ vp = static_cast<const uint16_t*>(a.v_pages);
  constexpr float kBig = float(1u << 16);  // 2^kSumCheckLog2
  static_assert(kSumCheckLog2 == 16.f, "kBig follows the threshold");

  // Per-lane LDS byte offsets, the same for every block and stage:
  //  * K operand of product kc: row 16 mb + l16 (mb in the immediate offset),
  //    chunk (4 kc + g16) ^ l16 = (g16 ^ l16) ^ 4 kc;
  //  * V^T operand of d-tile md: transpose read of keys 4 g16 + l16 / 4 (and
  //    + 16, + 32 h in the immediate offset) at head dims 16 md + 4 (l16 % 4),
  //    whose chunk 2 md + (l16 / 2) % 2 sits at position
  //    2 (md ^ (key & 7)) + (l16 / 2) % 2.
  uint32_t koff[4], voff[8];
  {
    const uint32_t x = uint32_t(g16 ^ l16);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) koff[kc] = uint32_t(l16) * 256u + ((x ^ uint32_t(4 * kc)) * 16u);
    const uint32_t key = uint32_t(4 * g16 + (l16 >> 2));
    const uint32_t c = key & 7u;
    const uint32_t b = uint32_t(l16 >> 1) & 1u;
#pragma unroll
    for (int md = 0; md < 8; ++md)
      voff[md] = (key * 128u + 16u * (uint32_t(md) ^ c) + 8u * b + 4u * uint32_t(l16 & 1)) * 2u;
  }
  // Refill loads: wave w fills rows 8 w .. 8 w + 7 of a stage, 4 rows per
  // instruction i (1 KB, lane l at byte 16 l): lane l takes row
  // r = 8 w + 4 i + l / 16 at chunk position l % 16, which holds the row's
  // logical chunk (l % 16) ^ swz(r). Element offsets within the wave's rows:
  uint32_t goffK[2], goffV[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 8 * wave + 4 * i + (lane >> 4);
    const int pos = lane & 15;
    goffK[i] = uint32_t((4 * i + (lane >> 4)) * tstride + ((pos ^ (r & 15)) * 8));
    goffV[i] = uint32_t((4 * i + (lane >> 4)) * tstride + ((pos ^ (2 * (r & 7))) * 8));
  }

  for (int s = s_begin; s < s_end; ++s) {
    const int tile = segs[4 * s];
    const int kv_begin = segs[4 * s + 1], kv_end = segs[4 * s + 2], slot = segs[4 * s + 3];
    const int b = tiles[4 * tile], h = tiles[4 * tile + 1], qt = tiles[4 * tile + 2];
    const int q0 = qo_indptr[b];
    const int qo_len = qo_indptr[b + 1] - q0;
    const int ip0 = kv_indptr[b];
    const int npg = kv_indptr[b + 1] - ip0;
    const int kv_len = npg > 0 ? (npg - 1) * P + a.kv_last_page_len[b] : 0;

    // ---- Q fragments (B operand of S^T = K Q^T) for this wave's 32 rows
    uint4 qf[2][4];
    int lim[2];
    int tloc_r[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int r = wave * 32 + nb * 16 + l16;
      const int tloc = qt * TQ + r / G;
      const int tl = min(tloc, qo_len - 1);
      tloc_r[nb] = tloc;
      lim[nb] = kv_len - qo_len + tl;
      const uint16_t* qptr = static_cast<const uint16_t*>(a.q) +
                             ((int64_t)(q0 + tl) * a.num_qo_heads + h * G + (r % G)) * kD + g16 * 8;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) qf[nb][kc] = *reinterpret_cast<const uint4*>(qptr + kc * 32);
    }
    // first row of the tile sees the fewest keys
    const int tile_min_lim = kv_len - qo_len + qt * TQ;

    float m[2] = {kNoRef, kNoRef};
    float mc[2] = {kNoRef * cl2, kNoRef * cl2};  // m * scale * log2 e
    float lsum[2] = {0.f, 0.f};
    f32x4_t O[8][2];
#pragma unroll
    for (int md = 0; md < 8; ++md)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) O[md][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // ---- global -> LDS: K or V rows kb + 8 w .. + 7 of this wave into a
    // stage. When all 8 rows are keys of the segment they share one page
    // (pages of >= 16 keys, rows 8-aligned): one page lookup, per-lane offsets
    // from the table above. Otherwise each lane translates its row, and rows
    // at or past kv_end re-read the last key (in bounds; their scores are
    // masked and their values finite even where the slot holds no token).
    // (fast path: unsigned 32 x 32 -> 64-bit scalar arithmetic on bases
    // fixed per segment; page ids and strides are non-negative)
    const char* const kseg = reinterpret_cast<const char*>(kp + h * kD);
    const char* const vseg = reinterpret_cast<const char*>(vp + h * kD);
    const ABP_CONST_AS uint32_t* const pids =
        reinterpret_cast<const ABP_CONST_AS uint32_t*>(kv_indices + ip0);
    const uint32_t page_bytes = uint32_t(a.page_stride) * 2u;
    const uint32_t row_bytes = uint32_t(tstride) * 2u;
    auto dload = [&](const uint16_t* src, uint16_t* dst, int kb, bool is_v) {
      const int r0 = kb + 8 * wave;
      if (FASTPAGE && r0 + 7 < kv_end) {
        const uint32_t pid = pids[uint32_t(r0) >> shift];
        const char* sb = (is_v ? vseg : kseg) + (uint64_t(pid) * page_bytes +
                                                 (uint32_t(r0) & uint32_t(P - 1)) * row_bytes);
        const uint16_t* sbe = reinterpret_cast<const uint16_t*>(sb);
#pragma unroll
        for (int i = 0; i < 2; ++i)
          __builtin_amdgcn_global_load_lds(sbe + (is_v ? goffV[i] : goffK[i]),
                                           (ABP_LDS void*)(dst + (8 * wave + 4 * i) * kD), 16, 0, 0);
      } else {
        const int pos = lane & 15;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = 8 * wave + 4 * i + (lane >> 4);
          const int q = is_v ? (pos ^ (2 * (r & 7))) : (pos ^ (r & 15));
          const int key = min(kb + r, kv_end - 1);
          int page, off;
          if (shift >= 0) {
            page = key >> shift;
            off = key & (P - 1);
          } else {
            page = key / P;
            off = key - page * P;
          }
          const int64_t rb = (int64_t)a.kv_indices[ip0 + page] * a.page_stride +
                             (int64_t)off * tstride + h * kD;
          __builtin_amdgcn_global_load_lds(src + rb + q * 8,
                                           (ABP_LDS void*)(dst + (8 * wave + 4 * i) * kD), 16, 0, 0);
        }
      }
    };

    // S^T of half hh of the block in stage sK (used outside the slotted steps)
    auto qk = [&](const uint16_t* sK, int hh, f32x4_t (&S)[2][2]) __attribute__((always_inline)) {
      const char* base = reinterpret_cast<const char*>(sK);
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const uint4 ka = *reinterpret_cast<const uint4*>(base + koff[kc] + (2 * hh + mb) * 4096);
          const f32x4_t z = f32x4_t{0.f, 0.f, 0.f, 0.f};
          S[mb][0] = mfma<T>(ka, qf[0][kc], kc == 0 ? z : S[mb][0]);
          S[mb][1] = mfma<T>(ka, qf[1][kc], kc == 0 ? z : S[mb][1]);
        }
    };
    // V^T operand of d-tile md, half hh of the block in stage sV
    auto vread = [&](const uint16_t* sV, int hh, int md) __attribute__((always_inline)) -> uint4 {
      const char* base = reinterpret_cast<const char*>(sV) + hh * 8192;
      const v4i16_t a4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ABP_LDS v4i16_t*)(base + voff[md]));
      const v4i16_t b4 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((ABP_LDS v4i16_t*)(base + voff[md] + 4096));
      const uint2 av = __builtin_bit_cast(uint2, a4), bv = __builtin_bit_cast(uint2, b4);
      return make_uint4(av.x, av.y, bv.x, bv.y);
    };
    // O^T += V^T P^T over half hh of the block in stage sV (the last half)
    auto pv = [&](const uint16_t* sV, int hh, const uint4 (&pB)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int md = 0; md < 8; ++md) {
        const uint4 va = vread(sV, hh, md);
        O[md][0] = mfma<T>(va, pB[0], O[md][0]);
        O[md][1] = mfma<T>(va, pB[1], O[md][1]);
      }
    };
    // Causal and segment-end masks of one half (keys kbh .. kbh + 31), taken
    // only on halves that cross a limit: kbh > edge_from.
    const int edge_from = CAUSAL ? min(kv_end - 32, tile_min_lim - 31) : kv_end - 32;
    auto mask = [&](f32x4_t (&S)[2][2], int kbh) __attribute__((always_inline)) {
      if (kbh > edge_from) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int key = kbh + mb * 16 + g16 * 4 + j;
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
              if (key >= kv_end || (CAUSAL && key > lim[nb])) S[mb][nb][j] = kNegInf;
          }
      }
    };
    auto partial_sums = [&](const float (&p)[2][2][4], float (&part)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        part[nb] = ((p[0][nb][0] + p[0][nb][1]) + (p[0][nb][2] + p[0][nb][3])) +
                   ((p[1][nb][0] + p[1][nb][1]) + (p[1][nb][2] + p[1][nb][3]));
    };

    // One pipeline step: the softmax of S_cur (keys kbh ..) beside the S
    // products of the next half (K half qh of stage sK, into S_nxt) and, with
    // PV, the P.V products of the previous half (V half vh of stage sV with
    // P pB_prev). Slot i: products (kc = i / 2, mb = i % 2) of S and d-tile i
    // of P.V, the scores (mb = i / 4, nb = (i / 2) % 2, j = 2 (i % 2) + 0, 1)
    // of S_cur, and the operand reads of slot i + 2.
    auto step = [&](auto with_pv, f32x4_t (&S_cur)[2][2], int kbh, uint4 (&pB_out)[2],
                    const uint16_t* sK, int qh, f32x4_t (&S_nxt)[2][2], const uint16_t* sV,
                    int vh, const uint4 (&pB_prev)[2]) __attribute__((always_inline)) {
      constexpr bool PV = decltype(with_pv)::value;
      mask(S_cur, kbh);
      const char* kbase = reinterpret_cast<const char*>(sK) + 2 * qh * 4096;
      auto kread = [&](int i) __attribute__((always_inline)) -> uint4 {
        return *reinterpret_cast<const uint4*>(kbase + koff[i >> 1] + (i & 1) * 4096);
      };
      uint4 kf[3], vf[3];
      kf[0] = kread(0);
      kf[1] = kread(1);
      if constexpr (PV) {
        vf[0] = vread(sV, vh, 0);
        vf[1] = vread(sV, vh, 1);
      }
      float p[2][2][4];
      float part[2] = {0.f, 0.f};
      uint32_t pk[2][4];  // P of the step, packed pairs, as they are produced
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        if (i + 2 < 8) {
          kf[(i + 2) % 3] = kread(i + 2);
          if constexpr (PV) vf[(i + 2) % 3] = vread(sV, vh, i + 2);
        }
        const int emb = i >> 2, enb = (i >> 1) & 1, ej = 2 * (i & 1);
        p[emb][enb][ej] = fast_exp2(__builtin_fmaf(S_cur[emb][enb][ej], cl2, -mc[enb]));
        p[emb][enb][ej + 1] = fast_exp2(__builtin_fmaf(S_cur[emb][enb][ej + 1], cl2, -mc[enb]));
        part[enb] += p[emb][enb][ej] + p[emb][enb][ej + 1];
        pk[enb][2 * emb + (i & 1)] = pack2<T>(p[emb][enb][ej], p[emb][enb][ej + 1]);
        const int kc = i >> 1, qmb = i & 1;
        const f32x4_t z = f32x4_t{0.f, 0.f, 0.f, 0.f};
        S_nxt[qmb][0] = mfma<T>(kf[i % 3], qf[0][kc], kc == 0 ? z : S_nxt[qmb][0]);
        S_nxt[qmb][1] = mfma<T>(kf[i % 3], qf[1][kc], kc == 0 ? z : S_nxt[qmb][1]);
        if constexpr (PV) {
          O[i][0] = mfma<T>(vf[i % 3], pB_prev[0], O[i][0]);
          O[i][1] = mfma<T>(vf[i % 3], pB_prev[1], O[i][1]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // every p <= the lane's partial sum <= 2^kSumCheckLog2 keeps the
      // reference; !(x <= kBig) also catches an overflow to inf (and a row
      // still at kNoRef overflows)
      const bool moved = __builtin_amdgcn_ballot_w64(!(part[0] <= kBig) | !(part[1] <= kBig)) != 0;
      float alpha[2];
      if (moved) {
        // exact row maximum over the half (4 lane groups), then evaluate again
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          float x = __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(S_cur[0][nb][0], S_cur[0][nb][1]),
                                                    __builtin_fmaxf(S_cur[0][nb][2], S_cur[0][nb][3])),
                                    __builtin_fmaxf(__builtin_fmaxf(S_cur[1][nb][0], S_cur[1][nb][1]),
                                                    __builtin_fmaxf(S_cur[1][nb][2], S_cur[1][nb][3])));
          x = max_over_groups(x);
          const float mn = __builtin_fmaxf(m[nb], x);
          alpha[nb] = fast_exp2((m[nb] - mn) * cl2);
          m[nb] = mn;
          mc[nb] = mn * cl2;
          lsum[nb] *= alpha[nb];
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              p[mb][nb][j] = fast_exp2(__builtin_fmaf(S_cur[mb][nb][j], cl2, -mc[nb]));
        }
        partial_sums(p, part);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int w = 0; w < 4; ++w) pk[nb][w] = pack2<T>(p[w >> 1][nb][2 * (w & 1)], p[w >> 1][nb][2 * (w & 1) + 1]);
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        // row sum in fp32 of the unrounded p: lse must not carry P's 16-bit rounding
        lsum[nb] += part[nb];
        // K-slots of lane group g16: keys 4 g16 .. + 3, then 16 + 4 g16 .. + 3
        pB_out[nb] = make_uint4(pk[nb][0], pk[nb][1], pk[nb][2], pk[nb][3]);
      }
      // O took the P.V products of the previous half against the old reference
      if (moved) {
#pragma unroll
        for (int md = 0; md < 8; ++md)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) O[md][nb] *= alpha[nb];
      }
    };

    const int nblk = kv_begin < kv_end ? (kv_end - kv_begin + kTk - 1) / kTk : 0;
    f32x4_t Sa[2][2], Sb[2][2];
    uint4 pB0[2], pB1[2];
    // Block j's K and V sit in stage j % NS. The prologue loads K(0) ..
    // K(NS - 1) and V(0) .. V(NS - 2); the barrier in the middle of block j
    // loads K(j + NS) and V(j + NS - 1) into the stages of K(j) and V(j - 1).
    if (nblk > 0) {
      dload(kp, sK_of(S0{}), kv_begin, false);
      dload(vp, sV_of(S0{}), kv_begin, true);
      if (nblk > 1) dload(kp, sK_of(S1{}), kv_begin + kTk, false);
      if constexpr (NS > 2) {
        if (nblk > 1) dload(vp, sV_of(S1{}), kv_begin + kTk, true);
        if (nblk > 2) dload(kp, sK_of(S2{}), kv_begin + 2 * kTk, false);
      }
    }
    // The global-to-LDS loads count as loads for the memory model, so a
    // barrier's release does not wait for them: each wave waits for its own
    // before the barrier that publishes them.
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    __syncthreads();
    if (nblk > 0) {
      // S of (0, h0), then step (0, h0): S of (0, h1), softmax of (0, h0)
      qk(sK_of(S0{}), 0, Sa);
      step(std::false_type{}, Sa, kv_begin, pB0, sK_of(S0{}), 1, Sb, sV_of(S0{}), 1, pB1);
    }
    // second half of block j (K(j + 1) and V(j) must have landed): barrier,
    // refills, then step (j, h1): S of (j + 1, h0) (a block past the end
    // reads a stale stage whose results are never used), softmax of (j, h1),
    // P.V of (j, h0). st, st1, stm: stages of block j, j + 1 and j - 1.
    auto half1 = [&](auto st, auto st1, auto stm, int j) __attribute__((always_inline)) {
      const int kb = kv_begin + j * kTk;
      // loads still allowed in flight: those of the previous middle barrier
      // (NS = 3 only; each refill is two instructions per wave)
      const int pend = (NS > 2 && j >= 1)
                           ? ((j - 1 + NS < nblk) ? 2 : 0) + ((j - 2 + NS < nblk) ? 2 : 0)
                           : 0;
      if (pend == 4) __builtin_amdgcn_s_waitcnt(0x0f74);       // vmcnt(4)
      else if (pend == 2) __builtin_amdgcn_s_waitcnt(0x0f72);  // vmcnt(2)
      else __builtin_amdgcn_s_waitcnt(0x0f70);                 // vmcnt(0)
      __syncthreads();
      if (j + NS < nblk) dload(kp, sK_of(st), kb + NS * kTk, false);
      if (j + NS - 1 < nblk) dload(vp, sV_of(stm), kb + (NS - 1) * kTk, true);
      step(std::true_type{}, Sb, kb + 32, pB1, sK_of(st1), 0, Sa, sV_of(st), 0, pB0);
    };
    // first half of block j >= 1: step (j, h0): S of (j, h1), softmax of
    // (j, h0), P.V of (j - 1, h1)
    auto half0 = [&](auto st, auto stm, int j) __attribute__((always_inline)) {
      const int kb = kv_begin + j * kTk;
      step(std::true_type{}, Sa, kb, pB0, sK_of(st), 1, Sb, sV_of(stm), 1, pB1);
    };
    if constexpr (NS == 2) {
      for (int j = 0; j < nblk; j += 2) {
        half1(S0{}, S1{}, S1{}, j);
        if (j + 1 < nblk) {
          half0(S1{}, S0{}, j + 1);
          half1(S1{}, S0{}, S0{}, j + 1);
          if (j + 2 < nblk) half0(S0{}, S1{}, j + 2);
        }
      }
    } else {
      for (int j = 0; j < nblk; j += 3) {
        half1(S0{}, S1{}, S2{}, j);
        if (j + 1 < nblk) {
          half0(S1{}, S0{}, j + 1);
          half1(S1{}, S2{}, S0{}, j + 1);
          if (j + 2 < nblk) {
            half0(S2{}, S1{}, j + 2);
            half1(S2{}, S0{}, S1{}, j + 2);
            if (j + 3 < nblk) half0(S0{}, S2{}, j + 3);
          }
        }
      }
    }
    if (nblk > 0) {
      // P.V of the last half; its stage is that of the last block
      const int last = (nblk - 1) % NS;
      if (last == 0) pv(sV_of(S0{}), 1, pB1);
      else if (NS == 2 || last == 1) pv(sV_of(S1{}), 1, pB1);
      else pv(sV_of(S2{}), 1, pB1);
    }
    // the next segment's loads overwrite the stages: every wave must be done
    __syncthreads();

    // ---- finalize rows: o = O / l, lse = m * scale + ln l
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float L = lsum[nb];
      L += __shfl_xor(L, 16);
      L += __shfl_xor(L, 32);
      const int r = wave * 32 + nb * 16 + l16;
      const bool valid = tloc_r[nb] < qo_len;
      const bool empty = !(L > 0.f);
      const float inv = empty ? 0.f : 1.f / L;
      const float lse = empty ? kNegInf : m[nb] * a.sm_scale + fast_log2(L) * kLn2;
      if (valid) {
        if (slot < 0) {
          const int64_t orow = (int64_t)(q0 + tloc_r[nb]) * a.num_qo_heads + h * G + (r % G);
#pragma unroll
          for (int md = 0; md < 8; ++md) {
            const int64_t off = orow * kD + md * 16 + g16 * 4;
            const f32x4_t v = O[md][nb] * inv;
            if (a.out_dtype == ABP_F32) {
              *reinterpret_cast<float4*>(static_cast<float*>(a.o) + off) =
                  make_float4(v[0], v[1], v[2], v[3]);
            } else if (a.out_dtype == ABP_BF16) {
              *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.o) + off) =
                  make_uint2(pack2<BF16>(v[0], v[1]), pack2<BF16>(v[2], v[3]));
            } else {
              *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.o) + off) =
                  make_uint2(pack2<F16>(v[0], v[1]), pack2<F16>(v[2], v[3]));
            }
          }
          if (a.lse && g16 == 0) a.lse[orow] = lse;
        } else {
          const int64_t prow = (int64_t)slot * kRows + r;
#pragma unroll
          for (int md = 0; md < 8; ++md) {
            const f32x4_t v = O[md][nb] * inv;
            *reinterpret_cast<float4*>(a.o_part + prow * kD + md * 16 + g16 * 4) =
                make_float4(v[0], v[1], v[2], v[3]);
          }
          if (g16 == 0) a.lse_part[prow] = lse;
        }
      }
    }
    if (slot >= 0 && plan[H_MERGE_KERNEL] == 0) {
      merge_if_last<kRows, 64 * NW>(a, tile, &s_last, [&](int r, int64_t* orow) {
        const int tloc = qt * TQ + r / G;
        if (tloc >= qo_len) return false;
        *orow = (int64_t)(q0 + tloc) * a.num_qo_heads + h * G + (r % G);
        return true;
      });
    }
  }
}

// The work of one append worker (a workgroup of append_waves<ROPE>() waves);
// bid is the workgroup's index among the launch's append workgroups; lds is
// the pipelined worker's LDS (the RoPE worker declares its own).
// NS: K/V stages of the pipelined worker. Two measured faster than three on
// the ragged causal append, also with the barriers' drain of in-flight refills
// taken out (734-738 against 693-708 us, same box): what the refills cost is
// their HBM traffic (it lowers the engine clock), not their latency.
template <typename T, int G, bool CAUSAL, bool ROPE, bool FASTPAGE, bool RIL, int NS = 2>
__device__ __forceinline__ void append_worker(const AttnArgs& a, int bid, const PipeLds& lds) {
  if constexpr (ROPE) append_worker_rope<T, G, CAUSAL, FASTPAGE, RIL>(a, bid);
  else append_worker_pipe<T, G, CAUSAL, FASTPAGE, NS>(a, bid, lds);
}

}  // namespace appi
}  // namespace
}  // namespace abp
