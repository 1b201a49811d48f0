// Host work-unit planner (pure C++, no HIP runtime calls).
//
// The paper summary (FlashInfer, "图谱动态｜学苑周刊 NO.266", section
// 动态负载均衡调度) describes a two-phase scheduler in the spirit of Stream-K:
// on the CPU, cut attention into work units from the length distribution and
// spread them over the compute units; on the GPU, a persistent kernel with a
// fixed grid follows the plan. The rule implemented here:
//
//  * tiles in order (request, kv-head group, query tile); a group is the
//    kernel's heads per tile (decode: 4 consecutive kv heads when the count is
//    a multiple of 4, else 1; append: 1); a tile's extent is the number of keys
//    its last row may see, and it costs max(1, ceil(extent / tile_kv)) blocks;
//  * the N blocks are split into equal contiguous ranges of quota = ceil(N / W)
//    blocks, one per worker;
//  * a segment is one tile's share of one worker's range; a tile cut into
//    several segments writes fp32 partial states to consecutive slots (in key
//    order) and is merged afterwards.
//
// Append plans with load balancing co-schedule query tiles that read the same
// keys: K workers of one XCD (K = the largest of 8, 4, 2 dividing the workers
// per XCD) form a group, and the Stream-K split runs over groups and K-tile
// units instead of workers and tiles. A unit is K consecutive query tiles of
// one (request, kv head) (the tiles of a (request, kv head) left over after
// its whole units are queued, and every K queued tiles form a unit, so those
// mix kv heads); slot i of an even unit, and slot K - 1 - i of an odd one, is
// lane i, worker K g + i of group g (under a causal mask a unit's tiles grow
// by one block per slot; mirrored, every lane runs about as many blocks over
// two units, so the lanes of a group stay close together in time).
// A unit costs the blocks of its longest tile; a group's range [g q, (g + 1) q)
// of unit blocks (q = ceil(units' blocks / (W / K))) gives each lane the same
// block range of its own tile, clipped to that tile's blocks. The lanes of a
// unit start its tiles together and walk the same keys at the same pace, so
// one read from HBM serves them all through the XCD's L2.
//
// The planner writes straight into the caller's host workspace and allocates
// nothing.
#include "plan.h"

#include <math.h>
#include <string.h>

#include <algorithm>

namespace abp {

namespace {

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline int64_t align4(int64_t x) { return (x + 3) & ~int64_t(3); }

constexpr int kCoLanesMax = 8;  // workers per co-scheduled group, at most

// Workers per co-scheduled group for this plan (1: plain Stream-K). The
// kernels place worker w on XCD w / (W / 8) when W is a multiple of 8, so a
// group of K consecutive workers shares one L2 when K divides W / 8.
int co_lanes(const Config& cfg, const Layout& L) {
  if (cfg.kind != ABP_KIND_APPEND || L.no_split || L.workers % 8 != 0) return 1;
  const int32_t per_xcd = L.workers / 8;
  for (int k = kCoLanesMax; k > 1; k >>= 1)
    if (per_xcd % k == 0) return k;
  return 1;
}

constexpr int32_t kMaxKvLen = 1 << 24;

}  // namespace

int check_params(int kind, const abp_params* p, Config* cfg, std::string* err) {
  if (!p || !cfg) {
    *err = "params is NULL";
    return ABP_ERR_INVALID_ARG;
  }
  if (kind != ABP_KIND_DECODE && kind != ABP_KIND_APPEND && kind != ABP_KIND_BSR) {
    *err = "kind must be ABP_KIND_DECODE, ABP_KIND_APPEND or ABP_KIND_BSR";
    return ABP_ERR_INVALID_ARG;
  }
  if (p->num_qo_heads < 1 || p->num_kv_heads < 1) {
    *err = "head counts must be >= 1";
    return ABP_ERR_INVALID_ARG;
  }
  if (p->num_qo_heads % p->num_kv_heads != 0) {
    *err = "num_qo_heads must be a multiple of num_kv_heads";
    return ABP_ERR_INVALID_ARG;
  }
  const int32_t g = p->num_qo_heads / p->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8 && g != 16) {
    *err = "group size num_qo_heads/num_kv_heads must be 1, 2, 4, 8 or 16";
    return ABP_ERR_UNSUPPORTED;
  }
  if (p->head_dim != 128) {
    *err = "only head_dim 128 is built";
    return ABP_ERR_UNSUPPORTED;
  }
  if (p->page_size < 1) {
    *err = "page_size must be >= 1";
    return ABP_ERR_INVALID_ARG;
  }
  // one page of K (or V) must stay under 2 GiB: kernels address within a
  // page with 32-bit byte offsets
  if (int64_t(p->page_size) * p->num_kv_heads * p->head_dim * 2 >= (int64_t(1) << 31)) {
    *err = "page_size * num_kv_heads * head_dim * 2 bytes must be below 2 GiB";
    return ABP_ERR_UNSUPPORTED;
  }
  if (p->qkv_dtype != ABP_F16 && p->qkv_dtype != ABP_BF16) {
    *err = "qkv_dtype must be ABP_F16 or ABP_BF16";
    return ABP_ERR_UNSUPPORTED;
  }
  if (p->out_dtype != ABP_F16 && p->out_dtype != ABP_BF16 && p->out_dtype != ABP_F32) {
    *err = "out_dtype must be ABP_F16, ABP_BF16 or ABP_F32";
    return ABP_ERR_UNSUPPORTED;
  }
  if (p->rope < 0 || p->rope > 2) {
    *err = "rope must be 0, 1 or 2";
    return ABP_ERR_INVALID_ARG;
  }
  if (p->rope != 0 && !(p->rope_theta > 1.f)) {
    *err = "rope_theta must be > 1";
    return ABP_ERR_INVALID_ARG;
  }
  if (p->rope == 2 && !(p->rope_factor > 0.f && p->rope_low_freq_factor > 0.f &&
                        p->rope_high_freq_factor > p->rope_low_freq_factor &&
                        p->rope_old_context_len > 0.f)) {
    *err = "LLaMA 3.1 RoPE needs factor > 0, low_freq_factor > 0, high_freq_factor > "
           "low_freq_factor and old_context_len > 0";
    return ABP_ERR_INVALID_ARG;
  }
  if (p->causal != 0 && p->causal != 1) {
    *err = "causal must be 0 or 1";
    return ABP_ERR_INVALID_ARG;
  }
  if (p->rope_interleave != 0 && p->rope_interleave != 1) {
    *err = "rope_interleave must be 0 or 1";
    return ABP_ERR_INVALID_ARG;
  }
  if (p->kv_fp8 != 0 && p->kv_fp8 != 1) {
    *err = "kv_fp8 must be 0 or 1";
    return ABP_ERR_INVALID_ARG;
  }
  if (p->kv_fp8 == 1) {
    if (kind != ABP_KIND_DECODE || p->rope != 0) {
      *err = "an fp8 KV cache is supported by decode without RoPE";
      return ABP_ERR_UNSUPPORTED;
    }
    if (!(p->k_scale > 0.f) || !(p->v_scale > 0.f)) {
      *err = "k_scale and v_scale must be > 0 with an fp8 KV cache";
      return ABP_ERR_INVALID_ARG;
    }
  }
  if (kind == ABP_KIND_BSR && (p->causal != 0 || p->rope != 0)) {
    *err = "block-sparse attention takes its mask from the BSR pattern: causal and rope must be 0";
    return ABP_ERR_UNSUPPORTED;
  }
  cfg->kind = kind;
  cfg->hq = p->num_qo_heads;
  cfg->hkv = p->num_kv_heads;
  cfg->group = g;
  cfg->head_dim = p->head_dim;
  cfg->page_size = p->page_size;
  cfg->qkv_dtype = p->qkv_dtype;
  cfg->out_dtype = p->out_dtype;
  cfg->sm_scale = p->sm_scale > 0.f ? p->sm_scale : (float)(1.0 / sqrt((double)p->head_dim));
  cfg->causal = kind == ABP_KIND_APPEND ? p->causal : 0;
  cfg->rope = p->rope;
  cfg->rope_theta = p->rope_theta;
  cfg->rope_interleave = p->rope != 0 ? p->rope_interleave : 0;
  if (p->kv_fp8 == 1) {
    cfg->kv_fp8 = 1;
    cfg->k_scale = p->k_scale;
    cfg->v_scale = p->v_scale;
  }
  if (p->rope == 2) {
    cfg->rope_factor = p->rope_factor;
    cfg->rope_low = p->rope_low_freq_factor;
    cfg->rope_high = p->rope_high_freq_factor;
    cfg->rope_old_ctx = p->rope_old_context_len;
  }
  return ABP_OK;
}

int make_layout_caps(const Config& cfg, int64_t max_tiles, int32_t workers, Layout* out,
                     std::string* err) {
  if (max_tiles < 0 || workers < 1) {
    *err = "capacities must be >= 0 and num_workers >= 1";
    return ABP_ERR_INVALID_ARG;
  }
  Layout L;
  L.workers = workers;
  if (cfg.kind == ABP_KIND_DECODE) {
    L.tile_q = 1;
    L.tile_kv = kDecodeTileKv;
    L.tile_heads = decode_tile_heads(cfg.hkv);
    L.rows = cfg.group * L.tile_heads;
  } else {
    L.rows = append_rows(cfg.rope != 0);
    L.tile_q = L.rows / cfg.group;
    L.tile_kv = kAppendTileKv;
  }
  const int64_t max_segs = max_tiles + workers - 1;
  // a tile cut k >= 2 times uses k slots and k - 1 of the W - 1 inner worker boundaries
  const int64_t max_partials = std::min<int64_t>(max_segs, 2 * int64_t(workers - 1));
  const int64_t max_merges = std::min<int64_t>(max_tiles, workers - 1);
  if (max_segs > (int64_t(1) << 28)) {
    *err = "capacities too large";
    return ABP_ERR_INVALID_ARG;
  }
  L.max_tiles = (int32_t)max_tiles;
  L.max_segs = (int32_t)max_segs;
  L.max_partials = (int32_t)max_partials;
  L.max_merges = (int32_t)max_merges;
  int64_t off = HEADER_INTS;
  L.off_wseg = off;
  off += align4(workers + 1);
  L.off_seg = off;
  off += 4 * max_segs;
  L.off_tile = off;
  off += 4 * max_tiles;
  L.off_ntile = off;
  off += align4(max_tiles);
  L.off_merge = off;
  off += 4 * max_merges;
  L.off_rope = off;
  off += 2 * kMaxRopePairs;
  L.off_cnt = off;
  off += align4(max_tiles);
  L.off_aux = off;
  if (cfg.kind == ABP_KIND_BSR) {
    L.aux_cap = (int32_t)(max_tiles / cfg.hkv);
    off += align4(int64_t(L.aux_cap) + 1) + align4(L.aux_cap);
  }
  L.plan_ints = off;
  L.plan_bytes = uint64_t(off) * 4;
  L.partial_offset = (L.plan_bytes + 255) & ~uint64_t(255);
  L.partial_bytes = uint64_t(max_partials) * L.rows * (cfg.head_dim + 1) * 4;
  L.dev_bytes = L.partial_offset + ((L.partial_bytes + 255) & ~uint64_t(255));
  *out = L;
  return ABP_OK;
}

int make_layout(const Config& cfg, int32_t max_batch, int32_t max_qo_tokens, int32_t workers,
                Layout* out, std::string* err) {
  if (max_batch < 0 || workers < 1 || (cfg.kind != ABP_KIND_DECODE && max_qo_tokens < 0)) {
    *err = "max_batch and max_qo_tokens must be >= 0 and num_workers >= 1";
    return ABP_ERR_INVALID_ARG;
  }
  int64_t max_tiles;
  if (cfg.kind == ABP_KIND_DECODE) {
    max_tiles = int64_t(max_batch) * (cfg.hkv / decode_tile_heads(cfg.hkv));
  } else {
    // sum_b ceil(qo_b / tile_q) <= sum_qo / tile_q + batch
    const int64_t tile_q = append_rows(cfg.rope != 0) / cfg.group;
    max_tiles = (ceil_div(max_qo_tokens, tile_q) + max_batch) * int64_t(cfg.hkv);
  }
  return make_layout_caps(cfg, max_tiles, workers, out, err);
}

uint64_t fingerprint(const Config& c, const Layout& L) {
  uint64_t h = 1469598103934665603ull;
  auto mix = [&h](uint64_t v) {
    for (int i = 0; i < 8; ++i) {
      h ^= (v >> (8 * i)) & 0xff;
      h *= 1099511628211ull;
    }
  };
  uint32_t scale_bits, theta_bits, l31[4], kvs[2];
  memcpy(&kvs[0], &c.k_scale, 4);
  memcpy(&kvs[1], &c.v_scale, 4);
  memcpy(&scale_bits, &c.sm_scale, 4);
  memcpy(&theta_bits, &c.rope_theta, 4);
  memcpy(&l31[0], &c.rope_factor, 4);
  memcpy(&l31[1], &c.rope_low, 4);
  memcpy(&l31[2], &c.rope_high, 4);
  memcpy(&l31[3], &c.rope_old_ctx, 4);
  const int64_t vals[] = {c.kind,      c.hq,          c.hkv,          c.head_dim,   c.page_size,
                          c.qkv_dtype, c.out_dtype,   scale_bits,     c.causal,     c.rope,
                          theta_bits,  L.workers,     L.max_tiles,    L.max_segs,   L.max_partials,
                          L.max_merges, L.tile_q,     L.tile_kv,      L.rows,       L.plan_ints,
                          (int64_t)L.partial_offset, l31[0], l31[1], l31[2], l31[3],
                          L.off_aux, L.aux_cap, c.kv_fp8, kvs[0], kvs[1], c.rope_interleave};
  for (int64_t v : vals) mix((uint64_t)v);
  return h;
}

namespace {

// The co-scheduled split of an append plan over groups of K workers (file
// header): writes the tile records, the segments grouped by worker with their
// partial slots, wseg, the per-tile partial counts and the merge list into the
// zeroed blob. The arrival counters serve as scratch and are zero again on
// return.
void co_schedule(const Config& cfg, const Layout& L, int32_t K, int32_t batch,
                 const int32_t* qo_indptr, const int32_t* kv_indptr, const int32_t* lpl,
                 int32_t* blob, int64_t* n_seg, int64_t* n_slot, int64_t* n_merge,
                 int64_t* max_nseg, int64_t* quota_out) {
  const int64_t P = cfg.page_size, Tq = L.tile_q, Tk = L.tile_kv;
  const int32_t W = L.workers;
  int32_t* wseg = blob + L.off_wseg;
  int32_t* seg = blob + L.off_seg;
  int32_t* tile = blob + L.off_tile;
  int32_t* ntile = blob + L.off_ntile;
  int32_t* mrg = blob + L.off_merge;
  int32_t* used = blob + L.off_cnt;

  int64_t T = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t nqt = ceil_div(int64_t(qo_indptr[b + 1]) - qo_indptr[b], Tq);
    for (int32_t h = 0; h < cfg.hkv; h += L.tile_heads)
      for (int64_t qt = 0; qt < nqt; ++qt, ++T) {
        int32_t* tr = tile + 4 * T;
        tr[0] = b;
        tr[1] = h;
        tr[2] = (int32_t)qt;
        tr[3] = -1;
      }
  }
  auto extent = [&](int64_t t) -> int64_t {
    const int32_t b = tile[4 * t];
    const int64_t n = int64_t(kv_indptr[b + 1]) - kv_indptr[b];
    const int64_t kv_len = n > 0 ? (n - 1) * P + lpl[b] : 0;
    const int64_t qo_len = int64_t(qo_indptr[b + 1]) - qo_indptr[b];
    return cfg.causal ? kv_len - qo_len + std::min((int64_t(tile[4 * t + 2]) + 1) * Tq, qo_len)
                      : kv_len;
  };
  auto blocks = [&](int64_t t) { return std::max<int64_t>(1, ceil_div(extent(t), Tk)); };

  // the units in order: fn(tiles of lanes 0 .. K - 1 (-1: idle lane), cost)
  auto walk = [&](auto&& fn) {
    int64_t u[kCoLanesMax], q[kCoLanesMax];
    int nq = 0;
    auto unit = [&](const int64_t* v) {
      int64_t c = 0;
      for (int j = 0; j < K; ++j)
        if (v[j] >= 0) c = std::max(c, blocks(v[j]));
      fn(v, c);
    };
    for (int64_t t0 = 0, t1; t0 < T; t0 = t1) {
      t1 = t0 + 1;
      while (t1 < T && tile[4 * t1] == tile[4 * t0] && tile[4 * t1 + 1] == tile[4 * t0 + 1]) ++t1;
      const int64_t whole = t0 + (t1 - t0) / K * K;
      for (int64_t i = t0; i < whole; i += K) {
        for (int j = 0; j < K; ++j) u[j] = i + j;
        unit(u);
      }
      for (int64_t i = whole; i < t1; ++i) {
        q[nq++] = i;
        if (nq == K) {
          unit(q);
          nq = 0;
        }
      }
    }
    if (nq > 0) {
      for (int j = nq; j < K; ++j) q[j] = -1;
      unit(q);
    }
  };
  int64_t N2 = 0;
  walk([&](const int64_t*, int64_t c) { N2 += c; });
  const int64_t groups = W / K;
  const int64_t quota = N2 > 0 ? ceil_div(N2, groups) : 1;
  // every (worker, tile, kv range) in unit order: fn(w, t, kv_begin, kv_end);
  // odd units give their slots to the lanes in reverse
  auto split = [&](auto&& fn) {
    int64_t g0 = 0, ui = 0;
    walk([&](const int64_t* v, int64_t c) {
      const int64_t g1 = g0 + c;
      const bool odd = (ui++ & 1) != 0;
      for (int64_t grp = g0 / quota; grp * quota < g1; ++grp) {
        const int64_t lo = std::max(g0, grp * quota) - g0;
        const int64_t hi = std::min(g1, (grp + 1) * quota) - g0;
        for (int j = 0; j < K; ++j) {
          const int64_t t = v[odd ? K - 1 - j : j];
          if (t < 0) continue;
          const int64_t nb = blocks(t);
          if (lo >= nb) continue;
          fn(grp * K + j, t, lo * Tk, std::min(std::min(hi, nb) * Tk, extent(t)));
        }
      }
      g0 = g1;
    });
  };
  split([&](int64_t w, int64_t t, int64_t, int64_t) {
    wseg[w + 1] += 1;
    ntile[t] += 1;
  });
  for (int32_t w = 0; w < W; ++w) wseg[w + 1] += wseg[w];
  int64_t slot = 0, m = 0, mx = 0;
  for (int64_t t = 0; t < T; ++t) {
    const int64_t n = ntile[t];
    mx = std::max(mx, n);
    if (n > 1) {
      tile[4 * t + 3] = (int32_t)slot;
      int32_t* mr = mrg + 4 * m++;
      mr[0] = (int32_t)t;
      mr[1] = (int32_t)slot;
      mr[2] = (int32_t)n;
      mr[3] = 0;
      slot += n;
    } else {
      ntile[t] = 0;
    }
  }
  // fill: wseg[w] walks worker w's records, ending at the next worker's start
  split([&](int64_t w, int64_t t, int64_t kb, int64_t ke) {
    int32_t* sr = seg + 4 * int64_t(wseg[w]++);
    sr[0] = (int32_t)t;
    sr[1] = (int32_t)kb;
    sr[2] = (int32_t)ke;
    sr[3] = ntile[t] > 1 ? tile[4 * t + 3] + used[t]++ : -1;
  });
  for (int32_t w = W; w > 0; --w) wseg[w] = wseg[w - 1];
  wseg[0] = 0;
  for (int64_t t = 0; t < T; ++t) used[t] = 0;
  *n_seg = wseg[W];
  *n_slot = slot;
  *n_merge = m;
  *max_nseg = mx;
  *quota_out = quota;
}

}  // namespace

int plan_compute(const Config& cfg, const Layout& L, int32_t batch, const int32_t* qo_indptr,
                 const int32_t* kv_indptr, const int32_t* lpl, int32_t* blob, abp_plan* plan,
                 std::string* err) {
  const bool append = cfg.kind != ABP_KIND_DECODE;
  if (batch < 0) {
    *err = "batch must be >= 0";
    return ABP_ERR_INVALID_ARG;
  }
  if (!blob || !plan || (batch > 0 && (!kv_indptr || !lpl)) || (append && !qo_indptr)) {
    *err = "NULL array";
    return ABP_ERR_INVALID_ARG;
  }
  if (!kv_indptr || kv_indptr[0] != 0) {
    *err = "kv_indptr[0] must be 0";
    return ABP_ERR_INVALID_ARG;
  }
  if (append && qo_indptr[0] != 0) {
    *err = "qo_indptr[0] must be 0";
    return ABP_ERR_INVALID_ARG;
  }
  const int32_t P = cfg.page_size;
  const int32_t Tq = L.tile_q, Tk = L.tile_kv, W = L.workers;
  const int32_t ngroups = cfg.hkv / L.tile_heads;  // kv-head groups (tiles) per query tile

  // validation and the block count N (pass 1)
  int64_t N = 0, T = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t n = int64_t(kv_indptr[b + 1]) - kv_indptr[b];
    if (n < 0) {
      *err = "kv_indptr must be non-decreasing";
      return ABP_ERR_INVALID_ARG;
    }
    int64_t kv_len = 0;
    if (n > 0) {
      if (lpl[b] < 1 || lpl[b] > P) {
        *err = "kv_last_page_len must lie in [1, page_size] for a request with pages";
        return ABP_ERR_INVALID_ARG;
      }
      kv_len = (n - 1) * P + lpl[b];
    }
    if (kv_len >= kMaxKvLen) {
      *err = "kv_len must be < 2^24";
      return ABP_ERR_INVALID_ARG;
    }
    int64_t qo_len = 1, nqt = 1;
    if (append) {
      qo_len = int64_t(qo_indptr[b + 1]) - qo_indptr[b];
      if (qo_len < 0) {
        *err = "qo_indptr must be non-decreasing";
        return ABP_ERR_INVALID_ARG;
      }
      if (cfg.causal && qo_len > kv_len) {
        *err = "causal append needs qo_len <= kv_len for every request";
        return ABP_ERR_INVALID_ARG;
      }
      nqt = ceil_div(qo_len, Tq);
    }
    for (int64_t qt = 0; qt < nqt; ++qt) {
      const int64_t e = cfg.causal ? kv_len - qo_len + std::min((qt + 1) * Tq, qo_len) : kv_len;
      N += int64_t(ngroups) * std::max<int64_t>(1, ceil_div(e, Tk));
    }
    T += nqt * ngroups;
  }
  if (T > L.max_tiles) {
    *err = "batch exceeds the workspace capacities (max_batch / max_qo_tokens)";
    return ABP_ERR_WORKSPACE_TOO_SMALL;
  }
  if (L.no_split && T > W) {
    *err = "one worker per tile needs num_workers >= the number of tiles";
    return ABP_ERR_INVALID_ARG;
  }
  const int64_t quota = N > 0 ? ceil_div(N, W) : 1;

  // the aux region (block-sparse plans) holds inputs of this call: keep it
  memset(blob, 0, sizeof(int32_t) * size_t(L.off_aux));
  int32_t* wseg = blob + L.off_wseg;
  int32_t* seg = blob + L.off_seg;
  int32_t* tile = blob + L.off_tile;
  int32_t* ntile = blob + L.off_ntile;
  int32_t* mrg = blob + L.off_merge;

  // tiles, segments, partial slots, merge list (pass 2)
  int64_t t = 0, s = 0, g0 = 0, slot = 0, m = 0, max_nseg = 0;
  int64_t plan_quota = quota;
  const int32_t lanes = co_lanes(cfg, L);
  if (lanes > 1) {
    co_schedule(cfg, L, lanes, batch, qo_indptr, kv_indptr, lpl, blob, &s, &slot, &m, &max_nseg,
                &plan_quota);
    t = T;
  }
  for (int32_t b = 0; b < batch && lanes == 1; ++b) {
    const int64_t n = int64_t(kv_indptr[b + 1]) - kv_indptr[b];
    const int64_t kv_len = n > 0 ? (n - 1) * P + lpl[b] : 0;
    const int64_t qo_len = append ? int64_t(qo_indptr[b + 1]) - qo_indptr[b] : 1;
    const int64_t nqt = append ? ceil_div(qo_len, Tq) : 1;
    for (int32_t h = 0; h < cfg.hkv; h += L.tile_heads) {
      for (int64_t qt = 0; qt < nqt; ++qt, ++t) {
        const int64_t e = cfg.causal ? kv_len - qo_len + std::min((qt + 1) * Tq, qo_len) : kv_len;
        const int64_t g1 = g0 + std::max<int64_t>(1, ceil_div(e, Tk));
        // Stream-K: the workers whose block ranges meet [g0, g1); without
        // splitting, worker t takes tile t whole
        const int64_t w_first = L.no_split ? t : g0 / quota;
        const int64_t w_last = L.no_split ? t : (g1 - 1) / quota;
        const int64_t nseg = w_last - w_first + 1;
        max_nseg = std::max(max_nseg, nseg);
        int32_t* tr = tile + 4 * t;
        tr[0] = b;
        tr[1] = h;
        tr[2] = (int32_t)qt;
        tr[3] = nseg > 1 ? (int32_t)slot : -1;
        ntile[t] = nseg > 1 ? (int32_t)nseg : 0;
        if (nseg > 1) {
          int32_t* mr = mrg + 4 * m++;
          mr[0] = (int32_t)t;
          mr[1] = (int32_t)slot;
          mr[2] = (int32_t)nseg;
          mr[3] = 0;
        }
        for (int64_t w = w_first; w <= w_last; ++w, ++s) {
          const int64_t lo = L.no_split ? g0 : std::max(g0, w * quota);
          const int64_t hi = L.no_split ? g1 : std::min(g1, (w + 1) * quota);
          int32_t* sr = seg + 4 * s;
          sr[0] = (int32_t)t;
          sr[1] = (int32_t)((lo - g0) * Tk);
          sr[2] = (int32_t)std::min((hi - g0) * Tk, e);
          sr[3] = nseg > 1 ? (int32_t)slot++ : -1;
          wseg[w + 1] += 1;
        }
        g0 = g1;
      }
    }
  }
  if (lanes == 1)
    for (int32_t w = 0; w < W; ++w) wseg[w + 1] += wseg[w];

  // RoPE frequencies in revolutions per position, as fp32 hi + lo
  float* rope = reinterpret_cast<float*>(blob + L.off_rope);
  const int half = cfg.head_dim / 2;
  for (int j = 0; j < kMaxRopePairs; ++j) {
    double f = 0.0;
    if (cfg.rope && j < half) {
      f = pow((double)cfg.rope_theta, -2.0 * j / cfg.head_dim);
      if (cfg.rope == 2) {
        // LLaMA 3.1: keep short wavelengths, divide long ones by the factor,
        // blend linearly in old_context_len / wavelength between the two
        const double w = 2.0 * M_PI / f;
        const double old = cfg.rope_old_ctx, lo = cfg.rope_low, hi = cfg.rope_high;
        if (w > old / lo) {
          f = f / cfg.rope_factor;
        } else if (w >= old / hi) {
          const double sm = (old / w - lo) / (hi - lo);
          f = (1.0 - sm) * f / cfg.rope_factor + sm * f;
        }
      }
      f /= 2.0 * M_PI;
    }
    const float hi = (float)f;
    rope[2 * j] = hi;
    rope[2 * j + 1] = (float)(f - (double)hi);
  }

  blob[H_MAGIC] = kMagic;
  blob[H_KIND] = cfg.kind;
  blob[H_BATCH] = batch;
  blob[H_WORKERS] = W;
  blob[H_NUM_TILES] = (int32_t)T;
  blob[H_NUM_SEGS] = (int32_t)s;
  blob[H_NUM_PARTIALS] = (int32_t)slot;
  blob[H_NUM_MERGES] = (int32_t)m;
  blob[H_TILE_Q] = Tq;
  blob[H_TILE_KV] = Tk;
  blob[H_ROWS] = L.rows;
  blob[H_GROUP] = cfg.group;
  blob[H_NUM_KV_HEADS] = cfg.hkv;
  blob[H_TILE_HEADS] = L.tile_heads;
  blob[H_PAGE_SIZE] = P;
  blob[H_NUM_BLOCKS] = (int32_t)std::min<int64_t>(N, INT32_MAX);
  blob[H_QUOTA] = (int32_t)std::min<int64_t>(plan_quota, INT32_MAX);
  blob[H_OFF_WSEG] = (int32_t)L.off_wseg;
  blob[H_OFF_SEG] = (int32_t)L.off_seg;
  blob[H_OFF_TILE] = (int32_t)L.off_tile;
  blob[H_OFF_MERGE] = (int32_t)L.off_merge;
  blob[H_OFF_ROPE] = (int32_t)L.off_rope;
  blob[H_MAX_TILES] = L.max_tiles;
  blob[H_MAX_SEGS] = L.max_segs;
  blob[H_MAX_PARTIALS] = L.max_partials;
  blob[H_CAUSAL] = cfg.causal;
  blob[H_OFF_CNT] = (int32_t)L.off_cnt;  // counters stay zero (memset above)
  blob[H_OFF_NTILE] = (int32_t)L.off_ntile;
  blob[H_MERGE_KERNEL] = (!append || max_nseg > kInKernelMergeMax) ? 1 : 0;
  blob[H_OFF_AUX] = (int32_t)L.off_aux;

  plan->kind = cfg.kind;
  plan->batch = batch;
  plan->num_workers = W;
  plan->tile_q = Tq;
  plan->tile_kv = Tk;
  plan->rows_per_tile = L.rows;
  plan->num_tiles = (int32_t)T;
  plan->num_segments = (int32_t)s;
  plan->num_partials = (int32_t)slot;
  plan->num_merges = (int32_t)m;
  plan->max_tiles = L.max_tiles;
  plan->max_segments = L.max_segs;
  plan->max_partials = L.max_partials;
  plan->upload_path = 0;
  plan->fingerprint = fingerprint(cfg, L);
  plan->plan_bytes = L.plan_bytes;
  plan->partial_offset = L.partial_offset;
  plan->dev_bytes = L.dev_bytes;
  return ABP_OK;
}

int bsr_plan_compute(const Config& cfg, const Layout& L, int32_t M, int32_t N, int32_t R,
                     const int32_t* indptr, int32_t* blob, abp_plan* plan, std::string* err) {
  if (cfg.kind != ABP_KIND_BSR) {
    *err = "not a block-sparse configuration";
    return ABP_ERR_INVALID_ARG;
  }
  if (M < 0 || N < 0 || R < 1) {
    *err = "block-sparse attention needs M >= 0, N >= 0 and R >= 1";
    return ABP_ERR_INVALID_ARG;
  }
  const int32_t C = cfg.page_size;
  if (N % C != 0) {
    *err = "N must be a multiple of the column block size (page_size)";
    return ABP_ERR_INVALID_ARG;
  }
  if (!blob || !plan || (M > 0 && !indptr)) {
    *err = "NULL array";
    return ABP_ERR_INVALID_ARG;
  }
  const int64_t nrb = ceil_div(M, R);
  if (nrb > L.aux_cap) {
    *err = "row blocks exceed the workspace capacity (max_row_blocks / max_M)";
    return ABP_ERR_WORKSPACE_TOO_SMALL;
  }
  const int64_t ncb = N / C;
  for (int64_t i = 0; i < nrb; ++i) {
    const int64_t n = int64_t(indptr[i + 1]) - indptr[i];
    if (indptr[0] != 0 || n < 0) {
      *err = "indptr must start at 0 and be non-decreasing";
      return ABP_ERR_INVALID_ARG;
    }
    if (n > ncb) {
      *err = "a row block lists more column blocks than N / C";
      return ABP_ERR_INVALID_ARG;
    }
  }
  // row block i = append request i: queries [i R, min((i+1) R, M)), its
  // pages are its column blocks, all full (kv_len = n_i C)
  int32_t* qo = blob + L.off_aux;
  int32_t* lpl = qo + align4(int64_t(L.aux_cap) + 1);
  for (int64_t i = 0; i <= nrb; ++i) qo[i] = (int32_t)std::min<int64_t>(i * R, M);
  for (int64_t i = 0; i < nrb; ++i) lpl[i] = C;
  const int32_t zero = 0;
  return plan_compute(cfg, L, (int32_t)nrb, qo, nrb > 0 ? indptr : &zero, lpl, blob, plan, err);
}

}  // namespace abp
