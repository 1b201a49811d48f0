// Randomised driver of the host planner and the C ABI's validation, built with
// the host address and undefined-behaviour sanitizers (no device code: the
// kernel launchers are stubs). Every valid batch's plan is checked for the
// Stream-K invariants (exact cover of each tile's key range in order,
// per-worker load at most the quota, contiguous partial slots, segment
// indptr consistent); invalid arrays must come back as the documented error
// codes. Prints "fuzz_abi ok <cases>" and exits 0, or reports and exits 1.
#include <stdio.h>
#include <stdlib.h>

#include <random>
#include <vector>

#include "../../include/abp.h"
#include "../../attention_bsr_paged_amd/csrc/layout.h"

namespace {

std::mt19937 rng(12345);
int rnd(int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); }

int fails = 0;
#define CHECK(c, ...)                                    \
  do {                                                   \
    if (!(c)) {                                          \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                      \
      fprintf(stderr, "\n");                             \
      ++fails;                                           \
    }                                                    \
  } while (0)

abp_params make(int hq, int hkv, int page, int causal) {
  abp_params p{};
  p.num_qo_heads = hq;
  p.num_kv_heads = hkv;
  p.head_dim = 128;
  p.page_size = page;
  p.qkv_dtype = ABP_BF16;
  p.out_dtype = ABP_BF16;
  p.causal = causal;
  return p;
}

// Check the invariants of a plan blob against the batch it was made from.
void check_plan(const std::vector<int32_t>& blob, const abp_plan& plan, bool append, bool causal,
                bool no_split, const std::vector<int32_t>& qo, const std::vector<int32_t>& kv) {
  using namespace abp;
  const int32_t* h = blob.data();
  CHECK(h[H_MAGIC] == kMagic, "magic");
  const int W = h[H_WORKERS], T = h[H_NUM_TILES], S = h[H_NUM_SEGS];
  const int Tk = h[H_TILE_KV], Tq = h[H_TILE_Q];
  CHECK(W == plan.num_workers && T == plan.num_tiles && S == plan.num_segments, "counts");
  // the plan fits the capacities the workspace was sized for
  CHECK(T <= h[H_MAX_TILES] && S <= h[H_MAX_SEGS] && h[H_NUM_PARTIALS] <= h[H_MAX_PARTIALS],
        "capacities: tiles %d/%d segs %d/%d partials %d/%d", T, h[H_MAX_TILES], S, h[H_MAX_SEGS],
        h[H_NUM_PARTIALS], h[H_MAX_PARTIALS]);
  CHECK(h[H_NUM_MERGES] <= std::max(0, std::min(h[H_MAX_TILES], W - 1)), "merges %d",
        h[H_NUM_MERGES]);
  const int32_t* wseg = h + h[H_OFF_WSEG];
  const int32_t* seg = h + h[H_OFF_SEG];
  const int32_t* tile = h + h[H_OFF_TILE];
  CHECK(wseg[0] == 0 && wseg[W] == S, "wseg ends %d %d", wseg[0], wseg[W]);
  std::vector<int64_t> next(T, 0);    // key where the tile's next segment must begin
  std::vector<int> nseg(T, 0), last_slot(T, -2);
  for (int w = 0; w < W; ++w) {
    CHECK(wseg[w] <= wseg[w + 1], "wseg order");
    int64_t load = 0;
    for (int s = wseg[w]; s < wseg[w + 1]; ++s) {
      const int t = seg[4 * s], b0 = seg[4 * s + 1], e0 = seg[4 * s + 2], sl = seg[4 * s + 3];
      CHECK(t >= 0 && t < T, "tile index");
      if (t < 0 || t >= T) return;
      CHECK(b0 == next[t], "tile %d: segment starts at %d, expected %lld", t, b0,
            (long long)next[t]);
      CHECK(b0 % Tk == 0 && e0 >= b0, "segment bounds");
      next[t] = e0;
      load += std::max<int64_t>(1, (e0 - b0 + Tk - 1) / Tk);
      ++nseg[t];
      if (sl >= 0) {
        CHECK(last_slot[t] == -2 || sl == last_slot[t] + 1, "partial slots contiguous");
        last_slot[t] = sl;
      }
    }
    if (!no_split) CHECK(load <= std::max(1, h[H_QUOTA]), "worker load above quota");
    else CHECK(wseg[w + 1] - wseg[w] <= 1, "one tile per worker");
  }
  // each tile covered to its extent
  for (int t = 0; t < T; ++t) {
    const int b = tile[4 * t], qt = tile[4 * t + 2];
    int64_t e = kv[b];
    if (append && causal) {
      const int64_t ql = qo[b];
      e = kv[b] - ql + std::min<int64_t>(int64_t(qt + 1) * Tq, ql);
    }
    CHECK(next[t] == e, "tile %d covered to %lld, extent %lld", t, (long long)next[t],
          (long long)e);
    CHECK((nseg[t] > 1) == (tile[4 * t + 3] >= 0), "split tiles own partial slots");
    // the arrival counters start every run at zero (co-scheduled plans use
    // them as scratch while planning)
    CHECK(h[h[H_OFF_CNT] + t] == 0, "tile %d: arrival counter %d", t, h[h[H_OFF_CNT] + t]);
  }
}

int run_case() {
  const bool append = rnd(0, 1);
  const int hkv = std::vector<int>{1, 2, 3, 4, 8, 12}[rnd(0, 5)];
  const int g = append ? std::vector<int>{1, 2, 4, 8, 16}[rnd(0, 4)]
                       : std::vector<int>{1, 2, 4, 8}[rnd(0, 3)];
  const int page = std::vector<int>{1, 3, 16, 256}[rnd(0, 3)];
  const bool causal = append && rnd(0, 1);
  abp_params p = make(hkv * g, hkv, page, causal);
  const int B = rnd(0, 20);
  std::vector<int32_t> kv(B), qo(B), indptr(B + 1, 0), lpl(B), qoptr(B + 1, 0);
  for (int b = 0; b < B; ++b) {
    kv[b] = rnd(0, 1) ? rnd(0, 70) : rnd(0, 5000);
    qo[b] = append ? (causal ? rnd(0, std::min(kv[b], 400)) : rnd(0, 400)) : 1;
    const int n = (kv[b] + page - 1) / page;
    indptr[b + 1] = indptr[b] + n;
    lpl[b] = n ? kv[b] - (n - 1) * page : 0;
    qoptr[b + 1] = qoptr[b] + qo[b];
  }
  const int kind = append ? ABP_KIND_APPEND : ABP_KIND_DECODE;
  const bool no_split = rnd(0, 4) == 0;
  const int W = no_split ? ABP_WORKERS_PER_TILE : rnd(1, 300);
  const int max_b = B + rnd(0, 3), max_q = qoptr[B] + rnd(0, 50);
  size_t hb = 0, db = 0;
  int st = abp_workspace_size(kind, &p, max_b, max_q, W, &hb, &db);
  CHECK(st == ABP_OK, "workspace_size %d %s", st, abp_last_error());
  if (st != ABP_OK) return 0;
  std::vector<int32_t> blob(hb / 4 + 1, -7);
  abp_plan plan{};
  st = abp_plan_host(kind, &p, B, append ? qoptr.data() : nullptr, indptr.data(), lpl.data(),
                     max_b, max_q, W, blob.data(), hb, &plan);
  CHECK(st == ABP_OK, "plan_host %d %s", st, abp_last_error());
  if (st == ABP_OK) check_plan(blob, plan, append, causal, no_split, qo, kv);

  // the same batch with one mistake must be refused without touching memory
  // beyond the arrays
  if (B > 0) {
    const int b = rnd(0, B - 1);
    std::vector<int32_t> bad_lpl = lpl, bad_ptr = indptr;
    int expect = ABP_ERR_INVALID_ARG;
    switch (rnd(0, 3)) {
      case 0:
        if (indptr[b + 1] > indptr[b]) bad_lpl[b] = rnd(0, 1) ? 0 : page + 1;
        else return 1;
        break;
      case 1:
        if (indptr[b + 1] > indptr[b]) bad_ptr[b + 1] = bad_ptr[b] - 1;
        else return 1;
        break;
      case 2:
        bad_ptr[0] = 1;
        break;
      default:
        st = abp_plan_host(kind, &p, B, append ? qoptr.data() : nullptr, indptr.data(),
                           lpl.data(), max_b, max_q, W, blob.data(), hb / 2, &plan);
        CHECK(hb < 8 || st == ABP_ERR_WORKSPACE_TOO_SMALL, "short host workspace %d", st);
        return 1;
    }
    st = abp_plan_host(kind, &p, B, append ? qoptr.data() : nullptr, bad_ptr.data(),
                       bad_lpl.data(), max_b, max_q, W, blob.data(), hb, &plan);
    CHECK(st == expect, "invalid arrays gave %d, expected %d", st, expect);
  }
  return 1;
}

int bsr_case() {
  const int hkv = std::vector<int>{1, 2, 8}[rnd(0, 2)];
  const int C = std::vector<int>{1, 3, 16, 64}[rnd(0, 3)];
  abp_params p = make(hkv * 4, hkv, C, 0);
  const int R = rnd(1, 100);
  const int M = rnd(0, 700);
  const int N = C * rnd(1, 40);
  const int nrb = (M + R - 1) / R;
  std::vector<int32_t> ip(nrb + 1, 0);
  for (int i = 0; i < nrb; ++i) ip[i + 1] = ip[i] + rnd(0, N / C);
  const int W = rnd(1, 64);
  size_t hb = 0, db = 0;
  int st = abp_workspace_size(ABP_KIND_BSR, &p, std::max(nrb, 1), std::max(M, 1), W, &hb, &db);
  CHECK(st == ABP_OK, "bsr workspace %d %s", st, abp_last_error());
  std::vector<int32_t> blob(hb / 4 + 1);
  abp_plan plan{};
  st = abp_bsr_plan_host(&p, M, N, R, ip.data(), std::max(nrb, 1), std::max(M, 1), W,
                         blob.data(), hb, &plan);
  CHECK(st == ABP_OK, "bsr plan %d %s", st, abp_last_error());
  if (nrb > 0) {
    ip[nrb] = ip[nrb - 1] - 1;  // decreasing row pointer
    st = abp_bsr_plan_host(&p, M, N, R, ip.data(), std::max(nrb, 1), std::max(M, 1), W,
                           blob.data(), hb, &plan);
    CHECK(st == ABP_ERR_INVALID_ARG, "bsr bad indptr gave %d", st);
  }
  return 1;
}

int pod_case() {
  const int hkv = std::vector<int>{4, 8}[rnd(0, 1)];
  const int g = std::vector<int>{4, 8}[rnd(0, 1)];
  abp_params p = make(hkv * g, hkv, 16, rnd(0, 1));
  const int Bd = rnd(0, 10), Ba = rnd(0, 6);
  std::vector<int32_t> dptr(Bd + 1, 0), dlpl(Bd), aptr(Ba + 1, 0), alpl(Ba), qptr(Ba + 1, 0);
  for (int b = 0; b < Bd; ++b) {
    const int kv = rnd(0, 3000), n = (kv + 15) / 16;
    dptr[b + 1] = dptr[b] + n;
    dlpl[b] = n ? kv - (n - 1) * 16 : 0;
  }
  for (int b = 0; b < Ba; ++b) {
    const int kv = rnd(1, 3000), n = (kv + 15) / 16;
    aptr[b + 1] = aptr[b] + n;
    alpl[b] = kv - (n - 1) * 16;
    qptr[b + 1] = qptr[b] + rnd(0, std::min(kv, 300));
  }
  const int groups = rnd(2, 300);
  size_t hb = 0, db = 0;
  int st = abp_pod_workspace_size(&p, std::max(Bd, 1), std::max(Ba, 1), std::max(qptr[Ba], 1),
                                  groups, &hb, &db);
  CHECK(st == ABP_OK, "pod workspace %d %s", st, abp_last_error());
  if (st != ABP_OK) return 0;
  std::vector<int32_t> blob(hb / 4 + 1);
  abp_pod_plan_t plan{};
  st = abp_pod_plan_host(&p, Bd, dptr.data(), dlpl.data(), Ba, qptr.data(), aptr.data(),
                         alpl.data(), std::max(Bd, 1), std::max(Ba, 1), std::max(qptr[Ba], 1),
                         groups, rnd(0, 1) ? 0 : rnd(1, groups - 1), blob.data(), hb, &plan);
  CHECK(st == ABP_OK, "pod plan %d %s", st, abp_last_error());
  return 1;
}

}  // namespace

int main(int argc, char** argv) {
  const int n = argc > 1 ? atoi(argv[1]) : 2000;
  int cases = 0;
  for (int i = 0; i < n; ++i) cases += run_case();
  for (int i = 0; i < n / 4; ++i) cases += bsr_case();
  for (int i = 0; i < n / 4; ++i) cases += pod_case();
  if (fails) {
    fprintf(stderr, "fuzz_abi: %d failures\n", fails);
    return 1;
  }
  printf("fuzz_abi ok %d\n", cases);
  return 0;
}
