// Persistent append / prefill attention over a paged block-sparse-row KV cache
// on gfx950 matrix cores.
//
// What it computes: for ragged query tokens (qo_indptr) of each request, exact
// softmax attention over the request's paged keys, optionally causal with the
// mask aligned to the end of the KV (query i sees keys t <= kv_len - qo_len + i).
// Prefill / append over paged and ragged caches are core kernels of the README
// (gittoolsai.com, section 核心功能 / 注意力机制内核); the block-sparse-row
// addressing is the paper summary's ("图谱动态｜学苑周刊 NO.266", section
// 统一的 KV 缓存存储格式), and the work split follows its load-balancing
// section (动态负载均衡调度). Unlike decode, each K/V element is reused by up
// to 128 query rows, so this path is bound by matrix-core throughput.
//
// Tiles: 256 rows = tile_q tokens x G qo heads of one kv head (row r is token
// r / G, head r % G), against blocks of 64 keys. A 512-thread workgroup (8
// waves) is one worker; wave w owns rows [32 w, 32 w + 32) (two 16-row column
// blocks). The RoPE variant (append_rope.hip) uses 128-row tiles, 16 rows a
// wave: its q operands are hi and lo parts.
//
//   S^T = K Q^T    v_mfma_f32_16x16x32 with A = K rows from LDS and B = Q^T
//                  from registers. The accumulator gives each lane one query
//                  row and 16 of the block's keys, so softmax statistics are
//                  lane-local except a 4-lane-group max.
//   softmax        fp32, base-2 exponentials, running max per row with a lazy
//                  rescale; P is rounded to the storage type for the next product.
//   O^T += V^T P^T v_mfma with A = V^T from LDS and B = P^T taken directly from
//                  the S registers: the K-slot order of the product is the
//                  order in which S holds the keys, so no lane exchange.
//
// Staging, two LDS stages (block j + 1 is loaded while block j is computed):
//   * without RoPE, K and V rows go straight from global memory into LDS with
//     the gfx950 global-to-LDS loads, rows unpadded with their 16-byte chunks
//     XOR-swizzled by row (K chunk q of row r at q ^ (r & 15), V at
//     q ^ 2 (r & 7)); K operands are plain 16-byte reads and V^T operands come
//     from ds_read_b64_tr_b16 transpose reads, both free of bank conflicts;
//   * with RoPE, K is loaded into registers, rotated in fp32 and stored as
//     16-bit hi and lo parts (padded rows), and V is stored transposed (key
//     pairs packed with v_perm); the waves take K and V rows alike.
// Rows past the segment end re-read the segment's last key (in bounds; their
// scores are masked, and their values are finite even where the slot holds no
// token). A tile split over a few workers is merged by the workgroup whose
// partial state arrives last (per-tile arrival counters). With a power-of-two
// page size >= 16, a block's page ids are scalar loads. Workers are mapped to
// workgroup ids XCD-major, so consecutive workers run on the same XCD and
// share its L2; the planner gives groups of them query tiles of one (request,
// kv head) to run side by side, and their K/V reads meet in that L2.
#include "append_impl.h"

namespace abp {

namespace {

using appi::append_waves;

template <typename T, int G, bool CAUSAL, bool FASTPAGE>
__global__ __launch_bounds__(64 * append_waves<false>(), 1) void append_kernel(AttnArgs a) {
  ABP_APPEND_PIPE_LDS(lds, 2);
  appi::append_worker<T, G, CAUSAL, false, FASTPAGE, false>(a, blockIdx.x, lds);
}

template <typename T, int G, bool CAUSAL>
hipError_t launch_c(const Config& cfg, const AttnArgs& a, hipStream_t s) {
  if (cfg.rope) return launch_append_rope(cfg, a, s);
  if (a.page_shift >= 4)
    append_kernel<T, G, CAUSAL, true><<<a.workers, 64 * append_waves<false>(), 0, s>>>(a);
  else
    append_kernel<T, G, CAUSAL, false><<<a.workers, 64 * append_waves<false>(), 0, s>>>(a);
  return hipGetLastError();
}

template <typename T, int G>
hipError_t launch_g(const Config& cfg, const AttnArgs& a, hipStream_t s) {
  return cfg.causal ? launch_c<T, G, true>(cfg, a, s) : launch_c<T, G, false>(cfg, a, s);
}

template <typename T>
hipError_t launch_t(const Config& cfg, const AttnArgs& a, hipStream_t s) {
  switch (cfg.group) {
    case 1: return launch_g<T, 1>(cfg, a, s);
    case 2: return launch_g<T, 2>(cfg, a, s);
    case 4: return launch_g<T, 4>(cfg, a, s);
    case 8: return launch_g<T, 8>(cfg, a, s);
    case 16: return launch_g<T, 16>(cfg, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_append(const Config& cfg, const AttnArgs& a, hipStream_t s) {
  if (cfg.qkv_dtype == ABP_BF16) return launch_t<BF16>(cfg, a, s);
  return launch_t<F16>(cfg, a, s);
}

int append_blocks_per_cu(const Config& cfg) {
  if (cfg.rope) return append_rope_blocks_per_cu();
  int n = 0;
  // the tile shape is shared by all variants, each built for one per CU
  const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &n, append_kernel<BF16, 4, true, true>, 64 * append_waves<false>(), 0);
  return e == hipSuccess && n > 0 ? n : 1;
}

}  // namespace abp
