// Plan blob layout shared by the host planner and the GPU kernels.
//
// The blob is an int32 array written on the host and copied once to the start
// of the device workspace. Every offset depends only on capacities fixed by
// (kind, params, max_batch, max_qo_tokens, num_workers), never on the lengths
// of one batch, so kernels captured in a graph stay valid after a re-plan:
// they read the counts of the current plan from the header at run time.
#pragma once
#include <stdint.h>

namespace abp {

enum Header : int {
  H_MAGIC = 0,
  H_KIND,
  H_BATCH,
  H_WORKERS,
  H_NUM_TILES,
  H_NUM_SEGS,
  H_NUM_PARTIALS,
  H_NUM_MERGES,
  H_TILE_Q,
  H_TILE_KV,
  H_ROWS,        // rows per tile = tile_q * group
  H_GROUP,       // qo heads per kv head
  H_NUM_KV_HEADS,
  H_PAGE_SIZE,
  H_NUM_BLOCKS,
  H_QUOTA,
  H_OFF_WSEG,    // int32 offsets of the arrays below
  H_OFF_SEG,
  H_OFF_TILE,
  H_OFF_MERGE,
  H_OFF_ROPE,
  H_MAX_TILES,
  H_MAX_SEGS,
  H_MAX_PARTIALS,
  H_CAUSAL,
  H_OFF_CNT,     // per-tile arrival counters of split tiles (zero in every upload)
  H_OFF_NTILE,   // per-tile number of partials
  H_MERGE_KERNEL,  // 1: split tiles are merged by the merge kernel after the
                   // main kernel; 0: by the last arriving workgroup (append)
  H_TILE_HEADS,    // consecutive kv heads per tile
  H_OFF_AUX,       // block-sparse plans: derived qo_indptr then kv_last_page_len
  HEADER_INTS = 32
};

constexpr int32_t kMagic = 0x41425031;  // "ABP1"
constexpr int kMaxRopePairs = 64;        // head_dim 128

// Records (16-byte aligned in the blob):
//   seg   int32 x 4 {tile, kv_begin, kv_end, partial_slot or -1}
//   tile  int32 x 4 {b, first kv_head, q_tile, first_partial or -1}
//   ntile int32 x 1 number of partials of the tile (0 if not split)
//   merge int32 x 4 {tile, first_partial, num_partials, 0}
//   cnt   int32 x 1 per tile: segments of a split tile that have written their
//         partial; the last one merges the tile and resets it to 0
// worker_seg_indptr has num_workers + 1 entries.
// rope: kMaxRopePairs x {hi, lo} float32 bit patterns of f_j / (2 pi)
//       (revolutions per position; f_j = theta^(-2j/d), LLaMA 3.1-scaled when
//       asked), split so hi + lo carries ~48 bits.
// aux (block-sparse plans only, at the end): int32 qo_indptr [aux_cap + 1]
//       then kv_last_page_len [aux_cap], aux_cap = max_tiles / num_kv_heads
//       (every row block has at least one tile per kv head).

struct Layout {
  int32_t workers = 0;
  int32_t max_tiles = 0;
  int32_t max_segs = 0;
  int32_t max_partials = 0;
  int32_t max_merges = 0;
  int32_t tile_q = 1;
  int32_t tile_kv = 64;
  int32_t rows = 1;
  int32_t tile_heads = 1;
  int64_t off_wseg = 0, off_seg = 0, off_tile = 0, off_ntile = 0, off_merge = 0, off_rope = 0,
          off_cnt = 0;
  int64_t off_aux = 0;         // == plan_ints when there is no aux region
  int32_t aux_cap = 0;         // row blocks the aux region holds
  int64_t plan_ints = 0;       // total int32 of the blob
  uint64_t plan_bytes = 0;
  uint64_t partial_offset = 0; // bytes, 256-aligned
  uint64_t partial_bytes = 0;
  uint64_t dev_bytes = 0;
  // planning mode (not part of the memory layout): one worker per tile, each
  // tile one segment, no partial states (workers = the tile capacity)
  bool no_split = false;
};

// Tile sizes of the kernels.
constexpr int kDecodeTileKv = 64;   // keys per work block (decode)
// kv heads per decode tile: the 4 waves of a decode workgroup take 4
// consecutive kv heads of one request when the head count allows it, so the
// workgroup reads 1 KB runs of each token row instead of 256-byte pieces;
// otherwise one head, with its keys split over the 4 waves
constexpr int decode_tile_heads(int hkv) { return hkv % 4 == 0 ? 4 : 1; }
// MFMA rows per append tile (= tile_q * group): 8 waves x 32 rows, or 8 waves
// x 16 rows for the RoPE variant (its q operands are hi and lo parts)
constexpr int append_rows(bool rope) { return rope ? 128 : 256; }
constexpr int kAppendTileKv = 64;   // keys per work block (append)
// An append tile split into more partials than this is merged by the merge
// kernel (spread over all CUs) rather than by one workgroup inside the kernel.
constexpr int kInKernelMergeMax = 4;

}  // namespace abp
