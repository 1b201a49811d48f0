// Host planner: pure C++ (no HIP runtime calls).
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <string>

#include "../../include/abp.h"
#include "layout.h"

namespace abp {

// Validated view of abp_params with derived values.
struct Config {
  int kind = ABP_KIND_DECODE;
  int32_t hq = 0, hkv = 0, group = 0, head_dim = 0, page_size = 0;
  int32_t qkv_dtype = 0, out_dtype = 0;
  float sm_scale = 0.f;
  int32_t causal = 0, rope = 0;
  float rope_theta = 0.f;
  // LLaMA 3.1 frequency scaling (rope == 2)
  float rope_factor = 1.f, rope_low = 1.f, rope_high = 1.f, rope_old_ctx = 1.f;
  // fp8 e4m3 KV pages with per-tensor scales (decode only)
  int32_t kv_fp8 = 0;
  float k_scale = 1.f, v_scale = 1.f;
  int32_t rope_interleave = 0;  // RoPE pairs (2j, 2j+1) instead of (j, j + d/2)
};

// Returns ABP_OK or an error status with `err` set.
int check_params(int kind, const abp_params* p, Config* cfg, std::string* err);

// Capacities and offsets from a tile capacity (the form *_run rebuilds).
int make_layout_caps(const Config& cfg, int64_t max_tiles, int32_t workers, Layout* out,
                     std::string* err);

// Capacities and offsets for the given maxima.
int make_layout(const Config& cfg, int32_t max_batch, int32_t max_qo_tokens, int32_t workers,
                Layout* out, std::string* err);

// The Stream-K planner. Writes the blob into host_ws (int32 array of
// layout.plan_ints entries) and fills `plan`.
int plan_compute(const Config& cfg, const Layout& lay, int32_t batch, const int32_t* qo_indptr,
                 const int32_t* kv_indptr, const int32_t* kv_last_page_len, int32_t* blob,
                 abp_plan* plan, std::string* err);

// Block-sparse attention plan: validates the BSR row pointer, writes the
// derived per-row-block query ranges and page counts into the blob's aux
// region and plans them as append requests over the column blocks.
int bsr_plan_compute(const Config& cfg, const Layout& lay, int32_t M, int32_t N, int32_t R,
                     const int32_t* indptr, int32_t* blob, abp_plan* plan, std::string* err);

uint64_t fingerprint(const Config& cfg, const Layout& lay);

}  // namespace abp
