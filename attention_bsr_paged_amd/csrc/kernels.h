// Kernel argument blocks and host-side launchers (defined in the .hip files).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace abp {

// Paged attention (decode and append share this argument block).
struct AttnArgs {
  const void* q;
  const void* k_pages;
  const void* v_pages;
  const int32_t* qo_indptr;      // append only
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* kv_last_page_len;
  const int32_t* q_pos;          // RoPE only, may be NULL
  const int32_t* kv_pos_offset;  // RoPE only, may be NULL
  void* o;
  float* lse;                    // may be NULL
  const int32_t* plan;           // plan blob in device memory
  float* o_part;                 // [max_partials, rows, head_dim]
  float* lse_part;               // [max_partials, rows]
  int32_t num_qo_heads;
  int32_t num_kv_heads;
  int32_t page_size;
  int32_t page_shift;            // log2(page_size) if a power of two, else -1
  int64_t page_stride;           // elements per page = page_size * Hkv * head_dim
  int32_t token_stride;          // elements per token inside a page = Hkv * head_dim
  int32_t out_dtype;
  float sm_scale;
  float sm_scale_log2;           // sm_scale * log2(e)
  int32_t workers;
  float v_scale;                 // fp8 V pages: value = v_scale * code value (else 1)
};

hipError_t launch_decode(const Config& cfg, const AttnArgs& a, hipStream_t stream);
// matrix-core decode (16-bit K/V, no RoPE, power-of-two pages >= 16, kv heads a
// multiple of 4, group 4 or 8); launch_decode picks it when it applies
bool decode_mfma_applies(const Config& cfg);
hipError_t launch_decode_mfma(const Config& cfg, const AttnArgs& a, hipStream_t stream);
int decode_mfma_blocks_per_cu(const Config& cfg);
// resident 256-thread workgroups per compute unit of the kernel chosen for cfg
int decode_blocks_per_cu(const Config& cfg);
int append_blocks_per_cu(const Config& cfg);
hipError_t launch_append(const Config& cfg, const AttnArgs& a, hipStream_t stream);
// the RoPE variants of the append kernel (append_rope.hip; launch_append
// dispatches to them)
int append_rope_blocks_per_cu();
hipError_t launch_append_rope(const Config& cfg, const AttnArgs& a, hipStream_t stream);
// mixed batch: workgroups [0, app.workers) run append workers, the next
// dec.workers run matrix-core decode workers (cfg: the append part's config)
bool pod_applies(const Config& cfg);
hipError_t launch_pod(const Config& cfg, const AttnArgs& app, const AttnArgs& dec,
                      hipStream_t stream);
// copies `bytes` (multiple of 4, 16-byte aligned pointers) from pinned host
// memory mapped into the GPU's address space to device memory
hipError_t launch_upload(void* dev_dst, const void* host_src_mapped, size_t bytes,
                         hipStream_t stream);
// merges the split tiles of a plan into o / lse after its main kernel (fixed
// grid; counts and the merge mode are read from the plan at run time)
// Cascade: the final (o, lse) of every (request, qo head) row from the prefix
// level's and the suffix level's states (direct fp32 outputs or partial slots)
hipError_t launch_cascade_merge(const AttnArgs& pre, const AttnArgs& suf, int32_t batch,
                                void* o, float* lse, int out_dtype, hipStream_t stream);
hipError_t launch_plan_merge(const Config& cfg, const AttnArgs& a, int32_t grid,
                             hipStream_t stream);

// writes nnz new K/V rows [nnz, hkv, 128] into the pages at the last
// positions of their requests (rows outside a request are skipped)
hipError_t launch_page_append(const void* k_new, const void* v_new, const int32_t* append_indptr,
                              void* k_pages, void* v_pages, const int32_t* kv_indptr,
                              const int32_t* kv_indices, const int32_t* kv_last_page_len,
                              int32_t batch, int64_t nnz, int32_t row_bytes, int32_t page_size,
                              hipStream_t stream);

// Host-side helpers shared with the no-allocation entry point (api.cpp):
// the default decode worker count of the current device for `params`, and
// recording a status message for abp_last_error() (returns `status`).
int default_decode_workers(const abp_params* params, int32_t* out);
int set_error(int status, const char* msg);

hipError_t launch_merge_two(const void* o_a, const float* lse_a, const void* o_b,
                            const float* lse_b, void* o_out, float* lse_out, int64_t rows,
                            int in_dtype, int out_dtype, hipStream_t stream);
hipError_t launch_merge_states(const void* o_in, const float* lse_in, int32_t num_states,
                               int64_t rows, int in_dtype, int out_dtype, void* o_out,
                               float* lse_out, hipStream_t stream);

}  // namespace abp
