// Batch decode in one call that allocates nothing, for callers that cannot
// allocate (code under graph capture of the caller's own making, tight serving
// loops, harnesses that forbid allocation). It is abp_decode_plan followed by
// abp_decode_run, with the two workspaces held by the library:
//   * the device workspace (plan blob, partial states of split tiles) is
//     `scratch`, a file-scope device array of ABP_STATIC_SCRATCH_BYTES on every
//     GPU the library runs on, kept until the process ends;
//   * the host workspace is a file-scope host array of ABP_STATIC_PLAN_BYTES.
// The plan is copied with hipMemcpyAsync from that pageable host array, which
// HIP performs synchronously with respect to the host, so the array may be
// reused as soon as the copy call returns; a mutex keeps two host threads from
// planning into it at once. Every call on one GPU uses that GPU's scratch and
// leaves its contents behind (the next call uploads a fresh plan, which also
// clears the per-tile counters, and partial states are written before they are
// read). Calls on one stream are ordered; calls that overlap on one GPU (other
// streams, other host threads) race on the scratch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "../../include/abp.h"
#include "kernels.h"

static __device__ __align__(256) unsigned char scratch[ABP_STATIC_SCRATCH_BYTES];

namespace {

alignas(256) int32_t g_host_plan[ABP_STATIC_PLAN_BYTES / sizeof(int32_t)];
std::mutex g_plan_mutex;

constexpr int kMaxDevices = 64;
std::mutex g_ptr_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's `scratch` (looked up once per device, with
// that device current). In host code the array's name is only a host-side
// handle: kernels and copies must be given this address.
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return abp::set_error(ABP_ERR_HIP, (std::string("hipGetDevice: ") + hipGetErrorString(e)).c_str());
  if (dev < 0 || dev >= kMaxDevices) return abp::set_error(ABP_ERR_INVALID_ARG, "device out of range");
  std::lock_guard<std::mutex> lock(g_ptr_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return abp::set_error(ABP_ERR_HIP, (std::string("hipGetSymbolAddress(scratch): ") +
                                          hipGetErrorString(e)).c_str());
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ABP_OK;
}

}  // namespace

extern "C" int abp_decode_static(const abp_params* params, int32_t batch,
                                 const int32_t* kv_indptr_h, const int32_t* kv_last_page_len_h,
                                 int32_t num_workers, const void* q, const void* k_pages,
                                 const void* v_pages, const int32_t* kv_indptr_d,
                                 const int32_t* kv_indices_d, const int32_t* kv_last_page_len_d,
                                 const int32_t* q_pos_d, const int32_t* kv_pos_offset_d, void* o,
                                 float* lse, abp_stream_t stream) {
  try {
    if (!params) return abp::set_error(ABP_ERR_INVALID_ARG, "params is NULL");
    if (batch < 0) return abp::set_error(ABP_ERR_INVALID_ARG, "batch < 0");
    int32_t workers = num_workers;
    int st = ABP_OK;
    if (workers <= 0 && workers != ABP_WORKERS_PER_TILE) {
      st = abp::default_decode_workers(params, &workers);
      if (st != ABP_OK) return st;
    }
    // sizes first: nothing reaches the GPU when the batch does not fit
    const int32_t cap = std::max<int32_t>(batch, 1);
    size_t host_bytes = 0, dev_bytes = 0;
    st = abp_workspace_size(ABP_KIND_DECODE, params, cap, 0, workers, &host_bytes, &dev_bytes);
    if (st != ABP_OK) return st;
    if (host_bytes > ABP_STATIC_PLAN_BYTES || dev_bytes > ABP_STATIC_SCRATCH_BYTES) {
      const std::string msg =
          "abp_decode_static: this batch needs " + std::to_string(host_bytes) +
          " bytes of plan and " + std::to_string(dev_bytes) + " bytes of device workspace; the " +
          "library holds " + std::to_string(ABP_STATIC_PLAN_BYTES) + " and " +
          std::to_string(ABP_STATIC_SCRATCH_BYTES) +
          " (use abp_decode_plan / abp_decode_run with caller workspaces)";
      return abp::set_error(ABP_ERR_WORKSPACE_TOO_SMALL, msg.c_str());
    }
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != ABP_OK) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    abp_plan plan{};
    {
      std::lock_guard<std::mutex> lock(g_plan_mutex);
      st = abp_plan_host(ABP_KIND_DECODE, params, batch, nullptr, kv_indptr_h, kv_last_page_len_h,
                         cap, 0, workers, g_host_plan, sizeof(g_host_plan), &plan);
      if (st != ABP_OK) return st;
      // pageable source: the copy has consumed g_host_plan when the call returns
      hipError_t e = hipMemcpyAsync(ws, g_host_plan, plan.plan_bytes, hipMemcpyHostToDevice, s);
      if (e != hipSuccess)
        return abp::set_error(ABP_ERR_HIP,
                              (std::string("hipMemcpyAsync(plan): ") + hipGetErrorString(e)).c_str());
    }
    return abp_decode_run(&plan, params, q, k_pages, v_pages, kv_indptr_d, kv_indices_d,
                          kv_last_page_len_d, q_pos_d, kv_pos_offset_d, o, lse, ws,
                          ABP_STATIC_SCRATCH_BYTES, stream);
  } catch (...) {
    return abp::set_error(ABP_ERR_HIP, "exception");
  }
}
