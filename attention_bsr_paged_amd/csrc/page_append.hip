// Writing new tokens into a paged KV cache on gfx950.
//
// The step before decode or append reads the pages: the new K/V rows of each
// request are scattered into the pages its page table already assigns to them
// (paged KV caches for dynamic batching, README page on gittoolsai.com, section
// 核心功能 / 注意力机制内核; the page table is the paper summary's block-sparse
// row format, "图谱动态｜学苑周刊 NO.266", section 统一的 KV 缓存存储格式).
//
// New row i of request b (rows append_indptr[b] .. append_indptr[b+1] - 1) is
// logical token t = kv_len_b - append_len_b + i and goes to slot t % P of page
// kv_indices[kv_indptr[b] + t / P]. The work is a copy, bound by HBM: every row
// is read once and written once.
//
// One wave moves one row (K and V). The row's source address depends only on
// its index, so the wave issues the loads of its first 2 KB of K and of V
// first and finds the destination while they are in flight: a binary search
// over append_indptr on the scalar unit (the row index is uniform over the
// wave), then the request's page-table entries. Without that overlap the copy
// waits on about six dependent index loads before its first data load. Rows
// outside their request's range are skipped, so a bad append_indptr cannot
// write outside the pages the table names. Rows are read once and written
// once, so both sides use non-temporal accesses.
#include "common.h"
#include "kernels.h"

namespace abp {

namespace {

constexpr int kWaves = 4;  // rows per 256-thread workgroup

__global__ __launch_bounds__(64 * kWaves) void page_append_kernel(
    const u32x4_t* __restrict__ k_new, const u32x4_t* __restrict__ v_new,
    const int32_t* append_indptr, u32x4_t* __restrict__ k_pages, u32x4_t* __restrict__ v_pages,
    const int32_t* kv_indptr, const int32_t* kv_indices, const int32_t* kv_last_page_len,
    int32_t batch, int64_t nnz, int32_t row_chunks, int32_t page_size) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t t = int64_t(blockIdx.x) * kWaves + wave;
  if (t >= nnz) return;
  const int64_t src = t * row_chunks;
  // pieces lane and lane + 64 of the row (row_chunks = Hkv * 128 * element bytes / 16)
  const bool has0 = lane < row_chunks, has1 = lane + 64 < row_chunks;
  u32x4_t k0 = {}, v0 = {}, k1 = {}, v1 = {};
  if (has0) {
    k0 = __builtin_nontemporal_load(k_new + src + lane);
    v0 = __builtin_nontemporal_load(v_new + src + lane);
  }
  if (has1) {
    k1 = __builtin_nontemporal_load(k_new + src + lane + 64);
    v1 = __builtin_nontemporal_load(v_new + src + lane + 64);
  }
  const ABP_CONST_AS int32_t* ai = const_as(append_indptr);
  // request b with ai[b] <= t < ai[b + 1]
  int lo = 0, hi = batch;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ai[mid] <= t) lo = mid;
    else hi = mid;
  }
  const int b = lo;
  const int a0 = ai[b], a1 = ai[b + 1];
  if (t < a0 || t >= a1) return;
  const ABP_CONST_AS int32_t* ip = const_as(kv_indptr);
  const int p0 = ip[b];
  const int npg = ip[b + 1] - p0;
  const int64_t kv_len = npg > 0 ? int64_t(npg - 1) * page_size + const_as(kv_last_page_len)[b] : 0;
  const int64_t pos = kv_len - (a1 - a0) + (t - a0);
  if (pos < 0 || pos >= kv_len) return;
  const int64_t page = const_as(kv_indices)[p0 + pos / page_size];
  const int64_t dst = (page * page_size + pos % page_size) * row_chunks;
  if (has0) {
    __builtin_nontemporal_store(k0, k_pages + dst + lane);
    __builtin_nontemporal_store(v0, v_pages + dst + lane);
  }
  if (has1) {
    __builtin_nontemporal_store(k1, k_pages + dst + lane + 64);
    __builtin_nontemporal_store(v1, v_pages + dst + lane + 64);
  }
  // rows of more than 8 kv heads: the rest, two pieces per tensor at a time
  for (int c = lane + 128; c < row_chunks; c += 128) {
    const bool two = c + 64 < row_chunks;
    const u32x4_t ka = __builtin_nontemporal_load(k_new + src + c);
    const u32x4_t va = __builtin_nontemporal_load(v_new + src + c);
    u32x4_t kb = ka, vb = va;
    if (two) {
      kb = __builtin_nontemporal_load(k_new + src + c + 64);
      vb = __builtin_nontemporal_load(v_new + src + c + 64);
    }
    __builtin_nontemporal_store(ka, k_pages + dst + c);
    __builtin_nontemporal_store(va, v_pages + dst + c);
    if (two) {
      __builtin_nontemporal_store(kb, k_pages + dst + c + 64);
      __builtin_nontemporal_store(vb, v_pages + dst + c + 64);
    }
  }
}

}  // namespace

hipError_t launch_page_append(const void* k_new, const void* v_new, const int32_t* append_indptr,
                              void* k_pages, void* v_pages, const int32_t* kv_indptr,
                              const int32_t* kv_indices, const int32_t* kv_last_page_len,
                              int32_t batch, int64_t nnz, int32_t row_bytes, int32_t page_size,
                              hipStream_t stream) {
  if (nnz <= 0 || batch <= 0) return hipSuccess;
  const int64_t blocks = (nnz + kWaves - 1) / kWaves;
  page_append_kernel<<<dim3((unsigned)blocks), 64 * kWaves, 0, stream>>>(
      static_cast<const u32x4_t*>(k_new), static_cast<const u32x4_t*>(v_new), append_indptr,
      static_cast<u32x4_t*>(k_pages), static_cast<u32x4_t*>(v_pages), kv_indptr, kv_indices,
      kv_last_page_len, batch, nnz, row_bytes / 16, page_size);
  return hipGetLastError();
}

}  // namespace abp
