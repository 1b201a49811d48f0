/*
 * abp.h -- C ABI of libabp: attention over a paged block-sparse-row (BSR) KV
 * cache on AMD Instinct MI355X (gfx950).
 *
 * Operations and where they are defined
 * -------------------------------------
 *  - The KV cache is a block-sparse-row matrix with a configurable block (page)
 *    size; one kernel serves contiguous and paged layouts (FlashInfer paper
 *    summary, "图谱动态｜学苑周刊 NO.266", section 统一的 KV 缓存存储格式).
 *  - Work is planned on the CPU from the length distribution and then run on
 *    the GPU by a persistent kernel with a fixed grid and a preallocated
 *    workspace, so the run can be captured in a graph (same page, section
 *    动态负载均衡调度).
 *  - Decode, append and prefill over paged and ragged caches, cascade attention
 *    for shared prefixes, and RoPE fused into attention (README translation on
 *    gittoolsai.com, section 核心功能 / 注意力机制内核; paper summary, section
 *    可定制的注意力模板 and 高级功能).
 *  - The single-request decode call of the README example (section 基本用法)
 *    is abp_decode_* with batch 1: q [num_qo_heads, head_dim], K/V
 *    [kv_len, num_kv_heads, head_dim] as one page of size kv_len.
 *
 * Attention computed (exactly, up to float rounding):
 *     s_t = sm_scale * <q, k_t>,  lse = ln sum_t exp(s_t),  o = sum_t exp(s_t - lse) v_t
 * over the keys t a query may see; with no visible key, o = 0 and lse = -inf.
 * lse is the natural log of the scaled logits.
 *
 * Layouts (all row-major, "NHD" inside a page)
 * --------------------------------------------
 *  q (decode)     [batch, num_qo_heads, head_dim]           qkv_dtype
 *  q (append)     [total_qo_tokens, num_qo_heads, head_dim] qkv_dtype, ragged by qo_indptr
 *  k_pages,
 *  v_pages        [num_pages, page_size, num_kv_heads, head_dim] qkv_dtype (two pools)
 *  kv_indptr      int32 [batch + 1]; request b owns page slots [kv_indptr[b], kv_indptr[b+1])
 *  kv_indices     int32 [kv_indptr[batch]]; physical page id of each slot, in logical order
 *  kv_last_page_len int32 [batch]; valid tokens in the last page, in [1, page_size]
 *                 (ignored for a request with no pages, whose kv_len is 0)
 *  kv_len[b] = (kv_indptr[b+1] - kv_indptr[b] - 1) * page_size + kv_last_page_len[b]
 *  o              same shape as q, out_dtype; lse float32 [rows of q, num_qo_heads]
 *  GQA: qo head h reads kv head h / (num_qo_heads / num_kv_heads).
 *  Causal append: query i (0-based) of a request with qo_len queries sees keys
 *  t <= kv_len - qo_len + i (aligned to the end of the KV).
 *  RoPE (params.rope = 1): LLaMA rotate-half; pair (j, j + head_dim/2) of q and k
 *  (or (2j, 2j + 1) with params.rope_interleave = 1) is turned by pos * f_j, f_j = rope_theta^(-2j/head_dim). params.rope = 2 uses
 *  the LLaMA 3.1 frequencies instead (README page, section 其他算子, lists
 *  LLaMA 3.1 RoPE; the rule is the one published with those models): with
 *  wavelength w = 2 pi / f_j, f_j is kept if w < old_context_len /
 *  high_freq_factor, divided by factor if w > old_context_len / low_freq_factor,
 *  and otherwise blended as (1 - s) f_j / factor + s f_j with s =
 *  (old_context_len / w - low_freq_factor) / (high_freq_factor - low_freq_factor).
 *  Key t of request b sits at
 *  kv_pos_offset[b] + t (default 0). A decode query sits at q_pos[b] (default
 *  kv_len - 1); append query i at q_pos[token] (default kv_len - qo_len + i).
 *  K is stored un-rotated; v is never rotated.
 *
 * Supported: head_dim 128; fp16 or bf16 q/k/v; num_qo_heads / num_kv_heads in
 * {1, 2, 4, 8, 16}; page_size >= 1 with one page of K (or V) under 2 GiB;
 * kv_len < 2^24; batch >= 0. Decode (without
 * RoPE) and page append also take an fp8 e4m3 KV cache (params.kv_fp8).
 *
 * Ownership and lifetime
 * ----------------------
 * The caller owns every buffer: tensors, index arrays, the host workspace (use
 * pinned memory for an asynchronous upload), the device workspace and the
 * abp_plan struct. The library allocates no memory in any call; its only state
 * is a per-device compute-unit count and a thread-local error string.
 * *_plan enqueues one host->device copy of the plan on `stream`; the host
 * workspace must not be modified until that copy has completed.
 *
 * Errors
 * ------
 * Every entry point returns an abp_status (0 = ABP_OK); no C++ exception
 * crosses this boundary. abp_last_error() gives a message for the calling
 * thread's last failure. *_plan validates the host index arrays fully; *_run
 * checks that its params match the plan (fingerprint) and that the device
 * workspace is large enough. Device-side index arrays are trusted: a page id
 * outside the pools is undefined behaviour.
 *
 * Graphs
 * ------
 * *_run and abp_merge_state(s) only enqueue kernels on `stream` (fixed grids,
 * no allocation, no copies), so they can be captured in a hipGraph and
 * replayed after a re-plan with the same capacities and worker count. *_plan
 * must not be called during capture.
 */
#ifndef ABP_H_
#define ABP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* abp_stream_t; /* a hipStream_t; NULL = default stream */

typedef enum abp_status {
  ABP_OK = 0,
  ABP_ERR_INVALID_ARG = -1,         /* bad pointer, size or index array */
  ABP_ERR_UNSUPPORTED = -2,         /* head_dim, dtype or group size not built */
  ABP_ERR_WORKSPACE_TOO_SMALL = -3, /* host or device workspace below the query */
  ABP_ERR_PLAN_MISMATCH = -4,       /* run params differ from the planned ones */
  ABP_ERR_HIP = -5                  /* a HIP runtime call failed (e.g. no device) */
} abp_status;

typedef enum abp_dtype { ABP_F16 = 0, ABP_BF16 = 1, ABP_F32 = 2 } abp_dtype;
typedef enum abp_kind { ABP_KIND_DECODE = 0, ABP_KIND_APPEND = 1, ABP_KIND_BSR = 2 } abp_kind;

typedef struct abp_params {
  int32_t num_qo_heads;
  int32_t num_kv_heads;
  int32_t head_dim;   /* 128 */
  int32_t page_size;  /* >= 1 */
  int32_t qkv_dtype;  /* ABP_F16 or ABP_BF16 */
  int32_t out_dtype;  /* ABP_F16, ABP_BF16 or ABP_F32 */
  float sm_scale;     /* <= 0 selects 1/sqrt(head_dim) */
  int32_t causal;     /* append only: 1 = causal mask aligned to the end of the KV */
  int32_t rope;       /* 0 = none, 1 = LLaMA rotate-half RoPE on q and k at load,
                         2 = the same with LLaMA 3.1 frequency scaling */
  float rope_theta;   /* RoPE base, e.g. 500000 */
  /* rope = 2 only (LLaMA 3.1 settings: 8, 1, 4, 8192); ignored otherwise */
  float rope_factor;            /* > 0 */
  float rope_low_freq_factor;   /* > 0 */
  float rope_high_freq_factor;  /* > rope_low_freq_factor */
  float rope_old_context_len;   /* > 0 */
  /* KV cache storage: 0 = qkv_dtype; 1 = OCP FP8 E4M3 codes (one byte per element,
     same page layout), whose values are k_scale (keys) or v_scale (values) times
     the codes' values. Decode and page append only. The README page (section
     特性) names FP8 attention without a scaling scheme: one scale per tensor. */
  int32_t kv_fp8;
  float k_scale;                /* > 0 when kv_fp8 = 1; ignored otherwise */
  float v_scale;                /* > 0 when kv_fp8 = 1; ignored otherwise */
  /* RoPE pairing (rope != 0): 0 = rotate-half pairs (j, j + head_dim/2);
     1 = adjacent pairs (2j, 2j + 1), the complex-number form */
  int32_t rope_interleave;
} abp_params;

/* Result of a plan: plain data, copied by value. Fields are informative; only
 * the library interprets them. */
typedef struct abp_plan {
  int32_t kind;          /* abp_kind */
  int32_t batch;
  int32_t num_workers;   /* grid size of the persistent kernel */
  int32_t tile_q;        /* query tokens per tile (1 for decode) */
  int32_t tile_kv;       /* keys per work block */
  int32_t rows_per_tile; /* append: tile_q * group; decode: group * kv heads per
                            tile (4 consecutive kv heads when num_kv_heads is a
                            multiple of 4, else 1) */
  int32_t num_tiles;
  int32_t num_segments;
  int32_t num_partials;  /* partial (o, lse) slots used by split tiles */
  int32_t num_merges;    /* tiles whose partial states are merged */
  int32_t max_tiles;     /* capacities fixed by (max_batch, max_qo_tokens, workers) */
  int32_t max_segments;
  int32_t max_partials;
  int32_t upload_path;   /* 1: a kernel read the pinned host_ws; 0: hipMemcpyAsync */
  uint64_t fingerprint;  /* hash of kind, params, capacities and tiling */
  uint64_t plan_bytes;   /* bytes uploaded from the host workspace */
  uint64_t partial_offset; /* byte offset of the partial-state region in dev_ws */
  uint64_t dev_bytes;    /* device workspace bytes this layout needs */
} abp_plan;

/* Static text for a status code. */
const char* abp_status_string(int status);

/* Message of the calling thread's last failing call ("" if none). */
const char* abp_last_error(void);

/* Number of compute units of HIP device `device` (cached). */
int abp_device_num_cus(int device, int32_t* num_cus);

/* num_workers value selecting the plan without load balancing, as an ablation
 * of the Stream-K split (paper summary, section 动态负载均衡调度): one worker
 * per tile, each tile one segment, no partial states. The grid is then the
 * tile capacity of the workspace (max_batch x kv-head groups for decode). */
#define ABP_WORKERS_PER_TILE (-1)

/* Workspace sizes for plans of `kind` with at most `max_batch` requests,
 * `max_qo_tokens` query tokens (append; ignored for decode) and `num_workers`
 * workers (ABP_WORKERS_PER_TILE: one per tile, no split; other values <= 0:
 * one per resident workgroup slot of the current device, i.e. compute units
 * times the workgroups of the selected kernel that fit on one).
 * Pure host code except the device query for num_workers <= 0. */
int abp_workspace_size(int kind, const abp_params* params, int32_t max_batch,
                       int32_t max_qo_tokens, int32_t num_workers, size_t* host_bytes,
                       size_t* dev_bytes);

/* The planner alone (host only, no HIP call): validate the index arrays and
 * write the plan into `host_ws` (>= host_bytes of abp_workspace_size).
 * qo_indptr_h is read for ABP_KIND_APPEND only. num_workers must be > 0 or
 * ABP_WORKERS_PER_TILE.
 * Work is cut into blocks of tile_kv keys and spread over the workers in equal
 * contiguous ranges (Stream-K), paper summary section 动态负载均衡调度. Append
 * plans whose num_workers is a multiple of 8 spread it over groups of K
 * workers instead (K = the largest of 8, 4, 2 dividing num_workers / 8), each
 * group running K query tiles of one (request, kv head) side by side on one
 * XCD; the outputs are the same up to rounding order. */
int abp_plan_host(int kind, const abp_params* params, int32_t batch, const int32_t* qo_indptr_h,
                  const int32_t* kv_indptr_h, const int32_t* kv_last_page_len_h,
                  int32_t max_batch, int32_t max_qo_tokens, int32_t num_workers, void* host_ws,
                  size_t host_bytes, abp_plan* plan);

/* Decode plan: abp_plan_host for ABP_KIND_DECODE, then the upload of the plan
 * from host_ws to dev_ws on `stream`. If host_ws is pinned host memory mapped at
 * the same address on the GPU (hipHostMalloc), a small kernel on `stream` reads
 * it directly (plan->upload_path = 1); otherwise hipMemcpyAsync copies it
 * (upload_path = 0). Either way host_ws must stay unchanged until the upload
 * has executed on the stream. */
int abp_decode_plan(const abp_params* params, int32_t batch, const int32_t* kv_indptr_h,
                    const int32_t* kv_last_page_len_h, int32_t max_batch, int32_t num_workers,
                    void* host_ws, size_t host_bytes, void* dev_ws, size_t dev_bytes,
                    abp_stream_t stream, abp_plan* plan);

/* Batch decode over the paged cache (one query token per request).
 * q [batch, Hq, d]; o [batch, Hq, d] (out_dtype); lse [batch, Hq] float32 or NULL.
 * q_pos_d [batch] and kv_pos_offset_d [batch] are read only with RoPE (NULL =
 * defaults). Launches the persistent decode kernel (grid = num_workers), then a
 * merge kernel (same grid) that combines the partial states of split tiles.
 * Partial states live in dev_ws: runs that share one dev_ws must not overlap.
 * The tensor pointers may be NULL only when the plan has no tiles (batch 0);
 * otherwise NULL gives ABP_ERR_INVALID_ARG. */
int abp_decode_run(const abp_plan* plan, const abp_params* params, const void* q,
                   const void* k_pages, const void* v_pages, const int32_t* kv_indptr_d,
                   const int32_t* kv_indices_d, const int32_t* kv_last_page_len_d,
                   const int32_t* q_pos_d, const int32_t* kv_pos_offset_d, void* o, float* lse,
                   void* dev_ws, size_t dev_bytes, abp_stream_t stream);

/* Append / prefill plan for ragged queries (qo_indptr_h [batch + 1]); uploads
 * like abp_decode_plan. */
int abp_append_plan(const abp_params* params, int32_t batch, const int32_t* qo_indptr_h,
                    const int32_t* kv_indptr_h, const int32_t* kv_last_page_len_h,
                    int32_t max_batch, int32_t max_qo_tokens, int32_t num_workers,
                    void* host_ws, size_t host_bytes, void* dev_ws, size_t dev_bytes,
                    abp_stream_t stream, abp_plan* plan);

/* Append / prefill attention (MFMA): q [total_qo, Hq, d] ragged by qo_indptr_d;
 * o [total_qo, Hq, d]; lse [total_qo, Hq] or NULL. Causal per params.causal.
 * q_pos_d [total_qo] and kv_pos_offset_d [batch] are read only with RoPE.
 * Launches the persistent append kernel (grid = num_workers), then a merge
 * kernel (same grid). A tile split over at most 4 workers is merged inside the
 * append kernel by the workgroup whose partial arrives last, counted with
 * per-tile counters in dev_ws that the merging workgroup resets to zero (every
 * plan upload also zeroes them); when some tile has more partials, the plan
 * leaves all merges to the merge kernel, which otherwise returns at once. Runs
 * that share one dev_ws must not overlap. The tensor pointers may be NULL only
 * when the plan has no tiles (no query tokens in the batch). */
int abp_append_run(const abp_plan* plan, const abp_params* params, const void* q,
                   const void* k_pages, const void* v_pages, const int32_t* qo_indptr_d,
                   const int32_t* kv_indptr_d, const int32_t* kv_indices_d,
                   const int32_t* kv_last_page_len_d, const int32_t* q_pos_d,
                   const int32_t* kv_pos_offset_d, void* o, float* lse, void* dev_ws,
                   size_t dev_bytes, abp_stream_t stream);

/* Block-sparse attention (README page, section 核心功能: block-sparse and
 * variable block-sparse attention; paper summary, section 统一的 KV 缓存存储格式:
 * one BSR format with a configurable block size serves every layout).
 *
 * A mask over q [M, Hq, d] and a dense k / v [N, Hkv, d] (qkv_dtype) in block-
 * sparse-row form: row block i holds queries [i R, min((i+1) R, M)) and sees the
 * column blocks indices[indptr[i] .. indptr[i+1]) of C = params->page_size keys
 * each (key block j = keys [j C, (j+1) C)); query r sees key t exactly when the
 * block (r / R, t / C) is listed. indptr has ceil(M / R) + 1 entries, indptr[0] = 0,
 * non-decreasing; indices are column block ids in [0, N / C) in any order, each
 * at most once per row (a repeated block would count its keys twice). A query
 * whose row block lists nothing gets o = 0, lse = -inf. Requires N % C == 0,
 * params->causal = 0 and params->rope = 0.
 *
 * Each row block is run as one append request whose pages are its column
 * blocks (k viewed as [N / C, C, Hkv, d]); the planner writes the derived
 * query ranges and page counts into the plan blob, so the run needs only the
 * caller's indptr / indices on the device.
 *
 * Workspace: abp_workspace_size(ABP_KIND_BSR, params, max_row_blocks, max_M,
 * num_workers, ...). abp_bsr_plan_host plans on the host only; abp_bsr_plan
 * also uploads like abp_decode_plan. */
int abp_bsr_plan_host(const abp_params* params, int32_t M, int32_t N, int32_t R,
                      const int32_t* indptr_h, int32_t max_row_blocks, int32_t max_M,
                      int32_t num_workers, void* host_ws, size_t host_bytes, abp_plan* plan);
int abp_bsr_plan(const abp_params* params, int32_t M, int32_t N, int32_t R,
                 const int32_t* indptr_h, int32_t max_row_blocks, int32_t max_M,
                 int32_t num_workers, void* host_ws, size_t host_bytes, void* dev_ws,
                 size_t dev_bytes, abp_stream_t stream, abp_plan* plan);

/* Block-sparse attention run (the append MFMA kernel, then the merge kernel):
 * q [M, Hq, d], k / v [N, Hkv, d], indptr_d / indices_d as planned (device
 * copies); o [M, Hq, d] (out_dtype), lse [M, Hq] float32 or NULL. Tensor
 * pointers may be NULL only when M = 0. Same workspace rules as abp_append_run. */
int abp_bsr_run(const abp_plan* plan, const abp_params* params, const void* q, const void* k,
                const void* v, const int32_t* indptr_d, const int32_t* indices_d, void* o,
                float* lse, void* dev_ws, size_t dev_bytes, abp_stream_t stream);

/* Write new tokens into a paged KV cache (the step that fills the pages before
 * decode / append read them; README page, section 核心功能: paged KV caches).
 * k_new / v_new [nnz, Hkv, d] (params->qkv_dtype) are ragged by
 * append_indptr_d [batch + 1] (append_indptr[batch] = nnz). The page table
 * (kv_indptr_d, kv_indices_d, kv_last_page_len_d, as in abp_decode_run) must
 * already cover the new tokens, which are the last ones of each request: new
 * row i of request b is logical token kv_len_b - append_len_b + i, stored in
 * slot t % page_size of page kv_indices[kv_indptr[b] + t / page_size]. Rows whose
 * position falls outside [0, kv_len_b) are skipped. Only num_kv_heads,
 * head_dim, page_size, qkv_dtype and kv_fp8 of params are used (with kv_fp8 the
 * rows and pages hold e4m3 codes, one byte per element). One kernel on `stream`,
 * no allocation, graph-capturable. All arrays are device memory; nnz = 0 is a
 * no-op. */
int abp_append_paged_kv(const abp_params* params, int32_t batch, int64_t nnz, const void* k_new,
                        const void* v_new, const int32_t* append_indptr_d, void* k_pages,
                        void* v_pages, const int32_t* kv_indptr_d, const int32_t* kv_indices_d,
                        const int32_t* kv_last_page_len_d, abp_stream_t stream);

/* Mixed batches: decode requests and append (prefill) requests in one plan and
 * one persistent launch (the POD kernels of the README page, section 核心功能 /
 * 注意力机制内核). Decode is bound by HBM bandwidth and append by the matrix
 * cores; the launch gives num_groups workgroups (one per compute unit) one
 * role each, decode or append, so both run at the same time.
 *
 * The plan holds two sub-plans, each exactly what abp_plan_host makes for its
 * kind with its own worker count: decode.num_workers decode workers and
 * append.num_workers = num_groups - decode.num_workers append workers (0 when
 * that part has no request). The split is decode_groups if > 0 (clamped so
 * each part with requests keeps at least one workgroup); otherwise the planner
 * chooses it so that both parts are predicted to end together, from the
 * decode part's K/V bytes against a measured curve of decode bandwidth over
 * compute units and the append part's visible (query, key) pairs at the
 * append kernel's measured rate per compute unit. Outputs are those of
 * abp_decode_run and abp_append_run on the two parts.
 *
 * Requires: no RoPE, 16-bit K/V (no kv_fp8), a power-of-two page_size >= 16,
 * num_kv_heads a multiple of 4, group 4 or 8 (ABP_ERR_UNSUPPORTED otherwise).
 * params->causal applies to the append part. Both parts read the same page
 * pools (k_pages, v_pages) through their own page tables.
 *
 * Workspace: abp_pod_workspace_size; the host and device workspaces hold the
 * decode sub-plan, then the append one, at the offsets the plan records.
 * num_groups <= 0 means the compute units of the current device. */
typedef struct abp_pod_plan_t {
  abp_plan decode;             /* decode sub-plan (num_workers 0: no decode part) */
  abp_plan append;             /* append sub-plan (num_workers 0: no append part) */
  int32_t num_groups;          /* workgroups of the launch */
  int32_t reserved;
  uint64_t decode_host_offset, append_host_offset; /* byte offsets in host_ws */
  uint64_t decode_dev_offset, append_dev_offset;   /* byte offsets in dev_ws */
  uint64_t decode_dev_bytes, append_dev_bytes;     /* device region sizes */
} abp_pod_plan_t;

int abp_pod_workspace_size(const abp_params* params, int32_t max_decode_batch,
                           int32_t max_append_batch, int32_t max_qo_tokens, int32_t num_groups,
                           size_t* host_bytes, size_t* dev_bytes);

/* Host-only planning (no HIP call when num_groups > 0): validates both parts'
 * index arrays as abp_plan_host does. The decode part has decode_batch
 * requests (d_*), the append part append_batch requests (qo_indptr_h, a_*). */
int abp_pod_plan_host(const abp_params* params, int32_t decode_batch,
                      const int32_t* d_kv_indptr_h, const int32_t* d_kv_last_page_len_h,
                      int32_t append_batch, const int32_t* qo_indptr_h,
                      const int32_t* a_kv_indptr_h, const int32_t* a_kv_last_page_len_h,
                      int32_t max_decode_batch, int32_t max_append_batch, int32_t max_qo_tokens,
                      int32_t num_groups, int32_t decode_groups, void* host_ws,
                      size_t host_bytes, abp_pod_plan_t* plan);

/* abp_pod_plan_host, then the upload of both sub-plans to dev_ws on `stream`
 * (as abp_decode_plan). */
int abp_pod_plan(const abp_params* params, int32_t decode_batch, const int32_t* d_kv_indptr_h,
                 const int32_t* d_kv_last_page_len_h, int32_t append_batch,
                 const int32_t* qo_indptr_h, const int32_t* a_kv_indptr_h,
                 const int32_t* a_kv_last_page_len_h, int32_t max_decode_batch,
                 int32_t max_append_batch, int32_t max_qo_tokens, int32_t num_groups,
                 int32_t decode_groups, void* host_ws, size_t host_bytes, void* dev_ws,
                 size_t dev_bytes, abp_stream_t stream, abp_pod_plan_t* plan);

/* One launch of num_groups workgroups runs both parts, then the plan-merge
 * launches of each part merge their split tiles. q_decode [decode_batch, Hq,
 * d] -> o_decode / lse_decode as abp_decode_run; q_append [total_qo_tokens,
 * Hq, d] -> o_append / lse_append as abp_append_run (lse pointers may be
 * NULL). Device index arrays as planned. No allocation; graph-capturable. A
 * captured run keeps the worker counts of the plan it was captured with, so it
 * may be replayed after a re-plan only if both sub-plans keep theirs: pass the
 * same decode_groups and num_groups, keep both parts non-empty and keep the
 * capacities. */
int abp_pod_run(const abp_pod_plan_t* plan, const abp_params* params, const void* q_decode,
                const void* q_append, const void* k_pages, const void* v_pages,
                const int32_t* d_kv_indptr_d, const int32_t* d_kv_indices_d,
                const int32_t* d_kv_last_page_len_d, const int32_t* qo_indptr_d,
                const int32_t* a_kv_indptr_d, const int32_t* a_kv_indices_d,
                const int32_t* a_kv_last_page_len_d, void* o_decode, float* lse_decode,
                void* o_append, float* lse_append, void* dev_ws, size_t dev_bytes,
                abp_stream_t stream);

/* Cascade decode in one call: a shared prefix level and a per-request suffix
 * level whose attention states are recombined (paper summary "图谱动态｜学苑周刊
 * NO.266", section 统一的 KV 缓存存储格式, composable formats). Runs the
 * prefix append kernel (non-causal, one request whose query tokens are the B
 * decode queries, its own page pool and table), the suffix decode kernel (B
 * requests, their own pool and table), then one merge launch that folds, for
 * every (request, qo head) row, the prefix level's state and the suffix
 * level's state, each read either from the level's fp32 output (an unsplit
 * tile) or from the level's partial slots (a split tile), so neither level
 * runs its own plan merge. Equals merge_state(prefix run, suffix run).
 *
 * Plans: prefix_plan from abp_append_plan with qo_indptr = [0, B] and
 * causal 0; suffix_plan from abp_decode_plan over the B suffixes; both params
 * with out_dtype ABP_F32 (the level states) and the same heads and q dtype
 * (ABP_ERR_PLAN_MISMATCH / ABP_ERR_UNSUPPORTED otherwise). Each plan keeps
 * its own device workspace. q [B, Hq, d] is both levels' query; RoPE (when
 * the params enable it): query b at q_pos_d[b] (NULL: each level's default),
 * prefix key t at t, suffix key t at kv_pos_offset_d[b] + t. o_prefix /
 * o_suffix [B, Hq, d] and lse_prefix / lse_suffix [B, Hq] are fp32 scratch
 * for the levels' direct states (caller-owned, contents undefined after the
 * call); o [B, Hq, d] in out_dtype and lse [B, Hq] (may be NULL) receive the
 * result. No allocation; graph-capturable under the same conditions as the
 * two runs. */
int abp_cascade_run(const abp_plan* prefix_plan, const abp_params* prefix_params,
                    void* prefix_dev_ws, size_t prefix_dev_bytes, const abp_plan* suffix_plan,
                    const abp_params* suffix_params, void* suffix_dev_ws, size_t suffix_dev_bytes,
                    const void* q, const void* prefix_k_pages, const void* prefix_v_pages,
                    const int32_t* prefix_qo_indptr_d, const int32_t* prefix_kv_indptr_d,
                    const int32_t* prefix_kv_indices_d, const int32_t* prefix_kv_last_page_len_d,
                    const void* k_pages, const void* v_pages, const int32_t* kv_indptr_d,
                    const int32_t* kv_indices_d, const int32_t* kv_last_page_len_d,
                    const int32_t* q_pos_d, const int32_t* kv_pos_offset_d, float* o_prefix,
                    float* lse_prefix, float* o_suffix, float* lse_suffix, void* o, float* lse,
                    int32_t out_dtype, abp_stream_t stream);

/* Merge two attention states over disjoint key sets (cascade: prefix and suffix).
 * o_a, o_b [num_rows, head_dim] in in_dtype; lse_a, lse_b [num_rows] float32;
 * writes o_out [num_rows, head_dim] in out_dtype and lse_out (may be NULL).
 * lse = ln(e^lse_a + e^lse_b); o = e^(lse_a - lse) o_a + e^(lse_b - lse) o_b;
 * two -inf states give (0, -inf). num_rows counts (token, head) pairs. */
int abp_merge_state(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                    void* o_out, float* lse_out, int64_t num_rows, int32_t head_dim,
                    int in_dtype, int out_dtype, abp_stream_t stream);

/* Merge `num_states` states stacked on a leading axis: o_in [num_states,
 * num_rows, head_dim] (in_dtype), lse_in [num_states, num_rows] float32 ->
 * o_out [num_rows, head_dim] (out_dtype), lse_out [num_rows] (may be NULL). */
int abp_merge_states(const void* o_in, const float* lse_in, int32_t num_states,
                     int64_t num_rows, int32_t head_dim, int in_dtype, int out_dtype,
                     void* o_out, float* lse_out, abp_stream_t stream);

/* Batch decode without any allocation, for callers that cannot allocate
 * (code under graph capture, tight serving loops, harnesses that forbid
 * allocation). Computes exactly abp_decode_plan followed by abp_decode_run
 * (same plan, same kernels, bit-identical results), but the caller passes no
 * workspace: the library keeps a device array of ABP_STATIC_SCRATCH_BYTES on
 * each GPU it runs on (allocated with the code object, held until the process
 * ends) for the plan blob and partial states, and a host array of
 * ABP_STATIC_PLAN_BYTES for the plan. Arguments are those of the two calls:
 * host kv_indptr_h [batch + 1] and kv_last_page_len_h [batch] for the plan
 * (validated as in abp_decode_plan), num_workers <= 0 for the device default,
 * and the device tensors of abp_decode_run. A batch whose plan or workspace
 * exceeds those sizes returns ABP_ERR_WORKSPACE_TOO_SMALL before any GPU work
 * (with 8 kv heads, group 4 or 8 and the default 256 workers, up to about
 * 12,000 requests fit; the device array holds the partial states of up to
 * 1024 workers at group 8, 2048 at group 4).
 * The plan is copied from pageable host memory, a copy HIP performs
 * synchronously with respect to the host; then the decode and merge kernels
 * are enqueued on `stream`. Not graph-capturable itself (the copy). Every
 * call on a GPU shares that GPU's scratch: calls on one stream are ordered,
 * calls that overlap on one GPU (other streams or threads) race. */
#define ABP_STATIC_SCRATCH_BYTES (32u << 20)
#define ABP_STATIC_PLAN_BYTES (1u << 20)
int abp_decode_static(const abp_params* params, int32_t batch, const int32_t* kv_indptr_h,
                      const int32_t* kv_last_page_len_h, int32_t num_workers, const void* q,
                      const void* k_pages, const void* v_pages, const int32_t* kv_indptr_d,
                      const int32_t* kv_indices_d, const int32_t* kv_last_page_len_d,
                      const int32_t* q_pos_d, const int32_t* kv_pos_offset_d, void* o,
                      float* lse, abp_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ABP_H_ */
