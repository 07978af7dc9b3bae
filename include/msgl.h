/*
 * msgl.h -- C ABI of libmsgl.so: attention over a paged KV cache on MI355X
 * (gfx950).
 *
 * The objects follow the Mini-SGLang pages:
 *   - the KV pool is one bf16 tensor shaped
 *     (2, num_layers, num_pages, page_size, num_kv_heads, head_dim), leading
 *     index 0 = K, 1 = V ("Code Notes: mini-sglang", section "Engine Layer:
 *     how to compute", table row BaseKVCachePool);
 *   - store_kv writes new K/V rows into it "by out_loc indices" (same row);
 *   - each request's KV is reached through one row of page_table, the row
 *     picked by table_idx (same page, section "Scheduler Layer: what to
 *     compute", table row TableManager);
 *   - prefill/extend and decode are separate calls, as the HybridBackend
 *     keeps separate prefill and decode backends (same page, Engine Layer
 *     table, row BaseAttnBackend; "Code Structure", Attention Backends).
 *
 * Conventions shared by every call:
 *   - A page_table entry is a page id in [0, num_pages).  Token p of a request
 *     lives in slot page_table[row*page_table_stride + p / page_size] *
 *     page_size + p % page_size of the (num_pages*page_size, num_kv_heads,
 *     head_dim) view of one (K or V, layer).  out_loc entries are such slots.
 *   - q head h reads kv head h / (num_qo_heads / num_kv_heads).
 *   - All pointers except the pool struct itself are device pointers.  The
 *     caller owns every buffer; the library allocates no device memory and
 *     keeps no state between calls other than a per-device architecture
 *     check -- except the decode-graph objects, which the caller creates
 *     and destroys explicitly.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *     default stream) and performs no host synchronisation, so calls are
 *     ordered by the stream: store_kv before the attention that reads it.
 *   - Errors are returned, never thrown: scalar arguments are validated on
 *     the host before any launch, and nothing is launched on error.  Device
 *     contents (slots, page ids, table_idx, lengths) are the caller's
 *     contract; with the environment variable MSGL_CHECK=1 each call copies
 *     them to the host (a synchronisation) and returns MSGL_ERR_RANGE when
 *     one is out of range, without launching.
 *   - dtype is bf16 for pool, q, k, v and out; attention arithmetic is fp32.
 *     head_dim must be 64 or 128, num_qo_heads a multiple of num_kv_heads
 *     with a ratio of at most 16, page_size >= 1.  q/k/v/out/pool pointers
 *     and row strides must be 16-byte aligned (strides a multiple of 8
 *     elements) for the attention calls; store_kv accepts any alignment.
 *   - Padding conventions for fixed-size batches: out_loc[t] < 0 skips row
 *     t; seq_lens[r] == 0 in decode writes zeros and reads no KV.
 *   - The attention calls address one (K or V, layer) sub-tensor of the pool
 *     with 32-bit byte offsets: num_pages*page_size*num_kv_heads*head_dim*2
 *     must be below 2^32 (MSGL_ERR_UNSUPPORTED otherwise); larger pools can
 *     be split into several pool structs.  sm_scale must be > 0.
 */
#ifndef MSGL_H
#define MSGL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSGL_ABI_VERSION 2

typedef int32_t msgl_status;
#define MSGL_OK 0
#define MSGL_ERR_NULL 1        /* a required pointer is NULL */
#define MSGL_ERR_SHAPE 2       /* inconsistent sizes, strides or alignment */
#define MSGL_ERR_UNSUPPORTED 3 /* head_dim, group size or device not supported */
#define MSGL_ERR_WORKSPACE 4   /* decode workspace too small */
#define MSGL_ERR_RANGE 5       /* checked mode: a device index/length out of range */
#define MSGL_ERR_HIP 6         /* a HIP runtime call or launch failed */

/* The KV pool: `data` is a device pointer to a contiguous bf16 tensor of
 * shape (2, num_layers, num_pages, page_size, num_kv_heads, head_dim).
 * The struct itself is read on the host during the call only. */
typedef struct msgl_kv_pool {
  void* data;
  int32_t num_layers;
  int32_t num_pages;
  int32_t page_size;
  int32_t num_kv_heads;
  int32_t head_dim;
} msgl_kv_pool;

/* Version of this ABI (MSGL_ABI_VERSION). */
int32_t msgl_abi_version(void);

/* Static English text for a status code; never NULL. */
const char* msgl_status_string(msgl_status status);

/*
 * store_kv: for t < num_tokens with out_loc[t] >= 0, copy row t of k into
 * K[layer] slot out_loc[t] and row t of v into V[layer] slot out_loc[t]
 * ("Code Notes: mini-sglang", Engine Layer table, BaseKVCachePool row).
 *   k, v        : (num_tokens, num_kv_heads, head_dim) bf16; heads and dims
 *                 contiguous inside a row, rows `k_row_stride` /
 *                 `v_row_stride` elements apart (>= num_kv_heads*head_dim),
 *                 so slices of a merged QKV projection can be passed as is.
 *   out_loc     : (num_tokens,) int32 slots in [0, num_pages*page_size), or
 *                 negative for padding rows.  Slots must be distinct.
 * A bit-exact copy: no value is converted.  num_tokens == 0 is a no-op.
 */
msgl_status msgl_store_kv(const msgl_kv_pool* pool, int32_t layer, const void* k,
                          int64_t k_row_stride, const void* v, int64_t v_row_stride,
                          const int32_t* out_loc, int32_t num_tokens, void* stream);

/*
 * Bytes of workspace msgl_paged_decode needs for a batch with these sizes:
 * a map of each request's pieces, and the fp32 partial outputs, with their
 * softmax statistics, of requests split over several workgroups.  It
 * depends on batch, num_qo_heads, head_dim and max_seq_len only (page_size
 * is accepted and checked, >= 1, but does not change the layout: the
 * decode splits tokens, not pages), and it grows with batch and
 * max_seq_len, so a workspace sized once for the largest batch and
 * max_seq_len serves every smaller call.  Returns 0 for batch 0 and for
 * invalid sizes.
 */
size_t msgl_paged_decode_workspace_size(int32_t batch, int32_t num_qo_heads, int32_t head_dim,
                                        int32_t max_seq_len, int32_t page_size);

/*
 * paged_decode: one query token per request attends to all seq_lens[r]
 * tokens of its KV (the new token's row already stored by store_kv), read
 * through page_table row table_idx[r] ("Code Notes: mini-sglang", Engine
 * Layer table rows BaseAttnBackend and GraphRunner -- decode batches of one
 * new token per request; Scheduler Layer table, TableManager row).
 *   out[r, h, :] = sum_j softmax_j(sm_scale * q[r,h,:] . K_j[h/G]) V_j[h/G]
 *   q           : (batch, num_qo_heads, head_dim) bf16, rows q_row_stride
 *                 elements apart.
 *   out         : (batch, num_qo_heads, head_dim) bf16, contiguous.
 *   page_table  : int32, row-major with page_table_stride entries per row;
 *                 row table_idx[r] must hold >= ceil(seq_lens[r]/page_size)
 *                 valid page ids (entries past that are never read).
 *   table_idx   : (batch,) int32 row indices.
 *   seq_lens    : (batch,) int32 in [0, max_seq_len]; 0 marks a padding row.
 *   max_seq_len : host-side bound used to size the grid and the workspace;
 *                 at most 1,048,511 tokens (MSGL_ERR_UNSUPPORTED beyond).
 *   sm_scale    : softmax scale, normally 1/sqrt(head_dim).
 *   workspace   : device buffer, 256-byte aligned, of >=
 *                 msgl_paged_decode_workspace_size(batch, num_qo_heads,
 *                 head_dim, max_seq_len, page_size) bytes; its contents
 *                 need no initialisation.  Calls that share a workspace must
 *                 not overlap in time (same stream, or synchronised).
 * The batch's tokens are split evenly over the workgroups, so a long
 * sequence is processed by several of them in parallel; a second kernel on
 * the same stream merges the partial results with a log-sum-exp combine.
 * Batches above 2048 requests are processed 2048 at a time.
 */
msgl_status msgl_paged_decode(const msgl_kv_pool* pool, int32_t layer, const void* q,
                              int64_t q_row_stride, void* out, const int32_t* page_table,
                              int32_t page_table_stride, const int32_t* table_idx,
                              const int32_t* seq_lens, int32_t batch, int32_t num_qo_heads,
                              int32_t max_seq_len, float sm_scale, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * paged_decode_noalloc: msgl_paged_decode for callers that cannot allocate
 * device memory -- code under graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments and result as msgl_paged_decode,
 * without the workspace: the call uses a device array inside the library
 * (64 MiB, msgl_paged_decode_noalloc_max_workspace(), one per GPU, held
 * until the process ends) and allocates nothing.  A call whose
 * msgl_paged_decode_workspace_size(...) exceeds that limit returns
 * MSGL_ERR_WORKSPACE before touching the GPU.  Every call on a GPU shares
 * that GPU's array: calls that overlap in time on one GPU (different
 * streams not ordered by events, or several threads) race and give wrong
 * results; order them.
 */
size_t msgl_paged_decode_noalloc_max_workspace(void);
msgl_status msgl_paged_decode_noalloc(const msgl_kv_pool* pool, int32_t layer, const void* q,
                                      int64_t q_row_stride, void* out, const int32_t* page_table,
                                      int32_t page_table_stride, const int32_t* table_idx,
                                      const int32_t* seq_lens, int32_t batch, int32_t num_qo_heads,
                                      int32_t max_seq_len, float sm_scale, void* stream);

/*
 * paged_extend: causal prefill/extend over a cached prefix.  Request r has
 * prefix_lens[r] tokens already in the pool (a radix-cache hit or earlier
 * prefill chunks) and extend_lens[r] new tokens, already stored, whose
 * queries are rows cu_extend_lens[r] .. cu_extend_lens[r+1]-1 of q.  New
 * token i sits at position prefix_lens[r] + i and attends to keys
 * 0 .. prefix_lens[r] + i ("Code Notes: mini-sglang", Scheduler Layer table
 * row PrefillManager -- chunked prefill; "Introduction", Key Features --
 * Radix Cache and Chunked Prefill).  Rows of different requests may share
 * page ids (shared prefixes).
 *   q, out         : (total_extend_tokens, num_qo_heads, head_dim) bf16; q
 *                    rows q_row_stride elements apart, out contiguous.
 *   cu_extend_lens : (batch+1,) int32 exclusive prefix sum of extend_lens.
 *   max_extend_len : host-side bound on extend_lens (sizes the grid).
 *   max_seq_len    : host-side bound on prefix_lens + extend_lens.
 * Requests with extend_lens[r] == 0 produce no rows.
 */
msgl_status msgl_paged_extend(const msgl_kv_pool* pool, int32_t layer, const void* q,
                              int64_t q_row_stride, void* out, const int32_t* page_table,
                              int32_t page_table_stride, const int32_t* table_idx,
                              const int32_t* prefix_lens, const int32_t* extend_lens,
                              const int32_t* cu_extend_lens, int32_t batch,
                              int32_t total_extend_tokens, int32_t max_extend_len,
                              int32_t max_seq_len, int32_t num_qo_heads, float sm_scale,
                              void* stream);

/*
 * paged_extend_split: msgl_paged_extend for calls too small to give every
 * compute unit a workgroup (a short prefill, few requests, or few kv heads
 * as on a tensor-parallel GPU's share): each row tile's keys are split
 * into shares, one workgroup each, and a second kernel on the same stream
 * combines the shares with a log-sum-exp merge (the passages cited for
 * paged_extend; the split itself is this library's, the pages are silent).
 * Same arguments and result as msgl_paged_extend, within the attention
 * tolerance (the shares round to fp32 before the merge), plus:
 *   workspace : device buffer, 256-byte aligned, of >=
 *               msgl_paged_extend_workspace_size(pool, total_extend_tokens,
 *               max_seq_len, num_qo_heads) bytes; no initialisation needed.
 *               NULL, or a size of 0 from that function (a call large
 *               enough to fill the device), runs msgl_paged_extend.
 * The size depends on the current device's compute-unit count and on
 * MSGL_EXTEND_SPLITS (n forces n shares, 1 to 8), so size the workspace on
 * the device and in the process that makes the call.  Returns
 * MSGL_ERR_WORKSPACE for a smaller workspace.  Calls sharing a workspace
 * must not overlap in time.
 */
size_t msgl_paged_extend_workspace_size(const msgl_kv_pool* pool, int32_t total_extend_tokens,
                                        int32_t max_seq_len, int32_t num_qo_heads);
msgl_status msgl_paged_extend_split(const msgl_kv_pool* pool, int32_t layer, const void* q,
                                    int64_t q_row_stride, void* out, const int32_t* page_table,
                                    int32_t page_table_stride, const int32_t* table_idx,
                                    const int32_t* prefix_lens, const int32_t* extend_lens,
                                    const int32_t* cu_extend_lens, int32_t batch,
                                    int32_t total_extend_tokens, int32_t max_extend_len,
                                    int32_t max_seq_len, int32_t num_qo_heads, float sm_scale,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * rope_store_kv: rotary position embedding of this step's new rows, fused
 * with store_kv ("Code Structure", section Model Layers, get_rope --
 * rotary position embeddings; "Code Notes: mini-sglang", Engine Layer
 * table, BaseKVCachePool row for the store).  For t < num_tokens, with p = positions[t]:
 *   q[t, h, :] <- rope(q[t, h, :], p) in place, for every q head h;
 *   K[layer] slot out_loc[t] <- rope(k[t], p), V[layer] slot <- v[t]
 *   (rows with out_loc[t] < 0 store nothing; q is still rotated).
 * rope pairs channel i < d/2 with channel i + d/2 and turns the pair by the
 * angle whose cosine and sine are cos_sin_table[p*head_dim + i] and
 * cos_sin_table[p*head_dim + head_dim/2 + i]:
 *   y_i = x_i cos - x_{i+d/2} sin,  y_{i+d/2} = x_{i+d/2} cos + x_i sin.
 * Each output is the exact value rounded once to bf16 (fp64 arithmetic).
 *   q            : (num_tokens, num_qo_heads, head_dim) bf16, rows
 *                  q_row_stride elements apart; may be NULL when
 *                  num_qo_heads == 0.
 *   k, v         : (num_tokens, num_kv_heads, head_dim), as for store_kv.
 *   positions    : (num_tokens,) int32 in [0, max_position) (values outside
 *                  are the caller's contract; they are clamped).
 *   cos_sin_table: (max_position, head_dim) fp32, e.g. from
 *                  msgl_rope_cos_sin_table.
 * head_dim 64 or 128; q/k/v/pool 16-byte aligned with row strides a
 * multiple of 8 elements; q rows must not overlap k or v rows.
 */
msgl_status msgl_rope_store_kv(const msgl_kv_pool* pool, int32_t layer, void* q,
                               int64_t q_row_stride, int32_t num_qo_heads, const void* k,
                               int64_t k_row_stride, const void* v, int64_t v_row_stride,
                               const int32_t* out_loc, const int32_t* positions,
                               int32_t num_tokens, const float* cos_sin_table,
                               int32_t max_position, void* stream);

/*
 * rope_cos_sin_table: fill table (max_position, head_dim) fp32 with
 * cos(p * base^(-2i/d)) in columns i < d/2 and the sines in columns
 * d/2 + i -- the angles, cosines and sines computed in fp64 and rounded
 * once to fp32.  head_dim even and > 0, max_position > 0, base > 0.
 */
msgl_status msgl_rope_cos_sin_table(float* table, int32_t max_position, int32_t head_dim,
                                    double base, void* stream);

/*
 * alloc_pages: device-side page allocation for one scheduling step
 * ("Code Notes: mini-sglang", Scheduler Layer table: CacheManager row --
 * free_slots, the free positions handed out to new tokens; TableManager
 * row -- one page_table row per request).  With P_r = prefix_lens[r]
 * tokens already held (ceil(P_r/page_size) pages in row table_idx[r]) and
 * E_r = extend_lens[r] new tokens:
 *   - request r receives ceil((P_r+E_r)/page_size) - ceil(P_r/page_size)
 *     pages, written to the next entries of its row;
 *   - pages are taken from the tail of the free list, requests in order:
 *     the k-th page taken is free_pages[*num_free - 1 - k];
 *   - out_loc (sum E_r entries, requests in order) receives the slot of
 *     every new token, position P_r + i of request r through its row;
 *   - *num_free drops by the number of pages taken.
 * All arrays and *num_free are on the device; nothing is read back to the
 * host, so a step can be enqueued (or captured) with no synchronisation.
 * *status (device) is set to 0 when the step is done; otherwise nothing is
 * written and it says why: 1 not enough free pages, 2 a row would exceed
 * page_table_stride entries, 3 a negative length or a table_idx outside
 * [0, page_table_rows), 4 out_loc_capacity below sum E_r.  The pages each
 * request already holds must be valid ids, rows must be distinct, and the
 * free list must hold *num_free valid, unused page ids (caller's contract).
 */
msgl_status msgl_alloc_pages(const int32_t* free_pages, int32_t* num_free, int32_t* page_table,
                             int32_t page_table_stride, int32_t page_table_rows,
                             const int32_t* table_idx, const int32_t* prefix_lens,
                             const int32_t* extend_lens, int32_t batch, int32_t page_size,
                             int32_t* out_loc, int64_t out_loc_capacity, int32_t* status,
                             void* stream);

/*
 * Decode graphs: store_kv of one new row per request followed by
 * paged_decode, captured once into a HIP graph for a fixed (padded) batch
 * size and replayed with one launch ("Code Notes: mini-sglang", Engine
 * Layer table, GraphRunner row -- decode batches are replayed from graphs
 * captured at fixed batch sizes to hide launch overhead).
 *
 * msgl_decode_graph_create captures, on a private stream of its own:
 *     msgl_store_kv(pool, layer, k, k_row_stride, v, v_row_stride, out_loc, batch)
 *     msgl_paged_decode(pool, layer, q, q_row_stride, out, page_table, ..., batch, ...)
 * with the arguments' meaning, layout and validation exactly as for those
 * two calls (every scalar and pointer is checked before capture begins).
 * The pointers are baked into the graph: the buffers they name are the
 * graph's static inputs and outputs, which the caller refills before each
 * launch and must keep allocated until the graph is destroyed.  Rows of a
 * smaller real batch are padded with out_loc = -1 and seq_lens = 0 (zeros
 * out, no KV read).  max_seq_len is the bound the grid is sized for; every
 * replayed seq_lens[r] must stay within it.
 *   graph_out : receives the new graph, a host object owning a HIP graph
 *               executable.  The library allocates no buffer for it; the
 *               HIP runtime keeps the executable's own resources until
 *               msgl_decode_graph_destroy.
 * Returns MSGL_ERR_UNSUPPORTED in checked mode (MSGL_CHECK=1), whose host
 * synchronisation cannot be captured, and MSGL_ERR_HIP when capture or
 * instantiation fails; *graph_out is then NULL.
 *
 * msgl_decode_graph_launch replays the graph on `stream` (asynchronous,
 * ordered like any other call on that stream).  Launches of one graph
 * share its workspace and static buffers: they must not overlap in time.
 * msgl_decode_graph_destroy releases it (NULL is a no-op); the caller
 * makes sure no launch of it is still pending.
 */
typedef struct msgl_decode_graph msgl_decode_graph;

msgl_status msgl_decode_graph_create(const msgl_kv_pool* pool, int32_t layer, const void* k,
                                     int64_t k_row_stride, const void* v, int64_t v_row_stride,
                                     const int32_t* out_loc, const void* q, int64_t q_row_stride,
                                     void* out, const int32_t* page_table,
                                     int32_t page_table_stride, const int32_t* table_idx,
                                     const int32_t* seq_lens, int32_t batch,
                                     int32_t num_qo_heads, int32_t max_seq_len, float sm_scale,
                                     void* workspace, size_t workspace_bytes,
                                     msgl_decode_graph** graph_out);
msgl_status msgl_decode_graph_launch(const msgl_decode_graph* graph, void* stream);
msgl_status msgl_decode_graph_destroy(msgl_decode_graph* graph);

/*
 * decode_graph_runner: decode graphs at several batch sizes over one set of
 * static buffers ("Code Notes: mini-sglang", Engine Layer table, GraphRunner
 * row: graphs for batch sizes 1, 2, 4, 8, ..., and at run time the nearest
 * captured size at or above the batch).
 *
 * create takes the arguments of msgl_decode_graph_create with max_batch
 * rows in every static buffer and captures one graph per size 1, 2, 4, ...
 * below max_batch and one at max_batch; each covers the first `size` rows
 * (the workspace must be sized for max_batch).  pick returns the size a
 * batch of `batch` rows runs at -- the smallest captured size >= batch --
 * or 0 when batch is outside 1 .. max_batch; launch replays that graph on
 * `stream` (MSGL_ERR_SHAPE for a batch outside 1 .. max_batch).  Rows
 * batch .. size-1 must hold padding (out_loc -1, seq_lens 0, table_idx 0):
 * the runner reads them as they stand.  Launches of one runner share its
 * buffers and must be stream-ordered.
 */
typedef struct msgl_decode_graph_runner msgl_decode_graph_runner;
msgl_status msgl_decode_graph_runner_create(
    const msgl_kv_pool* pool, int32_t layer, const void* k, int64_t k_row_stride, const void* v,
    int64_t v_row_stride, const int32_t* out_loc, const void* q, int64_t q_row_stride, void* out,
    const int32_t* page_table, int32_t page_table_stride, const int32_t* table_idx,
    const int32_t* seq_lens, int32_t max_batch, int32_t num_qo_heads, int32_t max_seq_len,
    float sm_scale, void* workspace, size_t workspace_bytes, msgl_decode_graph_runner** runner_out);
int32_t msgl_decode_graph_runner_pick(const msgl_decode_graph_runner* runner, int32_t batch);
msgl_status msgl_decode_graph_runner_launch(const msgl_decode_graph_runner* runner, int32_t batch,
                                            void* stream);
msgl_status msgl_decode_graph_runner_destroy(msgl_decode_graph_runner* runner);

/*
 * paged_mixed: one call for a batch that mixes decode rows and
 * prefill/extend rows, as a scheduler that runs chunked prefill beside
 * decoding builds it ("Code Notes: mini-sglang", Engine Layer table,
 * BaseAttnBackend row -- HybridBackend keeps a prefill and a decode
 * backend; Scheduler Layer table, PrefillManager row -- chunked prefill).
 * Arguments as for paged_extend, plus the decode workspace:
 * msgl_paged_decode_workspace_size(batch, num_qo_heads, head_dim,
 * max_seq_len, page_size) bytes.  Rows are dispatched on the device by
 * extend_lens, so the host never needs the lengths:
 *   - a row with extend_lens[r] == 1 is a decode row: decode and merge,
 *     with q / out row cu_extend_lens[r] and length prefix_lens[r] + 1;
 *   - every other row goes through the extend kernel (rows with
 *     extend_lens[r] == 0 produce nothing).
 * The result equals paged_extend on the same batch within the attention
 * tolerance; the decode rows equal paged_decode on those rows exactly, and
 * the extend rows equal paged_extend on the batch exactly.
 * Launches on `stream`: with batch <= 2048 and a power-of-two page_size,
 * one attention launch (extend tiles first, then the decode ranges, in
 * one grid) and the merge of split decode rows; otherwise decode, merge
 * and extend launches (also when MSGL_MIXED_SPLIT=1 is set);
 * max_extend_len <= 1 (decode rows only) runs decode and merge alone.
 * Calls sharing a workspace must not overlap.
 */
msgl_status msgl_paged_mixed(const msgl_kv_pool* pool, int32_t layer, const void* q,
                             int64_t q_row_stride, void* out, const int32_t* page_table,
                             int32_t page_table_stride, const int32_t* table_idx,
                             const int32_t* prefix_lens, const int32_t* extend_lens,
                             const int32_t* cu_extend_lens, int32_t batch,
                             int32_t total_extend_tokens, int32_t max_extend_len,
                             int32_t max_seq_len, int32_t num_qo_heads, float sm_scale,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * debug_gather_kv (for tests): copy tokens 0 .. len-1 of page_table row
 * `row` out of the pool in logical order -- the page-table address
 * translation the attention kernels use, exposed on its own.
 *   k_out, v_out : (len, num_kv_heads, head_dim) bf16, contiguous.
 */
msgl_status msgl_debug_gather_kv(const msgl_kv_pool* pool, int32_t layer,
                                 const int32_t* page_table, int32_t page_table_stride,
                                 int32_t row, int32_t len, void* k_out, void* v_out,
                                 void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MSGL_H */
