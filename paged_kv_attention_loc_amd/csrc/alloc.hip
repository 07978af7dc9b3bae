// Device-side page allocation for one scheduling step: new pages for the
// step's new tokens taken from a free list, written into the requests'
// page_table rows, and the out_loc slots of the new tokens -- the metadata
// store_kv and the attention calls read ("Code Notes: mini-sglang",
// Scheduler Layer table: CacheManager row -- free_slots, the free
// positions it hands out; TableManager row -- one page_table row per
// request).  Done on the device so that a step needs no host round trip.
//
// Rule (the pages describe the allocator in outline only):
//   * the first num_free entries of free_pages are free; the k-th page
//     taken in the step (k = 0, 1, ...) is free_pages[num_free - 1 - k],
//     requests in order;
//   * request r holds ceil(P_r / ps) pages and receives
//     ceil((P_r + E_r) / ps) - ceil(P_r / ps) more, written to the next
//     entries of its row;
//   * out_loc[t] for new token i of request r (t counted over requests in
//     order) is the slot of position P_r + i through the updated row;
//   * num_free drops by the pages taken.  A step that cannot be done (not
//     enough free pages, a row too short, an argument out of range, an
//     out_loc buffer too small) changes nothing and reports why in *status.
//
// One workgroup of 1024 threads: a first pass checks every request and
// sums the demand; a second walks the requests in chunks of 1024, where
// block-wide exclusive scans (wave shuffles, then the wave totals) give
// each request its first page and first token, the request's thread writes
// its pages, and all threads then fill the chunk's out_loc entries (a
// binary search over the token offsets finds each token's request).  A
// request's thread reads up to kAllocUnroll free-list entries before it
// writes them into its row, so that a prefill request's pages cost a few
// memory round trips rather than one each.
#include "common.h"

namespace msgl {

namespace {

constexpr int kAllocThreads = 1024;
constexpr int kAllocUnroll = 8;  // free-list reads a thread issues before their stores

// exclusive prefix sum of v over the block; returns this thread's
// exclusive sum and leaves the block total in *total.  Each wave scans its
// 64 values with shuffles, wave 0 scans the 16 wave totals, and every
// thread adds the totals of the waves before its own: three barriers.
// `wave_tot` holds 32 values (the totals, then their inclusive sums).
__device__ __forceinline__ int64_t block_exclusive_scan(int64_t v, int64_t* wave_tot, int64_t* total) {
  constexpr int kWaves = kAllocThreads / 64;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  int64_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) wave_tot[w] = x;
  __syncthreads();
  if (w == 0) {
    int64_t tw = lane < kWaves ? wave_tot[lane] : 0;
#pragma unroll
    for (int off = 1; off < kWaves; off <<= 1) {
      const int64_t y = __shfl_up(tw, off, 64);
      if (lane >= off) tw += y;
    }
    if (lane < kWaves) wave_tot[kWaves + lane] = tw;
  }
  __syncthreads();
  const int64_t before = w > 0 ? wave_tot[kWaves + w - 1] : 0;
  *total = wave_tot[2 * kWaves - 1];
  __syncthreads();  // wave_tot is reused by the next scan
  return before + x - v;
}

}  // namespace

__global__ __launch_bounds__(kAllocThreads) void alloc_pages_kernel(AllocParams p) {
  __shared__ int64_t scan_buf[2 * (kAllocThreads / 64)];
  __shared__ int64_t tok_first[kAllocThreads];  // exclusive token offsets of the chunk
  __shared__ int32_t req_row[kAllocThreads];
  __shared__ int32_t req_pos0[kAllocThreads];
  __shared__ int32_t s_bad;
  __shared__ int32_t s_num_free;
  const int t = threadIdx.x;
  const int ps = p.page_size;

  // ---- pass 1: checks and totals
  if (t == 0) {
    s_bad = 0;
    s_num_free = *p.num_free;
  }
  __syncthreads();
  int64_t need_sum = 0, tok_sum = 0;
  int bad = 0;
  for (int r = t; r < p.batch; r += kAllocThreads) {
    const int64_t P = p.prefix_lens[r], E = p.extend_lens[r];
    const int32_t row = p.table_idx[r];
    if (P < 0 || E < 0 || row < 0 || row >= p.pt_rows) {
      bad |= 1;
      continue;
    }
    const int64_t n = (P + E + ps - 1) / ps;
    if (n > p.pt_stride) bad |= 2;
    need_sum += n - (P + ps - 1) / ps;
    tok_sum += E;
  }
  if (bad) atomicOr(&s_bad, bad);  // LDS atomic
  int64_t need_total, tok_total;
  block_exclusive_scan(need_sum, scan_buf, &need_total);
  block_exclusive_scan(tok_sum, scan_buf, &tok_total);
  const int num_free = s_num_free;
  int32_t code = 0;
  if (s_bad & 1)
    code = 3;
  else if (s_bad & 2)
    code = 2;
  else if (need_total > num_free)
    code = 1;
  else if (tok_total > p.out_loc_capacity)
    code = 4;
  if (code != 0) {
    if (t == 0) *p.status = code;
    return;
  }

  // ---- pass 2: chunks of requests
  int64_t page_run = 0, tok_run = 0;
  for (int c = 0; c < p.batch; c += kAllocThreads) {
    const int r = c + t;
    const bool valid = r < p.batch;
    const int32_t P = valid ? p.prefix_lens[r] : 0;
    const int32_t E = valid ? p.extend_lens[r] : 0;
    const int32_t row = valid ? p.table_idx[r] : 0;
    const int64_t have = (static_cast<int64_t>(P) + ps - 1) / ps;
    const int64_t need = valid ? (static_cast<int64_t>(P) + E + ps - 1) / ps - have : 0;
    int64_t chunk_pages, chunk_toks;
    const int64_t page_first = block_exclusive_scan(need, scan_buf, &chunk_pages);
    const int64_t tok0 = block_exclusive_scan(E, scan_buf, &chunk_toks);
    // this request's new pages
    int32_t* prow = p.page_table + static_cast<int64_t>(row) * p.pt_stride;
    if (need == 1) {
      prow[have] = p.free_pages[num_free - 1 - (page_run + page_first)];
    } else {
      for (int64_t j0 = 0; j0 < need; j0 += kAllocUnroll) {
        int32_t pg[kAllocUnroll];
#pragma unroll
        for (int u = 0; u < kAllocUnroll; ++u)
          pg[u] = j0 + u < need ? p.free_pages[num_free - 1 - (page_run + page_first + j0 + u)] : 0;
#pragma unroll
        for (int u = 0; u < kAllocUnroll; ++u)
          if (j0 + u < need) prow[have + j0 + u] = pg[u];
      }
    }
    tok_first[t] = tok0;
    req_row[t] = row;
    req_pos0[t] = P;
    __threadfence_block();
    __syncthreads();
    // the chunk's new tokens, spread over the block
    const int nreq = min(kAllocThreads, p.batch - c);
    for (int64_t k = t; k < chunk_toks; k += kAllocThreads) {
      int lo = 0, hi = nreq - 1;  // last request whose first token is <= k
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tok_first[mid] <= k)
          lo = mid;
        else
          hi = mid - 1;
      }
      const int64_t pos = req_pos0[lo] + (k - tok_first[lo]);
      const int32_t* qrow = p.page_table + static_cast<int64_t>(req_row[lo]) * p.pt_stride;
      p.out_loc[tok_run + k] = qrow[pos / ps] * ps + static_cast<int32_t>(pos % ps);
    }
    page_run += chunk_pages;
    tok_run += chunk_toks;
    __syncthreads();  // LDS arrays are rewritten by the next chunk
  }
  if (t == 0) {
    *p.num_free = num_free - static_cast<int32_t>(need_total);
    *p.status = 0;
  }
}

hipError_t launch_alloc_pages(const AllocParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(alloc_pages_kernel, dim3(1), dim3(kAllocThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace msgl
