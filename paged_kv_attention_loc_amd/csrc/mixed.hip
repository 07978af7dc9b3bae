// A mixed batch -- decode rows (one new token) and extend rows (several) of
// one forward pass ("Code Notes: mini-sglang", Engine Layer table row
// BaseAttnBackend: one backend call per batch, whatever its rows) -- in one
// launch of attention, followed by the small merge of split decode rows.
//
// The decode rows are memory-bound (every K/V byte read once) and the
// extend rows are bound by the matrix cores.  In one grid, the CUs that
// the extend tiles leave free stream decode K/V meanwhile, and there is no
// gap between the two kinds of work:
//   * every workgroup first counts the extend row tiles of the batch (rows
//     with more than one new token, 256 packed rows per tile) into LDS;
//   * the extend items come first in the grid, then the decode workgroups:
//     an extend tile is the longest job, and the dispatcher hands out
//     workgroups in id order, round-robin over the shader engines, so a
//     long job dispatched late either waits for a busy engine or ends the
//     launch alone (interleaving the two kinds measured 1.5x slower on an
//     all-extend batch, for that reason);
//   * extend item j serves kv head j % Hkv and a tile of the list, the
//     heaviest tile of each row first (with 8 kv heads each XCD -- ids are
//     dealt to the 8 XCDs round-robin -- keeps one head's K/V in its L2, as
//     in the extend kernel).  The grid is sized on the host from an upper
//     bound of the tile count; the workgroups past the real count exit;
//   * the decode workgroups run the decode body over the balanced token
//     ranges of the decode rows (kDecodeGrid ranges per kv head group).
//     The extend body needs ~230 registers a lane, so one 8-wave workgroup
//     fits a CU; with one decode workgroup per CU, the decode body keeps
//     three 32 KiB LDS stages (two tiles in flight) instead of two (head
//     groups of one or two kv heads: four 16 KiB stages, as in the decode
//     kernel);
//   * LDS is one buffer that either body uses as its own.
// When the extend tiles alone fill every CU, the two kinds run one after
// the other, and the decode part, at one workgroup per CU, takes ~7% longer
// than in its own kernel.
#include "decode_block.h"
#include "extend_block.h"

namespace msgl {

namespace {

constexpr int kMixedStages = 3;   // decode LDS stages inside the mixed kernel
constexpr int kMixedWaves = 8;    // extend waves per workgroup (256 packed rows)
constexpr int kMixedThreads = 64 * kMixedWaves;

constexpr int cmax(int a, int b) { return a > b ? a : b; }

}  // namespace

// Extend row tiles of request r in a mixed batch: rows with one new token
// are decode rows and have none.  Lengths are clamped as the extend body
// clamps them.
__device__ __forceinline__ int mixed_row_tiles(const ExtendParams& p, int r) {
  constexpr int BM = 32 * kMixedWaves;
  const int E = min(p.extend_lens[r], p.max_extend_len);
  if (E <= 1) return 0;
  return (E * p.group + BM - 1) / BM;
}

template <int D, int RB>
__global__ __launch_bounds__(kMixedThreads, 2) void mixed_kernel(DecodeParams pd, ExtendParams pe,
                                                                  const int32_t* __restrict__ page_table) {
  // the decode body cuts tokens into the decode kernel's tiles: 32 KiB
  // stages, kMixedStages of them, or four of 16 KiB for small head groups
  constexpr int DSTB = decode_impl::decode_stage_bytes<D, RB>();
  constexpr int DS = DSTB == decode_impl::kStageBytes ? kMixedStages : 4;
  constexpr int SMEM = cmax(decode_impl::lds_bytes<DS, DSTB>(), extend_impl::lds_bytes<D, kMixedWaves>());
  static_assert(SMEM >= (kDecodeBatch + 1 + kMixedWaves) * 4, "tile list must fit");
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  int32_t* const tiles_pre = reinterpret_cast<int32_t*>(smem);  // (B + 1) prefix sums
  int32_t* const wave_tot = tiles_pre + kDecodeBatch + 1;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int B = pd.batch;

  // ---- extend row tiles of the batch and their exclusive prefix sums
  {
    constexpr int RPT = kDecodeBatch / kMixedThreads;  // requests per thread
    int cnt[RPT];
    int run = 0;
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int r = tid * RPT + j;
      cnt[j] = r < B ? mixed_row_tiles(pe, r) : 0;
      run += cnt[j];
    }
    int incl = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    if (lane == 63) wave_tot[w] = incl;
    __syncthreads();
    int excl = incl - run;
    int total = 0;
#pragma unroll
    for (int x = 0; x < kMixedWaves; ++x) {
      if (x < w) excl += wave_tot[x];
      total += wave_tot[x];
    }
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      tiles_pre[tid * RPT + j] = excl;
      excl += cnt[j];
    }
    if (tid == 0) tiles_pre[kDecodeBatch] = total;
    __syncthreads();
  }

  // ---- this workgroup's item: extend items [0, n_ext), then decode
  // workgroups [n_ext, n_ext + n_dec)
  const int Hkv = pe.num_kv_heads;
  const int64_t n_ext = static_cast<int64_t>(tiles_pre[kDecodeBatch]) * Hkv;
  const int64_t n_dec = static_cast<int64_t>(kDecodeGrid) * (pd.num_kv_heads / pd.head_group);
  const int64_t j = blockIdx.x;
  if (j >= n_ext + n_dec) return;  // past the real tile count: nothing to do
  if (j < n_ext) {
    const int g = static_cast<int>(j % Hkv);
    const int pair = static_cast<int>(j / Hkv);
    // the request holding tile `pair`: the last r with tiles_pre[r] <= pair
    int lo = 0, hi = B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tiles_pre[mid] <= pair) lo = mid; else hi = mid;
    }
    const int k = pair - tiles_pre[lo];
    const int mt = tiles_pre[lo + 1] - tiles_pre[lo] - 1 - k;  // heaviest tile first
    __syncthreads();  // every wave has read the list before LDS is reused
    extend_impl::extend_block<D, true, kMixedWaves>(pe, page_table, g, lo, mt, smem);
  } else {
    const int64_t db = j - n_ext;
    __syncthreads();
    decode_impl::decode_block<D, RB, DS, DSTB>(pd, static_cast<int>(db % kDecodeGrid), kDecodeGrid,
                                               static_cast<int>(db / kDecodeGrid), smem);
  }
}

namespace {

template <int D>
void launch_mixed_d(const DecodeParams& pd, const ExtendParams& pe, int64_t blocks,
                    hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>(blocks));
  switch (pd.head_group) {
    case 8:
      hipLaunchKernelGGL((mixed_kernel<D, 8 * D * 2>), grid, dim3(kMixedThreads), 0, stream, pd, pe,
                         pe.page_table);
      break;
    case 4:
      hipLaunchKernelGGL((mixed_kernel<D, 4 * D * 2>), grid, dim3(kMixedThreads), 0, stream, pd, pe,
                         pe.page_table);
      break;
    case 2:
      hipLaunchKernelGGL((mixed_kernel<D, 2 * D * 2>), grid, dim3(kMixedThreads), 0, stream, pd, pe,
                         pe.page_table);
      break;
    default:
      hipLaunchKernelGGL((mixed_kernel<D, D * 2>), grid, dim3(kMixedThreads), 0, stream, pd, pe,
                         pe.page_table);
      break;
  }
}

}  // namespace

hipError_t launch_mixed(const DecodeParams& pd, const ExtendParams& pe, int head_dim,
                        int64_t ext_tiles_bound, hipStream_t stream) {
  const int64_t blocks = static_cast<int64_t>(kDecodeGrid) * (pd.num_kv_heads / pd.head_group) +
                         ext_tiles_bound * pd.num_kv_heads;
  if (head_dim == 128)
    launch_mixed_d<128>(pd, pe, blocks, stream);
  else
    launch_mixed_d<64>(pd, pe, blocks, stream);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode_merge(pd, head_dim, stream);
}

}  // namespace msgl
