// store_kv: scatter of new K/V rows into the paged pool by out_loc, and the
// test-only gather through one page_table row.
//
// "Code Notes: mini-sglang", Engine Layer table, BaseKVCachePool row: the
// pool is (2, num_layers, num_pages, page_size, heads, head_dim) and
// store_kv writes rows by out_loc indices.  Both kernels are pure copies
// of bit patterns, so they are bit-exact by construction.
//
// Work item = one VEC-byte piece of one K or V row.  Consecutive lanes take
// consecutive pieces of the same row, so every wave reads and writes whole
// contiguous row segments (coalesced) even though the rows themselves are
// scattered across the pool.
#include "common.h"

namespace msgl {

template <int VEC>
struct VecType;
template <>
struct VecType<16> {
  using T = uint4;
};
template <>
struct VecType<8> {
  using T = uint2;
};
template <>
struct VecType<4> {
  using T = uint32_t;
};
template <>
struct VecType<2> {
  using T = uint16_t;
};

// Grid: x = groups of U tokens, y = blocks of blockDim.x pieces of a
// token's K row followed by its V row (blockDim.x: the two rows' pieces
// rounded up to whole waves, at most 256).  A thread owns one piece
// position and copies it for the U tokens of its group: the U loads are
// all issued before the first store, so each thread keeps U independent
// reads in flight.  The row loads do not wait for the slots (block-uniform
// scalar loads): every token below num_tokens has a source row, and only
// the stores depend on the slot.
template <int VEC, int U>
__global__ __launch_bounds__(256) void store_kv_kernel(StoreParams p) {
  using V = typename VecType<VEC>::T;
  const int ppr = p.pieces_per_row;
  const int j = static_cast<int>(blockIdx.y * blockDim.x + threadIdx.x);
  if (j >= 2 * ppr) return;
  const int half = j >= ppr;  // 0 = K, 1 = V
  const int64_t piece_off = static_cast<int64_t>(j - half * ppr) * VEC;
  const uint8_t* src = (half ? p.v : p.k) + piece_off;
  const int64_t src_stride = half ? p.v_stride_bytes : p.k_stride_bytes;
  uint8_t* dst = (half ? p.v_cache : p.k_cache) + piece_off;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * U;
  int32_t slot[U];
  V val[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t t = t0 + u;
    slot[u] = t < p.num_tokens ? p.out_loc[t] : -1;
    if (t < p.num_tokens) {
      if constexpr (VEC == 16) {
        typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
        val[u] = __builtin_bit_cast(V, __builtin_nontemporal_load(
                                           reinterpret_cast<const u32x4v*>(src + t * src_stride)));
      } else {
        val[u] = *reinterpret_cast<const V*>(src + t * src_stride);
      }
    }
  }
  // padding rows (out_loc < 0) and slots outside the pool are skipped
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (slot[u] >= 0 && slot[u] < p.num_slots) {
      uint8_t* d = dst + static_cast<int64_t>(slot[u]) * p.row_bytes;
      if constexpr (VEC == 16) {
        // nontemporal on both sides: the new rows are read once here, and
        // written through rather than left as dirty lines that a later,
        // bandwidth-bound kernel would have to write back
        typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4v, val[u]), reinterpret_cast<u32x4v*>(d));
      } else {
        *reinterpret_cast<V*>(d) = val[u];
      }
    }
  }
}

__global__ __launch_bounds__(256) void gather_kernel(GatherParams p) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int ppr = p.pieces_per_row;
  for (int64_t it = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; it < p.num_items;
       it += stride) {
    const int64_t t = it / (2 * ppr);
    const int rem = static_cast<int>(it - t * 2 * ppr);
    const int half = rem >= ppr;
    const int piece = rem - half * ppr;
    const int64_t slot = token_slot_safe(p.page_row, static_cast<int>(t), p.page_size, p.num_slots);
    const uint8_t* src = (half ? p.v_cache : p.k_cache) + slot * p.row_bytes + piece * 16;
    uint8_t* dst = (half ? p.v_out : p.k_out) + t * p.row_bytes + piece * 16;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  }
}

static int grid_for(int64_t items) {
  const int64_t blocks = (items + 255) / 256;
  return static_cast<int>(blocks < 65536 ? (blocks > 0 ? blocks : 1) : 65536);
}

// Tokens per thread: 4 once there are enough tokens to fill the chip with
// such groups, else 1 (small steps are latency-bound: more, smaller
// workgroups finish sooner).
constexpr int kStoreGroupMin = 2048;

template <int VEC>
static void launch_store_t(const StoreParams& p, hipStream_t stream) {
  const int pieces = 2 * p.pieces_per_row;
  const int tb = pieces >= 256 ? 256 : (pieces + 63) / 64 * 64;
  const int yb = (pieces + tb - 1) / tb;
  if (p.num_tokens >= kStoreGroupMin) {
    const dim3 grid((p.num_tokens + 3) / 4, yb);
    hipLaunchKernelGGL((store_kv_kernel<VEC, 4>), grid, dim3(tb), 0, stream, p);
  } else {
    const dim3 grid(p.num_tokens > 0 ? p.num_tokens : 1, yb);
    hipLaunchKernelGGL((store_kv_kernel<VEC, 1>), grid, dim3(tb), 0, stream, p);
  }
}

hipError_t launch_store_kv(const StoreParams& p, int vec_bytes, hipStream_t stream) {
  switch (vec_bytes) {
    case 16:
      launch_store_t<16>(p, stream);
      break;
    case 8:
      launch_store_t<8>(p, stream);
      break;
    case 4:
      launch_store_t<4>(p, stream);
      break;
    default:
      launch_store_t<2>(p, stream);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_gather(const GatherParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(gather_kernel, dim3(grid_for(p.num_items)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace msgl
