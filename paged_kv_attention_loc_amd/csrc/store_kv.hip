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

template <int VEC>
__global__ __launch_bounds__(256) void store_kv_kernel(StoreParams p) {
  using V = typename VecType<VEC>::T;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int ppr = p.pieces_per_row;
  for (int64_t it = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; it < p.num_items;
       it += stride) {
    const int64_t t = it / (2 * ppr);
    const int rem = static_cast<int>(it - t * 2 * ppr);
    const int half = rem >= ppr;  // 0 = K, 1 = V
    const int piece = rem - half * ppr;
    const int32_t slot = p.out_loc[t];
    if (slot < 0 || slot >= p.num_slots) continue;  // padding row (or outside the pool)
    const uint8_t* src = (half ? p.v + t * p.v_stride_bytes : p.k + t * p.k_stride_bytes) +
                         static_cast<int64_t>(piece) * VEC;
    uint8_t* dst = (half ? p.v_cache : p.k_cache) + static_cast<int64_t>(slot) * p.row_bytes +
                   static_cast<int64_t>(piece) * VEC;
    if constexpr (VEC == 16) {
      // nontemporal on both sides: the new rows are read once here, and
      // written through rather than left as dirty lines that a later,
      // bandwidth-bound kernel would have to write back
      typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
      __builtin_nontemporal_store(__builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(src)),
                                  reinterpret_cast<u32x4v*>(dst));
    } else {
      *reinterpret_cast<V*>(dst) = *reinterpret_cast<const V*>(src);
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

hipError_t launch_store_kv(const StoreParams& p, int vec_bytes, hipStream_t stream) {
  const dim3 grid(grid_for(p.num_items)), block(256);
  switch (vec_bytes) {
    case 16:
      hipLaunchKernelGGL(store_kv_kernel<16>, grid, block, 0, stream, p);
      break;
    case 8:
      hipLaunchKernelGGL(store_kv_kernel<8>, grid, block, 0, stream, p);
      break;
    case 4:
      hipLaunchKernelGGL(store_kv_kernel<4>, grid, block, 0, stream, p);
      break;
    default:
      hipLaunchKernelGGL(store_kv_kernel<2>, grid, block, 0, stream, p);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_gather(const GatherParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(gather_kernel, dim3(grid_for(p.num_items)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace msgl
