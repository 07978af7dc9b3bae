// Device helpers and kernel parameter blocks shared by the HIP sources of
// libmsgl.so.  gfx950 (CDNA4) only: wave64, bf16 dot2 and MFMA builtins.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msgl {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- bf16 bits
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// a.lo*b.lo + a.hi*b.hi + c, bf16 pairs in 32-bit words, fp32 accumulate.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// (a.lo16, b.lo16) and (a.hi16, b.hi16) as new bf16 pairs.
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------ wave64 reductions
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
// DPP controls: quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

// Maximum over the 16 lanes of each DPP row, left in every lane of the row.
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_mov<kDppXor1>(x));
  x = fmaxf(x, dpp_mov<kDppXor2>(x));
  x = fmaxf(x, dpp_mov<kDppHalfMirror>(x));
  x = fmaxf(x, dpp_mov<kDppMirror>(x));
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<kDppXor1>(x);
  x += dpp_mov<kDppXor2>(x);
  x += dpp_mov<kDppHalfMirror>(x);
  x += dpp_mov<kDppMirror>(x);
  return x;
}
__device__ __forceinline__ float lane_value(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}
// Wave-wide maximum / sum, returned uniformly.
__device__ __forceinline__ float wave_max(float x) {
  x = row16_max(x);
  return fmaxf(fmaxf(lane_value(x, 0), lane_value(x, 16)),
               fmaxf(lane_value(x, 32), lane_value(x, 48)));
}
__device__ __forceinline__ float wave_sum(float x) {
  x = row16_sum(x);
  return (lane_value(x, 0) + lane_value(x, 16)) + (lane_value(x, 32) + lane_value(x, 48));
}

__device__ __forceinline__ float shfl_xor_f(float x, int mask) {
  return __shfl_xor(x, mask, 64);
}

// max / sum of x over lanes l and l^32 (one v_permlane32_swap: lanes 0-31
// receive the upper half's values and vice versa).
__device__ __forceinline__ float xor32_max(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// --------------------------------------------------- page-table translation
// Slot of logical token `tok` of the request whose page_table row is `row`:
// page_table[row][tok / page_size] * page_size + tok % page_size.
__device__ __forceinline__ int64_t token_slot(const int32_t* __restrict__ row, int tok,
                                              int page_size) {
  const int pg = tok / page_size;
  return static_cast<int64_t>(row[pg]) * page_size + (tok - pg * page_size);
}
// The same, kept inside [0, num_slots): a page id outside the pool breaks
// the caller's contract, and clamping turns it into wrong values instead of
// an out-of-bounds access.
__device__ __forceinline__ int token_slot_safe(const int32_t* __restrict__ row, int tok,
                                               int page_size, int num_slots) {
  const int pg = tok / page_size;
  const int s = row[pg] * page_size + (tok - pg * page_size);
  return min(max(s, 0), num_slots - 1);
}

// ------------------------------------------------------- parameter blocks
struct StoreParams {
  const uint8_t* k;
  const uint8_t* v;
  int64_t k_stride_bytes;
  int64_t v_stride_bytes;
  const int32_t* out_loc;
  uint8_t* k_cache;  // K half of the layer, (slots, Hkv, d)
  uint8_t* v_cache;
  int64_t num_items;  // tokens * 2 * pieces_per_row
  int32_t pieces_per_row;
  int32_t row_bytes;
  int32_t num_tokens;
  int32_t num_slots;
};

struct GatherParams {
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* page_row;
  uint8_t* k_out;
  uint8_t* v_out;
  int64_t num_items;
  int32_t pieces_per_row;
  int32_t row_bytes;
  int32_t page_size;
  int32_t num_slots;
};

// Decode works on whole token rows and balanced token ranges: the batch's
// tokens, requests laid end to end, are split evenly over kDecodeGrid
// workgroups per group of `head_group` kv heads; a workgroup streams the
// group's part of every K and V row of its range, request by request.
constexpr int kDecodeGrid = 512;       // workgroups per head group and launch (two per CU)
constexpr int kDecodeBatch = 2048;     // requests per launch (prefix sums in LDS)
constexpr int kDecodeWindow = 1024;    // tokens whose slots are staged at once
constexpr int kDecodeMinTokens = 16;   // tokens per workgroup at least
constexpr int kDecodeMaxTile = 64;     // tokens per tile at most (lengths are padded to tiles)

struct DecodeParams {
  const uint16_t* k_cache;  // K half of the layer, (slots, Hkv, d)
  const uint16_t* v_cache;
  const uint16_t* q;
  int64_t q_stride;  // elements between consecutive requests' q rows
  uint16_t* out;
  const int32_t* page_table;
  int64_t pt_stride;
  const int32_t* table_idx;
  const int32_t* seq_lens;
  // workspace: per request, (first piece, pieces) of this call; the
  // unnormalised partial outputs of the (workgroup i, request r) pieces, at
  // piece i + r: (pieces, Hq, D); their (running maximum in log2 units, sum)
  // pairs (pieces, Hq, 2)
  int2* ws_map;
  float* ws_o;
  float* ws_ml;
  int32_t batch;       // requests of this launch, <= kDecodeBatch
  int32_t num_kv_heads;
  int32_t group;       // q heads per kv head
  int32_t head_group;  // kv heads per workgroup: a power of two <= 8 dividing num_kv_heads
  int32_t page_size;
  int32_t max_seq_len;
  int32_t num_slots;
  uint32_t half_bytes;  // bytes of one (K or V, layer) sub-tensor, < 2^32
  float scale_log2;     // sm_scale * log2(e)
  // mixed batches (all three set, seq_lens unused): request r is a decode
  // row only when mixed_extend[r] == 1 -- the others belong to the extend
  // kernel and are skipped; its length is mixed_prefix[r] + 1 and its q /
  // out row is mixed_cu[r]
  const int32_t* mixed_prefix;
  const int32_t* mixed_extend;
  const int32_t* mixed_cu;
};

struct ExtendParams {
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const uint16_t* q;
  int64_t q_stride;
  uint16_t* out;
  const int32_t* page_table;
  int64_t pt_stride;
  const int32_t* table_idx;
  const int32_t* prefix_lens;
  const int32_t* extend_lens;
  const int32_t* cu_extend;
  int32_t num_kv_heads;
  int32_t group;
  int32_t page_size;
  int32_t num_mtiles;
  int32_t page_shift;  // log2(page_size) when it is a power of two, else -1
  int32_t max_extend_len;
  int32_t max_seq_len;
  int32_t num_slots;
  uint32_t half_bytes;  // bytes of one (K or V, layer) sub-tensor, < 2^32
  float scale_log2;
  int32_t skip_single;  // mixed batches: rows with one new token are left to decode
  // key splits: with num_splits > 1 each (request, kv head, row tile) runs
  // as num_splits workgroups over shares of its key tiles, each writing
  // fp32 o / l and (m, l) per (token, q head, share) -- at
  // (token * Hq + head) * num_splits + share of ws_o (x D) and ws_ml (x 2) --
  // and the merge kernel combines them into out
  int32_t num_splits;
  float* ws_o;
  float* ws_ml;
};

struct RopeParams {
  uint16_t* q;          // rotated in place
  int64_t q_stride;     // elements between rows
  const uint16_t* k;
  int64_t k_stride;
  const uint16_t* v;
  int64_t v_stride;
  const int32_t* out_loc;
  const int32_t* positions;
  const float* table;   // (max_position, head_dim): cos then sin
  uint16_t* k_cache;    // K half of the layer, (slots, Hkv, d)
  uint16_t* v_cache;
  int64_t num_items;
  int32_t num_qo_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t max_position;
  int32_t num_slots;
};

struct AllocParams {
  const int32_t* free_pages;
  int32_t* num_free;       // device count of free pages, updated in place
  int32_t* page_table;
  int64_t pt_stride;
  int32_t pt_rows;
  const int32_t* table_idx;
  const int32_t* prefix_lens;
  const int32_t* extend_lens;
  int32_t batch;
  int32_t page_size;
  int32_t* out_loc;
  int64_t out_loc_capacity;
  int32_t* status;         // device: 0 done, else why nothing was done
};

// Launchers (defined next to their kernels); return the HIP status.
hipError_t launch_store_kv(const StoreParams& p, int vec_bytes, hipStream_t stream);
hipError_t launch_gather(const GatherParams& p, hipStream_t stream);
// one launch of at most kDecodeBatch requests (decode, then merge)
hipError_t launch_decode(const DecodeParams& p, int head_dim, hipStream_t stream);
// the merge of the requests that the decode kernel split
hipError_t launch_decode_merge(const DecodeParams& p, int head_dim, hipStream_t stream);
// A mixed batch of at most kDecodeBatch requests in one attention launch
// (8-wave extend workgroups, page_size a power of two), then the merge;
// ext_tiles_bound bounds the extend row tiles (256 packed rows) of the batch
hipError_t launch_mixed(const DecodeParams& pd, const ExtendParams& pe, int head_dim,
                        int64_t ext_tiles_bound, hipStream_t stream);
// `waves` (4 or 8) sets the query rows per workgroup (32 per wave); the
// caller sizes p.num_mtiles for it.
hipError_t launch_extend(const ExtendParams& p, int head_dim, int batch, int waves,
                         hipStream_t stream);
// the combine of the key shares of p.num_splits > 1 into out, for `tokens`
// token rows
hipError_t launch_extend_merge(const ExtendParams& p, int head_dim, int64_t tokens,
                               hipStream_t stream);
hipError_t launch_rope_store_kv(const RopeParams& p, hipStream_t stream);
hipError_t launch_alloc_pages(const AllocParams& p, hipStream_t stream);
hipError_t launch_rope_table(float* table, int32_t max_position, int32_t head_dim, double base,
                             hipStream_t stream);

}  // namespace msgl
