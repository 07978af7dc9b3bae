// Rotary position embedding fused with store_kv, and the cos/sin table
// builder.
//
// The pages list rotary position embeddings among the model layers ("Code
// Structure", section Model Layers, get_rope / set_rope_device; section
// Model Definitions, RotaryConfig) without the formula.  The standard rotary
// embedding is used, with the half-split pairing of the Llama family: for
// i < d/2 the pair (x_i, x_{i+d/2}) at position p turns by the angle
// a = p * base^(-2i/d):
//     y_i       = x_i cos a - x_{i+d/2} sin a
//     y_{i+d/2} = x_{i+d/2} cos a + x_i sin a.
// cos a and sin a come from a caller-supplied fp32 table (row p: the d/2
// cosines, then the d/2 sines).
//
// The fused kernel rotates this step's q rows in place and stores the
// rotated k rows and the v rows into the pool at out_loc, so that k is read
// once and written once instead of being rotated in a separate pass.  It is
// a pure streaming kernel (no reuse), bound by HBM bytes.
//
// Arithmetic: both products are exact in fp64 (a bf16 times an fp32 value
// has at most 32 significant bits), the difference or sum is rounded once
// to fp64, and that value is rounded to bf16 correctly -- toward zero to
// binary32 with the last bit set when anything was dropped (round to odd),
// then to nearest even.  The result is the exact rotation of the stored
// inputs rounded once, up to the fp64 rounding of the sum.
#include <algorithm>

#include "common.h"

namespace msgl {

namespace {

// A binary64 value rounded to bf16, to nearest, ties to even, in effect in
// one step.  When the result is a normal bf16 (or rounds up to infinity),
// that is integer work on the binary64 fields: the top 7 of the 52
// fraction bits are kept, and the 45 below decide the rounding against
// half a unit (2^44).  Otherwise (zero, results below bf16's normal range,
// infinities, NaN) the value is rounded to binary32 toward zero with the
// last bit set when anything was dropped (round to odd), which keeps the
// information the second rounding, to nearest even, needs.  Both give the
// correctly rounded result.
__device__ __forceinline__ uint16_t f64_to_bf16(double y) {
  const uint64_t bits = __builtin_bit_cast(uint64_t, y);
  const uint32_t hi = static_cast<uint32_t>(bits >> 32);
  const uint32_t lo = static_cast<uint32_t>(bits);
  const uint32_t e = (hi >> 20) & 0x7FFu;  // biased binary64 exponent
  if (e - 897u <= 1150u - 897u) {          // unbiased -126 .. 127
    const uint32_t m7 = (hi >> 13) & 0x7Fu;
    const uint32_t rhi = hi & 0x1FFFu;      // top 13 of the 45 dropped bits
    const bool above = rhi > 0x1000u || (rhi == 0x1000u && lo != 0u);
    const bool tie = rhi == 0x1000u && lo == 0u;
    const uint32_t up = (above || (tie && (m7 & 1u))) ? 1u : 0u;
    return static_cast<uint16_t>(((hi >> 16) & 0x8000u) | ((((e - 896u) << 7) | m7) + up));
  }
  const float t = __double2float_rz(y);
  const uint32_t u = __float_as_uint(t) | (static_cast<double>(t) != y ? 1u : 0u);
  return f32_to_bf16(__uint_as_float(u));
}

// rotate the 8 channel pairs (x1[j], x2[j]) in place
__device__ __forceinline__ void rotate8(uint4& x1, uint4& x2, const float* cs, const float* sn) {
  uint32_t* a = reinterpret_cast<uint32_t*>(&x1);
  uint32_t* b = reinterpret_cast<uint32_t*>(&x2);
  const float4 c0 = reinterpret_cast<const float4*>(cs)[0];
  const float4 c1 = reinterpret_cast<const float4*>(cs)[1];
  const float4 s0 = reinterpret_cast<const float4*>(sn)[0];
  const float4 s1 = reinterpret_cast<const float4*>(sn)[1];
  const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint16_t ya[2], yb[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const double xa = bf16_to_f32(static_cast<uint16_t>(a[w] >> (16 * h)));
      const double xb = bf16_to_f32(static_cast<uint16_t>(b[w] >> (16 * h)));
      const double c = cv[2 * w + h], s = sv[2 * w + h];
      ya[h] = f64_to_bf16(fma(xa, c, -(xb * s)));
      yb[h] = f64_to_bf16(fma(xb, c, xa * s));
    }
    a[w] = static_cast<uint32_t>(ya[0]) | (static_cast<uint32_t>(ya[1]) << 16);
    b[w] = static_cast<uint32_t>(yb[0]) | (static_cast<uint32_t>(yb[1]) << 16);
  }
}

}  // namespace

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

// 16 bytes read or written once (q, k and v rows stream through)
__device__ __forceinline__ uint4 load_once(const uint16_t* a) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(a)));
}
__device__ __forceinline__ void store_once(uint16_t* a, uint4 x) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4v, x), reinterpret_cast<u32x4v*>(a));
}

// Work items per token: Hq*G8 q items and Hkv*G8 k items (G8 = d/16: eight
// channel pairs each, two 16-byte loads), then Hkv*d/8 v items (one 16-byte
// piece each).  One workgroup per token (blockIdx.x): its slot, position
// and cos/sin row are workgroup-uniform (scalar loads), and consecutive
// threads take consecutive items.  The row loads do not wait for the slot:
// every token has its rows, and only the pool stores depend on the slot.
__global__ __launch_bounds__(1024) void rope_store_kv_kernel(RopeParams p) {
  const int d = p.head_dim, half = d / 2, g8 = d / 16;
  const int nq = p.num_qo_heads * g8;
  const int nk = p.num_kv_heads * g8;
  const int per_tok = nq + nk + p.num_kv_heads * (d / 8);
  const int64_t t = blockIdx.x;
  const int32_t slot = p.out_loc[t];
  const bool store = slot >= 0 && slot < p.num_slots;  // padding rows store nothing
  const int pos = min(max(p.positions[t], 0), p.max_position - 1);
  const float* row_cs = p.table + static_cast<int64_t>(pos) * d;
  for (int r = threadIdx.x; r < per_tok; r += blockDim.x) {
    if (r < nq + nk) {
      const bool is_q = r < nq;
      const int rr = is_q ? r : r - nq;
      const int head = rr / g8, c = rr % g8;
      const uint16_t* src = is_q ? p.q + t * p.q_stride + head * d : p.k + t * p.k_stride + head * d;
      uint4 x1 = load_once(src + 8 * c);
      uint4 x2 = load_once(src + half + 8 * c);
      rotate8(x1, x2, row_cs + 8 * c, row_cs + half + 8 * c);
      if (!is_q && !store) continue;
      uint16_t* dst = is_q ? p.q + t * p.q_stride + head * d
                           : p.k_cache + (static_cast<int64_t>(slot) * p.num_kv_heads + head) * d;
      store_once(dst + 8 * c, x1);
      store_once(dst + half + 8 * c, x2);
    } else {
      const int piece = r - nq - nk;  // 16-byte piece of the v row
      const uint4 x = load_once(p.v + t * p.v_stride + 8 * piece);
      if (!store) continue;
      store_once(p.v_cache + static_cast<int64_t>(slot) * p.num_kv_heads * d + 8 * piece, x);
    }
  }
}

// table[pos][i] = cos(pos * base^(-2i/d)), table[pos][d/2 + i] = sin(...):
// the angle, cosine and sine in fp64 (device library functions), rounded
// once to fp32.
__global__ __launch_bounds__(256) void rope_table_kernel(float* table, int32_t max_position,
                                                         int32_t head_dim, double base) {
  const int half = head_dim / 2;
  const int64_t n = static_cast<int64_t>(max_position) * half;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t it = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; it < n; it += stride) {
    const int64_t pos = it / half;
    const int i = static_cast<int>(it - pos * half);
    const double inv_freq = pow(base, -2.0 * i / head_dim);
    const double a = static_cast<double>(pos) * inv_freq;
    table[pos * head_dim + i] = static_cast<float>(cos(a));
    table[pos * head_dim + half + i] = static_cast<float>(sin(a));
  }
}

static int rope_grid(int64_t items) {
  const int64_t blocks = (items + 255) / 256;
  return static_cast<int>(blocks < 65536 ? (blocks > 0 ? blocks : 1) : 65536);
}

hipError_t launch_rope_store_kv(const RopeParams& p, hipStream_t stream) {
  // one workgroup per token, its items rounded up to whole waves (at most 1024)
  const int d = p.head_dim;
  const int per_tok = (p.num_qo_heads + p.num_kv_heads) * (d / 16) + p.num_kv_heads * (d / 8);
  const int threads = std::min(1024, (per_tok + 63) / 64 * 64);
  const int64_t tokens = p.num_items / per_tok;
  hipLaunchKernelGGL(rope_store_kv_kernel, dim3(static_cast<uint32_t>(tokens)), dim3(threads), 0,
                     stream, p);
  return hipGetLastError();
}

hipError_t launch_rope_table(float* table, int32_t max_position, int32_t head_dim, double base,
                             hipStream_t stream) {
  const int64_t n = static_cast<int64_t>(max_position) * (head_dim / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3(rope_grid(n)), dim3(256), 0, stream, table,
                     max_position, head_dim, base);
  return hipGetLastError();
}

}  // namespace msgl
