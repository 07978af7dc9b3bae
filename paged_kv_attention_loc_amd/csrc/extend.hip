// Causal paged prefill/extend attention on bf16 MFMA.
//
// Request r has P = prefix_lens[r] tokens in the pool (radix-shared prefix
// pages or earlier prefill chunks) and E = extend_lens[r] new tokens; new
// token i sits at position P + i and sees keys 0 .. P + i ("Code Notes:
// mini-sglang", Scheduler Layer table, PrefillManager row -- chunked
// prefill; "Introduction", Key Features -- Radix Cache, Chunked Prefill).
// This is a dense contraction (Q.K^T and P.V), so it runs on the matrix
// cores with v_mfma_f32_32x32x16_bf16.
//
// Tiling:
//   * the G query heads sharing a kv head are packed into the M dimension,
//     token-major (packed row m = i*G + head-in-group), so each row's causal
//     limit P + m/G is monotone in m;
//   * a workgroup of 4 waves owns 128 packed rows (32 per wave) of one
//     (request, kv head) and walks the keys in tiles of 64 up to the last
//     row's limit; the heaviest row tiles are launched first;
//   * K/V tiles are double-buffered in LDS.  While tile t is computed, tile
//     t+1 is already in registers on its way to the other buffer, and the
//     page-table entries of tile t+2 are in flight -- one barrier per tile;
//   * every loading thread owns 4 consecutive keys and one 16-byte column,
//     for K and for V, so one page-table lookup serves both; rows are read
//     with buffer loads at 32-bit offsets inside the (K or V, layer)
//     sub-tensor;
//   * each wave computes S^T = K Q^T, so a lane holds one query column and
//     16 keys per 32-key block: the row maximum and sum need only one
//     exchange with the lane 32 apart;
//   * K is staged row-major with a 16-byte XOR swizzle; V is staged
//     transposed (channel-major) so the A operand of O^T = V^T P^T is one
//     16-byte LDS read, with the keys of every 16-key group stored in the
//     order in which the S^T accumulator registers hold them -- P^T then
//     feeds the second MFMA straight from registers.  The V^T swizzle mixes
//     channel bits 1-3 and 4-6 so that both the row-parallel reads and the
//     column-parallel transposing writes spread over the banks;
//   * masking runs only on tiles that cross a row's causal limit, and the
//     O rescale is skipped when no row maximum moved.
#include "common.h"

namespace msgl {

namespace {

// Physical start position (within a 16-key group) of the 4-key group kq:
// S^T registers hold keys {0-3, 8-11} in lanes 0-31 and {4-7, 12-15} in
// lanes 32-63, so groups 0,1,2,3 go to positions 0,8,4,12.
__device__ __forceinline__ int vt_group_pos(int kq) {
  const int j = kq & 3;
  return 16 * (kq >> 2) + 4 * (((j & 1) << 1) | (j >> 1));
}

// 16-byte column swizzle of transposed V row `ch` (8 columns per row)
__device__ __forceinline__ int vt_swizzle(int ch) { return ((ch >> 1) ^ (ch >> 4)) & 7; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t extend_rsrc(const void* base, uint32_t bytes) {
  // dword 3 = 0x00020000: 32-bit data format, raw (unswizzled) addressing
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <int D>
struct ExtendShape {
  static constexpr int BM = 128;          // packed rows per workgroup
  static constexpr int BN = 64;           // keys per tile
  static constexpr int NCOL = D / 8;      // 16-byte columns per K row
  static constexpr int KS = D / 16;       // MFMA k-steps of Q.K^T
  static constexpr int CB = D / 32;       // 32-channel blocks of the output
  static constexpr int VT_ROW = BN * 2;   // bytes per transposed V row
  static constexpr int K_BYTES = BN * D * 2;
  static constexpr int V_BYTES = D * VT_ROW;
  static constexpr int LOADERS = (BN / 4) * NCOL;  // threads that load a tile
};

}  // namespace

template <int D, bool POW2>
__global__ __launch_bounds__(256, 2) void extend_kernel(ExtendParams p,
                                                        const int32_t* __restrict__ page_table) {
  using S = ExtendShape<D>;
  constexpr int BM = S::BM, BN = S::BN, NCOL = S::NCOL, KS = S::KS, CB = S::CB;
  constexpr int VT_ROW = S::VT_ROW, K_BYTES = S::K_BYTES, V_BYTES = S::V_BYTES;

  const int mt = p.num_mtiles - 1 - static_cast<int>(blockIdx.x);
  const int g = blockIdx.y;
  const int r = blockIdx.z;
  const int G = p.group;
  // lengths above the host-side bounds break the caller's contract; clamp
  // them so that no page_table entry past the row's bound is read
  const int E = min(p.extend_lens[r], p.max_extend_len);
  const int M = E * G;
  const int m0 = mt * BM;
  if (m0 >= M) return;
  const int P = max(0, min(p.prefix_lens[r], p.max_seq_len - E));
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int q32 = lane & 31;
  const int hi = lane >> 5;
  const int Hq = p.num_kv_heads * G;

  __shared__ __attribute__((aligned(16))) uint8_t k_lds[2][K_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t vt_lds[2][V_BYTES];

  // this lane's query row (rows past the end are clamped and not written)
  const int mrow = m0 + w * 32 + q32;
  const int mrow_c = min(mrow, M - 1);
  const int ti = mrow_c / G;
  const int hh = mrow_c - ti * G;
  const int lim = P + ti;

  const uint16_t* qp = p.q + static_cast<int64_t>(p.cu_extend[r] + ti) * p.q_stride +
                       static_cast<int64_t>(g * G + hh) * D + hi * 8;
  bf16x8_t qop[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qop[ks] = *reinterpret_cast<const bf16x8_t*>(qp + ks * 16);

  const int wrow0 = min(m0 + w * 32, M - 1);
  const int wrow1 = min(m0 + w * 32 + 31, M - 1);
  const int wlim_lo = P + wrow0 / G;
  const int wlim_hi = P + wrow1 / G;
  const int kv_end = P + min(m0 + BM - 1, M - 1) / G + 1;
  const int ntiles = (kv_end + BN - 1) / BN;

  const int32_t* pt = page_table + static_cast<int64_t>(p.table_idx[r]) * p.pt_stride;
  const int ps = p.page_size;
  const int sh = p.page_shift;
  const uint32_t row_bytes = static_cast<uint32_t>(p.num_kv_heads) * D * 2;
  const uint32_t head_off = static_cast<uint32_t>(g) * D * 2;
  const __amdgpu_buffer_rsrc_t krs =
      extend_rsrc(p.k_cache + static_cast<int64_t>(g) * D, p.half_bytes - head_off);
  const __amdgpu_buffer_rsrc_t vrs =
      extend_rsrc(p.v_cache + static_cast<int64_t>(g) * D, p.half_bytes - head_off);

  // loader role: keys 4kq .. 4kq+3 of a tile, 16-byte column cg
  const bool loader = tid < S::LOADERS;
  const int kq = tid / NCOL;
  const int cg = tid % NCOL;
  auto tile_key = [&](int t, int j) { return min(t * BN + 4 * kq + j, kv_end - 1); };
  auto page_entry = [&](int key) { return POW2 ? pt[key >> sh] : pt[key / ps]; };
  auto slot_of = [&](int key, int entry) {
    const int s = POW2 ? (entry << sh) + (key & (ps - 1)) : entry * ps + key % ps;
    return static_cast<uint32_t>(min(max(s, 0), p.num_slots - 1));
  };

  uint4 kr[4], vr[4];
  int ent[4];
  auto issue_loads = [&](int t) {  // tile t's rows, using the entries in ent
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t off = slot_of(tile_key(t, j), ent[j]) * row_bytes + cg * 16;
      const u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0);
      const u32x4_t b = __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0);
      kr[j] = make_uint4(a.x, a.y, a.z, a.w);
      vr[j] = make_uint4(b.x, b.y, b.z, b.w);
    }
  };
  auto fetch_entries = [&](int t) {
#pragma unroll
    for (int j = 0; j < 4; ++j) ent[j] = page_entry(tile_key(t, j));
  };
  // registers -> LDS buffer b: K row-major (swizzled), V transposed with 4
  // keys per 8-byte write
  auto store_tile = [&](int b) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = 4 * kq + j;
      *reinterpret_cast<uint4*>(k_lds[b] + (key * NCOL + (cg ^ (key & (NCOL - 1)))) * 16) = kr[j];
    }
    const int pos = vt_group_pos(kq);
    const int pcol = pos >> 3;       // 16-byte column of this 4-key group
    const int poff = (pos & 7) * 2;  // byte offset inside the column
    const uint32_t* a0 = reinterpret_cast<const uint32_t*>(&vr[0]);
    const uint32_t* a1 = reinterpret_cast<const uint32_t*>(&vr[1]);
    const uint32_t* a2 = reinterpret_cast<const uint32_t*>(&vr[2]);
    const uint32_t* a3 = reinterpret_cast<const uint32_t*>(&vr[3]);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int ch = cg * 8 + c;
      const int wi = c >> 1;
      uint2 wv;
      if (c & 1) {
        wv.x = pair_hi(a0[wi], a1[wi]);
        wv.y = pair_hi(a2[wi], a3[wi]);
      } else {
        wv.x = pair_lo(a0[wi], a1[wi]);
        wv.y = pair_lo(a2[wi], a3[wi]);
      }
      const int phys = pcol ^ vt_swizzle(ch);
      *reinterpret_cast<uint2*>(vt_lds[b] + ch * VT_ROW + phys * 16 + poff) = wv;
    }
  };

  f32x16_t o[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[cb][e] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  // prologue: tile 0 into buffer 0, tile 1 in registers, tile 2's entries
  if (loader) {
    fetch_entries(0);
    issue_loads(0);
    store_tile(0);
    if (ntiles > 1) fetch_entries(1);
  }
  __syncthreads();
  if (loader) {
    if (ntiles > 1) issue_loads(1);
    if (ntiles > 2) fetch_entries(2);
  }

  for (int t = 0; t < ntiles; ++t) {
    const int n0 = t * BN;
    const uint8_t* kt = k_lds[t & 1];
    const uint8_t* vt = vt_lds[t & 1];
    if (n0 <= wlim_hi) {
      // ---- S^T = K Q^T: two 32-key blocks
      f32x16_t sc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[kb][e] = 0.f;
        const int key = 32 * kb + q32;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int c = 2 * ks + hi;
          const bf16x8_t a =
              *reinterpret_cast<const bf16x8_t*>(kt + (key * NCOL + (c ^ (key & (NCOL - 1)))) * 16);
          sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[ks], sc[kb], 0, 0, 0);
        }
      }
      // ---- causal mask on diagonal tiles, online softmax in the log2
      // domain: the scale (> 0) is applied to the row maximum and folded
      // into one fma per score
      const bool need_mask = (n0 + BN - 1) > wlim_lo;
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = n0 + 32 * kb + 8 * (e >> 2) + 4 * hi + (e & 3);
            if (key > lim) sc[kb][e] = -INFINITY;
          }
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[kb][e]);
      mx = fmaxf(mx, shfl_xor_f(mx, 32));
      const float mnew = fmaxf(m_run, mx * p.scale_log2);
      const float alpha = fast_exp2(m_run - mnew);
      m_run = mnew;
      float lsum = 0.f;
      bf16x8_t pop[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        uint32_t wds[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const int e = 8 * (kk & 1) + 2 * e2;
          const float p0 = fast_exp2(fmaf(sc[kk >> 1][e], p.scale_log2, -mnew));
          const float p1 = fast_exp2(fmaf(sc[kk >> 1][e + 1], p.scale_log2, -mnew));
          lsum += p0 + p1;
          wds[e2] = pack_bf16(p0, p1);
        }
        pop[kk] = __builtin_bit_cast(bf16x8_t, make_uint4(wds[0], wds[1], wds[2], wds[3]));
      }
      l_run = l_run * alpha + lsum;
      // the rescale is skipped when no row of the wave moved its maximum
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[cb][e] *= alpha;
      }
      // ---- O^T += V^T P^T
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int ch = 32 * cb + q32;
        const uint8_t* vrow = vt + ch * VT_ROW;
        const int sw = vt_swizzle(ch);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int pc = (2 * kk + hi) ^ sw;
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(vrow + pc * 16);
          o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pop[kk], o[cb], 0, 0, 0);
        }
      }
    }
    // tile t+1: registers -> the other buffer; then tile t+2's loads and
    // tile t+3's page entries go out
    if (loader && t + 1 < ntiles) store_tile((t + 1) & 1);
    __syncthreads();
    if (loader) {
      if (t + 2 < ntiles) issue_loads(t + 2);
      if (t + 3 < ntiles) fetch_entries(t + 3);
    }
  }

  // ---- normalise and write: lane holds channels 32cb + 8(e/4) + 4hi + e%4
  const float l_tot = l_run + shfl_xor_f(l_run, 32);
  if (mrow < M) {
    const float inv = 1.f / l_tot;
    uint16_t* orow = p.out + (static_cast<int64_t>(p.cu_extend[r] + ti) * Hq + g * G + hh) * D;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int ch = 32 * cb + 8 * e4 + 4 * hi;
        uint2 wv;
        wv.x = pack_bf16(o[cb][4 * e4 + 0] * inv, o[cb][4 * e4 + 1] * inv);
        wv.y = pack_bf16(o[cb][4 * e4 + 2] * inv, o[cb][4 * e4 + 3] * inv);
        *reinterpret_cast<uint2*>(orow + ch) = wv;
      }
    }
  }
}

hipError_t launch_extend(const ExtendParams& p, int head_dim, int batch, hipStream_t stream) {
  const dim3 grid(p.num_mtiles, p.num_kv_heads, batch);
  const bool pow2 = p.page_shift >= 0;
  if (head_dim == 128) {
    if (pow2)
      hipLaunchKernelGGL((extend_kernel<128, true>), grid, dim3(256), 0, stream, p, p.page_table);
    else
      hipLaunchKernelGGL((extend_kernel<128, false>), grid, dim3(256), 0, stream, p, p.page_table);
  } else {
    if (pow2)
      hipLaunchKernelGGL((extend_kernel<64, true>), grid, dim3(256), 0, stream, p, p.page_table);
    else
      hipLaunchKernelGGL((extend_kernel<64, false>), grid, dim3(256), 0, stream, p, p.page_table);
  }
  return hipGetLastError();
}

}  // namespace msgl
