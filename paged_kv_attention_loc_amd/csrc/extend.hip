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
//   * each wave computes S^T = K Q^T, so a lane holds one query column and
//     16 keys per 32-key block: the row maximum and sum need only one
//     exchange with the lane 32 apart;
//   * K tiles are staged in LDS row-major with a 16-byte XOR swizzle;
//     V tiles are staged transposed (channel-major) so the A operand of
//     O^T = V^T P^T is one 16-byte LDS read, with the keys of every 16-key
//     group stored in the order in which the S^T accumulator registers hold
//     them -- P^T then feeds the second MFMA straight from registers;
//   * masking is applied only on tiles that cross a row's causal limit.
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

}  // namespace

template <int D>
__global__ __launch_bounds__(256) void extend_kernel(ExtendParams p) {
  constexpr int BM = 128;       // packed rows per workgroup
  constexpr int BN = 64;        // keys per tile
  constexpr int NCOL = D / 8;   // 16-byte columns per K row
  constexpr int KS = D / 16;    // MFMA k-steps of Q.K^T
  constexpr int CB = D / 32;    // 32-channel blocks of the output
  constexpr int VT_ROW = BN * 2;  // bytes per transposed V row

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

  __shared__ uint4 k_lds[BN * NCOL];
  __shared__ __attribute__((aligned(16))) uint8_t vt_lds[D * VT_ROW];

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

  const int32_t* pt = p.page_table + static_cast<int64_t>(p.table_idx[r]) * p.pt_stride;
  const int ps = p.page_size;
  const int64_t row_elems = static_cast<int64_t>(p.num_kv_heads) * D;
  const uint16_t* kbase = p.k_cache + static_cast<int64_t>(g) * D;
  const uint16_t* vbase = p.v_cache + static_cast<int64_t>(g) * D;

  f32x16_t o[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[cb][e] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  for (int n0 = 0; n0 < kv_end; n0 += BN) {
    // ---- K tile -> LDS (row-major, 16-byte XOR swizzle by key)
#pragma unroll
    for (int it = 0; it < (BN * NCOL) / 256; ++it) {
      const int pi = it * 256 + tid;
      const int key = pi / NCOL;
      const int c = pi % NCOL;
      const int kk = min(n0 + key, kv_end - 1);
      const int64_t slot = token_slot_safe(pt, kk, ps, p.num_slots);
      const uint4 val = *reinterpret_cast<const uint4*>(kbase + slot * row_elems + c * 8);
      k_lds[key * NCOL + (c ^ (key & (NCOL - 1)))] = val;
    }
    // ---- V tile -> LDS transposed: row = channel, 4 keys per 8-byte write
    if (tid < (BN / 4) * (D / 8)) {
      const int kq = tid / (D / 8);
      const int cg = tid % (D / 8);
      uint4 vv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kk = min(n0 + kq * 4 + j, kv_end - 1);
        const int64_t slot = token_slot_safe(pt, kk, ps, p.num_slots);
        vv[j] = *reinterpret_cast<const uint4*>(vbase + slot * row_elems + cg * 8);
      }
      const int pos = vt_group_pos(kq);
      const int pcol = pos >> 3;          // 16-byte column of this 4-key group
      const int poff = (pos & 7) * 2;     // byte offset inside the column
      const uint32_t* a0 = reinterpret_cast<const uint32_t*>(&vv[0]);
      const uint32_t* a1 = reinterpret_cast<const uint32_t*>(&vv[1]);
      const uint32_t* a2 = reinterpret_cast<const uint32_t*>(&vv[2]);
      const uint32_t* a3 = reinterpret_cast<const uint32_t*>(&vv[3]);
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
        const int phys = pcol ^ ((ch >> 1) & 7);
        *reinterpret_cast<uint2*>(vt_lds + ch * VT_ROW + phys * 16 + poff) = wv;
      }
    }
    __syncthreads();

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
              __builtin_bit_cast(bf16x8_t, k_lds[key * NCOL + (c ^ (key & (NCOL - 1)))]);
          sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[ks], sc[kb], 0, 0, 0);
        }
      }
      // ---- scale, causal mask on diagonal tiles, online softmax
      const bool need_mask = (n0 + BN - 1) > wlim_lo;
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float x = sc[kb][e] * p.scale_log2;
          if (need_mask) {
            const int key = n0 + 32 * kb + 8 * (e >> 2) + 4 * hi + (e & 3);
            if (key > lim) x = -INFINITY;
          }
          sc[kb][e] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = fmaxf(mx, shfl_xor_f(mx, 32));
      const float mnew = fmaxf(m_run, mx);
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
          const uint16_t b0 = f32_to_bf16(fast_exp2(sc[kk >> 1][e] - mnew));
          const uint16_t b1 = f32_to_bf16(fast_exp2(sc[kk >> 1][e + 1] - mnew));
          lsum += bf16_to_f32(b0) + bf16_to_f32(b1);
          wds[e2] = static_cast<uint32_t>(b0) | (static_cast<uint32_t>(b1) << 16);
        }
        pop[kk] = __builtin_bit_cast(bf16x8_t, make_uint4(wds[0], wds[1], wds[2], wds[3]));
      }
      l_run = l_run * alpha + lsum;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[cb][e] *= alpha;
      // ---- O^T += V^T P^T
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int ch = 32 * cb + q32;
        const uint8_t* vrow = vt_lds + ch * VT_ROW;
        const int sw = (ch >> 1) & 7;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int pc = (2 * kk + hi) ^ sw;
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(vrow + pc * 16);
          o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pop[kk], o[cb], 0, 0, 0);
        }
      }
    }
    __syncthreads();
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
  if (head_dim == 128)
    hipLaunchKernelGGL(extend_kernel<128>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(extend_kernel<64>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace msgl
