// Split-KV paged decode attention and the log-sum-exp merge of its partials.
//
// Decode attends one new query token per request over all of its KV, read
// through the request's page_table row ("Code Notes: mini-sglang", Engine
// Layer table rows BaseAttnBackend / GraphRunner; Scheduler Layer table row
// TableManager).  The work is HBM-bound: every K/V byte is read once and
// used for G = q_heads / kv_heads query heads, so the kernel is built around
// streaming K/V with wide loads, not around matrix cores.
//
// One wave64 workgroup handles (request, kv head, chunk of `chunk` tokens),
// in tiles of 64 tokens:
//   * each lane owns one token of the tile for q.K: the tile's K rows are
//     staged in LDS (16-byte pieces, XOR-swizzled by token so that the
//     token-per-lane reads are bank-conflict free) and every lane runs
//     v_dot2_f32_bf16 over its own row against the G query heads, which are
//     broadcast from LDS;
//   * softmax statistics are kept per head in the log2 domain (scale folded
//     into the exponent), the tile maximum via DPP row reductions;
//   * for p.V each lane owns 8 channels of every 4th (d = 128) or 8th
//     (d = 64) token, with V loaded straight into registers by coalesced
//     16-byte loads; two tokens' V values are paired with v_perm and
//     multiplied by the matching bf16 pair of probabilities with one
//     v_dot2_f32_bf16;
//   * a request with a single chunk writes its bf16 output directly, longer
//     ones write fp32 partials (unnormalised o, max, sum) for the merge.
#include "common.h"

namespace msgl {

template <int D, int GM>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeParams p) {
  constexpr int LPT = D / 8;     // lanes per 16-byte-piece token row
  constexpr int TPI = 64 / LPT;  // tokens per wave-wide load
  constexpr int NI = 64 / TPI;   // loads per 64-token tile
  constexpr int TILE = 64;
  static_assert(NI % 2 == 0, "token pairs");

  const int s = blockIdx.x;
  const int g = blockIdx.y;
  const int r = blockIdx.z;
  const int lane = threadIdx.x;
  const int G = p.group;
  const int Hq = p.num_kv_heads * G;
  // a length above max_seq_len breaks the caller's contract; clamp it so
  // that no page_table entry past the row's bound is read
  const int L = min(p.seq_lens[r], p.max_seq_len);

  if (L <= 0) {  // padding row: zeros, no KV read
    if (s == 0) {
      uint16_t* o = p.out + (static_cast<int64_t>(r) * Hq + g * G) * D;
      for (int i = lane; i < G * LPT; i += 64) reinterpret_cast<uint4*>(o)[i] = make_uint4(0, 0, 0, 0);
    }
    return;
  }
  const int nch = (L + p.chunk - 1) / p.chunk;
  if (s >= nch) return;

  __shared__ uint4 k_lds[TILE * LPT];
  __shared__ uint4 q_lds[GM * LPT];
  __shared__ uint32_t p_lds[(TILE / 2) * GM];

  const uint16_t* qrow = p.q + static_cast<int64_t>(r) * p.q_stride + static_cast<int64_t>(g) * G * D;
  for (int i = lane; i < G * LPT; i += 64) q_lds[i] = reinterpret_cast<const uint4*>(qrow)[i];

  const int32_t* pt = p.page_table + static_cast<int64_t>(p.table_idx[r]) * p.pt_stride;
  const int ps = p.page_size;
  const int64_t row_elems = static_cast<int64_t>(p.num_kv_heads) * D;
  const uint16_t* kbase = p.k_cache + static_cast<int64_t>(g) * D;
  const uint16_t* vbase = p.v_cache + static_cast<int64_t>(g) * D;

  const int t_begin = s * p.chunk;
  const int t_end = min(L, t_begin + p.chunk);
  const int sub = lane / LPT;  // token subset for p.V
  const int col = lane % LPT;  // 16-byte column for loads and p.V

  float m_run[GM], l_run[GM], acc[GM][8];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[h][j] = 0.f;
  }
  __syncthreads();

  for (int t0 = t_begin; t0 < t_end; t0 += TILE) {
    const int n = min(TILE, t_end - t0);
    // Lanes past the end reuse the last valid token's slot: in-bounds data,
    // weighted by an exact zero below.
    const int tok = t0 + min(lane, n - 1);
    const int slot = token_slot_safe(pt, tok, ps, p.num_slots);
    uint4 vr[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int tl = i * TPI + sub;
      const int sl = __shfl(slot, tl, 64);
      const int64_t off = static_cast<int64_t>(sl) * row_elems + col * 8;
      const uint4 kv = *reinterpret_cast<const uint4*>(kbase + off);
      vr[i] = *reinterpret_cast<const uint4*>(vbase + off);
      k_lds[tl * LPT + (col ^ (tl & (LPT - 1)))] = kv;
    }
    __syncthreads();

    // q.K with one token per lane
    float sc[GM];
#pragma unroll
    for (int h = 0; h < GM; ++h) sc[h] = 0.f;
#pragma unroll
    for (int c = 0; c < LPT; ++c) {
      const uint4 kk = k_lds[lane * LPT + (c ^ (lane & (LPT - 1)))];
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        if (h < G) {
          const uint4 qq = q_lds[h * LPT + c];
          float a = sc[h];
          a = dot2_bf16(kk.x, qq.x, a);
          a = dot2_bf16(kk.y, qq.y, a);
          a = dot2_bf16(kk.z, qq.z, a);
          a = dot2_bf16(kk.w, qq.w, a);
          sc[h] = a;
        }
      }
    }

    // online softmax, one head at a time; p stored as bf16 pairs of the
    // two tokens that the p.V lanes combine: (i*TPI+sub, (i+1)*TPI+sub)
    const bool valid = lane < n;
    const int ii = lane / TPI, ss = lane % TPI;
    const int pair = (ii >> 1) * TPI + ss;
    uint16_t* p16 = reinterpret_cast<uint16_t*>(p_lds);
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h < G) {
        const float x = valid ? sc[h] * p.scale_log2 : -INFINITY;
        const float mnew = fmaxf(m_run[h], wave_max(x));
        const float alpha = fast_exp2(m_run[h] - mnew);
        const uint16_t pb = f32_to_bf16(fast_exp2(x - mnew));
        l_run[h] = l_run[h] * alpha + bf16_to_f32(pb);
        m_run[h] = mnew;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[h][j] *= alpha;
        p16[(pair * GM + h) * 2 + (ii & 1)] = pb;
      }
    }
    __syncthreads();

    // p.V on token pairs
#pragma unroll
    for (int i = 0; i < NI; i += 2) {
      const uint4 va = vr[i], vb = vr[i + 1];
      const uint32_t lo[4] = {pair_lo(va.x, vb.x), pair_lo(va.y, vb.y), pair_lo(va.z, vb.z),
                              pair_lo(va.w, vb.w)};
      const uint32_t hi[4] = {pair_hi(va.x, vb.x), pair_hi(va.y, vb.y), pair_hi(va.z, vb.z),
                              pair_hi(va.w, vb.w)};
      const int pr = (i >> 1) * TPI + sub;
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        if (h < G) {
          const uint32_t pp = p_lds[pr * GM + h];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            acc[h][2 * k] = dot2_bf16(lo[k], pp, acc[h][2 * k]);
            acc[h][2 * k + 1] = dot2_bf16(hi[k], pp, acc[h][2 * k + 1]);
          }
        }
      }
    }
    __syncthreads();
  }

  // combine the token subsets that share a column, and the per-lane sums
  float l_tot[GM];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    l_tot[h] = (h < G) ? wave_sum(l_run[h]) : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float a = acc[h][j];
#pragma unroll
      for (int off = LPT; off < 64; off <<= 1) a += shfl_xor_f(a, off);
      acc[h][j] = a;
    }
  }
  if (nch == 1) {
    if (lane < LPT) {
      uint16_t* o = p.out + (static_cast<int64_t>(r) * Hq + g * G) * D + col * 8;
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        if (h < G) {
          const float inv = 1.f / l_tot[h];
          uint4 w;
          w.x = pack_bf16(acc[h][0] * inv, acc[h][1] * inv);
          w.y = pack_bf16(acc[h][2] * inv, acc[h][3] * inv);
          w.z = pack_bf16(acc[h][4] * inv, acc[h][5] * inv);
          w.w = pack_bf16(acc[h][6] * inv, acc[h][7] * inv);
          *reinterpret_cast<uint4*>(o + h * D) = w;
        }
      }
    }
  } else {
    const int64_t base = (static_cast<int64_t>(r) * p.max_chunks + s) * Hq + g * G;
    if (lane < LPT) {
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        if (h < G) {
          float4* o = reinterpret_cast<float4*>(p.ws_o + (base + h) * D + col * 8);
          o[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
          o[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
        }
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        if (h < G) {
          p.ws_ml[(base + h) * 2 + 0] = m_run[h];
          p.ws_ml[(base + h) * 2 + 1] = l_tot[h];
        }
      }
    }
  }
}

// out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s over the chunks s of
// one (request, q head); requests with a single chunk were finished above.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeParams p) {
  constexpr int CPL = D / 64;  // channels per lane
  const int h = blockIdx.x;
  const int r = blockIdx.y;
  const int lane = threadIdx.x;
  const int Hq = p.num_kv_heads * p.group;
  const int L = min(p.seq_lens[r], p.max_seq_len);
  if (L <= 0) return;
  const int nch = (L + p.chunk - 1) / p.chunk;
  if (nch <= 1) return;
  const int64_t base = static_cast<int64_t>(r) * p.max_chunks * Hq + h;
  float mx = -INFINITY;
  for (int s = 0; s < nch; ++s) mx = fmaxf(mx, p.ws_ml[(base + static_cast<int64_t>(s) * Hq) * 2]);
  float den = 0.f, num[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) num[c] = 0.f;
  for (int s = 0; s < nch; ++s) {
    const int64_t idx = base + static_cast<int64_t>(s) * Hq;
    const float w = fast_exp2(p.ws_ml[idx * 2] - mx);
    den += w * p.ws_ml[idx * 2 + 1];
    const float* o = p.ws_o + idx * D + lane * CPL;
#pragma unroll
    for (int c = 0; c < CPL; ++c) num[c] += w * o[c];
  }
  const float inv = 1.f / den;
  uint16_t* out = p.out + (static_cast<int64_t>(r) * Hq + h) * D + lane * CPL;
#pragma unroll
  for (int c = 0; c < CPL; ++c) out[c] = f32_to_bf16(num[c] * inv);
}

template <int D, int GM>
static void launch_decode_t(const DecodeParams& p, int batch, hipStream_t stream) {
  const dim3 grid(p.max_chunks, p.num_kv_heads, batch);
  hipLaunchKernelGGL((decode_split_kernel<D, GM>), grid, dim3(64), 0, stream, p);
  if (p.max_chunks > 1) {
    const dim3 mgrid(p.num_kv_heads * p.group, batch);
    hipLaunchKernelGGL((decode_merge_kernel<D>), mgrid, dim3(64), 0, stream, p);
  }
}

template <int D>
static void launch_decode_d(const DecodeParams& p, int batch, hipStream_t stream) {
  if (p.group <= 1)
    launch_decode_t<D, 1>(p, batch, stream);
  else if (p.group <= 2)
    launch_decode_t<D, 2>(p, batch, stream);
  else if (p.group <= 4)
    launch_decode_t<D, 4>(p, batch, stream);
  else if (p.group <= 8)
    launch_decode_t<D, 8>(p, batch, stream);
  else
    launch_decode_t<D, 16>(p, batch, stream);
}

hipError_t launch_decode(const DecodeParams& p, int head_dim, int batch, hipStream_t stream) {
  if (head_dim == 128)
    launch_decode_d<128>(p, batch, stream);
  else
    launch_decode_d<64>(p, batch, stream);
  return hipGetLastError();
}

}  // namespace msgl
