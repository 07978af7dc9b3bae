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
//   * a workgroup of WAVES waves owns 32*WAVES packed rows (32 per wave) of
//     one (request, kv head) and walks the keys in tiles of 64 up to its
//     last row's limit.  blockIdx.x is the kv head, so with a multiple of 8
//     kv heads every XCD (workgroups are dealt to the 8 XCDs round-robin)
//     serves one kv head and keeps its K/V -- a shared prefix above all --
//     in its own L2; the heaviest row tiles are launched first;
//   * K/V tiles are double-buffered in LDS, one barrier per tile.  While
//     tile t is computed, tile t+1 is in registers on its way to the other
//     buffer, the row offsets of tile t+2 wait in LDS, and the page-table
//     entries of tile t+3 are in flight;
//   * a tile's row offsets (slot * row bytes) are computed once, by one
//     thread per key, and shared through LDS; rows are read with buffer
//     loads at 32-bit offsets inside the (K or V, layer) sub-tensor, whose
//     range check also absorbs a wild page id;
//   * each wave computes S^T = K Q^T, so a lane holds one query column and
//     16 keys per 32-key block: the row maximum and sum need one exchange
//     with the lane 32 apart (v_permlane32_swap);
//   * K is staged row-major, V transposed (channel-major) so that the A
//     operand of O^T = V^T P^T is one 16-byte LDS read; inside every
//     16-key group V^T keeps the keys in the order in which the S^T
//     accumulator registers hold them, so P^T feeds the second MFMA
//     straight from registers.  Both layouts pad their rows by 16 bytes:
//     with 64 four-byte banks that makes the 16-lane groups of every read
//     and write hit distinct banks, and every LDS address is a per-lane
//     base plus a compile-time offset.  K and V use different loader
//     mappings (16 lanes per K row; 16 key groups per V^T row) for the
//     same reason;
//   * the running maximum only moves when a row's new maximum exceeds it by
//     more than 2^8 in exp2 terms, so the O rescale is rare; masking runs
//     only on tiles that cross a row's causal limit.
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

__device__ __forceinline__ __amdgpu_buffer_rsrc_t extend_rsrc(const void* base, uint32_t bytes) {
  // dword 3 = 0x00020000: 32-bit data format, raw (unswizzled) addressing
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Rows of the running maximum move only by more than this (log2 domain):
// probabilities stay below 2^8, far inside bf16 / fp32 range.
constexpr float kMaxSlack = 8.f;

template <int D, int WAVES>
struct ExtendShape {
  static constexpr int BM = 32 * WAVES;   // packed rows per workgroup
  static constexpr int BN = 64;           // keys per tile
  static constexpr int NCOL = D / 8;      // 16-byte columns per K/V row
  static constexpr int KS = D / 16;       // MFMA k-steps of Q.K^T
  static constexpr int CB = D / 32;       // 32-channel blocks of the output
  static constexpr int K_ROW = D * 2 + 16;   // bytes per staged K row
  static constexpr int V_ROW = BN * 2 + 16;  // bytes per staged V^T row
  static constexpr int K_BYTES = BN * K_ROW;
  static constexpr int V_BYTES = D * V_ROW;
  static constexpr int BUF = K_BYTES + V_BYTES;   // one pipeline stage
  static constexpr int LOADERS = (BN / 4) * NCOL;  // threads that load a tile
  static_assert(LOADERS <= 64 * WAVES, "not enough threads to load a tile");
  static_assert(BN <= 64 * WAVES, "one thread per key computes row offsets");
};

}  // namespace

template <int D, bool POW2, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 2) void extend_kernel(ExtendParams p,
                                                               const int32_t* __restrict__ page_table) {
  using S = ExtendShape<D, WAVES>;
  constexpr int BM = S::BM, BN = S::BN, NCOL = S::NCOL, KS = S::KS, CB = S::CB;
  constexpr int K_ROW = S::K_ROW, V_ROW = S::V_ROW, K_BYTES = S::K_BYTES, BUF = S::BUF;

  const int g = blockIdx.x;
  const int r = blockIdx.y;
  const int mt = p.num_mtiles - 1 - static_cast<int>(blockIdx.z);
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

  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * BUF];
  __shared__ __attribute__((aligned(16))) uint32_t row_off[2][BN];

  // this lane's query row (rows past the end are clamped and not written)
  const int mrow = m0 + w * 32 + q32;
  const int mrow_c = min(mrow, M - 1);
  const int ti = mrow_c / G;
  const int hh = mrow_c - ti * G;
  const int lim = P + ti;
  const bool wave_rows = m0 + w * 32 < M;  // does this wave own any row

  const uint16_t* qp = p.q + static_cast<int64_t>(p.cu_extend[r] + ti) * p.q_stride +
                       static_cast<int64_t>(g * G + hh) * D + hi * 8;
  bf16x8_t qop[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qop[ks] = *reinterpret_cast<const bf16x8_t*>(qp + ks * 16);

  const int wrow0 = min(m0 + w * 32, M - 1);
  const int wrow1 = min(m0 + w * 32 + 31, M - 1);
  const int wlim_lo = P + wrow0 / G;
  const int wlim_hi = P + wrow1 / G;
  const int kv_end = P + (min(m0 + BM, M) - 1) / G + 1;
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

  // row offsets: thread `tid` < BN owns key t*BN + tid (clamped to the last
  // key, whose row is valid; keys past kv_end are masked for every row)
  int ent = 0;
  auto off_key = [&](int t) { return min(t * BN + tid, kv_end - 1); };
  auto fetch_entry = [&](int t) {
    if (tid < BN) {
      const int key = off_key(t);
      ent = POW2 ? pt[key >> sh] : pt[key / ps];
    }
  };
  auto publish_offsets = [&](int t) {
    if (tid < BN) {
      const int key = off_key(t);
      const int slot = POW2 ? (ent << sh) + (key & (ps - 1)) : ent * ps + key % ps;
      row_off[t & 1][tid] = static_cast<uint32_t>(slot) * row_bytes;
    }
  };

  // loader roles: K -- keys 4kqk .. 4kqk+3, 16-byte column cgk (16 lanes
  // cover one row); V -- keys 4kqv .. 4kqv+3, column cgv (16 lanes cover
  // the 16 key groups of one channel column)
  const bool loader = tid < S::LOADERS;
  const int kqk = tid / NCOL, cgk = tid % NCOL;
  const int kqv = tid & 15, cgv = tid >> 4;
  uint4 kr[4], vr[4];
  auto issue_loads = [&](int t) {
    const uint4 ko = *reinterpret_cast<const uint4*>(&row_off[t & 1][4 * kqk]);
    const uint4 vo = *reinterpret_cast<const uint4*>(&row_off[t & 1][4 * kqv]);
    const uint32_t kof[4] = {ko.x, ko.y, ko.z, ko.w};
    const uint32_t vof[4] = {vo.x, vo.y, vo.z, vo.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(krs, kof[j] + cgk * 16, 0, 0);
      const u32x4_t b = __builtin_amdgcn_raw_buffer_load_b128(vrs, vof[j] + cgv * 16, 0, 0);
      kr[j] = make_uint4(a.x, a.y, a.z, a.w);
      vr[j] = make_uint4(b.x, b.y, b.z, b.w);
    }
  };
  // registers -> LDS stage b: K rows, then V transposed with 4 keys per
  // 8-byte write
  uint8_t* const k_st = lds + kqk * 4 * K_ROW + cgk * 16;
  uint8_t* const v_st = lds + K_BYTES + cgv * 8 * V_ROW + vt_group_pos(kqv) * 2;
  auto store_tile = [&](int b) {
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<uint4*>(k_st + b * BUF + j * K_ROW) = kr[j];
    const uint32_t* a0 = reinterpret_cast<const uint32_t*>(&vr[0]);
    const uint32_t* a1 = reinterpret_cast<const uint32_t*>(&vr[1]);
    const uint32_t* a2 = reinterpret_cast<const uint32_t*>(&vr[2]);
    const uint32_t* a3 = reinterpret_cast<const uint32_t*>(&vr[3]);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int wi = c >> 1;
      uint2 wv;
      if (c & 1) {
        wv.x = pair_hi(a0[wi], a1[wi]);
        wv.y = pair_hi(a2[wi], a3[wi]);
      } else {
        wv.x = pair_lo(a0[wi], a1[wi]);
        wv.y = pair_lo(a2[wi], a3[wi]);
      }
      *reinterpret_cast<uint2*>(v_st + b * BUF + c * V_ROW) = wv;
    }
  };

  f32x16_t o[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[cb][e] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  // prologue: offsets of tiles 0 and 1 in LDS, tile 0 staged, tile 1 in
  // registers, tile 2's offsets published and tile 3's entries in flight
  fetch_entry(0);
  publish_offsets(0);
  if (ntiles > 1) fetch_entry(1);
  __syncthreads();
  if (loader) issue_loads(0);
  if (ntiles > 1) publish_offsets(1);
  if (ntiles > 2) fetch_entry(2);
  if (loader) store_tile(0);
  __syncthreads();
  if (loader && ntiles > 1) issue_loads(1);
  if (ntiles > 2) publish_offsets(2);
  if (ntiles > 3) fetch_entry(3);

  // the q operands are redefined here by an empty asm: the waitcnt pass
  // would otherwise make the first MFMAs of every tile wait on the tile
  // loads in flight
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qop[ks]));

  const uint8_t* const k_rd = lds + q32 * K_ROW + hi * 16;
  const uint8_t* const v_rd = lds + K_BYTES + q32 * V_ROW + hi * 16;

  for (int t = 0; t < ntiles; ++t) {
    const int n0 = t * BN;
    if (wave_rows && n0 <= wlim_hi) {
      const uint8_t* kt = k_rd + (t & 1) * BUF;
      const uint8_t* vt = v_rd + (t & 1) * BUF;
      // ---- S^T = K Q^T: two 32-key blocks.  The K operands of block 1 are
      // read while block 0 multiplies, and the V^T operands of the first
      // channel block while block 1 does (the scheduling groups pin that
      // order: LDS reads stay several MFMAs ahead of their use)
      f32x16_t sc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[kb][e] = 0.f;
      bf16x8_t ka[KS];
      bf16x8_t va[4];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) ka[ks] = *reinterpret_cast<const bf16x8_t*>(kt + ks * 32);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qop[ks], sc[0], 0, 0, 0);
        ka[ks] = *reinterpret_cast<const bf16x8_t*>(kt + 32 * K_ROW + ks * 32);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        sc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qop[ks], sc[1], 0, 0, 0);
        if (ks < 4) va[ks] = *reinterpret_cast<const bf16x8_t*>(vt + ks * 32);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (ks < 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      // ---- causal mask on tiles that cross a row's limit
      if (n0 + BN - 1 > wlim_lo) {
        const int lim_rel = lim - n0 - 4 * hi;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (32 * kb + 8 * (e >> 2) + (e & 3) > lim_rel) sc[kb][e] = -INFINITY;
      }
      // ---- online softmax in the log2 domain: the scale (> 0) is applied
      // to the row maximum and folded into one fma per score
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[kb][e]);
      mx = xor32_max(mx) * p.scale_log2;
      const bool move = mx > m_run + kMaxSlack;
      const float mnew = move ? mx : m_run;
      const float alpha = fast_exp2(m_run - mnew);
      m_run = mnew;
      float lsum = 0.f;
      bf16x8_t pop[4];
      constexpr uint32_t kOnes = 0x3F803F80u;  // bf16 (1, 1)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        uint32_t wds[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const int e = 8 * (kk & 1) + 2 * e2;
          const float p0 = fast_exp2(fmaf(sc[kk >> 1][e], p.scale_log2, -mnew));
          const float p1 = fast_exp2(fmaf(sc[kk >> 1][e + 1], p.scale_log2, -mnew));
          wds[e2] = pack_bf16(p0, p1);
          // the row sum adds the bf16 values that the P.V product uses
          lsum = dot2_bf16(wds[e2], kOnes, lsum);
        }
        pop[kk] = __builtin_bit_cast(bf16x8_t, make_uint4(wds[0], wds[1], wds[2], wds[3]));
      }
      if (__builtin_amdgcn_ballot_w64(move) != 0) {
        l_run *= alpha;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[cb][e] *= alpha;
      }
      l_run += lsum;
      // ---- O^T += V^T P^T; the next channel block's operands are read one
      // MFMA ahead
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[kk], pop[kk], o[cb], 0, 0, 0);
          if (cb + 1 < CB)
            va[kk] = *reinterpret_cast<const bf16x8_t*>(vt + (cb + 1) * 32 * V_ROW + kk * 32);
        }
      }
#pragma unroll
      for (int i = 0; i < 4 * (CB - 1); ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    // tile t+1: registers -> the other stage; then tile t+2's loads, tile
    // t+3's offsets and tile t+4's page entries go out
    if (loader && t + 1 < ntiles) store_tile((t + 1) & 1);
    __syncthreads();
    if (loader && t + 2 < ntiles) issue_loads(t + 2);
    if (t + 3 < ntiles) publish_offsets(t + 3);
    if (t + 4 < ntiles) fetch_entry(t + 4);
  }

  // ---- normalise and write: lane holds channels 32cb + 8(e/4) + 4hi + e%4
  const float l_tot = xor32_sum(l_run);
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

namespace {

template <int D, int WAVES>
void launch_extend_t(const ExtendParams& p, int batch, hipStream_t stream) {
  const dim3 grid(p.num_kv_heads, batch, p.num_mtiles);
  if (p.page_shift >= 0)
    hipLaunchKernelGGL((extend_kernel<D, true, WAVES>), grid, dim3(64 * WAVES), 0, stream, p,
                       p.page_table);
  else
    hipLaunchKernelGGL((extend_kernel<D, false, WAVES>), grid, dim3(64 * WAVES), 0, stream, p,
                       p.page_table);
}

}  // namespace

hipError_t launch_extend(const ExtendParams& p, int head_dim, int batch, int waves,
                         hipStream_t stream) {
  if (head_dim == 128) {
    if (waves == 8)
      launch_extend_t<128, 8>(p, batch, stream);
    else
      launch_extend_t<128, 4>(p, batch, stream);
  } else {
    if (waves == 8)
      launch_extend_t<64, 8>(p, batch, stream);
    else
      launch_extend_t<64, 4>(p, batch, stream);
  }
  return hipGetLastError();
}

}  // namespace msgl
