// Body of one extend workgroup, shared by the extend kernel and the
// single-launch mixed kernel.  The design is described at the top of
// extend.hip; this header holds the device code only.
#pragma once

#include <type_traits>

#include "common.h"

namespace msgl {
namespace extend_impl {

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// ds_read_b64_tr_b16 at byte address `addr` of the LDS window
__device__ __forceinline__ i16x4_t lds_read_tr16(const uint8_t* addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4_t*)(__attribute__((address_space(3))) const uint8_t*)(addr));
}

// 16 bytes per lane from the buffer at byte offset `off` straight into LDS:
// lane i writes lds_base + 16*i (one 1 KiB run per wave instruction)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, uint8_t* lds_base, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc, (__attribute__((address_space(3))) void*)(__attribute__((address_space(3))) uint8_t*)lds_base,
      16, off, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t extend_rsrc(const void* base, uint32_t bytes) {
  // dword 3 = 0x00020000: 32-bit data format, raw (unswizzled) addressing
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// (lo, hi) rounded to nearest-even fp16 and packed (v_cvt_pk_f16_f32)
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, f16x2_t));
}
// a pair of bf16 values (one 32-bit word) as a pair of fp16 values
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  return pack_f16(__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u));
}
// a.lo*b.lo + a.hi*b.hi + c on fp16 pairs, fp32 accumulate
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c,
                                false);
}

// Rows of the running maximum move only by more than this (log2 domain):
// probabilities stay below 2^8, far inside bf16 / fp32 range.
constexpr float kMaxSlack = 8.f;
// A lane's row sum over one tile (32 probabilities) above this means some
// probability may exceed 2^kMaxSlack.
constexpr float kSumLimit = 256.f;

template <int D, int WAVES>
struct ExtendShape {
  static constexpr int BM = 32 * WAVES;   // packed rows per workgroup
  static constexpr int BN = 64;           // keys per tile
  static constexpr int KS = D / 16;       // MFMA k-steps of Q.K^T
  static constexpr int CB = D / 32;       // 32-channel blocks of the output
  static constexpr int ROWB = D * 2;      // bytes per staged K or V row
  static constexpr int SPR = ROWB / 16;   // 16-byte slots per row
  static constexpr int K_BYTES = BN * ROWB;
  static constexpr int STAGE = 2 * K_BYTES;        // K then V of one tile
  static constexpr int RPI = 1024 / ROWB;          // rows per DMA instruction
  static constexpr int NINST = BN / RPI;           // DMA instructions per tile and matrix
  static constexpr int IPW = NINST / WAVES;        // ... per wave
  static_assert(IPW >= 1 && IPW * WAVES == NINST, "DMA instructions must split evenly");
};

// XOR permutation of the 16-byte slots of staged row `row` (0..63 of a
// tile).  K: 16 lanes reading 16 consecutive rows at one logical slot hit
// 16 distinct bank groups.  V: the 32 lanes of one transpose-read pass
// (rows 4hi + j, j = 0..3, slots of two channel halves) hit 64 distinct
// banks.  Both depend only on row bits that are fixed for a lane.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}


// LDS bytes of one workgroup
template <int D, int WAVES>
constexpr int lds_bytes() {
  return 2 * ExtendShape<D, WAVES>::STAGE;
}

// Row tile `mt` (32*WAVES packed rows) of request r and kv head g; with
// p.num_splits > 1, share `split` of its key tiles.
// lds: lds_bytes<D, WAVES>() bytes of LDS, 16-byte aligned.
template <int D, bool POW2, int WAVES>
__device__ __forceinline__ void extend_block(const ExtendParams& p,
                                             const int32_t* __restrict__ page_table, int g, int r,
                                             int mt, uint8_t* lds, int split = 0) {
  using S = ExtendShape<D, WAVES>;
  constexpr int BM = S::BM, BN = S::BN, KS = S::KS, CB = S::CB;
  constexpr int ROWB = S::ROWB, SPR = S::SPR, K_BYTES = S::K_BYTES, STAGE = S::STAGE;
  constexpr int RPI = S::RPI, IPW = S::IPW;

  const int G = p.group;
  // lengths above the host-side bounds break the caller's contract; clamp
  // them so that no page_table entry past the row's bound is read
  const int E = min(p.extend_lens[r], p.max_extend_len);
  if (p.skip_single && E == 1) return;  // a decode row of a mixed batch
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

  // lds: the two K/V stages (2 * STAGE bytes)

  // this lane's query row (rows past the end are clamped and not written)
  const int mrow = m0 + w * 32 + q32;
  const int mrow_c = min(mrow, M - 1);
  const int ti = mrow_c / G;
  const int hh = mrow_c - ti * G;
  const int lim = P + ti;
  const bool wave_rows = m0 + w * 32 < M;  // does this wave own any row

  // first token row of the request, kept in a register: the output
  // stores could alias the array, so re-reading it would reload it each time
  const int cu_r = p.cu_extend[r];
  const uint16_t* qp = p.q + static_cast<int64_t>(cu_r + ti) * p.q_stride +
                       static_cast<int64_t>(g * G + hh) * D + hi * 8;
  // q enters the MFMA as stored; the scores are scaled in fp32
  bf16x8_t qop[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qop[ks] = *reinterpret_cast<const bf16x8_t*>(qp + ks * 16);
  const float c2 = p.scale_log2;

  const int wrow0 = min(m0 + w * 32, M - 1);
  const int wrow1 = min(m0 + w * 32 + 31, M - 1);
  const int wlim_lo = P + wrow0 / G;
  const int wlim_hi = P + wrow1 / G;
  const int kv_end = P + (min(m0 + BM, M) - 1) / G + 1;
  const int ntiles = (kv_end + BN - 1) / BN;
  // the key tiles this workgroup walks, [t0, t1): all of them, or one
  // share of the tiles that every row of the tile sees in full (keys up to
  // the first row's limit), the last share also taking the tiles that
  // cross the rows' limits.  A share's first tile is then fully visible to
  // every row, so each row's running maximum starts finite; a share can be
  // empty when few tiles are shared.
  const int nsplit = p.num_splits;
  int t0 = 0, t1 = ntiles;
  if (nsplit > 1) {
    const int nfull = min((P + m0 / G + 1) / BN, ntiles);
    t0 = split * nfull / nsplit;
    t1 = split + 1 == nsplit ? ntiles : (split + 1) * nfull / nsplit;
  }

  const int32_t* pt = page_table + static_cast<int64_t>(p.table_idx[r]) * p.pt_stride;
  const int ps = p.page_size;
  const int sh = p.page_shift;
  const uint32_t row_bytes = static_cast<uint32_t>(p.num_kv_heads) * D * 2;
  const uint32_t head_off = static_cast<uint32_t>(g) * D * 2;
  const __amdgpu_buffer_rsrc_t krs =
      extend_rsrc(p.k_cache + static_cast<int64_t>(g) * D, p.half_bytes - head_off);
  const __amdgpu_buffer_rsrc_t vrs =
      extend_rsrc(p.v_cache + static_cast<int64_t>(g) * D, p.half_bytes - head_off);

  // DMA role, all waves: wave w fills rows RPI*i .. RPI*i+RPI-1 of the K
  // and V tiles for i = w*IPW .. w*IPW+IPW-1; lane l fetches LDS slot
  // l % SPR of row RPI*i + l / SPR, i.e. the row's column slot ^ swz(row).
  // Its page entry is fetched a tile ahead; keys past kv_end are clamped
  // to the last key, whose row is valid (they are masked for every row).
  int ent[IPW];
  auto dma_row = [&](int k) { return RPI * (w * IPW + k) + lane / SPR; };
  auto dma_key = [&](int t, int k) { return min(t * BN + dma_row(k), kv_end - 1); };
  auto fetch_entries = [&](int t) {
#pragma unroll
    for (int k = 0; k < IPW; ++k) {
      const int key = dma_key(t, k);
      ent[k] = POW2 ? pt[key >> sh] : pt[key / ps];
    }
  };
  auto issue_dma = [&](int t, int stage) {  // tile t into stage, from the entries in ent
#pragma unroll
    for (int k = 0; k < IPW; ++k) {
      const int row = dma_row(k);
      const int key = dma_key(t, k);
      const int slot = POW2 ? (ent[k] << sh) + (key & (ps - 1)) : ent[k] * ps + key % ps;
      const uint32_t base = static_cast<uint32_t>(slot) * row_bytes;
      const int sl = lane % SPR;
      const int i = w * IPW + k;
      dma16(krs, lds + stage * STAGE + i * 1024, base + (sl ^ swz_k<D>(row)) * 16);
      dma16(vrs, lds + stage * STAGE + K_BYTES + i * 1024, base + (sl ^ swz_v<D>(row)) * 16);
    }
  };

  f32x16_t o[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[cb][e] = 0.f;
  // m_run: the running maximum of the scaled scores s*scale*log2(e) of
  // this lane's query column (log2 units)
  float m_run = -INFINITY;
  float l_run = 0.f;

  // the V rows this wave loaded into `stage`, bf16 -> fp16 in place (its
  // IPW KiB of the V tile; the DMA's LDS writes are waited for first)
  auto convert_v = [&](int stage) {
    uint8_t* vb = lds + stage * STAGE + K_BYTES + w * IPW * 1024 + lane * 16;
    __builtin_amdgcn_s_waitcnt(0x0F70);
#pragma unroll
    for (int k = 0; k < IPW; ++k) {
      u32x4_t x = *reinterpret_cast<const u32x4_t*>(vb + k * 1024);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = bf16x2_to_f16x2(x[e]);
      *reinterpret_cast<u32x4_t*>(vb + k * 1024) = x;
    }
  };

  // prologue: tile t0 in stage 0; tile t0+1 on its way to stage 1; tile
  // t0+2's entries in flight (the barrier's fence waits for the DMA)
  if (t1 > t0) {
    fetch_entries(t0);
    issue_dma(t0, 0);
    if (t0 + 1 < t1) fetch_entries(t0 + 1);
    convert_v(0);
    __syncthreads();
    if (t0 + 1 < t1) issue_dma(t0 + 1, 1);
    if (t0 + 2 < t1) fetch_entries(t0 + 2);
  }

  // the q operands are redefined here by an empty asm: the waitcnt pass
  // would otherwise make the first MFMAs of every tile wait on the tile
  // loads in flight
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qop[ks]));

  // per-lane LDS read offsets.  K operand (k-step ks): row q32 (+32 per
  // key block), logical slot 2ks + hi.  V operand (channel block cb):
  // lane 4j+q of each 16-lane group reads key row 4*hi + j (+8 for the
  // second read, +16 per k-step) at channels 16*(group&1) + 4q .. +3 of
  // the block, an 8-byte half of one slot.
  uint32_t kofs[KS], vofs[CB];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kofs[ks] = q32 * ROWB + ((2 * ks + hi) ^ swz_k<D>(q32)) * 16;
  {
    const int j = (lane & 15) >> 2, q = lane & 3, grp = lane >> 4;
    const int vrow = 4 * hi + j;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int logical = 4 * cb + 2 * (grp & 1) + (q >> 1);
      vofs[cb] = K_BYTES + vrow * ROWB + (logical ^ swz_v<D>(vrow)) * 16 + 8 * (q & 1);
    }
  }

  // one tile; ST (compile time) is its stage, so that stage offsets are
  // immediates of the LDS reads
  auto tile = [&](int t, auto stage_c) {
    constexpr int ST = decltype(stage_c)::value;
    const int n0 = t * BN;
    if (wave_rows && n0 <= wlim_hi) {
      const uint8_t* kt = lds + ST * STAGE;
      const uint8_t* vt = lds + ST * STAGE;
      // ---- S^T = K Q^T: two 32-key blocks.  The K operands of block 1 are
      // read while block 0 multiplies, and the V^T operands of the first
      // channel block while block 1 does (the scheduling groups pin that
      // order: LDS reads stay several MFMAs ahead of their use).  A V^T
      // operand (channel block cb, k-step kk) is two transpose reads: keys
      // 16kk + 4hi + 0..3 and 16kk + 8 + 4hi + 0..3 of the lane's channel.
      f32x16_t sc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[kb][e] = 0.f;
      bf16x8_t ka[KS];
      f16x8_t va[4];
      auto load_va = [&](int cb, int kk) {
        const i16x4_t lo = lds_read_tr16(vt + vofs[cb] + kk * 16 * ROWB);
        const i16x4_t hi8 = lds_read_tr16(vt + vofs[cb] + (kk * 16 + 8) * ROWB);
        return __builtin_bit_cast(f16x8_t, __builtin_shufflevector(lo, hi8, 0, 1, 2, 3, 4, 5, 6, 7));
      };
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) ka[ks] = *reinterpret_cast<const bf16x8_t*>(kt + kofs[ks]);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qop[ks], sc[0], 0, 0, 0);
        ka[ks] = *reinterpret_cast<const bf16x8_t*>(kt + kofs[ks] + 32 * ROWB);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        sc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qop[ks], sc[1], 0, 0, 0);
        if (ks < 4) va[ks] = load_va(0, ks);
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
        if (ks < 4) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
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
      // ---- online softmax in the log2 domain, on x = s*scale*log2(e).
      // Fast path: exponentiate against the running maximum as it stands;
      // that is exact softmax arithmetic as long as no probability exceeds
      // 2^8, which a lane row sum of at most 2^8 guarantees.  Otherwise (and
      // on a wave's first tile, whose maximum is still -inf) the tile
      // maximum is taken, the running maximum moves if the tile's exceeds
      // it by more than 2^8, and the probabilities are recomputed against
      // the new maximum.
      float lsum = 0.f;
      f16x8_t pop[4];
      constexpr uint32_t kOnes = 0x3C003C00u;  // fp16 (1, 1)
      auto probabilities = [&](float mref) {  // p = 2^(s*c2 - mref)
        // the row sum adds the fp16 values that the P.V product uses, in
        // four independent partial sums (one per k-step) so that the dot2
        // accumulations do not form one serial chain
        float part[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          uint32_t wds[4];
          part[kk] = 0.f;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const int e = 8 * (kk & 1) + 2 * e2;
            const float p0 = fast_exp2(__builtin_fmaf(sc[kk >> 1][e], c2, -mref));
            const float p1 = fast_exp2(__builtin_fmaf(sc[kk >> 1][e + 1], c2, -mref));
            wds[e2] = pack_f16(p0, p1);
            part[kk] = dot2_f16(wds[e2], kOnes, part[kk]);
          }
          pop[kk] = __builtin_bit_cast(f16x8_t, make_uint4(wds[0], wds[1], wds[2], wds[3]));
        }
        lsum = (part[0] + part[1]) + (part[2] + part[3]);
      };
      bool slow = m_run == -INFINITY;
      if (__builtin_amdgcn_ballot_w64(slow) == 0) {
        probabilities(m_run);
        slow = !(lsum <= kSumLimit);  // also catches inf
      }
      if (__builtin_amdgcn_ballot_w64(slow) != 0) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[kb][e]);
        mx = xor32_max(mx) * c2;  // scale > 0: the maximum commutes with it
        const bool move = mx > m_run + kMaxSlack;
        const float mnew = move ? mx : m_run;
        const float alpha = fast_exp2(m_run - mnew);
        probabilities(mnew);
        m_run = mnew;
        // the rescale is skipped when no row of the wave moved its maximum
        if (__builtin_amdgcn_ballot_w64(move) != 0) {
          l_run *= alpha;
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[cb][e] *= alpha;
        }
      }
      l_run += lsum;
      // ---- O^T += V^T P^T; the next channel block's operands are read one
      // MFMA ahead
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[kk], pop[kk], o[cb], 0, 0, 0);
          if (cb + 1 < CB) va[kk] = load_va(cb + 1, kk);
        }
      }
#pragma unroll
      for (int i = 0; i < 4 * (CB - 1); ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    // every wave is done with this stage and tile t+1 has landed in the
    // other one (vmcnt(0): the DMA is a vector-memory operation), its V
    // rows turned to fp16 by the waves that loaded them; then tile t+2
    // goes into this stage and tile t+3's page entries go out
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if (t + 1 < t1) convert_v(ST ^ 1);
    __syncthreads();
    if (t + 2 < t1) issue_dma(t + 2, ST);
    if (t + 3 < t1) fetch_entries(t + 3);
  };
  for (int t = t0; t < t1; t += 2) {
    tile(t, std::integral_constant<int, 0>{});
    if (t + 1 < t1) tile(t + 1, std::integral_constant<int, 1>{});
  }

  // ---- normalise; the lane holds channels 32cb + 8(e/4) + 4hi + e%4 of
  // its row.  The wave's 32 rows are staged in LDS (16-byte slots
  // XOR-permuted by row, so that the 8-byte writes and the 16-byte reads
  // spread over the banks) and stored as whole rows, 16 bytes a lane, so
  // that each store instruction covers full cache lines.  The stores are
  // nontemporal: nothing here reads the output again, and streaming it out
  // now keeps dirty lines from being written back later, in the middle of
  // whatever runs next.  Every wave has passed the loop's last barrier, so
  // the stages are free.
  static_assert(WAVES * 32 * ROWB <= 2 * STAGE, "output staging must fit in the stages");
  if (nsplit > 1) {
    // ---- one key share: o / l in fp32 and (m, l) of each of the wave's
    // rows, for the merge kernel.  The lane holds channels 32cb + 8e4 + 4hi
    // + 0..3 of its row for e4 = 0..3: one 16-byte store each.  A row that
    // saw no key (an empty share) gives (-inf, 0) and zeros.
    const float lt = xor32_sum(l_run);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (wave_rows && mrow < M) {
      const int64_t u = (static_cast<int64_t>(cu_r + ti) * Hq + g * G + hh) * nsplit + split;
      float* op = p.ws_o + u * D + 4 * hi;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4)
          *reinterpret_cast<float4*>(op + 32 * cb + 8 * e4) =
              make_float4(o[cb][4 * e4] * inv, o[cb][4 * e4 + 1] * inv, o[cb][4 * e4 + 2] * inv,
                          o[cb][4 * e4 + 3] * inv);
      if (hi == 0) *reinterpret_cast<float2*>(p.ws_ml + u * 2) = make_float2(lt > 0.f ? m_run : -INFINITY, lt);
    }
    return;
  }
  {
    const float inv = 1.f / xor32_sum(l_run);
    uint8_t* ow = lds + w * 32 * ROWB;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int slot = 4 * cb + e4;  // channels 8*slot .. 8*slot+7
        uint2 wv;
        wv.x = pack_bf16(o[cb][4 * e4 + 0] * inv, o[cb][4 * e4 + 1] * inv);
        wv.y = pack_bf16(o[cb][4 * e4 + 2] * inv, o[cb][4 * e4 + 3] * inv);
        *reinterpret_cast<uint2*>(ow + q32 * ROWB + (slot ^ (q32 & (SPR - 1))) * 16 + 8 * hi) = wv;
      }
    }
    __syncthreads();
    constexpr int RPS = 64 / SPR;  // rows per store instruction
    const int k = lane % SPR;
#pragma unroll
    for (int i = 0; i < 32 / RPS; ++i) {
      const int rr = i * RPS + lane / SPR;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ow + rr * ROWB + (k ^ (rr & (SPR - 1))) * 16);
      const int orow_m = m0 + w * 32 + rr;
      if (orow_m < M) {
        const int oti = orow_m / G;
        const int ohh = orow_m - oti * G;
        uint16_t* dst = p.out + (static_cast<int64_t>(cu_r + oti) * Hq + g * G + ohh) * D + k * 8;
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(dst));
      }
    }
  }
}

}  // namespace extend_impl
}  // namespace msgl
