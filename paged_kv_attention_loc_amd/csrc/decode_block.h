// Body of one decode workgroup, shared by the decode kernel and the
// single-launch mixed kernel.  The design is described at the top of
// decode.hip; this header holds the device code only.
#pragma once

#include <type_traits>

#include "common.h"

namespace msgl {
namespace decode_impl {

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kStageBytes = 32768;  // K tile then V tile
// Rows of the running maximum move only by more than this (log2 domain).
constexpr float kMaxSlack = 8.f;
// A lane's sum of 4 probabilities above this means one may exceed 2^kMaxSlack.
constexpr float kSumLimit = 256.f;

__device__ __forceinline__ i16x4_t lds_read_tr16(const uint8_t* addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4_t*)(__attribute__((address_space(3))) const uint8_t*)(addr));
}

// buffer resource words: base, 32-bit range, raw 32-bit addressing
__device__ __forceinline__ u32x4_t buffer_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return (u32x4_t){static_cast<uint32_t>(a), static_cast<uint32_t>(a >> 32) & 0xFFFFu, bytes,
                   0x00020000u};
}

// 16 bytes a lane from byte offset `off` of the buffer into LDS at
// `lds_base` + 16*lane (nontemporal: each byte is read once).  No register
// receives data, so nothing in flight can be overwritten; the caller waits
// with an explicit vmcnt before the barrier that publishes the tile.
// `rs` and `lds_base` are wave-uniform; readfirstlane puts them in SGPRs.
__device__ __forceinline__ void dma16(u32x4_t rs, const uint8_t* lds_base, uint32_t off) {
  // the low 32 bits of a generic pointer into LDS are its LDS address
  const uint32_t la =
      __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_base)));
  u32x4_t rsu;
#pragma unroll
  for (int i = 0; i < 4; ++i) rsu[i] = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(rs[i]));
  // M0 (the LDS address of the instruction) is an input operand: the
  // compiler sets it, and knows it holds that value afterwards
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen nt lds" : : "v"(off), "s"(rsu), "{m0}"(la) : "memory");
}


// Stage size of the decode body for a head group's part of a token row
// (RB bytes): 16 KiB when the group holds one or two kv heads of 128
// channels -- short rows, whose workgroups compute on one or two waves, so
// the stream is latency-bound; four such stages keep three tiles in flight
// in the LDS of two 32 KiB ones (the one-kv-head share of the Llama-3-8B
// batch: 23.7 against 26.2 us) -- else 32 KiB (at head_dim 64 the four
// stages measured 2% slower).  The decode kernel and the mixed kernel both
// take it, so that both cut a batch's tokens into the same tiles and
// ranges (and give the same bits).
template <int D, int RB>
constexpr int decode_stage_bytes() {
  return D == 128 && RB <= 2 * D * 2 ? 16384 : kStageBytes;
}

// LDS bytes of one workgroup with S stages of STB bytes
template <int S, int STB = kStageBytes>
constexpr int lds_bytes() {
  return S * STB + (kDecodeWindow + kDecodeBatch + 1 + kWaves) * 4;
}

// Workgroup `wg` of `nwg` over the token ranges of kv head group `grp`.
// RB: bytes of the head group's part of a token row (head_group * D * 2).
// S: LDS stages (tiles in flight while one is computed: S - 1) of STB
// bytes each (a K tile and a V tile).
// smem: lds_bytes<S, STB>() bytes of LDS, 16-byte aligned.
template <int D, int RB, int S, int STB = kStageBytes>
__device__ __forceinline__ void decode_block(const DecodeParams& p, int wg, int nwg, int grp,
                                             uint8_t* smem) {
  constexpr int KB = RB >= 2048 ? 8 : (STB / 2 / RB < kDecodeMaxTile ? STB / 2 / RB : kDecodeMaxTile);  // tokens per tile
  constexpr int KS = D / 32;                  // k-steps of S^T
  constexpr int CB = D / 16;                  // 16-channel blocks of O^T
  constexpr int NB = KB >= 16 ? KB / 16 : 1;  // 16-key blocks per tile
  constexpr int BK = KB >= 16 ? 16 : KB;      // keys in use per block
  constexpr int NI = 2 * KB * RB / 1024;      // DMA instructions of 1 KiB per tile (K then V)
  constexpr int IPW = NI / kWaves;            // ... per wave
  constexpr int LG_RB = RB == 128 ? 7 : RB == 256 ? 8 : RB == 512 ? 9 : RB == 1024 ? 10 : 11;
  // 16-byte columns of staged rows are XOR-permuted by row when a row spans
  // whole 256-byte bank windows: K reads of 16 rows at one column, and the V
  // transpose reads of 8 rows at one 32-byte piece, then hit distinct banks
  constexpr bool SWZ = (RB & 255) == 0;
  static_assert(IPW * kWaves == NI && KB * RB * 2 <= STB, "tile shape");

  static_assert(S >= 2 && S <= 4, "stages");
  // LDS: S stages, then the window's slots, the token prefix sums of the
  // requests and the per-wave totals of the scan
  uint8_t* const st0 = smem;
  uint8_t* const st1 = smem + STB;
  uint8_t* const st2 = smem + 2 * STB;
  uint8_t* const st3 = smem + 3 * STB;
  int32_t* const slot_of = reinterpret_cast<int32_t*>(smem + S * STB);
  int32_t* const pre = slot_of + kDecodeWindow;
  int32_t* const wave_tot = pre + kDecodeBatch + 1;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = p.group;
  const int hg = p.head_group;
  const int Hq = p.num_kv_heads * G;
  const int B = p.batch;

  // ---- lengths, rounded up to whole tiles, and their prefix sums: with
  // ranges of whole tiles, every range boundary falls on a tile boundary of
  // its request, so a tile never straddles two pages of a request whose page
  // size is a multiple of KB.  A length above max_seq_len breaks the
  // caller's contract and is clamped, so that no page_table entry past the
  // row's bound is read.  In a mixed batch only the rows with one new token
  // are decode rows (length prefix + 1); the others have none here.
  constexpr int RPT = kDecodeBatch / kThreads;  // requests per thread
  // page_table row indices of the thread's requests, loaded with the
  // lengths: the row of the workgroup's first request is then known without
  // another round trip once the range is found
  int32_t tix[RPT];
  {
    int lens[RPT];
    int run = 0;
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int r = tid * RPT + j;
      int L = 0;
      if (r < B) {
        if (p.mixed_cu)
          L = p.mixed_extend[r] == 1 ? min(p.mixed_prefix[r] + 1, p.max_seq_len) : 0;
        else
          L = min(p.seq_lens[r], p.max_seq_len);
      }
      tix[j] = r < B ? p.table_idx[r] : 0;
      lens[j] = (max(L, 0) + KB - 1) / KB * KB;  // whole tiles
      run += lens[j];
    }
    int incl = run;  // inclusive scan over the wave
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
    for (int x = 0; x < kWaves; ++x) {
      if (x < w) excl += wave_tot[x];
      total += wave_tot[x];
    }
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      pre[tid * RPT + j] = excl;
      excl += lens[j];
    }
    if (tid == 0) pre[kDecodeBatch] = total;
    __syncthreads();
  }
  const int T = pre[B];

  // ---- rows without tokens: their piece map says so (the merge then reads
  // nothing else for them); padding rows (seq_len 0) get zeros and no KV
  // read, while in a mixed batch they are the extend rows, not ours
  for (int r = wg; r < B; r += nwg) {
    if (pre[r + 1] == pre[r]) {
      if (tid == 0) p.ws_map[r] = make_int2(0, 0);
      if (!p.mixed_cu) {
        uint4* o = reinterpret_cast<uint4*>(p.out + (static_cast<int64_t>(r) * Hq + grp * hg * G) * D);
        for (int i = tid; i < hg * G * D / 8; i += kThreads) o[i] = make_uint4(0, 0, 0, 0);
      }
    }
  }

  // ---- this workgroup's token range [a0, b0)
  const int per = (max(kDecodeMinTokens, static_cast<int>((static_cast<int64_t>(T) + nwg - 1) / nwg)) +
                   KB - 1) / KB * KB;
  const int a0 = wg * per;
  if (a0 >= T) return;
  const int b0 = min(T, a0 + per);

  const uint32_t row_bytes = static_cast<uint32_t>(p.num_kv_heads) * D * 2;
  const uint32_t grp_off = static_cast<uint32_t>(grp) * RB;
  const u32x4_t krs = buffer_words(p.k_cache, p.half_bytes);
  const u32x4_t vrs = buffer_words(p.v_cache, p.half_bytes);

  // wave w computes kv head g; lane: head column h (valid below G), key
  // group n (keys 4n .. 4n+3 of a 16-key block)
  const int g = grp * hg + w;
  const bool computes = w < hg;
  const int h = lane & 15;
  const int n = lane >> 4;
  const float c2 = p.scale_log2;
  // per-lane LDS read offsets: K operand (row h of a block, column 4ks + n
  // of the head) and V transpose read (row 4n + j, 8 bytes at channel
  // 16cb + 4q of the head, j = (lane&15)/4, q = lane&3)
  const int kcol0 = w * D / 8 + n;
  const int vj = (lane & 15) >> 2;
  const int vq = lane & 3;

  auto stage = [&](auto kc) __attribute__((always_inline)) -> const uint8_t* {
    constexpr int K = decltype(kc)::value;
    if constexpr (K == 0) return st0;
    else if constexpr (K == 1) return st1;
    else if constexpr (K == 2) return st2;
    else return st3;
  };

  // DMA: wave w issues instructions w*IPW .. w*IPW+IPW-1 of tile t of the
  // window (the first NI/2 fill the K tile, the rest the V tile).  All
  // slots are read before the first DMA goes out: each DMA is a compiler
  // barrier for memory.
  auto issue = [&](int t, const uint8_t* st) __attribute__((always_inline)) {
    uint32_t off[IPW];
#pragma unroll
    for (int k = 0; k < IPW; ++k) {
      const int i = w * IPW + k;
      const bool mat = i >= NI / 2;
      const int o = (i - (mat ? NI / 2 : 0)) * 1024 + 16 * lane;  // byte of the matrix tile
      const int row = o >> LG_RB;
      const int pcol = (o & (RB - 1)) >> 4;
      const int lcol = pcol ^ (SWZ ? (mat ? ((row & 7) << 1) : (row & 15)) : 0);
      off[k] = static_cast<uint32_t>(slot_of[t * KB + row]) * row_bytes + grp_off + lcol * 16;
    }
#pragma unroll
    for (int k = 0; k < IPW; ++k) {
      const int i = w * IPW + k;
      const bool mat = i >= NI / 2;
      dma16(mat ? vrs : krs, st + (mat ? KB * RB : 0) + (i - (mat ? NI / 2 : 0)) * 1024, off[k]);
    }
  };

  // the request holding token a0: the last r with pre[r] <= a0
  const int r0 = [&] {
    int lo = 0, hi = B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pre[mid] <= a0) lo = mid; else hi = mid;
    }
    return lo;
  }();
  // its page_table row, from the thread that loaded it, through LDS (the
  // scan totals are not used past the prologue; the first barrier of the
  // request's first window publishes it)
  if (tid == r0 / RPT) {
    int32_t v = 0;
#pragma unroll
    for (int j = 0; j < RPT; ++j)
      if (j == r0 % RPT) v = tix[j];
    wave_tot[0] = v;
  }
  for (int r = r0; r < B && pre[r] < b0; ++r) {
    const int first = pre[r] / per;  // the workgroups holding request r
    const int pieces = (pre[r + 1] - 1) / per - first + 1;
    // this piece: tokens [sa, sb) of request r (both whole tiles; tokens past
    // the request's real length are masked)
    const int L = p.mixed_cu ? min(p.mixed_prefix[r] + 1, p.max_seq_len) : min(p.seq_lens[r], p.max_seq_len);
    const int sa = max(a0, pre[r]) - pre[r];
    const int sb = min(min(b0, pre[r + 1]) - pre[r], L);
    if (sb <= sa) continue;
    const int64_t io_row = p.mixed_cu ? p.mixed_cu[r] : r;
    // the merge finds a split request's pieces here
    if (wg == first && tid == 0) p.ws_map[r] = make_int2(first + r, pieces);

    bf16x8_t qop[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) qop[ks][e] = static_cast<__bf16>(0.f);

    float m_run = -INFINITY;
    float l_run = 0.f;
    f32x4_t o[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) o[cb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

    const int32_t row_later = r == r0 ? 0 : p.table_idx[r];
    const int32_t* pt = nullptr;
    for (int w0 = sa; w0 < sb; w0 += kDecodeWindow) {
      const int ntok = min(kDecodeWindow, sb - w0);
      const int ntiles = (ntok + KB - 1) / KB;
      // slots of the window's tokens (tokens past its end repeat the last
      // one: valid rows, masked below).  Every wave is done with the slot
      // table and the stages of the previous window.
      __syncthreads();
      if (w0 == sa)
        pt = p.page_table + static_cast<int64_t>(r == r0 ? wave_tot[0] : row_later) * p.pt_stride;
      // the request's q rows, in flight together with the window's page
      // entries
      if (w0 == sa && computes && h < G) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          qop[ks] = *reinterpret_cast<const bf16x8_t*>(p.q + io_row * p.q_stride +
                                                       static_cast<int64_t>(g * G + h) * D + ks * 32 + 8 * n);
      }
      {
        const int ps = p.page_size;
        for (int i = tid; i < ntiles * KB; i += kThreads) {
          const int tok = w0 + min(i, ntok - 1);
          const int pg = tok / ps;
          const int sl = pt[pg] * ps + (tok - pg * ps);
          slot_of[i] = min(max(sl, 0), p.num_slots - 1);
        }
      }
      __syncthreads();
      // the q operands are redefined by an empty asm once their loads are
      // done (the barrier waited for them): the waitcnt pass would otherwise
      // keep them pending and make the first MFMA of every tile wait for the
      // DMA in flight
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qop[ks]));

      auto compute = [&](int t, const uint8_t* kt) __attribute__((always_inline)) {
        const uint8_t* vt = kt + KB * RB;
        const int nvalid = ntok - t * KB;  // keys of this tile inside the window
        // blocks one after another (unrolled, the blocks' operands would not
        // fit the 128 registers that two workgroups per CU leave a lane)
#pragma unroll 1
        for (int b = 0; b < NB; ++b) {
          // ---- S^T = K Q^T for one block of keys
          const bool krow_ok = h < BK;
          const int krow = b * 16 + (krow_ok ? h : 0);
          const int kx = SWZ ? (krow & 15) : 0;
          f32x4_t sc = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(kt + krow * RB + ((kcol0 + 4 * ks) ^ kx) * 16);
            if (!krow_ok) {
#pragma unroll
              for (int e = 0; e < 8; ++e) ka[e] = static_cast<__bf16>(0.f);
            }
            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qop[ks], sc, 0, 0, 0);
          }
          // keys b*16 + 4n + e of head h; past the block's keys or the window: masked
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * n + e >= BK || b * 16 + 4 * n + e >= nvalid) sc[e] = -INFINITY;
          // ---- online softmax, log2 domain, on x = s * scale * log2(e)
          float pr[4];
          float lsum = 0.f;
          auto probabilities = [&](float mref) __attribute__((always_inline)) {
            lsum = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              pr[e] = fast_exp2(__builtin_fmaf(sc[e], c2, -mref));
              lsum += pr[e];
            }
          };
          bool slow = m_run == -INFINITY;
          if (__builtin_amdgcn_ballot_w64(slow) == 0) {
            probabilities(m_run);
            slow = !(lsum <= kSumLimit);  // also catches inf
          }
          if (__builtin_amdgcn_ballot_w64(slow) != 0) {
            // block maximum of head h over its 4 lane groups
            float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
            mx = fmaxf(mx, shfl_xor_f(mx, 16));
            mx = xor32_max(mx) * c2;  // scale > 0: the maximum commutes with it
            const bool move = mx > m_run + kMaxSlack;
            const float mnew = move ? mx : m_run;
            const float alpha = fast_exp2(m_run - mnew);
            probabilities(mnew);
            m_run = mnew;
            if (__builtin_amdgcn_ballot_w64(move) != 0) {
              l_run *= alpha;
#pragma unroll
              for (int cb = 0; cb < CB; ++cb) o[cb] *= alpha;
            }
          }
          // ---- P as a bf16 value plus its bf16 remainder
          const uint32_t h01 = pack_bf16(pr[0], pr[1]);
          const uint32_t h23 = pack_bf16(pr[2], pr[3]);
          const uint32_t l01 = pack_bf16(pr[0] - __uint_as_float(h01 << 16),
                                         pr[1] - __uint_as_float(h01 & 0xFFFF0000u));
          const uint32_t l23 = pack_bf16(pr[2] - __uint_as_float(h23 << 16),
                                         pr[3] - __uint_as_float(h23 & 0xFFFF0000u));
          constexpr uint32_t kOnes = 0x3F803F80u;  // bf16 (1, 1)
          l_run = dot2_bf16(h01, kOnes,
                            dot2_bf16(h23, kOnes, dot2_bf16(l01, kOnes, dot2_bf16(l23, kOnes, l_run))));
          const bf16x8_t pop = __builtin_bit_cast(bf16x8_t, make_uint4(h01, h23, l01, l23));
          // ---- O^T += V^T P^T: the lane's 4 keys of channel 16cb + h, twice
          const bool vrow_ok = 4 * n < BK;
          const int vrow = b * 16 + (vrow_ok ? 4 * n + vj : vj);
          const int vx = SWZ ? ((vrow & 7) << 1) : 0;
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            i16x4_t v4 = lds_read_tr16(vt + vrow * RB + (((w * D / 8 + 2 * cb) ^ vx) + (vq >> 1)) * 16 +
                                       8 * (vq & 1));
            if (!vrow_ok) v4 = (i16x4_t){0, 0, 0, 0};
            const bf16x8_t va =
                __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v4, v4, 0, 1, 2, 3, 0, 1, 2, 3));
            o[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pop, o[cb], 0, 0, 0);
          }
        }
      };

      // S stages: tiles t+1 .. t+S-1 land while tile t is computed
#pragma unroll
      for (int t = 0; t < S - 1; ++t)
        if (t < ntiles)
          issue(t, t == 0 ? st0 : t == 1 ? stage(std::integral_constant<int, 1>{})
                                         : stage(std::integral_constant<int, 2 % S>{}));
      auto step = [&](int t, auto kc) __attribute__((always_inline)) {
        constexpr int K = decltype(kc)::value;
        // tile t has landed for every wave (S-2 younger tiles may stay in
        // flight), and every wave is done with tile t-1, whose stage tile
        // t+S-1 now fills
        if (t + S - 2 < ntiles) {
          if constexpr (S == 2) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
          else asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"((S - 2) * IPW) : "memory");
        } else {
          asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        }
        if (t + S - 1 < ntiles) issue(t + S - 1, stage(std::integral_constant<int, (K + S - 1) % S>{}));
        if (computes) compute(t, stage(kc));
      };
      for (int t = 0; t < ntiles; t += S) {
        step(t, std::integral_constant<int, 0>{});
        if (t + 1 < ntiles) step(t + 1, std::integral_constant<int, 1>{});
        if constexpr (S > 2)
          if (t + 2 < ntiles) step(t + 2, std::integral_constant<int, 2 % S>{});
        if constexpr (S > 3)
          if (t + 3 < ntiles) step(t + 3, std::integral_constant<int, 3 % S>{});
      }
    }

    // ---- the piece's result: the head's sum over its 4 lane groups
    float l_tot = l_run + shfl_xor_f(l_run, 16);
    l_tot = xor32_sum(l_tot);
    if (pieces == 1) {
      if (computes && h < G) {
        const float inv = 1.f / l_tot;
        uint16_t* op = p.out + (io_row * Hq + g * G + h) * D + 4 * n;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          uint2 wv;
          wv.x = pack_bf16(o[cb][0] * inv, o[cb][1] * inv);
          wv.y = pack_bf16(o[cb][2] * inv, o[cb][3] * inv);
          *reinterpret_cast<uint2*>(op + cb * 16) = wv;
        }
      }
      continue;
    }
    if (computes && h < G) {
      const int64_t u = static_cast<int64_t>(wg + r) * Hq + g * G + h;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        *reinterpret_cast<f32x4_t*>(p.ws_o + u * D + cb * 16 + 4 * n) = o[cb];
      if (n == 0) *reinterpret_cast<float2*>(p.ws_ml + u * 2) = make_float2(m_run, l_tot);
    }
  }
}

}  // namespace decode_impl
}  // namespace msgl
