// Split-KV paged decode attention and the log-sum-exp merge of its partials.
//
// Decode attends one new query token per request over all of its KV, read
// through the request's page_table row ("Code Notes: mini-sglang", Engine
// Layer table rows BaseAttnBackend / GraphRunner; Scheduler Layer table row
// TableManager).  The work is HBM-bound: every K/V byte is read once and
// used for G = q_heads / kv_heads query heads, so the kernel is built to
// keep many waves -- and so many loads -- in flight per CU, with no matrix
// cores involved.
//
// One wave64 workgroup handles (request, kv head, chunk of `chunk` tokens)
// in tiles of 32 tokens.  A wave needs about 9-11 KiB of LDS and few
// registers, so a CU holds 16 of them and their loads overlap each other's
// arithmetic; chunks are short (384 tokens by default) so that many
// independent waves are in flight while the split partials stay a few
// percent of the KV bytes.
//   * the K/V loads carry the nontemporal hint: every byte is read once;
//   * addressing: one vector load per tile fetches the tile's page ids
//     (lane t: token t), one tile ahead; each token's row byte offset is
//     then moved into an SGPR (v_readlane) and every K/V load is a buffer
//     load of that whole token row (4 bytes per lane, one row per
//     instruction).  No lane holds a 64-bit address, and an offset past
//     the pool reads zeros instead of faulting;
//   * q.K: two neighbouring lanes own one token (half of the channels
//     each).  K rows pass through LDS with one 16-byte piece of padding per
//     row (conflict-free reads, addresses base + immediate), q is broadcast
//     from LDS one head at a time, v_dot2_f32_bf16 does the products and one
//     DPP add joins the halves;
//   * softmax statistics are kept per head in the log2 domain (scale folded
//     into the exponent); the tile maximum comes from DPP row reductions;
//   * p.V: each lane owns two channels of every token and keeps its V words
//     in registers; two tokens' values are paired with v_perm and weighted
//     by the matching bf16 pair of probabilities (an LDS broadcast) in one
//     v_dot2_f32_bf16: two accumulators per head;
//   * a request with a single chunk writes its bf16 output directly; longer
//     ones write fp32 partials (unnormalised o, max, sum) that the merge
//     kernel combines.
#include "common.h"

namespace msgl {

namespace {

template <int D>
struct DecodeShape {
  static constexpr int TILE = 32;     // tokens per tile
  static constexpr int LPT = D / 8;   // 16-byte pieces per token row
  static constexpr int HPC = LPT / 2; // pieces per q.K half-row
  static constexpr int CPL = D / 2;   // 4-byte words per token row
  // LDS row pitch of K in words: one 16-byte piece of padding per row
  static constexpr int KROW = CPL + 4;
};

// Waves per SIMD the register allocation must leave room for: occupancy is
// what hides the HBM latency here.
template <int GM>
struct DecodeOccupancy {
  static constexpr int value = GM <= 8 ? 4 : 2;
};

// Cache policy of the K/V loads: nontemporal (the nt bit of the buffer
// load).  Each K/V byte is read exactly once per launch, so the stream is
// marked as such and does not displace what the caches hold for the
// kernels around it; measured, the decode itself also runs faster so.
constexpr int kStream = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  // dword 3 = 0x00020000: 32-bit data format, raw (unswizzled) addressing
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

}  // namespace

template <int D, int GM>
__global__ __launch_bounds__(64, DecodeOccupancy<GM>::value) void decode_split_kernel(
    DecodeParams p, const int32_t* __restrict__ page_table) {
  using S = DecodeShape<D>;
  constexpr int TILE = S::TILE, LPT = S::LPT, HPC = S::HPC, CPL = S::CPL, KROW = S::KROW;

  const int s = blockIdx.x;
  const int g = blockIdx.y;
  const int r = blockIdx.z;
  const int lane = threadIdx.x;
  const int G = p.group;
  const int Hq = p.num_kv_heads * G;
  // a length above max_seq_len breaks the caller's contract; clamp it so
  // that no page_table entry past the row's bound is read.  In a mixed
  // batch only the rows with one new token are decoded here, and their
  // q / out row is the request's first row of the batch.
  int L;
  int64_t io_row = r;
  if (p.mixed_cu) {
    if (p.mixed_extend[r] != 1) return;
    L = min(p.mixed_prefix[r] + 1, p.max_seq_len);
    io_row = p.mixed_cu[r];
  } else {
    L = min(p.seq_lens[r], p.max_seq_len);
  }

  if (L <= 0) {  // padding row: zeros, no KV read
    if (s == 0) {
      uint16_t* o = p.out + (io_row * Hq + g * G) * D;
      for (int i = lane; i < G * LPT; i += 64) reinterpret_cast<uint4*>(o)[i] = make_uint4(0, 0, 0, 0);
    }
    return;
  }
  const int nch = (L + p.chunk - 1) / p.chunk;
  if (s >= nch) return;

  __shared__ uint4 k_lds[TILE * KROW / 4];
  __shared__ uint4 q_lds[GM * LPT];
  __shared__ uint32_t p_lds[(TILE / 2) * GM];

  // heads G .. GM-1 (a group size that is not a power of two) run on zero
  // queries and are never written
  const uint16_t* qrow = p.q + io_row * p.q_stride + static_cast<int64_t>(g) * G * D;
  for (int i = lane; i < GM * LPT; i += 64)
    q_lds[i] = (i < G * LPT) ? reinterpret_cast<const uint4*>(qrow)[i] : make_uint4(0, 0, 0, 0);

  const int32_t* pt = page_table + static_cast<int64_t>(p.table_idx[r]) * p.pt_stride;
  const int ps = p.page_size;
  const int sh = p.page_shift;
  const uint32_t row_bytes = static_cast<uint32_t>(p.num_kv_heads) * D * 2;
  const uint32_t head_off = static_cast<uint32_t>(g) * D * 2;
  const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(p.k_cache + static_cast<int64_t>(g) * D, p.half_bytes - head_off);
  const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(p.v_cache + static_cast<int64_t>(g) * D, p.half_bytes - head_off);

  const int t_begin = s * p.chunk;
  const int t_end = min(L, t_begin + p.chunk);
  const int cw = lane % CPL;  // this lane's word of a token row (channels 2cw, 2cw+1)
  const int qt = lane >> 1;   // q.K layout: token of the tile
  const int hf = lane & 1;    //              half of the channels

  float m_run[GM], l_run[GM], acc[GM][2];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
    acc[h][0] = acc[h][1] = 0.f;
  }
  __syncthreads();

  uint16_t* p16 = reinterpret_cast<uint16_t*>(p_lds);
  uint32_t* k_words = reinterpret_cast<uint32_t*>(k_lds);

  // lane t (mod TILE) returns the byte offset of token t0 + t's row in the
  // K/V sub-tensor; past the end, the last valid token again (in-bounds
  // data, weighted by an exact zero below)
  auto tile_offsets = [&](int t0) -> uint32_t {
    const int n = min(TILE, t_end - t0);
    const int tok = t0 + min(lane & (TILE - 1), n - 1);
    int slot;
    if (sh >= 0) {
      slot = (pt[tok >> sh] << sh) + (tok & (ps - 1));
    } else {
      const int pg = tok / ps;
      slot = pt[pg] * ps + (tok - pg * ps);
    }
    return static_cast<uint32_t>(min(max(slot, 0), p.num_slots - 1)) * row_bytes;
  };
  uint32_t off_cur = tile_offsets(t_begin);

  for (int t0 = t_begin; t0 < t_end; t0 += TILE) {
    const int n = min(TILE, t_end - t0);
    // page ids of the next tile go out now, so their latency hides behind
    // this tile
    const uint32_t off_next = (t0 + TILE < t_end) ? tile_offsets(t0 + TILE) : 0u;
    // one row load per token, at the token's wave-uniform byte offset
    uint32_t kw[TILE], vw[TILE];
#pragma unroll
    for (int t = 0; t < TILE; ++t)
      kw[t] = __builtin_amdgcn_raw_buffer_load_b32(krs, cw * 4, __builtin_amdgcn_readlane(off_cur, t), kStream);
#pragma unroll
    for (int t = 0; t < TILE; ++t)
      vw[t] = __builtin_amdgcn_raw_buffer_load_b32(vrs, cw * 4, __builtin_amdgcn_readlane(off_cur, t), kStream);
    if (lane < CPL) {
#pragma unroll
      for (int t = 0; t < TILE; ++t) k_words[t * KROW + cw] = kw[t];
    }
    __syncthreads();

    // q.K: lanes 2t and 2t+1 hold token t's two halves.  Each head's q
    // broadcasts are issued only once the previous head's sum exists (an
    // empty asm ties the LDS offset to it): the scheduler would otherwise
    // hoist every head's q reads at once and spill them.
    uint4 kk[HPC];
#pragma unroll
    for (int cc = 0; cc < HPC; ++cc) kk[cc] = k_lds[qt * (KROW / 4) + hf * HPC + cc];
    float sc[GM];
    int qoff = hf * HPC;
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h > 0) asm volatile("" : "+v"(qoff) : "v"(sc[h - 1]));
      else asm volatile("" : "+v"(qoff));
      float a = 0.f;
#pragma unroll
      for (int cc = 0; cc < HPC; ++cc) {
        const uint4 qq = q_lds[qoff + h * LPT + cc];
        a = dot2_bf16(kk[cc].x, qq.x, a);
        a = dot2_bf16(kk[cc].y, qq.y, a);
        a = dot2_bf16(kk[cc].z, qq.z, a);
        a = dot2_bf16(kk[cc].w, qq.w, a);
      }
      sc[h] = a;
    }

    const bool valid = qt < n;
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      const float full = sc[h] + dpp_mov<kDppXor1>(sc[h]);
      const float x = valid ? full * p.scale_log2 : -INFINITY;
      const float mnew = fmaxf(m_run[h], wave_max(x));
      const float alpha = fast_exp2(m_run[h] - mnew);
      const uint16_t pb = f32_to_bf16(fast_exp2(x - mnew));
      // both lanes of a token hold the same p: count it once, store it
      // from both (same value)
      l_run[h] = l_run[h] * alpha + (hf ? 0.f : bf16_to_f32(pb));
      m_run[h] = mnew;
      acc[h][0] *= alpha;
      acc[h][1] *= alpha;
      p16[((qt >> 1) * GM + h) * 2 + (qt & 1)] = pb;
    }
    __syncthreads();

    // p.V on token pairs (2j, 2j+1)
#pragma unroll
    for (int j = 0; j < TILE / 2; ++j) {
      const uint32_t lo = pair_lo(vw[2 * j], vw[2 * j + 1]);
      const uint32_t hi = pair_hi(vw[2 * j], vw[2 * j + 1]);
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        const uint32_t pp = p_lds[j * GM + h];
        acc[h][0] = dot2_bf16(lo, pp, acc[h][0]);
        acc[h][1] = dot2_bf16(hi, pp, acc[h][1]);
      }
    }
    __syncthreads();  // k_lds / p_lds are rewritten by the next tile
    off_cur = off_next;
  }

  float l_tot[GM];
#pragma unroll
  for (int h = 0; h < GM; ++h) l_tot[h] = wave_sum(l_run[h]);
  if (nch == 1) {
    if (lane < CPL) {
      uint16_t* o = p.out + (io_row * Hq + g * G) * D + 2 * cw;
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        if (h < G) {
          const float inv = 1.f / l_tot[h];
          *reinterpret_cast<uint32_t*>(o + h * D) = pack_bf16(acc[h][0] * inv, acc[h][1] * inv);
        }
      }
    }
    return;
  }
  const int64_t base = (static_cast<int64_t>(r) * p.max_chunks + s) * (Hq + 1) + g * G;
  if (lane < CPL) {
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h < G)
        *reinterpret_cast<float2*>(p.ws_o + (base + h) * D + 2 * cw) = make_float2(acc[h][0], acc[h][1]);
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

// out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s over the chunks s of
// one (request, q head), with M the largest chunk maximum.  One wave per
// (request, q head): lane l owns float4 piece l % (D/4) of the head and the
// chunks s = l / (D/4) (mod 64 / (D/4)); the lanes that share a piece are
// joined by exchanges 32 (and 16) lanes apart.
constexpr int kMergeThreads = 64;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeParams p) {
  constexpr int QPH = D / 4;          // float4 pieces per head
  constexpr int NH = 64 / QPH;        // lanes per piece (chunk phases)
  const int h = blockIdx.x;           // q head
  const int r = blockIdx.y;
  const int lane = threadIdx.x;
  int L;
  int64_t io_row = r;
  if (p.mixed_cu) {
    if (p.mixed_extend[r] != 1) return;
    L = min(p.mixed_prefix[r] + 1, p.max_seq_len);
    io_row = p.mixed_cu[r];
  } else {
    L = min(p.seq_lens[r], p.max_seq_len);
  }
  if (L <= 0) return;
  const int nch = (L + p.chunk - 1) / p.chunk;
  if (nch <= 1) return;
  const int Hq = p.num_kv_heads * p.group;
  // chunk s at base + s*(Hq+1): one unit of padding per chunk keeps the
  // chunk stride off powers of two
  const int64_t base = static_cast<int64_t>(r) * p.max_chunks * (Hq + 1) + h;
  const int64_t row = Hq + 1;
  const int cq = lane % QPH;
  const int ph = lane / QPH;

  float mx = -INFINITY;
  for (int s = lane; s < nch; s += 64) mx = fmaxf(mx, p.ws_ml[(base + s * row) * 2]);
  mx = wave_max(mx);

  float den = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int s = ph; s < nch; s += NH) {
    const int64_t u = base + s * row;
    const float2 ml = *reinterpret_cast<const float2*>(p.ws_ml + u * 2);
    const float w = fast_exp2(ml.x - mx);
    den += w * ml.y;
    const float4 o = reinterpret_cast<const float4*>(p.ws_o + u * D)[cq];
    acc.x += w * o.x;
    acc.y += w * o.y;
    acc.z += w * o.z;
    acc.w += w * o.w;
  }
  // join the NH lanes of each piece (their den values differ per phase)
#pragma unroll
  for (int off = 32; off >= QPH; off >>= 1) {
    den += shfl_xor_f(den, off);
    acc.x += shfl_xor_f(acc.x, off);
    acc.y += shfl_xor_f(acc.y, off);
    acc.z += shfl_xor_f(acc.z, off);
    acc.w += shfl_xor_f(acc.w, off);
  }
  if (lane < QPH) {
    const float inv = 1.f / den;
    uint2 wv;
    wv.x = pack_bf16(acc.x * inv, acc.y * inv);
    wv.y = pack_bf16(acc.z * inv, acc.w * inv);
    *reinterpret_cast<uint2*>(p.out + (io_row * Hq + h) * D + 4 * lane) = wv;
  }
}

template <int D, int GM>
static void launch_decode_t(const DecodeParams& p, int batch, hipStream_t stream) {
  // an odd grid width: with a multiple of 8 chunk columns every chunk
  // index lands on the same XCD in every row (workgroups are dealt to the 8
  // XCDs round-robin), which measured up to 1.6x slower
  const dim3 grid(p.max_chunks | 1, p.num_kv_heads, batch);
  hipLaunchKernelGGL((decode_split_kernel<D, GM>), grid, dim3(64), 0, stream, p, p.page_table);
  if (p.max_chunks > 1) {
    const dim3 mgrid(p.num_kv_heads * p.group, batch);
    hipLaunchKernelGGL((decode_merge_kernel<D>), mgrid, dim3(kMergeThreads), 0, stream, p);
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
