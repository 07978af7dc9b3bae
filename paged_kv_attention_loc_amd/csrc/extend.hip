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
//   * K/V tiles are double-buffered in LDS, one barrier per tile.  The
//     rows go from HBM straight into LDS (buffer_load ... lds, 16 bytes a
//     lane, each wave instruction filling 1 KiB of consecutive LDS), issued
//     by all waves one tile ahead, with no register staging; the page-table
//     entries of the tile after are in flight meanwhile.  Rows are read at
//     32-bit offsets inside the (K or V, layer) sub-tensor, whose range
//     check also absorbs a wild page id;
//   * each wave computes S^T = K Q^T, so a lane holds one query column and
//     16 keys per 32-key block: the row maximum and sum need one exchange
//     with the lane 32 apart (v_permlane32_swap);
//   * K and V are both staged row-major, unpadded, with the 16-byte
//     columns of each row XOR-permuted: the DMA fetches, for each LDS
//     slot, the column that the permutation puts there.  K reads (one
//     16-byte operand per lane and k-step) then hit distinct banks within
//     every 16-lane group, and so do the V reads: the A operand of O^T =
//     V^T P^T is two ds_read_b64_tr_b16 (the LDS transpose read of CDNA4:
//     in each 16-lane group, lane i receives element i%4 of the 8-byte
//     pieces addressed by lanes 4j + i/4, j = 0..3), which turns four key
//     rows into four keys of one channel per lane, in the order in which
//     the S^T accumulator registers hold the keys -- so P^T feeds the
//     second MFMA straight from registers.  Per-lane read addresses are
//     computed once; the tile, stage and block parts are immediates;
//   * the MFMA takes q exactly as stored (bf16 in, fp32 accumulate): the
//     scale*log2(e) factor is applied to the fp32 scores, fused with the
//     subtraction of the running maximum, so a probability is one fma and
//     one v_exp_f32 of the accumulator;
//   * P.V runs on the fp16 MFMA (v_mfma_f32_32x32x16_f16): probabilities
//     are rounded to fp16 (11 significant bits, against bf16's 8), and each
//     wave turns the V rows it loaded into fp16 in place, right after its
//     own DMA has landed and before the tile's barrier.  bf16 -> fp16 is
//     exact for |V| in [2^-14, 65504]; below, V is rounded on fp16's
//     subnormal grid (absolute error under 2^-25).  With bf16
//     probabilities, peaked softmaxes (logits of tens) leave a few outputs
//     per million beyond 1e-2 of exact attention; with fp16 none;
//   * the running maximum only moves when a row's new maximum exceeds it by
//     more than 2^8 in exp2 terms, so the O rescale is rare; masking runs
//     only on tiles that cross a row's causal limit;
//   * a call whose row tiles cannot give every CU a workgroup (a short
//     prefill, or few kv heads) can split each tile's keys into shares,
//     one workgroup each (z = tile * shares + share, heaviest tiles
//     first); the shares write fp32 partial outputs with their softmax
//     statistics and a second kernel combines them with a log-sum-exp
//     merge, as the decode does for its token ranges.
#include "extend_block.h"

namespace msgl {

using namespace extend_impl;

template <int D, bool POW2, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 2) void extend_kernel(ExtendParams p,
                                                               const int32_t* __restrict__ page_table) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[lds_bytes<D, WAVES>()];
  const int z = static_cast<int>(blockIdx.z);
  extend_block<D, POW2, WAVES>(p, page_table, blockIdx.x, blockIdx.y,
                               p.num_mtiles - 1 - z / p.num_splits, lds, z % p.num_splits);
}

// out = sum_s w_s o_s / sum_s w_s, w_s = l_s 2^(m_s - M), over the key
// shares s of one (token, q head), with M the largest share maximum and o_s
// already divided by l_s.  Thread: one float4 column of one (token, q head).
template <int D>
__global__ __launch_bounds__(256) void extend_merge_kernel(ExtendParams p, int64_t pairs) {
  constexpr int QPH = D / 4;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t pair = i / QPH;
  if (pair >= pairs) return;
  const int c4 = static_cast<int>(i - pair * QPH);
  const int S = p.num_splits;
  const float2* ml = reinterpret_cast<const float2*>(p.ws_ml) + pair * S;
  float mx = -INFINITY;
  for (int s = 0; s < S; ++s) mx = fmaxf(mx, ml[s].x);
  float den = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < S; ++s) {
    const float2 v = ml[s];
    const float wgt = v.y > 0.f ? v.y * fast_exp2(v.x - mx) : 0.f;
    const float4 o = reinterpret_cast<const float4*>(p.ws_o + (pair * S + s) * D)[c4];
    den += wgt;
    acc.x += wgt * o.x;
    acc.y += wgt * o.y;
    acc.z += wgt * o.z;
    acc.w += wgt * o.w;
  }
  const float inv = 1.f / den;
  uint2 wv;
  wv.x = pack_bf16(acc.x * inv, acc.y * inv);
  wv.y = pack_bf16(acc.z * inv, acc.w * inv);
  *reinterpret_cast<uint2*>(p.out + pair * D + 4 * c4) = wv;
}


namespace {

template <int D, int WAVES>
void launch_extend_t(const ExtendParams& p, int batch, hipStream_t stream) {
  const dim3 grid(p.num_kv_heads, batch, p.num_mtiles * p.num_splits);
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

hipError_t launch_extend_merge(const ExtendParams& p, int head_dim, int64_t tokens,
                               hipStream_t stream) {
  const int64_t pairs = tokens * p.num_kv_heads * p.group;
  const int64_t threads = pairs * (head_dim / 4);
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
  if (head_dim == 128)
    hipLaunchKernelGGL((extend_merge_kernel<128>), grid, dim3(256), 0, stream, p, pairs);
  else
    hipLaunchKernelGGL((extend_merge_kernel<64>), grid, dim3(256), 0, stream, p, pairs);
  return hipGetLastError();
}

}  // namespace msgl
