// Paged decode attention over whole token rows and balanced token ranges;
// a second, small kernel merges the requests that several ranges split.
//
// Decode attends one new query token per request over all of its KV, read
// through the request's page_table row ("Code Notes: mini-sglang", Engine
// Layer table rows BaseAttnBackend / GraphRunner; Scheduler Layer table row
// TableManager).  Every K/V byte is read once, so the kernel is built around
// the HBM stream:
//   * the batch's tokens, requests laid end to end, are split into equal
//     ranges, one per workgroup (kDecodeGrid of them per group of kv heads):
//     every workgroup moves the same number of bytes whatever the length
//     mix, and no workgroup is launched for nothing.  Each workgroup takes
//     the token prefix sums of the batch into LDS and walks the requests its
//     range touches;
//   * one workgroup of 8 waves streams the group's part of each token row --
//     a token's row in the pool holds every kv head (BaseKVCachePool row of
//     the same table: (..., kv_heads, head_dim) is innermost), so that part
//     is one contiguous run of up to 2 KiB.  16 bytes a lane, 1 KiB of
//     consecutive LDS per wave instruction (buffer_load ... lds), spread over
//     all 8 waves, a tile ahead of the arithmetic.  The DMA is issued as
//     assembly: the compiler would otherwise drain it before every LDS read,
//     because it cannot tell which stage those reads touch;
//   * tiles hold KB tokens (8 to 64: 16 KiB of K and 16 KiB of V), S stages,
//     one barrier per tile; the slots of up to kDecodeWindow tokens are
//     computed at a time into LDS;
//   * wave w computes kv head w of the group on the matrix cores
//     (v_mfma_f32_16x16x32_bf16): S^T = K Q^T with the G <= 16 query heads
//     as the 16 columns, then O^T = V^T P^T.  Each lane holds 4 keys of one
//     head per 16-key block, so the 32 k-slots of the P.V product carry 16
//     keys twice: once with the bf16-rounded probability and once with the
//     bf16 remainder p - bf16(p), against the same V (one ds_read_b64_tr_b16
//     transpose read used twice).  The product thus weights V with ~16-bit
//     probabilities in one MFMA, and V enters exactly as stored;
//   * the online softmax is in the log2 domain on fp32 scores (scale folded
//     into one fma); the running maximum moves only when a score exceeds it
//     by more than 2^8, so the rescale of O is rare;
//   * a request inside one range writes its bf16 output directly.  A
//     request spread over several ranges writes one fp32 partial per range
//     (piece i + r of range i and request r: both indices only grow along
//     the token axis, so pieces never collide), and a second kernel merges
//     them with a log-sum-exp combine, one wave per (request, q head).
//     Merging inside the first kernel -- the last range of a request to
//     finish, found with an atomic counter -- measured ~25 us slower on the
//     Llama-3-8B-geometry batch: the agent-scope release that publishes the
//     partials writes back the whole L2 of an XCD, once per range.
#include "decode_block.h"

namespace msgl {

using namespace decode_impl;

template <int D, int RB, int S, int STB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void decode_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[lds_bytes<S, STB>()];
  decode_block<D, RB, S, STB>(p, blockIdx.x, gridDim.x, blockIdx.y, smem);
}


// out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i over the pieces i of
// one (request, q head) that the decode kernel split, with M the largest
// piece maximum.  One wave per (request, q head): lane l owns float4 piece
// l % (D/4) of the head and the pieces i = l / (D/4) (mod 64 / (D/4)); the
// lanes that share a float4 are joined by exchanges 32 (and 16) lanes apart.
// Every request of the launch has a piece map entry (no pieces when it has
// no tokens), and the first kMergeRegs pieces of a lane are loaded together,
// statistics and partial outputs, before the maximum is known: two
// dependent rounds of global loads instead of four, for up to
// kMergeRegs * 64 / (D/4) pieces (32 at head_dim 128: a 512-token request
// split into 16-token ranges).  Sixteen against eight took a batch of 8
// such requests from 24 to 22 us per decode call.
constexpr int kMergeRegs = 16;

template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeParams p) {
  constexpr int QPH = D / 4;    // float4 pieces per head
  constexpr int NPH = 64 / QPH; // lanes per float4 (piece phases)
  const int head = blockIdx.x;
  const int r = blockIdx.y;
  const int lane = threadIdx.x;
  const int2 map = p.ws_map[r];
  const int pieces = map.y;
  if (pieces <= 1) return;  // no tokens, or written by the decode kernel itself
  const int Hq = p.num_kv_heads * p.group;
  const int64_t u0 = static_cast<int64_t>(map.x) * Hq + head;  // piece i at u0 + i*Hq
  const int c4 = lane % QPH;
  const int ph = lane / QPH;
  float2 ml[kMergeRegs];
  float4 ov[kMergeRegs];
#pragma unroll
  for (int k = 0; k < kMergeRegs; ++k) {
    const int i = ph + NPH * k;
    ml[k] = make_float2(-INFINITY, 0.f);
    ov[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < pieces) {
      const int64_t u = u0 + static_cast<int64_t>(i) * Hq;
      ml[k] = *reinterpret_cast<const float2*>(p.ws_ml + u * 2);
      ov[k] = reinterpret_cast<const float4*>(p.ws_o + u * D)[c4];
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < kMergeRegs; ++k) mx = fmaxf(mx, ml[k].x);
  for (int i = ph + NPH * kMergeRegs; i < pieces; i += NPH)
    mx = fmaxf(mx, p.ws_ml[(u0 + static_cast<int64_t>(i) * Hq) * 2]);
#pragma unroll
  for (int off = 32; off >= QPH; off >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, off));
  float den = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int k = 0; k < kMergeRegs; ++k) {
    const float wgt = fast_exp2(ml[k].x - mx);  // 0 for the pieces a lane does not have
    den += wgt * ml[k].y;
    acc.x += wgt * ov[k].x;
    acc.y += wgt * ov[k].y;
    acc.z += wgt * ov[k].z;
    acc.w += wgt * ov[k].w;
  }
#pragma unroll 4
  for (int i = ph + NPH * kMergeRegs; i < pieces; i += NPH) {
    const int64_t u = u0 + static_cast<int64_t>(i) * Hq;
    const float2 m2 = *reinterpret_cast<const float2*>(p.ws_ml + u * 2);
    const float wgt = fast_exp2(m2.x - mx);
    den += wgt * m2.y;
    const float4 v = reinterpret_cast<const float4*>(p.ws_o + u * D)[c4];
    acc.x += wgt * v.x;
    acc.y += wgt * v.y;
    acc.z += wgt * v.z;
    acc.w += wgt * v.w;
  }
#pragma unroll
  for (int off = 32; off >= QPH; off >>= 1) {
    den += shfl_xor_f(den, off);
    acc.x += shfl_xor_f(acc.x, off);
    acc.y += shfl_xor_f(acc.y, off);
    acc.z += shfl_xor_f(acc.z, off);
    acc.w += shfl_xor_f(acc.w, off);
  }
  if (lane < QPH) {
    const int64_t io_row = p.mixed_cu ? p.mixed_cu[r] : r;
    const float inv = 1.f / den;
    uint2 wv;
    wv.x = pack_bf16(acc.x * inv, acc.y * inv);
    wv.y = pack_bf16(acc.z * inv, acc.w * inv);
    *reinterpret_cast<uint2*>(p.out + (io_row * Hq + head) * D + 4 * lane) = wv;
  }
}

namespace {

// The head group's kernel: stages of decode_stage_bytes, two of 32 KiB or
// four of 16 KiB (the same LDS).
template <int D, int RB>
void launch_decode_rb(const DecodeParams& p, hipStream_t stream) {
  constexpr int STB = decode_stage_bytes<D, RB>();
  constexpr int S = STB == kStageBytes ? 2 : 4;
  const dim3 grid(kDecodeGrid, p.num_kv_heads / p.head_group);
  hipLaunchKernelGGL((decode_kernel<D, RB, S, STB>), grid, dim3(kThreads), 0, stream, p);
}

template <int D>
void launch_decode_d(const DecodeParams& p, hipStream_t stream) {
  switch (p.head_group) {
    case 8:
      launch_decode_rb<D, 8 * D * 2>(p, stream);
      break;
    case 4:
      launch_decode_rb<D, 4 * D * 2>(p, stream);
      break;
    case 2:
      launch_decode_rb<D, 2 * D * 2>(p, stream);
      break;
    default:
      launch_decode_rb<D, D * 2>(p, stream);
      break;
  }
}

}  // namespace

hipError_t launch_decode_merge(const DecodeParams& p, int head_dim, hipStream_t stream) {
  const dim3 mgrid(p.num_kv_heads * p.group, p.batch);
  if (head_dim == 128)
    hipLaunchKernelGGL((decode_merge_kernel<128>), mgrid, dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_merge_kernel<64>), mgrid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, int head_dim, hipStream_t stream) {
  // two workgroups of 8 waves per CU (LDS and registers allow no more);
  // stages as set in launch_decode_d.  Two 32 KiB stages measured faster
  // than three or four at one workgroup per CU.
  if (head_dim == 128)
    launch_decode_d<128>(p, stream);
  else
    launch_decode_d<64>(p, stream);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode_merge(p, head_dim, stream);
}

}  // namespace msgl
