// Host side of the C ABI declared in include/msgl.h: argument validation
// (before any HIP call), the gfx950 check, the optional checked mode, and
// the launch of the kernels on the caller's stream.
#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "msgl.h"
#include "common.h"

using namespace msgl;

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

bool env_on(const char* name) {
  const char* v = std::getenv(name);
  return v && v[0] && std::strcmp(v, "0") != 0;
}

msgl_status hip_status(hipError_t e) { return e == hipSuccess ? MSGL_OK : MSGL_ERR_HIP; }

// The kernels use gfx950 instructions (bf16 dot2, 32x32x16 bf16 MFMA).
msgl_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MSGL_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MSGL_ERR_UNSUPPORTED;
  int st = g_arch_state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MSGL_ERR_HIP;
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_state[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? MSGL_OK : MSGL_ERR_UNSUPPORTED;
}

msgl_status check_pool(const msgl_kv_pool* pool, int32_t layer) {
  if (!pool || !pool->data) return MSGL_ERR_NULL;
  if (pool->num_layers < 1 || pool->num_pages < 1 || pool->page_size < 1 ||
      pool->num_kv_heads < 1 || pool->head_dim < 1)
    return MSGL_ERR_SHAPE;
  if (layer < 0 || layer >= pool->num_layers) return MSGL_ERR_SHAPE;
  if (static_cast<int64_t>(pool->num_pages) * pool->page_size > INT32_MAX) return MSGL_ERR_SHAPE;
  return MSGL_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// log2(page_size) when it is a power of two, else -1 (the kernels then divide)
int32_t page_shift_of(int32_t page_size) {
  for (int b = 0; b < 31; ++b)
    if (page_size == (1 << b)) return b;
  return -1;
}

int64_t num_slots(const msgl_kv_pool* pool) {
  return static_cast<int64_t>(pool->num_pages) * pool->page_size;
}
int64_t half_elems(const msgl_kv_pool* pool) {  // elements of one (K or V, layer)
  return num_slots(pool) * pool->num_kv_heads * pool->head_dim;
}
const uint16_t* k_half(const msgl_kv_pool* pool, int32_t layer) {
  return static_cast<const uint16_t*>(pool->data) + static_cast<int64_t>(layer) * half_elems(pool);
}
const uint16_t* v_half(const msgl_kv_pool* pool, int32_t layer) {
  return static_cast<const uint16_t*>(pool->data) +
         static_cast<int64_t>(pool->num_layers + layer) * half_elems(pool);
}

// Attention calls: geometry the kernels are built for.
msgl_status check_attention_geometry(const msgl_kv_pool* pool, int32_t num_qo_heads) {
  if (pool->head_dim != 64 && pool->head_dim != 128) return MSGL_ERR_UNSUPPORTED;
  if (num_qo_heads < 1 || num_qo_heads % pool->num_kv_heads != 0) return MSGL_ERR_SHAPE;
  if (num_qo_heads / pool->num_kv_heads > 16) return MSGL_ERR_UNSUPPORTED;
  if (pool->num_kv_heads > 65535) return MSGL_ERR_UNSUPPORTED;
  if (!aligned16(pool->data)) return MSGL_ERR_SHAPE;
  return MSGL_OK;
}

// Compute units of the current device, looked up once per device.
std::atomic<int> g_cus[kMaxDevices];
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = g_cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 256;
    g_cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Waves per extend workgroup (32 query rows each).  MSGL_EXTEND_WAVES=4 or
// 8 forces one.  Otherwise 8 (256-row workgroups), except for a pure extend
// call whose 256-row tiles -- at least ceil(total * G / 256) per kv head --
// cannot give every CU a workgroup: there 4 (twice as many 128-row
// workgroups) measured 13-17% faster (one 512-token request, or the
// one-kv-head share of a tensor-parallel GPU), while at 256 tiles and more
// 8 stays 7-13% ahead.  The mixed launch keeps 8: its decode ranges fill the
// CUs the extend tiles leave.
int extend_waves(int64_t total_extend_tokens, int32_t G, int32_t num_kv_heads, bool allow_four) {
  const char* v = std::getenv("MSGL_EXTEND_WAVES");
  if (v && std::atoi(v) == 4) return 4;
  if (v && std::atoi(v) == 8) return 8;
  if (!allow_four) return 8;
  const int64_t tiles = (total_extend_tokens * G + 255) / 256 * num_kv_heads;
  return tiles < device_cus() ? 4 : 8;
}

// kv heads per decode workgroup: the largest power of two <= 8 dividing Hkv
int32_t decode_head_group(int32_t num_kv_heads) {
  int32_t hg = 8;
  while (num_kv_heads % hg) hg >>= 1;
  return hg;
}

// Decode workspace (bytes, each part 256-byte aligned): a piece map, one
// int2 per request; then, for each launch of up to kDecodeBatch requests,
// the fp32 partial outputs of its pieces (pieces, Hq, d) and their
// (max, sum) pairs.  A launch of b
// requests splits their lengths, each rounded up to whole tiles of at most
// kDecodeMaxTile tokens (so at most b * (max_seq_len + kDecodeMaxTile - 1)
// tokens), over at most kDecodeGrid ranges of >= kDecodeMinTokens, and
// piece i + r of range i and request r is below ranges + b.
int64_t decode_pieces(int64_t b, int64_t max_seq_len) {
  const int64_t tokens = b * (max_seq_len + kDecodeMaxTile - 1);
  const int64_t ranges = std::min<int64_t>(kDecodeGrid, (tokens + kDecodeMinTokens - 1) / kDecodeMinTokens);
  return ranges + b;
}
struct DecodeWorkspace {
  int64_t map_bytes, o_bytes, ml_bytes;
};
int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }
DecodeWorkspace decode_workspace(int32_t batch, int32_t num_qo_heads, int32_t head_dim,
                                 int32_t max_seq_len) {
  DecodeWorkspace w{0, 0, 0};
  if (batch <= 0) return w;
  int64_t pieces = 0;
  for (int64_t b0 = 0; b0 < batch; b0 += kDecodeBatch)
    pieces += decode_pieces(std::min<int64_t>(kDecodeBatch, batch - b0), max_seq_len);
  w.map_bytes = align256(static_cast<int64_t>(batch) * 8);
  w.o_bytes = align256(pieces * num_qo_heads * head_dim * 4);
  w.ml_bytes = pieces * num_qo_heads * 2 * 4;
  return w;
}

// Key shares per extend row tile (1: none).  MSGL_EXTEND_SPLITS=n forces n
// (1 to kExtendMaxSplits).  Otherwise a call whose 256-row tiles -- at
// least ceil(total * G / 256) per kv head -- are fewer than the CUs takes
// enough shares for one workgroup per CU, at most kExtendMaxSplits and at
// most one per kExtendKeysPerSplit keys of the longest row; with fewer
// than two it runs unsplit (128-row workgroups).  Measured against 2, 4
// and 8 shares forced, back-to-back calls: one 512-token piece on a 2048
// prefix (64 tiles) 44 us with 4 shares, 55 with 2, 58 with 8, 62
// unsplit; one 1024-token piece on 8192 (128 tiles) 161 with 2, 169 with
// 4, 209 unsplit; one 4096-token chunk on 12288 at 4 q / 1 kv head (64
// tiles) 143 with 4, 150 with 8, 350 unsplit; a 512-token piece with no
// prefix 16 us unsplit, 28 with 2; from 256 tiles up, unsplit is best.
constexpr int kExtendMaxSplits = 8;
constexpr int kExtendSplitFill = 1;
constexpr int kExtendKeysPerSplit = 512;
int extend_splits(int64_t total_extend_tokens, int32_t G, int32_t num_kv_heads,
                  int32_t max_seq_len) {
  const char* v = std::getenv("MSGL_EXTEND_SPLITS");
  if (v && v[0]) return std::min(std::max(std::atoi(v), 1), kExtendMaxSplits);
  const int64_t tiles = (total_extend_tokens * G + 255) / 256 * num_kv_heads;
  const int64_t cus = device_cus();
  if (tiles <= 0 || tiles >= cus) return 1;
  int64_t sp = (kExtendSplitFill * cus + tiles - 1) / tiles;
  sp = std::min<int64_t>(sp, kExtendMaxSplits);
  sp = std::min<int64_t>(sp, std::max<int64_t>(1, max_seq_len / kExtendKeysPerSplit));
  return static_cast<int>(std::max<int64_t>(sp, 1));
}

// Workspace of a key-split extend: fp32 o (tokens, Hq, shares, d), then
// (m, l) pairs (tokens, Hq, shares), the first part 256-byte aligned.
int64_t extend_split_o_bytes(int64_t tokens, int32_t num_qo_heads, int splits, int32_t head_dim) {
  return align256(tokens * num_qo_heads * splits * head_dim * 4);
}
int64_t extend_split_bytes(int64_t tokens, int32_t num_qo_heads, int splits, int32_t head_dim) {
  if (splits <= 1 || tokens <= 0) return 0;
  return extend_split_o_bytes(tokens, num_qo_heads, splits, head_dim) +
         tokens * num_qo_heads * splits * 2 * 4;
}

// Longest sequence a decode call takes: the token total of a launch, each
// length padded to whole tiles of up to kDecodeMaxTile tokens, fits in int32.
constexpr int64_t kDecodeMaxSeqLen = INT32_MAX / kDecodeBatch - kDecodeMaxTile;
static_assert(kDecodeBatch * (kDecodeMaxSeqLen + kDecodeMaxTile) <= INT32_MAX, "token total");

template <typename T>
bool copy_to_host(std::vector<T>& dst, const T* src, size_t n, hipStream_t stream) {
  dst.resize(n);
  if (n == 0) return true;
  if (hipMemcpyAsync(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return false;
  return hipStreamSynchronize(stream) == hipSuccess;
}

// Checked mode: the page ids that tokens 0 .. len-1 of a row would read.
msgl_status check_row_pages(const int32_t* page_table, int64_t stride, int32_t row, int32_t len,
                            const msgl_kv_pool* pool, hipStream_t stream) {
  if (row < 0) return MSGL_ERR_RANGE;
  if (len <= 0) return MSGL_OK;
  const int64_t npg = (len + pool->page_size - 1) / pool->page_size;
  std::vector<int32_t> ids;
  if (!copy_to_host(ids, page_table + static_cast<int64_t>(row) * stride, static_cast<size_t>(npg),
                    stream))
    return MSGL_ERR_HIP;
  for (int32_t id : ids)
    if (id < 0 || id >= pool->num_pages) return MSGL_ERR_RANGE;
  return MSGL_OK;
}

// Kernel parameters of a decode over validated arguments.
DecodeParams decode_params(const msgl_kv_pool* pool, int32_t layer, const void* q,
                           int64_t q_row_stride, void* out, const int32_t* page_table,
                           int32_t page_table_stride, const int32_t* table_idx,
                           const int32_t* seq_lens, int32_t batch, int32_t num_qo_heads,
                           int32_t max_seq_len, float sm_scale, void* workspace) {
  const int32_t d = pool->head_dim;
  const DecodeWorkspace ws = decode_workspace(batch, num_qo_heads, d, max_seq_len);
  DecodeParams p;
  p.k_cache = k_half(pool, layer);
  p.v_cache = v_half(pool, layer);
  p.q = static_cast<const uint16_t*>(q);
  p.q_stride = q_row_stride;
  p.out = static_cast<uint16_t*>(out);
  p.page_table = page_table;
  p.pt_stride = page_table_stride;
  p.table_idx = table_idx;
  p.seq_lens = seq_lens;
  p.batch = batch;
  p.num_kv_heads = pool->num_kv_heads;
  p.group = num_qo_heads / pool->num_kv_heads;
  p.head_group = decode_head_group(pool->num_kv_heads);
  p.page_size = pool->page_size;
  p.num_slots = static_cast<int32_t>(num_slots(pool));
  p.half_bytes = static_cast<uint32_t>(half_elems(pool) * 2);
  p.max_seq_len = max_seq_len;
  p.scale_log2 = sm_scale * kLog2e;
  p.mixed_prefix = nullptr;
  p.mixed_extend = nullptr;
  p.mixed_cu = nullptr;
  uint8_t* base = static_cast<uint8_t*>(workspace);
  p.ws_map = reinterpret_cast<int2*>(base);
  p.ws_o = reinterpret_cast<float*>(base + ws.map_bytes);
  p.ws_ml = reinterpret_cast<float*>(base + ws.map_bytes + ws.o_bytes);
  return p;
}

// One launch per kDecodeBatch requests, each with its own piece region of
// the workspace.
hipError_t launch_decode_batches(const DecodeParams& p, int32_t head_dim, hipStream_t stream) {
  const int64_t Hq = static_cast<int64_t>(p.num_kv_heads) * p.group;
  int64_t piece_off = 0;
  for (int32_t b0 = 0; b0 < p.batch; b0 += kDecodeBatch) {
    DecodeParams s = p;
    s.batch = std::min<int32_t>(kDecodeBatch, p.batch - b0);
    s.table_idx += b0;
    if (p.mixed_cu) {
      s.mixed_prefix += b0;
      s.mixed_extend += b0;
      s.mixed_cu += b0;
    } else {
      s.seq_lens += b0;
      s.q += b0 * p.q_stride;
      s.out += static_cast<int64_t>(b0) * Hq * head_dim;
    }
    s.ws_map += b0;
    s.ws_o += piece_off * Hq * head_dim;
    s.ws_ml += piece_off * Hq * 2;
    piece_off += decode_pieces(s.batch, p.max_seq_len);
    const hipError_t e = launch_decode(s, head_dim, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Kernel parameters of an extend over validated arguments.
ExtendParams extend_params(const msgl_kv_pool* pool, int32_t layer, const void* q,
                           int64_t q_row_stride, void* out, const int32_t* page_table,
                           int32_t page_table_stride, const int32_t* table_idx,
                           const int32_t* prefix_lens, const int32_t* extend_lens,
                           const int32_t* cu_extend_lens, int32_t num_qo_heads, int32_t mtiles,
                           int32_t max_extend_len, int32_t max_seq_len, float sm_scale,
                           int32_t skip_single) {
  const int32_t G = num_qo_heads / pool->num_kv_heads;
  ExtendParams p;
  p.k_cache = k_half(pool, layer);
  p.v_cache = v_half(pool, layer);
  p.q = static_cast<const uint16_t*>(q);
  p.q_stride = q_row_stride;
  p.out = static_cast<uint16_t*>(out);
  p.page_table = page_table;
  p.pt_stride = page_table_stride;
  p.table_idx = table_idx;
  p.prefix_lens = prefix_lens;
  p.extend_lens = extend_lens;
  p.cu_extend = cu_extend_lens;
  p.num_kv_heads = pool->num_kv_heads;
  p.group = G;
  p.page_size = pool->page_size;
  p.num_mtiles = mtiles;
  p.half_bytes = static_cast<uint32_t>(half_elems(pool) * 2);
  p.page_shift = page_shift_of(pool->page_size);
  p.max_extend_len = max_extend_len;
  p.max_seq_len = max_seq_len;
  p.num_slots = static_cast<int32_t>(num_slots(pool));
  p.scale_log2 = sm_scale * kLog2e;
  p.skip_single = skip_single;
  p.num_splits = 1;
  p.ws_o = nullptr;
  p.ws_ml = nullptr;
  return p;
}

// Host-side checks of an extend call (and of the extend half of a mixed
// call), checked mode included; sets the launch shape.
msgl_status extend_checks(const msgl_kv_pool* pool, int32_t layer, const void* q,
                          int64_t q_row_stride, void* out, const int32_t* page_table,
                          int32_t page_table_stride, const int32_t* table_idx,
                          const int32_t* prefix_lens, const int32_t* extend_lens,
                          const int32_t* cu_extend_lens, int32_t batch,
                          int32_t total_extend_tokens, int32_t max_extend_len,
                          int32_t max_seq_len, int32_t num_qo_heads, float sm_scale,
                          bool* nothing_to_do, int64_t* mtiles_out, int* waves_out,
                          bool allow_four_waves, hipStream_t stream) {
  *nothing_to_do = false;
  msgl_status st = check_pool(pool, layer);
  if (st != MSGL_OK) return st;
  if (batch < 0 || total_extend_tokens < 0 || max_extend_len < 0 || max_seq_len < 0)
    return MSGL_ERR_SHAPE;
  if (batch == 0 || total_extend_tokens == 0 || max_extend_len == 0) {
    *nothing_to_do = true;
    return MSGL_OK;
  }
  if (!q || !out || !page_table || !table_idx || !prefix_lens || !extend_lens || !cu_extend_lens)
    return MSGL_ERR_NULL;
  st = check_attention_geometry(pool, num_qo_heads);
  if (st != MSGL_OK) return st;
  if (batch > 65535) return MSGL_ERR_UNSUPPORTED;
  const int32_t d = pool->head_dim;
  if (q_row_stride < static_cast<int64_t>(num_qo_heads) * d || (q_row_stride % 8) != 0 ||
      !aligned16(q) || !aligned16(out))
    return MSGL_ERR_SHAPE;
  if (max_extend_len > max_seq_len) return MSGL_ERR_SHAPE;
  // extend addresses one (K or V, layer) sub-tensor with 32-bit byte offsets
  if (half_elems(pool) * 2 >= (int64_t{1} << 32)) return MSGL_ERR_UNSUPPORTED;
  if (!(sm_scale > 0.f)) return MSGL_ERR_SHAPE;
  if (page_table_stride < 1) return MSGL_ERR_SHAPE;
  const int32_t max_pages = (max_seq_len + pool->page_size - 1) / pool->page_size;
  if (max_pages > page_table_stride) return MSGL_ERR_SHAPE;
  const int32_t G = num_qo_heads / pool->num_kv_heads;
  const int waves = extend_waves(total_extend_tokens, G, pool->num_kv_heads, allow_four_waves);
  *waves_out = waves;
  const int64_t rows_per_tile = 32 * waves;
  const int64_t mtiles = (static_cast<int64_t>(max_extend_len) * G + rows_per_tile - 1) / rows_per_tile;
  if (mtiles > 65535) return MSGL_ERR_UNSUPPORTED;  // grid z
  *mtiles_out = mtiles;
  st = check_device();
  if (st != MSGL_OK) return st;
  if (env_on("MSGL_CHECK")) {
    std::vector<int32_t> ti, pl, el, cu;
    if (!copy_to_host(ti, table_idx, batch, stream) || !copy_to_host(pl, prefix_lens, batch, stream) ||
        !copy_to_host(el, extend_lens, batch, stream) ||
        !copy_to_host(cu, cu_extend_lens, batch + 1, stream))
      return MSGL_ERR_HIP;
    if (cu[0] != 0 || cu[batch] != total_extend_tokens) return MSGL_ERR_RANGE;
    for (int32_t b = 0; b < batch; ++b) {
      if (pl[b] < 0 || el[b] < 0 || el[b] > max_extend_len ||
          static_cast<int64_t>(pl[b]) + el[b] > max_seq_len || cu[b + 1] - cu[b] != el[b])
        return MSGL_ERR_RANGE;
      st = check_row_pages(page_table, page_table_stride, ti[b], pl[b] + el[b], pool, stream);
      if (st != MSGL_OK) return st;
    }
  }
  return MSGL_OK;
}

// Allocation-free decode: the workspace comes from this file-scope device
// array instead of the caller.  Each GPU the library runs on holds its own
// copy until the process ends; host code reaches a device's copy only
// through the address hipGetSymbolAddress returns with that device current
// (the array's name on the host is a stand-in, not a device address).
constexpr size_t kScratchBytes = size_t{64} << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch`, looked up once per device.
msgl_status scratch_for_current_device(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MSGL_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MSGL_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MSGL_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MSGL_OK;
}

}  // namespace

// A captured store_kv + decode: the instantiated HIP graph.
struct msgl_decode_graph {
  hipGraphExec_t exec;
};

// Graphs of one set of static buffers at batch sizes 1, 2, 4, ... and the
// largest size; a launch replays the smallest one that holds the batch.
constexpr int kMaxRunnerGraphs = 32;
struct msgl_decode_graph_runner {
  int32_t count;
  int32_t sizes[kMaxRunnerGraphs];
  msgl_decode_graph* graphs[kMaxRunnerGraphs];
};

extern "C" {

int32_t msgl_abi_version(void) { return MSGL_ABI_VERSION; }

const char* msgl_status_string(msgl_status s) {
  switch (s) {
    case MSGL_OK:
      return "ok";
    case MSGL_ERR_NULL:
      return "a required pointer is NULL";
    case MSGL_ERR_SHAPE:
      return "inconsistent sizes, strides or alignment";
    case MSGL_ERR_UNSUPPORTED:
      return "unsupported head_dim, group size or device (gfx950 required)";
    case MSGL_ERR_WORKSPACE:
      return "decode workspace too small";
    case MSGL_ERR_RANGE:
      return "an index or length on the device is out of range (checked mode)";
    case MSGL_ERR_HIP:
      return "a HIP runtime call or kernel launch failed";
    default:
      return "unknown status";
  }
}

msgl_status msgl_store_kv(const msgl_kv_pool* pool, int32_t layer, const void* k,
                          int64_t k_row_stride, const void* v, int64_t v_row_stride,
                          const int32_t* out_loc, int32_t num_tokens, void* stream) {
  msgl_status st = check_pool(pool, layer);
  if (st != MSGL_OK) return st;
  if (num_tokens < 0) return MSGL_ERR_SHAPE;
  if (num_tokens == 0) return MSGL_OK;
  if (!k || !v || !out_loc) return MSGL_ERR_NULL;
  const int64_t row = static_cast<int64_t>(pool->num_kv_heads) * pool->head_dim;
  if (k_row_stride < row || v_row_stride < row) return MSGL_ERR_SHAPE;
  const int row_bytes = static_cast<int>(row * 2);
  // widest piece that keeps every row start and the pool aligned
  int vec = 16;
  auto fits = [&](int a) {
    return (reinterpret_cast<uintptr_t>(k) % a) == 0 && (reinterpret_cast<uintptr_t>(v) % a) == 0 &&
           ((k_row_stride * 2) % a) == 0 && ((v_row_stride * 2) % a) == 0 && (row_bytes % a) == 0 &&
           (reinterpret_cast<uintptr_t>(pool->data) % a) == 0;
  };
  while (vec > 2 && !fits(vec)) vec >>= 1;
  if (!fits(2)) return MSGL_ERR_SHAPE;
  st = check_device();
  if (st != MSGL_OK) return st;
  if (env_on("MSGL_CHECK")) {
    std::vector<int32_t> loc;
    if (!copy_to_host(loc, out_loc, static_cast<size_t>(num_tokens), static_cast<hipStream_t>(stream)))
      return MSGL_ERR_HIP;
    std::vector<int32_t> live;
    for (int32_t s : loc) {
      if (s >= num_slots(pool)) return MSGL_ERR_RANGE;
      if (s >= 0) live.push_back(s);
    }
    // two rows into one slot: sorted, equal neighbours (host memory of the
    // step's size, not of the pool's)
    std::sort(live.begin(), live.end());
    if (std::adjacent_find(live.begin(), live.end()) != live.end()) return MSGL_ERR_RANGE;
  }
  StoreParams p;
  p.k = static_cast<const uint8_t*>(k);
  p.v = static_cast<const uint8_t*>(v);
  p.k_stride_bytes = k_row_stride * 2;
  p.v_stride_bytes = v_row_stride * 2;
  p.out_loc = out_loc;
  p.k_cache = reinterpret_cast<uint8_t*>(const_cast<uint16_t*>(k_half(pool, layer)));
  p.v_cache = reinterpret_cast<uint8_t*>(const_cast<uint16_t*>(v_half(pool, layer)));
  p.pieces_per_row = row_bytes / vec;
  p.row_bytes = row_bytes;
  p.num_tokens = num_tokens;
  p.num_slots = static_cast<int32_t>(num_slots(pool));
  p.num_items = static_cast<int64_t>(num_tokens) * 2 * p.pieces_per_row;
  return hip_status(launch_store_kv(p, vec, static_cast<hipStream_t>(stream)));
}

size_t msgl_paged_decode_workspace_size(int32_t batch, int32_t num_qo_heads, int32_t head_dim,
                                        int32_t max_seq_len, int32_t page_size) {
  // page_size does not change the layout: ranges split tokens, not pages
  if (batch < 0 || num_qo_heads < 1 || head_dim < 1 || max_seq_len < 0 || page_size < 1) return 0;
  const DecodeWorkspace w = decode_workspace(batch, num_qo_heads, head_dim, max_seq_len);
  return static_cast<size_t>(w.map_bytes + w.o_bytes + w.ml_bytes);
}

msgl_status msgl_paged_decode(const msgl_kv_pool* pool, int32_t layer, const void* q,
                              int64_t q_row_stride, void* out, const int32_t* page_table,
                              int32_t page_table_stride, const int32_t* table_idx,
                              const int32_t* seq_lens, int32_t batch, int32_t num_qo_heads,
                              int32_t max_seq_len, float sm_scale, void* workspace,
                              size_t workspace_bytes, void* stream) {
  msgl_status st = check_pool(pool, layer);
  if (st != MSGL_OK) return st;
  if (batch < 0 || max_seq_len < 0) return MSGL_ERR_SHAPE;
  if (batch == 0) return MSGL_OK;
  if (!q || !out || !page_table || !table_idx || !seq_lens) return MSGL_ERR_NULL;
  st = check_attention_geometry(pool, num_qo_heads);
  if (st != MSGL_OK) return st;
  if (batch > 65535) return MSGL_ERR_UNSUPPORTED;
  if (!(sm_scale > 0.f)) return MSGL_ERR_SHAPE;
  // decode addresses one (K or V, layer) sub-tensor with 32-bit byte offsets
  if (half_elems(pool) * 2 >= (int64_t{1} << 32)) return MSGL_ERR_UNSUPPORTED;
  const int32_t d = pool->head_dim;
  if (q_row_stride < static_cast<int64_t>(num_qo_heads) * d || (q_row_stride % 8) != 0 ||
      !aligned16(q) || !aligned16(out))
    return MSGL_ERR_SHAPE;
  if (page_table_stride < 1) return MSGL_ERR_SHAPE;
  const int32_t max_pages = (max_seq_len + pool->page_size - 1) / pool->page_size;
  if (max_pages > page_table_stride) return MSGL_ERR_SHAPE;
  if (max_seq_len > kDecodeMaxSeqLen) return MSGL_ERR_UNSUPPORTED;
  const size_t need =
      msgl_paged_decode_workspace_size(batch, num_qo_heads, d, max_seq_len, pool->page_size);
  if (!workspace || workspace_bytes < need) return MSGL_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return MSGL_ERR_SHAPE;
  st = check_device();
  if (st != MSGL_OK) return st;
  if (env_on("MSGL_CHECK")) {
    std::vector<int32_t> ti, sl;
    const hipStream_t cs = static_cast<hipStream_t>(stream);
    if (!copy_to_host(ti, table_idx, batch, cs) || !copy_to_host(sl, seq_lens, batch, cs))
      return MSGL_ERR_HIP;
    for (int32_t b = 0; b < batch; ++b) {
      if (sl[b] < 0 || sl[b] > max_seq_len) return MSGL_ERR_RANGE;
      st = check_row_pages(page_table, page_table_stride, ti[b], sl[b], pool, cs);
      if (st != MSGL_OK) return st;
    }
  }
  const DecodeParams p = decode_params(pool, layer, q, q_row_stride, out, page_table, page_table_stride,
                                       table_idx, seq_lens, batch, num_qo_heads, max_seq_len,
                                       sm_scale, workspace);
  return hip_status(launch_decode_batches(p, d, static_cast<hipStream_t>(stream)));
}

size_t msgl_paged_decode_noalloc_max_workspace(void) { return kScratchBytes; }

msgl_status msgl_paged_decode_noalloc(const msgl_kv_pool* pool, int32_t layer, const void* q,
                                      int64_t q_row_stride, void* out, const int32_t* page_table,
                                      int32_t page_table_stride, const int32_t* table_idx,
                                      const int32_t* seq_lens, int32_t batch, int32_t num_qo_heads,
                                      int32_t max_seq_len, float sm_scale, void* stream) {
  // sizes beyond the scratch array are refused before any HIP call
  msgl_status st = check_pool(pool, layer);
  if (st != MSGL_OK) return st;
  if (batch < 0 || max_seq_len < 0 || num_qo_heads < 1) return MSGL_ERR_SHAPE;
  if (batch == 0) return MSGL_OK;
  const size_t need = msgl_paged_decode_workspace_size(batch, num_qo_heads, pool->head_dim,
                                                       max_seq_len, pool->page_size);
  if (need > kScratchBytes) return MSGL_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != MSGL_OK) return st;
  return msgl_paged_decode(pool, layer, q, q_row_stride, out, page_table, page_table_stride,
                           table_idx, seq_lens, batch, num_qo_heads, max_seq_len, sm_scale, ws,
                           kScratchBytes, stream);
}

msgl_status msgl_paged_extend(const msgl_kv_pool* pool, int32_t layer, const void* q,
                              int64_t q_row_stride, void* out, const int32_t* page_table,
                              int32_t page_table_stride, const int32_t* table_idx,
                              const int32_t* prefix_lens, const int32_t* extend_lens,
                              const int32_t* cu_extend_lens, int32_t batch,
                              int32_t total_extend_tokens, int32_t max_extend_len,
                              int32_t max_seq_len, int32_t num_qo_heads, float sm_scale,
                              void* stream) {
  bool nothing = false;
  int64_t mtiles = 0;
  int waves = 8;
  msgl_status st = extend_checks(pool, layer, q, q_row_stride, out, page_table, page_table_stride,
                                 table_idx, prefix_lens, extend_lens, cu_extend_lens, batch,
                                 total_extend_tokens, max_extend_len, max_seq_len, num_qo_heads,
                                 sm_scale, &nothing, &mtiles, &waves, true,
                                 static_cast<hipStream_t>(stream));
  if (st != MSGL_OK || nothing) return st;
  const int32_t d = pool->head_dim;
  const ExtendParams p = extend_params(pool, layer, q, q_row_stride, out, page_table,
                                       page_table_stride, table_idx, prefix_lens, extend_lens,
                                       cu_extend_lens, num_qo_heads, static_cast<int32_t>(mtiles),
                                       max_extend_len, max_seq_len, sm_scale, 0);
  return hip_status(launch_extend(p, d, batch, waves, static_cast<hipStream_t>(stream)));
}

size_t msgl_paged_extend_workspace_size(const msgl_kv_pool* pool, int32_t total_extend_tokens,
                                        int32_t max_seq_len, int32_t num_qo_heads) {
  if (!pool || pool->num_kv_heads < 1 || num_qo_heads < 1 || num_qo_heads % pool->num_kv_heads != 0 ||
      total_extend_tokens <= 0 || max_seq_len < 1 || (pool->head_dim != 64 && pool->head_dim != 128))
    return 0;
  const int32_t G = num_qo_heads / pool->num_kv_heads;
  const int sp = extend_splits(total_extend_tokens, G, pool->num_kv_heads, max_seq_len);
  return static_cast<size_t>(extend_split_bytes(total_extend_tokens, num_qo_heads, sp, pool->head_dim));
}

msgl_status msgl_paged_extend_split(const msgl_kv_pool* pool, int32_t layer, const void* q,
                                    int64_t q_row_stride, void* out, const int32_t* page_table,
                                    int32_t page_table_stride, const int32_t* table_idx,
                                    const int32_t* prefix_lens, const int32_t* extend_lens,
                                    const int32_t* cu_extend_lens, int32_t batch,
                                    int32_t total_extend_tokens, int32_t max_extend_len,
                                    int32_t max_seq_len, int32_t num_qo_heads, float sm_scale,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  const size_t need =
      msgl_paged_extend_workspace_size(pool, total_extend_tokens, max_seq_len, num_qo_heads);
  if (need == 0 || !workspace)
    return msgl_paged_extend(pool, layer, q, q_row_stride, out, page_table, page_table_stride,
                             table_idx, prefix_lens, extend_lens, cu_extend_lens, batch,
                             total_extend_tokens, max_extend_len, max_seq_len, num_qo_heads,
                             sm_scale, stream);
  if (workspace_bytes < need) return MSGL_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return MSGL_ERR_SHAPE;
  bool nothing = false;
  int64_t mtiles = 0;
  int waves = 8;
  msgl_status st = extend_checks(pool, layer, q, q_row_stride, out, page_table, page_table_stride,
                                 table_idx, prefix_lens, extend_lens, cu_extend_lens, batch,
                                 total_extend_tokens, max_extend_len, max_seq_len, num_qo_heads,
                                 sm_scale, &nothing, &mtiles, &waves, false,
                                 static_cast<hipStream_t>(stream));
  if (st != MSGL_OK || nothing) return st;
  const int32_t d = pool->head_dim;
  const int32_t G = num_qo_heads / pool->num_kv_heads;
  const int sp = extend_splits(total_extend_tokens, G, pool->num_kv_heads, max_seq_len);
  if (waves != 8 || mtiles * sp > 65535)  // a forced workgroup size, or a grid too tall
    return msgl_paged_extend(pool, layer, q, q_row_stride, out, page_table, page_table_stride,
                             table_idx, prefix_lens, extend_lens, cu_extend_lens, batch,
                             total_extend_tokens, max_extend_len, max_seq_len, num_qo_heads,
                             sm_scale, stream);
  ExtendParams p = extend_params(pool, layer, q, q_row_stride, out, page_table, page_table_stride,
                                 table_idx, prefix_lens, extend_lens, cu_extend_lens, num_qo_heads,
                                 static_cast<int32_t>(mtiles), max_extend_len, max_seq_len, sm_scale,
                                 0);
  uint8_t* base = static_cast<uint8_t*>(workspace);
  p.num_splits = sp;
  p.ws_o = reinterpret_cast<float*>(base);
  p.ws_ml = reinterpret_cast<float*>(base + extend_split_o_bytes(total_extend_tokens, num_qo_heads, sp, d));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  st = hip_status(launch_extend(p, d, batch, 8, s));
  if (st != MSGL_OK) return st;
  return hip_status(launch_extend_merge(p, d, total_extend_tokens, s));
}

msgl_status msgl_paged_mixed(const msgl_kv_pool* pool, int32_t layer, const void* q,
                             int64_t q_row_stride, void* out, const int32_t* page_table,
                             int32_t page_table_stride, const int32_t* table_idx,
                             const int32_t* prefix_lens, const int32_t* extend_lens,
                             const int32_t* cu_extend_lens, int32_t batch,
                             int32_t total_extend_tokens, int32_t max_extend_len,
                             int32_t max_seq_len, int32_t num_qo_heads, float sm_scale,
                             void* workspace, size_t workspace_bytes, void* stream) {
  bool nothing = false;
  int64_t mtiles = 0;
  int waves = 8;
  msgl_status st = extend_checks(pool, layer, q, q_row_stride, out, page_table, page_table_stride,
                                 table_idx, prefix_lens, extend_lens, cu_extend_lens, batch,
                                 total_extend_tokens, max_extend_len, max_seq_len, num_qo_heads,
                                 sm_scale, &nothing, &mtiles, &waves, false,
                                 static_cast<hipStream_t>(stream));
  if (st != MSGL_OK || nothing) return st;
  const int32_t d = pool->head_dim;
  if (max_seq_len > kDecodeMaxSeqLen) return MSGL_ERR_UNSUPPORTED;
  const size_t need =
      msgl_paged_decode_workspace_size(batch, num_qo_heads, d, max_seq_len, pool->page_size);
  if (!workspace || workspace_bytes < need) return MSGL_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return MSGL_ERR_SHAPE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // rows with one new token: split-KV decode and its merge
  DecodeParams pd = decode_params(pool, layer, q, q_row_stride, out, page_table, page_table_stride,
                                  table_idx, nullptr, batch, num_qo_heads, max_seq_len, sm_scale,
                                  workspace);
  pd.mixed_prefix = prefix_lens;
  pd.mixed_extend = extend_lens;
  pd.mixed_cu = cu_extend_lens;
  if (max_extend_len <= 1) return hip_status(launch_decode_batches(pd, d, s));  // decode rows only
  // the other rows: causal extend
  const ExtendParams pe = extend_params(pool, layer, q, q_row_stride, out, page_table,
                                        page_table_stride, table_idx, prefix_lens, extend_lens,
                                        cu_extend_lens, num_qo_heads, static_cast<int32_t>(mtiles),
                                        max_extend_len, max_seq_len, sm_scale, 1);
  // one launch: a row of E > 1 new tokens has ceil(E*G/256) row tiles, so
  // the batch has at most total*G/256 + batch of them
  const int64_t G = num_qo_heads / pool->num_kv_heads;
  const int64_t bound = std::min<int64_t>(static_cast<int64_t>(batch) * mtiles,
                                          static_cast<int64_t>(total_extend_tokens) * G / 256 + batch);
  const int64_t blocks = bound * pool->num_kv_heads +
                         static_cast<int64_t>(kDecodeGrid) * (pool->num_kv_heads / pd.head_group);
  if (batch <= kDecodeBatch && waves == 8 && pe.page_shift >= 0 && blocks <= INT32_MAX &&
      !env_on("MSGL_MIXED_SPLIT"))
    return hip_status(launch_mixed(pd, pe, d, bound, s));
  st = hip_status(launch_decode_batches(pd, d, s));
  if (st != MSGL_OK) return st;
  return hip_status(launch_extend(pe, d, batch, waves, s));
}

msgl_status msgl_debug_gather_kv(const msgl_kv_pool* pool, int32_t layer,
                                 const int32_t* page_table, int32_t page_table_stride,
                                 int32_t row, int32_t len, void* k_out, void* v_out,
                                 void* stream) {
  msgl_status st = check_pool(pool, layer);
  if (st != MSGL_OK) return st;
  if (len < 0 || row < 0 || page_table_stride < 1) return MSGL_ERR_SHAPE;
  if (len == 0) return MSGL_OK;
  if (!page_table || !k_out || !v_out) return MSGL_ERR_NULL;
  if ((len + pool->page_size - 1) / pool->page_size > page_table_stride) return MSGL_ERR_SHAPE;
  const int64_t row_bytes = static_cast<int64_t>(pool->num_kv_heads) * pool->head_dim * 2;
  if ((row_bytes % 16) != 0 || !aligned16(k_out) || !aligned16(v_out) || !aligned16(pool->data))
    return MSGL_ERR_SHAPE;
  st = check_device();
  if (st != MSGL_OK) return st;
  if (env_on("MSGL_CHECK")) {
    st = check_row_pages(page_table, page_table_stride, row, len, pool,
                         static_cast<hipStream_t>(stream));
    if (st != MSGL_OK) return st;
  }
  GatherParams p;
  p.k_cache = reinterpret_cast<const uint8_t*>(k_half(pool, layer));
  p.v_cache = reinterpret_cast<const uint8_t*>(v_half(pool, layer));
  p.page_row = page_table + static_cast<int64_t>(row) * page_table_stride;
  p.k_out = static_cast<uint8_t*>(k_out);
  p.v_out = static_cast<uint8_t*>(v_out);
  p.row_bytes = static_cast<int32_t>(row_bytes);
  p.pieces_per_row = static_cast<int32_t>(row_bytes / 16);
  p.page_size = pool->page_size;
  p.num_slots = static_cast<int32_t>(num_slots(pool));
  p.num_items = static_cast<int64_t>(len) * 2 * p.pieces_per_row;
  return hip_status(launch_gather(p, static_cast<hipStream_t>(stream)));
}

msgl_status msgl_rope_store_kv(const msgl_kv_pool* pool, int32_t layer, void* q,
                               int64_t q_row_stride, int32_t num_qo_heads, const void* k,
                               int64_t k_row_stride, const void* v, int64_t v_row_stride,
                               const int32_t* out_loc, const int32_t* positions,
                               int32_t num_tokens, const float* cos_sin_table,
                               int32_t max_position, void* stream) {
  msgl_status st = check_pool(pool, layer);
  if (st != MSGL_OK) return st;
  if (num_tokens < 0 || num_qo_heads < 0 || max_position < 1) return MSGL_ERR_SHAPE;
  if (num_tokens == 0) return MSGL_OK;
  if (!k || !v || !out_loc || !positions || !cos_sin_table || (num_qo_heads > 0 && !q))
    return MSGL_ERR_NULL;
  const int32_t d = pool->head_dim;
  if (d != 64 && d != 128) return MSGL_ERR_UNSUPPORTED;
  const int64_t row = static_cast<int64_t>(pool->num_kv_heads) * d;
  if (k_row_stride < row || v_row_stride < row || (k_row_stride % 8) != 0 ||
      (v_row_stride % 8) != 0 || !aligned16(k) || !aligned16(v) || !aligned16(pool->data) ||
      !aligned16(cos_sin_table))
    return MSGL_ERR_SHAPE;
  if (num_qo_heads > 0 && (q_row_stride < static_cast<int64_t>(num_qo_heads) * d ||
                           (q_row_stride % 8) != 0 || !aligned16(q)))
    return MSGL_ERR_SHAPE;
  st = check_device();
  if (st != MSGL_OK) return st;
  if (env_on("MSGL_CHECK")) {
    std::vector<int32_t> loc, pos;
    const hipStream_t cs = static_cast<hipStream_t>(stream);
    if (!copy_to_host(loc, out_loc, static_cast<size_t>(num_tokens), cs) ||
        !copy_to_host(pos, positions, static_cast<size_t>(num_tokens), cs))
      return MSGL_ERR_HIP;
    std::vector<int32_t> live;
    for (int32_t i = 0; i < num_tokens; ++i) {
      if (pos[i] < 0 || pos[i] >= max_position || loc[i] >= num_slots(pool)) return MSGL_ERR_RANGE;
      if (loc[i] >= 0) live.push_back(loc[i]);
    }
    std::sort(live.begin(), live.end());  // two rows into one slot
    if (std::adjacent_find(live.begin(), live.end()) != live.end()) return MSGL_ERR_RANGE;
  }
  RopeParams p;
  p.q = static_cast<uint16_t*>(q);
  p.q_stride = q_row_stride;
  p.k = static_cast<const uint16_t*>(k);
  p.k_stride = k_row_stride;
  p.v = static_cast<const uint16_t*>(v);
  p.v_stride = v_row_stride;
  p.out_loc = out_loc;
  p.positions = positions;
  p.table = cos_sin_table;
  p.k_cache = const_cast<uint16_t*>(k_half(pool, layer));
  p.v_cache = const_cast<uint16_t*>(v_half(pool, layer));
  p.num_qo_heads = num_qo_heads;
  p.num_kv_heads = pool->num_kv_heads;
  p.head_dim = d;
  p.max_position = max_position;
  p.num_slots = static_cast<int32_t>(num_slots(pool));
  const int64_t per_tok = static_cast<int64_t>(num_qo_heads + pool->num_kv_heads) * (d / 16) +
                          static_cast<int64_t>(pool->num_kv_heads) * (d / 8);
  p.num_items = per_tok * num_tokens;
  return hip_status(launch_rope_store_kv(p, static_cast<hipStream_t>(stream)));
}

msgl_status msgl_rope_cos_sin_table(float* table, int32_t max_position, int32_t head_dim,
                                    double base, void* stream) {
  if (max_position < 1 || head_dim < 2 || (head_dim % 2) != 0 || !(base > 0.0))
    return MSGL_ERR_SHAPE;
  if (!table) return MSGL_ERR_NULL;
  const msgl_status st = check_device();
  if (st != MSGL_OK) return st;
  return hip_status(launch_rope_table(table, max_position, head_dim, base,
                                      static_cast<hipStream_t>(stream)));
}

msgl_status msgl_alloc_pages(const int32_t* free_pages, int32_t* num_free, int32_t* page_table,
                             int32_t page_table_stride, int32_t page_table_rows,
                             const int32_t* table_idx, const int32_t* prefix_lens,
                             const int32_t* extend_lens, int32_t batch, int32_t page_size,
                             int32_t* out_loc, int64_t out_loc_capacity, int32_t* status,
                             void* stream) {
  if (batch < 0 || page_size < 1 || page_table_stride < 1 || page_table_rows < 1 ||
      out_loc_capacity < 0)
    return MSGL_ERR_SHAPE;
  if (!num_free || !page_table || !status || (batch > 0 && (!table_idx || !prefix_lens ||
                                                            !extend_lens)) ||
      (out_loc_capacity > 0 && !out_loc) || !free_pages)
    return MSGL_ERR_NULL;
  const msgl_status st = check_device();
  if (st != MSGL_OK) return st;
  AllocParams p;
  p.free_pages = free_pages;
  p.num_free = num_free;
  p.page_table = page_table;
  p.pt_stride = page_table_stride;
  p.pt_rows = page_table_rows;
  p.table_idx = table_idx;
  p.prefix_lens = prefix_lens;
  p.extend_lens = extend_lens;
  p.batch = batch;
  p.page_size = page_size;
  p.out_loc = out_loc;
  p.out_loc_capacity = out_loc_capacity;
  p.status = status;
  return hip_status(launch_alloc_pages(p, static_cast<hipStream_t>(stream)));
}

msgl_status msgl_decode_graph_create(const msgl_kv_pool* pool, int32_t layer, const void* k,
                                     int64_t k_row_stride, const void* v, int64_t v_row_stride,
                                     const int32_t* out_loc, const void* q, int64_t q_row_stride,
                                     void* out, const int32_t* page_table,
                                     int32_t page_table_stride, const int32_t* table_idx,
                                     const int32_t* seq_lens, int32_t batch,
                                     int32_t num_qo_heads, int32_t max_seq_len, float sm_scale,
                                     void* workspace, size_t workspace_bytes,
                                     msgl_decode_graph** graph_out) {
  if (!graph_out) return MSGL_ERR_NULL;
  *graph_out = nullptr;
  msgl_status st = check_pool(pool, layer);
  if (st != MSGL_OK) return st;
  if (batch < 1) return MSGL_ERR_SHAPE;
  // checked mode copies device data to the host: not capturable
  if (env_on("MSGL_CHECK")) return MSGL_ERR_UNSUPPORTED;
  // the device query is made (and cached) outside the capture
  st = check_device();
  if (st != MSGL_OK) return st;
  hipStream_t cs = nullptr;
  if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) return MSGL_ERR_HIP;
  if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) {
    (void)hipStreamDestroy(cs);  // the capture error is the one reported
    return MSGL_ERR_HIP;
  }
  // the two calls validate every argument before they launch anything; a
  // validation error still ends the capture below
  st = msgl_store_kv(pool, layer, k, k_row_stride, v, v_row_stride, out_loc, batch, cs);
  if (st == MSGL_OK)
    st = msgl_paged_decode(pool, layer, q, q_row_stride, out, page_table, page_table_stride,
                           table_idx, seq_lens, batch, num_qo_heads, max_seq_len, sm_scale,
                           workspace, workspace_bytes, cs);
  hipGraph_t graph = nullptr;
  const hipError_t end = hipStreamEndCapture(cs, &graph);
  hipGraphExec_t exec = nullptr;
  if (st == MSGL_OK && end == hipSuccess && graph)
    st = hip_status(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0));
  else if (st == MSGL_OK)
    st = MSGL_ERR_HIP;
  // clean-up: a failure here leaves nothing to undo, and the status of the
  // capture (or of the instantiation) is the one reported
  if (graph) (void)hipGraphDestroy(graph);
  (void)hipStreamDestroy(cs);
  if (st != MSGL_OK) {
    if (exec) (void)hipGraphExecDestroy(exec);
    return st;
  }
  msgl_decode_graph* g = new (std::nothrow) msgl_decode_graph;
  if (!g) {
    (void)hipGraphExecDestroy(exec);
    return MSGL_ERR_HIP;
  }
  g->exec = exec;
  *graph_out = g;
  return MSGL_OK;
}

msgl_status msgl_decode_graph_launch(const msgl_decode_graph* graph, void* stream) {
  if (!graph || !graph->exec) return MSGL_ERR_NULL;
  return hip_status(hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream)));
}

msgl_status msgl_decode_graph_destroy(msgl_decode_graph* graph) {
  if (!graph) return MSGL_OK;
  const hipError_t e = graph->exec ? hipGraphExecDestroy(graph->exec) : hipSuccess;
  delete graph;
  return hip_status(e);
}

msgl_status msgl_decode_graph_runner_destroy(msgl_decode_graph_runner* runner) {
  if (!runner) return MSGL_OK;
  msgl_status st = MSGL_OK;
  for (int32_t i = 0; i < runner->count; ++i) {
    const msgl_status e = msgl_decode_graph_destroy(runner->graphs[i]);
    if (st == MSGL_OK) st = e;
  }
  delete runner;
  return st;
}

msgl_status msgl_decode_graph_runner_create(
    const msgl_kv_pool* pool, int32_t layer, const void* k, int64_t k_row_stride, const void* v,
    int64_t v_row_stride, const int32_t* out_loc, const void* q, int64_t q_row_stride, void* out,
    const int32_t* page_table, int32_t page_table_stride, const int32_t* table_idx,
    const int32_t* seq_lens, int32_t max_batch, int32_t num_qo_heads, int32_t max_seq_len,
    float sm_scale, void* workspace, size_t workspace_bytes, msgl_decode_graph_runner** runner_out) {
  if (!runner_out) return MSGL_ERR_NULL;
  *runner_out = nullptr;
  if (max_batch < 1) return MSGL_ERR_SHAPE;
  msgl_decode_graph_runner* r = new (std::nothrow) msgl_decode_graph_runner;
  if (!r) return MSGL_ERR_HIP;
  r->count = 0;
  for (int64_t s = 1;; s *= 2) {
    const int32_t size = static_cast<int32_t>(std::min<int64_t>(s, max_batch));
    msgl_decode_graph* g = nullptr;
    // each graph covers the first `size` rows of the same static buffers
    const msgl_status st = msgl_decode_graph_create(
        pool, layer, k, k_row_stride, v, v_row_stride, out_loc, q, q_row_stride, out, page_table,
        page_table_stride, table_idx, seq_lens, size, num_qo_heads, max_seq_len, sm_scale,
        workspace, workspace_bytes, &g);
    if (st != MSGL_OK) {
      msgl_decode_graph_runner_destroy(r);
      return st;
    }
    r->sizes[r->count] = size;
    r->graphs[r->count] = g;
    ++r->count;
    if (size == max_batch) break;
  }
  *runner_out = r;
  return MSGL_OK;
}

int32_t msgl_decode_graph_runner_pick(const msgl_decode_graph_runner* runner, int32_t batch) {
  if (!runner || batch < 1) return 0;
  for (int32_t i = 0; i < runner->count; ++i)
    if (runner->sizes[i] >= batch) return runner->sizes[i];
  return 0;
}

msgl_status msgl_decode_graph_runner_launch(const msgl_decode_graph_runner* runner, int32_t batch,
                                            void* stream) {
  if (!runner) return MSGL_ERR_NULL;
  for (int32_t i = 0; i < runner->count; ++i)
    if (batch >= 1 && runner->sizes[i] >= batch)
      return msgl_decode_graph_launch(runner->graphs[i], stream);
  return MSGL_ERR_SHAPE;
}

}  // extern "C"
