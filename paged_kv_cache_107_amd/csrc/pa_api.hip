// C ABI of libpa: argument validation and dispatch for the decode, cache-write
// and block-copy kernels.  Every check runs on the host before any launch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>

#include "pa.h"
#include "pa_internal.h"

// Scratch memory of pa_decode_noalloc, for callers that cannot allocate: the
// split-K workspace of one call lives here instead of in a caller buffer.
// Each device the library runs on holds its own copy until the process ends.
// In host code `scratch` only names the symbol; its device address on the
// current device comes from hipGetSymbolAddress (scratch_on_current_device).
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int32_t kAbiVersion = 6;
constexpr int32_t kDefaultPartition = 512;
constexpr int32_t kMaxPartition = 4096;
constexpr int32_t kMaxGridYZ = 65535;

std::atomic<int32_t> g_decode_path{PA_PATH_AUTO};
std::atomic<int32_t> g_decode_balance{1};
std::atomic<int32_t> g_prefill_path{PA_PREFILL_AUTO};

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int32_t elem_bytes(int32_t dtype) { return dtype == PA_F32 ? 4 : 2; }

inline int32_t ilog2(int32_t x) {
  int32_t r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

pa_status check_pool(const pa_pool_desc* pool) {
  if (!pool) return PA_ERR_ARG;
  if (pool->dtype != PA_F32 && pool->dtype != PA_F16 && pool->dtype != PA_BF16)
    return PA_ERR_DTYPE;
  if (pool->kv_dtype != PA_KV_SAME && pool->kv_dtype != PA_KV_FP8_E4M3) return PA_ERR_DTYPE;
  if (pool->kv_dtype == PA_KV_FP8_E4M3) {
    if (pool->dtype == PA_F32) return PA_ERR_DTYPE;
    if (pool->head_dim != 128) return PA_ERR_SHAPE;
    if (!std::isfinite(pool->k_scale) || !std::isfinite(pool->v_scale) || !(pool->k_scale > 0.f) ||
        !(pool->v_scale > 0.f))
      return PA_ERR_ARG;
  }
  if (pool->num_blocks <= 0 || pool->num_kv_heads <= 0) return PA_ERR_ARG;
  if (pool->block_size != 16 && pool->block_size != 32) return PA_ERR_SHAPE;
  if (pool->head_dim != 64 && pool->head_dim != 128) return PA_ERR_SHAPE;
  return PA_OK;
}

inline int32_t max_parts_of(int32_t max_ctx, int32_t part_tokens) {
  return max_ctx > 0 ? (max_ctx + part_tokens - 1) / part_tokens : 1;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Grid split workspace: (max, sum) pairs first, then the unnormalised
// outputs, one per (sequence, q head, partition); none with one partition.
size_t ws_ml_bytes(int32_t b, int32_t hq, int32_t parts) {
  return align256((size_t)b * hq * parts * sizeof(float2));
}
size_t grid_ws_bytes(int32_t b, int32_t hq, int32_t d, int32_t max_ctx, int32_t part_tokens) {
  const int32_t parts = max_parts_of(max_ctx, part_tokens);
  if (parts <= 1) return 0;
  return ws_ml_bytes(b, hq, parts) + (size_t)b * hq * parts * d * sizeof(float);
}

// Stream split workspace: the merge record of each wave rank
// [kStreamMaxWaves][4], then (max, sum) and the unnormalised outputs for
// slot-heads (b * hkv + kStreamMaxWaves) * g.
size_t stream_heads(int32_t b, int32_t hkv, int32_t g) {
  return ((size_t)b * hkv + pa::kStreamMaxWaves) * g;
}
constexpr size_t kStreamOwnerBytes = pa::kStreamMaxWaves * 4 * sizeof(int32_t);
size_t stream_ml_bytes(int32_t b, int32_t hkv, int32_t g) {
  return align256(stream_heads(b, hkv, g) * sizeof(float2));
}
// The balance header (kept between calls) comes first.
size_t stream_ws_bytes(int32_t b, int32_t hkv, int32_t g, int32_t d) {
  return pa::kStreamBalanceBytes + kStreamOwnerBytes + stream_ml_bytes(b, hkv, g) +
         stream_heads(b, hkv, g) * d * sizeof(float);
}

constexpr size_t kStaticScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up once per
// device with that device current.
pa_status scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return PA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return PA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return PA_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

struct Prepared {
  pa::DecodeArgs args;
  int32_t dtype;
  pa::KvType kv;
  int32_t head_dim;
  pa::DecodeKernel kernel;
};

inline pa::KvType kv_type(const pa_pool_desc* pool) {
  return pool->kv_dtype == PA_KV_FP8_E4M3 ? pa::KvType::kFp8 : pa::KvType::kSame;
}

// Small single-partition passes: every sequence fits one partition and the
// batch has at most kSmallPassTilesPerWave tiles per stream wave even if
// every sequence had the longest length.  The grid split then needs no
// reduce pass, and the hardware's workgroup dispatch balances it; the stream
// split's fixed costs (its prologue, the reduce pass) are a large part of
// such a pass.  Measured (bf16/f16, one call = partition + reduce): 128 CoW
// branches 50 against 55 us; 32 sequences up to 2048 tokens 31 against
// 40 us; 64 sequences of G = 1 up to 512 tokens 22 against 30 us; at 256
// tiles per wave the stream split wins (256 sequences up to 2048 tokens: 180
// against 188 us).
constexpr int64_t kSmallPassTilesPerWave = 80;
bool small_single_partition_pass(const pa_pool_desc* pool, int32_t num_seqs,
                                 int32_t max_context_len, int32_t partition_tokens) {
  if (max_context_len > partition_tokens) return false;
  const int64_t waves = pa::stream_waves();
  const int64_t tiles = (int64_t)num_seqs * pool->num_kv_heads * ((max_context_len + 15) / 16);
  return waves > 0 && tiles <= kSmallPassTilesPerWave * waves;
}

// The kernel pa_decode runs for this shape under the current path setting.
// 8-bit pools run on the matrix-core kernels only (any G up to 16).
pa_status choose_kernel(const pa_pool_desc* pool, int32_t group, int32_t num_seqs,
                        int32_t max_context_len, int32_t partition_tokens,
                        pa::DecodeKernel* k) {
  const bool mfma = pa::mfma_supports(pool->dtype, pool->head_dim, group);
  const bool stream = mfma && pa::stream_supports(num_seqs, pool->num_kv_heads, max_context_len);
  const int32_t path = g_decode_path.load();
  if (kv_type(pool) == pa::KvType::kFp8) {
    if (!mfma || path == PA_PATH_VALU) return PA_ERR_SHAPE;
    const bool small = path == PA_PATH_AUTO &&
                       small_single_partition_pass(pool, num_seqs, max_context_len, partition_tokens);
    *k = stream && path != PA_PATH_MFMA_GRID && !small ? pa::DecodeKernel::kMfmaStream
                                                       : pa::DecodeKernel::kMfmaGrid;
    return PA_OK;
  }
  if (path == PA_PATH_VALU) {
    if (!pa::valu_supports(pool->dtype, pool->head_dim, group)) return PA_ERR_SHAPE;
    *k = pa::DecodeKernel::kValu;
  } else if (path == PA_PATH_MFMA_GRID) {
    if (!mfma) return PA_ERR_SHAPE;
    *k = pa::DecodeKernel::kMfmaGrid;
  } else if (path == PA_PATH_MFMA) {
    if (!mfma) return PA_ERR_SHAPE;
    *k = stream ? pa::DecodeKernel::kMfmaStream : pa::DecodeKernel::kMfmaGrid;
  } else if (mfma) {  // PA_PATH_AUTO on a matrix-core shape, any G
    *k = stream && !small_single_partition_pass(pool, num_seqs, max_context_len, partition_tokens)
             ? pa::DecodeKernel::kMfmaStream
             : pa::DecodeKernel::kMfmaGrid;
  } else {
    if (!pa::valu_supports(pool->dtype, pool->head_dim, group)) return PA_ERR_SHAPE;
    *k = pa::DecodeKernel::kValu;
  }
  return PA_OK;
}

pa_status prepare_decode(const void* q, const void* k_pool, const void* v_pool,
                         const pa_pool_desc* pool, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                         int32_t num_q_heads, int32_t max_context_len, float scale,
                         int32_t sliding_window, void* out, void* workspace,
                         size_t workspace_bytes, int32_t partition_tokens, int32_t* status,
                         Prepared* pr, bool use_scratch = false) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_seqs > kMaxGridYZ || num_q_heads <= 0 || max_blocks_per_seq < 0 ||
      max_context_len < 0)
    return PA_ERR_ARG;
  if (max_parts_of(max_context_len, partition_tokens ? partition_tokens : kDefaultPartition) >
      kMaxGridYZ)
    return PA_ERR_ARG;
  if (!std::isfinite(scale) || sliding_window < 0) return PA_ERR_ARG;
  if (pool->num_kv_heads > kMaxGridYZ || num_q_heads > kMaxGridYZ) return PA_ERR_ARG;
  if (num_q_heads % pool->num_kv_heads != 0) return PA_ERR_SHAPE;
  const int32_t group = num_q_heads / pool->num_kv_heads;
  if (partition_tokens == 0) partition_tokens = kDefaultPartition;
  if (partition_tokens < 16 || partition_tokens > kMaxPartition || partition_tokens % 16 != 0 ||
      partition_tokens % pool->block_size != 0)
    return PA_ERR_ARG;
  pa::DecodeKernel kernel;
  st = choose_kernel(pool, group, num_seqs, max_context_len, partition_tokens, &kernel);
  if (st != PA_OK) return st;
  if (num_seqs == 0) {
    *pr = Prepared{};
    pr->args.num_seqs = 0;
    return PA_OK;
  }
  if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !out) return PA_ERR_ARG;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out))
    return PA_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(block_tables) & 3u) || (reinterpret_cast<uintptr_t>(context_lens) & 3u) ||
      (reinterpret_cast<uintptr_t>(status) & 3u))
    return PA_ERR_ARG;
  const bool stream = kernel == pa::DecodeKernel::kMfmaStream;
  const int32_t max_parts = max_parts_of(max_context_len, partition_tokens);
  const size_t need = stream ? stream_ws_bytes(num_seqs, pool->num_kv_heads, group, pool->head_dim)
                             : grid_ws_bytes(num_seqs, num_q_heads, pool->head_dim,
                                             max_context_len, partition_tokens);
  if (use_scratch) {  // the static scratch replaces the caller's workspace
    if (need > kStaticScratchBytes) return PA_ERR_SCRATCH;
    workspace = nullptr;
    workspace_bytes = 0;
    if (need > 0) {
      st = scratch_on_current_device(&workspace);
      if (st != PA_OK) return st;
      workspace_bytes = kStaticScratchBytes;
    }
  }
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return PA_ERR_ARG;

  pa::DecodeArgs& a = pr->args;
  a = pa::DecodeArgs{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.out = out;
  char* ws = static_cast<char*>(workspace);
  if (stream) {
    a.ws_balance = reinterpret_cast<pa::StreamBalance*>(ws);
    ws += pa::kStreamBalanceBytes;
    a.balance = g_decode_balance.load();
    a.ws_owner = reinterpret_cast<int32_t*>(ws);
    a.ws_ml = reinterpret_cast<float2*>(ws + kStreamOwnerBytes);
    a.ws_o = reinterpret_cast<float*>(ws + kStreamOwnerBytes +
                                      stream_ml_bytes(num_seqs, pool->num_kv_heads, group));
    a.stream_waves = pa::stream_waves();
    a.xcds = pa::device_xcds();
    if (a.stream_waves <= 0 || a.stream_waves > pa::kStreamMaxWaves) return PA_ERR_HIP;
  } else if (need > 0) {
    a.ws_ml = reinterpret_cast<float2*>(ws);
    a.ws_o = reinterpret_cast<float*>(ws + ws_ml_bytes(num_seqs, num_q_heads, max_parts));
  }
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.group = group;
  a.num_blocks = pool->num_blocks;
  a.log2_bs = ilog2(pool->block_size);
  a.max_blocks = max_blocks_per_seq;
  a.max_ctx = max_context_len;
  a.part_tokens = partition_tokens;
  a.max_parts = max_parts;
  const bool fp8 = kv_type(pool) == pa::KvType::kFp8;
  a.scale_log2 = scale * 1.4426950408889634f * (fp8 ? pool->k_scale : 1.f);
  a.window = sliding_window;
  a.v_scale = fp8 ? pool->v_scale : 1.f;
  a.status = status;
  pr->dtype = pool->dtype;
  pr->kv = kv_type(pool);
  pr->head_dim = pool->head_dim;
  pr->kernel = kernel;
  return PA_OK;
}

// Whether the partition pass leaves work for the reduce pass.
bool needs_reduce(const Prepared& pr) {
  return pr.kernel == pa::DecodeKernel::kMfmaStream || pr.args.max_parts > 1;
}

}  // namespace

// The device address of a pinned host range [host, host + bytes): both ends
// must lie in pinned host memory mapped for the device, at device addresses
// bytes - 1 apart.  PA_ERR_ARG otherwise (pageable memory would fault).
static pa_status mapped_host_range(void* host, int64_t bytes, void** dev_out) {
  char* first = static_cast<char*>(host);
  char* last = first + bytes - 1;
  void* dev[2] = {nullptr, nullptr};
  char* ends[2] = {first, last};
  for (int e = 0; e < 2; ++e) {
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, ends[e]) != hipSuccess) {
      (void)hipGetLastError();
      return PA_ERR_ARG;
    }
    if (attr.type != hipMemoryTypeHost) return PA_ERR_ARG;
    if (hipHostGetDevicePointer(&dev[e], ends[e], 0) != hipSuccess || !dev[e]) {
      (void)hipGetLastError();
      return PA_ERR_ARG;
    }
  }
  if (static_cast<char*>(dev[1]) - static_cast<char*>(dev[0]) != bytes - 1) return PA_ERR_ARG;
  *dev_out = dev[0];
  return PA_OK;
}

extern "C" {

int32_t pa_abi_version(void) { return kAbiVersion; }

const char* pa_status_string(int32_t s) {
  switch (s) {
    case PA_OK: return "PA_OK";
    case PA_ERR_ARG: return "PA_ERR_ARG";
    case PA_ERR_DTYPE: return "PA_ERR_DTYPE";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE";
    case PA_ERR_OOM: return "PA_ERR_OOM";
    case PA_ERR_REFCOUNT: return "PA_ERR_REFCOUNT";
    case PA_ERR_NOT_FOUND: return "PA_ERR_NOT_FOUND";
    case PA_ERR_HIP: return "PA_ERR_HIP";
    case PA_ERR_SWAPPED: return "PA_ERR_SWAPPED";
    case PA_ERR_SCRATCH: return "PA_ERR_SCRATCH";
    default: return "PA_ERR_UNKNOWN";
  }
}

int32_t pa_set_decode_path(int32_t path) {
  if (path != PA_PATH_AUTO && path != PA_PATH_VALU && path != PA_PATH_MFMA &&
      path != PA_PATH_MFMA_GRID)
    return -1;
  return g_decode_path.exchange(path);
}

int32_t pa_set_decode_balance(int32_t on) {
  if (on != 0 && on != 1) return -1;
  return g_decode_balance.exchange(on);
}

int32_t pa_set_prefill_path(int32_t path) {
  if (path != PA_PREFILL_AUTO && path != PA_PREFILL_LDS && path != PA_PREFILL_DMA) return -1;
  return g_prefill_path.exchange(path);
}

size_t pa_decode_workspace_bytes(const pa_pool_desc* pool, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t max_context_len,
                                 int32_t partition_tokens) {
  if (check_pool(pool) != PA_OK || num_seqs <= 0 || num_q_heads <= 0 || max_context_len < 0)
    return 0;
  if (num_q_heads % pool->num_kv_heads != 0) return 0;
  if (partition_tokens == 0) partition_tokens = kDefaultPartition;
  if (partition_tokens <= 0) return 0;
  const int32_t group = num_q_heads / pool->num_kv_heads;
  size_t need = grid_ws_bytes(num_seqs, num_q_heads, pool->head_dim, max_context_len,
                              partition_tokens);
  if (pa::mfma_supports(pool->dtype, pool->head_dim, group) &&
      pa::stream_supports(num_seqs, pool->num_kv_heads, max_context_len))
    need = std::max(need, stream_ws_bytes(num_seqs, pool->num_kv_heads, group, pool->head_dim));
  return need;
}

pa_status pa_decode_partition(const void* q, const void* k_pool, const void* v_pool,
                              const pa_pool_desc* pool, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* context_lens,
                              int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                              float scale, int32_t sliding_window, void* out, void* workspace,
                              size_t workspace_bytes, int32_t partition_tokens, int32_t* status,
                              void* hip_stream) {
  Prepared pr;
  pa_status st = prepare_decode(q, k_pool, v_pool, pool, block_tables, max_blocks_per_seq,
                                context_lens, num_seqs, num_q_heads, max_context_len, scale,
                                sliding_window, out, workspace, workspace_bytes, partition_tokens,
                                status, &pr);
  if (st != PA_OK || pr.args.num_seqs == 0) return st;
  return pa::launch_decode_partition(pr.args, pr.dtype, pr.kv, pr.head_dim, pr.kernel,
                                     static_cast<hipStream_t>(hip_stream));
}

pa_status pa_decode_reduce(const void* q, const void* k_pool, const void* v_pool,
                           const pa_pool_desc* pool, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                           float scale, int32_t sliding_window, void* out, void* workspace,
                           size_t workspace_bytes, int32_t partition_tokens, int32_t* status,
                           void* hip_stream) {
  Prepared pr;
  pa_status st = prepare_decode(q, k_pool, v_pool, pool, block_tables, max_blocks_per_seq,
                                context_lens, num_seqs, num_q_heads, max_context_len, scale,
                                sliding_window, out, workspace, workspace_bytes, partition_tokens,
                                status, &pr);
  if (st != PA_OK || pr.args.num_seqs == 0 || !needs_reduce(pr)) return st;
  return pa::launch_decode_reduce(pr.args, pr.dtype, pr.head_dim, pr.kernel,
                                  static_cast<hipStream_t>(hip_stream));
}

pa_status pa_decode(const void* q, const void* k_pool, const void* v_pool,
                    const pa_pool_desc* pool, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                    int32_t num_q_heads, int32_t max_context_len, float scale,
                    int32_t sliding_window, void* out, void* workspace,
                    size_t workspace_bytes, int32_t partition_tokens, int32_t* status,
                    void* hip_stream) {
  Prepared pr;
  pa_status st = prepare_decode(q, k_pool, v_pool, pool, block_tables, max_blocks_per_seq,
                                context_lens, num_seqs, num_q_heads, max_context_len, scale,
                                sliding_window, out, workspace, workspace_bytes, partition_tokens,
                                status, &pr);
  if (st != PA_OK || pr.args.num_seqs == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  st = pa::launch_decode_partition(pr.args, pr.dtype, pr.kv, pr.head_dim, pr.kernel, s);
  if (st != PA_OK || !needs_reduce(pr)) return st;
  return pa::launch_decode_reduce(pr.args, pr.dtype, pr.head_dim, pr.kernel, s);
}

pa_status pa_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                            const pa_pool_desc* pool, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                            float scale, int32_t sliding_window, void* out,
                            int32_t partition_tokens, int32_t* status, void* hip_stream) {
  Prepared pr;
  pa_status st = prepare_decode(q, k_pool, v_pool, pool, block_tables, max_blocks_per_seq,
                                context_lens, num_seqs, num_q_heads, max_context_len, scale,
                                sliding_window, out, nullptr, 0, partition_tokens, status, &pr,
                                /*use_scratch=*/true);
  if (st != PA_OK || pr.args.num_seqs == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  st = pa::launch_decode_partition(pr.args, pr.dtype, pr.kv, pr.head_dim, pr.kernel, s);
  if (st != PA_OK || !needs_reduce(pr)) return st;
  return pa::launch_decode_reduce(pr.args, pr.dtype, pr.head_dim, pr.kernel, s);
}

pa_status pa_prefill(const void* q, const void* k_pool, const void* v_pool,
                     const pa_pool_desc* pool, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* query_start,
                     const int32_t* context_lens, int32_t num_seqs, int32_t num_tokens,
                     int32_t num_q_heads, int32_t max_query_len, int32_t max_context_len,
                     float scale, int32_t sliding_window, void* out, int32_t* status,
                     void* hip_stream) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_seqs > kMaxGridYZ || num_tokens < 0 || num_q_heads <= 0 ||
      max_blocks_per_seq < 0 || max_query_len < 0 || max_context_len < 0)
    return PA_ERR_ARG;
  if (!std::isfinite(scale) || sliding_window < 0) return PA_ERR_ARG;
  if (pool->num_kv_heads > kMaxGridYZ || num_q_heads > kMaxGridYZ) return PA_ERR_ARG;
  if (num_q_heads % pool->num_kv_heads != 0) return PA_ERR_SHAPE;
  const int32_t group = num_q_heads / pool->num_kv_heads;
  if (!pa::prefill_supports(pool->dtype, pool->head_dim, group)) return PA_ERR_SHAPE;
  if (pa::prefill_query_blocks(max_query_len, group) > kMaxGridYZ * 4) return PA_ERR_ARG;
  if (num_seqs == 0 || num_tokens == 0 || max_query_len == 0) return PA_OK;
  if (!q || !k_pool || !v_pool || !block_tables || !query_start || !context_lens || !out)
    return PA_ERR_ARG;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(block_tables) & 3u) ||
      (reinterpret_cast<uintptr_t>(query_start) & 3u) ||
      (reinterpret_cast<uintptr_t>(context_lens) & 3u) ||
      (reinterpret_cast<uintptr_t>(status) & 3u))
    return PA_ERR_ARG;
  pa::PrefillArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.query_start = query_start;
  a.context_lens = context_lens;
  a.out = out;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.group = group;
  a.num_blocks = pool->num_blocks;
  a.log2_bs = ilog2(pool->block_size);
  a.max_blocks = max_blocks_per_seq;
  a.max_ctx = max_context_len;
  a.max_query = max_query_len;
  const bool fp8 = kv_type(pool) == pa::KvType::kFp8;
  a.scale_log2 = scale * 1.4426950408889634f * (fp8 ? pool->k_scale : 1.f);
  a.window = sliding_window;
  a.v_scale = fp8 ? pool->v_scale : 1.f;
  a.status = status;
  return pa::launch_prefill(a, pool->dtype, kv_type(pool), g_prefill_path.load(),
                            static_cast<hipStream_t>(hip_stream));
}

pa_status pa_reshape_and_cache(const void* k, const void* v, const int64_t* slot_mapping,
                               int32_t num_tokens, void* k_pool, void* v_pool,
                               const pa_pool_desc* pool, void* hip_stream) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return PA_ERR_ARG;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_pool || !v_pool) return PA_ERR_ARG;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_pool) || !aligned16(v_pool) ||
      (reinterpret_cast<uintptr_t>(slot_mapping) & 7u))
    return PA_ERR_ARG;
  return pa::launch_reshape_and_cache(k, v, slot_mapping, num_tokens, k_pool, v_pool, *pool,
                                      static_cast<hipStream_t>(hip_stream));
}

pa_status pa_update_tables(const int64_t* slot_mapping, const int32_t* new_lens, int32_t num_seqs,
                           int32_t tokens_per_seq, int32_t block_size, int32_t* block_tables,
                           int32_t max_blocks_per_seq, int32_t* context_lens, void* hip_stream) {
  if (num_seqs < 0 || tokens_per_seq < 0 || max_blocks_per_seq < 0 || block_size <= 0 ||
      block_size > 65536 || (block_size & (block_size - 1)) != 0)
    return PA_ERR_ARG;
  if (num_seqs == 0) return PA_OK;
  if (!new_lens || !context_lens || (tokens_per_seq > 0 && !slot_mapping) ||
      (tokens_per_seq > 0 && max_blocks_per_seq > 0 && !block_tables))
    return PA_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(slot_mapping) & 7u) ||
      (reinterpret_cast<uintptr_t>(new_lens) & 3u) ||
      (reinterpret_cast<uintptr_t>(block_tables) & 3u) ||
      (reinterpret_cast<uintptr_t>(context_lens) & 3u))
    return PA_ERR_ARG;
  return pa::launch_update_tables(slot_mapping, new_lens, num_seqs, tokens_per_seq,
                                  ilog2(block_size), block_tables, max_blocks_per_seq,
                                  context_lens, static_cast<hipStream_t>(hip_stream));
}

pa_status pa_copy_blocks(void* k_pool, void* v_pool, const pa_pool_desc* pool,
                         const int32_t* pairs, int32_t num_pairs, void* hip_stream) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (num_pairs < 0 || num_pairs > kMaxGridYZ) return PA_ERR_ARG;
  if (num_pairs == 0) return PA_OK;
  if (!k_pool || !v_pool || !pairs) return PA_ERR_ARG;
  if (!aligned16(k_pool) || !aligned16(v_pool) || (reinterpret_cast<uintptr_t>(pairs) & 3u))
    return PA_ERR_ARG;
  return pa::launch_copy_blocks(k_pool, v_pool, *pool, pairs, num_pairs,
                                static_cast<hipStream_t>(hip_stream));
}

pa_status pa_probe_tile_reads(const void* pool, const void* pool2, uint64_t pool_bytes,
                              const uint32_t* tile_offsets, int64_t num_tiles, int32_t tile_bytes,
                              int32_t num_waves, uint32_t* out, int32_t out_len, int32_t* waves,
                              void* hip_stream) {
  if (num_waves < 0 || num_waves > (1 << 24) || num_waves % 4 != 0) return PA_ERR_ARG;
  const int w = num_waves > 0 ? num_waves : pa::stream_waves();
  if (w <= 0) return PA_ERR_HIP;
  if (waves) *waves = w;
  if (num_tiles < 0 || num_tiles >= (1ll << 31) || pool_bytes == 0 || pool_bytes >= (1ull << 32) ||
      (tile_bytes != 1024 && tile_bytes != 2048 && tile_bytes != 4096) || out_len < w)
    return PA_ERR_ARG;
  if (!pool || !out || (num_tiles > 0 && !tile_offsets)) return PA_ERR_ARG;
  if (!aligned16(pool) || !aligned16(pool2) || (reinterpret_cast<uintptr_t>(out) & 3u) ||
      (reinterpret_cast<uintptr_t>(tile_offsets) & 3u))
    return PA_ERR_ARG;
  return pa::launch_probe_reads(pool, pool2, (uint32_t)pool_bytes, tile_offsets, num_tiles,
                                tile_bytes, out, w, static_cast<hipStream_t>(hip_stream));
}

pa_status pa_swap_blocks(void* k_pool, void* v_pool, void* k_host, void* v_host,
                         int32_t num_host_blocks, const pa_pool_desc* pool, const int32_t* pairs,
                         int32_t num_pairs, int32_t direction, void* hip_stream) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (num_pairs < 0 || num_pairs > kMaxGridYZ || num_host_blocks <= 0) return PA_ERR_ARG;
  if (direction != PA_SWAP_OUT && direction != PA_SWAP_IN) return PA_ERR_ARG;
  if (num_pairs == 0) return PA_OK;
  if (!k_pool || !v_pool || !k_host || !v_host || !pairs) return PA_ERR_ARG;
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_host) || !aligned16(v_host) ||
      (reinterpret_cast<uintptr_t>(pairs) & 3u))
    return PA_ERR_ARG;
  const int64_t block_bytes = (int64_t)pool->num_kv_heads * pool->block_size * pool->head_dim *
                              pa::pool_elem_bytes(*pool);
  void* k_dev = nullptr;
  void* v_dev = nullptr;
  st = mapped_host_range(k_host, (int64_t)num_host_blocks * block_bytes, &k_dev);
  if (st != PA_OK) return st;
  st = mapped_host_range(v_host, (int64_t)num_host_blocks * block_bytes, &v_dev);
  if (st != PA_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (direction == PA_SWAP_OUT)
    return pa::launch_swap_blocks(k_pool, v_pool, k_dev, v_dev, pool->num_blocks,
                                  num_host_blocks, *pool, pairs, num_pairs, s);
  return pa::launch_swap_blocks(k_dev, v_dev, k_pool, v_pool, num_host_blocks, pool->num_blocks,
                                *pool, pairs, num_pairs, s);
}

}  // extern "C"
