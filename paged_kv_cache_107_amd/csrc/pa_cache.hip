// KV-pool writes of the paged cache (gfx950): the new-token cache write and
// the copy-on-write block copy.  Both move raw 16-byte chunks (bit-exact).
//
//  * reshape_and_cache: decode appends the new token's K/V ("Lazy Allocation
//    与 Copy-on-Write 在 LLM 推理系统中的应用", section 2.1) into the slot the
//    block table gives (physical block slot / BS, offset slot % BS: "放下账簿，
//    打开源码", section "PagedAttention：虚实分离，按需取用").  One thread per
//    16-byte chunk of a (token, kv head) row; consecutive threads read
//    consecutive input bytes and write one contiguous pool row.  Into an
//    8-bit pool each 16-byte input chunk (8 values) becomes 8 E4M3 codes:
//    x * (1 / scale) in fp32, clamped to +-448, rounded to nearest even.
//  * copy_blocks: a writer's private copy of a shared block before its first
//    write ("Lazy Allocation 与 Copy-on-Write ...", section 4.4).  A block is
//    Hkv x BS rows, contiguous in the pool; each workgroup streams a slice of
//    one block of one pool.
//  * swap_blocks: a preempted sequence's blocks moved one by one between the
//    device pools and pinned host pools of the same block shape ("vLLM：把 KV
//    缓存当成虚拟内存", section "碎片从哪里来").  The same slicing as
//    copy_blocks, with the host side read or written directly over the host
//    link: many 16-byte accesses in flight per CU cover its latency.
#include <hip/hip_runtime.h>

#include "pa.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// Token and chunk of flat chunk index idx (32-bit division when the indices
// fit, which is every write but the very largest).
__device__ __forceinline__ void token_chunk(int64_t idx, int64_t total, int32_t per_token,
                                            int64_t& t, int32_t& c) {
  if (total <= 0x7FFFFFFF) {
    const uint32_t t32 = (uint32_t)idx / (uint32_t)per_token;
    t = t32;
    c = (int32_t)((uint32_t)idx - t32 * (uint32_t)per_token);
  } else {
    t = idx / per_token;
    c = (int32_t)(idx - t * per_token);
  }
}

__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const u32x4* __restrict__ k, const u32x4* __restrict__ v, const int64_t* __restrict__ slots,
    int64_t total_chunks, int32_t chunks_per_token, int32_t chunks_per_row, int32_t num_kv_heads,
    int32_t block_size, int64_t num_slots, u32x4* __restrict__ k_pool, u32x4* __restrict__ v_pool) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total_chunks) return;
  // the chunk's loads go out with its slot's, so a write waits for one
  // round trip to memory instead of two
  const u32x4 kc = k[idx], vc = v[idx];
  int64_t t;
  int32_t c;
  token_chunk(idx, total_chunks, chunks_per_token, t, c);
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;
  const int32_t h = c / chunks_per_row, cc = c - h * chunks_per_row;
  // block sizes are powers of two (the pool check admits 16 and 32)
  const int64_t blk = slot >> __builtin_ctz(block_size), off = slot & (block_size - 1);
  const int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * chunks_per_row + cc;
  k_pool[dst] = kc;
  v_pool[dst] = vc;
}

// 8 values of type E (one 16-byte chunk) -> 8 E4M3 codes of x * inv.
template <class E>
__device__ __forceinline__ uint2 quantize8(const u32x4& x, float inv) {
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a = lo16(E{}, x[j]) * inv, b = hi16(E{}, x[j]) * inv;
    w[j >> 1] = to_e4m3_pair(a, b, w[j >> 1], (j & 1) != 0);
  }
  return make_uint2(w[0], w[1]);
}

template <class E>
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(
    const u32x4* __restrict__ k, const u32x4* __restrict__ v, const int64_t* __restrict__ slots,
    int64_t total_chunks, int32_t chunks_per_token, int32_t chunks_per_row, int32_t num_kv_heads,
    int32_t block_size, int64_t num_slots, uint2* __restrict__ k_pool, uint2* __restrict__ v_pool,
    float k_inv, float v_inv) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total_chunks) return;
  const u32x4 kc = k[idx], vc = v[idx];
  int64_t t;
  int32_t c;
  token_chunk(idx, total_chunks, chunks_per_token, t, c);
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;
  const int32_t h = c / chunks_per_row, cc = c - h * chunks_per_row;
  // block sizes are powers of two (the pool check admits 16 and 32)
  const int64_t blk = slot >> __builtin_ctz(block_size), off = slot & (block_size - 1);
  const int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * chunks_per_row + cc;
  k_pool[dst] = quantize8<E>(kc, k_inv);
  v_pool[dst] = quantize8<E>(vc, v_inv);
}

__global__ __launch_bounds__(256) void copy_blocks_kernel(u32x4* __restrict__ k_pool,
                                                          u32x4* __restrict__ v_pool,
                                                          const int32_t* __restrict__ pairs,
                                                          int32_t num_blocks,
                                                          int64_t chunks_per_block) {
  const int32_t pr = blockIdx.y;
  const int32_t src = pairs[2 * pr], dst = pairs[2 * pr + 1];
  if ((unsigned)src >= (unsigned)num_blocks || (unsigned)dst >= (unsigned)num_blocks) return;
  u32x4* pool = blockIdx.z == 0 ? k_pool : v_pool;
  const u32x4* s = pool + (int64_t)src * chunks_per_block;
  u32x4* d = pool + (int64_t)dst * chunks_per_block;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks_per_block;
       c += (int64_t)gridDim.x * blockDim.x)
    d[c] = s[c];
}

__global__ __launch_bounds__(256) void swap_blocks_kernel(
    const u32x4* __restrict__ src_k, const u32x4* __restrict__ src_v, u32x4* __restrict__ dst_k,
    u32x4* __restrict__ dst_v, const int32_t* __restrict__ pairs, int32_t src_blocks,
    int32_t dst_blocks, int64_t chunks_per_block) {
  const int32_t pr = blockIdx.y;
  const int32_t src = pairs[2 * pr], dst = pairs[2 * pr + 1];
  if ((unsigned)src >= (unsigned)src_blocks || (unsigned)dst >= (unsigned)dst_blocks) return;
  const u32x4* s = (blockIdx.z == 0 ? src_k : src_v) + (int64_t)src * chunks_per_block;
  u32x4* d = (blockIdx.z == 0 ? dst_k : dst_v) + (int64_t)dst * chunks_per_block;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks_per_block;
       c += (int64_t)gridDim.x * blockDim.x)
    d[c] = s[c];
}

// Block-table upkeep of a decode step: one thread per new token; the token
// at position pos points its logical block at the block its slot lies in.
__global__ __launch_bounds__(256) void update_tables_kernel(
    const int64_t* __restrict__ slots, const int32_t* __restrict__ new_lens, int32_t num_seqs,
    int32_t n_tokens, int32_t log2_bs, int32_t* __restrict__ tables, int32_t max_blocks,
    int32_t* __restrict__ lens) {
  const int32_t per_seq = n_tokens > 0 ? n_tokens : 1;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)num_seqs * per_seq) return;
  const int32_t i = (int32_t)(idx / per_seq), t = (int32_t)(idx - (int64_t)i * per_seq);
  const int32_t len = new_lens[i];
  if (t == 0) lens[i] = len;
  if (n_tokens <= 0) return;
  const int64_t slot = slots[idx];
  const int64_t pos = (int64_t)len - n_tokens + t;
  if (slot < 0 || pos < 0) return;
  const int64_t j = pos >> log2_bs;
  if (j >= max_blocks) return;
  tables[(int64_t)i * max_blocks + j] = (int32_t)(slot >> log2_bs);
}

pa_status launch_update_tables(const int64_t* slots, const int32_t* new_lens, int32_t num_seqs,
                               int32_t n_tokens, int32_t log2_bs, int32_t* tables,
                               int32_t max_blocks, int32_t* lens, hipStream_t st) {
  const int64_t total = (int64_t)num_seqs * (n_tokens > 0 ? n_tokens : 1);
  const int64_t blocks = (total + 255) / 256;
  if (blocks == 0) return PA_OK;
  if (blocks > 0x7FFFFFFF) return PA_ERR_ARG;
  hipLaunchKernelGGL(update_tables_kernel, dim3((unsigned)blocks), dim3(256), 0, st, slots,
                     new_lens, num_seqs, n_tokens, log2_bs, tables, max_blocks, lens);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

static int elem_bytes(int dtype) { return dtype == PA_F32 ? 4 : 2; }

template <class E>
pa_status launch_fp8_write(const void* k, const void* v, const int64_t* slots, int64_t total,
                           int32_t chunks_per_token, int32_t chunks_per_row, void* k_pool,
                           void* v_pool, const pa_pool_desc& pool, hipStream_t st) {
  const int64_t blocks = (total + 255) / 256;
  if (blocks > 0x7FFFFFFF) return PA_ERR_ARG;
  hipLaunchKernelGGL((reshape_and_cache_fp8_kernel<E>), dim3((unsigned)blocks), dim3(256), 0, st,
                     static_cast<const u32x4*>(k), static_cast<const u32x4*>(v), slots, total,
                     chunks_per_token, chunks_per_row, pool.num_kv_heads, pool.block_size,
                     (int64_t)pool.num_blocks * pool.block_size, static_cast<uint2*>(k_pool),
                     static_cast<uint2*>(v_pool), 1.0f / pool.k_scale, 1.0f / pool.v_scale);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status launch_reshape_and_cache(const void* k, const void* v, const int64_t* slots,
                                   int32_t num_tokens, void* k_pool, void* v_pool,
                                   const pa_pool_desc& pool, hipStream_t st) {
  if (num_tokens == 0) return PA_OK;
  const int32_t chunks_per_row = pool.head_dim * elem_bytes(pool.dtype) / 16;
  const int32_t chunks_per_token = chunks_per_row * pool.num_kv_heads;
  const int64_t total = (int64_t)num_tokens * chunks_per_token;
  if (pool.kv_dtype == PA_KV_FP8_E4M3) {
    if (pool.dtype == PA_BF16)
      return launch_fp8_write<BF16>(k, v, slots, total, chunks_per_token, chunks_per_row, k_pool,
                                    v_pool, pool, st);
    if (pool.dtype == PA_F16)
      return launch_fp8_write<F16>(k, v, slots, total, chunks_per_token, chunks_per_row, k_pool,
                                   v_pool, pool, st);
    return PA_ERR_DTYPE;
  }
  const int64_t blocks = (total + 255) / 256;
  if (blocks > 0x7FFFFFFF) return PA_ERR_ARG;
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     static_cast<const u32x4*>(k), static_cast<const u32x4*>(v), slots, total,
                     chunks_per_token, chunks_per_row, pool.num_kv_heads, pool.block_size,
                     (int64_t)pool.num_blocks * pool.block_size, static_cast<u32x4*>(k_pool),
                     static_cast<u32x4*>(v_pool));
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status launch_copy_blocks(void* k_pool, void* v_pool, const pa_pool_desc& pool,
                             const int32_t* pairs, int32_t num_pairs, hipStream_t st) {
  if (num_pairs == 0) return PA_OK;
  const int64_t chunks_per_block = (int64_t)pool.num_kv_heads * pool.block_size * pool.head_dim *
                                   pool_elem_bytes(pool) / 16;
  const int64_t slices = (chunks_per_block + 255) / 256;
  const unsigned gx = (unsigned)(slices < 64 ? slices : 64);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(gx, (unsigned)num_pairs, 2), dim3(256), 0, st,
                     static_cast<u32x4*>(k_pool), static_cast<u32x4*>(v_pool), pairs,
                     pool.num_blocks, chunks_per_block);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status launch_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                             int32_t src_blocks, int32_t dst_blocks, const pa_pool_desc& pool,
                             const int32_t* pairs, int32_t num_pairs, hipStream_t st) {
  if (num_pairs == 0) return PA_OK;
  const int64_t chunks_per_block = (int64_t)pool.num_kv_heads * pool.block_size * pool.head_dim *
                                   pool_elem_bytes(pool) / 16;
  const int64_t slices = (chunks_per_block + 255) / 256;
  const unsigned gx = (unsigned)(slices < 64 ? slices : 64);
  hipLaunchKernelGGL(swap_blocks_kernel, dim3(gx, (unsigned)num_pairs, 2), dim3(256), 0, st,
                     static_cast<const u32x4*>(src_k), static_cast<const u32x4*>(src_v),
                     static_cast<u32x4*>(dst_k), static_cast<u32x4*>(dst_v), pairs, src_blocks,
                     dst_blocks, chunks_per_block);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace pa
