// Internal interfaces between the libpa C ABI (pa_api.hip) and the kernel
// launchers.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// Everything a decode kernel needs, passed by value.
struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;
  float2* ws_ml;  // [B][Hq][max_parts] (max, sum), log2 units
  float* ws_o;    // [B][Hq][max_parts][D] unnormalised outputs
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t num_blocks;
  int32_t log2_bs;
  int32_t max_blocks;
  int32_t max_ctx;
  int32_t part_tokens;
  int32_t max_parts;
  float scale_log2;  // softmax scale times log2(e)
};

bool mfma_supports(int dtype, int head_dim, int group);
bool valu_supports(int dtype, int head_dim, int group);
pa_status launch_decode_partition(const DecodeArgs& a, int dtype, int head_dim, bool use_mfma,
                                  hipStream_t st);
pa_status launch_decode_reduce(const DecodeArgs& a, int dtype, int head_dim, hipStream_t st);

pa_status launch_reshape_and_cache(const void* k, const void* v, const int64_t* slots,
                                   int32_t num_tokens, void* k_pool, void* v_pool,
                                   const pa_pool_desc& pool, hipStream_t st);
pa_status launch_copy_blocks(void* k_pool, void* v_pool, const pa_pool_desc& pool,
                             const int32_t* pairs, int32_t num_pairs, hipStream_t st);

}  // namespace pa
