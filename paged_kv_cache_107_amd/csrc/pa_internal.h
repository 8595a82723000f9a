// Internal interfaces between the libpa C ABI (pa_api.hip) and the kernel
// launchers.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// Everything a decode kernel needs, passed by value.
// Stream split limits: the sequence table lives in LDS, and the wave count
// (one 4-wave workgroup per CU of a 256-CU part) bounds the workspace.
constexpr int kStreamMaxSeqs = 4096;
constexpr int kStreamMaxWaves = 1024;

struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;
  // Split-K state, (max, sum) in log2 units and unnormalised outputs.  Grid
  // split: [B][Hq][max_parts] entries.  Stream split: [slot][G] entries for
  // slot < B * Hkv + stream_waves, plus ws_owner [stream_waves][4], the merge
  // record of each wave rank.
  float2* ws_ml;
  float* ws_o;
  int32_t* ws_owner;
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
  float scale_log2;      // softmax scale times log2(e) (times k_scale for 8-bit pools)
  int32_t stream_waves;  // waves of the stream split's grid
  int32_t window;        // sliding window in positions, 0 = none
  float v_scale;         // output factor: v_scale for 8-bit pools, else 1
  int32_t* status;       // caller's status word (kStatusBadBlock is ORed in), or null
  struct StreamBalance* ws_balance;  // stream split: the balance state, else null
  int32_t balance;       // stream split: cut the tile order by the measured rates
  int32_t xcds;          // stream split: dies (XCCs) the workgroups are dealt over, 1..8
};

// Balance of the stream split, kept between calls in the first
// kStreamBalanceBytes of a stream workspace.  The flat tile order is cut into
// one chunk per XCD; with weights, chunk x covers tiles [T cum[x] / 2^16,
// T cum[x + 1] / 2^16).  A partition pass records each chunk's tile count,
// and each wave the time it took (100 MHz ticks) in its own slot of
// wave_dur (plain stores: no atomics on shared words); the next reduce
// pass's extra workgroup takes each chunk's slowest wave and turns the
// record into the cut of the next call, with each chunk's share moved
// halfway towards its measured rate (left alone when the chunks ended within
// 1/64 of each other).  A workspace whose magic does not match starts from
// the even cut.
struct StreamBalance {
  uint32_t magic;    // kBalanceMagic when the fields below are valid
  uint32_t stamped;  // tiles and wave_dur hold a partition pass's record
  uint32_t pad[2];
  uint32_t cum[12];  // cum[0..8]: the cut, cum[0] = 0, cum[8] = 2^16
  uint32_t tiles[8];
  uint32_t pad2[40];
  uint32_t wave_dur[kStreamMaxWaves];  // by wave rank
};
constexpr size_t kStreamBalanceBytes = 256 + 4 * kStreamMaxWaves;
static_assert(sizeof(StreamBalance) <= kStreamBalanceBytes, "balance header");

// Bit of the caller's status word: a table entry inside an attended range
// named a block outside [0, num_blocks).
constexpr int32_t kStatusBadBlock = 1;

// Decode kernel families.
enum class DecodeKernel {
  kValu,        // vector ALU, one workgroup per (sequence, kv head, partition)
  kMfmaGrid,    // matrix cores, same grid
  kMfmaStream,  // matrix cores, flat tile order split evenly over the waves
};


// Pool element types the kernels are built for: the activation dtype itself,
// or 8-bit E4M3 codes (matrix-core kernels only).
enum class KvType { kSame, kFp8 };

bool mfma_supports(int dtype, int head_dim, int group);
bool valu_supports(int dtype, int head_dim, int group);
bool stream_supports(int num_seqs, int num_kv_heads, int max_ctx);
int stream_waves();  // on the current device; 0 if it cannot be queried
// The tile read probe (pa_probe.hip): `waves` waves (a multiple of 4) read
// tiles [n r / waves, n (r + 1) / waves) each, from pool and (if not null)
// pool2 at the same offsets.
pa_status launch_probe_reads(const void* pool, const void* pool2, uint32_t pool_bytes,
                             const uint32_t* offs, int64_t n, int tile_bytes, uint32_t* out,
                             int waves, hipStream_t st);
int device_xcds();   // XCCs of the current device, 1..8 (8 if it cannot be queried)
pa_status launch_decode_partition(const DecodeArgs& a, int dtype, KvType kv, int head_dim,
                                  DecodeKernel k, hipStream_t st);
pa_status launch_decode_reduce(const DecodeArgs& a, int dtype, int head_dim, DecodeKernel k,
                               hipStream_t st);

// Chunked prefill: sequence i's query rows are query_start[i] ..
// query_start[i+1] - 1, its chunk tokens at positions ctx_i - n_i .. ctx_i - 1.
struct PrefillArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* query_start;
  const int32_t* context_lens;
  void* out;
  int32_t num_seqs;
  int32_t num_tokens;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t num_blocks;
  int32_t log2_bs;
  int32_t max_blocks;
  int32_t max_ctx;
  int32_t max_query;
  float scale_log2;  // softmax scale times log2(e) (times k_scale for 8-bit pools)
  int32_t window;    // sliding window in positions, 0 = none
  float v_scale;     // output factor: v_scale for 8-bit pools, else 1
  int32_t* status;   // caller's status word, or null
};

bool prefill_supports(int dtype, int head_dim, int group);
int prefill_query_blocks(int max_query_len, int group);  // per sequence, grid bound
pa_status launch_prefill(const PrefillArgs& a, int dtype, KvType kv, int path, hipStream_t st);

// Pool element bytes for a valid descriptor.
inline int pool_elem_bytes(const pa_pool_desc& pool) {
  return pool.kv_dtype == PA_KV_FP8_E4M3 ? 1 : pool.dtype == PA_F32 ? 4 : 2;
}

pa_status launch_reshape_and_cache(const void* k, const void* v, const int64_t* slots,
                                   int32_t num_tokens, void* k_pool, void* v_pool,
                                   const pa_pool_desc& pool, hipStream_t st);
pa_status launch_update_tables(const int64_t* slots, const int32_t* new_lens, int32_t num_seqs,
                               int32_t n_tokens, int32_t log2_bs, int32_t* tables,
                               int32_t max_blocks, int32_t* lens, hipStream_t st);
pa_status launch_copy_blocks(void* k_pool, void* v_pool, const pa_pool_desc& pool,
                             const int32_t* pairs, int32_t num_pairs, hipStream_t st);
pa_status launch_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                             int32_t src_blocks, int32_t dst_blocks, const pa_pool_desc& pool,
                             const int32_t* pairs, int32_t num_pairs, hipStream_t st);

}  // namespace pa
