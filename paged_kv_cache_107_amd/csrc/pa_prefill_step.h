// Pieces shared by the two chunked-prefill kernels: prefill_mfma
// (pa_prefill.hip, a register ring of K/V tiles per wave) and
// prefill_mfma_lds (pa_prefill_lds.hip, tiles shared through LDS).  The
// step they both compute, the item order and the grid are described at the
// top of pa_prefill.hip.
#pragma once

#include <hip/hip_runtime.h>

#include "pa.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace prefill {

constexpr int kTile = 16;                   // keys per tile
constexpr float kRescaleSlack = 8.f;        // log2 units
constexpr float kMFloor = -1.0e30f;         // initial running maximum
constexpr int kLptSeqs = 4096;              // batches up to this size run longest first
constexpr int kLenClassShift = 9;           // length classes of 512 positions
constexpr int kClasses = 4 * 64;            // classes counted (longer ones share the top class)

// Score maxima: the IEEE maximum, which gfx950 does as v_maximum3_f32 on the
// MFMA results directly (fmaxf first quiets each operand with an extra
// instruction).  A NaN operand would propagate, but scores here are finite or
// already replaced by -inf where masked.
__device__ __forceinline__ float smax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// The P.V product over 32 keys (v_mfma_f32_16x16x32, both operands 8
// elements per lane), and acc + both 16-bit values of a word (a dot product
// with (1, 1)).
__device__ __forceinline__ f32x4 pv32(BF16, u32x4 v, u32x4 p, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v),
                                                 __builtin_bit_cast(bf16x8, p), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 pv32(F16, u32x4 v, u32x4 p, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, v),
                                                __builtin_bit_cast(f16x8, p), c, 0, 0, 0);
}
__device__ __forceinline__ float sum2(BF16, uint32_t w, float acc) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, w),
                                         __builtin_bit_cast(b2, 0x3F803F80u), acc, false);
}
__device__ __forceinline__ float sum2(F16, uint32_t w, float acc) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w), __builtin_bit_cast(h2, 0x3C003C00u),
                                acc, false);
}

__device__ __forceinline__ int clamp_ctx(const PrefillArgs& a, int i) {
  int ctx = a.context_lens[i];
  ctx = min(ctx, a.max_ctx);
  ctx = min(ctx, a.max_blocks << a.log2_bs);
  return ctx;
}

// The item (sequence i, query-block group zq) of workgroup item index k (Z
// groups per sequence): longest sequences first (length classes counted in
// LDS), a sequence's groups back to back within a class; batches above
// kLptSeqs in batch order.
// Every thread of the workgroup calls it (it has barriers).
template <int THREADS>
__device__ void pick_item(const PrefillArgs& a, int k, int Z, int& i, int& zq) {
  const int B = a.num_seqs;
  if (B <= kLptSeqs) {
    // Classes are counted in LDS; class C holds ranks [start(C), start(C) +
    // cnt(C)) with start(C) = sequences in longer classes, and items
    // [start * Z, (start + cnt) * Z), sequence by sequence.  The item's class is found
    // from the counts, then its sequence -- the j-th of the class in batch
    // order -- by one wave with ballots over 64 sequences at a time.
    __shared__ int s_cls[kLptSeqs], s_cnt[kClasses], s_pick[3];
    const int t = threadIdx.x;
    for (int c = t; c < kClasses; c += THREADS) s_cnt[c] = 0;
    __syncthreads();
    for (int u = t; u < B; u += THREADS) {
      const int c = min(max(clamp_ctx(a, u), 0) >> kLenClassShift, kClasses - 1);
      s_cls[u] = c;
      atomicAdd(&s_cnt[c], 1);
    }
    __syncthreads();
    // Wave 0: lane l holds the counts of classes 255 - 4l .. 252 - 4l (the
    // descending order), a wave-wide scan gives each class's first rank, and
    // the lane holding the item's rank finds its class; then the class's j-th
    // sequence is found with ballots.
    const int rr = k / Z;  // the item's rank
    if (wave_id() == 0) {
      const int lane = threadIdx.x % kWave;
      int cnt4[4], own = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        cnt4[e] = s_cnt[kClasses - 1 - (4 * lane + e)];
        own += cnt4[e];
      }
      int incl = own;  // inclusive scan over lanes
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        const int x = __shfl_up(incl, d, kWave);
        if (lane >= d) incl += x;
      }
      int first = incl - own;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (cnt4[e] > 0 && rr >= first && rr < first + cnt4[e]) {
          s_pick[0] = kClasses - 1 - (4 * lane + e);
          s_pick[1] = first;
        }
        first += cnt4[e];
      }
    }
    __syncthreads();
    const int cls = s_pick[0], first = s_pick[1], cnt = s_cnt[cls];
    const int off = k - first * Z;
    int j = off / Z;  // the j-th sequence of the class, in batch order
    zq = off - j * Z;
    if (wave_id() == 0) {
      const int lane = threadIdx.x % kWave;
      for (int base = 0; base < B; base += kWave) {
        const int u = base + lane;
        const uint64_t hit = __builtin_amdgcn_ballot_w64(u < B && s_cls[u] == cls);
        const int n = __builtin_popcountll(hit);
        if (j < n) {
          const uint64_t below = lane ? hit & (~0ull >> (64 - lane)) : 0ull;
          if (((hit >> lane) & 1ull) && __builtin_popcountll(below) == j) s_pick[2] = u;
          break;
        }
        j -= n;
      }
    }
    __syncthreads();
    i = s_pick[2];
  } else {
    i = k / Z;
    zq = k - i * Z;
  }
}

}  // namespace prefill

// Launches prefill_mfma_lds (16-bit pools).
pa_status launch_prefill_lds(const PrefillArgs& a, int dtype, hipStream_t st);

}  // namespace pa
