// Device-side helpers shared by the libpa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {

constexpr int kWave = 64;

// ------------------------------------------------------------- element types
// Storage types: the kernels move raw bits and convert explicitly.
struct F32 {
  using storage = uint32_t;
  static constexpr int bytes = 4;
};
struct F16 {
  using storage = uint16_t;
  static constexpr int bytes = 2;
};
struct BF16 {
  using storage = uint16_t;
  static constexpr int bytes = 2;
};

__device__ __forceinline__ float bits_to_float(F32, uint32_t b) { return __uint_as_float(b); }
__device__ __forceinline__ float bits_to_float(F16, uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}
__device__ __forceinline__ float bits_to_float(BF16, uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> element bits, round to nearest even.
__device__ __forceinline__ uint32_t float_to_bits(F32, float x) { return __float_as_uint(x); }
__device__ __forceinline__ uint32_t float_to_bits(F16, float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}
__device__ __forceinline__ uint32_t float_to_bits(BF16, float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;  // quiet NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two 16-bit elements of a 32-bit word as floats.
template <class E>
__device__ __forceinline__ float lo16(E e, uint32_t w) { return bits_to_float(e, w & 0xFFFFu); }
template <class E>
__device__ __forceinline__ float hi16(E e, uint32_t w) { return bits_to_float(e, w >> 16); }

// Element `i` of a 16-byte chunk (4 words) as float.
template <class E>
__device__ __forceinline__ float chunk_elem(E e, const uint4& c, int i) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  if constexpr (E::bytes == 4) {
    return bits_to_float(e, w[i]);
  } else {
    return (i & 1) ? hi16(e, w[i >> 1]) : lo16(e, w[i >> 1]);
  }
}

// ------------------------------------------------------------- vector types
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------- buffer loads
// A raw buffer descriptor over [base, base + bytes): loads at offsets past
// `bytes` return zeros and make no memory access (bytes = 0: every load).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kRsrcWord3 = 0x00020000;  // 32-bit data format, raw addressing

// `base` and `bytes` must be wave-uniform; they are moved to scalar registers
// so the descriptor is built with scalar instructions.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t v = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), kRsrcWord3);
}
__device__ __forceinline__ u32x4_t buffer_load16(rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
__device__ __forceinline__ u32x2 buffer_load8(rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0));
}

// ------------------------------------------------------------- status
// ORs kStatusBadBlock into the caller's status word when this wave met a
// table entry outside the pool inside an attended range (`bad`, uniform
// across the wave).  One lane does it, with a vector global atomic.
__device__ __forceinline__ void report_bad_block(int32_t* status, bool bad) {
  if (status != nullptr && bad && (threadIdx.x % kWave) == 0)
    __hip_atomic_fetch_or(status, kStatusBadBlock, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------- math
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

// ------------------------------------------------------------- cross-lane
// DPP controls (gfx9): quad_perm, row_mirror, row_half_mirror.
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float shfl_xor(float x, int mask) { return __shfl_xor(x, mask, kWave); }

// Sum over groups of N consecutive lanes (N = 8, 16, 32 or 64); every lane of
// a group ends with the group total.  Within a row of 16 the butterfly uses
// DPP: two quad exchanges, then the half-row and row mirrors pair each lane
// with a lane of the other half.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16 || N == 32 || N == 64, "group size");
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppRowMirror>(x);
  if constexpr (N >= 32) x += shfl_xor(x, 16);
  if constexpr (N >= 64) x += shfl_xor(x, 32);
  return x;
}

// Max / sum across lanes whose index differs only in bits >= log2(STRIDE)
// (i.e. over the 64 / STRIDE groups, lane-position-wise).
template <int STRIDE>
__device__ __forceinline__ float across_groups_max(float x) {
#pragma unroll
  for (int m = STRIDE; m < kWave; m <<= 1) x = fmaxf(x, shfl_xor(x, m));
  return x;
}
template <int STRIDE>
__device__ __forceinline__ float across_groups_sum(float x) {
#pragma unroll
  for (int m = STRIDE; m < kWave; m <<= 1) x += shfl_xor(x, m);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<kDppQuadXor1>(x));
  x = fmaxf(x, dpp<kDppQuadXor2>(x));
  x = fmaxf(x, dpp<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp<kDppRowMirror>(x));
  x = fmaxf(x, shfl_xor(x, 16));
  x = fmaxf(x, shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) { return group_sum<64>(x); }

// Wave index as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Wave-uniform loads through the constant address space become scalar loads:
// they are counted apart from the vector loads of a register ring, so the
// ring's waits stay exact.
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
__device__ __forceinline__ int scalar_load(const int32_t* p) {
  return *reinterpret_cast<const_i32_ptr>(reinterpret_cast<uintptr_t>(p));
}

// ------------------------------------------------------------- matrix cores
// The two products of a 16-token tile: qk = v_mfma_f32_16x16x32 (A and B 8
// elements per lane), pv = v_mfma_f32_16x16x16 (4 elements per lane);
// round16 rounds a probability to the 16-bit operand type.
template <class E>
struct Mfma;

template <>
struct Mfma<BF16> {
  static __device__ __forceinline__ f32x4 qk(u32x4 k, u32x4 q, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k),
                                                   __builtin_bit_cast(bf16x8, q), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 pv(u32x2 v, u32x2 p, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, v),
                                                     __builtin_bit_cast(i16x4, p), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t round16(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
  }
  // two probabilities rounded (RNE) and packed, the first in the low half
  static __device__ __forceinline__ uint32_t round16x2(float x, float y) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{x, y}, b2));
  }
};

template <>
struct Mfma<F16> {
  static __device__ __forceinline__ f32x4 qk(u32x4 k, u32x4 q, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, k),
                                                  __builtin_bit_cast(f16x8, q), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 pv(u32x2 v, u32x2 p, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, v),
                                                 __builtin_bit_cast(f16x4, p), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t round16(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  }
  static __device__ __forceinline__ uint32_t round16x2(float x, float y) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{x, y}, h2));
  }
};


// ------------------------------------------------------------- 8-bit pools
// Two E4M3 codes (the low or high 16 bits of w) -> two 16-bit operand values,
// packed low first.  Every E4M3 value is exactly a bf16 and an f16 value, so
// the widening is exact (scale operand 1).
template <class E>
__device__ __forceinline__ uint32_t widen2(uint32_t w, bool hi);
template <>
__device__ __forceinline__ uint32_t widen2<BF16>(uint32_t w, bool hi) {
  return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))
            : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}
template <>
__device__ __forceinline__ uint32_t widen2<F16>(uint32_t w, bool hi) {
  return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true))
            : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
}
// Eight codes in two words -> eight 16-bit values in the operand layout.
template <class E>
__device__ __forceinline__ u32x4 widen8(uint32_t w0, uint32_t w1) {
  return u32x4{widen2<E>(w0, false), widen2<E>(w0, true), widen2<E>(w1, false),
               widen2<E>(w1, true)};
}

// ------------------------------------------------------------- K/V tiles
// One 16-token tile of one kv head (head_dim 128) in the registers of lane
// (c16 = lane % 16, g4 = lane / 16), and the matrix-core operands built from
// it: k_op(s) is the A operand of k-step s of S^T = K . Q^T (K row c16, 8
// elements), v_row(r) holds V row 4 g4 + r, elements 8 c16 .. +7 (the
// source of the P.V product's A operands).  q_elem(s, g4) is where the q
// operand of k-step s starts, so that q and K agree on the order of the
// contraction.
//  * pools of the 16-bit operand type: k-step s takes elements 32 s + 8 g4
//    .. +7 (four 16-byte loads; a load instruction covers 64 contiguous bytes
//    of each row); V: four 16-byte loads.
//  * 8-bit pools: the lane loads bytes 16 g4 .. +15 and 64 + 16 g4 .. +15 of
//    its K row (two 16-byte loads), so k-step s takes elements 64 (s / 2) +
//    16 g4 + 8 (s % 2) .. +7; V: four 8-byte loads.  The codes are widened
//    when the operand is built.
template <class E, KvType KV>
struct KvTile;

template <class E>
struct KvTile<E, KvType::kSame> {
  using P = typename E::storage;                     // pool element
  static constexpr uint32_t kBytes = 16u * 128u * 2u;  // one tile of one kv head
  static constexpr uint32_t kRowBytes = kBytes / 16u;
  u32x4 k[4], v[4];
  static __device__ __forceinline__ int q_elem(int s, int g4) { return 32 * s + 8 * g4; }
  __device__ __forceinline__ void load(rsrc_t kr, rsrc_t vr, int c16, int g4) {
    const uint32_t ko = (uint32_t)(c16 * 128 + 8 * g4) * 2u;
    const uint32_t vo = (uint32_t)((4 * g4) * 128 + 8 * c16) * 2u;
#pragma unroll
    for (int s = 0; s < 4; ++s) k[s] = buffer_load16(kr, ko + 64u * s);
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = buffer_load16(vr, vo + 256u * r);
  }
  __device__ __forceinline__ u32x4 k_op(int s) const { return k[s]; }
  __device__ __forceinline__ u32x4 v_row(int r) const { return v[r]; }
};

template <class E>
struct KvTile<E, KvType::kFp8> {
  using P = uint8_t;
  static constexpr uint32_t kBytes = 16u * 128u;
  static constexpr uint32_t kRowBytes = kBytes / 16u;
  u32x4 k[2];
  u32x2 v[4];
  static __device__ __forceinline__ int q_elem(int s, int g4) {
    return 64 * (s >> 1) + 16 * g4 + 8 * (s & 1);
  }
  __device__ __forceinline__ void load(rsrc_t kr, rsrc_t vr, int c16, int g4) {
    const uint32_t ko = (uint32_t)(c16 * 128 + 16 * g4);
    const uint32_t vo = (uint32_t)((4 * g4) * 128 + 8 * c16);
    k[0] = buffer_load16(kr, ko);
    k[1] = buffer_load16(kr, ko + 64u);
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = buffer_load8(vr, vo + 128u * r);
  }
  __device__ __forceinline__ u32x4 k_op(int s) const {
    const u32x4& c = k[s >> 1];
    return (s & 1) ? widen8<E>(c[2], c[3]) : widen8<E>(c[0], c[1]);
  }
  __device__ __forceinline__ u32x4 v_row(int r) const { return widen8<E>(v[r][0], v[r][1]); }
};

// fp32 -> E4M3 code for a quantised cache write: the caller has already
// multiplied by 1 / scale; clamps to +-448, rounds to nearest even; NaN ->
// 0x7F.  Two values at a time into the low or high 16 bits of `old`.
__device__ __forceinline__ uint32_t to_e4m3_pair(float a, float b, uint32_t old, bool hi) {
  const float lim = 448.f;
  const bool na = a != a, nb = b != b;
  a = fminf(fmaxf(a, -lim), lim);
  b = fminf(fmaxf(b, -lim), lim);
  uint32_t r = hi ? (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, true)
                  : (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, false);
  const int sh = hi ? 16 : 0;
  if (na) r = (r & ~(0xFFu << sh)) | (0x7Fu << sh);
  if (nb) r = (r & ~(0xFFu << (sh + 8))) | (0x7Fu << (sh + 8));
  return r;
}

}  // namespace pa

