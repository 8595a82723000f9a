// Paged chunked-prefill attention for gfx950.
//
// A prefill step runs a chunk of a prompt's tokens through attention after
// writing their K/V into the cache; a long prompt is cut into chunks that run
// between decode steps (page "附录：Lazy Allocation 与 Copy-on-Write 在 LLM 推理
// 系统中的应用" §2.1; page "vLLM：把 KV 缓存当成虚拟内存", section "KV 的体积从哪来，
// 页表如何把它切开", which also notes that prefill is bound by compute and decode
// by KV bandwidth).  Sequence i's chunk holds its tokens at positions
// ctx_i - n_i .. ctx_i - 1; each attends to every earlier position of its
// sequence and to itself (the autoregressive rule of the same §2.1).  K/V
// rows are found through the block table as in decode.
//
// Two kernel designs share the grid, the item order and the walk below:
// the direct-to-LDS kernels, the default (prefill_dma on 16-bit pools,
// prefill_dma8 on 8-bit ones: tiles loaded straight into LDS, 32x32x16
// products), and prefill_mfma_lds on request (tiles staged through
// registers, 16x16x32 products); each is described above its code.  In both, the G query heads of a kv head and
// 32 / G consecutive chunk tokens make a wave's 32 query rows, keys are
// walked 32 at a time (two 16-key tiles), steps at and past the rows' first
// position are masked per element, and each lane keeps the softmax state of
// its query column with the decode kernel's lazy rescale (the running
// maximum starts at a finite floor, so a step has no branch between the
// rescale test and the P.V product).
//
// With a sliding window of W positions a row at position p attends only
// positions p - W + 1 .. p.  8-bit pools are widened exactly to the 16-bit
// operand type in LDS (prefill_dma8) or on the way into it
// (prefill_mfma_lds); the scales fold into the score factor and the
// output factor.
//
// Grid: kv head x, then a flat item index k over (sequence, query-block
// group z); group z takes query blocks nqb-1-4z .. nqb-4-4z of its sequence
// (one per wave), the heaviest first.  A workgroup's work grows with its
// sequence's length, so the items run longest sequence first: each
// workgroup ranks the batch by length class (512 positions) with counts in
// LDS (up to kLptSeqs sequences); short sequences then fill the tail instead
// of long sequences' last groups starting late.  Within a class a
// sequence's groups run back to back, so the workgroups running together on
// an XCD share few sequences and re-read their K/V from that XCD's L2.
// Larger batches run in batch order.  The kv heads of an item are
// neighbouring ids, so each XCD serves one kv head of every sequence.
#include <hip/hip_runtime.h>

#include "pa.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kTile = 16;                   // keys per tile
constexpr float kRescaleSlack = 8.f;        // log2 units
constexpr float kMFloor = -1.0e30f;         // initial running maximum
constexpr int kLptSeqs = 4096;              // batches up to this size run longest first
constexpr int kLenClassShift = 9;           // length classes of 512 positions
constexpr int kClasses = 4 * 64;            // classes counted (longer ones share the top class)
constexpr int kPickRanges = 1024;           // batches up to this size keep query ranges and lengths in LDS

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
// kLptSeqs in batch order.  Given s_qs and s_ctx, batches of up to
// kPickRanges sequences also leave every query range (s_qs[0 .. B]) and
// clamped length (s_ctx) there, read in the same pass as the lengths.
// Every thread of the workgroup calls it (it has barriers).
template <int THREADS>
__device__ void pick_item_in(const PrefillArgs& a, int k, int Z, int& i, int& zq,
                             uint8_t* s_cls, int* s_cnt, int* s_pick, int* s_qs = nullptr,
                             int* s_ctx = nullptr) {
  const int B = a.num_seqs;
  if (B <= kLptSeqs) {
    // Classes are counted in LDS; class C holds ranks [start(C), start(C) +
    // cnt(C)) with start(C) = sequences in longer classes, and items
    // [start * Z, (start + cnt) * Z), sequence by sequence.  The item's class is found
    // from the counts, then its sequence -- the j-th of the class in batch
    // order -- by one wave with ballots over 64 sequences at a time.
    const int t = threadIdx.x;
    for (int c = t; c < kClasses; c += THREADS) s_cnt[c] = 0;
    __syncthreads();
    const bool keep = s_qs != nullptr && B <= kPickRanges;
    for (int u = t; u < B; u += THREADS) {
      // all three loads in flight together
      const int raw = a.context_lens[u];
      const int qsu = keep ? a.query_start[u] : 0;
      const int qsb = keep && u == B - 1 ? a.query_start[B] : 0;
      const int cu = min(min(raw, a.max_ctx), a.max_blocks << a.log2_bs);
      const int c = min(max(cu, 0) >> kLenClassShift, kClasses - 1);
      s_cls[u] = (uint8_t)c;
      atomicAdd(&s_cnt[c], 1);
      if (keep) {
        s_ctx[u] = cu;
        s_qs[u] = qsu;
        if (u == B - 1) s_qs[B] = qsb;
      }
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
    const int cls = s_pick[0], first = s_pick[1];
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

template <int THREADS>
__device__ void pick_item(const PrefillArgs& a, int k, int Z, int& i, int& zq) {
  __shared__ uint8_t s_cls[kLptSeqs];  // length class of each sequence (< kClasses)
  __shared__ int s_cnt[kClasses], s_pick[3];
  pick_item_in<THREADS>(a, k, Z, i, zq, s_cls, s_cnt, s_pick);
}

// Register-staged kernel (prefill_mfma_lds).  A wave's 32 query rows are
// taken as two groups of 16; each group is the 16 columns of the decode
// kernel's tile products (S^T = K . Q^T with v_mfma_f32_16x16x32), so one K/V
// tile feeds both groups' products, and with 32 keys per step the P.V
// product also runs on the double-rate v_mfma_f32_16x16x32 (O^T += V^T .
// P^T).  The K/V tiles of a step are shared through LDS.  Four
// waves of 32 query rows each (two 16-column groups) take the 128 / G chunk
// tokens of one item, and each 32-key step's two K/V tiles are read from
// memory once per workgroup into a ring of three LDS buffers, one barrier per
// step, three steps ahead.  Wave w loads K pieces 2 w and 2 w + 1 (1 KiB
// each, in KvTile's layout) and rows 2 (w % 2), 2 (w % 2) + 1 of every
// four-row group of V tile w / 2, which it stores already permuted into the
// P.V product's A operands, so the byte permutes run once per workgroup, not
// once per wave.  Every wave runs every step of the workgroup's walk (keys
// 0 .. the item's last position), computing only the steps its own rows
// reach.  Two workgroups share a CU (two waves per SIMD) and, with a barrier
// each, run out of step: one's softmax overlaps the other's products.
// On 8-bit pools the loads carry the E4M3 codes, widened as they are stored.
// With a sliding window of W positions (WIN) the walk starts at the window
// of the item's earliest row, each wave computes only the steps its rows'
// windows reach, and keys below a row's window are masked per element.
constexpr int kLdsWaves = 4;
constexpr int kLdsThreads = kLdsWaves * kWave;
constexpr int kLdsGroups = 2;
constexpr int kLdsRows = 16 * kLdsGroups;  // query rows per wave
constexpr int kLdsBufs = 3;
constexpr int kLdsKPieces = 8;             // 1 KiB K pieces per step: tile-major, then k-step

template <class E, KvType KV, bool WIN>
__global__ __launch_bounds__(kLdsThreads) __attribute__((amdgpu_waves_per_eu(2))) void prefill_mfma_lds(PrefillArgs a) {
  constexpr int D = 128;
  using S = typename E::storage;
  using Tile = KvTile<E, KV>;
  using P = typename Tile::P;  // pool element: 16-bit value or E4M3 code
  __shared__ u32x4 s_k[kLdsBufs][kLdsKPieces][kWave];
  __shared__ u32x4 s_vw[kLdsBufs][8][kWave];  // A operands of the 8 P.V products
  __shared__ int s_ok[kLdsBufs][2];             // the step's tiles had blocks in the pool
  const int g = blockIdx.x;
  const int Z = gridDim.y;
  const int k = (int)blockIdx.y + Z * (int)blockIdx.z;
  int i, zq;
  pick_item<kLdsThreads>(a, k, Z, i, zq);
  const int G = a.group, QT = kLdsRows / G;  // chunk tokens per wave
  const int qa = a.query_start[i], qb = a.query_start[i + 1];
  if (qa < 0 || qb > a.num_tokens || qb <= qa) return;  // the whole workgroup
  const int n = qb - qa, nq = min(n, a.max_query);
  const int nqb = ceil_div(nq, QT);
  const int top = nqb - 1 - kLdsWaves * zq;  // the item's latest query block
  if (top < 0) return;                       // the whole workgroup
  const int w = wave_id();
  const int lane = threadIdx.x % kWave;
  const int c16 = lane & 15, g4 = lane >> 4;
  const int kswap = (g4 & 1) << 1;
  const int ctx = clamp_ctx(a, i);
  // the workgroup's walk: keys [0, kend_wg), in 32-key steps
  const int kend_wg = ctx - n + min(top * QT + QT, nq);
  // this wave's block (none when blk < 0)
  const int blk = top - w;
  const int tok0 = blk * QT, ntok = blk >= 0 ? min(QT, nq - tok0) : 0;
  const int pos0 = ctx - n + tok0;
  const int kend = blk >= 0 ? pos0 + ntok : 0;
  S* out = reinterpret_cast<S*>(a.out);

  int lim[kLdsGroups], row[kLdsGroups];
  bool live[kLdsGroups];
#pragma unroll
  for (int q = 0; q < kLdsGroups; ++q) {
    const int col = q * 16 + c16, tl = col / G, h = col - tl * G;
    live[q] = tl < ntok && pos0 + tl >= 0;
    lim[q] = live[q] ? pos0 + tl : kend - 1;
    row[q] = tl < ntok ? (qa + tok0 + tl) * a.num_q_heads + g * G + h : -1;
  }
  if (kend_wg <= 0) {  // every position of the item negative: zero rows
#pragma unroll
    for (int q = 0; q < kLdsGroups; ++q)
      if (row[q] >= 0)
        for (int d = 8 * g4; d < D; d += 32) *reinterpret_cast<u32x4*>(out + (size_t)row[q] * D + d) = u32x4{0, 0, 0, 0};
    return;  // the whole workgroup
  }
  const bool mine = kend > 0;  // this wave has keys to attend

  u32x4 qv[kLdsGroups][4];
#pragma unroll
  for (int q = 0; q < kLdsGroups; ++q) {
    const S* qrow = reinterpret_cast<const S*>(a.q) + (size_t)max(row[q], 0) * D;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qv[q][s] = row[q] >= 0 ? *reinterpret_cast<const u32x4*>(qrow + Tile::q_elem(s, g4))
                             : u32x4{0, 0, 0, 0};
  }
  const float c = fabsf(a.scale_log2), inv_c = 1.f / c;
  if (a.scale_log2 < 0.f) {
#pragma unroll
    for (int q = 0; q < kLdsGroups; ++q)
#pragma unroll
      for (int s = 0; s < 4; ++s) qv[q][s] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
  }

  const int bs_mask = (1 << a.log2_bs) - 1;
  const size_t head_stride = (size_t)D << a.log2_bs;
  const size_t block_stride = head_stride * a.num_kv_heads;
  const int32_t* table = a.block_tables + (size_t)i * a.max_blocks;
  const P* kbase0 = reinterpret_cast<const P*>(a.k_pool) + (size_t)g * head_stride;
  const P* vbase0 = reinterpret_cast<const P*>(a.v_pool) + (size_t)g * head_stride;
  const int ntiles = ceil_div(kend_wg, kTile);
  const int nsteps = ceil_div(ntiles, 2);
  const int unmasked = max(pos0, 0);
  // With a window: the walk starts at the step holding the first key of the
  // item's earliest row's window; this wave's rows reach back to kbeg.
  const int W = WIN ? a.window : 0;
  const int st_begin =
      WIN ? max(max(ctx - n + max(top - (kLdsWaves - 1), 0) * QT, 0) - W + 1, 0) / (2 * kTile) : 0;
  const int kbeg = WIN ? max(unmasked - W + 1, 0) : 0;

  // tile t of the walk: its block id when inside the pool, else -1
  auto block_of = [&](int t) __attribute__((always_inline)) -> int {
    if (t >= ntiles) return -1;
    const int b = scalar_load(table + ((t * kTile) >> a.log2_bs));
    return (unsigned)b < (unsigned)a.num_blocks ? b : -1;
  };
  // Loads of step st: wave w takes K pieces 2 w, 2 w + 1 (piece j: tile
  // j / 4, k-step j % 4) and its two V rows of each four-row group of tile
  // w / 2 (rows past the sequence read as zeros).
  struct Stage {
    u32x4 x0, x1, x2, x3;
  };
  // The block id each wave needs for its next step, read one step
  // ahead (tile 2 st + tw of step st).
  const int tw = w >> 1;
  int next_b = block_of(2 * st_begin + tw);
  // Key order within a tile: K operand row i holds key krow(i), which swaps
  // the row pairs (4a, 4a + 1) and (4a + 2, 4a + 3) for odd a.  S^T row
  // 4 g4 + r is then key 4 g4 + (r ^ kswap), and the V words of odd lane
  // groups are stored pair-swapped to match, so the two halves of a wave's
  // 4-byte V-operand stores fall on different LDS banks.
  const int krow = c16 ^ ((c16 >> 1) & 2);
  // ok: the wave's tile of the step had a block inside the pool
  auto gload = [&](int st, int& ok) __attribute__((always_inline)) -> Stage {
    Stage r = {};
    const int b = next_b;
    next_b = block_of(2 * (st + 1) + tw);
    ok = b >= 0;
    const int t = 2 * st + tw;
    const size_t off = b >= 0 ? (size_t)b * block_stride + (size_t)((t * kTile) & bs_mask) * D : 0;
    // K pieces 2 w and 2 w + 1: tile w / 2, k-steps 2 (w % 2) and 2 (w % 2) + 1
    const rsrc_t ks = make_rsrc(kbase0 + off, b >= 0 ? Tile::kBytes : 0u);
    // V rows 4 g4 + 2 (w % 2) and the next, dims 8 c16 .. 8 c16 + 7
    const uint32_t bytes = b >= 0 ? (uint32_t)min(kTile, ctx - t * kTile) * Tile::kRowBytes : 0u;
    const rsrc_t vs = make_rsrc(vbase0 + off, bytes);
    if constexpr (KV == KvType::kFp8) {
      // codes as loaded (KvTile<E, kFp8>'s k-slot order), widened when stored
      r.x0 = buffer_load16(ks, (uint32_t)(krow * 128 + 16 * g4) + 64u * (w & 1));
      const uint32_t vlo = (uint32_t)(4 * g4 * 128 + 8 * c16) + 256u * (w & 1);
      const u32x2 v0 = buffer_load8(vs, vlo), v1 = buffer_load8(vs, vlo + 128u);
      r.x2 = u32x4{v0[0], v0[1], v1[0], v1[1]};
    } else {
      const uint32_t klo = (uint32_t)(krow * 128 + 8 * g4) * 2u + 128u * (w & 1);
      r.x0 = buffer_load16(ks, klo);
      r.x1 = buffer_load16(ks, klo + 64u);
      const uint32_t vlo = (uint32_t)(4 * g4 * 128 + 8 * c16) * 2u + 512u * (w & 1);
      r.x2 = buffer_load16(vs, vlo);
      r.x3 = buffer_load16(vs, vlo + 256u);
    }
    return r;
  };
  auto lwrite = [&](int st, const Stage& r, int ok) __attribute__((always_inline)) {
    const int bf = st % kLdsBufs;
    u32x4 k0 = r.x0, k1 = r.x1, v0 = r.x2, v1 = r.x3;
    if constexpr (KV == KvType::kFp8) {
      k0 = widen8<E>(r.x0[0], r.x0[1]);
      k1 = widen8<E>(r.x0[2], r.x0[3]);
      v0 = widen8<E>(r.x2[0], r.x2[1]);
      v1 = widen8<E>(r.x2[2], r.x2[3]);
    }
    s_k[bf][2 * w][lane] = k0;
    s_k[bf][2 * w + 1][lane] = k1;
    if ((w & 1) == 0 && lane == 0) s_ok[bf][w >> 1] = ok;
    // Word 2 (w / 2) + (w % 2 ^ g4 % 2) of P.V operand e (words 0, 1: the
    // first tile's keys, 2, 3: the second's) pairs element e of the lane's 8
    // in the two rows (the key order of krow).
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      reinterpret_cast<uint32_t*>(&s_vw[bf][e][lane])[2 * (w >> 1) + ((w ^ g4) & 1)] =
          __builtin_amdgcn_perm(v1[e >> 1], v0[e >> 1], sel);
    }
  };

  float m[kLdsGroups], l[kLdsGroups];
  f32x4 o[kLdsGroups][8];
#pragma unroll
  for (int q = 0; q < kLdsGroups; ++q) {
    m[q] = kMFloor;
    l[q] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[q][e] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // One 32-key step from LDS buffer st % 3.
  auto compute = [&](int st) __attribute__((always_inline)) {
    const int k0 = 2 * st * kTile;
    const int bf = st % kLdsBufs;
    const bool oka = uni(s_ok[bf][0]) != 0, okb = uni(s_ok[bf][1]) != 0;
    if (!oka && !okb) return;
    u32x4 vw[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) vw[e] = s_vw[bf][e][lane];
    const bool masked =
        k0 + 2 * kTile - 1 > unmasked || (WIN && k0 < kend - W) || !oka || !okb;
    float sv[kLdsGroups][8];
    {
      u32x4 ka[4], kb[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        ka[s] = s_k[bf][s][lane];
        kb[s] = s_k[bf][4 + s][lane];
      }
      // A wave issuing matrix products takes issue priority over the other
      // workgroup's wave on its SIMD, whose vector instructions then fill
      // the cycles the products leave free.
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int q = 0; q < kLdsGroups; ++q) {
        f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) sa = Mfma<E>::qk(ka[s], qv[q][s], sa);
#pragma unroll
        for (int s = 0; s < 4; ++s) sb = Mfma<E>::qk(kb[s], qv[q][s], sb);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sv[q][r] = sa[r];
          sv[q][4 + r] = sb[r];
        }
      }
      __builtin_amdgcn_s_setprio(0);
    }
    if (masked) {
#pragma unroll
      for (int q = 0; q < kLdsGroups; ++q)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int key = k0 + (j < 4 ? 0 : kTile) + 4 * g4 + ((j & 3) ^ kswap);
          if (key > lim[q] || (WIN && key <= lim[q] - W) || !(j < 4 ? oka : okb))
            sv[q][j] = neg_inf();
        }
    }
    float mt[kLdsGroups];
    bool over = false;
#pragma unroll
    for (int q = 0; q < kLdsGroups; ++q) {
      mt[q] = smax(smax(smax(sv[q][0], sv[q][1]), smax(sv[q][2], sv[q][3])),
                   smax(smax(sv[q][4], sv[q][5]), smax(sv[q][6], sv[q][7])));
      over |= mt[q] > (m[q] + kRescaleSlack) * inv_c;
    }
    if (__builtin_amdgcn_ballot_w64(over)) {
#pragma unroll
      for (int q = 0; q < kLdsGroups; ++q) {
        float x = smax(mt[q], shfl_xor(mt[q], 16));
        x = smax(x, shfl_xor(x, 32));
        const float mn = smax(m[q], x * c);
        const float alpha = fast_exp2(m[q] - mn);
        l[q] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[q][e] *= alpha;
        m[q] = mn;
      }
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int q = 0; q < kLdsGroups; ++q) {
      float pf[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) pf[j] = fast_exp2(__builtin_fmaf(sv[q][j], c, -m[q]));
      const u32x4 pw = {Mfma<E>::round16x2(pf[0], pf[1]), Mfma<E>::round16x2(pf[2], pf[3]),
                        Mfma<E>::round16x2(pf[4], pf[5]), Mfma<E>::round16x2(pf[6], pf[7])};
      l[q] = sum2(E{}, pw[3], sum2(E{}, pw[2], sum2(E{}, pw[1], sum2(E{}, pw[0], l[q]))));
#pragma unroll
      for (int e = 0; e < 8; ++e) o[q][e] = pv32(E{}, vw[e], pw, o[q][e]);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // The ring: step st's pieces go global -> registers three steps ahead, in
  // three register stages (step k in stage k % 3), and registers -> LDS one
  // step ahead; the write to LDS waits only for its own stage's loads, and
  // the barrier after it makes the step visible to every wave and frees the
  // buffer written next.  All waves run the same steps, so every barrier is
  // reached by the whole workgroup.
  // this wave computes step st: its rows reach keys [kbeg, kend)
  auto runs = [&](int st) __attribute__((always_inline)) {
    return mine && st * 2 * kTile < kend && (!WIN || (st + 1) * 2 * kTile > kbeg);
  };
  const int s0 = st_begin;
  int ok0 = 0, ok1 = 0, ok2 = 0;
  Stage r0 = gload(s0, ok0), r1 = gload(s0 + 1, ok1), r2 = gload(s0 + 2, ok2);
  lwrite(s0, r0, ok0);
  __syncthreads();
  r0 = gload(s0 + 3, ok0);
  for (int st = s0; st < nsteps; st += 3) {
    lwrite(st + 1, r1, ok1);
    __syncthreads();
    r1 = gload(st + 4, ok1);
    if (runs(st)) compute(st);
    if (st + 1 >= nsteps) break;
    lwrite(st + 2, r2, ok2);
    __syncthreads();
    r2 = gload(st + 5, ok2);
    if (runs(st + 1)) compute(st + 1);
    if (st + 2 >= nsteps) break;
    lwrite(st + 3, r0, ok0);
    __syncthreads();
    r0 = gload(st + 6, ok0);
    if (runs(st + 2)) compute(st + 2);
  }

#pragma unroll
  for (int q = 0; q < kLdsGroups; ++q) {
    const float lsum = across_groups_sum<16>(l[q]);
    if (row[q] < 0) continue;
    const float inv = live[q] && lsum > 0.f ? a.v_scale / lsum : 0.f;
    S* dst = out + (size_t)row[q] * D + 32 * g4;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint32_t b[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        b[e] = Mfma<E>::round16x2(o[q][2 * e][r] * inv, o[q][2 * e + 1][r] * inv);
      *reinterpret_cast<u32x4*>(dst + 8 * r) = u32x4{b[0], b[1], b[2], b[3]};
    }
  }
  // Table entries outside the pool among the blocks some row of the item
  // attends (keys [kfirst, kend_wg)): reported to the caller's status word.
  // Checked after the walk, from the table alone, so the walk is unchanged.
  if (a.status != nullptr) {
    const int kfirst =
        WIN ? max(max(ctx - n + max(top - (kLdsWaves - 1), 0) * QT, 0) - W + 1, 0) : 0;
    bool bad = false;
    for (int j = (kfirst >> a.log2_bs) + (int)threadIdx.x; j <= ((kend_wg - 1) >> a.log2_bs);
         j += kLdsThreads)
      bad |= (unsigned)table[j] >= (unsigned)a.num_blocks;
    report_bad_block(a.status, __builtin_amdgcn_ballot_w64(bad) != 0);
  }
}

// ----------------------------------------------------------------------------
// Kernel for 16-bit pools: the step's K/V tiles go from memory straight into
// LDS (direct-to-LDS buffer loads: no register staging, no LDS stores), the
// products run on v_mfma_f32_32x32x16, and the P.V product's V^T operands
// come out of LDS transposed (ds_read_b64_tr_b16), so no byte permutes run.
//
// A wave owns 32 query rows, the 32 columns of S^T = K . Q^T; a step is 32
// keys (two 16-key tiles), so S^T is one 32 x 32 product (8 MFMAs over
// head_dim) and O^T += V^T . P^T is four 32-row d-tiles x two 16-key k-steps
// (8 MFMAs).  The rows of the K operand are permuted (key pi(m) in row m:
// bits 2 and 3 of m swapped) so that the S^T result a lane holds -- 16 keys
// of its own query column -- is in the order the P^T operand takes: value
// v = key 16 (v / 8) + 8 (lane / 32) + v % 8.  Each lane keeps the softmax
// state of its column (shared with its partner lane ^ 32) with the lazy
// rescale of the decode kernel.
//
// LDS: a ring of three stages of [K 32 x 128 | V 32 x 128] 16-bit rows.
// Every operand read is one of two per-lane base addresses plus an
// immediate, with no bank conflicts, and every 1 KiB load is four whole
// rows of one tile (contiguous in the pool).  A load fills 64 slots of 16
// bytes; inside such a 4-row piece a row's 16-byte chunk c sits at slot
// 4 (4 (c / 4) + r) + ((c % 4) ^ tau(r)): each row's 64-byte chunk groups
// stay contiguous (one per lane quad), and tau flips one chunk bit by row
// bit 1.  V pieces are packed; the four K pieces of a tile start at slots 0,
// 136, 66 and 202 (0, 8, 2 and 10 modulo 16), so the 16 rows of a K operand
// read, which share a chunk, land on 16 distinct bank groups (8 for each
// half of the lanes, should the LDS serve 128 bytes per cycle), as do the 4
// rows x 4 chunks of a transposed V read.  A workgroup's four waves load one
// step (four 1 KiB loads per wave) two steps ahead, with one barrier per
// step.  The operand reads are plain LDS loads of distinct stage arrays, so
// the compiler waits only for loads into the stage it reads.
//
// Three workgroups share a CU (three waves per SIMD: 49.5 KiB of LDS and at
// most 170 VGPRs each; the item choice's LDS scratch borrows the third
// stage): a wave's step is a chain of dependent phases (barrier, loads,
// scores, maxima, exponentials, P.V), so a third wave per SIMD gives more
// than overlapping the phases inside one wave, which needs the registers of
// a second score tile.  The block ids of a step are loaded by scalar loads
// one step before their first use, issued after the step's last LDS wait
// (scalar and LDS loads share a counter, and an outstanding scalar load
// makes every LDS wait a full one).  Groups of three steps that need no
// mask (every key inside the wave's rows' ranges -- below the first row
// and, with a window, at or above the last row's window start -- and three
// or more steps before the end of the walk) run a lean step without masks
// or bounds checks.
constexpr int kDmaWaves = 4;
constexpr int kDmaPieces = 8 / kDmaWaves;  // 1 KiB pieces of K (and of V) a wave loads per step
constexpr int kDmaThreads = kDmaWaves * kWave;
constexpr int kDmaRows = 32;                      // query rows per wave
constexpr int kDmaKeys = 32;                      // keys per step
constexpr int kRowBytes128 = 128 * 2;             // one 16-bit K or V row
constexpr int kVRegion = kDmaKeys * kRowBytes128;    // V of one step: 8 KiB
// K region: two 16-row tiles of 272 16-byte slots (a tile's four pieces at
// slots 0, 136, 66 and 202); V region: eight packed 1 KiB pieces
constexpr int kKTileSlots = 272;
constexpr int kKRegion = 2 * kKTileSlots * 16;      // 8704 bytes
constexpr int kStage = kKRegion + kVRegion;         // 16896 bytes
__device__ __forceinline__ int k_piece_slot(int q) { return (q & 1) * 136 + (q >> 1) * 66; }
// slot of (row r, chunk c) inside a 4-row piece
__device__ __forceinline__ int piece_slot(int r, int c, int tau) {
  return 4 * (4 * (c >> 2) + r) + ((c & 3) ^ tau);
}
__device__ __forceinline__ int tau_k(int r) { return (r >> 1) & 1; }
__device__ __forceinline__ int tau_v(int r) { return 2 * ((r >> 1) & 1); }

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4v lds_i16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) void lds_void;

template <class E>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c);
template <>
__device__ __forceinline__ f32x16 mfma32<BF16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma32<F16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <class E, bool WIN>
__global__ __launch_bounds__(kDmaThreads) __attribute__((amdgpu_waves_per_eu(3))) void prefill_dma(PrefillArgs a) {
  constexpr int D = 128;
  using S = typename E::storage;
  __shared__ __attribute__((aligned(256))) char s_st0[kStage];
  __shared__ __attribute__((aligned(256))) char s_st1[kStage];
  __shared__ __attribute__((aligned(256))) char s_st2[kStage];
  const int g = blockIdx.x;
  const int Z = gridDim.y;
  const int k = (int)blockIdx.y + Z * (int)blockIdx.z;
  int i, zq;
  // the item choice's scratch lives in stage 2, which no load fills before
  // the prologue's barrier
  int* const s_qs = reinterpret_cast<int*>(s_st2 + kLptSeqs + 4 * kClasses + 16);
  int* const s_ctx = s_qs + kPickRanges + 1;
  pick_item_in<kDmaThreads>(a, k, Z, i, zq, reinterpret_cast<uint8_t*>(s_st2),
                            reinterpret_cast<int*>(s_st2 + kLptSeqs),
                            reinterpret_cast<int*>(s_st2 + kLptSeqs + 4 * kClasses), s_qs, s_ctx);
  const int G = a.group, QT = kDmaRows / G;  // chunk tokens per wave
  // the item's query range and length: from the item choice's LDS copy when
  // it made one (small batches), else from memory
  i = __builtin_amdgcn_readfirstlane(i);  // the same in every lane
  zq = __builtin_amdgcn_readfirstlane(zq);
  int qa, qb, ctx;
  if (a.num_seqs <= kPickRanges) {
    qa = s_qs[i];
    qb = s_qs[i + 1];
    ctx = s_ctx[i];
  } else {
    qa = a.query_start[i];
    qb = a.query_start[i + 1];
    ctx = clamp_ctx(a, i);
  }
  qa = __builtin_amdgcn_readfirstlane(qa);
  qb = __builtin_amdgcn_readfirstlane(qb);
  ctx = __builtin_amdgcn_readfirstlane(ctx);
  if (qa < 0 || qb > a.num_tokens || qb <= qa) return;  // the whole workgroup
  const int n = qb - qa, nq = min(n, a.max_query);
  const int nqb = ceil_div(nq, QT);
  const int top = nqb - 1 - kDmaWaves * zq;  // the item's latest query block
  if (top < 0) return;                       // the whole workgroup
  const int w = wave_id();
  const int lane = threadIdx.x % kWave;
  const int c32 = lane & 31, h = lane >> 5;
  const int kend_wg = ctx - n + min(top * QT + QT, nq);  // the walk: keys [0, kend_wg)
  const int blk = top - w;                               // this wave's query block
  const int tok0 = blk * QT, ntok = blk >= 0 ? min(QT, nq - tok0) : 0;
  const int pos0 = ctx - n + tok0;
  const int kend = blk >= 0 ? pos0 + ntok : 0;
  S* out = reinterpret_cast<S*>(a.out);

  const int tl = c32 / G, hh = c32 - tl * G;
  const bool live = tl < ntok && pos0 + tl >= 0;
  const int lim = live ? pos0 + tl : kend - 1;
  const int row = tl < ntok ? (qa + tok0 + tl) * a.num_q_heads + g * G + hh : -1;
  if (kend_wg <= 0) {
    if (row >= 0)
      for (int d = 4 * h; d < D; d += 8)
        *reinterpret_cast<uint2*>(out + (size_t)row * D + d) = uint2{0u, 0u};
    return;
  }
  const bool mine = kend > 0;

  u32x4 qv[8];
  {
    const S* qrow = reinterpret_cast<const S*>(a.q) + (size_t)max(row, 0) * D + 8 * h;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qv[s] = row >= 0 ? *reinterpret_cast<const u32x4*>(qrow + 16 * s) : u32x4{0, 0, 0, 0};
  }
  const float c = fabsf(a.scale_log2), inv_c = 1.f / c;
  if (a.scale_log2 < 0.f) {
#pragma unroll
    for (int s = 0; s < 8; ++s) qv[s] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
  }

  const int bs_mask = (1 << a.log2_bs) - 1;
  const size_t head_stride = (size_t)D << a.log2_bs;
  const size_t block_stride = head_stride * a.num_kv_heads;
  const int32_t* table = a.block_tables + (size_t)i * a.max_blocks;
  const S* kbase0 = reinterpret_cast<const S*>(a.k_pool) + (size_t)g * head_stride;
  const S* vbase0 = reinterpret_cast<const S*>(a.v_pool) + (size_t)g * head_stride;
  const int ntiles = ceil_div(kend_wg, kTile);
  const int nsteps = ceil_div(ntiles, 2);
  const int unmasked = max(pos0, 0);
  const int W = WIN ? a.window : 0;
  const int st_begin =
      WIN ? max(max(ctx - n + max(top - (kDmaWaves - 1), 0) * QT, 0) - W + 1, 0) / kDmaKeys : 0;
  const int kbeg = WIN ? max(unmasked - W + 1, 0) : 0;

  struct Ids {
    int b0, b1;
  };
  // `inside`: the step lies inside the walk (every fast step), so its first
  // tile does; its second may be one past the walk's end (odd tile counts),
  // whose entry is then the last tile's (the tile is masked or not computed)
  auto raw_ids = [&](int st, bool inside) __attribute__((always_inline)) -> Ids {
    const int t = 2 * st;
    int b0 = -1, b1 = -1;
    if (inside || t < ntiles) b0 = scalar_load(table + ((t * kTile) >> a.log2_bs));
    if (inside || t + 1 < ntiles)
      b1 = scalar_load(table + ((min(t + 1, ntiles - 1) * kTile) >> a.log2_bs));
    return Ids{b0, b1};
  };
  auto checked = [&](const Ids& r) __attribute__((always_inline)) -> Ids {
    return Ids{(unsigned)r.b0 < (unsigned)a.num_blocks ? r.b0 : -1,
               (unsigned)r.b1 < (unsigned)a.num_blocks ? r.b1 : -1};
  };

  const int tw = (kDmaPieces * w) >> 2;
  // lane j of a piece load fills slot j: row (j / 4) % 4 of the piece, a
  // chunk of the row's 64-byte group j / 16
  uint32_t koff_g[kDmaPieces], voff_g[kDmaPieces];
  {
    const int pr = (lane >> 2) & 3, grp = lane >> 4, i4 = lane & 3;
#pragma unroll
    for (int x = 0; x < kDmaPieces; ++x) {
      const int q = (kDmaPieces * w + x) & 3;
      const int row = 4 * q + pr;
      koff_g[x] = (uint32_t)(row * kRowBytes128 + 16 * (4 * grp + (i4 ^ tau_k(pr))));
      voff_g[x] = (uint32_t)(row * kRowBytes128 + 16 * (4 * grp + (i4 ^ tau_v(pr))));
    }
  }
  const int kr = 16 * (c32 >> 4) + 8 * ((c32 >> 2) & 1) + 4 * ((c32 >> 3) & 1) + (c32 & 3);
  // K operand of k-step s at kb + 256 (s / 2) + 32 (s % 2)
  const uint32_t kb = (uint32_t)(16 * ((kr >> 4) * kKTileSlots + k_piece_slot((kr >> 2) & 3) +
                                       piece_slot(kr & 3, h, tau_k(kr & 3))));
  // V^T operand (k-step ks, row half hr, d-tile dt) at vb + 4096 ks + 1024 hr + 256 dt
  const uint32_t vb = (uint32_t)(kKRegion + 2048 * h +
                                 16 * piece_slot((lane & 15) >> 2, 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1),
                                                 tau_v((lane & 15) >> 2)) +
                                 8 * (lane & 1));

  // `full`: the tile lies wholly below the context length (every fast step)
  auto issue = [&](int st, char* buf, const Ids& id, bool full) __attribute__((always_inline)) {
    const int b = tw ? id.b1 : id.b0;
    const int t = 2 * st + tw;
    const size_t off = b >= 0 ? (size_t)b * block_stride + (size_t)((t * kTile) & bs_mask) * D : 0;
    const rsrc_t ks = make_rsrc(kbase0 + off, b >= 0 ? 16u * kRowBytes128 : 0u);
    const uint32_t vbytes =
        b < 0 ? 0u
              : full ? 16u * kRowBytes128
                     : (uint32_t)max(min(kTile, ctx - t * kTile), 0) * kRowBytes128;
    const rsrc_t vs = make_rsrc(vbase0 + off, vbytes);
#pragma unroll
    for (int x = 0; x < kDmaPieces; ++x) {
      const int pc = kDmaPieces * w + x;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ks, (lds_void*)(buf + 16 * (tw * kKTileSlots + k_piece_slot(pc & 3))), 16, koff_g[x], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          vs, (lds_void*)(buf + kKRegion + pc * 1024), 16, voff_g[x], 0, 0, 0);
    }
  };

  float m = kMFloor, lsum = 0.f, thr = (kMFloor + kRescaleSlack) * inv_c;
  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[dt][v] = 0.f;

  typedef const __attribute__((address_space(3))) char lds_cchar;
  // One step from stage `buf`: scores, mask, weights, P.V.  Every operand
  // read is one of two per-lane bases plus an immediate.
  auto compute = [&](int st, const char* buf, bool oka, bool okb, bool may_mask)
      __attribute__((always_inline)) {
    f32x16 sacc;
#pragma unroll
    for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const u32x4 kop =
          *reinterpret_cast<const lds_u32x4*>((lds_cchar*)buf + kb + (256u * (s >> 1) + 32u * (s & 1)));
      sacc = mfma32<E>(kop, qv[s], sacc);
    }
    const int k0 = st * kDmaKeys;
    float sv[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) sv[v] = sacc[v];
    if (may_mask && (k0 + kDmaKeys - 1 > unmasked || (WIN && k0 < kend - W) || !oka || !okb)) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = k0 + 16 * (v >> 3) + 8 * h + (v & 7);
        if (key > lim || (WIN && key <= lim - W) || !((v >> 3) ? okb : oka)) sv[v] = neg_inf();
      }
    }
    // maxima as a tree of three-input maxima (eight instructions)
    const float t0 = smax(smax(sv[0], sv[1]), sv[2]), t1 = smax(smax(sv[3], sv[4]), sv[5]);
    const float t2 = smax(smax(sv[6], sv[7]), sv[8]), t3 = smax(smax(sv[9], sv[10]), sv[11]);
    const float t4 = smax(smax(sv[12], sv[13]), sv[14]);
    const float mt = smax(smax(smax(t0, t1), sv[15]), smax(smax(t2, t3), t4));
    if (__builtin_amdgcn_ballot_w64(mt > thr)) {
      const float x = smax(mt, shfl_xor(mt, 32));
      const float mn = smax(m, x * c);
      const float alpha = fast_exp2(m - mn);
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
      m = mn;
      thr = (m + kRescaleSlack) * inv_c;
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float pf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = fast_exp2(__builtin_fmaf(sv[8 * ks + e], c, -m));
      const u32x4 pw = {Mfma<E>::round16x2(pf[0], pf[1]), Mfma<E>::round16x2(pf[2], pf[3]),
                        Mfma<E>::round16x2(pf[4], pf[5]), Mfma<E>::round16x2(pf[6], pf[7])};
      lsum = sum2(E{}, pw[3], sum2(E{}, pw[2], sum2(E{}, pw[1], sum2(E{}, pw[0], lsum))));
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const i16x4v lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)((__attribute__((address_space(3))) char*)(lds_cchar*)buf + vb + (4096u * ks + 256u * dt)));
        const i16x4v hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)((__attribute__((address_space(3))) char*)(lds_cchar*)buf + vb + (4096u * ks + 1024u + 256u * dt)));
        const u32x2 lo2 = __builtin_bit_cast(u32x2, lo4), hi2 = __builtin_bit_cast(u32x2, hi4);
        o[dt] = mfma32<E>(u32x4{lo2[0], lo2[1], hi2[0], hi2[1]}, pw, o[dt]);
      }
    }
  };
  auto runs = [&](int st) __attribute__((always_inline)) {
    return mine && st * kDmaKeys < kend && (!WIN || (st + 1) * kDmaKeys > kbeg);
  };

  // Ring of three stages, loads two steps ahead, one barrier per step: at
  // the top of step st a wave waits for its own loads of st (those of st + 1
  // may be in flight); the barrier makes every wave's visible and frees the
  // stage of st - 1, which the loads of st + 2 fill.
  const int s0 = st_begin;
  Ids id0 = checked(raw_ids(s0, false)), id1 = checked(raw_ids(s0 + 1, false));
  Ids raw2 = raw_ids(s0 + 2, false);
  issue(s0, s_st0, id0, false);
  if (s0 + 1 < nsteps) issue(s0 + 1, s_st1, id1, false);
  // lean steps: every key below the wave's first row (no causal mask) and,
  // with a window, at or above its last row's window start (no window mask)
  int fast_end = min(nsteps - 3, mine ? (unmasked + 1) / kDmaKeys : s0);
  int fast_begin = s0;
  if (WIN) {
    // the lean segment starts in step with the stage order (groups of three)
    const int first = max(ceil_div(max(kend - W, 0), kDmaKeys), s0);
    fast_begin = s0 + 3 * ceil_div(first - s0, 3);
    if (fast_begin + 3 > fast_end) fast_begin = fast_end = s0;  // no lean group
  }
  auto step = [&](int st, const char* cur, char* fill, bool fast) __attribute__((always_inline)) {
    if (fast || st + 1 < nsteps)
      __builtin_amdgcn_s_waitcnt(0x0070 | (2 * kDmaPieces));  // own loads of st landed
    else
      __builtin_amdgcn_s_waitcnt(0x0070);
    __builtin_amdgcn_s_barrier();
    const Ids id2 = checked(raw2);
    if (fast)
      issue(st + 2, fill, id2, true);
    else if (st + 2 < nsteps)
      issue(st + 2, fill, id2, false);
    if (fast)
      compute(st, cur, true, true, false);
    else if (runs(st) && (id0.b0 >= 0 || id0.b1 >= 0))
      compute(st, cur, id0.b0 >= 0, id0.b1 >= 0, true);
    // the next ids' scalar loads go out after the step's last LDS wait: the
    // two kinds share a counter, and an outstanding scalar load would make
    // every LDS wait a full one
    __builtin_amdgcn_sched_barrier(0);
    raw2 = raw_ids(st + 3, fast);
    id0 = id1;
    id1 = id2;
  };
  int st = s0;
  for (; st < fast_begin; st += 3) {  // window: the steps below the lean ones
    step(st, s_st0, s_st2, false);
    step(st + 1, s_st1, s_st0, false);
    step(st + 2, s_st2, s_st1, false);
  }
  for (; st + 3 <= fast_end; st += 3) {
    step(st, s_st0, s_st2, true);
    step(st + 1, s_st1, s_st0, true);
    step(st + 2, s_st2, s_st1, true);
  }
  for (; st < nsteps; st += 3) {
    step(st, s_st0, s_st2, false);
    if (st + 1 >= nsteps) break;
    step(st + 1, s_st1, s_st0, false);
    if (st + 2 >= nsteps) break;
    step(st + 2, s_st2, s_st1, false);
  }

  const float total = lsum + shfl_xor(lsum, 32);
  if (row >= 0) {
    const float inv = live && total > 0.f ? a.v_scale / total : 0.f;
    S* dst = out + (size_t)row * D + 4 * h;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<uint2*>(dst + 32 * dt + 8 * j) =
            uint2{Mfma<E>::round16x2(o[dt][4 * j] * inv, o[dt][4 * j + 1] * inv),
                  Mfma<E>::round16x2(o[dt][4 * j + 2] * inv, o[dt][4 * j + 3] * inv)};
  }
  if (a.status != nullptr) {
    const int kfirst =
        WIN ? max(max(ctx - n + max(top - (kDmaWaves - 1), 0) * QT, 0) - W + 1, 0) : 0;
    bool bad = false;
    for (int j = (kfirst >> a.log2_bs) + (int)threadIdx.x; j <= ((kend_wg - 1) >> a.log2_bs);
         j += kDmaThreads)
      bad |= (unsigned)table[j] >= (unsigned)a.num_blocks;
    report_bad_block(a.status, __builtin_amdgcn_ballot_w64(bad) != 0);
  }
}

// prefill_dma8 (8-bit pools): the same products and stage layout as
// prefill_dma, with the codes staged twice.  Each wave loads its own eight K
// and eight V rows of a step (1 KiB each, 16 bytes a lane) straight into a
// code stage, two steps ahead; one step ahead it widens them exactly to the
// operand type and writes them into a 16-bit stage in the piece layout
// above.  A wave widens only the codes it loaded, so its own load wait
// covers them, and the one barrier per step makes every wave's widened rows
// visible.  LDS: two 16-bit stages and two 8 KiB code stages (49 KiB, three
// workgroups per CU as before).
constexpr int kCodeStage = 2 * kDmaKeys * 128;  // K and V codes of one step

template <class E, bool WIN>
__global__ __launch_bounds__(kDmaThreads) __attribute__((amdgpu_waves_per_eu(3))) void prefill_dma8(PrefillArgs a) {
  constexpr int D = 128;
  using S = typename E::storage;
  __shared__ __attribute__((aligned(256))) char s_st0[kStage];
  __shared__ __attribute__((aligned(256))) char s_st1[kStage];
  __shared__ __attribute__((aligned(256))) char s_cd0[kCodeStage];
  __shared__ __attribute__((aligned(256))) char s_cd1[kCodeStage];
  const int g = blockIdx.x;
  const int Z = gridDim.y;
  const int k = (int)blockIdx.y + Z * (int)blockIdx.z;
  int i, zq;
  // the item choice's scratch lives in the second 16-bit stage, which no
  // wave writes before the first step's barrier
  int* const s_qs = reinterpret_cast<int*>(s_st1 + kLptSeqs + 4 * kClasses + 16);
  int* const s_ctx = s_qs + kPickRanges + 1;
  pick_item_in<kDmaThreads>(a, k, Z, i, zq, reinterpret_cast<uint8_t*>(s_st1),
                            reinterpret_cast<int*>(s_st1 + kLptSeqs),
                            reinterpret_cast<int*>(s_st1 + kLptSeqs + 4 * kClasses), s_qs, s_ctx);
  const int G = a.group, QT = kDmaRows / G;  // chunk tokens per wave
  // the item's query range and length: from the item choice's LDS copy when
  // it made one (small batches), else from memory
  i = __builtin_amdgcn_readfirstlane(i);  // the same in every lane
  zq = __builtin_amdgcn_readfirstlane(zq);
  int qa, qb, ctx;
  if (a.num_seqs <= kPickRanges) {
    qa = s_qs[i];
    qb = s_qs[i + 1];
    ctx = s_ctx[i];
  } else {
    qa = a.query_start[i];
    qb = a.query_start[i + 1];
    ctx = clamp_ctx(a, i);
  }
  qa = __builtin_amdgcn_readfirstlane(qa);
  qb = __builtin_amdgcn_readfirstlane(qb);
  ctx = __builtin_amdgcn_readfirstlane(ctx);
  if (qa < 0 || qb > a.num_tokens || qb <= qa) return;  // the whole workgroup
  const int n = qb - qa, nq = min(n, a.max_query);
  const int nqb = ceil_div(nq, QT);
  const int top = nqb - 1 - kDmaWaves * zq;  // the item's latest query block
  if (top < 0) return;                       // the whole workgroup
  const int w = wave_id();
  const int lane = threadIdx.x % kWave;
  const int c32 = lane & 31, h = lane >> 5;
  const int kend_wg = ctx - n + min(top * QT + QT, nq);  // the walk: keys [0, kend_wg)
  const int blk = top - w;                               // this wave's query block
  const int tok0 = blk * QT, ntok = blk >= 0 ? min(QT, nq - tok0) : 0;
  const int pos0 = ctx - n + tok0;
  const int kend = blk >= 0 ? pos0 + ntok : 0;
  S* out = reinterpret_cast<S*>(a.out);

  const int tl = c32 / G, hh = c32 - tl * G;
  const bool live = tl < ntok && pos0 + tl >= 0;
  const int lim = live ? pos0 + tl : kend - 1;
  const int row = tl < ntok ? (qa + tok0 + tl) * a.num_q_heads + g * G + hh : -1;
  if (kend_wg <= 0) {
    if (row >= 0)
      for (int d = 4 * h; d < D; d += 8)
        *reinterpret_cast<uint2*>(out + (size_t)row * D + d) = uint2{0u, 0u};
    return;
  }
  const bool mine = kend > 0;

  u32x4 qv[8];
  {
    const S* qrow = reinterpret_cast<const S*>(a.q) + (size_t)max(row, 0) * D + 8 * h;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qv[s] = row >= 0 ? *reinterpret_cast<const u32x4*>(qrow + 16 * s) : u32x4{0, 0, 0, 0};
  }
  const float c = fabsf(a.scale_log2), inv_c = 1.f / c;
  if (a.scale_log2 < 0.f) {
#pragma unroll
    for (int s = 0; s < 8; ++s) qv[s] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
  }

  const int bs_mask = (1 << a.log2_bs) - 1;
  const size_t head_stride = (size_t)D << a.log2_bs;
  const size_t block_stride = head_stride * a.num_kv_heads;
  const int32_t* table = a.block_tables + (size_t)i * a.max_blocks;
  const uint8_t* kbase0 = reinterpret_cast<const uint8_t*>(a.k_pool) + (size_t)g * head_stride;
  const uint8_t* vbase0 = reinterpret_cast<const uint8_t*>(a.v_pool) + (size_t)g * head_stride;
  const int ntiles = ceil_div(kend_wg, kTile);
  const int nsteps = ceil_div(ntiles, 2);
  const int unmasked = max(pos0, 0);
  const int W = WIN ? a.window : 0;
  const int st_begin =
      WIN ? max(max(ctx - n + max(top - (kDmaWaves - 1), 0) * QT, 0) - W + 1, 0) / kDmaKeys : 0;
  const int kbeg = WIN ? max(unmasked - W + 1, 0) : 0;

  struct Ids {
    int b0, b1;
  };
  // `inside`: the step lies inside the walk (every fast step), so its first
  // tile does; its second may be one past the walk's end (odd tile counts),
  // whose entry is then the last tile's (the tile is masked or not computed)
  auto raw_ids = [&](int st, bool inside) __attribute__((always_inline)) -> Ids {
    const int t = 2 * st;
    int b0 = -1, b1 = -1;
    if (inside || t < ntiles) b0 = scalar_load(table + ((t * kTile) >> a.log2_bs));
    if (inside || t + 1 < ntiles)
      b1 = scalar_load(table + ((min(t + 1, ntiles - 1) * kTile) >> a.log2_bs));
    return Ids{b0, b1};
  };
  auto checked = [&](const Ids& r) __attribute__((always_inline)) -> Ids {
    return Ids{(unsigned)r.b0 < (unsigned)a.num_blocks ? r.b0 : -1,
               (unsigned)r.b1 < (unsigned)a.num_blocks ? r.b1 : -1};
  };

  const int tw = w >> 1;  // the tile of the step this wave loads rows of
  // The lane's 16 codes: chunk jj of row rr of the wave's eight code rows
  // (rows 8 (w % 2) .. of its tile, rows 8 w .. 8 w + 7 of the step).  The
  // eight lanes of each group of the widened stores take the four rows of a
  // piece and two chunks with different bit 0 of jj, so their stores land on
  // eight distinct 16-byte bank groups.
  const int rr = 4 * ((lane >> 3) & 1) + (lane & 3), jj = 2 * (lane >> 4) + ((lane >> 2) & 1);
  const uint32_t coff = (uint32_t)(1024 * (w & 1) + 128 * rr + 16 * jj);
  // where the lane's two 16-byte chunks of 16-bit values (chunks 2 jj and
  // 2 jj + 1 of step row R) go in a 16-bit stage: the direct-to-LDS kernel's
  // piece layout
  uint32_t kdst[2], vdst[2];
  {
    const int R = 8 * w + rr, j = jj;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int c = 2 * j + x;
      kdst[x] = (uint32_t)(16 * ((R >> 4) * kKTileSlots + k_piece_slot((R & 15) >> 2) +
                                 piece_slot(R & 3, c, tau_k(R & 3))));
      vdst[x] = (uint32_t)(kKRegion + 1024 * (R >> 2) + 16 * piece_slot(R & 3, c, tau_v(R & 3)));
    }
  }
  const int kr = 16 * (c32 >> 4) + 8 * ((c32 >> 2) & 1) + 4 * ((c32 >> 3) & 1) + (c32 & 3);
  // K operand of k-step s at kb + 256 (s / 2) + 32 (s % 2)
  const uint32_t kb = (uint32_t)(16 * ((kr >> 4) * kKTileSlots + k_piece_slot((kr >> 2) & 3) +
                                       piece_slot(kr & 3, h, tau_k(kr & 3))));
  // V^T operand (k-step ks, row half hr, d-tile dt) at vb + 4096 ks + 1024 hr + 256 dt
  const uint32_t vb = (uint32_t)(kKRegion + 2048 * h +
                                 16 * piece_slot((lane & 15) >> 2, 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1),
                                                 tau_v((lane & 15) >> 2)) +
                                 8 * (lane & 1));

  // The codes of step st: this wave's eight K rows and eight V rows (1 KiB
  // each, contiguous in the pool) straight into the code stage.  `full`: the
  // tile lies wholly below the context length (every fast step).
  auto issue = [&](int st, char* buf, const Ids& id, bool full) __attribute__((always_inline)) {
    const int b = tw ? id.b1 : id.b0;
    const int t = 2 * st + tw;
    const size_t off = b >= 0 ? (size_t)b * block_stride + (size_t)((t * kTile) & bs_mask) * D : 0;
    const rsrc_t ks = make_rsrc(kbase0 + off, b >= 0 ? 16u * 128u : 0u);
    const uint32_t vbytes =
        b < 0 ? 0u
              : full ? 16u * 128u : (uint32_t)max(min(kTile, ctx - t * kTile), 0) * 128u;
    const rsrc_t vs = make_rsrc(vbase0 + off, vbytes);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ks, (lds_void*)(buf + 1024 * w), 16, coff, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vs, (lds_void*)(buf + 4096 + 1024 * w), 16, coff, 0,
                                             0, 0);
  };
  // This wave's codes of a step, widened exactly to the operand type into a
  // 16-bit stage (the rows it loaded itself, so its own wait covers them)
  typedef const __attribute__((address_space(3))) char lds_cchar8;
  typedef __attribute__((address_space(3))) char lds_char8;
  struct Codes {
    u32x4 k, v;
  };
  auto read_codes = [&](const char* cbuf) __attribute__((always_inline)) -> Codes {
    return Codes{
        *reinterpret_cast<const lds_u32x4*>((lds_cchar8*)cbuf + 1024 * w + 16 * lane),
        *reinterpret_cast<const lds_u32x4*>((lds_cchar8*)cbuf + 4096 + 1024 * w + 16 * lane)};
  };
  auto widen_into = [&](const Codes& cd, char* bf) __attribute__((always_inline)) {
    const u32x4 kc = cd.k, vc = cd.v;
    *reinterpret_cast<lds_u32x4*>((lds_char8*)bf + kdst[0]) = widen8<E>(kc[0], kc[1]);
    *reinterpret_cast<lds_u32x4*>((lds_char8*)bf + kdst[1]) = widen8<E>(kc[2], kc[3]);
    *reinterpret_cast<lds_u32x4*>((lds_char8*)bf + vdst[0]) = widen8<E>(vc[0], vc[1]);
    *reinterpret_cast<lds_u32x4*>((lds_char8*)bf + vdst[1]) = widen8<E>(vc[2], vc[3]);
  };

  float m = kMFloor, lsum = 0.f, thr = (kMFloor + kRescaleSlack) * inv_c;
  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[dt][v] = 0.f;

  typedef const __attribute__((address_space(3))) char lds_cchar;
  // One step from stage `buf`: scores, mask, weights, P.V.  Every operand
  // read is one of two per-lane bases plus an immediate.
  auto compute = [&](int st, const char* buf, bool oka, bool okb, bool may_mask)
      __attribute__((always_inline)) {
    f32x16 sacc;
#pragma unroll
    for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const u32x4 kop =
          *reinterpret_cast<const lds_u32x4*>((lds_cchar*)buf + kb + (256u * (s >> 1) + 32u * (s & 1)));
      sacc = mfma32<E>(kop, qv[s], sacc);
    }
    const int k0 = st * kDmaKeys;
    float sv[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) sv[v] = sacc[v];
    if (may_mask && (k0 + kDmaKeys - 1 > unmasked || (WIN && k0 < kend - W) || !oka || !okb)) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = k0 + 16 * (v >> 3) + 8 * h + (v & 7);
        if (key > lim || (WIN && key <= lim - W) || !((v >> 3) ? okb : oka)) sv[v] = neg_inf();
      }
    }
    // maxima as a tree of three-input maxima (eight instructions)
    const float t0 = smax(smax(sv[0], sv[1]), sv[2]), t1 = smax(smax(sv[3], sv[4]), sv[5]);
    const float t2 = smax(smax(sv[6], sv[7]), sv[8]), t3 = smax(smax(sv[9], sv[10]), sv[11]);
    const float t4 = smax(smax(sv[12], sv[13]), sv[14]);
    const float mt = smax(smax(smax(t0, t1), sv[15]), smax(smax(t2, t3), t4));
    if (__builtin_amdgcn_ballot_w64(mt > thr)) {
      const float x = smax(mt, shfl_xor(mt, 32));
      const float mn = smax(m, x * c);
      const float alpha = fast_exp2(m - mn);
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
      m = mn;
      thr = (m + kRescaleSlack) * inv_c;
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float pf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = fast_exp2(__builtin_fmaf(sv[8 * ks + e], c, -m));
      const u32x4 pw = {Mfma<E>::round16x2(pf[0], pf[1]), Mfma<E>::round16x2(pf[2], pf[3]),
                        Mfma<E>::round16x2(pf[4], pf[5]), Mfma<E>::round16x2(pf[6], pf[7])};
      lsum = sum2(E{}, pw[3], sum2(E{}, pw[2], sum2(E{}, pw[1], sum2(E{}, pw[0], lsum))));
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const i16x4v lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)((__attribute__((address_space(3))) char*)(lds_cchar*)buf + vb + (4096u * ks + 256u * dt)));
        const i16x4v hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)((__attribute__((address_space(3))) char*)(lds_cchar*)buf + vb + (4096u * ks + 1024u + 256u * dt)));
        const u32x2 lo2 = __builtin_bit_cast(u32x2, lo4), hi2 = __builtin_bit_cast(u32x2, hi4);
        o[dt] = mfma32<E>(u32x4{lo2[0], lo2[1], hi2[0], hi2[1]}, pw, o[dt]);
      }
    }
  };
  auto runs = [&](int st) __attribute__((always_inline)) {
    return mine && st * kDmaKeys < kend && (!WIN || (st + 1) * kDmaKeys > kbeg);
  };

  // Two 16-bit stages (the step computed, the next step's being widened) and
  // two code stages (the next step's codes, and those of the step after,
  // in flight); one barrier per step.  Step st: barrier (every wave's
  // widened rows of st visible; the 16-bit stage of st - 1 free), the codes
  // of st + 2 into the code stage of st, the products of st, then this
  // wave's codes of st + 1 (loaded a step earlier) widened into the other
  // 16-bit stage.
  const int s0 = st_begin;
  Ids id0 = checked(raw_ids(s0, false)), id1 = checked(raw_ids(s0 + 1, false));
  Ids raw2 = raw_ids(s0 + 2, false);
  issue(s0, s_cd0, id0, false);
  if (s0 + 1 < nsteps) {
    issue(s0 + 1, s_cd1, id1, false);
    __builtin_amdgcn_s_waitcnt(0x0F70 & ~0x000F | 2);  // own codes of s0 landed
  } else {
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }
  widen_into(read_codes(s_cd0), s_st0);
  // lean steps: every key below the wave's first row (no causal mask) and,
  // with a window, at or above its last row's window start (no window mask)
  int fast_end = min(nsteps - 3, mine ? (unmasked + 1) / kDmaKeys : s0);
  int fast_begin = s0;
  if (WIN) {
    // the lean segment starts in step with the stage order (groups of two)
    const int first = max(ceil_div(max(kend - W, 0), kDmaKeys), s0);
    fast_begin = s0 + 2 * ceil_div(first - s0, 2);
    if (fast_begin + 2 > fast_end) fast_begin = fast_end = s0;  // no lean group
  }
  // cur / next: the 16-bit stages of st and st + 1; codes: the code stage of
  // st + 1; fill: the code stage of st (free again), for st + 2
  auto step = [&](int st, const char* cur, char* next, const char* codes, char* fill, bool fast)
      __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0070 | 2);  // this wave's widened rows written
    __builtin_amdgcn_s_barrier();
    const Ids id2 = checked(raw2);
    if (fast)
      issue(st + 2, fill, id2, true);
    else if (st + 2 < nsteps)
      issue(st + 2, fill, id2, false);
    if (fast)
      compute(st, cur, true, true, false);
    else if (runs(st) && (id0.b0 >= 0 || id0.b1 >= 0))
      compute(st, cur, id0.b0 >= 0, id0.b1 >= 0, true);
    // The next ids' scalar loads go out after the step's products and with
    // the reads of the codes to widen: the two kinds share a counter (an
    // outstanding scalar load makes every LDS wait a full one), so the
    // latencies overlap in the one wait before the widening.
    if (fast || st + 1 < nsteps) {
      if (fast || st + 2 < nsteps)
        __builtin_amdgcn_s_waitcnt(0x0F70 & ~0x000F | 2);  // own codes of st + 1 landed
      else
        __builtin_amdgcn_s_waitcnt(0x0F70);
      const Codes cd = read_codes(codes);
      __builtin_amdgcn_sched_barrier(0);
      raw2 = raw_ids(st + 3, fast);
      __builtin_amdgcn_sched_barrier(0);
      widen_into(cd, next);
    } else {
      __builtin_amdgcn_sched_barrier(0);
      raw2 = raw_ids(st + 3, fast);
    }
    id0 = id1;
    id1 = id2;
  };
  int st = s0;
  for (; st < fast_begin; st += 2) {  // window: the steps below the lean ones
    step(st, s_st0, s_st1, s_cd1, s_cd0, false);
    step(st + 1, s_st1, s_st0, s_cd0, s_cd1, false);
  }
  for (; st + 2 <= fast_end; st += 2) {
    step(st, s_st0, s_st1, s_cd1, s_cd0, true);
    step(st + 1, s_st1, s_st0, s_cd0, s_cd1, true);
  }
  for (; st < nsteps; st += 2) {
    step(st, s_st0, s_st1, s_cd1, s_cd0, false);
    if (st + 1 >= nsteps) break;
    step(st + 1, s_st1, s_st0, s_cd0, s_cd1, false);
  }

  const float total = lsum + shfl_xor(lsum, 32);
  if (row >= 0) {
    const float inv = live && total > 0.f ? a.v_scale / total : 0.f;
    S* dst = out + (size_t)row * D + 4 * h;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<uint2*>(dst + 32 * dt + 8 * j) =
            uint2{Mfma<E>::round16x2(o[dt][4 * j] * inv, o[dt][4 * j + 1] * inv),
                  Mfma<E>::round16x2(o[dt][4 * j + 2] * inv, o[dt][4 * j + 3] * inv)};
  }
  if (a.status != nullptr) {
    const int kfirst =
        WIN ? max(max(ctx - n + max(top - (kDmaWaves - 1), 0) * QT, 0) - W + 1, 0) : 0;
    bool bad = false;
    for (int j = (kfirst >> a.log2_bs) + (int)threadIdx.x; j <= ((kend_wg - 1) >> a.log2_bs);
         j += kDmaThreads)
      bad |= (unsigned)table[j] >= (unsigned)a.num_blocks;
    report_bad_block(a.status, __builtin_amdgcn_ballot_w64(bad) != 0);
  }
}


template <class E>
pa_status launch_dma8(const PrefillArgs& a, hipStream_t st) {
  const int blocks = ceil_div(a.max_query, kDmaRows / a.group);
  if (blocks <= 0) return PA_OK;
  const dim3 grid(a.num_kv_heads, ceil_div(blocks, kDmaWaves), a.num_seqs);
  if (a.window > 0)
    hipLaunchKernelGGL((prefill_dma8<E, true>), grid, dim3(kDmaThreads), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_dma8<E, false>), grid, dim3(kDmaThreads), 0, st, a);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

template <class E>
pa_status launch_dma(const PrefillArgs& a, hipStream_t st) {
  const int blocks = ceil_div(a.max_query, kDmaRows / a.group);
  if (blocks <= 0) return PA_OK;
  const dim3 grid(a.num_kv_heads, ceil_div(blocks, kDmaWaves), a.num_seqs);
  if (a.window > 0)
    hipLaunchKernelGGL((prefill_dma<E, true>), grid, dim3(kDmaThreads), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_dma<E, false>), grid, dim3(kDmaThreads), 0, st, a);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

template <class E, KvType KV>
pa_status launch_lds(const PrefillArgs& a, hipStream_t st) {
  const int blocks = ceil_div(a.max_query, kLdsRows / a.group);
  if (blocks <= 0) return PA_OK;
  const dim3 grid(a.num_kv_heads, ceil_div(blocks, kLdsWaves), a.num_seqs);
  if (a.window > 0)
    hipLaunchKernelGGL((prefill_mfma_lds<E, KV, true>), grid, dim3(kLdsThreads), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_mfma_lds<E, KV, false>), grid, dim3(kLdsThreads), 0, st, a);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

bool prefill_supports(int dtype, int head_dim, int group) {
  return (dtype == PA_F16 || dtype == PA_BF16) && head_dim == 128 &&
         (group == 1 || group == 2 || group == 4 || group == 8 || group == 16);
}

int prefill_query_blocks(int max_query_len, int group) {
  return max_query_len > 0 ? ceil_div(max_query_len, kLdsRows / group) : 0;
}

pa_status launch_prefill(const PrefillArgs& a, int dtype, KvType kv, int path, hipStream_t st) {
  const bool fp8 = kv == KvType::kFp8;
  // The direct-to-LDS kernels unless the register-staged one is asked for
  // (AUTO: on the 8B chunked workload the direct kernel is 15-20% faster on
  // 16-bit pools and a few percent faster on 8-bit pools)
  const bool dma = path != PA_PREFILL_LDS;
  if (dtype == PA_BF16) {
    if (dma) return fp8 ? launch_dma8<BF16>(a, st) : launch_dma<BF16>(a, st);
    return fp8 ? launch_lds<BF16, KvType::kFp8>(a, st) : launch_lds<BF16, KvType::kSame>(a, st);
  }
  if (dtype == PA_F16) {
    if (dma) return fp8 ? launch_dma8<F16>(a, st) : launch_dma<F16>(a, st);
    return fp8 ? launch_lds<F16, KvType::kFp8>(a, st) : launch_lds<F16, KvType::kSame>(a, st);
  }
  return PA_ERR_SHAPE;
}

}  // namespace pa
