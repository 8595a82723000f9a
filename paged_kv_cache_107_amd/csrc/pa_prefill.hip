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
// Work split: one wave per (sequence, kv head, block of query tokens).  The
// G query heads of the kv head and 64 / G consecutive chunk tokens make 64
// query rows, taken as four groups of 16: each group is the 16 columns of the
// decode kernel's tile products (S^T = K . Q^T with v_mfma_f32_16x16x32), so
// one K/V tile load feeds four groups' products.  A wave walks the 16-key
// tiles from position 0 to its last token two at a time through a register
// ring of two pairs; with 32 keys per step the P.V product also runs on the
// double-rate v_mfma_f32_16x16x32 (O^T += V^T . P^T).  The steps at and past
// the block's first position are masked per element.  Each lane keeps the
// softmax state of its column in each group, with the decode kernel's lazy
// rescale; the running maximum starts at a finite floor, so a step has no
// branch between the rescale test and the P.V product.
//
// Two kernels compute this step.  prefill_mfma_lds (pa_prefill_lds.hip;
// 16-bit pools) runs four waves of 32 rows per item, two workgroups per CU,
// and shares each step's K/V tiles through LDS; prefill_mfma (this file;
// 8-bit pools) gives each of four waves 64 rows and its own register ring of
// tiles.
//
// With a sliding window of W positions a row at position p attends only
// positions p - W + 1 .. p: the wave starts at the tile of its first row's
// window and masks per element below each row's window as well.  8-bit pools
// are widened to the 16-bit operand type as the tiles are used (KvTile).
//
// Grid: kv head x, then a flat item index k over (sequence, query-block
// group z); with four waves per workgroup group z takes query blocks
// nqb-1-4z .. nqb-4-4z of its sequence, the heaviest first.  A wave's work grows with its sequence's
// length, so the items run longest sequence first: each workgroup ranks the
// batch by length class (512 positions) with counts in LDS (up to kLptSeqs
// sequences); short sequences then fill the tail instead of long sequences'
// last groups starting late.  Within a class a sequence's groups run back to
// back, so the workgroups running together on an XCD share few sequences and
// re-read their K/V from that XCD's L2.  Larger batches run in batch order.
// The kv heads of an item are neighbouring ids, so each XCD serves one kv
// head of every sequence.
#include <hip/hip_runtime.h>

#include "pa.h"
#include "pa_device.h"
#include "pa_internal.h"
#include "pa_prefill_step.h"

namespace pa {
namespace {

using namespace prefill;

constexpr int kPfWaves = 4;                 // waves per workgroup
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kGroups = 4;                  // 16-column groups per wave
constexpr int kRows = 16 * kGroups;         // query rows (token, head) per wave
constexpr int kPfPairs = 2;                 // tile pairs in the register ring

// WIN: a sliding window is set (a.window > 0); without one every column's
// first tile holds its key 0, so no column meets a fully masked tile before
// its first key and the guards below are compiled out.
template <class E, KvType KV, bool WIN>
__global__ __launch_bounds__(kPfThreads) void prefill_mfma(PrefillArgs a) {
  constexpr int D = 128;
  using S = typename E::storage;
  using Tile = KvTile<E, KV>;
  using P = typename Tile::P;
  const int g = blockIdx.x;
  const int Z = gridDim.y;
  const int k = (int)blockIdx.y + Z * (int)blockIdx.z;  // item index, 0 .. Z * B - 1
  int i, zq;
  pick_item<kPfThreads>(a, k, Z, i, zq);
  const int G = a.group, QT = kRows / G;  // chunk tokens per wave
  const int qa = a.query_start[i], qb = a.query_start[i + 1];
  if (qa < 0 || qb > a.num_tokens || qb <= qa) return;
  const int n = qb - qa;                   // chunk tokens: positions ctx - n ..
  const int nqb = ceil_div(min(n, a.max_query), QT);  // rows past max_query are not run
  const int blk = nqb - 1 - (zq * kPfWaves + wave_id());
  if (blk < 0) return;
  const int lane = threadIdx.x % kWave;
  const int c16 = lane & 15, g4 = lane >> 4;
  const int ctx = clamp_ctx(a, i);
  const int tok0 = blk * QT, ntok = min(QT, min(n, a.max_query) - tok0);
  const int pos0 = ctx - n + tok0;  // position of the block's first token
  const int kend = pos0 + ntok;     // keys [0, kend) are seen by some row

  // This lane's column in each group: chunk token tl, head h of the group.
  // lim = last position the column sees; rows without a query (past the
  // chunk, or at a negative position) see every key like the last row, which
  // keeps their state finite; they are never stored as attention outputs.
  int lim[kGroups], row[kGroups];
  bool live[kGroups];
#pragma unroll
  for (int q = 0; q < kGroups; ++q) {
    const int col = q * 16 + c16, tl = col / G, h = col - tl * G;
    live[q] = tl < ntok && pos0 + tl >= 0;
    lim[q] = live[q] ? pos0 + tl : kend - 1;
    row[q] = tl < ntok ? (qa + tok0 + tl) * a.num_q_heads + g * G + h : -1;
  }
  S* out = reinterpret_cast<S*>(a.out);
  if (kend <= 0) {  // every position negative: zero rows
#pragma unroll
    for (int q = 0; q < kGroups; ++q)
      if (row[q] >= 0)
        for (int d = 8 * g4; d < D; d += 32) *reinterpret_cast<u32x4*>(out + (size_t)row[q] * D + d) = u32x4{0, 0, 0, 0};
    return;
  }

  // q operand of each group: lane (c16, g4) holds the 8 elements of
  // q[column c16] that k-step s contracts (Tile::q_elem)
  u32x4 qv[kGroups][4];
#pragma unroll
  for (int q = 0; q < kGroups; ++q) {
    const S* qrow = reinterpret_cast<const S*>(a.q) + (size_t)max(row[q], 0) * D;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qv[q][s] = row[q] >= 0 ? *reinterpret_cast<const u32x4*>(qrow + Tile::q_elem(s, g4))
                             : u32x4{0, 0, 0, 0};
  }

  const int bs_mask = (1 << a.log2_bs) - 1;
  const size_t head_stride = (size_t)D << a.log2_bs;
  const size_t block_stride = head_stride * a.num_kv_heads;
  const int32_t* table = a.block_tables + (size_t)i * a.max_blocks;
  const P* kbase0 = reinterpret_cast<const P*>(a.k_pool) + (size_t)g * head_stride;
  const P* vbase0 = reinterpret_cast<const P*>(a.v_pool) + (size_t)g * head_stride;
  const int ntiles = ceil_div(kend, kTile);
  const int unmasked = max(pos0, 0);  // every row sees keys <= this position
  // Sliding window: the first row's window starts the walk; rows' windows
  // start at lim - W + 1, the latest at kend - W.
  const int W = WIN ? a.window : 0;
  const int t_begin = WIN ? max(unmasked - W + 1, 0) / kTile : 0;

  // Issue side: the block id of the next tile is read one issue ahead; tiles
  // past the last (or with a bad block id) get an empty descriptor, so every
  // issue has the same loads and the waits stay static.
  int it = t_begin;
  int iblk = scalar_load(table + ((it * kTile) >> a.log2_bs));
  auto issue = [&](Tile& tile) -> bool {
    bool ok = false;
    size_t off = 0;
    int rows = 0;  // V rows of the tile inside the sequence; the rest read as zeros
    if (it < ntiles) {
      ok = (unsigned)iblk < (unsigned)a.num_blocks;
      if (ok) off = (size_t)iblk * block_stride + (size_t)((it * kTile) & bs_mask) * D;
      rows = min(kTile, ctx - it * kTile);
      if (++it < ntiles) iblk = scalar_load(table + ((it * kTile) >> a.log2_bs));
    }
    const uint32_t kbytes = ok ? Tile::kBytes : 0u;
    const uint32_t vbytes = ok ? (uint32_t)rows * Tile::kRowBytes : 0u;
    tile.load(make_rsrc(kbase0 + off, kbytes), make_rsrc(vbase0 + off, vbytes), c16, g4);
    return ok;
  };

  // score scale c > 0 in log2 units: a negative scale flips q's sign (exact)
  const float c = fabsf(a.scale_log2), inv_c = 1.f / c;
  if (a.scale_log2 < 0.f) {
#pragma unroll
    for (int q = 0; q < kGroups; ++q)
#pragma unroll
      for (int s = 0; s < 4; ++s) qv[q][s] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
  }
  float m[kGroups], l[kGroups];
  f32x4 o[kGroups][8];
#pragma unroll
  for (int q = 0; q < kGroups; ++q) {
    m[q] = kMFloor;
    l[q] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[q][e] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Two 16-key tiles per step, so the P.V product runs on the double-rate
  // v_mfma_f32_16x16x32: its k-slot (g4, j) is key 4 g4 + j of the first
  // tile for j < 4 and key 4 g4 + j - 4 of the second for j >= 4, which is
  // where the lane's own S^T results of the two QK products sit.  A tile with
  // a bad block id (or past the last) is masked out; so are keys past a
  // column's position and, with a window, before its window.
  auto compute2 = [&](int t, const Tile& ta, const Tile& tb, bool oka, bool okb) {
    const int k0 = t * kTile;
    u32x4 vw[8];
    {
      u32x4 va[4], vb[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        va[r] = ta.v_row(r);
        vb[r] = tb.v_row(r);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        vw[e] = u32x4{__builtin_amdgcn_perm(va[1][e >> 1], va[0][e >> 1], sel),
                      __builtin_amdgcn_perm(va[3][e >> 1], va[2][e >> 1], sel),
                      __builtin_amdgcn_perm(vb[1][e >> 1], vb[0][e >> 1], sel),
                      __builtin_amdgcn_perm(vb[3][e >> 1], vb[2][e >> 1], sel)};
      }
    }
    const bool masked =
        k0 + 2 * kTile - 1 > unmasked || (WIN && k0 < kend - W) || !oka || !okb;
    float sv[kGroups][8];
#pragma unroll
    for (int q = 0; q < kGroups; ++q) {
      f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) sa = Mfma<E>::qk(ta.k_op(s), qv[q][s], sa);
#pragma unroll
      for (int s = 0; s < 4; ++s) sb = Mfma<E>::qk(tb.k_op(s), qv[q][s], sb);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sv[q][r] = sa[r];
        sv[q][4 + r] = sb[r];
      }
    }
    if (masked) {
#pragma unroll
      for (int q = 0; q < kGroups; ++q)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int key = k0 + (j < 4 ? 0 : kTile) + 4 * g4 + (j & 3);
          if (key > lim[q] || (WIN && key <= lim[q] - W) || !(j < 4 ? oka : okb))
            sv[q][j] = neg_inf();
        }
    }
    // m starts at a finite floor, so a column that has seen no key yet
    // (all -inf so far) gets weights exp2(-inf) = 0 and a rescale factor of
    // 0 or 1, never NaN: the weights need no guard and the step has no
    // branch between the rescale test and the P.V product.
    float mt[kGroups];
    bool over = false;
#pragma unroll
    for (int q = 0; q < kGroups; ++q) {
      mt[q] = smax(smax(smax(sv[q][0], sv[q][1]), smax(sv[q][2], sv[q][3])),
                   smax(smax(sv[q][4], sv[q][5]), smax(sv[q][6], sv[q][7])));
      over |= mt[q] > (m[q] + kRescaleSlack) * inv_c;
    }
    if (__builtin_amdgcn_ballot_w64(over)) {
#pragma unroll
      for (int q = 0; q < kGroups; ++q) {
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
    u32x4 pw[kGroups];
#pragma unroll
    for (int q = 0; q < kGroups; ++q) {
      float pf[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) pf[j] = fast_exp2(__builtin_fmaf(sv[q][j], c, -m[q]));
      pw[q] = u32x4{Mfma<E>::round16x2(pf[0], pf[1]), Mfma<E>::round16x2(pf[2], pf[3]),
                    Mfma<E>::round16x2(pf[4], pf[5]), Mfma<E>::round16x2(pf[6], pf[7])};
      // l sums the weights as rounded for the P.V product
      l[q] = sum2(E{}, pw[q][3], sum2(E{}, pw[q][2], sum2(E{}, pw[q][1], sum2(E{}, pw[q][0], l[q]))));
    }
#pragma unroll
    for (int q = 0; q < kGroups; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[q][e] = pv32(E{}, vw[e], pw[q], o[q][e]);
  };

  Tile tb[2 * kPfPairs];
  bool okb[2 * kPfPairs];
#pragma unroll
  for (int s = 0; s < 2 * kPfPairs; ++s) okb[s] = issue(tb[s]);
  // Every slot issues on every path and the loop exits at the bottom of the
  // unrolled body, so the compiler's wait counts stay static.
  int t = t_begin;
  do {
#pragma unroll
    for (int s = 0; s < 2 * kPfPairs; s += 2) {
      if (t < ntiles && (okb[s] || okb[s + 1])) compute2(t, tb[s], tb[s + 1], okb[s], okb[s + 1]);
      okb[s] = issue(tb[s]);
      okb[s + 1] = issue(tb[s + 1]);
      t += 2;
    }
  } while (t < ntiles);

  // Lane (c16, g4) holds O[column c16][32 g4 + 8 r + e] = o[q][e][r].
#pragma unroll
  for (int q = 0; q < kGroups; ++q) {
    const float lsum = across_groups_sum<16>(l[q]);
    if (row[q] < 0) continue;
    const float inv = live[q] && lsum > 0.f ? a.v_scale / lsum : 0.f;
    S* dst = out + (size_t)row[q] * D + 32 * g4;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint32_t b[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) b[e] = float_to_bits(E{}, o[q][e][r] * inv);
      *reinterpret_cast<u32x4*>(dst + 8 * r) =
          u32x4{b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16), b[6] | (b[7] << 16)};
    }
  }
}

template <class E, KvType KV>
pa_status launch(const PrefillArgs& a, int max_query_blocks, hipStream_t st) {
  const dim3 grid(a.num_kv_heads, ceil_div(max_query_blocks, kPfWaves), a.num_seqs);
  if (a.window > 0)
    hipLaunchKernelGGL((prefill_mfma<E, KV, true>), grid, dim3(kPfThreads), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_mfma<E, KV, false>), grid, dim3(kPfThreads), 0, st, a);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

bool prefill_supports(int dtype, int head_dim, int group) {
  return (dtype == PA_F16 || dtype == PA_BF16) && head_dim == 128 &&
         (group == 1 || group == 2 || group == 4 || group == 8 || group == 16);
}

int prefill_query_blocks(int max_query_len, int group) {
  return max_query_len > 0 ? (max_query_len + kRows / group - 1) / (kRows / group) : 0;
}

pa_status launch_prefill(const PrefillArgs& a, int dtype, KvType kv, hipStream_t st) {
  const int blocks = prefill_query_blocks(a.max_query, a.group);
  if (blocks <= 0) return PA_OK;
  const bool fp8 = kv == KvType::kFp8;
  if (!fp8) return launch_prefill_lds(a, dtype, st);  // 16-bit pools: shared tiles
  if (dtype == PA_BF16) return launch<BF16, KvType::kFp8>(a, blocks, st);
  if (dtype == PA_F16) return launch<F16, KvType::kFp8>(a, blocks, st);
  return PA_ERR_SHAPE;
}

}  // namespace pa
