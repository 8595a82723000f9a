// Paged decode attention for gfx950.
//
// The attention formula is plain scaled dot-product attention; paging only
// changes where K/V rows live, so the kernel follows the block table to each
// physical block (page "vLLM：把 KV 缓存当成虚拟内存", sections "破除误解" and
// "KV 的体积从哪来，页表如何把它切开": loop over blocks doing the Q x K/V
// multiply-adds, then reduce across blocks; page "放下账簿，打开源码", section
// "注意力计算的改写", whose block-loop sketch is completed here with a running
// maximum and rescaling, i.e. an online softmax).
//
// Work split: one workgroup (4 waves) per (sequence, kv head, partition of
// part_tokens positions).  The grid is (kv head, sequence, partition) with the
// partition slowest: workgroups go to the 8 XCDs round-robin by linear id, so
// neighbouring ids must carry similar work -- with the partition fastest, the
// XCD would be p % 8 and the first partitions (which every sequence has) would
// pile onto a few XCDs.  Partitions are visited last-first: only long
// sequences have high partitions and those are full, so the big uniform work
// starts early and the ragged last partitions fill the tail.  A partition is cut into 16-token tiles; wave w
// takes tiles w, w+4, ...  Each tile is one 16-token run of one physical
// block (a block of 32 tokens is two tiles), so the block-table entry is read
// once per tile, as a scalar load, one tile ahead of its use.
//
// Two tile kernels:
//  * MFMA (16-bit pools, head_dim 128, G = Hq/Hkv >= 2): the G query heads of
//    a kv head share every K row, so S^T = K_tile (16 x 128) . Q^T (128 x G)
//    is a small dense contraction: four v_mfma_f32_16x16x32 per tile with the
//    G heads in the 16 columns.  The P.V product runs on the matrix cores too
//    (O^T = V^T . P^T, eight v_mfma_f32_16x16x16 per tile): the S^T result
//    layout is exactly the B operand layout, and V's A operand is assembled
//    from the same 16-byte row loads with byte permutes.  Softmax state stays
//    per lane: each lane's column is one query head.
//  * VALU (every dtype, head_dim 64/128, G <= 8): lanes along head_dim, 16
//    bytes per lane per row, dot products reduced across the row's lanes with
//    DPP, online softmax per head in registers.
// Both keep K/V tiles in registers: the MFMA operand layouts and the VALU row
// layout are fed straight from coalesced 16-byte global loads.
//
// Split-K: a sequence with one partition is normalised and written to `out`
// by its workgroup.  Otherwise each partition writes (m, l, o) -- running max
// (log2 units), sum of exp2(s - m) and the unnormalised output -- and
// decode_reduce merges them: M = max m_p, out = sum 2^(m_p-M) o_p /
// sum 2^(m_p-M) l_p.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>

#include "pa.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int kWaves = 4;  // waves per workgroup
constexpr int kThreads = kWaves * kWave;
// Lane k of a wave holds the block id of the wave's k-th tile, so a wave
// takes at most 64 tiles: partitions of up to 4096 tokens need 4 waves.
static_assert(kWaves * kWave * 16 >= 4096, "partition_tokens <= 4096 needs >= 4 waves");
constexpr int kTile = 16;  // tokens per tile
// Tiles per wave in the register ring.  The grid kernel runs two workgroups
// per CU (two waves per SIMD) with a 3-deep ring; the stream kernel runs one
// workgroup per CU with a 4-deep ring, which keeps as many bytes in flight
// per CU without two co-resident workgroups competing (measured: with two,
// one of them takes most of the bandwidth and the other finishes late).
constexpr int kPrefetch = 3;
constexpr int kStreamPrefetch = 4;
constexpr float kRescaleSlack = 8.f;           // log2 units: p <= 256 between rescales

__device__ __forceinline__ int clamp_ctx(const DecodeArgs& a, int i) {
  int ctx = a.context_lens[i];
  ctx = min(ctx, a.max_ctx);
  ctx = min(ctx, a.max_blocks << a.log2_bs);
  return ctx;
}

// First position the query (at ctx - 1) attends: the sliding window's
// start, 0 without one.  Tile walks start at first & ~15 and mask below it.
__device__ __forceinline__ int first_pos(const DecodeArgs& a, int ctx) {
  return a.window > 0 ? max(ctx - a.window, 0) : 0;
}

// Partitions of the attended range [first & ~15, ctx).
__device__ __forceinline__ int num_parts(const DecodeArgs& a, int ctx) {
  return ctx > 0 ? (ctx - (first_pos(a, ctx) & ~(kTile - 1)) + a.part_tokens - 1) / a.part_tokens
                 : 1;
}

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// ----------------------------------------------------------------- epilogue
// LDS layout of the per-wave partial states: m[waves][16], l[waves][16],
// then o[waves][G][D + 4] (row padding staggers banks).
template <int D>
__host__ __device__ constexpr int o_stride() { return D + 4; }

template <int D>
size_t merge_smem_bytes(int group) {
  return (2 * kWaves * 16 + (size_t)kWaves * group * o_stride<D>()) * sizeof(float);
}

// Merge the waves' states and store either the normalised output or the
// partition's (m, l, o) for the reduce pass.  A thread owns 4 consecutive
// outputs of one head: it forms that head's per-wave weights 2^(m_w - M)
// once, then reads the 4 waves' partial vectors as float4s; everything it
// reads is independent, so the merge is a few LDS round trips long.
template <class E, int D>
__device__ void combine_store(const DecodeArgs& a, const float* smem, int group, int i, int g,
                              int p, int n_parts) {
  const float* sm_m = smem;
  const float* sm_l = smem + kWaves * 16;
  const float* sm_o = smem + 2 * kWaves * 16;
  constexpr int V = D / 4;  // float4 columns per head
  for (int idx = threadIdx.x; idx < group * V; idx += kThreads) {
    const int h = idx / V, d = (idx % V) * 4;
    float mw[kWaves], M = neg_inf();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      mw[w] = sm_m[w * 16 + h];
      M = fmaxf(M, mw[w]);
    }
    f32x4 O = {0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
    if (M != neg_inf()) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float wt = fast_exp2(mw[w] - M);
        L += wt * sm_l[w * 16 + h];
        O += wt * *reinterpret_cast<const f32x4*>(sm_o + ((size_t)w * group + h) * o_stride<D>() + d);
      }
    }
    const size_t row = (size_t)i * a.num_q_heads + (size_t)g * group + h;
    if (n_parts == 1) {
      const float inv = L > 0.f ? a.v_scale / L : 0.f;
      using S = typename E::storage;
      S* dst = reinterpret_cast<S*>(a.out) + row * D + d;
      if constexpr (E::bytes == 4) {
        *reinterpret_cast<f32x4*>(dst) = O * inv;
      } else {
        const uint32_t b0 = float_to_bits(E{}, O[0] * inv), b1 = float_to_bits(E{}, O[1] * inv);
        const uint32_t b2 = float_to_bits(E{}, O[2] * inv), b3 = float_to_bits(E{}, O[3] * inv);
        *reinterpret_cast<uint2*>(dst) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
      }
    } else {
      *reinterpret_cast<f32x4*>(a.ws_o + (row * a.max_parts + p) * D + d) = O;
      if (d == 0) a.ws_ml[row * a.max_parts + p] = make_float2(M, L);
    }
  }
}

template <class E, int D>
__device__ void store_zero_rows(const DecodeArgs& a, int group, int i, int g) {
  for (int idx = threadIdx.x; idx < group * D; idx += kThreads) {
    const size_t row = (size_t)i * a.num_q_heads + (size_t)g * group + idx / D;
    reinterpret_cast<typename E::storage*>(a.out)[row * D + idx % D] = 0;
  }
}

// ----------------------------------------------------------------- MFMA path
// Lane roles in a tile (c16 = lane % 16, g4 = lane / 16):
//  QK  A = K tile:   lane holds K[row c16][32 s + 8 g4 .. +7]   for k-step s = 0..3
//      B = Q^T:      lane holds q[head c16][32 s + 8 g4 .. +7]  (zero for c16 >= G)
//      S^T out:      lane holds S[token 4 g4 + r][head c16], r = 0..3
//  PV  A_e = V^T:    lane holds V[token 4 g4 + r][8 c16 + e], r = 0..3 (e = 0..7)
//      B = P^T:      lane holds P[head c16][token 4 g4 + r]  (= S^T out layout)
//      O^T_e out:    lane holds O[head c16][32 g4 + 8 r + e], r = 0..3
// so a lane keeps 32 output values of its own head, and the softmax rescale
// needs no cross-lane traffic.
template <class E, KvType KV>
__global__ __launch_bounds__(kThreads) void decode_partition_mfma(DecodeArgs a) {
  constexpr int D = 128;
  using Tile = KvTile<E, KV>;
  using P = typename Tile::P;
  extern __shared__ float smem[];
  const int g = blockIdx.x, i = blockIdx.y;
  const int p = (int)(gridDim.z - 1 - blockIdx.z);  // last partitions first
  const int ctx = clamp_ctx(a, i);
  const int n_parts = num_parts(a, ctx);
  if (p >= n_parts) return;
  const int G = a.group;
  if (ctx <= 0) {
    store_zero_rows<E, D>(a, G, i, g);
    return;
  }
  const int lane = threadIdx.x % kWave, w = wave_id();
  const int c16 = lane & 15, g4 = lane >> 4;
  const int first = first_pos(a, ctx);
  const int t0 = (first & ~(kTile - 1)) + p * a.part_tokens;
  const int ntok = min(a.part_tokens, ctx - t0);
  const int ntiles = (ntok + kTile - 1) / kTile;
  const int bs_mask = (1 << a.log2_bs) - 1;

  using S = typename E::storage;
  u32x4 qv[4];
  {
    const S* qrow = reinterpret_cast<const S*>(a.q) +
                    ((size_t)i * a.num_q_heads + (size_t)g * G + c16) * D;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qv[s] = c16 < G ? load16(qrow + Tile::q_elem(s, g4)) : u32x4{0, 0, 0, 0};
  }
  const int32_t* table = a.block_tables + (size_t)i * a.max_blocks;
  const size_t head_stride = (size_t)D << a.log2_bs;
  const size_t block_stride = head_stride * a.num_kv_heads;
  const P* kbase0 = reinterpret_cast<const P*>(a.k_pool) + (size_t)g * head_stride;
  const P* vbase0 = reinterpret_cast<const P*>(a.v_pool) + (size_t)g * head_stride;

  // This wave's tiles are w, w + 4, w + 8, ...; tile k of the wave is
  // partition tile w + 4k.  Lane k holds the physical block of the wave's
  // tile k, read once with one vector load (a partition has at most 4096
  // tokens, so a wave has at most 64 tiles).
  const int my_n = w < ntiles ? (ntiles - w + kWaves - 1) / kWaves : 0;
  const int ids =
      lane < my_n ? table[min((t0 + kTile * (w + kWaves * lane)) >> a.log2_bs, a.max_blocks - 1)]
                  : -1;

  // Issues the loads of the wave's tile k through per-tile buffer
  // descriptors.  A tile past the wave's last (or with a bad block id) gets
  // an empty descriptor: its loads return zeros without touching memory, so
  // every ring slot always has the same loads in flight and the wait counts
  // stay static.  Returns whether the tile holds data.
  bool bad = false;  // a tile of the partition named a block outside the pool
  auto issue = [&](int k, Tile& t) -> bool {
    const int blk = k < my_n ? __builtin_amdgcn_readlane(ids, k) : -1;
    const bool ok = (unsigned)blk < (unsigned)a.num_blocks;
    bad |= k < my_n && !ok;
    const int tok = t0 + kTile * (w + kWaves * k);
    const size_t off = ok ? (size_t)blk * block_stride + (size_t)(tok & bs_mask) * D : 0;
    const uint32_t bytes = ok ? Tile::kBytes : 0u;
    t.load(make_rsrc(kbase0 + off, bytes), make_rsrc(vbase0 + off, bytes), c16, g4);
    return ok;
  };

  float m = neg_inf(), l = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One tile: S^T = K Q^T, online softmax update, O^T += V^T P^T.
  //
  // The softmax uses a per-head reference m (log2 units) and p = 2^(s - m).
  // m, l and O are rescaled only when a score exceeds m + kRescaleSlack: then
  // m becomes the running maximum.  Any reference gives the same quotient
  // sum p v / sum p, and p <= 2^kRescaleSlack stays well inside the 16-bit
  // range of the P operand.  The check is lane-local plus one wave vote, so
  // the common case needs no cross-lane traffic and no accumulator rescale.
  // Rows before the window's first position or past the sequence are masked
  // (every tile keeps at least one attended row).
  auto compute = [&](int k, const Tile& t) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st) s = Mfma<E>::qk(t.k_op(st), qv[st], s);
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[r] = s[r] * a.scale_log2;
    u32x4 vc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) vc[r] = t.v_row(r);
    const int tok = t0 + kTile * (w + kWaves * k);
    const int valid = ntok - kTile * (w + kWaves * k), low = first - tok;
    if (valid < kTile || low > 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = 4 * g4 + r;
        if (e >= valid || e < low) {
          sv[r] = neg_inf();
          vc[r] = u32x4{0, 0, 0, 0};  // slots outside the range may hold anything
        }
      }
    }
    const float lim = m + kRescaleSlack;
    const bool over = sv[0] > lim || sv[1] > lim || sv[2] > lim || sv[3] > lim;
    if (__builtin_amdgcn_ballot_w64(over)) {
      float mt = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      mt = fmaxf(mt, shfl_xor(mt, 16));
      mt = fmaxf(mt, shfl_xor(mt, 32));
      const float mn = fmaxf(m, mt);
      const float alpha = fast_exp2(m - mn);
      l *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] *= alpha;
      m = mn;
    }
    uint32_t pb[4];
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pb[r] = Mfma<E>::round16(fast_exp2(sv[r] - m));
      psum += bits_to_float(E{}, pb[r]);  // the weights the P.V product uses
    }
    l += psum;
    const u32x2 pw = {pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16)};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      const u32x2 vw = {__builtin_amdgcn_perm(vc[1][e >> 1], vc[0][e >> 1], sel),
                        __builtin_amdgcn_perm(vc[3][e >> 1], vc[2][e >> 1], sel)};
      o[e] = Mfma<E>::pv(vw, pw, o[e]);
    }
  };

  // Register ring of kPrefetch tiles: while one tile is computed the loads
  // of the next kPrefetch - 1 are in flight.
  Tile tb[kPrefetch];
  bool okb[kPrefetch];
#pragma unroll
  for (int s = 0; s < kPrefetch; ++s) okb[s] = issue(s, tb[s]);
  for (int base = 0; base < my_n; base += kPrefetch) {
#pragma unroll
    for (int s = 0; s < kPrefetch; ++s) {
      if (okb[s]) compute(base + s, tb[s]);
      okb[s] = issue(base + s + kPrefetch, tb[s]);
    }
  }

  report_bad_block(a.status, bad);
  // wave state -> LDS
  l = across_groups_sum<16>(l);
  float* sm_m = smem;
  float* sm_l = smem + kWaves * 16;
  float* sm_o = smem + 2 * kWaves * 16;
  if (c16 < G) {
    if (g4 == 0) {
      sm_m[w * 16 + c16] = m;
      sm_l[w * 16 + c16] = l;
    }
    float* dst = sm_o + ((size_t)w * G + c16) * o_stride<D>() + 32 * g4;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      *reinterpret_cast<f32x4*>(dst + 8 * r) = f32x4{o[0][r], o[1][r], o[2][r], o[3][r]};
      *reinterpret_cast<f32x4*>(dst + 8 * r + 4) = f32x4{o[4][r], o[5][r], o[6][r], o[7][r]};
    }
  }
  __syncthreads();
  combine_store<E, D>(a, smem, G, i, g, p, n_parts);
}

// ----------------------------------------------------------------- stream MFMA path
// The tile math of decode_partition_mfma with another work split.  Every tile
// of the batch is put in one flat order -- kv head, then sequence, then
// token -- and the grid (kStreamWgPerCu workgroups per CU) is treated as a
// set of independent waves, each taking one contiguous run of that order
// (StreamSplit).  The waves of one XCD's chunk get the same number of tiles
// to within one (the chunks are equal, or sized by the XCDs' measured rates:
// StreamBalance), none waits on a sibling (no barrier after the prologue), and one
// register ring runs through the wave's whole run, across the (kv head,
// sequence) pairs it touches, so the next pair's loads are in flight while
// the current one is stored.  The run of a kv head stays on one or two XCDs,
// so sequences that share prefix blocks read them through the same L2.
//
// A pair that lies inside one wave's run is normalised and written to `out`
// by that wave.  The waves that share a pair each leave (m, l, o) for its G
// heads in workspace slot (pair + wave rank), and decode_reduce_stream merges
// them.  Slots never collide: pairs are numbered in the flat order and the
// first wave of the next pair is never below the last wave of this one.
// The wave in whose run a split pair starts owns its merge and records it:
// ws_owner[rank] = (pair, number of segments, tiles per kv head, whether
// every run is non-empty), or pair -1.  Rows of empty sequences are zeroed
// here.
//
// A wave's segment outputs (a whole pair's rows, or a split pair's (m, l, o))
// are staged in its own LDS area and written to memory after its walk (or
// when the area is full): stores count in the same counter as the ring's
// loads, so a store issued inside the walk made the following tiles' waits
// deeper than their own loads needed (measured on the 8B batch: about 1.5 us
// per pair in a wave's run with the stores in the walk, 0.5 us without).
constexpr int kStreamWgPerCu = 1;  // resident workgroups per CU: one wave per SIMD
constexpr int kXcds = 8;           // accelerator dies, each with its own L2
// s_waitcnt immediate for vmcnt(0) with expcnt and lgkmcnt left at their
// maxima (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[15:14]).
constexpr int kVmcnt0 = 0x0F70;

// Tiles of a sequence of ctx tokens whose first attended position is
// `first`: the 16-token tiles from first & ~15 to ctx (none when ctx = 0).
__device__ __forceinline__ int seq_tiles(int ctx, int first) {
  return ctx > 0 ? ceil_div(ctx, kTile) - (first >> 4) : 0;
}

// tb[i] = sum over j < i of seq_tiles(ctx[j], first[j]) (tile offset of
// sequence i within a kv head's run), tb[n] = total.  Block-wide; ends with a
// barrier.  Each thread sums a contiguous range of sequences; the ranges are
// scanned within each wave by lane shuffles and across the waves through
// tmp[0..kWaves), with two barriers.
__device__ void scan_tiles(const int* ctx, const int* first, int* tb, int n, int* tmp) {
  const int t = threadIdx.x, lane = t % kWave, w = t / kWave;
  const int per = (n + kThreads - 1) / kThreads;
  const int lo = min(n, t * per), hi = min(n, lo + per);
  int sum = 0;
  for (int k = lo; k < hi; ++k) sum += seq_tiles(ctx[k], first[k]);
  int incl = sum;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int x = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += x;
  }
  if (lane == kWave - 1) tmp[w] = incl;
  __syncthreads();
  int run = incl - sum;
  for (int v = 0; v < w; ++v) run += tmp[v];
  for (int k = lo; k < hi; ++k) {
    tb[k] = run;
    run += seq_tiles(ctx[k], first[k]);
  }
  if (t == kThreads - 1) tb[n] = run;
  __syncthreads();
}

// Split of T flat tiles over the kWaves * nwg waves of nwg workgroups.  The
// hardware deals workgroups to the device's XCDs round-robin, so workgroup b
// runs on XCD b % X (X = min(xcds, nwg); xcds is queried from the device: 8
// on a whole MI355X, fewer in a partition mode).  The tiles are cut into X
// contiguous chunks, chunk x going to the workgroups b = x, x + X, ...; each
// chunk is split evenly over its waves.  The chunks are equal, or, with
// weights (X = 8),
// chunk x covers [T cum[x] / 2^16, T cum[x + 1] / 2^16).  Ranks number the
// waves in flat order: rank r's run is [lo(r), lo(r + 1)).  Any monotone cut
// keeps the slot rule of the stream kernel.
constexpr uint32_t kBalanceMagic = 0x6C614257u;
constexpr uint32_t kBalanceOne = 1u << 16;
// a chunk's share of the tiles under weights: 1/16 .. 3/16
constexpr uint32_t kShareMin = kBalanceOne / 16, kShareMax = 3 * kBalanceOne / 16;
// weights apply (and passes are timed) from this many tiles per wave on
// (passes of about 80 us): below it the cut's prologue load and the timing
// record cost more than the balance returns (a 71-tile pass measured 57.5
// against 55.8 us even; a 96-tile one 146 against 149-151 us)
constexpr int kBalanceMinTilesPerWave = 80;

struct StreamSplit {
  long long T;
  int nwg;
  const int* cut = nullptr;  // weights: chunk x is [cut[x], cut[x + 1]) (in LDS)
  int xcds = kXcds;
  __device__ int chunks() const { return min(min(max(xcds, 1), kXcds), nwg); }
  __device__ int wgs_of(int x) const { return nwg / chunks() + (x < nwg % chunks() ? 1 : 0); }
  __device__ int base(int x) const {  // first rank of chunk x
    return kWaves * (x * (nwg / chunks()) + min(x, nwg % chunks()));
  }
  __device__ long long chunk_lo(int x) const { return cut ? cut[x] : T * x / chunks(); }
  __device__ long long lo(int r) const {
    if (r >= kWaves * nwg) return T;
    int x = 0;
    while (x + 1 < chunks() && base(x + 1) <= r) ++x;
    const long long c0 = chunk_lo(x);
    return c0 + (chunk_lo(x + 1) - c0) * (r - base(x)) / (kWaves * wgs_of(x));
  }
  // rank of workgroup b's wave w
  __device__ int rank(int b, int w) const {
    return base(b % chunks()) + (b / chunks()) * kWaves + w;
  }
  // every run non-empty: at least as many tiles in each chunk as waves
  __device__ int dense() const {
    if (!cut)
      return T / chunks() >= (long long)kWaves * ((nwg + chunks() - 1) / chunks()) ? 1 : 0;
    for (int x = 0; x < chunks(); ++x)
      if (chunk_lo(x + 1) - chunk_lo(x) < (long long)kWaves * wgs_of(x)) return 0;
    return 1;
  }
  // rank whose run holds tile t, 0 <= t < T
  __device__ int rank_of(long long t) const {
    int x;
    if (cut) {  // the last chunk starting at or before t (empty ones skipped)
      x = 0;
      while (x + 1 < chunks() && chunk_lo(x + 1) <= t) ++x;
    } else {
      x = (int)(((t + 1) * chunks() - 1) / T);
    }
    const long long c0 = chunk_lo(x), tx = chunk_lo(x + 1) - c0;
    return base(x) + (int)(((t - c0 + 1) * (kWaves * wgs_of(x)) - 1) / tx);
  }
  // whether passes of this size are timed and may use weights
  __device__ bool balanced_size() const {
    return xcds == kXcds && chunks() == kXcds &&
           T >= (long long)kBalanceMinTilesPerWave * kWaves * nwg;
  }
};

// A balance header's cut, if the header is valid: magic, cum[0] = 0,
// cum[8] = 2^16, every share within [kShareMin, kShareMax].  `w`: the
// header's words (magic at 0, cum at 4..12), in global memory or an LDS copy.
__device__ bool read_cut(const uint32_t* w, uint32_t (&cum)[kXcds + 1]) {
  if (w == nullptr || w[0] != kBalanceMagic) return false;
  for (int x = 0; x <= kXcds; ++x) cum[x] = w[4 + x];
  if (cum[0] != 0 || cum[kXcds] != kBalanceOne) return false;
  for (int x = 0; x < kXcds; ++x) {
    if (cum[x + 1] < cum[x]) return false;
    const uint32_t sh = cum[x + 1] - cum[x];
    if (sh < kShareMin || sh > kShareMax) return false;
  }
  return true;
}
__device__ const uint32_t* header_words(const StreamBalance* h) {
  return reinterpret_cast<const uint32_t*>(h);
}

// The header words the cut is read from (magic at 0, cum at 4..12), loaded
// by thread 0 at the start of a partition pass so that their latency
// overlaps the sequence table's.
constexpr int kHeaderCutWords = 4 + kXcds + 1;
__device__ void load_cut_words(const DecodeArgs& a, uint32_t (&hw)[kHeaderCutWords]) {
#pragma unroll
  for (int x = 0; x < kHeaderCutWords; ++x) hw[x] = 0;
  if (!a.balance || a.ws_balance == nullptr) return;
  const uint32_t* src = header_words(a.ws_balance);
  hw[0] = src[0];
#pragma unroll
  for (int x = 4; x < kHeaderCutWords; ++x) hw[x] = src[x];
}

// The cut of a partition pass, by thread 0 into s_cut[0..8] (LDS; the caller
// puts a barrier after it): weighted by the workspace's balance state when
// balancing is on, the pass is large enough, the header is valid and every
// run stays non-empty (so the reduce pass, which sees only dense records
// under weights, never needs the cut); else s_cut[0] = -1 (the even cut).
// hw: the header's words from load_cut_words.
__device__ void partition_cut(const DecodeArgs& a, long long T, int nwg, int* s_cut,
                              const uint32_t (&hw)[kHeaderCutWords]) {
  StreamSplit sp{T, nwg, nullptr, a.xcds};
  uint32_t cum[kXcds + 1];
  s_cut[0] = -1;
  if (!a.balance || a.ws_balance == nullptr || !sp.balanced_size() || !read_cut(hw, cum)) return;
  for (int x = 0; x <= kXcds; ++x) s_cut[x] = (int)((T * (long long)cum[x]) >> 16);
  sp.cut = s_cut;
  if (!sp.dense()) s_cut[0] = -1;
}

// The reduce pass's last workgroup (every thread): turn the last partition
// pass's record into the next cut, or initialise an invalid header with the
// even cut.  One round of loads: the header's first 24 words into LDS and
// each thread's wave slots, in parallel; each chunk's time is the largest
// of its waves' slots (a wave maximum per chunk when a wave's 64 ranks lie
// in one chunk, else per lane; then an LDS maximum); then eight lanes of
// wave 0, one per chunk, update the cut (sums and scans by lane shuffles).
// Plain vector loads and stores: the partition pass ran before on the same
// stream, so its stores are complete.  nwg: the partition pass's workgroups.
__device__ void update_balance(StreamBalance* h, int nwg) {
  constexpr int kWords = 24;  // magic, stamped, pad[2], cum[12], tiles[8]
  constexpr int kPer = kStreamMaxWaves / kThreads;
  __shared__ uint32_t s_hdr[kWords];
  __shared__ uint32_t s_dmax[kXcds];
  const int n = kWaves * nwg;  // wave ranks of the partition pass (<= kStreamMaxWaves)
  const int lane = threadIdx.x % kWave;
  if (threadIdx.x < kWords) s_hdr[threadIdx.x] = header_words(h)[threadIdx.x];
  if (threadIdx.x < kXcds) s_dmax[threadIdx.x] = 0;
  uint32_t d[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int r = (int)threadIdx.x + k * kThreads;
    d[k] = r < n ? h->wave_dur[r] : 0u;
  }
  __syncthreads();
  if (nwg % kXcds == 0) {
    // with nwg a multiple of 8, the ranks of chunk x are [x R, (x + 1) R)
    const int R = n / kXcds;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int r = (int)threadIdx.x + k * kThreads;
      if (R % kWave == 0) {  // the wave's 64 ranks share a chunk
        uint32_t v = d[k];
#pragma unroll
        for (int m = 1; m < kWave; m <<= 1) v = max(v, (uint32_t)__shfl_xor((int)v, m, kWave));
        if (lane == 0 && r < n) atomicMax(&s_dmax[r / R], v);
      } else if (r < n) {
        atomicMax(&s_dmax[r / R], d[k]);
      }
    }
  }
  __syncthreads();
  if (threadIdx.x >= kWave) return;
  // wave 0; lane x < 8 stands for chunk x
  const int x = lane;
  const bool lx = x < kXcds;
  uint32_t cum[kXcds + 1];
  if (!read_cut(s_hdr, cum)) {
    if (x <= kXcds) h->cum[x] = kBalanceOne / kXcds * x;
    if (lx) h->tiles[x] = 0;
    if (x == 0) {
      h->magic = kBalanceMagic;
      h->stamped = 0;
    }
    return;
  }
  if (!s_hdr[1] || nwg % kXcds != 0) return;  // no record to use
  const uint32_t nt = lx ? s_hdr[16 + x] : 0u, dd = lx ? s_dmax[x] : 0u;
  const bool ok = __builtin_amdgcn_ballot_w64(lx && (nt == 0 || dd == 0)) == 0;
  const float rate = dd > 0 ? (float)nt / (float)dd : 0.f;
  // sums, minima and maxima over the eight chunk lanes (lanes 0..7 hold
  // them; the xor shuffles below 8 stay inside that group)
  auto sum8 = [](float v) {
    v += __shfl_xor(v, 1, kWave);
    v += __shfl_xor(v, 2, kWave);
    v += __shfl_xor(v, 4, kWave);
    return v;
  };
  const float total = sum8(rate);
  uint32_t dmin = lx ? dd : 0xFFFFFFFFu, dmax = dd;
#pragma unroll
  for (int m = 1; m < kXcds; m <<= 1) {
    dmin = min(dmin, (uint32_t)__shfl_xor((int)dmin, m, kWave));
    dmax = max(dmax, (uint32_t)__shfl_xor((int)dmax, m, kWave));
  }
  // chunks ending within 1/64 of each other: balanced, the cut stays
  if (ok && total > 0.f && dmax - dmin > dmax / 64) {
    // halfway from the current share to the measured one, kept within
    // [1/16, 3/16] (a little inside, so rounding stays in range)
    const uint32_t c0 = lx ? s_hdr[4 + x] : 0u, c1 = lx ? s_hdr[5 + x] : 0u;
    float sh = lx ? 0.5f * (float)(c1 - c0) / (float)kBalanceOne + 0.5f * rate / total : 0.f;
    for (int it = 0; it < 4; ++it) {
      const float s = sum8(sh);
      sh = lx ? fminf(fmaxf(sh / s, 0.0675f), 0.1825f) : 0.f;
    }
    const float s = sum8(sh);
    float run = sh;  // inclusive scan over the chunk lanes
#pragma unroll
    for (int m = 1; m < kXcds; m <<= 1) {
      const float y = __shfl_up(run, m, kWave);
      if (x >= m) run += y;
    }
    const uint32_t next =
        x + 1 == kXcds ? kBalanceOne : (uint32_t)__float2uint_rn(run / s * kBalanceOne);
    // every lane takes part in the shuffle (a lane left out supplies no value)
    const uint32_t below = (uint32_t)__shfl_up((int)next, 1, kWave);
    const uint32_t prev = x == 0 ? 0u : below;
    const bool bad_x = lx && (next < prev || next - prev < kShareMin || next - prev > kShareMax);
    if (__builtin_amdgcn_ballot_w64(bad_x) == 0) {
      if (lx) h->cum[x + 1] = next;
      if (x == 0) h->cum[0] = 0;
    }
  }
  if (x == 0) h->stamped = 0;
}

// LDS of the stream kernel: the sequence table and scan scratch, then each
// wave's staging area for segment outputs (kStashBytes of entries, then
// kStashEntries descriptors).  An entry holds the 16-byte pieces of lanes
// (c16 < G, g4): piece k of lane j = 4 c16 + g4 at 16 (4 G k + j), so the
// lanes of one store or load cover contiguous bytes (eight pieces of a split
// pair's o, or four of a whole pair's rows), then G (m, l) pairs.
constexpr int kStashBytes = 16384;
constexpr int kStashEntries = 16;
constexpr int kStashWave = kStashBytes + 16 * kStashEntries;
__host__ __device__ constexpr int stash_offset(int num_seqs) {
  return ((3 * num_seqs + 1 + kThreads + kXcds + 1) * 4 + 15) & ~15;
}
__host__ __device__ constexpr int stash_entry_bytes(int group) {
  return (group * 520 + 15) & ~15;
}
static_assert(stash_entry_bytes(16) <= kStashBytes, "one entry of the largest group fits");

size_t stream_smem_bytes(int num_seqs) {
  return (size_t)stash_offset(num_seqs) + (size_t)kWaves * kStashWave;
}

template <class E, KvType KV>
__global__ __launch_bounds__(kThreads) void decode_partition_mfma_stream(DecodeArgs a) {
  constexpr int D = 128;
  using S = typename E::storage;
  using Tile = KvTile<E, KV>;
  using P = typename Tile::P;
  extern __shared__ __attribute__((aligned(16))) int s_int[];
  const int B = a.num_seqs, Hkv = a.num_kv_heads, G = a.group;
  int* s_ctx = s_int;         // [B] clamped lengths, >= 0
  int* s_first = s_ctx + B;   // [B] first attended position (sliding window)
  int* s_tb = s_first + B;    // [B + 1] tile offset of each sequence in a head's run
  int* s_tmp = s_tb + B + 1;  // [kThreads]
  int* s_cut = s_tmp + kThreads;  // [kXcds + 1] the weighted cut, or s_cut[0] = -1
  uint32_t hw[kHeaderCutWords];
  if (threadIdx.x == 0) load_cut_words(a, hw);
  for (int i = threadIdx.x; i < B; i += kThreads) {
    const int ctx = max(clamp_ctx(a, i), 0);
    s_ctx[i] = ctx;
    s_first[i] = first_pos(a, ctx);
  }
  __syncthreads();
  scan_tiles(s_ctx, s_first, s_tb, B, s_tmp);

  const int lane = threadIdx.x % kWave, w = wave_id();
  const int c16 = lane & 15, g4 = lane >> 4;
  const int Th = uni(s_tb[B]);  // tiles of one kv head's run
  if (threadIdx.x == 0) partition_cut(a, (long long)Th * Hkv, (int)gridDim.x, s_cut, hw);
  __syncthreads();
  StreamSplit split{(long long)Th * Hkv, (int)gridDim.x, nullptr, a.xcds};
  if (uni(s_cut[0]) >= 0) split.cut = s_cut;
  const int rank = split.rank(blockIdx.x, w);
  // the pass's record for the balance state: each chunk's tiles, and (at
  // the end) the longest time one of its waves took
  const bool timed = a.ws_balance != nullptr && split.balanced_size();
  const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
  if (timed && blockIdx.x == 0 && threadIdx.x < kXcds) {
    a.ws_balance->tiles[threadIdx.x] =
        (uint32_t)(split.chunk_lo(threadIdx.x + 1) - split.chunk_lo(threadIdx.x));
    if (threadIdx.x == 0) a.ws_balance->stamped = 1;
  }
  const int lo = (int)split.lo(rank), hi = (int)split.lo(rank + 1);
  // rows of empty sequences are zero; spread over the workgroups
  for (int i = blockIdx.x; i < B; i += gridDim.x) {
    if (s_ctx[i] > 0) continue;
    for (int k = threadIdx.x; k < a.num_q_heads * D; k += kThreads)
      reinterpret_cast<S*>(a.out)[(size_t)i * a.num_q_heads * D + k] = 0;
  }
  if (lo >= hi) {  // no barrier follows
    if (lane == 0) reinterpret_cast<int4*>(a.ws_owner)[rank] = int4{-1, 0, 0, 0};
    return;
  }

  const int bs_mask = (1 << a.log2_bs) - 1;
  const size_t head_stride = (size_t)D << a.log2_bs;
  const size_t block_stride = head_stride * Hkv;

  // Position in the flat order: kv head g, sequence i, tile t of its n; the
  // sequence's tiles start at tile ts of its positions (sliding window).
  struct Cur {
    int i, g, t, n, ts;
  };
  auto tiles_of = [&](int i) { return seq_tiles(uni(s_ctx[i]), uni(s_first[i])); };
  auto first_tile = [&](int i) { return uni(s_first[i]) >> 4; };
  auto next_seq = [&](int i) {  // next sequence with tiles, B if none
    do {
      ++i;
    } while (i < B && uni(s_ctx[i]) == 0);
    return i;
  };
  auto advance = [&](Cur& c) {
    if (++c.t < c.n) return;
    c.t = 0;
    c.i = next_seq(c.i);
    if (c.i == B) {
      c.i = next_seq(-1);
      ++c.g;
    }
    c.n = c.g < Hkv ? tiles_of(c.i) : 0;
    c.ts = c.g < Hkv ? first_tile(c.i) : 0;
  };
  Cur start;
  {
    const int g = lo / Th, off = lo - g * Th;
    int l = 0, r = B;  // last sequence whose first tile is <= off; it has tiles
    while (r - l > 1) {
      const int mid = (l + r) >> 1;
      if (uni(s_tb[mid]) <= off) l = mid; else r = mid;
    }
    start = Cur{l, g, off - uni(s_tb[l]), tiles_of(l), first_tile(l)};
  }

  // q rows of one pair through a buffer descriptor bounded to its G heads:
  // lanes with c16 >= G read zeros.  Lane (c16, g4) gets the 8 elements of
  // q[head c16] that k-step s contracts (Tile::q_elem), the B operand layout
  // of the QK product.
  auto load_q = [&](const Cur& c, u32x4 (&dst)[4]) {
    const rsrc_t rs = make_rsrc(reinterpret_cast<const S*>(a.q) +
                                    ((size_t)c.i * a.num_q_heads + (size_t)c.g * G) * D,
                                (uint32_t)(G * D * 2));
#pragma unroll
    for (int s = 0; s < 4; ++s)
      dst[s] = buffer_load16(rs, (uint32_t)(c16 * D + Tile::q_elem(s, g4)) * 2u);
  };

  // ---- issue side: the ring's loads, one tile at a time ----
  // The block id of the next tile is read (scalar load) one issue ahead of
  // its use.  Tiles past the range, or with a block id outside the pool, get
  // an empty buffer descriptor: the loads return zeros without touching
  // memory, and every issue has exactly 8 loads, so the waits stay static.
  // The first tile of a pair also fetches the pair's q into qn, ahead of its
  // K/V, unless qn still holds a q the compute side has not taken (pairs of
  // at most two tiles); that pair then loads q when it starts.
  Cur ic = start;
  int irem = hi - lo;
  auto table_entry = [&](const Cur& c) {
    return scalar_load(a.block_tables + (size_t)c.i * a.max_blocks +
                       (((c.t + c.ts) * kTile) >> a.log2_bs));
  };
  int iblk = table_entry(ic);
  u32x4 qn[4];
  bool qn_full = false;
  int qn_i = 0, qn_g = 0;
  bool bad = false;  // a tile of the run named a block outside the pool
  auto issue = [&](Tile& tile) -> bool {
    bool ok = false;
    size_t off = 0;
    if (irem > 0) {
      if (ic.t == 0 && !qn_full && irem < hi - lo) {
        load_q(ic, qn);
        qn_full = true;
        qn_i = ic.i;
        qn_g = ic.g;
      }
      ok = (unsigned)iblk < (unsigned)a.num_blocks;
      bad |= !ok;
      if (ok)
        off = (size_t)iblk * block_stride + (size_t)ic.g * head_stride +
              (size_t)(((ic.t + ic.ts) * kTile) & bs_mask) * D;
      if (--irem > 0) {
        advance(ic);
        iblk = table_entry(ic);
      }
    }
    const uint32_t bytes = ok ? Tile::kBytes : 0u;
    tile.load(make_rsrc(reinterpret_cast<const P*>(a.k_pool) + off, bytes),
              make_rsrc(reinterpret_cast<const P*>(a.v_pool) + off, bytes), c16, g4);
    return ok;
  };

  // ---- compute side ----
  Cur cc = start;
  int crem = hi - lo;
  int seg_t0 = 0, ctx_c = 0, first_c = 0;
  u32x4 qv[4];
  float m = neg_inf(), l = 0.f;
  f32x4 o[8];

  // A segment is the run of the current pair's tiles inside this range.
  auto begin_segment = [&]() {
    seg_t0 = cc.t;
    ctx_c = uni(s_ctx[cc.i]);
    first_c = uni(s_first[cc.i]);
    if (qn_full && qn_i == cc.i && qn_g == cc.g) {
#pragma unroll
      for (int s = 0; s < 4; ++s) qv[s] = qn[s];
      qn_full = false;
    } else {
      // Rare (start of the range, or a pair of at most two tiles): wait for
      // the load here, so the join does not leave qv pending in every path.
      load_q(cc, qv);
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
    }
    m = neg_inf();
    l = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  // One tile, as in decode_partition_mfma (lazy rescale, P rounded to the
  // 16-bit operand type and summed as rounded, rows outside [first, ctx)
  // masked).
  auto compute = [&](const Tile& tile) {
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) sacc = Mfma<E>::qk(tile.k_op(t), qv[t], sacc);
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[r] = sacc[r] * a.scale_log2;
    u32x4 vc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) vc[r] = tile.v_row(r);
    const int tok = kTile * (cc.t + cc.ts);
    const int valid = ctx_c - tok, low = first_c - tok;
    if (valid < kTile || low > 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = 4 * g4 + r;
        if (e >= valid || e < low) {
          sv[r] = neg_inf();
          vc[r] = u32x4{0, 0, 0, 0};
        }
      }
    }
    const float lim = m + kRescaleSlack;
    const bool over = sv[0] > lim || sv[1] > lim || sv[2] > lim || sv[3] > lim;
    if (__builtin_amdgcn_ballot_w64(over)) {
      float mt = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      mt = fmaxf(mt, shfl_xor(mt, 16));
      mt = fmaxf(mt, shfl_xor(mt, 32));
      const float mn = fmaxf(m, mt);
      const float alpha = fast_exp2(m - mn);
      l *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] *= alpha;
      m = mn;
    }
    uint32_t pb[4];
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pb[r] = Mfma<E>::round16(fast_exp2(sv[r] - m));
      psum += bits_to_float(E{}, pb[r]);
    }
    l += psum;
    const u32x2 pw = {pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16)};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      const u32x2 vw = {__builtin_amdgcn_perm(vc[1][e >> 1], vc[0][e >> 1], sel),
                        __builtin_amdgcn_perm(vc[3][e >> 1], vc[2][e >> 1], sel)};
      o[e] = Mfma<E>::pv(vw, pw, o[e]);
    }
  };

  // Segment outputs go through the wave's LDS staging area: `nst` entries
  // held, each described by (whole, sequence, kv head).
  char* const sd = reinterpret_cast<char*>(s_int) + stash_offset(B) + w * kStashWave;
  int4* const sdesc = reinterpret_cast<int4*>(sd + kStashBytes);
  const int es = stash_entry_bytes(G);
  const int cap = min(kStashEntries, kStashBytes / es);
  const int lj = 16 * (4 * c16 + g4), lk = 64 * G;  // lane's piece 0, piece stride
  int nst = 0;
  // Write the held entries: a whole pair's rows to `out`, a split pair's
  // (m, l, o) to slot (pair + rank).
  auto flush = [&]() {
    for (int e = 0; e < nst; ++e) {
      const int4 dsc = sdesc[e];
      const int whole = uni(dsc.x), i = uni(dsc.y), g = uni(dsc.z);
      const char* src = sd + e * es;
      if (c16 < G) {
        if (whole) {
          S* dst = reinterpret_cast<S*>(a.out) +
                   ((size_t)i * a.num_q_heads + (size_t)g * G + c16) * D + 32 * g4;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            *reinterpret_cast<u32x4*>(dst + 8 * r) =
                *reinterpret_cast<const u32x4*>(src + lj + lk * r);
        } else {
          const size_t slot = (size_t)g * B + i + rank;
          float* dst = a.ws_o + (slot * G + c16) * D + 32 * g4;
#pragma unroll
          for (int k = 0; k < 8; ++k)
            *reinterpret_cast<f32x4*>(dst + 4 * k) =
                *reinterpret_cast<const f32x4*>(src + lj + lk * k);
          if (g4 == 0)
            a.ws_ml[slot * G + c16] = *reinterpret_cast<const float2*>(src + G * 512 + 8 * c16);
        }
      }
    }
    nst = 0;
  };
  // End of a segment: the normalised rows when it is the whole pair, else its
  // (m, l, o), into the next entry.  Lane (c16, g4) holds
  // O[head c16][32 g4 + 8 r + e] = o[e][r].
  auto end_segment = [&]() {
    const float lsum = across_groups_sum<16>(l);
    const bool whole = seg_t0 == 0 && cc.t + 1 == cc.n;
    if (nst == cap) flush();
    char* dst = sd + nst * es;
    if (c16 < G) {
      if (whole) {
        const float inv = lsum > 0.f ? a.v_scale / lsum : 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *reinterpret_cast<u32x4*>(dst + lj + lk * r) =
              u32x4{Mfma<E>::round16x2(o[0][r] * inv, o[1][r] * inv),
                    Mfma<E>::round16x2(o[2][r] * inv, o[3][r] * inv),
                    Mfma<E>::round16x2(o[4][r] * inv, o[5][r] * inv),
                    Mfma<E>::round16x2(o[6][r] * inv, o[7][r] * inv)};
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          *reinterpret_cast<f32x4*>(dst + lj + lk * (2 * r)) = f32x4{o[0][r], o[1][r], o[2][r], o[3][r]};
          *reinterpret_cast<f32x4*>(dst + lj + lk * (2 * r + 1)) = f32x4{o[4][r], o[5][r], o[6][r], o[7][r]};
        }
        if (g4 == 0) *reinterpret_cast<float2*>(dst + G * 512 + 8 * c16) = make_float2(m, lsum);
      }
    }
    if (lane == 0) sdesc[nst] = int4{whole ? 1 : 0, cc.i, cc.g, 0};
    ++nst;
  };

  begin_segment();
  Tile tb[kStreamPrefetch];
  bool okb[kStreamPrefetch];
#pragma unroll
  for (int s = 0; s < kStreamPrefetch; ++s) okb[s] = issue(tb[s]);
  // Every slot issues on every path (past the range the descriptors are
  // empty) and the loop only exits at the bottom of the unrolled body: all
  // paths then carry the same load sequence, so no path in which some slot
  // was issued last can reach the loop header and make the waits
  // conservative.
  do {
#pragma unroll
    for (int s = 0; s < kStreamPrefetch; ++s) {
      const bool live = crem > 0;
      if (live && okb[s]) compute(tb[s]);
      okb[s] = issue(tb[s]);
      if (live) {
        --crem;
        if (cc.t + 1 == cc.n || crem == 0) {
          end_segment();
          if (crem > 0) {
            advance(cc);
            begin_segment();
          }
        } else {
          ++cc.t;
        }
      }
    }
  } while (crem > 0);
  flush();

  report_bad_block(a.status, bad);
  // The run's last segment (still in cc): if it starts its pair and the pair
  // goes on, this rank owns the pair's merge.  Only a last segment can.
  if (lane == 0) {
    int4 rec = {-1, 0, 0, 0};
    if (seg_t0 == 0 && cc.t + 1 < cc.n) {
      const long long last = (long long)cc.g * Th + uni(s_tb[cc.i]) + cc.n - 1;
      rec = int4{(int)((size_t)cc.g * B + cc.i), split.rank_of(last) - rank + 1, Th,
                 split.dense()};
    }
    reinterpret_cast<int4*>(a.ws_owner)[rank] = rec;
    if (timed) a.ws_balance->wave_dur[rank] = (uint32_t)(__builtin_amdgcn_s_memrealtime() - t_start);
  }
}

// ----------------------------------------------------------------- VALU path
// Lanes along head_dim: a K/V row of D elements is LPR lanes x 16 bytes; one
// 16-byte load per lane covers RPL rows; a 16-token tile is LPT loads.
template <class E, int D, int G>
__global__ __launch_bounds__(kThreads) void decode_partition_valu(DecodeArgs a) {
  constexpr int EB = E::bytes;
  constexpr int EPL = 16 / EB;
  constexpr int LPR = D * EB / 16;
  constexpr int RPL = kWave / LPR;
  constexpr int LPT = kTile / RPL;
  extern __shared__ float smem[];
  const int g = blockIdx.x, i = blockIdx.y;
  const int p = (int)(gridDim.z - 1 - blockIdx.z);  // last partitions first
  const int ctx = clamp_ctx(a, i);
  const int n_parts = num_parts(a, ctx);
  if (p >= n_parts) return;
  if (ctx <= 0) {
    store_zero_rows<E, D>(a, G, i, g);
    return;
  }
  const int lane = threadIdx.x % kWave, w = wave_id();
  const int r0 = lane / LPR, cl = lane % LPR;
  const int first = first_pos(a, ctx);
  const int t0 = (first & ~(kTile - 1)) + p * a.part_tokens;
  const int ntok = min(a.part_tokens, ctx - t0);
  const int ntiles = (ntok + kTile - 1) / kTile;
  const int bs_mask = (1 << a.log2_bs) - 1;

  using S = typename E::storage;
  float qf[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const S* qrow = reinterpret_cast<const S*>(a.q) +
                    ((size_t)i * a.num_q_heads + (size_t)g * G + h) * D + cl * EPL;
    const u32x4 c = load16(qrow);
    const uint4 cu = {c[0], c[1], c[2], c[3]};
#pragma unroll
    for (int e = 0; e < EPL; ++e) qf[h][e] = chunk_elem(E{}, cu, e) * a.scale_log2;
  }
  const int32_t* table = a.block_tables + (size_t)i * a.max_blocks;
  const size_t head_stride = (size_t)D << a.log2_bs;
  const size_t block_stride = head_stride * a.num_kv_heads;
  const S* kbase = reinterpret_cast<const S*>(a.k_pool) + (size_t)g * head_stride + r0 * D + cl * EPL;
  const S* vbase = reinterpret_cast<const S*>(a.v_pool) + (size_t)g * head_stride + r0 * D + cl * EPL;

  bool bad = false;  // a tile of the partition named a block outside the pool
  auto load_tile = [&](int j, uint4 (&kr)[LPT], uint4 (&vr)[LPT]) -> bool {
    const int tok = t0 + kTile * j;
    const int blk = table[tok >> a.log2_bs];
    if ((unsigned)blk >= (unsigned)a.num_blocks) {
      bad = true;
      return false;
    }
    const size_t off = (size_t)blk * block_stride + (size_t)(tok & bs_mask) * D;
#pragma unroll
    for (int k = 0; k < LPT; ++k) {
      const u32x4 x = load16(kbase + off + (size_t)k * RPL * D);
      const u32x4 y = load16(vbase + off + (size_t)k * RPL * D);
      kr[k] = uint4{x[0], x[1], x[2], x[3]};
      vr[k] = uint4{y[0], y[1], y[2], y[3]};
    }
    return true;
  };

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = neg_inf();
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  int j = w;
  uint4 kc[LPT], vc[LPT];
  bool okc = j < ntiles && load_tile(j, kc, vc);
  for (; j < ntiles; j += kWaves) {
    uint4 kn[LPT], vn[LPT];
    bool okn = false;
    if (j + kWaves < ntiles) okn = load_tile(j + kWaves, kn, vn);
    if (okc) {
      const int valid = ntok - kTile * j, low = first - (t0 + kTile * j);
      float s[G][LPT];
#pragma unroll
      for (int k = 0; k < LPT; ++k) {
        float kf[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) kf[e] = chunk_elem(E{}, kc[k], e);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float part = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) part = fmaf(qf[h][e], kf[e], part);
          s[h][k] = group_sum<LPR>(part);
        }
      }
      if (valid < kTile || low > 0) {
#pragma unroll
        for (int k = 0; k < LPT; ++k) {
          if (k * RPL + r0 >= valid || k * RPL + r0 < low) {
#pragma unroll
            for (int h = 0; h < G; ++h) s[h][k] = neg_inf();
            vc[k] = uint4{0, 0, 0, 0};
          }
        }
      }
      float vf[LPT][EPL];
#pragma unroll
      for (int k = 0; k < LPT; ++k)
#pragma unroll
        for (int e = 0; e < EPL; ++e) vf[k][e] = chunk_elem(E{}, vc[k], e);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float mt = s[h][0];
#pragma unroll
        for (int k = 1; k < LPT; ++k) mt = fmaxf(mt, s[h][k]);
        mt = across_groups_max<LPR>(mt);
        const float mn = fmaxf(m[h], mt);
        const float alpha = fast_exp2(m[h] - mn);
        m[h] = mn;
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
#pragma unroll
        for (int k = 0; k < LPT; ++k) {
          const float pk = fast_exp2(s[h][k] - mn);
          l[h] += pk;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pk, vf[k][e], acc[h][e]);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < LPT; ++k) {
      kc[k] = kn[k];
      vc[k] = vn[k];
    }
    okc = okn;
  }

  report_bad_block(a.status, bad);
  float* sm_m = smem;
  float* sm_l = smem + kWaves * 16;
  float* sm_o = smem + 2 * kWaves * 16;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l[h] = across_groups_sum<LPR>(l[h]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = across_groups_sum<LPR>(acc[h][e]);
  }
  if (r0 == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (cl == 0) {
        sm_m[w * 16 + h] = m[h];
        sm_l[w * 16 + h] = l[h];
      }
      float* dst = sm_o + ((size_t)w * G + h) * o_stride<D>() + cl * EPL;
#pragma unroll
      for (int e = 0; e < EPL; ++e) dst[e] = acc[h][e];
    }
  }
  __syncthreads();
  combine_store<E, D>(a, smem, G, i, g, p, n_parts);
}

// ----------------------------------------------------------------- reduce
// Merges the n partial states (m_k, l_k, o_k) of one output row in one pass
// and writes the normalised row (zeros when the total weight is 0).  A lane
// covers 8 consecutive outputs, so D / 8 lanes cover a vector and the wave's
// 64 / (D / 8) lane groups walk disjoint states k = group, group + groups,
// ..., U at a time, each group with its own running maximum; the groups are
// merged at the end.  The (m, l) and o loads of a step are independent of
// each other and of the maximum, so a row costs one round of loads.
// ok(k): state k exists; ml(k): its (m, l); ov(k): its D outputs.  The
// outputs are scaled by `factor` (an 8-bit pool's v_scale, else 1).
template <class E, int D, class Ok, class Ml, class Ov>
__device__ void merge_row(int n, Ok ok, Ml ml, Ov ov, typename E::storage* out, float factor) {
  constexpr int LPR = D / 8;           // lanes per output vector
  constexpr int GROUPS = kWave / LPR;  // states walked side by side
  constexpr int U = 4;
  const int lane = threadIdx.x % kWave, grp = lane / LPR, col = (lane % LPR) * 8;
  float Mg = neg_inf(), Lg = 0.f;
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  for (int k0 = grp; k0 < n; k0 += GROUPS * U) {
    float2 st[U];
    f32x4 o[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = k0 + u * GROUPS;
      const bool in = k < n && ok(k);
      st[u] = in ? ml(k) : make_float2(neg_inf(), 0.f);
      const f32x4* src = reinterpret_cast<const f32x4*>(ov(k) + col);
      o[u][0] = in ? src[0] : f32x4{0.f, 0.f, 0.f, 0.f};
      o[u][1] = in ? src[1] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float Mn = Mg;
#pragma unroll
    for (int u = 0; u < U; ++u) Mn = fmaxf(Mn, st[u].x);
    if (Mn != neg_inf()) {
      const float sc = fast_exp2(Mg - Mn);  // 0 while the group is empty
      Lg *= sc;
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] *= sc;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float wt = fast_exp2(st[u].x - Mn);
        Lg = fmaf(wt, st[u].y, Lg);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          acc[k] = fmaf(wt, o[u][0][k], acc[k]);
          acc[4 + k] = fmaf(wt, o[u][1][k], acc[4 + k]);
        }
      }
      Mg = Mn;
    }
  }
  const float M = across_groups_max<LPR>(Mg);
  const float sc = Mg == neg_inf() ? 0.f : fast_exp2(Mg - M);
  const float L = across_groups_sum<LPR>(Lg * sc);
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = across_groups_sum<LPR>(acc[k] * sc);
  if (grp == 0) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      out[col + k] =
          (typename E::storage)float_to_bits(E{}, L > 0.f ? acc[k] / L * factor : 0.f);
  }
}

// Grid split: one wave per (sequence, q head) with more than one partition.
template <class E, int D>
__global__ __launch_bounds__(kWave) void decode_reduce(DecodeArgs a) {
  const int h = blockIdx.x, i = blockIdx.y;
  const int n_parts = num_parts(a, clamp_ctx(a, i));
  if (n_parts <= 1) return;
  const size_t row = (size_t)i * a.num_q_heads + h;
  const float2* ml = a.ws_ml + row * a.max_parts;
  const float* wo = a.ws_o + row * a.max_parts * D;
  merge_row<E, D>(
      n_parts, [](int) { return true; }, [&](int k) { return ml[k]; },
      [&](int k) { return wo + (size_t)k * D; },
      reinterpret_cast<typename E::storage*>(a.out) + row * D, a.v_scale);
}

// Stream split: one workgroup per wave rank r of the partition pass.  If r
// owns a pair, its n segments are slots (pair + r), ..., (pair + r + n - 1);
// a rank with an empty run (possible only with fewer tiles than waves, when
// the record says so) left nothing and is skipped.  Wave w merges q heads
// w, w + 4, ... of the pair's G.
template <class E>
__global__ __launch_bounds__(kThreads) void decode_reduce_stream(DecodeArgs a) {
  constexpr int D = 128;
  const int r = blockIdx.x;
  // one workgroup past the records updates the balance state, beside the
  // merges rather than ahead of one of them
  if (r == a.stream_waves) {
    if (a.ws_balance != nullptr) update_balance(a.ws_balance, a.stream_waves / kWaves);
    return;
  }
  const int4 rec = reinterpret_cast<const int4*>(a.ws_owner)[r];
  const int pq = rec.x;
  if (pq < 0) return;
  const int B = a.num_seqs, G = a.group;
  const int g = pq / B, i = pq - g * B;
  // records of weighted passes are dense; others were cut evenly
  const StreamSplit split{(long long)rec.z * a.num_kv_heads, a.stream_waves / kWaves, nullptr, a.xcds};
  const bool dense = rec.w != 0;
  const size_t base = (size_t)pq + r;
  for (int hh = wave_id(); hh < G; hh += kWaves) {
    merge_row<E, D>(
        rec.y, [&](int k) { return dense || split.lo(r + k) < split.lo(r + k + 1); },
        [&](int k) { return a.ws_ml[(base + k) * G + hh]; },
        [&](int k) { return a.ws_o + ((base + k) * G + hh) * D; },
        reinterpret_cast<typename E::storage*>(a.out) +
            ((size_t)i * a.num_q_heads + (size_t)g * G + hh) * D,
        a.v_scale);
  }
}

// ----------------------------------------------------------------- launchers
namespace {

template <class E, int D, int G>
pa_status launch_valu(const DecodeArgs& a, hipStream_t st) {
  const dim3 grid(a.num_kv_heads, a.num_seqs, a.max_parts);
  hipLaunchKernelGGL((decode_partition_valu<E, D, G>), grid, dim3(kThreads),
                     merge_smem_bytes<D>(G), st, a);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

template <class E, int D>
pa_status launch_valu_g(const DecodeArgs& a, hipStream_t st) {
  switch (a.group) {
    case 1: return launch_valu<E, D, 1>(a, st);
    case 2: return launch_valu<E, D, 2>(a, st);
    case 4: return launch_valu<E, D, 4>(a, st);
    case 8: return launch_valu<E, D, 8>(a, st);
    default: return PA_ERR_SHAPE;
  }
}

template <class E>
pa_status launch_valu_d(const DecodeArgs& a, int head_dim, hipStream_t st) {
  return head_dim == 64 ? launch_valu_g<E, 64>(a, st) : launch_valu_g<E, 128>(a, st);
}

template <class E, KvType KV>
pa_status launch_mfma(const DecodeArgs& a, hipStream_t st) {
  const dim3 grid(a.num_kv_heads, a.num_seqs, a.max_parts);
  hipLaunchKernelGGL((decode_partition_mfma<E, KV>), grid, dim3(kThreads),
                     merge_smem_bytes<128>(a.group), st, a);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

// Compute units of the current device (cached per device).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load();
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
    cache[dev].store(n);
  }
  return n;
}

template <class E, KvType KV>
pa_status launch_mfma_stream(const DecodeArgs& a, hipStream_t st) {
  if (a.stream_waves <= 0 || a.stream_waves % kWaves != 0) return PA_ERR_ARG;
  hipLaunchKernelGGL((decode_partition_mfma_stream<E, KV>), dim3(a.stream_waves / kWaves),
                     dim3(kThreads), stream_smem_bytes(a.num_seqs), st, a);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

template <class E>
pa_status launch_reduce_stream(const DecodeArgs& a, hipStream_t st) {
  // one workgroup per merge record, plus one for the balance update
  hipLaunchKernelGGL((decode_reduce_stream<E>), dim3(a.stream_waves + (a.ws_balance != nullptr ? 1 : 0)),
                     dim3(kThreads), 0, st, a);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

template <class E, int D>
pa_status launch_reduce(const DecodeArgs& a, hipStream_t st) {
  const dim3 grid(a.num_q_heads, a.num_seqs);
  hipLaunchKernelGGL((decode_reduce<E, D>), grid, dim3(kWave), 0, st, a);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

int device_xcds() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kXcds;
  int n = cache[dev].load();
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || n <= 0) n = kXcds;
    n = std::min(n, kXcds);
    cache[dev].store(n);
  }
  return n;
}

int stream_waves() {
  const int cus = device_cus();
  if (cus <= 0) return 0;
  return std::min(kStreamWgPerCu * cus, kStreamMaxWaves / kWaves) * kWaves;
}

bool stream_supports(int num_seqs, int num_kv_heads, int max_ctx) {
  if (num_seqs > kStreamMaxSeqs) return false;  // sequence table in LDS
  const long long tiles_per_seq = ((long long)max_ctx + kTile - 1) / kTile;
  return tiles_per_seq * num_kv_heads * num_seqs < (1ll << 31);  // 32-bit flat tile ids
}

bool mfma_supports(int dtype, int head_dim, int group) {
  return (dtype == PA_F16 || dtype == PA_BF16) && head_dim == 128 && group >= 1 && group <= 16;
}

bool valu_supports(int /*dtype*/, int head_dim, int group) {
  return (head_dim == 64 || head_dim == 128) &&
         (group == 1 || group == 2 || group == 4 || group == 8);
}

pa_status launch_decode_partition(const DecodeArgs& a, int dtype, KvType kv, int head_dim,
                                  DecodeKernel k, hipStream_t st) {
  const bool fp8 = kv == KvType::kFp8;
  if (k == DecodeKernel::kMfmaStream) {
    if (dtype == PA_BF16)
      return fp8 ? launch_mfma_stream<BF16, KvType::kFp8>(a, st)
                 : launch_mfma_stream<BF16, KvType::kSame>(a, st);
    if (dtype == PA_F16)
      return fp8 ? launch_mfma_stream<F16, KvType::kFp8>(a, st)
                 : launch_mfma_stream<F16, KvType::kSame>(a, st);
    return PA_ERR_SHAPE;
  }
  if (k == DecodeKernel::kMfmaGrid) {
    if (dtype == PA_BF16)
      return fp8 ? launch_mfma<BF16, KvType::kFp8>(a, st) : launch_mfma<BF16, KvType::kSame>(a, st);
    if (dtype == PA_F16)
      return fp8 ? launch_mfma<F16, KvType::kFp8>(a, st) : launch_mfma<F16, KvType::kSame>(a, st);
    return PA_ERR_SHAPE;
  }
  if (fp8) return PA_ERR_SHAPE;
  switch (dtype) {
    case PA_F32: return launch_valu_d<F32>(a, head_dim, st);
    case PA_F16: return launch_valu_d<F16>(a, head_dim, st);
    case PA_BF16: return launch_valu_d<BF16>(a, head_dim, st);
    default: return PA_ERR_DTYPE;
  }
}

pa_status launch_decode_reduce(const DecodeArgs& a, int dtype, int head_dim, DecodeKernel k,
                               hipStream_t st) {
  if (k == DecodeKernel::kMfmaStream) {
    if (dtype == PA_BF16) return launch_reduce_stream<BF16>(a, st);
    if (dtype == PA_F16) return launch_reduce_stream<F16>(a, st);
    return PA_ERR_SHAPE;
  }
  const bool d64 = head_dim == 64;
  switch (dtype) {
    case PA_F32: return d64 ? launch_reduce<F32, 64>(a, st) : launch_reduce<F32, 128>(a, st);
    case PA_F16: return d64 ? launch_reduce<F16, 64>(a, st) : launch_reduce<F16, 128>(a, st);
    case PA_BF16: return d64 ? launch_reduce<BF16, 64>(a, st) : launch_reduce<BF16, 128>(a, st);
    default: return PA_ERR_DTYPE;
  }
}

}  // namespace pa
