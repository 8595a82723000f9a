// Read ceiling of the decode access pattern, a measurement aid.  The decode
// kernel is bound by memory (page "vLLM：把 KV 缓存当成虚拟内存", section "KV
// 的体积从哪来，页表如何把它切开": decode reads every cached K/V row once per
// step), but a step's tiles are scattered over the pool in 4 KiB pieces, and
// such reads do not reach the part's sequential bandwidth.  This kernel reads
// a list of tiles with the decode stream kernel's work split and nothing
// else: one 4-wave workgroup per compute unit, each wave a contiguous run of
// the list, 32 16-byte loads in flight per wave, each tile's offset read by a
// scalar load one tile ahead.  Its rate over a step's tiles is what that
// access pattern allows, the ceiling the attention kernel is measured against.
#include <hip/hip_runtime.h>

#include "pa.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kProbeWaves = 4;  // waves per workgroup

// C: 16-byte chunks per lane per tile (tile_bytes / 1024); NP: pools read
// per tile (1, or 2: the tile's bytes at the same offset of both, as the
// decode kernel reads a (block, head)'s K and V together); R: tiles in flight
// per wave (32 loads, or 1 tile when no wave has more than one, so the kernel
// holds few registers and many waves fit).  out[rank] = the XOR of every
// 32-bit word the wave read.
template <int C, int NP, int R>
__global__ __launch_bounds__(kProbeWaves * kWave) void probe_read_tiles(
    const char* pool0, const char* pool1, uint32_t pool_bytes, const uint32_t* offs, int64_t n,
    uint32_t* out) {
  const int lane = threadIdx.x % kWave;
  const int waves = (int)gridDim.x * kProbeWaves;
  const int rank = (int)blockIdx.x * kProbeWaves + (int)threadIdx.x / kWave;
  const int64_t lo = n * rank / waves, hi = n * (rank + 1) / waves;
  const rsrc_t full0 = make_rsrc(pool0, pool_bytes), full1 = make_rsrc(pool1, pool_bytes);
  const rsrc_t none = make_rsrc(pool0, 0u);
  int64_t t_issue = lo;
  uint32_t next = lo < hi ? (uint32_t)scalar_load(reinterpret_cast<const int32_t*>(offs + lo)) : 0u;
  // the next tile of the run (past its end: an empty descriptor, zeros)
  auto issue = [&](u32x4_t (&b)[NP * C]) {
    const bool live = t_issue < hi;
    const uint32_t off = next;
    ++t_issue;
    if (t_issue < hi) next = (uint32_t)scalar_load(reinterpret_cast<const int32_t*>(offs + t_issue));
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const rsrc_t r = live ? (q == 0 ? full0 : full1) : none;
#pragma unroll
      for (int c = 0; c < C; ++c)
        b[q * C + c] = buffer_load16(r, off + 16u * (uint32_t)(lane + kWave * c));
    }
  };
  u32x4_t buf[R][NP * C];
  u32x4_t acc = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int k = 0; k < R; ++k) issue(buf[k]);
  for (int64_t t = lo; t < hi; t += R) {
#pragma unroll
    for (int k = 0; k < R; ++k) {
#pragma unroll
      for (int c = 0; c < NP * C; ++c) acc ^= buf[k][c];
      issue(buf[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < R; ++k)  // past the run: zeros, folded so every load is waited for
#pragma unroll
    for (int c = 0; c < NP * C; ++c) acc ^= buf[k][c];
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) x ^= (uint32_t)__shfl_xor((int)x, m, kWave);
  if (lane == 0) out[rank] = x;
}

template <int C, int NP>
void launch(bool single, dim3 grid, dim3 block, hipStream_t st, const char* p0, const char* p1,
            uint32_t pool_bytes, const uint32_t* offs, int64_t n, uint32_t* out) {
  if (single)
    hipLaunchKernelGGL((probe_read_tiles<C, NP, 1>), grid, block, 0, st, p0, p1, pool_bytes, offs,
                       n, out);
  else
    hipLaunchKernelGGL((probe_read_tiles<C, NP, 32 / (NP * C)>), grid, block, 0, st, p0, p1,
                       pool_bytes, offs, n, out);
}

template <int C>
void launch_np(bool two, bool single, dim3 grid, dim3 block, hipStream_t st, const char* p0,
               const char* p1, uint32_t pool_bytes, const uint32_t* offs, int64_t n,
               uint32_t* out) {
  if (two)
    launch<C, 2>(single, grid, block, st, p0, p1, pool_bytes, offs, n, out);
  else
    launch<C, 1>(single, grid, block, st, p0, p0, pool_bytes, offs, n, out);
}

}  // namespace

pa_status launch_probe_reads(const void* pool, const void* pool2, uint32_t pool_bytes,
                             const uint32_t* offs, int64_t n, int tile_bytes, uint32_t* out,
                             int waves, hipStream_t st) {
  const dim3 grid((unsigned)(waves / kProbeWaves)), block(kProbeWaves * kWave);
  const char* p0 = static_cast<const char*>(pool);
  const char* p1 = static_cast<const char*>(pool2);
  const bool two = pool2 != nullptr, single = n <= waves;  // single: at most one tile per wave
  switch (tile_bytes) {
    case 1024: launch_np<1>(two, single, grid, block, st, p0, p1, pool_bytes, offs, n, out); break;
    case 2048: launch_np<2>(two, single, grid, block, st, p0, p1, pool_bytes, offs, n, out); break;
    case 4096: launch_np<4>(two, single, grid, block, st, p0, p1, pool_bytes, offs, n, out); break;
    default: return PA_ERR_ARG;
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace pa
