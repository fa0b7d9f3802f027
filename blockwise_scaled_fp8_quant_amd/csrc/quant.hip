// Activation (1x128) and weight (128x128) quantizers for gfx950.
//
// Both are HBM streams: 2 bytes of bf16 read and 1 byte of E4M3 written per
// element, plus one fp32 scale per block.  Loads are 16 bytes per lane and
// cover whole 128-byte lines; the block |max| is reduced in registers and
// through DPP lane exchanges, never through memory.
#include "fp8q_device.h"
#include "fp8q_internal.h"

namespace fp8q {

// ---------------------------------------------------------------------------
// 1x128 activation blocks (page "NVIDIA NeMo RL erreicht 48% ...", section
// "Der technische Durchbruch"; recomputed on every call, section
// "Leistungsgewinne in der Praxis").
//
// Because K is a multiple of 128 the row-major [M][K] tensor is a flat
// sequence of M*K/128 blocks, and block b's scale is scales[b].  Eight lanes
// own one block (256 bytes of bf16): lane j of the group reads chunks j and
// j+8 (16 bytes each), so one load instruction of the group covers one full
// 128-byte line.  A workgroup of 256 lanes handles 32 blocks per unroll step.
// ---------------------------------------------------------------------------
constexpr int kActThreads = 256;
constexpr int kActUnroll = 2;
constexpr int kActBlocksPerStep = kActThreads / 8;

template <int kMode>
__global__ __launch_bounds__(kActThreads) void quant_act_1x128_kernel(
    const uint16_t *__restrict__ x, uint8_t *__restrict__ q,
    float *__restrict__ scales, int64_t nblocks) {
  const int sub = threadIdx.x & 7;
  const int64_t first = (int64_t)blockIdx.x * (kActBlocksPerStep * kActUnroll) + (threadIdx.x >> 3);

  uint4 v[kActUnroll][2];
#pragma unroll
  for (int u = 0; u < kActUnroll; ++u) {
    const int64_t b = first + u * kActBlocksPerStep;
    if (b < nblocks) {
      const uint4 *p = reinterpret_cast<const uint4 *>(x + b * 128);
      v[u][0] = load_stream16(p + sub);
      v[u][1] = load_stream16(p + sub + 8);
    }
  }
#pragma unroll
  for (int u = 0; u < kActUnroll; ++u) {
    const int64_t b = first + u * kActBlocksPerStep;
    if (b < nblocks) {  // uniform over each group of 8 lanes
      float amax = chunk_absmax(v[u][1], chunk_absmax(v[u][0], 0.0f));
      amax = group8_max(amax);
      const BlockQ p = block_params<kMode>(amax);
      if (sub == 0) scales[b] = p.s;
      uint2 *o = reinterpret_cast<uint2 *>(q + b * 128);
      o[sub] = quant_chunk<kMode>(p, v[u][0]);
      o[sub + 8] = quant_chunk<kMode>(p, v[u][1]);
    }
  }
}

hipError_t launch_quant_act_1x128(const uint16_t *x, int64_t M, int64_t K,
                                  uint8_t *q, float *s, int mode,
                                  hipStream_t stream) {
  const int64_t nblocks = M * (K / 128);
  if (nblocks == 0) return hipSuccess;
  const int64_t per_wg = kActBlocksPerStep * kActUnroll;
  const int64_t grid = (nblocks + per_wg - 1) / per_wg;
  if (mode == kModeAmax)
    hipLaunchKernelGGL(quant_act_1x128_kernel<kModeAmax>, dim3((unsigned)grid), dim3(kActThreads), 0,
                       stream, x, q, s, nblocks);
  else
    hipLaunchKernelGGL(quant_act_1x128_kernel<kModePow2>, dim3((unsigned)grid), dim3(kActThreads), 0,
                       stream, x, q, s, nblocks);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 128x128 weight tiles (page 1, "Der technische Durchbruch"; recalibrated after
// every policy update, "Leistungsgewinne in der Praxis"; power-of-two option,
// "Warum dies fuer die KI-Oekonomie wichtig ist").
//
// One workgroup of 256 lanes per tile: lane t reads the 16-byte chunk t%16 of
// rows t/16 + 16*i, i = 0..7 (16 lanes cover a 256-byte row segment), keeps the
// 64 values in registers, reduces the tile |max| (DPP within each row of 16
// lanes, then the 16 row maxima through LDS), and writes 8 bytes per chunk.
// ---------------------------------------------------------------------------
constexpr int kWThreads = 256;

template <int kMode>
__global__ __launch_bounds__(kWThreads) void quant_weight_128x128_kernel(
    const uint16_t *__restrict__ w, uint8_t *__restrict__ q,
    float *__restrict__ scales, int64_t K, int64_t KB) {
  __shared__ float part[kWThreads / 16];
  const int64_t tile = blockIdx.x;
  const int64_t nb = tile / KB, kb = tile - nb * KB;
  const int c = threadIdx.x & 15;
  const int r0 = threadIdx.x >> 4;
  const uint16_t *base = w + (nb * 128 + r0) * K + kb * 128 + c * 8;

  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    v[i] = load_stream16(base + (int64_t)(16 * i) * K);

  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = chunk_absmax(v[i], amax);
  amax = group16_max(amax);
  if (c == 0) part[r0] = amax;
  __syncthreads();
  amax = part[0];
#pragma unroll
  for (int i = 1; i < kWThreads / 16; ++i) amax = __builtin_fmaxf(amax, part[i]);

  const BlockQ p = block_params<kMode>(amax);
  if (threadIdx.x == 0) scales[tile] = p.s;
  uint8_t *obase = q + (nb * 128 + r0) * K + kb * 128 + c * 8;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<uint2 *>(obase + (int64_t)(16 * i) * K) = quant_chunk<kMode>(p, v[i]);
}

hipError_t launch_quant_weight_128x128(const uint16_t *w, int64_t N, int64_t K,
                                       uint8_t *q, float *s, int mode,
                                       hipStream_t stream) {
  const int64_t KB = K / 128;
  const int64_t tiles = (N / 128) * KB;
  if (tiles == 0) return hipSuccess;
  if (mode == kModeAmax)
    hipLaunchKernelGGL(quant_weight_128x128_kernel<kModeAmax>, dim3((unsigned)tiles), dim3(kWThreads), 0,
                       stream, w, q, s, K, KB);
  else
    hipLaunchKernelGGL(quant_weight_128x128_kernel<kModePow2>, dim3((unsigned)tiles), dim3(kWThreads), 0,
                       stream, w, q, s, K, KB);
  return hipGetLastError();
}

}  // namespace fp8q
