// Activation (1x128) and weight (128x128) quantizers for gfx950, and the
// two-layout quantizer of the backward GEMMs.
//
// All are HBM streams: 2 bytes of bf16 read and 1 byte of E4M3 written per
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

// ---------------------------------------------------------------------------
// Both layouts in one pass, for the backward GEMMs of training end to end in
// FP8 (page 1, "Der technische Durchbruch": FP8 in training as in generation).
// Each GEMM wants its scale blocks along its contraction dimension, so the
// weight gradient dW = dY^T X reads dY and X in blocks of 128 tokens x 1
// channel, transposed ([channels][Mp], Mp = M rounded up to 128), and the data
// gradient dX = dY W reads W's 128x128 tiles transposed ([K][N]).
//
// One workgroup of 256 lanes per 128x128 tile of a row-major [M][K] bf16
// matrix.  Lane t owns the 8x8 sub-block rows 8*(t/16) .. +7, columns
// 8*(t%16) .. +7: eight 16-byte loads, 16 lanes covering a 256-byte row
// segment.
//  - kTile (weights): one |max| and scale per tile, used for the row-major
//    codes q [M][K] (scales [M/128][K/128]) and the transposed codes q_t [K][M]
//    (scales [K/128][M/128]).
//  - activations: the 1x128 row blocks (q [M][K], scales [M][K/128]; optional)
//    and the 128x1 column blocks, transposed (q_t [K][Mp], scales [K][Mp/128]);
//    rows past M read as +0, so the padding of q_t holds +0 codes and does not
//    change a scale.
// Row maxima reduce over the 16 lanes of a row segment (DPP), column maxima
// over the four lanes of a wave that share a column (lane shuffles) and then
// over the four waves (LDS).  The transposed codes are staged in LDS so that
// each lane stores 16 contiguous bytes and a wave stores whole 128-byte lines.
// ---------------------------------------------------------------------------
constexpr int kDThreads = 256;
constexpr int kTPitch = 128 + 16;  // LDS row pitch (bytes) of the transposed tile

__device__ __forceinline__ float elem(const uint4 &v, int j) {
  const uint32_t w = j < 2 ? v.x : (j < 4 ? v.y : (j < 6 ? v.z : v.w));
  return (j & 1) ? bf16_hi(w) : bf16_lo(w);
}

template <int kMode>
__device__ __forceinline__ float quot(const BlockQ &p, float x) {
  return (kMode == kModeAmax && p.slow) ? x / p.s : quotient<kMode>(p, x);
}

template <int kMode, bool kTile, bool kRowOut>
__global__ __launch_bounds__(kDThreads) void quant_dual_kernel(
    const uint16_t *__restrict__ x, int64_t M, int64_t K, int64_t Mp, uint8_t *__restrict__ q,
    float *__restrict__ s, uint8_t *__restrict__ qt, float *__restrict__ st) {
  __shared__ float red[4][128];
  __shared__ __align__(16) uint8_t tq[128 * kTPitch];
  const int64_t KB = K >> 7, MB = Mp >> 7;
  const int64_t mb = blockIdx.x / KB, kb = blockIdx.x - mb * KB;
  const int t = threadIdx.x, c = t & 15, g = t >> 4, wave = t >> 6;
  const int64_t m0 = mb * 128, k0 = kb * 128;

  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t m = m0 + 8 * g + i;
    v[i] = m < M ? load_stream16(x + m * K + k0 + 8 * c) : make_uint4(0u, 0u, 0u, 0u);
  }

  float ra[8], ca[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) ra[i] = chunk_absmax(v[i], 0.0f);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i += 2) a = max3_abs(a, elem(v[i], j), elem(v[i + 1], j));
    ca[j] = a;
  }

  float tmax = 0.0f;  // kTile: the tile |max|
  if constexpr (kTile) {
#pragma unroll
    for (int i = 0; i < 8; ++i) tmax = __builtin_fmaxf(tmax, ra[i]);
    tmax = group16_max(tmax);
    tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 32));
    if ((t & 63) == 0) red[0][wave] = tmax;
    __syncthreads();
    tmax = __builtin_fmaxf(__builtin_fmaxf(red[0][0], red[0][1]), __builtin_fmaxf(red[0][2], red[0][3]));
  } else {
    if constexpr (kRowOut) {
#pragma unroll
      for (int i = 0; i < 8; ++i) ra[i] = group16_max(ra[i]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ca[j] = __builtin_fmaxf(ca[j], __shfl_xor(ca[j], 16));
      ca[j] = __builtin_fmaxf(ca[j], __shfl_xor(ca[j], 32));
    }
    if ((t & 63) < 16) {
#pragma unroll
      for (int j = 0; j < 8; ++j) red[wave][8 * c + j] = ca[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j)
      ca[j] = __builtin_fmaxf(__builtin_fmaxf(red[0][8 * c + j], red[1][8 * c + j]),
                              __builtin_fmaxf(red[2][8 * c + j], red[3][8 * c + j]));
  }

  // Transposed codes: column j of the lane's sub-block is 8 consecutive bytes
  // of row 8c+j of the transposed tile.
  const BlockQ pt = block_params<kMode>(tmax);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const BlockQ pc = kTile ? pt : block_params<kMode>(ca[j]);
    float r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = quot<kMode>(pc, elem(v[i], j));
    uint2 o;
    o.x = pack4_e4m3(r[0], r[1], r[2], r[3]);
    o.y = pack4_e4m3(r[4], r[5], r[6], r[7]);
    *reinterpret_cast<uint2 *>(tq + (8 * c + j) * kTPitch + 8 * g) = o;
    if (!kTile && g == 0) st[(k0 + 8 * c + j) * MB + mb] = pc.s;
  }
  if (kTile && t == 0) st[kb * MB + mb] = pt.s;

  if constexpr (kRowOut || kTile) {
    if constexpr (kRowOut) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t m = m0 + 8 * g + i;
        if (m < M) {
          const BlockQ pr = kTile ? pt : block_params<kMode>(ra[i]);
          *reinterpret_cast<uint2 *>(q + m * K + k0 + 8 * c) = quant_chunk<kMode>(pr, v[i]);
          if (!kTile && c == 0) s[m * KB + kb] = pr.s;
        }
      }
      if (kTile && t == 0) s[mb * KB + kb] = pt.s;
    }
  }

  __syncthreads();
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int id = u * kDThreads + t;  // 16-byte chunk of the 128x128 transposed tile
    const int row = id >> 3, part = id & 7;
    const uint4 w = *reinterpret_cast<const uint4 *>(tq + row * kTPitch + part * 16);
    *reinterpret_cast<uint4 *>(qt + (k0 + row) * Mp + m0 + part * 16) = w;
  }
}

template <int kMode, bool kTile>
static void launch_dual(const uint16_t *x, int64_t M, int64_t K, int64_t Mp, uint8_t *q, float *s, uint8_t *qt,
                        float *st, hipStream_t stream) {
  const int64_t tiles = (Mp / 128) * (K / 128);
  if (q)
    hipLaunchKernelGGL((quant_dual_kernel<kMode, kTile, true>), dim3((unsigned)tiles), dim3(kDThreads), 0, stream,
                       x, M, K, Mp, q, s, qt, st);
  else
    hipLaunchKernelGGL((quant_dual_kernel<kMode, kTile, false>), dim3((unsigned)tiles), dim3(kDThreads), 0,
                       stream, x, M, K, Mp, q, s, qt, st);
}

hipError_t launch_quant_dual(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s, uint8_t *qt,
                             float *st, int mode, bool tile, hipStream_t stream) {
  const int64_t Mp = (M + 127) / 128 * 128;
  if (Mp == 0 || K == 0) return hipSuccess;
  if (mode == kModeAmax) {
    if (tile) launch_dual<kModeAmax, true>(x, M, K, Mp, q, s, qt, st, stream);
    else launch_dual<kModeAmax, false>(x, M, K, Mp, q, s, qt, st, stream);
  } else {
    if (tile) launch_dual<kModePow2, true>(x, M, K, Mp, q, s, qt, st, stream);
    else launch_dual<kModePow2, false>(x, M, K, Mp, q, s, qt, st, stream);
  }
  return hipGetLastError();
}

}  // namespace fp8q
