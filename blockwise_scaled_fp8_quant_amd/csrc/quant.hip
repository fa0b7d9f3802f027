// Activation (1x128) and weight (128x128) quantizers for gfx950, and the
// two-layout quantizer of the backward GEMMs.
//
// All are HBM streams: 2 bytes of bf16 read and 1 byte of E4M3 written per
// element, plus one fp32 scale per block.  Loads are 16 bytes per lane and
// cover whole 128-byte lines; the block |max| is reduced in registers and
// through DPP lane exchanges, never through memory.
#include "../../include/fp8q.h"
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
// 128-byte line.  One wave per workgroup, one block per lane group: many
// small workgroups ramp up and drain faster than fewer large ones (measured
// on 4096 x 4096 bf16: 10.1 us against 10.9 us for 256 lanes with two blocks
// per group, the same as a plain copy with this access pattern).
// ---------------------------------------------------------------------------
constexpr int kActThreads = 64;
constexpr int kActUnroll = 1;
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

// Tile (nb, kb) of w [N][K]; part holds kWThreads/16 floats of LDS.
template <int kMode>
__device__ __forceinline__ void quant_weight_tile(const uint16_t *__restrict__ w, uint8_t *__restrict__ q,
                                                  float *__restrict__ scales, int64_t K, int64_t nb, int64_t kb,
                                                  int64_t tile, float *part) {
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
    store_stream8(obase + (int64_t)(16 * i) * K, quant_chunk<kMode>(p, v[i]));  // read by later GEMMs
}

template <int kMode>
__global__ __launch_bounds__(kWThreads) void quant_weight_128x128_kernel(
    const uint16_t *__restrict__ w, uint8_t *__restrict__ q,
    float *__restrict__ scales, int64_t K, int64_t KB) {
  __shared__ float part[kWThreads / 16];
  const int64_t tile = blockIdx.x;
  const int64_t nb = tile / KB, kb = tile - nb * KB;
  quant_weight_tile<kMode>(w, q, scales, K, nb, kb, tile, part);
}

// ---------------------------------------------------------------------------
// A whole set of weight matrices in one launch (the recalibration after every
// policy update of page 1, "Leistungsgewinne in der Praxis", covers all linear
// weights of the model at once).  Workgroup t quantizes tile t of the
// concatenated tile sequence: its job is the last one whose tile_begin <= t,
// found with one coalesced load of 64 jobs' tile_begin per round and a
// ballot (no dependent search steps before the tile's own loads go out).  A
// separate launch per matrix pays the start-up and drain of a launch each
// time; here they are paid once.  The job table is caller data in device
// memory: a tile whose job is inconsistent (shape not a multiple of 128, tile
// outside the job's range) is skipped, so no access leaves a job's tensors.
// ---------------------------------------------------------------------------
template <int kMode>
__global__ __launch_bounds__(kWThreads) void quant_weight_batched_kernel(const fp8q_weight_job *__restrict__ jobs,
                                                                         int32_t count) {
  __shared__ float part[kWThreads / 16];
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x & 63;
  int32_t cnt = 0;
  for (int32_t base = 0; base < count; base += 64) {
    const int32_t j = base + lane;
    const int64_t b = j < count ? jobs[j].tile_begin : 0;
    cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(j < count && b <= t));
  }
  int32_t j = cnt - 1;
  j = j < 0 ? 0 : j;
  j = __builtin_amdgcn_readfirstlane(j);
  const uint16_t *w = jobs[j].w;
  uint8_t *q = jobs[j].q;
  float *scales = jobs[j].scales;
  const int64_t N = jobs[j].N, K = jobs[j].K, begin = jobs[j].tile_begin;
  if (N < 0 || K <= 0 || (N & 127) != 0 || (K & 127) != 0) return;
  const int64_t KB = K >> 7;
  const int64_t tile = t - begin;
  if (tile < 0 || tile >= (N >> 7) * KB) return;
  const int64_t nb = tile / KB, kb = tile - nb * KB;
  quant_weight_tile<kMode>(w, q, scales, K, nb, kb, tile, part);
}

hipError_t launch_quant_weight_batched(const fp8q_weight_job *jobs, int32_t count, int64_t total_tiles, int mode,
                                       hipStream_t stream) {
  if (count == 0 || total_tiles == 0) return hipSuccess;
  if (mode == kModeAmax)
    hipLaunchKernelGGL(quant_weight_batched_kernel<kModeAmax>, dim3((unsigned)total_tiles), dim3(kWThreads), 0,
                       stream, jobs, count);
  else
    hipLaunchKernelGGL(quant_weight_batched_kernel<kModePow2>, dim3((unsigned)total_tiles), dim3(kWThreads), 0,
                       stream, jobs, count);
  return hipGetLastError();
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

// Eight values of one block -> eight E4M3 bytes.  The block's parameters may
// differ between lanes.  Every pow2 block, and every amax block with a normal
// scale on the fast path, has |x / s| <= 448 * (1 + 2^-23), which the
// conversion rounds to at most 448 by itself; blocks with a subnormal scale or
// on the exact-division path (amax below 2^-100) take the clamped path.  The
// choice is one wave-uniform branch, so the common case has no per-element
// branches or clamps.
template <int kMode>
__device__ __forceinline__ uint2 quant8(const BlockQ &p, const float (&f)[8]) {
  float r[8];
  const bool plain = kMode == kModePow2 || (!p.slow && p.s >= 0x1p-126f);
  if (__ballot(!plain) == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = quotient<kMode>(p, f[i]);
    uint2 o;
    o.x = __builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], 0, false);
    o.x = __builtin_amdgcn_cvt_pk_fp8_f32(r[2], r[3], o.x, true);
    o.y = __builtin_amdgcn_cvt_pk_fp8_f32(r[4], r[5], 0, false);
    o.y = __builtin_amdgcn_cvt_pk_fp8_f32(r[6], r[7], o.y, true);
    return o;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float d = f[i] / p.s;
    const float e = quotient<kMode>(p, f[i]);
    r[i] = (kMode == kModeAmax && p.slow) ? d : e;
  }
  uint2 o;
  o.x = pack4_e4m3(r[0], r[1], r[2], r[3]);
  o.y = pack4_e4m3(r[4], r[5], r[6], r[7]);
  return o;
}

// Block parameters shared through LDS: (s, y) with y = RN(1/s) negated on the
// exact-division path (amax mode), or (s, e) (pow2 mode).
template <int kMode>
__device__ __forceinline__ float2 pack_params(const BlockQ &p) {
  return kMode == kModeAmax ? make_float2(p.s, p.slow ? -p.y : p.y) : make_float2(p.s, __int_as_float(p.e));
}

template <int kMode>
__device__ __forceinline__ BlockQ unpack_params(float2 v) {
  BlockQ p;
  p.s = v.x;
  if (kMode == kModeAmax) {
    p.y = __builtin_fabsf(v.y);
    p.slow = v.y < 0.0f;
    p.e = 0;
  } else {
    p.y = 0.0f;
    p.slow = false;
    p.e = __float_as_int(v.y);
  }
  return p;
}

// Marks the packed values as redefined, so the fp32 values unpacked from them
// in one phase are not kept alive (in 64 registers) for the next phase.
__device__ __forceinline__ void repack(uint4 (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(v[i].x), "+v"(v[i].y), "+v"(v[i].z), "+v"(v[i].w));
}

// Block maxima on magnitude bits: |x| of a bf16 orders like the integer
// (bits & 0x7FFF), so two magnitudes per word reduce with one packed 16-bit
// integer max; a maximum m converts back to fp32 exactly as m << 16.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pkmax(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t,
                            __builtin_elementwise_max(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
}
__device__ __forceinline__ float mag_lo(uint32_t m) { return __uint_as_float(m << 16); }
__device__ __forceinline__ float mag_hi(uint32_t m) { return __uint_as_float(m & 0xFFFF0000u); }

template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_pkmax(uint32_t v) {
  return pkmax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t group16_pkmax(uint32_t v) {
  v = dpp_pkmax<kDppQuadSwap1>(v);
  v = dpp_pkmax<kDppQuadSwap2>(v);
  v = dpp_pkmax<kDppHalfMirror>(v);
  return dpp_pkmax<kDppMirror>(v);
}

struct DualArgs {
  const uint16_t *x;
  int64_t M, K, Mp, KB, MB;
  uint8_t *q;
  float *s;
  uint8_t *qt;
  float *st;
};

// Workgroup barrier for LDS data: waits for this wave's LDS operations only
// (its global stores need not have completed).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int kMode, bool kTile, bool kRowOut>
__global__ __launch_bounds__(kDThreads) void quant_dual_kernel(DualArgs a) {
  __shared__ uint32_t red[4][64];               // per wave: column-pair maxima
  __shared__ __align__(16) float2 colp[128];  // parameters of the tile's 128 column blocks
  __shared__ __align__(16) float2 rowp[128];  // and of its 128 row blocks
  __shared__ __align__(16) uint8_t tq[128 * kTPitch];
  const int64_t KB = a.KB, MB = a.MB, M = a.M, K = a.K, Mp = a.Mp;
  const int64_t mb = blockIdx.x / KB, kb = blockIdx.x - mb * KB;
  const int t = threadIdx.x, c = t & 15, g = t >> 4, wave = t >> 6;
  const int64_t m0 = mb * 128, k0 = kb * 128;

  // Branch-free loads: a row past M reads row M-1 (M >= 1), then becomes zeros.
  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t m = m0 + 8 * g + i;
    v[i] = load_stream16(a.x + (m < M ? m : M - 1) * K + k0 + 8 * c);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (m0 + 8 * g + i >= M) v[i] = make_uint4(0u, 0u, 0u, 0u);

  // Magnitude maxima: cm[d] holds columns 8c+2d (low half) and 8c+2d+1 (high)
  // over the lane's 8 rows; rp[k] rows 8g+2k (low) and 8g+2k+1 (high) over
  // the lane's 8 columns.
  uint32_t cm[4] = {0u, 0u, 0u, 0u}, rp[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t rm[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 &w = v[2 * k + h];
      const uint32_t m_0 = w.x & 0x7FFF7FFFu, m_1 = w.y & 0x7FFF7FFFu;
      const uint32_t m_2 = w.z & 0x7FFF7FFFu, m_3 = w.w & 0x7FFF7FFFu;
      cm[0] = pkmax(cm[0], m_0);
      cm[1] = pkmax(cm[1], m_1);
      cm[2] = pkmax(cm[2], m_2);
      cm[3] = pkmax(cm[3], m_3);
      rm[h] = pkmax(pkmax(m_0, m_1), pkmax(m_2, m_3));
    }
    // low halves of both rows side by side, then the high halves
    rp[k] = pkmax((rm[0] & 0xFFFFu) | (rm[1] << 16), (rm[0] >> 16) | (rm[1] & 0xFFFF0000u));
  }

  BlockQ pt;  // kTile: the tile's parameters (every lane computes them)
  if constexpr (kTile) {
    uint32_t m2 = pkmax(pkmax(rp[0], rp[1]), pkmax(rp[2], rp[3]));
    m2 = group16_pkmax(m2);
    float m = __builtin_fmaxf(mag_lo(m2), mag_hi(m2));
    m = __builtin_fmaxf(m, __shfl_xor(m, 16));
    m = __builtin_fmaxf(m, __shfl_xor(m, 32));
    if ((t & 63) == 0) red[0][wave] = __float_as_uint(m);
    lds_barrier();
    m = __builtin_fmaxf(__builtin_fmaxf(__uint_as_float(red[0][0]), __uint_as_float(red[0][1])),
                        __builtin_fmaxf(__uint_as_float(red[0][2]), __uint_as_float(red[0][3])));
    pt = block_params<kMode>(m);
    if (t == 0) {
      a.st[kb * MB + mb] = pt.s;
      if (kRowOut) a.s[mb * KB + kb] = pt.s;
    }
  } else {
    // Column blocks: the four lanes of a wave that share a column, then the
    // four waves; lane t < 128 then computes column t's parameters once.
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      cm[d] = pkmax(cm[d], (uint32_t)__shfl_xor((int)cm[d], 16));
      cm[d] = pkmax(cm[d], (uint32_t)__shfl_xor((int)cm[d], 32));
    }
    if ((t & 63) < 16) {
#pragma unroll
      for (int d = 0; d < 4; ++d) red[wave][4 * c + d] = cm[d];
    }
    if constexpr (kRowOut) {
      // Row blocks: the 16 lanes of a row segment; lane c < 8 of the segment
      // then computes the parameters of row 8g + c.
#pragma unroll
      for (int k = 0; k < 4; ++k) rp[k] = group16_pkmax(rp[k]);
      const int ck = (c >> 1) & 3;
      const uint32_t w = ck == 0 ? rp[0] : (ck == 1 ? rp[1] : (ck == 2 ? rp[2] : rp[3]));
      if (c < 8) {
        const BlockQ pr = block_params<kMode>((c & 1) ? mag_hi(w) : mag_lo(w));
        rowp[8 * g + c] = pack_params<kMode>(pr);
        const int64_t m = m0 + 8 * g + c;
        if (m < M) a.s[m * KB + kb] = pr.s;
      }
    }
    lds_barrier();
    if (t < 128) {
      const uint32_t w = pkmax(pkmax(red[0][t >> 1], red[1][t >> 1]), pkmax(red[2][t >> 1], red[3][t >> 1]));
      const BlockQ pc = block_params<kMode>((t & 1) ? mag_hi(w) : mag_lo(w));
      colp[t] = pack_params<kMode>(pc);
      a.st[(k0 + t) * MB + mb] = pc.s;
    }
    lds_barrier();
  }

  // Transposed codes: column j of the lane's sub-block is 8 consecutive bytes
  // of row 8c+j of the transposed tile.
  repack(v);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const BlockQ pc = kTile ? pt : unpack_params<kMode>(colp[8 * c + j]);
    float f[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = elem(v[i], j);
    *reinterpret_cast<uint2 *>(tq + (8 * c + j) * kTPitch + 8 * g) = quant8<kMode>(pc, f);
  }

  if constexpr (kRowOut) {
    repack(v);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t m = m0 + 8 * g + i;
      const BlockQ pr = kTile ? pt : unpack_params<kMode>(rowp[8 * g + i]);
      float f[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = elem(v[i], j);
      const uint2 o = quant8<kMode>(pr, f);
      if (m < M) *reinterpret_cast<uint2 *>(a.q + m * K + k0 + 8 * c) = o;
    }
  }

  lds_barrier();
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int id = u * kDThreads + t;  // 16-byte chunk of the 128x128 transposed tile
    const int row = id >> 3, part = id & 7;
    const uint4 w = *reinterpret_cast<const uint4 *>(tq + row * kTPitch + part * 16);
    // weight codes stream out (read much later, by the backward GEMMs); the
    // transposed activation codes stay cacheable for the GEMM that follows
    if constexpr (kTile)
      store_stream16(a.qt + (k0 + row) * Mp + m0 + part * 16, w);
    else
      *reinterpret_cast<uint4 *>(a.qt + (k0 + row) * Mp + m0 + part * 16) = w;
  }
}

template <int kMode, bool kTile>
static void launch_dual(const uint16_t *x, int64_t M, int64_t K, int64_t Mp, uint8_t *q, float *s, uint8_t *qt,
                        float *st, hipStream_t stream) {
  const DualArgs a{x, M, K, Mp, K / 128, Mp / 128, q, s, qt, st};
  const int64_t tiles = a.MB * a.KB;
  if (q)
    hipLaunchKernelGGL((quant_dual_kernel<kMode, kTile, true>), dim3((unsigned)tiles), dim3(kDThreads), 0, stream,
                       a);
  else
    hipLaunchKernelGGL((quant_dual_kernel<kMode, kTile, false>), dim3((unsigned)tiles), dim3(kDThreads), 0,
                       stream, a);
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

// ---------------------------------------------------------------------------
// RMS normalization fused with the 1x128 quantization of its output: the
// norms ahead of the QKV and gate+up projections produce those layers' FP8
// activations in their own pass (page 1, "Leistungsgewinne in der Praxis":
// separate quantization kernels are overhead).
//   y = bf16_RNE((x * r) * gamma),  r = 1 / sqrt(sum(x^2) / K + eps)
// in fp32 (the sum of squares by paired bf16 dot products in a fixed order),
// then the activation rule on each 128 values of y.
//
// One wave per row.  Lane l holds chunk i = columns 512 i + 8 l .. +7, so the
// 16 lanes of each DPP row hold one 1x128 block (block 4 i + l / 16).  Every
// load is unconditional (addresses clamped into the tensors, values past the
// row masked) and all of them are issued before any math, so each wait counts
// only the loads it needs.  The 16 lanes of a block all hold its |max|; each
// derives the parameters (scale, reciprocal) of one of its kChunks blocks
// and passes them to the others through DPP row_share.  The block |max| is
// taken over the fp32 values before their bf16 rounding and rounded once:
// the rounding is monotonic, so this is the |max| of the rounded values.
// Between the |max| and the codes, y is held as packed bf16 pairs (half the
// registers of fp32 values: 93 VGPRs at K = 4096, 157 at K = 8192, which
// lets three waves share a SIMD there).
// With one row per wave the chip keeps 16 rows per CU in flight; giving a
// wave several rows, with the next row's loads overlapping the current row's
// math, measured slower, and so did two to eight waves per row.  The kernel
// is bound by its VALU work (about 12 instructions per element, ~5.5 us at
// 4096 x 4096) run after the row's data has arrived.
// ---------------------------------------------------------------------------
constexpr int kNormThreads = 256;
constexpr int kNormMaxK = 8192;

__device__ __forceinline__ uint32_t to_bf16x2(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 h2 __attribute__((ext_vector_type(2)));
  const f2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2));  // RNE
}

// a.lo * a.lo + a.hi * a.hi + c for a word of two bf16 values.
__device__ __forceinline__ float dot2_sq(uint32_t a, float c) {
  typedef __bf16 h2 __attribute__((ext_vector_type(2)));
  const h2 v = __builtin_bit_cast(h2, a);
  return __builtin_amdgcn_fdot2_f32_bf16(v, v, c, false);
}

// Lane i of each 16-lane DPP row -> every lane of that row.
template <int i>
__device__ __forceinline__ uint32_t row_share(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x150 + i, 0xF, 0xF, false);
}

// Parameters of the kChunks blocks a lane touches (block i: chunk i of its
// DPP row; every lane of the row holds the same amax[i]).  Lane j of the row
// derives those of block j % kChunks once, and row_share hands them out: one
// division pair per lane instead of one per chunk (measured 8% of the fused
// norm's time at K = 4096).
template <int kMode, int kChunks, int i = 0>
__device__ __forceinline__ void share_params(const BlockQ &mine, const float (&amax)[kChunks],
                                             BlockQ (&p)[kChunks]) {
  if constexpr (i < kChunks) {
    p[i].s = __uint_as_float(row_share<i>(__float_as_uint(mine.s)));
    if constexpr (kMode == kModeAmax) {
      p[i].y = __uint_as_float(row_share<i>(__float_as_uint(mine.y)));
      p[i].e = 0;
      p[i].slow = amax[i] < 0x1p-100f;  // as block_params decides it
    } else {
      p[i].y = 0.0f;
      p[i].e = (int)row_share<i>((uint32_t)mine.e);
      p[i].slow = false;
    }
    share_params<kMode, kChunks, i + 1>(mine, amax, p);
  }
}

// One row of the norm: w holds the lane's kChunks chunks of the row, gam the
// same chunks of gamma.
template <int kMode, int kChunks>
__device__ __forceinline__ void norm_row(const uint4 (&w)[kChunks], const uint4 (&gam)[kChunks], int K, float eps,
                                         int lane, uint8_t *__restrict__ qr, float *__restrict__ sr) {
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    float t = dot2_sq(w[i].x, ss);
    t = dot2_sq(w[i].y, t);
    t = dot2_sq(w[i].z, t);
    t = dot2_sq(w[i].w, t);
    ss = 512 * i + 8 * lane < K ? t : ss;  // a chunk past the row (clamped load) adds nothing
  }
  // butterfly: every lane ends with the same sum (each step adds a pair in
  // either order, and fp32 addition is commutative)
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  const float r = 1.0f / __builtin_sqrtf(ss * (1.0f / (float)K) + eps);

  uint32_t yb[kChunks][4];  // y rounded to bf16, two per word
  float amax[kChunks];
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const uint32_t xw[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
    const uint32_t gw[4] = {gam[i].x, gam[i].y, gam[i].z, gam[i].w};
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float lo = (bf16_lo(xw[k]) * r) * bf16_lo(gw[k]);
      const float hi = (bf16_hi(xw[k]) * r) * bf16_hi(gw[k]);
      m = max3_abs(m, lo, hi);
      yb[i][k] = to_bf16x2(lo, hi);
    }
    // y is held as packed bf16 until the block scales are known
    asm volatile("" : "+v"(yb[i][0]), "+v"(yb[i][1]), "+v"(yb[i][2]), "+v"(yb[i][3]));
    amax[i] = bf16_lo(to_bf16x2(group16_max(m), 0.0f));
  }
  BlockQ p[kChunks];
  if constexpr (kChunks == 1) {
    p[0] = block_params<kMode>(amax[0]);
  } else {
    const int j = lane & (kChunks - 1);
    float a = amax[0];
#pragma unroll
    for (int i = 1; i < kChunks; ++i) a = j == i ? amax[i] : a;
    share_params<kMode, kChunks>(block_params<kMode>(a), amax, p);
  }

#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int col = 512 * i + 8 * lane;
    float f[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f[2 * k] = bf16_lo(yb[i][k]);
      f[2 * k + 1] = bf16_hi(yb[i][k]);
    }
    const uint2 o = quant8<kMode>(p[i], f);
    if (col < K) {  // (uniform over each 16-lane block)
      if ((lane & 15) == 0) sr[col >> 7] = p[i].s;
      *reinterpret_cast<uint2 *>(qr + col) = o;
    }
  }
}

// The lane's chunks of one row of x (columns 512 i + 8 lane, clamped into the row).
template <int kChunks>
__device__ __forceinline__ void load_row(const uint16_t *__restrict__ xr, int K, int lane, uint4 (&w)[kChunks]) {
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int col = 512 * i + 8 * lane;
    w[i] = load_stream16(xr + (col < K ? col : K - 8));
  }
}

template <int kMode, int kChunks>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_quant_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ gamma, int64_t M, int K, float eps,
    uint8_t *__restrict__ q, float *__restrict__ scales) {
  static_assert(kChunks >= 1 && kChunks <= 16 && (kChunks & (kChunks - 1)) == 0, "chunks per lane");
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kNormThreads / 64) + (threadIdx.x >> 6);
  uint4 gam[kChunks], w[kChunks];
  load_row<kChunks>(x + (row < M ? row : M - 1) * K, K, lane, w);  // the row first: its data decides when the math can start
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int col = 512 * i + 8 * lane;
    gam[i] = *reinterpret_cast<const uint4 *>(gamma + (col < K ? col : K - 8));
  }
  __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the math
  if (row < M) norm_row<kMode, kChunks>(w, gam, K, eps, lane, q + row * K, scales + row * (K >> 7));
}

template <int kMode, int kChunks>
static void launch_norm(const uint16_t *x, const uint16_t *gamma, int64_t M, int64_t K, float eps, uint8_t *q,
                        float *s, hipStream_t stream) {
  constexpr int kWaves = kNormThreads / 64;
  hipLaunchKernelGGL((rmsnorm_quant_kernel<kMode, kChunks>), dim3((unsigned)((M + kWaves - 1) / kWaves)),
                     dim3(kNormThreads), 0, stream, x, gamma, M, (int)K, eps, q, s);
}

template <int kMode>
static void launch_norm_mode(const uint16_t *x, const uint16_t *gamma, int64_t M, int64_t K, float eps, uint8_t *q,
                             float *s, hipStream_t stream) {
  const int64_t chunks = (K + 511) / 512;
  if (chunks <= 1) launch_norm<kMode, 1>(x, gamma, M, K, eps, q, s, stream);
  else if (chunks <= 2) launch_norm<kMode, 2>(x, gamma, M, K, eps, q, s, stream);
  else if (chunks <= 4) launch_norm<kMode, 4>(x, gamma, M, K, eps, q, s, stream);
  else if (chunks <= 8) launch_norm<kMode, 8>(x, gamma, M, K, eps, q, s, stream);
  else launch_norm<kMode, 16>(x, gamma, M, K, eps, q, s, stream);
}

hipError_t launch_rmsnorm_quant_1x128(const uint16_t *x, const uint16_t *gamma, int64_t M, int64_t K, float eps,
                                      uint8_t *q, float *s, int mode, hipStream_t stream) {
  if (M == 0 || K == 0) return hipSuccess;
  if (K % 128 != 0 || K > kNormMaxK) return hipErrorInvalidValue;
  if (mode == kModeAmax) launch_norm_mode<kModeAmax>(x, gamma, M, K, eps, q, s, stream);
  else launch_norm_mode<kModePow2>(x, gamma, M, K, eps, q, s, stream);
  return hipGetLastError();
}

}  // namespace fp8q
