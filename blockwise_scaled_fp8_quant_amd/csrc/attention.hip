// FP8 KV cache and FP8 decode attention for gfx950.
//
// Page "NVIDIA NeMo RL erreicht 48% Geschwindigkeitssteigerung ...", section
// "Leistungsgewinne in der Praxis": FP8 for the KV cache and for attention is
// what lifts the recipe from 15-25% on the linear layers to about 48% end to
// end.  The recipe's activation rule is applied to the cache: every key and
// value row of one token and one key/value head (D = 128) is a 1x128 block
// with its own fp32 scale, and so is every query row.
//
// Cache layout: [B][Hkv][S][128] E4M3 bytes, scales [B][Hkv][S] -- the tokens
// of one sequence and head are contiguous 128-byte rows, the unit every load
// below reads whole.
#include <mutex>

#include "../../include/fp8q.h"
#include "fp8q_device.h"
#include "fp8q_internal.h"

namespace fp8q {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));

constexpr int kHeadDim = 128;

// ---------------------------------------------------------------------------
// Cache append: T new key rows and T new value rows per sequence and head,
// token-major ([B][T][Hkv][128], as a projection writes them), quantized with
// the activation rule; token t of sequence b goes to position start[b] + t.
// Eight lanes per row (as in the activation quantizer); row r of the
// 2*B*T*Hkv rows is a key row for r < B*T*Hkv, else a value row.
// ---------------------------------------------------------------------------
template <int kMode>
__global__ __launch_bounds__(256) void kv_append_kernel(const uint16_t *__restrict__ k_new,
                                                        const uint16_t *__restrict__ v_new,
                                                        const int32_t *__restrict__ start, uint8_t *__restrict__ kc,
                                                        float *__restrict__ ks, uint8_t *__restrict__ vc,
                                                        float *__restrict__ vs, int32_t B, int32_t T, int32_t H,
                                                        int64_t S) {
  const int64_t row = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  const int sub = threadIdx.x & 7;
  const int64_t rows = (int64_t)B * T * H;
  if (row >= 2 * rows) return;  // uniform over the 8 lanes of a row
  const bool is_v = row >= rows;
  const int64_t r = is_v ? row - rows : row;  // = (b * T + t) * H + h
  const int64_t h = r % H, bt = r / H;
  const int64_t b = bt / T, t = bt - b * T;
  const uint4 *src = reinterpret_cast<const uint4 *>((is_v ? v_new : k_new) + r * kHeadDim);
  const uint4 x0 = src[sub], x1 = src[sub + 8];
  float amax = group8_max(chunk_absmax(x1, chunk_absmax(x0, 0.0f)));
  const BlockQ p = block_params<kMode>(amax);
  const int64_t pos = (int64_t)start[b] + t;
  if (pos < 0 || pos >= S) return;
  const int64_t slot = (b * H + h) * S + pos;  // (b, h, pos)
  uint2 *dst = reinterpret_cast<uint2 *>((is_v ? vc : kc) + slot * kHeadDim);
  dst[sub] = quant_chunk<kMode>(p, x0);
  dst[sub + 8] = quant_chunk<kMode>(p, x1);
  if (sub == 0) (is_v ? vs : ks)[slot] = p.s;
}

hipError_t launch_kv_cache_append(const uint16_t *k_new, const uint16_t *v_new, const int32_t *start, uint8_t *kc,
                                  float *ks, uint8_t *vc, float *vs, int32_t B, int32_t T, int32_t H, int64_t S,
                                  int mode, hipStream_t stream) {
  const int64_t rows = 2 * (int64_t)B * T * H;
  if (rows == 0) return hipSuccess;
  const int64_t grid = (rows + 31) / 32;
  if (mode == kModeAmax)
    hipLaunchKernelGGL(kv_append_kernel<kModeAmax>, dim3((unsigned)grid), dim3(256), 0, stream, k_new, v_new, start,
                       kc, ks, vc, vs, B, T, H, S);
  else
    hipLaunchKernelGGL(kv_append_kernel<kModePow2>, dim3((unsigned)grid), dim3(256), 0, stream, k_new, v_new, start,
                       kc, ks, vc, vs, B, T, H, S);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Decode attention: one query token per sequence,
//   o[b][h] = sum_t softmax_t(q[b][h] . k[b][g][t] / sqrt(128)) v[b][g][t],
// g = h / GRP (GRP query heads share a key/value head), t < min(len[b], S).
//
// One workgroup per (sequence, key/value head, chunk of the sequence); its
// four waves take the 64-token tiles of the chunk in turn and keep their own
// running maximum, sum and output, merged through LDS at the end.  When the
// (sequence, head) pairs alone cannot fill the chip (fewer than kFillWgs) and
// a workspace is given, sequences are cut into chunks: each workgroup writes
// its chunk's maximum, sum and unnormalized output, and a second kernel
// merges the chunks of each sequence.  Otherwise one chunk is the whole
// sequence (measured: splitting a batch that already fills the chip only
// adds per-workgroup cost).
//  - Scores: one v_mfma_scale_f32_16x16x128_f8f6f4 per 16 tokens, E4M3 x
//    E4M3, with the GRP query rows as the A operand (rows of D, padded to 16
//    with zeros) and 16 key rows, read straight from the cache, as B.  Lane l
//    then holds the scores of token l%16 for heads 4*(l/16) .. +3.  The query
//    and key scales and log2(e)/sqrt(128) are applied to the fp32 result.
//  - Softmax in base 2 (v_exp_f32), online over the tiles; per-head maxima
//    and sums reduce over the 16 lanes of a row group with DPP and are then
//    read out as wave-uniform values.
//  - Values: lane l accumulates dims 8*(l%16) .. +7 for every head over the
//    tokens 16*(l/16) .. +15 of each tile (8-byte loads, a whole 128-byte row
//    per 16 lanes), weights p * v_scale passed through LDS; fp32 FMAs on the
//    exactly decoded E4M3 values.
// ---------------------------------------------------------------------------
constexpr int kAttnWaves = 4;
constexpr int kTileTok = 64;
constexpr int64_t kFillWgs = 512;  // workgroups that fill MI355X (256 CUs, two resident each)
constexpr int kMinChunkTiles = 4;  // at least one tile per wave

struct AttnArgs {
  const uint8_t *qq;
  const float *qs;
  const uint8_t *kc;
  const float *ks;
  const uint8_t *vc;
  const float *vs;
  const int32_t *len;
  uint16_t *out;
  float *ws_o;    // chunked: [B][Hq][nch][128] unnormalized outputs of each chunk
  float *ws_ml;   // chunked: [B][Hq][nch][2] maximum (base 2) and sum of each chunk
  int32_t Hq, Hkv;
  int64_t S;
  int32_t nch;    // chunks per sequence (1: the whole sequence)
  int32_t chunk_tiles;  // 64-token tiles per chunk (chunked)
  int32_t B;            // sequences
  int32_t balance_cus;  // > 0: length-balanced order over this many CUs (unchunked, B <= kBalanceMaxB)
};

template <int kCtrl>
__device__ __forceinline__ float dpp_fmax(float v) {
  return __builtin_fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false)));
}
template <int kCtrl>
__device__ __forceinline__ float dpp_fadd(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
// Max / sum over each row of 16 lanes (every lane gets the result).
__device__ __forceinline__ float row16_max(float v) {
  v = dpp_fmax<kDppQuadSwap1>(v);
  v = dpp_fmax<kDppQuadSwap2>(v);
  v = dpp_fmax<kDppHalfMirror>(v);
  return dpp_fmax<kDppMirror>(v);
}
__device__ __forceinline__ float row16_sum(float v) {
  v = dpp_fadd<kDppQuadSwap1>(v);
  v = dpp_fadd<kDppQuadSwap2>(v);
  v = dpp_fadd<kDppHalfMirror>(v);
  return dpp_fadd<kDppMirror>(v);
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Eight E4M3 bytes -> eight exact fp32 values.
__device__ __forceinline__ void dec8(uint2 w, float (&f)[8]) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  f2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false);
  f2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);
  f2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false);
  f2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);
  f[0] = a.x; f[1] = a.y; f[2] = b.x; f[3] = b.y;
  f[4] = c.x; f[5] = c.y; f[6] = d.x; f[7] = d.y;
}

// Length-balanced order of the unchunked launch.  With every (sequence, head)
// workgroup resident at once, a CU's time is the sum of its workgroups'
// lengths, and the launch lasts as long as the busiest CU: with lengths drawn
// in [2048, 6144] the natural order ran at 4.3 TB/s, equal lengths at 5.5.
// Each workgroup ranks the batch's lengths (longest first, ties by index) in
// LDS and takes the pair at its position in snake order over the CUs: round
// r of `cus` workgroups runs forward when r is even and backward when r is
// odd, so the CU that gets a long pair in one round gets a short one in the
// next.  The ranking is B comparisons per thread; batches above kBalanceMaxB
// keep the natural order.
constexpr int kBalanceMaxB = 256;

template <int GRP>
struct AttnLds {
  float w[kAttnWaves][kTileTok][GRP];          // p * v_scale of a tile, per token and head
  float m[kAttnWaves][GRP], l[kAttnWaves][GRP];
  float acc[kAttnWaves][GRP][kHeadDim];
};

template <int GRP, bool kChunked>
__global__ __launch_bounds__(64 * kAttnWaves) void attn_decode_kernel(AttnArgs a) {
  static_assert(GRP == 1 || GRP == 2 || GRP == 4 || GRP == 8, "query heads per key/value head");
  constexpr int kRowsPerLane = 4;  // MFMA output rows (heads) per lane
  __shared__ AttnLds<GRP> L;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t bg = blockIdx.x / a.nch;  // b * Hkv + g
  if (!kChunked && a.balance_cus > 0) {
    __shared__ int32_t lens[kBalanceMaxB], order[kBalanceMaxB];
    for (int i = threadIdx.x; i < a.B; i += 64 * kAttnWaves) {
      const int32_t v = a.len[i];
      lens[i] = v < 0 ? 0 : (v > a.S ? (int32_t)a.S : v);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < a.B; i += 64 * kAttnWaves) {
      const int32_t v = lens[i];
      int r = 0;
      for (int j = 0; j < a.B; ++j) r += (lens[j] > v || (lens[j] == v && j < i)) ? 1 : 0;
      order[r] = i;
    }
    __syncthreads();
    const int64_t P = (int64_t)a.B * a.Hkv, C = a.balance_cus;
    const int64_t w = blockIdx.x, rnd = w / C, pos = w - rnd * C;
    const int64_t width = (P - rnd * C) < C ? (P - rnd * C) : C;  // workgroups in this round
    const int64_t rank = rnd * C + ((rnd & 1) ? width - 1 - pos : pos);
    bg = (int64_t)order[rank / a.Hkv] * a.Hkv + rank % a.Hkv;
  }
  const int chunk = (int)(blockIdx.x - bg * a.nch);
  const int64_t b = bg / a.Hkv, g = bg - b * a.Hkv;
  int64_t len = a.len[b];
  len = len < 0 ? 0 : (len > a.S ? a.S : len);
  const int ntiles = (int)((len + kTileTok - 1) / kTileTok);
  const int tile_begin = kChunked ? chunk * a.chunk_tiles : 0;
  const int tile_end = kChunked ? (ntiles < tile_begin + a.chunk_tiles ? ntiles : tile_begin + a.chunk_tiles) : ntiles;
  if (kChunked && tile_begin >= ntiles) return;  // past the sequence: the merge skips this chunk

  const int64_t h0 = g * GRP;  // first query head of the group

  // Query rows as the A operand: lane l gives row l%16 (head h0 + l%16, zero
  // past GRP), bytes 32*(l/16) .. +31.
  v8i_t qf = {0, 0, 0, 0, 0, 0, 0, 0};
  if ((lane & 15) < GRP) {
    const uint4 *qp = reinterpret_cast<const uint4 *>(a.qq + ((b * a.Hq + h0 + (lane & 15)) * kHeadDim) + 32 * (lane >> 4));
    const uint4 x = qp[0], y = qp[1];
    qf[0] = x.x; qf[1] = x.y; qf[2] = x.z; qf[3] = x.w;
    qf[4] = y.x; qf[5] = y.y; qf[6] = y.z; qf[7] = y.w;
  }
  // Score multiplier of this lane's four output rows (heads 4*(l/16)+r):
  // query scale * log2(e) / sqrt(128); zero for padding rows.
  constexpr float kL2eRsqrtD = 1.4426950408889634f * 0.08838834764831845f;
  float qmul[kRowsPerLane];
#pragma unroll
  for (int r = 0; r < kRowsPerLane; ++r) {
    const int h = 4 * (lane >> 4) + r;
    qmul[r] = h < GRP ? a.qs[b * a.Hq + h0 + h] * kL2eRsqrtD : 0.0f;
  }

  const int64_t base = bg * a.S;  // (b, g, token 0) in the cache
  const uint8_t *kc = a.kc + base * kHeadDim;
  const uint8_t *vc = a.vc + base * kHeadDim;
  const float *ksc = a.ks + base;
  const float *vsc = a.vs + base;

  float m_run[GRP], l_run[GRP];  // wave-uniform running max (base 2) and sum per head
  float acc[GRP][8];             // dims 8*(l%16) .. +7, tokens 16*(l/16) .. of each tile
#pragma unroll
  for (int h = 0; h < GRP; ++h) {
    m_run[h] = -__builtin_inff();
    l_run[h] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[h][i] = 0.0f;
  }

  const int tg = lane >> 4;  // token group of the value pass
  const int dq = lane & 15;  // 8-dim slice of the value pass
  // A tile's key rows (this lane's part of the four 16-token MFMA operands)
  // and its 64 key and value scales (one per lane: one load instruction each;
  // a vector-memory instruction costs the same whatever its width).  They are
  // loaded one tile ahead: the next tile's go out as soon as this tile's score
  // MFMAs have read theirs, and land during the softmax and the value pass.
  // Rows past len read row len-1 (masked in the scores).
  uint4 kx[4], ky[4];
  float ks_l = 0.0f, vs_l = 0.0f;
  auto load_keys = [&](int tile) {
    const int64_t t0 = (int64_t)tile * kTileTok;
    int64_t ts = t0 + lane;
    ts = ts < len ? ts : len - 1;
    ks_l = ksc[ts];
    vs_l = vsc[ts];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int64_t t = t0 + 16 * j + (lane & 15);
      t = t < len ? t : len - 1;
      const uint4 *kp = reinterpret_cast<const uint4 *>(kc + t * kHeadDim + 32 * (lane >> 4));
      kx[j] = kp[0];
      ky[j] = kp[1];
    }
  };
  if (tile_begin + wave < tile_end) load_keys(tile_begin + wave);
  for (int tile = tile_begin + wave; tile < tile_end; tile += kAttnWaves) {
    const int64_t t0 = (int64_t)tile * kTileTok;
    // value rows of this lane (not needed until after the softmax)
    uint2 vb[16];
    float vsl[4];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      int64_t t = t0 + 16 * tg + i;
      t = t < len ? t : len - 1;
      vb[i] = *reinterpret_cast<const uint2 *>(vc + t * kHeadDim + 8 * dq);
    }
    // scores: four MFMAs of 16 tokens; B operand = key rows t0 + 16j + l%16
    float sc[4][kRowsPerLane];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool valid = t0 + 16 * j + (lane & 15) < len;
      const uint4 x = kx[j], y = ky[j];
      const v8i_t kf = {(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
      const float kscale = __shfl(ks_l, 16 * j + (lane & 15));
      vsl[j] = __shfl(vs_l, 16 * j + (lane & 15));
      const v4f_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
      const v4f_t d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qf, kf, zero, 0, 0, 0, 127, 0, 127);
#pragma unroll
      for (int r = 0; r < kRowsPerLane; ++r) sc[j][r] = valid ? d[r] * (qmul[r] * kscale) : -__builtin_inff();
    }
    // the next tile's keys and scales (their registers are free once the
    // MFMAs above have read them); the asm statements keep the loads here.
    // After the wave's last tile they reload this tile's rows (cache hits):
    // under a branch, the wait counts after it would have to assume the loads
    // absent and wait for them in the value pass.
    asm volatile("" ::: "memory");
    load_keys(tile + kAttnWaves < tile_end ? tile + kAttnWaves : tile);
    asm volatile("" ::: "memory");
    // online softmax per head
    float alpha[GRP];
#pragma unroll
    for (int r = 0; r < kRowsPerLane; ++r) {
      float mt = __builtin_fmaxf(__builtin_fmaxf(sc[0][r], sc[1][r]), __builtin_fmaxf(sc[2][r], sc[3][r]));
      mt = row16_max(mt);
      // row group q of the lanes holds heads 4q + r
#pragma unroll
      for (int q = 0; q < (GRP + 3) / 4; ++q) {
        const int h = 4 * q + r;
        if (h < GRP) {
          const float mnew = __builtin_fmaxf(m_run[h], readlane_f(mt, 16 * q));
          alpha[h] = __builtin_amdgcn_exp2f(m_run[h] - mnew);
          m_run[h] = mnew;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kRowsPerLane; ++r) {
      const int hl = 4 * tg + r;  // head of this lane's score row r
      float mh = -__builtin_inff();
#pragma unroll
      for (int q = 0; q < (GRP + 3) / 4; ++q)
        if (4 * q + r < GRP && tg == q) mh = m_run[4 * q + r];
      float ps = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = hl < GRP ? __builtin_amdgcn_exp2f(sc[j][r] - mh) : 0.0f;
        ps += p;
        if (hl < GRP) L.w[wave][16 * j + (lane & 15)][hl] = p * vsl[j];
      }
      ps = row16_sum(ps);
#pragma unroll
      for (int q = 0; q < (GRP + 3) / 4; ++q) {
        const int h = 4 * q + r;
        if (h < GRP) l_run[h] = l_run[h] * alpha[h] + readlane_f(ps, 16 * q);
      }
    }
    // weighted values: rescale, then this lane's 16 tokens x 8 dims
#pragma unroll
    for (int h = 0; h < GRP; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[h][i] *= alpha[h];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's weights are in LDS
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float f[8];
      dec8(vb[i], f);
      const float *wr = L.w[wave][16 * tg + i];
#pragma unroll
      for (int h = 0; h < GRP; ++h) {
        const float w = wr[h];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = __builtin_fmaf(w, f[e], acc[h][e]);
      }
    }
    asm volatile("" ::: "memory");  // the next tile's weights overwrite these only afterwards
  }

  // Merge the four token groups of the wave (same dims, lanes l, l^16, l^32, l^48).
#pragma unroll
  for (int h = 0; h < GRP; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v = acc[h][i];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      acc[h][i] = v;
    }
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < GRP; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i) L.acc[wave][h][8 * lane + i] = acc[h][i];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < GRP; ++h) {
      L.m[wave][h] = m_run[h];
      L.l[wave][h] = l_run[h];
    }
  }
  __syncthreads();
  // Merge the waves: o = sum_w acc_w 2^(m_w - M) / sum_w l_w 2^(m_w - M).
  for (int idx = threadIdx.x; idx < GRP * kHeadDim; idx += 64 * kAttnWaves) {
    const int h = idx / kHeadDim, d = idx - h * kHeadDim;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = __builtin_fmaxf(M, L.m[w][h]);
    float num = 0.0f, den = 0.0f;
    if (M != -__builtin_inff()) {
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
        const float c = __builtin_amdgcn_exp2f(L.m[w][h] - M);
        num += c * L.acc[w][h][d];
        den += c * L.l[w][h];
      }
    }
    if constexpr (kChunked) {
      const int64_t row = (b * a.Hq + h0 + h) * a.nch + chunk;
      a.ws_o[row * kHeadDim + d] = num;
      if (d == 0) {
        a.ws_ml[2 * row] = M;
        a.ws_ml[2 * row + 1] = den;
      }
    } else {
      const float o = den > 0.0f ? num / den : 0.0f;
      a.out[(b * a.Hq + h0 + h) * kHeadDim + d] = __builtin_bit_cast(uint16_t, (__bf16)o);  // RNE
    }
  }
}

// Merge of the chunks of each (sequence, query head): one 128-lane workgroup,
// lane d of the head dimension.  Chunks at or past the sequence's length were
// not written and are skipped.
__global__ __launch_bounds__(kHeadDim) void attn_merge_kernel(AttnArgs a) {
  const int64_t bh = blockIdx.x;  // b * Hq + h
  const int64_t b = bh / a.Hq;
  const int d = threadIdx.x;
  int64_t len = a.len[b];
  len = len < 0 ? 0 : (len > a.S ? a.S : len);
  const int64_t chunk_tok = (int64_t)a.chunk_tiles * kTileTok;
  const int nvalid = (int)((len + chunk_tok - 1) / chunk_tok);
  const float *ml = a.ws_ml + bh * a.nch * 2;
  const float *o = a.ws_o + bh * a.nch * kHeadDim;
  float M = -__builtin_inff();
  for (int c = 0; c < nvalid; ++c) M = __builtin_fmaxf(M, ml[2 * c]);
  float num = 0.0f, den = 0.0f;
  if (M != -__builtin_inff()) {
    for (int c = 0; c < nvalid; ++c) {
      const float w = __builtin_amdgcn_exp2f(ml[2 * c] - M);
      num += w * o[c * kHeadDim + d];
      den += w * ml[2 * c + 1];
    }
  }
  const float r = den > 0.0f ? num / den : 0.0f;
  a.out[bh * kHeadDim + d] = __builtin_bit_cast(uint16_t, (__bf16)r);  // RNE
}

// Chunks per sequence and tiles per chunk for B*Hkv (sequence, head) pairs and
// a cache of S tokens: enough chunks to give about kFillWgs workgroups, each
// chunk at least kMinChunkTiles tiles.  A function of the sizes only, so the
// workspace a call needs is known on the host.
void attention_decode_split(int64_t pairs, int64_t S, int64_t &nch, int64_t &chunk_tiles) {
  const int64_t tiles = (S + kTileTok - 1) / kTileTok;
  nch = 1;
  chunk_tiles = tiles;
  if (pairs <= 0 || pairs >= kFillWgs || tiles <= kMinChunkTiles) return;
  int64_t want = (kFillWgs + pairs - 1) / pairs;
  int64_t ct = (tiles + want - 1) / want;
  ct = ct < kMinChunkTiles ? kMinChunkTiles : ct;
  nch = (tiles + ct - 1) / ct;
  chunk_tiles = ct;
}

// Compute units of the current device (queried once per device).
static int32_t device_cus() {
  static std::once_flag once[kMaxDevices];
  static int32_t cus[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  std::call_once(once[dev], [dev]() {
    int n = 0;
    cus[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess ? n : 0;
  });
  return cus[dev];
}

template <bool kChunked>
static hipError_t launch_decode(const AttnArgs &a, int64_t B, hipStream_t stream) {
  const dim3 grid((unsigned)(B * a.Hkv * a.nch)), block(64 * kAttnWaves);
  switch (a.Hq / a.Hkv) {
    case 1: hipLaunchKernelGGL((attn_decode_kernel<1, kChunked>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((attn_decode_kernel<2, kChunked>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((attn_decode_kernel<4, kChunked>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((attn_decode_kernel<8, kChunked>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attention_decode(const uint8_t *qq, const float *qs, const uint8_t *kc, const float *ks,
                                   const uint8_t *vc, const float *vs, const int32_t *len, uint16_t *out,
                                   int32_t B, int32_t Hq, int32_t Hkv, int64_t S, float *workspace,
                                   hipStream_t stream) {
  if (B == 0) return hipSuccess;
  int64_t nch, ct;
  attention_decode_split((int64_t)B * Hkv, S, nch, ct);
  if (workspace == nullptr || nch <= 1) {
    AttnArgs a{qq, qs, kc, ks, vc, vs, len, out, nullptr, nullptr, Hq, Hkv, S, 1, 0, B, 0};
    if (B > 1 && B <= kBalanceMaxB) a.balance_cus = device_cus();
    return launch_decode<false>(a, B, stream);
  }
  float *ws_o = workspace;
  float *ws_ml = workspace + (int64_t)B * Hq * nch * kHeadDim;
  const AttnArgs a{qq, qs, kc, ks, vc, vs, len, out, ws_o, ws_ml, Hq, Hkv, S, (int32_t)nch, (int32_t)ct, B, 0};
  hipError_t e = launch_decode<true>(a, B, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)((int64_t)B * Hq)), dim3(kHeadDim), 0, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Decode attention without a caller workspace, for callers that cannot
// allocate: the chunked path's partial outputs and (max, sum) pairs live in
// this file-scope device array instead.  Its size covers every valid call:
// with fewer than kFillWgs (sequence, head) pairs, chunks per sequence <=
// ceil(kFillWgs / pairs), so pairs * chunks <= kFillWgs + pairs - 1 <= 1022,
// times at most 8 query heads per key/value head, each row 128 + 2 floats.
// Each GPU the library runs on holds its own copy until the process ends;
// calls on one GPU share it, so calls that overlap on one GPU race.
// ---------------------------------------------------------------------------
constexpr int64_t kNoAllocRows = 8 * (2 * kFillWgs - 2);
constexpr int64_t kNoAllocFloats = kNoAllocRows * (kHeadDim + 2);
static __device__ __align__(256) float scratch[kNoAllocFloats];
static_assert(kNoAllocFloats * sizeof(float) == FP8Q_NOALLOC_SCRATCH_BYTES, "scratch size in the header");

int64_t attention_noalloc_scratch_bytes() { return kNoAllocFloats * (int64_t)sizeof(float); }

// The device address of `scratch` on the current device.  In host code the
// array's name is only a host-side stand-in; the address comes from the
// runtime, once per device (with that device current), and is kept.
static hipError_t scratch_address(float **out) {
  static std::once_flag once[kMaxDevices];
  static float *addr[kMaxDevices];
  static hipError_t err[kMaxDevices];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(once[dev], [dev]() {
    void *p = nullptr;
    err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    addr[dev] = static_cast<float *>(p);
  });
  if (err[dev] != hipSuccess) return err[dev];
  if (addr[dev] == nullptr) return hipErrorInvalidSymbol;
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_attention_decode_noalloc(const uint8_t *qq, const float *qs, const uint8_t *kc,
                                           const float *ks, const uint8_t *vc, const float *vs,
                                           const int32_t *len, uint16_t *out, int32_t B, int32_t Hq,
                                           int32_t Hkv, int64_t S, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  int64_t nch, ct;
  attention_decode_split((int64_t)B * Hkv, S, nch, ct);
  float *ws = nullptr;
  if (nch > 1) {
    if ((int64_t)B * Hq * nch * (kHeadDim + 2) > kNoAllocFloats) return hipErrorInvalidValue;
    hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return e;
  }
  return launch_attention_decode(qq, qs, kc, ks, vc, vs, len, out, B, Hq, Hkv, S, ws, stream);
}


// ---------------------------------------------------------------------------
// Attention for many query tokens (prefill, chunked prefill, a training
// forward pass) over the FP8 cache, causal: query t of sequence b sits at
// position start[b] + t and attends to the cached tokens 0 .. start[b] + t
// below S (the queries' own keys and values are appended to the cache
// first).  Queries are token-major, q [B][T][Hq][128] E4M3 with one scale per
// row, as the QKV projection's quantized output holds them.
//
// One workgroup per (sequence, query head, 128 query tokens); its eight waves
// own 16 query tokens each.  Workgroups are ordered longest first (the last
// query tiles of every head start first).  Per 64-key tile:
//  - the workgroup stages the tile in LDS: the E4M3 key rows as they are, the
//    value rows decoded exactly to bf16 (every E4M3 value is a bf16 value),
//    row-major, and the 64 key and value scales; the global loads of the next
//    tile go out before the math of this one;
//  - scores S^T = K Q^T on the matrix cores in FP8: one
//    v_mfma_scale_f32_16x16x128_f8f6f4 per 16 keys (the whole head dimension
//    in one instruction), key rows as A and the wave's query rows as B, so
//    lane l holds keys 4(l/16)..+3 of query l%16 and every per-query quantity
//    (running maximum, sum, output column) lives in one lane column;
//  - online softmax in base 2; a query's maximum is raised only when a tile
//    exceeds it by more than 8 (a factor 2^8 in the weights), so the output
//    rescale is rare; masks only
//    on tiles that reach past some query's position; the weights p * v_scale
//    are rounded to bf16 (relative error at most 2^-8 each) and go straight
//    from the score registers into the B operand of the value product;
//  - O^T += V^T P^T with v_mfma_f32_16x16x32_bf16, eight per 32 keys (16 dims
//    each), fp32 accumulation: lane l holds dims 4(l/16)..+3 of each 16-dim
//    block for query l%16.  The MFMA's k slots of lane group q are keys
//    4q..4q+3 and 16+4q..16+4q+3 of the 32 (the keys whose scores that lane
//    group holds).  The V^T operand comes from the row-major value tile by
//    LDS transpose loads (ds_read_b64_tr_b16, two per MFMA), so the staging
//    writes whole rows instead of scattering a transpose.
// Key rows in LDS are XOR-swizzled in 16-byte chunks by row so that the 16
// lanes reading one chunk of 16 different rows hit different banks; value
// rows are padded by 32 bytes so that the eight rows a half-wave's transpose
// load touches start in different banks.
// ---------------------------------------------------------------------------
constexpr int kPfWaves = 8;
constexpr int kPfQ = 16 * kPfWaves;  // query tokens per workgroup
constexpr int kPfKeys = 64;          // keys per staged tile
constexpr int kPfThreads = 64 * kPfWaves;
static_assert(kPfThreads >= 128 && 512 % kPfThreads == 0, "staging roles");
// A query's running maximum moves only when a tile's maximum exceeds it by
// more than this (base 2): weights stay below 2^8 and the rescale of the
// output, a wave-uniform branch, is rare once the maximum has settled.
constexpr float kPfLazy = 8.0f;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

struct PrefillArgs {
  const uint8_t *qq;
  const float *qs;
  const uint8_t *kc;
  const float *ks;
  const uint8_t *vc;
  const float *vs;
  const int32_t *start;
  uint16_t *out;
  int32_t B, T, Hq, Hkv;
  int32_t S;       // below 2^31 (checked by the entry point)
  int32_t qtiles;  // ceil(T / kPfQ)
};

constexpr int kPfVRow = kHeadDim + 16;  // bf16 per value row in LDS (32 bytes of padding)

struct PrefillLds {
  uint8_t k[kPfKeys * kHeadDim];        // key rows, chunk c of row r at c ^ (r & 7)
  uint16_t v[kPfKeys * kPfVRow];        // value rows, bf16, row-major
  float ks[kPfKeys], vs[kPfKeys];       // ks times log2(e) / sqrt(128)
};

typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;

// Transpose load of 16-bit elements (ds_read_b64_tr_b16).  Within each group
// of 16 lanes, lane 4j + (i / 4) names an 8-byte window of four elements and
// lane i receives, as its element j, element i % 4 of that window (checked on
// gfx950 with distinct values).  So if lane r of a group names row key(r / 4),
// columns c0 + 4 (r % 4) .. +3 of a row-major tile, lane i receives column
// c0 + i of rows key(0) .. key(3).
__device__ __forceinline__ v4s_t lds_read_tr16(const uint16_t *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t *)(__attribute__((address_space(3))) void *)p);
}

__device__ __forceinline__ uint32_t bf16x2_of(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 h2 __attribute__((ext_vector_type(2)));
  const f2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2));  // RNE
}

__device__ __forceinline__ int clamp_pos(int64_t p, int32_t S) {  // last key a position may see, -1 for none
  return p < 0 ? -1 : (p < S ? (int)p : S - 1);
}

// Four waves per SIMD (two workgroups per CU): the register budget this asks
// for (128) costs a few spills outside the MFMA sequences; measured 220 us at
// 4096 tokens against 250 us at three waves per SIMD.  With four waves per
// workgroup the staging work per query doubles (300 us).
__global__ __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(4))) void attn_prefill_kernel(
    PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) PrefillLds L;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t BH = (int64_t)a.B * a.Hq;
  const int64_t blk = blockIdx.x;
  const int qt = a.qtiles - 1 - (int)(blk / BH);  // longest first
  const int64_t bh = blk - (int64_t)(a.qtiles - 1 - qt) * BH;
  const int64_t b = bh / a.Hq, h = bh - b * a.Hq;
  const int64_t g = h / (a.Hq / a.Hkv);
  const int64_t st = a.start[b];
  const int t0 = qt * kPfQ;
  const int tlast = (t0 + kPfQ < a.T ? t0 + kPfQ : a.T) - 1;  // last query token of the workgroup
  const int kend = clamp_pos(st + tlast, a.S) + 1;            // keys [0, kend) reach some output
  const int ntiles = (kend + kPfKeys - 1) / kPfKeys;

  // This lane's query (column l%16 of the wave's 16) and the last key it sees.
  const int tq = t0 + 16 * wave + (lane & 15);
  const bool qvalid = tq < a.T;
  const int lim = qvalid ? clamp_pos(st + tq, a.S) : -1;
  // the wave's last key (uniform): tiles past it hold nothing for the wave
  const int twl = t0 + 16 * wave + 15 < a.T ? t0 + 16 * wave + 15 : a.T - 1;
  const int wlim = t0 + 16 * wave < a.T ? clamp_pos(st + twl, a.S) : -1;

  // Query rows as the B operand: lane l gives query l%16, bytes 32(l/16)..+31.
  v8i_t qf = {0, 0, 0, 0, 0, 0, 0, 0};
  float qsc = 1.0f;  // (a query past T sees no key: its weights are all 0)
  if (qvalid) {
    const int64_t qrow = (b * a.T + tq) * a.Hq + h;
    const uint4 *qp = reinterpret_cast<const uint4 *>(a.qq + qrow * kHeadDim + 32 * (lane >> 4));
    const uint4 x = qp[0], y = qp[1];
    qf[0] = x.x; qf[1] = x.y; qf[2] = x.z; qf[3] = x.w;
    qf[4] = y.x; qf[5] = y.y; qf[6] = y.z; qf[7] = y.w;
    qsc = a.qs[qrow];
  }

  const int64_t base = (b * a.Hkv + g) * (int64_t)a.S;  // (b, g, token 0) in the cache
  // Staging roles: the key and the value tile are 512 chunks of 16 bytes each
  // (row c/8, chunk c%8), kParts of each per thread; scales: threads below 128.
  constexpr int kParts = 512 / kPfThreads;
  const uint8_t *kp = a.kc + (base + (tid >> 3)) * kHeadDim + 16 * (tid & 7);
  const uint8_t *vp = a.vc + (base + (tid >> 3)) * kHeadDim + 16 * (tid & 7);
  constexpr int kStepRows = kPfThreads / 8;  // key rows between a thread's parts (both kinds)
  const float *sp = (tid < 64 ? a.ks : a.vs) + base + (tid & 63);
  constexpr float kL2eRsqrtD = 1.4426950408889634f * 0.08838834764831845f;
  const float smul = tid < 64 ? kL2eRsqrtD : 1.0f;

  uint4 kreg[kParts], vreg[kParts];
  float sreg = 0.0f;
  auto fetch = [&](int kt) {
    const int k0 = kt * kPfKeys;
    if (k0 + kPfKeys <= a.S) {  // whole tile inside the cache (uniform)
#pragma unroll
      for (int u = 0; u < kParts; ++u) {
        kreg[u] = *reinterpret_cast<const uint4 *>(kp + (int64_t)(k0 + u * kStepRows) * kHeadDim);
        vreg[u] = *reinterpret_cast<const uint4 *>(vp + (int64_t)(k0 + u * kStepRows) * kHeadDim);
      }
      if (tid < 128) sreg = sp[k0];
    } else {  // last tile: rows past the cache read its last row (masked later)
#pragma unroll
      for (int u = 0; u < kParts; ++u) {
        const int r = (tid >> 3) + u * kStepRows;
        const int64_t off = (int64_t)(k0 + r < a.S ? k0 + u * kStepRows : a.S - 1 - (tid >> 3)) * kHeadDim;
        kreg[u] = *reinterpret_cast<const uint4 *>(kp + off);
        vreg[u] = *reinterpret_cast<const uint4 *>(vp + off);
      }
      if (tid < 128) sreg = sp[k0 + (tid & 63) < a.S ? k0 : a.S - 1 - (tid & 63)];
    }
  };
  auto stage = [&]() {
    typedef float f2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int u = 0; u < kParts; ++u) {
      const int r = (tid >> 3) + u * kStepRows, cc = tid & 7;
      *reinterpret_cast<uint4 *>(&L.k[r * kHeadDim + 16 * (cc ^ (r & 7))]) = kreg[u];
      // value dims 16cc .. 16cc+15 of key r, decoded exactly to bf16
      uint32_t w[8];
      const uint32_t x[4] = {vreg[u].x, vreg[u].y, vreg[u].z, vreg[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)x[j], false);
        const f2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)x[j], true);
        w[2 * j] = bf16x2_of(lo.x, lo.y);
        w[2 * j + 1] = bf16x2_of(hi.x, hi.y);
      }
      uint4 *vd = reinterpret_cast<uint4 *>(&L.v[r * kPfVRow + 16 * cc]);
      vd[0] = (uint4){w[0], w[1], w[2], w[3]};
      vd[1] = (uint4){w[4], w[5], w[6], w[7]};
    }
    if (tid < 128) (tid < 64 ? L.ks : L.vs)[tid & 63] = sreg * smul;
  };

  float m_run = -__builtin_inff(), l_run = 0.0f;  // per query (lane column); l_run per lane
  v4f_t acc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) acc[db] = (v4f_t){0.0f, 0.0f, 0.0f, 0.0f};

  if (ntiles > 0) fetch(0);
  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * kPfKeys;
    __syncthreads();  // every wave is done with the previous tile
    stage();
    __syncthreads();
    if (kt + 1 < ntiles) fetch(kt + 1);  // in flight during this tile's math
    if (k0 > wlim) continue;             // the whole tile lies after the wave's last query

    // scores of the 64 keys (base 2): four MFMAs of 16 keys, in two pairs
    // whose operands are read together, the scaling of one pair after the
    // MFMAs of the next
    float sc[4][4];
    {
      auto kread = [&](int j, v8i_t &kf, float4 &ksc) {
        const int r = 16 * j + (lane & 15);
        const uint4 x = *reinterpret_cast<const uint4 *>(&L.k[r * kHeadDim + 16 * ((2 * (lane >> 4)) ^ (r & 7))]);
        const uint4 y = *reinterpret_cast<const uint4 *>(&L.k[r * kHeadDim + 16 * ((2 * (lane >> 4) + 1) ^ (r & 7))]);
        kf = (v8i_t){(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
        ksc = *reinterpret_cast<const float4 *>(&L.ks[16 * j + 4 * (lane >> 4)]);
      };
      const v4f_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
      v8i_t kf[2];
      float4 ksc[4];
      v4f_t d[4];
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        kread(2 * pr, kf[0], ksc[2 * pr]);
        kread(2 * pr + 1, kf[1], ksc[2 * pr + 1]);
        d[2 * pr] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf[0], qf, zero, 0, 0, 0, 127, 0, 127);
        d[2 * pr + 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf[1], qf, zero, 0, 0, 0, 127, 0, 127);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sc[j][0] = d[j][0] * ksc[j].x;  // the query scale (> 0) is applied in the exponent
        sc[j][1] = d[j][1] * ksc[j].y;
        sc[j][2] = d[j][2] * ksc[j].z;
        sc[j][3] = d[j][3] * ksc[j].w;
      }
    }
    // keys past a query's position (the diagonal tiles and the cache end)
    if (__builtin_amdgcn_ballot_w64(k0 + kPfKeys - 1 > lim) != 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (k0 + 16 * j + 4 * (lane >> 4) + i > lim) sc[j][i] = -__builtin_inff();
    }
    // online softmax (the four lanes l, l^16, l^32, l^48 share a query); the
    // score is qsc * sc, and qsc > 0, so its maximum is qsc * max(sc)
    float mt = sc[0][0];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) mt = __builtin_fmaxf(mt, sc[j][i]);
    mt = __builtin_fmaxf(mt, __shfl_xor(mt, 16));
    mt = __builtin_fmaxf(mt, __shfl_xor(mt, 32));
    mt *= qsc;
    const bool raise = mt > m_run + kPfLazy;  // false for a tile with no key for this query
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
      const float m_new = raise ? mt : m_run;
      const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;  // 0 from -inf
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db) acc[db] *= alpha;
    }
    const float m_use = m_run == -__builtin_inff() ? 0.0f : m_run;
    float psum = 0.0f;
    uint32_t pw[2][4];  // bf16 pairs of p * v_scale: [32-key half][k-slot pair]
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const float4 va = *reinterpret_cast<const float4 *>(&L.vs[32 * hf + 4 * (lane >> 4)]);
      const float4 vb = *reinterpret_cast<const float4 *>(&L.vs[32 * hf + 16 + 4 * (lane >> 4)]);
      const float vsa[4] = {va.x, va.y, va.z, va.w}, vsb[4] = {vb.x, vb.y, vb.z, vb.w};
      float p[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(qsc, sc[2 * hf][i], -m_use));
        p[4 + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(qsc, sc[2 * hf + 1][i], -m_use));
        psum += p[i] + p[4 + i];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        pw[hf][i] = bf16x2_of(p[2 * i] * vsa[2 * i], p[2 * i + 1] * vsa[2 * i + 1]);
        pw[hf][2 + i] = bf16x2_of(p[4 + 2 * i] * vsb[2 * i], p[4 + 2 * i + 1] * vsb[2 * i + 1]);
      }
    }
    l_run += psum;
    // O^T += V^T P^T, 32 keys at a time; each value fragment is read two
    // MFMAs ahead of its use.  Fragment (hf, db): lane (q = l/16, i = l%16)
    // needs dim 16db + i of keys 32hf + 4q + j and 32hf + 16 + 4q + j
    // (j = 0..3), two transpose loads in which lane r of group q names key
    // 32hf + 4q + r/4 (+16), dims 16db + 4(r%4) .. +3.
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, (uint4){pw[hf][0], pw[hf][1], pw[hf][2], pw[hf][3]});
      const uint16_t *vrow = &L.v[(32 * hf + 4 * (lane >> 4) + ((lane >> 2) & 3)) * kPfVRow + 4 * (lane & 3)];
      auto vread = [&](int db) {
        const v4s_t lo = lds_read_tr16(vrow + 16 * db);
        const v4s_t hi = lds_read_tr16(vrow + 16 * kPfVRow + 16 * db);
        return (uint4){__builtin_bit_cast(uint2, lo).x, __builtin_bit_cast(uint2, lo).y,
                       __builtin_bit_cast(uint2, hi).x, __builtin_bit_cast(uint2, hi).y};
      };
      uint4 vf[3];
      vf[0] = vread(0);
      vf[1] = vread(1);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        if (db + 2 < 8) vf[(db + 2) % 3] = vread(db + 2);
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vf[db % 3]), pb, acc[db], 0, 0,
                                                          0);
      }
    }
  }

  // Normalize and store: lane l holds dims 16db + 4(l/16) .. +3 of query l%16.
  float ltot = l_run + __shfl_xor(l_run, 16);
  ltot += __shfl_xor(ltot, 32);
  if (!qvalid) return;
  const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
  uint16_t *o = a.out + ((b * a.T + tq) * a.Hq + h) * kHeadDim + 4 * (lane >> 4);
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    uint2 w;
    w.x = bf16x2_of(acc[db][0] * inv, acc[db][1] * inv);
    w.y = bf16x2_of(acc[db][2] * inv, acc[db][3] * inv);
    *reinterpret_cast<uint2 *>(o + 16 * db) = w;
  }
}

hipError_t launch_attention_prefill(const uint8_t *qq, const float *qs, const uint8_t *kc, const float *ks,
                                    const uint8_t *vc, const float *vs, const int32_t *start, uint16_t *out,
                                    int32_t B, int32_t T, int32_t Hq, int32_t Hkv, int64_t S,
                                    hipStream_t stream) {
  if ((int64_t)B * T * Hq == 0) return hipSuccess;
  PrefillArgs a{qq, qs, kc, ks, vc, vs, start, out, B, T, Hq, Hkv, (int32_t)S, (T + kPfQ - 1) / kPfQ};
  const int64_t grid = (int64_t)a.qtiles * B * Hq;
  hipLaunchKernelGGL(attn_prefill_kernel, dim3((unsigned)grid), dim3(kPfThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fp8q
