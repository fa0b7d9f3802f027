// Kernel launchers behind the C ABI (host side).  Arguments are validated by
// the ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

struct fp8q_weight_job;  // include/fp8q.h

namespace fp8q {

// Devices the library keeps per-device set-up for (ids 0 .. kMaxDevices-1).
constexpr int kMaxDevices = 64;

hipError_t launch_quant_act_1x128(const uint16_t *x, int64_t M, int64_t K,
                                  uint8_t *q, float *s, int mode,
                                  hipStream_t stream);

hipError_t launch_quant_weight_128x128(const uint16_t *w, int64_t N, int64_t K,
                                       uint8_t *q, float *s, int mode,
                                       hipStream_t stream);

// Many weight matrices in one launch: jobs [count] in device memory,
// total_tiles < 2^31 tiles in all.
hipError_t launch_quant_weight_batched(const fp8q_weight_job *jobs, int32_t count, int64_t total_tiles,
                                       int mode, hipStream_t stream);

// pow2: every scale is a power of two and the matrix core applies it (E8M0
// scale operands); otherwise the per-K-block scale fold runs on the VALU.
hipError_t launch_blockscaled_gemm(const uint8_t *a_q, const float *a_s,
                                   const uint8_t *b_q, const float *b_s,
                                   uint16_t *y, int64_t M, int64_t N, int64_t K,
                                   bool pow2, hipStream_t stream);

// The same GEMM with its output quantized to E4M3 in 1x128 blocks along N
// (mode: scale rule of those blocks), equal to quantizing the bf16 output.
hipError_t launch_blockscaled_gemm_quant(const uint8_t *a_q, const float *a_s,
                                         const uint8_t *b_q, const float *b_s,
                                         uint8_t *yq, float *ys, int64_t M, int64_t N, int64_t K,
                                         int mode, hipStream_t stream);

// Weight panels (256 rows each) of a dense M x N GEMM output that run on
// 256-row tiles; the others run on 128-row tiles (bf16_out: a bf16 output,
// which may be split between the two shapes).
// Tile plan of a dense M x N output: rows [0, rows_large) x panels
// [0, panels_large) on 256-token tiles, the rest on 128-token tiles.
void dense_tile_plan(int64_t M, int64_t N, bool may_split, int64_t &rows_large, int64_t &panels_large);

hipError_t launch_grouped_gemm(const uint8_t *a_q, const float *a_s,
                               const uint8_t *b_q, const float *b_s,
                               const int32_t *group_offsets, int32_t G,
                               int64_t M_total, int64_t N, int64_t K,
                               uint16_t *y, bool pow2, hipStream_t stream);

// GEMM with 1x128 scale blocks on both operands: a_s [M][K/128] and one
// scale per row and 128-block of K for b as well, b_s [N][K/128] (the weight
// gradient from 128-token column blocks of dY and X).
hipError_t launch_blockscaled_gemm_wgrad(const uint8_t *a_q, const float *a_s,
                                         const uint8_t *b_q, const float *b_s,
                                         uint16_t *y, int64_t M, int64_t N, int64_t K, bool pow2,
                                         hipStream_t stream);

// Fused gate+up GEMM of a SwiGLU MLP: b_q [2F][K] holds gate and up in
// alternating 128-row blocks; writes h = silu(gate) * up quantized in 1x128
// blocks, hq [M][F], hs [M][F/128].  F % 128 == 0.
hipError_t launch_blockscaled_gemm_swiglu_quant(const uint8_t *a_q, const float *a_s,
                                                const uint8_t *b_q, const float *b_s,
                                                uint8_t *hq, float *hs, int64_t M, int64_t F, int64_t K,
                                                int mode, hipStream_t stream);

// Row-major and transposed codes of x [M][K] in one pass.  tile: one scale per
// 128x128 tile (weights; M % 128 == 0), q_t [K][M], s_t [K/128][M/128].
// Otherwise 1x128 row blocks (q, s; may be null) and 128x1 column blocks
// stored transposed, q_t [K][Mp], s_t [K][Mp/128], Mp = M rounded up to 128.
hipError_t launch_quant_dual(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s, uint8_t *qt,
                             float *st, int mode, bool tile, hipStream_t stream);

// RMS normalization of x [M][K] by gamma [K] with eps, output quantized in
// 1x128 blocks: q [M][K], s [M][K/128].  K % 128 == 0, K <= 8192.
hipError_t launch_rmsnorm_quant_1x128(const uint16_t *x, const uint16_t *gamma, int64_t M, int64_t K, float eps,
                                      uint8_t *q, float *s, int mode, hipStream_t stream);

// Grouped GEMM whose token rows are gathered: routed row r reads token row
// row_index[r] of a_q [T][K] / a_s [T][K/128] (quantize before dispatch).
hipError_t launch_grouped_gemm_gather(const uint8_t *a_q, const float *a_s, int64_t T,
                                      const uint8_t *b_q, const float *b_s,
                                      const int32_t *group_offsets, const int32_t *row_index, int32_t G,
                                      int64_t M_total, int64_t N, int64_t K, uint16_t *y, bool pow2,
                                      hipStream_t stream);
// Grouped gate+up GEMM with the SwiGLU epilogue (row_index may be null: rows
// of a_q in order).
hipError_t launch_grouped_gemm_swiglu_quant(const uint8_t *a_q, const float *a_s, int64_t T,
                                            const uint8_t *b_q, const float *b_s,
                                            const int32_t *group_offsets, const int32_t *row_index, int32_t G,
                                            int64_t M_total, int64_t F, int64_t K, uint8_t *hq, float *hs,
                                            int mode, hipStream_t stream);

// MoE dispatch order: routing table ids [T][k] -> offsets [E+n_shared+1],
// row_index [T*(k+n_shared)], entry_row [T*k] (may be null), through a
// workspace of moe_permute_workspace_bytes(T*k, E).  1 <= E <= 1024.
int64_t moe_permute_workspace_bytes(int64_t n, int32_t E);
hipError_t launch_moe_permute(const int32_t *ids, int64_t T, int32_t k, int32_t E, int32_t n_shared,
                              int32_t *offsets, int32_t *row_index, int32_t *entry_row, void *workspace,
                              hipStream_t stream);

// FP8 KV cache: quantize T new key and value rows per sequence and head
// ([B][T][H][128] bf16, 1x128 blocks) into [B][H][S][128] caches, token t of
// sequence b at position start[b] + t.
hipError_t launch_kv_cache_append(const uint16_t *k_new, const uint16_t *v_new, const int32_t *start, uint8_t *kc,
                                  float *ks, uint8_t *vc, float *vs, int32_t B, int32_t T, int32_t H, int64_t S,
                                  int mode, hipStream_t stream);

// Causal attention of T query tokens per sequence ([B][T][Hq][128] E4M3)
// over the FP8 cache; query t of sequence b at position start[b] + t.
hipError_t launch_attention_prefill(const uint8_t *qq, const float *qs, const uint8_t *kc, const float *ks,
                                    const uint8_t *vc, const float *vs, const int32_t *start, uint16_t *out,
                                    int32_t B, int32_t T, int32_t Hq, int32_t Hkv, int64_t S,
                                    hipStream_t stream);

// Decode attention over the FP8 KV cache (Hq / Hkv in {1, 2, 4, 8}).  With a
// workspace of B*Hq*nch*130 floats (nch from attention_decode_split) and
// nch > 1, sequences are split into chunks merged by a second kernel;
// otherwise one workgroup covers a whole sequence.
void attention_decode_split(int64_t pairs, int64_t S, int64_t &nch, int64_t &chunk_tiles);
hipError_t launch_attention_decode(const uint8_t *qq, const float *qs, const uint8_t *kc, const float *ks,
                                   const uint8_t *vc, const float *vs, const int32_t *len, uint16_t *out,
                                   int32_t B, int32_t Hq, int32_t Hkv, int64_t S, float *workspace,
                                   hipStream_t stream);

// The same attention with the chunked path's workspace in a static device
// array of attention_noalloc_scratch_bytes() (no allocation, no workspace
// argument); shared by every call on a device.
int64_t attention_noalloc_scratch_bytes();
hipError_t launch_attention_decode_noalloc(const uint8_t *qq, const float *qs, const uint8_t *kc,
                                           const float *ks, const uint8_t *vc, const float *vs,
                                           const int32_t *len, uint16_t *out, int32_t B, int32_t Hq,
                                           int32_t Hkv, int64_t S, hipStream_t stream);

}  // namespace fp8q
