// Block-scaled FP8 GEMM (dense and grouped) for gfx950.
//
//   Y[m][n] = sum_kb a_s[m][kb] * b_s[n/128][kb] * P_kb[m][n],
//   P_kb[m][n] = sum_{k in block kb} dec(a_q[m][k]) * dec(b_q[n][k])
//
// (page "NVIDIA NeMo RL erreicht 48% Geschwindigkeitssteigerung ...", section
// "Der technische Durchbruch": FP8 linear layers with 1x128 activation and
// 128x128 weight scale blocks.)
//
// Design for CDNA4:
//  - One v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 x E4M3, neutral E8M0 scales)
//    covers exactly one 128-wide scale block of K, so P_kb comes out of a
//    single MFMA with a zero accumulator and is folded into the fp32
//    accumulator with one FMA per output: acc += P_kb * (a_s * b_s).  The
//    FMAs run on the VALU while the matrix core works on the next MFMAs.
//  - The weight tile is the MFMA "A" operand (rows of D) and the token tile the
//    "B" operand (columns of D).  Then each lane's four outputs are four
//    consecutive n of one token row m: they share one scale product and are
//    stored as one 8-byte bf16 quad.
//  - Each wave owns 128 (n) x 64 (m) outputs = 8 x 4 MFMA sub-tiles (128 fp32
//    accumulators per lane), or 64 (n) x 64 (m) in the 128-row tiles.  Tile
//    shapes (weight rows x token rows), all with a 2-stage pipeline:
//      256 x 256 tiles, 8 waves (2 per SIMD)               (large M)
//      256 x 128 tiles, 8 waves, 4 along n                 (small M, a
//                                      group's last slot, split plans)
//  - Everything a K block needs -- the weight and token tiles and both scale
//    vectors -- reaches LDS by direct global->LDS DMA (global_load_lds), so a
//    stage is a fixed number of vector-memory instructions per wave and the
//    wait for stage k is one s_waitcnt vmcnt(<later stages' count>).
//  - Rows are 128 B in LDS; 16-byte chunks are XOR-swizzled by row so that the
//    fragment reads (two ds_read_b128 per lane) hit distinct banks.
//  - Workgroup ids are remapped so that each XCD (own L2) gets a contiguous
//    range of tiles, enumerated in groups of 8 weight panels so that the tiles
//    running at the same time share operand panels.
#include <mutex>

#include "fp8q_device.h"
#include "fp8q_internal.h"

namespace fp8q {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

constexpr int kBN = 256;  // weight rows per tile
constexpr int kBK = 128;  // one scale block of K
constexpr int kSubN = 8;  // 16-row MFMA sub-tiles per wave along n, at most (128 rows)
constexpr int kSubM = 4;  // 16-col MFMA sub-tiles per wave along m (64 rows)
constexpr int kNumXcd = 8;
constexpr int kGroupN = 8;  // weight panels per rasterization group

// Output of a tile: bf16 Y, or Y quantized to E4M3 in 1x128 blocks along N
// with the activation quantizer's rule (kOut = its scale mode).
constexpr int kOutBf16 = -1;

// What a kernel instance computes:
//   kGrouped  groups of rows, each with its own weight matrix (device offsets)
//   kPow2     power-of-two scales, applied by the matrix cores (E8M0)
//   kOut      bf16 output, or the output quantized in the epilogue
//   kGather   grouped rows read by index from a token matrix
//   kBRow     the weight-side operand carries one scale per row and 128-block
//             of K (1x128 blocks on both operands) instead of 128x128 tiles
//   kSwiGLU   (with a quantized kOut) the weight rows alternate 128-row gate
//             and up blocks; the epilogue writes silu(gate) * up, quantized
template <bool kGrouped_, bool kPow2_, int kOut_ = kOutBf16, bool kGather_ = false, bool kBRow_ = false,
          bool kSwiGLU_ = false>
struct Variant {
  static constexpr bool kGrouped = kGrouped_;
  static constexpr bool kPow2 = kPow2_;
  static constexpr int kOut = kOut_;
  static constexpr bool kGather = kGather_;
  static constexpr bool kBRow = kBRow_;
  static constexpr bool kSwiGLU = kSwiGLU_;
  static_assert(!(kSwiGLU && (kOut == kOutBf16 || kBRow || kPow2)), "SwiGLU: quantized output, amax arithmetic");
  static_assert(!(kGather && !kGrouped), "gathered rows belong to groups");
  static_assert(!(kBRow && kGrouped), "per-row weight-side scales: dense only");
};

template <int kBM_, int kWaves_, int kStages_, int kLoaders_, int kDmaStep_, int kWAhead_ = 1, int kWavesN_ = 2,
          bool kPingPong_ = false>
struct TileCfg {
  // The ping-pong main loop (gemm_main_pp) instead of the lockstep one.
  static constexpr bool kPingPong = kPingPong_;
  static constexpr int kBM = kBM_;
  static constexpr int kWaves = kWaves_;
  static constexpr int kStages = kStages_;
  // The n step of a K block at which the waves issue the DMA of the next
  // block.  Issuing it mid-block keeps its LDS writes away from the fragment
  // reads that start each block.  256-row tiles (8 waves, lockstep loop):
  // step 3.  Against step 0 steps 2-4 gain 5-8% on the dense Llama shapes; at
  // step 5 and later the DMA is not finished when the block ends.  Step 3
  // against 4: dense +1-2%, grouped MoE GEMMs +1-10% (Qwen3 down +10%, gathered
  // rows +4-6%), whose tiles' operands miss in L2 more often, so the DMA needs
  // the extra step to land.  128-row tiles (8 waves, four sub-tile rows per
  // wave): step 2 (step 1: -1-3%, step 0: -3-7%).
  // The last kLoaders waves issue the stage DMA.
  static constexpr int kLoaders = kLoaders_;
  static constexpr int kDmaStep = kDmaStep_;
  // Weight sub-tiles whose LDS reads go out ahead of their MFMAs.
  static constexpr int kWAhead = kWAhead_;
  // Waves along n: 2 (128 weight rows each) or 4 (64 each); the rest along m.
  static constexpr int kWavesN = kWavesN_;
  static constexpr int kWaveN = kBN / kWavesN;  // weight rows per wave
  static constexpr int kSubN = kWaveN / 16;     // MFMA sub-tiles per wave along n
  static constexpr int kMfma = kSubN * kSubM;   // MFMAs per wave and K block
  static_assert(kWavesN == 2 || kWavesN == 4, "waves along n");
  static_assert(kDmaStep < kSubN - 1, "the DMA goes out in one of the n steps before the deferred last row");
  static constexpr int kFirstLoader = kWaves - kLoaders;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kWavesM = kWaves / kWavesN;  // waves along m
  static_assert(kBM == 64 * kWavesM, "each wave owns 64 token rows");
  static constexpr int kBytesB = kBN * kBK;        // weight tile
  static constexpr int kBytesA = kBM * kBK;        // token tile
  static constexpr int kBytesSA = kBM * 4;         // activation scales
  static constexpr int kBytesSB = kBN * 4;         // weight-side scales: per 128-row block or per row
  static constexpr int kOffA = kBytesB;
  static constexpr int kOffSA = kOffA + kBytesA;
  static constexpr int kOffSB = kOffSA + kBytesSA;
  static constexpr int kStageBytes = (kOffSB + kBytesSB + 1023) / 1024 * 1024;
  static constexpr int kLdsBytes = kStageBytes * kStages;
  // Scale chunks of the per-row-scale variant (issue_chunk_quarter): the
  // activation scales and the per-row weight-side scales of four K blocks,
  // double-buffered after the stages.
  static constexpr int kChunkSA = kBM * 16;
  static constexpr int kChunkBytes = kChunkSA + kBN * 16;
  static constexpr int kOffChunk = kStageBytes * kStages;
  static constexpr int kLdsBytesChunked = kOffChunk + 2 * kChunkBytes;
  static constexpr int kPiecesB = kBytesB / 1024 / kLoaders;  // 1 KB DMA pieces per loader wave
  static constexpr int kPiecesA = kBytesA / 1024 / kLoaders;
  static constexpr int kPieces = kPiecesB + kPiecesA;         // operand pieces per loader wave
  static constexpr int kScaleLoaders = kBM / 64;              // loaders 0.. each fetch 64 activation scales
  static_assert(kScaleLoaders <= kLoaders && kBM % 64 == 0, "activation scales: one per lane");
  static_assert(kStages == 2, "the DMA wait before a block's barrier is vmcnt(0): two stages");
  static_assert(kLdsBytesChunked <= 160 * 1024, "LDS budget");
};

// 256 x 256 tiles: on the ping-pong schedule (gemm_main_pp) when the
// matrix cores apply power-of-two scales, on the lockstep one when the VALU
// folds the scales in.  A VALU read of a register an MFMA wrote stalls the
// wave (measured on gfx950: an MFMA stream with a 4-FMA fold of an earlier
// product per MFMA reaches ~3.3 PFLOP/s against ~4.2 without, whatever the
// distance to the MFMA that wrote it; independent FMAs cost ~5%).  In
// lockstep the other wave of the SIMD keeps the matrix core busy through
// such a stall; in ping-pong it is reading LDS, so the folds cost 10% more
// (Llama gate+up and down).  Without folds the ping-pong loop is 3-6% ahead.
using CfgLarge = TileCfg<256, 8, 2, 8, 0, 1, 2, true>;
using CfgLargeLockstep = TileCfg<256, 8, 2, 8, 3>;
// 128-row tiles with 8 waves (4 along n, 64 weight rows each; 2 per SIMD).
// The quantized and SwiGLU epilogues split a 1x128 output block between two
// waves; per-row weight-side scales are staged for the wave's four sub-tile
// rows.
using CfgSmall8 = TileCfg<128, 8, 2, 8, 2, 1, 4>;
template <class V>
using LargeCfg = typename std::conditional<V::kPow2 && !V::kBRow, CfgLarge, CfgLargeLockstep>::type;
template <class V>
using SmallCfg = CfgSmall8;

// Row swizzle of the 16-byte chunks: chunk c of row r lives in slot
// c ^ (r & 7) ^ ((r >> 3) & 1).  Sixteen consecutive rows reading the same
// logical chunk then fall into 16 distinct (slot, row parity) pairs.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int lds_off(int r, int c) { return r * 128 + ((c ^ swz(r)) << 4); }

// Position in the activation-scale vector of row r = wm*64 + mi*16 + j:
// wm*64 + j*4 + mi, so that lane j of a wave reads its four rows (mi = 0..3)
// with one 16-byte LDS read.
__device__ __forceinline__ int sa_row_of_pos(int p) {
  const int wm = p >> 6, j = (p & 63) >> 2, mi = p & 3;
  return wm * 64 + mi * 16 + j;
}

// Scale chunks (the per-row-scale variant, 1x128 blocks on both operands).
// Both scale vectors are stored one row per token or weight-side row with the
// K blocks contiguous, so a 64-lane 4-byte load of one K block (one row per
// lane) touches 64 cache lines, and a CU's memory path pays per line.  With
// two such vectors per stage that cost the weight-gradient GEMM 10-28% of
// its time (measured against the same loads made contiguous, wrong values).
// Instead a chunk holds the scales of K blocks 4c .. 4c+3 and a load
// instruction covers 16 rows x 4 blocks (lane l: row slot t = l % 16, block
// l / 16), 16 cache lines: Llama weight gradients 8-11% faster with
// VALU-folded scales, 10-23% with power-of-two ones.  In LDS the 64 words of instruction i sit
// at [i][block][t].  Chunk c lives in buffer c % 2; the stage of block 0
// loads chunk 0 whole, and the stage of block kn >= 1 loads quarter
// (kn - 1) % 4 of chunk (kn - 1) / 4 + 1, so chunk c is complete with the
// stage of block 4c, and the previous chunk in its buffer (c - 2) was last
// read in block 4c - 5, before the stage of block 4c - 3 is issued.  (For
// the other variants, with one such vector and a scale per weight tile,
// chunks measured 1-2% slower than one load per block, and 5-8% slower with
// gathered rows, whose row offsets per chunk quarter take registers.)
constexpr int kScChunk = 4;

// Row of slot t in instruction i of a chunk, per scale vector.  Activation
// (token-side) scales: lane j of a wave reads its four token rows wm*64 +
// mi*16 + j (mi = 0..3) of one block as four consecutive words.
__host__ __device__ constexpr int sa_chunk_row(int i, int t) {
  return (i >> 2) * 64 + (t & 3) * 16 + 4 * (i & 3) + (t >> 2);
}
// Per-row weight-side scales folded by the VALU: row order, so the four rows
// of a lane's outputs (16ni + 4(l/16) + r) are consecutive.
__host__ __device__ constexpr int sbf_chunk_row(int i, int t) { return 16 * i + t; }
// Per-row power-of-two weight-side scales: the eight rows a lane supplies to
// the eight A sub-tiles of its wave (128w + 16s + c, c = l % 16) are
// consecutive.
__host__ __device__ constexpr int sbp_chunk_row(int i, int t) {
  return 128 * (i >> 3) + 16 * (t & 7) + 2 * (i & 7) + (t >> 3);
}
// The same for 64-row waves (the 128-row, 8-wave tiles): the four rows a lane
// supplies to the four A sub-tiles of its wave (64w + 16s + c) are
// consecutive.
__host__ __device__ constexpr int sbp64_chunk_row(int i, int t) {
  return (i >> 2) * 64 + (t & 3) * 16 + 4 * (i & 3) + (t >> 2);
}
// Every row of the tile exactly once per chunk.
template <int (*kRow)(int, int)>
constexpr bool chunk_covers(int rows) {
  int seen[256] = {};
  for (int i = 0; i < rows / 16; ++i)
    for (int t = 0; t < 16; ++t) {
      const int r = kRow(i, t);
      if (r < 0 || r >= rows || seen[r]) return false;
      seen[r] = 1;
    }
  return true;
}
static_assert(chunk_covers<sa_chunk_row>(256) && chunk_covers<sa_chunk_row>(128) &&
                  chunk_covers<sbf_chunk_row>(256) && chunk_covers<sbp_chunk_row>(256) &&
                  chunk_covers<sbp64_chunk_row>(256),
              "scale chunk rows");

// The chunk and quarter that the stage of block kn >= 1 loads.
__device__ __forceinline__ int chunk_of_stage(int kn) { return ((kn - 1) >> 2) + 1; }
__device__ __forceinline__ int quarter_of_stage(int kn) { return (kn - 1) & 3; }

// LDS byte offset of block k's scales in its chunk buffer ((k/4) % 2, block
// k % 4), and the words a lane reads there: its four token rows (16 bytes);
// the four rows of weight sub-tile row ni of its outputs (VALU fold, 16
// bytes); the eight rows it supplies to the A sub-tiles (power-of-two, 32
// bytes).
template <class C>
__device__ __forceinline__ int chunk_base(int k) {
  return C::kOffChunk + ((k >> 2) & 1) * C::kChunkBytes + (k & 3) * 64;
}
template <class C>
__device__ __forceinline__ const float4 *sa_chunk_ptr(const uint8_t *lds, int k, int wm, int lane) {
  const int j = lane & 15;
  return reinterpret_cast<const float4 *>(lds + chunk_base<C>(k) + (wm * 4 + (j >> 2)) * 256 + 16 * (j & 3));
}
template <class C>
__device__ __forceinline__ const float4 *sbf_chunk_ptr(const uint8_t *lds, int k, int wn, int ni, int lane) {
  return reinterpret_cast<const float4 *>(lds + chunk_base<C>(k) + C::kChunkSA + (wn * C::kSubN + ni) * 256 +
                                          16 * (lane >> 4));
}
template <class C>
__device__ __forceinline__ const float4 *sbp_chunk_ptr(const uint8_t *lds, int k, int wn, int lane) {
  const int c = lane & 15;
  if constexpr (C::kWaveN == 128)
    return reinterpret_cast<const float4 *>(lds + chunk_base<C>(k) + C::kChunkSA + (wn * 8 + (c >> 1)) * 256 +
                                            32 * (c & 1));
  else
    return reinterpret_cast<const float4 *>(lds + chunk_base<C>(k) + C::kChunkSA + (wn * 4 + (c >> 2)) * 256 +
                                            16 * (c & 3));
}

// This lane's index, computed where it is used.  The asm statement cannot be
// hoisted out of a loop, so the chunk-load offsets derived from it are
// recomputed at each stage (a few VALU operations) instead of being held
// through the main loop, where the register allocator spilled them (and the
// wait for a spill reload, vmcnt(0), also waits for the DMA already issued).
__device__ __forceinline__ uint32_t lane_id_now() {
  uint32_t l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Byte offset of this lane's word in chunk 0 of a scale vector whose
// instruction i (uniform) maps row slots by kRow: row slot lane % 16, K block
// lane / 16.
template <int (*kRow)(int, int)>
__device__ __forceinline__ uint32_t chunk_lane_off(int i, int KB) {
  const uint32_t ln = lane_id_now();
  return (uint32_t)(kRow(i, (int)(ln & 15u)) * KB + (int)(ln >> 4)) * 4u;
}

struct TileJob {
  const uint8_t *a_q;  // row 0 of the token tile (gathered: the token matrix)
  const float *a_s;    // scale row of token row 0 (gathered: the scale matrix)
  const int32_t *gidx; // gathered: source token row of each tile row; else null
  int64_t T;           // gathered: rows of the token matrix
  const uint8_t *b_q;  // row 0 of the weight tile
  const float *b_s;    // weight-scale row of the tile's first 128 rows
  int m_valid;         // token rows in the tile (1..kBM)
  int n_valid;         // weight rows in the tile (128 or 256)
  int64_t K;
  int KB;
};

// Raw buffer resources of the tile's scale vectors.  num_records bounds each
// one to the tile's valid rows, so a load past them returns zeros (those
// products only reach masked outputs) and never touches memory outside the
// tensors.
struct TileRsrc {
  __amdgpu_buffer_rsrc_t sa, sb;
};

constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) 32-bit buffer access

template <class V>
__device__ __forceinline__ TileRsrc make_rsrc(const TileJob &t) {
  constexpr bool kGather = V::kGather;
  TileRsrc r;
  // gathered: bounded to the whole scale matrix (the lanes' offsets select rows)
  r.sa = __builtin_amdgcn_make_buffer_rsrc((void *)t.a_s, (short)0,
                                           kGather ? (int)(t.T * t.KB * 4) : t.m_valid * t.KB * 4, kRsrcWord3);
  r.sb = __builtin_amdgcn_make_buffer_rsrc((void *)t.b_s, (short)0,
                                           (V::kBRow ? t.n_valid : (t.n_valid + 127) >> 7) * t.KB * 4, kRsrcWord3);
  return r;
}

// Resource of one 8-row DMA piece of an operand tile: based at row 8*piece and
// byte kbyte of the row, bounded to the piece's valid rows (0..8), so rows
// past the tile's last valid one read zeros exactly as with one resource per
// tile.  Its inputs are wave-uniform, so it is built in scalar registers and a
// lane's offset is only (row in piece)*K + chunk.  (The raw-buffer bound does
// not cover the scalar offset operand, which is why the row offset goes into
// the base rather than there.)
//
// kScalar: write the clamp so that it stays in scalar instructions.  As
// min(max(.)), the compiler folds it into one v_med3_i32 and keeps the
// per-piece bounds in vector registers; in the per-row-scale variant these
// were spilled (its in-loop reloads then wait for all vector-memory
// operations, the DMA included).  The other variants keep the fold: with the
// scalar form their register allocation spilled more.
template <bool kScalar = false>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t piece_rsrc(const uint8_t *rows, int valid_rows, int64_t K,
                                                              int piece, uint32_t kbyte) {
  int nr = valid_rows - 8 * piece;
  if (!kScalar) nr = nr < 0 ? 0 : nr;
  nr = nr > 8 ? 8 : nr;
  const uint64_t base = (uint64_t)(uintptr_t)(rows + (int64_t)(8 * piece) * K + kbyte);
  // Uniform by construction; readfirstlane tells the compiler so (it would
  // otherwise wrap each load in a loop over distinct resource values).
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
  const int n = __builtin_amdgcn_readfirstlane(kScalar ? (nr > 0 ? nr * (int)K : 0) : nr * (int)K);
  return __builtin_amdgcn_make_buffer_rsrc((void *)(uintptr_t)(((uint64_t)hi << 32) | lo), (short)0, n, kRsrcWord3);
}

constexpr int kMaxPiecesA = 4;
// An offset at or past every gathered resource's bound (token matrices are
// limited to fewer than 2^31 bytes).
constexpr uint32_t kGatherOOB = 0x80000000u;

// Resource over a whole gathered token matrix [T][K], based at byte kbyte of
// row 0; each lane's offset selects its row.  The bound T*K - kbyte (at least
// 128, as T >= 1) makes a valid row's 16 bytes always in range and kGatherOOB
// always out of it.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gather_rsrc(const uint8_t *a, int64_t T, int64_t K,
                                                               uint32_t kbyte) {
  const uint64_t base = (uint64_t)(uintptr_t)(a + kbyte);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
  const int n = __builtin_amdgcn_readfirstlane((int)(T * K - (int64_t)kbyte));
  return __builtin_amdgcn_make_buffer_rsrc((void *)(uintptr_t)(((uint64_t)hi << 32) | lo), (short)0, n, kRsrcWord3);
}

// Per-lane byte offsets of the DMA pattern (constant over K blocks).  Piece p
// of a tile holds rows 8p .. 8p+7; lane l fills row 8p + l/8, LDS slot l%8,
// which holds logical chunk c = (l%8) ^ swz(row) = (l%8) ^ (l/8) ^ (p%2).
struct DmaLane {
  uint32_t rc[2];  // (row in piece)*K + chunk offset, even / odd pieces
  // Scale rows (not the per-row variant, whose chunk loads recompute theirs):
  uint32_t sa;     // activation-scale row of this lane
  uint32_t sb;     // weight tile's 128-row block of this lane (lanes 0..1)
  // Gathered token rows: this lane's byte offset in the token matrix for each
  // of its loader's token pieces, and of its scale row; kGatherOOB for a row
  // past the tile or an index outside [0, T), which then reads zeros.
  uint32_t ga[kMaxPiecesA];
  uint32_t gsa;
};

template <class C, class V>
__device__ __forceinline__ DmaLane dma_lane(const TileJob &t, int wave, int lane) {
  constexpr bool kGather = V::kGather;
  DmaLane d;
  const uint32_t row = (uint32_t)(lane >> 3);
  const uint32_t c0 = (uint32_t)((lane & 7) ^ (lane >> 3));
  const uint32_t K = (uint32_t)t.K;
#pragma unroll
  for (int par = 0; par < 2; ++par) d.rc[par] = row * K + ((c0 ^ par) << 4);
  const int l = wave - C::kFirstLoader;  // meaningful for loader waves only
  d.sa = (uint32_t)sa_row_of_pos((l % C::kScaleLoaders) * 64 + lane) * (uint32_t)t.KB * 4u;
  d.sb = (uint32_t)(lane & 1) * (uint32_t)t.KB * 4u;
  if constexpr (kGather) {
    static_assert(C::kPiecesA <= kMaxPiecesA, "gather offsets per lane");
    auto src = [&](int r) -> int64_t {  // source token row of tile row r, or -1
      if (l < 0 || r >= t.m_valid) return -1;
      const int64_t s = t.gidx[r];
      return (s >= 0 && s < t.T) ? s : -1;
    };
#pragma unroll
    for (int i = 0; i < C::kPiecesA; ++i) {
      const int piece = l * C::kPiecesA + i;
      const int64_t s = src(8 * piece + (int)row);
      d.ga[i] = s < 0 ? kGatherOOB : (uint32_t)s * K + ((c0 ^ (uint32_t)(piece & 1)) << 4);
    }
    const int64_t s = src(sa_row_of_pos((l % C::kScaleLoaders) * 64 + lane));
    d.gsa = s < 0 ? kGatherOOB : (uint32_t)s * (uint32_t)t.KB * 4u;
  }
  return d;
}

// The DMA of K block k into one stage buffer: kPieces 16-byte operand pieces
// (1 KB each) per loader wave, plus the scales -- one 64-lane activation-scale
// load on each of the first kScaleLoaders loaders and one 2-lane weight-scale
// load on the first.  Each load is one vector-memory instruction; a CU's
// vector-memory path takes about one such 1 KB load every 20 clocks, so the
// count per stage is kept at the minimum the bytes need.
template <class C, class V>
__device__ __forceinline__ void issue_piece(const TileJob &t, const DmaLane &d, int k, uint8_t *buf, int wave,
                                            int q) {
  constexpr bool kGather = V::kGather;
  const uint32_t kbyte = (uint32_t)k * kBK;
  const int l = wave - C::kFirstLoader;  // loader index
  if (q < C::kPiecesB) {
    const int piece = l * C::kPiecesB + q;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(piece_rsrc<V::kBRow>(t.b_q, t.n_valid, t.K, piece, kbyte),
                                             (lds_void_t *)(buf + piece * 1024), 16, d.rc[piece & 1], 0, 0, 0);
  } else {
    const int piece = l * C::kPiecesA + (q - C::kPiecesB);
    if constexpr (kGather)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(gather_rsrc(t.a_q, t.T, t.K, kbyte),
                                               (lds_void_t *)(buf + C::kOffA + piece * 1024), 16,
                                               d.ga[q - C::kPiecesB], 0, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(piece_rsrc<V::kBRow>(t.a_q, t.m_valid, t.K, piece, kbyte),
                                               (lds_void_t *)(buf + C::kOffA + piece * 1024), 16, d.rc[piece & 1],
                                               0, 0, 0);
  }
}

// Quarter q of scale chunk c (per-row variant): loader l's activation-scale
// instruction (loaders 0 .. kScaleLoaders-1, instruction q*kScaleLoaders + l)
// and its per-row weight-side one (instruction 4q + j on loader
// (kScaleLoaders + j) % kLoaders), into chunk buffer c % 2 after lds.
template <class C, class V>
__device__ __forceinline__ void issue_chunk_quarter(const TileRsrc &rs, int KB, uint8_t *lds, int c, int q, int l) {
  static_assert(kBN / 64 <= C::kLoaders, "one weight-side chunk load per loader and stage");
  uint8_t *cb = lds + C::kOffChunk + (c & 1) * C::kChunkBytes;
  const uint32_t kb = (uint32_t)c * 16u;  // bytes of blocks 0 .. 4c-1 in a scale row
  if (l < C::kScaleLoaders) {
    const int i = q * C::kScaleLoaders + l;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs.sa, (lds_void_t *)(cb + i * 256), 4,
                                             chunk_lane_off<sa_chunk_row>(i, KB) + kb, 0, 0, 0);
  }
  const int j = (l - C::kScaleLoaders + C::kLoaders) % C::kLoaders;
  if (j < kBN / 64) {
    const int i = q * 4 + j;
    constexpr auto kRowB = !V::kPow2 ? sbf_chunk_row : (C::kWaveN == 128 ? sbp_chunk_row : sbp64_chunk_row);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs.sb, (lds_void_t *)(cb + C::kChunkSA + i * 256), 4,
                                             chunk_lane_off<kRowB>(i, KB) + kb, 0, 0, 0);
  }
}

// The scale loads of the stage of block k (buf: its stage buffer): one
// 64-lane activation-scale load on each of the first kScaleLoaders loaders
// and the weight tile's two block scales (lanes 0..1 of loader 0); with
// per-row weight-side scales, the chunk quarter the stage carries (first:
// block 0's stage, all of chunk 0; a literal at every call, so the branch
// folds away once inlined).
template <class C, class V>
__device__ __forceinline__ void issue_scales(const TileJob &t, const TileRsrc &rs, const DmaLane &d, int k,
                                             uint8_t *buf, int wave, int lane, bool first) {
  const int l = wave - C::kFirstLoader;
  if constexpr (V::kBRow) {
    uint8_t *lds = buf - (k & 1) * C::kStageBytes;  // block k's stage is buffer k % 2
    if (first) {
#pragma unroll
      for (int q = 0; q < kScChunk; ++q) issue_chunk_quarter<C, V>(rs, t.KB, lds, 0, q, l);
    } else {
      issue_chunk_quarter<C, V>(rs, t.KB, lds, chunk_of_stage(k), quarter_of_stage(k), l);
    }
  } else {
    if (l < C::kScaleLoaders)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs.sa, (lds_void_t *)(buf + C::kOffSA + l * 256), 4,
                                               (V::kGather ? d.gsa : d.sa) + (uint32_t)k * 4u, 0, 0, 0);
    if (l == 0 && lane < 2)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs.sb, (lds_void_t *)(buf + C::kOffSB), 4, d.sb + (uint32_t)k * 4u,
                                               0, 0, 0);
  }
}

// The DMA of block k's stage (first: block 0's, issued before the main loop).
template <class C, class V>
__device__ __forceinline__ void issue_stage(const TileJob &t, const TileRsrc &rs, const DmaLane &d, int k,
                                            uint8_t *buf, int wave, int lane, bool first) {
  issue_scales<C, V>(t, rs, d, k, buf, wave, lane, first);
#pragma unroll
  for (int q = 0; q < C::kPieces; ++q) issue_piece<C, V>(t, d, k, buf, wave, q);
}

// The DMA of a stage that the next block issues, right after its first LDS
// reads (so those are not queued behind it).
struct StageDma {
  const TileJob *t;
  const TileRsrc *rs;
  const DmaLane *d;
  int k;
  uint8_t *buf;
  int wave, lane;
  bool on;
};

// MFMA operand of a 16-row sub-tile: lane l supplies row (l % 16), bytes
// [32*(l/16), 32*(l/16) + 32) of the 128-byte K block.  A and B operands use
// the same (lane, byte) -> k assignment, so the contraction covers each k once.
__device__ __forceinline__ v8i frag(const uint8_t *lds, int row0, int lane) {
  const int r = row0 + (lane & 15);
  const int g = lane >> 4;
  const uint4 a = *reinterpret_cast<const uint4 *>(lds + lds_off(r, 2 * g));
  const uint4 b = *reinterpret_cast<const uint4 *>(lds + lds_off(r, 2 * g + 1));
  v8i f;
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  return f;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 h2 __attribute__((ext_vector_type(2)));
  const f2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2));  // RNE
}

// Fragments of one K block that a wave keeps in registers: the four token
// sub-tiles (B operands), the first weight sub-tile (A operand) and the four
// combined scales a_s[row] * b_s of this lane's token rows.
constexpr int kMaxWAhead = 3;  // weight sub-tiles read ahead of their MFMAs, at most

struct BlockFrags {
  v8i xf[kSubM];
  v8i wf[kMaxWAhead];  // the block's first weight sub-tiles (TileCfg::kWAhead of them)
  float scl[kSubM];
  // power-of-two scales: E8M0 exponent bytes (token rows mi = 0..3 in byte mi;
  // the weight block's), and which of them (bit mi; bit 4: the weight
  // block's) was, in some K block so far, not a power of two in [2^-127, 2^127]
  uint32_t ea, eb;
  // per-row power-of-two weight-side scales: this lane's row of sub-tile ni
  // in byte ni%4 of ebr[ni/4]; a bad one sets bit 16+ni of bad
  uint32_t ebr[2];
  uint32_t bad;
};

// E8M0 byte of a power-of-two fp32 scale 2^(e-127), 0 <= e <= 254: the
// exponent field for 2^-126 .. 2^127, and 0 for 2^-127 (the fp32 subnormal
// 0x00400000).  Sets `bit` in bad for anything else (a mantissa, a sign, zero,
// a smaller subnormal, infinity or NaN).
__device__ __forceinline__ uint32_t e8m0_of(float s, uint32_t &bad, uint32_t bit) {
  const uint32_t u = __float_as_uint(s);
  const uint32_t e = u >> 23;  // sign bit included: must be 0
  if (u == 0x00400000u) return 0u;
  if ((u & 0x7FFFFFu) != 0u || e == 0u || e >= 255u) bad |= bit;
  return e & 0xFFu;
}

// The raw scale words of a K block as read from LDS: the lane's four token
// rows' scales and the weight-side scale(s).
struct HeadRaw {
  float4 sa4;
  float sb;
  float4 lo, hi;  // per-row power-of-two weight-side scales (kPow2 && kBRow)
};

// Everything of a K block's fragments except the token sub-tiles, in two
// steps: the LDS reads (first weight sub-tile, scale words), then the scale
// arithmetic (combined per-lane scales, or E8M0 bytes), which can wait until
// the reads have landed without holding up other work.
// buf: block k's stage buffer; lds, k: where the per-row variant finds the
// block's scales (its chunk buffer).
template <class C, class V>
__device__ __forceinline__ void read_head(const uint8_t *buf, const uint8_t *lds, int k, int wn, int wm, int lane,
                                          BlockFrags &f, HeadRaw &h) {
#pragma unroll
  for (int a = 0; a < C::kWAhead; ++a) f.wf[a] = frag(buf, wn * C::kWaveN + a * 16, lane);
  if constexpr (V::kBRow)
    h.sa4 = *sa_chunk_ptr<C>(lds, k, wm, lane);
  else
    h.sa4 = *reinterpret_cast<const float4 *>(buf + C::kOffSA + (wm * 64 + (lane & 15) * 4) * 4);
  if constexpr (V::kPow2 && V::kBRow) {
    const float4 *rp = sbp_chunk_ptr<C>(lds, k, wn, lane);
    h.lo = rp[0];
    h.hi = C::kWaveN == 128 ? rp[1] : rp[0];  // 64-row waves: four rows (the copy sets no other row's bit)
  } else if constexpr (!V::kBRow) {
    h.sb = *reinterpret_cast<const float *>(buf + C::kOffSB + ((wn * C::kWaveN) >> 7) * 4);  // the wave's 128-row block
  }
}

template <class V>
__device__ __forceinline__ void finish_head(const HeadRaw &h, BlockFrags &f) {
  const float4 sa4 = h.sa4;
  if constexpr (V::kPow2) {
    f.ea = e8m0_of(sa4.x, f.bad, 1u) | (e8m0_of(sa4.y, f.bad, 2u) << 8) | (e8m0_of(sa4.z, f.bad, 4u) << 16) |
           (e8m0_of(sa4.w, f.bad, 8u) << 24);
    if constexpr (V::kBRow) {
      f.ebr[0] = e8m0_of(h.lo.x, f.bad, 1u << 16) | (e8m0_of(h.lo.y, f.bad, 1u << 17) << 8) |
                 (e8m0_of(h.lo.z, f.bad, 1u << 18) << 16) | (e8m0_of(h.lo.w, f.bad, 1u << 19) << 24);
      f.ebr[1] = e8m0_of(h.hi.x, f.bad, 1u << 20) | (e8m0_of(h.hi.y, f.bad, 1u << 21) << 8) |
                 (e8m0_of(h.hi.z, f.bad, 1u << 22) << 16) | (e8m0_of(h.hi.w, f.bad, 1u << 23) << 24);
    } else {
      f.eb = e8m0_of(h.sb, f.bad, 16u);
    }
  } else if constexpr (V::kBRow) {
    // the weight-side scale differs between a lane's four outputs: the folds
    // multiply it in
    f.scl[0] = sa4.x;
    f.scl[1] = sa4.y;
    f.scl[2] = sa4.z;
    f.scl[3] = sa4.w;
  } else {
    f.scl[0] = sa4.x * h.sb;
    f.scl[1] = sa4.y * h.sb;
    f.scl[2] = sa4.z * h.sb;
    f.scl[3] = sa4.w * h.sb;
  }
}

// Block 0's fragments and scales (its stage is buffer 0, at the LDS base).
template <class C, class V>
__device__ __forceinline__ void load_block(const uint8_t *buf, int wave, int wn, int wm, int lane,
                                           BlockFrags &f) {
  HeadRaw h;
  read_head<C, V>(buf, buf, 0, wn, wm, lane, f, h);
#pragma unroll
  for (int mi = 0; mi < kSubM; ++mi) f.xf[mi] = frag(buf + C::kOffA, wm * 64 + mi * 16, lane);
  finish_head<V>(h, f);
}

// Scheduling masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;

// The 32 MFMAs of one K block, j = 4*ni + mi (sub-tile row ni, column mi).
// Before row ni the LDS reads of weight sub-tile ni+1 are issued; after MFMA j
// the scale fold of MFMA j-2 follows, whose result is two MFMAs old.  The
// partial products live in a ring of three.  The folds of j = 30, 31 are left
// to the caller, which issues them after requesting the next block's
// fragments so that the LDS latency at the block boundary overlaps FMAs.
constexpr int kRing = 3;

// acc + A*B with the E8M0 scale eb on every row of A (one weight block) and,
// on column j of B, byte `sel` of the lane's ea (its token row's exponent).
template <int kSel>
__device__ __forceinline__ v4f mfma_pow2_sel(const v8i &a, const v8i &b, const v4f &c, uint32_t eb, uint32_t ea) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, (int)eb, kSel, (int)ea);
}

// acc + A*B with per-row E8M0 scales on A as well: byte selA of the lane's
// eb is the scale of the A row it supplies.
template <int kSelA, int kSelB>
__device__ __forceinline__ v4f mfma_pow2_ab(const v8i &a, const v8i &b, const v4f &c, uint32_t eb, uint32_t ea) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, kSelA, (int)eb, kSelB, (int)ea);
}

template <int kSelA>
__device__ __forceinline__ v4f mfma_pow2_rows(const v8i &a, const v8i &b, const v4f &c, uint32_t eb, uint32_t ea,
                                              int selb) {
  switch (selb) {
    case 0: return mfma_pow2_ab<kSelA, 0>(a, b, c, eb, ea);
    case 1: return mfma_pow2_ab<kSelA, 1>(a, b, c, eb, ea);
    case 2: return mfma_pow2_ab<kSelA, 2>(a, b, c, eb, ea);
    default: return mfma_pow2_ab<kSelA, 3>(a, b, c, eb, ea);
  }
}

__device__ __forceinline__ v4f mfma_pow2(const v8i &a, const v8i &b, const v4f &c, uint32_t eb, uint32_t ea,
                                         int sel) {
  switch (sel) {
    case 0: return mfma_pow2_sel<0>(a, b, c, eb, ea);
    case 1: return mfma_pow2_sel<1>(a, b, c, eb, ea);
    case 2: return mfma_pow2_sel<2>(a, b, c, eb, ea);
    default: return mfma_pow2_sel<3>(a, b, c, eb, ea);
  }
}

__device__ __forceinline__ void fold1(v4f &acc, const v4f &p, float s) {
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(p[r], s, acc[r]);
}

// The fold with per-row weight-side scales: a lane's four outputs are four
// weight-side rows, each with its own scale sb.
__device__ __forceinline__ void fold_rows(v4f &acc, const v4f &p, float sa, const float4 &sb) {
  acc[0] = __builtin_fmaf(p[0], sa * sb.x, acc[0]);
  acc[1] = __builtin_fmaf(p[1], sa * sb.y, acc[1]);
  acc[2] = __builtin_fmaf(p[2], sa * sb.z, acc[2]);
  acc[3] = __builtin_fmaf(p[3], sa * sb.w, acc[3]);
}

// Keeps a value's computation above this point: without it the compiler may
// sink the MFMAs and folds of a block past the block-boundary branch, away
// from the schedule laid out here.
__device__ __forceinline__ void pin(v4f &v) { asm volatile("" : "+v"(v)); }

//
// With power-of-two scales (kPow2) the matrix core applies them itself: the
// E8M0 scale operands of each MFMA carry the weight block's and the token
// row's exponents, and the MFMA accumulates straight into acc -- no partial
// products and no folds.
//
// With per-row weight-side scales (kBRow) the four scales of sub-tile row ni
// are read with its weight fragment (a ring of two rows, as a fold trails its
// MFMA by two) and each fold multiplies them in.
//
// Only MFMAs j < kJEnd are issued here.  With kJEnd = 28 the last row's weight
// fragment comes back in wlast and its four MFMAs are left to block_boundary,
// which issues them after the barrier, between the LDS reads of the next
// block's token fragments.
template <class C, class V, int kJEnd>
__device__ __forceinline__ void mma_steps(const uint8_t *tb, const uint8_t *lds, int k, int wn, int lane,
                                          const BlockFrags &f, v4f (&acc)[kSubN][kSubM], v4f (&p)[kRing],
                                          float4 (&sbq)[2], const StageDma &dma, v8i &wlast) {
  constexpr bool kPow2 = V::kPow2;
  // per-row weight-side scales on 256-row tiles: power-of-two step 4 (2%
  // ahead of 3); VALU-folded step 2 (at step 3 the compiler spilled four
  // registers in the loop; step 2 is 1-6% faster)
  constexpr int kDmaStep = (V::kBRow && C::kBM == 256) ? (kPow2 ? 4 : 2) : C::kDmaStep;
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  constexpr int kWAhead = C::kWAhead;
  static_assert(kWAhead >= 1 && kWAhead <= kMaxWAhead, "weight read-ahead");
  constexpr int R = kWAhead + 1;
  v8i wf[R];
#pragma unroll
  for (int a = 0; a < kWAhead; ++a) wf[a] = f.wf[a];
#pragma unroll
  for (int j = 0; j < kJEnd; ++j) {
    const int ni = j / kSubM, mi = j % kSubM;
    if (mi == 0) {
      // the reads of sub-tile ni+kWAhead go out before any MFMA of row ni
      __builtin_amdgcn_sched_barrier(0);
      if (ni + kWAhead < C::kSubN) wf[(ni + kWAhead) % R] = frag(tb, wn * C::kWaveN + (ni + kWAhead) * 16, lane);
      if constexpr (V::kBRow)
        sbq[ni & 1] = *sbf_chunk_ptr<C>(lds, k, wn, ni, lane);
      if (ni == kDmaStep && dma.on && dma.wave >= C::kFirstLoader)
        issue_stage<C, V>(*dma.t, *dma.rs, *dma.d, dma.k, dma.buf, dma.wave, dma.lane, false);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kPow2) {
      if constexpr (V::kBRow) {
        const uint32_t eb = f.ebr[ni >> 2];
        switch (ni & 3) {
          case 0: acc[ni][mi] = mfma_pow2_rows<0>(wf[ni % R], f.xf[mi], acc[ni][mi], eb, f.ea, mi); break;
          case 1: acc[ni][mi] = mfma_pow2_rows<1>(wf[ni % R], f.xf[mi], acc[ni][mi], eb, f.ea, mi); break;
          case 2: acc[ni][mi] = mfma_pow2_rows<2>(wf[ni % R], f.xf[mi], acc[ni][mi], eb, f.ea, mi); break;
          default: acc[ni][mi] = mfma_pow2_rows<3>(wf[ni % R], f.xf[mi], acc[ni][mi], eb, f.ea, mi); break;
        }
      } else {
        acc[ni][mi] = mfma_pow2(wf[ni % R], f.xf[mi], acc[ni][mi], f.eb, f.ea, mi);
      }
      continue;
    }
    p[j % kRing] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[ni % R], f.xf[mi], zero, 0, 0, 0, 127, 0,
                                                                     127);
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    if (j >= 2) {
      const int jj = j - 2;
      if constexpr (V::kBRow) {
        fold_rows(acc[jj / kSubM][jj % kSubM], p[jj % kRing], f.scl[jj % kSubM], sbq[(jj / kSubM) & 1]);
        __builtin_amdgcn_sched_group_barrier(kSchedValu, 8, 0);
      } else {
        fold1(acc[jj / kSubM][jj % kSubM], p[jj % kRing], f.scl[jj % kSubM]);
        __builtin_amdgcn_sched_group_barrier(kSchedValu, 4, 0);
      }
    }
  }
  if constexpr (V::kBRow && !kPow2 && kJEnd < C::kMfma) {
    // the row scales of the deferred last row (its slot's previous row has
    // had all its folds by now)
    constexpr int ni = kJEnd / kSubM;
    sbq[ni & 1] = *sbf_chunk_ptr<C>(lds, k, wn, ni, lane);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ni = 0; ni < C::kSubN; ++ni)
#pragma unroll
    for (int mi = 0; mi < kSubM; ++mi) pin(acc[ni][mi]);
#pragma unroll
  for (int r = 0; r < kRing; ++r) pin(p[r]);
  wlast = wf[(C::kSubN - 1) % R];
}

// The MFMA of sub-tile (ni, mi) = j with the block's scales: straight into
// acc (power-of-two scales), or into the partial-product ring.
template <class V>
__device__ __forceinline__ void mma_one(int ni, int mi, int j, const v8i &w, const BlockFrags &f,
                                        v4f (&acc)[kSubN][kSubM], v4f (&p)[kRing]) {
  if constexpr (V::kPow2) {
    if constexpr (V::kBRow) {
      const uint32_t eb = f.ebr[ni >> 2];
      switch (ni & 3) {
        case 0: acc[ni][mi] = mfma_pow2_rows<0>(w, f.xf[mi], acc[ni][mi], eb, f.ea, mi); break;
        case 1: acc[ni][mi] = mfma_pow2_rows<1>(w, f.xf[mi], acc[ni][mi], eb, f.ea, mi); break;
        case 2: acc[ni][mi] = mfma_pow2_rows<2>(w, f.xf[mi], acc[ni][mi], eb, f.ea, mi); break;
        default: acc[ni][mi] = mfma_pow2_rows<3>(w, f.xf[mi], acc[ni][mi], eb, f.ea, mi); break;
      }
    } else {
      acc[ni][mi] = mfma_pow2(w, f.xf[mi], acc[ni][mi], f.eb, f.ea, mi);
    }
  } else {
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    p[j % kRing] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, f.xf[mi], zero, 0, 0, 0, 127, 0, 127);
  }
}

// The scale fold of partial product jj.
template <class V>
__device__ __forceinline__ void fold_one(int jj, const float (&scl)[kSubM], v4f (&acc)[kSubN][kSubM],
                                         const v4f (&p)[kRing], const float4 (&sbq)[2]) {
  if constexpr (V::kBRow)
    fold_rows(acc[jj / kSubM][jj % kSubM], p[jj % kRing], scl[jj % kSubM], sbq[(jj / kSubM) & 1]);
  else
    fold1(acc[jj / kSubM][jj % kSubM], p[jj % kRing], scl[jj % kSubM]);
}

constexpr int kSchedDsRead = 0x100;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without a memory fence.  The only LDS writes are the DMA
// stages, whose completion each wave establishes with wait_vmcnt before it
// arrives; every LDS read of a buffer is consumed (lgkmcnt-waited) before the
// wave arrives at the barrier that allows the buffer to be refilled.  A fenced
// __syncthreads() would also wait for the DMA of the blocks still in flight.
__device__ __forceinline__ void barrier_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until the DMA of block kk has landed in every wave's view, then meet
// at the barrier.  With two stages nothing later than block kk has been
// issued when a wave arrives here, so the wait is for all of its loads.
__device__ __forceinline__ void wait_block() {
  wait_vmcnt<0>();
  barrier_nofence();
}

// The end of K block k and the start of block k+1, software-pipelined across
// the barrier: the four MFMAs of block k's last weight row (operands already
// in registers) are issued after the barrier, each followed by the LDS reads
// of one of block k+1's token sub-tiles, so the matrix core has work while
// those reads are in flight instead of idling until they land.  Every LDS
// read of block k has landed before this wave arrives at the barrier (after
// which the DMA of block k+2 may overwrite block k's buffer).
template <class C, class V>
__device__ __forceinline__ void block_boundary(const uint8_t *nbuf, const uint8_t *lds, int knext, int KB, int wave,
                                               int wn, int wm, int lane, BlockFrags &f, const v8i &wlast,
                                               v4f (&acc)[kSubN][kSubM], v4f (&p)[kRing], const float4 (&sbq)[2]) {
  constexpr bool kPow2 = V::kPow2;
  constexpr int ni = C::kSubN - 1;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  wait_block();
  __builtin_amdgcn_sched_barrier(0);
  BlockFrags g;
  g.bad = f.bad;
  HeadRaw h;
  read_head<C, V>(nbuf, lds, knext, wn, wm, lane, g, h);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int mi = 0; mi < kSubM; ++mi) {
    const int j = C::kMfma - kSubM + mi;
    mma_one<V>(ni, mi, j, wlast, f, acc, p);
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    if constexpr (!kPow2) {
      fold_one<V>(j - 2, f.scl, acc, p, sbq);
      __builtin_amdgcn_sched_group_barrier(kSchedValu, V::kBRow ? 8 : 4, 0);
    }
    g.xf[mi] = frag(nbuf + C::kOffA, wm * 64 + mi * 16, lane);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
  }
  if constexpr (!kPow2) {
    fold_one<V>(C::kMfma - 2, f.scl, acc, p, sbq);
    fold_one<V>(C::kMfma - 1, f.scl, acc, p, sbq);
  }
  finish_head<V>(h, g);
  __builtin_amdgcn_sched_barrier(0);
  f = g;
}

struct TileOut {
  uint16_t *y;   // bf16: tile origin of Y [M][N]
  uint8_t *yq;   // E4M3: tile origin of Yq [M][N]
  float *ys;     // E4M3: tile origin of the scales [M][N/128]
};

// ---------------------------------------------------------------------------
// Ping-pong main loop of the 256 x 256 tile (8 waves, two stage buffers).
//
// The eight waves form two groups, waves 0-3 and waves 4-7; a CU places wave
// w and wave w+4 on the same SIMD (checked on the hardware), so every SIMD
// holds one wave of each group.  A K block is cut into two halves along the
// wave's weight rows (sub-tile rows 0-3 and 4-7), and the work runs in
// phases separated by workgroup barriers.  In each phase one group computes
// a half (16 MFMAs and their scale folds, operands already in registers)
// while the other reads the fragments of its next half from LDS and issues
// its share of the DMA.  So the matrix core of every SIMD always has one
// wave feeding it, and the LDS reads and DMA of a block spread over the
// whole block instead of meeting at its start.
//
//   phase 4k-1: group 0 reads (k,0) and issues the weight tile of k+1
//   phase 4k  : group 0 computes (k,0); group 1 reads (k,0) and issues the
//               token tile of k+1
//   phase 4k+1: group 0 reads (k,1);    group 1 computes (k,0)
//   phase 4k+2: group 0 computes (k,1); group 1 reads (k,1); both wait for
//               their DMA of block k+1 before the barrier
//   phase 4k+3: group 0 reads (k+1,0);  group 1 computes (k,1)
//
// Block k's stage buffer is read in phases 4k-1 .. 4k+2; block k+2 goes into
// it from phase 4k+3 on (the barrier ending 4k+2 orders every read before
// that DMA) and is first read in phase 4k+7, so its DMA has a whole K block
// of time.  The last two scale folds of a compute phase are left to the
// wave's next (read) phase, when its VALU is otherwise idle.
// ---------------------------------------------------------------------------
constexpr int kPPPieces = 8;  // 1 KB DMA pieces per wave and operand tile

// Per-lane DMA offsets.  Group 0 loads the weight tile (wave l: pieces
// 8l .. 8l+7) and the two weight-block scales; group 1 the token tile and 64
// activation scales per wave.
struct PPLane {
  uint32_t rc[2];               // (row in piece)*K + chunk offset, even / odd pieces
  uint32_t s;                   // scale offset
  uint32_t ga[kPPPieces];       // gathered token rows: byte offset of this lane's row per piece
};

template <class V>
__device__ __forceinline__ PPLane pp_lane(const TileJob &t, int grp, int l, int lane) {
  PPLane d;
  const uint32_t row = (uint32_t)(lane >> 3);
  const uint32_t c0 = (uint32_t)((lane & 7) ^ (lane >> 3));
  const uint32_t K = (uint32_t)t.K;
#pragma unroll
  for (int par = 0; par < 2; ++par) d.rc[par] = row * K + ((c0 ^ par) << 4);
  if (grp == 0) {
    d.s = (uint32_t)(lane & 1) * (uint32_t)t.KB * 4u;
  } else {
    const int srow = sa_row_of_pos(l * 64 + lane);
    d.s = (uint32_t)srow * (uint32_t)t.KB * 4u;
    if constexpr (V::kGather) {
      auto src = [&](int r) -> int64_t {  // source token row of tile row r, or -1
        if (r >= t.m_valid) return -1;
        const int64_t s = t.gidx[r];
        return (s >= 0 && s < t.T) ? s : -1;
      };
#pragma unroll
      for (int i = 0; i < kPPPieces; ++i) {
        const int piece = l * kPPPieces + i;
        const int64_t s = src(8 * piece + (int)row);
        d.ga[i] = s < 0 ? kGatherOOB : (uint32_t)s * K + ((c0 ^ (uint32_t)(piece & 1)) << 4);
      }
      const int64_t s = src(srow);
      d.s = s < 0 ? kGatherOOB : (uint32_t)s * (uint32_t)t.KB * 4u;
    }
  }
  return d;
}

// Resource over the 64 rows (8 pieces) a wave loads of an operand tile: based
// at row 64l and byte kbyte of the row, bounded to the valid rows among them
// (0..64).  A lane's offset inside it, (8q + row) * K + chunk, is below the
// bound exactly when its row is valid, so rows past the tile's last valid
// one read zeros and no access leaves the tensor.  Wave-uniform, so it lives
// in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_rsrc(const uint8_t *rows, int valid_rows, int64_t K, int l,
                                                             uint32_t kbyte) {
  int nr = valid_rows - 64 * l;
  nr = nr < 0 ? 0 : (nr > 64 ? 64 : nr);
  const uint64_t base = (uint64_t)(uintptr_t)(rows + (int64_t)(64 * l) * K + kbyte);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
  const int n = __builtin_amdgcn_readfirstlane(nr * (int)K);
  return __builtin_amdgcn_make_buffer_rsrc((void *)(uintptr_t)(((uint64_t)hi << 32) | lo), (short)0, n, kRsrcWord3);
}

// Pieces [kQ0, kQ1) of this wave's share of block k's DMA into stage buffer
// buf, and (kScales) its scale load.
template <class C, class V, int kQ0, int kQ1, bool kScales>
__device__ __forceinline__ void pp_issue(const TileJob &t, const TileRsrc &rs, const PPLane &d, int k, uint8_t *buf,
                                         int grp, int l, int lane) {
  const uint32_t kbyte = (uint32_t)k * kBK;
  const uint32_t K8 = (uint32_t)t.K * 8u;
  if (grp == 0) {
    const __amdgpu_buffer_rsrc_t r = wave_rsrc(t.b_q, t.n_valid, t.K, l, kbyte);
#pragma unroll
    for (int q = kQ0; q < kQ1; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)(buf + (l * kPPPieces + q) * 1024), 16,
                                               d.rc[q & 1] + (uint32_t)q * K8, 0, 0, 0);
    if (kScales && l == 0 && lane < 2)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs.sb, (lds_void_t *)(buf + C::kOffSB), 4, d.s + (uint32_t)k * 4u,
                                               0, 0, 0);
  } else {
    if constexpr (V::kGather) {
      const __amdgpu_buffer_rsrc_t r = gather_rsrc(t.a_q, t.T, t.K, kbyte);
#pragma unroll
      for (int q = kQ0; q < kQ1; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)(buf + C::kOffA + (l * kPPPieces + q) * 1024), 16,
                                                 d.ga[q], 0, 0, 0);
    } else {
      const __amdgpu_buffer_rsrc_t r = wave_rsrc(t.a_q, t.m_valid, t.K, l, kbyte);
#pragma unroll
      for (int q = kQ0; q < kQ1; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)(buf + C::kOffA + (l * kPPPieces + q) * 1024), 16,
                                                 d.rc[q & 1] + (uint32_t)q * K8, 0, 0, 0);
    }
    if (kScales)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs.sa, (lds_void_t *)(buf + C::kOffSA + l * 256), 4,
                                               d.s + (uint32_t)k * 4u, 0, 0, 0);
  }
}

// The 16 MFMAs of half kH of a K block (weight sub-tile rows 4kH .. 4kH+3,
// all four token sub-tiles), j = 4*(ni - 4kH) + mi.  amax scales: after
// MFMA j the fold of MFMA j-2; the folds of j = 14 and 15 are left to
// pp_fold_tail.  Power-of-two scales: the MFMA applies them and accumulates.
template <class V, int kH>
__device__ __forceinline__ void pp_compute(const v8i (&wf)[4], const v8i (&xf)[kSubM], const float (&scl)[kSubM],
                                           uint32_t ea, uint32_t eb, v4f (&acc)[kSubN][kSubM], v4f (&p)[kRing]) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int ni = j / kSubM, mi = j % kSubM;
    if constexpr (V::kPow2) {
      acc[4 * kH + ni][mi] = mfma_pow2(wf[ni], xf[mi], acc[4 * kH + ni][mi], eb, ea, mi);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    } else {
      // MFMA j, then the fold of MFMA j-2, step by step.  Left to itself the
      // compiler clumps the MFMAs and leaves the folds to the end of the
      // phase (or pairs each MFMA with the fold of its own result, which
      // stalls the wave until the MFMA completes).  Two empty asm statements
      // fix the order: MFMA j takes its zero accumulator through one, so it
      // cannot rise above step j-1, and the fold's result passes through the
      // other, so it cannot sink below step j+1.  Two MFMAs after its MFMA a
      // fold's product is ready, and its four FMAs run while MFMA j does.
      v4f z = zero;
      asm volatile("" : "+v"(z));
      p[j % kRing] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[ni], xf[mi], z, 0, 0, 0, 127, 0, 127);
      if (j >= 2) {
        const int jj = j - 2;
        v4f &a = acc[4 * kH + jj / kSubM][jj % kSubM];
        fold1(a, p[jj % kRing], scl[jj % kSubM]);
        asm volatile("" : "+v"(a));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// The two folds a compute phase of half kH left (MFMAs 14 and 15).
template <int kH>
__device__ __forceinline__ void pp_fold_tail(v4f (&acc)[kSubN][kSubM], const v4f (&p)[kRing],
                                             const float (&scl)[kSubM]) {
  fold1(acc[4 * kH + 3][2], p[14 % kRing], scl[2]);
  fold1(acc[4 * kH + 3][3], p[15 % kRing], scl[3]);
}

// Weight fragments of half kH: sub-tile rows 4kH .. 4kH+3 of this wave's 128.
__device__ __forceinline__ void pp_read_w(const uint8_t *buf, int wn, int h, int lane, v8i (&wf)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) wf[i] = frag(buf, wn * 128 + (4 * h + i) * 16, lane);
}

// Everything of a phase stays in its phase: the barrier is a fence for the
// scheduler, and the accumulators and partial products are pinned on both
// sides of it (register-only work could otherwise move across).
__device__ __forceinline__ void pp_barrier(v4f (&acc)[kSubN][kSubM], v4f (&p)[kRing]) {
#pragma unroll
  for (int ni = 0; ni < kSubN; ++ni)
#pragma unroll
    for (int mi = 0; mi < kSubM; ++mi) pin(acc[ni][mi]);
#pragma unroll
  for (int r = 0; r < kRing; ++r) pin(p[r]);
  __builtin_amdgcn_sched_barrier(0);
  barrier_nofence();
  __builtin_amdgcn_sched_barrier(0);
}

template <class C, class V>
__device__ __forceinline__ void gemm_main_pp(const TileJob &t, uint8_t *lds, int wave, int lane, int wn, int wm,
                                             v4f (&acc)[kSubN][kSubM], uint32_t &bad) {
  static_assert(C::kBM == 256 && C::kWaves == 8 && C::kWavesN == 2 && C::kStages == 2, "ping-pong tile shape");
  static_assert(!V::kBRow, "per-row weight-side scales: lockstep loop");
  constexpr bool kPow2 = V::kPow2;
  const int grp = wave >> 2, l = wave & 3;
  const int KB = t.KB;
  const TileRsrc rs = make_rsrc<V>(t);
  const PPLane d = pp_lane<V>(t, grp, l, lane);
  v8i xf[kSubM], wf[4];
  float scl[kSubM] = {0.0f, 0.0f, 0.0f, 0.0f};
  uint32_t ea = 0, eb = 0;
  v4f p[kRing];
#pragma unroll
  for (int r = 0; r < kRing; ++r) p[r] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

  // Block k+1's DMA goes out in three parts (pieces 0-2 with the scales, 3-5,
  // 6-7), spread over the phases between the end of the last read of its
  // stage buffer (block k-1's, phase 4k-2) and the wait before its first read
  // (end of phase 4k+2): group 0 in its phases 4k-1 .. 4k+1, group 1 in
  // 4k-1 .. 4k+1 as well (its part 0 in the previous iteration's last
  // segment).  So no phase carries more than a quarter of a block's DMA.
  auto part = [&](int which, int kk) {
    uint8_t *b = lds + (kk & 1) * C::kStageBytes;
    if (which == 0) pp_issue<C, V, 0, 3, true>(t, rs, d, kk, b, grp, l, lane);
    else if (which == 1) pp_issue<C, V, 3, 6, false>(t, rs, d, kk, b, grp, l, lane);
    else pp_issue<C, V, 6, kPPPieces, false>(t, rs, d, kk, b, grp, l, lane);
  };
  part(0, 0);
  part(1, 0);
  part(2, 0);
  wait_vmcnt<0>();
  pp_barrier(acc, p);
  if (grp == 1) {
    if (1 < KB) part(0, 1);
    pp_barrier(acc, p);  // phase -1: group 0 reads the first half of block 0
  }
  for (int k = 0; k < KB; ++k) {
    const uint8_t *buf = lds + (k & 1) * C::kStageBytes;
    const bool more = k + 1 < KB;
    // read (k, 0): token fragments, weight rows 0-3, scale words
    HeadRaw h;
#pragma unroll
    for (int mi = 0; mi < kSubM; ++mi) wf[mi] = frag(buf, wn * 128 + mi * 16, lane);
#pragma unroll
    for (int mi = 0; mi < kSubM; ++mi) xf[mi] = frag(buf + C::kOffA, wm * 64 + mi * 16, lane);
    h.sa4 = *reinterpret_cast<const float4 *>(buf + C::kOffSA + (wm * 64 + (lane & 15) * 4) * 4);
    h.sb = *reinterpret_cast<const float *>(buf + C::kOffSB + wn * 4);
    if (more) part(grp == 0 ? 0 : 1, k + 1);
    if constexpr (!kPow2)
      if (k > 0) pp_fold_tail<1>(acc, p, scl);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if constexpr (kPow2) {
      BlockFrags g;
      g.bad = bad;
      finish_head<V>(h, g);
      ea = g.ea;
      eb = g.eb;
      bad = g.bad;
    } else {
      scl[0] = h.sa4.x * h.sb;
      scl[1] = h.sa4.y * h.sb;
      scl[2] = h.sa4.z * h.sb;
      scl[3] = h.sa4.w * h.sb;
    }
    pp_barrier(acc, p);
    if (more) part(grp == 0 ? 1 : 2, k + 1);
    pp_compute<V, 0>(wf, xf, scl, ea, eb, acc, p);
    pp_barrier(acc, p);
    // read (k, 1): weight rows 4-7
    pp_read_w(buf, wn, 1, lane, wf);
    if (more && grp == 0) part(2, k + 1);
    if constexpr (!kPow2) pp_fold_tail<0>(acc, p, scl);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (grp == 1) wait_vmcnt<0>();
    pp_barrier(acc, p);
    if (grp == 1 && k + 2 < KB) part(0, k + 2);
    pp_compute<V, 1>(wf, xf, scl, ea, eb, acc, p);
    if (grp == 0) wait_vmcnt<0>();
    pp_barrier(acc, p);
  }
  if constexpr (!kPow2) pp_fold_tail<1>(acc, p, scl);
  if (grp == 0) pp_barrier(acc, p);  // the last phase: group 1 computes block KB-1's second half
}


// Four words per lane, one per sub-tile j = 0..3, where the lanes of 16-lane
// row g hold n-group g (4 codes) of each sub-tile: transposed across the rows
// (v_permlane32_swap then v_permlane16_swap, lane patterns checked on gfx950)
// so that row g holds the four n-groups of sub-tile g, 16 consecutive codes.
// Every lane must take part (cross-lane).
__device__ __forceinline__ uint4 rows_to_subtiles(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
  const auto s02 = __builtin_amdgcn_permlane32_swap(w0, w2, false, false);
  const auto s13 = __builtin_amdgcn_permlane32_swap(w1, w3, false, false);
  const auto t01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
  const auto t23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
  return (uint4){t01[0], t01[1], t23[0], t23[1]};
}

// E4M3 codes of a block's values held as bf16 pairs (h[i] = values 4i .. 4i+3
// of the lane) with its parameters, by the activation rule.  A block whose
// quotients cannot exceed 448 (1 + 2^-23) -- power-of-two scales, or amax
// scales on the fast path with a normal scale -- converts without the
// explicit clamp: the hardware conversion (round to nearest even) takes such
// values to 448 itself.  The choice is one branch, uniform over the wave.
template <int kOut, int kN>
__device__ __forceinline__ void block_codes(const BlockQ &bq, const uint32_t (&h)[kN][2], uint32_t (&cw)[kN]) {
  const bool plain = kOut == kModePow2 || (!bq.slow && bq.s >= 0x1p-126f);
  if (__builtin_amdgcn_ballot_w64(!plain) == 0) {
#pragma unroll
    for (int ni = 0; ni < kN; ++ni) {
      const float q0 = quotient<kOut>(bq, bf16_lo(h[ni][0])), q1 = quotient<kOut>(bq, bf16_hi(h[ni][0]));
      const float q2 = quotient<kOut>(bq, bf16_lo(h[ni][1])), q3 = quotient<kOut>(bq, bf16_hi(h[ni][1]));
      cw[ni] = __builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false), true);
    }
  } else {
#pragma unroll
    for (int ni = 0; ni < kN; ++ni) {
      const float x[4] = {bf16_lo(h[ni][0]), bf16_hi(h[ni][0]), bf16_lo(h[ni][1]), bf16_hi(h[ni][1])};
      float qv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        qv[i] = (kOut == kModeAmax && bq.slow) ? x[i] / bq.s : quotient<kOut>(bq, x[i]);
      cw[ni] = pack4_e4m3(qv[0], qv[1], qv[2], qv[3]);
    }
  }
}

// Quantized epilogue of the 128-row, 8-wave tile (the 128-row part of a
// single-launch tile plan): four waves along n with 64 weight rows each, so
// the 1x128 block of a row's columns 128b .. 128b+127 is held by waves 2b
// and 2b+1, one 64-column half each.  Each wave rounds its values to bf16
// and takes their |max| over its half; the two waves exchange the partial
// maxima through LDS, then quantize their halves with the block's scale.
// The codes and scales equal those of the 256-row tile's epilogue (and so
// of quantizing the bf16 output).
template <class C, class V>
__device__ __forceinline__ void quant_epilogue_half(const TileJob &t, const TileOut &o, int64_t N, uint8_t *lds,
                                                    v4f (&acc)[kSubN][kSubM], int wn, int wm, int lane) {
  static_assert(C::kWaveN == 64 && C::kSubN == 4 && C::kWavesN == 4, "128-row quantized tile layout");
  constexpr int kOut = V::kOut;
  float *ml = reinterpret_cast<float *>(lds);  // [4 waves along n][kBM rows] partial maxima
  const int half = wn & 1;
  const bool live = (wn >> 1) * 128 < t.n_valid;  // this block's columns exist (N is a multiple of 128)
  const int64_t nbo = N >> 7;  // scale blocks per output row
  uint32_t h[kSubM][C::kSubN][2];
  float amax[kSubM];
#pragma unroll
  for (int mi = 0; mi < kSubM; ++mi) {
    float m = 0.0f;
#pragma unroll
    for (int ni = 0; ni < C::kSubN; ++ni) {
      h[mi][ni][0] = pack_bf16x2(acc[ni][mi][0], acc[ni][mi][1]);
      h[mi][ni][1] = pack_bf16x2(acc[ni][mi][2], acc[ni][mi][3]);
      m = max3_abs(m, bf16_lo(h[mi][ni][0]), bf16_hi(h[mi][ni][0]));
      m = max3_abs(m, bf16_lo(h[mi][ni][1]), bf16_hi(h[mi][ni][1]));
    }
    m = __builtin_fmaxf(m, __shfl_xor(m, 16));
    amax[mi] = __builtin_fmaxf(m, __shfl_xor(m, 32));
  }
  __syncthreads();  // the stage buffers are free once every wave is past the main loop
#pragma unroll
  for (int mi = 0; mi < kSubM; ++mi)
    if ((lane >> 4) == 0) ml[wn * C::kBM + wm * 64 + mi * 16 + (lane & 15)] = amax[mi];
  __syncthreads();
  if (!live) return;
#pragma unroll
  for (int mi = 0; mi < kSubM; ++mi) {
    const int r = wm * 64 + mi * 16 + (lane & 15);
    const BlockQ bq = block_params<kOut>(__builtin_fmaxf(amax[mi], ml[(wn ^ 1) * C::kBM + r]));
    uint32_t cw[C::kSubN];
    block_codes<kOut>(bq, h[mi], cw);
    if (r < t.m_valid && half == 0 && (lane >> 4) == 0) o.ys[(int64_t)r * nbo + (wn >> 1)] = bq.s;
    const uint4 v = rows_to_subtiles(cw[0], cw[1], cw[2], cw[3]);
    if (r < t.m_valid) store_stream16(o.yq + (int64_t)r * N + wn * 64 + 16 * (lane >> 4), v);
  }
}

// SwiGLU epilogue of the 128-row, 8-wave tile (a group's ragged last slot in
// the grouped GEMM): four waves along n with 64 weight rows each, wn = 0, 1
// holding gate columns 0-63 and 64-127 of the tile's 128 features and
// wn = 2, 3 the up columns of the same features.  Gate wave wn (< 2) and up
// wave wn + 2 split their 64 token rows as the 256-row tile's epilogue does
// (gate rows 0-31, up rows 32-63, the other half's values through LDS); a
// row's 1x128 block is then held by two waves, one per 64-column half, which
// exchange their partial |max| through LDS before quantizing.  Each value of
// h, each block |max| and so each code equal the 256-row tile's.
template <class C, class V>
__device__ __forceinline__ void swiglu_epilogue_half(const TileJob &t, const TileOut &o, int64_t N, uint8_t *lds,
                                                     v4f (&acc)[kSubN][kSubM], int wn, int wm, int lane) {
  static_assert(C::kWaveN == 64 && C::kSubN == 4 && kSubM == 4 && C::kWavesN == 4, "128-row SwiGLU tile layout");
  constexpr int kOut = V::kOut;
  constexpr int kXStride = 66;  // 32-bit words per LDS row (64 + 2: rows fall in different banks)
  uint32_t *xl = reinterpret_cast<uint32_t *>(lds);
  float *ml = reinterpret_cast<float *>(lds + C::kBM * kXStride * 4);  // [2 halves][kBM rows] partial maxima
  __syncthreads();  // the stage buffers are free once every wave is past the main loop
  const int half = wn & 1;     // which 64 columns of each row's block
  const bool gate = wn < 2;
  const int64_t F = N >> 1;
  const int64_t nbo = F >> 7;
  // Branch-free on gate / up: the sub-tiles a wave hands over or keeps are
  // picked by value (v_cndmask between two register values), never by an
  // index computed from the wave kind, which would put the accumulators in
  // scratch memory.
  // Gate waves hand over g of sub-tiles 2, 3; up waves u of sub-tiles 0, 1.
#pragma unroll
  for (int mh = 0; mh < 2; ++mh) {
    const int r = wm * 64 + (gate ? 2 + mh : mh) * 16 + (lane & 15);
#pragma unroll
    for (int ni = 0; ni < C::kSubN; ++ni) {
      const int nn = half * 64 + ni * 16 + 4 * (lane >> 4);
      v4f lo = acc[ni][mh], hi = acc[ni][2 + mh];
      asm volatile("" : "+v"(lo), "+v"(hi));  // two values, then a select (not a computed index)
      const v4f a = gate ? hi : lo;
      uint2 w;
      w.x = pack_bf16x2(a[0], a[1]);
      w.y = pack_bf16x2(a[2], a[3]);
      *reinterpret_cast<uint2 *>(xl + r * kXStride + (nn >> 1)) = w;
    }
  }
  __syncthreads();
  // h of the kept sub-tiles (gate: 0, 1; up: 2, 3) for this wave's 64 columns
  uint32_t h[2][C::kSubN][2];
  float amax[2];
#pragma unroll
  for (int mh = 0; mh < 2; ++mh) {
    const int r = wm * 64 + (gate ? mh : 2 + mh) * 16 + (lane & 15);
    float m = 0.0f;
#pragma unroll
    for (int ni = 0; ni < C::kSubN; ++ni) {
      const int nn = half * 64 + ni * 16 + 4 * (lane >> 4);
      const uint2 xw = *reinterpret_cast<const uint2 *>(xl + r * kXStride + (nn >> 1));
      v4f lo = acc[ni][mh], hi = acc[ni][2 + mh];
      asm volatile("" : "+v"(lo), "+v"(hi));
      const v4f a = gate ? lo : hi;
      const uint32_t m01 = pack_bf16x2(a[0], a[1]);
      const uint32_t m23 = pack_bf16x2(a[2], a[3]);
      const float mine[4] = {bf16_lo(m01), bf16_hi(m01), bf16_lo(m23), bf16_hi(m23)};
      const float other[4] = {bf16_lo(xw.x), bf16_hi(xw.x), bf16_lo(xw.y), bf16_hi(xw.y)};
      float hv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float g = gate ? mine[i] : other[i], u = gate ? other[i] : mine[i];
        hv[i] = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
      }
      h[mh][ni][0] = pack_bf16x2(hv[0], hv[1]);
      h[mh][ni][1] = pack_bf16x2(hv[2], hv[3]);
      m = max3_abs(m, bf16_lo(h[mh][ni][0]), bf16_hi(h[mh][ni][0]));
      m = max3_abs(m, bf16_lo(h[mh][ni][1]), bf16_hi(h[mh][ni][1]));
    }
    m = __builtin_fmaxf(m, __shfl_xor(m, 16));
    m = __builtin_fmaxf(m, __shfl_xor(m, 32));
    amax[mh] = m;
    if ((lane >> 4) == 0) ml[half * C::kBM + r] = m;
  }
  __syncthreads();
  // the block's |max| from both halves, then this half's codes
#pragma unroll
  for (int mh = 0; mh < 2; ++mh) {
    const int r = wm * 64 + (gate ? mh : 2 + mh) * 16 + (lane & 15);
    const BlockQ bq = block_params<kOut>(__builtin_fmaxf(amax[mh], ml[(half ^ 1) * C::kBM + r]));
    uint32_t cw[C::kSubN];
    block_codes<kOut>(bq, h[mh], cw);
    if (r < t.m_valid && half == 0 && (lane >> 4) == 0) o.ys[(int64_t)r * nbo] = bq.s;
    const uint4 v = rows_to_subtiles(cw[0], cw[1], cw[2], cw[3]);
    if (r < t.m_valid) store_stream16(o.yq + (int64_t)r * F + half * 64 + 16 * (lane >> 4), v);
  }
}

// After the main loop: the power-of-two NaN rule, zero rows of invalid
// gathered indices, then the epilogue of the variant (bf16, quantized or
// SwiGLU output).  bad: the pow2 scale-check bits of this lane.
template <class C, class V>
__device__ __forceinline__ void tile_finish(const TileJob &t, const TileOut &o, int64_t N, uint8_t *lds,
                                            v4f (&acc)[kSubN][kSubM], uint32_t bad, int wave, int wn, int wm,
                                            int lane) {
  constexpr bool kPow2 = V::kPow2;
  constexpr int kOut = V::kOut;
  constexpr bool kGather = V::kGather;
  // A scale outside the power-of-two contract turns the outputs that depend
  // on it into NaN rather than into a silently wrong product.
  if constexpr (kPow2 && V::kBRow) {
    // A bad weight-side row scale is seen by the lanes that supply that row
    // (lane % 16 of its sub-tile); the row's outputs sit in other lanes
    // (rows 4*(lane/16) .. +3), so its bit is shared with a ballot.
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int ni = 0; ni < kSubN; ++ni) {
      const uint64_t rb = __ballot((bad >> (16 + ni)) & 1u);
      if (rb != 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if ((rb >> (4 * (lane >> 4) + r)) & 1u)
#pragma unroll
            for (int mi = 0; mi < kSubM; ++mi) acc[ni][mi][r] = nan;
      }
    }
#pragma unroll
    for (int mi = 0; mi < kSubM; ++mi)
      if (bad & (1u << mi))
#pragma unroll
        for (int ni = 0; ni < C::kSubN; ++ni) acc[ni][mi] = (v4f){nan, nan, nan, nan};
  } else if (kPow2 && bad) {
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int mi = 0; mi < kSubM; ++mi)
      if (bad & ((1u << mi) | 16u))
#pragma unroll
        for (int ni = 0; ni < C::kSubN; ++ni) acc[ni][mi] = (v4f){nan, nan, nan, nan};
  }
  if constexpr (kGather) {
    // A routed row whose token index is outside [0, T) read zeros; its output
    // is zero in both scale modes (the power-of-two check above sees its zero
    // scale and would have made it NaN).
#pragma unroll
    for (int mi = 0; mi < kSubM; ++mi) {
      const int r = wm * 64 + mi * 16 + (lane & 15);
      const int64_t s = r < t.m_valid ? (int64_t)t.gidx[r] : 0;
      if (!(s >= 0 && s < t.T))
#pragma unroll
        for (int ni = 0; ni < C::kSubN; ++ni) acc[ni][mi] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
    }
  }

  if constexpr (kOut == kOutBf16) {
    // Epilogue through LDS: each wave writes its [64 m][kWaveN n] bf16 (RNE)
    // block into its own region of the stage buffers (free once every wave is
    // past the barrier; 16-byte chunks XOR-swizzled by row, so the 16 rows a
    // write instruction touches fall in distinct banks), then stores whole
    // rows with 16-byte stores: half the store instructions of 8-byte quads,
    // and each group of 8 lanes writes one full 128-byte line.  Measured
    // against the quads: dense Llama shapes +2-4%, MoE grouped GEMMs 6-17%
    // less time.  The stores carry the non-temporal hint: the output is not
    // read again by this GEMM, and with plain stores a round of tiles leaves
    // ~33 MB of dirty lines in L2 that evict the operand panels the next
    // round reuses.  Measured: MoE down projections 7-24% less time (K = 768
    // and 1408, where the output is as large as the operands), Llama layers
    // unchanged.
    constexpr int kRowB = C::kWaveN * 2;
    constexpr int kChunks = kRowB / 16;
    __syncthreads();
    uint8_t *wl = lds + wave * (64 * kRowB);
#pragma unroll
    for (int mi = 0; mi < kSubM; ++mi) {
      const int r = mi * 16 + (lane & 15);
#pragma unroll
      for (int ni = 0; ni < C::kSubN; ++ni) {
        const int c = ni * 2 + ((lane >> 4) >> 1);
        const int pc = c ^ (r & (kChunks - 1));
        uint2 w;
        w.x = pack_bf16x2(acc[ni][mi][0], acc[ni][mi][1]);
        w.y = pack_bf16x2(acc[ni][mi][2], acc[ni][mi][3]);
        *reinterpret_cast<uint2 *>(wl + r * kRowB + pc * 16 + ((lane >> 4) & 1) * 8) = w;
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    uint16_t *__restrict__ y = o.y;
#pragma unroll
    for (int it = 0; it < kChunks; ++it) {
      const int flat = it * 64 + lane;
      const int r = flat / kChunks, c = flat % kChunks;
      const uint4 v = *reinterpret_cast<const uint4 *>(wl + r * kRowB + (c ^ (r & (kChunks - 1))) * 16);
      const int rr = wm * 64 + r, nn = wn * C::kWaveN + c * 8;
      if (rr < t.m_valid && nn < t.n_valid) store_stream16(y + (int64_t)rr * N + nn, v);
    }
  } else if constexpr (V::kSwiGLU && C::kWaveN == 64) {
    swiglu_epilogue_half<C, V>(t, o, N, lds, acc, wn, wm, lane);
  } else if constexpr (V::kSwiGLU) {
    static_assert(C::kWaveN == 128, "SwiGLU epilogue: a wave holds 128 gate or up rows");
    static_assert(kSubM == 4, "SwiGLU epilogue: 64 rows per wave, split in two halves");
    // SwiGLU epilogue of a fused gate+up projection: the tile's weight rows
    // are 128 gate rows (waves wn = 0) and the 128 up rows of the same output
    // columns (waves wn = 1).  gate and up are rounded to bf16 as the bf16
    // epilogue rounds them.  The two waves holding the same 64 token rows
    // split them: the gate wave forms h for rows 0-31 (m sub-tiles 0, 1) and
    // the up wave for rows 32-63 (sub-tiles 2, 3), each receiving the other
    // half's up (or gate) values through LDS (the stage buffers are free once
    // every wave is past the barrier), so all eight waves share the exponent
    // and quantization work.  h = silu(g) * u = g / (1 + e^-g) * u in fp32 is
    // rounded to bf16 and each row's 128 values quantized as one 1x128 block
    // (the activation rule), row r's block written at column 128*(n0/256).
    constexpr int kXStride = 66;  // 32-bit words per LDS row (64 + 2: rows fall in different banks)
    uint32_t *xl = reinterpret_cast<uint32_t *>(lds);
    const int64_t F = N >> 1;   // columns of h
    const int64_t nbo = F >> 7;  // scale blocks per row of h
    // gate waves hand over g of sub-tiles 2, 3; up waves u of sub-tiles 0, 1
    auto hand_over = [&](auto MI) __attribute__((always_inline)) {
      constexpr int mi = decltype(MI)::value;
      const int r = wm * 64 + mi * 16 + (lane & 15);
#pragma unroll
      for (int ni = 0; ni < kSubN; ++ni) {
        const int nn = ni * 16 + 4 * (lane >> 4);
        uint2 w;
        w.x = pack_bf16x2(acc[ni][mi][0], acc[ni][mi][1]);
        w.y = pack_bf16x2(acc[ni][mi][2], acc[ni][mi][3]);
        *reinterpret_cast<uint2 *>(xl + r * kXStride + (nn >> 1)) = w;
      }
    };
    // h, its block scale and codes for sub-tile mi (kGate: this wave holds g)
    auto rows_out = [&](auto MI, auto GATE) __attribute__((always_inline)) {
      constexpr int mi = decltype(MI)::value;
      constexpr bool kGate = decltype(GATE)::value;
      const int r = wm * 64 + mi * 16 + (lane & 15);
      uint32_t h[kSubN][2];
      float amax = 0.0f;
#pragma unroll
      for (int ni = 0; ni < kSubN; ++ni) {
        const int nn = ni * 16 + 4 * (lane >> 4);
        const uint2 xw = *reinterpret_cast<const uint2 *>(xl + r * kXStride + (nn >> 1));
        const uint32_t m01 = pack_bf16x2(acc[ni][mi][0], acc[ni][mi][1]);
        const uint32_t m23 = pack_bf16x2(acc[ni][mi][2], acc[ni][mi][3]);
        const float mine[4] = {bf16_lo(m01), bf16_hi(m01), bf16_lo(m23), bf16_hi(m23)};
        const float other[4] = {bf16_lo(xw.x), bf16_hi(xw.x), bf16_lo(xw.y), bf16_hi(xw.y)};
        float hv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float g = kGate ? mine[i] : other[i], u = kGate ? other[i] : mine[i];
          hv[i] = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
        }
        h[ni][0] = pack_bf16x2(hv[0], hv[1]);
        h[ni][1] = pack_bf16x2(hv[2], hv[3]);
        amax = max3_abs(amax, bf16_lo(h[ni][0]), bf16_hi(h[ni][0]));
        amax = max3_abs(amax, bf16_lo(h[ni][1]), bf16_hi(h[ni][1]));
      }
      amax = __builtin_fmaxf(amax, __shfl_xor(amax, 16));
      amax = __builtin_fmaxf(amax, __shfl_xor(amax, 32));
      const BlockQ bq = block_params<kOut>(amax);
      uint32_t cw[kSubN];
      block_codes<kOut>(bq, h, cw);
      if (r < t.m_valid && (lane >> 4) == 0) o.ys[(int64_t)r * nbo] = bq.s;
#pragma unroll
      for (int q = 0; q < kSubN / 4; ++q) {
        const uint4 v = rows_to_subtiles(cw[4 * q], cw[4 * q + 1], cw[4 * q + 2], cw[4 * q + 3]);
        if (r < t.m_valid) store_stream16(o.yq + (int64_t)r * F + 16 * (4 * q + (lane >> 4)), v);
      }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using Gate = std::true_type;
    using Up = std::false_type;
    __syncthreads();
    if (wn == 0) {
      hand_over(I2{});
      hand_over(I3{});
    } else {
      hand_over(I0{});
      hand_over(I1{});
    }
    __syncthreads();
    if (wn == 0) {
      rows_out(I0{}, Gate{});
      rows_out(I1{}, Gate{});
    } else {
      rows_out(I2{}, Up{});
      rows_out(I3{}, Up{});
    }
  } else {
    // Quantized epilogue (the activation quantization of the next layer, done
    // by the producer instead of by a separate pass over bf16 Y; page 1,
    // "Leistungsgewinne in der Praxis", names quantization-kernel overhead as
    // part of the gap to the ideal speedup).  Each value is first rounded to
    // bf16 exactly as the bf16 epilogue rounds it; a wave's 128 columns are
    // one 1x128 block of each of its rows, held by the lanes l, l^16, l^32,
    // l^48.  Block |max|, scale and element rule are those of the activation
    // quantizer, so the result equals quantizing the bf16 output bit for bit.
    // The codes go out as 16 bytes per lane (rows_to_subtiles): 64 bytes of a
    // row per instruction instead of 16, +1-5% on the Llama shapes.
    if constexpr (C::kWaveN == 64) {
      quant_epilogue_half<C, V>(t, o, N, lds, acc, wn, wm, lane);
    } else if (wn * 128 < t.n_valid) {
      static_assert(C::kWaveN == 128, "quantized epilogue: a wave's 128 columns are one 1x128 block");
      const int64_t nbo = N >> 7;  // scale blocks per output row
#pragma unroll
      for (int mi = 0; mi < kSubM; ++mi) {
        const int r = wm * 64 + mi * 16 + (lane & 15);
        uint32_t h[kSubN][2];
        float amax = 0.0f;
#pragma unroll
        for (int ni = 0; ni < kSubN; ++ni) {
          h[ni][0] = pack_bf16x2(acc[ni][mi][0], acc[ni][mi][1]);
          h[ni][1] = pack_bf16x2(acc[ni][mi][2], acc[ni][mi][3]);
          amax = max3_abs(amax, bf16_lo(h[ni][0]), bf16_hi(h[ni][0]));
          amax = max3_abs(amax, bf16_lo(h[ni][1]), bf16_hi(h[ni][1]));
        }
        amax = __builtin_fmaxf(amax, __shfl_xor(amax, 16));
        amax = __builtin_fmaxf(amax, __shfl_xor(amax, 32));
        const BlockQ bq = block_params<kOut>(amax);
        uint32_t cw[kSubN];
        block_codes<kOut>(bq, h, cw);
        if (r < t.m_valid && (lane >> 4) == 0) o.ys[(int64_t)r * nbo + wn] = bq.s;
#pragma unroll
        for (int q = 0; q < kSubN / 4; ++q) {
          const uint4 v = rows_to_subtiles(cw[4 * q], cw[4 * q + 1], cw[4 * q + 2], cw[4 * q + 3]);
          if (r < t.m_valid) store_stream16(o.yq + (int64_t)r * N + wn * 128 + 16 * (4 * q + (lane >> 4)), v);
        }
      }
    }
  }
}

// One output tile: token rows t.a_q[0 .. m_valid), weight rows t.b_q[0 ..
// n_valid), written at the tile origins in o (row stride N).
template <class C, class V>
__device__ __forceinline__ void gemm_tile(const TileJob &t, const TileOut &o, int64_t N, uint8_t *lds) {
  constexpr bool kPow2 = V::kPow2;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar registers, scalar branches
  const int wn = wave & (C::kWavesN - 1), wm = wave / C::kWavesN;
  const int KB = t.KB;

  v4f acc[kSubN][kSubM];  // rows ni >= C::kSubN unused
#pragma unroll
  for (int ni = 0; ni < C::kSubN; ++ni)
#pragma unroll
    for (int mi = 0; mi < kSubM; ++mi) acc[ni][mi] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

  if constexpr (C::kPingPong) {
    uint32_t bad = 0;
    gemm_main_pp<C, V>(t, lds, wave, lane, wn, wm, acc, bad);
    tile_finish<C, V>(t, o, N, lds, acc, bad, wave, wn, wm, lane);
    return;
  }
  const TileRsrc rs = make_rsrc<V>(t);
  const DmaLane dl = dma_lane<C, V>(t, wave, lane);

  // Blocks 0 .. kStages-2 in flight; block kk lives in stage buffer kk % kStages.
#pragma unroll
  for (int s = 0; s < C::kStages - 1; ++s)
    if (s < KB && wave >= C::kFirstLoader)
      issue_stage<C, V>(t, rs, dl, s, lds + s * C::kStageBytes, wave, lane, true);

  wait_block();
  BlockFrags f;
  f.bad = 0;
  load_block<C, V>(lds, wave, wn, wm, lane, f);

  v4f p[kRing];
  float4 sbq[2];  // per-row weight-side scales of two sub-tile rows (kBRow)
  int cur = 0;  // stage buffer of block k
  StageDma dma{&t, &rs, &dl, C::kStages - 1, lds + (C::kStages - 1) * C::kStageBytes, wave, lane,
               C::kStages - 1 < KB};
  v8i wlast;
  for (int k = 0; k + 1 < KB; ++k) {
    mma_steps<C, V, C::kMfma - kSubM>(lds + cur * C::kStageBytes, lds, k, wn, lane, f, acc, p, sbq, dma, wlast);
    // Block k's buffer is free once every wave is past the barrier in
    // block_boundary; block k + kStages goes into it during the next block.
    dma.k = k + C::kStages;
    dma.buf = lds + cur * C::kStageBytes;
    dma.on = k + C::kStages < KB;
    cur = (cur + 1 == C::kStages) ? 0 : cur + 1;
    block_boundary<C, V>(lds + cur * C::kStageBytes, lds, k + 1, KB, wave, wn, wm, lane, f, wlast, acc, p, sbq);
  }
  // the last block: its last row's MFMAs and the trailing folds, no barrier
  mma_steps<C, V, C::kMfma - kSubM>(lds + cur * C::kStageBytes, lds, KB - 1, wn, lane, f, acc, p, sbq, dma,
                                    wlast);
#pragma unroll
  for (int mi = 0; mi < kSubM; ++mi) {
    const int j = C::kMfma - kSubM + mi;
    mma_one<V>(C::kSubN - 1, mi, j, wlast, f, acc, p);
    if constexpr (!kPow2) fold_one<V>(j - 2, f.scl, acc, p, sbq);
  }
  if constexpr (!kPow2) {
    fold_one<V>(C::kMfma - 2, f.scl, acc, p, sbq);
    fold_one<V>(C::kMfma - 1, f.scl, acc, p, sbq);
  }
  wait_vmcnt<0>();  // no DMA may still be writing LDS when the workgroup ends
  tile_finish<C, V>(t, o, N, lds, acc, f.bad, wave, wn, wm, lane);
}

// Workgroup id -> logical tile id such that XCD x (which receives ids
// x, x+8, x+16, ...) owns one contiguous range of logical ids.
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t nwg) {
  const int64_t xcd = bid % kNumXcd, idx = bid / kNumXcd;
  const int64_t q = nwg / kNumXcd, r = nwg % kNumXcd;
  return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

// Logical id -> (m slot, n tile): groups of kGroupN weight panels; inside a
// group the m slot varies slowest... fastest over the group's n tiles.
__device__ __forceinline__ void raster(int64_t L, int64_t slots_m, int64_t tiles_n, int64_t &tm,
                                       int64_t &tn) {
  const int64_t per_group = (int64_t)kGroupN * slots_m;
  const int64_t g = L / per_group;
  const int64_t r = L - g * per_group;
  const int64_t n0 = g * kGroupN;
  const int64_t gw = (tiles_n - n0) < kGroupN ? (tiles_n - n0) : kGroupN;
  tm = r / gw;
  tn = n0 + (r - tm * gw);
}

// The second region of a dense launch with two tile shapes: an M x N block of
// the output (a column slice or a band of rows) on 128-row tiles, with its
// operands' and output's origins.
struct GemmRegion {
  const uint8_t *a_q;
  const float *a_s;
  const uint8_t *b_q;
  const float *b_s;
  uint16_t *y;
  uint8_t *yq;
  float *ys;
  int64_t M, N;
  int64_t slots_m;
  int32_t tiles_n;
};

struct GemmParams {
  const uint8_t *a_q;
  const float *a_s;
  const uint8_t *b_q;
  const float *b_s;
  const int32_t *offsets;  // grouped: [G+1] on the device; dense: unused
  uint16_t *y;             // bf16 output
  uint8_t *yq;             // E4M3 output (quantized epilogue)
  float *ys;               // its 1x128 scales
  const int32_t *gather;   // grouped with gathered token rows: [M] source rows; else null
  int64_t T;               // rows of the gathered token matrix
  int64_t M;  // dense: M; grouped: M_total
  int64_t N, K;
  int64_t slots_m;
  int32_t G;
  int32_t tiles_n;
  int64_t ldy;  // row stride of y (bf16 output): N, or the full width for a column slice
  // Dense bf16 output with two tile shapes in one launch: workgroups
  // [0, wgs_large) take the 256-row tiles described above, the rest the
  // 128-row tiles of `small`.  0: one shape.
  int64_t wgs_large;
  GemmRegion small;
};

__device__ __forceinline__ int64_t clamp_off(const int32_t *off, int32_t g, int64_t M) {
  int64_t v = off[g];
  return v < 0 ? 0 : (v > M ? M : v);
}

// Group of m slot tm: the largest g in [0, G) with S_g = floor(off[g] / kBM) + g
// <= tm.  S is non-decreasing for valid offsets, so g is the number of groups
// with S_g <= tm, less one.  Each lane tests one group per round of 64 and the
// rounds' loads go out together, so a tile finds its group in one memory round
// trip for G <= 256 (a binary search costs one dependent round trip per
// halving -- seven for 128 experts -- before the tile's first DMA can go out).
// The result is clamped to [0, G), which keeps every access in bounds even for
// malformed offsets.
template <class C>
__device__ __forceinline__ int32_t group_of(const GemmParams &p, int64_t tm) {
  const int lane = threadIdx.x & 63;
  int32_t cnt = 0;
  for (int32_t base = 0; base < p.G; base += 256) {
    int32_t v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int32_t g = base + r * 64 + lane;
      v[r] = g < p.G ? p.offsets[g] : 0;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int32_t g = base + r * 64 + lane;
      const int64_t o = v[r] < 0 ? 0 : (v[r] > p.M ? p.M : (int64_t)v[r]);
      cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(g < p.G && o / C::kBM + g <= tm));
    }
  }
  const int32_t g = cnt - 1;
  return g < 0 ? 0 : (g >= p.G ? p.G - 1 : g);
}

// Dense: m slot = m tile.  Grouped: group g owns the m slots [S_g, S_{g+1})
// with S_g = floor(off[g] / kBM) + g, which always holds ceil(rows_g / kBM)
// tiles; a slot beyond its group's rows exits at once.  No prefix sums or
// workspace are needed and the offsets never leave the device.
template <class C, class V>
__global__ __launch_bounds__(C::kThreads, 1) void gemm_kernel(GemmParams p) {
  constexpr bool kGrouped = V::kGrouped;
  constexpr int kOut = V::kOut;
  constexpr bool kGather = V::kGather;
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];

  if constexpr (!kGrouped && C::kBM == 256 && !V::kSwiGLU) {
    if (p.wgs_large > 0 && (int64_t)blockIdx.x >= p.wgs_large) {
      // The workgroups are dispatched in order, so the 128-row tiles fill
      // the CUs as the 256-row ones finish (no launch boundary between the
      // two shapes).
      const GemmRegion &r = p.small;
      const int64_t Ls = xcd_remap(blockIdx.x - p.wgs_large, gridDim.x - p.wgs_large);
      int64_t sm, sn;
      raster(Ls, r.slots_m, r.tiles_n, sm, sn);
      const int64_t m0 = sm * CfgSmall8::kBM, n0 = sn * kBN;
      if (m0 >= r.M) return;
      TileJob t;
      t.KB = (int)(p.K / kBK);
      t.K = p.K;
      t.a_q = r.a_q + m0 * p.K;
      t.a_s = r.a_s + m0 * t.KB;
      t.gidx = nullptr;
      t.T = 0;
      t.b_q = r.b_q + n0 * p.K;
      t.b_s = r.b_s + (V::kBRow ? n0 : (n0 >> 7)) * t.KB;
      t.m_valid = (int)((r.M - m0) < CfgSmall8::kBM ? (r.M - m0) : CfgSmall8::kBM);
      t.n_valid = (int)((r.N - n0) < kBN ? (r.N - n0) : kBN);
      TileOut o{nullptr, nullptr, nullptr};
      if constexpr (kOut == kOutBf16) {
        o.y = r.y + m0 * p.ldy + n0;
      } else {
        o.yq = r.yq + m0 * p.ldy + n0;
        o.ys = r.ys + m0 * (p.ldy >> 7) + (n0 >> 7);
      }
      gemm_tile<CfgSmall8, V>(t, o, p.ldy, lds);
      return;
    }
  }
  const int64_t L = xcd_remap(blockIdx.x, p.wgs_large > 0 ? p.wgs_large : (int64_t)gridDim.x);
  int64_t tm, tn;
  raster(L, p.slots_m, p.tiles_n, tm, tn);
  const int64_t n0 = tn * kBN;
  const int n_valid = (int)((p.N - n0) < kBN ? (p.N - n0) : kBN);

  int64_t m0, m_end;
  const uint8_t *bq = p.b_q;
  const float *bs = p.b_s;
  if (!kGrouped) {
    m0 = tm * C::kBM;
    m_end = p.M;
  } else {
    const int32_t g = group_of<C>(p, tm);
    const int64_t g0 = clamp_off(p.offsets, g, p.M);
    const int64_t g1 = clamp_off(p.offsets, g + 1, p.M);
    m0 = g0 + (tm - (g0 / C::kBM + g)) * C::kBM;
    m_end = g1;
    bq += (int64_t)g * p.N * p.K;
    bs += (int64_t)g * (V::kBRow ? p.N : p.N / 128) * (p.K / kBK);
  }
  if (m0 >= m_end || m0 < 0) return;

  TileJob t;
  t.KB = (int)(p.K / kBK);
  t.K = p.K;
  if constexpr (kGather) {  // rows m0.. of the group are token rows gather[m0..]
    t.a_q = p.a_q;
    t.a_s = p.a_s;
    t.gidx = p.gather + m0;
    t.T = p.T;
  } else {
    t.a_q = p.a_q + m0 * p.K;
    t.a_s = p.a_s + m0 * t.KB;
    t.gidx = nullptr;
    t.T = 0;
  }
  t.b_q = bq + n0 * p.K;
  t.b_s = bs + (V::kBRow ? n0 : (n0 >> 7)) * t.KB;
  t.m_valid = (int)((m_end - m0) < C::kBM ? (m_end - m0) : C::kBM);
  t.n_valid = n_valid;
  TileOut o{nullptr, nullptr, nullptr};
  if constexpr (kOut == kOutBf16) {
    o.y = p.y + m0 * p.ldy + n0;
  } else if constexpr (V::kSwiGLU) {  // h [M][N/2]: this tile's 128 columns start at n0/2
    o.yq = p.yq + m0 * (p.N >> 1) + (n0 >> 1);
    o.ys = p.ys + m0 * (p.N >> 8) + (n0 >> 8);
  } else {  // a quantized output may be a column slice of a wider one (row stride ldy)
    o.yq = p.yq + m0 * p.ldy + n0;
    o.ys = p.ys + m0 * (p.ldy >> 7) + (n0 >> 7);
  }
  if constexpr (kGrouped && C::kBM == 256 && (kOut == kOutBf16 || V::kSwiGLU) && !V::kBRow) {
    // A group's last slot with at most 128 rows runs as a 128-row tile (same
    // eight waves): about half the padding of a 256-row tile, at ~0.7 of its
    // time (Qwen3 routing: padding rows 23% -> 12% of the rows).  Measured:
    // Qwen3 gate+up +2% (pow2), amax grouped GEMMs +1-6% (Moonlight down
    // -1.5%), gathered rows +1.5-3%.
    if (t.m_valid <= CfgSmall8::kBM) {
      gemm_tile<CfgSmall8, V>(t, o, V::kSwiGLU ? p.N : p.ldy, lds);
      return;
    }
  }
  gemm_tile<C, V>(t, o, V::kSwiGLU ? p.N : p.ldy, lds);
}

template <class C, class V>
constexpr int lds_bytes() {
  return V::kBRow ? C::kLdsBytesChunked : C::kLdsBytes;
}

template <class C, class V>
static hipError_t launch(GemmParams p, hipStream_t stream) {
  // The LDS size above the default limit is an attribute of the kernel on the
  // current device: set once per device (std::call_once, so concurrent first
  // calls from several host threads are safe), and the outcome kept.
  static std::once_flag once[kMaxDevices];
  static hipError_t attr_err[kMaxDevices];
  constexpr int kLds = lds_bytes<C, V>();
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(once[dev], [dev]() {
    attr_err[dev] = hipFuncSetAttribute((const void *)gemm_kernel<C, V>,
                                        hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
  });
  if (attr_err[dev] != hipSuccess) return attr_err[dev];
  const int64_t grid = p.slots_m * p.tiles_n + (p.wgs_large > 0 ? p.small.slots_m * p.small.tiles_n : 0);
  hipLaunchKernelGGL((gemm_kernel<C, V>), dim3((unsigned)grid), dim3(C::kThreads),
                     kLds, stream, p);
  return hipGetLastError();
}

// Tile plan of an M x N output: the tiles of token rows [0, R) and weight
// panels (256 rows each) [0, P) run as 256-token tiles, the rest as 128-token
// tiles.  The plan with the shortest estimated time: rounds of tiles over the
// 256 CUs times a tile's time, a 128-row tile taking about 0.7 of a 256-row one
// (measured on the Llama shapes).  Besides all-large (R = M, P = all) and
// all-small (R = 0), the output of every GEMM but the SwiGLU one may be split
// into slices of the output (bf16 Y, or the E4M3 codes and their scales): by
// weight panels (R = M, P < all) or by token rows (R < M, P = all), as one
// launch holding both tile shapes (8 waves each) or, with per-row weight
// scales, as two launches.  At 4096 tokens QKV's 24 panels make 384 large tiles (two rounds,
// the second half empty); 16 panels on large tiles (one round) and 8 on small
// ones (one round) cost 1.7 instead of 2 (measured on the quantized output:
// 1.09x).  The weight gradient of QKV (6144 rows of dW, 16 panels) splits by
// rows the same way: 4096 rows on large tiles, 2048 on small ones.  At 2048
// tokens QKV's 192 large tiles (one round) beat 384 small ones (+37%), while O
// and down (128 large tiles, half the CUs idle) take small tiles.
void dense_tile_plan(int64_t M, int64_t N, bool may_split, int64_t &rows_large, int64_t &panels_large) {
  const int64_t tiles_n = (N + kBN - 1) / kBN;
  const int64_t mt_large = (M + CfgLarge::kBM - 1) / CfgLarge::kBM;
  const int64_t mt_small = (M + CfgSmall8::kBM - 1) / CfgSmall8::kBM;
  auto rounds = [](int64_t tiles) { return (tiles + 255) / 256; };
  auto cost_n = [&](int64_t n1) {  // n1 panels on large tiles, the rest on small ones
    return rounds(mt_large * n1) * 10 + rounds(mt_small * (tiles_n - n1)) * 7;
  };
  auto cost_m = [&](int64_t m1) {  // m1 large row tiles (256 rows each), the rest on small ones
    return rounds(m1 * tiles_n) * 10 + rounds((M - m1 * CfgLarge::kBM + CfgSmall8::kBM - 1) / CfgSmall8::kBM * tiles_n) * 7;
  };
  int64_t best = cost_n(tiles_n), n1 = tiles_n, m1 = -1;
  if (cost_n(0) < best) {
    best = cost_n(0);
    n1 = 0;
  }
  if (may_split) {
    for (int64_t c = 1; c < tiles_n; ++c)
      if (cost_n(c) < best) {
        best = cost_n(c);
        n1 = c;
      }
    for (int64_t r = 1; r * CfgLarge::kBM < M; ++r)
      if (cost_m(r) < best) {
        best = cost_m(r);
        m1 = r;
      }
  }
  if (m1 > 0) {
    rows_large = m1 * CfgLarge::kBM;
    panels_large = tiles_n;
  } else {
    rows_large = n1 > 0 ? M : 0;
    panels_large = n1;
  }
}

template <bool kPow2, int kOut = kOutBf16, bool kBRow = false, bool kSwiGLU = false>
static hipError_t dense(const uint8_t *a_q, const float *a_s, const uint8_t *b_q, const float *b_s,
                        uint16_t *y, uint8_t *yq, float *ys, int64_t M, int64_t N, int64_t K,
                        hipStream_t stream) {
  using V = Variant<false, kPow2, kOut, false, kBRow, kSwiGLU>;
  if (M == 0 || N == 0) return hipSuccess;
  const int32_t tiles_n = (int32_t)((N + kBN - 1) / kBN);
  GemmParams p{a_q, a_s, b_q, b_s, nullptr, y, yq, ys, nullptr, 0, M, N, K, 0, 1, tiles_n, N, 0, {}};
  const int64_t mt_large = (M + CfgLarge::kBM - 1) / CfgLarge::kBM;
  const int64_t mt_small = (M + CfgSmall8::kBM - 1) / CfgSmall8::kBM;
  int64_t rows_large, n1;
  dense_tile_plan(M, N, !kSwiGLU, rows_large, n1);
  if (rows_large == M && n1 == tiles_n) {
    p.slots_m = mt_large;
    return launch<LargeCfg<V>, V>(p, stream);
  }
  if constexpr (!kSwiGLU) {
    // Both shapes in one launch (the 128-row tiles run 8 waves too): rows
    // [0, rows_large) x panels [0, n1) on 256-row tiles, the rest (the other
    // rows, or the other panels) on 128-row tiles.
    static_assert(CfgSmall8::kThreads == LargeCfg<V>::kThreads, "one workgroup size");
    const bool by_rows = rows_large > 0 && rows_large < M;
    if (by_rows || n1 > 0) {
      GemmRegion r;
      if (by_rows) {
        p.M = rows_large;
        p.slots_m = rows_large / CfgLarge::kBM;
        r = GemmRegion{a_q + rows_large * K, a_s + rows_large * (K / kBK), b_q, b_s,
                       y ? y + rows_large * p.ldy : nullptr, yq ? yq + rows_large * p.ldy : nullptr,
                       ys ? ys + rows_large * (p.ldy >> 7) : nullptr, M - rows_large, N, 0, tiles_n};
      } else {
        const int64_t n_off = n1 * kBN;
        p.N = n_off;
        p.tiles_n = (int32_t)n1;
        p.slots_m = mt_large;
        r = GemmRegion{a_q, a_s, b_q + n_off * K, b_s + (kBRow ? n_off : n_off / 128) * (K / kBK),
                       y ? y + n_off : nullptr,
                       yq ? yq + n_off : nullptr, ys ? ys + n_off / 128 : nullptr, M, N - n_off, 0,
                       (int32_t)(tiles_n - n1)};
      }
      r.slots_m = (r.M + CfgSmall8::kBM - 1) / CfgSmall8::kBM;
      p.wgs_large = p.slots_m * p.tiles_n;
      p.small = r;
      return launch<LargeCfg<V>, V>(p, stream);
    }
  }
  if (rows_large > 0 && rows_large < M) {
    // token rows [0, rows_large) on 256-row tiles, then the rest on 128-row tiles
    GemmParams q = p;
    q.M = rows_large;
    q.slots_m = rows_large / CfgLarge::kBM;
    hipError_t e = launch<LargeCfg<V>, V>(q, stream);
    if (e != hipSuccess) return e;
    p.a_q = a_q + rows_large * K;
    p.a_s = a_s + rows_large * (K / kBK);
    if constexpr (kOut == kOutBf16) {
      p.y = y + rows_large * p.ldy;
    } else {
      p.yq = yq + rows_large * p.ldy;
      p.ys = ys + rows_large * (p.ldy >> 7);
    }
    p.M = M - rows_large;
    p.slots_m = (p.M + CfgSmall8::kBM - 1) / CfgSmall8::kBM;
    return launch<SmallCfg<V>, V>(p, stream);
  }
  if (n1 > 0) {
    // panels [0, n1) on 256-row tiles, then the rest on 128-row tiles
    const int64_t n_off = n1 * kBN;
    GemmParams q = p;
    q.N = n_off;
    q.tiles_n = (int32_t)n1;
    q.slots_m = mt_large;
    hipError_t e = launch<LargeCfg<V>, V>(q, stream);
    if (e != hipSuccess) return e;
    p.b_q = b_q + n_off * K;
    p.b_s = b_s + (kBRow ? n_off : n_off / 128) * (K / kBK);
    if constexpr (kOut == kOutBf16) {
      p.y = y + n_off;
    } else {
      p.yq = yq + n_off;
      p.ys = ys + n_off / 128;
    }
    p.N = N - n_off;
    p.tiles_n = (int32_t)(tiles_n - n1);
  }
  p.slots_m = mt_small;
  return launch<SmallCfg<V>, V>(p, stream);
}

template <bool kPow2, bool kGather = false, int kOut = kOutBf16, bool kSwiGLU = false>
static hipError_t grouped(const uint8_t *a_q, const float *a_s, const uint8_t *b_q, const float *b_s,
                          const int32_t *group_offsets, int32_t G, int64_t M_total, int64_t N, int64_t K,
                          uint16_t *y, const int32_t *gather, int64_t T, hipStream_t stream,
                          uint8_t *yq = nullptr, float *ys = nullptr) {
  using V = Variant<true, kPow2, kOut, kGather, false, kSwiGLU>;
  if (M_total == 0 || N == 0) return hipSuccess;
  const int32_t tiles_n = (int32_t)((N + kBN - 1) / kBN);
  GemmParams p{a_q, a_s, b_q, b_s, group_offsets, y, yq, ys, gather, T, M_total, N, K, 0, G, tiles_n, N, 0, {}};
  // 256-row tiles once the average group fills one; their ragged last tile
  // per group then wastes at most half of the work it would at 128 rows.
  if (M_total >= (int64_t)G * CfgLarge::kBM) {
    p.slots_m = M_total / CfgLarge::kBM + G;
    return launch<LargeCfg<V>, V>(p, stream);
  }
  p.slots_m = M_total / CfgSmall8::kBM + G;
  return launch<SmallCfg<V>, V>(p, stream);
}

hipError_t launch_blockscaled_gemm(const uint8_t *a_q, const float *a_s,
                                   const uint8_t *b_q, const float *b_s,
                                   uint16_t *y, int64_t M, int64_t N, int64_t K,
                                   bool pow2, hipStream_t stream) {
  return pow2 ? dense<true>(a_q, a_s, b_q, b_s, y, nullptr, nullptr, M, N, K, stream)
              : dense<false>(a_q, a_s, b_q, b_s, y, nullptr, nullptr, M, N, K, stream);
}

hipError_t launch_blockscaled_gemm_quant(const uint8_t *a_q, const float *a_s,
                                         const uint8_t *b_q, const float *b_s,
                                         uint8_t *yq, float *ys, int64_t M, int64_t N, int64_t K,
                                         int mode, hipStream_t stream) {
  return mode == kModePow2 ? dense<false, kModePow2>(a_q, a_s, b_q, b_s, nullptr, yq, ys, M, N, K, stream)
                           : dense<false, kModeAmax>(a_q, a_s, b_q, b_s, nullptr, yq, ys, M, N, K, stream);
}

hipError_t launch_blockscaled_gemm_wgrad(const uint8_t *a_q, const float *a_s,
                                         const uint8_t *b_q, const float *b_s,
                                         uint16_t *y, int64_t M, int64_t N, int64_t K, bool pow2,
                                         hipStream_t stream) {
  return pow2 ? dense<true, kOutBf16, true>(a_q, a_s, b_q, b_s, y, nullptr, nullptr, M, N, K, stream)
              : dense<false, kOutBf16, true>(a_q, a_s, b_q, b_s, y, nullptr, nullptr, M, N, K, stream);
}

hipError_t launch_blockscaled_gemm_swiglu_quant(const uint8_t *a_q, const float *a_s,
                                                const uint8_t *b_q, const float *b_s,
                                                uint8_t *hq, float *hs, int64_t M, int64_t F, int64_t K,
                                                int mode, hipStream_t stream) {
  return mode == kModePow2
             ? dense<false, kModePow2, false, true>(a_q, a_s, b_q, b_s, nullptr, hq, hs, M, 2 * F, K, stream)
             : dense<false, kModeAmax, false, true>(a_q, a_s, b_q, b_s, nullptr, hq, hs, M, 2 * F, K, stream);
}

hipError_t launch_grouped_gemm(const uint8_t *a_q, const float *a_s,
                               const uint8_t *b_q, const float *b_s,
                               const int32_t *group_offsets, int32_t G,
                               int64_t M_total, int64_t N, int64_t K,
                               uint16_t *y, bool pow2, hipStream_t stream) {
  return pow2 ? grouped<true>(a_q, a_s, b_q, b_s, group_offsets, G, M_total, N, K, y, nullptr, 0, stream)
              : grouped<false>(a_q, a_s, b_q, b_s, group_offsets, G, M_total, N, K, y, nullptr, 0, stream);
}

hipError_t launch_grouped_gemm_gather(const uint8_t *a_q, const float *a_s, int64_t T,
                                      const uint8_t *b_q, const float *b_s,
                                      const int32_t *group_offsets, const int32_t *row_index, int32_t G,
                                      int64_t M_total, int64_t N, int64_t K, uint16_t *y, bool pow2,
                                      hipStream_t stream) {
  return pow2 ? grouped<true, true>(a_q, a_s, b_q, b_s, group_offsets, G, M_total, N, K, y, row_index, T, stream)
              : grouped<false, true>(a_q, a_s, b_q, b_s, group_offsets, G, M_total, N, K, y, row_index, T, stream);
}

hipError_t launch_grouped_gemm_swiglu_quant(const uint8_t *a_q, const float *a_s, int64_t T,
                                            const uint8_t *b_q, const float *b_s,
                                            const int32_t *group_offsets, const int32_t *row_index, int32_t G,
                                            int64_t M_total, int64_t F, int64_t K, uint8_t *hq, float *hs,
                                            int mode, hipStream_t stream) {
  const int64_t N = 2 * F;
  if (row_index) {
    return mode == kModePow2
               ? grouped<false, true, kModePow2, true>(a_q, a_s, b_q, b_s, group_offsets, G, M_total, N, K, nullptr,
                                                      row_index, T, stream, hq, hs)
               : grouped<false, true, kModeAmax, true>(a_q, a_s, b_q, b_s, group_offsets, G, M_total, N, K, nullptr,
                                                      row_index, T, stream, hq, hs);
  }
  return mode == kModePow2
             ? grouped<false, false, kModePow2, true>(a_q, a_s, b_q, b_s, group_offsets, G, M_total, N, K, nullptr,
                                                     nullptr, 0, stream, hq, hs)
             : grouped<false, false, kModeAmax, true>(a_q, a_s, b_q, b_s, group_offsets, G, M_total, N, K, nullptr,
                                                     nullptr, 0, stream, hq, hs);
}

}  // namespace fp8q
