// MoE dispatch order on the device: routing table -> group offsets and the
// token of every grouped row, for the grouped and gathering GEMMs.
//
// The recipe trains mixture-of-experts models (page "NVIDIA NeMo RL erreicht
// 48% Geschwindigkeitssteigerung ...", section "Leistungsgewinne in der
// Praxis": Qwen3-30B; section "Warum dies fuer die KI-Oekonomie wichtig ist":
// Moonlight 16B).  Their expert GEMMs take the routed rows grouped by expert.
// Order: rows sorted by expert, stable in routing-table order (entry t*k + j
// for token t, slot j); shared experts follow as groups of all tokens; an
// expert id outside [0, E) places its entry in no group, leaving rows with
// token -1 at the end.
//
// A stable counting sort in three launches, deterministic (no order depends
// on the timing of atomics) and with no host synchronisation:
//  1. rank: block b takes entries [kChunk*b, kChunk*(b+1)).  In steps of 256
//     entries (one per lane), each wave marks its lanes in a per-wave 64-bit
//     mask per expert (LDS atomic OR: the result does not depend on order);
//     an entry's rank inside the block is the running count of its expert
//     from earlier steps, plus the mask bits of earlier waves, plus those of
//     lower lanes of its own wave.  Writes every entry's in-block rank and the
//     block's count per expert ([E][nblocks], expert-major) to the workspace.
//  2. scan: one workgroup turns the counts, read expert-major, into exclusive
//     prefix sums -- the first row of (expert e, block b) -- and writes the
//     group offsets.
//  3. scatter: entry i of expert e goes to row base[e][b] + rank; shared
//     groups and the trailing rows of invalid entries are filled after the
//     routed rows (which end at offsets[E]).
#include "fp8q_internal.h"

namespace fp8q {

constexpr int kPermThreads = 256;
constexpr int kPermWaves = kPermThreads / 64;
constexpr int kPermChunk = 1024;  // entries per rank block (4 steps)
constexpr int kScanThreads = 1024;
constexpr int kScanPer = 8;       // consecutive counts per scan lane and tile

int64_t moe_permute_blocks(int64_t n) { return (n + kPermChunk - 1) / kPermChunk; }

// Workspace: in-block ranks [n] then counts [E][nblocks] (int32), each part
// starting on a 256-byte boundary.
int64_t moe_permute_workspace_bytes(int64_t n, int32_t E) {
  const int64_t ranks = (n * 4 + 255) / 256 * 256;
  const int64_t counts = (E * moe_permute_blocks(n) * 4 + 255) / 256 * 256;
  return ranks + counts;
}

__global__ __launch_bounds__(kPermThreads) void moe_rank_kernel(const int32_t *__restrict__ ids, int64_t n,
                                                                int32_t E, int64_t nblocks,
                                                                int32_t *__restrict__ rank,
                                                                int32_t *__restrict__ counts) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  unsigned long long *mask = reinterpret_cast<unsigned long long *>(smem);   // [kPermWaves][E]
  int32_t *run = reinterpret_cast<int32_t *>(smem + sizeof(unsigned long long) * kPermWaves * E);  // [E]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t b = blockIdx.x;
  for (int i = tid; i < kPermWaves * E; i += kPermThreads) mask[i] = 0ull;
  for (int i = tid; i < E; i += kPermThreads) run[i] = 0;
  __syncthreads();
  const int64_t begin = b * kPermChunk;
  const unsigned long long below = (1ull << lane) - 1ull;  // lanes under this one
  constexpr int kSteps = kPermChunk / kPermThreads;
  int32_t ev[kSteps];  // all of the block's ids in flight at once
#pragma unroll
  for (int step = 0; step < kSteps; ++step) {
    const int64_t i = begin + step * kPermThreads + tid;
    ev[step] = i < n ? ids[i] : -1;
  }
#pragma unroll
  for (int step = 0; step < kSteps; ++step) {
    const int64_t i = begin + step * kPermThreads + tid;
    const int32_t e = ev[step];
    const bool valid = e >= 0 && e < E;
    if (valid) atomicOr(&mask[w * E + e], 1ull << lane);
    __syncthreads();
    unsigned long long mine = 0ull;
    if (valid) {
      mine = mask[w * E + e];
      int r = run[e] + __popcll(mine & below);
      for (int v = 0; v < w; ++v) r += __popcll(mask[v * E + e]);
      rank[i] = r;
    }
    __syncthreads();
    if (valid) {
      // the lowest lane of each (wave, expert) group adds the group's size;
      // integer sums do not depend on the order of the atomics
      if ((mine & below) == 0ull) atomicAdd(&run[e], __popcll(mine));
      mask[w * E + e] = 0ull;
    }
    __syncthreads();
  }
  for (int e = tid; e < E; e += kPermThreads) counts[(int64_t)e * nblocks + b] = run[e];
}

// Exclusive prefix sums of counts[0 .. L) in place (L = E * nblocks, read
// expert-major), and the group offsets: offsets[e] = the sum of all counts of
// experts below e, offsets[E] = the number of valid entries, then the shared
// groups of T rows each.
__global__ __launch_bounds__(kScanThreads) void moe_scan_kernel(int32_t *__restrict__ counts, int32_t E,
                                                                int64_t nblocks, int64_t T, int32_t n_shared,
                                                                int32_t *__restrict__ offsets) {
  __shared__ int32_t wsum[kScanThreads / 64];
  __shared__ int32_t carry_s;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t L = (int64_t)E * nblocks;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int64_t base = 0; base < L; base += (int64_t)kScanThreads * kScanPer) {
    const int64_t f0 = base + (int64_t)tid * kScanPer;
    int32_t v[kScanPer];
    int32_t sum = 0;
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      v[j] = f0 + j < L ? counts[f0 + j] : 0;
      sum += v[j];
    }
    // inclusive scan of the lane sums inside the wave
    int32_t inc = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int32_t o = __shfl_up(inc, d);
      if (lane >= d) inc += o;
    }
    if (lane == 63) wsum[w] = inc;
    __syncthreads();
    int32_t before = carry_s;
    for (int v2 = 0; v2 < w; ++v2) before += wsum[v2];
    int32_t run = before + inc - sum;  // exclusive prefix of this lane's first count
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      const int64_t f = f0 + j;
      if (f < L) {
        counts[f] = run;
        if (f % nblocks == 0) offsets[f / nblocks] = run;  // block 0 of expert f / nblocks
      }
      run += v[j];
    }
    __syncthreads();
    if (tid == kScanThreads - 1) carry_s = run;  // the last lane's running sum is the tile's end
    __syncthreads();
  }
  if (tid == 0) {
    const int32_t total = carry_s;
    if (nblocks == 0)
      for (int32_t e = 0; e < E; ++e) offsets[e] = 0;
    offsets[E] = total;
    for (int32_t s = 0; s < n_shared; ++s) offsets[E + 1 + s] = total + (int32_t)((s + 1) * T);
  }
}

__global__ __launch_bounds__(kPermThreads) void moe_scatter_kernel(const int32_t *__restrict__ ids, int64_t n,
                                                                   int32_t k, int32_t E, int64_t T,
                                                                   int32_t n_shared, int64_t nblocks,
                                                                   const int32_t *__restrict__ rank,
                                                                   const int32_t *__restrict__ base,
                                                                   const int32_t *__restrict__ offsets,
                                                                   int32_t *__restrict__ row_index,
                                                                   int32_t *__restrict__ entry_row) {
  const int64_t j = (int64_t)blockIdx.x * kPermThreads + threadIdx.x;
  const int64_t rows = n + (int64_t)n_shared * T;
  if (j < n) {
    const int32_t e = ids[j];
    int64_t r = -1;
    if (e >= 0 && e < E) {
      r = (int64_t)base[(int64_t)e * nblocks + j / kPermChunk] + rank[j];
      row_index[r] = (int32_t)(j / k);
    }
    if (entry_row) entry_row[j] = (int32_t)r;
  }
  // rows after the routed ones: the shared groups, then the rows left by
  // invalid entries
  const int64_t nv = offsets[E];
  const int64_t r = nv + j;
  if (j < rows && r < rows) {
    const int64_t q = j;  // position after the routed rows
    row_index[r] = q < (int64_t)n_shared * T ? (int32_t)(q % T) : -1;
  }
}

hipError_t launch_moe_permute(const int32_t *ids, int64_t T, int32_t k, int32_t E, int32_t n_shared,
                              int32_t *offsets, int32_t *row_index, int32_t *entry_row, void *workspace,
                              hipStream_t stream) {
  const int64_t n = T * k;
  const int64_t nb = moe_permute_blocks(n);
  int32_t *rank = static_cast<int32_t *>(workspace);
  int32_t *counts = reinterpret_cast<int32_t *>(static_cast<uint8_t *>(workspace) + (n * 4 + 255) / 256 * 256);
  if (nb > 0) {
    const size_t lds = sizeof(unsigned long long) * kPermWaves * E + sizeof(int32_t) * E;
    hipLaunchKernelGGL(moe_rank_kernel, dim3((unsigned)nb), dim3(kPermThreads), lds, stream, ids, n, E, nb, rank,
                       counts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(moe_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, counts, E, nb, T, n_shared, offsets);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = n + (int64_t)n_shared * T;
  if (rows > 0) {
    hipLaunchKernelGGL(moe_scatter_kernel, dim3((unsigned)((rows + kPermThreads - 1) / kPermThreads)),
                       dim3(kPermThreads), 0, stream, ids, n, k, E, T, n_shared, nb, rank, counts, offsets,
                       row_index, entry_row);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace fp8q
