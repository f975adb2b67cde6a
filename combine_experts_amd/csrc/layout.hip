// Dispatch layout: per-expert counts, capacity cut, per-expert and per-rank offsets, and the stable
// (expert, pair id) permutation.
//
// The pages' dispatch step ("Expert Parallelism and All-to-All", section on the two exchanges; the
// EP-in-LLMs article, pipeline steps 1-2; the all-to-all article's dispatch example with
// destination = expert / experts_per_device and per-device bincount) groups each device's
// (token, expert) pairs contiguously by destination. Here the grouping is by expert, stable in
// pair id, which is also grouping by rank because ranks own contiguous expert blocks.
//
// Four steps, none of whose results depend on thread scheduling:
//   1. count       one wave per chunk of kLayoutChunk pairs: per-chunk expert histogram
//   2. scan_chunks one wave per expert: exclusive scan of the expert's chunk histogram column
//                  -> each chunk's first rank inside the expert; the column total is the count
//   3. scan_exp    one block: capacity cut, exclusive scan over experts, per-rank counts/offsets
//   4. assign      one wave per chunk, pairs visited in pair-id order 64 at a time: a pair's rank
//                  inside its expert = chunk base + earlier same-expert pairs of the chunk
//                  (wave ballots find same-expert lanes); row = offset + rank if rank < capacity.
// Large problems run them as four kernels with the chunk histograms in the caller's workspace.
// When every chunk histogram fits in LDS (at most kFusedChunks chunks, kFusedHist entries), one
// block of 16 waves runs all four steps with barriers between them: the same functions on the same
// data, so the same results, in one launch instead of four (these problems are launch-bound).
#include "moe_common.h"

#include <mutex>

// Per-chunk histograms of moe_dispatch_layout_noalloc: a static array of this library instead of a
// caller workspace, for callers that cannot allocate. Every GPU the library runs on holds its own
// copy until the process ends; all calls on one GPU share it. In host code this name only stands in
// for the array: its device address comes from hipGetSymbolAddress (layout_noalloc_scratch below).
static __device__ __align__(256) int32_t scratch[MOE_LAYOUT_NOALLOC_SCRATCH_BYTES / sizeof(int32_t)];

namespace moe {
namespace {

constexpr int kWavesPerBlock = 4;

constexpr int kChunkIters = kLayoutChunk / MOE_WAVE;  // pairs per lane in a chunk

// The expert ids of one chunk (pairs [p0, p1)), loaded by one wave all at once: lane l holds pair
// p0 + 64 i + l in ids[i]; slots past p1 hold E.
__device__ __forceinline__ void load_chunk(const int32_t* __restrict__ topk_idx, int p0, int p1, int32_t E, int lane,
                                           int (&ids)[kChunkIters]) {
#pragma unroll
  for (int i = 0; i < kChunkIters; ++i) {
    const int p = p0 + i * MOE_WAVE + lane;
    ids[i] = p < p1 ? topk_idx[p] : E;
  }
}

// Step 1 for one chunk, by one wave: adds the chunk's expert ids into hist[0, E) (LDS, zeroed by the
// caller). An id outside [0, E) counts nowhere.
__device__ __forceinline__ void count_chunk(const int (&ids)[kChunkIters], int32_t E, int32_t* hist) {
#pragma unroll
  for (int i = 0; i < kChunkIters; ++i) {
    const int e = ids[i];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
  }
}

// Wave-wide inclusive prefix sum of one int per lane.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < MOE_WAVE; off <<= 1) {
    int u = __shfl_up(v, off, MOE_WAVE);
    if (lane >= off) v += u;
  }
  return v;
}

// Step 2 for expert e, by one wave: column e of hist ([n_chunks][E]) becomes its exclusive prefix sum
// over the chunks; returns the column total.
__device__ __forceinline__ int scan_column(int32_t* hist, int e, int32_t E, int n_chunks, int lane) {
  int carry = 0;
  for (int c0 = 0; c0 < n_chunks; c0 += MOE_WAVE) {
    const int c = c0 + lane;
    const int v = (c < n_chunks) ? hist[(size_t)c * E + e] : 0;
    const int inc = wave_inclusive_scan(v);
    if (c < n_chunks) hist[(size_t)c * E + e] = carry + inc - v;  // exclusive base
    carry += __shfl(inc, MOE_WAVE - 1, MOE_WAVE);
  }
  return carry;
}

// Step 3, by a block of 1024 threads (E <= 1024): kept = min(count, capacity), exclusive scan over
// the experts into expert_offsets (and offs, LDS, E + 1 entries), per-rank counts and offsets.
// wave_tot: LDS, 16 entries. Ends with a block barrier.
__device__ __forceinline__ void scan_experts(const int32_t* counts, int32_t* __restrict__ expert_offsets,
                                             int32_t* __restrict__ rank_counts, int32_t* __restrict__ rank_offsets,
                                             int32_t E, int32_t ep_size, int32_t capacity, int32_t* wave_tot,
                                             int32_t* offs) {
  const int t = threadIdx.x;
  const int lane = t % MOE_WAVE, wave = t / MOE_WAVE;
  const int kept = (t < E) ? min(counts[t], capacity) : 0;
  const int inc = wave_inclusive_scan(kept);
  if (lane == MOE_WAVE - 1) wave_tot[wave] = inc;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wave_tot[w];
  const int excl = before + inc - kept;
  if (t < E) {
    offs[t] = excl;
    expert_offsets[t] = excl;
  }
  if (t == E - 1) {
    offs[E] = excl + kept;
    expert_offsets[E] = excl + kept;
  }
  __syncthreads();
  const int epr = E / ep_size;
  if (t < ep_size) {
    rank_offsets[t] = offs[t * epr];
    rank_counts[t] = offs[(t + 1) * epr] - offs[t * epr];
  }
  if (t == 0) rank_offsets[ep_size] = offs[E];
  __syncthreads();
}

// Step 4 for one chunk (pairs [p0, p1), ids as load_chunk gives them), by one wave, 64 pairs at a
// time in pair order: running[0, E) (LDS) holds the chunk's first rank inside each expert and is
// advanced as the pairs are placed; offsets[0, E] are the experts' row offsets (offsets[E] = kept rows).
__device__ __forceinline__ void assign_chunk(const int (&ids)[kChunkIters], int32_t* running, const int32_t* offsets,
                                             int32_t* __restrict__ pair_to_row, int32_t* __restrict__ row_to_pair,
                                             int p0, int p1, int32_t E, int32_t capacity, int32_t key_bits,
                                             int lane) {
  const int n_kept = offsets[E];
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (MOE_WAVE - lane));
#pragma unroll
  for (int i = 0; i < kChunkIters; ++i) {
    const int p = p0 + i * MOE_WAVE + lane;
    if (p0 + i * MOE_WAVE >= p1) break;  // uniform across the wave
    const bool in_chunk = p < p1;
    const int raw = ids[i];
    const bool valid = in_chunk && raw >= 0 && raw < E;
    const int key = valid ? raw : E;  // E: sentinel for lanes past the end or with an invalid id
    // lanes holding the same expert as this lane
    uint64_t same = ~0ull;
    for (int b = 0; b < key_bits; ++b) {
      const bool bit = (key >> b) & 1;
      const uint64_t bal = __ballot(bit);
      same &= bit ? bal : ~bal;
    }
    const int n_before = __popcll(same & below);
    const int n_same = __popcll(same);
    const int leader = __ffsll((long long)same) - 1;
    const int base = valid ? running[key] : 0;
    __builtin_amdgcn_wave_barrier();
    if (valid && lane == leader) running[key] = base + n_same;
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      const int rank = base + n_before;
      if (rank < capacity) {
        const int row = offsets[key] + rank;
        pair_to_row[p] = row;
        row_to_pair[row] = p;
      } else {
        pair_to_row[p] = -1;
      }
    } else if (in_chunk) {
      pair_to_row[p] = -1;  // an invalid expert id is treated as a dropped pair
    }
    if (in_chunk && p >= n_kept) row_to_pair[p] = -1;  // rows past N hold no pair
  }
}

__global__ void __launch_bounds__(256) layout_count(const int32_t* __restrict__ topk_idx,
                                                    int32_t* __restrict__ chunk_hist, int32_t n_pairs,
                                                    int32_t E, int32_t n_chunks) {
  extern __shared__ int32_t lds[];
  const int wave = threadIdx.x / MOE_WAVE;
  const int lane = threadIdx.x % MOE_WAVE;
  int32_t* hist = lds + wave * E;
  for (int e = lane; e < E; e += MOE_WAVE) hist[e] = 0;
  __builtin_amdgcn_wave_barrier();
  const int chunk = blockIdx.x * kWavesPerBlock + wave;
  if (chunk < n_chunks) {
    const int p0 = chunk * kLayoutChunk;
    int ids[kChunkIters];
    load_chunk(topk_idx, p0, min(p0 + kLayoutChunk, n_pairs), E, lane, ids);
    count_chunk(ids, E, hist);
  }
  __syncthreads();
  if (chunk < n_chunks) {
    for (int e = lane; e < E; e += MOE_WAVE) chunk_hist[(size_t)chunk * E + e] = hist[e];
  }
}

__global__ void __launch_bounds__(256) layout_scan_chunks(int32_t* __restrict__ chunk_hist,
                                                          int32_t* __restrict__ expert_counts,
                                                          int32_t E, int32_t n_chunks) {
  const int wave = threadIdx.x / MOE_WAVE;
  const int lane = threadIdx.x % MOE_WAVE;
  const int e = blockIdx.x * kWavesPerBlock + wave;
  if (e >= E) return;
  const int total = scan_column(chunk_hist, e, E, n_chunks, lane);
  if (lane == 0) expert_counts[e] = total;
}

// One block of 1024 threads; E <= 1024.
__global__ void __launch_bounds__(1024) layout_scan_experts(const int32_t* __restrict__ expert_counts,
                                                            int32_t* __restrict__ expert_offsets,
                                                            int32_t* __restrict__ rank_counts,
                                                            int32_t* __restrict__ rank_offsets, int32_t E,
                                                            int32_t ep_size, int32_t capacity) {
  __shared__ int32_t wave_tot[1024 / MOE_WAVE];
  __shared__ int32_t offs[1025];
  scan_experts(expert_counts, expert_offsets, rank_counts, rank_offsets, E, ep_size, capacity, wave_tot, offs);
}

__global__ void __launch_bounds__(256) layout_assign(const int32_t* __restrict__ topk_idx,
                                                     const int32_t* __restrict__ chunk_hist,
                                                     const int32_t* __restrict__ expert_offsets,
                                                     int32_t* __restrict__ pair_to_row,
                                                     int32_t* __restrict__ row_to_pair, int32_t n_pairs,
                                                     int32_t E, int32_t n_chunks, int32_t capacity,
                                                     int32_t key_bits) {
  extern __shared__ int32_t lds[];
  const int wave = threadIdx.x / MOE_WAVE;
  const int lane = threadIdx.x % MOE_WAVE;
  int32_t* running = lds + wave * E;
  const int chunk = blockIdx.x * kWavesPerBlock + wave;
  if (chunk >= n_chunks) return;  // whole wave leaves together; no block barrier follows
  const int p0 = chunk * kLayoutChunk, p1 = min(p0 + kLayoutChunk, n_pairs);
  int ids[kChunkIters];
  load_chunk(topk_idx, p0, p1, E, lane, ids);
  for (int e = lane; e < E; e += MOE_WAVE) running[e] = chunk_hist[(size_t)chunk * E + e];
  __builtin_amdgcn_wave_barrier();
  assign_chunk(ids, running, expert_offsets, pair_to_row, row_to_pair, p0, p1, E, capacity, key_bits, lane);
}

// All four steps in one block of 16 waves, the chunk histograms in LDS (n_chunks * E <= kFusedHist,
// n_chunks <= kFusedChunks): wave w takes chunks w, w + 16, ... in steps 1 and 4 (their ids stay in
// registers between the two) and experts w, w + 16, ... in step 2. The workspace is not touched.
constexpr int kFusedWaves = 16, kFusedChunks = 64, kFusedHist = 8192;
constexpr int kFusedPerWave = kFusedChunks / kFusedWaves;

__global__ void __launch_bounds__(kFusedWaves * MOE_WAVE) layout_fused(
    const int32_t* __restrict__ topk_idx, int32_t* __restrict__ expert_counts, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ rank_counts, int32_t* __restrict__ rank_offsets, int32_t* __restrict__ pair_to_row,
    int32_t* __restrict__ row_to_pair, int32_t n_pairs, int32_t E, int32_t ep_size, int32_t capacity,
    int32_t n_chunks, int32_t key_bits) {
  __shared__ int32_t hist[kFusedHist];
  __shared__ int32_t counts[1024];
  __shared__ int32_t offs[1025];
  __shared__ int32_t wave_tot[kFusedWaves];
  const int wave = threadIdx.x / MOE_WAVE;
  const int lane = threadIdx.x % MOE_WAVE;
  int ids[kFusedPerWave][kChunkIters];
#pragma unroll
  for (int j = 0; j < kFusedPerWave; ++j) {
    const int c = wave + j * kFusedWaves;
    if (c < n_chunks) load_chunk(topk_idx, c * kLayoutChunk, min(c * kLayoutChunk + kLayoutChunk, n_pairs), E, lane, ids[j]);
  }
  for (int i = threadIdx.x; i < n_chunks * E; i += kFusedWaves * MOE_WAVE) hist[i] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kFusedPerWave; ++j) {
    const int c = wave + j * kFusedWaves;
    if (c < n_chunks) count_chunk(ids[j], E, hist + c * E);
  }
  __syncthreads();
  for (int e = wave; e < E; e += kFusedWaves) {
    const int total = scan_column(hist, e, E, n_chunks, lane);
    if (lane == 0) {
      counts[e] = total;
      expert_counts[e] = total;
    }
  }
  __syncthreads();
  scan_experts(counts, expert_offsets, rank_counts, rank_offsets, E, ep_size, capacity, wave_tot, offs);
#pragma unroll
  for (int j = 0; j < kFusedPerWave; ++j) {
    const int c = wave + j * kFusedWaves;
    if (c < n_chunks)
      assign_chunk(ids[j], hist + c * E, offs, pair_to_row, row_to_pair, c * kLayoutChunk,
                   min(c * kLayoutChunk + kLayoutChunk, n_pairs), E, capacity, key_bits, lane);
  }
}

}  // namespace

size_t layout_ws_bytes(int32_t n_pairs, int32_t E) {
  const size_t n_chunks = (size_t)(n_pairs + kLayoutChunk - 1) / kLayoutChunk;
  return (n_chunks > 0 ? n_chunks : 1) * (size_t)E * sizeof(int32_t);
}

hipError_t layout_noalloc_scratch(int32_t** out) {
  // looked up once per device, with that device current, and kept: each GPU's copy of the array
  // sits at its own address
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static int32_t* ptr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = ptr[dev];
  return hipSuccess;
}

hipError_t launch_layout(const LayoutArgs& a, hipStream_t s) {
  const int n_chunks = (a.n_pairs + kLayoutChunk - 1) / kLayoutChunk;
  const int blocks = (n_chunks + kWavesPerBlock - 1) / kWavesPerBlock;
  const size_t lds = (size_t)kWavesPerBlock * a.E * sizeof(int32_t);
  int key_bits = 0;
  while ((1 << key_bits) <= a.E) ++key_bits;  // bits to hold 0..E (E = sentinel)
  if (n_chunks <= kFusedChunks && (long long)n_chunks * a.E <= kFusedHist) {
    hipLaunchKernelGGL(layout_fused, dim3(1), dim3(kFusedWaves * MOE_WAVE), 0, s, a.topk_idx, a.expert_counts,
                       a.expert_offsets, a.rank_counts, a.rank_offsets, a.pair_to_row, a.row_to_pair, a.n_pairs, a.E,
                       a.ep_size, a.capacity, n_chunks, key_bits);
    return hipGetLastError();
  }
  if (n_chunks > 0) {
    hipLaunchKernelGGL(layout_count, dim3(blocks), dim3(256), lds, s, a.topk_idx, a.chunk_hist, a.n_pairs, a.E,
                       n_chunks);
  }
  hipLaunchKernelGGL(layout_scan_chunks, dim3((a.E + kWavesPerBlock - 1) / kWavesPerBlock), dim3(256), 0, s,
                     a.chunk_hist, a.expert_counts, a.E, n_chunks);
  hipLaunchKernelGGL(layout_scan_experts, dim3(1), dim3(1024), 0, s, a.expert_counts, a.expert_offsets,
                     a.rank_counts, a.rank_offsets, a.E, a.ep_size, a.capacity);
  if (n_chunks > 0) {
    hipLaunchKernelGGL(layout_assign, dim3(blocks), dim3(256), lds, s, a.topk_idx, a.chunk_hist,
                       a.expert_offsets, a.pair_to_row, a.row_to_pair, a.n_pairs, a.E, n_chunks, a.capacity,
                       key_bits);
  }
  return hipGetLastError();
}

}  // namespace moe
