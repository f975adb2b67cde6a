// Dispatch layout: per-expert counts, capacity cut, per-expert and per-rank offsets, and the stable
// (expert, pair id) permutation.
//
// The pages' dispatch step ("Expert Parallelism and All-to-All", section on the two exchanges; the
// EP-in-LLMs article, pipeline steps 1-2; the all-to-all article's dispatch example with
// destination = expert / experts_per_device and per-device bincount) groups each device's
// (token, expert) pairs contiguously by destination. Here the grouping is by expert, stable in
// pair id, which is also grouping by rank because ranks own contiguous expert blocks.
//
// Four small kernels, none of whose results depend on thread scheduling:
//   1. count       one wave per chunk of kLayoutChunk pairs: per-chunk expert histogram
//   2. scan_chunks one wave per expert: exclusive scan of the expert's chunk histogram column
//                  -> each chunk's first rank inside the expert; the column total is the count
//   3. scan_exp    one block: capacity cut, exclusive scan over experts, per-rank counts/offsets
//   4. assign      one wave per chunk, pairs visited in pair-id order 64 at a time: a pair's rank
//                  inside its expert = chunk base + earlier same-expert pairs of the chunk
//                  (wave ballots find same-expert lanes); row = offset + rank if rank < capacity.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kWavesPerBlock = 4;

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
    const int p1 = min(p0 + kLayoutChunk, n_pairs);
    for (int p = p0 + lane; p < p1; p += MOE_WAVE) {
      const int e = topk_idx[p];
      if (e >= 0 && e < E) atomicAdd(&hist[e], 1);  // an id outside [0,E) counts nowhere
    }
  }
  __syncthreads();
  if (chunk < n_chunks) {
    for (int e = lane; e < E; e += MOE_WAVE) chunk_hist[(size_t)chunk * E + e] = hist[e];
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

__global__ void __launch_bounds__(256) layout_scan_chunks(int32_t* __restrict__ chunk_hist,
                                                          int32_t* __restrict__ expert_counts,
                                                          int32_t E, int32_t n_chunks) {
  const int wave = threadIdx.x / MOE_WAVE;
  const int lane = threadIdx.x % MOE_WAVE;
  const int e = blockIdx.x * kWavesPerBlock + wave;
  if (e >= E) return;
  int carry = 0;
  for (int c0 = 0; c0 < n_chunks; c0 += MOE_WAVE) {
    const int c = c0 + lane;
    const int v = (c < n_chunks) ? chunk_hist[(size_t)c * E + e] : 0;
    const int inc = wave_inclusive_scan(v);
    if (c < n_chunks) chunk_hist[(size_t)c * E + e] = carry + inc - v;  // exclusive base
    carry += __shfl(inc, MOE_WAVE - 1, MOE_WAVE);
  }
  if (lane == 0) expert_counts[e] = carry;
}

// One block of 1024 threads; E <= 1024.
__global__ void __launch_bounds__(1024) layout_scan_experts(const int32_t* __restrict__ expert_counts,
                                                            int32_t* __restrict__ expert_offsets,
                                                            int32_t* __restrict__ rank_counts,
                                                            int32_t* __restrict__ rank_offsets, int32_t E,
                                                            int32_t ep_size, int32_t capacity) {
  __shared__ int32_t wave_tot[1024 / MOE_WAVE];
  __shared__ int32_t offs[1025];
  const int t = threadIdx.x;
  const int lane = t % MOE_WAVE, wave = t / MOE_WAVE;
  const int kept = (t < E) ? min(expert_counts[t], capacity) : 0;
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
  for (int e = lane; e < E; e += MOE_WAVE) running[e] = chunk_hist[(size_t)chunk * E + e];
  __builtin_amdgcn_wave_barrier();
  const int n_kept = expert_offsets[E];
  const int p0 = chunk * kLayoutChunk;
  const int p1 = min(p0 + kLayoutChunk, n_pairs);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (MOE_WAVE - lane));
  for (int pb = p0; pb < p1; pb += MOE_WAVE) {
    const int p = pb + lane;
    const bool in_chunk = p < p1;
    const int raw = in_chunk ? topk_idx[p] : E;
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
        const int row = expert_offsets[key] + rank;
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

}  // namespace

size_t layout_ws_bytes(int32_t n_pairs, int32_t E) {
  const size_t n_chunks = (size_t)(n_pairs + kLayoutChunk - 1) / kLayoutChunk;
  return (n_chunks > 0 ? n_chunks : 1) * (size_t)E * sizeof(int32_t);
}

hipError_t launch_layout(const LayoutArgs& a, hipStream_t s) {
  const int n_chunks = (a.n_pairs + kLayoutChunk - 1) / kLayoutChunk;
  const int blocks = (n_chunks + kWavesPerBlock - 1) / kWavesPerBlock;
  const size_t lds = (size_t)kWavesPerBlock * a.E * sizeof(int32_t);
  int key_bits = 0;
  while ((1 << key_bits) <= a.E) ++key_bits;  // bits to hold 0..E (E = sentinel)
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
