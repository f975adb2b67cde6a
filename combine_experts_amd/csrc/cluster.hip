// Cluster view of the layer on one GPU, and the padded capacity layout.
//
// "Expert Parallelism > All-to-All Communication": with E experts over n devices, device r owns
// experts [r*E/n, (r+1)*E/n); each device counts the pairs it sends to every other device (a row
// of the [source, destination] dispatch matrix). "Expert Parallelism and All-to-All", "The two
// exchanges": after the dispatch exchange a device holds one chunk per source, each sorted by its
// local experts, and regroups them per expert for the grouped GEMM; the combine exchange sends the
// outputs back the same way. On one GPU the exchange is a row gather from the concatenated send
// buffers of all emulated sources, fused with the regroup (one pass over the rows), and its
// reverse is a row scatter.
//
// EP-in-LLMs article, "Static Capacity Factors and Token Dropping": the fixed-capacity layout gives
// every expert C rows of an [E*C] buffer; kept pairs are the compact layout's (the first C pairs of
// each expert in pair order), the rest of each expert's C rows is zero padding that the expert FFN
// still computes.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kMatThreads = 1024;

// matrix[s, d] = pairs of source shard s (tokens [s*Ts, (s+1)*Ts)) routed to experts of rank d.
// One block per source shard; an LDS histogram of integer counts (any order gives the same sums).
__global__ void __launch_bounds__(kMatThreads) dispatch_matrix_kernel(const int32_t* __restrict__ topk_idx, int Ts,
                                                                    int k, int E, int n_dst,
                                                                    int32_t* __restrict__ matrix) {
  extern __shared__ int hist[];
  const int s = blockIdx.x;
  const int epr = E / n_dst;
  for (int d = threadIdx.x; d < n_dst; d += blockDim.x) hist[d] = 0;
  __syncthreads();
  const int32_t* idx = topk_idx + (size_t)s * Ts * k;
  const int n = Ts * k;
  for (int p = threadIdx.x; p < n; p += blockDim.x) {
    const int e = idx[p];
    if (e >= 0 && e < E) atomicAdd(&hist[e / epr], 1);
  }
  __syncthreads();
  for (int d = threadIdx.x; d < n_dst; d += blockDim.x) matrix[(size_t)s * n_dst + d] = hist[d];
}

// Receive layout of rank r. Every block rebuilds the small [n_src x epr] count tables in LDS, then
// maps its share of the regrouped rows: regrouped row g -> (local expert el, source s, index m)
// -> send-buffer row s*stride + src_off[s][r*epr + el] + m.
constexpr int kRecvThreads = 256;

__global__ void __launch_bounds__(kRecvThreads) recv_layout_kernel(const int32_t* __restrict__ src_off, int n_src,
                                                                 int E, int n_dst, int r, long long stride,
                                                                 int32_t* __restrict__ recv_counts,
                                                                 int32_t* __restrict__ exp_off_out,
                                                                 int32_t* __restrict__ g2s, int n_rows_max) {
  extern __shared__ int sh[];
  const int epr = E / n_dst;
  const int lo = r * epr;
  int* cnt = sh;                      // [epr][n_src] rows of (local expert, source)
  int* sp = cnt + epr * n_src;        // [epr][n_src] exclusive prefix over sources inside an expert
  int* eo = sp + epr * n_src;         // [epr + 1] regrouped expert offsets
  for (int i = threadIdx.x; i < epr * n_src; i += blockDim.x) {
    const int el = i / n_src, s = i % n_src;
    const int32_t* o = src_off + (size_t)s * (E + 1) + lo + el;
    cnt[i] = o[1] - o[0];
  }
  __syncthreads();
  for (int el = threadIdx.x; el < epr; el += blockDim.x) {
    int acc = 0;
    for (int s = 0; s < n_src; ++s) {
      sp[el * n_src + s] = acc;
      acc += cnt[el * n_src + s];
    }
    eo[el + 1] = acc;  // column total for now
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    eo[0] = 0;
    for (int el = 0; el < epr; ++el) eo[el + 1] += eo[el];
  }
  __syncthreads();
  const int total = eo[epr];
  if (blockIdx.x == 0) {
    for (int el = threadIdx.x; el <= epr; el += blockDim.x) exp_off_out[el] = eo[el];
    for (int s = threadIdx.x; s < n_src; s += blockDim.x) {
      int acc = 0;
      for (int el = 0; el < epr; ++el) acc += cnt[el * n_src + s];
      recv_counts[s] = acc;
    }
  }
  for (int g = blockIdx.x * blockDim.x + threadIdx.x; g < n_rows_max; g += gridDim.x * blockDim.x) {
    if (g >= total) {
      g2s[g] = -1;
      continue;
    }
    int a = 0, b = epr - 1;  // last el with eo[el] <= g
    while (a < b) {
      const int mid = (a + b + 1) >> 1;
      if (eo[mid] <= g) a = mid; else b = mid - 1;
    }
    const int el = a;
    const int local = g - eo[el];
    const int* spe = sp + el * n_src;
    int u = 0, v = n_src - 1;  // last s with spe[s] <= local and a non-empty run
    while (u < v) {
      const int mid = (u + v + 1) >> 1;
      if (spe[mid] <= local) u = mid; else v = mid - 1;
    }
    // sources with no rows share their prefix with the next one: the owner is the last of them
    const int s = u;
    const int m = local - spe[s];
    const long long row = (long long)s * stride + src_off[(size_t)s * (E + 1) + lo + el] + m;
    g2s[g] = (int32_t)row;
  }
}

// dst[i] = src[map[i]] (gather) or dst[map[i]] = src[i] (scatter) for map[i] >= 0; one wave per row,
// 16-byte non-temporal copies. row_chunks = row bytes / 16.
template <bool SCATTER>
__global__ void __launch_bounds__(256) move_rows_kernel(const u32x4* __restrict__ src, const int32_t* __restrict__ map,
                                                        long long n_rows, int row_chunks, u32x4* __restrict__ dst) {
  const int wave = threadIdx.x / MOE_WAVE, lane = threadIdx.x % MOE_WAVE;
  for (long long i = (long long)blockIdx.x * 4 + wave; i < n_rows; i += (long long)gridDim.x * 4) {
    const int m = map[i];
    if (m < 0) continue;
    const u32x4* s = src + (SCATTER ? i : (long long)m) * row_chunks;
    u32x4* d = dst + (SCATTER ? (long long)m : i) * row_chunks;
    for (int c = lane; c < row_chunks; c += MOE_WAVE) __builtin_nontemporal_store(__builtin_nontemporal_load(s + c), d + c);
  }
}

// pair_to_slot over pairs, slot_to_pair over slots, padded_offsets over experts.
__global__ void __launch_bounds__(256) padded_layout_kernel(const int32_t* __restrict__ topk_idx,
                                                          const int32_t* __restrict__ eoff,
                                                          const int32_t* __restrict__ p2r,
                                                          const int32_t* __restrict__ r2p, int P, int E, int C,
                                                          int32_t* __restrict__ p2s, int32_t* __restrict__ s2p,
                                                          int32_t* __restrict__ poff) {
  const long long n_slots = (long long)E * C;
  long long n = n_slots > P ? n_slots : P;
  if (n < E + 1) n = E + 1;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x) {
    if (i < P) {
      const int row = p2r[i];
      int slot = -1;
      if (row >= 0) {
        const int e = topk_idx[i];
        slot = e * C + (row - eoff[e]);
      }
      p2s[i] = slot;
    }
    if (i < n_slots) {
      const int e = (int)(i / C), m = (int)(i % C);
      const int kept = eoff[e + 1] - eoff[e];
      s2p[i] = m < kept ? r2p[eoff[e] + m] : -1;
    }
    if (i <= E) poff[i] = (int32_t)(i * C);
  }
}

// x_pad[s] = x[s2p[s] / k] for filled slots, zeros for padding; one wave per slot row.
__global__ void __launch_bounds__(256) permute_padded_kernel(const u32x4* __restrict__ x, const int32_t* __restrict__ s2p,
                                                           long long n_slots, int k, int row_chunks,
                                                           u32x4* __restrict__ xp) {
  const int wave = threadIdx.x / MOE_WAVE, lane = threadIdx.x % MOE_WAVE;
  for (long long i = (long long)blockIdx.x * 4 + wave; i < n_slots; i += (long long)gridDim.x * 4) {
    const int p = s2p[i];
    u32x4* d = xp + i * row_chunks;
    if (p < 0) {
      for (int c = lane; c < row_chunks; c += MOE_WAVE) __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u}, d + c);
    } else {
      const u32x4* s = x + (long long)(p / k) * row_chunks;
      for (int c = lane; c < row_chunks; c += MOE_WAVE) __builtin_nontemporal_store(__builtin_nontemporal_load(s + c), d + c);
    }
  }
}

unsigned rows_grid(long long n_rows) {
  const long long b = (n_rows + 3) / 4;
  return (unsigned)(b < 1 ? 1 : (b > 65536 ? 65536 : b));
}

}  // namespace

hipError_t launch_dispatch_matrix(const int32_t* topk_idx, int n_src, int Ts, int k, int E, int n_dst, int32_t* matrix,
                                  hipStream_t s) {
  hipLaunchKernelGGL(dispatch_matrix_kernel, dim3(n_src), dim3(kMatThreads), (size_t)n_dst * sizeof(int), s, topk_idx,
                     Ts, k, E, n_dst, matrix);
  return hipGetLastError();
}

size_t recv_layout_lds_bytes(int n_src, int epr) { return ((size_t)2 * epr * n_src + epr + 1) * sizeof(int); }

hipError_t launch_recv_layout(const int32_t* src_off, int n_src, int E, int n_dst, int r, long long stride,
                              int32_t* recv_counts, int32_t* exp_off, int32_t* g2s, int n_rows_max, hipStream_t s) {
  const int epr = E / n_dst;
  const long long blocks_ll = ((long long)n_rows_max + kRecvThreads - 1) / kRecvThreads;
  const unsigned blocks = (unsigned)(blocks_ll < 1 ? 1 : (blocks_ll > 4096 ? 4096 : blocks_ll));
  hipLaunchKernelGGL(recv_layout_kernel, dim3(blocks), dim3(kRecvThreads), recv_layout_lds_bytes(n_src, epr), s,
                     src_off, n_src, E, n_dst, r, stride, recv_counts, exp_off, g2s, n_rows_max);
  return hipGetLastError();
}

hipError_t launch_move_rows(bool scatter, const void* src, const int32_t* map, long long n_rows, int row_bytes,
                            void* dst, hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  const int chunks = row_bytes / 16;
  if (scatter)
    hipLaunchKernelGGL(move_rows_kernel<true>, dim3(rows_grid(n_rows)), dim3(256), 0, s, (const u32x4*)src, map,
                       n_rows, chunks, (u32x4*)dst);
  else
    hipLaunchKernelGGL(move_rows_kernel<false>, dim3(rows_grid(n_rows)), dim3(256), 0, s, (const u32x4*)src, map,
                       n_rows, chunks, (u32x4*)dst);
  return hipGetLastError();
}

hipError_t launch_padded_layout(const int32_t* topk_idx, const int32_t* eoff, const int32_t* p2r, const int32_t* r2p,
                                int P, int E, int C, int32_t* p2s, int32_t* s2p, int32_t* poff, hipStream_t s) {
  const long long n_slots = (long long)E * C;
  const long long n = (n_slots > P ? n_slots : P) + E + 1;
  const long long b = (n + 255) / 256;
  hipLaunchKernelGGL(padded_layout_kernel, dim3((unsigned)(b > 65536 ? 65536 : b)), dim3(256), 0, s, topk_idx, eoff,
                     p2r, r2p, P, E, C, p2s, s2p, poff);
  return hipGetLastError();
}

hipError_t launch_permute_padded(const void* x, const int32_t* s2p, long long n_slots, int k, int row_bytes, void* xp,
                                 hipStream_t s) {
  if (n_slots == 0) return hipSuccess;
  hipLaunchKernelGGL(permute_padded_kernel, dim3(rows_grid(n_slots)), dim3(256), 0, s, (const u32x4*)x, s2p, n_slots,
                     k, row_bytes / 16, (u32x4*)xp);
  return hipGetLastError();
}

}  // namespace moe
