// Permute (dispatch side) and unpermute + combine (combine side) of the one-GPU MoE layer.
//
// EP-in-LLMs article, "The Execution Pipeline": step 2 reorders each token's k copies into
// contiguous per-expert / per-rank buffers; step 6 restores token order, scales each of the k
// expert outputs by its gate and sums them. On one GPU the send buffer of step 2 is also the
// receive buffer of step 4, so the two all-to-alls of steps 3 and 5 move nothing.
//
// Both kernels are HBM-bound row copies: one wave per token, 16-byte accesses, several chunks in
// flight per lane. Permute reads each x row once and writes it to its k rows; combine reads the k
// rows of a token, sums gate * row in float32 in slot order and rounds once.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kWaves = 4;
constexpr int kUnroll = 4;
constexpr int kCmbWaves = 2;  // waves (tokens in flight) per block of the k-rows-in-registers combine

template <typename T>
struct Vec;
template <>
struct Vec<bf16_t> {
  static constexpr int N = 8;
};
template <>
struct Vec<float> {
  static constexpr int N = 4;
};

__global__ void __launch_bounds__(256) permute_kernel(const u32x4* __restrict__ x, const int32_t* __restrict__ p2r,
                                                      u32x4* __restrict__ xp, int T, int row_chunks, int k) {
  const int wave = threadIdx.x / MOE_WAVE, lane = threadIdx.x % MOE_WAVE;
  for (int t = blockIdx.x * kWaves + wave; t < T; t += gridDim.x * kWaves) {
    const u32x4* src = x + (size_t)t * row_chunks;
    for (int c0 = 0; c0 < row_chunks; c0 += MOE_WAVE * kUnroll) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int c = c0 + u * MOE_WAVE + lane;
        if (c < row_chunks) v[u] = __builtin_nontemporal_load(src + c);
      }
      for (int j = 0; j < k; ++j) {
        const int row = p2r[(size_t)t * k + j];
        if (row < 0) continue;
        u32x4* dst = xp + (size_t)row * row_chunks;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const int c = c0 + u * MOE_WAVE + lane;
          if (c < row_chunks) dst[c] = v[u];
        }
      }
    }
  }
}

// ADD: y[t] also takes add[t] (a shared expert's output), summed in float32 after the k slots and
// before the one rounding.
template <typename T, bool ADD>
__global__ void __launch_bounds__(256) combine_kernel(const T* __restrict__ yp, const int32_t* __restrict__ p2r,
                                                      const float* __restrict__ gate, const T* __restrict__ add,
                                                      T* __restrict__ y, int T_, int D, int k) {
  constexpr int VN = Vec<T>::N;
  const int wave = threadIdx.x / MOE_WAVE, lane = threadIdx.x % MOE_WAVE;
  const int row_chunks = D / VN;
  for (int t = blockIdx.x * kWaves + wave; t < T_; t += gridDim.x * kWaves) {
    for (int c0 = 0; c0 < row_chunks; c0 += MOE_WAVE * kUnroll) {
      float acc[kUnroll][VN];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int i = 0; i < VN; ++i) acc[u][i] = 0.f;
      for (int j = 0; j < k; ++j) {
        const int row = p2r[(size_t)t * k + j];
        if (row < 0) continue;
        const float g = gate[(size_t)t * k + j];
        const T* src = yp + (size_t)row * D;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const int c = c0 + u * MOE_WAVE + lane;
          if (c < row_chunks) {
            const u32x4 raw = *reinterpret_cast<const u32x4*>(src + (size_t)c * VN);
            const T* e = reinterpret_cast<const T*>(&raw);
#pragma unroll
            for (int i = 0; i < VN; ++i) acc[u][i] = fmaf(g, to_f32<T>(e[i]), acc[u][i]);
          }
        }
      }
      if constexpr (ADD) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const int c = c0 + u * MOE_WAVE + lane;
          if (c < row_chunks) {
            const u32x4 raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(add + (size_t)t * D) + c);
            const T* e = reinterpret_cast<const T*>(&raw);
#pragma unroll
            for (int i = 0; i < VN; ++i) acc[u][i] += to_f32<T>(e[i]);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int c = c0 + u * MOE_WAVE + lane;
        if (c < row_chunks) {
          u32x4 raw;
          T* e = reinterpret_cast<T*>(&raw);
#pragma unroll
          for (int i = 0; i < VN; ++i) e[i] = from_f32<T>(acc[u][i]);
          __builtin_nontemporal_store(raw, reinterpret_cast<u32x4*>(y + (size_t)t * D) + c);
        }
      }
    }
  }
}

// Combine for k <= KMAX: the token's rows and gates are read once; for each group of U chunks per lane
// all k rows' loads are issued before the first FMA, so k*U 16-byte loads are in flight per lane
// (the k rows of a token sit in unrelated places of y_perm). Same slot-order float32 sums as
// combine_kernel, so the same bits. Blocks of two waves; the output rows go out with ordinary stores
// (measured against non-temporal stores and 4- or 8-wave blocks: 4.5 % faster at k = 8, 8 % at k = 2,
// with 4 chunks per lane at k = 8 and 8 at k = 2).
template <typename T, bool ADD, int KMAX, int U>
__global__ void __launch_bounds__(kCmbWaves * MOE_WAVE) combine_k_kernel(const T* __restrict__ yp, const int32_t* __restrict__ p2r,
                                                        const float* __restrict__ gate, const T* __restrict__ add,
                                                        T* __restrict__ y, int T_, int D, int k) {
  constexpr int VN = Vec<T>::N;
  const int wave = threadIdx.x / MOE_WAVE, lane = threadIdx.x % MOE_WAVE;
  const int row_chunks = D / VN;
  for (int t = blockIdx.x * kCmbWaves + wave; t < T_; t += gridDim.x * kCmbWaves) {
    int rows[KMAX];
    float g[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      rows[j] = j < k ? p2r[(size_t)t * k + j] : -1;
      g[j] = j < k ? gate[(size_t)t * k + j] : 0.f;
    }
    for (int c0 = 0; c0 < row_chunks; c0 += MOE_WAVE * U) {
      u32x4 raw[KMAX][U];
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + u * MOE_WAVE + lane;
          raw[j][u] = (rows[j] >= 0 && c < row_chunks)
                          ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(yp + (size_t)rows[j] * D) + c)
                          : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * MOE_WAVE + lane;
        float acc[VN];
#pragma unroll
        for (int i = 0; i < VN; ++i) acc[i] = 0.f;
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
          if (rows[j] < 0) continue;
          const T* e = reinterpret_cast<const T*>(&raw[j][u]);
#pragma unroll
          for (int i = 0; i < VN; ++i) acc[i] = fmaf(g[j], to_f32<T>(e[i]), acc[i]);
        }
        if (c < row_chunks) {
          if constexpr (ADD) {
            const u32x4 ra = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(add + (size_t)t * D) + c);
            const T* e = reinterpret_cast<const T*>(&ra);
#pragma unroll
            for (int i = 0; i < VN; ++i) acc[i] += to_f32<T>(e[i]);
          }
          u32x4 o;
          T* oe = reinterpret_cast<T*>(&o);
#pragma unroll
          for (int i = 0; i < VN; ++i) oe[i] = from_f32<T>(acc[i]);
          reinterpret_cast<u32x4*>(y + (size_t)t * D)[c] = o;
        }
      }
    }
  }
}

int grid_for(int T, int waves = kWaves) {
  const int blocks = (T + waves - 1) / waves;
  return blocks < 65535 * 4 ? blocks : 65535 * 4;
}

}  // namespace

hipError_t launch_permute(const void* x, const int32_t* pair_to_row, void* x_perm, int32_t T, int32_t D, int32_t k,
                          int dtype, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int elem = dtype == MOE_BF16 ? 2 : 4;
  const int row_chunks = D * elem / 16;
  hipLaunchKernelGGL(permute_kernel, dim3(grid_for(T)), dim3(256), 0, s, (const u32x4*)x, pair_to_row,
                     (u32x4*)x_perm, T, row_chunks, k);
  return hipGetLastError();
}

template <typename T, bool ADD>
bool launch_combine_k(const void* y_perm, const int32_t* pair_to_row, const float* gate, const void* add, void* y,
                      int32_t T_, int32_t D, int32_t k, hipStream_t s) {
#define MOE_COMBINE_K(KM, UU)                                                                                    \
  hipLaunchKernelGGL((combine_k_kernel<T, ADD, KM, UU>), dim3(grid_for(T_, kCmbWaves)), dim3(kCmbWaves * MOE_WAVE), \
                     0, s, (const T*)y_perm, pair_to_row, gate, (const T*)add, (T*)y, T_, D, k)
  if (k <= 2) MOE_COMBINE_K(2, 8);
  else if (k <= 4) MOE_COMBINE_K(4, 2);
  else if (k <= 8) MOE_COMBINE_K(8, 4);
  else return false;
#undef MOE_COMBINE_K
  return true;
}

template <typename T>
void launch_combine_t(const void* y_perm, const int32_t* pair_to_row, const float* gate, const void* add, void* y,
                      int32_t T_, int32_t D, int32_t k, hipStream_t s) {
  if (add != nullptr ? launch_combine_k<T, true>(y_perm, pair_to_row, gate, add, y, T_, D, k, s)
                     : launch_combine_k<T, false>(y_perm, pair_to_row, gate, add, y, T_, D, k, s))
    return;
  if (add != nullptr)
    hipLaunchKernelGGL((combine_kernel<T, true>), dim3(grid_for(T_)), dim3(256), 0, s, (const T*)y_perm, pair_to_row,
                       gate, (const T*)add, (T*)y, T_, D, k);
  else
    hipLaunchKernelGGL((combine_kernel<T, false>), dim3(grid_for(T_)), dim3(256), 0, s, (const T*)y_perm, pair_to_row,
                       gate, nullptr, (T*)y, T_, D, k);
}

hipError_t launch_combine(const void* y_perm, const int32_t* pair_to_row, const float* gate, const void* add, void* y,
                          int32_t T, int32_t D, int32_t k, int dtype, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (dtype == MOE_BF16) launch_combine_t<bf16_t>(y_perm, pair_to_row, gate, add, y, T, D, k, s);
  else launch_combine_t<float>(y_perm, pair_to_row, gate, add, y, T, D, k, s);
  return hipGetLastError();
}

}  // namespace moe
