// Backward of the one-GPU layer: everything except the grouped GEMMs (which live with the forward's
// in ffn.hip). The chain rule through the forward steps in reverse, the routing decision held fixed.
//
//   dy_perm[row(t,j)] = g[t,j] * dy[t]                 gather by pair_to_row, scaled by the gate
//   dgate[t,j]        = <dy[t], y_perm[row(t,j)]>      0 for a dropped pair
//   dl[t, :]          = gate backward of dgate          (softmax / sigmoid / full softmax)
//   dbias             = sum_t dl[t, :]
//   dW_g              = dl^T x
//   dx[t]             = sum_j dx_perm[row(t,j)] + sum_e dl[t,e] W_g[e]
//
// plus the transposes the weight-gradient GEMM and the data-gradient GEMMs read their operands from
// (both operands contiguous along the reduction index, as the matrix cores take them).
#include "moe_common.h"

namespace moe {
namespace {

template <typename T>
__device__ __forceinline__ float ld_f32(const T* p) {
  if constexpr (sizeof(T) == 2) return bf2f(*p);
  else return *p;
}
template <typename T>
__device__ __forceinline__ T st_cvt(float v) {
  if constexpr (sizeof(T) == 2) return f2bf(v);
  else return v;
}

// One wave per token: reads dy[t] once, writes its k gate-scaled rows and the k dot products; rows move
// in 16-byte chunks (8 bf16 or 4 float32).
template <typename T>
__global__ void __launch_bounds__(256) backward_combine_kernel(const T* __restrict__ dy, const int32_t* __restrict__ p2r,
                                                               const float* __restrict__ gate, const T* __restrict__ yp,
                                                               T* __restrict__ dyp, float* __restrict__ dgate, int T_,
                                                               int D, int k) {
  constexpr int VN = 16 / sizeof(T);
  const int wave = threadIdx.x / MOE_WAVE, lane = threadIdx.x % MOE_WAVE;
  const int nch = D / VN;
  for (int t = blockIdx.x * 4 + wave; t < T_; t += gridDim.x * 4) {
    const u32x4* dyr = reinterpret_cast<const u32x4*>(dy + (size_t)t * D);
    for (int j = 0; j < k; ++j) {
      const int row = p2r[(size_t)t * k + j];
      if (row < 0) {
        if (lane == 0) dgate[(size_t)t * k + j] = 0.f;
        continue;
      }
      const float g = gate[(size_t)t * k + j];
      const u32x4* yr = reinterpret_cast<const u32x4*>(yp + (size_t)row * D);
      u32x4* dr = reinterpret_cast<u32x4*>(dyp + (size_t)row * D);
      float dot = 0.f;
      for (int c = lane; c < nch; c += MOE_WAVE) {
        const u32x4 rv = dyr[c], ry = yr[c];
        const T* v = reinterpret_cast<const T*>(&rv);
        const T* w = reinterpret_cast<const T*>(&ry);
        u32x4 ro;
        T* o = reinterpret_cast<T*>(&ro);
#pragma unroll
        for (int i = 0; i < VN; ++i) {
          const float f = ld_f32(v + i);
          o[i] = st_cvt<T>(g * f);
          dot = fmaf(f, ld_f32(w + i), dot);
        }
        dr[c] = ro;
      }
      for (int off = MOE_WAVE / 2; off >= 1; off >>= 1) dot += __shfl_xor(dot, off, MOE_WAVE);
      if (lane == 0) dgate[(size_t)t * k + j] = dot;
    }
  }
}

// Gate backward, one wave per token; dl is a dense [T, E] float32 row (zeros where no gradient).
__global__ void __launch_bounds__(256) router_backward_kernel(const float* __restrict__ logits,
                                                              const int32_t* __restrict__ idx,
                                                              const float* __restrict__ gate,
                                                              const float* __restrict__ dgate, float* __restrict__ dl,
                                                              int T_, int E, int k, int mode) {
  const int wave = threadIdx.x / MOE_WAVE, lane = threadIdx.x % MOE_WAVE;
  for (int t = blockIdx.x * 4 + wave; t < T_; t += gridDim.x * 4) {
    const float* l = logits + (size_t)t * E;
    const int32_t* it = idx + (size_t)t * k;
    const float* gt = gate + (size_t)t * k;
    const float* dgt = dgate + (size_t)t * k;
    float* out = dl + (size_t)t * E;
    // sum_j g_j dg_j, in slot order on every lane
    float gdg = 0.f;
    for (int j = 0; j < k; ++j) gdg = fmaf(gt[j], dgt[j], gdg);
    if (mode == MOE_GATE_SOFTMAX_FULL) {
      float m = -INFINITY;
      for (int e = lane; e < E; e += MOE_WAVE) m = fmaxf(m, l[e]);
      for (int off = MOE_WAVE / 2; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, MOE_WAVE));
      float z = 0.f;
      for (int e = lane; e < E; e += MOE_WAVE) z += expf(l[e] - m);
      for (int off = MOE_WAVE / 2; off >= 1; off >>= 1) z += __shfl_xor(z, off, MOE_WAVE);
      for (int e = lane; e < E; e += MOE_WAVE) {
        float dp = 0.f;
        for (int j = 0; j < k; ++j)
          if (it[j] == e) dp = dgt[j];
        const float p = expf(l[e] - m) / z;
        out[e] = p * (dp - gdg);
      }
      continue;
    }
    float S = 0.f;  // sigmoid gates: sum of the selected experts' sigmoid scores
    if (mode == MOE_GATE_SIGMOID_TOPK)
      for (int j = 0; j < k; ++j)
        if (it[j] >= 0 && it[j] < E) S += 1.f / (1.f + expf(-l[it[j]]));
    // every column once: its gradient if the expert was selected, 0 otherwise
    for (int e = lane; e < E; e += MOE_WAVE) {
      int js = -1;
      for (int j = 0; j < k; ++j)
        if (it[j] == e) js = j;
      float v = 0.f;
      if (js >= 0) {
        if (mode == MOE_GATE_SIGMOID_TOPK) {
          const float sg = 1.f / (1.f + expf(-l[e]));
          v = sg * (1.f - sg) * (dgt[js] - gdg) / S;
        } else {
          v = gt[js] * (dgt[js] - gdg);
        }
      }
      out[e] = v;
    }
  }
}

// Column sums of a [rows, cols] float32 matrix in two fixed-order passes: block (cb, rb) sums rows
// [rb*chunk, ...) of 64 columns into part[rb][col]; then one thread per column adds the parts in order.
constexpr int kColChunk = 256;
__global__ void __launch_bounds__(256) colsum_part_kernel(const float* __restrict__ m, int rows, int cols,
                                                          float* __restrict__ part) {
  const int wave = threadIdx.x / MOE_WAVE, lane = threadIdx.x % MOE_WAVE;
  const int col = blockIdx.x * MOE_WAVE + lane, rb = blockIdx.y;
  __shared__ float s[4][MOE_WAVE];
  float acc = 0.f;
  if (col < cols) {
    const int r1 = min(rows, (rb + 1) * kColChunk);
    for (int r = rb * kColChunk + wave; r < r1; r += 4) acc += m[(size_t)r * cols + col];
  }
  s[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && col < cols) part[(size_t)rb * cols + col] = ((s[0][lane] + s[1][lane]) + s[2][lane]) + s[3][lane];
}
__global__ void __launch_bounds__(256) colsum_final_kernel(const float* __restrict__ part, int n_parts, int cols,
                                                           float* __restrict__ out) {
  const int col = blockIdx.x * blockDim.x + threadIdx.x;
  if (col >= cols) return;
  float acc = 0.f;
  for (int p = 0; p < n_parts; ++p) acc += part[(size_t)p * cols + col];
  out[col] = acc;
}

// C[m, n] = sum_k A[k, m] * B[k, n], A float32 [K, M], B [K, N] (T = bf16 or float32), C float32;
// 64 x 64 tiles, 16-deep K chunks through LDS, each thread 4 x 4 outputs. For dW_g = dl^T x.
template <typename T>
__global__ void __launch_bounds__(256) tn_f32_kernel(const float* __restrict__ A, const T* __restrict__ B, int K, int M,
                                                     int N, float* __restrict__ C) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * 256, kk = c / 64, col = c % 64;
      const int k = k0 + kk;
      As[kk][col] = (k < K && m0 + col < M) ? A[(size_t)k * M + m0 + col] : 0.f;
      Bs[kk][col] = (k < K && n0 + col < N) ? ld_f32(B + (size_t)k * N + n0 + col) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
      if (m < M && n < N) C[(size_t)m * N + n] = acc[i][j];
    }
}

// dW_g[e] = sum over the pairs (t, j) that selected e of dl[t, e] x[t], grouped by expert: rows
// [off[e], off[e+1]) of a dropless layout list those pairs (row_to_pair). Block (e, d-chunk of 64*VN
// columns); 4 waves split the rows round robin and are added in wave order: deterministic.
template <typename T>
__global__ void __launch_bounds__(256) router_wgrad_grouped_kernel(const T* __restrict__ x, const float* __restrict__ dl,
                                                                   const int32_t* __restrict__ off,
                                                                   const int32_t* __restrict__ r2p, int E, int D, int k,
                                                                   float* __restrict__ dwg) {
  constexpr int VN = 16 / sizeof(T);
  const int e = blockIdx.x;
  const int wave = threadIdx.x / MOE_WAVE, lane = threadIdx.x % MOE_WAVE;
  const int c = blockIdx.y * MOE_WAVE + lane;  // 16-byte chunk of the row
  const int nch = D / VN;
  __shared__ float part[4][MOE_WAVE * VN];
  float acc[VN];
#pragma unroll
  for (int i = 0; i < VN; ++i) acc[i] = 0.f;
  const int lo = off[e], hi = off[e + 1];
  if (c < nch) {
    for (int r = lo + wave; r < hi; r += 4) {
      const int t = r2p[r] / k;
      const float w = dl[(size_t)t * E + e];
      const u32x4 raw = reinterpret_cast<const u32x4*>(x + (size_t)t * D)[c];
      const T* v = reinterpret_cast<const T*>(&raw);
#pragma unroll
      for (int i = 0; i < VN; ++i) acc[i] = fmaf(w, ld_f32(v + i), acc[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < VN; ++i) part[wave][lane * VN + i] = acc[i];
  __syncthreads();
  for (int q = threadIdx.x; q < MOE_WAVE * VN; q += blockDim.x) {
    const int col = blockIdx.y * MOE_WAVE * VN + q;
    if (col < D) dwg[(size_t)e * D + col] = ((part[0][q] + part[1][q]) + part[2][q]) + part[3][q];
  }
}

// backward_combine_kernel for k <= KMAX: the token's rows, gates and the k dot products stay in
// registers, and for each group of U chunks per lane the dy chunks and all k y_perm chunks are loaded
// before the first FMA (k*U + U loads in flight per lane). Each lane accumulates its dot products over
// its chunks in the same order as backward_combine_kernel, so the same bits.
template <typename T, int KMAX, int U>
__global__ void __launch_bounds__(256) backward_combine_k_kernel(const T* __restrict__ dy, const int32_t* __restrict__ p2r,
                                                                 const float* __restrict__ gate,
                                                                 const T* __restrict__ yp, T* __restrict__ dyp,
                                                                 float* __restrict__ dgate, int T_, int D, int k) {
  constexpr int VN = 16 / sizeof(T);
  const int wave = threadIdx.x / MOE_WAVE, lane = threadIdx.x % MOE_WAVE;
  const int nch = D / VN;
  for (int t = blockIdx.x * 4 + wave; t < T_; t += gridDim.x * 4) {
    const u32x4* dyr = reinterpret_cast<const u32x4*>(dy + (size_t)t * D);
    int rows[KMAX];
    float g[KMAX], dot[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      rows[j] = j < k ? p2r[(size_t)t * k + j] : -1;
      g[j] = (rows[j] >= 0) ? gate[(size_t)t * k + j] : 0.f;
      dot[j] = 0.f;
    }
    for (int c0 = 0; c0 < nch; c0 += MOE_WAVE * U) {
      u32x4 rv[U], ry[KMAX][U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * MOE_WAVE + lane;
        rv[u] = c < nch ? dyr[c] : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + u * MOE_WAVE + lane;
          ry[j][u] = (rows[j] >= 0 && c < nch) ? reinterpret_cast<const u32x4*>(yp + (size_t)rows[j] * D)[c]
                                                : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (rows[j] < 0) continue;
        u32x4* dr = reinterpret_cast<u32x4*>(dyp + (size_t)rows[j] * D);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + u * MOE_WAVE + lane;
          if (c >= nch) continue;
          const T* v = reinterpret_cast<const T*>(&rv[u]);
          const T* w = reinterpret_cast<const T*>(&ry[j][u]);
          u32x4 ro;
          T* o = reinterpret_cast<T*>(&ro);
#pragma unroll
          for (int i = 0; i < VN; ++i) {
            const float f = ld_f32(v + i);
            o[i] = st_cvt<T>(g[j] * f);
            dot[j] = fmaf(f, ld_f32(w + i), dot[j]);
          }
          dr[c] = ro;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j >= k) break;
      float d = dot[j];
      for (int off = MOE_WAVE / 2; off >= 1; off >>= 1) d += __shfl_xor(d, off, MOE_WAVE);
      if (lane == 0) dgate[(size_t)t * k + j] = rows[j] >= 0 ? d : 0.f;
    }
  }
}

// dx[t] = sum over kept slots of dx_perm[row] + sum_e dl[t, e] W_g[e] (the selected experts, or all E
// under full-softmax gates), float32 sums in slot / expert order, one rounding. One wave per token,
// 16-byte chunks.
template <typename T>
__global__ void __launch_bounds__(256) backward_dx_kernel(const T* __restrict__ dxp, const int32_t* __restrict__ p2r,
                                                          const int32_t* __restrict__ idx, const float* __restrict__ dl,
                                                          const T* __restrict__ wg, T* __restrict__ dx, int T_, int D,
                                                          int E, int k, int all_experts) {
  constexpr int VN = 16 / sizeof(T);
  const int wave = threadIdx.x / MOE_WAVE, lane = threadIdx.x % MOE_WAVE;
  const int nch = D / VN;
  for (int t = blockIdx.x * 4 + wave; t < T_; t += gridDim.x * 4) {
    for (int c = lane; c < nch; c += MOE_WAVE) {
      float acc[VN];
#pragma unroll
      for (int i = 0; i < VN; ++i) acc[i] = 0.f;
      for (int j = 0; j < k; ++j) {
        const int row = p2r[(size_t)t * k + j];
        if (row < 0) continue;
        const u32x4 r = reinterpret_cast<const u32x4*>(dxp + (size_t)row * D)[c];
        const T* v = reinterpret_cast<const T*>(&r);
#pragma unroll
        for (int i = 0; i < VN; ++i) acc[i] += ld_f32(v + i);
      }
      const int n_r = all_experts ? E : k;
      for (int j = 0; j < n_r; ++j) {
        const int e = all_experts ? j : idx[(size_t)t * k + j];
        if (e < 0 || e >= E) continue;
        const float w = dl[(size_t)t * E + e];
        const u32x4 r = reinterpret_cast<const u32x4*>(wg + (size_t)e * D)[c];
        const T* v = reinterpret_cast<const T*>(&r);
#pragma unroll
        for (int i = 0; i < VN; ++i) acc[i] = fmaf(w, ld_f32(v + i), acc[i]);
      }
      u32x4 ro;
      T* o = reinterpret_cast<T*>(&ro);
#pragma unroll
      for (int i = 0; i < VN; ++i) o[i] = st_cvt<T>(acc[i]);
      reinterpret_cast<u32x4*>(dx + (size_t)t * D)[c] = ro;
    }
  }
}

// backward_dx_kernel for k <= KMAX with the selected experts only: rows, experts and dl weights in
// registers, and for each group of U chunks per lane the k dx_perm chunks and the k W_g chunks are
// loaded before the sums, which run in the same order as in backward_dx_kernel (same bits).
template <typename T, int KMAX, int U>
__global__ void __launch_bounds__(256) backward_dx_k_kernel(const T* __restrict__ dxp, const int32_t* __restrict__ p2r,
                                                            const int32_t* __restrict__ idx, const float* __restrict__ dl,
                                                            const T* __restrict__ wg, T* __restrict__ dx, int T_, int D,
                                                            int E, int k) {
  constexpr int VN = 16 / sizeof(T);
  const int wave = threadIdx.x / MOE_WAVE, lane = threadIdx.x % MOE_WAVE;
  const int nch = D / VN;
  for (int t = blockIdx.x * 4 + wave; t < T_; t += gridDim.x * 4) {
    int rows[KMAX], ex[KMAX];
    float w[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      rows[j] = j < k ? p2r[(size_t)t * k + j] : -1;
      const int e = j < k ? idx[(size_t)t * k + j] : -1;
      ex[j] = (e >= 0 && e < E) ? e : -1;
      w[j] = ex[j] >= 0 ? dl[(size_t)t * E + ex[j]] : 0.f;
    }
    for (int c0 = 0; c0 < nch; c0 += MOE_WAVE * U) {
      u32x4 rp[KMAX][U], rw[KMAX][U];
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + u * MOE_WAVE + lane;
          rp[j][u] = (rows[j] >= 0 && c < nch) ? reinterpret_cast<const u32x4*>(dxp + (size_t)rows[j] * D)[c]
                                                : u32x4{0u, 0u, 0u, 0u};
          rw[j][u] = (ex[j] >= 0 && c < nch) ? reinterpret_cast<const u32x4*>(wg + (size_t)ex[j] * D)[c]
                                              : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * MOE_WAVE + lane;
        if (c >= nch) continue;
        float acc[VN];
#pragma unroll
        for (int i = 0; i < VN; ++i) acc[i] = 0.f;
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
          if (rows[j] < 0) continue;
          const T* v = reinterpret_cast<const T*>(&rp[j][u]);
#pragma unroll
          for (int i = 0; i < VN; ++i) acc[i] += ld_f32(v + i);
        }
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
          if (ex[j] < 0) continue;
          const T* v = reinterpret_cast<const T*>(&rw[j][u]);
#pragma unroll
          for (int i = 0; i < VN; ++i) acc[i] = fmaf(w[j], ld_f32(v + i), acc[i]);
        }
        u32x4 ro;
        T* o = reinterpret_cast<T*>(&ro);
#pragma unroll
        for (int i = 0; i < VN; ++i) o[i] = st_cvt<T>(acc[i]);
        reinterpret_cast<u32x4*>(dx + (size_t)t * D)[c] = ro;
      }
    }
  }
}

// Batched transpose through 64 x 64 LDS tiles: dst[b][c][col_off + r] = src[b][r][c] (dst rows of
// ld_dst elements), for r < R, c < C. Global reads and writes move 16 bytes per lane; the tile is
// transposed on its way into LDS ([c][r] rows padded by one 16-byte chunk). Requires C % VN == 0.
template <typename T>
__global__ void __launch_bounds__(256) transpose_kernel(const T* __restrict__ src, int R, int C, long long src_batch,
                                                        T* __restrict__ dst, long long ld_dst, long long dst_batch,
                                                        int col_off) {
  constexpr int VN = 16 / sizeof(T), CPR = 64 / VN;  // elements per chunk, chunks per 64-wide row
  __shared__ __attribute__((aligned(16))) T tile[64][64 + VN];
  const int b = blockIdx.z, r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const T* s = src + b * src_batch;
  T* d = dst + b * dst_batch;
  const int tid = threadIdx.x;
  for (int q = tid; q < 64 * CPR; q += 256) {
    const int rl = q / CPR, cc = q % CPR;
    const int r = r0 + rl, c = c0 + cc * VN;
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (r < R && c < C) raw = *reinterpret_cast<const u32x4*>(s + (size_t)r * C + c);
    const T* v = reinterpret_cast<const T*>(&raw);
#pragma unroll
    for (int i = 0; i < VN; ++i) tile[cc * VN + i][rl] = v[i];
  }
  __syncthreads();
  for (int q = tid; q < 64 * CPR; q += 256) {
    const int cl = q / CPR, rc = q % CPR;
    const int c = c0 + cl, r = r0 + rc * VN;
    if (c >= C || r >= R) continue;
    T* out = d + (size_t)c * ld_dst + col_off + r;
    if (r + VN <= R && ((col_off + r) % VN) == 0 && (ld_dst % VN) == 0) {
      *reinterpret_cast<u32x4*>(out) = *reinterpret_cast<const u32x4*>(&tile[cl][rc * VN]);
    } else {
      for (int i = 0; i < VN && r + i < R; ++i) out[i] = tile[cl][rc * VN + i];
    }
  }
}

// Padded group offsets: koff[g] = sum over g' < g of roundup64(off[g'+1] - off[g']). One block.
__global__ void __launch_bounds__(256) group_koff_kernel(const int32_t* __restrict__ off, int G,
                                                         int32_t* __restrict__ koff) {
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int g = 0; g < G; ++g) {
      koff[g] = acc;
      acc += (off[g + 1] - off[g] + 63) / 64 * 64;
    }
    koff[G] = acc;
  }
}

// dst[c][koff[g] + j] = src[off[g] + j][c] for j < count_g, 0 for count_g <= j < padded count;
// 64-column tiles of the padded axis (each inside one group, as the padded groups are 64-aligned) x
// 64-row tiles of c, 16-byte global reads and writes. Requires C % VN == 0. With gidx, source row
// off[g] + j is src row gidx[off[g] + j] / gdiv instead (the permute fused into the transpose).
template <typename T>
__global__ void __launch_bounds__(256) group_transpose_kernel(const T* __restrict__ src, int C,
                                                              const int32_t* __restrict__ off,
                                                              const int32_t* __restrict__ koff, int G,
                                                              T* __restrict__ dst, long long ld,
                                                              const int32_t* __restrict__ gidx, int gdiv) {
  constexpr int VN = 16 / sizeof(T), CPR = 64 / VN;
  __shared__ __attribute__((aligned(16))) T tile[64][64 + VN];
  const int j0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int total = koff[G];
  if (j0 >= total) return;
  int a = 0, b = G - 1;  // last g with koff[g] <= j0
  while (a < b) {
    const int mid = (a + b + 1) >> 1;
    if (koff[mid] <= j0) a = mid; else b = mid - 1;
  }
  const int g = a;
  const int cnt = off[g + 1] - off[g], base = off[g] + (j0 - koff[g]);
  const int valid = cnt - (j0 - koff[g]);  // rows of this tile that exist (may be <= 0)
  const int tid = threadIdx.x;
  for (int q = tid; q < 64 * CPR; q += 256) {
    const int jl = q / CPR, cc = q % CPR;
    const int c = c0 + cc * VN;
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (jl < valid && c < C) {
      const size_t srow = gidx ? (size_t)(gidx[base + jl] / gdiv) : (size_t)(base + jl);
      raw = *reinterpret_cast<const u32x4*>(src + srow * C + c);
    }
    const T* v = reinterpret_cast<const T*>(&raw);
#pragma unroll
    for (int i = 0; i < VN; ++i) tile[cc * VN + i][jl] = v[i];
  }
  __syncthreads();
  for (int q = tid; q < 64 * CPR; q += 256) {
    const int cl = q / CPR, jc = q % CPR;
    const int c = c0 + cl;
    if (c < C)
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(&tile[cl][jc * VN]),
                                  reinterpret_cast<u32x4*>(dst + (size_t)c * ld + j0 + jc * VN));
  }
}

unsigned tok_grid(int T_) {
  const int b = (T_ + 3) / 4;
  return (unsigned)(b < 1 ? 1 : (b > 65535 ? 65535 : b));
}

}  // namespace

hipError_t launch_backward_combine(const void* dy, const int32_t* p2r, const float* gate, const void* yp, void* dyp,
                                   float* dgate, int T, int D, int k, int dtype, hipStream_t s) {
  if (T == 0) return hipSuccess;
#define MOE_BWC_K(TT, KM, UU)                                                                                       \
  hipLaunchKernelGGL((backward_combine_k_kernel<TT, KM, UU>), dim3(tok_grid(T)), dim3(256), 0, s, (const TT*)dy, p2r, \
                     gate, (const TT*)yp, (TT*)dyp, dgate, T, D, k)
  if (dtype == MOE_BF16) {
    if (k <= 2) MOE_BWC_K(bf16_t, 2, 4);
    else if (k <= 4) MOE_BWC_K(bf16_t, 4, 2);
    else if (k <= 8) MOE_BWC_K(bf16_t, 8, 2);
    else
      hipLaunchKernelGGL(backward_combine_kernel<bf16_t>, dim3(tok_grid(T)), dim3(256), 0, s, (const bf16_t*)dy, p2r,
                         gate, (const bf16_t*)yp, (bf16_t*)dyp, dgate, T, D, k);
  } else {
    if (k <= 2) MOE_BWC_K(float, 2, 4);
    else if (k <= 4) MOE_BWC_K(float, 4, 2);
    else if (k <= 8) MOE_BWC_K(float, 8, 2);
    else
      hipLaunchKernelGGL(backward_combine_kernel<float>, dim3(tok_grid(T)), dim3(256), 0, s, (const float*)dy, p2r,
                         gate, (const float*)yp, (float*)dyp, dgate, T, D, k);
  }
#undef MOE_BWC_K
  return hipGetLastError();
}

hipError_t launch_router_backward(const float* logits, const int32_t* idx, const float* gate, const float* dgate,
                                  float* dl, int T, int E, int k, int mode, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(router_backward_kernel, dim3(tok_grid(T)), dim3(256), 0, s, logits, idx, gate, dgate, dl, T, E, k,
                     mode);
  return hipGetLastError();
}

size_t colsum_ws_bytes(int rows, int cols) {
  return (size_t)((rows + kColChunk - 1) / kColChunk) * cols * sizeof(float);
}

hipError_t launch_colsum(const float* m, int rows, int cols, float* part, float* out, hipStream_t s) {
  const int nparts = (rows + kColChunk - 1) / kColChunk;
  if (nparts > 0)
    hipLaunchKernelGGL(colsum_part_kernel, dim3((cols + MOE_WAVE - 1) / MOE_WAVE, nparts), dim3(256), 0, s, m, rows,
                       cols, part);
  hipLaunchKernelGGL(colsum_final_kernel, dim3((cols + 255) / 256), dim3(256), 0, s, part, nparts, cols, out);
  return hipGetLastError();
}

hipError_t launch_tn_f32(const float* A, const void* B, int dtype, int K, int M, int N, float* C, hipStream_t s) {
  const dim3 grid((N + 63) / 64, (M + 63) / 64);
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(tn_f32_kernel<bf16_t>, grid, dim3(256), 0, s, A, (const bf16_t*)B, K, M, N, C);
  else
    hipLaunchKernelGGL(tn_f32_kernel<float>, grid, dim3(256), 0, s, A, (const float*)B, K, M, N, C);
  return hipGetLastError();
}

hipError_t launch_router_wgrad_grouped(const void* x, const float* dl, const int32_t* off, const int32_t* r2p, int E,
                                       int D, int k, int dtype, float* dwg, hipStream_t s) {
  const int VN = dtype == MOE_BF16 ? 8 : 4;
  const dim3 grid(E, (D / VN + MOE_WAVE - 1) / MOE_WAVE);
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(router_wgrad_grouped_kernel<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)x, dl, off, r2p, E, D,
                       k, dwg);
  else
    hipLaunchKernelGGL(router_wgrad_grouped_kernel<float>, grid, dim3(256), 0, s, (const float*)x, dl, off, r2p, E, D, k,
                       dwg);
  return hipGetLastError();
}

hipError_t launch_backward_dx(const void* dxp, const int32_t* p2r, const int32_t* idx, const float* dl, const void* wg,
                              void* dx, int T, int D, int E, int k, int all_experts, int dtype, hipStream_t s) {
  if (T == 0) return hipSuccess;
#define MOE_BDX_K(TT, KM, UU)                                                                                       \
  hipLaunchKernelGGL((backward_dx_k_kernel<TT, KM, UU>), dim3(tok_grid(T)), dim3(256), 0, s, (const TT*)dxp, p2r, idx, \
                     dl, (const TT*)wg, (TT*)dx, T, D, E, k)
  if (!all_experts && k <= 8) {
    if (dtype == MOE_BF16) {
      if (k <= 2) MOE_BDX_K(bf16_t, 2, 2);
      else if (k <= 4) MOE_BDX_K(bf16_t, 4, 2);
      else MOE_BDX_K(bf16_t, 8, 1);
    } else {
      if (k <= 2) MOE_BDX_K(float, 2, 2);
      else if (k <= 4) MOE_BDX_K(float, 4, 2);
      else MOE_BDX_K(float, 8, 1);
    }
    return hipGetLastError();
  }
#undef MOE_BDX_K
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(backward_dx_kernel<bf16_t>, dim3(tok_grid(T)), dim3(256), 0, s, (const bf16_t*)dxp, p2r, idx, dl,
                       (const bf16_t*)wg, (bf16_t*)dx, T, D, E, k, all_experts);
  else
    hipLaunchKernelGGL(backward_dx_kernel<float>, dim3(tok_grid(T)), dim3(256), 0, s, (const float*)dxp, p2r, idx, dl,
                       (const float*)wg, (float*)dx, T, D, E, k, all_experts);
  return hipGetLastError();
}

hipError_t launch_transpose(const void* src, int B, int R, int C, long long src_batch, void* dst, long long ld_dst,
                            long long dst_batch, int col_off, int dtype, hipStream_t s) {
  if (B == 0 || R == 0 || C == 0) return hipSuccess;
  const dim3 grid((C + 63) / 64, (R + 63) / 64, B);
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(transpose_kernel<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)src, R, C, src_batch,
                       (bf16_t*)dst, ld_dst, dst_batch, col_off);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, s, (const float*)src, R, C, src_batch, (float*)dst,
                       ld_dst, dst_batch, col_off);
  return hipGetLastError();
}

hipError_t launch_group_koff(const int32_t* off, int G, int32_t* koff, hipStream_t s) {
  hipLaunchKernelGGL(group_koff_kernel, dim3(1), dim3(256), 0, s, off, G, koff);
  return hipGetLastError();
}

hipError_t launch_group_transpose(const void* src, int C, const int32_t* off, const int32_t* koff, int G,
                                  long long ld, void* dst, int dtype, hipStream_t s, const int32_t* gidx, int gdiv) {
  if (ld == 0 || C == 0) return hipSuccess;
  const dim3 grid((unsigned)((ld + 63) / 64), (C + 63) / 64);
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(group_transpose_kernel<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)src, C, off, koff, G,
                       (bf16_t*)dst, ld, gidx, gdiv);
  else
    hipLaunchKernelGGL(group_transpose_kernel<float>, grid, dim3(256), 0, s, (const float*)src, C, off, koff, G,
                       (float*)dst, ld, gidx, gdiv);
  return hipGetLastError();
}

}  // namespace moe
