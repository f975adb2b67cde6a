// Grouped expert FFN: one GEMM per expert over that expert's contiguous rows, sizes read on device.
//
// EP-in-LLMs article, "The Execution Pipeline" step 4: all rows bound for one local expert are
// packed into one batched GEMM; the expert is W2 * (SiLU(W1 h) (*) (W3 h)) (read as SwiGLU: SiLU of
// W1 h alone). Its "dropless" section: ragged grouped GEMMs over exact per-expert counts, no
// padding rows and no dropped tokens. GELU experts ("Communication Overhead Analysis": two matrix
// products per token) use W2 * GELU(W1 h).
//
// Two launches per FFN:
//   up:   h[r, :]      = act(x_perm[r] · W1[e]^T, x_perm[r] · W3[e]^T)    (K = D, Nout = F)
//   down: y_perm[r, :] = h[r] · W2[e]^T                                   (K = F, Nout = D)
// Both operands are contiguous along K (weights are (out, in)), which is what the matrix cores
// want: each lane feeds 8 consecutive K elements (16 bytes) per operand per instruction.
//
// Tile map: blockIdx.y = output column tile, blockIdx.x = a slot in the concatenation of every
// expert's row tiles. Each block derives its (expert, row tile) from expert_offsets with a block
// scan of ceil(rows_e / BM); slots past the last tile exit. The grid is sized for the worst case
// (N_max / BM + E slots), so the host never reads counts.
#include "moe_common.h"

namespace moe {
namespace {

// Block-wide exclusive scan (256 threads); returns the exclusive prefix, sets *total.
__device__ __forceinline__ int block_scan_256(int v, int* lds4, int* total) {
  const int lane = threadIdx.x % MOE_WAVE, wave = threadIdx.x / MOE_WAVE;
  int inc = v;
#pragma unroll
  for (int off = 1; off < MOE_WAVE; off <<= 1) {
    const int u = __shfl_up(inc, off, MOE_WAVE);
    if (lane >= off) inc += u;
  }
  __syncthreads();
  if (lane == MOE_WAVE - 1) lds4[wave] = inc;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int x = lds4[w];
    if (w < wave) before += x;
    tot += x;
  }
  *total = tot;
  return before + inc - v;
}

// Find the (expert, row tile) of row-tile slot `slot`; returns false when the slot is past the end.
template <int BM>
__device__ bool map_tile(const int32_t* __restrict__ offsets, int E, int slot, int* e_out, int* row0_out,
                         int* rows_out) {
  __shared__ int s_e, s_tile;
  __shared__ int s_tmp[4];
  if (threadIdx.x == 0) s_e = -1;
  int carry = 0;
  for (int base = 0; base < E; base += 256) {
    const int e = base + threadIdx.x;
    const int cnt = (e < E) ? offsets[e + 1] - offsets[e] : 0;
    const int nt = (cnt + BM - 1) / BM;
    int tot;
    const int start = carry + block_scan_256(nt, s_tmp, &tot);
    if (e < E && slot >= start && slot < start + nt) {
      s_e = e;
      s_tile = slot - start;
    }
    carry += tot;
    if (carry > slot) break;  // uniform: every thread sees the same carry
  }
  __syncthreads();
  const int e = s_e;
  if (e < 0) return false;
  const int row0 = offsets[e] + s_tile * BM;
  *e_out = e;
  *row0_out = row0;
  *rows_out = min(BM, offsets[e + 1] - row0);
  return true;
}

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

__device__ __forceinline__ float act_silu(float a) { return a / (1.f + expf(-a)); }
__device__ __forceinline__ float act_gelu(float a) { return 0.5f * a * (1.f + erff(a * 0.70710678118654752f)); }

// ---------------------------------------------------------------------------------------------------
// bf16 grouped GEMM on matrix cores. BM x BN output tile per B matrix (two B matrices for SwiGLU),
// BK = 64, 4 waves in a 2 x 2 grid, each wave a 64 x 64 sub-tile of 2 x 2 32x32x16 MFMA blocks.
// LDS: double-buffered A and B tiles of 16-byte chunks, 8 chunks per 64-wide row, XOR-swizzled.
// ---------------------------------------------------------------------------------------------------
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int KCH = BK / 8;  // 16-byte chunks per tile row

template <int ACT, bool DUAL>
__global__ void __launch_bounds__(256) ffn_gemm_bf16(const bf16_t* __restrict__ A, const int32_t* __restrict__ offsets,
                                                     const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1,
                                                     bf16_t* __restrict__ out, int E, int K, int Nout) {
  constexpr int NB = DUAL ? 2 : 1;
  constexpr int A_CH = BM * KCH, B_CH = BN * KCH;
  constexpr int STAGE = A_CH + NB * B_CH;
  __shared__ bf16x8 lds[2 * STAGE];

  int e, row0, mrows;
  if (!map_tile<BM>(offsets, E, blockIdx.x, &e, &row0, &mrows)) return;
  const int n0 = blockIdx.y * BN;
  const int tid = threadIdx.x, lane = tid % MOE_WAVE, wave = tid / MOE_WAVE;
  const int wm = wave / 2, wn = wave % 2;

  const bf16_t* Ab = A + (size_t)row0 * K;
  const bf16_t* Bb[NB];
  Bb[0] = B0 + ((size_t)e * Nout + n0) * K;
  if constexpr (DUAL) Bb[NB - 1] = B1 + ((size_t)e * Nout + n0) * K;

  // global -> register staging: 4 A chunks and 4 chunks per B matrix per thread per K tile
  bf16x8 ra[A_CH / 256], rb[NB][B_CH / 256];
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < A_CH / 256; ++i) {
      const int c = tid + i * 256, row = c / KCH, ch = c % KCH;
      ra[i] = (row < mrows) ? *reinterpret_cast<const bf16x8*>(Ab + (size_t)row * K + k0 + ch * 8) : bf16x8{};
    }
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int i = 0; i < B_CH / 256; ++i) {
        const int c = tid + i * 256, row = c / KCH, ch = c % KCH;
        rb[m][i] = (n0 + row < Nout) ? *reinterpret_cast<const bf16x8*>(Bb[m] + (size_t)row * K + k0 + ch * 8)
                                     : bf16x8{};
      }
  };
  auto sstore = [&](int buf) {
    bf16x8* s = lds + buf * STAGE;
#pragma unroll
    for (int i = 0; i < A_CH / 256; ++i) {
      const int c = tid + i * 256, row = c / KCH, ch = c % KCH;
      s[row * KCH + swz(row, ch)] = ra[i];
    }
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int i = 0; i < B_CH / 256; ++i) {
        const int c = tid + i * 256, row = c / KCH, ch = c % KCH;
        s[A_CH + m * B_CH + row * KCH + swz(row, ch)] = rb[m][i];
      }
  };

  f32x16 acc[NB][2][2];
#pragma unroll
  for (int m = 0; m < NB; ++m)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[m][i][j][v] = 0.f;

  const int nk = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const bf16x8* s = lds + buf * STAGE;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int ch = ks * 2 + lane / 32;
      bf16x8 a[2], b[NB][2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wm * 64 + i * 32 + lane % 32;
        a[i] = s[row * KCH + swz(row, ch)];
      }
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int row = wn * 64 + j * 32 + lane % 32;
          b[m][j] = s[A_CH + m * B_CH + row * KCH + swz(row, ch)];
        }
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[m][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[m][j], acc[m][i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds C[i][j] for j = lane%32, i = (v/4)*8 + (lane/32)*4 + v%4
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * 64 + i * 32 + (v / 4) * 8 + (lane / 32) * 4 + (v % 4);
        const int c = n0 + wn * 64 + j * 32 + lane % 32;
        if (r < mrows && c < Nout) {
          float h = acc[0][i][j][v];
          if constexpr (ACT == MOE_ACT_SWIGLU && DUAL) h = act_silu(h) * acc[NB - 1][i][j][v];
          else if constexpr (ACT == MOE_ACT_GELU) h = act_gelu(h);
          out[(size_t)(row0 + r) * Nout + c] = f2bf(h);
        }
      }
}

// ---------------------------------------------------------------------------------------------------
// float32 grouped GEMM (plain FMA): 64 x 64 tiles, BK = 16, each thread 4 x 4 outputs per B matrix.
// ---------------------------------------------------------------------------------------------------
constexpr int FBM = 64, FBN = 64, FBK = 16;

template <int ACT, bool DUAL>
__global__ void __launch_bounds__(256) ffn_gemm_f32(const float* __restrict__ A, const int32_t* __restrict__ offsets,
                                                    const float* __restrict__ B0, const float* __restrict__ B1,
                                                    float* __restrict__ out, int E, int K, int Nout) {
  constexpr int NB = DUAL ? 2 : 1;
  __shared__ float As[FBK][FBM + 4];
  __shared__ float Bs[NB][FBK][FBN + 4];
  int e, row0, mrows;
  if (!map_tile<FBM>(offsets, E, blockIdx.x, &e, &row0, &mrows)) return;
  const int n0 = blockIdx.y * FBN;
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const float* Bb[NB];
  Bb[0] = B0 + ((size_t)e * Nout + n0) * K;
  if constexpr (DUAL) Bb[NB - 1] = B1 + ((size_t)e * Nout + n0) * K;
  float acc[NB][4][4] = {};
  for (int k0 = 0; k0 < K; k0 += FBK) {
    // 64 rows x 16 k = 1024 values: 4 per thread
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * 256, row = c / FBK, kk = c % FBK;
      As[kk][row] = (row < mrows) ? A[(size_t)(row0 + row) * K + k0 + kk] : 0.f;
#pragma unroll
      for (int m = 0; m < NB; ++m) Bs[m][kk][row] = (n0 + row < Nout) ? Bb[m][(size_t)row * K + k0 + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FBK; ++kk) {
      float a[4], b[NB][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) b[m][j] = Bs[m][kk][tx * 4 + j];
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[m][i][j] = fmaf(a[i], b[m][j], acc[m][i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = ty * 4 + i, c = n0 + tx * 4 + j;
      if (r < mrows && c < Nout) {
        float h = acc[0][i][j];
        if constexpr (ACT == MOE_ACT_SWIGLU && DUAL) h = act_silu(h) * acc[NB - 1][i][j];
        else if constexpr (ACT == MOE_ACT_GELU) h = act_gelu(h);
        out[(size_t)(row0 + r) * Nout + c] = h;
      }
    }
}

template <int TBM>
dim3 ffn_grid(const FfnArgs& a, int tbn) {
  const int slots = (a.n_rows_max + TBM - 1) / TBM + (a.E < a.n_rows_max ? a.E : a.n_rows_max);
  return dim3(slots, (a.Nout + tbn - 1) / tbn);
}

}  // namespace

hipError_t launch_ffn_bf16(const FfnArgs& a, hipStream_t s) {
  if (a.n_rows_max == 0) return hipSuccess;
  const dim3 grid = ffn_grid<BM>(a, BN);
  const bf16_t* A = (const bf16_t*)a.a;
  const bf16_t* b0 = (const bf16_t*)a.b0;
  const bf16_t* b1 = (const bf16_t*)a.b1;
  bf16_t* o = (bf16_t*)a.out;
  if (a.act == MOE_ACT_SWIGLU)
    hipLaunchKernelGGL((ffn_gemm_bf16<MOE_ACT_SWIGLU, true>), grid, dim3(256), 0, s, A, a.expert_offsets, b0, b1, o,
                       a.E, a.K, a.Nout);
  else if (a.act == MOE_ACT_GELU)
    hipLaunchKernelGGL((ffn_gemm_bf16<MOE_ACT_GELU, false>), grid, dim3(256), 0, s, A, a.expert_offsets, b0, b1, o,
                       a.E, a.K, a.Nout);
  else
    hipLaunchKernelGGL((ffn_gemm_bf16<-1, false>), grid, dim3(256), 0, s, A, a.expert_offsets, b0, b1, o, a.E, a.K,
                       a.Nout);
  return hipGetLastError();
}

hipError_t launch_ffn_f32(const FfnArgs& a, hipStream_t s) {
  if (a.n_rows_max == 0) return hipSuccess;
  const dim3 grid = ffn_grid<FBM>(a, FBN);
  const float* A = (const float*)a.a;
  const float* b0 = (const float*)a.b0;
  const float* b1 = (const float*)a.b1;
  float* o = (float*)a.out;
  if (a.act == MOE_ACT_SWIGLU)
    hipLaunchKernelGGL((ffn_gemm_f32<MOE_ACT_SWIGLU, true>), grid, dim3(256), 0, s, A, a.expert_offsets, b0, b1, o,
                       a.E, a.K, a.Nout);
  else if (a.act == MOE_ACT_GELU)
    hipLaunchKernelGGL((ffn_gemm_f32<MOE_ACT_GELU, false>), grid, dim3(256), 0, s, A, a.expert_offsets, b0, b1, o,
                       a.E, a.K, a.Nout);
  else
    hipLaunchKernelGGL((ffn_gemm_f32<-1, false>), grid, dim3(256), 0, s, A, a.expert_offsets, b0, b1, o, a.E, a.K,
                       a.Nout);
  return hipGetLastError();
}

}  // namespace moe
