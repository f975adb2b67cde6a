// Router: logits l[t,e] = x[t]·W_g[e] + bias[e] in float32, top-k selection, gate values.
//
// EP-in-LLMs article, "The Execution Pipeline" step 1: the router scores every local token against
// all E experts, keeps the top k and normalises their gates; the layer equation of "The
// Distributed MoE Dilemma" sums over TopK(G(x), k). Node-limited routing ("Expert Parallelism and
// All-to-All", section on fighting back) restricts a token to its best groups before the
// per-expert choice.
//
// One block = 4 waves = 64 tokens; all E (<= 256) experts of a token stay in one block, so the
// selection needs no second pass over HBM.
//   bf16: matrix cores (v_mfma_f32_16x16x32_bf16) with float32 accumulation. Each wave owns 16
//         tokens; the block stages a 64-wide K slice of W_g for all experts in LDS (double
//         buffered, 16-byte chunks XOR-swizzled against bank conflicts); x fragments come straight
//         from HBM (each x element is read once).
//   fp32: plain FMA dot products (the small fp32 workload only).
// The [64 x E] float32 logit tile then goes to LDS, and each wave selects for its 16 tokens:
// group scores (if limited), then k rounds of a wave-wide argmax on (value, -index), so exact
// ties go to the lower expert index.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kTokPerBlock = 64;
constexpr int kTokPerWave = 16;
constexpr int kKC = 64;           // K slice per pipeline stage (two MFMA k-steps of 32)
constexpr int kMaxE = 256;
constexpr int kMaxPerLane = kMaxE / MOE_WAVE;

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// ---- logits, bf16 on matrix cores ---------------------------------------------------------------
template <int NT>  // 16-expert MFMA column tiles; experts padded to NT*16
__device__ void logits_bf16(const bf16_t* __restrict__ x, const bf16_t* __restrict__ wg, const float* bias,
                            float* lds_logits, char* lds_raw, int T, int D, int E, int t0) {
  constexpr int epad = NT * 16;
  const int tid = threadIdx.x;
  const int wave = tid / MOE_WAVE, lane = tid % MOE_WAVE;
  bf16x8* wbuf = reinterpret_cast<bf16x8*>(lds_raw);  // [2][epad][8 chunks of 16 B]
  constexpr int stage_chunks = epad * (kKC / 8);

  f32x4 acc[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int r = lane % 16, q = lane / 16;          // MFMA row / k-quarter of this lane
  const int tok = t0 + wave * kTokPerWave + r;
  const bool tok_ok = tok < T;
  const bf16_t* xrow = x + (size_t)(tok_ok ? tok : 0) * D;
  const int n_kc = (D + kKC - 1) / kKC;

  auto load_w = [&](int kc, int buf) {
    for (int c = tid; c < stage_chunks; c += 256) {
      const int row = c / (kKC / 8), ch = c % (kKC / 8);
      const int k = kc * kKC + ch * 8;
      bf16x8 v = {};
      if (row < E && k < D) v = *reinterpret_cast<const bf16x8*>(wg + (size_t)row * D + k);
      wbuf[buf * stage_chunks + row * (kKC / 8) + swz(row, ch)] = v;
    }
  };

  load_w(0, 0);
  __syncthreads();
  for (int kc = 0; kc < n_kc; ++kc) {
    const int buf = kc & 1;
    if (kc + 1 < n_kc) load_w(kc + 1, buf ^ 1);
    // lane (r, q) supplies K elements [q*16, q*16+16) of this slice as two 8-wide MFMA fragments
    bf16x8 a[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int k = kc * kKC + q * 16 + s * 8;
      a[s] = (tok_ok && k < D) ? *reinterpret_cast<const bf16x8*>(xrow + k) : bf16x8{};
    }
    const bf16x8* wb = wbuf + buf * stage_chunks;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int row = nt * 16 + r;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 b = wb[row * (kKC / 8) + swz(row, q * 2 + s)];
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], b, acc[nt], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // acc[nt][i]: token row (lane/16)*4 + i of this wave, expert nt*16 + lane%16
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int e = nt * 16 + (lane % 16);
    const float bv = (bias != nullptr && e < E) ? bias[e] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int trow = wave * kTokPerWave + (lane / 16) * 4 + i;
      lds_logits[trow * epad + e] = acc[nt][i] + bv;
    }
  }
}

// ---- logits, fp32 FMA ------------------------------------------------------------------------------
__device__ void logits_f32(const float* __restrict__ x, const float* __restrict__ wg, const float* bias,
                           float* lds_logits, int epad, int T, int D, int E, int t0) {
  const int wave = threadIdx.x / MOE_WAVE, lane = threadIdx.x % MOE_WAVE;
  for (int i = 0; i < kTokPerWave; ++i) {
    const int trow = wave * kTokPerWave + i;
    const int tok = t0 + trow;
    for (int e = lane; e < epad; e += MOE_WAVE) {
      float s = 0.f;
      if (tok < T && e < E) {
        const float* xr = x + (size_t)tok * D;
        const float* wr = wg + (size_t)e * D;
        for (int d = 0; d < D; d += 4) {
          const f32x4 xv = *reinterpret_cast<const f32x4*>(xr + d);
          const f32x4 wv = *reinterpret_cast<const f32x4*>(wr + d);
          s = fmaf(xv[0], wv[0], s);
          s = fmaf(xv[1], wv[1], s);
          s = fmaf(xv[2], wv[2], s);
          s = fmaf(xv[3], wv[3], s);
        }
        if (bias != nullptr) s += bias[e];
      }
      lds_logits[trow * epad + e] = s;
    }
  }
}

__device__ __forceinline__ bool better(float v, int e, float ov, int oe) {
  return ov > v || (ov == v && oe < e);
}

__device__ __forceinline__ float sigmoidf_(float v) { return 1.f / (1.f + expf(-v)); }

// ---- selection and gates for one token ------------------------------------------------------------
__device__ void select_token(const float* lrow, int E, int k, int n_groups, int topk_groups, int gate,
                             int32_t* out_idx, float* out_gate) {
  const int lane = lane_id();
  const int n_per = (E + MOE_WAVE - 1) / MOE_WAVE;
  float v[kMaxPerLane];
  bool ok[kMaxPerLane];
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + i * MOE_WAVE;
    ok[i] = (i < n_per) && (e < E);
    v[i] = ok[i] ? lrow[e] : -INFINITY;
  }
  if (n_groups > 0) {
    // group score = sum of the `per` best member scores; lane g < n_groups scores group g
    const int gsize = E / n_groups;
    const int per = max(1, k / topk_groups);
    float gs = -INFINITY;
    if (lane < n_groups) {
      float best[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) best[j] = -INFINITY;
      for (int m = 0; m < gsize; ++m) {
        const float lv = lrow[lane * gsize + m];
        float sv = (gate == MOE_GATE_SIGMOID_TOPK) ? sigmoidf_(lv) : lv;
        // insert into the descending list best[0..per)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (j < per && sv > best[j]) {
            const float tmp = best[j];
            best[j] = sv;
            sv = tmp;
          }
        }
      }
      gs = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < per) gs += best[j];
    }
    // rank of each group among all groups by (-score, g)
    int rank = 0;
    for (int g = 0; g < n_groups; ++g) {
      const float og = __shfl(gs, g, MOE_WAVE);
      if (og > gs || (og == gs && g < lane)) ++rank;
    }
    const bool gkeep = (lane < n_groups) && (rank < topk_groups);
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + i * MOE_WAVE;
      const int g = (e < E) ? e / gsize : 0;
      const bool keep = __shfl((int)gkeep, g, MOE_WAVE) != 0;
      if (!keep) ok[i] = false;
    }
  }
  // k rounds of wave-wide argmax; lane j keeps slot j
  float my_v = 0.f;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + i * MOE_WAVE;
      if (ok[i] && better(bv, be, v[i], e)) {
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int off = MOE_WAVE / 2; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, MOE_WAVE);
      const int oe = __shfl_xor(be, off, MOE_WAVE);
      if (better(bv, be, ov, oe)) {
        bv = ov;
        be = oe;
      }
    }
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i)
      if (lane + i * MOE_WAVE == be) ok[i] = false;
    if (lane == j) {
      my_v = bv;
      my_e = be;
    }
  }
  // gates
  const float v0 = __shfl(my_v, 0, MOE_WAVE);
  float w = 0.f;
  if (lane < k) {
    if (gate == MOE_GATE_SIGMOID_TOPK) w = sigmoidf_(my_v);
    else w = expf(my_v - v0);
  }
  float denom;
  if (gate == MOE_GATE_SOFTMAX_FULL) {
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i)
      if (lane + i * MOE_WAVE < E) m = fmaxf(m, v[i]);
    for (int off = MOE_WAVE / 2; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, MOE_WAVE));
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i)
      if (lane + i * MOE_WAVE < E) z += expf(v[i] - m);
    for (int off = MOE_WAVE / 2; off >= 1; off >>= 1) z += __shfl_xor(z, off, MOE_WAVE);
    w = (lane < k) ? expf(my_v - m) : 0.f;
    denom = z;
  } else {
    // sum over slots in slot order 0..k-1 (same order on every lane)
    denom = 0.f;
    for (int j = 0; j < k; ++j) denom += __shfl(w, j, MOE_WAVE);
  }
  if (lane < k) {
    out_idx[lane] = my_e;
    out_gate[lane] = w / denom;
  }
}

template <typename T, int NT>
__global__ void __launch_bounds__(256) route_kernel(const T* __restrict__ x, const T* __restrict__ wg,
                                                    const float* __restrict__ bias, int32_t* __restrict__ topk_idx,
                                                    float* __restrict__ topk_gate, float* __restrict__ logits,
                                                    int T_, int D, int E, int k, int n_groups, int topk_groups,
                                                    int gate) {
  constexpr int epad = NT * 16;
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  float* lds_logits = reinterpret_cast<float*>(lds_raw);
  const int t0 = blockIdx.x * kTokPerBlock;
  if constexpr (sizeof(T) == 2) {
    logits_bf16<NT>(x, wg, bias, lds_logits, lds_raw, T_, D, E, t0);
  } else {
    logits_f32(x, wg, bias, lds_logits, epad, T_, D, E, t0);
  }
  __syncthreads();
  const int wave = threadIdx.x / MOE_WAVE, lane = threadIdx.x % MOE_WAVE;
  if (logits != nullptr) {
    for (int i = 0; i < kTokPerWave; ++i) {
      const int trow = wave * kTokPerWave + i;
      const int tok = t0 + trow;
      if (tok >= T_) break;
      for (int e = lane; e < E; e += MOE_WAVE) logits[(size_t)tok * E + e] = lds_logits[trow * epad + e];
    }
  }
  for (int i = 0; i < kTokPerWave; ++i) {
    const int trow = wave * kTokPerWave + i;
    const int tok = t0 + trow;
    if (tok >= T_) break;
    select_token(lds_logits + trow * epad, E, k, n_groups, topk_groups, gate, topk_idx + (size_t)tok * k,
                 topk_gate + (size_t)tok * k);
  }
}

template <int NT>
hipError_t launch_route_nt(const RouteArgs& a, int dtype, hipStream_t s) {
  constexpr int epad = NT * 16;
  const int blocks = (a.T + kTokPerBlock - 1) / kTokPerBlock;
  const size_t lds_logits = (size_t)kTokPerBlock * epad * sizeof(float);
  if (dtype == MOE_BF16) {
    const size_t lds_w = (size_t)2 * epad * kKC * sizeof(bf16_t);
    const size_t lds = lds_w > lds_logits ? lds_w : lds_logits;
    hipLaunchKernelGGL((route_kernel<bf16_t, NT>), dim3(blocks), dim3(256), lds, s, (const bf16_t*)a.x,
                       (const bf16_t*)a.w_gate, a.bias, a.topk_idx, a.topk_gate, a.logits, a.T, a.D, a.E, a.k,
                       a.n_groups, a.topk_groups, a.gate);
  } else {
    hipLaunchKernelGGL((route_kernel<float, NT>), dim3(blocks), dim3(256), lds_logits, s, (const float*)a.x,
                       (const float*)a.w_gate, a.bias, a.topk_idx, a.topk_gate, a.logits, a.T, a.D, a.E, a.k,
                       a.n_groups, a.topk_groups, a.gate);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, int dtype, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int nt = (a.E + 15) / 16;
  if (nt <= 1) return launch_route_nt<1>(a, dtype, s);
  if (nt <= 2) return launch_route_nt<2>(a, dtype, s);
  if (nt <= 4) return launch_route_nt<4>(a, dtype, s);
  if (nt <= 8) return launch_route_nt<8>(a, dtype, s);
  return launch_route_nt<16>(a, dtype, s);
}

}  // namespace moe
