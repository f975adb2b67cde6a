// Internal declarations shared by libmoe's translation units (device helpers + launch wrappers).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "moe.h"

#define MOE_WAVE 64

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// float -> bf16, round to nearest even (the C conversion; gfx950 has a native instruction for it)
__device__ __forceinline__ bf16_t f2bf(float f) { return static_cast<bf16_t>(f); }
__device__ __forceinline__ float bf2f(bf16_t b) { return static_cast<float>(b); }

// Element conversions used by the templated kernels.
template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf2f(v); }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f2bf(v); }

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// ------------------------------------------------------------------------------------------------
// Launch wrappers, one per translation unit (host-callable; all return hipError_t of the launch).
// ------------------------------------------------------------------------------------------------
namespace moe {

struct LayoutArgs {
  const int32_t* topk_idx;
  int32_t* expert_counts;
  int32_t* expert_offsets;
  int32_t* rank_counts;
  int32_t* rank_offsets;
  int32_t* pair_to_row;
  int32_t* row_to_pair;
  int32_t* chunk_hist;  // workspace: [n_chunks, E]
  int32_t n_pairs, E, ep_size, capacity;
};
constexpr int kLayoutChunk = 512;  // pairs per wave-sized chunk of the stable layout
size_t layout_ws_bytes(int32_t n_pairs, int32_t E);
hipError_t launch_layout(const LayoutArgs& a, hipStream_t s);
// device address of this GPU's static layout scratch (MOE_LAYOUT_NOALLOC_SCRATCH_BYTES)
hipError_t layout_noalloc_scratch(int32_t** out);

struct RouteArgs {
  const void* x;
  const void* w_gate;
  const float* bias;
  const float* select_bias;   // selection-only bias [E] or null
  int32_t* topk_idx;
  float* topk_gate;
  float* logits;              // [T,E] or null
  float* prob_partials;       // [ceil(T/64), E] per-block router-probability sums, or null
  int32_t T, D, E, k, n_groups, topk_groups, gate;
};
constexpr int kRouteTokPerBlock = 64;
hipError_t launch_route(const RouteArgs& a, int dtype, hipStream_t s);
hipError_t launch_load_balance(const int32_t* expert_counts, const float* prob_partials, int32_t n_partials,
                               int32_t T, int32_t E, int32_t k, float alpha, float* stats, float gamma,
                               float* select_bias, hipStream_t s);

hipError_t launch_permute(const void* x, const int32_t* pair_to_row, void* x_perm, int32_t T, int32_t D,
                          int32_t k, int dtype, hipStream_t s);
hipError_t launch_combine(const void* y_perm, const int32_t* pair_to_row, const float* gate, const void* add, void* y,
                          int32_t T, int32_t D, int32_t k, int dtype, hipStream_t s);

hipError_t launch_dispatch_matrix(const int32_t* topk_idx, int n_src, int Ts, int k, int E, int n_dst, int32_t* matrix,
                                  hipStream_t s);
size_t recv_layout_lds_bytes(int n_src, int epr);
hipError_t launch_recv_layout(const int32_t* src_off, int n_src, int E, int n_dst, int r, long long stride,
                              int32_t* recv_counts, int32_t* exp_off, int32_t* g2s, int n_rows_max, hipStream_t s);
hipError_t launch_move_rows(bool scatter, const void* src, const int32_t* map, long long n_rows, int row_bytes,
                            void* dst, hipStream_t s);
hipError_t launch_padded_layout(const int32_t* topk_idx, const int32_t* eoff, const int32_t* p2r, const int32_t* r2p,
                                int P, int E, int C, int32_t* p2s, int32_t* s2p, int32_t* poff, hipStream_t s);
hipError_t launch_permute_padded(const void* x, const int32_t* s2p, long long n_slots, int k, int row_bytes, void* xp,
                                 hipStream_t s);

hipError_t launch_backward_combine(const void* dy, const int32_t* p2r, const float* gate, const void* yp, void* dyp,
                                   float* dgate, int T, int D, int k, int dtype, hipStream_t s);
hipError_t launch_router_backward(const float* logits, const int32_t* idx, const float* gate, const float* dgate,
                                  float* dl, int T, int E, int k, int mode, hipStream_t s);
size_t colsum_ws_bytes(int rows, int cols);
hipError_t launch_colsum(const float* m, int rows, int cols, float* part, float* out, hipStream_t s);
hipError_t launch_tn_f32(const float* A, const void* B, int dtype, int K, int M, int N, float* C, hipStream_t s);
hipError_t launch_router_wgrad_grouped(const void* x, const float* dl, const int32_t* off, const int32_t* r2p, int E,
                                       int D, int k, int dtype, float* dwg, hipStream_t s);
hipError_t launch_backward_dx(const void* dxp, const int32_t* p2r, const int32_t* idx, const float* dl, const void* wg,
                              void* dx, int T, int D, int E, int k, int all_experts, int dtype, hipStream_t s);
hipError_t launch_transpose(const void* src, int B, int R, int C, long long src_batch, void* dst, long long ld_dst,
                            long long dst_batch, int col_off, int dtype, hipStream_t s);
hipError_t launch_group_koff(const int32_t* off, int G, int32_t* koff, hipStream_t s);
hipError_t launch_group_transpose(const void* src, int C, const int32_t* off, const int32_t* koff, int G,
                                  long long ld, void* dst, int dtype, hipStream_t s, const int32_t* gidx = nullptr,
                                  int gdiv = 1);

struct FfnArgs {
  const void* a;              // x_perm (up) or h (down): [N_max, K]
  const int32_t* expert_offsets;
  const void* b0;             // W1 (up) or W2 (down): [E, Nout, K]
  const void* b1;             // W3 (up, SwiGLU) or null
  void* out;                  // h (up) or y_perm (down): [N_max, Nout]
  int32_t n_rows_max, E, K, Nout;
  int act;                    // up: MOE_ACT_*; down: -1 (no activation); epi 2: the activation to differentiate
  int epi = 0;                // 0 plain; 1 also store pre-activations to `pre`; 2 activation backward
  void* pre = nullptr;        // epi 1: written; epi 2: read ([N_max, 2F] SwiGLU, [N_max, F] GELU)
  // when set, row r of A is row gather[r] / gather_div of `a` (up: a = x, gather = row_to_pair,
  // gather_div = top_k), so the permuted copy of x is never materialised
  const int32_t* gather = nullptr;
  int32_t gather_div = 1;
  // bf16 data-gradient forms only: b0 (and b1) stored K-major per expert, [K][Nout] (the weights as the
  // forward keeps them); with b1, rows k < ksplit of the reduction come from b0 ([ksplit][Nout] per
  // expert) and the rest from b1 ([K - ksplit][Nout])
  int bt = 0;
  int32_t ksplit = 0;
  // bf16 down-projection only: split K over `splits` blocks per tile, float32 partials in
  // part [splits][n_rows_max][Nout], then a fixed-order reduction into out
  int splits = 1;
  float* part = nullptr;
};
hipError_t launch_wgrad_bf16(const void* aT, const void* bT, const int32_t* koff, int G, int M, int N, long long ld,
                             float* out0, float* out1, int split, hipStream_t s);
hipError_t launch_ffn_bf16(const FfnArgs& a, hipStream_t s);
hipError_t launch_ffn_f32(const FfnArgs& a, hipStream_t s);

}  // namespace moe
