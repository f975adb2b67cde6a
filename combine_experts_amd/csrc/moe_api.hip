// libmoe C ABI: host-side argument checks and kernel launches. Nothing here allocates, frees or
// synchronises; every call enqueues work on the caller's stream and returns a status.
#include <cmath>
#include <cstdint>

#include <algorithm>

#include "moe_common.h"
#include "gemm_geometry.h"

namespace {

constexpr int kAbiVersion = 108;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
int elem_bytes(const moe_dims* d) { return d->dtype == MOE_BF16 ? 2 : 4; }

// Consistency of the problem statement itself (shared by every entry point).
int check_dims(const moe_dims* d) {
  if (d == nullptr) return MOE_ERR_INVALID_ARG;
  if (d->T < 0 || d->D <= 0 || d->E <= 0 || d->F <= 0) return MOE_ERR_INVALID_ARG;
  if (d->top_k < 1 || d->top_k > d->E) return MOE_ERR_INVALID_ARG;
  if ((int64_t)d->T * d->top_k > INT32_MAX) return MOE_ERR_INVALID_ARG;
  if (d->ep_size < 1 || d->E % d->ep_size != 0) return MOE_ERR_INVALID_ARG;
  if (d->ep_rank < 0 || d->ep_rank >= d->ep_size) return MOE_ERR_INVALID_ARG;
  if (d->n_groups < 0) return MOE_ERR_INVALID_ARG;
  if (d->n_groups > 0) {
    if (d->E % d->n_groups != 0) return MOE_ERR_INVALID_ARG;
    if (d->topk_groups < 1 || d->topk_groups > d->n_groups) return MOE_ERR_INVALID_ARG;
    if ((int64_t)d->topk_groups * (d->E / d->n_groups) < d->top_k) return MOE_ERR_INVALID_ARG;
  }
  if (d->gate < MOE_GATE_SOFTMAX_TOPK || d->gate > MOE_GATE_SOFTMAX_FULL) return MOE_ERR_INVALID_ARG;
  if (d->act != MOE_ACT_SWIGLU && d->act != MOE_ACT_GELU) return MOE_ERR_INVALID_ARG;
  if (d->dtype != MOE_F32 && d->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(d->capacity_factor)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

int32_t capacity_of(const moe_dims* d) {
  const int64_t n_pairs = (int64_t)d->T * d->top_k;
  if (d->capacity_factor <= 0.0) return (int32_t)n_pairs;
  // C = ceil(CF * k * T / E), in IEEE double, evaluated as CF * (k*T) / E
  const double c = std::ceil(d->capacity_factor * (double)n_pairs / (double)d->E);
  if (c >= (double)n_pairs) return (int32_t)n_pairs;
  return (int32_t)c;
}

// Splits of the down-projection's reduction: only when the tiles it can have (at most ceil(N_max/GBM)
// + E row tiles, and at most ceil(C/GBM) per expert) times ceil(D/GBR) column tiles fill at most a
// quarter of the 256 compute units and F is long enough to split (F/64 >= 32 stages); then as many
// as keep <= 2 blocks per compute unit and >= 16 stages per block.
int down_splits(const moe_dims* d) {
  if (d->dtype != MOE_BF16 || d->T == 0) return 1;
  const int64_t P = (int64_t)d->T * d->top_k, C = capacity_of(d), bm = moe::geom::GBM;
  const int64_t mt = std::min<int64_t>((P + bm - 1) / bm + std::min<int64_t>(d->E, P),
                                       (int64_t)d->E * ((C + bm - 1) / bm));
  const int64_t tiles = mt * ((d->D + moe::geom::GBR - 1) / moe::geom::GBR);
  const int nk = d->F / moe::geom::GBK;
  constexpr int64_t kCUs = 256;
  if (tiles > kCUs / 4 || nk < 32 || d->F % moe::geom::GBK != 0) return 1;
  int s = 1;
  while (s < 8 && tiles * s * 2 <= 2 * kCUs && nk / (s * 2) >= 16) s *= 2;
  return s;
}

size_t down_split_ws_bytes(const moe_dims* d) {
  const int s = down_splits(d);
  if (s <= 1) return 0;
  return ((size_t)s * d->T * d->top_k * d->D * sizeof(float) + 255) / 256 * 256;
}

size_t ffn_ws_bytes(const moe_dims* d) {
  const size_t n_max = (size_t)d->T * d->top_k;
  return (n_max * d->F * elem_bytes(d) + 255) / 256 * 256 + down_split_ws_bytes(d);
}

int row_vec_ok(const moe_dims* d, int n) { return (n * elem_bytes(d)) % 16 == 0; }

int ffn_shape_ok(const moe_dims* d) {
  if (d->dtype == MOE_BF16) return d->D % 64 == 0 && d->F % 64 == 0;
  return d->D % 16 == 0 && d->F % 16 == 0;
}

// hipErrorNotSupported is what a launcher returns for shapes its kernels cannot address
int hip_status(hipError_t e) {
  return e == hipSuccess ? MOE_OK : e == hipErrorNotSupported ? MOE_ERR_UNSUPPORTED : MOE_ERR_HIP;
}

size_t route_partial_rows(const moe_dims* d) {
  return ((size_t)d->T + moe::kRouteTokPerBlock - 1) / moe::kRouteTokPerBlock;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return kAbiVersion; }

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: null pointer, inconsistent dims or misaligned pointer";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: valid dims that no kernel of this library handles";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: kernel launch failed";
    default: return "unknown moe status";
  }
}

int moe_capacity(const moe_dims* d, int32_t* capacity) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  if (capacity == nullptr) return MOE_ERR_INVALID_ARG;
  *capacity = capacity_of(d);
  return MOE_OK;
}

int moe_workspace_size(const moe_dims* d, int stage, size_t* bytes) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
  if (stage == MOE_STAGE_LAYOUT) {
    *bytes = moe::layout_ws_bytes(d->T * d->top_k, d->E);
  } else if (stage == MOE_STAGE_FFN) {
    *bytes = ffn_ws_bytes(d);
  } else if (stage == MOE_STAGE_ROUTE_STATS) {
    *bytes = route_partial_rows(d) * (size_t)d->E * sizeof(float);
  } else if (stage == MOE_STAGE_ROUTER_BWD) {
    *bytes = moe::colsum_ws_bytes(d->T, d->E);
  } else if (stage == MOE_STAGE_FFN_DOWN) {
    *bytes = down_split_ws_bytes(d);
  } else {
    return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

int moe_route_ex(const moe_dims* d, const void* x, const void* w_gate, const float* bias, const float* select_bias,
                 int32_t* topk_idx, float* topk_gate, float* logits, float* prob_partials, hipStream_t stream) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;  // nothing to route
  if (x == nullptr || w_gate == nullptr || topk_idx == nullptr || topk_gate == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_gate) || !aligned4(topk_idx) || !aligned4(topk_gate)) return MOE_ERR_INVALID_ARG;
  if ((bias && !aligned4(bias)) || (logits && !aligned4(logits))) return MOE_ERR_INVALID_ARG;
  if ((select_bias && !aligned4(select_bias)) || (prob_partials && !aligned4(prob_partials)))
    return MOE_ERR_INVALID_ARG;
  if (d->E > 256 || d->top_k > 32 || d->D % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (d->dtype == MOE_BF16 && d->D % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if (d->n_groups > 64 || (d->n_groups > 0 && d->top_k / d->topk_groups > 8)) return MOE_ERR_UNSUPPORTED;
  moe::RouteArgs a{x, w_gate, bias, select_bias, topk_idx, topk_gate, logits, prob_partials, d->T, d->D, d->E,
                   d->top_k, d->n_groups, d->n_groups > 0 ? d->topk_groups : 0, d->gate};
  return hip_status(moe::launch_route(a, d->dtype, stream));
}

int moe_route(const moe_dims* d, const void* x, const void* w_gate, const float* bias, int32_t* topk_idx,
              float* topk_gate, float* logits, hipStream_t stream) {
  return moe_route_ex(d, x, w_gate, bias, nullptr, topk_idx, topk_gate, logits, nullptr, stream);
}

int moe_load_balance(const moe_dims* d, const int32_t* expert_counts, const float* prob_partials, float alpha,
                     float* stats, float gamma, float* select_bias, hipStream_t stream) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  if (expert_counts == nullptr || stats == nullptr) return MOE_ERR_INVALID_ARG;
  if (prob_partials == nullptr && d->T > 0) return MOE_ERR_INVALID_ARG;
  if (!aligned4(expert_counts) || !aligned4(stats) || (prob_partials && !aligned4(prob_partials)) ||
      (select_bias && !aligned4(select_bias)))
    return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(alpha) || !std::isfinite(gamma)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_load_balance(expert_counts, prob_partials, (int32_t)route_partial_rows(d), d->T, d->E,
                                             d->top_k, alpha, stats, gamma, select_bias, stream));
}

int moe_dispatch_layout(const moe_dims* d, const int32_t* topk_idx, int32_t* expert_counts, int32_t* expert_offsets,
                        int32_t* rank_counts, int32_t* rank_offsets, int32_t* pair_to_row, int32_t* row_to_pair,
                        void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  if (!expert_counts || !expert_offsets || !rank_counts || !rank_offsets) return MOE_ERR_INVALID_ARG;
  if (d->T > 0 && (!topk_idx || !pair_to_row || !row_to_pair)) return MOE_ERR_INVALID_ARG;
  if (d->E > 1024) return MOE_ERR_UNSUPPORTED;
  const int32_t n_pairs = d->T * d->top_k;
  if (ws == nullptr || ws_bytes < moe::layout_ws_bytes(n_pairs, d->E)) return MOE_ERR_WORKSPACE;
  if (!aligned4(ws)) return MOE_ERR_INVALID_ARG;
  moe::LayoutArgs a{topk_idx, expert_counts, expert_offsets, rank_counts, rank_offsets, pair_to_row, row_to_pair,
                    static_cast<int32_t*>(ws), n_pairs, d->E, d->ep_size, capacity_of(d)};
  return hip_status(moe::launch_layout(a, stream));
}

int moe_dispatch_layout_noalloc(const moe_dims* d, const int32_t* topk_idx, int32_t* expert_counts,
                                int32_t* expert_offsets, int32_t* rank_counts, int32_t* rank_offsets,
                                int32_t* pair_to_row, int32_t* row_to_pair, hipStream_t stream) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  if (!expert_counts || !expert_offsets || !rank_counts || !rank_offsets) return MOE_ERR_INVALID_ARG;
  if (d->T > 0 && (!topk_idx || !pair_to_row || !row_to_pair)) return MOE_ERR_INVALID_ARG;
  if (d->E > 1024) return MOE_ERR_UNSUPPORTED;
  const int32_t n_pairs = d->T * d->top_k;
  // the chunk histograms must fit the static array; nothing is allocated when they do not
  if (moe::layout_ws_bytes(n_pairs, d->E) > MOE_LAYOUT_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  int32_t* scratch = nullptr;
  if (moe::layout_noalloc_scratch(&scratch) != hipSuccess) return MOE_ERR_HIP;
  // every histogram entry a kernel reads is written earlier in the same call: nothing to clear
  moe::LayoutArgs a{topk_idx, expert_counts, expert_offsets, rank_counts, rank_offsets, pair_to_row, row_to_pair,
                    scratch, n_pairs, d->E, d->ep_size, capacity_of(d)};
  return hip_status(moe::launch_layout(a, stream));
}

int moe_permute(const moe_dims* d, const void* x, const int32_t* pair_to_row, void* x_perm, hipStream_t stream) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;
  if (!x || !pair_to_row || !x_perm) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(x_perm)) return MOE_ERR_INVALID_ARG;
  if (!row_vec_ok(d, d->D)) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_permute(x, pair_to_row, x_perm, d->T, d->D, d->top_k, d->dtype, stream));
}

int moe_expert_ffn_up(const moe_dims* d, const void* x_perm, const int32_t* expert_offsets, const void* w1,
                      const void* w3, void* h, hipStream_t stream) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;
  if (!x_perm || !expert_offsets || !w1 || !h || (d->act == MOE_ACT_SWIGLU && !w3)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x_perm) || !aligned16(w1) || !aligned16(h) || (w3 && !aligned16(w3))) return MOE_ERR_INVALID_ARG;
  if (!ffn_shape_ok(d)) return MOE_ERR_UNSUPPORTED;
  moe::FfnArgs a{x_perm, expert_offsets, w1, d->act == MOE_ACT_SWIGLU ? w3 : nullptr, h,
                 d->T * d->top_k, d->E, d->D, d->F, d->act};
  return hip_status(d->dtype == MOE_BF16 ? moe::launch_ffn_bf16(a, stream) : moe::launch_ffn_f32(a, stream));
}

int moe_expert_ffn_up_gather(const moe_dims* d, const void* x, const int32_t* row_to_pair,
                             const int32_t* expert_offsets, const void* w1, const void* w3, void* h,
                             hipStream_t stream) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;
  if (!x || !row_to_pair || !expert_offsets || !w1 || !h || (d->act == MOE_ACT_SWIGLU && !w3))
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w1) || !aligned16(h) || (w3 && !aligned16(w3))) return MOE_ERR_INVALID_ARG;
  if (!ffn_shape_ok(d)) return MOE_ERR_UNSUPPORTED;
  moe::FfnArgs a{x, expert_offsets, w1, d->act == MOE_ACT_SWIGLU ? w3 : nullptr, h,
                 d->T * d->top_k, d->E, d->D, d->F, d->act};
  a.gather = row_to_pair;
  a.gather_div = d->top_k;
  return hip_status(d->dtype == MOE_BF16 ? moe::launch_ffn_bf16(a, stream) : moe::launch_ffn_f32(a, stream));
}

int moe_expert_ffn_down(const moe_dims* d, const void* h, const int32_t* expert_offsets, const void* w2,
                        void* y_perm, hipStream_t stream) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;
  if (!h || !expert_offsets || !w2 || !y_perm) return MOE_ERR_INVALID_ARG;
  if (!aligned16(h) || !aligned16(w2) || !aligned16(y_perm)) return MOE_ERR_INVALID_ARG;
  if (!ffn_shape_ok(d)) return MOE_ERR_UNSUPPORTED;
  moe::FfnArgs a{h, expert_offsets, w2, nullptr, y_perm, d->T * d->top_k, d->E, d->F, d->D, -1};
  return hip_status(d->dtype == MOE_BF16 ? moe::launch_ffn_bf16(a, stream) : moe::launch_ffn_f32(a, stream));
}

int moe_expert_ffn_down_splitk(const moe_dims* d, const void* h, const int32_t* expert_offsets, const void* w2,
                               void* y_perm, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  const int splits = down_splits(d);
  if (ws == nullptr || splits <= 1) return moe_expert_ffn_down(d, h, expert_offsets, w2, y_perm, stream);
  if (d->T == 0) return MOE_OK;
  if (!h || !expert_offsets || !w2 || !y_perm) return MOE_ERR_INVALID_ARG;
  if (!aligned16(h) || !aligned16(w2) || !aligned16(y_perm) || !aligned16(ws)) return MOE_ERR_INVALID_ARG;
  if (!ffn_shape_ok(d)) return MOE_ERR_UNSUPPORTED;
  if (ws_bytes < down_split_ws_bytes(d)) return MOE_ERR_WORKSPACE;
  moe::FfnArgs a{h, expert_offsets, w2, nullptr, y_perm, d->T * d->top_k, d->E, d->F, d->D, -1};
  a.splits = splits;
  a.part = static_cast<float*>(ws);
  return hip_status(moe::launch_ffn_bf16(a, stream));
}

int moe_expert_ffn(const moe_dims* d, const void* x_perm, const int32_t* expert_offsets, const void* w1,
                   const void* w3, const void* w2, void* y_perm, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;
  if (ws == nullptr || ws_bytes < ffn_ws_bytes(d)) return MOE_ERR_WORKSPACE;
  st = moe_expert_ffn_up(d, x_perm, expert_offsets, w1, w3, ws, stream);
  if (st != MOE_OK) return st;
  // h first, then the down-projection's split-K scratch (when these dims split)
  const size_t h_bytes = ffn_ws_bytes(d) - down_split_ws_bytes(d);
  return moe_expert_ffn_down_splitk(d, ws, expert_offsets, w2, y_perm, static_cast<char*>(ws) + h_bytes,
                                    ws_bytes - h_bytes, stream);
}

int moe_unpermute_combine_add(const moe_dims* d, const void* y_perm, const int32_t* pair_to_row,
                              const float* topk_gate, const void* addend, void* y, hipStream_t stream) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;
  if (!y_perm || !pair_to_row || !topk_gate || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(y_perm) || !aligned16(y) || (addend && !aligned16(addend))) return MOE_ERR_INVALID_ARG;
  if (!row_vec_ok(d, d->D)) return MOE_ERR_UNSUPPORTED;
  return hip_status(
      moe::launch_combine(y_perm, pair_to_row, topk_gate, addend, y, d->T, d->D, d->top_k, d->dtype, stream));
}

int moe_unpermute_combine(const moe_dims* d, const void* y_perm, const int32_t* pair_to_row, const float* topk_gate,
                          void* y, hipStream_t stream) {
  return moe_unpermute_combine_add(d, y_perm, pair_to_row, topk_gate, nullptr, y, stream);
}

int moe_dispatch_matrix(const moe_dims* d, const int32_t* topk_idx, int32_t n_src, int32_t* matrix,
                        hipStream_t stream) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  if (n_src < 1 || d->T % n_src != 0) return MOE_ERR_INVALID_ARG;
  if (!matrix || (d->T > 0 && !topk_idx)) return MOE_ERR_INVALID_ARG;
  if (!aligned4(matrix) || (topk_idx && !aligned4(topk_idx))) return MOE_ERR_INVALID_ARG;
  if ((size_t)d->ep_size * sizeof(int) > 65536) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_dispatch_matrix(topk_idx, n_src, d->T / n_src, d->top_k, d->E, d->ep_size, matrix,
                                                stream));
}

int moe_recv_layout(const moe_dims* d, int32_t n_src, int32_t rank, int64_t src_stride,
                    const int32_t* src_expert_offsets, int32_t* recv_counts, int32_t* expert_offsets,
                    int32_t* grouped_to_src_row, int32_t n_rows_max, hipStream_t stream) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  if (n_src < 1 || rank < 0 || rank >= d->ep_size || src_stride < 0 || n_rows_max < 0) return MOE_ERR_INVALID_ARG;
  if ((int64_t)n_src * src_stride > INT32_MAX) return MOE_ERR_INVALID_ARG;
  if (!src_expert_offsets || !recv_counts || !expert_offsets || (n_rows_max > 0 && !grouped_to_src_row))
    return MOE_ERR_INVALID_ARG;
  const int epr = d->E / d->ep_size;
  if (moe::recv_layout_lds_bytes(n_src, epr) > 65536) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_recv_layout(src_expert_offsets, n_src, d->E, d->ep_size, rank, src_stride,
                                            recv_counts, expert_offsets, grouped_to_src_row, n_rows_max, stream));
}

static int move_rows(const moe_dims* d, bool scatter, int64_t n_rows, const int32_t* row_map, const void* src,
                     void* dst, hipStream_t stream) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  if (n_rows < 0) return MOE_ERR_INVALID_ARG;
  if (n_rows == 0) return MOE_OK;
  if (!row_map || !src || !dst || !aligned16(src) || !aligned16(dst)) return MOE_ERR_INVALID_ARG;
  if (!row_vec_ok(d, d->D)) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_move_rows(scatter, src, row_map, n_rows, d->D * elem_bytes(d), dst, stream));
}

int moe_gather_rows(const moe_dims* d, int64_t n_rows, const int32_t* row_map, const void* src, void* dst,
                    hipStream_t stream) {
  return move_rows(d, false, n_rows, row_map, src, dst, stream);
}

int moe_scatter_rows(const moe_dims* d, int64_t n_rows, const int32_t* row_map, const void* src, void* dst,
                     hipStream_t stream) {
  return move_rows(d, true, n_rows, row_map, src, dst, stream);
}

int moe_padded_layout(const moe_dims* d, const int32_t* topk_idx, const int32_t* expert_offsets,
                      const int32_t* pair_to_row, const int32_t* row_to_pair, int32_t* pair_to_slot,
                      int32_t* slot_to_pair, int32_t* padded_offsets, hipStream_t stream) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  if (d->capacity_factor <= 0.0) return MOE_ERR_INVALID_ARG;  // the padded layout needs a capacity
  const int64_t C = capacity_of(d);
  if ((int64_t)d->E * C > INT32_MAX) return MOE_ERR_INVALID_ARG;
  // with no slots (an empty batch) slot_to_pair is empty and may be NULL
  if (!padded_offsets || (d->E * C > 0 && !slot_to_pair)) return MOE_ERR_INVALID_ARG;
  if (d->T > 0 && (!topk_idx || !expert_offsets || !pair_to_row || !row_to_pair || !pair_to_slot))
    return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_padded_layout(topk_idx, expert_offsets, pair_to_row, row_to_pair, d->T * d->top_k,
                                              d->E, (int)C, pair_to_slot, slot_to_pair, padded_offsets, stream));
}

int moe_permute_padded(const moe_dims* d, const void* x, const int32_t* slot_to_pair, void* x_pad,
                       hipStream_t stream) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  if (d->capacity_factor <= 0.0) return MOE_ERR_INVALID_ARG;
  const int64_t n_slots = (int64_t)d->E * capacity_of(d);
  if (n_slots > INT32_MAX) return MOE_ERR_INVALID_ARG;
  if ((n_slots > 0 && (!slot_to_pair || !x_pad)) || (d->T > 0 && !x)) return MOE_ERR_INVALID_ARG;
  if ((x && !aligned16(x)) || (x_pad && !aligned16(x_pad))) return MOE_ERR_INVALID_ARG;
  if (!row_vec_ok(d, d->D)) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_permute_padded(x, slot_to_pair, n_slots, d->top_k, d->D * elem_bytes(d), x_pad,
                                               stream));
}

static int ffn_padded(const moe_dims* d, bool up, const void* a, const int32_t* padded_offsets, const void* b0,
                      const void* b1, void* out, hipStream_t stream) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  if (d->capacity_factor <= 0.0) return MOE_ERR_INVALID_ARG;
  const int64_t n_slots = (int64_t)d->E * capacity_of(d);
  if (n_slots > INT32_MAX) return MOE_ERR_INVALID_ARG;
  if (!padded_offsets || !b0 || (up && d->act == MOE_ACT_SWIGLU && !b1)) return MOE_ERR_INVALID_ARG;
  if (n_slots > 0 && (!a || !out)) return MOE_ERR_INVALID_ARG;
  if ((a && !aligned16(a)) || !aligned16(b0) || (out && !aligned16(out)) || (b1 && !aligned16(b1)))
    return MOE_ERR_INVALID_ARG;
  if (!ffn_shape_ok(d)) return MOE_ERR_UNSUPPORTED;
  moe::FfnArgs f = up ? moe::FfnArgs{a, padded_offsets, b0, d->act == MOE_ACT_SWIGLU ? b1 : nullptr, out,
                                     (int32_t)n_slots, d->E, d->D, d->F, d->act}
                      : moe::FfnArgs{a, padded_offsets, b0, nullptr, out, (int32_t)n_slots, d->E, d->F, d->D, -1};
  return hip_status(d->dtype == MOE_BF16 ? moe::launch_ffn_bf16(f, stream) : moe::launch_ffn_f32(f, stream));
}

int moe_expert_ffn_padded_up(const moe_dims* d, const void* x_pad, const int32_t* padded_offsets, const void* w1,
                             const void* w3, void* h_pad, hipStream_t stream) {
  return ffn_padded(d, true, x_pad, padded_offsets, w1, w3, h_pad, stream);
}

int moe_expert_ffn_padded_down(const moe_dims* d, const void* h_pad, const int32_t* padded_offsets, const void* w2,
                               void* y_pad, hipStream_t stream) {
  return ffn_padded(d, false, h_pad, padded_offsets, w2, nullptr, y_pad, stream);
}

// ---- backward ----------------------------------------------------------------------------------
int moe_wgrad_ld(const moe_dims* d, int64_t* ld) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  if (ld == nullptr) return MOE_ERR_INVALID_ARG;
  *ld = ((int64_t)d->T * d->top_k + 63LL * d->E + 63) / 64 * 64;
  return MOE_OK;
}

static int ffn_bwd_common(const moe_dims* d) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  if (d->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;  // the training GEMM epilogues are bf16 only
  if (!ffn_shape_ok(d)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int moe_expert_ffn_up_train(const moe_dims* d, const void* x_perm, const int32_t* expert_offsets, const void* w1,
                            const void* w3, void* h, void* pre, hipStream_t stream) {
  int st = ffn_bwd_common(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;
  if (!x_perm || !expert_offsets || !w1 || !h || !pre || (d->act == MOE_ACT_SWIGLU && !w3)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x_perm) || !aligned16(w1) || !aligned16(h) || !aligned16(pre) || (w3 && !aligned16(w3)))
    return MOE_ERR_INVALID_ARG;
  moe::FfnArgs a{x_perm, expert_offsets, w1, d->act == MOE_ACT_SWIGLU ? w3 : nullptr, h,
                 d->T * d->top_k, d->E, d->D, d->F, d->act, 1, pre};
  return hip_status(moe::launch_ffn_bf16(a, stream));
}

int moe_expert_ffn_up_train_gather(const moe_dims* d, const void* x, const int32_t* row_to_pair,
                                   const int32_t* expert_offsets, const void* w1, const void* w3, void* h, void* pre,
                                   hipStream_t stream) {
  int st = ffn_bwd_common(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;
  if (!x || !row_to_pair || !expert_offsets || !w1 || !h || !pre || (d->act == MOE_ACT_SWIGLU && !w3))
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w1) || !aligned16(h) || !aligned16(pre) || (w3 && !aligned16(w3)))
    return MOE_ERR_INVALID_ARG;
  moe::FfnArgs a{x, expert_offsets, w1, d->act == MOE_ACT_SWIGLU ? w3 : nullptr, h,
                 d->T * d->top_k, d->E, d->D, d->F, d->act, 1, pre};
  a.gather = row_to_pair;
  a.gather_div = d->top_k;
  return hip_status(moe::launch_ffn_bf16(a, stream));
}

int moe_transpose_weights(const moe_dims* d, const void* w1, const void* w3, const void* w2, void* w13t, void* w2t,
                          hipStream_t stream) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  if (!w1 || !w2 || !w13t || !w2t || (d->act == MOE_ACT_SWIGLU && !w3)) return MOE_ERR_INVALID_ARG;
  if (!row_vec_ok(d, d->D) || !row_vec_ok(d, d->F)) return MOE_ERR_UNSUPPORTED;  // 16-byte row chunks
  const int nm = d->act == MOE_ACT_SWIGLU ? 2 : 1;
  const long long FD = (long long)d->F * d->D;
  // w2t[e] [F, D] = w2[e]^T ([D, F]); w13t[e] [D, nm*F] = [w1[e]^T | w3[e]^T]
  hipError_t e = moe::launch_transpose(w2, d->E, d->D, d->F, FD, w2t, d->D, FD, 0, d->dtype, stream);
  if (e == hipSuccess)
    e = moe::launch_transpose(w1, d->E, d->F, d->D, FD, w13t, (long long)nm * d->F, nm * FD, 0, d->dtype, stream);
  if (e == hipSuccess && nm == 2)
    e = moe::launch_transpose(w3, d->E, d->F, d->D, FD, w13t, 2LL * d->F, 2 * FD, d->F, d->dtype, stream);
  return hip_status(e);
}

int moe_backward_combine(const moe_dims* d, const void* dy, const int32_t* pair_to_row, const float* topk_gate,
                         const void* y_perm, void* dy_perm, float* dgate, hipStream_t stream) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;
  if (!dy || !pair_to_row || !topk_gate || !y_perm || !dy_perm || !dgate) return MOE_ERR_INVALID_ARG;
  if (!aligned16(dy) || !aligned16(y_perm) || !aligned16(dy_perm)) return MOE_ERR_INVALID_ARG;
  if (!row_vec_ok(d, d->D)) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_backward_combine(dy, pair_to_row, topk_gate, y_perm, dy_perm, dgate, d->T, d->D,
                                                 d->top_k, d->dtype, stream));
}

int moe_expert_ffn_down_backward(const moe_dims* d, const void* dy_perm, const int32_t* expert_offsets,
                                 const void* w2t, const void* pre, void* da, hipStream_t stream) {
  int st = ffn_bwd_common(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;
  if (!dy_perm || !expert_offsets || !w2t || !pre || !da) return MOE_ERR_INVALID_ARG;
  if (!aligned16(dy_perm) || !aligned16(w2t) || !aligned16(pre) || !aligned16(da)) return MOE_ERR_INVALID_ARG;
  // dh = dy_perm W2 as A [rows, D] against w2t [F, D] per expert; the epilogue differentiates the activation
  moe::FfnArgs a{dy_perm, expert_offsets, w2t, nullptr, da, d->T * d->top_k, d->E, d->D, d->F, d->act, 2,
                 const_cast<void*>(pre)};
  return hip_status(moe::launch_ffn_bf16(a, stream));
}

int moe_expert_ffn_up_backward(const moe_dims* d, const void* da, const int32_t* expert_offsets, const void* w13t,
                               void* dx_perm, hipStream_t stream) {
  int st = ffn_bwd_common(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;
  if (!da || !expert_offsets || !w13t || !dx_perm) return MOE_ERR_INVALID_ARG;
  if (!aligned16(da) || !aligned16(w13t) || !aligned16(dx_perm)) return MOE_ERR_INVALID_ARG;
  const int K = (d->act == MOE_ACT_SWIGLU ? 2 : 1) * d->F;
  moe::FfnArgs a{da, expert_offsets, w13t, nullptr, dx_perm, d->T * d->top_k, d->E, K, d->D, -1};
  return hip_status(moe::launch_ffn_bf16(a, stream));
}

int moe_expert_ffn_down_backward_w(const moe_dims* d, const void* dy_perm, const int32_t* expert_offsets,
                                   const void* w2, const void* pre, void* da, hipStream_t stream) {
  int st = ffn_bwd_common(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;
  if (!dy_perm || !expert_offsets || !w2 || !pre || !da) return MOE_ERR_INVALID_ARG;
  if (!aligned16(dy_perm) || !aligned16(w2) || !aligned16(pre) || !aligned16(da)) return MOE_ERR_INVALID_ARG;
  // dh = dy_perm W2 with W2[e] read as stored, [D][F]: K = D rows of F columns
  moe::FfnArgs a{dy_perm, expert_offsets, w2, nullptr, da, d->T * d->top_k, d->E, d->D, d->F, d->act, 2,
                 const_cast<void*>(pre)};
  a.bt = 1;
  return hip_status(moe::launch_ffn_bf16(a, stream));
}

int moe_expert_ffn_up_backward_w(const moe_dims* d, const void* da, const int32_t* expert_offsets, const void* w1,
                                 const void* w3, void* dx_perm, hipStream_t stream) {
  int st = ffn_bwd_common(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;
  const bool swi = d->act == MOE_ACT_SWIGLU;
  if (!da || !expert_offsets || !w1 || !dx_perm || (swi && !w3)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(da) || !aligned16(w1) || !aligned16(dx_perm) || (swi && !aligned16(w3))) return MOE_ERR_INVALID_ARG;
  // dx_perm = [da1 | da3] [W1; W3]: W1[e], W3[e] read as stored, [F][D]; reduction rows k < F from W1
  moe::FfnArgs a{da, expert_offsets, w1, swi ? w3 : nullptr, dx_perm, d->T * d->top_k, d->E,
                 (swi ? 2 : 1) * d->F, d->D, -1};
  a.bt = 1;
  a.ksplit = d->F;
  return hip_status(moe::launch_ffn_bf16(a, stream));
}

int moe_router_backward(const moe_dims* d, const void* x, const float* logits, const int32_t* topk_idx,
                        const float* topk_gate, const float* dgate, const int32_t* all_expert_offsets,
                        const int32_t* all_row_to_pair, float* dl, float* dw_gate, float* dbias, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  // with no tokens dl is empty (it may be NULL); dW_g and dbias still come out as zeros
  if (!dw_gate || (d->T > 0 && (!dl || !x || !logits || !topk_idx || !topk_gate || !dgate))) return MOE_ERR_INVALID_ARG;
  if ((all_expert_offsets == nullptr) != (all_row_to_pair == nullptr)) return MOE_ERR_INVALID_ARG;
  if (d->top_k > 32) return MOE_ERR_UNSUPPORTED;
  if (!row_vec_ok(d, d->D)) return MOE_ERR_UNSUPPORTED;
  if (dbias != nullptr && (ws == nullptr || ws_bytes < moe::colsum_ws_bytes(d->T, d->E))) return MOE_ERR_WORKSPACE;
  hipError_t e = moe::launch_router_backward(logits, topk_idx, topk_gate, dgate, dl, d->T, d->E, d->top_k, d->gate,
                                             stream);
  // dW_g = dl^T x: only the selected experts' columns of dl are nonzero under top-k gates, so with a
  // dropless grouping of the pairs the product is a per-expert weighted row sum; dense otherwise
  if (e == hipSuccess) {
    if (all_expert_offsets != nullptr && d->gate != MOE_GATE_SOFTMAX_FULL)
      e = moe::launch_router_wgrad_grouped(x, dl, all_expert_offsets, all_row_to_pair, d->E, d->D, d->top_k, d->dtype,
                                           dw_gate, stream);
    else
      e = moe::launch_tn_f32(dl, x, d->dtype, d->T, d->E, d->D, dw_gate, stream);
  }
  if (e == hipSuccess && dbias != nullptr) e = moe::launch_colsum(dl, d->T, d->E, static_cast<float*>(ws), dbias, stream);
  return hip_status(e);
}

int moe_backward_dx(const moe_dims* d, const void* dx_perm, const int32_t* pair_to_row, const int32_t* topk_idx,
                    const float* dl, const void* w_gate, void* dx, hipStream_t stream) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;
  if (!dx_perm || !pair_to_row || !topk_idx || !dl || !w_gate || !dx) return MOE_ERR_INVALID_ARG;
  if (!aligned16(dx_perm) || !aligned16(w_gate) || !aligned16(dx)) return MOE_ERR_INVALID_ARG;
  if (!row_vec_ok(d, d->D)) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_backward_dx(dx_perm, pair_to_row, topk_idx, dl, w_gate, dx, d->T, d->D, d->E,
                                            d->top_k, d->gate == MOE_GATE_SOFTMAX_FULL, d->dtype, stream));
}

int moe_group_transpose(const moe_dims* d, const void* src, int32_t n_cols, const int32_t* expert_offsets,
                        int32_t* koff, void* dst, int64_t ld, hipStream_t stream) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  int64_t need = 0;
  moe_wgrad_ld(d, &need);
  if (n_cols < 0 || ld < need) return MOE_ERR_INVALID_ARG;
  if (!expert_offsets || !koff || (ld > 0 && n_cols > 0 && (!dst || (d->T > 0 && !src)))) return MOE_ERR_INVALID_ARG;
  if (!row_vec_ok(d, n_cols)) return MOE_ERR_UNSUPPORTED;  // 16-byte row chunks
  hipError_t e = moe::launch_group_koff(expert_offsets, d->E, koff, stream);
  if (e == hipSuccess) e = moe::launch_group_transpose(src, n_cols, expert_offsets, koff, d->E, ld, dst, d->dtype, stream);
  return hip_status(e);
}

int moe_group_transpose_gather(const moe_dims* d, const void* x, int32_t n_cols, const int32_t* expert_offsets,
                               const int32_t* row_to_pair, int32_t* koff, void* dst, int64_t ld, hipStream_t stream) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  int64_t need = 0;
  moe_wgrad_ld(d, &need);
  if (n_cols < 0 || ld < need) return MOE_ERR_INVALID_ARG;
  if (!expert_offsets || !koff || (ld > 0 && n_cols > 0 && (!dst || (d->T > 0 && (!x || !row_to_pair)))))
    return MOE_ERR_INVALID_ARG;
  if (!row_vec_ok(d, n_cols)) return MOE_ERR_UNSUPPORTED;  // 16-byte row chunks
  hipError_t e = moe::launch_group_koff(expert_offsets, d->E, koff, stream);
  if (e == hipSuccess)
    e = moe::launch_group_transpose(x, n_cols, expert_offsets, koff, d->E, ld, dst, d->dtype, stream, row_to_pair,
                                    d->top_k);
  return hip_status(e);
}

int moe_expert_wgrad(const moe_dims* d, const void* a_t, const void* b_t, const int32_t* koff, int32_t M, int32_t N,
                     int64_t ld, float* out0, float* out1, int32_t split, hipStream_t stream) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  if (d->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || ld < 0 || split < 0 || split > M || ld % 64 != 0) return MOE_ERR_INVALID_ARG;
  if (!a_t || !b_t || !koff || !out0 || (split < M && !out1)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(a_t) || !aligned16(b_t) || !aligned16(out0) || (out1 && !aligned16(out1))) return MOE_ERR_INVALID_ARG;
  if (N % 4 != 0) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_wgrad_bf16(a_t, b_t, koff, d->E, M, N, ld, out0, out1, split, stream));
}

}  // extern "C"
