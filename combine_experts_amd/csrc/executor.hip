// Layer executors: the forward's five steps over micro-batches, optionally on two streams, with an
// optional shared expert; and the backward's steps in order.
//
// "Expert Parallelism and All-to-All" (DeepSeek-V3 splits the work into micro-batches so that the
// exchange of one hides behind the computation of another) and the EP-in-LLMs article,
// "Overlapping All-to-All with Computation" (dual-stream scheduling: the dispatch is issued while
// the compute units run other dense work such as the shared expert). On one GPU the exchanges are
// the permute and the combine; the schedule is
//
//   main:  R0 L0 P0 | S0 | R1 L1 P1 | S1 | wait F0, C0 | R2 L2 P2 | S2 | wait F1, C1 | ... | wait Fn-1, Cn-1
//   side:            wait P0, F0 (up, down) | wait P1, F1 | ...
//
// R route, L layout, P permute, S shared expert, F grouped FFN, C combine (+ shared output). Without
// an x_perm buffer there is no P: the up-projection of F gathers its rows from x itself. Every
// micro-batch owns disjoint slices of the caller's buffers, so the two streams never write the same
// memory; the main stream ends after the last combine, which waited for the last FFN, so all work
// of the call is ordered before whatever the caller enqueues next on the main stream.
#include "moe_common.h"

extern "C" {

int moe_event_create(hipEvent_t* event) {
  if (event == nullptr) return MOE_ERR_INVALID_ARG;
  return hipEventCreateWithFlags(event, hipEventDisableTiming) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_event_destroy(hipEvent_t event) {
  return hipEventDestroy(event) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_layer_forward(const moe_dims* d, const moe_layer_args* a, int32_t n_chunks, hipStream_t stream,
                      hipStream_t side_stream, const hipEvent_t* events) {
  if (d == nullptr || a == nullptr) return MOE_ERR_INVALID_ARG;
  if (n_chunks < 1 || d->T % n_chunks != 0) return MOE_ERR_INVALID_ARG;
  if (side_stream != nullptr && events == nullptr) return MOE_ERR_INVALID_ARG;
  if (a->shared_w1 != nullptr && (a->shared_F <= 0 || !a->shared_w2 || !a->shared_h || !a->shared_y ||
                                  !a->shared_offsets || (d->act == MOE_ACT_SWIGLU && !a->shared_w3)))
    return MOE_ERR_INVALID_ARG;
  moe_dims c = *d;
  c.T = d->T / n_chunks;
  const int64_t tc = c.T, k = d->top_k, D = d->D, E = d->E, ep = d->ep_size;
  const int64_t eb = d->dtype == MOE_BF16 ? 2 : 4;
  size_t ws_chunk = 0;
  int st = moe_workspace_size(&c, MOE_STAGE_LAYOUT, &ws_chunk);
  if (st != MOE_OK) return st;
  ws_chunk = (ws_chunk + 255) / 256 * 256;
  if (a->layout_ws == nullptr || a->layout_ws_bytes < ws_chunk * (size_t)n_chunks) return MOE_ERR_WORKSPACE;
  moe_dims sd = c;  // the shared expert: one expert over every token of the micro-batch
  sd.E = 1;
  sd.top_k = 1;
  sd.F = a->shared_F;
  sd.ep_size = 1;
  sd.ep_rank = 0;
  sd.n_groups = 0;
  sd.topk_groups = 0;
  sd.capacity_factor = 0.0;
  const bool two = side_stream != nullptr;
  hipStream_t fs = two ? side_stream : stream;
  auto chunk = [&](const void* base, int64_t c_idx, int64_t elems) -> const char* {
    return static_cast<const char*>(base) + c_idx * elems;
  };
  auto combine = [&](int64_t ci) -> int {
    const int64_t p0 = ci * tc * k;
    void* yc = static_cast<char*>(a->y) + ci * tc * D * eb;
    const void* add = a->shared_w1 ? chunk(a->shared_y, ci, tc * D * eb) : nullptr;
    return moe_unpermute_combine_add(&c, chunk(a->y_perm, ci, tc * k * D * eb), a->pair_to_row + p0,
                                     a->topk_gate + p0, add, yc, stream);
  };
  for (int64_t ci = 0; ci < n_chunks; ++ci) {
    const int64_t p0 = ci * tc * k;
    const void* xc = chunk(a->x, ci, tc * D * eb);
    void* xp = a->x_perm ? static_cast<char*>(a->x_perm) + p0 * D * eb : nullptr;
    void* hc = static_cast<char*>(a->h) + p0 * (int64_t)d->F * eb;
    void* yp = static_cast<char*>(a->y_perm) + p0 * D * eb;
    int32_t* eoff = a->expert_offsets + ci * (E + 1);
    float* lg = a->logits ? a->logits + ci * tc * E : nullptr;
    if ((st = moe_route(&c, xc, a->w_gate, a->bias, a->topk_idx + p0, a->topk_gate + p0, lg, stream)) != MOE_OK)
      return st;
    if ((st = moe_dispatch_layout(&c, a->topk_idx + p0, a->expert_counts + ci * E, eoff, a->rank_counts + ci * ep,
                                  a->rank_offsets + ci * (ep + 1), a->pair_to_row + p0, a->row_to_pair + p0,
                                  static_cast<char*>(a->layout_ws) + ci * ws_chunk, ws_chunk, stream)) != MOE_OK)
      return st;
    if (xp && (st = moe_permute(&c, xc, a->pair_to_row + p0, xp, stream)) != MOE_OK) return st;
    if (two) {
      if (hipEventRecord(events[2 * ci], stream) != hipSuccess) return MOE_ERR_HIP;
      if (hipStreamWaitEvent(side_stream, events[2 * ci], 0) != hipSuccess) return MOE_ERR_HIP;
    }
    if (a->pre != nullptr) {
      void* pc = static_cast<char*>(a->pre) + p0 * (int64_t)d->F * (d->act == MOE_ACT_SWIGLU ? 2 : 1) * eb;
      st = xp ? moe_expert_ffn_up_train(&c, xp, eoff, a->w1, a->w3, hc, pc, fs)
              : moe_expert_ffn_up_train_gather(&c, xc, a->row_to_pair + p0, eoff, a->w1, a->w3, hc, pc, fs);
      if (st != MOE_OK) return st;
    } else if (xp) {
      if ((st = moe_expert_ffn_up(&c, xp, eoff, a->w1, a->w3, hc, fs)) != MOE_OK) return st;
    } else if ((st = moe_expert_ffn_up_gather(&c, xc, a->row_to_pair + p0, eoff, a->w1, a->w3, hc, fs)) != MOE_OK) {
      return st;
    }
    st = a->down_ws ? moe_expert_ffn_down_splitk(&c, hc, eoff, a->w2, yp, a->down_ws, a->down_ws_bytes, fs)
                    : moe_expert_ffn_down(&c, hc, eoff, a->w2, yp, fs);
    if (st != MOE_OK) return st;
    if (two && hipEventRecord(events[2 * ci + 1], side_stream) != hipSuccess) return MOE_ERR_HIP;
    if (a->shared_w1 != nullptr) {
      void* sh = static_cast<char*>(a->shared_h) + ci * tc * (int64_t)a->shared_F * eb;
      void* sy = static_cast<char*>(a->shared_y) + ci * tc * D * eb;
      if ((st = moe_expert_ffn_up(&sd, xc, a->shared_offsets, a->shared_w1, a->shared_w3, sh, stream)) != MOE_OK)
        return st;
      if ((st = moe_expert_ffn_down(&sd, sh, a->shared_offsets, a->shared_w2, sy, stream)) != MOE_OK) return st;
    }
    if (ci > 0) {
      if (two && hipStreamWaitEvent(stream, events[2 * (ci - 1) + 1], 0) != hipSuccess) return MOE_ERR_HIP;
      if ((st = combine(ci - 1)) != MOE_OK) return st;
    }
  }
  if (two && hipStreamWaitEvent(stream, events[2 * (n_chunks - 1) + 1], 0) != hipSuccess) return MOE_ERR_HIP;
  return combine(n_chunks - 1);
}

int moe_layer_backward(const moe_dims* d, const moe_backward_args* a, hipStream_t stream) {
  if (d == nullptr || a == nullptr) return MOE_ERR_INVALID_ARG;
  int st = MOE_OK;
  const int nm = d->act == MOE_ACT_SWIGLU ? 2 : 1;
  // without transposed copies the data-gradient GEMMs read the weights as stored
  const bool natural = a->w13t == nullptr && a->w2t == nullptr;
  if (a->refresh_weights && !natural) {
    if ((st = moe_transpose_weights(d, a->w1, a->w3, a->w2, a->w13t, a->w2t, stream)) != MOE_OK) return st;
  }
  if ((st = moe_backward_combine(d, a->dy, a->pair_to_row, a->topk_gate, a->y_perm, a->dy_perm, a->dgate, stream)) !=
      MOE_OK)
    return st;
  st = natural ? moe_expert_ffn_down_backward_w(d, a->dy_perm, a->expert_offsets, a->w2, a->pre, a->da, stream)
               : moe_expert_ffn_down_backward(d, a->dy_perm, a->expert_offsets, a->w2t, a->pre, a->da, stream);
  if (st != MOE_OK) return st;
  st = natural ? moe_expert_ffn_up_backward_w(d, a->da, a->expert_offsets, a->w1, a->w3, a->dx_perm, stream)
               : moe_expert_ffn_up_backward(d, a->da, a->expert_offsets, a->w13t, a->dx_perm, stream);
  if (st != MOE_OK) return st;
  // a dropless forward layout doubles as the router's grouping of the pairs by expert
  const bool grouped = d->capacity_factor <= 0.0;
  if ((st = moe_router_backward(d, a->x, a->logits, a->topk_idx, a->topk_gate, a->dgate,
                                grouped ? a->expert_offsets : nullptr, grouped ? a->row_to_pair : nullptr, a->dl,
                                a->dw_gate, a->dbias, a->router_ws, a->router_ws_bytes, stream)) != MOE_OK)
    return st;
  if ((st = moe_backward_dx(d, a->dx_perm, a->pair_to_row, a->topk_idx, a->dl, a->w_gate, a->dx, stream)) != MOE_OK)
    return st;
  if ((st = moe_group_transpose(d, a->dy_perm, d->D, a->expert_offsets, a->koff, a->dy_perm_t, a->ld, stream)) != MOE_OK)
    return st;
  if ((st = moe_group_transpose(d, a->h, d->F, a->expert_offsets, a->koff, a->h_t, a->ld, stream)) != MOE_OK) return st;
  if ((st = moe_expert_wgrad(d, a->dy_perm_t, a->h_t, a->koff, d->D, d->F, a->ld, a->dw2, nullptr, d->D, stream)) !=
      MOE_OK)
    return st;
  if ((st = moe_group_transpose(d, a->da, nm * d->F, a->expert_offsets, a->koff, a->da_t, a->ld, stream)) != MOE_OK)
    return st;
  // x_perm^T, or, without a saved x_perm, the same rows gathered from x on the way into the transpose
  st = a->x_perm ? moe_group_transpose(d, a->x_perm, d->D, a->expert_offsets, a->koff, a->x_perm_t, a->ld, stream)
                 : moe_group_transpose_gather(d, a->x, d->D, a->expert_offsets, a->row_to_pair, a->koff, a->x_perm_t,
                                              a->ld, stream);
  if (st != MOE_OK) return st;
  return moe_expert_wgrad(d, a->da_t, a->x_perm_t, a->koff, nm * d->F, d->D, a->ld, a->dw1, a->dw3, d->F, stream);
}

}  // extern "C"
