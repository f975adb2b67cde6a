/*
 * moe.h -- C ABI of libmoe: the one-GPU share of a sparse mixture-of-experts layer on MI355X (gfx950).
 *
 *   y = sum_{i in TopK(G(x), k)} g_i(x) * Expert_i(x)
 *
 * The layer runs as five steps, each an entry point below, all enqueued on the caller's HIP stream:
 *   moe_route              router logits, top-k selection, gate values
 *   moe_dispatch_layout    per-expert / per-rank counts and offsets, the stable permutation
 *   moe_permute            copy each kept (token, expert) pair's row into its expert's contiguous group
 *   moe_expert_ffn         grouped expert FFN over the contiguous groups (= ffn_up then ffn_down)
 *   moe_unpermute_combine  reverse permutation and gate-weighted sum of each token's k outputs
 *
 * Pages cited (titles as the pages give them):
 *   [EPA2A] "Expert Parallelism and All-to-All"
 *   [A2AC]  "Expert Parallelism > All-to-All Communication"
 *   [COMM]  "Expert Parallelism > Communication Overhead Analysis"
 *   [CH10]  "Chapter 10: MoE parallelism" (infra-guide), section 4 on load balancing
 *   [EPLLM] "Expert Parallelism in Large Language Models: How All-to-All Token Dispatch, Capacity
 *           Factors, and Parallel Folding Scale MoE Architectures"
 *
 * Conventions, all entry points:
 *   - Ownership: the caller allocates and owns every buffer (inputs, outputs, workspaces). The
 *     library never allocates, frees or synchronises; it only enqueues kernels on `stream`.
 *   - State: none kept between calls; calls on different streams do not interact.
 *   - Layout: row-major. x[T,D]; W_g[E,D]; W1, W3 [E,F,D]; W2 [E,D,F] (each weight matrix is
 *     (out, in), so every GEMM operand is contiguous along its reduction dimension).
 *   - Element type of x, weights, x_perm, h, y_perm, y: dims.dtype (MOE_F32 or MOE_BF16). Router
 *     logits, bias and gates are always float32; indices and counts are int32.
 *   - Sizes that depend on the routing (kept rows N, per-expert counts) stay on the device: the
 *     row-indexed buffers are sized for the worst case N_max = T*top_k rows and kernels read
 *     N = expert_offsets[E] themselves. The host never waits on the GPU.
 *   - Pointers to element arrays must be 16-byte aligned.
 *   - Empty inputs: T = 0 is valid everywhere. An array whose size is zero for the given dims (for
 *     T = 0: x, the per-pair and per-row arrays, dy, dl; with no padded slots: slot_to_pair,
 *     x_pad, h_pad, y_pad) may be NULL; outputs that do not scale with T (counts, offsets, weight
 *     and bias gradients) are still written (zeros).
 *   - Errors: every entry point returns an int status (MOE_OK = 0). Argument checks run on the host
 *     before anything is enqueued; MOE_ERR_HIP reports a launch failure (hipGetLastError).
 *     Device-side preconditions (topk_idx values in [0,E)) are the caller's to keep.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null required pointer, inconsistent dims, misaligned pointer */
  MOE_ERR_UNSUPPORTED = 2, /* valid dims no kernel of this library handles (see each entry point) */
  MOE_ERR_WORKSPACE = 3,   /* workspace pointer null or smaller than moe_workspace_size() */
  MOE_ERR_HIP = 4          /* a kernel launch failed */
};

enum moe_gate {
  MOE_GATE_SOFTMAX_TOPK = 0, /* g = softmax over the k selected logits ([EPLLM] pipeline step 1) */
  MOE_GATE_SIGMOID_TOPK = 1, /* g_j = sigmoid(l_j) / sum of sigmoid over the k selected */
  MOE_GATE_SOFTMAX_FULL = 2  /* g_j = softmax over all E logits at the selected experts */
};

enum moe_act {
  MOE_ACT_SWIGLU = 0, /* W2 * (SiLU(W1 h) (*) (W3 h))  -- three matrices per expert */
  MOE_ACT_GELU = 1    /* W2 * GELU(W1 h), exact erf GELU -- two matrices, w3 unused */
};

enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 };

enum moe_stage {
  MOE_STAGE_LAYOUT = 0,     /* scratch of moe_dispatch_layout */
  MOE_STAGE_FFN = 1,        /* scratch of moe_expert_ffn */
  MOE_STAGE_ROUTE_STATS = 2, /* the prob_partials buffer of moe_route_ex / moe_load_balance */
  MOE_STAGE_ROUTER_BWD = 3,  /* scratch of moe_router_backward (column-sum partials of dbias) */
  MOE_STAGE_FFN_DOWN = 4     /* split-K scratch of moe_expert_ffn_down_splitk; 0 bytes: these dims are
                                not split */
};

/* Problem statement of one layer call ([COMM] volume equation: B*S tokens as T, top-k as K,
 * hidden size D; [EPLLM] capacity equation; [A2AC] expert -> device map).
 *   T, D, E, top_k, F   tokens, hidden size, experts, experts per token, expert hidden size
 *   capacity_factor     <= 0: dropless. > 0: C = ceil(capacity_factor * top_k * T / E) rows/expert
 *   ep_size, ep_rank    emulated expert-parallel size (E % ep_size == 0; rank r owns experts
 *                       [r*E/ep_size, (r+1)*E/ep_size)); ep_rank only labels the local rank
 *   n_groups, topk_groups  0: no group limit. Otherwise experts form n_groups contiguous groups and
 *                       each token may only pick experts of its topk_groups best groups
 *                       ([EPA2A] node-limited routing); a group's score is the sum of its
 *                       top_k/topk_groups best member scores (sigmoid scores under
 *                       MOE_GATE_SIGMOID_TOPK, logits otherwise)
 *   gate, act, dtype    enum moe_gate, enum moe_act, enum moe_dtype */
typedef struct moe_dims {
  int32_t T, D, E, top_k, F;
  int32_t ep_size, ep_rank;
  int32_t n_groups, topk_groups;
  int32_t gate, act, dtype;
  double capacity_factor;
} moe_dims;

/* Expert capacity C ([EPLLM] "Static Capacity Factors and Token Dropping", capacity equation),
 * evaluated on the host in IEEE double; T*top_k when dropless. Host only. */
int moe_capacity(const moe_dims* d, int32_t* capacity);

/* Workspace bytes that `stage` needs (MOE_STAGE_LAYOUT: moe_dispatch_layout; MOE_STAGE_FFN:
 * moe_expert_ffn, which keeps the expert hidden activations h[T*top_k, F] there, followed by the
 * MOE_STAGE_FFN_DOWN scratch of its down-projection). Host only. */
int moe_workspace_size(const moe_dims* d, int stage, size_t* bytes);

/* Router ([EPLLM] "The Execution Pipeline" step 1; layer equation of "The Distributed MoE Dilemma").
 *   x [T,D] dtype; w_gate [E,D] dtype; bias [E] float32 or NULL (added to every token's logits).
 *   topk_idx [T,top_k] int32 out: slot j = the (j+1)-th best expert by (-logit, expert index), so
 *     exact ties go to the lower index; with a group limit only experts of kept groups qualify.
 *   topk_gate [T,top_k] float32 out: gate values per enum moe_gate.
 *   logits [T,E] float32 out, or NULL: the float32 logits the selection was taken on.
 * Logits are accumulated and kept in float32. Unsupported: E > 256, top_k > 32, D % 8 != 0, and
 * for MOE_BF16 D % 64 != 0. */
int moe_route(const moe_dims* d, const void* x, const void* w_gate, const float* bias,
              int32_t* topk_idx, float* topk_gate, float* logits, hipStream_t stream);

/* Router with the two load-balancing by-products (moe_route is this call with both NULL).
 *   select_bias [E] float32 or NULL: a per-expert bias that moves the selection only -- the
 *     bias-adjusted routing scores of aux-loss-free balancing ([EPLLM] "Modern Dropless Dynamic
 *     Dispatch"; [CH10] section 4, load balancing). The selection ranks s_e + select_bias[e], where
 *     s_e = sigmoid(logit_e) under MOE_GATE_SIGMOID_TOPK and s_e = logit_e otherwise, in float32,
 *     ties to the lower index; with a group limit the group scores are taken on these biased
 *     scores. Gate values are computed from the unbiased logits of the chosen experts.
 *   prob_partials [ceil(T/64), E] float32 out, or NULL: row b holds, for each expert, the sum of
 *     the router probabilities of tokens [64b, 64b+64) -- softmax over all E logits for softmax
 *     gates, sigmoid scores normalised over all E for sigmoid gates. Its size in bytes is
 *     moe_workspace_size(MOE_STAGE_ROUTE_STATS); moe_load_balance consumes it.
 * Everything else as moe_route. */
int moe_route_ex(const moe_dims* d, const void* x, const void* w_gate, const float* bias,
                 const float* select_bias, int32_t* topk_idx, float* topk_gate, float* logits,
                 float* prob_partials, hipStream_t stream);

/* Load-balance statistics of one routed batch ([EPLLM] "Static Capacity Factors and Token
 * Dropping", auxiliary-loss equation L_aux = alpha * E * sum_i f_i * P_i) and, optionally, one
 * aux-loss-free bias step.
 *   expert_counts [E] int32 in (moe_dispatch_layout's, before any capacity cut);
 *   prob_partials in (moe_route_ex's; may be NULL only when T == 0);
 *   stats [2E+2] float32 out: f_i = counts_i / (T*top_k) for i < E; P_i = mean router probability
 *     of expert i at E+i; L_aux at 2E; the load imbalance max_i counts_i / mean_i counts_i at 2E+1
 *     ([EPA2A] "When it breaks": the busiest expert sets the pace). All zero when T == 0.
 *   select_bias [E] float32 in/out, or NULL: b_i += gamma * sign(mean load - load_i), the sign
 *     decided exactly in integers, the add in float32.
 * Deterministic: every sum runs in a fixed order. One small kernel (one workgroup). */
int moe_load_balance(const moe_dims* d, const int32_t* expert_counts, const float* prob_partials,
                     float alpha, float* stats, float gamma, float* select_bias, hipStream_t stream);

/* Dispatch layout ([EPA2A] "The two exchanges": each device sorts its tokens by destination
 * expert; [EPLLM] pipeline steps 1-2: replicate each token k times tagged with expert and rank,
 * group them contiguously per rank; [A2AC] send counts per device).
 * Pair id p = t*top_k + j. Rows are ordered by (expert, p): stable. With a capacity C an expert
 * keeps its first C pairs in p order and drops the rest. Outputs (int32, device):
 *   expert_counts [E]     pairs routed to each expert before the capacity cut
 *   expert_offsets [E+1]  first row of each expert's kept group; expert_offsets[E] = N kept rows
 *   rank_counts [ep_size] kept rows bound for each emulated rank (the all-to-all send counts)
 *   rank_offsets [ep_size+1] first row of each rank's send chunk
 *   pair_to_row [T*top_k] row of pair p, or -1 when dropped
 *   row_to_pair [T*top_k] pair held by row r for r < N, -1 for r >= N
 *   ws, ws_bytes          scratch of moe_workspace_size(MOE_STAGE_LAYOUT) bytes
 * Deterministic: the result does not depend on the order in which the GPU runs its threads. */
int moe_dispatch_layout(const moe_dims* d, const int32_t* topk_idx, int32_t* expert_counts,
                        int32_t* expert_offsets, int32_t* rank_counts, int32_t* rank_offsets,
                        int32_t* pair_to_row, int32_t* row_to_pair, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* moe_dispatch_layout for callers that cannot allocate (code under HIP graph capture, serving loops
 * or harnesses that forbid hipMalloc): the same outputs, bit for bit, with no workspace argument.
 * Its per-chunk histograms live in a static device array of the library, MOE_LAYOUT_NOALLOC_SCRATCH_BYTES
 * (1 MiB) per GPU, held until the process ends; nothing is allocated, freed or cleared per call.
 * Limit: ceil(T*top_k / 512) * E * 4 bytes must fit that array (e.g. T*top_k = 131072 pairs over up
 * to E = 1024 experts); larger problems return MOE_ERR_WORKSPACE before anything is enqueued.
 * All calls on one GPU share the array: calls that overlap in time on one GPU (different streams,
 * or threads without ordering) race and must be serialised by the caller. */
#define MOE_LAYOUT_NOALLOC_SCRATCH_BYTES (1u << 20)
int moe_dispatch_layout_noalloc(const moe_dims* d, const int32_t* topk_idx, int32_t* expert_counts,
                                int32_t* expert_offsets, int32_t* rank_counts, int32_t* rank_offsets,
                                int32_t* pair_to_row, int32_t* row_to_pair, hipStream_t stream);

/* Permute ([EPLLM] pipeline step 2): x_perm[pair_to_row[t*k+j]] = x[t] for every kept pair.
 *   x [T,D] dtype in; pair_to_row [T*top_k] int32 in; x_perm [T*top_k, D] dtype out (rows >= N are
 *   left untouched). A bit-exact copy; each x row is read once. */
int moe_permute(const moe_dims* d, const void* x, const int32_t* pair_to_row, void* x_perm,
                hipStream_t stream);

/* Grouped expert FFN ([EPLLM] pipeline step 4: one batched GEMM per local expert over all of its
 * rows; expert = W2 * (SiLU(W1 h) (*) (W3 h)), or W2 * GELU(W1 h)). Rows [expert_offsets[e],
 * expert_offsets[e+1]) of x_perm go through expert e; no padding and no dropping.
 *   x_perm [T*top_k, D] in; w1, w3 [E,F,D]; w2 [E,D,F]; w3 may be NULL for MOE_ACT_GELU.
 *   y_perm [T*top_k, D] out (rows >= N untouched); ws: moe_workspace_size(MOE_STAGE_FFN) bytes.
 * bf16: matrix-core products with float32 accumulation; h is rounded to bf16 between the two
 * GEMMs; outputs rounded to nearest even. Unsupported: D or F not a multiple of 64, or (bf16) an
 * operand span of 4 GiB or more: 320 rows of x_perm, h or a weight matrix (320*D*2, 320*F*2 bytes)
 * or one expert's weight matrix read K-major by the data-gradient forms (D*F*2, or 2*D*F*2 for
 * W1 and W3), since the kernels address them with 32-bit offsets. */
int moe_expert_ffn(const moe_dims* d, const void* x_perm, const int32_t* expert_offsets,
                   const void* w1, const void* w3, const void* w2, void* y_perm, void* ws,
                   size_t ws_bytes, hipStream_t stream);

/* First half of moe_expert_ffn: h[r] = act(W1[e] x_perm[r], W3[e] x_perm[r]) for each kept row r of
 * expert e.  h [T*top_k, F] dtype out (rows >= N untouched). Same rules as moe_expert_ffn. */
int moe_expert_ffn_up(const moe_dims* d, const void* x_perm, const int32_t* expert_offsets,
                      const void* w1, const void* w3, void* h, hipStream_t stream);

/* moe_permute followed by moe_expert_ffn_up in one launch: the up-projection reads row r straight from
 * x[row_to_pair[r] / top_k] ([EPLLM] pipeline steps 2 and 4 with the permuted copy of x left out).
 * Output identical bit for bit to the two calls. x [T,D] in; row_to_pair [T*top_k] int32 in (as
 * moe_dispatch_layout wrote it: entries [0, N) are read); h [T*top_k, F] out. Also unsupported
 * (bf16): x of 4 GiB or more (T*D*2 bytes; the gathered rows are addressed by 32-bit offsets from
 * x); pass x through moe_permute and moe_expert_ffn_up instead. */
int moe_expert_ffn_up_gather(const moe_dims* d, const void* x, const int32_t* row_to_pair,
                             const int32_t* expert_offsets, const void* w1, const void* w3, void* h,
                             hipStream_t stream);

/* Second half of moe_expert_ffn: y_perm[r] = W2[e] h[r]. h [T*top_k, F] in; y_perm [T*top_k, D] out. */
int moe_expert_ffn_down(const moe_dims* d, const void* h, const int32_t* expert_offsets,
                        const void* w2, void* y_perm, hipStream_t stream);

/* moe_expert_ffn_down with an optional workspace that lets it split the reduction (K = F) over several
 * blocks per output tile when the problem has too few tiles to fill the GPU ([EPLLM] "Static Capacity
 * Factors and Token Dropping": a capacity-bound layer leaves each expert at most C rows, so the
 * down-projection has E x ceil(C/320) x ceil(D/256) tiles). Block s of a tile sums K stages
 * [s*F/S/64, (s+1)*F/S/64) into a float32 partial; one more pass adds the S partials in split order
 * and rounds once, so the result is deterministic (it differs from the unsplit sum by float32
 * rounding only). bf16 only; S > 1 when F >= 2048 and the layer has at most 64 such tiles.
 *   ws, ws_bytes  moe_workspace_size(MOE_STAGE_FFN_DOWN) bytes: S x T*top_k x D float32 partials. When
 *                 that size is 0, or ws is NULL, this is moe_expert_ffn_down.
 * Other arguments as moe_expert_ffn_down. The layer executor splits only when its caller hands it such a
 * workspace (moe_layer_args.down_ws); without one its micro-batches give the same bits as the whole batch. */
int moe_expert_ffn_down_splitk(const moe_dims* d, const void* h, const int32_t* expert_offsets, const void* w2,
                               void* y_perm, void* ws, size_t ws_bytes, hipStream_t stream);

/* Unpermute + combine ([EPLLM] pipeline step 6: restore order, weight each of the k expert
 * outputs by its gate and sum; the residual is left to the caller):
 *   y[t] = sum over slots j with pair_to_row[t*k+j] >= 0 of topk_gate[t*k+j] * y_perm[row].
 * Sums in float32 in slot order, rounds once. A token whose pairs were all dropped gets 0.
 *   y_perm [T*top_k, D] dtype in; pair_to_row, topk_gate [T*top_k]; y [T,D] dtype out. */
int moe_unpermute_combine(const moe_dims* d, const void* y_perm, const int32_t* pair_to_row,
                          const float* topk_gate, void* y, hipStream_t stream);

/* ---- Cluster view on one GPU: the expert-parallel data flow, emulated ----------------------------
 * n_src source shards of T/n_src contiguous tokens each route and lay out their own tokens
 * (moe_route / moe_dispatch_layout / moe_permute called with dims.T = T/n_src on pointer offsets);
 * source s keeps its sent rows at rows [s*src_stride, s*src_stride + N_s) of one concatenated send
 * buffer. Rank r (of dims.ep_size) owns experts [r*E/ep_size, (r+1)*E/ep_size) ([A2AC] dispatch
 * example). */

/* [src, dst] counts of (token, expert) pairs before any capacity cut: matrix[s*ep_size + d] = pairs
 * of tokens [s*T/n_src, (s+1)*T/n_src) routed to experts of rank d ([A2AC] routing simulation: the
 * per-device bincount, one row per source device). topk_idx [T, top_k]; matrix [n_src, ep_size]
 * int32 out. Requires T % n_src == 0. Ids outside [0, E) are not counted. */
int moe_dispatch_matrix(const moe_dims* d, const int32_t* topk_idx, int32_t n_src, int32_t* matrix,
                        hipStream_t stream);

/* Receive side of rank `rank` ([EPA2A] "The two exchanges": after the dispatch exchange a device
 * holds one chunk per source, each sorted by its local experts, and regroups them per expert).
 *   src_expert_offsets [n_src, E+1] int32 in: each source's own expert_offsets.
 *   recv_counts [n_src] out: rows each source sends to this rank.
 *   expert_offsets [E/ep_size + 1] out: offsets of this rank's local experts in the regrouped rows.
 *   grouped_to_src_row [n_rows_max] out: send-buffer row (s*src_stride + source row) of each
 *     regrouped row, regrouped order = (local expert, source, source row); -1 past the last row.
 * Feed it to moe_gather_rows to run the exchange and the regroup as one pass, and to
 * moe_scatter_rows to send expert outputs back. Unsupported: n_src*(2E/ep_size)+E/ep_size > 16384. */
int moe_recv_layout(const moe_dims* d, int32_t n_src, int32_t rank, int64_t src_stride,
                    const int32_t* src_expert_offsets, int32_t* recv_counts, int32_t* expert_offsets,
                    int32_t* grouped_to_src_row, int32_t n_rows_max, hipStream_t stream);

/* dst[i] = src[row_map[i]] for i < n_rows with row_map[i] >= 0 (rows of D elements of dims.dtype;
 * a bit-exact copy; rows with -1 untouched). */
int moe_gather_rows(const moe_dims* d, int64_t n_rows, const int32_t* row_map, const void* src, void* dst,
                    hipStream_t stream);

/* dst[row_map[i]] = src[i] for i < n_rows with row_map[i] >= 0. row_map must not repeat a target. */
int moe_scatter_rows(const moe_dims* d, int64_t n_rows, const int32_t* row_map, const void* src, void* dst,
                     hipStream_t stream);

/* ---- Fixed-capacity (padded) layout ---------------------------------------------------------------
 * [EPLLM] "Static Capacity Factors and Token Dropping": every expert owns C rows of an [E*C, D]
 * buffer (C = moe_capacity, dims.capacity_factor > 0 required); unused rows are zero padding that
 * the expert FFN still computes. Kept pairs are exactly those of the compact layout with the same C.
 *   In: topk_idx, and moe_dispatch_layout's expert_offsets, pair_to_row, row_to_pair (same dims).
 *   pair_to_slot [T*top_k] out: e*C + rank of the pair in its expert, or -1 when dropped.
 *   slot_to_pair [E*C] out: the pair in each slot, -1 for padding.
 *   padded_offsets [E+1] out: e*C (the expert_offsets of the padded buffer). */
int moe_padded_layout(const moe_dims* d, const int32_t* topk_idx, const int32_t* expert_offsets,
                      const int32_t* pair_to_row, const int32_t* row_to_pair, int32_t* pair_to_slot,
                      int32_t* slot_to_pair, int32_t* padded_offsets, hipStream_t stream);

/* x_pad[s] = x[slot_to_pair[s] / top_k] for filled slots, zeros for padding slots. x_pad [E*C, D]. */
int moe_permute_padded(const moe_dims* d, const void* x, const int32_t* slot_to_pair, void* x_pad,
                       hipStream_t stream);

/* The grouped expert FFN over the padded buffer: as moe_expert_ffn_up / _down with
 * expert_offsets = padded_offsets and E*C rows (x_pad, h_pad [E*C, F], y_pad [E*C, D]). Padding rows
 * come out as exact zeros. Combine with moe_unpermute_combine(pair_to_row = pair_to_slot). */
int moe_expert_ffn_padded_up(const moe_dims* d, const void* x_pad, const int32_t* padded_offsets,
                             const void* w1, const void* w3, void* h_pad, hipStream_t stream);
int moe_expert_ffn_padded_down(const moe_dims* d, const void* h_pad, const int32_t* padded_offsets,
                               const void* w2, void* y_pad, hipStream_t stream);

/* moe_unpermute_combine plus an addend: y[t] = sum_j g[t,j] * y_perm[row] + addend[t], summed in
 * float32 (the k slots in slot order, then the addend) and rounded once. addend [T, D] dtype, or NULL
 * (then this is moe_unpermute_combine). Used for a shared expert's output. */
int moe_unpermute_combine_add(const moe_dims* d, const void* y_perm, const int32_t* pair_to_row,
                              const float* topk_gate, const void* addend, void* y, hipStream_t stream);

/* ---- Layer executor: micro-batches on two streams, optional shared expert --------------------------
 * [EPA2A] (DeepSeek-V3 splits the work into micro-batches so one micro-batch's exchange hides behind
 * another's computation); [EPLLM] "Overlapping All-to-All with Computation" (dual-stream
 * scheduling; the shared expert's computation runs while the dispatch is in flight). On one GPU the
 * permute and the combine stand in for the two exchanges. With n_chunks micro-batches of
 * T/n_chunks tokens, micro-batch c's grouped FFN runs on `side_stream` while `stream` routes, lays
 * out and permutes micro-batch c+1, runs the shared expert and combines micro-batch c-1.
 *
 * Buffers (all caller-owned, device): the whole-batch buffers of the five steps; micro-batch c uses
 * entries / rows [c*Tc*top_k, (c+1)*Tc*top_k) of topk_idx, topk_gate, pair_to_row, row_to_pair,
 * x_perm, h, y_perm (whose row indices are local to the micro-batch), and slice c of the per-batch
 * arrays expert_counts [n_chunks, E], expert_offsets [n_chunks, E+1], rank_counts [n_chunks, ep],
 * rank_offsets [n_chunks, ep+1], layout_ws [n_chunks, roundup256(moe_workspace_size(LAYOUT) at
 * T = Tc)]. A capacity factor applies per micro-batch (C from Tc). */
typedef struct moe_layer_args {
  const void* x;             /* [T, D] */
  const void* w_gate;        /* [E, D] */
  const float* bias;         /* [E] or NULL */
  const void* w1;            /* [E, F, D] */
  const void* w3;            /* [E, F, D] or NULL (GELU) */
  const void* w2;            /* [E, D, F] */
  void* y;                   /* [T, D] out */
  int32_t* topk_idx;         /* [T*top_k] */
  float* topk_gate;          /* [T*top_k] */
  int32_t* pair_to_row;      /* [T*top_k] */
  int32_t* row_to_pair;      /* [T*top_k] */
  void* x_perm;              /* [T*top_k, D], or NULL: the up-projection gathers its rows from x
                                (moe_expert_ffn_up_gather, or moe_expert_ffn_up_train_gather when pre
                                is set) */
  void* h;                   /* [T*top_k, F] */
  void* y_perm;              /* [T*top_k, D] */
  int32_t* expert_counts;    /* [n_chunks, E] */
  int32_t* expert_offsets;   /* [n_chunks, E+1] */
  int32_t* rank_counts;      /* [n_chunks, ep_size] */
  int32_t* rank_offsets;     /* [n_chunks, ep_size+1] */
  void* layout_ws;
  size_t layout_ws_bytes;
  /* optional shared expert (shared_w1 == NULL: none), hidden size shared_F, same activation */
  const void* shared_w1;     /* [shared_F, D] */
  const void* shared_w3;     /* [shared_F, D] or NULL (GELU) */
  const void* shared_w2;     /* [D, shared_F] */
  int32_t shared_F;
  void* shared_h;            /* [T, shared_F] scratch */
  void* shared_y;            /* [T, D] scratch */
  const int32_t* shared_offsets; /* int32 [2] = {0, T/n_chunks} */
  /* optional training outputs: the router's float32 logits [T, E] and the up-projection's
   * pre-activations [T*top_k, 2F] (SwiGLU) or [T*top_k, F] (GELU), as moe_layer_backward reads them
   * (pre: bf16 only) */
  float* logits;
  void* pre;
  /* optional split-K scratch of the down-projection, or NULL (no split): each micro-batch's
   * down-projection runs as moe_expert_ffn_down_splitk at T = T/n_chunks with this workspace, which
   * must hold moe_workspace_size(MOE_STAGE_FFN_DOWN) at that T (else MOE_ERR_WORKSPACE) and be 16-byte
   * aligned. The micro-batches' FFNs run one after another on one stream, so one region serves them
   * all. With it, micro-batches give the whole batch's bits only where both split the same way. */
  void* down_ws;
  size_t down_ws_bytes;
} moe_layer_args;

/* Runs the layer as above. side_stream NULL: everything on `stream`, micro-batch after micro-batch.
 * Otherwise `events` holds 2*n_chunks events from moe_event_create (or hipEventCreateWithFlags with
 * hipEventDisableTiming), not shared with a concurrent call. All work of the call is ordered before
 * later work on `stream`. Requires T % n_chunks == 0; the rest as the five entry points. */
int moe_layer_forward(const moe_dims* d, const moe_layer_args* a, int32_t n_chunks, hipStream_t stream,
                      hipStream_t side_stream, const hipEvent_t* events);

/* Host helpers for the executor's events (hipEventCreateWithFlags(.., hipEventDisableTiming) and
 * hipEventDestroy). */
int moe_event_create(hipEvent_t* event);
int moe_event_destroy(hipEvent_t event);

/* ---- Backward of the one-GPU share -------------------------------------------------------------------
 * The chain rule through the forward steps in reverse with the routing decision (selection, drops)
 * held fixed ([EPLLM] "The Execution Pipeline" gives the forward steps; training runs them
 * backwards). For the upstream gradient dy [T, D] of y:
 *   dy_perm[row(t,j)] = g[t,j] dy[t]; dgate[t,j] = <dy[t], y_perm[row]>        moe_backward_combine
 *   da = act'(a) (dy_perm W2) per expert, from the saved pre-activations a     moe_expert_ffn_down_backward
 *   dx_perm = da [W1; W3] per expert                                           moe_expert_ffn_up_backward
 *   dl = gate backward of dgate; dW_g = dl^T x; dbias = sum_t dl               moe_router_backward
 *   dx[t] = sum_j dx_perm[row(t,j)] + sum_e dl[t,e] W_g[e]                     moe_backward_dx
 *   dW2[e] = dy_perm^T h, [dW1; dW3][e] = da^T x_perm (ragged sums over rows)   moe_expert_wgrad on
 *                                                                              moe_group_transpose'd operands
 * The grouped GEMM steps take bf16 only (MOE_ERR_UNSUPPORTED for float32). Weight gradients are float32. */

/* Forward up-projection for training: as moe_expert_ffn_up, and the pre-activations go to pre:
 * SwiGLU pre [T*top_k, 2F] = [W1 x | W3 x], GELU pre [T*top_k, F] = W1 x (bf16, rounded once). */
int moe_expert_ffn_up_train(const moe_dims* d, const void* x_perm, const int32_t* expert_offsets,
                            const void* w1, const void* w3, void* h, void* pre, hipStream_t stream);

/* moe_expert_ffn_up_train with its rows gathered from x (x_perm[r] = x[row_to_pair[r] / top_k], as
 * moe_expert_ffn_up_gather): the same h and pre, bit for bit, with no x_perm. Unsupported for x of
 * 4 GiB or more, as moe_expert_ffn_up_gather. */
int moe_expert_ffn_up_train_gather(const moe_dims* d, const void* x, const int32_t* row_to_pair,
                                   const int32_t* expert_offsets, const void* w1, const void* w3, void* h,
                                   void* pre, hipStream_t stream);

/* The weights as the data-gradient GEMMs read them: w2t [E, F, D] = W2^T; w13t [E, D, 2F] =
 * [W1^T | W3^T] (SwiGLU) or [E, D, F] = W1^T (GELU). Once per weight update. */
int moe_transpose_weights(const moe_dims* d, const void* w1, const void* w3, const void* w2, void* w13t,
                          void* w2t, hipStream_t stream);

/* dy_perm [T*top_k, D] out (rows >= N untouched); dgate [T*top_k] float32 out (0 for dropped pairs). */
int moe_backward_combine(const moe_dims* d, const void* dy, const int32_t* pair_to_row, const float* topk_gate,
                         const void* y_perm, void* dy_perm, float* dgate, hipStream_t stream);

/* da [T*top_k, 2F] (SwiGLU: [da1 | da3]) or [T*top_k, F] (GELU) out, from dh = dy_perm W2 and pre. */
int moe_expert_ffn_down_backward(const moe_dims* d, const void* dy_perm, const int32_t* expert_offsets,
                                 const void* w2t, const void* pre, void* da, hipStream_t stream);

/* dx_perm [T*top_k, D] out = da [W1; W3] per expert (w13t from moe_transpose_weights). */
int moe_expert_ffn_up_backward(const moe_dims* d, const void* da, const int32_t* expert_offsets,
                               const void* w13t, void* dx_perm, hipStream_t stream);

/* The two data-gradient GEMMs on the weights as the forward keeps them (w2 [E,D,F]; w1, w3 [E,F,D]),
 * with no transposed copies: the kernels load K-major weight slices and transpose them in the LDS
 * reads. Same arguments and results, bit for bit, as moe_expert_ffn_down_backward /
 * moe_expert_ffn_up_backward on moe_transpose_weights' output; w3 may be NULL for MOE_ACT_GELU. */
int moe_expert_ffn_down_backward_w(const moe_dims* d, const void* dy_perm, const int32_t* expert_offsets,
                                   const void* w2, const void* pre, void* da, hipStream_t stream);
int moe_expert_ffn_up_backward_w(const moe_dims* d, const void* da, const int32_t* expert_offsets, const void* w1,
                                 const void* w3, void* dx_perm, hipStream_t stream);

/* Router backward: dl [T, E] float32 out (0 where a logit gets no gradient), dw_gate [E, D] float32
 * out, dbias [E] float32 out or NULL (then ws may be NULL). logits: the forward's float32 logits;
 * topk_gate: the forward's gates. ws: moe_workspace_size(MOE_STAGE_ROUTER_BWD) bytes.
 * all_expert_offsets / all_row_to_pair: a dropless layout of topk_idx (moe_dispatch_layout with
 * capacity_factor <= 0; for a dropless layer the forward's own) -- then dW_g is summed per expert
 * over the pairs that selected it (k of E columns of dl are nonzero); NULL for both: dense dl^T x
 * (always so under MOE_GATE_SOFTMAX_FULL). Unsupported: top_k > 32. */
int moe_router_backward(const moe_dims* d, const void* x, const float* logits, const int32_t* topk_idx,
                        const float* topk_gate, const float* dgate, const int32_t* all_expert_offsets,
                        const int32_t* all_row_to_pair, float* dl, float* dw_gate, float* dbias, void* ws,
                        size_t ws_bytes, hipStream_t stream);

/* dx [T, D] out = sum over kept slots of dx_perm rows + sum_e dl[t,e] W_g[e] (float32 sums, one
 * rounding). */
int moe_backward_dx(const moe_dims* d, const void* dx_perm, const int32_t* pair_to_row, const int32_t* topk_idx,
                    const float* dl, const void* w_gate, void* dx, hipStream_t stream);

/* Columns of the transposed operands of moe_expert_wgrad: T*top_k + 63*E rounded up to 64. */
int moe_wgrad_ld(const moe_dims* d, int64_t* ld);

/* dst [n_cols, ld] = src [rows, n_cols] transposed, expert e's rows [off_e, off_e+1) going to columns
 * [koff[e], koff[e] + count_e) and zeros up to koff[e+1] = koff[e] + roundup64(count_e);
 * koff [E+1] int32 out. ld >= moe_wgrad_ld(). */
int moe_group_transpose(const moe_dims* d, const void* src, int32_t n_cols, const int32_t* expert_offsets,
                        int32_t* koff, void* dst, int64_t ld, hipStream_t stream);

/* moe_group_transpose of x_perm without x_perm: row r of the source is x[row_to_pair[r] / top_k]
 * (x [T, n_cols]), the permute done by the transpose's loads; the same dst bit for bit. */
int moe_group_transpose_gather(const moe_dims* d, const void* x, int32_t n_cols, const int32_t* expert_offsets,
                               const int32_t* row_to_pair, int32_t* koff, void* dst, int64_t ld,
                               hipStream_t stream);

/* Per expert e: out_e[m, n] = sum over columns [koff[e], koff[e+1]) of a_t[m, col] * b_t[n, col]
 * (a_t [M, ld], b_t [N, ld] bf16, as moe_group_transpose writes them); rows m < split go to
 * out0 [E, split, N], the rest to out1 [E, M - split, N] (float32). dW2 = wgrad(dy_perm^T, h^T,
 * M = D, N = F); [dW1; dW3] = wgrad(da^T, x_perm^T, M = 2F (or F), N = D, split = F).
 * MOE_ERR_UNSUPPORTED when 320 rows of a_t span 4 GiB or more (320*ld*2 bytes: the kernel's loads
 * use 32-bit offsets within a tile). */
int moe_expert_wgrad(const moe_dims* d, const void* a_t, const void* b_t, const int32_t* koff, int32_t M,
                     int32_t N, int64_t ld, float* out0, float* out1, int32_t split, hipStream_t stream);

/* The whole backward in order (the steps above), from one argument block. Buffers as the step entry
 * points take them; `ld` = the row length of the transposed wgrad operands (>= moe_wgrad_ld()).
 * w13t and w2t both NULL: the data-gradient GEMMs read w1, w3, w2 directly (the _w entry points;
 * refresh_weights is ignored). Otherwise refresh_weights != 0 rebuilds w13t / w2t from w1, w3, w2
 * first (after a weight update). For a layer with a capacity factor, dW_g takes the dense form (the
 * forward's layout is not dropless). */
typedef struct moe_backward_args {
  const void* x; const void* w_gate; const void* w1; const void* w3; const void* w2;
  const float* logits; const int32_t* topk_idx; const float* topk_gate;
  const int32_t* expert_offsets; const int32_t* pair_to_row; const int32_t* row_to_pair;
  const void* x_perm; const void* h; const void* pre; const void* y_perm;   /* saved forward tensors;
                                                   x_perm may be NULL: its rows are gathered from x */
  const void* dy;                                                          /* [T, D] upstream gradient */
  void* w13t; void* w2t; int32_t refresh_weights;
  void* dy_perm; float* dgate; void* da; void* dx_perm; float* dl;         /* backward activations */
  void* router_ws; size_t router_ws_bytes;
  int32_t* koff; void* dy_perm_t; void* h_t; void* da_t; void* x_perm_t; int64_t ld;
  void* dx; float* dw_gate; float* dbias; float* dw1; float* dw3; float* dw2;  /* gradients out */
} moe_backward_args;

int moe_layer_backward(const moe_dims* d, const moe_backward_args* a, hipStream_t stream);

/* Static description of a status code. */
const char* moe_status_str(int status);

/* ABI version of this header (major*100 + minor). */
int moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
