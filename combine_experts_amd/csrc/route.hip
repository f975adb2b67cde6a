// Router: logits l[t,e] = x[t]·W_g[e] + bias[e] in float32, top-k selection, gate values.
//
// EP-in-LLMs article, "The Execution Pipeline" step 1: the router scores every local token against
// all E experts, keeps the top k and normalises their gates; the layer equation of "The
// Distributed MoE Dilemma" sums over TopK(G(x), k). Node-limited routing ("Expert Parallelism and
// All-to-All", section on fighting back) restricts a token to its best groups before the
// per-expert choice.
//
// One block = 8 waves = 64 tokens; all E (<= 256) experts of a token stay in one block, so the
// selection needs no second pass over HBM.
//   bf16: matrix cores (v_mfma_f32_16x16x32_bf16) with float32 accumulation. The block streams
//         64-wide K slices of its 64 x rows and of W_g (all experts) into a ring of LDS stages with
//         direct global->LDS loads (16-byte chunks, XOR-swizzled against bank conflicts), several
//         slices in flight; each wave multiplies a 32-token x 64-expert piece of the tile from LDS.
//         Only direct loads are in flight, so every wait is an explicit count.
//   fp32: plain FMA dot products (the small fp32 workload only).
// The [64 x E] float32 logit tile then goes to LDS, and each wave selects for its 8 tokens:
// group scores (if limited), then k rounds of a wave-wide argmax on (value, -index), so exact
// ties go to the lower expert index.
#include <atomic>

#include "moe_common.h"
#include "route_geometry.h"

namespace moe {
namespace {

constexpr int kTokPerBlock = kRouteTokPerBlock;
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * MOE_WAVE;
constexpr int kTokPerWave = kTokPerBlock / kWaves;  // tokens each wave selects for
constexpr int kKC = 64;           // K slice per pipeline stage (two MFMA k-steps of 32)
constexpr int kMaxE = 256;
constexpr int kMaxPerLane = kMaxE / MOE_WAVE;

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// ---- logits, bf16 on matrix cores ---------------------------------------------------------------
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// Workgroup barrier without __syncthreads' release fence, which waits for every load in flight
// (the prefetched slices included). Each wave has already waited for its own loads of the slice it
// needs; the memory clobber keeps the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Stage geometry for NT 16-expert tiles (experts padded to NT*16): one stage holds a 64-wide K slice
// of the block's 64 x rows (512 chunks of 16 bytes) and of all padded W_g rows (128*NT chunks),
// padded to a whole number of chunks per thread so every thread issues the same number of loads.
template <int NT>
struct RouteStage {
  static_assert(rgeom::kTokPerBlock == kTokPerBlock && rgeom::kThreads == kThreads && rgeom::kKC == kKC,
                "router geometry");
  static constexpr int XCH = rgeom::stage_xch();
  static constexpr int CH = rgeom::stage_ch(NT);
  static constexpr int LPT = rgeom::stage_lpt(NT);  // direct loads per thread per stage
  static constexpr int PCH = LPT * kThreads;                   // padded chunks per stage
  static constexpr int DEPTH = NT >= 16 ? 4 : 6;               // ring slots
  static constexpr size_t BYTES = (size_t)DEPTH * PCH * 16;
  // waves: WT token groups x WE expert groups; each wave TT 16-token tiles x TE 16-expert tiles
  static constexpr int WE = NT < 4 ? NT : 4;
  static constexpr int WT = (kWaves / WE) < 4 ? kWaves / WE : 4;
  static constexpr int TT = 4 / WT;
  static constexpr int TE = NT / WE;
};

// Logit tile of the block: the K loop over DEPTH ring slots, DEPTH-1 slices in flight. Every
// iteration issues one slice (past the end, the last slice again into the slot just freed, never
// read), so the number of loads behind slice kc is fixed. Requires D % 64 == 0.
template <int NT>
__device__ __forceinline__ void logits_bf16(const bf16_t* __restrict__ x, const bf16_t* __restrict__ wg,
                                            const float* bias, float* lds_logits, char* lds_raw, int T, int D,
                                            int E, int t0) {
  using S = RouteStage<NT>;
  constexpr int epad = NT * 16;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / MOE_WAVE);
  const int lane = tid % MOE_WAVE;
  bf16x8* ring = reinterpret_cast<bf16x8*>(lds_raw);  // [DEPTH][PCH]

  // source of each of this thread's loads (chunk slot i*kThreads + tid of a stage)
  const bf16_t* src[S::LPT];
#pragma unroll
  for (int i = 0; i < S::LPT; ++i) {
    bool from_x;
    const size_t off = rgeom::load_src(NT, i, tid, t0, T, D, E, &from_x);
    src[i] = (from_x ? x : wg) + off;
  }
  auto issue = [&](int kc, int slot) {
#pragma unroll
    for (int i = 0; i < S::LPT; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(src[i] + kc * kKC),
                                       (__attribute__((address_space(3))) void*)(ring + slot * S::PCH + i * kThreads +
                                                                                 wave * MOE_WAVE),
                                       16, 0, 0);
  };

  // this wave's piece: token tiles [wt*TT, +TT), expert tiles [we*TE, +TE); waves past WT*WE idle
  const bool active = wave < S::WT * S::WE;
  const int wt = wave / S::WE, we = wave % S::WE;
  const int r = lane % 16, q = lane / 16;  // MFMA row / k-quarter of this lane
  int xoff[S::TT][2], woff[S::TE][2];
#pragma unroll
  for (int a = 0; a < S::TT; ++a) {
    const int row = (wt * S::TT + a) * 16 + r;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) xoff[a][s2] = row * (kKC / 8) + swz(row, q * 2 + s2);
  }
#pragma unroll
  for (int b = 0; b < S::TE; ++b) {
    const int row = (we * S::TE + b) * 16 + r;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) woff[b][s2] = S::XCH + row * (kKC / 8) + swz(row, q * 2 + s2);
  }
  f32x4 acc[S::TT][S::TE];
#pragma unroll
  for (int a = 0; a < S::TT; ++a)
#pragma unroll
    for (int b = 0; b < S::TE; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int n_kc = D / kKC;
#pragma unroll
  for (int st = 0; st < S::DEPTH - 1; ++st) issue(min(st, n_kc - 1), st);
  for (int kc0 = 0; kc0 < n_kc; kc0 += S::DEPTH) {
#pragma unroll
    for (int u = 0; u < S::DEPTH; ++u) {
      const int kc = kc0 + u;
      if (kc < n_kc) {
        wait_vmcnt<(S::DEPTH - 2) * S::LPT>();  // this wave's loads of slice kc landed ...
        lds_barrier();  // ... and everyone's; everyone is also done reading slot (kc-1) % DEPTH
        issue(min(kc + S::DEPTH - 1, n_kc - 1), (u + S::DEPTH - 1) % S::DEPTH);
        if (active) {
          // lane (r, q) supplies K elements [q*16, q*16+16) of the slice as two 8-wide fragments;
          // all of the slice's fragments are read first, then the MFMAs run (s2 = 0, then 1, for
          // every output, in slice order)
          const bf16x8* st = ring + u * S::PCH;
          bf16x8 xa[S::TT][2], wb[S::TE][2];
#pragma unroll
          for (int a = 0; a < S::TT; ++a)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) xa[a][s2] = st[xoff[a][s2]];
#pragma unroll
          for (int b = 0; b < S::TE; ++b)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) wb[b][s2] = st[woff[b][s2]];
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int a = 0; a < S::TT; ++a)
#pragma unroll
              for (int b = 0; b < S::TE; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[a][s2], wb[b][s2], acc[a][b], 0, 0, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2 * (S::TT + S::TE), 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2 * S::TT * S::TE, 0);
        }
      }
    }
  }
  wait_vmcnt<0>();  // the redundant tail loads land before the ring memory is reused
  lds_barrier();    // all waves done with the ring before the logit tile reuses the memory
  // acc[a][b][i]: token row (wt*TT + a)*16 + (lane/16)*4 + i, expert (we*TE + b)*16 + lane%16
  if (active) {
#pragma unroll
    for (int b = 0; b < S::TE; ++b) {
      const int e = (we * S::TE + b) * 16 + (lane % 16);
      const float bv = (bias != nullptr && e < E) ? bias[e] : 0.f;
#pragma unroll
      for (int a = 0; a < S::TT; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int trow = (wt * S::TT + a) * 16 + (lane / 16) * 4 + i;
          lds_logits[trow * epad + e] = acc[a][b][i] + bv;
        }
    }
  }
}

// ---- logits, fp32 FMA ------------------------------------------------------------------------------
__device__ __forceinline__ void logits_f32(const float* __restrict__ x, const float* __restrict__ wg, const float* bias,
                           float* lds_logits, int epad, int T, int D, int E, int t0) {
  const int wave = threadIdx.x / MOE_WAVE, lane = threadIdx.x % MOE_WAVE;
  // the wave's (token, expert) pairs spread over all lanes; each dot product in d order
  for (int p = lane; p < kTokPerWave * epad; p += MOE_WAVE) {
    const int i = p / epad, e = p % epad;
    const int trow = wave * kTokPerWave + i;
    const int tok = t0 + trow;
    {
      float s = 0.f;
      if (tok < T && e < E) {
        const float* xr = x + (size_t)tok * D;
        const float* wr = wg + (size_t)e * D;
#pragma unroll 4
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

// (ov, oe) ranks above (v, e): larger value, or the same value and a lower index. Bitwise operators,
// not short-circuit ones, so that the comparison and the selects that use it compile to straight-line
// vector code rather than a branch per element.
__device__ __forceinline__ bool better(float v, int e, float ov, int oe) {
  return (ov > v) | ((ov == v) & (oe < e));
}

// The same register of another lane of this lane's 16-lane row, through DPP (a modifier of a VALU
// move: no LDS round trip, unlike a general shuffle). Applied in the order xor 1, xor 2 (quad
// permutations), mirror within 8 lanes, mirror within 16, each step pairs a lane with one of the
// other half of the group merged so far, whose lanes all hold the same value by then: a butterfly
// over the row for any associative, commutative, exact reduction (max, argmax, merge of top lists).
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& bv, int& be) {
  const float ov = dpp_f<CTRL>(bv);
  const int oe = dpp_i<CTRL>(be);
  const bool t = better(bv, be, ov, oe);
  bv = t ? ov : bv;
  be = t ? oe : be;
}
// (value, -index) maximum over the 16-lane row, in every lane of the row
__device__ __forceinline__ void argmax16(float& bv, int& be) {
  argmax_step<kDppXor1>(bv, be);
  argmax_step<kDppXor2>(bv, be);
  argmax_step<kDppHalfMirror>(bv, be);
  argmax_step<kDppMirror>(bv, be);
}
__device__ __forceinline__ float max16(float m) {
  m = fmaxf(m, dpp_f<kDppXor1>(m));
  m = fmaxf(m, dpp_f<kDppXor2>(m));
  m = fmaxf(m, dpp_f<kDppHalfMirror>(m));
  return fmaxf(m, dpp_f<kDppMirror>(m));
}

__device__ __forceinline__ float sigmoidf_(float v) { return 1.f / (1.f + expf(-v)); }

// ---- selection and gates for one token ------------------------------------------------------------
// Selection score under a selection-only bias: the sigmoid score under sigmoid gating, else the
// logit, plus the expert's bias. Without a bias the selection ranks the logits themselves.
__device__ __forceinline__ float sel_key(float v, float b, int gate) {
  return ((gate == MOE_GATE_SIGMOID_TOPK) ? sigmoidf_(v) : v) + b;
}

// Router probability numerators of one token: exp(l - max) for softmax gates, sigmoid(l) for
// sigmoid gates; the caller divides by their sum over all E experts.
__device__ __forceinline__ float prob_num(float v, float m, int gate) {
  return (gate == MOE_GATE_SIGMOID_TOPK) ? sigmoidf_(v) : expf(v - m);
}

__device__ __forceinline__ void select_token(const float* lrow, int E, int k, int n_groups, int topk_groups, int gate,
                             const float* __restrict__ sbias, float (&pacc)[kMaxPerLane], bool want_p,
                             int32_t* out_idx, float* out_gate) {
  const int lane = lane_id();
  const int n_per = (E + MOE_WAVE - 1) / MOE_WAVE;
  float v[kMaxPerLane], key[kMaxPerLane];
  bool ok[kMaxPerLane];
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + i * MOE_WAVE;
    ok[i] = (i < n_per) && (e < E);
    v[i] = ok[i] ? lrow[e] : -INFINITY;
    key[i] = (ok[i] && sbias != nullptr) ? sel_key(v[i], sbias[e], gate) : v[i];
  }
  if (want_p) {
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) m = fmaxf(m, v[i]);
#pragma unroll
    for (int off = MOE_WAVE / 2; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, MOE_WAVE));
    float num[kMaxPerLane], z = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      num[i] = ok[i] ? prob_num(v[i], m, gate) : 0.f;
      z += num[i];
    }
#pragma unroll
    for (int off = MOE_WAVE / 2; off >= 1; off >>= 1) z += __shfl_xor(z, off, MOE_WAVE);
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) pacc[i] += num[i] / z;
  }
  if (n_groups > 0) {
    const int gsize = E / n_groups;
    const int per = max(1, k / topk_groups);
    float gs = -INFINITY;  // lane g < n_groups ends up with group g's score
    if (gsize <= MOE_WAVE && (gsize & (gsize - 1)) == 0 && E % MOE_WAVE == 0) {
      // expert e = lane + 64*i sits in lane e%64 of register i, so group g is the lane segment
      // [(g*gsize) % 64, +gsize) of register (g*gsize)/64: score it with `per` rounds of a
      // segment-wide max (ties: lowest lane), removing each round's winner.
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i) {
        if (i >= n_per) break;
        float sv = (sbias != nullptr) ? key[i] : ((gate == MOE_GATE_SIGMOID_TOPK) ? sigmoidf_(v[i]) : v[i]);
        float sum = 0.f;
        for (int rnd = 0; rnd < per; ++rnd) {
          float m = sv;
          int ml = lane;
          for (int off = 1; off < gsize; off <<= 1) {
            const float om = __shfl_xor(m, off, MOE_WAVE);
            const int ol = __shfl_xor(ml, off, MOE_WAVE);
            if (om > m || (om == m && ol < ml)) {
              m = om;
              ml = ol;
            }
          }
          sum += m;
          if (lane == ml) sv = -INFINITY;
        }
        // every lane of a segment holds its group's score: hand group g's to lane g
        for (int g = 0; g < n_groups; ++g) {
          const int src = (g * gsize) % MOE_WAVE;
          if ((g * gsize) / MOE_WAVE == i) {
            const float sg = __shfl(sum, src, MOE_WAVE);
            if (lane == g) gs = sg;
          }
        }
      }
    } else if (lane < n_groups) {
      // general group size: lane g walks its group's members, keeping the `per` best
      float best[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) best[j] = -INFINITY;
      for (int m = 0; m < gsize; ++m) {
        const int e = lane * gsize + m;
        const float lv = lrow[e];
        float sv = (sbias != nullptr) ? sel_key(lv, sbias[e], gate)
                                      : ((gate == MOE_GATE_SIGMOID_TOPK) ? sigmoidf_(lv) : lv);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const bool t = (j < per) & (sv > best[j]);
          const float bj = best[j];
          best[j] = t ? sv : bj;
          sv = t ? bj : sv;
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
      rank += ((og > gs) | ((og == gs) & (g < lane))) ? 1 : 0;
    }
    const bool gkeep = (lane < n_groups) & (rank < topk_groups);
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + i * MOE_WAVE;
      const int g = (e < E) ? e / gsize : 0;
      ok[i] = ok[i] & (__shfl((int)gkeep, g, MOE_WAVE) != 0);
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
      const bool t = ok[i] & better(bv, be, key[i], lane + i * MOE_WAVE);
      bv = t ? key[i] : bv;
      be = t ? lane + i * MOE_WAVE : be;
    }
#pragma unroll
    for (int off = MOE_WAVE / 2; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, MOE_WAVE);
      const int oe = __shfl_xor(be, off, MOE_WAVE);
      const bool t = better(bv, be, ov, oe);
      bv = t ? ov : bv;
      be = t ? oe : be;
    }
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) ok[i] = ok[i] & (lane + i * MOE_WAVE != be);
    if (lane == j) {
      my_v = bv;
      my_e = be;
    }
  }
  // gates, from the logits of the chosen experts (a selection bias never enters them)
  if (sbias != nullptr) my_v = lrow[lane < k ? my_e : 0];
  float v0 = __shfl(my_v, 0, MOE_WAVE);
  if (sbias != nullptr)  // slot 0 need not hold the largest chosen logit any more
    for (int j = 1; j < k; ++j) v0 = fmaxf(v0, __shfl(my_v, j, MOE_WAVE));
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

// ---- selection for 4 tokens at once --------------------------------------------------------------
// Each token of a group of four owns a 16-lane segment; lane L of the segment holds the NT experts
// [L*NT, L*NT + NT) (NT*16 = padded E). Used when E == 16*NT, k <= 16, and with a group limit
// when a group is a power-of-two number (<= 16) of whole lanes and there are at most 16 groups.
template <int NT>
__device__ bool fast_select_ok(int E, int k, int n_groups) {
  if (E != NT * 16 || k > 16) return false;
  if (n_groups == 0) return true;
  const int gsize = E / n_groups;
  if (gsize % NT != 0 || n_groups > 16) return false;
  const int lpg = gsize / NT;
  return lpg >= 1 && lpg <= 16 && (lpg & (lpg - 1)) == 0;
}

template <int NT>
__device__ __forceinline__ void select4(const float* lds_logits, int trow0, int ntok, int E, int k, int n_groups, int topk_groups,
                        int gate, bool has_sb, const float (&sb)[NT], float (&pacc)[NT], bool want_p,
                        int32_t* out_idx, float* out_gate) {
  constexpr int epad = NT * 16;
  const int lane = lane_id();
  const int seg = lane / 16, L = lane % 16;
  const bool tok_ok = seg < ntok;
  const float* ltok = lds_logits + (trow0 + (tok_ok ? seg : 0)) * epad;
  const float* lrow = ltok + L * NT;
  float v[NT], key[NT];
  bool ok[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    v[i] = lrow[i];
    key[i] = has_sb ? sel_key(v[i], sb[i], gate) : v[i];
    ok[i] = true;
  }
  if (want_p) {
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < NT; ++i) m = fmaxf(m, v[i]);
    m = max16(m);
    float num[NT], z = 0.f;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      num[i] = prob_num(v[i], m, gate);
      z += num[i];
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) z += __shfl_xor(z, off, MOE_WAVE);
    if (tok_ok) {
#pragma unroll
      for (int i = 0; i < NT; ++i) pacc[i] += num[i] / z;
    }
  }
  if (n_groups > 0) {
    const int gsize = E / n_groups;
    const int lpg = gsize / NT;                   // lanes per group
    const int per = max(1, k / topk_groups);      // members summed per group (<= 8)
    // Group score: the sum of the group's `per` best member scores, in descending order. Members are
    // ranked by the logit itself where the score is its sigmoid (monotonic: the same members, the
    // same order), so only the chosen ones pass through the sigmoid. P bounds `per` at compile time.
    const bool sig_after = !has_sb && gate == MOE_GATE_SIGMOID_TOPK;
    auto group_score = [&](auto pc) -> float {
      constexpr int P = decltype(pc)::value;
      float best[P];  // this lane's `per` best, descending
#pragma unroll
      for (int j = 0; j < P; ++j) best[j] = -INFINITY;
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        float sv = has_sb ? key[i] : v[i];
#pragma unroll
        for (int j = 0; j < P; ++j) {
          const bool t = (P <= 2 || j < per) & (sv > best[j]);
          const float bj = best[j];
          best[j] = t ? sv : bj;
          sv = t ? bj : sv;
        }
      }
      // merge sorted lists across the lanes of the group (lpg lanes: 1, 2, 4, 8 or 16)
      auto merge = [&](auto ctrl) {
        constexpr int C = decltype(ctrl)::value;
        float other[P];
#pragma unroll
        for (int j = 0; j < P; ++j) other[j] = dpp_f<C>(best[j]);
        float merged[P];
        int ia = 0, ib = 0;
#pragma unroll
        for (int j = 0; j < P; ++j) {
          float a = -INFINITY, b = -INFINITY;
#pragma unroll
          for (int q = 0; q < P; ++q) {
            if (q == ia) a = best[q];
            if (q == ib) b = other[q];
          }
          const bool take_a = a >= b;
          merged[j] = take_a ? a : b;
          ia += take_a ? 1 : 0;
          ib += take_a ? 0 : 1;
        }
#pragma unroll
        for (int j = 0; j < P; ++j) best[j] = merged[j];
      };
      if (lpg > 1) merge(std::integral_constant<int, kDppXor1>{});
      if (lpg > 2) merge(std::integral_constant<int, kDppXor2>{});
      if (lpg > 4) merge(std::integral_constant<int, kDppHalfMirror>{});
      if (lpg > 8) merge(std::integral_constant<int, kDppMirror>{});
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < P; ++j)
        if (j < per) sum += sig_after ? sigmoidf_(best[j]) : best[j];
      return sum;
    };
    // group score, in every lane of the group
    const float gs = per == 1   ? group_score(std::integral_constant<int, 1>{})
                     : per == 2 ? group_score(std::integral_constant<int, 2>{})
                                : group_score(std::integral_constant<int, 8>{});
    const int my_g = L / lpg;
    int rank = 0;
#pragma unroll
    for (int g = 0; g < 16; ++g) {  // n_groups <= 16 here; the reads are issued together
      const float og = __shfl(gs, seg * 16 + g * lpg, MOE_WAVE);
      rank += ((g < n_groups) & ((og > gs) | ((og == gs) & (g < my_g)))) ? 1 : 0;
    }
    const bool gkeep = rank < topk_groups;
#pragma unroll
    for (int i = 0; i < NT; ++i) ok[i] = ok[i] & gkeep;
  }
  // k rounds of a segment-wide argmax on (value, -expert); lane j of the segment keeps slot j
  float my_v = 0.f;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const bool t = ok[i] & better(bv, be, key[i], L * NT + i);
      bv = t ? key[i] : bv;
      be = t ? L * NT + i : be;
    }
    argmax16(bv, be);
#pragma unroll
    for (int i = 0; i < NT; ++i) ok[i] = ok[i] & (L * NT + i != be);
    if (L == j) {
      my_v = bv;
      my_e = be;
    }
  }
  if (has_sb) my_v = ltok[L < k ? my_e : 0];  // gates use the chosen experts' logits
  float v0 = __shfl(my_v, seg * 16, MOE_WAVE);
  if (has_sb)
    for (int j = 1; j < k; ++j) v0 = fmaxf(v0, __shfl(my_v, seg * 16 + j, MOE_WAVE));
  float w = 0.f, denom = 0.f;
  if (gate == MOE_GATE_SOFTMAX_FULL) {
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < NT; ++i) m = fmaxf(m, v[i]);
    m = max16(m);
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < NT; ++i) z += expf(v[i] - m);
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) z += __shfl_xor(z, off, MOE_WAVE);
    w = (L < k) ? expf(my_v - m) : 0.f;
    denom = z;
  } else {
    if (L < k) w = (gate == MOE_GATE_SIGMOID_TOPK) ? sigmoidf_(my_v) : expf(my_v - v0);
    // slot order 0 .. k-1 (k <= 16 here); the slots past k add exact zeros
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float wj = __shfl(w, seg * 16 + j, MOE_WAVE);
      denom += (j < k) ? wj : 0.f;
    }
  }
  if (tok_ok && L < k) {
    out_idx[seg * k + L] = my_e;
    out_gate[seg * k + L] = w / denom;
  }
}

// BAL = false is the plain router: the selection bias and the probability sums are compiled out.
template <typename T, int NT, bool BAL>
__global__ void __launch_bounds__(kThreads) route_kernel(const T* __restrict__ x, const T* __restrict__ wg,
                                                    const float* __restrict__ bias, const float* __restrict__ sbias_,
                                                    int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate,
                                                    float* __restrict__ logits, float* __restrict__ prob_partials_,
                                                    int T_, int D, int E, int k, int n_groups, int topk_groups,
                                                    int gate) {
  const float* sbias = BAL ? sbias_ : nullptr;
  float* prob_partials = BAL ? prob_partials_ : nullptr;
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
  const bool want_p = prob_partials != nullptr;
  // per-wave sums of router probabilities, one row of epad floats per wave, after the logit tile
  float* wsum = lds_logits + kTokPerBlock * epad;
  if (fast_select_ok<NT>(E, k, n_groups)) {
    const int L = lane % 16;
    float sb[NT], pacc[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      sb[i] = sbias != nullptr ? sbias[L * NT + i] : 0.f;
      pacc[i] = 0.f;
    }
    for (int i = 0; i < kTokPerWave; i += 4) {
      const int trow = wave * kTokPerWave + i;
      const int tok = t0 + trow;
      if (tok >= T_) break;
      select4<NT>(lds_logits, trow, min(4, T_ - tok), E, k, n_groups, topk_groups, gate, sbias != nullptr, sb, pacc,
                  want_p, topk_idx + (size_t)tok * k, topk_gate + (size_t)tok * k);
    }
    if (want_p) {
      // fold the four token segments: lane L of segment 0 ends with the wave's sums for its experts
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        pacc[i] += __shfl_xor(pacc[i], 16, MOE_WAVE);
        pacc[i] += __shfl_xor(pacc[i], 32, MOE_WAVE);
      }
      if (lane < 16)
#pragma unroll
        for (int i = 0; i < NT; ++i) wsum[wave * epad + L * NT + i] = pacc[i];
    }
  } else {
    float pacc[kMaxPerLane] = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < kTokPerWave; ++i) {
      const int trow = wave * kTokPerWave + i;
      const int tok = t0 + trow;
      if (tok >= T_) break;
      select_token(lds_logits + trow * epad, E, k, n_groups, topk_groups, gate, sbias, pacc, want_p,
                   topk_idx + (size_t)tok * k, topk_gate + (size_t)tok * k);
    }
    if (want_p)
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i)
        if (lane + i * MOE_WAVE < epad) wsum[wave * epad + lane + i * MOE_WAVE] = pacc[i];
  }
  if (want_p) {
    // block partial, waves summed in a fixed order: the result does not depend on scheduling
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
      float sum = wsum[e];
      for (int w = 1; w < kWaves; ++w) sum += wsum[w * epad + e];
      prob_partials[(size_t)blockIdx.x * E + e] = sum;
    }
  }
}

template <int NT, bool BAL>
hipError_t launch_route_nt(const RouteArgs& a, int dtype, hipStream_t s) {
  constexpr int epad = NT * 16;
  const int blocks = (a.T + kTokPerBlock - 1) / kTokPerBlock;
  // logit tile [64 x epad] plus one probability row per wave
  const size_t lds_logits = (size_t)(kTokPerBlock + kWaves) * epad * sizeof(float);
  if (dtype == MOE_BF16) {
    const size_t lds_w = RouteStage<NT>::BYTES;
    const size_t lds = lds_w > lds_logits ? lds_w : lds_logits;
    // dynamic LDS above the default 64 KB needs the per-kernel limit raised, once per device
    static std::atomic<unsigned long long> raised{0};  // one bit per device
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    const unsigned long long bit = 1ull << (dev & 63);
    if (!(raised.load(std::memory_order_acquire) & bit)) {
      const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&route_kernel<bf16_t, NT, BAL>),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (attr != hipSuccess) return attr;
      raised.fetch_or(bit, std::memory_order_release);
    }
    hipLaunchKernelGGL((route_kernel<bf16_t, NT, BAL>), dim3(blocks), dim3(kThreads), lds, s, (const bf16_t*)a.x,
                       (const bf16_t*)a.w_gate, a.bias, a.select_bias, a.topk_idx, a.topk_gate, a.logits,
                       a.prob_partials, a.T, a.D, a.E, a.k, a.n_groups, a.topk_groups, a.gate);
  } else {
    hipLaunchKernelGGL((route_kernel<float, NT, BAL>), dim3(blocks), dim3(kThreads), lds_logits, s, (const float*)a.x,
                       (const float*)a.w_gate, a.bias, a.select_bias, a.topk_idx, a.topk_gate, a.logits,
                       a.prob_partials, a.T, a.D, a.E, a.k, a.n_groups, a.topk_groups, a.gate);
  }
  return hipGetLastError();
}

template <int NT>
hipError_t launch_route_nt(const RouteArgs& a, int dtype, hipStream_t s) {
  if (a.select_bias != nullptr || a.prob_partials != nullptr) return launch_route_nt<NT, true>(a, dtype, s);
  return launch_route_nt<NT, false>(a, dtype, s);
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
