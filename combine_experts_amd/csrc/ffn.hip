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
// The up-projection can also read its rows straight from x (x_perm[r] = x[row_to_pair[r] / k]):
// the permutation then happens in the GEMM's own row loads and x_perm is never written.
// Both operands are contiguous along K (weights are (out, in)), which is what the matrix cores
// want: each lane feeds 8 consecutive K elements (16 bytes) per operand per instruction.
//
// Every block derives its tile from expert_offsets (a block scan of the per-expert tile counts); the
// grid is sized for the worst case (N_max / BM + E row tiles per column tile) and blocks past the
// last tile exit, so the host never reads counts. The bf16 path is described above its kernel;
// the float32 path (small workloads only) is a plain LDS-tiled FMA GEMM on a 2-D grid.
#include "moe_common.h"
#include "gemm_geometry.h"

#include <algorithm>

namespace moe {
namespace {

using namespace geom;

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

__device__ __forceinline__ float act_silu(float a) { return a / (1.f + expf(-a)); }
__device__ __forceinline__ float act_gelu(float a) { return 0.5f * a * (1.f + erff(a * 0.70710678118654752f)); }
// SiLU with the hardware exp2 and reciprocal (relative error a few float32 ulp; the result is rounded to bf16)
__device__ __forceinline__ float act_silu_fast(float a) { return a * __builtin_amdgcn_rcpf(1.f + __expf(-a)); }

// ---------------------------------------------------------------------------------------------------
// bf16 grouped GEMM on matrix cores.
//
// Block: 8 waves (2 per SIMD) own a 320-row x 256-B-row tile; for SwiGLU the 256 B rows are 128
// rows of W1 and the matching 128 rows of W3, so the block produces 320 x 128 of h. Wave (wm, wn)
// holds m-blocks {2i + wm} (32 rows each, interleaved so a ragged tile splits evenly between the
// two wave rows) against 2 B blocks of 32 rows: 10 v_mfma_f32_32x32x16_bf16 per 16-deep k-step,
// accumulators 5 x 2 x 16 floats (244-251 VGPRs, no spills). 320 rows rather than 256: an expert with
// 2*256 + a few rows, common when routing is near even, needs two tiles instead of three, and every
// tile re-streams the expert's weights. The weight fragment is the MFMA's first operand, so each lane
// ends up with 4 consecutive output columns of one token row; the plain epilogue regroups them in LDS
// so that its global stores write 16-byte row pieces (the down-projection 6 % faster than storing
// the 8-byte pieces directly).
//
// K runs in 64-deep stages through a 2-slot LDS ring (72 KB per slot). Loads go straight from
// global memory into LDS (buffer loads with the LDS flag, 16 bytes per lane, no register staging);
// a whole stage is issued at once, one stage ahead, at the start of the stage before it. Inside a slot each 64-element row of a tile is 8 16-byte chunks stored at chunk
// ch ^ ((row >> 1) & 7), so the 32 rows one fragment read touches fall on distinct banks.
//
// Tile order: a block's tile comes from its index through an XCD-aware map (workgroups are handed
// to the 8 XCDs round robin): XCD x takes a contiguous range of the expert-major tile list, so
// the tiles of one expert run together on one XCD and share its L2 (each x_perm row and weight
// row is fetched from HBM about once). Within an expert, tiles go in groups of 4 column tiles,
// row-tile-major inside a group. Rows past the expert's count are loaded from row 0 (finite
// values) and never stored; 32-row blocks entirely past the count are not multiplied.
// ---------------------------------------------------------------------------------------------------
static_assert(kLanes == MOE_WAVE, "the GEMM geometry assumes 64-wide wavefronts");

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

__device__ __forceinline__ int block_scan_g(int v, int* lds, int* total) {
  const int lane = threadIdx.x % MOE_WAVE, wave = threadIdx.x / MOE_WAVE;
  int inc = v;
#pragma unroll
  for (int off = 1; off < MOE_WAVE; off <<= 1) {
    const int u = __shfl_up(inc, off, MOE_WAVE);
    if (lane >= off) inc += u;
  }
  __syncthreads();
  if (lane == MOE_WAVE - 1) lds[wave] = inc;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < GW; ++w) {
    const int x = lds[w];
    if (w < wave) before += x;
    tot += x;
  }
  *total = tot;
  return before + inc - v;
}

// This block's (expert, row tile, column tile), or false when it has none.
__device__ bool map_tile_xcd(const int32_t* __restrict__ offsets, int E, int NT, int blk, int* e_out, int* mt_out,
                             int* nt_out, int* o0_out, int* cnt_out) {
  __shared__ int s_tmp[GW];
  __shared__ int s_e, s_local, s_cnt, s_o0;
  if (E <= GTH) {
    // one scan gives every expert's tile count, its first tile and the total
    const int e = threadIdx.x;
    const int o0 = (e < E) ? offsets[e] : 0;
    const int cnt = (e < E) ? offsets[e + 1] - o0 : 0;
    const int n = ((cnt + GBM - 1) / GBM) * NT;
    int L;
    const int start = block_scan_g(n, s_tmp, &L);
    const int per = (L + 7) / 8;
    const int xcd = blk % 8, j = blk / 8;
    if (j >= per) return false;
    const int t = xcd * per + j;
    if (t >= L) return false;
    if (e < E && t >= start && t < start + n) {
      s_e = e;
      s_local = t - start;
      s_cnt = cnt;
      s_o0 = o0;
    }
    __syncthreads();
    const int ee = s_e;
    const int MT = (s_cnt + GBM - 1) / GBM;
    const int gsz = G_GN * MT;
    const int g = s_local / gsz, r = s_local % gsz;
    const int gn = min(G_GN, NT - g * G_GN);
    *e_out = ee;
    *mt_out = r / gn;
    *nt_out = g * G_GN + r % gn;
    *o0_out = s_o0;
    *cnt_out = s_cnt;
    return true;
  }
  int L = 0;  // total tiles
  for (int base = 0; base < E; base += GTH) {
    const int e = base + threadIdx.x;
    const int cnt = (e < E) ? offsets[e + 1] - offsets[e] : 0;
    int tot;
    block_scan_g(((cnt + GBM - 1) / GBM) * NT, s_tmp, &tot);
    L += tot;
  }
  const int per = (L + 7) / 8;
  const int xcd = blk % 8, j = blk / 8;
  if (j >= per) return false;
  const int t = xcd * per + j;
  if (t >= L) return false;
  if (threadIdx.x == 0) s_e = -1;
  int carry = 0;
  for (int base = 0; base < E; base += GTH) {
    const int e = base + threadIdx.x;
    const int cnt = (e < E) ? offsets[e + 1] - offsets[e] : 0;
    const int n = ((cnt + GBM - 1) / GBM) * NT;
    int tot;
    const int start = carry + block_scan_g(n, s_tmp, &tot);
    if (e < E && t >= start && t < start + n) {
      s_e = e;
      s_local = t - start;
    }
    carry += tot;
    if (carry > t) break;  // uniform across the block
  }
  __syncthreads();
  const int e = s_e;
  const int o0 = offsets[e], cnt = offsets[e + 1] - o0;
  const int MT = (cnt + GBM - 1) / GBM;
  const int gsz = G_GN * MT;
  const int g = s_local / gsz, r = s_local % gsz;
  const int gn = min(G_GN, NT - g * G_GN);
  *e_out = e;
  *mt_out = r / gn;
  *nt_out = g * G_GN + r % gn;
  *o0_out = o0;
  *cnt_out = cnt;
  return true;
}

// B-tile row of the wave's j-th 32-row block
template <bool DUAL>
__device__ __forceinline__ int gbrow(int wn, int j) {
  if constexpr (DUAL) return j == 0 ? wn * 32 : GBR / 2 + wn * 32;
  else return wn * 64 + j * 32;
}


// B stored K-major per expert ([K][N], N contiguous: the weights as the forward keeps them, read by
// the data-gradient GEMMs). A stage's B slice is 64 rows of 256 columns (512 bytes each) in LDS, the
// 16-byte chunk c of row k stored at chunk c ^ 4*(k & 3). Rows k < ksplit come from b0 (per expert
// [ksplit][nout]), the rest from b1 (per expert [K - ksplit][nout]).
struct BtSrc {
  int ksplit, nout;
  int tro[2][2];  // byte offsets of the transposed fragment reads (k half h, block j) in the B region
};

// Where a lane's direct loads read: buffer resources for the A rows and the two B sources (the same
// resource twice for a single B matrix; W1 and W3 for the paired tile; the K-major slices below and
// above ksplit for BT) and one 32-bit byte offset per load; the stage's K offset goes in the scalar
// offset. Buffer loads rather than global ones: the compiler then tracks the fragment reads' LDS
// counter exactly and each MFMA waits only for its own operands (a global load into LDS makes it
// wait for every LDS read in flight).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
struct DmaSrc {
  rsrc_t a, b0, b1;
  uint32_t off[G_LPS];
};

// raw buffer resource over 4 GiB from base (no stride, no range clamp; word 3 is the gfx9 default)
__device__ __forceinline__ rsrc_t dma_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
}

__device__ __forceinline__ void dma16(rsrc_t r, uint32_t voff, uint32_t soff, bf16x8* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_dst, 16, voff, soff, 0, 0);
}

// ds_read_b64_tr_b16: within each 16-lane group, output lane i gets element e from the group's lane
// 4e + i/4, its element i % 4 (measured on the hardware). With lane 4e + q of the group reading row
// k0 + e, columns c0 + 4q .. + 3, lane i receives rows k0 .. k0 + 3 of column c0 + i.
__device__ __forceinline__ bf16x4 tr_read(const char* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<char*>(p)));
  return __builtin_bit_cast(bf16x4, v);
}

// LDS index (16-byte chunks) of a wave's fragment reads at k-step ks: A block i (rows (2i+wm)*32 + l)
// at lane[ks] + a + i*64*GKCH, B block j (rows gbrow(wn,j) + l) at lane[ks] + b[j], l = lane % 32. The
// blocks start at multiples of 32 rows, so the swizzle term depends on the lane alone.
struct FragIdx {
  int lane[G_KS];
  int a, b[2];
};

template <bool DUAL>
__device__ __forceinline__ FragIdx frag_idx(int lane, int wm, int wn) {
  FragIdx f;
  const int l = lane % 32;
#pragma unroll
  for (int ks = 0; ks < G_KS; ++ks) f.lane[ks] = l * GKCH + gswz(l, ks * 2 + lane / 32);
  f.a = wm * 32 * GKCH;
#pragma unroll
  for (int j = 0; j < 2; ++j) f.b[j] = G_ACH + gbrow<DUAL>(wn, j) * GKCH;
  return f;
}

// ACT: active 32-row blocks of this wave; BT: B stored K-major; EARLY: see `stage` below
template <int ACT, bool BT, bool EARLY = false>
__device__ __forceinline__ void gemm_kloop(f32x16 (&acc)[GMB][2], bf16x8* lds0, bf16x8* lds1, const DmaSrc& ds,
                                           const FragIdx& fi, const BtSrc& bt, int wave, int nk, int mrows) {
  // load i fills tile rows [i*64, i*64+64) of A (i < G_NAL) or a part of B (the first half of the B
  // loads from b0, the rest from b1); A loads wholly past the tile's rows are skipped (those rows
  // feed only accumulators that are never stored)
  auto issue = [&](int kt, bf16x8* slot, int i) {
    if (i < G_NAL && a_load_skipped(i, mrows)) return;
    bf16x8* dst = slot + i * GTH + wave * MOE_WAVE;
    if (i < G_NAL) {
      dma16(ds.a, ds.off[i], stage_soff(kt), dst);
    } else if constexpr (BT) {
      const int k0 = kt * GBK;
      const bool lo = k0 < bt.ksplit;
      dma16(lo ? ds.b0 : ds.b1, ds.off[i], (uint32_t)(lo ? k0 : k0 - bt.ksplit) * (uint32_t)bt.nout * 2u, dst);
    } else {
      dma16(b_load_second(i) ? ds.b1 : ds.b0, ds.off[i], stage_soff(kt), dst);
    }
  };
  bf16x8 fa[2][GMB], fb[2][2];
  auto frag = [&](const bf16x8* slot, int ks, int r) {
    const bf16x8* s = slot + fi.lane[ks];
    if constexpr (!BT) {
      // in the order the next k-step's MFMAs take them (B0 A0, B1, then A1 ...), so that each MFMA
      // waits only for its own two fragments
      fb[r][0] = s[fi.b[0]];
      fa[r][0] = s[fi.a];
      fb[r][1] = s[fi.b[1]];
#pragma unroll
      for (int i = 1; i < ACT; ++i) fa[r][i] = s[fi.a + i * 2 * 32 * GKCH];
      return;
    }
#pragma unroll
    for (int i = 0; i < ACT; ++i) fa[r][i] = s[fi.a + i * 2 * 32 * GKCH];
    if constexpr (BT) {
      // two transposed 8-byte reads per fragment: 4 consecutive k of this lane's column each
      const char* sb = reinterpret_cast<const char*>(slot + G_ACH) + ks * 16 * GBR * 2;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16x4 lo = tr_read(sb + bt.tro[0][j]), hi = tr_read(sb + bt.tro[1][j]);
        fb[r][j] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    }
  };
  // the first stage's weight slices go first: their addresses need no row lookup, so their latency
  // overlaps that of the gathered row indices the A loads wait for
#pragma unroll
  for (int i = G_NAL; i < G_LPS; ++i) issue(0, lds0, i);
#pragma unroll
  for (int i = 0; i < G_NAL; ++i) issue(0, lds0, i);
  wait_vmcnt<0>();
  __syncthreads();
  frag(lds0, 0, 0);
  // the two ring slots are two LDS arrays and the loop body is written out once per slot, so every
  // load and fragment read names its slot: the compiler then knows that a stage's reads (slot cur)
  // and the next stage's loads (slot nxt) do not overlap
  // With EARLY, the first stage of each pair of the loop below (first = true) also issues stage kt+2
  // into its own slot right after the barrier that ends its reads, before its last k-step, and the
  // second stage then issues nothing at its start: those loads get four k-steps to land instead of
  // three. Only the first stage of a pair does it, so that no load is in flight at the loop's head.
  auto stage = [&](int kt, bf16x8* cur, bf16x8* nxt, bool first) {
    const bool refill = kt + 1 < nk;
    const bool issued = EARLY && !first;  // stage kt+1 went out in the previous stage
#pragma unroll
    for (int ks = 0; ks < G_KS; ++ks) {
      const int c = ks & 1, n = c ^ 1;
      // all of stage kt+1 goes to the other slot at once (free since the barrier that ended iteration
      // kt-1), at the start of stage kt: the loads get a whole stage to land
      if (refill && !issued && ks == 0) {
#pragma unroll
        for (int i = 0; i < G_LPS; ++i) issue(kt + 1, nxt, i);
      }
      if (ks < G_KS - 1) {
        frag(cur, ks + 1, n);
      } else {
        // also after the last stage, so that no path through the loop leaves a load in flight at
        // its head (the compiler would otherwise wait for loads before the first stage's reads)
        wait_vmcnt<0>();  // this wave's part of stage kt+1 has landed ...
        __syncthreads();  // ... and everyone's; everyone is also done reading slot cur
        if (refill) frag(nxt, 0, n);
        if (EARLY && first && kt + 2 < nk) {
#pragma unroll
          for (int i = 0; i < G_LPS; ++i) issue(kt + 2, cur, i);
        }
      }
#pragma unroll
      for (int i = 0; i < ACT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[c][j], fa[c][i], acc[i][j], 0, 0, 0);
      // issue order: each fragment read for the next k-step goes right after one MFMA of this one,
      // rather than all reads in a batch behind a wait (measured 2-4 % faster, same results)
      {
        constexpr int NR = (BT ? 4 : 2) + ACT, NM = 2 * ACT, NP = NR < NM ? NR : NM;
#pragma unroll
        for (int q = 0; q < NP; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        }
        if constexpr (NM > NP) __builtin_amdgcn_sched_group_barrier(0x008, NM - NP, 0);
      }
    }
  };
  for (int kt = 0; kt < nk; kt += 2) {
    stage(kt, lds0, lds1, true);
    if (kt + 1 < nk) stage(kt + 1, lds1, lds0, false);
  }
}

__device__ __forceinline__ float act_silu_grad(float a) {
  const float s = 1.f / (1.f + expf(-a));
  return s * (1.f + a * (1.f - s));
}
__device__ __forceinline__ float act_gelu_grad(float a) {
  return 0.5f * (1.f + erff(a * 0.70710678118654752f)) + a * expf(-0.5f * a * a) * 0.39894228040143268f;
}

// Epilogue modes of the bf16 grouped GEMM.
//   EPI_PLAIN  out[r, n] = act(acc)                                     (row stride Nout)
//   EPI_PRE    as EPI_PLAIN, and the pre-activations go to pre: SwiGLU writes W1 x to columns [0, Nout)
//              and W3 x to [Nout, 2 Nout) of a 2*Nout-wide row; GELU writes W1 x (Nout wide)
//   EPI_BWD    acc = dh (no activation on the way in); with a1 (and a3) read from pre as EPI_PRE wrote
//              them: SwiGLU out[r, n] = dh*a3*SiLU'(a1), out[r, Nout + n] = dh*SiLU(a1) (2*Nout wide);
//              GELU out[r, n] = dh*GELU'(a1) (Nout wide)
//   EPI_PARTIAL  split K: block (tile, s) sums K stages [s*nk/S, (s+1)*nk/S) and stores the float32 partial
//              to part[s][row][n] ([S][n_rows_max][Nout]); splitk_reduce_bf16 adds the S partials in
//              order s = 0 .. S-1 and rounds once
constexpr int EPI_PLAIN = 0, EPI_PRE = 1, EPI_BWD = 2, EPI_PARTIAL = 3;

template <int ACTFN, bool DUAL, int EPI = EPI_PLAIN, bool BT = false, bool EARLY = false>
__global__ void __launch_bounds__(GTH) ffn_gemm_bf16(const bf16_t* __restrict__ A, const int32_t* __restrict__ offsets,
                                                     const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1,
                                                     bf16_t* __restrict__ out, int E, int K, int Nout,
                                                     bf16_t* __restrict__ pre, const int32_t* __restrict__ gather,
                                                     int gdiv, int ksplit, int splits, float* __restrict__ part,
                                                     int n_rows_max) {
  static_assert(!(BT && DUAL), "the K-major B form has no paired W1/W3 tile");
  static_assert(EPI != EPI_PARTIAL || (!BT && !DUAL && ACTFN < 0), "split K: plain down-projection tile only");
  constexpr int BNO = DUAL ? GBR / 2 : GBR;  // output columns per tile
  __shared__ bf16x8 lds0[G_STAGE], lds1[G_STAGE];  // the two slots of the K ring
  const int NT = (Nout + BNO - 1) / BNO;
  // split K: the S blocks of a tile are adjacent; block (tile, s) takes stages [s*nk/S, (s+1)*nk/S)
  const int split = EPI == EPI_PARTIAL ? (int)(blockIdx.x % splits) : 0;
  const int blk = EPI == EPI_PARTIAL ? (int)(blockIdx.x / splits) : (int)blockIdx.x;
  const int kt0 = EPI == EPI_PARTIAL ? split * (K / GBK) / splits : 0;
  const int kt1 = EPI == EPI_PARTIAL ? (split + 1) * (K / GBK) / splits : K / GBK;
  int e, mt, nt, o0, cnt;
  if (!map_tile_xcd(offsets, E, NT, blk, &e, &mt, &nt, &o0, &cnt)) return;
  const int row0 = o0 + mt * GBM;
  const int mrows = min(GBM, cnt - mt * GBM);
  const int n0 = nt * BNO;
  const int lane = threadIdx.x % MOE_WAVE;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / MOE_WAVE);
  const int wm = wave / 4, wn = wave % 4;
  // this lane's direct loads: load i fills LDS slots [i*GTH + wave*64, +64). A rows come from the
  // row tile's base, or from x itself (gathered rows: byte offsets from x, which the host keeps under
  // 4 GiB); the weights from the tile's first weight row
  DmaSrc ds;
  const int k0 = kt0 * GBK;  // first K column of this block's stages (split K), else 0
  ds.a = dma_rsrc((gather ? A : A + (size_t)row0 * K) + k0);
#pragma unroll
  for (int i = 0; i < G_NAL; ++i) {
    int row, ch;
    a_load_pos(i, wave, lane, &row, &ch);
    const int r = row < mrows ? row : 0;
    const uint32_t arow = gather ? (uint32_t)(gather[row0 + r] / gdiv) : (uint32_t)r;
    ds.off[i] = a_load_off(arow, K, ch);
  }
  const FragIdx fi = frag_idx<DUAL>(lane, wm, wn);
  BtSrc bt{};
  if constexpr (!BT) {
    ds.b0 = dma_rsrc(B0 + ((size_t)e * Nout + n0) * K + k0);
    ds.b1 = DUAL ? dma_rsrc(B1 + ((size_t)e * Nout + n0) * K + k0) : ds.b0;
#pragma unroll
    for (int i = G_NAL; i < G_LPS; ++i) {
      int row, ch;
      b_load_pos(i, wave, lane, &row, &ch);
      // the paired tile's second half (W3 rows) sits in the second half of the B loads; rows past
      // Nout re-read the slice's first row (never stored)
      ds.off[i] = b_load_off(b_weight_row(row, DUAL), n0, Nout, K, ch);
    }
  } else {
    ds.b0 = dma_rsrc(B0 + (size_t)e * ksplit * Nout + n0);
    ds.b1 = B1 ? dma_rsrc(B1 + (size_t)e * (K - ksplit) * Nout + n0) : ds.b0;
    bt.ksplit = ksplit;
    bt.nout = Nout;
#pragma unroll
    for (int i = G_NAL; i < G_LPS; ++i) {
      int k, c;
      bt_load_pos(i, wave, lane, &k, &c);     // chunk of the B region this lane fills
      ds.off[i] = bt_load_off(k, c, n0, Nout);  // columns past Nout: never stored
    }
    const int g = lane / 16, e4 = (lane % 16) / 4, q = lane % 4;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = (g / 2) * 8 + 4 * h + e4;  // row & 3 == e4
        const int c = (gbrow<false>(wn, j) / 8 + (g % 2) * 2 + q / 2) ^ (e4 << 2);
        bt.tro[h][j] = row * GBR * 2 + c * 16 + (q % 2) * 8;
      }
  }
  const int nblk = (mrows + 31) / 32;
  const int act = __builtin_amdgcn_readfirstlane((nblk - wm + 1) / 2);  // blocks 2i+wm < nblk
  f32x16 acc[GMB][2];
#pragma unroll
  for (int i = 0; i < GMB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  const int nk = kt1 - kt0;
  // every wave runs the same stages and barriers; a wave with no rows multiplies one block
  switch (act) {
    case 5: gemm_kloop<5, BT, EARLY>(acc, lds0, lds1, ds, fi, bt, wave, nk, mrows); break;
    case 4: gemm_kloop<4, BT, EARLY>(acc, lds0, lds1, ds, fi, bt, wave, nk, mrows); break;
    case 3: gemm_kloop<3, BT, EARLY>(acc, lds0, lds1, ds, fi, bt, wave, nk, mrows); break;
    case 2: gemm_kloop<2, BT, EARLY>(acc, lds0, lds1, ds, fi, bt, wave, nk, mrows); break;
    default: gemm_kloop<1, BT, EARLY>(acc, lds0, lds1, ds, fi, bt, wave, nk, mrows); break;
  }
  // acc[i][j][v]: token row (2i+wm)*32 + lane%32, B row gbrow(wn,j) + 8*(v/4) + 4*(lane/32) + v%4
  constexpr bool SWI = ACTFN == MOE_ACT_SWIGLU;
  if constexpr (EPI == EPI_PARTIAL) {
    // float32 tile out through LDS, as the weight-gradient tiles: each wave stages its 32-row blocks
    // (32 x 64 floats) in the ring slot the last stage did not read and stores 256-byte row pieces
    constexpr int SROW = 64 + 4;
    float* stg = reinterpret_cast<float*>((nk & 1) ? lds1 : lds0) + wave * 32 * SROW;
    float* pbase = part + (size_t)split * n_rows_max * Nout;
#pragma unroll
    for (int i = 0; i < GMB; ++i) {
      if (i >= act) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<f32x4*>(stg + (lane % 32) * SROW + j * 32 + 8 * q + 4 * (lane / 32)) =
              f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
#pragma unroll
      for (int rr = 0; rr < 32; rr += MOE_WAVE / 16) {
        const int r2 = rr + lane / 16, c2 = (lane % 16) * 4;
        const f32x4 v = *reinterpret_cast<const f32x4*>(stg + r2 * SROW + c2);
        const int r = (2 * i + wm) * 32 + r2, c = n0 + wn * 64 + c2;
        if (r < mrows && c < Nout) *reinterpret_cast<f32x4*>(pbase + (size_t)(row0 + r) * Nout + c) = v;
      }
    }
    return;
  }
  if constexpr (EPI == EPI_PLAIN) {
    // through LDS: each wave stages its 32-row blocks in the ring slot the last stage did not read
    // (every wave passed the barrier after its last read of it) and stores whole 16-byte row pieces,
    // WC/8 lanes per row, instead of 8-byte pieces of 32 rows per instruction
    constexpr int WC = DUAL ? 32 : 64;  // output columns per wave
    constexpr int SROW = WC + 8;        // staging row stride (elements; rows stay 16-byte aligned)
    bf16_t* stg = reinterpret_cast<bf16_t*>((nk & 1) ? lds1 : lds0) + wave * 32 * SROW;
    const int cw = DUAL ? wn * 32 : wn * 64;
#pragma unroll
    for (int i = 0; i < GMB; ++i) {
      if (i >= act) continue;
      const int rl = lane % 32;
#pragma unroll
      for (int j = 0; j < (DUAL ? 1 : 2); ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int cl = j * 32 + 8 * q + 4 * (lane / 32);
          bf16x4 pk;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            float h = acc[i][j][4 * q + u];
            if constexpr (SWI && DUAL) h = act_silu_fast(h) * acc[i][1][4 * q + u];
            else if constexpr (ACTFN == MOE_ACT_GELU) h = act_gelu(h);
            pk[u] = f2bf(h);
          }
          *reinterpret_cast<bf16x4*>(stg + rl * SROW + cl) = pk;
        }
      constexpr int LPR = WC / 8, RPI = MOE_WAVE / LPR;
#pragma unroll
      for (int rr = 0; rr < 32; rr += RPI) {
        const int r2 = rr + lane / LPR, c2 = (lane % LPR) * 8;
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(stg + r2 * SROW + c2);
        const int r = (2 * i + wm) * 32 + r2, c = cw + c2;
        if (r < mrows && n0 + c < Nout) *reinterpret_cast<bf16x8*>(out + (size_t)(row0 + r) * Nout + n0 + c) = v;
      }
    }
    return;
  }
  const int ldo = (EPI == EPI_BWD && SWI) ? 2 * Nout : Nout;   // out row stride
  const int ldp = SWI ? 2 * Nout : Nout;                         // pre row stride
  // Through LDS as the plain epilogue, with the float32 accumulators staged (the activation and its
  // derivative need them unrounded): each wave puts its 32-row blocks (64 columns: 32 of W1 x then 32
  // of W3 x for the paired tile) in the ring slot the last stage did not read, then each lane takes
  // 8 consecutive output columns of a row, so every global access is a 16-byte row piece.
  constexpr int SROWF = 64 + 4;                  // staging row stride (floats; rows stay 16-byte aligned)
  constexpr int OCW = DUAL ? 32 : 64;            // output columns per wave
  constexpr int LPR = OCW / 8, RPI = MOE_WAVE / LPR;
  float* stg = reinterpret_cast<float*>((nk & 1) ? lds1 : lds0) + wave * 32 * SROWF;
  const int cw = DUAL ? wn * 32 : wn * 64;
#pragma unroll
  for (int i = 0; i < GMB; ++i) {
    if (i >= act) continue;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4*>(stg + (lane % 32) * SROWF + jb * 32 + 8 * q + 4 * (lane / 32)) =
            f32x4{acc[i][jb][4 * q], acc[i][jb][4 * q + 1], acc[i][jb][4 * q + 2], acc[i][jb][4 * q + 3]};
#pragma unroll
    for (int rr = 0; rr < 32; rr += RPI) {
      const int r2 = rr + lane / LPR, c2 = (lane % LPR) * 8;
      const int r = (2 * i + wm) * 32 + r2, c = n0 + cw + c2;
      if (r >= mrows || c >= Nout) continue;
      const float* sr = stg + r2 * SROWF + c2;
      float v1[8], v3[8];  // W1 x (or dh) and, for the paired tile, W3 x of the 8 columns
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        v1[u] = sr[u];
        if constexpr (DUAL) v3[u] = sr[32 + u];
      }
      bf16_t* orow = out + (size_t)(row0 + r) * ldo;
      bf16_t* prow = pre + (size_t)(row0 + r) * ldp;
      if constexpr (EPI == EPI_BWD) {
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(prow + c);
        bf16x8 o1, o3;
        if constexpr (SWI) {
          const bf16x8 a3 = *reinterpret_cast<const bf16x8*>(prow + Nout + c);
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const float x1 = bf2f(a1[u]), x3 = bf2f(a3[u]);
            o1[u] = f2bf(v1[u] * x3 * act_silu_grad(x1));
            o3[u] = f2bf(v1[u] * act_silu(x1));
          }
          *reinterpret_cast<bf16x8*>(orow + Nout + c) = o3;
        } else {
#pragma unroll
          for (int u = 0; u < 8; ++u) o1[u] = f2bf(v1[u] * act_gelu_grad(bf2f(a1[u])));
        }
        *reinterpret_cast<bf16x8*>(orow + c) = o1;
      } else {  // EPI_PRE
        bf16x8 o, p1, p3;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          float h = v1[u];
          p1[u] = f2bf(h);
          if constexpr (SWI && DUAL) {
            p3[u] = f2bf(v3[u]);
            h = act_silu_fast(h) * v3[u];
          } else if constexpr (ACTFN == MOE_ACT_GELU) {
            h = act_gelu(h);
          }
          o[u] = f2bf(h);
        }
        *reinterpret_cast<bf16x8*>(orow + c) = o;
        *reinterpret_cast<bf16x8*>(prow + c) = p1;
        if constexpr (SWI && DUAL) *reinterpret_cast<bf16x8*>(prow + Nout + c) = p3;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------------
// Weight gradients: out_g = A_g^T-free form out_g[m, n] = sum_{k in group g} aT[m, k] * bT[n, k], with
// both operands stored transposed ([M, ld] and [N, ld], the reduction index contiguous) and group g
// owning columns [koff[g], koff[g+1]) of both, zero-padded to a multiple of 64. The k-loop is the
// forward's; tiles are 320 x 256 of (m, n); float32 output, rows m < split to out0[g] ([split, N])
// and the rest to out1[g] ([M - split, N]).
// ---------------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(GTH) ffn_wgrad_bf16(const bf16_t* __restrict__ aT, const bf16_t* __restrict__ bT,
                                                      const int32_t* __restrict__ koff, int G, int M, int N,
                                                      long long ld, float* __restrict__ out0,
                                                      float* __restrict__ out1, int split) {
  __shared__ bf16x8 lds0[G_STAGE], lds1[G_STAGE];  // the two slots of the K ring
  const int MT = (M + GBM - 1) / GBM, NT = (N + GBR - 1) / GBR;
  const int per_g = MT * NT;
  const int t = blockIdx.x;
  if (t >= G * per_g) return;
  const int g = t / per_g, rem = t % per_g;
  const int mt = rem / NT, nt = rem % NT;
  const int m0 = mt * GBM, n0 = nt * GBR;
  const int mrows = min(GBM, M - m0);
  const int k0 = koff[g], nk = (koff[g + 1] - k0) / GBK;
  const int lane = threadIdx.x % MOE_WAVE;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / MOE_WAVE);
  const int wm = wave / 4, wn = wave % 4;
  // direct loads from the tile's first operand rows at the group's first reduction column
  DmaSrc ds;
  ds.a = dma_rsrc(aT + (size_t)m0 * ld + k0);
  ds.b0 = dma_rsrc(bT + (size_t)n0 * ld + k0);
  ds.b1 = ds.b0;
#pragma unroll
  for (int i = 0; i < G_LPS; ++i) {
    int row, ch;
    if (i < G_NAL) {
      a_load_pos(i, wave, lane, &row, &ch);
      ds.off[i] = (uint32_t)((row < mrows ? row : 0) * ld) * 2u + ch * 16;
    } else {
      b_load_pos(i, wave, lane, &row, &ch);
      ds.off[i] = (uint32_t)((n0 + row < N ? row : 0) * ld) * 2u + ch * 16;
    }
  }
  const FragIdx fi = frag_idx<false>(lane, wm, wn);
  f32x16 acc[GMB][2];
#pragma unroll
  for (int i = 0; i < GMB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  if (nk > 0) gemm_kloop<GMB, false>(acc, lds0, lds1, ds, fi, BtSrc{}, wave, nk, mrows);  // uniform: an empty group writes zeros
  // the tile goes out through LDS: each wave stages its 32-row blocks (32 x 64 floats) in the ring slot
  // the last stage did not read and stores 256-byte row pieces, 16 lanes per row, instead of 16-byte
  // pieces of 32 rows per instruction
  constexpr int SROW = 64 + 4;  // staging row stride (floats; rows stay 16-byte aligned)
  float* stg = reinterpret_cast<float*>((nk & 1) ? lds1 : lds0) + wave * 32 * SROW;
#pragma unroll
  for (int i = 0; i < GMB; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4*>(stg + (lane % 32) * SROW + j * 32 + 8 * q + 4 * (lane / 32)) =
            f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
#pragma unroll
    for (int rr = 0; rr < 32; rr += MOE_WAVE / 16) {
      const int r2 = rr + lane / 16, c2 = (lane % 16) * 4;
      const f32x4 v = *reinterpret_cast<const f32x4*>(stg + r2 * SROW + c2);
      const int m = m0 + (2 * i + wm) * 32 + r2, c = n0 + wn * 64 + c2;
      if (m >= M || c >= N) continue;
      float* orow = m < split ? out0 + ((size_t)g * split + m) * N : out1 + ((size_t)g * (M - split) + (m - split)) * N;
      __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(orow + c));  // streamed: keeps L2 for the operands
    }
  }
}

// Split-K reduction: out[r, n] = bf16(part[0][r][n] + part[1][r][n] + ... + part[S-1][r][n]), the partials
// added in that order in float32, for the N = offsets[E] kept rows; 4 columns per thread.
__global__ void __launch_bounds__(256) splitk_reduce_bf16(const float* __restrict__ part, int splits,
                                                          const int32_t* __restrict__ offsets, int E,
                                                          int n_rows_max, int Nout, bf16_t* __restrict__ out) {
  const int N = offsets[E];
  const size_t n4 = (size_t)N * Nout / 4, plane = (size_t)n_rows_max * Nout;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x) {
    f32x4 v = *reinterpret_cast<const f32x4*>(part + i * 4);
    for (int s = 1; s < splits; ++s) v += *reinterpret_cast<const f32x4*>(part + s * plane + i * 4);
    bf16x4 o;
#pragma unroll
    for (int u = 0; u < 4; ++u) o[u] = f2bf(v[u]);
    __builtin_nontemporal_store(o, reinterpret_cast<bf16x4*>(out) + i);
  }
}

// ---------------------------------------------------------------------------------------------------
// float32 grouped GEMM (plain FMA): 64 x 64 tiles, BK = 16, each thread 4 x 4 outputs per B matrix.
// ---------------------------------------------------------------------------------------------------
constexpr int FBM = 64, FBN = 64, FBK = 16;

template <int ACT, bool DUAL>
__global__ void __launch_bounds__(256) ffn_gemm_f32(const float* __restrict__ A, const int32_t* __restrict__ offsets,
                                                    const float* __restrict__ B0, const float* __restrict__ B1,
                                                    float* __restrict__ out, int E, int K, int Nout,
                                                    const int32_t* __restrict__ gather, int gdiv) {
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
  // 64 rows x 16 k = 1024 values per stage: 4 per thread, the same 4 rows at every stage
  const float* arow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (tid + i * 256) / FBK;
    const int r = row0 + (row < mrows ? row : 0);
    arow[i] = A + (size_t)(gather ? gather[r] / gdiv : r) * K;
  }
  for (int k0 = 0; k0 < K; k0 += FBK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * 256, row = c / FBK, kk = c % FBK;
      As[kk][row] = (row < mrows) ? arow[i][k0 + kk] : 0.f;
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

// The plain GEMM (no activation: the down-projection, the data gradient through W1|W3) loads each ring
// stage one k-step earlier in every other stage when its reduction is this long: measured 2.6 % faster
// on the Mixtral-shaped down-projection (K = 14336) and slower or neutral at K <= 4096 (the Switch-,
// dsv3- and skew-shaped ones). The results are the same bits either way.
constexpr int kEarlyRefillK = 8192;

hipError_t launch_ffn_bf16(const FfnArgs& a, hipStream_t s) {
  if (a.n_rows_max == 0) return hipSuccess;
  // the direct loads address an operand by 32-bit byte offsets from a row tile's base, an expert's
  // K-major weight slice, or (rows gathered) the start of x: each of those spans must stay under 4 GiB
  const unsigned long long lim = 1ull << 32, K = a.K, NO = a.Nout;
  if (GBM * K * 2 >= lim || (a.bt && K * NO * 2 >= lim) ||
      (a.gather && (unsigned long long)(a.n_rows_max + a.gather_div - 1) / a.gather_div * K * 2 >= lim))
    return hipErrorNotSupported;
  // the up-projection tile pairs W1 and W3 rows (SwiGLU forward); every other form is a plain tile
  const bool dual = a.act == MOE_ACT_SWIGLU && a.epi != 2 && !a.bt;
  const int bno = dual ? GBR / 2 : GBR;
  const long long row_tiles = (a.n_rows_max + GBM - 1) / GBM + (a.E < a.n_rows_max ? a.E : a.n_rows_max);
  const dim3 grid((unsigned)(row_tiles * ((a.Nout + bno - 1) / bno) + 8));
  const bf16_t* A = (const bf16_t*)a.a;
  const bf16_t* b0 = (const bf16_t*)a.b0;
  const bf16_t* b1 = (const bf16_t*)a.b1;
  bf16_t* o = (bf16_t*)a.out;
  bf16_t* pr = (bf16_t*)a.pre;
#define MOE_FFN_LAUNCH(ACTV, DUALV, EPIV)                                                                          \
  hipLaunchKernelGGL((ffn_gemm_bf16<ACTV, DUALV, EPIV>), grid, dim3(GTH), 0, s, A, a.expert_offsets, b0, b1, o, a.E, \
                     a.K, a.Nout, pr, a.gather, a.gather_div, 0, 1, nullptr, a.n_rows_max)
#define MOE_FFN_LAUNCH_BT(ACTV, EPIV)                                                                              \
  hipLaunchKernelGGL((ffn_gemm_bf16<ACTV, false, EPIV, true>), grid, dim3(GTH), 0, s, A, a.expert_offsets, b0, b1, o, \
                     a.E, a.K, a.Nout, pr, a.gather, a.gather_div, a.ksplit > 0 ? a.ksplit : a.K, 1, nullptr,      \
                     a.n_rows_max)
  if (a.splits > 1) {
    // split K (plain down-projection only): S blocks per tile write float32 partials, then one pass adds
    // them in split order and rounds
    if (a.act >= 0 || a.epi != 0 || a.bt || a.gather || a.part == nullptr || a.K % GBK != 0 ||
        a.splits > a.K / GBK || a.Nout % 4 != 0)
      return hipErrorInvalidValue;
    const dim3 sgrid((unsigned)(grid.x * (unsigned)a.splits));
    hipLaunchKernelGGL((ffn_gemm_bf16<-1, false, EPI_PARTIAL>), sgrid, dim3(GTH), 0, s, A, a.expert_offsets, b0, b1,
                       o, a.E, a.K, a.Nout, pr, a.gather, a.gather_div, 0, a.splits, a.part, a.n_rows_max);
    const long long n4 = (long long)a.n_rows_max * a.Nout / 4;
    const unsigned rgrid = (unsigned)std::min<long long>((n4 + 255) / 256, 4096);
    hipLaunchKernelGGL(splitk_reduce_bf16, dim3(rgrid), dim3(256), 0, s, a.part, a.splits, a.expert_offsets, a.E,
                       a.n_rows_max, a.Nout, o);
    return hipGetLastError();
  }
  if (a.bt) {
    if (a.K % GBK != 0 || (a.ksplit > 0 && (a.ksplit % GBK != 0 || a.ksplit > a.K || (a.ksplit < a.K && !b1))))
      return hipErrorInvalidValue;
    if (a.epi == 2 && a.act == MOE_ACT_SWIGLU) MOE_FFN_LAUNCH_BT(MOE_ACT_SWIGLU, EPI_BWD);
    else if (a.epi == 2) MOE_FFN_LAUNCH_BT(MOE_ACT_GELU, EPI_BWD);
    else if (a.epi == 0 && a.act < 0) MOE_FFN_LAUNCH_BT(-1, EPI_PLAIN);
    else return hipErrorInvalidValue;
  } else if (a.epi == 1) {
    if (a.act == MOE_ACT_SWIGLU) MOE_FFN_LAUNCH(MOE_ACT_SWIGLU, true, EPI_PRE);
    else MOE_FFN_LAUNCH(MOE_ACT_GELU, false, EPI_PRE);
  } else if (a.epi == 2) {
    if (a.act == MOE_ACT_SWIGLU) MOE_FFN_LAUNCH(MOE_ACT_SWIGLU, false, EPI_BWD);
    else MOE_FFN_LAUNCH(MOE_ACT_GELU, false, EPI_BWD);
  } else if (a.act == MOE_ACT_SWIGLU) {
    MOE_FFN_LAUNCH(MOE_ACT_SWIGLU, true, EPI_PLAIN);
  } else if (a.act == MOE_ACT_GELU) {
    MOE_FFN_LAUNCH(MOE_ACT_GELU, false, EPI_PLAIN);
  } else if (a.K >= kEarlyRefillK) {
    hipLaunchKernelGGL((ffn_gemm_bf16<-1, false, EPI_PLAIN, false, true>), grid, dim3(GTH), 0, s, A, a.expert_offsets,
                       b0, b1, o, a.E, a.K, a.Nout, pr, a.gather, a.gather_div, 0, 1, nullptr, a.n_rows_max);
  } else {
    MOE_FFN_LAUNCH(-1, false, EPI_PLAIN);
  }
#undef MOE_FFN_LAUNCH
#undef MOE_FFN_LAUNCH_BT
  return hipGetLastError();
}

hipError_t launch_wgrad_bf16(const void* aT, const void* bT, const int32_t* koff, int G, int M, int N, long long ld,
                             float* out0, float* out1, int split, hipStream_t s) {
  const long long tiles = (long long)G * ((M + GBM - 1) / GBM) * ((N + GBR - 1) / GBR);
  if (tiles == 0) return hipSuccess;
  if ((unsigned long long)GBM * ld * 2 >= (1ull << 32)) return hipErrorNotSupported;  // 32-bit load offsets in a tile
  hipLaunchKernelGGL(ffn_wgrad_bf16, dim3((unsigned)tiles), dim3(GTH), 0, s, (const bf16_t*)aT, (const bf16_t*)bT,
                     koff, G, M, N, ld, out0, out1, split);
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
                       a.E, a.K, a.Nout, a.gather, a.gather_div);
  else if (a.act == MOE_ACT_GELU)
    hipLaunchKernelGGL((ffn_gemm_f32<MOE_ACT_GELU, false>), grid, dim3(256), 0, s, A, a.expert_offsets, b0, b1, o,
                       a.E, a.K, a.Nout, a.gather, a.gather_div);
  else
    hipLaunchKernelGGL((ffn_gemm_f32<-1, false>), grid, dim3(256), 0, s, A, a.expert_offsets, b0, b1, o, a.E, a.K,
                       a.Nout, a.gather, a.gather_div);
  return hipGetLastError();
}

}  // namespace moe
