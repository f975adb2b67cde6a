// Host-side bounds check of the direct loads of the bf16 grouped GEMM (forward, gathered, K-major,
// weight-gradient forms) and of the bf16 router. Their buffer resources set no range clamp, so the
// hardware would read whatever an offset names; this walks every block of a launch, every lane and
// every load (at the first and last K stage, and every stage where the K-major form switches matrix)
// and checks that each 16-byte access lies inside its operand. The per-lane positions and offsets come
// from the kernels' own geometry headers; the launch grid and the block -> tile map are restated here.
// Built with g++ by the test that uses it; test infrastructure, not part of the library.
#include <stdint.h>
#include <stdlib.h>

#include <vector>

#include "gemm_geometry.h"
#include "route_geometry.h"

using namespace moe::geom;

namespace {

struct Check {
  int64_t violations = 0, accesses = 0;
  int64_t first_bad[4] = {-1, -1, -1, -1};  // block, wave, lane, load of the first violation
  void access(int64_t start, int64_t len, int64_t extent, int block, int wave, int lane, int load) {
    ++accesses;
    if (start < 0 || start + len > extent) {
      if (violations == 0) {
        first_bad[0] = block, first_bad[1] = wave, first_bad[2] = lane, first_bad[3] = load;
      }
      ++violations;
    }
  }
  // a 32-bit offset computed by the kernel must equal the true (64-bit) one
  void wraps(uint32_t got, int64_t want, int block, int wave, int lane, int load) {
    ++accesses;
    if ((int64_t)got != want) {
      if (violations == 0) {
        first_bad[0] = block, first_bad[1] = wave, first_bad[2] = lane, first_bad[3] = load;
      }
      ++violations;
    }
  }
};

// The block -> (expert, row tile, column tile) map of the grouped GEMM: tiles listed expert-major
// (ceil(count / GBM) row tiles times NT column tiles per expert), the list cut into 8 equal contiguous
// ranges, block b taking entry b / 8 of range b % 8; inside an expert, groups of G_GN column tiles,
// row-tile-major inside a group.
bool tile_of(const int32_t* off, int E, int NT, int block, int* e_out, int* mt_out, int* nt_out) {
  int64_t L = 0;
  for (int e = 0; e < E; ++e) L += (int64_t)((off[e + 1] - off[e] + GBM - 1) / GBM) * NT;
  const int64_t per = (L + 7) / 8;
  const int64_t xcd = block % 8, j = block / 8;
  if (j >= per) return false;
  const int64_t t = xcd * per + j;
  if (t >= L) return false;
  int64_t start = 0;
  for (int e = 0; e < E; ++e) {
    const int cnt = off[e + 1] - off[e];
    const int64_t n = (int64_t)((cnt + GBM - 1) / GBM) * NT;
    if (t < start + n) {
      const int local = (int)(t - start);
      const int MT = (cnt + GBM - 1) / GBM;
      const int gsz = G_GN * MT;
      const int g = local / gsz, r = local % gsz;
      const int gn = (G_GN < NT - g * G_GN) ? G_GN : NT - g * G_GN;
      *e_out = e;
      *mt_out = r / gn;
      *nt_out = g * G_GN + r % gn;
      return true;
    }
    start += n;
  }
  return false;
}

}  // namespace

extern "C" {

// Grouped GEMM launch as launch_ffn_bf16 issues it. bt = 0: B as (out, in) rows, [E, nout, K] (two
// matrices when dual, the paired SwiGLU tile); bt = 1: B K-major per expert, rows k < ksplit from the
// first matrix ([E, ksplit, nout]), the rest from the second ([E, K - ksplit, nout]). gather: when not
// null, A row r is row gather[r] / gdiv of an a_rows-row source (x); else A is [n_rows_max, K].
// stats (8 int64): violations, accesses, tiles run, tiles missing or run twice, first violation
// (block, wave, lane, load). Returns the violation count.
// splits > 1: the split-K down-projection (block b is split b % splits of tile slot b / splits, over K
// stages [s*nk/S, (s+1)*nk/S)), whose epilogue stores float32 partials to [splits][n_rows_max][nout].
int64_t moe_check_ffn_loads(const int32_t* off, int E, int n_rows_max, int K, int nout, int dual, int bt,
                            int ksplit, const int32_t* gather, int gdiv, int64_t a_rows, int splits, int64_t* stats) {
  Check ck;
  const int bno = dual ? GBR / 2 : GBR;
  const int NT = (nout + bno - 1) / bno;
  const int64_t row_tiles = (n_rows_max + GBM - 1) / GBM + (E < n_rows_max ? E : n_rows_max);
  const int64_t grid = (row_tiles * NT + 8) * splits;
  const int nk_all = K / GBK;
  const int64_t a_extent = (gather ? a_rows : (int64_t)n_rows_max) * K * 2;
  std::vector<int> seen;
  int64_t tiles_expected = 0;
  std::vector<int64_t> first_tile(E + 1, 0);
  for (int e = 0; e < E; ++e) {
    first_tile[e] = tiles_expected;
    tiles_expected += (int64_t)((off[e + 1] - off[e] + GBM - 1) / GBM) * NT;
  }
  seen.assign(tiles_expected, 0);
  int64_t run = 0;
  for (int64_t b = 0; b < grid; ++b) {
    int e, mt, nt;
    const int s = (int)(b % splits);
    if (!tile_of(off, E, NT, (int)(b / splits), &e, &mt, &nt)) continue;
    ++run;
    const int cnt = off[e + 1] - off[e];
    const int MT = (cnt + GBM - 1) / GBM;
    if (s == 0) seen[first_tile[e] + (int64_t)mt * NT + nt] += 1;
    // the split's stages: its resources start k0 = kt0 * GBK columns in, so stage kt' of the split reads
    // what stage kt0 + kt' reads unsplit
    const int kt0 = s * nk_all / splits, kt1 = (s + 1) * nk_all / splits;
    const int nk = kt1;  // last stage index + 1, in unsplit stage numbers
    const int row0 = off[e] + mt * GBM;
    const int mrows = (GBM < cnt - mt * GBM) ? GBM : cnt - mt * GBM;
    const int n0 = nt * bno;
    (void)MT;
    for (int w = 0; w < GW; ++w)
      for (int l = 0; l < kLanes; ++l) {
        for (int i = 0; i < G_NAL; ++i) {
          if (a_load_skipped(i, mrows)) continue;
          int row, ch;
          a_load_pos(i, w, l, &row, &ch);
          const int r = row < mrows ? row : 0;
          int64_t arow, base;
          if (gather) {
            ck.access(row0 + r, 1, n_rows_max, (int)b, w, l, i);  // the gather index read itself
            if (row0 + r < 0 || row0 + r >= n_rows_max) continue;
            arow = gather[row0 + r] / gdiv;
            base = 0;
          } else {
            arow = r;
            base = (int64_t)row0 * K * 2;
          }
          const uint32_t voff = a_load_off((uint32_t)arow, K, ch);
          ck.wraps(voff, arow * K * 2 + ch * 16, (int)b, w, l, i);
          for (int kt : {kt0, nk - 1}) {
            ck.wraps(voff + stage_soff(kt - kt0), (int64_t)voff + (int64_t)(kt - kt0) * GBK * 2, (int)b, w, l, i);
            ck.access(base + voff + stage_soff(kt), 16, a_extent, (int)b, w, l, i);
          }
        }
        for (int i = G_NAL; i < G_LPS; ++i) {
          if (!bt) {
            int row, ch;
            b_load_pos(i, w, l, &row, &ch);
            const int f = b_weight_row(row, dual);
            const uint32_t voff = b_load_off(f, n0, nout, K, ch);
            const int64_t base = ((int64_t)e * nout + n0) * K * 2;
            ck.wraps(voff, (int64_t)(n0 + f < nout ? f : 0) * K * 2 + ch * 16, (int)b, w, l, i);
            for (int kt : {kt0, nk - 1})
              ck.access(base + voff + stage_soff(kt), 16, (int64_t)E * nout * K * 2, (int)b, w, l, i);
          } else {
            int k, c;
            bt_load_pos(i, w, l, &k, &c);
            const uint32_t voff = bt_load_off(k, c, n0, nout);
            ck.wraps(voff, ((int64_t)k * nout + (n0 + c * 8 < nout ? c * 8 : 0)) * 2, (int)b, w, l, i);
            const int ks = ksplit / GBK;  // first stage from the second matrix
            for (int kt : {0, ks - 1, ks, nk - 1}) {
              if (kt < 0 || kt >= nk) continue;
              const int k0 = kt * GBK;
              const bool lo = k0 < ksplit;
              const int64_t rows = lo ? ksplit : K - ksplit;
              const int64_t base = ((int64_t)e * rows * nout + n0) * 2;
              const int64_t soff = (int64_t)(lo ? k0 : k0 - ksplit) * nout * 2;
              ck.access(base + voff + soff, 16, (int64_t)E * rows * nout * 2, (int)b, w, l, i);
            }
          }
        }
      }
    // epilogue: 16-byte row pieces of rows < mrows, columns n0 + c < nout (c a multiple of 8); split K:
    // float32 partial pieces of 4 columns into plane s
    if (splits == 1) {
      for (int c = 0; c < bno; c += 8)
        if (n0 + c < nout) {
          ck.access(((int64_t)(row0 + mrows - 1) * nout + n0 + c) * 2, 16, (int64_t)n_rows_max * nout * 2, (int)b,
                    -1, c, -1);
          ck.access(((int64_t)row0 * nout + n0 + c) * 2, 16, (int64_t)n_rows_max * nout * 2, (int)b, -1, c, -1);
        }
    } else {
      const int64_t plane = (int64_t)n_rows_max * nout;
      for (int c = 0; c < bno; c += 4)
        if (n0 + c < nout)
          for (int64_t r : {(int64_t)row0, (int64_t)row0 + mrows - 1})
            ck.access((s * plane + r * nout + n0 + c) * 4, 16, splits * plane * 4, (int)b, -1, c, -1);
    }
  }
  int64_t bad_tiles = 0;
  for (int v : seen) bad_tiles += v != 1;
  stats[0] = ck.violations;
  stats[1] = ck.accesses;
  stats[2] = run;
  stats[3] = bad_tiles;
  for (int q = 0; q < 4; ++q) stats[4 + q] = ck.first_bad[q];
  return ck.violations + bad_tiles;
}

// Weight-gradient launch as launch_wgrad_bf16 issues it: group g owns reduction columns
// [koff[g], koff[g+1]) (multiples of 64) of aT [M, ld] and bT [N, ld]; tiles of GBM x GBR (m, n).
int64_t moe_check_wgrad_loads(const int32_t* koff, int G, int M, int N, int64_t ld, int64_t* stats) {
  Check ck;
  const int MT = (M + GBM - 1) / GBM, NT = (N + GBR - 1) / GBR;
  for (int64_t t = 0; t < (int64_t)G * MT * NT; ++t) {
    const int g = (int)(t / (MT * NT)), rem = (int)(t % (MT * NT));
    const int m0 = rem / NT * GBM, n0 = rem % NT * GBR;
    const int mrows = (GBM < M - m0) ? GBM : M - m0;
    const int k0 = koff[g], nk = (koff[g + 1] - k0) / GBK;
    if (nk <= 0) continue;
    for (int w = 0; w < GW; ++w)
      for (int l = 0; l < kLanes; ++l)
        for (int i = 0; i < G_LPS; ++i) {
          int row, ch;
          int64_t base, extent, r;
          if (i < G_NAL) {
            a_load_pos(i, w, l, &row, &ch);
            r = row < mrows ? row : 0;
            base = ((int64_t)m0 * ld + k0) * 2;
            extent = (int64_t)M * ld * 2;
          } else {
            b_load_pos(i, w, l, &row, &ch);
            r = n0 + row < N ? row : 0;
            base = ((int64_t)n0 * ld + k0) * 2;
            extent = (int64_t)N * ld * 2;
          }
          const uint32_t voff = (uint32_t)(r * ld) * 2u + ch * 16;
          ck.wraps(voff, r * ld * 2 + ch * 16, (int)t, w, l, i);
          for (int kt : {0, nk - 1}) ck.access(base + voff + stage_soff(kt), 16, extent, (int)t, w, l, i);
        }
  }
  stats[0] = ck.violations;
  stats[1] = ck.accesses;
  for (int q = 0; q < 4; ++q) stats[4 + q] = ck.first_bad[q];
  return ck.violations;
}

// bf16 router launch: blocks of 64 tokens, every thread's loads of every stage (x [T, D], W_g [E, D]).
int64_t moe_check_route_loads(int T, int D, int E, int64_t* stats) {
  Check ck;
  const int ntiles = (E + 15) / 16;
  const int nt = ntiles <= 1 ? 1 : ntiles <= 2 ? 2 : ntiles <= 4 ? 4 : ntiles <= 8 ? 8 : 16;
  const int lpt = moe::rgeom::stage_lpt(nt);
  const int n_kc = D / moe::rgeom::kKC;
  const int blocks = (T + moe::rgeom::kTokPerBlock - 1) / moe::rgeom::kTokPerBlock;
  for (int b = 0; b < blocks; ++b)
    for (int tid = 0; tid < moe::rgeom::kThreads; ++tid)
      for (int i = 0; i < lpt; ++i) {
        bool from_x;
        const int64_t src = (int64_t)moe::rgeom::load_src(nt, i, tid, b * moe::rgeom::kTokPerBlock, T, D, E, &from_x);
        const int64_t extent = (int64_t)(from_x ? T : E) * D;
        for (int kc : {0, n_kc - 1})
          ck.access(src + (int64_t)kc * moe::rgeom::kKC, 8, extent, b, tid / 64, tid % 64, i);
      }
  stats[0] = ck.violations;
  stats[1] = ck.accesses;
  for (int q = 0; q < 4; ++q) stats[4 + q] = ck.first_bad[q];
  return ck.violations;
}

}  // extern "C"
