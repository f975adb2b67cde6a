// Geometry of the bf16 grouped GEMM (ffn.hip): its tile constants and the position and 32-bit byte
// offset of every direct load it issues. The kernel and the host-side check of those loads' bounds
// (tests/bounds/load_bounds.cpp) both compute the offsets with these functions. Plain C++: MOE_HD
// marks the functions both sides compile.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define MOE_HD __host__ __device__ __forceinline__
#else
#define MOE_HD inline
#endif

namespace moe {
namespace geom {

constexpr int kLanes = 64;                          // wavefront width
constexpr int GW = 8, GTH = GW * kLanes;            // waves / threads per block
constexpr int GBM = 320, GBR = 256, GBK = 64;       // tile rows, B rows per tile, K per stage
constexpr int GMB = GBM / 64;                       // 32-row blocks per wave (two wave rows)
constexpr int GKCH = GBK / 8;                       // 16-byte chunks per tile row
constexpr int G_ACH = GBM * GKCH, G_STAGE = (GBM + GBR) * GKCH, G_LPS = G_STAGE / GTH, G_KS = GBK / 16;
constexpr int G_GN = 4;                             // column tiles per group in the tile order
constexpr int G_NAL = G_ACH / GTH;                  // A loads per stage and lane

// LDS chunk of a tile row: 16-byte chunk ch of row `row` sits at chunk ch ^ ((row >> 1) & 7)
MOE_HD int gswz(int row, int ch) { return ch ^ ((row >> 1) & 7); }

// Load i of a stage fills LDS chunk slot i*GTH + wave*64 + lane: loads i < G_NAL fill A rows (the
// block's token rows), the rest the B slice (weight rows, or K-major weight rows in the data-gradient
// form).
MOE_HD int load_slot(int i, int wave, int lane) { return i * GTH + wave * kLanes + lane; }

// A load i: tile row and the 16-byte chunk of the row's K stage it reads
MOE_HD void a_load_pos(int i, int wave, int lane, int* row, int* ch) {
  const int slot = load_slot(i, wave, lane);
  *row = slot / GKCH;
  *ch = gswz(*row, slot % GKCH);
}
// A load i reads only rows at or past the tile's row count: not issued
MOE_HD bool a_load_skipped(int i, int mrows) { return i * (GTH / GKCH) >= mrows; }
// byte offset of an A load from the rows' base: row `arow` (the tile row, or the gathered source row)
MOE_HD uint32_t a_load_off(uint32_t arow, int K, int ch) { return arow * (uint32_t)K * 2u + ch * 16; }

// B load i (weights as (out, in) rows): B-tile row and chunk
MOE_HD void b_load_pos(int i, int wave, int lane, int* row, int* ch) {
  const int bs = load_slot(i, wave, lane) - G_ACH;
  *row = bs / GKCH;
  *ch = gswz(*row, bs % GKCH);
}
// the paired SwiGLU tile takes its second half (W3 rows) from the second weight matrix
MOE_HD bool b_load_second(int i) { return i >= G_NAL + (G_LPS - G_NAL) / 2; }
// weight row (from the tile's first weight row) of B-tile row `row`
MOE_HD int b_weight_row(int row, bool dual) { return dual ? row % (GBR / 2) : row; }
// byte offset from the tile's first weight row; rows past Nout re-read the first row (never stored)
MOE_HD uint32_t b_load_off(int f, int n0, int nout, int K, int ch) {
  return (n0 + f < nout ? (uint32_t)f * (uint32_t)K * 2u : 0u) + ch * 16;
}

// K-major B load i: reduction row k of the stage and the 16-byte column chunk c (8 columns)
MOE_HD void bt_load_pos(int i, int wave, int lane, int* k, int* c) {
  const int bs = load_slot(i, wave, lane) - G_ACH;
  *k = bs / (GBR / 8);
  *c = (bs % (GBR / 8)) ^ ((*k & 3) << 2);
}
// byte offset from the expert slice's stage row 0, column n0; columns past Nout re-read column n0
MOE_HD uint32_t bt_load_off(int k, int c, int n0, int nout) {
  return (uint32_t)(k * nout + (n0 + c * 8 < nout ? c * 8 : 0)) * 2u;
}

// scalar byte offset of stage kt (rows contiguous along K)
MOE_HD uint32_t stage_soff(int kt) { return (uint32_t)kt * (GBK * 2); }

}  // namespace geom
}  // namespace moe
