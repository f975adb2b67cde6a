// Geometry of the bf16 router's direct loads (route.hip): which x or W_g element each thread's load
// of a K slice reads. The kernel and the host-side check of those loads' bounds
// (tests/bounds/load_bounds.cpp) both compute the sources with these functions. Plain C++.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "gemm_geometry.h"  // MOE_HD

namespace moe {
namespace rgeom {

constexpr int kTokPerBlock = 64;   // tokens per block
constexpr int kThreads = 512;      // 8 waves
constexpr int kKC = 64;            // K slice per pipeline stage

MOE_HD int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// One stage holds a 64-wide K slice of the block's 64 x rows (XCH 16-byte chunks) and of all NT*16
// padded W_g rows, padded to a whole number of chunks per thread.
MOE_HD constexpr int stage_xch() { return kTokPerBlock * (kKC / 8); }
MOE_HD constexpr int stage_ch(int nt) { return stage_xch() + nt * 16 * (kKC / 8); }
MOE_HD constexpr int stage_lpt(int nt) { return (stage_ch(nt) + kThreads - 1) / kThreads; }

// Element offset (at K slice 0; slice kc adds kc*kKC) of load i of thread tid in block t0/kTokPerBlock:
// into x when *from_x, else into W_g. Rows past T re-read row T-1, padded experts the last real row,
// padding slots chunk 0 of row 0; none of those values is used.
MOE_HD size_t load_src(int nt, int i, int tid, int t0, int T, int D, int E, bool* from_x) {
  const int slot = i * kThreads + tid;
  if (slot < stage_xch()) {
    const int row = slot / (kKC / 8), ch = swz(row, slot % (kKC / 8));
    const int tok = t0 + row;
    *from_x = true;
    return (size_t)(tok < T ? tok : T - 1) * D + ch * 8;
  }
  const int ws = slot < stage_ch(nt) ? slot - stage_xch() : 0;
  const int row = ws / (kKC / 8), ch = swz(row, ws % (kKC / 8));
  *from_x = false;
  return (size_t)(row < E ? row : E - 1) * D + ch * 8;
}

}  // namespace rgeom
}  // namespace moe
