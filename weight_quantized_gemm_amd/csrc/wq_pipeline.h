// Shared pieces of the LDS-staged GEMM pipelines: tile order, LDS swizzles, and the
// stage barrier.  (Buffer resources and the direct-to-LDS load live in wq_device.h.)
#pragma once
#include "wq_device.h"

namespace wq {

// Map a linear workgroup id to a tile.  Workgroups are dispatched round-robin over the 8
// XCDs; consecutive tile ids are handed to one XCD so that its L2 sees a compact band of
// rows and columns, and inside the band tiles are walked in groups of 4 m-tiles.
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  int t = bid;
  if ((total & 7) == 0) t = (bid & 7) * (total >> 3) + (bid >> 3);
  constexpr int kGroupM = 4;
  const int per_group = kGroupM * tiles_n;
  const int g = t / per_group;
  const int first_m = g * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int r = t - g * per_group;
  tm = first_m + r % gm;
  tn = r / gm;
}

// Row-major tile of RA-byte rows read by 16-byte A-fragment loads (lanes 0..15 hit 16
// consecutive rows at one chunk): chunk c of row r lives in slot c ^ ((r / W) % C), with
// C = RA / 16 chunks per row and W = 256 / RA rows per 256-byte bank window, so the 16
// rows land in 16 distinct bank groups.
template <int RA>
__device__ __forceinline__ int row_slot(int r, int c) {
  constexpr int C = RA / 16, W = 256 / RA;
  return c ^ ((r / W) % C);
}

// Row-major tile of RB-byte rows read by tr8 transpose loads (8 consecutive rows, 32
// bytes each, per 32 lanes): 32-byte pair p of row r lives in pair p ^ ((r / W) % (8 / W)),
// W = 256 / RB, so the 8 rows land in 8 distinct bank groups.
template <int RB>
__device__ __forceinline__ int pair_slot(int r, int p) {
  constexpr int W = 256 / RB;
  return p ^ ((r / W) & (8 / W - 1));
}

// vmcnt(N) then the workgroup barrier (N: per-wave loads allowed to stay in flight)
template <int N>
__device__ __forceinline__ void stage_barrier() {
  if constexpr (N == 0) WQ_STAGE_BARRIER(0);
  else if constexpr (N == 2) WQ_STAGE_BARRIER(2);
  else if constexpr (N == 4) WQ_STAGE_BARRIER(4);
  else if constexpr (N == 5) WQ_STAGE_BARRIER(5);
  else if constexpr (N == 6) WQ_STAGE_BARRIER(6);
  else if constexpr (N == 8) WQ_STAGE_BARRIER(8);
  else if constexpr (N == 9) WQ_STAGE_BARRIER(9);
  else if constexpr (N == 10) WQ_STAGE_BARRIER(10);
  else if constexpr (N == 12) WQ_STAGE_BARRIER(12);
  else if constexpr (N == 16) WQ_STAGE_BARRIER(16);
  else if constexpr (N == 18) WQ_STAGE_BARRIER(18);
  else if constexpr (N == 20) WQ_STAGE_BARRIER(20);
  else if constexpr (N == 24) WQ_STAGE_BARRIER(24);
  else static_assert(N < 0, "add this vmcnt value");
}

}  // namespace wq
