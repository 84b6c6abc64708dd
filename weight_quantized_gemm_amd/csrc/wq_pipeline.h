// Shared pieces of the LDS-staged GEMM pipelines: tile order, LDS swizzles, and the
// stage barrier.  (Buffer resources and the direct-to-LDS load live in wq_device.h.)
#pragma once
#include "wq_device.h"

namespace wq {

// Map a linear workgroup id to a tile.  Workgroups are dispatched round-robin over the 8
// XCDs, each with its own L2.  With rm > 0 (xcd_region_rows) the tile grid is cut into an
// rm x (8 / rm) grid of equal rectangles, one per XCD, so that each L2 sees the x1 rows and
// weight columns of one rectangle only; otherwise each XCD takes a contiguous band of tile
// ids.  Inside its share an XCD walks groups of 4 m-tiles, column by column, so that the
// tiles running at once on its CUs share both their x1 rows and their weight columns.
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int rm, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  constexpr int kGroupM = 4;
  if (rm > 0 && (total & 7) == 0) {
    const int rn = 8 / rm;
    const int Rm = tiles_m / rm, Rn = tiles_n / rn;   // rectangle size in tiles
    const int x = bid & 7, t = bid >> 3;              // XCD, index within its rectangle
    const int per_group = kGroupM * Rn;
    const int g = t / per_group;
    const int gm = min(Rm - g * kGroupM, kGroupM);
    const int r = t - g * per_group;
    tm = (x / rn) * Rm + g * kGroupM + r % gm;
    tn = (x % rn) * Rn + r / gm;
    return;
  }
  int t = bid;
  if ((total & 7) == 0) t = (bid & 7) * (total >> 3) + (bid >> 3);
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

// Wait until at most N vector-memory loads of this wave are in flight and all of its LDS
// reads have completed, then join the workgroup barrier.  After it, no wave still reads a
// stage that a direct-to-LDS load issued after the barrier may overwrite.
template <int N>
__device__ __forceinline__ void stage_barrier() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Wave-local form: at most N vector-memory loads of this wave in flight, no barrier.
template <int N>
__device__ __forceinline__ void wave_wait() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Direct-to-LDS load of the per-group scale and offset rows that a 64-row k block needs:
// the groups ga and gb that hold its rows 31 and 63 (group ends fall on multiples of 32,
// so these are the only groups a fold inside the block can close).  COLS 16-bit values
// from column n0 of each row land in an LDS block: scale rows at +0 and +2*COLS, offset
// rows at +P/2 and +P/2 + 2*COLS, where P = 1 KiB for COLS <= 128 (two loads, one per
// half-wave) and 2 KiB for COLS == 256 (two full-wave loads).  With no offset tensor the
// offset rows read zeros.  rs / ro cover the tensors from column n0 on.
template <int COLS>
__device__ __forceinline__ void dma_group_params(uint8_t* dst, const u32x4_t& rs, const u32x4_t& ro,
                                                 bool has_offset, int ga, int gb, int n, int lane) {
  if constexpr (COLS == 256) {
    const int e = lane >> 5, c = lane & 31;  // 32 chunks of 16 bytes per row
    const uint32_t off = (uint32_t)(e ? gb : ga) * (uint32_t)n * 2u + 16u * (uint32_t)c;
    dma16(rs, dst, off);
    dma16(has_offset ? ro : rs, dst + 1024, has_offset ? off : kOOB);
  } else {
    static_assert(COLS % 8 == 0 && 4 * COLS <= 512, "two rows of COLS 16-bit values per half");
    constexpr int L = COLS / 8;  // 16-byte chunks per row
    const int h = lane & 31, e = h / L, c = h % L;
    const uint32_t off = h < 2 * L ? (uint32_t)(e ? gb : ga) * (uint32_t)n * 2u + 16u * (uint32_t)c : kOOB;
    if (lane < 32) dma16(rs, dst, off);
    else dma16(has_offset ? ro : rs, dst, has_offset ? off : kOOB);  // lands at dst + 512 + 16 h
  }
}

}  // namespace wq
