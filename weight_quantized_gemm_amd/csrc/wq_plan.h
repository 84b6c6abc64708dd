// Call planning: which kernel serves a problem, its tile rows, its k splits and the
// workspace layout.  Host-only C++ (no HIP types), so that planning builds and runs
// without a GPU, e.g. in a sanitizer build together with the validation code.
#pragma once
#include <cstdint>

#include "wq_problem.h"

namespace wq {

// Compute units of the current device, read once per device and cached (the library's only
// state between calls).  Without a usable device it is an MI355X's 256.
int device_cu_count();
constexpr int kDefaultCUs = 256;

// Geometry the planners share with the kernels.
constexpr int kAqTileN = 256;     // columns of a tiled anti-quant workgroup tile
constexpr int kQmTileN = 256;     // columns of a W8A8 workgroup tile
constexpr int kSmWaves = 8;       // small-m kernel: waves per workgroup
constexpr int kSmSlab = 128;      // small-m kernel: columns per workgroup
constexpr int kSmRows = 64;       // small-m kernel: k rows per block (a wave's unit of work)
constexpr int64_t kSmallM = 32;   // the small-m kernel serves m <= 32

struct SplitPlan {
  int kchunk = 64;   // k rows per split (a multiple of 64)
  int splits = 1;
};

// Small m: k splits of the slab kernel, for `cus` compute units.
SplitPlan aq_smallm_plan(int64_t m, int k, int n, int group, bool grouped, int cus);
// Tiled kernels: split k when the tiles alone leave compute units idle.
SplitPlan gemm_split_plan(int64_t tiles, int k, int unit, int cus);
// Tile rows of the anti-quant and W8A8 tiled kernels' default configurations.
int aq_gemm_tile_m(int64_t m, int k, int n, bool grouped, int cus);
int qm_gemm_tile_m(int64_t m, int k, int n, int cus);

// Per-XCD tile rectangles: the tile grid (tiles_m x tiles_n, 8 XCDs) is cut into an
// rm x (8 / rm) grid of equal rectangles, rm in {1, 2, 4, 8}, the one whose rectangle needs
// the fewest operand bytes (rectangle rows x mtile_bytes + columns x ntile_bytes; ties go
// to the taller rectangle).  0 when no rm divides the grid evenly (the kernels then hand
// each XCD a band of consecutive tiles).
int xcd_region_rows(int64_t tiles_m, int64_t tiles_n, double mtile_bytes, double ntile_bytes);

struct AqPlan {
  bool empty_k = false;
  bool small_m = false;
  SplitPlan split;           // k splits of the small-m or the tiled kernel
  int bm = 0;                // tiled kernel: tile rows (aq_gemm_tile_m)
  int64_t partial_bytes = 0;
  int64_t rowsum_bytes = 0;
  int64_t param_bytes = 0;   // per-group scale / offset given transposed: row-major copies
  int64_t gsum_bytes = 0;    // large m, per-group: row sums of x1 per group, (groups, m) fp32
  int64_t workspace = 0;
};
AqPlan plan_antiquant(const AntiquantProblem& p, int cus);
// C, the constant the fed weight images add to the codes: bf16 images of int4 codes are
// code + 136 (the magic-exponent image, wq_device.h); all other images are exact.
float code_bias(const AntiquantProblem& p);

struct QmPlan {
  SplitPlan split;
  int bm = 128;
  int64_t workspace = 0;
};
QmPlan plan_quant(const QuantProblem& p, int cus);

}  // namespace wq
