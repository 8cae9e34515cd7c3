// Internal layout of ts_plan, shared by the host-only plan builder (plan.cpp,
// built with the host compiler) and the HIP side (abi.hip).  No HIP types here.
#pragma once
#include <cstdint>
#include <string>
#include <vector>

#include "../../include/tileshare.h"

// Query rows per block of the blended attention (one per lane of the eight
// wavefronts of a bf16 attention workgroup, one per thread of an fp32 one).
constexpr int32_t TS_QBLOCK = 256;

struct ts_plan {
  ts_tiling_desc desc;
  int32_t n_tiles = 0, n = 0, n_union = 0, n_entries = 0, max_cover = 0;
  int32_t ext[3] = {1, 1, 1};
  std::vector<int32_t> axis_starts[3];
  std::vector<int32_t> tile_start;   // [n_tiles*3]
  std::vector<int32_t> tile_rows;    // [n_tiles*n]
  std::vector<int32_t> cover_ptr;    // [n_union+1]
  std::vector<int32_t> cover_tile;   // [n_entries]
  std::vector<int32_t> cover_local;  // [n_entries]
  std::vector<float> cover_w;        // [n_entries]
  std::vector<int32_t> local_pos;    // [n] packed tau | y<<10 | x<<20
  // Query blocks of the blended attention of shared layers: the grid rows
  // grouped by the set of tiles that hold them with a nonzero w-bar, each
  // group cut into blocks of TS_QBLOCK rows.  A block's rows are attended in
  // every window of its set (ascending tile order) and blended in registers.
  int32_t nblk = 0, blk_maxc = 0;    // blocks; most tiles of one block
  std::vector<int32_t> blk_nt;       // [nblk] tiles of each block
  std::vector<int32_t> blk_tiles;    // [nblk*blk_maxc] those tiles, ascending (padding -1)
  std::vector<int32_t> blk_rows;     // [nblk*TS_QBLOCK] grid row of each slot (-1: empty)
  std::vector<float> blk_w;          // [nblk*blk_maxc*TS_QBLOCK] w-bar of (block, tile i, slot)
  // Job order of the blended attention.  Each head's blocks are split in two
  // halves of equal work (windows), A and B; every class of blocks with the
  // same number of windows is cut at its middle, the odd block going to the
  // half with less work.  blk_order lists half A then half B, each class by
  // class from the most windows down, blocks ascending; blk_cls holds, per
  // class, {count in A, offset in blk_order, count in B, offset}.
  int32_t blk_ncls = 0;
  std::vector<int32_t> blk_order;    // [nblk]
  std::vector<int32_t> blk_cls;      // [blk_ncls*4]

  // device copies (owned; void* to keep HIP out of this header)
  void* d_tile_rows = nullptr;   // int32 [n_tiles*n]
  void* d_tile_rows_local = nullptr;  // int32 [n_tiles*n]: t*(n+1)+j, the rows of per-tile layouts
  void* d_cover_ptr = nullptr;   // int32 [n_union+1]
  void* d_entry_row = nullptr;   // int32 [n_entries]: t*(n+1)+local of each entry
  void* d_cover_w = nullptr;     // fp32 [n_entries]
  void* d_local_pos = nullptr;   // int32 [n]
  void* d_rope_glob = nullptr;   // grid-coordinate (cos, sin) table, see rope_table_global
  void* d_tile_start = nullptr;  // int32 [n_tiles*3]
  void* d_blk_nt = nullptr;      // query blocks, as blk_* above
  void* d_blk_tiles = nullptr;
  void* d_blk_rows = nullptr;
  void* d_blk_w = nullptr;
  void* d_blk_order = nullptr;
  void* d_blk_cls = nullptr;
  int32_t rope_glob_off[3] = {0, 0, 0};
  int32_t rope_hd = 0;
  float rope_base = 0.f;
  int32_t rope_pairs[3] = {0, 0, 0};
  bool uploaded = false;
};

namespace tsplan {
// Builds every host-side map of the plan; returns an error message or "".
std::string build(const ts_tiling_desc& desc, ts_plan& p);
// Pairs per axis for a head size (t, h, w).
void rope_pairs(int32_t ndim, int32_t head_dim, int32_t out[3]);
// Tile-local RoPE values: cos/sin [n * head_dim/2] of pair k of local token j
// (fp64 angle pos * base^(-i/m), rounded to fp32), for export.
void rope_local(const ts_plan& p, int32_t head_dim, float base, float* cos_out, float* sin_out);
// RoPE table over grid coordinates: pair i of axis a at coordinate pos is
// (cos, sin) at tab[off[a] + 2*(pos*pairs[a] + i) + {0, 1}].  Rotating every
// row by its grid coordinate gives the same token-token scores as rotating by
// tile-local positions (the angle of a pair depends only on the coordinate
// difference); the global token of tile t is rotated by the tile's start.
void rope_table_global(const ts_plan& p, int32_t head_dim, float base, std::vector<float>& tab, int32_t off[3]);
}  // namespace tsplan
