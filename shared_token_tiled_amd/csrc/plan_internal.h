// Internal layout of ts_plan, shared by the host-only plan builder (plan.cpp,
// built with the host compiler) and the HIP side (abi.hip).  No HIP types here.
#pragma once
#include <cstdint>
#include <string>
#include <vector>

#include "../../include/tileshare.h"

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

  // device copies (owned; void* to keep HIP out of this header)
  void* d_tile_rows = nullptr;   // int32 [n_tiles*n]
  void* d_cover_ptr = nullptr;   // int32 [n_union+1]
  void* d_entry_row = nullptr;   // int32 [n_entries]: t*(n+1)+local of each entry
  void* d_cover_w = nullptr;     // fp32 [n_entries]
  void* d_local_pos = nullptr;   // int32 [n]
  void* d_rope = nullptr;        // compact per-axis (cos, sin) table, see rope_table
  void* d_rope_glob = nullptr;   // grid-coordinate (cos, sin) table, see rope_table_global
  void* d_tile_start = nullptr;  // int32 [n_tiles*3]
  int32_t rope_glob_off[3] = {0, 0, 0};
  int32_t rope_hd = 0;
  float rope_base = 0.f;
  int32_t rope_floats = 0;       // floats in the compact table
  int32_t rope_pairs[3] = {0, 0, 0};
  int32_t rope_off[3] = {0, 0, 0};
  int32_t rope_wbase[3] = {0, 0, 0};
  int32_t rope_wpairs[3] = {0, 0, 0};
  bool uploaded = false;
};

namespace tsplan {
// Builds every host-side map of the plan; returns an error message or "".
std::string build(const ts_tiling_desc& desc, ts_plan& p);
// Pairs per axis for a head size (t, h, w).
void rope_pairs(int32_t ndim, int32_t head_dim, int32_t out[3]);
// Compact RoPE table, one block per axis.  Axis a owns the global pairs
// [k0_a, k0_a + pairs[a]); its block covers the window of pairs
// [wbase[a], wbase[a] + wpairs[a]), that range widened to whole groups of 4
// pairs (8 dims), so a group's entries are 32-byte aligned and contiguous.
// The (cos, sin) of global pair k at position pos of axis a sits at
// tab[off[a] + 2*(pos*wpairs[a] + k - wbase[a]) + {0, 1}]; window slots of
// pairs that belong to another axis hold the identity (1, 0).
void rope_table(const ts_plan& p, int32_t head_dim, float base, std::vector<float>& tab, int32_t pairs[3],
                int32_t off[3], int32_t wbase[3], int32_t wpairs[3]);
// RoPE table over grid coordinates: pair i of axis a at coordinate pos is
// (cos, sin) at tab[off[a] + 2*(pos*pairs[a] + i) + {0, 1}].  Rotating every
// row by its grid coordinate gives the same token-token scores as rotating by
// tile-local positions (the angle of a pair depends only on the coordinate
// difference); the global token of tile t is rotated by the tile's start.
void rope_table_global(const ts_plan& p, int32_t head_dim, float base, std::vector<float>& tab, int32_t off[3]);
}  // namespace tsplan
