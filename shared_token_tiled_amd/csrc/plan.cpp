// Host-side tiling plan: tile starts, tile rows, coverage map, w-bar, RoPE.
//
// TileShare paper page, Figure 2 caption (overlap tokens stored once, attended
// in every window that holds them, blended with the released weights w-bar)
// and Figure 5 (tiles per pixel, tile-start lines).  Clamp rule, ramp shape,
// axis split of RoPE: see the readings in tileshare.h.
//
// Built with the host compiler and -ffp-contract=off: w-bar and the RoPE
// angles are float64 expressions evaluated in a fixed order and rounded once
// to fp32, so the maps are reproducible bit for bit.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <map>

#include "plan_internal.h"

namespace tsplan {

static void axis_starts(int32_t n, int32_t L, int32_t S, std::vector<int32_t>& starts,
                        int32_t& ext) {
  starts.clear();
  if (n <= L) {
    starts.push_back(0);
    ext = n;
    return;
  }
  const int32_t count = (n - L + S - 1) / S + 1;
  for (int32_t i = 0; i < count; ++i) {
    const int64_t s = int64_t(i) * S;
    starts.push_back(s < n - L ? int32_t(s) : n - L);
  }
  ext = L;
}

// Unnormalised ramp of tile i at local position u along one axis.
static double axis_ramp(const std::vector<int32_t>& st, int32_t L, size_t i, int32_t u) {
  const int32_t o_prev = i > 0 ? st[i - 1] + L - st[i] : 0;
  const int32_t o_next = i + 1 < st.size() ? st[i] + L - st[i + 1] : 0;
  const double lead = u < o_prev ? double(u + 1) / double(o_prev + 1) : 1.0;
  const double trail = u >= L - o_next ? double(L - u) / double(o_next + 1) : 1.0;
  return lead * trail;
}

// Query blocks of the blended attention.  Rows with the same set of tiles
// of nonzero weight form a group (a ramp weight is never zero, so the set is
// the row's cover; hard stitching keeps one tile); groups are ordered by
// decreasing set size (longest work first), then by their tile lists, and
// their rows ascending, cut into blocks of TS_QBLOCK slots.
static void build_blocks(ts_plan& p) {
  std::map<std::vector<int32_t>, std::vector<int32_t>> groups;
  std::vector<int32_t> key;
  for (int32_t q = 0; q < p.n_union; ++q) {
    key.clear();
    for (int32_t e = p.cover_ptr[q]; e < p.cover_ptr[q + 1]; ++e)
      if (p.cover_w[e] != 0.f) key.push_back(p.cover_tile[e]);
    groups[key].push_back(q);
  }
  std::vector<const std::pair<const std::vector<int32_t>, std::vector<int32_t>>*> order;
  p.blk_maxc = 0;
  for (const auto& g : groups) {
    order.push_back(&g);
    p.blk_maxc = std::max<int32_t>(p.blk_maxc, int32_t(g.first.size()));
  }
  std::stable_sort(order.begin(), order.end(),
                   [](const auto* a, const auto* b) { return a->first.size() > b->first.size(); });
  p.nblk = 0;
  for (const auto* g : order) p.nblk += int32_t((g->second.size() + TS_QBLOCK - 1) / TS_QBLOCK);
  p.blk_nt.assign(p.nblk, 0);
  p.blk_tiles.assign(size_t(p.nblk) * p.blk_maxc, -1);
  p.blk_rows.assign(size_t(p.nblk) * TS_QBLOCK, -1);
  p.blk_w.assign(size_t(p.nblk) * p.blk_maxc * TS_QBLOCK, 0.f);
  int32_t b = 0;
  for (const auto* g : order) {
    const std::vector<int32_t>& tiles = g->first;
    const std::vector<int32_t>& rows = g->second;
    for (size_t r0 = 0; r0 < rows.size(); r0 += TS_QBLOCK, ++b) {
      p.blk_nt[b] = int32_t(tiles.size());
      for (size_t i = 0; i < tiles.size(); ++i) p.blk_tiles[size_t(b) * p.blk_maxc + i] = tiles[i];
      for (int32_t s = 0; s < TS_QBLOCK && r0 + s < rows.size(); ++s) {
        const int32_t q = rows[r0 + s];
        p.blk_rows[size_t(b) * TS_QBLOCK + s] = q;
        for (int32_t e = p.cover_ptr[q]; e < p.cover_ptr[q + 1]; ++e)
          for (size_t i = 0; i < tiles.size(); ++i)
            if (p.cover_tile[e] == tiles[i])
              p.blk_w[(size_t(b) * p.blk_maxc + i) * TS_QBLOCK + s] = p.cover_w[e];
      }
    }
  }
  // halves of equal work; blocks are already ordered by decreasing windows,
  // so a class is a run of block indices
  std::vector<int32_t> ha, hb, cls;
  int64_t work_a = 0, work_b = 0;
  for (int32_t b0 = 0; b0 < p.nblk;) {
    int32_t b1 = b0;
    while (b1 < p.nblk && p.blk_nt[b1] == p.blk_nt[b0]) ++b1;
    const int32_t cnt = b1 - b0, w = p.blk_nt[b0];
    const int32_t ka = cnt / 2 + ((cnt & 1) && work_a <= work_b ? 1 : 0);
    cls.insert(cls.end(), {ka, int32_t(ha.size()), cnt - ka, int32_t(hb.size())});
    for (int32_t b = b0; b < b1; ++b) (b < b0 + ka ? ha : hb).push_back(b);
    work_a += int64_t(ka) * w;
    work_b += int64_t(cnt - ka) * w;
    b0 = b1;
  }
  p.blk_ncls = int32_t(cls.size() / 4);
  for (int32_t c = 0; c < p.blk_ncls; ++c) cls[4 * c + 3] += int32_t(ha.size());
  p.blk_order = ha;
  p.blk_order.insert(p.blk_order.end(), hb.begin(), hb.end());
  p.blk_cls = cls;
}

std::string build(const ts_tiling_desc& d, ts_plan& p) {
  if (d.ndim != 2 && d.ndim != 3) return "ndim must be 2 or 3";
  if (d.n_global != 1) return "n_global must be 1";
  if (d.blend != 0 && d.blend != 1) return "blend must be 0 (linear ramp) or 1 (hard stitching)";
  for (int a = 0; a < 3; ++a) {
    if (d.grid[a] < 1 || d.tile[a] < 1 || d.stride[a] < 1) return "grid, tile and stride must be >= 1";
  }
  if (d.ndim == 2 && (d.grid[0] != 1 || d.tile[0] != 1)) return "2D plans need grid[0] = tile[0] = 1";
  const int64_t nu = int64_t(d.grid[0]) * d.grid[1] * d.grid[2];
  if (nu >= (int64_t(1) << 31) / 2) return "grid too large";
  p.desc = d;
  for (int a = 0; a < 3; ++a) axis_starts(d.grid[a], d.tile[a], d.stride[a], p.axis_starts[a], p.ext[a]);
  if (p.ext[0] > 1023 || p.ext[1] > 1023 || p.ext[2] > 1023) return "tile extent must be < 1024";
  const int32_t T = d.grid[0], H = d.grid[1], W = d.grid[2];
  p.n_union = int32_t(nu);
  p.n = p.ext[0] * p.ext[1] * p.ext[2];
  p.n_tiles = int32_t(p.axis_starts[0].size() * p.axis_starts[1].size() * p.axis_starts[2].size());
  const int64_t nent = int64_t(p.n_tiles) * p.n;
  if (nent + p.n_tiles >= (int64_t(1) << 31)) return "too many tile tokens";
  (void)T;

  p.tile_start.clear();
  std::vector<int32_t> tidx;  // (it, ih, iw)
  for (size_t it = 0; it < p.axis_starts[0].size(); ++it)
    for (size_t ih = 0; ih < p.axis_starts[1].size(); ++ih)
      for (size_t iw = 0; iw < p.axis_starts[2].size(); ++iw) {
        p.tile_start.push_back(p.axis_starts[0][it]);
        p.tile_start.push_back(p.axis_starts[1][ih]);
        p.tile_start.push_back(p.axis_starts[2][iw]);
        tidx.push_back(int32_t(it));
        tidx.push_back(int32_t(ih));
        tidx.push_back(int32_t(iw));
      }

  p.local_pos.resize(p.n);
  for (int32_t a = 0, j = 0; a < p.ext[0]; ++a)
    for (int32_t b = 0; b < p.ext[1]; ++b)
      for (int32_t c = 0; c < p.ext[2]; ++c, ++j) p.local_pos[j] = a | (b << 10) | (c << 20);

  p.tile_rows.resize(size_t(nent));
  std::vector<double> ramp(static_cast<size_t>(nent));
  std::vector<int32_t> count(p.n_union, 0);
  for (int32_t t = 0; t < p.n_tiles; ++t) {
    const int32_t st = p.tile_start[3 * t], sh = p.tile_start[3 * t + 1], sw = p.tile_start[3 * t + 2];
    for (int32_t j = 0; j < p.n; ++j) {
      const int32_t u[3] = {p.local_pos[j] & 1023, (p.local_pos[j] >> 10) & 1023,
                            (p.local_pos[j] >> 20) & 1023};
      const int32_t row = ((st + u[0]) * H + (sh + u[1])) * W + (sw + u[2]);
      p.tile_rows[size_t(t) * p.n + j] = row;
      count[row] += 1;
      double r = 1.0;
      for (int a = 0; a < 3; ++a) r = r * axis_ramp(p.axis_starts[a], p.ext[a], size_t(tidx[3 * t + a]), u[a]);
      ramp[size_t(t) * p.n + j] = r;
    }
  }
  p.cover_ptr.assign(p.n_union + 1, 0);
  for (int32_t q = 0; q < p.n_union; ++q) {
    if (count[q] == 0) return "internal error: uncovered grid row";
    p.cover_ptr[q + 1] = p.cover_ptr[q] + count[q];
  }
  p.n_entries = p.cover_ptr[p.n_union];
  p.max_cover = 0;
  for (int32_t q = 0; q < p.n_union; ++q) p.max_cover = count[q] > p.max_cover ? count[q] : p.max_cover;
  p.cover_tile.assign(p.n_entries, 0);
  p.cover_local.assign(p.n_entries, 0);
  p.cover_w.assign(p.n_entries, 0.f);
  std::vector<int32_t> fill(p.cover_ptr.begin(), p.cover_ptr.end() - 1);
  for (int32_t t = 0; t < p.n_tiles; ++t)  // ascending tile order per row
    for (int32_t j = 0; j < p.n; ++j) {
      const int32_t row = p.tile_rows[size_t(t) * p.n + j];
      const int32_t e = fill[row]++;
      p.cover_tile[e] = t;
      p.cover_local[e] = j;
    }
  for (int32_t q = 0; q < p.n_union; ++q) {
    const int32_t e0 = p.cover_ptr[q], e1 = p.cover_ptr[q + 1];
    auto r_of = [&](int32_t e) { return ramp[size_t(p.cover_tile[e]) * p.n + p.cover_local[e]]; };
    if (d.blend == 1) {
      // hard stitching: weight 1 on the covering tile with the largest ramp
      // (ties to the lowest tile index, the first in the row's list)
      int32_t best = e0;
      for (int32_t e = e0 + 1; e < e1; ++e)
        if (r_of(e) > r_of(best)) best = e;
      for (int32_t e = e0; e < e1; ++e) p.cover_w[e] = e == best ? 1.f : 0.f;
      continue;
    }
    double total = 0.0;
    for (int32_t e = e0; e < e1; ++e) total = total + r_of(e);
    for (int32_t e = e0; e < e1; ++e) p.cover_w[e] = float(r_of(e) / total);
  }
  build_blocks(p);
  return "";
}

// Pairs per axis: contiguous chunks t, h, w; 3D h = w = floor(P/3) and t the
// rest, 2D h = floor(P/2) and w the rest.
void rope_pairs(int32_t ndim, int32_t head_dim, int32_t out[3]) {
  const int32_t P = head_dim / 2;
  if (ndim == 2) {
    out[0] = 0;
    out[1] = P / 2;
    out[2] = P - P / 2;
  } else {
    out[0] = P - 2 * (P / 3);
    out[1] = P / 3;
    out[2] = P / 3;
  }
}

void rope_local(const ts_plan& p, int32_t head_dim, float base, float* cos_out, float* sin_out) {
  int32_t pairs[3];
  rope_pairs(p.desc.ndim, head_dim, pairs);
  const int32_t P = head_dim / 2;
  for (int32_t j = 0; j < p.n; ++j)
    for (int32_t k = 0, a = 0, k0 = 0; k < P; ++k) {
      while (k >= k0 + pairs[a]) k0 += pairs[a++];
      const int32_t pos = (p.local_pos[j] >> (10 * a)) & 1023;
      const double ang = double(pos) * std::pow(double(base), double(-(k - k0)) / double(pairs[a]));
      cos_out[size_t(j) * P + k] = float(std::cos(ang));
      sin_out[size_t(j) * P + k] = float(std::sin(ang));
    }
}

// RoPE table over the whole grid: axis a's block holds, for every grid
// coordinate pos in [0, grid[a]) and every pair i of the axis, (cos, sin) of
// pos * base^(-i / pairs[a]) at tab[off[a] + 2*(pos*pairs[a] + i) + {0, 1}].
void rope_table_global(const ts_plan& p, int32_t head_dim, float base, std::vector<float>& tab, int32_t off[3]) {
  int32_t pairs[3];
  rope_pairs(p.desc.ndim, head_dim, pairs);
  int32_t total = 0;
  for (int a = 0; a < 3; ++a) {
    off[a] = total;
    total += 2 * pairs[a] * p.desc.grid[a];
  }
  tab.assign(size_t(total), 0.f);
  for (int a = 0; a < 3; ++a)
    for (int32_t i = 0; i < pairs[a]; ++i) {
      const double inv = std::pow(double(base), double(-i) / double(pairs[a]));
      for (int32_t pos = 0; pos < p.desc.grid[a]; ++pos) {
        const double ang = double(pos) * inv;
        tab[off[a] + 2 * (size_t(pos) * pairs[a] + i)] = float(std::cos(ang));
        tab[off[a] + 2 * (size_t(pos) * pairs[a] + i) + 1] = float(std::sin(ang));
      }
    }
}

}  // namespace tsplan
