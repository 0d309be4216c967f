// Host-side choice of which query-block rows share a workgroup.
//
// The forward kernel gives each workgroup two query-block rows and walks the union of
// their key-block lists: a K/V tile copied once serves both rows, and a tile in only
// one row leaves the other row's waves idle for that step. So the pairing decides how
// much of the work is shared. It does not change any result: each row's output depends
// only on its own key blocks, taken in ascending order.
//
// Rows with much in common are neighbours in the sequence (the same frame, spatially
// close), and rows at the same spatial position one or two frames apart. The radial
// mask narrows the spatial window as the frame distance grows ("Radial Attention: A
// Breakthrough in Efficient Long Video Generation", How Radial Attention Works), so for
// distant key frames two rows 128 tokens apart in one frame see different narrow
// windows, while two rows one frame apart see nearly the same windows. The builder
// scores candidate partners at row offsets 1, 2, 3 and, given the frame length, about
// one and two frames, by the number of key blocks they share. It then matches greedily,
// best score first, and orders the pairs for the kernel's XCD-wise work mapping.
#include <algorithm>
#include <climits>
#include <cstdint>
#include <vector>

#include "../../include/radial_attn.h"

namespace {

// Number of common entries of two ascending runs.
int64_t common(const int32_t* a, const int32_t* a_end, const int32_t* b, const int32_t* b_end) {
  int64_t c = 0;
  while (a != a_end && b != b_end) {
    if (*a < *b) {
      ++a;
    } else if (*b < *a) {
      ++b;
    } else {
      ++c;
      ++a;
      ++b;
    }
  }
  return c;
}

struct Edge {
  int64_t shared;
  int32_t offset, row;
};

}  // namespace

extern "C" int32_t radial_build_pairs(int32_t nb, const int32_t* row_ptr, const int32_t* col_idx,
                                      int32_t tokens_per_frame, int32_t* pairs,
                                      int32_t* npairs_out) {
  if (nb <= 0 || tokens_per_frame < 0 || !row_ptr || !pairs || !npairs_out)
    return RADIAL_ERR_INVALID_ARG;
  if (row_ptr[0] != 0) return RADIAL_ERR_INVALID_ARG;
  for (int32_t r = 0; r < nb; ++r)
    if (row_ptr[r + 1] < row_ptr[r]) return RADIAL_ERR_INVALID_ARG;
  const int64_t nnz = row_ptr[nb];
  if (nnz > 0 && !col_idx) return RADIAL_ERR_INVALID_ARG;

  // Candidate offsets: 1, 2, 3 and, with a frame length, round(k * blocks per frame) + d
  // for k = 1, 2 and d = -1, 0, 1.
  std::vector<int32_t> offsets = {1, 2, 3};
  if (tokens_per_frame > 0) {
    for (int k = 1; k <= 2; ++k) {
      const int64_t base = (2LL * k * tokens_per_frame + RADIAL_BLOCK) / (2LL * RADIAL_BLOCK);
      for (int64_t d = -1; d <= 1; ++d)
        if (base + d >= 1 && base + d < nb) offsets.push_back(static_cast<int32_t>(base + d));
    }
  }
  std::sort(offsets.begin(), offsets.end());
  offsets.erase(std::unique(offsets.begin(), offsets.end()), offsets.end());

  std::vector<uint8_t> used(static_cast<size_t>(nb), 0);
  std::vector<int32_t> out;
  out.reserve(2 * static_cast<size_t>(nb));
  // The scores cost one merge per candidate pair, about 2 * offsets * nnz steps. Past
  // 2^28 steps (dense masks of many thousand blocks, where neighbours share everything
  // anyway) the adjacent pairing is kept.
  const bool greedy = 2 * static_cast<int64_t>(offsets.size()) * nnz <= (int64_t{1} << 28);
  if (greedy) {
    std::vector<Edge> edges;
    edges.reserve(offsets.size() * static_cast<size_t>(nb));
    for (const int32_t d : offsets)
      for (int32_t q = 0; q + d < nb; ++q)
        edges.push_back({common(col_idx + row_ptr[q], col_idx + row_ptr[q + 1],
                                col_idx + row_ptr[q + d], col_idx + row_ptr[q + d + 1]),
                         d, q});
    // Best score first; ties go to the nearer partner, then the lower row, so the
    // result is deterministic.
    std::sort(edges.begin(), edges.end(), [](const Edge& x, const Edge& y) {
      if (x.shared != y.shared) return x.shared > y.shared;
      if (x.offset != y.offset) return x.offset < y.offset;
      return x.row < y.row;
    });
    for (const Edge& e : edges) {
      const int32_t a = e.row, b = e.row + e.offset;
      if (used[a] || used[b]) continue;
      used[a] = used[b] = 1;
      out.push_back(a);
      out.push_back(b);
    }
  }
  // Rows left over are paired in ascending order; an odd one out runs alone.
  int32_t waiting = -1;
  for (int32_t r = 0; r < nb; ++r) {
    if (used[r]) continue;
    if (waiting < 0) {
      waiting = r;
    } else {
      out.push_back(waiting);
      out.push_back(r);
      waiting = -1;
    }
  }
  if (waiting >= 0) {
    out.push_back(waiting);
    out.push_back(-1);
  }
  // The order of the table is the order the kernel takes the pairs in: each XCD takes a
  // head's pairs in contiguous runs of the table (the whole table, or one of 2, 4 or 8
  // runs when several XCDs share a head). Pairs are ordered
  // by their union length in bands of kBand key blocks, longest band first, and by
  // first row within a band. A run then holds pairs of nearly equal length that are
  // close in the sequence: the workgroups of an XCD start them together, walk their
  // lists in step, and so read the same K/V tiles at about the same time, which keeps
  // those tiles in the XCD's L2 (measured: 20% less traffic past L2 at Wan's shape, and
  // 1 to 3% less time on the three video workloads than by first row alone).
  constexpr int64_t kBand = 16;
  const int32_t np = static_cast<int32_t>(out.size() / 2);
  std::vector<int64_t> band(static_cast<size_t>(np));
  for (int32_t i = 0; i < np; ++i) {
    const int32_t a = out[2 * i], b = out[2 * i + 1];
    int64_t len = row_ptr[a + 1] - row_ptr[a];
    if (b >= 0)
      len += (row_ptr[b + 1] - row_ptr[b]) - common(col_idx + row_ptr[a], col_idx + row_ptr[a + 1],
                                                    col_idx + row_ptr[b], col_idx + row_ptr[b + 1]);
    band[i] = len / kBand;
  }
  std::vector<int32_t> idx(static_cast<size_t>(np));
  for (int32_t i = 0; i < np; ++i) idx[i] = i;
  std::sort(idx.begin(), idx.end(), [&](int32_t x, int32_t y) {
    if (band[x] != band[y]) return band[x] > band[y];
    return out[2 * x] < out[2 * y];
  });
  for (int32_t i = 0; i < np; ++i) {
    pairs[2 * i] = out[2 * idx[i]];
    pairs[2 * i + 1] = out[2 * idx[i] + 1];
  }
  *npairs_out = np;
  return RADIAL_OK;
}
