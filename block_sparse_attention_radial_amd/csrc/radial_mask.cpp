// Host-side block-mask builder for Radial Attention.
//
// The rule, after "Radial Attention: A Breakthrough in Efficient Long Video Generation",
// How Radial Attention Works (the window shrinks with temporal distance, density halves
// when the distance doubles, and the mask is applied in 128x128 blocks), and the
// radial-attention-video SKILL.md page, Step 1 (frame-major token layout):
//
//     key allowed  <=>  dist(s_q, s_k) * 2^floor(log2(|f_q - f_k| + 1)) < W0
//
// with dist = |s_q - s_k|, or, on a frame stored as a grid of H rows of W columns
// (s = y * W + x; the same page's grid-distance helper), the Manhattan distance
// |y_q - y_k| + |x_q - x_k|. The 1-D rule is the grid with one row (W = S).
//
// The builder never looks at single elements. For a query frame f_q and a key frame
// f_k at band k = floor(log2(|f_q - f_k| + 1)), the largest allowed distance is
// r_k = floor((W0 - 1) / 2^k), because dist * 2^k < W0 <=> dist * 2^k <= W0 - 1
// (integers). A query block is cut into frame pieces; a piece is a run of in-frame
// positions, i.e. a partial first grid row [x_a, W) of row y_a, whole rows, and a
// partial last row [0, x_b] of row y_b (or one run [x_a, x_b] when y_a = y_b). From
// these, key row y_k is reached in at most two column runs: within distance t of a
// partial row [c0, c1] lie the columns [c0 - t, c1 + t] with t = r_k - |y_k - y|, and a
// whole row within distance r_k reaches every column. Each run is contiguous in token
// order, so it maps to a contiguous range of key blocks. Cost is O(nb * pieces * F * H)
// plus the blocks marked; with one row it is the 1-D interval sweep.
#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstring>
#include <vector>

#include "../../include/radial_attn.h"

namespace {

// floor(log2(x)) for x >= 1.
inline int floor_log2(uint32_t x) { return 31 - __builtin_clz(x); }

int32_t check_args(int32_t frames, int32_t grid_h, int32_t grid_w, int32_t w0, int32_t block) {
  if (frames <= 0 || grid_h <= 0 || grid_w <= 0 || w0 <= 0) return RADIAL_ERR_INVALID_ARG;
  if (block != RADIAL_BLOCK) return RADIAL_ERR_INVALID_ARG;
  if (static_cast<int64_t>(frames) * grid_h * grid_w > INT32_MAX) return RADIAL_ERR_TOO_LARGE;
  return RADIAL_OK;
}

// Calls emit(row, ascending_key_blocks) for every query block row, in order. Frames are
// grids of H rows of W columns (H = 1 for the 1-D rule).
template <typename Emit>
void sweep(int32_t frames, int32_t H, int32_t W, int32_t w0, Emit&& emit) {
  const int64_t S = static_cast<int64_t>(H) * W;
  const int64_t n = frames * S;
  const int32_t nb = static_cast<int32_t>((n + RADIAL_BLOCK - 1) / RADIAL_BLOCK);
  // The radius at each frame distance, tabulated once.
  std::vector<int64_t> radius(frames);
  for (int32_t d = 0; d < frames; ++d)
    radius[d] = (w0 - 1) >> floor_log2(static_cast<uint32_t>(d) + 1u);
  std::vector<uint8_t> hit(nb, 0);
  std::vector<int32_t> cols;
  cols.reserve(nb);
  int32_t lo_blk = nb, hi_blk = -1;
  // Marks the key blocks of columns [x0, x1] (clipped to the row) of token row `row0`.
  auto mark = [&](int64_t row0, int64_t x0, int64_t x1) {
    x0 = std::max<int64_t>(x0, 0);
    x1 = std::min<int64_t>(x1, W - 1);
    if (x0 > x1) return;
    const int32_t b0 = static_cast<int32_t>((row0 + x0) / RADIAL_BLOCK);
    const int32_t b1 = static_cast<int32_t>((row0 + x1) / RADIAL_BLOCK);
    for (int32_t kb = b0; kb <= b1; ++kb) hit[kb] = 1;
    lo_blk = std::min(lo_blk, b0);
    hi_blk = std::max(hi_blk, b1);
  };
  for (int32_t row = 0; row < nb; ++row) {
    const int64_t t0 = static_cast<int64_t>(row) * RADIAL_BLOCK;
    const int64_t t1 = std::min<int64_t>(n, t0 + RADIAL_BLOCK);  // exclusive
    lo_blk = nb;
    hi_blk = -1;
    for (int64_t t = t0; t < t1;) {
      const int64_t fq = t / S;
      const int64_t piece_end = std::min<int64_t>(t1, (fq + 1) * S);
      const int64_t a = t - fq * S, b = piece_end - 1 - fq * S;
      const int64_t ya = a / W, xa = a % W, yb = b / W, xb = b % W;
      for (int64_t fk = 0; fk < frames; ++fk) {
        const int64_t r = radius[fq > fk ? fq - fk : fk - fq];
        const int64_t y_lo = std::max<int64_t>(0, ya - r);
        const int64_t y_hi = std::min<int64_t>(H - 1, yb + r);
        for (int64_t yk = y_lo; yk <= y_hi; ++yk) {
          const int64_t row0 = fk * S + yk * W;
          const int64_t ta = r - (yk > ya ? yk - ya : ya - yk);
          const int64_t tb = r - (yk > yb ? yk - yb : yb - yk);
          if (ya == yb) {
            if (ta >= 0) mark(row0, xa - ta, xb + ta);
            continue;
          }
          if (yb - ya >= 2) {  // whole rows ya + 1 .. yb - 1
            const int64_t dm = yk <= ya ? ya + 1 - yk : (yk >= yb ? yk - yb + 1 : 0);
            if (dm <= r) {
              mark(row0, 0, W - 1);
              continue;
            }
          }
          if (ta >= 0) mark(row0, xa - ta, W - 1);
          if (tb >= 0) mark(row0, 0, xb + tb);
        }
      }
      t = piece_end;
    }
    cols.clear();
    for (int32_t kb = lo_blk; kb <= hi_blk; ++kb) {
      if (hit[kb]) {
        cols.push_back(kb);
        hit[kb] = 0;
      }
    }
    emit(row, cols);
  }
}

int32_t dims(int32_t frames, int32_t grid_h, int32_t grid_w, int32_t w0, int32_t block,
             int32_t* nb_out, int64_t* nnz_out) {
  if (!nb_out || !nnz_out) return RADIAL_ERR_INVALID_ARG;
  const int32_t st = check_args(frames, grid_h, grid_w, w0, block);
  if (st != RADIAL_OK) return st;
  int64_t nnz = 0;
  int32_t rows = 0;
  sweep(frames, grid_h, grid_w, w0, [&](int32_t, const std::vector<int32_t>& cols) {
    nnz += static_cast<int64_t>(cols.size());
    ++rows;
  });
  if (nnz > INT32_MAX) return RADIAL_ERR_TOO_LARGE;
  *nb_out = rows;
  *nnz_out = nnz;
  return RADIAL_OK;
}

int32_t build(int32_t frames, int32_t grid_h, int32_t grid_w, int32_t w0, int32_t block,
              int32_t* row_ptr, int32_t* col_idx, int64_t nnz_capacity) {
  if (!row_ptr || !col_idx || nnz_capacity < 0) return RADIAL_ERR_INVALID_ARG;
  const int32_t st = check_args(frames, grid_h, grid_w, w0, block);
  if (st != RADIAL_OK) return st;
  int64_t nnz = 0;
  bool overflow = false;
  row_ptr[0] = 0;
  sweep(frames, grid_h, grid_w, w0, [&](int32_t row, const std::vector<int32_t>& cols) {
    const int64_t end = nnz + static_cast<int64_t>(cols.size());
    if (end > nnz_capacity || end > INT32_MAX) overflow = true;
    if (!overflow) std::memcpy(col_idx + nnz, cols.data(), cols.size() * sizeof(int32_t));
    nnz = end;
    row_ptr[row + 1] = static_cast<int32_t>(std::min<int64_t>(nnz, INT32_MAX));
  });
  if (nnz > INT32_MAX) return RADIAL_ERR_TOO_LARGE;
  if (overflow) return RADIAL_ERR_CAPACITY;
  return RADIAL_OK;
}

}  // namespace

extern "C" int32_t radial_mask_dims(int32_t frames, int32_t tokens_per_frame, int32_t w0,
                                    int32_t block, int32_t* nb_out, int64_t* nnz_out) {
  return dims(frames, 1, tokens_per_frame, w0, block, nb_out, nnz_out);
}

extern "C" int32_t radial_build_mask(int32_t frames, int32_t tokens_per_frame, int32_t w0,
                                     int32_t block, int32_t* row_ptr, int32_t* col_idx,
                                     int64_t nnz_capacity) {
  return build(frames, 1, tokens_per_frame, w0, block, row_ptr, col_idx, nnz_capacity);
}

extern "C" int32_t radial_mask_dims_grid(int32_t frames, int32_t grid_h, int32_t grid_w,
                                         int32_t w0, int32_t block, int32_t* nb_out,
                                         int64_t* nnz_out) {
  return dims(frames, grid_h, grid_w, w0, block, nb_out, nnz_out);
}

extern "C" int32_t radial_build_mask_grid(int32_t frames, int32_t grid_h, int32_t grid_w,
                                          int32_t w0, int32_t block, int32_t* row_ptr,
                                          int32_t* col_idx, int64_t nnz_capacity) {
  return build(frames, grid_h, grid_w, w0, block, row_ptr, col_idx, nnz_capacity);
}

extern "C" const char* radial_error_string(int32_t code) {
  switch (code) {
    case RADIAL_OK: return "ok";
    case RADIAL_ERR_INVALID_ARG: return "invalid argument";
    case RADIAL_ERR_UNSUPPORTED_HEAD_DIM: return "unsupported head_dim (64 or 128)";
    case RADIAL_ERR_CAPACITY: return "col_idx capacity smaller than the active-block count";
    case RADIAL_ERR_SHAPE_MISMATCH: return "nb does not equal ceil(seqlen / 128)";
    case RADIAL_ERR_MISALIGNED: return "pointer or stride not 16-byte aligned";
    case RADIAL_ERR_TOO_LARGE: return "size past the int32 index range";
    case RADIAL_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown error code";
  }
}

// The transposed block mask: for key block c, the query blocks whose rows list it,
// ascending. A counting sort over the columns; entries outside [0, nb) are dropped.
extern "C" int32_t radial_transpose_mask(int32_t nb, const int32_t* row_ptr,
                                         const int32_t* col_idx, int32_t* col_ptr,
                                         int32_t* row_idx) {
  if (nb <= 0 || !row_ptr || !col_ptr || !row_idx) return RADIAL_ERR_INVALID_ARG;
  if (row_ptr[0] != 0) return RADIAL_ERR_INVALID_ARG;
  for (int32_t r = 0; r < nb; ++r)
    if (row_ptr[r + 1] < row_ptr[r]) return RADIAL_ERR_INVALID_ARG;
  if (row_ptr[nb] > 0 && !col_idx) return RADIAL_ERR_INVALID_ARG;
  std::vector<int32_t> count(static_cast<size_t>(nb) + 1, 0);
  for (int32_t i = 0; i < row_ptr[nb]; ++i) {
    const int32_t c = col_idx[i];
    if (c >= 0 && c < nb) ++count[c + 1];
  }
  col_ptr[0] = 0;
  for (int32_t c = 0; c < nb; ++c) col_ptr[c + 1] = col_ptr[c] + count[c + 1];
  std::vector<int32_t> fill(col_ptr, col_ptr + nb);
  for (int32_t r = 0; r < nb; ++r)
    for (int32_t i = row_ptr[r]; i < row_ptr[r + 1]; ++i) {
      const int32_t c = col_idx[i];
      if (c >= 0 && c < nb) row_idx[fill[c]++] = r;
    }
  return RADIAL_OK;
}
