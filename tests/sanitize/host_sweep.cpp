// Host-side sweep of libradial's C ABI for a build with AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_host_sanitize.py builds and runs it; no GPU).
//
// Every buffer handed to the library is a heap vector of exactly the size the header
// documents, so a write or read past it is caught. It covers: the 1-D and grid mask
// builders on a seeded sweep of shapes and on the 4x-long video (84 frames of 1560
// tokens), their capacity errors (one entry short), the pair-table builder, the mask
// transpose (also on a random non-symmetric mask with out-of-range columns), and the
// argument checks of the attention entry points, which return before any HIP call.
// With no GPU, a call that passes its checks fails at its first HIP call and must say
// so with RADIAL_ERR_HIP.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "../../include/radial_attn.h"

namespace {

int g_failures = 0;

void expect(bool ok, const char* what, int a = 0, int b = 0, int c = 0) {
  if (!ok) {
    std::printf("FAIL %s (%d, %d, %d)\n", what, a, b, c);
    ++g_failures;
  }
}

// A mask's CSR form: row_ptr starts at 0, never decreases, ends at nnz, and each row is
// strictly ascending inside [0, nb).
bool valid_csr(int32_t nb, const std::vector<int32_t>& rp, const std::vector<int32_t>& ci) {
  if (rp[0] != 0 || rp[nb] != static_cast<int32_t>(ci.size())) return false;
  for (int32_t r = 0; r < nb; ++r) {
    if (rp[r + 1] < rp[r]) return false;
    for (int32_t i = rp[r]; i < rp[r + 1]; ++i) {
      if (ci[i] < 0 || ci[i] >= nb) return false;
      if (i > rp[r] && ci[i] <= ci[i - 1]) return false;
    }
  }
  return true;
}

// Builds one mask (grid_h = 0: the 1-D builder) in exact-size buffers, checks it, and
// runs the pair table and the transpose on it. Returns the block count.
int64_t one_mask(int32_t frames, int32_t grid_h, int32_t grid_w, int32_t w0) {
  const int32_t s = grid_h == 0 ? grid_w : grid_h * grid_w;
  int32_t nb = -1;
  int64_t nnz = -1;
  const int32_t rc = grid_h == 0 ? radial_mask_dims(frames, s, w0, 128, &nb, &nnz)
                                 : radial_mask_dims_grid(frames, grid_h, grid_w, w0, 128, &nb, &nnz);
  expect(rc == RADIAL_OK, "dims", frames, s, w0);
  if (rc != RADIAL_OK) return 0;
  std::vector<int32_t> rp(nb + 1), ci(nnz);
  // One entry short: CAPACITY, and nothing written past the shorter buffer (which keeps
  // one entry when the capacity is 0, as a null col_idx is an argument error).
  if (nnz > 0) {
    std::vector<int32_t> rp_short(nb + 1), ci_short(nnz > 1 ? nnz - 1 : 1);
    const int32_t e = grid_h == 0
        ? radial_build_mask(frames, s, w0, 128, rp_short.data(), ci_short.data(), nnz - 1)
        : radial_build_mask_grid(frames, grid_h, grid_w, w0, 128, rp_short.data(),
                                 ci_short.data(), nnz - 1);
    expect(e == RADIAL_ERR_CAPACITY, "capacity", frames, s, w0);
  }
  const int32_t b = grid_h == 0
      ? radial_build_mask(frames, s, w0, 128, rp.data(), ci.data(), nnz)
      : radial_build_mask_grid(frames, grid_h, grid_w, w0, 128, rp.data(), ci.data(), nnz);
  expect(b == RADIAL_OK && valid_csr(nb, rp, ci), "build", frames, s, w0);
  // Pairs: 2 * nb entries; every row exactly once.
  std::vector<int32_t> pairs(2 * static_cast<size_t>(nb));
  int32_t np = -1;
  expect(radial_build_pairs(nb, rp.data(), ci.data(), s, pairs.data(), &np) == RADIAL_OK,
         "pairs", frames, s, w0);
  std::vector<int> seen(nb, 0);
  for (int32_t i = 0; i < 2 * np; ++i)
    if (pairs[i] >= 0 && pairs[i] < nb) ++seen[pairs[i]];
  for (int32_t r = 0; r < nb; ++r) expect(seen[r] == 1, "pair rows", frames, s, r);
  // Transpose: exact sizes; a radial mask is its own transpose.
  std::vector<int32_t> cp(nb + 1), ri(nnz);
  expect(radial_transpose_mask(nb, rp.data(), ci.data(), cp.data(), ri.data()) == RADIAL_OK,
         "transpose", frames, s, w0);
  expect(cp == rp && ri == ci, "symmetric", frames, s, w0);
  return nnz;
}

void random_transpose(std::mt19937& rng) {
  const int32_t nb = 1 + static_cast<int32_t>(rng() % 40);
  std::vector<int32_t> rp(nb + 1, 0), ci;
  for (int32_t r = 0; r < nb; ++r) {
    const int32_t len = static_cast<int32_t>(rng() % 6);
    for (int32_t i = 0; i < len; ++i) ci.push_back(static_cast<int32_t>(rng() % (nb + 4)) - 2);
    rp[r + 1] = static_cast<int32_t>(ci.size());
  }
  std::vector<int32_t> cp(nb + 1), ri(ci.size() > 0 ? ci.size() : 1);
  const int32_t* cptr = ci.empty() ? nullptr : ci.data();
  expect(radial_transpose_mask(nb, rp.data(), cptr, cp.data(), ri.data()) == RADIAL_OK,
         "random transpose", nb);
  int64_t kept = 0;
  for (int32_t c : ci) kept += (c >= 0 && c < nb);
  expect(cp[nb] == kept, "random transpose count", nb);
  std::vector<int32_t> pairs(2 * static_cast<size_t>(nb));
  int32_t np = -1;
  expect(radial_build_pairs(nb, rp.data(), cptr, 0, pairs.data(), &np) == RADIAL_OK,
         "random pairs", nb);
}

// Argument checks of the attention entry points: every call below is invalid and must
// be refused on the host; a valid one, with no GPU, must fail with RADIAL_ERR_HIP.
void attention_checks() {
  alignas(16) static char buf[4096];
  void* p = buf;
  void* odd = buf + 8;
  float* lse = reinterpret_cast<float*>(buf);
  const int32_t* ip = reinterpret_cast<const int32_t*>(buf);
  const int32_t tokens[2] = {1000, 700};
  const int32_t frames[2] = {4, 3};
  // radial_attn_fwd
  expect(radial_attn_fwd(nullptr, p, p, p, nullptr, ip, ip, 8, nullptr, 0, 0.1f, 0, 0, 0, 1, 1,
                         1000, 128, 0, 0, 128, nullptr) == RADIAL_ERR_INVALID_ARG, "fwd null");
  expect(radial_attn_fwd(p, p, p, p, nullptr, ip, ip, 8, nullptr, 0, -1.f, 0, 0, 0, 1, 1, 1000,
                         128, 0, 0, 128, nullptr) == RADIAL_ERR_INVALID_ARG, "fwd scale");
  expect(radial_attn_fwd(p, p, p, p, nullptr, ip, ip, 8, nullptr, 0, 0.1f, 0, 0, 0, 1, 1, 1000,
                         96, 0, 0, 128, nullptr) == RADIAL_ERR_UNSUPPORTED_HEAD_DIM, "fwd D");
  expect(radial_attn_fwd(p, p, p, p, nullptr, ip, ip, 9, nullptr, 0, 0.1f, 0, 0, 0, 1, 1, 1000,
                         128, 0, 0, 128, nullptr) == RADIAL_ERR_SHAPE_MISMATCH, "fwd nb");
  expect(radial_attn_fwd(odd, p, p, p, nullptr, ip, ip, 8, nullptr, 0, 0.1f, 0, 0, 0, 1, 1,
                         1000, 128, 0, 0, 128, nullptr) == RADIAL_ERR_MISALIGNED, "fwd align");
  expect(radial_attn_fwd(p, p, p, p, nullptr, ip, ip, 8, nullptr, 0, 0.1f, 100, 5, 0, 1, 1,
                         1000, 128, 0, 0, 128, nullptr) == RADIAL_ERR_INVALID_ARG, "fwd element");
  expect(radial_attn_fwd(p, p, p, p, nullptr, ip, ip, 8, ip, 3, 0.1f, 0, 0, 0, 1, 1, 1000, 128,
                         0, 0, 128, nullptr) == RADIAL_ERR_INVALID_ARG, "fwd npairs");
  expect(radial_attn_fwd(p, p, p, p, lse, ip, ip, 8, nullptr, 0, 0.1f, 0, 0, 0, 1, 1, 1000, 128,
                         0, 0, 128, nullptr) == RADIAL_ERR_HIP, "fwd no GPU");
  // radial_attn_fwd_rule
  expect(radial_attn_fwd_rule(p, p, p, p, nullptr, 0, 100, 0, 10, 0, nullptr, 0, 0.1f, 1, 1, 128,
                              0, 0, 128, nullptr) == RADIAL_ERR_INVALID_ARG, "rule frames");
  expect(radial_attn_fwd_rule(p, p, p, p, nullptr, 4, 100, 7, 10, 0, nullptr, 0, 0.1f, 1, 1, 128,
                              0, 0, 128, nullptr) == RADIAL_ERR_INVALID_ARG, "rule grid");
  expect(radial_attn_fwd_rule(p, p, p, p, nullptr, 200000, 100, 0, 10, 0, nullptr, 0, 0.1f, 1, 1,
                              128, 0, 0, 128, nullptr) == RADIAL_ERR_TOO_LARGE, "rule size");
  expect(radial_attn_fwd_rule(p, p, p, p, nullptr, 4, 100, 0, 10, 0, nullptr, 0, 0.1f, 1, 1, 128,
                              0, 0, 128, nullptr) == RADIAL_ERR_HIP, "rule no GPU");
  // radial_attn_fwd_varlen and its rule form
  expect(radial_attn_fwd_varlen(p, p, p, p, nullptr, nullptr, 2, ip, ip, nullptr, nullptr, 0.1f,
                                0, 0, 0, 1, 128, 128, 128, nullptr) == RADIAL_ERR_INVALID_ARG,
         "varlen null");
  expect(radial_attn_fwd_varlen(p, p, p, p, nullptr, tokens, 65, ip, ip, nullptr, nullptr, 0.1f,
                                0, 0, 0, 1, 128, 128, 128, nullptr) == RADIAL_ERR_TOO_LARGE,
         "varlen batch");
  expect(radial_attn_fwd_varlen(p, p, p, p, nullptr, tokens, 2, ip, ip, ip, nullptr, 0.1f, 0, 0,
                                0, 1, 128, 128, 128, nullptr) == RADIAL_ERR_INVALID_ARG,
         "varlen pairs");
  expect(radial_attn_fwd_varlen(p, p, p, p, nullptr, tokens, 2, ip, ip, nullptr, nullptr, 0.1f,
                                0, 0, 0, 1, 128, 128, 128, nullptr) == RADIAL_ERR_HIP,
         "varlen no GPU");
  expect(radial_attn_fwd_varlen_rule(p, p, p, p, nullptr, frames, 2, 0, 0, 10, 0, nullptr,
                                     nullptr, 0.1f, 1, 128, 128, 128, nullptr) ==
             RADIAL_ERR_INVALID_ARG, "varlen rule frame");
  expect(radial_attn_fwd_varlen_rule(p, p, p, p, nullptr, frames, 2, 250, 0, 10, 0, nullptr,
                                     nullptr, 0.1f, 1, 128, 128, 128, nullptr) == RADIAL_ERR_HIP,
         "varlen rule no GPU");
  // radial_attn_bwd and its varlen form
  expect(radial_attn_bwd(p, p, p, p, p, lse, p, p, p, nullptr, ip, ip, ip, ip, 8, 0.1f, 0, 0, 0,
                         1, 1, 1000, 128, 0, 0, 128, nullptr) == RADIAL_ERR_INVALID_ARG,
         "bwd null delta");
  expect(radial_attn_bwd(p, p, p, p, p, lse + 1, p, p, p, lse, ip, ip, ip, ip, 8, 0.1f, 0, 0, 0,
                         1, 1, 1000, 128, 0, 0, 128, nullptr) == RADIAL_ERR_HIP,
         "bwd no GPU");
  expect(radial_attn_bwd(p, p, p, p, p, lse, p, p, p, lse, ip, ip, ip, ip, 8, 0.1f, 0, 0, 0, 1, 1,
                         1000, 64, 0, 0, 68, nullptr) == RADIAL_ERR_MISALIGNED, "bwd stride");
  expect(radial_attn_bwd_varlen(p, p, p, p, p, lse, p, p, p, lse, tokens, 0, ip, ip, ip, ip, 0.1f,
                                0, 0, 0, 1, 128, 128, 128, nullptr) == RADIAL_ERR_INVALID_ARG,
         "bwd varlen batch");
  expect(radial_attn_bwd_varlen(p, p, p, p, p, lse, p, p, p, lse, tokens, 2, ip, ip, ip, ip, 0.1f,
                                0, 0, 0, 1, 128, 128, 128, nullptr) == RADIAL_ERR_HIP,
         "bwd varlen no GPU");
  // radial_attn_bwd_noalloc: a shape past its static workspace, then a valid one.
  expect(radial_attn_bwd_noalloc(p, p, p, p, p, lse, p, p, p, ip, ip, ip, ip, 2048, 0.1f, 0, 0,
                                 0, 1, 33, 1 << 18, 128, 0, 0, 128, nullptr) ==
             RADIAL_ERR_TOO_LARGE, "bwd noalloc size");
  expect(radial_attn_bwd_noalloc(p, p, p, p, p, lse, p, p, p, nullptr, ip, ip, ip, 8, 0.1f, 0, 0,
                                 0, 1, 1, 1000, 128, 0, 0, 128, nullptr) ==
             RADIAL_ERR_INVALID_ARG, "bwd noalloc null");
  expect(radial_attn_bwd_noalloc(p, p, p, p, p, lse, p, p, p, ip, ip, ip, ip, 8, 0.1f, 0, 0, 0, 1,
                                 1, 1000, 128, 0, 0, 128, nullptr) == RADIAL_ERR_HIP,
         "bwd noalloc no GPU");
  // The element table and its entry points.
  int64_t bytes = -1;
  expect(radial_element_table_bytes(3, &bytes) == RADIAL_OK && bytes == 3 * 2048, "table bytes");
  expect(radial_element_table_bytes(-1, &bytes) == RADIAL_ERR_INVALID_ARG, "table bytes < 0");
  expect(radial_build_element_table(ip, ip, 8, 30, 0, 0, 0, p, 30 * 2048, nullptr) ==
             RADIAL_ERR_INVALID_ARG, "table no element");
  expect(radial_build_element_table(ip, ip, 8, 30, 1000, 50, 0, p, 30 * 2048 - 1, nullptr) ==
             RADIAL_ERR_CAPACITY, "table capacity");
  expect(radial_build_element_table(ip, ip, 8, 30, 1000, 50, 0, odd, 30 * 2048, nullptr) ==
             RADIAL_ERR_MISALIGNED, "table align");
  expect(radial_build_element_table(ip, ip, 8, 0, 1000, 50, 0, p, 0, nullptr) == RADIAL_OK,
         "table empty");
  expect(radial_build_element_table(ip, ip, 8, 30, 1000, 50, 0, p, 30 * 2048, nullptr) ==
             RADIAL_ERR_HIP, "table no GPU");
  expect(radial_attn_fwd_element_table(p, p, p, p, nullptr, ip, ip, 8, nullptr, 0, 0.1f, nullptr,
                                       1, 1, 1000, 128, 0, 0, 128, nullptr) ==
             RADIAL_ERR_INVALID_ARG, "fwd table null");
  expect(radial_attn_fwd_element_table(p, p, p, p, nullptr, ip, ip, 8, nullptr, 0, 0.1f, odd, 1,
                                       1, 1000, 128, 0, 0, 128, nullptr) ==
             RADIAL_ERR_MISALIGNED, "fwd table align");
  expect(radial_attn_fwd_element_table(p, p, p, p, lse, ip, ip, 8, nullptr, 0, 0.1f, p, 1, 1,
                                       1000, 128, 0, 0, 128, nullptr) == RADIAL_ERR_HIP,
         "fwd table no GPU");
  expect(radial_attn_bwd_element_table(p, p, p, p, p, lse, p, p, p, lse, ip, ip, ip, ip, 8, 0.1f,
                                       nullptr, 1, 1, 1000, 128, 0, 0, 128, nullptr) ==
             RADIAL_ERR_INVALID_ARG, "bwd table null");
  expect(radial_attn_bwd_element_table(p, p, p, p, p, lse, p, p, p, lse, ip, ip, ip, ip, 8, 0.1f,
                                       p, 1, 1, 1000, 128, 0, 0, 128, nullptr) == RADIAL_ERR_HIP,
         "bwd table no GPU");
  expect(radial_attn_fwd_varlen_element_table(p, p, p, p, nullptr, tokens, 2, ip, ip, nullptr,
                                              nullptr, 0.1f, nullptr, 1, 128, 128, 128,
                                              nullptr) == RADIAL_ERR_INVALID_ARG,
         "varlen table null");
  expect(radial_attn_fwd_varlen_element_table(p, p, p, p, nullptr, tokens, 2, ip, ip, nullptr,
                                              nullptr, 0.1f, p, 1, 128, 128, 128, nullptr) ==
             RADIAL_ERR_HIP, "varlen table no GPU");
  expect(radial_attn_bwd_varlen_element_table(p, p, p, p, p, lse, p, p, p, lse, tokens, 2, ip,
                                              ip, ip, ip, 0.1f, odd, 1, 128, 128, 128,
                                              nullptr) == RADIAL_ERR_MISALIGNED,
         "bwd varlen table align");
  expect(radial_attn_bwd_varlen_element_table(p, p, p, p, p, lse, p, p, p, lse, tokens, 2, ip,
                                              ip, ip, ip, 0.1f, p, 1, 128, 128, 128, nullptr) ==
             RADIAL_ERR_HIP, "bwd varlen table no GPU");
  for (int32_t code = -8; code <= 1; ++code) expect(radial_error_string(code) != nullptr, "text");
}

}  // namespace

int main() {
  std::mt19937 rng(2024);
  int cases = 0;
  for (int i = 0; i < 300; ++i) {
    const int32_t frames = 1 + static_cast<int32_t>(rng() % 12);
    const bool grid = rng() % 2;
    const int32_t gw = 1 + static_cast<int32_t>(rng() % 60);
    const int32_t gh = 1 + static_cast<int32_t>(rng() % 20);
    const int32_t s = grid ? gw * gh : 1 + static_cast<int32_t>(rng() % 700);
    const int32_t w0 = 1 + static_cast<int32_t>(rng() % (2 * s + 2));
    one_mask(frames, grid ? gh : 0, grid ? gw : s, w0);
    ++cases;
  }
  // Edge windows, frames shorter and longer than a block, and the 4x-long video.
  const int32_t edges[][3] = {{1, 1, 1}, {1, 129, 1}, {6, 1000, 100}, {21, 1560, 1560},
                              {5, 300, 2147483647}, {3, 127, 500}, {84, 1560, 1560}};
  for (const auto& e : edges) {
    one_mask(e[0], 0, e[1], e[2]);
    ++cases;
  }
  one_mask(21, 30, 52, 81);  // the Wan grid
  ++cases;
  for (int i = 0; i < 100; ++i) {
    random_transpose(rng);
    ++cases;
  }
  // Size-query errors.
  int32_t nb;
  int64_t nnz;
  expect(radial_mask_dims(0, 10, 10, 128, &nb, &nnz) == RADIAL_ERR_INVALID_ARG, "dims frames");
  expect(radial_mask_dims(4, 10, 10, 64, &nb, &nnz) == RADIAL_ERR_INVALID_ARG, "dims block");
  expect(radial_mask_dims(4, 10, 10, 128, nullptr, &nnz) == RADIAL_ERR_INVALID_ARG, "dims out");
  expect(radial_mask_dims(100000, 100000, 10, 128, &nb, &nnz) == RADIAL_ERR_TOO_LARGE, "dims big");
  attention_checks();
  if (g_failures) {
    std::printf("%d failures\n", g_failures);
    return 1;
  }
  std::printf("OK %d cases\n", cases);
  return 0;
}
