// Device helpers shared by the forward and backward kernels of Radial Attention on
// gfx950 (CDNA4): vector types, tile geometry and LDS bank swizzle, raw buffer
// descriptors, LDS-DMA tile copies and their waits, and the padding and element masks
// of a score tile in MFMA accumulator layout. Included by the kernel sources only.
#pragma once

#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBlock = 128;  // rows and keys of a block
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Fourth dword of a raw gfx9 buffer descriptor: 32-bit data format, no stride/swizzle.
constexpr int kBufferFlags = 0x00020000;

template <int D>
struct Tile {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;               // 16-byte chunks per row
  static constexpr int kBytes = kBlock * kRowBytes;   // one K or V tile
  static constexpr int kCopiesPerWave = kBytes / 1024 / 4;  // 1 KiB per copy instruction
  static_assert(kCopiesPerWave * 4 * 1024 == kBytes, "four waves' copies must cover a tile");
  // One copy instruction covers 1024 / kRowBytes rows, and the bank swizzle repeats
  // every 16 rows, so the lane offsets of a wave's copies repeat every kOffsetPeriod
  // instructions; the repeats differ only by 16 rows, which goes into the descriptor.
  static constexpr int kOffsetPeriod = kRowBytes / 64;
};

// Bank swizzle. The LDS has 64 four-byte banks, so a 256-byte span is one bank cycle:
// ds_read_b128 serves 16 lanes a cycle and ds_read_b64(_tr) 32 lanes. swz is chosen so
// that (1) the 16 consecutive rows one K read touches land on 16 distinct 16-byte bank
// slots, (2) the 4 rows x 4 chunks one transposed V read touches per 32 lanes do too.
// For 256-byte rows (D = 128) this is swz(r) = 4 (r mod 4) + (r / 4 mod 4). For
// 128-byte rows (D = 64) two rows share a bank cycle, and swz(r) = 4 (r / 2 mod 2) +
// (r / 4 mod 4).
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferFlags);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, int byte_offset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, 0));
}

// Workgroup barrier that orders LDS but leaves tile copies (vector-memory loads into LDS)
// in flight: it waits for this wave's own LDS reads (a copy issued after it may then
// overwrite what was read), and the "memory" clobber keeps the compiler from moving
// LDS accesses across it. Copies are waited for explicitly with wait_copies<N>.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// Wait until at most N of this wave's vector-memory loads are outstanding. They
// complete in issue order, so this waits for all but the N most recent.
template <int N>
__device__ __forceinline__ void wait_copies() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Raw buffer descriptor of a byte range (four scalar dwords): base address, no stride,
// `bytes` records, 32-bit data format. Reads at or past `bytes` return zero.
__device__ __forceinline__ i32x4 raw_descriptor(const char* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{static_cast<int>(a & 0xffffffffu), static_cast<int>((a >> 32) & 0xffffu), bytes,
               kBufferFlags};
}

// One 1 KiB tile-copy instruction: lane l's 16 bytes at byte_offset of the descriptor's
// range land at LDS address lds + 16 l (buffer_load_dwordx4 ... lds, LDS base in M0).
// It is written as inline asm so that the compiler does not track it as a pending LDS
// write: its own waits would then stop every later LDS read until the copy lands. The
// kernel orders these copies itself (wait_copies and lds_barrier). The instruction
// writes no VGPR, and M0 is used by nothing else in these kernels.
__device__ __forceinline__ void copy_1k(const i32x4& desc, uint32_t lds, int byte_offset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(byte_offset), "s"(desc)
               : "memory");
}

// Reductions over the two half-waves: for a symmetric op, op(lo, hi) of the pair that
// v_permlane32_swap(x, x) returns is the same in every lane.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// A pending copy of one 128-row tile into an LDS buffer: this wave's quarter of it,
// issued one 1 KiB instruction at a time.
template <int D>
struct Stage {
  // One descriptor per run of kOffsetPeriod instructions: run j starts 16 j rows into the
  // tile, so its lane offsets are those of run 0.
  i32x4 desc[Tile<D>::kCopiesPerWave / Tile<D>::kOffsetPeriod];
  uint32_t lds;
};

// The lane byte offsets of wave wi's tile copies. Copy t of wave wi fills bytes
// [(wi * kCopiesPerWave + t) KiB, +1 KiB) of a buffer; lane l writes 16 bytes at l * 16,
// i.e. chunk position p of row r, and so loads global chunk p ^ swz(r) of that row. The
// offsets repeat every kOffsetPeriod copies.
template <int D>
__device__ __forceinline__ void copy_offsets(int wi, int lane, int row_bytes,
                                             int (&off)[Tile<D>::kOffsetPeriod]) {
  using T = Tile<D>;
#pragma unroll
  for (int t = 0; t < T::kOffsetPeriod; ++t) {
    const int ci = (wi * T::kCopiesPerWave + t) * 64 + lane;
    const int row = ci / T::kChunks, p = ci % T::kChunks;
    off[t] = row * row_bytes + ((p ^ swz<D>(row)) << 4);
  }
}

// Wave wi's quarter of the copy of rows row0 .. row0 + 127 of a [rows][D] bf16 matrix at
// src (rows row_bytes apart) into buf. Rows at or past n read as zeros (the
// descriptor's range check); with on = false the copy fetches nothing and writes zeros.
template <int D>
__device__ __forceinline__ Stage<D> stage_rows(char* buf, const char* src, int row0, int n,
                                               int row_bytes, int wi, bool on) {
  using T = Tile<D>;
  const int key0 = on ? row0 : 0;
  const int rows = on ? (n - key0 < kBlock ? n - key0 : kBlock) : 0;
  const int bytes = rows > 0 ? (rows - 1) * row_bytes + T::kRowBytes : 0;
  Stage<D> st;
#pragma unroll
  for (int j = 0; j < T::kCopiesPerWave / T::kOffsetPeriod; ++j) {
    const int skip = 16 * j * row_bytes;
    st.desc[j] = raw_descriptor(src + static_cast<int64_t>(key0) * row_bytes + skip,
                                bytes > skip ? bytes - skip : 0);
  }
  st.lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)buf)) +
           wi * T::kCopiesPerWave * 1024;
  return st;
}

// Issue copy instruction t of a pending tile copy.
template <int D>
__device__ __forceinline__ void stage_issue(const Stage<D>& st,
                                            const int (&off)[Tile<D>::kOffsetPeriod], int t) {
  using T = Tile<D>;
  if (t < T::kCopiesPerWave)
    copy_1k(st.desc[t / T::kOffsetPeriod], st.lds + t * 1024, off[t % T::kOffsetPeriod]);
}

// LDS read offsets (bytes) of the two MFMA A-operand patterns on a swizzled tile; each is
// a lane part (base) plus a swizzle term that is XORed with the step index (x).
//  Row reads: the A operand [32 rows x 16 d] of k-step s for rows 32g + lane % 32, read
//  with ds_read_b128 at g * 32 rows + base + ((s << 5) ^ x). Row 32g + lq, chunk
//  2s + hl sits at position (2s + hl) ^ swz(lq); since 2s + hl = (s << 1) | hl, that is
//  ((s ^ (swz >> 1)) << 1) | ((hl ^ swz) & 1).
template <int D>
__device__ __forceinline__ void row_read_offsets(int lane, int& base, int& x) {
  const int lq = lane & 31, hl = lane >> 5;
  const int sw = swz<D>(lq);
  base = lq * Tile<D>::kRowBytes + (((hl ^ sw) & 1) << 4);
  x = (sw >> 1) << 5;
}
//  Transposed reads: the A operand [32 d x 16 rows] of step u (rows 16u .. 16u + 15 in
//  MFMA accumulator order) for d block db, from two ds_read_b64_tr_b16 at
//  16u rows + base0 + ((db << 6) ^ x0) and 16u rows + base1 + ((db << 6) ^ x1). In
//  16-lane group gi, source lane sl points at row 4hl + sl/4 (+ 8 for the second read)
//  and d = 32db + 16(gi&1) + 4(sl&3), i.e. chunk 4db + ch with ch = 2(gi&1) + (sl&3)/2,
//  at position (4db + ch) ^ swz(row) = ((db ^ (swz >> 2)) << 2) | ((ch ^ swz) & 3).
template <int D>
__device__ __forceinline__ void tr_read_offsets(int lane, int& base0, int& x0, int& base1,
                                                int& x1) {
  const int hl = lane >> 5, gi = (lane >> 4) & 3, sl = lane & 15;
  const int row = 4 * hl + (sl >> 2);
  const int ch = 2 * (gi & 1) + ((sl & 3) >> 1);
  const int sw0 = swz<D>(row), sw1 = swz<D>(row + 8);
  const int rd = row * Tile<D>::kRowBytes + 8 * (sl & 1);
  base0 = rd + (((ch ^ sw0) & 3) << 4);
  x0 = (sw0 & ~3) << 4;
  base1 = rd + 8 * Tile<D>::kRowBytes + (((ch ^ sw1) & 3) << 4);
  x1 = (sw1 & ~3) << 4;
}

// Element masking limits. Token indices stay below 2^21 (16352 blocks of 128), so no
// spatial distance reaches 2^22: a radius is clamped to kMaxReach without changing the
// rule, and a frame length is at most kMaxFrame, which keeps every position sum below
// 2^24 in magnitude.
constexpr int kMaxReach = 1 << 22;
constexpr int kMaxFrame = 1 << 22;

// Host check of the element-masking arguments: tokens_per_frame = 0 is block semantics
// (the others are then ignored); otherwise a frame of 128 .. kMaxFrame tokens (at least
// one key tile), W0 >= 1 (the diagonal stays allowed) and a grid width of 0 (the 1-D
// distance) or a divisor of the frame length.
inline bool element_args_valid(int32_t s, int32_t w0, int32_t grid_w) {
  if (s == 0) return true;
  if (s < kBlock || s > kMaxFrame || w0 < 1) return false;
  return grid_w == 0 || (grid_w > 0 && s % grid_w == 0);
}

// Base-2 score scale (host): c = scale * log2(e), kept >= FLT_MIN so that a masked score
// of -inf stays -inf after scaling (never -inf * 0 = NaN). For scale = 0 every finite
// score times FLT_MIN rounds away against the reference maximum, so each real key gets
// the same p: the scale-0 softmax, a mean over the key set.
inline float base2_scale(float scale) { return fmaxf(scale * kLog2e, FLT_MIN); }

// (a / S, a % S) for 0 <= a < 2^24 with a quotient below 2^21 (frame lengths S >= 128,
// or any grid width when a < 2^21), given inv_s within a few ulp of 1 / S: the float
// estimate of the quotient is then off by at most one, and one correction each way
// gives the exact result.
__device__ __forceinline__ void div_frame(int a, int S, float inv_s, int& f, int& s) {
  f = static_cast<int>(static_cast<float>(a) * inv_s);
  s = a - f * S;
  if (s >= S) { ++f; s -= S; }
  if (s < 0) { --f; s += S; }
}

// Bits lo .. hi (clamped to 0 .. 31) of a 32-bit word; none when hi < lo. With
// 0 <= a <= b <= 32, 2^b - 2^a has exactly bits [a, b) set, and its low word needs no
// case for b = 32: two 64-bit shifts and one add.
__device__ __forceinline__ uint32_t run_bits(int lo, int hi) {
  const int a = min(max(lo, 0), 32);
  const int b = max(min(hi + 1, 32), a);
  return static_cast<uint32_t>((1ull << b) - (1ull << a));
}

// Element masking of a 128 x 128 tile of scores in MFMA accumulator layout (the rule of
// "Radial Attention: A Breakthrough in Efficient Long Video Generation", How Radial
// Attention Works, applied to single entries, with frame-major coordinates and -inf for
// masked scores as on the radial-attention-video SKILL.md page, Step 1): tokens a and b
// may meet iff
//   |s_a - s_b| <= (W0 - 1) >> floor(log2(|f_a - f_b| + 1)),
// the integer form of |s_a - s_b| * 2^floor(log2(d + 1)) < W0. The rule is symmetric,
// so the same code serves scores with queries on the lanes and keys on the entries and
// the other way round. A lane holds one token, own0 + lane % 32 (own0: the wave's
// first), and entries ent0 + 4 hl + c, c = 32g + 8(e/4) + e%4, for accumulator entry
// (g, e). With S >= 128 the entries lie in at most two frames, kf and kf + 1 (c from
// cut on), and in each the allowed ones form one run of c: [lo_a, hi_a] and
// [lo_b, hi_b]. Per group of 32 entries the runs become a 32-bit mask; each entry then
// takes its bit as 0 or all ones (v_bfe_i32) and selects its score or -inf with it
// (v_bfi_b32): two VALU instructions and no lane masks. A tile that every lane of the
// wave keeps whole is left alone. NG is the number of 32-entry groups the lane holds: 4
// for a whole tile (entries c < 128), 2 for the first or second half of one (c < 64,
// with ent0 the half's first token).
template <int NG = 4>
__device__ __forceinline__ void element_mask_tile(int own0, int ent0, int S, int ew0m1, int lane,
                                                  f32x16 (&sacc)[NG]) {
  constexpr int kLast = 32 * NG - 4;  // one past the lane's last entry position c
  // S and own0 go through an empty asm so that what is derived from them is recomputed
  // here, per tile, rather than held in registers across the caller's loop.
  asm volatile("" : "+s"(S), "+s"(own0));
  // An approximate reciprocal is enough: div_frame corrects the quotient by one.
  const float inv_s = __builtin_amdgcn_rcpf(static_cast<float>(S));
  // Frame and spatial index of the wave's first own token and of the tile's first entry
  // (both the same in every lane), then this lane's own: one frame wrap at most.
  int fq, sq, kf, ks;
  div_frame(own0, S, inv_s, fq, sq);
  div_frame(ent0, S, inv_s, kf, ks);
  sq += lane & 31;
  if (sq >= S) { sq -= S; ++fq; }
  ks += 4 * (lane >> 5);
  if (ks >= S) { ks -= S; ++kf; }
  const int cut = S - ks;  // entries with c >= cut are tokens of frame kf + 1
  const int da = fq > kf ? fq - kf : kf - fq;
  const int db = fq > kf + 1 ? fq - kf - 1 : kf + 1 - fq;
  const int ra = min(ew0m1 >> (31 - __builtin_clz(static_cast<unsigned>(da) + 1u)), kMaxReach);
  const int rb = min(ew0m1 >> (31 - __builtin_clz(static_cast<unsigned>(db) + 1u)), kMaxReach);
  const int base = sq - ks;  // c of the entry at the lane's own spatial index, frame kf
  const int lo_a = max(base - ra, 0), hi_a = min(base + ra, cut - 1);
  const int lo_b = max(base + S - rb, cut), hi_b = base + S + rb;
  const bool full = lo_a <= 0 && hi_a >= min(cut, kLast) - 1 &&
                    (cut >= kLast || (lo_b <= cut && hi_b >= kLast - 1));
  if (__builtin_amdgcn_ballot_w64(!full) == 0) return;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const uint32_t bits = run_bits(lo_a - 32 * g, hi_a - 32 * g) |
                          run_bits(lo_b - 32 * g, hi_b - 32 * g);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t keep = static_cast<uint32_t>(
          __builtin_amdgcn_sbfe(static_cast<int>(bits), 8 * (e >> 2) + (e & 3), 1));
      sacc[g][e] = __uint_as_float((keep & __float_as_uint(sacc[g][e])) | (~keep & 0xff800000u));
    }
  }
}

// Element masking with the 2-D grid distance (the radial-attention-video SKILL.md page,
// Step 1, its grid-distance helper): a frame of S tokens is a grid of S / W rows of W
// columns stored row by row, and tokens a and b may meet iff
//   |y_a - y_b| + |x_a - x_b| <= (W0 - 1) >> floor(log2(|f_a - f_b| + 1)).
// Lanes and entries are laid out as in element_mask_tile, and the rule is symmetric as
// well. The tile's 128 entries are walked as segments of one grid row each (the same in
// every lane): in key row y of frame f, the lane's token reaches the columns
// [x - t, x + t], t = r(f) - |y_own - y|, which is one run of tile positions. The runs
// go into the lane's four 32-bit words and are applied as there. There are at most
// ceil(128 / W) + 1 segments; a frame ends at a row end, so frames add none. Divisions
// use the float reciprocal with one correction (all indices are below 2^21). NG as for
// element_mask_tile.
template <int NG = 4>
__device__ __forceinline__ void element_mask_grid_tile(int own0, int ent0, int S, int W,
                                                       int ew0m1, int lane,
                                                       f32x16 (&sacc)[NG]) {
  constexpr int kEntries = 32 * NG;
  asm volatile("" : "+s"(S), "+s"(W), "+s"(own0));
  const float inv_s = __builtin_amdgcn_rcpf(static_cast<float>(S));
  const float inv_w = __builtin_amdgcn_rcpf(static_cast<float>(W));
  int fq, sq, yq, xq;  // this lane's token
  div_frame(own0 + (lane & 31), S, inv_s, fq, sq);
  div_frame(sq, W, inv_w, yq, xq);
  int fk, sk, yk, x0;  // the tile's first entry (the same in every lane)
  div_frame(ent0, S, inv_s, fk, sk);
  div_frame(sk, W, inv_w, yk, x0);
  int row_end = sk - x0 + W;  // in-frame index one past the segment's row
  const int sh = 4 * (lane >> 5);  // this lane's entries sit sh positions later
  uint32_t bits[NG] = {};
  for (int c = 0; c < kEntries;) {
    const int len = min(W - x0, kEntries - c);
    const int d = fq > fk ? fq - fk : fk - fq;
    const int r = min(ew0m1 >> (31 - __builtin_clz(static_cast<unsigned>(d) + 1u)), kMaxReach);
    const int t = r - (yq > yk ? yq - yk : yk - yq);
    // Tile positions of columns [xq - t, xq + t] of this row, clipped to the segment, in
    // this lane's bit numbering. For t < 0 the run is empty as it stands (hi < lo).
    const int lo = max(c + xq - t - x0, c) - sh;
    const int hi = min(c + xq + t - x0, c + len - 1) - sh;
#pragma unroll
    for (int g = 0; g < NG; ++g)
      if (c <= 32 * g + 35 && c + len > 32 * g)  // the words the segment can reach
        bits[g] |= run_bits(lo - 32 * g, hi - 32 * g);
    c += len;
    x0 = 0;
    ++yk;
    row_end += W;
    if (row_end > S) {  // the next row is row 0 of the next frame
      row_end = W;
      yk = 0;
      ++fk;
    }
  }
  const uint32_t mine = 0x0f0f0f0fu;  // the bits of this lane's 16 entries of a word
  uint32_t all = mine;
#pragma unroll
  for (int g = 0; g < NG; ++g) all &= bits[g];
  const bool full = all == mine;
  if (__builtin_amdgcn_ballot_w64(!full) == 0) return;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t keep = static_cast<uint32_t>(
          __builtin_amdgcn_sbfe(static_cast<int>(bits[g]), 8 * (e >> 2) + (e & 3), 1));
      sacc[g][e] = __uint_as_float((keep & __float_as_uint(sacc[g][e])) | (~keep & 0xff800000u));
    }
  }
}

// Element masking of a tile: E = 1 takes the 1-D distance, E = 2 the grid distance with
// grid width gw.
template <int E, int NG = 4>
__device__ __forceinline__ void element_mask_any(int own0, int ent0, int S, int gw, int ew0m1,
                                                 int lane, f32x16 (&sacc)[NG]) {
  if constexpr (E == 2)
    element_mask_grid_tile<NG>(own0, ent0, S, gw, ew0m1, lane, sacc);
  else
    element_mask_tile<NG>(own0, ent0, S, ew0m1, lane, sacc);
}

// Element masking from stored bits (an element table, radial_build_element_table): bit
// 16g + e of `bits` keeps accumulator entry (g, e) of this lane (the lanes and entries
// of element_mask_tile), a clear bit makes it -inf. The table holds the same decisions
// as element_mask_any, taken once per mask instead of once per tile visit. A tile that
// every lane keeps whole is left alone.
template <int NG = 4>
__device__ __forceinline__ void element_mask_stored(uint64_t bits, f32x16 (&sacc)[NG]) {
  constexpr uint64_t kAll = NG == 4 ? ~0ull : (1ull << (16 * NG)) - 1;
  if (__builtin_amdgcn_ballot_w64((bits & kAll) != kAll) == 0) return;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const uint32_t word = static_cast<uint32_t>(bits >> (32 * (g >> 1)));
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t keep = static_cast<uint32_t>(
          __builtin_amdgcn_sbfe(static_cast<int>(word), 16 * (g & 1) + e, 1));
      sacc[g][e] = __uint_as_float((keep & __float_as_uint(sacc[g][e])) | (~keep & 0xff800000u));
    }
  }
}

// Padding of the entries of a tile in accumulator layout: entry (g, e) of a lane is
// token ent0 + 4 hl + 32g + 8(e/4) + e%4 (g < NG), and tokens at or past n get -inf. Applied
// arithmetically, min(s, +inf or -inf), so that the 64 tests need no lane masks; the
// per-group base goes through an empty asm so that the compiler does not fold the 64
// offsets into 64 scalar-register constants (the remaining offsets, 0 .. 27, are inline
// operands).
template <int NG = 4>
__device__ __forceinline__ void pad_mask_tile(int ent0, int n, int lane, f32x16 (&sacc)[NG]) {
  const int lim = n - ent0 - 4 * (lane >> 5);
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    int base = lim - 1 - 32 * g;
    asm volatile("" : "+v"(base));
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int pad = (base - (8 * (i >> 2) + (i & 3))) >> 31;  // -1: padding
      sacc[g][i] = fminf(sacc[g][i], __int_as_float(0x7f800000 | (pad & 0x80000000)));
    }
  }
}

}  // namespace
