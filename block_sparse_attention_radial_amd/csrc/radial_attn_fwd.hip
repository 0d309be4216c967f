// Block-sparse flash-style forward pass of Radial Attention for gfx950 (CDNA4).
//
// What is computed, after the radial-attention-video SKILL.md page, Step 2
// (scores = Q K^T * scale, masked entries -inf, softmax, times V, one mask for all batches
// and heads), and "Radial Attention: A Breakthrough in Efficient Long Video Generation",
// How Radial Attention Works (the static mask is applied in 128x128 blocks):
//   for every (batch, head, 128-row query block qb):
//     O[rows] = softmax(scale * Q[rows] K[keys]^T) V[keys]
//   where keys are the real tokens of the key blocks listed in the CSR row qb.
//
// Work decomposition. One workgroup of 8 wave64 owns a pair of neighbouring query blocks
// (2p and 2p+1, 128 rows each) and fills one CU. Its waves form two groups of four; group
// g owns query block 2p+g, wave i of a group owns its rows 32i .. 32i+31. Both groups
// walk the union of the two rows' key-block lists, in ascending order (a merge of the
// two sorted CSR rows); a group skips the tiles that are not in its own row. Each K/V
// tile is thus copied to LDS once and used by both query blocks: neighbouring query
// blocks share most of their key blocks, so this halves the traffic through each CU's
// L1, which bounds how fast tiles can be streamed in.
//
// Ping-pong. A group's work per tile is an MFMA part (P*V of the previous tile, then
// Q*K^T of this tile) and a VALU part (the softmax). Group 1 runs one phase behind group
// 0, with a workgroup barrier after every phase: while one group issues MFMAs the other
// runs its softmax, then the roles swap, so every SIMD's matrix core always has a wave
// feeding it. Tile t is used by group 0 in phase 2t and by group 1 in phase 2t+1, so K
// and V are double-buffered. The group in its softmax phase also issues the next copies
// (group 1 copies V(t) in phase 2t, group 0 copies K(t+1) in phase 2t+1), spread over
// its softmax steps: a copy instruction holds its wave back while the L1 drains it.
//
// Per tile:
//  - S^T = K Q^T runs on v_mfma_f32_32x32x16_bf16, with keys on M and queries on N. A
//    lane holds one query (lane % 32) and 64 of the tile's 128 keys, so the row max and
//    row sum are in-lane, plus one v_permlane32_swap between the half-waves.
//  - O^T = V^T P^T runs on the same MFMA, with head_dim on M and queries on N. The S^T
//    accumulator is, key for key, the B operand this product needs once the contraction
//    runs over keys in accumulator order. So P goes from registers into the MFMA after
//    one bf16 pack.
//  - K and V tiles are stored key-major in LDS ([key][d], no padding). Chunk c (16
//    bytes) of row r sits at position c ^ swz(r), which spreads every read pattern below
//    over all 64 banks.
//  - V^T operands come from ds_read_b64_tr_b16. One such read gives a lane 4 keys of one
//    V column, and two of them form an MFMA operand.
//  - Tiles are copied HBM/L2 -> LDS by buffer_load ... lds, with no staging registers.
//    The descriptor's range check returns zeros past the sequence end, so the ragged
//    last block needs no guarded loads.
//  - Online softmax in base 2: c = scale * log2(e), p = 2^(c*s - m). The running max m
//    moves only when a tile's max exceeds it by more than 2^8 for some row of the wave.
//    Until then p <= 256, and O and l are not rescaled. The final O / l is exact for
//    any m used consistently. The row sum adds the bf16-rounded p, the same values the
//    PV product multiplies.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <climits>
#include <cstdint>

#include "../../include/radial_attn.h"

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

constexpr int kBlock = 128;        // query rows per group, keys per tile
constexpr int kThreads = 512;      // 8 wave64: two groups of four
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;  // log2 units: p stays <= 256 between rescales
// Fourth dword of a raw gfx9 buffer descriptor: 32-bit data format, no stride/swizzle.
constexpr int kBufferFlags = 0x00020000;

template <int D>
struct Tile {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;               // 16-byte chunks per row
  static constexpr int kBytes = kBlock * kRowBytes;   // one K or V tile
  static constexpr int kCopiesPerWave = kBytes / 1024 / 4;  // 1 KiB per copy instruction
  static_assert(kCopiesPerWave * 4 * 1024 == kBytes, "a group's copies must cover the tile");
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
// writes no VGPR, and M0 is used by nothing else in this kernel.
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

// Everything one wave needs across the phase loop, gathered so that the two groups can
// run the same phase code over different (compile-time distinct) LDS buffers.
template <int D>
struct WaveState {
  using T = Tile<D>;
  // inputs
  const char* kh;  // K of this (batch, head), as bytes
  const char* vh;  // V of this (batch, head), as bytes
  int nb, n, row_bytes, wi, lane, hl;
  float c;
  // per-lane offsets
  int copy_off[T::kCopiesPerWave];
  int k_rd, k_sw, v_rd, v_sw0, v_sw1, v_ch;
  // Q^T fragments (bf16 pairs; kept as dwords so the struct is a valid host type too)
  u32x4 qf[D / 16];
  // softmax state
  f32x16 oacc[D / 32];
  float m_run, l_run;
};

// A pending copy of one K or V tile (128 rows) into a group buffer: this wave's quarter
// of it, issued one 1 KiB instruction at a time so that the copies can be spread over
// the compute instead of stalling the wave in one burst.
// A copy that is not wanted (on = false) gets a descriptor of zero bytes: its loads
// write zeros into the buffer, which is not read again before its next real copy.
// That keeps the copy code free of branches, so the scheduler can keep it interleaved.
template <int D>
struct Stage {
  i32x4 desc;
  uint32_t lds;
};

template <int D>
__device__ __forceinline__ Stage<D> stage_tile(const WaveState<D>& w, char* buf, const char* src,
                                               int kb, bool on) {
  using T = Tile<D>;
  const bool valid = on && static_cast<unsigned>(kb) < static_cast<unsigned>(w.nb);
  const int key0 = valid ? kb * kBlock : 0;
  const int rows = valid ? (w.n - key0 < kBlock ? w.n - key0 : kBlock) : 0;
  Stage<D> st;
  st.desc = raw_descriptor(src + static_cast<int64_t>(key0) * w.row_bytes,
                           rows > 0 ? (rows - 1) * w.row_bytes + T::kRowBytes : 0);
  st.lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)buf)) +
           w.wi * T::kCopiesPerWave * 1024;
  return st;
}

// Issue copy instruction t of a pending tile copy.
template <int D>
__device__ __forceinline__ void stage_issue(const WaveState<D>& w, const Stage<D>& st, int t) {
  if (t < Tile<D>::kCopiesPerWave) copy_1k(st.desc, st.lds + t * 1024, w.copy_off[t]);
}

// Issue a whole tile copy at once (prologue only).
template <int D>
__device__ __forceinline__ void stage_all(const WaveState<D>& w, char* buf, const char* src, int kb) {
  const Stage<D> st = stage_tile(w, buf, src, kb, true);
#pragma unroll
  for (int t = 0; t < Tile<D>::kCopiesPerWave; ++t) stage_issue(w, st, t);
}

// PV part of an MFMA phase: O += P(j-1) V(j-1). `sacc` holds P(j-1) packed as bf16
// (see softmax_tile). V^T fragments go through a two-step ring: the reads for step u + 1
// are issued before the MFMAs of step u (each step is 2 x D/32 transposed reads, and at
// most 15 LDS reads can be outstanding). The sched_group_barrier pairs pin that order
// against the scheduler's wish to save registers.
template <int D>
__device__ __forceinline__ void pv_part(WaveState<D>& w, const char* vbuf, const f32x16 (&sacc)[4]) {
  using T = Tile<D>;
  constexpr int R = 2 * (D / 32);  // transposed reads per step
  const char* vb = vbuf + w.v_rd;
  auto read_v = [&](int u, bf16x8 (&vf)[D / 32]) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const char* p0 = vb + 16 * u * T::kRowBytes;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(p0 + (((4 * db + w.v_ch) ^ w.v_sw0) << 4)));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(p0 + 8 * T::kRowBytes + (((4 * db + w.v_ch) ^ w.v_sw1) << 4)));
      vf[db] = __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo),
                                       __builtin_bit_cast(bf16x4, hi), 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  bf16x8 vf[2][D / 32];
  read_v(0, vf[0]);
  __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
#pragma unroll
  for (int u = 0; u < 8; ++u) {  // u = 2g + s2: 16 keys of the contraction
    if (u + 1 < 8) {
      read_v(u + 1, vf[(u + 1) & 1]);
      __builtin_amdgcn_sched_group_barrier(0x100, R, 0);  // reads of step u + 1
    }
    const f32x4 packed = {sacc[u >> 1][4 * (u & 1) + 0], sacc[u >> 1][4 * (u & 1) + 1],
                          sacc[u >> 1][4 * (u & 1) + 2], sacc[u >> 1][4 * (u & 1) + 3]};
    const bf16x8 pu = __builtin_bit_cast(bf16x8, packed);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
      w.oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[u & 1][db], pu, w.oacc[db], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, D / 32, 0);  // then the MFMAs of step u
  }
}

// QK part of an MFMA phase: S(j) = Q K(j)^T into `sacc`. The K fragments go through a
// two-step ring: the reads for k-step s + 2 are issued right after the MFMAs of step s
// have taken their operands, so 8 reads are in flight while MFMAs run (pinned the same
// way).
template <int D>
__device__ __forceinline__ void qk_part(WaveState<D>& w, const char* kbuf, f32x16 (&sacc)[4]) {
  using T = Tile<D>;
  constexpr int S = D / 16;
  const char* kbp = kbuf + w.k_rd;
  auto read_k = [&](int s, bf16x8 (&kf)[4]) {
    const int ch = ((2 * s + w.hl) ^ w.k_sw) << 4;
#pragma unroll
    for (int g = 0; g < 4; ++g)
      kf[g] = *reinterpret_cast<const bf16x8*>(kbp + g * 32 * T::kRowBytes + ch);
  };
  bf16x8 kf[2][4];
  read_k(0, kf[0]);
  read_k(1, kf[1]);
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // the 8 initial reads
#pragma unroll
  for (int s = 0; s < S; ++s) {
#pragma unroll
    for (int g = 0; g < 4; ++g)  // the first k-step takes an inline zero accumulator
      sacc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          kf[s & 1][g], __builtin_bit_cast(bf16x8, w.qf[s]), s == 0 ? f32x16{} : sacc[g], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // 4 MFMAs of step s
    if (s + 2 < S) {
      read_k(s + 2, kf[s & 1]);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // then the reads of step s + 2
    }
  }
}

// Softmax of tile j (column kb): mask padding keys, find the row max, rescale O and l
// when the max moves, and turn S(j) into P(j). P(j) is written back over S(j): the 8 bf16
// of P for (g, s2), made from sacc[g][8 s2 .. 8 s2 + 7], are packed into the dwords
// sacc[g][4 s2 .. 4 s2 + 3], so S and P share the same 64 registers. `hook(u)` runs
// after each eighth of the work (it issues tile copies).
template <int D, typename Hook>
__device__ __forceinline__ void softmax_tile(WaveState<D>& w, int kb, f32x16 (&sacc)[4],
                                             Hook&& hook) {
  if (static_cast<unsigned>(kb) >= static_cast<unsigned>(w.nb)) {
    // Out-of-range column: the tile contributes nothing (P = 0).
#pragma unroll
    for (int g = 0; g < 4; ++g) sacc[g] = f32x16{};
#pragma unroll
    for (int u = 0; u < 8; ++u) hook(u);
    return;
  }
  const int key_lim = w.n - kb * kBlock;  // keys at or past this index are padding
  if (key_lim < kBlock) {
    // Key of accumulator entry (g, i) is 32g + 8(i/4) + (i%4) + 4hl: compare the
    // constant part against one per-lane limit.
    const int lim = key_lim - 4 * w.hl;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (32 * g + 8 * (i >> 2) + (i & 3) >= lim) sacc[g][i] = -INFINITY;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[g][i]);
  const float m_tile = halves_max(mx) * w.c;
  if (__builtin_amdgcn_ballot_w64(m_tile > w.m_run + kRescaleThreshold) != 0) {
    const float m_new = fmaxf(w.m_run, m_tile);
    const float alpha = __builtin_amdgcn_exp2f(w.m_run - m_new);
    w.m_run = m_new;
    w.l_run *= alpha;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) w.oacc[i] *= alpha;
  }
  const float neg_m = -w.m_run;
  const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int g = u >> 1, s2 = u & 1;
    f32x8 p8;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
      p8[jj] = __builtin_amdgcn_exp2f(fmaf(sacc[g][8 * s2 + jj], w.c, neg_m));
    const bf16x8 pu = __builtin_convertvector(p8, bf16x8);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const bf16x2 pair = {pu[2 * jj], pu[2 * jj + 1]};
      w.l_run = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, w.l_run, false);
    }
    const f32x4 packed = __builtin_bit_cast(f32x4, pu);
#pragma unroll
    for (int e = 0; e < 4; ++e) sacc[g][4 * s2 + e] = packed[e];
    hook(u);
  }
}

// Ascending merge of two sorted CSR rows, the key-block list a workgroup walks. The
// state is the same in every lane (it lives in scalar registers); INT_MAX marks an
// exhausted row.
struct Merge {
  const int32_t* col;
  int ia, a_end, ib, b_end;
  int pa, pb;  // next entry of each row
};

__device__ __forceinline__ Merge merge_begin(const int32_t* col, int a0, int a1, int b0, int b1) {
  Merge m{col, a0, a1, b0, b1, INT_MAX, INT_MAX};
  if (a0 < a1) m.pa = col[a0];
  if (b0 < b1) m.pb = col[b0];
  return m;
}

// The next key block of the union and which rows hold it; false when both are done.
__device__ __forceinline__ bool merge_next(Merge& m, int& kb, bool& in_a, bool& in_b) {
  kb = m.pa < m.pb ? m.pa : m.pb;
  if (kb == INT_MAX) return false;
  in_a = m.pa == kb;
  in_b = m.pb == kb;
  if (in_a) m.pa = ++m.ia < m.a_end ? m.col[m.ia] : INT_MAX;
  if (in_b) m.pb = ++m.ib < m.b_end ? m.col[m.ib] : INT_MAX;
  return true;
}

// One union tile as a group sees it.
struct TileRef {
  int kb;     // key block
  bool here;  // the tile exists (index < union length)
  bool mine;  // ... and belongs to this group's row
};

// The phase loop of group G (G = 0: query block 2p, G = 1: query block 2p+1). With U the
// union length, phase 2t is group 0's MFMA phase for tile t and group 1's softmax phase
// for tile t-1; phase 2t+1 is the other way round. Each phase ends at a workgroup
// barrier, and both groups pass 2U + 3 of them.
//   group 0, MFMA t:    O += P(t-1) V(t-1); S(t) = Q K(t)^T
//   group 0, softmax t: softmax of tile t; copy K(t+1) meanwhile; wait for it
//   group 1, MFMA t:    O += P(t-1) V(t-1); S(t) = Q K(t)^T; wait for the V(t) copy
//   group 1, softmax t: softmax of tile t; copy V(t+1) meanwhile
// Tile t lives in K buffer t % 2 and V buffer t % 2. A copy into a buffer starts only
// after the barrier that ends the last phase reading its old tile. P(t-1) and S(t) share
// registers, so P V runs before Q K^T.
template <int D, int G>
__device__ __forceinline__ void run_group(WaveState<D>& w, Merge m, char* __restrict__ k0,
                                          char* __restrict__ k1, char* __restrict__ v0,
                                          char* __restrict__ v1) {
  f32x16 sacc[4];  // S(t) after an MFMA phase, P(t) after a softmax phase
  auto pick = [](int t, char* b0, char* b1) { return (t & 1) ? b1 : b0; };
  auto fetch = [&](TileRef& r) {
    bool in_a = false, in_b = false;
    r.here = merge_next(m, r.kb, in_a, in_b);
    r.mine = r.here && (G == 0 ? in_a : in_b);
  };
  TileRef prev{0, false, false}, cur, next;
  fetch(cur);
  fetch(next);
  if (G == 1) {  // phase 0: copy V(0)
    if (cur.here) stage_all(w, v0, w.vh, cur.kb);
    lds_barrier();
  }
  for (int t = 0;; ++t) {
    // ---- MFMA phase t ----
    __builtin_amdgcn_s_setprio(1);
    if (prev.mine) pv_part(w, pick(t - 1, v0, v1), sacc);
    if (cur.mine) qk_part(w, pick(t, k0, k1), sacc);
    if (G == 1) wait_copies<0>();  // V(t)
    lds_barrier();
    // ---- softmax phase t ----
    __builtin_amdgcn_s_setprio(0);
    const Stage<D> st = G == 0 ? stage_tile(w, pick(t + 1, k0, k1), w.kh, next.kb, next.here)
                               : stage_tile(w, pick(t + 1, v0, v1), w.vh, next.kb, next.here);
    auto hook = [&](int u) {
      // Keep the scheduler from bunching the copies: each softmax step's math stays
      // between its copy instructions.
      __builtin_amdgcn_sched_barrier(0);
      stage_issue(w, st, u);
      __builtin_amdgcn_sched_barrier(0);
    };
    if (cur.mine) {
      softmax_tile(w, cur.kb, sacc, hook);
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) stage_issue(w, st, u);
    }
    if (G == 0) wait_copies<0>();  // K(t+1)
    lds_barrier();
    if (!cur.here) break;  // phase 2U+1 (group 0) / 2U+2 (group 1) done
    prev = cur;
    cur = next;
    fetch(next);
  }
  if (G == 0) lds_barrier();  // group 1's last phase
  __builtin_amdgcn_s_setprio(0);
  wait_copies<0>();
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void radial_fwd_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ o, float* __restrict__ lse, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, int nb, int heads, int n, float c,
    int64_t stride_b, int64_t stride_h, int stride_s) {
  using T = Tile<D>;
  // Two K and two V buffers at fixed offsets.
  __shared__ __attribute__((aligned(1024))) char smem[4 * T::kBytes];
  char* const k0 = smem;
  char* const k1 = smem + T::kBytes;
  char* const v0 = smem + 2 * T::kBytes;
  char* const v1 = smem + 3 * T::kBytes;

  // Work mapping. Workgroup ids go to the 8 XCDs round-robin (XCD = id % 8) and are
  // dispatched in id order. Ids [bh * np, (bh + 1) * np) all belong to head bh (np query
  // block pairs per head), so the whole chip works on one or two heads at a time and
  // their K/V stays in the shared Infinity Cache. Inside a head, the ids that land on
  // XCD x take one contiguous run of pairs, in order, so neighbouring query blocks
  // (which read mostly the same K/V tiles) share that XCD's L2.
  const int np = (nb + 1) >> 1;
  const int pid = blockIdx.x;
  const int bh = pid / np;
  const int first_id = bh * np;
  const int xcd = pid & 7;
  int seg = 0;  // pairs of this head taken by XCDs 0 .. xcd-1
  for (int y = 0; y < xcd; ++y)
    seg += ((first_id + np - 1 - y) >> 3) - ((first_id - 1 - y) >> 3);
  const int first_here = first_id + ((xcd - first_id) & 7);  // first id of this head on xcd
  const int pair = seg + ((pid - first_here) >> 3);
  const int b = bh / heads, h = bh - b * heads;
  const int64_t base = b * stride_b + h * stride_h;

  const int tid = threadIdx.x;
  // The wave index is the same in every lane; saying so lets it live in a scalar
  // register (it feeds M0, the LDS base of the tile copies).
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;       // query block 2 pair + grp
  const int qb = 2 * pair + grp;   // may be nb (no rows) for the last pair of an odd nb

  WaveState<D> w;
  w.kh = reinterpret_cast<const char*>(k + base);
  w.vh = reinterpret_cast<const char*>(v + base);
  w.nb = nb;
  w.n = n;
  w.c = c;
  w.row_bytes = stride_s * 2;
  w.wi = wave & 3;  // query rows 32 wi .. 32 wi + 31
  w.lane = tid & 63;
  const int lq = w.lane & 31;  // query column owned by this lane
  w.hl = w.lane >> 5;          // half-wave

  // ---- Q^T as the MFMA B operand: d = 16s + 8hl .. +7 of this lane's query ----
  {
    const int q0 = qb * kBlock;
    const int rows = n - q0 < kBlock ? n - q0 : kBlock;
    const auto rq = make_rsrc(q + base + static_cast<int64_t>(q0 < n ? q0 : 0) * stride_s,
                              rows > 0 ? (rows - 1) * w.row_bytes + T::kRowBytes : 0);
    const int off = (w.wi * 32 + lq) * w.row_bytes + w.hl * 16;
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      w.qf[s] = buffer_load16(rq, off + s * 32);
    // Wait for Q here, where the compiler sees it. Otherwise its wait-count bookkeeping
    // carries the Q loads into the phase loop as pending and waits on the vector-memory
    // counter there, i.e. on the tile copies, every iteration.
    __builtin_amdgcn_s_waitcnt(0);
  }

  // ---- tile copies: this wave's quarter of a tile, 1 KiB per instruction ----
  // Copy t of wave wi fills bytes [(wi * kCopiesPerWave + t) KiB, +1 KiB) of a buffer;
  // lane l writes 16 bytes at l * 16, i.e. chunk position p of row r, and so loads
  // global chunk p ^ swz(r) of that row.
#pragma unroll
  for (int t = 0; t < T::kCopiesPerWave; ++t) {
    const int ci = (w.wi * T::kCopiesPerWave + t) * 64 + w.lane;
    const int row = ci / T::kChunks, p = ci % T::kChunks;
    w.copy_off[t] = row * w.row_bytes + ((p ^ swz<D>(row)) << 4);
  }

  // ---- per-lane LDS read offsets for the MFMA operands (bytes) ----
  // K (A operand of S^T): row 32g + lq, chunk 2s + hl.
  w.k_rd = lq * T::kRowBytes;
  w.k_sw = swz<D>(lq);
  // V^T (A operand of O^T) via ds_read_b64_tr_b16: in 16-lane group gi, source lane sl
  // points at key 4hl + sl/4 (+ 8 for the second read of a pair, + tile offsets) and
  // d = 32db + 16(gi&1) + 4(sl&3).
  const int gi = (w.lane >> 4) & 3, sl = w.lane & 15;
  const int v_key = 4 * w.hl + (sl >> 2);
  w.v_rd = v_key * T::kRowBytes + 8 * (sl & 1);
  w.v_sw0 = swz<D>(v_key);
  w.v_sw1 = swz<D>(v_key + 8);
  w.v_ch = 2 * (gi & 1) + ((sl & 3) >> 1);

#pragma unroll
  for (int i = 0; i < D / 32; ++i) w.oacc[i] = f32x16{};
  w.m_run = -INFINITY;  // max of c * s used for p, base-2 units
  w.l_run = 0.f;        // sum of bf16(p) over this lane's keys

  // The two rows' column ranges (the second row is empty past the last query block).
  const int qa = 2 * pair, qbb = 2 * pair + 1;
  const int a0 = row_ptr[qa], a1 = row_ptr[qa + 1];
  const int b0 = qbb < nb ? row_ptr[qbb] : 0, b1 = qbb < nb ? row_ptr[qbb + 1] : 0;
  const Merge m = merge_begin(col_idx, a0, a1, b0, b1);

  // Prologue: group 0's first K tile. The compiler does not see the tile copies, so a
  // barrier never waits for them by itself: every wait for a copy is explicit.
  if (grp == 0) {
    Merge m0 = m;
    int kb;
    bool in_a, in_b;
    if (merge_next(m0, kb, in_a, in_b)) stage_all(w, k0, w.kh, kb);
  }
  wait_copies<0>();
  __syncthreads();
  if (grp == 0)
    run_group<D, 0>(w, m, k0, k1, v0, v1);
  else
    run_group<D, 1>(w, m, k0, k1, v0, v1);

  // ---- epilogue: O / l, bf16, store rows < n ----
  const float l_tot = halves_sum(w.l_run);
  const float inv = 1.0f / l_tot;
  const int qrow = qb * kBlock + w.wi * 32 + lq;
  if (qrow < n) {
    __bf16* orow = o + base + static_cast<int64_t>(qrow) * stride_s;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        const f32x4 x = {w.oacc[db][4 * ib + 0] * inv, w.oacc[db][4 * ib + 1] * inv,
                         w.oacc[db][4 * ib + 2] * inv, w.oacc[db][4 * ib + 3] * inv};
        *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * ib + 4 * w.hl) =
            __builtin_convertvector(x, bf16x4);
      }
    if (lse != nullptr && w.hl == 0)
      lse[static_cast<int64_t>(bh) * n + qrow] = (w.m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" int32_t radial_attn_fwd(const void* q, const void* k, const void* v, void* o,
                                   float* lse, const int32_t* row_ptr, const int32_t* col_idx,
                                   int32_t nb, float scale, int32_t batch, int32_t heads,
                                   int32_t seqlen, int32_t head_dim, int64_t stride_b,
                                   int64_t stride_h, int64_t stride_s, void* stream) {
  if (!q || !k || !v || !o || !row_ptr || !col_idx) return RADIAL_ERR_INVALID_ARG;
  if (batch <= 0 || heads <= 0 || seqlen <= 0 || nb <= 0) return RADIAL_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || scale < 0.f) return RADIAL_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return RADIAL_ERR_UNSUPPORTED_HEAD_DIM;
  if (nb != (seqlen + kBlock - 1) / kBlock) return RADIAL_ERR_SHAPE_MISMATCH;
  if (stride_s < head_dim || stride_h < 0 || stride_b < 0) return RADIAL_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return RADIAL_ERR_MISALIGNED;
  if ((stride_s | stride_h | stride_b) & 7) return RADIAL_ERR_MISALIGNED;
  const int64_t items = static_cast<int64_t>(batch) * heads * ((nb + 1) / 2);
  // A tile of 128 rows is addressed with 32-bit byte offsets from its first row.
  if (items > INT32_MAX || stride_s > (INT32_MAX / 2) / kBlock) return RADIAL_ERR_TOO_LARGE;

  // Base-2 score scale. It is kept >= FLT_MIN so a padding score of -inf stays -inf
  // after scaling (never -inf * 0 = NaN). For scale = 0 every finite score times FLT_MIN
  // rounds away against the running max, giving p = 2^-m for each real key: the mean of
  // V over the key set, which is the scale-0 softmax.
  const float c = fmaxf(scale * kLog2e, FLT_MIN);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<uint32_t>(items)), block(kThreads);
  const auto* qq = static_cast<const __bf16*>(q);
  const auto* kk = static_cast<const __bf16*>(k);
  const auto* vv = static_cast<const __bf16*>(v);
  auto* oo = static_cast<__bf16*>(o);
  const int ss = static_cast<int>(stride_s);
  if (head_dim == 128) {
    hipLaunchKernelGGL(radial_fwd_kernel<128>, grid, block, 0, st, qq, kk, vv, oo, lse, row_ptr,
                       col_idx, nb, heads, seqlen, c, stride_b, stride_h, ss);
  } else {
    hipLaunchKernelGGL(radial_fwd_kernel<64>, grid, block, 0, st, qq, kk, vv, oo, lse, row_ptr,
                       col_idx, nb, heads, seqlen, c, stride_b, stride_h, ss);
  }
  return hipGetLastError() == hipSuccess ? RADIAL_OK : RADIAL_ERR_HIP;
}
