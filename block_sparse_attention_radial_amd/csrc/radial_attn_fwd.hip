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
// Work decomposition. One workgroup of 8 wave64 fills one CU and computes a pair of
// query blocks (128 rows each): the pair (a, b) from a host-built pair table that puts
// together rows with many key blocks in common, or blocks 2p and 2p+1 without one. Its
// waves form two groups of four; group 0 owns row a, group 1 row b, and wave i of a
// group owns its rows 32i .. 32i+31. Both groups walk the union of the two rows'
// key-block lists in ascending order; a group skips the tiles that are not in its own
// row. Each K/V tile is thus copied to LDS once and used by both query blocks. The union
// list is built once per pair, in the prologue, into LDS.
//
// Ping-pong. A group's work per tile is an MFMA part (P*V of the previous tile, then
// Q*K^T of this tile) and a VALU part (the softmax). Group 1 runs one phase behind group
// 0, with a workgroup barrier after every phase: while one group issues MFMAs the other
// runs its softmax, so every SIMD's matrix core always has a wave feeding it. Union tile
// t is read by group 0 in phase 2t and by group 1 in phase 2t+1. Group 1 issues every
// tile copy, from its softmax phases: V(t) and K(t+1) in phase 2t, into the buffers that
// phase 2t-1 finished reading. It waits for them at the end of phase 2t+1, so a copy has
// two phases to land before group 0 reads it in phase 2t+2.
//
// Per tile:
//  - S^T = K Q^T runs on v_mfma_f32_32x32x16_bf16, with keys on M and queries on N. A
//    lane holds one query (lane % 32) and 64 of the tile's 128 keys, so row reductions
//    are in-lane, plus one v_permlane32_swap between the half-waves.
//  - O^T = V^T P^T runs on the same MFMA, with head_dim on M and queries on N. The S^T
//    accumulator is, key for key, the B operand this product needs once the contraction
//    runs over keys in accumulator order, so P goes from registers into the MFMA after
//    one bf16 pack.
//  - K and V tiles are stored key-major in LDS ([key][d], no padding). Chunk c (16
//    bytes) of row r sits at position c ^ swz(r), which spreads every read pattern below
//    over all 64 banks.
//  - V^T operands come from ds_read_b64_tr_b16. One such read gives a lane 4 keys of one
//    V column, and two of them form an MFMA operand.
//  - Tiles are copied HBM/L2 -> LDS by buffer_load ... lds, with no staging registers.
//    The descriptor's range check returns zeros past the sequence end, so the ragged
//    last block needs no guarded loads.
//  - Online softmax in base 2: c = scale * log2(e), p = 2^(c*s - m). The reference m is
//    set from the row maximum of a wave's first tile and moves only when a tile's sum of
//    p for some lane exceeds 2^20, i.e. when the scores have grown by about 20 (base 2)
//    past m. That case is found after the fact from the sum, and the tile is redone
//    with the new m (O and l rescaled). So the common path has no row maximum. The final
//    O / l is exact for any m used consistently. The row sum adds p in fp32, with plain
//    adds: v_dot2 (which could add the bf16-rounded p) runs far slower while the other
//    wave of the SIMD keeps the matrix core busy.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cfloat>
#include <cmath>
#include <climits>
#include <cstdint>
#include <atomic>
#include <mutex>

#include "../../include/radial_attn.h"
#include "radial_device.h"

namespace {

constexpr int kThreads = 512;      // 8 wave64: two groups of four
// A lane's sum of p over one tile (64 keys) above this means m is stale: rescale.
// It bounds every p by 2^20 between rescales.
constexpr float kTileSumLimit = 1048576.0f;
// Union list: one 16-bit entry per key block (kb | in-row-A << 14 | in-row-B << 15).
// A union of two rows has at most nb entries, so nb <= kMaxBlocks bounds it. With four
// 32 KiB tile buffers, the list and a few counters fill the 160 KiB of LDS.
constexpr int kMaxBlocks = 16352;
constexpr int kListBytes = kMaxBlocks * 2;
static_assert(4 * Tile<64>::kBytes >= 2 * kMaxBlocks,
              "the two key-block maps must fit in the tile buffers");

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
  int copy_off[T::kOffsetPeriod];
  // LDS read offsets of the MFMA operands: a lane part (base) plus a swizzle term that
  // is XORed with the step index (x); see the prologue.
  int k_base, k_x, v_base0, v_x0, v_base1, v_x1;
  // Q^T fragments (bf16 pairs; kept as dwords so the struct is a valid host type too)
  u32x4 qf[D / 16];
  // softmax state
  f32x16 oacc[D / 32];
  float m_run, l_run;
  bool first;  // some lane of this wave has no reference m yet
  // element rule (element masking only): frame length, W0 - 1, and the first query of
  // the group's row
  int es, egw, ew0m1, q0;
  // element table (E = 3): this wave's part of the group's next table entry, and the
  // bits of the tile in hand
  const char* etab;
  uint64_t ebits;
};

// This wave's quarter of the copy of key block kb (K or V) into buf.
template <int D>
__device__ __forceinline__ Stage<D> stage_tile(const WaveState<D>& w, char* buf, const char* src,
                                               int kb, bool on) {
  return stage_rows<D>(buf, src, kb * kBlock, w.n, w.row_bytes, w.wi, on);
}

// Issue copy instruction t of a pending tile copy.
template <int D>
__device__ __forceinline__ void stage_issue(const WaveState<D>& w, const Stage<D>& st, int t) {
  stage_issue<D>(st, w.copy_off, t);
}

// The MFMA phase of one group for union tile t: O += P(t-1) V(t-1) (when PV), then
// S(t) = Q K(t)^T (when QK). LDS reads run ahead of the MFMAs that consume them: the V^T
// fragments of step u + 1 are read while the MFMAs of step u issue (two transposed
// reads between consecutive MFMAs), and K fragments of step s + 2 are read while the
// MFMAs of step s issue (one read between consecutive MFMAs). The sched_group_barrier
// sequences pin that interleaving against the scheduler's wish to save registers or to
// bunch the reads; spreading the reads keeps the LDS pipe busy without stalling MFMA
// issue. At most 15 LDS reads can be outstanding per wave.
template <int D, bool PV, bool QK>
__device__ __forceinline__ void mfma_phase(WaveState<D>& w, const char* vbuf, const char* kbuf,
                                           const bf16x8 (&pk)[8], f32x16 (&sacc)[4]) {
  using T = Tile<D>;
  constexpr int NDB = D / 32;  // d tiles of O^T
  constexpr int NS = D / 16;   // k-steps of S^T
  constexpr int R = 2 * NDB;   // transposed reads per PV step
  // The swizzle terms go through an empty asm so that the compiler recomputes the read
  // addresses in every phase (a few XORs) instead of keeping 2 x 8 of them in registers
  // across the loop.
  int vx0 = w.v_x0, vx1 = w.v_x1, kx = w.k_x;
  asm volatile("" : "+v"(vx0), "+v"(vx1), "+v"(kx));
  const char* vb0 = vbuf + w.v_base0;
  const char* vb1 = vbuf + w.v_base1;
  const char* kb = kbuf + w.k_base;
  auto read_v = [&](int u, bf16x8 (&vf)[NDB]) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(vb0 + 16 * u * T::kRowBytes + ((db << 6) ^ vx0)));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(vb1 + 16 * u * T::kRowBytes + ((db << 6) ^ vx1)));
      vf[db] = __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo),
                                       __builtin_bit_cast(bf16x4, hi), 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  auto read_k = [&](int s, bf16x8 (&kf)[4]) {
    const int ch = (s << 5) ^ kx;
#pragma unroll
    for (int g = 0; g < 4; ++g)
      kf[g] = *reinterpret_cast<const bf16x8*>(kb + g * 32 * T::kRowBytes + ch);
  };
  bf16x8 kf[2][4];
  if constexpr (PV) {
    bf16x8 vf[2][NDB];
    read_v(0, vf[0]);
    __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
#pragma unroll
    for (int u = 0; u < 8; ++u) {  // 16 keys of the contraction per step
      if (u + 1 < 8) read_v(u + 1, vf[(u + 1) & 1]);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        w.oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[u & 1][db], pk[u], w.oacc[db], 0, 0, 0);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        if (u + 1 < 8) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
    }
  }
  if constexpr (QK) {
    if constexpr (!PV) {
      read_k(0, kf[0]);
      read_k(1, kf[1]);
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // the 8 initial reads
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
      for (int g = 0; g < 4; ++g)  // the first k-step takes an inline zero accumulator
        sacc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            kf[s & 1][g], __builtin_bit_cast(bf16x8, w.qf[s]), s == 0 ? f32x16{} : sacc[g], 0, 0, 0);
      if (s + 2 < NS) read_k(s + 2, kf[s & 1]);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (s + 2 < NS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
  }
}

template <int D>
__device__ __forceinline__ void run_mfma(WaveState<D>& w, bool pv, bool qk, const char* vbuf,
                                         const char* kbuf, const bf16x8 (&pk)[8],
                                         f32x16 (&sacc)[4]) {
  if (pv) mfma_phase<D, true, false>(w, vbuf, kbuf, pk, sacc);
  if (qk) mfma_phase<D, false, true>(w, vbuf, kbuf, pk, sacc);
}

// Row maximum of c * S over this wave's tile (both half-waves), base-2 units.
template <int D>
__device__ __forceinline__ float tile_max(const WaveState<D>& w, const f32x16 (&sacc)[4]) {
  // Four independent chains (one per S^T block), then a small tree.
  float mx[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    mx[g] = sacc[g][0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx[g] = fmaxf(mx[g], sacc[g][i]);
  }
  return halves_max(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]))) * w.c;
}

// p = 2^(c s - m) for this lane's 64 scores, packed as bf16 into pk (the B operands of
// the PV steps: pk[u] holds the 8 p of accumulator entries 8 (u & 1) .. + 7 of S^T block
// u >> 1). Returns the lane's sum of p (fp32). hook(u) runs after each step.
template <int D, int E, typename Hook>
__device__ __forceinline__ float tile_p(const WaveState<D>& w, const f32x16 (&sacc)[4],
                                        bf16x8 (&pk)[8], Hook&& hook) {
  // With element masking a lane can still lack m (every key so far masked, m = -inf);
  // its scores are all -inf too, and m = 0 keeps their p at 0 rather than NaN.
  const float neg_m = E != 0 && w.m_run == -INFINITY ? 0.f : -w.m_run;
  // Four independent partial sums (one per step mod 4), each fed by a small tree, so
  // that the adds do not form one long dependency chain.
  float lt[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int g = u >> 1, s2 = u & 1;
    f32x8 p8;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
      p8[jj] = __builtin_amdgcn_exp2f(fmaf(sacc[g][8 * s2 + jj], w.c, neg_m));
    pk[u] = __builtin_convertvector(p8, bf16x8);
    const float a0 = p8[0] + p8[1], a1 = p8[2] + p8[3], a2 = p8[4] + p8[5], a3 = p8[6] + p8[7];
    lt[u & 3] += (a0 + a1) + (a2 + a3);
    hook(u);
  }
  return (lt[0] + lt[1]) + (lt[2] + lt[3]);
}

// Element masking of union tile kb (E = 1: 1-D distance, E = 2: grid distance): this
// wave's queries on the lanes, the tile's keys on the entries.
template <int D, int E>
__device__ __forceinline__ void element_mask(const WaveState<D>& w, int kb, f32x16 (&sacc)[4]) {
  element_mask_any<E>(w.q0 + 32 * w.wi, kb * kBlock, w.es, w.egw, w.ew0m1, w.lane, sacc);
}

// Softmax of union tile kb: mask padding keys (and, with E, disallowed entries), turn S
// into P (pk), and fold the tile into the running row sum. The first tile of a wave sets
// m from its row maximum. Later tiles use the m they find; if a lane's tile sum then
// exceeds kTileSumLimit (or is not finite), m is moved to the new row maximum, O and l
// are rescaled and P is redone. With E a lane whose keys have all been masked so far
// has m = -inf and takes m from the first tile that gives it a finite maximum.
template <int D, int E, typename Hook>
__device__ __forceinline__ void softmax_tile(WaveState<D>& w, int kb, f32x16 (&sacc)[4],
                                             bf16x8 (&pk)[8], Hook&& hook) {
  // Keys at or past n (only in the last key block) are padding.
  if (w.n - kb * kBlock < kBlock) pad_mask_tile(kb * kBlock, w.n, w.lane, sacc);
  if constexpr (E == 3)
    element_mask_stored(w.ebits, sacc);
  else if constexpr (E != 0)
    element_mask<D, E>(w, kb, sacc);
  if (w.first) {
    if constexpr (E != 0) {
      const float tm = tile_max(w, sacc);
      if (w.m_run == -INFINITY) w.m_run = tm;
      w.first = __builtin_amdgcn_ballot_w64(w.m_run == -INFINITY) != 0;
    } else {
      w.m_run = tile_max(w, sacc);
      w.first = false;
    }
  }
  float lt = tile_p<D, E>(w, sacc, pk, hook);
  if (__builtin_amdgcn_ballot_w64(!(lt <= kTileSumLimit)) != 0) {
    const float m_new = fmaxf(w.m_run, tile_max(w, sacc));
    // A lane still without m (both -inf) keeps its zero O and l.
    const float alpha = E != 0 && m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(w.m_run - m_new);
    w.m_run = m_new;
    w.l_run *= alpha;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) w.oacc[i] *= alpha;
    lt = tile_p<D, E>(w, sacc, pk, [](int) {});
  }
  w.l_run += lt;
}

// Most marking steps per row that radial_attn_fwd_rule accepts.
constexpr int64_t kMaxRuleSteps = 1 << 16;

typedef __attribute__((address_space(1))) const uint64_t GlobalU64;

// Bytes of one element-table entry: the 128 x 128 decisions of an active block, 64 bits
// per lane of each of the four query waves (element_mask_stored's layout).
constexpr int kTableEntryBytes = 2048;

// Union-list entry bits.
constexpr uint32_t kInA = 1u << 14, kInB = 1u << 15, kKbMask = kInA - 1;

// The radial rule for deriving a row's key blocks in the kernel instead of reading them
// from a CSR: frames of s tokens as grids of gw columns (gw = s for the 1-D distance),
// base window w0. s = 0: the mask is read from the CSR.
struct MaskRule {
  int s, gw, w0;
};
typedef __attribute__((address_space(4))) const MaskRule* RulePtr;

// Sets f[kb] for the key blocks of columns [lo, hi] (clipped to the row) of the grid row
// whose first token is row0.
__device__ __forceinline__ void mark_run(uint8_t* f, int row0, int lo, int hi, int gw) {
  lo = max(lo, 0);
  hi = min(hi, gw - 1);
  if (lo > hi) return;
  for (int kb = (row0 + lo) / kBlock; kb <= (row0 + hi) / kBlock; ++kb) f[kb] = 1;
}

// Marks in f the key blocks of query block `row` under the radial rule (the same sweep
// as the host builder, radial_build_mask_grid): for a query frame f_q, a key frame f_k
// at band k and a key grid row y, the radius is r = (W0 - 1) >> k, and the row is
// reached in at most two runs of columns, from the query block's partial first grid
// row, its whole middle rows and its partial last row. One (query frame piece, key
// frame, key row) per thread and step; byte marks are idempotent, so threads that mark
// the same block do not conflict. n = F * s tokens. Kept out of line: it runs once per
// item, and inlined its integer divisions would crowd the item loop's registers.
__device__ __noinline__ void mark_rule_row(uint8_t* f, int row, int n, int s, int gw, int w0,
                                           int tid) {
  const int frames = n / s, rows = s / gw;
  const int t0 = row * kBlock, t1 = min(n, t0 + kBlock);
  const int fq0 = t0 / s, fq1 = (t1 - 1) / s;
  const int per_piece = frames * rows;
  const int items = (fq1 - fq0 + 1) * per_piece;
  for (int it = tid; it < items; it += kThreads) {
    const int p = it / per_piece, rem = it - p * per_piece;
    const int fk = rem / rows, yk = rem - fk * rows;
    const int fq = fq0 + p;
    const int a = max(t0 - fq * s, 0), b = min(t1 - fq * s, s) - 1;  // the piece, in frame
    const int ya = a / gw, xa = a - ya * gw, yb = b / gw, xb = b - yb * gw;
    const int d = fq > fk ? fq - fk : fk - fq;
    const int r = min((w0 - 1) >> (31 - __builtin_clz(static_cast<unsigned>(d) + 1u)),
                      kMaxReach);
    const int ta = r - (yk > ya ? yk - ya : ya - yk);
    const int tb = r - (yk > yb ? yk - yb : yb - yk);
    const int row0 = fk * s + yk * gw;
    if (ya == yb) {
      if (ta >= 0) mark_run(f, row0, xa - ta, xb + ta, gw);
      continue;
    }
    const int dm = yk <= ya ? ya + 1 - yk : (yk >= yb ? yk - yb + 1 : 0);
    if (yb - ya >= 2 && dm <= r) {  // a whole middle row is within reach
      mark_run(f, row0, 0, gw - 1, gw);
      continue;
    }
    if (ta >= 0) mark_run(f, row0, xa - ta, gw - 1, gw);
    if (tb >= 0) mark_run(f, row0, 0, xb + tb, gw);
  }
}

// The phase loop of group G (G = 0: query block 2p, G = 1: query block 2p+1) over the U
// union tiles. Phase 2t is group 0's MFMA phase for tile t and group 1's softmax phase
// for tile t-1; phase 2t+1 is the other way round. Each phase ends at a workgroup
// barrier, and both groups pass 2U + 2 of them.
//   group 0, MFMA t (phase 2t):        O += P(t-1) V(t-1); S(t) = Q K(t)^T
//   group 0, softmax t (phase 2t+1):   softmax of tile t
//   group 1, MFMA t (phase 2t+1):      O += P(t-1) V(t-1); S(t) = Q K(t)^T; wait for this
//                                      wave's copies
//   group 1, softmax t (phase 2t+2):   copy V(t+1) and K(t+2); softmax of tile t
// Phase 0 is group 1's copy of V(0) and K(1). Tile t lives in K buffer t % 2 and V buffer
// t % 2; the copies of phase 2t overwrite tiles t-1 (K) and t-2 (V), whose last reads were
// in phase 2t-1. One loop iteration runs tile t's MFMA phase and then its softmax, so S
// is live only inside an iteration; P is carried to the next iteration's P V.
template <int D, int G, int E>
__device__ __forceinline__ void run_group(WaveState<D>& w, const uint16_t* list, int U,
                                          char* __restrict__ k0, char* __restrict__ k1,
                                          char* __restrict__ v0, char* __restrict__ v1) {
  constexpr uint32_t kMine = G == 0 ? kInA : kInB;
  bf16x8 pk[8];  // P(t) after a softmax phase
  auto pick = [](int t, char* b0, char* b1) { return (t & 1) ? b1 : b0; };
  // List entries are the same in every lane: readfirstlane keeps them (and every branch
  // on them) scalar.
  auto entry = [&](int t) -> uint32_t {
    return t < U ? static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(list[t])) : 0u;
  };
  // Group 1's copies of V(t) and K(t + 1), two instructions per softmax step: V in the
  // first half, K in the second. A copy past the last tile gets a descriptor of zero
  // bytes: its loads fetch nothing and write zeros into a buffer that is free (it held
  // tile t-2 or t-1), which keeps the copy code free of branches.
  auto copies = [&](int t, uint32_t e_t, uint32_t e_t1) {
    const Stage<D> sv = stage_tile(w, pick(t, v0, v1), w.vh, static_cast<int>(e_t & kKbMask), t < U);
    const Stage<D> sk =
        stage_tile(w, pick(t + 1, k0, k1), w.kh, static_cast<int>(e_t1 & kKbMask), t + 1 < U);
    return [=, &w](int u) {
      __builtin_amdgcn_sched_barrier(0);
      constexpr int C = Tile<D>::kCopiesPerWave;
      const int i0 = 2 * u, i1 = 2 * u + 1;
      stage_issue(w, i0 < C ? sv : sk, i0 < C ? i0 : i0 - C);
      stage_issue(w, i1 < C ? sv : sk, i1 < C ? i1 : i1 - C);
      __builtin_amdgcn_sched_barrier(0);
    };
  };
  uint32_t e_prev = 0, e_cur = entry(0), e_next = entry(1);
  if constexpr (G == 1) {
    // ---- phase 0: copy V(0), K(1) ----
    const auto hook = copies(0, e_cur, e_next);
#pragma unroll
    for (int u = 0; u < 8; ++u) hook(u);
    lds_barrier();
  }
  for (int t = 0; t <= U; ++t) {
    const bool prev_mine = (e_prev & kMine) != 0;  // e_prev = 0 for t = 0
    const bool cur_mine = t < U && (e_cur & kMine) != 0;
    f32x16 sacc[4];  // S(t)
    if constexpr (E == 3) {
      // This wave's stored bits of tile t (the next entry of the group's row), loaded
      // under the MFMA phase. Group 1's wait for its copies at the end of the phase
      // covers the load; group 0 has no other vector-memory load in flight.
      if (cur_mine) {
        // (A global load from a scalar base: a generic pointer would make it a flat load,
        // which the LDS waits of the MFMA phase would count too.)
        const char* entry = w.etab;
        asm volatile("" : "+s"(entry));
        w.ebits = *(GlobalU64*)(entry + w.lane * 8);
        w.etab = entry + kTableEntryBytes;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- MFMA phase of tile t ----
    __builtin_amdgcn_s_setprio(1);
    run_mfma(w, prev_mine, cur_mine, pick(t - 1, v0, v1), pick(t, k0, k1), pk, sacc);
    const uint32_t e_next2 = entry(t + 2);  // its LDS latency hides behind the MFMAs
    if constexpr (G == 1) wait_copies<0>();  // V(t) and K(t+1) are in LDS
    lds_barrier();
    if (t == U) break;
    // ---- softmax phase of tile t ----
    __builtin_amdgcn_s_setprio(0);
    if constexpr (G == 0) {
      if (cur_mine) softmax_tile<D, E>(w, static_cast<int>(e_cur & kKbMask), sacc, pk, [](int) {});
    } else {
      const auto hook = copies(t + 1, e_next, e_next2);
      if (cur_mine) {
        softmax_tile<D, E>(w, static_cast<int>(e_cur & kKbMask), sacc, pk, hook);
      } else {
#pragma unroll
        for (int u = 0; u < 8; ++u) hook(u);
      }
    }
    lds_barrier();
    e_prev = e_cur;
    e_cur = e_next;
    e_next = e_next2;
  }
  if constexpr (G == 0) lds_barrier();  // group 1's last phase
  __builtin_amdgcn_s_setprio(0);
}

// One work item: the two query-block rows of pair `pair` (from the pair table, or 2p and
// 2p+1) of one (batch, head). q, k, v, o point at row 0 of this (batch, head), lse (if
// not null) at its row 0's entry. smem holds two K and two V buffers at fixed offsets,
// then the union list; counts holds the per-wave sums of the list compaction, then the
// union length. The host orders the pair table so that neighbouring pairs have nearly
// equal length and lie close in the sequence: taken together by one XCD, they walk their
// lists in step and share that XCD's L2 (radial_build_pairs).
template <int D, int E>
__device__ __forceinline__ void run_item(
    int pair, int tid, char* smem, int* counts, const __bf16* __restrict__ q,
    const __bf16* __restrict__ k, const __bf16* __restrict__ v, __bf16* __restrict__ o,
    float* __restrict__ lse, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, const int32_t* __restrict__ pairs, int nb, int n,
    float c, int stride_s, int es, int egw, int ew0, RulePtr rule, const char* etab) {
  using T = Tile<D>;
  char* const k0 = smem;
  char* const k1 = smem + T::kBytes;
  char* const v0 = smem + 2 * T::kBytes;
  char* const v1 = smem + 3 * T::kBytes;
  uint16_t* const list = reinterpret_cast<uint16_t*>(smem + 4 * T::kBytes);

  // The pair's rows. A row outside [0, nb) (the second row of an odd nb's last pair, or
  // an absent entry of the table) adds no key blocks and has no queries: -1.
  int ra = 2 * pair, rb = 2 * pair + 1;
  if (pairs != nullptr) {
    ra = pairs[2 * pair];
    rb = pairs[2 * pair + 1];
  }
  ra = static_cast<unsigned>(ra) < static_cast<unsigned>(nb) ? ra : -1;
  rb = static_cast<unsigned>(rb) < static_cast<unsigned>(nb) ? rb : -1;

  // The wave index is the same in every lane; saying so lets it live in a scalar
  // register (it feeds M0, the LDS base of the tile copies).
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;                 // group 0: row ra, group 1: row rb
  const int q0 = (grp == 0 ? ra : rb) >= 0  // first query of the group's row; n: none
                     ? (grp == 0 ? ra : rb) * kBlock
                     : n;

  // ---- union list of the two rows ----
  // The rows' key blocks are marked in two byte maps over [0, nb) (in the tile buffers,
  // which are free until the first copy), from the CSR or, with a rule, derived here;
  // then every thread compacts a contiguous run of nb / 512 key blocks into the list at
  // its offset from a workgroup prefix sum. The list comes out ascending, each block
  // once; column indices outside [0, nb) are skipped.
  {
    const int lane = tid & 63, wv = tid >> 6;
    uint8_t* const fa = reinterpret_cast<uint8_t*>(smem);
    uint8_t* const fb = fa + kMaxBlocks;
    for (int i = tid; i < 2 * kMaxBlocks / 16; i += kThreads)
      reinterpret_cast<u32x4*>(smem)[i] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
    const int rule_s = rule->s;
    if (rule_s > 0) {
      if (ra >= 0) mark_rule_row(fa, ra, n, rule_s, rule->gw, rule->w0, tid);
      if (rb >= 0) mark_rule_row(fb, rb, n, rule_s, rule->gw, rule->w0, tid);
    } else {
      const int a0 = ra >= 0 ? row_ptr[ra] : 0, a1 = ra >= 0 ? row_ptr[ra + 1] : 0;
      const int b0 = rb >= 0 ? row_ptr[rb] : 0, b1 = rb >= 0 ? row_ptr[rb + 1] : 0;
      for (int i = a0 + tid; i < a1; i += kThreads) {
        const int x = col_idx[i];
        if (static_cast<unsigned>(x) < static_cast<unsigned>(nb)) fa[x] = 1;
      }
      for (int i = b0 + tid; i < b1; i += kThreads) {
        const int x = col_idx[i];
        if (static_cast<unsigned>(x) < static_cast<unsigned>(nb)) fb[x] = 1;
      }
    }
    __syncthreads();
    const int per = (nb + kThreads - 1) / kThreads;
    const int k_lo = min(tid * per, nb), k_hi = min(k_lo + per, nb);
    int cnt = 0;
    for (int kk = k_lo; kk < k_hi; ++kk) cnt += (fa[kk] | fb[kk]) != 0;
    int incl = cnt;  // inclusive prefix sum over the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    if (lane == 63) counts[wv] = incl;
    __syncthreads();
    int pos = incl - cnt;
    for (int w2 = 0; w2 < wv; ++w2) pos += counts[w2];
    for (int kk = k_lo; kk < k_hi; ++kk) {
      const uint32_t f = fa[kk] | (fb[kk] << 1);
      if (f) list[pos++] = static_cast<uint16_t>(kk | (f & 1 ? kInA : 0u) | (f & 2 ? kInB : 0u));
    }
    if (tid == kThreads - 1) counts[8] = pos;
    __syncthreads();  // the list is complete and the byte maps are free again
  }
  const int U = counts[8];

  WaveState<D> w;
  w.kh = reinterpret_cast<const char*>(k);
  w.vh = reinterpret_cast<const char*>(v);
  w.nb = nb;
  w.n = n;
  w.c = c;
  w.row_bytes = stride_s * 2;
  w.wi = wave & 3;  // query rows 32 wi .. 32 wi + 31
  w.lane = tid & 63;
  const int lq = w.lane & 31;  // query column owned by this lane
  w.hl = w.lane >> 5;          // half-wave

  // ---- tile copies: this wave's quarter of a tile, 1 KiB per instruction ----
  copy_offsets<D>(w.wi, w.lane, w.row_bytes, w.copy_off);

  // Prologue copy: K of union tile 0, by group 0. The compiler does not see the tile
  // copies, so a barrier never waits for them by itself: every wait for a copy is
  // explicit.
  if (grp == 0 && U > 0) {
    const int kb0 = __builtin_amdgcn_readfirstlane(list[0]) & kKbMask;
    const Stage<D> st = stage_tile(w, k0, w.kh, kb0, true);
#pragma unroll
    for (int t = 0; t < T::kCopiesPerWave; ++t) stage_issue(w, st, t);
  }

  // ---- Q^T as the MFMA B operand: d = 16s + 8hl .. +7 of this lane's query ----
  {
    const int rows = n - q0 < kBlock ? n - q0 : kBlock;
    const auto rq = make_rsrc(q + static_cast<int64_t>(q0 < n ? q0 : 0) * stride_s,
                              rows > 0 ? (rows - 1) * w.row_bytes + T::kRowBytes : 0);
    const int off = (w.wi * 32 + lq) * w.row_bytes + w.hl * 16;
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      w.qf[s] = buffer_load16(rq, off + s * 32);
    // Wait for Q (and the K(0) copy) here, where the compiler sees it. Otherwise its
    // wait-count bookkeeping carries the Q loads into the phase loop as pending and
    // waits on the vector-memory counter there, i.e. on the tile copies.
    __builtin_amdgcn_s_waitcnt(0);
  }

  // ---- per-lane LDS read offsets for the MFMA operands (bytes) ----
  // K (A operand of S^T) by row reads, V^T (A operand of O^T) by transposed reads.
  row_read_offsets<D>(w.lane, w.k_base, w.k_x);
  tr_read_offsets<D>(w.lane, w.v_base0, w.v_x0, w.v_base1, w.v_x1);

#pragma unroll
  for (int i = 0; i < D / 32; ++i) w.oacc[i] = f32x16{};
  // reference max of c * s, base-2 units (set by the first tile; -inf = not yet, which
  // element masking can prolong)
  w.m_run = E != 0 ? -INFINITY : 0.f;
  w.l_run = 0.f;   // sum of p over this lane's keys
  w.first = true;
  w.es = es;
  w.egw = egw;
  w.ew0m1 = ew0 - 1;
  w.q0 = q0;
  if constexpr (E == 3) {
    // The table's entries follow the CSR: entry row_ptr[r] + i is the i-th key block of
    // row r, whose union tiles come in the same ascending order.
    const int r = grp == 0 ? ra : rb;
    const int first = __builtin_amdgcn_readfirstlane(r >= 0 ? row_ptr[r] : 0);
    w.etab = etab + (static_cast<int64_t>(first) * kTableEntryBytes +
                     w.wi * (kTableEntryBytes / 4));
    w.ebits = ~0ull;
  }

  __syncthreads();  // K(0) is in LDS
  if (grp == 0)
    run_group<D, 0, E>(w, list, U, k0, k1, v0, v1);
  else
    run_group<D, 1, E>(w, list, U, k0, k1, v0, v1);

  // ---- epilogue: O / l, bf16, store rows < n ----
  const float l_tot = halves_sum(w.l_run);
  const float inv = 1.0f / l_tot;
  const int qrow = q0 + w.wi * 32 + lq;
  if (qrow < n) {
    __bf16* orow = o + static_cast<int64_t>(qrow) * stride_s;
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
      lse[qrow] = (w.m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
  }
}

// This lane's index in the wave, as a new value on every call: volatile asm is neither
// hoisted out of loops nor merged, so nothing derived from it stays live across a loop.
__device__ __forceinline__ int lane_id_fresh() {
  int lane;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  return lane;
}

// Work counters: slot s serves one launch. Entries 0..7 hand out the items of each XCD,
// entry 8 counts the workgroups that have finished. The loader zero-fills the array,
// and every launch leaves its slot at zero again.
constexpr int kCounterSlots = 256;
__device__ int g_work[kCounterSlots][16];

// Persistent grid: one workgroup per CU (a multiple of 8 workgroups). The hardware
// deals workgroup ids to the 8 XCDs round-robin, so workgroup i runs on XCD i % 8 and
// takes the items of its XCD x's list from counter x, in order, until they run out;
// then it helps the other XCDs, taking from counters x + 1, x + 2, ... (mod 8) in turn.
// The lists come from XCD groups (xg in FwdArgs): the XCDs form 8 / xg groups of xg;
// group g takes the (batch, head)s g, g + 8 / xg, ... one after another (for a varlen
// batch: those heads of sample 0, then of sample 1, ...), and each XCD of the group one
// contiguous run of a head's pair table, the run rotating from head to head. A CU that
// finishes early takes the next item at once: with one workgroup per item, the
// dispatcher left CUs idle between workgroups and the last CUs finished whole items
// after the rest, and under the chip's power limit the XCDs run at different clocks, so
// a fixed share per XCD left the faster ones idle at the end. The last workgroup to
// finish resets the counters.
// One sample of a varlen batch: its first token in the packed sequence, its tokens and
// query blocks, where its row_ptr array starts in the concatenated one, where its pairs
// start in the concatenated pair table, its pair count, its first work item, and its
// first entry in every XCD's list.
struct VarlenSample {
  int tok0, n, nb, rp0, pr0, np, it0, lo;
};
constexpr int kMaxVarlen = 64;

struct FwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const int32_t* pairs;
  int64_t stride_b, stride_h;
  int npairs, nb, heads, n, stride_s;
  int elem_s, elem_gw, elem_w0;
  MaskRule rule;  // rule.s > 0: key blocks derived in the kernel (row_ptr/col_idx unused)
  float c;
  int items, slot;
  // varlen: 0 for a uniform batch, else the number of samples in `plan` (q, k, v, o are
  // then one packed sequence of n tokens, and lse is [heads, n])
  int varlen;
  VarlenSample plan[kMaxVarlen];
  // XCDs per group (1, 2, 4 or 8); for a uniform batch the pairs of one XCD's run of a
  // head (ceil(npairs / xg)) and batch * heads, for a varlen batch the entries of every
  // XCD's list.
  int xg, run_len, bh_total, list_len;
  // element table (radial_build_element_table) for element masking from stored bits, or
  // null
  const uint64_t* etab;
};
typedef __attribute__((address_space(4))) const FwdArgs* ArgsPtr;

// Field-by-field copy out of the kernel-argument segment (scalar loads).
__device__ __forceinline__ FwdArgs load_args(ArgsPtr ap) {
  FwdArgs a;
  a.q = ap->q;
  a.k = ap->k;
  a.v = ap->v;
  a.o = ap->o;
  a.lse = ap->lse;
  a.row_ptr = ap->row_ptr;
  a.col_idx = ap->col_idx;
  a.pairs = ap->pairs;
  a.npairs = ap->npairs;
  a.stride_b = ap->stride_b;
  a.stride_h = ap->stride_h;
  a.nb = ap->nb;
  a.heads = ap->heads;
  a.n = ap->n;
  a.stride_s = ap->stride_s;
  a.elem_s = ap->elem_s;
  a.elem_gw = ap->elem_gw;
  a.elem_w0 = ap->elem_w0;
  a.c = ap->c;
  a.items = ap->items;
  a.slot = ap->slot;
  a.varlen = ap->varlen;
  a.xg = ap->xg;
  a.run_len = ap->run_len;
  a.bh_total = ap->bh_total;
  a.list_len = ap->list_len;
  a.etab = ap->etab;
  return a;
}

template <int D, int E>
__global__ __launch_bounds__(kThreads, 1) void radial_fwd_kernel(const FwdArgs args) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(1024))) char smem[4 * T::kBytes + kListBytes];
  __shared__ int counts[9];
  __shared__ int next_item, next_pair;
  (void)args;
  // The arguments are read again (scalar loads from the kernel-argument segment) for
  // every item: kept in scalar registers across the item loop, they would not fit beside
  // the item's own.
  ArgsPtr ap = (ArgsPtr)(__builtin_amdgcn_kernarg_segment_ptr());
  // The thread id is rebuilt for every item from the wave index (a scalar) and the lane
  // (v_mbcnt), so that no vector register is held across the items.
  const int wave64 = __builtin_amdgcn_readfirstlane(threadIdx.x) & ~63;
  __shared__ int lists_done;  // lists x, x + 1, ... found empty (thread 0's state)
  if (threadIdx.x == 0) lists_done = 0;
  for (;;) {
    // New values for the compiler, so that nothing derived from them is hoisted out of
    // the loop and kept live across the items.
    asm volatile("" : "+s"(ap));
    const int tid = wave64 + lane_id_fresh();
    const FwdArgs a = load_args(ap);
    const int x = blockIdx.x & 7;
    if (tid == 0) {
      int item = -1, pair = 0;
      for (int e = lists_done; e < 8 && item < 0; ++e) {
        const int y = (x + e) & 7;
        if (a.varlen == 0) {
          // Entry j of list y: head round h = j / run_len of XCD group y / xg takes the
          // (batch, head) y / xg + h * (8 / xg); XCD y % xg of the group takes run
          // (y % xg + h) % xg of its pair table. Entries past the table's end (the last
          // run can be short) are skipped.
          for (;;) {
            const int j = atomicAdd(&g_work[a.slot][y], 1);
            const int h = j / a.run_len;
            const int bh = y / a.xg + (8 / a.xg) * h;
            if (bh >= a.bh_total) break;  // list y is empty
            const int p = ((y % a.xg + h) % a.xg) * a.run_len + (j - h * a.run_len);
            if (p < a.npairs) {
              item = bh * a.npairs + p;
              pair = p;
              break;
            }
          }
        } else {
          // Entry j of list y: sample s, the last whose first list entry lo is at most j
          // (plan read with scalar loads); head round h = (j - lo) / run of it, as above,
          // with the sample's run length.
          for (;;) {
            const int j = atomicAdd(&g_work[a.slot][y], 1);
            if (j >= a.list_len) break;  // list y is empty
            int lo = 0, hi = a.varlen - 1;
            while (lo < hi) {
              const int mid = (lo + hi + 1) >> 1;
              if (ap->plan[mid].lo <= j) lo = mid;
              else hi = mid - 1;
            }
            const int np = ap->plan[lo].np, run = (np + a.xg - 1) / a.xg;
            const int r = j - ap->plan[lo].lo, h = r / run;
            const int p = ((y % a.xg + h) % a.xg) * run + (r - h * run);
            if (p < np) {
              item = ap->plan[lo].it0 + (y / a.xg + (8 / a.xg) * h) * np + p;
              pair = p;
              break;
            }
          }
        }
        if (item < 0) lists_done = e + 1;
      }
      next_item = item;
      next_pair = pair;
    }
    __syncthreads();  // every wave read the previous item's id before run_item's barriers
    const int item = __builtin_amdgcn_readfirstlane(next_item);
    const int pair = __builtin_amdgcn_readfirstlane(next_pair);
    if (item < 0) break;
    // The item's (batch, head), or its sample and head.
    int64_t base;
    float* lse_row = nullptr;
    const int32_t* row_ptr = a.row_ptr;
    const int32_t* pairs = a.pairs;
    int nb = a.nb, n = a.n;
    if (a.varlen == 0) {
      const int bh = item / a.npairs;
      const int b = bh / a.heads, h = bh - b * a.heads;
      base = b * a.stride_b + h * a.stride_h;
      if (a.lse != nullptr) lse_row = a.lse + static_cast<int64_t>(bh) * n;
    } else {
      // The last sample whose first item is at most `item` (plan read from the
      // kernel-argument segment with scalar loads).
      int lo = 0, hi = a.varlen - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (ap->plan[mid].it0 <= item) lo = mid;
        else hi = mid - 1;
      }
      const int tok0 = ap->plan[lo].tok0, it0 = ap->plan[lo].it0;
      const int np = ap->plan[lo].np;
      nb = ap->plan[lo].nb;
      n = ap->plan[lo].n;
      row_ptr += ap->plan[lo].rp0;
      if (pairs != nullptr) pairs += 2 * ap->plan[lo].pr0;
      const int h = (item - it0) / np;
      base = static_cast<int64_t>(tok0) * a.stride_s + h * a.stride_h;
      if (a.lse != nullptr) lse_row = a.lse + static_cast<int64_t>(h) * a.n + tok0;
    }
    run_item<D, E>(pair, tid, smem, counts, a.q + base, a.k + base, a.v + base, a.o + base,
                   lse_row, row_ptr, a.col_idx, pairs, nb, n, a.c, a.stride_s, a.elem_s,
                   a.elem_gw, a.elem_w0, &ap->rule, reinterpret_cast<const char*>(a.etab));
  }
  if (wave64 + lane_id_fresh() == 0) {
    int* const ctr = g_work[ap->slot];
    __threadfence();  // this workgroup's last takes come before its count
    if (atomicAdd(&ctr[8], 1) == static_cast<int>(gridDim.x) - 1) {
#pragma unroll
      for (int y = 0; y <= 8; ++y) atomicExch(&ctr[y], 0);
    }
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Compute units of the current device (cached per device), or -1 on a HIP error.
int cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < kMaxDevices) {
    const int cached = cache[dev].load(std::memory_order_relaxed);
    if (cached > 0) return cached;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return -1;
  if (dev < kMaxDevices) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// One launch of the forward kernel for these arguments (slot and item count set).
int32_t launch_kernel(const FwdArgs& args, int64_t per_xcd, int head_dim, hipStream_t st) {
  const dim3 grid(static_cast<uint32_t>(8 * per_xcd)), block(kThreads);
  const int mode = args.etab != nullptr ? 3 : (args.elem_s == 0 ? 0 : (args.elem_gw == 0 ? 1 : 2));
  if (head_dim == 128) {
    if (mode == 3)
      hipLaunchKernelGGL((radial_fwd_kernel<128, 3>), grid, block, 0, st, args);
    else if (mode == 2)
      hipLaunchKernelGGL((radial_fwd_kernel<128, 2>), grid, block, 0, st, args);
    else if (mode == 1)
      hipLaunchKernelGGL((radial_fwd_kernel<128, 1>), grid, block, 0, st, args);
    else
      hipLaunchKernelGGL((radial_fwd_kernel<128, 0>), grid, block, 0, st, args);
  } else {
    if (mode == 3)
      hipLaunchKernelGGL((radial_fwd_kernel<64, 3>), grid, block, 0, st, args);
    else if (mode == 2)
      hipLaunchKernelGGL((radial_fwd_kernel<64, 2>), grid, block, 0, st, args);
    else if (mode == 1)
      hipLaunchKernelGGL((radial_fwd_kernel<64, 1>), grid, block, 0, st, args);
    else
      hipLaunchKernelGGL((radial_fwd_kernel<64, 0>), grid, block, 0, st, args);
  }
  return hipGetLastError() == hipSuccess ? RADIAL_OK : RADIAL_ERR_HIP;
}

// Counter slots. Eager calls rotate through the first half of the ring, per device. Each
// slot keeps an event recorded after the launch that last used it; a new launch on that
// slot first makes its stream wait for that event if it has not completed, so two
// kernels never use one slot at the same time, however many calls are in flight and on
// however many streams. A call made under stream capture takes a slot from the second
// half instead (a captured graph cannot wait for an event recorded outside it), so the
// slot baked into a graph is not the one of any eager call.
constexpr int kMaxDevices = 64;
constexpr uint32_t kEagerSlots = kCounterSlots / 2;
struct EagerSlots {
  std::mutex mu;
  uint32_t next = 0;
  hipEvent_t done[kEagerSlots] = {};
};
EagerSlots g_eager[kMaxDevices];
std::atomic<uint32_t> g_next_capture_slot{0};

// Bytes of K and V that the heads in flight of a uniform batch may hold: about half of
// the 256 MB Infinity Cache.
constexpr int64_t kKvInFlight = int64_t(160) << 20;

// The launch shared by the uniform and the varlen entry points: a persistent grid of one
// workgroup per CU (a multiple of 8, at most one per item) and a counter slot.
int32_t launch_fwd(FwdArgs& args, int64_t items, int head_dim, void* stream) {
  const int cus = cu_count();
  if (cus < 0) return RADIAL_ERR_HIP;
  const int64_t per_xcd = std::min<int64_t>(std::max(cus / 8, 1), (items + 7) / 8);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  if (st != nullptr && hipStreamIsCapturing(st, &capture) != hipSuccess) return RADIAL_ERR_HIP;
  args.items = static_cast<int>(items);
  if (args.varlen == 0) {
    // XCD groups: the smallest xg (XCDs per group) whose 8 / xg heads in flight keep
    // their K and V within kKvInFlight bytes of the Infinity Cache, with a head for every
    // group. Small heads then run one per XCD (each XCD's L2 serves one head, and every
    // XCD ends on the shortest pairs of its last head); large ones are shared by several
    // XCDs, so that the K and V in flight still fit the Infinity Cache.
    const int64_t bh = items / args.npairs;
    const int64_t kv = int64_t(4) * args.n * head_dim;  // bytes of one head's K and V
    int xg = 1;
    while (xg < 8 && ((8 / xg) * kv > kKvInFlight || 8 / xg > bh)) xg *= 2;
    args.xg = xg;
    args.run_len = (args.npairs + xg - 1) / xg;
    args.bh_total = static_cast<int>(bh);
  }
  if (capture == hipStreamCaptureStatusActive) {
    const uint32_t turn = g_next_capture_slot.fetch_add(1, std::memory_order_relaxed);
    args.slot = static_cast<int>(kEagerSlots + turn % kEagerSlots);
    return launch_kernel(args, per_xcd, head_dim, st);
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RADIAL_ERR_HIP;
  EagerSlots& tab = g_eager[dev];
  // Held from the choice of the slot to the event that marks its new use, so that two
  // host threads never take one slot at once.
  std::lock_guard<std::mutex> lock(tab.mu);
  const uint32_t slot = tab.next;
  hipEvent_t& done = tab.done[slot];
  if (done == nullptr) {
    if (hipEventCreateWithFlags(&done, hipEventDisableTiming) != hipSuccess) {
      done = nullptr;
      return RADIAL_ERR_HIP;
    }
  } else {
    const hipError_t q = hipEventQuery(done);
    if (q == hipErrorNotReady) {
      if (hipStreamWaitEvent(st, done, 0) != hipSuccess) return RADIAL_ERR_HIP;
    } else if (q != hipSuccess) {
      return RADIAL_ERR_HIP;
    }
  }
  args.slot = static_cast<int>(slot);
  const int32_t err = launch_kernel(args, per_xcd, head_dim, st);
  if (err != RADIAL_OK) return err;
  if (hipEventRecord(done, st) != hipSuccess) return RADIAL_ERR_HIP;
  tab.next = (slot + 1) % kEagerSlots;
  return RADIAL_OK;
}

// Checks shared by both entry points.
int32_t check_common(const void* q, const void* k, const void* v, const void* o,
                     int32_t heads, float scale,
                     int32_t element_tokens_per_frame, int32_t element_w0,
                     int32_t element_grid_w, int32_t head_dim) {
  if (!q || !k || !v || !o) return RADIAL_ERR_INVALID_ARG;
  if (heads <= 0) return RADIAL_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || scale < 0.f) return RADIAL_ERR_INVALID_ARG;
  if (!element_args_valid(element_tokens_per_frame, element_w0, element_grid_w))
    return RADIAL_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return RADIAL_ERR_UNSUPPORTED_HEAD_DIM;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return RADIAL_ERR_MISALIGNED;
  return RADIAL_OK;
}

// The per-sample plan and launch of a varlen batch: tokens[b] is sample b's length. With
// a mask rule (args.rule.s > 0) there is no CSR: each sample's row offset is 0, so
// nothing is added to the null row_ptr.
int32_t launch_varlen(FwdArgs& args, const int32_t* tokens, int32_t batch,
                      const int32_t* pairs, const int32_t* npairs, int32_t heads,
                      int32_t head_dim, void* stream) {
  const bool rule = args.rule.s > 0;
  int64_t tok = 0, rows = 0, prs = 0, items = 0, max_n = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t n = tokens[b];
    if (n <= 0) return RADIAL_ERR_INVALID_ARG;
    const int32_t nb = (n + kBlock - 1) / kBlock;
    if (nb > kMaxBlocks) return RADIAL_ERR_TOO_LARGE;
    const int32_t np = pairs == nullptr ? (nb + 1) / 2 : npairs[b];
    if (np < (nb + 1) / 2 || np > nb) return RADIAL_ERR_INVALID_ARG;
    if (tok > INT32_MAX || rows > INT32_MAX || prs > INT32_MAX || items > INT32_MAX)
      return RADIAL_ERR_TOO_LARGE;
    args.plan[b] = VarlenSample{static_cast<int>(tok), n, nb, rule ? 0 : static_cast<int>(rows),
                                static_cast<int>(prs), np, static_cast<int>(items), 0};
    tok += n;
    rows += nb + 1;
    prs += np;
    items += static_cast<int64_t>(heads) * np;
    max_n = std::max<int64_t>(max_n, n);
  }
  if (tok > INT32_MAX || items > INT32_MAX) return RADIAL_ERR_TOO_LARGE;
  args.n = static_cast<int>(tok);  // the packed sequence; lse is [heads, n]
  // XCD groups as for a uniform batch (launch_fwd), sized by the longest sample, with
  // the same number of each sample's heads for every group. Every XCD's list then holds
  // heads / (8 / xg) runs of each sample, sample by sample.
  int xg = 1;
  const int64_t kv = int64_t(4) * max_n * head_dim;
  while (xg < 8 && ((8 / xg) * kv > kKvInFlight || heads % (8 / xg) != 0)) xg *= 2;
  int64_t entries = 0;
  for (int32_t b = 0; b < batch; ++b) {
    args.plan[b].lo = static_cast<int>(entries);
    entries += static_cast<int64_t>(heads / (8 / xg)) * ((args.plan[b].np + xg - 1) / xg);
  }
  if (entries > INT32_MAX / 2) return RADIAL_ERR_TOO_LARGE;
  args.xg = xg;
  args.list_len = static_cast<int>(entries);
  return launch_fwd(args, items, head_dim, stream);
}

// Element table: one workgroup per active block (CSR entry j = blockIdx.x), one wave per
// 32 queries. Each wave runs the in-kernel element rule (element_mask_any, E = 1 or 2)
// on a tile of zeros and stores which entries it kept, 64 bits per lane: the decisions
// the forward would take for this block, in the layout element_mask_stored reads. A
// column outside [0, nb) gets no bits (the forward never visits it).
template <int E>
__global__ __launch_bounds__(256) void radial_element_table_kernel(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int nb, int S,
    int gw, int ew0m1, uint64_t* __restrict__ table) {
  const int j = blockIdx.x;
  // The row of entry j: the last r with row_ptr[r] <= j.
  int lo = 0, hi = nb - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (__builtin_amdgcn_readfirstlane(row_ptr[mid]) <= j) lo = mid;
    else hi = mid - 1;
  }
  const int qb = lo;
  const int kb = __builtin_amdgcn_readfirstlane(col_idx[j]);
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  uint64_t bits = 0;
  if (static_cast<unsigned>(kb) < static_cast<unsigned>(nb)) {
    f32x16 sacc[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) sacc[g] = f32x16{};
    element_mask_any<E>(qb * kBlock + 32 * w, kb * kBlock, S, gw, ew0m1, lane, sacc);
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (sacc[g][e] == 0.f) bits |= 1ull << (16 * g + e);
  }
  table[static_cast<int64_t>(j) * (kTableEntryBytes / 8) + w * 64 + lane] = bits;
}

// The CSR forward for radial_attn_fwd and radial_attn_fwd_element_table: etab null
// takes the element arguments (zero frame length: block semantics), else the table.
int32_t fwd_csr(const void* q, const void* k, const void* v, void* o, float* lse,
                const int32_t* row_ptr, const int32_t* col_idx, int32_t nb,
                const int32_t* pairs, int32_t npairs, float scale,
                int32_t element_tokens_per_frame, int32_t element_w0, int32_t element_grid_w,
                const void* etab, int32_t batch, int32_t heads, int32_t seqlen,
                int32_t head_dim, int64_t stride_b, int64_t stride_h, int64_t stride_s,
                void* stream) {
  if (!row_ptr || !col_idx) return RADIAL_ERR_INVALID_ARG;
  const int32_t err = check_common(q, k, v, o, heads, scale, element_tokens_per_frame,
                                   element_w0, element_grid_w, head_dim);
  if (err != RADIAL_OK) return err;
  if (batch <= 0 || seqlen <= 0 || nb <= 0) return RADIAL_ERR_INVALID_ARG;
  if (nb != (seqlen + kBlock - 1) / kBlock) return RADIAL_ERR_SHAPE_MISMATCH;
  if (stride_s < head_dim || stride_h < 0 || stride_b < 0) return RADIAL_ERR_INVALID_ARG;
  if ((stride_s | stride_h | stride_b) & 7) return RADIAL_ERR_MISALIGNED;
  if (etab != nullptr && !aligned16(etab)) return RADIAL_ERR_MISALIGNED;
  if (pairs == nullptr) npairs = (nb + 1) / 2;
  else if (npairs < (nb + 1) / 2 || npairs > nb) return RADIAL_ERR_INVALID_ARG;
  const int64_t items = static_cast<int64_t>(batch) * heads * npairs;
  // A tile of 128 rows is addressed with 32-bit byte offsets from its first row, and
  // the union list holds one 16-bit entry per key block.
  if (items > INT32_MAX || stride_s > (INT32_MAX / 2) / kBlock || nb > kMaxBlocks)
    return RADIAL_ERR_TOO_LARGE;
  FwdArgs args{static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
               static_cast<const __bf16*>(v), static_cast<__bf16*>(o), lse, row_ptr, col_idx,
               pairs, stride_b, stride_h, npairs, nb, heads, seqlen,
               static_cast<int>(stride_s), element_tokens_per_frame, element_grid_w,
               element_w0, MaskRule{0, 0, 0}, base2_scale(scale), 0, 0, 0, {}};
  args.etab = static_cast<const uint64_t*>(etab);
  return launch_fwd(args, items, head_dim, stream);
}

}  // namespace

extern "C" int32_t radial_attn_fwd(const void* q, const void* k, const void* v, void* o,
                                   float* lse, const int32_t* row_ptr, const int32_t* col_idx,
                                   int32_t nb, const int32_t* pairs, int32_t npairs, float scale,
                                   int32_t element_tokens_per_frame, int32_t element_w0,
                                   int32_t element_grid_w, int32_t batch, int32_t heads,
                                   int32_t seqlen, int32_t head_dim,
                                   int64_t stride_b, int64_t stride_h, int64_t stride_s,
                                   void* stream) {
  return fwd_csr(q, k, v, o, lse, row_ptr, col_idx, nb, pairs, npairs, scale,
                 element_tokens_per_frame, element_w0, element_grid_w, nullptr, batch, heads,
                 seqlen, head_dim, stride_b, stride_h, stride_s, stream);
}

extern "C" int32_t radial_element_table_bytes(int64_t nnz, int64_t* bytes) {
  if (bytes == nullptr || nnz < 0) return RADIAL_ERR_INVALID_ARG;
  if (nnz > INT32_MAX) return RADIAL_ERR_TOO_LARGE;
  *bytes = nnz * kTableEntryBytes;
  return RADIAL_OK;
}

extern "C" int32_t radial_build_element_table(const int32_t* row_ptr, const int32_t* col_idx,
                                              int32_t nb, int64_t nnz,
                                              int32_t element_tokens_per_frame,
                                              int32_t element_w0, int32_t element_grid_w,
                                              void* table, int64_t table_bytes,
                                              void* stream) {
  if (!row_ptr || !col_idx || !table) return RADIAL_ERR_INVALID_ARG;
  if (nb <= 0 || nnz < 0) return RADIAL_ERR_INVALID_ARG;
  if (element_tokens_per_frame == 0 ||
      !element_args_valid(element_tokens_per_frame, element_w0, element_grid_w))
    return RADIAL_ERR_INVALID_ARG;
  if (nb > kMaxBlocks || nnz > INT32_MAX) return RADIAL_ERR_TOO_LARGE;
  if (table_bytes < nnz * kTableEntryBytes) return RADIAL_ERR_CAPACITY;
  if (!aligned16(table)) return RADIAL_ERR_MISALIGNED;
  if (nnz == 0) return RADIAL_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<uint32_t>(nnz)), block(256);
  uint64_t* const t = static_cast<uint64_t*>(table);
  if (element_grid_w == 0)
    hipLaunchKernelGGL((radial_element_table_kernel<1>), grid, block, 0, st, row_ptr, col_idx,
                       nb, element_tokens_per_frame, 0, element_w0 - 1, t);
  else
    hipLaunchKernelGGL((radial_element_table_kernel<2>), grid, block, 0, st, row_ptr, col_idx,
                       nb, element_tokens_per_frame, element_grid_w, element_w0 - 1, t);
  return hipGetLastError() == hipSuccess ? RADIAL_OK : RADIAL_ERR_HIP;
}

extern "C" int32_t radial_attn_fwd_element_table(
    const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* row_ptr,
    const int32_t* col_idx, int32_t nb, const int32_t* pairs, int32_t npairs, float scale,
    const void* element_table, int32_t batch, int32_t heads, int32_t seqlen, int32_t head_dim,
    int64_t stride_b, int64_t stride_h, int64_t stride_s, void* stream) {
  if (element_table == nullptr) return RADIAL_ERR_INVALID_ARG;
  return fwd_csr(q, k, v, o, lse, row_ptr, col_idx, nb, pairs, npairs, scale, 0, 0, 0,
                 element_table, batch, heads, seqlen, head_dim, stride_b, stride_h, stride_s,
                 stream);
}

extern "C" int32_t radial_attn_fwd_rule(const void* q, const void* k, const void* v, void* o,
                                        float* lse, int32_t frames, int32_t tokens_per_frame,
                                        int32_t grid_w, int32_t w0, int32_t element,
                                        const int32_t* pairs, int32_t npairs, float scale,
                                        int32_t batch, int32_t heads, int32_t head_dim,
                                        int64_t stride_b, int64_t stride_h, int64_t stride_s,
                                        void* stream) {
  // The rule itself: frames of tokens_per_frame tokens (grids of grid_w columns, or one
  // row for grid_w = 0), W0 >= 1.
  if (frames <= 0 || tokens_per_frame <= 0 || w0 <= 0 || grid_w < 0)
    return RADIAL_ERR_INVALID_ARG;
  if (grid_w > 0 && tokens_per_frame % grid_w != 0) return RADIAL_ERR_INVALID_ARG;
  const int64_t n = static_cast<int64_t>(frames) * tokens_per_frame;
  if (n > static_cast<int64_t>(kMaxBlocks) * kBlock) return RADIAL_ERR_TOO_LARGE;
  // A workgroup marks a row in (query frame pieces) x frames x grid rows steps; bound it
  // (realistic videos need a few thousand) so that no shape makes the marking crawl.
  const int64_t pieces = std::min<int64_t>(frames, (kBlock - 1) / tokens_per_frame + 2);
  const int64_t rows = grid_w > 0 ? tokens_per_frame / grid_w : 1;
  if (pieces * frames * rows > kMaxRuleSteps) return RADIAL_ERR_TOO_LARGE;
  const int32_t seqlen = static_cast<int32_t>(n);
  const int32_t err = check_common(q, k, v, o, heads, scale,
                                   element ? tokens_per_frame : 0, w0, grid_w, head_dim);
  if (err != RADIAL_OK) return err;
  if (batch <= 0) return RADIAL_ERR_INVALID_ARG;
  const int32_t nb = (seqlen + kBlock - 1) / kBlock;
  if (stride_s < head_dim || stride_h < 0 || stride_b < 0) return RADIAL_ERR_INVALID_ARG;
  if ((stride_s | stride_h | stride_b) & 7) return RADIAL_ERR_MISALIGNED;
  if (pairs == nullptr) npairs = (nb + 1) / 2;
  else if (npairs < (nb + 1) / 2 || npairs > nb) return RADIAL_ERR_INVALID_ARG;
  const int64_t items = static_cast<int64_t>(batch) * heads * npairs;
  if (items > INT32_MAX || stride_s > (INT32_MAX / 2) / kBlock) return RADIAL_ERR_TOO_LARGE;
  FwdArgs args{static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
               static_cast<const __bf16*>(v), static_cast<__bf16*>(o), lse, nullptr, nullptr,
               pairs, stride_b, stride_h, npairs, nb, heads, seqlen,
               static_cast<int>(stride_s), element ? tokens_per_frame : 0, grid_w, w0,
               MaskRule{tokens_per_frame, grid_w > 0 ? grid_w : tokens_per_frame, w0},
               base2_scale(scale), 0, 0, 0, {}};
  return launch_fwd(args, items, head_dim, stream);
}

namespace {

// The CSR varlen forward for radial_attn_fwd_varlen and
// radial_attn_fwd_varlen_element_table: etab null takes the element arguments, else the
// table (the samples' tables concatenated like their CSRs).
int32_t fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                   const int32_t* seq_tokens, int32_t batch, const int32_t* row_ptr,
                   const int32_t* col_idx, const int32_t* pairs, const int32_t* npairs,
                   float scale, int32_t element_tokens_per_frame, int32_t element_w0,
                   int32_t element_grid_w, const void* etab, int32_t heads, int32_t head_dim,
                   int64_t stride_h, int64_t stride_s, void* stream) {
  if (!row_ptr || !col_idx) return RADIAL_ERR_INVALID_ARG;
  const int32_t err = check_common(q, k, v, o, heads, scale, element_tokens_per_frame,
                                   element_w0, element_grid_w, head_dim);
  if (err != RADIAL_OK) return err;
  if (!seq_tokens || batch <= 0 || (pairs != nullptr && npairs == nullptr))
    return RADIAL_ERR_INVALID_ARG;
  if (batch > kMaxVarlen) return RADIAL_ERR_TOO_LARGE;
  if (stride_s < head_dim || stride_h < 0) return RADIAL_ERR_INVALID_ARG;
  if ((stride_s | stride_h) & 7) return RADIAL_ERR_MISALIGNED;
  if (etab != nullptr && !aligned16(etab)) return RADIAL_ERR_MISALIGNED;
  if (stride_s > (INT32_MAX / 2) / kBlock) return RADIAL_ERR_TOO_LARGE;
  FwdArgs args{static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
               static_cast<const __bf16*>(v), static_cast<__bf16*>(o), lse, row_ptr, col_idx,
               pairs, 0, stride_h, 0, 0, heads, 0, static_cast<int>(stride_s),
               element_tokens_per_frame, element_grid_w, element_w0, MaskRule{0, 0, 0},
               base2_scale(scale), 0, 0, batch, {}};
  args.etab = static_cast<const uint64_t*>(etab);
  return launch_varlen(args, seq_tokens, batch, pairs, npairs, heads, head_dim, stream);
}

}  // namespace

extern "C" int32_t radial_attn_fwd_varlen(const void* q, const void* k, const void* v, void* o,
                                          float* lse, const int32_t* seq_tokens, int32_t batch,
                                          const int32_t* row_ptr, const int32_t* col_idx,
                                          const int32_t* pairs, const int32_t* npairs,
                                          float scale, int32_t element_tokens_per_frame,
                                          int32_t element_w0, int32_t element_grid_w,
                                          int32_t heads, int32_t head_dim,
                                          int64_t stride_h, int64_t stride_s, void* stream) {
  return fwd_varlen(q, k, v, o, lse, seq_tokens, batch, row_ptr, col_idx, pairs, npairs, scale,
                    element_tokens_per_frame, element_w0, element_grid_w, nullptr, heads,
                    head_dim, stride_h, stride_s, stream);
}

extern "C" int32_t radial_attn_fwd_varlen_element_table(
    const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* seq_tokens,
    int32_t batch, const int32_t* row_ptr, const int32_t* col_idx, const int32_t* pairs,
    const int32_t* npairs, float scale, const void* element_table, int32_t heads,
    int32_t head_dim, int64_t stride_h, int64_t stride_s, void* stream) {
  if (element_table == nullptr) return RADIAL_ERR_INVALID_ARG;
  return fwd_varlen(q, k, v, o, lse, seq_tokens, batch, row_ptr, col_idx, pairs, npairs, scale,
                    0, 0, 0, element_table, heads, head_dim, stride_h, stride_s, stream);
}

extern "C" int32_t radial_attn_fwd_varlen_rule(
    const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* frames,
    int32_t batch, int32_t tokens_per_frame, int32_t grid_w, int32_t w0, int32_t element,
    const int32_t* pairs, const int32_t* npairs, float scale, int32_t heads, int32_t head_dim,
    int64_t stride_h, int64_t stride_s, void* stream) {
  if (tokens_per_frame <= 0 || w0 <= 0 || grid_w < 0) return RADIAL_ERR_INVALID_ARG;
  if (grid_w > 0 && tokens_per_frame % grid_w != 0) return RADIAL_ERR_INVALID_ARG;
  const int32_t err = check_common(q, k, v, o, heads, scale,
                                   element ? tokens_per_frame : 0, w0, grid_w, head_dim);
  if (err != RADIAL_OK) return err;
  if (!frames || batch <= 0 || (pairs != nullptr && npairs == nullptr))
    return RADIAL_ERR_INVALID_ARG;
  if (batch > kMaxVarlen) return RADIAL_ERR_TOO_LARGE;
  if (stride_s < head_dim || stride_h < 0) return RADIAL_ERR_INVALID_ARG;
  if ((stride_s | stride_h) & 7) return RADIAL_ERR_MISALIGNED;
  if (stride_s > (INT32_MAX / 2) / kBlock) return RADIAL_ERR_TOO_LARGE;
  int32_t tokens[kMaxVarlen];
  const int64_t rows = grid_w > 0 ? tokens_per_frame / grid_w : 1;
  for (int32_t b = 0; b < batch; ++b) {
    if (frames[b] <= 0) return RADIAL_ERR_INVALID_ARG;
    const int64_t n = static_cast<int64_t>(frames[b]) * tokens_per_frame;
    if (n > static_cast<int64_t>(kMaxBlocks) * kBlock) return RADIAL_ERR_TOO_LARGE;
    const int64_t pieces = std::min<int64_t>(frames[b], (kBlock - 1) / tokens_per_frame + 2);
    if (pieces * frames[b] * rows > kMaxRuleSteps) return RADIAL_ERR_TOO_LARGE;
    tokens[b] = static_cast<int32_t>(n);
  }
  FwdArgs args{static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
               static_cast<const __bf16*>(v), static_cast<__bf16*>(o), lse, nullptr, nullptr,
               pairs, 0, stride_h, 0, 0, heads, 0, static_cast<int>(stride_s),
               element ? tokens_per_frame : 0, grid_w, w0,
               MaskRule{tokens_per_frame, grid_w > 0 ? grid_w : tokens_per_frame, w0},
               base2_scale(scale), 0, 0, batch, {}};
  return launch_varlen(args, tokens, batch, pairs, npairs, heads, head_dim, stream);
}
