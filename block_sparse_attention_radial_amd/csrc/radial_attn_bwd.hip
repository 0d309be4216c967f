// Backward pass of block-sparse Radial Attention for gfx950 (CDNA4): dQ, dK, dV.
//
// The pages fine-tune the video models through the attention with LoRA (the
// radial-attention-video SKILL.md page, Step 4: loss.backward() through the attention
// layers), which needs the gradient of the forward pass over the same block mask. Per
// query row i with key set K_i, P = softmax(scale q_i K^T) and o_i = P V, so
//   D_i = <do_i, o_i>,  dP_ij = <do_i, v_j>,  dS_ij = P_ij (dP_ij - D_i),
//   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,  dv_j = sum_i P_ij do_i.
// P is recomputed from the forward's log-sum-exp: P_ij = exp(scale s_ij - lse_i).
//
// Three kernels, one stream:
//  1. delta: D_i and lse_i log2(e) for every row (fp32, into a caller workspace).
//  2. dq: one workgroup per (batch, head, query block), walking the block's CSR row. Per
//     key tile: S^T = K Q^T and dP^T = V dO^T on MFMA (keys on M, queries on N, K and V
//     rows from LDS, Q^T and dO^T in registers), P^T and dS^T in registers, then
//     dQ^T += K^T dS^T with K^T from transposing LDS reads: the dS^T accumulator is,
//     key for key, the B operand of that product, as P^T is for O^T in the forward.
//  3. dkdv: one workgroup per (batch, head, key block), walking the block's column of
//     the mask (the transposed CSR). Per query tile: S = Q K^T and dP = dO V^T (queries
//     on M, keys on N, Q and dO rows from LDS, K and V in registers), P and dS, then
//     dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T from transposing LDS reads.
// Tiles are copied HBM/L2 -> LDS with LDS-DMA. A dq workgroup is four wave64, one per
// SIMD, wave i owning rows 32i .. 32i+31 of its block; two of them share a CU, and each
// SIMD interleaves the two workgroups' waves. A dkdv workgroup is eight wave64 in two
// roles (S, P and dV beside dP, dS and dK), waves i and i + 4 sharing SIMD i and keys
// 32i .. 32i+31; one per CU (see the kernel). Accumulation is fp32; P and dS enter the
// MFMAs as bf16. Padding (rows or keys at or past n) and element masking work as in the
// forward.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/radial_attn.h"
#include "radial_device.h"

namespace {

constexpr int kBwdThreads = 256;  // four wave64, one per SIMD

// One sample of a varlen batch: its first token in the packed sequence, its length and
// block count, the offset of its rows in the concatenated row_ptr and col_ptr (nb + 1
// entries per sample), and its first workgroup id (workgroups go sample by sample, head
// by head, block by block).
struct BwdSample {
  int tok0, n, nb, rp0, wg0, pad0, pad1, pad2;
};
constexpr int kMaxBwdVarlen = 64;

struct BwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* o;
  const __bf16* g;  // dO
  const float* lse;
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  float* delta;  // D_i per row: the first half of the workspace
  float* lse2;   // lse_i log2(e) per row: its second half
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const int32_t* col_ptr;
  const int32_t* row_idx;
  int64_t stride_b, stride_h;
  int nb, heads, n, stride_s;
  int elem_s, elem_gw, elem_w0;  // element masking: frame length, grid width, W0
  float c;      // scale * log2(e), at least FLT_MIN (base2_scale)
  float scale;
  // varlen: 0 for a uniform batch, else the number of samples in `plan`; q, k, v, o, dO,
  // dq, dk, dv are then one packed sequence of n tokens, and lse, delta, lse2 are
  // [heads, n].
  int varlen;
  BwdSample plan[kMaxBwdVarlen];
  // element table (radial_build_element_table) for element masking from stored
  // decisions, or null
  const uint64_t* etab;
};
// Bytes of one element-table entry (one active block): for each of the four 32-token
// waves of the block's row and each lane, 64 decision bits, bit 16g + e for accumulator
// entry (g, e) of element_mask_tile's layout, as radial_build_element_table writes them.
constexpr int kEntryBytes = 2048;
typedef __attribute__((address_space(4))) const BwdArgs* BwdArgsPtr;
typedef __attribute__((address_space(4))) const int32_t ConstI32;
typedef __attribute__((address_space(3))) volatile int LdsFlag;

// Where a dq or dkdv workgroup works: the (batch, head) element offset, its rows of
// lse2 and delta, its mask rows (row_ptr / col_ptr point at its sample's), its sequence
// length and block count, and its block. Varlen plans are read from the kernel-argument
// segment (scalar loads; a copy of the plan would go to scratch memory under a dynamic
// index).
struct BwdGeometry {
  int64_t base;
  const float* lse2;
  const float* delta;
  const int32_t* row_ptr;
  const int32_t* col_ptr;
  int n, nb, blk;
};

// The block that the j-th workgroup of a (batch, head) works on. The hardware deals
// workgroup ids to the 8 XCDs round-robin; in each group of 32 blocks this gives each
// XCD a run of 4 neighbours (whose rows, or columns, of the mask are nearly the same, so
// they share that XCD's L2) while every XCD still samples the whole head evenly. The
// blocks past the last whole group keep their place.
__device__ __forceinline__ int block_of(int j, int nb) {
  if (j >= (nb & ~31)) return j;
  return (j & ~31) | ((j & 7) << 2) | ((j >> 3) & 3);
}

__device__ __forceinline__ BwdGeometry bwd_geometry(const BwdArgs& a, int wg) {
  BwdGeometry g;
  if (a.varlen == 0) {
    const int bh = wg / a.nb;
    const int b = bh / a.heads, h = bh - b * a.heads;
    g.base = b * a.stride_b + h * a.stride_h;
    g.lse2 = a.lse2 + static_cast<int64_t>(bh) * a.n;
    g.delta = a.delta + static_cast<int64_t>(bh) * a.n;
    g.row_ptr = a.row_ptr;
    g.col_ptr = a.col_ptr;
    g.n = a.n;
    g.nb = a.nb;
    g.blk = block_of(wg - bh * a.nb, a.nb);
    return g;
  }
  const BwdArgsPtr ap = (BwdArgsPtr)(__builtin_amdgcn_kernarg_segment_ptr());
  int lo = 0, hi = a.varlen - 1;  // the last sample whose first workgroup is at most wg
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (ap->plan[mid].wg0 <= wg) lo = mid;
    else hi = mid - 1;
  }
  const int tok0 = ap->plan[lo].tok0, nb = ap->plan[lo].nb, rp0 = ap->plan[lo].rp0;
  const int h = (wg - ap->plan[lo].wg0) / nb;
  g.base = static_cast<int64_t>(tok0) * a.stride_s + h * a.stride_h;
  g.lse2 = a.lse2 + static_cast<int64_t>(h) * a.n + tok0;
  g.delta = a.delta + static_cast<int64_t>(h) * a.n + tok0;
  g.row_ptr = a.row_ptr + rp0;
  g.col_ptr = a.col_ptr + rp0;
  g.n = ap->plan[lo].n;
  g.nb = nb;
  g.blk = block_of(wg - ap->plan[lo].wg0 - h * nb, nb);
  return g;
}

// ---- 1. D_i = <do_i, o_i>, and lse_i in base 2 ----
// D / 8 lanes per row, 8 bf16 each; 256 / (D / 8) rows per workgroup. The base-2 lse
// (lse_i log2(e), the exponent offset of P in 2^(c s - lse2)) is written beside D_i once
// per row, so that the dq and dkdv kernels, which read it once per tile, need no multiply
// per score for it.
template <int D>
__global__ __launch_bounds__(kBwdThreads) void radial_bwd_delta_kernel(const BwdArgs a,
                                                                       int rows_total) {
  constexpr int kLanes = D / 8;
  const int tid = threadIdx.x;
  const int r = blockIdx.x * (kBwdThreads / kLanes) + tid / kLanes;
  const int ch = tid % kLanes;
  float acc = 0.f;
  if (r < rows_total) {
    // Row r of the layout of delta, lse2 and lse: [batch, heads, n], or [heads, n] of a
    // packed varlen batch.
    const int bh = r / a.n, i = r - bh * a.n;
    const int b = a.varlen ? 0 : bh / a.heads, h = a.varlen ? bh : bh - b * a.heads;
    const int64_t off = b * a.stride_b + h * a.stride_h + static_cast<int64_t>(i) * a.stride_s +
                        8 * ch;
    const bf16x8 ov = *reinterpret_cast<const bf16x8*>(a.o + off);
    const bf16x8 gv = *reinterpret_cast<const bf16x8*>(a.g + off);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc += static_cast<float>(ov[j]) * static_cast<float>(gv[j]);
  }
#pragma unroll
  for (int m = kLanes / 2; m > 0; m >>= 1) acc += __shfl_xor(acc, m);
  if (r < rows_total && ch == 0) {
    a.delta[r] = acc;
    a.lse2[r] = a.lse[r] * kLog2e;
  }
}

// Row-read A operands of k-step s for the four 32-row groups of a tile (see
// row_read_offsets): frag[g] covers rows 32g .. 32g + 31, d = 16s .. 16s + 15.
template <int D>
__device__ __forceinline__ void read_rows(const char* tile_plus_base, int x, int s,
                                          bf16x8 (&frag)[4]) {
#pragma unroll
  for (int g = 0; g < 4; ++g)
    frag[g] = *reinterpret_cast<const bf16x8*>(tile_plus_base + g * 32 * Tile<D>::kRowBytes +
                                               ((s << 5) ^ x));
}

// Transposed-read A operand of step u (rows 16u .. 16u + 15 in accumulator order) for
// d block db (see tr_read_offsets).
template <int D>
__device__ __forceinline__ bf16x8 read_tr(const char* tile, int b0, int x0, int b1, int x1, int u,
                                          int db) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(tile + b0 + 16 * u * Tile<D>::kRowBytes + ((db << 6) ^ x0)));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(tile + b1 + 16 * u * Tile<D>::kRowBytes + ((db << 6) ^ x1)));
  return __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi),
                                 0, 1, 2, 3, 4, 5, 6, 7);
}

// The B operand of a 32-row block of one matrix, d = 16s + 8hl .. +7 of row r (a buffer
// descriptor over the block: rows past n read as zeros).
template <int D>
__device__ __forceinline__ void load_b_operand(const __bf16* m, int row0, int n, int row_bytes,
                                               int row_in_block, int hl,
                                               u32x4 (&f)[D / 16]) {
  const int rows = n - row0 < kBlock ? n - row0 : kBlock;
  const auto rs = make_rsrc(m + static_cast<int64_t>(row0) * (row_bytes / 2),
                            rows > 0 ? (rows - 1) * row_bytes + Tile<D>::kRowBytes : 0);
  const int off = row_in_block * row_bytes + hl * 16;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) f[s] = buffer_load16(rs, off + s * 32);
}

// Store a [D x 32] accumulator (d on M, this wave's 32 rows on N) times `mul` as bf16
// rows: lane owns row `row`, entries 4ib .. 4ib + 3 of d block db are d = 32db + 8ib + 4hl.
template <int D>
__device__ __forceinline__ void store_rows(__bf16* dst_row, const f32x16 (&acc)[D / 32], float mul,
                                           int hl) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      const f32x4 x = {acc[db][4 * ib + 0] * mul, acc[db][4 * ib + 1] * mul,
                       acc[db][4 * ib + 2] * mul, acc[db][4 * ib + 3] * mul};
      *reinterpret_cast<bf16x4*>(dst_row + 32 * db + 8 * ib + 4 * hl) =
          __builtin_convertvector(x, bf16x4);
    }
}

// One 256-byte copy instruction: lane l's 4 bytes at byte_offset land at lds + 4 l
// (buffer_load_dword ... lds), ordered like copy_1k.
__device__ __forceinline__ void copy_256(const i32x4& desc, uint32_t lds, int byte_offset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(byte_offset), "s"(desc)
               : "memory");
}

// ---- 2. dQ ----
// Two workgroups share a CU (64 KiB of LDS and at most 256 registers per wave each), so
// each SIMD runs two dQ waves from different workgroups and interleaves them: while one
// waits for its tile copy or works through its VALU steps, the other issues MFMAs. The
// K and V tiles are therefore single-buffered, but in halves of 64 keys: once every wave
// is done with one half, the next half is copied into its rows while the waves work on
// the other half.
template <int D, int E>
__global__ __launch_bounds__(kBwdThreads, 2) void radial_bwd_dq_kernel(const BwdArgs a) {
  using T = Tile<D>;
  constexpr int NDB = D / 32, NS = D / 16;
  // K and V tiles, then (element table only) this half's decision words of the four
  // waves, 256 bytes each, for each half parity.
  __shared__ __attribute__((aligned(1024))) char smem[2 * T::kBytes + (E == 3 ? 2048 : 0)];
  char* const kb0 = smem;
  char* const vb0 = smem + T::kBytes;
  char* const words = smem + 2 * T::kBytes;

  const BwdGeometry geo = bwd_geometry(a, blockIdx.x);
  const int nb = geo.nb, n = geo.n, qb = geo.blk;
  const int64_t base = geo.base;
  const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, hl = lane >> 5;
  const int wi = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row_bytes = a.stride_s * 2;
  const int q0 = qb * kBlock;
  const int qrow = q0 + 32 * wi + lq;
  const char* const kh = reinterpret_cast<const char*>(a.k + base);
  const char* const vh = reinterpret_cast<const char*>(a.v + base);

  // This lane's query: its log-sum-exp in base 2 and D_i.
  float lse2 = 0.f, dlt = 0.f;
  if (qrow < n) {
    lse2 = geo.lse2[qrow];
    dlt = geo.delta[qrow];
  }
  // A half tile (64 rows) of K or V is HC KiB per wave: lane offsets of copy i of wave
  // wi, which fills KiB wi * HC + i of the half (chunk position p of row r holds global
  // chunk p ^ swz(r)).
  constexpr int HC = 64 * T::kRowBytes / 1024 / 4;
  int copy_off[HC];
#pragma unroll
  for (int i = 0; i < HC; ++i) {
    const int ci = (wi * HC + i) * 64 + lane;
    const int row = ci / T::kChunks, pos = ci % T::kChunks;
    copy_off[i] = row * row_bytes + ((pos ^ swz<D>(row)) << 4);
  }
  int rbase, rx, tb0, tx0, tb1, tx1;
  row_read_offsets<D>(lane, rbase, rx);
  tr_read_offsets<D>(lane, tb0, tx0, tb1, tx1);

  const int r0 = geo.row_ptr[qb];
  const int L = geo.row_ptr[qb + 1] - r0;
  // The row's key blocks through the constant address space (scalar loads): a vector
  // load would be waited for with vmcnt(0), which counts the copies in flight too.
  ConstI32* const cols_of = (ConstI32*)(a.col_idx + r0);
  auto column = [&](int t) { return cols_of[t]; };
  // Half j of the walk (key block column(j / 2), keys 64 (j % 2) ..) into rows
  // 64 (j % 2) .. of the K and V buffers.
  auto copy_half = [&](int j) {
    const int t = j >> 1, h = j & 1;
    const int kb = column(t);
    const bool on = static_cast<unsigned>(kb) < static_cast<unsigned>(nb);
    const int row0 = on ? kb * kBlock + 64 * h : 0;
    const int left = n - row0;
    // (readfirstlane: the compiler clamps with a vector instruction, and the descriptors
    // built from this must be scalar.)
    const int rows = __builtin_amdgcn_readfirstlane(on ? (left < 64 ? (left > 0 ? left : 0) : 64) : 0);
    const int bytes = rows > 0 ? (rows - 1) * row_bytes + T::kRowBytes : 0;
    const i32x4 dk_ = raw_descriptor(kh + static_cast<int64_t>(row0) * row_bytes, bytes);
    const i32x4 dv_ = raw_descriptor(vh + static_cast<int64_t>(row0) * row_bytes, bytes);
    const uint32_t off = h * 64 * T::kRowBytes + wi * HC * 1024;
    const uint32_t kd = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)kb0)) + off;
    const uint32_t vd = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)vb0)) + off;
#pragma unroll
    for (int i = 0; i < HC; ++i) {
      copy_1k(dk_, kd + i * 1024, copy_off[i]);
      copy_1k(dv_, vd + i * 1024, copy_off[i]);
    }
    if constexpr (E == 3) {
      // This wave's decisions for the half: dword h of every lane's entry bits (the
      // table entry is CSR entry r0 + t, this block's t-th key block).
      const char* ent = reinterpret_cast<const char*>(a.etab) +
                        (static_cast<int64_t>(r0 + t) * kEntryBytes + wi * (kEntryBytes / 4));
      const uint32_t wd = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)words));
      copy_256(raw_descriptor(ent, kEntryBytes / 4), wd + h * 1024 + wi * 256, lane * 8 + h * 4);
    }
  };
  if (L > 0) copy_half(0);

  // Q^T and dO^T as MFMA B operands: d = 16s + 8hl .. +7 of this lane's query.
  u32x4 qf[NS], gf[NS];
  load_b_operand<D>(a.q + base, q0, n, row_bytes, 32 * wi + lq, hl, qf);
  load_b_operand<D>(a.g + base, q0, n, row_bytes, 32 * wi + lq, hl, gf);
  __builtin_amdgcn_s_waitcnt(0);  // Q, dO and the first half tile (see the forward prologue)

  f32x16 dq[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dq[i] = f32x16{};

  for (int t = 0; t < L; ++t) {
    const int kb = column(t);
    // A column outside [0, nb) was copied as zeros; every one of its keys is masked as
    // padding (n_eff = its first token), so it adds nothing. No branch skips it: a second
    // path through the loop would make the compiler copy dQ between register files.
    const bool valid = static_cast<unsigned>(kb) < static_cast<unsigned>(nb);
    const int n_eff = valid ? n : kb * kBlock;
    const char* const kt = kb0;
    const char* const vt = vb0;

    // The tile in two halves of 64 keys, so that only half of S^T and dP^T is live.
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      wait_copies<0>();  // this wave's part of half (t, h)
      lds_barrier();     // every wave's part landed, and every wave is done with the
                         // previous half, whose rows the next half now takes
      if (2 * t + h + 1 < 2 * L) copy_half(2 * t + h + 1);
      uint32_t ew = 0;  // this lane's decisions for the half (element table)
      if constexpr (E == 3)
        ew = *reinterpret_cast<const uint32_t*>(words + h * 1024 + wi * 256 + lane * 4);
      // S^T = K Q^T and dP^T = V dO^T for keys 64h .. 64h + 63 (keys on M, this wave's
      // queries on N), at raised wave priority: the SIMD's other dQ wave (from the other
      // workgroup) then issues its VALU work around these MFMAs rather than ahead of them.
      __builtin_amdgcn_s_setprio(1);
      f32x16 sacc[2], pacc[2];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        bf16x8 kf[2], vf[2];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const int off = rbase + (2 * h + g) * 32 * T::kRowBytes + ((s << 5) ^ rx);
          kf[g] = *reinterpret_cast<const bf16x8*>(kt + off);
          vf[g] = *reinterpret_cast<const bf16x8*>(vt + off);
        }
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          sacc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              kf[g], __builtin_bit_cast(bf16x8, qf[s]), s == 0 ? f32x16{} : sacc[g], 0, 0, 0);
          pacc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              vf[g], __builtin_bit_cast(bf16x8, gf[s]), s == 0 ? f32x16{} : pacc[g], 0, 0, 0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      const int key0 = kb * kBlock + 64 * h;
      if (n_eff - key0 < 64) pad_mask_tile<2>(key0, n_eff, lane, sacc);
      if constexpr (E == 3) {
        if (valid) element_mask_stored<2>(ew, sacc);
      } else if constexpr (E != 0) {
        if (valid)
          element_mask_any<E, 2>(q0 + 32 * wi, key0, a.elem_s, a.elem_gw, a.elem_w0 - 1, lane,
                                 sacc);
      }

      // Per step u of 16 keys: P^T = 2^(c s - lse2) and dS^T = P^T (dP^T - D), packed as
      // the B operand of dQ^T += K^T dS^T (d on M, queries on N, keys contracted in
      // accumulator order), whose MFMAs are issued right away: they run while the VALU
      // works on step u + 1.
#pragma unroll
      for (int u2 = 0; u2 < 4; ++u2) {
        const int g = u2 >> 1, s2 = u2 & 1;
        f32x8 d8;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[g][8 * s2 + jj], a.c, -lse2));
          d8[jj] = p * (pacc[g][8 * s2 + jj] - dlt);
        }
        const bf16x8 dsk = __builtin_convertvector(d8, bf16x8);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              read_tr<D>(kt, tb0, tx0, tb1, tx1, 4 * h + u2, db), dsk, dq[db], 0, 0, 0);
      }
    }
  }
  if (qrow < n) store_rows<D>(a.dq + base + static_cast<int64_t>(qrow) * a.stride_s, dq, a.scale, hl);
}

// ---- 3. dK, dV ----
// Eight waves in two roles over the block's 128 keys. Waves 0-3 (the P side) hold K as
// MFMA B operands, compute S = Q K^T and P, and accumulate dV^T += dO^T P; waves 4-7 (the
// dS side) hold V, compute dP = dO V^T, and accumulate dK^T += Q^T dS with
// dS = P (dP - D). Waves i and i + 4 share SIMD i and keys 32i .. 32i + 31, so each SIMD
// runs two waves whose VALU and MFMA work interleave, and neither needs more than half
// of the SIMD's registers. P goes from the P side to the dS side through LDS, as the
// bf16 values that also enter dV's MFMAs.
//
// The query tiles of the column are walked in halves of 64 queries, one half per phase,
// with one workgroup barrier between phases. In phase p both sides work on half p: the
// P side computes S and P, writes P to the exchange buffer and marks it written in an
// LDS word of its SIMD, then accumulates dV; the dS side computes dP meanwhile, waits
// for the mark, reads P and accumulates dK. (The dS side reads the buffer before the
// next barrier, and the P side writes it after that barrier, so one buffer serves.) Q
// and dO halves, with the lse and D of their 64 queries, sit in a ring of four slots:
// phase p reads half p and copies half p + 3.
constexpr int kDkdvThreads = 512;

template <int D>
struct DkdvLds {
  static constexpr int kHalfBytes = 64 * D * 2;             // 64 rows of Q or dO
  static constexpr int kCopies = kHalfBytes / 1024 / 4;     // per P-side wave and operand
  static constexpr int kLse = 2 * kHalfBytes;               // then 64 lse, then 64 D
  static constexpr int kWords = kLse + 512;  // then the element table's decision words
  static constexpr int kSlot = kWords + 1024;
  static constexpr int kExchange = 4 * kSlot;               // P: 64 queries x 128 keys, bf16
  static constexpr int kFlags = kExchange + 16384;          // one word per SIMD
  static constexpr int kBytes = kFlags + 16;
  static_assert(kCopies * 4 * 1024 == kHalfBytes, "four waves' copies must cover a half");
  static_assert(kSlot % 256 == 0, "slots keep the bank swizzle");
};

// acc[g] = (rows 32g .. 32g + 31 of a half tile) x B^T over all d: the row reads of
// step s + 2 are issued beside the MFMAs of step s (one read after each MFMA), pinned
// with sched_group_barrier; left to itself the compiler waits for each step's reads
// right before its MFMAs. tile_base is the half tile plus this lane's row offset.
template <int D>
__device__ __forceinline__ void half_rows_times(const char* tile_base, int x,
                                                const u32x4 (&b)[D / 16], f32x16 (&acc)[2]) {
  constexpr int NS = D / 16;
  bf16x8 f[2][2];
  // LDS reads that the caller issued before (the lse or D values of the half) stay ahead
  // of this fence; otherwise the pinned groups below count them as this product's first
  // reads, and each MFMA then waits for the read issued just before it.
  __builtin_amdgcn_sched_barrier(0);
  auto rd = [&](int s, bf16x8 (&dst)[2]) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
      dst[g] = *reinterpret_cast<const bf16x8*>(tile_base + g * 32 * Tile<D>::kRowBytes +
                                                 ((s << 5) ^ x));
  };
  rd(0, f[0]);
  rd(1, f[1]);
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int s = 0; s < NS; ++s) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
      acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          f[s & 1][g], __builtin_bit_cast(bf16x8, b[s]), s == 0 ? f32x16{} : acc[g], 0, 0, 0);
    if (s + 2 < NS) rd(s + 2, f[s & 1]);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (s + 2 < NS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  }
}

// acc[db] += (half tile)^T x B over the half's 64 rows, four steps of 16 rows with B
// operands b[u]: the transposed reads of step u + 1 are issued beside the MFMAs of step
// u (two reads after each MFMA), pinned as in half_rows_times.
template <int D>
__device__ __forceinline__ void half_trans_times(const char* tile, int b0, int x0, int b1, int x1,
                                                 const bf16x8 (&b)[4], f32x16 (&acc)[D / 32]) {
  constexpr int NDB = D / 32;
  bf16x8 f[2][NDB];
  auto rd = [&](int u, bf16x8 (&dst)[NDB]) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) dst[db] = read_tr<D>(tile, b0, x0, b1, x1, u, db);
  };
  rd(0, f[0]);
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * NDB, 0);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (u + 1 < 4) rd(u + 1, f[(u + 1) & 1]);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[u & 1][db], b[u], acc[db], 0, 0, 0);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      if (u + 1 < 4) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
  }
}

template <int D, int E>
__global__ __launch_bounds__(kDkdvThreads, 1) void radial_bwd_dkdv_kernel(const BwdArgs a) {
  using T = Tile<D>;
  using M = DkdvLds<D>;
  constexpr int NDB = D / 32, NS = D / 16;
  __shared__ __attribute__((aligned(1024))) char smem[M::kBytes];
  char* const xb = smem + M::kExchange;
  // (An LDS pointer: through a generic one the volatile accesses become flat memory
  // operations, whose waits include the tile copies in flight.)
  LdsFlag* const flags = (LdsFlag*)(smem + M::kFlags);

  const BwdGeometry geo = bwd_geometry(a, blockIdx.x);
  const int nb = geo.nb, n = geo.n, kb = geo.blk;
  const int64_t base = geo.base;
  const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, hl = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wi = w & 3;  // key slice (and SIMD)
  const int row_bytes = a.stride_s * 2;
  const int k0 = kb * kBlock;
  const int krow = k0 + 32 * wi + lq;
  const char* const qh = reinterpret_cast<const char*>(a.q + base);
  const char* const gh = reinterpret_cast<const char*>(a.g + base);

  // Lane offsets of a P-side wave's share of a half copy: KiB wi * kCopies + i of the
  // half, lane l's 16 bytes at chunk position p of row r, holding global chunk p ^ swz(r).
  int copy_off[M::kCopies];
#pragma unroll
  for (int i = 0; i < M::kCopies; ++i) {
    const int ci = (wi * M::kCopies + i) * 64 + lane;
    const int row = ci / T::kChunks, pos = ci % T::kChunks;
    copy_off[i] = row * row_bytes + ((pos ^ swz<D>(row)) << 4);
  }
  int rbase, rx, tb0, tx0, tb1, tx1;
  row_read_offsets<D>(lane, rbase, rx);
  tr_read_offsets<D>(lane, tb0, tx0, tb1, tx1);

  const int c0 = geo.col_ptr[kb];
  const int L = geo.col_ptr[kb + 1] - c0;
  const int halves = 2 * L;
  // Element table: the decisions of (key block kb, query block) pairs are row kb's
  // entries, in the same ascending order as the column walk when the mask is symmetric.
  const int rk0 = E == 3 ? geo.row_ptr[kb] : 0;
  const int rkl = E == 3 ? geo.row_ptr[kb + 1] - rk0 : 0;
  // The column's row blocks, read through the constant address space so that the
  // compiler uses scalar loads: a vector load would be waited for with vmcnt(0), which
  // also waits for the tile copies in flight.
  ConstI32* const rows_of = (ConstI32*)(a.row_idx + c0);
  auto qblock = [&](int t) { return rows_of[t]; };
  auto slot = [&](int j) { return smem + (j & 3) * M::kSlot; };
  // Copy half j (query tile j / 2, rows 64 (j % 2) ..) into its slot; the P-side waves
  // issue the copies (the dS side is the longer path through a phase), wave 0 also copies
  // the half's base-2 lse and wave 1 its D, one instruction more per half.
  auto copy_half = [&](int j) {
    const int t = j >> 1, h = j & 1;
    const int qb = qblock(t);
    const bool on = static_cast<unsigned>(qb) < static_cast<unsigned>(nb);
    const int row0 = on ? qb * kBlock + 64 * h : 0;
    const int left = n - row0;
    // (readfirstlane: the compiler clamps with a vector instruction, and the descriptors
    // built from this must be scalar.)
    const int rows = __builtin_amdgcn_readfirstlane(on ? (left < 64 ? (left > 0 ? left : 0) : 64) : 0);
    const int bytes = rows > 0 ? (rows - 1) * row_bytes + T::kRowBytes : 0;
    const uint32_t sb = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)slot(j)));
    const uint32_t dst = sb + wi * M::kCopies * 1024;
    const i32x4 dq_ = raw_descriptor(qh + static_cast<int64_t>(row0) * row_bytes, bytes);
    const i32x4 dg_ = raw_descriptor(gh + static_cast<int64_t>(row0) * row_bytes, bytes);
#pragma unroll
    for (int i = 0; i < M::kCopies; ++i) {
      copy_1k(dq_, dst + i * 1024, copy_off[i]);
      copy_1k(dg_, dst + M::kHalfBytes + i * 1024, copy_off[i]);
    }
    if (w < 2) {
      const float* src = (w == 0 ? geo.lse2 : geo.delta) + row0;
      copy_256(raw_descriptor(reinterpret_cast<const char*>(src), rows * 4),
               sb + M::kLse + w * 256, lane * 4);
    }
    if constexpr (E == 3) {
      // This wave's decisions for the half: dword h of every lane's entry bits (its keys
      // are the table's queries). A walk longer than row kb (a mask that is not
      // symmetric) copies zeros past the row's entries.
      const char* ent = reinterpret_cast<const char*>(a.etab) +
                        (static_cast<int64_t>(rk0 + t) * kEntryBytes + wi * (kEntryBytes / 4));
      copy_256(raw_descriptor(ent, t < rkl ? kEntryBytes / 4 : 0), sb + M::kWords + wi * 256,
               lane * 8 + h * 4);
    }
  };
  // Wait for this P-side wave's copies of half p, leaving those of halves p + 1 and
  // p + 2 (issued in the two phases before) in flight where they exist.
  auto wait_half = [&](int p) {
    // per half, plus one for waves 0 and 1, plus one with the element table
    constexpr int N = 2 * M::kCopies + (E == 3 ? 1 : 0);
    if (p + 2 < halves) {
      if (w < 2) wait_copies<2 * (N + 1)>();
      else wait_copies<2 * N>();
    } else if (p + 1 < halves) {
      if (w < 2) wait_copies<N + 1>();
      else wait_copies<N>();
    } else {
      wait_copies<0>();
    }
  };
  if (w < 4 && lane == 0) flags[wi] = 0;  // P of half p is written when flags[wi] > p
  char* const xw = xb + wi * 4096 + lane * 16;  // this SIMD's exchange area, lane part
  const int64_t out_off = base + static_cast<int64_t>(krow) * a.stride_s;

  if (w < 4) {
    // ---- P side: S, P, dV ----
    for (int j = 0; j < 3 && j < halves; ++j) copy_half(j);
    u32x4 kf[NS];  // K as MFMA B operand: d = 16s + 8hl .. +7 of this lane's key
    load_b_operand<D>(a.k + base, k0, n, row_bytes, 32 * wi + lq, hl, kf);
    __builtin_amdgcn_s_waitcnt(0);
    f32x16 dv[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) dv[i] = f32x16{};
    for (int p = 0; p < halves; ++p) {
      const int t = p >> 1, h = p & 1;
      // (The scalar load of the row block is waited for before the barrier: a wait after
      // it would also wait for the LDS reads issued below.)
      int qb = qblock(t);
      asm volatile("" : "+s"(qb));
      wait_half(p);
      lds_barrier();
      // A row block outside [0, nb) was copied as zeros; all of its queries are masked
      // as padding, so P is zero there (no second path through the loop).
      const bool valid = static_cast<unsigned>(qb) < static_cast<unsigned>(nb);
      const int n_eff = valid ? n : qb * kBlock;
      const char* const qt = slot(p);
      // The base-2 lse of query 32g + 8j + 4hl + r of the half at l4[4g + j][r], read
      // now so that they land while S is computed.
      const float* const lt = reinterpret_cast<const float*>(qt + M::kLse);
      f32x4 l4[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        l4[i] = *reinterpret_cast<const f32x4*>(lt + 32 * (i >> 2) + 8 * (i & 3) + 4 * hl);
      uint32_t ew = 0;  // this lane's decisions for the half (element table)
      if constexpr (E == 3)
        ew = *reinterpret_cast<const uint32_t*>(qt + M::kWords + wi * 256 + lane * 4);
      // S = Q K^T for the half's 64 queries (queries on M, this wave's keys on N).
      f32x16 sacc[2];
      half_rows_times<D>(qt + rbase, rx, kf, sacc);
      const int row0 = qb * kBlock + 64 * h;
      if (n_eff - row0 < 64) pad_mask_tile<2>(row0, n_eff, lane, sacc);
      if constexpr (E == 3) {
        if (valid) element_mask_stored<2>(ew, sacc);
      } else if constexpr (E != 0) {
        if (valid)
          element_mask_any<E, 2>(k0 + 32 * wi, row0, a.elem_s, a.elem_gw, a.elem_w0 - 1,
                                 lane, sacc);
      }
      // P = 2^(c s - lse2) per entry (query 32g + 8(e/4) + 4hl + e%4 of the half), packed
      // as the B operands of dV^T, written for the dS wave and marked.
      bf16x8 pk[4];
#pragma unroll
      for (int u2 = 0; u2 < 4; ++u2) {
        const int g = u2 >> 1, s2 = u2 & 1;
        f32x8 p8;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const f32x4 lh = l4[4 * g + 2 * s2 + half];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            p8[4 * half + r] =
                __builtin_amdgcn_exp2f(fmaf(sacc[g][8 * s2 + 4 * half + r], a.c, -lh[r]));
        }
        pk[u2] = __builtin_convertvector(p8, bf16x8);
        *reinterpret_cast<bf16x8*>(xw + u2 * 1024) = pk[u2];
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (lane == 0) flags[wi] = p + 1;
      // dV^T += dO^T P (d on M, keys on N, queries contracted).
      half_trans_times<D>(qt + M::kHalfBytes, tb0, tx0, tb1, tx1, pk, dv);
      // Half p + 3 goes into the slot that half p - 1 left at this phase's barrier.
      // (The copies are issued by this side, which has the shorter path through a phase:
      // a copy instruction can wait several cycles for the vector-memory path.)
      if (p + 3 < halves) copy_half(p + 3);
    }
    if (krow < n) store_rows<D>(a.dv + out_off, dv, 1.0f, hl);
  } else {
    // ---- dS side: dP, dS, dK ----
    u32x4 vf[NS];  // V as MFMA B operand
    load_b_operand<D>(a.v + base, k0, n, row_bytes, 32 * wi + lq, hl, vf);
    __builtin_amdgcn_s_waitcnt(0);
    f32x16 dk[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) dk[i] = f32x16{};
    for (int p = 0; p < halves; ++p) {
      lds_barrier();  // (the P side waits for the copies before it)
      const char* const qt = slot(p);
      // D of query 32g + 8j + 4hl + r of the half at d4[4g + j][r].
      const float* const dt = reinterpret_cast<const float*>(qt + M::kLse + 256);
      f32x4 d4[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        d4[i] = *reinterpret_cast<const f32x4*>(dt + 32 * (i >> 2) + 8 * (i & 3) + 4 * hl);
      // dP = dO V^T for the half (queries on M, this wave's keys on N).
      f32x16 pacc[2];
      half_rows_times<D>(qt + M::kHalfBytes + rbase, rx, vf, pacc);
      // The P wave has written P of this half (it marks p + 1 after writing).
      while (__builtin_amdgcn_readfirstlane(flags[wi]) <= p) __builtin_amdgcn_s_sleep(1);
      asm volatile("" ::: "memory");
      bf16x8 pv[4];
#pragma unroll
      for (int u2 = 0; u2 < 4; ++u2) pv[u2] = *reinterpret_cast<const bf16x8*>(xw + u2 * 1024);
      // dS = P (dP - D), then dK^T += Q^T dS (d on M, keys on N, queries contracted).
      bf16x8 dsk[4];
#pragma unroll
      for (int u2 = 0; u2 < 4; ++u2) {
        const int g = u2 >> 1, s2 = u2 & 1;
        f32x8 d8;
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            d8[4 * half + r] = static_cast<float>(pv[u2][4 * half + r]) *
                               (pacc[g][8 * s2 + 4 * half + r] - d4[4 * g + 2 * s2 + half][r]);
        dsk[u2] = __builtin_convertvector(d8, bf16x8);
      }
      half_trans_times<D>(qt, tb0, tx0, tb1, tx1, dsk, dk);
    }
    if (krow < n) store_rows<D>(a.dk + out_off, dk, a.scale, hl);
  }
}

bool aligned(const void* p, uintptr_t m) { return (reinterpret_cast<uintptr_t>(p) & (m - 1)) == 0; }

template <int D, int E>
void launch_bwd(const BwdArgs& args, int rows_total, int items, hipStream_t st) {
  constexpr int kRowsPerBlock = kBwdThreads / (D / 8);
  hipLaunchKernelGGL((radial_bwd_delta_kernel<D>), dim3((rows_total + kRowsPerBlock - 1) / kRowsPerBlock),
                     dim3(kBwdThreads), 0, st, args, rows_total);
  hipLaunchKernelGGL((radial_bwd_dq_kernel<D, E>), dim3(items), dim3(kBwdThreads), 0, st, args);
  hipLaunchKernelGGL((radial_bwd_dkdv_kernel<D, E>), dim3(items), dim3(kDkdvThreads), 0, st, args);
}

// The three kernels of one call, at the template instance of head_dim and the element
// mode (none, 1-D distance, grid distance, element table).
int32_t launch_all(const BwdArgs& args, int rows_total, int items, int head_dim,
                   int32_t element_tokens_per_frame, int32_t element_grid_w, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int mode = args.etab != nullptr ? 3
                   : element_tokens_per_frame == 0 ? 0 : (element_grid_w == 0 ? 1 : 2);
  if (head_dim == 128) {
    if (mode == 3) launch_bwd<128, 3>(args, rows_total, items, st);
    else if (mode == 2) launch_bwd<128, 2>(args, rows_total, items, st);
    else if (mode == 1) launch_bwd<128, 1>(args, rows_total, items, st);
    else launch_bwd<128, 0>(args, rows_total, items, st);
  } else {
    if (mode == 3) launch_bwd<64, 3>(args, rows_total, items, st);
    else if (mode == 2) launch_bwd<64, 2>(args, rows_total, items, st);
    else if (mode == 1) launch_bwd<64, 1>(args, rows_total, items, st);
    else launch_bwd<64, 0>(args, rows_total, items, st);
  }
  return hipGetLastError() == hipSuccess ? RADIAL_OK : RADIAL_ERR_HIP;
}

}  // namespace

namespace {

// The uniform backward: checks, then the three kernels. delta is the workspace of two
// fp32 per row, D_i then the base-2 lse (caller-owned, or the static scratch of
// radial_attn_bwd_noalloc); max_rows bounds batch * heads * seqlen (the rows the
// workspace holds), or is 0 for no bound. etab (an element table) replaces the element
// arguments when not null.
int32_t bwd_uniform(const void* q, const void* k, const void* v, const void* o,
                    const void* dout, const float* lse, void* dq, void* dk, void* dv,
                    float* delta, int64_t max_rows, const int32_t* row_ptr,
                    const int32_t* col_idx, const int32_t* col_ptr, const int32_t* row_idx,
                    int32_t nb, float scale, int32_t element_tokens_per_frame,
                    int32_t element_w0, int32_t element_grid_w, const void* etab,
                    int32_t batch, int32_t heads, int32_t seqlen, int32_t head_dim,
                    int64_t stride_b, int64_t stride_h, int64_t stride_s, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !delta || !row_ptr ||
      !col_idx || !col_ptr || !row_idx)
    return RADIAL_ERR_INVALID_ARG;
  if (batch <= 0 || heads <= 0 || seqlen <= 0 || nb <= 0) return RADIAL_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || scale < 0.f) return RADIAL_ERR_INVALID_ARG;
  if (!element_args_valid(element_tokens_per_frame, element_w0, element_grid_w))
    return RADIAL_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return RADIAL_ERR_UNSUPPORTED_HEAD_DIM;
  if (nb != (seqlen + kBlock - 1) / kBlock) return RADIAL_ERR_SHAPE_MISMATCH;
  if (stride_s < head_dim || stride_h < 0 || stride_b < 0) return RADIAL_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned(p, 16)) return RADIAL_ERR_MISALIGNED;
  if (!aligned(lse, 4) || !aligned(delta, 4)) return RADIAL_ERR_MISALIGNED;
  if (etab != nullptr && !aligned(etab, 16)) return RADIAL_ERR_MISALIGNED;
  if ((stride_s | stride_h | stride_b) & 7) return RADIAL_ERR_MISALIGNED;
  const int64_t items = static_cast<int64_t>(batch) * heads * nb;
  const int64_t rows_total = static_cast<int64_t>(batch) * heads * seqlen;
  if (items > INT32_MAX || rows_total > INT32_MAX || stride_s > (INT32_MAX / 2) / kBlock)
    return RADIAL_ERR_TOO_LARGE;
  if (max_rows > 0 && rows_total > max_rows) return RADIAL_ERR_TOO_LARGE;

  BwdArgs args;
  args.q = static_cast<const __bf16*>(q);
  args.k = static_cast<const __bf16*>(k);
  args.v = static_cast<const __bf16*>(v);
  args.o = static_cast<const __bf16*>(o);
  args.g = static_cast<const __bf16*>(dout);
  args.lse = lse;
  args.dq = static_cast<__bf16*>(dq);
  args.dk = static_cast<__bf16*>(dk);
  args.dv = static_cast<__bf16*>(dv);
  args.delta = delta;
  args.lse2 = delta + rows_total;
  args.row_ptr = row_ptr;
  args.col_idx = col_idx;
  args.col_ptr = col_ptr;
  args.row_idx = row_idx;
  args.stride_b = stride_b;
  args.stride_h = stride_h;
  args.nb = nb;
  args.heads = heads;
  args.n = seqlen;
  args.stride_s = static_cast<int>(stride_s);
  args.elem_s = element_tokens_per_frame;
  args.elem_gw = element_grid_w;
  args.elem_w0 = element_w0;
  args.c = base2_scale(scale);
  args.scale = scale;
  args.varlen = 0;
  args.etab = static_cast<const uint64_t*>(etab);
  return launch_all(args, static_cast<int>(rows_total), static_cast<int>(items), head_dim,
                    element_tokens_per_frame, element_grid_w, stream);
}

// radial_attn_bwd_noalloc's workspace: the backward's D_i and base-2 lse, two fp32 per
// row, for at most kScratchRows rows (64 MiB per device, held until the process ends). Host code never
// uses the array's name as an address: each device's address comes from
// hipGetSymbolAddress, once per device, with that device current.
constexpr int64_t kScratchRows = int64_t(1) << 23;
constexpr int kScratchDevices = 64;
float* g_scratch[kScratchDevices];
std::mutex g_scratch_mu;

}  // namespace

static __device__ __align__(256) float scratch[2 * kScratchRows];

namespace {

// The current device's address of `scratch`, looked up on the device's first call.
int32_t scratch_address(float** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices)
    return RADIAL_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return RADIAL_ERR_HIP;
    g_scratch[dev] = static_cast<float*>(ptr);
  }
  *out = g_scratch[dev];
  return RADIAL_OK;
}

}  // namespace

extern "C" int32_t radial_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                                   const void* dout, const float* lse, void* dq, void* dk,
                                   void* dv, float* delta, const int32_t* row_ptr,
                                   const int32_t* col_idx, const int32_t* col_ptr,
                                   const int32_t* row_idx, int32_t nb, float scale,
                                   int32_t element_tokens_per_frame, int32_t element_w0,
                                   int32_t element_grid_w, int32_t batch, int32_t heads,
                                   int32_t seqlen,
                                   int32_t head_dim, int64_t stride_b, int64_t stride_h,
                                   int64_t stride_s, void* stream) {
  return bwd_uniform(q, k, v, o, dout, lse, dq, dk, dv, delta, 0, row_ptr, col_idx, col_ptr,
                     row_idx, nb, scale, element_tokens_per_frame, element_w0, element_grid_w,
                     nullptr, batch, heads, seqlen, head_dim, stride_b, stride_h, stride_s,
                     stream);
}

extern "C" int32_t radial_attn_bwd_element_table(
    const void* q, const void* k, const void* v, const void* o, const void* dout,
    const float* lse, void* dq, void* dk, void* dv, float* delta, const int32_t* row_ptr,
    const int32_t* col_idx, const int32_t* col_ptr, const int32_t* row_idx, int32_t nb,
    float scale, const void* element_table, int32_t batch, int32_t heads, int32_t seqlen,
    int32_t head_dim, int64_t stride_b, int64_t stride_h, int64_t stride_s, void* stream) {
  if (element_table == nullptr) return RADIAL_ERR_INVALID_ARG;
  return bwd_uniform(q, k, v, o, dout, lse, dq, dk, dv, delta, 0, row_ptr, col_idx, col_ptr,
                     row_idx, nb, scale, 0, 0, 0, element_table, batch, heads, seqlen,
                     head_dim, stride_b, stride_h, stride_s, stream);
}

extern "C" int32_t radial_attn_bwd_noalloc(
    const void* q, const void* k, const void* v, const void* o, const void* dout,
    const float* lse, void* dq, void* dk, void* dv, const int32_t* row_ptr,
    const int32_t* col_idx, const int32_t* col_ptr, const int32_t* row_idx, int32_t nb,
    float scale, int32_t element_tokens_per_frame, int32_t element_w0, int32_t element_grid_w,
    int32_t batch, int32_t heads, int32_t seqlen, int32_t head_dim, int64_t stride_b,
    int64_t stride_h, int64_t stride_s, void* stream) {
  // Sizes first, so that an input past the workspace is refused before any HIP call.
  if (batch > 0 && heads > 0 && seqlen > 0 &&
      static_cast<int64_t>(batch) * heads * seqlen > kScratchRows)
    return RADIAL_ERR_TOO_LARGE;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !row_ptr || !col_idx ||
      !col_ptr || !row_idx)
    return RADIAL_ERR_INVALID_ARG;
  float* delta = nullptr;
  const int32_t err = scratch_address(&delta);
  if (err != RADIAL_OK) return err;
  return bwd_uniform(q, k, v, o, dout, lse, dq, dk, dv, delta, kScratchRows, row_ptr, col_idx,
                     col_ptr, row_idx, nb, scale, element_tokens_per_frame, element_w0,
                     element_grid_w, nullptr, batch, heads, seqlen, head_dim, stride_b,
                     stride_h, stride_s, stream);
}

namespace {

// The varlen backward for radial_attn_bwd_varlen and radial_attn_bwd_varlen_element_table:
// etab null takes the element arguments, else the table.
int32_t bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                   float* delta, const int32_t* seq_tokens, int32_t batch,
                   const int32_t* row_ptr, const int32_t* col_idx, const int32_t* col_ptr,
                   const int32_t* row_idx, float scale, int32_t element_tokens_per_frame,
                   int32_t element_w0, int32_t element_grid_w, const void* etab,
                   int32_t heads, int32_t head_dim, int64_t stride_h, int64_t stride_s,
                   void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !delta || !row_ptr ||
      !col_idx || !col_ptr || !row_idx || !seq_tokens)
    return RADIAL_ERR_INVALID_ARG;
  if (batch <= 0 || heads <= 0) return RADIAL_ERR_INVALID_ARG;
  if (batch > kMaxBwdVarlen) return RADIAL_ERR_TOO_LARGE;
  if (!std::isfinite(scale) || scale < 0.f) return RADIAL_ERR_INVALID_ARG;
  if (!element_args_valid(element_tokens_per_frame, element_w0, element_grid_w))
    return RADIAL_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return RADIAL_ERR_UNSUPPORTED_HEAD_DIM;
  if (stride_s < head_dim || stride_h < 0) return RADIAL_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned(p, 16)) return RADIAL_ERR_MISALIGNED;
  if (!aligned(lse, 4) || !aligned(delta, 4)) return RADIAL_ERR_MISALIGNED;
  if ((stride_s | stride_h) & 7) return RADIAL_ERR_MISALIGNED;
  if (etab != nullptr && !aligned(etab, 16)) return RADIAL_ERR_MISALIGNED;
  if (stride_s > (INT32_MAX / 2) / kBlock) return RADIAL_ERR_TOO_LARGE;

  BwdArgs args;
  args.q = static_cast<const __bf16*>(q);
  args.k = static_cast<const __bf16*>(k);
  args.v = static_cast<const __bf16*>(v);
  args.o = static_cast<const __bf16*>(o);
  args.g = static_cast<const __bf16*>(dout);
  args.lse = lse;
  args.dq = static_cast<__bf16*>(dq);
  args.dk = static_cast<__bf16*>(dk);
  args.dv = static_cast<__bf16*>(dv);
  args.delta = delta;
  args.row_ptr = row_ptr;
  args.col_idx = col_idx;
  args.col_ptr = col_ptr;
  args.row_idx = row_idx;
  args.stride_b = 0;
  args.stride_h = stride_h;
  args.heads = heads;
  args.stride_s = static_cast<int>(stride_s);
  args.elem_s = element_tokens_per_frame;
  args.elem_gw = element_grid_w;
  args.elem_w0 = element_w0;
  args.c = base2_scale(scale);
  args.scale = scale;
  args.varlen = batch;
  args.etab = static_cast<const uint64_t*>(etab);
  int64_t tok = 0, rows = 0, wgs = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t n = seq_tokens[b];
    if (n <= 0) return RADIAL_ERR_INVALID_ARG;
    const int32_t nb = (n + kBlock - 1) / kBlock;
    if (tok > INT32_MAX || rows > INT32_MAX || wgs > INT32_MAX) return RADIAL_ERR_TOO_LARGE;
    args.plan[b] = BwdSample{static_cast<int>(tok), n, nb, static_cast<int>(rows),
                             static_cast<int>(wgs), 0, 0, 0};
    tok += n;
    rows += nb + 1;
    wgs += static_cast<int64_t>(heads) * nb;
  }
  if (tok > INT32_MAX || wgs > INT32_MAX || static_cast<int64_t>(heads) * tok > INT32_MAX)
    return RADIAL_ERR_TOO_LARGE;
  args.n = static_cast<int>(tok);  // the packed sequence; lse and delta are [heads, n]
  args.nb = 0;                     // per sample, from the plan
  args.lse2 = delta + heads * tok;
  return launch_all(args, static_cast<int>(heads * tok), static_cast<int>(wgs), head_dim,
                    element_tokens_per_frame, element_grid_w, stream);
}

}  // namespace

extern "C" int32_t radial_attn_bwd_varlen(const void* q, const void* k, const void* v,
                                          const void* o, const void* dout, const float* lse,
                                          void* dq, void* dk, void* dv, float* delta,
                                          const int32_t* seq_tokens, int32_t batch,
                                          const int32_t* row_ptr, const int32_t* col_idx,
                                          const int32_t* col_ptr, const int32_t* row_idx,
                                          float scale, int32_t element_tokens_per_frame,
                                          int32_t element_w0, int32_t element_grid_w,
                                          int32_t heads, int32_t head_dim, int64_t stride_h,
                                          int64_t stride_s, void* stream) {
  return bwd_varlen(q, k, v, o, dout, lse, dq, dk, dv, delta, seq_tokens, batch, row_ptr,
                    col_idx, col_ptr, row_idx, scale, element_tokens_per_frame, element_w0,
                    element_grid_w, nullptr, heads, head_dim, stride_h, stride_s, stream);
}

extern "C" int32_t radial_attn_bwd_varlen_element_table(
    const void* q, const void* k, const void* v, const void* o, const void* dout,
    const float* lse, void* dq, void* dk, void* dv, float* delta, const int32_t* seq_tokens,
    int32_t batch, const int32_t* row_ptr, const int32_t* col_idx, const int32_t* col_ptr,
    const int32_t* row_idx, float scale, const void* element_table, int32_t heads,
    int32_t head_dim, int64_t stride_h, int64_t stride_s, void* stream) {
  if (element_table == nullptr) return RADIAL_ERR_INVALID_ARG;
  return bwd_varlen(q, k, v, o, dout, lse, dq, dk, dv, delta, seq_tokens, batch, row_ptr,
                    col_idx, col_ptr, row_idx, scale, 0, 0, 0, element_table, heads, head_dim,
                    stride_h, stride_s, stream);
}
