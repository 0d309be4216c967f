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
//  1. delta: D_i for every row (fp32, into a caller workspace).
//  2. dq: one workgroup per (batch, head, query block), walking the block's CSR row. Per
//     key tile: S^T = K Q^T and dP^T = V dO^T on MFMA (keys on M, queries on N, K and V
//     rows from LDS, Q^T and dO^T in registers), P^T and dS^T in registers, then
//     dQ^T += K^T dS^T with K^T from transposing LDS reads: the dS^T accumulator is,
//     key for key, the B operand of that product, as P^T is for O^T in the forward.
//  3. dkdv: one workgroup per (batch, head, key block), walking the block's column of
//     the mask (the transposed CSR). Per query tile: S = Q K^T and dP = dO V^T (queries
//     on M, keys on N, Q and dO rows from LDS, K and V in registers), P and dS, then
//     dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T from transposing LDS reads.
// A workgroup is four wave64, one per SIMD; wave i owns rows (dq) or keys (dkdv)
// 32i .. 32i+31 of its block. Tiles are copied HBM/L2 -> LDS with LDS-DMA into two
// buffers: tile t+1 is in flight while tile t is used. Accumulation is fp32; P and dS
// enter the MFMAs as bf16. Padding (rows or keys at or past n) and element masking work
// as in the forward.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <climits>
#include <cmath>
#include <cstdint>

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
  float* delta;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const int32_t* col_ptr;
  const int32_t* row_idx;
  int64_t stride_b, stride_h;
  int nb, heads, n, stride_s;
  int elem_s, elem_gw, elem_w0;  // element masking: frame length, grid width, W0
  float c;      // scale * log2(e)
  float scale;
  // varlen: 0 for a uniform batch, else the number of samples in `plan`; q, k, v, o, dO,
  // dq, dk, dv are then one packed sequence of n tokens, and lse, delta are [heads, n].
  int varlen;
  BwdSample plan[kMaxBwdVarlen];
};
typedef __attribute__((address_space(4))) const BwdArgs* BwdArgsPtr;

// Where a dq or dkdv workgroup works: the (batch, head) element offset, its rows of lse
// and delta, its mask rows (row_ptr / col_ptr point at its sample's), its sequence length
// and block count, and its block. Varlen plans are read from the kernel-argument segment
// (scalar loads; a copy of the plan would go to scratch memory under a dynamic index).
struct BwdGeometry {
  int64_t base;
  const float* lse;
  const float* delta;
  const int32_t* row_ptr;
  const int32_t* col_ptr;
  int n, nb, blk;
};

__device__ __forceinline__ BwdGeometry bwd_geometry(const BwdArgs& a, int wg) {
  BwdGeometry g;
  if (a.varlen == 0) {
    const int bh = wg / a.nb;
    const int b = bh / a.heads, h = bh - b * a.heads;
    g.base = b * a.stride_b + h * a.stride_h;
    g.lse = a.lse + static_cast<int64_t>(bh) * a.n;
    g.delta = a.delta + static_cast<int64_t>(bh) * a.n;
    g.row_ptr = a.row_ptr;
    g.col_ptr = a.col_ptr;
    g.n = a.n;
    g.nb = a.nb;
    g.blk = wg - bh * a.nb;
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
  g.lse = a.lse + static_cast<int64_t>(h) * a.n + tok0;
  g.delta = a.delta + static_cast<int64_t>(h) * a.n + tok0;
  g.row_ptr = a.row_ptr + rp0;
  g.col_ptr = a.col_ptr + rp0;
  g.n = ap->plan[lo].n;
  g.nb = nb;
  g.blk = wg - ap->plan[lo].wg0 - h * nb;
  return g;
}

// ---- 1. D_i = <do_i, o_i> ----
// D / 8 lanes per row, 8 bf16 each; 256 / (D / 8) rows per workgroup.
template <int D>
__global__ __launch_bounds__(kBwdThreads) void radial_bwd_delta_kernel(const BwdArgs a,
                                                                       int rows_total) {
  constexpr int kLanes = D / 8;
  const int tid = threadIdx.x;
  const int r = blockIdx.x * (kBwdThreads / kLanes) + tid / kLanes;
  const int ch = tid % kLanes;
  float acc = 0.f;
  if (r < rows_total) {
    // Row r of delta's layout: [batch, heads, n], or [heads, n] of a packed varlen batch.
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
  if (r < rows_total && ch == 0) a.delta[r] = acc;
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

// ---- 2. dQ ----
template <int D, int E>
__global__ __launch_bounds__(kBwdThreads, 1) void radial_bwd_dq_kernel(const BwdArgs a) {
  using T = Tile<D>;
  constexpr int NDB = D / 32, NS = D / 16;
  __shared__ __attribute__((aligned(1024))) char smem[4 * T::kBytes];
  char* const kb0 = smem;
  char* const vb0 = smem + 2 * T::kBytes;

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
    lse2 = geo.lse[qrow] * kLog2e;
    dlt = geo.delta[qrow];
  }
  int copy_off[T::kOffsetPeriod];
  copy_offsets<D>(wi, lane, row_bytes, copy_off);
  int rbase, rx, tb0, tx0, tb1, tx1;
  row_read_offsets<D>(lane, rbase, rx);
  tr_read_offsets<D>(lane, tb0, tx0, tb1, tx1);

  const int r0 = geo.row_ptr[qb];
  const int L = geo.row_ptr[qb + 1] - r0;
  auto column = [&](int t) { return __builtin_amdgcn_readfirstlane(a.col_idx[r0 + t]); };
  auto copy_tile = [&](int t) {
    const int kb = column(t);
    const bool on = static_cast<unsigned>(kb) < static_cast<unsigned>(nb);
    const int buf = (t & 1) * T::kBytes;
    const Stage<D> sk = stage_rows<D>(kb0 + buf, kh, kb * kBlock, n, row_bytes, wi, on);
    const Stage<D> sv = stage_rows<D>(vb0 + buf, vh, kb * kBlock, n, row_bytes, wi, on);
#pragma unroll
    for (int i = 0; i < T::kCopiesPerWave; ++i) {
      stage_issue<D>(sk, copy_off, i);
      stage_issue<D>(sv, copy_off, i);
    }
  };
  if (L > 0) copy_tile(0);

  // Q^T and dO^T as MFMA B operands: d = 16s + 8hl .. +7 of this lane's query.
  u32x4 qf[NS], gf[NS];
  load_b_operand<D>(a.q + base, q0, n, row_bytes, 32 * wi + lq, hl, qf);
  load_b_operand<D>(a.g + base, q0, n, row_bytes, 32 * wi + lq, hl, gf);
  __builtin_amdgcn_s_waitcnt(0);  // Q, dO and the first tile (see the forward prologue)

  f32x16 dq[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dq[i] = f32x16{};

  for (int t = 0; t < L; ++t) {
    wait_copies<0>();  // this wave's part of tile t
    lds_barrier();     // every wave's part landed; tile t-1 is no longer read
    if (t + 1 < L) copy_tile(t + 1);
    const int kb = column(t);
    if (static_cast<unsigned>(kb) >= static_cast<unsigned>(nb)) continue;
    const char* const kt = kb0 + (t & 1) * T::kBytes;
    const char* const vt = vb0 + (t & 1) * T::kBytes;

    // S^T = K Q^T and dP^T = V dO^T (keys on M, this wave's queries on N).
    f32x16 sacc[4], pacc[4];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      bf16x8 kf[4], vf[4];
      read_rows<D>(kt + rbase, rx, s, kf);
      read_rows<D>(vt + rbase, rx, s, vf);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        sacc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            kf[g], __builtin_bit_cast(bf16x8, qf[s]), s == 0 ? f32x16{} : sacc[g], 0, 0, 0);
        pacc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            vf[g], __builtin_bit_cast(bf16x8, gf[s]), s == 0 ? f32x16{} : pacc[g], 0, 0, 0);
      }
    }
    if (n - kb * kBlock < kBlock) pad_mask_tile(kb * kBlock, n, lane, sacc);
    if constexpr (E != 0)
      element_mask_any<E>(q0 + 32 * wi, kb * kBlock, a.elem_s, a.elem_gw, a.elem_w0 - 1, lane, sacc);

    // Per step u of 16 keys: P^T = 2^(c s - lse2) and dS^T = P^T (dP^T - D), packed as
    // the B operand of dQ^T += K^T dS^T (d on M, queries on N, keys contracted in
    // accumulator order), whose MFMAs are issued right away: they run while the VALU
    // works on step u + 1.
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int g = u >> 1, s2 = u & 1;
      f32x8 d8;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[g][8 * s2 + jj], a.c, -lse2));
        d8[jj] = p * (pacc[g][8 * s2 + jj] - dlt);
      }
      const bf16x8 dsk = __builtin_convertvector(d8, bf16x8);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr<D>(kt, tb0, tx0, tb1, tx1, u, db),
                                                         dsk, dq[db], 0, 0, 0);
    }
  }
  if (qrow < n) store_rows<D>(a.dq + base + static_cast<int64_t>(qrow) * a.stride_s, dq, a.scale, hl);
}

// ---- 3. dK, dV ----
template <int D, int E>
__global__ __launch_bounds__(kBwdThreads, 1) void radial_bwd_dkdv_kernel(const BwdArgs a) {
  using T = Tile<D>;
  constexpr int NDB = D / 32, NS = D / 16;
  // Q and dO tiles (two of each), then lse and D of the tile's 128 queries (two of each,
  // 1 KiB apiece: one 1 KiB copy writes 128 values and zeros after them).
  __shared__ __attribute__((aligned(1024))) char smem[4 * T::kBytes + 4 * 1024];
  char* const qb0 = smem;
  char* const gb0 = smem + 2 * T::kBytes;
  char* const lb0 = smem + 4 * T::kBytes;          // lse, buffers 0 and 1
  char* const db0 = smem + 4 * T::kBytes + 2048;   // D, buffers 0 and 1

  const BwdGeometry geo = bwd_geometry(a, blockIdx.x);
  const int nb = geo.nb, n = geo.n, kb = geo.blk;
  const int64_t base = geo.base;
  const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, hl = lane >> 5;
  const int wi = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row_bytes = a.stride_s * 2;
  const int k0 = kb * kBlock;
  const int krow = k0 + 32 * wi + lq;
  const char* const qh = reinterpret_cast<const char*>(a.q + base);
  const char* const gh = reinterpret_cast<const char*>(a.g + base);
  const float* const lse_bh = geo.lse;
  const float* const dl_bh = geo.delta;

  int copy_off[T::kOffsetPeriod];
  copy_offsets<D>(wi, lane, row_bytes, copy_off);
  int rbase, rx, tb0, tx0, tb1, tx1;
  row_read_offsets<D>(lane, rbase, rx);
  tr_read_offsets<D>(lane, tb0, tx0, tb1, tx1);

  const int c0 = geo.col_ptr[kb];
  const int L = geo.col_ptr[kb + 1] - c0;
  auto qblock = [&](int t) { return __builtin_amdgcn_readfirstlane(a.row_idx[c0 + t]); };
  auto copy_tile = [&](int t) {
    const int qb = qblock(t);
    const bool on = static_cast<unsigned>(qb) < static_cast<unsigned>(nb);
    const int buf = (t & 1) * T::kBytes;
    const Stage<D> sq = stage_rows<D>(qb0 + buf, qh, qb * kBlock, n, row_bytes, wi, on);
    const Stage<D> sg = stage_rows<D>(gb0 + buf, gh, qb * kBlock, n, row_bytes, wi, on);
#pragma unroll
    for (int i = 0; i < T::kCopiesPerWave; ++i) {
      stage_issue<D>(sq, copy_off, i);
      stage_issue<D>(sg, copy_off, i);
    }
    if (wi == 0) {  // lse and D of the 128 queries: 512 bytes each
      const int rows = on ? (n - qb * kBlock < kBlock ? n - qb * kBlock : kBlock) : 0;
      const int q0 = on ? qb * kBlock : 0;
      const uint32_t lb = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)lb0)) +
                          (t & 1) * 1024;
      const uint32_t dbv = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)db0)) +
                           (t & 1) * 1024;
      copy_1k(raw_descriptor(reinterpret_cast<const char*>(lse_bh + q0), rows * 4), lb, lane * 16);
      copy_1k(raw_descriptor(reinterpret_cast<const char*>(dl_bh + q0), rows * 4), dbv, lane * 16);
    }
  };
  if (L > 0) copy_tile(0);

  // K and V as MFMA B operands: d = 16s + 8hl .. +7 of this lane's key.
  u32x4 kf[NS], vf[NS];
  load_b_operand<D>(a.k + base, k0, n, row_bytes, 32 * wi + lq, hl, kf);
  load_b_operand<D>(a.v + base, k0, n, row_bytes, 32 * wi + lq, hl, vf);
  __builtin_amdgcn_s_waitcnt(0);

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dk[i] = dv[i] = f32x16{};

  for (int t = 0; t < L; ++t) {
    wait_copies<0>();
    lds_barrier();
    if (t + 1 < L) copy_tile(t + 1);
    const int qb = qblock(t);
    if (static_cast<unsigned>(qb) >= static_cast<unsigned>(nb)) continue;
    const char* const qt = qb0 + (t & 1) * T::kBytes;
    const char* const gt = gb0 + (t & 1) * T::kBytes;
    const float* const lt = reinterpret_cast<const float*>(lb0 + (t & 1) * 1024);
    const float* const dt = reinterpret_cast<const float*>(db0 + (t & 1) * 1024);

    // S = Q K^T and dP = dO V^T (queries on M, this wave's keys on N).
    f32x16 sacc[4], pacc[4];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      bf16x8 qf[4], gf[4];
      read_rows<D>(qt + rbase, rx, s, qf);
      read_rows<D>(gt + rbase, rx, s, gf);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        sacc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            qf[g], __builtin_bit_cast(bf16x8, kf[s]), s == 0 ? f32x16{} : sacc[g], 0, 0, 0);
        pacc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            gf[g], __builtin_bit_cast(bf16x8, vf[s]), s == 0 ? f32x16{} : pacc[g], 0, 0, 0);
      }
    }
    // Entries are queries here: padding rows and the element rule mask them.
    if (n - qb * kBlock < kBlock) pad_mask_tile(qb * kBlock, n, lane, sacc);
    if constexpr (E != 0)
      element_mask_any<E>(k0 + 32 * wi, qb * kBlock, a.elem_s, a.elem_gw, a.elem_w0 - 1, lane, sacc);

    // P = 2^(c s - lse2) and dS = P (dP - D), per entry (query 32g + 8(e/4) + 4hl + e%4),
    // packed as the B operands of dV^T and dK^T. (Issuing each step's MFMAs right after
    // its P and dS, as the dQ kernel does, measured 7% slower here: this kernel holds
    // every register, and the compiler then schedules worse.)
    bf16x8 pk[8], dsk[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int g = u >> 1, s2 = u & 1;
      f32x8 p8, d8;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int qi = 32 * g + 8 * (2 * s2 + half) + 4 * hl;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lt + qi);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(dt + qi);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = 8 * s2 + 4 * half + r;
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[g][e], a.c, -l4[r] * kLog2e));
          p8[4 * half + r] = p;
          d8[4 * half + r] = p * (pacc[g][e] - d4[r]);
        }
      }
      pk[u] = __builtin_convertvector(p8, bf16x8);
      dsk[u] = __builtin_convertvector(d8, bf16x8);
    }
    // dV^T += dO^T P and dK^T += Q^T dS (d on M, keys on N, queries contracted).
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr<D>(gt, tb0, tx0, tb1, tx1, u, db),
                                                         pk[u], dv[db], 0, 0, 0);
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr<D>(qt, tb0, tx0, tb1, tx1, u, db),
                                                         dsk[u], dk[db], 0, 0, 0);
      }
  }
  if (krow < n) {
    const int64_t off = base + static_cast<int64_t>(krow) * a.stride_s;
    store_rows<D>(a.dv + off, dv, 1.0f, hl);
    store_rows<D>(a.dk + off, dk, a.scale, hl);
  }
}

bool aligned(const void* p, uintptr_t m) { return (reinterpret_cast<uintptr_t>(p) & (m - 1)) == 0; }

template <int D, int E>
void launch_bwd(const BwdArgs& args, int rows_total, int items, hipStream_t st) {
  constexpr int kRowsPerBlock = kBwdThreads / (D / 8);
  hipLaunchKernelGGL((radial_bwd_delta_kernel<D>), dim3((rows_total + kRowsPerBlock - 1) / kRowsPerBlock),
                     dim3(kBwdThreads), 0, st, args, rows_total);
  hipLaunchKernelGGL((radial_bwd_dq_kernel<D, E>), dim3(items), dim3(kBwdThreads), 0, st, args);
  hipLaunchKernelGGL((radial_bwd_dkdv_kernel<D, E>), dim3(items), dim3(kBwdThreads), 0, st, args);
}

// The three kernels of one call, at the template instance of head_dim and the element
// mode (none, 1-D distance, grid distance).
int32_t launch_all(const BwdArgs& args, int rows_total, int items, int head_dim,
                   int32_t element_tokens_per_frame, int32_t element_grid_w, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int mode = element_tokens_per_frame == 0 ? 0 : (element_grid_w == 0 ? 1 : 2);
  if (head_dim == 128) {
    if (mode == 2) launch_bwd<128, 2>(args, rows_total, items, st);
    else if (mode == 1) launch_bwd<128, 1>(args, rows_total, items, st);
    else launch_bwd<128, 0>(args, rows_total, items, st);
  } else {
    if (mode == 2) launch_bwd<64, 2>(args, rows_total, items, st);
    else if (mode == 1) launch_bwd<64, 1>(args, rows_total, items, st);
    else launch_bwd<64, 0>(args, rows_total, items, st);
  }
  return hipGetLastError() == hipSuccess ? RADIAL_OK : RADIAL_ERR_HIP;
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
  if ((stride_s | stride_h | stride_b) & 7) return RADIAL_ERR_MISALIGNED;
  const int64_t items = static_cast<int64_t>(batch) * heads * nb;
  const int64_t rows_total = static_cast<int64_t>(batch) * heads * seqlen;
  if (items > INT32_MAX || rows_total > INT32_MAX || stride_s > (INT32_MAX / 2) / kBlock)
    return RADIAL_ERR_TOO_LARGE;

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
  args.stride_b = stride_b;
  args.stride_h = stride_h;
  args.nb = nb;
  args.heads = heads;
  args.n = seqlen;
  args.stride_s = static_cast<int>(stride_s);
  args.elem_s = element_tokens_per_frame;
  args.elem_gw = element_grid_w;
  args.elem_w0 = element_w0;
  args.c = scale * kLog2e;
  args.scale = scale;
  args.varlen = 0;
  return launch_all(args, static_cast<int>(rows_total), static_cast<int>(items), head_dim,
                    element_tokens_per_frame, element_grid_w, stream);
}

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
  args.c = scale * kLog2e;
  args.scale = scale;
  args.varlen = batch;
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
  return launch_all(args, static_cast<int>(heads * tok), static_cast<int>(wgs), head_dim,
                    element_tokens_per_frame, element_grid_w, stream);
}
