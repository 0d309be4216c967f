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
// Work decomposition: one workgroup = 4 wave64 = one query block of 128 rows. Each wave
// owns 32 query rows. Two workgroups share a CU, so each SIMD runs two waves: while one
// wave is in its softmax (VALU) the other keeps the matrix core busy. The register
// budget is therefore 256 per lane, with no accumulator spills.
//
//  - S^T = K Q^T runs on v_mfma_f32_32x32x16_bf16, with keys on M and queries on N. A
//    lane then holds one query (lane % 32) and 64 of the tile's 128 keys. The row max
//    and row sum are in-lane, plus one exchange between the half-waves
//    (v_permlane32_swap).
//  - O^T = V^T P^T uses the same MFMA with head_dim on M and queries on N. The S^T
//    accumulator of a lane is, key for key, the B operand this product needs once the
//    contraction runs over keys in accumulator order, so P goes from registers into the
//    MFMA after one bf16 pack.
//  - K and V tiles are both stored key-major in LDS ([key][d], no padding). Each 16-byte
//    chunk of a row is XOR-swizzled by a function of the row, so the K reads
//    (ds_read_b128, 8 rows per bank cycle) and the transposed V reads
//    (ds_read_b64_tr_b16, 4 rows x 32 bytes per 16-lane group) hit distinct banks.
//  - ds_read_b64_tr_b16 gives a lane 4 keys of one V column. Two of them form the V^T
//    A operand of one MFMA, so no register transpose is needed.
//  - Tiles go HBM/L2 -> registers -> LDS with buffer loads. The descriptor's range check
//    returns zeros past the sequence end, so the ragged last block needs no branches.
//    The next K tile is fetched while QK^T and the softmax run, and the next V tile
//    while PV runs.
//  - Online softmax in base 2: c = scale * log2(e), p = 2^(c*s - m). The running max m
//    moves only when a tile's max exceeds it by more than 2^8 for some row of the wave.
//    Until then p <= 256, and O and l are not rescaled. The final O / l is exact for
//    any m used consistently. The row sum adds the bf16-rounded p, the same values the
//    PV product multiplies.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
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
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kBlock = 128;    // query rows per workgroup, keys per tile
constexpr int kThreads = 256;  // 4 wave64
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;  // log2 units: p stays <= 256 between rescales
// Fourth dword of a raw gfx9 buffer descriptor: 32-bit data format, no stride/swizzle.
constexpr int kBufferFlags = 0x00020000;

template <int D>
struct Tile {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;                        // 16-byte chunks per row
  static constexpr int kLoads = kBlock * kChunks / kThreads;   // chunks per thread per tile
  static constexpr int kLdsElems = kBlock * D;
  static_assert(kLoads * kThreads == kBlock * kChunks, "staging must cover the tile");
};

// Bank swizzle: chunk c of row r lives at chunk position c ^ swz(r). Within 8
// consecutive rows swz takes all of 0..7 (K reads), and within rows 4h..4h+3 it takes
// {0, 2, 4, 6} + h (V transposed reads, whose 16-lane groups touch 4 rows x 2 chunks).
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferFlags);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, int byte_offset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, 0));
}

// Reduction over the two half-waves: for a symmetric op, op(lo, hi) of the pair
// returned by v_permlane32_swap(x, x) is the same in every lane.
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

template <int D>
__global__ __launch_bounds__(kThreads, 2) void radial_fwd_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ o, float* __restrict__ lse, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, int nb, int heads, int n, float c,
    int64_t stride_b, int64_t stride_h, int stride_s) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(16))) __bf16 k_lds[T::kLdsElems];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds[T::kLdsElems];

  // Workgroups are handed to the 8 XCDs round-robin (XCD = id % 8). Give every XCD a
  // contiguous run of (head, query block) items, so neighbouring query blocks of one
  // head, which read mostly the same K/V tiles, share that XCD's L2.
  const int grid = gridDim.x;
  const int pid = blockIdx.x;
  const int xcd = pid & 7, local = pid >> 3;
  const int per = grid >> 3, rem = grid & 7;
  const int item =
      (xcd < rem) ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  const int bh = item / nb;
  const int qb = item - bh * nb;
  const int b = bh / heads, h = bh - b * heads;
  const int64_t base = b * stride_b + h * stride_h;
  const int row_bytes = stride_s * 2;  // bytes between consecutive tokens

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lq = lane & 31;  // query column owned by this lane
  const int hl = lane >> 5;  // half-wave

  // ---- Q^T as the MFMA B operand: d = 16s + 8hl .. +7 of this lane's query ----
  bf16x8 qf[D / 16];
  {
    const int q0 = qb * kBlock;
    const int rows = min(kBlock, n - q0);
    const auto rq = make_rsrc(q + base + static_cast<int64_t>(q0) * stride_s,
                              (rows - 1) * row_bytes + T::kRowBytes);
    const int off = (wave * 32 + lq) * row_bytes + hl * 16;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[s] = __builtin_bit_cast(bf16x8, buffer_load16(rq, off + s * 32));
  }

  // ---- staging: thread's chunks of a tile, fixed offsets for every tile ----
  int g_off[T::kLoads];    // byte offset in global memory from the tile's first row
  int l_off[T::kLoads];    // byte offset in LDS (swizzled)
#pragma unroll
  for (int r = 0; r < T::kLoads; ++r) {
    const int idx = tid + r * kThreads;
    const int row = idx / T::kChunks, ch = idx % T::kChunks;
    g_off[r] = row * row_bytes + ch * 16;
    l_off[r] = row * T::kRowBytes + ((ch ^ swz(row)) << 4);
  }
  u32x4 stg[T::kLoads];
  const __bf16* kh = k + base;
  const __bf16* vh = v + base;
  auto fetch = [&](const __bf16* src, int kb) {
    const bool valid = static_cast<unsigned>(kb) < static_cast<unsigned>(nb);
    const int key0 = valid ? kb * kBlock : 0;
    const int rows = valid ? min(kBlock, n - key0) : 0;
    const auto r = make_rsrc(src + static_cast<int64_t>(key0) * stride_s,
                             rows > 0 ? (rows - 1) * row_bytes + T::kRowBytes : 0);
#pragma unroll
    for (int i = 0; i < T::kLoads; ++i) stg[i] = buffer_load16(r, g_off[i]);
  };
  auto stash = [&](__bf16* dst) {
    char* d = reinterpret_cast<char*>(dst);
#pragma unroll
    for (int i = 0; i < T::kLoads; ++i) *reinterpret_cast<u32x4*>(d + l_off[i]) = stg[i];
  };

  // ---- per-lane LDS read offsets for the MFMA operands (bytes) ----
  // K (A operand of S^T): row 32g + lq, chunk 2s + hl.
  const int k_rd = lq * T::kRowBytes;
  const int k_sw = swz(lq);
  // V^T (A operand of O^T) via ds_read_b64_tr_b16: in 16-lane group gi, source lane s
  // points at key 4hl + s/4 (+ tile offsets) and d = 32db + 16(gi&1) + 4(s&3).
  const int gi = (lane >> 4) & 3, sl = lane & 15;
  const int v_key = 4 * hl + (sl >> 2);
  const int v_rd = v_key * T::kRowBytes + 8 * (sl & 1);
  const int v_sw = swz(v_key);
  const int v_ch = 2 * (gi & 1) + ((sl & 3) >> 1);

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;  // max of c * s used for p, base-2 units
  float l_run = 0.f;        // sum of bf16(p) over this lane's keys

  const int start = row_ptr[qb];
  const int end = row_ptr[qb + 1];
  if (start < end) {
    fetch(kh, col_idx[start]);
    stash(k_lds);
    fetch(vh, col_idx[start]);
    stash(v_lds);
  }
  __syncthreads();

  const char* k_bytes = reinterpret_cast<const char*>(k_lds);
  const char* v_bytes = reinterpret_cast<const char*>(v_lds);

  for (int it = start; it < end; ++it) {
    const int kb = col_idx[it];
    const bool has_next = it + 1 < end;
    const int kb_next = has_next ? col_idx[it + 1] : 0;
    const bool valid = static_cast<unsigned>(kb) < static_cast<unsigned>(nb);
    if (has_next) fetch(kh, kb_next);

    bf16x8 pf[8];  // P^T as B operands: [4 * g + ... ] packed per (g, s2)
    if (valid) {
      // ---- S^T = K Q^T ----
      f32x16 sacc[4];
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const int ch = ((2 * s + hl) ^ k_sw) << 4;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(k_bytes + k_rd + g * 32 * T::kRowBytes + ch);
          // The first k-step takes an inline zero accumulator.
          sacc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], s == 0 ? f32x16{} : sacc[g],
                                                            0, 0, 0);
        }
      }

      // ---- padding keys of the ragged last block ----
      const int key_lim = n - kb * kBlock;  // keys at or past this index are padding
      if (key_lim < kBlock) {
        // Key of accumulator entry (g, i) is 32g + 8(i/4) + (i%4) + 4hl: compare the
        // constant part against one per-lane limit.
        const int lim = key_lim - 4 * hl;
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * g + 8 * (i >> 2) + (i & 3) >= lim) sacc[g][i] = -INFINITY;
      }

      // ---- online softmax ----
      float mx = -INFINITY;
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[g][i]);
      const float m_tile = halves_max(mx) * c;
      if (__builtin_amdgcn_ballot_w64(m_tile > m_run + kRescaleThreshold) != 0) {
        const float m_new = fmaxf(m_run, m_tile);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;
      }
      const float neg_m = -m_run;
      const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          f32x8 p8;
#pragma unroll
          for (int j = 0; j < 8; ++j)
            p8[j] = __builtin_amdgcn_exp2f(fmaf(sacc[g][8 * s2 + j], c, neg_m));
          pf[2 * g + s2] = __builtin_convertvector(p8, bf16x8);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bf16x2 pair = {pf[2 * g + s2][2 * j], pf[2 * g + s2][2 * j + 1]};
            l_run = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, l_run, false);
          }
        }
    }

    __syncthreads();  // every wave is done reading K(it)
    if (has_next) {
      stash(k_lds);
      fetch(vh, kb_next);
    }

    if (valid) {
      // ---- O^T += V^T P^T ----
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const int ch = ((4 * db + v_ch) ^ v_sw) << 4;
            const char* p0 = v_bytes + v_rd + (32 * g + 16 * s2) * T::kRowBytes + ch;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4*)(p0));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4*)(p0 + 8 * T::kRowBytes));
            const bf16x8 vf = __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo),
                                                      __builtin_bit_cast(bf16x4, hi),
                                                      0, 1, 2, 3, 4, 5, 6, 7);
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[2 * g + s2], oacc[db], 0, 0, 0);
          }
        }
    }

    __syncthreads();  // every wave is done reading V(it); K(it + 1) is in LDS
    if (has_next) stash(v_lds);
  }

  // ---- epilogue: O / l, bf16, store rows < n ----
  const float l_tot = halves_sum(l_run);
  const float inv = 1.0f / l_tot;
  const int qrow = qb * kBlock + wave * 32 + lq;
  if (qrow < n) {
    __bf16* orow = o + base + static_cast<int64_t>(qrow) * stride_s;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        const f32x4 x = {oacc[db][4 * ib + 0] * inv, oacc[db][4 * ib + 1] * inv,
                         oacc[db][4 * ib + 2] * inv, oacc[db][4 * ib + 3] * inv};
        *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * ib + 4 * hl) = __builtin_convertvector(x, bf16x4);
      }
    if (lse != nullptr && hl == 0)
      lse[static_cast<int64_t>(bh) * n + qrow] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
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
  const int64_t items = static_cast<int64_t>(batch) * heads * nb;
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
