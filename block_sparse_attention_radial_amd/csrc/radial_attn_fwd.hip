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
// Work decomposition (one workgroup = 4 wave64 = one query block of 128 rows):
//  - wave w owns queries 32w .. 32w+31 of the block;
//  - S^T = K Q^T is computed on v_mfma_f32_32x32x16_bf16 with the keys on the M axis and
//    the queries on the N axis. Each lane then holds one query (lane % 32) and 64 of
//    the tile's 128 keys, so the row max and row sum are in-lane, plus one exchange
//    between the two half-waves;
//  - O^T = V^T P^T uses the same MFMA with head_dim on M and the queries on N. The
//    S^T accumulator layout is exactly the B-operand layout of this product, if the
//    keys along K are put in the order the accumulator holds them. So P goes from
//    registers straight into the MFMA, after one bf16 pack (v_cvt_pk_bf16_f32);
//  - K tiles sit in LDS key-major ([key][d], rows padded by 16 bytes). V tiles are
//    transposed on the way into LDS ([d][key position], rows padded by 16 bytes), with
//    key position = key with bits 2 and 3 swapped, which is that accumulator order;
//  - the next tile's global loads are issued before the current tile's MFMAs, so HBM/L2
//    latency hides behind compute;
//  - online softmax in base 2: with c = scale * log2(e), p = 2^(c*s - m), and the
//    running max m and sum l are kept per lane in fp32.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/radial_attn.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlockM = 128;   // query rows per workgroup (one CSR row)
constexpr int kBlockN = 128;   // keys per tile (one CSR column)
constexpr int kThreads = 256;  // 4 wave64
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D>
struct Tile {
  static constexpr int kRowK = D + 8;           // K tile row stride, bf16 elements
  static constexpr int kRowV = kBlockN + 8;     // V^T tile row stride, bf16 elements
  static constexpr int kChunks = D / 8;         // 16-byte chunks per token row
  static constexpr int kKLoads = kBlockN * kChunks / kThreads;  // K chunks per thread
  static constexpr int kVKeys = D / 16;         // keys per thread in the V transpose
  static constexpr int kVGroups = kBlockN / kVKeys;
  static constexpr int kLdsK = kBlockN * kRowK;  // elements
  static constexpr int kLdsV = D * kRowV;
  static_assert(kVGroups * kChunks == kThreads, "V staging must cover the tile");
  static_assert(kKLoads * kThreads == kBlockN * kChunks, "K staging must cover the tile");
};

// Key position inside a 128-key tile <-> key offset: swap bits 2 and 3 (an involution).
__device__ __forceinline__ int swap_bits23(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

__device__ __forceinline__ float other_half(float x) { return __shfl_xor(x, 32); }

__device__ __forceinline__ u32x4 load16(const __bf16* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

template <int D>
__global__ __launch_bounds__(kThreads) void radial_fwd_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ o, float* __restrict__ lse, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, int nb, int heads, int n, float c,
    int64_t stride_b, int64_t stride_h, int64_t stride_s) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(16))) __bf16 k_lds[T::kLdsK];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds[T::kLdsV];

  // Workgroups are handed to the 8 XCDs round-robin (XCD = id % 8). Give every XCD a
  // contiguous run of (head, query block) items so neighbouring query blocks of one
  // head, which read mostly the same K/V tiles, share that XCD's L2.
  const int grid = gridDim.x;
  const int pid = blockIdx.x;
  const int xcd = pid & 7, local = pid >> 3;
  const int per = grid >> 3, rem = grid & 7;
  const int item = (xcd < rem) ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  const int bh = item / nb;
  const int qb = item - bh * nb;
  const int b = bh / heads, h = bh - b * heads;
  const int64_t base = b * stride_b + h * stride_h;
  const __bf16* qh = q + base;
  const __bf16* kh = k + base;
  const __bf16* vh = v + base;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lq = lane & 31;   // query column owned by this lane
  const int hl = lane >> 5;   // half-wave

  // Q^T as MFMA B operand: lane holds d = 16s + 8hl .. +7 of its query, for every s.
  const int qrow = qb * kBlockM + wave * 32 + lq;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (qrow < n) raw = load16(qh + qrow * stride_s + 16 * s + 8 * hl);
    qf[s] = __builtin_bit_cast(bf16x8, raw);
  }

  // Staging registers for the next tile.
  u32x4 kreg[T::kKLoads];
  u32x4 vreg[T::kVKeys];
  const int vgrp = tid % T::kVGroups;  // which run of kVKeys key positions
  const int vchk = tid / T::kVGroups;  // which 8-wide slice of head_dim

  auto global_load = [&](int kb) {
    const bool valid = static_cast<unsigned>(kb) < static_cast<unsigned>(nb);
    const int key0 = kb * kBlockN;
#pragma unroll
    for (int r = 0; r < T::kKLoads; ++r) {
      const int chunk = tid + r * kThreads;
      const int key = chunk / T::kChunks, dc = chunk % T::kChunks;
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (valid && key0 + key < n) raw = load16(kh + (key0 + key) * stride_s + dc * 8);
      kreg[r] = raw;
    }
#pragma unroll
    for (int j = 0; j < T::kVKeys; ++j) {
      const int key = swap_bits23(vgrp * T::kVKeys + j);
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (valid && key0 + key < n) raw = load16(vh + (key0 + key) * stride_s + vchk * 8);
      vreg[j] = raw;
    }
  };

  auto lds_store = [&]() {
#pragma unroll
    for (int r = 0; r < T::kKLoads; ++r) {
      const int chunk = tid + r * kThreads;
      const int key = chunk / T::kChunks, dc = chunk % T::kChunks;
      *reinterpret_cast<u32x4*>(k_lds + key * T::kRowK + dc * 8) = kreg[r];
    }
    // Transpose kVKeys (keys) x 8 (d) bf16 in registers; each output row is one d.
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int w = e >> 1;
      uint32_t packed[T::kVKeys / 2];
#pragma unroll
      for (int jp = 0; jp < T::kVKeys / 2; ++jp) {
        const uint32_t a = vreg[2 * jp][w], bw = vreg[2 * jp + 1][w];
        packed[jp] = (e & 1) ? ((a >> 16) | (bw & 0xffff0000u)) : ((a & 0xffffu) | (bw << 16));
      }
      __bf16* dst = v_lds + (vchk * 8 + e) * T::kRowV + vgrp * T::kVKeys;
      if constexpr (T::kVKeys == 8) {
        *reinterpret_cast<u32x4*>(dst) = u32x4{packed[0], packed[1], packed[2], packed[3]};
      } else {
        *reinterpret_cast<u32x2*>(dst) = u32x2{packed[0], packed[1]};
      }
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;  // running max of c * s, base-2 units
  float l_run = 0.f;        // running sum of p over this lane's keys

  int it = row_ptr[qb];
  const int end = row_ptr[qb + 1];
  if (it < end) global_load(col_idx[it]);

  for (; it < end; ++it) {
    const int kb = col_idx[it];
    __syncthreads();  // all waves are done reading the previous tile
    lds_store();
    __syncthreads();
    if (it + 1 < end) global_load(col_idx[it + 1]);
    if (static_cast<unsigned>(kb) >= static_cast<unsigned>(nb)) continue;

    // ---- S^T = K Q^T : 4 key groups of 32 x (D/16) k-steps ----
    f32x16 sacc[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) sacc[g] = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
            k_lds + (32 * g + lq) * T::kRowK + 16 * s + 8 * hl);
        sacc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[g], 0, 0, 0);
      }
    }

    // ---- padding keys of the ragged last block ----
    const bool ragged = (kb + 1) * kBlockN > n;
    if (ragged) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb * kBlockN + 32 * g + 8 * (i >> 2) + 4 * hl + (i & 3);
          if (key >= n) sacc[g][i] = -INFINITY;
        }
    }

    // ---- online softmax ----
    float mx = -INFINITY;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[g][i]);
    mx = fmaxf(mx, other_half(mx));
    const float m_new = fmaxf(m_run, mx * c);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;
    const float neg_m = -m_new;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[g][i] = __builtin_amdgcn_exp2f(fmaf(sacc[g][i], c, neg_m));
    if (ragged) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb * kBlockN + 32 * g + 8 * (i >> 2) + 4 * hl + (i & 3);
          if (key >= n) sacc[g][i] = 0.f;
        }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int i = 0; i < 16; ++i) l_run += sacc[g][i];

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        f32x8 p8;
#pragma unroll
        for (int j = 0; j < 8; ++j) p8[j] = sacc[g][8 * s2 + j];
        const bf16x8 pf = __builtin_convertvector(p8, bf16x8);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16x8 vf = *reinterpret_cast<const bf16x8*>(
              v_lds + (32 * db + lq) * T::kRowV + 32 * g + 16 * s2 + 8 * hl);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, oacc[db], 0, 0, 0);
        }
      }
    }
  }

  // ---- epilogue: O / l, bf16, store rows < n ----
  const float l_tot = l_run + other_half(l_run);
  const float inv = 1.0f / l_tot;
  if (qrow < n) {
    __bf16* orow = o + base + qrow * stride_s;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        f32x4 x = {oacc[db][4 * ib + 0] * inv, oacc[db][4 * ib + 1] * inv,
                   oacc[db][4 * ib + 2] * inv, oacc[db][4 * ib + 3] * inv};
        const bf16x4 y = __builtin_convertvector(x, bf16x4);
        *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * ib + 4 * hl) = y;
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
  if (nb != (seqlen + kBlockM - 1) / kBlockM) return RADIAL_ERR_SHAPE_MISMATCH;
  if (stride_s < head_dim || stride_h < 0 || stride_b < 0) return RADIAL_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return RADIAL_ERR_MISALIGNED;
  if ((stride_s | stride_h | stride_b) & 7) return RADIAL_ERR_MISALIGNED;
  const int64_t items = static_cast<int64_t>(batch) * heads * nb;
  if (items > INT32_MAX || static_cast<int64_t>(batch) * heads * seqlen > INT64_MAX / 4)
    return RADIAL_ERR_TOO_LARGE;

  const float c = scale * kLog2e;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<uint32_t>(items)), block(kThreads);
  const auto* qq = static_cast<const __bf16*>(q);
  const auto* kk = static_cast<const __bf16*>(k);
  const auto* vv = static_cast<const __bf16*>(v);
  auto* oo = static_cast<__bf16*>(o);
  if (head_dim == 128) {
    hipLaunchKernelGGL(radial_fwd_kernel<128>, grid, block, 0, st, qq, kk, vv, oo, lse, row_ptr,
                       col_idx, nb, heads, seqlen, c, stride_b, stride_h, stride_s);
  } else {
    hipLaunchKernelGGL(radial_fwd_kernel<64>, grid, block, 0, st, qq, kk, vv, oo, lse, row_ptr,
                       col_idx, nb, heads, seqlen, c, stride_b, stride_h, stride_s);
  }
  return hipGetLastError() == hipSuccess ? RADIAL_OK : RADIAL_ERR_HIP;
}
