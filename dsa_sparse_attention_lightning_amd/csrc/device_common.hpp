// Device-side building blocks shared by the gfx950 kernels: vector types,
// MFMA wrappers, order-preserving float keys and block-wide scans.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;

constexpr int kWave = 64;

// ---------------------------------------------------------------- MFMA
// 32x32 output tiles: lane l holds column (l & 31) and rows
// 8*(r/4) + 4*(l/32) + (r%4) for accumulator register r in 0..15.
// Operand A: lane l holds row (l & 31); operand B: column (l & 31); the
// reduction index inside a lane follows the same order for A and B, so any
// consistent assignment of reduction indices to (lane/32, element) works.
__device__ __forceinline__ f32x16 mfma32_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// fp8 e4m3 x fp8 e4m3, 64-deep reduction, unit block scales (E8M0 127 = 1.0).
__device__ __forceinline__ f32x16 mfma32_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
// 16x16 output tiles: lane l holds column (l & 15), rows 4*(l/16) + r.
__device__ __forceinline__ f32x4 mfma16_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- loads
__device__ __forceinline__ i32x4 ld16(const void* p) {
  return *reinterpret_cast<const i32x4*>(p);
}
__device__ __forceinline__ i32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p));
}
__device__ __forceinline__ bf16x8 as_bf16x8(i32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  // round to nearest even (inputs are finite)
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// ---------------------------------------------------------------- keys
// Order-preserving map float -> uint32: a > b (as floats, -0 == +0) iff
// key(a) > key(b).  -0 is folded onto +0 so equal values get equal keys.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- scans
// Inclusive prefix sum over the 64 lanes of a wave with DPP lane moves (no
// LDS round trips): shifts by 1, 2, 4, 8 inside each 16-lane row, then lane
// 15's total is added to rows 1 and 3 and lane 31's to rows 2 and 3.  A lane
// whose source lies outside its row receives 0.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  int v = (int)x;
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return (uint32_t)v;
}

// Inclusive prefix sum over lanes 0..15 (one DPP row); other lanes unused.
__device__ __forceinline__ uint32_t row16_incl_scan(uint32_t x) {
  int v = (int)x;
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  return (uint32_t)v;
}

// Block-wide exclusive prefix sum of one value per thread.  `scratch` holds
// NW words of LDS.  Returns the exclusive prefix; `total` gets the sum.
// Contains two __syncthreads, so every thread of the block must call it.
// The wave totals are scanned by every wave at once (lane i reads wave i's
// total, one DPP row scan, two lane reads), so the cross-wave step costs a
// handful of instructions per wave whatever NW is.
template <int NW>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* scratch,
                                                    uint32_t& total) {
  static_assert(NW >= 1 && NW <= 16, "wave totals fit one DPP row");
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  uint32_t incl = wave_incl_scan(v);
  if (lane == kWave - 1) scratch[wid] = incl;
  __syncthreads();
  const uint32_t ti = row16_incl_scan(lane < NW ? scratch[lane] : 0u);
  const uint32_t before = wid > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)ti, wid - 1) : 0u;
  total = (uint32_t)__builtin_amdgcn_readlane((int)ti, NW - 1);
  __syncthreads();
  return before + incl - v;
}

// ---------------------------------------------------------------- radix select
// Find the bin holding the kk-th largest element of a histogram of NB bins in
// LDS (bins scanned from the top): writes {bin, count strictly above it} to
// sel[0..1] in LDS.  `scan` holds NTH / 64 words.  All NTH threads call it;
// it ends with a barrier.
template <int NB, int NTH>
__device__ void select_bin(const uint32_t* hist, uint32_t kk, uint32_t* scan, uint32_t* sel) {
  constexpr int PER = NB / NTH;  // bins per thread
  const int tid = threadIdx.x;
  uint32_t c[PER];
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    c[i] = hist[NB - 1 - (tid * PER + i)];
    sum += c[i];
  }
  uint32_t total;
  uint32_t above = block_excl_scan<NTH / kWave>(sum, scan, total);
  // one bin of one thread holds the kk-th element: find it in registers and
  // write once
  int hit = -1;
  uint32_t hit_above = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (above < kk && kk <= above + c[i]) {
      hit = i;
      hit_above = above;
    }
    above += c[i];
  }
  if (hit >= 0) {
    sel[0] = NB - 1 - (tid * PER + hit);
    sel[1] = hit_above;
  }
  __syncthreads();
}

// The same selection by one wave and no barrier (the caller synchronises):
// lane l sums bins [NB - PER (l + 1), NB - PER l) (PER = NB / 64, read
// with a per-lane rotation so the lanes spread over the LDS banks), a wave
// prefix sum finds the lane whose range holds the kk-th largest, and the
// wave then scans that lane's PER bins one per lane.  Writes {bin, count
// strictly above it} to sel[0..1]; kk must be in [1, total].
template <int NB>
__device__ void wave_select_bin(const uint32_t* hist, uint32_t kk, uint32_t* sel) {
  constexpr int PER = NB / kWave;
  constexpr int V = PER / 4;
  static_assert(PER % 4 == 0 && PER <= kWave && (V & (V - 1)) == 0, "whole vectors per lane");
  const int lane = threadIdx.x & (kWave - 1);
  const int lo = NB - PER * (lane + 1);
  uint32_t sum = 0;
  if constexpr (V <= 4) {  // every read in flight before the first add
    uint4 x[V];
#pragma unroll
    for (int i = 0; i < V; ++i)
      x[i] = *reinterpret_cast<const uint4*>(hist + lo + 4 * ((i + lane) & (V - 1)));
#pragma unroll
    for (int i = 0; i < V; ++i) sum += x[i].x + x[i].y + x[i].z + x[i].w;
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int v = (i + lane) & (V - 1);
      const uint4 x = *reinterpret_cast<const uint4*>(hist + lo + 4 * v);
      sum += x.x + x.y + x.z + x.w;
    }
  }
  const uint32_t incl = wave_incl_scan(sum);
  const uint64_t m = __ballot(incl - sum < kk && kk <= incl);
  const int L = m ? (int)__builtin_ctzll(m) : kWave - 1;
  const uint32_t base = __builtin_amdgcn_readlane(incl - sum, L);
  const uint32_t c = lane < PER ? hist[NB - 1 - (L * PER + lane)] : 0u;
  const uint32_t ci = wave_incl_scan(c) + base;
  const uint64_t m2 = __ballot(lane < PER && ci - c < kk && kk <= ci);
  const int j = m2 ? (int)__builtin_ctzll(m2) : 0;
  if (lane == j) {
    sel[0] = (uint32_t)(NB - 1 - (L * PER + j));
    sel[1] = ci - c;
  }
}

}  // namespace dsa
