// KV-cache append: the write that precedes every decode step and every
// prefill chunk.  Each new token brings one latent row (the MLA key/value
// row shared by all heads) and one lightning-indexer key row; both go into
// the caches at the token's absolute position ctx_len[b] - T + t.
//
// The latent cache is bf16; the indexer key cache is bf16 or fp8 e4m3 with one
// fp32 scale per row (the DSA indexer keeps its keys in fp8 with fine-grained
// block scales; with D = 128 a row is one 128-element block).
//
// One wave per token row; the work is a pure stream (fp32 in, narrow out), so
// the kernel is HBM-bound: 16-byte loads, every lane busy on the latent row,
// a wave-wide max for the fp8 row scale, plain vector stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include "launchers.hpp"

namespace dsa {
namespace {

constexpr int kAppendWaves = 4;  // token rows per workgroup
constexpr float kFp8Max = 448.f;

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Two floats -> two bf16 in one word (v_cvt_pk_bf16_f32: round to nearest
// even), the first in the low half.
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// One float -> OCP fp8 E4M3FN code, round to nearest, ties to even.
// |x| >= 464 would round past the largest finite code; such magnitudes are
// saturated to 448 (code 0x7E) instead (the row scaling below keeps every
// magnitude at most 448 up to one rounding of the division).
//   normal (|x| >= 2^-6): drop 20 of the 23 fp32 mantissa bits with
//     round-half-even on the raw bit pattern (a carry moves into the exponent
//     field, which is what rounding up to the next binade means), then move
//     the exponent bias from 127 to 7;
//   subnormal (|x| < 2^-6): the codes are m * 2^-9 with m in 0..8, so
//     m = rne(|x| * 2^9) (the product is exact; m = 8 is the smallest normal).
__device__ __forceinline__ uint32_t e4m3_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  a = a < 0x43E00000u ? a : 0x43E00000u;  // 448.0f
  uint32_t code;
  if (a >= 0x3C800000u) {  // 2^-6
    const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
    code = r - ((127u - 7u) << 3);
  } else {
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.f);
  }
  return sign | code;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// kv_new [rows, d_qk] fp32 -> kv_cache [B, Lmax, d_qk] bf16 and
// k_new [rows, D] fp32 -> k_cache [B, Lmax, D] (bf16, or fp8 + k_scale).
// Either pair may be absent (null new-row pointer).
template <bool kFp8>
__global__ __launch_bounds__(kAppendWaves * kWave) void kv_append_kernel(
    const float* __restrict__ kv_new, const float* __restrict__ k_new,
    const int32_t* __restrict__ ctx_len, int B, int T, int Lmax, int d_qk, int D,
    uint16_t* __restrict__ kv_cache, void* __restrict__ k_cache, float* __restrict__ k_scale) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * kAppendWaves + (threadIdx.x >> 6);
  if (row >= (int64_t)B * T) return;
  const int b = (int)(row / T), t = (int)(row % T);
  const int64_t pos = (int64_t)ctx_len[b] - T + t;
  if (pos < 0 || pos >= Lmax) return;  // outside the cache: nothing is written
  const int64_t dst = (int64_t)b * Lmax + pos;

  if (kv_new != nullptr) {
    const int chunks = d_qk >> 2;
    const float* src = kv_new + row * d_qk;
    uint16_t* out = kv_cache + dst * d_qk;
    for (int c = lane; c < chunks; c += kWave) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(src + 4 * c);
      uint2 w;
      w.x = cvt_bf16x2(v.x, v.y);
      w.y = cvt_bf16x2(v.z, v.w);
      *reinterpret_cast<uint2*>(out + 4 * c) = w;
    }
  }

  if (k_new != nullptr) {
    // D <= 256: one 16-byte chunk per lane at most.
    const bool live = lane < (D >> 2);
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (live) v = *reinterpret_cast<const f32x4*>(k_new + row * D + 4 * lane);
    if (kFp8) {
      const float amax =
          wave_max(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
      const float scale = amax > 0.f ? amax / kFp8Max : 1.f;  // IEEE division
      if (live) {
        const uint32_t w = e4m3_rne(v.x / scale) | (e4m3_rne(v.y / scale) << 8) |
                           (e4m3_rne(v.z / scale) << 16) | (e4m3_rne(v.w / scale) << 24);
        *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(k_cache) + dst * D + 4 * lane) = w;
      }
      if (lane == 0) k_scale[dst] = scale;
    } else if (live) {
      uint2 w;
      w.x = cvt_bf16x2(v.x, v.y);
      w.y = cvt_bf16x2(v.z, v.w);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(k_cache) + dst * D + 4 * lane) = w;
    }
  }
}

}  // namespace

hipError_t launch_kv_append(const float* kv_new, const float* k_new, const int32_t* ctx_len,
                            int B, int T, int Lmax, int d_qk, int D, bool k_fp8, void* kv_cache,
                            void* k_cache, float* k_scale, hipStream_t stream) {
  const int64_t rows = (int64_t)B * T;
  const dim3 grid((unsigned)((rows + kAppendWaves - 1) / kAppendWaves));
  const dim3 block(kAppendWaves * kWave);
  uint16_t* kvc = static_cast<uint16_t*>(kv_cache);
  if (k_fp8)
    hipLaunchKernelGGL(kv_append_kernel<true>, grid, block, 0, stream, kv_new, k_new, ctx_len, B,
                       T, Lmax, d_qk, D, kvc, k_cache, k_scale);
  else
    hipLaunchKernelGGL(kv_append_kernel<false>, grid, block, 0, stream, kv_new, k_new, ctx_len,
                       B, T, Lmax, d_qk, D, kvc, k_cache, k_scale);
  return hipGetLastError();
}

}  // namespace dsa
