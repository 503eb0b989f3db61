// Streaming-read probe: reads a device buffer once and keeps nothing, the
// practical HBM ceiling that the decode indexer's stream is compared with.
// It is a measurement aid outside the attention path (no arithmetic of the
// method): the indexer's key sweep without its scoring.
//
// Two load patterns over 8 KB tiles, 16-byte non-temporal buffer loads:
//   tiles  - the decode indexer's own sweep: workgroup w owns a contiguous
//            run of tiles, its eight waves take them interleaved (wave j:
//            tiles j, j + 8, ...), two tiles (16 loads per lane) in flight;
//   stride - a grid-stride sweep of the whole buffer, eight 16-byte loads
//            per lane in flight.
// Loaded words are XOR-folded; a lane stores the fold only when it equals a
// fixed 32-bit pattern, so the loads cannot be dropped and the sink is
// (almost) never written.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include "launchers.hpp"

namespace dsa {
namespace {

constexpr int kProbeWaves = 8;
constexpr int kTile = 8192;
constexpr int kInFlight = 2;  // tiles per wave (tiles form)
constexpr int kStrideU = 8;   // 16-byte loads per lane (stride form)
constexpr int kWord3 = 0x00020000;
constexpr int kNonTemporal = 2;  // buffer-load cache policy bit: streaming
constexpr uint32_t kSinkPattern = 0x9E3779B9u;

typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void fold_out(i32x4 acc, int32_t* sink) {
  const uint32_t f = (uint32_t)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
  if (f == kSinkPattern) sink[0] = (int32_t)f;
}

__global__ __launch_bounds__(kProbeWaves * kWave) void stream_tiles_kernel(
    const uint8_t* __restrict__ src, int64_t tiles, int32_t* __restrict__ sink) {
  const int64_t t0 = tiles * blockIdx.x / gridDim.x;
  const int64_t t1 = tiles * (blockIdx.x + 1) / gridDim.x;
  const uint8_t* base = src + t0 * kTile;
  // The run is at most 2^31 bytes (checked on the host), so one resource
  // with 32-bit offsets covers it.
  __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)((t1 - t0) * kTile), kWord3);
  // Wave-uniform, so the tile offset goes in the scalar offset field.
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & (kWave - 1);
  const int n = (int)(t1 - t0);
  i32x4 acc = {0, 0, 0, 0};
  for (int t = wave; t < n; t += kProbeWaves * kInFlight) {
    i32x4 v[kInFlight][8];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const bool in_run = t + u * kProbeWaves < n;  // wave-uniform: no load past the run
#pragma unroll
      for (int j = 0; j < 8; ++j)
        v[u][j] = in_run ? __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                         r, 16 * lane + 1024 * j,
                                                         (t + u * kProbeWaves) * kTile,
                                                         kNonTemporal))
                         : i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc ^= v[u][j];
  }
  fold_out(acc, sink);
}

__global__ __launch_bounds__(kProbeWaves * kWave) void stream_stride_kernel(
    const uint8_t* __restrict__ src, int64_t tiles, int32_t* __restrict__ sink) {
  const int64_t nvec = tiles * (kTile / 16);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  i32x4 acc = {0, 0, 0, 0};
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i < nvec; i += kStrideU * stride) {
    i32x4 v[kStrideU];
#pragma unroll
    for (int u = 0; u < kStrideU; ++u) {
      const int64_t e = i + u * stride;
      v[u] = e < nvec ? __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(src) + e)
                      : i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kStrideU; ++u) acc ^= v[u];
  }
  fold_out(acc, sink);
}

}  // namespace

hipError_t launch_stream_probe(const void* src, int64_t tiles, int workgroups, bool stride_form,
                               int32_t* sink, hipStream_t stream) {
  const dim3 grid((unsigned)workgroups), block(kProbeWaves * kWave);
  const uint8_t* p = static_cast<const uint8_t*>(src);
  if (stride_form)
    hipLaunchKernelGGL(stream_stride_kernel, grid, block, 0, stream, p, tiles, sink);
  else
    hipLaunchKernelGGL(stream_tiles_kernel, grid, block, 0, stream, p, tiles, sink);
  return hipGetLastError();
}

}  // namespace dsa
