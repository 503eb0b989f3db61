// Lightning-indexer scores for one query row at a time (decode).
//
// Per (sequence b, query t) the work is a [H x D] . [D x L] product followed
// by ReLU, a head-weighted sum and the causal mask (IndexCache paper summary,
// technical §1: the indexer scores every previous token).  Per key the kernel
// reads D*e bytes (+4 for the fp8 scale) and writes one fp32 score, against
// 2*H*D flops: 63 flop/B in bf16, 120 in fp8 - far above what fp32 VALU can
// feed at HBM speed, far below the MFMA ridge.  So the product runs on MFMA
// with the query resident in registers while key rows stream from HBM:
//
//   A = q   [32 heads x D]   (per 32-head block, loaded once per wave)
//   B = k^T [D x 32 keys]    (one 32-key tile per step, two tiles in flight)
//   C       [32 heads x 32 keys] fp32
//
// Lane l supplies key (l & 31) and half (l >> 5) of its D dims, so each lane
// reads D*e/2 contiguous bytes of one key row.  The epilogue applies ReLU and
// the per-head weight w' = w (bf16) or w * q_scale (fp8: the positive
// per-row scales commute with the ReLU) and sums the heads: 16 rows per lane
// in registers, the other 16 in lane l ^ 32.  Lanes 0..31 then store 32
// consecutive fp32 scores (times the key's scale for fp8) or -inf past pos.
#include "device_common.hpp"
#include "launchers.hpp"

namespace dsa {
namespace {

constexpr int kDecWaves = 4;

template <int D, bool FP8, int HB>
__global__ __launch_bounds__(kDecWaves * kWave) void indexer_decode_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ k,
    const float* __restrict__ k_scale, const int32_t* __restrict__ ctx_len, int T, int H,
    int Lmax, float* __restrict__ scores, int64_t ld, int tiles_per_wave) {
  constexpr int EB = FP8 ? 1 : 2;
  constexpr int ROWB = D * EB;   // bytes per key row
  constexpr int HALF = ROWB / 2; // bytes of a row held by one lane
  constexpr int NV = HALF / 16;  // 16-byte vectors per lane per key
  static_assert(NV >= 2 || !FP8, "fp8 needs 32 bytes per lane per MFMA step");

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int g = lane >> 5;
  const int col = lane & 31;
  const int row = blockIdx.y;  // b * T + t
  const int b = row / T;
  const int t = row - b * T;
  const int tiles = (Lmax + 31) >> 5;
  const int tile0 = (blockIdx.x * kDecWaves + wave) * tiles_per_wave;
  if (tile0 >= tiles) return;
  const int tend = min(tile0 + tiles_per_wave, tiles);
  const int64_t pos = (int64_t)ctx_len[b] - T + t;

  // Query fragments (operand A) and per-row head weights.
  i32x4 qv[HB][NV];
  float wv[HB][16];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int head = hb * 32 + col;
    const uint8_t* qp = q + ((int64_t)row * H + head) * ROWB + g * HALF;
#pragma unroll
    for (int v = 0; v < NV; ++v) qv[hb][v] = (head < H) ? ld16(qp + 16 * v) : i32x4{0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int h = hb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
      float wt = 0.f;
      if (h < H) {
        wt = w[(int64_t)row * H + h];
        if (FP8) wt *= q_scale[(int64_t)row * H + h];
      }
      wv[hb][r] = wt;
    }
  }

  const uint8_t* kb = k + (int64_t)b * Lmax * ROWB + g * HALF;
  const float* ksb = FP8 ? k_scale + (int64_t)b * Lmax : nullptr;
  float* srow = scores + (int64_t)row * ld;

  i32x4 cur[NV], nxt[NV];
  float cur_s = 1.f, nxt_s = 1.f;
  {
    const int key = min(tile0 * 32 + col, Lmax - 1);
#pragma unroll
    for (int v = 0; v < NV; ++v) cur[v] = ld16_nt(kb + (int64_t)key * ROWB + 16 * v);
    if (FP8) cur_s = ksb[key];
  }
  for (int tile = tile0; tile < tend; ++tile) {
    if (tile + 1 < tend) {
      const int key = min((tile + 1) * 32 + col, Lmax - 1);
#pragma unroll
      for (int v = 0; v < NV; ++v) nxt[v] = ld16_nt(kb + (int64_t)key * ROWB + 16 * v);
      if (FP8) nxt_s = ksb[key];
    }
    f32x16 acc[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) acc[hb] = f32x16{};
    if constexpr (!FP8) {
#pragma unroll
      for (int s = 0; s < NV; ++s)
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
          acc[hb] = mfma32_bf16(as_bf16x8(qv[hb][s]), as_bf16x8(cur[s]), acc[hb]);
    } else {
#pragma unroll
      for (int s = 0; s < NV / 2; ++s) {
        const i32x8 bk = {cur[2 * s][0], cur[2 * s][1], cur[2 * s][2], cur[2 * s][3],
                          cur[2 * s + 1][0], cur[2 * s + 1][1], cur[2 * s + 1][2],
                          cur[2 * s + 1][3]};
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          const i32x8 aq = {qv[hb][2 * s][0], qv[hb][2 * s][1], qv[hb][2 * s][2],
                            qv[hb][2 * s][3], qv[hb][2 * s + 1][0], qv[hb][2 * s + 1][1],
                            qv[hb][2 * s + 1][2], qv[hb][2 * s + 1][3]};
          acc[hb] = mfma32_fp8(aq, bk, acc[hb]);
        }
      }
    }
    float sc = 0.f;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc = fmaf(wv[hb][r], fmaxf(acc[hb][r], 0.f), sc);
    sc += __shfl_xor(sc, 32, kWave);
    const int key = tile * 32 + col;
    if (g == 0 && key < Lmax) {
      float o = -INFINITY;
      if (key <= pos) o = FP8 ? sc * cur_s : sc;
      srow[key] = o;
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) cur[v] = nxt[v];
    cur_s = nxt_s;
  }
}

template <int D, bool FP8, int HB>
hipError_t launch_dec(const void* q, const float* q_scale, const float* w, const void* k,
                      const float* k_scale, const int32_t* ctx_len, int B, int T, int H,
                      int Lmax, float* scores, int64_t ld, hipStream_t stream) {
  const int rows = B * T;
  const int tiles = (Lmax + 31) / 32;
  // Aim for about 2048 workgroups (8 per CU) so every CU keeps several key
  // tiles in flight; each wave takes a contiguous run of tiles.
  int64_t want_waves = 2048LL * kDecWaves;
  int tpw = (int)(((int64_t)rows * tiles + want_waves - 1) / want_waves);
  tpw = max(1, min(tpw, 32));
  const int per_block = kDecWaves * tpw;
  dim3 grid((tiles + per_block - 1) / per_block, rows);
  hipLaunchKernelGGL((indexer_decode_kernel<D, FP8, HB>), grid, dim3(kDecWaves * kWave), 0,
                     stream, (const uint8_t*)q, q_scale, w, (const uint8_t*)k, k_scale, ctx_len,
                     T, H, Lmax, scores, ld, tpw);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer_decode(const void* q, bool fp8, const float* q_scale, const float* w,
                                 const void* k, const float* k_scale, const int32_t* ctx_len,
                                 int B, int T, int H, int D, int Lmax, float* scores,
                                 int64_t ld, hipStream_t stream) {
#define DSA_DEC(DD, F8, HBB) \
  return launch_dec<DD, F8, HBB>(q, q_scale, w, k, k_scale, ctx_len, B, T, H, Lmax, scores, ld, stream)
  const bool two = H > 32;
  if (D == 128) {
    if (fp8) { if (two) DSA_DEC(128, true, 2); DSA_DEC(128, true, 1); }
    if (two) DSA_DEC(128, false, 2);
    DSA_DEC(128, false, 1);
  }
  if (fp8) { if (two) DSA_DEC(64, true, 2); DSA_DEC(64, true, 1); }
  if (two) DSA_DEC(64, false, 2);
  DSA_DEC(64, false, 1);
#undef DSA_DEC
}

}  // namespace dsa
