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
//   B = k^T [D x 32 keys]    (32-key column blocks of an 8 KB key tile)
//   C       [32 heads x 32 keys] fp32
//
// Each wave streams 8 KB key tiles (64 fp8 or 32 bf16 rows of D = 128), the
// waves of a row interleaved tile by tile, with fully coalesced 16-byte
// loads, three tiles in flight, and regroups each tile through its own LDS
// region so that lane l holds D*e/2 contiguous bytes of key (l & 31).  (Loads
// straight into that layout touch 32 partial cache lines per instruction and
// run far slower.)  Keys, scales and scores go through buffer resources with
// a per-lane constant offset and a scalar per-tile offset, so the stream costs
// no vector address arithmetic, and the resource bounds replace clamping: a
// key past Lmax reads as zero and its score store is dropped.  The epilogue
// applies ReLU (a signed-integer max on the bit pattern: negative floats,
// -0 included, have negative patterns) and the per-head weight w' = w (bf16)
// or w * q_scale (fp8: the positive per-row scales commute with the ReLU) and
// sums the heads: 16 rows per lane in registers in four independent chains,
// the other 16 in lane l ^ 32.  Lanes 0..31 then store 32 consecutive fp32
// scores (times the key's scale for fp8) or -inf past pos.  A workgroup is
// eight waves, about one workgroup per CU (two waves per SIMD), and the launch
// bound of two waves per SIMD caps a wave at 256 registers, which keeps the
// MFMA accumulators in VGPRs where the epilogue reads them.
//
// Fused variant (FUSE): the same kernel feeding the top-k selection without
// writing scores to memory.  A workgroup's keys (at most kFuseKeys) keep
// their scores in LDS while the first radix histogram is built.  The
// workgroup then adds its counts to the row's histogram, meets the row's
// other workgroups at a per-row barrier, reads the finished histogram, finds
// the threshold bin b1, and compacts its own keys in bins >= b1 into the
// candidate slices of its chunks (a chunk is the kDecWaves consecutive tiles
// that one sweep of the workgroup's waves covers); a finishing kernel then
// concatenates the slices per row and completes the selection.
//
// The barrier needs no cache maintenance: every value that crosses
// workgroups goes through device-scope atomics.  A workgroup waits for the
// old values of its histogram adds (so each add has been performed) before
// it increments the row's arrival word, and a workgroup that has seen every
// arrival then reads the histogram with device-scope atomic loads.  The wait
// cannot deadlock: workgroups are dispatched in grid order, the rows are
// consecutive runs of the grid, and one row's workgroups (at most one per CU)
// fit on the GPU together, so the rows before a waiting row always finish
// and make room for the rest of it.  The wait is still bounded: on expiry
// the top bit of the arrival word is set and the finishing kernel gives the
// row an empty selection rather than a wrong one.
#include "device_common.hpp"
#include "launchers.hpp"

namespace dsa {
namespace {

constexpr int kDecWaves = 8;  // two per SIMD at one workgroup per CU

constexpr int kTileBytes = 8192;   // key bytes per wave step
constexpr int kHistBits = 12;      // first radix digit of the top-k selection
constexpr int kHistBins = 1 << kHistBits;
// Word 3 of a raw (untyped, unswizzled) buffer resource on gfx9; cache
// policy 2 marks a load nontemporal.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kNT = 2;
constexpr int kDeviceScope = 16;  // cache policy sc1: coherent at device scope
constexpr int kParts = 4;  // independent fma chains of the head sum
constexpr int kFuseKeys = 8192;        // keys whose scores a fused workgroup keeps in LDS
constexpr uint32_t kSpinLimit = 1u << 18;  // polls of the row barrier before giving up

// Outputs of the fused variant (chunk slices of the top-k workspace).
struct FuseArgs {
  int k;                // keys to select per row
  int n_chunks;         // chunks per row (kDecWaves tiles each)
  uint32_t* arrive;     // per-row arrival words (zero on entry)
  uint32_t* sel;        // per-row {b1, count above b1, listed}
  uint32_t* cnt;        // per-(row, chunk) candidate counts
  uint32_t* key;        // candidate keys, Lmax per row, chunk c at c * chunk keys
  int32_t* pos;         // candidate positions, same layout
};

template <int D, bool FP8, int HB, bool FUSE>
__global__ __launch_bounds__(kDecWaves * kWave, 2) void indexer_decode_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ k,
    const float* __restrict__ k_scale, const int32_t* __restrict__ ctx_len, int T, int H,
    int Lmax, float* __restrict__ scores, int64_t ld, int tiles_per_wave,
    uint32_t* __restrict__ row_hist, FuseArgs fa) {
  constexpr int EB = FP8 ? 1 : 2;
  constexpr int ROWB = D * EB;            // bytes per key row
  constexpr int HALF = ROWB / 2;          // bytes of a row held by one lane
  constexpr int NV = HALF / 16;           // 16-byte vectors per lane per key
  constexpr int TK = kTileBytes / ROWB;   // keys per tile (8 KB of keys)
  constexpr int CB = TK / 32;             // 32-key MFMA column blocks per tile
  constexpr int NL = kTileBytes / 1024;   // 16-byte loads per lane per tile (8)
  constexpr int PITCH = ROWB + 16;        // LDS row pitch (spreads banks)
  static_assert(NV >= 2 || !FP8, "fp8 needs 32 bytes per lane per MFMA step");
  __shared__ __align__(16) unsigned char stage[kDecWaves * TK * PITCH];
  __shared__ __align__(16) uint32_t lhist[kHistBins];  // used when row_hist is given
  __shared__ __align__(16) float sbuf[FUSE ? kFuseKeys : 1];  // fused: this workgroup's scores
  __shared__ uint32_t fscan[kDecWaves];
  __shared__ uint32_t fsel[4];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int g = lane >> 5;
  const int col = lane & 31;
  const int row = blockIdx.y;  // b * T + t
  const int b = row / T;
  const int t = row - b * T;
  const int tiles = (Lmax + TK - 1) / TK;
  // Wave w of the row's W waves takes tiles w, w + W, w + 2W, ...: all
  // waves sweep the row together, front to back (measurably closer to plain
  // streaming bandwidth than giving each wave its own contiguous run).  The
  // loop below runs over the wave's sequence numbers j = 0, 1, ...
  const int first = blockIdx.x * kDecWaves + wave;
  const int wstride = gridDim.x * kDecWaves;
  const int tile0 = 0;
  // (a wave past the row's last tile runs no iteration but stays for the
  // workgroup barriers of the histogram)
  const int tend = first < tiles ? min(tiles_per_wave, (tiles - first + wstride - 1) / wstride) : 0;
  if (row_hist) {
    for (int i = threadIdx.x; i < kHistBins; i += kDecWaves * kWave) lhist[i] = 0;
    __syncthreads();
  }
  auto tmap = [&](int j) { return __builtin_amdgcn_readfirstlane(first + j * wstride); };
  const int64_t pos = (int64_t)ctx_len[b] - T + t;
  unsigned char* my_stage = stage + wave * TK * PITCH;

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

  const uint8_t* kbase = k + (int64_t)b * Lmax * ROWB;
  const float* ksb = FP8 ? k_scale + (int64_t)b * Lmax : nullptr;
  float* srow = scores + (int64_t)row * ld;

  // A tile is 8 KB of consecutive key rows; lane l loads bytes 16 l + 1024 v
  // (fully coalesced) and the wave regroups them through its own LDS region
  // into the MFMA layout, where lane l needs D*e/2 bytes of key (l & 31).
  // Three register buffers keep tiles t+1 and t+2 in flight while tile t is
  // multiplied (the loop is unrolled by three so every buffer is static).
  i32x4 ba[NL], bb[NL], bc[NL];
  float sa[CB], sb[CB], sc_[CB];
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)kbase, 0, Lmax * ROWB, kBufferWord3);
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(FP8 ? ksb : k_scale), 0, FP8 ? Lmax * 4 : 0, kBufferWord3);
  const __amdgpu_buffer_rsrc_t outr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)srow, 0, FUSE ? 0 : Lmax * 4, kBufferWord3);
  auto load = [&](int seq, i32x4(&buf)[NL], float(&bs)[CB]) {
    const int tile = tmap(seq);
#pragma unroll
    for (int v = 0; v < NL; ++v)
      buf[v] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             kr, 16 * lane + 1024 * (v & 3),
                                             tile * kTileBytes + 4096 * (v >> 2), kNT));
    if (FP8) {
#pragma unroll
      for (int c = 0; c < CB; ++c)
        bs[c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                              sr, col * 4, (tile * TK + c * 32) * 4, kNT));
    }
  };
  auto compute = [&](int seq, const i32x4(&raw)[NL], const float(&cs)[CB]) {
    const int tile = tmap(seq);
#pragma unroll
    for (int v = 0; v < NL; ++v) {
      const int off = 16 * lane + 1024 * v;
      *reinterpret_cast<i32x4*>(my_stage + (off / ROWB) * PITCH + (off % ROWB)) = raw[v];
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      i32x4 cur[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v)
        cur[v] = *reinterpret_cast<const i32x4*>(my_stage + (c * 32 + col) * PITCH +
                                                 g * HALF + 16 * v);
      f32x16 acc[HB];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) acc[hb] = f32x16{};
      if constexpr (!FP8) {
#pragma unroll
        for (int st = 0; st < NV; ++st)
#pragma unroll
          for (int hb = 0; hb < HB; ++hb)
            acc[hb] = mfma32_bf16(as_bf16x8(qv[hb][st]), as_bf16x8(cur[st]), acc[hb]);
      } else {
#pragma unroll
        for (int st = 0; st < NV / 2; ++st) {
          const i32x8 bk = {cur[2 * st][0], cur[2 * st][1], cur[2 * st][2], cur[2 * st][3],
                            cur[2 * st + 1][0], cur[2 * st + 1][1], cur[2 * st + 1][2],
                            cur[2 * st + 1][3]};
#pragma unroll
          for (int hb = 0; hb < HB; ++hb) {
            const i32x8 aq = {qv[hb][2 * st][0], qv[hb][2 * st][1], qv[hb][2 * st][2],
                              qv[hb][2 * st][3], qv[hb][2 * st + 1][0], qv[hb][2 * st + 1][1],
                              qv[hb][2 * st + 1][2], qv[hb][2 * st + 1][3]};
            acc[hb] = mfma32_fp8(aq, bk, acc[hb]);
          }
        }
      }
      float part[kParts];
#pragma unroll
      for (int p = 0; p < kParts; ++p) part[p] = 0.f;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = __int_as_float(max(__float_as_int(acc[hb][r]), 0));
          part[(hb * 16 + r) % kParts] = fmaf(wv[hb][r], x, part[(hb * 16 + r) % kParts]);
        }
      float sc = part[0];
#pragma unroll
      for (int p = 1; p < kParts; ++p) sc += part[p];
      {
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(sc), __float_as_uint(sc),
                                                   false, false);
        sc = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
      const int key = tile * TK + c * 32 + col;
      const bool vis = key <= pos && key < Lmax;
      const float o = vis ? (FP8 ? sc * cs[c] : sc) : -INFINITY;
      if (g == 0) {
        if constexpr (FUSE)
          sbuf[(seq * kDecWaves + wave) * TK + c * 32 + col] = o;
        else
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o), outr, col * 4,
                                                (tile * TK + c * 32) * 4, 0);
        if (row_hist && vis) atomicAdd(&lhist[float_key(o) >> (32 - kHistBits)], 1u);
      }
    }
    __builtin_amdgcn_wave_barrier();
  };
  if (tile0 < tend) load(tile0, ba, sa);
  if (tile0 + 1 < tend) load(tile0 + 1, bb, sb);
  for (int tile = tile0; tile < tend; tile += 3) {
    if (tile + 2 < tend) load(tile + 2, bc, sc_);
    compute(tile, ba, sa);
    if (tile + 1 >= tend) break;
    if (tile + 3 < tend) load(tile + 3, ba, sa);
    compute(tile + 1, bb, sb);
    if (tile + 2 >= tend) break;
    if (tile + 4 < tend) load(tile + 4, bb, sb);
    compute(tile + 2, bc, sc_);
  }
  if constexpr (!FUSE) {
    if (row_hist) {  // add this workgroup's counts to the row's histogram
      __syncthreads();
      uint32_t* rh = row_hist + (int64_t)row * kHistBins;
      for (int i = threadIdx.x; i < kHistBins; i += kDecWaves * kWave) {
        const uint32_t c = lhist[i];
        if (c) atomicAdd(&rh[i], c);
      }
    }
  } else {
    constexpr int NT = kDecWaves * kWave;
    constexpr int HV = kHistBins / NT;  // bins per thread
    const int n = (int)max((int64_t)0, min(pos + 1, (int64_t)Lmax));  // visible keys
    if (n <= fa.k) return;  // the whole row is selected: nothing to meet for
    __syncthreads();
    uint32_t* rh = row_hist + (int64_t)row * kHistBins;
    // Add the counts, waiting for every add's old value: each add has then
    // been performed before the arrival below is.  All adds are issued
    // before the first old value is used (one round trip, not one each).
    {
      uint32_t cv[HV], old[HV];
#pragma unroll
      for (int u = 0; u < HV; ++u) cv[u] = lhist[threadIdx.x + NT * u];
#pragma unroll
      for (int u = 0; u < HV; ++u) {
        old[u] = 0;
        if (cv[u])
          old[u] = __hip_atomic_fetch_add(&rh[threadIdx.x + NT * u], cv[u], __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
      }
      uint32_t sink = 0;
#pragma unroll
      for (int u = 0; u < HV; ++u) sink |= old[u];
      asm volatile("" ::"v"(sink));
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t* a = fa.arrive + row;
      __hip_atomic_fetch_add(a, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (uint32_t it = 0;; ++it) {
        if (__hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= gridDim.x) break;
        if (it == kSpinLimit) {
          __hip_atomic_fetch_or(a, 0x80000000u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __syncthreads();
    // The row's finished histogram (16-byte loads at device scope: they
    // bypass this XCD's possibly stale L2 lines, as an atomic load does),
    // then its threshold bin.
    {
      constexpr int HV4 = HV / 4;
      const __amdgpu_buffer_rsrc_t hr =
          __builtin_amdgcn_make_buffer_rsrc((void*)rh, 0, kHistBins * 4, kBufferWord3);
      i32x4 hv[HV4];
#pragma unroll
      for (int u = 0; u < HV4; ++u)
        hv[u] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              hr, (threadIdx.x + NT * u) * 16, 0, kDeviceScope));
#pragma unroll
      for (int u = 0; u < HV4; ++u)
        *reinterpret_cast<i32x4*>(&lhist[4 * (threadIdx.x + NT * u)]) = hv[u];
    }
    __syncthreads();
    select_bin<kHistBins, NT>(lhist, (uint32_t)fa.k, fscan, fsel);
    const uint32_t b1 = fsel[0];
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      fa.sel[3 * row] = b1;
      fa.sel[3 * row + 1] = fsel[1];
      fa.sel[3 * row + 2] = fsel[1] + lhist[b1];
    }
    // Ordered compaction: wave w takes the workgroup's chunks w, w + W, ...;
    // lane l holds PL consecutive keys of the chunk.
    constexpr int G = kDecWaves * TK;  // keys per chunk
    constexpr int PL = G / kWave;
    static_assert(PL % 4 == 0, "whole 16-byte LDS reads per lane");
    uint32_t* ckr = fa.key + (int64_t)row * Lmax;
    int32_t* cpr = fa.pos + (int64_t)row * Lmax;
    for (int j = wave; j < tiles_per_wave; j += kDecWaves) {
      const int chunk = j * (int)gridDim.x + (int)blockIdx.x;
      if (chunk >= fa.n_chunks) break;
      const int p0 = chunk * G + lane * PL;
      uint32_t key[PL];
      bool ok[PL];
      uint32_t c = 0;
#pragma unroll
      for (int v = 0; v < PL / 4; ++v) {
        const float4 f = *reinterpret_cast<const float4*>(&sbuf[j * G + lane * PL + 4 * v]);
        key[4 * v] = float_key(f.x);
        key[4 * v + 1] = float_key(f.y);
        key[4 * v + 2] = float_key(f.z);
        key[4 * v + 3] = float_key(f.w);
      }
#pragma unroll
      for (int e = 0; e < PL; ++e) {
        ok[e] = (p0 + e) < n && (key[e] >> (32 - kHistBits)) >= b1;
        c += ok[e];
      }
      const uint32_t incl = wave_incl_scan(c);
      uint32_t at = chunk * G + incl - c;
#pragma unroll
      for (int e = 0; e < PL; ++e)
        if (ok[e]) {
          ckr[at] = key[e];
          cpr[at] = p0 + e;
          ++at;
        }
      if (lane == kWave - 1) fa.cnt[(int64_t)row * fa.n_chunks + chunk] = incl;
    }
  }
}

// Workgroups per launch the tile split aims for (one per CU measured best at
// the 128K decode shape: with four-wave workgroups 512 and 1024 were 2-25%
// slower; with eight-wave workgroups 128 was 12% slower).
constexpr int kDecWgTarget = 256;

// Tiles per wave and workgroups per row: enough waves to cover the GPU about
// once, each taking many key tiles so that its query fragments are loaded
// once; tpw_cap bounds the keys per workgroup.
struct DecPlan {
  int tk, tiles, tpw, gx;
};
DecPlan plan_dec(int rows, int D, bool fp8, int Lmax, int tpw_cap) {
  DecPlan p;
  p.tk = kTileBytes / (D * (fp8 ? 1 : 2));
  p.tiles = (Lmax + p.tk - 1) / p.tk;
  const int64_t want_waves = (int64_t)kDecWgTarget * kDecWaves;
  p.tpw = (int)(((int64_t)rows * p.tiles + want_waves - 1) / want_waves);
  p.tpw = max(1, min(p.tpw, tpw_cap));
  const int per_block = kDecWaves * p.tpw;
  p.gx = (p.tiles + per_block - 1) / per_block;
  return p;
}
DecPlan plan_fused(int rows, int D, bool fp8, int Lmax) {
  const int tk = kTileBytes / (D * (fp8 ? 1 : 2));
  return plan_dec(rows, D, fp8, Lmax, kFuseKeys / (kDecWaves * tk));
}
int fused_chunks(const DecPlan& p) { return (p.tiles + kDecWaves - 1) / kDecWaves; }

template <int D, bool FP8, int HB, bool FUSE>
hipError_t launch_dec(const DecPlan& p, const void* q, const float* q_scale, const float* w,
                      const void* k, const float* k_scale, const int32_t* ctx_len, int rows,
                      int T, int H, int Lmax, float* scores, int64_t ld, uint32_t* row_hist,
                      const FuseArgs& fa, hipStream_t stream) {
  dim3 grid(p.gx, rows);
  hipLaunchKernelGGL((indexer_decode_kernel<D, FP8, HB, FUSE>), grid, dim3(kDecWaves * kWave), 0,
                     stream, (const uint8_t*)q, q_scale, w, (const uint8_t*)k, k_scale, ctx_len,
                     T, H, Lmax, scores, ld, p.tpw, row_hist, fa);
  return hipGetLastError();
}

template <bool FUSE>
hipError_t dispatch_dec(const DecPlan& p, const void* q, bool fp8, const float* q_scale,
                        const float* w, const void* k, const float* k_scale,
                        const int32_t* ctx_len, int rows, int T, int H, int D, int Lmax,
                        float* scores, int64_t ld, uint32_t* row_hist, const FuseArgs& fa,
                        hipStream_t stream) {
#define DSA_DEC(DD, F8, HBB)                                                                 \
  return launch_dec<DD, F8, HBB, FUSE>(p, q, q_scale, w, k, k_scale, ctx_len, rows, T, H, Lmax, \
                                       scores, ld, row_hist, fa, stream)
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

}  // namespace

hipError_t launch_indexer_decode(const void* q, bool fp8, const float* q_scale, const float* w,
                                 const void* k, const float* k_scale, const int32_t* ctx_len,
                                 int B, int T, int H, int D, int Lmax, float* scores,
                                 int64_t ld, uint32_t* row_hist, hipStream_t stream) {
  const DecPlan p = plan_dec(B * T, D, fp8, Lmax, 64);
  return dispatch_dec<false>(p, q, fp8, q_scale, w, k, k_scale, ctx_len, B * T, T, H, D, Lmax,
                             scores, ld, row_hist, FuseArgs{}, stream);
}

bool indexer_topk_plan_ok(int B, int T, int D, bool fp8, int Lmax, int) {
  return fused_chunks(plan_fused(B * T, D, fp8, Lmax)) <= kTopkMaxChunks;
}

size_t indexer_topk_workspace_bytes(int B, int T, int D, bool fp8, int Lmax, int) {
  return topk_chunk_ws_bytes(B * T, Lmax, fused_chunks(plan_fused(B * T, D, fp8, Lmax)));
}

hipError_t launch_indexer_topk_decode(const void* q, bool fp8, const float* q_scale,
                                      const float* w, const void* k, const float* k_scale,
                                      const int32_t* ctx_len, int B, int T, int H, int D,
                                      int Lmax, int k_sel, int32_t* idx, void* workspace,
                                      hipStream_t stream) {
  const int rows = B * T;
  const DecPlan p = plan_fused(rows, D, fp8, Lmax);
  const int n_chunks = fused_chunks(p);
  if (n_chunks > kTopkMaxChunks) return hipErrorInvalidValue;
  // One row's workgroups must fit on the GPU together (one per CU).
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (p.gx > cus) return hipErrorInvalidConfiguration;
  const TopkWs ws = topk_chunk_ws(workspace, rows, Lmax, n_chunks);
  const FuseArgs fa{k_sel, n_chunks, ws.arrive, ws.sel, ws.cnt, ws.key, ws.pos};
  e = dispatch_dec<true>(p, q, fp8, q_scale, w, k, k_scale, ctx_len, rows, T, H, D, Lmax,
                         nullptr, 0, ws.hist, fa, stream);
  if (e != hipSuccess) return e;
  return launch_topk_finish(nullptr, 0, ctx_len, B, T, Lmax, k_sel, kDecWaves * p.tk, n_chunks,
                            ws, idx, stream);
}

}  // namespace dsa
