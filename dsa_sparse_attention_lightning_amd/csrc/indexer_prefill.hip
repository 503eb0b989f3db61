// Lightning-indexer scores for a prefill chunk (T > 1 query rows).
//
// Same score as the decode kernel (IndexCache paper summary, technical §1:
// the indexer scores every previous token; DSA form
// sum_h w * ReLU(q_h . k)), but here many queries share each key, so the
// problem is a dense [T*H x D] . [D x L] contraction - 2*H*D flops per
// (query, key) pair against a few bytes - and runs at MFMA speed:
//
//   * a workgroup holds 8 queries, one per wave; a wave keeps its query's
//     [64 heads x D] block in registers (operand A of 32x32 MFMAs);
//   * key tiles of 128 or 256 rows are staged through LDS (double-buffered, rows
//     padded by 16 bytes so the 32 lanes of a fragment read hit distinct
//     banks) and shared by the 8 waves: operand B, 32 keys per MFMA column
//     block;
//   * the fused epilogue (ReLU, head weight w' = w (bf16) or w * q_scale
//     (fp8), sum over heads, key scale, causal mask) runs on the fp32
//     accumulators, so only the final fp32 score reaches HBM;
//   * causality: a workgroup never computes keys beyond its last query's
//     position; those columns, and columns past each query's own position,
//     are written as -inf.
//
// Fused variant (FUSE, feeding the top-k without writing scores): a
// workgroup takes its 8 query rows over all their keys, so each wave owns
// one row.  The wave counts its visible scores' top 10 key bits in its own
// LDS histogram and, every 4 tiles, takes the bin holding the k-th largest
// count so far as its row's bound: the k-th largest of the keys seen so far
// is at most the row's, so every key of the row's top k lies in a bin at or
// above any bound taken on the way.  Inside the bound's bin the wave also
// counts the next 6 key bits (restarted whenever the bound moves to a higher
// bin, so it can only undercount) and takes a sub-bin bound the same way.
// Scores at or above the current bound are appended, in position order, to
// the row's candidate list (a wave-wide ballot gives each its slot); a
// per-row kernel then selects the top k among the candidates.  The eight
// histograms and the key tiles take 75 KB, so two workgroups share a CU.
#include "device_common.hpp"
#include "launchers.hpp"

namespace dsa {
namespace {

constexpr int kPfWaves = 8;    // queries per workgroup
constexpr int kPfThreads = kPfWaves * kWave;
// Keys per LDS tile: 256 for the bf16 score kernel (one workgroup per CU
// either way; half the tile barriers, measured 1% faster), 128 where two
// workgroups share a CU (fp8) or the histograms need the room (fused).
__host__ __device__ constexpr int pf_tile(bool fp8, bool fuse) { return (!fp8 && !fuse) ? 256 : 128; }
constexpr int kParts = 4;      // independent fma chains of the head sum
// Word 3 of a raw (untyped, unswizzled) buffer resource on gfx9.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kPfBinBits = 10;   // fused: top key bits of the running bound
constexpr int kPfBins = 1 << kPfBinBits;
constexpr int kPfSubBits = 6;    // fused: next key bits, counted inside the bound's bin
constexpr int kPfSubs = 1 << kPfSubBits;
// One pad word per 16 bins: a lane's 16 consecutive bins then sit in 16
// different banks from every other lane's.
constexpr int kPfHistWords = kPfBins + kPfBins / 16 + kPfSubs;  // + the sub-histogram
__device__ __forceinline__ int pf_bin_at(uint32_t b) { return (int)(b + (b >> 4)); }

// Outputs of the fused variant.
struct PfFuseArgs {
  int k;               // keys to select per row
  uint32_t* key;       // candidate keys, Lmax per row, in position order
  int32_t* pos;        // candidate positions, same layout
  uint32_t* cnt;       // candidates per row
};

// Bin of the kk-th largest count of a wave's histogram (bins from the top),
// or cur when it counts fewer than kk.  Lane l sums bins 16 (63 - l) ..
// 16 (63 - l) + 15, so the lane prefix runs from the top bin down.
__device__ uint32_t pf_wave_bound(const uint32_t* h, uint32_t kk, int lane, uint32_t cur,
                                  uint32_t& above) {
  constexpr int PER = kPfBins / kWave;
  const uint32_t lo = (uint32_t)(kWave - 1 - lane) * PER;  // lane 0: the top PER bins
  uint32_t c[PER];
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    c[i] = h[pf_bin_at(lo + i)];
    sum += c[i];
  }
  const uint32_t incl = wave_incl_scan(sum);
  const uint64_t m = __ballot(incl >= kk);
  if (m == 0) return cur;
  const int first = __builtin_ctzll(m);
  uint32_t acc = incl - sum, bin = lo, abv = 0;
  bool found = false;
#pragma unroll
  for (int i = PER - 1; i >= 0; --i) {
    if (!found && acc + c[i] >= kk) {
      bin = lo + i;
      abv = acc;
      found = true;
    }
    acc += c[i];
  }
  above = (uint32_t)__builtin_amdgcn_readlane((int)abv, first);
  return (uint32_t)__builtin_amdgcn_readlane((int)bin, first);
}

// Sub-bin bound inside the bound's bin: the highest sub-bin s with at least
// need counts in sub-bins >= s (lane l holds sub-bin 63 - l), or 0.
__device__ uint32_t pf_sub_bound(const uint32_t* sh, uint32_t need, int lane) {
  const uint32_t incl = wave_incl_scan(sh[kPfSubs - 1 - lane]);
  const uint64_t m = __ballot(incl >= need);
  return m == 0 ? 0u : (uint32_t)(kPfSubs - 1 - __builtin_ctzll(m));
}

// fp8: at most 128 registers per lane so that two workgroups share a CU (four
// waves per SIMD hide each other's MFMA and epilogue; measured 3% faster than
// two waves even with a few spilled registers).  bf16 needs more registers
// (its query block is twice the size) and keeps two waves per SIMD.
template <bool FP8, int D, int HB, bool FUSE>
__global__ __launch_bounds__(kPfThreads, FP8 ? 4 : 2) void indexer_prefill_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ k,
    const float* __restrict__ k_scale, const int32_t* __restrict__ ctx_len, int T, int H,
    int Lmax, float* __restrict__ scores, int64_t ld, int keys_per_wg, PfFuseArgs fa) {
  constexpr int TILE = pf_tile(FP8, FUSE);
  constexpr int EB = FP8 ? 1 : 2;
  constexpr int ROWB = D * EB;          // bytes per key row
  constexpr bool kPipe = !FUSE && !FP8;  // software-pipelined sub-blocks (bf16)
  // LDS row pitch: padded rows for the register-staged tiles; the pipelined
  // kernel's tiles arrive by LDS-DMA, unpadded, with each row's 16-byte
  // chunks permuted instead (chunk c of row r at position c ^ (r % CPR)).
  constexpr int PITCH = kPipe ? ROWB : ROWB + 16;
  constexpr int HALF = ROWB / 2;        // bytes of a row per lane
  constexpr int NV = HALF / 16;         // 16-byte vectors per lane per key
  constexpr int CPR = ROWB / 16;        // 16-byte chunks per row
  constexpr int CH = TILE * CPR / kPfThreads;  // staged chunks per thread
  static_assert(CH >= 1 && TILE * CPR % kPfThreads == 0, "tile staging");
  __shared__ __align__(16) uint8_t ks[2][TILE * PITCH];
  __shared__ float kss[2][TILE];
  __shared__ uint32_t whist[FUSE ? kPfWaves * kPfHistWords : 1];  // fused: per-wave histograms

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // wave-uniform (readfirstlane): the query row and every buffer resource
  // built from it are then scalar, so the compiler emits plain buffer
  // instructions instead of a per-instruction loop over lanes' resources
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int g = lane >> 5;
  const int col = lane & 31;
  const int b = blockIdx.z;
  const int t0 = blockIdx.x * kPfWaves;
  const int t = t0 + wave;
  const bool live = t < T;
  const int tq = min(t, T - 1);
  const int64_t row = (int64_t)b * T + tq;
  const int ctx = ctx_len[b];
  const int64_t pos = (int64_t)ctx - T + t;
  const int64_t pos_max = (int64_t)ctx - T + min(T - 1, t0 + kPfWaves - 1);
  const int k0 = blockIdx.y * keys_per_wg;
  const int k1 = min(Lmax, k0 + keys_per_wg);
  const int kc = (int)max((int64_t)k0, min((int64_t)k1, pos_max + 1));  // computed: [k0, kc)
  float* srow = FUSE ? nullptr : scores + row * ld;

  if (!FUSE && live)
    for (int s = kc + lane; s < k1; s += kWave) srow[s] = -INFINITY;
  if (kc <= k0) {  // uniform over the workgroup
    if (FUSE && live && lane == 0) fa.cnt[row] = 0;
    return;
  }
  if constexpr (FUSE)
    for (int i = tid; i < kPfWaves * kPfHistWords; i += kPfThreads) whist[i] = 0;
  uint32_t* wh = whist + (FUSE ? wave * kPfHistWords : 0);
  uint32_t* ckr = FUSE ? fa.key + row * Lmax : nullptr;
  int32_t* cpr = FUSE ? fa.pos + row * Lmax : nullptr;
  uint32_t* wsh = wh + kPfBins + kPfBins / 16;  // fused: sub-histogram of the bound's bin
  uint32_t wcount = 0, wbound = 0, wsub = 0;  // fused: candidates, bound bin and sub-bin

  // Query fragments and head weights (zero for padded heads; an idle wave
  // reads the last query row and stores nothing).
  i32x4 qv[HB][NV];
  float wv[HB][16];
  {
    // Buffer resources over this row's query block, weights and scales:
    // the loads are unconditional (all in flight together) and a padded
    // head (h >= H) reads zeros, so it adds nothing to any score.
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(q + row * H * ROWB), 0, H * ROWB, kBufferWord3);
    const __amdgpu_buffer_rsrc_t wr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(w + row * H), 0, H * 4, kBufferWord3);
    const __amdgpu_buffer_rsrc_t qsr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(FP8 ? q_scale + row * H : w), 0, FP8 ? H * 4 : 0, kBufferWord3);
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int head = hb * 32 + col;
#pragma unroll
      for (int v = 0; v < NV; ++v)
        qv[hb][v] = __builtin_bit_cast(
            i32x4, __builtin_amdgcn_raw_buffer_load_b128(qr, head * ROWB + g * HALF + 16 * v, 0, 0));
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int h = hb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        float wt = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(wr, h * 4, 0, 0));
        if (FP8)
          wt *= __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(qsr, h * 4, 0, 0));
        wv[hb][r] = wt;
      }
    }
  }

  // Keys, scales and scores through buffer resources over this sequence, the
  // whole offset in the vector offset (the part the compiler documents as
  // range-checked): reads past Lmax return zero without touching memory.
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(k + (int64_t)b * Lmax * ROWB), 0, Lmax * ROWB, kBufferWord3);
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(FP8 ? k_scale + (int64_t)b * Lmax : k_scale), 0, FP8 ? Lmax * 4 : 0, kBufferWord3);
  const __amdgpu_buffer_rsrc_t outr =
      __builtin_amdgcn_make_buffer_rsrc((void*)srow, 0, FUSE ? 0 : Lmax * 4, kBufferWord3);
  const int ntiles = (kc - k0 + TILE - 1) / TILE;

  i32x4 stage[CH];
  float stage_s = 1.f;
  auto gload = [&](int tile) {
    const int base = __builtin_amdgcn_readfirstlane(k0 + tile * TILE);
#pragma unroll
    for (int c = 0; c < CH; ++c)
      stage[c] = __builtin_bit_cast(
          i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     kr, base * ROWB + (tid + c * kPfThreads) * 16, 0, 0));
    if (FP8 && tid < TILE)
      stage_s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                              sr, (base + tid) * 4, 0, 0));
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int chunk = tid + c * kPfThreads;
      *reinterpret_cast<i32x4*>(&ks[buf][(chunk / CPR) * PITCH + (chunk % CPR) * 16]) = stage[c];
    }
    if (FP8 && tid < TILE) kss[buf][tid] = stage_s;
  };

  // The next tile by LDS-DMA: wave w's instruction j fills LDS slots
  // 64 (w + 8 j) .. + 63 of the tile; slot p is position p % CPR of row
  // p / CPR and takes chunk position ^ (row % CPR) of that key row.
  constexpr int DJ = TILE * CPR / (kPfWaves * kWave);
  static_assert(DJ * kPfWaves * kWave == TILE * CPR, "whole wave-loads per tile");
  auto dma = [&](int tile, int buf) {
    const int base = __builtin_amdgcn_readfirstlane(k0 + tile * TILE);
#pragma unroll
    for (int j = 0; j < DJ; ++j) {
      const int slot = kWave * (wave + kPfWaves * j) + lane;
      const int r = slot / CPR;
      const int c = (slot % CPR) ^ (r & (CPR - 1));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          kr, (__attribute__((address_space(3))) void*)(&ks[buf][kWave * 16 * (wave + kPfWaves * j)]),
          16, (unsigned)((base + r) * ROWB + c * 16), 0, 0, 0);
    }
  };
  if constexpr (kPipe) {
    dma(0, 0);
  } else {
    gload(0);
    lstore(0);
  }
  // Every prologue load (query block, head weights) lands before the tile
  // loop.  Left in flight, the compiler's wait counts carry them into the
  // loop, where the first epilogue then waits vmcnt(3..0) on each pass: that
  // wait also covers the next tile's key loads issued just before it, so
  // their whole latency would show once per tile.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt, lgkmcnt untouched
  __syncthreads();
  if constexpr (kPipe) {
    // bf16, two waves per SIMD: software-pipelined sub-blocks.  The products
    // of the next sub-block are issued one at a time between the epilogue
    // steps of the current one (two accumulator values per product), so a
    // wave keeps the matrix core busy through its own epilogue instead of
    // leaving it to the SIMD's other wave; a tile's last epilogue runs under
    // the first products of the next tile, after the tile barrier.  Every
    // sub-block of a tile is computed; keys past kc store nothing.
    constexpr int NP = NV * HB;      // products per sub-block
    constexpr int NE = HB * 16 / 2;  // epilogue steps, two values each
    constexpr int NS = TILE / 32;    // sub-blocks per tile
    static_assert(NS % 2 == 0, "a tile's last products land in the second accumulator");
    auto read_b = [&](int buf, int sb, i32x4(&bv)[NV]) {
      const int r = sb * 32 + col;
      const uint8_t* bp = &ks[buf][r * PITCH];
#pragma unroll
      for (int v = 0; v < NV; ++v)
        bv[v] = *reinterpret_cast<const i32x4*>(bp + 16 * ((g * NV + v) ^ (r & (CPR - 1))));
    };

    auto prod = [&](int i, const i32x4(&bv)[NV], f32x16(&acc)[HB]) {
      const int s = i / HB, hb = i % HB;
      acc[hb] = mfma32_bf16(as_bf16x8(qv[hb][s]), as_bf16x8(bv[s]), s == 0 ? f32x16{} : acc[hb]);
    };
    auto step = [&](int e, const f32x16(&acc)[HB], float(&part)[kParts]) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int v = 2 * e + j, hb = v / 16, r = v % 16;
        const float x = __int_as_float(max(__float_as_int(acc[hb][r]), 0));
        part[v % kParts] = fmaf(wv[hb][r], x, part[v % kParts]);
      }
    };
    // (pairing sub-blocks into one lane swap and one 64-lane store, as the
    // fp8 path below does, measured 0.7% slower here)
    auto finish = [&](int kbase, const float(&part)[kParts]) {
      float sc = part[0];
#pragma unroll
      for (int p = 1; p < kParts; ++p) sc += part[p];
      auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(sc), __float_as_uint(sc), false,
                                                 false);
      sc = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      const int key = kbase + col;
      const bool st = g == 0 && live && key < kc;
      const float o = key <= pos ? sc : -INFINITY;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o), outr,
                                            (uint32_t)(st ? key : Lmax) * 4u, 0, 0);
    };
    // Epilogue of cur (keys kbase ..) with the products of bv into nxt.
    auto overlap = [&](int kbase, const f32x16(&cur)[HB], const i32x4(&bv)[NV],
                       f32x16(&nxt)[HB]) {
      float part[kParts] = {};
      // One epilogue step ahead of the first product (measured: none, two,
      // three and six ahead are 1-2% slower)
      constexpr int PRE = 1;
#pragma unroll
      for (int e = 0; e < PRE; ++e) step(e, cur, part);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        prod(i, bv, nxt);
        if (i + PRE < NE) step(i + PRE, cur, part);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int e = NP + PRE; e < NE; ++e) step(e, cur, part);
      finish(kbase, part);
    };
    f32x16 acc0[HB], acc1[HB];
    i32x4 bv[NV];
    read_b(0, 0, bv);
#pragma unroll
    for (int i = 0; i < NP; ++i) prod(i, bv, acc0);
    for (int tile = 0; tile < ntiles; ++tile) {
      const int buf = tile & 1;
      const bool more = tile + 1 < ntiles;
      if (more) dma(tile + 1, buf ^ 1);  // (every wave finished that buffer before the barrier)
      const int tbase = k0 + tile * TILE;
#pragma unroll
      for (int sb = 0; sb + 1 < NS; ++sb) {
        read_b(buf, sb + 1, bv);
        overlap(tbase + 32 * sb, (sb & 1) ? acc1 : acc0, bv, (sb & 1) ? acc0 : acc1);
      }
      if (more) {
        // this wave's DMA of the next tile has landed (the memory counter
        // completes in order: only the NS - 1 score stores since are left),
        // then every wave's has
        __builtin_amdgcn_s_waitcnt(0x0F70 | (NS - 1));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        read_b(buf ^ 1, 0, bv);
        overlap(tbase + 32 * (NS - 1), acc1, bv, acc0);
      } else {
        float part[kParts] = {};
#pragma unroll
        for (int e = 0; e < NE; ++e) step(e, acc1, part);
        finish(tbase + 32 * (NS - 1), part);
      }
    }
  } else {
  float stash = 0.f;  // (the per-lane sums of an even sub-block, until its pair is stored)
  for (int tile = 0; tile < ntiles; ++tile) {
    const int buf = tile & 1;
    if (tile + 1 < ntiles) gload(tile + 1);
    const int tbase = k0 + tile * TILE;
    // Products of sub-block sb (32 keys x the wave's heads) into acc.
    auto mma = [&](int sb, f32x16(&acc)[HB]) {
      const uint8_t* bp = &ks[buf][(sb * 32 + col) * PITCH + g * HALF];
      i32x4 bv[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) bv[v] = *reinterpret_cast<const i32x4*>(bp + 16 * v);
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) acc[hb] = f32x16{};
      if constexpr (!FP8) {
#pragma unroll
        for (int s = 0; s < NV; ++s)
#pragma unroll
          for (int hb = 0; hb < HB; ++hb)
            acc[hb] = mfma32_bf16(as_bf16x8(qv[hb][s]), as_bf16x8(bv[s]), acc[hb]);
      } else {
#pragma unroll
        for (int s = 0; s < NV / 2; ++s) {
          const i32x8 bk = {bv[2 * s][0], bv[2 * s][1], bv[2 * s][2], bv[2 * s][3],
                            bv[2 * s + 1][0], bv[2 * s + 1][1], bv[2 * s + 1][2],
                            bv[2 * s + 1][3]};
#pragma unroll
          for (int hb = 0; hb < HB; ++hb) {
            const i32x8 aq = {qv[hb][2 * s][0], qv[hb][2 * s][1], qv[hb][2 * s][2],
                              qv[hb][2 * s][3], qv[hb][2 * s + 1][0], qv[hb][2 * s + 1][1],
                              qv[hb][2 * s + 1][2], qv[hb][2 * s + 1][3]};
            acc[hb] = mfma32_fp8(aq, bk, acc[hb]);
          }
        }
      }
    };
    // Fused epilogue of sub-block sb.  ReLU as a signed-integer max on the
    // bit pattern (negative floats, -0 included, have negative patterns),
    // head sum in kParts chains, the other 16 rows of each head block from
    // lane l ^ 32.
    auto epi = [&](int sb, const f32x16(&acc)[HB]) {
      const int kbase = tbase + sb * 32;
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
      if constexpr (FUSE) {
        {
          auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(sc), __float_as_uint(sc),
                                                     false, false);
          sc = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        }
        const int key = kbase + col;
        const bool vis = g == 0 && live && key < kc && key <= pos;
        const uint32_t kk = float_key(FP8 ? sc * kss[buf][sb * 32 + col] : sc);
        const uint32_t bin = kk >> (32 - kPfBinBits);
        const uint32_t sub = (kk >> (32 - kPfBinBits - kPfSubBits)) & (kPfSubs - 1);
        if (vis) atomicAdd(&wh[pf_bin_at(bin)], 1u);
        if (vis && bin == wbound) atomicAdd(&wsh[sub], 1u);
        const bool cand = vis && (bin > wbound || (bin == wbound && sub >= wsub));
        const uint64_t m = __ballot(cand);
        if (cand) {
          const uint32_t at =
              wcount + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
          ckr[at] = kk;
          cpr[at] = key;
        }
        wcount += (uint32_t)__popcll(m);
      } else {
        // Sub-blocks in pairs, as in the pipelined loop: the even one keeps
        // its per-lane sums, the odd one swaps lane halves with them and
        // stores 64 consecutive scores.  One store per lane, no branch: a
        // lane with nothing to store (an idle wave, a key past kc) points
        // past the row, where the buffer's range check drops the store.
        static_assert(TILE / 32 % 2 == 0, "whole pairs of sub-blocks per tile");
        if ((sb & 1) == 0) {
          stash = sc;
        } else {
          auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(stash), __float_as_uint(sc),
                                                     false, false);
          sc = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
          const int key = kbase - 32 + lane;
          const bool st = live && key < kc;
          const float o = key <= pos ? (FP8 ? sc * kss[buf][sb * 32 - 32 + lane] : sc) : -INFINITY;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o), outr,
                                                (uint32_t)(st ? key : Lmax) * 4u, 0, 0);
        }
      }
    };
#pragma unroll
    for (int sb = 0; sb < TILE / 32; ++sb) {
      // (the fused variant skips sub-blocks past the causal limit; the other
      // computes every pair and stores nothing past kc)
      if (FUSE && tbase + sb * 32 >= kc) break;
      f32x16 acc[HB];
      mma(sb, acc);
      epi(sb, acc);
    }
    if constexpr (FUSE) {  // tighten the bound every 4 tiles (its own lanes' adds are done)
      if ((tile & 3) == 3) {
        uint32_t above = 0;
        const uint32_t nb = pf_wave_bound(wh, (uint32_t)fa.k, lane, wbound, above);
        if (nb != wbound) {  // a higher bin: its earlier keys were not sub-counted, restart
          wbound = nb;
          wsub = 0;
          wsh[lane] = 0;
        } else if (nb > 0 || above > 0) {
          // the sub-histogram undercounts the bin (keys before it became the
          // bound), which can only lower the sub-bound: still a lower bound
          wsub = pf_sub_bound(wsh, (uint32_t)fa.k - above, lane);
        }
      }
    }
    if (tile + 1 < ntiles) lstore(buf ^ 1);
    __syncthreads();
  }
  }
  if constexpr (FUSE) {
    if (live && lane == 0) fa.cnt[row] = wcount;
  }
}

template <bool FP8, int D, int HB, bool FUSE>
hipError_t launch_pf(const void* q, const float* q_scale, const float* w, const void* k,
                     const float* k_scale, const int32_t* ctx_len, int B, int T, int H, int Lmax,
                     float* scores, int64_t ld, const PfFuseArgs& fa, hipStream_t stream) {
  const int qgroups = (T + kPfWaves - 1) / kPfWaves;
  constexpr int TILE = pf_tile(FP8, FUSE);
  const int tiles = (Lmax + TILE - 1) / TILE;
  // Split the keys so the grid holds >= ~8 workgroups per CU (the fused
  // variant keeps each row in one workgroup).
  int splits = (2048 + qgroups * B - 1) / (qgroups * B);
  splits = max(splits, 8);
  splits = FUSE ? 1 : max(1, min(splits, tiles));
  const int tiles_per = (tiles + splits - 1) / splits;
  const int keys_per_wg = tiles_per * TILE;
  const dim3 grid(qgroups, (Lmax + keys_per_wg - 1) / keys_per_wg, B);
  hipLaunchKernelGGL((indexer_prefill_kernel<FP8, D, HB, FUSE>), grid, dim3(kPfThreads), 0,
                     stream, (const uint8_t*)q, q_scale, w, (const uint8_t*)k, k_scale, ctx_len,
                     T, H, Lmax, scores, ld, keys_per_wg, fa);
  return hipGetLastError();
}

template <bool FUSE>
hipError_t dispatch_pf(const void* q, bool fp8, const float* q_scale, const float* w,
                       const void* k, const float* k_scale, const int32_t* ctx_len, int B, int T,
                       int H, int D, int Lmax, float* scores, int64_t ld, const PfFuseArgs& fa,
                       hipStream_t stream) {
#define DSA_PF(F8, DD, HBB)                                                                \
  return launch_pf<F8, DD, HBB, FUSE>(q, q_scale, w, k, k_scale, ctx_len, B, T, H, Lmax, \
                                      scores, ld, fa, stream)
  const bool two = H > 32;
  if (D == 128) {
    if (fp8) { if (two) DSA_PF(true, 128, 2); DSA_PF(true, 128, 1); }
    if (two) DSA_PF(false, 128, 2);
    DSA_PF(false, 128, 1);
  }
  if (fp8) { if (two) DSA_PF(true, 64, 2); DSA_PF(true, 64, 1); }
  if (two) DSA_PF(false, 64, 2);
  DSA_PF(false, 64, 1);
#undef DSA_PF
}

}  // namespace

bool indexer_prefill_supported(int H, int D) { return H >= 1 && H <= 64 && (D == 64 || D == 128); }

hipError_t launch_indexer_prefill(const void* q, bool fp8, const float* q_scale, const float* w,
                                  const void* k, const float* k_scale, const int32_t* ctx_len,
                                  int B, int T, int H, int D, int Lmax, float* scores,
                                  int64_t ld, hipStream_t stream) {
  return dispatch_pf<false>(q, fp8, q_scale, w, k, k_scale, ctx_len, B, T, H, D, Lmax, scores,
                            ld, PfFuseArgs{}, stream);
}

size_t indexer_topk_prefill_workspace_bytes(int B, int T, int Lmax) {
  const size_t rows = (size_t)B * T;
  auto a = [](size_t x) { return (x + 255) & ~size_t(255); };
  return 2 * a(rows * (size_t)Lmax * 4) + a(rows * 4);
}

hipError_t launch_indexer_topk_prefill(const void* q, bool fp8, const float* q_scale,
                                       const float* w, const void* k, const float* k_scale,
                                       const int32_t* ctx_len, int B, int T, int H, int D,
                                       int Lmax, int k_sel, int32_t* idx, void* workspace,
                                       hipStream_t stream) {
  const size_t rows = (size_t)B * T;
  auto a = [](size_t x) { return (x + 255) & ~size_t(255); };
  unsigned char* p = static_cast<unsigned char*>(workspace);
  uint32_t* key = reinterpret_cast<uint32_t*>(p);
  int32_t* pos = reinterpret_cast<int32_t*>(p + a(rows * (size_t)Lmax * 4));
  uint32_t* cnt = reinterpret_cast<uint32_t*>(p + 2 * a(rows * (size_t)Lmax * 4));
  const PfFuseArgs fa{k_sel, key, pos, cnt};
  hipError_t e = dispatch_pf<true>(q, fp8, q_scale, w, k, k_scale, ctx_len, B, T, H, D, Lmax,
                                   nullptr, 0, fa, stream);
  if (e != hipSuccess) return e;
  return launch_topk_candidates(ctx_len, B, T, Lmax, k_sel, key, pos, cnt, idx, stream);
}

}  // namespace dsa
