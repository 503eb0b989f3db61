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
// their scores in LDS while the first radix histogram is built, and the
// workgroup compacts its own candidates (keys in bins >= a threshold bin)
// into its slice of the candidate buffer (a workgroup covers one contiguous
// run of tiles); a finishing kernel then concatenates the slices per row and
// completes the selection from the row's finished histogram.
//
// No workgroup waits for another.  The threshold bin only has to be a lower
// bound of the true one: counts only grow, so the k-th largest key of any
// part of the row's histogram lies in a bin at or below that of the whole
// row, and keys in bins at or above it are a superset of the true candidates
// (the finishing pass never emits the extra ones).  Each wave hands its
// eighth of the workgroup's bins to the row histogram half way through its
// tiles (an LDS exchange with zero, then device-scope adds);
// at the end a workgroup reads the row histogram as it stands, adds the
// counts it has not handed off yet (they cannot be in what it read), takes
// the threshold bin of that sum, and hands those counts off after the read
// has returned.  So the bound covers about half of every workgroup's keys
// (more for those that finished first) plus all of its own.
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
// Buffer accesses here put their whole offset in the vector offset, the part
// the compiler documents as range-checked (gfx950 also checks the scalar
// offset, but nothing here relies on that): a load past the end returns zeros
// without touching memory and a store past it is dropped.  kPastEnd (in
// elements of 4 bytes) lies past the end of every buffer.
constexpr int kPastEnd = 1 << 28;
constexpr int kDeviceScope = 16;  // cache policy sc1: coherent at device scope
constexpr int kParts = 4;  // independent fma chains of the head sum
constexpr int kFuseKeys = 8192;        // keys whose scores a fused workgroup keeps in LDS

// Outputs of the fused variant (chunk slices of the top-k workspace).
struct FuseArgs {
  int k;                // keys to select per row
  int n_chunks;         // chunks per row (kDecWaves tiles each)
  uint32_t* cnt;        // per-(row, chunk) candidate counts
  uint32_t* key;        // candidate keys, Lmax per row, chunk c at c * chunk keys
  int32_t* pos;         // candidate positions, same layout
};

// The arguments the first loads depend on come first: the first 14 argument
// dwords are preloaded into scalar registers at launch.  `plan` packs the
// tiles per wave (low 16 bits) and the workgroups per row (high 16 bits),
// which spares the first loads a wait for the grid size.
template <int D, bool FP8, int HB, bool FUSE>
__global__ __launch_bounds__(kDecWaves * kWave, 2) void indexer_decode_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ k,
    const float* __restrict__ k_scale, int T, int H, int Lmax, int plan,
    const int32_t* __restrict__ ctx_len, float* __restrict__ scores, int64_t ld,
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
  const int tiles_per_wave = plan & 0xffff;
  const int b = row / T;
  const int t = row - b * T;
  const int tiles = (Lmax + TK - 1) / TK;
  // Wave w of the row's W waves takes tiles w, w + W, w + 2W, ...: all
  // waves sweep the row together, front to back (measurably closer to plain
  // streaming bandwidth than giving each wave its own contiguous run).  The
  // loop below runs over the wave's sequence numbers j = 0, 1, ...
  // The fused variant gives each workgroup one contiguous run of
  // kDecWaves * tiles_per_wave tiles instead (its waves interleaved inside
  // it), so that its candidates form one position-ordered slice.
  const int wg_end = FUSE ? min(tiles, (int)(blockIdx.x + 1) * kDecWaves * tiles_per_wave) : tiles;
  const int first = FUSE ? (int)blockIdx.x * kDecWaves * tiles_per_wave + wave
                         : (int)blockIdx.x * kDecWaves + wave;
  const int wstride = FUSE ? kDecWaves : (plan >> 16) * kDecWaves;
  const int tile0 = 0;
  // (a wave past the row's last tile runs no iteration but stays for the
  // workgroup barriers of the histogram)
  const int tend =
      first < wg_end ? min(tiles_per_wave, (wg_end - first + wstride - 1) / wstride) : 0;
  auto tmap = [&](int j) { return __builtin_amdgcn_readfirstlane(first + j * wstride); };
  // fused: the tile after which a wave hands its bins off (none if < 0)
  const int hand_off = tend / 2 - 1;
  int64_t pos = 0;  // the row's position: read after the first loads are issued
  unsigned char* my_stage = stage + wave * TK * PITCH;

  // The row's query block, head weights and query scales are the same for
  // all eight waves, so they are loaded once per workgroup and shared
  // through LDS: each thread loads one 16-byte share of the (zero-padded)
  // query block and every wave one weight and one scale per lane, through
  // buffer resources over this row (a head past H reads zeros and adds
  // nothing).  These few loads go out ahead of the first key tiles, whose
  // requests then do not queue behind 8 copies of the same prologue loads
  // (24 per wave: the first tiles were issued 5 us into the launch at the
  // median, 13 us for the last waves); the memory counter completes in
  // order, so waiting for these loads does not wait for the tiles.
  constexpr int QPITCH = ROWB + 16;                     // LDS row pitch of the query block
  constexpr int QCH = HB * 32 * ROWB / 16;              // 16-byte chunks of the block
  constexpr int QPT = (QCH + kDecWaves * kWave - 1) / (kDecWaves * kWave);  // per thread
  __shared__ __align__(16) unsigned char qsh[HB * 32 * QPITCH];
  __shared__ __align__(16) float wsh[HB * 32];
  i32x4 qld[QPT];
  float wl, ql;
  {
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(q + (int64_t)row * H * ROWB), 0, H * ROWB, kBufferWord3);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(w + (int64_t)row * H), 0, H * 4, kBufferWord3);
    const __amdgpu_buffer_rsrc_t qsr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(FP8 ? q_scale + (int64_t)row * H : w), 0, FP8 ? H * 4 : 0, kBufferWord3);
#pragma unroll
    for (int u = 0; u < QPT; ++u)
      qld[u] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             qr, (threadIdx.x + kDecWaves * kWave * u) * 16, 0, 0));
    wl = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(wr, lane * 4, 0, 0));
    ql = FP8 ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(qsr, lane * 4, 0, 0))
             : 1.f;
  }
  // Operand A fragments and head weights of this wave, from LDS after the
  // prologue barrier.
  i32x4 qv[HB][NV];
  float wv[HB][16];
  auto share_prologue = [&]() {  // before the barrier
#pragma unroll
    for (int u = 0; u < QPT; ++u) {
      const int c = threadIdx.x + kDecWaves * kWave * u;
      if (c < QCH)
        *reinterpret_cast<i32x4*>(qsh + (c / (ROWB / 16)) * QPITCH + (c % (ROWB / 16)) * 16) =
            qld[u];
    }
    // w' = w (bf16) or w * q_scale (fp8: the positive per-row scales commute
    // with the ReLU)
    if (wave == 0 && lane < HB * 32) wsh[lane] = wl * ql;
  };
  auto take_prologue = [&]() {  // after the barrier
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
      for (int v = 0; v < NV; ++v)
        qv[hb][v] = *reinterpret_cast<const i32x4*>(qsh + (hb * 32 + col) * QPITCH + g * HALF +
                                                    16 * v);
      // Accumulator rows r = 4j .. 4j+3 are heads hb*32 + 8j + 4g + 0..3.
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 wq = *reinterpret_cast<const f32x4*>(wsh + hb * 32 + 8 * j + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) wv[hb][4 * j + e] = wq[e];
      }
    }
  };

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
  // Every path through the tile loop issues the same vector-memory operations:
  // a sequence number past the wave's share reads tile `tiles`, wholly beyond
  // the buffers, which returns zeros without touching memory, and the score
  // stores of the upper half-wave go to an offset past the end of the row.
  // The compiler's memory waits are merged over all paths that reach a point,
  // so with a conditional load or store the steady state inherited the waits
  // of the last iteration (a full drain of the prefetched tiles inside every
  // tile's arithmetic).
  auto load = [&](int seq, i32x4(&buf)[NL], float(&bs)[CB]) {
    const int tile = seq < tend ? tmap(seq) : tiles;
#pragma unroll
    for (int v = 0; v < NL; ++v)
      buf[v] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             kr, tile * kTileBytes + 1024 * v + 16 * lane, 0,
                                             kNT));
    if (FP8) {
#pragma unroll
      for (int c = 0; c < CB; ++c)
        bs[c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                              sr, (tile * TK + c * 32 + col) * 4, 0, kNT));
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
    float scs[CB];  // per-lane head sums of each block (even CB)
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
      if constexpr (CB % 2 == 0) {
        scs[c] = sc;  // (the two lane halves are added below, two blocks at a time)
      } else {
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(sc), __float_as_uint(sc),
                                                   false, false);
        sc = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        const int key = tile * TK + c * 32 + col;
        const bool vis = key <= pos && key < Lmax;
        const float o = vis ? (FP8 ? sc * cs[c] : sc) : -INFINITY;
        if constexpr (!FUSE)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o), outr,
                                                (key + (g ? kPastEnd : 0)) * 4, 0, 0);
        if (g == 0) {
          if constexpr (FUSE) sbuf[(seq * kDecWaves + wave) * TK + c * 32 + col] = o;
          if (row_hist && vis) atomicAdd(&lhist[float_key(o) >> (32 - kHistBits)], 1u);
        }
      }
    }
    if constexpr (CB % 2 == 0) {
      // Blocks c and c + 1 in one lane swap: the swap exchanges the upper
      // half of its first operand with the lower half of its second, so the
      // sum of the two results holds block c's scores in lanes 0..31 and
      // block c + 1's in lanes 32..63, i.e. key c * 32 + lane, and one store
      // of 64 consecutive scores writes both.
#pragma unroll
      for (int c = 0; c < CB; c += 2) {
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(scs[c]),
                                                   __float_as_uint(scs[c + 1]), false, false);
        const float sc = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        const int key = tile * TK + c * 32 + lane;
        const bool vis = key <= pos && key < Lmax;
        const float o = vis ? (FP8 ? sc * (g ? cs[c + 1] : cs[c]) : sc) : -INFINITY;
        if constexpr (!FUSE)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o), outr, key * 4, 0, 0);
        if constexpr (FUSE) sbuf[(seq * kDecWaves + wave) * TK + c * 32 + lane] = o;
        if (row_hist && vis) atomicAdd(&lhist[float_key(o) >> (32 - kHistBits)], 1u);
      }
    }
    __builtin_amdgcn_wave_barrier();
    if constexpr (FUSE) {
      if (seq == hand_off) {  // this wave's eighth of the bins, counted so far
        uint32_t* rh = row_hist + (int64_t)row * kHistBins;
#pragma unroll
        for (int u = 0; u < kHistBins / kDecWaves / kWave; ++u) {
          const int i = wave * (kHistBins / kDecWaves) + lane + kWave * u;
          const uint32_t c = atomicExch(&lhist[i], 0u);
          if (c) __hip_atomic_fetch_add(&rh[i], c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  };
  __builtin_amdgcn_sched_barrier(0);  // the prologue loads go first
  load(tile0, ba, sa);
  load(tile0 + 1, bb, sb);
  __builtin_amdgcn_sched_barrier(0);  // then the first key tiles
  pos = (int64_t)ctx_len[b] - T + t;  // (its argument is not preloaded: read it now)
  share_prologue();
  if (row_hist)  // cleared while the first tiles stream in
    for (int i = threadIdx.x; i < kHistBins; i += kDecWaves * kWave) lhist[i] = 0;
  __syncthreads();
  take_prologue();
  // Whole rounds of three tiles, then the zero to two left over: the loop has
  // no exit in its body, so no path into its head skips a round's loads.
  int tile = tile0;
  for (; tile + 3 <= tend; tile += 3) {
    load(tile + 2, bc, sc_);
    compute(tile, ba, sa);
    load(tile + 3, ba, sa);
    compute(tile + 1, bb, sb);
    load(tile + 4, bb, sb);
    compute(tile + 2, bc, sc_);
  }
  if (tile < tend) compute(tile, ba, sa);
  if (tile + 1 < tend) compute(tile + 1, bb, sb);
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
    if (n <= fa.k) return;  // the whole row is selected: no candidates needed
    __syncthreads();  // every tile done; lhist holds the counts not handed off
    uint32_t* rh = row_hist + (int64_t)row * kHistBins;
    // A lower bound of the row's histogram: the row histogram as it stands
    // plus this workgroup's counts not handed off yet.  Thread t owns bins
    // 4 (t + NT u) .. +3; the 16-byte loads are device-scope (they bypass
    // this XCD's possibly stale L2 lines, as an atomic load does).
    constexpr int HV4 = HV / 4;
    i32x4 own[HV4];
    {
      const __amdgpu_buffer_rsrc_t hr =
          __builtin_amdgcn_make_buffer_rsrc((void*)rh, 0, kHistBins * 4, kBufferWord3);
      i32x4 hv[HV4];
#pragma unroll
      for (int u = 0; u < HV4; ++u)
        hv[u] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              hr, (threadIdx.x + NT * u) * 16, 0, kDeviceScope));
#pragma unroll
      for (int u = 0; u < HV4; ++u)
        own[u] = *reinterpret_cast<const i32x4*>(&lhist[4 * (threadIdx.x + NT * u)]);
#pragma unroll
      for (int u = 0; u < HV4; ++u)
        *reinterpret_cast<i32x4*>(&lhist[4 * (threadIdx.x + NT * u)]) = hv[u] + own[u];
    }
    // fewer than k keys counted so far: no bin holds the k-th, and bin 0
    // (every key a candidate) is the bound
    if (threadIdx.x == 0) fsel[0] = 0;
    __syncthreads();
    select_bin<kHistBins, NT>(lhist, (uint32_t)fa.k, fscan, fsel);
    const uint32_t b1 = fsel[0];
    // Hand off the rest; the read above has returned (its values were used),
    // so it cannot have counted these.
#pragma unroll
    for (int u = 0; u < HV4; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (own[u][e])
          __hip_atomic_fetch_add(&rh[4 * (threadIdx.x + NT * u) + e], (uint32_t)own[u][e],
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // Ordered compaction of the workgroup's keys (sbuf holds them in
    // position order from p_base) into its slice, 8 consecutive keys per
    // thread per pass.
    const int keys_wg = kDecWaves * tiles_per_wave * TK;
    const int p_base = (int)blockIdx.x * keys_wg;
    uint32_t* ck = fa.key + (int64_t)row * Lmax + p_base;
    int32_t* cp = fa.pos + (int64_t)row * Lmax + p_base;
    uint32_t run = 0;
    for (int b0 = 0; b0 < keys_wg; b0 += NT * 8) {
      const int l0 = b0 + (int)threadIdx.x * 8;
      const bool mine = l0 < keys_wg;  // keys_wg is a multiple of 8
      uint32_t key[8];
      bool ok[8];
      uint32_t c = 0;
      const float4 f0 = mine ? *reinterpret_cast<const float4*>(&sbuf[l0]) : float4{};
      const float4 f1 = mine ? *reinterpret_cast<const float4*>(&sbuf[l0 + 4]) : float4{};
      key[0] = float_key(f0.x); key[1] = float_key(f0.y);
      key[2] = float_key(f0.z); key[3] = float_key(f0.w);
      key[4] = float_key(f1.x); key[5] = float_key(f1.y);
      key[6] = float_key(f1.z); key[7] = float_key(f1.w);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ok[e] = mine && (p_base + l0 + e) < n && (key[e] >> (32 - kHistBits)) >= b1;
        c += ok[e];
      }
      uint32_t tot;
      uint32_t at = run + block_excl_scan<kDecWaves>(c, fscan, tot);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (ok[e]) {
          ck[at] = key[e];
          cp[at] = p_base + l0 + e;
          ++at;
        }
      run += tot;
    }
    if (threadIdx.x == 0) fa.cnt[(int64_t)row * fa.n_chunks + blockIdx.x] = run;
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
// The fused variant's chunks are its workgroups' runs of tiles.
int fused_chunks(const DecPlan& p) { return p.gx; }

template <int D, bool FP8, int HB, bool FUSE>
hipError_t launch_dec(const DecPlan& p, const void* q, const float* q_scale, const float* w,
                      const void* k, const float* k_scale, const int32_t* ctx_len, int rows,
                      int T, int H, int Lmax, float* scores, int64_t ld, uint32_t* row_hist,
                      const FuseArgs& fa, hipStream_t stream) {
  if (p.tpw >= (1 << 16) || p.gx >= (1 << 15)) return hipErrorInvalidValue;  // plan packing
  dim3 grid(p.gx, rows);
  hipLaunchKernelGGL((indexer_decode_kernel<D, FP8, HB, FUSE>), grid, dim3(kDecWaves * kWave), 0,
                     stream, (const uint8_t*)q, q_scale, w, (const uint8_t*)k, k_scale, T, H,
                     Lmax, p.tpw | (p.gx << 16), ctx_len, scores, ld, row_hist, fa);
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
  const TopkWs ws = topk_chunk_ws(workspace, rows, Lmax, n_chunks);
  const FuseArgs fa{k_sel, n_chunks, ws.cnt, ws.key, ws.pos};
  hipError_t e = dispatch_dec<true>(p, q, fp8, q_scale, w, k, k_scale, ctx_len, rows, T, H, D,
                                    Lmax, nullptr, 0, ws.hist, fa, stream);
  if (e != hipSuccess) return e;
  // no score row in memory, and the threshold is taken from the finished
  // histogram (the fused kernel's was only a lower bound)
  return launch_topk_finish(nullptr, 0, ctx_len, B, T, Lmax, k_sel, kDecWaves * p.tpw * p.tk,
                            n_chunks, ws, true, idx, stream);
}

}  // namespace dsa
