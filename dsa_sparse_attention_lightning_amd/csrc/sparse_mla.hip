// Sparse MLA attention over the selected latent rows (IndexCache paper
// summary, technical §1: core attention over only the k selected tokens).
//
// Absorbed MLA: every token has one latent row of 576 bf16 (512 value + 64
// rope) shared by all heads.  For one query row (b,t) the work is
//   S = q[Hq x 576] . kv_sel^T     P = online-softmax(S)     O = P . kv_sel[:, :512]
// over the k gathered rows: 2*Hq*k*(576+512) flops against k*1152 gathered
// bytes, so both products run on MFMA (16x16x32 bf16) with an fp32
// online-softmax accumulator.
//
// Work split: a workgroup owns one query row, 16*HGW heads and one slice of
// the k selected rows (split-KV; a combine kernel merges slices by their
// log-sum-exp; slice outputs are kept in bf16 after normalisation).  Each wave owns 16 heads: its query block stays in registers
// (operand B of S^T = K . q^T) and its O^T accumulator [512 x 16] is 128 fp32
// per lane.  Rows are processed 32 at a time:
//   * the 32 selected rows are gathered straight from HBM into LDS with
//     16-byte LDS-DMA loads (global_load_lds_dwordx4), double-buffered so the
//     next tile streams in while the current one is multiplied;
//   * the tile is stored row-major with a row pitch of 73 16-byte chunks
//     (1168 B): the 16-byte row reads of S^T hit 8 distinct bank groups per
//     8 lanes, the transposing reads at most 2-way conflicts, and every LDS
//     address is a per-lane base plus an immediate;
//   * S^T reads 16-byte row fragments (operand A);
//   * O^T += V^T . P^T takes operand A (8 consecutive rows of one latent dim
//     per lane) with two transposing LDS reads (ds_read_b64_tr_b16) from the
//     same row-major tile, and operand B straight from the S^T accumulator:
//     the reduction order kappa = 8g + j is mapped to tile rows
//     rho(kappa) = 4g + j (j < 4), 16 + 4g + j - 4 (j >= 4), which is where
//     the 16x16 accumulator of S^T leaves them.
#include "device_common.hpp"
#include "launchers.hpp"

namespace dsa {
namespace {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kRows = 32;                 // rows per tile
constexpr int kRowBytes = kDqk * 2;       // 1152
constexpr int kChunks = kDqk / 8;         // 16-byte chunks per row (72)
constexpr int kPitchChunks = kChunks + 1; // LDS row pitch in 16-byte chunks (73)
constexpr int kPitch = kPitchChunks * 16; // 1168
constexpr int kTileSlots = kRows * kPitchChunks;                  // 2336
constexpr int kTileLoads = (kTileSlots + kWave - 1) / kWave;      // 37 wave-loads
constexpr int kTileBytes = kTileLoads * kWave * 16;               // 37888 (with slack)
constexpr int kMaxSplitRows = 1024;
constexpr int kOutPitch = 528;            // LDS pitch of a staged 256-dim bf16 output row
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.f;   // log2 headroom of the lazy softmax rescale
#ifndef DSA_ATTN_XCD
#define DSA_ATTN_XCD 1
#endif

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i32x4 lds_i32x4;


// Slot of one 16-byte LDS-DMA load inside a tile: instruction i of the tile
// writes slots 64 i .. 64 i + 63, and slot p holds chunk p % 73 of row p / 73.
// The pad slot of each row and the slack after the last row receive a
// harmless copy of chunk 0 of row 0.  Packed as (row << 16) | byte offset.
__device__ __forceinline__ int gather_slot(int i, int lane) {
  const int p = i * kWave + lane;
  int r = p / kPitchChunks;
  int c = p - r * kPitchChunks;
  if (c >= kChunks) c = 0;
  if (r >= kRows) { r = 0; c = 0; }
  return (r << 16) | (c * 16);
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maximum), as a
// builtin so that the compiler's own wait-count tracking sees it.
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier for LDS-only exchanges: this wave's LDS writes are
// complete before the barrier, but in-flight global loads (the LDS-DMA of the
// next tile) are not waited for, unlike __syncthreads().
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Maximum over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float max_over_rows(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats to packed bf16 (round to nearest even, one instruction).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ v4i16 tr_read(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
}

// Merge the split-KV partials of one (query row, head, 8 dims) unit:
// out = sum_i exp(lse_i - lse) * o_i, lse = log sum_i exp(lse_i).
constexpr int kCombUnroll = 8;
__device__ __forceinline__ void combine_unit(const __bf16* __restrict__ part_o,
                                             const float* __restrict__ part_lse, int Hq,
                                             int n_split, int row, int head, int d,
                                             __bf16* __restrict__ out, float* __restrict__ lse,
                                             bool write_lse) {
  const float* pl = part_lse + (int64_t)row * n_split * Hq + head;
  float mx = -INFINITY;
  for (int i = 0; i < n_split; ++i) mx = fmaxf(mx, pl[(int64_t)i * Hq]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (mx != -INFINITY) {
    const __bf16* po = part_o + ((int64_t)row * n_split * Hq + head) * kDv + d;
    for (int i0 = 0; i0 < n_split; i0 += kCombUnroll) {
      i32x4 v[kCombUnroll];
      float wi[kCombUnroll];
#pragma unroll
      for (int u = 0; u < kCombUnroll; ++u) {
        const int i = min(i0 + u, n_split - 1);
        v[u] = ld16(po + (int64_t)i * Hq * kDv);
        const float li = pl[(int64_t)i * Hq];
        wi[u] = (i0 + u < n_split && li != -INFINITY) ? expf(li - mx) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kCombUnroll; ++u) {
        den += wi[u];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t x = (uint32_t)v[u][e];
          acc[2 * e] += wi[u] * __uint_as_float(x << 16);
          acc[2 * e + 1] += wi[u] * __uint_as_float(x & 0xFFFF0000u);
        }
      }
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  i32x4 pk;
#pragma unroll
  for (int e = 0; e < 4; ++e) pk[e] = (int)pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
  *reinterpret_cast<i32x4*>(out + ((int64_t)row * Hq + head) * kDv + d) = pk;
  if (write_lse && lse != nullptr)
    lse[(int64_t)row * Hq + head] = den > 0.f ? mx + logf(den) : -INFINITY;
}

// HGW head groups of 16 heads per workgroup, two waves per group.  Wave
// (hg, h) computes the partial S^T over latent dims [288 h, 288 h + 288),
// the pair exchanges partials through LDS, both apply the same online
// softmax, and wave h accumulates O^T for value dims [256 h, 256 h + 256).
template <int HGW>
__global__ __launch_bounds__(HGW * 2 * kWave) void sparse_mla_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ kv, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ ctx_len, int T, int Hq, int Lmax, int k, int rows_per_split,
    float scale_log2, __bf16* __restrict__ out, float* __restrict__ lse,
    __bf16* __restrict__ part_o, float* __restrict__ part_lse, int n_split, int head_groups,
    int n_work, int per_xcd) {
  constexpr int NW = HGW * 2;
  constexpr int NT = NW * kWave;
  constexpr int KJ = (kTileLoads + NW - 1) / NW;  // DMA instructions per wave per tile
  // Three tile buffers, as separate LDS objects so that the compiler can tell
  // that reading one buffer does not depend on the DMA still writing another.
  // While tile n is multiplied by P, tile n+1 is multiplied by q and tile n+2
  // streams in.
  __shared__ __attribute__((aligned(16))) unsigned char tileA[kTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char tileB[kTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char tileC[kTileBytes];
  __shared__ f32x4 xs[2][HGW][2][2][kWave];  // partial S^T exchange: [tile parity][group][half][mb][lane]
  __shared__ int32_t rows[kMaxSplitRows];
  __shared__ __attribute__((aligned(16))) float bias[kMaxSplitRows];  // 0 or -inf per row

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int hg = wave >> 1;      // head group inside the workgroup
  const int h = wave & 1;        // which half of the dims this wave owns
  const int g = lane >> 4;
  const int c16 = lane & 15;
  // Work item w = ((row * n_split) + split) * head_groups + head group.  The
  // dispatcher deals consecutive workgroups to the 8 XCDs in turn, so
  // workgroup i runs on XCD i % 8; giving each XCD one contiguous range of
  // work items keeps a query row's fragments and the rows its head groups
  // gather together in one XCD's L2 instead of fetching them 8 times.
#if DSA_ATTN_XCD
  const int bid = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
#else
  const int bid = blockIdx.x;
#endif
  if (bid >= n_work) return;
  const int hgi = bid % head_groups;
  const int rs = bid / head_groups;
  const int split = rs % n_split;
  const int row = rs / n_split;  // b * T + t
  const int b = row / T;
  const int t = row - b * T;
  const int head = (hgi * HGW + hg) * 16 + c16;
  const int64_t pos = (int64_t)ctx_len[b] - T + t;
  const int j0 = split * rows_per_split;
  const int nrows = max(0, min(k, j0 + rows_per_split) - j0);
  const int ntiles = (nrows + kRows - 1) / kRows;

  // Selected rows of this slice, validated once (invalid / padding -> -1,
  // whose score bias is -inf).
  const int32_t* ib = idx + (int64_t)row * k + j0;
  for (int j = tid; j < ntiles * kRows; j += NT) {
    int v = (j < nrows) ? ib[j] : -1;
    if (v < 0 || (int64_t)v > pos || v >= Lmax) v = -1;
    rows[j] = v;
    bias[j] = v >= 0 ? 0.f : -INFINITY;
  }
  // This wave's DMA slots are the same for every tile.
  int gslot[KJ];
#pragma unroll
  for (int j = 0; j < KJ; ++j) gslot[j] = gather_slot(wave + NW * j, lane);
  __syncthreads();
  const unsigned char* kvb = reinterpret_cast<const unsigned char*>(kv + (int64_t)b * Lmax * kDqk);
  // Issue the LDS-DMA gather of one 32-row tile: look up the rows of all of
  // this wave's slots first, then issue the loads back to back (a slot past
  // the tile's last instruction maps to row 0: its lookup is harmless and its
  // load is skipped; only the last j can be such a slot).
  auto gather = [&](unsigned char* tile, int tbase) {
    int src[KJ];
#pragma unroll
    for (int j = 0; j < KJ; ++j) src[j] = rows[tbase + (gslot[j] >> 16)];
#pragma unroll
    for (int j = 0; j < KJ; ++j)
      if (NW * j + NW - 1 < kTileLoads || wave + NW * j < kTileLoads)
        __builtin_amdgcn_global_load_lds(
            (const void*)(kvb + (int64_t)max(src[j], 0) * kRowBytes + (gslot[j] & 0xffff)),
            (lds_void*)(tile + (wave + NW * j) * kWave * 16), 16, 0, 0);
  };
  // The first two tiles are requested together: a slice of 64 rows (the
  // common decode case) then waits on a single round trip to HBM.
  if (ntiles > 0) gather(tileA, 0);
  if (ntiles > 1) gather(tileB, kRows);

  // Query fragments for this wave's half of the latent dims: operand B of
  // S^T (column = head, reduction = dims); lane group g covers dims
  // [288 h + 72 g, 288 h + 72 g + 72).
  bf16x8 qf[9];
  {
    const __bf16* qp = q + ((int64_t)row * Hq + head) * kDqk + 288 * h + 72 * g;
#pragma unroll
    for (int i = 0; i < 9; ++i) qf[i] = as_bf16x8(ld16(qp + 8 * i));
  }
  // The fragments must have arrived before the tile loop starts: otherwise
  // the compiler may move these loads below the barrier, and the wait for
  // them then sits at the loop head, where it would also wait for every
  // tile's DMA.
  asm volatile("" ::"v"(qf[0]), "v"(qf[1]), "v"(qf[2]), "v"(qf[3]), "v"(qf[4]), "v"(qf[5]),
               "v"(qf[6]), "v"(qf[7]), "v"(qf[8]));
  f32x4 o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // Per-lane LDS byte offsets that do not depend on the tile.
  // S^T operand A: row (16 mb + c16), dims 288 h + 72 g + 8 i.
  // O^T operand A (transposing reads): source row 4g + (c16 >> 2) (+16),
  // dims 256 h + 16 mb + 4 (c16 & 3).
  const int qk_base = c16 * kPitch + 576 * h + 144 * g;
  const int tr_base = (4 * g + (c16 >> 2)) * kPitch + 512 * h + 8 * (c16 & 3);

  // Partial S^T [32 rows x 16 heads] of one tile over this wave's dims.
  auto qk = [&](const unsigned char* tile, f32x4& s0, f32x4& s1) {
    i32x4 ka[9], kb[9];
    const unsigned char* ap = tile + qk_base;
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      ka[i] = *(const lds_i32x4*)(ap + 16 * i);
      kb[i] = *(const lds_i32x4*)(ap + 16 * kPitch + 16 * i);
    }
    s0 = f32x4{0.f, 0.f, 0.f, 0.f};
    s1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      s0 = mfma16_bf16(as_bf16x8(ka[i]), qf[i], s0);
      s1 = mfma16_bf16(as_bf16x8(kb[i]), qf[i], s1);
    }
  };

  f32x4 sp0, sp1;  // this wave's partial S^T of the tile about to be softmaxed
  if (ntiles > 0) {
    wait_vm_all();
    __syncthreads();
    qk(tileA, sp0, sp1);
  }

  // One step: softmax and P.V of tile n (buffer P) while S^T of tile n+1
  // (buffer Q, resident) is formed and tile n+2 streams into buffer D, which
  // held tile n-1.  One barrier per step: after it, tile n+1 has landed
  // (every wave waited for its own DMA), the partials of tile n are visible,
  // and every wave has finished tile n-1, so D may be overwritten.
  auto step = [&](int n, const unsigned char* P, const unsigned char* Q, unsigned char* D) {
    const int par = n & 1;
    f32x4* xs_mine = xs[par][hg][h][0];
    const f32x4* xs_other = xs[par][hg][h ^ 1][0];
    xs_mine[lane] = sp0;
    xs_mine[kWave + lane] = sp1;
    wait_vm_all();
    __syncthreads();
    if (n + 2 < ntiles) gather(D, (n + 2) * kRows);
    const int tbase = n * kRows;
    const f32x4 t0 = xs_other[lane];
    const f32x4 t1 = xs_other[kWave + lane];
    const f32x4 bias0 = *reinterpret_cast<const f32x4*>(bias + tbase + 4 * g);
    const f32x4 bias1 = *reinterpret_cast<const f32x4*>(bias + tbase + 16 + 4 * g);
    // both waves of the pair form the same sum in the same order
    const f32x4 s0 = h ? (t0 + sp0) : (sp0 + t0);
    const f32x4 s1 = h ? (t1 + sp1) : (sp1 + t1);
    // ---- S^T of the next tile: the products run on the matrix cores while
    // the softmax below runs on the vector ALUs.  Unconditional, so that both
    // sit in one scheduling region: after the last tile it multiplies a stale
    // buffer and the result is never used.
    qk(Q, sp0, sp1);
    // ---- operand A of O^T (value dims x rows), independent of P
    v4i16 va[16], vb[16];
    {
      const unsigned char* vp = P + tr_base;
#pragma unroll
      for (int mb = 0; mb < 16; ++mb) {
        va[mb] = tr_read(vp + 32 * mb);
        vb[mb] = tr_read(vp + 32 * mb + 16 * kPitch);
      }
    }
    // ---- online softmax (log2 domain); lane holds rows 4g+r and 16+4g+r
    float sv[8];
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sv[r] = fmaf(s0[r], scale_log2, bias0[r]);
      sv[4 + r] = fmaf(s1[r], scale_log2, bias1[r]);
      mt = fmaxf(mt, fmaxf(sv[r], sv[4 + r]));
    }
    mt = max_over_rows(mt);
    // Lazy rescaling: the reference max m_run only moves when a tile's max
    // exceeds it by more than 2^kLazy.  P = 2^(s - m_run) then stays below
    // 2^kLazy, and O, l and the log-sum-exp all use the same reference, so the
    // result is the exact softmax; the O rescale runs only when some head's
    // reference moves, which is rare after the first tile.
    const bool need = mt > m_run + kLazy;
    if (__any(need)) {
      const float m_new = need ? mt : m_run;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) o[i] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    // m_run is -inf only while every row so far was masked; then every s is
    // -inf and P is 0.
    const float mref = (m_run == -INFINITY) ? 0.f : m_run;
    float ls = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      sv[r] = __builtin_amdgcn_exp2f(sv[r] - mref);
      ls += sv[r];
    }
    l_run += ls;
    i32x4 pb;
    pb[0] = (int)cvt_pk_bf16(sv[0], sv[1]);
    pb[1] = (int)cvt_pk_bf16(sv[2], sv[3]);
    pb[2] = (int)cvt_pk_bf16(sv[4], sv[5]);
    pb[3] = (int)cvt_pk_bf16(sv[6], sv[7]);
    const bf16x8 pbf = as_bf16x8(pb);
    // ---- O^T [256 x 16] += V^T . P^T for this wave's value dims
#pragma unroll
    for (int mb = 0; mb < 16; ++mb) {
      const v4i16 pair[2] = {va[mb], vb[mb]};
      o[mb] = mfma16_bf16(__builtin_bit_cast(bf16x8, pair), pbf, o[mb]);
    }
  };

  // Unrolled by three so that every buffer role is static.
  for (int n = 0; n < ntiles; n += 3) {
    step(n, tileA, tileB, tileC);
    if (n + 1 >= ntiles) break;
    step(n + 1, tileB, tileC, tileA);
    if (n + 2 >= ntiles) break;
    step(n + 2, tileC, tileA, tileB);
  }
  __syncthreads();  // every wave is done with the tiles: they stage the output

  // ---- finish: total row sum over the four lane groups
  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16, kWave);
  l_tot += __shfl_xor(l_tot, 32, kWave);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  const float lse_v = (l_tot > 0.f) ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  // lane holds O^T[dim = 256 h + 16 mb + 4 g + r][head].  The wave's
  // [16 heads x 256 dims] bf16 block is staged in LDS (the tile buffers are
  // free now; rows padded to 528 bytes, half of the waves in each of two
  // buffers) and written out as contiguous rows: a normalised partial
  // (split-KV) or the final output.
  static_assert(HGW * 16 * kOutPitch <= kTileBytes, "output staging fits the tiles");
  unsigned char* st = (wave < HGW ? tileA : tileB) + (wave % HGW) * (16 * kOutPitch);
#pragma unroll
  for (int mb = 0; mb < 16; ++mb) {
    uint2 pk;
    pk.x = cvt_pk_bf16(o[mb][0] * inv, o[mb][1] * inv);
    pk.y = cvt_pk_bf16(o[mb][2] * inv, o[mb][3] * inv);
    *reinterpret_cast<uint2*>(st + c16 * kOutPitch + 32 * mb + 8 * g) = pk;
  }
  __builtin_amdgcn_wave_barrier();
  __bf16* dst = (n_split == 1)
                    ? out + ((int64_t)row * Hq + head - c16) * kDv
                    : part_o + (((int64_t)row * n_split + split) * Hq + head - c16) * kDv;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int hr = 2 * i + (lane >> 5);  // head row inside the wave's block
    const int cb = 16 * (lane & 31);     // byte inside the row's 512
    const i32x4 v = *reinterpret_cast<const i32x4*>(st + hr * kOutPitch + cb);
    *reinterpret_cast<i32x4*>(dst + (int64_t)hr * kDv + 256 * h + cb / 2) = v;
  }
  if (g == 0 && h == 0) {
    if (n_split == 1) {
      if (lse != nullptr) lse[(int64_t)row * Hq + head] = lse_v;
    } else {
      part_lse[((int64_t)row * n_split + split) * Hq + head] = lse_v;
    }
  }
}

// Merge split-KV partials.  One workgroup per (query row, 2 heads); a thread
// owns 8 dims.
constexpr int kCombHeads = 2;
__global__ __launch_bounds__(kCombHeads * 64) void sparse_mla_combine_kernel(
    const __bf16* __restrict__ part_o, const float* __restrict__ part_lse, int Hq, int n_split,
    __bf16* __restrict__ out, float* __restrict__ lse) {
  const int head = blockIdx.y * kCombHeads + threadIdx.x / 64;
  if (head >= Hq) return;
  combine_unit(part_o, part_lse, Hq, n_split, blockIdx.x, head, (threadIdx.x & 63) * 8, out,
               lse, (threadIdx.x & 63) == 0);
}

#ifndef DSA_ATTN_WG_TARGET
#define DSA_ATTN_WG_TARGET 256
#endif
#ifndef DSA_ATTN_MIN_SPLIT_ROWS
#define DSA_ATTN_MIN_SPLIT_ROWS 128
#endif
#ifndef DSA_ATTN_MAX_HGW
#define DSA_ATTN_MAX_HGW 4
#endif

struct SplitPlan {
  int hgw, head_groups, n_split, rows_per_split;
};

SplitPlan plan_split(int B, int T, int Hq, int k) {
  SplitPlan p;
  const int hb = Hq / 16;
  p.hgw = (hb % 4 == 0 && DSA_ATTN_MAX_HGW >= 4) ? 4 : (hb % 2 == 0 && DSA_ATTN_MAX_HGW >= 2) ? 2 : 1;
  p.head_groups = hb / p.hgw;
  const int base = B * T * p.head_groups;
  const int tiles = (k + kRows - 1) / kRows;
  // Enough workgroups to fill the CUs, but every split writes Hq*512 fp32
  // partials (the size of ~230 gathered rows), so keep splits long.
  int ns = (DSA_ATTN_WG_TARGET + base - 1) / base;
  ns = min(ns, max(1, tiles / (DSA_ATTN_MIN_SPLIT_ROWS / kRows)));
  ns = max(ns, (k + kMaxSplitRows - 1) / kMaxSplitRows);
  ns = max(1, min(ns, tiles));
  const int tiles_per = (tiles + ns - 1) / ns;
  p.rows_per_split = tiles_per * kRows;
  p.n_split = (k + p.rows_per_split - 1) / p.rows_per_split;
  return p;
}

}  // namespace

namespace {

size_t part_bytes(const SplitPlan& p, int B, int T, int Hq) {
  const size_t rows = (size_t)B * T * p.n_split * Hq;
  return (rows * kDv * 2 + rows * sizeof(float) + 255) & ~size_t(255);
}

template <int HGW>
hipError_t launch_attn(const SplitPlan& p, const __bf16* q, const __bf16* kv, const int32_t* idx,
                       const int32_t* ctx_len, int B, int T, int Hq, int Lmax, int k, float sl2,
                       __bf16* out, float* lse, __bf16* part_o, float* part_lse,
                       hipStream_t stream) {
  const int n_work = B * T * p.head_groups * p.n_split;
  const int per_xcd = (n_work + 7) / 8;
  const dim3 grid(DSA_ATTN_XCD ? 8 * per_xcd : n_work);
  hipLaunchKernelGGL((sparse_mla_kernel<HGW>), grid, dim3(HGW * 2 * kWave), 0, stream, q, kv,
                     idx, ctx_len, T, Hq, Lmax, k, p.rows_per_split, sl2, out, lse, part_o,
                     part_lse, p.n_split, p.head_groups, n_work, per_xcd);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_split <= 1) return e;
  hipLaunchKernelGGL(sparse_mla_combine_kernel, dim3(B * T, (Hq + kCombHeads - 1) / kCombHeads),
                     dim3(kCombHeads * 64), 0, stream, part_o, part_lse, Hq, p.n_split, out, lse);
  return hipGetLastError();
}

}  // namespace

size_t sparse_attn_workspace_bytes(int B, int T, int Hq, int k, int) {
  const SplitPlan p = plan_split(B, T, Hq, k);
  if (p.n_split <= 1) return 0;
  return part_bytes(p, B, T, Hq);
}

hipError_t launch_sparse_attn(const void* q, const void* kv, const int32_t* idx,
                              const int32_t* ctx_len, int B, int T, int Hq, int Lmax, int k,
                              float scale, void* out, float* lse, void* workspace,
                              size_t ws_bytes, hipStream_t stream) {
  const SplitPlan p = plan_split(B, T, Hq, k);
  __bf16* part_o = nullptr;
  float* part_lse = nullptr;
  if (p.n_split > 1) {
    part_o = reinterpret_cast<__bf16*>(workspace);
    part_lse = reinterpret_cast<float*>(part_o + (size_t)B * T * p.n_split * Hq * kDv);
  }
  const float sl2 = scale * kLog2e;
  const __bf16* qq = (const __bf16*)q;
  const __bf16* kk = (const __bf16*)kv;
  __bf16* oo = (__bf16*)out;
  switch (p.hgw) {
    case 4: return launch_attn<4>(p, qq, kk, idx, ctx_len, B, T, Hq, Lmax, k, sl2, oo, lse, part_o, part_lse, stream);
    case 2: return launch_attn<2>(p, qq, kk, idx, ctx_len, B, T, Hq, Lmax, k, sl2, oo, lse, part_o, part_lse, stream);
    default: return launch_attn<1>(p, qq, kk, idx, ctx_len, B, T, Hq, Lmax, k, sl2, oo, lse, part_o, part_lse, stream);
  }
}

}  // namespace dsa
