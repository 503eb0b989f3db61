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
// Work split: a workgroup owns one query row, 16*NW heads and one slice of
// the k selected rows (split-KV; a combine kernel merges slices by their
// log-sum-exp; slice outputs are kept in bf16 after normalisation).  Each of
// the NW waves owns 16 heads over all 576 latent dims, one wave per SIMD:
// its query block stays in registers (operand B of S^T = K . q^T, 72 VGPRs)
// and its O^T accumulator [512 x 16] is 128 fp32 per lane (AGPRs).  Rows are
// processed 32 at a time, in a three-stage pipeline: while tile n is
// softmaxed and multiplied into O, the products S^T of tile n+1 run on the
// matrix cores between the softmax's vector instructions, and tile n+2
// streams from HBM into the third buffer.
//   * the 32 selected rows are gathered straight from HBM into LDS with
//     16-byte LDS-DMA loads (buffer_load_dwordx4 ... lds);
//   * the tile is stored row-major with a pitch of 74 16-byte chunks
//     (1184 B) and the chunk index of row r XOR-ed with bit 2 ^ bit 3 of r:
//     the operand reads of S^T (8 or 16 rows per bank cycle) and the
//     transposing reads of O^T (4 or 8 rows of 32 bytes) then hit distinct
//     banks whether the LDS serves 32 or 64 banks per cycle, and every LDS
//     address is one of two per-lane bases plus an immediate;
//   * S^T reads 16-byte row fragments (operand A), lane group g covering
//     latent dims [144 g, 144 g + 144) in 18 steps;
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
constexpr int kPitchChunks = 74;          // LDS row pitch in 16-byte chunks
constexpr int kPitch = kPitchChunks * 16; // 1184
constexpr int kTileLoads = kRows * kPitchChunks / kWave;  // 37 wave-loads per tile
static_assert(kRows * kPitchChunks == kTileLoads * kWave, "a tile is whole wave-loads");
constexpr int kTileBytes = kRows * kPitch;                // 37888
// Longest slice a workgroup takes (its row list and score bias live in LDS;
// each thread keeps its share of the list in registers while the first
// gathers are issued, so fewer waves take shorter slices).  2048 rows let a
// four-wave workgroup take a whole top-2048 set: no split-KV partials and no
// combine when the rows alone fill the GPU (prefill).
__host__ __device__ constexpr int max_split_rows(int nw) { return nw == 4 ? 2048 : 1024; }
constexpr int kOutPitch = 1040;           // LDS pitch of a staged 512-dim bf16 output row
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.f;   // log2 headroom of the lazy softmax rescale
// Word 3 of a raw (untyped, unswizzled) buffer resource on gfx9.
constexpr int kBufferWord3 = 0x00020000;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i32x4 lds_i32x4;

// Chunk swizzle of tile row r: chunk c is stored at position c ^ swz(r).
__device__ __forceinline__ int swz(int r) { return ((r >> 2) ^ (r >> 3)) & 1; }

// Slot of one 16-byte LDS-DMA load inside a tile: instruction i of the tile
// writes slots 64 i .. 64 i + 63; slot p is chunk position p % 74 of row
// p / 74, which holds chunk position ^ swz(row).  The two pad positions of a
// row receive a harmless copy of the row's chunk 0.  Packed as
// (row << 16) | byte offset of the chunk in the source row.
__device__ __forceinline__ int gather_slot(int i, int lane) {
  const int p = i * kWave + lane;
  const int r = p / kPitchChunks;
  int c = (p - r * kPitchChunks) ^ swz(r);
  if (c >= kChunks) c = 0;
  return (r << 16) | (c * 16);
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maximum), as a
// builtin so that the compiler's own wait-count tracking sees it.
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Maximum / sum over the four 16-lane rows of a wave (lanes l, l^16, l^32,
// l^48), with the cross-row lane swaps of the vector ALU.
__device__ __forceinline__ float max_over_rows(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_rows(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Two floats to packed bf16 (round to nearest even, one instruction).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ v4i16 tr_read(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
}

// Merge the split-KV partials of one (query row, head, 8 dims) unit:
// out = sum_i exp(lse_i - lse) * o_i, lse = log sum_i exp(lse_i).  The
// partials are merged 16 splits at a time with all of a chunk's loads in
// flight together (one round trip to memory for up to 16 splits).
constexpr int kCombChunk = 16;
__device__ __forceinline__ void combine_unit(const __bf16* __restrict__ part_o,
                                             const float* __restrict__ part_lse, int Hq,
                                             int n_split, int row, int head, int d,
                                             __bf16* __restrict__ out, float* __restrict__ lse,
                                             bool write_lse) {
  const float* pl = part_lse + (int64_t)row * n_split * Hq + head;
  const __bf16* po = part_o + ((int64_t)row * n_split * Hq + head) * kDv + d;
  float m = -INFINITY, den = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int i0 = 0; i0 < n_split; i0 += kCombChunk) {
    i32x4 v[kCombChunk];
    float li[kCombChunk];
#pragma unroll
    for (int u = 0; u < kCombChunk; ++u) {
      const int i = min(i0 + u, n_split - 1);
      v[u] = ld16(po + (int64_t)i * Hq * kDv);
      li[u] = (i0 + u < n_split) ? pl[(int64_t)i * Hq] : -INFINITY;
    }
    float mc = -INFINITY;
#pragma unroll
    for (int u = 0; u < kCombChunk; ++u) mc = fmaxf(mc, li[u]);
    if (mc == -INFINITY) continue;
    const float mn = fmaxf(m, mc);
    const float a = (m == -INFINITY) ? 0.f : __expf(m - mn);
    den *= a;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= a;
#pragma unroll
    for (int u = 0; u < kCombChunk; ++u) {
      const float w = (li[u] == -INFINITY) ? 0.f : __expf(li[u] - mn);
      den += w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t x = (uint32_t)v[u][e];
        acc[2 * e] += w * __uint_as_float(x << 16);
        acc[2 * e + 1] += w * __uint_as_float(x & 0xFFFF0000u);
      }
    }
    m = mn;
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  i32x4 pk;
#pragma unroll
  for (int e = 0; e < 4; ++e) pk[e] = (int)cvt_pk_bf16(acc[2 * e] * inv, acc[2 * e + 1] * inv);
  *reinterpret_cast<i32x4*>(out + ((int64_t)row * Hq + head) * kDv + d) = pk;
  if (write_lse && lse != nullptr)
    lse[(int64_t)row * Hq + head] = den > 0.f ? m + logf(den) : -INFINITY;
}

// The arguments that the first gathers depend on come first: the first 14
// argument dwords are preloaded into scalar registers at launch (built with
// -amdgpu-kernarg-preload-count=14), so the gathers wait on no argument load.
template <int NW>
__global__ __launch_bounds__(NW * kWave) void sparse_mla_kernel(
    const int32_t* __restrict__ idx, const __bf16* __restrict__ kv, const __bf16* __restrict__ q,
    int T, int k, int rows_per_split, int n_split, int head_groups, int per_xcd, int Lmax, int Hq,
    const int32_t* __restrict__ ctx_len, float scale_log2, __bf16* __restrict__ out,
    float* __restrict__ lse, __bf16* __restrict__ part_o, float* __restrict__ part_lse) {
  constexpr int NT = NW * kWave;
  constexpr int kMaxSplitRows = max_split_rows(NW);
  constexpr int KJ = (kTileLoads + NW - 1) / NW;  // DMA instructions per wave per tile
  // Three tile buffers, as separate LDS objects so that the compiler can tell
  // that reading one buffer does not depend on the DMA still writing another.
  __shared__ __attribute__((aligned(16))) unsigned char tileA[kTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char tileB[kTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char tileC[kTileBytes];
  __shared__ int32_t rows[kMaxSplitRows];
  __shared__ __attribute__((aligned(16))) float bias[kMaxSplitRows];  // 0 or -inf per row

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int g = lane >> 4;
  const int c16 = lane & 15;
  // Work item w = ((row * n_split) + split) * head_groups + head group; the
  // grid holds exactly the work items.  The dispatcher deals consecutive
  // workgroups to the 8 XCDs in turn, so workgroup i runs on XCD i % 8; when
  // the work items split into 8 equal ranges (per_xcd > 0) each XCD takes one
  // contiguous range, which keeps a query row's fragments and the rows its
  // head groups gather together in one XCD's L2 instead of fetching them 8
  // times.
  const int bid = per_xcd > 0 ? (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3)
                              : (int)blockIdx.x;
  const int hgi = bid % head_groups;
  const int rs = bid / head_groups;
  const int split = rs % n_split;
  const int row = rs / n_split;  // b * T + t
  const int b = row / T;
  const int t = row - b * T;
  const int head = (hgi * NW + wave) * 16 + c16;
  const int j0 = split * rows_per_split;
  const int nrows = max(0, min(k, j0 + rows_per_split) - j0);
  const int ntiles = (nrows + kRows - 1) / kRows;

  // This wave's DMA instructions are the same for every tile.  Instruction
  // j is wave + NW j of the tile; a wave with fewer than KJ of its own
  // repeats the tile's last one (the same bytes to the same place), which
  // keeps the issue free of branches.
  auto dma_inst = [&](int j) { return min(wave + NW * j, kTileLoads - 1); };
  int gslot[KJ];
#pragma unroll
  for (int j = 0; j < KJ; ++j) gslot[j] = gather_slot(dma_inst(j), lane);

  // ---- Global loads in the order they are needed: the memory counter
  // completes in order, so waiting for the indices must not wait for the
  // query fragments behind them.  First the selected rows of tiles 0 and 1
  // (lane l loads row l of the slice; the DMA slots take theirs from it by
  // cross-lane reads) and this thread's share of the slice (its LDS copy),
  // then the query fragments.  The slice is read through a buffer resource:
  // every load is unconditional (past the slice it reads zero, which the
  // select turns into -1).  Few load instructions matter here: at the start
  // of the kernel every wave of the CU issues its loads at once, and the
  // address unit takes them one after another.
  static_assert(2 * kRows == kWave, "one lane per row of tiles 0 and 1");
  const __amdgpu_buffer_rsrc_t ir = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(idx + (int64_t)row * k + j0), 0, nrows * 4, kBufferWord3);
  auto sel = [&](int j) {
    const int v = (int)__builtin_amdgcn_raw_buffer_load_b32(ir, j * 4, 0, 0);
    return j < nrows ? v : -1;
  };
  const int first_rows = sel(lane);
  constexpr int kCopy = kMaxSplitRows / NT;
  int rc[kCopy];
#pragma unroll
  for (int u = 0; u < kCopy; ++u) rc[u] = sel(tid + NT * u);
  // Query fragments (nothing depends on them until the first tile): operand
  // B of S^T (column = head, reduction = dims); lane group g covers dims
  // [144 g, 144 g + 144), 8 per step.
  bf16x8 qf[18];
  {
    const __bf16* qp = q + ((int64_t)row * Hq + head) * kDqk + 144 * g;
#pragma unroll
    for (int i = 0; i < 18; ++i) qf[i] = as_bf16x8(ld16(qp + 8 * i));
  }
  // Every load above is issued before anything uses an index (left alone,
  // the compiler starts the first gather's address arithmetic in between, and
  // the rest of the loads then wait for the first index to arrive).
  __builtin_amdgcn_sched_barrier(0);
  int r0[KJ], r1[KJ];
#pragma unroll
  for (int j = 0; j < KJ; ++j) {
    const int rr = gslot[j] >> 16;
    r0[j] = __builtin_amdgcn_ds_bpermute(4 * rr, first_rows);
    r1[j] = __builtin_amdgcn_ds_bpermute(4 * (kRows + rr), first_rows);
  }

  // The DMA goes through a buffer resource over this sequence's latent rows
  // (MUBUF, not FLAT: a FLAT load that writes LDS makes every later LDS wait
  // of the wave a full drain, which would also wait for this DMA).  The whole
  // offset is in the range-checked vector offset, so row -1 (padding, or past
  // the slice) lies past the buffer: its DMA writes zeros and reads nothing.
  const __amdgpu_buffer_rsrc_t kvr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(kv + (int64_t)b * Lmax * kDqk), 0, Lmax * kRowBytes, kBufferWord3);
  auto issue_one = [&](unsigned char* tile, int j, int src) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        kvr, (lds_void*)(tile + dma_inst(j) * kWave * 16), 16,
        (unsigned)src * kRowBytes + (unsigned)(gslot[j] & 0xffff), 0, 0, 0);
  };
  // Tiles 0 and 1 are requested together as soon as the indices arrive (a
  // slice of 64 rows, the common decode case, then waits on a single round
  // trip to HBM).  They do not wait for the context length: a row the query
  // may not see is gathered all the same and masked by its score bias.  (The
  // requests are unconditional: a tile past the slice has only rows -1.)
#pragma unroll
  for (int j = 0; j < KJ; ++j) issue_one(tileA, j, r0[j]);
#pragma unroll
  for (int j = 0; j < KJ; ++j) issue_one(tileB, j, r1[j]);
  // A selected row is used only if it is a real position visible to the
  // query (invalid / padding -> -1, whose score bias is -inf).
  const int ctx = ctx_len[b];
  const int64_t pos = (int64_t)ctx - T + t;
  auto valid = [&](int v) { return (v < 0 || (int64_t)v > pos || v >= Lmax) ? -1 : v; };
  // LDS copy of the slice's rows (for later tiles' DMA) and score bias.
#pragma unroll
  for (int u = 0; u < kCopy; ++u) {
    const int j = tid + NT * u;
    if (j < ntiles * kRows) {
      const int v = valid(rc[u]);
      rows[j] = v;
      bias[j] = v >= 0 ? 0.f : -INFINITY;
    }
  }
  // The fragments must have arrived before the tile loop starts: otherwise
  // the compiler may move these loads below the barrier, and the wait for
  // them then sits at the loop head, where it would also wait for every
  // tile's DMA.
  // They also live in AGPRs (operand B of an MFMA may come from there),
  // leaving the VGPRs to the fragments in flight.
#pragma unroll
  for (int i = 0; i < 18; ++i) asm volatile("" : "+a"(qf[i]));
  f32x4 o[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // Per-lane LDS byte offsets that do not depend on the tile.
  // S^T operand A: row 16 mb + c16, logical chunk 18 g + i at position
  // (18 g + i) ^ x with x = swz(row): +16 x for even i, -16 x for odd.
  const int xq = swz(c16);
  const int qk_even = c16 * kPitch + 288 * g + 16 * xq;
  const int qk_odd = c16 * kPitch + 288 * g - 16 * xq;
  // O^T operand A (transposing reads): source row 4g + (c16 >> 2) (+16),
  // dims 16 mb + 4 (c16 & 3): the two chunks of a 32-byte window swap places
  // where swz(row) = 1, i.e. for lane groups 1 and 2.
  const int tr_base = (4 * g + (c16 >> 2)) * kPitch + ((8 * (c16 & 3)) ^ (16 * swz(4 * g)));

  // S^T operand reads of fragment i of one tile (dims 144 g + 8 i), rows
  // c16 and 16 + c16.
  auto kread = [&](const unsigned char* tile, int i, i32x4& ka, i32x4& kb) {
    const unsigned char* ap = tile + ((i & 1) ? qk_odd : qk_even) + 16 * i;
    ka = *(const lds_i32x4*)ap;
    kb = *(const lds_i32x4*)(ap + 16 * kPitch);
  };
  // Rows of a later tile's DMA slots and the score bias of the next tile are
  // read from LDS one step ahead (past the slice a row is -1: its DMA reads
  // nothing).
  auto lookup_rows = [&](int tbase, int (&src)[KJ]) {
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
      const int r = tbase + (gslot[j] >> 16);
      const int v = rows[min(r, kMaxSplitRows - 1)];
      src[j] = r < nrows ? v : -1;
    }
  };
  auto lookup_bias = [&](int tbase, f32x4& b0, f32x4& b1) {
    const int t0 = min(tbase, kMaxSplitRows - kRows);
    b0 = *reinterpret_cast<const f32x4*>(bias + t0 + 4 * g);
    b1 = *reinterpret_cast<const f32x4*>(bias + t0 + 16 + 4 * g);
  };

  // Scaled scores of the tile about to be exponentiated (lane: rows 4g+r and
  // 16+4g+r), and the reference it is taken against.
  float sv[8];
  float mref = 0.f;
  // First half of the online softmax for one tile: scale, mask, the tile max
  // and the lazy rescale of O.  The reference max m_run only moves when a
  // tile's max exceeds it by more than 2^kLazy; P = 2^(s - m_run) then stays
  // below 2^kLazy, and O, l and the log-sum-exp all use the same reference,
  // so the result is the exact softmax.  The O rescale runs only when some
  // head's reference moves, which is rare after the first tile.
  auto softmax_head = [&](const f32x4& s0, const f32x4& s1, const f32x4& b0, const f32x4& b1,
                          bool real, bool first) {
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sv[r] = fmaf(s0[r], scale_log2, b0[r]);
      sv[4 + r] = fmaf(s1[r], scale_log2, b1[r]);
      mt = fmaxf(mt, fmaxf(sv[r], sv[4 + r]));
    }
    mt = max_over_rows(mt);
    const bool need = real && mt > m_run + kLazy;  // (a stale tile never rescales)
    if (first) {
      m_run = mt;  // O and l are still zero: nothing to rescale
    } else if (__any(need)) {
      const float m_new = need ? mt : m_run;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
      // (O is taken from and returned to AGPRs here, so that it stays in
      // AGPRs on both paths instead of being shadowed in VGPRs every tile)
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        asm volatile("" : "+a"(o[i]));
        o[i] *= alpha;
        asm volatile("" : "+a"(o[i]));
      }
      l_run *= alpha;
      m_run = m_new;
    }
    // m_run is -inf only while every row so far was masked; then every s is
    // -inf and P is 0.
    mref = (m_run == -INFINITY) ? 0.f : m_run;
  };

  int nsrc[KJ];  // rows of the next tile to gather
#pragma unroll
  for (int j = 0; j < KJ; ++j) nsrc[j] = -1;
  f32x4 nb0, nb1;  // score bias of the tile after the one being softmaxed
  if (ntiles > 0) {
    wait_vm_all();
    __syncthreads();
    constexpr int kAhead = 6;
    f32x4 bias0, bias1;
    lookup_bias(0, bias0, bias1);
    lookup_rows(2 * kRows, nsrc);
    i32x4 ka[18], kb[18];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) kread(tileA, i, ka[i], kb[i]);
    __builtin_amdgcn_sched_barrier(0);
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, b0 = a0, b1 = a0;
#pragma unroll
    for (int i = 0; i < 18; ++i) {
      if (i & 1) {
        a1 = mfma16_bf16(as_bf16x8(ka[i]), qf[i], a1);
        b1 = mfma16_bf16(as_bf16x8(kb[i]), qf[i], b1);
      } else {
        a0 = mfma16_bf16(as_bf16x8(ka[i]), qf[i], a0);
        b0 = mfma16_bf16(as_bf16x8(kb[i]), qf[i], b0);
      }
      if (i + kAhead < 18) kread(tileA, i + kAhead, ka[i + kAhead], kb[i + kAhead]);
      __builtin_amdgcn_sched_barrier(0);
    }
    softmax_head(a0 + a1, b0 + b1, bias0, bias1, true, true);
  }

  // One step: P.V of tile n (buffer P) while S^T of tile n+1 (buffer Q,
  // resident) is formed and tile n+2 streams into buffer D, which held tile
  // n-1.  One barrier per step: after it, tile n+1 has landed (every wave
  // waited for its own DMA) and every wave has finished tile n-1, so D may
  // be overwritten.  The body is a single branch-free block whose order is
  // held by scheduling barriers (left alone, the compiler issues each LDS
  // read just before its use and the wave waits on every one): the DMA issue,
  // the next step's LDS lookups and the exponentials of tile n run between
  // the S^T products of tile n+1, whose operand reads are kept 6 fragments
  // ahead, and O^T += V^T . P^T for tile n follows with its transposing
  // reads 6 fragments ahead.  At most ~14 LDS reads are then in flight, so
  // every wait stays within what the 4-bit LDS wait counter can name.  The
  // softmax head of tile n+1 (and its rare O rescale) closes the step.  On
  // the last steps the DMA and S^T touch stale rows and buffers (the buffer
  // resource bounds every offset) and their results are never used.
  // O^T += V^T . P^T for one tile (P: its buffer; sv: its exponentials),
  // with the transposing reads 6 fragments ahead.
  auto pv = [&](const unsigned char* P) {
    constexpr int kAhead = 6;
    i32x4 pb;
    pb[0] = (int)cvt_pk_bf16(sv[0], sv[1]);
    pb[1] = (int)cvt_pk_bf16(sv[2], sv[3]);
    pb[2] = (int)cvt_pk_bf16(sv[4], sv[5]);
    pb[3] = (int)cvt_pk_bf16(sv[6], sv[7]);
    const bf16x8 pbf = as_bf16x8(pb);
    v4i16 va[32], vb[32];
    const unsigned char* vp = P + tr_base;
#pragma unroll
    for (int mb = 0; mb < kAhead; ++mb) {
      va[mb] = tr_read(vp + 32 * mb);
      vb[mb] = tr_read(vp + 32 * mb + 16 * kPitch);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mb = 0; mb < 32; ++mb) {
      const v4i16 pair[2] = {va[mb], vb[mb]};
      o[mb] = mfma16_bf16(__builtin_bit_cast(bf16x8, pair), pbf, o[mb]);
      if (mb + kAhead < 32) {
        va[mb + kAhead] = tr_read(vp + 32 * (mb + kAhead));
        vb[mb + kAhead] = tr_read(vp + 32 * (mb + kAhead) + 16 * kPitch);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto step = [&](int n, const unsigned char* P, const unsigned char* Q, unsigned char* D) {
    constexpr int kAhead = 6;
    wait_vm_all();
    __syncthreads();
    int src[KJ];
#pragma unroll
    for (int j = 0; j < KJ; ++j) src[j] = nsrc[j];
    lookup_rows((n + 3) * kRows, nsrc);
    f32x4 bias0, bias1;
    lookup_bias((n + 1) * kRows, bias0, bias1);
    i32x4 ka[18], kb[18];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) kread(Q, i, ka[i], kb[i]);
    __builtin_amdgcn_sched_barrier(0);
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, b0 = a0, b1 = a0;
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < 18; ++i) {
      if (i & 1) {
        a1 = mfma16_bf16(as_bf16x8(ka[i]), qf[i], a1);
        b1 = mfma16_bf16(as_bf16x8(kb[i]), qf[i], b1);
      } else {
        a0 = mfma16_bf16(as_bf16x8(ka[i]), qf[i], a0);
        b0 = mfma16_bf16(as_bf16x8(kb[i]), qf[i], b0);
      }
      if (i + kAhead < 18) kread(Q, i + kAhead, ka[i + kAhead], kb[i + kAhead]);
      if (i < 8) {
        sv[i] = __builtin_amdgcn_exp2f(sv[i] - mref);
        ls += sv[i];
      }
      if (i < KJ) issue_one(D, i, src[i]);
      __builtin_amdgcn_sched_barrier(0);  // keep this order
    }
#pragma unroll
    for (int j = 18; j < KJ; ++j) issue_one(D, j, src[j]);  // (narrow workgroups)
    l_run += ls;
    pv(P);
    softmax_head(a0 + a1, b0 + b1, bias0, bias1, n + 1 < ntiles, false);
  };

  // The last tile: its exponentials and O^T += V^T . P^T only (there is no
  // next tile to score and nothing more to gather).
  auto last_step = [&](const unsigned char* P) {
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      sv[i] = __builtin_amdgcn_exp2f(sv[i] - mref);
      ls += sv[i];
    }
    l_run += ls;
    pv(P);
  };

  // Every tile but the last takes a full step, unrolled by three so that
  // every buffer role is static; tile n sits in buffer n % 3.
  const int nfull = ntiles - 1;
  for (int n = 0; n < nfull; n += 3) {
    step(n, tileA, tileB, tileC);
    if (n + 1 >= nfull) break;
    step(n + 1, tileB, tileC, tileA);
    if (n + 2 >= nfull) break;
    step(n + 2, tileC, tileA, tileB);
  }
  if (ntiles > 0) {
    const int r = nfull % 3;
    last_step(r == 0 ? tileA : r == 1 ? tileB : tileC);
  }
  wait_vm_all();  // the last steps' DMA may still be writing a tile buffer
  __syncthreads();  // every wave is done with the tiles: they stage the output

  // ---- finish: total row sum over the four lane groups
  const float l_tot = sum_over_rows(l_run);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  const float lse_v = (l_tot > 0.f) ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  // lane holds O^T[dim = 16 mb + 4 g + r][head].  The wave's [16 heads x 512
  // dims] bf16 block is staged in LDS (the tile buffers are free now; rows
  // padded to 1040 bytes, two waves per buffer) and written out as contiguous
  // rows: a normalised partial (split-KV) or the final output.
  static_assert(NW <= 4 && 2 * 16 * kOutPitch <= kTileBytes, "output staging fits two tiles");
  unsigned char* st = (wave < 2 ? tileA : tileB) + (wave & 1) * (16 * kOutPitch);
#pragma unroll
  for (int mb = 0; mb < 32; ++mb) {
    uint2 pk;
    pk.x = cvt_pk_bf16(o[mb][0] * inv, o[mb][1] * inv);
    pk.y = cvt_pk_bf16(o[mb][2] * inv, o[mb][3] * inv);
    *reinterpret_cast<uint2*>(st + c16 * kOutPitch + 32 * mb + 8 * g) = pk;
  }
  __builtin_amdgcn_wave_barrier();
  __bf16* dst = (n_split == 1)
                    ? out + ((int64_t)row * Hq + head - c16) * kDv
                    : part_o + (((int64_t)row * n_split + split) * Hq + head - c16) * kDv;
  // One head row (1 KB) per instruction.  Split partials are streamed past
  // the L2 (the combine reads them once, from another XCD's point of view),
  // so the kernel does not end with megabytes of dirty lines to write back.
  if (n_split == 1) {
#pragma unroll
    for (int hr = 0; hr < 16; ++hr) {
      const i32x4 v = *reinterpret_cast<const i32x4*>(st + hr * kOutPitch + 16 * lane);
      *reinterpret_cast<i32x4*>(dst + (int64_t)hr * kDv + 8 * lane) = v;
    }
  } else {
#pragma unroll
    for (int hr = 0; hr < 16; ++hr) {
      const i32x4 v = *reinterpret_cast<const i32x4*>(st + hr * kOutPitch + 16 * lane);
      __builtin_nontemporal_store(v, reinterpret_cast<i32x4*>(dst + (int64_t)hr * kDv + 8 * lane));
    }
  }
  if (g == 0) {
    if (n_split == 1) {
      if (lse != nullptr) lse[(int64_t)row * Hq + head] = lse_v;
    } else {
      part_lse[((int64_t)row * n_split + split) * Hq + head] = lse_v;
    }
  }
}

// Merge split-KV partials.  One one-wave workgroup per (query row, head)
// (measured against 2 and 4 heads per workgroup: 19.7-19.9 against
// 19.8-20.1 us per layer with the main kernel); a thread owns 8 dims.
constexpr int kCombHeads = 1;
__global__ __launch_bounds__(kCombHeads * 64) void sparse_mla_combine_kernel(
    const __bf16* __restrict__ part_o, const float* __restrict__ part_lse, int Hq, int n_split,
    __bf16* __restrict__ out, float* __restrict__ lse) {
  // (wave-uniform: the 16 per-split log-sum-exps of the wave's head are then
  // scalar loads rather than 16 vector loads per lane of the same address)
  const int head = __builtin_amdgcn_readfirstlane(blockIdx.y * kCombHeads + threadIdx.x / 64);
  if (head >= Hq) return;
  combine_unit(part_o, part_lse, Hq, n_split, blockIdx.x, head, (threadIdx.x & 63) * 8, out,
               lse, (threadIdx.x & 63) == 0);
}

// Split-KV plan: about one workgroup per CU (the LDS tiles allow no more),
// slices of at least 128 rows (shorter ones multiply the partials the combine
// has to read: 32 slices of 64 rows measured 35 us against 23 us for 16 of 128
// at the 128K decode shape).
constexpr int kAttnWgTarget = 256;
constexpr int kAttnMinSplitRows = 128;

struct SplitPlan {
  int nw, head_groups, n_split, rows_per_split;
};

SplitPlan plan_split(int B, int T, int Hq, int k) {
  SplitPlan p;
  const int hb = Hq / 16;
  p.nw = (hb % 4 == 0) ? 4 : (hb % 2 == 0) ? 2 : 1;
  p.head_groups = hb / p.nw;
  const int base = B * T * p.head_groups;
  const int tiles = (k + kRows - 1) / kRows;
  // Enough workgroups to fill the CUs, but every split writes Hq*512 bf16
  // partials (the size of ~450 gathered rows), so keep splits long.
  int ns = (kAttnWgTarget + base - 1) / base;
  ns = min(ns, max(1, tiles / (kAttnMinSplitRows / kRows)));
  ns = max(ns, (k + max_split_rows(p.nw) - 1) / max_split_rows(p.nw));
  ns = max(1, min(ns, tiles));
  const int tiles_per = (tiles + ns - 1) / ns;
  p.rows_per_split = tiles_per * kRows;
  p.n_split = (k + p.rows_per_split - 1) / p.rows_per_split;
  return p;
}

size_t part_bytes(const SplitPlan& p, int B, int T, int Hq) {
  const size_t rows = (size_t)B * T * p.n_split * Hq;
  return (rows * kDv * 2 + rows * sizeof(float) + 255) & ~size_t(255);
}

template <int NW>
hipError_t launch_attn(const SplitPlan& p, const __bf16* q, const __bf16* kv, const int32_t* idx,
                       const int32_t* ctx_len, int B, int T, int Hq, int Lmax, int k, float sl2,
                       __bf16* out, float* lse, __bf16* part_o, float* part_lse,
                       hipStream_t stream) {
  const int n_work = B * T * p.head_groups * p.n_split;
  const int per_xcd = n_work % 8 == 0 ? n_work / 8 : 0;
  hipLaunchKernelGGL((sparse_mla_kernel<NW>), dim3(n_work), dim3(NW * kWave), 0, stream, idx, kv,
                     q, T, k, p.rows_per_split, p.n_split, p.head_groups, per_xcd, Lmax, Hq,
                     ctx_len, sl2, out, lse, part_o, part_lse);
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
  switch (p.nw) {
    case 4: return launch_attn<4>(p, qq, kk, idx, ctx_len, B, T, Hq, Lmax, k, sl2, oo, lse, part_o, part_lse, stream);
    case 2: return launch_attn<2>(p, qq, kk, idx, ctx_len, B, T, Hq, Lmax, k, sl2, oo, lse, part_o, part_lse, stream);
    default: return launch_attn<1>(p, qq, kk, idx, ctx_len, B, T, Hq, Lmax, k, sl2, oo, lse, part_o, part_lse, stream);
  }
}

}  // namespace dsa
