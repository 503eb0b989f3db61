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
// Work split: a workgroup owns one query row, WAVES*16 heads and one slice of
// the k selected rows (split-KV; a combine kernel merges the slices by their
// log-sum-exp).  Each wave owns 16 heads: its query block stays in registers
// (72 VGPRs) and its O^T accumulator [512 x 16] is 128 fp32 per lane.  Rows
// are processed 32 at a time; the workgroup gathers the 32 rows into LDS in
// two layouts:
//   Ks [32][576]  row-major        -> operand A of S^T = Ks . q^T
//   Vt [512][32]  dim-major        -> operand A of O^T += Vt . P^T
// Vt is produced with an in-register 8x8 transpose of the gathered 16-byte
// pieces.  The 32 rows are stored in Vt in the order kappa that matches where
// the S^T accumulator leaves them (lane group g holds rows 4g..4g+3 and
// 16+4g..16+4g+3), so P^T feeds the second product without any shuffle.
#include "device_common.hpp"
#include "launchers.hpp"

namespace dsa {
namespace {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kRows = 32;                 // rows per tile
constexpr int kKsPitch = kDqk + 8;        // bf16 elements (1168 B: spreads LDS banks)
constexpr int kVtPitch = kRows + 8;       // bf16 elements (80 B)
constexpr int kChunks = kDqk / 8;         // 16-byte pieces per row (72)
constexpr int kVChunks = kDv / 8;         // 64
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int WAVES>
struct AttnSmem {
  __bf16 ks[kRows * kKsPitch];
  __bf16 vt[kDv * kVtPitch];
  int32_t rowidx[kRows];
};

// Row r of a tile sits at position kappa(r) in Vt.
__device__ __forceinline__ int tile_row_of(int q, int j) {  // kappa = 8q + j -> row
  return (j < 4) ? (4 * q + j) : (16 + 4 * q + (j - 4));
}

template <int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void sparse_mla_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ kv, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ ctx_len, int T, int Hq, int Lmax, int k, int rows_per_split,
    float scale_log2, __bf16* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_lse, int n_split) {
  constexpr int NT = WAVES * kWave;
  __shared__ AttnSmem<WAVES> sm;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const int row = blockIdx.x;  // b * T + t
  const int b = row / T;
  const int t = row - b * T;
  const int head = blockIdx.y * (WAVES * 16) + wave * 16 + c16;
  const int split = blockIdx.z;
  const int64_t pos = (int64_t)ctx_len[b] - T + t;
  const int j0 = split * rows_per_split;
  const int j1 = min(k, j0 + rows_per_split);

  // Query fragments: operand B of S^T (column = head, reduction = dims).
  // Lane group g covers dims [144 g, 144 g + 144).
  bf16x8 qf[18];
  {
    const __bf16* qp = q + ((int64_t)row * Hq + head) * kDqk + 144 * g;
#pragma unroll
    for (int i = 0; i < 18; ++i) qf[i] = as_bf16x8(ld16(qp + 8 * i));
  }
  f32x4 o[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const __bf16* kvb = kv + (int64_t)b * Lmax * kDqk;
  const int32_t* ib = idx + (int64_t)row * k;

  for (int r0 = j0; r0 < j1; r0 += kRows) {
    // ---- gather 32 rows into LDS
    if (tid < kRows) {
      const int j = r0 + tid;
      int v = (j < j1) ? ib[j] : -1;
      if (v < 0 || (int64_t)v > pos || v >= Lmax) v = -1;
      sm.rowidx[tid] = v;
    }
    __syncthreads();
    for (int task = tid; task < 4 * kChunks; task += NT) {
      const int qg = task / kChunks;   // kappa group: rows 4qg..4qg+3, 16+4qg..16+4qg+3
      const int c = task - qg * kChunks;
      i32x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = tile_row_of(qg, j);
        const int src = max(sm.rowidx[r], 0);
        v[j] = ld16(kvb + (int64_t)src * kDqk + 8 * c);
        *reinterpret_cast<i32x4*>(&sm.ks[r * kKsPitch + 8 * c]) = v[j];
      }
      if (c < kVChunks) {
        // 8 rows x 8 dims -> 8 dims x 8 rows (kappa order) by byte permutes
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          const uint32_t sel = (d & 1) ? 0x07060302u : 0x05040100u;
          i32x4 tv;
#pragma unroll
          for (int p = 0; p < 4; ++p)
            tv[p] = (int)__builtin_amdgcn_perm((uint32_t)v[2 * p + 1][d >> 1],
                                               (uint32_t)v[2 * p][d >> 1], sel);
          *reinterpret_cast<i32x4*>(&sm.vt[(8 * c + d) * kVtPitch + 8 * qg]) = tv;
        }
      }
    }
    __syncthreads();

    // ---- S^T tile [32 rows x 16 heads] = Ks . q^T
    f32x4 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const __bf16* ap = &sm.ks[(16 * mb + c16) * kKsPitch + 144 * g];
#pragma unroll
      for (int i = 0; i < 18; ++i) acc = mfma16_bf16(as_bf16x8(ld16(ap + 8 * i)), qf[i], acc);
      s[mb] = acc;
    }
    // ---- online softmax (log2 domain); lane holds rows 4g+r and 16+4g+r
    float mt = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool valid = sm.rowidx[16 * mb + 4 * g + r] >= 0;
        s[mb][r] = valid ? s[mb][r] * scale_log2 : -INFINITY;
        mt = fmaxf(mt, s[mb][r]);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 16, kWave));
    mt = fmaxf(mt, __shfl_xor(mt, 32, kWave));
    const float m_new = fmaxf(m_run, mt);
    float alpha = 1.f;
    float p[2][4];
    if (m_new == -INFINITY) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) p[mb][r] = 0.f;
    } else {
      alpha = exp2f(m_run - m_new);
      float ls = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[mb][r] = exp2f(s[mb][r] - m_new);
          ls += p[mb][r];
        }
      l_run = l_run * alpha + ls;
      m_run = m_new;
    }
    if (alpha != 1.f) {
#pragma unroll
      for (int i = 0; i < 32; ++i) o[i] *= alpha;
    }
    // P^T operand: kappa = 8g + j  <->  rows 4g+j (j<4), 16+4g+j-4 (j>=4)
    i32x4 pb;
    pb[0] = (int)pack_bf16x2(p[0][0], p[0][1]);
    pb[1] = (int)pack_bf16x2(p[0][2], p[0][3]);
    pb[2] = (int)pack_bf16x2(p[1][0], p[1][1]);
    pb[3] = (int)pack_bf16x2(p[1][2], p[1][3]);
    const bf16x8 pbf = as_bf16x8(pb);
    // ---- O^T [512 x 16] += Vt . P^T
    const __bf16* vp = &sm.vt[c16 * kVtPitch + 8 * g];
#pragma unroll
    for (int mb = 0; mb < 32; ++mb)
      o[mb] = mfma16_bf16(as_bf16x8(ld16(vp + 16 * mb * kVtPitch)), pbf, o[mb]);
    __syncthreads();  // LDS tile is rewritten by the next iteration
  }

  // ---- finish: total row sum over the four lane groups
  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16, kWave);
  l_tot += __shfl_xor(l_tot, 32, kWave);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  const float lse_v = (l_tot > 0.f) ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  // lane holds O^T[dim = 16 mb + 4 g + r][head]
  if (n_split == 1) {
    __bf16* op = out + ((int64_t)row * Hq + head) * kDv + 4 * g;
#pragma unroll
    for (int mb = 0; mb < 32; ++mb) {
      uint2 pk;
      pk.x = pack_bf16x2(o[mb][0] * inv, o[mb][1] * inv);
      pk.y = pack_bf16x2(o[mb][2] * inv, o[mb][3] * inv);
      *reinterpret_cast<uint2*>(op + 16 * mb) = pk;
    }
    if (lse != nullptr && g == 0) lse[(int64_t)row * Hq + head] = lse_v;
  } else {
    float* pp = part_o + (((int64_t)row * n_split + split) * Hq + head) * kDv + 4 * g;
#pragma unroll
    for (int mb = 0; mb < 32; ++mb)
      *reinterpret_cast<f32x4*>(pp + 16 * mb) = o[mb] * inv;
    if (g == 0) part_lse[((int64_t)row * n_split + split) * Hq + head] = lse_v;
  }
}

// Merge split-KV partials: out = sum_i exp(lse_i - lse) * o_i, lse = log sum exp(lse_i).
__global__ __launch_bounds__(128) void sparse_mla_combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, int Hq, int n_split,
    __bf16* __restrict__ out, float* __restrict__ lse) {
  const int row = blockIdx.x;
  const int head = blockIdx.y;
  const int d = threadIdx.x * 4;
  const float* pl = part_lse + (int64_t)row * n_split * Hq + head;
  float mx = -INFINITY;
  for (int i = 0; i < n_split; ++i) mx = fmaxf(mx, pl[(int64_t)i * Hq]);
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (mx != -INFINITY) {
    for (int i = 0; i < n_split; ++i) {
      const float li = pl[(int64_t)i * Hq];
      const float wi = (li == -INFINITY) ? 0.f : expf(li - mx);
      den += wi;
      const float4 v = *reinterpret_cast<const float4*>(
          part_o + (((int64_t)row * n_split + i) * Hq + head) * kDv + d);
      acc.x += wi * v.x; acc.y += wi * v.y; acc.z += wi * v.z; acc.w += wi * v.w;
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  uint2 pk;
  pk.x = pack_bf16x2(acc.x * inv, acc.y * inv);
  pk.y = pack_bf16x2(acc.z * inv, acc.w * inv);
  *reinterpret_cast<uint2*>(out + ((int64_t)row * Hq + head) * kDv + d) = pk;
  if (lse != nullptr && threadIdx.x == 0)
    lse[(int64_t)row * Hq + head] = den > 0.f ? mx + logf(den) : -INFINITY;
}

struct SplitPlan {
  int waves, head_groups, n_split, rows_per_split;
};

SplitPlan plan_split(int B, int T, int Hq, int k) {
  SplitPlan p;
  const int hb = Hq / 16;
  p.waves = (hb % 4 == 0) ? 4 : (hb % 2 == 0) ? 2 : 1;
  p.head_groups = hb / p.waves;
  const int base = B * T * p.head_groups;
  // Enough workgroups to cover the 256 CUs twice, but keep >= 256 rows per
  // split: every split writes Hq*512 fp32 partials (the size of ~230 rows).
  const int tiles = (k + kRows - 1) / kRows;
  int ns = (512 + base - 1) / base;
  ns = max(1, min(ns, tiles / 8));
  ns = max(1, min(ns, 32));
  const int tiles_per = (tiles + ns - 1) / ns;
  p.rows_per_split = tiles_per * kRows;
  p.n_split = (k + p.rows_per_split - 1) / p.rows_per_split;
  return p;
}

}  // namespace

size_t sparse_attn_workspace_bytes(int B, int T, int Hq, int k, int d_v) {
  const SplitPlan p = plan_split(B, T, Hq, k);
  if (p.n_split <= 1) return 0;
  const size_t rows = (size_t)B * T * p.n_split * Hq;
  return rows * (size_t)d_v * sizeof(float) + rows * sizeof(float) + 256;
}

hipError_t launch_sparse_attn(const void* q, const void* kv, const int32_t* idx,
                              const int32_t* ctx_len, int B, int T, int Hq, int Lmax, int k,
                              float scale, void* out, float* lse, void* workspace,
                              size_t ws_bytes, hipStream_t stream) {
  const SplitPlan p = plan_split(B, T, Hq, k);
  float* part_o = nullptr;
  float* part_lse = nullptr;
  if (p.n_split > 1) {
    part_o = reinterpret_cast<float*>(workspace);
    part_lse = part_o + (size_t)B * T * p.n_split * Hq * kDv;
  }
  const dim3 grid(B * T, p.head_groups, p.n_split);
  const float sl2 = scale * kLog2e;
  const __bf16* qq = (const __bf16*)q;
  const __bf16* kk = (const __bf16*)kv;
  __bf16* oo = (__bf16*)out;
  switch (p.waves) {
    case 4:
      hipLaunchKernelGGL(sparse_mla_kernel<4>, grid, dim3(4 * kWave), 0, stream, qq, kk, idx,
                         ctx_len, T, Hq, Lmax, k, p.rows_per_split, sl2, oo, lse, part_o,
                         part_lse, p.n_split);
      break;
    case 2:
      hipLaunchKernelGGL(sparse_mla_kernel<2>, grid, dim3(2 * kWave), 0, stream, qq, kk, idx,
                         ctx_len, T, Hq, Lmax, k, p.rows_per_split, sl2, oo, lse, part_o,
                         part_lse, p.n_split);
      break;
    default:
      hipLaunchKernelGGL(sparse_mla_kernel<1>, grid, dim3(kWave), 0, stream, qq, kk, idx,
                         ctx_len, T, Hq, Lmax, k, p.rows_per_split, sl2, oo, lse, part_o,
                         part_lse, p.n_split);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_split <= 1) return e;
  hipLaunchKernelGGL(sparse_mla_combine_kernel, dim3(B * T, Hq), dim3(kDv / 4), 0, stream,
                     part_o, part_lse, Hq, p.n_split, oo, lse);
  return hipGetLastError();
}

}  // namespace dsa
