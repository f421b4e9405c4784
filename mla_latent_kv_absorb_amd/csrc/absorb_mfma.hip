// Matrix-core absorb-form MLA attention for the DeepSeek-V3 head shape
// (kv_lora_rank 512, qk_rope_head_dim 64, qk_nope_head_dim 128, v_head_dim 128), bf16 storage,
// fp32 accumulation.
//
// The computation is the absorb path of the page "Naive vs Absorb Attention Implementations in
// DeepSeek-V3" (section "Absorb Path Execution"), run as three kernels:
//   1. absorb_q_kernel       q_lat[row, :] = q_nope[row, :] . W_UK[h]            (query absorption)
//   2. attn_kernel           per (sequence, 128-row block, position split): scores against
//                            kv_cache (512) and pe_cache (64) as one 576-deep contraction, online
//                            softmax, probability-weighted sum over kv_cache in latent space
//   3. merge_upproj_kernel   merge the split partials (rescaled by exp2(m_i - M)), then project
//                            out through W_UV[h]
// Rows are the B*S*H query rows in (b, s, h) order.  Every kv/pe row of a split is read from HBM
// once per 128-row block and shared through LDS by all of the block's heads.
#include "common.h"
#include "launch.h"
#include "mfma_common.h"
#include "../../include/mla_absorb.h"

namespace mla {
namespace {

constexpr int kC = 512;        // kv_lora_rank
constexpr int kR = 64;         // qk_rope_head_dim
constexpr int kDn = 128;       // qk_nope_head_dim
constexpr int kDv = 128;       // v_head_dim
constexpr int kTile = 64;      // cached positions per LDS tile (two 32-position MFMA blocks)
constexpr int kRowsWG = 128;   // query rows per attention workgroup (4 waves x 32)
constexpr int kKvTileBytes = kTile * kC * 2;              // 64 KB
constexpr int kPeTileBytes = kTile * kR * 2;              // 8 KB
constexpr int kStageBytes = kKvTileBytes + kPeTileBytes;  // 72 KB; two stages fill 144 KB of LDS
constexpr float kLog2e = 1.4426950408889634f;

// XOR swizzle of 16-byte chunks inside a tile row (applied within aligned groups of 8 chunks).
// It makes both LDS read patterns conflict-free: the score read, where lanes 0..7 touch rows
// rho(0..7) = {0,1,2,3,8,9,10,11} at one chunk, and the transposing read, where each group of 16
// lanes touches 4 consecutive rows at one 32-byte chunk pair.
__device__ __forceinline__ int tile_swz(int row) { return ((row & 3) << 1) | ((row >> 3) & 1); }
__device__ __forceinline__ int swz_chunk(int chunk, int row) { return (chunk & ~7) | ((chunk & 7) ^ tile_swz(row)); }

// The score MFMA's output row i is fed from tile row rho(i) (bits 2 and 3 swapped).  With that
// order, registers 0..7 of lane l hold positions 8*(l/32) + 0..7 and registers 8..15 hold
// positions 16 + 8*(l/32) + 0..7, which is exactly the B-operand layout the P.V MFMA needs, so the
// probabilities never leave registers.
__device__ __forceinline__ int rho(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

struct AttnArgs {
  const uint16_t *q_lat;   // [rows, 512]
  const uint16_t *q_pe;    // [rows, 64]
  const uint16_t *kv;      // [Bmax, Tmax, 512]
  const uint16_t *pe;      // [Bmax, Tmax, 64]
  float *part_ml;          // [rows, splits, 2]   (max in log2 units, sum)
  uint16_t *part_o;        // [rows, splits, 512] (unnormalised, relative to the max)
  int64_t Tmax;
  int32_t S, H, SH;        // SH = S * H rows per sequence
  int32_t end_pos, splits, split_len, row_blocks;
  float scale_log2;        // softmax_scale * log2(e)
};

// Softmax rows keep a reference maximum m_ref and only move it (rescaling the running sum and the
// 512 accumulators) when a tile's maximum exceeds it by more than kRescale (log2 units), so
// p = exp2(x - m_ref) <= 2^kRescale.  The result is exact in any case: numerator and denominator
// share the same reference.
constexpr float kRescale = 8.f;

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kStageBytes];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, g = lane >> 5;

  int bid = blockIdx.x;
  const int rb = __builtin_amdgcn_readfirstlane(bid % a.row_blocks);
  bid /= a.row_blocks;
  const int split = __builtin_amdgcn_readfirstlane(bid % a.splits);
  const int b = __builtin_amdgcn_readfirstlane(bid / a.splits);

  // this lane's query row (its column of the score tile)
  const int lrow = rb * kRowsWG + wave * 32 + l32;
  const bool row_ok = lrow < a.SH;
  const int s = row_ok ? lrow / a.H : 0;
  const int64_t grow = int64_t(b) * a.SH + lrow;
  const int t_begin = split * a.split_len;
  const int t_split_end = min(t_begin + a.split_len, a.end_pos);
  const int row_end = row_ok ? min(t_split_end, a.end_pos - a.S + s + 1) : t_begin;
  // positions the whole workgroup needs: up to the last visible position of its last row
  // (integer division runs on the vector ALU, so the uniform results are re-scalarised)
  const int last_row = min(a.SH - 1, rb * kRowsWG + kRowsWG - 1);
  const int wg_end = __builtin_amdgcn_readfirstlane(min(t_split_end, a.end_pos - a.S + last_row / a.H + 1));
  const int ntiles = __builtin_amdgcn_readfirstlane(wg_end > t_begin ? (wg_end - t_begin + kTile - 1) / kTile : 0);

  // Absorbed query as the score B operand: lane holds q[row][16 ks + 8 g .. +7].
  u32x4 qf[36];
  {
    const uint16_t *qr = a.q_lat + grow * kC + 8 * g;
    const uint16_t *pr = a.q_pe + grow * kR + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) qf[ks] = row_ok ? *reinterpret_cast<const u32x4 *>(qr + 16 * ks) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[32 + ks] = row_ok ? *reinterpret_cast<const u32x4 *>(pr + 16 * ks) : u32x4{0, 0, 0, 0};
  }

  // DMA geometry.  kv: wave w moves tile rows 16w..16w+15, one 1 KB row per instruction; the
  // lane's 16-byte chunk position is `lane` and it fetches source chunk swz_chunk(lane, row).
  // pe: each instruction moves 8 rows of 128 bytes.  Rows past the last needed position repeat
  // the last one (valid data, masked in the softmax).
  const rsrc_t kvres = make_rsrc(a.kv + int64_t(b) * a.Tmax * kC, uint32_t(a.Tmax) * (kC * 2));
  const rsrc_t peres = make_rsrc(a.pe + int64_t(b) * a.Tmax * kR, uint32_t(a.Tmax) * (kR * 2));
  // the swizzle depends on row bits 0, 1 and 3 only, so row 16w + i uses the pattern of row i
  uint32_t kv_voff[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) kv_voff[i] = uint32_t(swz_chunk(lane, i)) * 16;
  uint32_t pe_voff[2];  // pe rows 8 (2w + i) + lane / 8: bit 3 of the row is i
#pragma unroll
  for (int i = 0; i < 2; ++i) pe_voff[i] = uint32_t((lane & 7) ^ tile_swz(8 * i + (lane >> 3))) * 16;
  auto issue = [&](int j) {
    unsigned char *st = smem + (j & 1) * kStageBytes;
    const int t0 = t_begin + j * kTile;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = min(t0 + wave * 16 + i, wg_end - 1);  // wavefront-uniform
      buf_load16_lds(kvres, st + (wave * 16 + i) * (kC * 2), kv_voff[i], uint32_t(t) * (kC * 2));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = (wave * 2 + i) * 8 + (lane >> 3);
      const int tp = min(t0 + row, wg_end - 1);
      buf_load16_lds(peres, st + kKvTileBytes + (wave * 2 + i) * 1024, pe_voff[i] + uint32_t(tp - t0) * (kR * 2),
                     uint32_t(t0) * (kR * 2));
    }
  };

  f32x16 acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = f32x16{};
  float m_ref = -INFINITY, lsum = 0.f;

  // score A-operand reads: tile row rho(l32), chunk 2 ks + g (swizzled)
  const int arow = rho(l32);
  const int afz = tile_swz(arow);
  uint32_t sc_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) sc_off[i] = uint32_t(arow) * (kC * 2) + uint32_t((2 * i + g) ^ afz) * 16;
  const uint32_t pe_off0 = kKvTileBytes + uint32_t(arow) * (kR * 2);
  // P.V A-operand (transposing) reads: rows 16 ks + 8 g + s16/4 (+4), chunk 4 cb + 2 chalf + (s16&3)/2
  const int s16 = lane & 15, chalf = (lane >> 4) & 1;
  uint32_t tr_off[2][2];  // [cb & 1][ks]
#pragma unroll
  for (int par = 0; par < 2; ++par)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int row0 = 16 * ks + 8 * g + (s16 >> 2);
      const int chunk = 4 * par + 2 * chalf + ((s16 & 3) >> 1);
      tr_off[par][ks] = uint32_t(row0) * (kC * 2) + uint32_t(swz_chunk(chunk, row0)) * 16 + (s16 & 1) * 8;
    }

  if (ntiles > 0) issue(0);

#pragma unroll 1
  for (int j = 0; j < ntiles; ++j) {
    // Only tile j's DMA is outstanding here.  A bare s_barrier follows: a __syncthreads() fence
    // would add nothing, and issuing tile j+1 inside the branch below lets the compiler's own LDS
    // DMA wait before the first LDS read resolve to "all but tile j+1".
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (j + 1 < ntiles) issue(j + 1);

    const unsigned char *st = smem + (j & 1) * kStageBytes;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int t0 = t_begin + j * kTile + 32 * half;
      const uint32_t hb = uint32_t(half) * 32 * (kC * 2);

      // ---- scores S^T[position][row] over the 576-wide concatenation of kv and pe
      f32x16 sacc = f32x16{};
      {
        u32x4 fr[2][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) fr[0][i] = lds_read16(st, hb + sc_off[i]);
#pragma unroll
        for (int grp = 0; grp < 9; ++grp) {
          const int cur = grp & 1;
          if (grp + 1 < 8) {
#pragma unroll
            for (int i = 0; i < 4; ++i) fr[cur ^ 1][i] = lds_read16(st, hb + sc_off[i] + (grp + 1) * 128);
          } else if (grp + 1 == 8) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              fr[cur ^ 1][i] = lds_read16(st, pe_off0 + uint32_t(half) * 32 * (kR * 2) + uint32_t((2 * i + g) ^ afz) * 16);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < 4; ++i) sacc = mfma32(fr[cur][i], qf[4 * grp + i], sacc);
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // ---- online softmax (log2 domain); register r holds position 16*(r/8) + 8*g + r%8
      float x[16];
      float mloc = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = t0 + 16 * (r >> 3) + 8 * g + (r & 7);
        x[r] = (t < row_end) ? sacc[r] * a.scale_log2 : -INFINITY;
        mloc = fmaxf(mloc, x[r]);
      }
      const float mrow = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
      if (m_ref == -INFINITY) {
        m_ref = mrow;  // first visible positions: nothing accumulated yet
      } else if (mrow > m_ref + kRescale) {
        const float alpha = fast_exp2(m_ref - mrow);
        lsum *= alpha;
        m_ref = mrow;
#pragma unroll
        for (int i = 0; i < 16; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][r] = agpr_write(agpr_read(acc[i][r]) * alpha);
      }
      const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
      float psum = 0.f;
      u32x4 pb[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float p[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          p[r] = fast_exp2(x[8 * h + r] - m_use);
          psum += p[r];
        }
        pb[h] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                      pack_bf16x2(p[6], p[7])};
      }
      lsum += psum;

      // ---- O^T[c][row] += KV^T[c][position] . P^T[position][row]
      {
        u32x4 fr[2][2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          fr[0][ks] = lds_read_tr_pair(st, hb + tr_off[0][ks], hb + tr_off[0][ks] + 4 * (kC * 2));
#pragma unroll
        for (int cb = 0; cb < 16; ++cb) {
          const int cur = cb & 1;
          if (cb + 1 < 16) {
            const uint32_t base = hb + uint32_t((cb + 1) >> 1) * 128;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
              fr[cur ^ 1][ks] = lds_read_tr_pair(st, base + tr_off[(cb + 1) & 1][ks],
                                                 base + tr_off[(cb + 1) & 1][ks] + 4 * (kC * 2));
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) acc[cb] = mfma32(fr[cur][ks], pb[ks], acc[cb]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }

  // ---- partial state of this split (max in log2 units, sum, unnormalised o)
  lsum += __shfl_xor(lsum, 32, 64);
  if (row_ok) {
    const int64_t idx = grow * a.splits + split;
    if (g == 0) {
      a.part_ml[2 * idx] = m_ref;
      a.part_ml[2 * idx + 1] = lsum;
    }
    uint16_t *po = a.part_o + idx * kC + 4 * g;
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x2 v{pack_bf16x2(agpr_read(acc[cb][4 * q]), agpr_read(acc[cb][4 * q + 1])),
                      pack_bf16x2(agpr_read(acc[cb][4 * q + 2]), agpr_read(acc[cb][4 * q + 3]))};
        *reinterpret_cast<u32x2 *>(po + 32 * cb + 8 * q) = v;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------------
// q_lat[row, c0 + c] = sum_d q_nope[row, d] * W_UK[h][d][c0 + c] for one head h and 128 columns.
// W_UK is staged in LDS once ([128 d][128 c], 16-byte chunks XOR-swizzled) and read transposed,
// because the contraction runs over d while c is the contiguous index of wkv_b.
struct AbsorbQArgs {
  const uint16_t *q_nope;  // [rows, Dn] with rows = M * H (row = m * H + h)
  const uint16_t *wkv_b;   // [H * 256, 512]
  uint16_t *q_lat;         // [rows, 512]
  int32_t H, M;            // M = B * S query rows per head
  int32_t row_blocks_per_wg;
};

__device__ __forceinline__ int w_swz(int row) { return (row & 3) << 1; }

__global__ void __launch_bounds__(256) absorb_q_kernel(AbsorbQArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char wt[kDn * 128 * 2];  // 32 KB
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, g = lane >> 5;
  const int h = blockIdx.x;
  const int c0 = blockIdx.y * 128;
  const int rb0 = blockIdx.z * a.row_blocks_per_wg;

  // stage W_UK[h][0:128][c0:c0+128]: each wave instruction moves 4 rows of 256 bytes; within it the
  // lane's row is lane / 16 and its chunk position lane % 16 (source chunk swizzled by the row)
  const rsrc_t wres = make_rsrc(a.wkv_b + int64_t(h) * (kDn + kDv) * kC, kDn * kC * 2);
  const uint32_t w_voff = uint32_t(lane >> 4) * (kC * 2) + uint32_t((lane & 15) ^ (((lane >> 4) & 3) << 1)) * 16;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    buf_load16_lds(wres, wt + (wave * 8 + i) * 1024, w_voff, uint32_t((wave * 8 + i) * 4) * (kC * 2) + c0 * 2);
  wait_vmcnt<0>();
  __syncthreads();

  const int s16 = lane & 15, chalf = (lane >> 4) & 1;
  const int nrb = (a.M + 31) / 32;
  for (int rb = rb0; rb < min(nrb, rb0 + a.row_blocks_per_wg); ++rb) {
    const int m = rb * 32 + l32;
    const bool ok = m < a.M;
    const uint16_t *xr = a.q_nope + (int64_t(m) * a.H + h) * kDn + 8 * g;
    f32x16 d = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kDn / 16; ++ks) {
      const u32x4 bf = ok ? *reinterpret_cast<const u32x4 *>(xr + 16 * ks) : u32x4{0, 0, 0, 0};
      const int row0 = 16 * ks + 8 * g + (s16 >> 2);
      const int chunk = 4 * wave + 2 * chalf + ((s16 & 3) >> 1);
      const int within = (s16 & 1) * 8;
      const uint32_t off0 = row0 * 256 + ((chunk & ~7) | ((chunk & 7) ^ w_swz(row0))) * 16 + within;
      const uint32_t off1 = (row0 + 4) * 256 + ((chunk & ~7) | ((chunk & 7) ^ w_swz(row0 + 4))) * 16 + within;
      const u32x4 af = lds_read_tr_pair(wt, off0, off1);
      d = mfma32(af, bf, d);
    }
    // D^T[c][m]: lane holds column m, c = 32 wave + 8 (r/4) + 4 g + r % 4
    if (ok) {
      uint16_t *dst = a.q_lat + (int64_t(m) * a.H + h) * kC + c0 + 32 * wave + 4 * g;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x2 v{pack_bf16x2(d[4 * q], d[4 * q + 1]), pack_bf16x2(d[4 * q + 2], d[4 * q + 3])};
        *reinterpret_cast<u32x2 *>(dst + 8 * q) = v;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------------
// Merge the split partials of 32 rows of one head into o_lat (bf16, LDS), then
// out[row, e] = sum_c o_lat[row, c] * W_UV[h][e][c]; wave w produces e in [32 w, 32 w + 32).
// The merge weights are w_i = exp2(m_i - M) / sum_i exp2(m_i - M) l_i (zero for an empty split).
struct MergeArgs {
  const float *part_ml;
  const uint16_t *part_o;
  const uint16_t *wkv_b;
  uint16_t *out;           // [rows, 128]
  int32_t H, M, splits, row_blocks_per_wg;
};

__global__ void __launch_bounds__(256) merge_upproj_kernel(MergeArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char ol[32 * kC * 2];  // 32 KB
  __shared__ float row_max[32], row_inv[32];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, g = lane >> 5;
  const int h = blockIdx.x;
  const int rb0 = blockIdx.y * a.row_blocks_per_wg;
  const int nrb = (a.M + 31) / 32;

  // W_UV[h] rows e = 32 wave + l32 as the B operand: lane holds W[e][16 ks + 8 g .. +7]
  u32x4 wf[32];
  {
    const rsrc_t wres = make_rsrc(a.wkv_b + (int64_t(h) * (kDn + kDv) + kDn) * kC, kDv * kC * 2);
    const uint32_t voff = uint32_t(32 * wave + l32) * (kC * 2) + 16 * g;
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) wf[ks] = buf_load16(wres, voff, ks * 32);
  }

  const int ch = threadIdx.x & 63;  // 16-byte chunk of the latent this thread merges
  const int r0 = threadIdx.x >> 6;  // rows r0, r0 + 4, ..., r0 + 28
  const int64_t stride_row = int64_t(a.H) * a.splits;  // partial rows between consecutive m
  for (int rb = rb0; rb < min(nrb, rb0 + a.row_blocks_per_wg); ++rb) {
    // ---- per-row maximum and 1 / denominator (8 threads per row share the splits)
    {
      const int r = threadIdx.x >> 3, q = threadIdx.x & 7;
      const int m = rb * 32 + r;
      const float *ml = a.part_ml + 2 * ((int64_t(m) * a.H + h) * a.splits);
      float mx = -INFINITY;
      if (m < a.M)
        for (int i = q; i < a.splits; i += 8) mx = fmaxf(mx, ml[2 * i]);
      mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 4, 64));
      float den = 0.f;
      if (m < a.M)
        for (int i = q; i < a.splits; i += 8) {
          const float mi = ml[2 * i];
          if (mi != -INFINITY) den += fast_exp2(mi - mx) * ml[2 * i + 1];
        }
      den += __shfl_xor(den, 1, 64);
      den += __shfl_xor(den, 2, 64);
      den += __shfl_xor(den, 4, 64);
      if (q == 0) {
        row_max[r] = mx;
        row_inv[r] = (m < a.M && den > 0.f) ? 1.f / den : 0.f;
      }
    }
    __syncthreads();
    // ---- o_lat[row][chunk] = sum_i w_i o_i[row][chunk]; the 8 rows of a thread load in parallel
    {
      float acc[8][8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[k][e] = 0.f;
      float mx[8], inv[8];
      uint32_t base[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = r0 + 4 * k;
        const int m = min(rb * 32 + r, a.M - 1);
        mx[k] = row_max[r];
        inv[k] = row_inv[r];
        base[k] = uint32_t((int64_t(m) * a.H + h) * a.splits) * (kC * 2) + ch * 16;
      }
      const rsrc_t pres = make_rsrc(a.part_o, 0xffffffffu);
      const float *mlb = a.part_ml;
      for (int i = 0; i < a.splits; ++i) {
        u32x4 v[8];
        float wgt[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          v[k] = buf_load16(pres, base[k], uint32_t(i) * (kC * 2));
          const int m = min(rb * 32 + r0 + 4 * k, a.M - 1);
          const float mi = mlb[2 * ((int64_t(m) * a.H + h) * a.splits + i)];
          wgt[k] = (mi == -INFINITY) ? 0.f : fast_exp2(mi - mx[k]) * inv[k];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[k][2 * e] = fmaf(wgt[k], __uint_as_float(v[k][e] << 16), acc[k][2 * e]);
            acc[k][2 * e + 1] = fmaf(wgt[k], __uint_as_float(v[k][e] & 0xffff0000u), acc[k][2 * e + 1]);
          }
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = r0 + 4 * k;
        const u32x4 pk{pack_bf16x2(acc[k][0], acc[k][1]), pack_bf16x2(acc[k][2], acc[k][3]),
                       pack_bf16x2(acc[k][4], acc[k][5]), pack_bf16x2(acc[k][6], acc[k][7])};
        const int pos = (ch & ~7) | ((ch & 7) ^ (r & 7));
        lds_write16(ol, uint32_t(r) * (kC * 2) + pos * 16, pk);
      }
    }
    __syncthreads();
    f32x16 d = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) {
      const int q = 2 * ks + g;
      const u32x4 af = lds_read16(ol, l32 * (kC * 2) + ((q & ~7) | ((q & 7) ^ (l32 & 7))) * 16);
      d = mfma32(af, wf[ks], d);
    }
    // D[row][e]: lane holds e = 32 wave + l32, rows 8 (r/4) + 4 g + r % 4
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int mm = rb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
      if (mm < a.M) a.out[(int64_t(mm) * a.H + h) * kDv + 32 * wave + l32] = f32_to_bf16(d[r]);
    }
    __syncthreads();  // row_max / row_inv / ol are rewritten by the next row block
  }
  (void)stride_row;
}

}  // namespace

bool mfma_attn_supported(const AttnCall &c, const char **why) {
  if (c.dtype != MLA_DTYPE_BF16) { *why = "needs bf16"; return false; }
  if (c.C != kC || c.R != kR || c.Dn != kDn || c.Dv != kDv) {
    *why = "needs kv_lora_rank 512, qk_rope_head_dim 64, qk_nope_head_dim 128, v_head_dim 128";
    return false;
  }
  // per-sequence buffer ranges are byte counts below 2^32
  if (c.Tmax >= (int64_t(1) << 22)) { *why = "cache_len must be below 4194304"; return false; }
  if (c.B * c.S * c.H * int64_t(kC) * 2 >= (int64_t(1) << 32)) { *why = "too many query rows"; return false; }
  return true;
}

int32_t mfma_attn_splits(const AttnCall &c, int num_cus) {
  // Aim for one workgroup per compute unit; never split below 128 positions per range.
  const int64_t row_blocks = (c.S * c.H + kRowsWG - 1) / kRowsWG;
  const int64_t units = c.B * row_blocks;
  int64_t splits = (num_cus + units / 2) / units;
  const int64_t max_by_len = (c.end_pos + 127) / 128;
  if (splits > max_by_len) splits = max_by_len;
  if (splits < 1) splits = 1;
  if (splits > 4096) splits = 4096;
  return int32_t(splits);
}

bool mfma_attn_plan_ok(const AttnCall &c, const char **why) {
  // split partials are addressed with 32-bit byte offsets
  if (c.B * c.S * c.H * int64_t(c.splits) * kC * 2 >= (int64_t(1) << 32)) {
    *why = "batch * seqlen_q * n_heads * num_splits too large for the split partials";
    return false;
  }
  return true;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t mfma_attn_workspace(const AttnCall &c) {
  const size_t rows = size_t(c.B * c.S * c.H);
  return align256(rows * kC * 2) + align256(rows * size_t(c.splits) * 2 * 4) + align256(rows * size_t(c.splits) * kC * 2);
}

hipError_t mfma_absorb_attn(const AttnCall &c) {
  const int64_t rows = c.B * c.S * c.H;
  unsigned char *ws = static_cast<unsigned char *>(c.ws);
  uint16_t *q_lat = reinterpret_cast<uint16_t *>(ws);
  float *part_ml = reinterpret_cast<float *>(ws + align256(size_t(rows) * kC * 2));
  uint16_t *part_o = reinterpret_cast<uint16_t *>(ws + align256(size_t(rows) * kC * 2) +
                                                  align256(size_t(rows) * c.splits * 2 * 4));
  const int32_t M = int32_t(c.B * c.S);

  AbsorbQArgs qa{static_cast<const uint16_t *>(c.q_nope), static_cast<const uint16_t *>(c.wkv_b), q_lat, int32_t(c.H), M, 4};
  const int nrb = (M + 31) / 32;
  timing_begin(MLA_KERNEL_ABSORB_Q, c.stream);
  absorb_q_kernel<<<dim3(unsigned(c.H), kC / 128, unsigned((nrb + qa.row_blocks_per_wg - 1) / qa.row_blocks_per_wg)), 256,
                    0, c.stream>>>(qa);
  timing_end(MLA_KERNEL_ABSORB_Q, c.stream);

  AttnArgs aa{};
  aa.q_lat = q_lat;
  aa.q_pe = static_cast<const uint16_t *>(c.q_pe);
  aa.kv = static_cast<const uint16_t *>(c.kv);
  aa.pe = static_cast<const uint16_t *>(c.pe);
  aa.part_ml = part_ml;
  aa.part_o = part_o;
  aa.Tmax = c.Tmax;
  aa.S = int32_t(c.S);
  aa.H = int32_t(c.H);
  aa.SH = int32_t(c.S * c.H);
  aa.end_pos = int32_t(c.end_pos);
  aa.splits = c.splits;
  aa.split_len = int32_t(c.split_len);
  aa.row_blocks = int32_t((c.S * c.H + kRowsWG - 1) / kRowsWG);
  aa.scale_log2 = c.scale * kLog2e;
  const int64_t nwg = c.B * int64_t(aa.splits) * aa.row_blocks;
  timing_begin(MLA_KERNEL_ATTN, c.stream);
  attn_kernel<<<dim3(unsigned(nwg)), 256, 0, c.stream>>>(aa);
  timing_end(MLA_KERNEL_ATTN, c.stream);

  MergeArgs ma{part_ml, part_o, static_cast<const uint16_t *>(c.wkv_b), static_cast<uint16_t *>(c.out), int32_t(c.H), M,
               c.splits, 8};
  timing_begin(MLA_KERNEL_MERGE_UPPROJ, c.stream);
  merge_upproj_kernel<<<dim3(unsigned(c.H), unsigned((nrb + ma.row_blocks_per_wg - 1) / ma.row_blocks_per_wg)), 256, 0,
                        c.stream>>>(ma);
  timing_end(MLA_KERNEL_MERGE_UPPROJ, c.stream);
  return hipGetLastError();
}

}  // namespace mla
