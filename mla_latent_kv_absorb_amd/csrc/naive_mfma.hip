// Matrix-core attention of the naive route (page "Naive vs Absorb Attention Implementations in
// DeepSeek-V3", section "Naive Path Execution") over keys and values that are already expanded:
//
//   score[b,s,h,t] = (q_nope[b,s,h,:] . k_nope[h,b,t,:] + q_pe[b,s,h,:] . pe[b,t,:]) * scale
//   out[b,s,h,:]   = sum_t softmax_t(score) * v[h,b,t,:]
//
// k_nope and v are head-major [H, Bmax, Tmax, 128] (what "Latent KV expansion with split" writes
// for the caches' rows in (b, t) order); the rope key pe[b,t,:] is shared by every head.  The
// mask and the softmax are those of the absorb path (query s at position end_pos - S + s sees
// t <= that position).  DeepSeek-V3 head shape only: qk_nope_head_dim 128, qk_rope_head_dim 64,
// v_head_dim 128; bf16 storage, fp32 accumulation.
//
// One workgroup per (sequence, head, 128 query tokens): four waves of 32 query rows.  Tiles of 32
// positions (8 KB of k_nope, 4 KB of pe, 8 KB of v) stream into LDS by DMA, four stages, taken in
// pairs: per pair one barrier, and per tile a wave runs 12 score MFMAs (a 192-deep contraction)
// and 8 MFMAs of the value sum, with one online-softmax update (log2 domain) per pair.
#include "common.h"
#include "launch.h"
#include "mfma_common.h"
#include "../../include/mla_absorb.h"

namespace mla {
namespace {

constexpr int kDn = 128, kR = 64, kDv = 128;
constexpr int kTile = 32;
constexpr int kStages = 4;
constexpr int kRowsWG = 128;
constexpr int kKBytes = kTile * kDn * 2;   // 8 KB
constexpr int kPeBytes = kTile * kR * 2;   // 4 KB
constexpr int kVBytes = kTile * kDv * 2;   // 8 KB
constexpr int kPeOff = kKBytes;
constexpr int kVOff = kKBytes + kPeBytes;
constexpr int kStageBytes = kKBytes + kPeBytes + kVBytes;  // 20 KB
constexpr float kRescale = 8.f;  // lazy rescale threshold (log2 units), as in the absorb kernel

// LDS swizzles (16-byte chunks XOR-ed by a function of the row):
//  k_nope rows (256 B) are read 16 rows x one chunk at a time (score operand): chunk ^ (row & 15);
//  pe rows (128 B) likewise, two rows per 256 B: chunk ^ ((row >> 1) & 7);
//  v rows (256 B) are read transposed, 4 rows x 4 chunks per 32 lanes: chunk ^ ((row & 3) << 2).
__device__ __forceinline__ int k_swz(int row) { return row & 15; }
__device__ __forceinline__ int pe_swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int v_swz(int row) { return (row & 3) << 2; }
// score output row i comes from tile row rho(i) (bits 2 and 3 swapped), which leaves the
// probabilities in the register layout of the value-sum operand (see the absorb kernel)
__device__ __forceinline__ int rho(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

struct NaiveArgs {
  const uint16_t *q_nope;  // [B, S, H, 128]
  const uint16_t *q_pe;    // [B, S, H, 64]
  const uint16_t *k_nope;  // [H, Bmax, Tmax, 128]
  const uint16_t *v;       // [H, Bmax, Tmax, 128]
  const uint16_t *pe;      // [Bmax, Tmax, 64]
  uint16_t *out;           // [B, S, H, 128]
  int64_t Bmax, Tmax;
  int32_t B, S, H, end_pos, row_blocks;
  float scale_log2;        // softmax_scale * log2(e)
};

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
naive_attn_kernel(NaiveArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kStages * kStageBytes];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, g = lane >> 5;

  // logical order: query block fastest, then head, then sequence (blocks of one head read the
  // same keys and values and land on one XCD)
  int bid = __builtin_amdgcn_readfirstlane(xcd_logical_id(blockIdx.x, gridDim.x));
  const int rb = __builtin_amdgcn_readfirstlane(bid % a.row_blocks);
  bid /= a.row_blocks;
  const int h = __builtin_amdgcn_readfirstlane(bid % a.H);
  const int b = __builtin_amdgcn_readfirstlane(bid / a.H);

  const int s = rb * kRowsWG + wave * 32 + l32;  // this lane's query token
  const bool row_ok = s < a.S;
  const int first_s = rb * kRowsWG, last_s = min(a.S - 1, first_s + kRowsWG - 1);
  const int row_end = row_ok ? a.end_pos - a.S + s + 1 : 0;                         // positions visible to s
  const int wg_end = __builtin_amdgcn_readfirstlane(a.end_pos - a.S + last_s + 1);  // >= 1
  const int wg_full = __builtin_amdgcn_readfirstlane(a.end_pos - a.S + first_s + 1);
  const int ntiles = __builtin_amdgcn_readfirstlane((wg_end + kTile - 1) / kTile);
  // tiles go in pairs (one barrier per 64 positions); an odd count ends with a tile past the
  // visible positions, which reads clamped rows and is masked whole
  const int npairs = (ntiles + 1) / 2;

  // ---- DMA: one instruction moves 1 KB; rows past the last needed position repeat it
  const int64_t kv_row0 = (int64_t(h) * a.Bmax + b) * a.Tmax;
  const rsrc_t kres = make_rsrc(a.k_nope + kv_row0 * kDn, uint32_t(a.Tmax) * (kDn * 2));
  const rsrc_t vres = make_rsrc(a.v + kv_row0 * kDv, uint32_t(a.Tmax) * (kDv * 2));
  const rsrc_t peres = make_rsrc(a.pe + int64_t(b) * a.Tmax * kR, uint32_t(a.Tmax) * (kR * 2));
  const uint32_t smem_lds = lds_addr(smem);
  // one of the five DMA instructions of tile j of this wave: parts 0 and 1 are k_nope rows
  // 4 (2 wave + part) .. +3, parts 2 and 3 the same v rows, part 4 the pe rows 8 wave .. +7
  auto issue_part = [&](int j, const int part) __attribute__((always_inline)) {
    const uint32_t st = smem_lds + uint32_t(j % kStages) * kStageBytes;
    const int t0 = j * kTile;
    if (part < 4) {
      const int i = part & 1;
      const int row = 4 * (2 * wave + i) + (lane >> 4);
      const int t = min(t0 + row, wg_end - 1);
      if (part < 2) {
        const uint32_t kchunk = uint32_t((lane & 15) ^ k_swz(row));
        buf_load16_lds_at(kres, st + (2 * wave + i) * 1024, uint32_t(t) * (kDn * 2) + kchunk * 16, 0);
      } else {
        const uint32_t vchunk = uint32_t((lane & 15) ^ v_swz(row));
        buf_load16_lds_at(vres, st + kVOff + (2 * wave + i) * 1024, uint32_t(t) * (kDv * 2) + vchunk * 16, 0);
      }
    } else {
      const int prow = 8 * wave + (lane >> 3);
      const int tp = min(t0 + prow, wg_end - 1);
      buf_load16_lds_at(peres, st + kPeOff + wave * 1024, uint32_t(tp) * (kR * 2) + uint32_t((lane & 7) ^ pe_swz(prow)) * 16, 0);
    }
  };
  auto issue = [&](int j) __attribute__((always_inline)) {
#pragma unroll
    for (int part = 0; part < 5; ++part) issue_part(j, part);
  };

  // ---- prologue: tiles 0 and 1, the query as score operand (row s: 16 bytes at 16 ks + 8 g), a
  // full wait (the query loads are the only compiler-tracked vector loads), then tiles 2 and 3
  issue(0);
  u32x4 qf[12];
  {
    // descriptors over this (sequence, head)'s query rows (uniform); the row goes into the
    // per-lane offset, and rows past S fall outside the range and read zeros
    const int64_t base = int64_t(b) * a.S * a.H + h;
    const rsrc_t qn = make_rsrc(a.q_nope + base * kDn, uint32_t(a.S) * a.H * (kDn * 2));
    const rsrc_t qp = make_rsrc(a.q_pe + base * kR, uint32_t(a.S) * a.H * (kR * 2));
    const uint32_t srow = uint32_t(s) * uint32_t(a.H);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = buf_load16(qn, srow * (kDn * 2) + uint32_t(16 * ks + 8 * g) * 2, 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[8 + ks] = buf_load16(qp, srow * (kR * 2) + uint32_t(16 * ks + 8 * g) * 2, 0);
  }
  issue(1);
  wait_vmcnt<0>();

  // score operand reads: tile row rho(l32), chunk 2 ks + g (k_nope) / 2 (ks - 8) + g (pe)
  const int arow = rho(l32);
  uint32_t k_off[8], p_off[4];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) k_off[ks] = uint32_t(arow) * (kDn * 2) + uint32_t((2 * ks + g) ^ k_swz(arow)) * 16;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) p_off[ks] = kPeOff + uint32_t(arow) * (kR * 2) + uint32_t((2 * ks + g) ^ pe_swz(arow)) * 16;
  // value operand (transposing) reads: lane -> column 32 cb + l32 of rows 16 ks + 8 g + 4 hh .. +3;
  // source lane s16 of a 16-lane group points at row + s16 / 4, chunk 4 cb + 2 chalf + (s16 & 3) / 2
  const int s16 = lane & 15, chalf = (lane >> 4) & 1;
  uint32_t tr_off[4][2];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int row = 8 * g + 4 * hh + (s16 >> 2);
      const int chunk = 4 * cb + 2 * chalf + ((s16 & 3) >> 1);
      tr_off[cb][hh] = kVOff + uint32_t(row) * (kDv * 2) + uint32_t(chunk ^ v_swz(row)) * 16 + (s16 & 1) * 8;
    }

  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
  float m_ref = -INFINITY, lsum = 0.f;

  // one pair of tiles; sp is the stage of its first tile (0 or 2, a constant in each inlined copy,
  // so that every LDS address is a loop-invariant register plus an immediate offset)
  auto pair = [&](int p, const int sp) __attribute__((always_inline)) {
    // pair p must have landed: pair 0 with the query, pair p > 0 as the latest issued
    if (p > 0) wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();  // every wave's part of pair p is in; every wave is done with pair p - 1
    compiler_fence();

    // scores S^T[position][row] of the pair's two tiles
    f32x16 sacc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const unsigned char *st = smem + (sp + u) * kStageBytes;
      u32x4 fr[12];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) fr[ks] = lds_read16(st, k_off[ks]);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) fr[8 + ks] = lds_read16(st, p_off[ks]);
      sacc[u] = f32x16{};
      // pair p + 1 goes into pair p - 1's stages, one DMA instruction after every second score
      // MFMA (unconditionally: past the last pair it re-reads clamped rows into finished stages)
#pragma unroll
      for (int ks = 0; ks < 12; ++ks) {
        sacc[u] = mfma32(fr[ks], qf[ks], sacc[u]);
        if ((ks & 1) && ks < 10) issue_part(2 * p + 2 + u, ks >> 1);
      }
    }
    const int t0 = 2 * p * kTile;
    if (t0 + 2 * kTile > wg_full) {  // wavefront-uniform: positions past some row's last visible one
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = t0 + kTile * u + 16 * (r >> 3) + 8 * g + (r & 7);
          if (t >= row_end) sacc[u][r] = -INFINITY;
        }
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, sacc[u][r]);
    const float mrow = xor32_max(mloc) * a.scale_log2;
    if (m_ref == -INFINITY) {
      m_ref = mrow;
    } else if (mrow > m_ref + kRescale) {
      const float alpha = fast_exp2(m_ref - mrow);
      lsum *= alpha;
      m_ref = mrow;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= alpha;
    }
    const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const unsigned char *st = smem + (sp + u) * kStageBytes;
      u32x4 pb[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float pr[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          pr[r] = fast_exp2(fmaf(sacc[u][8 * hh + r], a.scale_log2, -m_use));
          lsum += pr[r];
        }
        pb[hh] = u32x4{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]), pack_bf16x2(pr[4], pr[5]),
                       pack_bf16x2(pr[6], pr[7])};
      }
      // O^T[c][row] += V^T[c][position] . P^T[position][row]
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const u32x4 vf = lds_read_tr_pair(st, tr_off[cb][0] + ks * 16 * (kDv * 2), tr_off[cb][1] + ks * 16 * (kDv * 2));
          acc[cb] = mfma32(vf, pb[ks], acc[cb]);
        }
    }
  };
#pragma unroll 1
  for (int p = 0; p < npairs; p += 2) {  // pair p in stages 0 and 1, pair p + 1 in stages 2 and 3
    pair(p, 0);
    if (p + 1 < npairs) pair(p + 1, 2);
  }
  wait_vmcnt<0>();  // tiles issued past the last needed one land before the workgroup ends

  // ---- out[b, s, h, c]: lane holds row s, c = 32 cb + 8 q + 4 g + r % 4 in register 4 q + r % 4
  lsum = xor32_sum(lsum);
  if (!row_ok) return;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  uint16_t *dst = a.out + ((int64_t(b) * a.S + s) * a.H + h) * kDv + 4 * g;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x2 v2{pack_bf16x2(acc[cb][4 * q] * inv, acc[cb][4 * q + 1] * inv),
                     pack_bf16x2(acc[cb][4 * q + 2] * inv, acc[cb][4 * q + 3] * inv)};
      *reinterpret_cast<u32x2 *>(dst + 32 * cb + 8 * q) = v2;
    }
}

}  // namespace

bool mfma_naive_supported(const NaiveCall &c, const char **why) {
  if (c.dtype != MLA_DTYPE_BF16) { *why = "needs bf16"; return false; }
  if (c.R != kR || c.Dn != kDn || c.Dv != kDv) {
    *why = "needs qk_rope_head_dim 64, qk_nope_head_dim 128, v_head_dim 128";
    return false;
  }
  if (c.Tmax >= (int64_t(1) << 22)) { *why = "cache_len must be below 4194304"; return false; }
  // query offsets of one (sequence, head), up to the last row block, are 32-bit byte counts
  if ((c.S + kRowsWG) * c.H * int64_t(kDn) * 2 >= (int64_t(1) << 32)) { *why = "seqlen_q * n_heads too large"; return false; }
  return true;
}

hipError_t mfma_naive_attn(const NaiveCall &c) {
  NaiveArgs a{};
  a.q_nope = static_cast<const uint16_t *>(c.q_nope);
  a.q_pe = static_cast<const uint16_t *>(c.q_pe);
  a.k_nope = static_cast<const uint16_t *>(c.k_nope);
  a.v = static_cast<const uint16_t *>(c.v);
  a.pe = static_cast<const uint16_t *>(c.pe);
  a.out = static_cast<uint16_t *>(c.out);
  a.Bmax = c.Bmax;
  a.Tmax = c.Tmax;
  a.B = int32_t(c.B);
  a.S = int32_t(c.S);
  a.H = int32_t(c.H);
  a.end_pos = int32_t(c.end_pos);
  a.row_blocks = int32_t((c.S + kRowsWG - 1) / kRowsWG);
  a.scale_log2 = c.scale * 1.4426950408889634f;
  const int64_t nwg = c.B * c.H * int64_t(a.row_blocks);
  return launch_kernel(MLA_KERNEL_NAIVE, naive_attn_kernel, dim3(unsigned(nwg)), dim3(256), 0, c.stream, a);
}

}  // namespace mla
