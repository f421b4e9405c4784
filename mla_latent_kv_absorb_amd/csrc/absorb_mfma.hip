// Matrix-core absorb-form MLA attention for the DeepSeek-V3 head shape
// (kv_lora_rank 512, qk_rope_head_dim 64, qk_nope_head_dim 128, v_head_dim 128), bf16 storage,
// fp32 accumulation.
//
// The computation is the absorb path of the page "Naive vs Absorb Attention Implementations in
// DeepSeek-V3" (section "Absorb Path Execution"), run as three kernels:
//   1. absorb_q_kernel   q_lat[row, :] = q_nope[row, :] . W_UK[h]            (query absorption),
//                        stored together with q_pe in the attention kernel's operand order
//   2. attn_kernel       per (sequence, 128-row block, position split): scores against kv_cache
//                        (512) and pe_cache (64) as one 576-deep contraction, online softmax,
//                        probability-weighted sum over kv_cache in latent space.  The cache rows
//                        come from contiguous caches, from page pools through a block table, or
//                        from the positions a per-token index list names (one template; only the
//                        row addressing and the mask differ).  Each source has a second instance
//                        whose cache DMA carries the non-temporal hint, for launches with one row
//                        block, where every cache row has a single reader
//   3. combine_kernel    merge the split partials (running maximum, weights exp2(m_i - M)) and
//                        project out through W_UV[h]
// Rows are the B*S*H query rows in (b, s, h) order.  Every kv/pe row of a split is read from HBM
// once per 128-row block and shared through LDS by all of the block's heads.
#include <algorithm>
#include <numeric>
#include <type_traits>

#include "append_row.h"
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
constexpr int kTile = 32;      // cached positions per LDS tile (one 32-position MFMA block)
constexpr int kStages = 4;     // tiles in LDS: three in flight while one is consumed
constexpr int kRowsWG = 128;   // query rows per attention workgroup (4 waves x 32)
constexpr int kKvTileBytes = kTile * kC * 2;              // 32 KB
constexpr int kPeTileBytes = kTile * kR * 2;              // 4 KB
constexpr int kStageBytes = kKvTileBytes + kPeTileBytes;  // 36 KB; four stages fill 144 KB of LDS
constexpr int kLoadsPerTile = kTile * (kC + kR) * 2 / 16 / 256;  // 16-byte DMA loads per thread per tile (9)
constexpr float kLog2e = 1.4426950408889634f;

// LDS on gfx950 has 64 four-byte banks; a ds_read_b128 is serviced 16 lanes at a time and a
// (transposing) 8-byte read 32 lanes at a time.  kv tile rows are 1 KB, so every row starts on
// bank 0; 16-byte chunks are XOR-swizzled inside aligned groups of 16 (256 bytes) by
// F(row) = ((row & 3) << 2) | ((row >> 2) & 3):
//   - score read: 16 lanes read one chunk of rows r0..r0+15 -> F is a bijection on row & 15;
//   - P.V transposing read: 32 lanes read chunks 4k..4k+3 of rows r0..r0+3 -> the high two bits
//     of F are row & 3, so the four rows land on four different 64-byte quarters.
// pe rows are 128 bytes (two per bank period); their 8 chunks are XOR-swizzled by (row >> 1) & 7.
__device__ __forceinline__ int kv_swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ int swz_chunk(int chunk, int row) { return (chunk & ~15) | ((chunk & 15) ^ kv_swz(row)); }
__device__ __forceinline__ int pe_swz(int row) { return (row >> 1) & 7; }

// The score MFMA's output row i is fed from tile row rho(i) (bits 2 and 3 swapped).  With that
// order, registers 0..7 of lane l hold positions 8*(l/32) + 0..7 and registers 8..15 hold
// positions 16 + 8*(l/32) + 0..7, which is exactly the B-operand layout the P.V MFMA needs, so the
// probabilities never leave registers.
__device__ __forceinline__ int rho(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

// Absorbed query in fragment-major order, written by absorb_q_kernel and read by attn_kernel:
// [sequence][128-row block][wave][ks = 0..35][l32][g][8 bf16].  Lane l = l32 + 32 g of wave w
// holds row 128 rb + 32 w + l32 (rows in (s, h) order within the sequence), latent elements
// 16 ks + 8 g .. +7 for ks < 32 and rope elements 16 (ks - 32) + 8 g .. +7 for ks >= 32.  A wave's
// load of one ks is one contiguous 1 KB, and each row's two chunks of a ks are adjacent (32 bytes),
// so the absorb kernel's stores complete whole 32-byte sectors.
constexpr int kFragBytesPerWave = 36 * 1024;
constexpr int kFragElemsPerBlock = 4 * kFragBytesPerWave / 2;
constexpr int kQpeBytesPerWave = 4 * 1024;  // a wave's rope-query fragments, kept in LDS

struct AttnArgs {
  const uint16_t *q_frag;  // fragment-major absorbed + rope query (layout above)
  const uint16_t *kv;      // [Bmax, Tmax, 512]
  const uint16_t *pe;      // [Bmax, Tmax, 64]
  float *part_ml;          // [rows, splits, 2]   (max in log2 units, sum)
  uint16_t *part_o;        // [rows, splits, 512] (unnormalised, relative to the max; with one
                           // split: normalised, i.e. o_lat)
  int64_t Tmax;
  int64_t kv_bs, pe_bs;    // element strides between cache rows b and b + 1 (contiguous caches)
  int32_t kv_rb, pe_rb;    // bytes between positions t and t + 1 (and between rows of a page)
  int32_t S, H, SH;        // SH = S * H rows per sequence
  int32_t end_pos, splits, split_len, row_blocks;  // end_pos: uniform length or the bound of seq_lens
  const int32_t *seq_lens;  // per-sequence lengths [B] or null (every sequence has end_pos)
  float scale_log2;        // softmax_scale * log2(e)
  // paged caches: kv / pe are pools of 2^log2_page positions per page, block_table [B, max_pages]
  const int32_t *block_table;
  int32_t log2_page, max_pages, num_pages;
  // index lists [B, S, topk]: token (b, s) attends to the positions its list names
  const int32_t *indices;
  int32_t topk;
  // balanced ragged plan (bal_target > 0): sequence b's positions are cut into n_b chunks of one
  // common length (see balanced_chunk), long sequences into more of them; splits is the most
  // chunks a sequence may take, bal_target the number of workgroups per row block (one per chunk,
  // chunks packed in sequence order), and bal_nb [B * S] receives n_b for each query row of
  // sequence b (b * S + s), for the combine
  int32_t B, bal_target, bal_cap;  // bal_cap: longest chunk the row source allows (paged caches)
  int32_t rb_stride;  // row block of logical index r within a sequence: r * rb_stride mod row_blocks
  int32_t *bal_nb;
};

// Chunk length of a sequence of len positions in a balanced plan whose common chunk length is L:
// len / n rounded up to 32 positions, for n = ceil(len / L) chunks, or more where the row source
// caps a chunk at cap positions, at most smax.
__device__ __forceinline__ int bal_len(int len, int L, int smax, int cap) {
  const int n = min(smax, max((len + L - 1) / L, len <= cap ? 1 : (len - 1) / cap + 1));
  return ((len + n - 1) / n + 31) & ~31;
}
// Chunks of that sequence: every one starts before len (rounding can leave fewer than n).
__device__ __forceinline__ int bal_chunks(int len, int L, int smax, int cap) {
  const int sl = bal_len(len, L, smax, cap);
  return (len + sl - 1) / sl;
}

// Chunk length of a balanced ragged plan: the smallest multiple L of 32, at least 256 (or the
// bound), with sum_b bal_chunks(len_b, L) <= target (len_b the clamped lengths), found by a binary
// search in which every step is one wave-wide count.  Every wave of every workgroup computes it
// from the same inputs and gets the same L.  L = bound always qualifies: it gives each sequence
// one chunk, or ceil(len / cap) where the row source caps a chunk, and the plan's target covers
// B of the latter.
__device__ int balanced_chunk(const int32_t *lens, int len0, int B, int S, int bound, int smax, int cap, int target,
                              int lane) {
  auto count = [&](int L) {
    int c = lane < B ? bal_chunks(len0, L, smax, cap) : 0;
    for (int i = lane + 64; i < B; i += 64) c += bal_chunks(min(max(lens[i], S), bound), L, smax, cap);
    for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
    return __builtin_amdgcn_readfirstlane(c);
  };
  // in units of 32 positions; chunks of at least 256 positions where sequences allow: below that
  // a workgroup's fixed start and end (query and first tiles in, partial rows out) outweigh its
  // share of the positions, and every extra chunk adds a partial row to the combine
  int hi = (bound + 31) / 32, lo = min(8, hi);
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (count(32 * mid) <= target) hi = mid;
    else lo = mid + 1;
  }
  return 32 * lo;
}

// Whether a ragged batch runs the uniform plan inside the balanced launch: when its positions
// fill more than kUniformFill of B x the longest length.  Equal-length chunks pay off where a
// few long sequences would leave most of the uniform plan's workgroups idle; on a near-uniform
// spread the long sequences' extra chunks cost the combine more than they save.
constexpr float kUniformFill = 0.35f;
__device__ bool uniform_fits(const int32_t *lens, int len0, int B, int S, int bound, int lane) {
  float tot = lane < B ? float(len0) : 0.f;
  int mx = lane < B ? len0 : 0;
  for (int i = lane + 64; i < B; i += 64) {
    const int n = min(max(lens[i], S), bound);
    tot += float(n);
    mx = max(mx, n);
  }
  for (int o = 32; o > 0; o >>= 1) {
    tot += __shfl_xor(tot, o);
    mx = max(mx, __shfl_xor(mx, o));
  }
  return __builtin_amdgcn_readfirstlane(int(tot > kUniformFill * float(B) * float(mx)));
}

// Sequence and chunk of chunk rank r (chunks counted in sequence order), via a wave-wide prefix sum
// of the sequences' chunk counts, 64 sequences at a time.  False if r is past the last chunk.
__device__ bool balanced_find(const int32_t *lens, int len0, int B, int S, int bound, int smax, int cap, int L,
                              int r, int lane, int &b_out, int &c_out) {
  int base = 0;
  for (int j0 = 0; j0 < B; j0 += 64) {
    const int i = j0 + lane;
    const int n = j0 == 0 ? len0 : (i < B ? min(max(lens[i], S), bound) : 0);
    const int nb = i < B ? bal_chunks(n, L, smax, cap) : 0;
    int incl = nb;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    const uint64_t hit = __builtin_amdgcn_ballot_w64(base + incl > r);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      b_out = __builtin_amdgcn_readfirstlane(j0 + l);
      c_out = __builtin_amdgcn_readfirstlane(r - base - __shfl(incl - nb, l));
      return true;
    }
    base += __shfl(incl, 63);
  }
  return false;
}

// Where tile rows come from: contiguous caches [Bmax, Tmax, .]; page pools; or the rows an index
// list names (the tiles then run over list entries instead of positions).
enum : int { kModeContig = 0, kModePaged = 1, kModeSparse = 2 };

// A paged workgroup keeps the page ids of its positions, a sparse one the entries of its index
// list, in kPageRegs registers (one per lane and register): a split may touch at most 64 kPageRegs
// pages or list entries.
constexpr int kPageRegs = 4;

// Softmax rows keep a reference maximum m_ref and only move it (rescaling the running sum and the
// 512 accumulators) when a tile's maximum exceeds it by more than kRescale (log2 units), so
// p = exp2(x - m_ref) <= 2^kRescale.  The result is exact in any case: numerator and denominator
// share the same reference.
constexpr float kRescale = 8.f;

// kStream: one row block covers every query row of a sequence (decode), so each cache row is read
// by one workgroup only and its DMA carries the non-temporal hint
template <int kMode, bool kStream>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_kernel(AttnArgs a) {
  constexpr bool kPaged = kMode == kModePaged, kSparse = kMode == kModeSparse;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kStages * kStageBytes + 4 * kQpeBytesPerWave];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, g = lane >> 5;

  // logical order: row block fastest, then split, then sequence; the workgroups of one sequence
  // (which share its query rows and cache) land on one XCD
  int bid = __builtin_amdgcn_readfirstlane(xcd_logical_id(blockIdx.x, gridDim.x));
  // Row blocks go to the workgroups of a sequence in a strided order (a permutation: rb_stride is
  // coprime with row_blocks), so that each XCD's contiguous share mixes early and late query
  // tokens of a causal chunk, whose lengths differ, instead of taking all the short or all the
  // long ones.
  const int rb = __builtin_amdgcn_readfirstlane(
      int(uint64_t(bid % a.row_blocks) * uint32_t(a.rb_stride) % uint32_t(a.row_blocks)));
  bid /= a.row_blocks;
  // balanced ragged plan: bid is a chunk rank, and the plan comes from all lengths
  const bool balanced = !kSparse && a.bal_target > 0;
  int split = __builtin_amdgcn_readfirstlane(bid % a.splits);
  int b = __builtin_amdgcn_readfirstlane(bid / a.splits);
  int bal_L = 0;     // chunk length of the equal-chunk plan
  int uni_len = 0;   // > 0: the batch runs the uniform plan with splits of this length
  if (balanced) {
    // lane l holds sequence l's clamped length (the first 64; more are re-read as needed)
    const int len0 = lane < a.B ? min(max(a.seq_lens[lane], a.S), a.end_pos) : 0;
    if (uniform_fits(a.seq_lens, len0, a.B, a.S, a.end_pos, lane)) {
      // every sequence s0 splits of the bound's length (the grid holds B s0 workgroups); the
      // combine still reads only each sequence's non-empty ones
      const int s0 = a.bal_target / a.B;
      uni_len = __builtin_amdgcn_readfirstlane(((a.end_pos + s0 - 1) / s0 + 31) & ~31);
      b = __builtin_amdgcn_readfirstlane(bid / s0);
      split = __builtin_amdgcn_readfirstlane(bid - b * s0);
    } else {
      bal_L = __builtin_amdgcn_readfirstlane(
          balanced_chunk(a.seq_lens, len0, a.B, a.S, a.end_pos, a.splits, a.bal_cap, a.bal_target, lane));
      if (!balanced_find(a.seq_lens, len0, a.B, a.S, a.end_pos, a.splits, a.bal_cap, bal_L, bid, lane, b, split))
        return;  // fewer chunks than workgroups: nothing to do
    }
  }

  // this lane's query row (its column of the score tile)
  const int lrow = rb * kRowsWG + wave * 32 + l32;
  const bool row_ok = lrow < a.SH;
  const int s = row_ok ? lrow / a.H : 0;
  const int64_t grow = int64_t(b) * a.SH + lrow;
  // this sequence's length: a ragged batch reads it from seq_lens, clamped to [S, end_pos] so that
  // no access leaves the positions the caller vouched for
  const int end_pos = a.seq_lens ? __builtin_amdgcn_readfirstlane(min(max(a.seq_lens[b], a.S), a.end_pos)) : a.end_pos;
  // The split's positions [t_begin, t_split_end): a fixed split length, or (balanced ragged plan)
  // this sequence's share of its n_b chunks of about equal length, a multiple of 32.  Sparse: the
  // split covers list entries [t_begin, t_split_end) of one query token.
  int split_len = a.split_len, t_begin = split * a.split_len;
  if (balanced) {  // chunk `split` of the sequence's chunks (split < their count by construction,
                   // except in the uniform plan, whose splits past the sequence are empty)
    split_len = uni_len > 0 ? uni_len : __builtin_amdgcn_readfirstlane(bal_len(end_pos, bal_L, a.splits, a.bal_cap));
    t_begin = split * split_len;
    if (split == 0 && rb == 0)  // the chunk count, for the combine: one entry per query row
      for (int i = threadIdx.x; i < a.S; i += 256) a.bal_nb[b * a.S + i] = (end_pos + split_len - 1) / split_len;
  }
  const int t_split_end = min(t_begin + split_len, kSparse ? a.topk : end_pos);
  const int row_end = row_ok ? min(t_split_end, end_pos - a.S + s + 1) : t_begin;
  // Positions the workgroup needs (up to the last visible one of its last row), and the prefix
  // visible to all of its rows (tiles inside it need no mask).  Integer division runs on the
  // vector ALU, so the uniform results are re-scalarised.
  const int first_row = rb * kRowsWG;
  const int last_row = min(a.SH - 1, first_row + kRowsWG - 1);
  const int wg_end = __builtin_amdgcn_readfirstlane(kSparse ? t_split_end
                                                            : min(t_split_end, end_pos - a.S + last_row / a.H + 1));
  const int wg_full = __builtin_amdgcn_readfirstlane(kSparse ? t_split_end
                                                             : min(t_split_end, end_pos - a.S + first_row / a.H + 1));
  const int ntiles = __builtin_amdgcn_readfirstlane(wg_end > t_begin ? (wg_end - t_begin + kTile - 1) / kTile : 0);
  if (ntiles == 0) {
    // nothing of this split is visible to the workgroup's rows (a short sequence of a ragged
    // batch): only the statistics of an empty partial; the combine never reads its o rows.  (With
    // a single split every workgroup has a tile, so this needs the multi-split combine.)
    if (row_ok && g == 0) {
      const int64_t idx = grow * a.splits + split;
      a.part_ml[2 * idx] = -INFINITY;
      a.part_ml[2 * idx + 1] = 0.f;
    }
    return;
  }

  // DMA geometry.  kv: wave w moves tile rows 8w..8w+7, one 1 KB row per instruction; lane l owns
  // chunk position l and fetches source chunk swz_chunk(l, row).  pe: wave w moves rows
  // 8w..8w+7 (128 bytes each) in one instruction.  Rows past the last needed position repeat the
  // last one (valid data, masked in the softmax); wg_end >= 1, so that row always exists.
  //
  // Paged caches: splits start on 32-position boundaries and pages hold a power of two >= 32
  // positions, so each tile lies in one page, whose base goes into the tile's buffer descriptors
  // (64-bit, any pool size); the rows' offsets within the page stay 32-bit.  The page ids of the
  // split's positions sit in registers (slot 64 k + lane of register k is page index
  // t_begin / page_size + slot), read per tile with v_readlane; tile 0's id comes from a scalar
  // load so that its DMA need not wait for them.  Rows are clamped into [t0, t0 + 31] as well,
  // which keeps every offset inside the page even for a workgroup with no tile to compute.
  const rsrc_t kvres = make_rsrc(a.kv + (kPaged ? 0 : int64_t(b) * a.kv_bs),
                                 kPaged ? 0u : uint32_t(a.Tmax - 1) * uint32_t(a.kv_rb) + kC * 2);
  const rsrc_t peres = make_rsrc(a.pe + (kPaged ? 0 : int64_t(b) * a.pe_bs),
                                 kPaged ? 0u : uint32_t(a.Tmax - 1) * uint32_t(a.pe_rb) + kR * 2);
  const int pg_first = t_begin >> a.log2_page;
  int ptab[kPageRegs];
  int page0 = 0;
  if constexpr (kPaged) {
    const int32_t *bt = a.block_table + int64_t(b) * a.max_pages;
    page0 = __builtin_amdgcn_readfirstlane(min(max(bt[min(pg_first, a.max_pages - 1)], 0), a.num_pages - 1));
    const rsrc_t btres = make_rsrc(bt, uint32_t(a.max_pages) * 4u);
#pragma unroll
    for (int k = 0; k < kPageRegs; ++k)  // indices past the table row read 0
      ptab[k] = min(max(buf_load_i32(btres, uint32_t(pg_first + 64 * k + lane) * 4u, 0), 0), a.num_pages - 1);
  }
  auto tile_page = [&](int j, int t0) __attribute__((always_inline)) -> int {
    if (j == 0) return page0;
    const int slot = (t0 >> a.log2_page) - pg_first;  // < 64 kPageRegs by the split plan
    const int ln = slot & 63, k = slot >> 6;
    int p = __builtin_amdgcn_readlane(ptab[0], ln);
#pragma unroll
    for (int r = 1; r < kPageRegs; ++r) p = k == r ? __builtin_amdgcn_readlane(ptab[r], ln) : p;
    return p;
  };
  // Sparse: the workgroup's rows are the heads of one query token, at position `bound`; list entry
  // t_begin + 64 k + lane sits in lane `lane` of ivreg[k].  Tile j's 32 entries are lanes
  // 32 (j & 1) .. + 31 of ivreg[j >> 1].  Rows are read at the entry's position clamped into the
  // sequence; entries naming no visible position are masked in the softmax.
  // (four named registers rather than an array: a select among array elements by a run-time
  // index would be lowered to an indexed scratch access)
  static_assert(kPageRegs == 4, "sparse_reg selects among four registers");
  int iv0 = 0, iv1 = 0, iv2 = 0, iv3 = 0;
  int bound = 0;
  if constexpr (kSparse) {
    const int s_tok = __builtin_amdgcn_readfirstlane(first_row / a.H);
    bound = end_pos - a.S + s_tok;
    const rsrc_t ires = make_rsrc(a.indices + (int64_t(b) * a.S + s_tok) * a.topk, uint32_t(a.topk) * 4u);
    const uint32_t off = uint32_t(t_begin + lane) * 4u;
    iv0 = buf_load_i32(ires, off, 0);
    iv1 = buf_load_i32(ires, off + 256u, 0);
    iv2 = buf_load_i32(ires, off + 512u, 0);
    iv3 = buf_load_i32(ires, off + 768u, 0);
  }
  auto sparse_reg = [&](int j) __attribute__((always_inline)) -> int {
    const int k = j >> 1;
    const int lo = (k & 1) ? iv1 : iv0, hi = (k & 1) ? iv3 : iv2;
    return (k & 2) ? hi : lo;
  };
  const int pe_row = wave * 8 + (lane >> 3);
  const uint32_t pe_voff = uint32_t((lane & 7) ^ pe_swz(pe_row)) * 16;
  // One of the tile's nine DMA instructions per wave: part 0..7 moves kv row 8w+part, part 8 the pe rows.
  const uint32_t smem_lds = lds_addr(smem);
  const uint32_t lane16 = uint32_t(lane) * 16;
  // Where tile j's rows come from: buffer descriptors, the position at their offset 0, and the
  // last row to read (rows past it repeat it).
  struct TileSrc {
    rsrc_t kv, pe;
    int tb, tlast;
    int cur, pidx, lo;  // sparse: the entries' register, this lane's pe row, the tile's first lane
  };
  auto tile_src = [&](int j) __attribute__((always_inline)) -> TileSrc {
    if constexpr (kPaged) {
      const int t0 = t_begin + j * kTile;
      const int64_t page = tile_page(j, t0);
      return TileSrc{make_rsrc(a.kv + (page << a.log2_page) * (a.kv_rb >> 1), uint32_t(a.kv_rb) << a.log2_page),
                     make_rsrc(a.pe + (page << a.log2_page) * (a.pe_rb >> 1), uint32_t(a.pe_rb) << a.log2_page),
                     t0 & ~((1 << a.log2_page) - 1), max(wg_end - 1, t0), 0, 0, 0};
    } else if constexpr (kSparse) {
      const int cur = sparse_reg(j), lo = (j & 1) * 32;
      const int pidx = __builtin_amdgcn_ds_bpermute((lo + pe_row) * 4, cur);
      return TileSrc{kvres, peres, 0, 0, cur, min(max(pidx, 0), end_pos - 1), lo};
    } else {
      return TileSrc{kvres, peres, 0, wg_end - 1, 0, 0, 0};
    }
  };
  auto dma = [&](rsrc_t r, uint32_t lds, uint32_t voff, uint32_t soff) __attribute__((always_inline)) {
    if constexpr (kStream) buf_load16_lds_at_nt(r, lds, voff, soff);
    else buf_load16_lds_at(r, lds, voff, soff);
  };
  auto issue_part = [&](int j, int part, const TileSrc &src) __attribute__((always_inline)) {
    const uint32_t st = smem_lds + uint32_t(j % kStages) * kStageBytes;
    const int t0 = t_begin + j * kTile;
    if (kSparse && part < 8) {
      const int t = min(max(__builtin_amdgcn_readlane(src.cur, src.lo + wave * 8 + part), 0), end_pos - 1);
      dma(src.kv, st + (wave * 8 + part) * (kC * 2), lane16 ^ uint32_t(kv_swz(8 * (wave & 1) + part) * 16),
          uint32_t(t) * uint32_t(a.kv_rb));
    } else if (kSparse) {
      dma(src.pe, st + kKvTileBytes + wave * 8 * (kR * 2), pe_voff + uint32_t(src.pidx) * uint32_t(a.pe_rb), 0);
    } else if (part < 8) {
      const int t = min(t0 + wave * 8 + part, src.tlast);  // wavefront-uniform
      // source chunk swz_chunk(lane, row) = lane ^ kv_swz(row), kv_swz(row) wavefront-uniform
      dma(src.kv, st + (wave * 8 + part) * (kC * 2), lane16 ^ uint32_t(kv_swz(8 * (wave & 1) + part) * 16),
          uint32_t(t - src.tb) * uint32_t(a.kv_rb));
    } else {
      // rows from the tile's first one, or (a tile past the end) from the last needed one, so
      // that every offset is that of a row the workgroup may read
      const int tq = min(t0, src.tlast);
      const int tp = min(t0 + pe_row, src.tlast);
      dma(src.pe, st + kKvTileBytes + wave * 8 * (kR * 2), pe_voff + uint32_t(tp - tq) * uint32_t(a.pe_rb),
          uint32_t(tq - src.tb) * uint32_t(a.pe_rb));
    }
  };
  auto issue = [&](int j) __attribute__((always_inline)) {
    const TileSrc src = tile_src(j);
#pragma unroll
    for (int part = 0; part < 9; ++part) issue_part(j, part, src);
  };

  // Prologue: tile 0; the absorbed query into registers and the rope query into LDS; a full wait
  // (the query loads are the only vector loads the compiler tracks, so completing them here keeps
  // its own vmcnt waits out of the loop body); then tiles 1 and 2, always issued so that the
  // in-loop wait counts stay exact (past the last needed position they re-read its row).
  if constexpr (!kSparse) issue(0);  // (sparse: after the query loads, behind its index loads)
  // Absorbed query as the score B operand: lane holds q[row][16 ks + 8 g .. +7], ks < 32.
  // absorb_q_kernel stores it fragment-major, so instruction ks of a wave reads one contiguous
  // 1 KB; lanes past the sequence's last row read out of range and get zeros.  The rope part
  // (ks 32..35) is copied by DMA to this wave's 4 KB of LDS in the same order.
  u32x4 qf[32];
  const unsigned char *qpe_lds = smem + kStages * kStageBytes + wave * kQpeBytesPerWave;
  {
    const rsrc_t qres = make_rsrc(a.q_frag + (int64_t(b) * a.row_blocks + rb) * kFragElemsPerBlock,
                                  kFragElemsPerBlock * 2);
    const uint32_t lane_slot = uint32_t(l32 * 32 + g * 16);
    const uint32_t qoff = row_ok ? uint32_t(wave * kFragBytesPerWave) + lane_slot : 0x80000000u;
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) qf[ks] = buf_load16(qres, qoff, ks * 1024);
    // DMA lane l writes LDS bytes 16 l .. of the plane, so it fetches the fragment of lane slot 16 l
    const uint32_t doff = uint32_t(wave * kFragBytesPerWave) + uint32_t(lane) * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      buf_load16_lds(qres, const_cast<unsigned char *>(qpe_lds) + i * 1024, doff, (32 + i) * 1024);
  }
  if constexpr (kSparse) issue(0);
  wait_vmcnt<0>();
  issue(1);
  issue(2);

  f32x16 acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = f32x16{};
  float m_ref = -INFINITY, lsum = 0.f;

  // score A-operand reads: tile row rho(l32), chunk c = 2 i + g (i = k % 8 within a 256-byte group
  // k / 8).  c ^ kv_swz(arow) = 2 (i ^ (kv_swz >> 1)) + (g ^ (kv_swz & 1)), so the address of i is
  // sc_base ^ (32 i) (bits 5..7 of sc_base hold 32 (kv_swz >> 1)).  The pe rows work the same way.
  const int arow = rho(l32);
  const uint32_t sc_base = uint32_t(arow) * (kC * 2) + uint32_t(g ^ (kv_swz(arow) & 1)) * 16 + uint32_t(kv_swz(arow) >> 1) * 32;
  const uint32_t pe_base = kKvTileBytes + uint32_t(arow) * (kR * 2) + uint32_t(g ^ (pe_swz(arow) & 1)) * 16 +
                           uint32_t(pe_swz(arow) >> 1) * 32;
  const uint32_t qpe_off = uint32_t(l32 * 32 + g * 16);
  // P.V A-operand (transposing) reads: source lane s16 of a 16-lane group reads row
  // 16 ks + 8 g + 4 h + s16 / 4, chunk 4 cb + 2 chalf + (s16 & 3) / 2, half (s16 & 1).
  const int s16 = lane & 15, chalf = (lane >> 4) & 1;
  // With chunk = 4 c4 + (2 chalf + (s16 & 3) / 2), chunk ^ kv_swz(row0) = 4 (c4 ^ (row0 & 3)) +
  // ((2 chalf + (s16 & 3) / 2) ^ ((row0 >> 2) & 3)), so the address for c4 is tr_base[h] ^ (64 c4);
  // + 256 B per (cb >> 2) and + 16 KB for ks = 1 go into the instruction offset.
  uint32_t tr_base[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row0 = 8 * g + 4 * h + (s16 >> 2);
    const int chunk = 2 * chalf + ((s16 & 3) >> 1);
    tr_base[h] = uint32_t(row0) * (kC * 2) + uint32_t(swz_chunk(chunk, row0)) * 16 + (s16 & 1) * 8;
  }

  // ---- scores S^T[position][row] of tile j over the 576-wide concatenation of kv and pe: 36 MFMAs
  // (32 over kv, then 4 over pe), their kv/pe fragments read through a ring of kRing registers
  // kRing - 1 MFMAs ahead.  After each group of four MFMAs comes one of the nine DMA instructions
  // of tile `rtile` (when `refill`), so that a full memory queue stalls one instruction at a time.
  // (In the loop the refill is unconditional: a tile past the workgroup's last one re-reads its
  // last needed row into the stage of a finished tile, which is cheaper than a branch per part.)
  // the swizzled per-lane read addresses, XOR-ed once here instead of once per tile
  uint32_t scx[8], pex[4], trx[2][4];
#pragma unroll
  for (int i = 0; i < 8; ++i) scx[i] = sc_base ^ uint32_t(32 * i);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pex[i] = pe_base ^ uint32_t(32 * i);
    trx[0][i] = tr_base[0] ^ uint32_t(64 * i);
    trx[1][i] = tr_base[1] ^ uint32_t(64 * i);
  }
  constexpr int kRing = 6;
  auto scores = [&](int j, f32x16 &sc, bool refill, int rtile, const TileSrc &rsrc) __attribute__((always_inline)) {
    const unsigned char *st = smem + (j % kStages) * kStageBytes;
    auto frag = [&](int k) __attribute__((always_inline)) -> u32x4 {
      return k < 32 ? lds_read16(st, scx[k & 7] + (k >> 3) * 256)
                    : lds_read16(st, pex[k - 32]);
    };
    u32x4 fr[kRing], qp[4];
#pragma unroll
    for (int k = 0; k < kRing - 1; ++k) fr[k] = frag(k);
#pragma unroll
    for (int grp = 0; grp < 9; ++grp) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = 4 * grp + i;
        if (k + kRing - 1 < 36) fr[(k + kRing - 1) % kRing] = frag(k + kRing - 1);
        if (k >= 28 && k < 32) qp[k - 28] = lds_read16(qpe_lds, qpe_off + (k - 28) * 1024);
        __builtin_amdgcn_sched_barrier(0);
        const u32x4 &qb = k < 32 ? qf[k] : qp[k - 32];
        if (k == 0) mfma32_v_first(sc, fr[k % kRing], qb);
        else if (k == 35) mfma32_v_last(sc, fr[k % kRing], qb);
        else mfma32_v(sc, fr[k % kRing], qb);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (refill) issue_part(rtile, grp, rsrc);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- online softmax (log2 domain) of one tile's scores; register r holds position
  // 16*(r/8) + 8*g + r%8 of the tile
  float mrow = 0.f;
  auto sm_mask = [&](f32x16 &sc, int t0) __attribute__((always_inline)) {
    if constexpr (kSparse) {  // entries of the split naming a position in [0, bound]
      const int j = (t0 - t_begin) >> 5;
      const int cur = sparse_reg(j);
      const int e = t_begin + ((j >> 1) << 6) + lane;
      const bool ok = e < wg_end && cur >= 0 && cur <= bound;
      const uint32_t valid = uint32_t(__builtin_amdgcn_ballot_w64(ok) >> ((j & 1) * 32));
      if (valid != 0xffffffffu) {  // wavefront-uniform
        const uint32_t vg = valid >> (8 * g);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (!((vg >> (16 * (r >> 3) + (r & 7))) & 1u)) sc[r] = -INFINITY;
      }
      return;
    }
    if (t0 + kTile > wg_full) {  // wavefront-uniform: positions past a row's last visible one
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = t0 + 16 * (r >> 3) + 8 * g + (r & 7);
        if (t >= row_end) sc[r] = -INFINITY;
      }
    }
  };
  auto sm_max = [&](const f32x16 &sc) __attribute__((always_inline)) {
    float mloc = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, sc[r]);
    mrow = xor32_max(mloc) * a.scale_log2;  // scale > 0
  };
  // Moving the reference max scales the running sum at once; the accumulators are scaled by
  // apply_rescale() once the P.V product of the tiles before this one is complete (the softmax of
  // a tile runs while that product is still accumulating).
  // Written without branches so that it can be interleaved with the P.V MFMAs.
  float alpha_pending = 1.f;
  auto sm_ref = [&]() __attribute__((always_inline)) {
    const bool first = m_ref == -INFINITY;  // first visible positions: nothing accumulated yet
    const float m_new = (first || mrow > m_ref + kRescale) ? mrow : m_ref;
    const float alpha = first ? 1.f : fast_exp2(m_ref - m_new);  // exactly 1 when m_new == m_ref
    lsum *= alpha;
    alpha_pending = alpha;
    m_ref = m_new;
  };
  auto apply_rescale = [&]() __attribute__((always_inline)) {
    if (alpha_pending != 1.f) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = agpr_write(agpr_read(acc[i][r]) * alpha_pending);
      alpha_pending = 1.f;
    }
  };
  // probabilities of positions 16 h .. 16 h + 15 (the B operand of K half h of the P.V product)
  auto sm_probs = [&](const f32x16 &sc, int h) __attribute__((always_inline)) -> u32x4 {
    const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
    float p[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      p[r] = fast_exp2(fmaf(sc[8 * h + r], a.scale_log2, -m_use));
      lsum += p[r];
    }
    return u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                 pack_bf16x2(p[6], p[7])};
  };

  // ---- O^T[c][row] += KV^T[c][position] . P^T[position][row] for tile j: 32 MFMAs, first K half
  // (positions 0..15) over all 16 column blocks, then the second half.  The transposed A fragments
  // go through a ring of four registers, three MFMAs ahead.  pv_steps runs steps [lo, hi), so that
  // other work can be placed between ranges (the bounds are constants at every call).
  auto trl = [&](int j, int n, int ks) __attribute__((always_inline)) -> u32x4 {
    const unsigned char *st = smem + (j % kStages) * kStageBytes;
    return lds_read_tr_pair(st, trx[0][n & 3] + (n >> 2) * 256 + ks * 16384,
                            trx[1][n & 3] + (n >> 2) * 256 + ks * 16384);
  };
  u32x4 trf[4];
  auto pv_begin = [&](int j) __attribute__((always_inline)) {
#pragma unroll
    for (int step = 0; step < 3; ++step) trf[step] = trl(j, step, 0);
  };
  auto pv_steps = [&](int j, const u32x4 (&pb)[2], int lo, int hi) __attribute__((always_inline)) {
#pragma unroll
    for (int step = lo; step < hi; ++step) {
      const int ks = step >> 4, cb = step & 15;
      if (step + 3 < 32) trf[(step + 3) & 3] = trl(j, (step + 3) & 15, (step + 3) >> 4);
      __builtin_amdgcn_sched_barrier(0);
      acc[cb] = mfma32(trf[step & 3], pb[ks], acc[cb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // The same 32 steps with no fixed order, for a block that the caller interleaves with other
  // vector work through scheduling-group barriers.
  auto pv_all_free = [&](int j, const u32x4 (&pb)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int step = 0; step < 32; ++step) {
      const int ks = step >> 4, cb = step & 15;
      if (step + 3 < 32) trf[(step + 3) & 3] = trl(j, (step + 3) & 15, (step + 3) >> 4);
      acc[cb] = mfma32(trf[step & 3], pb[ks], acc[cb]);
    }
  };

  // Software pipeline over tiles: iteration j runs the score MFMAs of tile j + 1, then the P.V
  // MFMAs of tile j while the vector ALU does the softmax of tile j + 1.  Tiles j and j + 1 are
  // read in iteration j; tile j + 3 is refilled into the stage of tile j - 1, which every wave has
  // finished after the iteration's barrier.  Tiles 0..2 are issued by the prologue and one tile
  // per iteration by the loop in any case (rows clamped), which keeps the wait counts exact.
  f32x16 sacc;
  u32x4 pb[2];  // probabilities of the tile whose P.V product comes next
  if (ntiles > 0) {
    wait_vmcnt<2 * kLoadsPerTile>();  // tile 0 has landed; tiles 1 and 2 may be in flight
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    scores(0, sacc, false, 0, tile_src(0));
    sm_mask(sacc, t_begin);
    sm_max(sacc);
    sm_ref();
    pb[0] = sm_probs(sacc, 0);
    pb[1] = sm_probs(sacc, 1);
  }
#pragma unroll 1
  for (int j = 0; j + 1 < ntiles; ++j) {
    // tile j+1 must have landed; tile j+2 (issued one iteration ago, or by the prologue, real or
    // past the end) may not
    wait_vmcnt<kLoadsPerTile>();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    const TileSrc rs = tile_src(j + 3);
    if constexpr (kSparse) asm volatile("" ::"v"(rs.pidx));  // wait for the permute here, not among the score reads
    scores(j + 1, sacc, true, j + 3, rs);
    const int t1 = t_begin + (j + 1) * kTile;
    sm_mask(sacc, t1);
    u32x4 pn[2];
    pv_begin(j);
    __builtin_amdgcn_sched_barrier(0);
    // one block: the P.V MFMAs of tile j with the softmax of tile j + 1 spread between them (each
    // MFMA followed by up to three vector instructions and two LDS reads)
    pv_all_free(j, pb);
    sm_max(sacc);
    sm_ref();
    pn[0] = sm_probs(sacc, 0);
    pn[1] = sm_probs(sacc, 1);
    // keeps the compiler from sinking the softmax below the block (its results are used only later)
    asm volatile("" : "+v"(pn[0]), "+v"(pn[1]), "+v"(lsum));
#pragma unroll
    for (int step = 0; step < 32; ++step) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS read
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
    }
    __builtin_amdgcn_sched_barrier(0);
    apply_rescale();
    pb[0] = pn[0];
    pb[1] = pn[1];
  }
  if (ntiles > 0) {
    pv_begin(ntiles - 1);
    pv_steps(ntiles - 1, pb, 0, 32);
  }

  // ---- partial state of this split: max (log2 units), sum, unnormalised o.  o goes through LDS
  // so that every global store writes one whole 1 KB row.
  lsum = xor32_sum(lsum);
  // with a single split the result is final: normalise here (the combine kernel then only projects)
  const float oscale = (a.splits == 1 && lsum > 0.f) ? 1.f / lsum : 1.f;
  wait_vmcnt<0>();
  __syncthreads();  // every wave is done with the tiles
  unsigned char *stage = smem + wave * (32 * kC * 2);  // this wave's 32 rows
#pragma unroll
  for (int cb = 0; cb < 16; ++cb) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x2 v{pack_bf16x2(agpr_read(acc[cb][4 * q]) * oscale, agpr_read(acc[cb][4 * q + 1]) * oscale),
                    pack_bf16x2(agpr_read(acc[cb][4 * q + 2]) * oscale, agpr_read(acc[cb][4 * q + 3]) * oscale)};
      const int chunk = 4 * cb + q;
      lds_write8(stage, uint32_t(l32) * (kC * 2) + uint32_t((chunk & ~15) | ((chunk & 15) ^ (l32 & 15))) * 16 + 8 * g, v);
    }
  }
  if (row_ok && g == 0) {
    const int64_t idx = grow * a.splits + split;
    a.part_ml[2 * idx] = m_ref;
    a.part_ml[2 * idx + 1] = lsum;
  }
  // same wavefront wrote these rows; LDS operations of one wavefront complete in order
  const int rows_here = min(32, a.SH - (first_row + wave * 32));
  for (int r = 0; r < rows_here; ++r) {
    const u32x4 v = lds_read16(stage, uint32_t(r) * (kC * 2) + uint32_t((lane & ~15) | ((lane & 15) ^ (r & 15))) * 16);
    const int64_t idx = (int64_t(b) * a.SH + first_row + wave * 32 + r) * a.splits + split;
    // written through: the combine reads the rows from the XCD of their head, not this one
    buf_store16_sys(make_rsrc(a.part_o + idx * kC, kC * 2), v, uint32_t(lane) * 16, 0);
  }
}

// ------------------------------------------------------------------------------------------------
// q_lat[row, c0 + c] = sum_d q_nope[row, d] * W_UK[h][d][c0 + c] for one head h and 128 columns,
// written fragment-major for attn_kernel (the first column quarter also copies q_pe there).
// W_UK is staged in LDS once ([128 d][128 c], 16-byte chunks XOR-swizzled) and read transposed,
// because the contraction runs over d while c is the contiguous index of wkv_b.
constexpr int kQBlocksPerWG = 4;  // 32-row blocks of query rows per absorb_q workgroup

struct AbsorbQArgs {
  const uint16_t *q_nope;  // [rows, Dn] with rows = M * H (row = m * H + h)
  const uint16_t *q_pe;    // [rows, 64]
  const uint16_t *wkv_b;   // [H * 256, 512]
  uint16_t *q_frag;        // fragment-major q_lat and q_pe (see kFragBytesPerWave)
  int32_t H, M;            // M = B * S query rows per head
  int32_t S, row_blocks;   // query tokens per sequence; 128-row blocks per sequence
  int32_t row_blocks_per_wg;
  float inv_S;             // 1 / S
  int32_t qn_rs, qp_rs;    // elements between consecutive query rows of q_nope and of q_pe
  AppendCall app;          // fused cache append (kApp): its rows are written by this launch
};

// Byte offset of row (m, h)'s slot in the fragment buffer (add ks * 1024 + g * 16).
__device__ __forceinline__ int64_t frag_row_offset(int m, int h, const AbsorbQArgs &a) {
  // b = m / S without an integer division: m < 2^24, so the float quotient is off by at most one
  int b = int(float(m) * a.inv_S);
  b -= (b * a.S > m);
  b += ((b + 1) * a.S <= m);
  const int lrow = (m - b * a.S) * a.H + h;
  return ((int64_t(b) * a.row_blocks + (lrow >> 7)) * 4 + ((lrow >> 5) & 3)) * int64_t(kFragBytesPerWave) +
         (lrow & 31) * 32;
}

// W_UK tile rows are 256 bytes (one bank period, 16 chunks).  The transposing read touches 4
// consecutive rows x 4 chunks per 32 lanes; XOR-ing the chunk with (row & 3) << 2 puts the four
// rows in different 64-byte quarters.
__device__ __forceinline__ int w_swz(int row) { return (row & 3) << 2; }

// kApp: the launch also writes the rows of a fused cache append (a.app): an extra column of
// workgroups (blockIdx.y == kC / 128) does only that, one wavefront per token, beside the
// absorption; the attention kernel, launched after this one, reads the rows
template <bool kApp>
__global__ void __launch_bounds__(256) absorb_q_kernel(AbsorbQArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char wt[kDn * 128 * 2];  // 32 KB
  __shared__ __attribute__((aligned(16))) unsigned char xt[2][32 * kDn * 2];  // 2 x 8 KB
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (kApp && blockIdx.y == kC / 128) {
    const int64_t ntok = a.app.B * a.app.S;
    const int64_t stride = int64_t(gridDim.x) * gridDim.z * 4;
    for (int64_t tok = (int64_t(blockIdx.z) * gridDim.x + blockIdx.x) * 4 + wave; tok < ntok; tok += stride)
      append_token<uint16_t>(a.app, tok, lane);
    return;
  }
  const int l32 = lane & 31, g = lane >> 5;
  // Heads that share the fragment buffer's 128-byte lines (rows 4k .. 4k+3 of a 32-row group) run
  // on one XCD, so their partial-line stores merge in its L2.  Workgroups reach the XCDs
  // round-robin by linear id, whose residue mod 8 is blockIdx.x mod 8 (gridDim.x = H is a multiple
  // of 8 here; otherwise only the merging is lost).
  const int h = __builtin_amdgcn_readfirstlane(xcd_logical_id(blockIdx.x, gridDim.x));
  const int c0 = blockIdx.y * 128;
  const int rb0 = blockIdx.z * a.row_blocks_per_wg;
  const int nrb = (a.M + 31) / 32;
  const int rb_end = min(nrb, rb0 + a.row_blocks_per_wg);

  // stage W_UK[h][0:128][c0:c0+128]: each wave instruction moves 4 rows of 256 bytes; within it the
  // lane's row is lane / 16 and its chunk position lane % 16 (source chunk swizzled by the row)
  const rsrc_t wres = make_rsrc(a.wkv_b + int64_t(h) * (kDn + kDv) * kC, kDn * kC * 2);
  const uint32_t w_voff = uint32_t(lane >> 4) * (kC * 2) + uint32_t((lane & 15) ^ w_swz(lane >> 4)) * 16;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    buf_load16_lds(wres, wt + (wave * 8 + i) * 1024, w_voff, uint32_t((wave * 8 + i) * 4) * (kC * 2) + c0 * 2);

  // q_nope rows of head h (32 per row block, 256 bytes each) go to LDS by DMA, four rows per wave
  // instruction: lane l moves chunk position l % 16 of row l / 16 and fetches the chunk stored
  // there ((l % 16) ^ (row & 15)), so the B-operand reads below (16 lanes, 16 rows, one chunk) hit
  // 16 different bank groups.  Rows past M repeat row M - 1 (their results are not stored).
  const rsrc_t xres = make_rsrc(a.q_nope, uint32_t((int64_t(a.M) * a.H - 1) * a.qn_rs * 2 + kDn * 2));
  auto issue_x = [&](int rb, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = wave * 8 + i * 4 + (lane >> 4);
      const int m = min(rb * 32 + r, a.M - 1);
      const uint32_t src = uint32_t((int64_t(m) * a.H + h) * a.qn_rs * 2) + uint32_t((lane & 15) ^ (r & 15)) * 16;
      buf_load16_lds(xres, xt[buf] + (wave * 8 + i * 4) * 256, src, 0);
    }
  };
  if (rb0 < rb_end) issue_x(rb0, 0);
  // the first column quarter also moves the rope query rows of its row blocks into place: loaded
  // here, with the rest of the first round trip, and stored at the end
  const int pe_r = threadIdx.x >> 3, pe_chunk = threadIdx.x & 7;
  u32x4 pe_v[kQBlocksPerWG];
  const bool pe_copy = blockIdx.y == 0;
  if (pe_copy) {
#pragma unroll
    for (int k = 0; k < kQBlocksPerWG; ++k) {
      const int m = min((rb0 + k) * 32 + pe_r, a.M - 1);
      pe_v[k] = *reinterpret_cast<const u32x4 *>(a.q_pe + (int64_t(m) * a.H + h) * a.qp_rs + pe_chunk * 8);
    }
  }
  wait_vmcnt<0>();
  __syncthreads();

  const int s16 = lane & 15, chalf = (lane >> 4) & 1;
  for (int rb = rb0; rb < rb_end; ++rb) {
    const int m = rb * 32 + l32;
    const bool ok = m < a.M;
    const int buf = (rb - rb0) & 1;
    // the other buffer was last read in the previous iteration, before its closing barrier
    const bool prefetch = rb + 1 < rb_end;  // wavefront-uniform
    if (prefetch) issue_x(rb + 1, buf ^ 1);
    u32x4 xc[kDn / 16];
#pragma unroll
    for (int ks = 0; ks < kDn / 16; ++ks)
      xc[ks] = lds_read16(xt[buf], uint32_t(l32) * 256 + uint32_t((2 * ks + g) ^ (l32 & 15)) * 16);
    // all eight A fragments are read before the MFMA chain so their LDS latency is paid once
    u32x4 af[kDn / 16];
#pragma unroll
    for (int ks = 0; ks < kDn / 16; ++ks) {
      const int row0 = 16 * ks + 8 * g + (s16 >> 2);
      const int chunk = 4 * wave + 2 * chalf + ((s16 & 3) >> 1);
      const int within = (s16 & 1) * 8;
      const uint32_t off0 = row0 * 256 + (chunk ^ w_swz(row0)) * 16 + within;
      const uint32_t off1 = (row0 + 4) * 256 + (chunk ^ w_swz(row0 + 4)) * 16 + within;
      af[ks] = lds_read_tr_pair(wt, off0, off1);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x16 d = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kDn / 16; ++ks) d = mfma32(af[ks], xc[ks], d);
    // D^T[c][m]: lane holds column m, c = 32 wave + 8 (r/4) + 4 g + r % 4; the four elements of
    // register group q are half of the 16-byte chunk (c0 + 32 wave + 8 q) / 8 of the row
    if (ok) {
      unsigned char *dst = reinterpret_cast<unsigned char *>(a.q_frag) + frag_row_offset(m, h, a) + 8 * g;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int chunk = c0 / 8 + 4 * wave + q;
        const u32x2 v{pack_bf16x2(d[4 * q], d[4 * q + 1]), pack_bf16x2(d[4 * q + 2], d[4 * q + 3])};
        *reinterpret_cast<u32x2 *>(dst + (chunk >> 1) * 1024 + (chunk & 1) * 16) = v;
      }
    }
    if (prefetch) {
      wait_vmcnt<0>();  // the next row block's rows (and this block's stores)
      __syncthreads();
    }
  }
  if (pe_copy) {
#pragma unroll
    for (int k = 0; k < kQBlocksPerWG; ++k) {
      const int m = (rb0 + k) * 32 + pe_r;
      if (rb0 + k < rb_end && m < a.M)
        *reinterpret_cast<u32x4 *>(reinterpret_cast<unsigned char *>(a.q_frag) + frag_row_offset(m, h, a) +
                                   (32 + (pe_chunk >> 1)) * 1024 + (pe_chunk & 1) * 16) = pe_v[k];
    }
  }
}

constexpr int kMaxSplits = 4096;  // largest split count the API accepts

// ------------------------------------------------------------------------------------------------
// Split combine and projection out through W_UV in one kernel:
//   o_lat[row, :] = sum_i exp2(m_i - M) o_i[row, :] / sum_i exp2(m_i - M) l_i
//   out[row, e]   = sum_c o_lat[row, c] * W_UV[h][e][c]
// A workgroup owns head h and a range of 16-row groups of m.  W_UV[h] (128 rows of 1 KB) is staged
// in LDS by DMA once; for each group the workgroup combines the split partials of its rows into a
// bf16 tile in LDS, then each wave computes 32 output columns e for the 16 rows with 16x16x32 MFMAs
// (D^T[e][m] = W[e][:] . o[m][:]).  LDS rows of 1 KB are read 16 rows x one 16-byte chunk at a
// time, so chunks are XOR-swizzled inside their 256-byte group by (row & 15).
struct CombineArgs {
  const float *part_ml;    // [rows, splits, 2] (max in log2 units, sum)
  const uint16_t *part_o;  // [rows, splits, 512]
  const uint16_t *wkv_b;   // [H * 256, 512]
  uint16_t *out;           // [rows, 128], rows out_rs elements apart
  int64_t out_rs;
  int32_t H, M, splits;    // rows = M * H, row = m * H + h
  int32_t wgs_per_head, groups_per_wg;
  const int32_t *bal_nb;   // balanced ragged plan: [M] splits used by row m's sequence, else null
};

constexpr int kCombineRows = 16;
constexpr int kCombineLoads = 16;  // partial-row loads a wave keeps in flight

__device__ __forceinline__ uint32_t row_swz16(int row, int chunk) {
  return uint32_t(row) * 1024 + uint32_t((chunk & ~15) | ((chunk & 15) ^ (row & 15))) * 16;
}

// kSingle: one split, whose partial the attention kernel already normalised; the rows are copied
// into the tile four at a time per wave.
template <bool kSingle>
__global__ void __launch_bounds__(256) combine_kernel(CombineArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char wl[kDv * kC * 2];            // 128 KB
  __shared__ __attribute__((aligned(16))) unsigned char ol[kCombineRows * kC * 2];   // 16 KB
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  // the workgroups of one head share W_UV[h] and sit on one XCD
  const int lid = __builtin_amdgcn_readfirstlane(xcd_logical_id(blockIdx.x, gridDim.x));
  const int h = lid / a.wgs_per_head;
  const int groups = (a.M + kCombineRows - 1) / kCombineRows;
  const int g_begin = (lid - h * a.wgs_per_head) * a.groups_per_wg;
  const int g_end = min(groups, g_begin + a.groups_per_wg);

  // W_UV[h] -> LDS: wave w moves rows 32 w .. 32 w + 31, lane p lands at chunk position p of the
  // row and so fetches the chunk stored there
  {
    const rsrc_t wres = make_rsrc(a.wkv_b + (int64_t(h) * (kDn + kDv) + kDn) * kC, kDv * kC * 2);
    for (int i = 0; i < 32; ++i) {
      const int e = wave * 32 + i;
      const uint32_t src_chunk = uint32_t((lane & ~15) | ((lane & 15) ^ (e & 15)));
      buf_load16_lds(wres, wl + e * 1024, src_chunk * 16, uint32_t(e) * 1024);
    }
  }

  const int l16 = lane & 15, q = lane >> 4;
  // one split: the group's rows are copied to the o tile; the next group's rows are requested
  // before this group's projection, so their latency hides behind it
  u32x4 vrow[4];
  auto load_rows = [&](int grp, u32x4 (&v)[4]) __attribute__((always_inline)) {
    const int m0 = grp * kCombineRows;
    const int nrows = min(kCombineRows, a.M - m0);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = min(wave + 4 * k, nrows - 1);
      v[k] = *reinterpret_cast<const u32x4 *>(a.part_o + (int64_t(m0 + r) * a.H + h) * kC + lane * 8);
    }
  };
  if (kSingle && g_begin < g_end) load_rows(g_begin, vrow);
#pragma unroll 1
  for (int grp = g_begin; grp < g_end; ++grp) {
    const int m0 = grp * kCombineRows;
    const int nrows = min(kCombineRows, a.M - m0);
    // (with several splits each wave merges its own rows below, with running maxima)
    if (kSingle) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (wave + 4 * k < nrows) lds_write16(ol, row_swz16(wave + 4 * k, lane), vrow[k]);
      if (grp + 1 < g_end) load_rows(grp + 1, vrow);
    }
    // combine: wave w takes rows w, w + 4, w + 8, w + 12 (NR of them); lane = 16-byte chunk of the
    // row.  The split statistics and partial rows of all NR rows are loaded kCombineLoads at a
    // time (SB splits per row), and merged with a running maximum per row: a batch whose maximum
    // exceeds it rescales the row's sum and denominator first.  So a group costs
    // splits * NR / kCombineLoads memory round trips, with no pass over the statistics before.
    // A balanced ragged batch gives each row the split count its sequence used (bal_nb): the
    // first round does not wait for the counts (it reads slots of the row's own range, stale ones
    // masked), and the later rounds are bounded by them.
    auto combine_rows = [&](auto nr_tag, auto bal_tag) __attribute__((always_inline)) {
      constexpr int NR = decltype(nr_tag)::value;
      constexpr bool kBal = decltype(bal_tag)::value;  // counts per row (balanced ragged plan)
      constexpr int SB = kCombineLoads / NR;
      const uint16_t *po[NR];
      const float *ml[NR];
      float mx[NR], den[NR], acc[NR][8];
      // splits of row k as read (uniform in value, kept in vector registers: a zero the compiler
      // cannot see through keeps the count loads per lane, and nothing uses them before the first
      // round's partial rows are requested), and clamped to [1, splits] for the later rounds
      int ns[NR], lim[NR];
      int zero = 0;
      if constexpr (kBal) asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
#pragma unroll
      for (int k = 0; k < NR; ++k) {
        const int r = min(wave + 4 * k, nrows - 1);  // rows past nrows repeat a valid one, unwritten
        const int64_t row = int64_t(m0 + r) * a.H + h;
        po[k] = a.part_o + row * a.splits * kC + lane * 8;
        ml[k] = a.part_ml + row * a.splits * 2;
        ns[k] = kBal ? a.bal_nb[m0 + r + zero] : a.splits;
        mx[k] = -INFINITY;
        den[k] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[k][e] = 0.f;
      }
      // one round: splits i0 .. i0 + SB - 1 of every row.  The first reads slots of the row's own
      // range without the counts; splits past a row's last repeat it with weight 0 (no branches
      // between the loads); the statistics and partial rows are all requested before any is used
      auto round = [&](int i0, auto first_tag) __attribute__((always_inline)) {
        constexpr bool kFirst = decltype(first_tag)::value;
        u32x4 v[NR][SB];
        f32x2 st[NR][SB];
#pragma unroll
        for (int k = 0; k < NR; ++k)
#pragma unroll
          for (int s = 0; s < SB; ++s)
            st[k][s] = *reinterpret_cast<const f32x2 *>(ml[k] + 2 * min(i0 + s, (kFirst ? a.splits : lim[k]) - 1));
#pragma unroll
        for (int k = 0; k < NR; ++k)
#pragma unroll
          for (int s = 0; s < SB; ++s)
            v[k][s] = *reinterpret_cast<const u32x4 *>(po[k] + int64_t(min(i0 + s, (kFirst ? a.splits : lim[k]) - 1)) * kC);
        // balanced plan: nothing of the merge (which reads the counts) moves above the loads
        if constexpr (kBal) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < NR; ++k) {
          float bm = mx[k];
#pragma unroll
          for (int s = 0; s < SB; ++s) bm = fmaxf(bm, i0 + s < (kFirst ? ns[k] : lim[k]) ? st[k][s][0] : -INFINITY);
          // -inf only while no split of the row has seen a position (a sparse row may never)
          const float alpha = (mx[k] == -INFINITY) ? 0.f : fast_exp2(mx[k] - bm);
          mx[k] = bm;
          den[k] *= alpha;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[k][e] *= alpha;
#pragma unroll
          for (int s = 0; s < SB; ++s) {
            const float mi = st[k][s][0];
            const bool used = i0 + s < (kFirst ? ns[k] : lim[k]) && mi != -INFINITY;
            const float w = used ? fast_exp2(mi - bm) : 0.f;
            // an empty split's o row was never written: zero its bits rather than multiply
            // whatever the memory holds (possibly NaN) by 0
            const uint32_t keep = used ? 0xffffffffu : 0u;
            // (balanced plan: a first-round slot past the row's count may hold a stale sum)
            den[k] = fmaf(w, !kBal || used ? st[k][s][1] : 0.f, den[k]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t x = v[k][s][e] & keep;
              acc[k][2 * e] = fmaf(w, __uint_as_float(x << 16), acc[k][2 * e]);
              acc[k][2 * e + 1] = fmaf(w, __uint_as_float(x & 0xffff0000u), acc[k][2 * e + 1]);
            }
          }
        }
      };
      if constexpr (kBal) {
        round(0, std::true_type{});
        int nmax = 1;
#pragma unroll
        for (int k = 0; k < NR; ++k) {  // scalars now: the counts arrived with the first round
          lim[k] = __builtin_amdgcn_readfirstlane(min(max(ns[k], 1), a.splits));
          nmax = max(nmax, lim[k]);
        }
        for (int i0 = SB; i0 < nmax; i0 += SB) round(i0, std::false_type{});
      } else {  // every row has all the splits: scalar bounds
#pragma unroll
        for (int k = 0; k < NR; ++k) lim[k] = a.splits;
        for (int i0 = 0; i0 < a.splits; i0 += SB) round(i0, std::false_type{});
      }
#pragma unroll
      for (int k = 0; k < NR; ++k) {
        if (wave + 4 * k >= nrows) continue;
        const float inv = den[k] > 0.f ? 1.f / den[k] : 0.f;  // 0: a row no split saw (sparse)
        const u32x4 pk{pack_bf16x2(acc[k][0] * inv, acc[k][1] * inv), pack_bf16x2(acc[k][2] * inv, acc[k][3] * inv),
                       pack_bf16x2(acc[k][4] * inv, acc[k][5] * inv), pack_bf16x2(acc[k][6] * inv, acc[k][7] * inv)};
        lds_write16(ol, row_swz16(wave + 4 * k, lane), pk);
      }
    };
    if (!kSingle) {
      const int nr = wave < nrows ? (nrows - wave + 3) / 4 : 0;  // wavefront-uniform
      using I4 = std::integral_constant<int, 4>;
      using I2 = std::integral_constant<int, 2>;
      using I1 = std::integral_constant<int, 1>;
      if (a.bal_nb) {  // one instantiation (fewer registers held across the kernel's paths)
        if (nr > 0) combine_rows(I4{}, std::true_type{});
      } else {
        if (nr >= 3) combine_rows(I4{}, std::false_type{});
        else if (nr == 2) combine_rows(I2{}, std::false_type{});
        else if (nr == 1) combine_rows(I1{}, std::false_type{});
      }
    }
    // W_UV rows (LDS DMA) before the first use; with one split the next group's four row loads
    // (issued last) may stay in flight
    if (grp == g_begin) {
      if (kSingle && grp + 1 < g_end) wait_vmcnt<4>();
      else wait_vmcnt<0>();
    }
    __syncthreads();

    // D^T[e][m] for e in 32 wave + 16 blk + 0..15: A = W rows (lane: row l % 16, chunk 4 ks + l / 16),
    // B = o rows (lane: row l % 16, same chunk); tile rows past nrows hold stale data and their
    // columns are not stored
    f32x4 d[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int ks = 0; ks < kC / 32; ++ks) {
      const int chunk = 4 * ks + q;
      const u32x4 bo = lds_read16(ol, row_swz16(l16, chunk));
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const u32x4 aw = lds_read16(wl, row_swz16(32 * wave + 16 * blk + l16, chunk));
        d[blk] = mfma16(aw, bo, d[blk]);
      }
    }
    // lane holds D^T[e = 32 wave + 16 blk + 4 q + r][m = m0 + l16], r = 0..3: four consecutive e
    if (l16 < nrows) {
      uint16_t *dst = a.out + (int64_t(m0 + l16) * a.H + h) * a.out_rs + 32 * wave + 4 * q;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const u32x2 v{pack_bf16x2(d[blk][0], d[blk][1]), pack_bf16x2(d[blk][2], d[blk][3])};
        *reinterpret_cast<u32x2 *>(dst + 16 * blk) = v;
      }
    }
    __syncthreads();  // ol is rewritten by the next group
  }
  wait_vmcnt<0>();  // a workgroup without rows still lets its W_UV DMA land before it exits
}

}  // namespace

bool mfma_attn_supported(const AttnCall &c, const char **why) {
  if (c.dtype != MLA_DTYPE_BF16) { *why = "needs bf16"; return false; }
  if (c.C != kC || c.R != kR || c.Dn != kDn || c.Dv != kDv) {
    *why = "needs kv_lora_rank 512, qk_rope_head_dim 64, qk_nope_head_dim 128, v_head_dim 128";
    return false;
  }
  if (c.topk > 0) {
    if (c.page_size > 0) { *why = "index lists over paged caches are not supported"; return false; }
    // one index list per workgroup: its 128 rows must be heads of one query token
    if (!((c.S == 1 && c.H <= kRowsWG) || c.H % kRowsWG == 0)) {
      *why = "needs n_heads a multiple of 128, or seqlen_q 1 and n_heads <= 128";
      return false;
    }
  }
  if (c.page_size > 0) {
    // a tile must lie in one page; page ranges are 32-bit byte counts
    if (c.page_size < kTile || (c.page_size & (c.page_size - 1)) || c.page_size > 65536) {
      *why = "needs a page_size that is a power of two in [32, 65536]";
      return false;
    }
    if (c.max_pages >= (int64_t(1) << 28)) {  // the table row's byte range is 32-bit
      *why = "max_pages_per_seq must be below 2^28";
      return false;
    }
    if ((c.kv_ps << 1) * c.page_size >= (int64_t(1) << 32) || (c.pe_ps << 1) * c.page_size >= (int64_t(1) << 32)) {
      *why = "page_size * position stride must be below 2^31 elements";  // page ranges are byte counts
      return false;
    }
  } else if (c.Tmax * c.kv_ps * 2 >= (int64_t(1) << 32) || c.Tmax * c.pe_ps * 2 >= (int64_t(1) << 32)) {
    // per-sequence buffer ranges are byte counts below 2^32
    *why = "cache_len * position stride must be below 2^31 elements";
    return false;
  }
  if (c.B * c.S * c.H * int64_t(kC) * 2 >= (int64_t(1) << 32)) { *why = "too many query rows"; return false; }
  // strided query rows: byte offsets of the query buffers are 32-bit
  if (c.B * c.S * c.H * std::max(c.q_nope_rs, c.q_pe_rs) * 2 >= (int64_t(1) << 32)) {
    *why = "batch * seqlen_q * n_heads * query row stride too large";
    return false;
  }
  return true;
}

int32_t mfma_attn_splits(const AttnCall &c, int num_cus) {
  // Aim for one workgroup per compute unit; never split below 128 positions per range.
  const int64_t row_blocks = (c.S * c.H + kRowsWG - 1) / kRowsWG;
  const int64_t units = c.B * row_blocks;
  int64_t splits = (num_cus + units / 2) / units;
  const int64_t items = c.topk > 0 ? c.topk : c.end_pos;  // positions, or list entries
  const int64_t max_by_len = (items + 127) / 128;
  if (splits > max_by_len) splits = max_by_len;
  if (splits < 1) splits = 1;
  if (c.page_size > 0) {  // a split may span at most 64 kPageRegs pages
    const int64_t cap = mfma_paged_max_split_len(c);
    splits = std::max<int64_t>(splits, (c.end_pos + cap - 1) / cap);
  }
  if (c.topk > 0) splits = std::max<int64_t>(splits, (c.topk + 64 * kPageRegs - 1) / (64 * kPageRegs));
  if (splits > 4096) splits = 4096;
  return int32_t(splits);
}

int64_t mfma_paged_max_split_len(const AttnCall &c) { return (64 * kPageRegs - 1) * c.page_size; }

bool mfma_attn_plan_ok(const AttnCall &c, const char **why) {
  if (c.splits < 1 || c.splits > kMaxSplits) {
    *why = "num_splits outside [1, 4096]";
    return false;
  }
  if (c.page_size > 0 && (c.split_len % kTile || c.split_len > mfma_paged_max_split_len(c))) {
    *why = "paged splits must be multiples of 32 positions spanning at most 255 pages";
    return false;
  }
  if (c.topk > 0 && c.split_len > 64 * kPageRegs) {
    *why = "a split of an index list may hold at most 256 entries";
    return false;
  }
  // split partials are addressed with 32-bit byte offsets
  if (c.B * c.S * c.H * int64_t(c.splits) * kC * 2 >= (int64_t(1) << 32)) {
    *why = "batch * seqlen_q * n_heads * num_splits too large for the split partials";
    return false;
  }
  return true;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// An odd stride near 0.618 n that is coprime with n: multiples of it modulo n spread any run of
// consecutive indices evenly over [0, n).
static int32_t row_block_stride(int32_t n) {
  if (n <= 2) return 1;
  int32_t s = int32_t(double(n) * 0.6180339887498949) | 1;
  while (std::gcd(s, n) != 1) s += 2;
  return s % n;
}

// Workspace: [query fragments] [split m, l] [split o] [split counts of the balanced plan].
static size_t q_region_bytes(const AttnCall &c) {
  const size_t row_blocks = size_t((c.S * c.H + kRowsWG - 1) / kRowsWG);
  return align256(size_t(c.B) * row_blocks * 4 * kFragBytesPerWave);
}

size_t mfma_attn_workspace(const AttnCall &c) {
  const size_t rows = size_t(c.B * c.S * c.H);
  return q_region_bytes(c) + align256(rows * size_t(c.splits) * 2 * 4) + align256(rows * size_t(c.splits) * kC * 2) +
         (c.bal_target > 0 ? align256(size_t(c.B * c.S) * 4) : 0);
}

hipError_t mfma_absorb_attn(const AttnCall &c) {
  const int64_t rows = c.B * c.S * c.H;
  unsigned char *ws = static_cast<unsigned char *>(c.ws);
  uint16_t *q_frag = reinterpret_cast<uint16_t *>(ws);
  float *part_ml = reinterpret_cast<float *>(ws + q_region_bytes(c));
  uint16_t *part_o = reinterpret_cast<uint16_t *>(ws + q_region_bytes(c) + align256(size_t(rows) * c.splits * 2 * 4));
  int32_t *bal_nb = c.bal_target > 0 ? reinterpret_cast<int32_t *>(ws + q_region_bytes(c) +
                                                                  align256(size_t(rows) * c.splits * 2 * 4) +
                                                                  align256(size_t(rows) * c.splits * kC * 2))
                                     : nullptr;
  const int32_t M = int32_t(c.B * c.S);
  const int32_t row_blocks = int32_t((c.S * c.H + kRowsWG - 1) / kRowsWG);

  AbsorbQArgs qa{static_cast<const uint16_t *>(c.q_nope), static_cast<const uint16_t *>(c.q_pe),
                 static_cast<const uint16_t *>(c.wkv_b), q_frag, int32_t(c.H), M, int32_t(c.S), row_blocks, kQBlocksPerWG,
                 1.f / float(c.S), int32_t(c.q_nope_rs), int32_t(c.q_pe_rs), AppendCall{}};
  if (c.append) qa.app = *c.append;
  const int nrb = (M + 31) / 32;
  const unsigned qz = unsigned((nrb + qa.row_blocks_per_wg - 1) / qa.row_blocks_per_wg);
  hipError_t err = c.append ? launch_kernel(MLA_KERNEL_ABSORB_Q, absorb_q_kernel<true>, dim3(unsigned(c.H), kC / 128 + 1, qz),
                                            dim3(256), 0, c.stream, qa)
                            : launch_kernel(MLA_KERNEL_ABSORB_Q, absorb_q_kernel<false>, dim3(unsigned(c.H), kC / 128, qz),
                                            dim3(256), 0, c.stream, qa);
  if (err != hipSuccess) return err;

  AttnArgs aa{};
  aa.q_frag = q_frag;
  aa.kv = static_cast<const uint16_t *>(c.kv);
  aa.pe = static_cast<const uint16_t *>(c.pe);
  aa.part_ml = part_ml;
  aa.part_o = part_o;
  aa.Tmax = c.Tmax;
  aa.kv_bs = c.kv_bs;
  aa.pe_bs = c.pe_bs;
  aa.kv_rb = int32_t(c.kv_ps * 2);
  aa.pe_rb = int32_t(c.pe_ps * 2);
  aa.S = int32_t(c.S);
  aa.H = int32_t(c.H);
  aa.SH = int32_t(c.S * c.H);
  aa.end_pos = int32_t(c.end_pos);
  aa.seq_lens = c.seq_lens;
  aa.splits = c.splits;
  aa.split_len = int32_t(c.split_len);
  aa.B = int32_t(c.B);
  aa.bal_target = c.bal_target;
  aa.bal_cap = c.page_size > 0 ? int32_t(mfma_paged_max_split_len(c)) : (1 << 30);
  aa.bal_nb = bal_nb;
  aa.row_blocks = row_blocks;
  aa.rb_stride = row_block_stride(row_blocks);
  aa.scale_log2 = c.scale * kLog2e;
  // balanced plan: bal_target chunk workgroups per row block (the plan keeps it >= every chunk
  // count the lengths can produce), else one per (sequence, split)
  const int64_t nwg = (c.bal_target > 0 ? int64_t(c.bal_target) : c.B * int64_t(aa.splits)) * aa.row_blocks;
  if (c.topk > 0) {
    aa.indices = c.indices;
    aa.topk = int32_t(c.topk);
    err = row_blocks == 1
              ? launch_kernel(MLA_KERNEL_ATTN, attn_kernel<kModeSparse, true>, dim3(unsigned(nwg)), dim3(256), 0, c.stream, aa)
              : launch_kernel(MLA_KERNEL_ATTN, attn_kernel<kModeSparse, false>, dim3(unsigned(nwg)), dim3(256), 0, c.stream, aa);
  } else if (c.page_size > 0) {
    aa.block_table = c.block_table;
    aa.log2_page = 0;
    while ((int64_t(1) << aa.log2_page) < c.page_size) ++aa.log2_page;
    aa.max_pages = int32_t(c.max_pages);
    aa.num_pages = int32_t(c.num_pages);
    err = row_blocks == 1
              ? launch_kernel(MLA_KERNEL_ATTN, attn_kernel<kModePaged, true>, dim3(unsigned(nwg)), dim3(256), 0, c.stream, aa)
              : launch_kernel(MLA_KERNEL_ATTN, attn_kernel<kModePaged, false>, dim3(unsigned(nwg)), dim3(256), 0, c.stream, aa);
  } else {
    // one row block: every cache row has a single reader
    err = row_blocks == 1
              ? launch_kernel(MLA_KERNEL_ATTN, attn_kernel<kModeContig, true>, dim3(unsigned(nwg)), dim3(256), 0, c.stream, aa)
              : launch_kernel(MLA_KERNEL_ATTN, attn_kernel<kModeContig, false>, dim3(unsigned(nwg)), dim3(256), 0, c.stream, aa);
  }
  if (err != hipSuccess) return err;

  // split combine and W_UV projection: enough workgroups per head to fill the chip, each reusing
  // its W_UV[h] copy in LDS over up to groups_per_wg 16-row groups
  const int groups = (M + kCombineRows - 1) / kCombineRows;
  const int per_head = int(std::max<int64_t>(1, std::min<int64_t>(groups, (512 + c.H - 1) / c.H)));
  CombineArgs ca{part_ml, part_o, static_cast<const uint16_t *>(c.wkv_b), static_cast<uint16_t *>(c.out), c.out_rs,
                 int32_t(c.H), M, c.splits, per_head, (groups + per_head - 1) / per_head, bal_nb};
  const dim3 grid(unsigned(int64_t(c.H) * per_head));
  return c.splits == 1 ? launch_kernel(MLA_KERNEL_COMBINE, combine_kernel<true>, grid, dim3(256), 0, c.stream, ca)
                       : launch_kernel(MLA_KERNEL_COMBINE, combine_kernel<false>, grid, dim3(256), 0, c.stream, ca);
}

}  // namespace mla
