// Matrix-core latent KV expansion ("Latent KV expansion with split", kernelindex.com op 064) for
// kv_lora_rank 512, qk_nope_head_dim 128, v_head_dim 128, bf16 storage, fp32 accumulation.
//
//   n[t, :]   = c_kv[t, :] / sqrt(mean(c_kv[t, :]^2) + eps) * rms_w
//   y[t, j]   = sum_c n[t, c] * wkv_b[j, c]
//   k_nope[h, t, :] = y[t, 256 h .. 256 h + 127],   v[h, t, :] = y[t, 256 h + 128 .. 256 h + 255]
//
// Two kernels:
//   1. expand_prep_kernel  once per token: n[t, :] rounded to bf16, into the workspace; every head
//                          reuses it.
//   2. expand_kernel       y = n . wkv_b^T per (128 tokens, one head), two workgroups per compute
//                          unit so one's waits and epilogue overlap the other's MFMAs.  Both
//                          operands stream into LDS by DMA through a three-stage ring of 32-column
//                          tiles; the epilogue goes through LDS so every global store writes whole
//                          256-byte K / V rows with streaming (non-temporal) stores.
//
// Output rows: input token t = b * S_in + s lands in row b * out_seq_stride + out_row0 + s of each
// head's block.  The plain expansion writes row t; the naive path's cache append ("Naive vs Absorb
// Attention Implementations in DeepSeek-V3", section "Memory Layout and Cache Structure": keys and
// values are cached at full width) writes the new tokens' rows of the head-major caches
// [H, Bmax, Tmax, 128], and the prep kernel copies their rope keys into the rope cache alongside.
#include "common.h"
#include "launch.h"
#include "mfma_common.h"
#include "../../include/mla_absorb.h"

namespace mla {
namespace {

constexpr int kC = 512;
constexpr int kDn = 128;
constexpr int kDv = 128;
constexpr int kTT = 128;                   // tokens per workgroup
constexpr int kKC = 32;                    // contraction columns per stage
constexpr int kStages = 3;
constexpr int kWTile = 256 * kKC * 2;      // 16 KB: wkv_b rows of the head (K_nope then V)
constexpr int kNTile = kTT * kKC * 2;      // 8 KB: n rows of the token block
constexpr int kStageBytes = kWTile + kNTile;
constexpr int kChunks = kC / kKC;          // 16
constexpr int kWaves = 4;
constexpr int kWDma = kWTile / 1024 / kWaves;  // 1 KB DMA instructions per wave per W tile (4)
constexpr int kNDma = kNTile / 1024 / kWaves;  // per n tile (2)
constexpr int kEpiPitch = 272;             // bytes per staged output row (256 + 16 pad)
constexpr int kEpiWave = 64 * kEpiPitch;   // 17 KB per wave
constexpr int kLds = (kStages * kStageBytes > kWaves * kEpiWave) ? kStages * kStageBytes : kWaves * kEpiWave;
static_assert(2 * kLds <= 160 * 1024, "two workgroups share a compute unit");

__host__ __device__ __forceinline__ size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Row of an output block that input token t goes to (see the header).
__device__ __forceinline__ uint32_t out_row(uint32_t t, uint32_t S_in, uint32_t seq_stride, uint32_t row0) {
  const uint32_t b = t / S_in;
  return b * seq_stride + row0 + (t - b * S_in);
}

// ---- 1. per-token prep --------------------------------------------------------------------------
struct PrepArgs {
  const uint16_t *c_kv;   // [T, 512]
  const uint16_t *rms_w;  // [512]
  uint16_t *xn;           // [T, 512] workspace
  const uint16_t *k_pe;   // [T, R] or null
  uint16_t *pe_out;       // [out_rows, R] or null
  int32_t T, R, S_in, seq_stride, row0;
  float eps;
};

// One wave per token row: lane l owns columns 8 l .. 8 l + 7.  n = c_kv * rms_w / rms, rounded once.
// With a rope cache, lanes 0 .. R / 8 - 1 also copy the token's rope key row to its cache row.
__global__ void __launch_bounds__(256) expand_prep_kernel(PrepArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= a.T) return;
  const uint16_t *__restrict__ c_kv = a.c_kv;
  const uint16_t *__restrict__ rms_w = a.rms_w;
  uint16_t *__restrict__ xn = a.xn;
  const float eps = a.eps;
  if (a.pe_out && lane < a.R / 8) {
    const u32x4 pv = *reinterpret_cast<const u32x4 *>(a.k_pe + int64_t(t) * a.R + lane * 8);
    const uint32_t r = out_row(uint32_t(t), uint32_t(a.S_in), uint32_t(a.seq_stride), uint32_t(a.row0));
    *reinterpret_cast<u32x4 *>(a.pe_out + int64_t(r) * a.R + lane * 8) = pv;
  }
  const u32x4 xv = *reinterpret_cast<const u32x4 *>(c_kv + int64_t(t) * kC + lane * 8);
  const u32x4 wv = *reinterpret_cast<const u32x4 *>(rms_w + lane * 8);
  float x[8], ss = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = __uint_as_float(xv[e] << 16);
    x[2 * e + 1] = __uint_as_float(xv[e] & 0xffff0000u);
    ss = fmaf(x[2 * e], x[2 * e], fmaf(x[2 * e + 1], x[2 * e + 1], ss));
  }
  const float inv = 1.f / sqrtf(wave_sum(ss) * (1.f / kC) + eps);
  u32x4 out;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float w0 = __uint_as_float(wv[e] << 16), w1 = __uint_as_float(wv[e] & 0xffff0000u);
    out[e] = pack_bf16x2(x[2 * e] * inv * w0, x[2 * e + 1] * inv * w1);
  }
  *reinterpret_cast<u32x4 *>(xn + int64_t(t) * kC + lane * 8) = out;
}

// ---- 2. projection ------------------------------------------------------------------------------
struct ExpandArgs {
  const uint16_t *xn;     // [T, 512] normalised latent n, bf16
  const uint16_t *wkv_b;  // [H * 256, 512]
  uint16_t *k_nope;       // [H, out_rows, 128]
  uint16_t *v;            // [H, out_rows, 128]
  int32_t T, H, tblocks;
  int32_t S_in, seq_stride, row0, out_rows;  // output placement (see the header)
  int32_t grouped;        // 1: workgroups run in blocks of 8 heads x 4 token blocks (see below)
};

// Operand tiles have 64-byte rows (4 chunks of 16 bytes): four rows per 64-bank period.  A
// ds_read_b128 serves 16 lanes = 16 consecutive rows at once; XOR-ing the chunk with
// (row >> 2) & 3 gives rows r, r+4, r+8, r+12 (which share a period slot) four different chunks.
__device__ __forceinline__ int op_swz(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ uint32_t tile_off(int row, int chunk) {
  return uint32_t(row) * (kKC * 2) + uint32_t(chunk ^ op_swz(row)) * 16;
}

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
expand_kernel(ExpandArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kLds];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, g = lane >> 5;
  // Order: each XCD takes a contiguous range of logical ids, and (when the sizes allow) every 64
  // consecutive ids form a block of 8 heads x 8 token blocks, so the 64 workgroups an XCD runs at
  // once (two per compute unit) read 2 MB of wkv_b and 1 MB of n between them, reused from its L2.
  const int lid = __builtin_amdgcn_readfirstlane(xcd_logical_id(blockIdx.x, gridDim.x));
  int h, tb;
  if (a.grouped) {
    const int grp = lid >> 6, in = lid & 63, tgroups = a.tblocks >> 3;
    const int hg = grp / tgroups;
    h = __builtin_amdgcn_readfirstlane(hg * 8 + (in >> 3));
    tb = __builtin_amdgcn_readfirstlane((grp - hg * tgroups) * 8 + (in & 7));
  } else {
    h = __builtin_amdgcn_readfirstlane(lid / a.tblocks);
    tb = __builtin_amdgcn_readfirstlane(lid - h * a.tblocks);
  }
  const int t0 = tb * kTT;
  const int wt = wave & 1;   // token half of this wave (64 tokens)
  const int wj = wave >> 1;  // 0: K_nope features, 1: V features

  // DMA: one wave instruction moves 16 rows x 64 bytes; lane l lands at chunk position l % 4 of
  // row l / 4 and fetches the chunk stored there.  Wave w moves W rows 64 w .. 64 w + 63 (wkv_b
  // rows of head h) and n rows 32 w .. 32 w + 31 (tokens t0 ..; rows past T read 0).
  const int drow = lane >> 2;
  const uint32_t dchunk = uint32_t((lane & 3) ^ op_swz(drow)) * 16;  // op_swz(16 i + drow) == op_swz(drow)
  const rsrc_t wres = make_rsrc(a.wkv_b + int64_t(h) * (kDn + kDv) * kC, (kDn + kDv) * kC * 2);
  const rsrc_t xres = make_rsrc(a.xn + int64_t(t0) * kC, uint32_t(min(kTT, a.T - t0)) * (kC * 2));
  const uint32_t w_voff = uint32_t(wave * 64 + drow) * (kC * 2) + dchunk;
  const uint32_t n_voff = uint32_t(wave * 32 + drow) * (kC * 2) + dchunk;
  auto issue = [&](int kc) __attribute__((always_inline)) {
    unsigned char *st = smem + (kc % kStages) * kStageBytes;
    // row offsets stay in the per-lane offset, which the buffer range check always covers
#pragma unroll
    for (int i = 0; i < kWDma; ++i)
      buf_load16_lds(wres, st + (wave * 64 + i * 16) * (kKC * 2), w_voff + uint32_t(i * 16) * (kC * 2),
                     uint32_t(kc * kKC * 2));
#pragma unroll
    for (int i = 0; i < kNDma; ++i)
      buf_load16_lds(xres, st + kWTile + (wave * 32 + i * 16) * (kKC * 2), n_voff + uint32_t(i * 16) * (kC * 2),
                     uint32_t(kc * kKC * 2));
  };

  // operand reads: every operand row is 32 k + l32 (+ a multiple of 32), so it shares the swizzle of l32
  uint32_t rd_off[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) rd_off[ks] = tile_off(l32, 2 * ks + g);
  const uint32_t a_base = uint32_t(wj * 128) * (kKC * 2);
  const uint32_t b_base = kWTile + uint32_t(wt * 64) * (kKC * 2);

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int k = 0; k < 2; ++k) acc[i][k] = f32x16{};

#pragma unroll
  for (int kc = 0; kc < kStages - 1; ++kc) issue(kc);

  constexpr int kDma = kWDma + kNDma;  // DMA instructions per wave per chunk
#pragma unroll 1
  for (int kc = 0; kc < kChunks; ++kc) {
    // chunk kc must have landed (chunk kc+1 may still be in flight); after the barrier every wave
    // is done with chunk kc-1, whose stage takes chunk kc+2
    if (kc + 1 < kChunks) wait_vmcnt<kDma>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    if (kc + kStages - 1 < kChunks) issue(kc + kStages - 1);

    const unsigned char *stage = smem + (kc % kStages) * kStageBytes;
    // fragments of k-step 1 are read while the 8 MFMAs of k-step 0 run
    u32x4 af[2][4], bf[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) af[ks][jb] = lds_read16(stage, a_base + jb * 32 * (kKC * 2) + rd_off[ks]);
#pragma unroll
      for (int k = 0; k < 2; ++k) bf[ks][k] = lds_read16(stage, b_base + k * 32 * (kKC * 2) + rd_off[ks]);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int jb = 0; jb < 4; ++jb)
#pragma unroll
        for (int k = 0; k < 2; ++k) acc[jb][k] = mfma32(af[ks][jb], bf[ks][k], acc[jb][k]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();  // every wave is done with the stages before the epilogue reuses them

  // D^T[j][t] tiles: lane holds t = 64 wt + 32 k + l32, j = 128 wj + 32 jb + 8 (r/4) + 4 g + r % 4
  unsigned char *epi = smem + wave * kEpiWave;
  const uint32_t epi_lane = uint32_t(l32) * kEpiPitch + 8 * g;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x2 v{pack_bf16x2(agpr_read(acc[jb][k][4 * q]), agpr_read(acc[jb][k][4 * q + 1])),
                      pack_bf16x2(agpr_read(acc[jb][k][4 * q + 2]), agpr_read(acc[jb][k][4 * q + 3]))};
        lds_write8(epi, epi_lane + uint32_t(32 * k) * kEpiPitch + (32 * jb + 8 * q) * 2, v);
      }
    }
  }
  // same wavefront wrote these rows; LDS operations of one wavefront complete in order.  Each store
  // writes 4 token rows (16 lanes x 16 bytes each) to their output rows; rows past T get an offset
  // outside the head's block, and the store drops them.
  // (the descriptor is re-scalarised: it must live in scalar registers, or every store becomes a
  // loop over lanes)
  const rsrc_t ores = make_rsrc((wj == 0 ? a.k_nope : a.v) + int64_t(h) * a.out_rows * 128,
                                uint32_t(a.out_rows) * 256);
  const uint32_t rd_lane = uint32_t(lane >> 4) * kEpiPitch + (lane & 15) * 16;
  // this lane's token at store 0, its sequence and its index in the sequence
  uint32_t tok = uint32_t(t0 + wt * 64 + (lane >> 4));
  uint32_t sb = tok / uint32_t(a.S_in);
  uint32_t ss = tok - sb * uint32_t(a.S_in);
#pragma unroll 8
  for (int it = 0; it < 16; ++it) {
    const u32x4 v = lds_read16(epi, rd_lane + it * 4 * kEpiPitch);
    const uint32_t row = sb * uint32_t(a.seq_stride) + uint32_t(a.row0) + ss;
    const uint32_t voff = tok < uint32_t(a.T) ? row * 256u + (lane & 15) * 16 : 0x80000000u;
    buf_store16_nt(ores, v, voff, 0);
    tok += 4;
    ss += 4;
    while (ss >= uint32_t(a.S_in)) {  // at most once unless a sequence holds fewer than 4 tokens
      ss -= uint32_t(a.S_in);
      ++sb;
    }
  }
}

}  // namespace

bool mfma_expand_supported(const ExpandCall &c, const char **why) {
  if (c.dtype != MLA_DTYPE_BF16) { *why = "needs bf16"; return false; }
  if (c.C != kC || c.Dn != kDn || c.Dv != kDv) {
    *why = "needs kv_lora_rank 512, qk_nope_head_dim 128, v_head_dim 128";
    return false;
  }
  if (c.T > (int64_t(1) << 22)) { *why = "n_tokens must be at most 4194304"; return false; }
  // output offsets within one head's block are 32-bit byte counts below 2^31
  if (c.out_rows > (int64_t(1) << 23)) { *why = "output rows per head must be at most 8388608"; return false; }
  if (c.k_pe && (c.R % 8 != 0 || c.R > 512)) { *why = "rope width must be a multiple of 8 up to 512"; return false; }
  return true;
}

// Workspace: n [T x 512] bf16.
size_t mfma_expand_workspace(const ExpandCall &c) { return align256(size_t(c.T) * kC * 2); }

hipError_t mfma_expand_kv(const ExpandCall &c) {
  uint16_t *xn = static_cast<uint16_t *>(c.ws);
  PrepArgs p{static_cast<const uint16_t *>(c.c_kv), static_cast<const uint16_t *>(c.rms_w), xn,
             static_cast<const uint16_t *>(c.k_pe), static_cast<uint16_t *>(c.pe_out), int32_t(c.T),
             int32_t(c.R), int32_t(c.S_in), int32_t(c.out_seq_stride), int32_t(c.out_row0), c.eps};
  hipError_t err = launch_kernel(MLA_KERNEL_EXPAND_PREP, expand_prep_kernel, dim3(unsigned((c.T + 3) / 4)), dim3(256),
                                 0, c.stream, p);
  if (err != hipSuccess) return err;
  const int32_t tblocks = int32_t((c.T + kTT - 1) / kTT);
  ExpandArgs a{xn, static_cast<const uint16_t *>(c.wkv_b), static_cast<uint16_t *>(c.k_nope),
               static_cast<uint16_t *>(c.v), int32_t(c.T), int32_t(c.H), tblocks,
               int32_t(c.S_in), int32_t(c.out_seq_stride), int32_t(c.out_row0), int32_t(c.out_rows),
               (c.H % 8 == 0 && tblocks % 8 == 0) ? 1 : 0};
  return launch_kernel(MLA_KERNEL_EXPAND, expand_kernel, dim3(unsigned(int64_t(tblocks) * c.H)), dim3(kWaves * 64),
                       0, c.stream, a);
}

}  // namespace mla
