// Matrix-core latent KV expansion ("Latent KV expansion with split", kernelindex.com op 064) for
// kv_lora_rank 512, qk_nope_head_dim 128, v_head_dim 128, bf16 storage, fp32 accumulation.
//
//   n[t, :]   = c_kv[t, :] / sqrt(mean(c_kv[t, :]^2) + eps) * rms_w
//   y[t, j]   = sum_c n[t, c] * wkv_b[j, c]
//   k_nope[h, t, :] = y[t, 256 h .. 256 h + 127],   v[h, t, :] = y[t, 256 h + 128 .. 256 h + 255]
//
// One workgroup produces 256 tokens x one head (all 256 output features of that head), so its
// K_nope and V blocks are two contiguous 64 KB regions.  The per-column weight is applied while
// staging c_kv into LDS (bf16(c_kv * w)); the per-token 1/rms factor is accumulated on the way
// and applied in fp32 in the epilogue.  The epilogue goes through LDS so every global store is a
// full 16-byte, fully coalesced write.
#include "common.h"
#include "launch.h"
#include "mfma_common.h"
#include "../../include/mla_absorb.h"

namespace mla {
namespace {

constexpr int kC = 512;
constexpr int kDn = 128;
constexpr int kDv = 128;
constexpr int kTT = 256;        // tokens per workgroup
constexpr int kKC = 64;         // contraction columns per stage
constexpr int kStageHalf = kTT * kKC * 2;  // 32 KB: one operand tile of a stage
constexpr int kStage = 2 * kStageHalf;     // W tile + n tile
constexpr int kEpiPitch = 272;             // bytes per staged output row (256 + 16 pad)
constexpr int kEpiWave = 128 * kEpiPitch;  // 34 KB per wave
constexpr int kLds = (2 * kStage > 4 * kEpiWave) ? 2 * kStage : 4 * kEpiWave;

struct ExpandArgs {
  const uint16_t *c_kv;   // [T, 512]
  const uint16_t *rms_w;  // [512]
  const uint16_t *wkv_b;  // [H * 256, 512]
  uint16_t *k_nope;       // [H, T, 128]
  uint16_t *v;            // [H, T, 128]
  int32_t T, H, tblocks;
  float eps;
};

// Operand tiles have 128-byte rows (8 chunks of 16 bytes): two rows per 64-bank period.  A
// ds_read_b128 serves 16 lanes = 16 consecutive rows at once, so chunks are XOR-swizzled by
// (row >> 1) & 7: rows of equal parity then use eight different chunk slots.
__device__ __forceinline__ int op_swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ uint32_t tile_off(int row, int chunk) {
  return uint32_t(row) * (kKC * 2) + uint32_t(chunk ^ op_swz(row)) * 16;
}

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
expand_kernel(ExpandArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kLds];
  __shared__ float rs[kTT];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, g = lane >> 5;
  const int tb = blockIdx.x % a.tblocks;
  const int h = blockIdx.x / a.tblocks;
  const int t0 = tb * kTT;
  const int wt = wave & 1;   // token half of this wave
  const int wj = wave >> 1;  // 0: K_nope features, 1: V features

  // W rows of this head; each wave instruction moves 8 rows x 128 bytes.  Within instruction i
  // the lane's row is 8 (8 wave + i) + lane / 8 and its chunk position lane % 8, so the source
  // chunk (lane % 8) ^ op_swz(row) depends only on the lane and the parity of i.
  const rsrc_t wres = make_rsrc(a.wkv_b + int64_t(h) * (kDn + kDv) * kC, (kDn + kDv) * kC * 2);
  uint32_t w_lane_off[2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
    w_lane_off[par] = uint32_t(lane >> 3) * (kC * 2) + uint32_t((lane & 7) ^ op_swz(8 * par + (lane >> 3))) * 16;
  // c_kv staging: thread owns rows srow + 32 i and chunk schunk of every stage; rows past T read 0
  const int srow = threadIdx.x >> 3, schunk = threadIdx.x & 7;
  const rsrc_t xres = make_rsrc(a.c_kv + int64_t(t0) * kC, uint32_t(min(kTT, a.T - t0)) * (kC * 2));
  const rsrc_t rwres = make_rsrc(a.rms_w, kC * 2);
  const uint32_t x_lane_off = uint32_t(srow) * (kC * 2) + schunk * 16;
  float ss[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  u32x4 xr[8];

  auto issue_w = [&](int kc, int buf) {
    unsigned char *dst = smem + buf * kStage + wave * 8 * 1024;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      buf_load16_lds(wres, dst + i * 1024, w_lane_off[i & 1], uint32_t((wave * 8 + i) * 8 * (kC * 2) + kc * (kKC * 2)));
  };
  auto load_x = [&](int kc) {
#pragma unroll
    for (int i = 0; i < 8; ++i) xr[i] = buf_load16(xres, x_lane_off, uint32_t(i * 32 * (kC * 2) + kc * (kKC * 2)));
  };
  const uint32_t st_off0 = tile_off(srow, schunk);  // rows srow + 32 i share the swizzle
  auto store_x = [&](int kc, int buf) {
    const u32x4 wv = buf_load16(rwres, schunk * 16, kc * (kKC * 2));
    float w[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w[2 * e] = __uint_as_float(wv[e] << 16);
      w[2 * e + 1] = __uint_as_float(wv[e] & 0xffff0000u);
    }
    unsigned char *dst = smem + buf * kStage + kStageHalf;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(xr[i][e] << 16);
        x[2 * e + 1] = __uint_as_float(xr[i][e] & 0xffff0000u);
      }
      float acc = ss[i];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf(x[e], x[e], acc);
      ss[i] = acc;
      const u32x4 pk{pack_bf16x2(x[0] * w[0], x[1] * w[1]), pack_bf16x2(x[2] * w[2], x[3] * w[3]),
                     pack_bf16x2(x[4] * w[4], x[5] * w[5]), pack_bf16x2(x[6] * w[6], x[7] * w[7])};
      lds_write16(dst, st_off0 + i * 32 * (kKC * 2), pk);
    }
  };

  // operand reads: every operand row is 32 k + l32 (+ a multiple of 32), so it shares the swizzle of l32
  uint32_t rd_off[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) rd_off[ks] = tile_off(l32, 2 * ks + g);
  const uint32_t a_base = uint32_t(wj * 128) * (kKC * 2);
  const uint32_t b_base = kStageHalf + uint32_t(wt * 128) * (kKC * 2);

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[i][k] = f32x16{};

  issue_w(0, 0);
  load_x(0);
  store_x(0, 0);
  wait_vmcnt<0>();
  __syncthreads();

  constexpr int nk = kC / kKC;
#pragma unroll 1
  for (int kc = 0; kc < nk; ++kc) {
    const int buf = kc & 1;
    if (kc + 1 < nk) {
      issue_w(kc + 1, buf ^ 1);
      load_x(kc + 1);
    }
    const unsigned char *stage = smem + buf * kStage;
    // fragments of k-step ks+1 are read while the 16 MFMAs of k-step ks run
    u32x4 af[2][4], bf[2][4];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) af[0][jb] = lds_read16(stage, a_base + jb * 32 * (kKC * 2) + rd_off[0]);
#pragma unroll
    for (int k = 0; k < 4; ++k) bf[0][k] = lds_read16(stage, b_base + k * 32 * (kKC * 2) + rd_off[0]);
#pragma unroll
    for (int ks = 0; ks < kKC / 16; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < kKC / 16) {
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) af[cur ^ 1][jb] = lds_read16(stage, a_base + jb * 32 * (kKC * 2) + rd_off[ks + 1]);
#pragma unroll
        for (int k = 0; k < 4; ++k) bf[cur ^ 1][k] = lds_read16(stage, b_base + k * 32 * (kKC * 2) + rd_off[ks + 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int jb = 0; jb < 4; ++jb)
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[jb][k] = mfma32(af[cur][jb], bf[cur][k], acc[jb][k]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kc + 1 < nk) store_x(kc + 1, buf ^ 1);
    wait_vmcnt<0>();
    __syncthreads();
  }

  // 1 / rms per token: the 8 threads of a row hold disjoint column slices of its sum of squares
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float v = ss[i];
    v += __shfl_xor(v, 1, 64);
    v += __shfl_xor(v, 2, 64);
    v += __shfl_xor(v, 4, 64);
    if (schunk == 0) rs[srow + 32 * i] = 1.f / sqrtf(v * (1.f / kC) + a.eps);
  }
  __syncthreads();

  // D^T[j][t] tiles: lane holds t = 32 k + l32, j = 32 jb + 8 (r/4) + 4 g + r % 4
  unsigned char *epi = smem + wave * kEpiWave;
  const uint32_t epi_lane = uint32_t(l32) * kEpiPitch + 8 * g;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float sc = rs[wt * 128 + 32 * k + l32];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x2 v{pack_bf16x2(agpr_read(acc[jb][k][4 * q]) * sc, agpr_read(acc[jb][k][4 * q + 1]) * sc),
                      pack_bf16x2(agpr_read(acc[jb][k][4 * q + 2]) * sc, agpr_read(acc[jb][k][4 * q + 3]) * sc)};
        lds_write8(epi, epi_lane + uint32_t(32 * k) * kEpiPitch + (32 * jb + 8 * q) * 2, v);
      }
    }
  }
  __syncthreads();
  const int rows_valid = max(0, min(128, a.T - (t0 + wt * 128)));
  const rsrc_t ores = make_rsrc((wj == 0 ? a.k_nope : a.v) + (int64_t(h) * a.T + t0 + wt * 128) * 128,
                                uint32_t(rows_valid) * 256);
  const uint32_t rd_lane = uint32_t(lane >> 4) * kEpiPitch + (lane & 15) * 16;
  const uint32_t st_lane = uint32_t(lane >> 4) * 256 + (lane & 15) * 16;
#pragma unroll 8
  for (int it = 0; it < 32; ++it) {
    const u32x4 v = lds_read16(epi, rd_lane + it * 4 * kEpiPitch);
    buf_store16(ores, v, st_lane, uint32_t(it * 1024));
  }
}

}  // namespace

bool mfma_expand_supported(const ExpandCall &c, const char **why) {
  if (c.dtype != MLA_DTYPE_BF16) { *why = "needs bf16"; return false; }
  if (c.C != kC || c.Dn != kDn || c.Dv != kDv) {
    *why = "needs kv_lora_rank 512, qk_nope_head_dim 128, v_head_dim 128";
    return false;
  }
  if (c.T > (int64_t(1) << 30)) { *why = "too many tokens"; return false; }
  return true;
}

hipError_t mfma_expand_kv(const ExpandCall &c) {
  ExpandArgs a{static_cast<const uint16_t *>(c.c_kv), static_cast<const uint16_t *>(c.rms_w),
               static_cast<const uint16_t *>(c.wkv_b), static_cast<uint16_t *>(c.k_nope), static_cast<uint16_t *>(c.v),
               int32_t(c.T), int32_t(c.H), int32_t((c.T + kTT - 1) / kTT), c.eps};
  return launch_kernel(MLA_KERNEL_EXPAND, expand_kernel, dim3(unsigned(int64_t(a.tblocks) * c.H)), dim3(256), 0,
                       c.stream, a);
}

}  // namespace mla
