// The rows a cache append writes for one new token (page "Naive vs Absorb Attention
// Implementations in DeepSeek-V3", section "Memory Layout and Cache Structure": kv_cache holds each
// position's compressed latent, pe_cache its rotary key; the latent is stored RMS-normalised, the
// norm of "Latent KV expansion with split"):
//
//   kv_cache[b, p, :] = c_kv_new[b, s, :] / sqrt(mean(c_kv_new[b, s, :]^2) + eps) * rms_w
//   pe_cache[b, p, :] = k_pe_new[b, s, :]
//
// with p = end_pos - S + s, or seq_lens[b] - S + s (clamped to [S, end_pos]) for a ragged batch.
// Shared by the stand-alone append kernel and the query-absorption kernel of the fused call, so
// that both write the same bits.
#pragma once

#include "common.h"
#include "launch.h"

namespace mla {

// Element offsets of token tok's destination rows in kv_cache and pe_cache.
__device__ __forceinline__ void append_dest(const AppendCall &a, int64_t tok, int64_t &kv_off, int64_t &pe_off) {
  const int64_t b = tok / a.S, s = tok - b * a.S;
  int64_t end_pos = a.end_pos;
  if (a.seq_lens) {  // same clamp as the ragged attention: [S, end_pos]
    end_pos = a.seq_lens[b];
    if (end_pos < a.S) end_pos = a.S;
    if (end_pos > a.end_pos) end_pos = a.end_pos;
  }
  const int64_t p = end_pos - a.S + s;
  if (a.page_size > 0) {
    int64_t pg = a.block_table[b * a.max_pages + p / a.page_size];
    pg = pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);
    const int64_t row = pg * a.page_size + p % a.page_size;
    kv_off = row * a.kv_ps;
    pe_off = row * a.pe_ps;
  } else {
    kv_off = b * a.kv_bs + p * a.kv_ps;
    pe_off = b * a.pe_bs + p * a.pe_ps;
  }
}

typedef __attribute__((ext_vector_type(4))) uint32_t append_v4;

// Element e of a 16-byte chunk as fp32, and the chunk of 16 / sizeof(T) values rounded to T.
template <typename T> struct ChunkOf;
template <> struct ChunkOf<float> {
  static constexpr int E = 4;
  static __device__ __forceinline__ float get(const append_v4 &v, int e) { return __uint_as_float(v[e]); }
  static __device__ __forceinline__ void put(append_v4 &v, int e, float f) { v[e] = __float_as_uint(f); }
};
template <> struct ChunkOf<uint16_t> {
  static constexpr int E = 8;
  static __device__ __forceinline__ float get(const append_v4 &v, int e) {
    return bf16_to_f32(uint16_t(v[e >> 1] >> (16 * (e & 1))));
  }
  static __device__ __forceinline__ void put(append_v4 &v, int e, float f) {
    const uint32_t h = f32_to_bf16(f);
    v[e >> 1] = (e & 1) ? ((v[e >> 1] & 0xffffu) | (h << 16)) : ((v[e >> 1] & 0xffff0000u) | h);
  }
};

// One wavefront writes token tok's two rows.  Lane l takes the 16-byte chunks l, l + 64, ... of a
// row (one chunk per lane for a 512-wide bf16 latent), so every load of the row is in flight at
// once; the sum of squares runs over the lane's elements in order, then across the wavefront.
// fp32 arithmetic, stores rounded to T.
template <typename T>
__device__ __forceinline__ void append_token(const AppendCall &a, int64_t tok, int lane) {
  using Ch = ChunkOf<T>;
  constexpr int E = Ch::E;
  const append_v4 *__restrict__ x = reinterpret_cast<const append_v4 *>(static_cast<const T *>(a.c_kv_new) + tok * a.C);
  const append_v4 *__restrict__ w = reinterpret_cast<const append_v4 *>(a.rms_w);
  int64_t kv_off, pe_off;
  append_dest(a, tok, kv_off, pe_off);
  const int64_t nch = a.C / E;
  float ss = 0.f;
  for (int64_t ch = lane; ch < nch; ch += 64) {
    const append_v4 v = x[ch];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float f = Ch::get(v, e);
      ss = fmaf(f, f, ss);
    }
  }
  const float inv = 1.f / sqrtf(wave_sum(ss) / float(a.C) + a.eps);
  append_v4 *kv = reinterpret_cast<append_v4 *>(static_cast<T *>(a.kv_cache) + kv_off);
  for (int64_t ch = lane; ch < nch; ch += 64) {
    const append_v4 v = x[ch], wv = w[ch];
    append_v4 o{};
#pragma unroll
    for (int e = 0; e < E; ++e) Ch::put(o, e, Ch::get(v, e) * inv * Ch::get(wv, e));
    kv[ch] = o;
  }
  const append_v4 *kp = reinterpret_cast<const append_v4 *>(static_cast<const T *>(a.k_pe_new) + tok * a.R);
  append_v4 *pe = reinterpret_cast<append_v4 *>(static_cast<T *>(a.pe_cache) + pe_off);
  for (int64_t ch = lane; ch < a.R / E; ch += 64) pe[ch] = kp[ch];
}

}  // namespace mla
