// Cache append: the step just before absorb attention writes the new tokens' rows into the two
// caches the absorb path reads (page "Naive vs Absorb Attention Implementations in DeepSeek-V3",
// section "Memory Layout and Cache Structure": kv_cache holds each position's compressed latent,
// pe_cache its rotary key).  The latent is stored RMS-normalised (the norm of "Latent KV expansion
// with split", applied once per token here so that attention reads normalised rows):
//
//   kv_cache[b, p, :] = c_kv_new[b, s, :] / sqrt(mean(c_kv_new[b, s, :]^2) + eps) * rms_w
//   pe_cache[b, p, :] = k_pe_new[b, s, :]
//
// with p = end_pos - S + s, or seq_lens[b] - S + s for a ragged batch.  With paged caches the row
// of position p is row p % page_size of the sequence's page for p (the block table's id, clamped
// into the pool).  One wavefront per token; fp32 arithmetic, stores rounded to the cache's
// element type.
#include "common.h"
#include "launch.h"
#include "../../include/mla_absorb.h"

namespace mla {
namespace {

template <typename T>
__global__ void __launch_bounds__(256)
cache_append_kernel(const T *__restrict__ c_kv_new, const T *__restrict__ k_pe_new, const T *__restrict__ rms_w,
                    T *__restrict__ kv_cache, T *__restrict__ pe_cache, AppendCall a) {
  const int64_t tok = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);  // token (b, s) = tok / S, tok % S
  const int lane = threadIdx.x & 63;
  if (tok >= a.B * a.S) return;
  const int64_t b = tok / a.S, s = tok - b * a.S;
  int64_t end_pos = a.end_pos;
  if (a.seq_lens) {  // same clamp as the ragged attention: [S, end_pos]
    end_pos = a.seq_lens[b];
    if (end_pos < a.S) end_pos = a.S;
    if (end_pos > a.end_pos) end_pos = a.end_pos;
  }
  const int64_t p = end_pos - a.S + s;
  int64_t row = b * a.Tmax + p;  // destination row of kv_cache / pe_cache
  if (a.page_size > 0) {
    int64_t pg = a.block_table[b * a.max_pages + p / a.page_size];
    pg = pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);
    row = pg * a.page_size + p % a.page_size;
  }
  const T *x = c_kv_new + tok * a.C;
  float ss = 0.f;
  for (int64_t c = lane; c < a.C; c += 64) {
    const float v = Elem<T>::load(x, c);
    ss = fmaf(v, v, ss);
  }
  const float inv = 1.f / sqrtf(wave_sum(ss) / float(a.C) + a.eps);
  T *kv = kv_cache + row * a.C;
  for (int64_t c = lane; c < a.C; c += 64) Elem<T>::store(kv, c, Elem<T>::load(x, c) * inv * Elem<T>::load(rms_w, c));
  const T *kp = k_pe_new + tok * a.R;
  T *pe = pe_cache + row * a.R;
  for (int64_t r = lane; r < a.R; r += 64) pe[r] = kp[r];
}

}  // namespace

hipError_t cache_append(const AppendCall &a) {
  const dim3 grid(unsigned((a.B * a.S + 3) / 4)), block(256);
  if (a.dtype == MLA_DTYPE_F32)
    return launch_kernel(MLA_KERNEL_PLAIN, cache_append_kernel<float>, grid, block, 0, a.stream,
                         static_cast<const float *>(a.c_kv_new), static_cast<const float *>(a.k_pe_new),
                         static_cast<const float *>(a.rms_w), static_cast<float *>(a.kv_cache),
                         static_cast<float *>(a.pe_cache), a);
  return launch_kernel(MLA_KERNEL_PLAIN, cache_append_kernel<uint16_t>, grid, block, 0, a.stream,
                       static_cast<const uint16_t *>(a.c_kv_new), static_cast<const uint16_t *>(a.k_pe_new),
                       static_cast<const uint16_t *>(a.rms_w), static_cast<uint16_t *>(a.kv_cache),
                       static_cast<uint16_t *>(a.pe_cache), a);
}

}  // namespace mla
