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
// into the pool).  One wavefront per token (the rows of append_row.h); fp32 arithmetic, stores
// rounded to the cache's element type.
#include "append_row.h"
#include "common.h"
#include "launch.h"
#include "../../include/mla_absorb.h"

namespace mla {
namespace {

template <typename T>
__global__ void __launch_bounds__(256) cache_append_kernel(AppendCall a) {
  const int64_t tok = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);  // token (b, s) = tok / S, tok % S
  if (tok >= a.B * a.S) return;
  append_token<T>(a, tok, threadIdx.x & 63);
}

}  // namespace

hipError_t cache_append(const AppendCall &a) {
  const dim3 grid(unsigned((a.B * a.S + 3) / 4)), block(256);
  if (a.dtype == MLA_DTYPE_F32)
    return launch_kernel(MLA_KERNEL_PLAIN, cache_append_kernel<float>, grid, block, 0, a.stream, a);
  return launch_kernel(MLA_KERNEL_PLAIN, cache_append_kernel<uint16_t>, grid, block, 0, a.stream, a);
}

}  // namespace mla
