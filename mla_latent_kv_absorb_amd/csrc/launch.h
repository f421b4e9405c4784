// Internal interface between the C-ABI layer (mla_api.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla_absorb.h"

namespace mla {

// One validated absorb-attention call.  Rows are the B*S*H query rows in (b, s, h) order.
struct AttnCall {
  int64_t B, S, H, C, R, Dn, Dv, Bmax, Tmax;
  int64_t end_pos;           // uniform length, or the upper bound of the per-sequence lengths
  const int32_t *seq_lens;   // device [B] per-sequence lengths (clamped to [S, end_pos]), or null
  // paged caches (page_size > 0): kv / pe are pools [num_pages, page_size, C / R] and position t
  // of sequence b is row t % page_size of page block_table[b * max_pages + t / page_size]
  // (clamped into [0, num_pages)); with page_size 0 the caches are [Bmax, Tmax, C / R]
  const int32_t *block_table;
  int64_t page_size, num_pages, max_pages;
  // index lists (topk > 0): device [B, S, topk]; token (b, s) attends to the positions its list
  // names that lie in [0, end_pos - S + s] (end_pos per sequence as above); splits then cut the
  // list entries instead of the positions
  const int32_t *indices;
  int64_t topk;
  // balanced ragged plan (matrix-core path, bal_target > 0): splits is the most chunks one
  // sequence may take, bal_target the workgroups per row block, one chunk each (see attn_kernel)
  int32_t bal_target;
  float scale;
  int32_t dtype;      // MLA_DTYPE_*
  // element strides (dense values filled in when the caller gives none): query rows of q_nope and
  // q_pe, rows of out, cache rows (b) and positions (t) of kv and pe; page pools use the position
  // strides for rows within and across pages
  int64_t q_nope_rs, q_pe_rs, out_rs, kv_bs, kv_ps, pe_bs, pe_ps;
  int32_t splits;     // ranges the positions [0, end_pos) are cut into
  int64_t split_len;  // positions per range (the last may be shorter or empty)
  const void *q_nope, *q_pe, *kv, *pe, *wkv_b;
  void *out;
  void *ws;           // workspace (layout chosen by the path's workspace function)
  hipStream_t stream;
  // cache append fused into the call (mla_absorb_attn_append), or null: its rows are written
  // before the attention reads the caches
  const struct AppendCall *append;
};

struct ExpandCall {
  int64_t T, H, C, Dn, Dv;
  float eps;
  int32_t dtype;
  const void *c_kv, *rms_w, *wkv_b;
  void *k_nope, *v;
  // Output placement: input token t = b * S_in + s (s < S_in) goes to row
  // b * out_seq_stride + out_row0 + s of each head's [out_rows, Dn] / [out_rows, Dv] block.  A
  // plain expansion has S_in = out_seq_stride = out_rows = T and out_row0 = 0 (row t); the naive
  // path's cache append has S_in = new tokens per sequence, out_seq_stride = Tmax, out_row0 =
  // start_pos and out_rows = Bmax * Tmax.
  int64_t S_in, out_seq_stride, out_row0, out_rows;
  // Optional rope keys copied along (both null or both set): k_pe [T, R] row t to row
  // (placement as above) of pe_out [out_rows, R].
  const void *k_pe;
  void *pe_out;
  int64_t R;
  void *ws;  // workspace (layout chosen by the path's workspace function)
  hipStream_t stream;
};

// One validated naive-route attention call over expanded keys and values.
struct NaiveCall {
  int64_t B, S, H, R, Dn, Dv, Bmax, Tmax, end_pos;
  float scale;
  int32_t dtype;
  const void *q_nope, *q_pe, *k_nope, *v, *pe;  // k_nope / v: [H, Bmax, Tmax, Dn / Dv]
  void *out;
  hipStream_t stream;
};

// One validated cache append (the new tokens' latent, normalised, and rope key into the caches).
struct AppendCall {
  int64_t B, S, C, R, Tmax;
  int64_t end_pos;           // uniform length after the append, or the bound of seq_lens
  const int32_t *seq_lens;   // device [B] per-sequence lengths (clamped to [S, end_pos]), or null
  float eps;
  int32_t dtype;
  const void *c_kv_new, *k_pe_new, *rms_w;
  void *kv_cache, *pe_cache;  // [Bmax, Tmax, C / R], or page pools [num_pages, page_size, C / R]
  // element strides of the caches: sequence (b) and position (t) of kv and pe; page pools use the
  // position strides for rows within and across pages (dense: Tmax * C, C, Tmax * R, R)
  int64_t kv_bs, kv_ps, pe_bs, pe_ps;
  // paged caches (page_size > 0): position p of sequence b is row p % page_size of page
  // block_table[b * max_pages + p / page_size] (clamped into [0, num_pages))
  const int32_t *block_table;
  int64_t page_size, num_pages, max_pages;
  hipStream_t stream;
};

// ---- shared with the allocation-free entry point ------------------------------------------------
// Every check of mla_absorb_attn except the workspace's, with no HIP call and nothing launched;
// *need receives the workspace size the call would take.
int32_t absorb_attn_dry_run(const void *q_nope, const void *q_pe, const void *kv_cache, const void *pe_cache,
                            const void *wkv_b, int64_t end_pos, float softmax_scale, void *out,
                            const mla_attn_shape *shape, int32_t dtype, const mla_attn_options *options,
                            size_t *need);
// Records msg as this thread's last error and returns status.
int32_t set_error(int32_t status, const char *msg);

// ---- benchmark instrumentation (no-ops unless enabled for the kernel id) ----------------------
// Events recorded on the stream before and after a group of launches (the plain path's kernels).
void timing_begin(int kernel_id, hipStream_t stream);
void timing_end(int kernel_id, hipStream_t stream);
// Start/stop events for one launch of kernel_id (both null when its timing is off).  They are
// handed to hipExtLaunchKernel, which stamps them with the dispatch's own start and end times.
void timing_events(int kernel_id, hipEvent_t *start, hipEvent_t *stop);
void timing_record(int kernel_id, hipEvent_t start, hipEvent_t stop, hipError_t launch_status);

// Launch one kernel, timed per dispatch when timing is on for kernel_id; returns the launch status.
template <typename... Params, typename... Args>
hipError_t launch_kernel(int kernel_id, void (*kernel)(Params...), dim3 grid, dim3 block, uint32_t lds_bytes,
                         hipStream_t stream, Args... args) {
  hipEvent_t start = nullptr, stop = nullptr;
  timing_events(kernel_id, &start, &stop);
  hipExtLaunchKernelGGL(kernel, grid, block, lds_bytes, stream, start, stop, 0, args...);
  const hipError_t e = hipGetLastError();
  timing_record(kernel_id, start, stop, e);
  return e;
}

// ---- plain vector-ALU path (any shape, fp32 or bf16) -------------------------------------------
size_t plain_attn_workspace(const AttnCall &c);
int32_t plain_attn_splits(const AttnCall &c);
hipError_t plain_absorb_attn(const AttnCall &c);
hipError_t plain_expand_kv(const ExpandCall &c);

// ---- matrix-core path (bf16, shapes accepted by mfma_attn_supported) ---------------------------
bool mfma_attn_supported(const AttnCall &c, const char **why);
size_t mfma_attn_workspace(const AttnCall &c);
int32_t mfma_attn_splits(const AttnCall &c, int num_cus);
bool mfma_attn_plan_ok(const AttnCall &c, const char **why);  // limits that depend on the split count
int64_t mfma_paged_max_split_len(const AttnCall &c);           // longest split of a paged call
hipError_t mfma_absorb_attn(const AttnCall &c);

hipError_t cache_append(const AppendCall &a);

hipError_t plain_naive_attn(const NaiveCall &c);
bool mfma_naive_supported(const NaiveCall &c, const char **why);
hipError_t mfma_naive_attn(const NaiveCall &c);

bool mfma_expand_supported(const ExpandCall &c, const char **why);
size_t mfma_expand_workspace(const ExpandCall &c);
hipError_t mfma_expand_kv(const ExpandCall &c);

}  // namespace mla
