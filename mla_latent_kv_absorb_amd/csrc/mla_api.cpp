// C-ABI layer: argument validation, split planning and dispatch to the kernel paths.
// Every check runs before the first HIP call, so a rejected call enqueues nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/mla_absorb.h"
#include "launch.h"

namespace {

thread_local char g_last_error[512] = "";

int32_t fail(int32_t status, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

void clear_error() { g_last_error[0] = '\0'; }

bool misaligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

size_t elem_size(int32_t dtype) { return dtype == MLA_DTYPE_F32 ? 4 : 2; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

// Shape, dtype and option checks shared by the size query and the call.  Fills `c` (without
// pointers) and picks the kernel path.  Makes no HIP call: the plan depends only on the
// arguments, so the size query and the call always agree.
// With `paged` the caches are page pools: the shape's cache fields are replaced by the batch and
// the per-sequence capacity max_pages_per_seq * page_size.
// With topk > 0 each query token attends to an index list of topk entries, and the splits cut
// the entries.
// With ragged (per-sequence lengths in device memory) and an automatic split count, the matrix-core
// plan is the balanced one: as many workgroups as the uniform plan, each taking one chunk of one
// sequence.  The kernel plans from all lengths: a skewed batch gets one chunk length so that long
// sequences take more chunks (up to four times the uniform split count) and every workgroup
// about equal work; any other batch keeps the uniform splits.
int32_t plan_attn(const mla_attn_shape *shape, int64_t end_pos, const mla_paged_cache *paged, int64_t topk,
                  bool ragged, int32_t dtype, const mla_attn_options *options, mla::AttnCall &c, bool &use_mfma) {
  if (!shape) return fail(MLA_ERR_NULL, "shape is NULL");
  if (dtype != MLA_DTYPE_F32 && dtype != MLA_DTYPE_BF16) return fail(MLA_ERR_DTYPE, "unknown dtype %d", dtype);
  mla_attn_shape s = *shape;
  if (paged) {
    const mla_paged_cache &pg = *paged;
    if (pg.page_size < 1 || pg.page_size > (int64_t(1) << 20))
      return fail(MLA_ERR_SHAPE, "page_size = %lld outside [1, 1048576]", (long long)pg.page_size);
    if (pg.num_pages < 1 || pg.num_pages > (int64_t(1) << 31) - 1)
      return fail(MLA_ERR_SHAPE, "num_pages = %lld outside [1, 2^31 - 1]", (long long)pg.num_pages);
    if (pg.max_pages_per_seq < 1 || pg.max_pages_per_seq > (int64_t(1) << 31) - 1)
      return fail(MLA_ERR_SHAPE, "max_pages_per_seq = %lld outside [1, 2^31 - 1]", (long long)pg.max_pages_per_seq);
    if (s.batch > 0 && s.batch * pg.max_pages_per_seq > (int64_t(1) << 31) - 1)
      return fail(MLA_ERR_SHAPE, "batch * max_pages_per_seq is too large");
    if (pg.num_pages * pg.page_size > (int64_t(1) << 40))
      return fail(MLA_ERR_SHAPE, "num_pages * page_size is too large");
    s.cache_batch = s.batch;
    s.cache_len = std::min<int64_t>(pg.max_pages_per_seq * pg.page_size, int64_t(1) << 31);
  }
  const int64_t dims[] = {s.batch, s.seqlen_q, s.n_heads, s.kv_lora_rank, s.qk_rope_head_dim,
                          s.qk_nope_head_dim, s.v_head_dim, s.cache_batch, s.cache_len};
  const char *names[] = {"batch", "seqlen_q", "n_heads", "kv_lora_rank", "qk_rope_head_dim",
                         "qk_nope_head_dim", "v_head_dim", "cache_batch", "cache_len"};
  for (int i = 0; i < 9; ++i)
    if (dims[i] <= 0 || dims[i] > (int64_t(1) << 31))
      return fail(MLA_ERR_SHAPE, "%s = %lld is out of range", names[i], (long long)dims[i]);
  if (s.batch > s.cache_batch)
    return fail(MLA_ERR_RANGE, "batch %lld exceeds cache_batch %lld", (long long)s.batch, (long long)s.cache_batch);
  if (end_pos < 1 || end_pos > s.cache_len)
    return fail(MLA_ERR_RANGE, "end_pos %lld outside [1, cache_len=%lld]", (long long)end_pos, (long long)s.cache_len);
  if (s.seqlen_q > end_pos)
    return fail(MLA_ERR_RANGE, "seqlen_q %lld exceeds end_pos %lld", (long long)s.seqlen_q, (long long)end_pos);
  const int64_t rows = s.batch * s.seqlen_q * s.n_heads;
  if (rows > (int64_t(1) << 31) / 4)
    return fail(MLA_ERR_SHAPE, "batch*seqlen_q*n_heads = %lld is too large", (long long)rows);
  // every row of every tensor must start on a 16-byte boundary
  const int64_t ealign = 16 / int64_t(elem_size(dtype));
  if (s.kv_lora_rank % ealign || s.qk_rope_head_dim % ealign || s.qk_nope_head_dim % ealign ||
      s.v_head_dim % ealign)
    return fail(MLA_ERR_ALIGN, "kv_lora_rank, qk_rope_head_dim, qk_nope_head_dim and v_head_dim must be "
                               "multiples of %lld elements (16-byte rows)", (long long)ealign);

  mla_attn_options opt = {0, MLA_PATH_AUTO, nullptr};
  if (options) opt = *options;
  if (opt.num_splits < 0 || opt.num_splits > 4096)
    return fail(MLA_ERR_SHAPE, "num_splits %d outside [0, 4096]", opt.num_splits);
  if (opt.path != MLA_PATH_AUTO && opt.path != MLA_PATH_PLAIN && opt.path != MLA_PATH_MFMA)
    return fail(MLA_ERR_UNSUPPORTED, "unknown path %d", opt.path);

  c = mla::AttnCall{};
  c.B = s.batch; c.S = s.seqlen_q; c.H = s.n_heads; c.C = s.kv_lora_rank; c.R = s.qk_rope_head_dim;
  c.Dn = s.qk_nope_head_dim; c.Dv = s.v_head_dim; c.Bmax = s.cache_batch; c.Tmax = s.cache_len;
  c.end_pos = end_pos; c.dtype = dtype;
  // element strides: the caller's, a 0 field (or no struct) meaning the dense value
  const mla_attn_strides st = opt.strides ? *opt.strides : mla_attn_strides{0, 0, 0, 0, 0, 0, 0};
  c.q_nope_rs = st.q_nope_row ? st.q_nope_row : c.Dn;
  c.q_pe_rs = st.q_pe_row ? st.q_pe_row : c.R;
  c.out_rs = st.out_row ? st.out_row : c.Dv;
  c.kv_ps = st.kv_pos ? st.kv_pos : c.C;
  c.pe_ps = st.pe_pos ? st.pe_pos : c.R;
  // (page pools ignore the batch strides: a page is page_size rows at the position stride)
  c.kv_bs = paged ? 0 : (st.kv_batch ? st.kv_batch : c.Tmax * c.kv_ps);
  c.pe_bs = paged ? 0 : (st.pe_batch ? st.pe_batch : c.Tmax * c.pe_ps);
  {
    const int64_t vals[] = {c.q_nope_rs, c.q_pe_rs, c.out_rs, c.kv_ps, c.pe_ps, c.kv_bs, c.pe_bs};
    const int64_t mins[] = {c.Dn, c.R, c.Dv, c.C, c.R, 1, 1};
    const char *snames[] = {"q_nope_row", "q_pe_row", "out_row", "kv_pos", "pe_pos", "kv_batch", "pe_batch"};
    for (int i = 0; i < (paged ? 5 : 7); ++i) {
      if (vals[i] < mins[i] || vals[i] > (int64_t(1) << 40))
        return fail(MLA_ERR_SHAPE, "stride %s = %lld outside [%lld, 2^40]", snames[i], (long long)vals[i],
                    (long long)mins[i]);
      if (vals[i] % ealign)
        return fail(MLA_ERR_ALIGN, "stride %s = %lld is not a multiple of %lld elements (16 bytes)", snames[i],
                    (long long)vals[i], (long long)ealign);
    }
  }
  if (topk < 0 || topk > (int64_t(1) << 24)) return fail(MLA_ERR_SHAPE, "topk = %lld outside [1, 2^24]", (long long)topk);
  c.topk = topk;
  if (topk > 0 && s.batch * s.seqlen_q * topk > (int64_t(1) << 31) - 1)
    return fail(MLA_ERR_SHAPE, "batch * seqlen_q * topk is too large");
  if (paged) {
    c.page_size = paged->page_size; c.num_pages = paged->num_pages; c.max_pages = paged->max_pages_per_seq;
  }

  use_mfma = false;
  if (opt.path != MLA_PATH_PLAIN) {
    const char *why = "";
    const bool ok = mla::mfma_attn_supported(c, &why);
    if (opt.path == MLA_PATH_MFMA && !ok) return fail(MLA_ERR_UNSUPPORTED, "matrix-core path: %s", why);
    use_mfma = ok;
  }
  if (opt.num_splits > 0) {
    c.splits = opt.num_splits;
  } else {
    c.splits = use_mfma ? mla::mfma_attn_splits(c, 256) : mla::plain_attn_splits(c);
  }
  const int64_t items = topk > 0 ? topk : end_pos;  // positions, or list entries
  if (c.splits > items) c.splits = int32_t(items);
  c.split_len = (items + c.splits - 1) / c.splits;
  if (use_mfma && c.page_size > 0) c.split_len = (c.split_len + 31) / 32 * 32;  // tiles within pages
  if (use_mfma && ragged && topk == 0 && opt.num_splits == 0 && c.splits > 0) {
    const int64_t s0 = c.splits;
    const int64_t smax =
        c.B > 1 ? std::min<int64_t>(std::min<int64_t>(4 * s0, std::max<int64_t>(s0, (end_pos + 31) / 32)), 4096) : s0;
    // chunks a sequence needs at the longest chunk length: one, or more where pages cap a chunk
    // (s0 already covers that); the grid must hold B of them so that the kernel's search for a
    // chunk length always ends
    const int64_t cap = c.page_size > 0 ? mla::mfma_paged_max_split_len(c) : end_pos;
    const int64_t need = (end_pos + cap - 1) / cap;
    mla::AttnCall cb = c;
    cb.splits = int32_t(smax);
    cb.split_len = ((end_pos + smax - 1) / smax + 31) / 32 * 32;
    cb.bal_target = int32_t(c.B * std::max(s0, std::min(smax, need)));
    const char *why = "";
    if (mla::mfma_attn_plan_ok(cb, &why)) c = cb;  // else keep the uniform plan
  }
  if (use_mfma) {
    const char *why = "";
    if (!mla::mfma_attn_plan_ok(c, &why)) {
      if (opt.path == MLA_PATH_MFMA) return fail(MLA_ERR_UNSUPPORTED, "matrix-core path: %s", why);
      use_mfma = false;
      if (opt.num_splits == 0) {
        c.splits = mla::plain_attn_splits(c);
        if (c.splits > items) c.splits = int32_t(items);
        c.split_len = (items + c.splits - 1) / c.splits;
      }
    }
  }
  return MLA_OK;
}

}  // namespace

extern "C" {

const char *mla_strerror(int32_t status) {
  switch (status) {
    case MLA_OK: return "success";
    case MLA_ERR_NULL: return "a required pointer is NULL";
    case MLA_ERR_SHAPE: return "invalid or inconsistent sizes";
    case MLA_ERR_DTYPE: return "unknown element type";
    case MLA_ERR_RANGE: return "end_pos/batch outside the cache capacity or seqlen_q > end_pos";
    case MLA_ERR_ALIGN: return "pointer or row not 16-byte aligned";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_HIP: return "HIP runtime or kernel launch failure";
    case MLA_ERR_UNSUPPORTED: return "unsupported option or shape for the requested kernel path";
    default: return "unknown status";
  }
}

const char *mla_last_error(void) { return g_last_error; }

size_t mla_absorb_attn_workspace_size(const mla_attn_shape *shape, int64_t end_pos, int32_t dtype,
                                      const mla_attn_options *options) {
  clear_error();
  mla::AttnCall c;
  bool use_mfma = false;
  if (plan_attn(shape, end_pos, nullptr, 0, false, dtype, options, c, use_mfma) != MLA_OK) return 0;
  return use_mfma ? mla::mfma_attn_workspace(c) : mla::plain_attn_workspace(c);
}

size_t mla_absorb_attn_ragged_workspace_size(const mla_attn_shape *shape, int64_t max_seq_len, int32_t dtype,
                                             const mla_attn_options *options) {
  clear_error();
  mla::AttnCall c;
  bool use_mfma = false;
  if (plan_attn(shape, max_seq_len, nullptr, 0, true, dtype, options, c, use_mfma) != MLA_OK) return 0;
  return use_mfma ? mla::mfma_attn_workspace(c) : mla::plain_attn_workspace(c);
}

size_t mla_absorb_attn_paged_workspace_size(const mla_attn_shape *shape, int64_t max_seq_len,
                                            const mla_paged_cache *paged, int32_t dtype,
                                            const mla_attn_options *options) {
  clear_error();
  if (!paged) { fail(MLA_ERR_NULL, "paged is NULL"); return 0; }
  mla::AttnCall c;
  bool use_mfma = false;
  if (plan_attn(shape, max_seq_len, paged, 0, true, dtype, options, c, use_mfma) != MLA_OK) return 0;
  return use_mfma ? mla::mfma_attn_workspace(c) : mla::plain_attn_workspace(c);
}

size_t mla_absorb_attn_sparse_workspace_size(const mla_attn_shape *shape, int64_t end_pos, int64_t topk,
                                             int32_t dtype, const mla_attn_options *options) {
  clear_error();
  if (topk < 1) { fail(MLA_ERR_SHAPE, "topk = %lld must be >= 1", (long long)topk); return 0; }
  mla::AttnCall c;
  bool use_mfma = false;
  if (plan_attn(shape, end_pos, nullptr, topk, false, dtype, options, c, use_mfma) != MLA_OK) return 0;
  return use_mfma ? mla::mfma_attn_workspace(c) : mla::plain_attn_workspace(c);
}

}  // extern "C"

namespace {

// The new tokens of a fused cache append (mla_absorb_attn_append and its paged form).
struct AppendIn {
  const void *c_kv_new, *k_pe_new, *rms_w;
  float eps;
};

// The body of mla_absorb_attn, mla_absorb_attn_ragged and mla_absorb_attn_paged (seq_lens null
// for a uniform batch; paged and block_table null for contiguous caches), and with `app` of the
// fused append entry points, whose rows are written into the caches before the attention reads them.
int32_t absorb_attn_call(const void *q_nope, const void *q_pe, const void *kv_cache, const void *pe_cache,
                         const void *wkv_b, const int32_t *seq_lens, const int32_t *block_table,
                         const mla_paged_cache *paged, const int32_t *indices, int64_t topk, int64_t end_pos,
                         float softmax_scale, void *out, const mla_attn_shape *shape, int32_t dtype,
                         const mla_attn_options *options, void *workspace, size_t workspace_bytes, void *stream,
                         size_t *dry_need = nullptr, const AppendIn *app = nullptr) {
  mla::AttnCall c;
  bool use_mfma = false;
  int32_t rc = plan_attn(shape, end_pos, paged, indices ? topk : 0, seq_lens != nullptr, dtype, options, c, use_mfma);
  if (rc != MLA_OK) return rc;
  const void *ptrs[] = {q_nope, q_pe, kv_cache, pe_cache, wkv_b, out};
  const char *names[] = {"q_nope", "q_pe", "kv_cache", "pe_cache", "wkv_b", "out"};
  for (int i = 0; i < 6; ++i) {
    if (!ptrs[i]) return fail(MLA_ERR_NULL, "%s is NULL", names[i]);
    if (misaligned(ptrs[i])) return fail(MLA_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
  }
  if (!(softmax_scale == softmax_scale) || softmax_scale <= 0.f || softmax_scale > 1e30f)
    return fail(MLA_ERR_SHAPE, "softmax_scale must be a positive finite number");
  const size_t es = elem_size(dtype);
  const size_t rows = size_t(c.B * c.S * c.H);
  // byte extents of the (possibly strided) tensors: from the first element to past the last
  const int64_t cache_kv = paged ? (c.num_pages * c.page_size - 1) * c.kv_ps + c.C
                                 : (c.Bmax - 1) * c.kv_bs + (c.Tmax - 1) * c.kv_ps + c.C;
  const int64_t cache_pe = paged ? (c.num_pages * c.page_size - 1) * c.pe_ps + c.R
                                 : (c.Bmax - 1) * c.pe_bs + (c.Tmax - 1) * c.pe_ps + c.R;
  const size_t bytes_in[] = {size_t((int64_t(rows) - 1) * c.q_nope_rs + c.Dn) * es,
                             size_t((int64_t(rows) - 1) * c.q_pe_rs + c.R) * es, size_t(cache_kv) * es,
                             size_t(cache_pe) * es, size_t(c.H * (c.Dn + c.Dv) * c.C) * es};
  const size_t out_bytes = size_t((int64_t(rows) - 1) * c.out_rs + c.Dv) * es;
  for (int i = 0; i < 5; ++i)
    if (overlaps(out, out_bytes, ptrs[i], bytes_in[i])) return fail(MLA_ERR_SHAPE, "out overlaps %s", names[i]);
  const size_t lens_bytes = size_t(c.B) * sizeof(int32_t);
  if (seq_lens && overlaps(out, out_bytes, seq_lens, lens_bytes)) return fail(MLA_ERR_SHAPE, "out overlaps seq_lens");
  const size_t table_bytes = size_t(c.B * c.max_pages) * sizeof(int32_t);
  if (block_table && overlaps(out, out_bytes, block_table, table_bytes))
    return fail(MLA_ERR_SHAPE, "out overlaps block_table");
  const size_t index_bytes = size_t(c.B * c.S * c.topk) * sizeof(int32_t);
  if (indices && overlaps(out, out_bytes, indices, index_bytes)) return fail(MLA_ERR_SHAPE, "out overlaps indices");
  // fused append: the caches are written, so nothing else the call touches may overlap them
  mla::AppendCall ac{};
  const size_t toks = size_t(c.B * c.S);
  const void *aptrs[] = {app ? app->c_kv_new : nullptr, app ? app->k_pe_new : nullptr, app ? app->rms_w : nullptr};
  const char *anames[] = {"c_kv_new", "k_pe_new", "rms_w"};
  const size_t abytes[] = {toks * size_t(c.C) * es, toks * size_t(c.R) * es, size_t(c.C) * es};
  if (app) {
    for (int i = 0; i < 3; ++i) {
      if (!aptrs[i]) return fail(MLA_ERR_NULL, "%s is NULL", anames[i]);
      if (misaligned(aptrs[i])) return fail(MLA_ERR_ALIGN, "%s is not 16-byte aligned", anames[i]);
    }
    if (!(app->eps >= 0.f) || app->eps > 1.f) return fail(MLA_ERR_SHAPE, "eps must be in [0, 1]");
    if (overlaps(kv_cache, bytes_in[2], pe_cache, bytes_in[3])) return fail(MLA_ERR_SHAPE, "kv_cache overlaps pe_cache");
    const void *wr[] = {kv_cache, pe_cache};
    const size_t wr_bytes[] = {bytes_in[2], bytes_in[3]};
    for (int k = 0; k < 2; ++k) {
      for (int i : {0, 1, 4})
        if (overlaps(wr[k], wr_bytes[k], ptrs[i], bytes_in[i]))
          return fail(MLA_ERR_SHAPE, "%s overlaps %s", names[2 + k], names[i]);
      for (int i = 0; i < 3; ++i)
        if (overlaps(wr[k], wr_bytes[k], aptrs[i], abytes[i]))
          return fail(MLA_ERR_SHAPE, "%s overlaps %s", names[2 + k], anames[i]);
      if (seq_lens && overlaps(wr[k], wr_bytes[k], seq_lens, lens_bytes))
        return fail(MLA_ERR_SHAPE, "%s overlaps seq_lens", names[2 + k]);
      if (block_table && overlaps(wr[k], wr_bytes[k], block_table, table_bytes))
        return fail(MLA_ERR_SHAPE, "%s overlaps block_table", names[2 + k]);
    }
    for (int i = 0; i < 3; ++i)
      if (overlaps(out, out_bytes, aptrs[i], abytes[i])) return fail(MLA_ERR_SHAPE, "out overlaps %s", anames[i]);
    ac.B = c.B; ac.S = c.S; ac.C = c.C; ac.R = c.R; ac.Tmax = c.Tmax;
    ac.end_pos = end_pos; ac.seq_lens = seq_lens; ac.eps = app->eps; ac.dtype = dtype;
    ac.c_kv_new = app->c_kv_new; ac.k_pe_new = app->k_pe_new; ac.rms_w = app->rms_w;
    ac.kv_cache = const_cast<void *>(kv_cache); ac.pe_cache = const_cast<void *>(pe_cache);
    ac.kv_bs = c.kv_bs; ac.kv_ps = c.kv_ps; ac.pe_bs = c.pe_bs; ac.pe_ps = c.pe_ps;
    if (paged) {
      ac.block_table = block_table;
      ac.page_size = c.page_size; ac.num_pages = c.num_pages; ac.max_pages = c.max_pages;
    }
  }
  const size_t need = use_mfma ? mla::mfma_attn_workspace(c) : mla::plain_attn_workspace(c);
  if (dry_need) {  // every check but the workspace's; nothing is launched
    *dry_need = need;
    return MLA_OK;
  }
  if (need > 0) {
    if (!workspace) return fail(MLA_ERR_WORKSPACE, "workspace is NULL but %zu bytes are needed", need);
    if (workspace_bytes < need)
      return fail(MLA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
    if (misaligned(workspace)) return fail(MLA_ERR_ALIGN, "workspace is not 16-byte aligned");
    if (overlaps(workspace, need, out, out_bytes)) return fail(MLA_ERR_WORKSPACE, "workspace overlaps out");
    for (int i = 0; i < 5; ++i)
      if (overlaps(workspace, need, ptrs[i], bytes_in[i]))
        return fail(MLA_ERR_WORKSPACE, "workspace overlaps %s", names[i]);
    if (seq_lens && overlaps(workspace, need, seq_lens, lens_bytes))
      return fail(MLA_ERR_WORKSPACE, "workspace overlaps seq_lens");
    if (block_table && overlaps(workspace, need, block_table, table_bytes))
      return fail(MLA_ERR_WORKSPACE, "workspace overlaps block_table");
    if (indices && overlaps(workspace, need, indices, index_bytes))
      return fail(MLA_ERR_WORKSPACE, "workspace overlaps indices");
    if (app)
      for (int i = 0; i < 3; ++i)
        if (overlaps(workspace, need, aptrs[i], abytes[i]))
          return fail(MLA_ERR_WORKSPACE, "workspace overlaps %s", anames[i]);
  }
  c.scale = softmax_scale;
  c.q_nope = q_nope; c.q_pe = q_pe; c.kv = kv_cache; c.pe = pe_cache; c.wkv_b = wkv_b;
  c.out = out; c.ws = workspace; c.stream = static_cast<hipStream_t>(stream);
  c.seq_lens = seq_lens;
  c.block_table = block_table;
  c.indices = indices;
  if (use_mfma && c.splits == 0) c.splits = 1;
  hipError_t e = hipSuccess;
  if (app) {
    ac.stream = c.stream;
    if (use_mfma) {
      c.append = &ac;  // written by the query-absorption kernel
    } else {
      e = mla::cache_append(ac);
      if (e != hipSuccess) return fail(MLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    }
  }
  e = use_mfma ? mla::mfma_absorb_attn(c) : mla::plain_absorb_attn(c);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return MLA_OK;
}

}  // namespace

namespace mla {

int32_t set_error(int32_t status, const char *msg) { return fail(status, "%s", msg); }

int32_t absorb_attn_dry_run(const void *q_nope, const void *q_pe, const void *kv_cache, const void *pe_cache,
                            const void *wkv_b, int64_t end_pos, float softmax_scale, void *out,
                            const mla_attn_shape *shape, int32_t dtype, const mla_attn_options *options,
                            size_t *need) {
  clear_error();
  return absorb_attn_call(q_nope, q_pe, kv_cache, pe_cache, wkv_b, nullptr, nullptr, nullptr, nullptr, 0, end_pos,
                          softmax_scale, out, shape, dtype, options, nullptr, 0, nullptr, need);
}

}  // namespace mla

extern "C" {

int32_t mla_absorb_attn(const void *q_nope, const void *q_pe, const void *kv_cache, const void *pe_cache,
                        const void *wkv_b, int64_t end_pos, float softmax_scale, void *out,
                        const mla_attn_shape *shape, int32_t dtype, const mla_attn_options *options,
                        void *workspace, size_t workspace_bytes, void *stream) {
  clear_error();
  return absorb_attn_call(q_nope, q_pe, kv_cache, pe_cache, wkv_b, nullptr, nullptr, nullptr, nullptr, 0, end_pos,
                          softmax_scale, out, shape, dtype, options, workspace, workspace_bytes, stream);
}

int32_t mla_absorb_attn_ragged(const void *q_nope, const void *q_pe, const void *kv_cache, const void *pe_cache,
                               const void *wkv_b, const int32_t *seq_lens, int64_t max_seq_len,
                               float softmax_scale, void *out, const mla_attn_shape *shape, int32_t dtype,
                               const mla_attn_options *options, void *workspace, size_t workspace_bytes,
                               void *stream) {
  clear_error();
  if (!seq_lens) return fail(MLA_ERR_NULL, "seq_lens is NULL");
  if (reinterpret_cast<uintptr_t>(seq_lens) & 3u) return fail(MLA_ERR_ALIGN, "seq_lens is not 4-byte aligned");
  return absorb_attn_call(q_nope, q_pe, kv_cache, pe_cache, wkv_b, seq_lens, nullptr, nullptr, nullptr, 0,
                          max_seq_len, softmax_scale, out, shape, dtype, options, workspace, workspace_bytes, stream);
}

int32_t mla_absorb_attn_paged(const void *q_nope, const void *q_pe, const void *kv_pages, const void *pe_pages,
                              const void *wkv_b, const int32_t *block_table, const int32_t *seq_lens,
                              int64_t max_seq_len, float softmax_scale, void *out, const mla_attn_shape *shape,
                              const mla_paged_cache *paged, int32_t dtype, const mla_attn_options *options,
                              void *workspace, size_t workspace_bytes, void *stream) {
  clear_error();
  if (!paged) return fail(MLA_ERR_NULL, "paged is NULL");
  if (!block_table) return fail(MLA_ERR_NULL, "block_table is NULL");
  if (reinterpret_cast<uintptr_t>(block_table) & 3u) return fail(MLA_ERR_ALIGN, "block_table is not 4-byte aligned");
  if (reinterpret_cast<uintptr_t>(seq_lens) & 3u) return fail(MLA_ERR_ALIGN, "seq_lens is not 4-byte aligned");
  return absorb_attn_call(q_nope, q_pe, kv_pages, pe_pages, wkv_b, seq_lens, block_table, paged, nullptr, 0,
                          max_seq_len, softmax_scale, out, shape, dtype, options, workspace, workspace_bytes, stream);
}

int32_t mla_absorb_attn_append(const void *q_nope, const void *q_pe, const void *c_kv_new, const void *k_pe_new,
                               const void *rms_w, float eps, void *kv_cache, void *pe_cache, const void *wkv_b,
                               const int32_t *seq_lens, int64_t end_pos, float softmax_scale, void *out,
                               const mla_attn_shape *shape, int32_t dtype, const mla_attn_options *options,
                               void *workspace, size_t workspace_bytes, void *stream) {
  clear_error();
  if (reinterpret_cast<uintptr_t>(seq_lens) & 3u) return fail(MLA_ERR_ALIGN, "seq_lens is not 4-byte aligned");
  const AppendIn app{c_kv_new, k_pe_new, rms_w, eps};
  return absorb_attn_call(q_nope, q_pe, kv_cache, pe_cache, wkv_b, seq_lens, nullptr, nullptr, nullptr, 0, end_pos,
                          softmax_scale, out, shape, dtype, options, workspace, workspace_bytes, stream, nullptr, &app);
}

int32_t mla_absorb_attn_paged_append(const void *q_nope, const void *q_pe, const void *c_kv_new,
                                     const void *k_pe_new, const void *rms_w, float eps, void *kv_pages,
                                     void *pe_pages, const void *wkv_b, const int32_t *block_table,
                                     const int32_t *seq_lens, int64_t max_seq_len, float softmax_scale, void *out,
                                     const mla_attn_shape *shape, const mla_paged_cache *paged, int32_t dtype,
                                     const mla_attn_options *options, void *workspace, size_t workspace_bytes,
                                     void *stream) {
  clear_error();
  if (!paged) return fail(MLA_ERR_NULL, "paged is NULL");
  if (!block_table) return fail(MLA_ERR_NULL, "block_table is NULL");
  if (reinterpret_cast<uintptr_t>(block_table) & 3u) return fail(MLA_ERR_ALIGN, "block_table is not 4-byte aligned");
  if (reinterpret_cast<uintptr_t>(seq_lens) & 3u) return fail(MLA_ERR_ALIGN, "seq_lens is not 4-byte aligned");
  const AppendIn app{c_kv_new, k_pe_new, rms_w, eps};
  return absorb_attn_call(q_nope, q_pe, kv_pages, pe_pages, wkv_b, seq_lens, block_table, paged, nullptr, 0,
                          max_seq_len, softmax_scale, out, shape, dtype, options, workspace, workspace_bytes, stream,
                          nullptr, &app);
}

int32_t mla_absorb_attn_sparse(const void *q_nope, const void *q_pe, const void *kv_cache, const void *pe_cache,
                               const void *wkv_b, const int32_t *indices, int64_t topk, const int32_t *seq_lens,
                               int64_t end_pos, float softmax_scale, void *out, const mla_attn_shape *shape,
                               int32_t dtype, const mla_attn_options *options, void *workspace,
                               size_t workspace_bytes, void *stream) {
  clear_error();
  if (!indices) return fail(MLA_ERR_NULL, "indices is NULL");
  if (reinterpret_cast<uintptr_t>(indices) & 3u) return fail(MLA_ERR_ALIGN, "indices is not 4-byte aligned");
  if (reinterpret_cast<uintptr_t>(seq_lens) & 3u) return fail(MLA_ERR_ALIGN, "seq_lens is not 4-byte aligned");
  if (topk < 1) return fail(MLA_ERR_SHAPE, "topk = %lld must be >= 1", (long long)topk);
  return absorb_attn_call(q_nope, q_pe, kv_cache, pe_cache, wkv_b, seq_lens, nullptr, nullptr, indices, topk,
                          end_pos, softmax_scale, out, shape, dtype, options, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// The kernel path of a planned expansion (placement and rope copy already set in e).
int32_t choose_expand_path(const mla::ExpandCall &e, int32_t path, bool &use_mfma) {
  use_mfma = false;
  if (path != MLA_PATH_AUTO && path != MLA_PATH_PLAIN && path != MLA_PATH_MFMA)
    return fail(MLA_ERR_UNSUPPORTED, "unknown path %d", path);
  if (path != MLA_PATH_PLAIN) {
    const char *why = "";
    const bool ok = mla::mfma_expand_supported(e, &why);
    if (path == MLA_PATH_MFMA && !ok) return fail(MLA_ERR_UNSUPPORTED, "matrix-core path: %s", why);
    use_mfma = ok;
  }
  return MLA_OK;
}

// Validation shared by mla_expand_kv and mla_expand_kv_workspace_size; no HIP calls.
int32_t plan_expand(int64_t n_tokens, int64_t n_heads, int64_t kv_lora_rank, int64_t qk_nope_head_dim,
                    int64_t v_head_dim, float eps, int32_t dtype, int32_t path, mla::ExpandCall &e,
                    bool &use_mfma) {
  if (dtype != MLA_DTYPE_F32 && dtype != MLA_DTYPE_BF16) return fail(MLA_ERR_DTYPE, "unknown dtype %d", dtype);
  const int64_t dims[] = {n_tokens, n_heads, kv_lora_rank, qk_nope_head_dim, v_head_dim};
  const char *dnames[] = {"n_tokens", "n_heads", "kv_lora_rank", "qk_nope_head_dim", "v_head_dim"};
  for (int i = 0; i < 5; ++i)
    if (dims[i] <= 0 || dims[i] > (int64_t(1) << 31))
      return fail(MLA_ERR_SHAPE, "%s = %lld is out of range", dnames[i], (long long)dims[i]);
  const int64_t ealign = 16 / int64_t(elem_size(dtype));
  if (kv_lora_rank % ealign || qk_nope_head_dim % ealign || v_head_dim % ealign)
    return fail(MLA_ERR_ALIGN, "kv_lora_rank, qk_nope_head_dim and v_head_dim must be multiples of %lld "
                               "elements (16-byte rows)", (long long)ealign);
  if (n_heads * (qk_nope_head_dim + v_head_dim) > (int64_t(1) << 31))
    return fail(MLA_ERR_SHAPE, "n_heads * (qk_nope_head_dim + v_head_dim) is too large");
  if (!(eps >= 0.f) || eps > 1e30f) return fail(MLA_ERR_SHAPE, "eps must be finite and >= 0");
  if (path != MLA_PATH_AUTO && path != MLA_PATH_PLAIN && path != MLA_PATH_MFMA)
    return fail(MLA_ERR_UNSUPPORTED, "unknown path %d", path);
  e = mla::ExpandCall{};
  e.T = n_tokens; e.H = n_heads; e.C = kv_lora_rank; e.Dn = qk_nope_head_dim; e.Dv = v_head_dim;
  e.eps = eps; e.dtype = dtype;
  // plain placement (row t of each head's block); the cache append overrides it before the path
  // check, which depends on it
  e.S_in = n_tokens; e.out_seq_stride = n_tokens; e.out_row0 = 0; e.out_rows = n_tokens;
  use_mfma = false;
  return choose_expand_path(e, path, use_mfma);
}

// Enqueues a planned expansion (e without pointers) after the pointer, overlap and workspace
// checks.  ins: c_kv, rms_w, wkv_b[, k_pe]; outs: k_nope, v[, pe_out], with their byte sizes.
int32_t run_expand_call(mla::ExpandCall &e, bool use_mfma, const void *const *ptrs, const size_t *sizes,
                        const char *const *names, int n_in, int n_out, void *workspace, size_t workspace_bytes,
                        void *stream) {
  const int n = n_in + n_out;
  for (int i = 0; i < n; ++i) {
    if (!ptrs[i]) return fail(MLA_ERR_NULL, "%s is NULL", names[i]);
    if (misaligned(ptrs[i])) return fail(MLA_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
  }
  for (int o = n_in; o < n; ++o)
    for (int i = 0; i < n; ++i)
      if (i != o && overlaps(ptrs[o], sizes[o], ptrs[i], sizes[i]))
        return fail(MLA_ERR_SHAPE, "%s overlaps %s", names[o], names[i]);
  const size_t need = use_mfma ? mla::mfma_expand_workspace(e) : 0;
  if (need > 0) {
    if (!workspace) return fail(MLA_ERR_WORKSPACE, "workspace is NULL but %zu bytes are needed", need);
    if (workspace_bytes < need)
      return fail(MLA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
    if (misaligned(workspace)) return fail(MLA_ERR_ALIGN, "workspace is not 16-byte aligned");
    for (int i = 0; i < n; ++i)
      if (overlaps(workspace, need, ptrs[i], sizes[i]))
        return fail(MLA_ERR_WORKSPACE, "workspace overlaps %s", names[i]);
  }
  e.c_kv = ptrs[0]; e.rms_w = ptrs[1]; e.wkv_b = ptrs[2];
  e.k_pe = n_in > 3 ? ptrs[3] : nullptr;
  e.k_nope = const_cast<void *>(ptrs[n_in]); e.v = const_cast<void *>(ptrs[n_in + 1]);
  e.pe_out = n_out > 2 ? const_cast<void *>(ptrs[n_in + 2]) : nullptr;
  e.ws = workspace;
  e.stream = static_cast<hipStream_t>(stream);
  hipError_t err = use_mfma ? mla::mfma_expand_kv(e) : mla::plain_expand_kv(e);
  if (err != hipSuccess) return fail(MLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  return MLA_OK;
}

}  // namespace

extern "C" {

size_t mla_expand_kv_workspace_size(int64_t n_tokens, int64_t n_heads, int64_t kv_lora_rank,
                                    int64_t qk_nope_head_dim, int64_t v_head_dim, int32_t dtype, int32_t path) {
  clear_error();
  mla::ExpandCall e;
  bool use_mfma = false;
  if (plan_expand(n_tokens, n_heads, kv_lora_rank, qk_nope_head_dim, v_head_dim, 0.f, dtype, path, e, use_mfma) !=
      MLA_OK)
    return 0;
  return use_mfma ? mla::mfma_expand_workspace(e) : 0;
}

int32_t mla_expand_kv(const void *c_kv, const void *rms_w, const void *wkv_b, void *k_nope, void *v,
                      int64_t n_tokens, int64_t n_heads, int64_t kv_lora_rank, int64_t qk_nope_head_dim,
                      int64_t v_head_dim, float eps, int32_t dtype, int32_t path, void *workspace,
                      size_t workspace_bytes, void *stream) {
  clear_error();
  mla::ExpandCall e;
  bool use_mfma = false;
  const int32_t st = plan_expand(n_tokens, n_heads, kv_lora_rank, qk_nope_head_dim, v_head_dim, eps, dtype, path, e,
                                 use_mfma);
  if (st != MLA_OK) return st;
  const void *ptrs[] = {c_kv, rms_w, wkv_b, k_nope, v};
  const char *names[] = {"c_kv", "rms_w", "wkv_b", "k_nope", "v"};
  const size_t es = elem_size(dtype);
  const size_t sizes[] = {size_t(n_tokens * kv_lora_rank) * es, size_t(kv_lora_rank) * es,
                          size_t(n_heads * (qk_nope_head_dim + v_head_dim) * kv_lora_rank) * es,
                          size_t(n_heads * n_tokens * qk_nope_head_dim) * es,
                          size_t(n_heads * n_tokens * v_head_dim) * es};
  return run_expand_call(e, use_mfma, ptrs, sizes, names, 3, 2, workspace, workspace_bytes, stream);
}

int32_t mla_expand_kv_append(const void *c_kv_new, const void *k_pe_new, const void *rms_w, const void *wkv_b,
                             float eps, int64_t end_pos, void *k_cache, void *v_cache, void *pe_cache,
                             const mla_attn_shape *shape, int32_t dtype, int32_t path, void *workspace,
                             size_t workspace_bytes, void *stream) {
  clear_error();
  if (!shape) return fail(MLA_ERR_NULL, "shape is NULL");
  const mla_attn_shape s = *shape;
  const int64_t dims[] = {s.batch, s.seqlen_q, s.n_heads, s.kv_lora_rank, s.qk_rope_head_dim,
                          s.qk_nope_head_dim, s.v_head_dim, s.cache_batch, s.cache_len};
  const char *dnames[] = {"batch", "seqlen_q", "n_heads", "kv_lora_rank", "qk_rope_head_dim",
                          "qk_nope_head_dim", "v_head_dim", "cache_batch", "cache_len"};
  for (int i = 0; i < 9; ++i)
    if (dims[i] <= 0 || dims[i] > (int64_t(1) << 31))
      return fail(MLA_ERR_SHAPE, "%s = %lld is out of range", dnames[i], (long long)dims[i]);
  if (s.batch > s.cache_batch)
    return fail(MLA_ERR_RANGE, "batch %lld exceeds cache_batch %lld", (long long)s.batch, (long long)s.cache_batch);
  if (end_pos < 1 || end_pos > s.cache_len)
    return fail(MLA_ERR_RANGE, "end_pos %lld outside [1, cache_len=%lld]", (long long)end_pos, (long long)s.cache_len);
  if (s.seqlen_q > end_pos)
    return fail(MLA_ERR_RANGE, "seqlen_q %lld exceeds end_pos %lld", (long long)s.seqlen_q, (long long)end_pos);
  if ((k_pe_new == nullptr) != (pe_cache == nullptr))
    return fail(MLA_ERR_NULL, "k_pe_new and pe_cache must both be given or both be NULL");
  const int64_t T = s.batch * s.seqlen_q, rows = s.cache_batch * s.cache_len;
  if (T > (int64_t(1) << 31) || rows > (int64_t(1) << 40) ||
      double(s.n_heads) * double(rows) * double(std::max(s.qk_nope_head_dim, s.v_head_dim)) > 0x1p56)
    return fail(MLA_ERR_SHAPE, "batch * seqlen_q or the caches' element count is too large");
  mla::ExpandCall e;
  bool use_mfma = false;
  // the checks of mla_expand_kv for the B * S new tokens (path chosen below, after placement)
  int32_t st = plan_expand(T, s.n_heads, s.kv_lora_rank, s.qk_nope_head_dim, s.v_head_dim, eps, dtype,
                           MLA_PATH_PLAIN, e, use_mfma);
  if (st != MLA_OK) return st;
  const bool with_pe = pe_cache != nullptr;
  if (with_pe && s.qk_rope_head_dim % int64_t(16 / elem_size(dtype)))
    return fail(MLA_ERR_ALIGN, "qk_rope_head_dim must be a multiple of %lld elements (16-byte rows)",
                (long long)(16 / elem_size(dtype)));
  e.S_in = s.seqlen_q;
  e.out_seq_stride = s.cache_len;
  e.out_row0 = end_pos - s.seqlen_q;
  e.out_rows = rows;
  e.R = s.qk_rope_head_dim;
  e.k_pe = with_pe ? k_pe_new : nullptr;  // placeholders: the path check looks at the rope copy
  e.pe_out = with_pe ? pe_cache : nullptr;
  st = choose_expand_path(e, path, use_mfma);
  if (st != MLA_OK) return st;
  const size_t es = elem_size(dtype);
  const void *ptrs[] = {c_kv_new, rms_w, wkv_b, k_pe_new, k_cache, v_cache, pe_cache};
  const char *names[] = {"c_kv_new", "rms_w", "wkv_b", "k_pe_new", "k_cache", "v_cache", "pe_cache"};
  const size_t sizes[] = {size_t(T * s.kv_lora_rank) * es, size_t(s.kv_lora_rank) * es,
                          size_t(s.n_heads * (s.qk_nope_head_dim + s.v_head_dim) * s.kv_lora_rank) * es,
                          size_t(T * s.qk_rope_head_dim) * es, size_t(s.n_heads * rows * s.qk_nope_head_dim) * es,
                          size_t(s.n_heads * rows * s.v_head_dim) * es, size_t(rows * s.qk_rope_head_dim) * es};
  if (with_pe) return run_expand_call(e, use_mfma, ptrs, sizes, names, 4, 3, workspace, workspace_bytes, stream);
  const void *p2[] = {c_kv_new, rms_w, wkv_b, k_cache, v_cache};
  const char *n2[] = {"c_kv_new", "rms_w", "wkv_b", "k_cache", "v_cache"};
  const size_t s2[] = {sizes[0], sizes[1], sizes[2], sizes[4], sizes[5]};
  return run_expand_call(e, use_mfma, p2, s2, n2, 3, 2, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// The body of mla_cache_append and mla_cache_append_paged (block_table and paged null for
// contiguous caches).
int32_t cache_append_call(const void *c_kv_new, const void *k_pe_new, const void *rms_w, float eps,
                          const int32_t *seq_lens, int64_t end_pos, const int32_t *block_table,
                          const mla_paged_cache *paged, void *kv_cache, void *pe_cache,
                          const mla_attn_shape *shape, int32_t dtype, void *stream) {
  if (!shape) return fail(MLA_ERR_NULL, "shape is NULL");
  if (dtype != MLA_DTYPE_F32 && dtype != MLA_DTYPE_BF16) return fail(MLA_ERR_DTYPE, "unknown dtype %d", dtype);
  mla_attn_shape s = *shape;
  if (paged) {
    const mla_paged_cache &pg = *paged;
    if (pg.page_size < 1 || pg.page_size > (int64_t(1) << 20))
      return fail(MLA_ERR_SHAPE, "page_size = %lld outside [1, 1048576]", (long long)pg.page_size);
    if (pg.num_pages < 1 || pg.num_pages > (int64_t(1) << 31) - 1)
      return fail(MLA_ERR_SHAPE, "num_pages = %lld outside [1, 2^31 - 1]", (long long)pg.num_pages);
    if (pg.max_pages_per_seq < 1 || pg.max_pages_per_seq > (int64_t(1) << 31) - 1)
      return fail(MLA_ERR_SHAPE, "max_pages_per_seq = %lld outside [1, 2^31 - 1]", (long long)pg.max_pages_per_seq);
    if (s.batch > 0 && s.batch * pg.max_pages_per_seq > (int64_t(1) << 31) - 1)
      return fail(MLA_ERR_SHAPE, "batch * max_pages_per_seq is too large");
    if (pg.num_pages * pg.page_size > (int64_t(1) << 40)) return fail(MLA_ERR_SHAPE, "num_pages * page_size is too large");
    s.cache_batch = s.batch;
    s.cache_len = std::min<int64_t>(pg.max_pages_per_seq * pg.page_size, int64_t(1) << 31);
  }
  const int64_t dims[] = {s.batch, s.seqlen_q, s.kv_lora_rank, s.qk_rope_head_dim, s.cache_batch, s.cache_len};
  const char *dnames[] = {"batch", "seqlen_q", "kv_lora_rank", "qk_rope_head_dim", "cache_batch", "cache_len"};
  for (int i = 0; i < 6; ++i)
    if (dims[i] <= 0 || dims[i] > (int64_t(1) << 31))
      return fail(MLA_ERR_SHAPE, "%s = %lld is out of range", dnames[i], (long long)dims[i]);
  if (s.batch > s.cache_batch)
    return fail(MLA_ERR_RANGE, "batch %lld exceeds cache_batch %lld", (long long)s.batch, (long long)s.cache_batch);
  if (end_pos < 1 || end_pos > s.cache_len)
    return fail(MLA_ERR_RANGE, "end_pos %lld outside [1, cache_len=%lld]", (long long)end_pos, (long long)s.cache_len);
  if (s.seqlen_q > end_pos)
    return fail(MLA_ERR_RANGE, "seqlen_q %lld exceeds end_pos %lld", (long long)s.seqlen_q, (long long)end_pos);
  if (s.batch * s.seqlen_q > (int64_t(1) << 31) / 4)
    return fail(MLA_ERR_SHAPE, "batch*seqlen_q = %lld is too large", (long long)(s.batch * s.seqlen_q));
  if (!(eps >= 0.f) || eps > 1.f) return fail(MLA_ERR_SHAPE, "eps must be in [0, 1]");
  const int64_t ealign = 16 / int64_t(elem_size(dtype));
  if (s.kv_lora_rank % ealign || s.qk_rope_head_dim % ealign)
    return fail(MLA_ERR_ALIGN, "kv_lora_rank and qk_rope_head_dim must be multiples of %lld elements (16-byte rows)",
                (long long)ealign);
  const void *ptrs[] = {c_kv_new, k_pe_new, rms_w, kv_cache, pe_cache};
  const char *names[] = {"c_kv_new", "k_pe_new", "rms_w", "kv_cache", "pe_cache"};
  for (int i = 0; i < 5; ++i) {
    if (!ptrs[i]) return fail(MLA_ERR_NULL, "%s is NULL", names[i]);
    if (misaligned(ptrs[i])) return fail(MLA_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
  }
  if (seq_lens && (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
    return fail(MLA_ERR_ALIGN, "seq_lens is not 4-byte aligned");
  const size_t es = elem_size(dtype);
  const size_t toks = size_t(s.batch * s.seqlen_q);
  const size_t in_bytes[] = {toks * size_t(s.kv_lora_rank) * es, toks * size_t(s.qk_rope_head_dim) * es,
                             size_t(s.kv_lora_rank) * es};
  const size_t cache_rows = paged ? size_t(paged->num_pages * paged->page_size) : size_t(s.cache_batch * s.cache_len);
  const size_t kv_bytes = cache_rows * size_t(s.kv_lora_rank) * es;
  const size_t pe_bytes = cache_rows * size_t(s.qk_rope_head_dim) * es;
  if (overlaps(kv_cache, kv_bytes, pe_cache, pe_bytes)) return fail(MLA_ERR_SHAPE, "kv_cache overlaps pe_cache");
  for (int i = 0; i < 3; ++i) {
    if (overlaps(kv_cache, kv_bytes, ptrs[i], in_bytes[i])) return fail(MLA_ERR_SHAPE, "kv_cache overlaps %s", names[i]);
    if (overlaps(pe_cache, pe_bytes, ptrs[i], in_bytes[i])) return fail(MLA_ERR_SHAPE, "pe_cache overlaps %s", names[i]);
  }
  if (seq_lens && (overlaps(kv_cache, kv_bytes, seq_lens, size_t(s.batch) * 4) ||
                   overlaps(pe_cache, pe_bytes, seq_lens, size_t(s.batch) * 4)))
    return fail(MLA_ERR_SHAPE, "a cache overlaps seq_lens");
  if (block_table) {
    const size_t tb = size_t(s.batch * paged->max_pages_per_seq) * 4;
    if (overlaps(kv_cache, kv_bytes, block_table, tb) || overlaps(pe_cache, pe_bytes, block_table, tb))
      return fail(MLA_ERR_SHAPE, "a cache overlaps block_table");
  }
  mla::AppendCall a{};
  a.B = s.batch; a.S = s.seqlen_q; a.C = s.kv_lora_rank; a.R = s.qk_rope_head_dim; a.Tmax = s.cache_len;
  a.end_pos = end_pos; a.seq_lens = seq_lens; a.eps = eps; a.dtype = dtype;
  a.c_kv_new = c_kv_new; a.k_pe_new = k_pe_new; a.rms_w = rms_w; a.kv_cache = kv_cache; a.pe_cache = pe_cache;
  a.kv_ps = s.kv_lora_rank; a.pe_ps = s.qk_rope_head_dim;
  a.kv_bs = paged ? 0 : s.cache_len * a.kv_ps;
  a.pe_bs = paged ? 0 : s.cache_len * a.pe_ps;
  a.stream = static_cast<hipStream_t>(stream);
  if (paged) {
    a.block_table = block_table;
    a.page_size = paged->page_size; a.num_pages = paged->num_pages; a.max_pages = paged->max_pages_per_seq;
  }
  hipError_t e = mla::cache_append(a);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return MLA_OK;
}

}  // namespace

extern "C" {

int32_t mla_cache_append(const void *c_kv_new, const void *k_pe_new, const void *rms_w, float eps,
                         const int32_t *seq_lens, int64_t end_pos, void *kv_cache, void *pe_cache,
                         const mla_attn_shape *shape, int32_t dtype, void *stream) {
  clear_error();
  return cache_append_call(c_kv_new, k_pe_new, rms_w, eps, seq_lens, end_pos, nullptr, nullptr, kv_cache, pe_cache,
                           shape, dtype, stream);
}

int32_t mla_cache_append_paged(const void *c_kv_new, const void *k_pe_new, const void *rms_w, float eps,
                               const int32_t *seq_lens, int64_t max_seq_len, const int32_t *block_table,
                               void *kv_pages, void *pe_pages, const mla_attn_shape *shape,
                               const mla_paged_cache *paged, int32_t dtype, void *stream) {
  clear_error();
  if (!paged) return fail(MLA_ERR_NULL, "paged is NULL");
  if (!block_table) return fail(MLA_ERR_NULL, "block_table is NULL");
  if (reinterpret_cast<uintptr_t>(block_table) & 3u) return fail(MLA_ERR_ALIGN, "block_table is not 4-byte aligned");
  return cache_append_call(c_kv_new, k_pe_new, rms_w, eps, seq_lens, max_seq_len, block_table, paged, kv_pages,
                           pe_pages, shape, dtype, stream);
}

}  // extern "C"

extern "C" {

int32_t mla_naive_attn(const void *q_nope, const void *q_pe, const void *k_nope, const void *v, const void *pe_cache,
                       int64_t end_pos, float softmax_scale, void *out, const mla_attn_shape *shape, int32_t dtype,
                       int32_t path, void *stream) {
  clear_error();
  if (!shape) return fail(MLA_ERR_NULL, "shape is NULL");
  if (dtype != MLA_DTYPE_F32 && dtype != MLA_DTYPE_BF16) return fail(MLA_ERR_DTYPE, "unknown dtype %d", dtype);
  const mla_attn_shape &s = *shape;
  const int64_t dims[] = {s.batch, s.seqlen_q, s.n_heads, s.qk_rope_head_dim, s.qk_nope_head_dim,
                          s.v_head_dim, s.cache_batch, s.cache_len};
  const char *dnames[] = {"batch", "seqlen_q", "n_heads", "qk_rope_head_dim", "qk_nope_head_dim",
                          "v_head_dim", "cache_batch", "cache_len"};
  for (int i = 0; i < 8; ++i)
    if (dims[i] <= 0 || dims[i] > (int64_t(1) << 31))
      return fail(MLA_ERR_SHAPE, "%s = %lld is out of range", dnames[i], (long long)dims[i]);
  if (s.batch > s.cache_batch)
    return fail(MLA_ERR_RANGE, "batch %lld exceeds cache_batch %lld", (long long)s.batch, (long long)s.cache_batch);
  if (end_pos < 1 || end_pos > s.cache_len)
    return fail(MLA_ERR_RANGE, "end_pos %lld outside [1, cache_len=%lld]", (long long)end_pos, (long long)s.cache_len);
  if (s.seqlen_q > end_pos)
    return fail(MLA_ERR_RANGE, "seqlen_q %lld exceeds end_pos %lld", (long long)s.seqlen_q, (long long)end_pos);
  const int64_t rows = s.batch * s.seqlen_q * s.n_heads;
  if (rows > (int64_t(1) << 31) / 4) return fail(MLA_ERR_SHAPE, "batch*seqlen_q*n_heads = %lld is too large", (long long)rows);
  const int64_t ealign = 16 / int64_t(elem_size(dtype));
  if (s.qk_rope_head_dim % ealign || s.qk_nope_head_dim % ealign || s.v_head_dim % ealign)
    return fail(MLA_ERR_ALIGN, "qk_rope_head_dim, qk_nope_head_dim and v_head_dim must be multiples of %lld elements",
                (long long)ealign);
  if (!(softmax_scale == softmax_scale) || softmax_scale <= 0.f || softmax_scale > 1e30f)
    return fail(MLA_ERR_SHAPE, "softmax_scale must be a positive finite number");
  if (path != MLA_PATH_AUTO && path != MLA_PATH_PLAIN && path != MLA_PATH_MFMA)
    return fail(MLA_ERR_UNSUPPORTED, "unknown path %d", path);
  const void *ptrs[] = {q_nope, q_pe, k_nope, v, pe_cache, out};
  const char *names[] = {"q_nope", "q_pe", "k_nope", "v", "pe_cache", "out"};
  for (int i = 0; i < 6; ++i) {
    if (!ptrs[i]) return fail(MLA_ERR_NULL, "%s is NULL", names[i]);
    if (misaligned(ptrs[i])) return fail(MLA_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
  }
  const size_t es = elem_size(dtype);
  const size_t kv_rows = size_t(s.n_heads * s.cache_batch * s.cache_len);
  const size_t bytes_in[] = {size_t(rows * s.qk_nope_head_dim) * es, size_t(rows * s.qk_rope_head_dim) * es,
                             kv_rows * size_t(s.qk_nope_head_dim) * es, kv_rows * size_t(s.v_head_dim) * es,
                             size_t(s.cache_batch * s.cache_len * s.qk_rope_head_dim) * es};
  const size_t out_bytes = size_t(rows * s.v_head_dim) * es;
  for (int i = 0; i < 5; ++i)
    if (overlaps(out, out_bytes, ptrs[i], bytes_in[i])) return fail(MLA_ERR_SHAPE, "out overlaps %s", names[i]);
  mla::NaiveCall c{};
  c.B = s.batch; c.S = s.seqlen_q; c.H = s.n_heads; c.R = s.qk_rope_head_dim; c.Dn = s.qk_nope_head_dim;
  c.Dv = s.v_head_dim; c.Bmax = s.cache_batch; c.Tmax = s.cache_len; c.end_pos = end_pos;
  c.scale = softmax_scale; c.dtype = dtype;
  c.q_nope = q_nope; c.q_pe = q_pe; c.k_nope = k_nope; c.v = v; c.pe = pe_cache; c.out = out;
  c.stream = static_cast<hipStream_t>(stream);
  bool use_mfma = false;
  if (path != MLA_PATH_PLAIN) {
    const char *why = "";
    use_mfma = mla::mfma_naive_supported(c, &why);
    if (path == MLA_PATH_MFMA && !use_mfma) return fail(MLA_ERR_UNSUPPORTED, "matrix-core path: %s", why);
  }
  hipError_t e = use_mfma ? mla::mfma_naive_attn(c) : mla::plain_naive_attn(c);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return MLA_OK;
}

}  // extern "C"
