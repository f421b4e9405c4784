/*
 * mla_absorb.h -- C ABI of the MI355X (gfx950) MLA absorb-attention library.
 *
 * Two operations, each a set of HIP kernels enqueued on a caller stream:
 *
 *   mla_absorb_attn  DeepSeek-V3 Multi-Head Latent Attention in "absorb" form, as the page
 *                    "Naive vs Absorb Attention Implementations in DeepSeek-V3" describes it
 *                    (sections "Absorb Implementation Cache Design" and "Absorb Path
 *                    Execution"): the no-rope query is absorbed through each head's W_UK
 *                    slice of wkv_b into the kv_lora_rank latent space, scored against the
 *                    compressed kv_cache plus the separate pe_cache, softmax-normalised over
 *                    the cached positions, summed over kv_cache in latent space, and
 *                    projected out through each head's W_UV slice.
 *
 *   mla_expand_kv    "Latent KV expansion with split" (kernelindex.com, operation 064):
 *                    RMSNorm over the latent, the wkv_b projection to
 *                    n_heads * (qk_nope_head_dim + v_head_dim), then reshape, transpose and
 *                    split into head-major K_nope and V (the naive path's keys and values).
 *
 * Conventions shared by every entry point
 *   - Data pointers are DEVICE pointers (hipMalloc'd or torch CUDA tensors) on the current HIP
 *     device; the caller owns every buffer, including the workspace.  The library keeps no
 *     pointer after a call returns and never modifies inputs.
 *   - All tensors are row-major (innermost index contiguous) and of one element type:
 *     MLA_DTYPE_F32 (float) or MLA_DTYPE_BF16 (bfloat16 stored as uint16).  They are dense
 *     unless mla_attn_options.strides says otherwise (the absorb-attention entry points only).
 *     Every pointer must be 16-byte aligned.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL means the default stream); results
 *     are valid once the stream has synchronised.  Calls on one stream are ordered; concurrent
 *     calls on different streams must not share a workspace.
 *   - Every argument is validated before any HIP call: a failing call returns a negative status,
 *     enqueues nothing and sets a thread-local message (mla_last_error).  Launch failures return
 *     MLA_ERR_HIP.  Nothing aborts and no C++ exception crosses the ABI.
 *   - Accumulation, softmax and normalisation run in fp32; bf16 outputs are rounded to nearest
 *     even.
 */
#ifndef MLA_ABSORB_H
#define MLA_ABSORB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------------------------- */
#define MLA_OK 0
#define MLA_ERR_NULL (-1)        /* a required pointer is NULL                                 */
#define MLA_ERR_SHAPE (-2)       /* a size is not positive, or sizes disagree                  */
#define MLA_ERR_DTYPE (-3)       /* unknown element type                                       */
#define MLA_ERR_RANGE (-4)       /* end_pos / batch beyond the cache capacity, S > end_pos     */
#define MLA_ERR_ALIGN (-5)       /* a pointer is not 16-byte aligned                           */
#define MLA_ERR_WORKSPACE (-6)   /* workspace missing or smaller than the size query returns   */
#define MLA_ERR_HIP (-7)         /* a HIP runtime call or kernel launch failed                 */
#define MLA_ERR_UNSUPPORTED (-8) /* option or shape the requested kernel path cannot run       */

/* ---- element types ------------------------------------------------------------------------ */
#define MLA_DTYPE_F32 0
#define MLA_DTYPE_BF16 1

/* ---- kernel paths (mla_attn_options.path) --------------------------------------------------- */
#define MLA_PATH_AUTO 0    /* matrix-core kernels when the shape allows, else the plain path   */
#define MLA_PATH_PLAIN 1   /* plain vector-ALU kernels: any shape, fp32 or bf16 (slow)          */
#define MLA_PATH_MFMA 2    /* bf16 matrix-core kernels only; MLA_ERR_UNSUPPORTED otherwise      */

/* Sizes of one absorb-attention call (names follow DeepSeek-V3's ModelArgs). */
typedef struct mla_attn_shape {
  int64_t batch;            /* B   sequences attended: rows [0, B) of the caches               */
  int64_t seqlen_q;         /* S   new query tokens per sequence (1 = decode)                  */
  int64_t n_heads;          /* H                                                                */
  int64_t kv_lora_rank;     /* C   latent width                                                 */
  int64_t qk_rope_head_dim; /* R   rope width of q_pe and pe_cache                              */
  int64_t qk_nope_head_dim; /* Dn  no-rope query width (rows of W_UK per head)                  */
  int64_t v_head_dim;       /* Dv  value width (rows of W_UV per head)                          */
  int64_t cache_batch;      /* Bmax rows allocated in kv_cache / pe_cache (>= B)                */
  int64_t cache_len;        /* Tmax positions allocated per cache row (>= end_pos)              */
} mla_attn_shape;

/*
 * Element strides of the tensors of an absorb-attention call, for tensors that are views of larger
 * ones.  The page's absorb path splits each head's query into its no-rope part q_nope and its
 * rotary part q_pe ("Naive vs Absorb Attention Implementations in DeepSeek-V3", section "Absorb
 * Path Execution"), so the two usually arrive as the two halves of one [B, S, H, Dn + R] tensor:
 * then q_nope_row = q_pe_row = Dn + R and q_pe points Dn elements past q_nope.  Likewise kv_cache
 * and pe_cache may be the two parts of one [Bmax, Tmax, C + R] cache (kv_pos = pe_pos = C + R).
 *
 * The innermost index is always contiguous.  A field of 0 means the dense value given in its
 * comment.  A query row is one (b, s, h); rows are evenly spaced: row (b, s, h) of q_nope starts
 * at ((b * S + s) * H + h) * q_nope_row.  Every stride must be at least the row width it steps
 * over and keep every row 16-byte aligned (a multiple of 16 bytes); the extents they imply are
 * what the overlap checks and the kernels' bounds use.
 */
typedef struct mla_attn_strides {
  int64_t q_nope_row; /* between consecutive query rows of q_nope; dense: Dn                    */
  int64_t q_pe_row;   /* between consecutive query rows of q_pe; dense: R                       */
  int64_t out_row;    /* between consecutive rows of out; dense: Dv                             */
  int64_t kv_batch;   /* between cache rows b and b + 1 of kv_cache; dense: Tmax * kv_pos       */
  int64_t kv_pos;     /* between positions t and t + 1 of kv_cache (and of a kv page); dense: C */
  int64_t pe_batch;   /* between cache rows b and b + 1 of pe_cache; dense: Tmax * pe_pos       */
  int64_t pe_pos;     /* between positions t and t + 1 of pe_cache (and of a pe page); dense: R */
} mla_attn_strides;

/* Optional knobs of mla_absorb_attn; pass NULL for the defaults (all zero). */
typedef struct mla_attn_options {
  int32_t num_splits; /* 0: the planner chooses; n > 0: split [0, end_pos) into n ranges        */
  int32_t path;       /* MLA_PATH_*                                                             */
  const mla_attn_strides *strides; /* NULL: every tensor dense (row-major, no gaps).  Page pools
                                      take kv_pos / pe_pos (rows within and across pages; a
                                      page is page_size such rows) and ignore the batch strides */
} mla_attn_options;

/*
 * Bytes of device workspace mla_absorb_attn needs for this shape, end_pos, dtype and options
 * (the absorbed query and the per-split softmax partials).  Returns 0 when the arguments are
 * invalid (the same checks as mla_absorb_attn; see mla_last_error).
 */
size_t mla_absorb_attn_workspace_size(const mla_attn_shape *shape, int64_t end_pos, int32_t dtype,
                                      const mla_attn_options *options);

/*
 * Absorb-form MLA attention ("Naive vs Absorb Attention Implementations in DeepSeek-V3",
 * section "Absorb Path Execution").
 *
 *   q_nope    [B, S, H, Dn]                 no-rope query
 *   q_pe      [B, S, H, R]                  rope query (already rotated)
 *   kv_cache  [Bmax, Tmax, C]               compressed latent per cached position (already
 *                                           normalised; this call does no RMSNorm)
 *   pe_cache  [Bmax, Tmax, R]               rope key per cached position, shared by all heads
 *   wkv_b     [H * (Dn + Dv), C]            Linear weight; head h owns rows h*(Dn+Dv) ..
 *                                           (h+1)*(Dn+Dv)-1, the first Dn being W_UK[h] and the
 *                                           last Dv being W_UV[h]
 *   end_pos   attend to cache positions [0, end_pos) of rows [0, B)
 *   softmax_scale  multiplies (q_lat . kv + q_pe . pe) before the softmax
 *   out       [B, S, H, Dv]                 written; must not alias any input or the workspace
 *
 * With S > 1 the S query tokens sit at positions end_pos - S .. end_pos - 1 and query s sees
 * cache positions t <= end_pos - S + s (causal within the chunk); the caller has already
 * written their kv/pe rows.  Requires 1 <= S <= end_pos <= Tmax and 1 <= B <= Bmax.
 * workspace: at least mla_absorb_attn_workspace_size(...) bytes of device memory (may be NULL
 * when that size is 0).  Returns MLA_OK or a negative MLA_ERR_* status.
 */
int32_t mla_absorb_attn(const void *q_nope, const void *q_pe, const void *kv_cache,
                        const void *pe_cache, const void *wkv_b, int64_t end_pos,
                        float softmax_scale, void *out, const mla_attn_shape *shape,
                        int32_t dtype, const mla_attn_options *options, void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * mla_absorb_attn without a workspace argument, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * workspace lives in a file-scope device array of MLA_NOALLOC_SCRATCH_BYTES in the library (one
 * copy per GPU, held until the process ends; its device address is looked up once per device, on
 * the first call with that device current).  The call allocates nothing: no hipMalloc, no hipFree.
 *
 * Arguments, layouts, results and errors are those of mla_absorb_attn.  A call whose workspace
 * (mla_absorb_attn_workspace_size) exceeds MLA_NOALLOC_SCRATCH_BYTES fails with
 * MLA_ERR_WORKSPACE before any HIP call (64 MiB covers, for example, the DeepSeek-V3 decode step
 * of 32 sequences x 128 heads at any cache length, which takes 38.5 MB).  Every call on a GPU uses
 * that GPU's one array and leaves its contents behind; nothing in it has to start at zero (each
 * call writes every slot it reads).  Calls whose executions overlap on one GPU -- on different
 * streams, or from different threads -- race on the array and must be serialised by the caller.
 */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

int32_t mla_absorb_attn_noalloc(const void *q_nope, const void *q_pe, const void *kv_cache,
                                const void *pe_cache, const void *wkv_b, int64_t end_pos,
                                float softmax_scale, void *out, const mla_attn_shape *shape,
                                int32_t dtype, const mla_attn_options *options, void *stream);

/*
 * Absorb-form MLA attention over a ragged batch: sequence b attends to its own cache positions
 * [0, seq_lens[b]) (the page's uniform slice "[:bsz, :end_pos]" taken per sequence; its S query
 * tokens sit at seq_lens[b] - S .. seq_lens[b] - 1, causal as in mla_absorb_attn).
 *
 *   seq_lens     DEVICE array of B int32 lengths (4-byte aligned), read by the kernels on the
 *                stream; the caller guarantees S <= seq_lens[b] <= max_seq_len.  A value outside
 *                that range is clamped into it, so no call ever reads a cache position at or past
 *                max_seq_len (such a sequence's output is then that of the clamped length).
 *   max_seq_len  upper bound of the lengths; 1 <= S <= max_seq_len <= Tmax.  It plays the role
 *                of end_pos for validation and split planning.
 * workspace: mla_absorb_attn_ragged_workspace_size(shape, max_seq_len, ...) bytes.  With an
 * automatic split count the matrix-core kernels plan the batch on the device from the lengths:
 * a skewed batch (positions filling at most about a third of batch x the longest length) is cut
 * into chunks of about one common length (a multiple of 32), one per workgroup, so long
 * sequences take more workgroups than short ones (up to four times the splits of a uniform
 * batch); any other batch keeps the uniform split count.
 * Every other argument, the layouts and the error behaviour are those of mla_absorb_attn;
 * out, workspace and seq_lens must not overlap.  Returns MLA_OK or a negative MLA_ERR_* status
 * (MLA_ERR_NULL / MLA_ERR_ALIGN for seq_lens).
 */
size_t mla_absorb_attn_ragged_workspace_size(const mla_attn_shape *shape, int64_t max_seq_len,
                                             int32_t dtype, const mla_attn_options *options);

int32_t mla_absorb_attn_ragged(const void *q_nope, const void *q_pe, const void *kv_cache,
                               const void *pe_cache, const void *wkv_b, const int32_t *seq_lens,
                               int64_t max_seq_len, float softmax_scale, void *out,
                               const mla_attn_shape *shape, int32_t dtype,
                               const mla_attn_options *options, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * Paged caches.  The DeepSeek Sparse Attention explainer (sider.ai, sections on efficient batching
 * and memory, and on runtime complexity) notes that serving runtimes keep the KV cache in pages
 * (paged attention) under continuous batching.  Here the two caches of "Memory Layout and Cache
 * Structure" are pools of fixed-size pages:
 *
 *   kv_pages     [num_pages, page_size, C]   compressed latent (normalised, as kv_cache)
 *   pe_pages     [num_pages, page_size, R]   rope key (as pe_cache)
 *   block_table  DEVICE int32 [B, max_pages_per_seq]: position t of sequence b lives in page
 *                block_table[b, t / page_size], row t % page_size
 *
 * The attention is that of mla_absorb_attn_ragged over the cache each sequence's pages spell out.
 */
typedef struct mla_paged_cache {
  int64_t page_size;          /* positions per page, >= 1; the matrix-core kernels need a power
                                 of two >= 32 (other sizes run on the plain kernels) */
  int64_t num_pages;          /* pages in kv_pages and in pe_pages, >= 1 */
  int64_t max_pages_per_seq;  /* row length of block_table, >= 1 */
} mla_paged_cache;

/*
 * Bytes of device workspace mla_absorb_attn_paged needs for these arguments (0 if none, and 0
 * with mla_last_error set when they are invalid).  The split plan of a paged call may differ from
 * that of a contiguous one (the matrix-core kernels start every split on a 32-position boundary
 * and bound the pages one workgroup reads), so the size has its own query; it covers the balanced
 * plan of a call with seq_lens (see mla_absorb_attn_ragged), which a call without needs less of.
 */
size_t mla_absorb_attn_paged_workspace_size(const mla_attn_shape *shape, int64_t max_seq_len,
                                            const mla_paged_cache *paged, int32_t dtype,
                                            const mla_attn_options *options);

/*
 * Absorb-form MLA attention over paged caches (layout above).  Sequence b attends to its
 * positions [0, len_b) with len_b = seq_lens[b] (DEVICE int32 [B], 4-byte aligned) or, when
 * seq_lens is NULL, len_b = max_seq_len for every sequence; queries and the causal mask as in
 * mla_absorb_attn_ragged, lengths clamped to [S, max_seq_len] likewise.
 *
 *   block_table  DEVICE int32 [B, max_pages_per_seq], 4-byte aligned.  Entries of pages a
 *                sequence reads must be valid page ids; an id outside [0, num_pages) is clamped
 *                into it, so no call reads outside the pools.
 *   max_seq_len  1 <= S <= max_seq_len <= max_pages_per_seq * page_size.
 *   shape        B, S, H, C, R, Dn, Dv as for mla_absorb_attn; cache_batch and cache_len are
 *                not used.
 *   workspace    at least mla_absorb_attn_paged_workspace_size(...) bytes.
 * Pointers, ownership, options and errors as in mla_absorb_attn; out, the workspace, seq_lens
 * and block_table must not overlap.  Returns MLA_OK or a negative MLA_ERR_* status.
 */
int32_t mla_absorb_attn_paged(const void *q_nope, const void *q_pe, const void *kv_pages,
                              const void *pe_pages, const void *wkv_b, const int32_t *block_table,
                              const int32_t *seq_lens, int64_t max_seq_len, float softmax_scale,
                              void *out, const mla_attn_shape *shape, const mla_paged_cache *paged,
                              int32_t dtype, const mla_attn_options *options, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * Absorb-form MLA attention over selected positions.  The DeepSeek Sparse Attention explainer
 * (sider.ai, sections on how DSA differs from dense attention and on fine-grained sparse
 * attention) describes a cheap pre-selector (the "lightning indexer") that keeps a short list of
 * positions per query token, after which exact attention runs over that list only.  The
 * selection itself needs trained weights and is the caller's; this call is the attention over it:
 *
 *   indices  DEVICE int32 [B, S, topk], 4-byte aligned: the positions query token (b, s) attends
 *            to, shared by all of its heads.  An entry counts if 0 <= idx <= p with p =
 *            len_b - S + s the token's own position (so a list naming every position gives
 *            mla_absorb_attn's causal result); any other value (e.g. -1 as padding) is ignored and
 *            never read.  Each counting entry is one term of the softmax (a repeated position
 *            counts twice).  A token with no counting entry gets out = 0.
 *   topk     entries per list, 1 <= topk <= 2^24.
 *   seq_lens DEVICE int32 [B] or NULL: len_b as in mla_absorb_attn_ragged (clamped to
 *            [S, end_pos]); NULL gives every sequence the length end_pos.
 *   end_pos  uniform length, or the bound of seq_lens; 1 <= S <= end_pos <= Tmax.
 *
 * Caches, weights, shapes, options and errors as in mla_absorb_attn (contiguous caches); the
 * matrix-core kernels need each 128-row block of query rows to be the heads of one token
 * (n_heads a multiple of 128, or seqlen_q 1 with n_heads <= 128), other shapes run on the plain
 * kernels.  workspace: mla_absorb_attn_sparse_workspace_size(...) bytes (splits cut the list
 * entries).  out, the workspace, indices and seq_lens must not overlap.
 */
size_t mla_absorb_attn_sparse_workspace_size(const mla_attn_shape *shape, int64_t end_pos,
                                             int64_t topk, int32_t dtype,
                                             const mla_attn_options *options);

int32_t mla_absorb_attn_sparse(const void *q_nope, const void *q_pe, const void *kv_cache,
                               const void *pe_cache, const void *wkv_b, const int32_t *indices,
                               int64_t topk, const int32_t *seq_lens, int64_t end_pos,
                               float softmax_scale, void *out, const mla_attn_shape *shape,
                               int32_t dtype, const mla_attn_options *options, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * Cache append, the step before attending: writes the S new tokens of each sequence into the
 * two caches mla_absorb_attn reads ("Naive vs Absorb Attention Implementations in DeepSeek-V3",
 * section "Memory Layout and Cache Structure": kv_cache holds each position's compressed latent,
 * pe_cache its rotary key).  The latent is stored RMS-normalised, with the norm of "Latent KV
 * expansion with split":
 *
 *   c_kv_new  [B, S, C]       raw compressed latent of the new tokens
 *   k_pe_new  [B, S, R]       their rope keys, already rotated
 *   rms_w     [C]             RMSNorm weight
 *   kv_cache  [Bmax, Tmax, C] row (b, p) := c_kv_new[b, s] / sqrt(mean_c c_kv_new[b, s, c]^2 + eps) * rms_w
 *   pe_cache  [Bmax, Tmax, R] row (b, p) := k_pe_new[b, s]
 *
 * with p = end_pos - S + s, the positions mla_absorb_attn gives the same S query tokens; with
 * seq_lens (DEVICE [B] int32, or NULL) p = seq_lens[b] - S + s, each length clamped to
 * [S, end_pos] as in mla_absorb_attn_ragged.  Every other cache row is left untouched.  The shape
 * descriptor supplies B, S, C, R, Bmax and Tmax (its other fields are not used); requires
 * 1 <= S <= end_pos <= Tmax, B <= Bmax, 0 <= eps <= 1.  The caches must not overlap each other or
 * any input.  Arithmetic in fp32, stores rounded to the element type.  Returns MLA_OK or a
 * negative MLA_ERR_* status (validation before any HIP call, as everywhere).
 */
int32_t mla_cache_append(const void *c_kv_new, const void *k_pe_new, const void *rms_w, float eps,
                         const int32_t *seq_lens, int64_t end_pos, void *kv_cache, void *pe_cache,
                         const mla_attn_shape *shape, int32_t dtype, void *stream);

/*
 * Cache append into paged caches (the page pools of mla_absorb_attn_paged): the rows of
 * mla_cache_append, written at row p % page_size of page block_table[b, p / page_size] for each
 * new token's position p (end_pos - S + s, or seq_lens[b] - S + s clamped to [S, max_seq_len]).
 * Page ids outside [0, num_pages) are clamped into it, as in mla_absorb_attn_paged.
 *   block_table  DEVICE int32 [B, max_pages_per_seq], 4-byte aligned
 *   max_seq_len  1 <= S <= max_seq_len <= max_pages_per_seq * page_size
 *   shape        B, S, C, R; cache_batch and cache_len are not used
 * The pools must not overlap each other, the new rows, seq_lens or the table.  Returns MLA_OK or
 * a negative MLA_ERR_* status.
 */
int32_t mla_cache_append_paged(const void *c_kv_new, const void *k_pe_new, const void *rms_w,
                               float eps, const int32_t *seq_lens, int64_t max_seq_len,
                               const int32_t *block_table, void *kv_pages, void *pe_pages,
                               const mla_attn_shape *shape, const mla_paged_cache *paged,
                               int32_t dtype, void *stream);

/*
 * Cache append fused into absorb attention: one call writes the new tokens' cache rows and then
 * attends over the caches with those rows in place (page "Naive vs Absorb Attention
 * Implementations in DeepSeek-V3", sections "Memory Layout and Cache Structure" and "Absorb Path
 * Execution": the step writes the current tokens' latent and rope key into the caches at
 * [start_pos, end_pos), then attends over [0, end_pos)).  The result, and every cache byte, is that
 * of mla_cache_append followed by mla_absorb_attn (seq_lens NULL) or mla_absorb_attn_ragged
 * (seq_lens given) on the same stream, bit for bit.  On the matrix-core path the rows are written
 * by the query-absorption kernel, so the call launches one kernel fewer; the plain path makes the
 * two calls.
 *   c_kv_new, k_pe_new, rms_w, eps   as mla_cache_append (dense [B, S, C], [B, S, R], [C])
 *   kv_cache, pe_cache               written, then read: the caches of mla_absorb_attn, with the
 *                                    strides of options (the rows go where the attention reads)
 *   seq_lens, end_pos                as mla_absorb_attn_ragged (seq_lens NULL: uniform end_pos)
 *   everything else                  as mla_absorb_attn
 * The workspace is that of mla_absorb_attn_workspace_size (seq_lens NULL) or
 * mla_absorb_attn_ragged_workspace_size.  The caches must not overlap each other, the queries,
 * wkv_b, out, the new rows, seq_lens or the workspace.  Returns MLA_OK or a negative MLA_ERR_*
 * status (validation before any HIP call).
 */
int32_t mla_absorb_attn_append(const void *q_nope, const void *q_pe, const void *c_kv_new,
                               const void *k_pe_new, const void *rms_w, float eps, void *kv_cache,
                               void *pe_cache, const void *wkv_b, const int32_t *seq_lens,
                               int64_t end_pos, float softmax_scale, void *out,
                               const mla_attn_shape *shape, int32_t dtype,
                               const mla_attn_options *options, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * The same over page pools: mla_cache_append_paged followed by mla_absorb_attn_paged, bit for
 * bit, in one call (arguments as those two; workspace from
 * mla_absorb_attn_paged_workspace_size).
 */
int32_t mla_absorb_attn_paged_append(const void *q_nope, const void *q_pe, const void *c_kv_new,
                                     const void *k_pe_new, const void *rms_w, float eps,
                                     void *kv_pages, void *pe_pages, const void *wkv_b,
                                     const int32_t *block_table, const int32_t *seq_lens,
                                     int64_t max_seq_len, float softmax_scale, void *out,
                                     const mla_attn_shape *shape, const mla_paged_cache *paged,
                                     int32_t dtype, const mla_attn_options *options,
                                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * Attention of the naive route ("Naive vs Absorb Attention Implementations in DeepSeek-V3",
 * section "Naive Path Execution") over keys and values that are already expanded, e.g. by
 * mla_expand_kv of the caches' Bmax*Tmax latent rows in (b, t) order:
 *
 *   q_nope    [B, S, H, Dn]          query
 *   q_pe      [B, S, H, R]           rope query (already rotated)
 *   k_nope    [H, Bmax, Tmax, Dn]    per-head no-rope keys, head-major
 *   v         [H, Bmax, Tmax, Dv]    per-head values, head-major
 *   pe_cache  [Bmax, Tmax, R]        rope key per position, shared by every head
 *   out       [B, S, H, Dv]          written: sum_t softmax_t(score) v[h, b, t] with
 *             score = (q_nope[b,s,h] . k_nope[h,b,t] + q_pe[b,s,h] . pe_cache[b,t]) * softmax_scale
 *
 * Positions and the causal mask are those of mla_absorb_attn (query s at end_pos - S + s sees
 * t <= that position).  The shape descriptor supplies B, S, H, R, Dn, Dv, Bmax and Tmax
 * (kv_lora_rank is not used).  path: MLA_PATH_AUTO picks the matrix-core kernel for bf16 at
 * R = 64, Dn = Dv = 128, else the plain one; MLA_PATH_MFMA refuses other shapes with
 * MLA_ERR_UNSUPPORTED.  Needs no workspace.  out must not overlap an input.  Returns MLA_OK or a
 * negative MLA_ERR_* status.
 */
int32_t mla_naive_attn(const void *q_nope, const void *q_pe, const void *k_nope, const void *v,
                       const void *pe_cache, int64_t end_pos, float softmax_scale, void *out,
                       const mla_attn_shape *shape, int32_t dtype, int32_t path, void *stream);

/*
 * Bytes of device workspace mla_expand_kv needs (the normalised latent n, which the matrix-core
 * path computes once per token and every head reuses; 0 for the plain path).  Returns 0 when the
 * arguments are invalid (the same checks as mla_expand_kv; see mla_last_error).
 */
size_t mla_expand_kv_workspace_size(int64_t n_tokens, int64_t n_heads, int64_t kv_lora_rank,
                                    int64_t qk_nope_head_dim, int64_t v_head_dim, int32_t dtype,
                                    int32_t path);

/*
 * Latent KV expansion with split (kernelindex.com operation 064).
 *
 *   c_kv    [T, C]                 raw compressed latent of T tokens
 *   rms_w   [C]                    RMSNorm weight
 *   wkv_b   [H * (Dn + Dv), C]     Linear weight, rows laid out as in mla_absorb_attn
 *   k_nope  [H, T, Dn]             written: k_nope[h,t,:] = rows h*(Dn+Dv) .. +Dn-1 of
 *                                  wkv_b applied to n[t]
 *   v       [H, T, Dv]             written: the next Dv rows applied to n[t]
 * where n[t,:] = c_kv[t,:] / sqrt(mean_c c_kv[t,c]^2 + eps) * rms_w.
 * workspace: at least mla_expand_kv_workspace_size(...) bytes of device memory, 16-byte aligned
 * (may be NULL when that size is 0); owned by the caller, not kept after the call.
 * k_nope and v must not alias the inputs, the workspace or each other.  Returns MLA_OK or
 * MLA_ERR_*.
 */
int32_t mla_expand_kv(const void *c_kv, const void *rms_w, const void *wkv_b, void *k_nope,
                      void *v, int64_t n_tokens, int64_t n_heads, int64_t kv_lora_rank,
                      int64_t qk_nope_head_dim, int64_t v_head_dim, float eps, int32_t dtype,
                      int32_t path, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Cache append of the naive route: the page "Naive vs Absorb Attention Implementations in
 * DeepSeek-V3" (sections "Memory Layout and Cache Structure" and "Naive Path Execution") has the
 * naive path produce keys and values through wkv_b and cache them at full width.  This writes the
 * S new tokens of each sequence into such caches, in the head-major layout mla_naive_attn reads:
 *
 *   c_kv_new  [B, S, C]              raw compressed latent of the new tokens
 *   k_pe_new  [B, S, R]              their rope keys, already rotated (or NULL)
 *   rms_w     [C], wkv_b [H * (Dn + Dv), C]   as in mla_expand_kv
 *   k_cache   [H, Bmax, Tmax, Dn]    row (h, b, p) := the K_nope row mla_expand_kv computes for
 *                                    token (b, s)
 *   v_cache   [H, Bmax, Tmax, Dv]    row (h, b, p) := its V row
 *   pe_cache  [Bmax, Tmax, R]        row (b, p) := k_pe_new[b, s] (or NULL, with k_pe_new NULL)
 *
 * with p = end_pos - S + s, the positions mla_naive_attn gives the same S query tokens.  Every
 * other cache row is left untouched.  The shape descriptor supplies B, S, H, C, R, Dn, Dv, Bmax
 * and Tmax; requires 1 <= S <= end_pos <= Tmax and B <= Bmax.  The rows written are bit-identical
 * to mla_expand_kv's rows for the same tokens, dtype and kernel path; MLA_PATH_AUTO takes the
 * matrix-core kernels where mla_expand_kv would, unless Bmax * Tmax exceeds 2^23 or R is not a
 * multiple of 8 (then the plain ones).  workspace: at least
 * mla_expand_kv_workspace_size(B * S, H, C, Dn, Dv, dtype, path) bytes.  The caches must not
 * overlap each other, an input or the workspace.  Returns MLA_OK or a negative MLA_ERR_* status.
 */
int32_t mla_expand_kv_append(const void *c_kv_new, const void *k_pe_new, const void *rms_w,
                             const void *wkv_b, float eps, int64_t end_pos, void *k_cache,
                             void *v_cache, void *pe_cache, const mla_attn_shape *shape,
                             int32_t dtype, int32_t path, void *workspace, size_t workspace_bytes,
                             void *stream);

/* ---- kernel timing (benchmark instrumentation) ----------------------------------------------
 * While a kernel's bit is set in the mask given to mla_timing_enable (bit k = kernel id k), every
 * launch of it from this thread carries a pair of HIP events on the launch stream.  A single
 * matrix-core kernel is launched with hipExtLaunchKernel, whose events take the dispatch's own
 * start and end times; the plain path's kernels are bracketed together by events recorded
 * before and after them.  mla_timing_collect waits for the recorded events and returns, per kernel id, the
 * number of launches and their summed duration in milliseconds since the previous collect, then
 * forgets them.  The library owns the events.  Returns MLA_OK, or MLA_ERR_HIP if an event call
 * failed (the affected launches are then missing from the totals). */
#define MLA_KERNEL_ABSORB_Q 0 /* query absorption through W_UK                 */
#define MLA_KERNEL_ATTN 1     /* split-KV scores, softmax, latent sum           */
#define MLA_KERNEL_COMBINE 2      /* split combine + projection out through W_UV */
#define MLA_KERNEL_EXPAND_PREP 3  /* per-token weighted latent and 1/rms          */
#define MLA_KERNEL_EXPAND 4       /* projection + head-major split               */
#define MLA_KERNEL_PLAIN 5        /* any kernel of the plain vector-ALU path, and the cache append */
#define MLA_KERNEL_NAIVE 6        /* matrix-core naive-route attention           */
#define MLA_NUM_KERNELS 7

int32_t mla_timing_enable(uint32_t kernel_mask);
int32_t mla_timing_collect(int32_t launches[MLA_NUM_KERNELS], double ms[MLA_NUM_KERNELS]);
/* Short name of a kernel id ("" for an unknown id). */
const char *mla_kernel_name(int32_t kernel_id);

/* Static text for a status code (never NULL). */
const char *mla_strerror(int32_t status);

/* Thread-local detail of the most recent failing call on this thread ("" if none). */
const char *mla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_ABSORB_H */
