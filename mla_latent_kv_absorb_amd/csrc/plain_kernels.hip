// Plain vector-ALU kernels: any shape, fp32 or bf16 storage, fp32 arithmetic.
//
// They compute the same absorb-form attention and latent expansion as the matrix-core kernels
// (page "Naive vs Absorb Attention Implementations in DeepSeek-V3", section "Absorb Path
// Execution"; kernelindex op 064 "Latent KV expansion with split"), one output element per
// thread with no tiling, and serve the fp32 workloads and shapes the matrix-core kernels do not
// take.
#include "common.h"
#include "launch.h"
#include "../../include/mla_absorb.h"

namespace mla {
namespace {

constexpr int kThreads = 256;

// q_lat[row, c] = sum_d q_nope[row, d] * W_UK[h, d, c]   (h = row % H)
template <typename T>
__global__ void __launch_bounds__(kThreads)
plain_absorb_q_kernel(const T *__restrict__ q_nope, const T *__restrict__ wkv_b,
                      float *__restrict__ q_lat, int64_t H, int64_t C, int64_t Dn, int64_t Dv, int64_t q_rs) {
  const int64_t row = blockIdx.x;
  const int64_t c = int64_t(blockIdx.y) * kThreads + threadIdx.x;
  if (c >= C) return;
  const int64_t h = row % H;
  const T *q = q_nope + row * q_rs;
  const T *w = wkv_b + h * (Dn + Dv) * C + c;
  float acc = 0.f;
  for (int64_t d = 0; d < Dn; ++d) acc = fmaf(Elem<T>::load(q, d), Elem<T>::load(w, d * C), acc);
  q_lat[row * C + c] = acc;
}

// Element offsets of position t of sequence b in the kv and pe arrays: b * batch stride + t *
// position stride for contiguous caches; for paged ones row t % page_size of the sequence's page
// for t (its id clamped into [0, num_pages)), rows counted across pages at the position stride.
__device__ __forceinline__ void cache_offsets(const AttnCall &a, int64_t b, int64_t t, int64_t &kv_off,
                                              int64_t &pe_off) {
  if (a.page_size == 0) {
    kv_off = b * a.kv_bs + t * a.kv_ps;
    pe_off = b * a.pe_bs + t * a.pe_ps;
    return;
  }
  int64_t pg = a.block_table[b * a.max_pages + t / a.page_size];
  pg = pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);
  const int64_t r = pg * a.page_size + t % a.page_size;
  kv_off = r * a.kv_ps;
  pe_off = r * a.pe_ps;
}

// One block per (row, split): online softmax over the split's visible positions.
// Writes m (largest scaled score, -inf if none visible), l (sum of exp(score - m)) and
// o[c] = sum exp(score - m) * kv[t, c].
template <typename T>
__global__ void __launch_bounds__(kThreads)
plain_attn_partial_kernel(const float *__restrict__ q_lat, const T *__restrict__ q_pe,
                          const T *__restrict__ kv, const T *__restrict__ pe,
                          float *__restrict__ part_ml, float *__restrict__ part_o, AttnCall a) {
  extern __shared__ float sm[];
  float *sq = sm;             // C   absorbed query
  float *sqp = sq + a.C;      // R   rope query
  float *so = sqp + a.R;      // C   running weighted sum
  float *sp = so + a.C;       // kThreads probabilities of the current chunk
  float *red = sp + kThreads; // 16
  int64_t *skv = reinterpret_cast<int64_t *>(red + 16);  // kThreads kv offsets of the current chunk
  int64_t *spe = skv + kThreads;                          // kThreads pe offsets

  const int64_t row = blockIdx.x;
  const int split = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t b = row / (a.S * a.H);
  const int64_t s = (row / a.H) % a.S;
  // this sequence's length (a ragged batch clamps seq_lens[b] to [S, end_pos])
  int64_t end_pos = a.end_pos;
  if (a.seq_lens) {
    end_pos = a.seq_lens[b];
    if (end_pos < a.S) end_pos = a.S;
    if (end_pos > a.end_pos) end_pos = a.end_pos;
  }
  const int64_t last = end_pos - a.S + s;  // last visible position of this query
  // the split's positions [t0, t1), or with an index list its entries [t0, t1)
  const int64_t t0 = int64_t(split) * a.split_len;
  int64_t t1 = t0 + a.split_len;
  if (a.topk > 0) {
    if (t1 > a.topk) t1 = a.topk;
  } else {
    if (t1 > end_pos) t1 = end_pos;
    if (t1 > last + 1) t1 = last + 1;
  }
  const int32_t *list = a.topk > 0 ? a.indices + (b * a.S + s) * a.topk : nullptr;

  for (int64_t c = tid; c < a.C; c += kThreads) { sq[c] = q_lat[row * a.C + c]; so[c] = 0.f; }
  for (int64_t r = tid; r < a.R; r += kThreads) sqp[r] = Elem<T>::load(q_pe, row * a.q_pe_rs + r);
  __syncthreads();

  float m = -INFINITY, l = 0.f;
  for (int64_t tc = t0; tc < t1; tc += kThreads) {
    const int n = int((t1 - tc) < kThreads ? (t1 - tc) : kThreads);
    bool ok = tid < n;
    if (ok) {
      int64_t t = tc + tid;
      if (list) {  // an entry counts if it names a visible position; others read row 0, weight 0
        t = list[tc + tid];
        ok = t >= 0 && t <= last;
        if (!ok) t = 0;
      }
      cache_offsets(a, b, t, skv[tid], spe[tid]);
    }
    __syncthreads();
    float sc = -INFINITY;
    if (ok) {
      const int64_t k0 = skv[tid], p0 = spe[tid];
      float acc = 0.f;
      for (int64_t c = 0; c < a.C; ++c) acc = fmaf(sq[c], Elem<T>::load(kv, k0 + c), acc);
      for (int64_t r = 0; r < a.R; ++r) acc = fmaf(sqp[r], Elem<T>::load(pe, p0 + r), acc);
      sc = acc * a.scale;
    }
    const float m_new = fmaxf(m, block_max(sc, red));
    const float p = ok ? expf(sc - m_new) : 0.f;
    sp[tid] = p;
    const float alpha = (m == -INFINITY) ? 0.f : expf(m - m_new);
    l = l * alpha + block_sum(p, red);  // block_sum synchronises, so sp is visible below
    for (int64_t c = tid; c < a.C; c += kThreads) {
      float acc = so[c] * alpha;
      for (int j = 0; j < n; ++j) acc = fmaf(sp[j], Elem<T>::load(kv, skv[j] + c), acc);
      so[c] = acc;
    }
    m = m_new;
    __syncthreads();
  }
  const int64_t idx = row * a.splits + split;
  if (tid == 0) { part_ml[2 * idx] = m; part_ml[2 * idx + 1] = l; }
  for (int64_t c = tid; c < a.C; c += kThreads) part_o[idx * a.C + c] = so[c];
}

// One block per row: merge the split partials into o_lat, then out = W_UV[h] o_lat.
template <typename T>
__global__ void __launch_bounds__(kThreads)
plain_merge_upproj_kernel(const float *__restrict__ part_ml, const float *__restrict__ part_o,
                          const T *__restrict__ wkv_b, T *__restrict__ out, AttnCall a) {
  extern __shared__ float sm[];
  float *so = sm;  // C
  const int64_t row = blockIdx.x;
  const int64_t h = row % a.H;
  const int tid = threadIdx.x;
  const float *ml = part_ml + 2 * row * a.splits;
  float M = -INFINITY;
  for (int i = 0; i < a.splits; ++i) M = fmaxf(M, ml[2 * i]);
  float den = 0.f;
  for (int i = 0; i < a.splits; ++i)
    if (ml[2 * i] != -INFINITY) den += expf(ml[2 * i] - M) * ml[2 * i + 1];
  const float inv = den > 0.f ? 1.f / den : 0.f;  // 0: a sparse row whose list names no visible position
  for (int64_t c = tid; c < a.C; c += kThreads) {
    float acc = 0.f;
    for (int i = 0; i < a.splits; ++i)
      if (ml[2 * i] != -INFINITY) acc = fmaf(expf(ml[2 * i] - M), part_o[(row * a.splits + i) * a.C + c], acc);
    so[c] = acc * inv;
  }
  __syncthreads();
  const T *wuv = wkv_b + (h * (a.Dn + a.Dv) + a.Dn) * a.C;
  for (int64_t e = tid; e < a.Dv; e += kThreads) {
    float acc = 0.f;
    for (int64_t c = 0; c < a.C; ++c) acc = fmaf(so[c], Elem<T>::load(wuv, e * a.C + c), acc);
    Elem<T>::store(static_cast<T *>(a.out), row * a.out_rs + e, acc);
  }
}

// One block per (token, 256 output features): RMSNorm of the token's latent, then the
// projection; feature j of head h = j / (Dn+Dv) goes to k_nope or v by its offset in the head, in
// the token's output row (b * out_seq_stride + out_row0 + s for token t = b * S_in + s).  With a
// rope cache, the blocks of the first feature range also copy the token's rope key row.
template <typename T>
__global__ void __launch_bounds__(kThreads)
plain_expand_kernel(const T *__restrict__ c_kv, const T *__restrict__ rms_w, const T *__restrict__ wkv_b,
                    T *__restrict__ k_nope, T *__restrict__ v, ExpandCall e) {
  extern __shared__ float sm[];
  float *sn = sm;           // C
  float *red = sn + e.C;    // 16
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t orow = (t / e.S_in) * e.out_seq_stride + e.out_row0 + t % e.S_in;
  if (e.pe_out && blockIdx.y == 0)
    for (int64_t r = tid; r < e.R; r += kThreads)
      static_cast<T *>(e.pe_out)[orow * e.R + r] = static_cast<const T *>(e.k_pe)[t * e.R + r];
  float ss = 0.f;
  for (int64_t c = tid; c < e.C; c += kThreads) {
    const float x = Elem<T>::load(c_kv, t * e.C + c);
    sn[c] = x;
    ss = fmaf(x, x, ss);
  }
  ss = block_sum(ss, red);
  const float inv = 1.f / sqrtf(ss / float(e.C) + e.eps);
  for (int64_t c = tid; c < e.C; c += kThreads) sn[c] = sn[c] * inv * Elem<T>::load(rms_w, c);
  __syncthreads();
  const int64_t per_head = e.Dn + e.Dv;
  const int64_t j = int64_t(blockIdx.y) * kThreads + tid;
  if (j >= e.H * per_head) return;
  float acc = 0.f;
  for (int64_t c = 0; c < e.C; ++c) acc = fmaf(sn[c], Elem<T>::load(wkv_b, j * e.C + c), acc);
  const int64_t h = j / per_head, jj = j % per_head;
  if (jj < e.Dn) Elem<T>::store(k_nope, (h * e.out_rows + orow) * e.Dn + jj, acc);
  else Elem<T>::store(v, (h * e.out_rows + orow) * e.Dv + (jj - e.Dn), acc);
}

template <typename T>
hipError_t run_attn(const AttnCall &a) {
  const int64_t rows = a.B * a.S * a.H;
  float *q_lat = static_cast<float *>(a.ws);
  float *part_ml = q_lat + rows * a.C;
  float *part_o = part_ml + 2 * rows * a.splits;
  const T *q_nope = static_cast<const T *>(a.q_nope);
  timing_begin(MLA_KERNEL_PLAIN, a.stream);
  plain_absorb_q_kernel<T><<<dim3(unsigned(rows), unsigned((a.C + kThreads - 1) / kThreads)), kThreads, 0,
                             a.stream>>>(q_nope, static_cast<const T *>(a.wkv_b), q_lat, a.H, a.C, a.Dn, a.Dv,
                                         a.q_nope_rs);
  const size_t sm_attn = sizeof(float) * size_t(2 * a.C + a.R + kThreads + 16) + 2 * sizeof(int64_t) * kThreads;
  plain_attn_partial_kernel<T><<<dim3(unsigned(rows), unsigned(a.splits)), kThreads, sm_attn, a.stream>>>(
      q_lat, static_cast<const T *>(a.q_pe), static_cast<const T *>(a.kv), static_cast<const T *>(a.pe),
      part_ml, part_o, a);
  plain_merge_upproj_kernel<T><<<dim3(unsigned(rows)), kThreads, sizeof(float) * size_t(a.C), a.stream>>>(
      part_ml, part_o, static_cast<const T *>(a.wkv_b), static_cast<T *>(a.out), a);
  timing_end(MLA_KERNEL_PLAIN, a.stream);
  return hipGetLastError();
}

template <typename T>
hipError_t run_expand(const ExpandCall &e) {
  const int64_t feats = e.H * (e.Dn + e.Dv);
  timing_begin(MLA_KERNEL_PLAIN, e.stream);
  plain_expand_kernel<T><<<dim3(unsigned(e.T), unsigned((feats + kThreads - 1) / kThreads)), kThreads,
                           sizeof(float) * size_t(e.C + 16), e.stream>>>(
      static_cast<const T *>(e.c_kv), static_cast<const T *>(e.rms_w), static_cast<const T *>(e.wkv_b),
      static_cast<T *>(e.k_nope), static_cast<T *>(e.v), e);
  timing_end(MLA_KERNEL_PLAIN, e.stream);
  return hipGetLastError();
}

// Naive-route attention over expanded keys and values, one block per query row (b, s, h):
// score over the visible positions in chunks of kThreads (online softmax), then the value sum.
template <typename T>
__global__ void __launch_bounds__(kThreads)
plain_naive_attn_kernel(const T *__restrict__ q_nope, const T *__restrict__ q_pe, const T *__restrict__ k_nope,
                        const T *__restrict__ v, const T *__restrict__ pe, T *__restrict__ out, NaiveCall a) {
  extern __shared__ float sm[];
  float *sq = sm;              // Dn + R   query
  float *so = sq + a.Dn + a.R; // Dv       running weighted sum
  float *sp = so + a.Dv;       // kThreads probabilities of the current chunk
  float *red = sp + kThreads;  // 16
  const int64_t row = blockIdx.x;  // (b, s, h)
  const int tid = threadIdx.x;
  const int64_t b = row / (a.S * a.H), s = (row / a.H) % a.S, h = row % a.H;
  const int64_t t1 = a.end_pos - a.S + s + 1;  // visible positions [0, t1)
  for (int64_t d = tid; d < a.Dn; d += kThreads) sq[d] = Elem<T>::load(q_nope, row * a.Dn + d);
  for (int64_t r = tid; r < a.R; r += kThreads) sq[a.Dn + r] = Elem<T>::load(q_pe, row * a.R + r);
  for (int64_t c = tid; c < a.Dv; c += kThreads) so[c] = 0.f;
  __syncthreads();
  const T *kb = k_nope + (h * a.Bmax + b) * a.Tmax * a.Dn;
  const T *vb = v + (h * a.Bmax + b) * a.Tmax * a.Dv;
  const T *pb = pe + b * a.Tmax * a.R;
  float m = -INFINITY, l = 0.f;
  for (int64_t tc = 0; tc < t1; tc += kThreads) {
    const int n = int((t1 - tc) < kThreads ? (t1 - tc) : kThreads);
    float sc = -INFINITY;
    if (tid < n) {
      const int64_t t = tc + tid;
      float acc = 0.f;
      for (int64_t d = 0; d < a.Dn; ++d) acc = fmaf(sq[d], Elem<T>::load(kb, t * a.Dn + d), acc);
      for (int64_t r = 0; r < a.R; ++r) acc = fmaf(sq[a.Dn + r], Elem<T>::load(pb, t * a.R + r), acc);
      sc = acc * a.scale;
    }
    const float m_new = fmaxf(m, block_max(sc, red));
    const float p = (tid < n) ? expf(sc - m_new) : 0.f;
    sp[tid] = p;
    const float alpha = (m == -INFINITY) ? 0.f : expf(m - m_new);
    l = l * alpha + block_sum(p, red);  // block_sum synchronises, so sp is visible below
    for (int64_t c = tid; c < a.Dv; c += kThreads) {
      float acc = so[c] * alpha;
      for (int j = 0; j < n; ++j) acc = fmaf(sp[j], Elem<T>::load(vb, (tc + j) * a.Dv + c), acc);
      so[c] = acc;
    }
    m = m_new;
    __syncthreads();
  }
  for (int64_t c = tid; c < a.Dv; c += kThreads) Elem<T>::store(out, row * a.Dv + c, so[c] / l);
}

template <typename T>
hipError_t run_naive(const NaiveCall &c) {
  const size_t lds = sizeof(float) * size_t(c.Dn + c.R + c.Dv + kThreads + 16);
  return launch_kernel(MLA_KERNEL_PLAIN, plain_naive_attn_kernel<T>, dim3(unsigned(c.B * c.S * c.H)),
                       dim3(kThreads), uint32_t(lds), c.stream, static_cast<const T *>(c.q_nope),
                       static_cast<const T *>(c.q_pe), static_cast<const T *>(c.k_nope), static_cast<const T *>(c.v),
                       static_cast<const T *>(c.pe), static_cast<T *>(c.out), c);
}

}  // namespace

int32_t plain_attn_splits(const AttnCall &c) {
  // Enough blocks to spread over the chip, but never fewer than 256 positions (or list entries)
  // per split.
  const int64_t rows = c.B * c.S * c.H;
  int64_t splits = (2048 + rows - 1) / rows;
  const int64_t max_by_len = ((c.topk > 0 ? c.topk : c.end_pos) + 255) / 256;
  if (splits > max_by_len) splits = max_by_len;
  if (splits < 1) splits = 1;
  return int32_t(splits);
}

size_t plain_attn_workspace(const AttnCall &c) {
  const size_t rows = size_t(c.B * c.S * c.H);
  return sizeof(float) * (rows * size_t(c.C) + rows * size_t(c.splits) * (2 + size_t(c.C)));
}

hipError_t plain_absorb_attn(const AttnCall &c) {
  return c.dtype == MLA_DTYPE_F32 ? run_attn<float>(c) : run_attn<uint16_t>(c);
}

hipError_t plain_expand_kv(const ExpandCall &e) {
  return e.dtype == MLA_DTYPE_F32 ? run_expand<float>(e) : run_expand<uint16_t>(e);
}

hipError_t plain_naive_attn(const NaiveCall &c) {
  return c.dtype == MLA_DTYPE_F32 ? run_naive<float>(c) : run_naive<uint16_t>(c);
}

}  // namespace mla
