/*
 * ea_oracle.c -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.
 *
 * A plain, slow, obviously correct fp64 CPU reference for the routed hybrid-attention
 * prefill of Elastic Attention.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code, header or table with the
 * HIP library; the two meet only through the seeded input bytes the tests hand to both.
 *
 * Sources (web pages on Elastic Attention, "Elastic Attention: Test-time Adaptive
 * Sparsity Ratios for Efficient Transformers", arXiv:2601.17367):
 *   [Blog]  author-style blog post "Elastic Attention：将 MoE 路由引入 Attention ...",
 *           section 1 (hybrid heads: some heads see everything, others only a local or
 *           sliding window), section 2.1 "Attention Router" (the router reads the current
 *           key hidden states, an MLP emits one signal r per head, r=0 runs Full
 *           Attention, r=1 runs Sparse Attention, the per-mode results are concatenated),
 *           section 3 "Fused Kernel" (routing is handed to one kernel as metadata).
 *   [Expl]  gist.science lay explanation of the same paper, section "问题所在"
 *           (sparse reading looks only at the first and the last page of each book).
 *
 * Readings taken where the pages are silent (each one is listed in the design notes):
 *   - sparse head = attention sink (first `sink` keys of the sequence) united with a
 *     causal sliding window of `window` keys ending at the query (diagonal included);
 *   - both modes are causal; keys never cross sequence boundaries of a packed batch;
 *   - GQA: query head h reads KV head floor(h / (Hq/Hkv));
 *   - router input = mean over the sequence's tokens of the key states; MLP
 *     z = W2 SiLU(W1 x + b1) + b2; r = (z > 0), so z == 0 routes to full attention;
 *     an empty sequence pools to the zero vector;
 *   - work item cost = number of BN-wide key tiles that hold at least one visible
 *     (query, key) pair for the BM query rows of the item; order = cost descending,
 *     ties by (sequence, q-tile, head) ascending.
 *
 * Every floating-point step is done in double precision on the exact input values
 * (bf16 and fp32 inputs convert to double without rounding).
 *
 * Parity pins: every function here is checked in the CPU test suite against brute
 * force on tiny inputs, closed forms, identities and library routines.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_BF16 = 0, OR_F32 = 1, OR_F64 = 2 };

/* Exact widening of one stored element to double. */
static double elem(const void* base, int dtype, int64_t idx) {
  if (dtype == OR_BF16) {
    uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
  }
  if (dtype == OR_F32) return (double)((const float*)base)[idx];
  return ((const double*)base)[idx];
}

/* Is key j visible to query i (both positions inside one sequence)?
 * [Blog §2.1]: r = 0 -> full attention, r = 1 -> sparse attention.
 * [Blog §1] / [Expl "问题所在"]: sparse heads look at the start and a local window. */
static int key_visible(int64_t i, int64_t j, int sparse, int64_t sink, int64_t window) {
  if (j > i) return 0;            /* causal in both modes */
  if (!sparse) return 1;          /* full head: every earlier key and itself */
  return (j < sink) || (j > i - window);
}

static int seq_of_token(const int32_t* cu, int batch, int64_t t) {
  for (int b = 0; b < batch; ++b)
    if (t >= cu[b] && t < cu[b + 1]) return b;
  return -1;
}

/*
 * Masked-softmax attention, one (row, head) at a time, straight from the definition:
 *   x_j = scale * <q_i, k_j> for visible j,  m = max_j x_j,
 *   p_j = exp(x_j - m) / sum_j exp(x_j - m),  o_i = sum_j p_j v_j,  lse_i = m + log(sum).
 * Layouts (token-major, packed by cu_seqlens): q/o [T, hq, d], k/v [T, hkv, d].
 * cu_k (nullable): a separate packing of k/v [Tk, hkv, d] for a chunked prefill over a KV
 * prefix.  Sequence b then has Lk = cu_k[b+1] - cu_k[b] keys and Lq = cu_seqlens[b+1] -
 * cu_seqlens[b] <= Lk queries, the last Lq positions: query row r of the chunk sits at
 * position i = Lk - Lq + r.  NULL: cu_k = cu_seqlens (a plain prefill, i = r).
 * rows: packed token indices to evaluate (NULL = every token 0..T-1, n_rows = T).
 * o_out [n_rows, hq, d] and lse_out [n_rows, hq] (nullable) are doubles.
 * Returns 0, or -1 on bad arguments.
 */
int oracle_attn(const void* q, const void* k, const void* v, int dtype,
                const int32_t* cu_seqlens, const int32_t* cu_k, int batch, int hq, int hkv, int d,
                const uint8_t* route, int sink, int window, double scale,
                const int64_t* rows, int64_t n_rows,
                double* o_out, double* lse_out, int nthreads) {
  if (batch < 1 || hq < 1 || hkv < 1 || hq % hkv != 0 || d < 1 || window < 1 || sink < 0)
    return -1;
  const int group = hq / hkv;
  if (cu_k == NULL) cu_k = cu_seqlens;
  int64_t max_len = 0;
  for (int b = 0; b < batch; ++b) {
    const int64_t len = (int64_t)cu_seqlens[b + 1] - cu_seqlens[b];
    const int64_t len_k = (int64_t)cu_k[b + 1] - cu_k[b];
    if (len < 0 || len_k < len) return -1;
    if (len_k > max_len) max_len = len_k;
  }
  const int64_t total = cu_seqlens[batch];
  if (rows == NULL) n_rows = total;
  for (int64_t r = 0; rows != NULL && r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= total) return -1;
  const int64_t n_tasks = n_rows * hq;
  int bad = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel reduction(| : bad)
  {
    double* x = (double*)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
    double* acc = (double*)malloc(sizeof(double) * (size_t)d);
    if (!x || !acc) bad = 1;
#pragma omp for schedule(dynamic, 16)
    for (int64_t task = 0; task < n_tasks; ++task) {
      if (!x || !acc) continue;
      const int64_t r = task / hq;
      const int h = (int)(task % hq);
      const int64_t t = rows ? rows[r] : r;
      const int b = seq_of_token(cu_seqlens, batch, t);
      const int64_t start = cu_k[b];             /* the sequence's first key */
      /* position of the query: the chunk holds the last Lq of the sequence's Lk positions */
      const int64_t i = (int64_t)(cu_k[b + 1] - cu_k[b]) - (cu_seqlens[b + 1] - cu_seqlens[b]) +
                        (t - cu_seqlens[b]);
      const int g = h / group;                   /* KV head read by query head h */
      const int sparse = route[(int64_t)b * hq + h] != 0;

      double m = -INFINITY;
      for (int64_t j = 0; j <= i; ++j) {
        if (!key_visible(i, j, sparse, sink, window)) continue;
        double dot = 0.0;
        for (int e = 0; e < d; ++e)
          dot += elem(q, dtype, (t * hq + h) * (int64_t)d + e) *
                 elem(k, dtype, ((start + j) * hkv + g) * (int64_t)d + e);
        x[j] = scale * dot;
        if (x[j] > m) m = x[j];
      }
      double sum = 0.0;
      for (int e = 0; e < d; ++e) acc[e] = 0.0;
      for (int64_t j = 0; j <= i; ++j) {
        if (!key_visible(i, j, sparse, sink, window)) continue;
        const double p = exp(x[j] - m);
        sum += p;
        for (int e = 0; e < d; ++e)
          acc[e] += p * elem(v, dtype, ((start + j) * hkv + g) * (int64_t)d + e);
      }
      for (int e = 0; e < d; ++e) o_out[(r * hq + h) * (int64_t)d + e] = acc[e] / sum;
      if (lse_out) lse_out[r * hq + h] = m + log(sum);
    }
    free(x);
    free(acc);
  }
  return bad ? -2 : 0;
}

/*
 * One decode step of the same routed attention: sequence b holds seqlens[b] tokens in its
 * cache (the newest one, at position i = seqlens[b] - 1, is the query's own token), and
 * each query head attends from position i under its mode exactly as a prefill row at
 * position i would [Blog §2.1 modes; the sparse pattern as above].  Layouts: q/o
 * [batch, hq, d]; k_cache/v_cache [batch, cap, hkv, d]; seqlens [batch] with
 * 1 <= seqlens[b] <= cap.  lse_out [batch, hq] (nullable).
 */
int oracle_decode(const void* q, const void* kc, const void* vc, int dtype,
                  const int32_t* seqlens, int batch, int cap, int hq, int hkv, int d,
                  const uint8_t* route, int sink, int window, double scale,
                  double* o_out, double* lse_out, int nthreads) {
  if (batch < 1 || cap < 1 || hq < 1 || hkv < 1 || hq % hkv != 0 || d < 1 || window < 1 ||
      sink < 0)
    return -1;
  for (int b = 0; b < batch; ++b)
    if (seqlens[b] < 1 || seqlens[b] > cap) return -1;
  const int group = hq / hkv;
  const int64_t n_tasks = (int64_t)batch * hq;
  int bad = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel reduction(| : bad)
  {
    double* x = (double*)malloc(sizeof(double) * (size_t)cap);
    double* acc = (double*)malloc(sizeof(double) * (size_t)d);
    if (!x || !acc) bad = 1;
#pragma omp for schedule(dynamic, 1)
    for (int64_t task = 0; task < n_tasks; ++task) {
      if (!x || !acc) continue;
      const int b = (int)(task / hq);
      const int h = (int)(task % hq);
      const int g = h / group;
      const int64_t i = seqlens[b] - 1;
      const int sparse = route[task] != 0;
      double m = -INFINITY;
      for (int64_t j = 0; j <= i; ++j) {
        if (!key_visible(i, j, sparse, sink, window)) continue;
        double dot = 0.0;
        for (int e = 0; e < d; ++e)
          dot += elem(q, dtype, task * d + e) *
                 elem(kc, dtype, (((int64_t)b * cap + j) * hkv + g) * d + e);
        x[j] = scale * dot;
        if (x[j] > m) m = x[j];
      }
      double sum = 0.0;
      for (int e = 0; e < d; ++e) acc[e] = 0.0;
      for (int64_t j = 0; j <= i; ++j) {
        if (!key_visible(i, j, sparse, sink, window)) continue;
        const double p = exp(x[j] - m);
        sum += p;
        for (int e = 0; e < d; ++e)
          acc[e] += p * elem(vc, dtype, (((int64_t)b * cap + j) * hkv + g) * d + e);
      }
      for (int e = 0; e < d; ++e) o_out[task * d + e] = acc[e] / sum;
      if (lse_out) lse_out[task] = m + log(sum);
    }
    free(x);
    free(acc);
  }
  return bad ? -2 : 0;
}

/*
 * Attention Router [Blog §2.1]: reads the key hidden states of each sequence and emits
 * one routing signal per query head.  x = mean over the sequence's tokens of
 * ks[t, :] (an empty sequence gives x = 0); u = W1 x + b1; h = u * sigmoid(u) (SiLU);
 * z = W2 h + b2; r = (z > 0).
 * ks [T, kv_dim] (dtype), w1 [hidden, kv_dim], b1 [hidden], w2 [n_heads, hidden],
 * b2 [n_heads] (fp32).  pooled_out [batch, kv_dim] (nullable), logits_out
 * [batch, n_heads], route_out [batch, n_heads].
 */
int oracle_route(const void* ks, int dtype, int kv_dim, const int32_t* cu_seqlens, int batch,
                 const float* w1, const float* b1, int hidden,
                 const float* w2, const float* b2, int n_heads,
                 double* pooled_out, double* logits_out, uint8_t* route_out) {
  if (batch < 1 || kv_dim < 1 || hidden < 1 || n_heads < 1) return -1;
  double* x = (double*)malloc(sizeof(double) * (size_t)kv_dim);
  double* hvec = (double*)malloc(sizeof(double) * (size_t)hidden);
  if (!x || !hvec) { free(x); free(hvec); return -2; }
  for (int b = 0; b < batch; ++b) {
    const int64_t start = cu_seqlens[b], len = (int64_t)cu_seqlens[b + 1] - cu_seqlens[b];
    for (int c = 0; c < kv_dim; ++c) {
      double s = 0.0;
      for (int64_t t = 0; t < len; ++t) s += elem(ks, dtype, (start + t) * kv_dim + c);
      x[c] = len > 0 ? s / (double)len : 0.0;
      if (pooled_out) pooled_out[(int64_t)b * kv_dim + c] = x[c];
    }
    for (int j = 0; j < hidden; ++j) {
      double u = (double)b1[j];
      for (int c = 0; c < kv_dim; ++c) u += (double)w1[(int64_t)j * kv_dim + c] * x[c];
      hvec[j] = u / (1.0 + exp(-u));
    }
    for (int h = 0; h < n_heads; ++h) {
      double z = (double)b2[h];
      for (int j = 0; j < hidden; ++j) z += (double)w2[(int64_t)h * hidden + j] * hvec[j];
      logits_out[(int64_t)b * n_heads + h] = z;
      route_out[(int64_t)b * n_heads + h] = z > 0.0 ? 1 : 0;
    }
  }
  free(x);
  free(hvec);
  return 0;
}

/* Number of BN-wide key tiles holding at least one visible pair for query rows
 * [m0, m1) of one sequence.  Each row's visible keys form at most two intervals (sink
 * and window for a sparse head, [0, i] for a full head); an interval [lo, hi] of keys
 * overlaps exactly the tiles lo/bn .. hi/bn.  The union over rows is counted with a
 * coverage difference array: +1 at the first tile of every interval, -1 after its last. */
static int64_t touched_tiles(int64_t m0, int64_t m1, int sparse, int64_t sink, int64_t window,
                             int64_t bn, int64_t* cover, int64_t n_tiles) {
  for (int64_t tt = 0; tt <= n_tiles; ++tt) cover[tt] = 0;
  for (int64_t i = m0; i < m1; ++i) {
    int64_t lo[2], hi[2];
    int n = 0;
    if (!sparse) {
      lo[n] = 0; hi[n] = i; ++n;
    } else {
      const int64_t s_end = sink < i + 1 ? sink : i + 1;     /* sink keys: j < sink, j <= i */
      if (s_end > 0) { lo[n] = 0; hi[n] = s_end - 1; ++n; }
      const int64_t w_lo = i - window + 1;                    /* window keys: i-window < j <= i */
      lo[n] = w_lo > 0 ? w_lo : 0; hi[n] = i; ++n;
    }
    for (int a = 0; a < n; ++a) {
      cover[lo[a] / bn] += 1;
      cover[hi[a] / bn + 1] -= 1;
    }
  }
  int64_t count = 0, running = 0;
  for (int64_t tt = 0; tt < n_tiles; ++tt) {
    running += cover[tt];
    if (running > 0) ++count;
  }
  return count;
}

typedef struct { int32_t seq, head, q_tile, cost; } or_item;

/* Longest first; equal costs in (sequence, q-tile, head) ascending order. */
static int item_order(const void* pa, const void* pb) {
  const or_item* a = (const or_item*)pa;
  const or_item* b = (const or_item*)pb;
  if (a->cost != b->cost) return a->cost > b->cost ? -1 : 1;
  if (a->seq != b->seq) return a->seq < b->seq ? -1 : 1;
  if (a->q_tile != b->q_tile) return a->q_tile < b->q_tile ? -1 : 1;
  if (a->head != b->head) return a->head < b->head ? -1 : 1;
  return 0;
}

/*
 * Work list of the fused launch [Blog §3]: the routing bits reach the kernel as
 * metadata; here that metadata is one item per (sequence, query head, BM-row q-tile)
 * with its key-tile cost.  items_out [n, 4] int32 = {seq, head, q_tile, cost}, in the
 * order above.  *n_out receives the item count; items_out may be NULL to only count.
 * capacity bounds the number of items written.  cu_k (nullable) as for oracle_attn: the
 * q-tiles cover the chunk's Lq rows, whose positions start at Lk - Lq.
 */
int oracle_worklist(const uint8_t* route, const int32_t* cu_seqlens, const int32_t* cu_k,
                    int batch, int hq,
                    int sink, int window, int bm, int bn,
                    int32_t* items_out, int64_t capacity, int64_t* n_out) {
  if (batch < 1 || hq < 1 || bm < 1 || bn < 1 || window < 1 || sink < 0) return -1;
  if (cu_k == NULL) cu_k = cu_seqlens;
  int64_t n = 0, max_len = 0;
  for (int b = 0; b < batch; ++b) {
    const int64_t len = (int64_t)cu_seqlens[b + 1] - cu_seqlens[b];
    const int64_t len_k = (int64_t)cu_k[b + 1] - cu_k[b];
    if (len < 0 || len_k < len) return -1;
    n += (int64_t)hq * ((len + bm - 1) / bm);
    if (len_k > max_len) max_len = len_k;
  }
  *n_out = n;
  if (items_out == NULL) return 0;
  if (n > capacity) return -1;
  const int64_t n_tiles = (max_len + bn - 1) / bn;
  or_item* items = (or_item*)malloc(sizeof(or_item) * (size_t)(n > 0 ? n : 1));
  int64_t* cover = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_tiles + 2));
  if (!items || !cover) { free(items); free(cover); return -2; }
  int64_t at = 0;
  for (int b = 0; b < batch; ++b) {
    const int64_t len = (int64_t)cu_seqlens[b + 1] - cu_seqlens[b];
    const int64_t off = (int64_t)cu_k[b + 1] - cu_k[b] - len;  /* position of chunk row 0 */
    const int64_t n_q = (len + bm - 1) / bm;
    for (int h = 0; h < hq; ++h) {
      const int sparse = route[(int64_t)b * hq + h] != 0;
      for (int64_t qt = 0; qt < n_q; ++qt) {
        const int64_t m0 = qt * bm, m1 = (m0 + bm < len) ? m0 + bm : len;
        items[at].seq = b;
        items[at].head = h;
        items[at].q_tile = (int32_t)qt;
        items[at].cost =
            (int32_t)touched_tiles(off + m0, off + m1, sparse, sink, window, bn, cover, n_tiles);
        ++at;
      }
    }
  }
  qsort(items, (size_t)n, sizeof(or_item), item_order);
  for (int64_t a = 0; a < n; ++a) {
    items_out[4 * a + 0] = items[a].seq;
    items_out[4 * a + 1] = items[a].head;
    items_out[4 * a + 2] = items[a].q_tile;
    items_out[4 * a + 3] = items[a].cost;
  }
  free(items);
  free(cover);
  return 0;
}

/*
 * Backward of the routed attention (training of the method: [Blog §2.1] "training trick":
 * gradients must flow through the model; here the attention part of them), straight from
 * the chain rule of the definition above, per sequence b, query head h, row i:
 *   P_ij = exp(x_ij - m_i) / sum_j exp(x_ij - m_i) over visible j,  o_i = sum_j P_ij v_j,
 *   D_i = <dO_i, o_i>,  dP_ij = <dO_i, v_j>,  dS_ij = P_ij (dP_ij - D_i),
 *   dq_i = scale * sum_j dS_ij k_j,  dk_j += scale * dS_ij q_i,  dv_j += P_ij dO_i,
 * dk and dv summed over the query heads that read KV head g.  Same layouts and packing as
 * oracle_attn (cu_k: optional key packing); outputs are doubles: dq [Tq, hq, d],
 * dk / dv [Tk, hkv, d] (overwritten).  One task per (sequence, KV head), so dk and dv are
 * accumulated by one thread.  Returns 0, or -1 on bad arguments.
 */
int oracle_attn_backward(const void* q, const void* k, const void* v, const void* dout,
                         int dtype, const int32_t* cu_seqlens, const int32_t* cu_k, int batch,
                         int hq, int hkv, int d, const uint8_t* route, int sink, int window,
                         double scale, double* dq_out, double* dk_out, double* dv_out,
                         int nthreads) {
  if (batch < 1 || hq < 1 || hkv < 1 || hq % hkv != 0 || d < 1 || window < 1 || sink < 0)
    return -1;
  if (cu_k == NULL) cu_k = cu_seqlens;
  const int group = hq / hkv;
  int64_t max_len = 0;
  for (int b = 0; b < batch; ++b) {
    const int64_t len = (int64_t)cu_seqlens[b + 1] - cu_seqlens[b];
    const int64_t len_k = (int64_t)cu_k[b + 1] - cu_k[b];
    if (len < 0 || len_k < len) return -1;
    if (len_k > max_len) max_len = len_k;
  }
  memset(dq_out, 0, sizeof(double) * (size_t)cu_seqlens[batch] * hq * d);
  memset(dk_out, 0, sizeof(double) * (size_t)cu_k[batch] * hkv * d);
  memset(dv_out, 0, sizeof(double) * (size_t)cu_k[batch] * hkv * d);
  const int64_t n_tasks = (int64_t)batch * hkv;
  int bad = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel reduction(| : bad)
  {
    double* x = (double*)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
    double* o = (double*)malloc(sizeof(double) * (size_t)d);
    if (!x || !o) bad = 1;
#pragma omp for schedule(dynamic, 1)
    for (int64_t task = 0; task < n_tasks; ++task) {
      if (!x || !o) continue;
      const int b = (int)(task / hkv), g = (int)(task % hkv);
      const int64_t q0 = cu_seqlens[b], nq = cu_seqlens[b + 1] - q0;
      const int64_t k0 = cu_k[b], nk = cu_k[b + 1] - k0;
      for (int hh = 0; hh < group; ++hh) {
        const int h = g * group + hh;
        const int sparse = route[(int64_t)b * hq + h] != 0;
        for (int64_t r = 0; r < nq; ++r) {
          const int64_t t = q0 + r;
          const int64_t i = nk - nq + r;  /* position of the query */
          double m = -INFINITY;
          for (int64_t j = 0; j <= i; ++j) {
            if (!key_visible(i, j, sparse, sink, window)) continue;
            double dot = 0.0;
            for (int e = 0; e < d; ++e)
              dot += elem(q, dtype, (t * hq + h) * (int64_t)d + e) *
                     elem(k, dtype, ((k0 + j) * hkv + g) * (int64_t)d + e);
            x[j] = scale * dot;
            if (x[j] > m) m = x[j];
          }
          double sum = 0.0;
          for (int64_t j = 0; j <= i; ++j)
            if (key_visible(i, j, sparse, sink, window)) sum += exp(x[j] - m);
          /* P_ij stored back into x; o_i and D_i */
          for (int e = 0; e < d; ++e) o[e] = 0.0;
          for (int64_t j = 0; j <= i; ++j) {
            if (!key_visible(i, j, sparse, sink, window)) continue;
            x[j] = exp(x[j] - m) / sum;
            for (int e = 0; e < d; ++e)
              o[e] += x[j] * elem(v, dtype, ((k0 + j) * hkv + g) * (int64_t)d + e);
          }
          double Di = 0.0;
          for (int e = 0; e < d; ++e) Di += elem(dout, dtype, (t * hq + h) * (int64_t)d + e) * o[e];
          for (int64_t j = 0; j <= i; ++j) {
            if (!key_visible(i, j, sparse, sink, window)) continue;
            double dp = 0.0;
            for (int e = 0; e < d; ++e)
              dp += elem(dout, dtype, (t * hq + h) * (int64_t)d + e) *
                    elem(v, dtype, ((k0 + j) * hkv + g) * (int64_t)d + e);
            const double ds = x[j] * (dp - Di);
            for (int e = 0; e < d; ++e) {
              dq_out[(t * hq + h) * (int64_t)d + e] +=
                  scale * ds * elem(k, dtype, ((k0 + j) * hkv + g) * (int64_t)d + e);
              dk_out[((k0 + j) * hkv + g) * (int64_t)d + e] +=
                  scale * ds * elem(q, dtype, (t * hq + h) * (int64_t)d + e);
              dv_out[((k0 + j) * hkv + g) * (int64_t)d + e] +=
                  x[j] * elem(dout, dtype, (t * hq + h) * (int64_t)d + e);
            }
          }
        }
      }
    }
    free(x);
    free(o);
  }
  return bad ? -2 : 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
