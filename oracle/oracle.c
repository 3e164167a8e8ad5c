/*
 * Oracle for RelayAttention decode-time attention: plain, slow, fp64, CPU only.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark load this library.  The product path never calls it, and it
 * shares no code, header or table with the HIP library.
 *
 * What it computes (every value in fp64, inputs read as their exact fp32 / bf16
 * values):
 *
 *   For request b, query token t < n_b and query head h, with KV head
 *   h_kv = floor(h / g) (g = H_q / H_kv, consecutive grouping), the visible key
 *   sequence is the concatenation [system keys 0..L_s-1 ; context keys 0..p],
 *   p = c_b - n_b + t.  The system prompt precedes every request, so no system key
 *   is masked; the context part is causal.  (RelayAttention paper abstract: the
 *   method computes causal attention exactly; atyun.com article, section
 *   "RelayAttention": context positions follow the system prompt.)
 *
 *     s_j = scale * sum_c q[c] k_j[c]
 *     m   = max_j s_j,   Z = sum_j exp(s_j - m)
 *     out = sum_j exp(s_j - m) v_j / Z,   LSE = m + ln Z     (natural log)
 *
 *   oracle_attention_range() restricts j to a sub-range of that concatenated
 *   sequence.  The system part (the intermediate output of the system-attention
 *   step: attention over the system keys alone) is the range [0, L_s); the
 *   context part (attention over the request's own visible context alone) is
 *   [L_s, L_s + p + 1).  An empty range gives out = 0, LSE = -inf.
 *
 *   oracle_relay_fuse() is the relay-fusion step: the final output is a weighted
 *   average of the two intermediate outputs, with non-negative weights summing to
 *   one (atyun.com article, section "RelayAttention").  The pages fix nothing more
 *   about the weights; those used are alpha_s = e^LSE_s / (e^LSE_s + e^LSE_c),
 *   alpha_c = 1 - alpha_s, the only such weights for which the result equals
 *   exact attention.
 *   oracle_merge() is the same identity over k partial results.
 *
 * Sums over keys use Neumaier compensation so that the split-equals-unsplit
 * check holds to 1e-12 at 67k keys.
 *
 * Storage layouts (the C ABI's):
 *   q            [T_q, H_q, d]
 *   sys_k        [H_kv, ceil(L_s/16), d/G, 16, G]   (16-key tiles, chunk-major)
 *   sys_v        [H_kv, ceil(L_s/16), d, 16]   (16-key tiles, dim-major)
 *   ctx_k        [num_blocks, H_kv, d/G, 16, G]   (chunk-major within a page)
 *                G = elements per 16-byte chunk (8 bf16, 4 fp32; d when smaller): a key tile holds
 *                chunk 0 of its 16 keys, then chunk 1, ...; inside a chunk the keys are in
 *                slot order 0,1,2,3,8,9,10,11,4,5,6,7,12,13,14,15
 *   ctx_v        [num_blocks, H_kv, d, 16]     (dim-major within a page)
 *   block_tables [B, max_blocks]  context key j of request b lives in page
 *                block_tables[b][j/16], slot j%16
 *   ctx_lens [B], cu_q_lens [B+1] (token t of the flat batch belongs to request b
 *   with cu_q_lens[b] <= t < cu_q_lens[b+1])
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_BLOCK 16
#define ORACLE_SYS_TILE 16

typedef struct {
  int32_t dtype;
  int32_t batch, num_q_heads, num_kv_heads, head_dim;
  int32_t max_blocks_per_seq, sys_len;
  double scale;
  const void* q;
  const void* sys_k;
  const void* sys_v;
  const void* ctx_k;
  const void* ctx_v;
  const int32_t* block_tables;
  const int32_t* ctx_lens;
  const int32_t* cu_q_lens;
} oracle_problem;

/* The exact value of a stored element. */
static double elem(const void* base, size_t idx, int dtype) {
  if (dtype == ORACLE_BF16) {
    uint32_t u = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
  }
  return (double)((const float*)base)[idx];
}

/* Neumaier compensated accumulator. */
typedef struct { double s, c; } acc_t;
static void acc_add(acc_t* a, double x) {
  double t = a->s + x;
  if (fabs(a->s) >= fabs(x)) a->c += (a->s - t) + x;
  else a->c += (x - t) + a->s;
  a->s = t;
}
static double acc_val(const acc_t* a) { return a->s + a->c; }

/* Request that owns flat query token t. */
static int request_of(const oracle_problem* p, int t) {
  int b = 0;
  while (b + 1 < p->batch && p->cu_q_lens[b + 1] <= t) ++b;
  return b;
}

/* Index of element c of key r (0..15) inside one 16-key tile of keys (g elements per
 * 16-byte chunk; the whole row when d is smaller).  Inside a chunk the keys sit in
 * slot order: the key order with keys 4..7 and 8..11 exchanged. */
static size_t key_in_tile(int r, int c, int dtype, int d) {
  int g = dtype == ORACLE_BF16 ? 8 : 4;
  if (g > d) g = d;
  int slot = (r >= 4 && r < 8) ? r + 4 : (r >= 8 && r < 12) ? r - 4 : r;
  return ((size_t)(c / g) * ORACLE_BLOCK + slot) * g + c % g;
}

/* Element c of key j of the concatenated sequence for (request b, kv head hk). */
static double key_elem(const oracle_problem* p, int b, int hk, int j, int c) {
  int d = p->head_dim, Ls = p->sys_len;
  if (j < Ls) {
    size_t ntile = (size_t)(Ls + ORACLE_SYS_TILE - 1) / ORACLE_SYS_TILE;
    return elem(p->sys_k,
                ((size_t)hk * ntile + j / ORACLE_SYS_TILE) * ORACLE_SYS_TILE * d +
                    key_in_tile(j % ORACLE_SYS_TILE, c, p->dtype, d),
                p->dtype);
  }
  j -= Ls;
  int blk = p->block_tables[(size_t)b * p->max_blocks_per_seq + j / ORACLE_BLOCK];
  return elem(p->ctx_k,
              ((size_t)blk * p->num_kv_heads + hk) * ORACLE_BLOCK * d +
                  key_in_tile(j % ORACLE_BLOCK, c, p->dtype, d),
              p->dtype);
}

static double val_elem(const oracle_problem* p, int b, int hk, int j, int c) {
  int d = p->head_dim, Ls = p->sys_len;
  if (j < Ls) {
    size_t ntile = (size_t)(Ls + ORACLE_SYS_TILE - 1) / ORACLE_SYS_TILE;
    return elem(p->sys_v,
                (((size_t)hk * ntile + j / ORACLE_SYS_TILE) * d + c) * ORACLE_SYS_TILE +
                    j % ORACLE_SYS_TILE,
                p->dtype);
  }
  j -= Ls;
  int blk = p->block_tables[(size_t)b * p->max_blocks_per_seq + j / ORACLE_BLOCK];
  return elem(p->ctx_v,
              (((size_t)blk * p->num_kv_heads + hk) * d + c) * ORACLE_BLOCK + j % ORACLE_BLOCK,
              p->dtype);
}

/*
 * Attention of one query row over keys [lo, hi) of its visible concatenated
 * sequence [0, L_s + p + 1).  lo/hi are clipped to that range.
 * scores: scratch of at least L_s + max context length doubles.
 */
static void attend_row(const oracle_problem* p, int t, int h, long lo, long hi,
                       double* scores, double* out, double* lse) {
  int d = p->head_dim;
  int g = p->num_q_heads / p->num_kv_heads;
  int hk = h / g;
  int b = request_of(p, t);
  int n_b = p->cu_q_lens[b + 1] - p->cu_q_lens[b];
  int pos = p->ctx_lens[b] - n_b + (t - p->cu_q_lens[b]);
  long visible = (long)p->sys_len + pos + 1;
  if (lo < 0) lo = 0;
  if (hi > visible) hi = visible;
  for (int c = 0; c < d; ++c) out[c] = 0.0;
  if (hi <= lo) {
    *lse = -INFINITY;
    return;
  }
  size_t qoff = ((size_t)t * p->num_q_heads + h) * d;
  double m = -INFINITY;
  for (long j = lo; j < hi; ++j) {
    double s = 0.0;
    for (int c = 0; c < d; ++c) s += elem(p->q, qoff + c, p->dtype) * key_elem(p, b, hk, (int)j, c);
    s *= p->scale;
    scores[j - lo] = s;
    if (s > m) m = s;
  }
  acc_t z = {0.0, 0.0};
  for (long j = lo; j < hi; ++j) {
    scores[j - lo] = exp(scores[j - lo] - m);
    acc_add(&z, scores[j - lo]);
  }
  double zv = acc_val(&z);
  for (int c = 0; c < d; ++c) {
    acc_t o = {0.0, 0.0};
    for (long j = lo; j < hi; ++j) acc_add(&o, scores[j - lo] * val_elem(p, b, hk, (int)j, c));
    out[c] = acc_val(&o) / zv;
  }
  *lse = m + log(zv);
}

static long max_visible(const oracle_problem* p) {
  long mx = 0;
  for (int b = 0; b < p->batch; ++b)
    if (p->ctx_lens[b] > mx) mx = p->ctx_lens[b];
  return (long)p->sys_len + mx + 1;
}

/*
 * Shared driver.  mode 0: [lo, hi) given as absolute indices of the concatenated
 * sequence; mode 1: system part; mode 2: context part; mode 3: whole sequence.
 * rows: flat row ids r = t * H_q + h to compute (n_rows of them), or NULL for all
 * T_q * H_q rows in order.  out: [n_rows, d], lse: [n_rows].
 */
static int run(const oracle_problem* p, int mode, long lo, long hi, const int64_t* rows,
               long n_rows, double* out, double* lse) {
  if (!p || p->num_kv_heads <= 0 || p->num_q_heads % p->num_kv_heads) return -1;
  long total_rows = (long)p->cu_q_lens[p->batch] * p->num_q_heads;
  if (!rows) n_rows = total_rows;
  long scratch = max_visible(p);
  int err = 0;
#pragma omp parallel
  {
    double* scores = (double*)malloc(sizeof(double) * (size_t)scratch);
    if (!scores) {
#pragma omp atomic write
      err = -2;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (long i = 0; i < n_rows; ++i) {
        long r = rows ? (long)rows[i] : i;
        int t = (int)(r / p->num_q_heads), h = (int)(r % p->num_q_heads);
        long a = lo, e = hi;
        if (mode == 1) { a = 0; e = p->sys_len; }
        else if (mode == 2) { a = p->sys_len; e = 1L << 40; }
        else if (mode == 3) { a = 0; e = 1L << 40; }
        attend_row(p, t, h, a, e, scores, out + (size_t)i * p->head_dim, lse + i);
      }
      free(scores);
    }
  }
  return err;
}

/* Exact causal attention over [system; context] (what RelayAttention must equal). */
int oracle_attention(const oracle_problem* p, const int64_t* rows, long n_rows, double* out,
                     double* lse) {
  return run(p, 3, 0, 0, rows, n_rows, out, lse);
}

/* System-attention step: attention over the system keys only. */
int oracle_system_part(const oracle_problem* p, const int64_t* rows, long n_rows, double* out,
                       double* lse) {
  return run(p, 1, 0, 0, rows, n_rows, out, lse);
}

/* Context-attention step: attention over the request's own visible context only. */
int oracle_context_part(const oracle_problem* p, const int64_t* rows, long n_rows, double* out,
                        double* lse) {
  return run(p, 2, 0, 0, rows, n_rows, out, lse);
}

/* Attention restricted to keys [lo, hi) of the concatenated visible sequence. */
int oracle_attention_range(const oracle_problem* p, long lo, long hi, const int64_t* rows,
                           long n_rows, double* out, double* lse) {
  return run(p, 0, lo, hi, rows, n_rows, out, lse);
}

/*
 * Relay fusion: out = alpha_s * o_s + alpha_c * o_c, alpha_s + alpha_c = 1,
 * alpha_s = e^lse_s / (e^lse_s + e^lse_c).  A part with LSE = -inf has weight 0.
 * alpha (optional, [n_rows, 2]) receives the weights.  lse_out (optional) receives
 * ln(e^lse_s + e^lse_c).
 */
void oracle_relay_fuse(long n_rows, int d, const double* o_s, const double* lse_s,
                       const double* o_c, const double* lse_c, double* out, double* lse_out,
                       double* alpha) {
  for (long r = 0; r < n_rows; ++r) {
    double ls = lse_s[r], lc = lse_c[r];
    double as, ac, l;
    if (isinf(ls) && ls < 0 && isinf(lc) && lc < 0) {
      as = ac = 0.0;
      l = -INFINITY;
    } else if (ls >= lc) {
      double e = exp(lc - ls);
      as = 1.0 / (1.0 + e);
      ac = e / (1.0 + e);
      l = ls + log1p(e);
    } else {
      double e = exp(ls - lc);
      ac = 1.0 / (1.0 + e);
      as = e / (1.0 + e);
      l = lc + log1p(e);
    }
    for (int c = 0; c < d; ++c) out[r * d + c] = as * o_s[r * d + c] + ac * o_c[r * d + c];
    if (lse_out) lse_out[r] = l;
    if (alpha) {
      alpha[2 * r] = as;
      alpha[2 * r + 1] = ac;
    }
  }
}

/*
 * k-way merge of partial results over disjoint key sets:
 * out = sum_i e^(lse_i - L) o_i, L = ln sum_i e^lse_i.
 * o: [k, n_rows, d], lse: [k, n_rows].
 */
void oracle_merge(int k, long n_rows, int d, const double* o, const double* lse, double* out,
                  double* lse_out) {
  for (long r = 0; r < n_rows; ++r) {
    double m = -INFINITY;
    for (int i = 0; i < k; ++i)
      if (lse[(size_t)i * n_rows + r] > m) m = lse[(size_t)i * n_rows + r];
    for (int c = 0; c < d; ++c) out[r * d + c] = 0.0;
    if (isinf(m) && m < 0) {
      if (lse_out) lse_out[r] = -INFINITY;
      continue;
    }
    acc_t z = {0.0, 0.0};
    for (int i = 0; i < k; ++i) acc_add(&z, exp(lse[(size_t)i * n_rows + r] - m));
    double zv = acc_val(&z);
    for (int c = 0; c < d; ++c) {
      acc_t a = {0.0, 0.0};
      for (int i = 0; i < k; ++i)
        acc_add(&a, exp(lse[(size_t)i * n_rows + r] - m) * o[((size_t)i * n_rows + r) * d + c]);
      out[r * d + c] = acc_val(&a) / zv;
    }
    if (lse_out) lse_out[r] = m + log(zv);
  }
}

/* Threads of the following calls (a timing knob: the arithmetic is the same at any count). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int oracle_num_threads(void) {
  int n = 1;
#ifdef _OPENMP
#pragma omp parallel
  {
#pragma omp single
    n = omp_get_num_threads();
  }
#endif
  return n;
}
