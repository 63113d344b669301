/*
 * fp64 CPU oracle of the quantized Mixture-of-Experts FFN block.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load or call this library. The product path (the HIP
 * library) never links, loads or calls it, and shares no code with it.
 *
 * What it computes, for one MoE layer and each activation row x
 * (TurboFieldfare pages: the per-token flow "router -> pick 8 experts -> ...
 * -> merge" on the blog-mushroom article, "Why 26B fits"; 8 of 128 experts
 * per layer on the same page and on the ai-heartland review, introduction;
 * MLX affine 4-bit, group 64, BF16 scale and bias, 8-bit router on the
 * ai-heartland review, system-design summary, and the rebasdaily article,
 * "not shrinking the model"; the always-on shared expert merged with the
 * routed experts on the blog-mushroom article, "Why 26B fits"):
 *
 *   1. code of element i of row n: 4-bit -> nibble (i even: low, odd: high) of
 *      byte i/2; 8-bit -> byte i
 *   2. dequant  W[n,i] = s[n,i/64] * q[n,i] + b[n,i/64]   (s, b stored as bf16)
 *   3. router   l[e] = sum_i Wr[e,i] * x[i] + o[e]        (i ascending)
 *   4. top-k    experts ordered by (l desc, id asc); the first k are picked
 *   5. weights  p_j = exp(l_j - l_1) / sum_{t<k} exp(l_t - l_1)
 *   6. expert   E(x) = Wd (gelu_tanh(Wg x) * (Wu x))
 *   7. shared   S(x) = the same with the shared expert's matrices
 *   8. output   y = S(x) + sum_{j<k} p_j * E_{idx_j}(x)   (j in top-k order)
 *   9. grouping (row, slot) pairs stably sorted by expert id
 *  10. residual x' = bf16_rne(fp32_rne(x + y))   (stacked layers)
 *
 * The pages state no activation function and no weighting of the picks; the
 * reading taken here is GeGLU with the tanh form of GELU applied to the gate
 * projection, and a softmax over the k picked logits with the shared expert
 * at weight 1. Everything is evaluated in fp64 with plain loops. OpenMP only
 * splits independent rows; it changes no summation order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OQ_GROUP 64

typedef struct {
  const uint8_t* q;   /* 4-bit: [rows][cols/2]; 8-bit: [rows][cols] */
  const uint16_t* s;  /* bf16 bits [rows][cols/64] */
  const uint16_t* b;  /* bf16 bits [rows][cols/64] */
  int32_t rows, cols, bits;
} oq_mat;

typedef struct {
  oq_mat router;                    /* 8-bit [E x d] */
  oq_mat sgate, sup, sdown;         /* shared expert */
  const oq_mat* gate;               /* [E] routed experts, [f x d] */
  const oq_mat* up;                 /* [E] [f x d] */
  const oq_mat* down;               /* [E] [d x f] */
  int32_t n_experts, top_k;
} oq_layer;

static double bf16_value(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* step 1 */
int oracle_code(const oq_mat* m, int32_t n, int32_t i) {
  if (m->bits == 8) return m->q[(size_t)n * m->cols + i];
  uint8_t byte = m->q[(size_t)n * (m->cols / 2) + i / 2];
  return (i % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
}

/* step 2 */
double oracle_weight(const oq_mat* m, int32_t n, int32_t i) {
  size_t gi = (size_t)n * (m->cols / OQ_GROUP) + i / OQ_GROUP;
  return bf16_value(m->s[gi]) * (double)oracle_code(m, n, i) + bf16_value(m->b[gi]);
}

void oracle_dequant(const oq_mat* m, double* W) {
  for (int32_t n = 0; n < m->rows; ++n)
    for (int32_t i = 0; i < m->cols; ++i) W[(size_t)n * m->cols + i] = oracle_weight(m, n, i);
}

/* out[n] = sum_i W[n,i] v[i], i ascending */
void oracle_matvec(const oq_mat* m, const double* v, double* out) {
  for (int32_t n = 0; n < m->rows; ++n) {
    double acc = 0.0;
    for (int32_t i = 0; i < m->cols; ++i) acc += oracle_weight(m, n, i) * v[i];
    out[n] = acc;
  }
}

/* tanh form of GELU (Hendrycks & Gimpel) */
double oracle_gelu_tanh(double z) {
  const double c = sqrt(2.0 / M_PI);
  return 0.5 * z * (1.0 + tanh(c * (z + 0.044715 * z * z * z)));
}

/* step 3 */
void oracle_router_logits(const oq_mat* router, const double* x, const float* offset, double* logits) {
  oracle_matvec(router, x, logits);
  if (offset)
    for (int32_t e = 0; e < router->rows; ++e) logits[e] += (double)offset[e];
}

/* a ranks before b: larger logit first, ties to the lower expert id. The pages
   never meet a NaN logit; this oracle ranks a NaN below every number (as -inf),
   which keeps the order total. */
static double rank_key(double v) { return v != v ? -INFINITY : v; }
static int ranks_before(const double* l, int a, int b) {
  const double va = rank_key(l[a]), vb = rank_key(l[b]);
  return va > vb || (va == vb && a < b);
}

/* steps 4 and 5; gap = l_(k) - l_(k+1), the margin of the k-th pick (INFINITY if k == E) */
void oracle_topk_softmax(const double* logits, int32_t n_experts, int32_t k, int32_t* idx, double* p,
                         double* gap) {
  char* taken = (char*)calloc((size_t)n_experts, 1);
  int32_t next = -1;
  for (int32_t j = 0; j <= k && j < n_experts; ++j) {
    int32_t best = -1;
    for (int32_t e = 0; e < n_experts; ++e)
      if (!taken[e] && (best < 0 || ranks_before(logits, e, best))) best = e;
    taken[best] = 1;
    if (j < k) idx[j] = best; else next = best;
  }
  free(taken);
  if (gap) *gap = (next >= 0) ? logits[idx[k - 1]] - logits[next] : INFINITY;
  double sum = 0.0;
  for (int32_t j = 0; j < k; ++j) sum += exp(logits[idx[j]] - logits[idx[0]]);
  for (int32_t j = 0; j < k; ++j) p[j] = exp(logits[idx[j]] - logits[idx[0]]) / sum;
}

/* softmax over the logits of a given pick list (used when the picks come from elsewhere) */
void oracle_softmax_at(const double* logits, const int32_t* idx, int32_t k, double* p) {
  double sum = 0.0;
  for (int32_t j = 0; j < k; ++j) sum += exp(logits[idx[j]] - logits[idx[0]]);
  for (int32_t j = 0; j < k; ++j) p[j] = exp(logits[idx[j]] - logits[idx[0]]) / sum;
}

/* steps 6 and 7: out = Wd (gelu_tanh(Wg x) * (Wu x)) */
void oracle_expert(const oq_mat* gate, const oq_mat* up, const oq_mat* down, const double* x, double* out) {
  int32_t f = gate->rows;
  double* g = (double*)malloc(sizeof(double) * (size_t)f);
  double* u = (double*)malloc(sizeof(double) * (size_t)f);
  double* h = (double*)malloc(sizeof(double) * (size_t)f);
  oracle_matvec(gate, x, g);
  oracle_matvec(up, x, u);
  for (int32_t j = 0; j < f; ++j) h[j] = oracle_gelu_tanh(g[j]) * u[j];
  oracle_matvec(down, h, out);
  free(g);
  free(u);
  free(h);
}

/* step 8 for one row */
void oracle_combine(const double* shared_out, const double* expert_out, const double* p, int32_t k, int32_t d,
                    double* y) {
  for (int32_t n = 0; n < d; ++n) {
    double acc = shared_out[n];
    for (int32_t j = 0; j < k; ++j) acc += p[j] * expert_out[(size_t)j * d + n];
    y[n] = acc;
  }
}

/*
 * The whole block for `rows` rows of x ([rows][d], fp64 values of the stored
 * activations). Outputs (any may be NULL except idx and p):
 *   logits [rows][E], idx [rows][k], p [rows][k], gap [rows],
 *   expert_out [rows][k][d] (unweighted E_{idx}(x)), shared_out [rows][d], y [rows][d].
 * If use_idx is nonzero, idx is an INPUT (picks made elsewhere) and p is the
 * softmax of this oracle's logits at those picks.
 */
void oracle_moe_rows(const oq_layer* L, const double* x, int32_t rows, const float* offset, int32_t use_idx,
                     double* logits, int32_t* idx, double* p, double* gap, double* expert_out,
                     double* shared_out, double* y) {
  const int32_t d = L->router.cols, E = L->n_experts, k = L->top_k;
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t r = 0; r < rows; ++r) {
    const double* xr = x + (size_t)r * d;
    double* lg = (double*)malloc(sizeof(double) * (size_t)E);
    double* eo = (double*)malloc(sizeof(double) * (size_t)k * d);
    double* so = (double*)malloc(sizeof(double) * (size_t)d);
    oracle_router_logits(&L->router, xr, offset, lg);
    if (use_idx)
      oracle_softmax_at(lg, idx + (size_t)r * k, k, p + (size_t)r * k);
    else
      oracle_topk_softmax(lg, E, k, idx + (size_t)r * k, p + (size_t)r * k, gap ? gap + r : NULL);
    for (int32_t j = 0; j < k; ++j) {
      int32_t e = idx[(size_t)r * k + j];
      oracle_expert(&L->gate[e], &L->up[e], &L->down[e], xr, eo + (size_t)j * d);
    }
    oracle_expert(&L->sgate, &L->sup, &L->sdown, xr, so);
    if (y) oracle_combine(so, eo, p + (size_t)r * k, k, d, y + (size_t)r * d);
    if (logits) memcpy(logits + (size_t)r * E, lg, sizeof(double) * (size_t)E);
    if (expert_out) memcpy(expert_out + (size_t)r * k * d, eo, sizeof(double) * (size_t)k * d);
    if (shared_out) memcpy(shared_out + (size_t)r * d, so, sizeof(double) * (size_t)d);
    free(lg);
    free(eo);
    free(so);
  }
}

/* logits only, for rows of x */
void oracle_router_rows(const oq_mat* router, const double* x, int32_t rows, const float* offset,
                        double* logits) {
  const int32_t d = router->cols, E = router->rows;
#pragma omp parallel for schedule(static)
  for (int32_t r = 0; r < rows; ++r)
    oracle_router_logits(router, x + (size_t)r * d, offset, logits + (size_t)r * E);
}

/* one expert applied to rows of x: out [rows][d_out] */
void oracle_expert_rows(const oq_mat* gate, const oq_mat* up, const oq_mat* down, const double* x, int32_t rows,
                        double* out) {
  const int32_t d = gate->cols, dout = down->rows;
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t r = 0; r < rows; ++r) oracle_expert(gate, up, down, x + (size_t)r * d, out + (size_t)r * dout);
}

/*
 * step 9: counting sort of the rows*k (row, slot) pairs by expert id, stable,
 * so pairs of one expert keep (row, slot) order. Pair id = row*k + slot.
 *   count[e] = pairs routed to e; offset[0..E] = exclusive prefix sum of count;
 *   perm[j] = pair id at sorted position j; inv_perm[pair] = its sorted position.
 */
void oracle_group_by_expert(const int32_t* idx, int32_t rows, int32_t k, int32_t n_experts, int32_t* count,
                            int32_t* offset, int32_t* perm, int32_t* inv_perm) {
  const int32_t P = rows * k;
  for (int32_t e = 0; e < n_experts; ++e) count[e] = 0;
  for (int32_t pr = 0; pr < P; ++pr) count[idx[pr]] += 1;
  offset[0] = 0;
  for (int32_t e = 0; e < n_experts; ++e) offset[e + 1] = offset[e] + count[e];
  int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)n_experts);
  for (int32_t e = 0; e < n_experts; ++e) cursor[e] = offset[e];
  for (int32_t pr = 0; pr < P; ++pr) {
    int32_t pos = cursor[idx[pr]]++;
    perm[pos] = pr;
    inv_perm[pr] = pos;
  }
  free(cursor);
}

/* step 10: x' = bf16_rne(fp32_rne(x + y)); x and x' are bf16 bit patterns, y fp32 */
void oracle_residual_bf16(const uint16_t* x, const float* y, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) {
    uint32_t xb = (uint32_t)x[i] << 16;
    float xf;
    memcpy(&xf, &xb, sizeof xf);
    float t = xf + y[i]; /* one IEEE binary32 addition: the exact sum rounded to nearest even */
    uint32_t u;
    memcpy(&u, &t, sizeof u);
    u += 0x7FFFu + ((u >> 16) & 1u); /* round to nearest even at bit 16 */
    out[i] = (uint16_t)(u >> 16);
  }
}

/* thread control for timing runs (OpenMP splits rows only) */
#ifdef _OPENMP
#include <omp.h>
void oracle_set_threads(int32_t n) { omp_set_num_threads(n); }
int32_t oracle_threads(void) { return omp_get_max_threads(); }
#else
void oracle_set_threads(int32_t n) { (void)n; }
int32_t oracle_threads(void) { return 1; }
#endif
