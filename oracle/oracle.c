/*
 * oracle.c -- plain fp64 CPU reference of one decode step of a Gemma-4-E2B-
 * shaped decoder.  TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke
 * entry and the bench's CPU-baseline leg; never by the product path.  It
 * shares no code, header or table with the HIP library.
 *
 * Everything is computed in double.  Stored weights are decoded exactly:
 * bf16 -> double is a widening; an int4 code c (offset binary, q = c - 8)
 * times its bf16 group scale is exact in double.  The K/V cache holds double
 * values; with kv_bf16 set (the default of the Python wrapper) each stored K
 * and V element is rounded to bf16 first, because the pages fix the cache
 * dtype at bf16 ("Gemma 4 E2B in JAX on One TPU v5e", Step 2: "KV cache:
 * bf16"; "One TPU chip, eight agents", Feasibility part 1: 18.00 KiB/token
 * at bf16).
 *
 * Sources (pages named by title; sections as printed on them):
 *  - RMSNorm in f32/f64: mean of squares, + eps, rsqrt, optional gain
 *    ("Gemma 4 E2B in JAX on One TPU v5e ...", Step 4, rms_norm listing).
 *  - per-layer embeddings (PLE) build and mixing, gelu with the tanh
 *    approximation ("Porting Gemma 4 E2B to SGLang-JAX ...", Step 3).
 *  - K/V sharing, queries-only RoPE on sharing layers, post-norm post-RoPE K/V
 *    ("Porting ...", Step 4; "One TPU chip, eight agents", The engine:
 *    kv_share_map and "#3225" table: sharing layers hold no K-side weights).
 *  - layer table and widths ("Porting ...", Step 1 table and bullets; Step 5:
 *    double-wide MLP from the first shared layer on).
 *  - W4A16 format: eight int4 per int32, one bf16 scale per 32-group
 *    ("One TPU chip ...", The engine; "Gemma 4 E2B in Pure JAX on a Colab
 *    TPU ...", intro table and cell 3.1).
 *  - tied lm_head ("... Colab TPU ...", cell 2.2) and greedy argmax.
 * Readings where the pages are silent (embedding x sqrt(H), attention scale
 * 1/sqrt(hd), rotate-half RoPE, sandwich norms, v-norm without gain, layer
 * scalar multiplying the whole residual, lowest index on argmax ties, window
 * = W keys ending at the current one, a shared layer with no same-type
 * source owning its K/V) are readings, not statements of the pages; each is
 * applied the same way throughout.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int num_hidden_layers, num_kv_shared_layers, hidden_size, num_attention_heads,
      num_key_value_heads, head_dim, global_head_dim, sliding_window,
      layer_pattern_period, intermediate_size, use_double_wide_mlp,
      hidden_size_per_layer_input, vocab_size, quant /* 0 bf16, 1 w4a16 */, group_size;
  double rms_eps, rope_theta_sliding, rope_theta_full;
  int kv_bf16; /* 1: K/V stored in the cache rounded to bf16 (the pages' cache dtype) */
  int embed_quant; /* 0: bf16 vocabulary tables; 1: W4A16 (int4 codes, bf16 group scales) */
  int kv_quant;    /* 1: K/V cached as int8 with one fp32 scale per cached row (overrides kv_bf16) */
} orc_config;

typedef struct {
  int quant, N, K, G;
  const uint16_t* w;      /* bf16 [N, K] */
  const uint32_t* packed; /* [N, K/8] */
  const uint16_t* scale;  /* bf16 [N, K/G] */
} orc_lin;

typedef struct {
  int full, hd, I, src;
  double theta;
  orc_lin q, k, v, o, gate, up, down, pg, pp;
  const uint16_t *g_in, *g_q, *g_k, *g_pa, *g_pf, *g_ff, *g_pple, *scalar;
} orc_layer;

typedef struct {
  orc_config c;
  int L, H, P, V, nq, first_shared;
  const uint16_t *g_plpn, *g_final;
  orc_lin embed; /* tied token embedding / lm_head [V, H] */
  orc_lin ple;   /* per-layer table [V, L*P] */
  orc_lin plmp;
  orc_layer* layers;
  int max_seq, max_ctx;
  double **kc, **vc; /* per layer; non-NULL only where the layer owns K/V */
  double jitter;     /* test hook: relative jitter of K/V before the cache rounds them */
  uint64_t jitter_seed;
  /* scratch */
  double *e, *tok, *u, *pli, *h, *a, *q, *kv, *o, *t, *g, *up, *r, *y;
} orc_model;

static char g_err[512];
const char* orc_error(void) { return g_err; }

static double bf(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* nearest-even bf16 of the fp32 value of x (the cache stores bf16) */
static double round_bf16(double x) {
  float f = (float)x;
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  u &= 0xFFFF0000u;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* OpenMP threads the products use (the CPU baseline is timed on all host
 * cores and on one) */
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int orc_get_threads(void) { return omp_get_max_threads(); }

/* ---------------------------------------------------------------- pieces */

/* Symmetric int8 of one cached row (one token's K or V of one layer), the
 * int8 KV cache of "One TPU chip, eight agents" (Measured: int8 KV donated;
 * KV memory math): the pages fix the element size (one byte) but not the
 * scale granularity; the reading here is one scale per cached row, s =
 * max |x| / 127, code = nearest-even(x / s).  The codes are decided in fp32,
 * the kernels' precision, so that the same fp32 row gives the same codes on
 * both sides; a row of zeros has scale 0 and codes 0. */
void orc_quant_int8(const double* x, int n, int8_t* q, float* s) {
  float amax = 0.0f;
  for (int i = 0; i < n; ++i) {
    const float a = fabsf((float)x[i]);
    if (a > amax) amax = a;
  }
  const float sc = amax / 127.0f;
  for (int i = 0; i < n; ++i) {
    float c = sc > 0.0f ? rintf((float)x[i] / sc) : 0.0f;
    if (c > 127.0f) c = 127.0f;
    if (c < -127.0f) c = -127.0f;
    q[i] = (int8_t)c;
  }
  *s = sc;
}


/* decoded weight W[n][k] */
static double lin_w(const orc_lin* L, int64_t n, int64_t k) {
  if (L->quant == 0) return bf(L->w[n * L->K + k]);
  uint32_t word = L->packed[n * (L->K / 8) + k / 8];
  int code = (int)((word >> (4 * (k % 8))) & 15u);
  return (double)(code - 8) * bf(L->scale[n * (L->K / L->G) + k / L->G]);
}

static void linear(const orc_lin* L, const double* x, double* y) {
#pragma omp parallel for schedule(static)
  for (int n = 0; n < L->N; ++n) {
    double s = 0.0;
    for (int k = 0; k < L->K; ++k) s += lin_w(L, n, k) * x[k];
    y[n] = s;
  }
}

void orc_linear_apply(int quant, const void* w, const uint16_t* scale, int N, int K, int G,
                      const double* x, double* y) {
  orc_lin L = {quant, N, K, G, (const uint16_t*)w, (const uint32_t*)w, scale};
  linear(&L, x, y);
}

double orc_decode_weight(int quant, const void* w, const uint16_t* scale, int N, int K, int G,
                         int64_t n, int64_t k) {
  orc_lin L = {quant, N, K, G, (const uint16_t*)w, (const uint32_t*)w, scale};
  return lin_w(&L, n, k);
}

/* y = x / sqrt(mean(x^2) + eps) * g   (g NULL: no gain) */
void orc_rmsnorm(const double* x, int n, const uint16_t* g, double eps, double* y) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += x[i] * x[i];
  double r = 1.0 / sqrt(ss / n + eps);
  for (int i = 0; i < n; ++i) y[i] = x[i] * r * (g ? bf(g[i]) : 1.0);
}

/* gelu, tanh form: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) */
double orc_gelu_tanh(double x) {
  const double c = 0.79788456080286535587989211986876; /* sqrt(2/pi) */
  return 0.5 * x * (1.0 + tanh(c * (x + 0.044715 * x * x * x)));
}

/* rotate-half RoPE: pair (i, i + hd/2) turned by pos * theta^(-2i/hd) */
void orc_rope(double* x, int hd, int pos, double theta) {
  int half = hd / 2;
  for (int i = 0; i < half; ++i) {
    double ang = (double)pos * pow(theta, -2.0 * i / hd);
    double c = cos(ang), s = sin(ang);
    double a = x[i], b = x[i + half];
    x[i] = a * c - b * s;
    x[i + half] = a * s + b * c;
  }
}

/* o = sum_j softmax_j(q . K_j / sqrt(hd)) V_j over rows j0..j1 (inclusive) */
void orc_attend(const double* q, int hd, const double* K, const double* V, int j0, int j1,
                double* o) {
  int n = j1 - j0 + 1;
  double* s = (double*)malloc(sizeof(double) * n);
  double mx = -INFINITY, scale = 1.0 / sqrt((double)hd);
  for (int j = 0; j < n; ++j) {
    double d = 0.0;
    for (int i = 0; i < hd; ++i) d += q[i] * K[(int64_t)(j0 + j) * hd + i];
    s[j] = d * scale;
    if (s[j] > mx) mx = s[j];
  }
  double den = 0.0;
  for (int j = 0; j < n; ++j) { s[j] = exp(s[j] - mx); den += s[j]; }
  for (int i = 0; i < hd; ++i) o[i] = 0.0;
  for (int j = 0; j < n; ++j) {
    double w = s[j] / den;
    for (int i = 0; i < hd; ++i) o[i] += w * V[(int64_t)(j0 + j) * hd + i];
  }
  free(s);
}

/* lowest index of the maximum */
int orc_argmax(const double* x, int n) {
  int best = 0;
  for (int i = 1; i < n; ++i)
    if (x[i] > x[best]) best = i;
  return best;
}

/* --------------------------------------------------------------- layer map */

static int is_full(const orc_config* c, int l) {
  return (l % c->layer_pattern_period) == c->layer_pattern_period - 1;
}

/* source of each layer's K/V: itself below the first shared layer; above it,
 * the last earlier non-shared layer of its own type.  A shared layer with no
 * such source keeps its own K/V. */
static int kv_source(const orc_config* c, int l) {
  int first = c->num_hidden_layers - c->num_kv_shared_layers;
  if (l < first) return l;
  int src = -1;
  for (int i = 0; i < first; ++i)
    if (is_full(c, i) == is_full(c, l)) src = i;
  return src < 0 ? l : src;
}

/* ------------------------------------------------------------ construction */

typedef struct { int n; const char** names; const void** ptrs; } tab_t;

static const void* find(const tab_t* t, const char* name) {
  for (int i = 0; i < t->n; ++i)
    if (strcmp(t->names[i], name) == 0) return t->ptrs[i];
  snprintf(g_err, sizeof g_err, "missing tensor %s", name);
  return NULL;
}

static int get_lin_q(const tab_t* t, int quant, int G, const char* name, int N, int K, orc_lin* L) {
  char buf[256];
  L->quant = quant; L->N = N; L->K = K; L->G = G;
  L->w = NULL; L->packed = NULL; L->scale = NULL;
  if (quant == 0) {
    L->w = (const uint16_t*)find(t, name);
    return L->w != NULL;
  }
  snprintf(buf, sizeof buf, "%s_packed", name);
  L->packed = (const uint32_t*)find(t, buf);
  snprintf(buf, sizeof buf, "%s_scale", name);
  L->scale = (const uint16_t*)find(t, buf);
  return L->packed && L->scale;
}

static int get_lin(const tab_t* t, const orc_config* c, const char* name, int N, int K, orc_lin* L) {
  return get_lin_q(t, c->quant, c->group_size, name, N, K, L);
}

void orc_destroy(void* p);

void* orc_create(const orc_config* c, int n, const char** names, const void** ptrs, int max_seq,
                 int max_ctx) {
  tab_t t = {n, names, ptrs};
  orc_model* m = (orc_model*)calloc(1, sizeof(orc_model));
  char nm[256];
  m->c = *c;
  m->L = c->num_hidden_layers; m->H = c->hidden_size; m->P = c->hidden_size_per_layer_input;
  m->V = c->vocab_size; m->nq = c->num_attention_heads;
  m->first_shared = c->num_hidden_layers - c->num_kv_shared_layers;
  m->max_seq = max_seq; m->max_ctx = max_ctx;
  int L = m->L, H = m->H, P = m->P;
  int ok = 1;
  /* the vocabulary tables: bf16, or (embed_quant) the W4A16 format of the linears */
  ok &= get_lin_q(&t, c->embed_quant, c->group_size, "model.embed_tokens.weight", m->V, H, &m->embed);
  ok &= get_lin_q(&t, c->embed_quant, c->group_size, "model.embed_tokens_per_layer.weight", m->V,
                  L * P, &m->ple);
  ok &= (m->g_plpn = (const uint16_t*)find(&t, "model.per_layer_projection_norm.weight")) != NULL;
  ok &= (m->g_final = (const uint16_t*)find(&t, "model.norm.weight")) != NULL;
  ok &= get_lin(&t, c, "model.per_layer_model_projection.weight", L * P, H, &m->plmp);
  m->layers = (orc_layer*)calloc(L, sizeof(orc_layer));
  m->kc = (double**)calloc(L, sizeof(double*));
  m->vc = (double**)calloc(L, sizeof(double*));
  int maxhd = 0, maxI = 0;
  for (int l = 0; l < L && ok; ++l) {
    orc_layer* y = &m->layers[l];
    y->full = is_full(c, l);
    y->hd = y->full ? c->global_head_dim : c->head_dim;
    y->theta = y->full ? c->rope_theta_full : c->rope_theta_sliding;
    y->I = c->intermediate_size * ((c->use_double_wide_mlp && l >= m->first_shared) ? 2 : 1);
    y->src = kv_source(c, l);
    if (y->hd > maxhd) maxhd = y->hd;
    if (y->I > maxI) maxI = y->I;
#define G(field, s) (snprintf(nm, sizeof nm, "model.layers.%d.%s", l, s), \
                     ok &= (y->field = (const uint16_t*)find(&t, nm)) != NULL)
#define LIN(field, s, N_, K_) (snprintf(nm, sizeof nm, "model.layers.%d.%s", l, s), \
                               ok &= get_lin(&t, c, nm, N_, K_, &y->field))
    G(g_in, "input_layernorm.weight");
    G(g_q, "self_attn.q_norm.weight");
    G(g_pa, "post_attention_layernorm.weight");
    G(g_pf, "pre_feedforward_layernorm.weight");
    G(g_ff, "post_feedforward_layernorm.weight");
    G(g_pple, "post_per_layer_input_norm.weight");
    G(scalar, "layer_scalar");
    LIN(q, "self_attn.q_proj.weight", m->nq * y->hd, H);
    LIN(o, "self_attn.o_proj.weight", H, m->nq * y->hd);
    LIN(gate, "mlp.gate_proj.weight", y->I, H);
    LIN(up, "mlp.up_proj.weight", y->I, H);
    LIN(down, "mlp.down_proj.weight", H, y->I);
    LIN(pg, "per_layer_input_gate.weight", P, H);
    LIN(pp, "per_layer_projection.weight", H, P);
    if (y->src == l) {
      G(g_k, "self_attn.k_norm.weight");
      LIN(k, "self_attn.k_proj.weight", y->hd, H);
      LIN(v, "self_attn.v_proj.weight", y->hd, H);
      size_t cnt = (size_t)max_seq * max_ctx * y->hd;
      m->kc[l] = (double*)calloc(cnt, sizeof(double));
      m->vc[l] = (double*)calloc(cnt, sizeof(double));
      if (!m->kc[l] || !m->vc[l]) { snprintf(g_err, sizeof g_err, "out of memory"); ok = 0; }
    }
#undef G
#undef LIN
  }
  if (!ok) { orc_destroy(m); return NULL; }
  int nqhd = m->nq * maxhd;
  m->e = calloc(H, sizeof(double)); m->tok = calloc((size_t)L * P, sizeof(double));
  m->u = calloc((size_t)L * P, sizeof(double)); m->pli = calloc((size_t)L * P, sizeof(double));
  m->h = calloc(H, sizeof(double)); m->a = calloc(H, sizeof(double));
  m->q = calloc(nqhd, sizeof(double)); m->kv = calloc(2 * maxhd, sizeof(double));
  m->o = calloc(nqhd, sizeof(double)); m->t = calloc(H > nqhd ? H : nqhd, sizeof(double));
  m->g = calloc(maxI, sizeof(double)); m->up = calloc(maxI, sizeof(double));
  m->r = calloc(P > H ? P : H, sizeof(double)); m->y = calloc(H, sizeof(double));
  return m;
}

void orc_destroy(void* p) {
  orc_model* m = (orc_model*)p;
  if (!m) return;
  for (int l = 0; l < m->L; ++l) {
    if (m->kc) free(m->kc[l]);
    if (m->vc) free(m->vc[l]);
  }
  free(m->kc); free(m->vc); free(m->layers);
  free(m->e); free(m->tok); free(m->u); free(m->pli); free(m->h); free(m->a); free(m->q);
  free(m->kv); free(m->o); free(m->t); free(m->g); free(m->up); free(m->r); free(m->y);
  free(m);
}

int orc_kv_source(void* p, int l) { return ((orc_model*)p)->layers[l].src; }

/* K (which 0) or V (which 1) row consumed by layer l for (seq, pos) */
const double* orc_kv_row(void* p, int l, int which, int seq, int pos) {
  orc_model* m = (orc_model*)p;
  const orc_layer* y = &m->layers[l];
  double* base = which ? m->vc[y->src] : m->kc[y->src];
  return base + ((size_t)seq * m->max_ctx + pos) * y->hd;
}

/* Test set-up: store n cached positions pos0 .. pos0+n-1 of sequence seq
 * for layer l, which must own its K/V, from bf16 bit patterns ([n][hd] each
 * for K and V).  A long context can then be given as seeded cache contents
 * instead of a long prefill.  0, or -1 on a bad argument. */
int orc_kv_load(void* p, int l, int seq, int pos0, int n, const uint16_t* k, const uint16_t* v) {
  orc_model* m = (orc_model*)p;
  if (l < 0 || l >= m->L || m->layers[l].src != l || seq < 0 || seq >= m->max_seq || pos0 < 0 ||
      n < 0 || pos0 + n > m->max_ctx)
    return -1;
  const int hd = m->layers[l].hd;
  for (int i = 0; i < n; ++i)
    for (int d = 0; d < hd; ++d) {
      const size_t o = ((size_t)seq * m->max_ctx + pos0 + i) * hd + d;
      m->kc[l][o] = bf(k[(size_t)i * hd + d]);
      m->vc[l][o] = bf(v[(size_t)i * hd + d]);
    }
  return 0;
}

/* Test hook (conditioning checks): before the cache rounds a new K/V row,
 * multiply each element by (1 + rel * u), u uniform in [-1, 1) from a
 * SplitMix64 hash of (seed, layer, K/V, position, element).  It stands for an
 * implementation that computes the same row with a relative error of about
 * rel (fp32 against this fp64 reference); rel 0 turns it off. */
void orc_set_kv_jitter(void* p, double rel, uint64_t seed) {
  orc_model* m = (orc_model*)p;
  m->jitter = rel;
  m->jitter_seed = seed;
}

static double jitter_u(uint64_t seed, int l, int which, int pos, int i) {
  uint64_t z = seed ^ ((uint64_t)l << 48) ^ ((uint64_t)which << 47) ^ ((uint64_t)pos << 16) ^ (uint64_t)i;
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return (double)(z >> 11) * (1.0 / 9007199254740992.0) * 2.0 - 1.0;
}

/* Test set-up: overwrite one cached row (layer l must own its K/V) with the
 * given values, exactly as given.  0, or -1 on a bad argument. */
int orc_kv_set(void* p, int l, int which, int seq, int pos, const double* row) {
  orc_model* m = (orc_model*)p;
  if (l < 0 || l >= m->L || m->layers[l].src != l || seq < 0 || seq >= m->max_seq || pos < 0 ||
      pos >= m->max_ctx || (which != 0 && which != 1))
    return -1;
  const int hd = m->layers[l].hd;
  double* dst = (which ? m->vc[l] : m->kc[l]) + ((size_t)seq * m->max_ctx + pos) * hd;
  memcpy(dst, row, sizeof(double) * hd);
  return 0;
}

/* ------------------------------------------------------------- the step */

/* Embedding e = E[x] * sqrt(H), and the per-layer inputs pli [L, P]: the
 * token's row of the per-layer table scaled by sqrt(P), plus the projection
 * of e scaled by H^-1/2 and RMS-normed per layer slice, the sum times 2^-1/2
 * ("Porting Gemma 4 E2B to SGLang-JAX", Step 3). */
static void orc_inputs(orc_model* m, int x, double* e, double* pli) {
  const int L = m->L, H = m->H, P = m->P;
  for (int i = 0; i < H; ++i) e[i] = lin_w(&m->embed, x, i) * sqrt((double)H);
  for (int i = 0; i < L * P; ++i) m->tok[i] = lin_w(&m->ple, x, i) * sqrt((double)P);
  linear(&m->plmp, e, m->u);
  for (int i = 0; i < L * P; ++i) m->u[i] *= 1.0 / sqrt((double)H);
  for (int l = 0; l < L; ++l) orc_rmsnorm(m->u + l * P, P, m->g_plpn, m->c.rms_eps, m->u + l * P);
  for (int i = 0; i < L * P; ++i) pli[i] = (m->u[i] + m->tok[i]) * sqrt(0.5);
}

/* test hook: e [H] and pli [L*P] for token x */
int orc_debug_inputs(void* p, int x, double* e, double* pli) {
  orc_model* m = (orc_model*)p;
  if (x < 0 || x >= m->V) return -1;
  orc_inputs(m, x, e, pli);
  return 0;
}

/* One token x of sequence seq at position pos.  Writes logits[V] if given and
 * the final normed hidden state y[H] if given; returns the greedy token. */
int orc_step_ex(void* p, int seq, int x, int pos, int head, double* logits, double* y_out) {
  orc_model* m = (orc_model*)p;
  const orc_config* c = &m->c;
  const int L = m->L, H = m->H, P = m->P, nq = m->nq;
  const double eps = c->rms_eps;
  if (seq < 0 || seq >= m->max_seq || pos < 0 || pos >= m->max_ctx || x < 0 || x >= m->V) {
    snprintf(g_err, sizeof g_err, "step out of range (seq %d pos %d token %d)", seq, pos, x);
    return -1;
  }
  orc_inputs(m, x, m->e, m->pli);

  memcpy(m->h, m->e, sizeof(double) * H);
  for (int l = 0; l < L; ++l) {
    const orc_layer* y = &m->layers[l];
    const int hd = y->hd;
    /* attention block */
    orc_rmsnorm(m->h, H, y->g_in, eps, m->a);
    linear(&y->q, m->a, m->q);
    for (int i = 0; i < nq; ++i) {
      orc_rmsnorm(m->q + i * hd, hd, y->g_q, eps, m->q + i * hd);
      orc_rope(m->q + i * hd, hd, pos, y->theta);
    }
    if (y->src == l) {
      double* kr = m->kc[l] + ((size_t)seq * m->max_ctx + pos) * hd;
      double* vr = m->vc[l] + ((size_t)seq * m->max_ctx + pos) * hd;
      linear(&y->k, m->a, m->kv);
      orc_rmsnorm(m->kv, hd, y->g_k, eps, kr);
      orc_rope(kr, hd, pos, y->theta);
      linear(&y->v, m->a, m->kv);
      orc_rmsnorm(m->kv, hd, NULL, eps, vr);
      if (m->jitter != 0.0)
        for (int i = 0; i < hd; ++i) {
          kr[i] *= 1.0 + m->jitter * jitter_u(m->jitter_seed, l, 0, pos, i);
          vr[i] *= 1.0 + m->jitter * jitter_u(m->jitter_seed, l, 1, pos, i);
        }
      if (c->kv_quant) {
        /* the cache holds codes and a scale; attention reads code * scale */
        int8_t qk[512], qv[512];
        float sk, sv;
        orc_quant_int8(kr, hd, qk, &sk);
        orc_quant_int8(vr, hd, qv, &sv);
        for (int i = 0; i < hd; ++i) {
          kr[i] = (double)qk[i] * (double)sk;
          vr[i] = (double)qv[i] * (double)sv;
        }
      } else if (c->kv_bf16) {
        for (int i = 0; i < hd; ++i) {
          kr[i] = round_bf16(kr[i]);
          vr[i] = round_bf16(vr[i]);
        }
      }
    }
    {
      const double* K = m->kc[y->src] + (size_t)seq * m->max_ctx * hd;
      const double* Vv = m->vc[y->src] + (size_t)seq * m->max_ctx * hd;
      int j0 = y->full ? 0 : (pos - c->sliding_window + 1 > 0 ? pos - c->sliding_window + 1 : 0);
      for (int i = 0; i < nq; ++i) orc_attend(m->q + i * hd, hd, K, Vv, j0, pos, m->o + i * hd);
    }
    linear(&y->o, m->o, m->t);
    orc_rmsnorm(m->t, H, y->g_pa, eps, m->t);
    for (int i = 0; i < H; ++i) m->h[i] += m->t[i];
    /* MLP block (GeGLU) */
    orc_rmsnorm(m->h, H, y->g_pf, eps, m->a);
    linear(&y->gate, m->a, m->g);
    linear(&y->up, m->a, m->up);
    for (int i = 0; i < y->I; ++i) m->g[i] = orc_gelu_tanh(m->g[i]) * m->up[i];
    linear(&y->down, m->g, m->t);
    orc_rmsnorm(m->t, H, y->g_ff, eps, m->t);
    for (int i = 0; i < H; ++i) m->h[i] += m->t[i];
    /* per-layer input mixing, then the layer scalar */
    linear(&y->pg, m->h, m->r);
    for (int i = 0; i < P; ++i) m->r[i] = orc_gelu_tanh(m->r[i]) * m->pli[l * P + i];
    linear(&y->pp, m->r, m->t);
    orc_rmsnorm(m->t, H, y->g_pple, eps, m->t);
    double s = bf(y->scalar[0]);
    for (int i = 0; i < H; ++i) m->h[i] = (m->h[i] + m->t[i]) * s;
  }
  orc_rmsnorm(m->h, H, m->g_final, eps, m->y);
  if (y_out) memcpy(y_out, m->y, sizeof(double) * H);
  if (!head) return 0;
  /* tied lm_head and greedy choice */
  double* lg = logits ? logits : (double*)malloc(sizeof(double) * m->V);
  linear(&m->embed, m->y, lg);
  int best = orc_argmax(lg, m->V);
  if (!logits) free(lg);
  return best;
}

int orc_step(void* p, int seq, int x, int pos, double* logits, double* y_out) {
  return orc_step_ex(p, seq, x, pos, 1, logits, y_out);
}

/* prefill = the step applied to each prompt token in order; returns the
 * greedy token after the last one (logits of the last row if given) */
int orc_prefill(void* p, int seq, const int32_t* toks, int n, int pos0, double* logits_last) {
  int best = -1;
  for (int i = 0; i < n; ++i) {
    best = orc_step_ex(p, seq, toks[i], pos0 + i, i == n - 1, i == n - 1 ? logits_last : NULL, NULL);
    if (best < 0) return best;
  }
  return best;
}
