/*
 * moe_oracle.c -- plain, slow CPU oracle of the DeepSeekMoE layer forward with
 * auxiliary-loss-free load balancing.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this library: only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark use it.  It shares no source, header, table or constant with the HIP
 * library; every routine here is written from the definitions on the pages.
 *
 * Sources (web pages summarising the DeepSeek-V3 technical report):
 *   [mpbf]   mpbf.cn, "DeepSeek-V3技术报告" summary, section 2.2 "DeepSeekMoE 与
 *            无辅助损失" (structure, sigmoid gating, bias routing, bias update,
 *            node-limited routing, no token dropping), section 3.1 "FP8 混合精度"
 *            (tile-wise scaling, higher-precision accumulation), section 4.3
 *            (block-wise rather than global scaling), section 6.2 (bias rule
 *            driven by per-expert token counts in the batch).
 *   [joto]   joto.ai, "DeepSeek V3：AI领域的全新突破，性能与效率双重飞跃", items 1, 3
 *            and 6 (bias adjusted after each step; FP8 inputs and weights with FP32
 *            accumulation; at most 4 nodes per token).
 *   [p2hp]   p2hp.com, "Deepseek-v3技术报告简报", section 2 (256 routed experts,
 *            1 shared expert, top-8, width 7168).
 *   [resmic] blog.resmic.cn, "DeepSeek-V3架构深度解析", section "核心架构二" (output is
 *            the shared-expert output plus the gate-weighted routed outputs) and
 *            "核心架构三" (bias takes no part in back-propagation).
 *
 * Precision.  Routing decisions are integers decided by fp32 comparisons, so the
 * router (logits, sigmoid, keys, group scores, gates) is evaluated in fp32 in one
 * fixed order that the GPU kernels also follow:
 *   - logits are a sequential fused multiply-add chain over the hidden dimension,
 *     starting from +0;
 *   - exp is an own single-precision routine (Cody-Waite reduction by ln 2, then a
 *     degree-7 Taylor polynomial evaluated by Horner's rule with fused multiply-add),
 *     so both sides get the same bits;
 *   - division is IEEE (correctly rounded).
 * Expert FFN arithmetic is done in fp64 and rounded only where the layer stores a
 * tensor (h and Y at the activation dtype).  The FP8 path quantises exactly as
 * the GPU does (bit-exact codes and scales) and then accumulates in fp64.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -mfma -shared -fPIC -pthread.
 * fmaf() is the C99 single-rounding fused multiply-add.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { DT_F32 = 0, DT_BF16 = 1, DT_E4M3 = 2 };

/* ------------------------------------------------------------------------- */
/* Scalar number formats                                                      */
/* ------------------------------------------------------------------------- */

static float bits_to_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bfloat16 is the top half of an IEEE binary32; widening is exact. */
float oracle_bf16_to_f32(uint16_t b) { return bits_to_f32((uint32_t)b << 16); }

/* Round a double to the nearest value with `p` significant bits, ties to even,
 * with the quantum never below 2^qmin (gradual underflow).  Exact: the scaling is
 * by powers of two and rint() rounds half to even in the default mode. */
static double round_sig(double v, int p, int qmin) {
  if (v == 0.0 || !isfinite(v)) return v;
  int e;
  frexp(v, &e);                 /* |v| in [2^(e-1), 2^e) */
  int q = e - p;                /* quantum exponent */
  if (q < qmin) q = qmin;
  return ldexp(rint(ldexp(v, -q)), q);
}

/* bf16 round-to-nearest-even from double (8 significant bits, min quantum 2^-133). */
uint16_t oracle_bf16_from_f64(double v) {
  if (isnan(v)) return 0x7FC0;
  double r = round_sig(v, 8, -133);
  if (fabs(r) >= 0x1p128) return (uint16_t)(v < 0 ? 0xFF80 : 0x7F80);
  return (uint16_t)(f32_to_bits((float)r) >> 16); /* r has <= 8 significant bits */
}

/* binary32 round-to-nearest-even from double (24 significant bits, quantum >= 2^-149). */
float oracle_f32_from_f64(double v) { return (float)round_sig(v, 24, -149); }

/* OCP FP8 E4M3 ("fn"): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, no
 * infinities, S.1111.111 is NaN, largest finite 448, subnormals m/8 * 2^-6. */
float oracle_e4m3_to_f32(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m / 8.0, -6);
  else v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return (float)(s ? -v : v);
}

/* Encode a float to E4M3 with round-to-nearest-even and saturation at +-448. */
uint8_t oracle_e4m3_from_f32(float f) {
  if (isnan(f)) return 0x7F;
  uint8_t s = signbit(f) ? 0x80 : 0;
  double a = fabs((double)f);
  if (a > 448.0) a = 448.0;      /* saturate; every value above rounds to >= 448 */
  double r = round_sig(a, 4, -9); /* 4 significant bits; subnormal quantum 2^-9 */
  if (r > 448.0) r = 448.0;
  if (r == 0.0) return s;
  int e;
  frexp(r, &e);                   /* r in [2^(e-1), 2^e) */
  int be = e - 1 + 7;             /* biased exponent */
  if (be <= 0) {                  /* subnormal: r = m * 2^-9 */
    int m = (int)ldexp(r, 9);
    return (uint8_t)(s | m);
  }
  int m = (int)(ldexp(r, -(e - 1)) * 8.0) - 8;
  return (uint8_t)(s | (be << 3) | m);
}

/* ------------------------------------------------------------------------- */
/* Router numerics: own exp and sigmoid                                       */
/* ------------------------------------------------------------------------- */

/* ln 2 split for Cody-Waite reduction: the high part is ln 2 rounded to 16
 * significant bits (45426 / 2^16), so k * LN2_HI is exact for |k| < 2^8; the low
 * part is fl32(ln 2 - LN2_HI).  INV_LN2 is fl32(1 / ln 2). */
#define OR_LN2_HI 0x1.62e4p-1f
#define OR_LN2_LO 0x1.7f7d1cp-20f
#define OR_INV_LN2 0x1.715476p+0f

/* exp(a) for a in [-80, 80]: k = nearest integer to a / ln 2, r = a - k ln 2 in two
 * fused steps, p = sum_{n=0..7} r^n / n! with coefficients fl32(1/n!) by Horner's
 * rule in fused multiply-add, result p * 2^k (2^k built from exponent bits; exact
 * because the result stays a normal number). */
float oracle_exp_spec(float a) {
  float k = rintf(a * OR_INV_LN2);
  float r = fmaf(-k, OR_LN2_HI, a);
  r = fmaf(-k, OR_LN2_LO, r);
  float p = 0x1.a01a02p-13f;        /* 1/7! */
  p = fmaf(p, r, 0x1.6c16c2p-10f);  /* 1/6! */
  p = fmaf(p, r, 0x1.111112p-7f);   /* 1/5! */
  p = fmaf(p, r, 0x1.555556p-5f);   /* 1/4! */
  p = fmaf(p, r, 0x1.555556p-3f);   /* 1/3! */
  p = fmaf(p, r, 0.5f);             /* 1/2! */
  p = fmaf(p, r, 1.0f);             /* 1/1! */
  p = fmaf(p, r, 1.0f);             /* 1/0! */
  int ki = (int)k;
  return p * bits_to_f32((uint32_t)(ki + 127) << 23);
}

/* Token-expert affinity: sigmoid of the clamped logit ([mpbf] 2.2: V3 computes the
 * gating affinity with a sigmoid instead of softmax). */
float oracle_sigmoid(float z) {
  float zc = fminf(fmaxf(z, -80.0f), 80.0f);
  return 1.0f / (1.0f + oracle_exp_spec(-zc));
}

/* ------------------------------------------------------------------------- */
/* Threading helper: runs fn(ctx, i) for i in [0, n) split into contiguous     */
/* chunks.  Each output element is produced by one call with the same order of */
/* operations as a single-threaded run.                                        */
/* ------------------------------------------------------------------------- */

typedef void (*item_fn)(void* ctx, int64_t i);
typedef struct { item_fn fn; void* ctx; int64_t lo, hi; } chunk_arg;

static void* run_chunk(void* p) {
  chunk_arg* a = (chunk_arg*)p;
  for (int64_t i = a->lo; i < a->hi; ++i) a->fn(a->ctx, i);
  return NULL;
}

static void parallel_for(int64_t n, int nthreads, item_fn fn, void* ctx) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads == 1 || n < 2) {
    for (int64_t i = 0; i < n; ++i) fn(ctx, i);
    return;
  }
  pthread_t th[256];
  chunk_arg args[256];
  int64_t per = (n + nthreads - 1) / nthreads;
  int used = 0;
  for (int t = 0; t < nthreads; ++t) {
    int64_t lo = t * per, hi = lo + per < n ? lo + per : n;
    if (lo >= hi) break;
    args[t].fn = fn; args[t].ctx = ctx; args[t].lo = lo; args[t].hi = hi;
    if (pthread_create(&th[t], NULL, run_chunk, &args[t]) != 0) {
      run_chunk(&args[t]);
      th[t] = 0;
    }
    used = t + 1;
  }
  for (int t = 0; t < used; ++t)
    if (th[t]) pthread_join(th[t], NULL);
}

static float load_act(int dtype, const void* p, int64_t i) {
  if (dtype == DT_BF16) return oracle_bf16_to_f32(((const uint16_t*)p)[i]);
  return ((const float*)p)[i];
}

/* ------------------------------------------------------------------------- */
/* Router logits: z[t,e] = sum_h x[t,h] * W_r[e,h], fp32, sequential fma from +0 */
/* ------------------------------------------------------------------------- */

typedef struct {
  int64_t T; int H, E, x_dtype;
  const void* x; const float* w; float* z;
} logits_ctx;

static void logits_item(void* c, int64_t t) {
  logits_ctx* L = (logits_ctx*)c;
  for (int e = 0; e < L->E; ++e) {
    const float* w = L->w + (int64_t)e * L->H;
    float acc = 0.0f;
    for (int h = 0; h < L->H; ++h)
      acc = fmaf(load_act(L->x_dtype, L->x, t * L->H + h), w[h], acc);
    L->z[t * L->E + e] = acc;
  }
}

void oracle_router_logits(int64_t T, int H, int E, int x_dtype, const void* x,
                          const float* w_router, float* z, int nthreads) {
  logits_ctx c = {T, H, E, x_dtype, x, w_router, z};
  parallel_for(T, nthreads, logits_item, &c);
}

/* ------------------------------------------------------------------------- */
/* Selection ([mpbf] 2.2):                                                     */
/*   s = sigmoid(z); key = s + bias (the bias steers only the choice);          */
/*   group score = sum of the j largest keys in the group (node-limited routing */
/*   picks nodes by the summed affinity of their experts);                      */
/*   keep the M best groups; pick the K largest keys among their experts;       */
/*   gate = s / (sum of s over the K picked) -- from the unbiased affinity.     */
/* Orders are (value descending, index ascending), compared in fp32.            */
/* ------------------------------------------------------------------------- */

typedef struct { float v; int i; } vi_pair;

static int cmp_desc(const void* a, const void* b) {
  const vi_pair* x = (const vi_pair*)a;
  const vi_pair* y = (const vi_pair*)b;
  if (x->v > y->v) return -1;
  if (x->v < y->v) return 1;
  return (x->i > y->i) - (x->i < y->i);
}

typedef struct {
  int64_t T; int E, G, M, K, J;
  const float* z; const float* bias;
  int32_t* idx; float* gate;
} select_ctx;

static void select_item(void* c, int64_t t) {
  select_ctx* S = (select_ctx*)c;
  int E = S->E, G = S->G, gs = S->E / S->G;
  float* s = (float*)malloc(sizeof(float) * E);
  vi_pair* key = (vi_pair*)malloc(sizeof(vi_pair) * E);
  vi_pair* tmp = (vi_pair*)malloc(sizeof(vi_pair) * E);
  vi_pair* grp = (vi_pair*)malloc(sizeof(vi_pair) * G);
  char* kept = (char*)malloc(G);
  for (int e = 0; e < E; ++e) {
    s[e] = oracle_sigmoid(S->z[t * E + e]);
    key[e].v = s[e] + S->bias[e];
    key[e].i = e;
  }
  for (int g = 0; g < G; ++g) {
    memcpy(tmp, key + g * gs, sizeof(vi_pair) * gs);
    qsort(tmp, gs, sizeof(vi_pair), cmp_desc);
    float sc = 0.0f;
    for (int r = 0; r < S->J; ++r) sc = sc + tmp[r].v;
    grp[g].v = sc;
    grp[g].i = g;
  }
  qsort(grp, G, sizeof(vi_pair), cmp_desc);
  memset(kept, 0, G);
  for (int r = 0; r < S->M; ++r) kept[grp[r].i] = 1;
  int n = 0;
  for (int e = 0; e < E; ++e)
    if (kept[e / gs]) tmp[n++] = key[e];
  qsort(tmp, n, sizeof(vi_pair), cmp_desc);
  float sum = 0.0f;
  for (int k = 0; k < S->K; ++k) {
    S->idx[t * S->K + k] = tmp[k].i;
    sum = sum + s[tmp[k].i];
  }
  for (int k = 0; k < S->K; ++k) S->gate[t * S->K + k] = s[tmp[k].i] / sum;
  free(s); free(key); free(tmp); free(grp); free(kept);
}

/* Per-expert load over the whole batch: histogram of the chosen indices. */
void oracle_count(int64_t T, int E, int K, const int32_t* topk_idx, int32_t* counts) {
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t i = 0; i < T * K; ++i) counts[topk_idx[i]] += 1;
}

void oracle_select(int64_t T, int E, int G, int M, int K, int J, const float* z,
                   const float* bias, int32_t* topk_idx, float* topk_gate,
                   int32_t* counts, int nthreads) {
  select_ctx c = {T, E, G, M, K, J, z, bias, topk_idx, topk_gate};
  parallel_for(T, nthreads, select_item, &c);
  if (counts) oracle_count(T, E, K, topk_idx, counts);
}

/* Whole routing call: logits, selection and counts.  logits_out may be NULL. */
int oracle_route(int64_t T, int H, int E, int G, int M, int K, int J, int x_dtype,
                 const void* x, const float* w_router, const float* bias,
                 int32_t* topk_idx, float* topk_gate, int32_t* counts,
                 float* logits_out, int nthreads) {
  if (E % G || M < 1 || M > G || J < 1 || J > E / G || K < 1 || K > M * (E / G))
    return -1;
  float* z = logits_out ? logits_out : (float*)malloc(sizeof(float) * T * E);
  if (!z) return -2;
  oracle_router_logits(T, H, E, x_dtype, x, w_router, z, nthreads);
  oracle_select(T, E, G, M, K, J, z, bias, topk_idx, topk_gate, counts, nthreads);
  if (!logits_out) free(z);
  return 0;
}

/* ------------------------------------------------------------------------- */
/* FP8 quantisation ([mpbf] 3.1 and 4.3: scaling factors per small tile/block).  */
/* For each tile: amax = max |v|; scale = amax / 448 (fp32, IEEE division;     */
/* 1 when amax is 0); code = E4M3(v / scale) with the division in fp32.         */
/* ------------------------------------------------------------------------- */

/* Activations: one scale per (row, 128-column tile). */
void oracle_quantize_act_fp8(int64_t rows, int cols, int in_dtype, const void* in,
                             uint8_t* q, float* scale) {
  int nt = cols / 128;
  for (int64_t r = 0; r < rows; ++r)
    for (int c = 0; c < nt; ++c) {
      float amax = 0.0f;
      for (int i = 0; i < 128; ++i) {
        float v = fabsf(load_act(in_dtype, in, r * cols + c * 128 + i));
        if (v > amax) amax = v;
      }
      float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
      scale[r * nt + c] = sc;
      for (int i = 0; i < 128; ++i)
        q[r * cols + c * 128 + i] =
            oracle_e4m3_from_f32(load_act(in_dtype, in, r * cols + c * 128 + i) / sc);
    }
}

/* Weights: one scale per 128 x 128 block of a [rows, cols] bf16 matrix. */
void oracle_quantize_weight_fp8(int rows, int cols, const uint16_t* w, uint8_t* q,
                                float* scale) {
  int nbr = rows / 128, nbc = cols / 128;
  for (int br = 0; br < nbr; ++br)
    for (int bc = 0; bc < nbc; ++bc) {
      float amax = 0.0f;
      for (int i = 0; i < 128; ++i)
        for (int j = 0; j < 128; ++j) {
          float v = fabsf(oracle_bf16_to_f32(w[(int64_t)(br * 128 + i) * cols + bc * 128 + j]));
          if (v > amax) amax = v;
        }
      float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
      scale[br * nbc + bc] = sc;
      for (int i = 0; i < 128; ++i)
        for (int j = 0; j < 128; ++j) {
          int64_t o = (int64_t)(br * 128 + i) * cols + bc * 128 + j;
          q[o] = oracle_e4m3_from_f32(oracle_bf16_to_f32(w[o]) / sc);
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Permute (single-GPU form of the dispatch step): rows grouped by expert,      */
/* experts in index order, tokens ascending within an expert; the shared expert */
/* is the last group and takes every token in order.                            */
/* ------------------------------------------------------------------------- */

int oracle_permute(int64_t T, int H, int E, int K, int S, int x_dtype, const void* x,
                   const int32_t* topk_idx, const int32_t* counts, int32_t* offsets,
                   int32_t* sorted_token, int32_t* inv_perm, int out_dtype,
                   void* x_sorted, float* x_sorted_scale) {
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  if (offsets[E] != T * K) return -1;
  if (S) offsets[E + 1] = offsets[E] + (int32_t)T;
  int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * E);
  for (int e = 0; e < E; ++e) cursor[e] = offsets[e];
  for (int64_t t = 0; t < T; ++t)
    for (int k = 0; k < K; ++k) {
      int e = topk_idx[t * K + k];
      int32_t row = cursor[e]++;
      sorted_token[row] = (int32_t)t;
      inv_perm[t * K + k] = row;
    }
  free(cursor);
  int64_t R = (int64_t)T * K + (S ? T : 0);
  if (S)
    for (int64_t t = 0; t < T; ++t) sorted_token[T * K + t] = (int32_t)t;
  if (out_dtype == DT_E4M3) {
    /* quantise each token once; every copy of the row carries the same codes */
    int nt = H / 128;
    uint8_t* q = (uint8_t*)malloc((size_t)T * H);
    float* sc = (float*)malloc(sizeof(float) * T * nt);
    oracle_quantize_act_fp8(T, H, x_dtype, x, q, sc);
    for (int64_t r = 0; r < R; ++r) {
      int64_t t = sorted_token[r];
      memcpy((uint8_t*)x_sorted + r * H, q + t * H, H);
      memcpy(x_sorted_scale + r * nt, sc + t * nt, sizeof(float) * nt);
    }
    free(q); free(sc);
  } else {
    size_t es = out_dtype == DT_BF16 ? 2 : 4;
    if (out_dtype != x_dtype) return -1;
    for (int64_t r = 0; r < R; ++r)
      memcpy((char*)x_sorted + r * H * es, (const char*)x + (int64_t)sorted_token[r] * H * es,
             H * es);
  }
  return 0;
}

/* ------------------------------------------------------------------------- */
/* One expert's SwiGLU FFN on a block of rows ([mpbf] 2.2: each expert is an    */
/* FFN; the SwiGLU form and shared width follow the layer configuration):       */
/*   a_n = x . W13[n], u_n = x . W13[I+n], h_n = silu(a_n) u_n,                  */
/*   Y_m = h . W2[m].                                                            */
/* fp64 arithmetic; h and Y are rounded to the storage dtype.  For E4M3 the     */
/* dot products are sums over 128-wide blocks of (code x code) scaled by the    */
/* product of the two block scales, and h is quantised per (row, 128 columns).  */
/* ------------------------------------------------------------------------- */

static double dec(int dtype, const void* p, int64_t i) {
  if (dtype == DT_BF16) return oracle_bf16_to_f32(((const uint16_t*)p)[i]);
  if (dtype == DT_E4M3) return oracle_e4m3_to_f32(((const uint8_t*)p)[i]);
  return ((const float*)p)[i];
}

typedef struct {
  int H, I, dtype, out_dtype;
  const void* x; const float* x_scale;
  const void* w13; const float* w13_scale;
  const void* w2; const float* w2_scale;
  void* y;
  void* h_out; float* h_scale_out; /* optional copies of the stored h (NULL: not kept) */
} ffn_ctx;

static double dot_blocked(const ffn_ctx* F, const void* a, const float* a_scale, int64_t a_row,
                          const void* w, const float* w_scale, int64_t w_row, int len,
                          int w_cols_blocks) {
  if (F->dtype != DT_E4M3) {
    double acc = 0.0;
    for (int k = 0; k < len; ++k)
      acc += dec(F->dtype, a, a_row * len + k) * dec(F->dtype, w, w_row * len + k);
    return acc;
  }
  int nb = len / 128;
  double acc = 0.0;
  for (int b = 0; b < nb; ++b) {
    double part = 0.0; /* exact: at most 128 products of 4-bit-significand values */
    for (int k = b * 128; k < b * 128 + 128; ++k)
      part += dec(DT_E4M3, a, a_row * len + k) * dec(DT_E4M3, w, w_row * len + k);
    double sa = a_scale[a_row * nb + b];
    double sw = w_scale[(w_row / 128) * w_cols_blocks + b];
    acc += part * (sa * sw);
  }
  return acc;
}

static void ffn_item(void* c, int64_t r) {
  ffn_ctx* F = (ffn_ctx*)c;
  int H = F->H, I = F->I;
  double* h = (double*)malloc(sizeof(double) * I);
  for (int n = 0; n < I; ++n) {
    double a = dot_blocked(F, F->x, F->x_scale, r, F->w13, F->w13_scale, n, H, H / 128);
    double u = dot_blocked(F, F->x, F->x_scale, r, F->w13, F->w13_scale, I + n, H, H / 128);
    h[n] = a / (1.0 + exp(-a)) * u;
  }
  /* store h at the activation precision */
  void* hs;
  float* hscale = NULL;
  if (F->dtype == DT_E4M3) {
    float* hf = (float*)malloc(sizeof(float) * I);
    for (int n = 0; n < I; ++n) hf[n] = oracle_f32_from_f64(h[n]);
    hs = malloc(I);
    hscale = (float*)malloc(sizeof(float) * (I / 128));
    oracle_quantize_act_fp8(1, I, DT_F32, hf, (uint8_t*)hs, hscale);
    free(hf);
  } else if (F->dtype == DT_BF16) {
    hs = malloc(2 * (size_t)I);
    for (int n = 0; n < I; ++n) ((uint16_t*)hs)[n] = oracle_bf16_from_f64(h[n]);
  } else {
    hs = malloc(4 * (size_t)I);
    for (int n = 0; n < I; ++n) ((float*)hs)[n] = oracle_f32_from_f64(h[n]);
  }
  if (F->h_out) {
    const size_t es = F->dtype == DT_E4M3 ? 1 : (F->dtype == DT_BF16 ? 2 : 4);
    memcpy((char*)F->h_out + (size_t)r * I * es, hs, es * (size_t)I);
    if (hscale) memcpy(F->h_scale_out + r * (I / 128), hscale, sizeof(float) * (I / 128));
  }
  for (int m = 0; m < H; ++m) {
    double y = dot_blocked(F, hs, hscale, 0, F->w2, F->w2_scale, m, I, I / 128);
    if (F->out_dtype == DT_BF16) ((uint16_t*)F->y)[r * H + m] = oracle_bf16_from_f64(y);
    else ((float*)F->y)[r * H + m] = oracle_f32_from_f64(y);
  }
  free(h); free(hs); free(hscale);
}

/* rows: x [n_rows, H] (dtype; E4M3 with x_scale [n_rows, H/128]); w13 [2I, H];
 * w2 [H, I] (E4M3 with 128x128 block scales); y [n_rows, H] in out_dtype. */
int oracle_expert_ffn(int64_t n_rows, int H, int I, int dtype, const void* x,
                      const float* x_scale, const void* w13, const float* w13_scale,
                      const void* w2, const float* w2_scale, int out_dtype, void* y,
                      int nthreads) {
  if (dtype == DT_E4M3 && (H % 128 || I % 128)) return -1;
  ffn_ctx c = {H, I, dtype, out_dtype, x, x_scale, w13, w13_scale, w2, w2_scale, y, NULL, NULL};
  parallel_for(n_rows, nthreads, ffn_item, &c);
  return 0;
}

/* The same, also returning h as stored between the two GEMMs: h [n_rows, I] at the
 * activation dtype (E4M3 codes with h_scale [n_rows, I/128] for the FP8 path). */
int oracle_expert_ffn_h(int64_t n_rows, int H, int I, int dtype, const void* x,
                        const float* x_scale, const void* w13, const float* w13_scale,
                        const void* w2, const float* w2_scale, int out_dtype, void* y,
                        void* h, float* h_scale, int nthreads) {
  if (dtype == DT_E4M3 && (H % 128 || I % 128)) return -1;
  ffn_ctx c = {H, I, dtype, out_dtype, x, x_scale, w13, w13_scale, w2, w2_scale, y, h, h_scale};
  parallel_for(n_rows, nthreads, ffn_item, &c);
  return 0;
}

/* ------------------------------------------------------------------------- */
/* Combine ([resmic] 核心架构二: output = shared output + sum of gate-weighted    */
/* routed outputs): acc = 0; for k in rank order acc = fma(g, Y, acc); then    */
/* acc = Y_shared + acc (if a shared expert exists); round to the out dtype.   */
/* ------------------------------------------------------------------------- */

typedef struct {
  int64_t T; int H, K, S, dtype;
  const void* ys; const int32_t* inv_perm; const float* gate; void* y;
} combine_ctx;

static void combine_item(void* c, int64_t t) {
  combine_ctx* C = (combine_ctx*)c;
  for (int m = 0; m < C->H; ++m) {
    float acc = 0.0f;
    for (int k = 0; k < C->K; ++k) {
      int64_t row = C->inv_perm[t * C->K + k];
      acc = fmaf(C->gate[t * C->K + k], load_act(C->dtype, C->ys, row * C->H + m), acc);
    }
    if (C->S) acc = load_act(C->dtype, C->ys, (C->T * C->K + t) * C->H + m) + acc;
    if (C->dtype == DT_BF16) ((uint16_t*)C->y)[t * C->H + m] = oracle_bf16_from_f64(acc);
    else ((float*)C->y)[t * C->H + m] = acc;
  }
}

void oracle_combine(int64_t T, int H, int K, int S, int dtype, const void* y_sorted,
                    const int32_t* inv_perm, const float* topk_gate, void* y, int nthreads) {
  combine_ctx c = {T, H, K, S, dtype, y_sorted, inv_perm, topk_gate, y};
  parallel_for(T, nthreads, combine_item, &c);
}

/* ------------------------------------------------------------------------- */
/* Bias update ([mpbf] 2.2 and 6.2; [joto] item 1): once per step, an expert    */
/* whose share of the batch's routings exceeds the uniform share K/E gets its   */
/* bias lowered by gamma, one below it gets gamma added, equal is unchanged.    */
/* c/T > K/E  <=>  c*E > T*K, compared exactly in integers.                     */
/* ------------------------------------------------------------------------- */

void oracle_bias_update(int E, int64_t T, int K, const int32_t* counts, float gamma,
                        float* bias) {
  int64_t target = T * (int64_t)K;
  for (int e = 0; e < E; ++e) {
    int64_t load = (int64_t)counts[e] * E;
    if (load > target) bias[e] = bias[e] - gamma;
    else if (load < target) bias[e] = bias[e] + gamma;
  }
}

/* ------------------------------------------------------------------------- */
/* Sequence-wise load statistic [mpbf section 2.2: next to the bias rule, a     */
/* sequence-level balance term with a very small weight keeps any one sequence  */
/* from extreme imbalance.  The pages give that term no formula, so only the    */
/* loads it would be built from are computed: per (sequence, expert) counts of  */
/* the chosen indices, and per sequence the largest and smallest count, the     */
/* number of experts with no token, and max / mean, the mean being the uniform  */
/* share L*K/E of the sequence's L tokens].                                     */
/* Sequence s holds tokens seq_off[s] .. seq_off[s+1]-1 (seq_off nondecreasing, */
/* seq_off[0] = 0, seq_off[n_seq] = T).  ratio = (float)(max*E) / (float)(L*K), */
/* one IEEE division of two exactly converted integers (below 2^24); 0 when the */
/* sequence is empty.                                                           */
/* ------------------------------------------------------------------------- */

void oracle_seq_load_stats(int64_t T, int E, int K, const int32_t* topk_idx, int n_seq,
                           const int32_t* seq_off, int32_t* counts, int32_t* stats,
                           float* ratio) {
  (void)T;
  for (int s = 0; s < n_seq; ++s) {
    int32_t* c = counts + (int64_t)s * E;
    for (int e = 0; e < E; ++e) c[e] = 0;
    for (int64_t t = seq_off[s]; t < seq_off[s + 1]; ++t)
      for (int k = 0; k < K; ++k) c[topk_idx[t * K + k]] += 1;
    int32_t mx = c[0], mn = c[0], zeros = 0;
    for (int e = 0; e < E; ++e) {
      if (c[e] > mx) mx = c[e];
      if (c[e] < mn) mn = c[e];
      if (c[e] == 0) zeros += 1;
    }
    stats[s * 3 + 0] = mx;
    stats[s * 3 + 1] = mn;
    stats[s * 3 + 2] = zeros;
    const int64_t L = (int64_t)seq_off[s + 1] - seq_off[s];
    ratio[s] = L > 0 ? (float)((int64_t)mx * E) / (float)(L * K) : 0.0f;
  }
}

/* ------------------------------------------------------------------------- */
/* Array forms of the scalar routines (for tests that sweep many values).     */
/* ------------------------------------------------------------------------- */

void oracle_exp_spec_array(int64_t n, const float* a, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_exp_spec(a[i]);
}
void oracle_sigmoid_array(int64_t n, const float* z, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_sigmoid(z[i]);
}
void oracle_e4m3_from_f32_array(int64_t n, const float* v, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_from_f32(v[i]);
}
void oracle_bf16_from_f64_array(int64_t n, const double* v, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_from_f64(v[i]);
}

/* ========================================================================= */
/* Backward of the layer (the derivative of the forward above; the pages only  */
/* say that gradients accumulate in higher precision, that the block's input   */
/* and weight gradients are separate computations, and -- [resmic] 核心架构三 -- */
/* that the routing bias takes no part in back-propagation).  fp64 arithmetic; */
/* a tensor is rounded where the layer stores it: the expert-output gradient   */
/* dY and the SwiGLU-input gradient [da|du] at the activation dtype (they feed  */
/* the grouped GEMMs), the permuted input gradient at the activation dtype,    */
/* the input gradient dx at the activation dtype, weight gradients in fp32.    */
/* ========================================================================= */

/* v rounded to the activation dtype (round to nearest even) and widened again */
static double act_round(int dtype, double v) {
  if (dtype == DT_BF16) return oracle_bf16_to_f32(oracle_bf16_from_f64(v));
  return oracle_f32_from_f64(v);
}

static void store_act(int dtype, void* p, int64_t i, double v) {
  if (dtype == DT_BF16) ((uint16_t*)p)[i] = oracle_bf16_from_f64(v);
  else ((float*)p)[i] = oracle_f32_from_f64(v);
}

/* Combine backward: y[t] = Y_S[t] + sum_k g[t,k] Y[row(t,k)], so
 *   dY[row(t,k)] = g[t,k] * dy[t],  dY[T*K + t] = dy[t]  (shared expert),
 *   dg[t,k]      = <dy[t], Y[row(t,k)]>.                                        */
typedef struct {
  int64_t T; int H, K, S, dtype;
  const void* dy; const void* ys; const int32_t* inv_perm; const float* gate;
  void* dys; float* dgate;
} combine_bwd_ctx;

static void combine_bwd_item(void* c, int64_t t) {
  combine_bwd_ctx* C = (combine_bwd_ctx*)c;
  int H = C->H;
  for (int k = 0; k < C->K; ++k) {
    int64_t row = C->inv_perm[t * C->K + k];
    if (row < 0) { C->dgate[t * C->K + k] = 0.0f; continue; }
    double g = C->gate[t * C->K + k], dot = 0.0;
    for (int m = 0; m < H; ++m) {
      double d = load_act(C->dtype, C->dy, t * H + m);
      dot += d * load_act(C->dtype, C->ys, row * H + m);
      store_act(C->dtype, C->dys, row * H + m, g * d);
    }
    C->dgate[t * C->K + k] = oracle_f32_from_f64(dot);
  }
  if (C->S)
    for (int m = 0; m < H; ++m)
      store_act(C->dtype, C->dys, (C->T * C->K + t) * H + m,
                load_act(C->dtype, C->dy, t * H + m));
}

void oracle_combine_backward(int64_t T, int H, int K, int S, int dtype, const void* dy,
                             const void* y_sorted, const int32_t* inv_perm,
                             const float* topk_gate, void* dy_sorted, float* dgate,
                             int nthreads) {
  combine_bwd_ctx c = {T, H, K, S, dtype, dy, y_sorted, inv_perm, topk_gate, dy_sorted, dgate};
  parallel_for(T, nthreads, combine_bwd_item, &c);
}

/* Gate and router backward.  g_k = s_k / S with S = sum_j s_j over the chosen
 * experts ([mpbf] 2.2: selected scores renormalised), s = sigmoid(clamp(z, +-80)):
 *   ds_j = (dg_j - sum_k g_k dg_k) / S,   dz_j = ds_j s_j (1 - s_j)  (0 if |z| > 80),
 *   dx_r[t] = sum_j dz_j W_r[e_j],        dW_r[e] = sum over (t,j) with e_j = e of dz_j x[t].
 * The bias only chose the experts: it has no gradient and does not enter here.   */
typedef struct {
  int64_t T; int H, E, K, dtype;
  const void* x; const float* wr; const float* z; const int32_t* idx; const float* gate;
  const float* dgate; float* dz; float* dxr;
} router_bwd_ctx;

static void router_bwd_item(void* c, int64_t t) {
  router_bwd_ctx* R = (router_bwd_ctx*)c;
  int K = R->K, H = R->H;
  double S = 0.0, gd = 0.0;
  double s[32];
  for (int k = 0; k < K; ++k) {
    int e = R->idx[t * K + k];
    s[k] = oracle_sigmoid(R->z[t * R->E + e]);
    S += s[k];
    gd += (double)R->gate[t * K + k] * R->dgate[t * K + k];
  }
  for (int k = 0; k < K; ++k) {
    int e = R->idx[t * K + k];
    float zz = R->z[t * R->E + e];
    double ds = (R->dgate[t * K + k] - gd) / S;
    double dz = (zz > 80.0f || zz < -80.0f) ? 0.0 : ds * s[k] * (1.0 - s[k]);
    R->dz[t * K + k] = oracle_f32_from_f64(dz);
  }
  for (int m = 0; m < H; ++m) {
    double acc = 0.0;
    for (int k = 0; k < K; ++k)
      acc += (double)R->dz[t * K + k] * R->wr[(int64_t)R->idx[t * K + k] * H + m];
    R->dxr[t * H + m] = oracle_f32_from_f64(acc);
  }
}

typedef struct {
  int64_t T; int H, E, K, dtype;
  const void* x; const int32_t* idx; const float* dz; float* dwr;
} router_wgrad_ctx;

static void router_wgrad_item(void* c, int64_t e) {
  router_wgrad_ctx* W = (router_wgrad_ctx*)c;
  int H = W->H;
  double* acc = (double*)calloc(H, sizeof(double));
  for (int64_t t = 0; t < W->T; ++t)
    for (int k = 0; k < W->K; ++k)
      if (W->idx[t * W->K + k] == e) {
        double d = W->dz[t * W->K + k];
        for (int m = 0; m < H; ++m) acc[m] += d * load_act(W->dtype, W->x, t * H + m);
      }
  for (int m = 0; m < H; ++m) W->dwr[e * H + m] = oracle_f32_from_f64(acc[m]);
  free(acc);
}

/* x [T,H] act; w_router [E,H] f32; logits [T,E] f32; topk_idx/gate/dgate [T,K];
 * out: dz [T,K] f32, dx_router [T,H] f32, dw_router [E,H] f32.  K <= 32. */
int oracle_router_backward(int64_t T, int H, int E, int K, int dtype, const void* x,
                           const float* w_router, const float* logits, const int32_t* topk_idx,
                           const float* topk_gate, const float* dgate, float* dz,
                           float* dx_router, float* dw_router, int nthreads) {
  if (K > 32) return -1;
  router_bwd_ctx c = {T, H, E, K, dtype, x, w_router, logits, topk_idx, topk_gate, dgate, dz,
                      dx_router};
  parallel_for(T, nthreads, router_bwd_item, &c);
  router_wgrad_ctx w = {T, H, E, K, dtype, x, topk_idx, dz, dw_router};
  parallel_for(E, nthreads, router_wgrad_item, &w);
  return 0;
}

/* Expert FFN backward for the n rows of one group (x rows, dY rows; w13 [2I,H],
 * w2 [H,I] of that expert):  a = x W1^T, u = x W3^T, h = silu(a) u (stored at the
 * act dtype as in the forward; a and u are also kept at the act dtype, and the
 * backward works from those kept values),
 *   dh  = dY W2,                  da = dh u silu'(a),  du = dh silu(a)  -> [da|du] stored,
 *   dx  = [da|du] W13             (stored at the act dtype),
 *   dW2 = dY^T h,  dW13 = [da|du]^T x   (fp32).
 * silu(a) = a sigma(a), silu'(a) = sigma(a) (1 + a (1 - sigma(a))).                 */
typedef struct {
  int H, I, dtype;
  const void* x; const void* w13; const void* w2; const void* dy;
  void* hs; void* dau; void* dx;
} ebwd_ctx;

static void ebwd_row_item(void* c, int64_t r) {
  ebwd_ctx* B = (ebwd_ctx*)c;
  int H = B->H, I = B->I, dt = B->dtype;
  for (int n = 0; n < I; ++n) {
    double a = 0.0, u = 0.0, dh = 0.0;
    for (int k = 0; k < H; ++k) {
      double xv = dec(dt, B->x, r * H + k);
      a += xv * dec(dt, B->w13, (int64_t)n * H + k);
      u += xv * dec(dt, B->w13, (int64_t)(I + n) * H + k);
    }
    for (int m = 0; m < H; ++m)
      dh += dec(dt, B->dy, r * H + m) * dec(dt, B->w2, (int64_t)m * I + n);
    double sg = 1.0 / (1.0 + exp(-a));
    store_act(dt, B->hs, r * I + n, a * sg * u);
    /* the forward keeps a and u for the backward at the activation dtype */
    const double ar = act_round(dt, a), ur = act_round(dt, u);
    double sr = 1.0 / (1.0 + exp(-ar));
    store_act(dt, B->dau, r * 2 * I + n, dh * ur * sr * (1.0 + ar * (1.0 - sr)));
    store_act(dt, B->dau, r * 2 * I + I + n, dh * ar * sr);
  }
  for (int k = 0; k < H; ++k) {
    double acc = 0.0;
    for (int j = 0; j < 2 * I; ++j)
      acc += dec(dt, B->dau, r * 2 * I + j) * dec(dt, B->w13, (int64_t)j * H + k);
    store_act(dt, B->dx, r * H + k, acc);
  }
}

typedef struct {
  int64_t n; int H, I, dtype;
  const void* x; const void* dy; const void* hs; const void* dau;
  float* dw13; float* dw2;
} ewgrad_ctx;

/* item j < 2I: row j of dW13; item 2I + m: row m of dW2 */
static void ewgrad_item(void* c, int64_t j) {
  ewgrad_ctx* W = (ewgrad_ctx*)c;
  int H = W->H, I = W->I, dt = W->dtype;
  if (j < 2 * I) {
    for (int k = 0; k < H; ++k) {
      double acc = 0.0;
      for (int64_t r = 0; r < W->n; ++r)
        acc += dec(dt, W->dau, r * 2 * I + j) * dec(dt, W->x, r * H + k);
      W->dw13[j * H + k] = oracle_f32_from_f64(acc);
    }
  } else {
    int64_t m = j - 2 * I;
    for (int n = 0; n < I; ++n) {
      double acc = 0.0;
      for (int64_t r = 0; r < W->n; ++r)
        acc += dec(dt, W->dy, r * H + m) * dec(dt, W->hs, r * I + n);
      W->dw2[m * I + n] = oracle_f32_from_f64(acc);
    }
  }
}

/* x [n,H], dy [n,H] act (F32 or BF16); w13 [2I,H], w2 [H,I] act;
 * out: h [n,I] act, dau [n,2I] act, dx [n,H] act, dw13 [2I,H] f32, dw2 [H,I] f32. */
int oracle_expert_backward(int64_t n, int H, int I, int dtype, const void* x, const void* w13,
                           const void* w2, const void* dy, void* h, void* dau, void* dx,
                           float* dw13, float* dw2, int nthreads) {
  if (dtype == DT_E4M3) return -1;
  ebwd_ctx b = {H, I, dtype, x, w13, w2, dy, h, dau, dx};
  parallel_for(n, nthreads, ebwd_row_item, &b);
  if (!dw13 && !dw2) return 0; /* input part only */
  ewgrad_ctx w = {n, H, I, dtype, x, dy, h, dau, dw13, dw2};
  parallel_for(2 * I + H, nthreads, ewgrad_item, &w);
  return 0;
}

/* Input gradient: dx[t] = dx_router[t] + sum_k dx_sorted[row(t,k)] + dx_sorted[T*K+t]
 * (the last term if a shared expert exists), summed in fp64, rounded to the act dtype. */
typedef struct {
  int64_t T; int H, K, S, dtype;
  const void* dxs; const int32_t* inv_perm; const float* dxr; void* dx;
} unperm_ctx;

static void unperm_item(void* c, int64_t t) {
  unperm_ctx* U = (unperm_ctx*)c;
  for (int m = 0; m < U->H; ++m) {
    double acc = U->dxr ? U->dxr[t * U->H + m] : 0.0;
    for (int k = 0; k < U->K; ++k) {
      int64_t row = U->inv_perm[t * U->K + k];
      if (row >= 0) acc += load_act(U->dtype, U->dxs, row * U->H + m);
    }
    if (U->S) acc += load_act(U->dtype, U->dxs, (U->T * U->K + t) * U->H + m);
    store_act(U->dtype, U->dx, t * U->H + m, acc);
  }
}

void oracle_unpermute_sum(int64_t T, int H, int K, int S, int dtype, const void* dx_sorted,
                          const int32_t* inv_perm, const float* dx_router, void* dx,
                          int nthreads) {
  unperm_ctx c = {T, H, K, S, dtype, dx_sorted, inv_perm, dx_router, dx};
  parallel_for(T, nthreads, unperm_item, &c);
}
