/*
 * oracle.c -- plain, slow, fp64 CPU oracle of one paged-KV decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the package smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant
 * generator with the HIP library; it reads the same documented input formats.
 *
 * What it computes, per row r (sequence s, position p, input x), and where
 * that comes from:
 *   - storage formats: bfloat16 (round-to-nearest-even, as the KV storage of
 *     "GPU inference engine engineering", section "The same bits in any
 *     batch") and OCP E4M3 for the fp8 tier ("Engines for the card you have",
 *     section "One checkpoint, many engines": fp8 weights and fp8 KV cache
 *     with calibrated scales).  Both are written here from the format
 *     definitions with frexp/ldexp arithmetic, not from bit tricks.
 *   - projections: a naive matvec over the stored weight values ("llm-rs",
 *     section 2: decode reads every weight once to form one vector).
 *   - rows: each row carries its own sequence and position; all appends of a
 *     step precede all attention reads ("GPU inference engine engineering",
 *     section "Batching without running out of cache").
 *   - attention: softmax(q K^T / sqrt(d)) V over positions 0..p with KV held
 *     contiguously per sequence, in fp64 with the maximum subtracted.  The
 *     GPU's online softmax over pages ("Building an LLM runtime from scratch
 *     on NVIDIA H100", section "Bug #1") reaches this same value up to
 *     rounding, so the oracle is the plain definition.
 *   - FFN: silu(W_gate h) * (W_up h), gate/up fused as in "llm-rs" section 3;
 *     residuals h = x + W_o attn and y = h + W_down a.
 *   - optional RMSNorm before attention and before the FFN, gains folded into
 *     W_qkv and W_gate_up ("llm-rs", section 4, third lesson), and optional
 *     rotary positions on q and k (a reading: the pages never describe them).
 * Readings where the pages are silent (softmax scale, GQA mapping, rounding
 * points, residual form, fp8 activation scaling) are listed with the build's
 * design notes; each is marked where it is used below.
 *
 * Built with: gcc -O2 -fopenmp -shared -fPIC oracle.c -o liboracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8 = 2 };

int orc_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Storage formats                                                           */
/* ------------------------------------------------------------------------ */

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits;
 * exponent field 0 = zero/subnormal (fraction x 2^-133), 255 = inf/NaN. */
double orc_bf16_value(uint16_t code) {
  int sign = (code >> 15) & 1;
  int e = (code >> 7) & 0xFF;
  int f = code & 0x7F;
  double v;
  if (e == 0xFF) v = f ? NAN : INFINITY;
  else if (e == 0) v = ldexp((double)f, -133);
  else v = ldexp(1.0 + f / 128.0, e - 127);
  return sign ? -v : v;
}

/* OCP E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 fraction bits, no
 * infinities; S.1111.111 is NaN, so the largest magnitude is 1.75 x 2^8 = 448;
 * exponent field 0 = subnormal (fraction x 2^-9). */
double orc_e4m3_value(uint8_t code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 3) & 0xF;
  int f = code & 0x7;
  double v;
  if (e == 0xF && f == 0x7) v = NAN;
  else if (e == 0) v = ldexp((double)f, -9);
  else v = ldexp(1.0 + f / 8.0, e - 7);
  return sign ? -v : v;
}

/* Rounds |a| (finite, > 0) to the nearest value with `mbits` fraction bits
 * and minimum normal exponent `emin`, ties to even (rint in the default
 * rounding mode).  Returns the rounded magnitude; it may exceed the format's
 * largest finite value, which the caller handles. */
static double round_magnitude(double a, int mbits, int emin) {
  int k;
  frexp(a, &k);           /* a = m 2^k, m in [0.5, 1) */
  int e = k - 1;          /* a in [2^e, 2^(e+1)) */
  if (e < emin) e = emin; /* subnormal range: fixed quantum */
  double quantum = ldexp(1.0, e - mbits);
  return rint(a / quantum) * quantum;
}

uint16_t orc_bf16_round(double x) {
  if (isnan(x)) return signbit(x) ? 0xFFC0 : 0x7FC0;
  int sign = signbit(x) ? 1 : 0;
  double a = fabs(x);
  uint16_t s = (uint16_t)(sign << 15);
  if (a == 0.0) return s;
  if (isinf(a)) return s | 0x7F80;
  double r = round_magnitude(a, 7, -126);
  double maxf = ldexp(2.0 - ldexp(1.0, -7), 127);
  if (r > maxf) return s | 0x7F80; /* rounds past the largest finite: infinity */
  if (r == 0.0) return s;
  int k;
  frexp(r, &k);
  int e = k - 1;
  if (e < -126) { /* subnormal: r = f x 2^-133 */
    int f = (int)ldexp(r, 133);
    return s | (uint16_t)f;
  }
  int f = (int)((ldexp(r, -e) - 1.0) * 128.0);
  return s | (uint16_t)((e + 127) << 7) | (uint16_t)f;
}

/* Round to nearest even, saturating to +-448 (infinities too); NaN -> NaN. */
uint8_t orc_e4m3_round_sat(double x) {
  int sign = signbit(x) ? 1 : 0;
  uint8_t s = (uint8_t)(sign << 7);
  if (isnan(x)) return s | 0x7F;
  double a = fabs(x);
  if (a == 0.0) return s;
  if (isinf(a)) return s | 0x7E;
  double r = round_magnitude(a, 3, -6);
  if (r > 448.0) r = 448.0;
  if (r == 0.0) return s;
  int k;
  frexp(r, &k);
  int e = k - 1;
  if (e < -6) {
    int f = (int)ldexp(r, 9);
    return s | (uint8_t)f;
  }
  int f = (int)((ldexp(r, -e) - 1.0) * 8.0);
  return s | (uint8_t)((e + 7) << 3) | (uint8_t)f;
}

void orc_bf16_round_array(const double* x, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_round(x[i]);
}
void orc_bf16_value_array(const uint16_t* c, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_value(c[i]);
}
void orc_e4m3_round_array(const double* x, uint8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_round_sat(x[i]);
}
void orc_e4m3_value_array(const uint8_t* c, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_value(c[i]);
}

/* Value of element i of a stored array of `dtype` codes (no scale). */
static double code_value(const void* base, int dtype, int64_t i) {
  switch (dtype) {
    case ORC_F32: return (double)((const float*)base)[i];
    case ORC_BF16: return orc_bf16_value(((const uint16_t*)base)[i]);
    default: return orc_e4m3_value(((const uint8_t*)base)[i]);
  }
}

static int elem_size(int dtype) { return dtype == ORC_F32 ? 4 : dtype == ORC_BF16 ? 2 : 1; }

/* Rounds a value to the activation storage dtype (f32 or bf16), returning
 * the stored value. */
static double round_act(double v, int act_dtype) {
  if (act_dtype == ORC_F32) return (double)(float)v;
  return orc_bf16_value(orc_bf16_round(v));
}

/* Per-row fp8 quantisation of a projection input (fp8 MFMA tier; reading:
 * dynamic per-row scale s = fp32(max |z|) / 448 in fp32, codes = E4M3 RNE of
 * z / s in fp32; s = 1 for an all-zero row). */
void orc_act_quant(const double* z, int64_t n, uint8_t* codes, float* scale_out) {
  float amax = 0.0f;
  for (int64_t i = 0; i < n; ++i) {
    float a = fabsf((float)z[i]);
    if (a > amax) amax = a;
  }
  float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  for (int64_t i = 0; i < n; ++i) {
    float q = (float)z[i] / s;
    codes[i] = orc_e4m3_round_sat((double)q);
  }
  *scale_out = s;
}

/* ------------------------------------------------------------------------ */
/* Matrix-vector products                                                    */
/* ------------------------------------------------------------------------ */

/* Y[r][j] = sum_k (W[j][k] * scale) * X[r][k] for r < n, j < rows. */
void orc_matvec_rows(int dtype, const void* W, double scale, int rows, int cols,
                     const double* X, int n, double* Y) {
#pragma omp parallel for schedule(static)
  for (int j = 0; j < rows; ++j) {
    for (int r = 0; r < n; ++r) {
      double acc = 0.0;
      for (int k = 0; k < cols; ++k)
        acc += code_value(W, dtype, (int64_t)j * cols + k) * scale * X[(int64_t)r * cols + k];
      Y[(int64_t)r * rows + j] = acc;
    }
  }
}

/* Logits for a per-row candidate list only ("GPU inference engine
 * engineering": headline figure "Grammar-bounded output" and section "The
 * whole decode loop on the GPU": the output layer is evaluated for the rows
 * that can be emitted next, not for the whole vocabulary).  For r < n and
 * c < clamp(n_cand[r], 0, max_cand): j = cand[r][c];
 *   Y[r][c] = sum_k (W[j][k] * scale) * X[r][k]   if 0 <= j < rows,
 *   Y[r][c] = NaN                                  otherwise.
 * Entries at c >= the clamped count are left as the caller filled them. */
void orc_matvec_gathered(int dtype, const void* W, double scale, int rows, int cols,
                         const double* X, int n, const int32_t* cand, int max_cand,
                         const int32_t* n_cand, double* Y) {
#pragma omp parallel for schedule(static)
  for (int r = 0; r < n; ++r) {
    int cnt = n_cand[r];
    if (cnt < 0) cnt = 0;
    if (cnt > max_cand) cnt = max_cand;
    for (int c = 0; c < cnt; ++c) {
      int j = cand[(int64_t)r * max_cand + c];
      double acc = NAN;
      if (j >= 0 && j < rows) {
        acc = 0.0;
        for (int k = 0; k < cols; ++k)
          acc += code_value(W, dtype, (int64_t)j * cols + k) * scale * X[(int64_t)r * cols + k];
      }
      Y[(int64_t)r * max_cand + c] = acc;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Pool layout (read side), written from the documented layout of the ABI    */
/* ------------------------------------------------------------------------ */

static int64_t k_position(int t, int c, int d, int dtype) {
  int E = 16 / elem_size(dtype);
  int64_t vec = ((int64_t)(t / 16) * (d / E) + c / E) * 16 + t % 16;
  return vec * E + c % E;
}

static int64_t v_position(int t, int c, int d, int dtype) {
  int a = t / 16, b = (t % 16) / 4, i = t % 4;
  int64_t vec;
  int el, E;
  if (dtype == ORC_F32) {
    E = 4; vec = ((int64_t)(a * (d / 16) + c / 16) * 4 + b) * 16 + c % 16; el = i;
  } else if (dtype == ORC_BF16) {
    E = 8; vec = ((int64_t)(c / 16) * 4 + b) * 16 + c % 16; el = 4 * a + i;
  } else {
    E = 16; vec = ((int64_t)(c / 32) * 4 + b) * 16 + c % 16; el = 8 * ((c / 16) % 2) + 4 * a + i;
  }
  return vec * E + el;
}

/* Copies the first `len` positions of a sequence out of a host copy of the
 * pool's page region into contiguous [len][n_kv][d] code arrays. */
int orc_gather_history(const uint8_t* pages, int n_kv, int d, int kv_dtype,
                       const int32_t* table_row, int n_table, int len,
                       uint8_t* k_out, uint8_t* v_out) {
  int es = elem_size(kv_dtype);
  int64_t block_bytes = (int64_t)32 * d * es;
  for (int t = 0; t < len; ++t) {
    int lp = t / 32, slot = t % 32;
    if (lp >= n_table) return -1;
    int page = table_row[lp];
    if (page < 0) return -1;
    for (int g = 0; g < n_kv; ++g) {
      const uint8_t* kb = pages + ((int64_t)page * n_kv + g) * 2 * block_bytes;
      const uint8_t* vb = kb + block_bytes;
      for (int c = 0; c < d; ++c) {
        int64_t dst = (((int64_t)t * n_kv + g) * d + c) * es;
        memcpy(k_out + dst, kb + k_position(slot, c, d, kv_dtype) * es, es);
        memcpy(v_out + dst, vb + v_position(slot, c, d, kv_dtype) * es, es);
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Attention over contiguous per-sequence KV                                 */
/* ------------------------------------------------------------------------ */

typedef struct {
  int32_t n_q, n_kv, head_dim;
  int32_t kv_dtype;
  float k_scale, v_scale;
} orc_attn_geom;

typedef struct {
  int32_t n_seqs;
  const int64_t* hist_off; /* [n_seqs] first token of each sequence in k/v */
  const int32_t* hist_len; /* [n_seqs] */
  const void* k;           /* [total][n_kv][d] codes of kv_dtype */
  const void* v;
} orc_history;

/* Contiguous fp64 KV of one sequence, positions [0, cap). */
typedef struct {
  int cap;
  double* k; /* [cap][n_kv][d] */
  double* v;
  uint8_t* filled;
} seq_cache;

static void free_caches(seq_cache* c, int n) {
  if (!c) return;
  for (int i = 0; i < n; ++i) { free(c[i].k); free(c[i].v); free(c[i].filled); }
  free(c);
}

/* Builds caches for the sequences the rows touch: history decoded (code x
 * scale) into fp64.  Returns NULL on a bad row or allocation failure. */
static seq_cache* build_caches(const orc_attn_geom* G, const orc_history* H, int n_rows,
                               const int32_t* seq, const int32_t* pos) {
  seq_cache* c = (seq_cache*)calloc((size_t)H->n_seqs, sizeof(seq_cache));
  if (!c) return NULL;
  for (int r = 0; r < n_rows; ++r) {
    if (seq[r] < 0 || seq[r] >= H->n_seqs || pos[r] < 0) { free_caches(c, H->n_seqs); return NULL; }
    int need = pos[r] + 1;
    if (need > c[seq[r]].cap) c[seq[r]].cap = need;
  }
  int nkd = G->n_kv * G->head_dim;
  for (int s = 0; s < H->n_seqs; ++s) {
    if (c[s].cap == 0) continue;
    int cap = c[s].cap > H->hist_len[s] ? c[s].cap : H->hist_len[s];
    c[s].cap = cap;
    c[s].k = (double*)calloc((size_t)cap * nkd, sizeof(double));
    c[s].v = (double*)calloc((size_t)cap * nkd, sizeof(double));
    c[s].filled = (uint8_t*)calloc((size_t)cap, 1);
    if (!c[s].k || !c[s].v || !c[s].filled) { free_caches(c, H->n_seqs); return NULL; }
    for (int t = 0; t < H->hist_len[s]; ++t) {
      int64_t src = (H->hist_off[s] + t) * nkd;
      for (int i = 0; i < nkd; ++i) {
        c[s].k[(int64_t)t * nkd + i] = code_value(H->k, G->kv_dtype, src + i) * (double)G->k_scale;
        c[s].v[(int64_t)t * nkd + i] = code_value(H->v, G->kv_dtype, src + i) * (double)G->v_scale;
      }
      c[s].filled[t] = 1;
    }
  }
  return c;
}

/* Stores one value of the row's own key or value in the KV dtype (reading:
 * f32 and bf16 unchanged from the act-dtype value; fp8 = E4M3 RNE of
 * value / scale, the division in fp32, saturating). */
static double kv_store(double v, int kv_dtype, float scale) {
  if (kv_dtype == ORC_F32) return (double)(float)v;
  if (kv_dtype == ORC_BF16) return orc_bf16_value(orc_bf16_round(v));
  float q = (float)v / scale;
  return orc_e4m3_value(orc_e4m3_round_sat((double)q)) * (double)scale;
}

/* out[h][c] for one row: softmax over t in [0, p] of (q_h . K_t)/sqrt(d),
 * applied to V_t; q head h reads kv head h / (n_q / n_kv) (reading). */
static void attend(const orc_attn_geom* G, const seq_cache* sc, int p, const double* q,
                   int h, double* out) {
  int d = G->head_dim, grp = G->n_q / G->n_kv, g = h / grp;
  int nkd = G->n_kv * d;
  double* sc_t = (double*)malloc(sizeof(double) * (size_t)(p + 1));
  double m = -INFINITY;
  for (int t = 0; t <= p; ++t) {
    double dot = 0.0;
    for (int c = 0; c < d; ++c) dot += q[(int64_t)h * d + c] * sc->k[(int64_t)t * nkd + g * d + c];
    sc_t[t] = dot / sqrt((double)d);
    if (sc_t[t] > m) m = sc_t[t];
  }
  double l = 0.0;
  for (int t = 0; t <= p; ++t) { sc_t[t] = exp(sc_t[t] - m); l += sc_t[t]; }
  for (int c = 0; c < d; ++c) {
    double o = 0.0;
    for (int t = 0; t <= p; ++t) o += sc_t[t] * sc->v[(int64_t)t * nkd + g * d + c];
    out[(int64_t)h * d + c] = o / l;
  }
  free(sc_t);
}

/* Appends each row's key/value (if given), then attends every row.
 * q_val [n][n_q][d] fp64 (already the stored values), kv_new [n][n_kv][d]
 * fp64 or NULL.  Returns 0, or -1 for a bad row / gap in a sequence / OOM. */
static int attention_core(const orc_attn_geom* G, const orc_history* H, int n_rows,
                          const int32_t* seq, const int32_t* pos, const double* q_val,
                          const double* k_new, const double* v_new, double* out) {
  seq_cache* c = build_caches(G, H, n_rows, seq, pos);
  if (!c) return -1;
  int nkd = G->n_kv * G->head_dim;
  if (k_new && v_new) {
    for (int r = 0; r < n_rows; ++r) { /* every append precedes every read */
      seq_cache* s = &c[seq[r]];
      for (int i = 0; i < nkd; ++i) {
        s->k[(int64_t)pos[r] * nkd + i] = kv_store(k_new[(int64_t)r * nkd + i], G->kv_dtype, G->k_scale);
        s->v[(int64_t)pos[r] * nkd + i] = kv_store(v_new[(int64_t)r * nkd + i], G->kv_dtype, G->v_scale);
      }
      s->filled[pos[r]] = 1;
    }
  }
  for (int r = 0; r < n_rows; ++r)
    for (int t = 0; t <= pos[r]; ++t)
      if (!c[seq[r]].filled[t]) { free_caches(c, H->n_seqs); return -1; }
  int total = n_rows * G->n_q;
#pragma omp parallel for schedule(dynamic, 1)
  for (int i = 0; i < total; ++i) {
    int r = i / G->n_q, h = i % G->n_q;
    attend(G, &c[seq[r]], pos[r], q_val + (int64_t)r * G->n_q * G->head_dim, h,
           out + (int64_t)r * G->n_q * G->head_dim);
  }
  free_caches(c, H->n_seqs);
  return 0;
}

/* Attention-only entry: q (and k_new/v_new, may be NULL) are stored codes of
 * q_dtype (f32 or bf16), shapes [n][n_q][d] and [n][n_kv][d]. */
int orc_attention(const orc_attn_geom* G, const orc_history* H, int n_rows, const int32_t* seq,
                  const int32_t* pos, int q_dtype, const void* q, const void* k_new,
                  const void* v_new, double* out) {
  int64_t nq = (int64_t)n_rows * G->n_q * G->head_dim;
  int64_t nk = (int64_t)n_rows * G->n_kv * G->head_dim;
  double* qv = (double*)malloc(sizeof(double) * (size_t)(nq > 0 ? nq : 1));
  double* kv = k_new ? (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1)) : NULL;
  double* vv = v_new ? (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1)) : NULL;
  if (!qv || (k_new && !kv) || (v_new && !vv)) { free(qv); free(kv); free(vv); return -1; }
  for (int64_t i = 0; i < nq; ++i) qv[i] = code_value(q, q_dtype, i);
  for (int64_t i = 0; kv && i < nk; ++i) kv[i] = code_value(k_new, q_dtype, i);
  for (int64_t i = 0; vv && i < nk; ++i) vv[i] = code_value(v_new, q_dtype, i);
  int rc = attention_core(G, H, n_rows, seq, pos, qv, kv, vv, out);
  free(qv); free(kv); free(vv);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Norm factor and rotary positions (the steps on either side of the path)   */
/* ------------------------------------------------------------------------ */

/* RMSNorm's per-row factor 1 / sqrt(mean_k z[k]^2 + eps).  The norm's gain is
 * folded into the following projection's weights, so at step time only this
 * scalar remains, applied to the projection's outputs ("llm-rs", section 4,
 * third lesson: norms folded into the projections). */
double orc_inv_rms(const double* z, int cols, double eps) {
  double ss = 0.0;
  for (int k = 0; k < cols; ++k) ss += z[k] * z[k];
  return 1.0 / sqrt(ss / cols + eps);
}

void orc_inv_rms_rows(const double* Z, int n, int cols, double eps, double* out) {
  for (int r = 0; r < n; ++r) out[r] = orc_inv_rms(Z + (int64_t)r * cols, cols, eps);
}

/* Rotary position embedding (reading; the pages are silent): within each head
 * of width hd, the consecutive pair (v[2i], v[2i+1]) is rotated by the angle
 * pos * base^(-2i / hd):
 *   v[2i]   <- v[2i] cos - v[2i+1] sin,   v[2i+1] <- v[2i] sin + v[2i+1] cos. */
void orc_rope(double* v, int n_heads, int hd, int pos, double base) {
  for (int i = 0; i < hd / 2; ++i) {
    double theta = (double)pos * pow(base, -2.0 * i / hd);
    double c = cos(theta), sn = sin(theta);
    for (int h = 0; h < n_heads; ++h) {
      double* e = v + (int64_t)h * hd + 2 * i;
      double a = e[0], b = e[1];
      e[0] = a * c - b * sn;
      e[1] = a * sn + b * c;
    }
  }
}

void orc_rope_rows(double* V, int n, int n_heads, int hd, const int32_t* pos, double base) {
  for (int r = 0; r < n; ++r) orc_rope(V + (int64_t)r * n_heads * hd, n_heads, hd, pos[r], base);
}

/* ------------------------------------------------------------------------ */
/* One decode step of one layer                                              */
/* ------------------------------------------------------------------------ */

typedef struct {
  int32_t hidden, n_q, n_kv, head_dim, ffn;
  int32_t w_dtype;
  const void *w_qkv, *w_o, *w_gu, *w_d; /* stored codes, row-major [out][in] */
  double s_qkv, s_o, s_gu, s_d;         /* per-tensor scales (1 unless fp8) */
  int32_t act_dtype;                    /* ORC_F32 or ORC_BF16 */
  int32_t act_fp8;                      /* 1: projection inputs quantised per row to fp8 */
  int32_t kv_dtype;
  float k_scale, v_scale;
  int32_t flags;      /* ORC_NORM: RMSNorm before attention and FFN; ORC_ROPE: rotate q, k */
  double norm_eps;    /* RMSNorm epsilon */
  double rope_base;   /* RoPE base */
} orc_layer;

enum { ORC_NORM = 1, ORC_ROPE = 2 };

typedef struct {
  double *qkv, *attn, *h, *a, *y; /* [n][...] outputs, any may be NULL */
  /* the stored stages before their rounding to the activation dtype: the
   * exact value of each stage given the stored values of the one before */
  double *qkv_raw, *attn_raw, *a_raw;
} orc_outputs;

/* Projection of n input rows Z [n][cols] by W: the input is first taken in
 * the activation dtype (reading: every projection input is the activation
 * dtype), or quantised per row to fp8 in the fp8 matrix-core tier. */
static int project(const orc_layer* L, const void* W, double ws, int rows, int cols,
                   const double* Z, int n, double* Y) {
  double* in = (double*)malloc(sizeof(double) * (size_t)n * cols);
  double* sz = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  uint8_t* codes = (uint8_t*)malloc((size_t)cols);
  if (!in || !sz || !codes) { free(in); free(sz); free(codes); return -1; }
  for (int r = 0; r < n; ++r) {
    const double* z = Z + (int64_t)r * cols;
    double* o = in + (int64_t)r * cols;
    if (L->act_fp8) {
      float s;
      orc_act_quant(z, cols, codes, &s);
      for (int k = 0; k < cols; ++k) o[k] = orc_e4m3_value(codes[k]);
      sz[r] = (double)s;
    } else {
      for (int k = 0; k < cols; ++k) o[k] = round_act(z[k], L->act_dtype);
      sz[r] = 1.0;
    }
  }
  orc_matvec_rows(L->w_dtype, W, ws, rows, cols, in, n, Y);
  for (int r = 0; r < n; ++r)
    for (int j = 0; j < rows; ++j) Y[(int64_t)r * rows + j] *= sz[r];
  free(in); free(sz); free(codes);
  return 0;
}

int orc_decode_step(const orc_layer* L, const orc_history* H, int n, const int32_t* seq,
                    const int32_t* pos, const float* x, orc_outputs* out) {
  int D = L->hidden, d = L->head_dim, nq = L->n_q, nkv = L->n_kv, F = L->ffn;
  int nqkv = (nq + 2 * nkv) * d;
  int rc = -1;
  double *xd = NULL, *qkv = NULL, *qv = NULL, *kv = NULL, *vv = NULL, *att = NULL, *ao = NULL,
         *h = NULL, *gu = NULL, *a = NULL, *dn = NULL;
  size_t nn = (size_t)(n > 0 ? n : 1);
  xd = (double*)malloc(sizeof(double) * nn * D);
  qkv = (double*)malloc(sizeof(double) * nn * nqkv);
  qv = (double*)malloc(sizeof(double) * nn * nq * d);
  kv = (double*)malloc(sizeof(double) * nn * nkv * d);
  vv = (double*)malloc(sizeof(double) * nn * nkv * d);
  att = (double*)malloc(sizeof(double) * nn * nq * d);
  ao = (double*)malloc(sizeof(double) * nn * D);
  h = (double*)malloc(sizeof(double) * nn * D);
  if (!xd || !qkv || !qv || !kv || !vv || !att || !ao || !h) goto done;
  for (int64_t i = 0; i < (int64_t)n * D; ++i) xd[i] = (double)x[i];

  /* qkv = W_qkv x, stored in the activation dtype.  With the norm, W_qkv
   * carries the pre-attention gain and the outputs are scaled by the row's
   * 1/rms(x); with RoPE, the q and k heads are rotated by the row's position
   * before the rounding. */
  if (project(L, L->w_qkv, L->s_qkv, nqkv, D, xd, n, qkv)) goto done;
  for (int r = 0; r < n; ++r) {
    double* row = qkv + (int64_t)r * nqkv;
    if (L->flags & ORC_NORM) {
      double f = orc_inv_rms(xd + (int64_t)r * D, D, L->norm_eps);
      for (int j = 0; j < nqkv; ++j) row[j] *= f;
    }
    if (L->flags & ORC_ROPE) orc_rope(row, nq + nkv, d, pos[r], L->rope_base);
  }
  if (out && out->qkv_raw) memcpy(out->qkv_raw, qkv, sizeof(double) * n * nqkv);
  for (int64_t i = 0; i < (int64_t)n * nqkv; ++i) qkv[i] = round_act(qkv[i], L->act_dtype);
  for (int r = 0; r < n; ++r) {
    const double* row = qkv + (int64_t)r * nqkv;
    memcpy(qv + (int64_t)r * nq * d, row, sizeof(double) * nq * d);
    memcpy(kv + (int64_t)r * nkv * d, row + nq * d, sizeof(double) * nkv * d);
    memcpy(vv + (int64_t)r * nkv * d, row + (nq + nkv) * d, sizeof(double) * nkv * d);
  }
  if (out && out->qkv) memcpy(out->qkv, qkv, sizeof(double) * n * nqkv);

  /* append every row, then attend every row */
  orc_attn_geom G = {nq, nkv, d, L->kv_dtype, L->k_scale, L->v_scale};
  if (attention_core(&G, H, n, seq, pos, qv, kv, vv, att)) goto done;
  if (out && out->attn_raw) memcpy(out->attn_raw, att, sizeof(double) * n * nq * d);
  for (int64_t i = 0; i < (int64_t)n * nq * d; ++i) att[i] = round_act(att[i], L->act_dtype);
  if (out && out->attn) memcpy(out->attn, att, sizeof(double) * n * nq * d);

  /* h = x + W_o attn (residual stream unrounded) */
  if (project(L, L->w_o, L->s_o, D, nq * d, att, n, ao)) goto done;
  for (int64_t i = 0; i < (int64_t)n * D; ++i) h[i] = xd[i] + ao[i];
  if (out && out->h) memcpy(out->h, h, sizeof(double) * n * D);

  if (F > 0) {
    gu = (double*)malloc(sizeof(double) * nn * 2 * F);
    a = (double*)malloc(sizeof(double) * nn * F);
    dn = (double*)malloc(sizeof(double) * nn * D);
    if (!gu || !a || !dn) goto done;
    if (project(L, L->w_gu, L->s_gu, 2 * F, D, h, n, gu)) goto done;
    for (int r = 0; r < n; ++r) {
      /* pre-FFN norm: gain in W_gate_up, 1/rms(h) on both halves before silu */
      double f = (L->flags & ORC_NORM) ? orc_inv_rms(h + (int64_t)r * D, D, L->norm_eps) : 1.0;
      for (int j = 0; j < F; ++j) {
        double g = gu[(int64_t)r * 2 * F + j] * f, u = gu[(int64_t)r * 2 * F + F + j] * f;
        double v = g / (1.0 + exp(-g)) * u;
        if (out && out->a_raw) out->a_raw[(int64_t)r * F + j] = v;
        a[(int64_t)r * F + j] = round_act(v, L->act_dtype);
      }
    }
    if (out && out->a) memcpy(out->a, a, sizeof(double) * n * F);
    if (project(L, L->w_d, L->s_d, D, F, a, n, dn)) goto done;
    if (out && out->y)
      for (int64_t i = 0; i < (int64_t)n * D; ++i) out->y[i] = h[i] + dn[i];
  } else if (out && out->y) {
    memcpy(out->y, h, sizeof(double) * n * D);
  }
  rc = 0;
done:
  free(xd); free(qkv); free(qv); free(kv); free(vv); free(att); free(ao); free(h);
  free(gu); free(a); free(dn);
  return rc;
}
