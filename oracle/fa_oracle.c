/*
 * fa_oracle.c -- TEST INFRASTRUCTURE ONLY: the plain, slow fp64 CPU oracle of the
 * FlashAttention forward pass.  Only tests/, the smoke check and the bench's CPU
 * baseline may load it; the product path never does.  It shares no code, header or
 * table with the GPU library.
 *
 * What it computes (one query row at a time, textbook "mask -> softmax -> matmul"):
 *   "FlashAttention forward in C" (tinyllm L9.3), section 2.1 "What is computed":
 *     o_i = sum_{j in V_i} e^{s_ij} v_j / (sum_{j in V_i} e^{s_ij} + e^{z_h}),
 *     V_i = { j < Tk : (causal == 0 or j <= p_i) and (w <= 0 or j > p_i - w) },
 *     p_i = q_offset + i, head h reads KV head floor(h / (H / Hkv)),
 *     lse_i = log(sum_{j in V_i} e^{s_ij} + e^{z_h}); the sink term only with sinks;
 *     a row with no visible key and no sink gives o = 0 and lse = -inf.
 *   "Fused attention and softmax: fast and exact" (OneModel), "What is computed":
 *     the score is scale * q.k plus an optional additive mask [qLen, kLen] with free
 *     strides (a stride of 0 broadcasts).
 *   "IV.5: Flash attention", "The reference implementation": the materialised
 *     per-head reference (scores, mask, softmax, scores @ V) that flash must match.
 *   Score variants named by the candle page ("KV 缓存与注意力", attention/: the CPU flash
 *   attention's variants with ALiBi and softcap), in their usual definitions:
 *     softcap c > 0: the logit scale * q.k becomes c * tanh(scale * q.k / c);
 *     ALiBi slopes m_h: the score gets -m_h * |p_i - j| (the distance between the
 *     absolute positions of query and key);
 *     s_ij = [softcap](scale * q.k) - m_h |p_i - j| + mask_ij.
 * Readings where the pages leave a step open:
 *   - the mask is indexed by (row i of this call, key j), like q;
 *   - a mask entry of -inf makes the key invisible (it counts toward "no visible key");
 *   - the sink logit z_h is raw (not multiplied by scale), one per query head;
 *   - inputs are widened exactly from fp32 (or bf16 bits) to fp64; all arithmetic fp64;
 *   - softcap applies to the dot-product logit only; the ALiBi bias and the mask are added
 *     after it; ALiBi uses absolute positions (p_i = q_offset + i) and |p_i - j| for keys on
 *     either side (without causal).
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (see oracle/build.py).
 * Compile-time ORACLE_MUTANT=n plants one deliberate mistake; tests use those builds to
 * show that the pins catch each mistake.  The normal build defines none.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

enum { ORC_F64 = 0, ORC_F32 = 1, ORC_BF16 = 2 };

/* Exact widening of one input element to fp64. */
static double orc_load(const void *base, int dtype, int64_t idx) {
  if (dtype == ORC_F64) return ((const double *)base)[idx];
  if (dtype == ORC_F32) return (double)((const float *)base)[idx];
  uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16; /* bf16 = top half of fp32 */
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Key j visible to absolute position p (tinyllm section 2.1, the set V_i). */
static int orc_visible(int64_t j, int64_t p, int causal, int64_t window) {
#if ORACLE_MUTANT == 4 /* causal as j < p: a token cannot see itself */
  int causal_ok = !causal || j < p;
#else
  int causal_ok = !causal || j <= p;
#endif
#if ORACLE_MUTANT == 5 /* a window of w + 1 keys */
  int window_ok = window <= 0 || j >= p - window;
#else
  int window_ok = window <= 0 || j > p - window;
#endif
  return causal_ok && window_ok;
}

/*
 * orc_attention: computes o and lse for a list of query rows.
 *   q [B,Hq,Tq,d], k and v [B,Hkv,Tk,d] with element strides {b, h, t} and the d axis
 *   contiguous; all three in dtype (ORC_F64 / ORC_F32 / ORC_BF16 bits).
 *   sinks [Hq] fp32 or NULL; mask fp32 or NULL, element strides {b, h, i, j}.
 *   softcap: c > 0 caps the logit, 0 = none; alibi [Hq] fp32 slopes or NULL.
 *   rows: nrows triples (b, h, i), or NULL for every row in (b, h, i) order.
 *   Outputs are compact: o_out[r * d + x], lse_out[r] for the r-th listed row.
 * Returns 0, or -1 if Hq % Hkv != 0 or an argument is out of range.
 */
int orc_attention(const void *q, const int64_t *sq, const void *k, const int64_t *sk,
                  const void *v, const int64_t *sv, int dtype, int64_t B, int64_t Hq,
                  int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d, double scale,
                  int64_t q_offset, int causal, int64_t window, const float *sinks,
                  const float *mask, const int64_t *smask, double softcap, const float *alibi,
                  const int64_t *rows, int64_t nrows, double *o_out, double *lse_out) {
  if (B < 0 || Hq < 0 || Hkv <= 0 || Tq < 0 || Tk < 0 || d <= 0 || Hq % Hkv != 0) return -1;
  const int64_t total = rows ? nrows : B * Hq * Tq;
  const int64_t group = Hq / Hkv;
  int bad = 0;

#pragma omp parallel
  {
    double *s = (double *)malloc((size_t)(Tk > 0 ? Tk : 1) * sizeof(double));
    if (!s) {
#pragma omp atomic write
      bad = 1;
    }
#pragma omp for schedule(dynamic, 4)
    for (int64_t r = 0; r < total; ++r) {
      if (!s) continue;
      int64_t b, h, i;
      if (rows) {
        b = rows[3 * r]; h = rows[3 * r + 1]; i = rows[3 * r + 2];
      } else {
        b = r / (Hq * Tq); h = (r / Tq) % Hq; i = r % Tq;
      }
      double *o = o_out + r * d;
      if (b < 0 || b >= B || h < 0 || h >= Hq || i < 0 || i >= Tq) {
#pragma omp atomic write
        bad = 1;
        continue;
      }
#if ORACLE_MUTANT == 3 /* round-robin GQA */
      const int64_t hk = h % Hkv;
#else
      const int64_t hk = h / group;
#endif
#if ORACLE_MUTANT == 6 /* q_offset ignored */
      const int64_t p = i;
#else
      const int64_t p = q_offset + i;
#endif
      const void *qrow_base = q;
      const int64_t qoff = b * sq[0] + h * sq[1] + i * sq[2];

      /* 1. scores of the visible keys; invisible keys are -inf (the materialised mask) */
      double mx = -INFINITY;
      for (int64_t j = 0; j < Tk; ++j) {
        if (!orc_visible(j, p, causal, window)) { s[j] = -INFINITY; continue; }
        const int64_t koff = b * sk[0] + hk * sk[1] + j * sk[2];
        double dot = 0.0;
#if ORACLE_MUTANT == 10 /* a dropped term: the last head-dim element */
        for (int64_t x = 0; x + 1 < d; ++x)
#else
        for (int64_t x = 0; x < d; ++x)
#endif
          dot += orc_load(qrow_base, dtype, qoff + x) * orc_load(k, dtype, koff + x);
#if ORACLE_MUTANT == 11 /* scale dropped */
        double sc = dot;
#else
        double sc = scale * dot;
#endif
#if ORACLE_MUTANT != 19
        if (softcap > 0.0) {
#if ORACLE_MUTANT == 16 /* softcap without its outer factor */
          sc = tanh(sc / softcap);
#else
          sc = softcap * tanh(sc / softcap);
#endif
        }
#endif
        if (alibi) {
#if ORACLE_MUTANT == 17 /* ALiBi bias added with the wrong sign */
          sc += (double)alibi[h] * fabs((double)(p - j));
#elif ORACLE_MUTANT == 18 /* ALiBi distance from the call's row index, not the position */
          sc -= (double)alibi[h] * fabs((double)(i - j));
#else
          sc -= (double)alibi[h] * fabs((double)(p - j));
#endif
        }
        if (mask) {
#if ORACLE_MUTANT == 12 /* mask indexed by absolute position instead of the call's row */
          sc += (double)mask[b * smask[0] + h * smask[1] + p * smask[2] + j * smask[3]];
#elif ORACLE_MUTANT == 13 /* mask subtracted */
          sc -= (double)mask[b * smask[0] + h * smask[1] + i * smask[2] + j * smask[3]];
#else
          sc += (double)mask[b * smask[0] + h * smask[1] + i * smask[2] + j * smask[3]];
#endif
        }
#if ORACLE_MUTANT == 19 /* softcap applied after the bias and the mask */
        if (softcap > 0.0) sc = softcap * tanh(sc / softcap);
#endif
        s[j] = sc;
        if (sc > mx) mx = sc;
      }

      /* 2. softmax over the visible keys (plus the sink), then the weighted sum of V */
      const int has_sink = sinks != NULL;
      const double z = has_sink ? (double)sinks[h] : -INFINITY;
      if (has_sink && z > mx) mx = z;
      if (mx == -INFINITY) {
        /* no visible key and no sink: no distribution */
        for (int64_t x = 0; x < d; ++x) o[x] = 0.0;
#if ORACLE_MUTANT == 9 /* divide by l = 0 */
        for (int64_t x = 0; x < d; ++x) o[x] = 0.0 / 0.0;
#endif
        lse_out[r] = -INFINITY;
        continue;
      }
      double den = 0.0;
      for (int64_t x = 0; x < d; ++x) o[x] = 0.0;
      for (int64_t j = 0; j < Tk; ++j) {
        if (s[j] == -INFINITY) continue;
#if ORACLE_MUTANT == 14 /* wrong sign in the exponent */
        const double e = exp(mx - s[j]);
#else
        const double e = exp(s[j] - mx);
#endif
        den += e;
        const int64_t voff = b * sv[0] + hk * sv[1] + j * sv[2];
        for (int64_t x = 0; x < d; ++x) {
#if ORACLE_MUTANT == 15 /* transposed value operand: v[x][j] read as v[j][x] swapped */
          o[x] += e * orc_load(v, dtype, b * sv[0] + hk * sv[1] + (x % Tk) * sv[2] + (j % d));
#else
          o[x] += e * orc_load(v, dtype, voff + x);
#endif
        }
      }
#if ORACLE_MUTANT != 7 /* mutant 7: sink left out of the denominator */
      if (has_sink) den += exp(z - mx);
#endif
      for (int64_t x = 0; x < d; ++x) o[x] /= den;
#if ORACLE_MUTANT == 8 /* lse without the maximum */
      lse_out[r] = log(den);
#else
      lse_out[r] = mx + log(den);
#endif
    }
    free(s);
  }
  return bad ? -1 : 0;
}

/* Thread control for the OpenMP row loop (host-side timing of the oracle). */
void orc_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Number of visible (query, key) pairs of one (b, h): sum_i |V_i| (mask not counted). */
int64_t orc_visible_pairs(int64_t Tq, int64_t Tk, int64_t q_offset, int causal, int64_t window) {
  int64_t n = 0;
  for (int64_t i = 0; i < Tq; ++i)
    for (int64_t j = 0; j < Tk; ++j) n += orc_visible(j, q_offset + i, causal, window);
  return n;
}
