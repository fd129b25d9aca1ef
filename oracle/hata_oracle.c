/*
 * hata_oracle.c -- plain, slow CPU oracle for the HATA decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test-suite, the package smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * constant with the HIP library.
 *
 * Source of every step: the paper notes on "HATA: Trainable and
 * Hardware-Efficient Hash-Aware Top-k Attention for Scalable Large Model
 * Inference" (ACL 2025, arXiv 2506.02572), section "Key design", subsections
 * "Learning-to-Hash modelling" (the hash function h(x) = 2*Sigmoid(sigma*x*W_H)-1,
 * one W_H per head) and "Decode-stage algorithm" (HashEncode = matmul + Sign +
 * BitPack; append the key code; Hamming distance as bitcount of xor; GQA
 * aggregation of the query heads sharing a KV cache; top-k, gather, sparse
 * attention), and section "Overall framework" (phase 3: exact attention over
 * the selected KV pairs only).
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository):
 *   - inference hash = sign(x W_H): for sigma > 0 the sigmoid relaxation and
 *     the sign agree in sign, so sigma drops out;
 *   - bit = 1 iff the fp32 projection compares >= 0.0f (so -0.0 -> 1, NaN -> 0);
 *   - column c of the projection is bit (c mod 64) of 64-bit word c/64; a
 *     code of r bits takes ceil(r/64) words, bits r..63 of the last word zero
 *     (r = 32 keeps one 64-bit word per row);
 *   - one W_H per KV head, shared by its G query heads and by q and k;
 *     W_H is stored [d][r] and a row vector x is projected as x * W_H;
 *   - query head j belongs to KV head j / G;
 *   - GQA aggregation is the SUM of the G Hamming distances;
 *   - top-k keeps the k smallest summed distances, ties to the lower token
 *     index; when k >= n every token is kept; the kept set is reported in
 *     ascending token order, padded with -1;
 *   - attention: z_i = scale * <q, K_i>, softmax over the kept set only,
 *     output rounded to fp32.
 *
 * Arithmetic: the projection accumulates in fp32 in increasing input index,
 * one rounded product and one rounded add per term (build with
 * -ffp-contract=off); the attention runs in fp64.  popcount is a plain loop;
 * top-k is a full sort (qsort) of (score, index) pairs.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
static float bf16_to_float(uint16_t h) {
  uint32_t u = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* HashEncode of `rows` rows of length d: p = x * W (fp32), bit = (p >= 0),
 * packed LSB-first into r/64 words per row.  `proj` (nullable) receives p. */
void oracle_encode_rows(const uint16_t* x, int64_t rows, int d, const float* W,
                        int r, uint64_t* codes, float* proj) {
  const int words = (r + 63) / 64;
  for (int64_t row = 0; row < rows; ++row) {
    const uint16_t* xr = x + row * (int64_t)d;
    uint64_t* cr = codes + row * (int64_t)words;
    for (int w = 0; w < words; ++w) cr[w] = 0;
    for (int c = 0; c < r; ++c) {
      float acc = 0.0f;
      for (int i = 0; i < d; ++i) {
        float prod = bf16_to_float(xr[i]) * W[(int64_t)i * r + c];
        acc = acc + prod;
      }
      if (proj) proj[row * (int64_t)r + c] = acc;
      if (acc >= 0.0f) cr[c / 64] |= ((uint64_t)1) << (c % 64);
    }
  }
}

/* Number of set bits, by clearing the lowest set bit until none is left. */
static int popcount64(uint64_t v) {
  int n = 0;
  while (v) {
    v &= v - 1;
    ++n;
  }
  return n;
}

int oracle_popcount64(uint64_t v) { return popcount64(v); }

/* S[i] = sum over the G query codes of popcount(q_g XOR code_i), i < n. */
void oracle_hamming_gqa(const uint64_t* qcodes, int G, const uint64_t* kcodes,
                        int64_t n, int words, int32_t* S) {
  for (int64_t i = 0; i < n; ++i) {
    int32_t s = 0;
    for (int g = 0; g < G; ++g)
      for (int w = 0; w < words; ++w)
        s += popcount64(qcodes[g * words + w] ^ kcodes[i * words + w]);
    S[i] = s;
  }
}

typedef struct {
  int32_t s;
  int32_t i;
} score_pair;

static int cmp_pair(const void* a, const void* b) {
  const score_pair* x = (const score_pair*)a;
  const score_pair* y = (const score_pair*)b;
  if (x->s != y->s) return x->s < y->s ? -1 : 1;
  if (x->i != y->i) return x->i < y->i ? -1 : 1;
  return 0;
}

static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* idx[0:min(k,n)] = ascending token ids of the first min(k,n) entries of the
 * (score, id)-ascending order; idx[min(k,n):k] = -1.  Returns min(k,n), or -1
 * on allocation failure. */
int oracle_topk(const int32_t* S, int64_t n, int k, int32_t* idx) {
  score_pair* p = (score_pair*)malloc((size_t)(n > 0 ? n : 1) * sizeof *p);
  if (!p) return -1;
  for (int64_t i = 0; i < n; ++i) {
    p[i].s = S[i];
    p[i].i = (int32_t)i;
  }
  qsort(p, (size_t)n, sizeof *p, cmp_pair);
  int m = (int64_t)k < n ? k : (int)n;
  for (int j = 0; j < m; ++j) idx[j] = p[j].i;
  qsort(idx, (size_t)m, sizeof *idx, cmp_i32);
  for (int j = m; j < k; ++j) idx[j] = -1;
  free(p);
  return m;
}

/* Softmax attention of G query rows over the m rows K[idx[j]], V[idx[j]]
 * (entries < 0 are skipped), in fp64; out[g][c] rounded to fp32.
 * K and V point at the first row of one (sequence, KV head). */
void oracle_attention(const uint16_t* q, int G, const uint16_t* K,
                      const uint16_t* V, const int32_t* idx, int m, int d,
                      float scale, float* out) {
  double* z = (double*)malloc((size_t)(m > 0 ? m : 1) * sizeof *z);
  double* acc = (double*)malloc((size_t)d * sizeof *acc);
  for (int g = 0; g < G; ++g) {
    const uint16_t* qg = q + (int64_t)g * d;
    double zmax = -INFINITY;
    int any = 0;
    for (int j = 0; j < m; ++j) {
      if (idx[j] < 0) continue;
      const uint16_t* kr = K + (int64_t)idx[j] * d;
      double dot = 0.0;
      for (int c = 0; c < d; ++c)
        dot += (double)bf16_to_float(qg[c]) * (double)bf16_to_float(kr[c]);
      z[j] = (double)scale * dot;
      if (!any || z[j] > zmax) zmax = z[j];
      any = 1;
    }
    for (int c = 0; c < d; ++c) acc[c] = 0.0;
    double denom = 0.0;
    for (int j = 0; j < m; ++j) {
      if (idx[j] < 0) continue;
      double w = exp(z[j] - zmax);
      denom += w;
      const uint16_t* vr = V + (int64_t)idx[j] * d;
      for (int c = 0; c < d; ++c) acc[c] += w * (double)bf16_to_float(vr[c]);
    }
    for (int c = 0; c < d; ++c)
      out[(int64_t)g * d + c] = any ? (float)(acc[c] / denom) : 0.0f;
  }
  free(z);
  free(acc);
}

/* One whole decode step for every unit (b, h):
 *   1. encode the G query rows q[b, hG:(h+1)G] with W[h];
 *   2. encode K[b,h,n_b-1] and append it as codes[b,h,n_b-1];
 *   3. S_i = sum_g popcount(qcode_g XOR codes[b,h,i]), i < n_b;
 *   4. top-k of S (ties to lower index), ascending ids -> idx_out[b,h,:];
 *   5. fp64 softmax attention of each query head over the kept rows.
 * Layouts: q [B][Hq][d] bf16; K, V [B][Hkv][cap][d] bf16; W [Hkv][d][r];
 * codes [B][Hkv][cap][r/64] (rows < n_b-1 valid on entry); seq_lens [B]
 * (host); out [B][Hq][d] fp32; idx_out [B][Hkv][k].
 * Wk (nullable, same layout as W): a separate key encoder, used in step 2
 * instead of W (independent query and key encoders, as described on the
 * HashAttention summary page, "Approach"); NULL means W encodes both.
 * Nullable extras: scores_out [B][Hkv][cap] (rows < n_b written), qcodes_out
 * [B][Hq][r/64].  nthreads <= 0 means "all available" (OpenMP over units).
 * Returns 0, or -1 on bad arguments. */
int oracle_decode_step(const uint16_t* q, const uint16_t* K, const uint16_t* V,
                       const float* W, const float* Wk, uint64_t* codes, int B, int Hq, int Hkv,
                       int d, int r, int64_t cap, const int32_t* seq_lens,
                       int k, float scale, float* out, int32_t* idx_out,
                       int32_t* scores_out, uint64_t* qcodes_out,
                       int nthreads) {
  if (B < 1 || Hkv < 1 || Hq % Hkv != 0 || r < 1 || d < 1 || k < 1)
    return -1;
  for (int b = 0; b < B; ++b)
    if (seq_lens[b] < 1 || seq_lens[b] > cap) return -1;
  const int G = Hq / Hkv;
  const int words = (r + 63) / 64;
  const int units = B * Hkv;
  int bad = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
#endif
  for (int u = 0; u < units; ++u) {
    const int b = u / Hkv, h = u % Hkv;
    const int64_t n = seq_lens[b];
    const int64_t base = ((int64_t)b * Hkv + h) * cap;
    const float* Wh = W + (int64_t)h * d * r;
    const float* Wkh = (Wk ? Wk : W) + (int64_t)h * d * r;
    uint64_t* qc = (uint64_t*)malloc((size_t)G * words * sizeof *qc);
    int32_t* S = (int32_t*)malloc((size_t)n * sizeof *S);
    int32_t* idx = idx_out + (int64_t)u * k;
    if (!qc || !S) {
      bad = 1;
      free(qc);
      free(S);
      continue;
    }
    const uint16_t* qrows = q + ((int64_t)b * Hq + (int64_t)h * G) * d;
    oracle_encode_rows(qrows, G, d, Wh, r, qc, NULL);
    oracle_encode_rows(K + (base + n - 1) * d, 1, d, Wkh, r,
                       codes + (base + n - 1) * words, NULL);
    oracle_hamming_gqa(qc, G, codes + base * words, n, words, S);
    int m = oracle_topk(S, n, k, idx);
    if (m < 0) bad = 1;
    oracle_attention(qrows, G, K + base * d, V + base * d, idx, m < 0 ? 0 : m,
                     d, scale, out + ((int64_t)b * Hq + (int64_t)h * G) * d);
    if (scores_out)
      for (int64_t i = 0; i < n; ++i) scores_out[base + i] = S[i];
    if (qcodes_out)
      memcpy(qcodes_out + ((int64_t)b * Hq + (int64_t)h * G) * words, qc,
             (size_t)G * words * sizeof *qc);
    free(qc);
    free(S);
  }
  return bad ? -1 : 0;
}

/* Dense attention over all n_b rows of every unit (the k = n case of step 5). */
int oracle_dense_attention(const uint16_t* q, const uint16_t* K,
                           const uint16_t* V, int B, int Hq, int Hkv, int d,
                           int64_t cap, const int32_t* seq_lens, float scale,
                           float* out, int nthreads) {
  if (B < 1 || Hkv < 1 || Hq % Hkv != 0) return -1;
  const int G = Hq / Hkv;
  const int units = B * Hkv;
  int bad = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
#endif
  for (int u = 0; u < units; ++u) {
    const int b = u / Hkv, h = u % Hkv;
    const int64_t n = seq_lens[b];
    const int64_t base = ((int64_t)b * Hkv + h) * cap;
    int32_t* idx = (int32_t*)malloc((size_t)(n > 0 ? n : 1) * sizeof *idx);
    if (!idx) {
      bad = 1;
      continue;
    }
    for (int64_t i = 0; i < n; ++i) idx[i] = (int32_t)i;
    const uint16_t* qrows = q + ((int64_t)b * Hq + (int64_t)h * G) * d;
    oracle_attention(qrows, G, K + base * d, V + base * d, idx, (int)n, d,
                     scale, out + ((int64_t)b * Hq + (int64_t)h * G) * d);
    free(idx);
  }
  return bad ? -1 : 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
