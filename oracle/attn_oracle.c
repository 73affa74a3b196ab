/*
 * attn_oracle.c -- plain fp64 CPU oracle for causal prefill attention.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call
 * this file: only the tests, the package smoke check and the benchmark's CPU
 * baseline leg use it. It shares no code, header, table or constant with the
 * HIP kernels.
 *
 * What it computes (the plain definition of the operation the pages describe):
 *   causal prefill attention forward, O = softmax(Q K^T * scale + causal mask) V,
 *   in BF16 or FP8 e4m3 inputs with BF16 output.
 *   Sources: ZYFA abstract ("ZYFA: Speed and Accuracy of FP8 FlashAttention on
 *   AMD CDNA4", airebao.com page) -- prefill kernels, FlashAttention with a
 *   softmax between two matrix products; spbcomputers.ru ZYFA article, intro and
 *   FAQ -- causal forward only, FP8 e4m3 and BF16, flash_attn_func-compatible
 *   interface.
 *
 * Readings taken where the pages are silent:
 *   - layout is flash_attn_func's (batch, seq, heads, dim), contiguous;
 *   - grouped-query attention: query head h reads KV head h / (Hq / Hkv);
 *   - causal mask with equal query and key lengths: key j is visible to row i
 *     iff j <= i; with Sk > Sq keys the queries are the last Sq positions, so
 *     key j is visible to query i iff j <= i + Sk - Sq (flash_attn_func's
 *     alignment; oracle_attn_prefix_f64);
 *   - FP8 inputs carry one per-tensor dequantisation factor each (dq, dk, dv):
 *     the score scale becomes scale*dq*dk and dv multiplies the output.
 *
 * Arithmetic: every input element is decoded exactly (from the format
 * definitions, no library cast) to double; dot products, max, exp, sums and
 * the weighted V sum are all double. No tiling, no online rescaling: each row
 * is the textbook softmax over its visible keys.
 *
 * Parity pins (tests/test_oracle.py): brute force on tiny inputs (outputs,
 * log-sum-exp, the probability matrix of oracle_attn_probs_f64, queries after
 * a key prefix); a library routine (torch scaled_dot_product_attention,
 * float64, causal, and with an explicit bottom-right mask); closed forms (row
 * 0 equals V[0]; equal scores give the prefix mean of V); invariants
 * (probability rows sum to one, score shift invariance, GQA equals MHA with
 * repeated K/V, V column permutation); decoders against torch's casts on all
 * codes.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_BF16 0
#define ORACLE_FP8_E4M3 1

/* bfloat16: the upper 16 bits of an IEEE-754 binary32. Exact in double. */
double oracle_decode_bf16(uint16_t h) {
  uint32_t bits = (uint32_t)h << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* OCP FP8 e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.
 * Exponent field 0 is subnormal: m * 2^-9. Exponent 15 with mantissa 7
 * (0x7F / 0xFF) is NaN; there are no infinities, so the largest finite value
 * is 1.75 * 2^8 = 448. */
double oracle_decode_e4m3fn(uint8_t c) {
  int sign = c >> 7, e = (c >> 3) & 0xF, m = c & 7;
  double mag;
  if (e == 0xF && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m, -9);
  else
    mag = ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -mag : mag;
}

static double decode_elem(const void* base, int dtype, size_t idx) {
  if (dtype == ORACLE_BF16) return oracle_decode_bf16(((const uint16_t*)base)[idx]);
  return oracle_decode_e4m3fn(((const uint8_t*)base)[idx]);
}

typedef struct {
  /* inputs */
  const void *q, *k, *v;
  int dtype, B, Hq, Hkv, Sq, Sk, Dqk, Dv;
  double score_scale, dv;
  /* decoded K/V of the KV head being processed: [Sk][Dqk], [Sk][Dv] */
  const double *kd, *vd;
  int b, g;
  /* rows to compute: (h, i) pairs and where each result goes */
  const int32_t* row_h;
  const int32_t* row_i;
  double* const* row_out;
  double* const* row_lse; /* NULL, or where each row's log-sum-exp goes */
  int64_t nrows;
  /* work distribution */
  int64_t next;
  pthread_mutex_t lock;
} job_t;

/* The softmax weights of row i (of Sq), the definition of causal softmax in
 * fp64: scores s_j = scale * dq * dk * <q_i, k_j> for the visible keys
 * j <= last = i + Sk - Sq (with Sq = Sk: j <= i), their max m, and
 * w[j] = exp(s_j - m). Returns l = sum_j w[j]; *m_out = m. Query i sits at
 * position i + Sk - Sq of the key sequence. */
static double row_weights(const job_t* J, int h, int i, double* qrow, double* w, double* m_out) {
  const int Dqk = J->Dqk;
  const int last = i + (J->Sk - J->Sq); /* the last visible key */
  size_t qoff = (((size_t)J->b * J->Sq + i) * J->Hq + h) * Dqk;
  for (int d = 0; d < Dqk; ++d) qrow[d] = decode_elem(J->q, J->dtype, qoff + d);
  double m = -INFINITY;
  for (int j = 0; j <= last; ++j) {
    const double* kr = J->kd + (size_t)j * Dqk;
    double acc = 0.0;
    for (int d = 0; d < Dqk; ++d) acc += qrow[d] * kr[d];
    w[j] = J->score_scale * acc;
    if (w[j] > m) m = w[j];
  }
  double l = 0.0;
  for (int j = 0; j <= last; ++j) {
    w[j] = exp(w[j] - m);
    l += w[j];
  }
  *m_out = m;
  return l;
}

/* One output row: the weighted sum of V rows under row_weights' weights,
 * divided by their sum, times dv; also the row's log-sum-exp
 * ln sum_j exp(s_j) = m + ln l when lse is not NULL. */
static void one_row(const job_t* J, int h, int i, double* out, double* lse, double* qrow, double* w) {
  const int Dv = J->Dv;
  const int last = i + (J->Sk - J->Sq);
  double m;
  const double l = row_weights(J, h, i, qrow, w, &m);
  for (int d = 0; d < Dv; ++d) out[d] = 0.0;
  for (int j = 0; j <= last; ++j) {
    const double* vr = J->vd + (size_t)j * Dv;
    const double wj = w[j];
    for (int d = 0; d < Dv; ++d) out[d] += wj * vr[d];
  }
  for (int d = 0; d < Dv; ++d) out[d] = J->dv * out[d] / l;
  if (lse) *lse = m + log(l);
}

static void* worker(void* arg) {
  job_t* J = (job_t*)arg;
  double* qrow = (double*)malloc(sizeof(double) * (size_t)J->Dqk);
  double* w = (double*)malloc(sizeof(double) * (size_t)J->Sk);
  if (!qrow || !w) {
    free(qrow);
    free(w);
    return (void*)1;
  }
  for (;;) {
    int64_t r;
    pthread_mutex_lock(&J->lock);
    r = J->next++;
    pthread_mutex_unlock(&J->lock);
    if (r >= J->nrows) break;
    one_row(J, J->row_h[r], J->row_i[r], J->row_out[r], J->row_lse ? J->row_lse[r] : NULL, qrow, w);
  }
  free(qrow);
  free(w);
  return NULL;
}

int oracle_num_threads(int requested) {
  if (requested > 0) return requested;
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  return n > 0 ? (int)n : 1;
}

/*
 * oracle_attn_prefix_f64: exact causal attention of Sq queries over Sk >= Sq
 * keys, the queries being the last Sq positions (query i sees keys
 * j <= i + Sk - Sq), and the natural log-sum-exp of each row's logits
 * scale*dq*dk*<q_i, k_j> over its visible keys. oracle_attn_lse_f64 is the
 * case Sq = Sk = S, oracle_attn_f64 the same without the log-sum-exp.
 *
 *   q [B][Sq][Hq][Dqk], k [B][Sk][Hkv][Dqk], v [B][Sk][Hkv][Dv]: raw element
 *   codes (uint16 bfloat16 when dtype == 0, uint8 e4m3fn when dtype == 1), host memory.
 *   scale: softmax scale; dq, dk, dv: per-tensor dequantisation factors (1 for BF16).
 *   rows: NULL for every row, giving out [B][Sq][Hq][Dv] and lse [B][Hq][Sq];
 *   otherwise nrows triples (b, h, i) with out [nrows][Dv] and lse [nrows].
 *   lse: NULL, or where the log-sum-exps go.
 *   nthreads: worker threads, 0 for every online core.
 * Returns 0, or -1 on invalid arguments / allocation failure.
 */
int oracle_attn_prefix_f64(const void* q, const void* k, const void* v, int dtype, int B, int Hq, int Hkv, int Sq,
                           int Sk, int Dqk, int Dv, double scale, double dq, double dk, double dv,
                           const int64_t* rows, int64_t nrows, double* out, double* lse, int nthreads) {
  const int S = Sq;
  if (!q || !k || !v || !out) return -1;
  if (dtype != ORACLE_BF16 && dtype != ORACLE_FP8_E4M3) return -1;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || Sk < S || Dqk <= 0 || Dv <= 0 || Hq % Hkv) return -1;
  const int G = Hq / Hkv;
  const int64_t total = rows ? nrows : (int64_t)B * S * Hq;
  if (total < 0) return -1;
  for (int64_t r = 0; rows && r < nrows; ++r) {
    if (rows[3 * r] < 0 || rows[3 * r] >= B || rows[3 * r + 1] < 0 || rows[3 * r + 1] >= Hq ||
        rows[3 * r + 2] < 0 || rows[3 * r + 2] >= S)
      return -1;
  }
  nthreads = oracle_num_threads(nthreads);

  double* kd = (double*)malloc(sizeof(double) * (size_t)Sk * Dqk);
  double* vd = (double*)malloc(sizeof(double) * (size_t)Sk * Dv);
  int32_t* rh = (int32_t*)malloc(sizeof(int32_t) * (size_t)(total ? total : 1));
  int32_t* ri = (int32_t*)malloc(sizeof(int32_t) * (size_t)(total ? total : 1));
  double** ro = (double**)malloc(sizeof(double*) * (size_t)(total ? total : 1));
  double** rl = (double**)malloc(sizeof(double*) * (size_t)(total ? total : 1));
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  int rc = 0;
  if (!kd || !vd || !rh || !ri || !ro || !rl || !th) {
    rc = -1;
    goto done;
  }

  for (int b = 0; b < B && rc == 0; ++b) {
    for (int g = 0; g < Hkv && rc == 0; ++g) {
      /* collect the requested rows that read KV head (b, g); longest rows first */
      int64_t n = 0;
      if (rows) {
        for (int64_t r = 0; r < nrows; ++r) {
          if (rows[3 * r] != b || rows[3 * r + 1] / G != g) continue;
          rh[n] = (int32_t)rows[3 * r + 1];
          ri[n] = (int32_t)rows[3 * r + 2];
          ro[n] = out + (size_t)r * Dv;
          rl[n] = lse ? lse + r : NULL;
          ++n;
        }
      } else {
        for (int i = S - 1; i >= 0; --i)
          for (int h = g * G; h < (g + 1) * G; ++h) {
            rh[n] = h;
            ri[n] = i;
            ro[n] = out + (((size_t)b * S + i) * Hq + h) * Dv;
            rl[n] = lse ? lse + ((size_t)b * Hq + h) * S + i : NULL;
            ++n;
          }
      }
      if (n == 0) continue;
      for (int j = 0; j < Sk; ++j) {
        size_t ko = (((size_t)b * Sk + j) * Hkv + g) * Dqk, vo = (((size_t)b * Sk + j) * Hkv + g) * Dv;
        for (int d = 0; d < Dqk; ++d) kd[(size_t)j * Dqk + d] = decode_elem(k, dtype, ko + d);
        for (int d = 0; d < Dv; ++d) vd[(size_t)j * Dv + d] = decode_elem(v, dtype, vo + d);
      }
      job_t J;
      memset(&J, 0, sizeof J);
      J.q = q; J.k = k; J.v = v; J.dtype = dtype; J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.Sq = S; J.Sk = Sk;
      J.Dqk = Dqk; J.Dv = Dv; J.score_scale = scale * dq * dk; J.dv = dv;
      J.kd = kd; J.vd = vd; J.b = b; J.g = g;
      J.row_h = rh; J.row_i = ri; J.row_out = ro; J.row_lse = lse ? rl : NULL; J.nrows = n; J.next = 0;
      pthread_mutex_init(&J.lock, NULL);
      int nt = (int64_t)nthreads > n ? (int)n : nthreads, started = 0;
      for (int t = 0; t < nt; ++t)
        if (pthread_create(&th[t], NULL, worker, &J) == 0) ++started;
      if (started == 0) worker(&J); /* run inline if no thread could start */
      for (int t = 0; t < started; ++t) {
        void* ret = NULL;
        pthread_join(th[t], &ret);
        if (ret) rc = -1;
      }
      pthread_mutex_destroy(&J.lock);
    }
  }
done:
  free(kd); free(vd); free(rh); free(ri); free(ro); free(rl); free(th);
  return rc;
}

int oracle_attn_lse_f64(const void* q, const void* k, const void* v, int dtype, int B, int Hq, int Hkv, int S,
                        int Dqk, int Dv, double scale, double dq, double dk, double dv, const int64_t* rows,
                        int64_t nrows, double* out, double* lse, int nthreads) {
  return oracle_attn_prefix_f64(q, k, v, dtype, B, Hq, Hkv, S, S, Dqk, Dv, scale, dq, dk, dv, rows, nrows, out, lse,
                                nthreads);
}

int oracle_attn_f64(const void* q, const void* k, const void* v, int dtype, int B, int Hq, int Hkv, int S,
                    int Dqk, int Dv, double scale, double dq, double dk, double dv, const int64_t* rows,
                    int64_t nrows, double* out, int nthreads) {
  return oracle_attn_lse_f64(q, k, v, dtype, B, Hq, Hkv, S, Dqk, Dv, scale, dq, dk, dv, rows, nrows, out, NULL,
                             nthreads);
}

/*
 * oracle_attn_probs_f64: the full probability matrix P[i][j] of one (b, h)
 * slice, zero above the diagonal: row i is row_weights' w / l, the weights
 * one_row applies to V. For tiny S only (the "rows of P sum to one"
 * invariant). Same inputs and readings as oracle_attn_f64.
 */
int oracle_attn_probs_f64(const void* q, const void* k, int dtype, int B, int Hq, int Hkv, int S, int Dqk,
                          double scale, double dq, double dk, int b, int h, double* P) {
  if (!q || !k || !P || B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || Dqk <= 0 || Hq % Hkv) return -1;
  if (dtype != ORACLE_BF16 && dtype != ORACLE_FP8_E4M3) return -1;
  if (b < 0 || b >= B || h < 0 || h >= Hq) return -1;
  const int g = h / (Hq / Hkv);
  double* kd = (double*)malloc(sizeof(double) * (size_t)S * Dqk);
  double* qrow = (double*)malloc(sizeof(double) * (size_t)Dqk);
  double* w = (double*)malloc(sizeof(double) * (size_t)S);
  int rc = 0;
  if (!kd || !qrow || !w) {
    rc = -1;
    goto done;
  }
  for (int j = 0; j < S; ++j) {
    const size_t ko = (((size_t)b * S + j) * Hkv + g) * Dqk;
    for (int d = 0; d < Dqk; ++d) kd[(size_t)j * Dqk + d] = decode_elem(k, dtype, ko + d);
  }
  job_t J;
  memset(&J, 0, sizeof J);
  J.q = q; J.k = k; J.dtype = dtype; J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.Sq = S; J.Sk = S;
  J.Dqk = Dqk; J.score_scale = scale * dq * dk; J.kd = kd; J.b = b; J.g = g;
  for (int i = 0; i < S; ++i) {
    double m;
    const double l = row_weights(&J, h, i, qrow, w, &m);
    double* row = P + (size_t)i * S;
    for (int j = 0; j < S; ++j) row[j] = j <= i ? w[j] / l : 0.0;
  }
done:
  free(kd); free(qrow); free(w);
  return rc;
}
