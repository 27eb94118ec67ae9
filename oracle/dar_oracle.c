/*
 * DAR attention oracle: plain fp64 loops, written straight from the method's
 * equations.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * CPU-baseline leg of the benchmark may call it; the library never does.
 * It shares no code, header or table with the HIP path.
 *
 * Source: "Dual Dimensionality for Local and Global Attention" (the DAR
 * paper), Eq. (1) bottleneck h^D = h W_down, Eq. (2) lift h' = h^D W_up,
 * Eq. (3) distance-selected keys and values, Eq. (4) softmax attention with
 * the 1/sqrt(d_k) scale.  The paper states one head; several heads apply
 * that one-head form head by head (the paragraph before Eq. (2)).
 *
 * Readings taken where the paper is silent:
 *  - RoPE rotates both q_i (position i) and k_j (position j); rotate-half
 *    pairing (t, t + d_k/2) over the full head width, theta_t =
 *    base^(-2t/d_k), positions p = pos0 + n counted from 0.
 *  - One W_down / W_up per layer, shared by every head; head a owns the
 *    columns [a*d_k, (a+1)*d_k) of W_Q, W_K, W_V; o concatenates the heads.
 *  - Eq. (3)'s condition i - j < w selects the full-state path; w = 0 sends
 *    every pair, j = i included, through the bottleneck.
 *  - Decode keeps, for the query at position p, the full keys/values of
 *    positions p-w+1 .. p in a ring (slot = position mod w) and the latent
 *    h^D of every position; positions j <= p - w are rebuilt from h^D.
 *
 * All arrays are fp64, row-major, innermost index contiguous.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int dar_oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* y[c] = sum_k x[k] * W[k*ld + col0 + c] for c < ncol, k ascending. */
static void vec_mat(const double* x, const double* W, int K, int ld, int col0, int ncol,
                    double* y) {
  for (int c = 0; c < ncol; ++c) y[c] = 0.0;
  for (int k = 0; k < K; ++k) {
    const double xk = x[k];
    const double* row = W + (size_t)k * ld + col0;
    for (int c = 0; c < ncol; ++c) y[c] += xk * row[c];
  }
}

/* Rotary embedding at position pos, rotate-half pairing, in place. */
static void rope(double* x, int d_k, double pos, double base) {
  const int half = d_k / 2;
  for (int t = 0; t < half; ++t) {
    const double theta = pow(base, -2.0 * (double)t / (double)d_k);
    const double phi = pos * theta;
    const double c = cos(phi), s = sin(phi);
    const double a = x[t], b = x[t + half];
    x[t] = a * c - b * s;
    x[t + half] = a * s + b * c;
  }
}

/*
 * Projections of tokens n < n_tok of every sequence, heads [head_lo, head_hi):
 *   hD = h W_down                      (Eq. 1)      hD : [B, N, d_down]
 *        act = 1: hD = sigmoid(h W_down), 1 / (1 + e^-x) per element (the
 *        variant named in the paragraph after Eq. 1); act = 0: as written
 *   hp = hD W_up                       (Eq. 2)      hp : [B, N, d]
 *   Q  = RoPE_p(h  W_Q[:, S_a])        (q_i, Eq. 4 text)
 *   KL = RoPE_p(h  W_K[:, S_a]),  VL = h  W_V[:, S_a]   (Eq. 3, i - j <  w)
 *   KG = RoPE_p(hp W_K[:, S_a]),  VG = hp W_V[:, S_a]   (Eq. 3, otherwise)
 * Q, KL, VL, KG, VG : [B, H, N, d_k]; p = pos0 + n.
 * Returns 0, or -1 on a bad argument.
 */
int dar_oracle_project_act(const double* h, const double* W_down, const double* W_up,
                           const double* W_Q, const double* W_K, const double* W_V,
                           int B, int N, int d, int d_down, int H, int d_k, long pos0,
                           double base, int n_tok, int head_lo, int head_hi, int act,
                           double* hD, double* hp, double* Q, double* KL, double* VL,
                           double* KG, double* VG) {
  if (act != 0 && act != 1) return -1;
  if (B < 1 || N < 1 || d < 1 || d_down < 1 || H < 1 || d_k < 2 || (d_k & 1)) return -1;
  if (n_tok < 0 || n_tok > N || head_lo < 0 || head_hi > H || head_lo > head_hi) return -1;
  const int hd = H * d_k;
  const long total = (long)B * n_tok;
#pragma omp parallel for schedule(dynamic, 4)
  for (long bn = 0; bn < total; ++bn) {
    const int b = (int)(bn / n_tok), n = (int)(bn % n_tok);
    const size_t tok = (size_t)b * N + n;
    const double* x = h + tok * d;
    double* xD = hD + tok * d_down;
    double* xp = hp + tok * d;
    vec_mat(x, W_down, d, d_down, 0, d_down, xD);  /* Eq. 1 */
    if (act == 1) /* the variant with a sigmoid after the down-projection */
      for (int k = 0; k < d_down; ++k) xD[k] = 1.0 / (1.0 + exp(-xD[k]));
    vec_mat(xD, W_up, d_down, d, 0, d, xp);        /* Eq. 2 */
    const double pos = (double)(pos0 + n);
    for (int a = head_lo; a < head_hi; ++a) {
      const size_t off = (((size_t)b * H + a) * N + n) * d_k;
      vec_mat(x, W_Q, d, hd, a * d_k, d_k, Q + off);
      rope(Q + off, d_k, pos, base);
      vec_mat(x, W_K, d, hd, a * d_k, d_k, KL + off);
      rope(KL + off, d_k, pos, base);
      vec_mat(x, W_V, d, hd, a * d_k, d_k, VL + off);
      vec_mat(xp, W_K, d, hd, a * d_k, d_k, KG + off);
      rope(KG + off, d_k, pos, base);
      vec_mat(xp, W_V, d, hd, a * d_k, d_k, VG + off);
    }
  }
  return 0;
}

int dar_oracle_project(const double* h, const double* W_down, const double* W_up,
                       const double* W_Q, const double* W_K, const double* W_V,
                       int B, int N, int d, int d_down, int H, int d_k, long pos0,
                       double base, int n_tok, int head_lo, int head_hi,
                       double* hD, double* hp, double* Q, double* KL, double* VL,
                       double* KG, double* VG) {
  return dar_oracle_project_act(h, W_down, W_up, W_Q, W_K, W_V, B, N, d, d_down, H, d_k, pos0,
                                base, n_tok, head_lo, head_hi, 0, hD, hp, Q, KL, VL, KG, VG);
}

/*
 * One output row: query i of sequence b, head a (Eq. 3 selection, Eq. 4).
 * Keys j = 0 .. i; (k_j, v_j) = (KL_j, VL_j) if i - j < w else (KG_j, VG_j).
 * s_j = q_i . k_j / sqrt(d_k); o = sum_j softmax(s)_j v_j.
 * Writes o[0..d_k) and the sum of the softmax weights.
 */
static void attend_row(const double* Q, const double* KL, const double* VL,
                       const double* KG, const double* VG, int N, int H, int d_k, long w,
                       int b, int a, int i, double* s, double* o, double* rowsum) {
  const size_t base_off = ((size_t)b * H + a) * N;
  const double* q = Q + (base_off + i) * d_k;
  const double scale = 1.0 / sqrt((double)d_k);
  double m = -INFINITY;
  for (int j = 0; j <= i; ++j) {
    const int local = (long)(i - j) < w;
    const double* k = (local ? KL : KG) + (base_off + j) * d_k;
    double dot = 0.0;
    for (int t = 0; t < d_k; ++t) dot += q[t] * k[t];
    s[j] = dot * scale;
    if (s[j] > m) m = s[j];
  }
  double Z = 0.0;
  for (int j = 0; j <= i; ++j) {
    s[j] = exp(s[j] - m);
    Z += s[j];
  }
  for (int t = 0; t < d_k; ++t) o[t] = 0.0;
  double psum = 0.0;
  for (int j = 0; j <= i; ++j) {
    const int local = (long)(i - j) < w;
    const double* v = (local ? VL : VG) + (base_off + j) * d_k;
    const double p = s[j] / Z;
    psum += p;
    for (int t = 0; t < d_k; ++t) o[t] += p * v[t];
  }
  if (rowsum) *rowsum = psum;
}

/* Every row: o [B, N, H*d_k] (heads concatenated), rowsum [B, H, N] (may be NULL). */
int dar_oracle_attend(const double* Q, const double* KL, const double* VL, const double* KG,
                      const double* VG, int B, int N, int H, int d_k, long w, double* o,
                      double* rowsum) {
  if (B < 1 || N < 1 || H < 1 || d_k < 1 || w < 0) return -1;
  const long total = (long)B * H * N;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)N);
    double* orow = (double*)malloc(sizeof(double) * (size_t)d_k);
#pragma omp for schedule(dynamic, 8)
    for (long r = 0; r < total; ++r) {
      const int i = (int)(r % N), a = (int)((r / N) % H), b = (int)(r / ((long)N * H));
      double rs;
      attend_row(Q, KL, VL, KG, VG, N, H, d_k, w, b, a, i, s, orow, &rs);
      memcpy(o + ((size_t)b * N + i) * H * d_k + (size_t)a * d_k, orow, sizeof(double) * d_k);
      if (rowsum) rowsum[((size_t)b * H + a) * N + i] = rs;
    }
    free(s);
    free(orow);
  }
  return 0;
}

/* Selected rows (rb[r], rh[r], ri[r]) only: o_rows [n_rows, d_k], rowsum [n_rows]. */
int dar_oracle_attend_rows(const double* Q, const double* KL, const double* VL,
                           const double* KG, const double* VG, int B, int N, int H, int d_k,
                           long w, int n_rows, const int* rb, const int* rh, const int* ri,
                           double* o_rows, double* rowsum) {
  if (B < 1 || N < 1 || H < 1 || d_k < 1 || w < 0 || n_rows < 0) return -1;
  for (int r = 0; r < n_rows; ++r)
    if (rb[r] < 0 || rb[r] >= B || rh[r] < 0 || rh[r] >= H || ri[r] < 0 || ri[r] >= N)
      return -1;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
    for (int r = 0; r < n_rows; ++r)
      attend_row(Q, KL, VL, KG, VG, N, H, d_k, w, rb[r], rh[r], ri[r], s,
                 o_rows + (size_t)r * d_k, rowsum ? rowsum + r : NULL);
    free(s);
  }
  return 0;
}

/*
 * Softmax normaliser of each row of Eq. (4): lse_i = log sum_{j <= i}
 * exp(q_i . k_j / sqrt(d_k)), keys chosen by Eq. (3).  lse: [B, H, N].
 */
int dar_oracle_attend_lse(const double* Q, const double* KL, const double* KG, int B, int N,
                          int H, int d_k, long w, double* lse) {
  if (B < 1 || N < 1 || H < 1 || d_k < 1 || w < 0) return -1;
  const double scale = 1.0 / sqrt((double)d_k);
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 8)
    for (long r = 0; r < (long)B * H * N; ++r) {
      const int i = (int)(r % N);
      const size_t off = (size_t)(r / N) * N;
      const double* q = Q + (off + i) * d_k;
      double m = -INFINITY;
      for (int j = 0; j <= i; ++j) {
        const double* k = ((long)(i - j) < w ? KL : KG) + (off + j) * d_k;
        double dot = 0.0;
        for (int t = 0; t < d_k; ++t) dot += q[t] * k[t];
        s[j] = dot * scale;
        if (s[j] > m) m = s[j];
      }
      double Z = 0.0;
      for (int j = 0; j <= i; ++j) Z += exp(s[j] - m);
      lse[r] = m + log(Z);
    }
    free(s);
  }
  return 0;
}

/*
 * Backward of the attention of Eqs. (3)-(4) for a loss L with dL/do = dO.
 * The selection of Eq. (3) is a fixed choice per (i, j) pair, so each pair's
 * gradient flows to the source it used: with p_j = softmax(s)_j over j <= i
 * and s_j = q_i . k_j / sqrt(d_k),
 *   dv_j    += p_j dO_i                       (o_i = sum_j p_j v_j)
 *   dp_j     = dO_i . v_j
 *   ds_j     = p_j (dp_j - sum_l p_l dp_l)    (derivative of the softmax)
 *   dq_i    += ds_j k_j / sqrt(d_k),   dk_j += ds_j q_i / sqrt(d_k)
 * where (k_j, v_j, dk_j, dv_j) belong to the local source when i - j < w and
 * to the global one otherwise.  dO: [B, N, H*d_k] like o; every gradient is
 * [B, H, N, d_k] and is overwritten.
 */
int dar_oracle_attend_backward(const double* Q, const double* KL, const double* VL,
                               const double* KG, const double* VG, const double* dO, int B,
                               int N, int H, int d_k, long w, double* dQ, double* dKL,
                               double* dVL, double* dKG, double* dVG) {
  if (B < 1 || N < 1 || H < 1 || d_k < 1 || w < 0) return -1;
  const size_t n_all = (size_t)B * H * N * d_k;
  memset(dQ, 0, sizeof(double) * n_all);
  memset(dKL, 0, sizeof(double) * n_all);
  memset(dVL, 0, sizeof(double) * n_all);
  memset(dKG, 0, sizeof(double) * n_all);
  memset(dVG, 0, sizeof(double) * n_all);
  const double scale = 1.0 / sqrt((double)d_k);
#pragma omp parallel
  {
    double* p = (double*)malloc(sizeof(double) * (size_t)N);
    double* dp = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
    for (long ba = 0; ba < (long)B * H; ++ba) {
      const int b = (int)(ba / H), a = (int)(ba % H);
      const size_t off = (size_t)ba * N;
      for (int i = 0; i < N; ++i) {
        const double* q = Q + (off + i) * d_k;
        const double* g = dO + ((size_t)b * N + i) * H * d_k + (size_t)a * d_k;
        double m = -INFINITY;
        for (int j = 0; j <= i; ++j) {
          const double* k = ((long)(i - j) < w ? KL : KG) + (off + j) * d_k;
          double dot = 0.0;
          for (int t = 0; t < d_k; ++t) dot += q[t] * k[t];
          p[j] = dot * scale;
          if (p[j] > m) m = p[j];
        }
        double Z = 0.0;
        for (int j = 0; j <= i; ++j) {
          p[j] = exp(p[j] - m);
          Z += p[j];
        }
        double pdp = 0.0;
        for (int j = 0; j <= i; ++j) {
          p[j] /= Z;
          const int local = (long)(i - j) < w;
          const double* v = (local ? VL : VG) + (off + j) * d_k;
          double* dv = (local ? dVL : dVG) + (off + j) * d_k;
          double dot = 0.0;
          for (int t = 0; t < d_k; ++t) {
            dot += g[t] * v[t];
            dv[t] += p[j] * g[t];
          }
          dp[j] = dot;
          pdp += p[j] * dot;
        }
        double* dq = dQ + (off + i) * d_k;
        for (int j = 0; j <= i; ++j) {
          const int local = (long)(i - j) < w;
          const double* k = (local ? KL : KG) + (off + j) * d_k;
          double* dk = (local ? dKL : dKG) + (off + j) * d_k;
          const double ds = p[j] * (dp[j] - pdp) * scale;
          for (int t = 0; t < d_k; ++t) {
            dq[t] += ds * k[t];
            dk[t] += ds * q[t];
          }
        }
      }
    }
    free(p);
    free(dp);
  }
  return 0;
}

/*
 * Decode step over the mixed cache, one query per sequence at position
 * p = ctx - 1 (the latent-cache reading of the inference remarks: full keys
 * and values for the w most recent positions, the d_down latent beyond).
 *   q      [B, H, d_k]      query, already rotated at p
 *   K_win  [B, H, w, d_k]   rotated keys of positions p-w+1 .. p, slot = pos mod w
 *   V_win  [B, H, w, d_k]   values, same slots
 *   hD     [B, cap, d_down] latents h^D_j (Eq. 1); rows j <= p - w are read
 * For j <= p - w: h'_j = h^D_j W_up (Eq. 2), k_j = RoPE_j(h'_j W_K[:, S_a]),
 * v_j = h'_j W_V[:, S_a] (Eq. 3, global branch).  o [B, H*d_k]; heads outside
 * [head_lo, head_hi) are left untouched.
 */
int dar_oracle_decode(const double* q, const double* K_win, const double* V_win,
                      const double* hD, const double* W_up, const double* W_K,
                      const double* W_V, int B, long ctx, long cap, int H, int d_k, int d_down,
                      int d, long w, double base, int head_lo, int head_hi, double* o) {
  if (B < 1 || ctx < 1 || cap < 1 || H < 1 || d_k < 2 || (d_k & 1) || d_down < 1 || d < 1 ||
      w < 0 || head_lo < 0 || head_hi > H || head_lo > head_hi)
    return -1;
  const long p = ctx - 1;
  const long n_glob = p - w + 1 > 0 ? p - w + 1 : 0; /* positions 0 .. p-w */
  if (n_glob > cap) return -1;
  const int hd = H * d_k, nh = head_hi - head_lo;
  if (nh == 0) return 0;
  const double scale = 1.0 / sqrt((double)d_k);
  double* KGb = (double*)malloc(sizeof(double) * (size_t)(n_glob > 0 ? n_glob : 1) * nh * d_k);
  double* VGb = (double*)malloc(sizeof(double) * (size_t)(n_glob > 0 ? n_glob : 1) * nh * d_k);
  double* s = (double*)malloc(sizeof(double) * (size_t)(p + 1));
  if (!KGb || !VGb || !s) {
    free(KGb); free(VGb); free(s);
    return -2;
  }
  for (int b = 0; b < B; ++b) {
#pragma omp parallel
    {
      double* xp = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 16)
      for (long j = 0; j < n_glob; ++j) {
        vec_mat(hD + ((size_t)b * cap + j) * d_down, W_up, d_down, d, 0, d, xp); /* Eq. 2 */
        for (int a = head_lo; a < head_hi; ++a) {
          double* k = KGb + ((size_t)j * nh + (a - head_lo)) * d_k;
          double* v = VGb + ((size_t)j * nh + (a - head_lo)) * d_k;
          vec_mat(xp, W_K, d, hd, a * d_k, d_k, k);
          rope(k, d_k, (double)j, base);
          vec_mat(xp, W_V, d, hd, a * d_k, d_k, v);
        }
      }
      free(xp);
    }
    for (int a = head_lo; a < head_hi; ++a) {
      const double* qa = q + ((size_t)b * H + a) * d_k;
      double m = -INFINITY;
      for (long j = 0; j <= p; ++j) {
        const double* k = (p - j < w)
                              ? K_win + (((size_t)b * H + a) * w + (size_t)(j % w)) * d_k
                              : KGb + ((size_t)j * nh + (a - head_lo)) * d_k;
        double dot = 0.0;
        for (int t = 0; t < d_k; ++t) dot += qa[t] * k[t];
        s[j] = dot * scale;
        if (s[j] > m) m = s[j];
      }
      double Z = 0.0;
      for (long j = 0; j <= p; ++j) {
        s[j] = exp(s[j] - m);
        Z += s[j];
      }
      double* oa = o + (size_t)b * hd + (size_t)a * d_k;
      for (int t = 0; t < d_k; ++t) oa[t] = 0.0;
      for (long j = 0; j <= p; ++j) {
        const double* v = (p - j < w)
                              ? V_win + (((size_t)b * H + a) * w + (size_t)(j % w)) * d_k
                              : VGb + ((size_t)j * nh + (a - head_lo)) * d_k;
        const double pj = s[j] / Z;
        for (int t = 0; t < d_k; ++t) oa[t] += pj * v[t];
      }
    }
  }
  free(KGb);
  free(VGb);
  free(s);
  return 0;
}

/* ------------------------------------------------------------------------
 * Decoupled-RoPE variant.  The DAR paper names MLA's decoupled rotary
 * embedding as the route to an efficient implementation (the paragraph after
 * the inference remark) and calls its latent h^D the counterpart of MLA's
 * compressed vector (the paragraph after Eq. (1)); the papernotes summary's
 * efficiency analysis repeats the pairing.  The pages do not write the
 * variant out; the reading taken is MLA's construction carried over to Eqs.
 * (1)-(4):
 *   - every head's query and key get a rotary part of width d_R beside the
 *     content part of width d_k; only the rotary part is rotated;
 *   - content:  qC_i = h_i W_Q[:, S_a];  kC_j = h_j W_K[:, S_a] (i - j < w)
 *               or h'_j W_K[:, S_a] (otherwise), Eq. (3) without RoPE;
 *   - rotary:   qR_i = RoPE_i(h_i W_QR[:, R_a]), R_a = [a d_R, (a+1) d_R);
 *               kR_j = RoPE_j(h_j W_KR), one rotary key per token, from the
 *               full hidden state, shared by every head and by both paths;
 *   - values as Eq. (3); s_ij = (qC_i . kC_j + qR_i . kR_j) / sqrt(d_k + d_R);
 *     o_i = sum_j softmax(s)_j v_j (Eq. (4)).
 * d_R = 0 leaves the content part alone (no rotation anywhere, scale
 * 1/sqrt(d_k)).  RoPE over the rotary part: pairs (t, t + d_R/2), theta_t =
 * base^(-2t/d_R).
 * ------------------------------------------------------------------------ */

/*
 * Projections of the variant for tokens n < n_tok, heads [head_lo, head_hi):
 *   hD [B,N,d_down], hp [B,N,d]                 Eqs. (1)-(2)
 *   QC, KL, VL, KG, VG [B,H,N,d_k]              content parts, values
 *   QR [B,H,N,d_R]                              rotary queries
 *   KR [B,N,d_R]                                rotary keys (every token)
 * W_QR [d, H d_R], W_KR [d, d_R].
 */
int dar_oracle_project_drope(const double* h, const double* W_down, const double* W_up,
                             const double* W_Q, const double* W_K, const double* W_V,
                             const double* W_QR, const double* W_KR, int B, int N, int d,
                             int d_down, int H, int d_k, int d_R, long pos0, double base,
                             int n_tok, int head_lo, int head_hi, double* hD, double* hp,
                             double* QC, double* QR, double* KL, double* VL, double* KG,
                             double* VG, double* KR) {
  if (B < 1 || N < 1 || d < 1 || d_down < 1 || H < 1 || d_k < 1 || d_R < 0 || (d_R & 1))
    return -1;
  if (n_tok < 0 || n_tok > N || head_lo < 0 || head_hi > H || head_lo > head_hi) return -1;
  const int hd = H * d_k, hr = H * d_R;
  const long total = (long)B * n_tok;
#pragma omp parallel for schedule(dynamic, 4)
  for (long bn = 0; bn < total; ++bn) {
    const int b = (int)(bn / n_tok), n = (int)(bn % n_tok);
    const size_t tok = (size_t)b * N + n;
    const double* x = h + tok * d;
    double* xD = hD + tok * d_down;
    double* xp = hp + tok * d;
    vec_mat(x, W_down, d, d_down, 0, d_down, xD); /* Eq. 1 */
    vec_mat(xD, W_up, d_down, d, 0, d, xp);       /* Eq. 2 */
    const double pos = (double)(pos0 + n);
    if (d_R > 0) {
      vec_mat(x, W_KR, d, d_R, 0, d_R, KR + tok * d_R);
      rope(KR + tok * d_R, d_R, pos, base);
    }
    for (int a = head_lo; a < head_hi; ++a) {
      const size_t off = (((size_t)b * H + a) * N + n) * d_k;
      vec_mat(x, W_Q, d, hd, a * d_k, d_k, QC + off);
      vec_mat(x, W_K, d, hd, a * d_k, d_k, KL + off);
      vec_mat(x, W_V, d, hd, a * d_k, d_k, VL + off);
      vec_mat(xp, W_K, d, hd, a * d_k, d_k, KG + off);
      vec_mat(xp, W_V, d, hd, a * d_k, d_k, VG + off);
      if (d_R > 0) {
        const size_t offr = (((size_t)b * H + a) * N + n) * d_R;
        vec_mat(x, W_QR, d, hr, a * d_R, d_R, QR + offr);
        rope(QR + offr, d_R, pos, base);
      }
    }
  }
  return 0;
}

/* Attention of the variant, every row: o [B,N,H d_k], rowsum [B,H,N] (may be
 * NULL).  Keys j <= i; the content key and the value come from the local
 * arrays when i - j < w, else from the global ones; the rotary key KR_j is
 * the token's own in both cases. */
int dar_oracle_attend_drope(const double* QC, const double* QR, const double* KL,
                            const double* VL, const double* KG, const double* VG,
                            const double* KR, int B, int N, int H, int d_k, int d_R, long w,
                            double* o, double* rowsum) {
  if (B < 1 || N < 1 || H < 1 || d_k < 1 || d_R < 0 || w < 0) return -1;
  const double scale = 1.0 / sqrt((double)(d_k + d_R));
  const long total = (long)B * H * N;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 8)
    for (long r = 0; r < total; ++r) {
      const int i = (int)(r % N), a = (int)((r / N) % H), b = (int)(r / ((long)N * H));
      const size_t row0 = ((size_t)b * H + a) * N;
      const double* qc = QC + (row0 + i) * d_k;
      const double* qr = QR + (row0 + i) * d_R;
      double m = -INFINITY;
      for (int j = 0; j <= i; ++j) {
        const double* kc = (((long)(i - j) < w) ? KL : KG) + (row0 + j) * d_k;
        const double* kr = KR + ((size_t)b * N + j) * d_R;
        double dot = 0.0;
        for (int t = 0; t < d_k; ++t) dot += qc[t] * kc[t];
        for (int t = 0; t < d_R; ++t) dot += qr[t] * kr[t];
        s[j] = dot * scale;
        if (s[j] > m) m = s[j];
      }
      double Z = 0.0;
      for (int j = 0; j <= i; ++j) {
        s[j] = exp(s[j] - m);
        Z += s[j];
      }
      double* orow = o + ((size_t)b * N + i) * H * d_k + (size_t)a * d_k;
      for (int t = 0; t < d_k; ++t) orow[t] = 0.0;
      double psum = 0.0;
      for (int j = 0; j <= i; ++j) {
        const double* v = (((long)(i - j) < w) ? VL : VG) + (row0 + j) * d_k;
        const double p = s[j] / Z;
        psum += p;
        for (int t = 0; t < d_k; ++t) orow[t] += p * v[t];
      }
      if (rowsum) rowsum[r] = psum;
    }
    free(s);
  }
  return 0;
}

/*
 * Decode step of the variant over its mixed cache, one query per sequence at
 * p = ctx - 1:
 *   qC [B,H,d_k], qR [B,H,d_R]   the query's content part and rotary part
 *                                 (rotated at p)
 *   K_win, V_win [B,H,w,d_k]      content keys (not rotated) and values of
 *                                 positions p-w+1 .. p, slot = position mod w
 *   KR [B,cap,d_R]                rotary keys of every position (rotated)
 *   hD [B,cap,d_down]             latents; rows j <= p - w are read
 * Positions j <= p - w use kC_j = h^D_j W_up W_K[:, S_a] and v_j = h^D_j W_up
 * W_V[:, S_a] (Eqs. 2-3, in fp64, unfolded).  o [B, H d_k]; heads outside
 * [head_lo, head_hi) are left untouched.
 */
int dar_oracle_decode_drope(const double* qC, const double* qR, const double* K_win,
                            const double* V_win, const double* KR, const double* hD,
                            const double* W_up, const double* W_K, const double* W_V, int B,
                            long ctx, long cap, int H, int d_k, int d_R, int d_down, int d,
                            long w, int head_lo, int head_hi, double* o) {
  if (B < 1 || ctx < 1 || cap < 1 || H < 1 || d_k < 1 || d_R < 0 || d_down < 1 || d < 1 ||
      w < 0 || head_lo < 0 || head_hi > H || head_lo > head_hi)
    return -1;
  const long p = ctx - 1;
  const long n_glob = p - w + 1 > 0 ? p - w + 1 : 0;
  if (n_glob > cap || p >= cap) return -1;
  const int hd = H * d_k, nh = head_hi - head_lo;
  if (nh == 0) return 0;
  const double scale = 1.0 / sqrt((double)(d_k + d_R));
  double* KGb = (double*)malloc(sizeof(double) * (size_t)(n_glob > 0 ? n_glob : 1) * nh * d_k);
  double* VGb = (double*)malloc(sizeof(double) * (size_t)(n_glob > 0 ? n_glob : 1) * nh * d_k);
  double* s = (double*)malloc(sizeof(double) * (size_t)(p + 1));
  if (!KGb || !VGb || !s) {
    free(KGb); free(VGb); free(s);
    return -2;
  }
  for (int b = 0; b < B; ++b) {
#pragma omp parallel
    {
      double* xp = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 16)
      for (long j = 0; j < n_glob; ++j) {
        vec_mat(hD + ((size_t)b * cap + j) * d_down, W_up, d_down, d, 0, d, xp); /* Eq. 2 */
        for (int a = head_lo; a < head_hi; ++a) {
          vec_mat(xp, W_K, d, hd, a * d_k, d_k, KGb + ((size_t)j * nh + (a - head_lo)) * d_k);
          vec_mat(xp, W_V, d, hd, a * d_k, d_k, VGb + ((size_t)j * nh + (a - head_lo)) * d_k);
        }
      }
      free(xp);
    }
    for (int a = head_lo; a < head_hi; ++a) {
      const double* qc = qC + ((size_t)b * H + a) * d_k;
      const double* qr = qR + ((size_t)b * H + a) * d_R;
      double m = -INFINITY;
      for (long j = 0; j <= p; ++j) {
        const double* kc = (p - j < w)
                               ? K_win + (((size_t)b * H + a) * w + (size_t)(j % w)) * d_k
                               : KGb + ((size_t)j * nh + (a - head_lo)) * d_k;
        const double* kr = KR + ((size_t)b * cap + j) * d_R;
        double dot = 0.0;
        for (int t = 0; t < d_k; ++t) dot += qc[t] * kc[t];
        for (int t = 0; t < d_R; ++t) dot += qr[t] * kr[t];
        s[j] = dot * scale;
        if (s[j] > m) m = s[j];
      }
      double Z = 0.0;
      for (long j = 0; j <= p; ++j) {
        s[j] = exp(s[j] - m);
        Z += s[j];
      }
      double* oa = o + (size_t)b * hd + (size_t)a * d_k;
      for (int t = 0; t < d_k; ++t) oa[t] = 0.0;
      for (long j = 0; j <= p; ++j) {
        const double* v = (p - j < w)
                              ? V_win + (((size_t)b * H + a) * w + (size_t)(j % w)) * d_k
                              : VGb + ((size_t)j * nh + (a - head_lo)) * d_k;
        const double pj = s[j] / Z;
        for (int t = 0; t < d_k; ++t) oa[t] += pj * v[t];
      }
    }
  }
  free(KGb);
  free(VGb);
  free(s);
  return 0;
}
