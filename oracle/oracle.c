/*
 * oracle.c -- plain, slow, fp64 CPU oracle for the KDA gated delta-rule
 * recurrence.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link,
 * load or call this file: only the tests, the smoke check and the bench's CPU
 * baseline leg use it. It shares no code with the HIP library.
 *
 * What it computes (one unit = one (sequence, head) for prefill, one
 * (request slot, layer, head) for verify and fold), K key channels, V value
 * channels, state S[K][V] with the key channel as the row index:
 *
 *   for each token t, in order:
 *     a[c]    = exp(gk[t][c])                       per-key-channel decay
 *     u[j]    = sum_c a[c] * k[t][c] * S[c][j]      prediction of the decayed state
 *     w[j]    = beta[t] * (v[t][j] - u[j])          delta-rule error
 *     S[c][j] = a[c] * S[c][j] + k[t][c] * w[j]     decay, then rank-1 delta update
 *     o[t][j] = scale * sum_c q[t][c] * S[c][j]     readout from the updated state
 *
 * Sources (page title, section):
 *   - "SGLang and Miles Add Day-0 Support for Kimi K3" (LMSYS blog),
 *     section "Hybrid KDA Memory Management": a KDA layer keeps one
 *     fixed-size recurrent state per request that every token overwrites in
 *     place;
 *   - same post, section "ReplaySSM: raw-input replay for the KDA state":
 *     the state is K x V (64 KB per request, layer and head at K = V = 128);
 *     a step's raw inputs are (v, k, gk, beta); verify reads the committed
 *     checkpoint without writing it; the fold replays only the accepted
 *     prefix, in place, with the stored gate values;
 *   - Kimi K3 B200 deployment notes (zdszero.github.io), section on FlashKDA:
 *     the state is an fp32 [128, 128] tile per (sequence, head); section
 *     "DSPARK and KDA state": the ring keeps (v, k, gate, beta) per slot and
 *     the commit folds the accepted prefix into an fp32 checkpoint.
 * The pages never print the step equation. The one above is the plain reading
 * of "decay the state per key channel by exp(gk), delta-update it with beta,
 * k and v, read it out with q": the error is taken against the decayed state
 * and the readout uses the state after the update.
 *
 * Chunked form (kda_oracle_chunked) is the same result reorganised over
 * chunks of C tokens; it exists only so the tests can check the token loop
 * against a second, independently derived algebra.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- token-by-token recurrence ---------------------------------------- */

/* One recurrence step on S[K][V]; o_row (length V) may be NULL. */
static void step(int K, int V, const double* q, const double* k, const double* v,
                 const double* gk, double beta, double scale, double* S,
                 double* o_row, double* a, double* u) {
  for (int c = 0; c < K; ++c) a[c] = exp(gk[c]);
  for (int j = 0; j < V; ++j) u[j] = 0.0;
  for (int c = 0; c < K; ++c) {
    const double akc = a[c] * k[c];
    const double* Sc = S + (size_t)c * V;
    for (int j = 0; j < V; ++j) u[j] += akc * Sc[j];
  }
  /* u now holds the prediction; reuse it for w */
  for (int j = 0; j < V; ++j) u[j] = beta * (v[j] - u[j]);
  for (int c = 0; c < K; ++c) {
    double* Sc = S + (size_t)c * V;
    for (int j = 0; j < V; ++j) Sc[j] = a[c] * Sc[j] + k[c] * u[j];
  }
  if (o_row) {
    for (int j = 0; j < V; ++j) o_row[j] = 0.0;
    for (int c = 0; c < K; ++c) {
      const double* Sc = S + (size_t)c * V;
      for (int j = 0; j < V; ++j) o_row[j] += q[c] * Sc[j];
    }
    for (int j = 0; j < V; ++j) o_row[j] *= scale;
  }
}

/*
 * Run L tokens of one unit.
 *   q, k, gk : [L][K]      v : [L][V]      beta : [L]
 *   S        : [K][V] in/out (the caller passes state_in, or zeros)
 *   o        : [L][V] or NULL
 * Snapshots (prefix-cache checkpoints at chunk boundaries, ping-pong "extra
 * buffer" of the LMSYS post, section "Three state moves on the forward
 * stream"): if snap_interval > 0, after the token at absolute position
 * p = pos0 + t + 1 with p % snap_interval == 0, S is copied into
 * snaps[(m - 1) % snap_slots] with m = p / snap_interval, and *snap_count is
 * incremented. pos0 lets a long unit be fed in blocks.
 * Returns 0, or -1 on a bad argument.
 */
int kda_oracle_recurrent(int64_t L, int K, int V, const double* q, const double* k,
                         const double* v, const double* gk, const double* beta,
                         double scale, double* S, double* o, int64_t pos0,
                         int64_t snap_interval, int snap_slots, double* snaps,
                         int64_t* snap_count) {
  if (L < 0 || K <= 0 || V <= 0 || !S) return -1;
  if (L > 0 && (!q || !k || !v || !gk || !beta)) return -1;
  if (snap_interval > 0 && (snap_slots < 1 || !snaps)) return -1;
  double* a = (double*)malloc(sizeof(double) * (size_t)K);
  double* u = (double*)malloc(sizeof(double) * (size_t)V);
  if (!a || !u) { free(a); free(u); return -1; }
  for (int64_t t = 0; t < L; ++t) {
    step(K, V, q + t * K, k + t * K, v + t * V, gk + t * K, beta[t], scale, S,
         o ? o + t * V : NULL, a, u);
    const int64_t p = pos0 + t + 1;
    if (snap_interval > 0 && p % snap_interval == 0) {
      const int64_t m = p / snap_interval;
      memcpy(snaps + (size_t)((m - 1) % snap_slots) * K * V, S, sizeof(double) * (size_t)K * V);
      if (snap_count) ++*snap_count;
    }
  }
  free(a);
  free(u);
  return 0;
}

/*
 * Speculative verify of n_tok draft tokens (LMSYS post, section "ReplaySSM:
 * raw-input replay for the KDA state"): the same recurrence run on a private
 * copy of the committed state S0, which is never written. Each step's raw
 * inputs (v, k, gk, beta) are recorded exactly as given into ring_* (the
 * per-slot buffer of that section), in step order. If commit_len > 0, the
 * state after commit_len steps is written to S_commit ([K][V]).
 *   o : [n_tok][V] or NULL;  ring_k, ring_gk : [n_tok][K];  ring_v : [n_tok][V];
 *   ring_beta : [n_tok]. Any ring_* may be NULL (not recorded).
 */
int kda_oracle_verify(int n_tok, int K, int V, const double* q, const double* k,
                      const double* v, const double* gk, const double* beta,
                      double scale, const double* S0, double* o, int commit_len,
                      double* S_commit, double* ring_k, double* ring_v,
                      double* ring_gk, double* ring_beta) {
  if (n_tok < 0 || K <= 0 || V <= 0 || !S0 || commit_len < 0 || commit_len > n_tok) return -1;
  if (commit_len > 0 && !S_commit) return -1;
  double* S = (double*)malloc(sizeof(double) * (size_t)K * V);
  double* a = (double*)malloc(sizeof(double) * (size_t)K);
  double* u = (double*)malloc(sizeof(double) * (size_t)V);
  if (!S || !a || !u) { free(S); free(a); free(u); return -1; }
  memcpy(S, S0, sizeof(double) * (size_t)K * V);
  for (int t = 0; t < n_tok; ++t) {
    if (ring_k) memcpy(ring_k + (size_t)t * K, k + (size_t)t * K, sizeof(double) * (size_t)K);
    if (ring_v) memcpy(ring_v + (size_t)t * V, v + (size_t)t * V, sizeof(double) * (size_t)V);
    if (ring_gk) memcpy(ring_gk + (size_t)t * K, gk + (size_t)t * K, sizeof(double) * (size_t)K);
    if (ring_beta) ring_beta[t] = beta[t];
    step(K, V, q + (size_t)t * K, k + (size_t)t * K, v + (size_t)t * V, gk + (size_t)t * K,
         beta[t], scale, S, o ? o + (size_t)t * V : NULL, a, u);
    if (t + 1 == commit_len) memcpy(S_commit, S, sizeof(double) * (size_t)K * V);
  }
  free(S);
  free(a);
  free(u);
  return 0;
}

/*
 * Replay fold (LMSYS post, section "ReplaySSM: raw-input replay for the KDA
 * state"): advance the committed state S in place by the first n recorded
 * steps (the accepted prefix), using the stored (v, k, gk, beta), with no
 * readout. Rejected steps (index >= n) are never touched.
 */
int kda_oracle_fold(int n, int K, int V, const double* ring_k, const double* ring_v,
                    const double* ring_gk, const double* ring_beta, double* S) {
  if (n < 0 || K <= 0 || V <= 0 || !S) return -1;
  if (n > 0 && (!ring_k || !ring_v || !ring_gk || !ring_beta)) return -1;
  double* a = (double*)malloc(sizeof(double) * (size_t)K);
  double* u = (double*)malloc(sizeof(double) * (size_t)V);
  if (!a || !u) { free(a); free(u); return -1; }
  for (int i = 0; i < n; ++i)
    step(K, V, NULL, ring_k + (size_t)i * K, ring_v + (size_t)i * V, ring_gk + (size_t)i * K,
         ring_beta[i], 1.0, S, NULL, a, u);
  free(a);
  free(u);
  return 0;
}

/* ---- chunked form (self-check only) ------------------------------------ */

/*
 * The same result computed chunk by chunk. For a chunk of n tokens starting
 * from state S0, with G[i][c] = sum_{tau <= i} gk[tau][c] (inclusive, inside
 * the chunk):
 *   A[i][j]  = beta_i * sum_c k[i][c] k[j][c] exp(G[i][c] - G[j][c])   (j < i)
 *   (I + A) W = diag(beta) (V - Kt S0),     Kt[i][c] = k[i][c] exp(G[i][c])
 *   O[t]     = scale * ( sum_c q[t][c] exp(G[t][c]) S0[c][.]
 *                        + sum_{i <= t} P[t][i] W[i] ),
 *   P[t][i]  = sum_c q[t][c] k[i][c] exp(G[t][c] - G[i][c])
 *   S_end    = diag(exp(G[n-1])) S0 + sum_i (k[i] * exp(G[n-1] - G[i])) W[i]^T
 * W is found by forward substitution on the unit lower-triangular (I + A).
 * Argument layout as in kda_oracle_recurrent; C is the chunk length.
 */
int kda_oracle_chunked(int64_t L, int K, int V, int C, const double* q, const double* k,
                       const double* v, const double* gk, const double* beta, double scale,
                       double* S, double* o) {
  if (L < 0 || K <= 0 || V <= 0 || C <= 0 || !S) return -1;
  double* G = (double*)malloc(sizeof(double) * (size_t)C * K);
  double* A = (double*)malloc(sizeof(double) * (size_t)C * C);
  double* W = (double*)malloc(sizeof(double) * (size_t)C * V);
  double* Snew = (double*)malloc(sizeof(double) * (size_t)K * V);
  if (!G || !A || !W || !Snew) { free(G); free(A); free(W); free(Snew); return -1; }
  for (int64_t t0 = 0; t0 < L; t0 += C) {
    const int n = (int)((L - t0) < C ? (L - t0) : C);
    const double* qc = q + t0 * K;
    const double* kc = k + t0 * K;
    const double* vc = v + t0 * V;
    const double* gc = gk + t0 * K;
    const double* bc = beta + t0;
    for (int c = 0; c < K; ++c) {
      double acc = 0.0;
      for (int i = 0; i < n; ++i) { acc += gc[i * K + c]; G[i * K + c] = acc; }
    }
    for (int i = 0; i < n; ++i)
      for (int j = 0; j < n; ++j) {
        double s = 0.0;
        if (j < i)
          for (int c = 0; c < K; ++c) s += kc[i * K + c] * kc[j * K + c] * exp(G[i * K + c] - G[j * K + c]);
        A[i * C + j] = bc[i] * s;
      }
    /* right-hand side diag(beta) (V - Kt S0), then forward substitution */
    for (int i = 0; i < n; ++i) {
      for (int jv = 0; jv < V; ++jv) {
        double ks = 0.0;
        for (int c = 0; c < K; ++c) ks += kc[i * K + c] * exp(G[i * K + c]) * S[c * V + jv];
        double r = bc[i] * (vc[i * V + jv] - ks);
        for (int j = 0; j < i; ++j) r -= A[i * C + j] * W[j * V + jv];
        W[i * V + jv] = r;
      }
    }
    if (o) {
      for (int t = 0; t < n; ++t)
        for (int jv = 0; jv < V; ++jv) {
          double inter = 0.0;
          for (int c = 0; c < K; ++c) inter += qc[t * K + c] * exp(G[t * K + c]) * S[c * V + jv];
          double intra = 0.0;
          for (int i = 0; i <= t; ++i) {
            double p = 0.0;
            for (int c = 0; c < K; ++c) p += qc[t * K + c] * kc[i * K + c] * exp(G[t * K + c] - G[i * K + c]);
            intra += p * W[i * V + jv];
          }
          o[(t0 + t) * V + jv] = scale * (inter + intra);
        }
    }
    for (int c = 0; c < K; ++c) {
      const double gl = G[(n - 1) * K + c];
      for (int jv = 0; jv < V; ++jv) {
        double s = exp(gl) * S[c * V + jv];
        for (int i = 0; i < n; ++i) s += kc[i * K + c] * exp(gl - G[i * K + c]) * W[i * V + jv];
        Snew[c * V + jv] = s;
      }
    }
    memcpy(S, Snew, sizeof(double) * (size_t)K * V);
  }
  free(G);
  free(A);
  free(W);
  free(Snew);
  return 0;
}

/*
 * Output gated RMSNorm, one row of V values per (token, head):
 *   y[j] = o[j] / sqrt(mean_j' o[j']^2 + eps) * w[j] * sigmoid(g[j]),
 *   sigmoid(x) = 1 / (1 + exp(-x)).
 * Source: Kimi K3 B200 deployment notes (zdszero.github.io), the prefill /
 * decode kernel-fusion items: the KDA output goes through a gated RMSNorm
 * that reads the attention output at its native stride, the one fusion
 * allowed fast math (tolerance 8e-3). The notes name the operation but not its
 * formula; the reading here is the plain one for "RMSNorm with an output
 * gate": each row is divided by its root mean square (eps inside the root),
 * scaled per channel by a weight shared by all heads, and multiplied
 * elementwise by the logistic sigmoid of the gate.
 */
int kda_oracle_gated_rmsnorm(int64_t rows, int V, const double* o, const double* g, const double* w, double eps,
                             double* y) {
  if (rows < 0 || V < 1 || !(eps >= 0.0)) return 1;
  for (int64_t r = 0; r < rows; ++r) {
    const double* orow = o + r * V;
    const double* grow = g + r * V;
    double ss = 0.0;
    for (int j = 0; j < V; ++j) ss += orow[j] * orow[j];
    const double inv = 1.0 / sqrt(ss / V + eps);
    for (int j = 0; j < V; ++j) y[r * V + j] = orow[j] * inv * w[j] * (1.0 / (1.0 + exp(-grow[j])));
  }
  return 0;
}

/*
 * The KDA prologue for one sequence of L tokens, H heads of 128 channels (HC = 128 H channels per
 * row), conv width W (1..8):
 *   for each of the three projections x = xq, xk, xv (rows [L][HC]), with the W - 1 rows before the
 *   sequence taken from state_in ([3][W-1][HC], row W - 2 the latest):
 *     c_t[ch] = sum_{j < W} w[ch][j] * x_{t - W + 1 + j}[ch]       causal depthwise convolution
 *     u_t[ch] = c_t[ch] * sigmoid(c_t[ch])                          SiLU
 *   q_t, k_t = u_t / sqrt(sum over the head's 128 channels of u_t^2 + eps)   (per head)
 *   v_t      = u_t
 *   beta_t[h]  = sigmoid(b_raw_t[h]),   gk_t[ch] = -log(1 + exp(g_raw_t[ch]))
 *   state_out  = the last W - 1 rows of [state_in; x]   (per projection)
 * Sources: Kimi K3 B200 deployment notes (zdszero.github.io), the prefill / decode kernel-fusion
 * items: the three short conv1d calls on q, k and v with their SiLU and the conv-state carry become
 * one kernel, and the beta copy + sigmoid another, both bit-exact to the unfused path. The notes give
 * neither the conv width nor the decay-gate formula; the readings here: W is an argument (4 in the
 * tests and the bench), q and k are L2-normalised per head after the SiLU (eps inside the root), and
 * gk = -softplus(g_raw), the form under which exp(gk) = sigmoid(-g_raw) is a decay in (0, 1).
 */
int kda_oracle_prologue(int64_t L, int H, int W, const double* xq, const double* xk, const double* xv,
                        const double* conv_w, const double* state_in, const double* b_raw, const double* g_raw,
                        double eps, double* q, double* k, double* v, double* beta, double* gk, double* state_out) {
  if (L < 0 || H < 1 || W < 1 || W > 8 || !(eps >= 0.0)) return 1;
  const int64_t HC = (int64_t)H * 128;
  const double* xs[3] = {xq, xk, xv};
  double* outs[3] = {q, k, v};
  double* u = (double*)malloc(sizeof(double) * (size_t)HC);
  if (!u) return 2;
  for (int which = 0; which < 3; ++which) {
    const double* x = xs[which];
    const double* w = conv_w + (int64_t)which * HC * W;
    const double* st = state_in + (int64_t)which * (W - 1) * HC;
    for (int64_t t = 0; t < L; ++t) {
      for (int64_t ch = 0; ch < HC; ++ch) {
        double c = 0.0;
        for (int j = 0; j < W; ++j) {
          const int64_t p = t - (W - 1) + j;  // position of tap j, < 0 inside the carried state
          const double xv_ = p >= 0 ? x[p * HC + ch] : st[(p + (W - 1)) * HC + ch];
          c += w[ch * W + j] * xv_;
        }
        u[ch] = c / (1.0 + exp(-c));
      }
      for (int h = 0; h < H; ++h) {
        const double* uh = u + (int64_t)h * 128;
        double* o = outs[which] + t * HC + (int64_t)h * 128;
        if (which < 2) {
          double ss = 0.0;
          for (int j = 0; j < 128; ++j) ss += uh[j] * uh[j];
          const double inv = 1.0 / sqrt(ss + eps);
          for (int j = 0; j < 128; ++j) o[j] = uh[j] * inv;
        } else {
          for (int j = 0; j < 128; ++j) o[j] = uh[j];
        }
      }
    }
    double* so = state_out + (int64_t)which * (W - 1) * HC;
    for (int r = 0; r < W - 1; ++r) {
      const int64_t p = L - (W - 1) + r;
      for (int64_t ch = 0; ch < HC; ++ch) so[r * HC + ch] = p >= 0 ? x[p * HC + ch] : st[(p + (W - 1)) * HC + ch];
    }
  }
  for (int64_t t = 0; t < L; ++t)
    for (int h = 0; h < H; ++h) beta[t * H + h] = 1.0 / (1.0 + exp(-b_raw[t * H + h]));
  for (int64_t i = 0; i < L * HC; ++i) gk[i] = -log1p(exp(g_raw[i]));
  free(u);
  return 0;
}
