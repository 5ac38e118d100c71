/*
 * synth.c -- host build of the seeded input generator (see synth_core.h for
 * the element recipe and the published methods it follows).
 *
 * This module is shared by the CPU oracle side and the GPU side: both consume
 * the arrays it writes (the device build, synth_gpu.hip, writes the same
 * values straight into device memory). It holds no arithmetic of the
 * recurrence, only input distributions.
 *
 * Element e of the logical tensor (seed, tid, sub) uses Philox block
 *     counter = (p mod 2^32, p div 2^32, sub, seed div 2^32),
 *     key     = (seed mod 2^32, tid),          p = e div 2,
 * and takes the cosine (e even) or sine (e odd) Box-Muller deviate.
 */
#include <stdint.h>
#include <omp.h>

#include "synth_core.h"

void synth_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  uint32_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
  syn_philox(c, key_in[0], key_in[1]);
  for (int i = 0; i < 4; ++i) out[i] = c[i];
}

uint16_t synth_bf16_rne(double x) { return syn_bf16(x); }
double synth_log(double x) { return syn_log(x); }
double synth_exp(double x) { return syn_exp(x); }
double synth_sqrt(double x) { return syn_sqrt(x); }
double synth_log1p01(double x) { return syn_log1p01(x); }
void synth_sincos_2pi(double u, double* s, double* c) { syn_sincos_2pi(u, s, c); }

static inline void store(void* out, int dtype, int64_t i, double x) {
  if (dtype == SYN_F64) ((double*)out)[i] = x;
  else if (dtype == SYN_F32) ((float*)out)[i] = syn_f32(x);
  else ((uint16_t*)out)[i] = syn_bf16(x);
}

/*
 * Fill out[n_rows][row_len] (contiguous, in dtype) with rows
 * r = row_start + i*row_step of the logical tensor (seed, tid, sub) whose
 * flat element index is r*row_len + c.
 *   SYN_NORMAL:       scale * z
 *   SYN_UNIT_ROW:     z / ||z||_2 over the row (sum of squares in index order)
 *   SYN_NEG_SOFTPLUS: -softplus(z)
 *   SYN_SIGMOID:      1 / (1 + exp(-z))
 * Returns 0, or -1 on a bad argument.
 */
int synth_fill(uint64_t seed, uint32_t tid, uint32_t sub, int kind, int dtype,
               int64_t row_start, int64_t row_step, int64_t n_rows, int row_len,
               double scale, void* out) {
  if (n_rows < 0 || row_len <= 0 || row_len > 4096 || dtype < 0 || dtype > 2 || kind < 0 || kind > 3) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n_rows; ++i) {
    const int64_t e0 = (row_start + i * row_step) * (int64_t)row_len;
    double buf[4096];
    for (int c = 0; c < row_len; ++c) {
      const int64_t e = e0 + c;
      double z0, z1;
      syn_normal_pair(seed, tid, sub, (uint64_t)(e >> 1), &z0, &z1);
      if ((e & 1) == 0 && c + 1 < row_len) {
        buf[c] = z0;
        buf[c + 1] = z1;
        ++c;
      } else {
        buf[c] = (e & 1) ? z1 : z0;
      }
    }
    const int64_t o = i * (int64_t)row_len;
    if (kind == SYN_UNIT_ROW) {
      double ss = 0.0;
      for (int c = 0; c < row_len; ++c) ss = ss + buf[c] * buf[c];
      const double nrm = syn_sqrt(ss);
      for (int c = 0; c < row_len; ++c) store(out, dtype, o + c, buf[c] / nrm);
    } else {
      for (int c = 0; c < row_len; ++c) {
        const double z = buf[c];
        double x;
        if (kind == SYN_NORMAL) x = scale * z;
        else if (kind == SYN_NEG_SOFTPLUS) x = syn_neg_softplus(z);
        else x = syn_sigmoid(z);
        store(out, dtype, o + c, x);
      }
    }
  }
  return 0;
}

/* n uniforms in (0, 1] for flat indices start..start+n-1 of (seed, tid, sub) */
int synth_uniform(uint64_t seed, uint32_t tid, uint32_t sub, int64_t start, int64_t n, double* out) {
  if (n < 0) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = syn_uniform(seed, tid, sub, (uint64_t)(start + i));
  return 0;
}

/* exact bf16 (RNE) rounding of an fp64 array, exported for tests */
void synth_round_bf16(const double* x, uint16_t* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = syn_bf16(x[i]);
}

int synth_max_threads(void) { return omp_get_max_threads(); }
