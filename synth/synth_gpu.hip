/*
 * synth_gpu.hip -- device build of the seeded input generator.
 *
 * Writes the same values as synth.c (host build) straight into device
 * memory: both builds evaluate synth_core.h with IEEE basic operations only
 * and -ffp-contract=off, so they agree bit for bit. Holds input
 * distributions only, no arithmetic of the recurrence.
 */
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "synth_core.h"

__device__ static inline void put(void* out, int dtype, int64_t i, double x) {
  if (dtype == SYN_F64) ((double*)out)[i] = x;
  else if (dtype == SYN_F32) ((float*)out)[i] = syn_f32(x);
  else ((uint16_t*)out)[i] = syn_bf16(x);
}

/* one thread per row; the row's elements are produced in index order */
__global__ void __launch_bounds__(256) synth_fill_rows(uint64_t seed, uint32_t tid, uint32_t sub, int kind,
                                                       int dtype, int64_t row_start, int64_t row_step,
                                                       int64_t n_rows, int row_len, double scale,
                                                       void* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_rows) return;
  const int64_t e0 = (row_start + i * row_step) * (int64_t)row_len;
  const int64_t o = i * (int64_t)row_len;
  double nrm = 1.0;
  if (kind == SYN_UNIT_ROW) {
    double ss = 0.0;
    for (int c = 0; c < row_len; ++c) {
      const int64_t e = e0 + c;
      double z0, z1;
      syn_normal_pair(seed, tid, sub, (uint64_t)(e >> 1), &z0, &z1);
      if ((e & 1) == 0 && c + 1 < row_len) {
        ss = ss + z0 * z0;
        ss = ss + z1 * z1;
        ++c;
      } else {
        const double z = (e & 1) ? z1 : z0;
        ss = ss + z * z;
      }
    }
    nrm = syn_sqrt(ss);
  }
  for (int c = 0; c < row_len; ++c) {
    const int64_t e = e0 + c;
    double z0, z1;
    syn_normal_pair(seed, tid, sub, (uint64_t)(e >> 1), &z0, &z1);
    double zz[2];
    int n = 1;
    if ((e & 1) == 0 && c + 1 < row_len) { zz[0] = z0; zz[1] = z1; n = 2; }
    else zz[0] = (e & 1) ? z1 : z0;
    for (int m = 0; m < n; ++m) {
      const double z = zz[m];
      double x;
      if (kind == SYN_UNIT_ROW) x = z / nrm;
      else if (kind == SYN_NORMAL) x = scale * z;
      else if (kind == SYN_NEG_SOFTPLUS) x = syn_neg_softplus(z);
      else x = syn_sigmoid(z);
      put(out, dtype, o + c + m, x);
    }
    c += n - 1;
  }
}

/*
 * C ABI: fill dev_out[n_rows][row_len] (device memory, dtype elements) with
 * rows r = row_start + i*row_step of the logical tensor (seed, tid, sub), on
 * `stream` (a hipStream_t, may be NULL). Same semantics as synth_fill.
 * Returns 0, -1 on a bad argument, -2 if the launch failed.
 */
extern "C" int synth_gpu_fill(uint64_t seed, uint32_t tid, uint32_t sub, int kind, int dtype,
                              int64_t row_start, int64_t row_step, int64_t n_rows, int row_len,
                              double scale, void* dev_out, void* stream) {
  if (n_rows < 0 || row_len <= 0 || row_len > 4096 || dtype < 0 || dtype > 2 || kind < 0 || kind > 3) return -1;
  if (n_rows == 0) return 0;
  if (!dev_out) return -1;
  const int64_t blocks = (n_rows + 255) / 256;
  if (blocks > 0x7fffffffLL) return -1;
  hipLaunchKernelGGL(synth_fill_rows, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, seed, tid,
                     sub, kind, dtype, row_start, row_step, n_rows, row_len, scale, dev_out);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
