// kda_move.hip -- the state moves of the prefix-cache protocol as one stream-ordered copy launch: each
// move copies one whole slot of the state pool (every layer and head of a request) to another.
//
// Source: "SGLang and Miles Add Day-0 Support for Kimi K3" (LMSYS blog), section "Hybrid KDA Memory
// Management", subsection on the three state moves: the copy-on-write restore of a cached checkpoint
// into a working slot and the snapshot of a working slot are kernels on the serial forward stream, so
// stream order alone orders them against the forwards that produce and consume the state.
//
// Grid: y = move (strided when there are more than 65,535), x = pieces of the slot; each thread copies
// float4s with four loads in flight, non-temporal on both sides (the pool is read and written once).
// A move whose source or destination is outside [0, n_slots), or whose source is its destination, is
// skipped, so no move value addresses memory outside the pool.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) state_move_kernel(const kda_move* __restrict__ moves, int n_moves, int n_slots,
                                                         int64_t slot_f4, f32x4v* __restrict__ pool) {
  for (int m = blockIdx.y; m < n_moves; m += gridDim.y) {
    const int src = moves[m].src, dst = moves[m].dst;
    if (src < 0 || src >= n_slots || dst < 0 || dst >= n_slots || src == dst) continue;  // uniform
    const f32x4v* s = pool + (int64_t)src * slot_f4;
    f32x4v* d = pool + (int64_t)dst * slot_f4;
    const int64_t step = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + 3 * step < slot_f4; i += 4 * step) {
      f32x4v v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(s + i + u * step);
#pragma unroll
      for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(v[u], d + i + u * step);
    }
    for (; i < slot_f4; i += step) __builtin_nontemporal_store(__builtin_nontemporal_load(s + i), d + i);
  }
}

}  // namespace

hipError_t launch_state_move(int n_moves, const kda_move* moves, int n_slots, int64_t slot_floats, float* pool,
                             hipStream_t stream) {
  if (n_moves <= 0) return hipSuccess;
  const int64_t slot_f4 = slot_floats / 4;
  // about 8,192 workgroups in all, at most one per 4,096 float4s of a slot
  const int64_t per_move = std::max<int64_t>(1, std::min<int64_t>((slot_f4 + 4095) / 4096, (8192 + n_moves - 1) / n_moves));
  const dim3 grid((unsigned)per_move, (unsigned)std::min(n_moves, 65535));
  hipLaunchKernelGGL(state_move_kernel, grid, dim3(256), 0, stream, moves, n_moves, n_slots, slot_f4,
                     reinterpret_cast<f32x4v*>(pool));
  return hipGetLastError();
}

}  // namespace kda
