// Small wavefront / workgroup primitives shared by the kernels (gfx950,
// 64-lane wavefronts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fvattn {

constexpr int kWave = 64;

__device__ inline int lane_id() { return __lane_id(); }

// Inclusive prefix sum across the 64 lanes of a wavefront.
template <typename T>
__device__ inline T wave_inclusive_scan(T v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    T u = __shfl_up(v, off, kWave);
    if (lane >= off) v += u;
  }
  return v;
}

template <typename T>
__device__ inline T wave_sum(T v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

template <typename T>
__device__ inline T wave_max(T v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off, kWave));
  return v;
}

template <typename T>
__device__ inline T wave_min(T v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v = min(v, __shfl_xor(v, off, kWave));
  return v;
}

// Exclusive prefix sum over a workgroup of NT threads (NT a multiple of 64,
// at most 1024).  `total` receives the sum of all inputs.  Every thread of
// the workgroup must call it; `scratch` holds NT/64 entries.
template <int NT, typename T>
__device__ inline T block_exclusive_scan(T v, T* scratch, T& total) {
  constexpr int NW = NT / kWave;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  T inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) scratch[wave] = inc;
  __syncthreads();
  T base = 0;
  T all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    T s = scratch[w];
    if (w < wave) base += s;
    all += s;
  }
  __syncthreads();
  total = all;
  return base + inc - v;
}

// Workgroup-wide reductions; results are returned to every thread.
template <int NT, typename T, typename Op>
__device__ inline T block_reduce(T v, T* scratch, Op op) {
  constexpr int NW = NT / kWave;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v = op(v, __shfl_xor(v, off, kWave));
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  T r = scratch[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = op(r, scratch[w]);
  __syncthreads();
  return r;
}

}  // namespace fvattn
