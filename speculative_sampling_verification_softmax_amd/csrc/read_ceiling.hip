// read_ceiling.hip -- measurement probe, not part of the verify path: plain
// streaming reads of a device buffer with the access pattern of the stats
// kernel (16-byte non-temporal loads), so that the rate the stats kernel
// reaches can be compared with what this part delivers to a kernel that does
// nothing but read (and, one shape, the same reads with the default cache
// policy).  Built as its own library (libspec_probe.so) and loaded
// by the benchmark only.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace spec_probe {

__device__ __forceinline__ unsigned fold4(const uint4& v) { return v.x ^ v.y ^ v.z ^ v.w; }

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Grid-stride: thread i reads vectors i, i + S, i + 2S, ... (S = all threads),
// DEPTH of them in flight; one word per workgroup is written so the loads
// cannot be dropped.
template <int DEPTH>
__global__ __launch_bounds__(1024) void read_grid_stride(const uint4* __restrict__ p, size_t nvec,
                                                         unsigned* __restrict__ sink) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  unsigned acc = 0;
  for (; i + (DEPTH - 1) * stride < nvec; i += DEPTH * stride) {
    uint4 v[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) v[d] = load_nt(p + i + d * stride);
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) acc ^= fold4(v[d]);
  }
  for (; i < nvec; i += stride) acc ^= fold4(load_nt(p + i));
  __shared__ unsigned red[16];
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned r = 0;
    for (int w = 0; w < static_cast<int>(blockDim.x / 64); ++w) r ^= red[w];
    sink[blockIdx.x] = r;
  }
}

__device__ __forceinline__ uint4 load_cached(const uint4* p) { return *p; }

// One row per workgroup, as the stats kernel streams: groups of 4 vectors
// per thread, the next group's loads issued before the current one is used;
// NT: non-temporal loads (as the stats kernel), else the default policy.
template <bool NT>
__global__ __launch_bounds__(1024) void read_rows(const uint4* __restrict__ p, size_t row_vec,
                                                  unsigned* __restrict__ sink) {
  auto load = [](const uint4* q) { return NT ? load_nt(q) : load_cached(q); };
  const uint4* row = p + static_cast<size_t>(blockIdx.x) * row_vec;
  constexpr int G = 4;
  const size_t step = static_cast<size_t>(blockDim.x) * G;
  unsigned acc = 0;
  size_t i = threadIdx.x;
  uint4 v[G];
  bool have = i + (G - 1) * blockDim.x < row_vec;
  if (have)
#pragma unroll
    for (int g = 0; g < G; ++g) v[g] = load(row + i + g * blockDim.x);
  while (have) {
    uint4 cur[G];
#pragma unroll
    for (int g = 0; g < G; ++g) cur[g] = v[g];
    i += step;
    have = i + (G - 1) * blockDim.x < row_vec;
    if (have)
#pragma unroll
      for (int g = 0; g < G; ++g) v[g] = load(row + i + g * blockDim.x);
#pragma unroll
    for (int g = 0; g < G; ++g) acc ^= fold4(cur[g]);
  }
  for (; i < row_vec; i += blockDim.x) acc ^= fold4(load(row + i));
  __shared__ unsigned red[16];
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned r = 0;
    for (int w = 0; w < static_cast<int>(blockDim.x / 64); ++w) r ^= red[w];
    sink[blockIdx.x] = r;
  }
}

}  // namespace spec_probe

using spec_probe::read_grid_stride;
using spec_probe::read_rows;

extern "C" {

// Reads `bytes` (a multiple of 16) at the 16-byte aligned device address p.
//   mode 0: grid-stride, 8 loads in flight per thread, `groups` workgroups
//   mode 1: grid-stride, 4 loads in flight per thread
//   mode 2: one row of bytes/groups bytes per workgroup (a multiple of 16)
//   mode 3: as mode 2 with default (cached) loads
//   mode 4: as mode 2 with 512-thread workgroups (1024 threads otherwise)
// sink: device memory of at least `groups` words.  Returns 0, or 1 for bad
// arguments, 3 for a failed launch.
int spec_probe_read(const void* p, size_t bytes, int mode, int groups, unsigned* sink,
                    void* stream) {
  if (!p || !sink || groups < 1 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(p) & 15))
    return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint4* v = static_cast<const uint4*>(p);
  const size_t nvec = bytes / 16;
  (void)hipGetLastError();
  if (mode == 0) {
    hipLaunchKernelGGL(read_grid_stride<8>, dim3(groups), dim3(1024), 0, s, v, nvec, sink);
  } else if (mode == 1) {
    hipLaunchKernelGGL(read_grid_stride<4>, dim3(groups), dim3(1024), 0, s, v, nvec, sink);
  } else if (mode == 2 || mode == 3 || mode == 4) {
    if (nvec % static_cast<size_t>(groups) != 0) return 1;
    if (mode == 2 || mode == 4)
      hipLaunchKernelGGL(read_rows<true>, dim3(groups), dim3(mode == 4 ? 512 : 1024), 0, s, v,
                         nvec / groups, sink);
    else
      hipLaunchKernelGGL(read_rows<false>, dim3(groups), dim3(1024), 0, s, v, nvec / groups, sink);
  } else {
    return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
