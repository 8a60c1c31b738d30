// HBM read-bandwidth calibration: how fast plain 16-byte loads stream a
// device buffer on this GPU, with no other work per byte. It measures what
// the row kernels' roofline fraction is set against; it is not part of the
// verification path and lives in its own library (libsvcalib.so).
//
// Two access shapes:
//   mode 0  grid-stride: every workgroup walks the whole buffer with stride
//           grid * threads * 16 bytes (consecutive workgroups read adjacent
//           lines at any moment);
//   mode 1  one contiguous chunk per workgroup, the shape of the row kernels
//           (one logit row per workgroup, 512 threads, eight 16-byte loads in
//           flight per thread).
// Each thread folds what it reads with XOR and writes one word per workgroup,
// so no load can be dropped.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace svcal {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int RC_THREADS = 512;
constexpr int RC_UNROLL = 8;

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

__device__ __forceinline__ void block_out(uint32_t acc, uint32_t* out) {
  __shared__ uint32_t part[RC_THREADS / 64];
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x / 64] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < RC_THREADS / 64; ++w) r ^= part[w];
    out[blockIdx.x] = r;
  }
}

__global__ __launch_bounds__(RC_THREADS) void read_stride_kernel(const u32x4* p, int64_t n16,
                                                                 uint32_t* out) {
  const int64_t stride = (int64_t)gridDim.x * RC_THREADS;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * RC_THREADS + threadIdx.x;
  for (; i + (RC_UNROLL - 1) * stride < n16; i += RC_UNROLL * stride) {
    u32x4 v[RC_UNROLL];
#pragma unroll
    for (int u = 0; u < RC_UNROLL; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < RC_UNROLL; ++u) acc ^= fold(v[u]);
  }
  for (; i < n16; i += stride) acc ^= fold(__builtin_nontemporal_load(p + i));
  block_out(acc, out);
}

__global__ __launch_bounds__(RC_THREADS) void read_chunk_kernel(const u32x4* p, int64_t n16,
                                                                int64_t chunk16, uint32_t* out) {
  const int64_t c0 = (int64_t)blockIdx.x * chunk16;
  const int64_t c1 = c0 + chunk16 < n16 ? c0 + chunk16 : n16;
  const u32x4* q = p + c0;
  const int64_t n = c1 - c0;
  uint32_t acc = 0;
  for (int64_t k0 = threadIdx.x; k0 < n; k0 += RC_THREADS * RC_UNROLL) {
    u32x4 v[RC_UNROLL];
#pragma unroll
    for (int u = 0; u < RC_UNROLL; ++u) {
      const int64_t k = k0 + u * RC_THREADS;
      v[u] = k < n ? __builtin_nontemporal_load(q + k) : (u32x4){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < RC_UNROLL; ++u) acc ^= fold(v[u]);
  }
  block_out(acc, out);
}

}  // namespace svcal

// Number of output words (workgroups) a call with these arguments writes.
extern "C" int64_t sv_calib_read_blocks(int64_t bytes, int mode, int64_t chunk_bytes, int grid) {
  if (bytes <= 0 || (bytes & 15)) return -1;
  if (mode == 0) return grid > 0 ? grid : -1;
  if (mode == 1) {
    if (chunk_bytes <= 0 || (chunk_bytes & 15)) return -1;
    return (bytes + chunk_bytes - 1) / chunk_bytes;
  }
  return -1;
}

// Reads `bytes` (a multiple of 16) from the 16-byte aligned device buffer
// `buf` and writes one word per workgroup to `out` (sv_calib_read_blocks
// words). mode 0: grid-stride with `grid` workgroups; mode 1: one workgroup
// per `chunk_bytes` (a multiple of 16). Returns 0, -1 on bad arguments, -5 on
// a launch error. Asynchronous on `stream`.
extern "C" int sv_calib_read(const void* buf, int64_t bytes, int mode, int64_t chunk_bytes,
                             int grid, uint32_t* out, void* stream) {
  const int64_t nb = sv_calib_read_blocks(bytes, mode, chunk_bytes, grid);
  if (nb < 1 || nb > INT32_MAX || !buf || !out || ((uintptr_t)buf & 15)) return -1;
  const hipStream_t st = (hipStream_t)stream;
  const int64_t n16 = bytes / 16;
  if (mode == 0)
    hipLaunchKernelGGL(svcal::read_stride_kernel, dim3((unsigned)nb), dim3(svcal::RC_THREADS), 0,
                       st, (const svcal::u32x4*)buf, n16, out);
  else
    hipLaunchKernelGGL(svcal::read_chunk_kernel, dim3((unsigned)nb), dim3(svcal::RC_THREADS), 0,
                       st, (const svcal::u32x4*)buf, n16, chunk_bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
