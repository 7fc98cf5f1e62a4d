// calib.hip -- the on-box reference for "achievable HBM read bandwidth": a
// plain streaming read, against which the GEMV rows are judged.  Each
// workgroup of 256 threads reads one contiguous chunk of the buffer with
// 16-byte non-temporal loads (global_load_dwordx4, the instruction the GEMV
// streams its weights with), 4 in flight per lane; a contiguous chunk per
// workgroup keeps a workgroup's requests within few DRAM pages (bench.py's
// read-reference rows: 6.4-6.8 TB/s over 2 GiB).
// The workgroup's XOR of every word it read goes to out[blockIdx.x] with a
// plain store, so no read can be dropped and the host can check that every
// word was read exactly once; no atomics, which would serialise the end of
// the kernel on one address.
#include "q8_internal.h"

namespace q8 {
namespace {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 4;

__global__ __launch_bounds__(kReadThreads) void read_reduce_kernel(const u32x4* __restrict__ p,
                                                                   int64_t n16, int64_t chunk,
                                                                   uint32_t* out) {
  const int64_t b = (int64_t)blockIdx.x * chunk;
  const int64_t e = b + chunk < n16 ? b + chunk : n16;
  uint32_t acc = 0;
  int64_t i = b + threadIdx.x;
  for (; i + (kReadUnroll - 1) * kReadThreads < e; i += kReadUnroll * kReadThreads) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u)
      v[u] = __builtin_nontemporal_load(p + i + u * kReadThreads);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < e; i += kReadThreads) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // XOR over the wave, then over the workgroup's 4 waves
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= __shfl_xor(acc, m, 64);
  __shared__ uint32_t s[kReadThreads / 64];
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = s[0] ^ s[1] ^ s[2] ^ s[3];
}

}  // namespace

int launch_read_reduce(const void* buf, int64_t bytes, uint32_t* out, int grid,
                       hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  // chunk: a whole number of the workgroup's 256-load sweeps
  const int64_t per = cdiv(n16, (int64_t)grid);
  const int64_t chunk = cdiv(per, (int64_t)kReadThreads) * kReadThreads;
  hipLaunchKernelGGL(read_reduce_kernel, dim3(grid), dim3(kReadThreads), 0, stream,
                     static_cast<const u32x4*>(buf), n16, chunk, out);
  return hipGetLastError() == hipSuccess ? Q8_OK : Q8_ELAUNCH;
}

}  // namespace q8
