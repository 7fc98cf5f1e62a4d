// calib.hip -- the on-box reference for "achievable HBM read bandwidth": a
// plain streaming read-reduce, against which the GEMV rows are judged.  It
// reads `bytes` with 16-byte non-temporal loads (global_load_dwordx4, the
// same instruction the GEMV streams its weights with), 8 in flight per lane,
// grid-stride, and folds them into one word so the reads cannot be dropped.
#include "q8_internal.h"

namespace q8 {
namespace {

constexpr int kReadUnroll = 8;

__global__ __launch_bounds__(512) void read_reduce_kernel(const u32x4* __restrict__ p, int64_t n16,
                                                          uint32_t* out) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  int64_t i = tid;
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // one word per workgroup survives: the XOR of everything it read
  __shared__ uint32_t s;
  if (threadIdx.x == 0) s = 0;
  __syncthreads();
  atomicXor(&s, acc);
  __syncthreads();
  if (threadIdx.x == 0) atomicXor(out, s);
}

}  // namespace

int launch_read_reduce(const void* buf, int64_t bytes, uint32_t* out, int grid,
                       hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  if (n16 <= 0) return Q8_OK;
  hipLaunchKernelGGL(read_reduce_kernel, dim3(grid), dim3(512), 0, stream,
                     static_cast<const u32x4*>(buf), n16, out);
  return hipGetLastError() == hipSuccess ? Q8_OK : Q8_ELAUNCH;
}

}  // namespace q8
