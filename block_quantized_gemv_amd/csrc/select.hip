// select.hip -- greedy argmax over logits and the MoE top-k router.
//
// argmax: the greedy pick of the "augur" README ("Features": greedy generation
// chooses the highest-probability next token) with the tie rule of "fusedtok
// 1.3.0" ("API stability": selection ties resolve to the earliest index).
// Two phases in one launch, like the "two-phase partial-scan/reduce" resident
// top1 of the cogni-ml README: each workgroup reduces a contiguous slice to
// (value, index); the last workgroup to arrive (ticket counter) reduces the
// per-workgroup results and resets the counter.  Exact float comparisons make
// the result independent of the reduction order.
//
// router: top-k of the router logits with renormalised softmax weights (the
// "#144" Qwen1.5-MoE PR: router + top-k experts), one wave.
#include <math.h>

#include "q8_internal.h"

namespace q8 {

namespace {

__device__ __forceinline__ void better(float& v, int& i, float ov, int oi) {
  if (ov > v || (ov == v && oi < i)) {
    v = ov;
    i = oi;
  }
}

__device__ __forceinline__ void wave_best(float& v, int& i) { wave_best_pair(v, i); }

constexpr int kArgThreads = 256;
constexpr int kArgPerThread = 8;

int argmax_groups(int64_t n) {
  int64_t g = cdiv(n, (int64_t)kArgThreads * kArgPerThread);
  if (g < 1) g = 1;
  if (g > 1024) g = 1024;
  return (int)g;
}

}  // namespace

__global__ __launch_bounds__(kArgThreads) void argmax_kernel(const float* __restrict__ v, int n,
                                                             int32_t* out, uint32_t* ticket,
                                                             float* wv, int32_t* wi) {
  __shared__ float sv[kArgThreads / 64];
  __shared__ int si[kArgThreads / 64];
  __shared__ int s_last;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // contiguous slice per workgroup, strided by the workgroup's threads
  const int per = (int)(((int64_t)n + gridDim.x - 1) / gridDim.x);
  const int lo = blockIdx.x * per;
  const int hi = min(n, lo + per);
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  // kArgPerThread loads per thread are issued before any compare (one memory
  // round trip per batch rather than one per element)
  for (int i0 = lo + (int)threadIdx.x; i0 < hi; i0 += kArgThreads * kArgPerThread) {
    float tv[kArgPerThread];
#pragma unroll
    for (int j = 0; j < kArgPerThread; ++j) {
      const int i = i0 + j * kArgThreads;
      tv[j] = i < hi ? v[i] : -INFINITY;
    }
#pragma unroll
    for (int j = 0; j < kArgPerThread; ++j) {
      const int i = i0 + j * kArgThreads;
      if (i < hi) better(bv, bi, tv[j], i);
    }
  }
  wave_best(bv, bi);
  if (lane == 0) {
    sv[wave] = bv;
    si[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kArgThreads / 64; ++w) better(bv, bi, sv[w], si[w]);
    st_dev(wv + blockIdx.x, bv);
    st_dev(wi + blockIdx.x, bi);
    wait_stores();
    s_last = ticket_add(ticket) == gridDim.x - 1;
  }
  __syncthreads();
  if (!s_last || wave != 0) return;
  bv = -INFINITY;
  bi = 0x7fffffff;
  for (int g0 = 0; g0 < (int)gridDim.x; g0 += 256) {
    float tv[4];
    int ti[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int g = g0 + 64 * j + lane;
      tv[j] = g < (int)gridDim.x ? ld_dev(wv + g) : -INFINITY;
      ti[j] = g < (int)gridDim.x ? ld_dev(wi + g) : 0x7fffffff;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) better(bv, bi, tv[j], ti[j]);
  }
  wave_best(bv, bi);
  if (lane == 0) {
    *out = bi;
    st_dev(ticket, 0u);
  }
}

size_t argmax_ws_bytes(int64_t n) {
  if (n <= 0) return 0;
  const size_t g = (size_t)argmax_groups(n);
  return kCounterBytes + align_up(g * 4, 256) * 2;
}

int launch_argmax(const float* v, int64_t n, int32_t* out, void* ws, size_t ws_bytes,
                  hipStream_t stream) {
  if (n <= 0) return Q8_OK;
  if (!ws || ws_bytes < argmax_ws_bytes(n)) return Q8_EWORKSPACE;
  const int g = argmax_groups(n);
  uint8_t* base = static_cast<uint8_t*>(ws);
  auto* ticket = reinterpret_cast<uint32_t*>(base);  // counter 0
  auto* wv = reinterpret_cast<float*>(base + kCounterBytes);
  auto* wi = reinterpret_cast<int32_t*>(base + kCounterBytes + align_up((size_t)g * 4, 256));
  hipLaunchKernelGGL(argmax_kernel, dim3(g), dim3(kArgThreads), 0, stream, v, (int)n, out, ticket,
                     wv, wi);
  return hipGetLastError() == hipSuccess ? Q8_OK : Q8_ELAUNCH;
}

// One wave; lane l holds logits l, l+64, ... (E <= 1024).
__global__ __launch_bounds__(64) void route_kernel(const float* __restrict__ logits, int E, int k,
                                                   int32_t* ids, float* w) {
  float sel_v[Q8_MAX_SLOTS];
  int sel_i[Q8_MAX_SLOTS];
  route_topk_wave(logits, E, k, threadIdx.x, sel_v, sel_i);
  if (threadIdx.x == 0) route_store(sel_v, sel_i, k, ids, w);
}

int launch_route(const float* logits, int32_t E, int32_t k, int32_t* ids, float* w,
                 hipStream_t stream) {
  hipLaunchKernelGGL(route_kernel, dim3(1), dim3(64), 0, stream, logits, E, k, ids, w);
  return hipGetLastError() == hipSuccess ? Q8_OK : Q8_ELAUNCH;
}

}  // namespace q8
