// repack.hip -- load-time repack of GGUF Q8_0 blocks into the packed layout.
//
// GGUF stores a Q8_0 matrix as an array of 34-byte blocks (binary16 scale,
// then 32 signed quants; "skuznetsov/cogni-ml" README, cuda_q8_gemv_probe:
// "raw GGUF Q8_0 block layout").  The 34-byte stride leaves every block only
// 2-byte aligned, so the decode kernels cannot stream it with 16-byte loads.
// This kernel moves the bytes (no value changes) into:
//   qs: per 64-row tile, per 16-weight chunk, the 16 bytes of each of the 64
//       rows back to back (1 KiB per chunk per tile);
//   d:  per 64-row tile, per quad of 4 blocks, the 4 scales of each of the 64
//       rows back to back (512 B per quad per tile).
// Padding rows and blocks are written as zeros.  With the gate/up pairs layout
// packed row 64t + i holds matrix row 32t + i (i < 32) or M/2 + 32t + i - 32.
#include "q8_internal.h"

namespace q8 {

// Matrix row held by packed row p.
__device__ __forceinline__ int64_t src_row(int64_t p, int64_t M, int32_t layout) {
  if (layout != Q8_LAYOUT_GATE_UP_PAIRS) return p;
  const int64_t t = p >> 6, i = p & 63;
  return i < 32 ? 32 * t + i : M / 2 + 32 * t + (i - 32);
}

__global__ __launch_bounds__(256) void repack_qs_kernel(const uint16_t* __restrict__ aos16,
                                                        int64_t M, int64_t K, int32_t layout,
                                                        u32x4* __restrict__ qs, int64_t total) {
  const int64_t nchunk = K / 16;
  const int64_t nb = K / 32;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t lane = idx & 63;
    const int64_t c = (idx >> 6) % nchunk;
    const int64_t t = (idx >> 6) / nchunk;
    const int64_t pr = t * 64 + lane;
    const int64_t r = src_row(pr, M, layout);
    u32x4 out = {0u, 0u, 0u, 0u};
    if (pr < M) {
      // quants of block c/2 start 1 uint16 after the block's scale
      const uint16_t* src = aos16 + (r * nb + c / 2) * 17 + 1 + (c & 1) * 8;
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = (uint32_t)src[2 * i] | ((uint32_t)src[2 * i + 1] << 16);
      out = u32x4{w[0], w[1], w[2], w[3]};
    }
    qs[idx] = out;
  }
}

__global__ __launch_bounds__(256) void repack_d_kernel(const uint16_t* __restrict__ aos16,
                                                       int64_t M, int64_t K, int32_t layout,
                                                       u32x2* __restrict__ d, int64_t total) {
  const int64_t nb = K / 32;
  const int64_t G = (nb + 3) / 4;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t lane = idx & 63;
    const int64_t g = (idx >> 6) % G;
    const int64_t t = (idx >> 6) / G;
    const int64_t pr = t * 64 + lane;
    const int64_t r = src_row(pr, M, layout);
    uint32_t bits[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t b = 4 * g + j;
      bits[j] = (pr < M && b < nb) ? aos16[(r * nb + b) * 17] : 0u;
    }
    d[idx] = u32x2{bits[0] | (bits[1] << 16), bits[2] | (bits[3] << 16)};
  }
}

int launch_repack(const void* aos, int64_t M, int64_t K, int32_t layout, void* qs, void* d,
                  hipStream_t stream) {
  const int64_t T = cdiv(M, kTile);
  const int64_t nq = T * 64 * (K / 16);
  const int64_t nd = T * 64 * cdiv(K / 32, 4);
  const auto* a16 = static_cast<const uint16_t*>(aos);
  auto grid = [](int64_t n) { return (unsigned)(n / 256 + 1 < 65536 ? n / 256 + 1 : 65536); };
  hipLaunchKernelGGL(repack_qs_kernel, dim3(grid(nq)), dim3(256), 0, stream, a16, M, K, layout,
                     static_cast<u32x4*>(qs), nq);
  if (hipGetLastError() != hipSuccess) return Q8_ELAUNCH;
  hipLaunchKernelGGL(repack_d_kernel, dim3(grid(nd)), dim3(256), 0, stream, a16, M, K, layout,
                     static_cast<u32x2*>(d), nd);
  return hipGetLastError() == hipSuccess ? Q8_OK : Q8_ELAUNCH;
}

// ---- Q4_K ------------------------------------------------------------------
// GGUF Q4_K blocks ("skuznetsov/cogni-ml" README, cuda_q4k_gemv_probe: d,
// dmin, 12-byte packed scales/mins, 128-byte packed nibbles; 144 bytes per 256
// weights of one row) move into:
//   qs:   per 64-row tile, per 32-weight sub-block, 16 bytes of each of the 64
//         rows back to back; byte i holds the sub-block's weights i (low
//         nibble) and i + 16 (high nibble).  In a GGUF block, sub-block j's
//         weights are the low (j even) or high (j odd) nibbles of the 32 bytes
//         at 16 + 32 * (j / 2).
//   meta: per 64-row tile, per 256-weight block, the block's first 16 bytes
//         (d, dmin, the 12 scale/min bytes) of each of the 64 rows.
// Byte moves and nibble moves only; padding rows are zeros.
__global__ __launch_bounds__(256) void q4k_repack_qs_kernel(const uint32_t* __restrict__ src,
                                                            int64_t M, int64_t K,
                                                            u32x4* __restrict__ qs,
                                                            int64_t total) {
  const int64_t nsub = K / 32, nsb = K / 256;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t lane = idx & 63;
    const int64_t c = (idx >> 6) % nsub;
    const int64_t t = (idx >> 6) / nsub;
    const int64_t r = t * 64 + lane;
    u32x4 out = {0u, 0u, 0u, 0u};
    if (r < M) {
      const int j = (int)(c & 7);
      // the 32 bytes of sub-block pair j / 2 (144-byte blocks: dword aligned)
      const uint32_t* g = src + ((r * nsb + c / 8) * 144 + 16 + 32 * (j >> 1)) / 4;
      const int sh = (j & 1) * 4;
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = ((g[i] >> sh) & 0x0F0F0F0Fu) | (((g[4 + i] >> sh) & 0x0F0F0F0Fu) << 4);
      out = u32x4{o[0], o[1], o[2], o[3]};
    }
    qs[idx] = out;
  }
}

__global__ __launch_bounds__(256) void q4k_repack_meta_kernel(const uint32_t* __restrict__ src,
                                                              int64_t M, int64_t K,
                                                              u32x4* __restrict__ meta,
                                                              int64_t total) {
  const int64_t nsb = K / 256;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t lane = idx & 63;
    const int64_t b = (idx >> 6) % nsb;
    const int64_t t = (idx >> 6) / nsb;
    const int64_t r = t * 64 + lane;
    u32x4 out = {0u, 0u, 0u, 0u};
    if (r < M) {
      const uint32_t* h = src + (r * nsb + b) * 144 / 4;
      out = u32x4{h[0], h[1], h[2], h[3]};
    }
    meta[idx] = out;
  }
}

int launch_q4k_repack(const void* blocks, int64_t M, int64_t K, void* qs, void* meta,
                      hipStream_t stream) {
  const int64_t T = cdiv(M, kTile);
  const int64_t nq = T * 64 * (K / 32);
  const int64_t nm = T * 64 * (K / 256);
  const auto* s32 = static_cast<const uint32_t*>(blocks);
  auto grid = [](int64_t n) { return (unsigned)(n / 256 + 1 < 65536 ? n / 256 + 1 : 65536); };
  hipLaunchKernelGGL(q4k_repack_qs_kernel, dim3(grid(nq)), dim3(256), 0, stream, s32, M, K,
                     static_cast<u32x4*>(qs), nq);
  if (hipGetLastError() != hipSuccess) return Q8_ELAUNCH;
  hipLaunchKernelGGL(q4k_repack_meta_kernel, dim3(grid(nm)), dim3(256), 0, stream, s32, M, K,
                     static_cast<u32x4*>(meta), nm);
  return hipGetLastError() == hipSuccess ? Q8_OK : Q8_ELAUNCH;
}

// ---- Q5_K ------------------------------------------------------------------
// GGUF Q5_K blocks ("skuznetsov/cogni-ml" README, cuda_q5k_gemv_probe; 176
// bytes per 256 weights of one row: the 16-byte header of Q4_K, qh[32] whose
// bit j of byte l is the fifth bit of sub-block j's weight l, then the 128
// nibble bytes placed as in Q4_K) move into:
//   qs, meta: as for Q4_K (the nibbles start at byte 48 instead of 16)
//   qh:       per 64-row tile, per 128-weight quad, 16 bytes of each of the
//             64 rows: one dword per sub-block of the quad, whose bit 8b + i is
//             the fifth bit of weight 4i + b and bit 8b + 4 + i that of weight
//             16 + 4i + b (i, b < 4), the order in which the GEMV merges them
//             into its code bytes.
// Bit moves only; padding rows are zeros.
__global__ __launch_bounds__(256) void q5k_repack_qs_kernel(const uint32_t* __restrict__ src,
                                                            int64_t M, int64_t K,
                                                            u32x4* __restrict__ qs,
                                                            uint32_t* __restrict__ qh,
                                                            int64_t total) {
  const int64_t nsub = K / 32, nsb = K / 256;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t lane = idx & 63;
    const int64_t c = (idx >> 6) % nsub;
    const int64_t t = (idx >> 6) / nsub;
    const int64_t r = t * 64 + lane;
    u32x4 out = {0u, 0u, 0u, 0u};
    uint32_t fb = 0u;
    if (r < M) {
      const int j = (int)(c & 7);
      const uint32_t* blk = src + (r * nsb + c / 8) * 176 / 4;
      const uint32_t* g = blk + (48 + 32 * (j >> 1)) / 4;
      const int sh = (j & 1) * 4;
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = ((g[i] >> sh) & 0x0F0F0F0Fu) | (((g[4 + i] >> sh) & 0x0F0F0F0Fu) << 4);
      out = u32x4{o[0], o[1], o[2], o[3]};
      // qh bytes l = 0..31 at block bytes 16..47, bit j of each
      for (int l = 0; l < 32; ++l) {
        const uint32_t bit = (blk[4 + l / 4] >> (8 * (l & 3) + j)) & 1u;
        const int w = l & 15, i = w >> 2, b = w & 3;
        fb |= bit << (8 * b + i + (l >= 16 ? 4 : 0));
      }
    }
    qs[idx] = out;
    qh[((t * (nsub / 4) + c / 4) * 64 + lane) * 4 + (c & 3)] = fb;
  }
}

__global__ __launch_bounds__(256) void q5k_repack_meta_kernel(const uint32_t* __restrict__ src,
                                                              int64_t M, int64_t K,
                                                              u32x4* __restrict__ meta,
                                                              int64_t total) {
  const int64_t nsb = K / 256;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t lane = idx & 63;
    const int64_t b = (idx >> 6) % nsb;
    const int64_t t = (idx >> 6) / nsb;
    const int64_t r = t * 64 + lane;
    u32x4 out = {0u, 0u, 0u, 0u};
    if (r < M) {
      const uint32_t* h = src + (r * nsb + b) * 176 / 4;
      out = u32x4{h[0], h[1], h[2], h[3]};
    }
    meta[idx] = out;
  }
}

int launch_q5k_repack(const void* blocks, int64_t M, int64_t K, void* qs, void* qh, void* meta,
                      hipStream_t stream) {
  const int64_t T = cdiv(M, kTile);
  const int64_t nq = T * 64 * (K / 32);
  const int64_t nm = T * 64 * (K / 256);
  const auto* s32 = static_cast<const uint32_t*>(blocks);
  auto grid = [](int64_t n) { return (unsigned)(n / 256 + 1 < 65536 ? n / 256 + 1 : 65536); };
  hipLaunchKernelGGL(q5k_repack_qs_kernel, dim3(grid(nq)), dim3(256), 0, stream, s32, M, K,
                     static_cast<u32x4*>(qs), static_cast<uint32_t*>(qh), nq);
  if (hipGetLastError() != hipSuccess) return Q8_ELAUNCH;
  hipLaunchKernelGGL(q5k_repack_meta_kernel, dim3(grid(nm)), dim3(256), 0, stream, s32, M, K,
                     static_cast<u32x4*>(meta), nm);
  return hipGetLastError() == hipSuccess ? Q8_OK : Q8_ELAUNCH;
}

// ---- Q6_K ------------------------------------------------------------------
// GGUF Q6_K blocks ("skuznetsov/cogni-ml" README, cuda_q6k_gemv_probe: ql, qh,
// signed scales, d; 210 bytes per 256 weights: ql[128], qh[64], int8
// scales[16], d) move into, per 64-row tile:
//   ql:   per 32-weight sub-block, 16 bytes per row: byte i holds the low 4
//         bits of the sub-block's weights i (low nibble) and i + 16 (high)
//   qh:   per sub-block, 8 bytes per row: the high 2 bits of weights 0..15
//         (bits 2i of the first dword) and of 16..31 (the second dword)
//   meta: per 128-weight half block, 16 bytes per row: its 8 scales (one per
//         16 weights) and d, then zeros.
// In a GGUF block weight k = 128 h + 32 a + l has its low bits in
// ql[64 h + 32 (a % 2) + l] (low nibble for a < 2, else high) and its high
// bits at bits 2a of qh[32 h + l].  Bit moves only; padding rows are zeros.
__global__ __launch_bounds__(256) void q6k_repack_bits_kernel(const uint8_t* __restrict__ src,
                                                              int64_t M, int64_t K,
                                                              u32x4* __restrict__ ql,
                                                              u32x2* __restrict__ qh,
                                                              int64_t total) {
  const int64_t nsub = K / 32, nsb = K / 256;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t lane = idx & 63;
    const int64_t c = (idx >> 6) % nsub;
    const int64_t t = (idx >> 6) / nsub;
    const int64_t r = t * 64 + lane;
    uint32_t lo[4] = {0u, 0u, 0u, 0u}, hi[2] = {0u, 0u};
    if (r < M) {
      const uint8_t* b = src + (r * nsb + c / 8) * 210;
      const int j = (int)(c & 7), h = j >> 2, a = j & 3;
      const uint8_t* lb = b + 64 * h + 32 * (a & 1);
      const uint8_t* hb = b + 128 + 32 * h;
      const int nsh = 4 * (a >> 1), hsh = 2 * a;
      for (int i = 0; i < 16; ++i) {
        const uint32_t l0 = (lb[i] >> nsh) & 15u, l1 = (lb[16 + i] >> nsh) & 15u;
        lo[i >> 2] |= (l0 | (l1 << 4)) << (8 * (i & 3));
        hi[0] |= (uint32_t)((hb[i] >> hsh) & 3) << (2 * i);
        hi[1] |= (uint32_t)((hb[16 + i] >> hsh) & 3) << (2 * i);
      }
    }
    ql[idx] = u32x4{lo[0], lo[1], lo[2], lo[3]};
    qh[idx] = u32x2{hi[0], hi[1]};
  }
}

__global__ __launch_bounds__(256) void q6k_repack_meta_kernel(const uint8_t* __restrict__ src,
                                                              int64_t M, int64_t K,
                                                              u32x4* __restrict__ meta,
                                                              int64_t total) {
  const int64_t nq = K / 128, nsb = K / 256;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t lane = idx & 63;
    const int64_t g = (idx >> 6) % nq;
    const int64_t t = (idx >> 6) / nq;
    const int64_t r = t * 64 + lane;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (r < M) {
      const uint8_t* b = src + (r * nsb + g / 2) * 210;
      const uint8_t* sc = b + 192 + 8 * (g & 1);
      for (int i = 0; i < 8; ++i) w[i >> 2] |= (uint32_t)sc[i] << (8 * (i & 3));
      w[2] = (uint32_t)b[208] | ((uint32_t)b[209] << 8);
    }
    meta[idx] = u32x4{w[0], w[1], w[2], w[3]};
  }
}

int launch_q6k_repack(const void* blocks, int64_t M, int64_t K, void* ql, void* qh, void* meta,
                      hipStream_t stream) {
  const int64_t T = cdiv(M, kTile);
  const int64_t nb = T * 64 * (K / 32);
  const int64_t nm = T * 64 * (K / 128);
  const auto* s8 = static_cast<const uint8_t*>(blocks);
  auto grid = [](int64_t n) { return (unsigned)(n / 256 + 1 < 65536 ? n / 256 + 1 : 65536); };
  hipLaunchKernelGGL(q6k_repack_bits_kernel, dim3(grid(nb)), dim3(256), 0, stream, s8, M, K,
                     static_cast<u32x4*>(ql), static_cast<u32x2*>(qh), nb);
  if (hipGetLastError() != hipSuccess) return Q8_ELAUNCH;
  hipLaunchKernelGGL(q6k_repack_meta_kernel, dim3(grid(nm)), dim3(256), 0, stream, s8, M, K,
                     static_cast<u32x4*>(meta), nm);
  return hipGetLastError() == hipSuccess ? Q8_OK : Q8_ELAUNCH;
}

}  // namespace q8
