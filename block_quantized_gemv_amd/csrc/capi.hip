// capi.hip -- the extern "C" boundary: argument validation, problem setup and
// launch on the caller's stream.  Host-side checks follow the hardening notes
// of "fusedtok 1.3.0" (1.2.1: host-side validation, a documented device-tensor
// trust boundary, empty-input guards; 1.3: zero-copy helpers reject CPU
// operands because a host pointer in a kernel poisons the context).  Values
// that live in device memory (expert ids) are inside the trust boundary: the
// kernels bound-check them instead of reading through them.
#include <string.h>

#include <mutex>

#include "q8_internal.h"

using namespace q8;

namespace {

constexpr int kVersion = 10000;  // 1.0.0

int check_dev(const void* p) {
  if (!p) return Q8_ENULL;
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky last-error of the failed query
    return Q8_EHOSTPTR;
  }
  if (a.type != hipMemoryTypeDevice && a.type != hipMemoryTypeManaged) return Q8_EHOSTPTR;
  return Q8_OK;
}

int check_dev_aligned(const void* p, size_t align) {
  if (!p) return Q8_ENULL;
  if (reinterpret_cast<uintptr_t>(p) % align) return Q8_EALIGN;
  return check_dev(p);
}

bool shape_ok(int64_t M, int64_t K) {
  return M >= 0 && M <= (int64_t)0x7fffffff - 64 && K > 0 && K % 32 == 0 && K <= Q8_MAX_K;
}

// Scalar checks of a weight descriptor (no pointer queries).
int check_weights_shape(const q8_0_weights* W, int64_t M, int64_t K, bool stacked) {
  if (!W) return Q8_ENULL;
  if (W->M != M || W->K != K || !shape_ok(M, K)) return Q8_EINVAL;
  if (W->n_mats < 1 || (!stacked && W->n_mats != 1)) return Q8_EINVAL;
  if (W->layout != Q8_LAYOUT_ROWS && W->layout != Q8_LAYOUT_GATE_UP_PAIRS) return Q8_EINVAL;
  if (W->layout == Q8_LAYOUT_GATE_UP_PAIRS && M % kTile) return Q8_EINVAL;
  if (W->n_mats > 1) {
    size_t qb = 0, db = 0;
    q8_0_packed_size(M, K, &qb, &db);
    if (W->qs_stride < (int64_t)qb || W->d_stride < (int64_t)db || W->qs_stride % 16 ||
        W->d_stride % 8)
      return Q8_EINVAL;
  }
  return Q8_OK;
}

int check_weights_ptrs(const q8_0_weights* W) {
  int rc = check_dev_aligned(W->qs, 16);
  if (rc) return rc;
  return check_dev_aligned(W->d, 8);
}

SegDesc seg_of(const q8_0_weights* W, const float* x, int64_t x_stride) {
  SegDesc s;
  memset(&s, 0, sizeof(s));
  s.W = W;
  s.x = x;
  s.x_stride = x_stride;
  s.alpha_mode = A_ONE;
  return s;
}

// ---- problem builders (shared by sizing and launching) --------------------
int build_gemv(const q8_0_weights* W, const float* x, float* y, int64_t M, int64_t K, int64_t N,
               const q8_0_fusion* f, ProbDesc* pd) {
  memset(pd, 0, sizeof(*pd));
  pd->nseg = 1;
  pd->seg[0] = seg_of(W, x, K);
  pd->R = 1;
  pd->M = M;
  pd->y = y;
  pd->y_stride = M;
  if (W->layout == Q8_LAYOUT_GATE_UP_PAIRS) pd->flags |= F_PAIRED;
  if (!f) return Q8_OK;
  if (N != 1) return Q8_EINVAL;
  const int ep = f->epilogue;
  if (ep & ~(Q8_EPI_RESIDUAL | Q8_EPI_SWIGLU | Q8_EPI_ARGMAX)) return Q8_EINVAL;
  if (f->prologue == Q8_PRO_RMSNORM) {
    if (!(f->eps >= 0.f)) return Q8_EINVAL;
    pd->flags |= F_RMSNORM;
    pd->rms_x = x;
    pd->rms_K = K;
    pd->eps = f->eps;
  } else if (f->prologue == Q8_PRO_GQA) {
    if (f->n_heads <= 0 || f->n_kv_heads <= 0 || f->n_heads % f->n_kv_heads ||
        f->head_dim <= 0 || f->head_dim % 32 || (int64_t)f->n_heads * f->head_dim != K ||
        f->gqa_offset < 0)
      return Q8_EINVAL;
    pd->seg[0].gqa_group = f->n_heads / f->n_kv_heads;
    pd->seg[0].gqa_hd = f->head_dim;
    pd->seg[0].gqa_off = f->gqa_offset;
  } else if (f->prologue != Q8_PRO_NONE) {
    return Q8_EINVAL;
  }
  if (ep & Q8_EPI_SWIGLU) {
    if (ep & (Q8_EPI_RESIDUAL | Q8_EPI_ARGMAX)) return Q8_EINVAL;
    if (W->layout == Q8_LAYOUT_GATE_UP_PAIRS) {
      if (M % kTile) return Q8_EINVAL;
    } else {
      if (M % 2 || (M / 2) % kTile) return Q8_EINVAL;
      pd->R = 2;
    }
    pd->flags |= F_SWIGLU;
  }
  if (ep & Q8_EPI_RESIDUAL) {
    pd->flags |= F_RESIDUAL;
    pd->residual = f->residual;
  }
  if (ep & Q8_EPI_ARGMAX) {
    pd->flags |= F_ARGMAX;
    pd->argmax_out = f->argmax_out;
  }
  return Q8_OK;
}

int build_moe(const q8_0_weights* We, const int32_t* ids, const float* sw, const float* x,
              float* y, int64_t M, int64_t K, int32_t S, int32_t mode, const q8_0_weights* sh,
              const float* sgate, int32_t* status, ProbDesc* pd, int* nprob) {
  const bool swiglu = mode & Q8_MOE_SWIGLU;
  const int base = mode & ~Q8_MOE_SWIGLU;
  if (S < 1 || S > Q8_MAX_SLOTS) return Q8_EINVAL;
  if (base == Q8_MOE_SCATTER) {
    if (S + (sh ? 1 : 0) > kMaxProb) return Q8_EINVAL;
    // SwiGLU pairs gate and up rows: within a wave with the pairs layout,
    // else gate tile t with up tile t + M/128
    auto swiglu_ok = [](const q8_0_weights* w, int64_t m) {
      return w->layout == Q8_LAYOUT_GATE_UP_PAIRS ? m % kTile == 0
                                                  : (m % 2 == 0 && (m / 2) % kTile == 0);
    };
    if (swiglu && !swiglu_ok(We, M)) return Q8_EINVAL;
    if (swiglu && sh && !swiglu_ok(sh, sh->M)) return Q8_EINVAL;
    if (sh && sh->K != K) return Q8_EINVAL;
    const int64_t Mo = swiglu ? M / 2 : M;
    auto setup = [&](ProbDesc& p, const q8_0_weights* w, int64_t m) {
      const bool pairs = w->layout == Q8_LAYOUT_GATE_UP_PAIRS;
      p.R = (swiglu && !pairs) ? 2 : 1;
      p.M = m;
      p.flags = (swiglu ? F_SWIGLU : 0) | (pairs ? F_PAIRED : 0);
      p.y_stride = swiglu ? m / 2 : m;
      p.dev_status = status;
    };
    int n = 0;
    for (int s = 0; s < S; ++s, ++n) {
      ProbDesc& p = pd[n];
      memset(&p, 0, sizeof(p));
      p.nseg = 1;
      p.seg[0] = seg_of(We, x, K);
      p.seg[0].eid = ids;
      p.seg[0].slot = s;
      setup(p, We, M);
      p.y = y ? y + (int64_t)s * Mo : nullptr;
    }
    if (sh) {
      ProbDesc& p = pd[n++];
      memset(&p, 0, sizeof(p));
      p.nseg = 1;
      p.seg[0] = seg_of(sh, x, K);
      setup(p, sh, sh->M);
      p.y = y ? y + (int64_t)S * Mo : nullptr;
    }
    *nprob = n;
    return Q8_OK;
  }
  if (base == Q8_MOE_COMBINE) {
    if (swiglu) return Q8_EINVAL;
    if (S + (sh ? 1 : 0) > kMaxSeg) return Q8_EINVAL;
    if (sh && sh->M != M) return Q8_EINVAL;
    if (sh && sh->layout != We->layout) return Q8_EINVAL;  // segments share tile rows
    ProbDesc& p = pd[0];
    memset(&p, 0, sizeof(p));
    for (int s = 0; s < S; ++s) {
      p.seg[s] = seg_of(We, x ? x + (int64_t)s * K : nullptr, K);
      p.seg[s].eid = ids;
      p.seg[s].slot = s;
      p.seg[s].alpha_mode = A_PTR;
      p.seg[s].alpha_ptr = sw ? sw + s : nullptr;
    }
    p.nseg = S;
    if (sh) {
      p.seg[S] = seg_of(sh, x ? x + (int64_t)S * K : nullptr, sh->K);
      p.seg[S].alpha_mode = A_SIGMOID;
      p.seg[S].alpha_ptr = sgate;
      p.nseg = S + 1;
    }
    p.R = 1;
    p.M = M;
    p.flags = We->layout == Q8_LAYOUT_GATE_UP_PAIRS ? F_PAIRED : 0;
    p.y = y;
    p.y_stride = M;
    p.dev_status = status;
    *nprob = 1;
    return Q8_OK;
  }
  return Q8_EINVAL;
}

}  // namespace

extern "C" {

int q8_0_packed_size(int64_t M, int64_t K, size_t* qs_bytes, size_t* d_bytes) {
  if (!qs_bytes || !d_bytes) return Q8_ENULL;
  if (!shape_ok(M, K)) return Q8_EINVAL;
  const int64_t T = cdiv(M, kTile);
  *qs_bytes = (size_t)(T * kTile * K);
  *d_bytes = (size_t)(T * cdiv(K / 32, 4) * kTile * 8);
  return Q8_OK;
}

int q8_0_repack(const void* aos, int64_t M, int64_t K, void* qs, void* d, void* stream) {
  if (!shape_ok(M, K)) return Q8_EINVAL;
  if (!aos || !qs || !d) return Q8_ENULL;
  if (M == 0) return Q8_OK;
  int rc;
  if ((rc = check_dev_aligned(aos, 2)) || (rc = check_dev_aligned(qs, 16)) ||
      (rc = check_dev_aligned(d, 8)))
    return rc;
  return launch_repack(aos, M, K, Q8_LAYOUT_ROWS, qs, d, static_cast<hipStream_t>(stream));
}

int q8_0_repack_layout(const void* aos, int64_t M, int64_t K, int32_t layout, void* qs, void* d,
                       void* stream) {
  if (!shape_ok(M, K)) return Q8_EINVAL;
  if (layout != Q8_LAYOUT_ROWS && layout != Q8_LAYOUT_GATE_UP_PAIRS) return Q8_EINVAL;
  if (layout == Q8_LAYOUT_GATE_UP_PAIRS && M % kTile) return Q8_EINVAL;
  if (!aos || !qs || !d) return Q8_ENULL;
  if (M == 0) return Q8_OK;
  int rc;
  if ((rc = check_dev_aligned(aos, 2)) || (rc = check_dev_aligned(qs, 16)) ||
      (rc = check_dev_aligned(d, 8)))
    return rc;
  return launch_repack(aos, M, K, layout, qs, d, static_cast<hipStream_t>(stream));
}

// Rows of the GGUF matrix that one band of whole 64-row tiles moves through
// the staging buffer, or 0 when not even one tile fits.
static int64_t host_band_tiles(int64_t M, int64_t K, size_t staging_bytes) {
  const int64_t tile_bytes = (int64_t)kTile * (K / 32) * 34;
  const int64_t T = (M + kTile - 1) / kTile;
  const int64_t n = (int64_t)(staging_bytes / (size_t)tile_bytes);
  return n < T ? n : T;
}

size_t q8_0_repack_staging_bytes(int64_t M, int64_t K) {
  if (!shape_ok(M, K) || M == 0) return 0;
  return (size_t)kTile * (size_t)(K / 32) * 34;
}

int q8_0_repack_host(const void* aos_host, int64_t M, int64_t K, int32_t layout, void* qs,
                     void* d, void* staging, size_t staging_bytes, void* stream) {
  if (!shape_ok(M, K)) return Q8_EINVAL;
  if (layout != Q8_LAYOUT_ROWS && layout != Q8_LAYOUT_GATE_UP_PAIRS) return Q8_EINVAL;
  if (layout == Q8_LAYOUT_GATE_UP_PAIRS && M % kTile) return Q8_EINVAL;
  if (!aos_host || !qs || !d || !staging) return Q8_ENULL;
  if (M == 0) return Q8_OK;
  int rc;
  if ((rc = check_dev_aligned(qs, 16)) || (rc = check_dev_aligned(d, 8)) ||
      (rc = check_dev_aligned(staging, 16)))
    return rc;
  const int64_t band = host_band_tiles(M, K, staging_bytes);
  if (band < 1) return Q8_EWORKSPACE;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t row_bytes = (K / 32) * 34;
  const int64_t T = (M + kTile - 1) / kTile, G = (K / 32 + 3) / 4;
  const uint8_t* src = static_cast<const uint8_t*>(aos_host);
  uint8_t* stg = static_cast<uint8_t*>(staging);
  for (int64_t t0 = 0; t0 < T; t0 += band) {
    const int64_t nt = T - t0 < band ? T - t0 : band;
    int64_t rows;
    // stream order keeps each copy behind the previous band's repack kernels
    if (layout == Q8_LAYOUT_GATE_UP_PAIRS) {
      // gate rows 32 t0 .., then the matching up rows M/2 + 32 t0 ..: a
      // gate/up matrix of 64 nt rows whose tiles are tiles t0 .. of the whole
      const int64_t h = 32 * nt, g0 = 32 * t0, u0 = M / 2 + 32 * t0;
      if (hipMemcpyAsync(stg, src + g0 * row_bytes, (size_t)(h * row_bytes),
                         hipMemcpyHostToDevice, st) != hipSuccess ||
          hipMemcpyAsync(stg + h * row_bytes, src + u0 * row_bytes, (size_t)(h * row_bytes),
                         hipMemcpyHostToDevice, st) != hipSuccess) {
        (void)hipGetLastError();
        return Q8_ELAUNCH;
      }
      rows = 2 * h;
    } else {
      const int64_t r0 = kTile * t0;
      rows = M - r0 < kTile * nt ? M - r0 : kTile * nt;
      if (hipMemcpyAsync(stg, src + r0 * row_bytes, (size_t)(rows * row_bytes),
                         hipMemcpyHostToDevice, st) != hipSuccess) {
        (void)hipGetLastError();
        return Q8_ELAUNCH;
      }
    }
    if ((rc = launch_repack(stg, rows, K, layout, static_cast<uint8_t*>(qs) + t0 * kTile * K,
                            static_cast<uint8_t*>(d) + t0 * G * kTile * 8, st)))
      return rc;
  }
  return Q8_OK;
}

static int gemv_common(const q8_0_weights* W, const float* x, float* y, int64_t M, int64_t K,
                       int64_t N, const q8_0_fusion* f, int32_t* col_argmax, void* ws,
                       size_t wsb, void* stream) {
  int rc = check_weights_shape(W, M, K, false);
  if (rc) return rc;
  if (N < 1 || N > Q8_MAX_N) return Q8_EINVAL;
  if (!x || !y) return Q8_ENULL;
  ProbDesc pd;
  if ((rc = build_gemv(W, x, y, M, K, N, f, &pd))) return rc;
  if (col_argmax) {
    pd.flags |= F_ARGMAX;
    pd.argmax_out = col_argmax;
  }
  if (M == 0) return Q8_OK;
  if ((rc = check_weights_ptrs(W)) || (rc = check_dev_aligned(x, 4)) ||
      (rc = check_dev_aligned(y, 4)))
    return rc;
  if ((pd.flags & F_RESIDUAL) && (rc = check_dev_aligned(pd.residual, 4))) return rc;
  if ((pd.flags & F_ARGMAX) && (rc = check_dev_aligned(pd.argmax_out, 4))) return rc;
  if (ws && (rc = check_dev(ws))) return rc;
  return launch_problems(&pd, 1, (int)N, ws, wsb, static_cast<hipStream_t>(stream));
}

int q8_0_gemv(const q8_0_weights* W, const float* x, float* y, int64_t M, int64_t K, int64_t N,
              void* workspace, size_t workspace_bytes, void* stream) {
  return gemv_common(W, x, y, M, K, N, nullptr, nullptr, workspace, workspace_bytes, stream);
}

// ---- q8_0_gemv without allocation ---------------------------------------------
// For callers that cannot allocate (code under graph capture, tight serving
// loops): the split-K partials and tickets live in a file-scope device array
// instead of a caller workspace.  Each device holds its own copy until the
// process ends; its address is looked up once per device, with that device
// current, and only that address is handed to kernels.
}  // extern "C"

namespace {
constexpr size_t kScratchBytes = (size_t)8 << 20;  // 8 MiB per device
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];  // device address of `scratch` per device (nullptr: not looked up)

// The current device's copy of `scratch` (set up on the first call per device).
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return Q8_ELAUNCH;
  }
  if (dev < 0 || dev >= kMaxDevices) return Q8_ELAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return Q8_ELAUNCH;
    }
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return Q8_OK;
}

__global__ void zero_words_kernel(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}
}  // namespace

extern "C" {

int q8_0_gemv_noalloc(const q8_0_weights* W, const float* x, float* y, int64_t M, int64_t K,
                      int64_t N, void* stream) {
  int rc = check_weights_shape(W, M, K, false);
  if (rc) return rc;
  if (N < 1 || N > Q8_MAX_N) return Q8_EINVAL;
  if (!x || !y) return Q8_ENULL;
  ProbDesc pd;
  if ((rc = build_gemv(W, x, y, M, K, N, nullptr, &pd))) return rc;
  if (M == 0) return Q8_OK;
  Plan plan;
  if ((rc = plan_problems(&pd, 1, (int)N, &plan))) return rc;
  if (plan.ws_bytes > kScratchBytes) return Q8_EWORKSPACE;
  if ((rc = check_weights_ptrs(W)) || (rc = check_dev_aligned(x, 4)) ||
      (rc = check_dev_aligned(y, 4)))
    return rc;
  void* ws = nullptr;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (plan.ws_bytes > 0) {
    if ((rc = scratch_address(&ws))) return rc;
    // the array keeps the last call's contents: clear the ticket counters,
    // which must start at zero, with a kernel on the same stream (no memset
    // node, so the call can be captured)
    hipLaunchKernelGGL(zero_words_kernel, dim3(64), dim3(256), 0, s, static_cast<uint32_t*>(ws),
                       (int)(kCounterBytes / 4));
    if (hipGetLastError() != hipSuccess) return Q8_ELAUNCH;
  }
  return launch_problems(&pd, 1, (int)N, ws, kScratchBytes, s);
}

int q8_0_gemv_argmax(const q8_0_weights* W, const float* x, float* y, int64_t M, int64_t K,
                     int64_t N, int32_t* argmax_out, void* workspace, size_t workspace_bytes,
                     void* stream) {
  if (!argmax_out) return Q8_ENULL;
  return gemv_common(W, x, y, M, K, N, nullptr, argmax_out, workspace, workspace_bytes, stream);
}

int q8_0_gemv_fused(const q8_0_weights* W, const float* x, float* y, int64_t M, int64_t K,
                    const q8_0_fusion* fusion, void* workspace, size_t workspace_bytes,
                    void* stream) {
  if (!fusion) return Q8_ENULL;
  return gemv_common(W, x, y, M, K, 1, fusion, nullptr, workspace, workspace_bytes, stream);
}

// ---- K-quants (Q4_K, Q5_K, Q6_K) ---------------------------------------------
static bool q4k_shape_ok(int64_t M, int64_t K) { return shape_ok(M, K) && K % 256 == 0; }

// The GEMV over packed K-quant weights: the launch machinery sees the nibble
// (or low-bit) stream as qs, the per-block headers as d and the extra bit
// stream (Q5_K, Q6_K) as qh.  Columns go kMaxQ4kN at a time; each launch
// reads the weights once.  Pointers and alignments are checked by the caller.
static int kquant_gemv(int32_t fmt, const void* qs, const void* qh, const void* meta,
                       const float* x, float* y, int64_t M, int64_t K, int64_t N,
                       void* workspace, size_t workspace_bytes, void* stream) {
  int rc;
  if (workspace && (rc = check_dev(workspace))) return rc;
  const q8_0_weights w8 = {qs, meta, M, K, 1, 0, 0, Q8_LAYOUT_ROWS, 0};
  for (int64_t n0 = 0; n0 < N; n0 += kMaxQ4kN) {
    const int64_t n = N - n0 < kMaxQ4kN ? N - n0 : kMaxQ4kN;
    ProbDesc pd;
    if ((rc = build_gemv(&w8, x + n0 * K, y + n0 * M, M, K, n, nullptr, &pd))) return rc;
    pd.seg[0].fmt = fmt;
    pd.seg[0].qh = qh;
    if ((rc = launch_problems(&pd, 1, (int)n, workspace, workspace_bytes,
                              static_cast<hipStream_t>(stream))))
      return rc;
  }
  return Q8_OK;
}

int q4k_packed_size(int64_t M, int64_t K, size_t* qs_bytes, size_t* meta_bytes) {
  if (!qs_bytes || !meta_bytes) return Q8_ENULL;
  if (!q4k_shape_ok(M, K)) return Q8_EINVAL;
  const int64_t T = cdiv(M, kTile);
  *qs_bytes = (size_t)(T * kTile * (K / 2));
  *meta_bytes = (size_t)(T * kTile * (K / 256) * 16);
  return Q8_OK;
}

int q4k_repack(const void* blocks, int64_t M, int64_t K, void* qs, void* meta, void* stream) {
  if (!q4k_shape_ok(M, K)) return Q8_EINVAL;
  if (!blocks || !qs || !meta) return Q8_ENULL;
  if (M == 0) return Q8_OK;
  int rc;
  if ((rc = check_dev_aligned(blocks, 4)) || (rc = check_dev_aligned(qs, 16)) ||
      (rc = check_dev_aligned(meta, 16)))
    return rc;
  return launch_q4k_repack(blocks, M, K, qs, meta, static_cast<hipStream_t>(stream));
}

int q4k_gemv(const q4k_weights* W, const float* x, float* y, int64_t M, int64_t K, int64_t N,
             void* workspace, size_t workspace_bytes, void* stream) {
  if (!W) return Q8_ENULL;
  if (W->M != M || W->K != K || !q4k_shape_ok(M, K) || N < 1 || N > Q8_MAX_N) return Q8_EINVAL;
  if (!x || !y || !W->qs || !W->meta) return Q8_ENULL;
  if (M == 0) return Q8_OK;
  int rc;
  if ((rc = check_dev_aligned(W->qs, 16)) || (rc = check_dev_aligned(W->meta, 16)) ||
      (rc = check_dev_aligned(x, 4)) || (rc = check_dev_aligned(y, 4)))
    return rc;
  return kquant_gemv(FMT_Q4K, W->qs, nullptr, W->meta, x, y, M, K, N, workspace, workspace_bytes,
                     stream);
}

int q5k_packed_size(int64_t M, int64_t K, size_t* qs_bytes, size_t* qh_bytes,
                    size_t* meta_bytes) {
  if (!qs_bytes || !qh_bytes || !meta_bytes) return Q8_ENULL;
  if (!q4k_shape_ok(M, K)) return Q8_EINVAL;
  const int64_t T = cdiv(M, kTile);
  *qs_bytes = (size_t)(T * kTile * (K / 2));
  *qh_bytes = (size_t)(T * kTile * (K / 8));
  *meta_bytes = (size_t)(T * kTile * (K / 256) * 16);
  return Q8_OK;
}

int q5k_repack(const void* blocks, int64_t M, int64_t K, void* qs, void* qh, void* meta,
               void* stream) {
  if (!q4k_shape_ok(M, K)) return Q8_EINVAL;
  if (!blocks || !qs || !qh || !meta) return Q8_ENULL;
  if (M == 0) return Q8_OK;
  int rc;
  if ((rc = check_dev_aligned(blocks, 4)) || (rc = check_dev_aligned(qs, 16)) ||
      (rc = check_dev_aligned(qh, 16)) || (rc = check_dev_aligned(meta, 16)))
    return rc;
  return launch_q5k_repack(blocks, M, K, qs, qh, meta, static_cast<hipStream_t>(stream));
}

int q5k_gemv(const q5k_weights* W, const float* x, float* y, int64_t M, int64_t K, int64_t N,
             void* workspace, size_t workspace_bytes, void* stream) {
  if (!W) return Q8_ENULL;
  if (W->M != M || W->K != K || !q4k_shape_ok(M, K) || N < 1 || N > Q8_MAX_N) return Q8_EINVAL;
  if (!x || !y || !W->qs || !W->qh || !W->meta) return Q8_ENULL;
  if (M == 0) return Q8_OK;
  int rc;
  if ((rc = check_dev_aligned(W->qs, 16)) || (rc = check_dev_aligned(W->qh, 16)) ||
      (rc = check_dev_aligned(W->meta, 16)) || (rc = check_dev_aligned(x, 4)) ||
      (rc = check_dev_aligned(y, 4)))
    return rc;
  return kquant_gemv(FMT_Q5K, W->qs, W->qh, W->meta, x, y, M, K, N, workspace, workspace_bytes,
                     stream);
}

int q6k_packed_size(int64_t M, int64_t K, size_t* ql_bytes, size_t* qh_bytes,
                    size_t* meta_bytes) {
  if (!ql_bytes || !qh_bytes || !meta_bytes) return Q8_ENULL;
  if (!q4k_shape_ok(M, K)) return Q8_EINVAL;
  const int64_t T = cdiv(M, kTile);
  *ql_bytes = (size_t)(T * kTile * (K / 2));
  *qh_bytes = (size_t)(T * kTile * (K / 4));
  *meta_bytes = (size_t)(T * kTile * (K / 128) * 16);
  return Q8_OK;
}

int q6k_repack(const void* blocks, int64_t M, int64_t K, void* ql, void* qh, void* meta,
               void* stream) {
  if (!q4k_shape_ok(M, K)) return Q8_EINVAL;
  if (!blocks || !ql || !qh || !meta) return Q8_ENULL;
  if (M == 0) return Q8_OK;
  int rc;
  if ((rc = check_dev(blocks)) || (rc = check_dev_aligned(ql, 16)) ||
      (rc = check_dev_aligned(qh, 8)) || (rc = check_dev_aligned(meta, 16)))
    return rc;
  return launch_q6k_repack(blocks, M, K, ql, qh, meta, static_cast<hipStream_t>(stream));
}

int q6k_gemv(const q6k_weights* W, const float* x, float* y, int64_t M, int64_t K, int64_t N,
             void* workspace, size_t workspace_bytes, void* stream) {
  if (!W) return Q8_ENULL;
  if (W->M != M || W->K != K || !q4k_shape_ok(M, K) || N < 1 || N > Q8_MAX_N) return Q8_EINVAL;
  if (!x || !y || !W->ql || !W->qh || !W->meta) return Q8_ENULL;
  if (M == 0) return Q8_OK;
  int rc;
  if ((rc = check_dev_aligned(W->ql, 16)) || (rc = check_dev_aligned(W->qh, 8)) ||
      (rc = check_dev_aligned(W->meta, 16)) || (rc = check_dev_aligned(x, 4)) ||
      (rc = check_dev_aligned(y, 4)))
    return rc;
  return kquant_gemv(FMT_Q6K, W->ql, W->qh, W->meta, x, y, M, K, N, workspace, workspace_bytes,
                     stream);
}

int q8_0_quantize_act(const float* x, int64_t K, int64_t N, int8_t* qx, uint16_t* dx,
                      void* stream) {
  if (!shape_ok(1, K) || N < 1 || N > Q8_MAX_N) return Q8_EINVAL;
  if (!x || !qx || !dx) return Q8_ENULL;
  int rc;
  if ((rc = check_dev_aligned(x, 4)) || (rc = check_dev_aligned(qx, 4)) ||
      (rc = check_dev_aligned(dx, 2)))
    return rc;
  return launch_quantize_act(x, K, N, qx, dx, static_cast<hipStream_t>(stream));
}

int q8_0_gemv_q8act(const q8_0_weights* W, const int8_t* qx, const uint16_t* dx, float* y,
                    int64_t M, int64_t K, int64_t N, void* workspace, size_t workspace_bytes,
                    void* stream) {
  int rc = check_weights_shape(W, M, K, false);
  if (rc) return rc;
  if (N < 1 || N > Q8_MAX_N) return Q8_EINVAL;
  if (!qx || !dx || !y) return Q8_ENULL;
  ProbDesc pd;
  if ((rc = build_gemv(W, nullptr, y, M, K, N, nullptr, &pd))) return rc;
  pd.seg[0].qx = qx;
  pd.seg[0].dx = dx;
  if (M == 0) return Q8_OK;
  if ((rc = check_weights_ptrs(W)) || (rc = check_dev_aligned(qx, 4)) ||
      (rc = check_dev_aligned(dx, 2)) || (rc = check_dev_aligned(y, 4)))
    return rc;
  if (workspace && (rc = check_dev(workspace))) return rc;
  return launch_problems(&pd, 1, (int)N, workspace, workspace_bytes,
                         static_cast<hipStream_t>(stream));
}

int q8_0_argmax(const float* v, int64_t n, int32_t* out_idx, void* workspace,
                size_t workspace_bytes, void* stream) {
  if (n < 0 || n >= ((int64_t)1 << 31)) return Q8_EINVAL;
  if (!v || !out_idx) return Q8_ENULL;
  if (n == 0) return Q8_OK;
  int rc;
  if ((rc = check_dev_aligned(v, 4)) || (rc = check_dev_aligned(out_idx, 4))) return rc;
  if (workspace && (rc = check_dev(workspace))) return rc;
  return launch_argmax(v, n, out_idx, workspace, workspace_bytes,
                       static_cast<hipStream_t>(stream));
}

int q8_0_route_topk(const float* logits, int32_t E, int32_t k, int32_t* expert_ids,
                    float* slot_weights, void* stream) {
  if (E < 1 || E > 1024 || k < 1 || k > E || k > Q8_MAX_SLOTS) return Q8_EINVAL;
  if (!logits || !expert_ids || !slot_weights) return Q8_ENULL;
  int rc;
  if ((rc = check_dev_aligned(logits, 4)) || (rc = check_dev_aligned(expert_ids, 4)) ||
      (rc = check_dev_aligned(slot_weights, 4)))
    return rc;
  return launch_route(logits, E, k, expert_ids, slot_weights, static_cast<hipStream_t>(stream));
}

int q8_0_moe_gemv(const q8_0_weights* W_experts, const int32_t* expert_ids,
                  const float* slot_weights, const float* x, float* y, int64_t M, int64_t K,
                  int32_t n_slots, int32_t mode, const q8_0_weights* shared,
                  const float* shared_gate, int32_t* dev_status, void* workspace,
                  size_t workspace_bytes, void* stream) {
  int rc = check_weights_shape(W_experts, M, K, true);
  if (rc) return rc;
  const int base = mode & ~Q8_MOE_SWIGLU;
  if (shared) {
    const int64_t shK = base == Q8_MOE_COMBINE ? shared->K : K;
    const int64_t shM = base == Q8_MOE_COMBINE ? M : shared->M;
    if ((rc = check_weights_shape(shared, shM, shK, false))) return rc;
  }
  if (!x || !y || !expert_ids) return Q8_ENULL;
  if (base == Q8_MOE_COMBINE && (!slot_weights || (shared && !shared_gate))) return Q8_ENULL;
  ProbDesc pd[kMaxProb];
  int np = 0;
  if ((rc = build_moe(W_experts, expert_ids, slot_weights, x, y, M, K, n_slots, mode, shared,
                      shared_gate, dev_status, pd, &np)))
    return rc;
  if (M == 0) return Q8_OK;
  if ((rc = check_weights_ptrs(W_experts)) || (rc = check_dev_aligned(x, 4)) ||
      (rc = check_dev_aligned(y, 4)) || (rc = check_dev_aligned(expert_ids, 4)))
    return rc;
  if (shared && (rc = check_weights_ptrs(shared))) return rc;
  if (base == Q8_MOE_COMBINE) {
    if ((rc = check_dev_aligned(slot_weights, 4))) return rc;
    if (shared && (rc = check_dev_aligned(shared_gate, 4))) return rc;
  }
  if (dev_status && (rc = check_dev_aligned(dev_status, 4))) return rc;
  if (workspace && (rc = check_dev(workspace))) return rc;
  return launch_problems(pd, np, 1, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

int q8_0_moe_route_gemv(const q8_0_weights* W_experts, const float* router_logits, int32_t E,
                        int32_t* expert_ids, float* slot_weights, const float* x, float* y,
                        int64_t M, int64_t K, int32_t n_slots, int32_t mode,
                        const q8_0_weights* shared, int32_t* dev_status, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if ((mode & ~Q8_MOE_SWIGLU) != Q8_MOE_SCATTER) return Q8_EINVAL;
  int rc = check_weights_shape(W_experts, M, K, true);
  if (rc) return rc;
  if (shared && (rc = check_weights_shape(shared, shared->M, K, false))) return rc;
  if (!router_logits || !expert_ids || !slot_weights || !x || !y) return Q8_ENULL;
  if (E < 1 || E > 1024 || E > W_experts->n_mats || n_slots < 1 || n_slots > E ||
      n_slots > Q8_MAX_SLOTS)
    return Q8_EINVAL;
  ProbDesc pd[kMaxProb];
  int np = 0;
  // expert_ids marks the routed segments; the kernel writes it, never reads it
  if ((rc = build_moe(W_experts, expert_ids, nullptr, x, y, M, K, n_slots, mode, shared, nullptr,
                      dev_status, pd, &np)))
    return rc;
  if ((rc = check_dev_aligned(router_logits, 4)) || (rc = check_dev_aligned(expert_ids, 4)) ||
      (rc = check_dev_aligned(slot_weights, 4)))
    return rc;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (M == 0) return launch_route(router_logits, E, n_slots, expert_ids, slot_weights, st);
  if ((rc = check_weights_ptrs(W_experts)) || (rc = check_dev_aligned(x, 4)) ||
      (rc = check_dev_aligned(y, 4)))
    return rc;
  if (shared && (rc = check_weights_ptrs(shared))) return rc;
  if (dev_status && (rc = check_dev_aligned(dev_status, 4))) return rc;
  if (workspace && (rc = check_dev(workspace))) return rc;
  const RouteParams rp = {router_logits, E, n_slots, expert_ids, slot_weights};
  return launch_problems(pd, np, 1, workspace, workspace_bytes, st, &rp);
}

size_t q8_0_workspace_bytes(int32_t op, int64_t M, int64_t K, int64_t N, int64_t M2, int64_t K2,
                            int32_t flags) {
  Plan plan;
  if (op == Q8_OP_ARGMAX) return argmax_ws_bytes(M);
  if (op == Q8_OP_Q4K_GEMV || op == Q8_OP_Q5K_GEMV || op == Q8_OP_Q6K_GEMV) {
    // the largest need of the launches q4k/q5k/q6k_gemv make: columns in
    // groups of kMaxQ4kN, each planned for its own format
    if (!shape_ok(M, K) || M == 0 || K % 256 || N < 1 || N > Q8_MAX_N) return 0;
    size_t need = 0;
    const int64_t groups[2] = {N < kMaxQ4kN ? N : kMaxQ4kN, N > kMaxQ4kN ? N % kMaxQ4kN : 0};
    for (const int64_t n : groups) {
      if (n == 0) continue;
      q8_0_weights W = {nullptr, nullptr, M, K, 1, 0, 0};
      ProbDesc pd;
      if (build_gemv(&W, nullptr, nullptr, M, K, n, nullptr, &pd)) return 0;
      pd.seg[0].fmt = op == Q8_OP_Q6K_GEMV ? FMT_Q6K : op == Q8_OP_Q5K_GEMV ? FMT_Q5K : FMT_Q4K;
      if (plan_problems(&pd, 1, (int)n, &plan)) return 0;
      if (plan.ws_bytes > need) need = plan.ws_bytes;
    }
    return need;
  }
  if (op == Q8_OP_GEMV || op == Q8_OP_GEMV_FUSED || op == Q8_OP_GEMV_ARGMAX) {
    if (!shape_ok(M, K) || M == 0) return 0;
    q8_0_weights W = {nullptr, nullptr, M, K, 1, 0, 0};
    q8_0_fusion f;
    memset(&f, 0, sizeof(f));
    const q8_0_fusion* fp = nullptr;
    int64_t n = N;
    if (op == Q8_OP_GEMV_FUSED) {
      f.epilogue = (int32_t)N;
      fp = &f;
      n = 1;
    } else if (N < 1 || N > Q8_MAX_N) {
      return 0;
    }
    ProbDesc pd;
    if (build_gemv(&W, nullptr, nullptr, M, K, n, fp, &pd)) return 0;
    if (op == Q8_OP_GEMV_ARGMAX) pd.flags |= F_ARGMAX;
    if (plan_problems(&pd, 1, (int)n, &plan)) return 0;
    return plan.ws_bytes;
  }
  if (op == Q8_OP_MOE_SCATTER || op == Q8_OP_MOE_COMBINE) {
    if (!shape_ok(M, K) || M == 0) return 0;
    q8_0_weights W = {nullptr, nullptr, M, K, 1, 0, 0};
    q8_0_weights S2 = {nullptr, nullptr, M2, K2, 1, 0, 0};
    const bool has_sh = M2 > 0 && K2 > 0;
    const int mode = (op == Q8_OP_MOE_SCATTER ? Q8_MOE_SCATTER : Q8_MOE_COMBINE) |
                     (flags & Q8_MOE_SWIGLU);
    ProbDesc pd[kMaxProb];
    int np = 0;
    if (build_moe(&W, nullptr, nullptr, nullptr, nullptr, M, K, (int32_t)N, mode,
                  has_sh ? &S2 : nullptr, nullptr, nullptr, pd, &np))
      return 0;
    if (plan_problems(pd, np, 1, &plan)) return 0;
    return plan.ws_bytes;
  }
  return 0;
}

int q8_0_gemv_plan(int64_t M, int64_t K, int64_t N, int32_t epilogue, int32_t out[4]) {
  if (!out) return Q8_ENULL;
  if (!shape_ok(M, K) || M == 0 || N < 1 || N > Q8_MAX_N) return Q8_EINVAL;
  q8_0_weights W = {nullptr, nullptr, M, K, 1, 0, 0};
  q8_0_fusion f;
  memset(&f, 0, sizeof(f));
  f.epilogue = epilogue;
  ProbDesc pd;
  if (build_gemv(&W, nullptr, nullptr, M, K, epilogue ? 1 : N, epilogue ? &f : nullptr, &pd))
    return Q8_EINVAL;
  Plan plan;
  if (plan_problems(&pd, 1, (int)(epilogue ? 1 : N), &plan)) return Q8_EINVAL;
  out[0] = plan.total_wg;
  out[1] = plan.W;
  out[2] = plan.U[0];
  out[3] = plan.P[0];
  return Q8_OK;
}

// ---- persistent decode chain ------------------------------------------------
namespace {
int check_chain_desc(const q8_0_chain_desc* c, bool ptrs) {
  if (!c) return Q8_ENULL;
  if (q8::chain_ws_bytes(c) == 0) return Q8_EINVAL;
  const int64_t H = c->hidden, I = c->intermediate, NHD = (int64_t)c->n_heads * c->head_dim;
  const int64_t Mq = ((int64_t)c->n_heads + 2 * (int64_t)c->n_kv_heads) * c->head_dim;
  if (c->n_layers > 0 && (!c->qkv || !c->wo || !c->gate_up || !c->down)) return Q8_ENULL;
  for (int l = 0; l < c->n_layers; ++l) {
    const q8_0_weights* m[4] = {&c->qkv[l], &c->wo[l], &c->gate_up[l], &c->down[l]};
    const int64_t shp[4][2] = {{Mq, H}, {H, NHD}, {2 * I, H}, {H, I}};
    for (int k = 0; k < 4; ++k) {
      int rc = check_weights_shape(m[k], shp[k][0], shp[k][1], false);
      if (rc) return rc;
      if (m[k]->layout != (k == 2 ? Q8_LAYOUT_GATE_UP_PAIRS : Q8_LAYOUT_ROWS)) return Q8_EINVAL;
      if (ptrs && (rc = check_weights_ptrs(m[k]))) return rc;
    }
  }
  if (c->vocab > 0) {
    if (!c->lm_head) return Q8_ENULL;
    int rc = check_weights_shape(c->lm_head, c->vocab, H, false);
    if (rc) return rc;
    if (c->lm_head->layout != Q8_LAYOUT_ROWS) return Q8_EINVAL;
    if (ptrs && (rc = check_weights_ptrs(c->lm_head))) return rc;
  } else if (c->lm_head) {
    return Q8_EINVAL;
  }
  return Q8_OK;
}

bool plan_ok(const q8_0_chain_plan* p) {
  return p->grid > 0 && p->threads > 0 && p->n_layers >= 0 && p->hidden > 0 && p->vocab >= 0 &&
         p->ws_bytes > 0;
}
}  // namespace

size_t q8_0_chain_workspace_bytes(const q8_0_chain_desc* desc) {
  if (check_chain_desc(desc, false)) return 0;
  return q8::chain_ws_bytes(desc);
}

int q8_0_chain_prepare(const q8_0_chain_desc* desc, void* workspace, size_t workspace_bytes,
                       q8_0_chain_plan* plan, void* stream) {
  if (!plan) return Q8_ENULL;
  int rc = check_chain_desc(desc, false);
  if (rc) return rc;
  if ((rc = check_dev_aligned(workspace, 256))) return rc;
  if (workspace_bytes < q8::chain_ws_bytes(desc)) return Q8_EWORKSPACE;
  if ((rc = check_chain_desc(desc, true))) return rc;
  return q8::chain_prepare(desc, workspace, workspace_bytes, plan, (hipStream_t)stream);
}

int q8_0_chain_run(const q8_0_chain_plan* plan, void* workspace, const float* h_in, float* h_out,
                   float* logits, int32_t* next_token, void* stream) {
  if (!plan) return Q8_ENULL;
  if (!plan_ok(plan)) return Q8_EINVAL;
  int rc = check_dev_aligned(workspace, 256);
  if (rc) return rc;
  if ((rc = check_dev_aligned(h_in, 4))) return rc;
  if (h_out && (rc = check_dev_aligned(h_out, 4))) return rc;
  if (plan->vocab > 0) {
    if ((rc = check_dev_aligned(logits, 4))) return rc;
    if ((rc = check_dev_aligned(next_token, 4))) return rc;
  }
  return q8::chain_run(plan, workspace, h_in, h_out, logits, next_token, nullptr,
                       (hipStream_t)stream);
}

int q8_0_chain_run_stamped(const q8_0_chain_plan* plan, void* workspace, const float* h_in,
                           float* h_out, float* logits, int32_t* next_token, int64_t* stamps,
                           void* stream) {
  if (!plan || !stamps) return Q8_ENULL;
  if (!plan_ok(plan)) return Q8_EINVAL;
  int rc = check_dev_aligned(workspace, 256);
  if (rc) return rc;
  if ((rc = check_dev_aligned(h_in, 4)) || (rc = check_dev_aligned(stamps, 8))) return rc;
  if (h_out && (rc = check_dev_aligned(h_out, 4))) return rc;
  if (plan->vocab > 0) {
    if ((rc = check_dev_aligned(logits, 4))) return rc;
    if ((rc = check_dev_aligned(next_token, 4))) return rc;
  }
  return q8::chain_run(plan, workspace, h_in, h_out, logits, next_token, stamps,
                       (hipStream_t)stream);
}

int q8_0_chain_read(const q8_0_chain_plan* plan, const void* workspace, int32_t layer,
                    int32_t which, float* dst, void* stream) {
  if (!plan) return Q8_ENULL;
  if (!plan_ok(plan) || which < 0 || which > 3 || layer < 0 || layer >= plan->n_layers)
    return Q8_EINVAL;
  int rc = check_dev_aligned(workspace, 256);
  if (rc) return rc;
  if ((rc = check_dev_aligned(dst, 4))) return rc;
  return q8::chain_read(plan, workspace, layer, which, dst, (hipStream_t)stream);
}

int q8_0_chain_status(const void* workspace, int32_t* dev_status, void* stream) {
  int rc = check_dev_aligned(workspace, 256);
  if (rc) return rc;
  if ((rc = check_dev_aligned(dev_status, 4))) return rc;
  return q8::chain_status(workspace, dev_status, (hipStream_t)stream);
}

int q8_stream_read(const void* buf, int64_t bytes, uint32_t* out, int32_t grid, void* stream) {
  if (bytes < 0 || grid < 1 || grid > (1 << 20)) return Q8_EINVAL;
  int rc;
  if ((rc = check_dev_aligned(buf, 16)) || (rc = check_dev_aligned(out, 4))) return rc;
  return launch_read_reduce(buf, bytes, out, grid, static_cast<hipStream_t>(stream));
}

const char* q8_0_strerror(int status) {
  switch (status) {
    case Q8_OK: return "ok";
    case Q8_EINVAL: return "invalid argument (shape, count or flags)";
    case Q8_ENULL: return "required pointer is NULL";
    case Q8_EALIGN: return "pointer is not aligned as required";
    case Q8_EHOSTPTR: return "pointer is not device memory";
    case Q8_EWORKSPACE: return "workspace missing or too small";
    case Q8_ELAUNCH: return "HIP runtime error";
    default: return "unknown status";
  }
}

int q8_0_version(void) { return kVersion; }

}  // extern "C"
