// q8_internal.h -- internal definitions shared by the HIP translation units of
// the Q8_0 GEMV library (never installed, never included by callers).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "q8gemv.h"

namespace q8 {

constexpr int kTile = Q8_TILE_ROWS;  // rows per packed tile, one per lane
// Most waves per GEMV workgroup: 16 for N <= 2 (a wave fits in 128 VGPRs);
// 8 for more columns, so that a wave may use up to 256 VGPRs (the
// activations of a double-buffered quad take 16 N of them).
constexpr int kMaxWaves = 16;
constexpr int kMaxThreads = 64 * kMaxWaves;
// (Q5_K and Q6_K keep more per column in flight: 16-wave workgroups only at
// N = 1.)
constexpr int max_waves_for(int N, bool wide_quads = false) {
  return N <= (wide_quads ? 1 : 2) ? 16 : 8;
}
constexpr int kMaxSeg = 9;           // K-segments over all problems of one launch
constexpr int kMaxProb = 9;          // problems (independent GEMVs) per launch
// Every workspace starts with a fixed region of 32-bit counters that each
// call leaves at zero; data (partials) always lives after it, so calls of
// different shapes can share one workspace without a counter ever landing on
// another call's data.
constexpr size_t kCounterBytes = 65536;
constexpr int kMaxCounters = (int)(kCounterBytes / 4);

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Problem flags (the epilogue/prologue work of one problem).
enum : int32_t { F_RMSNORM = 1, F_RESIDUAL = 2, F_SWIGLU = 4, F_ARGMAX = 8, F_PAIRED = 16 };
// Weight formats: Q8_0 (qs = quants, d = scales); Q4_K and Q5_K (qs = nibbles
// of 32-weight sub-blocks, d = 16-byte block headers: d, dmin, scales/mins;
// Q5_K's fifth bits in qh); Q6_K (qs = low nibbles, qh = 2-bit fields, d =
// scales and d).
enum : int32_t { FMT_Q8_0 = 0, FMT_Q4K = 1, FMT_Q6K = 2, FMT_Q5K = 3 };
// Columns per K-quant launch (all of them: N > 4 uses a ring of sub-block
// buffers whose registers fit every N).
constexpr int kMaxQ4kN = 8;
// How a segment's partial sum is weighted in the fold.
enum : int32_t { A_ONE = 0, A_PTR = 1, A_SIGMOID = 2 };

// One K-segment: a packed matrix (possibly chosen by a device-side expert id)
// times one activation vector.
struct Seg {
  const uint8_t* qs;     // packed quants of matrix 0
  const uint8_t* d;      // packed scales of matrix 0
  int64_t qs_stride;     // bytes between stacked matrices
  int64_t d_stride;
  const int32_t* eid;    // nullptr: matrix 0; else matrix eid[slot]
  int32_t slot;
  int32_t n_mats;
  const float* x;        // activations [N][x_stride]
  int64_t x_stride;
  int32_t K;
  int32_t nblk;          // K / 32
  int32_t G;             // scale quads per row, ceil(nblk / 4)
  int32_t units;         // K-splits of this segment per tile
  int32_t alpha_mode;    // A_*
  const float* alpha_ptr;
  int32_t gqa_group;     // > 0: x index mapping of grouped-query attention
  int32_t gqa_hd;
  int64_t gqa_off;
  const int8_t* qx;      // integer activations [N][K] (opt-in path), or nullptr
  const uint16_t* dx;    // their binary16 block scales [N][K / 32]
  int32_t fmt;           // FMT_*: how qs / d are packed
  const uint8_t* qh;     // Q6_K: packed high 2-bit fields; Q5_K: fifth bits
};

// One problem: an output of Mout rows computed from R row-tiles per output
// tile (R = 2 pairs the gate tile t with the up tile t + Tout).  F_PAIRED:
// the matrix uses the gate/up pairs layout (R = 1; lanes 0..31 gate rows,
// 32..63 the matching up rows).
struct Prob {
  int32_t seg0, nseg;
  int32_t R;
  int32_t M;             // matrix rows
  int32_t Mout;          // output rows
  int32_t Tout;          // output tiles
  int32_t U;             // units per output tile (R * sum of segment units)
  int32_t P;             // workgroups per output tile
  int32_t fold_lds;      // P > 1: the last workgroup stages the tile's partials in LDS
  int32_t wg0;           // first workgroup of this problem
  int32_t flags;         // F_*
  float eps;
  float* y;
  int64_t y_stride;      // between columns n
  const float* residual;
  const float* rms_x;    // vector whose RMS scales the output
  int32_t rms_K;
  int32_t* argmax_out;
  uint32_t* tile_tickets;  // [Tout] arrivals per output tile (P > 1)
  float* am_val;         // [Tout] per-tile argmax partials (F_ARGMAX)
  int32_t* am_idx;       // [Tout]
  float* part;           // [Tout][U][N][64] partial sums when P > 1
  int32_t* dev_status;
};

// Router fused into a routed-expert launch: every wave with a routed segment
// picks its slot's expert from the logits itself, and workgroup 0 also writes
// the ids and renormalised weights of all k slots for the next launch.
struct RouteParams {
  const float* logits;   // [E], or nullptr: ids are read from Seg::eid
  int32_t E, k;
  int32_t* ids_out;      // [k]
  float* w_out;          // [k]
};

struct GemvParams {
  Seg seg[kMaxSeg];
  Prob prob[kMaxProb];
  int32_t nprob;
  int32_t total_wg;
  int32_t W;             // waves per workgroup
  int32_t prio;          // every wave resident at once: issue priority by progress
  RouteParams route;
};

// Host-side launcher shared by the C entry points (gemv.hip).
struct SegDesc {
  const int8_t* qx;      // integer activations (opt-in path), or nullptr
  const uint16_t* dx;
  int32_t fmt;           // FMT_*
  const void* qh;        // Q6_K high bits, Q5_K fifth bits
  const q8_0_weights* W;
  const int32_t* eid;
  int32_t slot;
  const float* x;
  int64_t x_stride;
  int32_t alpha_mode;
  const float* alpha_ptr;
  int32_t gqa_group, gqa_hd;
  int64_t gqa_off;
};

struct ProbDesc {
  SegDesc seg[kMaxSeg];
  int32_t nseg;
  int32_t R;
  int64_t M;
  int32_t flags;
  float eps;
  float* y;
  int64_t y_stride;
  const float* residual;
  const float* rms_x;
  int64_t rms_K;
  int32_t* argmax_out;
  int32_t* dev_status;
};

// Plan (units, workgroups per tile, workspace layout) for a set of problems.
struct Plan {
  int32_t U[kMaxProb];
  int32_t P[kMaxProb];
  int32_t seg_units[kMaxSeg];
  int32_t cnt_off[kMaxProb];   // first counter of each problem
  size_t data_off[kMaxProb];   // byte offset of each problem's data (after the counters)
  size_t ws_bytes;             // total (0: no workspace needed)
  int32_t total_wg;
  int32_t W;                   // waves per workgroup
};

int plan_problems(const ProbDesc* probs, int nprob, int N, Plan* plan);
int launch_problems(const ProbDesc* probs, int nprob, int N, void* ws, size_t ws_bytes,
                    hipStream_t stream, const RouteParams* route = nullptr);

// argmax / router / repack launchers (select.hip, repack.hip)
size_t argmax_ws_bytes(int64_t n);
int launch_argmax(const float* v, int64_t n, int32_t* out, void* ws, size_t ws_bytes,
                  hipStream_t stream);
int launch_route(const float* logits, int32_t E, int32_t k, int32_t* ids, float* w,
                 hipStream_t stream);
int launch_q4k_repack(const void* blocks, int64_t M, int64_t K, void* qs, void* meta,
                      hipStream_t stream);
int launch_q5k_repack(const void* blocks, int64_t M, int64_t K, void* qs, void* qh, void* meta,
                      hipStream_t stream);
int launch_q6k_repack(const void* blocks, int64_t M, int64_t K, void* ql, void* qh, void* meta,
                      hipStream_t stream);
int launch_quantize_act(const float* x, int64_t K, int64_t N, int8_t* qx, uint16_t* dx,
                        hipStream_t stream);
int launch_repack(const void* aos, int64_t M, int64_t K, int32_t layout, void* qs, void* d,
                  hipStream_t stream);

// streaming read-reduce (calib.hip): the achievable-read-bandwidth reference
int launch_read_reduce(const void* buf, int64_t bytes, uint32_t* out, int grid,
                       hipStream_t stream);

// persistent decode chain (chain.hip); arguments validated by the C entry points
size_t chain_ws_bytes(const q8_0_chain_desc* c);
int chain_prepare(const q8_0_chain_desc* c, void* ws, size_t ws_bytes, q8_0_chain_plan* plan,
                  hipStream_t stream);
int chain_run(const q8_0_chain_plan* plan, void* ws, const float* h_in, float* h_out,
              float* logits, int32_t* next_token, int64_t* stamps, hipStream_t stream);
int chain_read(const q8_0_chain_plan* plan, const void* ws, int32_t layer, int32_t which,
               float* dst, hipStream_t stream);
int chain_status(const void* ws, int32_t* out, hipStream_t stream);

// ---- data exchanged between workgroups of one launch ------------------------
// The 8 XCDs of an MI355X each have their own L2, not coherent with the
// others; an agent-scope fence writes back and invalidates a whole L2, which
// is far too costly per workgroup.  Data handed from one workgroup to another
// is therefore written and read with device-scope atomic stores/loads
// (coherent at the memory side), the writer waits for its stores to complete
// (vmcnt 0) before it signals, and the signal is a device-scope atomic add.
template <typename T>
__device__ __forceinline__ void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_dev(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory store this wave issued has completed (vmcnt(0);
// expcnt and lgkmcnt left at their maxima).
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ unsigned ticket_add(uint32_t* t) {
  return __hip_atomic_fetch_add(t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- (value, index) selection, one wave ---------------------------------------
// pair_better keeps the larger value, then the lower index: a total order on
// finite values, so any reduction order selects the same pair.
__device__ __forceinline__ void pair_better(float& v, int& i, float ov, int oi) {
  if (ov > v || (ov == v && oi < i)) {
    v = ov;
    i = oi;
  }
}
// The best (largest value, then lowest index) of the wave's 64 pairs, in
// every lane: DPP row rotations within each 16-lane row, then the row-pair
// and half swaps (v_permlane16/32_swap, VALU moves; the nop covers the
// VALU-write to permlane-read hazard).  A total order on the pairs, so the
// result does not depend on the reduction order.  About 30 VALU operations
// against 12 LDS-routed shuffles (ds_bpermute) for a butterfly.
template <int CTRL>
__device__ __forceinline__ int pair_dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ void wave_best_pair(float& v, int& i) {
#define Q8_PAIR_ROR(C)                                                                   \
  pair_better(v, i, __builtin_bit_cast(float, pair_dpp<C>(__builtin_bit_cast(int, v))), \
               pair_dpp<C>(i))
  Q8_PAIR_ROR(0x121);  // row_ror:1
  Q8_PAIR_ROR(0x122);  // row_ror:2
  Q8_PAIR_ROR(0x124);  // row_ror:4
  Q8_PAIR_ROR(0x128);  // row_ror:8
#undef Q8_PAIR_ROR
  float va = v, vb = v;
  int ia = i, ib = i;
  __asm__ volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(va), "+v"(vb));
  __asm__ volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(ia), "+v"(ib));
  v = va;
  i = ia;
  pair_better(v, i, vb, ib);
  va = v;
  vb = v;
  ia = i;
  ib = i;
  __asm__ volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(va), "+v"(vb));
  __asm__ volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(ia), "+v"(ib));
  v = va;
  i = ia;
  pair_better(v, i, vb, ib);
}

// ---- top-k routing, one wave ------------------------------------------------
// The k largest of E <= 1024 router logits in descending order, ties to the
// lower index (lane l holds logits l, l + 64, ...); every lane ends with the
// same picks.  Exact comparisons, so every caller selects identically.
__device__ __forceinline__ void route_topk_wave(const float* logits, int E, int k, int lane,
                                                float* sel_v, int* sel_i) {
  float lv[16];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    lv[i] = -INFINITY;
    if (64 * i < E) {  // uniform: the loads of one row of 64 are issued together
      const int e = lane + 64 * i;
      const float t = logits[e < E ? e : E - 1];
      lv[i] = e < E ? t : -INFINITY;
    }
  }
  // (unrolled over the slot bound so the picks stay in registers)
#pragma unroll
  for (int s = 0; s < Q8_MAX_SLOTS; ++s) {
    sel_v[s] = -INFINITY;
    sel_i[s] = 0x7fffffff;
    if (s < k) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (64 * i >= E) break;  // uniform: rows of 64 logits that exist
        const int e = lane + 64 * i;
        if (e < E && !(taken >> i & 1u)) pair_better(bv, bi, lv[i], e);
      }
      wave_best_pair(bv, bi);
      sel_v[s] = bv;
      sel_i[s] = bi;
      if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    }
  }
}
// Expert of slot s alone (the (s+1)-th largest logit), same selection.
__device__ __forceinline__ int route_pick_wave(const float* logits, int E, int s_target,
                                               int lane) {
  float lv[16];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    lv[i] = -INFINITY;
    if (64 * i < E) {
      const int e = lane + 64 * i;
      const float t = logits[e < E ? e : E - 1];
      lv[i] = e < E ? t : -INFINITY;
    }
  }
  int pick = 0x7fffffff;
  for (int s = 0; s <= s_target; ++s) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (64 * i >= E) break;  // uniform: rows of 64 logits that exist
      const int e = lane + 64 * i;
      if (e < E && !(taken >> i & 1u)) pair_better(bv, bi, lv[i], e);
    }
    wave_best_pair(bv, bi);
    pick = bi;
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
  }
  return pick;
}
// Renormalised softmax weight of pick s: exp(l_s - l_0) / sum_t exp(l_t - l_0),
// the sum in pick order.
__device__ __forceinline__ float route_denominator(const float* sel_v, int k) {
  float den = 0.f;
#pragma unroll
  for (int t = 0; t < Q8_MAX_SLOTS; ++t)
    if (t < k) den += expf(sel_v[t] - sel_v[0]);
  return den;
}
// Writes ids[s] and the renormalised weight w[s] of every pick s < k.
__device__ __forceinline__ void route_store(const float* sel_v, const int* sel_i, int k,
                                            int32_t* ids, float* w) {
  const float den = route_denominator(sel_v, k);
#pragma unroll
  for (int s = 0; s < Q8_MAX_SLOTS; ++s) {
    if (s < k) {
      ids[s] = sel_i[s];
      w[s] = expf(sel_v[s] - sel_v[0]) / den;
    }
  }
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace q8
