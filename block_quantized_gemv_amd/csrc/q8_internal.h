// q8_internal.h -- internal definitions shared by the HIP translation units of
// the Q8_0 GEMV library (never installed, never included by callers).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "q8gemv.h"

namespace q8 {

constexpr int kTile = Q8_TILE_ROWS;  // rows per packed tile, one per lane
constexpr int kWaves = 4;            // waves per GEMV workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxSeg = 9;           // K-segments over all problems of one launch
constexpr int kMaxProb = 9;          // problems (independent GEMVs) per launch

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Problem flags (the epilogue/prologue work of one problem).
enum : int32_t { F_RMSNORM = 1, F_RESIDUAL = 2, F_SWIGLU = 4, F_ARGMAX = 8 };
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
};

// One problem: an output of Mout rows computed from R row-tiles per output
// tile (R = 2 pairs the gate tile t with the up tile t + Tout).
struct Prob {
  int32_t seg0, nseg;
  int32_t R;
  int32_t M;             // matrix rows
  int32_t Mout;          // output rows
  int32_t Tout;          // output tiles
  int32_t U;             // units per output tile (R * sum of segment units)
  int32_t P;             // workgroups per output tile
  int32_t wg0;           // first workgroup of this problem
  int32_t flags;         // F_*
  float eps;
  float* y;
  int64_t y_stride;      // between columns n
  const float* residual;
  const float* rms_x;    // vector whose RMS scales the output
  int32_t rms_K;
  int32_t* argmax_out;
  uint32_t* tickets;     // [Tout + 1]; the last one counts argmax partials
  float* am_val;         // [Tout]
  int32_t* am_idx;       // [Tout]
  float* part;           // [Tout][U][N][64] partial sums when P > 1
  int32_t* dev_status;
};

struct GemvParams {
  Seg seg[kMaxSeg];
  Prob prob[kMaxProb];
  int32_t nprob;
  int32_t total_wg;
};

// Host-side launcher shared by the C entry points (gemv.hip).
struct SegDesc {
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
  size_t ws_off[kMaxProb];   // start of each problem's workspace region
  size_t ws_bytes;           // total
  int32_t total_wg;
};

int plan_problems(const ProbDesc* probs, int nprob, int N, Plan* plan);
int launch_problems(const ProbDesc* probs, int nprob, int N, void* ws, size_t ws_bytes,
                    hipStream_t stream);

// argmax / router / repack launchers (select.hip, repack.hip)
size_t argmax_ws_bytes(int64_t n);
int launch_argmax(const float* v, int64_t n, int32_t* out, void* ws, size_t ws_bytes,
                  hipStream_t stream);
int launch_route(const float* logits, int32_t E, int32_t k, int32_t* ids, float* w,
                 hipStream_t stream);
int launch_repack(const void* aos, int64_t M, int64_t K, void* qs, void* d, hipStream_t stream);

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace q8
