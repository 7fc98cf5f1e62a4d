// chain.hip -- a whole decode step of a Qwen2-style decoder (every layer's
// qkv, wo, gate_up and down projections with their glue, then the LM head and
// greedy argmax) in one persistent launch.
//
// Why: at batch 1 each projection moves 0.9-9 MB, a few microseconds of HBM
// time, so a chain of one launch per projection is bound by launch and
// hand-off latency rather than bandwidth (the pages' graph and slot-fusion
// results: a per-layer task graph of fixed launches; capturing it gains about
// a third, fusing slots cuts launches).  Here one workgroup per compute unit
// stays resident for the whole step and streams each projection's weights
// into registers well before its input arrives.
//
// The MI355X has 8 XCDs of 32 compute units, each XCD with its own L2.  A
// hand-off inside one XCD goes through that L2: a plain store, then a load
// that skips the compute unit's L1 (device-scope policy), about 0.23 us per
// hop.  Between XCDs the store must be written through to memory (device
// scope as well), about 0.45 us per hop, and when every workgroup reads the
// same few lines the memory side serialises them.  So the step is organised
// so that each layer needs one exchange across XCDs, with 8 readers per line,
// and four inside an XCD (workgroup b belongs to group x = b % 8 as member
// j = b / 8; the dispatcher deals workgroups to the XCDs in turn, so a group
// shares one XCD, which q8_0_chain_prepare checks):
//
//   A  v = Wv rmsnorm(h)      every XCD computes all value rows (its members
//                             split them), exchanged inside the XCD;
//                             the query/key rows, which nothing downstream
//                             reads at position 0, are computed once over
//                             the whole grid
//   B  h1 = h + Wo gqa(v)     every XCD computes all of h1 (wo is read by
//                             each XCD), exchanged inside the XCD
//   C  s = swiglu(Wgu rmsnorm(h1)) XCD x computes its own slice of s,
//                             exchanged inside the XCD
//   D  P_x = Wdown[:, slice x] s[slice x]  (a split of down's K over XCDs)
//                             sent across XCDs: member j of every XCD reads
//                             the rows it owns from all 8 partials
//   E  h2 = h1 + sum_x P_x    (x ascending), member j's rows, exchanged
//                             inside the XCD as the next layer's h
//
// Hand-off records.  Every activation vector of the step has its own record
// in the workspace (no reuse within a step).  Each entry is one 8-byte word:
// the fp32 bits and, in the upper half, those bits XOR the step number.  A
// consumer polls the words it needs until every word decodes to the current
// step: the data itself is the signal, so there are no flags or fences
// between workgroups, and a read that raced a write can never be taken for
// current data (a torn word fails the check).  The step number lives in the
// workspace; the last workgroup to finish advances it.
//
// Inside a workgroup, waves 0-3 poll: they wait for the next stage's input
// and stage it in LDS while waves 4-15 compute the current stage.  A task is
// 4 output rows over a K range of at most 1024 (4 rounds of 16 chunks of 16
// weights): lane 4m + r holds row r's chunks 16k + m, so a task ends with
// whole dot products after a reduction over the 16 lanes of each row.  A
// weight wave owns at most one task per stage, in one of three register
// slots, and reloads a slot with the next layer's weights once the slot is
// free, so every load has most of a layer to arrive.  A compute unit's vector
// memory requests drain in order, so a burst delays every hand-off load or
// store issued behind it until the burst has streamed in (about 24 GB/s per
// compute unit while all of them load).  A burst therefore either follows the
// dot product of its stage (the down and gate/up reloads: the compiler cannot
// count loads issued under branches, so a dot product behind a reload would
// wait for the whole burst, vmcnt 0) or, for the wo reload, goes out before
// the gate/up dot products with an explicit wait for the wave's older loads
// first, so that it drains during the layer's longest compute window.
// Measured per 24-layer step: reloads before their stage's dot product
// 406 us, after it 349 us, with the wo burst moved into stage C 340 us.
//
// Every wait is bounded.  An expired wait sets bit 1 of the step's error
// word; the step then writes next_token = -1, the bit is added to the sticky
// status word, and the kernel runs to completion.  The hand-offs inside an
// XCD need every member of a group on one XCD (which one does not matter);
// q8_0_chain_prepare checks that with a probe launch of the same shape and
// otherwise sets Q8_CHAIN_COHERENT (every store device-scope).  A member that
// still lands elsewhere cannot make a consumer take wrong data (each word
// carries its step); at worst its hand-offs wait until its L2 writes the line
// back, or the wait expires.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "q8_internal.h"

namespace q8 {
namespace {

constexpr int kCT = 1024;          // threads per workgroup
constexpr int kCW = kCT / 64;      // waves per workgroup
constexpr int kPW = 4;             // poll waves
constexpr int kPL = 64 * kPW;      // poll lanes
constexpr int kXW = kCW - kPW;     // weight waves
constexpr int kRounds = 4;         // rounds of 16 chunks per task
constexpr int kTaskChunks = 16 * kRounds;
constexpr int kMaxK = 16 * kTaskChunks;  // longest K a task covers (1024)
constexpr int kNX = 8;             // XCD groups
constexpr int kMaxGrid = 1024;
constexpr int kHdrBytes = 256;
constexpr uint32_t kDefaultSpin = 1u << 16;
constexpr int kAuxDev = 16;        // cache policy sc1: device scope
constexpr int kMaxTw = 12;         // wo/down tasks of one workgroup (<= kXW)
// Optional stage timestamps (q8_0_chain_run_stamped): per workgroup,
// Q8_CHAIN_STAMP_POINTS points of each of the first Q8_CHAIN_STAMP_LAYERS
// layers, then Q8_CHAIN_STAMP_KERNEL points of the whole step.
constexpr int kStampL = Q8_CHAIN_STAMP_LAYERS;
constexpr int kStampP = Q8_CHAIN_STAMP_POINTS;
constexpr int kStampK = Q8_CHAIN_STAMP_KERNEL;
constexpr int kStampWords = kStampL * kStampP + kStampK;

enum { ST_QKV = 0, ST_WO = 1, ST_GU = 2, ST_DN = 3 };

struct ChainMat {
  const uint8_t* qs;
  const uint8_t* d;
};

// Kernel arguments: everything the step needs except the per-layer weight
// table, which lives in the workspace after the 256-byte header (ChainMat
// [L][4]: qkv, wo, gate_up, down) and is copied to LDS at the start.
struct ChainArgs {
  uint8_t* ws;
  const float* h_in;
  float* h_out;
  float* logits;
  int32_t* next_token;
  int32_t L, H, NH, NKV, HD, I, V;
  int32_t G, GS;          // grid, members per XCD group (G = kNX * GS)
  int32_t Mq, KV, NHD;    // qkv rows, value rows, attention width
  float eps;
  uint32_t flags;         // Q8_CHAIN_COHERENT
  uint32_t spin;          // polling rounds before a wait gives up
  int64_t o_qkv, o_v, o_h1, o_s, o_p, o_h2;  // byte offsets of layer 0's records
  int32_t gv, gh;         // words between the group copies of v- / h-sized records
  int64_t layer_stride;   // bytes between layers' record sets
  int64_t am_off;         // argmax partials: [kMaxGrid] (fp32 value, int32 index)
  int64_t ws_bytes;
  ChainMat lm;
  int64_t* stamps;        // [G][kStampWords] s_memrealtime ticks, or nullptr
};

struct Hdr {  // first 256 bytes of the workspace
  uint32_t step;
  uint32_t pad0[15];
  uint32_t ticket;
  uint32_t pad1[15];
  uint32_t status;  // sticky: every error bit of every run since prepare
  uint32_t pad2[15];
  uint32_t err;     // error bits of the current step (cleared at its end)
  uint32_t pad3[15];
};

__device__ __forceinline__ unsigned xcc_id() {
  unsigned v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 15u;
}

__device__ __forceinline__ float q_at(uint32_t w, int k) {
  return (float)(int32_t)(int8_t)(w >> (8 * k));
}
__device__ __forceinline__ float f16_to_f32(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}
__device__ __forceinline__ void wave_argmax(float& v, int& i) { wave_best_pair(v, i); }

// Weight pointers come from a table in memory, so the compiler cannot prove
// they are global; flat loads would also count against lgkmcnt and make every
// LDS wait (and so every barrier) wait for the prefetched weights.
template <typename T>
__device__ __forceinline__ T ld_w(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const __attribute__((address_space(1))) T*>(
      reinterpret_cast<uintptr_t>(p)));
}

// One tagged word: the fp32 bits, and those bits XOR the step.  AUX is the
// cache policy of the store: 0 inside an XCD (the L2 is shared), kAuxDev
// across XCDs (written through to memory).
template <int AUX>
__device__ __forceinline__ void st_tag(__amdgpu_buffer_rsrc_t rs, int64_t off, float v,
                                       uint32_t step) {
  const uint32_t b = __float_as_uint(v);
  const u32x2 w = {b, b ^ step};
  __builtin_amdgcn_raw_buffer_store_b64(w, rs, (int)off, 0, AUX);
}
__device__ __forceinline__ void st_tag_local(__amdgpu_buffer_rsrc_t rs, int64_t off, float v,
                                             uint32_t step, bool coherent) {
  if (coherent)
    st_tag<kAuxDev>(rs, off, v, step);
  else
    st_tag<0>(rs, off, v, step);
}

// LDS position of input entry k: 4 floats of padding after every 16, so the
// 16 chunks that the lanes of a wave read at once fall in distinct banks.
__device__ __forceinline__ int xpad(int k) { return k + ((k >> 4) << 2); }

// ---- tasks -----------------------------------------------------------------
// Tile and position (within the 64-row packed tile) of row r of a task.
struct RowPos {
  int tile, pos;
};
// rows layout: item `it` is rows 4 it .. 4 it + 3
__device__ __forceinline__ RowPos rows_item(int it, int r) { return {it >> 4, 4 * (it & 15) + r}; }
// gate/up pairs layout: pair item p is gate rows 2p, 2p + 1 (positions
// 2 (p % 16) + r) and the matching up rows (positions 32 + 2 (p % 16) + r - 2)
__device__ __forceinline__ RowPos rows_pair(int p, int r) {
  return {p >> 4, r < 2 ? 2 * (p & 15) + r : 30 + 2 * (p & 15) + r};
}

// A lane's share of one task: kRounds x (16 quants of its row in chunk
// 16 k + lane / 4, and that chunk's binary16 scale).
struct TaskW {
  u32x4 q[kRounds];
  uint32_t d[kRounds];
};

// Issue the loads of one task: chunks [c0, c0 + nc) of the row at rp of a
// matrix whose rows are Kfull long.
__device__ __forceinline__ void load_task(const ChainMat& W, int Kfull, int c0, int nc, RowPos rp,
                                          int lane, TaskW& w) {
  __asm__ volatile("" : "+v"(lane), "+v"(rp.tile), "+v"(rp.pos));
  const int Cf = Kfull >> 4, Gq = (Kfull + 127) >> 7;
#pragma unroll
  for (int k = 0; k < kRounds; ++k) {
    const int c = 16 * k + (lane >> 2);
    w.q[k] = u32x4{0, 0, 0, 0};
    w.d[k] = 0;
    if (16 * k < nc && c < nc) {
      const int cg = c0 + c;
      w.q[k] = ld_w<u32x4>(W.qs + ((int64_t)rp.tile * Cf + cg) * 1024 + rp.pos * 16);
      w.d[k] = ld_w<uint16_t>(W.d + ((int64_t)rp.tile * Gq + (cg >> 3)) * 512 + rp.pos * 8 +
                              ((cg >> 1) & 3) * 2);
    }
  }
}

// d * sum_k q[k] * x[xo + k]
__device__ __forceinline__ float lane_dot(u32x4 q, uint32_t d, const float* xs, int xo) {
  const float4* xp = reinterpret_cast<const float4*>(xs + xo);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  float p = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 v = xp[i];
    p = fmaf(q_at(w[i], 0), v.x, p);
    p = fmaf(q_at(w[i], 1), v.y, p);
    p = fmaf(q_at(w[i], 2), v.z, p);
    p = fmaf(q_at(w[i], 3), v.w, p);
  }
  return f16_to_f32(d) * p;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xf, 0xf, false));
}
// v + (the same in the other row of a pair) + (the same in the other half),
// in the same order in every lane.  The swaps are written out because both
// results of v_permlane16/32_swap are needed (VALU data moves, not loads);
// the nop covers the VALU-write to permlane-read hazard.
__device__ __forceinline__ float sum_rows(float v) {
  float a = v, b = v;
  __asm__ volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  v = a + b;
  float c = v, d = v;
  __asm__ volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(c), "+v"(d));
  return c + d;
}
// Sum over all 64 lanes (every lane gets the same bits).
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f<0x121>(v);  // row_ror:1
  v += dpp_f<0x122>(v);  // row_ror:2
  v += dpp_f<0x124>(v);  // row_ror:4
  v += dpp_f<0x128>(v);  // row_ror:8
  return sum_rows(v);
}
// Sum over the 16 lanes that hold the same row (lane & 3); every lane ends
// with the sum for its row, in the same order in every lane.
__device__ __forceinline__ float row_sum(float v) {
  v += dpp_f<0x124>(v);  // row_ror:4
  v += dpp_f<0x128>(v);  // row_ror:8
  return sum_rows(v);
}

// The 4 row sums of one task (lane r < 4 holds row r), over nc chunks of the
// input staged in LDS (padded layout, chunk c at 20 c).
__device__ __forceinline__ float task_dot(const TaskW& w, int nc, const float* xs, int lane) {
  float v = 0.f;
#pragma unroll
  for (int k = 0; k < kRounds; ++k) {
    if (16 * k < nc) {
      const int c = 16 * k + (lane >> 2);
      const float t = lane_dot(w.q[k], w.d[k], xs, 20 * (c < nc ? c : 0));
      v += c < nc ? t : 0.f;
    }
  }
  return row_sum(v);
}

// ---- polling ----------------------------------------------------------------
// Wait (bounded) until slots [0, nslots) of a record carry the current step.
// Slot sl (16 bytes, two entries) lives at byte offset addr(sl); lane pl of
// `stride` polling lanes owns slots pl + stride * q (q < NSL) and loads all
// of them every round, unconditionally: a load under a lane-dependent branch
// makes the compiler wait for every earlier load before issuing it (the
// register may still be the target of the previous round's load), which
// turns one round into NSL serial memory round trips.  put(sl, a, b) receives
// each owned slot's two values.  On expiry the lane sets bit 1 of the status
// word and `failed`, and later polls of that lane return at once.
template <int NSL, typename Addr, typename Put>
__device__ __forceinline__ void poll_rec(__amdgpu_buffer_rsrc_t rs, int nslots, int stride,
                                         uint32_t step, int pl, uint32_t spin, bool& failed,
                                         uint32_t* status, Addr addr, Put put) {
  // recompute the per-lane offsets at each poll rather than let the compiler
  // keep them live (and spilled) across the whole step
  __asm__ volatile("" : "+v"(pl));
  uint32_t todo = 0;
  int own = 0;
#pragma unroll
  for (int q = 0; q < NSL; ++q)
    if (pl + stride * q < nslots) {
      todo |= 1u << q;
      own = q;
    }
  const uint32_t all = todo;
  int off[NSL];
#pragma unroll
  for (int q = 0; q < NSL; ++q) off[q] = addr(pl + stride * (q < own ? q : own));
  u32x4 v[NSL];
  uint32_t spins = 0;
  if (failed) todo = 0;
  while (todo) {
#pragma unroll
    for (int q = 0; q < NSL; ++q) {
      // an opaque offset each round, so the loads are issued again
      __asm__ volatile("" : "+v"(off[q]));
      v[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, off[q], 0, kAuxDev);
    }
#pragma unroll
    for (int q = 0; q < NSL; ++q)
      if (((todo >> q) & 1u) && (v[q].x ^ v[q].y) == step && (v[q].z ^ v[q].w) == step)
        todo &= ~(1u << q);
    if (todo && ++spins > spin) {
      atomicOr(status, 2u);
      failed = true;
      break;
    }
  }
  if (failed) return;
#pragma unroll
  for (int q = 0; q < NSL; ++q)
    if ((all >> q) & 1u) put(pl + stride * q, __uint_as_float(v[q].x), __uint_as_float(v[q].z));
}

// The record poll of the staging waves (kPL lanes): at most 2 slots a lane
// (records of at most 1024 entries).
template <typename Addr, typename Put>
__device__ __forceinline__ void poll_stage_rec(__amdgpu_buffer_rsrc_t rs, int nslots, uint32_t step,
                                               int pl, uint32_t spin, bool& failed,
                                               uint32_t* status, Addr addr, Put put) {
  if (nslots <= kPL)
    poll_rec<1>(rs, nslots, kPL, step, pl, spin, failed, status, addr, put);
  else
    poll_rec<2>(rs, nslots, kPL, step, pl, spin, failed, status, addr, put);
}

// 1 / sqrt(mean of squares + eps) from the poll waves' partial sums, added in
// wave order.
__device__ __forceinline__ float rms_scale(const float* s_ss, int n, float eps) {
  float ss = s_ss[0];
#pragma unroll
  for (int w = 1; w < kPW; ++w) ss += s_ss[w];
  return 1.0f / sqrtf(ss / (float)n + eps);
}

// Dot product of row `lane` of 64-row tile `tile` with x (LDS, length K).
__device__ __forceinline__ float lm_tile_dot(const ChainMat& W, int K, int tile, int lane,
                                             const float* xs) {
  const int nblk = K >> 5, Gq = (nblk + 3) >> 2;
  const u32x4* qp = reinterpret_cast<const u32x4*>(W.qs + (int64_t)tile * 64 * K) + lane;
  const u32x2* dp = reinterpret_cast<const u32x2*>(W.d + (int64_t)tile * Gq * 512) + lane;
  float acc = 0.f;
  for (int g = 0; g < Gq; ++g) {
    const int nb = nblk - 4 * g < 4 ? nblk - 4 * g : 4;
    u32x4 q[8];
    const u32x2 sc = ld_w<u32x2>(dp + g * 64);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < 2 * nb) q[i] = ld_w<u32x4>(qp + (8 * g + i) * 64);
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      if (jb < nb) {
        // the block's two 16-entry chunks, each followed by 4 floats of padding
        const float4* xb0 = reinterpret_cast<const float4*>(xs + 40 * (4 * g + jb));
        const float4* xb1 = reinterpret_cast<const float4*>(xs + 40 * (4 * g + jb) + 20);
        const uint32_t w[8] = {q[2 * jb].x, q[2 * jb].y, q[2 * jb].z, q[2 * jb].w,
                               q[2 * jb + 1].x, q[2 * jb + 1].y, q[2 * jb + 1].z, q[2 * jb + 1].w};
        float p = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float4 xv = i < 4 ? xb0[i] : xb1[i - 4];
          p = fmaf(q_at(w[i], 0), xv.x, p);
          p = fmaf(q_at(w[i], 1), xv.y, p);
          p = fmaf(q_at(w[i], 2), xv.z, p);
          p = fmaf(q_at(w[i], 3), xv.w, p);
        }
        const uint32_t hb = (jb & 2) ? sc.y : sc.x;
        acc = fmaf(f16_to_f32((jb & 1) ? (hb >> 16) : (hb & 0xffffu)), p, acc);
      }
    }
  }
  return acc;
}

// [lo, hi): part i of n items split into `parts` contiguous near-equal parts
__device__ __forceinline__ void span(int n, int parts, int i, int& lo, int& hi) {
  lo = (int)((int64_t)n * i / parts);
  hi = (int)((int64_t)n * (i + 1) / parts);
}

// kStamp: the q8_0_chain_run_stamped instance; the plain instance has no
// stamp code at all (its presence alone cost 2 % of the step).
template <bool kStamp>
__global__ __launch_bounds__(kCT) void chain_kernel(const ChainArgs P) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  __shared__ float s_ss[2][kPW];  // poll waves' sums of squares: [0] h (stage A), [1] h1 (stage C)
  __shared__ float s_cv[kCW];
  __shared__ int s_ci[kCW];
  __shared__ int s_last;
  __shared__ long long s_st[kStamp ? kStampWords : 1];

  uint8_t* const ws = P.ws;
  Hdr* hdr = reinterpret_cast<Hdr*>(ws);
  const int G = P.G, GS = P.GS, L = P.L, H = P.H;
  const int b = blockIdx.x;
  const int x = b % kNX, j = b / kNX;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const bool poller = wave < kPW;
  const int cw = wave - kPW;
  const int pl = threadIdx.x;  // poll lane (poll waves only)
  const bool coherent = (P.flags & Q8_CHAIN_COHERENT) != 0;
  uint32_t* const status = &hdr->err;
  bool failed = false;
  // stage timestamps: uniform branch, nothing when stamps == nullptr
  constexpr bool stamping = kStamp;
  auto stamp = [&](int slot) { s_st[slot] = (long long)__builtin_amdgcn_s_memrealtime(); };
  auto stamp_l = [&](int l, int k) {
    if (l < kStampL) stamp(l * kStampP + k);
  };
  if (stamping) {
    for (int i = threadIdx.x; i < kStampWords; i += kCT) s_st[i] = 0;
    __syncthreads();
    if (threadIdx.x == 0) stamp(kStampL * kStampP + 0);
  }

  uint32_t step = ld_dev(&hdr->step) + 1u;
  if (step == 0u) step = 1u;

  // ---- this workgroup's tasks ------------------------------------------------
  int v0, v1, q0, q1, w0, w1, g0, g1, cs0, cs1;
  span(P.KV / 4, GS, j, v0, v1);                       // value items of member j
  span((P.Mq - P.KV) / 4, G, b, q0, q1);               // query/key items of workgroup b
  span(H / 4, GS, j, w0, w1);                          // wo / down items of member j
  span(P.I / 16, kNX, x, cs0, cs1);                    // s chunks of XCD x
  span(8 * (cs1 - cs0), GS, j, g0, g1);                // gate/up pair items of member j
  g0 += 8 * cs0;
  g1 += 8 * cs0;
  const int tv = v1 - v0, tq = q1 - q0, tw = w1 - w0, tc = g1 - g0;
  // wave assignment: A and gate/up tasks from the top weight wave down,
  // wo/down tasks from the bottom
  const int ta = kXW - 1 - cw;                         // top-down index of this wave
  const bool hasA = !poller && ta < tv + tq;
  const bool hasB = !poller && cw < tw;
  const bool hasC = !poller && ta < tc;
  const bool hasD = hasB;
  const int cslice = cs1 - cs0;                        // down's K chunks on this XCD

  // LDS: stage inputs (A and C in xb0, B and D in xb1), the layer input h
  // (residual of wo), this member's h1 rows (for E), E's partials, the table
  const int XS = max(max(H, P.NHD), 16 * cslice);
  const int XSa = (xpad(XS) + 3) & ~3, Ha = (H + 3) & ~3;
  float* const xb0 = lds;
  float* const xb1 = xb0 + XSa;
  float* const hres = xb1 + XSa;
  float* const h1s = hres + Ha;             // [4 kMaxTw]
  float* const pbuf = h1s + 4 * kMaxTw;     // [kNX][4 kMaxTw]
  ChainMat* const wt = reinterpret_cast<ChainMat*>(pbuf + kNX * 4 * kMaxTw);
  {
    const ChainMat* wg = reinterpret_cast<const ChainMat*>(ws + kHdrBytes);
    for (int i = threadIdx.x; i < 4 * L; i += kCT) wt[i] = wg[i];
  }
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      ws, 0, (int)(P.ws_bytes > 0x7fffffff ? 0x7fffffff : P.ws_bytes), 0x00020000);
  auto lrec = [&](int64_t o0, int l) -> int64_t { return o0 + (int64_t)l * P.layer_stride; };
  __syncthreads();

  // ---- weight slots: 0 = A (top waves) or D (bottom waves), 1 = B, 2 = C ----
  TaskW s0, s1, s2;
  const int KA = H, KB = P.NHD, KC = H;
  auto loadA = [&](int l) {
    // value items first, then query/key items
    const int it = ta < tv ? P.Mq / 4 - P.KV / 4 + v0 + ta : q0 + ta - tv;
    load_task(wt[4 * l + ST_QKV], KA, 0, KA >> 4, rows_item(it, lane & 3), lane, s0);
  };
  auto loadB = [&](int l) {
    load_task(wt[4 * l + ST_WO], KB, 0, KB >> 4, rows_item(w0 + cw, lane & 3), lane, s1);
  };
  auto loadC = [&](int l) {
    load_task(wt[4 * l + ST_GU], KC, 0, KC >> 4, rows_pair(g0 + ta, lane & 3), lane, s2);
  };
  auto loadD = [&](int l) {
    load_task(wt[4 * l + ST_DN], P.I, cs0, cslice, rows_item(w0 + cw, lane & 3), lane, s0);
  };
  if (L > 0) {
    if (hasA) loadA(0);
    if (hasB) loadB(0);
    if (hasC) loadC(0);
    if (hasD) loadD(0);
  }

  // ---- poll waves: stage the input h of layer 0 --------------------------------
  if (poller) {
    float ss = 0.f;
    for (int k = pl; k < H; k += kPL) {
      const float v = P.h_in[k];
      xb0[xpad(k)] = v;
      hres[k] = v;
      ss = fmaf(v, v, ss);
    }
    ss = wave_sum_dpp(ss);
    if (lane == 0) s_ss[0][wave] = ss;
  }

  const int grp = P.NH / P.NKV;
  for (int l = 0; l < L; ++l) {
    // ================= stage A: value rows (and query/key rows) ===============
    __syncthreads();
    if (stamping && threadIdx.x == 0) stamp_l(l, 0);
    if (!poller) {
      if (hasD && l > 0) loadD(l);  // slot 0 of the bottom waves is free since D(l - 1)
      if (hasA) {
        if (stamping && ta == 0) {
          __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the task's weights are in
          if (lane == 0) stamp_l(l, 12);
        }
        const float c = rms_scale(s_ss[0], H, P.eps);
        const float y = task_dot(s0, KA >> 4, xb0, lane) * c;
        if (stamping && ta == 0) {
          __builtin_amdgcn_s_waitcnt(0xC07F);
          if (lane == 0 && y == y + 0.0f) stamp_l(l, 14);
        }
        if (lane < 4) {
          if (ta < tv) {
            const int row = 4 * (v0 + ta) + lane;  // value row
            st_tag_local(rs, lrec(P.o_v, l) + ((int64_t)x * P.gv + row) * 8, y, step, coherent);
            if (x == 0)
              st_tag<0>(rs, lrec(P.o_qkv, l) + (int64_t)(P.Mq - P.KV + row) * 8, y, step);
          } else {
            const int row = 4 * (q0 + ta - tv) + lane;
            st_tag<0>(rs, lrec(P.o_qkv, l) + (int64_t)row * 8, y, step);
          }
        }
        if (stamping && lane == 0 && ta == 0) stamp_l(l, 1);
      }
    } else {
      // the value vector of this XCD -> the position-0 attention output: query
      // head h returns value head h / (n_heads / n_kv_heads)
      poll_stage_rec(
          rs, P.KV / 2, step, pl, P.spin, failed, status,
          [&](int sl) { return (int)(lrec(P.o_v, l) + ((int64_t)x * P.gv + 2 * sl) * 8); },
          [&](int sl, float a, float c2) {
            const int k = 2 * sl, g = k / P.HD, jj = k - g * P.HD;
            for (int hh = g * grp; hh < (g + 1) * grp; ++hh) {
              xb1[xpad(hh * P.HD + jj)] = a;
              xb1[xpad(hh * P.HD + jj + 1)] = c2;
            }
          });
    }
    // ================= stage B: h1 = h + Wo attn (all of h1 on every XCD) =====
    __syncthreads();
    if (stamping && threadIdx.x == 0) stamp_l(l, 2);
    if (!poller) {
      if (hasA && l + 1 < L) loadA(l + 1);
      if (hasB) {
        const float y = task_dot(s1, KB >> 4, xb1, lane);
        if (lane < 4) {
          const int row = 4 * (w0 + cw) + lane;
          const float h1 = hres[row] + y;
          h1s[4 * cw + lane] = h1;
          st_tag_local(rs, lrec(P.o_h1, l) + ((int64_t)x * P.gh + row) * 8, h1, step, coherent);
        }
        if (stamping && lane == 0 && cw == 0) stamp_l(l, 3);
      }
    } else {
      float ss = 0.f;
      poll_stage_rec(
          rs, H / 2, step, pl, P.spin, failed, status,
          [&](int sl) { return (int)(lrec(P.o_h1, l) + ((int64_t)x * P.gh + 2 * sl) * 8); },
          [&](int sl, float a, float c2) {
            xb0[xpad(2 * sl)] = a;
            xb0[xpad(2 * sl + 1)] = c2;
            ss = fmaf(a, a, ss);
            ss = fmaf(c2, c2, ss);
          });
      ss = wave_sum_dpp(ss);
      if (lane == 0) s_ss[1][wave] = ss;
    }
    // ================= stage C: this XCD's slice of s = swiglu(gate, up) ======
    __syncthreads();
    if (stamping && threadIdx.x == 0) stamp_l(l, 4);
    if (!poller) {
      // The next layer's wo burst goes out before this stage's dot products,
      // so that it drains while they run (the longest compute window of the
      // layer) instead of in front of the next hand-off.  Waiting for this
      // wave's older loads first (long complete) lets the compiler see that
      // the gate/up weights need no wait behind the new burst.
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      if (hasB && l + 1 < L) loadB(l + 1);
      if (hasC) {
        if (stamping && ta == 0) {
          __builtin_amdgcn_s_waitcnt(0x0F70);
          if (lane == 0) stamp_l(l, 13);
        }
        const float c = rms_scale(s_ss[1], H, P.eps);
        const float y = task_dot(s2, KC >> 4, xb0, lane) * c;
        if (stamping && ta == 0) {
          __builtin_amdgcn_s_waitcnt(0xC07F);
          if (lane == 0 && y == y + 0.0f) stamp_l(l, 15);
        }
        // lanes 0, 1: gate rows; 2, 3: the matching up rows (quad_perm [2,3,2,3])
        const float up = dpp_f<0xEE>(y);
        if (lane < 2) {
          const int o = 2 * (g0 + ta) + lane;
          st_tag_local(rs, lrec(P.o_s, l) + (int64_t)o * 8, y / (1.0f + expf(-y)) * up, step,
                       coherent);
        }
        if (stamping && lane == 0 && ta == 0) stamp_l(l, 5);
        if (stamping && lane == 0 && ta == tc - 1) stamp_l(l, 6);
      }
    } else {
      const int base = 16 * cs0;
      poll_stage_rec(
          rs, 8 * cslice, step, pl, P.spin, failed, status,
          [&](int sl) { return (int)(lrec(P.o_s, l) + (int64_t)(base + 2 * sl) * 8); },
          [&](int sl, float a, float c2) {
            xb1[xpad(2 * sl)] = a;
            xb1[xpad(2 * sl + 1)] = c2;
          });
    }
    // ================= stage D: this XCD's split-K partial of down ============
    __syncthreads();
    if (stamping && threadIdx.x == 0) stamp_l(l, 7);
    if (!poller) {
      if (hasD) {
        const float y = task_dot(s0, cslice, xb1, lane);
        if (lane < 4) {
          const int row = 4 * (w0 + cw) + lane;
          st_tag<kAuxDev>(rs, lrec(P.o_p, l) + ((int64_t)x * P.gh + row) * 8, y, step);
        }
        if (stamping && lane == 0 && cw == 0) stamp_l(l, 8);
      }
      if (hasC && l + 1 < L) loadC(l + 1);
    } else {
      // ---- stage E (wave 0): this member's rows of h2 = h1 + the XCDs'
      // partials in XCD order; then every poll wave stages the next h
      if (wave == 0) {
        const int nr = 4 * tw;   // rows owned, from row 4 w0
        const int per = 2 * tw;  // slots per partial
        auto addr = [&](int sl) {
          const int xs = sl / per, k = sl - xs * per;
          return (int)(lrec(P.o_p, l) + ((int64_t)xs * P.gh + 4 * w0 + 2 * k) * 8);
        };
        auto put = [&](int sl, float a, float c2) {
          const int xs = sl / per, k = sl - xs * per;
          pbuf[xs * 4 * kMaxTw + 2 * k] = a;
          pbuf[xs * 4 * kMaxTw + 2 * k + 1] = c2;
        };
        const int nsl = kNX * per;
        if (nsl > 0) {
          if (nsl <= 64)
            poll_rec<1>(rs, nsl, 64, step, lane, P.spin, failed, status, addr, put);
          else if (nsl <= 128)
            poll_rec<2>(rs, nsl, 64, step, lane, P.spin, failed, status, addr, put);
          else
            poll_rec<3>(rs, nsl, 64, step, lane, P.spin, failed, status, addr, put);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's partials are in LDS
        if (stamping && lane == 0) stamp_l(l, 9);
        if (lane < nr) {
          float h2 = h1s[lane];
#pragma unroll
          for (int xs = 0; xs < kNX; ++xs) h2 += pbuf[xs * 4 * kMaxTw + lane];
          const int row = 4 * w0 + lane;
          st_tag_local(rs, lrec(P.o_h2, l) + ((int64_t)x * P.gh + row) * 8, h2, step, coherent);
          if (x == 0 && l == L - 1 && P.h_out) P.h_out[row] = h2;
        }
        if (stamping && lane == 0) stamp_l(l, 10);
      }
      float ss = 0.f;
      poll_stage_rec(
          rs, H / 2, step, pl, P.spin, failed, status,
          [&](int sl) { return (int)(lrec(P.o_h2, l) + ((int64_t)x * P.gh + 2 * sl) * 8); },
          [&](int sl, float a, float c2) {
            xb0[xpad(2 * sl)] = a;
            xb0[xpad(2 * sl + 1)] = c2;
            hres[2 * sl] = a;
            hres[2 * sl + 1] = c2;
            ss = fmaf(a, a, ss);
            ss = fmaf(c2, c2, ss);
          });
      ss = wave_sum_dpp(ss);
      if (lane == 0) s_ss[0][wave] = ss;
      if (stamping && wave == 0 && lane == 0) stamp_l(l, 11);
    }
  }

  // ---- LM head + argmax ---------------------------------------------------
  const int V = P.V;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  if (V > 0) {
    __syncthreads();  // the final h is staged in xb0
    if (stamping && threadIdx.x == 0) stamp(kStampL * kStampP + 1);
    const float c = rms_scale(s_ss[0], H, P.eps);
    const int T = (V + 63) >> 6;
    for (int tile = wave * G + b; tile < T; tile += kCW * G) {
      const float y = lm_tile_dot(P.lm, H, tile, lane, xb0) * c;
      const int row = tile * 64 + lane;
      if (row < V) {
        P.logits[row] = y;
        if (y > bv || (y == bv && row < bi)) {
          bv = y;
          bi = row;
        }
      }
    }
    wave_argmax(bv, bi);
    if (lane == 0) {
      s_cv[wave] = bv;
      s_ci[wave] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int w = 1; w < kCW; ++w)
        if (s_cv[w] > bv || (s_cv[w] == bv && s_ci[w] < bi)) {
          bv = s_cv[w];
          bi = s_ci[w];
        }
      // one 8-byte word: the value's bits, then the index
      st_dev(reinterpret_cast<uint64_t*>(ws + P.am_off) + b,
             (uint64_t)__float_as_uint(bv) | (uint64_t)(uint32_t)bi << 32);
      if (stamping) stamp(kStampL * kStampP + 2);
    }
  }

  // ---- end of step: the last workgroup folds the argmax and advances the step.
  // The partials above are device-scope stores; each wave waits for its stores
  // to complete before the barrier, and the ticket is taken after it, so the
  // last arriver's device-scope loads see every partial.
  wait_stores();
  __syncthreads();
  if (stamping) {
    if (threadIdx.x == 0) stamp(kStampL * kStampP + 3);
    __syncthreads();
    for (int i = threadIdx.x; i < kStampWords; i += kCT)
      P.stamps[(int64_t)b * kStampWords + i] = s_st[i];
  }
  if (threadIdx.x == 0) s_last = ticket_add(&hdr->ticket) == (unsigned)(G - 1);
  __syncthreads();
  if (!s_last || wave != 0) return;
  __asm__ volatile("" ::: "memory");
  // the status word and every partial are loaded before any is compared, so
  // this fold costs one round trip (G <= kMaxGrid = 16 * 64 partials)
  const uint32_t st = ld_dev(status);
  if (V > 0) {
    const uint64_t* am = reinterpret_cast<const uint64_t*>(ws + P.am_off);
    uint64_t pw[kMaxGrid / 64];
#pragma unroll
    for (int k = 0; k < kMaxGrid / 64; ++k) {
      const int g = lane + 64 * k;
      pw[k] = 64 * k < G ? ld_dev(am + (g < G ? g : G - 1)) : 0;
    }
    float v = -INFINITY;
    int i = 0x7fffffff;
#pragma unroll
    for (int k = 0; k < kMaxGrid / 64; ++k) {
      const int g = lane + 64 * k;
      if (64 * k < G && g < G) {
        const float tv2 = __uint_as_float((uint32_t)pw[k]);
        const int ti = (int)(pw[k] >> 32);
        if (tv2 > v || (tv2 == v && ti < i)) {
          v = tv2;
          i = ti;
        }
      }
    }
    wave_argmax(v, i);
    // an expired wait anywhere in this step makes its outputs invalid: say so
    // in the token itself
    if (lane == 0) *P.next_token = st ? -1 : i;
  }
  if (lane == 0) {
    if (st) atomicOr(&hdr->status, st);
    st_dev(status, 0u);
    st_dev(&hdr->ticket, 0u);
    st_dev(&hdr->step, step);
  }
}

// Copies the values of one tagged record (n entries) to dst as plain fp32.
__global__ void chain_unpack_kernel(const uint64_t* src, int n, float* dst) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = __uint_as_float((uint32_t)src[i]);
}

__global__ void chain_status_kernel(const uint32_t* st, int32_t* out) { *out = (int32_t)*st; }

// Records the XCD of every workgroup of a grid shaped like the chain's.
__global__ __launch_bounds__(kCT) void chain_place_kernel(int32_t* out) {
  if (threadIdx.x == 0) out[blockIdx.x] = (int32_t)xcc_id();
}

// ---- host side ---------------------------------------------------------------
struct Layout {
  int32_t Mq, KV, NHD, XS, gv, gh;
  int64_t par_bytes, o_qkv, o_v, o_h1, o_s, o_p, o_h2, layer_stride, am_off, total;
  int32_t lds_bytes;
};

int64_t a256(int64_t v) { return (v + 255) / 256 * 256; }

int layout_of(const q8_0_chain_desc* c, Layout* lo) {
  if (!c) return Q8_ENULL;
  const int64_t L = c->n_layers, H = c->hidden, NH = c->n_heads, NKV = c->n_kv_heads,
                HD = c->head_dim, I = c->intermediate;
  if (L < 0 || L > 1024 || H <= 0 || NH <= 0 || NKV <= 0 || HD <= 0 || I <= 0) return Q8_EINVAL;
  if (NH % NKV || H % 32 || (NH * HD) % 32 || I % 32 || HD % 2) return Q8_EINVAL;
  if (!(c->eps >= 0.f)) return Q8_EINVAL;
  const int64_t KV = NKV * HD, Mq = (NH + 2 * NKV) * HD;
  if (KV % 4 || Mq % 4) return Q8_EINVAL;
  // a task covers a whole row of at most kMaxK weights
  if (H > kMaxK || NH * HD > kMaxK || KV > kMaxK) return Q8_EINVAL;
  if ((I / 16 + kNX - 1) / kNX * 16 > kMaxK) return Q8_EINVAL;
  if (c->vocab < 0 || c->vocab > 0x7fffffff - 64) return Q8_EINVAL;
  lo->Mq = (int32_t)Mq;
  lo->KV = (int32_t)KV;
  lo->NHD = (int32_t)(NH * HD);
  lo->XS = (int32_t)std::max(std::max(H, NH * HD), (I / 16 + kNX - 1) / kNX * 16);
  lo->gv = (int32_t)(a256(KV * 8) / 8);
  lo->gh = (int32_t)(a256(H * 8) / 8);
  lo->par_bytes = a256((int64_t)sizeof(ChainMat) * (4 * L + 1));
  int64_t o = kHdrBytes + lo->par_bytes;
  lo->o_qkv = o;
  o += a256(Mq * 8);
  lo->o_v = o;
  o += kNX * (int64_t)lo->gv * 8;
  lo->o_h1 = o;
  o += kNX * (int64_t)lo->gh * 8;
  lo->o_s = o;
  o += a256(I * 8);
  lo->o_p = o;
  o += kNX * (int64_t)lo->gh * 8;
  lo->o_h2 = o;
  o += kNX * (int64_t)lo->gh * 8;
  lo->layer_stride = o - lo->o_qkv;
  o = lo->o_qkv + lo->layer_stride * L;
  lo->am_off = o;
  o += kMaxGrid * 8;
  lo->total = o;
  const int64_t XSp = lo->XS + (lo->XS >> 4) * 4;  // padded input length
  const int64_t lds = 4 * (2 * ((XSp + 3) & ~3) + ((H + 3) & ~3) + 4 * kMaxTw +
                           kNX * 4 * kMaxTw) +
                      (int64_t)sizeof(ChainMat) * 4 * L;
  lo->lds_bytes = (int32_t)lds;
  return Q8_OK;
}

// Every workgroup's tasks fit the weight waves: value + query/key tasks on
// the top waves and wo/down tasks on the bottom ones without overlap, gate/up
// tasks within the weight waves.
int tasks_fit(const q8_0_chain_desc* c, const Layout& lo, int G) {
  if (G % kNX || G / kNX < 1) return Q8_EINVAL;
  const int GS = G / kNX;
  const int64_t I = c->intermediate;
  auto cnt = [](int64_t n, int64_t parts, int64_t i) {
    return (int)(n * (i + 1) / parts - n * i / parts);
  };
  for (int b = 0; b < G; ++b) {
    const int x = b % kNX, jm = b / kNX;
    const int tv = cnt(lo.KV / 4, GS, jm), tq = cnt((lo.Mq - lo.KV) / 4, G, b);
    const int tw = cnt(c->hidden / 4, GS, jm);
    const int64_t cs0 = I / 16 * x / kNX, cs1 = I / 16 * (x + 1) / kNX;
    const int tc = cnt(8 * (cs1 - cs0), GS, jm);
    if (tw > kMaxTw || tv + tq + tw > kXW || tc > kXW) return Q8_EINVAL;
  }
  return Q8_OK;
}

}  // namespace

size_t chain_ws_bytes(const q8_0_chain_desc* c) {
  Layout lo;
  if (layout_of(c, &lo) != Q8_OK) return 0;
  return (size_t)lo.total;
}

int chain_prepare(const q8_0_chain_desc* c, void* ws, size_t ws_bytes, q8_0_chain_plan* plan,
                  hipStream_t stream) {
  Layout lo;
  int rc = layout_of(c, &lo);
  if (rc) return rc;
  if (ws_bytes < (size_t)lo.total) return Q8_EWORKSPACE;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return Q8_ELAUNCH;
  if (cus < kNX || cus > kMaxGrid) return Q8_EINVAL;
  if ((rc = tasks_fit(c, lo, cus))) return rc;
  int maxlds = 0;
  if (hipDeviceGetAttribute(&maxlds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
      hipSuccess)
    return Q8_ELAUNCH;
  // one workgroup per compute unit: ask for more than half of the LDS when
  // the device allows it, so two workgroups never share a unit
  int lds = lo.lds_bytes;
  if (maxlds >= 96 * 1024 && lds < 84 * 1024) lds = 84 * 1024;
  if (lds > maxlds) return Q8_EINVAL;
  const void* kernels[3] = {(const void*)chain_kernel<false>, (const void*)chain_kernel<true>,
                            (const void*)chain_place_kernel};
  for (const void* k : kernels) {
    if (lds > 64 * 1024 &&
        hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess) {
      (void)hipGetLastError();
      return Q8_ELAUNCH;
    }
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, chain_kernel<true>, kCT, lds) !=
          hipSuccess ||
      per_cu < 1) {
    (void)hipGetLastError();
    return Q8_ELAUNCH;
  }

  // weight table
  std::vector<ChainMat> host((size_t)4 * c->n_layers + 1);
  for (int l = 0; l < c->n_layers; ++l) {
    const q8_0_weights* m[4] = {&c->qkv[l], &c->wo[l], &c->gate_up[l], &c->down[l]};
    for (int k = 0; k < 4; ++k) {
      host[4 * l + k].qs = static_cast<const uint8_t*>(m[k]->qs);
      host[4 * l + k].d = static_cast<const uint8_t*>(m[k]->d);
    }
  }
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  // Where the workgroups of a chain-shaped grid run: the hand-offs inside an
  // XCD rely on the members b, b + 8, b + 16, ... of a group sharing one XCD
  // (the dispatcher deals workgroups to the XCDs in turn); if a grid of this
  // shape does not, every hand-off goes through device-scope stores instead.
  std::vector<int32_t> place(cus, -1);
  int32_t* dplace = reinterpret_cast<int32_t*>(w8 + lo.am_off);
  if (hipMemsetAsync(ws, 0, (size_t)lo.total, stream) != hipSuccess) {
    (void)hipGetLastError();
    return Q8_ELAUNCH;
  }
  hipLaunchKernelGGL(chain_place_kernel, dim3(cus), dim3(kCT), lds, stream, dplace);
  if (hipGetLastError() != hipSuccess ||
      hipMemcpyAsync(place.data(), dplace, (size_t)cus * 4, hipMemcpyDeviceToHost, stream) !=
          hipSuccess ||
      hipMemsetAsync(dplace, 0, (size_t)cus * 4, stream) != hipSuccess ||
      hipMemcpyAsync(w8 + kHdrBytes, host.data(), host.size() * sizeof(ChainMat),
                     hipMemcpyHostToDevice, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess) {
    (void)hipGetLastError();
    return Q8_ELAUNCH;
  }
  bool placed = true;
  for (int i = 0; i < cus; ++i) placed &= place[i] == place[i % kNX] && place[i] >= 0;
  memset(plan, 0, sizeof(*plan));
  plan->grid = cus;
  plan->threads = kCT;
  plan->lds_bytes = lds;
  plan->n_layers = c->n_layers;
  plan->hidden = c->hidden;
  plan->n_heads = c->n_heads;
  plan->n_kv_heads = c->n_kv_heads;
  plan->head_dim = c->head_dim;
  plan->intermediate = c->intermediate;
  plan->vocab = c->vocab;
  plan->eps = c->eps;
  plan->flags = placed ? 0u : (uint32_t)Q8_CHAIN_COHERENT;
  plan->ws_bytes = lo.total;
  plan->off[Q8_CHAIN_QKV] = lo.o_qkv;
  plan->off[Q8_CHAIN_H_ATTN] = lo.o_h1;  // the copy of XCD group 0
  plan->off[Q8_CHAIN_SWIGLU] = lo.o_s;
  plan->off[Q8_CHAIN_H_OUT] = lo.o_h2;   // the copy of XCD group 0
  plan->layer_stride = lo.layer_stride;
  plan->am_off = lo.am_off;
  if (c->vocab > 0) {
    plan->lm_qs = c->lm_head->qs;
    plan->lm_d = c->lm_head->d;
  }
  plan->len[0] = lo.Mq;
  plan->len[1] = c->hidden;
  plan->len[2] = c->intermediate;
  plan->len[3] = c->hidden;
  plan->spin_limit = 0;
  plan->groups = kNX;
  plan->off_v = lo.o_v;
  plan->off_p = lo.o_p;
  plan->group_words_v = lo.gv;
  plan->group_words_h = lo.gh;
  return Q8_OK;
}

int chain_run(const q8_0_chain_plan* plan, void* ws, const float* h_in, float* h_out,
              float* logits, int32_t* next_token, int64_t* stamps, hipStream_t stream) {
  if (plan->groups != kNX || plan->grid % kNX) return Q8_EINVAL;
  ChainArgs a;
  memset(&a, 0, sizeof(a));
  a.ws = static_cast<uint8_t*>(ws);
  a.h_in = h_in;
  a.h_out = h_out;
  a.logits = logits;
  a.next_token = next_token;
  a.L = plan->n_layers;
  a.H = plan->hidden;
  a.NH = plan->n_heads;
  a.NKV = plan->n_kv_heads;
  a.HD = plan->head_dim;
  a.I = plan->intermediate;
  a.V = plan->vocab;
  a.G = plan->grid;
  a.GS = plan->grid / kNX;
  a.Mq = plan->len[0];
  a.KV = plan->n_kv_heads * plan->head_dim;
  a.NHD = plan->n_heads * plan->head_dim;
  a.eps = plan->eps;
  a.flags = plan->flags;
  a.spin = plan->spin_limit ? plan->spin_limit : kDefaultSpin;
  a.o_qkv = plan->off[Q8_CHAIN_QKV];
  a.o_h1 = plan->off[Q8_CHAIN_H_ATTN];
  a.o_s = plan->off[Q8_CHAIN_SWIGLU];
  a.o_h2 = plan->off[Q8_CHAIN_H_OUT];
  a.o_v = plan->off_v;
  a.o_p = plan->off_p;
  a.gv = plan->group_words_v;
  a.gh = plan->group_words_h;
  a.layer_stride = plan->layer_stride;
  a.am_off = plan->am_off;
  a.ws_bytes = plan->ws_bytes;
  a.lm.qs = static_cast<const uint8_t*>(plan->lm_qs);
  a.lm.d = static_cast<const uint8_t*>(plan->lm_d);
  a.stamps = stamps;
  if (stamps)
    hipLaunchKernelGGL(chain_kernel<true>, dim3(plan->grid), dim3(kCT), plan->lds_bytes, stream, a);
  else
    hipLaunchKernelGGL(chain_kernel<false>, dim3(plan->grid), dim3(kCT), plan->lds_bytes, stream,
                       a);
  if (hipGetLastError() != hipSuccess) return Q8_ELAUNCH;
  return Q8_OK;
}

int chain_read(const q8_0_chain_plan* plan, const void* ws, int32_t layer, int32_t which,
               float* dst, hipStream_t stream) {
  const uint64_t* src = reinterpret_cast<const uint64_t*>(
      static_cast<const uint8_t*>(ws) + plan->off[which] + (int64_t)layer * plan->layer_stride);
  const int n = plan->len[which];
  hipLaunchKernelGGL(chain_unpack_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, src, n,
                     dst);
  if (hipGetLastError() != hipSuccess) return Q8_ELAUNCH;
  return Q8_OK;
}

int chain_status(const void* ws, int32_t* out, hipStream_t stream) {
  const Hdr* hdr = static_cast<const Hdr*>(ws);
  hipLaunchKernelGGL(chain_status_kernel, dim3(1), dim3(1), 0, stream, &hdr->status, out);
  if (hipGetLastError() != hipSuccess) return Q8_ELAUNCH;
  return Q8_OK;
}

}  // namespace q8
