// chain.hip -- a whole decode step of a Qwen2-style decoder (every layer's
// qkv, wo, gate_up and down projections with their glue, then the LM head and
// greedy argmax) in one persistent launch.
//
// Why: at batch 1 each projection moves 0.9-9 MB, a few microseconds of HBM
// time, so a chain of one launch per projection is bound by launch and
// hand-off latency rather than bandwidth (the pages' graph and slot-fusion
// results: a per-layer task graph of fixed launches; capturing it gains about
// a third, fusing slots cuts launches).  Here one workgroup per compute unit
// stays resident for the whole step; only the activations between projections
// are dependent, so each workgroup streams the next projection's weights into
// registers while it waits for the current one's inputs.
//
// Hand-off between workgroups.  Every activation vector of the step has its
// own buffer in the workspace (no reuse within a step, so no write-after-read
// hazards).  Each entry is one 8-byte word: the fp32 bits and, in the upper
// half, those bits XOR the step number.  A consumer polls the words it needs
// with device-coherent 16-byte loads until every word decodes to the current
// step: the data itself is the signal, so there are no flags, fences or
// barriers between workgroups, and a read that raced a write can never be
// taken for current data (a torn word fails the XOR check).  The step number
// lives in the workspace; the last workgroup to finish advances it.
//
// Work split.  A layer projection is cut into items of 4 output rows (gate
// and up pairs: 2 gate + the 2 matching up rows) over the full K, spread
// round-robin over the workgroups, so no K-split partials cross workgroups.
// Inside a workgroup a wave task is (item, 16 consecutive 16-weight chunks):
// lane 4m + r holds the 16 quants of row r in chunk m of the task and its
// scale, so the four lanes of a chunk read the item's 64 contiguous packed
// bytes of that chunk (16 cache lines per load instruction, not 64) and share
// one broadcast 16-float slice of the input from LDS (laid out with 4 floats
// of padding after every 16, so the 16 slices a wave reads fall in distinct
// banks).  The 16 lanes of a row are summed by DPP/permlane rotations, and
// the tasks of one item are added in task order by whichever of them
// finishes last, which also runs the epilogue (RMS scale, residual, SwiGLU,
// tagged store).  Small tasks spread even the smallest projections over many
// waves.  Each weight wave keeps its first kPre tasks of the next projection
// with work for it in registers.  Waves 0-5 poll the inputs into LDS; waves
// 6-15 hold the weights.  The LM head is streamed: one 64-row tile per wave,
// lane = row, input broadcast from LDS.
//
// Every spin is bounded; on expiry bit 1 of the status word is set and the
// kernel runs to completion with whatever it read.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "q8_internal.h"

namespace q8 {
namespace {

constexpr int kCT = 1024;       // threads per workgroup
constexpr int kCW = kCT / 64;   // waves per workgroup
constexpr int kPW = 6;          // poll/epilogue waves
constexpr int kPL = 64 * kPW;   // poll lanes
constexpr int kXW = kCW - kPW;  // waves holding prefetched weights
constexpr int kSlots = 7;       // 16-byte poll slots per poll lane
constexpr int kMaxIn = 2 * kPL * kSlots;  // longest polled vector (5376 entries)
constexpr int kMaxTasks = 1024; // wave tasks of one workgroup in one projection
constexpr int kRounds = 4;      // rounds of 16 chunks (4 lanes each) per wave task
constexpr int kTaskChunks = 16 * kRounds;  // 16-weight chunks per wave task
constexpr int kPre = 1;         // tasks of the next projection a wave holds in registers
constexpr int kSpinMax = 1 << 18;
// Cache policy of the polling loads: sc1 (device scope: coherent across the
// XCDs' separate L2s).
constexpr int kPollAux = 16;
constexpr int kHdrBytes = 256;
constexpr int kMaxGrid = 1024;

enum { ST_QKV = 0, ST_WO = 1, ST_GU = 2, ST_DN = 3 };

struct ChainMat {
  const uint8_t* qs;
  const uint8_t* d;
};

// Kernel arguments: everything the step needs except the per-layer weight
// table, which lives in the workspace after the 256-byte header (ChainMat
// [L][4]: qkv, wo, gate_up, down) and is copied to LDS at the start.  Kernel
// arguments sit in constant memory, so reading them never waits on the
// wave's outstanding vector memory traffic.
struct ChainArgs {
  uint8_t* ws;
  const float* h_in;
  float* h_out;
  float* logits;
  int32_t* next_token;
  int32_t L, H, NH, NKV, HD, I, V, G;
  int32_t Mq;
  float eps;
  int64_t off_qkv, off_h1, off_s, off_h2;  // byte offsets of layer 0's records
  int64_t layer_stride;  // bytes between layers' record sets
  int64_t am_off;        // argmax partials: [kMaxGrid] (fp32 value, int32 index)
  int64_t ws_bytes;
  ChainMat lm;
};

struct Hdr {  // first 256 bytes of the workspace
  uint32_t step;
  uint32_t pad0[15];
  uint32_t ticket;
  uint32_t pad1[15];
  uint32_t status;
  uint32_t pad2[31];
};

__device__ __forceinline__ float q_at(uint32_t w, int k) {
  return (float)(int32_t)(int8_t)(w >> (8 * k));
}
__device__ __forceinline__ float f16_to_f32(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(v, o, 64);
    const int oi = __shfl_xor(i, o, 64);
    if (ov > v || (ov == v && oi < i)) {
      v = ov;
      i = oi;
    }
  }
}

__device__ __forceinline__ void st_tag(uint64_t* p, float v, uint32_t step) {
  const uint32_t b = __float_as_uint(v);
  st_dev(p, (uint64_t)b | ((uint64_t)(b ^ step) << 32));
}

// Weight pointers come from a table in memory, so the compiler cannot prove
// they are global; flat loads would also count against lgkmcnt and make every
// LDS wait (and so every barrier) wait for the prefetched weights.
template <typename T>
__device__ __forceinline__ T ld_w(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const __attribute__((address_space(1))) T*>(
      reinterpret_cast<uintptr_t>(p)));
}

// Per-kind constants of one workgroup's share of a projection, computed once
// per launch (integer divisions kept off the per-stage path).
struct KindInfo {
  int K, C, tpi, ntask;
  int tpi_mul;  // ceil(2^20 / tpi): tau / tpi == (tau * tpi_mul) >> 20 for tau < 1024
};

__device__ __forceinline__ KindInfo kind_info(const ChainArgs& P, int kind, int vwg) {
  int M, K;
  switch (kind) {
    case ST_QKV: M = P.Mq; K = P.H; break;
    case ST_WO: M = P.H; K = P.NH * P.HD; break;
    case ST_GU: M = 2 * P.I; K = P.H; break;
    default: M = P.H; K = P.I; break;
  }
  KindInfo ki;
  ki.K = K;
  ki.C = K >> 4;
  ki.tpi = (ki.C + kTaskChunks - 1) / kTaskChunks;
  const int n_items = M >> 2;
  const int n_it = n_items > vwg ? (n_items - 1 - vwg) / P.G + 1 : 0;
  ki.ntask = n_it * ki.tpi;
  ki.tpi_mul = ((1 << 20) + ki.tpi - 1) / ki.tpi;
  return ki;
}

// One projection of the step as seen by one workgroup.
struct Stage {
  ChainMat W;
  int kind, layer;
  int K, C, tpi, ntask, tpi_mul;
  bool pairs;
};

__device__ __forceinline__ Stage stage_of(const KindInfo* ki, const ChainMat* wt, int s) {
  Stage st;
  st.layer = s >> 2;
  st.kind = s & 3;
  st.W = wt[s];
  st.pairs = st.kind == ST_GU;
  const KindInfo k = ki[st.kind];
  st.K = k.K;
  st.C = k.C;
  st.tpi = k.tpi;
  st.ntask = k.ntask;
  st.tpi_mul = k.tpi_mul;
  return st;
}

// item (within this workgroup) and chunk block of wave task tau
__device__ __forceinline__ int task_item(const Stage& st, int tau) {
  return (tau * st.tpi_mul) >> 20;
}

// Packed-tile position of row r (0..3) of item j (0..15) of a tile.
__device__ __forceinline__ int item_pos(bool pairs, int j, int r) {
  return pairs ? (r < 2 ? 2 * j + r : 30 + 2 * j + r) : 4 * j + r;
}

// Chunk of this lane in round k of wave task tau (may be >= C: no work).
__device__ __forceinline__ int task_chunk(const Stage& st, int tau, int k, int lane) {
  return (tau - task_item(st, tau) * st.tpi) * kTaskChunks + 16 * k + (lane >> 2);
}

// The weights of one lane for one wave task: kRounds x (16 quants + scale).
struct TaskRegs {
  u32x4 q[kRounds];
  uint32_t d[kRounds];
};

// LDS position of input entry k: 4 floats of padding after every 16, so the
// 16 chunks that the lanes of a wave read at once fall in distinct banks.
__device__ __forceinline__ int xpad(int k) { return k + ((k >> 4) << 2); }

// The 16 quants of row (lane & 3) in chunk c of item `item`, and its scale.
__device__ __forceinline__ void load_lane(const Stage& st, int item, int c, int lane, u32x4& q,
                                          uint32_t& d) {
  const int Gq = (st.K + 127) >> 7;
  const int t = item >> 4;
  const int p = item_pos(st.pairs, item & 15, lane & 3);
  q = ld_w<u32x4>(st.W.qs + ((int64_t)t * st.C + c) * 1024 + p * 16);
  d = ld_w<uint16_t>(st.W.d + ((int64_t)t * Gq + (c >> 3)) * 512 + p * 8 + ((c >> 1) & 3) * 2);
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
// Sum over all 64 lanes (lane 0's value is used).
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f<0x121>(v);  // row_ror:1
  v += dpp_f<0x122>(v);  // row_ror:2
  v += dpp_f<0x124>(v);  // row_ror:4
  v += dpp_f<0x128>(v);  // row_ror:8
  return sum_rows(v);
}

// Sum over the 16 lanes that hold the same row (lane & 3); every lane ends
// with the sum for its row, in the same order in every lane.  Rotations
// within 16-lane rows (DPP) and swaps of row pairs and wave halves
// (v_permlane16/32_swap): VALU operations only, no LDS round trips.
__device__ __forceinline__ float row_sum(float v) {
  v += dpp_f<0x124>(v);  // row_ror:4
  v += dpp_f<0x128>(v);  // row_ror:8
  return sum_rows(v);
}

// Wait (bounded) until entries [0, n) of the tagged record at byte offset off
// carry the current step; put(k, value) for each, then return the sum of
// squares accumulated in a fixed order.  Poll lanes (pl < kPL) only; n even.
// Each lane owns NSL 16-byte slots (the last one repeated when it owns
// fewer) and loads all of them every round, unconditionally: a load under a
// lane-dependent branch would make the compiler wait for every earlier load
// before issuing it (the register may still be the target of the previous
// round's load), turning one round into NSL serial memory round trips.
template <int NSL, typename Put>
__device__ __forceinline__ float poll_tagged_n(__amdgpu_buffer_rsrc_t rs, int64_t off, int n,
                                               uint32_t step, int pl, uint32_t* status, Put put) {
  // recompute the per-lane offsets here rather than keep them live (and
  // spilled) across the whole step
  __asm__ volatile("" : "+v"(pl));
  const int nsl = n >> 1;
  uint32_t todo = 0;
  int own = 0;
#pragma unroll
  for (int j = 0; j < NSL; ++j)
    if (pl + kPL * j < nsl) {
      todo |= 1u << j;
      own = j;
    }
  const uint32_t all = todo;
  u32x4 v[NSL];
  int spins = 0;
  int base = (int)(off + (int64_t)pl * 16);
  while (todo) {
    // an opaque offset each round, so the loads are issued again
    __asm__ volatile("" : "+v"(base));
#pragma unroll
    for (int j = 0; j < NSL; ++j)
      v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, base + kPL * 16 * (j < own ? j : own), 0,
                                                   kPollAux);
#pragma unroll
    for (int j = 0; j < NSL; ++j)
      if (((todo >> j) & 1u) && (v[j].x ^ v[j].y) == step && (v[j].z ^ v[j].w) == step)
        todo &= ~(1u << j);
    if (todo && ++spins > kSpinMax) {
      atomicOr(status, 2u);
      break;
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NSL; ++j) {
    if ((all >> j) & 1u) {
      const int k = 2 * (pl + kPL * j);
      const float a = __uint_as_float(v[j].x), b = __uint_as_float(v[j].z);
      put(k, a);
      put(k + 1, b);
      ss = fmaf(a, a, ss);
      ss = fmaf(b, b, ss);
    }
  }
  return ss;
}

template <typename Put>
__device__ __forceinline__ float poll_tagged(__amdgpu_buffer_rsrc_t rs, int64_t off, int n,
                                             uint32_t step, int pl, uint32_t* status, Put put) {
  const int nsl = (n >> 1) > 0 ? (n >> 1) : 1;
  switch ((nsl + kPL - 1) / kPL) {
    case 1: return poll_tagged_n<1>(rs, off, n, step, pl, status, put);
    case 2: return poll_tagged_n<2>(rs, off, n, step, pl, status, put);
    case 3: return poll_tagged_n<3>(rs, off, n, step, pl, status, put);
    case 4: return poll_tagged_n<4>(rs, off, n, step, pl, status, put);
    case 5: return poll_tagged_n<5>(rs, off, n, step, pl, status, put);
    case 6: return poll_tagged_n<6>(rs, off, n, step, pl, status, put);
    default: return poll_tagged_n<kSlots>(rs, off, n, step, pl, status, put);
  }
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

__global__ __launch_bounds__(kCT) void chain_kernel(const ChainArgs P) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  __shared__ float s_ss[2][kPW];     // poll waves' sums of squares, by stage parity
  __shared__ int s_cnt[kMaxTasks];   // per-item arrivals of wave tasks
  __shared__ KindInfo s_ki[4];
  __shared__ float s_cv[kCW];
  __shared__ int s_ci[kCW];
  __shared__ int s_last;

  uint8_t* const ws = P.ws;
  Hdr* hdr = reinterpret_cast<Hdr*>(ws);
  const int G = P.G, L = P.L, H = P.H;
  const int bid = blockIdx.x;
  const int vwg = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const bool poller = wave < kPW;
  const int cw = wave - kPW;
  const int pl = threadIdx.x;  // poll lane (poll waves only)
  const int NS = 4 * L;

  uint32_t step = ld_dev(&hdr->step) + 1u;
  if (step == 0u) step = 1u;

  // LDS: stage inputs and residual copies are double-buffered so that the
  // poll waves can stage projection s+1 while the weight waves work on s
  const int XS = P.I > H ? (P.I > P.NH * P.HD ? P.I : P.NH * P.HD)
                        : (H > P.NH * P.HD ? H : P.NH * P.HD);
  const int XSa = (xpad(XS) + 3) & ~3, Ha = (H + 3) & ~3;
  float* const xsb = lds;                    // [2][XSa] inputs by stage parity
  float* const hres = xsb + 2 * XSa;         // [2][Ha]: before attention, before MLP
  float* const red = hres + 2 * Ha;          // [task][4] row partial sums
  ChainMat* const wt = reinterpret_cast<ChainMat*>(red + kMaxTasks * 4);
  {
    const ChainMat* wg = reinterpret_cast<const ChainMat*>(ws + kHdrBytes);
    for (int i = threadIdx.x; i < 4 * L; i += kCT) wt[i] = wg[i];
    for (int i = threadIdx.x; i < kMaxTasks; i += kCT) s_cnt[i] = 0;
    if (threadIdx.x < 4) s_ki[threadIdx.x] = kind_info(P, threadIdx.x, vwg);
  }
  __syncthreads();
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      ws, 0, (int)(P.ws_bytes > 0x7fffffff ? 0x7fffffff : P.ws_bytes), 0x00020000);
  auto rec = [&](int layer, int kind) -> int64_t {
    const int64_t o = kind == ST_QKV ? P.off_qkv
                      : kind == ST_WO  ? P.off_h1
                      : kind == ST_GU  ? P.off_s
                                       : P.off_h2;
    return o + (int64_t)layer * P.layer_stride;
  };
  auto recp = [&](int layer, int kind) -> uint64_t* {
    return reinterpret_cast<uint64_t*>(ws + rec(layer, kind));
  };

  // ---- poll waves: stage the input of projection s (s == NS: LM head) ------
  auto poll_stage = [&](int s) {
    float* xs = xsb + (s & 1) * XSa;
    const int kind = s & 3, l = s >> 2;
    float ss = 0.f;
    if (s == NS || kind == ST_QKV || kind == ST_GU) {
      float* hr = hres + (kind == ST_GU && s < NS ? Ha : 0);
      if (s == 0) {
        for (int k = pl; k < H; k += kPL) {
          const float v = P.h_in[k];
          xs[xpad(k)] = v;
          hr[k] = v;
          ss = fmaf(v, v, ss);
        }
      } else {
        const int64_t off = kind == ST_GU && s < NS ? rec(l, ST_WO) : rec(l - 1, ST_DN);
        ss = poll_tagged(rs, off, H, step, pl, &hdr->status, [&](int k, float v) {
          xs[xpad(k)] = v;
          hr[k] = v;
        });
      }
      ss = wave_sum_dpp(ss);
      if (lane == 0) s_ss[s & 1][wave] = ss;
    } else if (kind == ST_WO) {
      // the position-0 attention output: query head h returns the value
      // vector of key/value head h / (n_heads / n_kv_heads), so value entry
      // k goes to every query head of its group
      const int64_t off = rec(l, ST_QKV) + (int64_t)(P.NH + P.NKV) * P.HD * 8;
      const int grp = P.NH / P.NKV;
      poll_tagged(rs, off, P.NKV * P.HD, step, pl, &hdr->status, [&](int k, float v) {
        const int g = k / P.HD, j = k - g * P.HD;
        for (int h = g * grp; h < (g + 1) * grp; ++h) xs[xpad(h * P.HD + j)] = v;
      });
    } else {
      poll_tagged(rs, rec(l, ST_GU), P.I, step, pl, &hdr->status,
                  [&](int k, float v) { xs[xpad(k)] = v; });
    }
  };

  // ---- weight waves: which wave takes which task ----------------------------
  // Tasks of the small projections go to different waves (down from wave 0,
  // qkv after it, wo after that; gate_up spreads over all), so that most
  // waves' next task is one or more projections away and its weights can be
  // loaded that early.
  int nt[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) nt[k] = NS > 0 ? s_ki[k].ntask : 0;
  const int cap_dn = nt[ST_DN] < kXW ? nt[ST_DN] : kXW;
  const int cap_qkv = nt[ST_QKV] < kXW ? nt[ST_QKV] : kXW;
  auto base_of = [&](int kind) {
    return kind == ST_QKV ? cap_dn % kXW : kind == ST_WO ? (cap_dn + cap_qkv) % kXW : 0;
  };
  auto first_task = [&](int kind) { return (cw - base_of(kind) + kXW) % kXW; };
  // next projection (from s on, within one layer's worth) with a task for
  // this wave, or -1
  auto next_work = [&](int s) {
    const int end = s + 4 < NS ? s + 4 : NS;
    for (int s2 = s; s2 < end; ++s2)
      if (first_task(s2 & 3) < nt[s2 & 3]) return s2;
    return -1;
  };
  TaskRegs pf[kPre];
  int pf_s = -1;
  // the weights of this wave's first kPre tasks of projection s
  auto prefetch = [&](int s) {
    pf_s = s;
    if (s < 0) return;
    const Stage nx = stage_of(s_ki, wt, s);
    const int tau0 = first_task(nx.kind);
#pragma unroll
    for (int j = 0; j < kPre; ++j) {
      const int tau = tau0 + j * kXW;
      if (tau < nx.ntask) {
        const int item = vwg + task_item(nx, tau) * G;
#pragma unroll
        for (int k = 0; k < kRounds; ++k) {
          const int c = task_chunk(nx, tau, k, lane);
          pf[j].q[k] = u32x4{0, 0, 0, 0};
          pf[j].d[k] = 0;
          if (c < nx.C) load_lane(nx, item, c, lane, pf[j].q[k], pf[j].d[k]);
        }
      }
    }
  };

  if (poller) {
    poll_stage(0);
  } else if (NS > 0) {
    prefetch(next_work(0));
  }

  for (int s = 0; s < NS; ++s) {
    __syncthreads();  // A(s): input of s staged; every wave done with s - 1
    if (poller) {
      // start polling once this workgroup's own outputs of s are written:
      // the others' finish at about the same time, so one round usually
      // finds everything, and idle rounds would only add memory traffic
      __syncthreads();  // B(s)
      if (s + 1 < NS || P.V > 0) poll_stage(s + 1);
      continue;
    }
    const Stage st = stage_of(s_ki, wt, s);
    const int l = st.layer;
    const float* xs = xsb + (s & 1) * XSa;
    auto x_off = [&](int c) { return 20 * c; };
    // one wave task: 16 chunks of one item (4 rows); the last task of an item
    // to finish folds the item's partials in task order and writes its outputs
    auto run_task = [&](int tau, const TaskRegs& w) {
      float v = 0.f;
#pragma unroll
      for (int k = 0; k < kRounds; ++k) {
        // every round reads a valid chunk (its own, else chunk 0), with no
        // branch, so that the rounds' LDS reads can be issued together; the
        // weights of a chunk past the row end are zero and its sum is dropped
        const int c = task_chunk(st, tau, k, lane);
        const float t = lane_dot(w.q[k], w.d[k], xs, x_off(c < st.C ? c : 0));
        v += c < st.C ? t : 0.f;
      }
      v = row_sum(v);
      const int it = task_item(st, tau);
      float y = v;
      if (st.tpi > 1) {
        if (lane < 4) red[tau * 4 + lane] = v;
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): partials written
        int arrived = 0;
        if (lane == 0) arrived = atomicAdd(&s_cnt[it], 1);
        arrived = __builtin_amdgcn_readfirstlane(arrived);
        if (arrived != st.tpi - 1) return;
        if (lane == 0) s_cnt[it] = 0;
        y = 0.f;
        if (lane < 4) {
          const float* rp = red + it * st.tpi * 4 + lane;
          for (int cb = 0; cb < st.tpi; ++cb) y += rp[cb * 4];
        }
      }
      const int item = vwg + it * G;
      const int t = item >> 4, j = item & 15;
      if (st.kind == ST_QKV || st.kind == ST_GU) y *= rms_scale(s_ss[s & 1], H, P.eps);
      if (st.kind == ST_GU) {
        // lanes 0, 1: gate rows; 2, 3: the matching up rows (quad_perm [2,3,2,3])
        const float up = dpp_f<0xEE>(y);
        if (lane < 2) st_tag(recp(l, ST_GU) + 32 * t + 2 * j + lane, y / (1.0f + expf(-y)) * up, step);
      } else if (lane < 4) {
        const int row = 64 * t + 4 * j + lane;
        if (st.kind == ST_QKV) {
          st_tag(recp(l, ST_QKV) + row, y, step);
        } else {
          const float out = hres[(st.kind == ST_DN ? Ha : 0) + row] + y;
          st_tag(recp(l, st.kind) + row, out, step);
          if (st.kind == ST_DN && l == L - 1 && P.h_out) P.h_out[row] = out;
        }
      }
    };
    int tau = first_task(st.kind);
    if (pf_s == s) {
#pragma unroll
      for (int j = 0; j < kPre; ++j) {
        if (tau < st.ntask) {
          TaskRegs w = pf[j];
          // keep arithmetic on the prefetched registers after barrier A
#pragma unroll
          for (int k = 0; k < kRounds; ++k) __asm__ volatile("" : "+v"(w.q[k]), "+v"(w.d[k]));
          run_task(tau, w);
        }
        tau += kXW;
      }
    }
    for (; tau < st.ntask; tau += kXW) {
      TaskRegs w;
      const int item = vwg + task_item(st, tau) * G;
#pragma unroll
      for (int k = 0; k < kRounds; ++k) {
        const int c = task_chunk(st, tau, k, lane);
        w.q[k] = u32x4{0, 0, 0, 0};
        w.d[k] = 0;
        if (c < st.C) load_lane(st, item, c, lane, w.q[k], w.d[k]);
      }
      run_task(tau, w);
    }
    __syncthreads();  // B(s)
    // the next projection with work for this wave streams in from now on
    // (issued after B: a full memory pipeline stalls the issuing wave)
    if (pf_s <= s) prefetch(next_work(s + 1));
  }

  // ---- LM head + argmax ---------------------------------------------------
  const int V = P.V;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  if (V > 0) {
    __syncthreads();  // A(LM)
    const float* xs = xsb + (NS & 1) * XSa;
    const float c = rms_scale(s_ss[NS & 1], H, P.eps);
    const int T = (V + 63) >> 6;
    for (int tile = wave * G + vwg; tile < T; tile += kCW * G) {
      const float y = lm_tile_dot(P.lm, H, tile, lane, xs) * c;
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
      st_dev(reinterpret_cast<float*>(ws + P.am_off) + 2 * vwg, bv);
      st_dev(reinterpret_cast<int32_t*>(ws + P.am_off) + 2 * vwg + 1, bi);
    }
  }

  // ---- end of step: the last workgroup folds the argmax and advances the step
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) s_last = ticket_add(&hdr->ticket) == (unsigned)(G - 1);
  __syncthreads();
  if (!s_last || wave != 0) return;
  if (V > 0) {
    float v = -INFINITY;
    int i = 0x7fffffff;
    for (int g = lane; g < G; g += 64) {
      const float tv = ld_dev(reinterpret_cast<const float*>(ws + P.am_off) + 2 * g);
      const int ti = ld_dev(reinterpret_cast<const int32_t*>(ws + P.am_off) + 2 * g + 1);
      if (tv > v || (tv == v && ti < i)) {
        v = tv;
        i = ti;
      }
    }
    wave_argmax(v, i);
    if (lane == 0) *P.next_token = i;
  }
  if (lane == 0) {
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

// ---- host side ---------------------------------------------------------------
struct Layout {
  int32_t Mq, XS;
  int64_t par_bytes, off[4], layer_stride, am_off, total;
  int32_t lds_bytes;
};

int layout_of(const q8_0_chain_desc* c, Layout* lo) {
  if (!c) return Q8_ENULL;
  const int64_t L = c->n_layers, H = c->hidden, NH = c->n_heads, NKV = c->n_kv_heads,
                HD = c->head_dim, I = c->intermediate;
  if (L < 0 || L > 1024 || H <= 0 || NH <= 0 || NKV <= 0 || HD <= 0 || I <= 0) return Q8_EINVAL;
  if (NH % NKV || H % 32 || (NH * HD) % 32 || I % 32 || HD % 16) return Q8_EINVAL;
  if (!(c->eps >= 0.f)) return Q8_EINVAL;
  const int64_t Mq = (NH + 2 * NKV) * HD;
  if (Mq % 4) return Q8_EINVAL;
  if (H > kMaxIn || NH * HD > kMaxIn || I > kMaxIn || NKV * HD > kMaxIn) return Q8_EINVAL;
  if (c->vocab < 0 || c->vocab > 0x7fffffff - 64) return Q8_EINVAL;
  // wave tasks per workgroup must fit the partial-sum area (checked for one
  // workgroup per compute unit at launch; 64 is the smallest grid accepted)
  const int64_t shapes[4][2] = {{Mq, H}, {H, NH * HD}, {2 * I, H}, {H, I}};
  for (auto& sh : shapes) {
    const int64_t items = sh[0] / 4, tpi = (sh[1] / 16 + kTaskChunks - 1) / kTaskChunks;
    if (((items + 63) / 64) * tpi > kMaxTasks) return Q8_EINVAL;
  }
  lo->Mq = (int32_t)Mq;
  lo->XS = (int32_t)std::max(std::max(H, NH * HD), I);
  lo->par_bytes = (int64_t)align_up(sizeof(ChainMat) * (4 * L + 1), 256);
  int64_t o = kHdrBytes + lo->par_bytes;
  const int64_t len[4] = {Mq, H, I, H};
  for (int k = 0; k < 4; ++k) {
    lo->off[k] = o;
    o += (int64_t)align_up(len[k] * 8, 256);
  }
  lo->layer_stride = o - lo->off[0];
  o = lo->off[0] + lo->layer_stride * L;
  lo->am_off = o;
  o += kMaxGrid * 8;
  lo->total = o;
  const int64_t XSp = lo->XS + (lo->XS >> 4) * 4;  // padded input length
  const int64_t lds = 4 * (2 * ((XSp + 3) & ~3) + 2 * ((H + 3) & ~3) + kMaxTasks * 4) +
                      (int64_t)sizeof(ChainMat) * 4 * L;
  lo->lds_bytes = (int32_t)lds;
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
  if (cus < 64 || cus > kMaxGrid) return Q8_EINVAL;
  // the partial-sum area must hold every workgroup's wave tasks at this grid
  const int64_t H = c->hidden, I = c->intermediate, NHD = (int64_t)c->n_heads * c->head_dim;
  const int64_t shapes[4][2] = {{lo.Mq, H}, {H, NHD}, {2 * I, H}, {H, I}};
  for (auto& sh : shapes) {
    const int64_t items = sh[0] / 4, tpi = (sh[1] / 16 + kTaskChunks - 1) / kTaskChunks;
    if (((items + cus - 1) / cus) * tpi > kMaxTasks) return Q8_EINVAL;
  }
  int maxlds = 0;
  if (hipDeviceGetAttribute(&maxlds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
      hipSuccess)
    return Q8_ELAUNCH;
  // one workgroup per compute unit: ask for more than half of the LDS when
  // the device allows it, so two workgroups never share a unit
  int lds = lo.lds_bytes;
  if (maxlds >= 96 * 1024 && lds < 84 * 1024) lds = 84 * 1024;
  if (lds > maxlds) return Q8_EINVAL;
  if (lds > 64 * 1024 &&
      hipFuncSetAttribute((const void*)chain_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                          lds) != hipSuccess) {
    (void)hipGetLastError();
    return Q8_ELAUNCH;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, chain_kernel, kCT, lds) !=
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
  if (hipMemsetAsync(ws, 0, (size_t)lo.total, stream) != hipSuccess ||
      hipMemcpyAsync(w8 + kHdrBytes, host.data(), host.size() * sizeof(ChainMat),
                     hipMemcpyHostToDevice, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess) {
    (void)hipGetLastError();
    return Q8_ELAUNCH;
  }
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
  plan->ws_bytes = lo.total;
  for (int k = 0; k < 4; ++k) plan->off[k] = lo.off[k];
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
  return Q8_OK;
}

int chain_run(const q8_0_chain_plan* plan, void* ws, const float* h_in, float* h_out,
              float* logits, int32_t* next_token, hipStream_t stream) {
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
  a.Mq = plan->len[0];
  a.eps = plan->eps;
  a.off_qkv = plan->off[0];
  a.off_h1 = plan->off[1];
  a.off_s = plan->off[2];
  a.off_h2 = plan->off[3];
  a.layer_stride = plan->layer_stride;
  a.am_off = plan->am_off;
  a.ws_bytes = plan->ws_bytes;
  a.lm.qs = static_cast<const uint8_t*>(plan->lm_qs);
  a.lm.d = static_cast<const uint8_t*>(plan->lm_d);
  hipLaunchKernelGGL(chain_kernel, dim3(plan->grid), dim3(kCT), plan->lds_bytes, stream, a);
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
