// gemv.hip -- Q8_0 GEMV kernels for gfx950 (CDNA4) and their host launcher.
//
// One kernel body serves every GEMV-shaped step of the decode path: the dense
// projections (qkv, wo, gate_up, down, lm_head) of the decode step profiled in
// the "Lumen v0.3.0" release notes ("Phase 7.E.0"), the small-N verify chunk
// ("skuznetsov/cogni-ml" README, target-verifier chunks), and the routed-expert
// FFN of the "#144" Qwen1.5-MoE PR with all slots in one launch (routed-expert
// fusion comments: slot index folded into the work-group id for gate/up; the
// down projection looping over slots with one running accumulation).
//
// Mapping (MI355X-first, not the pages' warp-per-row designs):
//  * A packed tile holds 64 rows; lane i of a wave owns row i of the tile, so a
//    wave's 16-byte quant load covers 64 rows x 16 weights = 1 KiB of
//    contiguous HBM (global_load_dwordx4, non-temporal), and its 8-byte scale
//    load covers 4 blocks of all 64 rows (512 B contiguous).
//  * The activation vector is the same for every lane.  Each wave keeps the
//    activations of the blocks in flight in VGPRs, 16 lanes' worth replicated
//    in the four 16-lane rows, loaded one quad ahead with the weights, and the
//    FMA reads them through a DPP row broadcast (v_fmac_f32_dpp
//    row_newbcast): each weight costs one int8->fp32 convert (SDWA byte
//    select) and one FMA per column, with no instruction spent moving the
//    activation and no scalar-cache latency on the critical path.  No LDS
//    traffic on the hot loop and no cross-lane reduction per row.
//  * A tile's K range is split into "units", one per wave; units of one tile
//    are folded in a fixed order (bitwise reproducible).  When a tile's units
//    span several workgroups, each writes its partials to the workspace and
//    the last-arriving workgroup (ticket counter) folds them in unit order and
//    resets the ticket for the next call.  The L2 of each of the 8 XCDs is not
//    coherent with the others, and an agent-scope fence writes back and
//    invalidates a whole L2; issued by every workgroup that costs more than
//    the GEMV itself.  So everything exchanged between workgroups is written
//    and read with device-scope atomic stores/loads (coherent at the memory
//    side), each wave waits for its stores to complete (vmcnt 0) before the
//    workgroup barrier, and only then is the ticket incremented.
//  * No matrix cores: at N <= 8 the product is HBM-bound, not a dense
//    contraction worth MFMA tiles.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <utility>

#include "q8_internal.h"

namespace q8 {

// Signed byte k of a 32-bit word, converted exactly to fp32.
__device__ __forceinline__ float q_at(uint32_t w, int k) {
  return (float)(int32_t)(int8_t)(w >> (8 * k));
}

// binary16 bits -> fp32 (exact, subnormals included).
__device__ __forceinline__ float f16_to_f32(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// Scale of block j (0..3) of a quad held as two dwords.
__device__ __forceinline__ uint32_t quad_bits(u32x2 sc, int j) {
  const uint32_t w = (j & 2) ? sc.y : sc.x;
  return (j & 1) ? (w >> 16) : (w & 0xffffu);
}

// Start of the 32 activations of block b (all columns offset by n * xs).
__device__ __forceinline__ const float* x_block(const float* x, int b, int gqa_group, int gqa_hd,
                                                int64_t gqa_off) {
  if (gqa_group > 0) {
    const int k = b * 32;
    const int head = k / gqa_hd;
    return x + gqa_off + (int64_t)(head / gqa_group) * gqa_hd + (k - head * gqa_hd);
  }
  return x + (int64_t)b * 32;
}

// ---- activations in VGPRs, read through a DPP row broadcast ----------------
// The activations are the same for every lane (row).  Each wave holds them in
// VGPRs: for block b and column n, lane l of every 16-lane row holds
// x[n][32b + (l % 16)] in `a` and x[n][32b + 16 + (l % 16)] in `b` (plain
// dword loads of 64 distinct bytes; the four rows read the same addresses,
// and they are loaded one quad ahead together with the weights, so their
// latency hides behind the weight stream).  The FMA of weight j reads
// lane j % 16 of its row through the DPP row_newbcast operand, so every lane
// sees the same activation and no instruction is spent moving it.  The DPP
// source registers are only ever written by loads: a VALU write to a DPP
// source needs wait states, which inline assembly would not get.

// acc += (xv of lane J of this lane's 16-lane row) * q
template <int J>
__device__ __forceinline__ void fmac_row_bcast(float& acc, float xv, float q) {
  asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
      : "+v"(acc)
      : "v"(xv), "v"(q), "i"(J));
}

template <int N>
struct XBlock {
  float a[N], b[N];
};

template <int N>
__device__ __forceinline__ void load_xblock(const float* xg, int64_t xs, int xl, XBlock<N>& X) {
#pragma unroll
  for (int n = 0; n < N; ++n) {
    X.a[n] = xg[n * xs + xl];
    X.b[n] = xg[n * xs + 16 + xl];
  }
}

template <int N, int J>
__device__ __forceinline__ void xv_step(const uint32_t (&w)[8], const XBlock<N>& X,
                                        float (&p)[N]) {
  const float qf = q_at(w[J >> 2], J & 3);
#pragma unroll
  for (int n = 0; n < N; ++n) fmac_row_bcast<J & 15>(p[n], J < 16 ? X.a[n] : X.b[n], qf);
}

template <int N, int... J>
__device__ __forceinline__ void xv_steps(const uint32_t (&w)[8], const XBlock<N>& X, float (&p)[N],
                                         std::integer_sequence<int, J...>) {
  (xv_step<N, J>(w, X, p), ...);
}

// acc[n] += d * sum_j q[j] * x[n][32b + j] with the activations of XBlock.
template <int N>
__device__ __forceinline__ void block_fma_xv(u32x4 q0, u32x4 q1, const XBlock<N>& X, float dsc,
                                             float (&acc)[N]) {
  const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
  float p[N];
#pragma unroll
  for (int n = 0; n < N; ++n) p[n] = 0.f;
  xv_steps<N>(w, X, p, std::make_integer_sequence<int, 32>{});
#pragma unroll
  for (int n = 0; n < N; ++n) acc[n] = fmaf(dsc, p[n], acc[n]);
}

// One scale quad of one tile: 8 quant chunks, the scales, the activations.
template <int N>
struct QuadBuf {
  u32x4 q[8];
  u32x2 sc;
  XBlock<N> x[4];
};

template <int N>
__device__ __forceinline__ void quad_load(QuadBuf<N>& B, const u32x4* qp, const u32x2* dp, int g,
                                          const float* x, int64_t xs, int xl, int gg, int ghd,
                                          int64_t goff) {
  B.sc = __builtin_nontemporal_load(dp + g * 64);
#pragma unroll
  for (int i = 0; i < 8; ++i) B.q[i] = __builtin_nontemporal_load(qp + (8 * g + i) * 64);
#pragma unroll
  for (int j = 0; j < 4; ++j) load_xblock<N>(x_block(x, 4 * g + j, gg, ghd, goff), xs, xl, B.x[j]);
}

template <int N>
__device__ __forceinline__ void quad_fma(const QuadBuf<N>& B, float (&acc)[N]) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    block_fma_xv<N>(B.q[2 * j], B.q[2 * j + 1], B.x[j], f16_to_f32(quad_bits(B.sc, j)), acc);
}

// Partial dot products of the 64 rows of one tile over blocks [b0, b1).
// qs_tile / d_tile point at the tile's packed quants / scales.  Whole quads
// are double-buffered without loop-carried register copies (two named
// buffers, two quads per trip).
template <int N>
__device__ __forceinline__ void dot_range(const uint8_t* qs_tile, const uint8_t* d_tile, int b0,
                                             int b1, int lane, const float* x, int64_t xs, int gg,
                                             int ghd, int64_t goff, float (&acc)[N]) {
  const u32x4* qp = reinterpret_cast<const u32x4*>(qs_tile) + lane;
  const u32x2* dp = reinterpret_cast<const u32x2*>(d_tile) + lane;
  const int xl = lane & 15;
  int b = b0;
  for (; b < b1 && (b & 3); ++b) {
    XBlock<N> X;
    const u32x2 sc = __builtin_nontemporal_load(dp + (b >> 2) * 64);
    const u32x4 q0 = __builtin_nontemporal_load(qp + (2 * b) * 64);
    const u32x4 q1 = __builtin_nontemporal_load(qp + (2 * b + 1) * 64);
    load_xblock<N>(x_block(x, b, gg, ghd, goff), xs, xl, X);
    block_fma_xv<N>(q0, q1, X, f16_to_f32(quad_bits(sc, b & 3)), acc);
  }
  const int nq = (b1 - b) >> 2;
  if (nq > 0) {
    const int g0 = b >> 2;
    QuadBuf<N> A, B;
    quad_load<N>(A, qp, dp, g0, x, xs, xl, gg, ghd, goff);
    int it = 0;
    for (; it + 1 < nq; it += 2) {
      quad_load<N>(B, qp, dp, g0 + it + 1, x, xs, xl, gg, ghd, goff);
      quad_fma<N>(A, acc);
      if (it + 2 < nq) quad_load<N>(A, qp, dp, g0 + it + 2, x, xs, xl, gg, ghd, goff);
      quad_fma<N>(B, acc);
    }
    if (it < nq) quad_fma<N>(A, acc);
    b += 4 * nq;
  }
  for (; b < b1; ++b) {
    XBlock<N> X;
    const u32x2 sc = __builtin_nontemporal_load(dp + (b >> 2) * 64);
    const u32x4 q0 = __builtin_nontemporal_load(qp + (2 * b) * 64);
    const u32x4 q1 = __builtin_nontemporal_load(qp + (2 * b + 1) * 64);
    load_xblock<N>(x_block(x, b, gg, ghd, goff), xs, xl, X);
    block_fma_xv<N>(q0, q1, X, f16_to_f32(quad_bits(sc, b & 3)), acc);
  }
}

// ---- row groups: several columns, activations not replicated ---------------
// With N >= kRowGroupN columns the replicated activations above cost 16 N
// VGPRs per block in flight (64 N per quad), which caps the waves a SIMD
// holds and with them the hiding of each wave's load latency.  Here the 16-
// lane row r of a wave takes block r of each quad instead, for the 64 rows of
// the tile in four row groups: lane 16r + j computes rows 16q + j (q = 0..3)
// of block 4g + r.  A lane row then needs the activations of its own block
// only (one XBlock a quad instead of four), the weights are loaded as the
// same 16-byte pieces of the same packed tile (four 256-byte runs per load
// instead of one 1 KiB run), and each lane keeps four partial sums per
// column.  Each row group's weights of the next quad are loaded right after
// that row group's products, into the registers they just freed, so one quad
// of weights is in flight with one quad's registers.  Loads are never
// conditional (past the range they re-read the last quad, which the L2 still
// holds), so the compiler's wait counts stay exact.  At the end of the range
// the four lane rows' sums of each row group are added across rows with two
// lane-half swaps (permlane32, then permlane16) in a fixed order,
// ((r0 + r2) + (r1 + r3)), which leaves row 16q + j's total in lane 16q + j:
// the layout dot_range produces.
constexpr int kRowGroupN = 4;

// Where lane row r finds block 4g + r of a quad (clamped into [b0, b1)).
// Offsets are 32-bit and from bases every lane shares, so the loads take the
// scalar-base, vector-offset form with no 64-bit address arithmetic.
struct RgPos {
  uint32_t qoff;   // byte offset of the lane's first 16 weights (row group 0)
  uint32_t doff;   // byte offset of the dword holding the lane's block scale
  uint32_t xoff;   // byte offset of activation j of the lane row's block
  uint32_t sh;     // 0 or 16: the half of that dword
  bool ok;         // the block lies in [b0, b1) (else it adds nothing)
};

__device__ __forceinline__ RgPos rg_pos(int g, int r, int j, int b0, int b1) {
  RgPos P;
  const int blk = 4 * g + r;
  P.ok = blk >= b0 && blk < b1;
  const int bc = blk < b0 ? b0 : (blk < b1 ? blk : b1 - 1);
  P.qoff = (uint32_t)((2 * bc * 64 + j) * 16);
  P.doff = (uint32_t)((128 * (bc >> 2) + 2 * j + ((bc >> 1) & 1)) * 4);
  P.sh = (uint32_t)(bc & 1) * 16;
  P.xoff = (uint32_t)((bc * 32 + j) * 4);
  return P;
}

// Activations of the lane row's block: x[n][k0 + j] and x[n][k0 + 16 + j].
template <int N>
__device__ __forceinline__ void rg_xload(const float* x, int64_t xs, uint32_t xoff,
                                         XBlock<N>& X) {
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const char* xn = reinterpret_cast<const char*>(x + n * xs);
    X.a[n] = *reinterpret_cast<const float*>(xn + xoff);
    X.b[n] = *reinterpret_cast<const float*>(xn + xoff + 64);
  }
}

// The 32 weights and the scale dword of row group q at P.
__device__ __forceinline__ void rg_wload(u32x4 (&w)[2], uint32_t& sc, const uint8_t* qs_tile,
                                         const uint8_t* d_tile, const RgPos& P, int q) {
  w[0] = __builtin_nontemporal_load(
      reinterpret_cast<const u32x4*>(qs_tile + P.qoff + 256 * q));
  w[1] = __builtin_nontemporal_load(
      reinterpret_cast<const u32x4*>(qs_tile + P.qoff + 1024 + 256 * q));
  sc = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(d_tile + P.doff + 128 * q));
}

// a[n] += d * sum_k w[k] x[n][k] for row group q of the lane row's block.
template <int N>
__device__ __forceinline__ void rg_fma(const u32x4 (&wq)[2], uint32_t sc, const XBlock<N>& X,
                                       const RgPos& P, float (&a)[N]) {
  const uint32_t w[8] = {wq[0].x, wq[0].y, wq[0].z, wq[0].w, wq[1].x, wq[1].y, wq[1].z, wq[1].w};
  float p[N];
#pragma unroll
  for (int n = 0; n < N; ++n) p[n] = 0.f;
  xv_steps<N>(w, X, p, std::make_integer_sequence<int, 32>{});
  const float d = P.ok ? f16_to_f32(sc >> P.sh) : 0.f;
#pragma unroll
  for (int n = 0; n < N; ++n) a[n] = fmaf(d, p[n], a[n]);
}

// Issue priority falls with progress through the unit (quads done of nq,
// four levels).  A SIMD issues from its oldest wave first, so without this
// the waves sharing it finish one after another and the last runs alone,
// unable to hide its loads; with it a wave that is ahead yields to the ones
// behind, and they finish together.
__device__ __forceinline__ void rg_progress_prio(int done, int nq) {
  const int level = (4 * done) / nq;
  if (level == 0)
    __builtin_amdgcn_s_setprio(3);
  else if (level == 1)
    __builtin_amdgcn_s_setprio(2);
  else if (level == 2)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
}

template <int N>
__device__ __forceinline__ void dot_range_rg(const uint8_t* qs_tile, const uint8_t* d_tile, int b0,
                                             int b1, int lane, const float* x, int64_t xs,
                                             bool prio, float (&acc)[N]) {
  const int r = lane >> 4, j = lane & 15;
  float a4[4][N];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int n = 0; n < N; ++n) a4[q][n] = 0.f;
  const int g0 = b0 >> 2;
  const int nq = b1 > b0 ? ((b1 + 3) >> 2) - g0 : 0;
  if (nq > 0) {
    u32x4 W[4][2];
    uint32_t SC[4];
    XBlock<N> XA, XB;
    RgPos PA = rg_pos(g0, r, j, b0, b1), PB;
    rg_xload<N>(x, xs, PA.xoff, XA);
#pragma unroll
    for (int q = 0; q < 4; ++q) rg_wload(W[q], SC[q], qs_tile, d_tile, PA, q);
    // An odd quad count starts with one quad alone; then two quads a trip in
    // two named buffers (no loop-carried copies).  The loads of the last
    // trip are for quads past the range: those have no block in [b0, b1),
    // so they re-read the last block and are never used.  No product is
    // conditional (a conditional one lets the compiler sink its weights'
    // load down to it), and the scheduling barriers keep each load where it
    // is issued (within one basic block the scheduler would otherwise move
    // the loads down to their uses to save registers).
    int it = 0;
    if (nq & 1) {
      if (prio) rg_progress_prio(0, nq);
      const RgPos P1 = rg_pos(g0 + 1, r, j, b0, b1);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        rg_fma<N>(W[q], SC[q], XA, PA, a4[q]);
        rg_wload(W[q], SC[q], qs_tile, d_tile, P1, q);
        __builtin_amdgcn_sched_barrier(0);
      }
      PA = P1;
      rg_xload<N>(x, xs, PA.xoff, XA);
      it = 1;
    }
    for (; it < nq; it += 2) {
      // (once a trip: a second call mid-trip split the loop's block and cost
      // 20-27 more VGPRs)
      if (prio) rg_progress_prio(it, nq);
      PB = rg_pos(g0 + it + 1, r, j, b0, b1);
      rg_xload<N>(x, xs, PB.xoff, XB);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        rg_fma<N>(W[q], SC[q], XA, PA, a4[q]);
        rg_wload(W[q], SC[q], qs_tile, d_tile, PB, q);
        __builtin_amdgcn_sched_barrier(0);
      }
      PA = rg_pos(g0 + it + 2, r, j, b0, b1);
      rg_xload<N>(x, xs, PA.xoff, XA);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        rg_fma<N>(W[q], SC[q], XB, PB, a4[q]);
        rg_wload(W[q], SC[q], qs_tile, d_tile, PA, q);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  __builtin_amdgcn_s_setprio(0);
#pragma unroll
  for (int n = 0; n < N; ++n) {
    float s0 = a4[0][n], s2 = a4[2][n], s1 = a4[1][n], s3 = a4[3][n];
    __asm__ volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(s0), "+v"(s2));
    __asm__ volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(s1), "+v"(s3));
    float u = s0 + s2, v = s1 + s3;
    __asm__ volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(u), "+v"(v));
    acc[n] += u + v;
  }
}

// ---- matrix cores: several columns as a skinny product ---------------------
// With N >= kRowGroupN columns the lane dot product above issues N FMAs per
// weight and is bound by VALU issue, not by HBM.  Here each block is one
// v_mfma_f32_16x16x32_bf16 per 16 rows, with the weights as the B operand:
// an int8 quant is exact in bf16.  The fp32 activations are cut into three
// bf16 parts, x = h + m + l with h = x truncated to bf16 and m, l the next
// eight significant bits each, so every product is exact and only the fp32
// accumulation order differs from the FMA loop.  The 16 A rows are [h of
// columns 0..7 | m of columns 0..7] in a first product and [0 | l] in a second
// chained onto it; column n's block sum is D[n] + D[n + 8].
//
// Operand layout of the 16x16x32 product (lane l, e = 0..7): A row l % 16 and
// B column l % 16 take k = 8 (l / 16) + e; D slot t of lane l is row
// 4 (l / 16) + t, column l % 16.  So lane (j = l % 16, g = l / 16) loads
// bytes 8 (g & 1) .. + 7 of half g >> 1 of row 16 q + j's block (two 256-byte
// runs per row group), and 8 activations of column l & 7 from k = 8 g.  D
// slot t of lane l then holds, for row 16 q + j, column 4 (g & 1) + t: the h
// part for g < 2, the m + l parts for g >= 2.  One quad of weights and
// activations is in flight with one quad's registers: the source reloads each
// block's registers with the next quad after its products, and the compiler
// moves those loads to the end of the quad, then waits block by block.  At
// the end, a permlane32 swap adds the two parts and a permlane16 swap moves
// row 16 q + j's columns 0..3 and 4..7 into lane 16 q + j: the layout
// dot_range produces.
//
// Each block's products run without scheduling barriers, so the compiler
// overlaps one block's conversions with the previous block's products.  C4
// gate_up 24576x4096 / down 4096x12288, same box, lane loop -> this: N = 8
// 38.0 -> 29.9 / 26.5 -> 22.4 us; N = 6 32.2 -> 28.5 / 23.0 -> 20.9; N = 5
// 31.1 -> 28.0 / 20.7 -> 21.6; N = 4 28.5 -> 27.7 / 18.3 -> 20.5 (kept on
// the lane loop: its registers leave 5 waves a SIMD against 4).  With the
// barriers that keep each load where it is issued (as the lane loop needs)
// N = 8 took 32.6 / 24.1 us: the loop then waited for the whole next quad at
// its top.  Two quad buffers (244 VGPRs, 2 waves a SIMD) took 35-45 us.
constexpr int kMfmaN = 5;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));

// High halves of (lo, hi) as two packed bf16 (lo in bits 0..15).
__device__ __forceinline__ uint32_t bf16_hi_pair(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// The 8 quants of a u32x2 as bf16 (exact).
__device__ __forceinline__ bf16x8 mf_weights(u32x2 w) {
  u32x4 r;
  r.x = bf16_hi_pair(q_at(w.x, 0), q_at(w.x, 1));
  r.y = bf16_hi_pair(q_at(w.x, 2), q_at(w.x, 3));
  r.z = bf16_hi_pair(q_at(w.y, 0), q_at(w.y, 1));
  r.w = bf16_hi_pair(q_at(w.y, 2), q_at(w.y, 3));
  return __builtin_bit_cast(bf16x8, r);
}

// A operands of one block from the lane's 8 activations: a1 = h (lanes of the
// first half row) or m (second half), a2 = 0 or l.  m1 = 0 / 0xffff0000 and
// m2 = 0 / ~0 select the half; m2 also zeroes columns >= N.
__device__ __forceinline__ void mf_split(const f32x4 (&xv)[2], uint32_t m1, uint32_t m1z,
                                         uint32_t m2, bf16x8& a1, bf16x8& a2) {
  float t[8], r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float v = xv[e >> 2][e & 3];
    t[e] = v - __uint_as_float(__float_as_uint(v) & m1);          // x, or x - h
    r[e] = t[e] - __uint_as_float(__float_as_uint(t[e]) & 0xffff0000u);  // below its bf16
  }
  u32x4 p1, p2;
  p1.x = bf16_hi_pair(t[0], t[1]) & m1z;
  p1.y = bf16_hi_pair(t[2], t[3]) & m1z;
  p1.z = bf16_hi_pair(t[4], t[5]) & m1z;
  p1.w = bf16_hi_pair(t[6], t[7]) & m1z;
  p2.x = bf16_hi_pair(r[0], r[1]) & m2;
  p2.y = bf16_hi_pair(r[2], r[3]) & m2;
  p2.z = bf16_hi_pair(r[4], r[5]) & m2;
  p2.w = bf16_hi_pair(r[6], r[7]) & m2;
  a1 = __builtin_bit_cast(bf16x8, p1);
  a2 = __builtin_bit_cast(bf16x8, p2);
}

template <int N>
__device__ __forceinline__ void dot_range_mf(const uint8_t* qs_tile, const uint8_t* d_tile, int b0,
                                             int b1, int lane, const float* x, int64_t xs,
                                             bool prio, float (&acc)[N]) {
  static_assert(N >= 1 && N <= 8, "one product holds 8 columns");
  const int j = lane & 15, g = lane >> 4, c = lane & 7;
  const bool second = (lane >> 3) & 1;
  const uint32_t m1 = second ? 0xffff0000u : 0u;
  const uint32_t m1z = c < N ? ~0u : 0u;
  const uint32_t m2 = second ? m1z : 0u;
  const float* xl = x + (int64_t)(c < N ? c : N - 1) * xs + 8 * g;
  const uint32_t wofs = (uint32_t)((g >> 1) * 1024 + j * 16 + (g & 1) * 8);
  const uint32_t dofs = (uint32_t)(j * 8);
  f32x4 a4[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) a4[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int g0 = b0 >> 2;
  const int nq = b1 > b0 ? ((b1 + 3) >> 2) - g0 : 0;
  if (nq > 0) {
    const int gl = (b1 - 1) >> 2;
    // block clamped into [b0, b1): loads past the range re-read the last
    // block (never used), so no load is conditional
    auto bcl = [&](int b) { return b < b0 ? b0 : (b < b1 ? b : b1 - 1); };
    auto wload = [&](int b, int q) {
      return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(
          qs_tile + (uint32_t)bcl(b) * 2048u + wofs + 256u * q));
    };
    auto xload = [&](int b, f32x4 (&v)[2]) {
      const float* p = xl + 32 * bcl(b);
      v[0] = *reinterpret_cast<const f32x4u*>(p);
      v[1] = *reinterpret_cast<const f32x4u*>(p + 4);
    };
    auto dload = [&](int G, int q) {
      return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(
          d_tile + (uint32_t)(G < gl ? G : gl) * 512u + dofs + 128u * q));
    };
    u32x2 W[4][4];  // [block of the quad][row group]
    f32x4 X[4][2];  // [block of the quad]
    u32x2 D[4], DN[4];
#pragma unroll
    for (int bq = 0; bq < 4; ++bq) {
      xload(4 * g0 + bq, X[bq]);
#pragma unroll
      for (int q = 0; q < 4; ++q) W[bq][q] = wload(4 * g0 + bq, q);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) DN[q] = dload(g0, q);
    for (int it = 0; it < nq; ++it) {
      const int G = g0 + it;
      if (prio) rg_progress_prio(it, nq);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        D[q] = DN[q];
        DN[q] = dload(G + 1, q);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int bq = 0; bq < 4; ++bq) {
        const int b = 4 * G + bq;
        const bool ok = b >= b0 && b < b1;
        bf16x8 a1, a2;
        mf_split(X[bq], m1, m1z, m2, a1, a2);
        xload(b + 4, X[bq]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bf16x8 wb = mf_weights(W[bq][q]);
          W[bq][q] = wload(b + 4, q);
          f32x4 s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, wb, f32x4{0.f, 0.f, 0.f, 0.f},
                                                            0, 0, 0);
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2, wb, s, 0, 0, 0);
          const float dq = ok ? f16_to_f32(quad_bits(D[q], bq)) : 0.f;
#pragma unroll
          for (int t = 0; t < 4; ++t) a4[q][t] = fmaf(dq, s[t], a4[q][t]);
        }
      }
    }
  }
  __builtin_amdgcn_s_setprio(0);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    float s0 = a4[0][t], s2 = a4[2][t], s1 = a4[1][t], s3 = a4[3][t];
    __asm__ volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(s0), "+v"(s2));
    __asm__ volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(s1), "+v"(s3));
    // u: row groups 0 (lanes 0..31) and 2, v: 1 and 3; lanes 16..31 of each
    // 32 hold columns 4..7
    float u = s0 + s2, v = s1 + s3;
    __asm__ volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(u), "+v"(v));
    if (t < N) acc[t] += u;
    if (4 + t < N) acc[4 + t] += v;
  }
}

// ---- Q4_K and Q5_K weights ---------------------------------------------------
// A quad is half of a 256-weight block: 4 sub-blocks of 32.  Sub-block j of
// a row is 16 bytes whose byte i holds weights i (low nibble) and i + 16 (high
// nibble), matching the activations' lanes (lanes 0..15 of a row hold x[i]
// and x[i + 16]), so weight i and i + 16 both read lane i through the row
// broadcast.  Per sub-block and column: y += d s * sum(q x) - dmin m * sum(x),
// the sum of the 32 activations taken by DPP rotations within the row.
// Q5_K adds a dword of fifth bits per sub-block and row, arranged so that the
// 4 fifth bits of each half of a nibble dword reach bit 4 of its bytes with
// one shift and one masked OR: bit 8b + I is that of weight 4I + b and bit
// 8b + 4 + I that of weight 16 + 4I + b.

template <int N, bool Q5>
struct QuadQ4 {
  u32x4 q[4];
  u32x4 meta;  // d, dmin (binary16), 12 bytes of 6-bit scales and mins
  u32x4 f;     // Q5_K: fifth bits of the 4 sub-blocks
  XBlock<N> x[4];
};

template <int N, bool Q5>
__device__ __forceinline__ void q4_load(QuadQ4<N, Q5>& B, const u32x4* qp, const u32x4* mp,
                                        const u32x4* fp, int g, const float* x, int64_t xs,
                                        int xl) {
  B.meta = __builtin_nontemporal_load(mp + (g >> 1) * 64);
  if constexpr (Q5) B.f = __builtin_nontemporal_load(fp + g * 64);
#pragma unroll
  for (int i = 0; i < 4; ++i) B.q[i] = __builtin_nontemporal_load(qp + (4 * g + i) * 64);
#pragma unroll
  for (int i = 0; i < 4; ++i) load_xblock<N>(x + 32 * (4 * g + i), xs, xl, B.x[i]);
}

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// Scale s and min m (6 bits each) of sub-block i of quad half h.
__device__ __forceinline__ void q4_scale_min(u32x4 meta, int h, int i, float& s, float& m) {
  if (h == 0) {
    s = (float)((meta.y >> (8 * i)) & 63u);
    m = (float)((meta.z >> (8 * i)) & 63u);
  } else {
    s = (float)(((meta.w >> (8 * i)) & 15u) | (((meta.y >> (8 * i + 6)) & 3u) << 4));
    m = (float)(((meta.w >> (8 * i + 4)) & 15u) | (((meta.z >> (8 * i + 6)) & 3u) << 4));
  }
}

// p[n] += the 8 codes held in the bytes of cl (weights 4I .. 4I + 3 of the
// sub-block) and ch (weights 16 + 4I ..) times their activations.  Byte b of a
// dword to fp32 is one v_cvt_f32_ubyteN.
template <int N, int I>
__device__ __forceinline__ void codes_fma(uint32_t cl, uint32_t ch, const XBlock<N>& X,
                                          float (&p)[N]) {
  const float l0 = (float)(cl & 255u), l1 = (float)((cl >> 8) & 255u);
  const float l2 = (float)((cl >> 16) & 255u), l3 = (float)(cl >> 24);
  const float h0 = (float)(ch & 255u), h1 = (float)((ch >> 8) & 255u);
  const float h2 = (float)((ch >> 16) & 255u), h3 = (float)(ch >> 24);
#pragma unroll
  for (int n = 0; n < N; ++n) {
    fmac_row_bcast<4 * I + 0>(p[n], X.a[n], l0);
    fmac_row_bcast<4 * I + 1>(p[n], X.a[n], l1);
    fmac_row_bcast<4 * I + 2>(p[n], X.a[n], l2);
    fmac_row_bcast<4 * I + 3>(p[n], X.a[n], l3);
    fmac_row_bcast<4 * I + 0>(p[n], X.b[n], h0);
    fmac_row_bcast<4 * I + 1>(p[n], X.b[n], h1);
    fmac_row_bcast<4 * I + 2>(p[n], X.b[n], h2);
    fmac_row_bcast<4 * I + 3>(p[n], X.b[n], h3);
  }
}

template <int N, bool Q5, int I>
__device__ __forceinline__ void q4_dword(uint32_t w, uint32_t f, const XBlock<N>& X,
                                         float (&p)[N]) {
  // The nibble masks are written as opaque VALU ops so the compiler keeps the
  // byte conversions instead of folding each mask into a per-weight bit-field
  // extract (two ops a weight).
  uint32_t lo, hi;
  asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(lo) : "v"(w));
  asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(hi) : "v"(w >> 4));
  if constexpr (Q5) {
    lo |= (f << (4 - I)) & 0x10101010u;
    hi |= (f >> I) & 0x10101010u;
    asm("" : "+v"(lo), "+v"(hi));
  }
  codes_fma<N, I>(lo, hi, X, p);
}

template <int N, bool Q5>
__device__ __forceinline__ void q4_fma(const QuadQ4<N, Q5>& B, int h, float (&acc)[N]) {
  const float d = f16_to_f32(B.meta.x & 0xffffu), dmin = f16_to_f32(B.meta.x >> 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float s, m;
    q4_scale_min(B.meta, h, i, s, m);
    float p[N];
#pragma unroll
    for (int n = 0; n < N; ++n) p[n] = 0.f;
    const uint32_t f = Q5 ? B.f[i] : 0u;
    q4_dword<N, Q5, 0>(B.q[i].x, f, B.x[i], p);
    q4_dword<N, Q5, 1>(B.q[i].y, f, B.x[i], p);
    q4_dword<N, Q5, 2>(B.q[i].z, f, B.x[i], p);
    q4_dword<N, Q5, 3>(B.q[i].w, f, B.x[i], p);
    const float ds = d * s, dm = dmin * m;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      // sum of the sub-block's 32 activations: every lane of a 16-lane row
      // holds two of them; rotations add the row
      float sx = B.x[i].a[n] + B.x[i].b[n];
      sx = dpp_add<0x128>(sx);  // row_ror:8
      sx = dpp_add<0x124>(sx);  // row_ror:4
      sx = dpp_add<0x122>(sx);  // row_ror:2
      sx = dpp_add<0x121>(sx);  // row_ror:1
      acc[n] = fmaf(ds, p[n], acc[n]);
      acc[n] = fmaf(-dm, sx, acc[n]);
    }
  }
}

// Q4_K (Q5 false) or Q5_K dot products of the 64 rows of one tile over
// 32-weight blocks [b0, b1) (multiples of 4: whole quads), quads
// double-buffered.  f_tile: Q5_K fifth bits (16 bytes per quad and row).
template <int N, bool Q5>
__device__ __forceinline__ void dot_range_q4k(const uint8_t* qs_tile, const uint8_t* meta_tile,
                                              const uint8_t* f_tile, int b0, int b1, int lane,
                                              const float* x, int64_t xs, float (&acc)[N]) {
  const u32x4* qp = reinterpret_cast<const u32x4*>(qs_tile) + lane;
  const u32x4* mp = reinterpret_cast<const u32x4*>(meta_tile) + lane;
  const u32x4* fp = reinterpret_cast<const u32x4*>(f_tile) + lane;
  const int xl = lane & 15;
  const int g0 = b0 >> 2, nq = (b1 - b0) >> 2;
  if (nq <= 0) return;
  QuadQ4<N, Q5> A, B;
  q4_load<N, Q5>(A, qp, mp, fp, g0, x, xs, xl);
  int it = 0;
  for (; it + 1 < nq; it += 2) {
    q4_load<N, Q5>(B, qp, mp, fp, g0 + it + 1, x, xs, xl);
    q4_fma<N, Q5>(A, (g0 + it) & 1, acc);
    if (it + 2 < nq) q4_load<N, Q5>(A, qp, mp, fp, g0 + it + 2, x, xs, xl);
    q4_fma<N, Q5>(B, (g0 + it + 1) & 1, acc);
  }
  if (it < nq) q4_fma<N, Q5>(A, (g0 + it) & 1, acc);
}

// ---- Q6_K weights ------------------------------------------------------------
// A quad is half of a 256-weight block: 4 sub-blocks of 32.  Per sub-block
// and row: 16 bytes of low nibbles laid out as for Q4_K, 8 bytes of dense
// 2-bit high fields, and per quad 8 signed scales (one per 16 weights) and d.
// The 6-bit code of a weight is low + 16 high; per 16-weight group and
// column y += d s * (sum(code x) - 32 sum(x)).

template <int N>
struct QuadQ6 {
  u32x4 q[4];
  u32x2 h[4];
  u32x4 meta;  // 8 int8 scales, then d (binary16)
  XBlock<N> x[4];
};

template <int N>
__device__ __forceinline__ void q6_load(QuadQ6<N>& B, const u32x4* qp, const u32x2* hp,
                                        const u32x4* mp, int g, const float* x, int64_t xs,
                                        int xl) {
  B.meta = __builtin_nontemporal_load(mp + g * 64);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    B.q[i] = __builtin_nontemporal_load(qp + (4 * g + i) * 64);
    B.h[i] = __builtin_nontemporal_load(hp + (4 * g + i) * 64);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) load_xblock<N>(x + 32 * (4 * g + i), xs, xl, B.x[i]);
}

// Four 2-bit fields (bits 0-7 of b) to bits 0-1 of the four bytes.
__device__ __forceinline__ uint32_t spread2(uint32_t b) {
  uint32_t v = (b | (b << 12)) & 0x000F000Fu;
  return (v | (v << 6)) & 0x03030303u;
}

// 6-bit codes of 4 weights as the 4 bytes of a dword: nibbles (4 bits each,
// one per byte) plus 16 times the matching high fields.  The result is kept
// opaque so that each byte converts with one v_cvt_f32_ubyteN.
__device__ __forceinline__ uint32_t q6_codes(uint32_t nib, uint32_t hb) {
  uint32_t c = nib | (spread2(hb) << 4);
  asm("" : "+v"(c));
  return c;
}

template <int N, int I>
__device__ __forceinline__ void q6_dword(uint32_t w, uint32_t h0, uint32_t h1, const XBlock<N>& X,
                                         float (&pl)[N], float (&ph)[N]) {
  uint32_t lo, hi;
  asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(lo) : "v"(w));
  asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(hi) : "v"(w >> 4));
  const uint32_t cl = q6_codes(lo, (h0 >> (8 * I)) & 255u);
  const uint32_t ch = q6_codes(hi, (h1 >> (8 * I)) & 255u);
  const float l0 = (float)(cl & 255u), l1 = (float)((cl >> 8) & 255u);
  const float l2 = (float)((cl >> 16) & 255u), l3 = (float)(cl >> 24);
  const float g0 = (float)(ch & 255u), g1 = (float)((ch >> 8) & 255u);
  const float g2 = (float)((ch >> 16) & 255u), g3 = (float)(ch >> 24);
#pragma unroll
  for (int n = 0; n < N; ++n) {
    fmac_row_bcast<4 * I + 0>(pl[n], X.a[n], l0);
    fmac_row_bcast<4 * I + 1>(pl[n], X.a[n], l1);
    fmac_row_bcast<4 * I + 2>(pl[n], X.a[n], l2);
    fmac_row_bcast<4 * I + 3>(pl[n], X.a[n], l3);
    fmac_row_bcast<4 * I + 0>(ph[n], X.b[n], g0);
    fmac_row_bcast<4 * I + 1>(ph[n], X.b[n], g1);
    fmac_row_bcast<4 * I + 2>(ph[n], X.b[n], g2);
    fmac_row_bcast<4 * I + 3>(ph[n], X.b[n], g3);
  }
}

template <int N>
__device__ __forceinline__ void q6_fma(const QuadQ6<N>& B, float (&acc)[N]) {
  const float d = f16_to_f32(B.meta.z & 0xffffu);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t sw = i < 2 ? B.meta.x : B.meta.y;
    const float sl = d * (float)(int8_t)(sw >> (16 * (i & 1)));
    const float sh = d * (float)(int8_t)(sw >> (16 * (i & 1) + 8));
    float pl[N], ph[N];
#pragma unroll
    for (int n = 0; n < N; ++n) pl[n] = ph[n] = 0.f;
    q6_dword<N, 0>(B.q[i].x, B.h[i].x, B.h[i].y, B.x[i], pl, ph);
    q6_dword<N, 1>(B.q[i].y, B.h[i].x, B.h[i].y, B.x[i], pl, ph);
    q6_dword<N, 2>(B.q[i].z, B.h[i].x, B.h[i].y, B.x[i], pl, ph);
    q6_dword<N, 3>(B.q[i].w, B.h[i].x, B.h[i].y, B.x[i], pl, ph);
#pragma unroll
    for (int n = 0; n < N; ++n) {
      // sums of the 16 activations of each group, by rotations within the row
      float sa = B.x[i].a[n], sb = B.x[i].b[n];
      sa = dpp_add<0x128>(sa);
      sb = dpp_add<0x128>(sb);
      sa = dpp_add<0x124>(sa);
      sb = dpp_add<0x124>(sb);
      sa = dpp_add<0x122>(sa);
      sb = dpp_add<0x122>(sb);
      sa = dpp_add<0x121>(sa);
      sb = dpp_add<0x121>(sb);
      acc[n] = fmaf(sl, pl[n], acc[n]);
      acc[n] = fmaf(-32.0f * sl, sa, acc[n]);
      acc[n] = fmaf(sh, ph[n], acc[n]);
      acc[n] = fmaf(-32.0f * sh, sb, acc[n]);
    }
  }
}

// Q6_K dot products of the 64 rows of one tile over 32-weight blocks
// [b0, b1) (whole quads), quads double-buffered.
template <int N>
__device__ __forceinline__ void dot_range_q6k(const uint8_t* qs_tile, const uint8_t* qh_tile,
                                              const uint8_t* meta_tile, int b0, int b1,
                                              int lane, const float* x, int64_t xs,
                                              float (&acc)[N]) {
  const u32x4* qp = reinterpret_cast<const u32x4*>(qs_tile) + lane;
  const u32x2* hp = reinterpret_cast<const u32x2*>(qh_tile) + lane;
  const u32x4* mp = reinterpret_cast<const u32x4*>(meta_tile) + lane;
  const int xl = lane & 15;
  const int g0 = b0 >> 2, nq = (b1 - b0) >> 2;
  if (nq <= 0) return;
  QuadQ6<N> A, B;
  q6_load<N>(A, qp, hp, mp, g0, x, xs, xl);
  int it = 0;
  for (; it + 1 < nq; it += 2) {
    q6_load<N>(B, qp, hp, mp, g0 + it + 1, x, xs, xl);
    q6_fma<N>(A, acc);
    if (it + 2 < nq) q6_load<N>(A, qp, hp, mp, g0 + it + 2, x, xs, xl);
    q6_fma<N>(B, acc);
  }
  if (it < nq) q6_fma<N>(A, acc);
}

// Several columns (N > 4): a ring of single sub-block buffers, so that the
// activations of only RING sub-blocks are live and all N columns fit one
// launch (the weights are read once; N = 8, Q4_K 24576x4096: two launches of
// 4 columns 61.6 us, one launch with a ring of 2 48.1 us).
template <int N>
struct SubQ4 {
  u32x4 q;
  u32x4 meta;
  uint32_t f;
  XBlock<N> x;
};

template <int N, bool Q5>
__device__ __forceinline__ void sub_load_q4(SubQ4<N>& B, const u32x4* qp, const u32x4* mp,
                                            const uint32_t* fp, int sb, const float* x,
                                            int64_t xs, int xl) {
  B.q = __builtin_nontemporal_load(qp + sb * 64);
  B.meta = __builtin_nontemporal_load(mp + (sb >> 3) * 64);
  if constexpr (Q5) B.f = __builtin_nontemporal_load(fp + (sb >> 2) * 256 + (sb & 3));
  load_xblock<N>(x + 32 * sb, xs, xl, B.x);
}

template <int N, bool Q5>
__device__ __forceinline__ void sub_fma_q4(const SubQ4<N>& B, int sb, float (&acc)[N]) {
  const float d = f16_to_f32(B.meta.x & 0xffffu), dmin = f16_to_f32(B.meta.x >> 16);
  float s, m;
  q4_scale_min(B.meta, (sb >> 2) & 1, sb & 3, s, m);
  float p[N];
#pragma unroll
  for (int n = 0; n < N; ++n) p[n] = 0.f;
  const uint32_t f = Q5 ? B.f : 0u;
  q4_dword<N, Q5, 0>(B.q.x, f, B.x, p);
  q4_dword<N, Q5, 1>(B.q.y, f, B.x, p);
  q4_dword<N, Q5, 2>(B.q.z, f, B.x, p);
  q4_dword<N, Q5, 3>(B.q.w, f, B.x, p);
  const float ds = d * s, dm = dmin * m;
#pragma unroll
  for (int n = 0; n < N; ++n) {
    float sx = B.x.a[n] + B.x.b[n];
    sx = dpp_add<0x128>(sx);
    sx = dpp_add<0x124>(sx);
    sx = dpp_add<0x122>(sx);
    sx = dpp_add<0x121>(sx);
    acc[n] = fmaf(ds, p[n], acc[n]);
    acc[n] = fmaf(-dm, sx, acc[n]);
  }
}

template <int N, bool Q5, int RING>
__device__ __forceinline__ void dot_range_q4k_ring(const uint8_t* qs_tile, const uint8_t* meta_tile,
                                                   const uint8_t* f_tile, int b0, int b1, int lane,
                                                   const float* x, int64_t xs, float (&acc)[N]) {
  const u32x4* qp = reinterpret_cast<const u32x4*>(qs_tile) + lane;
  const u32x4* mp = reinterpret_cast<const u32x4*>(meta_tile) + lane;
  const uint32_t* fp = reinterpret_cast<const uint32_t*>(f_tile) + 4 * lane;
  const int xl = lane & 15;
  SubQ4<N> S[RING];
#pragma unroll
  for (int r = 0; r < RING; ++r)
    if (b0 + r < b1) sub_load_q4<N, Q5>(S[r], qp, mp, fp, b0 + r, x, xs, xl);
  for (int b = b0; b < b1; b += RING) {
#pragma unroll
    for (int r = 0; r < RING; ++r) {
      if (b + r < b1) {
        sub_fma_q4<N, Q5>(S[r], b + r, acc);
        if (b + r + RING < b1) sub_load_q4<N, Q5>(S[r], qp, mp, fp, b + r + RING, x, xs, xl);
      }
    }
  }
}

template <int N>
struct SubQ6 {
  u32x4 q;
  u32x2 h;
  u32x4 meta;
  XBlock<N> x;
};

template <int N>
__device__ __forceinline__ void sub_load_q6(SubQ6<N>& B, const u32x4* qp, const u32x2* hp,
                                            const u32x4* mp, int sb, const float* x, int64_t xs,
                                            int xl) {
  B.q = __builtin_nontemporal_load(qp + sb * 64);
  B.h = __builtin_nontemporal_load(hp + sb * 64);
  B.meta = __builtin_nontemporal_load(mp + (sb >> 2) * 64);
  load_xblock<N>(x + 32 * sb, xs, xl, B.x);
}

template <int N>
__device__ __forceinline__ void sub_fma_q6(const SubQ6<N>& B, int sb, float (&acc)[N]) {
  const float d = f16_to_f32(B.meta.z & 0xffffu);
  const int i = sb & 3;
  const uint32_t sw = i < 2 ? B.meta.x : B.meta.y;
  const float sl = d * (float)(int8_t)(sw >> (16 * (i & 1)));
  const float sh = d * (float)(int8_t)(sw >> (16 * (i & 1) + 8));
  float pl[N], ph[N];
#pragma unroll
  for (int n = 0; n < N; ++n) pl[n] = ph[n] = 0.f;
  q6_dword<N, 0>(B.q.x, B.h.x, B.h.y, B.x, pl, ph);
  q6_dword<N, 1>(B.q.y, B.h.x, B.h.y, B.x, pl, ph);
  q6_dword<N, 2>(B.q.z, B.h.x, B.h.y, B.x, pl, ph);
  q6_dword<N, 3>(B.q.w, B.h.x, B.h.y, B.x, pl, ph);
#pragma unroll
  for (int n = 0; n < N; ++n) {
    float sa = B.x.a[n], sbx = B.x.b[n];
    sa = dpp_add<0x128>(sa);
    sbx = dpp_add<0x128>(sbx);
    sa = dpp_add<0x124>(sa);
    sbx = dpp_add<0x124>(sbx);
    sa = dpp_add<0x122>(sa);
    sbx = dpp_add<0x122>(sbx);
    sa = dpp_add<0x121>(sa);
    sbx = dpp_add<0x121>(sbx);
    acc[n] = fmaf(sl, pl[n], acc[n]);
    acc[n] = fmaf(-32.0f * sl, sa, acc[n]);
    acc[n] = fmaf(sh, ph[n], acc[n]);
    acc[n] = fmaf(-32.0f * sh, sbx, acc[n]);
  }
}

template <int N, int RING>
__device__ __forceinline__ void dot_range_q6k_ring(const uint8_t* qs_tile, const uint8_t* qh_tile,
                                                   const uint8_t* meta_tile, int b0, int b1,
                                                   int lane, const float* x, int64_t xs,
                                                   float (&acc)[N]) {
  const u32x4* qp = reinterpret_cast<const u32x4*>(qs_tile) + lane;
  const u32x2* hp = reinterpret_cast<const u32x2*>(qh_tile) + lane;
  const u32x4* mp = reinterpret_cast<const u32x4*>(meta_tile) + lane;
  const int xl = lane & 15;
  SubQ6<N> S[RING];
#pragma unroll
  for (int r = 0; r < RING; ++r)
    if (b0 + r < b1) sub_load_q6<N>(S[r], qp, hp, mp, b0 + r, x, xs, xl);
  for (int b = b0; b < b1; b += RING) {
#pragma unroll
    for (int r = 0; r < RING; ++r) {
      if (b + r < b1) {
        sub_fma_q6<N>(S[r], b + r, acc);
        if (b + r + RING < b1) sub_load_q6<N>(S[r], qp, hp, mp, b + r + RING, x, xs, xl);
      }
    }
  }
}

// ---- integer activations (opt-in variant) ------------------------------------
// Activations quantized per 32-entry block to int8 with a binary16 scale
// (q8_0_quantize_act).  Per block and column the 32 int8 x int8 products are
// accumulated exactly in int32 with v_dot4c_i32_i8, whose first operand is
// read through the DPP row broadcast like the fp32 path: lanes 0..15 of every
// 16-lane row hold 64 consecutive codes (two blocks) of a column, one dword
// each, and the dot of dword i of a block reads lane 8 (block & 1) + i.
// Then acc += float(isum) * (dw * dx).  (The DPP source registers are only
// written by loads.)  A dot instruction's result must not be read by another
// VALU instruction within three wait states; chained dots reading it as
// their accumulator need none.  The compiler does not see through the asm,
// so the last dot of a chain carries its own s_nop 2.

template <int I, bool LAST>
__device__ __forceinline__ int dot4_row_bcast(int acc, int xv, uint32_t w) {
  if (LAST)
    asm("v_dot4c_i32_i8_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf\n\ts_nop 2"
        : "+v"(acc)
        : "v"(xv), "v"(w), "i"(I));
  else
    asm("v_dot4c_i32_i8_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
        : "+v"(acc)
        : "v"(xv), "v"(w), "i"(I));
  return acc;
}

// int32 sum of the 32 products of one block: weights q0|q1 (this lane's row),
// codes in lanes 8 * half + 0..7 of xv's 16-lane row.
template <int HALF>
__device__ __forceinline__ int block_isum(u32x4 q0, u32x4 q1, int xv) {
  int s = 0;
  s = dot4_row_bcast<8 * HALF + 0, false>(s, xv, q0.x);
  s = dot4_row_bcast<8 * HALF + 1, false>(s, xv, q0.y);
  s = dot4_row_bcast<8 * HALF + 2, false>(s, xv, q0.z);
  s = dot4_row_bcast<8 * HALF + 3, false>(s, xv, q0.w);
  s = dot4_row_bcast<8 * HALF + 4, false>(s, xv, q1.x);
  s = dot4_row_bcast<8 * HALF + 5, false>(s, xv, q1.y);
  s = dot4_row_bcast<8 * HALF + 6, false>(s, xv, q1.z);
  s = dot4_row_bcast<8 * HALF + 7, true>(s, xv, q1.w);
  return s;
}

// One quad of one tile for the integer path: weights, scales, the codes of
// the quad (two dwords per column and lane) and the 4 activation scales.
template <int N>
struct QuadI {
  u32x4 q[8];
  u32x2 sc;
  int xa[N], xb[N];    // codes of blocks 0-1 / 2-3 of the quad
  uint32_t dxb[N][4];  // binary16 activation scales of the quad's blocks
};

template <int N>
__device__ __forceinline__ void quadi_load(QuadI<N>& B, const u32x4* qp, const u32x2* dp, int g,
                                           const int8_t* qx, const uint16_t* dx, int64_t K,
                                           int nblk, int lane) {
  B.sc = __builtin_nontemporal_load(dp + g * 64);
#pragma unroll
  for (int i = 0; i < 8; ++i) B.q[i] = __builtin_nontemporal_load(qp + (8 * g + i) * 64);
  const int xl = lane & 15;
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const int* xq = reinterpret_cast<const int*>(qx + n * K + 128 * g);
    B.xa[n] = xq[xl];
    B.xb[n] = xq[16 + xl];
#pragma unroll
    for (int j = 0; j < 4; ++j) B.dxb[n][j] = dx[n * nblk + 4 * g + j];
  }
}

template <int N>
__device__ __forceinline__ void quadi_fma(const QuadI<N>& B, float (&acc)[N]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float dw = f16_to_f32(quad_bits(B.sc, j));
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const int xv = j < 2 ? B.xa[n] : B.xb[n];
      const int isum = (j & 1) ? block_isum<1>(B.q[2 * j], B.q[2 * j + 1], xv)
                               : block_isum<0>(B.q[2 * j], B.q[2 * j + 1], xv);
      acc[n] = fmaf((float)isum, dw * f16_to_f32(B.dxb[n][j]), acc[n]);
    }
  }
}

// Integer-activation dot products of the 64 rows of one tile over blocks
// [b0, b1): whole quads double-buffered, then the blocks of a short last quad.
template <int N>
__device__ __forceinline__ void dot_range_i8(const uint8_t* qs_tile, const uint8_t* d_tile, int b0,
                                             int b1, int lane, const int8_t* qx,
                                             const uint16_t* dx, int64_t K, int nblk,
                                             float (&acc)[N]) {
  const u32x4* qp = reinterpret_cast<const u32x4*>(qs_tile) + lane;
  const u32x2* dp = reinterpret_cast<const u32x2*>(d_tile) + lane;
  const int nq = (b1 - b0) >> 2;
  int b = b0;
  if (nq > 0) {
    const int g0 = b0 >> 2;
    QuadI<N> A, B;
    quadi_load<N>(A, qp, dp, g0, qx, dx, K, nblk, lane);
    int it = 0;
    for (; it + 1 < nq; it += 2) {
      quadi_load<N>(B, qp, dp, g0 + it + 1, qx, dx, K, nblk, lane);
      quadi_fma<N>(A, acc);
      if (it + 2 < nq) quadi_load<N>(A, qp, dp, g0 + it + 2, qx, dx, K, nblk, lane);
      quadi_fma<N>(B, acc);
    }
    if (it < nq) quadi_fma<N>(A, acc);
    b += 4 * nq;
  }
  // blocks of a row's short last quad: lanes 0..7 of each 16-lane row read
  // the block's 8 code dwords
  for (; b < b1; ++b) {
    const u32x2 sc = __builtin_nontemporal_load(dp + (b >> 2) * 64);
    const u32x4 q0 = __builtin_nontemporal_load(qp + (2 * b) * 64);
    const u32x4 q1 = __builtin_nontemporal_load(qp + (2 * b + 1) * 64);
    const float dw = f16_to_f32(quad_bits(sc, b & 3));
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const int xv = reinterpret_cast<const int*>(qx + n * K + 32 * b)[lane & 7];
      const int isum = block_isum<0>(q0, q1, xv);
      acc[n] = fmaf((float)isum, dw * f16_to_f32(dx[n * nblk + b]), acc[n]);
    }
  }
}

// Quantize fp32 activations [N][K] to int8 codes and binary16 block scales:
// d = amax / 127, q = x / d rounded to nearest even (fp32 IEEE divisions),
// zeros for an all-zero block.  32 lanes per block.
__global__ __launch_bounds__(256) void quantize_act_kernel(const float* __restrict__ x, int64_t K,
                                                           int64_t nblocks, int8_t* __restrict__ qx,
                                                           uint16_t* __restrict__ dx) {
  const int64_t blk = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  if (blk >= nblocks) return;
  const int j = threadIdx.x & 31;
  const int64_t i = blk * 32 + j;  // K % 32 == 0: blocks never cross columns
  const float v = x[i];
  float amax = fabsf(v);
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 32));
  const float d = __fdiv_rn(amax, 127.0f);
  const float q = amax > 0.0f ? __builtin_rintf(__fdiv_rn(v, d)) : 0.0f;
  qx[i] = (int8_t)(int)q;
  if (j == 0) dx[blk] = __builtin_bit_cast(uint16_t, (_Float16)d);
}

// Butterfly all-reduce over the wave; every lane ends with the same bits.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// (value, index) maximum with ties to the lower index; all lanes agree.
// VALU data movement only: DPP rotations within each 16-lane row, then
// v_permlane16/32_swap across rows (inline asm: the swap builtins are not
// used because both of their results are needed; the nop covers the
// VALU-write to permlane-read hazard).  The combination is symmetric, so the
// result does not depend on the order in which lanes are combined.
__device__ __forceinline__ void argmax_comb(float& v, int& i, float ov, int oi) {
  if (ov > v || (ov == v && oi < i)) {
    v = ov;
    i = oi;
  }
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ void argmax_ror(float& v, int& i) {
  const float ov = __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
  const int oi = dpp_i<CTRL>(i);
  argmax_comb(v, i, ov, oi);
}
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  argmax_ror<0x121>(v, i);  // row_ror:1
  argmax_ror<0x122>(v, i);  // row_ror:2
  argmax_ror<0x124>(v, i);  // row_ror:4
  argmax_ror<0x128>(v, i);  // row_ror:8
  int a = __builtin_bit_cast(int, v), b = a, ia = i, ib = i;
  __asm__ volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\tv_permlane16_swap_b32 %2, %3"
                   : "+v"(a), "+v"(b), "+v"(ia), "+v"(ib));
  v = __builtin_bit_cast(float, a);
  i = ia;
  argmax_comb(v, i, __builtin_bit_cast(float, b), ib);
  a = __builtin_bit_cast(int, v);
  b = a;
  ia = i;
  ib = i;
  __asm__ volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\tv_permlane32_swap_b32 %2, %3"
                   : "+v"(a), "+v"(b), "+v"(ia), "+v"(ib));
  v = __builtin_bit_cast(float, a);
  i = ia;
  argmax_comb(v, i, __builtin_bit_cast(float, b), ib);
}

__device__ __forceinline__ float seg_alpha(const Seg& s) {
  if (s.alpha_mode == A_PTR) return *s.alpha_ptr;
  if (s.alpha_mode == A_SIGMOID) return 1.0f / (1.0f + expf(-*s.alpha_ptr));
  return 1.0f;
}

// val[ts][n] = sum over segments (in order) of alpha_seg * (sum of the
// segment's unit partials), for each tile of a pair.  The unit partials are
// added in a fixed three-level order: batches of 8 consecutive units, groups
// of 8 batches, then the groups in order, so the fold adds at most
// 8 + 8 + ceil(units / 64) roundings to an output's chain (bitwise the same
// on every call).  Each batch's 8 partials are fetched before any is added,
// so their global loads are in flight together.
template <int N, typename Get>
__device__ __forceinline__ void fold_units(const GemvParams& p, const Prob& pr, int us, Get get,
                                           float (&val)[2][N]) {
#pragma unroll
  for (int ts = 0; ts < 2; ++ts) {
    if (ts >= pr.R) break;
#pragma unroll
    for (int n = 0; n < N; ++n) val[ts][n] = 0.f;
    int uu = ts * us;
    for (int si = pr.seg0; si < pr.seg0 + pr.nseg; ++si) {
      const Seg& s = p.seg[si];
      float ssum[N];
#pragma unroll
      for (int n = 0; n < N; ++n) ssum[n] = 0.f;
      for (int g0 = 0; g0 < s.units; g0 += 64) {
        float gsum[N];
#pragma unroll
        for (int n = 0; n < N; ++n) gsum[n] = 0.f;
        const int gend = s.units - g0 < 64 ? s.units : g0 + 64;
        for (int i0 = g0; i0 < gend; i0 += 8) {
          const int cnt = gend - i0 < 8 ? gend - i0 : 8;
          float buf[8][N];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if (j < cnt) {
#pragma unroll
              for (int n = 0; n < N; ++n) buf[j][n] = get(uu + j, n);
            }
          }
          float bsum[N];
#pragma unroll
          for (int n = 0; n < N; ++n) bsum[n] = buf[0][n];
#pragma unroll
          for (int j = 1; j < 8; ++j) {
            if (j < cnt) {
#pragma unroll
              for (int n = 0; n < N; ++n) bsum[n] += buf[j][n];
            }
          }
#pragma unroll
          for (int n = 0; n < N; ++n) gsum[n] += bsum[n];
          uu += cnt;
        }
#pragma unroll
        for (int n = 0; n < N; ++n) ssum[n] += gsum[n];
      }
      if (s.alpha_mode == A_ONE) {
#pragma unroll
        for (int n = 0; n < N; ++n) val[ts][n] += ssum[n];
      } else {
        const float a = seg_alpha(s);
#pragma unroll
        for (int n = 0; n < N; ++n) val[ts][n] = fmaf(a, ssum[n], val[ts][n]);
      }
    }
  }
}

// ONE: a single problem with a single segment (dense GEMVs and the decode
// chain): every kernel argument sits at a fixed offset, so no search loops.
// MODE: 0 Q8_0 weights and fp32 activations; 1 integer activations; 2 Q4_K,
// 3 Q6_K and 4 Q5_K weights with fp32 activations.
template <int N, bool ONE, int MODE>
__global__ __launch_bounds__(64 * max_waves_for(N, MODE >= 3)) void gemv_kernel(const GemvParams p) {
  extern __shared__ float lds_part[];  // [W][N][64]
  __shared__ int s_last;

  const int g = blockIdx.x;
  int pi = 0;
  if (!ONE) {
    while (pi + 1 < p.nprob && g >= p.prob[pi + 1].wg0) ++pi;
  }
  const Prob& pr = p.prob[pi];

  const int W = p.W;
  const int lg = g - pr.wg0;
  const int ot = lg / pr.P;
  const int pp = lg - ot * pr.P;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int u = pp * W + wave;
  const int us = pr.U / pr.R;  // units per tile of a pair

  // RMS prologue: wave 0 (the folding wave) issues its loads of the vector
  // first and reduces them after the dot products.
  float rx[16];
  const bool want_rms = (pr.flags & F_RMSNORM) && wave == 0 && pr.rms_K <= 1024;
  if (want_rms) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int k = lane + 64 * i;
      rx[i] = k < pr.rms_K ? pr.rms_x[k] : 0.f;
    }
  }

  // fused router: workgroup 0 also publishes every slot's id and weight for
  // the launch that combines the slots
  if (!ONE && p.route.logits && g == 0 && wave == 0) {
    float sel_v[Q8_MAX_SLOTS];
    int sel_i[Q8_MAX_SLOTS];
    route_topk_wave(p.route.logits, p.route.E, p.route.k, lane, sel_v, sel_i);
    if (lane == 0) route_store(sel_v, sel_i, p.route.k, p.route.ids_out, p.route.w_out);
  }

  float acc[N];
#pragma unroll
  for (int n = 0; n < N; ++n) acc[n] = 0.f;
  if (u < pr.U) {
    const int tsel = u / us;
    int v = u - tsel * us;
    int si = ONE ? 0 : pr.seg0;
    if (!ONE) {
      while (v >= p.seg[si].units) {
        v -= p.seg[si].units;
        ++si;
      }
    }
    const Seg& s = p.seg[si];
    int e = 0;
    bool ok = true;
    if (s.eid) {
      // the slot's expert: picked here from the router logits when the router
      // is fused into this launch, else read from the id array
      e = __builtin_amdgcn_readfirstlane(
          p.route.logits ? route_pick_wave(p.route.logits, p.route.E, s.slot, lane)
                         : s.eid[s.slot]);
      ok = e >= 0 && e < s.n_mats;
    }
    if (ok) {
      const int t = ot + tsel * pr.Tout;
      // bytes of one packed tile's quants: 64 rows of K (Q8_0) or K / 2 (Q4_K)
      const uint8_t* qs_tile =
          s.qs + (int64_t)e * s.qs_stride + (int64_t)t * kTile * (MODE >= 2 ? s.K / 2 : s.K);
      const uint8_t* d_tile = s.d + (int64_t)e * s.d_stride + (int64_t)t * s.G * 512;
      // units own whole scale quads (4 blocks); only a row's last may be short
      const int b0 = 4 * (int)((int64_t)v * s.G / s.units);
      const int b1e = 4 * (int)((int64_t)(v + 1) * s.G / s.units);
      const int b1 = b1e < s.nblk ? b1e : s.nblk;
      if (MODE == 1)
        dot_range_i8<N>(qs_tile, d_tile, b0, b1, lane, s.qx, s.dx, s.K, s.nblk, acc);
      else if (MODE == 2) {
        if constexpr (N > 4)
          dot_range_q4k_ring<N, false, 2>(qs_tile, d_tile, nullptr, b0, b1, lane, s.x,
                                              s.x_stride, acc);
        else
          dot_range_q4k<N, false>(qs_tile, d_tile, nullptr, b0, b1, lane, s.x, s.x_stride, acc);
      } else if (MODE == 4) {
        // Q5_K: 4 bytes of fifth bits per sub-block and row
        if constexpr (N > 4)
          dot_range_q4k_ring<N, true, 2>(qs_tile, d_tile,
                                             s.qh + (int64_t)t * kTile * (s.K / 8), b0, b1, lane,
                                             s.x, s.x_stride, acc);
        else
          dot_range_q4k<N, true>(qs_tile, d_tile, s.qh + (int64_t)t * kTile * (s.K / 8), b0, b1,
                                 lane, s.x, s.x_stride, acc);
      } else if (MODE == 3) {
        // Q6_K: 8 bytes of high fields per sub-block and row, 16 bytes of
        // scales and d per quad and row
        if constexpr (N > 4)
          dot_range_q6k_ring<N, 2>(qs_tile, s.qh + (int64_t)t * kTile * (s.K / 4),
                                       s.d + (int64_t)t * s.G * 1024, b0, b1, lane, s.x,
                                       s.x_stride, acc);
        else
          dot_range_q6k<N>(qs_tile, s.qh + (int64_t)t * kTile * (s.K / 4),
                           s.d + (int64_t)t * s.G * 1024, b0, b1, lane, s.x, s.x_stride, acc);
      }
      else
      {
        // (the GQA prologue exists for one column only, which the launcher
        // enforces; the row-group instances carry no replicated path, whose
        // registers would set the whole kernel's occupancy)
        // N >= kMfmaN: matrix-core products.  N = 4: row groups always.
        // N = 2, 3: row groups when every wave is
        // resident (C4 down 4096x12288 N = 2: 16.7 -> 15.2 us), the
        // replicated loop in launches of several rounds with short units
        // (lm_head N = 2: 31.5 us replicated, 33.9 with row groups).
        if constexpr (N >= kMfmaN)
          dot_range_mf<N>(qs_tile, d_tile, b0, b1, lane, s.x, s.x_stride, p.prio != 0, acc);
        else if constexpr (N >= kRowGroupN)
          dot_range_rg<N>(qs_tile, d_tile, b0, b1, lane, s.x, s.x_stride, p.prio != 0, acc);
        else if constexpr (N >= 2) {
          if (p.prio)
            dot_range_rg<N>(qs_tile, d_tile, b0, b1, lane, s.x, s.x_stride, true, acc);
          else
            dot_range<N>(qs_tile, d_tile, b0, b1, lane, s.x, s.x_stride, s.gqa_group, s.gqa_hd,
                         s.gqa_off, acc);
        } else
          dot_range<N>(qs_tile, d_tile, b0, b1, lane, s.x, s.x_stride, s.gqa_group, s.gqa_hd,
                       s.gqa_off, acc);
      }
    } else if (lane == 0 && pr.dev_status) {
      atomicOr(pr.dev_status, 1);
    }
  }

  // ---- fold the units of this output tile in unit order -------------------
  float val[2][N];
  if (pr.P == 1) {
#pragma unroll
    for (int n = 0; n < N; ++n) lds_part[(wave * N + n) * 64 + lane] = acc[n];
    __syncthreads();
    if (wave != 0) return;
    fold_units<N>(p, pr, us, [&](int uu, int n) { return lds_part[(uu * N + n) * 64 + lane]; },
                  val);
  } else {
    float* gp = pr.part + (int64_t)ot * pr.U * N * 64;
    if (u < pr.U) {
#pragma unroll
      for (int n = 0; n < N; ++n) st_dev(gp + (u * N + n) * 64 + lane, acc[n]);
    }
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0) s_last = ticket_add(&pr.tile_tickets[ot]) == (unsigned)(pr.P - 1);
    __syncthreads();
    if (!s_last) return;
    if (threadIdx.x == 0) st_dev(&pr.tile_tickets[ot], 0u);  // ready for the next call
    if (pr.fold_lds) {
      // every wave of the last workgroup fetches a share of the tile's
      // partials, 8 loads a lane in flight together (indexes past the end
      // clamp to the last word and are not kept), into LDS; wave 0 then
      // folds them in the same order as from memory
      const int tot = pr.U * N * 64;
      const int nt = (int)blockDim.x;
      for (int b = (int)threadIdx.x; b < tot; b += 8 * nt) {
        float t[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = b + j * nt;
          t[j] = ld_dev(gp + (i < tot ? i : tot - 1));
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (b + j * nt < tot) lds_part[b + j * nt] = t[j];
      }
      __syncthreads();
      if (wave != 0) return;
      fold_units<N>(p, pr, us, [&](int uu, int n) { return lds_part[(uu * N + n) * 64 + lane]; },
                    val);
    } else {
      if (wave != 0) return;
      fold_units<N>(p, pr, us,
                    [&](int uu, int n) { return ld_dev(gp + (uu * N + n) * 64 + lane); }, val);
    }
  }

  // ---- epilogue ---------------------------------------------------------------
  float c = 1.0f;
  if (pr.flags & F_RMSNORM) {
    float ss = 0.f;
    if (pr.rms_K <= 1024) {
#pragma unroll
      for (int i = 0; i < 16; ++i) ss = fmaf(rx[i], rx[i], ss);
    } else {
      for (int k = lane; k < pr.rms_K; k += 64) {
        const float t = pr.rms_x[k];
        ss = fmaf(t, t, ss);
      }
    }
    ss = wave_sum(ss);
    c = 1.0f / sqrtf(ss / (float)pr.rms_K + pr.eps);
  }
  // matrix row of this lane's output
  int row = ot * kTile + lane;
  if (pr.flags & F_PAIRED) row = lane < 32 ? 32 * ot + lane : pr.M / 2 + 32 * ot + (lane - 32);
  bool valid = row < pr.Mout;
  if ((pr.flags & (F_PAIRED | F_SWIGLU)) == (F_PAIRED | F_SWIGLU)) {
    // lanes 0..31 hold gate rows, lanes 32..63 the matching up rows
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const float v = val[0][n] * c;
      const float up = __shfl(v, (lane + 32) & 63, 64);
      const float h = v / (1.0f + expf(-v)) * up;
      if (lane < 32 && valid) pr.y[n * pr.y_stride + row] = h;
    }
    return;
  }
  if (pr.R == 2) {
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const float gt = val[0][n] * c;
      const float up = val[1][n] * c;
      const float h = gt / (1.0f + expf(-gt)) * up;
      if (valid) pr.y[n * pr.y_stride + row] = h;
    }
    return;
  }
  float out[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    float v = val[0][n] * c;
    if ((pr.flags & F_RESIDUAL) && valid) v += pr.residual[row];
    out[n] = v;
    if (valid) pr.y[n * pr.y_stride + row] = v;
  }
  if (pr.flags & F_ARGMAX) {
    // per tile and column (max, lowest index); the fold over tiles runs in
    // the next kernel of the same call, ordered by the kernel boundary
#pragma unroll
    for (int n = 0; n < N; ++n) {
      float mv = valid ? out[n] : -INFINITY;
      int mi = row;
      wave_argmax(mv, mi);
      if (lane == 0) {
        pr.am_val[n * pr.Tout + ot] = mv;
        pr.am_idx[n * pr.Tout + ot] = mi;
      }
    }
  }
}

// Fold of per-tile argmax partials: lowest index among the largest values.
__global__ __launch_bounds__(256) void argmax_fold_kernel(const float* __restrict__ v,
                                                          const int32_t* __restrict__ idx, int n,
                                                          int32_t* out) {
  // block b folds column b: partials [b * n, (b + 1) * n) into out[b]
  v += (int64_t)blockIdx.x * n;
  idx += (int64_t)blockIdx.x * n;
  out += blockIdx.x;
  __shared__ float sv[4];
  __shared__ int si[4];
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  // loads of 16 entries per thread are issued before any compare, so a
  // launch waits about one memory round trip per 4096 partials
  constexpr int kU = 16;
  for (int i0 = 0; i0 < n; i0 += 256 * kU) {
    float tv[kU];
    int ti[kU];
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const int i = i0 + j * 256 + (int)threadIdx.x;
      tv[j] = i < n ? v[i] : -INFINITY;
      ti[j] = i < n ? idx[i] : 0x7fffffff;
    }
#pragma unroll
    for (int j = 0; j < kU; ++j)
      if (tv[j] > bv || (tv[j] == bv && ti[j] < bi)) {
        bv = tv[j];
        bi = ti[j];
      }
  }
  wave_argmax(bv, bi);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sv[wave] = bv;
    si[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w)
      if (sv[w] > bv || (sv[w] == bv && si[w] < bi)) {
        bv = sv[w];
        bi = si[w];
      }
    *out = bi;
  }
}

// ---------------------------------------------------------------------------
// Host side: planning and launch.
// ---------------------------------------------------------------------------
namespace {

int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  if (!v || !*v) return dflt;
  const int x = atoi(v);
  return x > 0 ? x : dflt;
}

// Planner targets, overridable for tuning sweeps (the overrides change the
// summation order, never the result beyond the stated tolerance):
//  Q8G_TARGET_WAVES  waves aimed for across one launch
//  Q8G_MIN_QUADS     fewest 4-block scale quads a unit (one wave's K range) owns
//  Q8G_MIN_UNITS     fewest units per 64-row tile when K allows
//  Q8G_MAX_WAVES     most waves per workgroup (units of one tile beyond it
//                    spill into more workgroups and a ticketed fold)
//  Q8G_WIDE_UNITS    units per tile of a plan with one to two tiles per
//                    compute unit at N >= 2 (default 8)
//  Q8G_WIDE_WAVES    most waves per workgroup in plans with a tile or more
//                    per compute unit (default 4)
int target_waves() {
  static const int v = env_int("Q8G_TARGET_WAVES", 2048);
  return v;
}
int min_quads() {
  static const int v = env_int("Q8G_MIN_QUADS", 1);
  return v;
}
int min_units() {
  static const int v = env_int("Q8G_MIN_UNITS", 4);
  return v;
}
int wide_units() {
  static const int v = env_int("Q8G_WIDE_UNITS", 8);
  return v;
}
int wide_waves() {
  static const int v = env_int("Q8G_WIDE_WAVES", 4);
  return v;
}
// Compute units of the current device (256 on an MI355X; that value when no
// device can be queried, e.g. when only sizing a workspace).
int num_cus() {
  static const int v = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0) {
      (void)hipGetLastError();
      return 256;
    }
    return n;
  }();
  return v;
}
int max_waves() {
  static const int v = env_int("Q8G_MAX_WAVES", kMaxWaves);
  return v < kMaxWaves ? v : kMaxWaves;
}

// Units of one tile of a pair, spread over the segments in proportion to
// their scale quads (each segment >= 1 unit, <= its quads).
void distribute(const ProbDesc& pd, int64_t us, int64_t blocks, int64_t* su) {
  int64_t left = us;
  for (int s = 0; s < pd.nseg; ++s) {
    const int64_t nb = cdiv(pd.seg[s].W->K / 32, 4);
    su[s] = us * nb / blocks;
    if (su[s] < 1) su[s] = 1;
    if (su[s] > nb) su[s] = nb;
    left -= su[s];
  }
  while (left > 0) {  // the segment with the most blocks per unit takes one more
    int best = -1;
    double bestr = 0;
    for (int s = 0; s < pd.nseg; ++s) {
      const int64_t nb = cdiv(pd.seg[s].W->K / 32, 4);
      if (su[s] >= nb) continue;
      const double r = (double)nb / (double)su[s];
      if (r > bestr) {
        bestr = r;
        best = s;
      }
    }
    if (best < 0) break;
    ++su[best];
    --left;
  }
  while (left < 0) {  // over budget because of the one-per-segment minimum
    int best = -1;
    double bestr = 1e300;
    for (int s = 0; s < pd.nseg; ++s) {
      if (su[s] <= 1) continue;
      const double r = (double)(cdiv(pd.seg[s].W->K / 32, 4)) / (double)su[s];
      if (r < bestr) {
        bestr = r;
        best = s;
      }
    }
    if (best < 0) break;
    --su[best];
    ++left;
  }
}

}  // namespace

// Output rows and output tiles of a problem.
static int64_t prob_mout(const ProbDesc& pd) {
  return (pd.R == 2 || (pd.flags & F_SWIGLU)) ? pd.M / 2 : pd.M;
}
static int64_t prob_tout(const ProbDesc& pd) {
  return (pd.flags & F_PAIRED) ? cdiv(pd.M, kTile) : cdiv(prob_mout(pd), kTile);
}

int plan_problems(const ProbDesc* probs, int nprob, int N, Plan* plan) {
  memset(plan, 0, sizeof(*plan));
  int64_t total_tout = 0;
  int segc = 0;
  for (int i = 0; i < nprob; ++i) {
    const ProbDesc& pd = probs[i];
    total_tout += prob_tout(pd);
    segc += pd.nseg;
  }
  if (segc > kMaxSeg || nprob > kMaxProb || total_tout <= 0) return Q8_EINVAL;
  // Several columns with at least one tile per compute unit: workgroups of
  // 4 waves (4 K-units each, longer-lived waves, more workgroups resident)
  // measured best for every N >= 2 (C4 gate_up 24576x4096: N=2 28.3 -> 25.4
  // us, N=8 69 -> 52 us); with fewer tiles the K split such a plan needs
  // costs more than it gains.  One plain problem with fewer than two tiles
  // per compute unit takes 8 units in two workgroups per tile instead: one
  // workgroup per tile would leave half the compute units with twice the
  // work of the others (the same gate_up shape at N = 4 and 8, Q8_0: 33.1 ->
  // 29.6 and 52.5 -> 47.3 us; Q6_K at N = 8: 83.3 -> 71.8 us).  Not for the
  // integer-activation path, which measured slower so (N = 8: 30.0 -> 35.4).
  // K-quant weights (a quad is 4-7 KB instead of 8.5) take the same 4-wave
  // plans at N = 1, with half the waves per launch when the tiles are few:
  // longer units amortise each wave's first load (N = 1, Q5_K / Q6_K gate_up
  // 24576x4096: 21.0 -> 20.6, 26.2 -> 24.6 us; down 4096x12288: 15.5 -> 14.3,
  // 17.2 -> 16.8 us).
  const int f0 = probs[0].seg[0].fmt;
  const bool kq = f0 != FMT_Q8_0 && N == 1;
  const bool wide = (N >= 2 || kq) && total_tout >= num_cus();
  const bool wide_split = wide && nprob == 1 && probs[0].nseg == 1 && probs[0].R == 1 &&
                          !probs[0].seg[0].qx && total_tout < 2 * (int64_t)num_cus();
  // Q8_0 with few tiles and a long K (one problem, N <= 4; K summed over its
  // segments) takes the same shape: C4 down 4096x12288 went from 32 units of
  // 3 quads in 8-wave workgroups to 16 units of 6 quads in 4-wave ones, N = 1
  // / 2 / 4: 15.8 -> 14.6, 17.8 -> 16.3, 21.7 -> 19.9 us; the MoE combine
  // (five segments, K = 11264) 13.6 -> 13.0 us.
  int64_t k_total = 0;
  for (int s = 0; s < probs[0].nseg; ++s) k_total += probs[0].seg[s].W->K;
  const bool few = !wide && f0 == FMT_Q8_0 && N <= 4 && nprob == 1 && probs[0].R == 1 &&
                   !probs[0].seg[0].qx && total_tout < num_cus() && k_total >= 4096;
  const int64_t want_u =
      wide ? (wide_split ? wide_units() : 4)
           : cdiv((kq || few) ? target_waves() / 2 : target_waves(), total_tout);
  const int wfmt = max_waves_for(N, f0 == FMT_Q6K || f0 == FMT_Q5K);
  int wmax = max_waves() < wfmt ? max_waves() : wfmt;
  if ((wide || kq || few) && wmax > wide_waves()) wmax = wide_waves();
  // units per tile
  int sbase = 0;
  int64_t U[kMaxProb];
  for (int i = 0; i < nprob; ++i) {
    const ProbDesc& pd = probs[i];
    // a unit owns whole scale quads of one segment; `blocks` below counts quads
    int64_t blocks = 0;
    for (int s = 0; s < pd.nseg; ++s) blocks += cdiv(pd.seg[s].W->K / 32, 4);
    const int64_t us_max = blocks / min_quads() > pd.nseg ? blocks / min_quads() : pd.nseg;
    int64_t us = cdiv(want_u, pd.R);
    const int64_t us_min = cdiv(min_units(), pd.R);
    if (us < us_min) us = us_min;
    if (us > us_max) us = us_max;
    // (few tiles, long K: at least 2 quads a unit; C2 down 896x4864 with 38
    // units of 1 quad 8.2 us, 19 units of 2 quads 7.2 us)
    if (few && us > blocks / 2) us = blocks / 2 > 0 ? blocks / 2 : 1;
    if (us < pd.nseg) us = pd.nseg;
    // a unit covers at most 16 scale quads (64 blocks), which with the
    // three-level fold keeps every output's chain of roundings short
    if (us < cdiv(blocks, 16)) us = cdiv(blocks, 16);
    if (us > blocks) us = blocks;
    // With few tiles per compute unit the slowest wave sets the pace: prefer
    // the nearest larger unit count that splits the quads evenly, while the
    // tile still fits one workgroup (C4 gate_up 24576x4096 at N = 1: 6 units
    // of 5-6 quads 24.7 us, 8 units of 4 quads 23.0 us).  With many tiles per
    // compute unit the overlap of workgroups hides the imbalance instead.  (Not
    // for the integer-activation path or several problems, where it measured
    // slower.)
    if (nprob == 1 && pd.nseg == 1 && pd.R == 1 && !pd.seg[0].qx &&
        total_tout < 2 * (int64_t)num_cus() && blocks % us) {
      for (int64_t c = us + 1; c < 2 * us && c <= wmax && c <= us_max; ++c)
        if (blocks % c == 0) {
          us = c;
          break;
        }
    }
    int64_t su[kMaxSeg];
    distribute(pd, us, blocks, su);
    int64_t usum = 0;
    for (int s = 0; s < pd.nseg; ++s) {
      plan->seg_units[sbase + s] = (int32_t)su[s];
      usum += su[s];
    }
    U[i] = usum * pd.R;
    sbase += pd.nseg;
  }
  // waves per workgroup (common to the launch) and workgroups per tile;
  // while the launch has fewer workgroups than the device has compute units,
  // smaller workgroups (more of them per tile) spread it over more units
  auto waves_per_wg = [&](int64_t cap) {
    int64_t W = 1;
    for (int i = 0; i < nprob; ++i) {
      const int64_t P = cdiv(U[i], cap);
      const int64_t w = cdiv(U[i], P);
      if (w > W) W = w;
    }
    return W;
  };
  auto workgroups = [&](int64_t W) {
    int64_t n = 0;
    for (int i = 0; i < nprob; ++i) n += prob_tout(probs[i]) * cdiv(U[i], W);
    return n;
  };
  int64_t cap = wmax;
  int64_t W = waves_per_wg(cap);
  // (only launches whose tiles already span several workgroups: a tile that
  // fits one workgroup keeps its cheaper in-workgroup fold)
  bool split = false;
  for (int i = 0; i < nprob; ++i) split |= cdiv(U[i], W) > 1;
  while (split && cap > 4 && workgroups(W) < num_cus()) {
    cap /= 2;
    W = waves_per_wg(cap);
  }
  int64_t cnt = 0;
  size_t data = 0;
  int64_t wg = 0;
  for (int i = 0; i < nprob; ++i) {
    const ProbDesc& pd = probs[i];
    const int64_t Tout = prob_tout(pd);
    const int64_t P = cdiv(U[i], W);
    plan->U[i] = (int32_t)U[i];
    plan->P[i] = (int32_t)P;
    plan->cnt_off[i] = (int32_t)cnt;
    plan->data_off[i] = data;
    if (P > 1) cnt += Tout;
    if (pd.flags & F_ARGMAX) data += align_up((size_t)Tout * N * 4, 256) * 2;
    if (P > 1) data += align_up((size_t)Tout * U[i] * N * 64 * 4, 256);
    wg += Tout * P;
  }
  if (cnt > kMaxCounters || wg > 0x7fffffff) return Q8_EINVAL;
  plan->W = (int32_t)W;
  plan->ws_bytes = (cnt > 0 || data > 0) ? kCounterBytes + data : 0;
  plan->total_wg = (int32_t)wg;
  return Q8_OK;
}

template <int N>
static hipError_t launch_n(const GemvParams& gp, int wgs, hipStream_t stream) {
  size_t lds = (size_t)gp.W * N * 64 * sizeof(float);
  for (int i = 0; i < gp.nprob; ++i)
    if (gp.prob[i].fold_lds) {
      const size_t f = (size_t)gp.prob[i].U * N * 64 * sizeof(float);
      if (f > lds) lds = f;
    }
  if (gp.seg[0].qx)  // the integer-activation path: one plain problem
    hipLaunchKernelGGL((gemv_kernel<N, true, 1>), dim3(wgs), dim3(64 * gp.W), lds, stream, gp);
  else if (gp.seg[0].fmt != FMT_Q8_0) {  // K-quants: one plain problem, N <= 4
    if constexpr (N <= kMaxQ4kN) {
      if (gp.seg[0].fmt == FMT_Q4K)
        hipLaunchKernelGGL((gemv_kernel<N, true, 2>), dim3(wgs), dim3(64 * gp.W), lds, stream,
                           gp);
      else if (gp.seg[0].fmt == FMT_Q5K)
        hipLaunchKernelGGL((gemv_kernel<N, true, 4>), dim3(wgs), dim3(64 * gp.W), lds, stream,
                           gp);
      else
        hipLaunchKernelGGL((gemv_kernel<N, true, 3>), dim3(wgs), dim3(64 * gp.W), lds, stream,
                           gp);
    } else {
      return hipErrorInvalidValue;
    }
  } else if (gp.nprob == 1 && gp.prob[0].nseg == 1)
    hipLaunchKernelGGL((gemv_kernel<N, true, 0>), dim3(wgs), dim3(64 * gp.W), lds, stream, gp);
  else
    hipLaunchKernelGGL((gemv_kernel<N, false, 0>), dim3(wgs), dim3(64 * gp.W), lds, stream, gp);
  return hipGetLastError();
}

int launch_problems(const ProbDesc* probs, int nprob, int N, void* ws, size_t ws_bytes,
                    hipStream_t stream, const RouteParams* route) {
  // the GQA prologue is a one-column operation; the kernels with several
  // columns do not implement it
  for (int i = 0; i < nprob; ++i)
    for (int s = 0; s < probs[i].nseg; ++s)
      if (probs[i].seg[s].gqa_group > 0 && N > 1) return Q8_EINVAL;
  Plan plan;
  int rc = plan_problems(probs, nprob, N, &plan);
  if (rc) return rc;
  if (plan.ws_bytes > 0 && (ws == nullptr || ws_bytes < plan.ws_bytes)) return Q8_EWORKSPACE;
  GemvParams gp;
  memset(&gp, 0, sizeof(gp));
  gp.nprob = nprob;
  int sbase = 0;
  int wg = 0;
  for (int i = 0; i < nprob; ++i) {
    const ProbDesc& pd = probs[i];
    Prob& pr = gp.prob[i];
    const int64_t Mout = prob_mout(pd);
    const int64_t Tout = prob_tout(pd);
    pr.seg0 = sbase;
    pr.nseg = pd.nseg;
    pr.R = pd.R;
    pr.M = (int32_t)pd.M;
    pr.Mout = (int32_t)Mout;
    pr.Tout = (int32_t)Tout;
    pr.U = plan.U[i];
    pr.P = plan.P[i];
    // In a launch of at most one workgroup per compute unit the last tile's
    // fold is the launch's tail: split tiles whose partials fit a
    // workgroup's LDS share at the kernel's occupancy (16 waves a compute
    // unit: 160 KB / 16 = 10 KB a wave, 8 KB kept) stage them there first
    // (MoE combine, 4 routed down 2048x1408 + shared 2048x5632 at N = 1:
    // 13.4 -> 12.4 us).  So do row-group launches whose waves are all
    // resident at once (C4 gate_up N = 8: 41.5 -> 39.2 us).  In launches of
    // several rounds other workgroups hide the fold, and the staging measured
    // slightly slower.
    pr.fold_lds = pr.P > 1 &&
                  (plan.total_wg <= num_cus() ||
                   (N >= 2 && (int64_t)plan.total_wg * plan.W <= 3 * 4 * (int64_t)num_cus())) &&
                  (int64_t)pr.U * N <= 32 * (int64_t)plan.W && pr.U * N <= 128;
    pr.wg0 = wg;
    pr.flags = pd.flags;
    pr.eps = pd.eps;
    pr.y = pd.y;
    pr.y_stride = pd.y_stride;
    pr.residual = pd.residual;
    pr.rms_x = pd.rms_x;
    pr.rms_K = (int32_t)pd.rms_K;
    pr.argmax_out = pd.argmax_out;
    pr.dev_status = pd.dev_status;
    if (plan.ws_bytes > 0) {
      uint8_t* base = static_cast<uint8_t*>(ws) + kCounterBytes + plan.data_off[i];
      if (pr.P > 1) pr.tile_tickets = static_cast<uint32_t*>(ws) + plan.cnt_off[i];
      if (pd.flags & F_ARGMAX) {
        pr.am_val = reinterpret_cast<float*>(base);
        base += align_up((size_t)Tout * N * 4, 256);
        pr.am_idx = reinterpret_cast<int32_t*>(base);
        base += align_up((size_t)Tout * N * 4, 256);
      }
      if (pr.P > 1) pr.part = reinterpret_cast<float*>(base);
    }
    for (int s = 0; s < pd.nseg; ++s) {
      const SegDesc& sd = pd.seg[s];
      Seg& sg = gp.seg[sbase + s];
      const int64_t K = sd.W->K;
      sg.qs = static_cast<const uint8_t*>(sd.W->qs);
      sg.d = static_cast<const uint8_t*>(sd.W->d);
      sg.qs_stride = sd.W->qs_stride;
      sg.d_stride = sd.W->d_stride;
      sg.eid = sd.eid;
      sg.slot = sd.slot;
      sg.n_mats = (int32_t)sd.W->n_mats;
      sg.x = sd.x;
      sg.x_stride = sd.x_stride;
      sg.K = (int32_t)K;
      sg.nblk = (int32_t)(K / 32);
      sg.G = (int32_t)cdiv(K / 32, 4);
      sg.units = plan.seg_units[sbase + s];
      sg.alpha_mode = sd.alpha_mode;
      sg.alpha_ptr = sd.alpha_ptr;
      sg.gqa_group = sd.gqa_group;
      sg.gqa_hd = sd.gqa_hd;
      sg.gqa_off = sd.gqa_off;
      sg.qx = sd.qx;
      sg.dx = sd.dx;
      sg.fmt = sd.fmt;
      sg.qh = static_cast<const uint8_t*>(sd.qh);
    }
    sbase += pd.nseg;
    wg += (int)(Tout * pr.P);
  }
  gp.total_wg = wg;
  gp.W = plan.W;
  // Progress priorities pay when all of a launch's waves are resident from
  // the start (the row-group instances hold at least 3 waves per SIMD); in
  // launches of several rounds, oldest-first issue frees slots sooner
  // (lm_head at N = 8: 62.5 us without, 64.9 with).
  gp.prio = (int64_t)wg * plan.W <= 3 * 4 * (int64_t)num_cus();
  if (route) gp.route = *route;  // (memset above: no router otherwise)
  if (wg <= 0) return Q8_OK;
  hipError_t e;
  switch (N) {
    case 1: e = launch_n<1>(gp, wg, stream); break;
    case 2: e = launch_n<2>(gp, wg, stream); break;
    case 3: e = launch_n<3>(gp, wg, stream); break;
    case 4: e = launch_n<4>(gp, wg, stream); break;
    case 5: e = launch_n<5>(gp, wg, stream); break;
    case 6: e = launch_n<6>(gp, wg, stream); break;
    case 7: e = launch_n<7>(gp, wg, stream); break;
    case 8: e = launch_n<8>(gp, wg, stream); break;
    default: return Q8_EINVAL;
  }
  if (e != hipSuccess) return Q8_ELAUNCH;
  for (int i = 0; i < nprob; ++i) {
    const Prob& pr = gp.prob[i];
    if (!(pr.flags & F_ARGMAX)) continue;
    hipLaunchKernelGGL(argmax_fold_kernel, dim3(N), dim3(256), 0, stream, pr.am_val, pr.am_idx,
                       pr.Tout, pr.argmax_out);
    if (hipGetLastError() != hipSuccess) return Q8_ELAUNCH;
  }
  return Q8_OK;
}

int launch_quantize_act(const float* x, int64_t K, int64_t N, int8_t* qx, uint16_t* dx,
                        hipStream_t stream) {
  const int64_t nblocks = N * (K / 32);
  if (nblocks <= 0) return Q8_OK;
  hipLaunchKernelGGL(quantize_act_kernel, dim3((unsigned)((nblocks + 7) / 8)), dim3(256), 0,
                     stream, x, K, nblocks, qx, dx);
  return hipGetLastError() == hipSuccess ? Q8_OK : Q8_ELAUNCH;
}

}  // namespace q8
