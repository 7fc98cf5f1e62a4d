/*
 * q8gemv.h -- C ABI of the MI355X (gfx950) Q8_0 decode GEMV library.
 *
 * What it computes.  Batch-1 (and small-batch) decode matrix-vector products
 * of a Qwen-style decoder with Q8_0 block-quantised weights and fp32
 * activations: the qkv, wo, fused gate_up, down and lm_head projections
 * ("Lumen v0.3.0" release notes, section "Phase 7.E.0", where these matmuls
 * take 88.6 % of decode time), greedy argmax over the logits ("augur" README,
 * "Features": greedy generation), and the routed-expert FFN of a Qwen-MoE
 * layer with all selected expert slots in one launch ("Add Qwen1.5-MoE Q8_0
 * CPU and single-token TornadoVM GPU inference - #144", the routed-expert
 * fusion comments: slot index folded into the work-group id for gate/up, the
 * down projection looping over slots).
 *
 * Q8_0 block (GGUF, "raw GGUF Q8_0 block layout" on the cogni-ml README,
 * cuda_q8_gemv_probe): 32 consecutive weights of one row share one binary16
 * scale d; each weight is d * q with q a signed 8-bit integer.  In GGUF files
 * a block is 34 bytes: d (little-endian) then the 32 quants.
 *
 * Arithmetic: quants and scales are converted exactly to fp32, products and
 * sums are fp32 FMAs, activations stay fp32 (no requantisation).  The GEMV
 * at N >= 5 columns runs each block as bf16 matrix-core products on an exact
 * three-part bf16 split of each activation.  Its products are exact too, and
 * only the fp32 summation order differs.  Results
 * agree with the exact value within 2e-5 * sum_k |w_k x_k| + 1e-6 per output.
 * For a fixed (M, K, N) and device the summation order is fixed: repeated
 * calls give bitwise identical results.
 *
 * Conventions for every entry point:
 *  - Device pointers are device memory of the current HIP device (hipMalloc
 *    or torch CUDA tensors).  Host pointers passed where device memory is
 *    required are rejected with Q8_EHOSTPTR before any launch.
 *  - The library never allocates, frees or synchronises inside a call; all
 *    work is enqueued on `stream` (a hipStream_t; NULL = the default stream),
 *    so calls are stream-ordered with other work and may be captured into a
 *    HIP graph.
 *  - The caller owns every buffer.  Outputs are written only by the kernels,
 *    after the call returns Q8_OK (i.e. when the stream reaches them).
 *  - Return value: Q8_OK (0) or a negative Q8_E* code; nothing is enqueued
 *    when a call returns an error.  q8_0_strerror() names the code.
 *  - Empty problems (M == 0, or n == 0 for argmax) return Q8_OK and enqueue
 *    nothing.
 *  - Workspace: calls that take one need workspace_bytes >= the value from
 *    q8_0_workspace_bytes() for the same op and shape (0 means none is
 *    needed and the pointer may be NULL).  Its first 64 KiB are arrival
 *    counters used to hand partial results between workgroups; every call
 *    leaves them at zero, and partial results always live after them, so one
 *    workspace, zero-filled once before its first use, serves any sequence of
 *    stream-ordered calls of any shapes.  Calls that may run concurrently
 *    (different streams, or the same stream inside concurrent graph
 *    branches) need distinct workspaces.
 */
#ifndef Q8GEMV_H
#define Q8GEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define Q8_OK 0
#define Q8_EINVAL (-1)     /* bad scalar argument: shape, count, flag combination */
#define Q8_ENULL (-2)      /* a required pointer is NULL */
#define Q8_EALIGN (-3)     /* a pointer lacks the alignment stated below */
#define Q8_EHOSTPTR (-4)   /* a pointer that must be device memory is not */
#define Q8_EWORKSPACE (-5) /* workspace missing or smaller than required */
#define Q8_ELAUNCH (-6)    /* the HIP runtime reported an error */

/* ---- limits -------------------------------------------------------------- */
#define Q8_QK 32            /* weights per block */
#define Q8_TILE_ROWS 64     /* rows per packed tile (one row per wave64 lane) */
#define Q8_MAX_N 8          /* activation columns per call */
#define Q8_MAX_SLOTS 8      /* routed-expert slots per MoE call */
#define Q8_MAX_K (1 << 20)  /* largest K accepted */

/* ---- packed weight layout (output of q8_0_repack) -------------------------
 * For an M x K matrix (K % 32 == 0), T = ceil(M / 64) tiles of 64 rows,
 * nb = K / 32 blocks per row, G = ceil(nb / 4) scale quads per row.
 *  qs: T * 64 * K bytes.  The 16 quants k = 16c .. 16c+15 of row r sit at byte
 *      ((t * (K/16) + c) * 64 + i) * 16, t = r / 64, i = r % 64: one 16-byte
 *      chunk per row, 64 rows of one chunk contiguous (1 KiB).
 *  d:  T * G * 64 * 8 bytes.  The scale of block b of row r sits at uint16
 *      index ((t * G + b / 4) * 64 + i) * 4 + b % 4 (binary16 bits).
 *  Rows M .. 64T-1 and blocks nb .. 4G-1 are zero.  Alignment: qs 16 bytes,
 *  d 8 bytes.  A stack of E matrices (MoE experts) is E packed matrices at a
 *  fixed byte stride. */
typedef struct {
  const void* qs;    /* device, packed quants of matrix 0 */
  const void* d;     /* device, packed scales of matrix 0 */
  int64_t M, K;      /* shape of one matrix */
  int64_t n_mats;    /* stacked matrices (experts); 1 for a dense matrix */
  int64_t qs_stride; /* bytes from one matrix's qs to the next (>= packed qs size) */
  int64_t d_stride;  /* bytes from one matrix's d to the next */
  int32_t layout;    /* Q8_LAYOUT_ROWS or Q8_LAYOUT_GATE_UP_PAIRS (how it was repacked) */
  int32_t reserved;  /* 0 */
} q8_0_weights;

/* Row order inside the packed tiles.
 *  Q8_LAYOUT_ROWS: packed row r is matrix row r.
 *  Q8_LAYOUT_GATE_UP_PAIRS: for a fused gate/up matrix (rows 0..M/2-1 gate,
 *    M/2..M-1 up; M % 64 == 0), lanes 0..31 of tile t hold gate rows
 *    32t..32t+31 and lanes 32..63 the matching up rows M/2+32t..M/2+32t+31,
 *    so a SwiGLU epilogue pairs rows within one wave and every tile yields 32
 *    outputs.  GEMV outputs are still written in matrix row order. */
#define Q8_LAYOUT_ROWS 0
#define Q8_LAYOUT_GATE_UP_PAIRS 1

/* Bytes of the packed quants and scales of one M x K matrix.
 * Errors: Q8_EINVAL (M < 0, K <= 0, K % 32, K > Q8_MAX_K), Q8_ENULL. */
int q8_0_packed_size(int64_t M, int64_t K, size_t* qs_bytes, size_t* d_bytes);

/* Load-time repack of GGUF Q8_0 blocks into the packed layout above (no value
 * changes; byte moves only).
 *  aos: device, M * K/32 blocks of 34 bytes, row-major, 2-byte aligned.
 *  qs, d: device outputs of q8_0_packed_size() bytes (16- and 8-byte aligned);
 *  every byte, padding included, is written.
 * Errors: Q8_EINVAL, Q8_ENULL, Q8_EALIGN, Q8_EHOSTPTR, Q8_ELAUNCH. */
int q8_0_repack(const void* aos, int64_t M, int64_t K, void* qs, void* d, void* stream);

/* The repack from host memory: aos_host holds the M * K/32 blocks of 34
 * bytes (row-major, as read from a GGUF file; pageable or pinned host
 * memory, or device memory).  They move to the device through `staging`, a
 * caller-owned device buffer of staging_bytes (16-byte aligned), in bands of
 * whole 64-row tiles: each band is one stream-ordered copy (two for the
 * gate/up pairs layout: its gate rows, then the matching up rows) followed
 * by the repack of those tiles, so staging is reused band after band and
 * the library allocates nothing.  A larger staging buffer means fewer
 * bands; q8_0_repack_staging_bytes(M, K) gives the smallest (one tile of
 * rows).  layout, qs and d as q8_0_repack_layout; the packed bytes are the
 * same as q8_0_repack_layout's on a device copy of aos_host.  The call
 * returns once the last copy is queued (pageable host memory may make the
 * copies synchronous); aos_host must stay valid until the stream has run
 * them.  Errors: Q8_EINVAL, Q8_ENULL, Q8_EALIGN, Q8_EHOSTPTR (qs, d or
 * staging not device memory), Q8_EWORKSPACE (staging_bytes below one tile
 * of rows), Q8_ELAUNCH. */
int q8_0_repack_host(const void* aos_host, int64_t M, int64_t K, int32_t layout, void* qs,
                     void* d, void* staging, size_t staging_bytes, void* stream);

/* Smallest staging buffer q8_0_repack_host accepts for an M x K matrix:
 * 64 rows of 34-byte blocks (0 for an invalid shape or M == 0). */
size_t q8_0_repack_staging_bytes(int64_t M, int64_t K);

/* The same with a row order: layout Q8_LAYOUT_ROWS (as q8_0_repack) or
 * Q8_LAYOUT_GATE_UP_PAIRS (M % 64 == 0).  Set the descriptor's `layout` to
 * the same value.  Errors as q8_0_repack. */
int q8_0_repack_layout(const void* aos, int64_t M, int64_t K, int32_t layout, void* qs, void* d,
                       void* stream);

/* ---- GEMV ------------------------------------------------------------------
 * y[n][r] = sum_k w[r][k] * x[n][k],  n < N, r < M.
 *  W: host pointer to a descriptor of packed device weights (n_mats == 1);
 *     W->M and W->K must equal M and K.
 *  x: device fp32 [N][K], 4-byte aligned.  y: device fp32 [N][M].
 *  1 <= N <= Q8_MAX_N.  x and y must not overlap.
 * The N = 1 case is the decode projection; N in {2,4,8} is a small verify
 * chunk ("skuznetsov/cogni-ml" README, "Qwen 3.5 Native Metal":
 * target-verifier chunks), weights read once for all N columns.
 * Arithmetic: every product q * x is exact and sums run in fp32, in an order
 * fixed by (M, K, N), so repeated calls give bitwise the same y.  N <= 4 uses
 * fp32 FMAs on the converted quants.  N >= 5 uses bf16 matrix-core products,
 * with each activation split into three bf16 parts whose sum is x (for
 * |x| above about 2^-110).  So a
 * column's last bits may differ between an N <= 4 and an N >= 5 call.
 * Errors: Q8_EINVAL, Q8_ENULL, Q8_EALIGN, Q8_EHOSTPTR, Q8_EWORKSPACE,
 * Q8_ELAUNCH. */
int q8_0_gemv(const q8_0_weights* W, const float* x, float* y, int64_t M, int64_t K, int64_t N,
              void* workspace, size_t workspace_bytes, void* stream);

/* ---- GEMV without allocation -------------------------------------------------
 * For callers that cannot allocate or pass a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  The same
 * product as q8_0_gemv (same kernels and plan, so bitwise the same y), with
 * the split-K partials and tickets in a library-owned device array of 8 MiB
 * per device (held until the process ends) instead of a workspace; it calls
 * no allocator.  Every call on one device shares that array: calls that
 * overlap on a device (different streams without ordering) race and must not
 * be issued; stream-ordered calls are fine (each clears the array's ticket
 * counters first, with a small kernel on the same stream).  Errors as
 * q8_0_gemv, and Q8_EWORKSPACE if the plan for (M, K, N) needs more than the
 * array holds (q8_0_workspace_bytes(Q8_OP_GEMV, ...) > 8 MiB). */
int q8_0_gemv_noalloc(const q8_0_weights* W, const float* x, float* y, int64_t M, int64_t K,
                      int64_t N, void* stream);

/* ---- GEMV with fused decode-chain glue (N = 1) ----------------------------
 * The non-matmul steps between the projections of one Qwen2-style decoder
 * layer ("augur" README, "Features": RMSNorm before attention, before the MLP
 * and after the last layer; grouped-query attention; SwiGLU MLP; decoder
 * block order norm, attention, residual, norm, MLP, residual), folded into
 * the GEMV so the chain needs no extra launches:
 *  prologue Q8_PRO_RMSNORM: the GEMV input is a = x / sqrt(mean(x^2) + eps)
 *      (unit norm weight) over the K entries of x.
 *  prologue Q8_PRO_GQA: the GEMV input is the position-0 attention output
 *      a[h*hd + j] = x[gqa_offset + (h / (n_heads/n_kv_heads)) * hd + j],
 *      K == n_heads * hd, hd % 32 == 0 (with one key the softmax weight is 1,
 *      so each query head returns its key/value head's value vector).
 *  epilogue Q8_EPI_SWIGLU: rows 0..M/2-1 are gate, M/2..M-1 up; y gets M/2
 *      values silu(g) * u, silu(z) = z/(1+e^-z).  Needs M % 64 == 0 with the
 *      Q8_LAYOUT_GATE_UP_PAIRS layout, else (M/2) % 64 == 0.
 *  epilogue Q8_EPI_RESIDUAL: y[r] = residual[r] + (W a)[r]; residual may be y
 *      itself (in-place h += W a).
 *  epilogue Q8_EPI_ARGMAX: also writes to *argmax_out the lowest index of the
 *      largest y value (fp32 comparisons, "fusedtok 1.3.0", "API stability":
 *      ties resolve to the earliest index).
 *  SWIGLU excludes RESIDUAL and ARGMAX.
 * Errors as q8_0_gemv. */
#define Q8_PRO_NONE 0
#define Q8_PRO_RMSNORM 1
#define Q8_PRO_GQA 2
#define Q8_EPI_RESIDUAL 1
#define Q8_EPI_SWIGLU 2
#define Q8_EPI_ARGMAX 4
typedef struct {
  int32_t prologue;       /* Q8_PRO_* */
  int32_t epilogue;       /* OR of Q8_EPI_* */
  float eps;              /* RMSNORM epsilon */
  int32_t n_heads;        /* GQA */
  int32_t n_kv_heads;     /* GQA */
  int32_t head_dim;       /* GQA */
  int64_t gqa_offset;     /* GQA: index in x of the first value-head element */
  const float* residual;  /* RESIDUAL: device fp32 [M] */
  int32_t* argmax_out;    /* ARGMAX: device int32 [1] */
} q8_0_fusion;

int q8_0_gemv_fused(const q8_0_weights* W, const float* x, float* y, int64_t M, int64_t K,
                    const q8_0_fusion* fusion, void* workspace, size_t workspace_bytes,
                    void* stream);

/* ---- GEMV with one argmax per column (verify chunk) --------------------------
 * y as q8_0_gemv (1 <= N <= Q8_MAX_N columns), and argmax_out[n] (device int32
 * [N]) = min{ r : y[n][r] == max_j y[n][j] }: the greedy pick of each of the
 * N logit rows of a verify chunk ("skuznetsov/cogni-ml" README, "Qwen 3.5
 * Native Metal": target-verifier chunks and the resident top-1 over logits)
 * with ties to the earliest index ("fusedtok 1.3.0", "API stability").  The
 * picks compare the same fp32 values the call writes to y.  One GEMV launch
 * (per-tile maxima in its epilogue) plus one small fold launch.
 * Errors as q8_0_gemv; argmax_out must be 4-byte aligned device memory. */
int q8_0_gemv_argmax(const q8_0_weights* W, const float* x, float* y, int64_t M, int64_t K,
                     int64_t N, int32_t* argmax_out, void* workspace, size_t workspace_bytes,
                     void* stream);

/* ---- integer-activation variant (opt-in; not the fp32 path) ---------------------
 * The Qwen1.5-MoE PR ("#144", "Key implementation notes") quantizes each
 * fp32 activation block to int8 before the dot product and accumulates
 * int8 x int8 products with the Q8_0 scales.  Reading taken for the
 * quantizer (the page does not give it): each block of 32 activations
 * becomes a Q8_0 block like the weights,
 *   d = max_j |x_j| / 127 (fp32 division, round to nearest even),
 *   q_j = x_j / d (fp32 division) rounded to the nearest integer, ties to
 *         even (all zero when max_j |x_j| == 0),
 *   stored scale dx = binary16(d), round to nearest even;
 * the product uses the stored scale:
 *   y[n][r] = sum_b dw[r][b] * dx[n][b] * sum_j qw[r][b][j] * qx[n][b][j],
 * with each block's integer sum exact (int32) and the rest in fp32.  Results
 * differ from q8_0_gemv by the activation rounding (about 0.4 % of a block's
 * largest activation per entry), so this is a separate, opt-in product.
 *
 * q8_0_quantize_act: x device fp32 [N][K] (4-byte aligned) -> qx device
 *   int8 [N][K] (4-byte aligned) and dx device binary16 bits [N][K/32]
 *   (2-byte aligned); K % 32 == 0, 1 <= N <= Q8_MAX_N.  Activation blocks
 *   whose d would be an fp32 subnormal (max |x| below about 1.5e-36) are
 *   outside the contract.
 * q8_0_gemv_q8act: y [N][M] from packed weights W (as q8_0_gemv) and the
 *   output of q8_0_quantize_act; workspace as q8_0_gemv (Q8_OP_GEMV).
 * Errors as q8_0_gemv. */
int q8_0_quantize_act(const float* x, int64_t K, int64_t N, int8_t* qx, uint16_t* dx,
                      void* stream);
int q8_0_gemv_q8act(const q8_0_weights* W, const int8_t* qx, const uint16_t* dx, float* y,
                    int64_t M, int64_t K, int64_t N, void* workspace, size_t workspace_bytes,
                    void* stream);

/* ---- Q4_K weights (NEXT-2) -------------------------------------------------------
 * GGUF Q4_K ("skuznetsov/cogni-ml" README, cuda_q4k_gemv_probe: d, dmin,
 * 12-byte packed scales/mins, 128-byte packed nibbles).  Reading of the packing
 * (the page lists the fields; the arrangement is GGUF's): a 144-byte block holds
 * 256 weights of one row as 8 sub-blocks of 32;
 *   bytes 0-1 d, 2-3 dmin (binary16, little-endian);
 *   bytes 4-15 sc[12]: sub-block j's 6-bit scale s_j and min m_j are, for
 *     j < 4, the low 6 bits of sc[j] and sc[j+4]; for j >= 4, the low and high
 *     nibbles of sc[j+4] plus 16 times the top two bits of sc[j-4] and sc[j];
 *   bytes 16-143: weight k's 4-bit quant q_k in byte 32 (k / 64) + k % 32,
 *     low nibble when k % 64 < 32, else high nibble;
 *   w_k = d * s_j * q_k - dmin * m_j, j = k / 32.
 *
 * Packed layout (q4k_repack), T = ceil(M / 64) tiles of 64 rows:
 *  qs:   T * (K/32) * 64 * 16 bytes; sub-block c of row r is the 16 bytes at
 *        ((t * (K/32) + c) * 64 + i) * 16 (t = r / 64, i = r % 64), whose byte
 *        b holds the sub-block's weights b (low nibble) and b + 16 (high).
 *  meta: T * (K/256) * 64 * 16 bytes; block B of row r: its first 16 GGUF bytes
 *        (d, dmin, sc) at ((t * (K/256) + B) * 64 + i) * 16.
 *  Rows M .. 64T-1 are zero.  Both 16-byte aligned. */
typedef struct {
  const void* qs;    /* device, packed nibbles */
  const void* meta;  /* device, packed block headers */
  int64_t M, K;
} q4k_weights;

/* Bytes of the packed nibbles and headers of one M x K Q4_K matrix.
 * Errors: Q8_ENULL, Q8_EINVAL (M < 0, K <= 0, K % 256, K > Q8_MAX_K). */
int q4k_packed_size(int64_t M, int64_t K, size_t* qs_bytes, size_t* meta_bytes);

/* Load-time repack of GGUF Q4_K blocks (device, M * K/256 blocks of 144 bytes,
 * row-major, 4-byte aligned) into qs and meta (device, q4k_packed_size() bytes,
 * 16-byte aligned; every byte written).  Nibble and byte moves only.
 * Errors: Q8_EINVAL, Q8_ENULL, Q8_EALIGN, Q8_EHOSTPTR, Q8_ELAUNCH. */
int q4k_repack(const void* blocks, int64_t M, int64_t K, void* qs, void* meta, void* stream);

/* y[n][r] = sum_k w[r][k] * x[n][k] with Q4_K weights, x fp32 [N][K] and y
 * fp32 [N][M] (device, 4-byte aligned), 1 <= N <= Q8_MAX_N, K % 256 == 0.
 * Each sub-block adds d s_j * sum_k q_k x_k - dmin m_j * sum_k x_k in fp32.
 * All N columns run in one launch (the weights are read once).
 * Workspace: q8_0_workspace_bytes(Q8_OP_Q4K_GEMV, M, K, N, 0, 0, 0) bytes
 * (device; NULL when 0), as for q8_0_gemv.  Errors as q8_0_gemv. */
int q4k_gemv(const q4k_weights* W, const float* x, float* y, int64_t M, int64_t K, int64_t N,
             void* workspace, size_t workspace_bytes, void* stream);

/* ---- Q5_K weights (NEXT-2) -------------------------------------------------------
 * GGUF Q5_K ("skuznetsov/cogni-ml" README, cuda_q5k_gemv_probe).  Reading of
 * the packing (the page names the format; the arrangement is GGUF's): a
 * 176-byte block holds 256 weights of one row: bytes 0-15 the Q4_K header (d,
 * dmin, 12 bytes of 6-bit scales and mins), 16-47 qh (bit j of byte l is the
 * fifth bit of weight 32 j + l), 48-175 the low 4 bits placed as Q4_K's
 * nibbles; w_k = d s_j (low + 16 fifth) - dmin m_j, j = k / 32.
 *
 * Packed layout (q5k_repack), T = ceil(M / 64) tiles of 64 rows, t = r / 64,
 * i = r % 64, c = 32-weight sub-block:
 *  qs:   T * (K/32) * 64 * 16 bytes, the low 4 bits as q4k_repack's qs.
 *  qh:   T * (K/128) * 64 * 16 bytes; at ((t * (K/128) + c / 4) * 64 + i) * 16
 *        + 4 (c % 4) a dword whose bit 8b + a is the fifth bit of the
 *        sub-block's weight 4a + b and bit 8b + 4 + a that of weight
 *        16 + 4a + b (a, b < 4).
 *  meta: as q4k_repack's meta (the 16-byte header of every block).
 *  Rows M .. 64T-1 are zero.  Alignment: 16 bytes each. */
typedef struct {
  const void* qs;    /* device, packed low 4 bits */
  const void* qh;    /* device, packed fifth bits */
  const void* meta;  /* device, packed block headers */
  int64_t M, K;
} q5k_weights;

/* Bytes of the packed arrays of one M x K Q5_K matrix.
 * Errors: Q8_ENULL, Q8_EINVAL (M < 0, K <= 0, K % 256, K > Q8_MAX_K). */
int q5k_packed_size(int64_t M, int64_t K, size_t* qs_bytes, size_t* qh_bytes,
                    size_t* meta_bytes);

/* Load-time repack of GGUF Q5_K blocks (device, M * K/256 blocks of 176 bytes,
 * row-major, 4-byte aligned) into qs, qh and meta (device, q5k_packed_size()
 * bytes, 16-byte aligned; every byte written).  Bit moves only.
 * Errors: Q8_EINVAL, Q8_ENULL, Q8_EALIGN, Q8_EHOSTPTR, Q8_ELAUNCH. */
int q5k_repack(const void* blocks, int64_t M, int64_t K, void* qs, void* qh, void* meta,
               void* stream);

/* y[n][r] = sum_k w[r][k] * x[n][k] with Q5_K weights; x, y, N, K and the
 * workspace (op Q8_OP_Q5K_GEMV) as q4k_gemv.  Each sub-block adds
 * d s_j * sum_k code_k x_k - dmin m_j * sum_k x_k in fp32 (code = low + 16
 * fifth); all columns run in one launch.  Errors as q8_0_gemv. */
int q5k_gemv(const q5k_weights* W, const float* x, float* y, int64_t M, int64_t K, int64_t N,
             void* workspace, size_t workspace_bytes, void* stream);

/* ---- Q6_K weights (NEXT-2) -------------------------------------------------------
 * GGUF Q6_K ("skuznetsov/cogni-ml" README, cuda_q6k_gemv_probe: ql, qh, signed
 * scales, d).  Reading of the packing (the page lists the fields; the
 * arrangement is GGUF's): a 210-byte block holds 256 weights of one row;
 * bytes 0-127 ql (low 4 bits), 128-191 qh (high 2 bits), 192-207 sixteen int8
 * scales (one per 16 weights), 208-209 d (binary16).  Weight k = 128 h + 32 a + l
 * (h < 2, a < 4, l < 32) takes its low bits from ql[64 h + 32 (a % 2) + l]
 * (low nibble for a < 2, else high) and its high bits from bits 2a, 2a + 1 of
 * qh[32 h + l]; w_k = d * scale[k / 16] * (low + 16 high - 32).
 *
 * Packed layout (q6k_repack), T = ceil(M / 64) tiles of 64 rows, t = r / 64,
 * i = r % 64, c = 32-weight sub-block, g = 128-weight quad:
 *  ql:   T * (K/32) * 64 * 16 bytes; at ((t * (K/32) + c) * 64 + i) * 16, byte b
 *        holds the low bits of the sub-block's weights b (low nibble) and
 *        b + 16 (high nibble).
 *  qh:   T * (K/32) * 64 * 8 bytes; at ((t * (K/32) + c) * 64 + i) * 8, two
 *        dwords: the high bits of weights 0..15 (bits 2b, 2b+1 for weight b),
 *        then of weights 16..31.
 *  meta: T * (K/128) * 64 * 16 bytes; at ((t * (K/128) + g) * 64 + i) * 16 the
 *        quad's 8 scales, d (binary16), then 6 zero bytes.
 *  Rows M .. 64T-1 are zero.  Alignment: ql, meta 16 bytes; qh 8 bytes. */
typedef struct {
  const void* ql;    /* device, packed low bits */
  const void* qh;    /* device, packed high bits */
  const void* meta;  /* device, packed scales and d */
  int64_t M, K;
} q6k_weights;

/* Bytes of the packed arrays of one M x K Q6_K matrix.
 * Errors: Q8_ENULL, Q8_EINVAL (M < 0, K <= 0, K % 256, K > Q8_MAX_K). */
int q6k_packed_size(int64_t M, int64_t K, size_t* ql_bytes, size_t* qh_bytes,
                    size_t* meta_bytes);

/* Load-time repack of GGUF Q6_K blocks (device, M * K/256 blocks of 210 bytes,
 * row-major, any alignment) into ql, qh and meta (device, q6k_packed_size()
 * bytes; every byte written).  Bit moves only.
 * Errors: Q8_EINVAL, Q8_ENULL, Q8_EALIGN, Q8_EHOSTPTR, Q8_ELAUNCH. */
int q6k_repack(const void* blocks, int64_t M, int64_t K, void* ql, void* qh, void* meta,
               void* stream);

/* y[n][r] = sum_k w[r][k] * x[n][k] with Q6_K weights; x, y, N, K and the
 * workspace (op Q8_OP_Q6K_GEMV) as q4k_gemv.  Each 16-weight group adds
 * d s * (sum(code x) - 32 sum(x)) in fp32; all columns run in one launch.
 * Errors as q8_0_gemv. */
int q6k_gemv(const q6k_weights* W, const float* x, float* y, int64_t M, int64_t K, int64_t N,
             void* workspace, size_t workspace_bytes, void* stream);

/* ---- argmax ------------------------------------------------------------------
 * *out_idx = min{ i : v[i] == max_j v[j] } over fp32 v[0..n) (device), as
 * int32 (device).  Inputs are finite (NaN is outside the contract).
 * Errors: Q8_EINVAL (n < 0 or n >= 2^31), Q8_ENULL, Q8_EHOSTPTR,
 * Q8_EWORKSPACE, Q8_ELAUNCH. */
int q8_0_argmax(const float* v, int64_t n, int32_t* out_idx, void* workspace,
                size_t workspace_bytes, void* stream);

/* ---- MoE router --------------------------------------------------------------
 * Top-k of E fp32 router logits (device): expert_ids[s] (device int32 [k]) are
 * the k largest logits in descending order, ties to the lower expert index;
 * slot_weights[s] (device fp32 [k]) = exp(l_s - l_max) / sum over the chosen
 * t of exp(l_t - l_max), i.e. softmax over all experts renormalised over the
 * chosen ones (#144 PR: router + top-k experts).  Selection compares the
 * logits themselves.  1 <= k <= min(E, Q8_MAX_SLOTS), E <= 1024.
 * Errors: Q8_EINVAL, Q8_ENULL, Q8_EHOSTPTR, Q8_ELAUNCH. */
int q8_0_route_topk(const float* logits, int32_t E, int32_t k, int32_t* expert_ids,
                    float* slot_weights, void* stream);

/* ---- MoE expert GEMV, all slots in one launch -------------------------------
 * W_experts: stacked packed matrices (n_mats experts, M x K each).
 * expert_ids: device int32 [n_slots]; read on the device, so the call needs no
 *   host round trip.  An id outside [0, n_mats) makes that slot contribute
 *   zeros and sets bit 0 of *dev_status (if dev_status != NULL); no memory is
 *   read through it.
 * mode Q8_MOE_SCATTER (gate_up of every slot, one launch):
 *   y[s][r] = (W_e[s] x)[r], x device fp32 [K], y [n_slots][M]; if `shared`
 *   is given (M_sh x K), its product follows at y + n_slots*M.
 *   With Q8_MOE_SWIGLU each matrix's rows are gate then up halves and y gets
 *   silu(g)*u instead: [n_slots][M/2] then [M_sh/2] ((M/2) % 64 == 0).
 * mode Q8_MOE_COMBINE (down of every slot plus the shared expert, one launch):
 *   y[r] = sum_s slot_weights[s] * (W_e[s] x_s)[r]
 *          + sigmoid(*shared_gate) * (shared x_sh)[r],
 *   x = [n_slots][K] then [shared->K], y [M]; folded per output row in slot
 *   order, then the shared expert (#144 PR: each slot reduced with the same
 *   tree and folded in the same order).  shared may be NULL (no shared term).
 *   slot_weights: device fp32 [n_slots]; shared_gate: device fp32 scalar.
 * Errors: Q8_EINVAL, Q8_ENULL, Q8_EALIGN, Q8_EHOSTPTR, Q8_EWORKSPACE,
 * Q8_ELAUNCH. */
#define Q8_MOE_SCATTER 1
#define Q8_MOE_COMBINE 2
#define Q8_MOE_SWIGLU 4
int q8_0_moe_gemv(const q8_0_weights* W_experts, const int32_t* expert_ids,
                  const float* slot_weights, const float* x, float* y, int64_t M, int64_t K,
                  int32_t n_slots, int32_t mode, const q8_0_weights* shared,
                  const float* shared_gate, int32_t* dev_status, void* workspace,
                  size_t workspace_bytes, void* stream);

/* ---- MoE router fused into the gate_up launch ----------------------------------
 * The router of q8_0_route_topk and the Q8_MOE_SCATTER launch of
 * q8_0_moe_gemv in one launch (#144 PR: the router may share the routed-
 * expert launch, fewer launches per layer): every wave that computes a routed
 * slot picks its own expert from router_logits (device fp32 [E]), with the
 * same selection rule, so no kernel boundary separates routing from the
 * experts' weights.  The launch also writes expert_ids (device int32
 * [n_slots]) and slot_weights (device fp32 [n_slots]) exactly as
 * q8_0_route_topk would, for the Q8_MOE_COMBINE call that follows.
 * mode: Q8_MOE_SCATTER, optionally | Q8_MOE_SWIGLU; x, y, M, K, shared,
 * dev_status and the workspace as in q8_0_moe_gemv (workspace size: op
 * Q8_OP_MOE_SCATTER).  1 <= n_slots <= min(E, Q8_MAX_SLOTS), E <= 1024 and
 * E <= W_experts->n_mats.  With M == 0 only the ids and weights are written.
 * Errors: Q8_EINVAL, Q8_ENULL, Q8_EALIGN, Q8_EHOSTPTR, Q8_EWORKSPACE,
 * Q8_ELAUNCH. */
int q8_0_moe_route_gemv(const q8_0_weights* W_experts, const float* router_logits, int32_t E,
                        int32_t* expert_ids, float* slot_weights, const float* x, float* y,
                        int64_t M, int64_t K, int32_t n_slots, int32_t mode,
                        const q8_0_weights* shared, int32_t* dev_status, void* workspace,
                        size_t workspace_bytes, void* stream);

/* ---- persistent decode chain --------------------------------------------------
 * One launch runs a whole decode step of a Qwen2-style decoder at position 0,
 * the per-layer steps of the fused GEMVs above in the decoder block order of
 * the "augur" README ("Features": RMSNorm, grouped-query attention, SwiGLU
 * MLP, residuals), unit norm weights and no biases.  For each layer l:
 *     a = rmsnorm(h);  qkv = Wqkv_l a;            (q, k, v rows in that order)
 *     h = h + Wo_l gqa(v);                        (position 0: head i reads
 *                                                  value head i / (n_heads/n_kv_heads))
 *     a = rmsnorm(h);  s = silu(g) * u, [g; u] = Wgu_l a;
 *     h = h + Wdown_l s;
 * then logits = Wlm rmsnorm(h) and *next_token = the lowest index of the
 * largest logit.  Each projection's output agrees with the exact product of
 * its own fp32 input within 2e-5 * sum_k |w_k a_k| + 1e-6 (plus a few ulps
 * of the RMS scale); repeated runs are bitwise identical.
 *
 * The launch keeps one workgroup resident on every compute unit for the whole
 * step and hands activations between workgroups through the workspace; all of
 * them must be resident at once, so nothing else may occupy the device while
 * a step runs.  Most hand-offs stay inside one XCD (its L2 is shared); that
 * needs the members b, b + 8, b + 16, ... of each of the 8 groups on one XCD,
 * which q8_0_chain_prepare checks with a probe launch of the same shape
 * (otherwise it sets Q8_CHAIN_COHERENT in the plan: every hand-off then goes
 * through device-scope stores, slower but independent of placement).
 *
 * Every wait in the kernel is bounded (plan.spin_limit polling rounds).  A
 * wait that expires marks the step invalid: *next_token is set to -1 (never
 * a valid index) and bit 1 of the status word is set; the kernel still runs
 * to completion.  A step with no expired wait writes a valid token, whatever
 * earlier steps did.  Concurrent work that keeps workgroups from being
 * resident therefore shows up as -1 tokens, never as plausible wrong ones.
 *
 * Limits: hidden, n_heads*head_dim and n_kv_heads*head_dim at most 1024;
 * hidden, n_heads*head_dim and intermediate multiples of 32; intermediate/8
 * rounded up to 16 at most 1024; n_heads % n_kv_heads == 0; head_dim even;
 * the grid (one workgroup per compute unit) a multiple of 8 whose per-
 * workgroup shares fit its 12 computing waves.  Weights: qkv_l
 * ((n_heads + 2 n_kv_heads) head_dim x hidden), wo_l (hidden x
 * n_heads*head_dim) and down_l (hidden x intermediate) in Q8_LAYOUT_ROWS;
 * gate_up_l (2 intermediate x hidden, gate rows first) in
 * Q8_LAYOUT_GATE_UP_PAIRS; lm_head (vocab x hidden) in Q8_LAYOUT_ROWS, or
 * NULL with vocab == 0 (no LM head: the step ends with the last layer). */
typedef struct {
  int32_t n_layers;
  int32_t hidden;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t intermediate;
  int32_t vocab;
  float eps;                    /* RMSNorm epsilon */
  const q8_0_weights* qkv;      /* host arrays of n_layers descriptors each */
  const q8_0_weights* wo;
  const q8_0_weights* gate_up;
  const q8_0_weights* down;
  const q8_0_weights* lm_head;  /* one descriptor, or NULL */
} q8_0_chain_desc;

/* Filled by q8_0_chain_prepare; passed unchanged to the other chain calls
 * (it holds the launch configuration, so a run needs no device reads).  The
 * caller may set `flags` and `spin_limit` between prepare and run. */
#define Q8_CHAIN_COHERENT 1u  /* flags: every hand-off through device-scope stores */
typedef struct {
  int32_t grid;          /* workgroups of the launch (one per compute unit) */
  int32_t threads;       /* threads per workgroup */
  int32_t lds_bytes;     /* dynamic LDS per workgroup */
  int32_t n_layers;
  int32_t hidden;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t intermediate;
  int32_t vocab;
  float eps;
  uint32_t flags;        /* Q8_CHAIN_COHERENT, set by prepare when workgroup b of a
                            chain-shaped grid does not run on XCD b % groups */
  int64_t ws_bytes;      /* workspace bytes in use */
  int64_t off[4];        /* workspace offsets of layer 0's four activation records */
  int64_t layer_stride;  /* bytes between layers' records */
  int64_t am_off;        /* workspace offset of the per-workgroup argmax partials */
  const void* lm_qs;     /* LM head weights (NULL without LM head) */
  const void* lm_d;
  int32_t len[4];        /* entries of the four records */
  uint32_t spin_limit;   /* polling rounds before a wait gives up (0: 65536) */
  int32_t groups;        /* XCD groups the workgroups are split into (8) */
  int64_t off_v;         /* workspace offset of layer 0's per-group value records */
  int64_t off_p;         /* workspace offset of layer 0's down-projection partials */
  int32_t group_words_v; /* entries between the group copies of a value record */
  int32_t group_words_h; /* entries between the group copies of a hidden-sized record */
} q8_0_chain_plan;

/* Workspace bytes for a chain (0 if the description is invalid). */
size_t q8_0_chain_workspace_bytes(const q8_0_chain_desc* desc);

/* Validates the description and weight pointers, writes the chain's tables
 * into the workspace (device memory, 256-byte aligned, at least
 * q8_0_chain_workspace_bytes), clears its records and fills *plan.  Set-up
 * call: it synchronises `stream` before returning.  The weights must stay
 * allocated, and the workspace dedicated to this chain, while it is used.
 * Errors: Q8_EINVAL, Q8_ENULL, Q8_EALIGN, Q8_EHOSTPTR, Q8_EWORKSPACE,
 * Q8_ELAUNCH. */
int q8_0_chain_prepare(const q8_0_chain_desc* desc, void* workspace, size_t workspace_bytes,
                       q8_0_chain_plan* plan, void* stream);

/* One decode step: one kernel launch on `stream` (capturable).
 *  h_in: device fp32 [hidden], the residual stream entering layer 0.
 *  h_out: device fp32 [hidden] or NULL, the residual stream after the last layer.
 *  logits: device fp32 [vocab]; next_token: device int32 [1] (both ignored
 *  when vocab == 0).  Runs on one workspace must be stream-ordered.
 * Errors: Q8_ENULL, Q8_EALIGN, Q8_EHOSTPTR, Q8_EINVAL, Q8_ELAUNCH. */
int q8_0_chain_run(const q8_0_chain_plan* plan, void* workspace, const float* h_in, float* h_out,
                   float* logits, int32_t* next_token, void* stream);

/* q8_0_chain_run that also records stage timestamps, for profiling.
 * stamps: device int64 [plan->grid][Q8_CHAIN_STAMP_WORDS], written at the end
 * of the step: for workgroup b, word b * Q8_CHAIN_STAMP_WORDS + l *
 * Q8_CHAIN_STAMP_POINTS + k is the 100 MHz s_memrealtime counter at point k
 * of layer l (first Q8_CHAIN_STAMP_LAYERS layers; 0 where a workgroup has no
 * such point):
 *   0 stage A starts, 1 a value/query/key task stored, 2 stage B starts,
 *   3 a wo task stored, 4 stage C starts, 5 / 6 the first / last gate-up task
 *   of the workgroup stored, 7 stage D starts, 8 a down partial stored,
 *   9 the 8 partials of the workgroup's rows received, 10 its h2 rows stored,
 *   11 the next h staged, 12 / 13 the first value/query/key and gate-up
 *   tasks' weights in registers (the stamped instance waits for them there),
 *   14 / 15 the same tasks' dot products done;
 * then Q8_CHAIN_STAMP_KERNEL words: 0 step start, 1 LM head start, 2 LM
 * partial stored, 3 step end.  Results equal those of q8_0_chain_run; the
 * stamps cost a few percent of the step.
 * Errors: as q8_0_chain_run. */
#define Q8_CHAIN_STAMP_LAYERS 32
#define Q8_CHAIN_STAMP_POINTS 16
#define Q8_CHAIN_STAMP_KERNEL 4
#define Q8_CHAIN_STAMP_WORDS (Q8_CHAIN_STAMP_LAYERS * Q8_CHAIN_STAMP_POINTS + Q8_CHAIN_STAMP_KERNEL)
int q8_0_chain_run_stamped(const q8_0_chain_plan* plan, void* workspace, const float* h_in,
                           float* h_out, float* logits, int32_t* next_token, int64_t* stamps,
                           void* stream);

/* Copies one activation vector of layer `layer` from the last run to dst
 * (device fp32): Q8_CHAIN_QKV ([q; k; v], (n_heads + 2 n_kv_heads) head_dim),
 * Q8_CHAIN_H_ATTN (h after the attention residual, hidden), Q8_CHAIN_SWIGLU
 * (s, intermediate), Q8_CHAIN_H_OUT (h after the MLP residual, hidden).
 * Errors: Q8_EINVAL, Q8_ENULL, Q8_EHOSTPTR, Q8_ELAUNCH. */
#define Q8_CHAIN_QKV 0
#define Q8_CHAIN_H_ATTN 1
#define Q8_CHAIN_SWIGLU 2
#define Q8_CHAIN_H_OUT 3
int q8_0_chain_read(const q8_0_chain_plan* plan, const void* workspace, int32_t layer,
                    int32_t which, float* dst, void* stream);

/* Copies the chain's status word to *dev_status (device int32): 0, or bit 1
 * if a wait for another workgroup's data expired in some run since prepare
 * (sticky; each step's own validity is in its next_token).
 * Errors: Q8_ENULL, Q8_EHOSTPTR, Q8_ELAUNCH. */
int q8_0_chain_status(const void* workspace, int32_t* dev_status, void* stream);

/* ---- measurement utility ------------------------------------------------------
 * The on-box reference for achievable HBM read bandwidth: reads the first
 * `bytes` (rounded down to 16) of device buffer buf (16-byte aligned) with
 * 16-byte non-temporal loads, the GEMV's weight-streaming instruction; each
 * of `grid` workgroups (1 .. 2^20) of 256 threads reads one contiguous chunk
 * and writes the XOR of every 32-bit word it read to out[workgroup] (device
 * uint32 [grid]), so no read can be dropped; the XOR of all grid words is the
 * XOR of the buffer's words.  Bandwidth = bytes / kernel time.  Not part of
 * the GEMV path.  bytes == 0 (or < 16) still writes grid zero words.
 * Errors: Q8_EINVAL, Q8_ENULL, Q8_EALIGN, Q8_EHOSTPTR, Q8_ELAUNCH. */
int q8_stream_read(const void* buf, int64_t bytes, uint32_t* out, int32_t grid, void* stream);

/* ---- workspace sizes --------------------------------------------------------
 * op Q8_OP_GEMV: (M, K, N) of q8_0_gemv.
 * op Q8_OP_GEMV_FUSED: (M, K, epilogue flags in N) of q8_0_gemv_fused.
 * op Q8_OP_GEMV_ARGMAX: (M, K, N) of q8_0_gemv_argmax.
 * op Q8_OP_Q4K_GEMV: (M, K, N) of q4k_gemv.
 * op Q8_OP_Q6K_GEMV: (M, K, N) of q6k_gemv.
 * op Q8_OP_Q5K_GEMV: (M, K, N) of q5k_gemv.
 * op Q8_OP_ARGMAX: (n, 0, 0).
 * op Q8_OP_MOE_SCATTER / Q8_OP_MOE_COMBINE: (M, K, n_slots) with the
 *   shared expert's shape in (M2, K2) (0, 0 for none) and mode flags in flags.
 * Returns the byte count, or 0 when none is needed or the shape is invalid. */
#define Q8_OP_GEMV 1
#define Q8_OP_GEMV_FUSED 2
#define Q8_OP_ARGMAX 3
#define Q8_OP_MOE_SCATTER 4
#define Q8_OP_MOE_COMBINE 5
#define Q8_OP_GEMV_ARGMAX 6
#define Q8_OP_Q4K_GEMV 7
#define Q8_OP_Q6K_GEMV 8
#define Q8_OP_Q5K_GEMV 9
size_t q8_0_workspace_bytes(int32_t op, int64_t M, int64_t K, int64_t N, int64_t M2, int64_t K2,
                            int32_t flags);

/* Launch plan the library picks for a GEMV of this shape (for reports):
 * out[0] = workgroups, out[1] = waves per workgroup, out[2] = K-splits per
 * 64-row tile, out[3] = workgroups per tile.  Returns Q8_OK or Q8_EINVAL. */
int q8_0_gemv_plan(int64_t M, int64_t K, int64_t N, int32_t epilogue, int32_t out[4]);

/* Human-readable name of a status code (static string, never NULL). */
const char* q8_0_strerror(int status);

/* Library version as major*10000 + minor*100 + patch. */
int q8_0_version(void);

#ifdef __cplusplus
}
#endif
#endif /* Q8GEMV_H */
