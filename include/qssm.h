/*
 * qssm.h — C ABI of libqssm, the quantized state-space scan library for AMD MI355X (gfx950).
 *
 * What the library computes (sources, by page title and section):
 *  - "Quamba2: A Robust and Scalable Post-training Quantization Framework for Selective State
 *    Space Models", abstract and method summary (offline steps 1-4): 8-bit quantization of the
 *    input x of the linear recurrence with per-group scales over sorted and clustered channels,
 *    per-state-group quantization of the input-dependent B and C, weights rearranged offline in
 *    cluster order so the SSM output is unchanged; W8A8 for Mamba1 and Mamba2 backbones,
 *    prefill and generation.
 *  - "Quantizing Small-Scale State-Space Models for Edge AI", abstract: quantized S4D layer;
 *    the state matrix A and the internal state are the sensitive parts; per-component precision.
 *  - SSDi8 (post-training quantization for the Mamba-2 structured state-space duality), abstract:
 *    a persistent INT8 path through the chunked SSD form, with activations quantized at
 *    cost-effective points.
 *  - Quamba-SE soft-edge quantization (blog post), sections 2.1, 2.2 and 4.1: a three-scale
 *    8-bit code (scale/4, scale, scale*4) with the mode in the top bits.
 *
 * The recurrence, per channel d and state n:
 *     h_t = exp(delta_t * A) * h_{t-1} + delta_t * B_t * x_t,     y_t = sum_n C_t * h_t + D * x_t
 * with int8 x, B, C (dequantized as scale * code), fp32 delta/A/D, a higher-precision state and
 * a dequantized (fp32 or fp16) output.
 *
 * Conventions shared by every entry point:
 *  - Tensor arguments are DEVICE pointers owned by the caller, unless the comment says "host".
 *    Shapes are row-major (the last index is contiguous). Outputs must not alias inputs.
 *  - Calls validate their arguments on the host first. On a bad argument they return a
 *    non-zero qssm_status, launch nothing, and leave a message for qssm_last_error().
 *  - Launches are asynchronous on the given stream; nothing synchronizes. A device fault shows up
 *    at the caller's next synchronization. A failed launch returns QSSM_ERR_DEVICE.
 *  - No C++ exception ever crosses this boundary.
 *  - The library allocates no device memory at run time. Entry points that need scratch take a
 *    caller-provided workspace whose size a *_workspace_size call reports; the one exception,
 *    qssm_scan_w8a8_noalloc, uses a fixed-size array that is part of the library's device code.
 *  - Group maps hold indices below the group count; a larger index is read as the last group.
 *
 * Quantization rule used everywhere (int8 codes, bit-exact):
 *     q = clamp(RNE(v / s), -128, 127)
 *  where v / s is the exact rational quotient of the fp32 values and RNE rounds half to even.
 *  NaN encodes as 0; +-Inf saturate. A scale s is valid when it is finite and
 *  2^-100 <= s <= 2^100; every code of a group whose scale is not valid is 0, and the scans
 *  take every value of such a group (x, B or C) as 0.
 */
#ifndef QSSM_H
#define QSSM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QSSM_VERSION 180 /* 1.8.0: instruction-rate probes */

typedef int32_t qssm_status;
enum {
  QSSM_OK = 0,
  QSSM_ERR_INVALID_ARG = 1, /* null required pointer, bad shape, bad enum value */
  QSSM_ERR_UNSUPPORTED = 2, /* a valid request this library version does not implement */
  QSSM_ERR_WORKSPACE = 3,   /* workspace pointer missing or smaller than *_workspace_size */
  QSSM_ERR_DEVICE = 4       /* the HIP runtime reported an error at launch */
};

/* Element types of optional-precision buffers. */
enum { QSSM_F32 = 0, QSSM_F16 = 1, QSSM_I16 = 2, QSSM_I8 = 3 };

/* Encodings of the scan input x. */
enum {
  QSSM_X_INT8 = 0,    /* int8 code, value = s[g] * q */
  QSSM_X_SOFTEDGE = 1, /* three-scale soft-edge byte, mode ratio 4, see qssm_softedge_encode */
  QSSM_X_SOFTEDGE2 = 2 /* the same byte with the shift-only mode ratio 2 */
};

/* ---------------------------------------------------------------------------------------------
 * a1. Per-group int8 quantization of the scan input x over sorted, clustered channel groups.
 * Quamba2, abstract and method steps 1-2 (sort and cluster x channels; per-group scales).
 *
 * x is viewed as [outer, C, inner] fp32. Output channel c takes input channel perm[c]
 * (perm == NULL: identity) and belongs to group group_of[c] < G:
 *     q[o, c, i] = quant(x[o, perm[c], i], scales[group_of[c]])
 * compute_scales == 0: scales[G] is an input (static, calibrated offline).
 * compute_scales != 0: scales[G] is an output, computed first on the device from the tensor
 *     itself: scales[g] = fl32(absmax_g / 127) with absmax_g the largest finite |x| of group g
 *     (after the permutation); a group with absmax 0 gets scale 1; the result is clamped to
 *     [2^-100, 2^100].
 * q: int8 [outer, C, inner]. 1 <= G <= 256, perm must be a permutation of 0..C-1.
 * Empty tensors (outer, C or inner == 0) are valid and launch nothing (compute_scales then writes
 * scale 1 for every group).
 */
qssm_status qssm_quant_group_x(const float* x, int64_t outer, int64_t C, int64_t inner,
                               const int32_t* perm, const uint8_t* group_of, int32_t G,
                               float* scales, int32_t compute_scales, int8_t* q,
                               hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * a2. Per-state-group int8 quantization of the input-dependent B or C.
 * Quamba2, abstract and method step 3 (per-state-group quantization of B and C).
 *
 * bc is viewed as [outer, Gbc, N, inner] fp32 (Gbc = number of B/C groups of the model, N = state
 * size). State n of B/C group g uses scale scales[g * (N / gs) + n / gs]; N % gs == 0.
 * compute_scales has the same meaning as in qssm_quant_group_x, one scale per (g, state group).
 * q: int8 [outer, Gbc, N, inner].
 */
qssm_status qssm_quant_state_group_BC(const float* bc, int64_t outer, int32_t Gbc, int32_t N,
                                      int64_t inner, int32_t gs, float* scales,
                                      int32_t compute_scales, int8_t* q, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * a3. Soft-edge three-scale 8-bit code. Quamba-SE blog, section 2.1 (three modes: scale/4 for
 * |v| < L, scale for the middle, scale*4 for |v| > H), section 2.2 (classifier and byte layout:
 * 0xxxxxxx standard, 10xxxxxx small, 11xxxxxx large), section 4.1 (thresholds; on small hardware
 * scale/2 and scale*2, one shift instead of a multiplier).
 *
 * form selects the mode ratio m: QSSM_X_SOFTEDGE (m = 4) or QSSM_X_SOFTEDGE2 (m = 2); nothing
 * else depends on it. Per group g with base scale s = s[g] and thresholds L = L[g], H = H[g]:
 *   small    (|v| < L and not |v| > H): q = clamp(RNE(v / (s/m)), -32, 31), byte = 0x80 | (q & 0x3F)
 *   large    (|v| > H and not |v| < L): q = clamp(RNE(v / (s*m)), -32, 31), byte = 0xC0 | (q & 0x3F)
 *   standard (otherwise):               q = clamp(RNE(v / s),     -64, 63), byte = q & 0x7F
 * NaN encodes as 0x00; +-Inf fall in the large mode and saturate (0xDF / 0xE0). A group whose
 * base scale is not valid (see above) encodes every value as 0x00.
 * x / out: fp32 [outer, C, inner]; code: uint8 [outer, C, inner]; perm and group_of as in a1.
 * Decode: 0xxxxxxx -> sext7 * s, 10xxxxxx -> sext6 * (s/m), 11xxxxxx -> sext6 * (s*m), each one
 * fp32 multiply (correctly rounded). A group with an invalid scale decodes to 0.
 */
qssm_status qssm_softedge_encode(const float* x, int64_t outer, int64_t C, int64_t inner,
                                 const int32_t* perm, const uint8_t* group_of, int32_t G,
                                 const float* s, const float* L, const float* H, int32_t form,
                                 uint8_t* code, hipStream_t stream);
qssm_status qssm_softedge_decode(const uint8_t* code, int64_t outer, int64_t C, int64_t inner,
                                 const uint8_t* group_of, int32_t G, const float* s, int32_t form,
                                 float* out, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * f3. On-device soft-edge threshold tracking. Quamba-SE blog, section 4.1: L at the 5th and H at
 * the 99.9th percentile of the activations, followed over mini-batches by an exponential moving
 * average with factor alpha (0.1 there).
 *
 * For each group g, over the values of x [outer, C, inner] (device fp32) whose output channel c
 * (reading input channel perm[c]; perm NULL = identity) has group_of[c] == g:
 *   L_new = P5(|v|), H_new = P99.9(|v|), linear interpolation between order statistics:
 *     vi = (n - 1)*q with q = p/100 (fp64), k = floor(vi), t = vi - k,
 *     P = a + (b - a)*t if t < 1/2 else b - (b - a)*(1 - t), a, b = the k-th and (k+1)-th smallest
 *     (P = the largest when vi >= n - 1), every step rounded in fp64 as written;
 *   ema_valid != 0: L = alpha*L_new + (1 - alpha)*L_prev (same for H), else L = L_new;
 *   ema_state[2g], ema_state[2g+1] (device fp64, in/out): the previous and then the new (L, H);
 *   L[g], H[g] = fl32 of them; s[g] = fl32(H[g] / 63) (1 when H[g] is 0): the arguments
 *   qssm_softedge_encode reads, so an encode queued after this call uses the updated thresholds.
 * These are the numbers qssm_calib_softedge computes on the host from the same values.
 * A group with no values keeps its ema_state (0, 0 when ema_valid == 0) and gets L, H, s from it.
 * Values must be finite; a NaN or Inf yields unspecified thresholds (no fault).
 * 1 <= G <= 32; 0 <= alpha <= 1. Group indices >= G count as the last group.
 * Workspace: qssm_softedge_track_workspace_size(G) bytes of device memory (histograms and
 * selection state; the call clears what it uses). No synchronization: four counting passes over x
 * and five small selection kernels on the stream.
 */
size_t qssm_softedge_track_workspace_size(int32_t G);
qssm_status qssm_softedge_track(const float* x, int64_t outer, int64_t C, int64_t inner,
                                const int32_t* perm, const uint8_t* group_of, int32_t G,
                                double alpha, int32_t ema_valid, double* ema_state, float* s,
                                float* L, float* H, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * a4-a7. Mamba1 selective scan with int8 (or soft-edge) x and int8 B, C (W8A8 recurrence).
 * Quamba2, abstract (8-bit linear recurrence for the Mamba1 backbone).
 *
 * Layouts: x, delta, y [B, D, L]; A [D, N]; Bq, Cq [B, Gbc, N, L] (channel d uses B/C group
 * d / (D / Gbc)); Dskip [D]; h0, h_last [B, D, N] fp32.
 * Per (b, d, n), t = 0 .. L-1, with xh = dequantized x, Bh/Ch = dequantized B/C:
 *     h = exp(delta * A[d,n]) * h + delta * Bh[n,t] * xh,   y[t] = sum_n Ch[n,t] * h + Dskip[d] * xh
 * h starts from h0 (zero when NULL); h_last receives the final state when not NULL.
 * seqlen == 0 is valid: x, delta, Bq, Cq and y are then not accessed (they may be NULL) and
 * h_last receives h0 (or zeros).
 * The state and all arithmetic are fp32. y is fp32 or fp16 (y_dtype), or int8 codes for the
 * next W8A8 module (QSSM_I8; SSDi8, abstract: a persistent int8 path, and an error-correction
 * term from per-channel error statistics):
 *     y_code[b,d,t] = clamp(RNE(v / s), -128, 127),  v = fl32(y[b,d,t] + y_bias[d]),
 *     s = y_scales[y_group_of[d]]
 * by the quantization rule above (exact quotient; an invalid scale gives codes 0), where y[b,d,t]
 * is the fp32 value the QSSM_F32 output would hold. y_bias (NULL = no correction) is the
 * calibrated correction term, e.g. from qssm_calib_channel_error_mean. The y_* fields are read
 * only for QSSM_I8.
 * bc_code selects how Bq and Cq are coded: QSSM_X_INT8 (int8 codes, value = scale * q) or a
 * soft-edge form (QSSM_X_SOFTEDGE or QSSM_X_SOFTEDGE2: the bytes of qssm_softedge_encode, with
 * B_scales / C_scales as the state groups' base scales; the code of the Quamba-SE blog, sections
 * 2.1-2.2, applied to the input-dependent B and C as well as to x). Bq and Cq then hold those
 * bytes; their thresholds only matter to the encoder.
 * Time windows (the scan's second form, an associative scan over time blocks with a carry
 * between blocks): the recurrence h_t = a_t h_{t-1} + u_t composes over a block of steps into
 * h_end = (prod a_t) h_start + (the block's state from h_start = 0). With K windows the library
 * runs every window from 0 in parallel, then runs every window again from its entering state,
 * which it folds from h0 and the earlier windows' end states in order
 * (h_in[k + 1] = exp(A * sum of delta over window k) h_in[k] + end[k], per chain), and writes y. This doubles the recurrence work for
 * K-fold parallelism over time; time_blocks = 0 uses it when batch x channel blocks of 64 are
 * fewer than 128 (small layers), choosing K for about 256 workgroups. K <= 16, and K <= the
 * number of 16-step blocks of the sequence. The int8 output (QSSM_I8)
 * always uses one chain. Results agree with the chain form to fp32 rounding.
 * Workspace: qssm_scan_workspace_size bytes (dequantized B and C staging, and with windows the
 * carries: K * B * D * (N + 1) floats).
 */
typedef struct qssm_scan_args {
  int64_t batch, seqlen, dim, dstate; /* B, L, D, N */
  int32_t x_code;                     /* QSSM_X_INT8, QSSM_X_SOFTEDGE or QSSM_X_SOFTEDGE2 */
  int32_t x_groups;                   /* G, 1..256 */
  const void* x;                      /* int8 or soft-edge uint8 codes [B, D, L] */
  const uint8_t* x_group_of;          /* [D] group of each channel */
  const float* x_scales;              /* [G] scale (soft-edge: base scale) */
  const float* delta;                 /* [B, D, L] fp32 */
  const float* A;                     /* [D, N] fp32 */
  int32_t bc_groups;                  /* Gbc, D % Gbc == 0 */
  int32_t bc_group_size;              /* gs, N % gs == 0 */
  const int8_t* Bq;                   /* [B, Gbc, N, L] */
  const int8_t* Cq;                   /* [B, Gbc, N, L] */
  const float* B_scales;              /* [Gbc * N / gs] */
  const float* C_scales;              /* [Gbc * N / gs] */
  const float* Dskip;                 /* [D] or NULL */
  const float* h0;                    /* [B, D, N] or NULL */
  void* y;                            /* [B, D, L], y_dtype */
  int32_t y_dtype;                    /* QSSM_F32, QSSM_F16 or QSSM_I8 */
  float* h_last;                      /* [B, D, N] or NULL */
  int32_t y_groups;                   /* QSSM_I8: Gy, 1..256 */
  const uint8_t* y_group_of;          /* QSSM_I8: [D] output group (< y_groups) of each channel */
  const float* y_scales;              /* QSSM_I8: [Gy] static output scales */
  const float* y_bias;                /* QSSM_I8: [D] correction added before quantizing, or NULL */
  int32_t bc_code;                    /* QSSM_X_INT8, QSSM_X_SOFTEDGE or QSSM_X_SOFTEDGE2 */
  int32_t time_blocks;                /* 0: library choice, 1: one chain per (b, d, n) in time
                                         order, K >= 2: K time windows (see above) */
} qssm_scan_args;

size_t qssm_scan_workspace_size(const qssm_scan_args* a);
qssm_status qssm_scan_w8a8(const qssm_scan_args* a, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* Allocation-free variant of qssm_scan_w8a8, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. Same arguments
 * (minus the workspace), same kernels, same results. The B/C staging goes to a library-owned
 * device array of QSSM_SCAN_SCRATCH_BYTES bytes, one per GPU, which exists from the library's
 * loading on that GPU until the process ends. A call whose staging needs more
 * (qssm_scan_workspace_size(a) - 256 bytes) returns QSSM_ERR_UNSUPPORTED and launches nothing.
 * All calls on one GPU share its array and it keeps the last call's contents (every call rewrites
 * what it reads): calls that overlap in time on one GPU (other streams, other host threads) race,
 * so the caller serializes them. The first call on each device looks up the array's address
 * (thread-safe). */
#define QSSM_SCAN_SCRATCH_BYTES (32u << 20)
qssm_status qssm_scan_w8a8_noalloc(const qssm_scan_args* a, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * a5-a7 (S4D form). Diagonal LTI scan with int8 parameters and input.
 * "Quantizing Small-Scale State-Space Models for Edge AI", abstract (S4D under PTQ; A and the
 * state are sensitive; heterogeneous per-component precision).
 *
 * Input: when wq != NULL, uq is [B, L] int8 (a scalar sequence) lifted to H channels by int8
 *   weights:  u[b,h,t] = (u_scale[0] * w_scale[0]) * (uq[b,t] * wq[h]);
 *   when wq == NULL, uq is [B, H, L] and u[b,h,t] = u_scale[h] * uq[b,h,t].
 * Parameters, per channel h and state n (int8 [H, N] planes, one scale per channel and plane):
 *   Ah = A_re_s[h]*A_re[h,n] + i*A_im_s[h]*A_im[h,n], Bh and Ch likewise; dt = exp(log_dt[h]).
 * Zero-order hold: Abar = exp(dt*Ah), Bbar = (Abar - 1) / Ah * Bh  (dt * Bh when Ah == 0).
 * Recurrence: h_t = Abar * h_{t-1} + Bbar * u_t (complex), y_t = Re(sum_n Ch * h_t) + Dskip[h]*u_t.
 * State: QSSM_F32 keeps complex fp32; QSSM_I16 rounds each real and imaginary part to
 *   state_scale[h] * clamp(RNE(part / state_scale[h]), -32768, 32767) after every step.
 * h0 / h_last: [B, H, N] complex, interleaved (re, im): float pairs (F32) or int16 code pairs (I16).
 * y: fp32 [B, H, L]. seqlen == 0 is valid: uq and y are then not accessed (they may be NULL) and
 * h_last receives h0 (or zeros).
 */
typedef struct qssm_s4d_args {
  int64_t batch, seqlen, channels, dstate; /* B, L, H, N */
  const int8_t* uq;
  const float* u_scale;
  const int8_t* wq;
  const float* w_scale;
  const int8_t *A_re, *A_im, *B_re, *B_im, *C_re, *C_im; /* [H, N] */
  const float *A_re_s, *A_im_s, *B_re_s, *B_im_s, *C_re_s, *C_im_s; /* [H] */
  const float* log_dt;      /* [H] */
  const float* Dskip;       /* [H] or NULL */
  int32_t state_dtype;      /* QSSM_F32 or QSSM_I16 */
  const float* state_scale; /* [H], required for QSSM_I16 */
  const void* h0;           /* or NULL */
  float* y;                 /* [B, H, L] */
  void* h_last;             /* or NULL */
} qssm_s4d_args;

qssm_status qssm_s4d_scan(const qssm_s4d_args* a, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * a8-a13. Mamba2 SSD chunked form with an int8 path.
 * SSDi8 abstract (persistent INT8 path through SSD; requantization at cost-effective points);
 * Quamba2 abstract (W8A8 for the Mamba2 backbone).
 *
 * Layouts: xq, y [B, L, nh, P]; delta [B, L, nh]; A, Dskip [nh]; Bq, Cq [B, L, Gbc, N] (head h
 * uses group h / (nh / Gbc)); h0, h_last [B, nh, P, N] fp32. x channel (h, p) has group
 * x_group_of[h * P + p].
 * The result equals the sequential recurrence with A[h] shared by all (p, n) of head h, computed
 * per chunk of `chunk` steps (chunks start at t = 0, the last may be partial):
 *   cum_i = sum_{k<=i} delta_k * A[h];  G = Ch Bh^T (int8 MFMA, int32 accumulation per state group);
 *   Y_intra = (G o exp(cum_i - cum_j) [j<=i] o delta_j) . xh  (fp16 operands, fp32 accumulate);
 *   chunk state S = sum_j w_j xh_j Bh_j^T with w_j = delta_j exp(cum_last - cum_j), contracted over
 *   time on MFMA: state_mma == QSSM_MMA_F16 uses fp16 operands fp16(w_j * qx) and the exact B codes
 *   (fp32 accumulate); state_mma == QSSM_MMA_I8 requantizes the weighted x per (b, chunk, head) to
 *   r = sat8(RNE(qx * w_j / w_max)) and runs int8 MFMA with int32 accumulate (faster operands, but
 *   the rounding of r is a floating-point decision inside the contraction);
 *   inter-chunk state passing in fp32;  Y_inter = exp(cum_i) * Ch . H_prev^T;
 *   y = Y_intra + Y_inter + Dskip * xh.
 * intra_mma == QSSM_MMA_I8 runs Y_intra on int8 MFMA (the SSDi8 persistent int8 path through the
 *   intra-chunk product): row i of the weights W[i, j] = G[i, j] exp(cum_i - cum_j) delta_j
 *   (j <= i) is requantized with its own scale, m_i = max_j |W[i, j]| (fp32),
 *   r[i, j] = clamp(rint(W[i, j] * 127 / m_i), -127, 127) (0 when m_i = 0), and
 *   Y_intra[i, p] = (m_i / 127) * sx[p] * sum_j r[i, j] * qx[j, p] (int32 accumulate). The codes
 *   are floating-point decisions inside the contraction (fp32 W); the requantization error per
 *   output is at most (m_i / 254) sum_j |xh_j|.
 * y is fp32 or fp16 (y_dtype), or int8 codes for the next W8A8 module (QSSM_I8; SSDi8, abstract:
 * a persistent int8 path and an error-correction term from per-channel error statistics):
 *   y_code[b,t,h,p] = clamp(RNE(v / s), -128, 127),  v = fl32(y[b,t,h,p] + y_bias[h*P + p]),
 *   s = y_scales[y_group_of[h*P + p]]
 * by the quantization rule above, where y is the fp32 value the QSSM_F32 output would hold. The y_*
 * fields are read only for QSSM_I8.
 * Requires chunk == 256, P == 64, N == 128, gs == 16 in this version (else QSSM_ERR_UNSUPPORTED),
 * and Lc * nh * P < 2^31 and Lc * ngroups * N < 2^31 with Lc = seqlen rounded up to a multiple of
 * 256, plus 256 (one sequence's codes are addressed with 32-bit offsets; else QSSM_ERR_UNSUPPORTED).
 * seqlen == 0 is valid: xq, delta, Bq, Cq and y are then not accessed (they may be NULL) and
 * h_last receives h0 (or zeros).
 */
enum { QSSM_MMA_F16 = 0, QSSM_MMA_I8 = 1 };

typedef struct qssm_ssd_args {
  int64_t batch, seqlen, nheads, headdim, dstate; /* B, L, nh, P, N */
  int32_t ngroups;                                /* Gbc, nh % Gbc == 0 */
  int32_t chunk;                                  /* Q */
  int32_t x_groups;                               /* G, 1..256 */
  const int8_t* xq;                               /* [B, L, nh, P] */
  const uint8_t* x_group_of;                      /* [nh * P] */
  const float* x_scales;                          /* [G] */
  const float* delta;                             /* [B, L, nh] */
  const float* A;                                 /* [nh] */
  const float* Dskip;                             /* [nh] or NULL */
  int32_t bc_group_size;                          /* gs */
  const int8_t* Bq;                               /* [B, L, Gbc, N] */
  const int8_t* Cq;                               /* [B, L, Gbc, N] */
  const float* B_scales;                          /* [Gbc * N / gs] */
  const float* C_scales;                          /* [Gbc * N / gs] */
  const float* h0;                                /* [B, nh, P, N] or NULL */
  void* y;                                        /* [B, L, nh, P], y_dtype */
  int32_t y_dtype;                                /* QSSM_F32, QSSM_F16 or QSSM_I8 */
  float* h_last;                                  /* [B, nh, P, N] or NULL */
  int32_t fused;                                  /* reserved, must be 0 */
  int32_t state_mma;                              /* QSSM_MMA_F16 (default) or QSSM_MMA_I8 */
  int32_t y_groups;                               /* QSSM_I8: Gy, 1..256 */
  const uint8_t* y_group_of;                      /* QSSM_I8: [nh * P] output group of each channel */
  const float* y_scales;                          /* QSSM_I8: [Gy] static output scales */
  const float* y_bias;                            /* QSSM_I8: [nh * P] correction term, or NULL */
  int32_t intra_mma;                              /* QSSM_MMA_F16 (default) or QSSM_MMA_I8 */
} qssm_ssd_args;

size_t qssm_ssd_workspace_size(const qssm_ssd_args* a);
qssm_status qssm_ssd_chunk_int8(const qssm_ssd_args* a, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * a14. Fused decode state update (one new token per sequence), Mamba2-shaped.
 * Quamba2, abstract (W8A8 generation stage).
 *
 * Per call, with static scales: x [B, nh, P], B and C [B, Gbc, N] fp32 are quantized with the a1
 * and a2 rules (x channel (h, p) in group x_group_of[h*P + p]; B/C state n of group g in state
 * group g * (N/gs) + n/gs), then for every (b, h, p, n), g = h / (nh / Gbc):
 *     dA = exp(delta[b,h] * A[h]);  state = dA * state + delta[b,h] * xh[p] * Bh[n]
 *     y[b,h,p] = sum_n Ch[n] * state + Dskip[h] * xh[p]
 * state [B, nh, P, N] is read and written in place, fp32 or fp16 (state_dtype; fp16 is rounded
 * to nearest even on store, arithmetic is fp32). y: fp32 [B, nh, P], or int8 codes for the next
 * W8A8 module (y_dtype QSSM_I8; SSDi8, abstract: persistent int8 path, per-channel error
 * correction): y_code = clamp(RNE(fl32(y + y_bias[h*P + p]) / y_scales[y_group_of[h*P + p]]),
 * -128, 127) by the quantization rule above.
 * xq_out [B, nh, P], Bq_out / Cq_out [B, Gbc, N] receive the codes when not NULL.
 * Supported: N = 4 * 2^k with 4 <= N <= 256 (N >= 8 for an fp16 state), (P rounded up to a
 * multiple of 4, + 2N) * 4 bytes <= 64 KiB; state 16-byte aligned. Other shapes return
 * QSSM_ERR_UNSUPPORTED.
 */
typedef struct qssm_update_args {
  int64_t batch, nheads, headdim, dstate; /* B, nh, P, N */
  int32_t ngroups;                        /* Gbc */
  int32_t x_groups;                       /* G */
  const float* x;                         /* [B, nh, P] */
  const uint8_t* x_group_of;              /* [nh * P] */
  const float* x_scales;                  /* [G] */
  const float* B;                         /* [B, Gbc, N] */
  const float* C;                         /* [B, Gbc, N] */
  int32_t bc_group_size;                  /* gs */
  const float* B_scales;                  /* [Gbc * N / gs] */
  const float* C_scales;                  /* [Gbc * N / gs] */
  const float* delta;                     /* [B, nh] */
  const float* A;                         /* [nh] */
  const float* Dskip;                     /* [nh] or NULL */
  int32_t state_dtype;                    /* QSSM_F32 or QSSM_F16 */
  void* state;                            /* [B, nh, P, N] in/out */
  void* y;                                /* [B, nh, P], fp32 or int8 codes (y_dtype) */
  int8_t* xq_out;                         /* [B, nh, P] or NULL */
  int8_t* Bq_out;                         /* [B, Gbc, N] or NULL */
  int8_t* Cq_out;                         /* [B, Gbc, N] or NULL */
  int32_t y_dtype;                        /* QSSM_F32 (0, the default) or QSSM_I8 */
  int32_t y_groups;                       /* QSSM_I8: Gy, 1..256 */
  const uint8_t* y_group_of;              /* QSSM_I8: [nh * P] output group of each channel */
  const float* y_scales;                  /* QSSM_I8: [Gy] static output scales */
  const float* y_bias;                    /* QSSM_I8: [nh * P] correction term, or NULL */
} qssm_update_args;

qssm_status qssm_state_update(const qssm_update_args* a, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * W4A8 linear layer: 4-bit weights x int8 activations on int8 MFMA with int32 accumulation.
 * Quamba2, abstract (W4A8 for large-batch decoding: the in and out projections around the
 * recurrence).
 *   y[m, n] = bias[n] + sum_g (sa * sw[n, g]) * sum_{k in group g} qa[m, k] * qw[n, k]
 * a: int8 activation codes [M, K] (row-major) with one scale a_scale[0] (device; an invalid scale
 *    gives y = bias); w: packed 4-bit codes [N, K / 2] as written by qssm_quant_w4 (each run of 8
 *    input channels k0 .. k0 + 7 in 4 bytes, byte b = code k0 + b in the low nibble and k0 + 4 + b
 *    in the high nibble, two's complement); w_scales [N, K / group] fp32 (a scale outside the valid
 *    range gives that group 0); bias [N] fp32 or NULL; y [M, N] fp32 or fp16 (y_dtype).
 * Requires K a positive multiple of 64, group a multiple of 64 dividing K (group == K: one scale per
 * output channel), group <= 131072; a and w 16-byte aligned. Each group's integer sum is exact
 * (int32) and scaled once in fp32. */
typedef struct qssm_gemm_args {
  int64_t M, N, K;
  int32_t group;
  int32_t y_dtype;          /* QSSM_F32 or QSSM_F16 */
  const int8_t* a;          /* [M, K] */
  const float* a_scale;     /* [1] */
  const uint8_t* w;         /* [N, K / 2] packed */
  const float* w_scales;    /* [N, K / group] */
  const float* bias;        /* [N] or NULL */
  void* y;                  /* [M, N] */
} qssm_gemm_args;

qssm_status qssm_gemm_w4a8(const qssm_gemm_args* a, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Host-side offline calibration (CPU only; every pointer below is a HOST pointer).
 * Quamba2, method steps 1-2 (offline activation statistics; sort and cluster the x channels);
 * Quamba-SE, section 4.1 (L at the 5th and H at the 99.9th percentile, EMA with alpha = 0.1).
 */

/* absmax_out[c] = largest finite |x[o, c, i]| over o and i of a host tensor [outer, C, inner]. */
qssm_status qssm_calib_channel_absmax(const float* x, int64_t outer, int64_t C, int64_t inner,
                                      float* absmax_out);

/* scales[i] = fl32(absmax[i] / 127); absmax 0 -> 1; clamped to [2^-100, 2^100].
 * absmax values must be finite and >= 0. */
qssm_status qssm_calib_scales(const float* absmax, int64_t n, float* scales);

/* Sort channels by absmax ascending (stable) and split the sorted list into G contiguous groups
 * with the least total within-group squared deviation (exact 1-D k-means by dynamic programming;
 * ties go to the smallest split index). perm_out[c] = source channel of sorted position c;
 * group_of_out[c] = group of sorted position c (ascending with magnitude). 1 <= G <= min(C, 256). */
qssm_status qssm_calib_cluster_channels(const float* absmax, int32_t C, int32_t G,
                                        int32_t* perm_out, uint8_t* group_of_out);

/* Soft-edge thresholds of one group from samples v[n] (finite values):
 *   L_new = P5(|v|), H_new = P99.9(|v|) (linear interpolation between order statistics),
 *   computed in fp64. When ema_state[0..1] holds a previous (L, H) and ema_valid != 0:
 *   L = alpha * L_new + (1 - alpha) * L_prev (same for H), else L = L_new.
 *   ema_state (fp64, in/out) receives the new (L, H); L_out, H_out are fl32 of them;
 *   s_out = fl32(H_out / 63) (so standard codes span [-H, H]); s_out = 1 if H_out is 0. */
qssm_status qssm_calib_softedge(const float* v, int64_t n, double alpha, int32_t ema_valid,
                                double* ema_state, float* s_out, float* L_out, float* H_out);

/* Error-correction term (SSDi8, abstract: per-channel error statistics): for host tensors
 * ref, approx [outer, C, inner] (the unquantized layer's output and the W8A8 path's output on a
 * calibration draw), mean_out[c] = fl32 of the mean over o and i of (ref - approx), accumulated
 * in fp64. Values must be finite; outer * inner >= 1. */
qssm_status qssm_calib_channel_error_mean(const float* ref, const float* approx, int64_t outer,
                                          int64_t C, int64_t inner, float* mean_out);

/* out[g] = largest absmax[c] over the channels c with group_of[c] == g (0 for an empty group), the
 * group absmax from which qssm_calib_scales makes per-group scales. absmax values must be finite
 * and >= 0; group_of[c] < G <= 256. */
qssm_status qssm_calib_group_absmax(const float* absmax, const uint8_t* group_of, int64_t C,
                                    int32_t G, float* out);

/* out[k] = largest of absmax[k * block .. k * block + block - 1] (contiguous state groups of B or C:
 * absmax over the Gbc * N states, block = gs). block must divide n; values finite and >= 0. */
qssm_status qssm_calib_block_absmax(const float* absmax, int64_t n, int32_t block, float* out);

/* Per-channel scale of the int16 S4D state ("Quantizing Small-Scale State-Space Models for Edge
 * AI", abstract: the internal state is a sensitive part), from the quantized parameters alone:
 * for each state n of channel h, with Re A = A_re_s[h] A_re[h,n], B = B_re_s[h] B_re[h,n] +
 * i B_im_s[h] B_im[h,n],
 * dt = exp(log_dt[h]) and |u| <= umax[h], the state obeys |h_t| <= dt |B| e^{max(0, dt Re A)}
 * umax sum_{k < L} |Abar|^k with |Abar| = e^{dt Re A} (the sum is 1 / (1 - |Abar|) at most when
 * |Abar| < 1). out[h] = headroom * max_n(bound) / 32767, clamped to [2^-100, 2^100], so the int16
 * codes of both parts never saturate. Planes [H, N] int8, scales [H]; headroom >= 1. */
qssm_status qssm_calib_s4d_state_scale(int64_t H, int64_t N, int64_t L, const int8_t* A_re,
                                       const float* A_re_s, const int8_t* B_re,
                                       const float* B_re_s, const int8_t* B_im,
                                       const float* B_im_s, const float* log_dt,
                                       const float* umax, double headroom, float* out);

/* Offline 4-bit weight quantization for qssm_gemm_w4a8 (host): for weights w [N, K] fp32,
 * scales[n * (K / group) + g] = fl32(absmax / 7) of the group's finite values (absmax 0 -> 1,
 * clamped to [2^-100, 2^100]), codes clamp(RNE(w / s), -8, 7) by the exact quotient (NaN -> 0,
 * +-Inf saturate), packed into packed [N, K / 2] in the layout qssm_gemm_w4a8 reads. group must be a
 * multiple of 8 dividing K. */
qssm_status qssm_quant_w4(const float* w, int64_t N, int64_t K, int32_t group, float* scales,
                          uint8_t* packed);

/* ---------------------------------------------------------------------------------------------
 * Library information. */
const char* qssm_status_string(qssm_status s);
/* Message of the last failing call on this host thread ("" if none). */
const char* qssm_last_error(void);
int32_t qssm_version(void);
/* sizeof of the argument structs as compiled (0: scan, 1: s4d, 2: ssd, 3: update, 4: gemm), so
 * bindings can check their layout. Returns 0 for an unknown kind. */
size_t qssm_args_size(int32_t kind);

/* ---------------------------------------------------------------------------------------------
 * Measurement support (not part of the method): instruction-rate loops behind the roofline
 * figures. `blocks` workgroups of 256 threads each run `iters` iterations of:
 *   QSSM_PROBE_EXP       8 v_exp_f32 per thread (8 independent chains),
 *   QSSM_PROBE_FMA       8 v_fma_f32 per thread,
 *   QSSM_PROBE_EXP_FMA   8 v_exp_f32 and 8 v_fma_f32 per thread (interleaved, independent),
 *   QSSM_PROBE_MFMA_I8   2 v_mfma_i32_32x32x32_i8 per wave (32768 int8 multiply-adds each),
 *   QSSM_PROBE_MFMA_F16  2 v_mfma_f32_32x32x16_f16 per wave (16384 fp16 multiply-adds each).
 * sink (device, blocks * 256 floats) receives values that keep the loops from being removed.
 * Time the call with events on the stream; rate = operations / time. */
enum { QSSM_PROBE_EXP = 0, QSSM_PROBE_FMA = 1, QSSM_PROBE_EXP_FMA = 2, QSSM_PROBE_MFMA_I8 = 3,
       QSSM_PROBE_MFMA_F16 = 4 };
qssm_status qssm_probe_rate(int32_t kind, int64_t iters, int32_t blocks, float* sink,
                            hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* QSSM_H */
