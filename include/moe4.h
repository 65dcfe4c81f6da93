/*
 * moe4.h - C ABI of the NVFP4-forward / MXFP8-backward MoE expert-layer library
 * for AMD Instinct MI355X (gfx950).
 *
 * What the library computes is the expert-layer recipe reported on the pages
 * about Thinking Machines Lab's "End-to-End 4-Bit Training" post: NVFP4 in the
 * expert layers' forward pass with a dedicated kernel, MXFP8 in the backward
 * pass after a dequantise -> transpose -> requantise step with stochastic
 * rounding (agihunt.info page, "Confirmed"; lhc.media page, paragraphs on
 * NVFP4, on transposition and on stochastic rounding), and Four-Over-Six
 * activation quantisation (agihunt.info page, "Confirmed").
 *
 * Conventions (every entry point):
 *  - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *    allocates no device memory; where scratch is needed the caller passes a
 *    workspace (ws, ws_bytes) sized by the matching *_ws_bytes() query.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Each call
 *    enqueues its kernels on that stream and returns without synchronising.
 *  - Return value: 0 on success, a negative MOE4_E* code on error.  On a
 *    host-side validation error nothing is enqueued; moe4_last_error() returns
 *    a message for the calling thread.  Nothing throws across the ABI.
 *  - Preconditions that need the device's data (monotone offsets, indices in
 *    range, finite inputs) are the caller's; kernels clamp indices so that a
 *    violated precondition gives wrong values, never an out-of-bounds access.
 *    Kernels that clamp a routed row index, and the bounded wait between
 *    workgroups of nvfp4_quant_requant_T, also set a bit in the library's
 *    device-side error word, which moe4_debug_check() reports.
 *  - The library's only device state is that error word (one per device) and
 *    its constant SiLU / SiLU' tables (data of the code object): no call
 *    fills anything at run time, so any call may be the first one on a device
 *    and may be made inside a stream capture.
 *  - Sizes are int64_t; offsets and indices are int32_t device arrays.
 *  - Pointers must be 16-byte aligned.
 *
 * Formats (row-major everywhere):
 *  NVFP4: codes [R, C/2] uint8, element 2j of a row in the low nibble of byte
 *         j (E2M1: magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6; bit 3 = sign); block
 *         scales [R, C/16] uint8 E4M3 (one per 16 consecutive elements of a
 *         row); one float32 tensor scale per row group.  Value of an element:
 *         fl(fl(q * sc) * S).
 *  MXFP8: codes [R, C] uint8 E4M3FN; scales [R, C/32] uint8 E8M0 (value
 *         2**(byte - 127)), one per 32 consecutive elements along the block
 *         direction.
 *  Group-major padded (transposed MXFP8): rows of the source matrix [R, C]
 *         are cut into groups by off[G+1]; group g is stored at code offset
 *         C * off_pad[g] as a row-major block [C][P_g], P_g = pad32(R_g) =
 *         off_pad[g+1] - off_pad[g], padded with zero codes; its scales at
 *         offset C * off_pad[g] / 32, row-major [C][P_g / 32] (MOE4_SF_ROWS)
 *         or block-major [P_g / 32][C] (MOE4_SF_BLOCKS: per 32-row block, the
 *         scales of all C columns in order, so the scales of consecutive
 *         columns for one block are consecutive bytes).  MX blocks run along
 *         the source rows and never straddle a group.
 */
#ifndef MOE4_H
#define MOE4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ codes */
#define MOE4_OK 0
#define MOE4_EINVAL (-1)      /* bad shape, mode, dtype or NULL pointer        */
#define MOE4_EALIGN (-2)      /* a pointer is not 16-byte aligned              */
#define MOE4_EWORKSPACE (-3)  /* workspace missing or too small                */
#define MOE4_EHIP (-4)        /* a HIP launch failed                           */
#define MOE4_EUNSUPPORTED (-5)
#define MOE4_EDEVICE (-6)     /* moe4_debug_check: a kernel reported an error   */

/* Bits of the device-side error word (moe4_debug_check's message names them) */
#define MOE4_DEVERR_WAIT 1u   /* a bounded wait between workgroups gave up: that
                                 call's results are wrong                       */
#define MOE4_DEVERR_INDEX 2u  /* a routed row index outside its range was
                                 clamped (gather, combine, un-permute, dgates)  */

#define MOE4_BF16 0
#define MOE4_F32 1

#define MOE4_NVFP4_6 6        /* block scale maps the block amax to 6          */
#define MOE4_NVFP4_4OVER6 46  /* Four-Over-Six: keep the better of amax->6, ->4 */

#define MOE4_PRE_NONE 0
#define MOE4_PRE_SILU 1       /* quantise silu(x) (x must be bf16)             */
#define MOE4_PRE_SILU_AMAX 2  /* as MOE4_PRE_SILU, with ws[0..n_groups) already  \
                                 holding each group's max |silu(x)| as float    \
                                 bits (moe_grouped_gemm_fwd_silu_amax)          */

#define MOE4_RNE 0
#define MOE4_SR 1

#define MOE4_SF_ROWS 0        /* group-major scales [C][P_g/32]                */
#define MOE4_SF_BLOCKS 1      /* group-major scales [P_g/32][C]                */

/* ------------------------------------------------------------ diagnostics */
/* Message of the last failing call on this thread ("" if none). */
const char* moe4_last_error(void);
/* Library version string. */
const char* moe4_version(void);
/* Waits for the stream (a synchronising debugging aid, never called by the
 * library itself).  Returns MOE4_EHIP with the runtime's message for a failed
 * launch or a runtime error; otherwise reads and clears the current device's
 * device-side error word and returns MOE4_EDEVICE, naming the MOE4_DEVERR_*
 * conditions, if a kernel set any bit since the last check (of any stream:
 * a check while other streams run may report their errors, or clear a bit
 * one of them sets meanwhile); else MOE4_OK.  The error word and the
 * reporting follow the debugging contract of this library's interface: the
 * kernels cannot check data-dependent preconditions without a
 * synchronisation, so they clamp and report instead. */
int moe4_debug_check(void* stream);
/* Test hook for the error path above: with on != 0, every later
 * nvfp4_quant_requant_T launch makes its bounded waits wait for a count that
 * never arrives, with a small spin limit, so each wait gives up and sets
 * MOE4_DEVERR_WAIT (every kernel still exits; that call's results are
 * wrong).  on = 0 restores normal operation.  Process-wide; always MOE4_OK. */
int moe4_debug_force_wait_timeout(int on);

/* ---------------------------------------------------------------- NVFP4 */
/*
 * nvfp4_quant_46 - two-level NVFP4 quantisation with the Four-Over-Six choice.
 * Pages: lhc.media page, paragraph on NVFP4 (4-bit values, a scale shared by
 * sixteen values, about 4.5 bits per value); agihunt.info page, "Confirmed"
 * (activation quantisation chooses between two scaling factors).
 *
 * x            [rows, cols] bf16 (dtype MOE4_BF16) or float32 (MOE4_F32).
 * group_row_off  NULL (one group) or [n_groups+1] ascending row offsets with
 *              off[0] = 0 and off[n_groups] = rows; each group gets its own
 *              tensor scale.
 * mode         MOE4_NVFP4_6 or MOE4_NVFP4_4OVER6.
 * pre_op       MOE4_PRE_NONE, or MOE4_PRE_SILU to quantise the correctly
 *              rounded float32 silu(x) of a bf16 x.
 * codes        out [rows, cols/2];  sf  out [rows, cols/16];
 * tensor_scale out [n_groups] float32:
 *              S_g = fl(amax_g / (m_max * 448)), m_max = 4 (4/6) or 6 (mode 6);
 *              S_g = 1 for an all-zero group.
 * Per 16-block, candidate m in {6, 4}: sc_m = e4m3_rne(fl(amax_b / fl(m*S)));
 * q_i = e2m1_rne(fl(x_i * fl(1 / fl(dec(sc_m) * S)))) (signed zeros when sc_m
 * or the effective scale is 0); error = sequential float32 sum over i of
 * fl(t*t), t = fl(x_i - fl(fl(q_i*sc_m)*S)); 4 is kept iff err_4 < err_6.
 * cols % 16 == 0, n_groups >= 1.  ws: nvfp4_quant_46_ws_bytes(n_groups)
 * (up to eight amax words per group, so that a tensor of few groups does not
 * serialise its maxima on one word).
 */
int nvfp4_quant_46(const void* x, int dtype, int64_t rows, int64_t cols,
                   const int32_t* group_row_off, int32_t n_groups, int mode, int pre_op,
                   uint8_t* codes, uint8_t* sf, float* tensor_scale,
                   void* ws, size_t ws_bytes, void* stream);
size_t nvfp4_quant_46_ws_bytes(int32_t n_groups);

/*
 * nvfp4_quant_46_noalloc - nvfp4_quant_46 without a workspace, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Its scratch (the group
 * amax words, nvfp4_quant_46_ws_bytes(n_groups)) is a static device array of
 * the library, 4096 words (16 KB)
 * per device, held until the process ends; each call clears the words it
 * uses with a kernel first.  Arguments and results as nvfp4_quant_46 (byte
 * for byte), except: pre_op MOE4_PRE_NONE or MOE4_PRE_SILU only
 * (MOE4_PRE_SILU_AMAX takes the GEMM's amax buffer: use nvfp4_quant_46);
 * 1 <= n_groups <= 4096, else MOE4_EINVAL with nothing enqueued.  Every call
 * on one device shares that device's array: calls that overlap on one device
 * (on any streams) race and give wrong results.  Allocates nothing.
 */
int nvfp4_quant_46_noalloc(const void* x, int dtype, int64_t rows, int64_t cols,
                           const int32_t* group_row_off, int32_t n_groups, int mode, int pre_op,
                           uint8_t* codes, uint8_t* sf, float* tensor_scale, void* stream);

/*
 * nvfp4_quant_requant_T - weights: both low-precision copies in one pass.
 * Byte for byte the result of nvfp4_quant_46 on float32 x [rows, cols] in
 * mode MOE4_NVFP4_6 with n_groups equal row groups (one tensor scale each),
 * followed by mxfp8_requant_sr_T of that result with ts per group, the same
 * groups and MOE4_SF_ROWS: the forward NVFP4 operand and the backward
 * transposed MXFP8 operand of a weight matrix (lhc.media page, the paragraphs
 * on FP32 master weights and on requantising the dequantised, transposed
 * values with stochastic rounding; agihunt.info page, "Confirmed").
 * rows = n_groups * R_g with R_g % 32 == 0, so no padding: mx_codes
 * [cols * rows] holds group g's [cols][R_g] block at cols * g * R_g, mx_sf
 * [cols * rows / 32] its [cols][R_g / 32] scales at cols * g * R_g / 32.
 * codes [rows, cols/2], sf [rows, cols/16], tensor_scale [n_groups] as in
 * nvfp4_quant_46; seed, stream_id as in mxfp8_requant_sr_T.  cols % 32 == 0;
 * x, codes and mx_codes 16-byte aligned.
 * ws: nvfp4_quant_requant_T_ws_bytes(n_groups) bytes (3 KB per group),
 * cleared by the call (per-group partial maxima and counts); calls in flight
 * at the same time need workspaces of their own.
 */
int nvfp4_quant_requant_T(const float* x, int64_t rows, int64_t cols, int32_t n_groups,
                          uint8_t* codes, uint8_t* sf, float* tensor_scale, uint64_t seed, uint32_t stream_id,
                          uint8_t* mx_codes, uint8_t* mx_sf, void* ws, size_t ws_bytes, void* stream);
size_t nvfp4_quant_requant_T_ws_bytes(int32_t n_groups);

/*
 * nvfp4_dequant - float32 values fl(fl(q*sc)*S) of an NVFP4 tensor: the
 * dequantisation that precedes the transpose and requantisation of the
 * backward (lhc.media page, the paragraph on dequantising the forward values
 * before transposing them), here as a test and debugging aid.
 * codes [rows, cols/2], sf [rows, cols/16] as written by nvfp4_quant_46;
 * ts_per_group = 0: ts[0] applies to every row, 1: ts[g] to the rows of group
 * g of group_row_off [n_groups+1]; out [rows, cols] float32.  cols % 16 == 0;
 * codes and out 16-byte aligned.
 */
int nvfp4_dequant(const uint8_t* codes, const uint8_t* sf, const float* ts, int ts_per_group,
                  const int32_t* group_row_off, int32_t n_groups, int64_t rows, int64_t cols,
                  float* out, void* stream);

/* ---------------------------------------------------------------- MXFP8 */
/*
 * mxfp8_requant_sr_T - NVFP4 [rows, cols] -> dequantise (float32, as
 * nvfp4_dequant) -> transpose -> MXFP8 with stochastic rounding, in the
 * group-major padded layout.  Pages: lhc.media page, the paragraphs on
 * transposition regrouping the values that share a scale and on requantising
 * the dequantised, transposed values into MXFP8 with stochastic rounding.
 *
 * group_row_off / group_off_pad  [n_groups+1] unpadded and padded (pad32)
 *              row offsets (device); n_groups >= 1.
 * ts, ts_per_group  tensor scales: one per group, or ts[0] for all rows.
 * seed, stream_id   stochastic-rounding key.
 * sf_layout    MOE4_SF_ROWS or MOE4_SF_BLOCKS (arrangement of out_sf).
 * out_codes    [cols * off_pad[n_groups]], out_sf [cols * off_pad[n_groups] / 32].
 * MX scale per 32-block: e = least integer with amax <= 448 * 2**e, clamped to
 * [-127, 127] (e = -127 for an all-zero block).  Element i = r * cols + c (r, c
 * in the source matrix) rounds |w| = |v| * 2**-e up to the next E4M3 value iff
 * floor(frac * 2**16) + r16_i >= 2**16, where frac is |w|'s position between
 * its two E4M3 neighbours and r16_i is 16 bits of the counter hash
 *   word_j = fmix32(lo32(j) ^ fmix32(K ^ hi32(j))),  j = i >> 1,
 *   K = fmix32(fmix32(fmix32(lo32(seed)) ^ hi32(seed)) ^ stream_id),
 *   r16_i = (word_j >> (16 * (i & 1))) & 0xFFFF
 * (fmix32: MurmurHash3's 32-bit finaliser).  cols % 32 == 0.
 * max_padded_rows: an upper bound of off_pad[n_groups] (e.g. rows + 31*n_groups)
 * used to size the grid; the kernels read the real bound from the device.
 */
int mxfp8_requant_sr_T(const uint8_t* codes, const uint8_t* sf, const float* ts, int ts_per_group,
                       int64_t rows, int64_t cols, const int32_t* group_row_off,
                       const int32_t* group_off_pad, int32_t n_groups, int64_t max_padded_rows,
                       uint64_t seed, uint32_t stream_id, int sf_layout,
                       uint8_t* out_codes, uint8_t* out_sf, void* stream);

/*
 * mxfp8_requant_mx_sr_T - as mxfp8_requant_sr_T for a forward operand that is
 * itself MXFP8 row-wise (codes [rows, cols] E4M3, scales [rows, cols/32]
 * E8M0, no tensor scale): exact values code * 2**(scale - 127) -> transpose ->
 * MXFP8 with stochastic rounding (same exponent rule, random words and
 * layouts).  For the layers the pages keep in MXFP8 (agihunt.info page,
 * "Confirmed": the last 16.6% of layers; lhc.media page, the paragraph on
 * requantising dequantised, transposed values with stochastic rounding).
 */
int mxfp8_requant_mx_sr_T(const uint8_t* codes, const uint8_t* sf, int64_t rows, int64_t cols,
                          const int32_t* group_row_off, const int32_t* group_off_pad, int32_t n_groups,
                          int64_t max_padded_rows, uint64_t seed, uint32_t stream_id, int sf_layout,
                          uint8_t* out_codes, uint8_t* out_sf, void* stream);

/*
 * mxfp8_quant_requant_T - weights of the MXFP8-forward layers: both copies in
 * one pass.  Byte for byte the result of mxfp8_quant on float32 x [rows, cols]
 * (RNE, row-wise blocks of 32 along the row) followed by mxfp8_requant_mx_sr_T
 * of that result with n_groups equal row groups, no padding and
 * MOE4_SF_ROWS (agihunt.info page, "Confirmed": the last 16.6% of layers in
 * MXFP8; lhc.media page, the paragraphs on FP32 master weights and on
 * requantising the dequantised, transposed values with stochastic rounding).
 * rows = n_groups * R_g with R_g % 32 == 0; codes [rows, cols], sf
 * [rows, cols/32]; t_codes [cols * rows] holds group g's [cols][R_g] block at
 * cols * g * R_g, t_sf [cols * rows / 32] its [cols][R_g / 32] scales at
 * cols * g * R_g / 32; seed, stream_id as in mxfp8_requant_mx_sr_T.
 * cols % 32 == 0; x, codes and t_codes 16-byte aligned.  No workspace.
 */
int mxfp8_quant_requant_T(const float* x, int64_t rows, int64_t cols, int32_t n_groups, uint64_t seed,
                          uint32_t stream_id, uint8_t* codes, uint8_t* sf, uint8_t* t_codes, uint8_t* t_sf,
                          void* stream);

/*
 * mxfp8_quant - MXFP8 quantisation of a gradient (or, for the MXFP8-forward
 * layer, of a forward operand).  The value of source element (r, c) is:
 *   v = x[src(r), c]                                    (no options)
 *   v = fl(row_scale[a] * x[a / map_div, c]), a = row_map[r]   (row_map given;
 *       row_scale may be NULL: a plain gather)
 *   v = fl(x[r, c] * dsilu(u[r, c]))                    (dsilu_src given)
 *   v = silu(x[r, c])                                   (pre_op MOE4_PRE_SILU)
 * with x bf16 or float32 (dtype), u bf16, silu / dsilu the correctly rounded
 * float32 silu and silu' of a bf16 value (MOE4_PRE_SILU needs bf16 x).
 * row_map, dsilu_src and MOE4_PRE_SILU are exclusive.  rows = number of
 * output rows.
 * transpose = 0: blocks of 32 along cols, out [rows, cols] + [rows, cols/32].
 * transpose = 1: blocks along rows per group, group-major padded layout
 *                with row-major scales (group_row_off, group_off_pad,
 *                n_groups, max_padded_rows as in mxfp8_requant_sr_T);
 * transpose = 2: as 1 with block-major scales (MOE4_SF_BLOCKS).
 * rnd: MOE4_RNE, or MOE4_SR with (seed, stream_id) and the same random words
 *      as mxfp8_requant_sr_T (element index r * cols + c of the [rows, cols]
 *      matrix of values v).  Pages: the MXFP8 backward of the agihunt.info
 *      page, "Confirmed".  cols % 32 == 0.
 */
int mxfp8_quant(const void* x, int dtype, int64_t rows, int64_t cols,
                const int32_t* row_map, int32_t map_div, const float* row_scale,
                const uint16_t* dsilu_src, int pre_op, int transpose,
                const int32_t* group_row_off, const int32_t* group_off_pad, int32_t n_groups,
                int64_t max_padded_rows, int rnd, uint64_t seed, uint32_t stream_id,
                uint8_t* out_codes, uint8_t* out_sf, void* stream);

/*
 * mxfp8_quant_rows_T - both MXFP8 copies of a gradient from one read: the
 * row-wise one (the data-gradient operand) and the transposed one per group
 * (the weight-gradient operand), as in the agihunt.info page, "Confirmed".
 * Byte for byte the results of mxfp8_quant with transpose = 0 (row_codes
 * [rows, cols], row_sf [rows, cols/32]) and with transpose = 1 (sf_layout
 * MOE4_SF_ROWS) or 2 (MOE4_SF_BLOCKS) (t_codes, t_sf), for the same source
 * options (row_map / row_scale or dsilu_src; no pre_op), rnd, seed and
 * stream_id.  Needs group_row_off[n_groups] == rows (every row in a group:
 * rows outside the groups are not written).
 */
int mxfp8_quant_rows_T(const void* x, int dtype, int64_t rows, int64_t cols,
                       const int32_t* row_map, int32_t map_div, const float* row_scale,
                       const uint16_t* dsilu_src, const int32_t* group_row_off,
                       const int32_t* group_off_pad, int32_t n_groups, int64_t max_padded_rows,
                       int rnd, uint64_t seed, uint32_t stream_id, int sf_layout,
                       uint8_t* row_codes, uint8_t* row_sf, uint8_t* t_codes, uint8_t* t_sf,
                       void* stream);

/* ------------------------------------------------------------- routing */
/*
 * moe_route_topk - top-k routing and the stable expert permutation.  The pages
 * describe a token routed to 8 of 384 experts and inputs dispatched to the
 * experts that hold them (fourweekmba.com page, "Update"; lhc.media page,
 * paragraph on communication).
 * logits [T, E] float32, bias [E] or NULL.  z = fl(logit + bias); top-k in
 * descending z, equal values by lower expert index; gates
 * g_j = fl(w_j / s), w_j = RN32(exp_f64(fl(z_j - z_0))), s = sequential fp32 sum.
 * Outputs: topk_idx [T, k] int32, gates [T, k] float32, expert_off [E+1],
 * expert_off_pad [E+1] (pad32 of the counts), perm [T*k] (row -> assignment
 * a = t*k + j, rows ordered by (expert, token)), inv_perm [T*k].
 * 1 <= k <= E <= 1024, k <= 16.  ws: moe_route_topk_ws_bytes(T, E, k).
 */
int moe_route_topk(const float* logits, const float* bias, int64_t T, int32_t E, int32_t k,
                   int32_t* topk_idx, float* gates, int32_t* expert_off, int32_t* expert_off_pad,
                   int32_t* perm, int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream);
size_t moe_route_topk_ws_bytes(int64_t T, int32_t E, int32_t k);

/*
 * moe_route_backward - gradient in the router logits from the gate gradient
 * (moe_dgates): the gates of moe_route_topk are a softmax of z = logit + bias
 * over the k selected experts, so for token t, slot j (expert e_j = topk_idx[t,j]):
 *   s = 0; for i = 0..k-1: s = fl(s + fl(g_i * dg_i));
 *   dlogits[t, e_j] = fl(g_j * fl(dg_j - s)),  dlogits[t, e] = 0 otherwise
 * (float32, no fused multiply-add; the top-k choice itself has no gradient).
 * The routing itself is the local stand-in for the pages' 8-of-384 routing
 * (fourweekmba.com page, "Update").  dg, gates [T, k] float32, topk_idx
 * [T, k] int32 (distinct experts per token), dlogits [T, E] float32 out.
 * 1 <= k <= min(E, 16).
 */
int moe_route_backward(const float* dg, const float* gates, const int32_t* topk_idx, int64_t T, int32_t E,
                       int32_t k, float* dlogits, void* stream);

/*
 * moe_gather_rows - NVFP4 dispatch: out row r = source row perm[r] / k (codes
 * and block scales; the tensor scale is shared).  The local stand-in for the
 * pages' NVFP4 dispatch (lhc.media page, paragraph on communication).
 * n_rows_out = T * k; cols % 16 == 0.
 */
int moe_gather_rows(const uint8_t* codes, const uint8_t* sf, int64_t n_rows_in, int64_t cols,
                    const int32_t* perm, int32_t k, int64_t n_rows_out,
                    uint8_t* out_codes, uint8_t* out_sf, void* stream);

/* --------------------------------------------------------- grouped GEMMs */
/*
 * moe_grouped_gemm_fwd - C[rows of e] = A[rows of e] . B[e]^T with NVFP4 A
 * [M_total, K] (tensor scale a_ts[0], or a_ts[e] if a_ts_per_group) and NVFP4
 * B [E, N, K] (tensor scale b_ts[e]); rows grouped by expert_off [E+1].
 * Pages: agihunt.info page, "Confirmed" (NVFP4 expert-layer forward with a
 * dedicated kernel); fourweekmba.com page, "Why the Gain Is 8%, Not 3x".
 * The block-scaled products are exact (operands dequantised exactly to f16),
 * accumulated in float32; the tensor scales are applied in the epilogue.
 * c [M_total, N]: bf16 (c_dtype MOE4_BF16) or float32.  K % 64 == 0,
 * N % 32 == 0; a_codes, b_codes and c 16-byte aligned (MOE4_EALIGN).
 */
int moe_grouped_gemm_fwd(const uint8_t* a_codes, const uint8_t* a_sf, const float* a_ts, int a_ts_per_group,
                         const uint8_t* b_codes, const uint8_t* b_sf, const float* b_ts,
                         const int32_t* expert_off, int32_t E, int64_t M_total, int64_t N, int64_t K,
                         void* c, int c_dtype, void* stream);

/*
 * moe_grouped_gemm_fwd_silu_amax - moe_grouped_gemm_fwd with bf16 output U,
 * which also writes, per expert e, the float bits of max |silu(u)| over the
 * stored bf16 values of e's rows into silu_amax[e] (cleared by the call):
 * SiLU and the per-expert maximum of the next quantisation folded into the
 * up GEMM's epilogue (lhc.media page, the paragraph on fused kernels).
 * nvfp4_quant_46 with pre_op MOE4_PRE_SILU_AMAX and ws = silu_amax then
 * skips its own amax pass; the result is byte for byte that of
 * MOE4_PRE_SILU.  silu_amax: nvfp4_quant_46_ws_bytes(E) bytes of device
 * memory (the caller's; the call writes its first E words).
 * Returns MOE4_EUNSUPPORTED (nothing launched) unless the shape selects the
 * warp-specialised kernels (K % 256 == 0, N % 128 == 0, 32-bit offsets).
 */
int moe_grouped_gemm_fwd_silu_amax(const uint8_t* a_codes, const uint8_t* a_sf, const float* a_ts, int a_ts_per_group,
                                   const uint8_t* b_codes, const uint8_t* b_sf, const float* b_ts,
                                   const int32_t* expert_off, int32_t E, int64_t M_total, int64_t N, int64_t K,
                                   uint16_t* c, uint32_t* silu_amax, void* stream);

/*
 * moe_grouped_gemm_bwd_dgrad - C[rows of e] = A[rows of e] . B[e]^T with MXFP8
 * A [M_total, K] (+ scales [M_total, K/32]) and MXFP8 B [E, N, K] (+ [E, N,
 * K/32]); float32 C [M_total, N].  Native block-scaled FP8 MFMA (exact
 * products, float32 accumulation).  K % 32 == 0, N % 32 == 0; A and each
 * expert's B below 2 GiB (32-bit buffer offsets).
 * Pages: agihunt.info page, "Confirmed" (MXFP8 backpropagation).
 */
int moe_grouped_gemm_bwd_dgrad(const uint8_t* a_codes, const uint8_t* a_sf,
                               const uint8_t* b_codes, const uint8_t* b_sf,
                               const int32_t* expert_off, int32_t E, int64_t M_total, int64_t N, int64_t K,
                               float* c, void* stream);

/*
 * moe_grouped_gemm_mx - the same product as moe_grouped_gemm_bwd_dgrad with
 * a choice of output: c_dtype MOE4_F32 (identical to the dgrad call) or
 * MOE4_BF16 (the float32 result rounded to nearest even; needs K % 128 ==
 * 0).  The forward GEMMs of the MXFP8 layers (agihunt.info page,
 * "Confirmed": the last 16.6% of layers in MXFP8; fourweekmba.com page, the
 * MXFP8 rate in the hardware table).
 */
int moe_grouped_gemm_mx(const uint8_t* a_codes, const uint8_t* a_sf, const uint8_t* b_codes, const uint8_t* b_sf,
                        const int32_t* expert_off, int32_t E, int64_t M_total, int64_t N, int64_t K,
                        void* c, int c_dtype, void* stream);

/*
 * moe_grouped_gemm_bwd_wgrad - dW[e] = A_e . B_e^T over expert e's padded token
 * dimension: the weight-gradient products of the MXFP8 backward (agihunt.info
 * page, "Confirmed"), float32 master-weight gradients (lhc.media page,
 * paragraph on the precisions that remain).  A and B in the group-major
 * padded MXFP8 layout with block-major scales (MOE4_SF_BLOCKS), A_e [N1][P_e]
 * (scales [P_e/32][N1]), B_e [N2][P_e] (scales [P_e/32][N2]) with
 * P_e = off_pad[e+1] - off_pad[e].  dw [E, N1, N2] float32; beta = 0
 * overwrites, beta = 1 accumulates.  Experts with no rows: with beta = 0 their
 * dw[e] is written with zeros, unless flags holds MOE4_WGRAD_SKIP_EMPTY, which
 * leaves it untouched (the caller knows them from off_pad: dw[e] is written
 * iff off_pad[e+1] > off_pad[e]); with beta = 1 nothing is added.
 * N1 % 32 == 0, N2 % 32 == 0; each expert's operands (N1 * P_e and N2 * P_e
 * bytes) below 2 GiB (32-bit buffer offsets).
 */
#define MOE4_WGRAD_SKIP_EMPTY 1
int moe_grouped_gemm_bwd_wgrad(const uint8_t* a_codes, const uint8_t* a_sf,
                               const uint8_t* b_codes, const uint8_t* b_sf,
                               const int32_t* expert_off_pad, int32_t E, int64_t N1, int64_t N2,
                               float* dw, float beta, int flags, void* stream);

/*
 * moe_grouped_gemm_bwd - dgrad and wgrad of one expert linear layer in one
 * call (both enqueued on `stream`, dgrad first): the MXFP8 backward of the
 * expert layers (agihunt.info page, "Confirmed"; lhc.media page, the
 * paragraphs on requantising the transposed operands into MXFP8).
 * For the linear y = x . W^T with W [E][Nout][Nin] per expert:
 *   dx (float32 [M_total, Nin]) = moe_grouped_gemm_bwd_dgrad(dy row-wise
 *       [M_total, Nout], W^T requantised [E][Nin][Nout], expert_off),
 *   dw (float32 [E, Nout, Nin]) = moe_grouped_gemm_bwd_wgrad(dy transposed
 *       group-major [Nout][P_e], x transposed group-major [Nin][P_e], both
 *       with block-major scales, expert_off_pad, beta, flags).
 * Arguments, layouts and constraints as in the two calls; returns the first
 * error (nothing enqueued when the dgrad's checks fail).
 */
int moe_grouped_gemm_bwd(const uint8_t* dy_codes, const uint8_t* dy_sf,           /* [M_total, Nout] row-wise */
                         const uint8_t* wT_codes, const uint8_t* wT_sf,           /* [E, Nin, Nout]           */
                         const uint8_t* dyT_codes, const uint8_t* dyT_sf,         /* group-major [Nout][P_e]  */
                         const uint8_t* xT_codes, const uint8_t* xT_sf,           /* group-major [Nin][P_e]   */
                         const int32_t* expert_off, const int32_t* expert_off_pad, int32_t E,
                         int64_t M_total, int64_t Nin, int64_t Nout,
                         float* dx, float* dw, float beta, int flags, void* stream);

/* ----------------------------------------------------- combine / scatter */
/*
 * moe_combine - the gate-weighted return of the expert outputs to their
 * tokens, the local stand-in for the pages' combine (lhc.media page,
 * paragraph on communication; fourweekmba.com page, "Update": a token's
 * output sums its 8 routed experts): y[t] = bf16(acc), acc = 0; for
 * j = 0..k-1: acc = fl(acc + fl(gates[t,j] * yp[inv_perm[t*k+j]])).
 * yp [T*k, d] float32, gates [T, k], inv_perm [T*k] (moe_route_topk), y
 * [T, d] bf16.  1 <= k <= 16, d % 4 == 0.
 */
int moe_combine(const float* yp, const float* gates, const int32_t* inv_perm, int64_t T, int32_t k,
                int64_t d, uint16_t* y, void* stream);

/*
 * moe_unpermute_sum - the backward of the dispatch (lhc.media page,
 * paragraph on communication: inputs sent to the experts that hold them):
 * each token's input gradient sums the rows of its k routed copies,
 * dx[t] = bf16(acc), acc = 0; for j = 0..k-1: acc = fl(acc + dxp[inv_perm[t*k+j]]).
 * dxp [T*k, d] float32, inv_perm [T*k], dx [T, d] bf16.  1 <= k <= 16,
 * d % 4 == 0.
 */
int moe_unpermute_sum(const float* dxp, const int32_t* inv_perm, int64_t T, int32_t k, int64_t d,
                      uint16_t* dx, void* stream);

/*
 * moe_dgates - gate gradient dg[t*k+j] = sum_c dy[t,c] * yp[inv_perm[t*k+j], c]:
 * the derivative of moe_combine's weighted sum in gates[t,j] (the combine is
 * the local stand-in for the pages' return of expert outputs: lhc.media page,
 * paragraph on communication).  dy [T, d] bf16, yp [T*k, d] float32 (the
 * forward's expert outputs), dg [T, k] float32 out.  Float32 accumulation:
 * each lane sums its columns 8l + 512i in order, then a fixed butterfly over
 * the 64 lanes (deterministic).  1 <= k <= 16, d % 8 == 0; dy and yp 16-byte
 * aligned.
 */
int moe_dgates(const uint16_t* dy, const float* yp, const int32_t* inv_perm, int64_t T, int32_t k, int64_t d,
               float* dg, void* stream);

/* ------------------------------------------- combine-path quantiser (8.25 bits) */
/*
 * The expert results travelling back for the combine are sent as 8-bit
 * fixed-point values with one E8M0 scale per 32 values after a Hadamard
 * transform that spreads extreme values over each block; 16 bits per value
 * become 8.25 (lhc.media page, paragraph on communication).  The page names
 * the element format "S2F6" and gives nothing more; it is read here as signed
 * fixed point with 2 integer bits (sign included) and 6 fraction bits, the
 * element of OCP's MXINT8:
 *  - transform: the unnormalised Sylvester H_32 (entries +-1) over each block
 *    of 32 consecutive values of a row, in float32 as five butterfly stages
 *    (a, b) -> (a + b, a - b) with partner distance 1, 2, 4, 8, 16;
 *  - scale: e = floor(log2 max|y|) over the block, clamped to [-127, 127]
 *    (-127 for an all-zero block), one byte e + 127;
 *  - codes: int8 c = clamp(rne(y * 2^(6 - e)), -127, 127), worth c * 2^(e - 6).
 * Inputs must be finite with |x| <= 2^122.  Rows are contiguous; cols % 32 == 0.
 */

/*
 * moe_hmx8_quant - x [rows, cols] float32 (16-byte aligned) -> codes int8
 * [rows, cols] (8-byte aligned) and scales uint8 [rows, cols/32].  Buffers are
 * the caller's (device memory).  Returns MOE4_EINVAL / MOE4_EALIGN on bad
 * sizes or pointers (nothing launched).
 */
int moe_hmx8_quant(const float* x, int64_t rows, int64_t cols, int8_t* codes, uint8_t* scales, void* stream);

/*
 * moe_hmx8_dequant - exact decode of moe_hmx8_quant's payload:
 * out = H_32 (c * 2^(e - 6)) / 32 per block, float32 [rows, cols] (16-byte
 * aligned).  The integer butterflies and the power-of-two scale make every
 * value exact.
 */
int moe_hmx8_dequant(const int8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols, float* out,
                     void* stream);

/*
 * moe_combine_hmx8 - moe_combine over the decoded payload: y[t] = bf16(acc),
 * acc = 0; for j = 0..k-1: acc = fl(acc + fl(gates[t,j] * Yhat[inv_perm[t*k+j]])),
 * Yhat the exact decode of codes / scales ([T*k, d], the moe_hmx8_quant layout).
 * y [T, d] bf16 and codes 16-byte aligned; 1 <= k <= 16, d % 32 == 0.
 */
int moe_combine_hmx8(const int8_t* codes, const uint8_t* scales, const float* gates, const int32_t* inv_perm,
                     int64_t T, int32_t k, int64_t d, uint16_t* y, void* stream);

/*
 * moe_grouped_gemm_fwd_hmx8 - moe_grouped_gemm_fwd with float32 output c
 * [M_total, N] whose epilogue also writes the combine-path payload of the
 * stored values: codes int8 [M_total, N] and scales uint8 [M_total, N/32],
 * byte for byte those of moe_hmx8_quant(c).  The down projection's output and
 * its communication format in one pass (lhc.media page, paragraphs on fused
 * kernels and on communication).  The three buffers are the caller's (device
 * memory); c 16-byte aligned.  Returns MOE4_EUNSUPPORTED (nothing launched)
 * unless the shape selects the warp-specialised kernels (K % 256 == 0,
 * N % 128 == 0, more than 32 rows per expert on average), MOE4_EINVAL if
 * M_total * N >= 2^32.
 */
int moe_grouped_gemm_fwd_hmx8(const uint8_t* a_codes, const uint8_t* a_sf, const float* a_ts, int a_ts_per_group,
                              const uint8_t* b_codes, const uint8_t* b_sf, const float* b_ts,
                              const int32_t* expert_off, int32_t E, int64_t M_total, int64_t N, int64_t K, float* c,
                              int8_t* codes, uint8_t* scales, void* stream);

/* ------------------------------------------------------------------ router */
/*
 * The router in front of the expert layer, read as a linear map in BF16: the
 * pages route each token to 8 of 384 experts (fourweekmba.com page,
 * "Update") and keep some activations in BF16 (lhc.media page, paragraph on
 * the precisions that remain); the router's arithmetic is not on the pages.
 *
 * moe_router_logits - logits [T, E] float32 = x [T, d] bf16 . w [E, d]^T bf16,
 * bf16 MFMA with float32 accumulation.  d % 64 == 0; x and w 16-byte aligned;
 * buffers the caller's.
 */
int moe_router_logits(const uint16_t* x, const uint16_t* w, int64_t T, int32_t E, int64_t d, float* logits,
                      void* stream);

/*
 * moe_unpermute_sum_router - moe_unpermute_sum with the router's input
 * gradient added: for token t, column c, with e_j = topk_idx[t, j] and
 * dz_j = dlogits[t, e_j] (moe_route_backward's output),
 *   acc = 0; for j = 0..k-1: acc = fl(acc + dxp[inv_perm[t*k+j], c]);
 *   for j = 0..k-1: acc = fl(acc + fl(dz_j * w[e_j, c]));  dx[t, c] = bf16(acc)
 * (float32, no fused multiply-add).  dxp [T*k, d] float32 (16-byte aligned),
 * dlogits [T, E] float32, topk_idx [T, k], w [E, d] bf16 and dx [T, d] bf16
 * (8-byte aligned).  1 <= k <= min(E, 16), d % 4 == 0.  Out-of-range rows or
 * experts are clamped and reported (MOE4_DEVERR_INDEX).
 */
int moe_unpermute_sum_router(const float* dxp, const int32_t* inv_perm, int64_t T, int32_t k, int64_t d,
                             const float* dlogits, const int32_t* topk_idx, int32_t E, const uint16_t* w,
                             uint16_t* dx, void* stream);

/*
 * moe_router_wgrad - dw [E, d] float32: dw[e, c] = sum over the rows r of
 * expert e (expert_off from moe_route_topk; t = perm[r] / k) of
 * dlogits[t, e] * x[t, c].  Float32 sums in a fixed order: each expert's rows
 * in chunks of 128 (each chunk: four interleaved row shares in row order, then
 * the four shares in order), then the chunks in order; deterministic; experts
 * without rows get zeros.  x [T, d] bf16, dlogits [T, E], perm [T*k]; x, dw
 * and ws 16-byte aligned.  1 <= k <= E, d % 8 == 0, T*k < 2^31.
 * ws: moe_router_wgrad_ws_bytes(T, E, k, d) bytes (the chunk partial rows,
 * d floats each, for at most ceil(T*k / 128) + E chunks), the caller's,
 * overwritten.  Offsets that are not monotone within [0, T*k] are clamped and
 * reported (MOE4_DEVERR_INDEX).
 */
int moe_router_wgrad(const uint16_t* x, const float* dlogits, const int32_t* perm, const int32_t* expert_off,
                     int64_t T, int32_t E, int32_t k, int64_t d, float* dw, void* ws, size_t ws_bytes, void* stream);
size_t moe_router_wgrad_ws_bytes(int64_t T, int32_t E, int32_t k, int64_t d);

/*
 * moe_silu_eval - correctly rounded float32 silu(u) and silu'(u) of bf16 u
 * (either output may be NULL).  Test aid for the activation fused into
 * nvfp4_quant_46 (MOE4_PRE_SILU) and mxfp8_quant (dsilu_src).
 */
int moe_silu_eval(const uint16_t* u, int64_t n, float* silu_out, float* dsilu_out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE4_H */
