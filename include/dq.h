/*
 * dq.h -- C ABI of the MI355X (gfx950) DualQuant dual-scale quantizer.
 *
 * The method (paper summary "DualQuant: Dual-scale Calibration-free
 * Weight-and-Activation Quantization for LLMs", §3, §4.2-4.4, App. A-B;
 * reproduction README "DualQuant: Calibration-Free Dual-Scale Weight and
 * Activation Quantization", section "Core equations"):
 *
 *   W [rows, cols] ~= D_a Q D_b,   Q_ij = q(W_ij / (a_{i,g(j)} b_j)),
 *
 * with a [rows, cols/G] row/block inverse scales (G contiguous columns per
 * block), b [cols] column inverse scales and q a black-box element grid.
 * Block-coordinate descent alternates closed-form least-squares updates
 *   a_i <- Pi_Fa(sum_j W_ij R_ij / sum_j R_ij^2),  R = Q D_b  (per block)
 *   b_j <- Pi_Fb(sum_i W_ij S_ij / sum_i S_ij^2),  S = D_a Q  (all rows)
 * each projected onto the format's legal scale values, with Q requantized
 * after each update; a slice whose codes are all zero gets scale 1.
 *
 * Conventions for every call
 *  - All array arguments are DEVICE pointers owned by the caller. The
 *    library allocates nothing, keeps no state between calls, never writes
 *    W or X, and enqueues all work on `stream` (a hipStream_t; NULL = the
 *    default stream). Calls return after enqueueing; kernel faults surface
 *    at the caller's next synchronization.
 *  - Return value: DQ_OK (0) or a negative dq_status. Argument errors are
 *    detected on the host before anything is launched; then nothing is
 *    written. DQ_ERR_HIP reports a failed launch.
 *  - Matrices are row-major. W rows start ldw elements apart; the base
 *    pointer and the row pitch (ldw * element size) must be multiples of
 *    16 bytes. cols must be a multiple of the group size G.
 *  - Scale encodings: a uses the native encoding of a_fmt -- uint16 fp16
 *    bits, or one byte per scale (E8M0 biased exponent, E4M3 byte, OCP
 *    E4M3FN without sign). b is uint16 fp16 bits. Arrays are dense:
 *    a[i * (cols/G) + g], b[j].
 *  - Element codes: INT4 two's complement in [-8, 7], or E2M1 (sign bit,
 *    then level index 0..7 of 0, .5, 1, 1.5, 2, 3, 4, 6), two per byte:
 *    packed rows hold cols/2 bytes and the low nibble is the even column.
 *    The 8-bit grids of the MX formats the summary evaluates at 8 bits
 *    (§G.2) store one code per byte (rows of cols bytes): INT8 two's
 *    complement in [-127, 127], or an OCP E4M3FN byte (finite values,
 *    saturating at 448). A zero code is always stored as +0.
 *  - Rounding: element codes round to nearest with ties to even (INT4) or
 *    to the even encoding (E2M1), decided on the exact quotient; scales are
 *    projected to the nearest legal value (ties to even for fp16 / E4M3,
 *    upward for E8M0), clamped to the smallest legal value and saturated
 *    at the largest. Least-squares sums run in float64.
 *  - Calls that overlap on one stream are ordered; concurrent calls on
 *    different streams must not share output buffers or workspace.
 *  - Non-finite inputs are outside the contract (results unspecified).
 */
#ifndef DQ_H_
#define DQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DQ_OK = 0,
  DQ_ERR_INVALID_ARG = -1, /* null pointer, misaligned W, bad count      */
  DQ_ERR_SHAPE = -2,       /* rows/cols/ld inconsistent, cols % G != 0   */
  DQ_ERR_UNSUPPORTED = -3, /* format combination not built               */
  DQ_ERR_WORKSPACE = -4,   /* workspace missing or smaller than needed   */
  DQ_ERR_HIP = -5          /* a kernel launch failed                     */
} dq_status;

typedef enum { DQ_GRID_INT4 = 0, DQ_GRID_E2M1 = 1, DQ_GRID_INT8 = 2, DQ_GRID_E4M3 = 3 } dq_grid;
typedef enum { DQ_SCALE_FP16 = 0, DQ_SCALE_E8M0 = 1, DQ_SCALE_E4M3 = 2 } dq_scale_fmt;
typedef enum { DQ_W_F32 = 0, DQ_W_BF16 = 1 } dq_wtype;

/* One quantization problem. Fields are int32/int64 for a stable ABI.
 *   rows, cols  W is rows x cols (1 <= rows < 2^31, cols >= G)
 *   ldw         row pitch of W (and of X) in elements, cols <= ldw < 2^31
 *   group       G in {16, 32, 64}: block size along each row
 *   grid        dq_grid of the element codes
 *   a_fmt       dq_scale_fmt of the block scales
 *   b_fmt       dq_scale_fmt of the column scales (only DQ_SCALE_FP16)
 *   w_type      dq_wtype of W and of X (float32 or bf16)
 * Formats of the DualQuant summary §3 and §G.2: INT4 {grid INT4, G 64,
 * fp16}, MXINT4 {INT4, 32, E8M0}, NVFP4 {E2M1, 16, E4M3}, MXFP4 {E2M1, 32,
 * E8M0}, MXINT8 {INT8, 32, E8M0}, MXFP8 {E4M3, 32, E8M0}; every grid x
 * group x block-scale combination is accepted. */
typedef struct {
  int64_t rows, cols, ldw;
  int32_t group, grid, a_fmt, b_fmt, w_type, reserved;
} dq_problem;

/* Bytes of device workspace dq_bcd_iterate, dq_init_colnorm and
 * dq_quant_report need for problem p (0 if p is invalid). Depends only on
 * p's shape and format. */
size_t dq_workspace_bytes(const dq_problem* p);

/* Bytes of device workspace dq_bcd_iterate needs when it is given a stats
 * array (0 if p is invalid): dq_workspace_bytes(p) plus room for one
 * state's codes (rows x cols/2 bytes for 4-bit grids, rows x cols for
 * 8-bit grids) and per-workgroup sums. A workspace of this size serves
 * every call. */
size_t dq_stats_workspace_bytes(const dq_problem* p);

/* Absmax round-to-nearest initialization (DualQuant summary §3: symmetric
 * scale max|W| / qmax per block of G contiguous row elements; §5.3:
 * format-native row absmax scales). Writes a[i, g] = Pi_Fa(absmax / qmax)
 * (qmax 7 for INT4, 6 for E2M1, 127 for INT8, 448 for E4M3; 1 for an
 * all-zero block) and b[j] = 1.
 *   W  in   [rows, ldw] of w_type
 *   a  out  [rows, cols/G] in a_fmt's encoding
 *   b  out  [cols] fp16 bits */
int dq_init_rtn(const dq_problem* p, const void* W, void* a, uint16_t* b,
                void* stream);

/* Column-norm initialization, the alternative starting point of the
 * summary §5.3 (format-native row absmax scales together with per-column
 * L1-norm scales; the page gives no formula, so the following is this
 * library's reading): b_j = Pi_fp16(sum_i |W_ij| / rows) (1 for an all-zero
 * column), then a[i, g] = Pi_Fa(max_{j in g} |W_ij / b_j| / qmax) with
 * correctly rounded float64 quotients (1 for an all-zero block). Compared
 * with dq_init_rtn it moves the column magnitudes into b, which keeps the
 * block scales of small-valued formats such as NVFP4 out of E4M3's
 * subnormal range. Deterministic: the column sums run in a fixed order.
 *   W, a, b    as for dq_init_rtn
 *   workspace  scratch of at least dq_workspace_bytes(p) bytes, 256-byte
 *              aligned (the same workspace dq_bcd_iterate takes) */
int dq_init_colnorm(const dq_problem* p, const void* W, void* a, uint16_t* b,
                    void* workspace, size_t workspace_bytes, void* stream);

/* n_iters BCD iterations from the state (a, b), in place (reproduction
 * README "Core equations" and its flowchart; summary §4.3, App. A-B).
 * Each iteration: Q = q(W/(a b)); row/block update of a with R = Q D_b;
 * requantize; column update of b with S = D_a Q over all rows; requantize
 * (the last requantization is the next iteration's first step). The state
 * is exactly (a, b): iterate(k1) then iterate(k2) equals iterate(k1+k2).
 * n_iters = 0 leaves a and b as they are (with stats it writes row 0).
 *   W          in      [rows, ldw] of w_type
 *   a, b       in/out  as written by dq_init_rtn
 *   workspace  scratch of at least dq_workspace_bytes(p) bytes (with stats:
 *              dq_stats_workspace_bytes(p)), 256-byte aligned; its contents
 *              are private to the call, and it must not be shared by calls
 *              that may run concurrently
 *   stats      NULL, or out [n_iters + 1][3] float64 (device, 8-byte
 *              aligned): row k describes the state after k iterations of
 *              this call (row 0: the state passed in) with the quantities
 *              of dq_quant_report -- sum (W - D_a Q D_b)^2, sum W^2 and the
 *              number of codes that differ from those of state k - 1 (0 in
 *              row 0). These are the convergence diagnostics the pages
 *              follow (summary §5.3, App. B). Each pass measures the state
 *              it starts from while it reads W, so rows 0 .. n_iters - 1
 *              cost no extra read of W; row n_iters costs one. Sums run in
 *              a fixed order (deterministic); a and b come out exactly as
 *              without stats. */
int dq_bcd_iterate(const dq_problem* p, const void* W, void* a, uint16_t* b,
                   int32_t n_iters, void* workspace, size_t workspace_bytes,
                   double* stats, void* stream);

/* dq_bcd_iterate for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same iterations, with a, b and every bit of the result
 * as dq_bcd_iterate (stats = NULL) leaves them, but with no workspace
 * argument. The partial column sums live in a fixed array inside the
 * library of DQ_NOALLOC_SCRATCH_BYTES bytes, which each GPU the library
 * runs on holds until the process ends; nothing is allocated or freed.
 *   W, a, b, n_iters, stream  as for dq_bcd_iterate
 * Returns DQ_ERR_WORKSPACE when the problem's partial sums need more than
 * DQ_NOALLOC_SCRATCH_BYTES (dq_workspace_bytes(p) <= that bound always
 * fits), and DQ_ERR_HIP if the array's device address cannot be obtained.
 * Every call on one GPU shares that GPU's array, so calls that may overlap
 * on one GPU (on different streams) race and must not be issued; calls on
 * one stream are ordered and safe. The array keeps the last call's partial
 * sums; no call depends on its earlier contents. */
#define DQ_NOALLOC_SCRATCH_BYTES (16u << 20)
int dq_bcd_iterate_noalloc(const dq_problem* p, const void* W, void* a, uint16_t* b,
                           int32_t n_iters, void* stream);

/* The whole solve in one call: dq_init_rtn, dq_bcd_iterate(n_iters) and
 * dq_pack_codes, with a, b and packed exactly as those three calls leave
 * them. The absmax initialization is formed inside the first iteration's
 * pass from the rows it reads, which saves one read of W and a launch;
 * n_iters = 0 runs the initialization and the packing alone.
 *   W          in   [rows, ldw] of w_type
 *   a, b       out  the final state, encodings as for dq_init_rtn; b
 *                   16-byte aligned
 *   packed     out  as for dq_pack_codes
 *   workspace  scratch of at least dq_workspace_bytes(p) bytes, 256-byte
 *              aligned */
int dq_solve(const dq_problem* p, const void* W, void* a, uint16_t* b, int32_t n_iters,
             uint8_t* packed, void* workspace, size_t workspace_bytes, void* stream);

/* Final codes Q = q(W/(a b)), packed two per byte (summary App. I: packed
 * offline for deployment).
 *   b       in   [cols] fp16 bits, 16-byte aligned
 *   packed  out  4-bit grids: [rows, cols/2] uint8, row pitch cols/2,
 *                8-byte aligned; 8-bit grids: [rows, cols], 16-byte aligned */
int dq_pack_codes(const dq_problem* p, const void* W, const void* a,
                  const uint16_t* b, uint8_t* packed, void* stream);

/* Report on the state (a, b): its codes Q = q(W/(a b)) and
 *   report[0] = sum (W - D_a Q D_b)^2        squared reconstruction error
 *   report[1] = sum W^2                      (normalized error = [0] / [1])
 *   report[2] = number of codes that differ from prev_packed (0 if NULL)
 * as float64, summed in a fixed order (deterministic). These are the
 * quantities the pages follow over the iterations (summary §5.3 and the
 * convergence figure of App. B: normalized MSE and the share of codes that
 * change); calling dq_bcd_iterate(1) and this in turn gives them per
 * iteration, at the cost of one more read of W each.
 *   prev_packed  in, may be NULL   codes of an earlier state, in
 *                                  dq_pack_codes' layout and alignment
 *   packed       out, may be NULL  this state's codes, as dq_pack_codes
 *   report       out               3 float64 (device), 8-byte aligned
 *   workspace    scratch of at least dq_workspace_bytes(p) bytes,
 *                256-byte aligned */
int dq_quant_report(const dq_problem* p, const void* W, const void* a, const uint16_t* b,
                    const uint8_t* prev_packed, uint8_t* packed, double* report,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Activation side of the factorization X W^T ~= (X D_b) Q^T D_a (summary
 * §4.4: the column scale multiplies the activations inside the
 * activation-quantization kernel, then format-native blockwise
 * quantization; reproduction README "Core equations"). For every token t
 * and block g of G channels: X' = X D_b, s = Pi_Fa(absmax(X'_tg) / qmax)
 * (1 if zero), codes = q(X'_tg / s).
 *   X         in   [tokens, ldx] of p->w_type (bf16 only); p->cols channels
 *                  are used; base and row pitch 16-byte aligned
 *   tokens    number of rows of X (>= 0; 0 is a no-op)
 *   b         in   [cols] fp16 bits, 16-byte aligned
 *   xq        out  [tokens, cols/2] (4-bit grids) or [tokens, cols] (8-bit)
 *                  codes, 16-byte aligned
 *   x_scales  out  [tokens, cols/G] in a_fmt's encoding */
int dq_rescale_quantize_act(const dq_problem* p, const void* X, int64_t tokens,
                            int64_t ldx, const uint16_t* b, uint8_t* xq,
                            void* x_scales, void* stream);

/* Static description of a status code. */
const char* dq_status_string(int status);

/* ABI version of this header (incremented on incompatible changes). */
int dq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DQ_H_ */
