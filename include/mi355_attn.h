/*
 * mi355_attn.h -- C ABI of the MI355X (gfx950) FlashAttention-2 forward
 * (attn_fwd; attn_fwd_dv for a value head dim of its own), its gradient
 * (attn_bwd), and the fused axial-attention block built around it
 * (axial_pass, axial_block).
 *
 * The operation (FlashAttention-2 forward, as stated by "Extend Thunder with
 * CUDA-Python", Python reference section, and "Blackwell Attention Example",
 * attention kernel): for every batch b, head h and query row i
 *
 *     s_j  = scale * <q[b,h,i,:], k[b,h,j,:]>      j = 0 .. N-1
 *            (causal: only j <= i, top-left aligned, as the reference's mask
 *             keeps key index <= query index in absolute positions)
 *     O[b,h,i,:] = sum_j softmax(s)_j * v[b,h,j,:]
 *     L[b,h,i]   = ln( sum_j exp(s_j) )            natural-log logsumexp
 *
 * computed tile by tile with a running max and running sum so that the
 * M x N score matrix is never stored. L is what the Python reference returns
 * as m + log(l); the Helion example returns the same quantity in base 2 and
 * it is converted here to the natural log.
 *
 * Layout: contiguous row-major. q and o are [B, H, M, D]; k and v are
 * [B, H, N, D]; lse is [B, H, M] fp32 (the reference's [.., M, 1] is the same
 * memory). q, k, v and o share one element type (MI355_ATTN_FP32,
 * MI355_ATTN_BF16 or MI355_ATTN_FP16); lse is always fp32. With 16-bit inputs
 * both products accumulate in fp32 and P is rounded to the input type before
 * the second one, as the Blackwell example does for its 16-bit inputs.
 *
 * Ownership: every pointer is caller-owned device memory on the current HIP
 * device. The library allocates nothing, keeps no pointer after a call
 * returns, and has no mutable global state.
 *
 * Execution: every entry point enqueues its kernels on `stream` (a
 * hipStream_t; NULL is the null stream) and return without synchronising.
 * Faults inside a kernel surface at the caller's next synchronisation. Calls
 * are reentrant.
 *
 * Errors: every argument check happens before any HIP call; a call that fails
 * a check launches nothing and writes nothing.
 */
#ifndef MI355_ATTN_H
#define MI355_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and o. fp16: the Blackwell example's main
 * function describes its test as float16 (its calls pass bf16), and the
 * Thunder page's native-kernel section proposes 16-bit floats. The forward
 * accepts all three types, the backward bf16 and fp16. */
#define MI355_ATTN_FP32 0
#define MI355_ATTN_BF16 1
#define MI355_ATTN_FP16 2

/* Status codes. */
#define MI355_ATTN_OK                0 /* success (also: nothing to do)            */
#define MI355_ATTN_ERR_INVALID_ARG   1 /* bad pointer / size / flag / overlap      */
#define MI355_ATTN_ERR_UNSUPPORTED   2 /* valid but not implemented (D, size)      */
#define MI355_ATTN_ERR_MISALIGNED    3 /* q/k/v/o not 16-byte or lse not 4-byte    */
#define MI355_ATTN_ERR_HIP           4 /* the HIP launch reported an error         */
#define MI355_ATTN_ERR_SCRATCH       5 /* B*H*M above the no-alloc scratch capacity */

/* Kernel paths (attn_fwd_path / attn_fwd_select_path). */
#define MI355_ATTN_PATH_AUTO  0 /* let the library choose                        */
#define MI355_ATTN_PATH_MAIN  1 /* tiled MFMA kernel with the online softmax      */
#define MI355_ATTN_PATH_SMALL 2 /* one-tile, register-resident short-row kernel */

/*
 * attn_fwd -- O and L of scaled-dot-product attention (see the top of this
 * file for the definition and layouts).
 *
 *   q, k, v    device pointers to the inputs, element type `dtype`.
 *   o          device pointer to the output [B,H,M,D], element type `dtype`.
 *   lse        device pointer to the fp32 output [B,H,M] (natural log).
 *   B, H       batch and head counts (>= 0).
 *   M, N       query and key lengths (M >= 0; N >= 1 whenever B*H*M > 0).
 *   D          head dimension: 16, 32, 64 or 128.
 *   scale      multiplier of q.k, finite; the pages' default is 1/sqrt(D)
 *              (the Python binding passes that when scale is None).
 *   is_causal  0 or 1; 1 masks key j > query i (top-left aligned).
 *   dtype      MI355_ATTN_FP32, MI355_ATTN_BF16 or MI355_ATTN_FP16.
 *   stream     hipStream_t to enqueue on (NULL: null stream).
 *
 * Returns MI355_ATTN_OK, or:
 *   INVALID_ARG  a null pointer while B*H*M > 0; B, H or M < 0; N < 1 while
 *                B*H*M > 0; D < 1; non-finite scale; is_causal not 0/1; bad
 *                dtype; o or lse overlapping q, k, v or each other.
 *   UNSUPPORTED  D not in {16, 32, 64, 128}; a size whose element count or
 *                launch grid does not fit the kernels' index types.
 *   MISALIGNED   q, k, v or o not 16-byte aligned, or lse not 4-byte aligned.
 *   HIP_ERROR    the launch failed (hipGetLastError).
 * B*H*M == 0 returns OK without launching.
 */
int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
             int64_t B, int64_t H, int64_t M, int64_t N, int64_t D,
             float scale, int is_causal, int dtype, void *stream);

/*
 * attn_fwd_validate -- the status attn_fwd would return for these arguments
 * before launching (never HIP_ERROR). Makes no HIP call and dereferences no
 * pointer, so it is usable without a GPU.
 */
int attn_fwd_validate(const void *q, const void *k, const void *v, void *o,
                      const float *lse, int64_t B, int64_t H, int64_t M,
                      int64_t N, int64_t D, float scale, int is_causal,
                      int dtype);

/*
 * attn_fwd_path -- attn_fwd with an explicit kernel choice (one of the
 * MI355_ATTN_PATH_* values). PATH_AUTO is attn_fwd. PATH_SMALL on a shape the
 * small kernel cannot hold (see attn_fwd_select_path) returns UNSUPPORTED;
 * an unknown path value returns INVALID_ARG. Results of the two paths agree
 * to rounding; this exists so that each kernel can be checked on the same
 * inputs.
 */
int attn_fwd_path(const void *q, const void *k, const void *v, void *o,
                  float *lse, int64_t B, int64_t H, int64_t M, int64_t N,
                  int64_t D, float scale, int is_causal, int dtype, int path,
                  void *stream);

/*
 * attn_fwd_select_path -- which kernel PATH_AUTO runs for this problem
 * (MI355_ATTN_PATH_MAIN or MI355_ATTN_PATH_SMALL), or -1 if the sizes are
 * invalid or unsupported. The small kernel keeps a whole (batch, head)
 * sequence in the registers of one to four waves (one per 16 query rows):
 * it is chosen for M <= 64, N <= 64 and D <= 32. Pure host logic.
 */
int attn_fwd_select_path(int64_t B, int64_t H, int64_t M, int64_t N,
                         int64_t D, int is_causal, int dtype);

/*
 * attn_bwd -- gradient of attention with respect to q, k and v (the backward
 * of "Blackwell Attention Example": preprocess kernel, backward kernel and
 * autograd function sections). For the forward above and an upstream
 * gradient dO, with P_ij = exp(s_ij - L_i) (zero where masked):
 *
 *     delta_i = sum_d O[i,d] * dO[i,d]
 *     dV_j    = sum_i P_ij dO_i
 *     dS_ij   = P_ij (<dO_i, v_j> - delta_i)
 *     dQ_i    = scale * sum_j dS_ij k_j
 *     dK_j    = scale * sum_i dS_ij q_i
 *
 *   q, k, v    the forward's inputs (device, element type `dtype`).
 *   o, lse     the forward's outputs for the same q, k, v, scale and
 *              is_causal (attn_fwd's O and natural-log L).
 *   dout       upstream gradient dO, [B,H,M,D], element type `dtype`.
 *   dq         output [B,H,M,D]; dk, dv outputs [B,H,N,D]; element type
 *              `dtype`. Every element is written (dk, dv rows that no query
 *              sees get zeros).
 *   delta      caller-owned device workspace of B*H*M fp32 values; after the
 *              call's work completes it holds delta_i. Its prior contents are
 *              ignored.
 *   B, H, M, N, D, scale, is_causal, dtype, stream  as for attn_fwd, except
 *              that N may be 0 when M is 0.
 *
 * Enqueues two kernels on `stream` (dQ and delta first, then dK and dV) and
 * returns without synchronising; results are deterministic (no atomics).
 *
 * Returns MI355_ATTN_OK, or:
 *   INVALID_ARG  a null k, v, dk or dv while B*H*N > 0, or any null pointer
 *                while B*H*M > 0 (with M == 0 the query-side pointers are
 *                not used); B, H, M, N < 0; N < 1
 *                while B*H*M > 0; D < 1; non-finite scale; is_causal not 0/1;
 *                bad dtype; dq, dk, dv or delta overlapping an input or each
 *                other (inputs may alias).
 *   UNSUPPORTED  dtype MI355_ATTN_FP32 (bf16 and fp16 are supported); D not
 *                in {32, 64, 128}; a size whose
 *                element count or launch grid does not fit the kernels'
 *                index types.
 *   MISALIGNED   q, k, v, o, dout, dq, dk or dv not 16-byte aligned, or lse
 *                or delta not 4-byte aligned.
 *   HIP_ERROR    a launch failed (hipGetLastError).
 * B*H*(M+N) == 0 returns OK without launching.
 */
int attn_bwd(const void *q, const void *k, const void *v, const void *o,
             const float *lse, const void *dout, void *dq, void *dk, void *dv,
             float *delta, int64_t B, int64_t H, int64_t M, int64_t N,
             int64_t D, float scale, int is_causal, int dtype, void *stream);

/*
 * attn_bwd_validate -- the status attn_bwd would return for these arguments
 * before launching (never HIP_ERROR). No HIP call, no dereference.
 */
int attn_bwd_validate(const void *q, const void *k, const void *v,
                      const void *o, const float *lse, const void *dout,
                      const void *dq, const void *dk, const void *dv,
                      const float *delta, int64_t B, int64_t H, int64_t M,
                      int64_t N, int64_t D, float scale, int is_causal,
                      int dtype);

/*
 * attn_bwd_ws -- attn_bwd with a device work area, which lets it run the
 * backward in one pass over the keys ("Blackwell Attention Example",
 * backward kernel section: the key-tile loop that adds each tile's share of
 * dQ). Here the shares are added in a fixed order (key tile 0, 1, 2, ...)
 * instead of with atomics, so the results are the same on every run, like
 * attn_bwd's; S and dP are then formed once per (query, key) pair instead of
 * twice.
 *
 *   work, work_bytes  caller-owned device memory, 256-byte aligned, not
 *              overlapping any other argument; its prior contents are
 *              ignored and the call overwrites the first
 *              attn_bwd_work_bytes(...) bytes. Calls whose work may overlap
 *              in time (different streams) need different work areas.
 *   all other arguments as for attn_bwd.
 *
 * The one-pass path applies to bf16 and fp16 with D = 128, no causal mask,
 * B*H*M <= 2^30, M and N <= 2^24 and B*H*ceil(M/32) <= 2^26, on a device
 * whose XCD count
 * (hipDeviceAttributeNumberOfXccs) is 1, 2, 4 or 8; otherwise, or with
 * work == NULL or work_bytes below attn_bwd_work_bytes(...), the call is
 * exactly attn_bwd.
 * Enqueues two kernels on `stream` (delta, then the one-pass kernel). The
 * dQ, dK and dV it returns are deterministic but need not equal attn_bwd's
 * bit for bit (dQ is summed in another order).
 *
 * Returns what attn_bwd returns, or MISALIGNED (work not 256-byte aligned)
 * or INVALID_ARG (work overlapping another argument, work_bytes < 0) when
 * the one-pass path would run.
 */
int attn_bwd_ws(const void *q, const void *k, const void *v, const void *o,
                const float *lse, const void *dout, void *dq, void *dk, void *dv,
                float *delta, int64_t B, int64_t H, int64_t M, int64_t N,
                int64_t D, float scale, int is_causal, int dtype, void *work,
                int64_t work_bytes, void *stream);

/*
 * attn_bwd_work_bytes -- bytes of work area with which attn_bwd_ws runs its
 * one-pass path for these sizes (B*H*M*D*4 for the fp32 dQ sums, B*H*M*4 for
 * L in base 2, and counters), or 0 where that path does not apply. No HIP
 * call.
 */
int64_t attn_bwd_work_bytes(int64_t B, int64_t H, int64_t M, int64_t N,
                            int64_t D, int is_causal, int dtype);

/*
 * attn_bwd_work_error_offset -- byte offset in the work area of an int that
 * the one-pass kernel leaves at 0; it is non-zero only if a wait of that
 * kernel gave up (its spin limit) or the workgroups were not spread over the
 * XCDs as the launch assumes, in which case dQ is not valid. For tests and
 * diagnostics; reading it requires the call's work to have completed.
 * The waits assume that every key workgroup of a head gets a compute unit
 * within a bounded time: kernels that run concurrently on the same device
 * and hold its compute units for longer than the spin limit (about 10^6
 * polls, a fraction of a second) can make a wait give up.
 */
int attn_bwd_work_error_offset(void);

/*
 * attn_bwd_noalloc -- attn_bwd for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same arguments, results and errors as attn_bwd, without
 * the delta workspace: delta lives in a static device array of the library
 * that holds MI355_ATTN_NOALLOC_MAX_ROWS fp32 values (4 MiB), which every GPU
 * the library runs on keeps until the process ends. The call makes no
 * allocation of any kind; its first call on a device looks the array's
 * address up once (a HIP call, no allocation).
 *
 * B*H*M above MI355_ATTN_NOALLOC_MAX_ROWS returns MI355_ATTN_ERR_SCRATCH
 * (after every check attn_bwd makes, still before any HIP call) and
 * launches nothing. Every call on one GPU shares that GPU's array, which
 * keeps the last call's delta: calls whose work overlaps on one GPU (on
 * different streams) race and must be ordered by the caller. Nothing in the
 * array needs clearing: each call writes every value it reads.
 */
#define MI355_ATTN_NOALLOC_MAX_ROWS 1048576
int attn_bwd_noalloc(const void *q, const void *k, const void *v, const void *o,
                     const float *lse, const void *dout, void *dq, void *dk,
                     void *dv, int64_t B, int64_t H, int64_t M, int64_t N,
                     int64_t D, float scale, int is_causal, int dtype,
                     void *stream);

/*
 * attn_fwd_fp8 -- attn_fwd with fp8 inputs ("Blackwell Attention Example",
 * attention kernel: P is cast to the value dtype before the second product,
 * and fp8 values in their natural layout are noted there as Blackwell-only,
 * so fp8 V is taken transposed):
 *
 *   q          [B, H, M, D] OCP e4m3 (1 sign, 4 exponent bits with bias 7,
 *              3 mantissa bits; 0x7f / 0xff are NaN), device memory.
 *   k          [B, H, N, D] e4m3.
 *   vt         [B, H, D, N] e4m3: V transposed (vt[b,h,d,j] = v[b,h,j,d]).
 *   o          [B, H, M, D] bf16 output.
 *   lse        [B, H, M] fp32 output, natural log.
 *
 * Both products run in e4m3 with fp32 accumulation; P is rounded to e4m3
 * (nearest even) before the second one, and the row sum is taken from the
 * same rounded P, so O is an exact convex combination of value rows up to
 * fp32 accumulation; O is rounded to bf16 on the store. Scores, masking,
 * scale and L as attn_fwd. Supported: D in {64, 128} and N a multiple of 16
 * (else UNSUPPORTED); q, k, vt and o 16-byte aligned, lse 4-byte aligned
 * (MISALIGNED); o and lse must not overlap the inputs or each other
 * (INVALID_ARG). Other argument rules, ownership, execution and errors as
 * attn_fwd; B*H*M == 0 returns OK without launching.
 */
int attn_fwd_fp8(const void *q, const void *k, const void *vt, void *o, float *lse,
                 int64_t B, int64_t H, int64_t M, int64_t N, int64_t D,
                 float scale, int is_causal, void *stream);

/* attn_fwd_fp8_validate -- the checks of attn_fwd_fp8 without a launch. */
int attn_fwd_fp8_validate(const void *q, const void *k, const void *vt,
                          const void *o, const float *lse, int64_t B,
                          int64_t H, int64_t M, int64_t N, int64_t D,
                          float scale, int is_causal);

/* attn_fwd_dv -- attn_fwd with a value head dim Dv of its own ("Blackwell
 * Attention Example", attention kernel: v may be [.., N, Dv]):
 *
 *     O[b,h,i,:] = sum_j softmax(s)_j * v[b,h,j,:]      O is [B, H, M, Dv]
 *
 * with s and L exactly as attn_fwd. q and k are [B, H, M, D] / [B, H, N, D],
 * v is [B, H, N, Dv], o is [B, H, M, Dv], lse [B, H, M] fp32; layout,
 * ownership, execution and errors as attn_fwd. Dv == D is attn_fwd itself
 * (every dtype). Dv != D: every dtype, D and Dv each in {16, 32, 64, 128};
 * other head dims return MI355_ATTN_ERR_UNSUPPORTED.
 */
int attn_fwd_dv(const void *q, const void *k, const void *v, void *o, float *lse,
                int64_t B, int64_t H, int64_t M, int64_t N, int64_t D, int64_t Dv,
                float scale, int is_causal, int dtype, void *stream);

/* attn_fwd_dv_validate -- the checks of attn_fwd_dv without a launch. */
int attn_fwd_dv_validate(const void *q, const void *k, const void *v, void *o,
                         const float *lse, int64_t B, int64_t H, int64_t M,
                         int64_t N, int64_t D, int64_t Dv, float scale,
                         int is_causal, int dtype);

/* ------------------------------------------------------------------------
 * Fused axial-attention block (the PopcornBench axial-attention trajectory:
 * the model's reference forward and its per-pass attention helper).
 *
 * x and out are fp32 images [B, Hh, W, C], contiguous. One residual pass over
 * the sequences of one axis (MI355_AXIAL_ROW: each image row (b, y) is a
 * sequence of W tokens; MI355_AXIAL_COL: each image column (b, x) is a
 * sequence of Hh tokens) computes, for every token t of every sequence,
 *
 *     u    = LayerNorm(x_t) * ln_w + ln_b        biased variance, + eps
 *     q,k,v = split(u W_qkv^T)                   [3C] read as (3, heads, C/heads)
 *     a_h  = softmax_j(q_h . k_h,j / sqrt(C/heads)) v_h,j   per head, no mask
 *     out_t = x_t + concat_h(a_h) W_out^T + b_out
 *
 * with the weights stored as torch's linear layers store them: ln_w, ln_b
 * and b_out [C]; w_qkv [3C, C]; w_out [C, C] (row = output feature); all
 * fp32, caller-owned device memory. Supported: C = 64, heads = 4, and a
 * sequence length (W for rows, Hh for columns) of 1..64; other values return
 * MI355_ATTN_ERR_UNSUPPORTED. out may be x itself (in place); otherwise it
 * must not overlap x, and it never may overlap a weight. x, out, w_qkv,
 * w_out, ln_w and ln_b must be 16-byte aligned, b_out 4-byte aligned
 * (MI355_ATTN_ERR_MISALIGNED). eps must be finite and >= 0; B, Hh, W >= 0
 * (B * Hh * W = 0 is a no-op). Asynchronous on `stream`, like attn_fwd.
 */
#define MI355_AXIAL_ROW 0
#define MI355_AXIAL_COL 1

int axial_pass(const float *x, float *out, const float *ln_w, const float *ln_b,
               const float *w_qkv, const float *w_out, const float *b_out,
               int64_t B, int64_t Hh, int64_t W, int64_t C, int64_t heads,
               int axis, float eps, void *stream);

/* axial_pass_validate -- the checks of axial_pass without a launch. */
int axial_pass_validate(const float *x, const float *out, const float *ln_w,
                        const float *ln_b, const float *w_qkv, const float *w_out,
                        const float *b_out, int64_t B, int64_t Hh, int64_t W,
                        int64_t C, int64_t heads, int axis, float eps);

/* axial_pass_split -- workgroups per sequence of the launch axial_pass makes
 * for this image and axis: 2 when the pass has at most 128 sequences and
 * out != x (each of the two takes half of the query tokens and projects keys
 * and values for all of them), else 1. An in-place pass never splits: one
 * half would read tokens the other half has already overwritten. Returns -1
 * for an invalid axis, negative or empty sizes, or a sequence length above
 * 64. Pure host logic: no HIP call, no dereference. */
int axial_pass_split(const float *x, const float *out, int64_t B, int64_t Hh,
                     int64_t W, int axis);

/* axial_block -- the whole block: the row pass from x into out with the
 * row_* weights, then the column pass on out, in place, with the col_*
 * weights (the column pass attends over the row pass's result). Two
 * launches on `stream`; every argument rule of axial_pass applies to both
 * weight sets, and both sequence lengths must be 1..64. */
int axial_block(const float *x, float *out, const float *row_ln_w,
                const float *row_ln_b, const float *row_w_qkv,
                const float *row_w_out, const float *row_b_out,
                const float *col_ln_w, const float *col_ln_b,
                const float *col_w_qkv, const float *col_w_out,
                const float *col_b_out, int64_t B, int64_t Hh, int64_t W,
                int64_t C, int64_t heads, float eps, void *stream);

/* attn_status_string -- a static, NUL-terminated name for a status code
 * ("unknown status" for values outside the list above). */
const char *attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MI355_ATTN_H */
