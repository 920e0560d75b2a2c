/*
 * brq.h -- matrix products against binarized LLM weights on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libbrq.so. Every pointer argument named as device memory must be a
 * device (or device-accessible) pointer; every call enqueues its kernels on
 * `stream` (a hipStream_t passed as void*, NULL = the null stream) and returns
 * without synchronising the host. Buffers and workspaces are owned by the
 * caller; the library's own device memory is two arrays that every GPU it runs
 * on holds until the process ends: the scratch of brq_moe_ffn_noalloc
 * (BRQ_NOALLOC_SCRATCH_BYTES) and the wait counters of the single-launch
 * chains (brq_set_decode_fusion, 272 KiB). A call that returns a
 * status other than BRQ_OK has enqueued nothing and written nothing, except
 * BRQ_E_HIP, which reports a failed launch.
 *
 * Formats (the pages these follow are named at each call):
 *
 *  SIGN1 plane   -- uint64_t words, 64 signs per word; element k of a row is
 *                   bit (k % 64) of word (k / 64) of that row (least significant
 *                   bit first); bit 0 means +1 and bit 1 means -1, the IEEE 754
 *                   sign-bit convention ("LLM binarization, Episode 01: DBF",
 *                   sections 1 and 3).
 *  group-128     -- a SIGN1 plane plus one fp16 scale per run of 128 consecutive
 *                   weights of a row ("Behaviour-Relearned Quantization", item 02:
 *                   sign bits with one scale per 128 of them; "Banyan: Converting Pretrained
 *                   Language Models to 1-Bit Weights ...", Abstract: one sign per
 *                   weight and one shared scale per small group, 1.125 bits per
 *                   weight). Scale of row n, group g at index n*(cols/128) + g.
 *                   The dequantised weight is (bit ? -1 : +1) * scale.
 *  activations   -- bf16 (raw uint16 bits), row-major [rows][cols].
 *  outputs       -- bf16 or fp32 (brq_dtype), row-major. BRQ_BF16 is the fp32
 *                   result rounded to nearest, ties to even.
 *
 * Numerics: every product multiplies exactly representable operands and
 * accumulates in fp32; bf16 activations of any finite magnitude are accepted
 * (brq_dbf_gemm_q8 aside, which quantises them by definition). How each path
 * carries them:
 *  - brq_gemm, M = 1, K % 512 == 0, K <= 23040: fp8 x fp4 matrix cores; each
 *    activation is a 24-bit fixed-point field under the largest power of two
 *    of its slice of the row (a change of less than 2^-23 of that slice's
 *    maximum; bf16 subnormals count as zero), split into six 4-bit digits
 *    whose products and partial sums are exact;
 *  - the gate/up products of brq_moe_ffn on its grouped path (T > 4, H a
 *    multiple of 512 up to 8192): the same digit scheme per route and wave
 *    slice; the gate/up V factors of brq_moe_dbf_ffn (H a multiple of 512 up
 *    to 8192) and the first stage of brq_dbf_gemm for one row with n % 512
 *    == 0 (n <= 16384): the digit scheme on x_s = d_in * x (exact in fp32;
 *    an x_s below 2^-126 counts as zero), so that bits below 2^-23 of the
 *    slice's largest |x_s| are dropped;
 *  - brq_gemm with 9 <= M <= 64: bf16 matrix cores with +-1 weights (bf16
 *    activations as they are), each scale group's sum scaled in fp32;
 *  - every other product on the fp16 matrix cores takes the activations as
 *    fp16(x * 2^s), s a power of two per row (per staged slice of a row on the
 *    few-row paths) that puts the largest |x| in [2^14, 2^15) when it lies
 *    outside [2^-8, 2^15), else 0, undone exactly after the product; every
 *    staged value of at least 2^-17 is then exact, smaller ones move by at
 *    most 2^-25 (at most 2^-17 of the row maximum);
 *  - fp32 intermediates (DBF h_s, the MoE SwiGLU output) are stored as fp32
 *    and enter the next product as two fp16 pieces of v * 2^s (s as above for
 *    the staged slice or row, the largest near 2^14): about 22 significant
 *    bits for every value down to 2^-18 of that maximum.
 * The paths differ only in fp32 rounding order, so one row gives the same
 * result to fp32 rounding at any M. Results are deterministic (sums in a
 * fixed order, no floating-point atomics). Inputs must be finite.
 *
 * Alignment: weight planes, scales and activation rows must be 16-byte
 * aligned; workspaces 256-byte aligned.
 *
 * Errors: each call validates its arguments on the host before touching the
 * device, and returns a brq_status; brq_last_error() gives a thread-local text
 * for the last non-OK status of the calling thread. Calls never abort.
 */
#ifndef BRQ_H
#define BRQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BRQ_ABI_VERSION 1
#define BRQ_GROUP 128

typedef enum {
  BRQ_OK = 0,
  BRQ_E_NULL = 1,      /* a required pointer is NULL                                  */
  BRQ_E_SHAPE = 2,     /* a size is out of range or not the multiple the format needs */
  BRQ_E_ALIGN = 3,     /* a pointer is not aligned as stated above                    */
  BRQ_E_DTYPE = 4,     /* unknown output dtype                                        */
  BRQ_E_WORKSPACE = 5, /* workspace NULL, misaligned or smaller than its size query   */
  BRQ_E_DEVICE = 6,    /* no current HIP device, or it is not gfx950                  */
  BRQ_E_HIP = 7        /* a HIP runtime call or a kernel launch failed                */
} brq_status;

typedef enum { BRQ_BF16 = 0, BRQ_F32 = 1 } brq_dtype;

/* Version of this header's ABI (BRQ_ABI_VERSION). */
int brq_abi_version(void);

/* Status name, e.g. "BRQ_E_SHAPE". Never NULL. */
const char* brq_status_str(brq_status s);

/* Text describing the last non-OK status returned on the calling thread
   ("" if none). Valid until the next brq_* call on the same thread. */
const char* brq_last_error(void);

/*
 * brq_set_decode_fusion -- single-launch decode chains ("LLM binarization,
 * Episode 01: DBF", section 7: a joint V - D_mid - U kernel with one grid-wide
 * synchronisation between the products, and a persistent MoE kernel running
 * gate/up, SwiGLU and down in one launch). brq_dbf_gemm with M <= 8 and
 * brq_moe_ffn / brq_moe_ffn_noalloc with T <= 4 can each run as one launch
 * whose workgroups (all resident on the device at once) wait for one another
 * once, instead of two launches. The result bits are the same either way,
 * except brq_dbf_gemm with M = 1 and n % 512 == 0, whose multi-launch first
 * stage takes the fp8 x fp4 digit path (see Numerics) and the single launch
 * the fp16 one: both meet the same bound, not the same bits.
 *
 *   mode        BRQ_FUSION_DEFAULT: the library's choice per path, the one
 *               that measured faster on MI355X (today the multi-launch path
 *               everywhere: the grid-wide wait costs about what a kernel
 *               boundary inside a HIP graph does); BRQ_FUSION_OFF: always the
 *               multi-launch path; BRQ_FUSION_ON: one launch wherever all its
 *               workgroups fit the device at once.
 *   spin_limit  polls of the grid-wide wait before a workgroup gives up (0:
 *               the default, 2^22, about a second); a wait that gives up
 *               writes NaN to the outputs that workgroup owns. It ends only
 *               when the device cannot run all workgroups of the launch at
 *               once (see below).
 * Process-wide; applies to calls issued after it returns. A single-launch
 * chain needs all its workgroups resident at once: a caller that runs two of
 * them concurrently on one device (two streams), or one beside a kernel that
 * holds compute units until it ends, can see that wait give up.
 * BRQ_E_SHAPE for an unknown mode.
 */
typedef enum { BRQ_FUSION_DEFAULT = 0, BRQ_FUSION_OFF = 1, BRQ_FUSION_ON = 2 } brq_fusion;
brq_status brq_set_decode_fusion(brq_fusion mode, uint32_t spin_limit);

/*
 * brq_debug_fail_launches -- test hook for callers' error handling: the next
 * `count` calls of the process whose arguments pass validation return
 * BRQ_E_HIP ("injected launch failure") instead of enqueueing their kernels;
 * they enqueue and write nothing. 0 disarms it. BRQ_E_SHAPE if count < 0.
 */
brq_status brq_debug_fail_launches(int32_t count);

/* Number of uint64_t words of a SIGN1 plane of rows x cols (cols % 64 == 0). */
size_t brq_sign_words(int64_t rows, int64_t cols);

/* Number of fp16 scales of a group-128 matrix of rows x cols (cols % 128 == 0). */
size_t brq_scale_count(int64_t rows, int64_t cols);

/*
 * brq_pack -- quantise fp32 weights to the group-128 format, or to a bare SIGN1
 * plane.
 *
 * Follows "Behaviour-Relearned Quantization" (item 02), "Banyan ..." (Abstract)
 * and "LLM binarization, Episode 01: DBF" (sections 1 and 3). For row n and
 * group g: bit[n,k] = sign bit of w[n,k]; scale[n,g] = mean of |w[n,k]| over
 * the 128 k of group g, accumulated in fp64 and rounded once to fp16 (nearest,
 * ties to even). mean|w| is the least-squares optimum of
 * ||w - a*sign(w)||^2 over a.
 *
 *   w       device, fp32 [rows][cols], row-major, 16-byte aligned
 *   signs   device, out, brq_sign_words(rows, cols) words
 *   scales  device, out, brq_scale_count(rows, cols) fp16 (raw bits), or NULL
 *           to write the SIGN1 plane alone (the DBF factors carry no scale)
 *   rows >= 1; cols % 128 == 0 when scales != NULL, else cols % 64 == 0.
 */
brq_status brq_pack(const float* w, int64_t rows, int64_t cols,
                    uint64_t* signs, uint16_t* scales, void* stream);

/*
 * brq_gemm -- y[m][n] = sum_k x[m][k] * Wq[n][k]  (y = x . Wq^T), where Wq is
 * the dequantised group-128 matrix [N][K]: the activation x binary-weight
 * product ("Banyan ...", Abstract; "LLM binarization, Episode 01: DBF",
 * section 1: a binary weight selects x or -x).
 *
 *   x       device, bf16 [M][K]
 *   signs   device, SIGN1 plane of W [N][K]; scales device, fp16 [N][K/128],
 *           each a non-negative finite value (the mean magnitude of its group,
 *           as brq_pack writes it; the sign of a weight lives in its bit)
 *   y       device, out, [M][N] of y_dtype
 *   ws      device workspace of at least brq_gemm_workspace_bytes(M, N, K)
 *           bytes (may be NULL when that size is 0)
 *   M >= 1, N >= 1, K >= 128 and K % 128 == 0.
 */
size_t brq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
brq_status brq_gemm(const uint16_t* x, int64_t M, int64_t N, int64_t K,
                    const uint64_t* signs, const uint16_t* scales,
                    void* y, brq_dtype y_dtype,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * brq_gemm_lr -- y = x . (Wq + U V)^T = x . Wq^T + (x . V^T) . U^T: the
 * binary product plus a rank-r correction of the weights (BWLA commentary,
 * section 4: the residual left by binarisation is approximated by a
 * truncated SVD and added to the binarised weights; rank about 0.5% of the
 * dimension, ~20 for 4096).
 *
 *   x, signs, scales, y   as for brq_gemm
 *   v       device, fp16 [r][K] (row i: the i-th right factor)
 *   u       device, fp16 [N][r]
 *   ws      device workspace of at least brq_gemm_lr_workspace_bytes(M, N, K, r)
 *   1 <= r <= 64; M, N, K as for brq_gemm. x . V^T must stay inside the fp16
 *   range (it is carried as an fp16 hi/lo pair on the many-row path).
 * For M > 64 the correction runs on the matrix cores inside the product's
 * epilogue (one extra k-step per tile); for M <= 64 it is added to the fp32
 * product before the output is written. One rounding to y_dtype either way.
 */
size_t brq_gemm_lr_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r);
brq_status brq_gemm_lr(const uint16_t* x, int64_t M, int64_t N, int64_t K,
                       const uint64_t* signs, const uint16_t* scales,
                       const uint16_t* v, const uint16_t* u, int64_t r,
                       void* y, brq_dtype y_dtype,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * brq_dbf_gemm -- the Double Binary Factorization chain
 *   y = D_out . U . D_mid . V . D_in . x   (one output row per row of x)
 * evaluated in the deployed order x_s = D_in x; h = V x_s; h_s = D_mid h;
 * y_core = U h_s; y = D_out y_core ("LLM binarization, Episode 01: DBF",
 * section 1 for the representation, section 4 for the order and the record
 * din / v / dmid / u / dout). h and h_s are kept in fp32.
 *
 *   x      device, bf16 [M][n]
 *   d_in   device, fp16 [n];  v device, SIGN1 plane of V [r][n]
 *   d_mid  device, fp16 [r];  u device, SIGN1 plane of U [m][r]
 *   d_out  device, fp16 [m]   (the three diagonals are real-valued: either sign)
 *   y      device, out, [M][m] of y_dtype
 *   ws     device workspace, >= brq_dbf_workspace_bytes(M, m, n, r)
 *   M >= 1; m >= 1; n, r >= 128 and multiples of 128.
 */
size_t brq_dbf_workspace_bytes(int64_t M, int64_t m, int64_t n, int64_t r);
brq_status brq_dbf_gemm(const uint16_t* x, int64_t M, int64_t m, int64_t n, int64_t r,
                        const uint16_t* d_in, const uint64_t* v, const uint16_t* d_mid,
                        const uint64_t* u, const uint16_t* d_out,
                        void* y, brq_dtype y_dtype,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * brq_dbf_gemm_q8 -- the same DBF chain as brq_dbf_gemm with both binary
 * products taken over sign-magnitude Q8 activation codes, the prompt-side
 * formulation of "LLM binarization, Episode 01: DBF" (section 5, item 4: one
 * exponent per reduction row, a sign and seven magnitude bits, an exact
 * integer reduction against the weight signs, then one shared scale; item 1
 * names the same integer as a signed int8 dot product against +-1 weights).
 * Per row of the product's input v (x_s = D_in x, exact in fp32, for V; h_s
 * for U): e = the smallest integer with max|v| <= 127 * 2^e (0 for an all-zero
 * row); q = round-half-to-even(v / 2^e), |q| <= 127. Then
 *   h   = (q1 . V^T) * 2^e1            (an exact integer times a power of two)
 *   h_s = fp32(d_mid * h)              (one fp32 rounding)
 *   y   = d_out * (q2 . U^T) * 2^e2    (one fp32 rounding, then y_dtype)
 * The codes and exponents are decided in fp32, where every input to them is
 * exact, so they match an fp64 evaluation of the same definition bit for bit.
 * Arguments and layouts are those of brq_dbf_gemm, with n and r at most
 * 131072 (so that 127 * n < 2^24 and every integer sum is exact in fp32). The
 * workspace holds the two code planes, the row exponents, h_s (fp32 [M][r])
 * and, when few output tiles split the reductions along k, their int32
 * partial sums (added exactly, in any order).
 * Alignment: x, v, u, d_in and d_mid 16 bytes; y 4 bytes; d_out 2 bytes.
 */
size_t brq_dbf_q8_workspace_bytes(int64_t M, int64_t m, int64_t n, int64_t r);
brq_status brq_dbf_gemm_q8(const uint16_t* x, int64_t M, int64_t m, int64_t n, int64_t r,
                           const uint16_t* d_in, const uint64_t* v, const uint16_t* d_mid,
                           const uint64_t* u, const uint16_t* d_out,
                           void* y, brq_dtype y_dtype,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * brq_moe_ffn -- routed mixture-of-experts SwiGLU layer on group-128 experts:
 *   for each token t: ids = the top_k experts by descending fp32 router logit
 *   (ties to the lower expert index); w = softmax over the top_k selected
 *   logits; y_t = sum_j w_j * Wd_e (silu(Wg_e x_t) * (Wu_e x_t)), e = ids_j,
 *   silu(z) = z / (1 + exp(-z)).
 * Each (token, slot) route carries an expert id and a route weight; gate/up
 * share the token's hidden vector across its experts, down consumes the
 * route's own intermediate ("LLM binarization, Episode 01: DBF", section 4).
 * 256 experts with 8 routed and an f32 router is the layer of the "BTL-4
 * Compact" news item. The sum over slots is taken in slot order (deterministic).
 *
 *   x        device, bf16 [T][H];  logits device, fp32 [T][E]
 *   gate_s / up_s    device, SIGN1 planes [E][I][H/64]; gate_sc / up_sc fp16 [E][I][H/128]
 *   down_s           device, SIGN1 plane [E][H][I/64];   down_sc fp16 [E][H][I/128]
 *                    (scales non-negative and finite, as for brq_gemm)
 *   y        device, out, [T][H] of y_dtype
 *   ids, w   device, out, [T][top_k] int32 / fp32, or NULL
 *   ws       device workspace, >= brq_moe_workspace_bytes(T, H, I, E, top_k)
 *   1 <= T <= 256; 1 <= top_k <= min(E, 16); 1 <= E <= 1024;
 *   H, I multiples of 128 with H <= 32768 and I <= 2048.
 */
size_t brq_moe_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t top_k);
brq_status brq_moe_ffn(const uint16_t* x, const float* logits,
                       int64_t T, int64_t H, int64_t I, int64_t E, int64_t top_k,
                       const uint64_t* gate_s, const uint16_t* gate_sc,
                       const uint64_t* up_s, const uint16_t* up_sc,
                       const uint64_t* down_s, const uint16_t* down_sc,
                       void* y, brq_dtype y_dtype,
                       int32_t* ids, float* w,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * brq_moe_ffn_noalloc -- brq_moe_ffn without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, serving
 * loops, harnesses that forbid hipMalloc). The workspace is a scratch array of
 * BRQ_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends; the call allocates nothing.
 *
 *   arguments as for brq_moe_ffn, minus ws and ws_bytes
 *   BRQ_E_WORKSPACE when brq_moe_workspace_bytes(T, H, I, E, top_k) exceeds
 *   BRQ_NOALLOC_SCRATCH_BYTES (16 MiB: e.g. T <= 64 at H = 4096, I = 2048,
 *   top_k = 8); every other status as for brq_moe_ffn.
 * All calls on one GPU share its array: calls that overlap on one GPU (two
 * streams, two host threads) race and must be serialised by the caller.
 */
#define BRQ_NOALLOC_SCRATCH_BYTES (16u << 20)
brq_status brq_moe_ffn_noalloc(const uint16_t* x, const float* logits,
                               int64_t T, int64_t H, int64_t I, int64_t E, int64_t top_k,
                               const uint64_t* gate_s, const uint16_t* gate_sc,
                               const uint64_t* up_s, const uint16_t* up_sc,
                               const uint64_t* down_s, const uint16_t* down_sc,
                               void* y, brq_dtype y_dtype,
                               int32_t* ids, float* w, void* stream);

/*
 * One DBF chain record (the five tensors of a routed expert projection,
 * "LLM binarization, Episode 01: DBF", section 4): for E experts of an m x n
 * projection with inner dimension r,
 *   d_in  fp16 [E][n];  v  SIGN1 [E][r][n/64];  d_mid fp16 [E][r];
 *   u     SIGN1 [E][m][r/64];  d_out fp16 [E][m]  (diagonals of either sign).
 */
typedef struct {
  const uint16_t* d_in;
  const uint64_t* v;
  const uint16_t* d_mid;
  const uint64_t* u;
  const uint16_t* d_out;
} brq_dbf_factors;

/*
 * brq_moe_dbf_ffn -- the routed SwiGLU layer of brq_moe_ffn with every routed
 * gate, up and down projection a DBF chain y = D_out U D_mid V D_in x, each
 * evaluated in the deployed order (DBF post, section 4: the deployed model
 * converts its routed experts to DBDBD with r = 1024 on 512 x 2048 gate/up and
 * 2048 x 512 down). Routing as in brq_moe_ffn. gate/up first factors consume
 * the token's hidden vector shared by its experts; second factors and the down
 * chain consume the route's own intermediates (section 4's two input
 * topologies). Intermediates are fp32, taken by the next product as scaled
 * fp16 pieces (see Numerics above).
 *
 *   x, logits, T, E, top_k, y, ids, w   as for brq_moe_ffn
 *   gate, up   host pointers to records of H -> I chains (m = I, n = H)
 *   down       host pointer to a record of an I -> H chain (m = H, n = I)
 *   ws       device workspace, >= brq_moe_dbf_workspace_bytes(T, H, I, E, top_k, r)
 *   H, I, r multiples of 128 with H <= 8192, I <= 2048, r <= 2048; T, E, top_k
 *   as for brq_moe_ffn. x, y, the sign planes and d_in 16-byte aligned, d_mid
 *   and d_out 2-byte aligned.
 */
size_t brq_moe_dbf_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t top_k, int64_t r);
brq_status brq_moe_dbf_ffn(const uint16_t* x, const float* logits,
                           int64_t T, int64_t H, int64_t I, int64_t E, int64_t top_k, int64_t r,
                           const brq_dbf_factors* gate, const brq_dbf_factors* up,
                           const brq_dbf_factors* down,
                           void* y, brq_dtype y_dtype,
                           int32_t* ids, float* w,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * brq_kron_rotate -- Kronecker-factored orthogonal activation rotation
 *   x'_t = (H (x) R) x_t, computed as X'_t = H . X_t . R^T where X_t is row t
 *   of x reshaped row-major to [n1][n2]
 * (BWLA commentary: section 3, OKT with Kronecker factors H and R, n1*n2 = n;
 * section 5, the same orthogonal transform applied to the activations so that
 * the product with the correspondingly rotated weights is unchanged).
 * fp32 arithmetic; the output is rounded to bf16 (nearest, ties to even).
 *
 *   x   device, bf16 [M][n1*n2];  H device, fp32 [n1][n1];  R device, fp32 [n2][n2]
 *   y   device, out, bf16 [M][n1*n2]; must not overlap x
 *   M >= 1; n1 and n2 each 32, 64 or 96 with n1 * n2 <= 6144 (rows of 1024,
 *   2048, 3072, 4096 or 6144 values; the prefill workload is 64 x 64); other
 *   factor sizes (e.g. 48, which 3072 = 48 x 64 would need, or 96 x 96) give
 *   BRQ_E_SHAPE.
 *   Errors: BRQ_E_NULL (a NULL pointer), BRQ_E_SHAPE (M or factor sizes out
 *   of range, x and y overlapping), BRQ_E_ALIGN (x or y not 16-byte aligned,
 *   H or R not 4-byte aligned).
 */
brq_status brq_kron_rotate(const uint16_t* x, int64_t M, const float* H, int64_t n1,
                           const float* R, int64_t n2, uint16_t* y, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* BRQ_H */
