/*
 * bt.h -- C ABI of libbt.so, the MI355X (gfx950) BitNet b1.58 W1.58A8 ternary
 * linear layer.
 *
 * The method (BitNet b1.58, as described on the pages this library follows):
 *   weights   W [N,K] fp32 -> gamma = mean|W| (one fp32 scale per matrix) and
 *             t = RoundClip(W / gamma, -1, 1) in {-1, 0, +1}, packed 2 bits each;
 *   inputs    X [M,K] fp32 -> per token m: a = max_k |X[m,k]|,
 *             q = clamp(rint(X * (127 / a)), -127, 127) int8, s_x = a / 127;
 *   product   acc[m,n] = sum_k t[n,k] * q[m,k] in int32 (add, subtract or skip);
 *   output    Y[m,n] = fp32(acc[m,n]) * (gamma * s_x[m]).
 * Every integer result (codes, q, sum q, acc) is exact; Y carries two fp32 roundings.
 *
 * Conventions shared by every entry point:
 *  - All array arguments are DEVICE pointers owned by the caller; the library never
 *    allocates, frees or keeps them. Scales stay on the device (no host readback).
 *  - `stream` is a hipStream_t (NULL = the null stream). Work is only enqueued:
 *    calls return before the GPU finishes, never synchronize, and can be captured
 *    into a HIP graph. A fault inside a kernel surfaces at the caller's next sync.
 *  - Arguments are validated on the host before any HIP call; on failure nothing
 *    is enqueued and a non-zero bt_status is returned (bt_last_error() says why).
 *  - Matrices are row-major. M = tokens, N = output features (rows of W),
 *    K = input features. 0 <= M, N <= BT_MAX_DIM; 0 <= K <= BT_MAX_K; products
 *    also M * N <= BT_MAX_MN (every launch then stays within 2^32 work-items).
 *    Larger shapes fail with BT_ERR_SHAPE. M == 0 or N == 0 is a no-op.
 *  - Non-finite inputs are outside the contract; the results are then unspecified
 *    (but the kernels still stay in bounds).
 *  - Calls on different streams may run concurrently; a call reads only its
 *    inputs and writes only its outputs. The library holds no mutable global state
 *    other than a thread-local error string.
 *  - Row-group weight scales (the "_rows" / "_rs" entry points): the rows of W may be
 *    cut into groups that each get the absmean scale of their own rows (the Q, K and
 *    V blocks of a fused projection, or one group per row). The scale then travels as
 *    an array of N fp32 values, one per output row, and Y[m,n] uses entry n. Integer
 *    results are computed exactly as with one scale per matrix.
 */
#ifndef BT_H
#define BT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t bt_status;

#define BT_OK 0
#define BT_ERR_NULL 1        /* a required pointer is NULL (or both outputs are) */
#define BT_ERR_SHAPE 2       /* a dimension is negative or above its limit      */
#define BT_ERR_UNSUPPORTED 3 /* valid arguments the chosen kernel cannot take    */
#define BT_ERR_ALIGN 4       /* a pointer lacks the alignment stated below      */
#define BT_ERR_HIP 5         /* the HIP runtime rejected a launch               */

/* K is bounded so that |acc| <= 127*K < 2^24: acc then converts to fp32 exactly. */
#define BT_MAX_K 131072
/* Largest M and N: 2^23 (8.4 M tokens or output features). */
#define BT_MAX_DIM 8388608LL
/* Largest M * N of a product: 2^36 (a 256 GiB fp32 output). */
#define BT_MAX_MN 68719476736LL
/* Largest token count the decode GEMV entry point accepts. */
#define BT_GEMV_MAX_M 16
/* Largest number of explicit row groups bt_pack_weights_rows takes. */
#define BT_MAX_ROW_GROUPS 8

/* Decode GEMV kernel choices for bt_ternary_gemv_algo. */
#define BT_GEMV_AUTO 0 /* BT_GEMV_STAGED (BT_GEMV_MFMA when K == 0)                 */
#define BT_GEMV_DOT4 1 /* one lane per weight row, v_dot4 with the x chunk in SGPRs */
#define BT_GEMV_MFMA 2 /* int8 MFMA 16x16x64, 64 weight rows per wave             */
#define BT_GEMV_STAGED 4 /* int8 MFMA with the int8 activations staged per workgroup in
                            LDS: whole rows once where M * (K rounded up to 256) <=
                            131072 bytes, else in K-blocks through two LDS buffers
                            (any K up to BT_MAX_K, M <= 16) */
#define BT_GEMV_LUT 3  /* table lookup (T-MAC / TL1 style): M == 1 only, and K small
                          enough for its LDS tables (16 bytes per k; the device's
                          per-workgroup LDS limit), else BT_ERR_UNSUPPORTED      */

/*
 * Packed weight layout (the library's own format, produced by bt_pack_weights):
 *   Np = N rounded up to 64, Kp = K rounded up to 64. The matrix is cut into
 *   1024-byte chunks of 64 rows x 64 k; chunk (rb, c) covers rows 64*rb .. +63 and
 *   k = 64*c .. +63 and starts at byte ((rb * Kp/64) + c) * 1024. Row r of the chunk
 *   is the 16 bytes at offset 16*r, i.e. 4 little-endian 32-bit words; word j holds
 *   the 16 codes of k = 64*c + 16*j + b (b = 0..15), code b at bits
 *   8*(b%4) + 2*(b/4) .. +1. A code is t + 1 (0 = -1, 1 = 0, 2 = +1). Padding
 *   rows and columns hold code 1 (weight 0). Size: Np * Kp / 4 bytes.
 */
size_t bt_packed_weight_bytes(int64_t N, int64_t K);

/* Row stride, in bytes, of the int8 activation matrix Xq: K rounded up to 256 (one
 * k-step of the product kernels). Bytes k >= K of each row are zero (bt_quant_act
 * writes them), so the kernels never guard the k tail of an activation row. */
int64_t bt_act_row_bytes(int64_t K);

/* Workspace, in bytes, that bt_pack_weights needs (fp64 per-row |W| sums). */
size_t bt_pack_workspace_bytes(int64_t N, int64_t K);

/*
 * bt_pack_weights -- absmean ternarization and 2-bit packing of one weight matrix
 * (once per matrix, offline). Follows the "bit-floor" page, "What's inside"
 * (pack.rs: mean-abs threshold zero-suppression for ternary weights) and the
 * "BitCompute" page, "Future Roadmap" (four 1.58-bit weights per byte).
 *   W         [N,K] fp32, row-major, 16-byte aligned, read only.
 *   Wp        output, bt_packed_weight_bytes(N,K) bytes, 16-byte aligned.
 *   w_scale   output, one fp32: gamma = fp32(sum_n sum_k |W| / (N*K)) where each
 *             row is summed k = 0..K-1 in fp64 and the row sums n = 0..N-1 in fp64
 *             (this fixed order makes gamma reproducible bit for bit).
 *             Codes: t = +1 if w > gamma/2, -1 if w < -gamma/2, else 0.
 *   workspace bt_pack_workspace_bytes(N,K) bytes of device scratch, 8-byte aligned;
 *             contents on entry are ignored; it may be reused after the call's
 *             kernels complete (stream order).
 * N == 0 or K == 0 writes gamma = 0 and nothing else.
 */
bt_status bt_pack_weights(const float *W, int64_t N, int64_t K, void *Wp, float *w_scale,
                          void *workspace, void *stream);

/*
 * bt_pack_weights_rows -- bt_pack_weights with row-group scales. Follows the BitNet GPU
 * guide, "Frequently Asked Questions" (the kernel wrapper assumes model-specific
 * quantization scales and group dimensions): here a group is a run of output rows that
 * was one matrix of the model (fused Q/K/V, fused gate/up), or a single row.
 *   group_rows  HOST array of ngroups row counts (each >= 1, summing to N), in row
 *               order, 1 <= ngroups <= BT_MAX_ROW_GROUPS; or NULL for one group per
 *               row (ngroups ignored).
 *   row_scale   output, N fp32 on the device: row n receives its group's scale,
 *               computed like bt_pack_weights' gamma over the group's rows alone (each
 *               row summed k = 0..K-1 in fp64, the group's row sums in row order in
 *               fp64, one division, one rounding to fp32). Codes of row n use
 *               row_scale[n] / 2 as the threshold.
 *   W, Wp, workspace   as for bt_pack_weights (same layout and workspace size).
 * With K == 0 every scale is 0. Errors: BT_ERR_SHAPE when the groups do not cover the
 * N rows exactly or a group is empty; otherwise those of bt_pack_weights.
 */
bt_status bt_pack_weights_rows(const float *W, int64_t N, int64_t K, const int64_t *group_rows,
                               int64_t ngroups, void *Wp, float *row_scale, void *workspace,
                               void *stream);

/*
 * bt_unpack_weights -- inverse of the packing (a test and inspection aid):
 *   T [N,K] int8 receives t in {-1, 0, +1}. Wp 16-byte aligned.
 */
bt_status bt_unpack_weights(const void *Wp, int64_t N, int64_t K, int8_t *T, void *stream);

/*
 * bt_quant_act -- fused per-token absmax int8 quantization, one pass per token.
 * Follows the BitNet GPU guide ("How to Run BitNet Inference on GPU Using CUDA
 * Kernels"), section "Understanding the Two-Phase Architecture" (inputs quantized
 * to INT8 with their own scales before the INT8 x INT2 kernel), and the "bit-floor"
 * page, "What's inside" (scale.rs: absmax, quantized before each GEMV).
 *   X        [M,K] fp32 row-major, 4-byte aligned (16-byte aligned rows are faster).
 *   Xq       output [M, bt_act_row_bytes(K)] int8, 16-byte aligned; bytes k >= K
 *            of every row are written as 0.
 *   x_scale  output [M] fp32: s_x = a / 127 (fp32 division), 0 for an all-zero row.
 *   x_sum    output [M] int32: sum_k q[m,k] (needed by the GEMV/GEMM).
 * q = clamp(rint(x * inv), -127, 127) with inv = 127.0f / a (correctly rounded fp32
 * division, fp32 multiply, round half to even); an all-zero row gives q = 0.
 */
bt_status bt_quant_act(const float *X, int64_t M, int64_t K, int8_t *Xq, float *x_scale,
                       int32_t *x_sum, void *stream);

/*
 * bt_ternary_gemv -- decode product for 1 <= M <= BT_GEMV_MAX_M tokens: the integer
 * ternary dot product with the scale epilogue fused. Follows the "bit-floor" page,
 * "The core math" (integer inner loop, one floating-point scale multiply at the end)
 * and the "BitCompute" page, "Features" (ternary weights make the product add /
 * subtract / skip).
 *   Wp       packed weights from bt_pack_weights(N, K).
 *   w_scale  device pointer to gamma.
 *   Xq, x_scale, x_sum   from bt_quant_act(M, K) (Xq rows of bt_act_row_bytes(K)
 *            bytes with zero padding).
 *   Y        output [M,N] fp32 or NULL; Y[m,n] = fp32(acc) * (gamma * s_x[m]).
 *   acc      output [M,N] int32 or NULL: the exact accumulator sum_k t*q.
 *   Y and acc may not both be NULL. Y and acc need 4-byte alignment. With K == 0
 *   (an empty dot product: acc = 0) Wp and Xq may be NULL.
 * Returns BT_ERR_UNSUPPORTED for M > BT_GEMV_MAX_M (use bt_ternary_gemm).
 */
bt_status bt_ternary_gemv(const void *Wp, const float *w_scale, const int8_t *Xq,
                          const float *x_scale, const int32_t *x_sum, int64_t M, int64_t N,
                          int64_t K, float *Y, int32_t *acc, void *stream);

/* bt_ternary_gemv with an explicit kernel choice (BT_GEMV_AUTO / _DOT4 / _MFMA / _STAGED / _LUT).
 * BT_GEMV_DOT4 takes M <= 4, BT_GEMV_LUT M == 1; all return bit-identical acc and Y.
 * The table-lookup kernel follows the "Run 100B Models on Your Laptop CPU" page, "What is
 * Microsoft BitNet?" (kernels on T-MAC's lookup-table method) and "Key Features That Make
 * BitNet Insane" (the TL1 / TL2 ternary lookup kernels). */
bt_status bt_ternary_gemv_algo(const void *Wp, const float *w_scale, const int8_t *Xq,
                               const float *x_scale, const int32_t *x_sum, int64_t M, int64_t N,
                               int64_t K, float *Y, int32_t *acc, int32_t algo, void *stream);

/* bt_ternary_gemv_algo with row scales: row_scale[N] (from bt_pack_weights_rows) in
 * place of w_scale, Y[m,n] = fp32(acc) * (row_scale[n] * s_x[m]). Same passages as
 * bt_ternary_gemv, plus the GPU guide's FAQ on model-specific scales. */
bt_status bt_ternary_gemv_rs(const void *Wp, const float *row_scale, const int8_t *Xq,
                             const float *x_scale, const int32_t *x_sum, int64_t M, int64_t N,
                             int64_t K, float *Y, int32_t *acc, int32_t algo, void *stream);

/*
 * bt_ternary_gemm -- prefill product for any M >= 1 on int8 MFMA: the packed
 * weight tiles are unpacked in registers straight into MFMA operands, the int8
 * activation tiles are staged in LDS, and the scale epilogue is fused. Shapes with
 * K >= 512 and at most 256 output tiles of 64 x 64 (e.g. a few hundred tokens) split
 * each tile's K range over the four waves of its workgroup and sum the parts in LDS;
 * others take 64 x 256 tiles. Same arguments and results as bt_ternary_gemv, with no
 * limit on M. Follows the BitNet
 * GPU guide, "Key Components and Source Code Architecture" (prefill is the
 * compute-bound phase) and the "BitCompute" page, "Future Roadmap" (moving the
 * ternary product onto the matrix cores).
 */
bt_status bt_ternary_gemm(const void *Wp, const float *w_scale, const int8_t *Xq,
                          const float *x_scale, const int32_t *x_sum, int64_t M, int64_t N,
                          int64_t K, float *Y, int32_t *acc, void *stream);

/*
 * bt_ternary_gemm_ws -- bt_ternary_gemm with a caller workspace that lets shapes whose
 * output tiles alone would leave most of the GPU idle (few tokens, or few output
 * columns with long rows) split the k-range of every tile over several workgroups. The
 * splits hand their int32 partial tiles over through the workspace and the last one to
 * finish adds them up and runs the epilogue, so acc and Y are bit-identical to
 * bt_ternary_gemm (integer partial sums, one scale multiply at the end). Follows the
 * same passages as bt_ternary_gemm.
 *   workspace        NULL (no split), or device memory of workspace_bytes bytes,
 *                    256-byte aligned. The split route runs only when workspace_bytes >=
 *                    bt_gemm_workspace_bytes(M, N, K) > 0; otherwise the call is
 *                    bt_ternary_gemm.
 *   Ownership        the caller owns the workspace. It must be zero-filled once before
 *                    its first use (its leading words are per-tile arrival counters);
 *                    every completed call leaves them zero again. Calls that share a
 *                    workspace must not run concurrently.
 * Errors are those of bt_ternary_gemm, plus BT_ERR_ALIGN for a misaligned workspace.
 */
size_t bt_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
/*
 * bt_gemm_split_plan -- how bt_ternary_gemm_ws spreads an M x N x K product over
 * workgroups when given its workspace (host-only query, no device call). Output tiles are
 * 64 tokens x 256 weight rows; the first *full_tiles of the library's tile order are
 * computed whole and each later one is split over *splits workgroups (each over a
 * contiguous share of K). The shapes that bt_ternary_gemm splits inside its workgroups
 * (see there) report every tile whole. *splits == 1: no split (bt_gemm_workspace_bytes is then 0);
 * *full_tiles == 0 with *splits > 1: every tile is split. The workspace's leading
 * (tiles - *full_tiles) 32-bit words are the arrival counters of the split tiles.
 *   full_tiles, splits   host pointers, written on BT_OK.
 * Errors: BT_ERR_NULL, BT_ERR_SHAPE (negative or oversized M, N or K).
 */
bt_status bt_gemm_split_plan(int64_t M, int64_t N, int64_t K, int64_t *full_tiles, int32_t *splits);
bt_status bt_ternary_gemm_ws(const void *Wp, const float *w_scale, const int8_t *Xq,
                             const float *x_scale, const int32_t *x_sum, int64_t M, int64_t N,
                             int64_t K, float *Y, int32_t *acc, void *workspace,
                             size_t workspace_bytes, void *stream);

/* bt_ternary_gemm_ws with row scales: row_scale[N] (from bt_pack_weights_rows) in place
 * of w_scale, Y[m,n] = fp32(acc) * (row_scale[n] * s_x[m]); workspace as for
 * bt_ternary_gemm_ws (NULL: no split). Same passages as bt_ternary_gemm, plus the GPU
 * guide's FAQ on model-specific scales. */
bt_status bt_ternary_gemm_rs(const void *Wp, const float *row_scale, const int8_t *Xq,
                             const float *x_scale, const int32_t *x_sum, int64_t M, int64_t N,
                             int64_t K, float *Y, int32_t *acc, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * bt_ternary_linear -- the whole per-call path of the layer in one entry point:
 * fp32 activations in, fp32 outputs out (per-token absmax int8 quantization, the
 * integer ternary product and the scale epilogue). Follows the BitNet GPU guide,
 * "Understanding the Two-Phase Architecture" (the kernel-backed linear layer
 * quantizes its inputs to INT8 and calls the INT8 x INT2 product) and "Key
 * Components and Source Code Architecture" (decode is memory-bound: one launch per
 * layer keeps the per-call latency down).
 *   X          [M,K] fp32 row-major, 4-byte aligned.
 *   Y, acc     as for bt_ternary_gemv (either may be NULL, not both).
 *   workspace  bt_linear_workspace_bytes(M,N,K) bytes of device scratch, 256-byte
 *              aligned, or NULL when that size is 0. No initialization is needed: the
 *              call writes every part it reads (for M > BT_GEMV_MAX_M it includes the
 *              split-K workspace of bt_ternary_gemm_ws, whose counters the quantizer
 *              launch zero-fills). Calls sharing a workspace must not overlap.
 * For M <= 4 tokens with M * K <= 32768 the quantizer runs inside the decode kernel
 * (one launch, no workspace); otherwise the
 * call runs bt_quant_act into the workspace, then bt_ternary_gemv or
 * bt_ternary_gemm. Both routes give results bit-identical to calling bt_quant_act
 * and bt_ternary_gemv / bt_ternary_gemm yourself.
 */
size_t bt_linear_workspace_bytes(int64_t M, int64_t N, int64_t K);
bt_status bt_ternary_linear(const void *Wp, const float *w_scale, const float *X, int64_t M,
                            int64_t N, int64_t K, float *Y, int32_t *acc, void *workspace,
                            void *stream);

/* bt_ternary_linear with row scales: row_scale[N] (from bt_pack_weights_rows) in place of
 * w_scale; the same routes, workspace (bt_linear_workspace_bytes) and errors. Same
 * passages as bt_ternary_linear, plus the GPU guide's FAQ on model-specific scales. */
bt_status bt_ternary_linear_rs(const void *Wp, const float *row_scale, const float *X, int64_t M,
                               int64_t N, int64_t K, float *Y, int32_t *acc, void *workspace,
                               void *stream);

/*
 * bt_ternary_linear_static -- bt_ternary_linear that allocates nothing and takes no
 * workspace: for callers that cannot allocate device memory or pass one in (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation). Where
 * bt_ternary_linear needs a workspace (bt_linear_workspace_bytes(M, N, K) > 0) this call
 * uses a scratch array of BT_STATIC_SCRATCH_BYTES bytes that the library holds on every
 * GPU it runs on until the process ends (its address is looked up once per device, on the
 * first such call there). The caller still owns X, Y and acc.
 *   Arguments, routes and results are those of bt_ternary_linear: bit-identical outputs.
 *   Limit: bt_linear_workspace_bytes(M, N, K) <= BT_STATIC_SCRATCH_BYTES, else
 *   BT_ERR_UNSUPPORTED and nothing is enqueued (2B-class prefill at 2048 tokens needs about
 *   31 MB of it).
 *   Concurrency: every call on one GPU shares that GPU's scratch. Calls whose kernels may
 *   overlap (different streams, or other host threads) race and give undefined results;
 *   serialize them (one stream, or events). A call writes all the scratch it reads before
 *   reading it (the quantizer zero-fills the GEMM's arrival counters), so no clearing is
 *   needed between calls.
 */
#define BT_STATIC_SCRATCH_BYTES 67108864LL
bt_status bt_ternary_linear_static(const void *Wp, const float *w_scale, const float *X, int64_t M, int64_t N,
                                   int64_t K, float *Y, int32_t *acc, void *stream);

/*
 * 1-bit activations: the binary GEMV (W1A1) and ternary weights against binarized
 * tokens (W1.58A1). Follows the "bit-floor" page, "The core math" (binary GEMV =
 * 2 * POPCNT(XNOR(W, x)) - K over packed sign bits; ternary GEMV = POPCNT(mag &
 * XNOR(sign, x)) - POPCNT(mag & XOR(sign, x)) over a magnitude and a sign plane) and
 * "What's inside" (pack.rs: absmax scale for binary weights; scale.rs: activations
 * binarized before each GEMV). A value v binarizes to +1 when v >= 0 and to -1 when
 * v < 0; a set bit means -1 in every plane.
 *
 * Bit layouts of the activations (rows of bt_act_bits_row_bytes(K, layout) bytes, bits
 * past K clear):
 *   BT_BITS_PLAIN  bit b of 32-bit word i is k = 32 i + b (for bt_binary_gemv);
 *   BT_BITS_CODES  word i holds k = 16 i + b at bit 8 (b % 4) + 2 (b / 4), where code b's
 *                  low bit sits in a packed ternary word (for bt_ternary_gemv_a1, which
 *                  reads the weights of bt_pack_weights as they are).
 */
#define BT_BITS_PLAIN 1
#define BT_BITS_CODES 2

/* Binary weight layout: chunks of 64 rows x 128 k, 1024 bytes, chunk (rb, c) at byte
 * ((rb * ceil(K/128)) + c) * 1024; row r of the chunk is the 16 bytes at 16 r; 32-bit word
 * j holds k = 128 c + 32 j + b at bit b; padding bits clear. Size Np * Kp / 8 bytes with
 * Np = N rounded up to 64, Kp = K rounded up to 128. */
size_t bt_binary_weight_bytes(int64_t N, int64_t K);
int64_t bt_act_bits_row_bytes(int64_t K, int32_t layout);

/* bt_pack_weights_binary -- sign bits of W [N,K] fp32 (row-major, 4-byte aligned) into
 * Wb (bt_binary_weight_bytes(N,K) bytes, 16-byte aligned) and w_scale[0] = max |W|
 * (exact). workspace: bt_pack_workspace_bytes(N,K) bytes, 8-byte aligned. N, K > 0. */
bt_status bt_pack_weights_binary(const float *W, int64_t N, int64_t K, void *Wb, float *w_scale,
                                 void *workspace, void *stream);

/* bt_binarize_act -- per token m: x_scale[m] = max_k |X[m,k]| (exact) and the sign bits
 * of the row in `layout` into Xb (M rows of bt_act_bits_row_bytes(K, layout) bytes,
 * 16-byte aligned). M, K > 0. */
bt_status bt_binarize_act(const float *X, int64_t M, int64_t K, int32_t layout, uint32_t *Xb,
                          float *x_scale, void *stream);

/* bt_binary_gemv -- W1A1 for 1 <= M <= BT_GEMV_MAX_M tokens: acc[m,n] = sum_k
 * sign(W[n,k]) sign(X[m,k]) = K - 2 * popcount(Wb_n xor Xb_m) (int32, exact) and
 * Y[m,n] = fp32(acc) * (w_scale[0] * x_scale[m]). Wb from bt_pack_weights_binary, Xb
 * from bt_binarize_act with BT_BITS_PLAIN. Y or acc may be NULL, not both. */
bt_status bt_binary_gemv(const void *Wb, const float *w_scale, const uint32_t *Xb,
                         const float *x_scale, int64_t M, int64_t N, int64_t K, float *Y,
                         int32_t *acc, void *stream);

/* bt_ternary_gemv_a1 -- W1.58A1 for 1 <= M <= BT_GEMV_MAX_M tokens: acc[m,n] = sum_k
 * t[n,k] sign(X[m,k]) (int32, exact), from the packed ternary weights of bt_pack_weights
 * and Xb from bt_binarize_act with BT_BITS_CODES; Y[m,n] = fp32(acc) * (gamma *
 * x_scale[m]), gamma = w_scale[0]. Y or acc may be NULL, not both. */
bt_status bt_ternary_gemv_a1(const void *Wp, const float *w_scale, const uint32_t *Xb,
                             const float *x_scale, int64_t M, int64_t N, int64_t K, float *Y,
                             int32_t *acc, void *stream);

/*
 * bt_kernel_plan -- the kernel instances a call would launch, as text (a host-only query:
 * no device call, nothing enqueued). For checking which specialisations a workload runs,
 * e.g. that every one of them is covered by a test. The activation rows are taken to be
 * 16-byte aligned (the fused and quantizer kernels pick their register path from that).
 *   call        BT_CALL_LINEAR (bt_ternary_linear / _rs), BT_CALL_GEMV (bt_ternary_gemv_algo /
 *               _rs with `algo`), BT_CALL_GEMM (bt_ternary_gemm, no workspace) or
 *               BT_CALL_GEMM_WS (bt_ternary_gemm_ws / _rs with a workspace of
 *               bt_gemm_workspace_bytes(M, N, K) bytes) or BT_CALL_QUANT (bt_quant_act).
 *   M, N, K     the call's shape (N is ignored for BT_CALL_QUANT); algo is read for
 *               BT_CALL_GEMV only; row_scales != 0 for the _rs entry points.
 *   buf, len    host buffer receiving a NUL-terminated text (truncated to len - 1 bytes):
 *               the kernels in launch order joined by " + ", each as name<template
 *               arguments>; empty when the call launches nothing (M == 0 or N == 0).
 * Errors: BT_ERR_NULL (buf), BT_ERR_SHAPE, BT_ERR_UNSUPPORTED -- those the call itself
 * would return for the shape and kernel choice.
 */
#define BT_CALL_LINEAR 0
#define BT_CALL_GEMV 1
#define BT_CALL_GEMM 2
#define BT_CALL_GEMM_WS 3
#define BT_CALL_QUANT 4
bt_status bt_kernel_plan(int32_t call, int64_t M, int64_t N, int64_t K, int32_t algo, int32_t row_scales,
                         char *buf, size_t len);

/* Static text for a status code. */
const char *bt_status_str(bt_status s);

/* Text of the last error on the calling thread ("" if none). */
const char *bt_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BT_H */
