// Internal helpers shared by the libbt kernels (gfx950 / CDNA4, wave64).
//
// Packed weight layout (matches the public description in bt.h):
//   chunk (rb, c) = rows 64*rb .. +63, k = 64*c .. +63, 1024 bytes at
//   ((rb * KC) + c) * 1024 with KC = Kp / 64. Row r of a chunk is one uint4 at
//   uint4 index ((rb * KC) + c) * 64 + r. Word j of that uint4 holds codes for
//   k = 64c + 16j + b, b = 0..15, code b at bit 8*(b&3) + 2*(b>>2); code = t + 1.
//
// Why this bit order: masking a word with 0x03030303 << 2s (s = 0..2), or
// (word >> 2) & 0x30303030 for s = 3, leaves four int8 lanes that each hold one
// code of four CONSECUTIVE k (k = 64c + 16j + 4s + e, byte e), times 4^s (s <= 2)
// or 16 (s = 3). Each such dword feeds one v_dot4 / one MFMA operand dword
// against the matching dword of int8 activations without any shift, and the
// per-mask accumulators are recombined exactly as a1 + (a4 >> 2) + (a16 >> 4).
// With offset codes (t + 1 in {0,1,2}) the bytes are non-negative and small
// (<= 32), so the signed int8 dot product is exact; the "+1" is removed at the
// end by subtracting sum_k q (computed once per token by the quantizer).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

namespace bt {

constexpr int kRowsPerChunk = 64;   // weight rows per packed chunk (one per lane)
constexpr int kKPerChunk = 64;      // k per packed chunk (16 bytes per row)
constexpr uint32_t kPadWord = 0x55555555u;  // sixteen codes "1" = sixteen zero weights

constexpr uint32_t kMask0 = 0x03030303u;  // codes b = e        (weight 1)
constexpr uint32_t kMask1 = 0x0C0C0C0Cu;  // codes b = 4 + e    (weight 4)
constexpr uint32_t kMask2 = 0x30303030u;  // codes b = 8 + e    (weight 16); also (w>>2) for b = 12+e

typedef int v4i __attribute__((ext_vector_type(4)));

__host__ __device__ inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Wave-uniform value the compiler can keep in an SGPR.
__device__ inline int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Row groups of bt_pack_weights_rows: group g covers rows end[g-1] .. end[g]-1 (end[-1] = 0).
constexpr int kMaxRowGroups = 8;
struct RowGroups {
    int64_t end[kMaxRowGroups];
    int n;
};

// Launchers (each returns hipGetLastError() after the launch).
hipError_t launch_pack(const float *W, int64_t N, int64_t K, uint4 *Wp, float *gamma, double *rowsum,
                       hipStream_t s);
// Row-group scales into row_scale[N]; groups == NULL: one group per row.
hipError_t launch_pack_rows(const float *W, int64_t N, int64_t K, const RowGroups *groups, uint4 *Wp,
                            float *row_scale, double *rowsum, hipStream_t s);
hipError_t launch_unpack(const uint4 *Wp, int64_t N, int64_t K, int8_t *T, hipStream_t s);
// The quantizer also zero-fills `clear_words` 32-bit words at `clear` (split-K arrival
// counters of the product that follows it; NULL / 0 for none).
hipError_t launch_quant_act(const float *X, int64_t M, int64_t K, int64_t ldq, int8_t *Xq, float *sx,
                            int32_t *xsum, unsigned *clear, int64_t clear_words, hipStream_t s);
// The product launchers take the weight scale as w_scale[0] (row_scales false) or as
// one scale per output row, w_scale[n] (row_scales true).
hipError_t launch_gemv_dot4(const uint4 *Wp, const float *w_scale, bool row_scales, const int8_t *Xq, int64_t ldq,
                            const float *sx, const int32_t *xsum, int64_t M, int64_t N, int64_t K, float *Y,
                            int32_t *acc, hipStream_t s);
hipError_t launch_gemv_mfma(const uint4 *Wp, const float *w_scale, bool row_scales, const int8_t *Xq, int64_t ldq,
                            const float *sx, const int32_t *xsum, int64_t M, int64_t N, int64_t K, float *Y,
                            int32_t *acc, hipStream_t s);
// 1-bit activations: binary weights (pack, W1A1 GEMV), activation bits (layout 1: plain,
// 2: aligned with the ternary codes) and the ternary-weight W1.58A1 GEMV.
int64_t act_bits_words(int64_t K, int layout);
hipError_t launch_pack_binary(const float *W, int64_t N, int64_t K, uint4 *Wb, float *w_scale, float *rowmax,
                              hipStream_t s);
hipError_t launch_binarize(const float *X, int64_t M, int64_t K, int layout, uint32_t *Xb, float *sx, hipStream_t s);
hipError_t launch_gemv_binary(const uint4 *Wb, const float *w_scale, const uint32_t *Xb, const float *sx, int64_t M,
                              int64_t N, int64_t K, float *Y, int32_t *acc, hipStream_t s);
hipError_t launch_gemv_ternary_a1(const uint4 *Wp, const float *w_scale, const uint32_t *Xb, const float *sx,
                                  int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc, hipStream_t s);
// Table-lookup GEMV for one token; the LDS bytes its tables take.
hipError_t launch_gemv_lut(const uint4 *Wp, const float *w_scale, bool row_scales, const int8_t *Xq,
                           const float *sx, const int32_t *xsum, int64_t N, int64_t K, float *Y, int32_t *acc,
                           hipStream_t s);
size_t gemv_lut_lds_bytes(int64_t K);
// Pre-quantized activations staged in LDS (1 <= M <= 16 with the int8 rows within 128 KB).
bool gemv_staged_fits(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemv_staged(const uint4 *Wp, const float *w_scale, bool row_scales, const int8_t *Xq,
                              const float *sx, const int32_t *xsum, int64_t M, int64_t N, int64_t K, float *Y,
                              int32_t *acc, hipStream_t s);
// Fused decode (quantize + product + epilogue) for M <= 4; LDS bytes it needs.
hipError_t launch_linear_decode(const uint4 *Wp, const float *w_scale, bool row_scales, const float *X, int64_t M,
                                int64_t N, int64_t K, float *Y, int32_t *acc, hipStream_t s);
size_t decode_fused_lds_bytes(int64_t M, int64_t N, int64_t K);
// Prefill GEMM. With a workspace of at least gemm_workspace_bytes(M, N, K) bytes whose
// first gemm_arrival_words(M, N, K) words are zero, shapes that gain from it split the K
// range of their tiles after the first `full` over `nsplit` workgroups each (gemm_plan;
// the words are zero again afterwards); otherwise (NULL or smaller workspace) one
// workgroup per tile.
struct GemmPlan {
    int64_t full;  // tiles computed whole (the first ones of the tile order)
    int nsplit;    // workgroups per later tile; 1: no split at all
};
GemmPlan gemm_plan(int64_t M, int64_t N, int64_t K);
int64_t gemm_tiles(int64_t M, int64_t N);  // 64 x 256 output tiles
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
int64_t gemm_arrival_words(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm(const uint4 *Wp, const float *w_scale, bool row_scales, const int8_t *Xq, int64_t ldq,
                       const float *sx, const int32_t *xsum, int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc,
                       void *workspace, size_t workspace_bytes, hipStream_t s);

// Names of the kernel instances the launchers pick for a call (host-only, snprintf
// semantics; 16-byte aligned activation rows assumed), for bt_kernel_plan.
int plan_quant_act(int64_t M, int64_t K, char *buf, size_t len);
int plan_linear_decode(int64_t M, int64_t N, int64_t K, bool row_scales, char *buf, size_t len);
int plan_gemv_staged(int64_t M, int64_t N, int64_t K, bool row_scales, char *buf, size_t len);
int plan_gemv_mfma(int64_t M, int64_t N, int64_t K, bool row_scales, char *buf, size_t len);
int plan_gemm(int64_t M, int64_t N, int64_t K, bool row_scales, bool split_workspace, char *buf, size_t len);

}  // namespace bt
