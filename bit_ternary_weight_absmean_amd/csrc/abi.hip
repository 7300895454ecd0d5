// C ABI of libbt.so: argument validation, kernel selection and status codes.
// Every check runs on the host before any HIP call, so a rejected call enqueues
// nothing. The library allocates nothing and keeps no pointer past a call.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "bt.h"
#include "bt_internal.h"

// Scratch of bt_ternary_linear_static: one copy per GPU, held by the loaded library until
// the process ends. Host code never passes `scratch` itself to a kernel (in host code the
// name stands for a host-side shadow); it uses the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[BT_STATIC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512];

bt_status fail(bt_status code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

bt_status ok()
{
    g_err[0] = '\0';
    return BT_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bt_status hip_status(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return fail(BT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

bt_status check_k(int64_t K)
{
    if (K < 0 || K > BT_MAX_K)
        return fail(BT_ERR_SHAPE, "K = %lld outside [0, %d]", (long long)K, BT_MAX_K);
    return BT_OK;
}

// Weight-matrix shapes: N rows of K, at most BT_MAX_MN elements.
bt_status check_nk(int64_t N, int64_t K)
{
    if (N < 0 || N > BT_MAX_DIM)
        return fail(BT_ERR_SHAPE, "N = %lld outside [0, 2^23]", (long long)N);
    if (bt_status s = check_k(K))
        return s;
    if (N * K > BT_MAX_MN)
        return fail(BT_ERR_SHAPE, "N * K = %lld above 2^36", (long long)(N * K));
    return BT_OK;
}

// Common validation of the GEMV / GEMM arguments.
bt_status check_product(const void *Wp, const float *w_scale, const int8_t *Xq, const float *x_scale,
                        const int32_t *x_sum, int64_t M, int64_t N, int64_t K, const float *Y, const int32_t *acc)
{
    if (M < 0 || N < 0)
        return fail(BT_ERR_SHAPE, "negative shape M = %lld, N = %lld", (long long)M, (long long)N);
    if (bt_status s = check_k(K))
        return s;
    if (N > BT_MAX_DIM || M > BT_MAX_DIM)
        return fail(BT_ERR_SHAPE, "M = %lld or N = %lld above 2^23", (long long)M, (long long)N);
    if (M * N > BT_MAX_MN)
        return fail(BT_ERR_SHAPE, "M * N = %lld above 2^36", (long long)(M * N));
    if (!Y && !acc)
        return fail(BT_ERR_NULL, "Y and acc are both NULL");
    if (M == 0 || N == 0)
        return BT_OK;
    // With K == 0 there are no weight or activation bytes: Wp and Xq may be NULL.
    if (!w_scale || !x_scale || !x_sum || (K > 0 && (!Wp || !Xq)))
        return fail(BT_ERR_NULL, "NULL input pointer");
    if ((Wp && !aligned(Wp, 16)) || (Xq && !aligned(Xq, 16)))
        return fail(BT_ERR_ALIGN, "Wp and Xq must be 16-byte aligned");
    if (!aligned(w_scale, 4) || !aligned(x_scale, 4) || !aligned(x_sum, 4) || (Y && !aligned(Y, 4)) ||
        (acc && !aligned(acc, 4)))
        return fail(BT_ERR_ALIGN, "scale, sum and output arrays must be 4-byte aligned");
    return BT_OK;
}

}  // namespace

extern "C" {

size_t bt_packed_weight_bytes(int64_t N, int64_t K)
{
    if (N <= 0 || K <= 0)
        return 0;
    return (size_t)(bt::round_up(N, 64) * bt::round_up(K, 64) / 4);
}

int64_t bt_act_row_bytes(int64_t K) { return K <= 0 ? 0 : bt::round_up(K, 256); }

size_t bt_pack_workspace_bytes(int64_t N, int64_t K)
{
    if (N <= 0 || K <= 0)
        return 0;
    return (size_t)bt::round_up(N * 8, 256);
}

bt_status bt_pack_weights(const float *W, int64_t N, int64_t K, void *Wp, float *w_scale, void *workspace,
                          void *stream)
{
    if (bt_status s = check_nk(N, K))
        return s;
    if (!w_scale)
        return fail(BT_ERR_NULL, "w_scale is NULL");
    if (!aligned(w_scale, 4))
        return fail(BT_ERR_ALIGN, "w_scale must be 4-byte aligned");
    const bool empty = (N == 0 || K == 0);
    if (!empty) {
        if (!W || !Wp || !workspace)
            return fail(BT_ERR_NULL, "NULL W, Wp or workspace");
        if (!aligned(W, 16) || !aligned(Wp, 16))
            return fail(BT_ERR_ALIGN, "W and Wp must be 16-byte aligned");
        if (!aligned(workspace, 8))
            return fail(BT_ERR_ALIGN, "workspace must be 8-byte aligned");
    }
    return hip_status(bt::launch_pack(W, N, K, static_cast<uint4 *>(Wp), w_scale, static_cast<double *>(workspace),
                                      static_cast<hipStream_t>(stream)),
                      "bt_pack_weights launch");
}

bt_status bt_pack_weights_rows(const float *W, int64_t N, int64_t K, const int64_t *group_rows, int64_t ngroups,
                               void *Wp, float *row_scale, void *workspace, void *stream)
{
    if (bt_status s = check_nk(N, K))
        return s;
    bt::RowGroups groups{};
    if (group_rows) {
        if (ngroups < 1 || ngroups > BT_MAX_ROW_GROUPS)
            return fail(BT_ERR_SHAPE, "ngroups = %lld outside [1, %d]", (long long)ngroups, BT_MAX_ROW_GROUPS);
        int64_t end = 0;
        for (int64_t g = 0; g < ngroups; ++g) {
            if (group_rows[g] < 1)
                return fail(BT_ERR_SHAPE, "group %lld has %lld rows", (long long)g, (long long)group_rows[g]);
            end += group_rows[g];
            if (end > N)
                break;
            groups.end[g] = end;
        }
        if (end != N)
            return fail(BT_ERR_SHAPE, "the row groups cover %lld rows, not N = %lld", (long long)end, (long long)N);
        groups.n = (int)ngroups;
    }
    if (N == 0)
        return ok();
    if (!W && K > 0)
        return fail(BT_ERR_NULL, "NULL W");
    if (!row_scale || (K > 0 && (!Wp || !workspace)))
        return fail(BT_ERR_NULL, "NULL Wp, row_scale or workspace");
    if ((W && !aligned(W, 16)) || (Wp && !aligned(Wp, 16)))
        return fail(BT_ERR_ALIGN, "W and Wp must be 16-byte aligned");
    if (!aligned(row_scale, 4) || (workspace && !aligned(workspace, 8)))
        return fail(BT_ERR_ALIGN, "row_scale must be 4-byte aligned, workspace 8-byte aligned");
    return hip_status(bt::launch_pack_rows(W, N, K, group_rows ? &groups : nullptr, static_cast<uint4 *>(Wp),
                                           row_scale, static_cast<double *>(workspace),
                                           static_cast<hipStream_t>(stream)),
                      "bt_pack_weights_rows launch");
}

bt_status bt_unpack_weights(const void *Wp, int64_t N, int64_t K, int8_t *T, void *stream)
{
    if (bt_status s = check_nk(N, K))
        return s;
    if (N == 0 || K == 0)
        return ok();
    if (!Wp || !T)
        return fail(BT_ERR_NULL, "NULL Wp or T");
    if (!aligned(Wp, 16))
        return fail(BT_ERR_ALIGN, "Wp must be 16-byte aligned");
    return hip_status(bt::launch_unpack(static_cast<const uint4 *>(Wp), N, K, T, static_cast<hipStream_t>(stream)),
                      "bt_unpack_weights launch");
}

bt_status bt_quant_act(const float *X, int64_t M, int64_t K, int8_t *Xq, float *x_scale, int32_t *x_sum,
                       void *stream)
{
    if (M < 0 || M > BT_MAX_DIM)
        return fail(BT_ERR_SHAPE, "M = %lld outside [0, 2^23]", (long long)M);
    if (bt_status s = check_k(K))
        return s;
    if (M == 0)
        return ok();
    if (!x_scale || !x_sum || (K > 0 && (!X || !Xq)))
        return fail(BT_ERR_NULL, "NULL X, Xq, x_scale or x_sum");
    if ((X && !aligned(X, 4)) || !aligned(x_scale, 4) || !aligned(x_sum, 4))
        return fail(BT_ERR_ALIGN, "X, x_scale and x_sum must be 4-byte aligned");
    if (Xq && !aligned(Xq, 16))
        return fail(BT_ERR_ALIGN, "Xq must be 16-byte aligned");
    return hip_status(bt::launch_quant_act(X, M, K, bt_act_row_bytes(K), Xq, x_scale, x_sum, nullptr, 0,
                                           static_cast<hipStream_t>(stream)),
                      "bt_quant_act launch");
}

// The products and the linear layer, with the weight scale as w_scale[0] (rows false)
// or one scale per output row, w_scale[n] (rows true). The row-scale array needs the same
// 4-byte alignment; its N entries are not otherwise checked.
static bt_status gemv_impl(const void *Wp, const float *w_scale, bool rows, const int8_t *Xq, const float *x_scale,
                           const int32_t *x_sum, int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc,
                           int32_t algo, void *stream)
{
    if (bt_status s = check_product(Wp, w_scale, Xq, x_scale, x_sum, M, N, K, Y, acc))
        return s;
    if (M > BT_GEMV_MAX_M)
        return fail(BT_ERR_UNSUPPORTED, "gemv takes M <= %d (got %lld); use bt_ternary_gemm", BT_GEMV_MAX_M,
                    (long long)M);
    if (algo != BT_GEMV_AUTO && algo != BT_GEMV_DOT4 && algo != BT_GEMV_MFMA && algo != BT_GEMV_LUT &&
        algo != BT_GEMV_STAGED)
        return fail(BT_ERR_UNSUPPORTED, "unknown gemv algo %d", (int)algo);
    if (M == 0 || N == 0)
        return ok();
    if (algo == BT_GEMV_AUTO)
        // Measured on the 2B, 7B and 100B decode shapes at 1 to 16 tokens: staging the
        // int8 rows in LDS once per workgroup beats re-reading them per step (k_gemv_direct)
        // by 20-30% at every size that fits whole, and rows too long for that are staged in
        // K-blocks (k_gemv_blocked).
        algo = BT_GEMV_STAGED;
    if (algo == BT_GEMV_STAGED && K == 0)
        algo = BT_GEMV_MFMA;
    if (algo == BT_GEMV_DOT4 && M > 4)
        return fail(BT_ERR_UNSUPPORTED, "dot4 gemv takes M <= 4 (got %lld)", (long long)M);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (algo == BT_GEMV_LUT) {
        if (M != 1)
            return fail(BT_ERR_UNSUPPORTED, "lut gemv takes M == 1 (got %lld)", (long long)M);
        int dev = 0, lds_max = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
            return fail(BT_ERR_HIP, "cannot query the LDS limit");
        if (bt::gemv_lut_lds_bytes(K) + 1024 > (size_t)lds_max)
            return fail(BT_ERR_UNSUPPORTED, "lut gemv tables for K = %lld need %zu bytes of LDS (limit %d)",
                        (long long)K, bt::gemv_lut_lds_bytes(K), lds_max);
        if (K == 0)
            return gemv_impl(Wp, w_scale, rows, Xq, x_scale, x_sum, M, N, K, Y, acc, BT_GEMV_MFMA, stream);
    }
    const int64_t ldq = bt_act_row_bytes(K);
    const uint4 *W = static_cast<const uint4 *>(Wp);
    hipError_t e = (algo == BT_GEMV_DOT4)
                       ? bt::launch_gemv_dot4(W, w_scale, rows, Xq, ldq, x_scale, x_sum, M, N, K, Y, acc, s)
                   : (algo == BT_GEMV_STAGED)
                       ? bt::launch_gemv_staged(W, w_scale, rows, Xq, x_scale, x_sum, M, N, K, Y, acc, s)
                   : (algo == BT_GEMV_LUT)
                       ? bt::launch_gemv_lut(W, w_scale, rows, Xq, x_scale, x_sum, N, K, Y, acc, s)
                       : bt::launch_gemv_mfma(W, w_scale, rows, Xq, ldq, x_scale, x_sum, M, N, K, Y, acc, s);
    return hip_status(e, "bt_ternary_gemv launch");
}

static bt_status gemm_impl(const void *Wp, const float *w_scale, bool rows, const int8_t *Xq, const float *x_scale,
                           const int32_t *x_sum, int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc,
                           void *workspace, size_t workspace_bytes, void *stream)
{
    if (bt_status s = check_product(Wp, w_scale, Xq, x_scale, x_sum, M, N, K, Y, acc))
        return s;
    if (workspace && !aligned(workspace, 256))
        return fail(BT_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (M == 0 || N == 0)
        return ok();
    const int64_t ldq = bt_act_row_bytes(K);
    return hip_status(bt::launch_gemm(static_cast<const uint4 *>(Wp), w_scale, rows, Xq, ldq, x_scale, x_sum, M, N,
                                      K, Y, acc, workspace, workspace ? workspace_bytes : 0,
                                      static_cast<hipStream_t>(stream)),
                      "bt_ternary_gemm launch");
}

// Largest LDS footprint the fused decode kernel is launched with.
static const size_t kFusedLdsLimit = 64 * 1024;

// The fused kernel re-reads and re-quantizes all M fp32 token rows in every workgroup.
// Measured on the 2B, 7B and 100B decode shapes: that beats a separate quantizer launch
// plus the GEMV up to 4 tokens of up to 8192 values (M * K <= 32768; against the staged
// GEMV at M = 4: 2B 0.60 vs 0.73 ms per step, 7B 0.90 vs 1.01 ms, 100B even), and loses
// beyond (7B at M = 8, 7B down at M = 4).
static bool linear_fused(int64_t M, int64_t N, int64_t K)
{
    return M <= 4 && M * K <= 32768 && bt::decode_fused_lds_bytes(M, N, K) <= kFusedLdsLimit;
}

// Workspace of the unfused route: [Xq | x_scale | x_sum | split-K GEMM workspace], each
// part 256-byte aligned.
static size_t linear_quant_bytes(int64_t M, int64_t K)
{
    return (size_t)(bt::round_up(M * bt_act_row_bytes(K), 256) + 2 * bt::round_up(4 * M, 256));
}

static bt_status linear_impl(const void *Wp, const float *w_scale, bool rows, const float *X, int64_t M, int64_t N,
                             int64_t K, float *Y, int32_t *acc, void *workspace, void *stream)
{
    if (M < 0 || N < 0 || M > BT_MAX_DIM || N > BT_MAX_DIM)
        return fail(BT_ERR_SHAPE, "shape M = %lld, N = %lld out of range", (long long)M, (long long)N);
    if (M * N > BT_MAX_MN)
        return fail(BT_ERR_SHAPE, "M * N = %lld above 2^36", (long long)(M * N));
    if (bt_status s = check_k(K))
        return s;
    if (!Y && !acc)
        return fail(BT_ERR_NULL, "Y and acc are both NULL");
    if (M == 0 || N == 0)
        return ok();
    if (!w_scale || (K > 0 && (!Wp || !X)))
        return fail(BT_ERR_NULL, "NULL input pointer");
    if ((Wp && !aligned(Wp, 16)) || (X && !aligned(X, 4)) || !aligned(w_scale, 4) || (Y && !aligned(Y, 4)) ||
        (acc && !aligned(acc, 4)))
        return fail(BT_ERR_ALIGN, "Wp must be 16-byte aligned; X, w_scale, Y and acc 4-byte aligned");
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (linear_fused(M, N, K))
        return hip_status(
            bt::launch_linear_decode(static_cast<const uint4 *>(Wp), w_scale, rows, X, M, N, K, Y, acc, s),
            "bt_ternary_linear launch");
    if (!workspace)
        return fail(BT_ERR_NULL, "workspace is NULL but bt_linear_workspace_bytes(%lld, %lld, %lld) = %zu",
                    (long long)M, (long long)N, (long long)K, bt_linear_workspace_bytes(M, N, K));
    if (!aligned(workspace, 256))
        return fail(BT_ERR_ALIGN, "workspace must be 256-byte aligned");
    int8_t *Xq = static_cast<int8_t *>(workspace);
    float *sx = reinterpret_cast<float *>(Xq + bt::round_up(M * bt_act_row_bytes(K), 256));
    int32_t *xsum = reinterpret_cast<int32_t *>(reinterpret_cast<char *>(sx) + bt::round_up(4 * M, 256));
    if (M <= BT_GEMV_MAX_M) {
        if (bt_status st = bt_quant_act(X, M, K, Xq, sx, xsum, stream))
            return st;
        return gemv_impl(Wp, w_scale, rows, Xq, sx, xsum, M, N, K, Y, acc, BT_GEMV_AUTO, stream);
    }
    // The quantizer also zero-fills the split-K arrival counters of the GEMM workspace,
    // so the caller's workspace needs no initialization.
    char *gws = static_cast<char *>(workspace) + linear_quant_bytes(M, K);
    const size_t gbytes = bt_gemm_workspace_bytes(M, N, K);
    if (bt_status st = hip_status(bt::launch_quant_act(X, M, K, bt_act_row_bytes(K), Xq, sx, xsum,
                                                       reinterpret_cast<unsigned *>(gws),
                                                       gbytes ? bt::gemm_arrival_words(M, N, K) : 0, s),
                                  "bt_quant_act launch"))
        return st;
    return gemm_impl(Wp, w_scale, rows, Xq, sx, xsum, M, N, K, Y, acc, gbytes ? gws : nullptr, gbytes, stream);
}

// Device address of `scratch` on the current device, looked up once per device.
static bt_status static_scratch(void **out)
{
    constexpr int kMaxDevices = 64;
    static std::mutex lock;
    static void *addr[kMaxDevices];
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess)
        return fail(BT_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(BT_ERR_UNSUPPORTED, "device %d beyond the %d this library tracks", dev, kMaxDevices);
    std::lock_guard<std::mutex> g(lock);
    if (!addr[dev]) {
        void *p = nullptr;
        if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)); e != hipSuccess || !p)
            return fail(BT_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        e != hipSuccess ? hipGetErrorString(e) : "null address");
        addr[dev] = p;
    }
    *out = addr[dev];
    return BT_OK;
}

static bt_status linear_static_impl(const void *Wp, const float *w_scale, bool rows, const float *X, int64_t M,
                                    int64_t N, int64_t K, float *Y, int32_t *acc, void *stream)
{
    if (M < 0 || N < 0 || M > BT_MAX_DIM || N > BT_MAX_DIM || K < 0 || K > BT_MAX_K || M * N > BT_MAX_MN)
        return linear_impl(Wp, w_scale, rows, X, M, N, K, Y, acc, nullptr, stream);  // its shape error
    const size_t need = bt_linear_workspace_bytes(M, N, K);
    if (need > (size_t)BT_STATIC_SCRATCH_BYTES)
        return fail(BT_ERR_UNSUPPORTED,
                    "M = %lld, N = %lld, K = %lld needs %zu bytes of scratch, above the static %lld bytes "
                    "(use bt_ternary_linear with a workspace)",
                    (long long)M, (long long)N, (long long)K, need, (long long)BT_STATIC_SCRATCH_BYTES);
    void *ws = nullptr;
    if (need > 0)
        if (bt_status s = static_scratch(&ws))
            return s;
    return linear_impl(Wp, w_scale, rows, X, M, N, K, Y, acc, ws, stream);
}

bt_status bt_ternary_gemv_algo(const void *Wp, const float *w_scale, const int8_t *Xq, const float *x_scale,
                               const int32_t *x_sum, int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc,
                               int32_t algo, void *stream)
{
    return gemv_impl(Wp, w_scale, false, Xq, x_scale, x_sum, M, N, K, Y, acc, algo, stream);
}

bt_status bt_ternary_gemv(const void *Wp, const float *w_scale, const int8_t *Xq, const float *x_scale,
                          const int32_t *x_sum, int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc, void *stream)
{
    return gemv_impl(Wp, w_scale, false, Xq, x_scale, x_sum, M, N, K, Y, acc, BT_GEMV_AUTO, stream);
}

bt_status bt_ternary_gemv_rs(const void *Wp, const float *row_scale, const int8_t *Xq, const float *x_scale,
                             const int32_t *x_sum, int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc,
                             int32_t algo, void *stream)
{
    return gemv_impl(Wp, row_scale, true, Xq, x_scale, x_sum, M, N, K, Y, acc, algo, stream);
}

size_t bt_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || N <= 0 || K <= 0 || M > BT_MAX_DIM || N > BT_MAX_DIM || K > BT_MAX_K)
        return 0;
    return bt::gemm_workspace_bytes(M, N, K);
}

bt_status bt_gemm_split_plan(int64_t M, int64_t N, int64_t K, int64_t *full_tiles, int32_t *splits)
{
    if (!full_tiles || !splits)
        return fail(BT_ERR_NULL, "full_tiles and splits must not be NULL");
    if (M < 0 || N < 0 || M > BT_MAX_DIM || N > BT_MAX_DIM)
        return fail(BT_ERR_SHAPE, "shape M = %lld, N = %lld out of range", (long long)M, (long long)N);
    if (bt_status s = check_k(K))
        return s;
    const int64_t tiles = bt::gemm_tiles(M, N);
    const bt::GemmPlan pl = (M > 0 && N > 0 && K > 0) ? bt::gemm_plan(M, N, K) : bt::GemmPlan{tiles, 1};
    *full_tiles = pl.nsplit == 1 ? tiles : pl.full;
    *splits = pl.nsplit;
    return ok();
}

bt_status bt_ternary_gemm_ws(const void *Wp, const float *w_scale, const int8_t *Xq, const float *x_scale,
                             const int32_t *x_sum, int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc,
                             void *workspace, size_t workspace_bytes, void *stream)
{
    return gemm_impl(Wp, w_scale, false, Xq, x_scale, x_sum, M, N, K, Y, acc, workspace, workspace_bytes, stream);
}

bt_status bt_ternary_gemm(const void *Wp, const float *w_scale, const int8_t *Xq, const float *x_scale,
                          const int32_t *x_sum, int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc, void *stream)
{
    return gemm_impl(Wp, w_scale, false, Xq, x_scale, x_sum, M, N, K, Y, acc, nullptr, 0, stream);
}

bt_status bt_ternary_gemm_rs(const void *Wp, const float *row_scale, const int8_t *Xq, const float *x_scale,
                             const int32_t *x_sum, int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc,
                             void *workspace, size_t workspace_bytes, void *stream)
{
    return gemm_impl(Wp, row_scale, true, Xq, x_scale, x_sum, M, N, K, Y, acc, workspace, workspace_bytes, stream);
}

size_t bt_linear_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || N <= 0 || K < 0 || linear_fused(M, N, K))
        return 0;
    const size_t gemm = M > BT_GEMV_MAX_M ? bt_gemm_workspace_bytes(M, N, K) : 0;
    return linear_quant_bytes(M, K) + gemm;
}

bt_status bt_ternary_linear(const void *Wp, const float *w_scale, const float *X, int64_t M, int64_t N, int64_t K,
                            float *Y, int32_t *acc, void *workspace, void *stream)
{
    return linear_impl(Wp, w_scale, false, X, M, N, K, Y, acc, workspace, stream);
}

bt_status bt_ternary_linear_rs(const void *Wp, const float *row_scale, const float *X, int64_t M, int64_t N,
                               int64_t K, float *Y, int32_t *acc, void *workspace, void *stream)
{
    return linear_impl(Wp, row_scale, true, X, M, N, K, Y, acc, workspace, stream);
}

bt_status bt_ternary_linear_static(const void *Wp, const float *w_scale, const float *X, int64_t M, int64_t N,
                                   int64_t K, float *Y, int32_t *acc, void *stream)
{
    return linear_static_impl(Wp, w_scale, false, X, M, N, K, Y, acc, stream);
}

size_t bt_binary_weight_bytes(int64_t N, int64_t K)
{
    if (N <= 0 || K <= 0)
        return 0;
    return (size_t)(bt::round_up(N, 64) * bt::round_up(K, 128) / 8);
}

int64_t bt_act_bits_row_bytes(int64_t K, int32_t layout)
{
    if (K <= 0 || (layout != BT_BITS_PLAIN && layout != BT_BITS_CODES))
        return 0;
    return 4 * bt::act_bits_words(K, layout);
}

bt_status bt_pack_weights_binary(const float *W, int64_t N, int64_t K, void *Wb, float *w_scale, void *workspace,
                                 void *stream)
{
    if (bt_status s = check_nk(N, K))
        return s;
    if (N == 0 || K == 0)
        return fail(BT_ERR_SHAPE, "binary packing needs N > 0 and K > 0");
    if (!W || !Wb || !w_scale || !workspace)
        return fail(BT_ERR_NULL, "NULL W, Wb, w_scale or workspace");
    if (!aligned(W, 4) || !aligned(Wb, 16) || !aligned(w_scale, 4) || !aligned(workspace, 8))
        return fail(BT_ERR_ALIGN, "Wb must be 16-byte aligned; W, w_scale and workspace 4/8-byte aligned");
    return hip_status(bt::launch_pack_binary(W, N, K, static_cast<uint4 *>(Wb), w_scale,
                                             static_cast<float *>(workspace), static_cast<hipStream_t>(stream)),
                      "bt_pack_weights_binary launch");
}

bt_status bt_binarize_act(const float *X, int64_t M, int64_t K, int32_t layout, uint32_t *Xb, float *x_scale,
                          void *stream)
{
    if (M < 0 || M > BT_MAX_DIM)
        return fail(BT_ERR_SHAPE, "M = %lld outside [0, 2^23]", (long long)M);
    if (bt_status s = check_k(K))
        return s;
    if (layout != BT_BITS_PLAIN && layout != BT_BITS_CODES)
        return fail(BT_ERR_UNSUPPORTED, "unknown bit layout %d", (int)layout);
    if (M == 0 || K == 0)
        return fail(BT_ERR_SHAPE, "binarizing needs M > 0 and K > 0");
    if (!X || !Xb || !x_scale)
        return fail(BT_ERR_NULL, "NULL X, Xb or x_scale");
    if (!aligned(X, 4) || !aligned(Xb, 16) || !aligned(x_scale, 4))
        return fail(BT_ERR_ALIGN, "Xb must be 16-byte aligned; X and x_scale 4-byte aligned");
    return hip_status(bt::launch_binarize(X, M, K, layout, Xb, x_scale, static_cast<hipStream_t>(stream)),
                      "bt_binarize_act launch");
}

static bt_status check_bits_product(const void *Wq, const float *w_scale, const uint32_t *Xb, const float *x_scale,
                                    int64_t M, int64_t N, int64_t K, const float *Y, const int32_t *acc)
{
    if (M < 1 || M > BT_GEMV_MAX_M)
        return fail(BT_ERR_UNSUPPORTED, "1-bit GEMVs take 1 <= M <= %d (got %lld)", BT_GEMV_MAX_M, (long long)M);
    if (N < 1 || N > BT_MAX_DIM)
        return fail(BT_ERR_SHAPE, "N = %lld outside [1, 2^23]", (long long)N);
    if (K < 1 || K > BT_MAX_K)
        return fail(BT_ERR_SHAPE, "K = %lld outside [1, %d]", (long long)K, BT_MAX_K);
    if (!Y && !acc)
        return fail(BT_ERR_NULL, "Y and acc are both NULL");
    if (!Wq || !w_scale || !Xb || !x_scale)
        return fail(BT_ERR_NULL, "NULL input pointer");
    if (!aligned(Wq, 16) || !aligned(Xb, 16) || !aligned(w_scale, 4) || !aligned(x_scale, 4) ||
        (Y && !aligned(Y, 4)) || (acc && !aligned(acc, 4)))
        return fail(BT_ERR_ALIGN, "weights and bits 16-byte aligned, scales and outputs 4-byte aligned");
    return BT_OK;
}

bt_status bt_binary_gemv(const void *Wb, const float *w_scale, const uint32_t *Xb, const float *x_scale, int64_t M,
                         int64_t N, int64_t K, float *Y, int32_t *acc, void *stream)
{
    if (bt_status s = check_bits_product(Wb, w_scale, Xb, x_scale, M, N, K, Y, acc))
        return s;
    return hip_status(bt::launch_gemv_binary(static_cast<const uint4 *>(Wb), w_scale, Xb, x_scale, M, N, K, Y, acc,
                                             static_cast<hipStream_t>(stream)),
                      "bt_binary_gemv launch");
}

bt_status bt_ternary_gemv_a1(const void *Wp, const float *w_scale, const uint32_t *Xb, const float *x_scale,
                             int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc, void *stream)
{
    if (bt_status s = check_bits_product(Wp, w_scale, Xb, x_scale, M, N, K, Y, acc))
        return s;
    return hip_status(bt::launch_gemv_ternary_a1(static_cast<const uint4 *>(Wp), w_scale, Xb, x_scale, M, N, K, Y,
                                                 acc, static_cast<hipStream_t>(stream)),
                      "bt_ternary_gemv_a1 launch");
}

bt_status bt_kernel_plan(int32_t call, int64_t M, int64_t N, int64_t K, int32_t algo, int32_t row_scales, char *buf,
                         size_t len)
{
    if (!buf || len == 0)
        return fail(BT_ERR_NULL, "buf is NULL or len is 0");
    buf[0] = '\0';
    if (call < BT_CALL_LINEAR || call > BT_CALL_QUANT)
        return fail(BT_ERR_UNSUPPORTED, "unknown call %d", (int)call);
    if (M < 0 || N < 0 || M > BT_MAX_DIM || N > BT_MAX_DIM || M * N > BT_MAX_MN)
        return fail(BT_ERR_SHAPE, "shape M = %lld, N = %lld out of range", (long long)M, (long long)N);
    if (bt_status s = check_k(K))
        return s;
    const bool rows = row_scales != 0;
    if (M == 0 || (N == 0 && call != BT_CALL_QUANT))
        return ok();  // no launch
    int used = 0;
    auto room = [&]() { return len > (size_t)used ? len - (size_t)used : 0; };
    auto add = [&](int n) { used += n > 0 ? n : 0; };
    auto gemv_plan = [&](int32_t a) -> bt_status {
        if (M > BT_GEMV_MAX_M)
            return fail(BT_ERR_UNSUPPORTED, "gemv takes M <= %d", BT_GEMV_MAX_M);
        if (a == BT_GEMV_AUTO)
            a = BT_GEMV_STAGED;
        if (a == BT_GEMV_STAGED && K == 0)
            a = BT_GEMV_MFMA;
        if (a == BT_GEMV_LUT && K == 0)
            a = BT_GEMV_MFMA;
        switch (a) {
        case BT_GEMV_STAGED:
            add(bt::plan_gemv_staged(M, N, K, rows, buf + used, room()));
            return ok();
        case BT_GEMV_MFMA: add(bt::plan_gemv_mfma(M, N, K, rows, buf + used, room())); return ok();
        case BT_GEMV_DOT4:
            if (M > 4)
                return fail(BT_ERR_UNSUPPORTED, "dot4 gemv takes M <= 4");
            add(snprintf(buf + used, room(), "k_gemv_dot4<MT=%d>(rows=%d)", (int)M, (int)rows));
            return ok();
        case BT_GEMV_LUT:
            if (M != 1)
                return fail(BT_ERR_UNSUPPORTED, "lut gemv takes M == 1");
            add(snprintf(buf + used, room(), "k_gemv_lut(rows=%d)", (int)rows));
            return ok();
        default: return fail(BT_ERR_UNSUPPORTED, "unknown gemv algo %d", (int)a);
        }
    };
    switch (call) {
    case BT_CALL_GEMV: return gemv_plan(algo);
    case BT_CALL_GEMM: add(bt::plan_gemm(M, N, K, rows, false, buf, len)); return ok();
    case BT_CALL_GEMM_WS: add(bt::plan_gemm(M, N, K, rows, true, buf, len)); return ok();
    case BT_CALL_QUANT: add(bt::plan_quant_act(M, K, buf, len)); return ok();
    default: break;
    }
    if (linear_fused(M, N, K)) {
        add(bt::plan_linear_decode(M, N, K, rows, buf, len));
        return ok();
    }
    add(bt::plan_quant_act(M, K, buf, len));
    add(snprintf(buf + used, room(), " + "));
    if (M <= BT_GEMV_MAX_M)
        return gemv_plan(BT_GEMV_AUTO);
    add(bt::plan_gemm(M, N, K, rows, true, buf + used, room()));
    return ok();
}

const char *bt_status_str(bt_status s)
{
    switch (s) {
    case BT_OK: return "BT_OK";
    case BT_ERR_NULL: return "BT_ERR_NULL";
    case BT_ERR_SHAPE: return "BT_ERR_SHAPE";
    case BT_ERR_UNSUPPORTED: return "BT_ERR_UNSUPPORTED";
    case BT_ERR_ALIGN: return "BT_ERR_ALIGN";
    case BT_ERR_HIP: return "BT_ERR_HIP";
    default: return "BT_ERR_UNKNOWN";
    }
}

const char *bt_last_error(void) { return g_err; }

}  // extern "C"
