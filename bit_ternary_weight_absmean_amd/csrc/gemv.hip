// Decode GEMV (1 <= M <= 16 tokens): acc[m,n] = sum_k t[n,k] q[m,k] in int32 with
// the scale epilogue y = fp32(acc) * (gamma * s_x[m]) fused.
//
// "bit-floor" page, "The core math": the product runs on integers and floating
// point appears only in the final scale multiply; "BitCompute" page, "Features":
// with ternary weights the product is add / subtract / skip. The decode phase is
// bound by weight bandwidth (BitNet GPU guide, "Key Components and Source Code
// Architecture": decode is the memory-bound phase), so both kernels stream the
// 2-bit weights once, 16 bytes per lane per load (1 KiB per wave instruction,
// fully coalesced), and unpack them in registers.
//
// Two kernels share the packed layout:
//  * dot4: lane = weight row (64 rows per wave). Every lane of the wave works on
//    the same 64-k chunk, so the int8 activation chunk is wave-uniform and is read
//    through the scalar cache into SGPRs; the inner loop is 5 bit-ops + 4*M v_dot4
//    per 16 codes. Waves of a workgroup split K; one LDS pass adds their partials.
//  * mfma: v_mfma_i32_16x16x64_i8 with the weights as the A operand (16 rows) and
//    up to 16 tokens as the B operand; per 64 codes a lane needs 20 bit-ops and 4
//    MFMAs whatever M is, so it takes over once dot4's VALU cost (grows with M)
//    exceeds the HBM budget.
#include "bt_internal.h"

namespace bt {
namespace {

// ---------------------------------------------------------------- dot4 kernel
constexpr int kDot4Waves = 8;
constexpr int kDot4Unroll = 4;  // chunks loaded back to back per wave

template <int MT>
__global__ __launch_bounds__(kDot4Waves * 64) void k_gemv_dot4(
    const uint4 *__restrict__ Wp, const float *__restrict__ w_scale, const int8_t *__restrict__ Xq, int64_t ldq,
    const float *__restrict__ sx, const int32_t *__restrict__ xsum, int M, int64_t N, int KC,
    float *__restrict__ Y, int32_t *__restrict__ ACC)
{
    __shared__ int red[kDot4Waves][MT][64];
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int64_t rb = blockIdx.x;
    const uint4 *wrow = Wp + rb * (int64_t)KC * 64 + lane;

    int a1[MT], a4[MT], a16[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
        a1[m] = a4[m] = a16[m] = 0;

    for (int c0 = wave * kDot4Unroll; c0 < KC; c0 += kDot4Waves * kDot4Unroll) {
        uint4 p[kDot4Unroll];
#pragma unroll
        for (int u = 0; u < kDot4Unroll; ++u)
            p[u] = (c0 + u < KC) ? wrow[(int64_t)(c0 + u) * 64] : make_uint4(kPadWord, kPadWord, kPadWord, kPadWord);
#pragma unroll
        for (int u = 0; u < kDot4Unroll; ++u) {
            const int c = c0 + u;
            if (c >= KC)
                break;
            const uint32_t pw[4] = {p[u].x, p[u].y, p[u].z, p[u].w};
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                // 64 int8 activations of chunk c for token m: wave-uniform address.
                const int32_t *xc = reinterpret_cast<const int32_t *>(Xq + (int64_t)m * ldq + (int64_t)c * 64);
                int32_t xw[16];
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    xw[i] = xc[i];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t w = pw[j];
                    a1[m] = __builtin_amdgcn_sdot4((int)(w & kMask0), xw[4 * j + 0], a1[m], false);
                    a4[m] = __builtin_amdgcn_sdot4((int)(w & kMask1), xw[4 * j + 1], a4[m], false);
                    a16[m] = __builtin_amdgcn_sdot4((int)(w & kMask2), xw[4 * j + 2], a16[m], false);
                    a16[m] = __builtin_amdgcn_sdot4((int)((w >> 2) & kMask2), xw[4 * j + 3], a16[m], false);
                }
            }
        }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m)
        red[wave][m][lane] = a1[m] + (a4[m] >> 2) + (a16[m] >> 4);
    __syncthreads();

    const float gamma = w_scale[0];
    for (int o = threadIdx.x; o < MT * 64; o += kDot4Waves * 64) {
        const int m = o >> 6;
        const int r = o & 63;
        const int64_t n = rb * 64 + r;
        if (m >= M || n >= N)
            continue;
        int s = 0;
#pragma unroll
        for (int w = 0; w < kDot4Waves; ++w)
            s += red[w][m][r];
        const int acc = s - xsum[m];
        if (ACC)
            ACC[(int64_t)m * N + n] = acc;
        if (Y)
            Y[(int64_t)m * N + n] = (float)acc * (gamma * sx[m]);
    }
}

// ---------------------------------------------------------------- mfma kernel
constexpr int kMfmaWaves = 4;

// One workgroup per 64 weight rows (four 16-row MFMA blocks). A "step" is 256 k:
// lane group g = lane / 16 takes chunk 4*step + g, lane row r = lane % 16.
//  A operand (weights), block i, mask s: dword j = word j of row 16i + r & mask s.
//  B operand (tokens):  lane (g, m = r) holds x[m][64c .. 64c + 63] as 16 dwords
//  xw; for mask s its dword j is xw[4j + s] (the same k as the A byte).
// MFMA output: lane holds D[4g + v][r], i.e. row 16i + 4g + v, token r.
__global__ __launch_bounds__(kMfmaWaves * 64) void k_gemv_mfma(
    const uint4 *__restrict__ Wp, const float *__restrict__ w_scale, const int8_t *__restrict__ Xq, int64_t ldq,
    const float *__restrict__ sx, const int32_t *__restrict__ xsum, int M, int64_t N, int KC,
    float *__restrict__ Y, int32_t *__restrict__ ACC)
{
    __shared__ int red[kMfmaWaves][4][4][64];
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int r = lane & 15;
    const int64_t rb = blockIdx.x;
    const int nsteps = (KC + 3) >> 2;

    v4i acc1[4], acc4[4], acc16[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc1[i] = acc4[i] = acc16[i] = v4i{0, 0, 0, 0};

    for (int st = wave; st < nsteps; st += kMfmaWaves) {
        const int c = 4 * st + g;
        const bool valid = c < KC;
        uint4 w[4];
        const uint4 *base = Wp + (rb * (int64_t)KC + c) * 64 + r;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = valid ? base[16 * i] : make_uint4(kPadWord, kPadWord, kPadWord, kPadWord);
        int32_t xw[16];
        if (valid && r < M) {
            const uint4 *xs = reinterpret_cast<const uint4 *>(Xq + (int64_t)r * ldq + (int64_t)c * 64);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint4 v = xs[q];
                xw[4 * q + 0] = (int32_t)v.x;
                xw[4 * q + 1] = (int32_t)v.y;
                xw[4 * q + 2] = (int32_t)v.z;
                xw[4 * q + 3] = (int32_t)v.w;
            }
        } else {
#pragma unroll
            for (int q = 0; q < 16; ++q)
                xw[q] = 0;
        }
        const v4i b0 = {xw[0], xw[4], xw[8], xw[12]};
        const v4i b1 = {xw[1], xw[5], xw[9], xw[13]};
        const v4i b2 = {xw[2], xw[6], xw[10], xw[14]};
        const v4i b3 = {xw[3], xw[7], xw[11], xw[15]};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t pw[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
            v4i a0, a1, a2, a3;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                a0[j] = (int)(pw[j] & kMask0);
                a1[j] = (int)(pw[j] & kMask1);
                a2[j] = (int)(pw[j] & kMask2);
                a3[j] = (int)((pw[j] >> 2) & kMask2);
            }
            acc1[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, acc1[i], 0, 0, 0);
            acc4[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, acc4[i], 0, 0, 0);
            acc16[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a2, b2, acc16[i], 0, 0, 0);
            acc16[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a3, b3, acc16[i], 0, 0, 0);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            red[wave][i][v][lane] = acc1[i][v] + (acc4[i][v] >> 2) + (acc16[i][v] >> 4);
    __syncthreads();

    const float gamma = w_scale[0];
    // Output o = m * 64 + nl (nl fastest, so stores of one token are contiguous).
    for (int o = threadIdx.x; o < M * 64; o += kMfmaWaves * 64) {
        const int m = o >> 6;
        const int nl = o & 63;
        const int64_t n = rb * 64 + nl;
        if (n >= N)
            continue;
        const int i = nl >> 4, gg = (nl >> 2) & 3, v = nl & 3;
        const int src_lane = gg * 16 + m;
        int s = 0;
#pragma unroll
        for (int w = 0; w < kMfmaWaves; ++w)
            s += red[w][i][v][src_lane];
        const int acc = s - xsum[m];
        if (ACC)
            ACC[(int64_t)m * N + n] = acc;
        if (Y)
            Y[(int64_t)m * N + n] = (float)acc * (gamma * sx[m]);
    }
}

}  // namespace

hipError_t launch_gemv_dot4(const uint4 *Wp, const float *w_scale, const int8_t *Xq, int64_t ldq,
                            const float *sx, const int32_t *xsum, int64_t M, int64_t N, int64_t K, float *Y,
                            int32_t *acc, hipStream_t s)
{
    const int64_t NB = (N + 63) / 64;
    const int KC = (int)((K + 63) / 64);
    const dim3 grid((unsigned)NB), block(kDot4Waves * 64);
    switch (M) {
    case 1:
        hipLaunchKernelGGL(k_gemv_dot4<1>, grid, block, 0, s, Wp, w_scale, Xq, ldq, sx, xsum, (int)M, N, KC, Y, acc);
        break;
    case 2:
        hipLaunchKernelGGL(k_gemv_dot4<2>, grid, block, 0, s, Wp, w_scale, Xq, ldq, sx, xsum, (int)M, N, KC, Y, acc);
        break;
    case 3:
        hipLaunchKernelGGL(k_gemv_dot4<3>, grid, block, 0, s, Wp, w_scale, Xq, ldq, sx, xsum, (int)M, N, KC, Y, acc);
        break;
    default:
        hipLaunchKernelGGL(k_gemv_dot4<4>, grid, block, 0, s, Wp, w_scale, Xq, ldq, sx, xsum, (int)M, N, KC, Y, acc);
        break;
    }
    return hipGetLastError();
}

hipError_t launch_gemv_mfma(const uint4 *Wp, const float *w_scale, const int8_t *Xq, int64_t ldq,
                            const float *sx, const int32_t *xsum, int64_t M, int64_t N, int64_t K, float *Y,
                            int32_t *acc, hipStream_t s)
{
    const int64_t NB = (N + 63) / 64;
    const int KC = (int)((K + 63) / 64);
    hipLaunchKernelGGL(k_gemv_mfma, dim3((unsigned)NB), dim3(kMfmaWaves * 64), 0, s, Wp, w_scale, Xq, ldq, sx, xsum,
                       (int)M, N, KC, Y, acc);
    return hipGetLastError();
}

}  // namespace bt
