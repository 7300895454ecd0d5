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
// This file holds the dot4 kernel: lane = weight row (64 rows per wave). Every lane
// of the wave works on the same 64-k chunk, so the int8 activation chunk is
// wave-uniform and is read through the scalar cache into SGPRs; the inner loop is
// 5 bit-ops + 4*M v_dot4 per 16 codes. Waves of a workgroup split K; one LDS pass
// adds their partials. The int8-MFMA decode kernel (decode.hip) needs fewer VALU
// instructions per weight byte and is the library's default.
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
    float *__restrict__ Y, int32_t *__restrict__ ACC, int rs)
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
            Y[(int64_t)m * N + n] = (float)acc * (w_scale[rs ? n : 0] * sx[m]);
    }
}

}  // namespace

hipError_t launch_gemv_dot4(const uint4 *Wp, const float *w_scale, bool row_scales, const int8_t *Xq, int64_t ldq,
                            const float *sx, const int32_t *xsum, int64_t M, int64_t N, int64_t K, float *Y,
                            int32_t *acc, hipStream_t s)
{
    const int64_t NB = (N + 63) / 64;
    const int KC = (int)((K + 63) / 64);
    const dim3 grid((unsigned)NB), block(kDot4Waves * 64);
    switch (M) {
    case 1:
        hipLaunchKernelGGL(k_gemv_dot4<1>, grid, block, 0, s, Wp, w_scale, Xq, ldq, sx, xsum, (int)M, N, KC, Y, acc, (int)row_scales);
        break;
    case 2:
        hipLaunchKernelGGL(k_gemv_dot4<2>, grid, block, 0, s, Wp, w_scale, Xq, ldq, sx, xsum, (int)M, N, KC, Y, acc, (int)row_scales);
        break;
    case 3:
        hipLaunchKernelGGL(k_gemv_dot4<3>, grid, block, 0, s, Wp, w_scale, Xq, ldq, sx, xsum, (int)M, N, KC, Y, acc, (int)row_scales);
        break;
    default:
        hipLaunchKernelGGL(k_gemv_dot4<4>, grid, block, 0, s, Wp, w_scale, Xq, ldq, sx, xsum, (int)M, N, KC, Y, acc, (int)row_scales);
        break;
    }
    return hipGetLastError();
}

}  // namespace bt
