// Prefill GEMM on int8 MFMA: acc[m,n] = sum_k t[n,k] q[m,k], any M, with the scale
// epilogue fused. BitNet GPU guide, "Key Components and Source Code Architecture":
// prefill is the compute-bound phase; "BitCompute" page, "Future Roadmap": move the
// add/subtract loops of the ternary product onto the matrix cores.
//
// Tiling (gfx950, wave64, v_mfma_i32_16x16x64_i8):
//  * workgroup = 4 waves = a 128 (tokens) x 128 (weight rows) output block;
//    wave (wm, wn) owns 64 x 64 = 4 x 4 MFMA tiles.
//  * k advances 256 per step: lane group g = lane / 16 covers the 64-k chunk
//    4*step + g, lane row r = lane % 16.
//  * weights (B operand, columns = weight rows): each lane loads its 16 packed bytes
//    straight from HBM (a wave instruction reads 1 KiB contiguous); word j
//    unpacks with shifts and one mask into the four operand dwords
//    (word >> 2s) & 0x03030303, s = 0..3, whose byte e is code k = 64c + 16j + 4s + e.
//    No LDS is used for weights.
//  * activations (A operand, rows = tokens): the 128 x 256 int8 tile is staged in
//    LDS with a 272-byte row pitch (conflict-free 16-byte reads); for substep j a
//    lane reads x[m][64c + 16j .. +15], which is exactly the A operand that pairs
//    with weight word j.
//  * output: lane holds D[4g + v][r] of each tile = token 16a + 4g + v, row 16i + r.
#include "bt_internal.h"

namespace bt {
namespace {

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kStepK = 256;
constexpr int kPitch = kStepK + 16;  // LDS row pitch in bytes
constexpr int kThreads = 256;
constexpr int kXLoads = kBM * kStepK / 16 / kThreads;  // uint4 per thread per step (= 8)

__device__ inline v4i unpack_word(uint32_t w)
{
    return v4i{(int)(w & kMask0), (int)((w >> 2) & kMask0), (int)((w >> 4) & kMask0), (int)((w >> 6) & kMask0)};
}

__global__ __launch_bounds__(kThreads) void k_gemm(const uint4 *__restrict__ Wp, const float *__restrict__ w_scale,
                                                  const int8_t *__restrict__ Xq, int64_t ldq,
                                                  const float *__restrict__ sx, const int32_t *__restrict__ xsum,
                                                  int64_t M, int64_t N, int KC, int NB64, float *__restrict__ Y,
                                                  int32_t *__restrict__ ACC)
{
    __shared__ __attribute__((aligned(16))) int8_t xs[kBM * kPitch];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int g = lane >> 4, r = lane & 15;
    const int64_t m0 = (int64_t)blockIdx.y * kBM;
    const int64_t rg = (int64_t)blockIdx.x * 2 + wn;  // this wave's 64-row weight group
    const bool has_rows = rg < NB64;
    const int nsteps = (KC + 3) >> 2;

    v4i acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc[a][i] = v4i{0, 0, 0, 0};

    // Global -> register prefetch of the activation tile for one step.
    uint4 xreg[kXLoads];
    auto load_x = [&](int st) {
#pragma unroll
        for (int q = 0; q < kXLoads; ++q) {
            const int u = tid + q * kThreads;  // 16-byte unit in the 128 x 256 tile
            const int row = u >> 4, col = u & 15;
            const int64_t m = m0 + row;
            const int chunk = 4 * st + (col >> 2);
            xreg[q] = make_uint4(0, 0, 0, 0);
            if (m < M && chunk < KC)
                xreg[q] = *reinterpret_cast<const uint4 *>(Xq + m * ldq + (int64_t)st * kStepK + col * 16);
        }
    };
    auto load_w = [&](int st, uint4 (&w)[4]) {
        const int c = 4 * st + g;
        const bool valid = has_rows && c < KC;
        const uint4 *base = Wp + (rg * (int64_t)KC + c) * 64 + r;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = valid ? base[16 * i] : make_uint4(kPadWord, kPadWord, kPadWord, kPadWord);
    };

    uint4 wcur[4];
    if (nsteps > 0) {
        load_x(0);
        load_w(0, wcur);
    }
    for (int st = 0; st < nsteps; ++st) {
        __syncthreads();  // previous step's LDS reads are done
#pragma unroll
        for (int q = 0; q < kXLoads; ++q) {
            const int u = tid + q * kThreads;
            *reinterpret_cast<uint4 *>(xs + (u >> 4) * kPitch + (u & 15) * 16) = xreg[q];
        }
        __syncthreads();
        uint4 wnext[4];
        if (st + 1 < nsteps) {
            load_x(st + 1);
            load_w(st + 1, wnext);
        }
        if (has_rows) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v4i bop[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t word = (j == 0) ? wcur[i].x : (j == 1) ? wcur[i].y : (j == 2) ? wcur[i].z : wcur[i].w;
                    bop[i] = unpack_word(word);
                }
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const int row = wm * 64 + a * 16 + r;
                    const v4i aop = *reinterpret_cast<const v4i *>(xs + row * kPitch + g * 64 + j * 16);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[a][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop, bop[i], acc[a][i], 0, 0, 0);
                }
            }
        }
        if (st + 1 < nsteps) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                wcur[i] = wnext[i];
        }
    }

    if (!has_rows)
        return;
    const float gamma = w_scale[0];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t m = m0 + wm * 64 + a * 16 + 4 * g + v;
            if (m >= M)
                continue;
            const int32_t xs_m = xsum[m];
            const float scale = gamma * sx[m];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t n = rg * 64 + i * 16 + r;
                if (n >= N)
                    continue;
                const int accv = acc[a][i][v] - xs_m;
                if (ACC)
                    ACC[m * N + n] = accv;
                if (Y)
                    Y[m * N + n] = (float)accv * scale;
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm(const uint4 *Wp, const float *w_scale, const int8_t *Xq, int64_t ldq, const float *sx,
                       const int32_t *xsum, int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc, hipStream_t s)
{
    const int NB64 = (int)((N + 63) / 64);
    const int KC = (int)((K + 63) / 64);
    const dim3 grid((unsigned)((NB64 + 1) / 2), (unsigned)((M + kBM - 1) / kBM));
    hipLaunchKernelGGL(k_gemm, grid, dim3(kThreads), 0, s, Wp, w_scale, Xq, ldq, sx, xsum, M, N, KC, NB64, Y, acc);
    return hipGetLastError();
}

}  // namespace bt
