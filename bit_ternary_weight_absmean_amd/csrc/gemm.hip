// Prefill GEMM on int8 MFMA: acc[m,n] = sum_k t[n,k] q[m,k], any M, with the scale
// epilogue fused. BitNet GPU guide, "Key Components and Source Code Architecture":
// prefill is the compute-bound phase; "BitCompute" page, "Future Roadmap": move the
// add/subtract loops of the ternary product onto the matrix cores.
//
// Tiling (gfx950, wave64, v_mfma_i32_16x16x64_i8, 160 KB LDS per CU):
//  * a workgroup of WM x WN waves computes a BM (tokens) x BN (weight rows) block; each
//    wave owns a 64 x 64 tile of 4 x 4 MFMA tiles, so every activation operand read
//    from LDS feeds 4 MFMAs and every unpacked weight operand feeds 4, with the 64
//    accumulator registers and both operand pipelines within 256 VGPRs (two waves per
//    SIMD, so one wave's MFMAs cover the other's loads and unpacking).
//  * k advances 256 per step: lane group g = lane / 16 covers the 64-k chunk 4*step + g,
//    lane row r = lane % 16.
//  * weights (B operand): each lane loads its 16 packed bytes per 16-row tile straight
//    from memory (a 256-byte segment per 16 lanes), one step ahead, and unpacks word j
//    with shifts and one mask into the operand dwords (word >> 2s) & 0x03030303, whose
//    byte e is the code of k = 64c + 16j + 4s + e. No LDS is used for weights.
//  * activations (A operand): the BM x 256 int8 tile is staged in LDS (row pitch 272
//    bytes: 16-byte reads of 16 rows hit distinct banks), double-buffered, filled from
//    registers loaded one step ahead; for substep j a lane reads x[m][64c + 16j .. +15],
//    exactly the A operand that pairs with weight word j. One barrier per step.
//  * output: lane holds D[4g + v][r] of each tile = token 16a + 4g + v, row 16i + r;
//    y = (acc - sum_k q) * (gamma * s_x) is stored directly.
//  * workgroup -> tile map is XCD-aware: consecutive workgroup ids land on different
//    XCDs, so the tile order is remapped to give each XCD a contiguous run of tiles that
//    share activation rows (kept in that XCD's L2).
#include <atomic>

#include "bt_internal.h"

namespace bt {
namespace {

constexpr int kStepK = 256;
constexpr int kPitch = kStepK + 16;  // LDS row pitch in bytes
constexpr int kXcds = 8;

__device__ inline v4i unpack_word(uint32_t w)
{
    return v4i{(int)(w & kMask0), (int)((w >> 2) & kMask0), (int)((w >> 4) & kMask0), (int)((w >> 6) & kMask0)};
}

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gemm(
    const uint4 *__restrict__ Wp, const float *__restrict__ w_scale, const int8_t *__restrict__ Xq, int64_t ldq,
    const float *__restrict__ sx, const int32_t *__restrict__ xsum, int64_t M, int64_t N, int KC, int NB16,
    int tiles_m, int tiles_n, float *__restrict__ Y, int32_t *__restrict__ ACC)
{
    constexpr int kThreads = WM * WN * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
    constexpr int TM = WTM / 16, TN = WTN / 16;
    constexpr int XL = BM * kStepK / 16 / kThreads;  // 16-byte activation units per thread per step
    extern __shared__ __attribute__((aligned(16))) int8_t xs[];  // [2][BM][kPitch]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int wm = wave % WM, wn = wave / WM;
    const int g = lane >> 4, r = lane & 15;
    const int nsteps = (KC + 3) >> 2;

    // XCD-aware tile order: workgroup b runs on XCD b % 8; give each XCD a contiguous
    // range of the m-major tile list.
    const int total = tiles_m * tiles_n;
    const int per_xcd = (total + kXcds - 1) / kXcds;
    const int b = blockIdx.x;
    const int t = (b % kXcds) * per_xcd + b / kXcds;
    if (t >= total)
        return;
    const int tm = t / tiles_n, tn = t - tm * tiles_n;
    const int64_t m0 = (int64_t)tm * BM;
    const int n16_0 = (tn * BN + wn * WTN) / 16;  // first 16-row weight block of this wave

    v4i acc[TM][TN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int i = 0; i < TN; ++i)
            acc[a][i] = v4i{0, 0, 0, 0};

    // Native vectors, not uint4: copies of HIP's struct vector type through an array
    // lower to memcpy, which keeps the array in scratch memory.
    v4i xreg[XL];
    // Branch-free loads (a divergent guard makes the compiler wait at every join):
    // rows past M read row M-1 (their outputs are never stored) and activation rows
    // are zero-padded to a multiple of 256 bytes, so every step's chunks exist.
    auto load_x = [&](int st) {
#pragma unroll
        for (int q = 0; q < XL; ++q) {
            const int u = tid + q * kThreads;  // 16-byte unit of the BM x 256 tile
            const int row = u >> 4, col = u & 15;
            const int64_t m = min(m0 + row, M - 1);
            xreg[q] = *reinterpret_cast<const v4i *>(Xq + m * ldq + (int64_t)st * kStepK + col * 16);
        }
    };
    auto store_x = [&](int buf) {
        int8_t *base = xs + buf * BM * kPitch;
#pragma unroll
        for (int q = 0; q < XL; ++q) {
            const int u = tid + q * kThreads;
            *reinterpret_cast<v4i *>(base + (u >> 4) * kPitch + (u & 15) * 16) = xreg[q];
        }
    };
    // Clamped, unconditional weight loads: a chunk past K meets zero activations (the
    // activation rows are zero-padded to the step) and a row past N is never stored,
    // so neither needs the padding code.
    auto load_w = [&](int st, v4i (&w)[TN]) {
        const int cc = min(4 * st + g, KC - 1);
#pragma unroll
        for (int i = 0; i < TN; ++i) {
            const int bc = min(n16_0 + i, NB16 - 1);
            w[i] = reinterpret_cast<const v4i *>(Wp)[((int64_t)(bc >> 2) * KC + cc) * 64 + 16 * (bc & 3) + r];
        }
    };

    // One step of MFMAs on LDS buffer `buf` with the weight registers w. The A operands
    // of substep j + 1 are read while the MFMAs of substep j run.
    auto compute = [&](int buf, const v4i (&w)[TN]) {
        const int8_t *xb = xs + buf * BM * kPitch + (wm * WTM + r) * kPitch + g * 64;
        v4i aop[2][TM];
#pragma unroll
        for (int a = 0; a < TM; ++a)
            aop[0][a] = *reinterpret_cast<const v4i *>(xb + a * 16 * kPitch);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j < 3) {
#pragma unroll
                for (int a = 0; a < TM; ++a)
                    aop[(j + 1) & 1][a] = *reinterpret_cast<const v4i *>(xb + a * 16 * kPitch + (j + 1) * 16);
            }
            v4i bop[TN];
#pragma unroll
            for (int i = 0; i < TN; ++i) {
                bop[i] = unpack_word((uint32_t)w[i][j]);
            }
#pragma unroll
            for (int a = 0; a < TM; ++a)
#pragma unroll
                for (int i = 0; i < TN; ++i)
                    acc[a][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop[j & 1][a], bop[i], acc[a][i], 0, 0, 0);
        }
    };

    // Ping-pong: even steps use weight registers wA and LDS buffer 0, odd steps wB and
    // buffer 1; the activation registers always hold the step after the one being
    // computed. Buffer b is rewritten only after the barrier that ends the step that
    // last read it. The loop body is branch-free (prefetches past the last step reload
    // the last step, harmlessly), so the compiler's wait counts stay exact and a step
    // only waits for loads issued a full step earlier.
    v4i wA[TN], wB[TN];
    if (nsteps > 0) {
        load_x(0);
        load_w(0, wA);
        store_x(0);
        const int s1 = min(1, nsteps - 1);
        load_x(s1);
        load_w(s1, wB);
    }
    __syncthreads();
    const int last = nsteps - 1;
    const int npairs = nsteps >> 1;
    for (int p = 0; p < npairs; ++p) {
        const int st = 2 * p;
        compute(0, wA);
        store_x(1);  // the activation registers hold step st + 1
        load_x(min(st + 2, last));
        load_w(min(st + 2, last), wA);
        __syncthreads();
        compute(1, wB);
        store_x(0);  // step st + 2 (unused past the last step)
        load_x(min(st + 3, last));
        load_w(min(st + 3, last), wB);
        __syncthreads();
    }
    if (nsteps & 1)
        compute(0, wA);

    const float gamma = w_scale[0];
#pragma unroll
    for (int a = 0; a < TM; ++a) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t m = m0 + wm * WTM + a * 16 + 4 * g + v;
            if (m >= M)
                continue;
            const int32_t xs_m = xsum[m];
            const float scale = gamma * sx[m];
#pragma unroll
            for (int i = 0; i < TN; ++i) {
                const int64_t n = (int64_t)(n16_0 + i) * 16 + r;
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

template <int BM, int BN, int WM, int WN>
hipError_t launch_t(const uint4 *Wp, const float *w_scale, const int8_t *Xq, int64_t ldq, const float *sx,
                    const int32_t *xsum, int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc, hipStream_t s)
{
    const int KC = (int)((K + 63) / 64);
    const int NB16 = (int)(((N + 63) / 64) * 4);
    const int tiles_m = (int)((M + BM - 1) / BM);
    const int tiles_n = (int)((N + BN - 1) / BN);
    const int total = tiles_m * tiles_n;
    const int per_xcd = (total + kXcds - 1) / kXcds;
    const size_t lds = (size_t)2 * BM * kPitch;
    // Raising this kernel's dynamic-LDS cap is idempotent; do it once per process.
    static std::atomic<bool> attr_set{false};
    if (lds > 64 * 1024 && !attr_set.load(std::memory_order_acquire)) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_gemm<BM, BN, WM, WN>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess)
            return e;
        attr_set.store(true, std::memory_order_release);
    }
    hipLaunchKernelGGL((k_gemm<BM, BN, WM, WN>), dim3((unsigned)(per_xcd * kXcds)), dim3(WM * WN * 64), lds, s, Wp,
                       w_scale, Xq,
                       ldq, sx, xsum, M, N, KC, NB16, tiles_m, tiles_n, Y, acc);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const uint4 *Wp, const float *w_scale, const int8_t *Xq, int64_t ldq, const float *sx,
                       const int32_t *xsum, int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc, hipStream_t s)
{
    // 128 x 256 blocks (8 waves) share each staged activation tile between twice as
    // many weight rows; they win once there are enough of them to occupy most CUs.
    // With fewer tiles the 128 x 128 blocks (4 waves) spread the work wider.
    const int64_t t128x256 = ((M + 127) / 128) * ((N + 255) / 256);
    if (t128x256 >= 192)
        return launch_t<128, 256, 2, 4>(Wp, w_scale, Xq, ldq, sx, xsum, M, N, K, Y, acc, s);
    return launch_t<128, 128, 2, 2>(Wp, w_scale, Xq, ldq, sx, xsum, M, N, K, Y, acc, s);
}

}  // namespace bt
