// Decode GEMV for one token by table lookup (T-MAC / TL1 style): instead of unpacking
// the 2-bit codes and multiplying (dot4, MFMA), every workgroup first tabulates, for each
// pair of codes that shares a 4-bit nibble of the packed weights, the sixteen possible
// values of c_lo * q[k] + c_hi * q[k + 4]; the product of a weight row with x is then one
// LDS lookup and one add per nibble. acc = sum - sum_k q (offset codes c = t + 1), and
// the scale epilogue is the one of the other kernels.
//
// Passages: the "Run 100B Models on Your Laptop CPU" page, "What is Microsoft BitNet?"
// (kernels built on the lookup-table method of T-MAC) and "Key Features That Make BitNet
// Insane" (TL1 / TL2, the ternary lookup kernels), and the "bit-floor" page, "The core
// math" (integer inner loop, floating point only in the final scale multiply).
// The LUT trades the VALU unpack of the other kernels for LDS reads; on this GPU it is a
// second algorithm to measure against them, not the default.
//
// Table layout (int16, one table of 16 entries = 32 bytes per nibble position): 16-k
// group g = 4 c + j (word j of chunk c), nibble p = bits 4p .. 4p+3 of that word, which
// holds codes b = (p >> 1) + 8 (p & 1) and b + 4 of the word (code b at bits
// 8 (b % 4) + 2 (b / 4)), i.e. k0 = 16 g + (p >> 1) + 8 (p & 1) and k0 + 4. Entry v =
// (v & 3) q[k0] + (v >> 2) q[k0 + 4]; |entry| <= 3 * 127 * 2 fits int16. 256 bytes per
// group: K = 4096 takes 64 KB of LDS.
#include "bt_internal.h"

namespace bt {
namespace {

constexpr int kLutWaves = 4;
constexpr int kLutRows = 16;   // weight rows per workgroup: lane = 4 * row + word
constexpr int kLutBatch = 8;   // chunks per weight batch (two batches in flight per wave)
constexpr int kLutBuild = 8;   // tables whose activation bytes each thread loads together

template <int CTRL>
__device__ inline int lut_dpp(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}

__global__ __launch_bounds__(kLutWaves * 64) void k_gemv_lut(const uint32_t *__restrict__ Wp,
                                                             const float *__restrict__ w_scale, int rs,
                                                             const int8_t *__restrict__ Xq,
                                                             const float *__restrict__ sx,
                                                             const int32_t *__restrict__ xsum, int64_t N, int KC,
                                                             float *__restrict__ Y, int32_t *__restrict__ ACC)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ int red[kLutWaves][kLutRows];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int KG = KC * 4;

    // Lane (r, j) = (lane / 4, lane % 4) reads word j of row r's 16 bytes in each chunk the
    // wave owns (chunks wave, wave + 4, ...): 256 contiguous bytes per wave and chunk. Rows
    // past N (up to the packed 64-row padding) are read and never stored.
    const int r = lane >> 2, j = lane & 3;
    const int64_t n = (int64_t)blockIdx.x * kLutRows + r;
    const int64_t rb = n >> 6, rr = n & 63;
    const uint32_t *wrow = Wp + (rb * KC * 64 + rr) * 4 + j;  // + 256 words per chunk
    const int nmine = wave < KC ? (KC - 1 - wave) / kLutWaves + 1 : 0;
    const int nb = (nmine + kLutBatch - 1) / kLutBatch;
    uint32_t wa[kLutBatch], wb[kLutBatch];
    auto load_batch = [&](uint32_t (&w)[kLutBatch], int b) {  // unconditional, at clamped chunks
#pragma unroll
        for (int u = 0; u < kLutBatch; ++u)
            w[u] = wrow[(int64_t)min(wave + kLutWaves * (b * kLutBatch + u), KC - 1) * 256];
    };

    // 1. The tables: thread t fills the tables (g, p) = t, t + 256, ... (16 entries,
    //    two 16-byte LDS stores each). Xq rows are zero past K up to a multiple of 256,
    //    so every k read here lies in the row. The two activation bytes of kLutBuild
    //    tables are loaded together (unconditionally, at clamped tables) before any is
    //    built. The first such loads go out before the wave's first two weight batches
    //    (vector-memory loads complete in order: building then waits for the activation
    //    bytes only, while the weights stream in under it).
    constexpr int T = kLutWaves * 64;
    const int npairs = KG * 8;
    int q0[kLutBuild], q1[kLutBuild];
    auto load_q = [&](int base) {
#pragma unroll
        for (int i = 0; i < kLutBuild; ++i) {
            const int pair = min(base + i * T, npairs - 1);
            const int g = pair >> 3, p = pair & 7;
            const int k0 = 16 * g + (p >> 1) + 8 * (p & 1);
            q0[i] = Xq[k0];
            q1[i] = Xq[k0 + 4];
        }
    };
    load_q(tid);
    load_batch(wa, 0);
    load_batch(wb, 1);
    for (int base = tid; base < npairs; base += T * kLutBuild) {
        if (base != tid)
            load_q(base);
#pragma unroll
        for (int i = 0; i < kLutBuild; ++i) {
            const int pair = base + i * T;
            if (pair < npairs) {
                uint32_t packed[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int v0 = 2 * e, v1 = 2 * e + 1;
                    const int e0 = (v0 & 3) * q0[i] + (v0 >> 2) * q1[i];
                    const int e1 = (v1 & 3) * q0[i] + (v1 >> 2) * q1[i];
                    packed[e] = ((uint32_t)e0 & 0xFFFFu) | ((uint32_t)e1 << 16);
                }
                uint4 *dst = reinterpret_cast<uint4 *>(smem + (size_t)pair * 32);
                dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
                dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
            }
        }
    }
    __syncthreads();

    // 2. Lookups, one batch while the next one's loads are in flight: pairs of batches
    //    with unconditional loads, then the last pair with none.
    const int16_t *tab = reinterpret_cast<const int16_t *>(smem);
    int acc = 0;
    auto lookup_batch = [&](const uint32_t (&w)[kLutBatch], int b) {
#pragma unroll
        for (int u = 0; u < kLutBatch; ++u) {
            const int i = b * kLutBatch + u;
            if (i < nmine) {  // wave-uniform
                const int16_t *t = tab + (4 * (wave + kLutWaves * i) + j) * 128;
#pragma unroll
                for (int p = 0; p < 8; ++p)
                    acc += t[p * 16 + ((w[u] >> (4 * p)) & 15u)];
            }
        }
    };
    int b = 0;
    for (; b + 2 < nb; b += 2) {
        lookup_batch(wa, b);
        load_batch(wa, b + 2);
        lookup_batch(wb, b + 1);
        load_batch(wb, b + 3);
    }
    lookup_batch(wa, b);
    lookup_batch(wb, b + 1);

    // 3. Row sums: the four words of a row (a quad of lanes), then the waves.
    acc += lut_dpp<0xB1>(acc);  // quad_perm [1,0,3,2]
    acc += lut_dpp<0x4E>(acc);  // quad_perm [2,3,0,1]
    if (j == 0)
        red[wave][r] = acc;
    __syncthreads();
    if (tid < kLutRows) {
        const int64_t nn = (int64_t)blockIdx.x * kLutRows + tid;
        if (nn < N) {
            int s = 0;
#pragma unroll
            for (int w = 0; w < kLutWaves; ++w)
                s += red[w][tid];
            const int a = s - xsum[0];
            if (ACC)
                ACC[nn] = a;
            if (Y)
                Y[nn] = (float)a * (w_scale[rs ? nn : 0] * sx[0]);
        }
    }
}

}  // namespace

size_t gemv_lut_lds_bytes(int64_t K) { return (size_t)((K + 63) / 64) * 1024; }

hipError_t launch_gemv_lut(const uint4 *Wp, const float *w_scale, bool row_scales, const int8_t *Xq,
                           const float *sx, const int32_t *xsum, int64_t N, int64_t K, float *Y, int32_t *acc,
                           hipStream_t s)
{
    const int KC = (int)((K + 63) / 64);
    const dim3 grid((unsigned)((N + kLutRows - 1) / kLutRows)), block(kLutWaves * 64);
    hipLaunchKernelGGL(k_gemv_lut, grid, block, gemv_lut_lds_bytes(K), s, reinterpret_cast<const uint32_t *>(Wp),
                       w_scale, (int)row_scales, Xq, sx, xsum, N, KC, Y, acc);
    return hipGetLastError();
}

}  // namespace bt
