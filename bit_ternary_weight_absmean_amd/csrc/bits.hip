// 1-bit activations: the binary GEMV (W1A1: +-1 weights, one bit each) and the ternary-
// weight GEMV against binarized tokens (W1.58A1), after the "bit-floor" page, "The core
// math": the binary dot product is K - 2 * popcount(w xor x) over sign bits (the page's
// 2 * POPCNT(XNOR) - K), the ternary one takes a magnitude plane and a sign plane,
// popcount(mag & (sign xnor x)) - popcount(mag & (sign xor x)); "What's inside" gives the
// scales (absmax for binary weights; activations binarized before each GEMV).
//
// A bit set means "negative" in every plane (weights and activations): agreement of two
// sign bits is a product of +1. v >= 0 binarizes to +1 (bit clear).
//
// Layouts (all little-endian 32-bit words):
//  - binary weights: chunks of 64 rows x 128 k, 1 KiB each, chunk (rb, c) at byte
//    ((rb * KC128) + c) * 1024; row r of the chunk is the 16 bytes at 16 r; word j holds
//    k = 128 c + 32 j + b at bit b. Padding bits are 0.
//  - activation bits, BT_BITS_PLAIN: k = 32 i + b at bit b of word i (rows of
//    ceil(K / 128) * 16 bytes, matching the weight chunks);
//  - activation bits, BT_BITS_CODES: word i holds k = 16 i + b at bit 8 (b % 4) + 2 (b / 4),
//    the low bit of code b in a packed ternary word (rows of ceil(K / 64) * 16 bytes), so
//    that the W1.58A1 kernel reads the 2-bit packed weights of bt_pack_weights as they are:
//    with M = 0x55555555, the non-zero plane is ~w & M and the negative plane
//    ~(w | w >> 1) & M (codes 0, 1, 2 = t + 1).
#include "bt_internal.h"
#include "wave.h"

namespace bt {
namespace {

constexpr int kBitWaves = 8;
constexpr uint32_t kLowBits = 0x55555555u;

// max |V[r, :]| of each row, one workgroup per row (exact: max does not round).
__global__ __launch_bounds__(256) void k_absmax_rows(const float *__restrict__ V, int64_t C,
                                                     float *__restrict__ amax)
{
    __shared__ float s[4];
    const float *v = V + (int64_t)blockIdx.x * C;
    float a = 0.0f;
    for (int64_t c = threadIdx.x; c < C; c += 256)
        a = fmaxf(a, fabsf(v[c]));
    a = wave_max_nonneg_f32(a);
    if ((threadIdx.x & 63) == 0)
        s[threadIdx.x >> 6] = a;
    __syncthreads();
    if (threadIdx.x == 0)
        amax[blockIdx.x] = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
}

// One workgroup: the max of n values (the row maxima).
__global__ __launch_bounds__(256) void k_max_of(const float *__restrict__ v, int64_t n, float *__restrict__ out)
{
    __shared__ float s[4];
    float a = 0.0f;
    for (int64_t i = threadIdx.x; i < n; i += 256)
        a = fmaxf(a, v[i]);
    a = wave_max_nonneg_f32(a);
    if ((threadIdx.x & 63) == 0)
        s[threadIdx.x >> 6] = a;
    __syncthreads();
    if (threadIdx.x == 0)
        out[0] = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
}

// One thread per weight word (32 codes of one row in one chunk).
__global__ __launch_bounds__(256) void k_pack_binary(const float *__restrict__ W, int64_t N, int64_t K, int64_t KC,
                                                     int64_t total, uint32_t *__restrict__ Wb)
{
    const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (id >= total)
        return;
    const int j = (int)(id & 3);
    const int r = (int)((id >> 2) & 63);
    const int64_t chunk = id >> 8;
    const int64_t c = chunk % KC, rb = chunk / KC;
    const int64_t n = rb * 64 + r;
    const int64_t k0 = c * 128 + 32 * j;
    uint32_t word = 0;
    if (n < N)
        for (int b = 0; b < 32; ++b)
            if (k0 + b < K && W[n * K + k0 + b] < 0.0f)
                word |= 1u << b;
    Wb[id] = word;
}

// Activation bits of one token per workgroup (plus its absmax): thread t builds words
// t, t + 256, ... of the row (layout as above), every slot of the padded row included.
__global__ __launch_bounds__(256) void k_binarize(const float *__restrict__ X, int64_t K, int layout, int64_t words,
                                                  uint32_t *__restrict__ Xb, float *__restrict__ sx)
{
    __shared__ float s[4];
    const int64_t m = blockIdx.x;
    const float *x = X + m * K;
    uint32_t *out = Xb + m * words;
    float a = 0.0f;
    const int per = layout == 1 ? 32 : 16;  // values per word
    for (int64_t i = threadIdx.x; i < words; i += 256) {
        uint32_t word = 0;
        for (int b = 0; b < per; ++b) {
            const int64_t k = i * per + b;
            if (k < K) {
                const float v = x[k];
                a = fmaxf(a, fabsf(v));
                if (v < 0.0f)
                    word |= 1u << (layout == 1 ? b : 8 * (b & 3) + 2 * (b >> 2));
            }
        }
        out[i] = word;
    }
    a = wave_max_nonneg_f32(a);
    if ((threadIdx.x & 63) == 0)
        s[threadIdx.x >> 6] = a;
    __syncthreads();
    if (threadIdx.x == 0)
        sx[m] = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
}

// The two GEMVs. A workgroup takes 16 weight rows; lane (r, j) = (lane / 4, lane % 4)
// reads word j of row r's 16 bytes in every chunk its wave owns (chunks wave, wave + 8,
// ...): 256 contiguous bytes per wave and chunk, and a grid of N / 16 workgroups. Per
// token and word: binary: xor, bcnt; ternary: xor, and, bcnt, with the word's non-zero
// count shared by the tokens. The four words of a row meet in a quad DPP sum, the waves
// in LDS. acc = K - 2 * differ (binary) or nonzero - 2 * differ (ternary); y = fp32(acc)
// * (scale_w * s_x[m]).
constexpr int kBitRows = 16;
constexpr int kBitUnroll = 8;

template <int CTRL>
__device__ inline int bits_dpp(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}

template <int MT, bool TERNARY>
__global__ __launch_bounds__(kBitWaves * 64) void k_gemv_bits(const uint32_t *__restrict__ Wq,
                                                              const float *__restrict__ w_scale,
                                                              const uint32_t *__restrict__ Xb, int64_t xwords,
                                                              const float *__restrict__ sx, int M, int64_t N, int64_t K,
                                                              int KC, float *__restrict__ Y, int32_t *__restrict__ ACC)
{
    __shared__ int red[kBitWaves][MT][kBitRows];
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int r = lane >> 2, j = lane & 3;
    // Rows past N (up to the packed 64-row padding) are read and never stored.
    const int64_t n = (int64_t)blockIdx.x * kBitRows + r;
    const uint32_t *wrow = Wq + ((n >> 6) * KC * 64 + (n & 63)) * 4 + j;  // + 256 words per chunk
    int differ[MT], nonzero = 0;
#pragma unroll
    for (int m = 0; m < MT; ++m)
        differ[m] = 0;
    // U chunks per wave in flight: every load of a batch -- the weight words, then the
    // token words -- is issued, unconditionally at clamped valid addresses (chunks past KC
    // re-read the last one, tokens past M re-read token M - 1), before any is used; the
    // arithmetic is guarded instead. A load under a branch would make each wait cover every
    // load issued before it, one round trip per chunk.
    constexpr int U = MT <= 4 ? kBitUnroll : kBitUnroll / 2;
    for (int c0 = wave; c0 < KC; c0 += kBitWaves * U) {
        uint32_t wv[U], xv[U][MT];
#pragma unroll
        for (int u = 0; u < U; ++u)
            wv[u] = wrow[(int64_t)min(c0 + u * kBitWaves, KC - 1) * 256];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int cc = min(c0 + u * kBitWaves, KC - 1);
#pragma unroll
            for (int m = 0; m < MT; ++m)
                xv[u][m] = Xb[(int64_t)min(m, M - 1) * xwords + 4 * cc + j];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u * kBitWaves;
            if (c < KC) {  // wave-uniform
                const uint32_t w = wv[u];
                uint32_t mag = 0, neg = w;
                if constexpr (TERNARY) {
                    mag = ~w & kLowBits;
                    neg = ~(w | (w >> 1)) & kLowBits;
                    nonzero += __builtin_popcount(mag);
                }
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    if (m < M) {
                        const uint32_t d = neg ^ xv[u][m];
                        differ[m] += __builtin_popcount(TERNARY ? (d & mag) : d);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        int v = (TERNARY ? nonzero : 0) - 2 * differ[m];
        v += bits_dpp<0xB1>(v);  // quad_perm [1,0,3,2]
        v += bits_dpp<0x4E>(v);  // quad_perm [2,3,0,1]
        if (j == 0)
            red[wave][m][r] = v;
    }
    __syncthreads();
    const float g = w_scale[0];
    for (int o = threadIdx.x; o < MT * kBitRows; o += kBitWaves * 64) {
        const int m = o / kBitRows, rr = o % kBitRows;
        const int64_t nn = (int64_t)blockIdx.x * kBitRows + rr;
        if (m >= M || nn >= N)
            continue;
        int s = TERNARY ? 0 : (int)K;
#pragma unroll
        for (int w = 0; w < kBitWaves; ++w)
            s += red[w][m][rr];
        if (ACC)
            ACC[(int64_t)m * N + nn] = s;
        if (Y)
            Y[(int64_t)m * N + nn] = (float)s * (g * sx[m]);
    }
}

template <bool TERNARY>
hipError_t launch_bits(const uint4 *W4, const float *w_scale, const uint32_t *Xb, int64_t xwords, const float *sx,
                       int64_t M, int64_t N, int64_t K, int KC, float *Y, int32_t *acc, hipStream_t s)
{
    const uint32_t *Wq = reinterpret_cast<const uint32_t *>(W4);
    const dim3 grid((unsigned)((N + kBitRows - 1) / kBitRows)), block(kBitWaves * 64);
    if (M <= 1)
        hipLaunchKernelGGL((k_gemv_bits<1, TERNARY>), grid, block, 0, s, Wq, w_scale, Xb, xwords, sx, (int)M, N, K,
                           KC, Y, acc);
    else if (M <= 4)
        hipLaunchKernelGGL((k_gemv_bits<4, TERNARY>), grid, block, 0, s, Wq, w_scale, Xb, xwords, sx, (int)M, N, K,
                           KC, Y, acc);
    else
        hipLaunchKernelGGL((k_gemv_bits<16, TERNARY>), grid, block, 0, s, Wq, w_scale, Xb, xwords, sx, (int)M, N, K,
                           KC, Y, acc);
    return hipGetLastError();
}

}  // namespace

int64_t act_bits_words(int64_t K, int layout)
{
    return layout == 1 ? (K + 127) / 128 * 4 : (K + 63) / 64 * 4;
}

hipError_t launch_pack_binary(const float *W, int64_t N, int64_t K, uint4 *Wb, float *w_scale, float *rowmax,
                              hipStream_t s)
{
    const int64_t NB = (N + 63) / 64, KC = (K + 127) / 128;
    hipLaunchKernelGGL(k_absmax_rows, dim3((unsigned)N), dim3(256), 0, s, W, K, rowmax);
    hipLaunchKernelGGL(k_max_of, dim3(1), dim3(256), 0, s, rowmax, N, w_scale);
    const int64_t total = NB * KC * 256;
    hipLaunchKernelGGL(k_pack_binary, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, W, N, K, KC, total,
                       reinterpret_cast<uint32_t *>(Wb));
    return hipGetLastError();
}

hipError_t launch_binarize(const float *X, int64_t M, int64_t K, int layout, uint32_t *Xb, float *sx, hipStream_t s)
{
    hipLaunchKernelGGL(k_binarize, dim3((unsigned)M), dim3(256), 0, s, X, K, layout, act_bits_words(K, layout), Xb,
                       sx);
    return hipGetLastError();
}

hipError_t launch_gemv_binary(const uint4 *Wb, const float *w_scale, const uint32_t *Xb, const float *sx, int64_t M,
                              int64_t N, int64_t K, float *Y, int32_t *acc, hipStream_t s)
{
    return launch_bits<false>(Wb, w_scale, Xb, act_bits_words(K, 1), sx, M, N, K, (int)((K + 127) / 128), Y, acc,
                              s);
}

hipError_t launch_gemv_ternary_a1(const uint4 *Wp, const float *w_scale, const uint32_t *Xb, const float *sx,
                                  int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc, hipStream_t s)
{
    return launch_bits<true>(Wp, w_scale, Xb, act_bits_words(K, 2), sx, M, N, K, (int)((K + 63) / 64), Y, acc, s);
}

}  // namespace bt
