// Absmean ternarization and 2-bit packing of a weight matrix (offline, once per
// matrix), plus the inverse unpack used to inspect the packed codes.
//
// gamma = mean |W| is computed in a fixed fp64 order so that it is reproducible
// bit for bit: every row is summed k = 0..K-1 by one thread (the row tile is staged
// through LDS so the HBM reads stay coalesced), then one thread adds the row sums
// n = 0..N-1, divides by N*K in fp64 and rounds once to fp32. Codes follow
// RoundClip(W / gamma, -1, 1): +1 above gamma/2, -1 below -gamma/2, else 0
// ("bit-floor" page, "What's inside": pack.rs mean-abs threshold; "BitCompute"
// page, "Future Roadmap": four 1.58-bit weights per byte).
#include "bt_internal.h"

namespace bt {
namespace {

// One wave per 64 rows. For every 64-wide k slab the wave stages a 64x64 fp32
// tile in LDS (row-coalesced global reads), then thread t adds row t's 64 values
// in k order into its fp64 running sum.
__global__ __launch_bounds__(64) void k_row_abs_sum(const float *__restrict__ W, int64_t N, int64_t K,
                                                    double *__restrict__ rowsum)
{
    __shared__ float tile[64][65];
    const int t = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.x * 64;
    double acc = 0.0;
    for (int64_t k0 = 0; k0 < K; k0 += 64) {
        const int64_t col = k0 + t;
#pragma unroll 8
        for (int i = 0; i < 64; ++i) {
            const int64_t row = r0 + i;
            tile[i][t] = (row < N && col < K) ? W[row * K + col] : 0.0f;
        }
        __syncthreads();
        const int kmax = (int)((K - k0) < 64 ? (K - k0) : 64);
        for (int j = 0; j < kmax; ++j)
            acc += fabs((double)tile[t][j]);
        __syncthreads();
    }
    if (r0 + t < N)
        rowsum[r0 + t] = acc;
}

// Single workgroup: row sums are staged 256 at a time through LDS and thread 0
// adds them in row order.
__global__ __launch_bounds__(256) void k_gamma(const double *__restrict__ rowsum, int64_t N, int64_t K,
                                               float *__restrict__ gamma)
{
    __shared__ double buf[256];
    double total = 0.0;
    for (int64_t n0 = 0; n0 < N; n0 += 256) {
        const int64_t n = n0 + threadIdx.x;
        buf[threadIdx.x] = (n < N) ? rowsum[n] : 0.0;
        __syncthreads();
        if (threadIdx.x == 0) {
            const int cnt = (int)((N - n0) < 256 ? (N - n0) : 256);
            for (int i = 0; i < cnt; ++i)
                total += buf[i];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0)
        gamma[0] = (N > 0 && K > 0) ? (float)(total / (double)(N * K)) : 0.0f;
}

// Row-group scales: workgroup g adds the row sums of group g (rows end[g-1] .. end[g]-1)
// in row order exactly as k_gamma does for the whole matrix, then writes the group's
// scale to each of its rows.
__global__ __launch_bounds__(256) void k_gamma_groups(const double *__restrict__ rowsum, int64_t K, RowGroups groups,
                                                      float *__restrict__ row_scale)
{
    __shared__ double buf[256];
    __shared__ float s_gamma;
    const int gi = blockIdx.x;
    const int64_t r0 = gi == 0 ? 0 : groups.end[gi - 1], r1 = groups.end[gi];
    double total = 0.0;
    for (int64_t n0 = r0; n0 < r1; n0 += 256) {
        const int64_t n = n0 + threadIdx.x;
        buf[threadIdx.x] = (n < r1 && K > 0) ? rowsum[n] : 0.0;
        __syncthreads();
        if (threadIdx.x == 0) {
            const int cnt = (int)((r1 - n0) < 256 ? (r1 - n0) : 256);
            for (int i = 0; i < cnt; ++i)
                total += buf[i];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0)
        s_gamma = K > 0 ? (float)(total / (double)((r1 - r0) * K)) : 0.0f;
    __syncthreads();
    for (int64_t n = r0 + threadIdx.x; n < r1; n += 256)
        row_scale[n] = s_gamma;
}

// One group per row: the row's own mean |W|.
__global__ __launch_bounds__(256) void k_gamma_per_row(const double *__restrict__ rowsum, int64_t N, int64_t K,
                                                       float *__restrict__ row_scale)
{
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (n < N)
        row_scale[n] = K > 0 ? (float)(rowsum[n] / (double)K) : 0.0f;
}

__device__ inline uint32_t code_of(float w, float half)
{
    // t + 1 with t = +1 if w > gamma/2, -1 if w < -gamma/2, 0 otherwise.
    return (w > half) ? 2u : ((w < -half) ? 0u : 1u);
}

// One thread per packed row segment (16 bytes = 64 codes of one row in one chunk).
// gstride 0: one scale for the matrix (gamma[0]); 1: row n's scale is gamma[n].
__global__ __launch_bounds__(256) void k_pack(const float *__restrict__ W, int64_t N, int64_t K, int64_t KC,
                                              int64_t total, const float *__restrict__ gamma, int gstride,
                                              uint4 *__restrict__ Wp)
{
    const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (id >= total)
        return;
    const int r = (int)(id & 63);
    const int64_t chunk = id >> 6;
    const int64_t c = chunk % KC;
    const int64_t rb = chunk / KC;
    const int64_t n = rb * 64 + r;
    const float half = gamma[n < N ? n * gstride : 0] * 0.5f;
    uint32_t words[4];
    const bool full = (n < N) && (c * 64 + 64 <= K) && ((K & 3) == 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t k0 = c * 64 + 16 * j;
        float v[16];
        if (full) {
            const float4 *src = reinterpret_cast<const float4 *>(W + n * K + k0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 f = src[q];
                v[4 * q + 0] = f.x;
                v[4 * q + 1] = f.y;
                v[4 * q + 2] = f.z;
                v[4 * q + 3] = f.w;
            }
        }
        uint32_t word = 0;
#pragma unroll
        for (int b = 0; b < 16; ++b) {
            uint32_t code = 1u;  // padding: weight 0
            if (full)
                code = code_of(v[b], half);
            else if (n < N && k0 + b < K)
                code = code_of(W[n * K + k0 + b], half);
            word |= code << (8 * (b & 3) + 2 * (b >> 2));
        }
        words[j] = word;
    }
    Wp[id] = make_uint4(words[0], words[1], words[2], words[3]);
}

// One thread per packed word (16 codes): writes t = code - 1 into T [N,K].
__global__ __launch_bounds__(256) void k_unpack(const uint32_t *__restrict__ Wp, int64_t N, int64_t K,
                                                int64_t KC, int64_t total_words, int8_t *__restrict__ T)
{
    const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (id >= total_words)
        return;
    const int j = (int)(id & 3);
    const int r = (int)((id >> 2) & 63);
    const int64_t chunk = id >> 8;
    const int64_t c = chunk % KC;
    const int64_t rb = chunk / KC;
    const int64_t n = rb * 64 + r;
    if (n >= N)
        return;
    const uint32_t word = Wp[id];
    const int64_t k0 = c * 64 + 16 * j;
#pragma unroll
    for (int b = 0; b < 16; ++b) {
        if (k0 + b < K) {
            const int code = (int)((word >> (8 * (b & 3) + 2 * (b >> 2))) & 3u);
            T[n * K + k0 + b] = (int8_t)(code - 1);
        }
    }
}

}  // namespace

hipError_t launch_pack(const float *W, int64_t N, int64_t K, uint4 *Wp, float *gamma, double *rowsum,
                       hipStream_t s)
{
    const int64_t NB = (N + 63) / 64;
    const int64_t KC = (K + 63) / 64;
    if (N > 0 && K > 0)
        hipLaunchKernelGGL(k_row_abs_sum, dim3((unsigned)NB), dim3(64), 0, s, W, N, K, rowsum);
    hipLaunchKernelGGL(k_gamma, dim3(1), dim3(256), 0, s, rowsum, (N > 0 && K > 0) ? N : 0, K, gamma);
    const int64_t total = NB * KC * 64;
    if (total > 0)
        hipLaunchKernelGGL(k_pack, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, W, N, K, KC, total,
                           gamma, 0, Wp);
    return hipGetLastError();
}

hipError_t launch_pack_rows(const float *W, int64_t N, int64_t K, const RowGroups *groups, uint4 *Wp,
                            float *row_scale, double *rowsum, hipStream_t s)
{
    const int64_t NB = (N + 63) / 64;
    const int64_t KC = (K + 63) / 64;
    if (N == 0)
        return hipSuccess;
    if (K > 0)
        hipLaunchKernelGGL(k_row_abs_sum, dim3((unsigned)NB), dim3(64), 0, s, W, N, K, rowsum);
    if (groups)
        hipLaunchKernelGGL(k_gamma_groups, dim3((unsigned)groups->n), dim3(256), 0, s, rowsum, K, *groups,
                           row_scale);
    else
        hipLaunchKernelGGL(k_gamma_per_row, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s, rowsum, N, K,
                           row_scale);
    const int64_t total = NB * KC * 64;
    if (total > 0)
        hipLaunchKernelGGL(k_pack, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, W, N, K, KC, total,
                           row_scale, 1, Wp);
    return hipGetLastError();
}

hipError_t launch_unpack(const uint4 *Wp, int64_t N, int64_t K, int8_t *T, hipStream_t s)
{
    const int64_t NB = (N + 63) / 64;
    const int64_t KC = (K + 63) / 64;
    const int64_t words = NB * KC * 256;
    if (words > 0)
        hipLaunchKernelGGL(k_unpack, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s,
                           reinterpret_cast<const uint32_t *>(Wp), N, K, KC, words, T);
    return hipGetLastError();
}

}  // namespace bt
