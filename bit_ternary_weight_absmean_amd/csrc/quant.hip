// Fused per-token absmax int8 activation quantizer: one workgroup per token row.
// Rows of up to 32768 floats (16-byte aligned, K % 4 == 0) stay in registers between
// the absmax and the quantize pass (the row is read from memory once); other rows
// take a two-pass kernel that re-reads the row from cache.
//
// BitNet GPU guide ("How to Run BitNet Inference on GPU Using CUDA Kernels"),
// "Understanding the Two-Phase Architecture": activations are quantized to INT8
// with their own scales right before the INT8 x INT2 product; "bit-floor" page,
// "What's inside" (scale.rs): absmax scale, quantized on the fly before each GEMV.
//
// Per row m: a = max_k |x| (exact, order-free), inv = 127.0f / a (IEEE fp32
// division, correctly rounded), q = clamp(rint(x * inv), -127, 127) (round half to
// even; computed by quant_pack4_sum, which needs no clamp), s_x = a / 127.0f and
// sum_k q. The int8 row is written with stride ldq
// (K rounded up to 256) and zero padding, four codes per 32-bit store.
#include "bt_internal.h"
#include "wave.h"

namespace bt {
namespace {

constexpr int kThreads = 256;

__device__ inline float wave_max(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

__device__ inline int wave_sum(int v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v += __shfl_xor(v, off);
    return v;
}

// Zero-fill words [0, n) of `p`, spread over the whole grid (one store per word).
__device__ inline void clear_words_strided(unsigned *p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
        p[i] = 0u;
}

__global__ __launch_bounds__(kThreads) void k_quant_act(const float *__restrict__ X, int64_t K, int64_t ldq,
                                                        int8_t *__restrict__ Xq, float *__restrict__ sx,
                                                        int32_t *__restrict__ xsum,
    unsigned *__restrict__ clear, int64_t clear_words)
{
    __shared__ float red_f[kThreads / 64];
    __shared__ int red_i[kThreads / 64];
    const int tid = threadIdx.x;
    const int64_t m = blockIdx.x;
    clear_words_strided(clear, clear_words);
    const float *x = X + m * K;
    const bool vec = ((K & 3) == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);

    // Pass 1: absmax.
    float amax = 0.0f;
    if (vec) {
        for (int64_t k = 4 * tid; k < K; k += 4 * kThreads) {
            const float4 v = *reinterpret_cast<const float4 *>(x + k);
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        }
    } else {
        for (int64_t k = tid; k < K; k += kThreads)
            amax = fmaxf(amax, fabsf(x[k]));
    }
    amax = wave_max(amax);
    if ((tid & 63) == 0)
        red_f[tid >> 6] = amax;
    __syncthreads();
    amax = red_f[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w)
        amax = fmaxf(amax, red_f[w]);

    // Pass 2: quantize (the row is re-read from cache), pad with zeros, sum q.
    const bool zero = (amax == 0.0f);
    const float inv = zero ? 0.0f : 127.0f / amax;
    int8_t *q = Xq + m * ldq;
    int sum = 0;
    for (int64_t k = 4 * tid; k < ldq; k += 4 * kThreads) {
        // Values past K (and every value of an all-zero row, inv = 0) quantize to 0.
        float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (vec && k + 4 <= K) {
            v = *reinterpret_cast<const float4 *>(x + k);
        } else {
            if (k + 0 < K) v.x = x[k + 0];
            if (k + 1 < K) v.y = x[k + 1];
            if (k + 2 < K) v.z = x[k + 2];
            if (k + 3 < K) v.w = x[k + 3];
        }
        *reinterpret_cast<uint32_t *>(q + k) = quant_pack4_sum(v, inv, sum);
    }
    sum = wave_sum(sum);
    if ((tid & 63) == 0)
        red_i[tid >> 6] = sum;
    __syncthreads();
    if (tid == 0) {
        int total = 0;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w)
            total += red_i[w];
        sx[m] = zero ? 0.0f : amax / 127.0f;
        xsum[m] = total;
    }
}

// Register-resident variant: thread t holds float4 chunks t, t + 256, ... (at most C).
// Loads are clamped and masked rather than guarded, so they all issue before the
// first wait.
template <int C>
__global__ __launch_bounds__(kThreads) void k_quant_act_reg(const float *__restrict__ X, int64_t K, int64_t ldq,
                                                            int8_t *__restrict__ Xq, float *__restrict__ sx,
                                                            int32_t *__restrict__ xsum,
    unsigned *__restrict__ clear, int64_t clear_words)
{
    __shared__ float red_f[kThreads / 64];
    __shared__ int red_i[kThreads / 64];
    const int tid = threadIdx.x;
    const int64_t m = blockIdx.x;
    clear_words_strided(clear, clear_words);
    const float4 *x = reinterpret_cast<const float4 *>(X + m * K);
    const int nch = (int)(K >> 2);  // float4 chunks in the row (>= 1)

    float4 v[C];
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int idx = tid + c * kThreads;
        const float4 t = x[min(idx, nch - 1)];
        const bool in = idx < nch;
        v[c].x = in ? t.x : 0.0f;
        v[c].y = in ? t.y : 0.0f;
        v[c].z = in ? t.z : 0.0f;
        v[c].w = in ? t.w : 0.0f;
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[c].x), fabsf(v[c].y)), fmaxf(fabsf(v[c].z), fabsf(v[c].w))));
    }
    amax = wave_max(amax);
    if ((tid & 63) == 0)
        red_f[tid >> 6] = amax;
    __syncthreads();
    amax = red_f[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w)
        amax = fmaxf(amax, red_f[w]);

    const bool zero = (amax == 0.0f);
    const float inv = zero ? 0.0f : 127.0f / amax;
    uint32_t *q = reinterpret_cast<uint32_t *>(Xq + m * ldq);
    int sum = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int idx = tid + c * kThreads;
        // chunks past the row were loaded as zeros: they add 0 to the sum
        const uint32_t packed = quant_pack4_sum(v[c], inv, sum);
        if (idx < nch)
            q[idx] = packed;
    }
    // Zero padding up to ldq (a multiple of 4 bytes, as K is here).
    for (int64_t idx = nch + tid; idx < (ldq >> 2); idx += kThreads)
        q[idx] = 0u;
    sum = wave_sum(sum);
    if ((tid & 63) == 0)
        red_i[tid >> 6] = sum;
    __syncthreads();
    if (tid == 0) {
        int total = 0;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w)
            total += red_i[w];
        sx[m] = zero ? 0.0f : amax / 127.0f;
        xsum[m] = total;
    }
}

// Register kernel's float4 per thread (k_quant_act_reg<C>), or 0 for the two-pass kernel:
// the exact count up to 8, so that few loads are clamped duplicates (K = 2560 takes 3, not 4:
// 2B prefill at M = 2048 5.39 -> 5.38 ms, 7B decode at M = 8 1.049 -> 1.046 ms).
int quant_reg_chunks(int64_t K, bool aligned16)
{
    if (K <= 0 || (K % 4) != 0 || !aligned16)
        return 0;
    const int64_t per_thread = (K / 4 + kThreads - 1) / kThreads;  // float4 chunks per thread
    for (int c : {1, 2, 3, 4, 5, 6, 7, 8, 12, 16, 24, 32})
        if (per_thread <= c)
            return c;
    return 0;
}

}  // namespace

int plan_quant_act(int64_t M, int64_t K, char *buf, size_t len)
{
    (void)M;
    const int c = quant_reg_chunks(K, true);
    return c ? snprintf(buf, len, "k_quant_act_reg<C=%d>", c) : snprintf(buf, len, "k_quant_act");
}

hipError_t launch_quant_act(const float *X, int64_t M, int64_t K, int64_t ldq, int8_t *Xq, float *sx,
                            int32_t *xsum, unsigned *clear, int64_t clear_words, hipStream_t s)
{
    if (M <= 0)
        return hipGetLastError();
    const dim3 grid((unsigned)M), block(kThreads);
    const int c = quant_reg_chunks(K, (reinterpret_cast<uintptr_t>(X) % 16) == 0);
    const bool reg = c > 0;
    const int64_t per_thread = c;
    if (reg && per_thread <= 1)
        hipLaunchKernelGGL(k_quant_act_reg<1>, grid, block, 0, s, X, K, ldq, Xq, sx, xsum, clear, clear_words);
    else if (reg && per_thread <= 2)
        hipLaunchKernelGGL(k_quant_act_reg<2>, grid, block, 0, s, X, K, ldq, Xq, sx, xsum, clear, clear_words);
    else if (reg && per_thread <= 3)
        hipLaunchKernelGGL(k_quant_act_reg<3>, grid, block, 0, s, X, K, ldq, Xq, sx, xsum, clear, clear_words);
    else if (reg && per_thread <= 4)
        hipLaunchKernelGGL(k_quant_act_reg<4>, grid, block, 0, s, X, K, ldq, Xq, sx, xsum, clear, clear_words);
    else if (reg && per_thread <= 5)
        hipLaunchKernelGGL(k_quant_act_reg<5>, grid, block, 0, s, X, K, ldq, Xq, sx, xsum, clear, clear_words);
    else if (reg && per_thread <= 6)
        hipLaunchKernelGGL(k_quant_act_reg<6>, grid, block, 0, s, X, K, ldq, Xq, sx, xsum, clear, clear_words);
    else if (reg && per_thread <= 7)
        hipLaunchKernelGGL(k_quant_act_reg<7>, grid, block, 0, s, X, K, ldq, Xq, sx, xsum, clear, clear_words);
    else if (reg && per_thread <= 8)
        hipLaunchKernelGGL(k_quant_act_reg<8>, grid, block, 0, s, X, K, ldq, Xq, sx, xsum, clear, clear_words);
    else if (reg && per_thread <= 12)
        hipLaunchKernelGGL(k_quant_act_reg<12>, grid, block, 0, s, X, K, ldq, Xq, sx, xsum, clear, clear_words);
    else if (reg && per_thread <= 16)
        hipLaunchKernelGGL(k_quant_act_reg<16>, grid, block, 0, s, X, K, ldq, Xq, sx, xsum, clear, clear_words);
    else if (reg && per_thread <= 24)
        hipLaunchKernelGGL(k_quant_act_reg<24>, grid, block, 0, s, X, K, ldq, Xq, sx, xsum, clear, clear_words);
    else if (reg && per_thread <= 32)
        hipLaunchKernelGGL(k_quant_act_reg<32>, grid, block, 0, s, X, K, ldq, Xq, sx, xsum, clear, clear_words);
    else
        hipLaunchKernelGGL(k_quant_act, grid, block, 0, s, X, K, ldq, Xq, sx, xsum, clear, clear_words);
    return hipGetLastError();
}

}  // namespace bt
