// Ceiling kernels: what the hardware gives the workload's launch structure with no method
// arithmetic at all. Built into libbt_ceilings.so and used only by the benchmark to report
// the achievable roofline beside the published one:
//  - an empty kernel (optionally one store per workgroup): the per-launch floor of a HIP
//    graph of back-to-back launches;
//  - a plain streaming read of a buffer (16-byte loads, every load of a thread issued
//    before the first wait, an XOR fold that the compiler cannot drop): the time to move
//    the same bytes as a product launch, in one launch;
//  - an int8 MFMA loop (v_mfma_i32_16x16x64_i8, sixteen independent accumulators per
//    wave, operands that vary per lane, no memory traffic): the matrix-core rate the chip
//    sustains at the clock it runs under that load.
// None of this is part of the layer; it shares nothing with libbt.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int btc_v4i __attribute__((ext_vector_type(4)));

namespace {

constexpr uint32_t kNever = 0x9E3779B9u;  // a fold value the inputs are assumed not to give

__global__ void k_empty() {}

__global__ void k_store_one(uint32_t *out)
{
    if (threadIdx.x == 0)
        out[blockIdx.x] = blockIdx.x;
}

template <int U>
__global__ __launch_bounds__(256) void k_read(const uint4 *__restrict__ p, int64_t n16, uint32_t *__restrict__ out)
{
    const int64_t threads = (int64_t)gridDim.x * 256;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    uint4 v[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
        const int64_t idx = t + i * threads;
        v[i] = idx < n16 ? p[idx] : make_uint4(0, 0, 0, 0);
    }
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < U; ++i)
        x ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    if (x == kNever)
        out[blockIdx.x] = x;
}

__global__ __launch_bounds__(256) void k_mfma_loop(int iters, uint32_t seed, uint32_t *__restrict__ out)
{
    // Operands: a xorshift of the lane and the seed, so the matrix core sees data that
    // changes from lane to lane and from iteration to iteration like real operands.
    uint32_t s = seed ^ (threadIdx.x * 0x9E3779B1u) ^ (blockIdx.x * 0x85EBCA77u);
    auto next = [&]() {
        s ^= s << 13;
        s ^= s >> 17;
        s ^= s << 5;
        return s;
    };
    // Four operand pairs, taken in turn: consecutive MFMAs see different random bits.
    btc_v4i a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = btc_v4i{(int)next(), (int)next(), (int)next(), (int)next()};
        b[i] = btc_v4i{(int)next(), (int)next(), (int)next(), (int)next()};
    }
    btc_v4i acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        acc[i] = btc_v4i{0, 0, 0, 0};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i & 3], b[(i >> 2) & 3], acc[i], 0, 0, 0);
    }
    int x = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        x ^= acc[i].x ^ acc[i].y ^ acc[i].z ^ acc[i].w;
    if ((uint32_t)x == kNever)
        out[blockIdx.x] = (uint32_t)x;
}

}  // namespace

extern "C" {

// Launch `grid` workgroups of `block` threads of an empty kernel (with_store: each
// workgroup's first thread writes one word of out[grid]). Returns a hipError_t.
int btc_launch_empty(int grid, int block, int with_store, uint32_t *out, void *stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (with_store)
        hipLaunchKernelGGL(k_store_one, dim3(grid), dim3(block), 0, s, out);
    else
        hipLaunchKernelGGL(k_empty, dim3(grid), dim3(block), 0, s);
    return (int)hipGetLastError();
}

// Read `bytes` (a multiple of 16) from p once, `loads` 16-byte loads per thread (1, 2, 4
// or 8). out needs one word per workgroup: ceil(bytes / 16 / loads / 256) words.
int btc_read_blocks(int64_t bytes, int loads) { return (int)((bytes / 16 + (int64_t)loads * 256 - 1) / ((int64_t)loads * 256)); }

int btc_launch_read(const void *p, int64_t bytes, int loads, uint32_t *out, void *stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t n16 = bytes / 16;
    const dim3 grid((unsigned)btc_read_blocks(bytes, loads)), block(256);
    const uint4 *q = static_cast<const uint4 *>(p);
    switch (loads) {
    case 1: hipLaunchKernelGGL(k_read<1>, grid, block, 0, s, q, n16, out); break;
    case 2: hipLaunchKernelGGL(k_read<2>, grid, block, 0, s, q, n16, out); break;
    case 4: hipLaunchKernelGGL(k_read<4>, grid, block, 0, s, q, n16, out); break;
    case 8: hipLaunchKernelGGL(k_read<8>, grid, block, 0, s, q, n16, out); break;
    default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

// int8 MFMA loop on `blocks` workgroups of four waves, each wave issuing iters * 16
// v_mfma_i32_16x16x64_i8 (16 * 16 * 64 * 2 ops each). out needs `blocks` words.
int btc_launch_mfma(int blocks, int iters, uint32_t seed, uint32_t *out, void *stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(k_mfma_loop, dim3(blocks), dim3(256), 0, s, iters, seed, out);
    return (int)hipGetLastError();
}

}  // extern "C"
