// Device helpers shared by the kernels: wave64 reductions on gfx950 without LDS traffic
// (DPP within each 16-lane row -- quad swaps, half-row mirror, row mirror -- then
// v_permlane16_swap and v_permlane32_swap to combine the four rows; every lane ends with
// the result), the per-token int8 quantizer of four values, and vector-memory reads of
// the weight scales.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bt {

// Every control used below reads a lane of the same 16-lane row, so no lane is masked
// and the fill value never shows; passing 0 with bound_ctrl lets the compiler fold the
// move into the instruction that consumes it (that instruction's DPP form).
template <int CTRL>
__device__ inline int dpp_i(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}

constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <typename Op>
__device__ inline uint32_t wave_reduce_bits(uint32_t v, Op op)
{
    v = op(v, (uint32_t)dpp_i<kDppQuadXor1>((int)v));
    v = op(v, (uint32_t)dpp_i<kDppQuadXor2>((int)v));
    v = op(v, (uint32_t)dpp_i<kDppRowHalfMirror>((int)v));
    v = op(v, (uint32_t)dpp_i<kDppRowMirror>((int)v));
    // Each lane of a row sees its own row in one output of the swap and the partner
    // row in the other, so a symmetric op of the pair reduces across the pair of rows.
    auto p16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = op((uint32_t)p16[0], (uint32_t)p16[1]);
    auto p32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    v = op((uint32_t)p32[0], (uint32_t)p32[1]);
    return v;
}

// Maximum of values that are >= +0 and not NaN (absolute values reduced with fmaxf from
// 0): their bit patterns order like the values, so an unsigned maximum gives the same
// result without the float maximum's canonicalization of each operand.
__device__ inline float wave_max_nonneg_f32(float v)
{
    return __uint_as_float(wave_reduce_bits(__float_as_uint(v), [](uint32_t a, uint32_t b) { return a > b ? a : b; }));
}

__device__ inline int wave_sum_i32(int v)
{
    return (int)wave_reduce_bits((uint32_t)v, [](uint32_t a, uint32_t b) { return (uint32_t)((int)a + (int)b); });
}

// Per-token int8 quantization of four values (the rule of bt_quant_act), with the sum of the four
// codes. Both steps of the rule are kept exactly:
//  * p = x * inv rounded to fp32 (its own instruction, never contracted into an FMA);
//  * p + 1.5 * 2^23 lands in [2^23, 2^24), where the fp32 spacing is 1, so the addition
//    rounds p to the nearest integer with ties to even (rintf) and leaves q in the low
//    mantissa bits: bits = 0x4B400000 + q, low byte = q as int8.
// The clamp to +-127 is dropped because it never applies: with inv = RN(127 / a) and
// |x| <= a, |x * inv| <= 127 * (1 + 2^-24), so p is at most one ulp above 127 in
// magnitude and still rounds to +-127 (finite inputs; a = 0 gives inv = 0 and q = 0).
constexpr float kQuantMagic = 12582912.0f;  // 1.5 * 2^23
constexpr uint32_t kQuantMagicBits = 0x4B400000u;

__device__ inline uint32_t quant_pack4_sum(float4 v, float inv, int &sum)
{
    const uint32_t b0 = __float_as_uint(__fadd_rn(__fmul_rn(v.x, inv), kQuantMagic));
    const uint32_t b1 = __float_as_uint(__fadd_rn(__fmul_rn(v.y, inv), kQuantMagic));
    const uint32_t b2 = __float_as_uint(__fadd_rn(__fmul_rn(v.z, inv), kQuantMagic));
    const uint32_t b3 = __float_as_uint(__fadd_rn(__fmul_rn(v.w, inv), kQuantMagic));
    sum += (int)(b0 + b1 + b2 + b3 - 4u * kQuantMagicBits);
    // low bytes of b0..b3 into one dword (v_perm_b32: selector byte 0-3 picks a byte of
    // the second source, 4-7 of the first, 0x0c gives zero)
    const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x04000c0cu);
    return lo | hi;
}

// One fp32 value every lane needs (a matrix's gamma), read as a vector-memory load. It
// is then waited for through vmcnt, in order with the loads issued before it. A scalar
// load is waited for through lgkmcnt, which every LDS wait and workgroup barrier before
// the value's use also drains, so a slow read of the scale would stall those first.
__device__ inline float load_scale_vmem(const float *p)
{
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(p), (short)0, 4, 0x00020000);
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, 0, 0, 0));
}

// The weight scales of output rows n .. n+3: with row scales, entries n .. n+3 of the
// N-entry scale array (an entry past N reads 0); otherwise the matrix's one scale, four
// times. Four dword loads in both cases, with no branch: a branch here would make the
// compiler wait for the loads where the two paths meet instead of where the values are
// used, and offsets that are not constant apart keep it from merging the four loads into
// one 16-byte load whose range check would cover all four entries at once. N <= 2^30.
__device__ inline float4 load_scales4(const float *w_scale, int64_t n, int64_t N, bool rows)
{
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(w_scale), (short)0, rows ? (int)(uint32_t)min(4 * N, (int64_t)0xFFFFFFFF) : 4,
        0x00020000);
    const uint32_t off = rows ? (uint32_t)(4 * n) : 0u, step = rows ? 4u : 0u;
    return make_float4(__builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0)),
                       __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off + step, 0, 0)),
                       __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off + 2 * step, 0, 0)),
                       __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off + 3 * step, 0, 0)));
}

}  // namespace bt
