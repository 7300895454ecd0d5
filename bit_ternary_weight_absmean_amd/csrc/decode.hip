// Decode product on int8 MFMA for 1 <= M <= 16 tokens (pre-quantized activations), and for
// M <= 4 also with the per-token activation quantizer fused in (fp32 x in, fp32 y out: one
// launch per linear layer).
//
// "bit-floor" page, "The core math": integer inner loop, one scale multiply at the
// end; "BitCompute" page, "Features": ternary weights make the product add /
// subtract / skip; BitNet GPU guide, "Key Components and Source Code Architecture":
// decode is the memory-bound phase. At decode sizes a launch is dominated by fixed
// latency (dispatch, one HBM round trip, reductions), so both kernels put every
// memory request of a wave in flight first and keep the dependent chain short.
//
// Work split. A workgroup owns RB 16-row weight blocks (RB = 1, 2 or 4, picked so
// that small matrices still spread over the 256 CUs) and all of K. A "step" is 256 k:
// lane group g = lane / 16 takes the 64-k chunk 4*step + g and lane row r = lane % 16,
// so one step of one block is 64 lanes x 16 bytes. Waves take steps round-robin and
// load U of them per register batch (U * RB <= 8 uint4 per lane), one batch ahead.
//
// MFMA mapping (v_mfma_i32_16x16x64_i8, D = A * B): A = weights, 16 rows x 64 k;
// B = tokens, 64 k x 16 columns (columns m >= M: zero in the direct kernel, a repeat of
// token M - 1 in the fused one; either way never stored). For mask s the A dword j
// of a lane is (word j & mask s): its byte e is the code of k = 64c + 16j + 4s + e
// times 4^s (times 16 for s = 3). The matching B dword is bytes 16j + 4s .. +3 of
// the lane's 64 activation bytes. Three accumulators (weights 1, 4, 16) recombine
// exactly as a1 + (a4 >> 2) + (a16 >> 4); the code offset (+1) is removed by
// subtracting sum_k q. The output lane holds D[4g + v][r]: weight row 4g + v of the
// block, token r.
//
// Fused quantization (k_linear_decode). BitNet GPU guide, "Understanding the
// Two-Phase Architecture": activations are quantized to INT8 with their own scale
// before the INT8 x INT2 product. Each workgroup loads the fp32 tokens into
// registers first (they are small and L2-resident), then issues its weight loads,
// so the quantizer only waits for the activations. It uses the arithmetic of
// bt_quant_act (a = max |x|, inv = 127.0f / a, q = clamp(rint(x * inv), -127, 127),
// s_x = a / 127.0f) and stages the int8 tokens in LDS (row pitch = the bytes the
// quantizer stores per token, at least K rounded up to a whole 256-k step and zero
// past K, plus 16 so that the 16-byte operand reads of 16 tokens hit distinct banks; see
// fused_pitch). Within each 64-k chunk the quantizer stores the 4 x 4 dwords
// transposed: bytes 16s .. 16s + 15 hold dwords s, s + 4, s + 8, s + 12 of the chunk, the
// B operand of mask s, so each operand is one 16-byte LDS read with no register moves.
// Slots outside the matrix need no masking there: weight chunks past K (clamped
// duplicates) meet zero activations, and rows past N are never stored.
#include "bt_internal.h"
#include "wave.h"

namespace bt {
namespace {

constexpr int kMaxM = 16;
constexpr int kPitchPad = 16;
constexpr int kXRegs = 16;     // float4 of fp32 activations a thread keeps in registers
constexpr int kFusedWaves = 8;
constexpr int kDirectWaves = 4;

__host__ __device__ constexpr int batch_steps(int rb) { return 8 / rb; }

// Four MFMAs of one step for each of the RB row blocks.
template <int RB>
__device__ inline void mfma_step(const uint4 (&w)[RB], const int32_t (&xw)[16], v4i (&a1)[RB], v4i (&a4)[RB],
                                 v4i (&a16)[RB])
{
    const v4i b0 = {xw[0], xw[4], xw[8], xw[12]};
    const v4i b1 = {xw[1], xw[5], xw[9], xw[13]};
    const v4i b2 = {xw[2], xw[6], xw[10], xw[14]};
    const v4i b3 = {xw[3], xw[7], xw[11], xw[15]};
#pragma unroll
    for (int k = 0; k < RB; ++k) {
        const uint32_t pw[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
        v4i s0, s1, s2, s3;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            s0[j] = (int)(pw[j] & kMask0);
            s1[j] = (int)(pw[j] & kMask1);
            s2[j] = (int)(pw[j] & kMask2);
            s3[j] = (int)((pw[j] >> 2) & kMask2);
        }
        a1[k] = __builtin_amdgcn_mfma_i32_16x16x64_i8(s0, b0, a1[k], 0, 0, 0);
        a4[k] = __builtin_amdgcn_mfma_i32_16x16x64_i8(s1, b1, a4[k], 0, 0, 0);
        a16[k] = __builtin_amdgcn_mfma_i32_16x16x64_i8(s2, b2, a16[k], 0, 0, 0);
        a16[k] = __builtin_amdgcn_mfma_i32_16x16x64_i8(s3, b3, a16[k], 0, 0, 0);
    }
}

// Weight uint4 of block b16, chunk c, lane row r, from a clamped, always valid address
// (callers load only with KC >= 1). Slots outside the matrix are not masked here: a
// select or a branch right after a load would make the compiler wait for that load before
// the next one. k_gemv_direct masks them where the values are used (mask_w); the other
// kernels need no mask, because chunks past K meet zero activations there and rows past
// N are never stored.
__device__ inline v4i load_w_raw(const uint4 *__restrict__ Wp, int b16, int NB16, int c, int KC, int r)
{
    const int bb = min(b16, NB16 - 1), cc = min(max(c, 0), KC - 1);
    return reinterpret_cast<const v4i *>(Wp)[((int64_t)(bb >> 2) * KC + cc) * 64 + 16 * (bb & 3) + r];
}

// The loaded words where keep, else four padding words (sixteen zero weights).
__device__ inline uint4 mask_w(const v4i &w, bool keep)
{
    const int k = keep ? -1 : 0;
    const int pad = (int)kPadWord & ~k;
    return make_uint4((uint32_t)((w[0] & k) | pad), (uint32_t)((w[1] & k) | pad), (uint32_t)((w[2] & k) | pad),
                      (uint32_t)((w[3] & k) | pad));
}

__device__ inline void unpack16(const uint4 (&v)[4], int32_t (&xw)[16])
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        xw[4 * q + 0] = (int32_t)v[q].x;
        xw[4 * q + 1] = (int32_t)v[q].y;
        xw[4 * q + 2] = (int32_t)v[q].z;
        xw[4 * q + 3] = (int32_t)v[q].w;
    }
}

// One step, one row block, with the four B operands already in mask order (the fused
// kernel's transposed LDS chunks): mfma_step<1> without the register transpose.
__device__ inline void mfma_step_t(const v4i &w, const v4i (&b)[4], v4i &a1, v4i &a4, v4i &a16)
{
    v4i s0, s1, s2, s3;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t pw = (uint32_t)w[j];
        s0[j] = (int)(pw & kMask0);
        s1[j] = (int)(pw & kMask1);
        s2[j] = (int)(pw & kMask2);
        s3[j] = (int)((pw >> 2) & kMask2);
    }
    a1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(s0, b[0], a1, 0, 0, 0);
    a4 = __builtin_amdgcn_mfma_i32_16x16x64_i8(s1, b[1], a4, 0, 0, 0);
    a16 = __builtin_amdgcn_mfma_i32_16x16x64_i8(s2, b[2], a16, 0, 0, 0);
    a16 = __builtin_amdgcn_mfma_i32_16x16x64_i8(s3, b[3], a16, 0, 0, 0);
}

// Byte offset, within an LDS token row, of the activation dword k4 (k = 4 k4 .. + 3):
// chunk k4 / 16, transposed inside the chunk (dword d = k4 % 16 goes to 16 (d % 4) +
// 4 (d / 4)).
__device__ inline int lds_x_offset(int k4) { return (k4 >> 4) * 64 + 16 * (k4 & 3) + 4 * ((k4 >> 2) & 3); }

// The epilogue wave's sum of the other k-splits' partials: all NP LDS reads are issued before
// the first add (one round trip; left to itself the compiler reuses the first reads'
// registers for the later ones and waits in between). red: the first partner's slot, the
// partners 64 slots apart.
template <int NP>
__device__ inline void add_ksplit_partials(const int4 *red, int (&part)[4])
{
    if constexpr (NP > 0) {
        int4 o[NP];
#pragma unroll
        for (int j = 0; j < NP; ++j)
            o[j] = red[j * 64];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NP; ++j)
            part[0] += o[j].x, part[1] += o[j].y, part[2] += o[j].z, part[3] += o[j].w;
    }
}

// Partial accumulators of all waves -> y and acc. red[w][k][v][lane]; o = m * rows + nl.
// token_stats(m, qs, sx) supplies sum_k q and s_x of token m.
// w_scale[rs ? n : 0] is the weight scale of output row n.
template <int WAVES, int RB, typename Stats>
__device__ inline void epilogue(const int *red, int tid, int M, int64_t N, const float *__restrict__ w_scale, int rs,
                                Stats token_stats, float *__restrict__ Y, int32_t *__restrict__ ACC)
{
    constexpr int rows = 16 * RB;
    for (int o = tid; o < M * rows; o += WAVES * 64) {
        const int m = o / rows;
        const int nl = o - m * rows;
        const int64_t n = (int64_t)blockIdx.x * rows + nl;
        if (n >= N)
            continue;
        const int k = nl >> 4, gg = (nl >> 2) & 3, v = nl & 3;
        const int src = gg * 16 + m;
        int s = 0;
#pragma unroll
        for (int w = 0; w < WAVES; ++w)
            s += red[((w * RB + k) * 4 + v) * 64 + src];
        int qs;
        float sxm;
        token_stats(m, qs, sxm);
        const int acc = s - qs;
        if (ACC)
            ACC[(int64_t)m * N + n] = acc;
        if (Y)
            Y[(int64_t)m * N + n] = (float)acc * (w_scale[rs ? n : 0] * sxm);
    }
}

// ------------------------------------------------------------ direct kernels
// Pre-quantized int8 activations read straight from global memory (L2) per step.
// k_gemv_direct (two or four row blocks per workgroup): one batch of U = 2 steps at a
// time, masks where the values are used. k_gemv_direct_db (one row block): see below.
template <int RB>
__global__ __launch_bounds__(kDirectWaves * 64) void k_gemv_direct(
    const uint4 *__restrict__ Wp, const float *__restrict__ w_scale, const int8_t *__restrict__ Xq, int64_t ldq,
    const float *__restrict__ sx_in, const int32_t *__restrict__ xsum_in, int M, int64_t N, int KC, int NB16,
    float *__restrict__ Y, int32_t *__restrict__ ACC, int rs)
{
    constexpr int WAVES = kDirectWaves;
    constexpr int U = 2;
    __shared__ int red[WAVES * RB * 256];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int g = lane >> 4;
    const int r = lane & 15;
    const int nsteps = (KC + 3) >> 2;
    const int nmine = (wave < nsteps) ? (nsteps - 1 - wave) / WAVES + 1 : 0;

    v4i a1[RB], a4[RB], a16[RB];
#pragma unroll
    for (int k = 0; k < RB; ++k)
        a1[k] = a4[k] = a16[k] = v4i{0, 0, 0, 0};

    for (int i0 = 0; i0 < nmine; i0 += U) {
        // Every load of the batch first, at clamped addresses; the masks where used.
        v4i w[U][RB];
        v4i xv[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = 4 * (wave + WAVES * (i0 + u)) + g;
#pragma unroll
            for (int k = 0; k < RB; ++k)
                w[u][k] = load_w_raw(Wp, blockIdx.x * RB + k, NB16, c, KC, r);
            const v4i *p = reinterpret_cast<const v4i *>(Xq + (int64_t)min(r, M - 1) * ldq +
                                                         (int64_t)min(c, KC - 1) * 64);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                xv[u][q] = p[q];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (i0 + u >= nmine)
                break;
            const int c = 4 * (wave + WAVES * (i0 + u)) + g;
            const int keep = (c < KC && r < M) ? -1 : 0;
            uint4 xk[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                xk[q] = make_uint4((uint32_t)(xv[u][q][0] & keep), (uint32_t)(xv[u][q][1] & keep),
                                   (uint32_t)(xv[u][q][2] & keep), (uint32_t)(xv[u][q][3] & keep));
            int32_t xw[16];
            unpack16(xk, xw);
            uint4 wm[RB];
#pragma unroll
            for (int k = 0; k < RB; ++k)
                wm[k] = mask_w(w[u][k], c < KC && blockIdx.x * RB + k < NB16);
            mfma_step<RB>(wm, xw, a1, a4, a16);
        }
    }
#pragma unroll
    for (int k = 0; k < RB; ++k)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            red[((wave * RB + k) * 4 + v) * 64 + lane] = a1[k][v] + (a4[k][v] >> 2) + (a16[k][v] >> 4);
    __syncthreads();
    epilogue<WAVES, RB>(red, tid, M, N, w_scale, rs,
                        [&](int m, int &qs, float &sxm) {
                            qs = xsum_in[m];
                            sxm = sx_in[m];
                        },
                        Y, ACC);
}

// k_gemv_direct_db: wave w of the workgroup takes steps w, w + 4, ... of the workgroup's
// RB row blocks, U steps per register batch, two batches in flight (as in the fused
// kernel: measured faster with one row block per workgroup, e.g. 7B down at M = 8 9.9 ->
// 7.8 us). Every load is issued
// raw at a clamped address and nothing is masked: activation chunks past K come from the
// zero padding of the Xq rows (bt_act_row_bytes(K) bytes: whole 256-k steps), so weight
// chunks past K (clamped duplicates) meet zeros; token columns r >= M re-read token
// M - 1 and rows past N are never stored.
template <int RB, int U>
__global__ __launch_bounds__(kDirectWaves * 64) void k_gemv_direct_db(
    const uint4 *__restrict__ Wp, const float *__restrict__ w_scale, const int8_t *__restrict__ Xq, int64_t ldq,
    const float *__restrict__ sx_in, const int32_t *__restrict__ xsum_in, int M, int64_t N, int KC, int NB16,
    float *__restrict__ Y, int32_t *__restrict__ ACC, int rs)
{
    constexpr int WAVES = kDirectWaves;
    __shared__ int red[WAVES * RB * 256];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int g = lane >> 4;
    const int r = lane & 15;
    const int nsteps = (KC + 3) >> 2;
    const int nmine = (wave < nsteps) ? (nsteps - 1 - wave) / WAVES + 1 : 0;
    const int nb = (nmine + U - 1) / U;
    const int8_t *xrow = Xq + (int64_t)min(r, M - 1) * ldq;
    const int cmax = 4 * nsteps - 1;  // last 64-k chunk of the zero-padded activation row

    v4i a1[RB], a4[RB], a16[RB];
#pragma unroll
    for (int k = 0; k < RB; ++k)
        a1[k] = a4[k] = a16[k] = v4i{0, 0, 0, 0};

    v4i w0[U][RB], x0[U][4], w1[U][RB], x1[U][4];
    auto load_batch = [&](auto &w, auto &x, int b) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = 4 * (wave + WAVES * (b * U + u)) + g;
#pragma unroll
            for (int k = 0; k < RB; ++k)
                w[u][k] = load_w_raw(Wp, blockIdx.x * RB + k, NB16, c, KC, r);
            const v4i *p = reinterpret_cast<const v4i *>(xrow + (int64_t)min(c, cmax) * 64);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                x[u][q] = p[q];
        }
    };
    auto compute_batch = [&](const auto &w, const auto &x, int b) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (b * U + u < nmine) {
                int32_t xw[16];
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int d = 0; d < 4; ++d)
                        xw[4 * q + d] = x[u][q][d];
                uint4 wk[RB];
#pragma unroll
                for (int k = 0; k < RB; ++k)
                    wk[k] = make_uint4((uint32_t)w[u][k][0], (uint32_t)w[u][k][1], (uint32_t)w[u][k][2],
                                       (uint32_t)w[u][k][3]);
                mfma_step<RB>(wk, xw, a1, a4, a16);
            }
        }
    };
    // K = 0 (nsteps = 0): no loads at all (the operand pointers may be null).
    if (nsteps > 0) {
        load_batch(w0, x0, 0);
        load_batch(w1, x1, 1);
    }
    // Pairs of batches while the next pair exists, its loads unconditional (at clamped valid
    // addresses: at most one batch past the last), then the last pair with no loads. A load
    // under a branch would leave the compiler unable to count the loads issued after a batch,
    // and its waits for that batch would then cover the batch behind it too.
    int b = 0;
    for (; b + 2 < nb; b += 2) {
        compute_batch(w0, x0, b);
        load_batch(w0, x0, b + 2);
        compute_batch(w1, x1, b + 1);
        load_batch(w1, x1, b + 3);
    }
    compute_batch(w0, x0, b);
    compute_batch(w1, x1, b + 1);
#pragma unroll
    for (int k = 0; k < RB; ++k)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            red[((wave * RB + k) * 4 + v) * 64 + lane] = a1[k][v] + (a4[k][v] >> 2) + (a16[k][v] >> 4);
    __syncthreads();
    epilogue<WAVES, RB>(red, tid, M, N, w_scale, rs,
                        [&](int m, int &qs, float &sxm) {
                            qs = xsum_in[m];
                            sxm = sx_in[m];
                        },
                        Y, ACC);
}

// ------------------------------------------------------------- fused kernel
// Bytes of one token's quantized row in LDS. The register path (RX > 0) stores every
// slot a thread holds, RX * 512 dwords (at least the KC4 * 64 bytes the products read:
// the launcher's RX covers K), so its stores need no per-lane guard; the streaming path
// stores KC4 * 64 bytes. The 16-byte pad staggers the rows across LDS banks.
__host__ __device__ constexpr int fused_pitch(int KC4, int rx)
{
    return (rx > 0 && rx * kFusedWaves * 64 * 4 > KC4 * 64 ? rx * kFusedWaves * 64 * 4 : KC4 * 64) + kPitchPad;
}

// Eight waves per workgroup. Wave w owns the 16-row block blockIdx.x * (8/S) + w / S
// and the k-split w % S of it: steps st = w % S, w % S + S, ... For S = 1 a wave owns
// all of K and its epilogue runs straight from its MFMA registers; for S > 1 the S
// partial sums of a block are added through LDS by the block's last k-split, which owns
// the fewest steps. MT = compile-time token capacity (M <= MT). RX > 0: each thread keeps
// RX float4 of each token in registers for the quantizer (the launcher picks the smallest
// power of two that covers K, so the loads need no guards); RX = 0: the tokens are
// streamed from memory twice (large or unaligned K).
//
// Every instruction between the arrival of the activations and the stores is on the
// launch's critical path (at 2B sizes the weights are in registers well before the
// quantizer is done), and a SIMD runs two of the eight waves: the work that does not
// need the token maxima is done before or after the barriers around the quantizer (one,
// after the absmax, with one row block per workgroup: each wave then reads back only the
// activations it quantized itself; two otherwise).
template <int MT, int S, int RX, int U, bool ROWS>
__global__ __launch_bounds__(kFusedWaves * 64) void k_linear_decode(
    const uint4 *__restrict__ Wp, const float *__restrict__ w_scale, const float *__restrict__ X,
    float *__restrict__ Y, int32_t *__restrict__ ACC, int M, int N, int K)
{
    // The arguments fill the 13 dwords gfx950 preloads into SGPRs, so no scalar load of
    // the kernel arguments is pending at the first barrier. ROWS: w_scale holds one scale
    // per output row (else w_scale[0] is the matrix's scale: one load instead of four).
    constexpr int WAVES = kFusedWaves;
    static_assert(WAVES == 8, "the token maxima are read as two float4");
    const int KC = (K + 63) >> 6;
    const int NB16 = ((N + 63) >> 6) * 4;
    constexpr int T = WAVES * 64;
    // U: steps per register batch (two batches in flight), sized by the launcher to the
    // steps a wave owns, so the first two batches hold few clamped duplicate loads.
    constexpr int RPT = RX > 0 ? RX : 1;
    constexpr int RBW = WAVES / S;    // row blocks per workgroup
    constexpr bool regpath = RX > 0;  // then K4 >= 1 and K4 <= RX * T (the launcher checks)
    // One row block per workgroup (S = 8): all eight waves' partials meet in the k-split
    // sum, so each wave subtracts its own share of sum_k q there instead of publishing it
    // to the other waves.
    constexpr bool fold_q = regpath && RBW == 1;
    // Register path with k-splits: the wave sums of q are formed after the quantizer's
    // LDS stores, off the path to the first MFMA.
    constexpr bool late_q = regpath && S > 1;
    constexpr int KE = S - 1;         // the k-split that runs the epilogue
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    float *s_apart = reinterpret_cast<float *>(smem);                  // [kMaxM][WAVES]
    int *s_qpart = reinterpret_cast<int *>(s_apart + WAVES * kMaxM);   // [kMaxM][WAVES]
    int4 *red = reinterpret_cast<int4 *>(s_qpart + WAVES * kMaxM);    // [WAVES][64] (S > 1)
    int8_t *xq = reinterpret_cast<int8_t *>(red + (S > 1 ? WAVES * 64 : 0));
    const int KC4 = (KC + 3) & ~3;  // chunks in whole 256-k steps (zero-filled past KC)
    const int pitch = fused_pitch(KC4, RX);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int g = lane >> 4;
    const int r = lane & 15;
    const int ks = wave % S;
    const int b16 = blockIdx.x * RBW + wave / S;
    const int K4 = (K + 3) >> 2;

    auto load4 = [&](const float *xr, int k4) -> float4 {
        if (K % 4 == 0 && (reinterpret_cast<uintptr_t>(X) & 15) == 0)
            return reinterpret_cast<const float4 *>(xr)[k4];
        const int k = 4 * k4;
        return make_float4(xr[k], (k + 1 < K) ? xr[k + 1] : 0.0f, (k + 2 < K) ? xr[k + 2] : 0.0f,
                           (k + 3 < K) ? xr[k + 3] : 0.0f);
    };

    // 1. Activations first (waiting for them then does not wait for the weights): RX
    //    unconditional loads per token at clamped addresses (tokens past M re-read
    //    token M - 1); the masks are applied in step 3, where the values are used.
    v4i xraw[MT][RPT];
    if constexpr (regpath) {
        const v4i *X4 = reinterpret_cast<const v4i *>(X);
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int i = 0; i < RPT; ++i)
                xraw[m][i] = X4[(m == 0 ? 0 : (int64_t)min(m, M - 1) * K4) + min(tid + i * T, K4 - 1)];
        // Keep them ahead of the weight loads in issue order: the quantizer then waits
        // for the activations only (vector-memory operations complete in order). Nothing
        // else is computed before them.
        __builtin_amdgcn_sched_barrier(0);
    }
    const int nsteps = (KC + 3) >> 2;
    const int nmine = (ks < nsteps) ? (nsteps - 1 - ks) / S + 1 : 0;
    const int nb = (nmine + U - 1) / U;

    // 2. The wave's first weight batch.
    v4i wa[U], wb[U];
    auto load_batch = [&](v4i (&w)[U], int b) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            w[u] = load_w_raw(Wp, b16, NB16, 4 * (ks + S * (b * U + u)) + g, KC, r);
    };
    if constexpr (regpath) {
        // K >= 4, so KC >= 1 and the clamped addresses are valid: no guard (a branch
        // here would make the quantizer's wait cover the weight loads as well).
        load_batch(wa, 0);
        load_batch(wb, 1);
    } else {
        if (nb > 0)
            load_batch(wa, 0);
        if (nb > 1)
            load_batch(wb, 1);
    }
    // After the weights: the epilogue is the only user, and it waits for them anyway.
    // Lane (g, r) stores rows 4g .. 4g+3 of its block.
    float4 gam;
    if constexpr (ROWS) {
        gam = load_scales4(w_scale, (int64_t)b16 * 16 + 4 * g, N, true);
    } else {
        const float g1 = load_scale_vmem(w_scale);
        gam = make_float4(g1, g1, g1, g1);
    }

    // 3. Per-token absmax: wave partials in LDS.
    float4 xr[MT][RPT];
    if constexpr (regpath) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int keep = (m < M && tid + i * T < K4) ? -1 : 0;
                xr[m][i] = make_float4(__int_as_float(xraw[m][i][0] & keep), __int_as_float(xraw[m][i][1] & keep),
                                       __int_as_float(xraw[m][i][2] & keep), __int_as_float(xraw[m][i][3] & keep));
            }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m < M) {  // a guard, not a break: the loop must stay fully unrolled
                float a = 0.0f;
#pragma unroll
                for (int i = 0; i < RPT; ++i)
                    a = fmaxf(a, fmaxf(fmaxf(fabsf(xr[m][i].x), fabsf(xr[m][i].y)),
                                       fmaxf(fabsf(xr[m][i].z), fabsf(xr[m][i].w))));
                a = wave_max_nonneg_f32(a);
                if (lane == 0)
                    s_apart[m * WAVES + wave] = a;
            }
        }
    } else {
        for (int m = 0; m < M; ++m) {
            const float *xm = X + (int64_t)m * K;
            float a = 0.0f;
#pragma unroll 4
            for (int k4 = tid; k4 < K4; k4 += T) {
                const float4 v = load4(xm, k4);
                a = fmaxf(a, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
            }
            a = wave_max_nonneg_f32(a);
            if (lane == 0)
                s_apart[m * WAVES + wave] = a;
        }
    }
    __syncthreads();

    // 4. Quantize into LDS; per-lane (register path with k-splits) or per-wave partial
    //    sums of q.
    auto token_amax = [&](int m) {
        // the eight wave maxima, compared as bit patterns (all >= +0, none NaN)
        const uint4 u = reinterpret_cast<const uint4 *>(s_apart + m * WAVES)[0];
        const uint4 v = reinterpret_cast<const uint4 *>(s_apart + m * WAVES)[1];
        const uint32_t a = max(max(max(u.x, u.y), max(u.z, u.w)), max(max(v.x, v.y), max(v.z, v.w)));
        return __uint_as_float(a);
    };
    // absmax of the token this lane's output column holds (token r), for the epilogue.
    float amax_r = 0.0f;
    int qlane[MT];  // late_q: this lane's sum of q per token
    if constexpr (regpath) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            qlane[m] = 0;
            if (m < M) {
                const float amax = token_amax(m);
                const float inv = (amax == 0.0f) ? 0.0f : 127.0f / amax;
                if (m == r)
                    amax_r = amax;
                int8_t *qrow = xq + m * pitch;
                int sum = 0;
#pragma unroll
                for (int i = 0; i < RPT; ++i) {
                    // Wave-uniform: skip slots wholly past the part of the row the products
                    // read; the rest store unguarded (the pitch holds every slot, and xr is
                    // zero past K, so the padding up to KC4 chunks comes out zero).
                    if (wave * 64 + i * T < KC4 * 16) {
                        const uint32_t p = quant_pack4_sum(xr[m][i], inv, sum);
                        *reinterpret_cast<uint32_t *>(qrow + lds_x_offset(tid + i * T)) = p;
                    }
                }
                if constexpr (late_q) {
                    qlane[m] = sum;
                } else {
                    sum = wave_sum_i32(sum);
                    if (lane == 0)
                        s_qpart[m * WAVES + wave] = sum;
                }
            }
        }
    } else {
        for (int m = 0; m < M; ++m) {
            const float amax = token_amax(m);
            const float inv = (amax == 0.0f) ? 0.0f : 127.0f / amax;
            if (m == r)
                amax_r = amax;
            int8_t *qrow = xq + m * pitch;
            const float *xm = X + (int64_t)m * K;
            int sum = 0;
            for (int k4 = tid; k4 < KC4 * 16; k4 += T) {
                const uint32_t p = (k4 < K4) ? quant_pack4_sum(load4(xm, k4), inv, sum) : 0u;
                *reinterpret_cast<uint32_t *>(qrow + lds_x_offset(k4)) = p;
            }
            sum = wave_sum_i32(sum);
            if (lane == 0)
                s_qpart[m * WAVES + wave] = sum;
        }
    }
    if constexpr (regpath && S == WAVES) {
        // One row block per workgroup: thread tid quantized float4 tid + i * T, the 256-k
        // step wave + 8 i, which is exactly the step the wave's MFMAs take as k-split
        // wave; and its sums of q fold into its own partials. Each wave therefore reads
        // back only LDS it wrote itself: its own writes retiring is all it waits for.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else {
        __syncthreads();
    }

    // 5. Stream the wave's weights, two batches in flight, MFMAs on the older one.
    //    Token columns r >= M read token M - 1 (their outputs are never stored); every
    //    chunk read, c < 4 * nsteps <= KC4, lies in the zero-filled row.
    v4i a1[1], a4[1], a16[1];
    a1[0] = a4[0] = a16[0] = v4i{0, 0, 0, 0};
    const int8_t *xrow = xq + min(r, M - 1) * pitch;
    if constexpr (U == 1) {
        // At most two steps (the launcher's batch size): both activation operands are read
        // before the first MFMA.
        v4i b0[4], b1[4];
        if (nmine > 0) {
            const v4i *p = reinterpret_cast<const v4i *>(xrow + (4 * ks + g) * 64);
            b0[0] = p[0], b0[1] = p[1], b0[2] = p[2], b0[3] = p[3];
        }
        if (nmine > 1) {
            const v4i *p = reinterpret_cast<const v4i *>(xrow + (4 * (ks + S) + g) * 64);
            b1[0] = p[0], b1[1] = p[1], b1[2] = p[2], b1[3] = p[3];
        }
        if (nmine > 0)
            mfma_step_t(wa[0], b0, a1[0], a4[0], a16[0]);
        if (nmine > 1)
            mfma_step_t(wb[0], b1, a1[0], a4[0], a16[0]);
    } else {
        auto compute_batch = [&](const v4i (&w)[U], int b) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = b * U + u;
                if (i < nmine) {
                    const int c = 4 * (ks + S * i) + g;
                    const v4i *p = reinterpret_cast<const v4i *>(xrow + c * 64);
                    const v4i b[4] = {p[0], p[1], p[2], p[3]};
                    mfma_step_t(w[u], b, a1[0], a4[0], a16[0]);
                }
            }
        };
        // Batch pairs with unconditional loads, then the last pair (as in k_gemv_direct_db).
        int b = 0;
        for (; b + 2 < nb; b += 2) {
            compute_batch(wa, b);
            load_batch(wa, b + 2);
            compute_batch(wb, b + 1);
            load_batch(wb, b + 3);
        }
        compute_batch(wa, b);
        compute_batch(wb, b + 1);
    }

    // 6. Combine the k-splits of each block (S > 1) and write y / acc. Lane (g, r) holds
    //    rows 4g + v of its block for token r.
    int part[4];
#pragma unroll
    for (int v = 0; v < 4; ++v)
        part[v] = a1[0][v] + (a4[0][v] >> 2) + (a16[0][v] >> 4);
    if constexpr (late_q) {
        int qr = 0;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m < M) {
                const int qw = wave_sum_i32(qlane[m]);
                if constexpr (fold_q) {
                    if (m == r)
                        qr = qw;
                } else if (lane == 0) {
                    s_qpart[m * WAVES + wave] = qw;
                }
            }
        }
        if constexpr (fold_q) {
#pragma unroll
            for (int v = 0; v < 4; ++v)
                part[v] -= qr;
        }
    }
    // The epilogue wave's scale, formed before it waits for the other k-splits (it owns
    // the fewest steps, so it reaches the barrier first).
    float4 scale = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (ks == KE) {
        const float sx = (amax_r == 0.0f) ? 0.0f : amax_r / 127.0f;
        scale = make_float4(gam.x * sx, gam.y * sx, gam.z * sx, gam.w * sx);
    }
    if constexpr (S > 1) {
        if (ks != KE)
            red[wave * 64 + lane] = make_int4(part[0], part[1], part[2], part[3]);
        __syncthreads();
        if (ks == KE)
            add_ksplit_partials<KE>(red + (wave - KE) * 64 + lane, part);
    }
    if (ks == KE && r < M) {
        int qs = 0;
        if constexpr (!fold_q) {
            const int4 u = reinterpret_cast<const int4 *>(s_qpart + r * WAVES)[0];
            const int4 v = reinterpret_cast<const int4 *>(s_qpart + r * WAVES)[1];
            qs = (u.x + u.y) + (u.z + u.w) + (v.x + v.y) + (v.z + v.w);
        }
        const int64_t n0 = (int64_t)b16 * 16 + 4 * g;
        if ((N & 3) == 0 && n0 < N && ((reinterpret_cast<uintptr_t>(Y) | reinterpret_cast<uintptr_t>(ACC)) & 15) == 0) {
            // four consecutive outputs of one row of y (N % 4 == 0 keeps the row 16-byte aligned)
            const int4 acc = make_int4(part[0] - qs, part[1] - qs, part[2] - qs, part[3] - qs);
            if (ACC)
                *reinterpret_cast<int4 *>(ACC + (int64_t)r * N + n0) = acc;
            if (Y)
                *reinterpret_cast<float4 *>(Y + (int64_t)r * N + n0) = make_float4(
                    (float)acc.x * scale.x, (float)acc.y * scale.y, (float)acc.z * scale.z, (float)acc.w * scale.w);
        } else {
            const float sc[4] = {scale.x, scale.y, scale.z, scale.w};
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t n = n0 + v;
                if (n < N) {
                    const int acc = part[v] - qs;
                    if (ACC)
                        ACC[(int64_t)r * N + n] = acc;
                    if (Y)
                        Y[(int64_t)r * N + n] = (float)acc * sc[v];
                }
            }
        }
    }
}

// ------------------------------------------------------------- staged kernel
// Pre-quantized activations for 1 <= M <= 16 tokens whose int8 rows fit the LDS limit
// below (BT_GEMV_AUTO takes it wherever they fit: bt_ternary_gemv, and the unfused route
// of bt_ternary_linear): the fused kernel's streaming design -- eight waves, k-splits
// S, two weight batches in flight, every MFMA B operand one 16-byte LDS read -- with its
// quantizer replaced by a copy of the int8 rows (bt_act_row_bytes(K) bytes each, zero past
// K) into the same transposed chunk layout. The activations then cross the L2 once per
// workgroup instead of once per step and row block (k_gemv_direct). Each thread copies at
// most CH 64-byte chunks (CH = 2 up to 64 KB of staged rows, 4 up to 128 KB): its loads go
// out first, then the weights', so the copy waits for the activations only.
constexpr int kStagedMaxChunks = 4;

template <int MT, int S, int U, bool ROWS, int CH>
__global__ __launch_bounds__(kFusedWaves * 64) void k_gemv_staged(
    const uint4 *__restrict__ Wp, const float *__restrict__ w_scale, const int8_t *__restrict__ Xq,
    float *__restrict__ Y, int32_t *__restrict__ ACC, int M, int N, int K, const float *__restrict__ sx_in,
    const int32_t *__restrict__ xsum_in)
{
    constexpr int WAVES = kFusedWaves;
    constexpr int T = WAVES * 64;
    constexpr int RBW = WAVES / S;
    constexpr int KE = S - 1;  // the k-split that runs the epilogue (it owns the fewest steps)
    const int KC = (K + 63) >> 6;
    const int NB16 = ((N + 63) >> 6) * 4;
    const int KC4 = (KC + 3) & ~3;
    const int ldq = KC4 * 64;  // K rounded up to 256: the Xq row stride
    const int pitch = fused_pitch(KC4, 0);
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    int4 *red = reinterpret_cast<int4 *>(smem);  // [WAVES][64] (S > 1)
    int8_t *xq = reinterpret_cast<int8_t *>(smem + (S > 1 ? WAVES * 64 * 16 : 0));

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int g = lane >> 4;
    const int r = lane & 15;
    const int ks = wave % S;
    const int b16 = blockIdx.x * RBW + wave / S;

    // 1. The activation chunks (token m, 64-k chunk c), at clamped valid addresses.
    const int nchunks = M * KC4;
    v4i cb[CH][4];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int ch = min(tid + i * T, nchunks - 1);
        const int m = ch / KC4, c = ch - m * KC4;
        const v4i *src = reinterpret_cast<const v4i *>(Xq + (int64_t)m * ldq + c * 64);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            cb[i][q] = src[q];
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2. The wave's first two weight batches, then the epilogue's inputs.
    const int nsteps = (KC + 3) >> 2;
    const int nmine = (ks < nsteps) ? (nsteps - 1 - ks) / S + 1 : 0;
    const int nb = (nmine + U - 1) / U;
    v4i wa[U], wb[U];
    auto load_batch = [&](v4i (&w)[U], int b) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            w[u] = load_w_raw(Wp, b16, NB16, 4 * (ks + S * (b * U + u)) + g, KC, r);
    };
    load_batch(wa, 0);  // K >= 1: valid clamped addresses
    load_batch(wb, 1);
    float4 gam;
    if constexpr (ROWS) {
        gam = load_scales4(w_scale, (int64_t)b16 * 16 + 4 * g, N, true);
    } else {
        const float g1 = load_scale_vmem(w_scale);
        gam = make_float4(g1, g1, g1, g1);
    }
    const int rt = min(r, M - 1);  // token of this lane's output column
    const float sx_r = sx_in[rt];
    const int qs_r = xsum_in[rt];

    // 3. Into LDS, transposed within each chunk: bytes 16s .. 16s + 15 take dwords
    //    s, s + 4, s + 8, s + 12 (the B operand of mask s).
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int ch = tid + i * T;
        if (ch < nchunks) {
            const int m = ch / KC4, c = ch - m * KC4;
            v4i *dst = reinterpret_cast<v4i *>(xq + m * pitch + c * 64);
#pragma unroll
            for (int sidx = 0; sidx < 4; ++sidx)
                dst[sidx] = v4i{cb[i][0][sidx], cb[i][1][sidx], cb[i][2][sidx], cb[i][3][sidx]};
        }
    }
    __syncthreads();

    // 4. Stream the wave's weights, two batches in flight, MFMAs on the older one. Token
    //    columns r >= M read token M - 1 (never stored); chunks read lie in the rows.
    v4i a1 = v4i{0, 0, 0, 0}, a4 = a1, a16 = a1;
    const int8_t *xrow = xq + rt * pitch;
    auto compute_batch = [&](const v4i (&w)[U], int b) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = b * U + u;
            if (i < nmine) {
                const v4i *p = reinterpret_cast<const v4i *>(xrow + (4 * (ks + S * i) + g) * 64);
                const v4i bo[4] = {p[0], p[1], p[2], p[3]};
                mfma_step_t(w[u], bo, a1, a4, a16);
            }
        }
    };
    // Batch pairs with unconditional loads, then the last pair (as in k_gemv_direct_db).
    int b = 0;
    for (; b + 2 < nb; b += 2) {
        compute_batch(wa, b);
        load_batch(wa, b + 2);
        compute_batch(wb, b + 1);
        load_batch(wb, b + 3);
    }
    compute_batch(wa, b);
    compute_batch(wb, b + 1);

    // 5. k-split sum (S > 1) and the epilogue; lane (g, r) holds rows 4g + v for token r.
    int part[4];
#pragma unroll
    for (int v = 0; v < 4; ++v)
        part[v] = a1[v] + (a4[v] >> 2) + (a16[v] >> 4);
    if constexpr (S > 1) {
        if (ks != KE)
            red[wave * 64 + lane] = make_int4(part[0], part[1], part[2], part[3]);
        __syncthreads();
        if (ks == KE)
            add_ksplit_partials<KE>(red + (wave - KE) * 64 + lane, part);
    }
    if (ks == KE && r < M) {
        const float sc[4] = {gam.x * sx_r, gam.y * sx_r, gam.z * sx_r, gam.w * sx_r};
        const int64_t n0 = (int64_t)b16 * 16 + 4 * g;
        if ((N & 3) == 0 && n0 < N && ((reinterpret_cast<uintptr_t>(Y) | reinterpret_cast<uintptr_t>(ACC)) & 15) == 0) {
            const int4 acc = make_int4(part[0] - qs_r, part[1] - qs_r, part[2] - qs_r, part[3] - qs_r);
            if (ACC)
                *reinterpret_cast<int4 *>(ACC + (int64_t)r * N + n0) = acc;
            if (Y)
                *reinterpret_cast<float4 *>(Y + (int64_t)r * N + n0) =
                    make_float4((float)acc.x * sc[0], (float)acc.y * sc[1], (float)acc.z * sc[2], (float)acc.w * sc[3]);
        } else {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t n = n0 + v;
                if (n < N) {
                    const int acc = part[v] - qs_r;
                    if (ACC)
                        ACC[(int64_t)r * N + n] = acc;
                    if (Y)
                        Y[(int64_t)r * N + n] = (float)acc * sc[v];
                }
            }
        }
    }
}

// ------------------------------------------------------------ blocked kernel
// k_gemv_staged for int8 rows too long to stage whole (M * K above the staged kernel's LDS
// limit, e.g. 16 tokens x 28672): K is walked in blocks of KB = BPB * S * U steps of 256 k,
// so that every wave owns exactly BPB (1 or 2) weight batches of each block and all waves run
// the same number of blocks (and barriers). Block kb's rows sit in LDS buffer kb % 2, in the staged
// kernel's transposed chunk layout; block kb + 1's chunks are loaded into registers when
// block kb starts (global -> registers, two 64-byte chunks per thread), written into the
// other buffer once block kb's MFMAs are issued, and published by the one barrier per block.
// The weight stream keeps two batches in flight across the block boundaries.
template <int S, int U, int BPB, bool ROWS>
__global__ __launch_bounds__(kFusedWaves * 64) void k_gemv_blocked(
    const uint4 *__restrict__ Wp, const float *__restrict__ w_scale, const int8_t *__restrict__ Xq,
    float *__restrict__ Y, int32_t *__restrict__ ACC, int M, int N, int K, const float *__restrict__ sx_in,
    const int32_t *__restrict__ xsum_in)
{
    constexpr int WAVES = kFusedWaves;
    constexpr int T = WAVES * 64;
    constexpr int RBW = WAVES / S;
    constexpr int KE = S - 1;
    constexpr int KB = BPB * S * U;      // steps per block
    constexpr int KBC = 4 * KB;          // 64-byte chunks per token and block
    constexpr int CH = 2;                // chunks each thread copies per block (M * KBC <= 2 * T)
    constexpr int BPITCH = KBC * 64 + kPitchPad;
    const int KC = (K + 63) >> 6;
    const int NB16 = ((N + 63) >> 6) * 4;
    const int KC4 = (KC + 3) & ~3;
    const int ldq = KC4 * 64;
    const int nsteps = KC4 >> 2;
    const int nblocks = (nsteps + KB - 1) / KB;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    int4 *red = reinterpret_cast<int4 *>(smem);  // [WAVES][64] (S > 1)
    int8_t *xbuf = reinterpret_cast<int8_t *>(smem + (S > 1 ? WAVES * 64 * 16 : 0));  // 2 x [M][BPITCH]
    const int bufbytes = M * BPITCH;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int g = lane >> 4;
    const int r = lane & 15;
    const int ks = wave % S;
    const int b16 = blockIdx.x * RBW + wave / S;
    const int nchunks = M * KBC;

    // Chunk i of this thread in block kb: token m, row chunk c (clamped into the row; slots
    // past the last step are never read).
    v4i cb[CH][4];
    auto load_block = [&](int kb) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int ch = min(tid + i * T, nchunks - 1);
            const int m = ch / KBC, cl = ch - m * KBC;
            const int c = min(kb * KBC + cl, KC4 - 1);
            const v4i *src = reinterpret_cast<const v4i *>(Xq + (int64_t)m * ldq + c * 64);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                cb[i][q] = src[q];
        }
    };
    auto store_block = [&](int kb) {
        int8_t *dstbuf = xbuf + (kb & 1) * bufbytes;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int ch = tid + i * T;
            if (ch < nchunks) {
                const int m = ch / KBC, cl = ch - m * KBC;
                v4i *dst = reinterpret_cast<v4i *>(dstbuf + m * BPITCH + cl * 64);
#pragma unroll
                for (int sidx = 0; sidx < 4; ++sidx)
                    dst[sidx] = v4i{cb[i][0][sidx], cb[i][1][sidx], cb[i][2][sidx], cb[i][3][sidx]};
            }
        }
    };

    // 1. Block 0's chunks, then the wave's first two weight batches (block 0's), then the
    //    epilogue's inputs.
    load_block(0);
    __builtin_amdgcn_sched_barrier(0);
    const int nmine = (ks < nsteps) ? (nsteps - 1 - ks) / S + 1 : 0;
    const int nb = (nmine + U - 1) / U;
    v4i wa[U], wb[U];
    auto load_batch = [&](v4i (&w)[U], int b) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            w[u] = load_w_raw(Wp, b16, NB16, 4 * (ks + S * (b * U + u)) + g, KC, r);
    };
    load_batch(wa, 0);  // K >= 1: valid clamped addresses
    load_batch(wb, 1);
    float4 gam;
    if constexpr (ROWS) {
        gam = load_scales4(w_scale, (int64_t)b16 * 16 + 4 * g, N, true);
    } else {
        const float g1 = load_scale_vmem(w_scale);
        gam = make_float4(g1, g1, g1, g1);
    }
    const int rt = min(r, M - 1);
    const float sx_r = sx_in[rt];
    const int qs_r = xsum_in[rt];
    store_block(0);
    __syncthreads();

    // 2. Block by block: the next block's chunks go out first, then block kb's BPB batches
    //    (MFMAs on LDS buffer kb % 2, the batch two ahead loaded behind each), then the next
    //    block into the other buffer and the block's barrier.
    v4i a1 = v4i{0, 0, 0, 0}, a4 = a1, a16 = a1;
    auto compute_batch = [&](const v4i (&w)[U], int b, const int8_t *xrow) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = b * U + u;
            if (i < nmine) {
                // step ks + S i is step ks + S (i - kb * BPB * U) of block kb = b / BPB
                const int cl = 4 * (ks + S * (i - (b / BPB) * BPB * U)) + g;
                const v4i *p = reinterpret_cast<const v4i *>(xrow + cl * 64);
                const v4i bo[4] = {p[0], p[1], p[2], p[3]};
                mfma_step_t(w[u], bo, a1, a4, a16);
            }
        }
    };
    auto next_block = [&](int kb) {
        if (kb + 1 < nblocks) {  // uniform
            store_block(kb + 1);
            __syncthreads();
        }
    };
    // Every load below is unconditional, at clamped valid addresses (past the last block or
    // batch they re-read the row's last chunk, which stays cached): a load under a branch
    // would leave the compiler unable to count the loads issued after a batch, and every
    // wait for that batch would then wait for the next block's activations as well.
    if constexpr (BPB == 2) {
        for (int kb = 0; kb < nblocks; ++kb) {
            load_block(kb + 1);
            const int8_t *xrow = xbuf + (kb & 1) * bufbytes + rt * BPITCH;
            const int b = 2 * kb;
            compute_batch(wa, b, xrow);
            load_batch(wa, b + 2);
            compute_batch(wb, b + 1, xrow);
            load_batch(wb, b + 3);
            next_block(kb);
        }
    } else {
        // one batch per block: blocks alternate between the two register batches
        auto one_block = [&](v4i (&w)[U], int kb) {
            load_block(kb + 1);
            compute_batch(w, kb, xbuf + (kb & 1) * bufbytes + rt * BPITCH);
            load_batch(w, kb + 2);
            next_block(kb);
        };
        for (int kb = 0; kb < nblocks; kb += 2) {
            one_block(wa, kb);
            if (kb + 1 < nblocks)
                one_block(wb, kb + 1);
        }
    }

    // 3. k-split sum (S > 1) and the epilogue, as in k_gemv_staged.
    int part[4];
#pragma unroll
    for (int v = 0; v < 4; ++v)
        part[v] = a1[v] + (a4[v] >> 2) + (a16[v] >> 4);
    if constexpr (S > 1) {
        if (ks != KE)
            red[wave * 64 + lane] = make_int4(part[0], part[1], part[2], part[3]);
        __syncthreads();
        if (ks == KE)
            add_ksplit_partials<KE>(red + (wave - KE) * 64 + lane, part);
    }
    if (ks == KE && r < M) {
        const float sc[4] = {gam.x * sx_r, gam.y * sx_r, gam.z * sx_r, gam.w * sx_r};
        const int64_t n0 = (int64_t)b16 * 16 + 4 * g;
        if ((N & 3) == 0 && n0 < N && ((reinterpret_cast<uintptr_t>(Y) | reinterpret_cast<uintptr_t>(ACC)) & 15) == 0) {
            const int4 acc = make_int4(part[0] - qs_r, part[1] - qs_r, part[2] - qs_r, part[3] - qs_r);
            if (ACC)
                *reinterpret_cast<int4 *>(ACC + (int64_t)r * N + n0) = acc;
            if (Y)
                *reinterpret_cast<float4 *>(Y + (int64_t)r * N + n0) =
                    make_float4((float)acc.x * sc[0], (float)acc.y * sc[1], (float)acc.z * sc[2], (float)acc.w * sc[3]);
        } else {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t n = n0 + v;
                if (n < N) {
                    const int acc = part[v] - qs_r;
                    if (ACC)
                        ACC[(int64_t)r * N + n] = acc;
                    if (Y)
                        Y[(int64_t)r * N + n] = (float)acc * sc[v];
                }
            }
        }
    }
}

int pick_rb(int64_t N)
{
    const int64_t nb16 = (N + 15) / 16;
    if (nb16 / 4 >= 256)
        return 4;
    if (nb16 / 2 >= 256)
        return 2;
    return 1;
}

// Token capacity of the fused kernel (it takes M <= 4: past that one quantizer launch
// and a pre-quantized GEMV are faster).
int pick_mt(int64_t M) { return M <= 1 ? 1 : M <= 2 ? 2 : 4; }

// k-splits per 16-row block: enough waves to give every SIMD one (1024 waves), two for
// matrices of at most 512 row blocks (8192 rows): their rows are few, so each wave's share
// of a long row is what keeps enough bytes in flight. Measured on the 2B, 7B and 100B
// decode shapes at M = 1 (100B down 24.3 -> 17.3 us, 100B O 9.0 -> 7.0 us, 7B O and down
// 10-15% faster, the rest unchanged).
int pick_s(int64_t N)
{
    const int64_t nb16 = (N + 15) / 16;
    const int64_t target = nb16 <= 512 ? 2048 : 1024;
    int s = 1;
    while (s < 8 && nb16 * s < target)
        s *= 2;
    return s;
}

// Batch size: the steps of 256 k a wave owns (at most ceil(steps / S)) over two batches.
int pick_u(int64_t K, int s)
{
    const int64_t mine = ((K + 255) / 256 + s - 1) / s;
    return mine <= 2 ? 1 : mine <= 4 ? 2 : mine <= 6 ? 3 : 4;
}

size_t fused_lds(int64_t M, int64_t K, int s, int rx)
{
    const int64_t KC = (K + 63) / 64;
    const int KC4 = (int)((KC + 3) / 4 * 4);
    return 2 * kFusedWaves * kMaxM * 4 + (s > 1 ? kFusedWaves * 256 * 4 : 0) + (size_t)M * fused_pitch(KC4, rx);
}

// The register path's float4 per thread and token (0: streaming path): for rows that are
// 16-byte aligned with K % 4 == 0 and whose share per thread fits kXRegs float4 over all
// the kernel's tokens, the smallest power of two RX with RX * 512 >= K / 4. It also sets
// the LDS row pitch.
int fused_rx(int64_t M, int64_t K, bool aligned16)
{
    const int64_t K4 = K / 4, T = kFusedWaves * 64;
    if (K <= 0 || (K & 3) != 0 || !aligned16)
        return 0;
    int rx = 1;
    while ((int64_t)rx * T < K4)
        rx *= 2;
    return rx * pick_mt(M) > kXRegs ? 0 : rx;
}

// Template arguments of the fused kernel for one call (k_linear_decode<MT, S, RX, U>).
struct FusedPick {
    int mt, s, rx, u;
};

FusedPick pick_fused(int64_t M, int64_t N, int64_t K, bool aligned16)
{
    const int s = pick_s(N);
    return {pick_mt(M), s, fused_rx(M, K, aligned16), pick_u(K, s)};
}

template <int MT, int S, int RX, int U>
hipError_t launch_fused_u(const uint4 *Wp, const float *w_scale, bool row_scales, const float *X, int64_t M, int64_t N,
                          int64_t K, float *Y, int32_t *acc, hipStream_t s)
{
    constexpr int RBW = kFusedWaves / S;
    const int64_t nb16 = (N + 15) / 16;
    const dim3 grid((unsigned)((nb16 + RBW - 1) / RBW)), block(kFusedWaves * 64);
    if (row_scales)
        hipLaunchKernelGGL((k_linear_decode<MT, S, RX, U, true>), grid, block, fused_lds(M, K, S, RX), s, Wp, w_scale,
                           X, Y, acc, (int)M, (int)N, (int)K);
    else
        hipLaunchKernelGGL((k_linear_decode<MT, S, RX, U, false>), grid, block, fused_lds(M, K, S, RX), s, Wp, w_scale,
                           X, Y, acc, (int)M, (int)N, (int)K);
    return hipGetLastError();
}

template <int MT, int S, int RX>
hipError_t launch_fused_rx(const FusedPick &p, const uint4 *Wp, const float *w_scale, bool row_scales, const float *X,
                           int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc, hipStream_t s)
{
    switch (p.u) {
    case 1: return launch_fused_u<MT, S, RX, 1>(Wp, w_scale, row_scales, X, M, N, K, Y, acc, s);
    case 2: return launch_fused_u<MT, S, RX, 2>(Wp, w_scale, row_scales, X, M, N, K, Y, acc, s);
    case 3: return launch_fused_u<MT, S, RX, 3>(Wp, w_scale, row_scales, X, M, N, K, Y, acc, s);
    default: return launch_fused_u<MT, S, RX, 4>(Wp, w_scale, row_scales, X, M, N, K, Y, acc, s);
    }
}

// RX * MT <= kXRegs holds for every pick (fused_rx), so the clamps below only keep
// combinations that are never launched from being instantiated.
template <int MT, int S>
hipError_t launch_fused_t(const FusedPick &p, const uint4 *Wp, const float *w_scale, bool row_scales, const float *X,
                          int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc, hipStream_t s)
{
    switch (p.rx) {
    case 0: return launch_fused_rx<MT, S, 0>(p, Wp, w_scale, row_scales, X, M, N, K, Y, acc, s);
    case 1: return launch_fused_rx<MT, S, 1>(p, Wp, w_scale, row_scales, X, M, N, K, Y, acc, s);
    case 2: return launch_fused_rx<MT, S, (MT <= 8 ? 2 : 1)>(p, Wp, w_scale, row_scales, X, M, N, K, Y, acc, s);
    case 4: return launch_fused_rx<MT, S, (MT <= 4 ? 4 : 1)>(p, Wp, w_scale, row_scales, X, M, N, K, Y, acc, s);
    case 8: return launch_fused_rx<MT, S, (MT <= 2 ? 8 : 1)>(p, Wp, w_scale, row_scales, X, M, N, K, Y, acc, s);
    default: return launch_fused_rx<MT, S, (MT <= 1 ? 16 : 1)>(p, Wp, w_scale, row_scales, X, M, N, K, Y, acc, s);
    }
}

template <int MT>
hipError_t launch_fused_mt(const FusedPick &p, const uint4 *Wp, const float *w_scale, bool row_scales, const float *X,
                           int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc, hipStream_t s)
{
    switch (p.s) {
    case 1: return launch_fused_t<MT, 1>(p, Wp, w_scale, row_scales, X, M, N, K, Y, acc, s);
    case 2: return launch_fused_t<MT, 2>(p, Wp, w_scale, row_scales, X, M, N, K, Y, acc, s);
    case 4: return launch_fused_t<MT, 4>(p, Wp, w_scale, row_scales, X, M, N, K, Y, acc, s);
    default: return launch_fused_t<MT, 8>(p, Wp, w_scale, row_scales, X, M, N, K, Y, acc, s);
    }
}

size_t staged_lds(int64_t M, int64_t K, int s)
{
    const int KC4 = (int)(((K + 63) / 64 + 3) / 4 * 4);
    return (s > 1 ? kFusedWaves * 64 * 16 : 0) + (size_t)M * fused_pitch(KC4, 0);
}

// Template arguments of the staged kernel for one call (k_gemv_staged<MT, S, U, CH>): token
// capacity 8 or 16, the fused kernel's k-splits and batch size, and the staged rows' 64-byte
// chunks over the workgroup's threads (CH = 2 up to 64 KB, 4 up to 128 KB).
struct StagedPick {
    int mt, s, u, ch;
};

StagedPick pick_staged(int64_t M, int64_t N, int64_t K)
{
    const int s = pick_s(N);
    const int64_t nchunks = M * (((K + 63) / 64 + 3) / 4 * 4);
    return {M <= 8 ? 8 : 16, s, pick_u(K, s), nchunks <= 2 * kFusedWaves * 64 ? 2 : 4};
}

template <int MT, int S, int U, int CH>
hipError_t launch_staged_ch(const uint4 *Wp, const float *w_scale, bool row_scales, const int8_t *Xq, const float *sx,
                            const int32_t *xsum, int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc, hipStream_t s)
{
    constexpr int RBW = kFusedWaves / S;
    const int64_t nb16 = (N + 15) / 16;
    const dim3 grid((unsigned)((nb16 + RBW - 1) / RBW)), block(kFusedWaves * 64);
    if (row_scales)
        hipLaunchKernelGGL((k_gemv_staged<MT, S, U, true, CH>), grid, block, staged_lds(M, K, S), s, Wp, w_scale, Xq,
                           Y, acc, (int)M, (int)N, (int)K, sx, xsum);
    else
        hipLaunchKernelGGL((k_gemv_staged<MT, S, U, false, CH>), grid, block, staged_lds(M, K, S), s, Wp, w_scale, Xq,
                           Y, acc, (int)M, (int)N, (int)K, sx, xsum);
    return hipGetLastError();
}

template <int MT, int S, int U>
hipError_t launch_staged_u(const StagedPick &p, const uint4 *Wp, const float *w_scale, bool row_scales,
                           const int8_t *Xq, const float *sx, const int32_t *xsum, int64_t M, int64_t N, int64_t K,
                           float *Y, int32_t *acc, hipStream_t s)
{
    if (p.ch == 2)
        return launch_staged_ch<MT, S, U, 2>(Wp, w_scale, row_scales, Xq, sx, xsum, M, N, K, Y, acc, s);
    return launch_staged_ch<MT, S, U, 4>(Wp, w_scale, row_scales, Xq, sx, xsum, M, N, K, Y, acc, s);
}

template <int MT, int S>
hipError_t launch_staged_s(const StagedPick &p, const uint4 *Wp, const float *w_scale, bool row_scales,
                           const int8_t *Xq, const float *sx, const int32_t *xsum, int64_t M, int64_t N, int64_t K,
                           float *Y, int32_t *acc, hipStream_t s)
{
    switch (p.u) {
    case 1: return launch_staged_u<MT, S, 1>(p, Wp, w_scale, row_scales, Xq, sx, xsum, M, N, K, Y, acc, s);
    case 2: return launch_staged_u<MT, S, 2>(p, Wp, w_scale, row_scales, Xq, sx, xsum, M, N, K, Y, acc, s);
    case 3: return launch_staged_u<MT, S, 3>(p, Wp, w_scale, row_scales, Xq, sx, xsum, M, N, K, Y, acc, s);
    default: return launch_staged_u<MT, S, 4>(p, Wp, w_scale, row_scales, Xq, sx, xsum, M, N, K, Y, acc, s);
    }
}

template <int MT>
hipError_t launch_staged_mt(const StagedPick &p, const uint4 *Wp, const float *w_scale, bool row_scales,
                            const int8_t *Xq, const float *sx, const int32_t *xsum, int64_t M, int64_t N, int64_t K,
                            float *Y, int32_t *acc, hipStream_t s)
{
    switch (p.s) {
    case 1: return launch_staged_s<MT, 1>(p, Wp, w_scale, row_scales, Xq, sx, xsum, M, N, K, Y, acc, s);
    case 2: return launch_staged_s<MT, 2>(p, Wp, w_scale, row_scales, Xq, sx, xsum, M, N, K, Y, acc, s);
    case 4: return launch_staged_s<MT, 4>(p, Wp, w_scale, row_scales, Xq, sx, xsum, M, N, K, Y, acc, s);
    default: return launch_staged_s<MT, 8>(p, Wp, w_scale, row_scales, Xq, sx, xsum, M, N, K, Y, acc, s);
    }
}

// Template arguments of the blocked kernel (k_gemv_blocked<S, U, BPB>): the staged kernel's
// k-splits, then the largest batch U <= 4 and batches per block BPB <= 2 whose block
// (BPB S U steps of M rows, M taken as 8 or 16) each thread stages in two 64-byte chunks
// (M * 4 * BPB * S * U <= 1024 chunks); the two LDS buffers then hold at most 128 KB of rows.
// A large U keeps the weight bytes in flight; the second batch per block halves the barriers.
struct BlockedPick {
    int s, u, bpb;
};

BlockedPick pick_blocked(int64_t M, int64_t N)
{
    const int s = pick_s(N);
    const int64_t mcap = M <= 8 ? 8 : 16;
    const int64_t chunks = 2 * kFusedWaves * 64;
    int u = 4;
    while (u > 1 && mcap * 4 * s * u > chunks)
        --u;
    return {s, u, mcap * 4 * 2 * s * u <= chunks ? 2 : 1};
}

size_t blocked_lds(int64_t M, int s, int u, int bpb)
{
    return (s > 1 ? kFusedWaves * 64 * 16 : 0) + 2 * (size_t)M * (size_t)(4 * bpb * s * u * 64 + kPitchPad);
}

template <int S, int U, int BPB>
hipError_t launch_blocked_su(const uint4 *Wp, const float *w_scale, bool row_scales, const int8_t *Xq,
                             const float *sx, const int32_t *xsum, int64_t M, int64_t N, int64_t K, float *Y,
                             int32_t *acc, hipStream_t s)
{
    constexpr int RBW = kFusedWaves / S;
    const int64_t nb16 = (N + 15) / 16;
    const dim3 grid((unsigned)((nb16 + RBW - 1) / RBW)), block(kFusedWaves * 64);
    const size_t lds = blocked_lds(M, S, U, BPB);
    if (row_scales)
        hipLaunchKernelGGL((k_gemv_blocked<S, U, BPB, true>), grid, block, lds, s, Wp, w_scale, Xq, Y, acc, (int)M,
                           (int)N, (int)K, sx, xsum);
    else
        hipLaunchKernelGGL((k_gemv_blocked<S, U, BPB, false>), grid, block, lds, s, Wp, w_scale, Xq, Y, acc, (int)M,
                           (int)N, (int)K, sx, xsum);
    return hipGetLastError();
}

// The direct kernel for one call: RB row blocks per workgroup, and for one row block the
// double-buffered form with batches of U steps. One row block: two-step batches, two in
// flight once a wave owns more than two steps. More row blocks: the single-batch kernel
// (measured faster there: more waves resident).
struct DirectPick {
    int rb, u;  // u == 0: k_gemv_direct<RB>; else k_gemv_direct_db<RB, u>
};

DirectPick pick_direct(int64_t N, int64_t K)
{
    const int rb = pick_rb(N);
    const int64_t mine = ((K + 255) / 256 + kDirectWaves - 1) / kDirectWaves;
    return {rb, rb > 1 ? 0 : mine <= 2 ? 1 : 2};
}

template <int RB>
hipError_t launch_direct_t(const DirectPick &p, const uint4 *Wp, const float *w_scale, bool row_scales,
                           const int8_t *Xq, int64_t ldq, const float *sx, const int32_t *xsum, int64_t M, int64_t N,
                           int64_t K, float *Y, int32_t *acc, hipStream_t s)
{
    const int KC = (int)((K + 63) / 64);
    const int NB16 = (int)(((N + 63) / 64) * 4);
    const int64_t nb16 = (N + 15) / 16;
    const dim3 grid((unsigned)((nb16 + RB - 1) / RB)), block(kDirectWaves * 64);
    if (p.u == 0)
        hipLaunchKernelGGL((k_gemv_direct<RB>), grid, block, 0, s, Wp, w_scale, Xq, ldq, sx, xsum, (int)M, N, KC, NB16, Y,
                           acc, (int)row_scales);
    else if (p.u == 1)
        hipLaunchKernelGGL((k_gemv_direct_db<RB, 1>), grid, block, 0, s, Wp, w_scale, Xq, ldq, sx, xsum, (int)M,
                           N, KC, NB16, Y, acc, (int)row_scales);
    else
        hipLaunchKernelGGL((k_gemv_direct_db<RB, 2>), grid, block, 0, s, Wp, w_scale, Xq, ldq, sx, xsum, (int)M,
                           N, KC, NB16, Y, acc, (int)row_scales);
    return hipGetLastError();
}

}  // namespace

// An upper bound for any activation alignment: the register path's pitch is the larger.
size_t decode_fused_lds_bytes(int64_t M, int64_t N, int64_t K)
{
    return fused_lds(M, K, pick_s(N), fused_rx(M, K, true));
}

// The staged kernel takes up to 16 tokens whose int8 rows fit kStagedLdsLimit bytes of LDS
// (each thread then copies at most kStagedMaxChunks chunks; with the k-split area and the
// row padding a workgroup stays within the 160 KB of one CU).
constexpr size_t kStagedLdsLimit = (size_t)kStagedMaxChunks * kFusedWaves * 64 * 64;

bool gemv_staged_fits(int64_t M, int64_t N, int64_t K)
{
    const int64_t KC4 = ((K + 63) / 64 + 3) / 4 * 4;
    return M >= 1 && M <= 16 && K >= 1 && M * KC4 * 64 <= (int64_t)kStagedLdsLimit;
}

hipError_t launch_gemv_staged(const uint4 *Wp, const float *w_scale, bool row_scales, const int8_t *Xq,
                              const float *sx, const int32_t *xsum, int64_t M, int64_t N, int64_t K, float *Y,
                              int32_t *acc, hipStream_t s)
{
    if (M < 1 || M > 16 || K < 1)
        return hipErrorInvalidValue;
    if (!gemv_staged_fits(M, N, K)) {
        // rows too long to stage whole: the blocked form (the picks below are all it takes)
        const BlockedPick b = pick_blocked(M, N);
        switch (b.s * 100 + b.u * 10 + b.bpb) {
        case 142: return launch_blocked_su<1, 4, 2>(Wp, w_scale, row_scales, Xq, sx, xsum, M, N, K, Y, acc, s);
        case 242: return launch_blocked_su<2, 4, 2>(Wp, w_scale, row_scales, Xq, sx, xsum, M, N, K, Y, acc, s);
        case 442: return launch_blocked_su<4, 4, 2>(Wp, w_scale, row_scales, Xq, sx, xsum, M, N, K, Y, acc, s);
        case 441: return launch_blocked_su<4, 4, 1>(Wp, w_scale, row_scales, Xq, sx, xsum, M, N, K, Y, acc, s);
        case 841: return launch_blocked_su<8, 4, 1>(Wp, w_scale, row_scales, Xq, sx, xsum, M, N, K, Y, acc, s);
        case 821: return launch_blocked_su<8, 2, 1>(Wp, w_scale, row_scales, Xq, sx, xsum, M, N, K, Y, acc, s);
        default: return hipErrorInvalidValue;
        }
    }
    const StagedPick p = pick_staged(M, N, K);
    if (p.mt == 8)
        return launch_staged_mt<8>(p, Wp, w_scale, row_scales, Xq, sx, xsum, M, N, K, Y, acc, s);
    return launch_staged_mt<16>(p, Wp, w_scale, row_scales, Xq, sx, xsum, M, N, K, Y, acc, s);
}

hipError_t launch_gemv_mfma(const uint4 *Wp, const float *w_scale, bool row_scales, const int8_t *Xq, int64_t ldq,
                            const float *sx, const int32_t *xsum, int64_t M, int64_t N, int64_t K, float *Y,
                            int32_t *acc, hipStream_t s)
{
    const DirectPick p = pick_direct(N, K);
    switch (p.rb) {
    case 4: return launch_direct_t<4>(p, Wp, w_scale, row_scales, Xq, ldq, sx, xsum, M, N, K, Y, acc, s);
    case 2: return launch_direct_t<2>(p, Wp, w_scale, row_scales, Xq, ldq, sx, xsum, M, N, K, Y, acc, s);
    default: return launch_direct_t<1>(p, Wp, w_scale, row_scales, Xq, ldq, sx, xsum, M, N, K, Y, acc, s);
    }
}

hipError_t launch_linear_decode(const uint4 *Wp, const float *w_scale, bool row_scales, const float *X, int64_t M, int64_t N,
                                int64_t K, float *Y, int32_t *acc, hipStream_t s)
{
    if (M > 4)
        return hipErrorInvalidValue;
    const FusedPick p = pick_fused(M, N, K, (reinterpret_cast<uintptr_t>(X) & 15) == 0);
    switch (p.mt) {
    case 1: return launch_fused_mt<1>(p, Wp, w_scale, row_scales, X, M, N, K, Y, acc, s);
    case 2: return launch_fused_mt<2>(p, Wp, w_scale, row_scales, X, M, N, K, Y, acc, s);
    default: return launch_fused_mt<4>(p, Wp, w_scale, row_scales, X, M, N, K, Y, acc, s);
    }
}

// Names of the kernel instances the launchers above pick (host-only; for bt_kernel_plan).
int plan_linear_decode(int64_t M, int64_t N, int64_t K, bool row_scales, char *buf, size_t len)
{
    const FusedPick p = pick_fused(M, N, K, true);
    return snprintf(buf, len, "k_linear_decode<MT=%d,S=%d,RX=%d,U=%d,ROWS=%d>", p.mt, p.s, p.rx, p.u,
                    (int)row_scales);
}

int plan_gemv_staged(int64_t M, int64_t N, int64_t K, bool row_scales, char *buf, size_t len)
{
    if (!gemv_staged_fits(M, N, K)) {
        const BlockedPick b = pick_blocked(M, N);
        return snprintf(buf, len, "k_gemv_blocked<S=%d,U=%d,BPB=%d,ROWS=%d>", b.s, b.u, b.bpb, (int)row_scales);
    }
    const StagedPick p = pick_staged(M, N, K);
    return snprintf(buf, len, "k_gemv_staged<MT=%d,S=%d,U=%d,ROWS=%d,CH=%d>", p.mt, p.s, p.u, (int)row_scales, p.ch);
}

int plan_gemv_mfma(int64_t M, int64_t N, int64_t K, bool row_scales, char *buf, size_t len)
{
    (void)M;
    const DirectPick p = pick_direct(N, K);
    if (p.u == 0)
        return snprintf(buf, len, "k_gemv_direct<RB=%d>(rows=%d)", p.rb, (int)row_scales);
    return snprintf(buf, len, "k_gemv_direct_db<RB=%d,U=%d>(rows=%d)", p.rb, p.u, (int)row_scales);
}

}  // namespace bt
