// Prefill GEMM on int8 MFMA: acc[m,n] = sum_k t[n,k] q[m,k], any M, with the scale
// epilogue fused. BitNet GPU guide, "Key Components and Source Code Architecture":
// prefill is the compute-bound phase; "BitCompute" page, "Future Roadmap": move the
// add/subtract loops of the ternary product onto the matrix cores.
//
// Tiling (gfx950, wave64, v_mfma_i32_16x16x64_i8, 160 KB LDS per CU):
//  * a workgroup of WM x WN waves computes a BM (tokens) x BN (weight rows) block; each
//    wave owns a 64 x 64 tile of 4 x 4 MFMA tiles, so every activation operand read
//    from LDS feeds 4 MFMAs and every unpacked weight operand feeds 4.
//  * k advances 128 per step, in two MFMA substeps j = 0, 1 of 64 k. At substep j, lane
//    (g, r) with g = lane / 16, r = lane % 16 holds row r's 16 bytes of the 16-k piece
//    p = 2 g + j of the step (k = step * 128 + 16 p .. + 15) of both operands: the
//    activations as int8, the weights as packed word p % 4 of chunk p / 4 (the lane's
//    two words of a step are adjacent: one 8-byte LDS read), unpacked with shifts and one
//    mask into (word >> 2s) & 0x03030303 (byte e of dword s is the code of
//    k = 16 (p % 4) + 4 s + e within the chunk).
//  * both operand tiles of a step travel HBM/L2 -> LDS by direct loads
//    (global_load_lds_dwordx4: each lane's 16 bytes land at LDS offset 16 * lane of a
//    1 KB block), through a ring of NS stages, with no register staging and no LDS
//    store instructions. Each lane quad of a load reads one 64-byte segment (adjacent
//    lanes, adjacent addresses): scattering a quad over rows measured 10% slower.
//  * LDS layouts (in the 4-byte bank model every 16-lane group of an operand read covers all
//    64 banks; the hardware still counts ~1.45 conflict cycles per LDS read, as it does for
//    any 16-lane read spread over 16 rows):
//      activations: per 16-row tile, two 1 KB halves of 8 rows x 128 bytes; row rho of
//                   half h keeps piece p in 16-byte slot p ^ rho ^ h;
//      weights:     the packed layout itself, [64-row block][64-k chunk][row][16 bytes].
//  * software pipeline: a lane's substep-1 operands are read while its substep-0 MFMAs
//    run; one barrier per step, between the two substeps, publishes the next step's
//    stage and frees the current one for the load NS steps ahead; the next step's
//    substep-0 operands are then read while this step's substep-1 MFMAs run.
//  * output: lane holds D[4g + v][r] of each tile = token 16a + 4g + v, weight row
//    16i + r; the wave transposes its tile through LDS 16 tokens at a time and stores
//    y = (acc - sum_k q) * (gamma_n * s_x) row-contiguously, 16 bytes per lane, with
//    non-temporal stores (gamma_n: the matrix's gamma, or weight row n's scale with row
//    scales; the workgroup's BN scales wait in LDS with the row statistics).
//  * workgroup -> tile map is XCD-aware: consecutive workgroup ids land on different
//    XCDs, so each XCD is given a contiguous run of a grouped tile order (8 token-tile
//    rows walked weight-tile column by column): the workgroups resident on an XCD then
//    share 8 activation panels and a few weight panels in its L2, instead of streaming a
//    different weight panel each from HBM.
//  * products with too few tiles to fill the CUs (a few hundred tokens) take a second
//    kernel, k_gemm_ks: 64 x 64 tiles whose k-steps four waves of a workgroup share, with
//    the partial tiles summed in LDS (see its comment below).
#include <algorithm>
#include <type_traits>

#include "bt_internal.h"

namespace bt {
namespace {

constexpr int kXcds = 8;
// Token-tile rows per group of the tile order: with two 4-wave workgroups per CU, an
// XCD's 32 CUs hold 64 workgroups, an 8 x 8 block of tiles.
#ifndef BT_GEMM_GROUP
#define BT_GEMM_GROUP 8
#endif
constexpr int kGroup = BT_GEMM_GROUP;
// Fewest 128-k steps a share of a tail-split tile keeps.
constexpr int64_t kMinTailSteps = 12;

typedef __attribute__((address_space(3))) void lds_void;
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const void global_void;

__device__ inline v4i unpack_word(uint32_t w)
{
    return v4i{(int)(w & kMask0), (int)((w >> 2) & kMask0), (int)((w >> 4) & kMask0), (int)((w >> 6) & kMask0)};
}

// s_waitcnt immediate that waits until at most `vm` vector-memory operations of this
// wave are outstanding (expcnt and lgkmcnt left at their maxima: no wait on them).
constexpr int vmcnt_imm(int vm) { return (vm & 0xF) | ((vm >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

constexpr int kBK = 128;  // k per step
template <int BM, int BN, int WM, int WN, int NS>
struct GemmCfg {
    static constexpr int kWaves = WM * WN;
    static constexpr int kThreads = kWaves * 64;
    static constexpr int TM = BM / WM / 16, TN = BN / WN / 16;
    static constexpr int kABytes = BM * kBK;          // activation tile per stage
    static constexpr int kBBytes = BN * kBK / 4;      // packed weight tile per stage
    static constexpr int kStage = kABytes + kBBytes;
    static constexpr int kABlocks = kABytes / 1024;   // 1 KB direct-load blocks
    static constexpr int kBBlocks = kBBytes / 1024;
    static constexpr int kAPerWave = kABlocks / kWaves;  // activation blocks per wave per step
    static constexpr int kBPerWave = kBBlocks / kWaves;  // weight blocks per wave per step
    static constexpr int kBlocksPerWave = kAPerWave + kBPerWave;
    static_assert(BM / WM == 64 && BN / WN == 64, "wave tile is 64 x 64");
    static_assert(kABlocks % kWaves == 0 && kBBlocks % kWaves == 0, "direct-load blocks split evenly over waves");
    static_assert(NS >= 2 && NS <= 4, "ring of two to four stages");
    static_assert((kWaves / 2) * 16 * 68 * 4 <= kStage, "epilogue slabs fit in two stages");
};

// Split-K partial tile: the int32 accumulators of a BM x BN block.
template <int BM, int BN>
constexpr int kPartialBytes = BM * BN * 4;
// Buffer-resource word 3 for raw (untyped) dword access on gfx9, and the cache-policy
// operand of the buffer load / store builtins that selects sc1 (device coherence).
constexpr int kBufferWord3 = 0x00020000;
constexpr int kSc1 = 1 << 4;

template <int BM, int BN, int WM, int WN, int NS, int WPE, bool SPLITK>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void k_gemm(
    const uint4 *__restrict__ Wp, const float *__restrict__ w_scale, const int8_t *__restrict__ Xq, int64_t ldq,
    const float *__restrict__ sx, const int32_t *__restrict__ xsum, int64_t M, int64_t N, int KC, int NBLK,
    int tiles_m, int tiles_n, int group, float *__restrict__ Y, int32_t *__restrict__ ACC, int flags,
    char *__restrict__ partials, unsigned *__restrict__ arrivals, int full, int nsplit, int full_x, int split_x)
{
    // flags bit 0: 16-byte output stores; bit 1: w_scale holds one scale per output row.
    const int vec = flags & 1;
    const bool rows = (flags & 2) != 0;
    using C = GemmCfg<BM, BN, WM, WN, NS>;
    constexpr int TM = C::TM, TN = C::TN;
    // One LDS array per ring stage ([A tile | B tile] each): distinct objects let the
    // compiler see that a direct load into one stage cannot alias reads of another, so
    // it adds no wait of its own between them (the stage index is a compile-time
    // constant in every unrolled step below).
    __shared__ __attribute__((aligned(1024))) int8_t lds0[C::kStage];
    __shared__ __attribute__((aligned(1024))) int8_t lds1[C::kStage];
    __shared__ __attribute__((aligned(1024))) int8_t lds2[NS > 2 ? C::kStage : 16];
    __shared__ __attribute__((aligned(1024))) int8_t lds3[NS > 3 ? C::kStage : 16];
    auto stage_mem = [&](auto sc) -> int8_t * {
        constexpr int S = decltype(sc)::value;
        if constexpr (S == 0)
            return lds0;
        else if constexpr (S == 1)
            return lds1;
        else if constexpr (S == 2)
            return lds2;
        else
            return lds3;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int wm = wave % WM, wn = wave / WM;
    const int g = lane >> 4, r = lane & 15;

    // Work order. The first `full` tiles of the tile list are computed whole; each later
    // tile is split over `nsplit` workgroups, each taking a contiguous share of its k-steps
    // (SPLITK only). Workgroup b runs on XCD b % 8 and is the (b / 8)-th of that XCD: every
    // XCD takes a contiguous run of full_x whole tiles, then of split_x split tiles with
    // their nsplit shares side by side (the shares of a tile meet in one XCD's L2). Tiles
    // follow a grouped list: groups of `group` token-tile rows, walked weight-tile column
    // by column, so the workgroups resident on one XCD at a time cover a compact block of
    // tiles whose activation and weight panels are shared in that XCD's L2.
    const int total = tiles_m * tiles_n;
    const int b = blockIdx.x;
    const int xcd = b % kXcds, j = b / kXcds;
    int t, split = 0, nsp = 1;
    if (j < full_x) {
        t = xcd * full_x + j;
        if (t >= full)
            return;
    } else {
        if constexpr (!SPLITK)
            return;
        const int p = j - full_x;
        const int ts = xcd * split_x + p / nsplit;  // index among the split tiles
        if (ts >= total - full)
            return;
        t = full + ts;
        split = p % nsplit;
        nsp = nsplit;
    }
    // This share's 128-k steps: [step0, step0 + nsteps) of the tile's ceil(KC / 2).
    const int nsteps_all = (KC + 1) / 2;
    const int per_split = (nsteps_all + nsp - 1) / nsp;
    const int step0 = min(split * per_split, nsteps_all);
    const int nsteps = min(per_split, nsteps_all - step0);
    const int last = nsteps - 1;
    const int KCl = KC - 2 * step0;  // 64-k chunks from this split's first step on
    const int gsz = group * tiles_n;
    const int gid = t / gsz, gin = t - gid * gsz;
    const int gm0 = gid * group;
    const int grows = min(group, tiles_m - gm0);
    const int tm = gm0 + gin % grows, tn = gin / grows;
    const int64_t m0 = (int64_t)tm * BM;
    const int rb0 = tn * (BN / 64);  // first 64-row weight block of the workgroup

    // The epilogue's inputs, requested now so that their round trip overlaps the main loop
    // instead of following it: the weight scales of the workgroup's BN output columns
    // (thread t holds column t's, clamped: the scale array or the one matrix scale), and
    // the row statistics of the workgroup's BM rows
    // (thread t holds row m0 + t % BM, clamped; every thread loads, so the loads need no
    // branch). The first BM threads park them in LDS once the prologue's wait has retired
    // them (they are older than every operand load).
    static_assert(BN == C::kThreads, "one column scale per thread");
    __shared__ int32_t s_xsum[BM];
    __shared__ float s_sx[BM];
    __shared__ __attribute__((aligned(16))) float s_gam[BN];
    const float gam_t = w_scale[rows ? min((int64_t)tn * BN + tid, N - 1) : 0];
    const int64_t m_stat = min(m0 + tid % BM, M - 1);
    const int32_t xsum_t = xsum[m_stat];
    const float sx_t = sx[m_stat];
    auto park_stats = [&] {
        s_gam[tid] = gam_t;
        if (tid < BM) {
            s_xsum[tid] = xsum_t;
            s_sx[tid] = sx_t;
        }
    };

    // This wave's direct-load blocks per step. Activation block (16-row tile at, half h):
    // lane L brings row 16 at + 8 h + L / 8, the piece that slot L % 8 of that row holds
    // (slot ^ row ^ h). Weight block (64-row block rbl, chunk gq of the step): lane L
    // brings row L's 16 bytes. Each load is a wave-uniform 64-bit base (advanced per step
    // in scalar registers) plus a loop-invariant per-lane offset. Rows past M read row
    // M - 1 and blocks past N read the last block: their outputs are never stored. Chunks
    // past K read the last chunk against zero activations (activation rows are
    // zero-padded to a multiple of 256 bytes).
    constexpr int NA = C::kAPerWave, NB = C::kBPerWave;
    const int8_t *xbase = Xq + m0 * ldq + (int64_t)step0 * kBK;  // + st * 128 per step
    uint32_t aoff[NA];
    int adst[NA];
#pragma unroll
    for (int q = 0; q < NA; ++q) {
        const int blk = wave * NA + q;
        const int at = blk >> 1, h = blk & 1;
        const int rho = lane >> 3, slot = lane & 7;
        const int64_t m = min(m0 + at * 16 + 8 * h + rho, M - 1);
        aoff[q] = (uint32_t)((m - m0) * ldq + (slot ^ rho ^ h) * 16);
        adst[q] = blk * 1024;
    }
    const int8_t *wrow[NB];  // uniform: start of the weight block's row of chunks
    int bdst[NB], bchunk[NB];
#pragma unroll
    for (int q = 0; q < NB; ++q) {
        const int blk = wave * NB + q;
        const int rbl = blk >> 1, gq = blk & 1;
        wrow[q] = reinterpret_cast<const int8_t *>(Wp) + (int64_t)min(rb0 + rbl, NBLK - 1) * KC * 1024 +
                  (int64_t)step0 * 2048;
        bdst[q] = C::kABytes + blk * 1024;
        bchunk[q] = gq;
    }
    const uint32_t boff = (uint32_t)(lane * 16);
    auto issue = [&](int st, int8_t *sdst) {
        const int8_t *xs = xbase + (int64_t)st * kBK;
#pragma unroll
        for (int q = 0; q < NA; ++q)
            __builtin_amdgcn_global_load_lds((global_void *)(xs + aoff[q]), (lds_void *)(sdst + adst[q]), 16, 0, 0);
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            const int8_t *ws = wrow[q] + (int64_t)min(2 * st + bchunk[q], KCl - 1) * 1024;
            __builtin_amdgcn_global_load_lds((global_void *)(ws + boff), (lds_void *)(sdst + bdst[q]), 16, 0, 0);
        }
    };

    v4i acc[TM][TN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int i = 0; i < TN; ++i)
            acc[a][i] = v4i{0, 0, 0, 0};

    // LDS read offsets within a stage. Activations: row r of the wave's tile a is row
    // rho = r % 8 of half r / 8 (+ a * 2048); piece 2 g + j sits in slot (2 g + j) ^ c with
    // c = rho ^ (r / 8). Weights: words 2 (g & 1), +1 of chunk g / 2 of row 16 i + r
    // (+ i * 256).
    const int hr = r >> 3, rho_r = r & 7, c = rho_r ^ hr;
    const int a_row = ((wm * TM) * 2 + hr) * 1024 + rho_r * 128;
    const int a_off0 = a_row + ((2 * g) ^ c) * 16;      // substep 0
    const int a_off1 = a_row + ((2 * g + 1) ^ c) * 16;  // substep 1
    const int b_off = C::kABytes + (wn * 2 + (g >> 1)) * 1024 + r * 16 + 8 * (g & 1);
    typedef uint32_t v2u __attribute__((ext_vector_type(2)));
    v4i fa0[TM], fa1[TM];  // activation operands of substeps 0 and 1
    v2u fb[TN], fbn[TN];   // weight words of this step and of the next
    auto read_a = [&](const int8_t *sp, int off, v4i (&fa)[TM]) {
#pragma unroll
        for (int a = 0; a < TM; ++a)
            fa[a] = *reinterpret_cast<const v4i *>(sp + off + a * 2048);
    };
    auto read_b = [&](const int8_t *sp, v2u (&f)[TN]) {
#pragma unroll
        for (int i = 0; i < TN; ++i)
            f[i] = *reinterpret_cast<const v2u *>(sp + b_off + i * 256);
    };
    auto mma = [&](const v4i (&fa)[TM], const v2u (&f)[TN], int j) {
#pragma unroll
        for (int i = 0; i < TN; ++i) {
            const v4i bop = unpack_word(f[i][j]);
#pragma unroll
            for (int a = 0; a < TM; ++a)
                acc[a][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[a], bop, acc[a][i], 0, 0, 0);
        }
    };
    // The barrier: a bare s_barrier after an explicit wait (__syncthreads() adds a fence
    // that would wait for every outstanding load, the steps still ahead included), with
    // compiler-only memory clobbers so that no LDS access moves across it.
    auto barrier = [] {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // Before step st's barrier this wave's loads of steps st + 1 .. st + NS - 1 are
    // outstanding; waiting until at most NS - 2 steps of them remain (vector-memory
    // operations complete in issue order) lands step st + 1, and lgkmcnt(0) retires this
    // wave's reads of the current stage.
    constexpr int kWaitStep = vmcnt_imm((NS - 2) * C::kBlocksPerWave) & ~(0xF << 8);

    // One step on ring stage S (a compile-time constant), with substep-0 operands of step
    // st already in fa0 / fb.
    auto step = [&](auto sc, int st) {
        constexpr int S = decltype(sc)::value;
        int8_t *sp = stage_mem(sc);
        read_a(sp, a_off1, fa1);
        mma(fa0, fb, 0);
        __builtin_amdgcn_s_waitcnt(kWaitStep);
        barrier();
        // Every wave is past its reads of stage S: refill it with step st + NS (clamped
        // to the last step, whose reloaded copy is never read), then read step st + 1's
        // substep-0 operands from the next stage.
        issue(min(st + NS, last), sp);
        int8_t *sn = stage_mem(std::integral_constant<int, (S + 1) % NS>{});
        read_a(sn, a_off0, fa0);
        read_b(sn, fbn);
        mma(fa1, fb, 1);
#pragma unroll
        for (int i = 0; i < TN; ++i)
            fb[i] = fbn[i];
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;

    // K = 0 (nsteps = 0): no loads at all (the operand pointers may be null); the
    // accumulators stay zero.
    if (nsteps > 0) {
        issue(0, lds0);
        issue(min(1, last), lds1);
        if constexpr (NS > 2)
            issue(min(2, last), lds2);
        if constexpr (NS > 3)
            issue(min(3, last), lds3);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 1) * C::kBlocksPerWave));
        barrier();
        park_stats();
        read_a(lds0, a_off0, fa0);
        read_b(lds0, fb);
        // Steps in groups of NS (step st uses stage st % NS), then the remainder.
        int st = 0;
        for (; st + NS <= nsteps; st += NS) {
            step(I0{}, st);
            step(I1{}, st + 1);
            if constexpr (NS > 2)
                step(I2{}, st + 2);
            if constexpr (NS > 3)
                step(I3{}, st + 3);
        }
        if (st < nsteps)
            step(I0{}, st);
        if (st + 1 < nsteps)
            step(I1{}, st + 1);
        if constexpr (NS > 3) {
            if (st + 2 < nsteps)
                step(I2{}, st + 2);
        }
    } else {
        park_stats();
    }
    // Retire the trailing (clamped, unused) loads, then wait until every wave is done
    // with the stages: the epilogue reuses their LDS.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();

    if (SPLITK && nsp > 1) {
        // Split-K hand-off, with no workgroup ever waiting for another: every split stores
        // its int32 partial tile (the MFMA layout, 16 bytes per lane per 16 x 16 tile) with
        // device-coherent stores (sc1: visible to every XCD once performed, so no L2
        // write-back fence is needed), waits until they are performed, then counts its
        // arrival on the tile's counter. The split that arrives last adds the others'
        // partials (device-coherent loads), returns the counter to zero for the next call
        // and runs the epilogue; the others are done.
        __shared__ unsigned arrived;
        constexpr int kSlotBytes = kPartialBytes<BM, BN>;
        const int lane_off = (wave * TM * TN * 64 + lane) * 16;
        auto slot = [&](int sp) {
            return __builtin_amdgcn_make_buffer_rsrc(partials + ((int64_t)(t - full) * nsp + sp) * kSlotBytes, (short)0,
                                                     kSlotBytes, kBufferWord3);
        };
        const __amdgpu_buffer_rsrc_t mine = slot(split);
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
            for (int i = 0; i < TN; ++i)
                __builtin_amdgcn_raw_buffer_store_b128(acc[a][i], mine, lane_off + (a * TN + i) * 1024, 0, kSc1);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __syncthreads();
        if (tid == 0)
            arrived = __hip_atomic_fetch_add(arrivals + (t - full), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (arrived != (unsigned)(nsp - 1))
            return;
        for (int sp = 0; sp < nsp; ++sp) {
            if (sp == split)
                continue;
            const __amdgpu_buffer_rsrc_t other = slot(sp);
#pragma unroll
            for (int a = 0; a < TM; ++a)
#pragma unroll
                for (int i = 0; i < TN; ++i)
                    acc[a][i] += __builtin_amdgcn_raw_buffer_load_b128(other, lane_off + (a * TN + i) * 1024, 0, kSc1);
        }
        if (tid == 0)
            arrivals[t - full] = 0u;
    }

    // Epilogue: each wave passes its 64 x 64 accumulator tile through a private LDS
    // slab, 16 tokens at a time, so that stores are row-contiguous (16 bytes per lane
    // when vec, else 4), instead of the MFMA layout's 4-byte column fragments.
    // Slab pitch 68 words: the MFMA-layout writes (16 columns x 4 rows per instruction)
    // and the row reads both hit 64 distinct banks.
    constexpr int kPitchW = 68;
    // (the first half of the waves in stage 0's memory, the second half in stage 1's)
    constexpr int kHalf = C::kWaves / 2;
    int32_t *slab = reinterpret_cast<int32_t *>(wave < kHalf ? lds0 : lds1) + (wave % kHalf) * 16 * kPitchW;
    const int64_t n0 = (int64_t)tn * BN + wn * 64;
    // Weight scales of the lane's columns (n0 + 4r .. +3 when vec, n0 + lane otherwise) and
    // row statistics of the lane's 16 rows, from LDS.
    const float4 gam = vec ? *reinterpret_cast<const float4 *>(s_gam + wn * 64 + 4 * r)
                           : make_float4(s_gam[wn * 64 + lane], 0.0f, 0.0f, 0.0f);
    int32_t xs_r[TM * 4];
    float sx_r[TM * 4];
#pragma unroll
    for (int c = 0; c < TM * 4; ++c) {
        const int row = wm * 64 + (c >> 2) * 16 + 4 * (c & 3) + g;
        xs_r[c] = s_xsum[row];
        sx_r[c] = s_sx[row];
    }
    // LDS runs one wave's accesses in issue order, so the slab of token tile a + 1 is written
    // right behind the reads of tile a (which still see tile a), and those reads are all
    // issued before any is waited for: one LDS round trip per tile, not one per row.
    auto write_slab = [&](int a) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int i = 0; i < TN; ++i)
                slab[(4 * g + v) * kPitchW + 16 * i + r] = acc[a][i][v];
    };
    write_slab(0);
#pragma unroll
    for (int a = 0; a < TM; ++a) {
        const int64_t mt = m0 + wm * 64 + a * 16;  // first token of this 16-row slab
        if (vec) {
            v4i rows4[4];  // slab rows 4 q + g, columns 4 r .. 4 r + 3
#pragma unroll
            for (int q = 0; q < 4; ++q)
                rows4[q] = *reinterpret_cast<const v4i *>(slab + (4 * q + g) * kPitchW + 4 * r);
            if (a + 1 < TM)
                write_slab(a + 1);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int rr = 4 * q + g;  // slab row of this lane
                const int64_t m = mt + rr;
                const int64_t n = n0 + 4 * r;
                const v4i a4 = rows4[q];
                if (m < M && n < N) {
                    const int32_t xs_m = xs_r[4 * a + q];
                    const float sxm = sx_r[4 * a + q];
                    const v4i d = a4 - xs_m;
                    // Non-temporal: the output is not read again by this kernel, and
                    // streaming it past the caches measured 3-9% faster here.
                    if (ACC)
                        __builtin_nontemporal_store(d, reinterpret_cast<v4i *>(ACC + m * N + n));
                    if (Y) {
                        const v4f y = {(float)d[0] * (gam.x * sxm), (float)d[1] * (gam.y * sxm),
                                       (float)d[2] * (gam.z * sxm), (float)d[3] * (gam.w * sxm)};
                        __builtin_nontemporal_store(y, reinterpret_cast<v4f *>(Y + m * N + n));
                    }
                }
            }
        } else {
            for (int rr = 0; rr < 16; ++rr) {
                const int64_t m = mt + rr;
                const int64_t n = n0 + lane;
                const int32_t a1 = slab[rr * kPitchW + lane];
                if (m < M && n < N) {
                    const int32_t d = a1 - xsum[m];
                    if (ACC)
                        __builtin_nontemporal_store(d, ACC + m * N + n);
                    if (Y)
                        __builtin_nontemporal_store((float)d * (gam.x * sx[m]), Y + m * N + n);
                }
            }
            if (a + 1 < TM)
                write_slab(a + 1);
        }
    }
}

// ------------------------------------------------------------ small-M form
// For products whose 64 x 256 tiles would leave most CUs idle (a few hundred tokens against
// a few thousand rows): 64 x 64 output tiles, one per workgroup of four waves, with the
// tile's 128-k steps split four ways inside the workgroup. Wave w streams a contiguous
// share of the steps through NS stages of its own (NS = 3 at one workgroup per CU, 2 where
// two share a CU; each stage: the step's 64 x 128 activation block and 64 x 32 packed
// weight block, brought by direct loads in k_gemm's LDS layouts), so the main loop has no
// workgroup barrier: a wave's own waits order its loads and its reads. The four partial
// tiles then meet in LDS, and wave w finishes token rows 16 w .. 16 w + 15 of the tile.
// Against k_gemm's split-K form the partial tiles never leave the CU (no workspace), and
// the work spreads over more CUs in shorter shares.
constexpr int kKsWaves = 4;
constexpr int kKsA = 64 * kBK;         // activation block of a step: 64 rows x 128 bytes
constexpr int kKsB = 64 * kBK / 4;     // packed weight block of a step: 64 rows x 32 bytes
constexpr int kKsStage = kKsA + kKsB;  // one wave's stage: 10 KB
constexpr int kKsLoads = kKsA / 1024 + kKsB / 1024;  // direct loads per wave and step

template <int NS>
__global__ __launch_bounds__(kKsWaves * 64) void k_gemm_ks(
    const uint4 *__restrict__ Wp, const float *__restrict__ w_scale, const int8_t *__restrict__ Xq, int64_t ldq,
    const float *__restrict__ sx, const int32_t *__restrict__ xsum, int64_t M, int64_t N, int KC, int tiles_m,
    int tiles, int per_xcd, float *__restrict__ Y, int32_t *__restrict__ ACC, int rows)
{
    static_assert(NS == 2 || NS == 3, "a ring of two or three stages");
    // One array per ring stage, each holding the four waves' copies of that stage (as in
    // k_gemm: distinct objects let the compiler tell which stage a direct load writes).
    __shared__ __attribute__((aligned(1024))) int8_t lds0[kKsWaves * kKsStage];
    __shared__ __attribute__((aligned(1024))) int8_t lds1[kKsWaves * kKsStage];
    __shared__ __attribute__((aligned(1024))) int8_t lds2[NS > 2 ? kKsWaves * kKsStage : 16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int g = lane >> 4, r = lane & 15;

    // Workgroup b runs on XCD b % 8; each XCD takes a contiguous run of tiles, token tiles
    // fastest, so the tiles that share a weight block share that XCD's L2.
    const int b = blockIdx.x;
    const int t = (b % kXcds) * per_xcd + b / kXcds;
    if (t >= tiles)
        return;
    const int tm = t % tiles_m, tn = t / tiles_m;
    const int64_t m0 = (int64_t)tm * 64;
    const int64_t n0 = (int64_t)tn * 64;

    // The epilogue's inputs, requested first so that their round trip overlaps the main
    // loop: the scales of the lane's four weight rows 16 i + r, the statistics of its four
    // tokens 16 wave + 4 g + v (clamped: rows past N and tokens past M are never stored).
    float gam_i[4];
    int32_t xs_v[4];
    float sx_v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        gam_i[i] = w_scale[rows ? min(n0 + 16 * i + r, N - 1) : 0];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int64_t m = min(m0 + 16 * wave + 4 * g + v, M - 1);
        xs_v[v] = xsum[m];
        sx_v[v] = sx[m];
    }

    // This wave's steps: [step0, step0 + nsteps) of the tile's ceil(KC / 2).
    const int nsteps_all = (KC + 1) / 2;
    const int per = (nsteps_all + kKsWaves - 1) / kKsWaves;
    const int step0 = min(wave * per, nsteps_all);
    const int nsteps = min(per, nsteps_all - step0);
    const int last = nsteps - 1;
    const int KCl = KC - 2 * step0;  // 64-k chunks from the wave's first step on

    // Direct loads of one step. Activation block q (16-row tile q / 2, half q % 2): lane L
    // brings row 8 (q % 2) + L / 8 of the tile, the piece slot L % 8 of that row holds
    // (slot ^ row ^ half); rows past M read row M - 1. Weight block gq: chunk gq of the step,
    // lane L bringing row L's 16 bytes; chunks past K read the last chunk (against zero
    // activations: activation rows are zero-padded to a multiple of 256 bytes).
    const int8_t *xbase = Xq + m0 * ldq + (int64_t)step0 * kBK;
    uint32_t aoff[kKsA / 1024];
#pragma unroll
    for (int q = 0; q < kKsA / 1024; ++q) {
        const int at = q >> 1, h = q & 1;
        const int rho = lane >> 3, slot = lane & 7;
        const int64_t m = min(m0 + at * 16 + 8 * h + rho, M - 1);
        aoff[q] = (uint32_t)((m - m0) * ldq + (slot ^ rho ^ h) * 16);
    }
    const int8_t *wrow = reinterpret_cast<const int8_t *>(Wp) + (int64_t)tn * KC * 1024 + (int64_t)step0 * 2048 +
                         lane * 16;
    const int wslot = wave * kKsStage;
    auto issue = [&](int st, int8_t *stage) {
        int8_t *sdst = stage + wslot;
        const int8_t *xs = xbase + (int64_t)st * kBK;
#pragma unroll
        for (int q = 0; q < kKsA / 1024; ++q)
            __builtin_amdgcn_global_load_lds((global_void *)(xs + aoff[q]), (lds_void *)(sdst + q * 1024), 16, 0, 0);
#pragma unroll
        for (int gq = 0; gq < 2; ++gq)
            __builtin_amdgcn_global_load_lds((global_void *)(wrow + (int64_t)min(2 * st + gq, KCl - 1) * 1024),
                                             (lds_void *)(sdst + kKsA + gq * 1024), 16, 0, 0);
    };

    v4i acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc[a][i] = v4i{0, 0, 0, 0};

    // Operand reads within the wave's stage, as in k_gemm (one wave tile of 4 x 4 MFMA
    // tiles): activation row r of 16-row tile a, piece 2 g + j; weight words 2 (g & 1), +1
    // of chunk g / 2 of row 16 i + r.
    const int hr = r >> 3, rho_r = r & 7, c = rho_r ^ hr;
    const int a_row = wslot + hr * 1024 + rho_r * 128;
    const int a_off0 = a_row + ((2 * g) ^ c) * 16;
    const int a_off1 = a_row + ((2 * g + 1) ^ c) * 16;
    const int b_off = wslot + kKsA + (g >> 1) * 1024 + r * 16 + 8 * (g & 1);
    typedef uint32_t v2u __attribute__((ext_vector_type(2)));
    v4i fa0[4], fa1[4];
    v2u fb[4], fbn[4];
    auto read_a = [&](const int8_t *sp, int off, v4i (&fa)[4]) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
            fa[a] = *reinterpret_cast<const v4i *>(sp + off + a * 2048);
    };
    auto read_b = [&](const int8_t *sp, v2u (&f)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            f[i] = *reinterpret_cast<const v2u *>(sp + b_off + i * 256);
    };
    auto mma = [&](const v4i (&fa)[4], const v2u (&f)[4], int j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const v4i bop = unpack_word(f[i][j]);
#pragma unroll
            for (int a = 0; a < 4; ++a)
                acc[a][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[a], bop, acc[a][i], 0, 0, 0);
        }
    };
    // Before refilling a stage: step st + 1's loads landed (at most one step of loads still
    // outstanding) and this wave's reads of the stage returned (lgkmcnt(0)).
    constexpr int kWaitStep = vmcnt_imm((NS - 2) * kKsLoads) & ~(0xF << 8);
    auto step = [&](int8_t *sp, int8_t *sn, int st) {
        read_a(sp, a_off1, fa1);
        mma(fa0, fb, 0);
        __builtin_amdgcn_s_waitcnt(kWaitStep);
        asm volatile("" ::: "memory");
        issue(min(st + NS, last), sp);
        read_a(sn, a_off0, fa0);
        read_b(sn, fbn);
        mma(fa1, fb, 1);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            fb[i] = fbn[i];
    };
    if (nsteps > 0) {
        issue(0, lds0);
        issue(min(1, last), lds1);
        if constexpr (NS > 2)
            issue(min(2, last), lds2);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 1) * kKsLoads));
        asm volatile("" ::: "memory");
        read_a(lds0, a_off0, fa0);
        read_b(lds0, fb);
        int st = 0;
        if constexpr (NS == 3) {
            for (; st + NS <= nsteps; st += NS) {
                step(lds0, lds1, st);
                step(lds1, lds2, st + 1);
                step(lds2, lds0, st + 2);
            }
            if (st < nsteps)
                step(lds0, lds1, st);
            if (st + 1 < nsteps)
                step(lds1, lds2, st + 1);
        } else {
            for (; st + NS <= nsteps; st += NS) {
                step(lds0, lds1, st);
                step(lds1, lds0, st + 1);
            }
            if (st < nsteps)
                step(lds0, lds1, st);
        }
    }
    // The trailing (clamped, unused) loads retire, then every wave is done with the rings.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();

    // Partial tiles through LDS: wave w sends token tile a (acc[a][*]) to wave a, into slot
    // (w - a - 1) mod 4 of a's area (48 KB in all: tiles 0, 1 in lds0, 2, 3 in lds1).
    auto area = [&](int a) -> int8_t * { return (a < 2 ? lds0 : lds1) + (a & 1) * (3 * 4 * 64 * 16); };
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        if (a == wave)
            continue;
        const int s = (wave - a - 1) & 3;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<v4i *>(area(a) + ((s * 4 + i) * 64 + lane) * 16) = acc[a][i];
    }
    __syncthreads();
    v4i d[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        d[i] = acc[0][i];
#pragma unroll
        for (int a = 1; a < 4; ++a)
            if (a == wave)
                d[i] = acc[a][i];
    }
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            d[i] += *reinterpret_cast<const v4i *>(area(wave) + ((s * 4 + i) * 64 + lane) * 16);

    // Epilogue of token tile `wave`: lane (g, r) holds tokens 16 wave + 4 g + v, row 16 i + r.
    const bool vec = (N & 3) == 0 && ((reinterpret_cast<uintptr_t>(Y) | reinterpret_cast<uintptr_t>(ACC)) & 15) == 0;
    if (vec) {
        // Row-contiguous 16-byte stores (16 lanes per 256-byte row piece) instead of 4-byte
        // fragments: each output passes through a slab of 16 tokens x 64 rows (pitch 68
        // words: the MFMA-layout writes and the 16-byte row reads hit distinct banks) in the
        // wave's own exchange area, whose partials it has read. The compiler barriers keep the
        // slab's write / read / next write order; LDS performs a wave's accesses in that order.
        constexpr int kPitchW = 68;
        int32_t *slab = reinterpret_cast<int32_t *>(area(wave));
        const int rq = lane & 15, rrow = lane >> 4;  // read: 4-row quad rq, slab row 4 p + rrow
        auto through = [&](auto value, auto store) {
            asm volatile("" ::: "memory");
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    slab[(4 * g + v) * kPitchW + 16 * i + r] = value(i, v);
            asm volatile("" ::: "memory");
            v4i rows4[4];
#pragma unroll
            for (int p = 0; p < 4; ++p)
                rows4[p] = *reinterpret_cast<const v4i *>(slab + (4 * p + rrow) * kPitchW + 4 * rq);
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int64_t m = m0 + 16 * wave + 4 * p + rrow, n = n0 + 4 * rq;
                if (m < M && n < N)
                    store(m * N + n, rows4[p]);
            }
        };
        if (ACC)
            through([&](int i, int v) { return d[i][v] - xs_v[v]; },
                    [&](int64_t o, v4i x) { __builtin_nontemporal_store(x, reinterpret_cast<v4i *>(ACC + o)); });
        if (Y)
            through([&](int i, int v) { return __float_as_int((float)(d[i][v] - xs_v[v]) * (gam_i[i] * sx_v[v])); },
                    [&](int64_t o, v4i x) {
                        const v4f y = {__int_as_float(x[0]), __int_as_float(x[1]), __int_as_float(x[2]),
                                       __int_as_float(x[3])};
                        __builtin_nontemporal_store(y, reinterpret_cast<v4f *>(Y + o));
                    });
        return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t n = n0 + 16 * i + r;
        const float gam = gam_i[i];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t m = m0 + 16 * wave + 4 * g + v;
            if (m < M && n < N) {
                const int32_t dv = d[i][v] - xs_v[v];
                if (ACC)
                    __builtin_nontemporal_store(dv, ACC + m * N + n);
                if (Y)
                    __builtin_nontemporal_store((float)dv * (gam * sx_v[v]), Y + m * N + n);
            }
        }
    }
}

template <int BM, int BN, int WM, int WN, int NS, int WPE, bool SPLITK>
hipError_t launch_t(const uint4 *Wp, const float *w_scale, bool row_scales, const int8_t *Xq, int64_t ldq, const float *sx,
                    const int32_t *xsum, int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc, char *partials,
                    unsigned *arrivals, int64_t full, int nsplit, hipStream_t s)
{
    using C = GemmCfg<BM, BN, WM, WN, NS>;
    const int KC = (int)((K + 63) / 64);
    const int NBLK = (int)((N + 63) / 64);
    const int tiles_m = (int)((M + BM - 1) / BM);
    const int tiles_n = (int)((N + BN - 1) / BN);
    const int64_t total = (int64_t)tiles_m * tiles_n;
    const int full_x = (int)((full + kXcds - 1) / kXcds);
    const int split_x = (int)((total - full + kXcds - 1) / kXcds);
    const int64_t grid = (int64_t)kXcds * (full_x + (int64_t)split_x * nsplit);
    // 16-byte output stores need every row start 16-byte aligned.
    const int vec = (N % 4 == 0) && (reinterpret_cast<uintptr_t>(Y) % 16 == 0) &&
                    (reinterpret_cast<uintptr_t>(acc) % 16 == 0);
    hipLaunchKernelGGL((k_gemm<BM, BN, WM, WN, NS, WPE, SPLITK>), dim3((unsigned)grid), dim3(C::kThreads), 0, s, Wp,
                       w_scale, Xq, ldq, sx, xsum, M, N, KC, NBLK, tiles_m, tiles_n, kGroup, Y, acc,
                       vec | (row_scales ? 2 : 0), partials, arrivals, (int)full, nsplit, full_x, split_x);
    return hipGetLastError();
}

constexpr int kBM = 64, kBN = 256;
constexpr int64_t kCUs = 256;

}  // namespace

int64_t gemm_tiles(int64_t M, int64_t N) { return ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN); }

// How a shape's tiles are spread over workgroups: the first `full` tiles whole, each later
// one split over `nsplit` workgroups, each over a contiguous share of its k-steps.
// Measured on the 2B-class prefill shapes at M = 256 to 4096:
//  * Tail split: when the tiles fill whole rounds of one per CU and leave a last round of at
//    most half the CUs, that round's tiles split up to one share per CU, every share keeping
//    at least kMinTailSteps steps. A CU runs about one tile per period whatever else it
//    holds, so without it the last round's CUs finish a whole tile after the rest. The
//    K = 6912 shapes gain (320 tiles: 43.5 -> 38.8 us; 640: 66.8 -> 58.7 us); at K = 2560
//    the 5-10 step shares cost what they save.
//  * Otherwise every tile split in 2-4 (full = 0): it pays when the tiles alone leave most
//    of the 768 workgroup slots (three per CU) empty and every split keeps enough steps to
//    amortize its prologue, epilogue and the partial-tile hand-off through memory.
// The small-M form (k_gemm_ks): at least four 128-k steps (one per wave), and at most two
// 64 x 64 tiles per CU: up to 256 tiles one workgroup per CU with a 3-stage ring (120 KB of
// LDS), up to 512 two per CU with a 2-stage ring (80 KB). Measured on the 2B prefill shapes
// against k_gemm (split-K where it splits), us per launch in the step:
//  * M = 256: QKV 12.6 -> 9.0, O 12.1 -> 8.9, down 16.5 -> 13.8 (step 2.07 -> 1.80 ms);
//  * M = 512: QKV 17.3 -> 11.7, O 12.6 -> 11.6, down 22.4 -> 20.2 (step 2.75 -> 2.48 ms),
//    where a 3-stage ring at one workgroup per CU (two rounds) was 5-35% slower;
//  * M = 768: O and down (480 tiles) 17.1 -> 11.5 and 24.4 -> 20.7, but QKV (720 tiles)
//    14.4 -> 18.3, and at M = 1024 (640-960 tiles) QKV 15.0 -> 22.0, O 14.7 -> 18.2.
static bool gemm_small_form(int64_t M, int64_t N, int64_t K)
{
    const int64_t tiles64 = ((M + 63) / 64) * ((N + 63) / 64);
    return M > 0 && N > 0 && K >= 4 * 128 && tiles64 <= 2 * kCUs;
}

GemmPlan gemm_plan(int64_t M, int64_t N, int64_t K)
{
    const int64_t tiles = gemm_tiles(M, N);
    if (gemm_small_form(M, N, K))
        return {tiles, 1};  // no split: the small form sums its k-shares inside the workgroup
    const int64_t steps = ((K + 63) / 64 + 1) / 2;
    const int64_t r = tiles % kCUs;
    if (tiles >= kCUs && r > 0 && r <= kCUs / 2) {
        int P = (int)std::min<int64_t>(4, kCUs / r);
        while (P > 1 && steps < (int64_t)P * kMinTailSteps)
            --P;
        if (P > 1)
            return {tiles - r, P};
    }
    const int64_t min_steps = tiles <= 128 ? 6 : 13;
    for (int S = 4; S >= 2; --S)
        if (tiles * S <= 768 && steps >= S * min_steps)
            return {0, S};
    return {tiles, 1};
}

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    const GemmPlan pl = gemm_plan(M, N, K);
    if (pl.nsplit == 1)
        return 0;
    const int64_t split_tiles = gemm_tiles(M, N) - pl.full;
    return (size_t)(round_up(4 * split_tiles, 256) + split_tiles * pl.nsplit * (int64_t)kPartialBytes<kBM, kBN>);
}

hipError_t launch_gemm(const uint4 *Wp, const float *w_scale, bool row_scales, const int8_t *Xq, int64_t ldq, const float *sx,
                       const int32_t *xsum, int64_t M, int64_t N, int64_t K, float *Y, int32_t *acc, void *workspace,
                       size_t workspace_bytes, hipStream_t s)
{
    // Few tiles (gemm_small_form): 64 x 64 tiles with the k-steps split over a workgroup's
    // four waves; needs no workspace.
    if (gemm_small_form(M, N, K)) {
        const int64_t tiles_m = (M + 63) / 64, tiles64 = tiles_m * ((N + 63) / 64);
        const int per_xcd = (int)((tiles64 + kXcds - 1) / kXcds);
        const dim3 grid((unsigned)(per_xcd * kXcds)), block(kKsWaves * 64);
        const int KC = (int)((K + 63) / 64), rows = row_scales ? 1 : 0;
        if (tiles64 <= kCUs)
            hipLaunchKernelGGL((k_gemm_ks<3>), grid, block, 0, s, Wp, w_scale, Xq, ldq, sx, xsum, M, N, KC,
                               (int)tiles_m, (int)tiles64, per_xcd, Y, acc, rows);
        else
            hipLaunchKernelGGL((k_gemm_ks<2>), grid, block, 0, s, Wp, w_scale, Xq, ldq, sx, xsum, M, N, KC,
                               (int)tiles_m, (int)tiles64, per_xcd, Y, acc, rows);
        return hipGetLastError();
    }
    // Otherwise 64 x 256 blocks of 4 waves, three workgroups per CU (3-stage ring, 48 KB of
    // LDS each): with three waves per SIMD one wave's LDS reads, unpacking and barrier wait
    // hide under the others' MFMAs. Measured on the 2B-class prefill shapes against
    // 128 x 256 blocks of 8 waves, 64 x 128 blocks of 2 waves, wave tiles of 32 and 128
    // tokens and two workgroups per CU with a 4-stage ring.
    const int64_t tiles = gemm_tiles(M, N);
    const GemmPlan pl = gemm_plan(M, N, K);
    const size_t need = gemm_workspace_bytes(M, N, K);
    if (pl.nsplit == 1 || !workspace || workspace_bytes < need)
        return launch_t<kBM, kBN, 1, 4, 3, 3, false>(Wp, w_scale, row_scales, Xq, ldq, sx, xsum, M, N, K, Y, acc,
                                                     nullptr, nullptr, tiles, 1, s);
    unsigned *arrivals = static_cast<unsigned *>(workspace);
    char *partials = static_cast<char *>(workspace) + round_up(4 * (tiles - pl.full), 256);
    return launch_t<kBM, kBN, 1, 4, 3, 3, true>(Wp, w_scale, row_scales, Xq, ldq, sx, xsum, M, N, K, Y, acc, partials,
                                                arrivals, pl.full, pl.nsplit, s);
}

int plan_gemm(int64_t M, int64_t N, int64_t K, bool row_scales, bool split_workspace, char *buf, size_t len)
{
    if (gemm_small_form(M, N, K))
        return snprintf(buf, len, "k_gemm_ks<NS=%d,ROWS=%d>", ((M + 63) / 64) * ((N + 63) / 64) <= kCUs ? 3 : 2,
                        (int)row_scales);
    const GemmPlan pl = gemm_plan(M, N, K);
    const int64_t tiles = gemm_tiles(M, N);
    if (!split_workspace || pl.nsplit == 1)
        return snprintf(buf, len, "k_gemm<SPLITK=0,ROWS=%d>[tiles=%lld]", (int)row_scales, (long long)tiles);
    return snprintf(buf, len, "k_gemm<SPLITK=1,ROWS=%d>[tiles=%lld,full=%lld,splits=%d]", (int)row_scales,
                    (long long)tiles, (long long)pl.full, pl.nsplit);
}

int64_t gemm_arrival_words(int64_t M, int64_t N, int64_t K)
{
    const GemmPlan pl = gemm_plan(M, N, K);
    return pl.nsplit == 1 ? 0 : gemm_tiles(M, N) - pl.full;
}

}  // namespace bt
