// Block-scaled 8-bit GEMM for gfx950 (OCP Microscaling formats).
//
// C[i][j] = sum over k of (2^(SA[i][k/32]-127) A[i][k]) * (2^(SB[j][k/32]-127) B[k][j]),
// with E4M3 or E5M2 element codes and E8M0 block scales, FP32 accumulation
// and output. Page "fix(fp4_gemm autotune) SM107 kernel family excluded from
// autotune candidates and heuristics update - #4856" is about choosing among
// tile variants of a block-scaled low-precision GEMM; it names no format,
// and these are the block-scaled formats gfx950's matrix cores implement.
//
// Storage: A is M rows and B is given as Bt, N rows of K codes (Bt[j][k] =
// B[k][j]); SA is M rows and SB N rows of K/32 scale codes; C is M rows of N
// floats. K % 32 == 0. Block scaling runs along K, so both operands and both
// scale arrays are K-contiguous.
//
//  * The scaled MFMA (32x32x64, f8f6f4 family) takes per lane 32 K values
//    of one row of A (one column of B) in two 16-byte halves, and one E8M0
//    scale per lane. Its two 32-value scale blocks are split over the lane
//    groups: block 0 is the low halves of lanes 0-31 and 32-63 (K 0..15 and
//    16..31), block 1 their high halves (K 32..47 and 48..63), and lane
//    group g supplies the scale of block g (established with one-hot
//    operands and distinct block scales). So lane group g, half h holds K
//    32 h + 16 g .. + 15 of a k-step, and each lane loads the scale of the
//    MX block 2 t + g of its own row or column: a scale is never broadcast.
//  * Global -> LDS: buffer loads that write LDS directly, 1 KB per wave
//    instruction, two stages of BK values of K. Out-of-range offsets write
//    zeros, so M, N and K tails need no other care.
//  * Both operands sit in LDS as K-contiguous rows of BK bytes, 16-byte
//    chunks XOR-swizzled by row, and a fragment is two 128-bit LDS reads (no
//    transposing read is needed for either operand).
//  * Scales (SDMA form, K % 128 == 0): a stage's BK/32 scale bytes of every
//    row travel with the stage's operands as 4-byte LDS loads (one wave
//    instruction moves one dword for each of 64 rows), and each lane reads
//    its rows' dwords from LDS once the stage has landed and extracts the
//    byte of its K block. Loading the scales per lane straight from memory
//    touches one cache line per row per instruction, which took more L1
//    lookups than the operands themselves and halved the throughput.
//    Byte form (other K, where the dwords would be misaligned): one byte
//    load per (MFMA block, K block) of the next stage, issued during the
//    current stage's first k-step. Either way the scale sits in byte 0 of
//    its register (scale byte select 0).
//  * One barrier per stage before its last k-step, as in the 16-bit kernel.
// No atomics and a fixed K order per output: repeated runs give the same
// bits.
#include "sam_dma.h"
#include "sam_internal.h"
#include "sam_variants.h"

namespace sam {

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned u4 __attribute__((ext_vector_type(4)));
typedef unsigned u8v __attribute__((ext_vector_type(8)));

// EB: element bits, 8 (FA, FB: 0 E4M3, 1 E5M2) or 4 (FA = FB = 4, E2M1 packed
// two per byte, element 2 i in the low nibble). BK counts values of K.
template <int FA, int FB, int BM, int BN, int WM, int WN, int BK, bool SDMA, int EB>
__global__ void __launch_bounds__(WM * WN * 64)
__attribute__((amdgpu_waves_per_eu(1, (160 * 1024 / (2 * (BM + BN) * (BK + 8))) * WM * WN / 4 > 0
                                           ? (160 * 1024 / (2 * (BM + BN) * (BK + 8))) * WM * WN / 4 : 1)))
gemm_mx8_kernel(GemmArgs args)
{
    using namespace dma;
    constexpr int NBUF = 2;
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int ROW = BK * EB / 8;                   // bytes per LDS row
    constexpr int VPC = 128 / EB;                      // values of K per 16-byte chunk
    constexpr int RPB = EB == 8 ? 2 : 1;               // 128-bit LDS reads per MFMA operand block
    constexpr int CPR = ROW / 16;                      // 16-byte chunks per row
    constexpr int RPL = 64 / CPR;                      // rows per 1 KB wave load
    constexpr int RSW = CPR >= 16 ? 1 : 16 / CPR;      // rows sharing one 256-byte bank sweep
    constexpr int KSTEPS = BK / 64;                    // MFMA k-steps per stage
    constexpr int A_BYTES = BM * ROW, B_BYTES = BN * ROW;
    constexpr int SDW = BK / 128;                      // scale dwords per row per stage (SDMA)
    constexpr int S_BYTES = SDMA ? (BM + BN) * SDW * 4 : 0;   // [dword d][A rows, then Bt rows]
    constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
    constexpr int A_PW = A_BYTES / 1024 / NW, B_PW = B_BYTES / 1024 / NW;
    constexpr int SPL = SDMA ? (BM + BN) / 64 * SDW : 0;      // 64-row scale loads per stage
    constexpr int SPW = (SPL + NW - 1) / NW;           // ... per wave, at most
    constexpr int LPS = A_PW + B_PW + SPW;             // wave loads per stage (a wave may skip its last)
    constexpr int NSB = TM + TN;                       // MFMA blocks whose scales a lane uses
    constexpr int NSR = SDMA ? SDW : KSTEPS;           // raw scale registers per block
    static_assert(EB == 8 || (EB == 4 && FA == 4 && FB == 4), "8-bit formats or E2M1");
    static_assert(ROW == 128 || ROW == 256, "K per stage: 128- or 256-byte rows");
    static_assert(BK % 128 == 0, "whole scale dwords per stage");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "loads must split evenly over waves");
    static_assert(NBUF * STAGE <= 160 * 1024, "LDS");
    static_assert(LPS + (SDMA ? 0 : NSB * KSTEPS) < 64, "vmcnt range");
    static_assert(BM % 64 == 0 && BN % 64 == 0, "scale loads cover 64 rows");
    static_assert(NBUF == 2, "the prologue fills two stages");

    __shared__ __attribute__((aligned(1024))) unsigned char lds[NBUF * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches and selects
    int tm, tn, s;
    tile_coords(blockIdx.x, args, tm, tn, s);
    const int M = args.M, N = args.N, K = args.K;
    const int KB = K / 32;                             // scale codes per row
    const int RB = K * EB / 8;                         // bytes per operand row
    const int m0 = tm * BM, n0 = tn * BN;
    const int kbeg = s * args.k_chunk;
    const int kend = min(K, kbeg + args.k_chunk);
    const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
    const int wm0 = (wave / WN) * WTM;
    const int wn0 = (wave % WN) * WTN;

    const i4 rA = rsrc_words(static_cast<const char*>(args.A) + (long long)m0 * RB, (long long)(M - m0) * RB);
    const i4 rB = rsrc_words(static_cast<const char*>(args.B) + (long long)n0 * RB, (long long)(N - n0) * RB);
    const __amdgpu_buffer_rsrc_t rSA = make_rsrc(args.sa + (long long)m0 * KB, (long long)(M - m0) * KB);
    const __amdgpu_buffer_rsrc_t rSB = make_rsrc(args.sb + (long long)n0 * KB, (long long)(N - n0) * KB);
    const i4 rSAw = rsrc_words(args.sa + (long long)m0 * KB, (long long)(M - m0) * KB);
    const i4 rSBw = rsrc_words(args.sb + (long long)n0 * KB, (long long)(N - n0) * KB);

    // Wave load q of stage `st`: q < A_PW fetch A rows, the rest Bt rows.
    // Lane l lands at dst + 16 l: row I * RPL + l / CPR, physical chunk
    // l % CPR, which holds logical chunk (K values 16 c .. 16 c + 15)
    // c = (l % CPR) ^ swizzle(row).
    auto issue_one = [&](int st, int q) {
        const int k0 = kbeg + st * BK;
        unsigned char* buf = lds + (st % NBUF) * STAGE;
        if (q >= A_PW + B_PW) {
            // SDMA: scale load sq moves dword d of 64 consecutive rows (A
            // rows first, then Bt rows), i.e. scale codes 4 d .. 4 d + 3 of
            // the stage; dwords past the split's K and rows past M / N load
            // zero.
            const int sq = wave + (q - A_PW - B_PW) * NW;
            if (SPL % NW != 0 && sq >= SPL) return;
            constexpr int G = (BM + BN) / 64;              // 64-row groups
            const int d = sq / G, grp = sq % G;
            const bool is_a = grp * 64 < BM;
            const int r = grp * 64 - (is_a ? 0 : BM) + lane;   // row of A or of Bt
            const int kb = k0 / 32 + 4 * d;
            lds_load4(is_a ? rSAw : rSBw, lds_addr(buf + A_BYTES + B_BYTES + (d * (BM + BN) + grp * 64) * 4),
                      kb * 32 < kend ? r * KB + kb : kOOB);   // rows past M / N: past the record count
            return;
        }
        // Rows past M (N) need no test: the panel's record count ends at row
        // M - m0 (N - n0), so their offsets read zero. K past the split's end
        // must be cut explicitly (it is the next split's, or the next row's).
        const bool is_a = q < A_PW;
        const int I = wave + (is_a ? q : q - A_PW) * NW;
        const int row = I * RPL + lane / CPR;
        const int c = (lane % CPR) ^ ((row / RSW) % CPR);
        const int gk = k0 + c * VPC;                   // first value of K in the chunk
        const int off = gk < kend ? row * RB + gk * EB / 8 : kOOB;
        if (is_a)
            lds_load16(rA, lds_addr(buf + I * 1024), off);
        else
            lds_load16(rB, lds_addr(buf + A_BYTES + I * 1024), off);
    };

    // Scales of MFMA block b (b < TM: A block b, else Bt block b - TM): k-step
    // t uses K block 2 t + (lane >> 5) of the stage. sn holds the next
    // stage's raw registers, sc the current stage's:
    //  byte form: one code per k-step, in byte 0 (scale byte select 0);
    //  SDMA: the row's scale dword d (K blocks 4 d .. 4 d + 3) shifted down by
    //  8 (lane >> 5) bits, so that k-step t finds its code in byte 2 (t & 1)
    //  of register t >> 1 (scale byte select 2 (t & 1)).
    unsigned sc[NSB][NSR], sn[NSB][NSR];
    // Byte form: the next stage's codes straight from memory. Blocks past the
    // split's K, and rows past M / N, load zero (their elements are zero too).
    auto issue_scales = [&](int st, int b) {
        const int kb0 = (kbeg + st * BK) / 32;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            const int kb = kb0 + 2 * t + (lane >> 5);
            const bool kin = kb * 32 < kend;   // rows past M / N: past the record count
            if (b < TM) {
                const int row = wm0 + 32 * b + (lane & 31);
                sn[b][t] = __builtin_amdgcn_raw_buffer_load_b8(rSA, kin ? row * KB + kb : kOOB, 0, 0);
            } else {
                const int row = wn0 + 32 * (b - TM) + (lane & 31);
                sn[b][t] = __builtin_amdgcn_raw_buffer_load_b8(rSB, kin ? row * KB + kb : kOOB, 0, 0);
            }
        }
    };

    // SDMA: the scale dwords of block b's rows for the stage in `buf`.
    auto read_scales = [&](const unsigned char* buf, int b) {
        const int r = (b < TM ? wm0 + 32 * b : BM + wn0 + 32 * (b - TM)) + (lane & 31);
#pragma unroll
        for (int d = 0; d < NSR; ++d)
            sn[b][d] = *reinterpret_cast<const unsigned*>(buf + A_BYTES + B_BYTES + (d * (BM + BN) + r) * 4);
    };

    // Fragment reads, one 128-bit LDS read each; RPB per MFMA block: read
    // r < RPB TM is part r % RPB of A block r / RPB, the rest parts of Bt
    // blocks. A block i of k-step t sits in row wm0 + 32 i + (lane & 31).
    //  8-bit: half h holds K 64 t + 32 h + 16 (lane >> 5) .. + 15 of the
    //  stage (logical chunk 4 t + 2 h + (lane >> 5)), registers 4 h .. 4 h + 3:
    //  the instruction's scale block h is the h halves of both lane groups.
    //  4-bit: the lane holds K 64 t + 32 (lane >> 5) .. + 31 (logical chunk
    //  2 t + (lane >> 5)) in registers 0..3 (4..7 stay zero): for E2M1 the
    //  instruction applies lane group g's scale to all of lane group g's
    //  values, so each lane's share is exactly one MX block. (Both layouts
    //  were established with one-hot operands and distinct block scales.)
    auto read_one = [&](const unsigned char* buf, int t, int r, u8v (&fa)[TM], u8v (&fb)[TN]) {
        const bool is_a = r < RPB * TM;
        const int blk = is_a ? r / RPB : (r - RPB * TM) / RPB;
        const int h = r % RPB;
        const int row = (is_a ? wm0 : wn0) + 32 * blk + (lane & 31);
        u8v& f = is_a ? fa[blk] : fb[blk];
        const int lc = EB == 8 ? 4 * t + 2 * h + (lane >> 5) : 2 * t + (lane >> 5);
        const int c = lc ^ ((row / RSW) % CPR);
        const u4 v = *reinterpret_cast<const u4*>(buf + (is_a ? 0 : A_BYTES) + row * ROW + c * 16);
        if (h) f.hi = v; else f.lo = v;
    };

    v16f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    constexpr int NMF = TM * TN;                  // MFMAs per k-step
    constexpr int NRB = RPB * TN;                 // LDS reads of Bt fragments per k-step
    constexpr int RPS = (NRB + NMF - 1) / NMF;    // ... per MFMA slot
    constexpr int NRD = RPB * (TM + TN);          // all fragment reads of a k-step

    // One k-step: slot m issues MFMA m (A block m / TN, Bt block m % TN),
    // then the next k-step's Bt reads m * RPS .. (into the other Bt set),
    // then, after the last MFMA of A block i, the next k-step's reads of A
    // block i into the same registers (A fragments are single-buffered: each
    // is dead once its row of MFMAs has issued), then its share of the stage
    // loads (last k-step) or of the next stage's scales (first k-step:
    // global byte loads; last k-step, SDMA: LDS reads), evenly spread over
    // the slots.
    auto kstep = [&](u8v (&fa)[TM], const u8v (&fb)[TN], int t, const unsigned char* rbuf, int rt,
                     u8v (&nb)[TN], int load_stage, int scale_stage, int sread_stage) {
#pragma unroll
        for (int m = 0; m < NMF; ++m) {
            const int i = m / TN, j = m % TN;
            if constexpr (SDMA) {
                if (t & 1)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        __builtin_bit_cast(v8i, fa[i]), __builtin_bit_cast(v8i, fb[j]), acc[i][j], FA, FB, 2,
                        (int)sc[i][t >> 1], 2, (int)sc[TM + j][t >> 1]);
                else
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        __builtin_bit_cast(v8i, fa[i]), __builtin_bit_cast(v8i, fb[j]), acc[i][j], FA, FB, 0,
                        (int)sc[i][t >> 1], 0, (int)sc[TM + j][t >> 1]);
            } else {
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    __builtin_bit_cast(v8i, fa[i]), __builtin_bit_cast(v8i, fb[j]), acc[i][j], FA, FB, 0,
                    (int)sc[i][t], 0, (int)sc[TM + j][t]);
            }
#pragma unroll
            for (int r = m * RPS; r < (m + 1) * RPS; ++r)
                if (r < NRB) read_one(rbuf, rt, RPB * TM + r, fa, nb);
            if (j == TN - 1) {
#pragma unroll
                for (int h = 0; h < RPB; ++h) read_one(rbuf, rt, RPB * i + h, fa, nb);
            }
            if (load_stage >= 0) {
#pragma unroll
                for (int q = (m * LPS + NMF - 1) / NMF; q < ((m + 1) * LPS + NMF - 1) / NMF; ++q)
                    if (q < LPS) issue_one(load_stage, q);
            }
            if (scale_stage >= 0) {
#pragma unroll
                for (int b = (m * NSB + NMF - 1) / NMF; b < ((m + 1) * NSB + NMF - 1) / NMF; ++b)
                    if (b < NSB) issue_scales(scale_stage, b);
            }
            if (SDMA && sread_stage >= 0) {
#pragma unroll
                for (int b = (m * NSB + NMF - 1) / NMF; b < ((m + 1) * NSB + NMF - 1) / NMF; ++b)
                    if (b < NSB) read_scales(lds + (sread_stage % NBUF) * STAGE, b);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto take_scales = [&]() {
#pragma unroll
        for (int b = 0; b < NSB; ++b)
#pragma unroll
            for (int d = 0; d < NSR; ++d) sc[b][d] = SDMA ? sn[b][d] >> (8 * (lane >> 5)) : sn[b][d];
    };

    u8v fa[TM], fb[2][TN];
    if constexpr (EB == 4) {
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[i].hi = u4{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[0][j].hi = fb[1][j].hi = u4{0, 0, 0, 0};
    }
    // Stage 0 and its scales, drained completely (so that no scale load is
    // still counted as pending when the loop starts), then stage 1.
    if constexpr (!SDMA) {
#pragma unroll
        for (int b = 0; b < NSB; ++b) issue_scales(0, b);
    }
#pragma unroll
    for (int q = 0; q < LPS; ++q) issue_one(0, q);
    wait_cnt<0, 15>();
    if constexpr (!SDMA) take_scales();
#pragma unroll
    for (int q = 0; q < LPS; ++q) issue_one(1, q);
    barrier();
    if constexpr (SDMA) {
#pragma unroll
        for (int b = 0; b < NSB; ++b) read_scales(lds, b);
        take_scales();
    }
#pragma unroll
    for (int r = 0; r < NRD; ++r) read_one(lds, 0, r, fa, fb[0]);
    __builtin_amdgcn_sched_barrier(0);

    for (int k = 0; k < nk; ++k) {
        const unsigned char* cur = lds + (k % NBUF) * STAGE;
        const unsigned char* nxt = lds + ((k + 1) % NBUF) * STAGE;
        // k-steps 0 .. KSTEPS-2 of stage k, each reading the next k-step; the
        // first also loads stage k+1's scales.
#pragma unroll
        for (int t = 0; t + 1 < KSTEPS; ++t)
            kstep(fa, fb[t & 1], t, cur, t + 1, fb[(t + 1) & 1], -1, (!SDMA && t == 0) ? k + 1 : -1, -1);
        // Stage k fully read by this wave; stage k+1 and its scales landed.
        wait_cnt<0, 0>();
        barrier();
        // Last k-step of stage k: read k-step 0 of stage k+1 (and, SDMA, its
        // scales) and refill the slot stage k leaves with stage k + 2.
        constexpr int L = (KSTEPS - 1) & 1;
        kstep(fa, fb[L], KSTEPS - 1, nxt, 0, fb[L ^ 1], k + NBUF, -1, SDMA ? k + 1 : -1);
        static_assert(L == 1, "an even number of k-steps per stage");
        take_scales();
    }
    wait_cnt<0, 0>();   // no LDS load may still be in flight when the workgroup ends

    float* outp = args.out + (long long)s * args.part_stride + (long long)m0 * N + n0;
    const __amdgpu_buffer_rsrc_t rC = make_rsrc(outp, ((long long)(M - m0) * N - n0) * 4);
    const int lrow = lane & 31, lgrp = lane >> 5;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = wn0 + 32 * j + lrow;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm0 + 32 * i + ((r >> 2) << 3) + (lgrp << 2) + (r & 3);
                const bool ok = m0 + row < M && n0 + col < N;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][r]), rC,
                                                      ok ? (row * N + col) * 4 : kOOB, 0, 0);
            }
        }
    }
}

typedef void (*KernelFn)(GemmArgs);

struct Mx8Kernels {
    int id;
    KernelFn fn[2][2][2];   // 8-bit: [scales through LDS][format of A][format of B]: 0 E4M3, 1 E5M2
    KernelFn fn4[2];        // E2M1: [scales through LDS]
    int threads;
};

#define SAM_MX8_FORMS(BM, BN, WM, WN, BK, SD)                                                                   \
    {{gemm_mx8_kernel<0, 0, BM, BN, WM, WN, BK, SD, 8>, gemm_mx8_kernel<0, 1, BM, BN, WM, WN, BK, SD, 8>},      \
     {gemm_mx8_kernel<1, 0, BM, BN, WM, WN, BK, SD, 8>, gemm_mx8_kernel<1, 1, BM, BN, WM, WN, BK, SD, 8>}}
// The E2M1 form runs twice the values of K per stage (same 128-byte rows).
#define SAM_MX8_ENTRY(id, name, BM, BN, WM, WN, BK, SD, gm, xr, ms, e8, e4)                                  \
    {id, {SAM_MX8_FORMS(BM, BN, WM, WN, BK, false), SAM_MX8_FORMS(BM, BN, WM, WN, BK, SD != 0)},               \
     {gemm_mx8_kernel<4, 4, BM, BN, WM, WN, 2 * BK, false, 4>, gemm_mx8_kernel<4, 4, BM, BN, WM, WN, 2 * BK, SD != 0, 4>}, \
     WM * WN * 64},

const Mx8Kernels kMx8Table[] = {SAM_MX8_VARIANTS(SAM_MX8_ENTRY)};

}  // namespace

hipError_t launch_mx8(const Plan& p, const GemmArgs& a, hipStream_t s)
{
    const bool fp4 = p.dtype == DT_MX4;
    if (!fp4 && (a.fmt_a < 0 || a.fmt_a > 1 || a.fmt_b < 0 || a.fmt_b > 1)) return hipErrorInvalidValue;
    for (const Mx8Kernels& d : kMx8Table) {
        if (d.id != p.variant_id) continue;
        // The scale dwords are 4-byte aligned when K % 128 == 0.
        const int sd = a.K % 128 == 0;
        KernelFn fn = fp4 ? d.fn4[sd] : d.fn[sd][a.fmt_a][a.fmt_b];
        hipLaunchKernelGGL(fn, dim3((unsigned)p.grid), dim3(d.threads), 0, s, a);
        return hipGetLastError();
    }
    return hipErrorInvalidDeviceFunction;
}

}  // namespace sam
