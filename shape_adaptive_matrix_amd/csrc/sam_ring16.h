// 16-bit GEMM kernel for gfx950 built on the CDNA4 LDS data path.
//
// C = A*B with bfloat16 / binary16 operands, FP32 accumulation and output
// (page "Measured data point on fixed-tile vs shape-adaptive GEMM", section
// "One more result that surprised us": the 16-bit port that a fixed,
// occupancy-bound design could not speed up). Shape: row-major A[M][K],
// B[K][N], both K % 8 == 0 and N % 8 == 0 (16-byte rows pieces).
//
//  * Global -> LDS goes through buffer loads that write LDS directly (no
//    VGPR staging, no VALU on the way): each wave instruction moves 1 KB,
//    lane l landing at base + 16 l. Out-of-range offsets write zeros, so M,
//    N and K tails cost nothing extra. A stage is BK = 32 values of K; the
//    LDS holds a ring of NBUF stages, NBUF - 1 of them in flight while one is
//    consumed, which covers HBM latency without registers.
//  * A sits in LDS K-contiguous (64-byte rows, 16-byte chunks XOR-swizzled
//    by row >> 2) and is read as one 128-bit fragment per MFMA block.
//  * B sits in LDS in its natural N-contiguous layout (16-byte chunks
//    XOR-swizzled by K row, nsw below) and is read with the transposing LDS
//    load:
//    within each 16-lane group, lane d receives, for k = kbase..kbase+3,
//    the value at column (4 (source lane % 4) + d % 4) of the row that source
//    lane 4 i + d / 4 points at. Two such loads give the eight consecutive K
//    values of one column that the MFMA takes per lane.
//  * Two MFMA block shapes: 32x32x16 and 16x16x32. Both read the same bytes
//    of LDS per FLOP; the 16x16 form issues twice the MFMAs of half the
//    length and sustains about 7% more of the matrix peak on gfx950, at the
//    cost of twice the fragment registers per k-step.
//  * One barrier per stage, placed between the stage's two MFMA k-steps:
//    before it every wave has finished reading the stage (so its buffer can
//    be refilled) and has seen its own loads of the next stage land; after
//    it, the next stage's first fragments are read while the second k-step's
//    MFMAs run.
// No atomics and a fixed K order per output: repeated runs give the same
// bits.
// Shared by the kernel tables of the plain layout (sam_kernels_dma.hip) and
// of the transposed operand layouts (sam_kernels_dma_t.hip).
#pragma once

#include "sam_dma.h"
#include "sam_internal.h"
#include "sam_sk.h"

namespace sam {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));
typedef unsigned int u2 __attribute__((ext_vector_type(2)));

#define SAM_LDS(p) ((__attribute__((address_space(3))) void*)(p))
#define SAM_LDS4S(p) ((__attribute__((address_space(3))) v4s*)(p))

namespace dma {

// 16-bit lane select: half H of x and y -> (x_H | y_H << 16).
template <int H>
__device__ __forceinline__ unsigned pack_halves(unsigned x, unsigned y) {
    return __builtin_amdgcn_perm(y, x, H ? 0x07060302u : 0x05040100u);
}

// The two MFMA block shapes. BLK 32: 32x32x16, lane l holds K values
// 8 (l / 32) .. +7 of row / column l % 32, and accumulator value r is row
// 8 (r / 4) + 4 (l / 32) + r % 4. BLK 16: 16x16x32, lane l holds K values
// 8 (l / 16) .. +7 of row / column l % 16, and value r is row 4 (l / 16) + r.
template <int DT, int BLK> struct Mf;
template <int DT> struct Mf<DT, 32> {
    typedef v16f T;
    static constexpr int KSTEP = 16, NV = 16;
    static __device__ __forceinline__ void mfma(T& c, const u4& a, const u4& b) {
        if constexpr (DT == DT_BF16)
            c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
        else
            c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ int row(int lane, int r) { return ((r >> 2) << 3) + ((lane >> 5) << 2) + (r & 3); }
};
template <int DT> struct Mf<DT, 16> {
    typedef v4f T;
    static constexpr int KSTEP = 32, NV = 4;
    static __device__ __forceinline__ void mfma(T& c, const u4& a, const u4& b) {
        if constexpr (DT == DT_BF16)
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
        else
            c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ int row(int lane, int r) { return ((lane >> 4) << 2) + r; }
};

}  // namespace dma

// Chunk swizzle of a row of K-row-major data in LDS (B in the plain layout,
// A given transposed): LDS slot c of row `row` holds logical 16-byte chunk
// c ^ nsw(row). The transposing fragment reads of one pass (32 lanes: two
// groups of 16 reading rows 8 apart, four rows x four column pairs each)
// then fall on 32 distinct bank pairs: bits 2-3 separate the four rows of a
// group, bit 1 the two groups.
__device__ __forceinline__ int nsw(int row) { return (4 * (row & 3)) ^ (2 * ((row >> 3) & 1)); }

// MODE 0: loads write LDS directly (ring of NBUF stages).
// MODE 1: loads go to registers and are written to LDS with ds_write_b128
//         (NBUF = 2): the loads of stage k+1 are spread over the first k-step
//         of stage k and their LDS writes over the next-to-last one, so the
//         faster register load path overlaps the MFMAs completely.
// MODE 2: A as in MODE 0 (straight into LDS, NBUF = 2); B through registers,
//         transposed there (one v_perm per output dword) and stored
//         K-contiguous, so its fragments are full-rate 128-bit LDS reads
//         instead of half-rate transposing reads.
// MODE 3: B given transposed (op(B) = B^T with B stored N x K, K-contiguous
//         rows, row stride ldb): both operands load straight into LDS the
//         same way, and B's fragments are 128-bit reads like A's (the layout
//         both MFMA operands take natively). Used by the general entry point
//         for a transposed B; the ring and the schedule are MODE 0's.
// MODE 4: A given transposed (op(A) = A^T with A stored K x M, M-contiguous
//         rows, row stride lda): A loads and sits in LDS as B does in MODE 0
//         and its fragments are transposing reads like B's; B as in MODE 0.
// MODE 5: both given transposed: A as in MODE 4, B as in MODE 3.
//
// SWAP (16x16x32 blocks only): the MFMA takes the B fragment as its first
// operand and the A fragment as its second, so it computes the transposed
// block (C^T = B^T A^T on the block) and each lane's four accumulator values
// are four adjacent columns of one row of C, stored with one 16-byte store
// instead of four 4-byte ones (the operand-swap schedule of page
// "fix(fp4_gemm autotune) SM107 kernel family excluded from autotune
// candidates and heuristics update - #4856", section "Swap microbenchmarks
// across M, N, and K", in its form for a symmetric matrix instruction).
//
// One output tile over K values [kbeg, kend). SEG = false: the tile goes to C
// or to split `ostride`'s partial slice; SEG = true (a segment of a stream-K
// workgroup): to `outp` with row stride `ostride`, of which `orows` x `ocols`
// are stored. The ring is this function's own LDS array, so a kernel that
// instantiates it once holds one ring.
template <int DT, int BM, int BN, int WM, int WN, int BK, int NBUF, int MODE, int BLK, int SWAP, bool SEG>
__device__ __forceinline__ void ring16_segment(const GemmArgs& args, int tm, int tn, int kbeg, int kend, float* outp,
                                               int ostride, int orows, int ocols, bool to_c)
{
    using namespace dma;
    static_assert(DT == DT_BF16 || DT == DT_F16, "16-bit operands only");
    static_assert(BK == 32 || BK == 64, "K per stage: 64- or 128-byte A rows");
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    typedef Mf<DT, BLK> MF;
    constexpr int TM = WTM / BLK, TN = WTN / BLK;
    constexpr int A_ROW = BK * 2;              // bytes per A row in LDS
    constexpr int CPA = A_ROW / 16;            // 16-byte chunks per A row
    constexpr int RPA = 64 / CPA;              // A rows per wave load
    constexpr int RSW = 16 / CPA;              // A rows sharing one 256-byte bank sweep
    constexpr int KSTEPS = BK / MF::KSTEP;     // MFMA k-steps per stage
    constexpr int A_BYTES = BM * A_ROW;
    constexpr int B_ROW = BN * 2;              // bytes per B row (MODE 0/1: N-contiguous rows)
    constexpr int B_BYTES = BK * B_ROW;
    constexpr int STAGE = A_BYTES + B_BYTES;
    constexpr int A_INS = A_BYTES / 1024, B_INS = B_BYTES / 1024;   // 1 KB wave loads per stage
    constexpr int A_PW = A_INS / NW, B_PW = B_INS / NW;
    // MODE 2: B stored K-contiguous like A (BN rows of BK values); each thread
    // owns NBS blocks of 8 K x 8 N values.
    constexpr int NT = NW * 64;
    constexpr int NBS = MODE == 2 ? (BK / 8) * (BN / 8) / NT : 0;
    constexpr int LPS = MODE == 2 ? A_PW + 8 * NBS : A_PW + B_PW;   // loads per stage per lane
    constexpr bool DIRECT = MODE == 0 || MODE >= 3;   // every load straight into LDS
    constexpr bool BKC = MODE == 2 || MODE == 3 || MODE == 5;   // B K-contiguous in LDS (rows of BK values)
    constexpr bool ATR = MODE == 4 || MODE == 5;      // A M-contiguous in LDS (BK rows of BM values)
    constexpr int A_ROW_T = BM * 2;            // bytes per A row in LDS when ATR
    constexpr int CPRA = BM / 8;               // 16-byte chunks per A row when ATR
    constexpr int RPIA = 64 / CPRA;            // A rows per wave load when ATR
    constexpr int CPR = BN / 8;                // 16-byte chunks per B row
    constexpr int RPI = 64 / CPR;              // B rows per wave load
    static_assert(WTM % BLK == 0 && WTN % BLK == 0, "wave tile must be whole MFMA blocks");
    static_assert(BLK == 32 || DIRECT, "16x16 blocks: loads straight into LDS only");
    static_assert(A_INS % NW == 0 && B_INS % NW == 0, "loads must split evenly over waves");
    static_assert(CPR >= 16 && 64 % CPR == 0, "BN must be 128 or 256");
    static_assert(!ATR || (CPRA >= 16 && 64 % CPRA == 0), "transposed A: BM must be 128 or 256");
    static_assert(NBUF >= 2 && NBUF * STAGE <= 160 * 1024, "LDS ring");
    static_assert(DIRECT || (NBUF == 2 && KSTEPS >= 3), "register-filled stages need NBUF 2, >= 3 k-steps");
    static_assert(MODE != 2 || NBS * NT == (BK / 8) * (BN / 8), "B blocks must split evenly over threads");
    static_assert((NBUF - 1) * LPS < 64, "vmcnt range");
    static_assert(SWAP == 0 || BLK == 16, "operand swap: 16x16x32 blocks");
    static_assert(!SEG || DIRECT, "stream-K segments: loads straight into LDS");

    __shared__ __attribute__((aligned(1024))) unsigned char lds[NBUF * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // Uniform across the wave: held in a scalar register, so everything
    // derived from it alone stays out of the vector registers (at 256 VGPRs
    // the difference decides whether addresses spill inside the K loop).
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int M = args.M, N = args.N, K = args.K;
    const int m0 = tm * BM, n0 = tn * BN;
    const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
    const int wm0 = (wave / WN) * WTM;
    const int wn0 = (wave % WN) * WTN;

    // Row strides of A and B in elements (K and N for compact operands; a
    // padded copy's stride when a row is not whole 16-byte pieces).
    const int lda = args.lda, ldb = args.ldb;
    const i4 rA = rsrc_words(static_cast<const char*>(args.A) + (long long)m0 * lda * 2,
                             (long long)(M - m0) * lda * 2);
    const __amdgpu_buffer_rsrc_t rAb = make_rsrc(static_cast<const char*>(args.A) + (long long)m0 * lda * 2,
                                                 (long long)(M - m0) * lda * 2);
    const long long b_bytes = (long long)K * ldb * 2;
    const long long a_bytes = (long long)K * lda * 2;   // A given transposed: K rows of lda values

    // One 1 KB wave load of stage `st` (relative to this split): loads
    // 0 .. A_PW-1 fetch A rows, the rest B rows. Slot layout in LDS is the
    // same in both modes: lane l of load q lands at dst(q) + 16 l.
    u4 R[LPS];
    auto issue_one = [&](int st, int q) {
        const int k0 = kbeg + st * BK;
        unsigned char* buf = lds + (st % NBUF) * STAGE;
        if (ATR && q < A_PW) {
            // A^T rows k0 + row (M-contiguous), placed and swizzled as B's in MODE 0.
            const int I = wave + q * NW;
            const int row = I * RPIA + lane / CPRA;
            const int c = (lane % CPRA) ^ nsw(row);
            const bool ok = k0 + row < kend && m0 + c * 8 < M;
            const long long abase = ((long long)k0 * lda + m0) * 2;
            const i4 rAt = rsrc_words(static_cast<const char*>(args.A) + abase, a_bytes - abase);
            lds_load16(rAt, lds_addr(buf + I * 1024), ok ? (row * lda + c * 8) * 2 : kOOB);
        } else if (q < A_PW) {
            const int I = wave + q * NW;                   // RPA rows per load
            const int row = I * RPA + lane / CPA;
            const int c = (lane % CPA) ^ ((row / RSW) % CPA);   // logical chunk stored at this slot
            const int gk = k0 + c * 8;
            const bool ok = m0 + row < M && gk < kend;
            const int off = ok ? (row * lda + gk) * 2 : kOOB;
            if constexpr (MODE != 1)
                lds_load16(rA, lds_addr(buf + I * 1024), off);
            else
                R[q] = __builtin_amdgcn_raw_buffer_load_b128(rAb, off, 0, 0);
        } else if constexpr (MODE == 3 || MODE == 5) {
            // B^T rows n0 + row (K-contiguous), placed and swizzled as A's.
            const int I = wave + (q - A_PW) * NW;
            const int row = I * RPA + lane / CPA;
            const int c = (lane % CPA) ^ ((row / RSW) % CPA);
            const int gk = k0 + c * 8;
            const bool ok = n0 + row < N && gk < kend;
            const i4 rBt = rsrc_words(static_cast<const char*>(args.B) + (long long)n0 * ldb * 2,
                                      (long long)(N - n0) * ldb * 2);
            lds_load16(rBt, lds_addr(buf + A_BYTES + I * 1024), ok ? (row * ldb + gk) * 2 : kOOB);
        } else {
            const int I = wave + (q - A_PW) * NW;
            const int row = I * RPI + lane / CPR;
            const int c = (lane % CPR) ^ nsw(row);
            const bool ok = k0 + row < kend && n0 + c * 8 < N;
            const long long bbase = ((long long)k0 * ldb + n0) * 2;
            const int off = ok ? (row * ldb + c * 8) * 2 : kOOB;
            if constexpr (DIRECT) {
                const i4 rB = rsrc_words(static_cast<const char*>(args.B) + bbase, b_bytes - bbase);
                lds_load16(rB, lds_addr(buf + A_BYTES + I * 1024), off);
            } else {
                const __amdgpu_buffer_rsrc_t rB = make_rsrc(static_cast<const char*>(args.B) + bbase, b_bytes - bbase);
                R[q] = __builtin_amdgcn_raw_buffer_load_b128(rB, off, 0, 0);
            }
        }
    };
    // MODE 2: B block q (8 K rows x 8 columns) into registers, one 16-byte
    // load per K row; rows past the split's K and columns past N load zero.
    u4 RB[NBS > 0 ? NBS : 1][8];
    auto issue_b = [&](int st, int q) {
        const int k0 = kbeg + st * BK;
        const int sb = tid + q * NT;
        const int kc = sb % (BK / 8);
        const int nb = (sb / (BK / 8)) * 8;
        const long long bbase = ((long long)k0 * ldb + n0) * 2;
        const __amdgpu_buffer_rsrc_t rB = make_rsrc(static_cast<const char*>(args.B) + bbase, b_bytes - bbase);
        // Only K rows past the split's end must read zero. Columns past N read
        // the next row's values (or zero past the end of B): they only reach
        // output columns that are never stored.
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const bool ok = k0 + kc * 8 + r < kend;
            RB[q][r] = __builtin_amdgcn_raw_buffer_load_b128(rB, ok ? ((kc * 8 + r) * ldb + nb) * 2 : kOOB, 0, 0);
        }
    };
    // MODE 2: transpose block q and store column nb + c as chunk kc of LDS
    // row nb + c. Blocks with odd nb / 8 store their columns in the order
    // c ^ 1, so the 16 lanes of one store hit rows of both parities (all 16
    // bank groups).
    auto write_b = [&](int st, int q) {
        unsigned char* bb = lds + (st % NBUF) * STAGE + A_BYTES;
        const int sb = tid + q * NT;
        const int kc = sb % (BK / 8);
        const int nb = (sb / (BK / 8)) * 8;
        const unsigned odd = (nb >> 3) & 1;
        // Column c ^ odd of the block is stored by store c: the 16-bit half
        // picked from each dword is selected per lane through the v_perm
        // selector, so no register is ever indexed by a lane-dependent value.
        const unsigned sel_lo = odd ? 0x07060302u : 0x05040100u;   // even c
        const unsigned sel_hi = odd ? 0x05040100u : 0x07060302u;   // odd c
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int d = c >> 1;
            const unsigned sel = (c & 1) ? sel_hi : sel_lo;
            u4 v;
            v[0] = __builtin_amdgcn_perm(RB[q][1][d], RB[q][0][d], sel);
            v[1] = __builtin_amdgcn_perm(RB[q][3][d], RB[q][2][d], sel);
            v[2] = __builtin_amdgcn_perm(RB[q][5][d], RB[q][4][d], sel);
            v[3] = __builtin_amdgcn_perm(RB[q][7][d], RB[q][6][d], sel);
            const int row = nb + (c ^ (int)odd);
            const int ph = kc ^ ((row / RSW) % CPA);
            *reinterpret_cast<u4*>(bb + row * A_ROW + ph * 16) = v;
        }
    };

    // MODE 1: write register slot q of stage `st` to its LDS place.
    auto write_one = [&](int st, int q) {
        unsigned char* buf = lds + (st % NBUF) * STAGE;
        const int dst = q < A_PW ? (wave + q * NW) * 1024 : A_BYTES + (wave + (q - A_PW) * NW) * 1024;
        *reinterpret_cast<u4*>(buf + dst + lane * 16) = R[q];
    };

    const int lrow = lane % BLK;
    const int lgrp = lane / BLK;               // K group of 8 values within a k-step
    const int g16 = lane >> 4, s16 = lane & 15;
    // Fragment reads, one LDS instruction each. Read r < TM: A block r;
    // read TM + 2 j + h: half h (K rows 4h..4h+3 of the lane's eight) of B block j.
    //  A: row wm0 + BLK i + lrow, K KSTEP t + 8 lgrp .. +7, one 128-bit read.
    //  B: column wn0 + BLK j + lrow, the same K, two transposing 64-bit reads;
    //     the 16 lanes of a group address 4 K rows x 16 columns.
    auto read_one = [&](const unsigned char* buf, int t, int r, u4 (&fa)[TM], u2 (&fb)[TN][2]) {
        if (ATR && r < TM) {
            // Two transposing reads, as for B below, give the lane's eight K
            // values of row wm0 + BLK r + lrow.
            u2 h[2];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int col = wm0 + BLK * r + (lrow & ~15) + 4 * (s16 & 3);
                const int row = MF::KSTEP * t + 8 * lgrp + 4 * half + (s16 >> 2);
                const int c = (col >> 3) ^ nsw(row);
                const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    SAM_LDS4S(buf + row * A_ROW_T + c * 16 + (col & 7) * 2));
                h[half] = __builtin_bit_cast(u2, v);
            }
            fa[r] = u4{h[0][0], h[0][1], h[1][0], h[1][1]};
        } else if (r < TM) {
            const int row = wm0 + BLK * r + lrow;
            const int c = ((MF::KSTEP / 8) * t + lgrp) ^ ((row / RSW) % CPA);
            fa[r] = *reinterpret_cast<const u4*>(buf + row * A_ROW + c * 16);
        } else if constexpr (BKC) {
            const int j = r - TM;
            const int row = wn0 + BLK * j + lrow;
            const int c = ((MF::KSTEP / 8) * t + lgrp) ^ ((row / RSW) % CPA);
            const u4 v = *reinterpret_cast<const u4*>(buf + A_BYTES + row * A_ROW + c * 16);
            fb[j][0] = u2{v[0], v[1]};
            fb[j][1] = u2{v[2], v[3]};
        } else {
            const int j = (r - TM) >> 1, half = (r - TM) & 1;
            const int col = wn0 + BLK * j + (lrow & ~15) + 4 * (s16 & 3);
            const int row = MF::KSTEP * t + 8 * lgrp + 4 * half + (s16 >> 2);
            const int c = (col >> 3) ^ nsw(row);
            const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                SAM_LDS4S(buf + A_BYTES + row * B_ROW + c * 16 + (col & 7) * 2));
            fb[j][half] = __builtin_bit_cast(u2, v);
        }
    };

    typename MF::T acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < MF::NV; ++r) acc[i][j][r] = 0.0f;

    auto mfma_one = [&](int m, const u4 (&fa)[TM], const u2 (&fb)[TN][2]) {
        const int i = m / TN, j = m % TN;
        const u4 b = u4{fb[j][0][0], fb[j][0][1], fb[j][1][0], fb[j][1][1]};
        if constexpr (SWAP)
            MF::mfma(acc[i][j], b, fa[i]);
        else
            MF::mfma(acc[i][j], fa[i], b);
    };

    constexpr int NMF = TM * TN;          // MFMAs per k-step
    constexpr int NBR = BKC ? TN : 2 * TN;                  // B reads per k-step
    constexpr int NRD = TM + NBR;                            // LDS reads per k-step
    constexpr int RPS = (NRD + NMF - 1) / NMF;   // reads per MFMA slot
    // 16x16 blocks hold twice the fragment registers per k-step; their A
    // fragments are single-buffered (each block's next read follows its last
    // MFMA) so that eight waves fit 256 registers without spilling.
    constexpr bool ASB = BLK == 16;
    constexpr int FA = ASB ? 0 : 1;   // index mask of the A fragment set

    // One k-step: MFMA slot m issues MFMA m, then (while m < NRD) the next
    // step's read m into the other fragment set, then (in the second k-step)
    // one of this wave's LDS loads every NMF / LPS slots. The order is pinned
    // so that no burst of loads ever blocks MFMA issue behind it.
    auto kstep = [&](const u4 (&fa)[TM], const u2 (&fb)[TN][2], const unsigned char* rbuf, int rt,
                     u4 (&na)[TM], u2 (&nb)[TN][2], int load_stage, int write_stage, int bload_stage = -1) {
#pragma unroll
        for (int m = 0; m < NMF; ++m) {
            mfma_one(m, fa, fb);
            if constexpr (ASB) {
                // A single-buffered: block i of the next k-step is read right
                // after its last MFMA (m = TN i + TN - 1); the NBR B reads go
                // to the other set, one every NMF / NBR slots.
                if (m % TN == TN - 1) read_one(rbuf, rt, m / TN, na, nb);
#pragma unroll
                for (int q = 0; q < NBR; ++q)
                    if ((q * NMF) / NBR == m) read_one(rbuf, rt, TM + q, na, nb);
            } else {
#pragma unroll
                for (int r = m * RPS; r < (m + 1) * RPS; ++r)
                    if (r < NRD) read_one(rbuf, rt, r, na, nb);
            }
            if constexpr (MODE == 2) {
                // A: the A_PW straight-to-LDS loads; B: NBS blocks loaded (k-step 0)
                // and transposed into LDS (next-to-last k-step), spread over slots.
                if (load_stage >= 0) {
#pragma unroll
                    for (int q = (m * A_PW + NMF - 1) / NMF; q < ((m + 1) * A_PW + NMF - 1) / NMF; ++q)
                        if (q < A_PW) issue_one(load_stage, q);
                }
                if (bload_stage >= 0) {
#pragma unroll
                    for (int q = (m * NBS + NMF - 1) / NMF; q < ((m + 1) * NBS + NMF - 1) / NMF; ++q)
                        if (q < NBS) issue_b(bload_stage, q);
                }
                if (write_stage >= 0) {
#pragma unroll
                    for (int q = (m * NBS + NMF - 1) / NMF; q < ((m + 1) * NBS + NMF - 1) / NMF; ++q)
                        if (q < NBS) write_b(write_stage, q);
                }
            } else {
                if (load_stage >= 0) {
                    // loads q with ceil(q * NMF / LPS) == m, i.e. spread evenly over the slots
#pragma unroll
                    for (int q = (m * LPS + NMF - 1) / NMF; q < ((m + 1) * LPS + NMF - 1) / NMF; ++q)
                        if (q < LPS) issue_one(load_stage, q);
                }
                if (write_stage >= 0) {
#pragma unroll
                    for (int q = (m * LPS + NMF - 1) / NMF; q < ((m + 1) * LPS + NMF - 1) / NMF; ++q)
                        if (q < LPS) write_one(write_stage, q);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    u4 fa[2][TM];
    u2 fb[2][TN][2];
    if constexpr (DIRECT) {
        // Fill the whole ring, then wait for stage 0.
#pragma unroll
        for (int st = 0; st < NBUF; ++st)
#pragma unroll
            for (int q = 0; q < LPS; ++q) issue_one(st, q);
        wait_cnt<(NBUF - 1) * LPS, 15>();
    } else if constexpr (MODE == 1) {
#pragma unroll
        for (int q = 0; q < LPS; ++q) issue_one(0, q);
#pragma unroll
        for (int q = 0; q < LPS; ++q) write_one(0, q);
        wait_cnt<63, 0>();
    } else {
        // A of stages 0 and 1 straight to LDS, B of stage 0 through registers.
#pragma unroll
        for (int q = 0; q < A_PW; ++q) issue_one(0, q);
#pragma unroll
        for (int q = 0; q < NBS; ++q) issue_b(0, q);
#pragma unroll
        for (int q = 0; q < NBS; ++q) write_b(0, q);
#pragma unroll
        for (int q = 0; q < A_PW; ++q) issue_one(1, q);
        wait_cnt<A_PW, 0>();   // everything but stage 1's A
    }
    barrier();
#pragma unroll
    for (int r = 0; r < NRD; ++r) read_one(lds, 0, r, fa[0], fb[0]);
    __builtin_amdgcn_sched_barrier(0);

    // One stage of the K loop. REFILL: its last k-step refills the LDS slot
    // the stage leaves. With two stages the loop's wait is for every load
    // issued, so the last two stages, whose refill would lie past the end,
    // run without it (a separate copy of the loop, not a branch inside it);
    // with more stages the wait's count assumes every refill is issued.
    auto stage = [&](int k, auto refill) {
        constexpr bool REFILL = decltype(refill)::value;
        const unsigned char* cur = lds + (k % NBUF) * STAGE;
        const unsigned char* nxt = lds + ((k + 1) % NBUF) * STAGE;
        // k-steps 0 .. KSTEPS-2 of stage k, each reading the next k-step.
        // MODE 1 loads stage k+1 into registers during k-step 0 and writes it
        // to the free LDS slot during k-step KSTEPS-2; MODE 2 does the same
        // for B only.
#pragma unroll
        for (int t = 0; t + 1 < KSTEPS; ++t) {
            if constexpr (MODE == 2)
                kstep(fa[t & FA], fb[t & 1], cur, t + 1, fa[(t + 1) & FA], fb[(t + 1) & 1], -1,
                      t == KSTEPS - 2 ? k + 1 : -1, t == 0 ? k + 1 : -1);
            else
                kstep(fa[t & FA], fb[t & 1], cur, t + 1, fa[(t + 1) & FA], fb[(t + 1) & 1],
                      (MODE == 1 && t == 0) ? k + 1 : -1, (MODE == 1 && t == KSTEPS - 2) ? k + 1 : -1);
        }
        // Stage k fully read by this wave; this wave's part of stage k+1 landed.
        if constexpr (DIRECT)
            wait_cnt<(NBUF - 2) * LPS, 0>();
        else if constexpr (MODE == 1)
            wait_cnt<63, 0>();
        else
            wait_cnt<0, 0>();
        barrier();
        // Last k-step of stage k: read k-step 0 of stage k+1 and refill the
        // LDS slot stage k leaves (MODE 0: whole stage k + NBUF; MODE 2: A of
        // stage k + 2).
        constexpr int L = (KSTEPS - 1) & 1;
        kstep(fa[L & FA], fb[L], nxt, 0, fa[(L ^ 1) & FA], fb[L ^ 1],
              REFILL ? (DIRECT ? k + NBUF : (MODE == 2 ? k + 2 : -1)) : -1, -1);
        if constexpr (L == 0) {   // odd number of k-steps: next stage starts in set 1
#pragma unroll
            for (int i = 0; i < TM; ++i) fa[0][i] = fa[FA][i];
#pragma unroll
            for (int j = 0; j < TN; ++j) { fb[0][j][0] = fb[1][j][0]; fb[0][j][1] = fb[1][j][1]; }
        }
    };
    constexpr bool TRIM = DIRECT && NBUF == 2 && !SEG;   // stream-K segments keep one loop (registers)
    const int nk_refill = TRIM ? (nk > NBUF ? nk - NBUF : 0) : nk;
    int k = 0;
    for (; k < nk_refill; ++k) stage(k, std::true_type{});
    if constexpr (TRIM)
        for (; k < nk; ++k) stage(k, std::false_type{});
    wait_cnt<0, 0>();   // no LDS load may still be in flight when the segment ends

    // The data-parallel form stores to C or to split `ostride`'s partial
    // slice, at (m0, n0) with row stride ldc (N for partials; formed here,
    // so nothing of it is live through the K loop).
    if constexpr (!SEG) {
        outp = args.out + (long long)ostride * args.part_stride + (long long)m0 * args.ldc + n0;
        orows = M - m0;
        ocols = N - n0;
        ostride = args.ldc;
    }
    const __amdgpu_buffer_rsrc_t rC =
        make_rsrc(outp, orows > 0 && ocols > 0 ? ((long long)(orows - 1) * ostride + ocols) * 4 : 0);
    const bool gen = to_c && args.epi;       // the general entry point's alpha / beta
    // The plain and the alpha / beta stores are separate straight-line loops.
    auto store_all = [&](auto genc) {
        constexpr bool GEN = decltype(genc)::value;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                if constexpr (SWAP) {
                    // Transposed block: lane l holds row l % 16 of the block,
                    // columns 4 (l / 16) .. + 3 (N % 8 == 0, so the four are
                    // all inside C or all past it).
                    const int row = wm0 + BLK * i + lrow;
                    const int col = wn0 + BLK * j + 4 * lgrp;
                    const bool ok = row < orows && col < ocols;
                    const u4 v = {__float_as_uint(acc[i][j][0]), __float_as_uint(acc[i][j][1]),
                                  __float_as_uint(acc[i][j][2]), __float_as_uint(acc[i][j][3])};
                    StoreC<4>::run(v, rC, ok ? (row * ostride + col) * 4 : kOOB, args, GEN);
                } else {
                    const int col = wn0 + BLK * j + lrow;
#pragma unroll
                    for (int r = 0; r < MF::NV; ++r) {
                        const int row = wm0 + BLK * i + MF::row(lane, r);
                        const bool ok = row < orows && col < ocols;
                        StoreC<1>::run(__float_as_uint(acc[i][j][r]), rC, ok ? (row * ostride + col) * 4 : kOOB,
                                       args, GEN);
                    }
                }
            }
        }
    };
    if (gen)
        store_all(std::true_type{});
    else
        store_all(std::false_type{});
}

template <int BM, int BN, int WM, int WN, int BK, int NBUF>
constexpr int ring16_waves_per_eu()
{
    return (160 * 1024 / (NBUF * (BM + BN) * BK * 2)) * WM * WN / 4 > 0
               ? (160 * 1024 / (NBUF * (BM + BN) * BK * 2)) * WM * WN / 4 : 1;
}

// Data-parallel form: one workgroup per (tile, split).
template <int DT, int BM, int BN, int WM, int WN, int BK, int NBUF, int MODE, int BLK, int SWAP>
__global__ void __launch_bounds__(WM * WN * 64)
__attribute__((amdgpu_waves_per_eu(1, ring16_waves_per_eu<BM, BN, WM, WN, BK, NBUF>())))
gemm16_dma_kernel(GemmArgs args)
{
    int tm, tn, s;
    dma::tile_coords(blockIdx.x, args, tm, tn, s);
    const int kbeg = s * args.k_chunk;
    const int kend = min(args.K, kbeg + args.k_chunk);
    ring16_segment<DT, BM, BN, WM, WN, BK, NBUF, MODE, BLK, SWAP, false>(args, tm, tn, kbeg, kend, nullptr, s, 0, 0,
                                                                        true);
}

// Data-parallel + stream-K form (page "fix(fp4_gemm autotune) SM107 kernel
// family excluded from autotune candidates and heuristics update - #4856",
// section "Swap microbenchmarks across M, N, and K": a last wave of tiles
// that leaves CUs idle). The first sk_dp tiles (whole waves of resident
// workgroups) run one per workgroup; the remaining T_sk tiles x I
// K-iterations form W = T_sk I iterations shared by sk_grid workgroups in
// equal ranges [floor(W g / G), floor(W (g + 1) / G)). Since T_sk < G, a
// range spans at most two tiles. A tile wholly inside one range goes to C; a
// shared tile leaves each share in a workspace slot (a range's first segment
// in slot 2 g, its second in slot 2 g + 1) and the fix-up kernel adds them in
// range order. All split points depend on the plan alone.
template <int DT, int BM, int BN, int WM, int WN, int BK, int NBUF, int MODE, int BLK, int SWAP>
__global__ void __launch_bounds__(WM * WN * 64)
__attribute__((amdgpu_waves_per_eu(1, ring16_waves_per_eu<BM, BN, WM, WN, BK, NBUF>())))
gemm16_dma_sk_kernel(GemmArgs args)
{
    const long long I = args.sk_iters, dp = args.sk_dp;
    const long long T = (long long)args.tiles_m * args.tiles_n;
    const long long G = args.sk_grid, W = (T - dp) * I;
    // Workgroups are dispatched in id order, so ids below sk_dp (whole waves)
    // run the data-parallel tiles and the last wave the stream-K ranges. Each
    // part is remapped onto the XCDs on its own: one remap over the whole
    // grid would put stream-K ranges into the first wave and push
    // data-parallel tiles into the last.
    const bool is_dp = blockIdx.x < dp;
    const long long L = is_dp ? dma::logical_wg(blockIdx.x, (int)dp, args.xcd_remap)
                              : dp + dma::logical_wg(blockIdx.x - (int)dp, (int)G, args.xcd_remap);
    // A data-parallel workgroup runs one job (its whole tile); a stream-K
    // one runs the segments of its range. One copy of the tile pipeline
    // serves every job (the loop is not unrolled), so nothing is held in
    // registers from one job to the next.
    const long long g = L - dp;
    long long it = is_dp ? 0 : W * g / G;
    const long long end = is_dp ? I : W * (g + 1) / G;
#pragma clang loop unroll(disable)
    for (int seg = 0; seg < 2; ++seg) {
        if (it >= end) break;
        const long long t = is_dp ? L : dp + it / I;
        const int k0 = (int)(is_dp ? 0 : it - (t - dp) * I);
        const int k1 = (int)min(I, (long long)k0 + (end - it));
        int tm, tn;
        dma::tile_of((int)t, args, tm, tn);
        const int m0 = tm * BM, n0 = tn * BN;
        if (seg > 0) dma::barrier();   // the previous segment's last LDS reads are done
        const bool whole = k0 == 0 && k1 == I;
        float* outp = whole ? args.out + (long long)m0 * args.ldc + n0
                            : args.ws + (2 * g + seg) * (long long)(BM * BN);
        ring16_segment<DT, BM, BN, WM, WN, BK, NBUF, MODE, BLK, SWAP, true>(
            args, tm, tn, k0 * BK, min(args.K, k1 * BK), outp, whole ? args.ldc : BN, whole ? args.M - m0 : BM,
            whole ? args.N - n0 : BN, whole);
        it += k1 - k0;
    }
}

}  // namespace sam
