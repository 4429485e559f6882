// FP32 GEMM kernel for gfx950 on the CDNA4 LDS data path.
//
// C = A*B in FP32 (page "Measured data point on fixed-tile vs shape-adaptive
// GEMM", the FP32 square sizes of its results table), row-major A[M][K],
// B[K][N]; K % 4 == 0 and N % 4 == 0 take 16-byte loads, other shapes the
// element-load form.
//
//  * Global -> LDS goes through buffer loads that write LDS directly, 1 KB
//    per wave instruction (lane l lands at base + 16 l); an operand whose rows
//    are not 16-byte pieces (A with K % 4 != 0, B with N % 4 != 0) takes 256
//    bytes per instruction, one element per lane, into the same layout
//    (its element form, ELA / ELB). Neither operand
//    passes through registers and no VALU work is spent on the way. The LDS
//    holds a ring of NBUF stages of BK values of K; the loads of a stage are
//    issued NBUF - 1 stages ahead, spread one per MFMA slot. Out-of-range
//    offsets write zeros, so M, N and K tails cost nothing extra.
//  * A sits in LDS K-contiguous (BK * 4-byte rows, 16-byte chunks
//    XOR-swizzled by the row) and is read as one 128-bit fragment per lane:
//    four consecutive K values of one row.
//  * B sits in LDS in its natural N-contiguous layout and is read V = 4 (or
//    2) consecutive columns of one K row at a time (128- or 64-bit reads).
//    B given transposed (BT: N rows of K values, as the general entry point
//    takes op(B) = B^T) sits K-contiguous like A and is read four
//    consecutive K values of one column at a time, one read per column of
//    the V: the same values reach the same MFMAs, gathered the other way.
//  * A given transposed (AT: K rows of M values) sits M-contiguous like B
//    and is read VA = 4 (or 2) adjacent rows of one K row at a time: lane l
//    of a group of VA row blocks holds rows VA l .. VA l + VA - 1, so block
//    u of the group covers every VA-th row (rows VA l + u). Only the output
//    row order is permuted, and the store undoes it.
//    The 32x32x2 MFMA takes one B value per lane (column lane % 32), so the V
//    columns feed V MFMAs that each cover every V-th column of a 32 V-column
//    group: MFMA v produces columns n + V j + v, j < 32. Only the output
//    column order is permuted, and it is undone at the store, where each
//    lane writes its V adjacent columns as one 4 V-byte store.
//  * K slots: lanes 32..63 of an MFMA take the second K value of its pair.
//    Within a chunk step a lane with K-slot group g reads A chunk 2 c + g
//    (values 8 c + 4 g .. + 3) and B rows 8 c + 4 g + e; MFMA e of the step
//    multiplies element e of both, so every product pairs matching K.
//  * KS = 2 splits each stage's chunk steps between two halves of the
//    workgroup's waves, so 8 waves can each own a 64x64 piece of a 128x128
//    tile (more MFMAs per LDS read than 8 disjoint 32x64 pieces). The two
//    partial sums of each piece meet once at the end through LDS; a + b is
//    the same in either order, so the result does not depend on which wave
//    adds, and the K order stays fixed.
//  * One barrier per stage, between its last two chunk steps: before it
//    every wave has read the whole stage and seen its own loads of the next
//    stage land; after it the next stage's first fragments are read while
//    the last chunk step's MFMAs run, and the freed slot is refilled.
// No atomics and a fixed K order per output: repeated runs give the same
// bits.
#include "sam_dma.h"
#include "sam_internal.h"
#include "sam_sk.h"
#include "sam_variants.h"

namespace sam {

namespace f32ring {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));

// The two FP32 MFMA shapes: G K-slot groups of BLK lanes, N accumulator
// values per lane, and the output row of accumulator value r of a lane.
template <int BLK> struct Blk;
template <> struct Blk<32> {
    typedef v16f T;
    static constexpr int G = 2, N = 16;
    static __device__ __forceinline__ void mfma(T& c, unsigned a, unsigned b) {
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a), __uint_as_float(b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ int row(int lane, int r) { return ((r >> 2) << 3) + ((lane >> 5) << 2) + (r & 3); }
};
template <> struct Blk<16> {
    typedef v4f T;
    static constexpr int G = 4, N = 4;
    static __device__ __forceinline__ void mfma(T& c, unsigned a, unsigned b) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a), __uint_as_float(b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ int row(int lane, int r) { return ((lane >> 4) << 2) + r; }
};

}  // namespace f32ring

template <int BM, int BN, int BK, int NBUF>
constexpr int ring_lds_bytes() { return NBUF * (BM + BN) * BK * 4; }

// One output tile over K values [kbeg, kend): the whole ring pipeline from
// the first loads to the stores. The ring is this function's own LDS array
// (one per instantiation; each kernel instantiates it once), so the
// direct-to-LDS loads address it without a generic-to-LDS conversion. SEG: the tile's result goes to `outp` (row
// stride `ostride` floats), of which `orows` x `ocols` are stored; otherwise
// to C or to the partial slice of split `ostride`.
template <int BM, int BN, int WM, int WN, int BK, int NBUF, int V, int KS, int BLK, bool ELA, bool ELB, bool ELC,
          bool SEG, bool BT, bool AT>
__device__ __forceinline__ void ring_segment(const GemmArgs& args, int tm, int tn, int kbeg, int kend, float* outp,
                                             int ostride, int orows, int ocols, bool to_c)
{
    using namespace dma;
    using namespace f32ring;
    static_assert(BK == 32 || BK == 64, "K per stage: 128- or 256-byte A rows");
    constexpr int NP = WM * WN;                // wave positions in the tile
    constexpr int NW = NP * KS;                // waves
    constexpr int WTM = BM / WM, WTN = BN / WN;
    typedef Blk<BLK> MF;
    typedef typename MF::T acc_t;
    constexpr int G = MF::G;                   // K-slot groups per MFMA
    constexpr int CG = BLK * V;                // columns per column group
    constexpr int TM = WTM / BLK, TN = WTN / CG;
    constexpr int A_ROW = BK * 4;              // bytes per A row in LDS
    constexpr int CPA = A_ROW / 16;            // 16-byte chunks per A row
    constexpr int RPA = 1024 / A_ROW;          // A rows per wave load
    constexpr int RSW = 256 / A_ROW;           // A rows sharing one 256-byte bank sweep
    constexpr int KSTEPS = BK / (4 * G);       // chunk steps per stage
    constexpr int KH = KSTEPS / KS;            // chunk steps per stage per wave
    constexpr int A_BYTES = BM * A_ROW;
    constexpr int B_ROW = BN * 4;
    constexpr int B_BYTES = BK * B_ROW;
    constexpr int STAGE = A_BYTES + B_BYTES;
    constexpr int A_INS = A_BYTES / 1024, B_INS = B_BYTES / 1024;
    constexpr int A_PW = A_INS / NW, B_PW = B_INS / NW;
    constexpr int LA = ELA ? 4 : 1, LB = ELB ? 4 : 1;   // load instructions per 1 KB block
    constexpr int LPS = A_PW * LA + B_PW * LB;          // load instructions per stage per wave
    static_assert(V == 2 || V == 4, "B read width");
    static_assert(WTM % BLK == 0 && WTN % CG == 0, "wave tile: BLK-row blocks, BLK V-column groups");
    static_assert(A_INS % NW == 0 && B_INS % NW == 0, "loads must split evenly over waves");
    static_assert(NBUF >= 2 && NBUF * STAGE <= 160 * 1024, "LDS ring");
    static_assert((NBUF - 1) * LPS < 64, "vmcnt range");
    static_assert(KS == 1 || KS == 2, "intra-workgroup K split");
    static_assert(KH >= 2, "the barrier sits before each wave's last chunk step");
    static_assert(KS == 1 || TM % 2 == 0, "K-split halves exchange half of the row blocks");
    static_assert(!BT || (V == 4 && !ELA && !ELB), "B given transposed: 16-byte loads, four-column reads");
    // BT: B rows are columns of op(B), BK values each, placed like A's rows;
    // RPB of them per 1 KB load. Column n's logical chunk c sits in physical
    // row bt_row(n) at chunk slot c ^ bt_swz(n): the 16 lanes of one read
    // (columns 4 l + v, l < 16, one chunk) then cover all 64 banks.
    constexpr int RPB = 1024 / A_ROW;
    // AT: A rows are K values of op(A), BM values each (A_ROW_T bytes); VA
    // row blocks form a group read VA rows at a time (NRA reads per step).
    constexpr int VA = AT ? (TM % 4 == 0 ? 4 : 2) : 1;
    constexpr int A_ROW_T = BM * 4;
    constexpr int NRA = AT ? (TM / VA) * 4 : TM;
    static_assert(!AT || (TM % VA == 0 && !ELA && !BT && BLK == 16), "A given transposed: groups of VA row blocks");

    __shared__ __attribute__((aligned(1024))) unsigned char lds[NBUF * STAGE];

    // SEG (one of several segments of a stream-K workgroup): the thread id is
    // made opaque so values derived from it are recomputed per segment
    // instead of being kept live across all of them.
    int tid = threadIdx.x;
    if constexpr (SEG) asm volatile("" : "+v"(tid));
    const int lane = tid & 63, lane_id = lane;
    const int wave = tid >> 6;
    const int M = args.M, N = args.N, K = args.K;
    const int m0 = tm * BM, n0 = tn * BN;
    const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
    const int pos = wave % NP, half = wave / NP;
    const int wm0 = (pos / WN) * WTM;
    const int wn0 = (pos % WN) * WTN;
    const int tbase = half * KH;               // this wave's first chunk step of a stage

    const int lda = args.lda, ldb = args.ldb;    // operand row strides (elements)
    const i4 rA = rsrc_words(reinterpret_cast<const char*>(args.A) + (long long)m0 * lda * 4,
                             (long long)(M - m0) * lda * 4);
    const long long b_bytes = (long long)K * ldb * 4;
    const long long a_bytes_t = (long long)K * lda * 4;   // A given transposed: K rows of lda values
    auto bt_row = [](int n) { return RSW == 2 ? n ^ ((n >> 2) & 1) : n; };   // an involution
    auto bt_swz = [](int n) { return (RSW == 2 ? n >> 3 : n >> 2) & (CPA - 1); };

    // Wave load q of stage `st`: the first A_PW LA loads fetch A rows into
    // 1 KB blocks (RPA rows per block, chunks placed swizzled: physical chunk
    // p holds logical chunk p ^ ((row / RSW) % CPA)), the rest B rows in
    // natural order. An operand in element form (ELA / ELB: its rows are not
    // 16-byte pieces) fills each block with four loads, load u covering bytes
    // 256 u .. + 255 of the block, one float per lane.
    auto issue_el = [&](int st, int q) {
        int lane = lane_id;
        if constexpr (SEG) asm volatile("" : "+v"(lane));   // see issue_one
        const int k0 = kbeg + st * BK;
        unsigned char* buf = lds + (st % NBUF) * STAGE;
        if (q < A_PW * LA) {
            const int qb = q / 4, d = 64 * (q % 4) + lane;      // dword of the block
            const int I = wave + qb * NW;
            const int row = I * RPA + (4 * d) / A_ROW;
            const int p = ((4 * d) % A_ROW) / 16;
            const int gk = k0 + 4 * (p ^ ((row / RSW) % CPA)) + (d & 3);
            const bool ok = m0 + row < M && gk < kend;
            lds_load4(rA, lds_addr(buf + I * 1024 + 256 * (q % 4)), ok ? (row * lda + gk) * 4 : kOOB);
        } else {
            const int qq = q - A_PW * LA;
            const int qb = qq / 4, d = 64 * (qq % 4) + lane;
            const int I = wave + qb * NW;
            const int byte = I * 1024 + 4 * d;
            const int row = byte / B_ROW, col = (byte % B_ROW) / 4;
            const bool ok = k0 + row < kend && n0 + col < N;
            const long long bbase = ((long long)k0 * ldb + n0) * 4;
            const i4 rB = rsrc_words(reinterpret_cast<const char*>(args.B) + bbase, b_bytes - bbase);
            lds_load4(rB, lds_addr(buf + A_BYTES + I * 1024 + 256 * (qq % 4)), ok ? (row * ldb + col) * 4 : kOOB);
        }
    };
    auto issue_one = [&](int st, int q) {
        if ((ELA && q < A_PW * LA) || (ELB && q >= A_PW * LA)) {
            issue_el(st, q);
            return;
        }
        if (q >= A_PW * LA) q = A_PW + (q - A_PW * LA);   // 16-byte B loads follow A's
        // Stream-K segments form load offsets at issue rather than keeping
        // them live across segments; the data-parallel form keeps them (the
        // compiler hoists them out of the K loop, which leaves only an add
        // per load inside it: forming them per load costs enough VALU issue
        // to leave the matrix pipe idle).
        int lane = lane_id;
        if constexpr (SEG) asm volatile("" : "+v"(lane));
        const int k0 = kbeg + st * BK;
        unsigned char* buf = lds + (st % NBUF) * STAGE;
        if (AT && q < A_PW) {
            // A^T rows k0 + row, M-contiguous, in their natural order (as B's).
            const int I = wave + q * NW;
            const int byte = I * 1024 + 16 * lane;
            const int row = byte / A_ROW_T, col = (byte % A_ROW_T) / 4;
            const bool ok = k0 + row < kend && m0 + col < M;
            const long long abase = ((long long)k0 * lda + m0) * 4;
            const i4 rAt = rsrc_words(reinterpret_cast<const char*>(args.A) + abase, a_bytes_t - abase);
            lds_load16(rAt, lds_addr(buf + I * 1024), ok ? (row * lda + col) * 4 : kOOB);
        } else if (q < A_PW) {
            const int I = wave + q * NW;
            const int row = I * RPA + lane / CPA;
            const int c = (lane % CPA) ^ ((row / RSW) % CPA);
            const int gk = k0 + 4 * c;
            const bool ok = m0 + row < M && gk < kend;
            lds_load16(rA, lds_addr(buf + I * 1024), ok ? (row * lda + gk) * 4 : kOOB);
        } else if constexpr (BT) {
            // Physical row / slot of this lane -> column n and its chunk c.
            const int I = wave + (q - A_PW) * NW;
            const int prow = I * RPB + lane / CPA;
            const int n = bt_row(prow);
            const int c = (lane % CPA) ^ bt_swz(n);
            const int gk = k0 + 4 * c;
            const bool ok = n0 + n < N && gk < kend;
            const i4 rBt = rsrc_words(reinterpret_cast<const char*>(args.B) + (long long)n0 * ldb * 4,
                                      (long long)(N - n0) * ldb * 4);
            lds_load16(rBt, lds_addr(buf + A_BYTES + I * 1024), ok ? (n * ldb + gk) * 4 : kOOB);
        } else {
            const int I = wave + (q - A_PW) * NW;
            const int byte = I * 1024 + 16 * lane;
            const int row = byte / B_ROW, col = (byte % B_ROW) / 4;
            const bool ok = k0 + row < kend && n0 + col < N;
            const long long bbase = ((long long)k0 * ldb + n0) * 4;
            const i4 rB = rsrc_words(reinterpret_cast<const char*>(args.B) + bbase, b_bytes - bbase);
            lds_load16(rB, lds_addr(buf + A_BYTES + I * 1024), ok ? (row * ldb + col) * 4 : kOOB);
        }
    };

    const int lrow = lane % BLK;
    const int g = lane / BLK;
    // Fragment read r of chunk step t: r < TM is A block r (row wm0 + BLK r +
    // lrow, chunk G t + g) (AT: the NRA reads of its row-block groups); then
    // B reads (j, e) = ((r - NRA) / 4, (r - NRA) % 4):
    // row 4 (G t + g) + e, columns wn0 + CG j + V lrow .. + V - 1.
    constexpr int NRD = NRA + 4 * TN;
    auto read_one = [&](const unsigned char* buf, int t, int r, u4 (&fa)[TM], u4 (&fb)[TN][4]) {
        if (AT && r < NRA) {
            // Read (I, e): rows wm0 + BLK VA I + VA lrow .. + VA - 1 at K row
            // 4 (G t + g) + e; value (I, e, u) is kept at flat index
            // 4 VA I + VA e + u of fa.
            const int I = r >> 2, e = r & 3;
            const unsigned char* p = buf + (4 * (G * t + g) + e) * A_ROW_T + (wm0 + BLK * VA * I + VA * lrow) * 4;
            if constexpr (VA == 4) {
                fa[4 * I + e] = *reinterpret_cast<const u4*>(p);
            } else {
                typedef unsigned int u2 __attribute__((ext_vector_type(2)));
                const u2 x = *reinterpret_cast<const u2*>(p);
                fa[2 * I + (e >> 1)][2 * (e & 1)] = x[0];
                fa[2 * I + (e >> 1)][2 * (e & 1) + 1] = x[1];
            }
        } else if (r < TM) {
            const int row = wm0 + BLK * r + lrow;
            const int c = (G * t + g) ^ ((row / RSW) % CPA);
            fa[r] = *reinterpret_cast<const u4*>(buf + row * A_ROW + c * 16);
        } else if constexpr (BT) {
            // Read (j, v): column wn0 + CG j + V lrow + v, K values 4 (G t + g) .. + 3,
            // held as fb[j][v] (element e is K value e).
            const int j = (r - NRA) >> 2, v = (r - NRA) & 3;
            const int n = wn0 + CG * j + V * lrow + v;
            fb[j][v] = *reinterpret_cast<const u4*>(buf + A_BYTES + bt_row(n) * A_ROW + ((G * t + g) ^ bt_swz(n)) * 16);
        } else {
            const int j = (r - NRA) >> 2, e = (r - NRA) & 3;
            const int row = 4 * (G * t + g) + e;
            const unsigned char* p = buf + A_BYTES + row * B_ROW + (wn0 + CG * j + V * lrow) * 4;
            if constexpr (V == 4) {
                fb[j][e] = *reinterpret_cast<const u4*>(p);
            } else {
                typedef unsigned int u2 __attribute__((ext_vector_type(2)));
                const u2 x = *reinterpret_cast<const u2*>(p);
                fb[j][e] = u4{x[0], x[1], 0u, 0u};
            }
        }
    };

    acc_t acc[TM][TN][V];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < V; ++v)
#pragma unroll
                for (int r = 0; r < MF::N; ++r) acc[i][j][v][r] = 0.0f;

    // MFMA m of a chunk step: e = K element, then A block i, column group j,
    // column phase v (so the same accumulator recurs every V TM TN MFMAs).
    constexpr int NMF = 4 * V * TM * TN;
    auto mfma_one = [&](int m, const u4 (&fa)[TM], const u4 (&fb)[TN][4]) {
        const int e = m / (V * TM * TN);
        const int rest = m % (V * TM * TN);
        const int i = rest / (V * TN), j = (rest / V) % TN, v = rest % V;
        // AT: block i is u = i % VA of group i / VA, its value at flat index
        // 4 VA (i / VA) + VA e + u.
        const unsigned a = AT ? fa[(4 * VA * (i / VA) + VA * e + i % VA) / 4][(VA * e + i % VA) % 4] : fa[i][e];
        MF::mfma(acc[i][j][v], a, BT ? fb[j][v][e] : fb[j][e][v]);
    };

    constexpr int RPS = (NRD + NMF - 1) / NMF;   // reads per MFMA slot
    // One chunk step: MFMA slot m issues MFMA m, then (while reads remain) the
    // next step's read(s) into the other fragment set, then the wave loads q
    // with ceil(q NMF / LPS) == m when a stage is being loaded. The order is
    // pinned so no burst of loads ever blocks MFMA issue behind it.
    auto kstep = [&](const u4 (&fa)[TM], const u4 (&fb)[TN][4], const unsigned char* rbuf, int rt,
                     u4 (&na)[TM], u4 (&nb)[TN][4], int load_stage) {
#pragma unroll
        for (int m = 0; m < NMF; ++m) {
            mfma_one(m, fa, fb);
#pragma unroll
            for (int r = m * RPS; r < (m + 1) * RPS; ++r)
                if (r < NRD) read_one(rbuf, rt, r, na, nb);
            if (load_stage >= 0) {
#pragma unroll
                for (int q = (m * LPS + NMF - 1) / NMF; q < ((m + 1) * LPS + NMF - 1) / NMF; ++q)
                    if (q < LPS) issue_one(load_stage, q);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    u4 fa[2][TM];
    u4 fb[2][TN][4];
    // Fill the whole ring, then wait for stage 0.
#pragma unroll
    for (int st = 0; st < NBUF; ++st)
#pragma unroll
        for (int q = 0; q < LPS; ++q) issue_one(st, q);
    wait_cnt<(NBUF - 1) * LPS, 15>();
    barrier();
#pragma unroll
    for (int r = 0; r < NRD; ++r) read_one(lds, tbase, r, fa[0], fb[0]);
    __builtin_amdgcn_sched_barrier(0);

    // One stage of the K loop. REFILL: its last chunk step refills the slot
    // the stage leaves with stage k + NBUF. With two stages the loop's wait
    // is for every load issued, so the last two stages, whose refill would
    // lie past the end, run without it (a separate copy of the loop, not a
    // branch inside it); with more the wait's count assumes every refill.
    auto stage = [&](int k, auto refill) {
        constexpr bool REFILL = decltype(refill)::value;
        const unsigned char* cur = lds + (k % NBUF) * STAGE;
        const unsigned char* nxt = lds + ((k + 1) % NBUF) * STAGE;
#pragma unroll
        for (int t = 0; t + 1 < KH; ++t)
            kstep(fa[t & 1], fb[t & 1], cur, tbase + t + 1, fa[(t + 1) & 1], fb[(t + 1) & 1], -1);
        // Stage k fully read by this wave; this wave's part of stage k+1 landed.
        wait_cnt<(NBUF - 2) * LPS, 0>();
        barrier();
        // Last chunk step of stage k: read this wave's first step of stage k+1
        // and refill the slot stage k leaves with stage k + NBUF.
        constexpr int L = (KH - 1) & 1;
        kstep(fa[L], fb[L], nxt, tbase, fa[L ^ 1], fb[L ^ 1], REFILL ? k + NBUF : -1);
        if constexpr (L == 0) {   // odd number of chunk steps: next stage starts in set 1
#pragma unroll
            for (int i = 0; i < TM; ++i) fa[0][i] = fa[1][i];
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) fb[0][j][e] = fb[1][j][e];
        }
    };
    constexpr bool TRIM = NBUF == 2;
    const int nk_refill = TRIM ? (nk > NBUF ? nk - NBUF : 0) : nk;
    int k = 0;
    for (; k < nk_refill; ++k) stage(k, std::true_type{});
    if constexpr (TRIM)
        for (; k < nk; ++k) stage(k, std::false_type{});
    wait_cnt<0, 0>();   // no LDS load may still be in flight when the workgroup ends

    // K split: the half-0 wave of a position keeps row blocks [0, TM/2) and
    // the half-1 wave [TM/2, TM); each hands the other half's partial sums
    // over through LDS (the ring is idle now) and adds the partner's. The
    // tail is instantiated per half so every accumulator index is static.
    constexpr int I0 = KS == 2 ? TM / 2 : TM;  // row blocks each wave stores
    // Data-parallel form (outp carries nothing): the tile goes to C, or to
    // split `ostride`'s partial slice, at (m0, n0) with row stride ldc (N
    // for partials). Formed here rather than by the caller, so it is not live
    // through the K loop.
    // ct: the tile goes to C transposed, element (row, col) at C[col][row].
    const bool ct = to_c && args.ct;
    if constexpr (!SEG) {
        outp = args.out + (long long)ostride * args.part_stride +
               (ct ? (long long)n0 * args.ldc + m0 : (long long)m0 * args.ldc + n0);
        orows = M - m0;
        ocols = N - n0;
        ostride = args.ldc;
    }
    const __amdgpu_buffer_rsrc_t rC =
        make_rsrc(outp, orows > 0 && ocols > 0
                            ? (ct ? (long long)(ocols - 1) * ostride + orows : (long long)(orows - 1) * ostride + ocols) * 4
                            : 0);
    const bool gen = to_c && args.epi;       // the general entry point's alpha / beta
    auto finish = [&](auto hc) {
        constexpr int H = decltype(hc)::value;
        constexpr int IB = KS == 2 ? H * I0 : 0;
        if constexpr (KS == 2) {
            constexpr int GF = I0 * TN * V * MF::N;   // floats handed over per lane
            static_assert(NP * 2 * 64 * GF * 4 <= NBUF * STAGE, "exchange fits the ring");
            v4f* xs = reinterpret_cast<v4f*>(lds);
            const int mine = (pos * 2 + H) * 64 * (GF / 4), theirs = (pos * 2 + (1 - H)) * 64 * (GF / 4);
            barrier();   // every wave is past its last read of the ring
#pragma unroll
            for (int ii = 0; ii < I0; ++ii)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int v = 0; v < V; ++v)
#pragma unroll
                        for (int r4 = 0; r4 < MF::N / 4; ++r4) {
                            const int f4 = ((ii * TN + j) * V + v) * (MF::N / 4) + r4;
                            const acc_t& x = acc[(1 - H) * I0 + ii][j][v];
                            xs[mine + f4 * 64 + lane] = v4f{x[4 * r4], x[4 * r4 + 1], x[4 * r4 + 2], x[4 * r4 + 3]};
                        }
            __syncthreads();
#pragma unroll
            for (int ii = 0; ii < I0; ++ii)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int v = 0; v < V; ++v)
#pragma unroll
                        for (int r4 = 0; r4 < MF::N / 4; ++r4) {
                            const int f4 = ((ii * TN + j) * V + v) * (MF::N / 4) + r4;
                            const v4f x = xs[theirs + f4 * 64 + lane];
                            acc_t& y = acc[IB + ii][j][v];
#pragma unroll
                            for (int q = 0; q < 4; ++q) y[4 * r4 + q] = y[4 * r4 + q] + x[q];
                        }
        }
        // Accumulator element r of acc[i][j][v], lane (lrow, g): row wm0 +
        // BLK i + MF::row(lane, r), column wn0 + CG j + V lrow + v. The
        // plain and the alpha / beta stores are separate straight-line loops.
        auto store_all = [&](auto genc) {
            constexpr bool GEN = decltype(genc)::value;
#pragma unroll
            for (int ii = 0; ii < I0; ++ii)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int col = wn0 + CG * j + V * lrow;
#pragma unroll
                    for (int r = 0; r < MF::N; ++r) {
                        const int ib = IB + ii;   // AT: block u = ib % VA of group ib / VA holds every VA-th row
                        const int row = AT ? wm0 + BLK * VA * (ib / VA) + VA * MF::row(lane, r) + ib % VA
                                           : wm0 + BLK * ib + MF::row(lane, r);
                        if constexpr (ELB || ELC) {
                            // Rows need not be 16-byte pieces: one float per
                            // store, each column checked against N.
#pragma unroll
                            for (int v = 0; v < V; ++v) {
                                const bool okv = row < orows && col + v < ocols;
                                StoreC<1>::run(__float_as_uint(acc[IB + ii][j][v][r]), rC,
                                               okv ? (row * ostride + col + v) * 4 : kOOB, args, GEN);
                            }
                            continue;
                        }
                        const bool ok = row < orows && col < ocols;
                        const int off = ok ? (row * ostride + col) * 4 : kOOB;
                        if constexpr (V == 4) {
                            const u4 v = {__float_as_uint(acc[IB + ii][j][0][r]), __float_as_uint(acc[IB + ii][j][1][r]),
                                          __float_as_uint(acc[IB + ii][j][2][r]), __float_as_uint(acc[IB + ii][j][3][r])};
                            StoreC<4>::run(v, rC, off, args, GEN);
                        } else {
                            typedef unsigned int u2 __attribute__((ext_vector_type(2)));
                            const u2 v = {__float_as_uint(acc[IB + ii][j][0][r]),
                                          __float_as_uint(acc[IB + ii][j][1][r])};
                            StoreC<2>::run(v, rC, off, args, GEN);
                        }
                    }
                }
        };
        // Transposed: rows 4 q .. 4 q + 3 of a block are consecutive for
        // every lane, so each of its V columns is stored as four adjacent
        // values of one row of C (one 16-byte store; value by value where
        // the four cross the tile's last row).
        auto store_all_t = [&](auto genc) {
            constexpr bool GEN = decltype(genc)::value;
#pragma unroll
            for (int ii = 0; ii < I0; ++ii)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int col = wn0 + CG * j + V * lrow;
#pragma unroll
                    for (int v = 0; v < V; ++v)
#pragma unroll
                        for (int r4 = 0; r4 < MF::N / 4; ++r4) {
                            const int row0 = wm0 + BLK * (IB + ii) + MF::row(lane, 4 * r4);
                            const acc_t& a = acc[IB + ii][j][v];
                            if (row0 + 3 < orows) {
                                const u4 x = {__float_as_uint(a[4 * r4]), __float_as_uint(a[4 * r4 + 1]),
                                              __float_as_uint(a[4 * r4 + 2]), __float_as_uint(a[4 * r4 + 3])};
                                StoreC<4>::run(x, rC, col + v < ocols ? ((col + v) * ostride + row0) * 4 : kOOB, args,
                                               GEN);
                            } else {
#pragma unroll
                                for (int q = 0; q < 4; ++q)
                                    StoreC<1>::run(__float_as_uint(a[4 * r4 + q]), rC,
                                                   row0 + q < orows && col + v < ocols
                                                       ? ((col + v) * ostride + row0 + q) * 4 : kOOB,
                                                   args, GEN);
                            }
                        }
                }
        };
        if (!AT && ct) {   // the transposed store takes four adjacent rows: not with AT's row order
            if (gen)
                store_all_t(std::true_type{});
            else
                store_all_t(std::false_type{});
        } else if (gen) {
            store_all(std::true_type{});
        } else {
            store_all(std::false_type{});
        }
    };
    if (KS == 1 || half == 0)
        finish(std::integral_constant<int, 0>{});
    else
        finish(std::integral_constant<int, 1>{});
}

// Data-parallel form: one workgroup per (tile, split); split s covers K
// values [s k_chunk, (s + 1) k_chunk) and writes C or its partial slice.
template <int BM, int BN, int WM, int WN, int BK, int NBUF, int V, int KS, int BLK, bool ELA, bool ELB, bool ELC,
          bool BT, bool AT>
__global__ void __launch_bounds__(WM * WN * KS * 64)
__attribute__((amdgpu_waves_per_eu(1, ((160 * 1024 / ring_lds_bytes<BM, BN, BK, NBUF>()) * WM * WN * KS + 3) / 4)))
gemm_f32_ring_kernel(GemmArgs args)
{
    int tm, tn, s;
    dma::tile_coords(blockIdx.x, args, tm, tn, s);
    const int m0 = tm * BM, n0 = tn * BN;
    const int kbeg = s * args.k_chunk;
    const int kend = min(args.K, kbeg + args.k_chunk);
    ring_segment<BM, BN, WM, WN, BK, NBUF, V, KS, BLK, ELA, ELB, ELC, false, BT, AT>(args, tm, tn, kbeg, kend, nullptr,
                                                                                    s, 0, 0, true);
}

// Stream-K form (page "fix(fp4_gemm autotune) SM107 kernel family excluded
// from autotune candidates and heuristics update - #4856", section "Swap
// microbenchmarks across M, N, and K": tile counts that do not fill the
// machine). The T tiles x I K-iterations (BK values each) form one range of
// W = T I iterations, and workgroup g of the G launched owns iterations
// [floor(W g / G), floor(W (g + 1) / G)). A tile wholly inside one range is
// written to C; a tile shared by several ranges leaves each share in a
// workspace slot (the range's first segment in slot 2 g, its last in slot
// 2 g + 1, BM x BN floats each) and the fix-up kernel adds the shares in
// range order. Ranges are numbered by logical workgroup (each XCD holds
// consecutive ranges). The split points depend only on the plan, so the
// result does not depend on timing.
template <int BM, int BN, int WM, int WN, int BK, int NBUF, int V, int KS, int BLK, bool ELA, bool ELB, bool ELC,
          bool BT, bool AT>
__global__ void __launch_bounds__(WM * WN * KS * 64)
__attribute__((amdgpu_waves_per_eu(1, ((160 * 1024 / ring_lds_bytes<BM, BN, BK, NBUF>()) * WM * WN * KS + 3) / 4)))
gemm_f32_ring_sk_kernel(GemmArgs args)
{
    const long long I = args.sk_iters, T = (long long)args.tiles_m * args.tiles_n;
    const long long W = T * I, G = gridDim.x;
    const long long g = dma::logical_wg(blockIdx.x, (int)G, args.xcd_remap);
    long long it = W * g / G;
    const long long end = W * (g + 1) / G;
    // A range spans at most three tiles: the planner keeps W / G <= 2 I.
#pragma unroll
    for (int seg = 0; seg < 3; ++seg) {
        if (it >= end) break;
        const bool first = seg == 0;
        const long long t = it / I;
        const int k0 = (int)(it - t * I);
        const int k1 = (int)min(I, (long long)k0 + (end - it));
        int tm, tn;
        dma::tile_of((int)t, args, tm, tn);
        const int m0 = tm * BM, n0 = tn * BN;
        if (!first) dma::barrier();   // the previous segment's last LDS reads are done
        const int kbeg = k0 * BK, kend = min(args.K, k1 * BK);
        const bool whole = k0 == 0 && k1 == I;
        float* outp = whole ? args.out + (args.ct ? (long long)n0 * args.ldc + m0 : (long long)m0 * args.ldc + n0)
                            : args.ws + (2 * g + (first ? 0 : 1)) * (long long)(BM * BN);
        ring_segment<BM, BN, WM, WN, BK, NBUF, V, KS, BLK, ELA, ELB, ELC, true, BT, AT>(
            args, tm, tn, kbeg, kend, outp, whole ? args.ldc : BN, whole ? args.M - m0 : BM,
            whole ? args.N - n0 : BN, whole);
        it += k1 - k0;
    }
}

typedef void (*F32RingFn)(GemmArgs);

// Stream-K forms exist for tiles up to 128 x 256: larger tiles run out of
// registers across segments, and their tile counts fill the machine anyway.
constexpr int kSkMaxTile = 128 * 256;

// A kernel of the table: data-parallel or stream-K (SK), each operand in
// 16-byte or element form, C stored 16 bytes or one value at a time (ELC:
// its rows are not 16-byte pieces; always so with an element-form B, whose
// rows are C's length). The element forms exist only for variants that have
// them (EL = 1 in the table): they need four times the loads in flight, and
// their address arithmetic costs registers that the largest tiles do not
// have to spare. The padding forms (EL = 2) load both operands 16 bytes at a
// time (from padded copies where need be) and store C either way.
template <int BM, int BN, int WM, int WN, int BK, int NBUF, int V, int KS, int BLK, int EL, bool ELA, bool ELB, bool ELC,
          bool SK>
constexpr F32RingFn ring_kernel() {
    constexpr bool form = EL == 2 ? (!ELA && !ELB) : (ELC == ELB && (EL != 0 || (!ELA && !ELB)));
    if constexpr (form && (!SK || BM * BN <= kSkMaxTile)) {
        static_assert((NBUF - 1) * (((BM + BN) * BK * 4 / 1024) / (WM * WN * KS) * (ELA || ELB ? 4 : 1)) < 64,
                      "loads in flight must stay countable");
        if constexpr (SK)
            return gemm_f32_ring_sk_kernel<BM, BN, WM, WN, BK, NBUF, V, KS, BLK, ELA, ELB, ELC, false, false>;
        else
            return gemm_f32_ring_kernel<BM, BN, WM, WN, BK, NBUF, V, KS, BLK, ELA, ELB, ELC, false, false>;
    } else {
        return nullptr;
    }
}

// A-given-transposed forms (B in its plain layout, N % 4 == 0): the 16x16x4
// variants that read four columns at a time and whose wave tiles hold whole
// groups of two or four row blocks, the 256 x 256 tile included (its reads
// of A^T share one address per group); stream-K forms as for the others.
template <int BM, int BN, int WM, int WN, int BK, int NBUF, int V, int KS, int BLK, bool SK>
constexpr F32RingFn ring_at_kernel() {
    if constexpr (V == 4 && BLK == 16 && (!SK || BM * BN <= kSkMaxTile) && (BM / WM / BLK) % 2 == 0) {
        if constexpr (SK)
            return gemm_f32_ring_sk_kernel<BM, BN, WM, WN, BK, NBUF, V, KS, BLK, false, false, false, false, true>;
        else
            return gemm_f32_ring_kernel<BM, BN, WM, WN, BK, NBUF, V, KS, BLK, false, false, false, false, true>;
    } else {
        return nullptr;
    }
}

struct F32RingKernel {
    int id;
    F32RingFn fn[2][2][2][2];   // [stream-K][a_vec][b_vec][c_vec]: 16-byte pieces (1) or one value at a time (0)
    F32RingFn fixup;
    int fixup_wgs;   // fix-up workgroups per tile
    int threads;
    F32RingFn bt[2][2];         // B given transposed: [stream-K][c_vec] (16-byte loads of A and B)
    F32RingFn at[2];            // A given transposed: [stream-K] (B rows and C rows 16-byte pieces)
};

// B-given-transposed forms: for the 16x16x4 variants that read four columns
// at a time, with tiles of at most 128 x 256 (each of the read addresses of
// a column group is formed per lane, and the 256 x 256 tile has no
// registers to spare for them).
template <int BM, int BN, int WM, int WN, int BK, int NBUF, int V, int KS, int BLK, bool ELC, bool SK>
constexpr F32RingFn ring_bt_kernel() {
    if constexpr (V == 4 && BLK == 16 && BM * BN <= kSkMaxTile) {
        if constexpr (SK)
            return gemm_f32_ring_sk_kernel<BM, BN, WM, WN, BK, NBUF, V, KS, BLK, false, false, ELC, true, false>;
        else
            return gemm_f32_ring_kernel<BM, BN, WM, WN, BK, NBUF, V, KS, BLK, false, false, ELC, true, false>;
    } else {
        return nullptr;
    }
}

#define SAM_F32RING_CSET(BM, BN, WM, WN, BK, NBUF, V, KS, BLK, EL, A, B, SK)            \
    {ring_kernel<BM, BN, WM, WN, BK, NBUF, V, KS, BLK, EL, A, B, true, SK>(),             \
     ring_kernel<BM, BN, WM, WN, BK, NBUF, V, KS, BLK, EL, A, B, false, SK>()}
#define SAM_F32RING_KSET(BM, BN, WM, WN, BK, NBUF, V, KS, BLK, EL, SK)                              \
    {{SAM_F32RING_CSET(BM, BN, WM, WN, BK, NBUF, V, KS, BLK, EL, true, true, SK),                  \
      SAM_F32RING_CSET(BM, BN, WM, WN, BK, NBUF, V, KS, BLK, EL, true, false, SK)},                \
     {SAM_F32RING_CSET(BM, BN, WM, WN, BK, NBUF, V, KS, BLK, EL, false, true, SK),                 \
      SAM_F32RING_CSET(BM, BN, WM, WN, BK, NBUF, V, KS, BLK, EL, false, false, SK)}}

#define SAM_F32RING_ENTRY(id, name, BM, BN, WM, WN, BK, NBUF, V, KS, BLK, EL, gm, xr, ms, e32)      \
    {id,                                                                                         \
     {SAM_F32RING_KSET(BM, BN, WM, WN, BK, NBUF, V, KS, BLK, EL, false),                          \
      SAM_F32RING_KSET(BM, BN, WM, WN, BK, NBUF, V, KS, BLK, EL, true)},                          \
     sk_fixup_kernel<BM, BN>, sk_fixup_wgs<BM, BN>(), WM * WN * KS * 64,                          \
     {{ring_bt_kernel<BM, BN, WM, WN, BK, NBUF, V, KS, BLK, true, false>(),                        \
       ring_bt_kernel<BM, BN, WM, WN, BK, NBUF, V, KS, BLK, false, false>()},                      \
      {ring_bt_kernel<BM, BN, WM, WN, BK, NBUF, V, KS, BLK, true, true>(),                         \
       ring_bt_kernel<BM, BN, WM, WN, BK, NBUF, V, KS, BLK, false, true>()}},                      \
     {ring_at_kernel<BM, BN, WM, WN, BK, NBUF, V, KS, BLK, false>(),                               \
      ring_at_kernel<BM, BN, WM, WN, BK, NBUF, V, KS, BLK, true>()}},
// The padding forms: the same kernels, EL 2, and no B-given-transposed form
// (a padded copy is made in the plain layout).
#define SAM_F32PAD_ENTRY(id, name, BM, BN, WM, WN, BK, NBUF, V, KS, BLK, EL, gm, xr, ms, e32)     \
    {id,                                                                                         \
     {SAM_F32RING_KSET(BM, BN, WM, WN, BK, NBUF, V, KS, BLK, 2, false),                           \
      SAM_F32RING_KSET(BM, BN, WM, WN, BK, NBUF, V, KS, BLK, 2, true)},                           \
     sk_fixup_kernel<BM, BN>, sk_fixup_wgs<BM, BN>(), WM * WN * KS * 64, {{nullptr, nullptr}, {nullptr, nullptr}},     \
     {nullptr, nullptr}},

static const F32RingKernel kF32RingTable[] = {SAM_F32RING_VARIANTS(SAM_F32RING_ENTRY)
                                                  SAM_F32PAD_VARIANTS(SAM_F32PAD_ENTRY)};

hipError_t launch_f32_ring(const Plan& p, const GemmArgs& a, hipStream_t s)
{
    for (const F32RingKernel& k : kF32RingTable) {
        if (k.id != p.variant_id) continue;
        if (p.dtype != DT_F32) return hipErrorInvalidDeviceFunction;
        const int sk = p.sk ? 1 : 0;
        const F32RingFn fn = (p.tr & 2)   ? (p.tr == 2 && p.b_vec && p.c_vec ? k.at[sk] : nullptr)
                             : (p.tr & 1) ? (p.a_vec ? k.bt[sk][p.c_vec ? 1 : 0] : nullptr)
                                          : k.fn[sk][p.a_vec ? 1 : 0][p.b_vec ? 1 : 0][p.c_vec ? 1 : 0];
        if (!fn) return hipErrorInvalidDeviceFunction;
        hipLaunchKernelGGL(fn, dim3((unsigned)p.grid), dim3(k.threads), 0, s, a);
        return hipGetLastError();
    }
    return hipErrorInvalidDeviceFunction;
}

bool f32_has_at(int variant_id, bool stream_k)
{
    for (const F32RingKernel& k : kF32RingTable)
        if (k.id == variant_id) return k.at[stream_k ? 1 : 0] != nullptr;
    return false;
}

bool f32_has_bt(int variant_id, bool stream_k)
{
    for (const F32RingKernel& k : kF32RingTable)
        if (k.id == variant_id) return k.bt[stream_k ? 1 : 0][0] != nullptr && k.bt[stream_k ? 1 : 0][1] != nullptr;
    return false;
}

hipError_t launch_sk_fixup(const Plan& p, const GemmArgs& a, hipStream_t s)
{
    if (p.kind == KIND_DMA) return launch_sk_fixup_dma(p, a, s);
    for (const F32RingKernel& k : kF32RingTable) {
        if (k.id != p.variant_id) continue;
        hipLaunchKernelGGL(k.fixup, dim3((unsigned)((long long)p.tiles_m * p.tiles_n * k.fixup_wgs)), dim3(256), 0, s,
                           a);
        return hipGetLastError();
    }
    return hipErrorInvalidDeviceFunction;
}

}  // namespace sam
