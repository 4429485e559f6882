// FP32 GEMM for short K (K <= 64): C = A*B, row-major A[M][K], B[K][N].
//
// With K this short a 128 x 128 tile is 2 MFLOP of multiplies against 64 KB
// of C to write: at 8192 x 8192 the C write (268 MB) is a large share of the
// time, and the per-tile fill and drain of the K loop (counted as a fixed
// cost per tile on page "Measured data point on fixed-tile vs shape-adaptive
// GEMM", section "The wall, and why we think it's structural") are paid once
// for only two K stages. A data-parallel launch runs each tile's fill,
// multiplies and store one after the other. Here each workgroup stays
// resident and walks its tiles t = g, g + G, ...:
//
//  * Two LDS buffers, each holding one tile's whole A panel (128 rows x KP
//    values of K) and B panel (KP rows x 128 columns). While tile t is
//    multiplied from one, tile t + G's panels load into the other with
//    buffer loads that write LDS directly.
//  * The stores of tile t are issued at the end of its multiplies and drain
//    while tile t + G is multiplied. Loads and stores share the vector
//    memory counter, in issue order, so the wait for tile t + G's panels
//    lets exactly the NS stores issued after them stay in flight. (Staging
//    C through the free operand buffer for 16-byte stores cost two more
//    barriers per tile and measured slower.)
//  * Eight waves, 4 x 2, each a 32 x 64 piece of the tile as 2 x 4 blocks of
//    16x16x4 FP32 MFMAs. Lane l carries row / column l % 16 and, for each 16
//    values of K, the four K values 4 (l / 16) + e, e = 0..3, in A (one
//    128-bit read of a K-contiguous row) and in B (four 32-bit reads of
//    N-contiguous rows), so MFMA step e pairs the same K index in both.
//  * A rows hold 16-byte chunks XOR-swizzled by row, B rows by (k / 4) % 4,
//    so that neither read pattern has bank conflicts.
//  * K past the operand, rows past M and columns past N load zero (out of
//    range buffer offsets); stores past M or N are dropped the same way.
// No atomics, one workgroup per tile, a fixed K order: repeated runs give
// the same bits.
#include "sam_dma.h"
#include "sam_internal.h"
#include "sam_variants.h"

namespace sam {

namespace kp {
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));
}  // namespace kp

template <int KP>
constexpr int kp_lds_bytes() { return 2 * 2 * 128 * KP * 4; }

template <int KP>
__global__ void __launch_bounds__(512)
__attribute__((amdgpu_waves_per_eu(1, 2 * (160 * 1024 / kp_lds_bytes<KP>()))))
gemm_f32_kp_kernel(GemmArgs args)
{
    using namespace kp;
    static_assert(KP == 32 || KP == 64, "K panel: 32 or 64 values");
    constexpr int BT = 128;                    // tile edge
    constexpr int NW = 8;                      // waves
    constexpr int A_ROW = KP * 4;              // bytes per A row in LDS
    constexpr int CPA = KP / 4;                // 16-byte chunks per A row
    constexpr int RPA = 1024 / A_ROW;          // A rows per 1 KB wave load
    constexpr int A_BYTES = BT * A_ROW;
    constexpr int B_ROW = BT * 4;              // bytes per B row (512)
    constexpr int B_BYTES = KP * B_ROW;
    constexpr int BUF = A_BYTES + B_BYTES;
    constexpr int A_PW = A_BYTES / 1024 / NW, B_PW = B_BYTES / 1024 / NW;
    constexpr int NS = 2 * 4 * 4;              // stores per wave per tile: 2 x 4 blocks x 4 values
    static_assert(A_PW * NW * 1024 == A_BYTES && B_PW * NW * 1024 == B_BYTES, "loads split evenly");
    static_assert(A_PW + B_PW + NS < 64, "vmcnt range");

    __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * BUF];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int M = args.M, N = args.N, K = args.K;
    const int T = args.tiles_m * args.tiles_n;
    const int G = gridDim.x;
    const int g = dma::logical_wg(blockIdx.x, G, args.xcd_remap);
    const int wm0 = (wave >> 1) * 32, wn0 = (wave & 1) * 64;
    const int r16 = lane & 15, q = lane >> 4;

    // Swizzled chunk of A row `row` (bank groups distinct over 16 rows).
    auto swz_a = [](int row) { return KP == 64 ? (row & 15) : ((row >> 1) & 7); };

    // The panels of tile t into buffer b.
    auto issue = [&](int t, int b) {
        int tm, tn;
        dma::tile_of(t, args, tm, tn);
        const int m0 = tm * BT, n0 = tn * BT;
        unsigned char* buf = lds + b * BUF;
        const dma::i4 rA = dma::rsrc_words(static_cast<const char*>(args.A) + (long long)m0 * K * 4,
                                           (long long)(M - m0) * K * 4);
        const dma::i4 rB = dma::rsrc_words(static_cast<const char*>(args.B) + (long long)n0 * 4,
                                           (long long)K * N * 4 - (long long)n0 * 4);
#pragma unroll
        for (int u = 0; u < A_PW; ++u) {
            const int I = wave + u * NW;
            const int row = I * RPA + lane / CPA;
            const int c = (lane % CPA) ^ swz_a(row);
            const bool ok = m0 + row < M && 4 * c < K;
            dma::lds_load16(rA, dma::lds_addr(buf + I * 1024), ok ? (row * K + 4 * c) * 4 : dma::kOOB);
        }
#pragma unroll
        for (int u = 0; u < B_PW; ++u) {
            const int I = wave + u * NW;
            const int row = I * 2 + lane / 32;
            const int c = (lane % 32) ^ (4 * ((row >> 2) & 3));
            const bool ok = row < K && n0 + 4 * c < N;
            dma::lds_load16(rB, dma::lds_addr(buf + A_BYTES + I * 1024), ok ? (row * N + 4 * c) * 4 : dma::kOOB);
        }
    };

    int it = 0;
    if (g < T) issue(g, 0);
    for (int t = g; t < T; t += G, ++it) {
        const int b = it & 1;
        // This wave's panels of tile t have landed (only the previous tile's
        // NS stores may still be in flight), then every wave's have.
        if (it == 0)
            dma::wait_cnt<0, 15>();
        else
            dma::wait_cnt<NS, 15>();
        dma::barrier();
        // Every wave is done reading the other buffer (tile t - G).
        if (t + G < T) issue(t + G, b ^ 1);

        const unsigned char* bA = lds + b * BUF;
        const unsigned char* bB = bA + A_BYTES;
        v4f acc[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        // Fragments of 16 values of K; the next group's are read while the
        // current group's MFMAs run.
        u4 fa[2][2];
        float fb[2][4][4];
        auto read = [&](int kk, int f) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = wm0 + 16 * i + r16;
                const int c = (4 * kk + q) ^ swz_a(row);
                fa[f][i] = *reinterpret_cast<const u4*>(bA + row * A_ROW + c * 16);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int k = 16 * kk + 4 * q + e;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int col = wn0 + 16 * j + r16;
                    const int c = (col >> 2) ^ (4 * ((k >> 2) & 3));
                    fb[f][j][e] = *reinterpret_cast<const float*>(bB + k * B_ROW + c * 16 + (col & 3) * 4);
                }
            }
        };
        read(0, 0);
#pragma unroll
        for (int kk = 0; kk < KP / 16; ++kk) {
            const int f = kk & 1;
            if (kk + 1 < KP / 16) read(kk + 1, f ^ 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(fa[f][i][e]), fb[f][j][e],
                                                                          acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }

        // Value r of block (i, j) is element (16 i + 4 q + r, 16 j + r16) of
        // this wave's piece. Out-of-range elements get the out-of-range bits
        // OR-ed into their offsets (no select, which would become branches).
        int tm, tn;
        dma::tile_of(t, args, tm, tn);
        const int m0 = tm * BT, n0 = tn * BT;
        const __amdgpu_buffer_rsrc_t rC = dma::make_rsrc(args.out + (long long)m0 * N, (long long)(M - m0) * N * 4);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = n0 + wn0 + 16 * j + r16;
                const int cmask = ((N - 1 - col) >> 31) & dma::kOOB;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = wm0 + 16 * i + 4 * q + r;
                    const int rmask = ((M - m0 - 1 - row) >> 31) & dma::kOOB;
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][r]), rC,
                                                          ((row * N + col) * 4) | cmask | rmask, 0, 0);
                }
            }
    }
    dma::wait_cnt<0, 0>();   // no LDS load may still be in flight when the workgroup ends
}

typedef void (*KpFn)(GemmArgs);

struct KpKernels {
    int id;
    KpFn fn;
};

#define SAM_KP_ENTRY(id, name, KP, gm, xr, e32) {id, gemm_f32_kp_kernel<KP>},

static const KpKernels kKpTable[] = {SAM_KP_VARIANTS(SAM_KP_ENTRY)};

hipError_t launch_kp(const Plan& p, const GemmArgs& a, hipStream_t s)
{
    for (const KpKernels& k : kKpTable) {
        if (k.id != p.variant_id) continue;
        hipLaunchKernelGGL(k.fn, dim3((unsigned)p.grid), dim3(512), 0, s, a);
        return hipGetLastError();
    }
    return hipErrorInvalidDeviceFunction;
}

}  // namespace sam
