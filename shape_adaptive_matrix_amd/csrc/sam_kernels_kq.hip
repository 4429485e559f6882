// FP32 GEMM in one launch for products too small to fill the machine:
// C = A*B, row-major A[M][K], B[K][N], FP32 in and out.
//
// Page "Measured data point on fixed-tile vs shape-adaptive GEMM" lists a
// D=768 configuration ("What we measured"); it and page "Post-mortem: a GPU
// stack without nvcc, cuBLAS, or LLVM" (section 2.1) count the K-loop drain
// as a fixed cost per tile. At D <= ~1000 the work per CU is a few
// microseconds, so a split-K plan that ends in a second, reducing launch
// pays fixed costs as large as the product itself. Here the K split stays
// inside the workgroup instead:
//
//  * A workgroup owns one 16 TB x 16 TB tile of C and runs four waves, one
//    per SIMD, or eight, two per SIMD; wave w takes K values
//    [w kq, (w + 1) kq), kq a multiple of 64 (four waves) or 32 (eight).
//  * Each wave streams its K range straight from memory into registers, 16
//    values of K per chunk with three chunks (four waves) or one (eight) in
//    flight ahead of the one being multiplied, and runs 16x16x4 FP32 MFMAs on them. Lane l carries row /
//    column l % 16 and the K values 4 (l / 16) + e, e = 0..3, of a chunk, in
//    A and in B alike, so every product pairs the same K index. A is read as
//    one 16-byte piece per row and chunk when K % 4 == 0, else per value; B
//    per value (its 16 lanes of one K row read 64 contiguous bytes).
//  * Every read stays inside A or B (buffer loads; offsets past an operand
//    read zero). Values past the wave's K range are zeroed in both operands,
//    so a value beyond K (an Inf in the next row, say) is never multiplied.
//  * The partial tiles meet in LDS and each element of C is stored as
//    ((P0 + P1) + P2) + ... in wave order: a fixed order, so repeated runs
//    give the same bits, with no atomics and no second launch.
#include "sam_dma.h"
#include "sam_internal.h"
#include "sam_variants.h"

namespace sam {

namespace kq {
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));
}  // namespace kq

// NW waves split K: 4 (one per SIMD, four register sets: three chunks in
// flight) or 8 (two per SIMD, two sets: one chunk in flight, the other wave
// on the SIMD covering the wait).
template <int NW> constexpr int kq_sets() { return NW == 4 ? 4 : 2; }

template <int TB, bool VA, int NW>
__global__ void __launch_bounds__(64 * NW) gemm_f32_kq_kernel(GemmArgs args)
{
    using namespace kq;
    static_assert(NW == 4 || NW == 8, "four or eight waves");
    constexpr int BT = 16 * TB;                // tile edge
    constexpr int LS = BT + 4;                 // LDS row stride (floats): conflict-free partial stores
    constexpr int NSET = kq_sets<NW>();        // register sets: one in use, NSET - 1 in flight
    __shared__ float part[NW][BT * LS];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: the loop below is not divergent
    int tm, tn, s;
    dma::tile_coords(blockIdx.x, args, tm, tn, s);
    const int M = args.M, N = args.N, K = args.K;
    const int m0 = tm * BT, n0 = tn * BT;
    const int kbeg = wave * args.k_chunk;
    const int kend = min(K, kbeg + args.k_chunk);
    const int nch = kend > kbeg ? (kend - kbeg + 15) / 16 : 0;
    const int r16 = lane & 15, q = lane >> 4;

    // A's tile rows and all of B as buffers: rows of A past M and K rows of
    // B past K read zero. Columns of B past N read other values of B, which
    // reach only columns of C that are never stored.
    const __amdgpu_buffer_rsrc_t rA = dma::make_rsrc(static_cast<const char*>(args.A) + (long long)m0 * K * 4,
                                                     (long long)(M - m0) * K * 4);
    const __amdgpu_buffer_rsrc_t rB = dma::make_rsrc(args.B, (long long)K * N * 4);

    // Register set: A values a[i][e] (row block i) and B values b[j][e]
    // (column block j) of one chunk. Values whose K is past kend read zero in
    // both operands (A's would otherwise be the next row's values): their
    // offsets get the out-of-range bits OR-ed in. That is done with a shift
    // and a mask rather than a select, which the compiler would turn into
    // branches around the load, or a select on the loaded value, which it
    // places right after the load and so waits for it at once.
    float a[NSET][TB][4], b[NSET][TB][4];
    auto past = [&](int k) { return ((kend - 1 - k) >> 31) & dma::kOOB; };   // kOOB if k >= kend, else 0
    auto load = [&](int set, int c) {
        const int k = kbeg + 16 * c + 4 * q;
#pragma unroll
        for (int i = 0; i < TB; ++i) {
            const int row = 16 * i + r16;
            if constexpr (VA) {
                // K % 4 == 0, so the four values are all below kend or all past it.
                const u4 v = __builtin_amdgcn_raw_buffer_load_b128(rA, ((row * K + k) * 4) | past(k), 0, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) a[set][i][e] = __uint_as_float(v[e]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    a[set][i][e] = __uint_as_float(
                        __builtin_amdgcn_raw_buffer_load_b32(rA, ((row * K + k + e) * 4) | past(k + e), 0, 0));
            }
        }
#pragma unroll
        for (int j = 0; j < TB; ++j) {
            const int col = n0 + 16 * j + r16;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                b[set][j][e] = __uint_as_float(
                    __builtin_amdgcn_raw_buffer_load_b32(rB, (((k + e) * N + col) * 4) | past(k + e), 0, 0));
        }
    };

    v4f acc[TB][TB];
#pragma unroll
    for (int i = 0; i < TB; ++i)
#pragma unroll
        for (int j = 0; j < TB; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    auto compute = [&](int set) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int i = 0; i < TB; ++i)
#pragma unroll
                for (int j = 0; j < TB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[set][i][e], b[set][j][e], acc[i][j], 0, 0, 0);
    };

    // NSET chunks per trip, with no branch inside it (a branch makes the
    // compiler wait for every load in flight). Chunks past this wave's range
    // hold zeros in both operands, so multiplying them leaves the partial
    // tile unchanged (its values start at +0 and never become -0); the plan
    // makes kq a multiple of 16 NSET, so only the last wave can run such
    // chunks.
    // The scheduling barriers keep each set's loads ahead of the multiplies
    // they are to overlap: left alone, the scheduler sinks loads to their
    // uses to shorten live ranges, and every chunk would wait for its data.
#pragma unroll
    for (int u = 0; u + 1 < NSET; ++u) {
        load(u, u);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int c = 0; c < nch; c += NSET) {
#pragma unroll
        for (int u = 0; u < NSET; ++u) {
            load((u + NSET - 1) % NSET, c + u + NSET - 1);
            __builtin_amdgcn_sched_barrier(0);
            compute(u);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Partial tile of this wave -> LDS, row-major with stride LS. Value r of
    // block (i, j) in lane l is element (16 i + 4 (l / 16) + r, 16 j + l % 16).
#pragma unroll
    for (int i = 0; i < TB; ++i)
#pragma unroll
        for (int j = 0; j < TB; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                part[wave][(16 * i + 4 * q + r) * LS + 16 * j + r16] = acc[i][j][r];
    __syncthreads();

    // (((P0 + P1) + P2) + ...) in wave order, one element per thread and
    // pass, row-major so that consecutive threads store consecutive columns.
    float* crow = args.out + (long long)m0 * N + n0;
    for (int x = threadIdx.x; x < BT * BT; x += 64 * NW) {
        const int row = x / BT, col = x % BT;
        const int o = row * LS + col;
        float v = part[0][o];
#pragma unroll
        for (int w = 1; w < NW; ++w) v = v + part[w][o];
        if (m0 + row < M && n0 + col < N) crow[(long long)row * N + col] = v;
    }
}

typedef void (*KqFn)(GemmArgs);

struct KqKernels {
    int id;
    KqFn fn[2];   // [A rows are whole 16-byte pieces]
    int waves;
};

#define SAM_KQ_ENTRY(id, name, TB, NW, gm, xr, e32) \
    {id, {gemm_f32_kq_kernel<TB, false, NW>, gemm_f32_kq_kernel<TB, true, NW>}, NW},

static const KqKernels kKqTable[] = {SAM_KQ_VARIANTS(SAM_KQ_ENTRY) SAM_KQ8_VARIANTS(SAM_KQ_ENTRY)};

hipError_t launch_kq(const Plan& p, const GemmArgs& a, hipStream_t s)
{
    for (const KqKernels& k : kKqTable) {
        if (k.id != p.variant_id) continue;
        hipLaunchKernelGGL(k.fn[p.a_vec ? 1 : 0], dim3((unsigned)p.grid), dim3(64 * k.waves), 0, s, a);
        return hipGetLastError();
    }
    return hipErrorInvalidDeviceFunction;
}

}  // namespace sam
