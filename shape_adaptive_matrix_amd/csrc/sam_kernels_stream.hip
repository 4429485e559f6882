// Streaming kernels for skinny FP32 products (M <= 16 or N <= 16).
//
// With at most 16 rows (or columns) of C the product is HBM-bound: the large
// operand has to be read once at full bandwidth and little else matters. Few
// output tiles cannot fill the device, so the work is also split along K (the
// tile-count argument of page "fix(fp4_gemm autotune) SM107 kernel family
// excluded from autotune candidates and heuristics update - #4856", section
// "Swap microbenchmarks across M, N, and K"). The kernels
//  * stream the large operand straight from memory into MFMA operand
//    registers, 16 bytes per lane per load, with many light waves per CU so
//    that many bytes are in flight (no LDS staging on the way in);
//  * keep the small operand's slice for the wave's K range in registers;
//  * use 16x16x4 FP32 MFMAs. One 16-byte load carries four consecutive values
//    for one lane; the four MFMAs it feeds take one element each, which only
//    permutes the output columns (skinny M) or the K order (skinny N). Both
//    permutations are fixed, so every run sums in the same order;
//  * give each wave of a workgroup its own K sub-range and add the waves'
//    results through LDS in wave order 0, 1, ..., then write C or the split's
//    partial slice, which the ordered split-K reduce sums afterwards.
// Tails: every load is a buffer load; positions past M, N or K (or past the
// split's K end) get an out-of-range offset and read zero; stores past M or N
// are dropped. Buffer bases sit at the tile's (or the wave's) first row, so
// every offset stays below 257 rows of A, B or C, the range the C ABI checks.
#include "sam_internal.h"

namespace sam {

namespace stream {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));

constexpr int kOOB = 0x7FFFFFF0;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, long long bytes)
{
    const int n = bytes <= 0 ? 0 : (bytes >= kOOB ? kOOB : (int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

__device__ __forceinline__ v4f mfma(float a, float b, v4f c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

}  // namespace stream

// Skinny M (M <= 16): a workgroup computes C[0..16)[n0 .. n0 + 64 NT) over
// the split's K range, in blocks of NW * KW values of K. Within a block wave w
// owns [kw, kw + KW), kw = block start + w KW; lane group q = lane / 16 owns
// the quarter starting at kq = kw + q KW / 4 and step st of the wave handles
// K value kq + st. Lane (i = lane % 16, q) holds A[i][kq .. kq + KW/4) in
// registers and loads B[kq + st][n0 + 64 t + 4 i .. + 3] for t < NT. MFMA e
// of column block t accumulates output column n0 + 64 t + 4 j + e in MFMA
// column j, with the MFMA's four K slots being the four quarters.
//
// One wave's share of a K block. rA spans A (M rows), so rows past M read
// zero; rB starts at row kw of B and ends at the split's K end, so rows past
// it read zero. Columns past N may read the next row's values: they only
// reach output columns that are never stored. TAIL (the wave that runs past
// K, the only place a K range can end inside a row of A) zeroes A values at
// or past K one by one.
template <int KQ, int PD, int NT, bool AV, bool BV, bool TAIL>
__device__ __forceinline__ void stream_m_block(stream::v4f (&acc)[NT][4], __amdgpu_buffer_rsrc_t rA, int a_off,
                                               int a_lim, __amdgpu_buffer_rsrc_t rB, int b_off, int N4)
{
    using namespace stream;
    float a[KQ];
#pragma unroll
    for (int c = 0; c < KQ / 4; ++c) {
        u4 v;
        if (AV) {
            v = __builtin_amdgcn_raw_buffer_load_b128(rA, TAIL && 4 * c >= a_lim ? kOOB : a_off + 16 * c, 0, 0);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = __builtin_amdgcn_raw_buffer_load_b32(rA, TAIL && 4 * c + e >= a_lim ? kOOB
                                                                                           : a_off + 4 * (4 * c + e), 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) a[4 * c + e] = __uint_as_float(v[e]);
    }

    // Row strides go into the vector offset: the bounds check covers the
    // vector and immediate offsets, not the scalar one. The empty asm makes
    // the block's base opaque so the per-step offsets are formed step by step
    // instead of being hoisted out of the K-block loop into 64 registers.
    asm volatile("" : "+v"(b_off));
    auto bload = [&](int st, int t) -> u4 {
        const int off = b_off + st * N4 + 256 * t;
        if (BV) return __builtin_amdgcn_raw_buffer_load_b128(rB, off, 0, 0);
        u4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = __builtin_amdgcn_raw_buffer_load_b32(rB, off + 4 * e, 0, 0);
        return v;
    };

    u4 ring[PD][NT];
#pragma unroll
    for (int st = 0; st < PD; ++st)
#pragma unroll
        for (int t = 0; t < NT; ++t) ring[st][t] = bload(st, t);
#pragma unroll
    for (int st = 0; st < KQ; ++st) {
        u4 b[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) b[t] = ring[st % PD][t];
        if (st + PD < KQ) {
#pragma unroll
            for (int t = 0; t < NT; ++t) ring[st % PD][t] = bload(st + PD, t);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[t][e] = mfma(a[st], __uint_as_float(b[t][e]), acc[t][e]);
        // Keep program order per step: without this the scheduler hoists the
        // loads of the unrolled loop and runs out of registers.
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int NW, int KW, int PD, int NT, bool AV, bool BV>
__global__ void __launch_bounds__(NW * 64)
stream_m_kernel(GemmArgs args)
{
    using namespace stream;
    constexpr int KQ = KW / 4;
    constexpr int BN = 64 * NT;
    static_assert(KW % 16 == 0 && PD >= 1 && PD <= KQ, "wave K range");
    __shared__ __attribute__((aligned(16))) float red[NW][16][BN];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, q = lane >> 4;
    const int tn = blockIdx.x % args.tiles_n, s = blockIdx.x / args.tiles_n;
    const long long M = args.M, N = args.N, K = args.K;
    const int n0 = tn * BN;
    const long long kbeg = (long long)s * args.k_chunk;
    const long long kend = K < kbeg + args.k_chunk ? K : kbeg + args.k_chunk;

    const __amdgpu_buffer_rsrc_t rA = make_rsrc(args.A, M * K * 4);
    const float* Bf = static_cast<const float*>(args.B);
    const int N4 = (int)(N * 4);

    v4f acc[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[t][e] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    for (long long kb = kbeg; kb < kend; kb += NW * KW) {
        const long long kw = kb + (long long)wave * KW;
        if (kw >= kend) continue;                      // wave-uniform
        const long long kq = kw + q * KQ;
        const int a_off = (int)((li * K + kq) * 4);
        const int a_lim = (int)(kend - kq < 0 ? 0 : (kend - kq < KQ ? kend - kq : KQ));
        const __amdgpu_buffer_rsrc_t rB = make_rsrc(Bf + kw * N, (kend - kw) * N * 4);
        const int b_off = (int)(((long long)q * KQ * N + n0 + 4 * li) * 4);
        if (kw + KW <= kend)
            stream_m_block<KQ, PD, NT, AV, BV, false>(acc, rA, a_off, a_lim, rB, b_off, N4);
        else
            stream_m_block<KQ, PD, NT, AV, BV, true>(acc, rA, a_off, a_lim, rB, b_off, N4);
    }

    // acc[t][e] element r of lane (j = li, g = q): row 4 g + r, column 64 t + 4 j + e.
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const v4f v = {acc[t][0][r], acc[t][1][r], acc[t][2][r], acc[t][3][r]};
            *reinterpret_cast<v4f*>(&red[wave][4 * q + r][64 * t + 4 * li]) = v;
        }
    __syncthreads();

    float* out = args.out + (long long)s * args.part_stride;
    const __amdgpu_buffer_rsrc_t rC = make_rsrc(out, M * N * 4);
    for (int o = tid; o < 16 * BN / 4; o += NW * 64) {
        const int row = o / (BN / 4), c4 = (o % (BN / 4)) * 4;
        v4f sum = *reinterpret_cast<const v4f*>(&red[0][row][c4]);
#pragma unroll
        for (int w = 1; w < NW; ++w) {
            const v4f x = *reinterpret_cast<const v4f*>(&red[w][row][c4]);
            sum[0] = sum[0] + x[0];
            sum[1] = sum[1] + x[1];
            sum[2] = sum[2] + x[2];
            sum[3] = sum[3] + x[3];
        }
        const long long cc = n0 + c4;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sum[e]), rC,
                                                  row < M && cc + e < N ? (int)((row * N + cc + e) * 4) : kOOB, 0, 0);
    }
}

// Skinny N (N <= 16): a workgroup computes C[m0 .. m0 + 16 MT)[0..16) over
// the split's K range, in blocks of NW * KW values of K; wave w owns
// [kw, kw + KW). Step u of a wave covers kw + 16 u .. + 15: lane
// (i = lane % 16, q = lane / 16) loads A[m0 + 16 t + i][kw + 16 u + 4 q .. + 3]
// for t < MT, and MFMA e of the step takes K value kw + 16 u + 4 q + e in
// MFMA K slot q. The B values for exactly those K sit in registers, loaded
// once per K block.
//
// One wave's share of a K block. rA starts at row m0 of A and ends with A, so
// rows past M read zero; rB starts at row kw of B and ends at the split's K
// end, so B rows past it read zero; columns of B past N may read the next
// row's values and only reach output columns that are never stored. TAIL
// (the wave that runs past K) zeroes A values at or past K one by one, since
// there the next row of A follows.
template <int NU, int PD, int MT, bool AV, bool TAIL>
__device__ __forceinline__ void stream_n_block(stream::v4f (&acc)[MT], __amdgpu_buffer_rsrc_t rA, int a_off,
                                               int K4, int a_lim, __amdgpu_buffer_rsrc_t rB, int b_off, int N4)
{
    using namespace stream;
    // Offsets in the vector operand only (the bounds check ignores the
    // scalar one); the opaque base keeps them from being hoisted.
    asm volatile("" : "+v"(b_off), "+v"(a_off));
    float b[NU][4];
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            b[u][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rB, b_off + (16 * u + e) * N4, 0, 0));

    // A[16 t + i][kw + 16 u + 4 q + e]: a_off covers row i and 4 q; a_lim is
    // the number of valid K values from kw + 4 q on.
    auto aload = [&](int u, int t) -> u4 {
        const int off = a_off + t * 16 * K4 + 64 * u;
        if (AV) return __builtin_amdgcn_raw_buffer_load_b128(rA, TAIL && 16 * u >= a_lim ? kOOB : off, 0, 0);
        u4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            v[e] = __builtin_amdgcn_raw_buffer_load_b32(rA, TAIL && 16 * u + e >= a_lim ? kOOB : off + 4 * e, 0, 0);
        return v;
    };

    u4 ring[PD][MT];
#pragma unroll
    for (int u = 0; u < PD; ++u)
#pragma unroll
        for (int t = 0; t < MT; ++t) ring[u][t] = aload(u, t);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        u4 av[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) av[t] = ring[u % PD][t];
        if (u + PD < NU) {
#pragma unroll
            for (int t = 0; t < MT; ++t) ring[u % PD][t] = aload(u + PD, t);
        }
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[t] = mfma(__uint_as_float(av[t][e]), b[u][e], acc[t]);
        __builtin_amdgcn_sched_barrier(0);      // program order per step, as above
    }
}

template <int NW, int KW, int PD, int MT, bool AV>
__global__ void __launch_bounds__(NW * 64)
stream_n_kernel(GemmArgs args)
{
    using namespace stream;
    constexpr int NU = KW / 16;
    constexpr int BM = 16 * MT;
    static_assert(KW % 16 == 0 && PD >= 1 && PD <= NU, "wave K range");
    __shared__ float red[NW][BM][17];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, q = lane >> 4;
    const int tm = blockIdx.x % args.tiles_m, s = blockIdx.x / args.tiles_m;
    const long long M = args.M, N = args.N, K = args.K;
    const long long m0 = (long long)tm * BM;
    const long long kbeg = (long long)s * args.k_chunk;
    const long long kend = K < kbeg + args.k_chunk ? K : kbeg + args.k_chunk;

    const __amdgpu_buffer_rsrc_t rA = make_rsrc(static_cast<const float*>(args.A) + m0 * K, (M - m0) * K * 4);
    const float* Bf = static_cast<const float*>(args.B);
    const int N4 = (int)(N * 4), K4 = (int)(K * 4);

    v4f acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    for (long long kb = kbeg; kb < kend; kb += NW * KW) {
        const long long kw = kb + (long long)wave * KW;
        if (kw >= kend) continue;                      // wave-uniform
        const int a_off = (int)((li * K + kw + 4 * q) * 4);
        const long long left = kend - (kw + 4 * q);
        const int a_lim = (int)(left < 0 ? 0 : (left < KW ? left : KW));
        const __amdgpu_buffer_rsrc_t rB = make_rsrc(Bf + kw * N, (kend - kw) * N * 4);
        const int b_off = (int)(((long long)4 * q * N + li) * 4);
        if (kw + KW <= kend)
            stream_n_block<NU, PD, MT, AV, false>(acc, rA, a_off, K4, a_lim, rB, b_off, N4);
        else
            stream_n_block<NU, PD, MT, AV, true>(acc, rA, a_off, K4, a_lim, rB, b_off, N4);
    }

    // acc[t] element r of lane (j = li, g = q): row 16 t + 4 g + r, column j.
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][16 * t + 4 * q + r][li] = acc[t][r];
    __syncthreads();

    float* out = args.out + (long long)s * args.part_stride + m0 * N;
    const __amdgpu_buffer_rsrc_t rC = make_rsrc(out, (M - m0) * N * 4);
    for (int o = tid; o < BM * 16; o += NW * 64) {
        const int r = o >> 4, c = o & 15;
        float sum = red[0][r][c];
#pragma unroll
        for (int w = 1; w < NW; ++w) sum = sum + red[w][r][c];
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sum), rC,
                                              m0 + r < M && c < N ? (int)((r * N + c) * 4) : kOOB, 0, 0);
    }
}

namespace {

// Streaming variants run 8 waves of KW = K block / 8 values of K each.
constexpr int kStreamWaves = 8;

using StreamKernel = void (*)(GemmArgs);

// Kernels of one K block size, indexed by a_vec (and b_vec for skinny M).
// Skinny M keeps PM rows of B in flight per lane; skinny N keeps PN steps of
// 4 row blocks of A in flight. Both are sized so that the kernel stays within
// 128 VGPRs, i.e. two 8-wave workgroups per CU.
template <int KW, int PM, int PN>
struct StreamSet {
    StreamKernel m[2][2] = {{stream_m_kernel<kStreamWaves, KW, PM, 1, false, false>,
                             stream_m_kernel<kStreamWaves, KW, PM, 1, false, true>},
                            {stream_m_kernel<kStreamWaves, KW, PM, 1, true, false>,
                             stream_m_kernel<kStreamWaves, KW, PM, 1, true, true>}};
    StreamKernel n[2] = {stream_n_kernel<kStreamWaves, KW, PN, 4, false>,
                         stream_n_kernel<kStreamWaves, KW, PN, 4, true>};
};

const StreamSet<256, 4, 1> kSet2048;
const StreamSet<128, 8, 2> kSet1024;

}  // namespace

// Kernel for a streaming plan: skinny M when the tile is 16 x 64, skinny N
// when it is 64 x 16; the K block (plan bk) is 8 waves x KW.
hipError_t launch_stream(const Plan& p, const GemmArgs& a, hipStream_t s)
{
    if (p.dtype != DT_F32 || (p.bk != 2048 && p.bk != 1024)) return hipErrorInvalidDeviceFunction;
    const int av = p.a_vec ? 1 : 0, bv = p.b_vec ? 1 : 0;
    StreamKernel k = nullptr;
    if (p.bm == 16 && p.bn == 64)
        k = p.bk == 2048 ? kSet2048.m[av][bv] : kSet1024.m[av][bv];
    else if (p.bm == 64 && p.bn == 16)
        k = p.bk == 2048 ? kSet2048.n[av] : kSet1024.n[av];
    if (!k) return hipErrorInvalidDeviceFunction;
    hipLaunchKernelGGL(k, dim3((unsigned)p.grid), dim3(kStreamWaves * 64), 0, s, a);
    return hipGetLastError();
}

}  // namespace sam
