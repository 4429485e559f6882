// GEMM kernels for gfx950 (CDNA4) on the matrix cores (MFMA).
//
// C = A*B, row-major A[M][K], B[K][N], C[M][N], alpha 1, beta 0 (page "Scale
// coverage exposes a remaining GEMM gap", section "Measurement contract and
// evidence"). One templated macro-tile kernel covers every variant:
//
//  * Workgroup -> tile: the linear workgroup id is first remapped so that
//    each XCD (workgroups are handed to the 8 XCDs round-robin) owns one
//    contiguous range of logical ids, then walked in grouped-raster order
//    (group_m tile rows sweep N together) so neighbouring tiles share A and B
//    panels in the same XCD's L2. The split-K index is the outermost part of
//    the logical id.
//  * Global -> LDS: both operands are stored K-contiguous in LDS, one
//    128-byte row per M (or N) index and 16-byte chunks XOR-swizzled by the
//    row, double-buffered. A rows are K-contiguous in memory already; B rows
//    are N-contiguous, so each thread loads a VExVE block of B (VE = elements
//    per 16 bytes) and transposes it in registers before the LDS write.
//    Rows and K past the tail are zero-filled (an Inf in a neighbouring row
//    must never meet a zero weight), loads past M/N are simply zero.
//  * LDS -> MFMA: each lane reads one 16-byte chunk per operand block. The K
//    index inside a stage is permuted so that one chunk holds the lane's
//    share of consecutive MFMA steps; A and B use the same permutation, so
//    the product is unchanged and the order is fixed per variant.
//  * Epilogue: accumulators go straight to C (or to the split's partial
//    slice of the workspace), masked at the M/N tails. C is never read.
// No atomics: the K order of every output is fixed, which makes repeated
// runs bitwise identical (page "Measured data point on fixed-tile vs
// shape-adaptive GEMM", question 2).
#include "sam_internal.h"
#include "sam_variants.h"

namespace sam {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));

template <int DT> struct Elem { typedef uint16_t T; static constexpr int VE = 8; };
template <> struct Elem<DT_F32> { typedef float T; static constexpr int VE = 4; };

template <int BLK> struct Acc;
template <> struct Acc<32> { typedef v16f T; static constexpr int N = 16; };
template <> struct Acc<16> { typedef v4f T; static constexpr int N = 4; };

// One MFMA on element e of a 16-byte chunk (FP32: four steps per chunk;
// 16-bit: the chunk is the whole 8-element operand). FP32 elements are taken
// with __uint_as_float: this compiler turned __builtin_bit_cast of a vector
// element into element 0 for every E.
template <int DT, int BLK> struct Mfma;
template <> struct Mfma<DT_F32, 32> {
    static constexpr int PER_CHUNK = 4;
    template <int E>
    static __device__ __forceinline__ void run(v16f& c, const u4& a, const u4& b) {
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[E]),
                                                 __uint_as_float(b[E]), c, 0, 0, 0);
    }
};
template <> struct Mfma<DT_F32, 16> {
    static constexpr int PER_CHUNK = 4;
    template <int E>
    static __device__ __forceinline__ void run(v4f& c, const u4& a, const u4& b) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[E]),
                                                 __uint_as_float(b[E]), c, 0, 0, 0);
    }
};
template <> struct Mfma<DT_BF16, 32> {
    static constexpr int PER_CHUNK = 1;
    template <int E>
    static __device__ __forceinline__ void run(v16f& c, const u4& a, const u4& b) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a),
                                                    __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
    }
};
template <> struct Mfma<DT_BF16, 16> {
    static constexpr int PER_CHUNK = 1;
    template <int E>
    static __device__ __forceinline__ void run(v4f& c, const u4& a, const u4& b) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a),
                                                    __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
    }
};
template <> struct Mfma<DT_F16, 32> {
    static constexpr int PER_CHUNK = 1;
    template <int E>
    static __device__ __forceinline__ void run(v16f& c, const u4& a, const u4& b) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a),
                                                   __builtin_bit_cast(v8h, b), c, 0, 0, 0);
    }
};
template <> struct Mfma<DT_F16, 16> {
    static constexpr int PER_CHUNK = 1;
    template <int E>
    static __device__ __forceinline__ void run(v4f& c, const u4& a, const u4& b) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a),
                                                   __builtin_bit_cast(v8h, b), c, 0, 0, 0);
    }
};

// Byte offset of 16-byte chunk `ch` of LDS row `row` (rows are 128 bytes).
// XOR swizzle: eight consecutive rows read at one logical chunk land in
// eight different 16-byte bank groups.
__device__ __forceinline__ int lds_off(int row, int ch) {
    return (row << 7) + (((ch ^ row) & 7) << 4);
}

// Output row of accumulator element r held by `lane` (MFMA result layout).
template <int BLK> __device__ __forceinline__ int acc_row(int lane, int r);
template <> __device__ __forceinline__ int acc_row<32>(int lane, int r) {
    return ((r >> 2) << 3) + ((lane >> 5) << 2) + (r & 3);
}
template <> __device__ __forceinline__ int acc_row<16>(int lane, int r) {
    return ((lane >> 4) << 2) + r;
}

__device__ __forceinline__ void tile_coords(int wg, const GemmArgs& a, int& tm, int& tn, int& s) {
    const int total = a.tiles_m * a.tiles_n * a.split;
    int L = wg;
    if (a.xcd_remap) {
        const int q = total >> 3, rem = total & 7, x = wg & 7, y = wg >> 3;
        L = (x < rem) ? x * (q + 1) + y : rem * (q + 1) + (x - rem) * q + y;
    }
    const int tiles = a.tiles_m * a.tiles_n;
    s = L / tiles;
    const int t = L - s * tiles;
    const int per_group = a.group_m * a.tiles_n;
    const int g = t / per_group;
    const int first_m = g * a.group_m;
    const int gsz = min(a.tiles_m - first_m, a.group_m);
    const int r = t - g * per_group;
    tm = first_m + r % gsz;
    tn = r / gsz;
}

// 16-bit lane select: half `h` (0 low, 1 high) of x and y -> (x_h | y_h << 16).
template <int H>
__device__ __forceinline__ unsigned pack_halves(unsigned x, unsigned y) {
    return __builtin_amdgcn_perm(y, x, H ? 0x07060302u : 0x05040100u);
}

template <int DT, int BM, int BN, int WM, int WN, int BLK, bool AV, bool BV>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_kernel(GemmArgs args)
{
    typedef typename Elem<DT>::T T;
    constexpr int VE = Elem<DT>::VE;          // elements per 16-byte chunk
    constexpr int BK = 8 * VE;                // K per stage: one 128-byte row
    constexpr int NT = WM * WN * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / BLK, TN = WTN / BLK;
    constexpr int G = 64 / BLK;               // K-slot groups per MFMA
    constexpr int CS = 8 / G;                 // chunk steps per stage
    constexpr int STAGE = (BM + BN) * 128;    // bytes per LDS stage
    constexpr int NA = (BM * 8 + NT - 1) / NT;            // A chunks per thread
    constexpr int NBT = 8 * BN / VE;                       // B VExVE blocks per stage
    constexpr int NB = (NBT + NT - 1) / NT;                // per thread
    typedef typename Acc<BLK>::T acc_t;
    static_assert(WTM % BLK == 0 && WTN % BLK == 0, "wave tile must be whole MFMA blocks");
    static_assert(2 * STAGE <= 160 * 1024, "LDS budget");

    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    int tm, tn, s;
    tile_coords(blockIdx.x, args, tm, tn, s);
    const int M = args.M, N = args.N, K = args.K;
    const int m0 = tm * BM, n0 = tn * BN;
    const int kbeg = s * args.k_chunk;
    const int kend = min(K, kbeg + args.k_chunk);
    const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
    const T* __restrict__ A = static_cast<const T*>(args.A);
    const T* __restrict__ B = static_cast<const T*>(args.B);

    const int wm0 = (wave / WN) * WTM;
    const int wn0 = (wave % WN) * WTN;

    u4 ra[NA];
    u4 rb[NB][VE];

    auto load_stage = [&](int k0) {
#pragma unroll
        for (int q = 0; q < NA; ++q) {
            const int id = tid + q * NT;
            u4 v = {0u, 0u, 0u, 0u};
            if (id < BM * 8) {
                const int gm = m0 + (id >> 3);
                const int gk = k0 + (id & 7) * VE;
                if (gm < M) {
                    const T* p = A + (long long)gm * K + gk;
                    if constexpr (AV) {
                        if (gk < kend) v = *reinterpret_cast<const u4*>(p);
                    } else {
                        T e[VE];
#pragma unroll
                        for (int i = 0; i < VE; ++i) e[i] = (gk + i < kend) ? p[i] : T(0);
                        v = __builtin_bit_cast(u4, e);
                    }
                }
            }
            ra[q] = v;
        }
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            const int id = tid + q * NT;
            const int gk = k0 + (id & 7) * VE;
            const int gn = n0 + (id >> 3) * VE;
#pragma unroll
            for (int r = 0; r < VE; ++r) {
                u4 v = {0u, 0u, 0u, 0u};
                if (id < NBT && gk + r < kend) {
                    const T* p = B + (long long)(gk + r) * N + gn;
                    if constexpr (BV) {
                        if (gn < N) v = *reinterpret_cast<const u4*>(p);
                    } else {
                        T e[VE];
#pragma unroll
                        for (int i = 0; i < VE; ++i) e[i] = (gn + i < N) ? p[i] : T(0);
                        v = __builtin_bit_cast(u4, e);
                    }
                }
                rb[q][r] = v;
            }
        }
    };

    auto store_stage = [&](unsigned char* buf) {
#pragma unroll
        for (int q = 0; q < NA; ++q) {
            const int id = tid + q * NT;
            if (id < BM * 8)
                *reinterpret_cast<u4*>(buf + lds_off(id >> 3, id & 7)) = ra[q];
        }
        unsigned char* bbuf = buf + BM * 128;
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            const int id = tid + q * NT;
            if (id >= NBT) continue;
            const int kc = id & 7;
            const int nb = (id >> 3) * VE;
            if constexpr (VE == 4) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    u4 t = {rb[q][0][c], rb[q][1][c], rb[q][2][c], rb[q][3][c]};
                    *reinterpret_cast<u4*>(bbuf + lds_off(nb + c, kc)) = t;
                }
            } else {
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    u4 t;
                    const int d = c >> 1;
                    if (c & 1) {
                        t[0] = pack_halves<1>(rb[q][0][d], rb[q][1][d]);
                        t[1] = pack_halves<1>(rb[q][2][d], rb[q][3][d]);
                        t[2] = pack_halves<1>(rb[q][4][d], rb[q][5][d]);
                        t[3] = pack_halves<1>(rb[q][6][d], rb[q][7][d]);
                    } else {
                        t[0] = pack_halves<0>(rb[q][0][d], rb[q][1][d]);
                        t[1] = pack_halves<0>(rb[q][2][d], rb[q][3][d]);
                        t[2] = pack_halves<0>(rb[q][4][d], rb[q][5][d]);
                        t[3] = pack_halves<0>(rb[q][6][d], rb[q][7][d]);
                    }
                    *reinterpret_cast<u4*>(bbuf + lds_off(nb + c, kc)) = t;
                }
            }
        }
    };

    acc_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < Acc<BLK>::N; ++r) acc[i][j][r] = 0.0f;

    const int lrow = lane % BLK;       // row (or column) inside an MFMA block
    const int lgrp = lane / BLK;       // K-slot group

    if (nk > 0) {
        load_stage(kbeg);
        store_stage(lds);
    }
    __syncthreads();

    for (int kb = 0; kb < nk; ++kb) {
        const bool more = kb + 1 < nk;
        if (more) load_stage(kbeg + (kb + 1) * BK);

        const unsigned char* abuf = lds + (kb & 1) * STAGE;
        const unsigned char* bbuf = abuf + BM * 128;
#pragma unroll
        for (int c = 0; c < CS; ++c) {
            const int ch = c * G + lgrp;
            u4 fa[TM], fb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                fa[i] = *reinterpret_cast<const u4*>(abuf + lds_off(wm0 + i * BLK + lrow, ch));
#pragma unroll
            for (int j = 0; j < TN; ++j)
                fb[j] = *reinterpret_cast<const u4*>(bbuf + lds_off(wn0 + j * BLK + lrow, ch));
            constexpr int PC = Mfma<DT, BLK>::PER_CHUNK;
            if constexpr (PC == 4) {
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) Mfma<DT, BLK>::template run<0>(acc[i][j], fa[i], fb[j]);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) Mfma<DT, BLK>::template run<1>(acc[i][j], fa[i], fb[j]);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) Mfma<DT, BLK>::template run<2>(acc[i][j], fa[i], fb[j]);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) Mfma<DT, BLK>::template run<3>(acc[i][j], fa[i], fb[j]);
            } else {
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) Mfma<DT, BLK>::template run<0>(acc[i][j], fa[i], fb[j]);
            }
        }

        if (more) store_stage(lds + ((kb + 1) & 1) * STAGE);
        __syncthreads();
    }

    float* __restrict__ out = args.out + (long long)s * args.part_stride;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = n0 + wn0 + j * BLK + lrow;
#pragma unroll
            for (int r = 0; r < Acc<BLK>::N; ++r) {
                const int row = m0 + wm0 + i * BLK + acc_row<BLK>(lane, r);
                if (row < M && col < N) out[(long long)row * N + col] = acc[i][j][r];
            }
        }
    }
}

// C = P[0] + P[1] + ... + P[S-1], added left to right for every element.
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float* __restrict__ P, int S, long long stride,
                     float* __restrict__ C, long long count)
{
    const long long step = (long long)gridDim.x * blockDim.x;
    long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if ((stride & 3) == 0 && (count & 3) == 0) {
        const long long n4 = count >> 2, s4 = stride >> 2;
        const v4f* P4 = reinterpret_cast<const v4f*>(P);
        v4f* C4 = reinterpret_cast<v4f*>(C);
        for (; i < n4; i += step) {
            v4f acc = P4[i];
            for (int s = 1; s < S; ++s) {
                const v4f x = P4[s * s4 + i];
                acc[0] = acc[0] + x[0];
                acc[1] = acc[1] + x[1];
                acc[2] = acc[2] + x[2];
                acc[3] = acc[3] + x[3];
            }
            C4[i] = acc;
        }
    } else {
        for (; i < count; i += step) {
            float acc = P[i];
            for (int s = 1; s < S; ++s) acc = acc + P[s * stride + i];
            C[i] = acc;
        }
    }
}

__global__ void __launch_bounds__(256)
zero_kernel(float* __restrict__ C, long long count)
{
    const long long step = (long long)gridDim.x * blockDim.x;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += step)
        C[i] = 0.0f;
}

// ---------------------------------------------------------------------------
// Launch table: [variant][dtype][a_vec][b_vec] -> kernel.
typedef void (*KernelFn)(GemmArgs);

template <int DT, int BM, int BN, int WM, int WN, int BLK>
struct KernelSet {
    static constexpr KernelFn fn[2][2] = {
        {gemm_kernel<DT, BM, BN, WM, WN, BLK, false, false>,
         gemm_kernel<DT, BM, BN, WM, WN, BLK, false, true>},
        {gemm_kernel<DT, BM, BN, WM, WN, BLK, true, false>,
         gemm_kernel<DT, BM, BN, WM, WN, BLK, true, true>}};
};

struct VariantKernels {
    KernelFn fn[3][2][2];
    int threads;
};

#define SAM_KERNELS_ENTRY(id, name, BM, BN, WM, WN, BLK, gm, xr, ms, e32, e16)              \
    {{{{KernelSet<DT_F32, BM, BN, WM, WN, BLK>::fn[0][0], KernelSet<DT_F32, BM, BN, WM, WN, BLK>::fn[0][1]}, \
       {KernelSet<DT_F32, BM, BN, WM, WN, BLK>::fn[1][0], KernelSet<DT_F32, BM, BN, WM, WN, BLK>::fn[1][1]}}, \
      {{KernelSet<DT_BF16, BM, BN, WM, WN, BLK>::fn[0][0], KernelSet<DT_BF16, BM, BN, WM, WN, BLK>::fn[0][1]}, \
       {KernelSet<DT_BF16, BM, BN, WM, WN, BLK>::fn[1][0], KernelSet<DT_BF16, BM, BN, WM, WN, BLK>::fn[1][1]}}, \
      {{KernelSet<DT_F16, BM, BN, WM, WN, BLK>::fn[0][0], KernelSet<DT_F16, BM, BN, WM, WN, BLK>::fn[0][1]}, \
       {KernelSet<DT_F16, BM, BN, WM, WN, BLK>::fn[1][0], KernelSet<DT_F16, BM, BN, WM, WN, BLK>::fn[1][1]}}}, \
     WM * WN * 64},

static const VariantKernels kTable[] = {SAM_VARIANT_LIST(SAM_KERNELS_ENTRY)};

hipError_t launch_gemm(const Plan& p, const GemmArgs& a, hipStream_t s)
{
    const VariantKernels& vk = kTable[p.variant_id];
    KernelFn fn = vk.fn[p.dtype][p.a_vec][p.b_vec];
    hipLaunchKernelGGL(fn, dim3((unsigned)p.grid), dim3(vk.threads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_reduce(const float* parts, int split, long long part_stride,
                         float* C, long long count, hipStream_t s)
{
    const long long work = ((part_stride & 3) == 0 && (count & 3) == 0) ? count / 4 : count;
    long long blocks = (work + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       parts, split, part_stride, C, count);
    return hipGetLastError();
}

hipError_t launch_zero(float* C, long long count, hipStream_t s)
{
    long long blocks = (count + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, C, count);
    return hipGetLastError();
}

const void* probe_kernel()
{
    return reinterpret_cast<const void*>(kTable[1].fn[DT_F32][1][1]);
}

}  // namespace sam
