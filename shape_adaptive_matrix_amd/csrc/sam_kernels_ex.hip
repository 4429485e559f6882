// Kernels of the general entry point C = alpha op(A) op(B) + beta C:
// packing an operand into the compact row-major form the GEMM kernels take,
// and the alpha / beta pass over C. Both are HBM-bound copies.
#include "sam_internal.h"

namespace sam {

namespace {

constexpr int kPackTile = 64;

// out[r][c] (rows x cols, compact) from `in` with row stride `ld`:
// TRANS: out[r][c] = in[c][r] (in holds cols rows of at least rows values);
// otherwise out[r][c] = in[r][c]. One 64 x 64 tile per workgroup, staged
// through LDS (one padding column) so that reads and writes both run along
// contiguous rows.
template <typename T, bool TRANS>
__global__ void __launch_bounds__(256)
pack_kernel(const T* __restrict__ in, long long ld, T* __restrict__ out, long long rows, long long cols,
            long long tiles_c)
{
    __shared__ T tile[kPackTile][kPackTile + 1];
    const long long r0 = (blockIdx.x / tiles_c) * kPackTile, c0 = (blockIdx.x % tiles_c) * kPackTile;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    if (TRANS) {
#pragma unroll
        for (int i = 0; i < kPackTile / 4; ++i) {
            const long long c = c0 + ty + 4 * i, r = r0 + tx;
            if (c < cols && r < rows) tile[ty + 4 * i][tx] = in[c * ld + r];
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kPackTile / 4; ++i) {
            const long long r = r0 + ty + 4 * i, c = c0 + tx;
            if (r < rows && c < cols) out[r * cols + c] = tile[tx][ty + 4 * i];
        }
    } else {
#pragma unroll
        for (int i = 0; i < kPackTile / 4; ++i) {
            const long long r = r0 + ty + 4 * i, c = c0 + tx;
            if (r < rows && c < cols) out[r * cols + c] = in[r * ld + c];
        }
    }
}

// dst[r][c] = c < cols ? src[r][c] : 0 for c < ldd, values of ES bytes (2
// or 4): the copy of an operand whose rows are not whole 16-byte pieces into
// rows that are (ldd ES a multiple of 16, dst 16-byte aligned), so the ring
// kernels can load it 16 bytes at a time. One thread per 16-byte piece of
// dst. The source piece starts at any ES-byte boundary: the thread reads the
// two aligned 16-byte blocks around it (the second only while it starts
// inside the source; src is 16-byte aligned) and shifts the 16 bytes out of
// them.
__device__ __forceinline__ unsigned pick4(int d, unsigned a, unsigned b, unsigned c, unsigned e)
{
    return d == 0 ? a : (d == 1 ? b : (d == 2 ? c : e));
}

template <int ES>
__device__ __forceinline__ void pad_piece(const PadCopy& p, long long e)
{
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    constexpr int PER = 16 / ES;   // values per 16-byte piece
    const long long per_row = p.ldd / PER;
    const long long ext = ((p.rows - 1) * p.lds + p.cols) * ES;   // bytes of src that belong to the operand
    const char* sb = static_cast<const char*>(p.src);
    const long long r = e / per_row, c0 = (e - r * per_row) * PER;
    u4 out = {0u, 0u, 0u, 0u};
    if (c0 < p.cols) {
        const long long b = (r * p.lds + c0) * ES, a = b & ~15ll;
        const int sh = (int)(b & 15);   // a multiple of ES
        const u4 w0 = *reinterpret_cast<const u4*>(sb + a);
        const u4 w1 = a + 16 < ext ? *reinterpret_cast<const u4*>(sb + a + 16) : u4{0u, 0u, 0u, 0u};
        const unsigned W[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
        const int d = sh >> 2;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const unsigned lo = pick4(d, W[q], W[q + 1], W[q + 2], W[q + 3]);
            if constexpr (ES == 2) {
                const unsigned hi = pick4(d, W[q + 1], W[q + 2], W[q + 3], W[q + 4]);
                out[q] = (sh & 2) ? (lo >> 16) | (hi << 16) : lo;
            } else {
                out[q] = lo;
            }
        }
        if (c0 + PER > p.cols) {   // the row's last piece: values past cols are zero
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if constexpr (ES == 2) {
                    if (c0 + 2 * q >= p.cols) out[q] = 0u;
                    else if (c0 + 2 * q + 1 >= p.cols) out[q] &= 0xFFFFu;
                } else {
                    if (c0 + q >= p.cols) out[q] = 0u;
                }
            }
        }
    }
    *reinterpret_cast<u4*>(static_cast<char*>(p.dst) + (r * p.ldd + c0) * ES) = out;
}

template <int ES>
__global__ void __launch_bounds__(256) pad_kernel(PadCopy a, PadCopy b)
{
    constexpr int PER = 16 / ES;
    const long long ta = a.rows * (a.ldd / PER), total = ta + b.rows * (b.ldd / PER);
    const long long step = (long long)gridDim.x * blockDim.x;
    for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += step) {
        if (e < ta)
            pad_piece<ES>(a, e);
        else
            pad_piece<ES>(b, e - ta);
    }
}

// C[i][j] (row stride ldc) = alpha T[i][j] + beta C[i][j], evaluated as
// fmaf(alpha, t, beta * c) in FP32. T is the product with row stride ldt, or
// absent (alpha == 0 or K == 0: it counts as zero). C is read only when
// read_c (beta != 0), so values in C never leak into a beta == 0 result.
// T may be C itself (the in-place scale C = alpha C): every element is read
// and written by the same thread.
__global__ void __launch_bounds__(256)
axpby_kernel(const float* T, long long ldt, float* C, long long ldc, long long M, long long N,
             float alpha, float beta, int read_c)
{
    const long long total = M * N;
    const long long step = (long long)gridDim.x * blockDim.x;
    for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += step) {
        const long long i = e / N, j = e - i * N;
        const float t = T ? T[i * ldt + j] : 0.0f;
        const float c = read_c ? C[i * ldc + j] : 0.0f;
        C[i * ldc + j] = read_c ? __fmaf_rn(alpha, t, beta * c) : alpha * t;
    }
}

}  // namespace

hipError_t launch_pad(const PadCopy& a, const PadCopy& b, int es, hipStream_t s)
{
    if (es != 2 && es != 4) return hipErrorInvalidValue;
    const int per = 16 / es;
    const long long total = a.rows * (a.ldd / per) + b.rows * (b.ldd / per);
    long long blocks = (total + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    if (blocks < 1) blocks = 1;
    if (es == 2)
        hipLaunchKernelGGL(pad_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, s, a, b);
    else
        hipLaunchKernelGGL(pad_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, s, a, b);
    return hipGetLastError();
}

hipError_t launch_pack(const void* in, long long ld, void* out, long long rows, long long cols, int elem_bytes,
                       int trans, hipStream_t s)
{
    if (rows == 0 || cols == 0) return hipSuccess;
    const long long tr = (rows + kPackTile - 1) / kPackTile, tc = (cols + kPackTile - 1) / kPackTile;
    const dim3 grid((unsigned)(tr * tc)), block(256);
    if (elem_bytes == 4) {
        if (trans)
            hipLaunchKernelGGL((pack_kernel<unsigned, true>), grid, block, 0, s, static_cast<const unsigned*>(in), ld,
                               static_cast<unsigned*>(out), rows, cols, tc);
        else
            hipLaunchKernelGGL((pack_kernel<unsigned, false>), grid, block, 0, s, static_cast<const unsigned*>(in), ld,
                               static_cast<unsigned*>(out), rows, cols, tc);
    } else {
        if (trans)
            hipLaunchKernelGGL((pack_kernel<unsigned short, true>), grid, block, 0, s,
                               static_cast<const unsigned short*>(in), ld, static_cast<unsigned short*>(out), rows,
                               cols, tc);
        else
            hipLaunchKernelGGL((pack_kernel<unsigned short, false>), grid, block, 0, s,
                               static_cast<const unsigned short*>(in), ld, static_cast<unsigned short*>(out), rows,
                               cols, tc);
    }
    return hipGetLastError();
}

hipError_t launch_axpby(const float* T, long long ldt, float* C, long long ldc, long long M, long long N, float alpha,
                        float beta, hipStream_t s)
{
    if (M == 0 || N == 0) return hipSuccess;
    long long blocks = (M * N + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    hipLaunchKernelGGL(axpby_kernel, dim3((unsigned)blocks), dim3(256), 0, s, T, ldt, C, ldc, M, N, alpha, beta,
                       beta != 0.0f ? 1 : 0);
    return hipGetLastError();
}

}  // namespace sam
