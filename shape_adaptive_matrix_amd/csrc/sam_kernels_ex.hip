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

// dst[r][c] = c < cols ? src[r][c] : 0 for 16-bit values, c < ldd: the
// copy of an operand whose rows are not whole 16-byte pieces into rows that
// are (ldd a multiple of 8, dst 16-byte aligned), so the ring kernel can load
// it 16 bytes at a time. One thread per 16-byte piece of dst; the source is
// read one value at a time (its rows start at any 2-byte boundary).
__global__ void __launch_bounds__(256)
pad16_kernel(const unsigned short* __restrict__ src, long long lds, unsigned short* __restrict__ dst, long long ldd,
             long long rows, long long cols)
{
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    const long long per_row = ldd / 8, total = rows * per_row;
    const long long step = (long long)gridDim.x * blockDim.x;
    for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += step) {
        const long long r = e / per_row, c0 = (e - r * per_row) * 8;
        unsigned short v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = c0 + q < cols ? src[r * lds + c0 + q] : (unsigned short)0;
        const u4 w = {v[0] | ((unsigned)v[1] << 16), v[2] | ((unsigned)v[3] << 16), v[4] | ((unsigned)v[5] << 16),
                      v[6] | ((unsigned)v[7] << 16)};
        *reinterpret_cast<u4*>(dst + r * ldd + c0) = w;
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

hipError_t launch_pad16(const void* src, long long lds, void* dst, long long ldd, long long rows, long long cols,
                        hipStream_t s)
{
    const long long total = rows * (ldd / 8);
    long long blocks = (total + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(pad16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<const unsigned short*>(src),
                       lds, static_cast<unsigned short*>(dst), ldd, rows, cols);
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
