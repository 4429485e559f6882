// Stream-K fix-up shared by the FP32 and 16-bit ring kernels.
//
// The stream-K tiles (those after the first sk_dp, which run one per
// workgroup) times I = sk_iters K-iterations form W iterations, shared by
// sk_grid ranges [floor(W g / G), floor(W (g + 1) / G)). A range leaves its
// first segment's share of a tile in workspace slot 2 g and its last
// segment's share in slot 2 g + 1 (BM x BN floats each) when the tile is not
// wholly inside it. This kernel, sk_fixup_wgs() workgroups per stream-K
// tile, adds a shared tile's shares in range order,
// (((share of range g0) + share of g0 + 1) + ...), and stores the sum to C
// (through the general entry point's epilogue when args.epi is set);
// tiles that lie in one range were stored by the main kernel.
#pragma once

#include "sam_dma.h"
#include "sam_internal.h"

namespace sam {

__device__ __forceinline__ long long sk_start(long long W, long long G, long long g) { return W * g / G; }

__device__ __forceinline__ long long sk_range_of(long long W, long long G, long long x) {
    long long g = x * G / W;
    while (g + 1 < G && sk_start(W, G, g + 1) <= x) ++g;
    while (g > 0 && sk_start(W, G, g) > x) --g;
    return g;
}

// Workgroups per tile in the fix-up: one float4 of the tile per thread.
template <int BM, int BN>
constexpr int sk_fixup_wgs() { return BM * BN / (256 * 4); }

template <int BM, int BN>
__global__ void __launch_bounds__(256) sk_fixup_kernel(GemmArgs args)
{
    typedef float v4f __attribute__((ext_vector_type(4)));
    constexpr int CH = sk_fixup_wgs<BM, BN>();
    const long long I = args.sk_iters, dp = args.sk_dp;
    const long long T = (long long)args.tiles_m * args.tiles_n;
    const long long W = (T - dp) * I, G = args.sk_grid, u = blockIdx.x / CH;
    const long long lo = u * I, hi = (u + 1) * I - 1;
    const long long g0 = sk_range_of(W, G, lo), g1 = sk_range_of(W, G, hi);
    if (g0 == g1) return;
    int tm, tn;
    dma::tile_of((int)(dp + u), args, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int e4 = (blockIdx.x % CH) * 256 + threadIdx.x;
    const int r = e4 / (BN / 4), c = (e4 % (BN / 4)) * 4;
    if (m0 + r >= args.M || n0 + c >= args.N) return;
    const long long first_slot = sk_start(W, G, g0) == lo ? 2 * g0 : 2 * g0 + 1;
    v4f sum = reinterpret_cast<const v4f*>(args.ws + first_slot * (BM * BN))[e4];
#pragma unroll 4
    for (long long g = g0 + 1; g <= g1; ++g) {
        if (sk_start(W, G, g) == sk_start(W, G, g + 1)) continue;   // empty range
        const v4f x = reinterpret_cast<const v4f*>(args.ws + 2 * g * (BM * BN))[e4];
        sum[0] = sum[0] + x[0];
        sum[1] = sum[1] + x[1];
        sum[2] = sum[2] + x[2];
        sum[3] = sum[3] + x[3];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
        if (n0 + c + q < args.N) {
            // args.ct: the product is stored transposed, (row, col) at C[col][row].
            float* cp = args.ct ? args.out + (long long)(n0 + c + q) * args.ldc + (m0 + r)
                                : args.out + (long long)(m0 + r) * args.ldc + n0 + c + q;
            *cp = args.epi ? dma::epi_value(sum[q], args.beta != 0.0f ? *cp : 0.0f, args) : sum[q];
        }
}

}  // namespace sam
