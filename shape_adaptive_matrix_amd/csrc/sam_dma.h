// Device helpers shared by the kernels that load LDS straight from memory.
#pragma once

#include "sam_internal.h"

namespace sam {
namespace dma {

typedef int i4 __attribute__((ext_vector_type(4)));

constexpr int kOOB = 0x7FFFFFF0;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, long long bytes) {
    const int n = bytes <= 0 ? 0 : (bytes >= kOOB ? kOOB : (int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// The same raw buffer resource as four dwords (base, stride 0, record count
// in bytes, default format word) for the LDS load below.
__device__ __forceinline__ i4 rsrc_words(const void* base, long long bytes) {
    const int n = bytes <= 0 ? 0 : (bytes >= kOOB ? kOOB : (int)bytes);
    const unsigned long long a = reinterpret_cast<unsigned long long>(base);
    return i4{(int)(unsigned)a, (int)((unsigned)(a >> 32) & 0xFFFFu), n, 0x00020000};
}

// 16 bytes per lane from buffer offset `voff` into LDS at (wave-uniform)
// `lds_base` + 16 * lane; offsets past the record count store zeros. Written
// as inline assembly so that the compiler does not treat every later LDS
// read as dependent on it (it would otherwise wait for all outstanding loads
// before them); the kernels count these loads themselves with wait_cnt.
__device__ __forceinline__ void lds_load16(const i4& rsrc, unsigned lds_base, int voff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}

// The same with 4 bytes per lane: LDS at `lds_base` + 4 * lane.
__device__ __forceinline__ void lds_load4(const i4& rsrc, unsigned lds_base, int voff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}

__device__ __forceinline__ unsigned lds_addr(const void* p) {
    return (unsigned)(size_t)(__attribute__((address_space(3))) const void*)p;
}

// s_waitcnt with vmcnt <= VM and lgkmcnt <= LG (expcnt untouched).
template <int VM, int LG>
__device__ __forceinline__ void wait_cnt() {
    static_assert(VM >= 0 && VM < 64 && LG >= 0 && LG < 16, "counter range");
    __builtin_amdgcn_s_waitcnt((VM & 0xF) | (0x7 << 4) | (LG << 8) | ((VM >> 4) << 14));
}

// Workgroup barrier without the memory fence __syncthreads adds (that fence
// would drain every outstanding LDS load); the asm statements keep the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Logical index of workgroup `wg` of `total`: workgroups go to the 8 XCDs
// round-robin, and with `remap` each XCD owns one contiguous range of
// logical indices, so work with neighbouring indices shares an XCD's L2.
__device__ __forceinline__ int logical_wg(int wg, int total, int remap) {
    if (!remap) return wg;
    const int q = total >> 3, rem = total & 7, x = wg & 7, y = wg >> 3;
    return (x < rem) ? x * (q + 1) + y : rem * (q + 1) + (x - rem) * q + y;
}

// Tile index -> (tile row, tile column) in grouped-raster order. M-major
// (raster_n = 0): group_m tile rows sweep the tile columns together, the
// rows of a group taking consecutive indices. N-major (raster_n = 1): the
// same with rows and columns exchanged, group_m tile columns sweeping the
// rows (the raster-order choice of page "fix(fp4_gemm autotune) SM107 kernel
// family excluded from autotune candidates and heuristics update - #4856",
// section "Swap × raster experiment: tile reuse root cause").
__device__ __forceinline__ void tile_of(int t, const GemmArgs& a, int& tm, int& tn) {
    const int lead = a.raster_n ? a.tiles_n : a.tiles_m;    // the grouped dimension
    const int other = a.raster_n ? a.tiles_m : a.tiles_n;
    const int per_group = a.group_m * other;
    const int grp = t / per_group;
    const int first = grp * a.group_m;
    const int gsz = min(lead - first, a.group_m);
    const int r = t - grp * per_group;
    const int x = first + r % gsz, y = r / gsz;
    tm = a.raster_n ? y : x;
    tn = a.raster_n ? x : y;
}

// Workgroup id -> (tile row, tile column, split); the split index is the
// outermost part of the logical id.
__device__ __forceinline__ void tile_coords(int wg, const GemmArgs& a, int& tm, int& tn, int& s) {
    const int total = a.tiles_m * a.tiles_n * a.split;
    const int L = logical_wg(wg, total, a.xcd_remap);
    const int tiles = a.tiles_m * a.tiles_n;
    s = L / tiles;
    tile_of(L - s * tiles, a, tm, tn);
}

// Stores of C with the general entry point's epilogue. With gen, each
// product value t becomes alpha t + beta c, evaluated as fmaf(alpha, t,
// beta c) in FP32 with c the value C holds at that place, read first and only
// when beta != 0 (so values in C never reach a beta == 0 result); without
// gen, t is stored as it is. An out-of-range offset reads zero and drops the
// store, as for the plain stores.
__device__ __forceinline__ float epi_value(float t, float c, const GemmArgs& a) {
    return a.beta != 0.0f ? __fmaf_rn(a.alpha, t, a.beta * c) : a.alpha * t;
}

template <int W>
struct StoreC;

template <>
struct StoreC<4> {
    typedef unsigned int V __attribute__((ext_vector_type(4)));
    static __device__ __forceinline__ void run(V v, __amdgpu_buffer_rsrc_t rC, int off, const GemmArgs& a, bool gen) {
        if (gen) {
            V c = {0u, 0u, 0u, 0u};
            if (a.beta != 0.0f) c = __builtin_amdgcn_raw_buffer_load_b128(rC, off, 0, 0);
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = __float_as_uint(epi_value(__uint_as_float(v[q]), __uint_as_float(c[q]), a));
        }
        __builtin_amdgcn_raw_buffer_store_b128(v, rC, off, 0, 0);
    }
};

template <>
struct StoreC<2> {
    typedef unsigned int V __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ void run(V v, __amdgpu_buffer_rsrc_t rC, int off, const GemmArgs& a, bool gen) {
        if (gen) {
            V c = {0u, 0u};
            if (a.beta != 0.0f) c = __builtin_amdgcn_raw_buffer_load_b64(rC, off, 0, 0);
#pragma unroll
            for (int q = 0; q < 2; ++q) v[q] = __float_as_uint(epi_value(__uint_as_float(v[q]), __uint_as_float(c[q]), a));
        }
        __builtin_amdgcn_raw_buffer_store_b64(v, rC, off, 0, 0);
    }
};

template <>
struct StoreC<1> {
    typedef unsigned int V;
    static __device__ __forceinline__ void run(V v, __amdgpu_buffer_rsrc_t rC, int off, const GemmArgs& a, bool gen) {
        if (gen) {
            const V c = a.beta != 0.0f ? __builtin_amdgcn_raw_buffer_load_b32(rC, off, 0, 0) : 0u;
            v = __float_as_uint(epi_value(__uint_as_float(v), __uint_as_float(c), a));
        }
        __builtin_amdgcn_raw_buffer_store_b32(v, rC, off, 0, 0);
    }
};

}  // namespace dma
}  // namespace sam
