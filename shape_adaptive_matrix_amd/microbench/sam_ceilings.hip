// sam_ceilings: measured ceilings of one MI355X (gfx950) next to the spec
// peaks the GEMM is reported against.
//
//  * MFMA loop: every wave of 4 x 256 CUs x `occ` workgroups issues long
//    runs of independent MFMAs of one shape (8 accumulators, no memory
//    traffic); FLOP/s = waves x iterations x 8 x FLOPs per MFMA / time.
//  * HBM: a 16-byte-per-lane streaming copy and a streaming read-reduce over
//    buffers far larger than the 256 MB Infinity Cache.
//  * Operand delivery into a CU: one workgroup of 8 waves per CU streams
//    32 KB blocks of a source region into a ring of D LDS buffers with the
//    direct-to-LDS buffer loads the GEMM kernels use (D - 1 blocks in
//    flight, a barrier per block, no arithmetic), and, for comparison, into
//    registers with ordinary 16-byte buffer loads (16 KB in flight per
//    wave). Regions of 2 MB (resident in each XCD's 4 MB L2), 64 MB (beyond
//    L2, inside the Infinity Cache) and 1 GB. Reported as GB/s over the chip
//    and bytes per clock per CU at the reported clock.
// Prints one JSON object. Timing uses HIP events on one stream.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));

#include "../csrc/sam_dma.h"

#define CHECK(x)                                                                      \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));           \
            exit(1);                                                                  \
        }                                                                             \
    } while (0)

// Eight independent accumulators per wave, each with its own start value and
// its own A operand, so the compiler keeps them in fixed registers (with
// identical ones it rotated registers between iterations and chained every
// MFMA on the previous one). The empty asm per iteration keeps the loop from
// being collapsed.
template <int KIND>
__global__ void __launch_bounds__(256) mfma_loop(float* out, int iters, float seed)
{
    const float x = seed + threadIdx.x;
    u4 av[8];
    for (int i = 0; i < 8; ++i)
        av[i] = u4{__float_as_uint(x + i), __float_as_uint(x + 2 * i), __float_as_uint(x - i), __float_as_uint(x * i)};
    const u4 bv = {__float_as_uint(x), __float_as_uint(x + 1), __float_as_uint(x + 2), __float_as_uint(x + 3)};
    // KIND 5 / 6: the block-scaled 32x32x64 MFMA with E4M3 / E2M1 operands and
    // per-lane scales in registers.
    const int sc = 120 + (threadIdx.x & 7);
    if constexpr (KIND == 0 || KIND == 2 || KIND == 3 || KIND == 5 || KIND == 6) {   // 32x32 blocks: 16 acc regs
        v16f acc[8];
        for (int i = 0; i < 8; ++i) for (int r = 0; r < 16; ++r) acc[i][r] = (float)(i * 16 + r);
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if constexpr (KIND == 0)
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(av[i][0]), x, acc[i], 0, 0, 0);
                else if constexpr (KIND == 2)
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, av[i]), __builtin_bit_cast(v8bf, bv), acc[i], 0, 0, 0);
                else if constexpr (KIND == 3)
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, av[i]), __builtin_bit_cast(v8h, bv), acc[i], 0, 0, 0);
                else
                    acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        __builtin_bit_cast(v8i, __builtin_shufflevector(av[i], bv, 0, 1, 2, 3, 4, 5, 6, 7)),
                        __builtin_bit_cast(v8i, __builtin_shufflevector(bv, av[i], 0, 1, 2, 3, 4, 5, 6, 7)), acc[i],
                        KIND == 6 ? 4 : 0, KIND == 6 ? 4 : 0, 0, sc, 0, sc + 1);
            }
            asm volatile("" ::: "memory");
        }
        float s = 0.0f;
        for (int i = 0; i < 8; ++i) for (int r = 0; r < 16; ++r) s += acc[i][r];
        out[blockIdx.x * blockDim.x + threadIdx.x] = s;
    } else {                                                // 16x16 blocks: 4 acc regs
        v4f acc[8];
        for (int i = 0; i < 8; ++i) for (int r = 0; r < 4; ++r) acc[i][r] = (float)(i * 4 + r);
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if constexpr (KIND == 1)
                    acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(av[i][0]), x, acc[i], 0, 0, 0);
                else
                    acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, av[i]), __builtin_bit_cast(v8bf, bv), acc[i], 0, 0, 0);
            }
            asm volatile("" ::: "memory");
        }
        float s = 0.0f;
        for (int i = 0; i < 8; ++i) for (int r = 0; r < 4; ++r) s += acc[i][r];
        out[blockIdx.x * blockDim.x + threadIdx.x] = s;
    }
}

__global__ void __launch_bounds__(256) copy16(const u4* __restrict__ src, u4* __restrict__ dst, long long n)
{
    const long long step = (long long)gridDim.x * blockDim.x;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += step) dst[i] = src[i];
}

__global__ void __launch_bounds__(256) read16(const u4* __restrict__ src, unsigned* __restrict__ out, long long n)
{
    const long long step = (long long)gridDim.x * blockDim.x;
    unsigned acc = 0;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += step) {
        const u4 v = src[i];
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    if (acc == 0x9E3779B9u) out[0] = acc;   // practically never true; keeps the loads alive
}

// D-deep LDS ring of 32 KB blocks; block b of workgroup g is source block
// (7 g + b) mod (region / 32 KB). Every offset is inside the region.
template <int D>
__global__ void __launch_bounds__(512) lds_stream(const char* src, int region_bytes, int iters, unsigned* sink)
{
    __shared__ __attribute__((aligned(1024))) unsigned char lds[D * 32768];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const sam::dma::i4 r0 = sam::dma::rsrc_words(src, region_bytes);
    // Wave-uniform by construction; said explicitly so that the resource
    // stays in scalar registers, as the load instruction requires.
    const sam::dma::i4 r = {__builtin_amdgcn_readfirstlane(r0[0]), __builtin_amdgcn_readfirstlane(r0[1]),
                            __builtin_amdgcn_readfirstlane(r0[2]), __builtin_amdgcn_readfirstlane(r0[3])};
    const int blocks = region_bytes / 32768;
    auto issue = [&](int b) {
        const int blk = (int)(((long long)blockIdx.x * 7 + b) % blocks);
        unsigned char* buf = lds + (b % D) * 32768;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int I = wave + q * 8;   // 1 KB piece of the block
            sam::dma::lds_load16(r, sam::dma::lds_addr(buf + I * 1024), blk * 32768 + I * 1024 + lane * 16);
        }
    };
#pragma unroll
    for (int b = 0; b < D - 1; ++b) issue(b);
    for (int it = 0; it < iters; ++it) {
        issue(it + D - 1);   // its slot held block it - 1, released by the last barrier
        sam::dma::wait_cnt<(D - 1) * 4, 15>();   // block `it` has landed
        sam::dma::barrier();
    }
    sam::dma::wait_cnt<0, 0>();
    if (lds[threadIdx.x] == 0xAB && lds[threadIdx.x + 512] == 0xCD) sink[0] = 1;   // keeps the loads live
}

// The same blocks into registers: 16 loads of 16 bytes per lane in flight.
__global__ void __launch_bounds__(512) vgpr_stream(const char* src, int region_bytes, int iters, unsigned* sink)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const __amdgpu_buffer_rsrc_t r = sam::dma::make_rsrc(src, region_bytes);
    const int blocks = region_bytes / 32768;
    unsigned acc = 0;
    for (int it = 0; it < iters; it += 4) {
        u4 v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {   // blocks it .. it + 3, 4 pieces each
            const int blk = (int)(((long long)blockIdx.x * 7 + it + u / 4) % blocks);
            const int I = wave + (u % 4) * 8;
            v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, blk * 32768 + I * 1024 + lane * 16, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

// LDS read rate of one CU: one workgroup of 8 waves per CU (the 96 KB array
// keeps a second one off the CU), every lane issuing 16 independent reads per
// iteration; read j of wave w covers the contiguous 64 x BYTES bytes at
// ((16 w + j) x 64 x BYTES) mod 64 KB, so every address is inside the array
// and the lanes of one read hit consecutive banks. KIND 0: 128-bit reads,
// 1: 64-bit reads, 2: the transposing 64-bit read of 16-bit values. The
// shader clock counter and the constant 100 MHz counter bracket the loop, so
// the rate comes out per clock of the clock the CU actually ran at.
template <int KIND>
__global__ void __launch_bounds__(512) lds_read_rate(int iters, unsigned* sink, unsigned long long* ticks)
{
    __shared__ __attribute__((aligned(1024))) unsigned char lds[96 * 1024];
    for (int i = threadIdx.x; i < 65536 / 4; i += 512) reinterpret_cast<unsigned*>(lds)[i] = i * 2654435761u;
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr int BYTES = KIND == 0 ? 16 : 8;
    unsigned acc = 0;
    const unsigned long long c0 = clock64(), r0 = wall_clock64();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int off = (((wave * 16 + j) * 64 * BYTES) & 65535) + lane * BYTES;
            if constexpr (KIND == 0) {
                const u4 v = *reinterpret_cast<const u4*>(lds + off);
                acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
            } else if constexpr (KIND == 1) {
                const unsigned long long v = *reinterpret_cast<const unsigned long long*>(lds + off);
                acc ^= (unsigned)v ^ (unsigned)(v >> 32);
            } else {
                typedef short v4s __attribute__((ext_vector_type(4)));
                const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4s*)(lds + off));
                acc ^= (unsigned)(unsigned short)v[0] ^ ((unsigned)(unsigned short)v[1] << 16) ^
                       (unsigned)(unsigned short)v[2] ^ ((unsigned)(unsigned short)v[3] << 16);
            }
        }
        asm volatile("" ::: "memory");   // the reads stay inside the loop
    }
    __syncthreads();
    const unsigned long long c1 = clock64(), r1 = wall_clock64();
    if (threadIdx.x == 0) {
        ticks[2 * blockIdx.x] = c1 - c0;
        ticks[2 * blockIdx.x + 1] = r1 - r0;
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

// Which SIMD each wave of a 512-thread workgroup runs on: the SIMD field of
// the HW_ID hardware register (bits 5:4 on gfx9-family parts), one entry per
// wave of every workgroup.
__global__ void __launch_bounds__(512) wave_simd(int* out)
{
    const unsigned hw = __builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 4);
    if ((threadIdx.x & 63) == 0) out[blockIdx.x * 8 + (threadIdx.x >> 6)] = (int)((hw >> 4) & 3);
}

static float time_ms(hipEvent_t a, hipEvent_t b) {
    float ms = 0;
    CHECK(hipEventElapsedTime(&ms, a, b));
    return ms;
}

int main(int argc, char** argv)
{
    const int cus_arg = argc > 1 ? atoi(argv[1]) : 0;
    hipDeviceProp_t prop;
    CHECK(hipGetDeviceProperties(&prop, 0));
    const int cus = cus_arg > 0 ? cus_arg : prop.multiProcessorCount;
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    float* out;
    const int wgs = cus * 2;           // 2 workgroups of 4 waves per CU: 2 waves per SIMD
    CHECK(hipMalloc(&out, (size_t)wgs * 256 * sizeof(float)));

    struct { int kind; const char* name; double flops; } kinds[] = {
        {0, "f32_32x32x2", 32.0 * 32 * 2 * 2}, {1, "f32_16x16x4", 16.0 * 16 * 4 * 2},
        {2, "bf16_32x32x16", 32.0 * 32 * 16 * 2}, {3, "f16_32x32x16", 32.0 * 32 * 16 * 2},
        {4, "bf16_16x16x32", 16.0 * 16 * 32 * 2}, {5, "mxfp8_32x32x64", 32.0 * 32 * 64 * 2},
        {6, "mxfp4_32x32x64", 32.0 * 32 * 64 * 2}};
    printf("{\"device\": \"%s\", \"cus\": %d, \"clock_khz\": %d, \"mfma\": {", prop.gcnArchName, cus, prop.clockRate);
    for (int k = 0; k < 7; ++k) {
        const int iters = kinds[k].kind <= 1 ? 2000 : 8000;
        for (int rep = 0; rep < 2; ++rep) {   // first pass warms the clocks
            CHECK(hipEventRecord(e0, 0));
            switch (kinds[k].kind) {
            case 0: hipLaunchKernelGGL(mfma_loop<0>, dim3(wgs), dim3(256), 0, 0, out, iters, 1.0f); break;
            case 1: hipLaunchKernelGGL(mfma_loop<1>, dim3(wgs), dim3(256), 0, 0, out, iters, 1.0f); break;
            case 2: hipLaunchKernelGGL(mfma_loop<2>, dim3(wgs), dim3(256), 0, 0, out, iters, 1.0f); break;
            case 3: hipLaunchKernelGGL(mfma_loop<3>, dim3(wgs), dim3(256), 0, 0, out, iters, 1.0f); break;
            case 4: hipLaunchKernelGGL(mfma_loop<4>, dim3(wgs), dim3(256), 0, 0, out, iters, 1.0f); break;
            case 5: hipLaunchKernelGGL(mfma_loop<5>, dim3(wgs), dim3(256), 0, 0, out, iters, 1.0f); break;
            default: hipLaunchKernelGGL(mfma_loop<6>, dim3(wgs), dim3(256), 0, 0, out, iters, 1.0f); break;
            }
            CHECK(hipGetLastError());
            CHECK(hipEventRecord(e1, 0));
            CHECK(hipEventSynchronize(e1));
            if (rep == 1) {
                const double ms = time_ms(e0, e1);
                const double tf = (double)wgs * 4 * iters * 8 * kinds[k].flops / (ms * 1e-3) / 1e12;
                printf("%s\"%s\": {\"tflops\": %.1f, \"ms\": %.3f}", k ? ", " : "", kinds[k].name, tf, ms);
            }
        }
    }
    printf("}, ");

    const long long bytes = 2ll << 30;   // 2 GiB each way
    const long long n16 = bytes / 16;
    u4 *src, *dst;
    unsigned* sink;
    CHECK(hipMalloc(&src, bytes));
    CHECK(hipMalloc(&dst, bytes));
    CHECK(hipMalloc(&sink, 64));
    CHECK(hipMemset(src, 1, bytes));
    const int grid = cus * 8;
    float best_copy = 1e30f, best_read = 1e30f;
    for (int rep = 0; rep < 6; ++rep) {
        CHECK(hipEventRecord(e0, 0));
        hipLaunchKernelGGL(copy16, dim3(grid), dim3(256), 0, 0, src, dst, n16);
        CHECK(hipEventRecord(e1, 0));
        CHECK(hipEventSynchronize(e1));
        if (rep) best_copy = fminf(best_copy, time_ms(e0, e1));
        CHECK(hipEventRecord(e0, 0));
        hipLaunchKernelGGL(read16, dim3(grid), dim3(256), 0, 0, src, sink, n16);
        CHECK(hipEventRecord(e1, 0));
        CHECK(hipEventSynchronize(e1));
        if (rep) best_read = fminf(best_read, time_ms(e0, e1));
    }
    printf("\"hbm\": {\"copy_gbs\": %.1f, \"read_gbs\": %.1f, \"bytes_each_way\": %lld}, ",
           2.0 * bytes / (best_copy * 1e-3) / 1e9, bytes / (best_read * 1e-3) / 1e9, bytes);
    // Operand delivery: 32 KB blocks into LDS (ring depth D) or registers.
    {
        const double clk_ghz = prop.clockRate * 1e-6;
        const int regions[3] = {2 << 20, 64 << 20, 1 << 30};
        const char* rnames[3] = {"l2_2MB", "mall_64MB", "hbm_1GB"};
        printf("\"delivery\": {");
        for (int ri = 0; ri < 3; ++ri) {
            const int rb = regions[ri];
            const int iters = 512;
            printf("%s\"%s\": {", ri ? ", " : "", rnames[ri]);
            for (int kind = 0; kind < 4; ++kind) {
                float best = 1e30f;
                for (int rep = 0; rep < 4; ++rep) {
                    CHECK(hipEventRecord(e0, 0));
                    switch (kind) {
                    case 0: hipLaunchKernelGGL(lds_stream<2>, dim3(cus), dim3(512), 0, 0, (const char*)src, rb, iters, sink); break;
                    case 1: hipLaunchKernelGGL(lds_stream<3>, dim3(cus), dim3(512), 0, 0, (const char*)src, rb, iters, sink); break;
                    case 2: hipLaunchKernelGGL(lds_stream<4>, dim3(cus), dim3(512), 0, 0, (const char*)src, rb, iters, sink); break;
                    default: hipLaunchKernelGGL(vgpr_stream, dim3(cus), dim3(512), 0, 0, (const char*)src, rb, iters, sink); break;
                    }
                    CHECK(hipGetLastError());
                    CHECK(hipEventRecord(e1, 0));
                    CHECK(hipEventSynchronize(e1));
                    if (rep) best = fminf(best, time_ms(e0, e1));
                }
                const double bytes = (double)cus * iters * 32768.0;
                const double gbs = bytes / (best * 1e-3) / 1e9;
                const char* kn[4] = {"lds_ring2", "lds_ring3", "lds_ring4", "vgpr_16"};
                printf("%s\"%s\": {\"gbs\": %.1f, \"bytes_per_clk_cu\": %.1f}", kind ? ", " : "", kn[kind], gbs,
                       gbs / cus / clk_ghz);
            }
            printf("}");
        }
        printf("}, ");
    }
    // LDS read rate per CU, bytes per shader clock (mean over CUs).
    {
        unsigned long long* ticks;
        CHECK(hipMalloc(&ticks, (size_t)cus * 2 * sizeof(unsigned long long)));
        const int iters = 4096;
        const char* kn[3] = {"ds_read_b128", "ds_read_b64", "ds_read_b64_tr_b16"};
        const int bytes_per_lane[3] = {16, 8, 8};
        printf("\"lds_read\": {");
        for (int kind = 0; kind < 3; ++kind) {
            double bpc = 0, ghz = 0;
            for (int rep = 0; rep < 3; ++rep) {
                switch (kind) {
                case 0: hipLaunchKernelGGL(lds_read_rate<0>, dim3(cus), dim3(512), 0, 0, iters, sink, ticks); break;
                case 1: hipLaunchKernelGGL(lds_read_rate<1>, dim3(cus), dim3(512), 0, 0, iters, sink, ticks); break;
                default: hipLaunchKernelGGL(lds_read_rate<2>, dim3(cus), dim3(512), 0, 0, iters, sink, ticks); break;
                }
                CHECK(hipGetLastError());
                CHECK(hipDeviceSynchronize());
            }
            unsigned long long* h = (unsigned long long*)malloc((size_t)cus * 2 * sizeof(unsigned long long));
            CHECK(hipMemcpy(h, ticks, (size_t)cus * 2 * sizeof(unsigned long long), hipMemcpyDeviceToHost));
            const double per_cu = 8.0 * iters * 16 * 64 * bytes_per_lane[kind];
            for (int c = 0; c < cus; ++c) {
                bpc += per_cu / (double)h[2 * c];
                ghz += (double)h[2 * c] / (double)h[2 * c + 1] * 0.1;   // wall clock counter runs at 100 MHz
            }
            free(h);
            printf("%s\"%s\": {\"bytes_per_clk_cu\": %.1f, \"clock_ghz\": %.3f}", kind ? ", " : "", kn[kind],
                   bpc / cus, ghz / cus);
        }
        printf("}, ");
        CHECK(hipFree(ticks));
    }
    // SIMD of each wave: how often wave w of a workgroup sits on SIMD w % 4.
    {
        int* d;
        CHECK(hipMalloc(&d, (size_t)cus * 8 * sizeof(int)));
        hipLaunchKernelGGL(wave_simd, dim3(cus), dim3(512), 0, 0, d);
        CHECK(hipGetLastError());
        int* h = (int*)malloc((size_t)cus * 8 * sizeof(int));
        CHECK(hipMemcpy(h, d, (size_t)cus * 8 * sizeof(int), hipMemcpyDeviceToHost));
        int match = 0, pair_split = 0;
        for (int b = 0; b < cus; ++b) {
            for (int w = 0; w < 8; ++w) match += h[b * 8 + w] == w % 4;
            int ok = 1;   // waves w and w + 4 on one SIMD, the four SIMDs all used
            for (int w = 0; w < 4; ++w) ok &= h[b * 8 + w] == h[b * 8 + w + 4];
            pair_split += ok;
        }
        printf("\"wave_simd\": {\"block0\": [%d, %d, %d, %d, %d, %d, %d, %d], \"waves_on_simd_w_mod_4\": %d, "
               "\"blocks_with_w_and_w_plus_4_together\": %d, \"blocks\": %d}}\n",
               h[0], h[1], h[2], h[3], h[4], h[5], h[6], h[7], match, pair_split, cus);
        free(h);
        CHECK(hipFree(d));
    }
    CHECK(hipFree(src));
    CHECK(hipFree(dst));
    CHECK(hipFree(sink));
    CHECK(hipFree(out));
    return 0;
}
