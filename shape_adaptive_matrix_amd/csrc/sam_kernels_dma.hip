// Kernel table of the 16-bit ring variants for the plain layout (A M x K,
// B K x N, both row-major): data-parallel and stream-K forms, the stream-K
// fix-up, and the launchers. The kernels themselves are in sam_ring16.h.
#include "sam_ring16.h"
#include "sam_variants.h"

namespace sam {

struct DmaKernels {
    int id;
    KernelFn fn[3];
    KernelFn sk[3];      // stream-K form (16x16x32 variants only)
    KernelFn fixup;
    int fixup_wgs;
    int threads;
};

template <int DT, int BM, int BN, int WM, int WN, int BK, int NBUF, int MODE, int BLK, int SWAP>
constexpr KernelFn ring16_sk()
{
    if constexpr (MODE == 0 && BLK == 16)
        return gemm16_dma_sk_kernel<DT, BM, BN, WM, WN, BK, NBUF, MODE, BLK, SWAP>;
    else
        return nullptr;
}

#define SAM_DMA_ENTRY(id, name, BM, BN, WM, WN, BK, NBUF, MODE, BLK, SW, gm, xr, ms, e16)                  \
    {id,                                                                                               \
     {nullptr, gemm16_dma_kernel<DT_BF16, BM, BN, WM, WN, BK, NBUF, MODE, BLK, SW>,                    \
      gemm16_dma_kernel<DT_F16, BM, BN, WM, WN, BK, NBUF, MODE, BLK, SW>},                             \
     {nullptr, ring16_sk<DT_BF16, BM, BN, WM, WN, BK, NBUF, MODE, BLK, SW>(),                          \
      ring16_sk<DT_F16, BM, BN, WM, WN, BK, NBUF, MODE, BLK, SW>()},                                   \
     sk_fixup_kernel<BM, BN>, sk_fixup_wgs<BM, BN>(), WM * WN * 64},
#define SAM_DMA_ENTRY0(id, name, BM, BN, WM, WN, BK, NBUF, MODE, BLK, gm, xr, ms, e16) \
    SAM_DMA_ENTRY(id, name, BM, BN, WM, WN, BK, NBUF, MODE, BLK, 0, gm, xr, ms, e16)

static const DmaKernels kDmaTable[] = {SAM_DMA_VARIANTS(SAM_DMA_ENTRY0) SAM_DMA16_VARIANTS(SAM_DMA_ENTRY0)
                                           SAM_DMA16S_VARIANTS(SAM_DMA_ENTRY)
                                               SAM_DMA16M_VARIANTS(SAM_DMA_ENTRY) SAM_DMA16D_VARIANTS(SAM_DMA_ENTRY)};

static const DmaKernels* dma_entry(int id)
{
    for (const DmaKernels& d : kDmaTable)
        if (d.id == id) return &d;
    return nullptr;
}

hipError_t launch_gemm_dma(const Plan& p, const GemmArgs& a, hipStream_t s)
{
    const DmaKernels* d = dma_entry(p.variant_id);
    if (!d) return hipErrorInvalidDeviceFunction;
    KernelFn fn = p.tr ? dma_t_kernel(p.variant_id, p.tr, p.sk != 0, p.dtype)
                       : (p.sk ? d->sk[p.dtype] : d->fn[p.dtype]);
    if (!fn) return hipErrorInvalidDeviceFunction;
    hipLaunchKernelGGL(fn, dim3((unsigned)p.grid), dim3(d->threads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_sk_fixup_dma(const Plan& p, const GemmArgs& a, hipStream_t s)
{
    const DmaKernels* d = dma_entry(p.variant_id);
    if (!d) return hipErrorInvalidDeviceFunction;
    const long long tiles = (long long)p.tiles_m * p.tiles_n - p.sk_dp;
    hipLaunchKernelGGL(d->fixup, dim3((unsigned)(tiles * d->fixup_wgs)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace sam
