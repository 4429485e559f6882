// Kernel table of the 16-bit 16x16x32 ring variants for operands given
// transposed, as the general entry point takes them: B as N rows of K values
// (layout 1, kernel MODE 3), A as K rows of M values (layout 2, MODE 4), or
// both (layout 3, MODE 5); data-parallel and stream-K forms. Kept apart from
// the plain table so the two compile in parallel.
#include "sam_ring16.h"
#include "sam_variants.h"

namespace sam {

namespace {

struct DmaTKernels {
    int id;
    KernelFn fn[4][2][3];   // [layout][stream-K][dtype]
};

template <int DT, int BM, int BN, int WM, int WN, int BK, int NBUF, int MODE, int BLK, int SWAP, bool SK>
constexpr KernelFn ring16_t()
{
    constexpr bool ATR = MODE == 4 || MODE == 5;   // A^T rows: BM must be whole 1 KB loads
    if constexpr (BLK == 16 && (!ATR || BM == 128 || BM == 256)) {
        if constexpr (SK)
            return gemm16_dma_sk_kernel<DT, BM, BN, WM, WN, BK, NBUF, MODE, BLK, SWAP>;
        else
            return gemm16_dma_kernel<DT, BM, BN, WM, WN, BK, NBUF, MODE, BLK, SWAP>;
    } else {
        return nullptr;
    }
}

#define SAM_DMA_T_LAYOUT(MODE, BM, BN, WM, WN, BK, NBUF, BLK, SW)                                              \
    {{nullptr, ring16_t<DT_BF16, BM, BN, WM, WN, BK, NBUF, MODE, BLK, SW, false>(),                          \
      ring16_t<DT_F16, BM, BN, WM, WN, BK, NBUF, MODE, BLK, SW, false>()},                                   \
     {nullptr, ring16_t<DT_BF16, BM, BN, WM, WN, BK, NBUF, MODE, BLK, SW, true>(),                           \
      ring16_t<DT_F16, BM, BN, WM, WN, BK, NBUF, MODE, BLK, SW, true>()}}
#define SAM_DMA_T_ENTRY(id, name, BM, BN, WM, WN, BK, NBUF, MODE, BLK, SW, gm, xr, ms, e16)                     \
    {id,                                                                                                      \
     {{{nullptr, nullptr, nullptr}, {nullptr, nullptr, nullptr}},                                            \
      SAM_DMA_T_LAYOUT(3, BM, BN, WM, WN, BK, NBUF, BLK, SW), SAM_DMA_T_LAYOUT(4, BM, BN, WM, WN, BK, NBUF, BLK, SW), \
      SAM_DMA_T_LAYOUT(5, BM, BN, WM, WN, BK, NBUF, BLK, SW)}},
#define SAM_DMA_T_ENTRY0(id, name, BM, BN, WM, WN, BK, NBUF, MODE, BLK, gm, xr, ms, e16) \
    SAM_DMA_T_ENTRY(id, name, BM, BN, WM, WN, BK, NBUF, MODE, BLK, 0, gm, xr, ms, e16)

// Only the straight-load 16x16x32 variants (MODE 0, BLK 16) have these forms.
#define SAM_DMA_T_IF16(id, name, BM, BN, WM, WN, BK, NBUF, MODE, BLK, gm, xr, ms, e16) \
    SAM_DMA_T_ENTRY0(id, name, BM, BN, WM, WN, BK, NBUF, MODE, BLK, gm, xr, ms, e16)

const DmaTKernels kDmaTTable[] = {SAM_DMA16_VARIANTS(SAM_DMA_T_IF16) SAM_DMA16S_VARIANTS(SAM_DMA_T_ENTRY)
                                      SAM_DMA16M_VARIANTS(SAM_DMA_T_ENTRY) SAM_DMA16D_VARIANTS(SAM_DMA_T_ENTRY)};

}  // namespace

KernelFn dma_t_kernel(int variant_id, int layout, bool stream_k, int dtype)
{
    if (layout < 1 || layout > 3 || dtype < 1 || dtype > 2) return nullptr;
    for (const DmaTKernels& d : kDmaTTable)
        if (d.id == variant_id) return d.fn[layout][stream_k ? 1 : 0][dtype];
    return nullptr;
}

bool dma_has_layout(int variant_id, int layout, int dtype)
{
    return dma_t_kernel(variant_id, layout, false, dtype) && dma_t_kernel(variant_id, layout, true, dtype);
}

}  // namespace sam
