// Dispatcher: (M, N, K, dtype) -> variant, split-K and launch geometry.
//
// The point of the pages (page "Measured data point on fixed-tile vs
// shape-adaptive GEMM", section "The wall, and why we think it's
// structural"; page "Post-mortem: a GPU stack without nvcc, cuBLAS, or
// LLVM", section 2.1): one fixed tile reaches parity in one shape band and
// loses elsewhere, so the library carries several tiles/schedules and a
// selector. This selector is a pure function over a frozen table:
//
//  * Admission (page "Scale coverage exposes a remaining GEMM gap", section
//    "Why the fixed view request rejects tails": candidates are admitted only
//    within the target's local-memory limits, and a tail never silently
//    swaps in another block): a variant is admitted for a dtype when its
//    double-buffered LDS stages fit the CU's 160 KB, and a split is admitted
//    only when every split owns at least one K stage. Tails are handled
//    inside every variant, so no shape is rejected.
//  * Score = estimated time. Tiles are counted in waves of workgroups over
//    the 256 CUs (wave quantisation, the tile-count argument of page
//    "fix(fp4_gemm autotune) SM107 kernel family excluded...", section "Swap
//    microbenchmarks across M, N, and K"), each workgroup costing its MFMA
//    work at the variant's calibrated efficiency; the estimate is the larger
//    of that and the HBM / L2 transfer time, plus the split-K reduce pass.
//  * Ties go to the lowest variant id, so list order can never leak into the
//    choice through an unstable sort (the tie-break problem raised in the
//    review of that same page).
//  * Shapes that were measured offline (tune.py) take the fastest measured
//    (variant, split) from the frozen table in sam_tuned.h before the cost
//    model is consulted.
// No timing at run time: the same shape always gets the same plan.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "sam_internal.h"
#include "sam_tuned.h"
#include "sam_variants.h"

namespace sam {

#define SAM_STAGED_ROW(id, name, BM, BN, WM, WN, BLK, gm, xr, ms, e32, e16, pf32, pf16) \
    {id, name, KIND_STAGED, 7, BM, BN, WM, WN, BLK, 2, 0, gm, xr, ms, 1, 0, e32, e16},
#define SAM_DMA_ROWS(id, name, BM, BN, WM, WN, BK, NBUF, MODE, BLK, SW, gm, xr, ms, e16) \
    {id, name, KIND_DMA, (1 << DT_BF16) | (1 << DT_F16), BM, BN, WM, WN, BLK, NBUF, BK, gm, xr, ms, 0, SW, 0.0, e16},
#define SAM_DMA_ROW(id, name, BM, BN, WM, WN, BK, NBUF, MODE, BLK, gm, xr, ms, e16) \
    SAM_DMA_ROWS(id, name, BM, BN, WM, WN, BK, NBUF, MODE, BLK, 0, gm, xr, ms, e16)

#define SAM_STREAM_ROW(id, name, BM, BN, KB, ms, eff) \
    {id, name, KIND_STREAM, (1 << DT_F32), BM, BN, 1, 1, 16, 1, KB, 1, 0, ms, 1, 0, eff, 0.0},

#define SAM_F32RING_ROW(id, name, BM, BN, WM, WN, BK, NBUF, V, KS, BLK, EL, gm, xr, ms, e32) \
    {id, name, KIND_F32RING, (1 << DT_F32), BM, BN, WM, WN * KS, BLK, NBUF, BK, gm, xr, ms, EL, 0, e32, 0.0},

#define SAM_F32PAD_ROW(id, name, BM, BN, WM, WN, BK, NBUF, V, KS, BLK, EL, gm, xr, ms, e32)                   \
    {id, name, KIND_F32RING, (1 << DT_F32), BM, BN, WM, WN * KS, BLK, NBUF, BK, gm, xr, ms, 0, 0, e32, 0.0, 0.0, 0.0, \
     1},

#define SAM_MX8_ROW(id, name, BM, BN, WM, WN, BK, SD, gm, xr, ms, e8, e4) \
    {id, name, KIND_MX8, (1 << DT_MX8) | (1 << DT_MX4), BM, BN, WM, WN, 32, 2, BK, gm, xr, ms, 0, 0, 0.0, 0.0, e8, e4},

#define SAM_KQ_ROW(id, name, TB, NW, gm, xr, e32) \
    {id, name, KIND_KQ, (1 << DT_F32), 16 * TB, 16 * TB, 1, NW, 16, NW == 4 ? 4 : 2, 16, gm, xr, 1, 1, 0, e32, 0.0},

#define SAM_KP_ROW(id, name, KP, gm, xr, e32) \
    {id, name, KIND_KP, (1 << DT_F32), 128, 128, 4, 2, 16, 2, KP, gm, xr, 1, 0, 0, e32, 0.0},

static const Variant kVariants[] = {SAM_STAGED_VARIANTS(SAM_STAGED_ROW) SAM_DMA_VARIANTS(SAM_DMA_ROW)
                                        SAM_STREAM_VARIANTS(SAM_STREAM_ROW) SAM_F32RING_VARIANTS(SAM_F32RING_ROW)
                                            SAM_MX8_VARIANTS(SAM_MX8_ROW) SAM_DMA16_VARIANTS(SAM_DMA_ROW)
                                                SAM_KQ_VARIANTS(SAM_KQ_ROW) SAM_KP_VARIANTS(SAM_KP_ROW)
                                                    SAM_KQ8_VARIANTS(SAM_KQ_ROW) SAM_DMA16S_VARIANTS(SAM_DMA_ROWS)
                                                        SAM_DMA16M_VARIANTS(SAM_DMA_ROWS)
                                                            SAM_F32PAD_VARIANTS(SAM_F32PAD_ROW)
                                                                SAM_DMA16D_VARIANTS(SAM_DMA_ROWS)};

static const int kVariantCount = (int)(sizeof(kVariants) / sizeof(kVariants[0]));

int variant_count() { return kVariantCount; }

const Variant* variant_get(int id)
{
    return (id >= 0 && id < kVariantCount) ? &kVariants[id] : nullptr;
}

int swap_twin(int id)
{
    const Variant* v = variant_get(id);
    if (!v || v->swap) return -1;
    char want[96];
    snprintf(want, sizeof want, "%s_sw", v->name);
    for (int i = 0; i < kVariantCount; ++i)
        if (strcmp(kVariants[i].name, want) == 0) return i;
    return -1;
}

int tile256_twin(int id)
{
    const Variant* v = variant_get(id);
    if (!v || v->kind != KIND_DMA) return -1;
    for (int i = 0; i < kVariantCount; ++i) {
        const Variant& w = kVariants[i];
        if (w.kind == KIND_DMA && w.bm == 256 && w.bn == v->bn && w.wm == v->wm && w.wn == v->wn && w.bk == v->bk &&
            w.nbuf == v->nbuf && w.blk == v->blk && w.swap == v->swap)
            return i;
    }
    return -1;
}

int k_stage(const Variant& v, int dtype)
{
    if (v.kind == KIND_MX8 && dtype == DT_MX4) return 2 * v.bk;   // E2M1: twice the values per LDS row
    if (v.kind != KIND_STAGED) return v.bk;
    return dtype == DT_F32 ? 32 : 64;   // one 128-byte LDS row
}

static int vec_elems(int dtype) { return dtype == DT_F32 ? 4 : (dtype == DT_MX8 ? 16 : (dtype == DT_MX4 ? 32 : 8)); }

static double in_bytes(int dtype)
{
    return dtype == DT_F32 ? 4.0 : (dtype == DT_MX8 ? 1.0 : (dtype == DT_MX4 ? 0.5 : 2.0));
}

static long long cdiv(long long a, long long b) { return (a + b - 1) / b; }

static const DeviceModel kDev;

// Share of a tile kernel's operand requests that miss the XCD's L2: the
// first tiles the XCD runs at once (one workgroup per CU, 32 per XCD, taken
// in the raster order of tile_of: groups of group_m rows, or with raster_n of
// group_m columns) request their A and B panels; panels shared by several of
// them are fetched from beyond L2 once. Exact for the first wave of XCD 0,
// representative of the rest.
static double reuse_miss_frac(const Variant& v, long long tiles_m, long long tiles_n, int raster_n)
{
    const long long c = std::min<long long>(kDev.cus / kDev.xcds, tiles_m * tiles_n);
    if (c <= 0) return 1.0;
    const long long lead = raster_n ? tiles_n : tiles_m, other = raster_n ? tiles_m : tiles_n;
    const long long gm = v.group_m > 0 ? v.group_m : 1;
    // Tiles 0 .. c-1: whole groups of gm x other, then part of the next.
    long long lead_used = 0, other_used = 0;
    for (long long first = 0, left = c; left > 0 && first < lead; first += gm) {
        const long long gsz = std::min(gm, lead - first);
        const long long take = std::min(left, gsz * other);
        lead_used += std::min(gsz, take);
        other_used = std::max(other_used, cdiv(take, gsz));
        left -= take;
    }
    const double rows = (double)(raster_n ? other_used : lead_used);
    const double cols = (double)(raster_n ? lead_used : other_used);
    // A B panel is K rows of BN values (short row pieces), an A panel BM rows
    // of K values: re-fetching B costs more per byte (loads of B alone took
    // 1.2x those of A alone for the same bytes, 256 x 256 16-bit tiles), so
    // its misses are weighted by that.
    constexpr double kBWeight = 1.2;
    return (rows * v.bm + kBWeight * cols * v.bn) / ((double)c * (v.bm + v.bn));
}

// Rounds of workgroups over the CUs. A last, partial round costs less than a
// full one (its workgroups share the memory system with fewer others):
// 0.7 + 0.3 x its fill, fitted to bf16 5120^3 and 6144^3 on the 256 x 256
// 16-bit tiles (0.56 and 0.25 full).
static double wave_rounds(long long wgs)
{
    const long long full = wgs / kDev.cus, rem = wgs - full * kDev.cus;
    return (double)full + (rem > 0 ? 0.7 + 0.3 * (double)rem / kDev.cus : 0.0);
}

static double estimate_us(const Variant& v, long long M, long long N, long long K, int dtype,
                          int split, int a_vec, int b_vec, int raster_n)
{
    const int bk = k_stage(v, dtype);
    const long long nkb = cdiv(K, bk);
    const long long kc = cdiv(nkb, split) * bk;               // K per split, padded
    const long long tiles_m = cdiv(M, v.bm), tiles_n = cdiv(N, v.bn);
    const long long wgs = tiles_m * tiles_n * split;
    const double in_b = in_bytes(dtype);
    const double mb = 1e-6;                                   // bytes -> MB; GB/s = MB/ms

    if (v.kind == KIND_KP) {
        // Resident workgroups (one per CU for the 64-value panel, two for
        // 32) walk the tiles; each tile's multiplies overlap the previous
        // tile's C write, so a round of 256 tiles costs the larger of the two.
        const double peak_cu = kDev.f32_flop_per_clk_cu * kDev.clock_ghz * 1e3;
        const double t_mfma = 2.0 * v.bm * v.bn * (double)v.bk / (peak_cu * v.eff_f32);
        const double t_write = kDev.cus * v.bm * v.bn * 4.0 * mb / kDev.hbm_write_gbs * 1e3;
        const double t_fill = 2.0 * v.bm * v.bk * 4.0 * kDev.cus * mb / kDev.hbm_gbs * 1e3;
        return (double)cdiv(tiles_m * tiles_n, kDev.cus) * fmax(t_mfma, t_write) + t_fill + kDev.launch_us;
    }
    if (v.kind == KIND_STREAM) {
        // HBM-bound: the operands cross HBM once at the variant's share of the
        // read rate, scaled down while fewer than two 8-wave workgroups per CU
        // are resident to keep loads in flight; then the split-K partials.
        const double alg = in_b * (double)(M * K + K * N) + 4.0 * (double)(M * N);
        const double part = split > 1 ? 4.0 * (double)(M * N) * split : 0.0;
        const double occ = fmin(1.0, (double)wgs / (2.0 * kDev.cus));
        double t = (alg + part) * mb / (kDev.hbm_gbs * v.eff_f32 * occ) * 1e3 + kDev.launch_us;
        if (split > 1) t += (part + 4.0 * M * N) * mb / kDev.hbm_gbs * 1e3 + kDev.launch_us;
        return t;
    }

    double eff = dtype == DT_F32 ? v.eff_f32
                 : dtype == DT_MX8 ? v.eff_mx8
                 : dtype == DT_MX4 ? v.eff_mx4 : v.eff_h16;
    if (!a_vec) eff *= 0.85;
    if (!b_vec && v.kind != KIND_KQ) eff *= 0.85;   // the single-launch kernels read B per value anyway
    const double flop_clk = dtype == DT_F32 ? kDev.f32_flop_per_clk_cu
                            : dtype == DT_MX8 ? kDev.mx8_flop_per_clk_cu
                            : dtype == DT_MX4 ? kDev.mx4_flop_per_clk_cu : kDev.h16_flop_per_clk_cu;
    const double peak_cu = flop_clk * kDev.clock_ghz * 1e3;   // FLOP per microsecond
    const double t_wg = 2.0 * v.bm * v.bn * (double)kc / (peak_cu * eff);
    const double rounds = wave_rounds(wgs);
    // Every workgroup ends by writing its BM x BN FP32 tile (to C or to its
    // split's partials). Workgroups of one round finish together, so that
    // write is an HBM-bound phase of its own rather than hidden under MFMA.
    const double concurrent = (double)(wgs < kDev.cus ? wgs : kDev.cus);
    const double t_epi = concurrent * v.bm * v.bn * 4.0 * mb / kDev.hbm_write_gbs * 1e3;
    const double t_mfma = rounds * (t_wg + t_epi);

    const double alg = in_b * (double)(M * K + K * N) + 4.0 * (double)(M * N);
    const double part = split > 1 ? 4.0 * (double)(M * N) * split : 0.0;
    const double t_hbm = (alg + part) * mb / (kDev.hbm_gbs * kDev.tiled_hbm_frac) * 1e3;
    // Operand delivery: every tile reads its A and B panels; the share that
    // misses L2 (set by how the tiles running together share panels, i.e. by
    // the raster order) comes from beyond L2 at the fabric rate.
    const double tile_traffic = in_b * ((double)M * K * tiles_n + (double)K * N * tiles_m);
    const double miss = reuse_miss_frac(v, tiles_m, tiles_n, raster_n);
    const double t_deliver = tile_traffic * mb * ((1.0 - miss) / kDev.l2_gbs + miss / kDev.fabric_gbs) * 1e3;

    double t = fmax(t_mfma, fmax(t_hbm, t_deliver)) + kDev.launch_us;
    if (split > 1) t += (part + 4.0 * M * N) * mb / kDev.hbm_gbs * 1e3 + kDev.launch_us;
    return t;
}

static bool split_admissible(const Variant& v, long long K, int dtype, int split)
{
    if (split < 1) return false;
    if (split == 1) return true;
    const long long nkb = cdiv(K, k_stage(v, dtype));
    if (split > nkb) return false;
    const long long per = cdiv(nkb, split);
    return cdiv(nkb, per) == split;                           // no empty split
}

static unsigned long long align256(unsigned long long x) { return (x + 255ull) & ~255ull; }

// The 16-bit ring kernels, and the FP32 ring kernels of the padding forms,
// load whole 16-byte pieces of A and B rows. When K (A's rows) or N (B's
// rows) is not a multiple of 8 (16-bit) or 4 (FP32), that operand is first
// copied into the workspace with its row stride rounded up to such a
// multiple and zeros in the gap; the kernel reads the copy, whose K and N
// tails it masks as always. C is written in place. p->ws_bytes holds the
// plan's own workspace on entry; the copies go in front of it.
static void apply_pad(const Variant& v, long long M, long long N, long long K, Plan* p)
{
    p->pad_a = p->pad_b = 0;
    p->lda = K;
    p->ldb = N;
    p->ws_inner = 0;
    if (v.kind != KIND_DMA && !v.pad) return;
    const long long q = v.kind == KIND_DMA ? 8 : 4;          // values per 16-byte piece
    const unsigned long long es = v.kind == KIND_DMA ? 2 : 4;
    if (K % q == 0 && N % q == 0) return;
    p->pad_a = K % q != 0;
    p->pad_b = N % q != 0;
    p->lda = p->pad_a ? (K + q - 1) / q * q : K;
    p->ldb = p->pad_b ? (N + q - 1) / q * q : N;
    unsigned long long off = 0;
    if (p->pad_a) off = align256((unsigned long long)(M * p->lda) * es);
    if (p->pad_b) off = align256(off + (unsigned long long)(K * p->ldb) * es);
    p->ws_inner = off;
    p->ws_bytes += off;
    // One launch reads each copied operand once and writes its copy, 16
    // bytes at a time, at about half the streaming rate of a plain copy.
    const double mb = 1e-6;
    const double bytes_a = p->pad_a ? (double)es * (M * K + M * p->lda) : 0.0;
    const double bytes_b = p->pad_b ? (double)es * (K * N + K * p->ldb) : 0.0;
    p->est_us += (bytes_a + bytes_b) * mb / (0.5 * kDev.hbm_gbs) * 1e3 + kDev.launch_us;
}

static void fill_plan(const Variant& v, long long M, long long N, long long K, int dtype, int split,
                      int raster_n, Plan* p)
{
    const int bk = k_stage(v, dtype);
    const int ve = vec_elems(dtype);
    p->variant_id = v.id;
    p->kind = v.kind;
    p->dtype = dtype;
    p->bm = v.bm;
    p->bn = v.bn;
    p->bk = bk;
    p->wm = v.wm;
    p->wn = v.wn;
    p->blk = v.blk;
    p->split = split;
    p->k_chunk = (int)(cdiv(cdiv(K, bk), split) * bk);
    if (v.kind == KIND_KQ) {   // K per wave: NW waves (v.wn), whole trips of nbuf 16-value chunks
        const long long trip = 16ll * v.nbuf;
        p->k_chunk = (int)(cdiv(cdiv(K, trip), v.wn) * trip);
    }
    p->group_m = v.group_m;
    p->xcd_remap = v.xcd_remap;
    p->a_vec = (K % ve) == 0;
    p->b_vec = v.kind == KIND_MX8 ? p->a_vec : (N % ve) == 0;   // block-scaled B rows run along K
    p->tiles_m = (int)cdiv(M, v.bm);
    p->tiles_n = (int)cdiv(N, v.bn);
    p->grid = (long long)p->tiles_m * p->tiles_n * split;
    if (v.kind == KIND_KP) {   // resident workgroups: as many as fit the CUs' LDS, at most one per tile
        const long long per_cu = kDev.lds_bytes / (2 * 2 * v.bm * v.bk * 4);
        const long long g = kDev.cus * per_cu;
        p->grid = p->grid < g ? p->grid : g;
        p->k_chunk = (int)K;
    }
    p->ws_bytes = split > 1 ? (unsigned long long)split * (unsigned long long)(M * N) * 4ull : 0ull;
    p->raster_n = raster_n;
    p->swap = v.swap;
    p->sk = 0;
    p->sk_dp = 0;
    p->sk_g = 0;
    // Always 16-byte pieces (of a padded copy if need be).
    if (v.kind == KIND_DMA || v.pad) p->a_vec = p->b_vec = 1;
    p->c_vec = p->b_vec && N % 4 == 0;
    p->est_us = estimate_us(v, M, N, K, dtype, split, p->a_vec, p->b_vec, raster_n);
    apply_pad(v, M, N, K, p);
}

// Stream-K (split_k = -1 in the ABI).
//  * FP32 ring variants with tiles of at most 128 x 256: G = resident
//    workgroups (256 CUs x those that fit one CU's LDS) share all tiles x I
//    K-iterations, W >= G (no empty range) and at most 2 I iterations per
//    range (a range then touches at most three tiles).
//  * 16-bit ring variants with 16x16x32 blocks: whole waves of tiles (sk_dp,
//    a multiple of the resident count R) run one per workgroup, and the
//    T_sk < R tiles of the last, partial wave share their T_sk x I
//    iterations over G = min(R, W) workgroups (a range then touches at most
//    two tiles).
static int sk_wgs_per_cu(const Variant& v)
{
    const int es = v.kind == KIND_F32RING ? 4 : 2;
    const int lds = v.nbuf * (v.bm + v.bn) * v.bk * es;
    const int w = kDev.lds_bytes / lds;
    return w < 1 ? 1 : w;
}

struct SkGeom {
    long long G, I, dp;
};

static bool sk_geometry(const Variant& v, long long M, long long N, long long K, SkGeom* g)
{
    if (K == 0 || M == 0 || N == 0) return false;
    const long long tiles = cdiv(M, v.bm) * cdiv(N, v.bn);
    if (tiles >= (1ll << 31)) return false;
    if (v.kind == KIND_F32RING && (long long)v.bm * v.bn <= 128 * 256) {
        g->I = cdiv(K, v.bk);
        g->G = (long long)kDev.cus * sk_wgs_per_cu(v);
        g->dp = 0;
        const long long W = tiles * g->I;
        return W >= g->G && cdiv(W, g->G) <= 2 * g->I;
    }
    if (v.kind == KIND_DMA && v.blk == 16) {
        g->I = cdiv(K, v.bk);
        const long long R = (long long)kDev.cus * sk_wgs_per_cu(v);
        g->dp = tiles / R * R;
        const long long W = (tiles - g->dp) * g->I;
        g->G = std::min(R, W);
        return W > 0;
    }
    return false;
}

static double estimate_sk_us(const Variant& v, long long M, long long N, long long K, int dtype, const SkGeom& g,
                             int a_vec, int b_vec, int raster_n)
{
    double eff = dtype == DT_F32 ? v.eff_f32 : v.eff_h16;
    if (!a_vec) eff *= 0.85;
    if (!b_vec) eff *= 0.85;
    const double flop_clk = dtype == DT_F32 ? kDev.f32_flop_per_clk_cu : kDev.h16_flop_per_clk_cu;
    const double peak_cu = flop_clk * kDev.clock_ghz * 1e3;   // FLOP per microsecond
    const double t_iter = 2.0 * v.bm * v.bn * v.bk / (peak_cu * eff);
    const long long T = cdiv(M, v.bm) * cdiv(N, v.bn);
    const long long W = (T - g.dp) * g.I;
    const long long per_cu = sk_wgs_per_cu(v);
    const double mb = 1e-6;
    const double t_round_epi = kDev.cus * per_cu * v.bm * v.bn * 4.0 * mb / kDev.hbm_write_gbs * 1e3;
    // Whole waves of data-parallel tiles, each ending with its tile store;
    // then every range runs ceil(W / G) iterations with the CU shared by the
    // workgroups resident on it, and ends up to three (FP32) or two (16-bit)
    // segments with a tile store; the fix-up reads at most two slots per
    // range and writes C.
    const double t_dp = (double)(g.dp / (kDev.cus * per_cu)) * (g.I * t_iter * per_cu + t_round_epi);
    const double t_main = (double)cdiv(W, g.G) * t_iter * per_cu;
    const double segs = v.kind == KIND_F32RING ? 3.0 : 2.0;
    // Each segment ends with a tile store of the whole round and starts by
    // filling the LDS ring (about 5 us of load latency before its first MFMA).
    const double t_epi = segs * (t_round_epi + 5.0);
    const double fix = (2.0 * g.G * v.bm * v.bn * 4.0 + 4.0 * (double)(T - g.dp) * v.bm * v.bn) * mb / kDev.hbm_gbs * 1e3;
    // Operand delivery as for the data-parallel form.
    const double in_b = dtype == DT_F32 ? 4.0 : 2.0;
    const long long tiles_m = cdiv(M, v.bm), tiles_n = cdiv(N, v.bn);
    const double tile_traffic = in_b * ((double)M * K * tiles_n + (double)K * N * tiles_m);
    const double miss = reuse_miss_frac(v, tiles_m, tiles_n, raster_n);
    const double t_deliver = tile_traffic * mb * ((1.0 - miss) / kDev.l2_gbs + miss / kDev.fabric_gbs) * 1e3;
    return fmax(t_dp + t_main + t_epi, t_deliver) + fix + 2 * kDev.launch_us;
}

static void fill_plan_sk(const Variant& v, long long M, long long N, long long K, int dtype, const SkGeom& g,
                         int raster_n, Plan* p)
{
    fill_plan(v, M, N, K, dtype, 1, raster_n, p);
    p->sk = 1;
    p->sk_dp = (int)g.dp;
    p->sk_g = (int)g.G;
    p->grid = g.dp + g.G;
    p->ws_bytes = 2ull * (unsigned long long)g.G * (unsigned long long)(v.bm * v.bn) * 4ull;
    p->est_us = estimate_sk_us(v, M, N, K, dtype, g, p->a_vec, p->b_vec, raster_n);
    apply_pad(v, M, N, K, p);
}

static const int kSplits[] = {1, 2, 3, 4, 6, 8, 12, 16, 24, 32};

// Split-K is for filling the machine when there are fewer output tiles than
// CUs, not for smoothing wave quantisation of large grids; and its partials
// must stay a modest multiple of C.
static const unsigned long long kMaxWorkspace = 512ull << 20;

static bool split_wanted(const Plan& p)
{
    if (p.split == 1) return true;
    return (long long)p.tiles_m * p.tiles_n < kDev.cus && p.ws_bytes <= kMaxWorkspace;
}

bool plan_for_variant(int vid, long long M, long long N, long long K, int dtype, int split_req,
                      Plan* out, int raster_req)
{
    if (raster_req < -1 || raster_req > 1) return false;
    const Variant* v = variant_get(vid);
    if (!v || dtype < DT_F32 || dtype > DT_MX4 || !(v->dtype_mask & (1 << dtype))) return false;
    if (M < 0 || N < 0 || K < 0) return false;
    // Block-scaled operands come in whole blocks of 32 values of K.
    if (v->kind == KIND_MX8 && K % 32 != 0) return false;
    // The LDS-ring kernels take whole 16-byte pieces of A and B rows (of a
    // padded copy when K or N is not a multiple of 8, see apply_pad); the
    // operand-swap forms store four adjacent columns of C at once, so C's
    // rows must be whole 16-byte pieces.
    if (v->kind == KIND_DMA && v->swap && N % 4 != 0) return false;
    // FP32 ring kernels take rows that are not 16-byte pieces only in their
    // element-load form, which not every variant has, or through padded
    // copies (the padding forms, which are only for such shapes).
    if (v->kind == KIND_F32RING && (K % 4 != 0 || N % 4 != 0) && !v->elem_loads && !v->pad) return false;
    if (v->kind == KIND_F32RING && v->pad && K % 4 == 0 && N % 4 == 0) return false;
    // The single-launch small-tile kernels split K inside the workgroup only,
    // and address A's tile rows and all of B with 32-bit byte offsets.
    // Prefetches run up to 48 values of K past a wave's range (the plan's
    // K per wave may itself end up to 63 values past K).
    if (v->kind == KIND_KQ && (split_req > 1 || (long long)v->bm * (K + 128) * 4 >= 0x7FFFFFF0ll ||
                               (K + 128) * N * 4 >= 0x7FFFFFF0ll))
        return false;
    // They are for products that 128 x 128 tiles cannot spread over the
    // CUs: with enough such tiles their small tiles only re-read operands
    // (a 64 x 64 tile reads twice the bytes per FLOP of a 128 x 128 one).
    if (v->kind == KIND_KQ && split_req <= 0 && cdiv(M, 128) * cdiv(N, 128) >= kDev.cus) return false;
    // The persistent short-K kernels hold a whole K panel per tile in LDS and
    // load A and B rows as 16-byte pieces.
    if (v->kind == KIND_KP && (split_req > 1 || K > v->bk || K % 4 != 0 || N % 4 != 0)) return false;
    // The streaming kernels cover at most 16 rows (16 x 64 tile) or 16
    // columns (64 x 16 tile) of C.
    if (v->kind == KIND_STREAM && (v->bm == 16 ? M > 16 : N > 16)) return false;
    // Raster orders to consider: the requested one, or both (M-major first,
    // so it wins ties). Only tiled kernels walk tiles in raster order.
    const bool tiled = v->kind != KIND_STREAM;
    const int r_lo = raster_req >= 0 ? raster_req : 0;
    const int r_hi = raster_req >= 0 ? raster_req : (tiled ? 1 : 0);
    if (!tiled && raster_req == 1) return false;
    SkGeom g{};
    const bool sk_ok = sk_geometry(*v, M, N, K, &g);
    bool found = false;
    Plan best{};
    auto consider = [&](const Plan& p) {
        if (!found || p.est_us < best.est_us) {   // strict: ties keep the earlier candidate
            best = p;
            found = true;
        }
    };
    for (int r = r_lo; r <= r_hi; ++r) {
        if (split_req == -1) {
            if (!sk_ok) return false;
            Plan p{};
            fill_plan_sk(*v, M, N, K, dtype, g, r, &p);
            consider(p);
            continue;
        }
        if (split_req > 0) {
            if (split_req > 1 && (K == 0 || !split_admissible(*v, K, dtype, split_req))) return false;
            Plan p{};
            fill_plan(*v, M, N, K, dtype, split_req, r, &p);
            if (p.grid >= (1ll << 31)) return false;
            consider(p);
            continue;
        }
        for (int s : kSplits) {
            if (s > v->max_split) break;
            if (s > 1 && (K == 0 || !split_admissible(*v, K, dtype, s))) continue;
            Plan p{};
            fill_plan(*v, M, N, K, dtype, s, r, &p);
            if (p.grid >= (1ll << 31) || !split_wanted(p)) continue;
            consider(p);
        }
        if (sk_ok) {
            Plan p{};
            fill_plan_sk(*v, M, N, K, dtype, g, r, &p);
            consider(p);
        }
    }
    if (found) *out = best;
    return found;
}

struct TunedPlan {
    int dtype;
    long long M, N, K;
    int variant, split, raster;
};

#define SAM_TUNED_ROW(dt, M, N, K, v, s, r) {dt, M, N, K, v, s, r},
static const TunedPlan kTuned[] = {SAM_TUNED_PLANS(SAM_TUNED_ROW){-1, 0, 0, 0, 0, 0, 0}};

// Half-octave bucket of a size: round(2 log2 x). Sizes within a factor of
// about 1.19 of each other share a bucket edge-to-edge.
static int bucket_of(long long x) { return x <= 0 ? -1 : (int)lround(2.0 * log2((double)x)); }

// Distance between two shapes in log2 units, summed over M, N and K.
static double shape_distance(long long M, long long N, long long K, const TunedPlan& t)
{
    return fabs(log2((double)M / t.M)) + fabs(log2((double)N / t.N)) + fabs(log2((double)K / t.K));
}

bool plan_auto(long long M, long long N, long long K, int dtype, Plan* out)
{
    // 1. A shape measured offline: its fastest (variant, split, raster).
    for (const TunedPlan& t : kTuned) {
        if (t.dtype != dtype || t.M != M || t.N != N || t.K != K) continue;
        Plan p{};
        if (plan_for_variant(t.variant, M, N, K, dtype, t.split, &p, t.raster)) {
            p.tuned = 1;
            *out = p;
            return true;
        }
    }
    // 2. A measured shape in the same half-octave bucket in M, N and K (the
    //    nearest one, ties to the earlier table row): its variant and raster
    //    order. Its split too when the variant gives this shape the same
    //    number of tiles (and the split is admissible here); otherwise the
    //    variant's own split or stream-K choice, since how a split fills the
    //    CUs depends on the tile count. The bucketed fallback of page
    //    "fix(fp4_gemm autotune) SM107 kernel family excluded from autotune
    //    candidates and heuristics update - #4856", description item 4.
    if (M > 0 && N > 0 && K > 0) {
        const TunedPlan* near = nullptr;
        double dist = 0.0;
        for (const TunedPlan& t : kTuned) {
            if (t.dtype != dtype || bucket_of(t.M) != bucket_of(M) || bucket_of(t.N) != bucket_of(N) ||
                bucket_of(t.K) != bucket_of(K))
                continue;
            Plan probe{};
            if (!plan_for_variant(t.variant, M, N, K, dtype, 0, &probe, t.raster)) continue;
            const double d = shape_distance(M, N, K, t);
            if (!near || d < dist) {
                near = &t;
                dist = d;
            }
        }
        if (near) {
            Plan p{};
            const Variant* v = variant_get(near->variant);
            const bool same_tiles =
                cdiv(M, v->bm) * cdiv(N, v->bn) == cdiv(near->M, v->bm) * cdiv(near->N, v->bn);
            if (!same_tiles || !plan_for_variant(near->variant, M, N, K, dtype, near->split, &p, near->raster))
                plan_for_variant(near->variant, M, N, K, dtype, 0, &p, near->raster);
            p.tuned = 2;
            *out = p;
            return true;
        }
    }
    // 3. The cost model over every admissible variant.
    bool found = false;
    Plan best{};
    for (int id = 0; id < kVariantCount; ++id) {
        Plan p{};
        if (!plan_for_variant(id, M, N, K, dtype, 0, &p, -1)) continue;
        if (!found || p.est_us < best.est_us) {   // strict: ties keep the lower id
            best = p;
            found = true;
        }
    }
    if (found) *out = best;
    return found;
}

bool plan_model(long long M, long long N, long long K, int dtype, Plan* out)
{
    bool found = false;
    Plan best{};
    for (int id = 0; id < kVariantCount; ++id) {
        Plan p{};
        if (!plan_for_variant(id, M, N, K, dtype, 0, &p, -1)) continue;
        if (!found || p.est_us < best.est_us) {
            best = p;
            found = true;
        }
    }
    if (found) *out = best;
    return found;
}

void plan_name(const Plan& p, char* buf, int n)
{
    static const char* dt[] = {"f32", "bf16", "f16", "mxfp8", "mxfp4"};
    const Variant* v = variant_get(p.variant_id);
    char sp[16];
    if (p.sk)
        snprintf(sp, sizeof(sp), "sk");
    else
        snprintf(sp, sizeof(sp), "s%d", p.split);
    snprintf(buf, n, "%s_%s_%s%s%s%s%s", dt[p.dtype], v ? v->name : "?", sp, p.raster_n ? "_rn" : "",
             p.a_vec ? "" : "_ua", p.b_vec ? "" : "_ub", p.tuned == 1 ? "_tuned" : (p.tuned == 2 ? "_bucket" : ""));
}

}  // namespace sam
