// The C ABI (declared in include/sam.h): argument checks, the device check,
// plan lookup and the launches. Everything that can be rejected is rejected
// here, before any HIP call, so a bad call never reaches the device; a
// missing or foreign GPU is reported as an error, never as a zero-filled C
// (the silent wrong-architecture failure of page "Post-mortem: a GPU stack
// without nvcc, cuBLAS, or LLVM", section 8).
#include <atomic>
#include <mutex>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/sam.h"
#include "sam_internal.h"

#ifndef SAM_BUILD_STAMP
#define SAM_BUILD_STAMP "sam (unstamped build)"
#endif

// Workspace of sam_gemm_noalloc: split-K partials and stream-K slots live in
// this array instead of caller memory. Each GPU the library runs on holds its
// own copy until the process ends. In host code `scratch` only names the
// symbol; its device address, which differs per GPU, comes from
// hipGetSymbolAddress with that GPU current and is kept per device below.
static __device__ __align__(256) unsigned char scratch[SAM_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

sam_status fail(sam_status s, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

// Per-device result of the architecture/loadability check:
// 0 = not checked yet, 1 = good, 2 = unsupported.
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];
std::mutex g_dev_mu;

sam_status device_check_impl()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return fail(SAM_ERR_UNSUPPORTED_DEVICE, "no usable HIP device");
    }
    int st = g_dev_state[dev].load(std::memory_order_acquire);
    if (st == 1) return SAM_OK;
    if (st == 2) return fail(SAM_ERR_UNSUPPORTED_DEVICE, "device %d is not a gfx950 GPU", dev);
    std::lock_guard<std::mutex> lk(g_dev_mu);
    st = g_dev_state[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t prop;
        bool ok = hipGetDeviceProperties(&prop, dev) == hipSuccess &&
                  strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        if (ok) {
            hipFuncAttributes attr;
            ok = hipFuncGetAttributes(&attr, sam::probe_kernel()) == hipSuccess;
        }
        (void)hipGetLastError();
        st = ok ? 1 : 2;
        g_dev_state[dev].store(st, std::memory_order_release);
    }
    if (st != 1)
        return fail(SAM_ERR_UNSUPPORTED_DEVICE,
                    "device %d is not gfx950 or the library's gfx950 kernels do not load", dev);
    return SAM_OK;
}

bool ranges_overlap(const void* a, unsigned long long abytes, const void* b, unsigned long long bbytes)
{
    if (!a || !b || abytes == 0 || bbytes == 0) return false;
    const unsigned long long x = (unsigned long long)a, y = (unsigned long long)b;
    return x < y + bbytes && y < x + abytes;
}

bool aligned16(const void* p) { return ((unsigned long long)p & 15ull) == 0; }

constexpr long long kMaxDim = (1ll << 31) - 1;

sam_status check_shape(long long M, long long N, long long K)
{
    if (M < 0 || N < 0 || K < 0) return fail(SAM_ERR_INVALID_ARG, "negative size M=%lld N=%lld K=%lld", M, N, K);
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim)
        return fail(SAM_ERR_INVALID_ARG, "a size exceeds 2^31-1");
    // Every operand must be addressable with int64 byte offsets.
    const long long lim = (1ll << 61);
    if ((M && K && M > lim / K) || (K && N && K > lim / N) || (M && N && M > lim / N))
        return fail(SAM_ERR_INVALID_ARG, "operand size overflows int64");
    return SAM_OK;
}

void to_public(const sam::Plan& p, sam_plan* out)
{
    memset(out, 0, sizeof(*out));
    out->struct_size = sizeof(sam_plan);
    out->variant_id = p.variant_id;
    sam::plan_name(p, out->name, sizeof(out->name));
    out->dtype = p.dtype;
    out->tile_m = p.bm;
    out->tile_n = p.bn;
    out->tile_k = p.bk;
    out->waves_m = p.wm;
    out->waves_n = p.wn;
    out->mfma_m = p.blk;
    out->split_k = p.sk ? -1 : p.split;
    out->group_m = p.group_m;
    out->xcd_remap = p.xcd_remap;
    out->a_vector = p.a_vec;
    out->b_vector = p.b_vec;
    out->grid_wgs = p.grid;
    out->workspace_bytes = p.ws_bytes;
    out->est_us = p.est_us;
    out->raster_n = p.raster_n;
    out->operand_swap = p.swap;
    out->sk_dp_tiles = p.sk ? p.sk_dp : 0;
    out->tuned = p.tuned;
}

std::atomic<void*> g_scratch[kMaxDevices];

sam_status scratch_address(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return fail(SAM_ERR_UNSUPPORTED_DEVICE, "no usable HIP device");
    }
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lk(g_dev_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p) {
                (void)hipGetLastError();
                return fail(SAM_ERR_INTERNAL, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                            hipGetErrorString(e));
            }
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return SAM_OK;
}

// Block-scaled operands: scale codes and element formats (B is then given
// as N rows of K codes).
struct MxExtra {
    const uint8_t* sa;
    const uint8_t* sb;
    int fmt_a, fmt_b;
};

// Shared body of every GEMM entry point once a plan is known.
// The general entry point's strides of A, B and C (elements) and its
// alpha / beta, taken inside a ring plan's loads and stores.
struct ExTail {
    long long lda, ldb, ldc;
    float alpha, beta;
    int tr;    // operands given transposed, read straight: bit 0 B (N rows of K), bit 1 A (K rows of M)
    bool ct;   // the product (M x N here) goes to C transposed: C is N rows of M values with stride ldc
};

// Whether a plan can take A rows with stride lda != K in place: a ring plan
// whose rows stay 16-byte pieces or which copies A into padded rows anyway
// (the copy reads any stride), or an FP32 ring plan which reads A one value
// at a time. Likewise B.
bool reads_strided(const sam::Plan& p, bool a_side, long long ld)
{
    if (p.kind == sam::KIND_DMA) return (a_side ? p.pad_a : p.pad_b) || ld % 8 == 0;
    if (p.kind == sam::KIND_F32RING)
        return (a_side ? p.pad_a : p.pad_b) || !(a_side ? p.a_vec : p.b_vec) || ld % 4 == 0;
    return false;
}

// Whether a ring plan can read operands given transposed straight (tr: bit
// 0 B as N rows of K values, bit 1 A as K rows of M values): its variant has
// the kernels of that layout, neither operand needs a padded copy (16-bit: K
// and N multiples of 8) and each transposed operand's rows are whole 16-byte
// pieces. FP32 ring plans read one operand given transposed: B with A's
// rows whole 16-byte pieces (K % 4 == 0), or A with B's and C's rows whole
// 16-byte pieces (N % 4 == 0).
bool reads_transposed(const sam::Plan& p, int tr, long long lda, long long ldb)
{
    if (p.kind == sam::KIND_F32RING) {
        if (p.pad_a || p.pad_b) return false;
        if (tr == 1) return p.a_vec && ldb % 4 == 0 && sam::f32_has_bt(p.variant_id, p.sk != 0);
        if (tr == 2) return p.b_vec && p.c_vec && lda % 4 == 0 && sam::f32_has_at(p.variant_id, p.sk != 0);
        return false;
    }
    return p.kind == sam::KIND_DMA && !p.pad_a && !p.pad_b && (!(tr & 1) || ldb % 8 == 0) &&
           (!(tr & 2) || lda % 8 == 0) && sam::dma_has_layout(p.variant_id, tr, p.dtype);
}

// Ring plans store C with row stride ldc (a multiple of 4: 16-byte stores)
// and through the alpha / beta epilogue, in the kernel or the split-K /
// stream-K pass that writes C.
bool writes_general_c(const sam::Plan& p, long long ldc)
{
    return (p.kind == sam::KIND_DMA || p.kind == sam::KIND_F32RING) && ldc % 4 == 0;
}

// x: null for compact operands and C = A B; otherwise what the plan must
// honour, which the caller has checked with reads_strided / writes_general_c.
sam_status run(const sam::Plan& p, const void* A, const void* B, float* C, long long M, long long N,
               long long K, void* ws, unsigned long long ws_bytes, void* stream, const MxExtra* mx = nullptr,
               const ExTail* x = nullptr)
{
    const bool blockscaled = p.dtype == sam::DT_MX8 || p.dtype == sam::DT_MX4;
    // Bytes per element (E2M1: counted as one here; the operand sizes below halve it).
    const unsigned long long es = p.dtype == sam::DT_F32 ? 4 : (blockscaled ? 1 : 2);
    const unsigned long long half = p.dtype == sam::DT_MX4 ? 2 : 1;
    if (blockscaled != (mx != nullptr)) return fail(SAM_ERR_INTERNAL, "scale arguments mismatch");
    const int tr = x ? x->tr : 0;
    const bool at = tr & 2, bt = tr & 1;
    const bool ct = x && x->ct;
    const long long lda = x ? x->lda : (at ? M : K), ldb = x ? x->ldb : (bt ? K : N), ldc = x ? x->ldc : N;
    const float alpha = x ? x->alpha : 1.0f, beta = x ? x->beta : 0.0f;
    const bool gen = alpha != 1.0f || beta != 0.0f;
    if (x && (K == 0 || lda < (at ? M : K) || ldb < (bt ? K : N) || ldc < (ct ? M : N) ||
              (ct && (p.kind != sam::KIND_F32RING || tr || ldc % 4)) ||
              (tr && !reads_transposed(p, tr, lda, ldb)) || (!at && lda != K && !reads_strided(p, true, lda)) ||
              (!bt && ldb != N && !reads_strided(p, false, ldb)) || ((ldc != N || gen) && !writes_general_c(p, ldc))))
        return fail(SAM_ERR_INTERNAL, "strides, transposed operands or alpha / beta on a plan that cannot take them");
    if (M == 0 || N == 0) return SAM_OK;
    // Kernels address a workgroup's operand panels with 32-bit byte offsets:
    // up to 257 rows of A (lda elements each), 129 rows of B and 257 rows of C.
    const long long lim = 0x7FFFFFF0ll;
    if ((long long)lda * (long long)es * 257 >= lim || (long long)ldb * (long long)es * 129 >= lim ||
        ldc * 4ll * 257 >= lim)
        return fail(SAM_ERR_INVALID_ARG, "K=%lld or N=%lld beyond the supported offset range", K, N);
    if (!C) return fail(SAM_ERR_INVALID_ARG, "C is null");
    if (K > 0 && (!A || !B)) return fail(SAM_ERR_INVALID_ARG, "A or B is null");
    if (mx && K > 0 && (!mx->sa || !mx->sb)) return fail(SAM_ERR_INVALID_ARG, "a scale array is null");
    if (!aligned16(C) || (K > 0 && (!aligned16(A) || !aligned16(B))) || (ws && !aligned16(ws)))
        return fail(SAM_ERR_MISALIGNED, "A, B, C and workspace must be 16-byte aligned");
    const unsigned long long cbytes = (unsigned long long)(ct ? (N - 1) * ldc + M : (M - 1) * ldc + N) * 4ull;
    const unsigned long long abytes =
        K ? (unsigned long long)(at ? (K - 1) * lda + M : (M - 1) * lda + K) * es / half : 0;
    const unsigned long long bbytes =
        K ? (unsigned long long)(bt ? (N - 1) * ldb + K : (K - 1) * ldb + N) * es / half : 0;
    if (ranges_overlap(C, cbytes, A, abytes) || ranges_overlap(C, cbytes, B, bbytes))
        return fail(SAM_ERR_INVALID_ARG, "C overlaps A or B");
    if (mx && (ranges_overlap(C, cbytes, mx->sa, (unsigned long long)(M * (K / 32))) ||
               ranges_overlap(C, cbytes, mx->sb, (unsigned long long)(N * (K / 32)))))
        return fail(SAM_ERR_INVALID_ARG, "C overlaps a scale array");
    if (p.ws_bytes > 0) {
        if (!ws || ws_bytes < p.ws_bytes)
            return fail(SAM_ERR_WORKSPACE, "plan %d needs %llu workspace bytes, got %llu", p.variant_id,
                        (unsigned long long)p.ws_bytes, (unsigned long long)(ws ? ws_bytes : 0));
        if (ranges_overlap(C, cbytes, ws, p.ws_bytes) || ranges_overlap(A, abytes, ws, p.ws_bytes) ||
            ranges_overlap(B, bbytes, ws, p.ws_bytes))
            return fail(SAM_ERR_INVALID_ARG, "workspace overlaps A, B or C");
    }
    sam_status d = device_check_impl();
    if (d != SAM_OK) return d;

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    if (K == 0) {
        e = sam::launch_zero(C, M * N, s);
    } else {
        // Operands whose rows are not whole 16-byte pieces, on a plan that
        // pads them (16-bit ring plans always, FP32 ring plans of a padding
        // variant): padded copies in front of the plan's own workspace.
        char* wsb = static_cast<char*>(ws);
        if (p.pad_a || p.pad_b) {
            sam::PadCopy pa{}, pb{};
            char* bb = wsb + (p.pad_a ? ((unsigned long long)(M * p.lda) * es + 255ull) & ~255ull : 0ull);
            if (p.pad_a) pa = {A, lda, wsb, p.lda, M, K};
            if (p.pad_b) pb = {B, ldb, bb, p.ldb, K, N};
            e = sam::launch_pad(pa, pb, (int)es, s);
            if (p.pad_a) A = wsb;
            if (p.pad_b) B = bb;
        }
        if (e != hipSuccess) return fail(SAM_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
        ws = p.ws_bytes > 0 ? wsb + p.ws_inner : ws;
        sam::GemmArgs a{};
        a.A = A;
        a.B = B;
        a.lda = (int)(p.pad_a ? p.lda : lda);
        a.ldb = (int)(p.pad_b ? p.ldb : ldb);
        a.out = p.split > 1 ? static_cast<float*>(ws) : C;
        a.ldc = (int)(p.split > 1 ? N : ldc);   // split-K: the reduce pass writes C
        a.epi = p.split > 1 ? 0 : (int)gen;
        a.ct = p.split > 1 ? 0 : (int)ct;
        a.alpha = alpha;
        a.beta = beta;
        a.M = (int)M;
        a.N = (int)N;
        a.K = (int)K;
        a.k_chunk = p.k_chunk;
        a.split = p.split;
        a.tiles_m = p.tiles_m;
        a.tiles_n = p.tiles_n;
        a.group_m = p.group_m;
        a.xcd_remap = p.xcd_remap;
        a.raster_n = p.raster_n;
        a.part_stride = M * N;
        if (mx) {
            a.sa = mx->sa;
            a.sb = mx->sb;
            a.fmt_a = mx->fmt_a;
            a.fmt_b = mx->fmt_b;
        }
        if (p.sk) {
            a.ws = static_cast<float*>(ws);
            a.sk_iters = (int)((K + p.bk - 1) / p.bk);
            a.sk_grid = p.sk_g;
            a.sk_dp = p.sk_dp;
        }
        sam::Plan q = p;
        q.tr = tr;
        e = sam::launch_gemm(q, a, s);
        if (e == hipSuccess && p.split > 1)
            e = ldc != N || gen || ct
                    ? sam::launch_reduce_ex(static_cast<const float*>(ws), p.split, M * N, C, M, N, ldc, alpha, beta,
                                            (int)ct, s)
                    : sam::launch_reduce(static_cast<const float*>(ws), p.split, M * N, C, M * N, s);
        if (e == hipSuccess && p.sk) e = sam::launch_sk_fixup(p, a, s);
    }
    if (e != hipSuccess) return fail(SAM_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
    g_err[0] = '\0';
    return SAM_OK;
}

sam_status gemm_auto(int dtype, const void* A, const void* B, float* C, int64_t M, int64_t N,
                     int64_t K, void* ws, uint64_t ws_bytes, void* stream)
{
    sam_status st = check_shape(M, N, K);
    if (st != SAM_OK) return st;
    sam::Plan p{};
    if (!sam::plan_auto(M, N, K, dtype, &p)) return fail(SAM_ERR_INTERNAL, "no admissible plan");
    return run(p, A, B, C, M, N, K, ws, ws_bytes, stream);
}

// The general entry point: which passes a call needs and where each one's
// buffer sits in the caller's workspace (256-byte aligned regions).
struct ExLayout {
    bool fast;            // plain C = A*B: straight to the GEMM path
    bool product;         // alpha != 0 and K > 0
    bool pack_a, pack_b;  // op(A) / op(B) copied into compact rows first
    bool direct_a, direct_b;  // strided A / B read in place by a ring plan
    bool fused_c;         // a ring plan stores C itself (stride ldc, alpha / beta)
    int tr;               // operands given transposed read straight by a 16-bit ring plan (bit 0 B, bit 1 A)
    bool ct;              // FP32 A^T B^T as (B A)^T: a ring plan for N x M x K storing C transposed
    bool use_t;           // product into a temporary, then C = alpha T + beta C
    unsigned long long off_a, off_b, off_t, off_w, total;
    sam::Plan plan;
};

unsigned long long align256(unsigned long long x) { return (x + 255ull) & ~255ull; }

// A forced plan for the general entry point: variant, split and raster as
// for sam_gemm_variant_r.
struct ExForced {
    int id, split, raster;
};

sam_status ex_layout(int dtype, int ta, int tb, long long M, long long N, long long K, long long lda, long long ldb,
                     long long ldc, float alpha, float beta, ExLayout* L, const ExForced* f = nullptr)
{
    if (dtype < SAM_F32 || dtype > SAM_F16) return fail(SAM_ERR_INVALID_ARG, "bad dtype %d", dtype);
    if ((ta != SAM_OP_N && ta != SAM_OP_T) || (tb != SAM_OP_N && tb != SAM_OP_T))
        return fail(SAM_ERR_INVALID_ARG, "trans flags must be SAM_OP_N or SAM_OP_T");
    sam_status st = check_shape(M, N, K);
    if (st != SAM_OK) return st;
    const long long min_lda = ta ? M : K, min_ldb = tb ? K : N;
    if (lda < (min_lda > 1 ? min_lda : 1) || ldb < (min_ldb > 1 ? min_ldb : 1) || ldc < (N > 1 ? N : 1))
        return fail(SAM_ERR_INVALID_ARG, "leading dimension too small (lda=%lld ldb=%lld ldc=%lld)", lda, ldb, ldc);
    const long long lim = (1ll << 61);
    if ((M && lda > lim / (M > K ? M : (K ? K : 1))) || (N && ldb > lim / (N > K ? N : (K ? K : 1))) ||
        (M && ldc > lim / M))
        return fail(SAM_ERR_INVALID_ARG, "strided operand size overflows int64");
    const unsigned long long es = dtype == SAM_F32 ? 4 : 2;
    *L = ExLayout{};
    L->product = alpha != 0.0f && K > 0 && M > 0 && N > 0;
    L->fast = !ta && !tb && lda == K && ldb == N && ldc == N && alpha == 1.0f && beta == 0.0f;
    if ((L->product || L->fast) && f) {
        if (f->raster < -1 || f->raster > 1 || f->split < -1)
            return fail(SAM_ERR_INVALID_ARG, "split %d / raster %d out of range", f->split, f->raster);
        if (!sam::variant_get(f->id)) return fail(SAM_ERR_INVALID_ARG, "no variant %d", f->id);
        if (!sam::plan_for_variant(f->id, M, N, K, dtype, f->split, &L->plan, f->raster))
            return fail(SAM_ERR_UNSUPPORTED, "variant %d cannot run dtype %d with split %d, raster %d for K=%lld",
                        f->id, dtype, f->split, f->raster, K);
    } else if (L->product || L->fast) {
        if (!sam::plan_auto(M, N, K, dtype, &L->plan)) return fail(SAM_ERR_INTERNAL, "no admissible plan");
    }
    if (L->fast) {
        L->total = L->plan.ws_bytes;
        return SAM_OK;
    }
    // Both operands given transposed on the FP32 path: A^T B^T = (B A)^T, a
    // plain product of the operands as stored (B as N rows of K, A as K rows
    // of M) whose ring plan stores C transposed, with no copies.
    if (!f && L->product && ta && tb && dtype == SAM_F32 && ldc % 4 == 0) {
        sam::Plan q{};
        if (sam::plan_auto(N, M, K, dtype, &q) && q.kind == sam::KIND_F32RING &&
            (ldb == K || reads_strided(q, true, ldb)) && (lda == M || reads_strided(q, false, lda))) {
            L->ct = true;
            L->fused_c = true;
            L->plan = q;
            L->off_a = L->off_b = L->off_t = L->off_w = 0;
            L->total = q.ws_bytes;
            return SAM_OK;
        }
    }
    // A 16-bit ring tile with no form for A given transposed (192 rows: an
    // A^T row is not whole 1 KB loads) gives way to the same schedule on
    // 256-row tiles, which reads A^T straight instead of packing it.
    if (!f && L->product && ta && L->plan.kind == sam::KIND_DMA &&
        !sam::dma_has_layout(L->plan.variant_id, tb ? 3 : 2, dtype)) {
        const int twin = sam::tile256_twin(L->plan.variant_id);
        sam::Plan q{};
        if (twin >= 0 && (sam::plan_for_variant(twin, M, N, K, dtype, L->plan.sk ? -1 : L->plan.split, &q,
                                                L->plan.raster_n) ||
                          sam::plan_for_variant(twin, M, N, K, dtype, 0, &q, L->plan.raster_n)))
            L->plan = q;
    }
    // A 16-bit ring plan that has to read C (beta != 0) takes the operand-swap
    // form of its variant when there is one: the same tile and schedule, with
    // C read and written 16 bytes per lane instead of 4.
    if (!f && L->product && beta != 0.0f && L->plan.kind == sam::KIND_DMA && !L->plan.swap) {
        const int twin = sam::swap_twin(L->plan.variant_id);
        sam::Plan q{};
        if (twin >= 0 && sam::plan_for_variant(twin, M, N, K, dtype, L->plan.sk ? -1 : L->plan.split, &q,
                                               L->plan.raster_n))
            L->plan = q;
    }
    L->direct_a = L->product && !ta && lda != K && reads_strided(L->plan, true, lda);
    L->direct_b = L->product && !tb && ldb != N && reads_strided(L->plan, false, ldb);
    // Transposed operands read straight where the plan can (both, else B
    // alone, else A alone); the rest is packed.
    L->tr = 0;
    if (L->product) {
        for (int tr : {3, 1, 2})
            if ((tr & 1) <= (tb ? 1 : 0) && (tr & 2) <= (ta ? 2 : 0) && reads_transposed(L->plan, tr, lda, ldb)) {
                L->tr = tr;
                break;
            }
    }
    L->fused_c = L->product && writes_general_c(L->plan, ldc);
    L->pack_a = L->product && (ta || lda != K) && !L->direct_a && !(L->tr & 2);
    L->pack_b = L->product && (tb || ldb != N) && !L->direct_b && !(L->tr & 1);
    L->use_t = L->product && !L->fused_c && !(ldc == N && beta == 0.0f);
    L->off_a = 0;
    L->off_b = align256(L->off_a + (L->pack_a ? (unsigned long long)(M * K) * es : 0));
    L->off_t = align256(L->off_b + (L->pack_b ? (unsigned long long)(K * N) * es : 0));
    L->off_w = align256(L->off_t + (L->use_t ? (unsigned long long)(M * N) * 4 : 0));
    L->total = L->off_w + (L->product ? L->plan.ws_bytes : 0);
    return SAM_OK;
}

// The general entry point once its layout (and plan) is known.
sam_status gemm_ex_run(const ExLayout& L, sam_dtype dtype, sam_op trans_a, sam_op trans_b, int64_t M, int64_t N,
                       int64_t K, float alpha, const void* A, int64_t lda, const void* B, int64_t ldb, float beta,
                       float* C, int64_t ldc, void* workspace, uint64_t workspace_bytes, void* stream)
{
    sam_status st = SAM_OK;
    if (L.fast) return run(L.plan, A, B, C, M, N, K, workspace, workspace_bytes, stream);
    if (M == 0 || N == 0) return SAM_OK;
    if (!C) return fail(SAM_ERR_INVALID_ARG, "C is null");
    if (L.product && (!A || !B)) return fail(SAM_ERR_INVALID_ARG, "A or B is null");
    if (!aligned16(C) || (L.product && (!aligned16(A) || !aligned16(B))) || (workspace && !aligned16(workspace)))
        return fail(SAM_ERR_MISALIGNED, "A, B, C and workspace must be 16-byte aligned");
    if (L.total > 0 && (!workspace || workspace_bytes < L.total))
        return fail(SAM_ERR_WORKSPACE, "sam_gemm_ex needs %llu workspace bytes, got %llu", L.total,
                    (unsigned long long)(workspace ? workspace_bytes : 0));
    const unsigned long long es = dtype == SAM_F32 ? 4 : 2;
    const unsigned long long cbytes = ((unsigned long long)(M - 1) * ldc + N) * 4;
    const unsigned long long abytes = L.product ? ((unsigned long long)((trans_a ? K : M) - 1) * lda + (trans_a ? M : K)) * es : 0;
    const unsigned long long bbytes = L.product ? ((unsigned long long)((trans_b ? N : K) - 1) * ldb + (trans_b ? K : N)) * es : 0;
    if (ranges_overlap(C, cbytes, A, abytes) || ranges_overlap(C, cbytes, B, bbytes))
        return fail(SAM_ERR_INVALID_ARG, "C overlaps A or B");
    if (ranges_overlap(workspace, L.total, C, cbytes) || ranges_overlap(workspace, L.total, A, abytes) ||
        ranges_overlap(workspace, L.total, B, bbytes))
        return fail(SAM_ERR_INVALID_ARG, "workspace overlaps A, B or C");
    sam_status d = device_check_impl();
    if (d != SAM_OK) return d;

    hipStream_t s = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    hipError_t e = hipSuccess;
    if (!L.product) {
        e = sam::launch_axpby(nullptr, 0, C, ldc, M, N, alpha, beta, s);   // alpha * 0 + beta * C
    } else {
        const void* a = A;
        const void* b = B;
        if (L.pack_a) {
            e = sam::launch_pack(A, lda, ws + L.off_a, M, K, (int)es, trans_a, s);
            a = ws + L.off_a;
        }
        if (e == hipSuccess && L.pack_b) {
            e = sam::launch_pack(B, ldb, ws + L.off_b, K, N, (int)es, trans_b, s);
            b = ws + L.off_b;
        }
        if (e != hipSuccess) return fail(SAM_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
        if (L.ct) {   // (B A)^T: B as the N x K left operand, A as the K x M right one
            const ExTail y{ldb, lda, ldc, alpha, beta, 0, true};
            return run(L.plan, B, A, C, N, M, K, L.plan.ws_bytes ? ws : nullptr, L.plan.ws_bytes, stream, nullptr, &y);
        }
        float* out = L.use_t ? reinterpret_cast<float*>(ws + L.off_t) : C;
        const ExTail x{(L.direct_a || (L.tr & 2)) ? lda : K, (L.direct_b || (L.tr & 1)) ? ldb : N,
                       L.fused_c ? ldc : N, L.fused_c ? alpha : 1.0f, L.fused_c ? beta : 0.0f, L.tr, false};
        st = run(L.plan, a, b, out, M, N, K, L.plan.ws_bytes ? ws + L.off_w : nullptr, L.plan.ws_bytes, stream,
                 nullptr, &x);
        if (st != SAM_OK) return st;
        if (L.fused_c) {
            // alpha / beta and the stride of C were applied where C was written
        } else if (L.use_t)
            e = sam::launch_axpby(out, N, C, ldc, M, N, alpha, beta, s);
        else if (alpha != 1.0f)
            e = sam::launch_axpby(C, ldc, C, ldc, M, N, alpha, 0.0f, s);   // in place: C = alpha C
    }
    if (e != hipSuccess) return fail(SAM_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
    g_err[0] = '\0';
    return SAM_OK;
}

}  // namespace

extern "C" {

sam_status sam_gemm_ex_workspace(sam_dtype dtype, sam_op trans_a, sam_op trans_b, int64_t M, int64_t N, int64_t K,
                                 int64_t lda, int64_t ldb, int64_t ldc, float alpha, float beta, uint64_t* bytes)
{
    if (!bytes) return fail(SAM_ERR_INVALID_ARG, "bytes is null");
    ExLayout L;
    sam_status st = ex_layout(dtype, trans_a, trans_b, M, N, K, lda, ldb, ldc, alpha, beta, &L);
    if (st != SAM_OK) return st;
    *bytes = L.total;
    return SAM_OK;
}

sam_status sam_gemm_ex(sam_dtype dtype, sam_op trans_a, sam_op trans_b, int64_t M, int64_t N, int64_t K, float alpha,
                       const void* A, int64_t lda, const void* B, int64_t ldb, float beta, float* C, int64_t ldc,
                       void* workspace, uint64_t workspace_bytes, void* stream)
{
    ExLayout L;
    sam_status st = ex_layout(dtype, trans_a, trans_b, M, N, K, lda, ldb, ldc, alpha, beta, &L);
    if (st != SAM_OK) return st;
    return gemm_ex_run(L, dtype, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace,
                       workspace_bytes, stream);
}

sam_status sam_gemm_ex_variant_workspace(int32_t id, int32_t split_k, int32_t raster_n, sam_dtype dtype,
                                         sam_op trans_a, sam_op trans_b, int64_t M, int64_t N, int64_t K, int64_t lda,
                                         int64_t ldb, int64_t ldc, float alpha, float beta, uint64_t* bytes)
{
    if (!bytes) return fail(SAM_ERR_INVALID_ARG, "bytes is null");
    ExLayout L;
    const ExForced f{id, split_k, raster_n};
    sam_status st = ex_layout(dtype, trans_a, trans_b, M, N, K, lda, ldb, ldc, alpha, beta, &L, &f);
    if (st != SAM_OK) return st;
    *bytes = L.total;
    return SAM_OK;
}

sam_status sam_gemm_ex_variant(int32_t id, int32_t split_k, int32_t raster_n, sam_dtype dtype, sam_op trans_a,
                               sam_op trans_b, int64_t M, int64_t N, int64_t K, float alpha, const void* A,
                               int64_t lda, const void* B, int64_t ldb, float beta, float* C, int64_t ldc,
                               void* workspace, uint64_t workspace_bytes, void* stream)
{
    ExLayout L;
    const ExForced f{id, split_k, raster_n};
    sam_status st = ex_layout(dtype, trans_a, trans_b, M, N, K, lda, ldb, ldc, alpha, beta, &L, &f);
    if (st != SAM_OK) return st;
    return gemm_ex_run(L, dtype, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace,
                       workspace_bytes, stream);
}


sam_status sam_gemm_plan(int64_t M, int64_t N, int64_t K, sam_dtype dtype, sam_plan* out)
{
    if (!out) return fail(SAM_ERR_INVALID_ARG, "out is null");
    if (dtype < SAM_F32 || dtype > SAM_MXFP4) return fail(SAM_ERR_INVALID_ARG, "bad dtype %d", (int)dtype);
    sam_status st = check_shape(M, N, K);
    if (st != SAM_OK) return st;
    if ((dtype == SAM_MXFP8 || dtype == SAM_MXFP4) && K % 32 != 0)
        return fail(SAM_ERR_INVALID_ARG, "block-scaled operands need K %% 32 == 0 (K=%lld)", (long long)K);
    sam::Plan p{};
    if (!sam::plan_auto(M, N, K, dtype, &p)) return fail(SAM_ERR_INTERNAL, "no admissible plan");
    to_public(p, out);
    return SAM_OK;
}

sam_status sam_gemm_f32(const float* A, const float* B, float* C, int64_t M, int64_t N, int64_t K,
                        void* workspace, uint64_t workspace_bytes, void* stream)
{
    return gemm_auto(sam::DT_F32, A, B, C, M, N, K, workspace, workspace_bytes, stream);
}

sam_status sam_gemm_bf16(const uint16_t* A, const uint16_t* B, float* C, int64_t M, int64_t N,
                         int64_t K, void* workspace, uint64_t workspace_bytes, void* stream)
{
    return gemm_auto(sam::DT_BF16, A, B, C, M, N, K, workspace, workspace_bytes, stream);
}

sam_status sam_gemm_f16(const uint16_t* A, const uint16_t* B, float* C, int64_t M, int64_t N,
                        int64_t K, void* workspace, uint64_t workspace_bytes, void* stream)
{
    return gemm_auto(sam::DT_F16, A, B, C, M, N, K, workspace, workspace_bytes, stream);
}

int32_t sam_variant_count(void) { return sam::variant_count(); }

sam_status sam_variant_info(int32_t id, sam_plan* out)
{
    if (!out) return fail(SAM_ERR_INVALID_ARG, "out is null");
    const sam::Variant* v = sam::variant_get(id);
    if (!v) return fail(SAM_ERR_INVALID_ARG, "no variant %d", id);
    memset(out, 0, sizeof(*out));
    out->struct_size = sizeof(sam_plan);
    out->variant_id = v->id;
    snprintf(out->name, sizeof(out->name), "%s", v->name);
    out->dtype = -1;
    out->tile_m = v->bm;
    out->tile_n = v->bn;
    out->tile_k = 0;
    out->waves_m = v->wm;
    out->waves_n = v->wn;
    out->mfma_m = v->blk;
    out->split_k = 1;
    out->group_m = v->group_m;
    out->xcd_remap = v->xcd_remap;
    return SAM_OK;
}

sam_status sam_variant_plan(int32_t id, int64_t M, int64_t N, int64_t K, sam_dtype dtype,
                            int32_t split_k, sam_plan* out)
{
    return sam_variant_plan_r(id, M, N, K, dtype, split_k, -1, out);
}

sam_status sam_variant_plan_r(int32_t id, int64_t M, int64_t N, int64_t K, sam_dtype dtype, int32_t split_k,
                              int32_t raster_n, sam_plan* out)
{
    if (!out) return fail(SAM_ERR_INVALID_ARG, "out is null");
    if (raster_n < -1 || raster_n > 1)
        return fail(SAM_ERR_INVALID_ARG, "raster_n %d (-1 the dispatcher's choice, 0 M-major, 1 N-major)", raster_n);
    if (dtype < SAM_F32 || dtype > SAM_MXFP4) return fail(SAM_ERR_INVALID_ARG, "bad dtype %d", (int)dtype);
    if (split_k < -1) return fail(SAM_ERR_INVALID_ARG, "split %d (-1 is stream-K, 0 the variant's choice)", split_k);
    sam_status st = check_shape(M, N, K);
    if (st != SAM_OK) return st;
    if (!sam::variant_get(id)) return fail(SAM_ERR_INVALID_ARG, "no variant %d", id);
    sam::Plan p{};
    if (!sam::plan_for_variant(id, M, N, K, dtype, split_k, &p, raster_n))
        return fail(SAM_ERR_UNSUPPORTED, "variant %d cannot run dtype %d with split %d, raster %d for K=%lld", id,
                    (int)dtype, split_k, raster_n, (long long)K);
    to_public(p, out);
    return SAM_OK;
}

sam_status sam_gemm_variant(int32_t id, sam_dtype dtype, int32_t split_k, const void* A, const void* B,
                            float* C, int64_t M, int64_t N, int64_t K, void* workspace,
                            uint64_t workspace_bytes, void* stream)
{
    return sam_gemm_variant_r(id, dtype, split_k, -1, A, B, C, M, N, K, workspace, workspace_bytes, stream);
}

sam_status sam_gemm_variant_r(int32_t id, sam_dtype dtype, int32_t split_k, int32_t raster_n, const void* A,
                              const void* B, float* C, int64_t M, int64_t N, int64_t K, void* workspace,
                              uint64_t workspace_bytes, void* stream)
{
    if (raster_n < -1 || raster_n > 1)
        return fail(SAM_ERR_INVALID_ARG, "raster_n %d (-1 the dispatcher's choice, 0 M-major, 1 N-major)", raster_n);
    if (dtype == SAM_MXFP8 || dtype == SAM_MXFP4)
        return fail(SAM_ERR_INVALID_ARG, "block-scaled operands go through sam_gemm_mxfp8_variant / sam_gemm_mxfp4_variant");
    if (dtype < SAM_F32 || dtype > SAM_F16) return fail(SAM_ERR_INVALID_ARG, "bad dtype %d", (int)dtype);
    if (split_k < -1) return fail(SAM_ERR_INVALID_ARG, "split %d (-1 is stream-K, 0 the variant's choice)", split_k);
    sam_status st = check_shape(M, N, K);
    if (st != SAM_OK) return st;
    if (!sam::variant_get(id)) return fail(SAM_ERR_INVALID_ARG, "no variant %d", id);
    sam::Plan p{};
    if (!sam::plan_for_variant(id, M, N, K, dtype, split_k, &p, raster_n))
        return fail(SAM_ERR_UNSUPPORTED, "variant %d cannot run dtype %d with split %d, raster %d for K=%lld", id,
                    (int)dtype, split_k, raster_n, (long long)K);
    return run(p, A, B, C, M, N, K, workspace, workspace_bytes, stream);
}

sam_status sam_gemm_plan_model(int64_t M, int64_t N, int64_t K, sam_dtype dtype, sam_plan* out)
{
    if (!out) return fail(SAM_ERR_INVALID_ARG, "out is null");
    if (dtype < SAM_F32 || dtype > SAM_MXFP4) return fail(SAM_ERR_INVALID_ARG, "bad dtype %d", (int)dtype);
    sam_status st = check_shape(M, N, K);
    if (st != SAM_OK) return st;
    sam::Plan p{};
    if (!sam::plan_model(M, N, K, dtype, &p)) return fail(SAM_ERR_INTERNAL, "no admissible plan");
    to_public(p, out);
    return SAM_OK;
}

// dtype DT_MX8 (formats fmt_a / fmt_b) or DT_MX4 (E2M1; formats ignored).
static sam_status gemm_mx_impl(int dtype, int32_t id, int32_t split_k, int fmt_a, int fmt_b, const uint8_t* A,
                               const uint8_t* scale_a, const uint8_t* Bt, const uint8_t* scale_b, float* C,
                               int64_t M, int64_t N, int64_t K, void* workspace, uint64_t workspace_bytes,
                               void* stream)
{
    if (dtype == sam::DT_MX8 &&
        ((fmt_a != SAM_E4M3 && fmt_a != SAM_E5M2) || (fmt_b != SAM_E4M3 && fmt_b != SAM_E5M2)))
        return fail(SAM_ERR_INVALID_ARG, "element formats must be SAM_E4M3 or SAM_E5M2 (got %d, %d)", (int)fmt_a,
                    (int)fmt_b);
    if (split_k < 0) return fail(SAM_ERR_INVALID_ARG, "split %d (0 is the variant's choice)", split_k);
    sam_status st = check_shape(M, N, K);
    if (st != SAM_OK) return st;
    if (K % 32 != 0)
        return fail(SAM_ERR_INVALID_ARG, "block-scaled operands need K %% 32 == 0 (K=%lld)", (long long)K);
    sam::Plan p{};
    if (id < 0) {
        if (!sam::plan_auto(M, N, K, dtype, &p)) return fail(SAM_ERR_INTERNAL, "no admissible plan");
    } else {
        if (!sam::variant_get(id)) return fail(SAM_ERR_INVALID_ARG, "no variant %d", id);
        if (!sam::plan_for_variant(id, M, N, K, dtype, split_k, &p))
            return fail(SAM_ERR_UNSUPPORTED, "variant %d cannot run block-scaled operands with split %d", id, split_k);
    }
    const MxExtra mx{scale_a, scale_b, dtype == sam::DT_MX8 ? fmt_a : 4, dtype == sam::DT_MX8 ? fmt_b : 4};
    return run(p, A, Bt, C, M, N, K, workspace, workspace_bytes, stream, &mx);
}

sam_status sam_gemm_mxfp8(sam_fp8_format fmt_a, sam_fp8_format fmt_b, const uint8_t* A, const uint8_t* scale_a,
                          const uint8_t* Bt, const uint8_t* scale_b, float* C, int64_t M, int64_t N, int64_t K,
                          void* workspace, uint64_t workspace_bytes, void* stream)
{
    return gemm_mx_impl(sam::DT_MX8, -1, 0, fmt_a, fmt_b, A, scale_a, Bt, scale_b, C, M, N, K, workspace,
                        workspace_bytes, stream);
}

sam_status sam_gemm_mxfp8_variant(int32_t id, int32_t split_k, sam_fp8_format fmt_a, sam_fp8_format fmt_b,
                                  const uint8_t* A, const uint8_t* scale_a, const uint8_t* Bt,
                                  const uint8_t* scale_b, float* C, int64_t M, int64_t N, int64_t K,
                                  void* workspace, uint64_t workspace_bytes, void* stream)
{
    if (id < 0) return fail(SAM_ERR_INVALID_ARG, "no variant %d", id);
    return gemm_mx_impl(sam::DT_MX8, id, split_k, fmt_a, fmt_b, A, scale_a, Bt, scale_b, C, M, N, K, workspace,
                        workspace_bytes, stream);
}

sam_status sam_gemm_mxfp4(const uint8_t* A, const uint8_t* scale_a, const uint8_t* Bt, const uint8_t* scale_b,
                          float* C, int64_t M, int64_t N, int64_t K, void* workspace, uint64_t workspace_bytes,
                          void* stream)
{
    return gemm_mx_impl(sam::DT_MX4, -1, 0, 0, 0, A, scale_a, Bt, scale_b, C, M, N, K, workspace, workspace_bytes,
                        stream);
}

sam_status sam_gemm_mxfp4_variant(int32_t id, int32_t split_k, const uint8_t* A, const uint8_t* scale_a,
                                  const uint8_t* Bt, const uint8_t* scale_b, float* C, int64_t M, int64_t N,
                                  int64_t K, void* workspace, uint64_t workspace_bytes, void* stream)
{
    if (id < 0) return fail(SAM_ERR_INVALID_ARG, "no variant %d", id);
    return gemm_mx_impl(sam::DT_MX4, id, split_k, 0, 0, A, scale_a, Bt, scale_b, C, M, N, K, workspace,
                        workspace_bytes, stream);
}

sam_status sam_gemm_noalloc(sam_dtype dtype, const void* A, const void* B, float* C, int64_t M, int64_t N,
                            int64_t K, void* stream)
{
    if (dtype < SAM_F32 || dtype > SAM_F16) return fail(SAM_ERR_INVALID_ARG, "bad dtype %d", (int)dtype);
    sam_status st = check_shape(M, N, K);
    if (st != SAM_OK) return st;
    sam::Plan p{};
    if (!sam::plan_auto(M, N, K, dtype, &p)) return fail(SAM_ERR_INTERNAL, "no admissible plan");
    if (p.ws_bytes > SAM_SCRATCH_BYTES) {
        char name[64];
        sam::plan_name(p, name, sizeof(name));
        return fail(SAM_ERR_WORKSPACE,
                    "plan %s needs %llu workspace bytes; the scratch array of sam_gemm_noalloc holds %llu",
                    name, (unsigned long long)p.ws_bytes, (unsigned long long)SAM_SCRATCH_BYTES);
    }
    void* ws = nullptr;
    if (p.ws_bytes > 0 && M > 0 && N > 0 && K > 0) {
        st = device_check_impl();
        if (st != SAM_OK) return st;
        st = scratch_address(&ws);
        if (st != SAM_OK) return st;
    }
    return run(p, A, B, C, M, N, K, ws, p.ws_bytes, stream);
}

sam_status sam_device_check(void) { return device_check_impl(); }

const char* sam_status_string(sam_status s)
{
    switch (s) {
    case SAM_OK: return "SAM_OK";
    case SAM_ERR_INVALID_ARG: return "SAM_ERR_INVALID_ARG";
    case SAM_ERR_MISALIGNED: return "SAM_ERR_MISALIGNED";
    case SAM_ERR_WORKSPACE: return "SAM_ERR_WORKSPACE";
    case SAM_ERR_UNSUPPORTED: return "SAM_ERR_UNSUPPORTED";
    case SAM_ERR_UNSUPPORTED_DEVICE: return "SAM_ERR_UNSUPPORTED_DEVICE";
    case SAM_ERR_LAUNCH: return "SAM_ERR_LAUNCH";
    case SAM_ERR_INTERNAL: return "SAM_ERR_INTERNAL";
    }
    return "SAM_ERR_UNKNOWN";
}

const char* sam_last_error(void) { return g_err; }

const char* sam_build_info(void) { return SAM_BUILD_STAMP; }

}  // extern "C"
