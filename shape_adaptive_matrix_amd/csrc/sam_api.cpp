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
}

// Shared body of every GEMM entry point once a plan is known.
sam_status run(const sam::Plan& p, const void* A, const void* B, float* C, long long M, long long N,
               long long K, void* ws, unsigned long long ws_bytes, void* stream)
{
    const unsigned long long es = p.dtype == sam::DT_F32 ? 4 : 2;
    if (M == 0 || N == 0) return SAM_OK;
    // Kernels address a workgroup's operand panels with 32-bit byte offsets:
    // up to 257 rows of A (K elements each), 129 rows of B and 257 rows of C.
    const long long lim = 0x7FFFFFF0ll;
    if ((long long)K * (long long)es * 257 >= lim || (long long)N * (long long)es * 129 >= lim ||
        N * 4ll * 257 >= lim)
        return fail(SAM_ERR_INVALID_ARG, "K=%lld or N=%lld beyond the supported offset range", K, N);
    if (!C) return fail(SAM_ERR_INVALID_ARG, "C is null");
    if (K > 0 && (!A || !B)) return fail(SAM_ERR_INVALID_ARG, "A or B is null");
    if (!aligned16(C) || (K > 0 && (!aligned16(A) || !aligned16(B))) || (ws && !aligned16(ws)))
        return fail(SAM_ERR_MISALIGNED, "A, B, C and workspace must be 16-byte aligned");
    const unsigned long long cbytes = (unsigned long long)(M * N) * 4ull;
    if (ranges_overlap(C, cbytes, A, (unsigned long long)(M * K) * es) ||
        ranges_overlap(C, cbytes, B, (unsigned long long)(K * N) * es))
        return fail(SAM_ERR_INVALID_ARG, "C overlaps A or B");
    if (p.ws_bytes > 0) {
        if (!ws || ws_bytes < p.ws_bytes)
            return fail(SAM_ERR_WORKSPACE, "plan %d needs %llu workspace bytes, got %llu", p.variant_id,
                        (unsigned long long)p.ws_bytes, (unsigned long long)(ws ? ws_bytes : 0));
        if (ranges_overlap(C, cbytes, ws, p.ws_bytes) || ranges_overlap(A, (unsigned long long)(M * K) * es, ws, p.ws_bytes) ||
            ranges_overlap(B, (unsigned long long)(K * N) * es, ws, p.ws_bytes))
            return fail(SAM_ERR_INVALID_ARG, "workspace overlaps A, B or C");
    }
    sam_status d = device_check_impl();
    if (d != SAM_OK) return d;

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (K == 0) {
        e = sam::launch_zero(C, M * N, s);
    } else {
        sam::GemmArgs a{};
        a.A = A;
        a.B = B;
        a.out = p.split > 1 ? static_cast<float*>(ws) : C;
        a.M = (int)M;
        a.N = (int)N;
        a.K = (int)K;
        a.k_chunk = p.k_chunk;
        a.split = p.split;
        a.tiles_m = p.tiles_m;
        a.tiles_n = p.tiles_n;
        a.group_m = p.group_m;
        a.xcd_remap = p.xcd_remap;
        a.part_stride = M * N;
        if (p.sk) {
            a.ws = static_cast<float*>(ws);
            a.sk_iters = (int)((K + p.bk - 1) / p.bk);
            a.sk_grid = (int)p.grid;
        }
        e = sam::launch_gemm(p, a, s);
        if (e == hipSuccess && p.split > 1)
            e = sam::launch_reduce(static_cast<const float*>(ws), p.split, M * N, C, M * N, s);
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

}  // namespace

extern "C" {

sam_status sam_gemm_plan(int64_t M, int64_t N, int64_t K, sam_dtype dtype, sam_plan* out)
{
    if (!out) return fail(SAM_ERR_INVALID_ARG, "out is null");
    if (dtype < SAM_F32 || dtype > SAM_F16) return fail(SAM_ERR_INVALID_ARG, "bad dtype %d", (int)dtype);
    sam_status st = check_shape(M, N, K);
    if (st != SAM_OK) return st;
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
    if (!out) return fail(SAM_ERR_INVALID_ARG, "out is null");
    if (dtype < SAM_F32 || dtype > SAM_F16) return fail(SAM_ERR_INVALID_ARG, "bad dtype %d", (int)dtype);
    if (split_k < -1) return fail(SAM_ERR_INVALID_ARG, "split %d (-1 is stream-K, 0 the variant's choice)", split_k);
    sam_status st = check_shape(M, N, K);
    if (st != SAM_OK) return st;
    if (!sam::variant_get(id)) return fail(SAM_ERR_INVALID_ARG, "no variant %d", id);
    sam::Plan p{};
    if (!sam::plan_for_variant(id, M, N, K, dtype, split_k, &p))
        return fail(SAM_ERR_UNSUPPORTED, "variant %d cannot run dtype %d with split %d for K=%lld", id,
                    (int)dtype, split_k, (long long)K);
    to_public(p, out);
    return SAM_OK;
}

sam_status sam_gemm_variant(int32_t id, sam_dtype dtype, int32_t split_k, const void* A, const void* B,
                            float* C, int64_t M, int64_t N, int64_t K, void* workspace,
                            uint64_t workspace_bytes, void* stream)
{
    if (dtype < SAM_F32 || dtype > SAM_F16) return fail(SAM_ERR_INVALID_ARG, "bad dtype %d", (int)dtype);
    if (split_k < -1) return fail(SAM_ERR_INVALID_ARG, "split %d (-1 is stream-K, 0 the variant's choice)", split_k);
    sam_status st = check_shape(M, N, K);
    if (st != SAM_OK) return st;
    if (!sam::variant_get(id)) return fail(SAM_ERR_INVALID_ARG, "no variant %d", id);
    sam::Plan p{};
    if (!sam::plan_for_variant(id, M, N, K, dtype, split_k, &p))
        return fail(SAM_ERR_UNSUPPORTED, "variant %d cannot run dtype %d with split %d for K=%lld", id,
                    (int)dtype, split_k, (long long)K);
    return run(p, A, B, C, M, N, K, workspace, workspace_bytes, stream);
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
