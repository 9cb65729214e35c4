// C-ABI layer: argument validation, workspace sizing, kernel dispatch and
// the benchmark timing hooks.  Every check runs before any HIP call, so an
// invalid call launches nothing (and can be tested without a GPU).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/attn.h"
#include "attn_internal.hpp"

namespace {

thread_local std::string g_last_error;

attn_status fail(attn_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
attn_status fail(attn_status st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

attn_status ok()
{
    g_last_error.clear();
    return ATTN_OK;
}

attn_status from_hip(hipError_t e, const char *what)
{
    if (e == hipSuccess)
        return ok();
    return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool valid_scale(float s) { return std::isfinite(s) && s > 0.f; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// a * b * c <= limit for non-negative factors, decided without forming a
// product that could overflow
bool product_le(long long a, long long b, long long c, long long limit)
{
    if (a == 0 || b == 0 || c == 0)
        return true;
    if (a > limit / b)
        return false;
    return c <= limit / (a * b);
}

// ---------------------------------------------------------------- profiler
// Events come from a pool created when the profiler is enabled, so that the
// timed region itself creates no events; the pool grows only if a run
// records more launches than it holds.
struct ProfEvent {
    const char *name;  // a string literal of the launcher
    hipEvent_t begin, end;
};
constexpr size_t kProfReserve = 1024;  // launches recorded without growing the pool
thread_local bool g_prof_on = false;
thread_local std::vector<ProfEvent> g_prof;  // pool; the first g_prof_used are recorded
thread_local size_t g_prof_used = 0;

bool prof_grow(size_t n)
{
    while (g_prof.size() < n) {
        ProfEvent ev{nullptr, nullptr, nullptr};
        if (hipEventCreate(&ev.begin) != hipSuccess)
            return false;
        if (hipEventCreate(&ev.end) != hipSuccess) {
            hipEventDestroy(ev.begin);
            return false;
        }
        g_prof.push_back(ev);
    }
    return true;
}

void prof_release()
{
    for (auto &ev : g_prof) {
        hipEventDestroy(ev.begin);
        hipEventDestroy(ev.end);
    }
    g_prof.clear();
    g_prof_used = 0;
}

}  // namespace

namespace attn {

void prof_begin(const char *name, hipStream_t s)
{
    if (!g_prof_on)
        return;
    if (g_prof_used == g_prof.size() && !prof_grow(g_prof.size() + kProfReserve))
        return;
    ProfEvent &ev = g_prof[g_prof_used++];
    ev.name = name;
    hipEventRecord(ev.begin, s);
}

void prof_end(hipStream_t s)
{
    if (!g_prof_on || g_prof_used == 0)
        return;
    hipEventRecord(g_prof[g_prof_used - 1].end, s);
}

}  // namespace attn

namespace {

// The partial outputs and LSEs of the split kernel, carved from `base` (the
// layout attn_decode_workspace_size counts).
void set_partials(attn::DecodeArgs &a, void *base)
{
    const size_t slots = attn::decode_partial_slots(a.B, a.Hkv);
    a.part_o = (float *)base;
    a.part_lse =
        (float *)((char *)base + align_up(sizeof(float) * slots * (a.H / a.Hkv) * a.d, 256));
}

// The quantised prefill modes (valid modes that only attn_fwd implements).
bool quant_mode(int mode)
{
    return mode == ATTN_MODE_SAGE_QK_I8_BLK64_PV_FP8_E4M3 ||
           mode == ATTN_MODE_SAGE3_QK_MXFP4_PV_MXFP4 || mode == ATTN_MODE_SAGE3_QK_MXFP6_PV_MXFP6;
}

// Checks shared by the contiguous and the paged decode; fills everything of
// DecodeArgs but the cache layout.
attn_status decode_common(const void *q, const void *k_cache, const void *v_cache,
                          const int32_t *seqlens, void *o, float *lse, int B, int H, int Hkv,
                          int N_max, int d, float scale, int mode, int o_dtype, int split_tokens,
                          void *workspace, size_t workspace_bytes, attn::DecodeArgs &a)
{
    if (!q || !k_cache || !v_cache || !seqlens || !o)
        return fail(ATTN_ERR_INVALID_ARG,
                    "q, k_cache, v_cache, seqlens and o must be non-null device pointers");
    if (B <= 0 || H <= 0 || Hkv <= 0 || N_max <= 0 || d <= 0)
        return fail(ATTN_ERR_INVALID_ARG, "sizes must be positive (B=%d H=%d Hkv=%d N_max=%d d=%d)",
                    B, H, Hkv, N_max, d);
    if (H % Hkv != 0)
        return fail(ATTN_ERR_INVALID_ARG, "H=%d is not a multiple of Hkv=%d", H, Hkv);
    if (!valid_scale(scale))
        return fail(ATTN_ERR_INVALID_ARG, "scale must be finite and > 0");
    if (o_dtype != ATTN_OUT_BF16 && o_dtype != ATTN_OUT_FP32)
        return fail(ATTN_ERR_INVALID_ARG, "unknown output dtype %d", o_dtype);
    if (split_tokens <= 0 || split_tokens % 64 != 0)
        return fail(ATTN_ERR_INVALID_ARG, "split_tokens=%d must be a positive multiple of 64",
                    split_tokens);
    if (mode != ATTN_MODE_EXACT_BF16)
        return fail(quant_mode(mode) ? ATTN_ERR_UNSUPPORTED
                        : ATTN_ERR_INVALID_ARG,
                    "decode supports only the exact bf16 mode (mode=%d)", mode);
    if (d != 64 && d != 128)
        return fail(ATTN_ERR_UNSUPPORTED, "head dim d=%d (supported: 64, 128)", d);
    const int G = H / Hkv;
    if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
        return fail(ATTN_ERR_UNSUPPORTED,
                    "query heads per kv head %d (supported: 1, 2, 4, 8, 16)", G);
    // global key offsets (Hkv * sum of lengths) and slot indices stay far
    // inside 64-bit and 32-bit arithmetic
    if (!product_le(B, Hkv, N_max, 1LL << 40) || (long long)B * H > 0x7fffff00LL ||
        (long long)B * Hkv > 0x7fff0000LL)
        return fail(ATTN_ERR_UNSUPPORTED, "problem too large for the work split");
    const size_t need = attn_decode_workspace_size(B, H, Hkv, d);
    if (!workspace || workspace_bytes < need)
        return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);

    a = attn::DecodeArgs{};
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.seqlens = seqlens;
    a.o = o;
    a.lse = lse;
    a.B = B;
    a.H = H;
    a.Hkv = Hkv;
    a.N_max = N_max;
    a.d = d;
    a.scale = scale;
    a.out_fp32 = o_dtype == ATTN_OUT_FP32;
    a.split_tokens = split_tokens;
    set_partials(a, workspace);
    return ATTN_OK;
}

}  // namespace

extern "C" {

const char *attn_status_string(int status)
{
    switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

const char *attn_last_error(void) { return g_last_error.c_str(); }

// Sizes attn_fwd accepts (positive, H a multiple of Hkv, d of 64 or 128, and
// within the grid mapping's limits); the workspace arithmetic below stays far
// inside 64 bits for them.
bool fwd_sizes_supported(int B, int H, int Hkv, int N, int d)
{
    return B > 0 && H > 0 && Hkv > 0 && N > 0 && H % Hkv == 0 && (d == 64 || d == 128) &&
           (long long)B * H <= 0x7fffffffLL && N <= (1 << 24);
}

size_t attn_fwd_workspace_size(int B, int H, int Hkv, int N, int d, int mode)
{
    if (!fwd_sizes_supported(B, H, Hkv, N, d))
        return 0;
    if (mode == ATTN_MODE_SAGE_QK_I8_BLK64_PV_FP8_E4M3)
        return attn::sage_workspace_bytes(B, H, Hkv, N, d);
    if (mode == ATTN_MODE_SAGE3_QK_MXFP4_PV_MXFP4)
        return attn::mx_workspace_bytes(B, H, Hkv, N, d, 4);
    if (mode == ATTN_MODE_SAGE3_QK_MXFP6_PV_MXFP6)
        return attn::mx_workspace_bytes(B, H, Hkv, N, d, 6);
    return 0;
}

attn_status attn_sage_workspace_layout(int B, int H, int Hkv, int N, int d, size_t *offsets)
{
    if (!offsets)
        return fail(ATTN_ERR_INVALID_ARG, "offsets must be non-null");
    if (!fwd_sizes_supported(B, H, Hkv, N, d))
        return fail(ATTN_ERR_INVALID_ARG, "invalid sizes (B=%d H=%d Hkv=%d N=%d d=%d)", B, H, Hkv,
                    N, d);
    attn::sage_workspace_layout(B, H, Hkv, N, d, offsets);
    return ok();
}

attn_status attn_mx_workspace_layout(int B, int H, int Hkv, int N, int d, int mode,
                                     size_t *offsets)
{
    if (!offsets)
        return fail(ATTN_ERR_INVALID_ARG, "offsets must be non-null");
    if (mode != ATTN_MODE_SAGE3_QK_MXFP4_PV_MXFP4 && mode != ATTN_MODE_SAGE3_QK_MXFP6_PV_MXFP6)
        return fail(ATTN_ERR_INVALID_ARG, "mode %d is not an MX mode", mode);
    if (!fwd_sizes_supported(B, H, Hkv, N, d))
        return fail(ATTN_ERR_INVALID_ARG, "invalid sizes (B=%d H=%d Hkv=%d N=%d d=%d)", B, H, Hkv,
                    N, d);
    attn::mx_workspace_layout(B, H, Hkv, N, d,
                              mode == ATTN_MODE_SAGE3_QK_MXFP6_PV_MXFP6 ? 6 : 4, offsets);
    return ok();
}

attn_status attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                     int H, int Hkv, int N, int d, int causal, float scale, int mode,
                     int o_dtype, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!q || !k || !v || !o)
        return fail(ATTN_ERR_INVALID_ARG, "q, k, v and o must be non-null device pointers");
    if (B <= 0 || H <= 0 || Hkv <= 0 || N <= 0 || d <= 0)
        return fail(ATTN_ERR_INVALID_ARG, "sizes must be positive (B=%d H=%d Hkv=%d N=%d d=%d)",
                    B, H, Hkv, N, d);
    if (H % Hkv != 0)
        return fail(ATTN_ERR_INVALID_ARG, "H=%d is not a multiple of Hkv=%d", H, Hkv);
    if (!valid_scale(scale))
        return fail(ATTN_ERR_INVALID_ARG, "scale must be finite and > 0");
    if (o_dtype != ATTN_OUT_BF16 && o_dtype != ATTN_OUT_FP32)
        return fail(ATTN_ERR_INVALID_ARG, "unknown output dtype %d", o_dtype);
    if (mode != ATTN_MODE_EXACT_BF16 && !quant_mode(mode))
        return fail(ATTN_ERR_INVALID_ARG, "unknown mode %d", mode);
    if (d != 64 && d != 128)
        return fail(ATTN_ERR_UNSUPPORTED, "head dim d=%d (supported: 64, 128)", d);
    if ((long long)B * H > 0x7fffffffLL || (long long)N > (1LL << 24))
        return fail(ATTN_ERR_UNSUPPORTED, "problem too large for the grid mapping");
    const size_t need = attn_fwd_workspace_size(B, H, Hkv, N, d, mode);
    if (need && (!workspace || workspace_bytes < need))
        return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);

    const long long nqt = ((long long)N + 255) / 256;
    if (!product_le(B, H, nqt, 0x7fffffffLL))
        return fail(ATTN_ERR_UNSUPPORTED, "problem too large for the grid mapping");
    attn::PrefillArgs a{q, k, v, o, lse, B, H, Hkv, N, d, causal != 0, scale,
                        o_dtype == ATTN_OUT_FP32};
    hipStream_t s = (hipStream_t)stream;
    if (mode == ATTN_MODE_EXACT_BF16)
        return from_hip(attn::launch_prefill_exact(a, s), "prefill launch");
    attn::SageArgs sa{a, workspace, workspace_bytes};
    if (mode == ATTN_MODE_SAGE3_QK_MXFP4_PV_MXFP4)
        return from_hip(attn::launch_mx(sa, 4, s), "mxfp4 launch");
    if (mode == ATTN_MODE_SAGE3_QK_MXFP6_PV_MXFP6)
        return from_hip(attn::launch_mx(sa, 6, s), "mxfp6 launch");
    return from_hip(attn::launch_sage(sa, s), "sage launch");
}

attn_status attn_fwd_varlen(const void *q, const void *k, const void *v, void *o, float *lse,
                            const int32_t *cu_seqlens, int B, int H, int Hkv, int total,
                            int max_seqlen, int d, int causal, float scale, int mode,
                            int o_dtype, void *stream)
{
    if (!q || !k || !v || !o || !cu_seqlens)
        return fail(ATTN_ERR_INVALID_ARG,
                    "q, k, v, o and cu_seqlens must be non-null device pointers");
    if (B <= 0 || H <= 0 || Hkv <= 0 || d <= 0 || total <= 0 || max_seqlen <= 0)
        return fail(ATTN_ERR_INVALID_ARG,
                    "sizes must be positive (B=%d H=%d Hkv=%d d=%d total=%d max_seqlen=%d)", B,
                    H, Hkv, d, total, max_seqlen);
    if (H % Hkv != 0)
        return fail(ATTN_ERR_INVALID_ARG, "H=%d is not a multiple of Hkv=%d", H, Hkv);
    if (!valid_scale(scale))
        return fail(ATTN_ERR_INVALID_ARG, "scale must be finite and > 0");
    if (o_dtype != ATTN_OUT_BF16 && o_dtype != ATTN_OUT_FP32)
        return fail(ATTN_ERR_INVALID_ARG, "unknown output dtype %d", o_dtype);
    if (mode != ATTN_MODE_EXACT_BF16)
        return fail(quant_mode(mode) ? ATTN_ERR_UNSUPPORTED
                        : ATTN_ERR_INVALID_ARG,
                    "the packed variable-length call supports only the exact mode (mode=%d)",
                    mode);
    if (d != 64 && d != 128)
        return fail(ATTN_ERR_UNSUPPORTED, "head dim d=%d (supported: 64, 128)", d);
    const long long nqt = ((long long)max_seqlen + 255) / 256;
    // grid of B*H*(query tiles) workgroups; 64 key rows of one tile must stay
    // within the 32-bit offsets of a buffer resource
    if (!product_le(B, H, nqt, 0x7fffffffLL) || (long long)H * d > (1 << 20) ||
        max_seqlen > (1 << 24))
        return fail(ATTN_ERR_UNSUPPORTED, "problem too large for the grid mapping");
    attn::PrefillArgs a{q, k, v, o, lse, B, H, Hkv, max_seqlen, d, causal != 0, scale,
                        o_dtype == ATTN_OUT_FP32};
    a.cu_seqlens = cu_seqlens;
    a.total = total;
    return from_hip(attn::launch_prefill_exact(a, (hipStream_t)stream), "varlen prefill launch");
}

size_t attn_bwd_workspace_size(int B, int H, int N)
{
    // 0 as well beyond the sizes attn_bwd accepts
    if (B <= 0 || H <= 0 || N <= 0 || N > (1 << 24) || !product_le(B, H, N, 0x7fffffffLL))
        return 0;
    return 2 * align_up(sizeof(float) * (size_t)B * H * attn::bwd_rows(N), 256);
}

attn_status attn_bwd(const void *q, const void *k, const void *v, const void *o,
                     const float *lse, const void *dout, void *dq, void *dk, void *dv, int B,
                     int H, int Hkv, int N, int d, int causal, float scale, int grad_dtype,
                     void *workspace, size_t workspace_bytes, void *stream)
{
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv)
        return fail(ATTN_ERR_INVALID_ARG,
                    "q, k, v, o, lse, dout, dq, dk and dv must be non-null device pointers");
    if (B <= 0 || H <= 0 || Hkv <= 0 || N <= 0 || d <= 0)
        return fail(ATTN_ERR_INVALID_ARG, "sizes must be positive (B=%d H=%d Hkv=%d N=%d d=%d)",
                    B, H, Hkv, N, d);
    if (H % Hkv != 0)
        return fail(ATTN_ERR_INVALID_ARG, "H=%d is not a multiple of Hkv=%d", H, Hkv);
    if (!valid_scale(scale))
        return fail(ATTN_ERR_INVALID_ARG, "scale must be finite and > 0");
    // the kernels work with -lse/scale, which must stay finite
    if (scale < 0x1p-64f)
        return fail(ATTN_ERR_INVALID_ARG, "the backward needs scale >= 2^-64 (got %g)",
                    (double)scale);
    if (grad_dtype != ATTN_OUT_BF16 && grad_dtype != ATTN_OUT_FP32)
        return fail(ATTN_ERR_INVALID_ARG, "unknown gradient dtype %d", grad_dtype);
    if (d != 64 && d != 128)
        return fail(ATTN_ERR_UNSUPPORTED, "head dim d=%d (supported: 64, 128)", d);
    const long long nt = ((long long)N + 127) / 128;
    if (!product_le(B, H, nt, 0x7fffffffLL) || !product_le(B, H, N, 0x7fffffffLL) ||
        N > (1 << 24))
        return fail(ATTN_ERR_UNSUPPORTED, "problem too large for the grid mapping");
    const size_t need = attn_bwd_workspace_size(B, H, N);
    if (!workspace || workspace_bytes < need)
        return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    attn::BwdArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.dout = dout;
    a.lse = lse;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.B = B;
    a.H = H;
    a.Hkv = Hkv;
    a.N = N;
    a.d = d;
    a.causal = causal != 0;
    a.scale = scale;
    a.out_fp32 = grad_dtype == ATTN_OUT_FP32;
    a.ndelta = (float *)workspace;
    a.nlse = (float *)((char *)workspace +
                       align_up(sizeof(float) * (size_t)B * H * attn::bwd_rows(N), 256));
    return from_hip(attn::launch_bwd(a, (hipStream_t)stream), "backward launch");
}

size_t attn_decode_workspace_size(int B, int H, int Hkv, int d)
{
    if (B <= 0 || H <= 0 || Hkv <= 0 || d <= 0 || H % Hkv != 0)
        return 0;
    const size_t slots = attn::decode_partial_slots(B, Hkv);
    const size_t G = (size_t)(H / Hkv);
    return align_up(sizeof(float) * slots * G * d, 256) + align_up(sizeof(float) * slots * G, 256);
}

attn_status attn_decode(const void *q, const void *k_cache, const void *v_cache,
                        const int32_t *seqlens, void *o, float *lse, int B, int H, int Hkv,
                        int N_max, int d, float scale, int mode, int o_dtype, int split_tokens,
                        void *workspace, size_t workspace_bytes, void *stream)
{
    attn::DecodeArgs a;
    const attn_status st = decode_common(q, k_cache, v_cache, seqlens, o, lse, B, H, Hkv, N_max,
                                         d, scale, mode, o_dtype, split_tokens, workspace,
                                         workspace_bytes, a);
    if (st != ATTN_OK)
        return st;
    return from_hip(attn::launch_decode(a, (hipStream_t)stream), "decode launch");
}

attn_status attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                const int32_t *seqlens, void *o, float *lse, int B, int H,
                                int Hkv, int N_max, int d, float scale, int mode, int o_dtype,
                                int split_tokens, void *stream)
{
    attn::DecodeArgs a;
    // every check of attn_decode but the workspace's (a stand-in pointer
    // that is never used: the partials are re-pointed below)
    attn_status st = decode_common(q, k_cache, v_cache, seqlens, o, lse, B, H, Hkv, N_max, d,
                                   scale, mode, o_dtype, split_tokens, (void *)q, SIZE_MAX, a);
    if (st != ATTN_OK)
        return st;
    const size_t need = attn_decode_workspace_size(B, H, Hkv, d);
    if (need > ATTN_DECODE_SCRATCH_BYTES)
        return fail(ATTN_ERR_UNSUPPORTED,
                    "attn_decode_noalloc: the partials need %zu bytes, the library's fixed "
                    "array holds %zu (use attn_decode with a workspace)",
                    need, (size_t)ATTN_DECODE_SCRATCH_BYTES);
    void *scratch = nullptr;
    st = from_hip(attn::decode_scratch(&scratch), "attn_decode_noalloc scratch address");
    if (st != ATTN_OK)
        return st;
    set_partials(a, scratch);
    return from_hip(attn::launch_decode(a, (hipStream_t)stream), "decode launch");
}

attn_status attn_decode_paged(const void *q, const void *k_pages, const void *v_pages,
                              const int32_t *block_table, const int32_t *seqlens, void *o,
                              float *lse, int B, int H, int Hkv, int num_pages, int page_size,
                              int max_pages, int d, float scale, int mode, int o_dtype,
                              int split_tokens, void *workspace, size_t workspace_bytes,
                              void *stream)
{
    if (!block_table)
        return fail(ATTN_ERR_INVALID_ARG, "block_table must be a non-null device pointer");
    if (num_pages <= 0 || max_pages <= 0)
        return fail(ATTN_ERR_INVALID_ARG, "num_pages=%d and max_pages=%d must be positive",
                    num_pages, max_pages);
    if (page_size <= 0 || (page_size & (page_size - 1)) != 0)
        return fail(ATTN_ERR_INVALID_ARG, "page_size=%d is not a power of two", page_size);
    if (page_size < 16)
        return fail(ATTN_ERR_UNSUPPORTED, "page_size=%d (supported: >= 16)", page_size);
    const long long n_max = (long long)max_pages * page_size;
    if (n_max > 0x7fffffffLL)
        return fail(ATTN_ERR_UNSUPPORTED, "max_pages * page_size = %lld exceeds 2^31 - 1", n_max);
    attn::DecodeArgs a;
    const attn_status st = decode_common(q, k_pages, v_pages, seqlens, o, lse, B, H, Hkv,
                                         (int)n_max, d, scale, mode, o_dtype, split_tokens,
                                         workspace, workspace_bytes, a);
    if (st != ATTN_OK)
        return st;
    a.block_table = block_table;
    a.page_shift = __builtin_ctz((unsigned)page_size);
    a.max_pages = max_pages;
    a.num_pages = num_pages;
    return from_hip(attn::launch_decode(a, (hipStream_t)stream), "paged decode launch");
}

attn_status attn_profiler_enable(int enable)
{
    prof_release();
    g_prof_on = false;
    if (enable) {
        if (!prof_grow(kProfReserve)) {
            prof_release();
            return fail(ATTN_ERR_HIP, "profiler: hipEventCreate failed");
        }
        g_prof_on = true;
    }
    return ok();
}

int attn_profiler_read(char *names, int name_stride, double *total_ms, int *launches, int cap)
{
    if (!names || !total_ms || !launches || name_stride <= 1 || cap <= 0)
        return fail(ATTN_ERR_INVALID_ARG, "profiler_read: bad output buffers");
    std::vector<std::string> seen;
    std::vector<double> tot;
    std::vector<int> cnt;
    attn_status st = ATTN_OK;
    for (size_t j = 0; j < g_prof_used; ++j) {
        const ProfEvent &ev = g_prof[j];
        float ms = 0.f;
        hipError_t e = hipEventSynchronize(ev.end);
        if (e == hipSuccess)
            e = hipEventElapsedTime(&ms, ev.begin, ev.end);
        if (e != hipSuccess) {
            st = fail(ATTN_ERR_HIP, "profiler_read: %s", hipGetErrorString(e));
            break;
        }
        size_t i = 0;
        while (i < seen.size() && seen[i] != ev.name)
            ++i;
        if (i == seen.size()) {
            seen.push_back(ev.name);
            tot.push_back(0.0);
            cnt.push_back(0);
        }
        tot[i] += ms;
        cnt[i] += 1;
    }
    g_prof_used = 0;  // the pool is kept for the next run
    if (st != ATTN_OK)
        return st;
    int n = (int)seen.size() < cap ? (int)seen.size() : cap;
    for (int i = 0; i < n; ++i) {
        std::snprintf(names + (size_t)i * name_stride, name_stride, "%s", seen[i].c_str());
        total_ms[i] = tot[i];
        launches[i] = cnt[i];
    }
    ok();
    return n;
}

int attn_profiler_launches(char *names, int name_stride, float *ms, int cap)
{
    if (!names || !ms || name_stride <= 1 || cap <= 0)
        return fail(ATTN_ERR_INVALID_ARG, "profiler_launches: bad output buffers");
    const int n = (int)g_prof_used < cap ? (int)g_prof_used : cap;
    attn_status st = ATTN_OK;
    for (int j = 0; j < n; ++j) {
        const ProfEvent &ev = g_prof[j];
        hipError_t e = hipEventSynchronize(ev.end);
        if (e == hipSuccess)
            e = hipEventElapsedTime(&ms[j], ev.begin, ev.end);
        if (e != hipSuccess) {
            st = fail(ATTN_ERR_HIP, "profiler_launches: %s", hipGetErrorString(e));
            break;
        }
        std::snprintf(names + (size_t)j * name_stride, name_stride, "%s", ev.name);
    }
    g_prof_used = 0;
    if (st != ATTN_OK)
        return st;
    ok();
    return n;
}

}  // extern "C"
