// Split-KV GQA decode for gfx950 (Flash-Decoding, "flashattention-kernels"
// page §3; GQA from the "cuda-kernel-pretrain" page §3).
//
// decode_split_kernel: one workgroup per (chunk, kv head, sequence).  It
// streams its chunk of the K and V caches exactly once for all G = H/Hkv query
// heads of the group (the GQA saving: each cache byte is read once per group,
// not once per query head), computes the chunk's scores, a local softmax and
// the partial output O_s with its log2-domain LSE.  Workgroups whose chunk
// starts at or beyond the sequence length exit at once.
//
// decode_merge_kernel: one workgroup per (sequence, query head) combines the
// chunk partials with log-sum-exp weights into O and the natural-log LSE.
//
// The path is HBM bound (a few FLOPs per byte), so the kernels use plain fp32
// VALU arithmetic and spend their effort on memory: 16-byte coalesced loads
// (16 lanes read one 256-byte cache row), eight loads in flight per thread,
// and no register spills.
#include "attn_internal.hpp"
#include "cdna4.hpp"

namespace attn {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr int kHeadsPerPass = 4;  // heads reduced per LDS pass

// LDS bytes of decode_split_kernel: scores [G][S], row-group partials
// [RPP][min(G,4)][D], per-head max and sum.
inline size_t split_lds_bytes(int D, int G, int S)
{
    const int rpp = kThreads / (D / 8);
    const int hp = G < kHeadsPerPass ? G : kHeadsPerPass;
    return sizeof(float) * ((size_t)G * S + (size_t)rpp * hp * D + 2 * G);
}

template <int TPR>
__device__ __forceinline__ float group_sum(float x)
{
#pragma unroll
    for (int off = 1; off < TPR; off <<= 1)
        x += __shfl_xor(x, off, 64);
    return x;
}

__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int off = 1; off < 64; off <<= 1)
        x = fmaxf(x, __shfl_xor(x, off, 64));
    return x;
}

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int off = 1; off < 64; off <<= 1)
        x += __shfl_xor(x, off, 64);
    return x;
}

__device__ __forceinline__ int clamp_len(const int32_t *seqlens, int b, int n_max)
{
    int L = seqlens[b];
    return L < 1 ? 1 : (L > n_max ? n_max : L);
}

// Dynamic LDS: see split_lds_bytes().
template <int D, int G>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a)
{
    constexpr int TPR = D / 8;           // threads per cache row (16 bytes each)
    constexpr int RPP = kThreads / TPR;  // rows per pass
    extern __shared__ __attribute__((aligned(16))) float lds[];
    const int S = a.split_tokens;
    float *sc = lds;                  // [G][S]
    constexpr int HP = G < kHeadsPerPass ? G : kHeadsPerPass;
    float *red = lds + G * S;          // [RPP][HP][D]
    float *stat = red + RPP * HP * D;  // [2][G]

    const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int L = clamp_len(a.seqlens, b, a.N_max);
    const int c0 = split * S;
    if (c0 >= L)
        return;
    const int n = min(S, L - c0);
    const int tid = threadIdx.x, fc = tid % TPR, rg = tid / TPR;
    const int wave = tid >> 6, lane = tid & 63;
    const size_t cache_off = ((size_t)(b * a.Hkv + kvh) * a.N_max + c0) * D;
    const uint16_t *kb = (const uint16_t *)a.k + cache_off;
    const uint16_t *vb = (const uint16_t *)a.v + cache_off;
    const float cs = a.scale * kLog2e;

    // q fragment of every head of the group, features fc*8 .. fc*8+7
    float qv[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        u32x4 w = ld16((const uint16_t *)a.q + ((size_t)b * a.H + kvh * G + h) * D + fc * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qv[h][2 * e] = bf16_lo(w[e]) * cs;
            qv[h][2 * e + 1] = bf16_hi(w[e]) * cs;
        }
    }

    // scores (log2 domain) of every key of the chunk
    for (int r0 = 0; r0 < n; r0 += RPP * kUnroll) {
        u32x4 kw[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            int row = r0 + u * RPP + rg;
            kw[u] = row < n ? ld16(kb + (size_t)row * D + fc * 8) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            int row = r0 + u * RPP + rg;
            float kf[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kf[2 * e] = bf16_lo(kw[u][e]);
                kf[2 * e + 1] = bf16_hi(kw[u][e]);
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float dot = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    dot = fmaf(qv[h][e], kf[e], dot);
                dot = group_sum<TPR>(dot);
                if (fc == 0 && row < n)
                    sc[h * S + row] = dot;
            }
        }
    }
    __syncthreads();

    // chunk-local softmax per head: p = 2^(s - m), l = sum p
    for (int h = wave; h < G; h += kThreads / 64) {
        float mx = -INFINITY;
        for (int j = lane; j < n; j += 64)
            mx = fmaxf(mx, sc[h * S + j]);
        mx = wave_max(mx);
        float sum = 0.f;
        for (int j = lane; j < n; j += 64) {
            float p = fast_exp2(sc[h * S + j] - mx);
            sc[h * S + j] = p;
            sum += p;
        }
        sum = wave_sum(sum);
        if (lane == 0) {
            stat[h] = mx;
            stat[G + h] = sum;
        }
    }
    __syncthreads();

    // partial P V: thread accumulates features fc*8..+7 over rows rg, rg+RPP, ...
    float acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[h][e] = 0.f;
    for (int r0 = 0; r0 < n; r0 += RPP * kUnroll) {
        u32x4 vw[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            int row = r0 + u * RPP + rg;
            vw[u] = row < n ? ld16(vb + (size_t)row * D + fc * 8) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            int row = r0 + u * RPP + rg;
            if (row < n) {
                float vf[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    vf[2 * e] = bf16_lo(vw[u][e]);
                    vf[2 * e + 1] = bf16_hi(vw[u][e]);
                }
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    float p = sc[h * S + row];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        acc[h][e] = fmaf(p, vf[e], acc[h][e]);
                }
            }
        }
    }
    // reduce the RPP row-group partials through LDS, four heads at a time
#pragma unroll
    for (int hg = 0; hg < G; hg += kHeadsPerPass) {
#pragma unroll
        for (int hh = 0; hh < HP; ++hh)
#pragma unroll
            for (int e = 0; e < 8; e += 4)
                *(f32x4 *)(red + ((size_t)rg * HP + hh) * D + fc * 8 + e) =
                    f32x4{acc[hg + hh][e], acc[hg + hh][e + 1], acc[hg + hh][e + 2],
                          acc[hg + hh][e + 3]};
        __syncthreads();
        for (int idx = tid; idx < HP * D; idx += kThreads) {
            const int hh = idx / D, dd = idx % D, h = hg + hh;
            float sum = 0.f;
#pragma unroll 4
            for (int r = 0; r < RPP; ++r)
                sum += red[((size_t)r * HP + hh) * D + dd];
            const float l = stat[G + h];
            const size_t pidx = ((size_t)b * a.H + kvh * G + h) * a.max_splits + split;
            a.part_o[pidx * D + dd] = sum / l;
            if (dd == 0)
                a.part_lse[pidx] = stat[h] + log2f(l);
        }
        __syncthreads();
    }
}

template <int D, bool OUT_F32>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecodeArgs a)
{
    const int bh = blockIdx.x, b = bh / a.H, dd = threadIdx.x;
    const int L = clamp_len(a.seqlens, b, a.N_max);
    const int ns = (L + a.split_tokens - 1) / a.split_tokens;
    const float *pl = a.part_lse + (size_t)bh * a.max_splits;
    const float *po = a.part_o + (size_t)bh * a.max_splits * D;
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s)
        M = fmaxf(M, pl[s]);
    float wsum = 0.f, acc = 0.f;
    for (int s = 0; s < ns; ++s) {
        const float w = fast_exp2(pl[s] - M);
        wsum += w;
        acc = fmaf(w, po[(size_t)s * D + dd], acc);
    }
    const float out = acc / wsum;
    if constexpr (OUT_F32)
        ((float *)a.o)[(size_t)bh * D + dd] = out;
    else
        ((__bf16 *)a.o)[(size_t)bh * D + dd] = (__bf16)out;
    if (a.lse && dd == 0)
        a.lse[bh] = (M + log2f(wsum)) * kLn2;
}

template <int D, int G>
hipError_t launch_split(const DecodeArgs &a, hipStream_t s)
{
    const size_t lds = split_lds_bytes(D, G, a.split_tokens);
    dim3 grid(a.max_splits, a.Hkv, a.B);
    ProfScope ps("decode_split", s);
    hipLaunchKernelGGL((decode_split_kernel<D, G>), grid, dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs &a, hipStream_t s)
{
    hipError_t e;
    switch (a.H / a.Hkv) {
    case 1: e = launch_split<D, 1>(a, s); break;
    case 2: e = launch_split<D, 2>(a, s); break;
    case 4: e = launch_split<D, 4>(a, s); break;
    default: e = launch_split<D, 8>(a, s); break;
    }
    if (e != hipSuccess)
        return e;
    ProfScope ps("decode_merge", s);
    if (a.out_fp32)
        hipLaunchKernelGGL((decode_merge_kernel<D, true>), dim3(a.B * a.H), dim3(D), 0, s, a);
    else
        hipLaunchKernelGGL((decode_merge_kernel<D, false>), dim3(a.B * a.H), dim3(D), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s)
{
    return a.d == 64 ? launch_d<64>(a, s) : launch_d<128>(a, s);
}

}  // namespace attn
