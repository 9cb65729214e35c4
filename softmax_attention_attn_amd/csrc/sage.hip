// SageAttention-style quantised attention forward for gfx950.
//
// The recipe ("GPU kernel overview" page: SageAttention chain, Smooth-K, and
// the insight that QK^T suits symmetric INT8 while PV suits FP8 E4M3):
//   1. Smooth-K: K' = K - kmean, kmean the per-channel mean of K over all N
//      tokens of the (batch, kv head) (fp32);
//   2. Q and K' quantised to INT8 per block of 64 consecutive tokens of one
//      (batch, head): delta = max|x| / 127, x^ = rint(x / delta) in [-127, 127];
//   3. V quantised per (batch, kv head, channel) to E4M3 with
//      delta_V = max_n |V| / 448;
//   4. S = scale * dQ * dK * (Q^ K^^T) with exact int32 accumulation;
//   5. online softmax over 64-key tiles with the exact running max m:
//      P^ = E4M3(448 * 2^(S*log2e - m)) (<= 448 by construction), the row sum
//      l over the unquantised values, O += P^ V^ in fp32 (FP8 MFMA);
//   6. O = O * delta_V / l;  lse = m + ln l + scale * (q . kmean), the true LSE
//      (Smooth-K shifts every score of row i by the constant -scale*q_i.kmean,
//      which leaves O unchanged).
//
// Kernels (all launched by launch_sage on one stream):
//   sage_stats      partial per-channel sums of K and maxima of |V| per chunk
//   sage_finalize   kmean and the V scales from the partials
//   sage_quant_qk   INT8 blocks of Q and K' (and q . kmean per query row)
//   sage_quant_v    E4M3 V, written transposed (feature-major) per 64-key tile
//   sage_attn       the fused quantised attention
//
// sage_attn follows the exact kernel's mapping: 8 waves x 32 queries per
// workgroup, S^T = K^ Q^^T with v_mfma_i32_32x32x32_i8 (keys are MFMA rows;
// K rows are taken in perm32 order so that lane half g holds keys 16g..16g+15
// of each 32-key block), O^T += V^^T P^^T with the FP8 MFMA
// v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales): the 32 FP8
// probabilities a lane holds (keys 16g+r and 32+16g+r) are directly its B
// operand, and its A operand is the matching 32 bytes of two feature rows of
// the transposed V tile.  Key tiles equal the 64-token quantisation blocks,
// so dK is one scalar per tile and dQ one scalar per wave.
#include "../../include/attn.h"
#include "attn_internal.hpp"
#include "cdna4.hpp"

namespace attn {
namespace {

constexpr int kBlk = 64;   // quantisation block = key tile (tokens)
constexpr int kNCh = 16;   // sequence chunks of the statistics pass
constexpr int kThreads = 256;
constexpr float kLog2_448 = 8.807354922057604f;

// Biased integer scores.  Every QK accumulator starts at the bit pattern of
// the float 1.5 * 2^23 instead of zero.  A score is at most 128 * 127^2 <
// 2^22 in magnitude, so the int32 result stays inside that float's binade and
// its bits read as the float 1.5 * 2^23 + s exactly: the scaled exponent
// c * s + bias is then one FMA on the raw bits, c * bits + (bias - 1.5 * 2^23
// * c), with no int-to-float conversion.  Signed integer order of the biased
// scores is still score order (all of them are positive ints).  A masked score
// is set to the bits of -inf, a negative int below every real score, and its
// exponent c * (-inf) + bias' is -inf, so p = 0 with no per-score test.
constexpr int kSBias = 0x4B400000;       // bits of 12582912.0f = 1.5 * 2^23
constexpr float kSBiasF = 12582912.f;
constexpr int kSMasked = (int)0xFF800000u;  // bits of -inf

// The bias block is built once per query tile and kept in registers (the
// empty asm hides its value), so the first MFMA of every score block reads it
// as its accumulator input instead of a fresh copy being made each tile.
__device__ __forceinline__ i32x16 sbias16()
{
    i32x16 v;
#pragma unroll
    for (int r = 0; r < 16; ++r)
        v[r] = kSBias;
    asm volatile("" : "+v"(v));
    return v;
}

// the lane's biased integer max in log2 units (-inf when every key is masked)
__device__ __forceinline__ float smax_log2(int imx, float c)
{
    return imx < 0 ? -INFINITY : (__int_as_float(imx) - kSBiasF) * c;
}

// the per-tile constant of the exponent for biased scores
__device__ __forceinline__ float sbias_exp(float bias, float c) { return fmaf(-kSBiasF, c, bias); }

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

struct SageWs {
    double *ksum_part; // [BG][kNCh][D]  (fp64: kmean rounds to fp32 exactly as an fp64 mean)
    float *vmax_part;  // [BG][kNCh][D]
    float *kmean;      // [BG][D]
    float *vscale;     // [BG][D]   delta_V
    float *vinv;       // [BG][D]   1 / delta_V = 448 / max|V|
    float *qdelta;     // [BH][nblk]
    float *kdelta;     // [BG][nblk]
    float *qkdot;      // [BH][N]   q_i . kmean
    int8_t *qhat;      // [BH][Npad][D]
    int8_t *khat;      // [BG][Npad][D]
    uint8_t *vhatT;    // [BG][D][Npad]  E4M3 codes, feature-major
};

// Byte offsets of the workspace pieces, in SageWsPiece order; the last entry
// is the total size.
static_assert(ATTN_SAGE_WS_COUNT == kSageWsPieces, "workspace pieces");

void layout(int B, int H, int Hkv, int N, int d, size_t (&off)[kSageWsPieces + 1])
{
    const size_t BH = (size_t)B * H, BG = (size_t)B * Hkv;
    const size_t nblk = ((size_t)N + kBlk - 1) / kBlk, Npad = nblk * kBlk;
    const size_t bytes[kSageWsPieces] = {
        sizeof(double) * BG * kNCh * d,  // ATTN_SAGE_WS_KSUM_PART
        sizeof(float) * BG * kNCh * d,   // ATTN_SAGE_WS_VMAX_PART
        sizeof(float) * BG * d,          // ATTN_SAGE_WS_KMEAN
        sizeof(float) * BG * d,          // ATTN_SAGE_WS_VSCALE
        sizeof(float) * BG * d,          // ATTN_SAGE_WS_VINV
        sizeof(float) * BH * nblk,       // ATTN_SAGE_WS_QDELTA
        sizeof(float) * BG * nblk,       // ATTN_SAGE_WS_KDELTA
        sizeof(float) * BH * N,          // ATTN_SAGE_WS_QKDOT
        BH * Npad * d,                   // ATTN_SAGE_WS_QHAT
        BG * Npad * d,                   // ATTN_SAGE_WS_KHAT
        BG * d * Npad,                   // ATTN_SAGE_WS_VHATT
    };
    size_t p = 0;
    for (int i = 0; i < kSageWsPieces; ++i) {
        off[i] = p;
        p += align256(bytes[i]);
    }
    off[kSageWsPieces] = p;
}

SageWs carve(void *base, int B, int H, int Hkv, int N, int d)
{
    size_t off[kSageWsPieces + 1];
    layout(B, H, Hkv, N, d, off);
    char *p = (char *)base;
    SageWs w;
    w.ksum_part = (double *)(p + off[ATTN_SAGE_WS_KSUM_PART]);
    w.vmax_part = (float *)(p + off[ATTN_SAGE_WS_VMAX_PART]);
    w.kmean = (float *)(p + off[ATTN_SAGE_WS_KMEAN]);
    w.vscale = (float *)(p + off[ATTN_SAGE_WS_VSCALE]);
    w.vinv = (float *)(p + off[ATTN_SAGE_WS_VINV]);
    w.qdelta = (float *)(p + off[ATTN_SAGE_WS_QDELTA]);
    w.kdelta = (float *)(p + off[ATTN_SAGE_WS_KDELTA]);
    w.qkdot = (float *)(p + off[ATTN_SAGE_WS_QKDOT]);
    w.qhat = (int8_t *)(p + off[ATTN_SAGE_WS_QHAT]);
    w.khat = (int8_t *)(p + off[ATTN_SAGE_WS_KHAT]);
    w.vhatT = (uint8_t *)(p + off[ATTN_SAGE_WS_VHATT]);
    return w;
}

// ----------------------------------------------------------------- prologue

// Partial per-channel sum of K and max |V| over one sequence chunk.  Thread t
// reads 16 bytes (8 channels) of rows t / (D/8), t / (D/8) + 256/(D/8), ...
template <int D>
__global__ __launch_bounds__(kThreads) void sage_stats_kernel(const uint16_t *k, const uint16_t *v,
                                                              SageWs w, int N)
{
    constexpr int TPR = D / 8, RPP = kThreads / TPR;
    __shared__ double red_s[RPP][D];
    __shared__ float red_m[RPP][D];
    const int bg = blockIdx.x, chunk = blockIdx.y, tid = threadIdx.x;
    const int fc = tid % TPR, rg = tid / TPR;
    const int len = (N + kNCh - 1) / kNCh;
    const int r0 = chunk * len, r1 = min(N, r0 + len);
    const uint16_t *kb = k + (size_t)bg * N * D, *vb = v + (size_t)bg * N * D;
    double ks[8] = {};
    float vm[8] = {};
    // unrolled, so that several rows' loads are in flight per thread
#pragma unroll 4
    for (int r = r0 + rg; r < r1; r += RPP) {
        const u32x4 kw = ld16_nt(kb + (size_t)r * D + fc * 8);
        const u32x4 vw = ld16_nt(vb + (size_t)r * D + fc * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ks[2 * e] += bf16_lo(kw[e]);
            ks[2 * e + 1] += bf16_hi(kw[e]);
            vm[2 * e] = fmaxf(vm[2 * e], fabsf(bf16_lo(vw[e])));
            vm[2 * e + 1] = fmaxf(vm[2 * e + 1], fabsf(bf16_hi(vw[e])));
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        red_s[rg][fc * 8 + e] = ks[e];
        red_m[rg][fc * 8 + e] = vm[e];
    }
    __syncthreads();
    for (int c = tid; c < D; c += kThreads) {
        double s = 0.0;
        float m = 0.f;
        for (int r = 0; r < RPP; ++r) {
            s += red_s[r][c];
            m = fmaxf(m, red_m[r][c]);
        }
        w.ksum_part[((size_t)bg * kNCh + chunk) * D + c] = s;
        w.vmax_part[((size_t)bg * kNCh + chunk) * D + c] = m;
    }
}

// kmean = sum / N (fp64, rounded to fp32); delta_V = max|V| / 448 and its
// inverse 448 / max|V| (both 1 for an all-zero channel).
template <int D>
__global__ __launch_bounds__(D) void sage_finalize_kernel(SageWs w, int N)
{
    const int bg = blockIdx.x, c = threadIdx.x;
    double s = 0.0;
    float m = 0.f;
    for (int i = 0; i < kNCh; ++i) {
        s += w.ksum_part[((size_t)bg * kNCh + i) * D + c];
        m = fmaxf(m, w.vmax_part[((size_t)bg * kNCh + i) * D + c]);
    }
    w.kmean[(size_t)bg * D + c] = (float)(s / (double)N);
    w.vscale[(size_t)bg * D + c] = m > 0.f ? m / 448.f : 1.f;
    w.vinv[(size_t)bg * D + c] = m > 0.f ? 448.f / m : 1.f;
}

__device__ __forceinline__ float block_max_256(float x, float *scratch)
{
#pragma unroll
    for (int off = 1; off < 64; off <<= 1)
        x = fmaxf(x, __shfl_xor(x, off, 64));
    if ((threadIdx.x & 63) == 0)
        scratch[threadIdx.x >> 6] = x;
    __syncthreads();
    x = fmaxf(fmaxf(scratch[0], scratch[1]), fmaxf(scratch[2], scratch[3]));
    return x;
}

__device__ __forceinline__ int q_i8(float x, float inv)
{
    float r = __builtin_rintf(x * inv);
    r = fminf(fmaxf(r, -127.f), 127.f);
    return (int)r;
}

// One 64-token block of Q (blockIdx.x < BH*nblk) or of K' = K - kmean.
// The block is 64 rows of D bf16 (CR = D/8 16-byte chunks per row); thread t
// takes chunks t, t + 256, ...: every load and store instruction of a wave
// covers one contiguous run of memory, and a thread's channels are the same
// 8 in every chunk (256 is a multiple of CR).
template <int D>
__global__ __launch_bounds__(kThreads) void sage_quant_qk_kernel(const uint16_t *q, const uint16_t *k,
                                                                 SageWs w, int B, int H, int Hkv,
                                                                 int N)
{
    constexpr int CR = D / 8;               // chunks per row
    constexpr int NCH = kBlk * CR / kThreads;  // chunks per thread
    static_assert(kThreads % CR == 0 && NCH * kThreads == kBlk * CR, "chunk split");
    __shared__ float scratch[4];
    const int nblk = (N + kBlk - 1) / kBlk, Npad = nblk * kBlk;
    const int tid = threadIdx.x, c0 = (tid % CR) * 8;
    int id = blockIdx.x;
    const bool is_q = id < B * H * nblk;
    if (!is_q)
        id -= B * H * nblk;
    const int seq = id / nblk, blk = id % nblk;  // seq = b*H + h or b*Hkv + g
    const int tok0 = blk * kBlk;
    const uint16_t *src = (is_q ? q : k) + ((size_t)seq * N + tok0) * D;
    const int g = is_q ? (seq / H) * Hkv + (seq % H) / (H / Hkv) : seq;
    float km[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        km[e] = w.kmean[(size_t)g * D + c0 + e];

    float x[NCH][8];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int chunk = kThreads * j + tid, row = chunk / CR;
        u32x4 u = {0, 0, 0, 0};
        if (tok0 + row < N)
            u = ld16(src + (size_t)chunk * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[j][2 * e] = bf16_lo(u[e]);
            x[j][2 * e + 1] = bf16_hi(u[e]);
        }
    }
    if (is_q) {
        // q . kmean per row, for the LSE correction: CR consecutive lanes
        // hold one row
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                dot = fmaf(x[j][e], km[e], dot);
#pragma unroll
            for (int off = 1; off < CR; off <<= 1)
                dot += __shfl_xor(dot, off, 64);
            const int row = (kThreads * j + tid) / CR;
            if (tid % CR == 0 && tok0 + row < N)
                w.qkdot[(size_t)seq * N + tok0 + row] = dot;
        }
    } else {
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            if (tok0 + (kThreads * j + tid) / CR < N) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    x[j][e] -= km[e];
            }
        }
    }
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < NCH; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            amax = fmaxf(amax, fabsf(x[j][e]));
    amax = block_max_256(amax, scratch);
    const float inv = amax > 0.f ? 127.f / amax : 1.f;
    if (tid == 0)
        (is_q ? w.qdelta : w.kdelta)[(size_t)seq * nblk + blk] = amax > 0.f ? amax / 127.f : 1.f;
    int8_t *dst = (is_q ? w.qhat : w.khat) + ((size_t)seq * Npad + tok0) * D;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        uint32_t out[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
            out[h] = (uint32_t)(q_i8(x[j][4 * h], inv) & 0xff) |
                     ((uint32_t)(q_i8(x[j][4 * h + 1], inv) & 0xff) << 8) |
                     ((uint32_t)(q_i8(x[j][4 * h + 2], inv) & 0xff) << 16) |
                     ((uint32_t)(q_i8(x[j][4 * h + 3], inv) & 0xff) << 24);
        *(uint2 *)(dst + (size_t)(kThreads * j + tid) * 8) = make_uint2(out[0], out[1]);
    }
}

// E4M3 of V / delta_V (round to nearest even, saturated to +-448) for one
// 64-key tile, written feature-major: vhatT[bg][c][tile*64 + key].  Thread t
// takes channels 8 (t % CR) .. +7 of the 4 consecutive tokens 4 (t / CR) ..
// +3 (CR = D/8: 256 threads cover the 64 tokens when D = 128, the first 128
// when D = 64); a channel's 4 bytes form one word, written to LDS rows of 68
// bytes (the 17-word pitch spreads a wave's words over the banks), then whole
// 16-byte runs of a channel go out.
template <int D>
__global__ __launch_bounds__(kThreads) void sage_quant_v_kernel(const uint16_t *v, SageWs w, int N)
{
    constexpr int CR = D / 8;         // 16-byte chunks per row
    constexpr int kPitch = kBlk + 4;  // bytes per LDS row (channel)
    static_assert(kBlk / 4 * CR <= kThreads, "one group of 4 tokens per thread");
    __shared__ __attribute__((aligned(16))) uint32_t tile[D * kPitch / 4];
    const int nblk = (N + kBlk - 1) / kBlk, Npad = nblk * kBlk;
    const int bg = blockIdx.x, blk = blockIdx.y, tid = threadIdx.x;
    const int c0 = (tid % CR) * 8;
    float vi[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        vi[e] = w.vinv[(size_t)bg * D + c0 + e];
    const int tg = tid / CR;  // tokens 4tg .. 4tg+3
    if (tg < kBlk / 4) {
        u32x4 u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tok = blk * kBlk + 4 * tg + i;
            u[i] = u32x4{0, 0, 0, 0};
            if (tok < N)
                u[i] = ld16(v + ((size_t)bg * N + tok) * D + c0);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float f = (e & 1) ? bf16_hi(u[i][e >> 1]) : bf16_lo(u[i][e >> 1]);
                x[i] = fminf(fmaxf(f * vi[e], -448.f), 448.f);
            }
            int wd = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
            wd = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], wd, true);
            tile[((c0 + e) * kPitch + 4 * tg) / 4] = (uint32_t)wd;
        }
    }
    __syncthreads();
    // D rows x 64 bytes = D*4 runs of 16 bytes
    for (int i = tid; i < D * 4; i += kThreads) {
        const int c = i >> 2, part = i & 3;
        const uint32_t *r = tile + (c * kPitch + part * 16) / 4;
        st16(w.vhatT + ((size_t)bg * D + c) * Npad + blk * kBlk + part * 16,
             u32x4{r[0], r[1], r[2], r[3]});
    }
}

// ----------------------------------------------------------------- attention

constexpr int kWaves = 8;
constexpr int kAThreads = 64 * kWaves;
constexpr int kQW = 32;
constexpr int kBM = kQW * kWaves;

template <int D>
struct SCfg {
    static constexpr int kKChunks = D / 16;       // 16-byte chunks of a K^ row
    static constexpr int kKBytes = kBlk * D;      // K^ tile (int8)
    static constexpr int kVBytes = D * kBlk;      // V^^T tile (e4m3, feature-major)
    static constexpr int kKPieces = kKBytes / 1024;
    static constexpr int kVPieces = kVBytes / 1024;
    static constexpr int kNC = D / 32;            // 32-feature blocks of O (PV MFMAs per tile)
    static constexpr int kNQK = 2 * (D / 32);     // QK MFMAs per tile
    static_assert(kKPieces <= kWaves && kVPieces <= kWaves, "at most one direct load per wave");
};

// K^ tile: 16-byte chunk index XOR swizzle by row, so the 16 perm32 rows
// read together by lanes 0..15 fall on distinct bank slots.
template <int D>
__device__ __forceinline__ int kswz(int row)
{
    return (((row >> 1) & 3) | (((row >> 4) & 1) << 2)) & (SCfg<D>::kKChunks - 1);
}
// V^^T tile (64-byte rows = 4 chunks): chunk XOR by feature row.
__device__ __forceinline__ int vswz(int d) { return ((d >> 2) & 1) | (((d >> 4) & 1) << 1); }

// Slot schedule of one pipeline step: slots 0 .. NQK-1 issue the INT8 QK
// MFMAs of tile t+2 (slot i: key block i % 2, k-step i / 2), slots NQK ..
// NS-1 the FP8 PV MFMAs of tile t (feature block c = slot - NQK).  A PV MFMA
// takes twice as long as a QK MFMA, so it carries twice the VALU work: the
// 32 scores of tile t+1 are spread by weight (1 per QK slot, 2 per PV slot).
// The integer max of tile t+2 runs in the PV slots after the first.
template <int D>
struct SSched {
    static constexpr int NQK = SCfg<D>::kNQK, NS = NQK + SCfg<D>::kNC, RA = 2;
    static constexpr int weight(int s) { return s < NQK ? 1 : 2; }
    static constexpr int wsum(int s)
    {
        int w = 0;
        for (int i = 0; i < s && i < NS; ++i)
            w += weight(i);
        return w;
    }
    static constexpr int first_score(int s) { return s >= NS ? 32 : wsum(s) * 32 / wsum(NS); }
    static constexpr int nops(int s) { return s < NQK ? 1 : 2; }  // LDS reads of slot s
    static constexpr int after(int s)
    {
        int n = 0;
        for (int j = s + 1; j <= s + RA && j < NS; ++j)
            n += nops(j);
        return n;
    }
    static constexpr int max_slot(int k) { return NQK + 1 + k * (NS - NQK - 1) / 16; }
    static constexpr int dma_slot(int d) { return 1 + d * (NS - 2) / 2; }  // d = 0: K, 1: V
};

// Per-lane LDS read offsets within a stage.
template <int D>
struct SLanes {
    uint32_t k[D / 32];  // K^ operand of k-step ks: row perm32(n), chunk (2ks+g) ^ kswz
    uint32_t vlo, vhi;   // V^^T operand: feature row perm32(n), chunks g ^ vswz and (2+g) ^ vswz
};

template <int D>
__device__ __forceinline__ SLanes<D> s_lanes(int lane)
{
    const int g = lane >> 5, n = lane & 31;
    const int row = perm32(n), sw = kswz<D>(row), vs = vswz(row);
    SLanes<D> o;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
        o.k[ks] = row * D + (((2 * ks + g) ^ sw) << 4);
    o.vlo = row * kBlk + ((g ^ vs) << 4);
    o.vhi = row * kBlk + (((2 + g) ^ vs) << 4);
    return o;
}

// Per-lane global byte offsets of this wave's direct loads (one 1 KB piece
// of the K^ tile and one of the V^^T tile per wave).
template <int D>
struct SDma {
    uint32_t k, v;
};

template <int D>
__device__ __forceinline__ SDma<D> s_dma(int wave, int lane, int Npad)
{
    constexpr int C = SCfg<D>::kKChunks;
    const int q = wave * 64 + lane;
    SDma<D> o;
    {
        const int row = q / C;
        o.k = row * D + (((q % C) ^ kswz<D>(row)) << 4);
    }
    {
        const int d = q >> 2;
        o.v = d * Npad + (((q & 3) ^ vswz(d)) << 4);
    }
    return o;
}

// S^T = K^ Q^^T for one tile, unpipelined (the first two tiles of a query tile).
template <int D>
__device__ __forceinline__ void qk_tile_i8(i32x16 (&s)[2], const i32x4 (&qf)[D / 32], uint32_t kst,
                                           const SLanes<D> &ln, const i32x16 &sbias)
{
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
        u32x4 a0 = lds_read_b128<0>(kst + ln.k[ks]);
        u32x4 a1 = lds_read_b128<32 * D>(kst + ln.k[ks]);
        lgkm_wait<1>(a0);
        s[0] = mfma_i8_32x32x32(__builtin_bit_cast(i32x4, a0), qf[ks], ks ? s[0] : sbias);
        lgkm_wait<0>(a1);
        s[1] = mfma_i8_32x32x32(__builtin_bit_cast(i32x4, a1), qf[ks], ks ? s[1] : sbias);
    }
}

// Masked keys of a score tile (past the sequence end, or above the causal
// diagonal) become kSMasked.
template <bool CAUSAL>
__device__ __forceinline__ void mask_i8(i32x16 (&s)[2], int k0, int N, int g, int my_q)
{
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * blk + 16 * g + r;
            if (key >= N || (CAUSAL && key > my_q))
                s[blk][r] = kSMasked;
        }
}

__device__ __forceinline__ int imax_tile(const i32x16 (&s)[2])
{
    int m = INT_MIN;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; r += 2)
            m = vmax3_i32(m, s[blk][r], s[blk][r + 1]);
    return m;
}

// Running state of one wave: O^T accumulators, the exact running max m (log2
// units, the reference P is quantised against), the row sum l of the
// unquantised 448-scaled probabilities, and a pending O rescale.
template <int D>
struct SState {
    f32x16 o[D / 32];
    float m, l, alpha;
    bool pending;
};

// Raise m to include a tile whose lane-half max is mx (log2 units, -inf for a
// fully masked row).  l is rescaled now; O only after the PV product of the
// tile exponentiated against the old m (apply_pending, one step later).
template <int D>
__device__ __forceinline__ void s_raise(SState<D> &st, float mx)
{
    mx = max_xor32(mx);
    if (__any(mx > st.m)) {
        const float m_new = fmaxf(st.m, mx);
        const float alpha = fast_exp2(st.m - m_new);
        st.l *= alpha;
        st.alpha = alpha;
        st.pending = true;
        st.m = m_new;
    }
}

template <int D>
__device__ __forceinline__ void s_apply_pending(SState<D> &st)
{
    if (st.pending) {
#pragma unroll
        for (int c = 0; c < D / 32; ++c)
            st.o[c] *= st.alpha;
        st.pending = false;
    }
}

// p = 448 * 2^(c * s + log2(448) - m - log2(448)) for the whole tile, E4M3-packed
// (byte 16*blk + r of the lane = score s[blk][r]); returns the lane's row sum.
__device__ __forceinline__ float s_exp_tile(const i32x16 (&s)[2], float c, float bias,
                                            uint32_t (&pk)[8])
{
    const float b = sbias_exp(bias, c);
    float rs = 0.f;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
            float p[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // (the element goes through a scalar: a bit cast of a vector
                // element itself compiles to a read of element 0)
                const int v = s[blk][r + e];
                p[e] = fast_exp2(fmaf(__int_as_float(v), c, b));
                rs += p[e];
            }
            int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
            wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], wd, true);
            pk[4 * blk + r / 4] = (uint32_t)wd;
        }
    return rs;
}

// One pipeline step t: PV(t) with P(t) (E4M3, computed against the running
// max before the last raise), QK(t+2) into s_qk (masked when mask_qk), and
// the exponentials of tile t+1 (s_exp, scale c_exp, against the current m)
// into p_next, adding their row sum to l.  Returns the lane's integer max of
// the masked s_qk.
template <int D, bool CAUSAL, class Dma>
__device__ __forceinline__ int s_step(SState<D> &st, const i32x4 (&qf)[D / 32], uint32_t kst,
                                      uint32_t vst, const SLanes<D> &ln, const i32x16 (&s_exp)[2],
                                      i32x16 (&s_qk)[2], const uint32_t (&p_cur)[8],
                                      uint32_t (&p_next)[8], float c_exp, bool mask_qk, int k0_qk,
                                      int N, int g, int my_q, const i32x16 &sbias,
                                      const Dma &dma)
{
    using SC = SSched<D>;
    constexpr int NS = SC::NS, NQK = SC::NQK, RA = SC::RA;
    const float bexp = sbias_exp(kLog2_448 - st.m, c_exp);
    // operand of slot S: u32x4 for QK, two of them for PV
    u32x4 opa[RA + 1], opb[RA + 1];
    auto read_op = [&](auto sc) {
        constexpr int S = decltype(sc)::value;
        if constexpr (S < NQK) {
            constexpr int blk = S % 2, ks = S / 2;
            opa[S % (RA + 1)] = lds_read_b128<blk * 32 * D>(kst + ln.k[ks]);
        } else {
            constexpr int c = S - NQK;
            opa[S % (RA + 1)] = lds_read_b128<c * 32 * kBlk>(vst + ln.vlo);
            opb[S % (RA + 1)] = lds_read_b128<c * 32 * kBlk>(vst + ln.vhi);
        }
    };
    float p[32];
    float rs0 = 0.f, rs1 = 0.f;
    int imx0 = INT_MIN, imx1 = INT_MIN;
    // fold score R (exponentiated in an earlier slot): row sum and E4M3 packing
    auto fold = [&](auto rc) {
        constexpr int R = decltype(rc)::value;
        if constexpr (R % 2 == 0) {
            rs0 += p[R];
        } else {
            rs1 += p[R];
            constexpr int blk = R / 16, r = R % 16, w = 4 * blk + r / 4;
            // the pair goes straight into its word of P: low half, then high half
            if constexpr ((r & 3) == 1) {
                p_next[w] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(p[R - 1], p[R], 0, false);
            } else {
                p_next[w] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(p[R - 1], p[R],
                                                                      (int)p_next[w], true);
            }
            asm volatile("" : "+v"(p_next[w]));
        }
        asm volatile("" : "+v"(rs0), "+v"(rs1));
    };
    static_for<0, RA>([&](auto i) { read_op(i); });
    static_for<0, NS>([&](auto sc) {
        constexpr int S = decltype(sc)::value;
        if constexpr (S + RA < NS)
            read_op(std::integral_constant<int, S + RA>{});
        if constexpr (S < NQK) {
            lgkm_wait<SC::after(S)>(opa[S % (RA + 1)]);
            s_qk[S % 2] = mfma_i8_32x32x32(__builtin_bit_cast(i32x4, opa[S % (RA + 1)]),
                                           qf[S / 2], S < 2 ? sbias : s_qk[S % 2]);
        } else {
            constexpr int c = S - NQK;
            lgkm_wait<SC::after(S)>(opb[S % (RA + 1)]);
            const u32x4 lo = opa[S % (RA + 1)], hi = opb[S % (RA + 1)];
            const i32x8 va = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                              (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            const i32x8 pb = {(int)p_cur[0], (int)p_cur[1], (int)p_cur[2], (int)p_cur[3],
                              (int)p_cur[4], (int)p_cur[5], (int)p_cur[6], (int)p_cur[7]};
            st.o[c] = mfma_fp8_32x32x64(va, pb, st.o[c]);
        }
        dma(sc);
        static_for<SC::first_score(S), SC::first_score(S + 1)>([&](auto rc) {
            constexpr int R = decltype(rc)::value;
            const int v = s_exp[R / 16][R % 16];
            p[R] = fast_exp2(fmaf(__int_as_float(v), c_exp, bexp));
            asm volatile("" : "+v"(p[R]));
        });
        if constexpr (S > 0)
            static_for<SC::first_score(S - 1), SC::first_score(S)>(fold);
        if constexpr (S == NQK) {
            if (mask_qk)
                mask_i8<CAUSAL>(s_qk, k0_qk, N, g, my_q);
        }
        static_for<0, 16>([&](auto kc) {
            constexpr int k = decltype(kc)::value;
            if constexpr (SC::max_slot(k) == S) {
                constexpr int R = 2 * k, blk = R / 16, r = R % 16;
                if constexpr (k % 2 == 0)
                    imx0 = vmax3_i32(imx0, s_qk[blk][r], s_qk[blk][r + 1]);
                else
                    imx1 = vmax3_i32(imx1, s_qk[blk][r], s_qk[blk][r + 1]);
                asm volatile("" : "+v"(imx0), "+v"(imx1));
            }
        });
        __builtin_amdgcn_sched_barrier(0);
    });
    static_for<SC::first_score(NS - 1), 32>(fold);
    st.l += rs0 + rs1;
    return imx0 > imx1 ? imx0 : imx1;
}

// TAIL: some key tile runs past N (N not a multiple of 64); without it and
// without a causal mask no tile is masked and the mask pass compiles away.
template <int D, bool CAUSAL, bool OUT_F32, bool TAIL>
__device__ __forceinline__ void sage_qtile(const PrefillArgs &a, const SageWs &w,
                                           unsigned char *smem, int bh, int qt, int wave, int lane)
{
    constexpr int kK = SCfg<D>::kKBytes, kV = SCfg<D>::kVBytes;
    const int g = lane >> 5, n = lane & 31;
    const int N = a.N, nblk = (N + kBlk - 1) / kBlk, Npad = nblk * kBlk;
    const int h = bh % a.H, b = bh / a.H;
    const int bg = b * a.Hkv + h / (a.H / a.Hkv);
    const int q0 = qt * kBM, qw0 = q0 + wave * kQW, my_q = qw0 + n;
    const int8_t *khat = w.khat + (size_t)bg * Npad * D;
    const uint8_t *vhatT = w.vhatT + (size_t)bg * D * Npad;
    const float *kdel = w.kdelta + (size_t)bg * nblk;
    const int kend = CAUSAL ? min(N, q0 + kBM) : N;
    const int ntiles = (kend + kBlk - 1) / kBlk;
    const int ntw = CAUSAL ? min(ntiles, (qw0 + kQW - 1) / kBlk + 1) : ntiles;
    auto kst = [&](int t) { return smem + (t & 3) * kK; };
    auto vst = [&](int t) { return smem + 4 * kK + (t & 3) * kV; };
    auto needs_mask = [&](int t) {
        const int k0 = t * kBlk;
        return (CAUSAL && k0 + kBlk - 1 > qw0) || (TAIL && k0 + kBlk > N);
    };
    // direct loads: one 1 KB piece of each tile per wave (waves beyond the
    // piece count load nothing); the V^^T tile's rows are Npad bytes apart
    const SDma<D> dm = s_dma<D>(wave, lane, Npad);
    const bool has_k = wave < SCfg<D>::kKPieces, has_v = wave < SCfg<D>::kVPieces;
    auto load_k = [&](int t) {
        if (t < ntiles && has_k)
            dma16_rsrc(raw_rsrc(khat + (size_t)t * kBlk * D, kK), dm.k, kst(t) + wave * 1024);
    };
    auto load_v = [&](int t) {
        if (t < ntiles && has_v)
            dma16_rsrc(raw_rsrc(vhatT + (size_t)t * kBlk, (uint32_t)((D - 1) * Npad + kBlk)), dm.v,
                       vst(t) + wave * 1024);
    };
    load_k(0);
    load_k(1);
    load_k(2);
    load_v(0);
    load_k(3);
    load_v(1);

    // Q^^T fragments (B operand of the INT8 MFMA, K = 32 per step): lane holds
    // Q^[my_q][32*ks + 16*g .. +15].  Rows past N are zero in the workspace.
    i32x4 qf[D / 32];
    const int8_t *qrow = w.qhat + ((size_t)bh * Npad + min(my_q, Npad - 1)) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
        qf[ks] = __builtin_bit_cast(i32x4, ld16(qrow + ks * 32 + g * 16));
    // the 32 queries of a wave lie in one 64-token block
    const float cq = a.scale * kLog2e * w.qdelta[(size_t)bh * nblk + min(qw0, N - 1) / kBlk];
    // per-tile score scales c(t) = cq * dK(t) for tiles t+1 .. t+5 of an even
    // step t; those of tiles t+4, t+5 are loaded at step t and land by the
    // synchronisation before step t+2
    // (kept >= the smallest normal float, so that a masked score's -inf times c stays -inf)
    auto kd = [&](int t) { return t < ntiles ? kdel[t] : 1.f; };
    auto tc = [&](float kdv) { return fmaxf(cq * kdv, __FLT_MIN__); };
    float c1 = tc(kd(1)), c2 = tc(kd(2)), c3 = tc(kd(3)), kd4 = 1.f, kd5 = 1.f;
    const float c0 = tc(kd(0));

    const SLanes<D> ln = s_lanes<D>(lane);
    SState<D> st;
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
        st.o[c] = f32x16{};
    st.l = 0.f;
    st.alpha = 1.f;
    st.pending = false;

    i32x16 sA[2], sB[2];   // S(j): sA for even j, sB for odd j
    const i32x16 sbias = sbias16();
    uint32_t pA[8], pB[8];  // P(j) likewise

    // pre-step: S(0), S(1); m from S(0) (exact), P(0); raise for S(1)
    vm_wait_n<0>();
    __syncthreads();
    if (0 < ntw) {
        qk_tile_i8<D>(sA, qf, lds_addr(kst(0)), ln, sbias);
        if (ntw > 1)
            qk_tile_i8<D>(sB, qf, lds_addr(kst(1)), ln, sbias);
        if (needs_mask(0))
            mask_i8<CAUSAL>(sA, 0, N, g, my_q);
        const int i0 = imax_tile(sA);
        st.m = max_xor32(smax_log2(i0, c0));
        st.l = s_exp_tile(sA, c0, kLog2_448 - st.m, pA);
        if (ntw > 1) {
            if (needs_mask(1))
                mask_i8<CAUSAL>(sB, kBlk, N, g, my_q);
            const int i1 = imax_tile(sB);
            s_raise<D>(st, smax_log2(i1, c1));
        }
    }

    // step t: as in the exact kernel, 4-stage rings, synchronisation before
    // every even step, loads of K(t+4) and V(t+2) spread over the slots
    auto step = [&](int t, auto par, float c_exp, float c_qk) {
        constexpr int E = decltype(par)::value;
        if constexpr (E == 0) {
            vm_wait_n<0>();
            __syncthreads();
            if (t + 4 < ntiles)
                kd4 = kdel[t + 4];
            if (t + 5 < ntiles)
                kd5 = kdel[t + 5];
        }
        const bool lk = t + 4 < ntiles && has_k, lv = t + 2 < ntiles && has_v;
        const __amdgpu_buffer_rsrc_t rk = raw_rsrc(khat + (size_t)(lk ? t + 4 : 0) * kBlk * D, kK);
        const __amdgpu_buffer_rsrc_t rv =
            raw_rsrc(vhatT + (size_t)(lv ? t + 2 : 0) * kBlk, (uint32_t)((D - 1) * Npad + kBlk));
        unsigned char *const k_st = kst(t + 4) + wave * 1024, *const v_st = vst(t + 2) + wave * 1024;
        auto dma = [&](auto sc) {
            constexpr int S = decltype(sc)::value;
            if constexpr (S == SSched<D>::dma_slot(0)) {
                if (lk)
                    dma16_rsrc(rk, dm.k, k_st);
            }
            if constexpr (S == SSched<D>::dma_slot(1)) {
                if (lv)
                    dma16_rsrc(rv, dm.v, v_st);
            }
        };
        i32x16(&s_exp)[2] = E ? sA : sB;  // S(t+1)
        i32x16(&s_qk)[2] = E ? sB : sA;   // S(t+2)
        uint32_t(&pc)[8] = E ? pB : pA;   // P(t)
        uint32_t(&pn)[8] = E ? pA : pB;   // P(t+1)
        const float l_before = st.l;
        const int imx = s_step<D, CAUSAL>(st, qf, lds_addr(kst(t + 2)), lds_addr(vst(t)), ln,
                                          s_exp, s_qk, pc, pn, c_exp, needs_mask(t + 2),
                                          (t + 2) * kBlk, N, g, my_q, sbias, dma);
        if (t + 1 >= ntw)
            st.l = l_before;  // tile t+1 does not exist for this wave
        // PV(t) has been issued with P(t): O can take the factor of the raise
        // that P(t+1) was computed after
        s_apply_pending<D>(st);
        if (t + 2 < ntw)
            s_raise<D>(st, smax_log2(imx, c_qk));
    };
    int t = 0;
    for (; t + 1 < ntw; t += 2) {
        step(t, std::integral_constant<int, 0>{}, c1, c2);
        step(t + 1, std::integral_constant<int, 1>{}, c2, c3);
        c1 = c3;
        c2 = tc(kd4);
        c3 = tc(kd5);
    }
    if (t < ntw) {
        step(t, std::integral_constant<int, 0>{}, c1, c2);
        ++t;
    }
    for (; t < ntiles; ++t) {
        if ((t & 1) == 0) {
            vm_wait_n<0>();
            __syncthreads();
        }
        load_k(t + 4);
        load_v(t + 2);
    }
    s_apply_pending<D>(st);

    // O = acc * delta_V / l448 ; lse = (m + log2 l448 - log2 448) ln2 + scale * q.kmean
    const float lt = sum_xor32(st.l);
    if (my_q < N) {
        const float inv = 1.f / lt;
        const float *vs = w.vscale + (size_t)bg * D;
#pragma unroll
        for (int cc = 0; cc < D / 32; ++cc) {
            float val[16];
#pragma unroll
            for (int r = 0; r < 16; ++r)
                val[r] = st.o[cc][r] * vs[32 * cc + 16 * g + r] * inv;
            if constexpr (OUT_F32) {
                float *orow = (float *)a.o + ((size_t)bh * N + my_q) * D + 32 * cc + 16 * g;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *(f32x4 *)(orow + 4 * j) =
                        f32x4{val[4 * j], val[4 * j + 1], val[4 * j + 2], val[4 * j + 3]};
            } else {
                uint16_t *orow = (uint16_t *)a.o + ((size_t)bh * N + my_q) * D + 32 * cc + 16 * g;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    u32x4 wv;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        wv[e] = pack_bf16x2(val[8 * j + 2 * e], val[8 * j + 2 * e + 1]);
                    st16(orow + 8 * j, wv);
                }
            }
        }
        if (a.lse && g == 0)
            a.lse[(size_t)bh * N + my_q] = (st.m + log2f(lt) - kLog2_448) * kLn2 +
                                           a.scale * w.qkdot[(size_t)bh * N + my_q];
    }
}

template <int D, bool CAUSAL, bool OUT_F32, bool TAIL>
__global__ __launch_bounds__(kAThreads) void sage_attn_kernel(PrefillArgs a, SageWs w)
{
    __shared__ __attribute__((aligned(1024)))
    unsigned char smem[4 * SCfg<D>::kKBytes + 4 * SCfg<D>::kVBytes];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nqt = (a.N + kBM - 1) / kBM;
    // causal: workgroup j of a head takes query tiles nqt-1-j and j (equal work)
    const int nw = CAUSAL ? (nqt + 1) / 2 : nqt;
    const int BH = a.B * a.H;
    int bh, j;
    const int wg = blockIdx.x;
    if ((BH & 7) == 0) {
        const int xcd = wg & 7, slot = wg >> 3;
        bh = xcd + 8 * (slot / nw);
        j = slot % nw;
    } else {
        bh = wg / nw;
        j = wg % nw;
    }
    if (CAUSAL) {
        sage_qtile<D, CAUSAL, OUT_F32, TAIL>(a, w, smem, bh, nqt - 1 - j, wave, lane);
        if (j < nqt - 1 - j) {
            __syncthreads();  // every wave is done with the LDS stages
            sage_qtile<D, CAUSAL, OUT_F32, TAIL>(a, w, smem, bh, j, wave, lane);
        }
    } else {
        sage_qtile<D, CAUSAL, OUT_F32, TAIL>(a, w, smem, bh, j, wave, lane);
    }
}

template <int D>
hipError_t launch_d(const SageArgs &sa, hipStream_t s)
{
    const PrefillArgs &a = sa.p;
    const SageWs w = carve(sa.workspace, a.B, a.H, a.Hkv, a.N, D);
    const int nblk = (a.N + kBlk - 1) / kBlk;
    const int BG = a.B * a.Hkv, BH = a.B * a.H;
    const uint16_t *q = (const uint16_t *)a.q, *k = (const uint16_t *)a.k,
                   *v = (const uint16_t *)a.v;
    {
        ProfScope ps("sage_stats", s);
        hipLaunchKernelGGL(sage_stats_kernel<D>, dim3(BG, kNCh), dim3(kThreads), 0, s, k, v, w, a.N);
    }
    {
        ProfScope ps("sage_finalize", s);
        hipLaunchKernelGGL(sage_finalize_kernel<D>, dim3(BG), dim3(D), 0, s, w, a.N);
    }
    {
        ProfScope ps("sage_quant_qk", s);
        hipLaunchKernelGGL(sage_quant_qk_kernel<D>, dim3((BH + BG) * nblk), dim3(kThreads), 0, s, q, k,
                           w, a.B, a.H, a.Hkv, a.N);
    }
    {
        ProfScope ps("sage_quant_v", s);
        hipLaunchKernelGGL(sage_quant_v_kernel<D>, dim3(BG, nblk), dim3(kThreads), 0, s, v, w, a.N);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int nqt = (a.N + kBM - 1) / kBM;
    ProfScope ps("sage_attn", s);
    dim3 grid(BH * (a.causal ? (nqt + 1) / 2 : nqt)), block(kAThreads);
    const bool tail = a.N % kBlk != 0;
    if (a.causal) {
        if (a.out_fp32)
            hipLaunchKernelGGL((sage_attn_kernel<D, true, true, true>), grid, block, 0, s, a, w);
        else
            hipLaunchKernelGGL((sage_attn_kernel<D, true, false, true>), grid, block, 0, s, a, w);
    } else if (tail) {
        if (a.out_fp32)
            hipLaunchKernelGGL((sage_attn_kernel<D, false, true, true>), grid, block, 0, s, a, w);
        else
            hipLaunchKernelGGL((sage_attn_kernel<D, false, false, true>), grid, block, 0, s, a, w);
    } else {
        if (a.out_fp32)
            hipLaunchKernelGGL((sage_attn_kernel<D, false, true, false>), grid, block, 0, s, a, w);
        else
            hipLaunchKernelGGL((sage_attn_kernel<D, false, false, false>), grid, block, 0, s, a,
                               w);
    }
    return hipGetLastError();
}

}  // namespace

size_t sage_workspace_bytes(int B, int H, int Hkv, int N, int d)
{
    size_t off[kSageWsPieces + 1];
    layout(B, H, Hkv, N, d, off);
    return off[kSageWsPieces];
}

void sage_workspace_layout(int B, int H, int Hkv, int N, int d, size_t *offsets)
{
    size_t off[kSageWsPieces + 1];
    layout(B, H, Hkv, N, d, off);
    for (int i = 0; i < kSageWsPieces; ++i)
        offsets[i] = off[i];
}

hipError_t launch_sage(const SageArgs &sa, hipStream_t s)
{
    return sa.p.d == 64 ? launch_d<64>(sa, s) : launch_d<128>(sa, s);
}

}  // namespace attn
