// MX quantised attention forward for gfx950: SageAttention3's FP4
// microscaling ("gpu-kernel-porting-with-ai-agents" page, SageAttention 3
// section: P normalised per token, then FP4 with per-block scales; "GPU
// kernel overview" page, insights: FP4 and FP6 on CDNA4) on the MX block
// formats the gfx950 matrix cores take: E2M1 (FP4) or E2M3 (FP6) elements
// with one power-of-two E8M0 scale per block of 32 along the contraction
// dimension.
//
// The recipe (element format F = 4 or 6, largest magnitude 6 or 7.5):
//   1. Smooth-K: K' = K - kmean (per channel over all N tokens, fp32);
//   2. Q and K' to MX blocks of 32 consecutive channels of a token, V in
//      blocks of 32 consecutive tokens of a channel; a block's scale is 2^e
//      with e the smallest exponent such that max|x| <= emax * 2^e (nothing
//      saturates); elements are the nearest codes of x / 2^e (ties to even);
//   3. S = scale * Q^ K^^T on v_mfma_scale_f32_32x32x64_f8f6f4 (the per-lane
//      scale byte applied in the MFMA);
//   4. online softmax over 64-key tiles with the exact running max m:
//      p = 2^(S log2e - m) in (0, 1] (the per-token normalisation), l sums
//      the unquantised p, and P^ = MX(p) per block of 32 consecutive keys
//      (the conversion instructions with the block's scale);
//   5. O += P^ V^ on the same MFMA; O / l at the end, lse = m + ln l +
//      scale * (q . kmean).
//
// Kernels: mx_ksum (partial per-channel K sums, fp64) and mx_kmean,
// mx_quant_qk / mx6_quant_qk (Q and K' blocks and q . kmean), mx_quant_v (V
// blocks, read by channel through LDS), mx_attn (the fused attention).
//
// mx_attn: 4 waves x 32 queries per workgroup, three workgroups per CU (the
// kernel is held to 168 registers, three waves per SIMD: the per-score
// vector work of one wave then hides behind two others; at two waves per
// SIMD the FP4 kernel ran 25% slower); S^T = K^ Q^^T (keys are MFMA
// rows).  Key rows are fed to the two 32-row MFMA blocks of a tile in the
// order that leaves lane half g holding keys 32g .. 32g+31 of the tile in its
// 32 accumulator registers: those are one P block, so a lane quantises its
// block alone, and its codes are directly the B operand of O^T += V^^T P^^T
// (lane half g supplies keys 32g .. 32g+31, one block, one scale byte).  K^,
// V^^T and their scales go global -> LDS through direct loads into two
// stages, one workgroup barrier per tile.  Every operand read is a per-lane
// base offset plus an immediate, and a V^^T tile is laid out [key
// block][feature], so that the 16 lanes of a 16-byte read take 256
// contiguous bytes (with feature rows of 32 bytes, as first built, they
// conflicted two ways; the change made the FP4 kernel 6% faster).
//
// An FP6 block is 24 bytes: the MFMA takes a lane's 32 six-bit codes in bit
// order over six registers.  Its first 16 bytes are laid out as a whole FP4
// block is (so the FP4 kernel's LDS swizzle and reads apply unchanged) and
// its last 8 bytes go to a separate block-major area of the tile, where the
// 32 lanes of a read take 256 contiguous bytes.
#include "../../include/attn.h"
#include "attn_internal.hpp"
#include "cdna4.hpp"

namespace attn {
namespace {

constexpr int kTile = 64;  // keys per tile; token padding of the quantised tensors
constexpr int kNCh = 16;   // sequence chunks of the K-mean pass
constexpr int kThreads = 256;

// The element formats: MFMA format code, and the mantissa bits (of a float
// in [1, 2)) of emax / 4: 1.5 for E2M1 (emax 6), 1.875 for E2M3 (emax 7.5).
template <int F>
struct Elem;
template <>
struct Elem<4> {
    static constexpr int kCode = 4;
    static constexpr uint32_t kCut = 0x400000;
};
template <>
struct Elem<6> {
    static constexpr int kCode = 2;
    static constexpr uint32_t kCut = 0x700000;
};

// E8M0 exponent of a block scale from the block's max magnitude (bits of a
// non-negative float): the smallest e with amax <= emax * 2^e.  For amax =
// f * 2^k (f in [1, 2)), emax * 2^(k-2) = (emax / 4) * 2^k, so e = k - 2 when
// f <= emax / 4 and k - 1 otherwise; zero (and subnormal) maxima clamp into
// E8M0's range.
template <int F>
__device__ __forceinline__ int mx_exp(float amax)
{
    if (!(amax > 0.f))
        return 0;
    const uint32_t b = __float_as_uint(amax);
    const int k = (int)((b >> 23) & 0xff) - 127;
    const int e = k - 2 + ((b & 0x7fffff) > Elem<F>::kCut ? 1 : 0);
    return e < -126 ? -126 : (e > 127 ? 127 : e);
}

// the float 2^e (e in [-126, 127])
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// Two values to two E2M1 codes in byte `sel` of w: nearest (ties to even)
// of a / scale and b / scale (scale a power of two), a in the low nibble.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2(uint32_t w, float a, float b, float scale)
{
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, scale, SEL);
}

// 32 values (v[0..31]) to 32 E2M1 codes in four words (element i in nibble
// i % 8 of word i / 8, low nibble first), with the scale 2^e.
__device__ __forceinline__ u32x4 fp4x32(const float (&v)[32], int e)
{
    const float s = pow2f(e);
    u32x4 out;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t x = 0;
        x = fp4x2<0>(x, v[8 * w + 0], v[8 * w + 1], s);
        x = fp4x2<1>(x, v[8 * w + 2], v[8 * w + 3], s);
        x = fp4x2<2>(x, v[8 * w + 4], v[8 * w + 5], s);
        x = fp4x2<3>(x, v[8 * w + 6], v[8 * w + 7], s);
        out[w] = x;
    }
    return out;
}

typedef int i32x6 __attribute__((ext_vector_type(6)));

// 32 values (v[0..31]) to 32 E2M3 codes of v / 2^e (nearest, ties to even)
// in six words, element i in bits 6i .. 6i+5 of the 192-bit little-endian
// group.  The instruction takes element 2i from its first source and 2i+1
// from its second.  Its result is wrong where its destination registers
// overlap its sources, which the compiler allows for the builtin, so it is
// issued as asm with an early-clobber destination.
__device__ __forceinline__ i32x6 fp6x32(const float (&v)[32], int e)
{
    f32x16 a, b;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        a[i] = v[2 * i];
        b[i] = v[2 * i + 1];
    }
    i32x6 r;
    asm("v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, %3" : "=&v"(r) : "v"(a), "v"(b), "v"(pow2f(e)));
    return r;
}

// An MFMA operand: a lane's 32 codes; FP4 fills four registers, FP6 six (the
// first 16 bytes in lo, the last 8 in hi).
template <int F>
__device__ __forceinline__ i32x8 mx_operand(u32x4 lo, u32x2 hi)
{
    if constexpr (F == 4)
        return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], 0, 0, 0, 0};
    else
        return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], 0, 0};
}

// 32x32x64 MFMA of two F-format operands with per-lane E8M0 scale bytes (sa
// for A's lane block, sb for B's).
template <int F>
__device__ __forceinline__ f32x16 mfma_mx(i32x8 a, i32x8 b, f32x16 c, int sa, int sb)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, Elem<F>::kCode, Elem<F>::kCode,
                                                           0, sa, 0, sb);
}

// Position of token r (0..63) of a tile in the block-major area of an FP6
// tile: bits 4 and 5 swapped, so that the 32 keys one read of the attention
// kernel takes (bit 5 and bits 0-3 free, bit 4 fixed) are 32 consecutive
// slots.
__device__ __forceinline__ int kperm(int r) { return (r & 15) | ((r >> 1) & 16) | ((r << 1) & 32); }

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace pieces (byte-addressed; Npad = N rounded up to kTile).  FP4:
// Q^ and K^ rows of D/2 bytes (channel 2i in the low nibble); V^^T in tiles
// of 64 keys, each [key block][feature] x 16 bytes (key 2i in the low
// nibble).  FP6: tiles of 64 tokens of 48 D bytes each; a Q^ / K^ tile holds
// the first 16 bytes of every block token-major ([token][block]) and then
// their last 8 bytes block-major ([block][kperm(token)]); a V^^T tile holds
// the first 16 bytes as [key block][feature] and then the last 8 bytes the
// same way.
struct MxWs {
    double *ksum_part;  // [BG][kNCh][D]
    float *kmean;       // [BG][D]
    float *qkdot;       // [BH][N]
    uint8_t *qhat;      // [BH][Npad * D * F / 8]
    uint8_t *qsc;       // [BH][Npad][D/32]  E8M0 scale bytes
    uint8_t *khat;      // [BG][Npad * D * F / 8]
    uint8_t *ksc;       // [BG][Npad][D/32]
    uint8_t *vhatT;     // [BG][D * Npad * F / 8]
    uint8_t *vscT;      // [BG][Npad/32][D]  block-major scale bytes
};

void mx_layout(int B, int H, int Hkv, int N, int d, int F, size_t (&off)[10])
{
    const size_t BH = (size_t)B * H, BG = (size_t)B * Hkv;
    const size_t Npad = ((size_t)N + kTile - 1) / kTile * kTile;
    const size_t bytes[9] = {sizeof(double) * BG * kNCh * d, sizeof(float) * BG * d,
                             sizeof(float) * BH * N,       BH * Npad * d * F / 8,
                             BH * Npad * d / 32,           BG * Npad * d * F / 8,
                             BG * Npad * d / 32,           BG * d * Npad * F / 8,
                             BG * Npad / 32 * d};
    size_t p = 0;
    for (int i = 0; i < 9; ++i) {
        off[i] = p;
        p += align256(bytes[i]);
    }
    off[9] = p;
}

MxWs mx_carve(void *base, int B, int H, int Hkv, int N, int d, int F)
{
    size_t off[10];
    mx_layout(B, H, Hkv, N, d, F, off);
    char *p = (char *)base;
    MxWs w;
    w.ksum_part = (double *)(p + off[0]);
    w.kmean = (float *)(p + off[1]);
    w.qkdot = (float *)(p + off[2]);
    w.qhat = (uint8_t *)(p + off[3]);
    w.qsc = (uint8_t *)(p + off[4]);
    w.khat = (uint8_t *)(p + off[5]);
    w.ksc = (uint8_t *)(p + off[6]);
    w.vhatT = (uint8_t *)(p + off[7]);
    w.vscT = (uint8_t *)(p + off[8]);
    return w;
}

// ----------------------------------------------------------------- prologue

// Partial per-channel sums of K over one sequence chunk (fp64).
template <int D>
__global__ __launch_bounds__(kThreads) void mx_ksum_kernel(const uint16_t *k, MxWs w, int N)
{
    constexpr int TPR = D / 8, RPP = kThreads / TPR;
    __shared__ double red[RPP][D];
    const int bg = blockIdx.x, chunk = blockIdx.y, tid = threadIdx.x;
    const int fc = tid % TPR, rg = tid / TPR;
    const int len = (N + kNCh - 1) / kNCh;
    const int r0 = chunk * len, r1 = min(N, r0 + len);
    const uint16_t *kb = k + (size_t)bg * N * D;
    double s[8] = {};
    // unrolled, so that several rows' loads are in flight per thread
#pragma unroll 4
    for (int r = r0 + rg; r < r1; r += RPP) {
        const u32x4 kw = ld16_nt(kb + (size_t)r * D + fc * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s[2 * e] += bf16_lo(kw[e]);
            s[2 * e + 1] += bf16_hi(kw[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
        red[rg][fc * 8 + e] = s[e];
    __syncthreads();
    for (int c = tid; c < D; c += kThreads) {
        double t = 0.0;
        for (int r = 0; r < RPP; ++r)
            t += red[r][c];
        w.ksum_part[((size_t)bg * kNCh + chunk) * D + c] = t;
    }
}

// kmean = sum / N in fp64, rounded to fp32.
template <int D>
__global__ __launch_bounds__(D) void mx_kmean_kernel(MxWs w, int N)
{
    const int bg = blockIdx.x, c = threadIdx.x;
    double s = 0.0;
    for (int i = 0; i < kNCh; ++i)
        s += w.ksum_part[((size_t)bg * kNCh + i) * D + c];
    w.kmean[(size_t)bg * D + c] = (float)(s / (double)N);
}

// Q rows, then K' = K - kmean rows (each sequence padded to Npad rows, the
// rows past N all zero): every 32-channel block gets its E8M0 exponent (R24)
// and 16 bytes of E2M1 codes.  A workgroup takes 64 rows of one sequence as
// CR = D/8 16-byte chunks per row; thread t takes chunks t, t + 256, ..., so
// every load and store instruction of a wave covers contiguous memory and a
// thread's channels are the same 8 in every chunk.  A block's four chunks sit
// in four consecutive lanes: its amax is two lane shuffles, and each lane
// writes the block's word for its chunk.
template <int D>
__global__ __launch_bounds__(kThreads) void mx_quant_qk_kernel(const uint16_t *q, const uint16_t *k,
                                                               MxWs w, int B, int H, int Hkv, int N)
{
    constexpr int CR = D / 8;                  // chunks per row
    constexpr int NB = D / 32;                 // blocks per row
    constexpr int NCH = kTile * CR / kThreads;  // chunks per thread
    static_assert(kThreads % CR == 0 && NCH * kThreads == kTile * CR, "chunk split");
    const int Npad = (N + kTile - 1) / kTile * kTile;
    const int tid = threadIdx.x, ch = tid % CR;  // channels 8ch .. 8ch+7
    const long long row0 = (long long)blockIdx.x * kTile;  // seq * Npad + tok0
    const long long nqrows = (long long)B * H * Npad;
    const bool is_q = row0 < nqrows;
    const long long u0 = is_q ? row0 : row0 - nqrows;
    const long long seq = u0 / Npad;  // b*H + h or b*Hkv + g
    const int tok0 = (int)(u0 % Npad);
    const int g = is_q ? (int)((seq / H) * Hkv + (seq % H) / (H / Hkv)) : (int)seq;
    float km[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        km[e] = w.kmean[(size_t)g * D + 8 * ch + e];
    const uint16_t *src = (is_q ? q : k) + ((size_t)seq * N + tok0) * D;
    uint8_t *dst = (is_q ? w.qhat : w.khat) + (size_t)u0 * (D / 2);
    uint8_t *dsc = (is_q ? w.qsc : w.ksc) + (size_t)u0 * NB;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int chunk = kThreads * j + tid, r = chunk / CR;
        const bool real = tok0 + r < N;
        float x[8];
        {
            u32x4 v = {0, 0, 0, 0};
            if (real)
                v = ld16(src + (size_t)chunk * 8);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[2 * e] = bf16_lo(v[e]);
                x[2 * e + 1] = bf16_hi(v[e]);
            }
        }
        if (is_q) {
            // q . kmean for the LSE correction; the row's CR lanes are consecutive
            float dot = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                dot = fmaf(x[i], km[i], dot);
#pragma unroll
            for (int off = 1; off < CR; off <<= 1)
                dot += __shfl_xor(dot, off, 64);
            if (ch == 0 && real)
                w.qkdot[(size_t)seq * N + tok0 + r] = dot;
        } else if (real) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                x[i] -= km[i];
        }
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            amax = fmaxf(amax, fabsf(x[i]));
        amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
        const int e = mx_exp<4>(amax);
        const float sc = pow2f(e);
        uint32_t word = 0;
        word = fp4x2<0>(word, x[0], x[1], sc);
        word = fp4x2<1>(word, x[2], x[3], sc);
        word = fp4x2<2>(word, x[4], x[5], sc);
        word = fp4x2<3>(word, x[6], x[7], sc);
        *(uint32_t *)(dst + (size_t)chunk * 4) = word;
        if ((ch & 3) == 0)
            dsc[(size_t)r * NB + ch / 4] = (uint8_t)(e + 127);
    }
}

// FP6 Q rows, then K' rows: one 64-token tile per workgroup, staged in LDS
// as bf16 (rows of D + 8 elements) by contiguous 16-byte loads; thread t <
// 64 D/32 then takes block t % (D/32) of token t / (D/32): its 32 channels,
// their amax and exponent, and their codes in one conversion instruction.
// The block's first 16 bytes are written token-major (contiguous over the
// threads), its last 8 bytes block-major at slot kperm(token), its scale
// byte as for FP4.
template <int D>
__global__ __launch_bounds__(kThreads) void mx6_quant_qk_kernel(const uint16_t *q, const uint16_t *k,
                                                                MxWs w, int B, int H, int Hkv, int N)
{
    constexpr int NB = D / 32, P = D + 8, TB = kTile * D * 6 / 8;
    static_assert(kTile * NB <= kThreads, "one thread per block of the tile");
    __shared__ __attribute__((aligned(16))) uint16_t tile[kTile * P];
    __shared__ __attribute__((aligned(16))) float kms[D];  // the kv head's kmean
    const int Npad = (N + kTile - 1) / kTile * kTile;
    const int tid = threadIdx.x;
    const long long row0 = (long long)blockIdx.x * kTile;  // seq * Npad + tok0
    const long long nqrows = (long long)B * H * Npad;
    const bool is_q = row0 < nqrows;
    const long long u0 = is_q ? row0 : row0 - nqrows;
    const long long seq = u0 / Npad;  // b*H + h or b*Hkv + g
    const int tok0 = (int)(u0 % Npad);
    const int g = is_q ? (int)((seq / H) * Hkv + (seq % H) / (H / Hkv)) : (int)seq;
    const uint16_t *src = (is_q ? q : k) + ((size_t)seq * N + tok0) * D;
    if (tid < D)
        kms[tid] = w.kmean[(size_t)g * D + tid];
    for (int i = tid; i < kTile * D / 8; i += kThreads) {
        const int r = i / (D / 8);
        u32x4 u = {0, 0, 0, 0};
        if (tok0 + r < N)
            u = ld16_nt(src + (size_t)i * 8);
        *(u32x4 *)&tile[r * P + (i % (D / 8)) * 8] = u;
    }
    __syncthreads();
    if (tid >= kTile * NB)
        return;
    const int r = tid / NB, blk = tid % NB;
    const bool real = tok0 + r < N;
    float x[32];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const u32x4 u = *(const u32x4 *)&tile[r * P + 32 * blk + 8 * j];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[8 * j + 2 * e] = bf16_lo(u[e]);
            x[8 * j + 2 * e + 1] = bf16_hi(u[e]);
        }
    }
    const float *km = kms + 32 * blk;
    if (is_q) {
        // q . kmean for the LSE correction; the token's NB lanes are consecutive
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i)
            dot = fmaf(x[i], km[i], dot);
#pragma unroll
        for (int off = 1; off < NB; off <<= 1)
            dot += __shfl_xor(dot, off, 64);
        if (blk == 0 && real)
            w.qkdot[(size_t)seq * N + tok0 + r] = dot;
    } else if (real) {
#pragma unroll
        for (int i = 0; i < 32; ++i)
            x[i] -= km[i];
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i)
        amax = fmaxf(amax, fabsf(x[i]));
    const int e = mx_exp<6>(amax);
    const i32x6 c6 = fp6x32(x, e);
    uint8_t *dst = (is_q ? w.qhat : w.khat) + (size_t)(u0 / kTile) * TB;
    st16(dst + r * (D / 2) + 16 * blk,
         u32x4{(uint32_t)c6[0], (uint32_t)c6[1], (uint32_t)c6[2], (uint32_t)c6[3]});
    *(u32x2 *)(dst + 32 * D + (blk * kTile + kperm(r)) * 8) = u32x2{(uint32_t)c6[4], (uint32_t)c6[5]};
    (is_q ? w.qsc : w.ksc)[(size_t)u0 * NB + tid] = (uint8_t)(e + 127);
}

// One 64-key tile of V for one (batch, kv head): thread (c, h) turns the 32
// keys 32h .. 32h+31 of channel c into one block: its codes and its scale
// byte.  The tile is staged through LDS as bf16 (rows of D + 8 elements, 17
// KB, so that nine workgroups fit a CU) to read it by channel.
template <int D, int F>
__global__ __launch_bounds__(kThreads) void mx_quant_v_kernel(const uint16_t *v, MxWs w, int N)
{
    static_assert(2 * D <= kThreads, "one thread per (channel, half tile)");
    constexpr int P = D + 8;  // row pitch (elements): 16-byte aligned rows
    __shared__ __attribute__((aligned(16))) uint16_t tile[kTile * P];
    const int Npad = (N + kTile - 1) / kTile * kTile;
    const int bg = blockIdx.x, tt = blockIdx.y, tid = threadIdx.x;
    for (int i = tid; i < kTile * D / 8; i += kThreads) {
        const int r = i / (D / 8), c8 = (i % (D / 8)) * 8;
        const int tok = tt * kTile + r;
        u32x4 u = {0, 0, 0, 0};
        if (tok < N)
            u = ld16_nt(v + ((size_t)bg * N + tok) * D + c8);
        *(u32x4 *)&tile[r * P + c8] = u;
    }
    __syncthreads();
    if (tid < 2 * D) {
        const int c = tid % D, h = tid / D;
        float x[32];
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            x[i] = __uint_as_float((uint32_t)tile[(32 * h + i) * P + c] << 16);
            amax = fmaxf(amax, fabsf(x[i]));
        }
        const int e = mx_exp<F>(amax);
        // thread tid = h D + c writes slot tid of the tile's [key block][feature]
        // area(s): contiguous over the threads
        if constexpr (F == 4) {
            uint8_t *tb = w.vhatT + ((size_t)bg * (Npad / kTile) + tt) * (kTile * D / 2);
            st16(tb + (size_t)tid * 16, fp4x32(x, e));
        } else {
            // the tile's [key block][feature] areas: 16-byte parts, then 8-byte parts
            const i32x6 c6 = fp6x32(x, e);
            uint8_t *tb = w.vhatT + ((size_t)bg * (Npad / kTile) + tt) * (kTile * D * 6 / 8);
            st16(tb + (size_t)tid * 16,
                 u32x4{(uint32_t)c6[0], (uint32_t)c6[1], (uint32_t)c6[2], (uint32_t)c6[3]});
            *(u32x2 *)(tb + 32 * D + (size_t)tid * 8) = u32x2{(uint32_t)c6[4], (uint32_t)c6[5]};
        }
        w.vscT[((size_t)bg * (Npad / 32) + 2 * tt + h) * D + c] = (uint8_t)(e + 127);
    }
}

// ----------------------------------------------------------------- attention

constexpr int kWaves = 4;
constexpr int kAThreads = 64 * kWaves;
constexpr int kQW = 32;
constexpr int kBM = kQW * kWaves;
constexpr int kStages = 2;  // LDS stages of K^ / V^^T tiles

template <int D, int F>
struct MCfg {
    static constexpr int kRow = D / 2;                // bytes of a key's 16-byte block parts
    static constexpr int kNB = D / 32;                // scale blocks of a K^ row
    static constexpr int kKLoBytes = kTile * kRow;    // the K^ tile's 16-byte parts
    static constexpr int kKBytes = kTile * D * F / 8; // K^ tile (FP6: then its 8-byte parts)
    static constexpr int kKScBytes = kTile * kNB;     // its scales
    static constexpr int kVLoBytes = D * kTile / 2;   // the V^^T tile's 16-byte parts
    static constexpr int kVBytes = D * kTile * F / 8; // V^^T tile
    static constexpr int kVScBytes = 2 * D;           // its scales (two key blocks of D)
    // stage: K^ tile | V^^T tile | K^ scales (256 B) | V^ scales (256 B)
    static constexpr int kKSc = kKBytes + kVBytes, kVSc = kKSc + 256;
    static constexpr int kStage = kVSc + 256;
    static constexpr int kKLoPieces = kKLoBytes / 1024;
    static constexpr int kKPieces = kKBytes / 1024, kVPieces = kVBytes / 1024;
    static constexpr int kKH = D / 64;                // QK MFMAs per key block (64 channels each)
    static constexpr int kChunks = kRow / 16;         // 16-byte chunks of a K^ row
    static constexpr int kPieceLoads = (kKPieces + kVPieces + kWaves - 1) / kWaves;
    static_assert(kKBytes % 1024 == 0 && kVBytes % 1024 == 0, "whole 1 KB pieces");
    static_assert(kKScBytes <= 256 && kVScBytes <= 256, "scale pieces");
};

// K^ tile chunk swizzle: chunk c of key row `key` is stored at chunk
// c ^ kswz(key).  A QK operand read takes one chunk of 16 rows per 16 lanes,
// rows that differ in key bits 0-1, 2 and 5 (key_of_row below); with rows of
// 64 bytes (d = 128) bits 0-1 already select distinct banks and bits 2 and 5
// move the chunk, with rows of 32 bytes (d = 64) bits 0-2 do and bit 5 moves
// it, so the 16 reads fall on distinct banks.
template <int D>
__device__ __forceinline__ int kswz(int key)
{
    if constexpr (D == 128)
        return ((key >> 2) & 1) | (((key >> 5) & 1) << 1);
    else
        return (key >> 5) & 1;
}

// MFMA row rho of key block b reads key 32 ((rho >> 2) & 1) + 16 b +
// 4 (rho >> 3) + (rho & 3): accumulator register r of lane half g then holds
// key 32 g + 16 b + r.
__device__ __forceinline__ int key_of_row(int rho, int b)
{
    return 32 * ((rho >> 2) & 1) + 16 * b + 4 * (rho >> 3) + (rho & 3);
}

// LDS reads of one byte (zero-extended) and of 8 bytes, as asm for the
// reason given for the other LDS reads (cdna4.hpp): completion is awaited
// with lgkm_wait.  OFF is an immediate byte offset.
template <int OFF = 0>
__device__ __forceinline__ uint32_t lds_read_u8(uint32_t addr)
{
    uint32_t r;
    asm volatile("ds_read_u8 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF) : "memory");
    return r;
}
template <int OFF = 0>
__device__ __forceinline__ u32x2 lds_read_b64(uint32_t addr)
{
    u32x2 r;
    asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF) : "memory");
    return r;
}

// One query tile of one (batch, head).
template <int D, int F, bool CAUSAL, bool OUT_F32>
__device__ __forceinline__ void mx_qtile(const PrefillArgs &a, const MxWs &w, unsigned char *smem,
                                         int bh, int qt, int wave, int lane)
{
    using C = MCfg<D, F>;
    constexpr int NB = C::kNB, KH = C::kKH, NC = D / 32;
    const int g = lane >> 5, n = lane & 31;
    const int N = a.N, Npad = (N + kTile - 1) / kTile * kTile;
    const int h = bh % a.H, b = bh / a.H;
    const int bg = b * a.Hkv + h / (a.H / a.Hkv);
    const int q0 = qt * kBM, qw0 = q0 + wave * kQW, my_q = qw0 + n;
    const int kend = CAUSAL ? min(N, q0 + kBM) : N;
    const int ntiles = (kend + kTile - 1) / kTile;
    // tiles this wave computes (the rest lie above its causal diagonal)
    const int ntw = CAUSAL ? min(ntiles, (qw0 + kQW - 1) / kTile + 1) : ntiles;
    const uint8_t *khat = w.khat + (size_t)bg * (Npad / kTile) * C::kKBytes;
    const uint8_t *ksc = w.ksc + (size_t)bg * Npad * NB;
    const uint8_t *vhatT = w.vhatT + (size_t)bg * D * (Npad / 8) * F;
    const uint8_t *vscT = w.vscT + (size_t)bg * (Npad / 32) * D;
    auto stage = [&](int t) { return smem + (t % kStages) * C::kStage; };
    // direct loads of tile t: 1 KB piece j of the tile goes to wave j %
    // kWaves; pieces 0 .. kKLoPieces-1 are the K^ rows (lane l of piece j
    // fills chunk l % kChunks of row (64 j + l) / kChunks, with the chunk
    // swizzle), then (FP6) the K^ tile's block-major 8-byte parts as they
    // are, then the V^^T tile as it is.  Wave 0 also loads the scales: lanes
    // 0..15 the K^ scales of the tile's 64 keys, lanes 16..31 its two V^
    // scale rows (each contiguous; lane l writes LDS bytes 16 l .. 16 l + 15
    // of the scale area)
    auto load = [&](int t) {
        if (t >= ntiles)
            return;
        unsigned char *st = stage(t);
        const int ln = lane;
#pragma unroll
        for (int u = 0; u < C::kPieceLoads; ++u) {
            const int pc = wave + kWaves * u;
            if (pc < C::kKLoPieces) {
                const int i = pc * 64 + ln, row = i / C::kChunks, c = i % C::kChunks;
                dma16_rsrc(raw_rsrc(khat + (size_t)t * C::kKBytes, C::kKLoBytes),
                           (uint32_t)(row * C::kRow + ((c ^ kswz<D>(row)) * 16)), st + pc * 1024);
            } else if (pc < C::kKPieces) {
                // the piece's offset is wave-uniform (a scalar operand): every
                // such load of a wave shares the one lane-offset register
                dma16_rsrc_so(raw_rsrc(khat + (size_t)t * C::kKBytes, C::kKBytes), 16 * ln,
                              C::kKLoBytes + (pc - C::kKLoPieces) * 1024, st + pc * 1024);
            } else if (pc < C::kKPieces + C::kVPieces) {
                dma16_rsrc_so(raw_rsrc(vhatT + (size_t)t * C::kVBytes, C::kVBytes), 16 * ln,
                              (pc - C::kKPieces) * 1024, st + pc * 1024);
            }
        }
        if (wave == 0) {
            if (ln < 16)
                dma16_rsrc(raw_rsrc(ksc + (size_t)t * C::kKScBytes, C::kKScBytes), ln * 16,
                           st + C::kKSc);
            else if (ln < 32)
                dma16_rsrc(raw_rsrc(vscT + (size_t)t * C::kVScBytes, C::kVScBytes),
                           (ln - 16) * 16, st + C::kKSc);
        }
    };

    // Q^ fragments (B operand of QK): lane holds query my_q, channels
    // 64 hh + 32 g .. +31 for each 64-channel half hh, and their scales
    u32x4 qf[KH];
    u32x2 qh[KH];
    int qs[KH];
    {
        const int qr = min(my_q, Npad - 1);
        const size_t qrow = (size_t)bh * Npad + qr;
#pragma unroll
        for (int hh = 0; hh < KH; ++hh) {
            if constexpr (F == 4) {
                qf[hh] = ld16(w.qhat + qrow * C::kRow + (2 * hh + g) * 16);
                qh[hh] = u32x2{0, 0};
            } else {
                // read once: the non-temporal policy keeps Q^ from pushing the
                // head's K^ / V^^T (3.2 MB at d = 128, N = 16384) out of the
                // XCD's 4 MB L2 (HBM reads 564 -> 449 MB at that shape)
                const uint8_t *qt = w.qhat + (qrow / kTile) * C::kKBytes;
                qf[hh] = ld16_nt(qt + (qr % kTile) * C::kRow + (2 * hh + g) * 16);
                qh[hh] = __builtin_nontemporal_load(
                    (const u32x2 *)(qt + C::kKLoBytes + ((2 * hh + g) * kTile + kperm(qr % kTile)) * 8));
            }
            qs[hh] = w.qsc[qrow * NB + 2 * hh + g];
        }
    }
    // operand reads: per-lane byte offsets within a stage (the rest of each
    // address is an immediate)
    uint32_t k_lo[KH], k_hi = 0, k_sc = 0, v_lo = 0, v_hi = 0, v_sc = 0;
    {
        const int key0 = key_of_row(n, 0);
#pragma unroll
        for (int hh = 0; hh < KH; ++hh)
            k_lo[hh] = key0 * C::kRow + (((2 * hh + g) ^ kswz<D>(key0)) * 16);
        k_hi = C::kKLoBytes + (g * kTile + kperm(key0)) * 8;
        k_sc = C::kKSc + key0 * NB + g;
        v_lo = C::kKBytes + (g * D + n) * 16;
        v_hi = C::kKBytes + C::kVLoBytes + (g * D + n) * 8;
        v_sc = C::kVSc + g * D + n;
    }
    const float cs = a.scale * kLog2e;
    f32x16 o[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
        o[c] = f32x16{};
    float m = -INFINITY, l = 0.f;

    // two stages, loads one tile ahead (three stages, two tiles ahead,
    // measured 5% slower)
    load(0);
    for (int t = 0; t < ntiles; ++t) {
        vm_wait_all();
        __syncthreads();  // tile t is in its stage; every wave is done with tile t-1's
        load(t + 1);
        if (t >= ntw)
            continue;  // above this wave's diagonal: keep the barrier cadence only
        const uint32_t st = lds_addr(stage(t));
        // operands: K^ rows of both key blocks, V^^T rows, and their scales
        u32x4 kf[2][KH], vf[NC];
        u32x2 kh[2][KH], vh[NC];
        uint32_t ks[2][KH], vs[NC];
        if constexpr (F == 4) {
            static_for<0, 2>([&](auto bbc) {
                constexpr int bb = decltype(bbc)::value;
                static_for<0, KH>([&](auto hhc) {
                    constexpr int hh = decltype(hhc)::value;
                    kf[bb][hh] = lds_read_b128<bb * 16 * C::kRow>(st + k_lo[hh]);
                    kh[bb][hh] = u32x2{0, 0};
                    ks[bb][hh] = lds_read_u8<bb * 16 * NB + 2 * hh>(st + k_sc);
                });
            });
            static_for<0, NC>([&](auto cc) {
                constexpr int c = decltype(cc)::value;
                vf[c] = lds_read_b128<32 * c * 16>(st + v_lo);
                vh[c] = u32x2{0, 0};
                vs[c] = lds_read_u8<32 * c>(st + v_sc);
            });
        } else {
            // key block bb is key_of_row(n, 0) + 16 bb: the same swizzle, the
            // next 16 rows, the next 32 slots of the block-major area
            static_for<0, 2>([&](auto bbc) {
                constexpr int bb = decltype(bbc)::value;
                static_for<0, KH>([&](auto hhc) {
                    constexpr int hh = decltype(hhc)::value;
                    kf[bb][hh] = lds_read_b128<bb * 16 * C::kRow>(st + k_lo[hh]);
                    kh[bb][hh] = lds_read_b64<(2 * hh * kTile + 32 * bb) * 8>(st + k_hi);
                    ks[bb][hh] = lds_read_u8<bb * 16 * NB + 2 * hh>(st + k_sc);
                });
            });
        }
        // S^T = K^ Q^^T
        f32x16 s[2];
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
            s[bb] = f32x16{};
#pragma unroll
            for (int hh = 0; hh < KH; ++hh) {
                lgkm_wait<0>(kf[bb][hh]);
                asm volatile("" : "+v"(ks[bb][hh]));
                if constexpr (F == 6)
                    asm volatile("" : "+v"(kh[bb][hh]));
                s[bb] = mfma_mx<F>(mx_operand<F>(kf[bb][hh], kh[bb][hh]),
                                   mx_operand<F>(qf[hh], qh[hh]), s[bb], (int)ks[bb][hh], qs[hh]);
            }
        }
        // mask: keys past N, and above the diagonal (register r of block bb
        // is key 32 g + 16 bb + r of the tile)
        const int k0 = t * kTile;
        if ((CAUSAL && k0 + kTile - 1 > qw0) || k0 + kTile > N) {
#pragma unroll
            for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + 32 * g + 16 * bb + r;
                    if (key >= N || (CAUSAL && key > my_q))
                        s[bb][r] = -INFINITY;
                }
        }
        // exact running max (log2 units; the scale is positive)
        float smax = -INFINITY;  // this lane's 32 scores: its P block
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                smax = fmaxf(smax, s[bb][r]);
        const float tmax = max_xor32(smax) * cs;
        if (__any(tmax > m)) {
            const float m_new = fmaxf(m, tmax);
            const float alpha = fast_exp2(m - m_new);
            l *= alpha;
#pragma unroll
            for (int c = 0; c < NC; ++c)
                o[c] *= alpha;
            m = m_new;
        }
        // p for this lane's block (keys 32 g .. 32 g + 31 of the tile), its
        // row sum, and the block's MXFP4 codes against its own max.  The
        // exponent and the exponential are non-decreasing, so the block's
        // largest p is the one of its largest score.
        float p[32];
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                p[16 * bb + r] = fast_exp2(fmaf(s[bb][r], cs, -m));
                l += p[16 * bb + r];
            }
        const int pe = mx_exp<F>(fast_exp2(fmaf(smax, cs, -m)));
        i32x8 pf;
        if constexpr (F == 4) {
            pf = mx_operand<4>(fp4x32(p, pe), u32x2{0, 0});
        } else {
            const i32x6 c6 = fp6x32(p, pe);
            pf = i32x8{c6[0], c6[1], c6[2], c6[3], c6[4], c6[5], 0, 0};
            // V operands only now: with the K operands, the scores and the
            // probabilities dead, the kernel stays within its register budget
            // (the other waves of the SIMD hide the read latency)
            static_for<0, NC>([&](auto cc) {
                constexpr int c = decltype(cc)::value;
                vf[c] = lds_read_b128<32 * c * 16>(st + v_lo);
                vh[c] = lds_read_b64<32 * c * 8>(st + v_hi);
                vs[c] = lds_read_u8<32 * c>(st + v_sc);
            });
        }
        // O^T += V^^T P^^T: feature block c, A operand = feature row 32 c + n,
        // keys 32 g .. +31 of the tile with that block's scale
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            lgkm_wait<0>(vf[c]);
            asm volatile("" : "+v"(vs[c]));
            if constexpr (F == 6)
                asm volatile("" : "+v"(vh[c]));
            o[c] = mfma_mx<F>(mx_operand<F>(vf[c], vh[c]), pf, o[c], (int)vs[c], pe + 127);
        }
    }
    // O = O^T / l ; lse = (m + log2 l) ln 2 + scale * q . kmean
    const float lt = sum_xor32(l);
    if (my_q < N) {
        const float inv = 1.f / lt;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // register 4 j + i holds feature 32 c + 8 j + 4 g + i
                const int f = 32 * c + 8 * j + 4 * g;
                if constexpr (OUT_F32) {
                    float *orow = (float *)a.o + ((size_t)bh * N + my_q) * D;
                    *(f32x4 *)(orow + f) = f32x4{o[c][4 * j] * inv, o[c][4 * j + 1] * inv,
                                                 o[c][4 * j + 2] * inv, o[c][4 * j + 3] * inv};
                } else {
                    uint16_t *orow = (uint16_t *)a.o + ((size_t)bh * N + my_q) * D;
                    const u32x2 wv = {pack_bf16x2(o[c][4 * j] * inv, o[c][4 * j + 1] * inv),
                                      pack_bf16x2(o[c][4 * j + 2] * inv, o[c][4 * j + 3] * inv)};
                    *(u32x2 *)(orow + f) = wv;
                }
            }
        }
        if (a.lse && g == 0)
            a.lse[(size_t)bh * N + my_q] =
                (m + log2f(lt)) * kLn2 + a.scale * w.qkdot[(size_t)bh * N + my_q];
    }
}

template <int D, int F, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(kAThreads) __attribute__((amdgpu_waves_per_eu(3, 3))) void mx_attn_kernel(PrefillArgs a, MxWs w)
{
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kStages * MCfg<D, F>::kStage];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nqt = (a.N + kBM - 1) / kBM;
    // causal: workgroup j of a head takes query tiles nqt-1-j and j (equal work)
    const int nw = CAUSAL ? (nqt + 1) / 2 : nqt;
    const int BH = a.B * a.H;
    int bh, j;
    const int wg = blockIdx.x;
    if ((BH & 7) == 0) {
        // workgroup i runs on XCD i % 8: keep a head's workgroups on one XCD
        const int xcd = wg & 7, slot = wg >> 3;
        bh = xcd + 8 * (slot / nw);
        j = slot % nw;
    } else {
        bh = wg / nw;
        j = wg % nw;
    }
    if (CAUSAL) {
        mx_qtile<D, F, CAUSAL, OUT_F32>(a, w, smem, bh, nqt - 1 - j, wave, lane);
        if (j < nqt - 1 - j) {
            __syncthreads();  // every wave is done with the LDS stages
            mx_qtile<D, F, CAUSAL, OUT_F32>(a, w, smem, bh, j, wave, lane);
        }
    } else {
        mx_qtile<D, F, CAUSAL, OUT_F32>(a, w, smem, bh, j, wave, lane);
    }
}

template <int D, int F>
hipError_t launch_d(const SageArgs &sa, hipStream_t s)
{
    const PrefillArgs &a = sa.p;
    const MxWs w = mx_carve(sa.workspace, a.B, a.H, a.Hkv, a.N, D, F);
    const int Npad = (a.N + kTile - 1) / kTile * kTile;
    const int BG = a.B * a.Hkv, BH = a.B * a.H;
    const uint16_t *q = (const uint16_t *)a.q, *k = (const uint16_t *)a.k,
                   *v = (const uint16_t *)a.v;
    {
        ProfScope ps("mx_ksum", s);
        hipLaunchKernelGGL(mx_ksum_kernel<D>, dim3(BG, kNCh), dim3(kThreads), 0, s, k, w, a.N);
    }
    {
        ProfScope ps("mx_kmean", s);
        hipLaunchKernelGGL(mx_kmean_kernel<D>, dim3(BG), dim3(D), 0, s, w, a.N);
    }
    {
        const long long rows = (long long)(BH + BG) * Npad;  // 64 rows per workgroup
        if constexpr (F == 4) {
            ProfScope ps("mx_quant_qk", s);
            hipLaunchKernelGGL(mx_quant_qk_kernel<D>, dim3((unsigned)(rows / kTile)),
                               dim3(kThreads), 0, s, q, k, w, a.B, a.H, a.Hkv, a.N);
        } else {
            ProfScope ps("mx6_quant_qk", s);
            hipLaunchKernelGGL(mx6_quant_qk_kernel<D>, dim3((unsigned)(rows / kTile)),
                               dim3(kThreads), 0, s, q, k, w, a.B, a.H, a.Hkv, a.N);
        }
    }
    {
        ProfScope ps(F == 4 ? "mx_quant_v" : "mx6_quant_v", s);
        hipLaunchKernelGGL((mx_quant_v_kernel<D, F>), dim3(BG, Npad / kTile), dim3(kThreads), 0, s,
                           v, w, a.N);
    }
    const int nqt = (a.N + kBM - 1) / kBM;
    const dim3 grid(BH * (a.causal ? (nqt + 1) / 2 : nqt)), block(kAThreads);
    ProfScope ps(F == 4 ? "mx_attn" : "mx6_attn", s);
    if (a.causal) {
        if (a.out_fp32)
            hipLaunchKernelGGL((mx_attn_kernel<D, F, true, true>), grid, block, 0, s, a, w);
        else
            hipLaunchKernelGGL((mx_attn_kernel<D, F, true, false>), grid, block, 0, s, a, w);
    } else {
        if (a.out_fp32)
            hipLaunchKernelGGL((mx_attn_kernel<D, F, false, true>), grid, block, 0, s, a, w);
        else
            hipLaunchKernelGGL((mx_attn_kernel<D, F, false, false>), grid, block, 0, s, a, w);
    }
    return hipGetLastError();
}

}  // namespace

size_t mx_workspace_bytes(int B, int H, int Hkv, int N, int d, int elem_bits)
{
    size_t off[10];
    mx_layout(B, H, Hkv, N, d, elem_bits, off);
    return off[9];
}

void mx_workspace_layout(int B, int H, int Hkv, int N, int d, int elem_bits, size_t *offsets)
{
    size_t off[10];
    mx_layout(B, H, Hkv, N, d, elem_bits, off);
    for (int i = 0; i < kMxWsPieces; ++i)
        offsets[i] = off[i];
}

hipError_t launch_mx(const SageArgs &sa, int elem_bits, hipStream_t s)
{
    if (elem_bits == 6)
        return sa.p.d == 64 ? launch_d<64, 6>(sa, s) : launch_d<128, 6>(sa, s);
    return sa.p.d == 64 ? launch_d<64, 4>(sa, s) : launch_d<128, 4>(sa, s);
}

}  // namespace attn
