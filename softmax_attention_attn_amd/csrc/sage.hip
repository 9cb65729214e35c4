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
#include "attn_internal.hpp"
#include "cdna4.hpp"

namespace attn {
namespace {

constexpr int kBlk = 64;   // quantisation block = key tile (tokens)
constexpr int kNCh = 16;   // sequence chunks of the statistics pass
constexpr int kThreads = 256;
constexpr float kLog2_448 = 8.807354922057604f;

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

SageWs carve(void *base, int B, int H, int Hkv, int N, int d)
{
    const size_t BH = (size_t)B * H, BG = (size_t)B * Hkv;
    const size_t nblk = (N + kBlk - 1) / kBlk, Npad = nblk * kBlk;
    char *p = (char *)base;
    SageWs w;
    auto take = [&](size_t bytes) {
        char *r = p;
        p += align256(bytes);
        return r;
    };
    w.ksum_part = (double *)take(sizeof(double) * BG * kNCh * d);
    w.vmax_part = (float *)take(sizeof(float) * BG * kNCh * d);
    w.kmean = (float *)take(sizeof(float) * BG * d);
    w.vscale = (float *)take(sizeof(float) * BG * d);
    w.vinv = (float *)take(sizeof(float) * BG * d);
    w.qdelta = (float *)take(sizeof(float) * BH * nblk);
    w.kdelta = (float *)take(sizeof(float) * BG * nblk);
    w.qkdot = (float *)take(sizeof(float) * BH * N);
    w.qhat = (int8_t *)take(BH * Npad * d);
    w.khat = (int8_t *)take(BG * Npad * d);
    w.vhatT = (uint8_t *)take(BG * d * Npad);
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
    for (int r = r0 + rg; r < r1; r += RPP) {
        const u32x4 kw = ld16(kb + (size_t)r * D + fc * 8);
        const u32x4 vw = ld16(vb + (size_t)r * D + fc * 8);
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
// Thread t owns row t / 4 and channels (t % 4) * D/4 .. + D/4.
template <int D>
__global__ __launch_bounds__(kThreads) void sage_quant_qk_kernel(const uint16_t *q, const uint16_t *k,
                                                                 SageWs w, int B, int H, int Hkv,
                                                                 int N)
{
    constexpr int CPT = D / 4;  // channels per thread
    __shared__ float scratch[4];
    const int nblk = (N + kBlk - 1) / kBlk, Npad = nblk * kBlk;
    const int tid = threadIdx.x, row = tid >> 2, c0 = (tid & 3) * CPT;
    int id = blockIdx.x;
    const bool is_q = id < B * H * nblk;
    if (!is_q)
        id -= B * H * nblk;
    const int seq = id / nblk, blk = id % nblk;  // seq = b*H + h or b*Hkv + g
    const int tok = blk * kBlk + row;
    const uint16_t *src = (is_q ? q : k) + ((size_t)seq * N + tok) * D + c0;
    const int g = is_q ? (seq / H) * Hkv + (seq % H) / (H / Hkv) : seq;
    const float *km = w.kmean + (size_t)g * D + c0;

    float x[CPT];
    if (tok < N) {
#pragma unroll
        for (int j = 0; j < CPT / 8; ++j) {
            const u32x4 u = ld16(src + 8 * j);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[8 * j + 2 * e] = bf16_lo(u[e]);
                x[8 * j + 2 * e + 1] = bf16_hi(u[e]);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < CPT; ++i)
            x[i] = 0.f;
    }
    if (is_q) {
        // q . kmean for the LSE correction
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < CPT; ++i)
            dot = fmaf(x[i], km[i], dot);
        dot += __shfl_xor(dot, 1, 64);
        dot += __shfl_xor(dot, 2, 64);
        if ((tid & 3) == 0 && tok < N)
            w.qkdot[(size_t)seq * N + tok] = dot;
    } else if (tok < N) {
#pragma unroll
        for (int i = 0; i < CPT; ++i)
            x[i] -= km[i];
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < CPT; ++i)
        amax = fmaxf(amax, fabsf(x[i]));
    amax = block_max_256(amax, scratch);
    const float inv = amax > 0.f ? 127.f / amax : 1.f;
    if (tid == 0)
        (is_q ? w.qdelta : w.kdelta)[(size_t)seq * nblk + blk] = amax > 0.f ? amax / 127.f : 1.f;
    int8_t *dst = (is_q ? w.qhat : w.khat) + ((size_t)seq * Npad + tok) * D + c0;
#pragma unroll
    for (int j = 0; j < CPT / 16; ++j) {
        u32x4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int b = 16 * j + 4 * e;
            out[e] = (uint32_t)(q_i8(x[b], inv) & 0xff) | ((uint32_t)(q_i8(x[b + 1], inv) & 0xff) << 8) |
                     ((uint32_t)(q_i8(x[b + 2], inv) & 0xff) << 16) |
                     ((uint32_t)(q_i8(x[b + 3], inv) & 0xff) << 24);
        }
        st16(dst + 16 * j, out);
    }
}

// E4M3 of V / delta_V (round to nearest even, saturated to +-448) for one
// 64-key tile, written feature-major: vhatT[bg][c][tile*64 + key].
template <int D>
__global__ __launch_bounds__(kThreads) void sage_quant_v_kernel(const uint16_t *v, SageWs w, int N)
{
    constexpr int CPT = D / 4;
    __shared__ __attribute__((aligned(16))) uint8_t tile[D][kBlk];
    const int nblk = (N + kBlk - 1) / kBlk, Npad = nblk * kBlk;
    const int bg = blockIdx.x, blk = blockIdx.y, tid = threadIdx.x;
    const int row = tid >> 2, c0 = (tid & 3) * CPT;
    const int tok = blk * kBlk + row;
    const float *vi = w.vinv + (size_t)bg * D + c0;
#pragma unroll
    for (int j = 0; j < CPT / 8; ++j) {
        u32x4 u = {0, 0, 0, 0};
        if (tok < N)
            u = ld16(v + ((size_t)bg * N + tok) * D + c0 + 8 * j);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const int c = 8 * j + e;
            float a = bf16_lo(u[e >> 1]);
            float b = bf16_hi(u[e >> 1]);
            a = fminf(fmaxf(a * vi[c], -448.f), 448.f);
            b = fminf(fmaxf(b * vi[c + 1], -448.f), 448.f);
            const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
            tile[c0 + c][row] = (uint8_t)(pk & 0xff);
            tile[c0 + c + 1][row] = (uint8_t)((pk >> 8) & 0xff);
        }
    }
    __syncthreads();
    // D rows x 64 bytes = D*4 chunks of 16 bytes
    for (int i = tid; i < D * 4; i += kThreads) {
        const int c = i >> 2, part = i & 3;
        st16(w.vhatT + ((size_t)bg * D + c) * Npad + blk * kBlk + part * 16,
             *(const u32x4 *)&tile[c][part * 16]);
    }
}

// ----------------------------------------------------------------- attention

constexpr int kWaves = 8;
constexpr int kAThreads = 64 * kWaves;
constexpr int kQW = 32;
constexpr int kBM = kQW * kWaves;

template <int D>
struct SCfg {
    static constexpr int kKRow = D;                        // K^ row bytes
    static constexpr int kKChunks = D / 16;
    static constexpr int kKBytes = kBlk * D;               // K^ tile
    static constexpr int kVBytes = D * kBlk;               // V^^T tile
    static constexpr int kStage = kKBytes + kVBytes;
    static constexpr int kKPieces = kKBytes / 1024;
    static constexpr int kVPieces = kVBytes / 1024;
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

template <int D>
__device__ __forceinline__ void issue_tile(unsigned char *stage, const int8_t *khat,
                                           const uint8_t *vhatT, int Npad, int k0, int wave,
                                           int lane)
{
    constexpr int C = SCfg<D>::kKChunks;
    for (int piece = wave; piece < SCfg<D>::kKPieces; piece += kWaves) {
        const int p = piece * 64 + lane, row = p / C;
        const int c = (p % C) ^ kswz<D>(row);
        dma16(khat + (size_t)(k0 + row) * D + c * 16, stage + piece * 1024);
    }
    for (int piece = wave; piece < SCfg<D>::kVPieces; piece += kWaves) {
        const int p = piece * 64 + lane, d = p >> 2;
        const int c = (p & 3) ^ vswz(d);
        dma16(vhatT + (size_t)d * Npad + k0 + c * 16, stage + SCfg<D>::kKBytes + piece * 1024);
    }
}

template <int D, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(kAThreads) void sage_attn_kernel(PrefillArgs a, SageWs w)
{
    constexpr int kStage = SCfg<D>::kStage;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * kStage];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, n = lane & 31;
    const int N = a.N, nblk = (N + kBlk - 1) / kBlk, Npad = nblk * kBlk;
    const int nqt = (N + kBM - 1) / kBM;
    const int BH = a.B * a.H;
    int bh, qi;
    const int wg = blockIdx.x;
    if ((BH & 7) == 0) {
        const int xcd = wg & 7, slot = wg >> 3;
        bh = xcd + 8 * (slot / nqt);
        qi = slot % nqt;
    } else {
        bh = wg / nqt;
        qi = wg % nqt;
    }
    const int qt = CAUSAL ? nqt - 1 - qi : qi;
    const int h = bh % a.H, b = bh / a.H;
    const int bg = b * a.Hkv + h / (a.H / a.Hkv);
    const int q0 = qt * kBM, qw0 = q0 + wave * kQW, my_q = qw0 + n;
    const int8_t *khat = w.khat + (size_t)bg * Npad * D;
    const uint8_t *vhatT = w.vhatT + (size_t)bg * D * Npad;
    const int kend = CAUSAL ? min(N, q0 + kBM) : N;
    const int ntiles = (kend + kBlk - 1) / kBlk;

    issue_tile<D>(smem, khat, vhatT, Npad, 0, wave, lane);

    // Q^^T fragments (B operand of the INT8 MFMA, K = 32 per step): lane holds
    // Q^[my_q][32*ks + 16*g .. +15].  Rows past N are zero in the workspace.
    i32x4 qf[D / 32];
    const int8_t *qrow = w.qhat + ((size_t)bh * Npad + min(my_q, Npad - 1)) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
        qf[ks] = __builtin_bit_cast(i32x4, ld16(qrow + ks * 32 + g * 16));
    // the 32 queries of a wave lie in one 64-token block
    const float dq = w.qdelta[(size_t)bh * nblk + min(qw0, N - 1) / kBlk];
    const float cq = a.scale * kLog2e * dq;
    const float *kdel = w.kdelta + (size_t)bg * nblk;

    const int krow = perm32(n);  // K^ row of MFMA row n, + 32*blk
    f32x16 o[D / 32];
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
        o[c] = f32x16{};
    float m = -INFINITY, l = 0.f;
    // the K scale of tile t is read one tile ahead, before the next tile's
    // direct loads are issued, so that waiting for it never waits for them
    float kd_next = kdel[0];

    for (int t = 0; t < ntiles; ++t) {
        const int k0 = t * kBlk;
        unsigned char *stage = smem + (t & 1) * kStage;
        vm_wait_all();
        __syncthreads();
        const float kd = kd_next;
        if (t + 1 < ntiles) {
            kd_next = kdel[t + 1];
            issue_tile<D>(smem + ((t + 1) & 1) * kStage, khat, vhatT, Npad, k0 + kBlk, wave, lane);
        }
        if (CAUSAL && k0 > qw0 + kQW - 1)
            continue;

        // S^T = K^ Q^^T (exact int32)
        i32x16 s[2] = {i32x16{}, i32x16{}};
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const int row = 32 * blk + krow;
            const int sw = kswz<D>(row);
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
                const int chunk = (2 * ks + g) ^ sw;
                const i32x4 ka = *(const i32x4 *)(stage + row * D + chunk * 16);
                s[blk] = mfma_i8_32x32x32(ka, qf[ks], s[blk]);
            }
        }

        // scores in log2 units: S * log2e = c * int (c > 0).  The tile max is
        // taken on the integers (masked keys as INT_MIN), the exponent
        // 2^(c*int + log2(448) - m) with one FMA per score; on tiles that
        // need the mask, masked keys get -inf (a key masked through INT_MIN
        // alone would not vanish when c is tiny).
        const float c = cq * kd;
        const bool need_mask = (CAUSAL && k0 + kBlk - 1 > qw0) || k0 + kBlk > N;
        int imx = INT_MIN;
        if (need_mask) {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + 32 * blk + 16 * g + r;
                    if (key >= N || (CAUSAL && key > my_q))
                        s[blk][r] = INT_MIN;
                }
        }
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int r = 0; r < 16; r += 2)
                imx = vmax3_i32(imx, s[blk][r], s[blk][r + 1]);
        // a row with every key of the tile masked contributes -inf
        const float mx = max_xor32(imx == INT_MIN ? -INFINITY : (float)imx * c);
        // exact running max (P is quantised against it)
        if (__any(mx > m)) {
            const float m_new = fmaxf(m, mx);
            const float alpha = fast_exp2(m - m_new);
            l *= alpha;
#pragma unroll
            for (int cc = 0; cc < D / 32; ++cc)
                o[cc] *= alpha;
            m = m_new;
        }
        // p = 448 * 2^(c*int - m) <= 448; E4M3 codes packed 4 per dword:
        // byte 16*blk + r of the lane = key 32*blk + 16*g + r
        uint32_t pk[8];
        float rs0 = 0.f, rs1 = 0.f;
        const float bias = kLog2_448 - m;
        auto expo = [&](int v) {
            const float x = fmaf((float)v, c, bias);
            return fast_exp2(need_mask && v == INT_MIN ? -INFINITY : x);
        };
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int r = 0; r < 16; r += 4) {
                const float p0 = expo(s[blk][r]);
                const float p1 = expo(s[blk][r + 1]);
                const float p2 = expo(s[blk][r + 2]);
                const float p3 = expo(s[blk][r + 3]);
                rs0 += p0 + p2;
                rs1 += p1 + p3;
                int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
                wd = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, wd, true);
                pk[4 * blk + r / 4] = (uint32_t)wd;
            }
        l += rs0 + rs1;

        // O^T += V^^T P^^T (FP8, K = 64 keys per MFMA)
        const i32x8 pb = {(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3],
                          (int)pk[4], (int)pk[5], (int)pk[6], (int)pk[7]};
        const unsigned char *vt = stage + SCfg<D>::kKBytes;
#pragma unroll
        for (int cc = 0; cc < D / 32; ++cc) {
            const int d = 32 * cc + perm32(n);
            const int sw = vswz(d);
            const u32x4 lo = *(const u32x4 *)(vt + d * kBlk + ((g ^ sw) << 4));
            const u32x4 hi = *(const u32x4 *)(vt + d * kBlk + (((2 + g) ^ sw) << 4));
            const i32x8 va = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                              (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            o[cc] = mfma_fp8_32x32x64(va, pb, o[cc]);
        }
    }

    // O = acc * delta_V / l448 ; lse = (m + log2 l448 - log2 448) ln2 + scale * q.kmean
    const float lt = sum_xor32(l);
    if (my_q < N) {
        const float inv = 1.f / lt;
        const float *vs = w.vscale + (size_t)bg * D;
#pragma unroll
        for (int cc = 0; cc < D / 32; ++cc) {
            float val[16];
#pragma unroll
            for (int r = 0; r < 16; ++r)
                val[r] = o[cc][r] * vs[32 * cc + 16 * g + r] * inv;
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
            a.lse[(size_t)bh * N + my_q] = (m + log2f(lt) - kLog2_448) * kLn2 +
                                           a.scale * w.qkdot[(size_t)bh * N + my_q];
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
    dim3 grid(BH * nqt), block(kAThreads);
    if (a.causal) {
        if (a.out_fp32)
            hipLaunchKernelGGL((sage_attn_kernel<D, true, true>), grid, block, 0, s, a, w);
        else
            hipLaunchKernelGGL((sage_attn_kernel<D, true, false>), grid, block, 0, s, a, w);
    } else {
        if (a.out_fp32)
            hipLaunchKernelGGL((sage_attn_kernel<D, false, true>), grid, block, 0, s, a, w);
        else
            hipLaunchKernelGGL((sage_attn_kernel<D, false, false>), grid, block, 0, s, a, w);
    }
    return hipGetLastError();
}

}  // namespace

size_t sage_workspace_bytes(int B, int H, int Hkv, int N, int d)
{
    const size_t BH = (size_t)B * H, BG = (size_t)B * Hkv;
    const size_t nblk = (N + kBlk - 1) / kBlk, Npad = nblk * kBlk;
    return align256(sizeof(double) * BG * kNCh * d) + align256(sizeof(float) * BG * kNCh * d) +
           align256(sizeof(float) * BG * d) * 3 +
           align256(sizeof(float) * BH * nblk) + align256(sizeof(float) * BG * nblk) +
           align256(sizeof(float) * BH * N) + align256(BH * Npad * d) + align256(BG * Npad * d) +
           align256(BG * d * Npad);
}

hipError_t launch_sage(const SageArgs &sa, hipStream_t s)
{
    return sa.p.d == 64 ? launch_d<64>(sa, s) : launch_d<128>(sa, s);
}

}  // namespace attn
