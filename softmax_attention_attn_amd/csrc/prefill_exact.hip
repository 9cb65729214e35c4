// Exact bf16 fused attention forward for gfx950.
//
// Dataflow ("flashattention-kernels" page, §0/§1; "cuda-kernel-pretrain"
// page, §2): one workgroup owns a tile of kBM queries of one (batch, head);
// each of its 4 waves keeps the Q fragments of its 32 queries in registers
// for the whole pass; K and V tiles of kBN keys stream through a double
// buffered LDS stage; an online softmax (running row max m and row sum l,
// rescaled per tile) accumulates O without ever writing scores to memory;
// causal tiles entirely above the diagonal are never loaded.
//
// MFMA orientation: each wave computes S^T = K Q^T (keys are MFMA rows,
// queries are columns) so that a lane owns one query column and 16 keys of
// it.  Row reductions over keys are then 16-register in-lane reductions plus
// one exchange with lane l ^ 32.  The probability fragment P^T produced in the
// accumulator registers is directly the B operand of O^T = V^T P^T once
// rounded to bf16: K rows are loaded in the permuted order perm32() so that
// accumulator register r of lane group g holds key 16*g + r, and V^T is
// kept in LDS so that the matching A operand is one 16-byte read.
//
// Work partitioning (FlashAttention-2 style, same page §2): the grid is
// (B*H, query tiles); the heaviest causal tiles are dispatched first and, for
// B*H a multiple of 8, consecutive workgroups of one head land on the same
// XCD (workgroups are dealt to the 8 XCDs round robin), so the K/V of a head
// is shared through one L2 ("GPU kernel overview" page, NUMA-aware attention
// entry: head-first chiplet mapping).
#include "attn_internal.hpp"
#include "cdna4.hpp"

namespace attn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kQW = 32;            // queries per wave
constexpr int kBM = kQW * kWaves;  // queries per workgroup
constexpr int kBN = 64;            // keys per tile

// Row m of a 32-row MFMA block is loaded from index perm32(m), so that lane
// group g = l/32 holds the 16 consecutive indices 16g .. 16g+15 in registers
// r = 0..15 of the 32x32 accumulator.
__device__ __forceinline__ int perm32(int m) { return ((m >> 2) & 1) * 16 + (m >> 3) * 4 + (m & 3); }

template <int D>
struct Cfg {
    static constexpr int kChunks = D / 8;                       // 16-byte chunks per row
    static constexpr int kKBytes = kBN * D * 2;                 // K tile, [kBN][D]
    static constexpr int kVBytes = D * kBN * 2;                 // V^T tile, [D][kBN]
    static constexpr int kStage = kKBytes + kVBytes;
    static constexpr int kSmem = 2 * kStage;                    // double buffer
    static constexpr int kKLoads = kBN * kChunks / kThreads;    // 16-byte K loads per thread
    static constexpr int kVSub = (kBN / 4) * kChunks;           // 4-key x 8-feature V blocks
    static_assert(kKLoads * kThreads == kBN * kChunks, "K tile split");
    static_assert(kVSub <= kThreads, "one V block per thread");
};

// K tile: byte offset of 16-byte chunk c of row `row` (XOR swizzled so the
// 32 rows read by one MFMA operand load fall on distinct bank groups).
template <int D>
__device__ __forceinline__ int k_off(int row, int c)
{
    int sw = (D >= 128) ? ((row & 7) | (((row >> 4) & 1) << 3)) : (row & 7);
    return row * (D * 2) + ((c ^ sw) << 4);
}

// V^T tile: byte offset of 16-byte chunk c (8 keys) of feature row d.
__device__ __forceinline__ int vt_off(int d, int c)
{
    int sw = ((d >> 1) & 3) | ((d >> 2) & 4);
    return d * (kBN * 2) + ((c ^ sw) << 4);
}

template <int D>
struct TileRegs {
    u32x4 k[Cfg<D>::kKLoads];
    u32x4 v[4];
};

template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D> &r, const uint16_t *kb, const uint16_t *vb,
                                          int k0, int N, int tid)
{
    constexpr int C = Cfg<D>::kChunks;
#pragma unroll
    for (int i = 0; i < Cfg<D>::kKLoads; ++i) {
        int c = tid + i * kThreads;
        int key = k0 + c / C;
        r.k[i] = key < N ? ld16(kb + (size_t)key * D + (c % C) * 8) : u32x4{0, 0, 0, 0};
    }
    if (tid < Cfg<D>::kVSub) {
        int kq = tid / C, dc = tid % C;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int key = k0 + 4 * kq + j;
            r.v[j] = key < N ? ld16(vb + (size_t)key * D + dc * 8) : u32x4{0, 0, 0, 0};
        }
    }
}

template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D> &r, unsigned char *stage, int tid)
{
    constexpr int C = Cfg<D>::kChunks;
#pragma unroll
    for (int i = 0; i < Cfg<D>::kKLoads; ++i) {
        int c = tid + i * kThreads;
        *(u32x4 *)(stage + k_off<D>(c / C, c % C)) = r.k[i];
    }
    if (tid < Cfg<D>::kVSub) {
        unsigned char *vs = stage + Cfg<D>::kKBytes;
        int kq = tid / C, dc = tid % C;
        // transpose the 4 keys x 8 features block: feature e of key j is
        // bf16 e of r.v[j]
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint32_t w[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                w[j] = (e & 1) ? (r.v[j][e >> 1] >> 16) : (r.v[j][e >> 1] & 0xffffu);
            u32x2 pair = {w[0] | (w[1] << 16), w[2] | (w[3] << 16)};
            *(u32x2 *)(vs + vt_off(dc * 8 + e, kq >> 1) + (kq & 1) * 8) = pair;
        }
    }
}

template <int D, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(kThreads) void prefill_exact_kernel(PrefillArgs a)
{
    __shared__ __attribute__((aligned(16))) unsigned char smem[Cfg<D>::kSmem];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, n = lane & 31;
    const int bh = blockIdx.x;
    const int h = bh % a.H, b = bh / a.H;
    const int nqt = gridDim.y;
    const int qt = CAUSAL ? (nqt - 1 - (int)blockIdx.y) : (int)blockIdx.y;
    const int q0 = qt * kBM;
    const int N = a.N;
    const int kvh = h / (a.H / a.Hkv);
    const uint16_t *qb = (const uint16_t *)a.q + (size_t)bh * N * D;
    const uint16_t *kb = (const uint16_t *)a.k + (size_t)(b * a.Hkv + kvh) * N * D;
    const uint16_t *vb = (const uint16_t *)a.v + (size_t)(b * a.Hkv + kvh) * N * D;
    const int qw0 = q0 + wave * kQW;
    const int my_q = qw0 + n;

    // Q^T fragments (B operand): lane holds Q[my_q][16*ks + 8*g .. +7].
    bf16x8 qf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
        qf[ks] = as_bf16x8(my_q < N ? ld16(qb + (size_t)my_q * D + ks * 16 + g * 8)
                                    : u32x4{0, 0, 0, 0});

    const int kend = CAUSAL ? min(N, q0 + kBM) : N;
    const int ntiles = (kend + kBN - 1) / kBN;

    TileRegs<D> regs;
    load_tile<D>(regs, kb, vb, 0, N, tid);
    store_tile<D>(regs, smem, tid);
    __syncthreads();

    f32x16 o[D / 32];
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
        o[c] = f32x16{};
    float m = -INFINITY;  // running max of score * scale * log2(e)
    float l = 0.f;        // this lane's part of the running sum (16 of every 32 keys)
    const float cs = a.scale * kLog2e;

    for (int t = 0; t < ntiles; ++t) {
        const int k0 = t * kBN;
        const int stage = t & 1;
        if (t + 1 < ntiles)
            load_tile<D>(regs, kb, vb, k0 + kBN, N, tid);

        const bool active = !CAUSAL || k0 <= qw0 + kQW - 1;
        if (active) {
            const unsigned char *ks_ = smem + stage * Cfg<D>::kStage;
            const unsigned char *vs_ = ks_ + Cfg<D>::kKBytes;
            f32x16 s[2];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                s[blk] = f32x16{};
                const int row = 32 * blk + perm32(n);
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks) {
                    bf16x8 ka = as_bf16x8(*(const u32x4 *)(ks_ + k_off<D>(row, 2 * ks + g)));
                    s[blk] = mfma_bf16_32x32x16(ka, qf[ks], s[blk]);
                }
            }
            const bool need_mask = (CAUSAL && k0 + kBN - 1 > qw0) || (k0 + kBN > N);
            if (need_mask) {
#pragma unroll
                for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        int key = k0 + 32 * blk + 16 * g + r;
                        if (key >= N || (CAUSAL && key > my_q))
                            s[blk][r] = -INFINITY;
                    }
            }
            float mx = s[0][0];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    mx = fmaxf(mx, s[blk][r]);
            mx = fmaxf(mx, xor32(mx));
            const float m_new = fmaxf(m, mx * cs);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = fast_exp2(m - m_use);
            l *= alpha;
#pragma unroll
            for (int c = 0; c < D / 32; ++c)
                o[c] *= alpha;
            m = m_new;

            uint32_t pk[2][8];
            float rs = 0.f;
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    float p0 = fast_exp2(fmaf(s[blk][r], cs, -m_use));
                    float p1 = fast_exp2(fmaf(s[blk][r + 1], cs, -m_use));
                    rs += p0 + p1;
                    pk[blk][r >> 1] = pack_bf16x2(p0, p1);
                }
            l += rs;

#pragma unroll
            for (int c = 0; c < D / 32; ++c) {
                const int vrow = 32 * c + perm32(n);
#pragma unroll
                for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        bf16x8 va = as_bf16x8(
                            *(const u32x4 *)(vs_ + vt_off(vrow, 4 * blk + 2 * g + hh)));
                        u32x4 pw = {pk[blk][4 * hh], pk[blk][4 * hh + 1], pk[blk][4 * hh + 2],
                                    pk[blk][4 * hh + 3]};
                        o[c] = mfma_bf16_32x32x16(va, as_bf16x8(pw), o[c]);
                    }
            }
        }
        if (t + 1 < ntiles)
            store_tile<D>(regs, smem + (stage ^ 1) * Cfg<D>::kStage, tid);
        __syncthreads();
    }

    const float lt = l + xor32(l);
    if (my_q < N) {
        const float inv = 1.f / lt;
        if constexpr (OUT_F32) {
            float *orow = (float *)a.o + ((size_t)bh * N + my_q) * D;
#pragma unroll
            for (int c = 0; c < D / 32; ++c)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    f32x4 w = {o[c][4 * j] * inv, o[c][4 * j + 1] * inv, o[c][4 * j + 2] * inv,
                               o[c][4 * j + 3] * inv};
                    *(f32x4 *)(orow + 32 * c + 16 * g + 4 * j) = w;
                }
        } else {
            uint16_t *orow = (uint16_t *)a.o + ((size_t)bh * N + my_q) * D;
#pragma unroll
            for (int c = 0; c < D / 32; ++c)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    u32x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        w[e] = pack_bf16x2(o[c][8 * j + 2 * e] * inv, o[c][8 * j + 2 * e + 1] * inv);
                    st16(orow + 32 * c + 16 * g + 8 * j, w);
                }
        }
        if (a.lse && g == 0)
            a.lse[(size_t)bh * N + my_q] = (m + log2f(lt)) * kLn2;
    }
}

template <int D, bool CAUSAL, bool OUT_F32>
hipError_t launch_t(const PrefillArgs &a, hipStream_t s)
{
    dim3 grid(a.B * a.H, (a.N + kBM - 1) / kBM);
    ProfScope ps("prefill_exact", s);
    hipLaunchKernelGGL((prefill_exact_kernel<D, CAUSAL, OUT_F32>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PrefillArgs &a, hipStream_t s)
{
    if (a.causal)
        return a.out_fp32 ? launch_t<D, true, true>(a, s) : launch_t<D, true, false>(a, s);
    return a.out_fp32 ? launch_t<D, false, true>(a, s) : launch_t<D, false, false>(a, s);
}

}  // namespace

hipError_t launch_prefill_exact(const PrefillArgs &a, hipStream_t s)
{
    return a.d == 64 ? launch_d<64>(a, s) : launch_d<128>(a, s);
}

}  // namespace attn
