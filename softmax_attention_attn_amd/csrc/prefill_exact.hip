// Exact bf16 fused attention forward for gfx950.
//
// Dataflow ("flashattention-kernels" page, §0/§1; "cuda-kernel-pretrain"
// page, §2): one workgroup owns a tile of kBM = 256 queries of one
// (batch, head); each of its 8 waves keeps the Q fragments of its 32 queries
// in registers for the whole pass; K and V tiles of kBN = 64 keys stream
// through a double-buffered LDS stage; an online softmax (running row max m
// and row sum l) accumulates O in registers without ever writing scores to
// memory; causal tiles entirely above the diagonal are never loaded.
//
// gfx950 mapping:
//  * 8 waves = 2 per SIMD, each within 256 registers, so that one wave's
//    transcendental softmax work overlaps the other wave's MFMAs.
//  * K and V tiles go from global memory straight into LDS with 16-byte
//    global_load_lds (no register staging); 16-byte chunks are XOR-swizzled
//    by row so that MFMA operand reads hit distinct LDS banks.
//  * Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys are
//    rows, queries columns): a lane owns one query column and 16 keys of a
//    32-key block, so row reductions are in-lane plus one permlane32 swap.
//    K rows are read in the order perm32() so that accumulator register r of
//    lane half g holds key 16g + r; the bf16-rounded probabilities in those
//    registers are then directly the B operand of O^T = V^T P^T.
//  * The V^T operand comes from the row-major V tile through the transposing
//    LDS read ds_read_b64_tr_b16 (within a 16-lane group, output lane i,
//    element j is element i%4 of the 8 bytes addressed by lane 4j + i/4).
//  * Lazy rescaling: the running max used for the exponent is only raised
//    when a tile's max exceeds it by more than 2^8, so P stays <= 256 and the
//    O / l rescale is skipped on most tiles; the result is unchanged because
//    the same stale max enters numerator and denominator.
//  * Grid: one workgroup per (b*H + h, query tile).  Workgroup i runs on XCD
//    i % 8, so when B*H is a multiple of 8 consecutive slots of one XCD are
//    mapped to the query tiles of one head (heaviest causal tile first): the
//    head's K/V stays in that XCD's L2 ("GPU kernel overview" page,
//    NUMA-aware attention entry: head-first chiplet swizzle).
#include "attn_internal.hpp"
#include "cdna4.hpp"

namespace attn {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kQW = 32;            // queries per wave
constexpr int kBM = kQW * kWaves;  // queries per workgroup
constexpr int kBN = 64;            // keys per tile
constexpr float kRescaleLog2 = 8.f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Row m of a 32-row MFMA block is taken from index perm32(m): lane half g
// then holds indices 16g .. 16g+15 in accumulator registers 0..15.
__device__ __forceinline__ int perm32(int m) { return ((m >> 2) & 1) * 16 + (m >> 3) * 4 + (m & 3); }

template <int D>
struct Cfg {
    static constexpr int kChunks = D / 8;                 // 16-byte chunks per row
    static constexpr int kTileBytes = kBN * D * 2;        // one K or V tile
    static constexpr int kStage = 2 * kTileBytes;         // K + V
    static constexpr int kSmem = 2 * kStage;              // double buffer
    static constexpr int kLoads = kBN * kChunks / 64 / kWaves;  // 1 KB loads per wave per tile
    static_assert(kLoads * 64 * kWaves == kBN * kChunks, "tile split");
};

template <int D>
__device__ __forceinline__ int swz_k(int row)
{
    return ((row & 7) | (((row >> 4) & 1) << 3)) & (Cfg<D>::kChunks - 1);
}
template <int D>
__device__ __forceinline__ int swz_v(int row) { return row & (Cfg<D>::kChunks - 1); }

// Issue the direct global->LDS loads of one K or V tile.  Every wave moves
// kLoads contiguous 1 KB pieces of the tile; lane l of a piece fills LDS
// chunk p = piece*64 + l, i.e. row p / C, physical chunk p % C, which holds
// logical chunk (p % C) ^ swz(row).  Rows past the sequence end re-read the
// last valid row (finite data; those keys are masked).
template <int D, bool IS_K>
__device__ __forceinline__ void issue_tile(unsigned char *lds_tile, const uint16_t *src, int k0,
                                           int N, int wave, int lane)
{
    constexpr int C = Cfg<D>::kChunks;
#pragma unroll
    for (int i = 0; i < Cfg<D>::kLoads; ++i) {
        const int piece = wave * Cfg<D>::kLoads + i;
        const int p = piece * 64 + lane;
        const int row = p / C;
        const int c = (p % C) ^ (IS_K ? swz_k<D>(row) : swz_v<D>(row));
        const int grow = min(k0 + row, N - 1);
        __builtin_amdgcn_global_load_lds(
            (const void *)(src + (size_t)grow * D + c * 8),
            (__attribute__((address_space(3))) void *)(lds_tile + piece * 1024), 16, 0, 0);
    }
}

template <int D, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(kThreads) void prefill_exact_kernel(PrefillArgs a)
{
    __shared__ __attribute__((aligned(1024))) unsigned char smem[Cfg<D>::kSmem];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, n = lane & 31;
    const int N = a.N;
    const int nqt = (N + kBM - 1) / kBM;
    const int BH = a.B * a.H;

    // workgroup -> (head, query tile)
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
    const int q0 = qt * kBM;
    const int kvh = h / (a.H / a.Hkv);
    const uint16_t *qb = (const uint16_t *)a.q + (size_t)bh * N * D;
    const uint16_t *kb = (const uint16_t *)a.k + (size_t)(b * a.Hkv + kvh) * N * D;
    const uint16_t *vb = (const uint16_t *)a.v + (size_t)(b * a.Hkv + kvh) * N * D;
    const int qw0 = q0 + wave * kQW;
    const int my_q = qw0 + n;

    const int kend = CAUSAL ? min(N, q0 + kBM) : N;
    const int ntiles = (kend + kBN - 1) / kBN;

    // first tile in flight while Q is fetched
    issue_tile<D, true>(smem, kb, 0, N, wave, lane);
    issue_tile<D, false>(smem + Cfg<D>::kTileBytes, vb, 0, N, wave, lane);

    // Q^T fragments (B operand): lane holds Q[my_q][16*ks + 8*g .. +7].
    bf16x8 qf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
        qf[ks] = as_bf16x8(my_q < N ? ld16(qb + (size_t)my_q * D + ks * 16 + g * 8)
                                    : u32x4{0, 0, 0, 0});

    // per-lane LDS addressing of the MFMA operands
    const int krow = perm32(n);  // + 32*blk; the swizzle is the same for both blocks
    const int kswz = swz_k<D>(krow);
    const int L = lane & 15, G = lane >> 4;
    const int tr_row = L >> 2;                                   // + key base + 4*t
    const int tr_chunk = 2 * (L & 1) + (G & 1);                  // + 4*c
    const int tr_half = ((L >> 1) & 1) * 8;

    f32x16 o[D / 32];
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
        o[c] = f32x16{};
    float m = -INFINITY;  // reference max of score * scale * log2(e), raised lazily
    float l = 0.f;        // this lane's part of the row sum (its 16 of every 32 keys)
    const float cs = a.scale * kLog2e;

    for (int t = 0; t < ntiles; ++t) {
        const int k0 = t * kBN;
        unsigned char *kbuf = smem + (t & 1) * Cfg<D>::kStage;
        unsigned char *vbuf = kbuf + Cfg<D>::kTileBytes;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (t + 1 < ntiles) {
            unsigned char *nb = smem + ((t + 1) & 1) * Cfg<D>::kStage;
            issue_tile<D, true>(nb, kb, k0 + kBN, N, wave, lane);
            issue_tile<D, false>(nb + Cfg<D>::kTileBytes, vb, k0 + kBN, N, wave, lane);
        }
        if (CAUSAL && k0 > qw0 + kQW - 1)
            continue;  // every key of this tile lies above the diagonal for this wave

        f32x16 s[2];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            s[blk] = f32x16{};
            const unsigned char *rowp = kbuf + (32 * blk + krow) * (D * 2);
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                bf16x8 ka = as_bf16x8(*(const u32x4 *)(rowp + (((2 * ks + g) ^ kswz) << 4)));
                s[blk] = mfma_bf16_32x32x16(ka, qf[ks], s[blk]);
            }
        }
        if ((CAUSAL && k0 + kBN - 1 > qw0) || k0 + kBN > N) {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + 32 * blk + 16 * g + r;
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
        mx = max_xor32(mx) * cs;
        // the first tile always holds key 0, visible to every query, so m is
        // finite from the first tile on
        if (__any(mx > m + kRescaleLog2)) {
            const float m_new = mx > m + kRescaleLog2 ? mx : m;
            const float alpha = fast_exp2(m - m_new);
            l *= alpha;
#pragma unroll
            for (int c = 0; c < D / 32; ++c)
                o[c] *= alpha;
            m = m_new;
        }

        // probabilities, rounded to bf16 for the PV product; the row sum is
        // taken over the unrounded fp32 values (a bf16-rounded sum would carry
        // up to 2^-9 relative error into the LSE of rows with few keys)
        uint32_t pk[2][8];
        float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = fast_exp2(fmaf(s[blk][r], cs, -m));
                const float p1 = fast_exp2(fmaf(s[blk][r + 1], cs, -m));
                rs0 += p0;
                rs1 += p1;
                pk[blk][r >> 1] = pack_bf16x2(p0, p1);
            }
        l += rs0 + rs1;

#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int kbase = 32 * blk + 16 * g + 8 * hh + tr_row;
                    const int chunk = 4 * c + tr_chunk;
                    const int r0 = kbase, r1 = kbase + 4;
                    const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4 *)(vbuf + r0 * (D * 2) + ((chunk ^ swz_v<D>(r0)) << 4) + tr_half));
                    const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4 *)(vbuf + r1 * (D * 2) + ((chunk ^ swz_v<D>(r1)) << 4) + tr_half));
                    const u32x2 w0 = __builtin_bit_cast(u32x2, v0);
                    const u32x2 w1 = __builtin_bit_cast(u32x2, v1);
                    const u32x4 vw = {w0[0], w0[1], w1[0], w1[1]};
                    const u32x4 pw = {pk[blk][4 * hh], pk[blk][4 * hh + 1], pk[blk][4 * hh + 2],
                                      pk[blk][4 * hh + 3]};
                    o[c] = mfma_bf16_32x32x16(as_bf16x8(vw), as_bf16x8(pw), o[c]);
                }
        }
    }

    const float lt = sum_xor32(l);
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
    const int nqt = (a.N + kBM - 1) / kBM;
    dim3 grid(a.B * a.H * nqt);
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
