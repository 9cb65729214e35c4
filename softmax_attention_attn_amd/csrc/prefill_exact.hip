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
//    global_load_lds (no register staging).  K rows are padded by one
//    16-byte chunk (the 16 rows read together fall on 16 distinct bank
//    groups); V rows keep their natural layout with the 64-byte blocks of a
//    row XOR-swizzled by the row index, so the four rows of one transposing
//    read fall on distinct bank blocks.
//  * Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys are
//    rows, queries columns): a lane owns one query column, so row reductions
//    are in-lane plus one permlane32 swap.  Accumulator register r of lane
//    half g holds key 8*(r/4) + 4*g + r%4 of each 32-key block: four
//    consecutive registers are four consecutive keys, so the bf16-rounded
//    probabilities in those registers are directly the B operand of
//    O^T = V^T P^T once the V^T operand is gathered in the same key order.
//  * The V^T operand comes from the row-major V tile through the transposing
//    LDS read ds_read_b64_tr_b16 (within a 16-lane group, output lane i,
//    element j is element i%4 of the 8 bytes addressed by lane 4j + i/4).
//  * Operand reads from LDS are issued a few MFMAs ahead with explicit
//    LDS-counter waits tied to the operand registers.
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

template <int D>
struct Cfg {
    static constexpr int kChunks = D / 8;                  // 16-byte chunks per row
    static constexpr int kKPitch = D * 2 + 16;             // padded K row (bytes)
    static constexpr int kKPieces = kBN * (kChunks + 1) / 64;  // 1 KB direct loads per K tile
    static constexpr int kKBytes = kKPieces * 1024;
    static constexpr int kVPitch = D * 2;
    static constexpr int kVPieces = kBN * kChunks / 64;
    static constexpr int kVBytes = kVPieces * 1024;
    static_assert(kKPieces * 64 == kBN * (kChunks + 1), "K tile split");
    static_assert(kVPieces % kWaves == 0, "V tile split");
};

// V tile: the 64-byte block index of row `row` is XORed with this value.
template <int D>
__device__ __forceinline__ int vswz(int row)
{
    return D >= 128 ? (row & 3) : ((row >> 1) & 1);
}

// Direct global->LDS loads of one K tile (padded rows): LDS slot p of the
// tile (16 bytes) is row p / (C+1), chunk p % (C+1); the pad chunk re-reads
// chunk 0.  Rows past the sequence end re-read the last valid row (finite
// data; those keys are masked).  Waves take the 1 KB pieces round robin.
template <int D>
__device__ __forceinline__ void issue_k(unsigned char *lds_tile, const uint16_t *src, int k0, int N,
                                        int wave, int lane)
{
    constexpr int C = Cfg<D>::kChunks;
    for (int piece = wave; piece < Cfg<D>::kKPieces; piece += kWaves) {
        const int p = piece * 64 + lane;
        const int row = p / (C + 1);
        int c = p % (C + 1);
        c = c == C ? 0 : c;
        const int grow = min(k0 + row, N - 1);
        __builtin_amdgcn_global_load_lds(
            (const void *)(src + (size_t)grow * D + c * 8),
            (__attribute__((address_space(3))) void *)(lds_tile + piece * 1024), 16, 0, 0);
    }
}

// Direct loads of one V tile: LDS slot p is row p / C, physical chunk p % C,
// which holds logical chunk (p % C) ^ (vswz(row) << 2).
template <int D>
__device__ __forceinline__ void issue_v(unsigned char *lds_tile, const uint16_t *src, int k0, int N,
                                        int wave, int lane)
{
    constexpr int C = Cfg<D>::kChunks;
#pragma unroll
    for (int i = 0; i < Cfg<D>::kVPieces / kWaves; ++i) {
        const int piece = wave + i * kWaves;
        const int p = piece * 64 + lane;
        const int row = p / C;
        const int c = (p % C) ^ (vswz<D>(row) << 2);
        const int grow = min(k0 + row, N - 1);
        __builtin_amdgcn_global_load_lds(
            (const void *)(src + (size_t)grow * D + c * 8),
            (__attribute__((address_space(3))) void *)(lds_tile + piece * 1024), 16, 0, 0);
    }
}

// Per-wave running state of the online softmax and the output accumulator.
template <int D>
struct WaveState {
    f32x16 o[D / 32];  // O^T accumulator: register r of lane (n, g) = O[query n][32c + 16g + r]
    float m;           // reference max of score * scale * log2(e), raised lazily
    float l;           // this lane's part of the row sum (its 16 of every 32 keys)
    float lp;          // the same sum over the bf16-rounded P that enters the PV MFMA
};

// Per-lane LDS offsets of the MFMA operand reads (independent of the stage).
template <int D>
struct LaneOffsets {
    uint32_t k;          // K operand: row n, chunk g
    uint32_t v[D / 32];  // V^T operand for feature block c
};

template <int D>
__device__ __forceinline__ LaneOffsets<D> lane_offsets(int lane)
{
    const int g = lane >> 5, n = lane & 31;
    const int G = lane >> 4, L = lane & 15, q = L & 3, j = L >> 2;
    LaneOffsets<D> off;
    off.k = n * Cfg<D>::kKPitch + g * 16;
    // Lane L = 4j + q of 16-lane group G reads key row (base + 4g + j),
    // features 32c + 16(q&1) + 8(G&1) + 4(q>>1) .. +3: output lane i of the
    // group then holds feature 32c + perm(16(G&1) + i) for the 4 keys, with
    // perm(m) = 16((m>>2)&1) + 4(m>>3) + (m&3), which makes the PV output
    // register r of lane half g hold feature 32c + 16g + r.
    const int chunk_lo = 2 * (q & 1) + (G & 1);
    const int xj = vswz<D>(j);  // rows base + 4g + j with base % 8 == 0
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
        off.v[c] = (4 * g + j) * Cfg<D>::kVPitch + ((((c ^ xj) << 2) + chunk_lo) << 4) +
                   (q >> 1) * 8;
    return off;
}

// S^T = K Q^T for one key tile: MFMA i = KS*blk + ks reads K row 32*blk + n,
// chunk 2*ks + g; the reads run four MFMAs ahead.
template <int D>
__device__ __forceinline__ void qk_tile(f32x16 (&s)[2], const bf16x8 (&qf)[D / 16], uint32_t kaddr)
{
    constexpr int KS = D / 16, NK = 2 * KS, KLA = 4;
    u32x4 kv[KLA + 1];
    s[0] = f32x16{};
    s[1] = f32x16{};
    static_for<0, KLA>([&](auto i) {
        constexpr int I = decltype(i)::value;
        kv[I] = lds_read_b128<(I / KS) * 32 * Cfg<D>::kKPitch + (I % KS) * 32>(kaddr);
    });
    static_for<0, NK>([&](auto i) {
        constexpr int I = decltype(i)::value;
        if constexpr (I + KLA < NK) {
            constexpr int J = I + KLA;
            kv[J % (KLA + 1)] =
                lds_read_b128<(J / KS) * 32 * Cfg<D>::kKPitch + (J % KS) * 32>(kaddr);
            lgkm_wait<KLA>(kv[I % (KLA + 1)]);
        } else {
            lgkm_wait<NK - 1 - I>(kv[I % (KLA + 1)]);
        }
        s[I / KS] = mfma_bf16_32x32x16(as_bf16x8(kv[I % (KLA + 1)]), qf[I % KS], s[I / KS]);
    });
}

// O^T += V^T P^T for one key tile: MFMA i = 4c + 2*blk + hh takes as B
// operand registers 8*hh .. 8*hh+7 of s[blk], i.e. keys 32*blk + 16*hh +
// 8*(e/4) + 4*g + e%4 for element e; its V^T operand is two transposing reads
// of key rows 32*blk + 16*hh + 4g + 0..3 and +8..11.  Reads run two MFMAs
// ahead.
template <int D>
__device__ __forceinline__ void pv_tile(f32x16 (&o)[D / 32], const uint32_t (&pk)[2][8],
                                        uint32_t vaddr, const LaneOffsets<D> &off)
{
    constexpr int NV = 4 * (D / 32), VLA = 2;
    u32x4 vw[VLA + 1];
    auto read_v = [&](auto i) -> u32x4 {
        constexpr int I = decltype(i)::value;
        constexpr int c = I >> 2, blk = (I >> 1) & 1, hh = I & 1;
        constexpr int row0 = 32 * blk + 16 * hh;
        const uint32_t a = vaddr + off.v[c];
        const u32x2 w0 = lds_read_tr16_b64<row0 * Cfg<D>::kVPitch>(a);
        const u32x2 w1 = lds_read_tr16_b64<(row0 + 8) * Cfg<D>::kVPitch>(a);
        return u32x4{w0[0], w0[1], w1[0], w1[1]};
    };
    static_for<0, VLA>([&](auto i) { vw[decltype(i)::value] = read_v(i); });
    static_for<0, NV>([&](auto i) {
        constexpr int I = decltype(i)::value;
        if constexpr (I + VLA < NV) {
            vw[(I + VLA) % (VLA + 1)] = read_v(std::integral_constant<int, I + VLA>{});
            lgkm_wait<2 * VLA>(vw[I % (VLA + 1)]);
        } else {
            lgkm_wait<2 * (NV - 1 - I)>(vw[I % (VLA + 1)]);
        }
        constexpr int c = I >> 2, blk = (I >> 1) & 1, hh = I & 1;
        const u32x4 pw = {pk[blk][4 * hh], pk[blk][4 * hh + 1], pk[blk][4 * hh + 2],
                          pk[blk][4 * hh + 3]};
        o[c] = mfma_bf16_32x32x16(as_bf16x8(vw[I % (VLA + 1)]), as_bf16x8(pw), o[c]);
    });
}

__device__ __forceinline__ float tile_max(const f32x16 (&s)[2])
{
    float mx = s[0][0];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            mx = fmaxf(mx, s[blk][r]);
    return mx;
}

template <bool CAUSAL>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[2], int k0, int N, int g, int my_q)
{
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * blk + 8 * (r >> 2) + 4 * g + (r & 3);
            if (key >= N || (CAUSAL && key > my_q))
                s[blk][r] = -INFINITY;
        }
}

// Raise the reference max when the tile max (log2 units) exceeds it by more
// than 2^8 for some lane of the wave, rescaling O and l.  The first tile
// always holds key 0, visible to every query, so m is finite from the first
// tile on.
template <int D>
__device__ __forceinline__ void update_max(WaveState<D> &st, float mx)
{
    if (__any(mx > st.m + kRescaleLog2)) {
        const float m_new = mx > st.m + kRescaleLog2 ? mx : st.m;
        const float alpha = fast_exp2(st.m - m_new);
        st.l *= alpha;
        st.lp *= alpha;
#pragma unroll
        for (int c = 0; c < D / 32; ++c)
            st.o[c] *= alpha;
        st.m = m_new;
    }
}

// Phase A of the software pipeline: the QK MFMAs of the next tile, each
// followed by a slice of the exponentials of the current tile.  The two
// 32-key accumulators alternate so that consecutive MFMAs are independent.
// Each step exponentiates two scores and folds the two of the previous step
// into the row sums and the bf16 P fragment (the exp latency is then covered
// by the MFMA in between).  p = 2^(s*cs - m) is rounded to bf16 for the PV
// product, and two row sums are kept: l over the unrounded values, for the
// LSE (a rounded sum would carry up to 2^-9 relative error into the LSE of
// rows with few keys), and lp over the rounded values, for normalising O (the
// weights applied to V then sum to one, so a row dominated by one key returns
// that key's V row rather than V times the bf16 rounding error of its p).  Steps are fenced with scheduling barriers and
// their results pinned, so the wave issues VALU work between its MFMAs
// instead of in one block.
template <int D>
__device__ __forceinline__ void phase_a(f32x16 (&s_next)[2], const bf16x8 (&qf)[D / 16],
                                        uint32_t kaddr, const f32x16 (&s_cur)[2], float m,
                                        float cs, uint32_t (&pk)[2][8], float &l, float &lp)
{
    constexpr int KS = D / 16, NK = 2 * KS, KLA = 4;
    constexpr int EPS = 32 / NK;  // scores exponentiated per step
    static_assert(EPS == 2 || EPS == 4, "slice size");
    u32x4 kv[KLA + 1];
    s_next[0] = f32x16{};
    s_next[1] = f32x16{};
    float rs0 = 0.f, rs1 = 0.f;
    float pp[2][EPS];  // exponentials of the previous and the current step
    // MFMA i: block i % 2, k-step i / 2
    auto kread = [&](auto i) -> u32x4 {
        constexpr int I = decltype(i)::value;
        return lds_read_b128<(I % 2) * 32 * Cfg<D>::kKPitch + (I / 2) * 32>(kaddr);
    };
    auto fold = [&](auto i) {  // row sum and bf16 packing of step i's slice
        constexpr int I = decltype(i)::value;
        static_for<0, EPS / 2>([&](auto e) {
            constexpr int R = I * EPS + 2 * decltype(e)::value;
            constexpr int blk = R / 16, r = R % 16;
            const float p0 = pp[I % 2][2 * decltype(e)::value];
            const float p1 = pp[I % 2][2 * decltype(e)::value + 1];
            rs0 += p0;
            rs1 += p1;
            pk[blk][r >> 1] = pack_bf16x2(p0, p1);
            lp = add_bf16x2(pk[blk][r >> 1], lp);
            asm volatile("" : "+v"(pk[blk][r >> 1]), "+v"(rs0), "+v"(rs1), "+v"(lp));
        });
    };
    static_for<0, KLA>([&](auto i) { kv[decltype(i)::value] = kread(i); });
    static_for<0, NK>([&](auto i) {
        constexpr int I = decltype(i)::value;
        if constexpr (I + KLA < NK) {
            kv[(I + KLA) % (KLA + 1)] = kread(std::integral_constant<int, I + KLA>{});
            lgkm_wait<KLA>(kv[I % (KLA + 1)]);
        } else {
            lgkm_wait<NK - 1 - I>(kv[I % (KLA + 1)]);
        }
        s_next[I % 2] =
            mfma_bf16_32x32x16(as_bf16x8(kv[I % (KLA + 1)]), qf[I / 2], s_next[I % 2]);
        static_for<0, EPS>([&](auto e) {
            constexpr int R = I * EPS + decltype(e)::value;
            pp[I % 2][decltype(e)::value] = fast_exp2(fmaf(s_cur[R / 16][R % 16], cs, -m));
            asm volatile("" : "+v"(pp[I % 2][decltype(e)::value]));
        });
        if constexpr (I > 0)
            fold(std::integral_constant<int, I - 1>{});
        __builtin_amdgcn_sched_barrier(0);
    });
    fold(std::integral_constant<int, NK - 1>{});
    l += rs0 + rs1;
}

// Phase B: the PV MFMAs of the current tile, each followed by a slice of the
// row max of the next tile; returns that max (this lane's keys only).
// Consecutive MFMAs accumulate into different feature blocks.
template <int D>
__device__ __forceinline__ float phase_b(f32x16 (&o)[D / 32], const uint32_t (&pk)[2][8],
                                         uint32_t vaddr, const LaneOffsets<D> &off,
                                         const f32x16 (&s_next)[2])
{
    constexpr int NC = D / 32, NV = 4 * NC, VLA = 2;
    constexpr int MPS = 32 / NV;  // scores reduced per step
    u32x4 vw[VLA + 1];
    // MFMA i: feature block i % NC, key quarter q = i / NC (blk = q / 2, hh = q % 2)
    auto read_v = [&](auto i) -> u32x4 {
        constexpr int I = decltype(i)::value;
        constexpr int c = I % NC, q = I / NC, blk = q >> 1, hh = q & 1;
        constexpr int row0 = 32 * blk + 16 * hh;
        const uint32_t a = vaddr + off.v[c];
        const u32x2 w0 = lds_read_tr16_b64<row0 * Cfg<D>::kVPitch>(a);
        const u32x2 w1 = lds_read_tr16_b64<(row0 + 8) * Cfg<D>::kVPitch>(a);
        return u32x4{w0[0], w0[1], w1[0], w1[1]};
    };
    float mx0 = -INFINITY, mx1 = -INFINITY;
    static_for<0, VLA>([&](auto i) { vw[decltype(i)::value] = read_v(i); });
    static_for<0, NV>([&](auto i) {
        constexpr int I = decltype(i)::value;
        if constexpr (I + VLA < NV) {
            vw[(I + VLA) % (VLA + 1)] = read_v(std::integral_constant<int, I + VLA>{});
            lgkm_wait<2 * VLA>(vw[I % (VLA + 1)]);
        } else {
            lgkm_wait<2 * (NV - 1 - I)>(vw[I % (VLA + 1)]);
        }
        constexpr int c = I % NC, q = I / NC, blk = q >> 1, hh = q & 1;
        const u32x4 pw = {pk[blk][4 * hh], pk[blk][4 * hh + 1], pk[blk][4 * hh + 2],
                          pk[blk][4 * hh + 3]};
        o[c] = mfma_bf16_32x32x16(as_bf16x8(vw[I % (VLA + 1)]), as_bf16x8(pw), o[c]);
        static_for<0, MPS / 2>([&](auto e) {
            constexpr int R = I * MPS + 2 * decltype(e)::value;
            constexpr int sb = R / 16, r = R % 16;
            if constexpr ((I * (MPS / 2) + decltype(e)::value) % 2 == 0)
                mx0 = vmax3(mx0, s_next[sb][r], s_next[sb][r + 1]);
            else
                mx1 = vmax3(mx1, s_next[sb][r], s_next[sb][r + 1]);
            asm volatile("" : "+v"(mx0), "+v"(mx1));
        });
        __builtin_amdgcn_sched_barrier(0);
    });
    return vmax3(mx0, mx1, mx1);
}

// One query tile of one (batch, head): load its Q fragments, stream every
// visible K/V tile through the LDS stages, write O and the LSE.
template <int D, bool CAUSAL, bool OUT_F32>
__device__ __forceinline__ void attend_qtile(const PrefillArgs &a, unsigned char *smem, int bh,
                                             int qt, int wave, int lane)
{
    constexpr int kStage = Cfg<D>::kKBytes + Cfg<D>::kVBytes;
    const int g = lane >> 5, n = lane & 31;
    const int N = a.N;
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
    // tiles this wave computes (the rest lie above its causal diagonal)
    const int ntw = CAUSAL ? min(ntiles, (qw0 + kQW - 1) / kBN + 1) : ntiles;
    auto kst = [&](int t) { return smem + (t % 3) * kStage; };
    auto vst = [&](int t) { return smem + (t % 3) * kStage + Cfg<D>::kKBytes; };
    auto needs_mask = [&](int t) {
        const int k0 = t * kBN;
        return (CAUSAL && k0 + kBN - 1 > qw0) || k0 + kBN > N;
    };

    issue_k<D>(kst(0), kb, 0, N, wave, lane);
    issue_v<D>(vst(0), vb, 0, N, wave, lane);
    if (ntiles > 1) {
        issue_k<D>(kst(1), kb, kBN, N, wave, lane);
        issue_v<D>(vst(1), vb, kBN, N, wave, lane);
    }

    // Q^T fragments (B operand): lane holds Q[my_q][16*ks + 8*g .. +7].
    bf16x8 qf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
        qf[ks] = as_bf16x8(my_q < N ? ld16(qb + (size_t)my_q * D + ks * 16 + g * 8)
                                    : u32x4{0, 0, 0, 0});

    const LaneOffsets<D> off = lane_offsets<D>(lane);
    WaveState<D> st;
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
        st.o[c] = f32x16{};
    st.m = -INFINITY;
    st.l = 0.f;
    st.lp = 0.f;
    const float cs = a.scale * kLog2e;

    // Software pipeline: iteration t runs the QK MFMAs of tile t+1 next to
    // the exponentials of tile t, then the PV MFMAs of tile t next to the
    // masking and max of tile t+1, so each wave has independent VALU work to
    // issue between its MFMAs.  The loop is unrolled twice so that the two
    // score buffers swap roles without register copies.
    f32x16 sa[2], sb[2];
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    qk_tile<D>(sa, qf, lds_addr(kst(0)) + off.k);
    if (needs_mask(0))
        mask_tile<CAUSAL>(sa, 0, N, g, my_q);
    update_max<D>(st, max_xor32(tile_max(sa)) * cs);

    auto step = [&](int t, f32x16(&s_cur)[2], f32x16(&s_next)[2]) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (t + 2 < ntiles) {
            issue_k<D>(kst(t + 2), kb, (t + 2) * kBN, N, wave, lane);
            issue_v<D>(vst(t + 2), vb, (t + 2) * kBN, N, wave, lane);
        }
        if (t >= ntw)
            return;
        // QK(t+1) also runs when this wave does not need tile t+1 (the result
        // is then dropped) so that phase A has no branch.
        uint32_t pk[2][8];
        phase_a<D>(s_next, qf, lds_addr(kst(t + 1)) + off.k, s_cur, st.m, cs, pk, st.l,
                   st.lp);
        const bool more = t + 1 < ntw;
        if (more && needs_mask(t + 1))
            mask_tile<CAUSAL>(s_next, (t + 1) * kBN, N, g, my_q);
        const float mx = phase_b<D>(st.o, pk, lds_addr(vst(t)), off, s_next);
        if (more)
            update_max<D>(st, max_xor32(mx) * cs);
    };
    for (int t = 0; t < ntiles; t += 2) {
        step(t, sa, sb);
        if (t + 1 < ntiles)
            step(t + 1, sb, sa);
    }

    const float lt = sum_xor32(st.l);
    const float ltp = sum_xor32(st.lp);
    if (my_q < N) {
        const float inv = 1.f / ltp;
        if constexpr (OUT_F32) {
            float *orow = (float *)a.o + ((size_t)bh * N + my_q) * D;
#pragma unroll
            for (int c = 0; c < D / 32; ++c)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    f32x4 w = {st.o[c][4 * j] * inv, st.o[c][4 * j + 1] * inv,
                               st.o[c][4 * j + 2] * inv, st.o[c][4 * j + 3] * inv};
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
                        w[e] = pack_bf16x2(st.o[c][8 * j + 2 * e] * inv,
                                           st.o[c][8 * j + 2 * e + 1] * inv);
                    st16(orow + 32 * c + 16 * g + 8 * j, w);
                }
        }
        if (a.lse && g == 0)
            a.lse[(size_t)bh * N + my_q] = (st.m + log2f(lt)) * kLn2;
    }
}

template <int D, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(kThreads) void prefill_exact_kernel(PrefillArgs a)
{
    // three K/V stages: tile t+2 loads while tile t+1's K and tile t's V are read
    constexpr int kStage = Cfg<D>::kKBytes + Cfg<D>::kVBytes;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[3 * kStage];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nqt = (a.N + kBM - 1) / kBM;
    // Causal: workgroup j of a head takes query tiles nqt-1-j and j, so every
    // workgroup streams the same number of key tiles (no long tail of heavy
    // tiles started last).  Non-causal: one query tile per workgroup.
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
        attend_qtile<D, CAUSAL, OUT_F32>(a, smem, bh, nqt - 1 - j, wave, lane);
        if (j < nqt - 1 - j) {
            __syncthreads();  // every wave is done with the LDS stages
            attend_qtile<D, CAUSAL, OUT_F32>(a, smem, bh, j, wave, lane);
        }
    } else {
        attend_qtile<D, CAUSAL, OUT_F32>(a, smem, bh, j, wave, lane);
    }
}

template <int D, bool CAUSAL, bool OUT_F32>
hipError_t launch_t(const PrefillArgs &a, hipStream_t s)
{
    const int nqt = (a.N + kBM - 1) / kBM;
    dim3 grid(a.B * a.H * (CAUSAL ? (nqt + 1) / 2 : nqt));
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
