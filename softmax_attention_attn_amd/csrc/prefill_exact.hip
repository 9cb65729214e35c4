// Exact bf16 fused attention forward for gfx950.
//
// Dataflow ("flashattention-kernels" page, §0/§1; "cuda-kernel-pretrain"
// page, §2): one workgroup owns a tile of kBM = 256 queries of one
// (batch, head); each of its 8 waves keeps the Q fragments of its 32 queries
// in registers for the whole pass; K and V tiles of kBN = 64 keys stream
// through 4-stage LDS rings; an online softmax (running row max m
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

// Direct global->LDS loads.  Each tile is split into 1 KB pieces that the
// waves take round robin (piece p = wave + kWaves * i); lane l of piece p
// fills LDS slot 64p + l (16 bytes).
//  * K tile, padded rows: slot q is row q / (C+1), chunk q % (C+1); the pad
//    chunk re-reads chunk 0.
//  * V tile: slot q is row q / C, physical chunk q % C, which holds logical
//    chunk (q % C) ^ (vswz(row) << 2).
// A lane's source offset within the tile is the same for every tile, so it is
// computed once (DmaLanes); a tile's loads go through a buffer resource whose
// base is the tile and whose size stops at the sequence end, so on a ragged
// last tile the rows past the end read as zero (those keys are masked).
template <int D>
struct DmaLanes {
    static constexpr int kKMax = (Cfg<D>::kKPieces + kWaves - 1) / kWaves;
    uint32_t k[kKMax];  // byte offset of the lane's 16 bytes within the K tile
    uint32_t v;         // the same for V piece `wave`
    uint32_t v_step;    // piece wave + kWaves*i is i * v_step bytes further on
};

// row_bytes: distance between consecutive key rows in memory (2d for the
// [B, H, N, d] layout, 2*Hkv*d for packed tokens)
template <int D>
__device__ __forceinline__ DmaLanes<D> dma_lanes(int wave, int lane, uint32_t row_bytes)
{
    constexpr int C = Cfg<D>::kChunks;
    DmaLanes<D> dl;
#pragma unroll
    for (int i = 0; i < DmaLanes<D>::kKMax; ++i) {
        const int q = (wave + kWaves * i) * 64 + lane;
        const int row = q / (C + 1), c = q % (C + 1);
        dl.k[i] = row * row_bytes + (c == C ? 0 : c) * 16;
    }
    // a V piece is 64/C whole rows, and vswz depends only on the row modulo
    // 4 (a divisor of a piece's row count), so pieces differ by whole rows
    static_assert(64 % Cfg<D>::kChunks == 0 && (64 / Cfg<D>::kChunks) % 4 == 0, "V piece rows");
    {
        const int q = wave * 64 + lane;
        const int row = q / C;
        dl.v = row * row_bytes + ((q % C) ^ (vswz<D>(row) << 2)) * 16;
        dl.v_step = kWaves * (64 / C) * row_bytes;
    }
    return dl;
}

// the tile of kBN rows at key k0 (k0 < N), cut at the sequence end; rows are
// `stride` elements apart
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t *src, int k0, int N,
                                                            int stride)
{
    const uint32_t rows = (uint32_t)min(kBN, N - k0);
    return raw_rsrc(src + (size_t)k0 * stride, ((rows - 1) * (uint32_t)stride + D) * 2);
}

// this wave's pieces of the K tile at key k0 (wave is wave-uniform)
template <int D>
__device__ __forceinline__ void issue_k(unsigned char *lds_tile, const uint16_t *src, int k0, int N,
                                        int stride, int wave, const DmaLanes<D> &dl)
{
    const __amdgpu_buffer_rsrc_t r = tile_rsrc<D>(src, k0, N, stride);
#pragma unroll
    for (int i = 0; i < DmaLanes<D>::kKMax; ++i) {
        const int piece = wave + kWaves * i;
        if (piece < Cfg<D>::kKPieces)
            dma16_rsrc(r, dl.k[i], lds_tile + piece * 1024);
    }
}

template <int D>
__device__ __forceinline__ void issue_v(unsigned char *lds_tile, const uint16_t *src, int k0, int N,
                                        int stride, int wave, const DmaLanes<D> &dl)
{
    const __amdgpu_buffer_rsrc_t r = tile_rsrc<D>(src, k0, N, stride);
#pragma unroll
    for (int i = 0; i < Cfg<D>::kVPieces / kWaves; ++i)
        dma16_rsrc(r, dl.v + i * dl.v_step, lds_tile + (wave + kWaves * i) * 1024);
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

// p = 2^(s*cs - m) for one tile, rounded to bf16 for the PV product.  Two
// row sums are kept: l over the unrounded values, for the LSE (a rounded sum
// would carry up to 2^-9 relative error into the LSE of rows with few keys),
// and lp over the rounded values, for normalising O (the weights applied to V
// then sum to one, so a row dominated by one key returns that key's V row
// rather than V times the bf16 rounding error of its p).
__device__ __forceinline__ void softmax_tile(const f32x16 (&s)[2], float m, float cs,
                                             uint32_t (&pk)[2][8], float &l, float &lp)
{
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
            lp = add_bf16x2(pk[blk][r >> 1], lp);
        }
    l += rs0 + rs1;
}

// The exponentials of a tile are taken against the current reference max m
// of each row, without first reducing the tile's own max.  They are kept
// only if every lane's share of the tile's row sum stays <= 2^8 (so every p
// is <= 2^8 and finite); otherwise -- rarely, when a row's scores climb well
// above its reference -- the tile is redone: m is raised to the exact running
// max, the sums and O are rescaled, and the tile is exponentiated again.
constexpr float kPSumMax = 256.f;

template <int D>
__device__ __forceinline__ void redo_tile(WaveState<D> &st, const f32x16 (&s)[2], float cs,
                                          uint32_t (&pk)[2][8], float &rs, float &lp_tile)
{
    const float mx = max_xor32(tile_max(s)) * cs;
    const float m_new = mx > st.m ? mx : st.m;
    const float alpha = fast_exp2(st.m - m_new);
    st.l *= alpha;
    st.lp *= alpha;
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
        st.o[c] *= alpha;
    st.m = m_new;
    rs = 0.f;
    lp_tile = 0.f;
    softmax_tile(s, st.m, cs, pk, rs, lp_tile);
}

// Slot schedule of one pipeline step.  Step t issues NS MFMAs, one per slot:
// slots 0 .. NQK-1 are the QK MFMAs of tile t+2 (slot i: key block i % 2,
// k-step i / 2, so consecutive MFMAs accumulate into different blocks), the
// remaining slots the PV MFMAs of tile t (slot NQK + j: feature block j % NC,
// key quarter j / NC).  The VALU work of the step -- the exponentials, row
// sums and bf16 packing of tile t+1 and the masking and max of tile t+2 --
// is spread over the slots so that every MFMA has about the same amount of
// independent VALU work issued behind it, and the operand reads from LDS run
// RA slots ahead.
template <int D>
struct Sched {
    static constexpr int NC = D / 32;
    static constexpr int NQK = 2 * (D / 16);
    static constexpr int NPV = 4 * NC;
    static constexpr int NS = NQK + NPV;
    static constexpr int RA = 3;
    static constexpr int nops(int s) { return s < NQK ? 1 : 2; }  // LDS reads of slot s
    // LDS reads issued after those of slot s by the time slot s's MFMA issues
    static constexpr int after(int s)
    {
        int n = 0;
        for (int j = s + 1; j <= s + RA && j < NS; ++j)
            n += nops(j);
        return n;
    }
    // scores first_score(s) .. first_score(s+1)-1 are exponentiated in slot s
    static constexpr int first_score(int s) { return s >= NS ? 32 : (s * 32) / NS; }
    // direct-load instruction d of nd is issued in slot dma_slot(d, nd)
    static constexpr int dma_slot(int d, int nd) { return 1 + (d * (NS - 2)) / nd; }
};

// One pipeline step t: PV(t) with P(t), QK(t+2) into s_qk (masked), and the
// exponentials of tile t+1 (s_exp, against the current reference max) into
// p_next.  Returns this lane's share of tile t+1's row sum and (in lp_tile)
// the same over the bf16-rounded values; the caller checks and commits them.
// Every step runs the same code so that the score and P buffers keep their
// registers from step to step: on the last two steps of a wave the QK
// product and the exponentials run on whatever the stages hold and their
// results are dropped.
template <int D, bool CAUSAL, class Dma>
__device__ __forceinline__ float pipe_step(WaveState<D> &st, const bf16x8 (&qf)[D / 16],
                                           uint32_t kaddr, uint32_t vaddr,
                                           const LaneOffsets<D> &off, const f32x16 (&s_exp)[2],
                                           f32x16 (&s_qk)[2], const uint32_t (&p_cur)[2][8],
                                           uint32_t (&p_next)[2][8], float cs, bool mask_qk,
                                           int k0_qk, int N, int g, int my_q, float &lp_tile,
                                           const Dma &dma)
{
    using SC = Sched<D>;
    constexpr int NS = SC::NS, NQK = SC::NQK, NC = SC::NC, RA = SC::RA;
    constexpr int S0 = 0;
    constexpr bool DO_EXP = true, DO_QK = true;
    u32x4 opb[RA + 1];
    auto read_op = [&](auto sc) -> u32x4 {
        constexpr int S = decltype(sc)::value;
        if constexpr (S < NQK) {
            return lds_read_b128<(S % 2) * 32 * Cfg<D>::kKPitch + (S / 2) * 32>(kaddr);
        } else {
            constexpr int j = S - NQK, c = j % NC, q = j / NC;
            constexpr int row0 = 32 * (q >> 1) + 16 * (q & 1);
            const uint32_t a = vaddr + off.v[c];
            const u32x2 w0 = lds_read_tr16_b64<row0 * Cfg<D>::kVPitch>(a);
            const u32x2 w1 = lds_read_tr16_b64<(row0 + 8) * Cfg<D>::kVPitch>(a);
            return u32x4{w0[0], w0[1], w1[0], w1[1]};
        }
    };
    const float m = st.m;
    float pv[32];
    float rs0 = 0.f, rs1 = 0.f, lp = 0.f;
    if constexpr (DO_QK) {
        s_qk[0] = f32x16{};
        s_qk[1] = f32x16{};
    }
    // fold score r (exponentiated in an earlier slot) into the sums and P
    auto fold = [&](auto rc) {
        constexpr int R = decltype(rc)::value;
        if constexpr (R % 2 == 0) {
            rs0 += pv[R];
        } else {
            rs1 += pv[R];
            constexpr int blk = R / 16, r = R % 16;
            p_next[blk][r >> 1] = pack_bf16x2(pv[R - 1], pv[R]);
            lp = add_bf16x2(p_next[blk][r >> 1], lp);
            asm volatile("" : "+v"(p_next[blk][r >> 1]), "+v"(lp));
        }
        asm volatile("" : "+v"(rs0), "+v"(rs1));
    };
    static_for<S0, (S0 + RA < NS ? S0 + RA : NS)>(
        [&](auto i) { opb[decltype(i)::value % (RA + 1)] = read_op(i); });
    static_for<S0, NS>([&](auto sc) {
        constexpr int S = decltype(sc)::value;
        if constexpr (S + RA < NS)
            opb[(S + RA) % (RA + 1)] = read_op(std::integral_constant<int, S + RA>{});
        lgkm_wait<SC::after(S)>(opb[S % (RA + 1)]);
        if constexpr (S < NQK) {
            s_qk[S % 2] = mfma_bf16_32x32x16(as_bf16x8(opb[S % (RA + 1)]), qf[S / 2], s_qk[S % 2]);
        } else {
            constexpr int j = S - NQK, c = j % NC, q = j / NC, blk = q >> 1, hh = q & 1;
            const u32x4 pw = {p_cur[blk][4 * hh], p_cur[blk][4 * hh + 1], p_cur[blk][4 * hh + 2],
                              p_cur[blk][4 * hh + 3]};
            st.o[c] = mfma_bf16_32x32x16(as_bf16x8(opb[S % (RA + 1)]), as_bf16x8(pw), st.o[c]);
        }
        dma(sc);
        if constexpr (DO_EXP) {
            static_for<SC::first_score(S), SC::first_score(S + 1)>([&](auto rc) {
                constexpr int R = decltype(rc)::value;
                pv[R] = fast_exp2(fmaf(s_exp[R / 16][R % 16], cs, -m));
                asm volatile("" : "+v"(pv[R]));
            });
            // fold the scores exponentiated two slots ago (covers the exp latency)
            if constexpr (S > S0 + 1)
                static_for<SC::first_score(S - 2), SC::first_score(S - 1)>(fold);
        }
        if constexpr (DO_QK) {
            if constexpr (S == NQK + 1) {
                if (mask_qk)
                    mask_tile<CAUSAL>(s_qk, k0_qk, N, g, my_q);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    });
    static_for<SC::first_score(NS - 2), 32>(fold);
    lp_tile = lp;
    return rs0 + rs1;
}

// One (batch, head) as the kernel sees it: row 0 of its Q, K, V, O and LSE,
// its length, and the distance between consecutive rows (in elements) of
// Q/O and of K/V.
struct SeqView {
    const uint16_t *q, *k, *v;
    void *o;
    float *lse;  // may be null
    int N;
    int q_stride, kv_stride;
};

// One query tile of one (batch, head): load its Q fragments, stream every
// visible K/V tile through the LDS rings, write O and the LSE.
//
// LDS: 4-stage K and V rings (tile t in stage t % 4).  Step t reads K(t+2)
// and V(t) and issues the loads of K(t+4) and V(t+2).  The workgroup
// synchronises before every even step t: all loads issued by then (those of
// the two previous steps, K(t+2), K(t+3), V(t), V(t+1)) are what steps t and
// t+1 read, and the stages the two steps load into were last read before the
// previous synchronisation.  The prologue loads K0..K3, V0 and V1.
template <int D, bool CAUSAL, bool OUT_F32>
__device__ __forceinline__ void attend_qtile(const PrefillArgs &a, unsigned char *smem,
                                             const SeqView &sv, int qt, int wave, int lane)
{
    constexpr int kK = Cfg<D>::kKBytes, kV = Cfg<D>::kVBytes;
    const int g = lane >> 5, n = lane & 31;
    const int N = sv.N;
    const int q0 = qt * kBM;
    const uint16_t *qb = sv.q, *kb = sv.k, *vb = sv.v;
    const int kvs = sv.kv_stride;
    const int qw0 = q0 + wave * kQW;
    const int my_q = qw0 + n;

    const int kend = CAUSAL ? min(N, q0 + kBM) : N;
    const int ntiles = (kend + kBN - 1) / kBN;
    // tiles this wave computes (the rest lie above its causal diagonal)
    const int ntw = CAUSAL ? min(ntiles, (qw0 + kQW - 1) / kBN + 1) : ntiles;
    auto kst = [&](int t) { return smem + (t & 3) * kK; };
    auto vst = [&](int t) { return smem + 4 * kK + (t & 3) * kV; };
    auto needs_mask = [&](int t) {
        const int k0 = t * kBN;
        return (CAUSAL && k0 + kBN - 1 > qw0) || k0 + kBN > N;
    };
    // direct loads per wave for one K / V tile
    const DmaLanes<D> dl = dma_lanes<D>(wave, lane, (uint32_t)kvs * 2);
    auto load_k = [&](int t) {
        if (t < ntiles)
            issue_k<D>(kst(t), kb, t * kBN, N, kvs, wave, dl);
    };
    auto load_v = [&](int t) {
        if (t < ntiles)
            issue_v<D>(vst(t), vb, t * kBN, N, kvs, wave, dl);
    };

    load_k(0);
    load_k(1);
    load_k(2);
    load_v(0);
    load_k(3);
    load_v(1);

    // Q^T fragments (B operand): lane holds Q[my_q][16*ks + 8*g .. +7].
    bf16x8 qf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
        qf[ks] = as_bf16x8(my_q < N ? ld16(qb + (size_t)my_q * sv.q_stride + ks * 16 + g * 8)
                                    : u32x4{0, 0, 0, 0});

    const LaneOffsets<D> off = lane_offsets<D>(lane);
    WaveState<D> st;
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
        st.o[c] = f32x16{};
    st.l = 0.f;
    st.lp = 0.f;
    const float cs = a.scale * kLog2e;

    // S(j) lives in sA for even j, sB for odd j; P(j) likewise in pA / pB.
    f32x16 sA[2], sB[2];
    uint32_t pA[2][8], pB[2][8];

    // pre-step: S(0) and S(1); the reference max from S(0), and P(0)
    vm_wait_n<0>();  // K0 K1 (the first loads take their full latency anyway)
    __syncthreads();
    if (0 < ntw) {
        qk_tile<D>(sA, qf, lds_addr(kst(0)) + off.k);
        if (ntw > 1)
            qk_tile<D>(sB, qf, lds_addr(kst(1)) + off.k);
        if (needs_mask(0))
            mask_tile<CAUSAL>(sA, 0, N, g, my_q);
        st.m = max_xor32(tile_max(sA)) * cs;
        softmax_tile(sA, st.m, cs, pA, st.l, st.lp);
        if (ntw > 1 && needs_mask(1))
            mask_tile<CAUSAL>(sB, kBN, N, g, my_q);
    }

    // Computed steps (t < ntw) first, then the steps of tiles above this
    // wave's causal diagonal, in which it only keeps the workgroup's
    // synchronisation and load cadence.  The workgroup synchronises before
    // every even step (see above).
    auto sync = [&](int t) {
        if ((t & 1) == 0) {
            vm_wait_n<0>();
            __syncthreads();
        }
    };
    auto step = [&](int t, auto par) {
        constexpr int E = decltype(par)::value;  // t % 2
        if constexpr (E == 0) {
            vm_wait_n<0>();
            __syncthreads();
        }
        // the loads of K(t+4) and V(t+2) go to stages no wave reads in this
        // step; they are spread over the MFMA slots
        const bool lk = t + 4 < ntiles, lv = t + 2 < ntiles;
        const __amdgpu_buffer_rsrc_t rk = tile_rsrc<D>(kb, lk ? (t + 4) * kBN : 0, N, kvs);
        const __amdgpu_buffer_rsrc_t rv = tile_rsrc<D>(vb, lv ? (t + 2) * kBN : 0, N, kvs);
        unsigned char *const lk_st = kst(t + 4), *const lv_st = vst(t + 2);
        auto dma = [&](auto sc) {
            constexpr int S = decltype(sc)::value;
            constexpr int NK = DmaLanes<D>::kKMax, NV = Cfg<D>::kVPieces / kWaves;
            static_for<0, NK + NV>([&](auto dc) {
                constexpr int d = decltype(dc)::value;
                if constexpr (Sched<D>::dma_slot(d, NK + NV) == S) {
                    if constexpr (d < NK) {
                        const int piece = wave + kWaves * d;
                        if (lk && piece < Cfg<D>::kKPieces)
                            dma16_rsrc(rk, dl.k[d], lk_st + piece * 1024);
                    } else {
                        constexpr int i = d - NK;
                        if (lv)
                            dma16_rsrc(rv, dl.v + i * dl.v_step,
                                       lv_st + (wave + kWaves * i) * 1024);
                    }
                }
            });
        };
        const uint32_t kaddr = lds_addr(kst(t + 2)) + off.k;
        const uint32_t vaddr = lds_addr(vst(t));
        f32x16(&s_exp)[2] = E ? sA : sB;  // S(t+1)
        f32x16(&s_qk)[2] = E ? sB : sA;   // S(t+2)
        uint32_t(&pc)[2][8] = E ? pB : pA;  // P(t)
        uint32_t(&pn)[2][8] = E ? pA : pB;  // P(t+1)
        float lp_tile;
        float rs = pipe_step<D, CAUSAL>(st, qf, kaddr, vaddr, off, s_exp, s_qk, pc, pn, cs,
                                        needs_mask(t + 2), (t + 2) * kBN, N, g, my_q, lp_tile,
                                        dma);
        if (t + 1 < ntw) {
            // !(rs <= max) also catches an overflow to inf or NaN
            if (__any(!(rs <= kPSumMax)))
                redo_tile<D>(st, s_exp, cs, pn, rs, lp_tile);
            st.l += rs;
            st.lp += lp_tile;
        }
    };
    int t = 0;
    for (; t + 1 < ntw; t += 2) {
        step(t, std::integral_constant<int, 0>{});
        step(t + 1, std::integral_constant<int, 1>{});
    }
    if (t < ntw) {
        step(t, std::integral_constant<int, 0>{});
        ++t;
    }
    for (; t < ntiles; ++t) {
        sync(t);
        load_k(t + 4);
        load_v(t + 2);
    }
    const float lt = sum_xor32(st.l);
    const float ltp = sum_xor32(st.lp);
    if (my_q < N) {
        const float inv = 1.f / ltp;
        if constexpr (OUT_F32) {
            float *orow = (float *)sv.o + (size_t)my_q * sv.q_stride;
#pragma unroll
            for (int c = 0; c < D / 32; ++c)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    f32x4 w = {st.o[c][4 * j] * inv, st.o[c][4 * j + 1] * inv,
                               st.o[c][4 * j + 2] * inv, st.o[c][4 * j + 3] * inv};
                    *(f32x4 *)(orow + 32 * c + 16 * g + 4 * j) = w;
                }
        } else {
            uint16_t *orow = (uint16_t *)sv.o + (size_t)my_q * sv.q_stride;
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
        if (sv.lse && g == 0)
            sv.lse[my_q] = (st.m + log2f(lt)) * kLn2;
    }
}

// Packed batch: the sequence of rank r when the sequences are ordered by
// length, longest first (ties by index), for B <= 64 (lane x holds sequence
// x's clamped length); larger batches keep their own order.  Dispatching the
// longest sequences first leaves the short ones to fill the end of the grid.
__device__ __forceinline__ int seq_of_rank(const PrefillArgs &a, int r)
{
    if (a.B > 64)
        return r;
    const int x = (int)(threadIdx.x & 63);
    int len = -1;
    if (x < a.B) {
        const int t0 = min(max(a.cu_seqlens[x], 0), a.total);
        const int t1 = min(max(a.cu_seqlens[x + 1], t0), a.total);
        len = min(t1 - t0, a.N);
    }
    int rank = 0;
    for (int y = 0; y < a.B; ++y) {
        const int ly = __shfl(len, y, 64);
        rank += (ly > len || (ly == len && y < x)) ? 1 : 0;
    }
    const unsigned long long hit = __ballot(x < a.B && rank == r);
    return hit ? __ffsll((long long)hit) - 1 : r;
}

template <int D, bool CAUSAL, bool OUT_F32, bool VARLEN>
__global__ __launch_bounds__(kThreads) void prefill_exact_kernel(PrefillArgs a)
{
    // four K stages and four V stages (see attend_qtile)
    __shared__ __attribute__((aligned(1024)))
    unsigned char smem[4 * Cfg<D>::kKBytes + 4 * Cfg<D>::kVBytes];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    // Causal: workgroup j of a head takes query tiles nqt-1-j and j, so every
    // workgroup streams the same number of key tiles (no long tail of heavy
    // tiles started last).  Non-causal: one query tile per workgroup.  In a
    // packed batch the grid is sized for the longest sequence (N) and the
    // workgroups past a shorter sequence's tiles return at once.
    const int nqt_grid = (a.N + kBM - 1) / kBM;
    const int nw = CAUSAL ? (nqt_grid + 1) / 2 : nqt_grid;
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
    const int h = bh % a.H;
    const int b = VARLEN ? seq_of_rank(a, bh / a.H) : bh / a.H;
    const int kvh = h / (a.H / a.Hkv);
    SeqView sv;
    if constexpr (VARLEN) {
        // offsets are clamped into [0, total], so malformed offsets cannot
        // move an access out of the tensors
        const int t0 = min(max(a.cu_seqlens[b], 0), a.total);
        const int t1 = min(max(a.cu_seqlens[b + 1], t0), a.total);
        sv.N = min(t1 - t0, a.N);
        sv.q = (const uint16_t *)a.q + ((size_t)t0 * a.H + h) * D;
        sv.k = (const uint16_t *)a.k + ((size_t)t0 * a.Hkv + kvh) * D;
        sv.v = (const uint16_t *)a.v + ((size_t)t0 * a.Hkv + kvh) * D;
        sv.o = (char *)a.o + ((size_t)t0 * a.H + h) * D * (OUT_F32 ? 4 : 2);
        sv.lse = a.lse ? a.lse + (size_t)h * a.total + t0 : nullptr;
        sv.q_stride = a.H * D;
        sv.kv_stride = a.Hkv * D;
    } else {
        const size_t N = a.N;
        sv.N = a.N;
        sv.q = (const uint16_t *)a.q + (size_t)bh * N * D;
        sv.k = (const uint16_t *)a.k + (size_t)(b * a.Hkv + kvh) * N * D;
        sv.v = (const uint16_t *)a.v + (size_t)(b * a.Hkv + kvh) * N * D;
        sv.o = (char *)a.o + (size_t)bh * N * D * (OUT_F32 ? 4 : 2);
        sv.lse = a.lse ? a.lse + (size_t)bh * N : nullptr;
        sv.q_stride = D;
        sv.kv_stride = D;
    }
    const int nqt = (sv.N + kBM - 1) / kBM;
    if (j >= (CAUSAL ? (nqt + 1) / 2 : nqt))
        return;  // past this sequence's tiles (no barrier has been reached)
    if (CAUSAL) {
        attend_qtile<D, CAUSAL, OUT_F32>(a, smem, sv, nqt - 1 - j, wave, lane);
        if (j < nqt - 1 - j) {
            __syncthreads();  // every wave is done with the LDS stages
            attend_qtile<D, CAUSAL, OUT_F32>(a, smem, sv, j, wave, lane);
        }
    } else {
        attend_qtile<D, CAUSAL, OUT_F32>(a, smem, sv, j, wave, lane);
    }
}

template <int D, bool CAUSAL, bool OUT_F32>
hipError_t launch_t(const PrefillArgs &a, hipStream_t s)
{
    const int nqt = (a.N + kBM - 1) / kBM;
    dim3 grid(a.B * a.H * (CAUSAL ? (nqt + 1) / 2 : nqt));
    ProfScope ps(a.cu_seqlens ? "prefill_exact_varlen" : "prefill_exact", s);
    if (a.cu_seqlens)
        hipLaunchKernelGGL((prefill_exact_kernel<D, CAUSAL, OUT_F32, true>), grid,
                           dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((prefill_exact_kernel<D, CAUSAL, OUT_F32, false>), grid,
                           dim3(kThreads), 0, s, a);
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
