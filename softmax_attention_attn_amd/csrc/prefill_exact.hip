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
#include <type_traits>

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

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
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

// LDS byte address of a __shared__ pointer.
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// LDS reads issued as inline asm: the compiler cannot tell them from the
// next stage's in-flight direct loads and would otherwise wait for those.
// Their completion is awaited explicitly with lgkm_wait.
template <int OFF>
__device__ __forceinline__ u32x4 lds_read_b128(uint32_t addr)
{
    u32x4 r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF) : "memory");
    return r;
}
template <int OFF>
__device__ __forceinline__ u32x2 lds_read_tr16_b64(uint32_t addr)
{
    u32x2 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF) : "memory");
    return r;
}

// Wait until at most N LDS operations are outstanding; the operand is tied
// to the wait so that its consumer cannot be scheduled above it.
template <int N>
__device__ __forceinline__ void lgkm_wait(u32x4 &v)
{
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(v) : "n"(N));
}

// Per-wave running state of the online softmax and the output accumulator.
template <int D>
struct WaveState {
    f32x16 o[D / 32];  // O^T accumulator: register r of lane (n, g) = O[query n][32c + 16g + r]
    float m;           // reference max of score * scale * log2(e), raised lazily
    float l;           // this lane's part of the row sum (its 16 of every 32 keys)
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

// Everything one wave does for key tile t: wait for the tile, start the
// next tile's loads into the other stage, S^T = K Q^T, mask, online softmax,
// O^T += V^T P^T.
template <int D, bool CAUSAL>
__device__ __forceinline__ void process_tile(WaveState<D> &st, const bf16x8 (&qf)[D / 16],
                                             const LaneOffsets<D> &off, unsigned char *kbuf,
                                             unsigned char *vbuf, unsigned char *nkbuf,
                                             unsigned char *nvbuf, int t, int ntiles,
                                             const uint16_t *kb, const uint16_t *vb, int N,
                                             int qw0, int my_q, float cs, int wave, int lane)
{
    const int g = lane >> 5;
    const int k0 = t * kBN;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t + 1 < ntiles) {
        issue_k<D>(nkbuf, kb, k0 + kBN, N, wave, lane);
        issue_v<D>(nvbuf, vb, k0 + kBN, N, wave, lane);
    }
    if (CAUSAL && k0 > qw0 + kQW - 1)
        return;  // every key of this tile lies above the diagonal for this wave

    // S^T = K Q^T: MFMA i = KS*blk + ks reads K row 32*blk + n, chunk 2*ks + g;
    // the reads run four MFMAs ahead.
    constexpr int KS = D / 16, NK = 2 * KS, KLA = 4;
    const uint32_t kaddr = lds_addr(kbuf) + off.k;
    u32x4 kv[KLA + 1];
    f32x16 s[2] = {f32x16{}, f32x16{}};
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

    if ((CAUSAL && k0 + kBN - 1 > qw0) || k0 + kBN > N) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = k0 + 32 * blk + 8 * (r >> 2) + 4 * g + (r & 3);
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
    // The first tile always holds key 0, visible to every query, so m is
    // finite from the first tile on.
    if (__any(mx > st.m + kRescaleLog2)) {
        const float m_new = mx > st.m + kRescaleLog2 ? mx : st.m;
        const float alpha = fast_exp2(st.m - m_new);
        st.l *= alpha;
#pragma unroll
        for (int c = 0; c < D / 32; ++c)
            st.o[c] *= alpha;
        st.m = m_new;
    }

    // probabilities, rounded to bf16 for the PV product; the row sum is taken
    // over the unrounded fp32 values (a bf16-rounded sum would carry up to
    // 2^-9 relative error into the LSE of rows with few keys)
    uint32_t pk[2][8];
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const float p0 = fast_exp2(fmaf(s[blk][r], cs, -st.m));
            const float p1 = fast_exp2(fmaf(s[blk][r + 1], cs, -st.m));
            rs0 += p0;
            rs1 += p1;
            pk[blk][r >> 1] = pack_bf16x2(p0, p1);
        }
    st.l += rs0 + rs1;

    // O^T += V^T P^T: MFMA i = 4c + 2*blk + hh takes as B operand registers
    // 8*hh .. 8*hh+7 of s[blk], i.e. keys 32*blk + 16*hh + 8*(e/4) + 4*g + e%4
    // for element e; its V^T operand is two transposing reads of key rows
    // 32*blk + 16*hh + 4g + 0..3 and +8..11.  Reads run two MFMAs ahead.
    constexpr int NV = 4 * (D / 32), VLA = 2;
    const uint32_t vaddr = lds_addr(vbuf);
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
        st.o[c] = mfma_bf16_32x32x16(as_bf16x8(vw[I % (VLA + 1)]), as_bf16x8(pw), st.o[c]);
    });
}

template <int D, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(kThreads) void prefill_exact_kernel(PrefillArgs a)
{
    __shared__ __attribute__((aligned(1024))) unsigned char k_st0[Cfg<D>::kKBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char v_st0[Cfg<D>::kVBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char k_st1[Cfg<D>::kKBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char v_st1[Cfg<D>::kVBytes];
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
    issue_k<D>(k_st0, kb, 0, N, wave, lane);
    issue_v<D>(v_st0, vb, 0, N, wave, lane);

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
    const float cs = a.scale * kLog2e;

    for (int t = 0; t < ntiles; t += 2) {
        process_tile<D, CAUSAL>(st, qf, off, k_st0, v_st0, k_st1, v_st1, t, ntiles, kb, vb, N,
                                qw0, my_q, cs, wave, lane);
        if (t + 1 < ntiles)
            process_tile<D, CAUSAL>(st, qf, off, k_st1, v_st1, k_st0, v_st0, t + 1, ntiles, kb,
                                    vb, N, qw0, my_q, cs, wave, lane);
    }

    const float lt = sum_xor32(st.l);
    if (my_q < N) {
        const float inv = 1.f / lt;
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
