// Split-KV GQA decode for gfx950 (Flash-Decoding, "flashattention-kernels"
// page §3; GQA from the "cuda-kernel-pretrain" page §3).
//
// The valid keys of all (sequence, kv head) segments, taken in (sequence,
// kv head, position) order, form one list of K = Hkv * sum_b L_b keys.  A
// fixed set of resident waves (kDecodeWaves, fewer on small problems) splits
// that list into equal contiguous ranges, so every wave -- and every XCD --
// streams the same number of bytes whatever the length mix, and each wave
// reads long contiguous runs of the caches.
//
// decode_split_kernel: a wave walks its range sub-tile by sub-tile (32
// keys, aligned to multiples of 32 within the sequence).  Within one
// (sequence, kv head) segment the keys form split_tokens-key chunks (chunk c
// is [c * split_tokens, (c + 1) * split_tokens)); the wave computes each
// chunk's partial attention for all G = H/Hkv query heads of the group at
// once (each K/V byte is read once per group, the GQA saving) and folds it
// into its running partial for the segment with log-sum-exp weights.  Where
// its range leaves a segment it writes that partial (O normalised by its own
// row sum, and its log2 LSE) to the slot (segment index + wave index).  A
// chunk cut by a range boundary contributes a partial to each of the two
// waves.
//
// decode_merge_kernel: one wave per (sequence, query head) merges the
// partials of the waves whose ranges met its segment -- consecutive slots --
// with log-sum-exp weights into O and the natural-log LSE.
//
// The caches are either contiguous per sequence ([B, Hkv, N_max, d]) or a
// pool of fixed-size pages named by a per-sequence page table (the paged KV
// layout of serving caches, "flashattention-kernels" page §3).  A paged wave
// reads the page numbers of each sub-tile two load groups ahead of its K/V
// loads (a sub-tile touches at most two pages, as pages hold >= 16 rows) and
// finds each row's page with a lane shuffle; everything else is shared.
//
// The path is HBM bound (a few FLOPs per byte): each wave keeps two sub-tiles
// of K and V in flight (about 32 KB), uses the matrix cores for the small
// products so the VALU stays free, and never waits on other waves.
#include <mutex>

#include "../../include/attn.h"
#include "attn_internal.hpp"
#include "cdna4.hpp"

namespace attn {
namespace {

constexpr int kSub = 32;  // keys per sub-tile
constexpr int kVStages = 3;
constexpr int kWavesPerWG = 4;
constexpr int kMinKeysPerWave = 256;  // a small problem uses fewer waves
static_assert(kDecodeWaves % kWavesPerWG == 0, "whole workgroups");

__device__ __forceinline__ int clamp_len(const int32_t *seqlens, int b, int n_max)
{
    int L = seqlens[b];
    return L < 1 ? 1 : (L > n_max ? n_max : L);
}

// s_waitcnt for the vector-memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt and lgkmcnt left at their maxima), through the
// builtin so that the compiler's own wait insertion sees it
template <int N>
__device__ __forceinline__ void vm_wait()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

template <int D>
struct DCfg {
    static constexpr int kVBytes = kSub * D * 2;  // one V sub-tile
    static constexpr int kChunks = D / 8;         // 16-byte chunks per row
    static constexpr int kVPieces = kVBytes / 1024;
    static constexpr int kQLoads = D / 32;                  // q fragments per lane
    static constexpr int kKVLoads = 2 * (D / 32) + kVPieces;  // K rows + V pieces per lane
};

// V sub-tile: 16-byte chunk c of row r is stored at chunk c ^ (2 * (r & 7))
// (mod the row's chunk count), so the 8 rows x 32 bytes that 32 lanes read
// with one transposing read fall on distinct bank slots.
template <int D>
__device__ __forceinline__ int dvswz(int r)
{
    return (2 * (r & 7)) & (DCfg<D>::kChunks - 1);
}

__device__ __forceinline__ long long uniform64(long long x)
{
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)x);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)((unsigned long long)x >> 32));
    return (long long)(((unsigned long long)hi << 32) | lo);
}

// The key list and its split among the waves.  Every wave of both kernels
// computes the same K and the same number of working waves W.
struct KeySplit {
    long long K;  // total valid keys, Hkv * sum_b L_b
    int W;        // waves with work: min(kDecodeWaves, max(1, K / kMinKeysPerWave))
    __device__ long long start(int w) const { return (long long)w * K / W; }
    // the wave whose range holds global key x: the largest w with start(w) <= x
    __device__ int wave_of(long long x) const
    {
        return (int)(((x + 1) * W - 1) / K);
    }
};

// the split of Hkv * (sum of the clamped lengths) keys
__device__ __forceinline__ KeySplit key_split_of(const DecodeArgs &a, long long len_sum)
{
    KeySplit ks;
    ks.K = uniform64(len_sum * a.Hkv);
    const long long w = ks.K / kMinKeysPerWave;
    ks.W = (int)(w < 1 ? 1 : (w > kDecodeWaves ? kDecodeWaves : w));
    return ks;
}

__device__ __forceinline__ KeySplit key_split(const DecodeArgs &a, int lane)
{
    long long s = 0;
    for (int b0 = 0; b0 < a.B; b0 += 64) {
        const int bb = b0 + lane;
        s += bb < a.B ? clamp_len(a.seqlens, bb, a.N_max) : 0;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        s += __shfl_xor(s, off, 64);
    return key_split_of(a, s);
}

// The segment holding global key x: its sequence b, the global offset of its
// sequence's first key (Hkv * sum_{b' < b} L_b'), and L_b.  A wave-wide
// prefix sum over the sequences, 64 at a time.
__device__ __forceinline__ void locate_key(const DecodeArgs &a, long long x, int lane, int &b,
                                           long long &seq0, int &L)
{
    long long base = 0;
    b = a.B - 1;
    seq0 = 0;
    L = 1;
    for (int b0 = 0; b0 < a.B; b0 += 64) {
        const int bb = b0 + lane;
        const int len = bb < a.B ? clamp_len(a.seqlens, bb, a.N_max) : 0;
        long long inc = (long long)len * a.Hkv;
        const long long cnt = inc;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const long long t = __shfl_up(inc, off, 64);
            if (lane >= off)
                inc += t;
        }
        const long long total = __shfl(inc, 63, 64);
        if (x < base + total) {
            const unsigned long long m = __ballot(base + inc > x);
            const int l = __builtin_ctzll(m);
            b = b0 + l;
            seq0 = base + __shfl(inc - cnt, l, 64);
            L = __shfl(len, l, 64);
            return;
        }
        base += total;
    }
}

// Walks the sub-tiles of a wave's key range in order.  All fields are
// wave-uniform (scalar registers).
struct Cursor {
    int b, kvh, L;
    long long seg0;  // global offset of the current segment's key 0
    int pos;         // first key of the next sub-tile, within the segment
    long long end;   // global end of the wave's range
    bool first;      // the next sub-tile starts a new piece
    bool done;
};

// One sub-tile: keys [lo, hi) of segment (b, kvh), inside the 32-aligned
// block that starts at base.
struct SubTile {
    int b, kvh;
    int base, lo, hi;
    bool valid, first, last, chunk_end;
};

// Running (unnormalised) attention state of one chunk or one piece: the
// reference max m of score * scale * log2(e) (per head column), this lane's
// parts of the row sums over the unrounded p (l, for the LSE) and over the
// bf16-rounded p that enter the PV MFMA (lp, for normalising O), and O^T.
template <int D>
struct State {
    float m, l, lp;
    f32x4 o[D / 16];
    __device__ void reset()
    {
        m = -INFINITY;
        l = lp = 0.f;
#pragma unroll
        for (int c = 0; c < D / 16; ++c)
            o[c] = f32x4{};
    }
};

// acc <- the log-sum-exp merge of acc and part (both relative to their own
// reference max); the empty acc (m = -inf) takes part as it is.
template <int D>
__device__ __forceinline__ void fold(State<D> &acc, const State<D> &part)
{
    const float mn = fmaxf(acc.m, part.m);
    const float a1 = fast_exp2(acc.m - mn), a2 = fast_exp2(part.m - mn);
    acc.l = acc.l * a1 + part.l * a2;
    acc.lp = acc.lp * a1 + part.lp * a2;
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
        acc.o[c] = acc.o[c] * a1 + part.o[c] * a2;
    acc.m = mn;
}

template <int D, int G, bool PAGED>
__global__ __launch_bounds__(64 * kWavesPerWG) void decode_split_kernel(DecodeArgs a)
{
    __shared__ __attribute__((aligned(1024)))
    unsigned char vlds[kWavesPerWG][kVStages][DCfg<D>::kVBytes];
    constexpr int KVL = DCfg<D>::kKVLoads, QL = DCfg<D>::kQLoads;
    constexpr int kGroup = KVL + QL + (PAGED ? 1 : 0);  // loads per group
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const KeySplit ks = key_split(a, lane);
    const int w = (int)blockIdx.x * kWavesPerWG + wave;
    if (w >= ks.W)
        return;  // no barrier follows
    const long long g0 = ks.start(w), g1 = ks.start(w + 1);

    const int col = lane & 15, G4 = lane >> 4;  // MFMA column (head) and lane group
    unsigned char *vst = &vlds[wave][0][0];
    const uint16_t *kcache = (const uint16_t *)a.k, *vcache = (const uint16_t *)a.v;
    const int pmask = (1 << a.page_shift) - 1;
    const float cs = a.scale * kLog2e;
    // per-lane transposing-read offset: lane 4j + q of its 16-lane group
    // reads key row (base + j), features 16c + 4q .. +3
    const int trl = lane & 15, trj = trl >> 2, trq = trl & 3;

    // element offset of key `key` of segment (b, kvh); paged: `tab` holds (in
    // lanes 0 and 1) the pages of the sub-tile's 32-aligned block at `base`
    auto row_off = [&](int b, int kvh, int base, int key, int tab) -> size_t {
        if constexpr (PAGED) {
            const int pg = __shfl(tab, (key >> a.page_shift) - (base >> a.page_shift), 64);
            return ((((size_t)pg * a.Hkv + kvh) << a.page_shift) + (key & pmask)) * D;
        } else {
            return ((size_t)(b * a.Hkv + kvh) * a.N_max + key) * D;
        }
    };
    // page numbers of a sub-tile's block (lanes 0 and 1: its first and second
    // page; a page holds >= 16 rows, so 32 aligned keys touch at most two),
    // clamped into the table row and the pool
    auto load_tab = [&](const SubTile &s) -> int {
        const int pi = min((s.base >> a.page_shift) + (lane & 1), a.max_pages - 1);
        const int pg = a.block_table[(size_t)s.b * a.max_pages + pi];
        return pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);
    };
    // q^T fragments (B operand of QK): lane holds q[head col][32*j + 8*G4 .. +7]
    // (lanes of columns >= G load head 0's row; their q is zeroed when used)
    auto load_q = [&](const SubTile &s, u32x4 (&qd)[D / 32]) {
        const uint16_t *qrow =
            (const uint16_t *)a.q + ((size_t)s.b * a.H + s.kvh * G + (col < G ? col : 0)) * D;
#pragma unroll
        for (int j = 0; j < D / 32; ++j)
            qd[j] = ld16(qrow + 32 * j + 8 * G4);
    };
    // K sub-tile into registers: MFMA (blk, j) A operand = row 16*blk + col,
    // features 32*j + 8*G4 .. +7; V sub-tile into LDS stage `stage` (row-major
    // rows of D bf16, swizzled).  Rows outside [lo, hi) re-read a valid row
    // (their scores are masked).
    auto load_kv = [&](const SubTile &s, int tab, u32x4 (&kr)[2][D / 32], int stage) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const int key = min(max(s.base + 16 * blk + col, s.lo), s.hi - 1);
            const uint16_t *krow = kcache + row_off(s.b, s.kvh, s.base, key, tab);
#pragma unroll
            for (int j = 0; j < D / 32; ++j)
                kr[blk][j] = ld16_nt(krow + 32 * j + 8 * G4);
        }
        unsigned char *dst = vst + stage * DCfg<D>::kVBytes;
        constexpr int C = DCfg<D>::kChunks;
#pragma unroll
        for (int piece = 0; piece < DCfg<D>::kVPieces; ++piece) {
            const int p = piece * 64 + lane;
            const int r = p / C;
            const int c = (p % C) ^ dvswz<D>(r);
            const int key = min(max(s.base + r, s.lo), s.hi - 1);
            dma16_nt(vcache + row_off(s.b, s.kvh, s.base, key, tab) + c * 8, dst + piece * 1024);
        }
    };

    State<D> ch, pc;  // the current chunk's state and the current piece's
    ch.reset();
    pc.reset();
    bf16x8 qf[D / 32];

    // sub-tile i: descriptor s, K in kr, q in qd, V in stage i % 3
    auto compute = [&](const SubTile &s, const u32x4(&kr)[2][D / 32], const u32x4(&qd)[D / 32],
                       int stage) {
        // every group loads q, so its registers are read here on every path
        // (a load whose result is dropped would make the compiler wait for
        // all loads before reusing its registers)
#pragma unroll
        for (int j = 0; j < D / 32; ++j)
            asm volatile("" ::"v"(qd[j]));
        if (s.first) {
            // the piece's query rows (lanes of columns >= G hold zeros)
#pragma unroll
            for (int j = 0; j < D / 32; ++j)
                qf[j] = as_bf16x8(col < G ? qd[j] : u32x4{0, 0, 0, 0});
        }
        // S^T = K q^T: lane holds head col, keys 16*blk + 4*G4 + r of the block
        f32x4 sc[2] = {f32x4{}, f32x4{}};
#pragma unroll
        for (int j = 0; j < D / 32; ++j)
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
                sc[blk] = mfma_bf16_16x16x32(as_bf16x8(kr[blk][j]), qf[j], sc[blk]);
        float mx = -INFINITY;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = s.base + 16 * blk + 4 * G4 + r;
                sc[blk][r] = key >= s.lo && key < s.hi ? sc[blk][r] * cs : -INFINITY;
                mx = fmaxf(mx, sc[blk][r]);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        // lazy rescale (the reference max moves only by more than 2^8); every
        // sub-tile has a visible key, so a chunk's first sub-tile sets m
        if (__any(mx > ch.m + 8.f)) {
            const float m_new = mx > ch.m + 8.f ? mx : ch.m;
            const float alpha = fast_exp2(ch.m - m_new);
            ch.l *= alpha;
            ch.lp *= alpha;
#pragma unroll
            for (int c = 0; c < D / 16; ++c)
                ch.o[c] *= alpha;
            ch.m = m_new;
        }
        // P^T B operand: element e is key 16*(e/4) + 4*G4 + e%4
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            p[e] = fast_exp2(sc[e >> 2][e & 3] - ch.m);
            ch.l += p[e];
        }
        const u32x4 pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                          pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            ch.lp = add_bf16x2(pw[e], ch.lp);
        // O^T += V^T P^T: per 16-feature block c, the A operand is keys
        // 4*G4 + 0..3 and 16 + 4*G4 + 0..3 of features 16c + col, gathered by
        // two transposing reads
        const uint32_t vbase = lds_addr(vst + stage * DCfg<D>::kVBytes);
        auto vaddr = [&](int row, int c) {
            const int chunk = 2 * c + (trq >> 1);
            return vbase + row * (D * 2) + ((chunk ^ dvswz<D>(row)) << 4) + (trq & 1) * 8;
        };
        u32x4 va[2];
        auto read_va = [&](int c) -> u32x4 {
            const u32x2 w0 = lds_read_tr16_b64<0>(vaddr(4 * G4 + trj, c));
            const u32x2 w1 = lds_read_tr16_b64<0>(vaddr(16 + 4 * G4 + trj, c));
            return u32x4{w0[0], w0[1], w1[0], w1[1]};
        };
        va[0] = read_va(0);
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
            if (c + 1 < D / 16) {
                va[(c + 1) & 1] = read_va(c + 1);
                lgkm_wait<2>(va[c & 1]);
            } else {
                lgkm_wait<0>(va[c & 1]);
            }
            ch.o[c] = mfma_bf16_16x16x32(as_bf16x8(va[c & 1]), as_bf16x8(pw), ch.o[c]);
        }
        if (s.chunk_end) {
            fold(pc, ch);
            ch.reset();
        }
        if (s.last) {
            // the piece's partial: O_s = acc / lp, lse_s = m + log2 l (log2
            // units); lane holds head col, features 16c + 4*G4 + r
            float lt = pc.l + __shfl_xor(pc.l, 16, 64);
            lt += __shfl_xor(lt, 32, 64);
            float ltp = pc.lp + __shfl_xor(pc.lp, 16, 64);
            ltp += __shfl_xor(ltp, 32, 64);
            if (col < G) {
                const float inv = 1.f / ltp;
                const size_t slot = (size_t)(s.b * a.Hkv + s.kvh) + w;
                float *po = a.part_o + (slot * G + col) * D;
#pragma unroll
                for (int c = 0; c < D / 16; ++c)
                    *(f32x4 *)(po + 16 * c + 4 * G4) = pc.o[c] * inv;
                if (G4 == 0)
                    a.part_lse[slot * G + col] = pc.m + log2f(lt);
            }
            pc.reset();
        }
    };

    // The wave's range in windows of at most 64 sequences, so that a lane can
    // hold each sequence length of the window and the pipelined loop issues no
    // load but its load groups (a range crosses more than 64 sequences only
    // when they are short).  The pipeline drains between windows.
    int b, L;
    long long seq0;
    locate_key(a, g0, lane, b, seq0, L);
    b = __builtin_amdgcn_readfirstlane(b);
    seq0 = uniform64(seq0);
    long long x = g0;  // first key of the next window's part of the range
    while (x < g1) {
        // window: sequences b .. b+63 (lane i: length of sequence b + i)
        const int wb = b;
        const int len = wb + lane < a.B ? clamp_len(a.seqlens, wb + lane, a.N_max) : 0;
        long long wend = (long long)len * a.Hkv;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
            wend += __shfl_xor(wend, off, 64);
        wend = uniform64(seq0 + wend);  // global end of the window's last sequence
        const long long x1 = wend < g1 ? wend : g1;

        Cursor kc;  // the K/V load cursor
        {
            L = __builtin_amdgcn_readlane(len, b - wb);
            const long long off = x - seq0;
            kc.b = b;
            kc.L = L;
            kc.kvh = (int)(off / L);
            kc.seg0 = seq0 + (long long)kc.kvh * L;
            kc.pos = (int)(x - kc.seg0);
            kc.end = x1;
            kc.first = true;
            kc.done = false;
        }
        Cursor tc = kc;  // the page-table cursor, two sub-tiles ahead of kc
        auto advance = [&](Cursor &c) -> SubTile {
            SubTile st;
            st.valid = !c.done;
            if (c.done) {
                // past the range: a stand-in that names key 0 of segment
                // (0, 0), so that every load group keeps its size (its loads
                // are never used)
                st.b = st.kvh = st.base = st.lo = 0;
                st.hi = 1;
                st.first = st.last = st.chunk_end = false;
                return st;
            }
            const long long rem = c.end - c.seg0;
            const int pend = rem < c.L ? (int)rem : c.L;  // the piece ends here
            st.b = c.b;
            st.kvh = c.kvh;
            st.base = c.pos & ~(kSub - 1);
            st.lo = c.pos;
            st.hi = min(st.base + kSub, pend);
            st.first = c.first;
            st.last = st.hi == pend;
            st.chunk_end = st.last || st.hi % a.split_tokens == 0;
            c.first = false;
            c.pos = st.hi;
            if (st.last) {
                c.seg0 += c.L;
                c.pos = 0;
                c.first = true;
                if (c.seg0 >= c.end) {
                    c.done = true;
                } else if (++c.kvh == a.Hkv) {
                    c.kvh = 0;
                    ++c.b;
                    c.L = __builtin_amdgcn_readlane(len, c.b - wb);
                }
            }
            return st;
        };

        // sub-tile descriptors, their K registers, q fragments and page
        // numbers rotate over three slots (sub-tile i in slot i % 3)
        SubTile st0, st1, st2;
        u32x4 kr0[2][D / 32], kr1[2][D / 32], kr2[2][D / 32];
        u32x4 qb0[D / 32], qb1[D / 32], qb2[D / 32];
        int tb0 = 0, tb1 = 0, tb2 = 0;

        // group of sub-tile j: [the page numbers of sub-tile j + 2], q of j's
        // (sequence, kv head), K and V of j; issued two steps before sub-tile
        // j is computed.  Every group issues the same loads whether or not j
        // exists or starts a piece (stand-ins past the range), so the number
        // of loads in flight is the same on every path and the wait for a
        // group is exact.
        auto issue_group = [&](const SubTile &s, int tab, u32x4(&kr)[2][D / 32],
                               u32x4(&qd)[D / 32], int stage, int &tnext) {
            if constexpr (PAGED)
                tnext = load_tab(advance(tc));
            load_q(s, qd);
            load_kv(s, tab, kr, stage);
        };
        // step i: wait for sub-tile i's group (at most sub-tile i+1's group
        // pending), issue sub-tile i+2's group, compute sub-tile i
        auto step = [&](const SubTile &s, const u32x4(&kr)[2][D / 32],
                        const u32x4(&qd)[D / 32], int stage, SubTile &s2,
                        u32x4(&kr2)[2][D / 32], u32x4(&qd2)[D / 32], int stage2, int tab2,
                        int &tab4) {
            vm_wait<kGroup>();
            s2 = advance(kc);
            issue_group(s2, tab2, kr2, qd2, stage2, tab4);
            compute(s, kr, qd, stage);
        };

        // prologue: sub-tiles 0 and 1 (paged: their page numbers first)
        st0 = advance(kc);
        st1 = advance(kc);
        if constexpr (PAGED) {
            tb0 = load_tab(advance(tc));
            tb1 = load_tab(advance(tc));
            vm_wait<0>();
        }
        issue_group(st0, tb0, kr0, qb0, 0, tb2);  // + sub-tile 2's page numbers
        issue_group(st1, tb1, kr1, qb1, 1, tb0);  // + sub-tile 3's (slot 3 % 3)
        for (;;) {
            if (!st0.valid)
                break;
            step(st0, kr0, qb0, 0, st2, kr2, qb2, 2, tb2, tb1);
            if (!st1.valid)
                break;
            step(st1, kr1, qb1, 1, st0, kr0, qb0, 0, tb0, tb2);
            if (!st2.valid)
                break;
            step(st2, kr2, qb2, 2, st1, kr1, qb1, 1, tb1, tb0);
        }
        vm_wait<0>();  // the stand-ins' loads: nothing stays in flight
        // next window: the sequence after this window's last one
        x = x1;
        b = wb + 64;
        seq0 = wend;
    }
}

// One wave per (sequence, query head): the partials of the waves whose
// ranges met the head's segment sit in consecutive slots; lanes take their
// LSEs 64 at a time for the max and the weight sum, then each lane
// accumulates D/64 features over the partials.
constexpr int kMergeWaves = 4;

template <int D, bool OUT_F32>
__global__ __launch_bounds__(64 * kMergeWaves) void decode_merge_kernel(DecodeArgs a)
{
    constexpr int F = D / 64;  // features per lane
    const int lane = threadIdx.x & 63;
    const int bh = (int)blockIdx.x * kMergeWaves + (int)(threadIdx.x >> 6);
    if (bh >= a.B * a.H)
        return;
    const int G = a.H / a.Hkv;
    const int b = bh / a.H, h = bh % a.H, kvh = h / G, g = h % G;
    // one pass over the lengths gives both the key split (their sum, as
    // key_split computes it) and the global offset of the segment (b, kvh)
    // (the sum over the sequences before b)
    KeySplit ks{};
    long long seq0 = 0;
    {
        long long tot = 0, base = 0;
        for (int b0 = 0; b0 < a.B; b0 += 64) {
            const int bb = b0 + lane;
            const long long len = bb < a.B ? clamp_len(a.seqlens, bb, a.N_max) : 0;
            tot += len;
            base += bb < b ? len : 0;
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            tot += __shfl_xor(tot, off, 64);
            base += __shfl_xor(base, off, 64);
        }
        ks = key_split_of(a, tot);
        seq0 = base * a.Hkv;
    }
    const int L = clamp_len(a.seqlens, b, a.N_max);
    const long long s0 = seq0 + (long long)kvh * L;
    const int seg = b * a.Hkv + kvh;
    const int first = seg + ks.wave_of(s0), last = seg + ks.wave_of(s0 + L - 1);
    const int n = last - first + 1;
    const float *pl = a.part_lse + g;             // slot s: pl[s * G]
    const float *po = a.part_o + (size_t)g * D + F * lane;  // slot s: po[s * G * D]
    // the first 64 partials' LSEs stay in registers for their weights
    const float l0 = lane < n ? pl[(size_t)(first + lane) * G] : -INFINITY;
    float M = l0;
    for (int j = lane + 64; j < n; j += 64)
        M = fmaxf(M, pl[(size_t)(first + j) * G]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        M = fmaxf(M, __shfl_xor(M, off, 64));
    float wsum = 0.f;
    float acc[F] = {};
    for (int j0 = 0; j0 < n; j0 += 64) {
        const float lj = j0 == 0 ? l0 : (j0 + lane < n ? pl[(size_t)(first + j0 + lane) * G] : 0.f);
        const float wj_l = j0 + lane < n ? fast_exp2(lj - M) : 0.f;
        wsum += wj_l;
        const int m = min(64, n - j0);
        for (int j = 0; j < m; ++j) {
            const float wj = __shfl(wj_l, j, 64);
            const float *row = po + (size_t)(first + j0 + j) * G * D;
#pragma unroll
            for (int f = 0; f < F; ++f)
                acc[f] = fmaf(wj, row[f], acc[f]);
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        wsum += __shfl_xor(wsum, off, 64);
    const float inv = 1.f / wsum;
#pragma unroll
    for (int f = 0; f < F; ++f) {
        const float out = acc[f] * inv;
        if constexpr (OUT_F32)
            ((float *)a.o)[(size_t)bh * D + F * lane + f] = out;
        else
            ((__bf16 *)a.o)[(size_t)bh * D + F * lane + f] = (__bf16)out;
    }
    if (a.lse && lane == 0)
        a.lse[bh] = (M + log2f(wsum)) * kLn2;
}

template <int D, int G>
hipError_t launch_split(const DecodeArgs &a, hipStream_t s)
{
    const dim3 grid(kDecodeWaves / kWavesPerWG);
    ProfScope ps(a.block_table ? "decode_split_paged" : "decode_split", s);
    if (a.block_table)
        hipLaunchKernelGGL((decode_split_kernel<D, G, true>), grid, dim3(64 * kWavesPerWG), 0, s,
                           a);
    else
        hipLaunchKernelGGL((decode_split_kernel<D, G, false>), grid, dim3(64 * kWavesPerWG), 0, s,
                           a);
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
    case 8: e = launch_split<D, 8>(a, s); break;
    default: e = launch_split<D, 16>(a, s); break;
    }
    if (e != hipSuccess)
        return e;
    ProfScope ps("decode_merge", s);
    const dim3 grid((unsigned)((a.B * a.H + kMergeWaves - 1) / kMergeWaves));
    if (a.out_fp32)
        hipLaunchKernelGGL((decode_merge_kernel<D, true>), grid, dim3(64 * kMergeWaves), 0, s, a);
    else
        hipLaunchKernelGGL((decode_merge_kernel<D, false>), grid, dim3(64 * kMergeWaves), 0, s, a);
    return hipGetLastError();
}

// The partials of attn_decode_noalloc: a fixed array on every GPU the library
// runs on, held until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device array: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __align__(256) unsigned char scratch[ATTN_DECODE_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

}  // namespace

size_t decode_partial_slots(int B, int Hkv) { return (size_t)B * Hkv + kDecodeWaves; }

hipError_t decode_scratch(void **ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s)
{
    return a.d == 64 ? launch_d<64>(a, s) : launch_d<128>(a, s);
}

}  // namespace attn
