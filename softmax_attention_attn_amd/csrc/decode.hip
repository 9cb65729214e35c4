// Split-KV GQA decode for gfx950 (Flash-Decoding, "flashattention-kernels"
// page §3; GQA from the "cuda-kernel-pretrain" page §3).
//
// decode_split_kernel: each wave owns one chunk of split_tokens keys of one
// (sequence, kv head) and computes the chunk's partial attention for all
// G = H/Hkv query heads of the group at once: each K/V cache byte is read
// once per group, not once per query head (the GQA saving).  It writes the
// partial output O_s (normalised by the chunk's own row sum) and its log2
// LSE.  Chunks starting at or beyond the sequence length do no work.
//
// The caches are either contiguous per sequence ([B, Hkv, N_max, d]) or a
// pool of fixed-size pages named by a per-sequence page table (the paged KV
// layout of serving caches, "flashattention-kernels" page §3).  A paged
// wave reads its chunk's page numbers once, one per lane, and looks up the
// page of each row it loads with a lane shuffle; everything else is shared.
//
// decode_merge_kernel: one wave per (sequence, query head) combines the
// chunk partials with log-sum-exp weights into O and the natural-log LSE.
//
// The path is HBM bound (a few FLOPs per byte): the split kernel keeps two
// sub-tiles of K and V in flight per wave (about 32 KB), uses the matrix
// cores for the small products so the VALU stays free, and never stalls on
// other waves.
#include "attn_internal.hpp"
#include "cdna4.hpp"

namespace attn {
namespace {

__device__ __forceinline__ int clamp_len(const int32_t *seqlens, int b, int n_max)
{
    int L = seqlens[b];
    return L < 1 ? 1 : (L > n_max ? n_max : L);
}

// Work items are the non-empty chunks, ordered by sequence, then kv head,
// then chunk, and item i goes to wave i of the grid.  Consecutive workgroups
// land on consecutive XCDs, so every XCD gets an equal share of the chunks
// whatever the length mix (a grid over (chunk, kv head, sequence) would give
// the XCDs that own high chunk indices nothing to do on short sequences).
// The wave maps its item to (b, kvh, split) with a wave-wide prefix sum of
// the per-sequence item counts, 64 sequences at a time.
__device__ __forceinline__ bool locate_item(const DecodeArgs &a, int item, int lane, int &b,
                                            int &kvh, int &split, int &L)
{
    const int S = a.split_tokens;
    int base = 0;  // items of the sequences before b0
    for (int b0 = 0; b0 < a.B; b0 += 64) {
        const int bb = b0 + lane;
        const int nch = bb < a.B ? (clamp_len(a.seqlens, bb, a.N_max) + S - 1) / S : 0;
        const int cnt = a.Hkv * nch;
        int inc = cnt;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int t = __shfl_up(inc, off, 64);
            if (lane >= off)
                inc += t;
        }
        const int total = __shfl(inc, 63, 64);
        if (item < base + total) {
            const unsigned long long m = __ballot(base + inc > item);
            const int l = __builtin_ctzll(m);  // first sequence whose items reach past item
            const int excl = __shfl(inc - cnt, l, 64);
            const int nch_l = __shfl(nch, l, 64);
            b = b0 + l;
            L = clamp_len(a.seqlens, b, a.N_max);
            const int r = item - base - excl;
            kvh = r / nch_l;
            split = r - kvh * nch_l;
            return true;
        }
        base += total;
    }
    return false;
}

// One 512-token (split_tokens) chunk per wave.  The wave streams its chunk
// in sub-tiles of kSub keys: K straight into the registers of the MFMA A
// operand, V into a 3-stage LDS ring of this wave through direct loads; both
// run two sub-tiles ahead.  S^T = K q^T and O^T += V^T P^T run on
// v_mfma_f32_16x16x32_bf16 with the G query heads of the group as the MFMA
// columns (columns >= G are zero), so the chunk's keys are read once for all
// G heads.  Waves never synchronise with each other.
constexpr int kSub = 32;       // keys per sub-tile
constexpr int kVStages = 3;
constexpr int kWavesPerWG = 4;

template <int D>
struct DCfg {
    static constexpr int kVBytes = kSub * D * 2;   // one V sub-tile
    static constexpr int kChunks = D / 8;          // 16-byte chunks per row
    static constexpr int kVPieces = kVBytes / 1024;
};

// V sub-tile: 16-byte chunk c of row r is stored at chunk c ^ (2 * (r & 7))
// (mod the row's chunk count), so the 8 rows x 32 bytes that 32 lanes read
// with one transposing read fall on distinct bank slots.
template <int D>
__device__ __forceinline__ int dvswz(int r)
{
    return (2 * (r & 7)) & (DCfg<D>::kChunks - 1);
}

template <int D, int G, bool PAGED>
__global__ __launch_bounds__(64 * kWavesPerWG) void decode_split_kernel(DecodeArgs a)
{
    __shared__ __attribute__((aligned(1024)))
    unsigned char vlds[kWavesPerWG][kVStages][DCfg<D>::kVBytes];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int S = a.split_tokens;
    int b, kvh, split, L;
    if (!locate_item(a, (int)blockIdx.x * kWavesPerWG + wave, lane, b, kvh, split, L))
        return;  // past the last chunk (no barrier follows)
    const int c0 = split * S;
    const int n = min(S, L - c0);
    const int nsub = (n + kSub - 1) / kSub;
    const int col = lane & 15, G4 = lane >> 4;  // MFMA column (head) and lane group
    unsigned char *vst = &vlds[wave][0][0];
    // Element offset of key row r (0 <= r < n) of the chunk in the K and V
    // caches.  Paged: lane l holds the page of the chunk's l-th page slot
    // (a chunk spans at most 64 pages; out-of-range page numbers are clamped
    // into the pool), and a row's page is read from its lane.
    size_t cache_off = 0;
    int first_page = 0, my_page = 0;
    if constexpr (PAGED) {
        first_page = c0 >> a.page_shift;
        const int npc = ((c0 + n - 1) >> a.page_shift) - first_page + 1;
        if (lane < npc) {
            const int pg = a.block_table[(size_t)b * a.max_pages + first_page + lane];
            my_page = pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);
        }
    } else {
        cache_off = ((size_t)(b * a.Hkv + kvh) * a.N_max + c0) * D;
    }
    auto row_off = [&](int r) -> size_t {
        if constexpr (PAGED) {
            const int pos = c0 + r;
            const int pg = __shfl(my_page, (pos >> a.page_shift) - first_page, 64);
            const int in_page = pos & ((1 << a.page_shift) - 1);
            return ((((size_t)pg * a.Hkv + kvh) << a.page_shift) + in_page) * D;
        } else {
            return cache_off + (size_t)r * D;
        }
    };
    const uint16_t *kc = (const uint16_t *)a.k, *vc = (const uint16_t *)a.v;

    // q^T fragments (B operand of QK): lane holds q[head col][32*ks + 8*G4 .. +7]
    bf16x8 qf[D / 32];
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
        qf[ks] = as_bf16x8(col < G ? ld16((const uint16_t *)a.q +
                                          ((size_t)b * a.H + kvh * G + col) * D + 32 * ks + 8 * G4)
                                   : u32x4{0, 0, 0, 0});

    // K sub-tile into registers: MFMA (blk, ks) A operand = row 16*blk + col,
    // features 32*ks + 8*G4 .. +7.  Rows past the chunk re-read its last row.
    auto load_k = [&](int i, u32x4 (&kr)[2][D / 32]) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const uint16_t *krow = kc + row_off(min(i * kSub + 16 * blk + col, n - 1));
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks)
                kr[blk][ks] = ld16(krow + 32 * ks + 8 * G4);
        }
    };
    // V sub-tile into LDS stage i % 3 (row-major rows of D bf16, swizzled)
    auto load_v = [&](int i) {
        unsigned char *dst = vst + (i % kVStages) * DCfg<D>::kVBytes;
        constexpr int C = DCfg<D>::kChunks;
#pragma unroll
        for (int piece = 0; piece < DCfg<D>::kVPieces; ++piece) {
            const int p = piece * 64 + lane;
            const int r = p / C;
            const int c = (p % C) ^ dvswz<D>(r);
            dma16(vc + row_off(min(i * kSub + r, n - 1)) + c * 8, dst + piece * 1024);
        }
    };

    u32x4 kr0[2][D / 32], kr1[2][D / 32], kr2[2][D / 32];
    load_k(0, kr0);
    load_v(0);
    if (nsub > 1) {
        load_k(1, kr1);
        load_v(1);
    }
    const float cs = a.scale * kLog2e;
    // l: row sum of the unrounded p (for the LSE); lp: of the bf16-rounded p
    // that enter the PV MFMA (normalises O, so the weights on V sum to one)
    float m = -INFINITY, l = 0.f, lp = 0.f;
    f32x4 o[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
        o[c] = f32x4{};
    // per-lane transposing-read offset: lane 4j + q of its 16-lane group
    // reads key row (base + j), features 16c + 4q .. +3
    const int trl = lane & 15, trj = trl >> 2, trq = trl & 3;

    // sub-tile i: K in registers k (loaded two sub-tiles earlier), V in LDS
    // stage i % 3; the loads of sub-tile i+2 go to kn and stage (i+2) % 3
    auto step = [&](int i, const u32x4(&k)[2][D / 32], u32x4(&kn)[2][D / 32]) {
        // sub-tile i has landed when at most the loads of sub-tile i+1 are pending
        if (i + 1 < nsub)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * (D / 32) + DCfg<D>::kVPieces) : "memory");
        else
            vm_wait_all();
        if (i + 2 < nsub) {
            load_k(i + 2, kn);
            load_v(i + 2);
        }
        // S^T = K q^T: lane holds head col, keys 16*blk + 4*G4 + r
        f32x4 s[2] = {f32x4{}, f32x4{}};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
                s[blk] = mfma_bf16_16x16x32(as_bf16x8(k[blk][ks]), qf[ks], s[blk]);
        float mx = -INFINITY;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = i * kSub + 16 * blk + 4 * G4 + r;
                s[blk][r] = key < n ? s[blk][r] * cs : -INFINITY;
                mx = fmaxf(mx, s[blk][r]);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        // lazy rescale (the reference max moves only by more than 2^8); the
        // first sub-tile always has a visible key
        if (__any(mx > m + 8.f)) {
            const float m_new = mx > m + 8.f ? mx : m;
            const float alpha = fast_exp2(m - m_new);
            l *= alpha;
            lp *= alpha;
#pragma unroll
            for (int c = 0; c < D / 16; ++c)
                o[c] *= alpha;
            m = m_new;
        }
        // P^T B operand: element e is key 16*(e/4) + 4*G4 + e%4
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            p[e] = fast_exp2(s[e >> 2][e & 3] - m);
            l += p[e];
        }
        const u32x4 pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                          pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            lp = add_bf16x2(pw[e], lp);
        // O^T += V^T P^T: per 16-feature block c, the A operand is keys
        // 4*G4 + 0..3 and 16 + 4*G4 + 0..3 of features 16c + col, gathered by
        // two transposing reads
        const uint32_t vbase = lds_addr(vst + (i % kVStages) * DCfg<D>::kVBytes);
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
            o[c] = mfma_bf16_16x16x32(as_bf16x8(va[c & 1]), as_bf16x8(pw), o[c]);
        }
    };
    for (int i = 0; i < nsub; i += 3) {
        step(i, kr0, kr2);
        if (i + 1 < nsub)
            step(i + 1, kr1, kr0);
        if (i + 2 < nsub)
            step(i + 2, kr2, kr1);
    }

    // partial of this chunk: O_s = acc / lp, lse_s = m + log2 l (log2 units);
    // lane holds head col, features 16c + 4*G4 + r
    float lt = l + __shfl_xor(l, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    float ltp = lp + __shfl_xor(lp, 16, 64);
    ltp += __shfl_xor(ltp, 32, 64);
    if (col < G) {
        const float inv = 1.f / ltp;
        const size_t pidx = ((size_t)b * a.H + kvh * G + col) * a.max_splits + split;
        float *po = a.part_o + pidx * D;
#pragma unroll
        for (int c = 0; c < D / 16; ++c)
            *(f32x4 *)(po + 16 * c + 4 * G4) =
                f32x4{o[c][0] * inv, o[c][1] * inv, o[c][2] * inv, o[c][3] * inv};
        if (G4 == 0)
            a.part_lse[pidx] = m + log2f(lt);
    }
}

// One wave per (sequence, query head): lanes take the chunk LSEs 64 at a
// time for the max and the weight sum, then each lane accumulates D/64
// features over the chunks, with the rows of 64 chunks in flight at once.
constexpr int kMergeWaves = 4;

template <int D, bool OUT_F32>
__global__ __launch_bounds__(64 * kMergeWaves) void decode_merge_kernel(DecodeArgs a)
{
    constexpr int F = D / 64;  // features per lane
    const int lane = threadIdx.x & 63;
    const int bh = (int)blockIdx.x * kMergeWaves + (int)(threadIdx.x >> 6);
    if (bh >= a.B * a.H)
        return;
    const int b = bh / a.H;
    const int L = clamp_len(a.seqlens, b, a.N_max);
    const int ns = (L + a.split_tokens - 1) / a.split_tokens;
    const float *pl = a.part_lse + (size_t)bh * a.max_splits;
    const float *po = a.part_o + (size_t)bh * a.max_splits * D + F * lane;
    float M = -INFINITY;
    for (int s = lane; s < ns; s += 64)
        M = fmaxf(M, pl[s]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        M = fmaxf(M, __shfl_xor(M, off, 64));
    float wsum = 0.f;
    float acc[F] = {};
    for (int s0 = 0; s0 < ns; s0 += 64) {
        const float w = s0 + lane < ns ? fast_exp2(pl[s0 + lane] - M) : 0.f;
        wsum += w;
        const int n = min(64, ns - s0);
        // all 64 chunk rows of the batch in flight at once (rows past the
        // last chunk re-read it and carry weight 0)
        float x[64][F];
#pragma unroll
        for (int j = 0; j < 64; ++j)
#pragma unroll
            for (int f = 0; f < F; ++f)
                x[j][f] = po[(size_t)(s0 + min(j, n - 1)) * D + f];
#pragma unroll
        for (int j = 0; j < 64; ++j) {
            const float wj = __shfl(w, j, 64);
#pragma unroll
            for (int f = 0; f < F; ++f)
                acc[f] = fmaf(wj, x[j][f], acc[f]);
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
    // one wave per possible chunk; waves past the last non-empty chunk exit
    const long long items = (long long)a.B * a.Hkv * a.max_splits;
    dim3 grid((unsigned)((items + kWavesPerWG - 1) / kWavesPerWG));
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

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s)
{
    return a.d == 64 ? launch_d<64>(a, s) : launch_d<128>(a, s);
}

}  // namespace attn
