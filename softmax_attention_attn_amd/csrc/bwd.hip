// Attention backward for gfx950: dQ, dK and dV of the exact forward
// O = softmax(Q K^T * s + mask) V for an upstream gradient dO, with the
// forward's LSE (the backward pass of the training kernels the pages discuss:
// "GPU kernel overview" page, SageBwd and the training gaps;
// "flashattention-kernels" page §0, FA2/FA3).  Per row i, with P recomputed
// from the LSE:
//     P_ij = exp(s Q_i.K_j - lse_i),  dP_ij = dO_i.V_j,  D_i = dO_i.O_i,
//     dS_ij = P_ij (dP_ij - D_i),
//     dQ_i = s sum_j dS_ij K_j,  dK_j = s sum_i dS_ij Q_i,  dV_j = sum_i P_ij dO_i,
// and a kv head's dK/dV sum over the query heads of its group.
//
// Two kernels, no atomics (every output element has one writer, so the
// result is deterministic):
//  * bwd_dq: query-stationary.  A workgroup owns 128 queries (4 waves x 32)
//    of one head, keeps their Q and dO in registers and streams the K/V
//    tiles (64 keys) through LDS: S^T = K Q^T and dP^T = V dO^T on the MFMA,
//    dS^T in registers, dQ^T += K^T dS^T with K^T gathered by transposing
//    LDS reads.  It computes D_i = dO_i . O_i (fp32) for its own queries and
//    also writes -D_i and -lse_i / s for the dK/dV kernel, which runs after
//    it.
//  * bwd_dkv: key-stationary.  A workgroup owns 128 keys (4 waves x 32) of
//    one kv head, keeps their K and V in registers and streams, for every
//    query head of the group, the Q/dO tiles (64 queries) through LDS:
//    S = Q K^T, dP = dO V^T, dS, then dV^T += dO^T P and dK^T += Q^T dS with
//    dO^T and Q^T gathered by transposing reads.
// Products take bf16 operands (P and dS rounded to bf16) with fp32
// accumulation; the outputs are bf16 or fp32.
#include "attn_internal.hpp"
#include "cdna4.hpp"

namespace attn {
namespace {

constexpr int kBWaves = 4;
constexpr int kBThreads = 64 * kBWaves;
constexpr int kRows = 32 * kBWaves;  // queries (dq) or keys (dkv) per workgroup
constexpr int kTile = 64;            // streamed rows per step

// LDS tile of kTile rows of D bf16 (16-byte chunks, 16 chunks = the 64 banks).
//  * Padded (SWZ false): rows of 2D + 16 bytes.  A lane group reading 16 bytes
//    of 16 consecutive rows hits 16 distinct bank quads; the transposing reads
//    (4 rows x 64 bytes per 32 lanes) fall partly on the same banks.
//  * Swizzled (SWZ true, D = 128): rows of 2D + 64 bytes, so consecutive rows
//    start 4 bank quads apart, and the low two bits of a row's chunk index
//    are XORed with bits 2-3 of the row (swz).  Both read patterns then touch
//    each of the 64 banks once per phase: 16 rows of one chunk for a row read,
//    and 4 rows x one 64-byte block for a transposing read.
template <int D, bool SWZ = false>
struct BCfg {
    static constexpr int kChunks = D / 8;             // 16-byte chunks per row
    static constexpr int kPad = SWZ ? 4 : 1;          // pad chunks per row
    static constexpr int kPitch = D * 2 + 16 * kPad;  // bytes per LDS row
    static constexpr int kPieces = kTile * (kChunks + kPad) / 64;  // 1 KB direct loads
    static constexpr int kBytes = kPieces * 1024;
    static constexpr int kPerWave = (kPieces + kBWaves - 1) / kBWaves;
    static_assert(kPieces * 64 == kTile * (kChunks + kPad), "tile split");
    static_assert(!SWZ || D == 128, "swizzled layout is laid out for 16 chunks per row");
};

// chunk-index XOR of row `row` in the swizzled layout
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

// Direct loads of one padded tile: piece p = wave + 4i of the tile's pieces,
// lane l fills LDS slot 64p + l = row (64p+l)/(C+1), chunk (64p+l)%(C+1) (the
// pad chunk re-reads chunk 0).  Rows at or past `rows` read as zero (the
// buffer resource ends there).
template <int D, bool SWZ = false>
struct TileLanes {
    uint32_t off[BCfg<D, SWZ>::kPerWave];  // source byte offset within the tile
};

// slot 64p + l of the tile is row q / (C + pad), physical chunk q % (C + pad);
// a swizzled row's physical chunk c holds logical chunk c ^ swz(row).  Pad
// chunks are not loaded (offset kPadSlot): they stay free for other data.
constexpr uint32_t kPadSlot = 0xffffffffu;
template <int D, bool SWZ = false>
__device__ __forceinline__ TileLanes<D, SWZ> tile_lanes(int wave, int lane)
{
    constexpr int C = BCfg<D, SWZ>::kChunks, W = C + BCfg<D, SWZ>::kPad;
    TileLanes<D, SWZ> t;
#pragma unroll
    for (int i = 0; i < BCfg<D, SWZ>::kPerWave; ++i) {
        const int q = (wave + kBWaves * i) * 64 + lane;
        const int row = q / W, c = q % W;
        t.off[i] = c >= C ? kPadSlot : row * (D * 2) + (SWZ ? c ^ swz(row) : c) * 16;
    }
    return t;
}

template <int D, bool SWZ = false>
__device__ __forceinline__ void load_tile(unsigned char *lds, const uint16_t *src, int r0, int N,
                                          int wave, const TileLanes<D, SWZ> &tl)
{
    const int rows = min(kTile, N - r0);
    const __amdgpu_buffer_rsrc_t r = raw_rsrc(src + (size_t)r0 * D, (uint32_t)rows * D * 2);
#pragma unroll
    for (int i = 0; i < BCfg<D, SWZ>::kPerWave; ++i) {
        const int piece = wave + kBWaves * i;
        if (piece < BCfg<D, SWZ>::kPieces && tl.off[i] != kPadSlot)
            dma16_rsrc(r, tl.off[i], lds + piece * 1024);
    }
}

// A operand read straight from a padded tile: lane (n, g) takes row
// row0 + n, bf16 columns 16*ks + 8g .. +7.
template <int D>
__device__ __forceinline__ uint32_t direct_addr(uint32_t tile, int row0, int lane)
{
    return tile + (row0 + (lane & 31)) * BCfg<D>::kPitch + (lane >> 5) * 16;
}

// A operand X^T read from a padded tile of X (rows = the contraction index):
// for the 16 contraction rows base .. base+15 and the 32 columns 32c ..
// 32c+31, lane l (half h = l/32) gets column 32c + l%32 at rows
// base + 4h + 0..3 and base + 8 + 4h + 0..3, the order in which an MFMA
// accumulator of S (rows 8(r/4) + 4g + r%4) hands its registers 8u .. 8u+7 to
// the B operand.  Two transposing reads: in each 16-lane group lane 4j + q
// points at row (base + 4h + j), columns 32c + 16(G&1) + 4q .. +3, and lane i
// of the group receives column 32c + 16(G&1) + i of the four rows.
template <int D>
__device__ __forceinline__ uint32_t trans_addr(uint32_t tile, int lane)
{
    const int G = lane >> 4, L = lane & 15, j = L >> 2, q = L & 3, h = G >> 1;
    return tile + (4 * h + j) * BCfg<D>::kPitch + (16 * (G & 1) + 4 * q) * 2;
}

// Swizzled tiles (row0 and ROW0 multiples of 16, so swz depends on the lane
// only).  Row read of k-step ks: lane (n, g) takes logical chunk 2ks + g of
// row row0 + n, physical chunk 4(ks/2) + ((2(ks%2) + g) ^ swz(n)); the address
// for each parity of ks is kept, and 64(ks/2) bytes go into the offset.
template <int PAR>
__device__ __forceinline__ uint32_t swz_row_addr(uint32_t tile, int lane)
{
    const int n = lane & 31, g = lane >> 5;
    return tile + n * BCfg<128, true>::kPitch + (((2 * PAR + g) ^ swz(n)) << 4);
}

// Transposing read of rows ROW0 + SEC + 4h + j (SEC 0 or 8): lane 4j + q of
// 16-lane group G takes bytes 32(G&1) + 8q of a 64-byte block, that is chunk
// 2(G&1) + q/2 of the block, half q%2; swz of its row is (SEC/4 + h) % 4.
template <int SEC>
__device__ __forceinline__ uint32_t swz_trans_addr(uint32_t tile, int lane)
{
    const int G = lane >> 4, L = lane & 15, j = L >> 2, q = L & 3, h = G >> 1;
    const int kk = (2 * (G & 1) + (q >> 1)) ^ ((SEC / 4 + h) & 3);
    return tile + (SEC + 4 * h + j) * BCfg<128, true>::kPitch + (kk << 4) + (q & 1) * 8;
}

// the 16 contraction rows starting at ROW0 and the column block C of a
// swizzled tile, from the two lane addresses of swz_trans_addr<0> and <8>
template <int ROW0, int C>
__device__ __forceinline__ u32x4 swz_trans_read(uint32_t a0, uint32_t a8)
{
    static_assert(ROW0 % 16 == 0, "row block");
    constexpr int off = ROW0 * BCfg<128, true>::kPitch + C * 64;
    const u32x2 a = lds_read_tr16_b64<off>(a0);
    const u32x2 b = lds_read_tr16_b64<off>(a8);
    return u32x4{a[0], a[1], b[0], b[1]};
}

// the 16 contraction rows starting at ROW0 and the column block C of the
// tile (both compile-time, folded into the read offsets)
template <int D, int ROW0, int C>
__device__ __forceinline__ u32x4 trans_read(uint32_t addr)
{
    constexpr int off = ROW0 * BCfg<D>::kPitch + C * 64;
    const u32x2 a = lds_read_tr16_b64<off>(addr);
    const u32x2 b = lds_read_tr16_b64<off + 8 * BCfg<D>::kPitch>(addr);
    return u32x4{a[0], a[1], b[0], b[1]};
}

// The 16 bf16 of an MFMA accumulator, rounded and packed in register order.
__device__ __forceinline__ void pack16(const float (&x)[16], uint32_t (&w)[8])
{
#pragma unroll
    for (int i = 0; i < 8; ++i)
        w[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
}

// Store a transposed accumulator: acc[c] holds rows 32c + 8(r/4) + 4g + r%4
// (feature index) of column `row` (the lane's query or key); four
// consecutive features per (c, r/4).
template <int D, bool OUT_F32>
__device__ __forceinline__ void store_rows(void *base, size_t row, int g, const f32x16 (&acc)[D / 32],
                                           float mul)
{
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            const int col = 32 * c + 8 * R + 4 * g;
            const float x0 = acc[c][4 * R] * mul, x1 = acc[c][4 * R + 1] * mul,
                        x2 = acc[c][4 * R + 2] * mul, x3 = acc[c][4 * R + 3] * mul;
            if constexpr (OUT_F32) {
                *(f32x4 *)((float *)base + row * D + col) = f32x4{x0, x1, x2, x3};
            } else {
                *(u32x2 *)((uint16_t *)base + row * D + col) =
                    u32x2{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
            }
        }
}

// The lane index, recomputed where it is used.  The instruction pair is
// opaque to the compiler, so it neither keeps the value live across a loop
// nor spills it: a spilled value reloaded inside the dK/dV loop made the
// scratch load's wait also wait for the tile loads issued just before it.
__device__ __forceinline__ uint32_t lane_here()
{
    uint32_t l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// Workgroup -> (outer index, tile) with the outer index's tiles kept on one
// XCD (workgroup i runs on XCD i % 8) when the outer count is a multiple of 8.
__device__ __forceinline__ void bwd_task(int wg, int ntile, int nouter, int &outer, int &tile)
{
    if ((nouter & 7) == 0) {
        const int xcd = wg & 7, slot = wg >> 3;
        outer = xcd + 8 * (slot / ntile);
        tile = slot % ntile;
    } else {
        outer = wg / ntile;
        tile = wg % ntile;
    }
}

// N products, each taking two LDS operands read by rd(i) (OPS read
// instructions in all); the reads run RA products ahead of the MFMAs.
template <int N, int RA, int OPS, class Rd, class Use>
__device__ __forceinline__ void operand_stream(Rd &&rd, Use &&use)
{
    static_assert(OPS * RA <= 15, "lgkmcnt field");
    u32x4 x[RA + 1], y[RA + 1];
    static_for<0, (RA < N ? RA : N)>([&](auto i) {
        constexpr int I = decltype(i)::value;
        rd(i, x[I % (RA + 1)], y[I % (RA + 1)]);
    });
    static_for<0, N>([&](auto i) {
        constexpr int I = decltype(i)::value, B = I % (RA + 1);
        if constexpr (I + RA < N) {
            rd(std::integral_constant<int, I + RA>{}, x[(I + RA) % (RA + 1)],
               y[(I + RA) % (RA + 1)]);
            lgkm_wait<OPS * RA>(x[B]);
            lgkm_wait<OPS * RA>(y[B]);
        } else {
            lgkm_wait<OPS * (N - 1 - I)>(x[B]);
            lgkm_wait<OPS * (N - 1 - I)>(y[B]);
        }
        use(i, x[B], y[B]);
    });
}

// ---------------------------------------------------------------- dQ
// Workgroup: 128 queries of one (b, h); wave w owns queries q0 + 32w .. +31
// (lane n = l % 32 is query q0 + 32w + n).  Key tiles of 64 stream through a
// 2-stage LDS ring (K and V, padded rows), loaded by direct loads one step
// ahead; the workgroup synchronises once per step.
// Compiled for two waves per SIMD: without the bound the compiler kept the
// dQ accumulators in AGPRs and copied them to VGPRs and back around every
// tile (128 extra VALU moves per tile).
template <int D, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(kBThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dq_kernel(BwdArgs a)
{
    // K is read both row-wise and transposed: the swizzled layout (d = 128)
    constexpr bool SW = D == 128;
    using Cf = BCfg<D, SW>;
    constexpr int KB = Cf::kBytes, KS = D / 16, NC = D / 32;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[4 * KB];
    const int lane = threadIdx.x & 63, g = lane >> 5, n = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int N = a.N;
    const int nqt = (N + kRows - 1) / kRows;
    int bh, qt;
    bwd_task(blockIdx.x, nqt, a.B * a.H, bh, qt);
    // causal: a query tile's work grows with its index, so dispatch the
    // longest first (the dK/dV kernel's key tiles already shrink with the index)
    if (CAUSAL)
        qt = nqt - 1 - qt;
    const int h = bh % a.H, b = bh / a.H, kvh = h / (a.H / a.Hkv);
    const int q0 = qt * kRows, qw0 = q0 + 32 * wave, my_q = qw0 + n;
    const uint16_t *kb = (const uint16_t *)a.k + (size_t)(b * a.Hkv + kvh) * N * D;
    const uint16_t *vb = (const uint16_t *)a.v + (size_t)(b * a.Hkv + kvh) * N * D;
    const size_t qrow = (size_t)bh * N + my_q;

    const int kend = CAUSAL ? min(N, q0 + kRows) : N;
    const int ntiles = (kend + kTile - 1) / kTile;
    const int ntw = CAUSAL ? min(ntiles, (qw0 + 31) / kTile + 1) : ntiles;  // this wave's tiles

    const TileLanes<D, SW> tl = tile_lanes<D, SW>(wave, lane);
    auto kst = [&](int t) { return smem + (t & 1) * 2 * KB; };
    auto vst = [&](int t) { return smem + (t & 1) * 2 * KB + KB; };
    load_tile<D, SW>(kst(0), kb, 0, N, wave, tl);
    load_tile<D, SW>(vst(0), vb, 0, N, wave, tl);
    // lane parts of the swizzled read addresses (tile-independent)
    const uint32_t lrow0 = SW ? swz_row_addr<0>(0, lane) : 0;
    const uint32_t lrow1 = SW ? swz_row_addr<1>(0, lane) : 0;
    const uint32_t ltr0 = SW ? swz_trans_addr<0>(0, lane) : 0;
    const uint32_t ltr8 = SW ? swz_trans_addr<8>(0, lane) : 0;

    // Q^T and dO^T fragments (B operands): lane holds row my_q, columns 16ks + 8g .. +7
    bf16x8 qf[KS], df[KS];
    const bool valid_q = my_q < N;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        qf[ks] = as_bf16x8(valid_q ? ld16((const uint16_t *)a.q + qrow * D + 16 * ks + 8 * g)
                                   : u32x4{0, 0, 0, 0});
        df[ks] = as_bf16x8(valid_q ? ld16((const uint16_t *)a.dout + qrow * D + 16 * ks + 8 * g)
                                   : u32x4{0, 0, 0, 0});
    }
    // D = dO . O (fp32 from the bf16 tensors): the lane holds columns
    // 16ks + 8g .. +7 of its query's dO; the other half-wave the rest
    float dpart = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const u32x4 o4 = valid_q ? ld16_nt((const uint16_t *)a.o + qrow * D + 16 * ks + 8 * g)
                                 : u32x4{0, 0, 0, 0};
        const u32x4 d4 = __builtin_bit_cast(u32x4, df[ks]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            dpart += bf16_lo(d4[e]) * bf16_lo(o4[e]) + bf16_hi(d4[e]) * bf16_hi(o4[e]);
    }
    const float dlt = dpart + xor32(dpart);
    const float lse = valid_q ? a.lse[qrow] : 0.f;
    const float cs = a.scale * kLog2e;
    const float lse2 = lse * kLog2e;
    // the dK/dV kernel's per-row -D and -lse/s, 0 on the padding rows past N
    // (the workgroups cover every row of bwd_rows(N))
    if (g == 0 && my_q < bwd_rows(N)) {
        const size_t prow = (size_t)bh * bwd_rows(N) + my_q;
        a.ndelta[prow] = valid_q ? -dlt : 0.f;
        a.nlse[prow] = valid_q ? -lse / a.scale : 0.f;
    }

    f32x16 acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
        acc[c] = f32x16{};

    for (int t = 0; t < ntiles; ++t) {
        vm_wait_n<0>();
        __syncthreads();  // tile t landed; stage (t+1)&1 no longer read
        if (t + 1 < ntiles) {
            load_tile<D, SW>(kst(t + 1), kb, (t + 1) * kTile, N, wave, tl);
            load_tile<D, SW>(vst(t + 1), vb, (t + 1) * kTile, N, wave, tl);
        }
        if (t >= ntw)
            continue;
        const uint32_t ka = lds_addr(kst(t)), va = lds_addr(vst(t));
        const uint32_t kd = SW ? ka + lrow0 : direct_addr<D>(ka, 0, lane);
        const uint32_t vd = SW ? ka + lrow1 : direct_addr<D>(va, 0, lane);
        // S^T = K Q^T and dP^T = V dO^T: rows = keys 32 blk + 8(r/4) + 4g + r%4
        f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
        // product i: block i % 2 (alternating accumulators), k-step i / 2;
        // two products of read-ahead keep two waves per SIMD within 256 registers
        operand_stream<2 * KS, 2, 2>(
            [&](auto i, u32x4 &x, u32x4 &y) {
                constexpr int I = decltype(i)::value;
                if constexpr (SW) {
                    // kd / vd: the addresses for even / odd k-steps; the V tile
                    // is KB bytes after the K tile
                    constexpr int ks = I / 2, off = 32 * (I % 2) * Cf::kPitch + 64 * (ks / 2);
                    const uint32_t a = (ks & 1) ? vd : kd;
                    x = lds_read_b128<off>(a);
                    y = lds_read_b128<off + KB>(a);
                } else {
                    constexpr int off = 32 * (I % 2) * Cf::kPitch + 32 * (I / 2);
                    x = lds_read_b128<off>(kd);
                    y = lds_read_b128<off>(vd);
                }
            },
            [&](auto i, const u32x4 &x, const u32x4 &y) {
                constexpr int I = decltype(i)::value;
                s[I % 2] = mfma_bf16_32x32x16(as_bf16x8(x), qf[I / 2], s[I % 2]);
                dp[I % 2] = mfma_bf16_32x32x16(as_bf16x8(y), df[I / 2], dp[I % 2]);
            });
        // dS^T = P^T (dP^T - D), P^T = 2^(s cs - lse2).  The mask is tested
        // only on tiles that reach past N or past the wave's first query: a
        // masked exponent becomes -inf, so its P and dS are 0.  Queries past
        // N need no test (their Q, dO, lse2 and D read as zero, and their
        // lane is not stored); keys past N are masked, as their zero K rows
        // would meet a P that may overflow.
        const int tend = (t + 1) * kTile;  // one past the tile's last key
        const bool any_masked = tend > N || (CAUSAL && tend - 1 > qw0);
        uint32_t dsw[2][8];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                s[blk][r] = s[blk][r] * cs - lse2;
            if (any_masked) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = t * kTile + 32 * blk + 8 * (r >> 2) + 4 * g + (r & 3);
                    const bool ok = key < N && (!CAUSAL || key <= my_q);
                    s[blk][r] = ok ? s[blk][r] : -INFINITY;
                }
            }
            float ds[16];
#pragma unroll
            for (int r = 0; r < 16; ++r)
                ds[r] = fast_exp2(s[blk][r]) * (dp[blk][r] - dlt);
            pack16(ds, dsw[blk]);
        }
        // dQ^T += K^T dS^T: contraction over the tile's keys, 16 per MFMA
        const uint32_t kt = SW ? ka + ltr0 : trans_addr<D>(ka, lane);
        const uint32_t kt8 = SW ? ka + ltr8 : 0;
        // product pair i: keys 16u .. 16u+15 (u = i / (NC/2)) into the
        // feature blocks c0 = 2(i % (NC/2)) and c0 + 1, so that consecutive
        // MFMAs accumulate into different blocks
        operand_stream<2 * NC, 2, 4>(
            [&](auto i, u32x4 &x, u32x4 &y) {
                constexpr int I = decltype(i)::value, u = I / (NC / 2), c0 = 2 * (I % (NC / 2));
                if constexpr (SW) {
                    x = swz_trans_read<16 * u, c0>(kt, kt8);
                    y = swz_trans_read<16 * u, c0 + 1>(kt, kt8);
                } else {
                    x = trans_read<D, 16 * u, c0>(kt);
                    y = trans_read<D, 16 * u, c0 + 1>(kt);
                }
            },
            [&](auto i, const u32x4 &x, const u32x4 &y) {
                constexpr int I = decltype(i)::value, u = I / (NC / 2), c0 = 2 * (I % (NC / 2));
                const u32x4 w = {dsw[u >> 1][4 * (u & 1)], dsw[u >> 1][4 * (u & 1) + 1],
                                 dsw[u >> 1][4 * (u & 1) + 2], dsw[u >> 1][4 * (u & 1) + 3]};
                acc[c0] = mfma_bf16_32x32x16(as_bf16x8(x), as_bf16x8(w), acc[c0]);
                acc[c0 + 1] = mfma_bf16_32x32x16(as_bf16x8(y), as_bf16x8(w), acc[c0 + 1]);
            });
    }
    if (valid_q)
        store_rows<D, OUT_F32>(a.dq, qrow, g, acc, a.scale);
}

// ---------------------------------------------------------------- dK, dV
// Workgroup: 128 keys of one (b, kv head); wave w owns keys k0 + 32w .. +31
// (lane n is key k0 + 32w + n).  For each query head of the group, query
// tiles of 64 (with their -lse/s and -D rows) stream through a 2-stage LDS ring.
// Two waves per SIMD (two workgroups per CU): the register budget of 256
// then holds the dK/dV accumulators (128), the K/V fragments (64) and the
// operand read-ahead: one product while the S and dP accumulators are live,
// two in the dV/dK products after them.  The second wave hides the LDS
// latency and the score arithmetic, which the read-ahead of a single wave
// did not.
// d = 128: the Q and dO tiles use the swizzled layout (rows of 320 bytes; the
// row reads of S and dP and the transposing reads of dV and dK fall on
// distinct banks), two stages fill 80 KB, so the tile's -lse/s and -D go
// into the row padding: pad chunks 0 and 1 of row j hold them for rows
// 4j .. 4j+3.  d = 64: padded rows and a separate -lse/s, -D area.
// The S and dP accumulators of a step start from those values, so the
// products deliver S - lse/s and dP - D, and a score costs a multiply, an
// exponential, a multiply and the two bf16 conversions.
template <int D, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(kBThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dkv_kernel(BwdArgs a)
{
    constexpr bool SW = D == 128;
    using Cf = BCfg<D, SW>;
    constexpr int KB = Cf::kBytes, KS = D / 16, NC = D / 32;
    constexpr int STAGE = 2 * KB + (SW ? 0 : 2 * kTile * 4);  // Q, dO (, -lse/s, -D)
    __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE];
    const int lane = threadIdx.x & 63, g = lane >> 5, n = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int N = a.N, NP = bwd_rows(N);
    const int G = a.H / a.Hkv;
    const int nkt = (N + kRows - 1) / kRows;
    int bg, kt;
    bwd_task(blockIdx.x, nkt, a.B * a.Hkv, bg, kt);
    const int b = bg / a.Hkv, g_kv = bg % a.Hkv;
    const int k0 = kt * kRows, kw0 = k0 + 32 * wave, my_k = kw0 + n;
    const bool valid_k = my_k < N;
    const size_t krow = (size_t)bg * N + my_k;

    // K and V fragments (B operands): lane holds row my_k, columns 16ks + 8g .. +7
    bf16x8 kf[KS], vf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        kf[ks] = as_bf16x8(valid_k ? ld16((const uint16_t *)a.k + krow * D + 16 * ks + 8 * g)
                                   : u32x4{0, 0, 0, 0});
        vf[ks] = as_bf16x8(valid_k ? ld16((const uint16_t *)a.v + krow * D + 16 * ks + 8 * g)
                                   : u32x4{0, 0, 0, 0});
    }
    const float cs = a.scale * kLog2e;
    f32x16 dk[NC], dv[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        dk[c] = f32x16{};
        dv[c] = f32x16{};
    }

    // the (head, query tile) sequence: for a causal mask the query tiles
    // start at the tile holding this workgroup's first key
    const int t0 = CAUSAL ? k0 / kTile : 0;
    const int nqt = (N + kTile - 1) / kTile;
    const int per_head = nqt - t0;
    const int nsteps = G * per_head;
    auto stage = [&](int i) { return smem + (i & 1) * STAGE; };
    auto load_step = [&](int i) {
        const int hh = b * a.H + g_kv * G + i / per_head;
        const int q0 = (t0 + i % per_head) * kTile;
        unsigned char *st = stage(i);
        // the lane offsets are recomputed per piece from the lane index
        // (lane_here: opaque, so the compiler neither keeps them live across
        // the loop nor spills them; a spilled offset's reload would also wait
        // for the loads issued before it)
        const __amdgpu_buffer_rsrc_t rq =
            raw_rsrc((const uint16_t *)a.q + ((size_t)hh * N + q0) * D,
                     (uint32_t)min(kTile, N - q0) * D * 2);
        const __amdgpu_buffer_rsrc_t rd =
            raw_rsrc((const uint16_t *)a.dout + ((size_t)hh * N + q0) * D,
                     (uint32_t)min(kTile, N - q0) * D * 2);
#pragma unroll
        for (int u = 0; u < Cf::kPerWave; ++u) {
            constexpr int C = Cf::kChunks, W = C + Cf::kPad;
            const int piece = wave + kBWaves * u;
            if (piece < Cf::kPieces) {
                const int q = piece * 64 + (int)lane_here();
                const int row = q / W, c = q % W;
                if (c < C) {  // pad chunks are not loaded
                    const uint32_t off = row * (D * 2) + (SW ? c ^ swz(row) : c) * 16;
                    dma16_rsrc(rq, off, st + piece * 1024);
                    dma16_rsrc(rd, off, st + KB + piece * 1024);
                }
            }
        }
        const float *lsrc = a.nlse + (size_t)hh * NP + q0, *dsrc = a.ndelta + (size_t)hh * NP + q0;
        if constexpr (SW) {
            // wave w fills the pads of rows 4w .. 4w+3: lane 20i + c writes
            // pad chunk c of row 4w + i (rows are 20 chunks apart), 16 bytes
            // of -lse/s (c = 0) or -D (c = 1) of rows 4(4w+i) .. +3; the other
            // lanes are off
            const int l = (int)lane_here(), li = l / 20, c = l - 20 * li;
            const uint32_t off = 16 * (4 * wave + li);
            unsigned char *pad = st + 4 * wave * Cf::kPitch + 2 * D;
            if (li < 4 && c == 0)
                dma16_rsrc(raw_rsrc(lsrc, kTile * 4), off, pad);
            if (li < 4 && c == 1)
                dma16_rsrc(raw_rsrc(dsrc, kTile * 4), off, pad);
        } else {
            const int rows = min(kTile, N - q0);
            const int l = (int)lane_here();
            if (wave == 0)
                dma4_rsrc(raw_rsrc(lsrc, rows * 4), l * 4, st + 2 * KB);
            else if (wave == 1)
                dma4_rsrc(raw_rsrc(dsrc, rows * 4), l * 4, st + 2 * KB + kTile * 4);
        }
    };
    if (nsteps > 0)
        load_step(0);
    for (int i = 0; i < nsteps; ++i) {
        vm_wait_n<0>();
        __syncthreads();  // step i landed; stage (i+1)&1 no longer read
        if (i + 1 < nsteps)
            load_step(i + 1);
        const int q0 = (t0 + i % per_head) * kTile;
        unsigned char *st = stage(i);
        const uint32_t qa = lds_addr(st), da = lds_addr(st + KB);
        static_for<0, 2>([&](auto qc) {
            constexpr int qs = decltype(qc)::value;  // queries q0 + 32 qs .. +31
            // causal: skip when every query of the step precedes every key of the wave
            if (CAUSAL && q0 + 32 * qs + 31 < kw0)
                return;
            // S = Q K^T - lse/s and dP = dO V^T - D: rows = queries
            // 32 qs + 8(r/4) + 4g + r%4; the accumulators start from -lse/s
            // and -D of their rows (rows r0 .. r0+3 for registers 4R .. 4R+3)
            f32x16 s, dp;
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                const int r0 = 32 * qs + 8 * R + 4 * g;
                f32x4 l4, d4;
                if constexpr (SW) {
                    const unsigned char *pad = st + (r0 / 4) * Cf::kPitch + 2 * D;
                    l4 = *(const f32x4 *)pad;
                    d4 = *(const f32x4 *)(pad + 16);
                } else {
                    const float *lse_s = (const float *)(st + 2 * KB);
                    l4 = *(const f32x4 *)(lse_s + r0);
                    d4 = *(const f32x4 *)(lse_s + kTile + r0);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    s[4 * R + e] = l4[e];
                    dp[4 * R + e] = d4[e];
                }
            }
            // the lane parts of the swizzled addresses are recomputed here
            // from the lane index (lane_here), not kept live across the loop:
            // at the 256-register bound they spilled
            const int lh = SW ? (int)lane_here() : lane;
            const uint32_t lrow0 = SW ? swz_row_addr<0>(0, lh) : 0;
            const uint32_t lrow1 = SW ? swz_row_addr<1>(0, lh) : 0;
            const uint32_t qd = SW ? qa : direct_addr<D>(qa, 32 * qs, lane);
            const uint32_t dd = SW ? da : direct_addr<D>(da, 32 * qs, lane);
            operand_stream<KS, 1, 2>(
                [&](auto i, u32x4 &x, u32x4 &y) {
                    constexpr int ks = decltype(i)::value;
                    if constexpr (SW) {
                        // logical chunk 2ks + g of row 32qs + n: the lane part
                        // for the parity of ks, 64 (ks / 2) bytes in the offset
                        constexpr int off = 32 * qs * Cf::kPitch + 64 * (ks / 2);
                        const uint32_t lr = (ks & 1) ? lrow1 : lrow0;
                        x = lds_read_b128<off>(qd + lr);
                        y = lds_read_b128<off>(dd + lr);
                    } else {
                        x = lds_read_b128<32 * ks>(qd);
                        y = lds_read_b128<32 * ks>(dd);
                    }
                },
                [&](auto i, const u32x4 &x, const u32x4 &y) {
                    constexpr int ks = decltype(i)::value;
                    s = mfma_bf16_32x32x16(as_bf16x8(x), kf[ks], s);
                    dp = mfma_bf16_32x32x16(as_bf16x8(y), vf[ks], dp);
                });
            // P = 2^((S - lse/s) s log2(e)), dS = P (dP - D).  Only the
            // causal mask is tested, and only on sub-steps with a query before
            // the wave's last key (a masked exponent becomes -inf, so P = 0).
            // Queries past N need no test: their Q, dO, -lse/s and -D rows
            // read as zero, so P = 1 and dP - D = 0 and both products add
            // nothing.  Keys past N touch only their own (unstored) lane.
            const int qf = q0 + 32 * qs;  // the sub-step's first query
            if (CAUSAL && qf < kw0 + 31) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int q = qf + 8 * (r >> 2) + 4 * g + (r & 3);
                    s[r] = my_k <= q ? s[r] : -INFINITY;
                }
            }
            float p[16], ds[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                p[r] = fast_exp2(s[r] * cs);
                ds[r] = p[r] * dp[r];
            }
            uint32_t pw[8], dsw[8];
            pack16(p, pw);
            pack16(ds, dsw);
            // dV^T += dO^T P and dK^T += Q^T dS: contraction over the step's queries
            // product pair i: queries 16u .. 16u+15 of the step (u = i / NC),
            // feature block c = i % NC (consecutive pairs use different
            // blocks); the reads run two pairs ahead
            const int lt = SW ? (int)lane_here() : lane;
            const uint32_t ltr0 = SW ? swz_trans_addr<0>(0, lt) : 0;
            const uint32_t ltr8 = SW ? swz_trans_addr<8>(0, lt) : 0;
            const uint32_t qt_a = SW ? qa + ltr0 : trans_addr<D>(qa, lane);
            const uint32_t dt_a = SW ? da + ltr0 : trans_addr<D>(da, lane);
            const uint32_t qt8 = qa + ltr8, dt8 = da + ltr8;
            operand_stream<2 * NC, 2, 4>(
                [&](auto i, u32x4 &x, u32x4 &y) {
                    constexpr int I = decltype(i)::value, c = I % NC, u = I / NC;
                    if constexpr (SW) {
                        x = swz_trans_read<32 * qs + 16 * u, c>(dt_a, dt8);
                        y = swz_trans_read<32 * qs + 16 * u, c>(qt_a, qt8);
                    } else {
                        x = trans_read<D, 32 * qs + 16 * u, c>(dt_a);
                        y = trans_read<D, 32 * qs + 16 * u, c>(qt_a);
                    }
                },
                [&](auto i, const u32x4 &x, const u32x4 &y) {
                    constexpr int I = decltype(i)::value, c = I % NC, u = I / NC;
                    const u32x4 wp = {pw[4 * u], pw[4 * u + 1], pw[4 * u + 2], pw[4 * u + 3]};
                    const u32x4 wd = {dsw[4 * u], dsw[4 * u + 1], dsw[4 * u + 2],
                                      dsw[4 * u + 3]};
                    dv[c] = mfma_bf16_32x32x16(as_bf16x8(x), as_bf16x8(wp), dv[c]);
                    dk[c] = mfma_bf16_32x32x16(as_bf16x8(y), as_bf16x8(wd), dk[c]);
                });
        });
    }
    if (valid_k) {
        store_rows<D, OUT_F32>(a.dk, krow, g, dk, a.scale);
        store_rows<D, OUT_F32>(a.dv, krow, g, dv, 1.f);
    }
}

template <int D, bool CAUSAL, bool OUT_F32>
hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t s)
{
    const int nt = (a.N + kRows - 1) / kRows;
    {
        ProfScope ps("bwd_dq", s);
        hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, OUT_F32>), dim3(a.B * a.H * nt),
                           dim3(kBThreads), 0, s, a);
    }
    ProfScope ps("bwd_dkv", s);
    hipLaunchKernelGGL((bwd_dkv_kernel<D, CAUSAL, OUT_F32>), dim3(a.B * a.Hkv * nt),
                       dim3(kBThreads), 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs &a, hipStream_t s)
{
    if (a.causal)
        return a.out_fp32 ? launch_bwd_t<D, true, true>(a, s) : launch_bwd_t<D, true, false>(a, s);
    return a.out_fp32 ? launch_bwd_t<D, false, true>(a, s) : launch_bwd_t<D, false, false>(a, s);
}

}  // namespace

hipError_t launch_bwd(const BwdArgs &a, hipStream_t s)
{
    return a.d == 64 ? launch_bwd_d<64>(a, s) : launch_bwd_d<128>(a, s);
}

}  // namespace attn
