// Internal interface between the C-ABI layer (api.cpp) and the HIP kernels.
// Not installed; the public contract is include/attn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

struct PrefillArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;  // may be null
    int B, H, Hkv, N, d;
    int causal;
    float scale;
    int out_fp32;  // 0: bf16 output, 1: fp32 output
    // Packed variable-length batch (cu_seqlens non-null): sequence b holds
    // tokens [cu_seqlens[b], cu_seqlens[b+1]) of q/o [total, H, d] and k/v
    // [total, Hkv, d]; lse is [H, total]; N is then the longest sequence.
    const int32_t *cu_seqlens = nullptr;
    int total = 0;
};

struct DecodeArgs {
    const void *q, *k, *v;
    const int32_t *seqlens;
    void *o;
    float *lse;  // may be null
    int B, H, Hkv, N_max, d;
    float scale;
    int out_fp32;
    int split_tokens;
    // partials of the split kernel, one slot per (wave, segment) piece:
    // slot = b * Hkv + kvh + wave, decode_partial_slots(B, Hkv) slots
    float *part_o;    // [slots, H / Hkv, d]
    float *part_lse;  // [slots, H / Hkv], log2 units
    // Paged caches (block_table non-null): k and v are [num_pages, Hkv,
    // page_size, d] with page_size = 1 << page_shift, and key position n of
    // sequence b lives in page block_table[b * max_pages + (n >> page_shift)].
    // N_max = max_pages * page_size.
    const int32_t *block_table = nullptr;
    int page_shift = 0, max_pages = 0, num_pages = 0;
};

struct BwdArgs {
    const void *q, *k, *v, *o, *dout;  // bf16; q/o/dout [B,H,N,d], k/v [B,Hkv,N,d]
    const float *lse;                  // [B,H,N], natural log, from the forward
    void *dq, *dk, *dv;                // dq [B,H,N,d], dk/dv [B,Hkv,N,d]
    int B, H, Hkv, N, d;
    int causal;
    float scale;
    int out_fp32;  // gradients in fp32 (1) or bf16 (0)
    float *ndelta;  // workspace [B,H,bwd_rows(N)]: -(dO . O) per row, 0 past N
    float *nlse;    // workspace [B,H,bwd_rows(N)]: -lse / scale per row, 0 past N
};

// Rows per head of the backward's -D and -lse/scale arrays: N rounded up to
// the 64-row tiles the dK/dV kernel loads whole (the rows past N hold 0).
constexpr int kBwdRowPad = 64;
__host__ __device__ inline int bwd_rows(int N) { return (N + kBwdRowPad - 1) / kBwdRowPad * kBwdRowPad; }

struct SageArgs {
    PrefillArgs p;
    void *workspace;
    size_t workspace_bytes;
};

// Kernel launchers (defined in the .hip files).  They assume validated
// arguments and return the launch status.
hipError_t launch_prefill_exact(const PrefillArgs &a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t s);  // contiguous or paged caches
// The split-KV decode divides the keys of a call among at most this many
// waves (four per CU of a 256-CU MI355X, all resident at once).
constexpr int kDecodeWaves = 1024;
size_t decode_partial_slots(int B, int Hkv);
// Device address, on the current device, of the fixed array that holds the
// partials of attn_decode_noalloc (ATTN_DECODE_SCRATCH_BYTES bytes).
hipError_t decode_scratch(void **ptr);
hipError_t launch_sage(const SageArgs &a, hipStream_t s);
// the MX modes (same arguments): elem_bits 4 = MXFP4 (E2M1), 6 = MXFP6 (E2M3)
hipError_t launch_mx(const SageArgs &a, int elem_bits, hipStream_t s);
size_t mx_workspace_bytes(int B, int H, int Hkv, int N, int d, int elem_bits);
// byte offset of each piece of an MX mode's workspace (attn.h's
// attn_mx_ws_piece order, kMxWsPieces entries)
constexpr int kMxWsPieces = 9;
void mx_workspace_layout(int B, int H, int Hkv, int N, int d, int elem_bits, size_t *offsets);
hipError_t launch_bwd(const BwdArgs &a, hipStream_t s);
size_t sage_workspace_bytes(int B, int H, int Hkv, int N, int d);
// byte offset of each piece of the quantised mode's workspace (attn.h's
// attn_sage_ws_piece order, kSageWsPieces entries)
constexpr int kSageWsPieces = 11;
void sage_workspace_layout(int B, int H, int Hkv, int N, int d, size_t *offsets);

// Benchmark timing hooks (api.cpp): bracket one kernel launch with events when
// the profiler is enabled on this thread.
void prof_begin(const char *name, hipStream_t s);
void prof_end(hipStream_t s);

struct ProfScope {
    hipStream_t s;
    ProfScope(const char *name, hipStream_t st) : s(st) { prof_begin(name, s); }
    ~ProfScope() { prof_end(s); }
};

}  // namespace attn
