// Internal interface between the C-ABI front end (sdpa_api.cpp) and the
// kernel launchers.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

struct ForwardArgs {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    const int32_t* key_lens;  // nullptr unless key padding is on
    int B, Hq, Hkv, Sq, Sk, D;
    float scale;
    bool causal;
    bool padded;
    float* lse = nullptr;     // optional [B, Hq, Sq] natural-log log-sum-exp (16-bit dense path)
    // Optional additive mask (16-bit dense path): element (b, h, i, j) at
    // bias[b * bias_sb + h * bias_sh + i * Sk + j], input dtype.
    const void* bias = nullptr;
    int64_t bias_sb = 0, bias_sh = 0;
    // Value / output head dim (v rows and out rows); equal to D except on the
    // paged prefill, where V may be narrower or wider (up to 256).
    int Dv = 0;
    // Workgroups one XCD holds at once (set at launch from the kernel's
    // occupancy; 0: unknown).  Dense non-causal launches sweep the keys
    // backwards in every other such group of an XCD's run, so a group starts
    // on the keys the previous one left in the XCD's L2.
    int sweep_group = 0;
};

// Attention backward (16-bit inputs): dq [B,Hq,Sq,D], dk / dv [B,Hkv,Sk,D].
struct BackwardArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* out;
    const void* dout;
    const float* lse;         // [B, Hq, Sq] from the forward
    const int32_t* key_lens;  // nullptr unless key padding is on
    void* dq;
    void* dk;
    void* dv;
    float* delta;             // workspace [B, Hq, Sq]: rowsum(dO * O)
    float* dq_acc = nullptr;  // atomic variant: fp32 [B, Hq, Sq, D] dQ accumulator (workspace)
    // Optional additive bias as in ForwardArgs (element (b, h, i, j) at
    // bias[b * bias_sb + h * bias_sh + i * Sk + j]) and its gradient dS,
    // dbias [B, Hq, Sq, Sk] (nullptr: not wanted).
    const void* bias = nullptr;
    int64_t bias_sb = 0, bias_sh = 0;
    void* dbias = nullptr;
    int B, Hq, Hkv, Sq, Sk, D;
    float scale;
    bool causal;
    bool padded;
};

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    const int32_t* key_lens;  // nullptr = every key valid
    float* o_part;            // [B, Hq, splits, Dv]
    float* lse_part;          // [B, Hq, splits]
    int B, Hq, Hkv, Sk, D;
    int splits;
    float scale;
    int Dv = 0;               // value / output head dim (v rows, o_part, out); set to D when equal
};

// Paged K/V cache (packed queries).  With these, DecodeArgs holds B = queries,
// Sk = max_seq_len, k / v = the page caches [pages, page_size, Hkv, D] and
// [pages, page_size, Hkv, Dv], and no key_lens.
struct PagedArgs {
    const int32_t* block_tables;  // [num_seqs, max_pages]
    const int32_t* seq_lens;      // [num_seqs]
    const int32_t* query_seq;     // [queries]      (per-query attention)
    const int32_t* query_pos;     // [queries]      (per-query attention)
    const int32_t* cu_seqlens_q;  // [num_seqs + 1] (prefill chunks)
    int num_seqs, max_pages, pages, page_size;
    int total_q;                  // packed query rows (prefill chunks)
    bool causal;
};

hipError_t launch_forward_bf16(const ForwardArgs& a, hipStream_t s);
hipError_t launch_forward_f16(const ForwardArgs& a, hipStream_t s);
hipError_t launch_forward_f32(const ForwardArgs& a, hipStream_t s);
// Dense 16-bit forward with 256 < D <= 1024 (the head-dim-split kernel).
hipError_t launch_forward_wide(const ForwardArgs& a, bool f16, hipStream_t s);
hipError_t launch_paged_prefill_wide(const ForwardArgs& a, const PagedArgs& p, bool f16, hipStream_t s);
// Paged prefill chunks: a.B = num_seqs, a.Sq = longest chunk, a.Sk = max_seq_len;
// bf16 or (f16) fp16; head dims above 256 go to the head-dim-split kernel
// (launch_paged_prefill_wide).
hipError_t launch_paged_prefill_16bit(const ForwardArgs& a, const PagedArgs& p, bool f16,
                                      hipStream_t s);
// fp32 paged prefill chunks (D a multiple of 4 up to 128, Dv = D).
hipError_t launch_paged_prefill_f32(const ForwardArgs& a, const PagedArgs& p, hipStream_t s);
// C = A . B (16-bit, fp32 accumulation) for the attention block's
// projections.  a_heads: A [M = B*S, K = model] is read from (batch, head,
// seq, headDim) layout; c_heads: C [M, N = model] is written to it (headDim
// hd, sequence length S).  blockIdx.y < nz selects (b_z, c_z).
struct GemmArgs {
    const void* a;
    const void* b0;
    const void* b1;
    const void* b2;
    void* c0;
    void* c1;
    void* c2;
    int M, N, K;
    int S, hd;
    int nz;
    bool a_heads, c_heads;
    uint32_t a_bytes;  // extent of A in bytes (< 2 GiB)
};
hipError_t launch_gemm_16bit(const GemmArgs& g, bool f16, hipStream_t s);

// Backward: the dQ pass (also writes delta), then the dK / dV pass.
hipError_t launch_backward_16bit(const BackwardArgs& a, bool f16, hipStream_t s);
// fp32 inputs: ordered backward without a bias, D a multiple of 4 up to 128.
hipError_t launch_backward_f32(const BackwardArgs& a, hipStream_t s);

// Attention backward through a page cache (packed prefill chunks of the paged
// forward): gathers into the dense sections, the dense ordered backward,
// scatters back.  Sizes: L = max_seq_len; D = Dv, a multiple of 8.
struct PagedBackwardArgs {
    const void* q;          // [total_q, Hq, D]
    const void* k_cache;    // [pages, page_size, Hkv, D]
    const void* v_cache;    // [pages, page_size, Hkv, Dv]
    const void* out;        // [total_q, Hq, Dv], the forward's output
    const void* dout;
    const float* lse;       // [total_q, Hq], the forward's log-sum-exp
    void* dq;               // [total_q, Hq, D]
    void* dk_cache;         // [pages, page_size, Hkv, D]
    void* dv_cache;         // [pages, page_size, Hkv, Dv]
    const int32_t* block_tables;  // [num_seqs, max_pages]
    const int32_t* seq_lens;      // [num_seqs]
    const int32_t* cu_seqlens_q;  // [num_seqs + 1]
    int total_q, Hq, Hkv, D, Dv, W, num_seqs, max_pages, pages, page_size, L;
    float scale;
    bool causal;
    // workspace sections, rows W wide (W = max(D, Dv) rounded up to 8; the
    // dims past D of Q, K, dQ, dK and past Dv of V, O, dO, dV are zeros)
    void* qd;    // [num_seqs, Hq, L, W] each: Q, dO, O and dQ at absolute positions
    void* dod;
    void* od;
    void* dqd;
    void* kd;    // [num_seqs, Hkv, L, W] each: K, V, dK, dV of the reachable keys
    void* vd;
    void* dkd;
    void* dvd;
    float* lsed;   // [num_seqs, Hq, L]
    float* stats;  // the dense backward's workspace
};
hipError_t launch_paged_backward_16bit(const PagedBackwardArgs& a, bool f16, hipStream_t s);
// fp32 caches and rows (D = Dv = W a multiple of 4 up to 128).
hipError_t launch_paged_backward_f32(const PagedBackwardArgs& a, hipStream_t s);
// Ordered backward without a bias for 128 < D <= 512 (head dim split across waves).
hipError_t launch_backward_wide(const BackwardArgs& a, bool f16, hipStream_t s);

// Split-KV decode and paged attention, bf16 or (f16) fp16.
hipError_t launch_decode_16bit(const DecodeArgs& a, bool f16, hipStream_t s);
// The split pass of decode for 256 < D <= 1024 (head-dim-split kernel), dense
// (p == nullptr) or through a page cache; writes a.o_part / a.lse_part like
// the narrow split pass.
hipError_t launch_decode_wide_split(const DecodeArgs& a, const PagedArgs* p, bool f16, hipStream_t s);
hipError_t launch_paged_16bit(const DecodeArgs& a, const PagedArgs& p, bool f16, hipStream_t s);
// fp32 inputs (D a multiple of 4 up to 128, Dv = D): the same split pass and
// merge on fp32 MFMAs.
hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t s);
hipError_t launch_paged_f32(const DecodeArgs& a, const PagedArgs& p, hipStream_t s);

// Work items of the decode split pass: (batch, K/V head, block of <= 16 query
// heads, split).
int64_t decode_work_items(int64_t B, int64_t Hq, int64_t Hkv, int splits);

}  // namespace sdpa
