// C-ABI front end of libsdpa: argument validation (on the host, before any
// HIP call), kernel choice and launch on the caller's stream.  The contract
// is documented in include/sdpa.h.
#include "sdpa.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>

#include "launch.hpp"

namespace {

thread_local char g_last_error[512] = "";

sdpa_status_t fail(sdpa_status_t s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return s;
}

sdpa_status_t ok() {
    g_last_error[0] = '\0';
    return SDPA_OK;
}

bool mul_ok(int64_t a, int64_t b, int64_t* r) { return !__builtin_mul_overflow(a, b, r); }

// Element count of a 4-D tensor, or -1 on int64 overflow.
int64_t numel4(int64_t a, int64_t b, int64_t c, int64_t d) {
    int64_t r;
    if (!mul_ok(a, b, &r) || !mul_ok(r, c, &r) || !mul_ok(r, d, &r)) return -1;
    return r;
}

bool overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    if (!a || !b || abytes <= 0 || bbytes <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

int64_t elem_size(int dtype) { return dtype == SDPA_F32 ? 4 : 2; }
bool known_dtype(int dtype) { return dtype == SDPA_F32 || dtype == SDPA_BF16 || dtype == SDPA_F16; }

// Head dims the kernels cover: 16-bit inputs any multiple of 8 up to max16
// (the 64-, 128- and 256-wide kernels read the missing chunks as zeros),
// fp32 any multiple of 4 up to 128 (likewise on the 64- and 128-wide fp32
// kernel).  max16: the widest 16-bit head dim of the entry point (1024 for
// every forward entry point, whose heads above 256 run on the head-dim-split
// kernel; 512 for the ordered backward, above 128 on its head-dim-split
// kernels; 128 for the atomic backward and the backward with a bias, whose
// lanes hold a full-width operand and gradient).  any16: the entry point
// also takes every 16-bit head dim from 1 to max16 (the forward and decode
// kernels' element-wise load path for widths that are not multiples of 8).
bool head_dim_ok(int64_t D, int dtype, int64_t max16 = 128, bool any16 = false) {
    if (dtype == SDPA_F32) return D >= 4 && D <= 128 && D % 4 == 0;
    if (any16) return D >= 1 && D <= max16;
    return D >= 8 && D <= max16 && D % 8 == 0;
}

// Value head dim of the paged entry points: Dv == D on every kernel; Dv != D
// on the 16-bit kernels with D and Dv both up to 1024 (above 256 on the
// head-dim-split kernel, whose waves cover the larger of the two).
sdpa_status_t check_value_dim(int64_t D, int64_t Dv, int dtype) {
    if (Dv == D) return SDPA_OK;
    if (dtype == SDPA_F32 || !head_dim_ok(D, dtype, 1024, true) || !head_dim_ok(Dv, dtype, 1024, true))
        return fail(SDPA_ERR_UNSUPPORTED,
                    "value head dim Dv=%lld differs from D=%lld: supported for bf16 / fp16 with "
                    "both up to 1024",
                    (long long)Dv, (long long)D);
    return SDPA_OK;
}

// Floats per row of the split partials: the value head dim rounded up to 4,
// so each row starts 16-byte aligned.
int64_t partial_pitch(int64_t Dv) { return (Dv + 3) & ~int64_t(3); }

// Head dim of the paged backward's dense pass: the larger of D and Dv
// rounded up to a multiple of 8 (the narrower operands are zero-padded).
int64_t paged_backward_width(int64_t D, int64_t Dv) { return ((D > Dv ? D : Dv) + 7) & ~int64_t(7); }

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Shared checks of both entry points.  On success fills the tensor byte sizes.
sdpa_status_t check_common(const void* q, const void* k, const void* v, void* out, int64_t B,
                           int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D,
                           float scale, int dtype, int64_t* qbytes, int64_t* kbytes,
                           int64_t max16 = 128, bool any16 = false) {
    if (!q || !k || !v || !out) return fail(SDPA_ERR_INVALID_ARGUMENT, "null tensor pointer");
    if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < 1 || D < 1)
        return fail(SDPA_ERR_INVALID_ARGUMENT,
                    "every size must be >= 1 (B=%lld Hq=%lld Hkv=%lld Sq=%lld Sk=%lld D=%lld)",
                    (long long)B, (long long)Hq, (long long)Hkv, (long long)Sq, (long long)Sk,
                    (long long)D);
    if (Hq % Hkv != 0)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "Hq (%lld) must be a multiple of Hkv (%lld)",
                    (long long)Hq, (long long)Hkv);
    if (!std::isfinite(scale) || !(scale > 0.f))
        return fail(SDPA_ERR_INVALID_ARGUMENT, "scale must be finite and > 0");
    if (!known_dtype(dtype)) return fail(SDPA_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
    const int64_t es = elem_size(dtype);
    const int64_t nq = numel4(B, Hq, Sq, D), nk = numel4(B, Hkv, Sk, D);
    if (nq < 0 || nk < 0 || !mul_ok(nq, es, qbytes) || !mul_ok(nk, es, kbytes))
        return fail(SDPA_ERR_INVALID_ARGUMENT, "tensor byte size overflows int64");
    if (overlap(out, *qbytes, q, *qbytes) || overlap(out, *qbytes, k, *kbytes) ||
        overlap(out, *qbytes, v, *kbytes))
        return fail(SDPA_ERR_INVALID_ARGUMENT, "out overlaps q, k or v");
    if (B > INT_MAX || Hq > INT_MAX || Sq > INT_MAX || Sk > INT_MAX)
        return fail(SDPA_ERR_UNSUPPORTED, "a size exceeds the kernels' 32-bit index range");
    // Per-head rows are addressed through buffer resources with 32-bit extents.
    if (Sq * D * es > INT_MAX || Sk * D * es > INT_MAX)
        return fail(SDPA_ERR_UNSUPPORTED, "one head of q, k or v exceeds 2 GiB");
    if (!head_dim_ok(D, dtype, max16, any16))
        return fail(SDPA_ERR_UNSUPPORTED, "head dim D=%lld not supported (%s%lld)", (long long)D,
                    dtype == SDPA_F32 ? "fp32: a multiple of 4 up to "
                    : any16           ? "any width up to "
                                      : "a multiple of 8 up to ",
                    dtype == SDPA_F32 ? 128LL : (long long)max16);
    return SDPA_OK;
}

sdpa_status_t hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess)
        return fail(SDPA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

const char* sdpa_status_string(int status) {
    switch (status) {
        case SDPA_OK: return "ok";
        case SDPA_ERR_INVALID_ARGUMENT: return "invalid argument";
        case SDPA_ERR_UNSUPPORTED: return "unsupported configuration";
        case SDPA_ERR_WORKSPACE: return "workspace missing or too small";
        case SDPA_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* sdpa_last_error(void) { return g_last_error; }

}  // extern "C"

namespace {

sdpa_status_t forward_impl(const void* q, const void* k, const void* v, int64_t B, int64_t Hq,
                           int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D, float scale,
                           int mask_kind, const int32_t* key_lens, void* out, float* lse,
                           int dtype, void* stream, const void* bias = nullptr,
                           int64_t bias_sb = 0, int64_t bias_sh = 0) {
    int64_t qbytes = 0, kbytes = 0;
    sdpa_status_t st = check_common(q, k, v, out, B, Hq, Hkv, Sq, Sk, D, scale, dtype, &qbytes,
                                    &kbytes, 1024, bias == nullptr);
    if (st != SDPA_OK) return st;
    if (mask_kind & ~(SDPA_MASK_CAUSAL | SDPA_MASK_KEY_PADDING))
        return fail(SDPA_ERR_INVALID_ARGUMENT, "unknown mask flags 0x%x", mask_kind);
    const bool causal = mask_kind & SDPA_MASK_CAUSAL;
    const bool padded = mask_kind & SDPA_MASK_KEY_PADDING;
    if (causal && Sq != Sk)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "causal mask needs Sq == Sk (got %lld, %lld)",
                    (long long)Sq, (long long)Sk);
    if (padded != (key_lens != nullptr))
        return fail(SDPA_ERR_INVALID_ARGUMENT,
                    "key_lens must be given exactly when SDPA_MASK_KEY_PADDING is set");
    if (padded && overlap(out, qbytes, key_lens, B * (int64_t)sizeof(int32_t)))
        return fail(SDPA_ERR_INVALID_ARGUMENT, "out overlaps key_lens");
    if (lse) {
        const int64_t lbytes = B * Hq * Sq * (int64_t)sizeof(float);
        if (overlap(lse, lbytes, out, qbytes) || overlap(lse, lbytes, q, qbytes) ||
            overlap(lse, lbytes, k, kbytes) || overlap(lse, lbytes, v, kbytes) ||
            (padded && overlap(lse, lbytes, key_lens, B * (int64_t)sizeof(int32_t))))
            return fail(SDPA_ERR_INVALID_ARGUMENT, "lse overlaps another tensor");
    }
    if (bias) {
        if (dtype == SDPA_F32)
            return fail(SDPA_ERR_UNSUPPORTED, "an additive bias needs 16-bit inputs");
        if (bias_sb < 0 || bias_sh < 0)
            return fail(SDPA_ERR_INVALID_ARGUMENT, "bias strides must be >= 0");
        if (Sk % 8 != 0 || bias_sb % 8 != 0 || bias_sh % 8 != 0 ||
            reinterpret_cast<uintptr_t>(bias) % 16 != 0)
            return fail(SDPA_ERR_UNSUPPORTED,
                        "bias rows must be 16-byte aligned (Sk and the strides multiples of 8, "
                        "pointer 16-byte aligned)");
        if (Sq * Sk * 2 > INT_MAX)
            return fail(SDPA_ERR_UNSUPPORTED, "one head's bias exceeds 2 GiB");
        int64_t last = 0;
        if (!mul_ok(B - 1, bias_sb, &last)) return fail(SDPA_ERR_INVALID_ARGUMENT, "bias extent overflows");
        int64_t hext = 0;
        if (!mul_ok(Hq - 1, bias_sh, &hext) || __builtin_add_overflow(last, hext, &last) ||
            __builtin_add_overflow(last, Sq * Sk, &last) || last > INT64_MAX / 2)
            return fail(SDPA_ERR_INVALID_ARGUMENT, "bias extent overflows");
        const int64_t bbytes = last * 2;
        if (overlap(out, qbytes, bias, bbytes) ||
            (lse && overlap(lse, B * Hq * Sq * (int64_t)sizeof(float), bias, bbytes)))
            return fail(SDPA_ERR_INVALID_ARGUMENT, "out or lse overlaps the bias");
    }
    const int64_t blocks = ((Sq + 31) / 32) * B * Hq;  // the wide-head kernel's 32-row blocks
    if (blocks > INT_MAX / 512)
        return fail(SDPA_ERR_UNSUPPORTED, "launch grid too large (%lld workgroups)", (long long)blocks);

    sdpa::ForwardArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.key_lens = key_lens;
    a.B = (int)B;
    a.Hq = (int)Hq;
    a.Hkv = (int)Hkv;
    a.Sq = (int)Sq;
    a.Sk = (int)Sk;
    a.D = (int)D;
    a.Dv = (int)D;
    a.scale = scale;
    a.causal = causal;
    a.padded = padded;
    a.lse = lse;
    a.bias = bias;
    a.bias_sb = bias_sb;
    a.bias_sh = bias_sh;
    (void)hipGetLastError();  // clear an unrelated pending error
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = dtype == SDPA_BF16  ? sdpa::launch_forward_bf16(a, s)
                         : dtype == SDPA_F16 ? sdpa::launch_forward_f16(a, s)
                                             : sdpa::launch_forward_f32(a, s);
    return hip_status(e, "sdpa_forward launch");
}

// Rows per head in the backward's statistics workspace (8 bytes per row):
// Sq rounded up to even, as the kernels index it.
int64_t stats_rows(int64_t Sq) { return (Sq + 1) & ~int64_t(1); }

}  // namespace

extern "C" {

sdpa_status_t sdpa_forward(const void* q, const void* k, const void* v, int64_t B, int64_t Hq,
                           int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D, float scale,
                           int mask_kind, const int32_t* key_lens, void* out, int dtype,
                           void* stream) {
    return forward_impl(q, k, v, B, Hq, Hkv, Sq, Sk, D, scale, mask_kind, key_lens, out, nullptr,
                        dtype, stream);
}

sdpa_status_t sdpa_forward_lse(const void* q, const void* k, const void* v, int64_t B,
                               int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D,
                               float scale, int mask_kind, const int32_t* key_lens, void* out,
                               float* lse, int dtype, void* stream) {
    if (!lse) return fail(SDPA_ERR_INVALID_ARGUMENT, "null lse pointer");
    return forward_impl(q, k, v, B, Hq, Hkv, Sq, Sk, D, scale, mask_kind, key_lens, out, lse,
                        dtype, stream);
}

sdpa_status_t sdpa_forward_bias(const void* q, const void* k, const void* v, int64_t B,
                                int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D,
                                float scale, int mask_kind, const int32_t* key_lens,
                                const void* bias, int64_t bias_stride_b, int64_t bias_stride_h,
                                void* out, float* lse, int dtype, void* stream) {
    if (!bias) return fail(SDPA_ERR_INVALID_ARGUMENT, "null bias pointer");
    return forward_impl(q, k, v, B, Hq, Hkv, Sq, Sk, D, scale, mask_kind, key_lens, out, lse,
                        dtype, stream, bias, bias_stride_b, bias_stride_h);
}

size_t sdpa_backward_workspace_size(int64_t B, int64_t Hq, int64_t Sq) {
    if (B < 1 || Hq < 1 || Sq < 1) return 0;
    const int64_t rows = numel4(B, Hq, stats_rows(Sq), 1);
    if (rows < 0 || rows > INT64_MAX / 16) return 0;
    return round_up((size_t)rows * 2 * sizeof(float));
}

}  // extern "C"

namespace {

sdpa_status_t backward_impl(const void* q, const void* k, const void* v, const void* out,
                            const void* dout, const float* lse, int64_t B, int64_t Hq,
                            int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D, float scale,
                            int mask_kind, const int32_t* key_lens, void* dq, void* dk, void* dv,
                            void* workspace, size_t workspace_bytes, int dtype, void* stream,
                            bool atomic, const void* bias = nullptr, int64_t bias_sb = 0,
                            int64_t bias_sh = 0, void* dbias = nullptr) {
    if (!out || !dout || !lse || !dk || !dv)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "null tensor pointer");
    int64_t qbytes = 0, kbytes = 0;
    // head dims of any width up to 512 on the ordered backward without a
    // bias (above 128 on the head-dim-split kernels); multiples of 8 up to
    // 128 with a bias or atomic dQ
    sdpa_status_t st = check_common(q, k, v, dq, B, Hq, Hkv, Sq, Sk, D, scale, dtype, &qbytes,
                                    &kbytes, (atomic || bias) ? 128 : 512, !(atomic || bias));
    if (st != SDPA_OK) return st;
    if (dtype == SDPA_F32 && (atomic || bias))
        return fail(SDPA_ERR_UNSUPPORTED,
                    "the atomic backward and the backward with a bias need 16-bit inputs (bf16 or "
                    "fp16)");
    if (mask_kind & ~(SDPA_MASK_CAUSAL | SDPA_MASK_KEY_PADDING))
        return fail(SDPA_ERR_INVALID_ARGUMENT, "unknown mask flags 0x%x", mask_kind);
    const bool causal = mask_kind & SDPA_MASK_CAUSAL;
    const bool padded = mask_kind & SDPA_MASK_KEY_PADDING;
    if (causal && Sq != Sk)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "causal mask needs Sq == Sk (got %lld, %lld)",
                    (long long)Sq, (long long)Sk);
    if (padded != (key_lens != nullptr))
        return fail(SDPA_ERR_INVALID_ARGUMENT,
                    "key_lens must be given exactly when SDPA_MASK_KEY_PADDING is set");
    const size_t need = atomic ? sdpa_backward_atomic_workspace_size(B, Hq, Sq, D)
                               : sdpa_backward_workspace_size(B, Hq, Sq);
    if (atomic && Sq * D * 4 > INT_MAX)
        return fail(SDPA_ERR_UNSUPPORTED, "one head's fp32 dQ accumulator exceeds 2 GiB");
    if (!workspace || workspace_bytes < need)
        return fail(SDPA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace_bytes);
    // Outputs and workspace overlap nothing else.
    const int64_t lbytes = B * Hq * Sq * (int64_t)sizeof(float);
    const int64_t kl = padded ? B * (int64_t)sizeof(int32_t) : 0;
    struct Span {
        const void* p;
        int64_t n;
    };
    // Bias (as sdpa_forward_bias) and its gradient [B, Hq, Sq, Sk].
    int64_t bbytes = 0, dbbytes = 0;
    if (bias) {
        if (bias_sb < 0 || bias_sh < 0)
            return fail(SDPA_ERR_INVALID_ARGUMENT, "bias strides must be >= 0");
        if (Sk % 8 != 0 || bias_sb % 8 != 0 || bias_sh % 8 != 0 ||
            reinterpret_cast<uintptr_t>(bias) % 16 != 0)
            return fail(SDPA_ERR_UNSUPPORTED,
                        "bias rows must be 16-byte aligned (Sk and the strides multiples of 8, "
                        "pointer 16-byte aligned)");
        if (Sq * Sk * 2 > INT_MAX)
            return fail(SDPA_ERR_UNSUPPORTED, "one head's bias exceeds 2 GiB");
        int64_t last = 0, hext = 0;
        if (!mul_ok(B - 1, bias_sb, &last) || !mul_ok(Hq - 1, bias_sh, &hext) ||
            __builtin_add_overflow(last, hext, &last) || __builtin_add_overflow(last, Sq * Sk, &last) ||
            last > INT64_MAX / 2)
            return fail(SDPA_ERR_INVALID_ARGUMENT, "bias extent overflows");
        bbytes = last * 2;
        if (dbias) {
            if (reinterpret_cast<uintptr_t>(dbias) % 16 != 0)
                return fail(SDPA_ERR_UNSUPPORTED, "dbias must be 16-byte aligned");
            const int64_t n = numel4(B, Hq, Sq, Sk);
            if (n < 0 || n > INT64_MAX / 2) return fail(SDPA_ERR_INVALID_ARGUMENT, "dbias size overflows");
            dbbytes = n * 2;
        }
    } else if (dbias) {
        return fail(SDPA_ERR_INVALID_ARGUMENT, "dbias needs a bias");
    }
    const Span ins[] = {{q, qbytes}, {k, kbytes}, {v, kbytes}, {out, qbytes},
                        {dout, qbytes}, {lse, lbytes}, {key_lens, kl}, {bias, bbytes}};
    const Span outs[] = {{dq, qbytes}, {dk, kbytes}, {dv, kbytes}, {workspace, (int64_t)need},
                         {dbias, dbbytes}};
    for (int i = 0; i < 5; ++i) {
        for (const Span& x : ins)
            if (overlap(outs[i].p, outs[i].n, x.p, x.n))
                return fail(SDPA_ERR_INVALID_ARGUMENT, "an output or the workspace overlaps an input");
        for (int j = 0; j < i; ++j)
            if (overlap(outs[i].p, outs[i].n, outs[j].p, outs[j].n))
                return fail(SDPA_ERR_INVALID_ARGUMENT, "outputs overlap each other or the workspace");
    }
    const int64_t qblocks = ((Sq + 127) / 128) * B * Hq, kblocks = ((Sk + 127) / 128) * B * Hkv;
    if (qblocks > INT_MAX / 256 || kblocks > INT_MAX / 256)
        return fail(SDPA_ERR_UNSUPPORTED, "launch grid too large");

    sdpa::BackwardArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.dout = dout;
    a.lse = lse;
    a.key_lens = key_lens;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.delta = static_cast<float*>(workspace);
    if (atomic)
        a.dq_acc = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                            sdpa_backward_workspace_size(B, Hq, Sq));
    a.B = (int)B;
    a.Hq = (int)Hq;
    a.Hkv = (int)Hkv;
    a.Sq = (int)Sq;
    a.Sk = (int)Sk;
    a.D = (int)D;
    a.scale = scale;
    a.causal = causal;
    a.padded = padded;
    a.bias = bias;
    a.bias_sb = bias_sb;
    a.bias_sh = bias_sh;
    a.dbias = dbias;
    (void)hipGetLastError();
    const hipStream_t s = static_cast<hipStream_t>(stream);
    return hip_status(dtype == SDPA_F32 ? sdpa::launch_backward_f32(a, s)
                                        : sdpa::launch_backward_16bit(a, dtype == SDPA_F16, s),
                      "sdpa_backward launch");
}

}  // namespace

extern "C" {

sdpa_status_t sdpa_backward(const void* q, const void* k, const void* v, const void* out,
                            const void* dout, const float* lse, int64_t B, int64_t Hq,
                            int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D, float scale,
                            int mask_kind, const int32_t* key_lens, void* dq, void* dk, void* dv,
                            void* workspace, size_t workspace_bytes, int dtype, void* stream) {
    return backward_impl(q, k, v, out, dout, lse, B, Hq, Hkv, Sq, Sk, D, scale, mask_kind, key_lens,
                         dq, dk, dv, workspace, workspace_bytes, dtype, stream, false);
}

sdpa_status_t sdpa_backward_bias(const void* q, const void* k, const void* v, const void* out,
                                 const void* dout, const float* lse, int64_t B, int64_t Hq,
                                 int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D, float scale,
                                 int mask_kind, const int32_t* key_lens, const void* bias,
                                 int64_t bias_stride_b, int64_t bias_stride_h, void* dq, void* dk,
                                 void* dv, void* dbias, void* workspace, size_t workspace_bytes,
                                 int dtype, void* stream) {
    if (!bias) return fail(SDPA_ERR_INVALID_ARGUMENT, "null bias pointer");
    return backward_impl(q, k, v, out, dout, lse, B, Hq, Hkv, Sq, Sk, D, scale, mask_kind, key_lens,
                         dq, dk, dv, workspace, workspace_bytes, dtype, stream, false, bias,
                         bias_stride_b, bias_stride_h, dbias);
}

size_t sdpa_backward_atomic_workspace_size(int64_t B, int64_t Hq, int64_t Sq, int64_t D) {
    const size_t st = sdpa_backward_workspace_size(B, Hq, Sq);
    if (st == 0 || D < 1) return 0;
    const int64_t n = numel4(B, Hq, Sq, D);
    if (n < 0 || n > INT64_MAX / 8) return 0;
    return st + round_up((size_t)n * sizeof(float));
}

sdpa_status_t sdpa_backward_atomic(const void* q, const void* k, const void* v, const void* out,
                                   const void* dout, const float* lse, int64_t B, int64_t Hq,
                                   int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D, float scale,
                                   int mask_kind, const int32_t* key_lens, void* dq, void* dk,
                                   void* dv, void* workspace, size_t workspace_bytes, int dtype,
                                   void* stream) {
    return backward_impl(q, k, v, out, dout, lse, B, Hq, Hkv, Sq, Sk, D, scale, mask_kind, key_lens,
                         dq, dk, dv, workspace, workspace_bytes, dtype, stream, true);
}

size_t sdpa_block_workspace_size(int64_t B, int64_t S, int64_t model) {
    if (B < 1 || S < 1 || model < 1) return 0;
    const int64_t n = numel4(B, S, model, 1);
    if (n < 0 || n > INT64_MAX / 16) return 0;
    return 4 * round_up((size_t)n * 2);
}

sdpa_status_t sdpa_block_forward(const void* x, const void* wq, const void* wk, const void* wv,
                                 const void* wo, int64_t B, int64_t S, int64_t model,
                                 int64_t heads, float scale, int mask_kind,
                                 const int32_t* key_lens, void* y, void* workspace,
                                 size_t workspace_bytes, int dtype, void* stream) {
    if (!x || !wq || !wk || !wv || !wo || !y)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "null tensor pointer");
    if (B < 1 || S < 1 || model < 1 || heads < 1)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "every size must be >= 1");
    if (!known_dtype(dtype)) return fail(SDPA_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
    if (dtype == SDPA_F32)
        return fail(SDPA_ERR_UNSUPPORTED, "the attention block needs 16-bit inputs (bf16 or fp16)");
    if (model % heads != 0)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "model width %lld is not a multiple of heads %lld",
                    (long long)model, (long long)heads);
    const int64_t hd = model / heads;
    if (!head_dim_ok(hd, dtype, 1024))
        return fail(SDPA_ERR_UNSUPPORTED, "head dim %lld not supported (a multiple of 8 up to 1024)",
                    (long long)hd);
    if (!std::isfinite(scale) || !(scale > 0.f))
        return fail(SDPA_ERR_INVALID_ARGUMENT, "scale must be finite and > 0");
    if (mask_kind & ~(SDPA_MASK_CAUSAL | SDPA_MASK_KEY_PADDING))
        return fail(SDPA_ERR_INVALID_ARGUMENT, "unknown mask flags 0x%x", mask_kind);
    const bool padded = mask_kind & SDPA_MASK_KEY_PADDING;
    if (padded != (key_lens != nullptr))
        return fail(SDPA_ERR_INVALID_ARGUMENT,
                    "key_lens must be given exactly when SDPA_MASK_KEY_PADDING is set");
    const int64_t n = numel4(B, S, model, 1);
    if (n < 0 || n > INT_MAX / 2 || model * model > INT_MAX / 2)
        return fail(SDPA_ERR_UNSUPPORTED, "an activation or weight exceeds 2 GiB");
    const size_t need = sdpa_block_workspace_size(B, S, model);
    if (!workspace || workspace_bytes < need)
        return fail(SDPA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace_bytes);
    const int64_t xb = n * 2, wb = model * model * 2;
    const void* ins[] = {x, wq, wk, wv, wo};
    const int64_t insz[] = {xb, wb, wb, wb, wb};
    for (int i = 0; i < 5; ++i)
        if (overlap(y, xb, ins[i], insz[i]) || overlap(workspace, (int64_t)need, ins[i], insz[i]))
            return fail(SDPA_ERR_INVALID_ARGUMENT, "y or the workspace overlaps an input");
    if (overlap(y, xb, workspace, (int64_t)need) ||
        (padded && (overlap(y, xb, key_lens, B * 4) || overlap(workspace, (int64_t)need, key_lens, B * 4))))
        return fail(SDPA_ERR_INVALID_ARGUMENT, "y, the workspace and key_lens overlap");

    char* ws = static_cast<char*>(workspace);
    const size_t part = round_up((size_t)n * 2);
    void *qb = ws, *kb = ws + part, *vb = ws + 2 * part, *ob = ws + 3 * part;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const bool f16 = dtype == SDPA_F16;
    (void)hipGetLastError();
    // q, k, v = heads(x . w): one launch, written straight into head layout.
    sdpa::GemmArgs g{};
    g.a = x;
    g.b0 = wq;
    g.b1 = wk;
    g.b2 = wv;
    g.c0 = qb;
    g.c1 = kb;
    g.c2 = vb;
    g.M = (int)(B * S);
    g.N = (int)model;
    g.K = (int)model;
    g.S = (int)S;
    g.hd = (int)hd;
    g.nz = 3;
    g.a_heads = false;
    g.c_heads = true;
    g.a_bytes = (uint32_t)xb;
    hipError_t e = sdpa::launch_gemm_16bit(g, f16, s);
    if (e != hipSuccess) return hip_status(e, "sdpa_block_forward projection launch");
    sdpa::ForwardArgs a;
    a.q = qb;
    a.k = kb;
    a.v = vb;
    a.out = ob;
    a.key_lens = key_lens;
    a.B = (int)B;
    a.Hq = (int)heads;
    a.Hkv = (int)heads;
    a.Sq = (int)S;
    a.Sk = (int)S;
    a.D = (int)hd;
    a.Dv = (int)hd;
    a.scale = scale;
    a.causal = mask_kind & SDPA_MASK_CAUSAL;
    a.padded = padded;
    e = f16 ? sdpa::launch_forward_f16(a, s) : sdpa::launch_forward_bf16(a, s);
    if (e != hipSuccess) return hip_status(e, "sdpa_block_forward attention launch");
    // y = heads^-1(o) . wo: A read from head layout.
    sdpa::GemmArgs go = g;
    go.a = ob;
    go.b0 = wo;
    go.c0 = y;
    go.nz = 1;
    go.a_heads = true;
    go.c_heads = false;
    e = sdpa::launch_gemm_16bit(go, f16, s);
    return hip_status(e, "sdpa_block_forward output projection launch");
}

size_t sdpa_decode_workspace_size(int64_t B, int64_t Hq, int64_t D, int num_splits) {
    if (B < 1 || Hq < 1 || D < 1 || num_splits < 1 || num_splits > SDPA_MAX_SPLITS) return 0;
    const int64_t rows = numel4(B, Hq, num_splits, 1);
    const int64_t no = numel4(B, Hq, num_splits, partial_pitch(D));
    if (rows < 0 || no < 0 || no > INT64_MAX / 8) return 0;
    return round_up((size_t)no * sizeof(float)) + round_up((size_t)rows * sizeof(float));
}

namespace {

// Device scratch of sdpa_decode_noalloc: its split partials, laid out as the
// workspace of sdpa_decode.  One copy per GPU, held until the process ends.
// No part of it has to start at zero: the split pass writes every partial
// slot (an empty split writes o_part = 0, lse = -inf) before the merge reads.
static __device__ __align__(256) unsigned char scratch[SDPA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of the current device's copy of scratch, looked up once per
// device.  In host code the array's own name is only a host-side stand-in.
sdpa_status_t scratch_address(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(SDPA_ERR_UNSUPPORTED, "device ordinal %d beyond %d", dev, kMaxDevices - 1);
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p) return hip_status(e, "hipGetSymbolAddress(scratch)");
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return SDPA_OK;
}

// sdpa_decode's checks and launch.  With noalloc the partials go to the
// current device's scratch (workspace and workspace_bytes are ignored).
sdpa_status_t decode_impl(const void* q, const void* k, const void* v, int64_t B, int64_t Hq,
                          int64_t Hkv, int64_t Sk, int64_t D, float scale,
                          const int32_t* key_lens, int num_splits, void* workspace,
                          size_t workspace_bytes, void* out, int dtype, void* stream,
                          bool noalloc) {
    int64_t qbytes = 0, kbytes = 0;
    sdpa_status_t st =
        check_common(q, k, v, out, B, Hq, Hkv, 1, Sk, D, scale, dtype, &qbytes, &kbytes, 1024, true);
    if (st != SDPA_OK) return st;
    if (num_splits < 1 || num_splits > SDPA_MAX_SPLITS)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "num_splits=%d outside 1..%d", num_splits,
                    SDPA_MAX_SPLITS);
    if (key_lens && overlap(out, qbytes, key_lens, B * (int64_t)sizeof(int32_t)))
        return fail(SDPA_ERR_INVALID_ARGUMENT, "out overlaps key_lens");
    const size_t need = sdpa_decode_workspace_size(B, Hq, D, num_splits);
    if (need == 0) return fail(SDPA_ERR_INVALID_ARGUMENT, "workspace size overflows");
    if (noalloc) {
        if (need > (size_t)SDPA_NOALLOC_SCRATCH_BYTES)
            return fail(SDPA_ERR_WORKSPACE,
                        "decode partials need %zu bytes, beyond the %zu-byte device scratch of "
                        "sdpa_decode_noalloc (fewer splits, or sdpa_decode with a workspace)",
                        need, (size_t)SDPA_NOALLOC_SCRATCH_BYTES);
    } else if (!workspace || workspace_bytes < need) {
        return fail(SDPA_ERR_WORKSPACE, "decode needs a workspace of %zu bytes (got %zu)", need,
                    workspace ? workspace_bytes : (size_t)0);
    } else if (overlap(out, qbytes, workspace, (int64_t)need)) {
        return fail(SDPA_ERR_INVALID_ARGUMENT, "out overlaps the workspace");
    }
    const int64_t items = sdpa::decode_work_items(B, Hq, Hkv, num_splits);
    if (items > INT_MAX)
        return fail(SDPA_ERR_UNSUPPORTED, "too many decode work items (%lld)", (long long)items);
    if (noalloc) {
        st = scratch_address(&workspace);
        if (st != SDPA_OK) return st;
    }

    sdpa::DecodeArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.key_lens = key_lens;
    a.o_part = static_cast<float*>(workspace);
    a.lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                          round_up((size_t)numel4(B, Hq, num_splits, partial_pitch(D)) * 4));
    a.B = (int)B;
    a.Hq = (int)Hq;
    a.Hkv = (int)Hkv;
    a.Sk = (int)Sk;
    a.D = (int)D;
    a.Dv = (int)D;
    a.splits = num_splits;
    a.scale = scale;
    (void)hipGetLastError();
    const hipError_t e =
        dtype == SDPA_F32
            ? sdpa::launch_decode_f32(a, static_cast<hipStream_t>(stream))
            : sdpa::launch_decode_16bit(a, dtype == SDPA_F16, static_cast<hipStream_t>(stream));
    return hip_status(e, noalloc ? "sdpa_decode_noalloc launch" : "sdpa_decode launch");
}

}  // namespace

sdpa_status_t sdpa_decode(const void* q, const void* k, const void* v, int64_t B, int64_t Hq,
                          int64_t Hkv, int64_t Sk, int64_t D, float scale,
                          const int32_t* key_lens, int num_splits, void* workspace,
                          size_t workspace_bytes, void* out, int dtype, void* stream) {
    return decode_impl(q, k, v, B, Hq, Hkv, Sk, D, scale, key_lens, num_splits, workspace,
                       workspace_bytes, out, dtype, stream, false);
}

sdpa_status_t sdpa_decode_noalloc(const void* q, const void* k, const void* v, int64_t B,
                                  int64_t Hq, int64_t Hkv, int64_t Sk, int64_t D, float scale,
                                  const int32_t* key_lens, int num_splits, void* out, int dtype,
                                  void* stream) {
    return decode_impl(q, k, v, B, Hq, Hkv, Sk, D, scale, key_lens, num_splits, nullptr, 0, out,
                       dtype, stream, true);
}

sdpa_status_t sdpa_paged_attention(const void* q, const void* k_cache, const void* v_cache,
                                   int64_t queries, int64_t Hq, int64_t Hkv, int64_t D, int64_t Dv,
                                   int64_t pages, int64_t page_size, const int32_t* block_tables,
                                   int64_t num_seqs, int64_t max_pages_per_seq,
                                   const int32_t* seq_lens, const int32_t* query_seq,
                                   const int32_t* query_pos, int64_t max_seq_len, float scale,
                                   int causal, int num_splits, void* workspace,
                                   size_t workspace_bytes, void* out, int dtype, void* stream) {
    if (!q || !k_cache || !v_cache || !out || !block_tables || !seq_lens || !query_seq || !query_pos)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "null pointer argument");
    if (queries < 1 || Hq < 1 || Hkv < 1 || D < 1 || Dv < 1 || pages < 1 || page_size < 1 ||
        num_seqs < 1 || max_pages_per_seq < 1 || max_seq_len < 1)
        return fail(SDPA_ERR_INVALID_ARGUMENT,
                    "every size must be >= 1 (queries=%lld Hq=%lld Hkv=%lld D=%lld Dv=%lld "
                    "pages=%lld page_size=%lld num_seqs=%lld max_pages_per_seq=%lld "
                    "max_seq_len=%lld)",
                    (long long)queries, (long long)Hq, (long long)Hkv, (long long)D, (long long)Dv,
                    (long long)pages, (long long)page_size, (long long)num_seqs,
                    (long long)max_pages_per_seq, (long long)max_seq_len);
    if (Hq % Hkv != 0)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "Hq (%lld) must be a multiple of Hkv (%lld)",
                    (long long)Hq, (long long)Hkv);
    if (!std::isfinite(scale) || !(scale > 0.f))
        return fail(SDPA_ERR_INVALID_ARGUMENT, "scale must be finite and > 0");
    if (!known_dtype(dtype)) return fail(SDPA_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
    if (causal != 0 && causal != 1)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1 (got %d)", causal);
    if (num_splits < 1 || num_splits > SDPA_MAX_SPLITS)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "num_splits=%d outside 1..%d", num_splits,
                    SDPA_MAX_SPLITS);
    int64_t cap = 0;
    if (!mul_ok(max_pages_per_seq, page_size, &cap) || max_seq_len > cap)
        return fail(SDPA_ERR_INVALID_ARGUMENT,
                    "max_seq_len (%lld) exceeds the page table capacity max_pages_per_seq * "
                    "page_size",
                    (long long)max_seq_len);
    const int64_t es = elem_size(dtype);
    const int64_t nq = numel4(queries, Hq, D, 1), no = numel4(queries, Hq, Dv, 1);
    const int64_t nc = numel4(pages, page_size, Hkv, D), nvc = numel4(pages, page_size, Hkv, Dv);
    const int64_t nt = numel4(num_seqs, max_pages_per_seq, 1, 1);
    int64_t qbytes = 0, obytes = 0, cbytes = 0, vcbytes = 0;
    if (nq < 0 || no < 0 || nc < 0 || nvc < 0 || nt < 0 || !mul_ok(nq, es, &qbytes) ||
        !mul_ok(no, es, &obytes) || !mul_ok(nc, es, &cbytes) || !mul_ok(nvc, es, &vcbytes))
        return fail(SDPA_ERR_INVALID_ARGUMENT, "tensor byte size overflows int64");
    if (overlap(out, obytes, q, qbytes) || overlap(out, obytes, k_cache, cbytes) ||
        overlap(out, obytes, v_cache, vcbytes) || overlap(out, obytes, block_tables, nt * 4) ||
        overlap(out, obytes, seq_lens, num_seqs * 4) || overlap(out, obytes, query_seq, queries * 4) ||
        overlap(out, obytes, query_pos, queries * 4))
        return fail(SDPA_ERR_INVALID_ARGUMENT, "out overlaps an input");
    const size_t need = sdpa_decode_workspace_size(queries, Hq, Dv, num_splits);
    if (need == 0) return fail(SDPA_ERR_INVALID_ARGUMENT, "workspace size overflows");
    if (!workspace || workspace_bytes < need)
        return fail(SDPA_ERR_WORKSPACE, "paged attention needs a workspace of %zu bytes (got %zu)",
                    need, workspace ? workspace_bytes : (size_t)0);
    if (overlap(out, obytes, workspace, (int64_t)need))
        return fail(SDPA_ERR_INVALID_ARGUMENT, "out overlaps the workspace");
    if (queries > INT_MAX || Hq > INT_MAX || pages > INT_MAX || num_seqs > INT_MAX ||
        max_pages_per_seq > INT_MAX || max_seq_len > INT_MAX)
        return fail(SDPA_ERR_UNSUPPORTED, "a size exceeds the kernels' 32-bit index range");
    if (!head_dim_ok(D, dtype, 1024, true))
        return fail(SDPA_ERR_UNSUPPORTED,
                    "head dim D=%lld not supported (16-bit: any width up to 1024; fp32: a "
                    "multiple of 4 up to 128)",
                    (long long)D);
    const sdpa_status_t vst = check_value_dim(D, Dv, dtype);
    if (vst != SDPA_OK) return vst;
    if (page_size % 16 != 0)
        return fail(SDPA_ERR_UNSUPPORTED, "page_size=%lld is not a multiple of 16",
                    (long long)page_size);
    const int64_t page_elems = numel4(page_size, Hkv, D > Dv ? D : Dv, es);
    if (page_elems < 0 || page_elems > INT_MAX)
        return fail(SDPA_ERR_UNSUPPORTED, "one page exceeds 2 GiB");
    const int64_t items = sdpa::decode_work_items(queries, Hq, Hkv, num_splits);
    if (items > INT_MAX)
        return fail(SDPA_ERR_UNSUPPORTED, "too many work items (%lld)", (long long)items);

    sdpa::DecodeArgs a;
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.out = out;
    a.key_lens = nullptr;
    a.o_part = static_cast<float*>(workspace);
    a.lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                          round_up((size_t)numel4(queries, Hq, num_splits, partial_pitch(Dv)) * 4));
    a.B = (int)queries;
    a.Hq = (int)Hq;
    a.Hkv = (int)Hkv;
    a.Sk = (int)max_seq_len;
    a.D = (int)D;
    a.Dv = (int)Dv;
    a.splits = num_splits;
    a.scale = scale;
    sdpa::PagedArgs p;
    p.block_tables = block_tables;
    p.seq_lens = seq_lens;
    p.query_seq = query_seq;
    p.query_pos = query_pos;
    p.num_seqs = (int)num_seqs;
    p.max_pages = (int)max_pages_per_seq;
    p.pages = (int)pages;
    p.page_size = (int)page_size;
    p.causal = causal != 0;
    (void)hipGetLastError();
    const hipError_t e =
        dtype == SDPA_F32
            ? sdpa::launch_paged_f32(a, p, static_cast<hipStream_t>(stream))
            : sdpa::launch_paged_16bit(a, p, dtype == SDPA_F16, static_cast<hipStream_t>(stream));
    return hip_status(e, "sdpa_paged_attention launch");
}

sdpa_status_t sdpa_paged_prefill(const void* q, const void* k_cache, const void* v_cache,
                                 int64_t total_q, int64_t Hq, int64_t Hkv, int64_t D, int64_t Dv,
                                 int64_t pages,
                                 int64_t page_size, const int32_t* block_tables, int64_t num_seqs,
                                 int64_t max_pages_per_seq, const int32_t* seq_lens,
                                 const int32_t* cu_seqlens_q, int64_t max_q, int64_t max_seq_len,
                                 float scale, int causal, void* out, float* lse, int dtype,
                                 void* stream) {
    if (!q || !k_cache || !v_cache || !out || !block_tables || !seq_lens || !cu_seqlens_q)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "null pointer argument");
    if (total_q < 1 || Hq < 1 || Hkv < 1 || D < 1 || Dv < 1 || pages < 1 || page_size < 1 ||
        num_seqs < 1 || max_pages_per_seq < 1 || max_q < 1 || max_seq_len < 1)
        return fail(SDPA_ERR_INVALID_ARGUMENT,
                    "every size must be >= 1 (total_q=%lld Hq=%lld Hkv=%lld D=%lld Dv=%lld "
                    "pages=%lld page_size=%lld num_seqs=%lld max_pages_per_seq=%lld max_q=%lld "
                    "max_seq_len=%lld)",
                    (long long)total_q, (long long)Hq, (long long)Hkv, (long long)D, (long long)Dv,
                    (long long)pages, (long long)page_size, (long long)num_seqs,
                    (long long)max_pages_per_seq, (long long)max_q, (long long)max_seq_len);
    if (Hq % Hkv != 0)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "Hq (%lld) must be a multiple of Hkv (%lld)",
                    (long long)Hq, (long long)Hkv);
    if (!std::isfinite(scale) || !(scale > 0.f))
        return fail(SDPA_ERR_INVALID_ARGUMENT, "scale must be finite and > 0");
    if (!known_dtype(dtype)) return fail(SDPA_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
    if (causal != 0 && causal != 1)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1 (got %d)", causal);
    int64_t cap = 0;
    if (!mul_ok(max_pages_per_seq, page_size, &cap) || max_seq_len > cap)
        return fail(SDPA_ERR_INVALID_ARGUMENT,
                    "max_seq_len (%lld) exceeds the page table capacity max_pages_per_seq * "
                    "page_size",
                    (long long)max_seq_len);
    const int64_t es = elem_size(dtype);
    const int64_t nq = numel4(total_q, Hq, D, 1), no = numel4(total_q, Hq, Dv, 1);
    const int64_t nc = numel4(pages, page_size, Hkv, D), nvc = numel4(pages, page_size, Hkv, Dv);
    const int64_t nt = numel4(num_seqs, max_pages_per_seq, 1, 1);
    int64_t qbytes = 0, obytes = 0, cbytes = 0, vcbytes = 0;
    if (nq < 0 || no < 0 || nc < 0 || nvc < 0 || nt < 0 || !mul_ok(nq, es, &qbytes) ||
        !mul_ok(no, es, &obytes) || !mul_ok(nc, es, &cbytes) || !mul_ok(nvc, es, &vcbytes))
        return fail(SDPA_ERR_INVALID_ARGUMENT, "tensor byte size overflows int64");
    if (overlap(out, obytes, q, qbytes) || overlap(out, obytes, k_cache, cbytes) ||
        overlap(out, obytes, v_cache, vcbytes) || overlap(out, obytes, block_tables, nt * 4) ||
        overlap(out, obytes, seq_lens, num_seqs * 4) ||
        overlap(out, obytes, cu_seqlens_q, (num_seqs + 1) * 4))
        return fail(SDPA_ERR_INVALID_ARGUMENT, "out overlaps an input");
    const int64_t lbytes = lse ? numel4(total_q, Hq, 4, 1) : 0;
    if (lse && (overlap(lse, lbytes, out, obytes) || overlap(lse, lbytes, q, qbytes) ||
                overlap(lse, lbytes, k_cache, cbytes) || overlap(lse, lbytes, v_cache, vcbytes) ||
                overlap(lse, lbytes, block_tables, nt * 4) || overlap(lse, lbytes, seq_lens, num_seqs * 4) ||
                overlap(lse, lbytes, cu_seqlens_q, (num_seqs + 1) * 4)))
        return fail(SDPA_ERR_INVALID_ARGUMENT, "lse overlaps out or an input");
    if (total_q > INT_MAX || Hq > INT_MAX || pages > INT_MAX || num_seqs > INT_MAX ||
        max_pages_per_seq > INT_MAX || max_q > INT_MAX || max_seq_len > INT_MAX)
        return fail(SDPA_ERR_UNSUPPORTED, "a size exceeds the kernels' 32-bit index range");
    if (!head_dim_ok(D, dtype, 1024, true))
        return fail(SDPA_ERR_UNSUPPORTED,
                    "head dim D=%lld not supported (16-bit: any width up to 1024; fp32: a "
                    "multiple of 4 up to 128)",
                    (long long)D);
    const sdpa_status_t vst = check_value_dim(D, Dv, dtype);
    if (vst != SDPA_OK) return vst;
    if (page_size % 16 != 0)
        return fail(SDPA_ERR_UNSUPPORTED, "page_size=%lld is not a multiple of 16",
                    (long long)page_size);
    const int64_t DM = D > Dv ? D : Dv;
    const int64_t page_elems = numel4(page_size, Hkv, DM, es);
    const int64_t chunk_bytes = numel4(max_q + 127, Hq, DM, es);  // one workgroup's Q / O rows
    if (page_elems < 0 || page_elems > INT_MAX || chunk_bytes < 0 || chunk_bytes > INT_MAX)
        return fail(SDPA_ERR_UNSUPPORTED, "one page or one chunk of q exceeds 2 GiB");
    const int64_t blocks = ((max_q + 127) / 128) * num_seqs * Hq;
    if (blocks > INT_MAX / 256)
        return fail(SDPA_ERR_UNSUPPORTED, "launch grid too large (%lld workgroups)", (long long)blocks);

    sdpa::ForwardArgs a;
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.out = out;
    a.key_lens = nullptr;
    a.B = (int)num_seqs;
    a.Hq = (int)Hq;
    a.Hkv = (int)Hkv;
    a.Sq = (int)max_q;
    a.Sk = (int)max_seq_len;
    a.D = (int)D;
    a.Dv = (int)Dv;
    a.scale = scale;
    a.causal = causal != 0;
    a.padded = false;
    a.lse = lse;
    sdpa::PagedArgs p{};
    p.block_tables = block_tables;
    p.seq_lens = seq_lens;
    p.cu_seqlens_q = cu_seqlens_q;
    p.num_seqs = (int)num_seqs;
    p.max_pages = (int)max_pages_per_seq;
    p.pages = (int)pages;
    p.page_size = (int)page_size;
    p.total_q = (int)total_q;
    p.causal = causal != 0;
    (void)hipGetLastError();
    const hipError_t e =
        dtype == SDPA_F32
            ? sdpa::launch_paged_prefill_f32(a, p, static_cast<hipStream_t>(stream))
            : sdpa::launch_paged_prefill_16bit(a, p, dtype == SDPA_F16, static_cast<hipStream_t>(stream));
    return hip_status(e, "sdpa_paged_prefill launch");
}

size_t sdpa_paged_backward_workspace_size(int64_t num_seqs, int64_t Hq, int64_t Hkv,
                                          int64_t max_seq_len, int64_t D, int64_t Dv, int dtype) {
    if (num_seqs < 1 || Hq < 1 || Hkv < 1 || max_seq_len < 1 || D < 1 || Dv < 1 || D > 1 << 20 ||
        Dv > 1 << 20 || !known_dtype(dtype))
        return 0;
    const int64_t W = dtype == SDPA_F32 ? D : paged_backward_width(D, Dv);
    const int64_t es = elem_size(dtype);
    const int64_t rows = numel4(num_seqs, Hq, max_seq_len, W), kv = numel4(num_seqs, Hkv, max_seq_len, W);
    const int64_t l = numel4(num_seqs, Hq, max_seq_len, 1);
    if (rows < 0 || kv < 0 || l < 0 || rows > INT64_MAX / 64 || kv > INT64_MAX / 64) return 0;
    const size_t stats = sdpa_backward_workspace_size(num_seqs, Hq, max_seq_len);
    if (stats == 0) return 0;
    return 4 * round_up((size_t)(rows * es)) + 4 * round_up((size_t)(kv * es)) + round_up((size_t)l * 4) + stats;
}

sdpa_status_t sdpa_paged_backward(const void* q, const void* k_cache, const void* v_cache,
                                  const void* out, const void* dout, const float* lse,
                                  int64_t total_q, int64_t Hq, int64_t Hkv, int64_t D, int64_t Dv,
                                  int64_t pages,
                                  int64_t page_size, const int32_t* block_tables, int64_t num_seqs,
                                  int64_t max_pages_per_seq, const int32_t* seq_lens,
                                  const int32_t* cu_seqlens_q, int64_t max_seq_len, float scale,
                                  int causal, void* dq, void* dk_cache, void* dv_cache,
                                  void* workspace, size_t workspace_bytes, int dtype, void* stream) {
    if (!q || !k_cache || !v_cache || !out || !dout || !lse || !block_tables || !seq_lens ||
        !cu_seqlens_q || !dq || !dk_cache || !dv_cache)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "null pointer argument");
    if (total_q < 1 || Hq < 1 || Hkv < 1 || D < 1 || Dv < 1 || pages < 1 || page_size < 1 ||
        num_seqs < 1 || max_pages_per_seq < 1 || max_seq_len < 1)
        return fail(SDPA_ERR_INVALID_ARGUMENT,
                    "every size must be >= 1 (total_q=%lld Hq=%lld Hkv=%lld D=%lld Dv=%lld "
                    "pages=%lld page_size=%lld num_seqs=%lld max_pages_per_seq=%lld "
                    "max_seq_len=%lld)",
                    (long long)total_q, (long long)Hq, (long long)Hkv, (long long)D, (long long)Dv,
                    (long long)pages, (long long)page_size, (long long)num_seqs,
                    (long long)max_pages_per_seq, (long long)max_seq_len);
    if (Hq % Hkv != 0)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "Hq (%lld) must be a multiple of Hkv (%lld)",
                    (long long)Hq, (long long)Hkv);
    if (!std::isfinite(scale) || !(scale > 0.f))
        return fail(SDPA_ERR_INVALID_ARGUMENT, "scale must be finite and > 0");
    if (!known_dtype(dtype)) return fail(SDPA_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
    if (causal != 0 && causal != 1)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1 (got %d)", causal);
    int64_t cap = 0;
    if (!mul_ok(max_pages_per_seq, page_size, &cap) || max_seq_len > cap)
        return fail(SDPA_ERR_INVALID_ARGUMENT,
                    "max_seq_len (%lld) exceeds the page table capacity max_pages_per_seq * "
                    "page_size",
                    (long long)max_seq_len);
    const int64_t es = elem_size(dtype);
    const int64_t nq = numel4(total_q, Hq, D, 1), nc = numel4(pages, page_size, Hkv, D);
    const int64_t no = numel4(total_q, Hq, Dv, 1), nvc = numel4(pages, page_size, Hkv, Dv);
    const int64_t nt = numel4(num_seqs, max_pages_per_seq, 1, 1);
    int64_t qbytes = 0, cbytes = 0, obytes = 0, vcbytes = 0;
    if (nq < 0 || nc < 0 || no < 0 || nvc < 0 || nt < 0 || !mul_ok(nq, es, &qbytes) ||
        !mul_ok(nc, es, &cbytes) || !mul_ok(no, es, &obytes) || !mul_ok(nvc, es, &vcbytes))
        return fail(SDPA_ERR_INVALID_ARGUMENT, "tensor byte size overflows int64");
    const size_t need = sdpa_paged_backward_workspace_size(num_seqs, Hq, Hkv, max_seq_len, D, Dv, dtype);
    if (need == 0) return fail(SDPA_ERR_INVALID_ARGUMENT, "workspace size overflows");
    if (!workspace || workspace_bytes < need)
        return fail(SDPA_ERR_WORKSPACE, "paged backward needs a workspace of %zu bytes (got %zu)",
                    need, workspace ? workspace_bytes : (size_t)0);
    // Outputs and the workspace overlap no input and each other.
    struct Span {
        const void* p;
        int64_t n;
    };
    const Span ins[] = {{q, qbytes},         {k_cache, cbytes},         {v_cache, vcbytes},
                        {out, obytes},       {dout, obytes},            {lse, total_q * Hq * 4},
                        {block_tables, nt * 4}, {seq_lens, num_seqs * 4}, {cu_seqlens_q, (num_seqs + 1) * 4}};
    const Span outs[] = {{dq, qbytes}, {dk_cache, cbytes}, {dv_cache, vcbytes}, {workspace, (int64_t)need}};
    for (const Span& o : outs) {
        for (const Span& i : ins)
            if (overlap(o.p, o.n, i.p, i.n))
                return fail(SDPA_ERR_INVALID_ARGUMENT, "an output or the workspace overlaps an input");
        for (const Span& o2 : outs)
            if (&o2 != &o && overlap(o.p, o.n, o2.p, o2.n))
                return fail(SDPA_ERR_INVALID_ARGUMENT, "outputs overlap each other or the workspace");
    }
    if (dtype == SDPA_F32 && (Dv != D || !head_dim_ok(D, dtype)))
        return fail(SDPA_ERR_UNSUPPORTED,
                    "head dims D=%lld Dv=%lld not supported by the fp32 paged backward (Dv = D, a "
                    "multiple of 4 up to 128)",
                    (long long)D, (long long)Dv);
    if (D > 512 || Dv > 512)
        return fail(SDPA_ERR_UNSUPPORTED,
                    "head dims D=%lld Dv=%lld not supported by the paged backward (any width up to 512)",
                    (long long)D, (long long)Dv);
    const int64_t W = dtype == SDPA_F32 ? D : paged_backward_width(D, Dv);
    if (page_size % 16 != 0)
        return fail(SDPA_ERR_UNSUPPORTED, "page_size=%lld is not a multiple of 16",
                    (long long)page_size);
    // The copies launch one thread per element (per 16-byte chunk when D =
    // Dv = W): a launch's thread count must fit 32 bits.
    const int64_t row_elems = numel4(num_seqs, Hq, max_seq_len, W);
    const int64_t kv_elems = numel4(num_seqs, Hkv, max_seq_len, W);
    const int64_t cache_elems = numel4(pages, page_size, Hkv, D > Dv ? D : Dv);
    const int64_t qblocks = ((max_seq_len + 127) / 128) * num_seqs * Hq;
    constexpr int64_t kMaxThreads = (int64_t)UINT32_MAX - 256;
    if (total_q > INT_MAX || Hq > INT_MAX || pages > INT_MAX || num_seqs > INT_MAX ||
        max_pages_per_seq > INT_MAX || max_seq_len > INT_MAX || row_elems < 0 ||
        row_elems > kMaxThreads || kv_elems < 0 || kv_elems > kMaxThreads || cache_elems < 0 ||
        cache_elems > kMaxThreads || nq > kMaxThreads || qblocks > INT_MAX / 256)
        return fail(SDPA_ERR_UNSUPPORTED, "a size exceeds the kernels' 32-bit index range");

    const size_t rowsz = (size_t)numel4(num_seqs, Hq, max_seq_len, W) * es;
    const size_t kvsz = (size_t)numel4(num_seqs, Hkv, max_seq_len, W) * es;
    char* w = static_cast<char*>(workspace);
    auto take = [&](size_t bytes) {
        char* p = w;
        w += round_up(bytes);
        return p;
    };
    sdpa::PagedBackwardArgs a;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.out = out;
    a.dout = dout;
    a.lse = lse;
    a.dq = dq;
    a.dk_cache = dk_cache;
    a.dv_cache = dv_cache;
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.cu_seqlens_q = cu_seqlens_q;
    a.total_q = (int)total_q;
    a.Hq = (int)Hq;
    a.Hkv = (int)Hkv;
    a.D = (int)D;
    a.Dv = (int)Dv;
    a.W = (int)W;
    a.num_seqs = (int)num_seqs;
    a.max_pages = (int)max_pages_per_seq;
    a.pages = (int)pages;
    a.page_size = (int)page_size;
    a.L = (int)max_seq_len;
    a.scale = scale;
    a.causal = causal != 0;
    a.qd = take(rowsz);
    a.dod = take(rowsz);
    a.od = take(rowsz);
    a.dqd = take(rowsz);
    a.kd = take(kvsz);
    a.vd = take(kvsz);
    a.dkd = take(kvsz);
    a.dvd = take(kvsz);
    a.lsed = reinterpret_cast<float*>(take((size_t)numel4(num_seqs, Hq, max_seq_len, 4)));
    a.stats = reinterpret_cast<float*>(w);
    (void)hipGetLastError();
    const hipStream_t s = static_cast<hipStream_t>(stream);
    return hip_status(dtype == SDPA_F32 ? sdpa::launch_paged_backward_f32(a, s)
                                        : sdpa::launch_paged_backward_16bit(a, dtype == SDPA_F16, s),
                      "sdpa_paged_backward launch");
}

}  // extern "C"
