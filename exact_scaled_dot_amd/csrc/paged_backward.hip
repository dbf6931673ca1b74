// Attention backward through a K/V page cache (ruDNN user guide, section 11:
// the paged plan's attention backward returns dq and the history gradients
// dk, dv, recomputing the probabilities from the forward's log-sum-exp).
//
// The packed prefill chunks of the paged forward are laid out, per sequence,
// at the absolute positions of their rows: row i of sequence s's chunk of
// n_s rows sits at position len_s - n_s + i (len_s = its cached keys, the
// chunk included).  Written into dense per-sequence tensors at those
// positions, with every other position a zero row of no visible key
// (lse = -inf), the paged attention of the chunk is the dense attention of
// the sequence under the causal flag and the key limit len_s, and its
// gradients are those of the dense backward: rows without a query have
// dO = 0 and probabilities 0, so they add nothing to dK or dV.  So the pass
// is
//   1. gathers: Q, dO, O, lse of the chunks into [S, Hq, L, W] at their
//      positions; K and V of each sequence's reachable keys through its page
//      table into [S, Hkv, L, W];
//   2. the ordered dense backward (causal and key padding with key_lens =
//      seq_lens), deterministic, at head dim W;
//   3. scatters: dQ back to the packed rows, dK and dV into the cache slots
//      their keys sit in, every other slot zeroed first.
// W is the larger of the key and value head dims D and Dv rounded up to a
// multiple of 8.  The gathers write zeros past D (Q, K) and past Dv (V, O,
// dO): the scores Q K^T, dO V^T and the row terms rowsum(dO * O) are those
// of the true widths, and the dims past D of dQ = dS K, dK = dS^T Q and past
// Dv of dV = P^T dO come out zero and are not scattered.  With D = Dv a
// multiple of 8 (W = D) the copies move 16-byte chunks; otherwise elements.
// The page logic lives only in the copies, which are HBM-bound; the
// backward's tiles are the tuned dense ones.
#include "device_common.hpp"
#include "launch.hpp"

namespace sdpa {
namespace {

constexpr int kPbThreads = 256;

// Rows of sequence s's chunk in the packed tensors ([r0, r1), clamped as the
// paged forward clamps them) and their first absolute position qoff.
struct ChunkRows {
    int r0, r1, kv_lim, qoff;
};
__device__ __forceinline__ ChunkRows chunk_rows(const PagedBackwardArgs& a, int s) {
    ChunkRows c;
    c.r0 = min(max(a.cu_seqlens_q[s], 0), a.total_q);
    c.r1 = min(max(a.cu_seqlens_q[s + 1], c.r0), a.total_q);
    c.kv_lim = max(0, min(a.seq_lens[s], a.L));
    c.qoff = c.kv_lim - (c.r1 - c.r0);
    return c;
}

// Dense row (s, h, p) <- packed row of position p, or zeros and lse = -inf.
// One thread per 16-byte chunk.
__global__ __launch_bounds__(kPbThreads) void pb_gather_rows_kernel(PagedBackwardArgs a) {
    const int cpr = a.D / 8;
    const int64_t n = (int64_t)a.num_seqs * a.Hq * a.L * cpr;
    const int64_t idx = (int64_t)blockIdx.x * kPbThreads + threadIdx.x;
    if (idx >= n) return;
    const int c = (int)(idx % cpr);
    int64_t r = idx / cpr;
    const int pos = (int)(r % a.L);
    r /= a.L;
    const int h = (int)(r % a.Hq);
    const int s = (int)(r / a.Hq);
    const ChunkRows cr = chunk_rows(a, s);
    const int i = pos - cr.qoff;
    const bool live = pos < cr.kv_lim && i >= 0;
    const int64_t src = live ? (((int64_t)(cr.r0 + i) * a.Hq + h) * cpr + c) : 0;
    const int64_t dst = (((int64_t)s * a.Hq + h) * a.L + pos) * cpr + c;
    const u32x4 z = {0u, 0u, 0u, 0u};
    reinterpret_cast<u32x4*>(a.qd)[dst] = live ? reinterpret_cast<const u32x4*>(a.q)[src] : z;
    reinterpret_cast<u32x4*>(a.dod)[dst] = live ? reinterpret_cast<const u32x4*>(a.dout)[src] : z;
    reinterpret_cast<u32x4*>(a.od)[dst] = live ? reinterpret_cast<const u32x4*>(a.out)[src] : z;
    if (c == 0)
        a.lsed[((int64_t)s * a.Hq + h) * a.L + pos] =
            live ? a.lse[(int64_t)(cr.r0 + i) * a.Hq + h] : -INFINITY;
}

// Physical slot element (chunk c) of logical key j of sequence s, K/V head g;
// -1 when the key is past the sequence or its table entry is outside the cache.
__device__ __forceinline__ int64_t slot_chunk(const PagedBackwardArgs& a, int s, int g, int j, int c,
                                              int kv_lim) {
    if (j >= kv_lim) return -1;
    const int lp = j / a.page_size;
    const int pg = lp < a.max_pages ? a.block_tables[(int64_t)s * a.max_pages + lp] : -1;
    if (pg < 0 || pg >= a.pages) return -1;
    return (((int64_t)pg * a.page_size + j % a.page_size) * a.Hkv + g) * (a.D / 8) + c;
}

// Dense K, V [S, Hkv, L, D] <- the keys each sequence reaches (zeros past it).
__global__ __launch_bounds__(kPbThreads) void pb_gather_kv_kernel(PagedBackwardArgs a) {
    const int cpr = a.D / 8;
    const int64_t n = (int64_t)a.num_seqs * a.Hkv * a.L * cpr;
    const int64_t idx = (int64_t)blockIdx.x * kPbThreads + threadIdx.x;
    if (idx >= n) return;
    const int c = (int)(idx % cpr);
    int64_t r = idx / cpr;
    const int j = (int)(r % a.L);
    r /= a.L;
    const int g = (int)(r % a.Hkv);
    const int s = (int)(r / a.Hkv);
    const int kv_lim = max(0, min(a.seq_lens[s], a.L));
    const int64_t src = slot_chunk(a, s, g, j, c, kv_lim);
    const u32x4 z = {0u, 0u, 0u, 0u};
    reinterpret_cast<u32x4*>(a.kd)[idx] = src >= 0 ? reinterpret_cast<const u32x4*>(a.k_cache)[src] : z;
    reinterpret_cast<u32x4*>(a.vd)[idx] = src >= 0 ? reinterpret_cast<const u32x4*>(a.v_cache)[src] : z;
}

// Zero n 16-byte chunks of p and q (the cache gradients, before the scatter).
__global__ __launch_bounds__(kPbThreads) void pb_zero_kernel(u32x4* p, u32x4* q, int64_t n) {
    const int64_t idx = (int64_t)blockIdx.x * kPbThreads + threadIdx.x;
    if (idx >= n) return;
    const u32x4 z = {0u, 0u, 0u, 0u};
    p[idx] = z;
    q[idx] = z;
}

// Cache slots <- dK, dV of the keys each sequence reaches.
__global__ __launch_bounds__(kPbThreads) void pb_scatter_kv_kernel(PagedBackwardArgs a) {
    const int cpr = a.D / 8;
    const int64_t n = (int64_t)a.num_seqs * a.Hkv * a.L * cpr;
    const int64_t idx = (int64_t)blockIdx.x * kPbThreads + threadIdx.x;
    if (idx >= n) return;
    const int c = (int)(idx % cpr);
    int64_t r = idx / cpr;
    const int j = (int)(r % a.L);
    r /= a.L;
    const int g = (int)(r % a.Hkv);
    const int s = (int)(r / a.Hkv);
    const int kv_lim = max(0, min(a.seq_lens[s], a.L));
    const int64_t dst = slot_chunk(a, s, g, j, c, kv_lim);
    if (dst < 0) return;
    reinterpret_cast<u32x4*>(a.dk_cache)[dst] = reinterpret_cast<const u32x4*>(a.dkd)[idx];
    reinterpret_cast<u32x4*>(a.dv_cache)[dst] = reinterpret_cast<const u32x4*>(a.dvd)[idx];
}

// Packed dQ rows <- dense dQ at their positions (zeros for a row that no
// chunk places in [0, len_s)).  The row's sequence by binary search over
// cu_seqlens_q (non-decreasing by contract).
__global__ __launch_bounds__(kPbThreads) void pb_scatter_rows_kernel(PagedBackwardArgs a) {
    const int cpr = a.D / 8;
    const int64_t n = (int64_t)a.total_q * a.Hq * cpr;
    const int64_t idx = (int64_t)blockIdx.x * kPbThreads + threadIdx.x;
    if (idx >= n) return;
    const int c = (int)(idx % cpr);
    const int64_t r = idx / cpr;
    const int h = (int)(r % a.Hq);
    const int t = (int)(r / a.Hq);
    // last s with clamped r0(s) <= t
    int lo = 0, hi = a.num_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (min(max(a.cu_seqlens_q[mid], 0), a.total_q) <= t) lo = mid;
        else hi = mid - 1;
    }
    const ChunkRows cr = chunk_rows(a, lo);
    const int pos = cr.qoff + (t - cr.r0);
    const bool live = t >= cr.r0 && t < cr.r1 && pos >= 0 && pos < cr.kv_lim;
    const u32x4 z = {0u, 0u, 0u, 0u};
    reinterpret_cast<u32x4*>(a.dq)[idx] =
        live ? reinterpret_cast<const u32x4*>(a.dqd)[(((int64_t)lo * a.Hq + h) * a.L + pos) * cpr + c] : z;
}

// Element-wise forms (any D, Dv; rows W wide in the workspace), for 16-bit
// (E = uint16_t) or fp32 (E = float) elements.  One thread per element of a
// W-wide row; consecutive threads take consecutive elements.

template <class E>
__global__ __launch_bounds__(kPbThreads) void pb_gather_rows_elem_kernel(PagedBackwardArgs a) {
    const int64_t n = (int64_t)a.num_seqs * a.Hq * a.L * a.W;
    const int64_t idx = (int64_t)blockIdx.x * kPbThreads + threadIdx.x;
    if (idx >= n) return;
    const int e = (int)(idx % a.W);
    int64_t r = idx / a.W;
    const int pos = (int)(r % a.L);
    r /= a.L;
    const int h = (int)(r % a.Hq);
    const int s = (int)(r / a.Hq);
    const ChunkRows cr = chunk_rows(a, s);
    const int i = pos - cr.qoff;
    const bool live = pos < cr.kv_lim && i >= 0;
    const int64_t row = live ? (int64_t)(cr.r0 + i) * a.Hq + h : 0;
    const E* q = static_cast<const E*>(a.q);
    const E* dout = static_cast<const E*>(a.dout);
    const E* out = static_cast<const E*>(a.out);
    static_cast<E*>(a.qd)[idx] = live && e < a.D ? q[row * a.D + e] : E(0);
    static_cast<E*>(a.dod)[idx] = live && e < a.Dv ? dout[row * a.Dv + e] : E(0);
    static_cast<E*>(a.od)[idx] = live && e < a.Dv ? out[row * a.Dv + e] : E(0);
    if (e == 0) a.lsed[r * a.L + pos] = live ? a.lse[row] : -INFINITY;
}

// Physical slot (page row) of logical key j of sequence s, K/V head g; -1
// when the key is past the sequence or its table entry is outside the cache.
__device__ __forceinline__ int64_t slot_row(const PagedBackwardArgs& a, int s, int g, int j, int kv_lim) {
    if (j >= kv_lim) return -1;
    const int lp = j / a.page_size;
    const int pg = lp < a.max_pages ? a.block_tables[(int64_t)s * a.max_pages + lp] : -1;
    if (pg < 0 || pg >= a.pages) return -1;
    return ((int64_t)pg * a.page_size + j % a.page_size) * a.Hkv + g;
}

template <class E>
__global__ __launch_bounds__(kPbThreads) void pb_gather_kv_elem_kernel(PagedBackwardArgs a) {
    const int64_t n = (int64_t)a.num_seqs * a.Hkv * a.L * a.W;
    const int64_t idx = (int64_t)blockIdx.x * kPbThreads + threadIdx.x;
    if (idx >= n) return;
    const int e = (int)(idx % a.W);
    int64_t r = idx / a.W;
    const int j = (int)(r % a.L);
    r /= a.L;
    const int g = (int)(r % a.Hkv);
    const int s = (int)(r / a.Hkv);
    const int kv_lim = max(0, min(a.seq_lens[s], a.L));
    const int64_t slot = slot_row(a, s, g, j, kv_lim);
    const E* kc = static_cast<const E*>(a.k_cache);
    const E* vc = static_cast<const E*>(a.v_cache);
    static_cast<E*>(a.kd)[idx] = slot >= 0 && e < a.D ? kc[slot * a.D + e] : E(0);
    static_cast<E*>(a.vd)[idx] = slot >= 0 && e < a.Dv ? vc[slot * a.Dv + e] : E(0);
}

// Zero n elements of p.
template <class E>
__global__ __launch_bounds__(kPbThreads) void pb_zero_elem_kernel(E* p, int64_t n) {
    const int64_t idx = (int64_t)blockIdx.x * kPbThreads + threadIdx.x;
    if (idx < n) p[idx] = E(0);
}

template <class E>
__global__ __launch_bounds__(kPbThreads) void pb_scatter_kv_elem_kernel(PagedBackwardArgs a) {
    const int64_t n = (int64_t)a.num_seqs * a.Hkv * a.L * a.W;
    const int64_t idx = (int64_t)blockIdx.x * kPbThreads + threadIdx.x;
    if (idx >= n) return;
    const int e = (int)(idx % a.W);
    int64_t r = idx / a.W;
    const int j = (int)(r % a.L);
    r /= a.L;
    const int g = (int)(r % a.Hkv);
    const int s = (int)(r / a.Hkv);
    const int kv_lim = max(0, min(a.seq_lens[s], a.L));
    const int64_t slot = slot_row(a, s, g, j, kv_lim);
    if (slot < 0) return;
    if (e < a.D) static_cast<E*>(a.dk_cache)[slot * a.D + e] = static_cast<const E*>(a.dkd)[idx];
    if (e < a.Dv) static_cast<E*>(a.dv_cache)[slot * a.Dv + e] = static_cast<const E*>(a.dvd)[idx];
}

template <class E>
__global__ __launch_bounds__(kPbThreads) void pb_scatter_rows_elem_kernel(PagedBackwardArgs a) {
    const int64_t n = (int64_t)a.total_q * a.Hq * a.D;
    const int64_t idx = (int64_t)blockIdx.x * kPbThreads + threadIdx.x;
    if (idx >= n) return;
    const int e = (int)(idx % a.D);
    const int64_t r = idx / a.D;
    const int h = (int)(r % a.Hq);
    const int t = (int)(r / a.Hq);
    int lo = 0, hi = a.num_seqs - 1;  // last s with clamped r0(s) <= t
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (min(max(a.cu_seqlens_q[mid], 0), a.total_q) <= t) lo = mid;
        else hi = mid - 1;
    }
    const ChunkRows cr = chunk_rows(a, lo);
    const int pos = cr.qoff + (t - cr.r0);
    const bool live = t >= cr.r0 && t < cr.r1 && pos >= 0 && pos < cr.kv_lim;
    static_cast<E*>(a.dq)[idx] =
        live ? static_cast<const E*>(a.dqd)[(((int64_t)lo * a.Hq + h) * a.L + pos) * a.W + e] : E(0);
}

dim3 grid_of(int64_t n) { return dim3((unsigned)((n + kPbThreads - 1) / kPbThreads)); }

}  // namespace

hipError_t launch_paged_backward_16bit(const PagedBackwardArgs& a, bool f16, hipStream_t s) {
    if (a.D < 1 || a.Dv < 1 || a.W % 8 != 0 || a.W < a.D || a.W < a.Dv || a.W > 512) return hipErrorInvalidValue;
    // 16-byte chunks when every row is W = D = Dv wide
    const bool chunks = a.D == a.W && a.Dv == a.W;
    const int64_t cpr = a.W / 8;
    const int64_t rows = (int64_t)a.num_seqs * a.Hq * a.L * cpr;
    const int64_t kv = (int64_t)a.num_seqs * a.Hkv * a.L * cpr;
    const int64_t cache = (int64_t)a.pages * a.page_size * a.Hkv * cpr;
    if (chunks) {
        hipLaunchKernelGGL(pb_gather_rows_kernel, grid_of(rows), dim3(kPbThreads), 0, s, a);
        hipLaunchKernelGGL(pb_gather_kv_kernel, grid_of(kv), dim3(kPbThreads), 0, s, a);
    } else {
        hipLaunchKernelGGL(pb_gather_rows_elem_kernel<uint16_t>, grid_of(rows * 8), dim3(kPbThreads), 0, s, a);
        hipLaunchKernelGGL(pb_gather_kv_elem_kernel<uint16_t>, grid_of(kv * 8), dim3(kPbThreads), 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    BackwardArgs b;
    b.q = a.qd;
    b.k = a.kd;
    b.v = a.vd;
    b.out = a.od;
    b.dout = a.dod;
    b.lse = a.lsed;
    b.key_lens = a.seq_lens;
    b.dq = a.dqd;
    b.dk = a.dkd;
    b.dv = a.dvd;
    b.delta = a.stats;
    b.B = a.num_seqs;
    b.Hq = a.Hq;
    b.Hkv = a.Hkv;
    b.Sq = a.L;
    b.Sk = a.L;
    b.D = a.W;
    b.scale = a.scale;
    b.causal = a.causal;
    b.padded = true;
    e = launch_backward_16bit(b, f16, s);
    if (e != hipSuccess) return e;
    if (chunks) {
        hipLaunchKernelGGL(pb_zero_kernel, grid_of(cache), dim3(kPbThreads), 0, s,
                           static_cast<u32x4*>(a.dk_cache), static_cast<u32x4*>(a.dv_cache), cache);
        hipLaunchKernelGGL(pb_scatter_kv_kernel, grid_of(kv), dim3(kPbThreads), 0, s, a);
        hipLaunchKernelGGL(pb_scatter_rows_kernel, grid_of((int64_t)a.total_q * a.Hq * cpr), dim3(kPbThreads),
                           0, s, a);
    } else {
        const int64_t slots = (int64_t)a.pages * a.page_size * a.Hkv;
        hipLaunchKernelGGL(pb_zero_elem_kernel<uint16_t>, grid_of(slots * a.D), dim3(kPbThreads), 0, s,
                           static_cast<uint16_t*>(a.dk_cache), slots * a.D);
        hipLaunchKernelGGL(pb_zero_elem_kernel<uint16_t>, grid_of(slots * a.Dv), dim3(kPbThreads), 0, s,
                           static_cast<uint16_t*>(a.dv_cache), slots * a.Dv);
        hipLaunchKernelGGL(pb_scatter_kv_elem_kernel<uint16_t>, grid_of(kv * 8), dim3(kPbThreads), 0, s, a);
        hipLaunchKernelGGL(pb_scatter_rows_elem_kernel<uint16_t>, grid_of((int64_t)a.total_q * a.Hq * a.D),
                           dim3(kPbThreads), 0, s, a);
    }
    return hipGetLastError();
}

// fp32: the same three stages with fp32 copies (W = D = Dv) and the fp32
// dense backward.
hipError_t launch_paged_backward_f32(const PagedBackwardArgs& a, hipStream_t s) {
    if (a.D != a.Dv || a.W != a.D || a.D % 4 != 0 || a.D < 4 || a.D > 128) return hipErrorInvalidValue;
    const int64_t rows = (int64_t)a.num_seqs * a.Hq * a.L * a.W;
    const int64_t kv = (int64_t)a.num_seqs * a.Hkv * a.L * a.W;
    const int64_t slots = (int64_t)a.pages * a.page_size * a.Hkv;
    hipLaunchKernelGGL(pb_gather_rows_elem_kernel<float>, grid_of(rows), dim3(kPbThreads), 0, s, a);
    hipLaunchKernelGGL(pb_gather_kv_elem_kernel<float>, grid_of(kv), dim3(kPbThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    BackwardArgs b;
    b.q = a.qd;
    b.k = a.kd;
    b.v = a.vd;
    b.out = a.od;
    b.dout = a.dod;
    b.lse = a.lsed;
    b.key_lens = a.seq_lens;
    b.dq = a.dqd;
    b.dk = a.dkd;
    b.dv = a.dvd;
    b.delta = a.stats;
    b.B = a.num_seqs;
    b.Hq = a.Hq;
    b.Hkv = a.Hkv;
    b.Sq = a.L;
    b.Sk = a.L;
    b.D = a.W;
    b.scale = a.scale;
    b.causal = a.causal;
    b.padded = true;
    e = launch_backward_f32(b, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(pb_zero_elem_kernel<float>, grid_of(slots * a.D), dim3(kPbThreads), 0, s,
                       static_cast<float*>(a.dk_cache), slots * a.D);
    hipLaunchKernelGGL(pb_zero_elem_kernel<float>, grid_of(slots * a.D), dim3(kPbThreads), 0, s,
                       static_cast<float*>(a.dv_cache), slots * a.D);
    hipLaunchKernelGGL(pb_scatter_kv_elem_kernel<float>, grid_of(kv), dim3(kPbThreads), 0, s, a);
    hipLaunchKernelGGL(pb_scatter_rows_elem_kernel<float>, grid_of((int64_t)a.total_q * a.Hq * a.D),
                       dim3(kPbThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace sdpa
