// Single-query decode with split-KV and a log-sum-exp merge (ruDNN user guide,
// section 9: the history is split into 2..=32 pieces whose partial statistics
// and merge are kept in FP32).  The split pass is memory bound: every byte of
// K and V of a (batch, K/V head) is read once for all the query heads that
// share it.
//
// Split pass: see decode_split_bf16_kernel.  Every byte of K and V of a
// (batch, K/V head) is read once for up to 16 query heads that share it.
//
// Merge pass: one thread per (batch, query head, dim) combines the splits:
// O = sum_s exp(lse_s - M) O_s / sum_s exp(lse_s - M), M = max_s lse_s.
#include "device_common.hpp"
#include "launch.hpp"

namespace sdpa {
namespace {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = 4;
constexpr int kQ = 16;         // query heads per workgroup (the 16 MFMA columns)
constexpr int kStep = 32;      // keys per wave step
constexpr float kTau = 8.0f;   // lazy-rescale threshold, log2 units

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ u32x2 lds_read_tr16x4(const uint16_t* p) {
    lds_i16x4* lp = (lds_i16x4*)((__attribute__((address_space(3))) char*)p);
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(lp));
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint16_t* lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (lds_void*)((__attribute__((address_space(3))) char*)lds), 16, voff, 0, 0, 0);
}

template <int D>
struct DecGeo {
    static constexpr int CPR = D / 8;                 // 16-byte chunks per row
    static constexpr int RPW = 256 / (2 * D);         // rows per 256-byte bank window
    static constexpr int STAGE = kStep * D;           // bf16 elements of one V step
    static constexpr int DMA = STAGE * 2 / 1024;      // 1-KB DMA loads per step
    static constexpr int KSTEPS = D / 32;             // MFMA contraction steps
    // V chunk swizzle: the 8 rows x 32 B one 32-lane transposed read touches
    // fall on 16 distinct 16-byte bank groups.
    __device__ static int fv(int r) { return 2 * ((r / RPW) % (8 / RPW)); }
};

// Split pass.  Workgroup = (batch, K/V head, block of <= 16 query heads, split);
// each wave walks 32-key steps (wave w takes steps w, w+4, ...) with no
// workgroup barrier until the final merge:
//   S^T[32 keys x 16 queries] = K Q^T      two v_mfma_f32_16x16x32_bf16 chains
//   O^T[D x 16 queries]      += V^T P^T    D/16 v_mfma_f32_16x16x32_bf16
// K goes straight from HBM into the A-operand registers (one step ahead);
// V goes HBM -> LDS by buffer-load DMA into a per-wave 2-stage ring and comes
// back transposed with ds_read_b64_tr_b16.  Lane l owns query column l % 16;
// its 8 scores per step are keys 4*(l/16) + i and 16 + 4*(l/16) + i, which are
// exactly the 8 contraction slots it feeds to the P.V product.
template <int D>
__global__ __launch_bounds__(kDecThreads, 2) void decode_split_bf16_kernel(DecodeArgs a) {
    using L = DecGeo<D>;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[kDecWaves * 2 * L::STAGE];

    const int G = a.Hq / a.Hkv;
    const int nqc = (G + kQ - 1) / kQ;
    int idx = blockIdx.x;
    const int split = idx % a.splits;
    idx /= a.splits;
    const int qc = idx % nqc;
    idx /= nqc;
    const int gk = idx % a.Hkv;
    const int b = idx / a.Hkv;
    const int h0 = gk * G + qc * kQ;
    const int nh = min(kQ, G - qc * kQ);

    int len = a.Sk;
    if (a.key_lens) len = min(len, a.key_lens[b]);
    const int chunk = (a.Sk + a.splits - 1) / a.splits;
    const int lo = split * chunk;
    const int hi = min(lo + chunk, len);
    const int nsteps = hi > lo ? (hi - lo + kStep - 1) / kStep : 0;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int col = lane & 15;   // query column (and key row within a 16-key tile)
    const int grp = lane >> 4;   // lane group: contraction slots 8*grp .. 8*grp+7

    const int64_t kvh = ((int64_t)b * a.Hkv + gk) * a.Sk * D;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(static_cast<const uint16_t*>(a.k) + kvh,
                                                 (uint32_t)a.Sk * D * 2);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(static_cast<const uint16_t*>(a.v) + kvh,
                                                 (uint32_t)a.Sk * D * 2);

    // Contraction slot (kstep t, group g, element e) <-> dim (D/4)*g + 8t + e, so a
    // lane's K operand over all ksteps is (D/4) contiguous dims of one key row.
    bf16x8 qb[L::KSTEPS];
    {
        const __amdgpu_buffer_rsrc_t qrs = make_rsrc(
            static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.Hq + h0) * D, (uint32_t)nh * D * 2);
#pragma unroll
        for (int t = 0; t < L::KSTEPS; ++t)
            qb[t] = as_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(
                qrs, (col * D + (D / 4) * grp + 8 * t) * 2, 0, 0));  // columns >= nh read 0
    }
    const float c = a.scale * kLog2e;
    const float tau = kTau / c;

    // Per-lane byte offsets (relative to the step's first key).
    uint32_t koff[2][L::KSTEPS];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile)
#pragma unroll
        for (int t = 0; t < L::KSTEPS; ++t)
            koff[tile][t] = ((16 * tile + col) * D + (D / 4) * grp + 8 * t) * 2;
    uint32_t voff[L::DMA];
#pragma unroll
    for (int i = 0; i < L::DMA; ++i) {
        const int p = 64 * i + lane, row = p / L::CPR, pc = p % L::CPR;
        voff[i] = row * D * 2 + (pc ^ L::fv(row)) * 16;
    }
    // Transposed V read: lane j of group grp points at row k0 + j/4, dims d0 + 4*(j%4),
    // k0 = 4*grp (+16), d0 = 16*dt; it receives V[k0..k0+3][d0 + col].
    const int tr_row = 4 * grp + (col >> 2);
    int vrd[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
        const int e = 16 * dt + 4 * (col & 3);
        vrd[dt] = tr_row * D + (((e >> 3) ^ L::fv(tr_row)) * 8) + (e & 7);
    }

    uint16_t* ring = smem + wave * 2 * L::STAGE;
    auto issue = [&](int st, int stage, u32x4 (&kr)[2][L::KSTEPS]) {
        const uint32_t base = (uint32_t)(lo + kStep * st) * D * 2;
#pragma unroll
        for (int i = 0; i < L::DMA; ++i) dma16(vrs, ring + stage * L::STAGE + 512 * i, base + voff[i]);
#pragma unroll
        for (int tile = 0; tile < 2; ++tile)
#pragma unroll
            for (int t = 0; t < L::KSTEPS; ++t)
                kr[tile][t] = __builtin_amdgcn_raw_buffer_load_b128(krs, base + koff[tile][t], 0, 0);
    };

    f32x4 oacc[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    u32x4 kcur[2][L::KSTEPS], knext[2][L::KSTEPS];
    if (wave < nsteps) issue(wave, 0, kcur);
    int n = 0;
    for (int st = wave; st < nsteps; st += kDecWaves, ++n) {
        const int stage = n & 1;
        const bool more = st + kDecWaves < nsteps;
        if (more) issue(st + kDecWaves, stage ^ 1, knext);
        // Everything but the loads just issued for the next step has landed.
        if (more)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(L::DMA + 2 * L::KSTEPS) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

        const int k0 = lo + kStep * st;
        f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int t = 0; t < L::KSTEPS; ++t)
#pragma unroll
            for (int tile = 0; tile < 2; ++tile)
                sacc[tile] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kcur[tile][t]), qb[t],
                                                                     sacc[tile], 0, 0, 0);
        if (k0 + kStep > hi) {
#pragma unroll
            for (int tile = 0; tile < 2; ++tile)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (k0 + 16 * tile + 4 * grp + i >= hi) sacc[tile][i] = -INFINITY;
        }
        float mx = fmaxf(fmaxf(fmaxf(sacc[0][0], sacc[0][1]), fmaxf(sacc[0][2], sacc[0][3])),
                         fmaxf(fmaxf(sacc[1][0], sacc[1][1]), fmaxf(sacc[1][2], sacc[1][3])));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));  // all four lanes of a column agree
        if (__any(mx > m_run + tau)) {
            const float m_new = fmaxf(m_run, mx);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = fast_exp2((m_run - m_use) * c);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) oacc[dt] *= alpha;
        }
        const float neg = -((m_run == -INFINITY) ? 0.f : m_run) * c;
        uint32_t pk[4];
#pragma unroll
        for (int tile = 0; tile < 2; ++tile)
#pragma unroll
            for (int i = 0; i < 4; i += 2)
                pk[2 * tile + (i >> 1)] = pack_bf16x2(fast_exp2(fmaf(sacc[tile][i], c, neg)),
                                                      fast_exp2(fmaf(sacc[tile][i + 1], c, neg)));
        {
            typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
            const bf16x2_t one = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
            float ps = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w)
                ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[w]), one, ps, false);
            l_run += ps;
        }
        const bf16x8 pb = as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]});
        const uint16_t* vs = ring + stage * L::STAGE;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            const u32x2 lo4 = lds_read_tr16x4(vs + vrd[dt]);
            const u32x2 hi4 = lds_read_tr16x4(vs + vrd[dt] + 16 * D);
            const bf16x8 vf = as_bf16x8(u32x4{lo4[0], lo4[1], hi4[0], hi4[1]});
            oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb, oacc[dt], 0, 0, 0);
        }
#pragma unroll
        for (int tile = 0; tile < 2; ++tile)
#pragma unroll
            for (int t = 0; t < L::KSTEPS; ++t) kcur[tile][t] = knext[tile][t];
    }

    // Column totals: the denominator is spread over the 4 lane groups.
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);

    // Merge the 4 waves through LDS (the ring is free now).
    __syncthreads();
    float* red_o = reinterpret_cast<float*>(smem);              // [wave][q][D]
    float* red_m = red_o + kDecWaves * kQ * D;                  // [wave][q]
    float* red_l = red_m + kDecWaves * kQ;                      // [wave][q]
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i)  // O^T register i of tile dt: dim 16*dt + 4*grp + i, column col
            red_o[(wave * kQ + col) * D + 16 * dt + 4 * grp + i] = oacc[dt][i];
    if (grp == 0) {
        red_m[wave * kQ + col] = m_run;
        red_l[wave * kQ + col] = l_run;
    }
    __syncthreads();
    for (int e = tid; e < nh * D; e += kDecThreads) {
        const int q = e / D, d = e % D;
        float M = -INFINITY;
#pragma unroll
        for (int wv = 0; wv < kDecWaves; ++wv) M = fmaxf(M, red_m[wv * kQ + q]);
        const int64_t prow = ((int64_t)b * a.Hq + h0 + q) * a.splits + split;
        if (M == -INFINITY) {  // no visible key in this split
            a.o_part[prow * D + d] = 0.f;
            if (d == 0) a.lse_part[prow] = -INFINITY;
            continue;
        }
        float Ls = 0.f, acc = 0.f;
#pragma unroll
        for (int wv = 0; wv < kDecWaves; ++wv) {
            const float mw = red_m[wv * kQ + q];
            const float w = (mw == -INFINITY) ? 0.f : fast_exp2((mw - M) * c);
            Ls = fmaf(w, red_l[wv * kQ + q], Ls);
            acc = fmaf(w, red_o[(wv * kQ + q) * D + d], acc);
        }
        a.o_part[prow * D + d] = acc / Ls;
        if (d == 0) a.lse_part[prow] = M * a.scale + __logf(Ls);
    }
}

template <int D>
__global__ __launch_bounds__(256) void decode_merge_bf16_kernel(DecodeArgs a) {
    constexpr int RPB = 256 / D;  // rows (batch, query head) per block
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / D;
    const int d = threadIdx.x % D;
    if (row >= (int64_t)a.B * a.Hq) return;
    const float* lse = a.lse_part + row * a.splits;
    const float* op = a.o_part + row * a.splits * D + d;
    float M = -INFINITY;
    for (int s = 0; s < a.splits; ++s) M = fmaxf(M, lse[s]);
    float den = 0.f, acc = 0.f;
    for (int s = 0; s < a.splits; ++s) {
        const float w = fast_exp2((lse[s] - M) * kLog2e);  // empty split: exp(-inf) = 0
        den += w;
        acc = fmaf(w, op[(int64_t)s * D], acc);
    }
    // Every split empty (no visible key): M = -inf, w = NaN, and the row is NaN.
    static_cast<uint16_t*>(a.out)[row * D + d] = (uint16_t)f32_to_bf16_bits(acc / den);
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s) {
    const int G = a.Hq / a.Hkv;
    const int nqc = (G + kQ - 1) / kQ;
    const dim3 grid((unsigned)((int64_t)a.B * a.Hkv * nqc * a.splits));
    const dim3 mgrid((unsigned)(((int64_t)a.B * a.Hq * a.D + 255) / 256));
    if (a.D == 64) {
        hipLaunchKernelGGL(decode_split_bf16_kernel<64>, grid, dim3(kDecThreads), 0, s, a);
        hipLaunchKernelGGL(decode_merge_bf16_kernel<64>, mgrid, dim3(256), 0, s, a);
    } else if (a.D == 128) {
        hipLaunchKernelGGL(decode_split_bf16_kernel<128>, grid, dim3(kDecThreads), 0, s, a);
        hipLaunchKernelGGL(decode_merge_bf16_kernel<128>, mgrid, dim3(256), 0, s, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace sdpa
