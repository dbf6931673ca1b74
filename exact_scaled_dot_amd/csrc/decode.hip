// Single-query decode with split-KV and a log-sum-exp merge (ruDNN user guide,
// section 9: the history is split into 2..=32 pieces whose partial statistics
// and merge are kept in FP32).  The split pass is memory bound: every byte of
// K and V of a (batch, K/V head) is read once for all the query heads that
// share it.
//
// Split pass: one workgroup per (batch, K/V head, block of up to 4 query
// heads of that group, split).  Each wave walks 16-key steps of the split.
// Scores come from one v_mfma_f32_16x16x32_bf16 per 32 dims: A = the (up to 4)
// query rows, each repeated 4 times to fill the 16 rows, B = K^T of 16 keys,
// so every lane receives the scores of all 4 queries for ONE key (lane % 16).
// Lane quarter l/16 owns a quarter of the head dimension and accumulates
// p * V for its key over those dims in fp32 on the vector ALU.  Each lane
// keeps its own running max / sum / output over the keys it saw; the max is
// moved only when a score exceeds it by more than 2^8 (the ratio O / l is
// unchanged by a stale max, so this is exact), which removes almost every
// rescale.  At the end the lane states are merged inside the wave (DPP row
// reductions) and across the 4 waves (LDS), and the normalised partial output
// and its natural-log log-sum-exp are written to the workspace.
//
// Merge pass: one thread per (batch, query head, dim) combines the splits:
// O = sum_s exp(lse_s - M) O_s / sum_s exp(lse_s - M), M = max_s lse_s.
#include "device_common.hpp"
#include "launch.hpp"

namespace sdpa {
namespace {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = 4;
constexpr int kQ = 4;          // query heads per workgroup
constexpr float kTau = 8.0f;   // lazy-rescale threshold, log2 units

__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, __shfl_xor(x, 1));
    x = fmaxf(x, __shfl_xor(x, 2));
    x = fmaxf(x, __shfl_xor(x, 4));
    x = fmaxf(x, __shfl_xor(x, 8));
    return x;
}
__device__ __forceinline__ float row16_sum(float x) {
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    x += __shfl_xor(x, 8);
    return x;
}

template <int D>
__global__ __launch_bounds__(kDecThreads, 1) void decode_split_bf16_kernel(DecodeArgs a) {
    constexpr int DQ = D / 4;       // dims owned by one lane quarter
    constexpr int KSTEPS = D / 32;  // MFMA steps per 16-key score tile
    __shared__ float red_m[kDecWaves][kQ];
    __shared__ float red_l[kDecWaves][kQ];
    __shared__ __attribute__((aligned(16))) float red_o[kDecWaves][kQ][D];

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
    const int nsteps = hi > lo ? (hi - lo + 15) / 16 : 0;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int kslot = lane & 15;
    const int quarter = lane >> 4;

    const uint16_t* qbase = static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.Hq + h0) * D;
    const int64_t kvh = ((int64_t)b * a.Hkv + gk) * a.Sk * D;
    const uint16_t* kp = static_cast<const uint16_t*>(a.k) + kvh + DQ * quarter;
    const uint16_t* vp = static_cast<const uint16_t*>(a.v) + kvh + DQ * quarter;

    // A operand: row kslot is query head h0 + kslot % 4 (rows repeat every 4);
    // contraction slot (step t, quarter, element e) <-> dim DQ*quarter + 8t + e.
    bf16x8 qa[KSTEPS];
    {
        const int qh = kslot & 3;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            u32x4 w = {0u, 0u, 0u, 0u};
            if (qh < nh) w = ldg128(qbase + (int64_t)qh * D + DQ * quarter + 8 * t);
            qa[t] = as_bf16x8(w);
        }
    }
    const float c = a.scale * kLog2e;

    float m_run[kQ], l_run[kQ], o[kQ][DQ];
#pragma unroll
    for (int i = 0; i < kQ; ++i) {
        m_run[i] = -INFINITY;
        l_run[i] = 0.f;
#pragma unroll
        for (int d = 0; d < DQ; ++d) o[i][d] = 0.f;
    }

    for (int st = wave; st < nsteps; st += kDecWaves) {
        const int key = lo + 16 * st + kslot;
        const bool valid = key < hi;
        u32x4 kw[KSTEPS], vw[DQ / 8];
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            kw[t] = u32x4{0u, 0u, 0u, 0u};
            if (valid) kw[t] = ldg128(kp + (int64_t)key * D + 8 * t);
        }
#pragma unroll
        for (int e = 0; e < DQ / 8; ++e) {
            vw[e] = u32x4{0u, 0u, 0u, 0u};
            if (valid) vw[e] = ldg128(vp + (int64_t)key * D + 8 * e);
        }
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t)
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[t], as_bf16x8(kw[t]), sacc, 0, 0, 0);

        float p[kQ];
#pragma unroll
        for (int i = 0; i < kQ; ++i) {
            const float s = sacc[i] * c;  // log2-scaled score of query i for this key
            if (valid && s > m_run[i] + kTau) {
                const float alpha = fast_exp2(m_run[i] - s);
                m_run[i] = s;
                l_run[i] *= alpha;
#pragma unroll
                for (int d = 0; d < DQ; ++d) o[i][d] *= alpha;
            }
            p[i] = valid ? fast_exp2(s - m_run[i]) : 0.f;
            l_run[i] += p[i];
        }
#pragma unroll
        for (int e = 0; e < DQ / 8; ++e)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float v0 = bf16_lo_to_f32(vw[e][w]);
                const float v1 = bf16_hi_to_f32(vw[e][w]);
#pragma unroll
                for (int i = 0; i < kQ; ++i) {
                    o[i][8 * e + 2 * w] = fmaf(p[i], v0, o[i][8 * e + 2 * w]);
                    o[i][8 * e + 2 * w + 1] = fmaf(p[i], v1, o[i][8 * e + 2 * w + 1]);
                }
            }
    }

    // Merge the 16 key slots of this wave (lanes of one 16-lane row).
#pragma unroll
    for (int i = 0; i < kQ; ++i) {
        const float M = row16_max(m_run[i]);
        const float w = (m_run[i] == -INFINITY) ? 0.f : fast_exp2(m_run[i] - M);
        l_run[i] = row16_sum(l_run[i] * w);
#pragma unroll
        for (int d = 0; d < DQ; ++d) o[i][d] = row16_sum(o[i][d] * w);
        m_run[i] = M;
    }
    if (kslot == 0) {
#pragma unroll
        for (int i = 0; i < kQ; ++i) {
#pragma unroll
            for (int d = 0; d < DQ; d += 4)
                *reinterpret_cast<f32x4*>(&red_o[wave][i][DQ * quarter + d]) =
                    f32x4{o[i][d], o[i][d + 1], o[i][d + 2], o[i][d + 3]};
            if (quarter == 0) {
                red_m[wave][i] = m_run[i];
                red_l[wave][i] = l_run[i];
            }
        }
    }
    __syncthreads();

    // Merge the 4 waves and write the normalised partial and its lse.
    for (int e = tid; e < kQ * D; e += kDecThreads) {
        const int i = e / D, d = e % D;
        if (i >= nh) continue;
        float M = -INFINITY;
#pragma unroll
        for (int wv = 0; wv < kDecWaves; ++wv) M = fmaxf(M, red_m[wv][i]);
        const int64_t prow = ((int64_t)b * a.Hq + h0 + i) * a.splits + split;
        if (M == -INFINITY) {  // no visible key in this split
            a.o_part[prow * D + d] = 0.f;
            if (d == 0) a.lse_part[prow] = -INFINITY;
            continue;
        }
        float L = 0.f, acc = 0.f;
#pragma unroll
        for (int wv = 0; wv < kDecWaves; ++wv) {
            const float w = (red_m[wv][i] == -INFINITY) ? 0.f : fast_exp2(red_m[wv][i] - M);
            L = fmaf(w, red_l[wv][i], L);
            acc = fmaf(w, red_o[wv][i][d], acc);
        }
        a.o_part[prow * D + d] = acc / L;
        if (d == 0) a.lse_part[prow] = (M + __log2f(L)) * kLn2;
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
