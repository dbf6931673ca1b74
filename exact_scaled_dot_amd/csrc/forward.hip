// Prefill / full forward kernels: O = softmax(Q K^T * scale + mask) V with the
// score matrix kept on chip (HOF Flash Attention essay, section 4: a tiled
// exact kernel gives the dense kernel's result without holding the n x n
// scores in HBM; the mask and last-axis softmax follow the tensai autograd
// guide, section "Attention の組み立て").
//
// Work decomposition (both dtypes): one workgroup of 4 waves owns 128 query
// rows of one (batch, query head); each wave owns 32 rows.  The kernel walks
// the key axis in tiles of 64 keys.  Each tile of K and V is staged through
// LDS, shared by the 4 waves, and the wave computes the transposed score tile
// S^T = K Q^T with MFMA so that every lane holds the scores of ONE query
// (lanes l and l^32 share a query and split its keys).  Row statistics then
// need a single cross-lane exchange per tile, and the softmax weights already
// sit in the B-operand layout of the second product O^T += V^T P^T.
//
// Online softmax: running max m (raw score units), lane-partial running sum,
// and the output accumulator rescaled by exp2((m_old - m_new) * scale*log2e)
// whenever the max moves.  Keys past a row's limit (causal, key padding, Sk)
// get -inf and hence weight exactly 0; tiles past the workgroup's last
// visible key are never loaded.
#include "device_common.hpp"
#include "launch.hpp"

namespace sdpa {
namespace {

constexpr int kBr = 128;       // query rows per workgroup
constexpr int kBc = 64;        // keys per tile
constexpr int kThreads = 256;  // 4 waves of 64

// LDS row that holds tile key j in the bf16 K tile: bits 2 and 3 of j are
// swapped inside each group of 32 keys.  With this order the 32x32 score
// accumulator register r of lane half h holds key 16*(r/8) + 8*h + r%8, so
// the 8 weights a lane contributes to one 16-key slice of P V are 8
// consecutive keys, and the matching V^T operand is one 16-byte LDS read.
__device__ __forceinline__ int k_lds_row(int j) {
    return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
}

struct TileInfo {
    int b, h, gk, q0;
};

// Workgroup -> (batch, head, query block).  Consecutive workgroups take
// consecutive (batch, head) pairs of one query block: workgroups are dealt to
// the 8 XCDs round-robin, so as long as B*Hq is a multiple of 8 every
// workgroup of a given head lands on the same XCD and its K/V stays in that
// XCD's L2.  With a causal mask the longest query blocks come first so the
// short ones fill the tail.
__device__ __forceinline__ TileInfo decode_tile(const ForwardArgs& a) {
    const int nqb = (a.Sq + kBr - 1) / kBr;
    const int BH = a.B * a.Hq;
    const int bh = blockIdx.x % BH;
    int qb = blockIdx.x / BH;
    if (a.causal) qb = nqb - 1 - qb;
    TileInfo t;
    t.b = bh / a.Hq;
    t.h = bh % a.Hq;
    t.gk = t.h / (a.Hq / a.Hkv);
    t.q0 = qb * kBr;
    return t;
}

// Number of keys this workgroup must visit and the per-batch key limit.
__device__ __forceinline__ void key_extent(const ForwardArgs& a, int b, int q0, int& kv_lim,
                                           int& kv_end) {
    kv_lim = a.Sk;
    if (a.padded) kv_lim = min(kv_lim, a.key_lens[b]);
    kv_end = kv_lim;
    if (a.causal) kv_end = min(kv_end, q0 + kBr);
}

// ---------------------------------------------------------------------------
// bf16 inputs, bf16 MFMA (v_mfma_f32_32x32x16_bf16), fp32 accumulation.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads, 2) void forward_bf16_kernel(ForwardArgs a) {
    constexpr int KS = D + 8;    // K row stride in LDS (bf16), 16 B of padding
    constexpr int VS = kBc + 8;  // V^T row stride in LDS (bf16)
    __shared__ __attribute__((aligned(16))) uint16_t ks[kBc * KS];
    __shared__ __attribute__((aligned(16))) uint16_t vt[D * VS];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hg = lane >> 5;  // which half of the wave

    const TileInfo ti = decode_tile(a);
    const int64_t bh = (int64_t)ti.b * a.Hq + ti.h;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + bh * a.Sq * D;
    const int64_t kvh = ((int64_t)ti.b * a.Hkv + ti.gk) * a.Sk * D;
    const uint16_t* kp = static_cast<const uint16_t*>(a.k) + kvh;
    const uint16_t* vp = static_cast<const uint16_t*>(a.v) + kvh;
    uint16_t* op = static_cast<uint16_t*>(a.out) + bh * a.Sq * D;

    const int qw = ti.q0 + wave * 32;  // first query row of this wave
    const int qi = qw + l32;           // this lane's query row
    int kv_lim, kv_end;
    key_extent(a, ti.b, ti.q0, kv_lim, kv_end);
    const int ntiles = kv_end > 0 ? (kv_end + kBc - 1) / kBc : 0;

    // Q fragment for the B operand of S^T = K Q^T: lane holds Q[qi][16t + 8hg .. +7].
    bf16x8 qr[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (qi < a.Sq) w = ldg128(qp + (int64_t)qi * D + 16 * t + 8 * hg);
        qr[t] = as_bf16x8(w);
    }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
    float m_run = -INFINITY;  // running max of the raw scores of row qi
    float l_run = 0.f;        // this lane's share of the running denominator
    const float c = a.scale * kLog2e;

    for (int jt = 0; jt < ntiles; ++jt) {
        const int j0 = jt * kBc;
        __syncthreads();  // previous tile fully consumed
        // K tile, row-major, rows permuted by k_lds_row; keys >= Sk read as 0.
#pragma unroll
        for (int cidx = tid; cidx < kBc * (D / 8); cidx += kThreads) {
            const int row = cidx / (D / 8), cc = cidx % (D / 8);
            const int key = j0 + row;
            u32x4 w = {0u, 0u, 0u, 0u};
            if (key < a.Sk) w = ldg128(kp + (int64_t)key * D + cc * 8);
            *reinterpret_cast<u32x4*>(ks + k_lds_row(row) * KS + cc * 8) = w;
        }
        // V tile, stored transposed (V^T[d][key]): each item moves 4 keys x 8 dims.
#pragma unroll
        for (int it = tid; it < (kBc / 4) * (D / 8); it += kThreads) {
            const int dg = it % (D / 8), kg = it / (D / 8);
            u32x4 r[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int key = j0 + 4 * kg + rr;
                r[rr] = u32x4{0u, 0u, 0u, 0u};
                if (key < a.Sk) r[rr] = ldg128(vp + (int64_t)key * D + dg * 8);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {  // dword e holds dims 2e (low half) and 2e+1
                const u32x2 lo = {pack_lo16(r[0][e], r[1][e]), pack_lo16(r[2][e], r[3][e])};
                const u32x2 hi = {pack_hi16(r[0][e], r[1][e]), pack_hi16(r[2][e], r[3][e])};
                *reinterpret_cast<u32x2*>(vt + (dg * 8 + 2 * e) * VS + 4 * kg) = lo;
                *reinterpret_cast<u32x2*>(vt + (dg * 8 + 2 * e + 1) * VS + 4 * kg) = hi;
            }
        }
        __syncthreads();
        if (a.causal && j0 > qw + 31) continue;  // every key here is after every row of this wave

        // S^T tile: sacc[kb2] covers keys j0 + 32*kb2 .. +31 for query qi.
        f32x16 sacc[2];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
            sacc[kb2] = f32x16{};
            const uint16_t* krow = ks + (32 * kb2 + l32) * KS + 8 * hg;
#pragma unroll
            for (int t = 0; t < D / 16; ++t) {
                const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + 16 * t);
                sacc[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qr[t], sacc[kb2], 0, 0, 0);
            }
        }

        const bool need_mask = (a.causal && j0 + kBc - 1 > qw) || (j0 + kBc > kv_lim);
        if (need_mask) {
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = j0 + 32 * kb2 + 16 * (r >> 3) + 8 * hg + (r & 7);
                    const bool hide = key >= kv_lim || (a.causal && key > qi);
                    if (hide) sacc[kb2][r] = -INFINITY;
                }
        }

        float mx = sacc[0][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[0][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[1][r]);
        mx = fmaxf(mx, swap_half_wave(mx));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = fast_exp2((m_run - m_use) * c);
        const float neg = -m_use * c;
        m_run = m_new;

        float psum = 0.f;
        uint32_t pk[2][8];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = fast_exp2(fmaf(sacc[kb2][r], c, neg));
                const float p1 = fast_exp2(fmaf(sacc[kb2][r + 1], c, neg));
                psum += p0 + p1;
                pk[kb2][r >> 1] = pack_bf16x2(p0, p1);
            }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;

        // O^T += V^T P^T over four 16-key slices.
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int kb2 = kk >> 1, half = kk & 1;
            const u32x4 pw = {pk[kb2][4 * half], pk[kb2][4 * half + 1], pk[kb2][4 * half + 2],
                              pk[kb2][4 * half + 3]};
            const bf16x8 pb = as_bf16x8(pw);
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const bf16x8 vf = *reinterpret_cast<const bf16x8*>(
                    vt + (32 * db + l32) * VS + 32 * kb2 + 16 * half + 8 * hg);
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, oacc[db], 0, 0, 0);
            }
        }
    }

    // Epilogue: O = O_acc / l, rounded to bf16.  Register r of d-block db holds
    // dim 32*db + 8*(r/4) + 4*hg + r%4 of row qi.
    const float lt = l_run + swap_half_wave(l_run);
    const float inv = 1.f / lt;
    if (qi < a.Sq) {
        uint16_t* orow = op + (int64_t)qi * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const u32x2 w = {pack_bf16x2(oacc[db][4 * r4] * inv, oacc[db][4 * r4 + 1] * inv),
                                 pack_bf16x2(oacc[db][4 * r4 + 2] * inv, oacc[db][4 * r4 + 3] * inv)};
                *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * r4 + 4 * hg) = w;
            }
    }
}

// ---------------------------------------------------------------------------
// fp32 inputs, fp32 MFMA (v_mfma_f32_32x32x2_f32): every product exact in fp32.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads, 1) void forward_f32_kernel(ForwardArgs a) {
    constexpr int RS = D + 4;  // row stride in LDS (floats), 16 B of padding
    __shared__ __attribute__((aligned(16))) float ks[kBc * RS];
    __shared__ __attribute__((aligned(16))) float vs[kBc * RS];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hg = lane >> 5;

    const TileInfo ti = decode_tile(a);
    const int64_t bh = (int64_t)ti.b * a.Hq + ti.h;
    const float* qp = static_cast<const float*>(a.q) + bh * a.Sq * D;
    const int64_t kvh = ((int64_t)ti.b * a.Hkv + ti.gk) * a.Sk * D;
    const float* kp = static_cast<const float*>(a.k) + kvh;
    const float* vp = static_cast<const float*>(a.v) + kvh;
    float* op = static_cast<float*>(a.out) + bh * a.Sq * D;

    const int qw = ti.q0 + wave * 32;
    const int qi = qw + l32;
    int kv_lim, kv_end;
    key_extent(a, ti.b, ti.q0, kv_lim, kv_end);
    const int ntiles = kv_end > 0 ? (kv_end + kBc - 1) / kBc : 0;

    // Contraction slot (step t, lane half hg) <-> dim 8*(t/4) + 4*hg + t%4, so a
    // lane's operands for 4 consecutive steps are 4 consecutive floats.
    f32x4 qf[D / 8];
#pragma unroll
    for (int T = 0; T < D / 8; ++T) {
        qf[T] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (qi < a.Sq) qf[T] = *reinterpret_cast<const f32x4*>(qp + (int64_t)qi * D + 8 * T + 4 * hg);
    }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
    float m_run = -INFINITY;  // running max, log2-scaled units
    float l_run = 0.f;
    const float c = a.scale * kLog2e;

    for (int jt = 0; jt < ntiles; ++jt) {
        const int j0 = jt * kBc;
        __syncthreads();
#pragma unroll
        for (int cidx = tid; cidx < kBc * (D / 4); cidx += kThreads) {
            const int row = cidx / (D / 4), cc = cidx % (D / 4);
            const int key = j0 + row;
            f32x4 wk = {0.f, 0.f, 0.f, 0.f}, wv = {0.f, 0.f, 0.f, 0.f};
            if (key < a.Sk) {
                wk = *reinterpret_cast<const f32x4*>(kp + (int64_t)key * D + cc * 4);
                wv = *reinterpret_cast<const f32x4*>(vp + (int64_t)key * D + cc * 4);
            }
            *reinterpret_cast<f32x4*>(ks + row * RS + cc * 4) = wk;
            *reinterpret_cast<f32x4*>(vs + row * RS + cc * 4) = wv;
        }
        __syncthreads();
        if (a.causal && j0 > qw + 31) continue;

        // S^T: register r of sacc[kb2] holds key j0 + 32*kb2 + 8*(r/4) + 4*hg + r%4.
        f32x16 sacc[2];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
            sacc[kb2] = f32x16{};
            const float* krow = ks + (32 * kb2 + l32) * RS + 4 * hg;
#pragma unroll
            for (int T = 0; T < D / 8; ++T) {
                const f32x4 kv = *reinterpret_cast<const f32x4*>(krow + 8 * T);
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    sacc[kb2] = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[u], qf[T][u], sacc[kb2], 0, 0, 0);
            }
        }

        const bool need_mask = (a.causal && j0 + kBc - 1 > qw) || (j0 + kBc > kv_lim);
        if (need_mask) {
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = j0 + 32 * kb2 + 8 * (r >> 2) + 4 * hg + (r & 3);
                    const bool hide = key >= kv_lim || (a.causal && key > qi);
                    if (hide) sacc[kb2][r] = -INFINITY;
                }
        }
        // Work in log2-scaled units t = s * scale * log2(e): the row maximum
        // then gets weight exp2(t - m) = exp2(0) = 1 exactly.  __fmul_rn keeps
        // the product rounded on its own (no fusion into the later subtraction).
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kb2][r] = __fmul_rn(sacc[kb2][r], c);

        float mx = sacc[0][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[0][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[1][r]);
        mx = fmaxf(mx, swap_half_wave(mx));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        m_run = m_new;

        float psum = 0.f;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = fast_exp2(sacc[kb2][r] - m_use);
                sacc[kb2][r] = p;
                psum += p;
            }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;

        // O^T += V^T P^T: step u of block kb2 contracts the key held in register u.
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int key = 32 * kb2 + 8 * (u >> 2) + 4 * hg + (u & 3);
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const float vv = vs[key * RS + 32 * db + l32];
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv, sacc[kb2][u], oacc[db], 0, 0, 0);
                }
            }
    }

    const float lt = l_run + swap_half_wave(l_run);
    const float inv = 1.f / lt;
    if (qi < a.Sq) {
        float* orow = op + (int64_t)qi * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f32x4 w = {oacc[db][4 * r4] * inv, oacc[db][4 * r4 + 1] * inv,
                                 oacc[db][4 * r4 + 2] * inv, oacc[db][4 * r4 + 3] * inv};
                *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * r4 + 4 * hg) = w;
            }
    }
}

inline dim3 forward_grid(const ForwardArgs& a) {
    const int nqb = (a.Sq + kBr - 1) / kBr;
    return dim3((unsigned)(nqb * a.B * a.Hq));
}

}  // namespace

hipError_t launch_forward_bf16(const ForwardArgs& a, hipStream_t s) {
    if (a.D == 64)
        hipLaunchKernelGGL(forward_bf16_kernel<64>, forward_grid(a), dim3(kThreads), 0, s, a);
    else if (a.D == 128)
        hipLaunchKernelGGL(forward_bf16_kernel<128>, forward_grid(a), dim3(kThreads), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_forward_f32(const ForwardArgs& a, hipStream_t s) {
    if (a.D == 64)
        hipLaunchKernelGGL(forward_f32_kernel<64>, forward_grid(a), dim3(kThreads), 0, s, a);
    else if (a.D == 128)
        hipLaunchKernelGGL(forward_f32_kernel<128>, forward_grid(a), dim3(kThreads), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace sdpa
