// Attention backward for fp32 inputs (ruDNN user guide section 9: the paged
// plan takes F32, F16 or BF16 and supports the first-order backward; section
// 11: dq, dk, dv with the probabilities recomputed from the forward's
// log-sum-exp, ordered reductions).  The derivatives are those of the 16-bit
// backward (tensai autograd guide, "Attention の組み立て"):
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - delta),  delta_i = sum_d dO_id O_id,
//   dQ = scale dS K,  dK = scale dS^T Q,
// with P_ij = exp(scale s_ij - lse_i), hidden keys at P = 0, and grouped K/V
// heads summing their query heads' contributions.  Everything stays fp32:
// the products run on v_mfma_f32_32x32x2_f32 (exact fp32 products, fp32
// sums), P and dS are never rounded to 16 bits.
//
// Three kernels, every sum in a fixed order (bitwise reproducible):
//   1. row statistics: (lse * log2 e, delta) per query row into the
//      workspace, the layout of the 16-bit backward's statistics;
//   2. dQ, query-parallel: a workgroup owns 128 rows of one (batch, query
//      head) (32 per wave) and walks its visible keys in tiles of 64;
//   3. dK and dV, key-parallel: a workgroup owns 128 keys of one (batch, K/V
//      head) (32 per wave) and walks the 64-query tiles of every query head
//      of the group.
// Tiles pass through LDS with plain loads and workgroup barriers, as in the
// fp32 forward.
//
// MFMA layout (32x32x2, fp32): contraction step t of a 32x32 product takes
// from lane half hg the value at slot 8*(t/4) + 4*hg + t%4 of the contracted
// axis, so a lane's operands for four consecutive steps are four consecutive
// floats; the accumulator holds column l%32 and row 8*(r/4) + 4*hg + r%4 in
// register r.  An accumulator whose rows run over the contracted axis of the
// next product is therefore already that product's B operand, register u
// being the value at row 8*(u/4) + 4*hg + u%4, and the matching A operand is
// one float per lane of the other tensor's row at that index.
#include "device_common.hpp"
#include "launch.hpp"

namespace sdpa {
namespace {

constexpr int kFbThreads = 256;  // 4 waves
constexpr int kFbRows = 128;     // rows a workgroup owns (queries, or keys)
constexpr int kFbTile = 64;      // rows of the streamed operand per step

__host__ __device__ __forceinline__ int64_t f_stats_stride(int Sq) { return (Sq + 1) & ~1; }

__device__ __forceinline__ int f_xcd_order(int total) {
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    const int nx = total >> 3, rem = total & 7;
    return xcd * nx + min(xcd, rem) + local;
}

// 1. (lse2, delta) per row: 32 lanes per row, 4 dims each (D <= 128).
__global__ __launch_bounds__(kFbThreads) void bwd_f32_stats_kernel(BackwardArgs a) {
    const int64_t row = (int64_t)blockIdx.x * (kFbThreads / 32) + (threadIdx.x >> 5);
    const int j = threadIdx.x & 31;
    const bool live = row < (int64_t)a.B * a.Hq * a.Sq;
    float part = 0.f;
    if (live && 4 * j < a.D) {
        const f32x4 o = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.out) + row * a.D + 4 * j);
        const f32x4 d = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.dout) + row * a.D + 4 * j);
        part = o[0] * d[0] + o[1] * d[1] + o[2] * d[2] + o[3] * d[3];
    }
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1) part += __shfl_xor(part, m);
    if (live && j == 0) {
        const int64_t bh = row / a.Sq, i = row % a.Sq;
        const float l = a.lse[row];
        float2* st = reinterpret_cast<float2*>(a.delta) + bh * f_stats_stride(a.Sq) + i;
        // a row with no visible key: +inf makes every recomputed probability 0
        *st = l == -INFINITY ? make_float2(INFINITY, 0.f) : make_float2(l * kLog2e, part);
    }
}

// Rows r0 .. r0+63 of a [rows, DR] fp32 tensor into an LDS tile [64][RS]
// (rows past `rows` and dims past DR as zeros).
template <int D>
__device__ __forceinline__ void f_load_tile(float* __restrict__ tile, const float* src, int r0, int rows, int DR,
                                            int tid) {
    constexpr int RS = D + 4;
#pragma unroll
    for (int c = tid; c < kFbTile * (D / 4); c += kFbThreads) {
        const int r = c / (D / 4), cc = c % (D / 4);
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (r0 + r < rows && 4 * cc < DR) v = *reinterpret_cast<const f32x4*>(src + (int64_t)(r0 + r) * DR + 4 * cc);
        *reinterpret_cast<f32x4*>(tile + r * RS + 4 * cc) = v;
    }
}

// This lane's row of a [rows, DR] tensor as contraction operands: slot
// 8*T + 4*hg + u in element u of x[T] (zeros past the row or the tensor).
template <int D>
__device__ __forceinline__ void f_load_row(f32x4 (&x)[D / 8], const float* src, int row, int rows, int DR, int hg) {
#pragma unroll
    for (int T = 0; T < D / 8; ++T) {
        x[T] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (row < rows && 8 * T + 4 * hg < DR)
            x[T] = *reinterpret_cast<const f32x4*>(src + (int64_t)row * DR + 8 * T + 4 * hg);
    }
}

// acc (rows = 32 rows of `tile` from row t0, columns = the lane operands x)
// = tile[t0 + l32] . x over the head dim.
template <int D>
__device__ __forceinline__ f32x16 f_rows_dot(const float* __restrict__ tile, int t0, const f32x4 (&x)[D / 8], int l32,
                                             int hg) {
    constexpr int RS = D + 4;
    f32x16 acc = {};
    const float* row = tile + (t0 + l32) * RS + 4 * hg;
#pragma unroll
    for (int T = 0; T < D / 8; ++T) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(row + 8 * T);
#pragma unroll
        for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[u], x[T][u], acc, 0, 0, 0);
    }
    return acc;
}

// acc[db] (rows = dims 32db .. 32db+31, columns as w) += tile^T w, contracting
// over tile rows t0 + 8*(u/4) + 4*hg + u%4 (register u of w).
template <int D>
__device__ __forceinline__ void f_tile_t_dot(f32x16 (&acc)[D / 32], const float* __restrict__ tile, int t0,
                                             const f32x16& w, int l32, int hg) {
    constexpr int RS = D + 4;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const int r = t0 + 8 * (u >> 2) + 4 * hg + (u & 3);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(tile[r * RS + 32 * db + l32], w[u], acc[db], 0, 0, 0);
    }
}

// 2. dQ.  Lane: query qi = q0 + 32*wave + l32; S^T and dP^T hold keys
// j0 + 32*kb2 + 8*(r/4) + 4*hg + r%4 in register r.
template <int D>
__global__ __launch_bounds__(kFbThreads, 1) void bwd_f32_dq_kernel(BackwardArgs a) {
    constexpr int RS = D + 4;
    __shared__ __attribute__((aligned(16))) float ks[kFbTile * RS];
    __shared__ __attribute__((aligned(16))) float vs[kFbTile * RS];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hg = lane >> 5;
    const int DR = a.D;

    const int G = a.Hq / a.Hkv;
    const int nqb = (a.Sq + kFbRows - 1) / kFbRows;
    int t = f_xcd_order(a.B * a.Hkv * nqb * G);
    const int hsub = t % G;
    t /= G;
    const int qord = t % nqb;
    const int unit = t / nqb;
    const int b = unit / a.Hkv, gk = unit % a.Hkv, h = gk * G + hsub;
    const int q0 = (a.causal ? nqb - 1 - qord : qord) * kFbRows;
    const int64_t bh = (int64_t)b * a.Hq + h;
    const int64_t kvh = ((int64_t)b * a.Hkv + gk) * a.Sk * DR;
    const float* kp = static_cast<const float*>(a.k) + kvh;
    const float* vp = static_cast<const float*>(a.v) + kvh;

    int kv_lim = a.Sk;
    if (a.padded) kv_lim = max(0, min(kv_lim, a.key_lens[b]));
    int kv_end = kv_lim;
    if (a.causal) kv_end = min(kv_end, q0 + kFbRows);
    const int ntiles = kv_end > 0 ? (kv_end + kFbTile - 1) / kFbTile : 0;
    const int qw = q0 + 32 * wave, qi = qw + l32;

    f32x4 qf[D / 8], df[D / 8];
    f_load_row<D>(qf, static_cast<const float*>(a.q) + bh * a.Sq * DR, qi, a.Sq, DR, hg);
    f_load_row<D>(df, static_cast<const float*>(a.dout) + bh * a.Sq * DR, qi, a.Sq, DR, hg);
    float lse2 = INFINITY, delta = 0.f;
    if (qi < a.Sq) {
        const float2 st = reinterpret_cast<const float2*>(a.delta)[bh * f_stats_stride(a.Sq) + qi];
        lse2 = st.x;
        delta = st.y;
    }
    const float c = a.scale * kLog2e;

    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

    for (int jt = 0; jt < ntiles; ++jt) {
        const int j0 = jt * kFbTile;
        __syncthreads();  // the previous tile's reads are done
        f_load_tile<D>(ks, kp, j0, a.Sk, DR, tid);
        f_load_tile<D>(vs, vp, j0, a.Sk, DR, tid);
        __syncthreads();
        if (qw >= a.Sq || (a.causal && j0 > qw + 31)) continue;  // wave-uniform
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
            const f32x16 s = f_rows_dot<D>(ks, 32 * kb2, qf, l32, hg);
            const f32x16 dp = f_rows_dot<D>(vs, 32 * kb2, df, l32, hg);
            f32x16 ds;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = j0 + 32 * kb2 + 8 * (r >> 2) + 4 * hg + (r & 3);
                const bool hide = key >= kv_lim || (a.causal && key > qi);
                const float p = hide ? 0.f : fast_exp2(fmaf(s[r], c, -lse2));
                ds[r] = p * (dp[r] - delta);
            }
            f_tile_t_dot<D>(acc, ks, 32 * kb2, ds, l32, hg);
        }
    }

    if (qi < a.Sq) {
        float* row = static_cast<float*>(a.dq) + (bh * a.Sq + qi) * DR;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d0 = 32 * db + 8 * r4 + 4 * hg;  // 4 dims, all < DR or none
                if (d0 < DR)
                    *reinterpret_cast<f32x4*>(row + d0) =
                        f32x4{acc[db][4 * r4] * a.scale, acc[db][4 * r4 + 1] * a.scale,
                              acc[db][4 * r4 + 2] * a.scale, acc[db][4 * r4 + 3] * a.scale};
            }
    }
}

// 3. dK and dV.  Lane: key kj = k0 + 32*wave + l32; S and dP of query block
// qb hold queries q0 + 32*qb + 8*(r/4) + 4*hg + r%4 in register r.
template <int D>
__global__ __launch_bounds__(kFbThreads, 1) void bwd_f32_dkdv_kernel(BackwardArgs a) {
    constexpr int RS = D + 4;
    __shared__ __attribute__((aligned(16))) float qs[kFbTile * RS];
    __shared__ __attribute__((aligned(16))) float dos[kFbTile * RS];
    __shared__ float2 sts[kFbTile];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hg = lane >> 5;
    const int DR = a.D;

    const int G = a.Hq / a.Hkv;
    const int nkb = (a.Sk + kFbRows - 1) / kFbRows;
    const int t = f_xcd_order(a.B * a.Hkv * nkb);
    const int unit = t / nkb;
    const int k0 = (t % nkb) * kFbRows;
    const int b = unit / a.Hkv, gk = unit % a.Hkv;
    const int64_t kvh = ((int64_t)b * a.Hkv + gk) * a.Sk * DR;
    int kv_lim = a.Sk;
    if (a.padded) kv_lim = max(0, min(kv_lim, a.key_lens[b]));
    const int kw = k0 + 32 * wave, kj = kw + l32;

    f32x4 kf[D / 8], vf[D / 8];
    f_load_row<D>(kf, static_cast<const float*>(a.k) + kvh, kj, a.Sk, DR, hg);
    f_load_row<D>(vf, static_cast<const float*>(a.v) + kvh, kj, a.Sk, DR, hg);
    const float c = a.scale * kLog2e;

    // Query tiles: all, or (causal) those holding a query >= k0; none when
    // every key of the block is past the key limit.
    const int qt0 = a.causal ? k0 / kFbTile : 0;
    const int nqt = k0 < kv_lim ? max(0, (a.Sq + kFbTile - 1) / kFbTile - qt0) : 0;
    const int steps = G * nqt;

    f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        dka[db] = f32x16{};
        dva[db] = f32x16{};
    }
    for (int st = 0; st < steps; ++st) {
        const int h = gk * G + st / nqt;
        const int q0 = (qt0 + st % nqt) * kFbTile;
        const int64_t bh = (int64_t)b * a.Hq + h;
        __syncthreads();
        f_load_tile<D>(qs, static_cast<const float*>(a.q) + bh * a.Sq * DR, q0, a.Sq, DR, tid);
        f_load_tile<D>(dos, static_cast<const float*>(a.dout) + bh * a.Sq * DR, q0, a.Sq, DR, tid);
        if (tid < kFbTile)  // rows past Sq: lse2 = +inf, so P = 0
            sts[tid] = q0 + tid < a.Sq ? reinterpret_cast<const float2*>(a.delta)[bh * f_stats_stride(a.Sq) + q0 + tid]
                                       : make_float2(INFINITY, 0.f);
        __syncthreads();
        if (kw >= kv_lim || (a.causal && q0 + kFbTile - 1 < kw)) continue;  // wave-uniform: no visible pair
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const f32x16 s = f_rows_dot<D>(qs, 32 * qb, kf, l32, hg);
            const f32x16 dp = f_rows_dot<D>(dos, 32 * qb, vf, l32, hg);
            f32x16 p, ds;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qt = 32 * qb + 8 * (r >> 2) + 4 * hg + (r & 3);
                const float2 sv = sts[qt];
                const bool hide = kj >= kv_lim || (a.causal && kj > q0 + qt);
                p[r] = hide ? 0.f : fast_exp2(fmaf(s[r], c, -sv.x));
                ds[r] = p[r] * (dp[r] - sv.y);
            }
            f_tile_t_dot<D>(dva, dos, 32 * qb, p, l32, hg);
            f_tile_t_dot<D>(dka, qs, 32 * qb, ds, l32, hg);
        }
    }

    // register r of d-block db: dim 32db + 8*(r/4) + 4*hg + r%4 of key kj;
    // keys past the key limit were never visible (their sums are 0)
    if (kj < a.Sk) {
        float* krow = static_cast<float*>(a.dk) + kvh + (int64_t)kj * DR;
        float* vrow = static_cast<float*>(a.dv) + kvh + (int64_t)kj * DR;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d0 = 32 * db + 8 * r4 + 4 * hg;
                if (d0 < DR) {
                    *reinterpret_cast<f32x4*>(krow + d0) =
                        f32x4{dka[db][4 * r4] * a.scale, dka[db][4 * r4 + 1] * a.scale,
                              dka[db][4 * r4 + 2] * a.scale, dka[db][4 * r4 + 3] * a.scale};
                    *reinterpret_cast<f32x4*>(vrow + d0) =
                        f32x4{dva[db][4 * r4], dva[db][4 * r4 + 1], dva[db][4 * r4 + 2], dva[db][4 * r4 + 3]};
                }
            }
    }
}

template <int D>
hipError_t launch_f32_d(const BackwardArgs& a, hipStream_t s) {
    const int64_t rows = (int64_t)a.B * a.Hq * a.Sq;
    const int rpb = kFbThreads / 32;
    hipLaunchKernelGGL(bwd_f32_stats_kernel, dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(kFbThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nqb = (a.Sq + kFbRows - 1) / kFbRows;
    hipLaunchKernelGGL(bwd_f32_dq_kernel<D>, dim3((unsigned)(a.B * a.Hq * nqb)), dim3(kFbThreads), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nkb = (a.Sk + kFbRows - 1) / kFbRows;
    hipLaunchKernelGGL(bwd_f32_dkdv_kernel<D>, dim3((unsigned)(a.B * a.Hkv * nkb)), dim3(kFbThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_backward_f32(const BackwardArgs& a, hipStream_t s) {
    if (a.D < 4 || a.D > 128 || a.D % 4 != 0 || a.bias || a.dq_acc) return hipErrorInvalidValue;
    return a.D <= 64 ? launch_f32_d<64>(a, s) : launch_f32_d<128>(a, s);
}

}  // namespace sdpa
