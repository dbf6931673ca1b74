// Projections of the multi-head attention block (tensai autograd guide,
// section "Attention の組み立て": q, k, v = heads(x . w), y = heads^-1(o) . wo):
// C = A . B with 16-bit A [M x K] and B [K x N], fp32 accumulation, C rounded
// to the input type.  The guide's heads reshape / transpose is folded into
// the addressing: with CH the result is written in (batch, head, seq, headDim)
// layout, with AH the A operand is read from that layout, so no separate
// transpose pass exists.  blockIdx.y selects one of up to three (B, C) pairs
// (the q, k and v projections in one launch).
//
// Tiles: a workgroup of 4 waves owns C rows m0 .. m0+255 and columns
// n0 .. n0+127; wave w owns rows m0 + 64w .. +63.  The kernel computes the
// transposed tile C^T = B^T A^T with v_mfma_f32_32x32x16 so that each lane's
// accumulator holds 4 consecutive columns of one row (8-byte stores, and the
// 4 columns stay inside one head).  A and B tiles of depth 32 reach LDS by
// buffer-load DMA into two stages; MFMA A operands (B^T) are transposed LDS
// reads of the B tile, B operands (A^T) are row reads of the A tile.
#include "device_common.hpp"
#include "launch.hpp"

namespace sdpa {
namespace {

constexpr int kGThreads = 256;
constexpr int kTM = 256;  // C rows per workgroup
constexpr int kTN = 128;  // C columns per workgroup
constexpr int kTK = 32;   // contraction per stage
constexpr uint32_t kFar = 0x80000000u;  // a buffer offset past any num_records (<= INT_MAX)

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ u32x2 lds_tr(const uint16_t* __restrict__ p) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    lds_i16x4* lp = (lds_i16x4*)((__attribute__((address_space(3))) char*)p);
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(lp));
}
__device__ __forceinline__ u32x4 lds_row(const uint16_t* __restrict__ p) {
    return *(const __attribute__((address_space(3))) u32x4*)(
        (const __attribute__((address_space(3))) char*)p);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ void dma(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (lds_void*)((__attribute__((address_space(3))) char*)lds), 16, voff, 0, 0, 0);
}

// Element offset of (row m, column c) of a [M x width] matrix stored either
// row-major (heads = false) or, for m = b*S + s and c = h*hd + d, in
// (batch, head, seq, headDim) layout.
__device__ __forceinline__ int64_t mat_off(int m, int c, int width, bool heads, int S, int hd) {
    if (!heads) return (int64_t)m * width + c;
    const int b = m / S, s = m - b * S, h = c / hd, d = c - h * hd;
    const int H = width / hd;
    return (((int64_t)b * H + h) * S + s) * hd + d;
}

// LDS swizzles (16-byte chunk c of tile row r stored at c ^ f(r)):
//   A tile, rows of 32 elements (4 chunks, 4 rows per 256-byte bank window):
//     fa(r) = (r / 4) % 4 — a row read (one chunk of 16 consecutive rows)
//     hits 16 distinct bank groups.
//   B tile, rows of 128 elements (16 chunks, one bank window):
//     fb(r) = 4 * (r % 4) — a transposed read (4 consecutive rows x 4 chunks
//     per 32 lanes) hits 16 distinct bank groups.
__device__ __forceinline__ int fa(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int fb(int r) { return 4 * (r & 3); }

template <class T, bool AH, bool CH>
__global__ __launch_bounds__(kGThreads, 2) void gemm_kernel(GemmArgs g) {
    constexpr int A_EL = kTM * kTK;   // 8192 elements
    constexpr int B_EL = kTK * kTN;   // 4096
    constexpr int STAGE = A_EL + B_EL;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hg = lane >> 5;

    const int z = blockIdx.y;
    const void* bsrc = z == 0 ? g.b0 : (z == 1 ? g.b1 : g.b2);
    uint16_t* cdst = static_cast<uint16_t*>(z == 0 ? g.c0 : (z == 1 ? g.c1 : g.c2));

    // Tile order: each XCD (workgroups are dealt round-robin, id % 8) owns a
    // contiguous run of tiles, N tiles innermost, so an XCD's workgroups share
    // A row bands in its L2.
    const int ntn = (g.N + kTN - 1) / kTN, ntm = (g.M + kTM - 1) / kTM;
    const int total = ntn * ntm;
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    const int nx = total >> 3, rem = total & 7;
    const int t = xcd * nx + min(xcd, rem) + local;
    const int m0 = (t / ntn) * kTM, n0 = (t % ntn) * kTN;

    const __amdgpu_buffer_rsrc_t ra = rsrc(g.a, g.a_bytes);
    const __amdgpu_buffer_rsrc_t rb = rsrc(bsrc, (uint32_t)g.K * g.N * 2);

    // DMA slots of this wave: A tile 1024 slots (4 loads), B tile 512 (2 loads).
    // A slot s: tile row s/4, stored chunk s%4; B slot s: tile row s/16, stored chunk s%16.
    int a_row[4], a_chk[4], b_row[2], b_chk[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int s = 64 * (4 * wave + i) + lane;
        a_row[i] = s >> 2;
        a_chk[i] = (s & 3) ^ fa(s >> 2);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int s = 64 * (2 * wave + i) + lane;
        b_row[i] = s >> 4;
        b_chk[i] = (s & 15) ^ fb(s >> 4);
    }
    auto issue = [&](int k0, int stage) {
        uint16_t* sa = smem + stage * STAGE + 512 * 4 * wave;
        uint16_t* sb = smem + stage * STAGE + A_EL + 512 * 2 * wave;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = m0 + a_row[i], k = k0 + 8 * a_chk[i];
            const uint32_t off = (m < g.M && k < g.K)
                                     ? (uint32_t)(mat_off(m, k, g.K, AH, g.S, g.hd) * 2)
                                     : kFar;
            dma(ra, sa + 512 * i, off);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int k = k0 + b_row[i], n = n0 + 8 * b_chk[i];
            const uint32_t off = (k < g.K && n < g.N) ? (uint32_t)(((int64_t)k * g.N + n) * 2) : kFar;
            dma(rb, sb + 512 * i, off);
        }
    };

    // LDS read offsets (elements within a stage).
    // A^T operand of block mb: tile row 64*wave + 32*mb + l32, logical chunk 2t + hg.
    int ard[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int r = 64 * wave + 32 * mb + l32;
            ard[mb][k] = r * kTK + (((2 * k + hg) ^ fa(r)) * 8);
        }
    // B^T operand of block nb: lane j of 16-lane group g16 points at tile row
    // 16t + 8hg + j/4 (+4 for the second read), columns 32nb + 16(g16&1) + 4(j%4).
    const int g16 = lane >> 4, j16 = lane & 15;
    int brd[4][2];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = 8 * hg + (j16 >> 2) + 4 * h;
            const int col = 32 * nb + 16 * (g16 & 1) + 4 * (j16 & 3);
            brd[nb][h] = A_EL + r * kTN + (((col >> 3) ^ fb(r)) * 8) + (col & 7);
        }

    f32x16 acc[4][2];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) acc[nb][mb] = f32x16{};

    auto compute = [&](const uint16_t* st) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {  // 16-deep MFMA steps
            u32x4 af[2], bf[4];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) af[mb] = lds_row(st + ard[mb][k]);
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const u32x2 lo = lds_tr(st + brd[nb][0] + 16 * k * kTN);
                const u32x2 hi = lds_tr(st + brd[nb][1] + 16 * k * kTN);
                bf[nb] = u32x4{lo[0], lo[1], hi[0], hi[1]};
            }
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
                    acc[nb][mb] = mfma_32x32x16<T>(bf[nb], af[mb], acc[nb][mb]);
        }
    };

    const int nk = (g.K + kTK - 1) / kTK;
    issue(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    auto step = [&](int kt, const int cur) __attribute__((always_inline)) {
        if (kt + 1 < nk) issue((kt + 1) * kTK, cur ^ 1);
        compute(smem + cur * STAGE);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };
    for (int kt = 0; kt < nk; kt += 2) {
        step(kt, 0);
        if (kt + 1 < nk) step(kt + 1, 1);
    }

    // acc[nb][mb] register r: column n0 + 32nb + 8(r/4) + 4hg + r%4 of row
    // m0 + 64w + 32mb + l32; four consecutive columns per 8-byte store.
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int m = m0 + 64 * wave + 32 * mb + l32;
        if (m >= g.M) continue;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int n = n0 + 32 * nb + 8 * r4 + 4 * hg;
                if (n >= g.N) continue;
                const f32x16& x = acc[nb][mb];
                const u32x2 w = {pack2<T>(x[4 * r4], x[4 * r4 + 1]), pack2<T>(x[4 * r4 + 2], x[4 * r4 + 3])};
                *reinterpret_cast<u32x2*>(cdst + mat_off(m, n, g.N, CH, g.S, g.hd)) = w;
            }
    }
}

template <class T, bool AH, bool CH>
hipError_t launch_gemm_t(const GemmArgs& g, hipStream_t s) {
    const int ntn = (g.N + kTN - 1) / kTN, ntm = (g.M + kTM - 1) / kTM;
    hipLaunchKernelGGL((gemm_kernel<T, AH, CH>), dim3(ntn * ntm, g.nz), dim3(kGThreads), 0, s, g);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_16bit(const GemmArgs& g, bool f16, hipStream_t s) {
    if (g.K % 8 != 0 || g.N % 8 != 0 || g.nz < 1 || g.nz > 3) return hipErrorInvalidValue;
    if (g.a_heads && g.c_heads) return hipErrorInvalidValue;
    if (g.a_heads)
        return f16 ? launch_gemm_t<F16T, true, false>(g, s) : launch_gemm_t<Bf16T, true, false>(g, s);
    if (g.c_heads)
        return f16 ? launch_gemm_t<F16T, false, true>(g, s) : launch_gemm_t<Bf16T, false, true>(g, s);
    return f16 ? launch_gemm_t<F16T, false, false>(g, s) : launch_gemm_t<Bf16T, false, false>(g, s);
}

}  // namespace sdpa
