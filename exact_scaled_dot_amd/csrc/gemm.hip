// Projections of the multi-head attention block (tensai autograd guide,
// section "Attention の組み立て": q, k, v = heads(x . w), y = heads^-1(o) . wo):
// C = A . B with 16-bit A [M x K] and B [K x N], fp32 accumulation, C rounded
// to the input type.  The guide's heads reshape / transpose is folded into
// the addressing: with CH the result is written in (batch, head, seq, headDim)
// layout, with AH the A operand is read from that layout, so no separate
// transpose pass exists.  blockIdx.y selects one of up to three (B, C) pairs
// (the q, k and v projections in one launch).
//
// Tiles: a workgroup of 4 waves owns C rows m0 .. m0+64WM-1 and columns
// n0 .. n0+64WN-1; wave w owns the quarter at rows + 32WM (w % 2), columns
// + 32WN (w / 2).  Large products use WM = WN = 4 (256 x 256 tiles, 256
// accumulator registers, one wave per SIMD); products too small to fill the
// chip with those use 128 x 128 or 64 x 64 tiles.  The
// kernel computes the transposed tile C^T = B^T A^T with v_mfma_f32_32x32x16
// so that each lane's accumulator holds 4 consecutive columns of one row
// (8-byte stores, and the 4 columns stay inside one head).  A and B tiles of
// depth 32 reach LDS by buffer-load DMA into a ring of four stages (32 KB
// each), each load issued between the MFMAs of the stage three before its
// use, so it has over two stages of MFMA work to land; MFMA A operands (B^T)
// are transposed LDS reads of the B tile,
// B operands (A^T) are row reads of the A tile.  Per 16-deep step a wave
// reads 8 KB of LDS for 16 MFMAs, so operand reads plus the DMA writes stay
// under the LDS bandwidth while the matrix cores run.
#include "device_common.hpp"
#include "launch.hpp"

namespace sdpa {
namespace {

constexpr int kGThreads = 256;
constexpr int kTK = 32;   // contraction per stage
constexpr int kStages = 4;  // LDS ring depth
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

// LDS swizzles (16-byte chunk c of tile row r stored at c ^ f(r)):
//   A tile, rows of 32 elements (4 chunks, 4 rows per 256-byte bank window):
//     fa(r) = (r / 4) % 4 — a row read (one chunk of 16 consecutive rows)
//     hits 16 distinct bank groups.
//   B tile, rows of 64WN elements (8WN chunks): fb(r) = 4 * (r % 4) for
//     rows of one or two bank windows, 4 * ((r / 2) % 2) for half-window
//     rows (WN = 1) — a transposed read (4 consecutive rows x 4 aligned
//     chunks per 16 lanes) hits 16 distinct bank groups.
// Workgroup barrier for LDS hand-over only.  __syncthreads() would also
// fence global memory, which waits for every buffer load in flight (the DMA
// stages issued ahead included) and so undoes the prefetch; the waves' own
// vmcnt waits before the barrier cover the DMA that the next stage reads.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ int fa(int r) { return (r >> 2) & 3; }
template <int WN>
__device__ __forceinline__ int fb(int r) { return WN >= 2 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <class T, bool AH, bool CH, int WM, int WN>
__global__ __launch_bounds__(kGThreads, WM * WN >= 16 ? 1 : 2) void gemm_kernel(GemmArgs g) {
    constexpr int NST = kStages;
    constexpr int kTM = 64 * WM;       // C rows per workgroup
    constexpr int kTN = 64 * WN;       // C columns per workgroup
    constexpr int CPR = kTK / 8;       // 16-byte chunks per A tile row
    constexpr int BCH = kTN / 8;       // 16-byte chunks per B tile row
    constexpr int LA = WM, LB = WN;    // DMA loads per wave per A / B tile
    constexpr int A_EL = kTM * kTK;
    constexpr int B_EL = kTK * kTN;
    constexpr int STAGE = A_EL + B_EL;
    static_assert(NST * STAGE * 2 <= 160 * 1024, "LDS ring exceeds 160 KB");
    __shared__ __attribute__((aligned(1024))) uint16_t smem[NST * STAGE];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
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

    // DMA slots of this wave: LA loads per A tile, LB per B tile.
    // A slot s: tile row s/CPR, stored chunk s%CPR; B slot s: tile row s/BCH, stored chunk s%BCH.
    // Byte offsets are 32-bit (every operand is under 2 GiB): a per-slot base
    // set once (kFar for a row or column past the matrix, which keeps any sum
    // below 2^32 and past num_records, so the load returns zeros) plus the
    // part that moves with k.
    const float inv_hd = 1.0f / (float)g.hd;
    uint32_t a_base[LA], b_base[LB];
    int a_kx[LA], b_row[LB];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int s = 64 * (LA * wave + i) + lane;
        const int ar = s / CPR, m = m0 + ar;
        a_kx[i] = 8 * ((s % CPR) ^ fa(ar));
        if (AH) {
            const int b = m / g.S, sq = m - b * g.S;
            a_base[i] = m < g.M ? 2u * (uint32_t)(b * g.S * g.K + sq * g.hd) : kFar;
        } else {
            a_base[i] = m < g.M ? 2u * (uint32_t)m * (uint32_t)g.K : kFar;
        }
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        const int s = 64 * (LB * wave + i) + lane;
        const int br = s / BCH, n = n0 + 8 * ((s % BCH) ^ fb<WN>(br));
        b_row[i] = br;
        b_base[i] = n < g.N ? 2u * (uint32_t)n : kFar;
    }
    auto issue = [&](int k0, int stage) {
        uint16_t* sa = smem + stage * STAGE + 512 * LA * wave;
        uint16_t* sb = smem + stage * STAGE + A_EL + 512 * LB * wave;
#pragma unroll
        for (int i = 0; i < LA; ++i) {
            const int k = k0 + a_kx[i];
            uint32_t part = 2u * (uint32_t)k;
            if (AH) {
                // head h = k / hd by a float reciprocal: (k + 1/2) / hd is at
                // least 1/(2 hd) from an integer, i.e. (k < 2^16) at least
                // 2^-17 of its value, far above the product's rounding error
                const int h = (int)(((float)k + 0.5f) * inv_hd);
                part = 2u * ((uint32_t)h * (uint32_t)(g.S * g.hd) + (uint32_t)(k - h * g.hd));
            }
            // k past K: bit 31 set (the sum stays below 2^32), so the load
            // reads zeros; an OR rather than a select keeps the loop body one
            // basic block for the schedule below
            dma(ra, sa + 512 * i, (a_base[i] + part) | (k < g.K ? 0u : kFar));
        }
#pragma unroll
        for (int i = 0; i < LB; ++i) {
            const int k = k0 + b_row[i];
            dma(rb, sb + 512 * i, (b_base[i] + 2u * (uint32_t)k * (uint32_t)g.N) | (k < g.K ? 0u : kFar));
        }
    };

    // LDS read offsets (elements within a stage).
    // A^T operand of block mb, step kk: tile row 32WM wm + 32mb + l32, logical
    // chunk 2kk + hg; fa of that row equals fa(l32) (32WM wm + 32mb is a
    // multiple of 16), so one swizzle register serves every mb.
    const int ard0 = (32 * WM * wm + l32) * kTK;
    const int afx0 = hg ^ fa(l32);
    // B^T operand of block nb: lane j of 16-lane group g16 points at tile row
    // 16kk + 8hg + j/4 (+4 for the second read), columns 32WN wn + 32nb +
    // 16(g16&1) + 4(j%4); the swizzle depends on the row only through j/4.
    const int g16 = lane >> 4, j16 = lane & 15;
    int brd[WN][2];
#pragma unroll
    for (int nb = 0; nb < WN; ++nb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = 8 * hg + (j16 >> 2) + 4 * h;
            const int col = 32 * WN * wn + 32 * nb + 16 * (g16 & 1) + 4 * (j16 & 3);
            brd[nb][h] = A_EL + r * kTN + (((col >> 3) ^ fb<WN>(r)) * 8) + (col & 7);
        }

    f32x16 acc[WN][WM];
#pragma unroll
    for (int nb = 0; nb < WN; ++nb)
#pragma unroll
        for (int mb = 0; mb < WM; ++mb) acc[nb][mb] = f32x16{};

    auto read_frags = [&](const uint16_t* st, int kk, u32x4 (&af)[WM], u32x4 (&bf)[WN])
                          __attribute__((always_inline)) {
#pragma unroll
        for (int mb = 0; mb < WM; ++mb) af[mb] = lds_row(st + ard0 + 32 * mb * kTK + ((2 * kk) ^ afx0) * 8);
#pragma unroll
        for (int nb = 0; nb < WN; ++nb) {
            const u32x2 lo = lds_tr(st + brd[nb][0] + 16 * kk * kTN);
            const u32x2 hi = lds_tr(st + brd[nb][1] + 16 * kk * kTN);
            bf[nb] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
    };
    auto mfmas = [&](const u32x4 (&af)[WM], const u32x4 (&bf)[WN]) __attribute__((always_inline)) {
#pragma unroll
        for (int nb = 0; nb < WN; ++nb)
#pragma unroll
            for (int mb = 0; mb < WM; ++mb) acc[nb][mb] = mfma_32x32x16<T>(bf[nb], af[mb], acc[nb][mb]);
    };

    // Ring of four buffers: stage kt lives in buffer kt % 4; the prologue
    // fills all four.  Iteration kt runs stage kt's first 16-deep step (its
    // fragments were read at the end of the previous iteration) while reading
    // the second step's; then waits for its own loads of stage kt + 1 (those
    // of kt + 2 and kt + 3, LA + LB per stage, may stay in flight) and meets the
    // other waves at an LDS-only barrier: stage kt + 1 has landed for every
    // wave, and every wave is done reading buffer kt % 4.  The second step's
    // MFMAs then run next to the reads of stage kt + 1's first step and the
    // refill of buffer kt % 4 with stage kt + 4.  Every iteration refills
    // (with zeros once past K), so the wait counts never change.  The
    // refill follows the reads in program order because the compiler cannot
    // tell the ring buffers apart; on the large tiles the schedule puts two
    // MFMAs between consecutive groups of reads or loads (a burst of loads
    // stalls the wave's MFMA issue, a read right before its MFMA exposes its
    // latency).
    const int nk = (g.K + kTK - 1) / kTK;
#pragma unroll
    for (int p = 0; p < NST; ++p) issue(p * kTK, p);
    wait_vmcnt<(LA + LB) * (NST - 1)>();
    lds_barrier();
    u32x4 a0[WM], b0[WN], a1[WM], b1[WN];
    constexpr bool kSched = WM == 4 && WN == 4;
    read_frags(smem, 0, a0, b0);
    for (int kt = 0; kt < nk; ++kt) {
        const uint16_t* st = smem + (kt % NST) * STAGE;
        mfmas(a0, b0);
        read_frags(st, 1, a1, b1);
        if constexpr (kSched) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        wait_vmcnt<(LA + LB) * (NST - 2)>();
        lds_barrier();
        mfmas(a1, b1);
        read_frags(smem + ((kt + 1) % NST) * STAGE, 0, a0, b0);
        issue((kt + NST) * kTK, kt % NST);
        if constexpr (kSched) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
        }
    }
    wait_vmcnt<0>();  // no LDS DMA may land after the workgroup ends

    // acc[nb][mb] register r: column n0 + 32WN wn + 32nb + 8(r/4) + 4hg + r%4
    // of row m0 + 32WM wm + 32mb + l32; four consecutive columns per 8-byte
    // store.  Element offset = row part + column part (both int: C is under
    // 2 GiB).
#pragma unroll
    for (int mb = 0; mb < WM; ++mb) {
        const int m = m0 + 32 * WM * wm + 32 * mb + l32;
        if (m >= g.M) continue;
        int rp = m * g.N;
        if (CH) {
            const int b = m / g.S, sq = m - b * g.S;
            rp = b * g.S * g.N + sq * g.hd;
        }
#pragma unroll
        for (int nb = 0; nb < WN; ++nb)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int n = n0 + 32 * WN * wn + 32 * nb + 8 * r4 + 4 * hg;
                if (n >= g.N) continue;
                int cp = n;
                if (CH) {
                    const int h = n / g.hd;
                    cp = h * g.S * g.hd + (n - h * g.hd);
                }
                const f32x16& x = acc[nb][mb];
                const u32x2 w = {pack2<T>(x[4 * r4], x[4 * r4 + 1]), pack2<T>(x[4 * r4 + 2], x[4 * r4 + 3])};
                *reinterpret_cast<u32x2*>(cdst + rp + cp) = w;
            }
    }
}

template <class T, bool AH, bool CH, int W>
hipError_t launch_gemm_w(const GemmArgs& g, hipStream_t s) {
    const int ntn = (g.N + 64 * W - 1) / (64 * W), ntm = (g.M + 64 * W - 1) / (64 * W);
    hipLaunchKernelGGL((gemm_kernel<T, AH, CH, W, W>), dim3(ntn * ntm, g.nz), dim3(kGThreads), 0, s, g);
    return hipGetLastError();
}

// The largest square tile (256, 128 or 64) whose grid still has at least
// 256 workgroups (one per CU), else the smallest.
template <class T, bool AH, bool CH>
hipError_t launch_gemm_t(const GemmArgs& g, hipStream_t s) {
    auto wgs = [&](int t) { return (int64_t)((g.M + t - 1) / t) * ((g.N + t - 1) / t) * g.nz; };
    if (wgs(256) >= 256) return launch_gemm_w<T, AH, CH, 4>(g, s);
    if (wgs(128) >= 256) return launch_gemm_w<T, AH, CH, 2>(g, s);
    return launch_gemm_w<T, AH, CH, 1>(g, s);
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
