// Attention backward: dQ, dK and dV of O = softmax(Q K^T * scale + mask) V
// for a loss whose gradient with respect to O is dO.  The probabilities are
// recomputed from the forward's per-row log-sum-exp instead of being stored
// (ruDNN user guide, section 11: the attention backward returns dq, dk, dv and
// never keeps the full score matrix).  The derivatives are those of the
// tensai autograd guide's attention block (reshape, two batched products, a
// scale, the mask and a last-axis softmax):
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - delta),  delta_i = sum_d dO_id O_id,
//   dQ = scale dS K,  dK = scale dS^T Q,
// with P_ij = exp(scale * s_ij - lse_i) and hidden keys at P = 0.  Grouped K/V
// heads sum the contributions of their Hq / Hkv query heads.
//
// Two passes, both deterministic (every sum has a fixed order; the ruDNN
// guide's ordered history reduction, section 11):
//   1. dQ pass, query-parallel: a workgroup owns 128 rows of one (batch, query
//      head) and walks its visible keys in tiles of 64.  It also forms delta
//      from the rows of O and dO it holds and writes (lse * log2 e, delta) per
//      row to the workspace for pass 2.
//   2. dK / dV pass, key-parallel: a workgroup owns 128 keys of one (batch,
//      K/V head) and walks the query tiles of every query head of the group.
// Neither pass needs an atomic: each output element is owned by one lane.
//
// MFMA layouts (v_mfma_f32_32x32x16, fp32 accumulation).  Lane l, half
// hg = l / 32: the A operand holds row l%32 with contraction slots
// k = 8*hg + e (e = 0..7), the B operand column l%32 with the same slots, and
// the accumulator column l%32 with row 8*(r/4) + 4*hg + r%4 in register r.  So
// an accumulator tile X [M x N] is, after rounding to 16 bits, already the B
// operand of a product that contracts over M, provided the A operand maps
// slot (hg, e) of 16-row step kk to row 16*kk + 8*(e/4) + 4*hg + e%4.  A
// transposed LDS read (ds_read_b64_tr_b16) of four consecutive rows gives
// exactly that: the rows 4*hg..4*hg+3 (e < 4) and 8+4*hg.. (e >= 4).
//
//   dQ pass (per wave: 32 queries, Q and dO in registers as B operands):
//     S^T = K Q^T, dP^T = V dO^T         (K, V: row reads of the LDS tile)
//     dQ^T += K^T dS^T                    (K^T: transposed reads)
//   dK / dV pass (per wave: 32 keys, K and V in registers as B operands):
//     S = Q K^T, dP = dO V^T              (Q, dO: row reads)
//     dV^T += dO^T P,  dK^T += Q^T dS     (dO^T, Q^T: transposed reads)
#include "device_common.hpp"
#include "launch.hpp"

namespace sdpa {
namespace {

constexpr int kBwThreads = 256;  // 4 waves of 64
constexpr int kBwRows = 128;     // rows a workgroup owns (queries in pass 1, keys in pass 2)
constexpr int kBwTile = 64;      // rows of the streamed operand per step
constexpr uint32_t kOutside = 0x80000000u;  // a buffer offset past any num_records (<= INT_MAX)
// Cache policy of the bias-gradient stores: non-temporal (written once, read
// by nobody here; 3.5% faster than the default policy for the causal S=4096
// backward with a bias, whose 2.15 GB of dS would otherwise pass through L2).
// The bias loads keep the default policy: the batches that share a bias
// re-read it from cache (non-temporal loads were 7% slower).
constexpr int kStreamed = 2;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// LDS helpers.  The __restrict__ parameters give each inlined access an alias
// scope of its own, which keeps the compiler from putting a vmcnt(0) drain of
// the in-flight LDS-DMA writes in front of it (explicit waits order those).
__device__ __forceinline__ u32x2 lds_tr(const uint16_t* __restrict__ p) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    lds_i16x4* lp = (lds_i16x4*)((__attribute__((address_space(3))) char*)p);
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(lp));
}
__device__ __forceinline__ u32x4 lds_row(const uint16_t* __restrict__ p) {
    return *(const __attribute__((address_space(3))) u32x4*)(
        (const __attribute__((address_space(3))) char*)p);
}
__device__ __forceinline__ f32x4 lds_f4(const float* __restrict__ p) {
    return *(const __attribute__((address_space(3))) f32x4*)(
        (const __attribute__((address_space(3))) char*)p);
}

__device__ __forceinline__ void lds_st4(uint32_t* __restrict__ p, u32x4 v) {
    *(__attribute__((address_space(3))) u32x4*)((__attribute__((address_space(3))) char*)p) = v;
}
__device__ __forceinline__ void lds_st2(uint16_t* __restrict__ p, u32x2 v) {
    *(__attribute__((address_space(3))) u32x2*)((__attribute__((address_space(3))) char*)p) = v;
}
__device__ __forceinline__ u32x2 lds_ld2(const uint16_t* __restrict__ p) {
    return *(const __attribute__((address_space(3))) u32x2*)(
        (const __attribute__((address_space(3))) char*)p);
}
__device__ __forceinline__ u32x4 lds_ld4(const uint32_t* __restrict__ p) {
    return *(const __attribute__((address_space(3))) u32x4*)(
        (const __attribute__((address_space(3))) char*)p);
}
// Workgroup barrier for LDS traffic only: this wave's LDS accesses complete,
// then s_barrier (__syncthreads() would also drain the DMA loads in flight).
// The memory clobbers keep the compiler from moving accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
// A packed 16-bit pair back to two floats (exact).
template <class T>
__device__ __forceinline__ float2 unpack2(uint32_t w) {
    if constexpr (T::kF16) {
        const f16x2 h = __builtin_bit_cast(f16x2, w);
        return make_float2((float)h[0], (float)h[1]);
    } else {
        return make_float2(__builtin_bit_cast(float, w << 16), __builtin_bit_cast(float, w & 0xffff0000u));
    }
}

// Raw buffer resource over [base, base + bytes); loads beyond it return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}
// 16 bytes (8 elements) of a row from 2-byte loads, for head dims that are
// not multiples of 8 (such rows are not 16-byte aligned): element e from byte
// offset off + 2e when e < valid, else zero.
__device__ __forceinline__ u32x4 elem16(__amdgpu_buffer_rsrc_t r, uint32_t off, int valid) {
    u32x4 v;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(r, 2 * w < valid ? off + 4 * w : kOutside, 0, 0);
        const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(r, 2 * w + 1 < valid ? off + 4 * w + 2 : kOutside, 0, 0);
        v[w] = lo | (hi << 16);
    }
    return v;
}
// Four 16-bit values of a row stored element by element (e < valid).
__device__ __forceinline__ void store4_elem(uint16_t* p, u32x2 w, int valid) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (e < valid) p[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
}

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at
// lds + 16*l (the destination is wave-uniform).
__device__ __forceinline__ void dma(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (lds_void*)((__attribute__((address_space(3))) char*)lds), 16, voff, 0, 0, 0);
}

// sum of the eight products of two packed 16-bit vectors, added to acc (fp32).
// The words are copied to scalars before the bit casts: this hipcc folds
// __builtin_bit_cast of a vector element to element 0.
template <class T>
__device__ __forceinline__ float dot8(u32x4 x, u32x4 y, float acc) {
    const uint32_t xs[4] = {x[0], x[1], x[2], x[3]}, ys[4] = {y[0], y[1], y[2], y[3]};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (T::kF16)
            acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, xs[i]),
                                         __builtin_bit_cast(f16x2, ys[i]), acc, false);
        else
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xs[i]),
                                                  __builtin_bit_cast(bf16x2, ys[i]), acc, false);
    }
    return acc;
}

// LDS tile of kBwTile rows x D 16-bit elements, rows unpadded, 16-byte chunk c
// of row r stored at chunk c ^ f(r).  With u = r / RPW (RPW = rows per
// 256-byte bank window) and NB = D / 32 blocks of four chunks per row,
// f(r) = 4 * (u % NB) + (u / NB) % 4:
//   - a row read (one chunk of 16 consecutive rows, one lane each) hits 16
//     distinct 16-byte bank groups, since f is one-to-one over 16 rows;
//   - a transposed read (4 consecutive rows x 4 consecutive chunks per 32
//     lanes) does too, since the four rows differ in f's block bits.
// f repeats every 16 rows, so offsets computed for rows 0..31 serve every
// 16-aligned row block.
template <int D>
struct BwGeo {
    static constexpr int CPR = D / 8;                // 16-byte chunks per row
    static constexpr int RPW = 256 / (2 * D);        // rows per bank window
    static constexpr int NB = CPR / 4;               // 4-chunk blocks per row
    static constexpr int TILE = kBwTile * D;         // elements per tile
    static constexpr int DMA = TILE * 2 / 1024 / 4;  // 1-KB DMA loads per wave per tile
    __device__ static int f(int r) {
        const int u = r / RPW;
        return 4 * (u % NB) + (u / NB) % 4;
    }
};

// Lane-constant LDS offsets (elements) shared by both passes.
template <int D>
struct BwOffsets {
    using L = BwGeo<D>;
    int row[D / 16];  // row read: row l32, logical chunk 2t + hg
    int trl[D / 32];  // transposed read, rows 4hg + j/4 of a 16-row step, dims 32db + ...
    int trh[D / 32];  // the same 8 rows further on
    uint32_t dma[L::DMA];  // DMA source offsets (bytes) of this wave's tile slots
    int dmv[L::DMA];       // elements of each slot inside the row (element-wise loads)
    // DR: head dim in memory (rows DR wide in HBM; chunks at or past DR are
    // pointed outside the buffer and read as zeros).
    __device__ BwOffsets(int wave, int lane, int DR) {
        const int l32 = lane & 31, hg = lane >> 5;
#pragma unroll
        for (int t = 0; t < D / 16; ++t) row[t] = l32 * D + (((2 * t + hg) ^ L::f(l32)) * 8);
        // Inside each 16-lane group, lane j points at row k0 + j/4, dims
        // d0 + 4*(j%4) .. +3; lane j then receives rows k0..k0+3 of dim d0 + j.
        const int g16 = lane >> 4, j16 = lane & 15;
        const int rl = 4 * hg + (j16 >> 2), rh = rl + 8;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const int col = 32 * db + 16 * (g16 & 1) + 4 * (j16 & 3);
            trl[db] = rl * D + (((col >> 3) ^ L::f(rl)) * 8) + (col & 7);
            trh[db] = rh * D + (((col >> 3) ^ L::f(rh)) * 8) + (col & 7);
        }
        // DMA load i of this wave fills 16-byte slot s = 64*(DMA*wave + i) + lane
        // of the tile: row s / CPR, stored chunk s % CPR.
#pragma unroll
        for (int i = 0; i < L::DMA; ++i) {
            const int s = 64 * (L::DMA * wave + i) + lane;
            const int r = s / L::CPR, c = (s % L::CPR) ^ L::f(r);  // logical chunk
            dma[i] = 8 * c < DR ? (uint32_t)r * DR * 2 + (uint32_t)(c * 16) : kOutside;
            dmv[i] = min(8, max(0, DR - 8 * c));
        }
    }
};

// Rows of one head in the (lse2, delta) workspace: Sq rounded up to even, so
// every head's slice starts 16-byte aligned.
__host__ __device__ __forceinline__ int64_t stats_stride(int Sq) { return (Sq + 1) & ~1; }

// Workgroup id -> position in a logical order in which each of the 8 XCDs
// (workgroups are dealt to them round-robin, id % 8) owns one contiguous run,
// so workgroups sharing K/V (pass 1) or Q/dO (pass 2) share one L2.
__device__ __forceinline__ int xcd_order(int total) {
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    const int nx = total >> 3, rem = total & 7;
    return xcd * nx + min(xcd, rem) + local;
}

// ---------------------------------------------------------------------------
// Pass 1: dQ (and the per-row statistics for pass 2).
// Logical order: (batch, K/V head) outermost, query block, then the query
// heads of the group innermost; under a causal mask the longest blocks (the
// last rows) first.
// ---------------------------------------------------------------------------
// BIAS: P is recomputed from the biased scores (exp2(s c + bias log2e -
// lse2)).  Each wave moves its [32 query x 32 key] block of the bias, and of
// the bias gradient dS, through a 2-KB LDS staging region per block: HBM
// sees 64-byte row pieces (16 rows per instruction) while the products see
// one query row per lane.  The bias of block b of tile jt+1 is loaded into
// registers before block b of tile jt computes; after it, that block's dS
// is read back row-major and stored (issued after the step's loads, so the
// step's wait leaves the stores in flight), and the loaded bias takes its
// place.  Keys a wave never visits get their (zero) gradient after the loop.
// Staging layout: row r (a query of the wave) holds 8 units of 4 keys;
// logical unit u sits at unit u ^ ((r >> 2) & 7), which keeps both the
// per-lane 8-byte accesses (32 rows, one unit) and the row-major 16-byte
// ones (4 rows, 4 chunks) free of bank conflicts.
// ELEM (with GEN, no bias; head dims that are not multiples of 8): Q, dO, O
// and the K/V tile slots are read element by element (the slots written to
// LDS by the lane the DMA would have filled), dQ stored element by element.
template <int D, class T, bool GEN = false, bool BIAS = false, bool ELEM = false>
__global__ __launch_bounds__(kBwThreads, 2) void bwd_dq_kernel(BackwardArgs a,
                                                               const int32_t* __restrict__ key_lens) {
    using L = BwGeo<D>;
    // Stage s: K tile at 2*s*TILE, V tile at (2*s+1)*TILE; (BIAS) then two
    // 1024-element staging regions per wave.
    __shared__ __attribute__((aligned(1024))) uint16_t smem[4 * L::TILE + (BIAS ? 4 * 2048 : 0)];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hg = lane >> 5;

    const int G = a.Hq / a.Hkv;
    const int nqb = (a.Sq + kBwRows - 1) / kBwRows;
    int t = xcd_order(a.B * a.Hkv * nqb * G);
    const int hsub = t % G;
    t /= G;
    const int qord = t % nqb;
    const int unit = t / nqb;
    const int b = unit / a.Hkv, gk = unit % a.Hkv, h = gk * G + hsub;
    const int q0 = (a.causal ? nqb - 1 - qord : qord) * kBwRows;

    // Head dim in memory: DR (GEN: a multiple of 8 below D; else D).
    const int DR = GEN ? a.D : D;
    const int64_t bh = (int64_t)b * a.Hq + h;
    const int64_t kvh = ((int64_t)b * a.Hkv + gk) * a.Sk * DR;
    const uint16_t* kp = static_cast<const uint16_t*>(a.k) + kvh;
    const uint16_t* vp = static_cast<const uint16_t*>(a.v) + kvh;
    const int64_t qoff = bh * a.Sq * DR;

    int kv_lim = a.Sk;
    if (a.padded) kv_lim = max(0, min(kv_lim, key_lens[b]));
    int kv_end = kv_lim;
    if (a.causal) kv_end = min(kv_end, q0 + kBwRows);
    const int qw = q0 + 32 * wave;  // first query row of this wave
    const int qi = qw + l32;        // this lane's query row
    const int ntiles = kv_end > 0 ? (kv_end + kBwTile - 1) / kBwTile : 0;
    // Tiles this wave computes on (it still takes part in every load and barrier).
    int wave_tiles = a.causal ? max(0, min(ntiles, (qw + 31) / kBwTile + 1)) : ntiles;
    if (qw >= a.Sq) wave_tiles = 0;

    // Q and dO rows as B operands: lane holds row qi, dims 16t + 8hg .. +7
    // (rows >= Sq read as zeros).  delta_i = sum_d dO_id O_id in fp32.
    u32x4 qr[D / 16], dr[D / 16];
    float delta;
    {
        const uint32_t bytes = (uint32_t)a.Sq * DR * 2;
        const __amdgpu_buffer_rsrc_t rq = rsrc(static_cast<const uint16_t*>(a.q) + qoff, bytes);
        const __amdgpu_buffer_rsrc_t rd = rsrc(static_cast<const uint16_t*>(a.dout) + qoff, bytes);
        const __amdgpu_buffer_rsrc_t ro = rsrc(static_cast<const uint16_t*>(a.out) + qoff, bytes);
        float part = 0.f;
#pragma unroll
        for (int k = 0; k < D / 16; ++k) {
            const int d0 = 16 * k + 8 * hg;
            const uint32_t off = d0 < DR ? (uint32_t)qi * DR * 2 + d0 * 2 : kOutside;
            if constexpr (ELEM) {
                qr[k] = elem16(rq, off, DR - d0);
                dr[k] = elem16(rd, off, DR - d0);
                part = dot8<T>(dr[k], elem16(ro, off, DR - d0), part);
            } else {
                qr[k] = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
                dr[k] = __builtin_amdgcn_raw_buffer_load_b128(rd, off, 0, 0);
                part = dot8<T>(dr[k], __builtin_amdgcn_raw_buffer_load_b128(ro, off, 0, 0), part);
            }
        }
        delta = part + swap_half_wave(part);
    }
    // lse in log2 units; a row with no visible key (lse = -inf) gets +inf so
    // that every recomputed probability of it is exactly 0, and delta 0 (its
    // forward output row is 0/0, so O o dO would be NaN).
    float lse2 = INFINITY;
    if (qi < a.Sq) {
        const float l = a.lse[bh * a.Sq + qi];
        lse2 = (l == -INFINITY) ? INFINITY : l * kLog2e;
        if (l == -INFINITY) delta = 0.f;
        if (hg == 0) {
            float2* st = reinterpret_cast<float2*>(a.delta) + bh * stats_stride(a.Sq) + qi;
            *st = make_float2(lse2, delta);
        }
    }

    // Bias and bias gradient: resources over this (batch, head)'s [Sq, Sk]
    // slices (out-of-range offsets read 0 / are dropped).  Row-major staging
    // access i of lane l: row 16i + l/4 of the wave, keys 8*(l%4) .. +7 of
    // the block (stored chunk cs, halves swapped when sw).
    const bool DB = BIAS && a.dbias != nullptr;
    uint16_t* const stg = smem + 4 * L::TILE + 2048 * wave;
    const __amdgpu_buffer_rsrc_t rbias =
        rsrc(BIAS ? static_cast<const uint16_t*>(a.bias) + b * a.bias_sb + h * a.bias_sh
                  : static_cast<const uint16_t*>(a.q),
             BIAS ? (uint32_t)a.Sq * a.Sk * 2 : 0u);
    const __amdgpu_buffer_rsrc_t rdb =
        rsrc(DB ? static_cast<uint16_t*>(a.dbias) + bh * a.Sq * a.Sk : a.q, DB ? (uint32_t)a.Sq * a.Sk * 2 : 0u);
    const int crow = lane >> 2, cchk = lane & 3;
    auto stg_at = [&](int kb2, int i) {  // staging element offset of row-major access i
        const int r = 16 * i + crow, x = (r >> 2) & 7;
        return 1024 * kb2 + r * 32 + ((cchk ^ (x >> 1)) * 8);
    };
    auto swapped = [&](u32x4 v, int i) {  // logical <-> stored order of a chunk
        return (((16 * i + crow) >> 2) & 1) ? u32x4{v[2], v[3], v[0], v[1]} : v;
    };
    // global byte offset of row-major access i of the block at key kb0
    auto gofs = [&](int kb0, int i) -> uint32_t {
        const int row = qw + 16 * i + crow, key = kb0 + 8 * cchk;
        return (row < a.Sq && key < a.Sk) ? ((uint32_t)row * a.Sk + key) * 2 : kOutside;
    };
    u32x4 bl[2];  // bias of one block of the next tile, row-major
    auto load_bias = [&](int kb0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) bl[i] = __builtin_amdgcn_raw_buffer_load_b128(rbias, gofs(kb0, i), 0, 0);
    };
    auto put_bias = [&](int kb2) {
#pragma unroll
        for (int i = 0; i < 2; ++i) lds_st4(reinterpret_cast<uint32_t*>(stg + stg_at(kb2, i)), swapped(bl[i], i));
    };
    // dS of the block at key kb0 (staging region kb2), or zeros, to the bias gradient
    auto flush = [&](int kb2, int kb0, bool zero) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const u32x4 v = zero ? u32x4{0u, 0u, 0u, 0u} : swapped(lds_row(stg + stg_at(kb2, i)), i);
            __builtin_amdgcn_raw_buffer_store_b128(v, rdb, gofs(kb0, i), 0, kStreamed);
        }
    };
    // per-lane staging offsets: row l32, logical unit 2g + hg of region kb2
    auto stg_unit = [&](int kb2, int g) { return 1024 * kb2 + l32 * 32 + (((2 * g + hg) ^ ((l32 >> 2) & 7)) * 4); };

    const BwOffsets<D> off(wave, lane, DR);
    auto issue = [&](int j0, int stage) {
        const uint32_t bytes = (uint32_t)(a.Sk - j0) * DR * 2;
        const __amdgpu_buffer_rsrc_t rk = rsrc(kp + (int64_t)j0 * DR, bytes);
        const __amdgpu_buffer_rsrc_t rv = rsrc(vp + (int64_t)j0 * DR, bytes);
        uint16_t* dk = smem + 2 * stage * L::TILE + 512 * L::DMA * wave;
        uint16_t* dv = dk + L::TILE;
#pragma unroll
        for (int i = 0; i < L::DMA; ++i) {
            if constexpr (ELEM) {  // the slots the DMA would fill: 16 bytes at lane * 16
                lds_st4(reinterpret_cast<uint32_t*>(dk + 512 * i + 8 * lane), elem16(rk, off.dma[i], off.dmv[i]));
                lds_st4(reinterpret_cast<uint32_t*>(dv + 512 * i + 8 * lane), elem16(rv, off.dma[i], off.dmv[i]));
            } else {
                dma(rk, dk + 512 * i, off.dma[i]);
                dma(rv, dv + 512 * i, off.dma[i]);
            }
        }
    };

    const float c = a.scale * kLog2e;
    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

    // One 64-key tile: per 32-key block, S^T and dP^T, then dS^T, then
    // dQ^T += K^T dS^T.  Register r of a score block holds key
    // j0 + 32*kb2 + 8*(r/4) + 4*hg + r%4 of query qi.
    auto compute = [&](const uint16_t* ks, const uint16_t* vs, int j0) __attribute__((always_inline)) {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
            const int kb0 = j0 + 32 * kb2;
            const bool more = BIAS && j0 + kBwTile < wave_tiles * kBwTile;  // a next tile to stage
            if (kb0 >= kv_lim || (a.causal && kb0 > qw + 31)) {  // wave-uniform
                // every key of the block is hidden: dS = 0
                if (DB) flush(kb2, kb0, true);
                if (more) {
                    load_bias(kb0 + kBwTile);
                    put_bias(kb2);
                }
                continue;
            }
            if (more) load_bias(kb0 + kBwTile);
            f32x16 s = {}, dp = {};
            {
                // K and V row fragments two contraction steps ahead of their
                // MFMAs (0.9% on the causal S=4096 backward, same output)
                constexpr int NK = D / 16;
                u32x4 fk[3], fv[3];
                auto rd = [&](int k, int slot) __attribute__((always_inline)) {
                    fk[slot] = lds_row(ks + 32 * kb2 * D + off.row[k]);
                    fv[slot] = lds_row(vs + 32 * kb2 * D + off.row[k]);
                };
                rd(0, 0);
                rd(1, 1);
#pragma unroll
                for (int k = 0; k < NK; ++k) {
                    if (k + 2 < NK) rd(k + 2, (k + 2) % 3);
                    s = mfma_32x32x16<T>(fk[k % 3], qr[k], s);
                    dp = mfma_32x32x16<T>(fv[k % 3], dr[k], dp);
                }
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 7);
#pragma unroll
                for (int k = 0; k < NK; ++k) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 7);
                    if (k + 2 < NK) __builtin_amdgcn_sched_group_barrier(0x100, 2, 7);
                }
            }
            // bias of keys kb0 + 8g + 4hg .. +3 (registers 4g .. 4g+3), read
            // after the products (fewer registers live across them)
            u32x2 bz[4];
            if constexpr (BIAS) {
#pragma unroll
                for (int g = 0; g < 4; ++g) bz[g] = lds_ld2(stg + stg_unit(kb2, g));
            }
            const bool need_mask = kb0 + 32 > kv_lim || (a.causal && kb0 + 31 > qw);
            uint32_t w[8];
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                float e0 = -lse2, e1 = -lse2;
                if constexpr (BIAS) {
                    const uint32_t bw2 = bz[r >> 2][(r & 3) >> 1];
                    e0 = fmaf(bias_elem<T>(bw2, 0), kLog2e, e0);
                    e1 = fmaf(bias_elem<T>(bw2, 1), kLog2e, e1);
                }
                float p0 = fast_exp2(fmaf(s[r], c, e0));
                float p1 = fast_exp2(fmaf(s[r + 1], c, e1));
                if (need_mask) {
                    const int key = kb0 + 8 * (r >> 2) + 4 * hg + (r & 3);
                    if (key >= kv_lim || (a.causal && key > qi)) p0 = 0.f;
                    if (key + 1 >= kv_lim || (a.causal && key + 1 > qi)) p1 = 0.f;
                }
                w[r >> 1] = pack2<T>(p0 * (dp[r] - delta), p1 * (dp[r + 1] - delta));
            }
            if (DB) {
                // the bias gradient is dS: keys kb0 + 8g + 4hg .. +3 are words 2g, 2g+1
#pragma unroll
                for (int g = 0; g < 4; ++g) lds_st2(stg + stg_unit(kb2, g), u32x2{w[2 * g], w[2 * g + 1]});
                flush(kb2, kb0, false);
            }
            if (more) put_bias(kb2);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const u32x4 bw = {w[4 * kk], w[4 * kk + 1], w[4 * kk + 2], w[4 * kk + 3]};
                const uint16_t* kt = ks + (32 * kb2 + 16 * kk) * D;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const u32x2 lo = lds_tr(kt + off.trl[db]);
                    const u32x2 hi = lds_tr(kt + off.trh[db]);
                    acc[db] = mfma_32x32x16<T>(u32x4{lo[0], lo[1], hi[0], hi[1]}, bw, acc[db]);
                }
            }
        }
    };

    if (ntiles > 0) issue(0, 0);
    if (BIAS && wave_tiles > 0) {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
            load_bias(32 * kb2);
            put_bias(kb2);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // Tile jt sits in stage jt % 2; the next one is loaded into the other
    // stage meanwhile (it was last read before the previous barrier).  A
    // computing wave's last VMEM operations of a step are its 2 bias-gradient
    // stores of the last block (when DB); vmcnt counts in issue order, so
    // vmcnt(2) has every load of the step landed and leaves them in flight.
    auto step = [&](int jt, const int cur) __attribute__((always_inline)) {
        if (jt + 1 < ntiles) issue((jt + 1) * kBwTile, cur ^ 1);
        if (jt < wave_tiles)
            compute(smem + 2 * cur * L::TILE, smem + (2 * cur + 1) * L::TILE, jt * kBwTile);
        if (DB && jt < wave_tiles) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };
    for (int jt = 0; jt < ntiles; jt += 2) {
        step(jt, 0);
        if (jt + 1 < ntiles) step(jt + 1, 1);
    }
    if (DB && qw < a.Sq) {
        // zeros for every key past the computed tiles (all hidden): 8 rows of
        // 128 bytes per store
        for (int j0 = wave_tiles * kBwTile; j0 < a.Sk; j0 += kBwTile) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = qw + 8 * i + (lane >> 3), key = j0 + 8 * (lane & 7);
                __builtin_amdgcn_raw_buffer_store_b128(
                    u32x4{0u, 0u, 0u, 0u}, rdb,
                    (row < a.Sq && key < a.Sk) ? ((uint32_t)row * a.Sk + key) * 2 : kOutside, 0, kStreamed);
            }
        }
    }

    // dQ = scale * (dS K): register r of d-block db holds dim
    // 32*db + 8*(r/4) + 4*hg + r%4 of row qi.
    if (qi < a.Sq) {
        uint16_t* row = static_cast<uint16_t*>(a.dq) + qoff + (int64_t)qi * DR;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f32x16& x = acc[db];
                const u32x2 w = {pack2<T>(x[4 * r4] * a.scale, x[4 * r4 + 1] * a.scale),
                                 pack2<T>(x[4 * r4 + 2] * a.scale, x[4 * r4 + 3] * a.scale)};
                const int d0 = 32 * db + 8 * r4 + 4 * hg;  // 4 dims, all < DR or none (unless ELEM)
                if constexpr (ELEM) store4_elem(row + d0, w, DR - d0);
                else if (d0 < DR) *reinterpret_cast<u32x2*>(row + d0) = w;
            }
    }
}

// ---------------------------------------------------------------------------
// Pass 2: dK and dV.
// A workgroup of 8 waves owns 128 keys of one (batch, K/V head).  Waves w and
// w + 4 (one pair per SIMD) share keys 32w .. 32w+31 and split the work:
//   wave w     (role P):  S = Q K^T, P = exp(scale S - lse) (masked), P to LDS,
//                         dV^T += dO^T P
//   wave w + 4 (role dS): dP = dO V^T, then (P from LDS) dS = P o (dP - delta),
//                         dK^T += Q^T dS
// so each wave holds one K/V operand and one accumulator (two waves fit per
// SIMD) while the LDS reads per product stay those of 32-key blocks.  One LDS
// barrier inside each step hands P over.  Products are v_mfma_f32_32x32x16:
// S and dP are [query x key] with Q / dO as row-read A operands and K / V in
// registers, so their accumulators hold key l%32 in each lane and are already
// the B operands of the gradient products, whose A operands are transposed
// reads of dO and Q.  P is exchanged rounded to the input type (the values
// multiplied into dV).
// Logical order: (batch, K/V head) outermost, then key blocks; under a causal
// mask the first key blocks (which see the most queries) first.
// ---------------------------------------------------------------------------
constexpr int kKvThreads = 512;  // 8 waves

//
// DQ (the atomic variant): the same pass also forms dQ.  After P is handed
// over, each role-dS wave writes its dS block ([key][query], 16-bit) into its
// pair's dS slot; after a second barrier every wave takes one 32x32
// tile of dQ = dS K over the block's 128 keys (both operands by transposed
// reads: dS from the slots, K from a copy of the key block kept in LDS) and
// adds it into the fp32 accumulator dq_acc with buffer atomics.  Keys past
// the batch's limit get P = 0 here, so they add nothing.  Atomics count in
// vmcnt on this GPU, so each step ends with vmcnt(0) and the tiles use two
// LDS stages (loaded one step ahead) instead of three.
// BIAS: the P role adds the bias of its query rows at its key before the
// exp, and hides keys past the key limit itself (their bias may be anything).
// The bias of a step ([64 queries x the block's 128 keys], the layout of a
// 128-wide tile) comes into a two-slot LDS ring by DMA: the bias of step
// st+2 goes into the slot of step st as soon as the P hand-over barrier of
// step st has passed (role P reads the bias only before it), so each load
// has a step and a half to land.  A transposed read then gives a lane its
// key at 4 consecutive query rows.
// ELEM (with GEN, no bias, no DQ; head dims that are not multiples of 8): K
// and V rows and the Q/dO tile slots are read element by element, dK and dV
// stored element by element.
template <int D, class T, bool GEN = false, bool DQ = false, bool BIAS = false, bool ELEM = false>
__global__ __launch_bounds__(kKvThreads, 1) void bwd_dkdv_kernel(BackwardArgs a,
                                                                 const int32_t* __restrict__ key_lens) {
    using L = BwGeo<D>;
    using L64 = BwGeo<64>;                  // the [32 key x 64 query] dS slots
    constexpr int NK = D / 16;              // contraction steps of S and dP
    constexpr int ND = D / 32;              // 32-dim blocks of dK and dV
    constexpr int DMA = L::TILE * 2 / 1024 / 8;  // 1-KB DMA loads per wave per tile
    // NSTG stages of: Q tile, dO tile, the tile rows' (lse2, delta) pairs
    // (512 B used of a 1-KB slot); then the P hand-over, 64 B per lane of
    // each role-P wave; (DQ) then the dS slots [pair][32 keys][64 queries]
    // and the workgroup's 128 K rows.
    constexpr int NSTG = DQ ? 2 : 3;
    constexpr int STAGE = 2 * L::TILE + 512;
    constexpr int EX = NSTG * STAGE;
    constexpr int DSX = EX + 4 * 64 * 32;
    constexpr int KB = DSX + 4 * 32 * 64;
    constexpr int BT = kBwTile * kBwRows;  // (BIAS) one bias slot, after the hand-over
    static_assert(!(DQ && BIAS), "the atomic variant takes no bias");
    __shared__ __attribute__((aligned(1024))) uint16_t smem[DQ ? KB + kBwRows * D : DSX + (BIAS ? 2 * BT : 0)];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int role = wave >> 2;  // 0: P and dV; 1: dS and dK
    const int pair = wave & 3;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hg = lane >> 5;

    const int G = a.Hq / a.Hkv;
    const int nkb = (a.Sk + kBwRows - 1) / kBwRows;
    const int t = xcd_order(a.B * a.Hkv * nkb);
    const int unit = t / nkb;
    const int k0 = (t % nkb) * kBwRows;
    const int b = unit / a.Hkv, gk = unit % a.Hkv;

    const int DR = GEN ? a.D : D;  // head dim in memory (a multiple of 8, <= D)
    const int64_t kvh = ((int64_t)b * a.Hkv + gk) * a.Sk * DR;
    int kv_lim = a.Sk;
    if (a.padded) kv_lim = max(0, min(kv_lim, key_lens[b]));
    const int kw = k0 + 32 * pair;  // first key of this pair
    const int kj = kw + l32;        // this lane's key

    // Role P holds K, role dS holds V, as B operands: key kj, dims 16t + 8hg .. +7.
    u32x4 xr[NK];
    {
        const void* src = role ? a.v : a.k;
        const __amdgpu_buffer_rsrc_t rx =
            rsrc(static_cast<const uint16_t*>(src) + kvh, (uint32_t)a.Sk * DR * 2);
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            const int d0 = 16 * k + 8 * hg;
            const uint32_t off = d0 < DR ? (uint32_t)kj * DR * 2 + d0 * 2 : kOutside;
            if constexpr (ELEM)
                xr[k] = elem16(rx, off, DR - d0);
            else
                xr[k] = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
        }
    }

    // Query tiles: all of them, or (causal) those holding a row >= k0; a block
    // whose keys are all hidden does no work at all.
    const int qt0 = a.causal ? k0 / kBwTile : 0;
    const int nqt = (k0 < kv_lim) ? max(0, (a.Sq + kBwTile - 1) / kBwTile - qt0) : 0;
    const int steps = G * nqt;

    if constexpr (DQ) {
        // The block's 128 K rows into LDS (same swizzle as the tiles; rows
        // past Sk and chunks past DR read as zeros).
        constexpr int KD = kBwRows * D * 2 / 1024 / 8;  // 1-KB loads per wave
        const __amdgpu_buffer_rsrc_t rk =
            rsrc(static_cast<const uint16_t*>(a.k) + kvh + (int64_t)k0 * DR, (uint32_t)(a.Sk - k0) * DR * 2);
#pragma unroll
        for (int i = 0; i < KD; ++i) {
            const int s = 64 * (KD * wave + i) + lane;
            const int r = s / L::CPR, c = (s % L::CPR) ^ L::f(r);
            dma(rk, smem + KB + 512 * (KD * wave + i),
                8 * c < DR ? (uint32_t)r * DR * 2 + (uint32_t)(c * 16) : kOutside);
        }
    }

    const BwOffsets<D> off(0, lane, DR);  // row and transposed read offsets
    uint32_t dmo[DMA];
    int dmv[DMA];  // (ELEM) elements of each slot inside the row
#pragma unroll
    for (int i = 0; i < DMA; ++i) {
        const int s = 64 * (DMA * wave + i) + lane;
        const int r = s / L::CPR, c = (s % L::CPR) ^ L::f(r);  // logical chunk
        dmo[i] = 8 * c < DR ? (uint32_t)r * DR * 2 + (uint32_t)(c * 16) : kOutside;
        dmv[i] = min(8, max(0, DR - 8 * c));
    }

    // Bias DMA: 2 loads per wave fill slot s = 64*(2*wave + i) + lane of a
    // 128-wide tile: row s / 16 (a query), stored chunk s % 16 (8 keys).
    using LB = BwGeo<kBwRows>;
    int brow[2], boff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int s = 64 * (2 * wave + i) + lane;
        const int r = s / LB::CPR, key = k0 + 8 * ((s % LB::CPR) ^ LB::f(r));
        brow[i] = r;
        boff[i] = key < a.Sk ? key * 2 : -1;  // key bytes (the row is added per step)
    }
    auto issue_bias = [&](int st, int slot) {
        const int h = gk * G + st / nqt;
        const int q0 = (qt0 + st % nqt) * kBwTile;
        const __amdgpu_buffer_rsrc_t rb =
            rsrc(static_cast<const uint16_t*>(a.bias) + b * a.bias_sb + h * a.bias_sh, (uint32_t)a.Sq * a.Sk * 2);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            dma(rb, smem + DSX + slot * BT + 512 * (2 * wave + i),
                (boff[i] >= 0 && q0 + brow[i] < a.Sq) ? (uint32_t)(q0 + brow[i]) * a.Sk * 2 + (uint32_t)boff[i]
                                                       : kOutside);
    };
    // Transposed-read offsets into a bias slot: rows 4hg + j/4 (lo) and 8 more
    // (hi) of a 16-row step, keys 32*pair + ... (lane receives key kj).
    int btr_lo, btr_hi;
    {
        const int g16 = lane >> 4, j16 = lane & 15;
        const int rl = 4 * hg + (j16 >> 2), rh = rl + 8;
        const int col = 32 * pair + 16 * (g16 & 1) + 4 * (j16 & 3);
        btr_lo = rl * kBwRows + (((col >> 3) ^ LB::f(rl)) * 8) + (col & 7);
        btr_hi = rh * kBwRows + (((col >> 3) ^ LB::f(rh)) * 8) + (col & 7);
    }

    auto issue = [&](int st, int stage) {
        const int h = gk * G + st / nqt;
        const int q0 = (qt0 + st % nqt) * kBwTile;
        const int64_t bh = (int64_t)b * a.Hq + h;
        const int64_t qoff = (bh * a.Sq + q0) * DR;
        const uint32_t bytes = (uint32_t)(a.Sq - q0) * DR * 2;
        const __amdgpu_buffer_rsrc_t rq = rsrc(static_cast<const uint16_t*>(a.q) + qoff, bytes);
        const __amdgpu_buffer_rsrc_t rd = rsrc(static_cast<const uint16_t*>(a.dout) + qoff, bytes);
        uint16_t* dq = smem + stage * STAGE + 512 * DMA * wave;
        uint16_t* dd = dq + L::TILE;
#pragma unroll
        for (int i = 0; i < DMA; ++i) {
            if constexpr (ELEM) {  // the slots the DMA would fill: 16 bytes at lane * 16
                lds_st4(reinterpret_cast<uint32_t*>(dq + 512 * i + 8 * lane), elem16(rq, dmo[i], dmv[i]));
                lds_st4(reinterpret_cast<uint32_t*>(dd + 512 * i + 8 * lane), elem16(rd, dmo[i], dmv[i]));
            } else {
                dma(rq, dq + 512 * i, dmo[i]);
                dma(rd, dd + 512 * i, dmo[i]);
            }
        }
        if (wave == 0) {
            // 8 bytes per row; rows >= Sq read as zeros (and meet zero Q and
            // dO rows, which contribute nothing).
            const __amdgpu_buffer_rsrc_t rs =
                rsrc(reinterpret_cast<const float2*>(a.delta) + bh * stats_stride(a.Sq) + q0,
                     (uint32_t)(a.Sq - q0) * 8);
            dma(rs, smem + stage * STAGE + 2 * L::TILE, 16 * lane);
        }
    };

    const float c = a.scale * kLog2e;
    f32x16 acc[ND];  // role P: dV^T; role dS: dK^T
#pragma unroll
    for (int db = 0; db < ND; ++db) acc[db] = f32x16{};
    // The hand-over keeps 4 chunks of 16 B per lane; chunk i of lane l sits in
    // slot (i + l/4) % 4, so 16 lanes storing one chunk hit 16 bank groups.
    uint32_t* const ex = reinterpret_cast<uint32_t*>(smem + EX) + (pair * 64 + lane) * 16;
    auto exslot = [&](int i) { return 4 * ((i + (lane >> 2)) & 3); };

    // S (role P) or dP (role dS) of 32-query block qb: A = Q or dO rows.
    // Register r holds query 32*qb + 8*(r/4) + 4*hg + r%4 of the tile, key kj.
    auto scores = [&](const uint16_t* xs, int qb) __attribute__((always_inline)) -> f32x16 {
        f32x16 sacc = {};
        u32x4 fr[3];
        fr[0] = lds_row(xs + 32 * qb * D + off.row[0]);
        fr[1] = lds_row(xs + 32 * qb * D + off.row[1]);
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            if (k + 2 < NK) fr[(k + 2) % 3] = lds_row(xs + 32 * qb * D + off.row[k + 2]);
            sacc = mfma_32x32x16<T>(fr[k % 3], xr[k], sacc);
        }
        return sacc;
    };
    // acc^T += X^T W over 32-query block qb: A = transposed reads of X (dO for
    // role P, Q for role dS), B = the block's 16-bit weights w (word 4*kk + i
    // holds registers 8*kk + 2*i, +1).
    auto grads = [&](const uint16_t* xs, int qb, const uint32_t* w) __attribute__((always_inline)) {
        // all of a 16-query step's fragments are read before its MFMAs
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const u32x4 bw = {w[4 * kk], w[4 * kk + 1], w[4 * kk + 2], w[4 * kk + 3]};
            const uint16_t* xt = xs + (32 * qb + 16 * kk) * D;
            u32x4 fa[ND];
#pragma unroll
            for (int db = 0; db < ND; ++db) {
                const u32x2 lo = lds_tr(xt + off.trl[db]), hi = lds_tr(xt + off.trh[db]);
                fa[db] = u32x4{lo[0], lo[1], hi[0], hi[1]};
            }
#pragma unroll
            for (int db = 0; db < ND; ++db) acc[db] = mfma_32x32x16<T>(fa[db], bw, acc[db]);
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * ND, 2);
            __builtin_amdgcn_sched_group_barrier(0x008, ND, 2);
        }
    };

    // One 64-query tile.  live: this pair has work here; mask: hide queries
    // before key kj (causal diagonal).
    auto compute = [&](const uint16_t* qs, const uint16_t* ds, const float* st, int q0, bool live,
                       bool mask, int hstep, const uint16_t* bs, int step_no) __attribute__((always_inline)) {
        // after the hand-over barrier: the bias of step step_no+2 into this step's slot
        auto next_bias = [&]() {
            if (BIAS && step_no + 2 < steps) issue_bias(step_no + 2, step_no & 1);
        };
        if (role == 0) {
            uint32_t pw[16];
            if (live) {
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    // bias of tile rows 32qb + 8i + 4hg + j at key kj (rows past Sq read 0)
                    float bb[16];
                    if constexpr (BIAS) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int ii = 4 * qb + i;  // 8-row group of the tile
                            const u32x2 v = lds_tr(bs + (ii >> 1) * 16 * kBwRows + ((ii & 1) ? btr_hi : btr_lo));
#pragma unroll
                            for (int j = 0; j < 4; ++j) bb[4 * i + j] = bias_elem<T>(v[j >> 1], j & 1);
                        }
                    }
                    const f32x16 s = scores(qs, qb);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        // lse2 of tile rows 32*qb + 8*i + 4*hg + 0..3
                        const float* sp = st + 2 * (32 * qb + 8 * i + 4 * hg);
                        const f32x4 s01 = lds_f4(sp), s23 = lds_f4(sp + 4);
                        const float l2[4] = {s01[0], s01[2], s23[0], s23[2]};
                        float p[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float e = BIAS ? fmaf(bb[4 * i + j], kLog2e, -l2[j]) : -l2[j];
                            p[j] = fast_exp2(fmaf(s[4 * i + j], c, e));
                            if (mask) p[j] = kj > q0 + 32 * qb + 8 * i + 4 * hg + j ? 0.f : p[j];
                            // dQ must not see them; with a bias they may be anything
                            if (DQ || BIAS) p[j] = kj >= kv_lim ? 0.f : p[j];
                        }
                        pw[8 * qb + 2 * i] = pack2<T>(p[0], p[1]);
                        pw[8 * qb + 2 * i + 1] = pack2<T>(p[2], p[3]);
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    lds_st4(ex + exslot(i), u32x4{pw[4 * i], pw[4 * i + 1], pw[4 * i + 2], pw[4 * i + 3]});
            }
            lds_barrier();  // P handed over
            next_bias();
            if (live) {
                grads(ds, 0, pw);
                grads(ds, 1, pw + 8);
            }
        } else {
            f32x16 dp[2];
            if (live) {
                dp[0] = scores(ds, 0);
                dp[1] = scores(ds, 1);
            }
            lds_barrier();  // P handed over
            next_bias();
            if (live) {
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    uint32_t dw[8];
                    const u32x4 p0 = lds_ld4(ex + exslot(2 * qb)), p1 = lds_ld4(ex + exslot(2 * qb + 1));
                    const uint32_t pv[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        // delta of tile rows 32*qb + 8*i + 4*hg + 0..3
                        const float* sp = st + 2 * (32 * qb + 8 * i + 4 * hg);
                        const f32x4 s01 = lds_f4(sp), s23 = lds_f4(sp + 4);
                        const float dl[4] = {s01[1], s01[3], s23[1], s23[3]};
                        const float2 pa = unpack2<T>(pv[2 * i]), pb = unpack2<T>(pv[2 * i + 1]);
                        const f32x16& x = dp[qb];
                        dw[2 * i] = pack2<T>(pa.x * (x[4 * i] - dl[0]), pa.y * (x[4 * i + 1] - dl[1]));
                        dw[2 * i + 1] = pack2<T>(pb.x * (x[4 * i + 2] - dl[2]), pb.y * (x[4 * i + 3] - dl[3]));
                    }
                    if constexpr (DQ) {
                        // dS of queries 32*qb + 8*i + 4*hg .. +3, key l32: one 8-byte
                        // run of slot row l32 (64 queries wide, swizzled).
                        uint16_t* slot = smem + DSX + pair * 2048;
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            lds_st2(slot + l32 * 64 + (((4 * qb + i) ^ L64::f(l32)) * 8) + 4 * hg,
                                    u32x2{dw[2 * i], dw[2 * i + 1]});
                    }
                    grads(qs, qb, dw);
                }
            }
        }
        if constexpr (DQ) {
            lds_barrier();  // every live pair's dS is in its slot
            // Wave w: queries 32*(w%2) .. +31 of the tile, dims 32*(w/2) .. +31.
            const int qb3 = wave & 1, db3 = wave >> 1;
            if (db3 < ND) {
                // transposed-read offsets into a dS slot (64 queries wide)
                int slot_lo, slot_hi;
                {
                    const int g16 = lane >> 4, j16 = lane & 15;
                    const int rl = 4 * hg + (j16 >> 2), rh = rl + 8;
                    const int col = 32 * qb3 + 16 * (g16 & 1) + 4 * (j16 & 3);
                    slot_lo = rl * 64 + (((col >> 3) ^ L64::f(rl)) * 8) + (col & 7);
                    slot_hi = rh * 64 + (((col >> 3) ^ L64::f(rh)) * 8) + (col & 7);
                }
                f32x16 acc3 = {};
                bool any = false;
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) {  // 16 keys per step, 32 per pair slot
                    const int pr = kk >> 1, kp0 = k0 + 32 * pr;
                    const bool plive = kp0 < kv_lim && (!a.causal || q0 + kBwTile - 1 >= kp0);
                    if (!plive) continue;  // workgroup-uniform
                    any = true;
                    const uint16_t* sl = smem + DSX + pr * 2048 + 16 * (kk & 1) * 64;
                    const uint16_t* kb = smem + KB + 16 * kk * D;
                    const u32x2 alo = lds_tr(sl + slot_lo), ahi = lds_tr(sl + slot_hi);
                    const u32x2 blo = lds_tr(kb + off.trl[db3]), bhi = lds_tr(kb + off.trh[db3]);
                    acc3 = mfma_32x32x16<T>(u32x4{alo[0], alo[1], ahi[0], ahi[1]},
                                            u32x4{blo[0], blo[1], bhi[0], bhi[1]}, acc3);
                }
                // register r: query q0 + 32*qb3 + 8*(r/4) + 4*hg + r%4, dim 32*db3 + l32.
                // Buffer atomics over this head's [Sq, DR] accumulator: rows past
                // Sq fall outside it and are dropped; dims past DR go nowhere.
                const int dim = 32 * db3 + l32;
                if (any) {
                    const __amdgpu_buffer_rsrc_t ra = rsrc(a.dq_acc + ((int64_t)b * a.Hq + hstep) * a.Sq * DR,
                                                           (uint32_t)a.Sq * DR * 4);
                    const uint32_t base = dim < DR ? (uint32_t)((q0 + 32 * qb3 + 4 * hg) * DR + dim) * 4
                                                   : kOutside;
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(
                            acc3[r], ra, base + (uint32_t)((8 * (r >> 2) + (r & 3)) * DR * 4), 0, 0);
                }
            }
        }
    };

    // Three LDS stages: the loads of step st+2 are issued at the start of step
    // st, so each tile has two steps to arrive.
    // (BIAS: the two bias loads of step st+2, issued after them, may stay in
    // flight as well.)
    constexpr int BN = BIAS ? 2 : 0;
    auto wait_older = [&](bool last) __attribute__((always_inline)) {
        // Everything but this step's own loads has landed (vmcnt counts loads
        // in issue order; wave 0 also issued the statistics load).
        if (last) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        else if (DQ) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // atomics count too
        else if (wave == 0) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * DMA + 1 + BN) : "memory");
        else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * DMA + BN) : "memory");
    };
    // The barriers below are LDS-only: __syncthreads() would fence global
    // memory, i.e. wait for every load in flight, the newest stage's included,
    // and cut the prefetch to one step.  Each wave's own wait covers what the
    // next step reads; the barrier then covers every wave's.
    if (BIAS && steps > 0) issue_bias(0, 0);
    if (steps > 0) issue(0, 0);
    if (NSTG == 3 && steps > 1) issue(1, 1);
    if (BIAS && steps > 1) issue_bias(1, 1);
    wait_older(steps <= NSTG - 2);
    lds_barrier();
    auto step = [&](int st, const int cur) __attribute__((always_inline)) {
        if (st + NSTG - 1 < steps) issue(st + NSTG - 1, (cur + NSTG - 1) % NSTG);
        const int q0 = (qt0 + st % nqt) * kBwTile;
        const bool live = kw < kv_lim && (!a.causal || q0 + kBwTile - 1 >= kw);
        const uint16_t* base = smem + cur * STAGE;
        compute(base, base + L::TILE, reinterpret_cast<const float*>(base + 2 * L::TILE), q0, live,
                a.causal && q0 < kw + 31, gk * G + st / nqt, smem + DSX + (st & 1) * BT, st);
        wait_older(st + NSTG - 1 >= steps);
        lds_barrier();
    };
    for (int st = 0; st < steps; st += NSTG) {
        step(st, 0);
        if (st + 1 < steps) step(st + 1, 1);
        if (NSTG == 3 && st + 2 < steps) step(st + 2, 2);
    }

    // Role P: dV = P^T dO; role dS: dK = scale * (dS^T Q).  Register r of
    // d-block db holds dim 32*db + 8*(r/4) + 4*hg + r%4 of key kj.  Keys at or
    // past the batch's key limit were never visible: their gradients are 0.
    if (kj < a.Sk) {
        const bool keep = kj < kv_lim;
        const float sc = keep ? (role ? a.scale : 1.f) : 0.f;
        uint16_t* row = static_cast<uint16_t*>(role ? a.dk : a.dv) + kvh + (int64_t)kj * DR;
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f32x16& x = acc[db];
                const u32x2 w = {pack2<T>(x[4 * r4] * sc, x[4 * r4 + 1] * sc),
                                 pack2<T>(x[4 * r4 + 2] * sc, x[4 * r4 + 3] * sc)};
                const int d0 = 32 * db + 8 * r4 + 4 * hg;  // 4 dims, all < DR or none (unless ELEM)
                if constexpr (ELEM) store4_elem(row + d0, w, DR - d0);
                else if (d0 < DR) *reinterpret_cast<u32x2*>(row + d0) = w;
            }
    }
}

// ---------------------------------------------------------------------------
// Atomic variant, around the fused pass: the row statistics (what the dQ
// pass writes in the ordered variant) plus a zeroed fp32 dQ accumulator, and
// the final conversion dQ = scale * dq_acc rounded to the input type.
// ---------------------------------------------------------------------------
template <class T>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BackwardArgs a) {
    // 16 lanes per row, 8 dims each; a 16-lane group leaves together.
    const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int j = threadIdx.x & 15;
    if (row >= (int64_t)a.B * a.Hq * a.Sq) return;
    const int DR = a.D;
    float part = 0.f;
    if (8 * j < DR) {
        const uint32_t* o = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.out) + row * DR + 8 * j);
        const uint32_t* d = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.dout) + row * DR + 8 * j);
        part = dot8<T>(u32x4{d[0], d[1], d[2], d[3]}, u32x4{o[0], o[1], o[2], o[3]}, 0.f);
        float* z = a.dq_acc + row * DR + 8 * j;
        *reinterpret_cast<f32x4*>(z) = f32x4{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<f32x4*>(z + 4) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) part += __shfl_xor(part, m);
    if (j == 0) {
        const int64_t bh = row / a.Sq, i = row % a.Sq;
        const float l = a.lse[row];
        float2* st = reinterpret_cast<float2*>(a.delta) + bh * stats_stride(a.Sq) + i;
        *st = l == -INFINITY ? make_float2(INFINITY, 0.f) : make_float2(l * kLog2e, part);
    }
}

template <class T>
__global__ __launch_bounds__(256) void bwd_dq_convert_kernel(BackwardArgs a) {
    const int64_t n = (int64_t)a.B * a.Hq * a.Sq * a.D;  // a multiple of 8
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (i >= n) return;
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(a.dq_acc + i);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(a.dq_acc + i + 4);
    uint16_t* dq = static_cast<uint16_t*>(a.dq) + i;
    *reinterpret_cast<u32x2*>(dq) = u32x2{pack2<T>(x0[0] * a.scale, x0[1] * a.scale),
                                          pack2<T>(x0[2] * a.scale, x0[3] * a.scale)};
    *reinterpret_cast<u32x2*>(dq + 4) = u32x2{pack2<T>(x1[0] * a.scale, x1[1] * a.scale),
                                              pack2<T>(x1[2] * a.scale, x1[3] * a.scale)};
}

template <int D, class T, bool GEN>
hipError_t launch_backward_atomic_d(const BackwardArgs& a, hipStream_t s) {
    const int64_t rows = (int64_t)a.B * a.Hq * a.Sq;
    hipLaunchKernelGGL(bwd_prep_kernel<T>, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nkb = (a.Sk + kBwRows - 1) / kBwRows;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, T, GEN, true>), dim3(a.B * a.Hkv * nkb), dim3(kKvThreads), 0,
                       s, a, a.key_lens);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n8 = rows * a.D / 8;
    hipLaunchKernelGGL(bwd_dq_convert_kernel<T>, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int D, class T, bool GEN, bool BIAS>
hipError_t launch_backward_db(const BackwardArgs& a, hipStream_t s) {
    const int nqb = (a.Sq + kBwRows - 1) / kBwRows;
    const int nkb = (a.Sk + kBwRows - 1) / kBwRows;
    hipLaunchKernelGGL((bwd_dq_kernel<D, T, GEN, BIAS>), dim3(a.B * a.Hq * nqb), dim3(kBwThreads), 0, s,
                       a, a.key_lens);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, T, GEN, false, BIAS>), dim3(a.B * a.Hkv * nkb), dim3(kKvThreads),
                       0, s, a, a.key_lens);
    return hipGetLastError();
}

template <int D, class T, bool GEN>
hipError_t launch_backward_d(const BackwardArgs& a, hipStream_t s) {
    return a.bias ? launch_backward_db<D, T, GEN, true>(a, s) : launch_backward_db<D, T, GEN, false>(a, s);
}

// Head dims that are not multiples of 8 (ordered, no bias): the element-wise forms.
template <int D, class T>
hipError_t launch_backward_elem(const BackwardArgs& a, hipStream_t s) {
    const int nqb = (a.Sq + kBwRows - 1) / kBwRows;
    const int nkb = (a.Sk + kBwRows - 1) / kBwRows;
    hipLaunchKernelGGL((bwd_dq_kernel<D, T, true, false, true>), dim3(a.B * a.Hq * nqb), dim3(kBwThreads), 0, s,
                       a, a.key_lens);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, T, true, false, false, true>), dim3(a.B * a.Hkv * nkb),
                       dim3(kKvThreads), 0, s, a, a.key_lens);
    return hipGetLastError();
}

template <class T>
hipError_t launch_backward_t(const BackwardArgs& a, hipStream_t s) {
    if (a.D % 8 != 0) {
        if (a.bias || a.dq_acc) return hipErrorInvalidValue;
        return a.D < 64 ? launch_backward_elem<64, T>(a, s) : launch_backward_elem<128, T>(a, s);
    }
    if (a.dq_acc) {  // atomic dQ (no bias variant)
        if (a.bias) return hipErrorInvalidValue;
        if (a.D == 128) return launch_backward_atomic_d<128, T, false>(a, s);
        if (a.D == 64) return launch_backward_atomic_d<64, T, false>(a, s);
        if (a.D < 64) return launch_backward_atomic_d<64, T, true>(a, s);
        return launch_backward_atomic_d<128, T, true>(a, s);
    }
    if (a.D == 128) return launch_backward_d<128, T, false>(a, s);
    if (a.D == 64) return launch_backward_d<64, T, false>(a, s);
    // other multiples of 8: the 64- or 128-wide kernels with zero-filled chunks
    if (a.D < 64) return launch_backward_d<64, T, true>(a, s);
    return launch_backward_d<128, T, true>(a, s);
}

}  // namespace

hipError_t launch_backward_16bit(const BackwardArgs& a, bool f16, hipStream_t s) {
    if (a.D > 128) return launch_backward_wide(a, f16, s);
    if (a.D < 1 || a.D > 128) return hipErrorInvalidValue;
    return f16 ? launch_backward_t<F16T>(a, s) : launch_backward_t<Bf16T>(a, s);
}

}  // namespace sdpa
