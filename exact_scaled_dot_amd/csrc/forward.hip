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
#include <mutex>
#include <utility>
#include <vector>

#include "device_common.hpp"
#include "launch.hpp"

namespace sdpa {
namespace {

constexpr int kBr = 128;       // query rows per workgroup
constexpr int kBc = 64;        // keys per tile
constexpr int kThreads = 256;  // 4 waves of 64
// Cache-policy operand of a buffer load: non-temporal (streamed through the
// L2 with early eviction).
constexpr int kNonTemporal = 2;

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
    bool rev;  // sweep the keys last tile first (only honoured where order is free)
};

// Workgroup -> (batch, head, query block).  Workgroups are dealt to the 8
// XCDs round-robin (id % 8), and each XCD has its own L2, so the id is first
// turned into a position in a logical order in which every XCD owns one
// contiguous run.  The logical order walks K/V heads ("units") outermost and
// the Hq/Hkv query heads that share a K/V head innermost, so the workgroups
// an XCD runs together read the same K/V rows and every K/V head is fetched
// into one L2.  Under a causal mask the work of a query block grows with its
// index; there the units go in pairs and, inside a pair, query blocks run
// longest first across both units (a longest-first list schedule, which
// keeps the XCD's last workgroups short).  Without a causal mask every
// workgroup of a K/V head sweeps all its keys, and the XCD runs its
// workgroups in groups of what it holds at once: every other group sweeps
// the keys backwards (rev), so it starts on the keys the group before it
// touched last, which the L2 still holds.
__device__ __forceinline__ TileInfo decode_tile(const ForwardArgs& a) {
    const int nqb = (a.Sq + kBr - 1) / kBr;
    const int G = a.Hq / a.Hkv;
    const int units = a.B * a.Hkv;
    const int T = units * G * nqb;
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    const int nx = T >> 3, rem = T & 7;
    int t = xcd * nx + min(xcd, rem) + local;
    const int hsub = t % G;
    t /= G;
    int unit, qord;
    if (a.causal && (units & 1) == 0) {
        const int pair_member = t & 1;
        t >>= 1;
        qord = t % nqb;
        unit = 2 * (t / nqb) + pair_member;
    } else {
        qord = t % nqb;
        unit = t / nqb;
    }
    TileInfo ti;
    ti.b = unit / a.Hkv;
    ti.gk = unit % a.Hkv;
    ti.h = ti.gk * G + hsub;
    ti.q0 = (a.causal ? nqb - 1 - qord : qord) * kBr;
    ti.rev = !a.causal && a.sweep_group > 0 && ((local / a.sweep_group) & 1);
    return ti;
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
//
// Tiles reach LDS by buffer-load DMA (buffer_load_dwordx4 ... lds): each
// instruction writes 64 lanes x 16 B = 1 KB contiguously, loads past the
// buffer's num_records return zeros (keys >= Sk need no branch), and no VGPR
// holds the in-flight tile.  K and V have two LDS stages each and K runs one
// tile ahead: while tile j's weights are formed on the VALU, tile j+1's
// scores run on the MFMA unit; one barrier per tile.
//
// LDS rows are unpadded, so 16-byte chunks are XOR-swizzled instead:
//   K: chunk c of LDS row r sits at c ^ fk(r), fk(r) = (r / RPW) % (16 / RPW);
//      the 16 rows one MFMA operand read touches land in 16 distinct 16-byte
//      bank groups.
//   V: chunk c of row r sits at c ^ fv(r), fv(r) = 4 * ((r / RPW) % (4 / RPW));
//      the 4 rows x 64 B of one 32-lane transposed read are conflict free.
// (RPW = rows per 256-byte bank window: 1 for D = 128, 2 for D = 64.)
//
// The V^T operand of the second product is read with ds_read_b64_tr_b16:
// inside each 16-lane group, lane t receives element t%4 of the 8-byte chunks
// addressed by lanes t/4, 4+t/4, 8+t/4 and 12+t/4, so pointing lane j at
// V[k0 + j/4][d0 + 4*(j%4)] hands lane t the four keys V[k0..k0+3][d0 + t].
// ---------------------------------------------------------------------------
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

// The __restrict__ parameter gives the inlined read its own alias scope, which
// keeps the compiler from putting a vmcnt(0) drain of the in-flight LDS-DMA
// writes in front of it (the explicit waits and barriers order those).
__device__ __forceinline__ u32x2 lds_read_tr16x4(const uint16_t* __restrict__ p) {
    lds_i16x4* lp = (lds_i16x4*)((__attribute__((address_space(3))) char*)p);
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(lp));
}

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at
// lds + 16*l (the destination is wave-uniform; M0 carries it).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint16_t* lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (lds_void*)((__attribute__((address_space(3))) char*)lds), 16, voff, 0, 0, 0);
}

// Same with a wave-uniform scalar offset added to the address.  The buffer
// range check covers voff but not soff.
__device__ __forceinline__ void dma16s(__amdgpu_buffer_rsrc_t r, uint16_t* lds, uint32_t voff,
                                       uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (lds_void*)((__attribute__((address_space(3))) char*)lds), 16, voff, soff, 0, 0);
}

// 32-bit LDS store / 4 x 32-bit load with an alias scope of their own (see
// lds_read_tr16x4).
__device__ __forceinline__ void lds_store_i32(int* __restrict__ p, int v) {
    *(__attribute__((address_space(3))) int*)((__attribute__((address_space(3))) char*)p) = v;
}
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 lds_load_i32x4(const int* __restrict__ p) {
    return *(const __attribute__((address_space(3))) i32x4*)(
        (const __attribute__((address_space(3))) char*)p);
}

// Raw buffer resource over [base, base + bytes); loads beyond it return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

template <int D>
struct Bf16Geo {
    static constexpr int CPR = D / 8;                // 16-byte chunks per row
    static constexpr int RPW = D > 128 ? 1 : 256 / (2 * D);  // rows per 256-byte bank window (1: a row spans two)
    static constexpr int TILE = kBc * D;             // bf16 elements per K or V tile
    static constexpr int STAGE = 2 * TILE;           // K tile then V tile
    static constexpr int DMA = TILE * 2 / 1024 / 4;  // 1-KB DMA loads per wave per tensor
    __device__ static int fk(int r) { return (r / RPW) % (16 / RPW); }
    __device__ static int fv(int r) { return 4 * ((r / RPW) % (4 / RPW)); }
};

// PAGED: prefill chunks over a page cache.  Workgroup = (sequence, head,
// 128-row block of the sequence's chunk); the chunk's rows are packed rows
// cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1 of q / out ([rows, Hq, D]) and row i
// sits at absolute position seq_lens[s] - n_s + i (n_s = chunk length).  In a
// 64-key tile wave w loads keys 16w .. 16w+15, which lie in one page (page
// size a multiple of 16): one table lookup per wave and tile, a buffer
// resource over that page, the wave-uniform row offset in the scalar offset.
// A table entry outside the cache is never read; its 16 keys are hidden
// (validity shared through LDS).
//
// BIAS (dense only): an additive mask tile is added to the scaled scores.
// Lane (row qi, half hg) holds keys 16g + 8hg .. +7 (g = 0..3) of a tile, so
// it loads those four 16-byte runs of its bias row (one tile ahead, next to
// the DMA issue) and adds bias / scale in raw-score units during the mask
// step; every visited tile takes the mask step.
//
// DV < D (head dims above 128): the workgroup computes the scores over all D
// dims but only the DV output dims of slice blockIdx.y (V columns
// DV*y .. DV*y + DV - 1), so the registers hold D-wide Q fragments and a
// DV-wide output; the slices of a query block recompute its scores.
//
// ELEM (with GEN; head dims that are not multiples of 8): rows of such a
// width do not start on 16-byte boundaries, and a row's last 16-byte chunk
// would carry the next row's first elements, so Q, K and V are read one
// element at a time (2-byte buffer loads; elements past the row read as
// zeros through the same out-of-range offsets) and each 16-byte LDS slot is
// written by the lane the DMA would have filled it with, in the same
// layout; the output is stored element by element.  The loads are waited
// for where they are written: no prefetch across steps on this path.
template <int D, bool PAGED, class T, bool BIAS = false, bool GEN = false, int DV = D, bool ELEM = false>
__global__ __launch_bounds__(kThreads, D > 128 ? 1 : 2) void forward_bf16_kernel(
    ForwardArgs a, PagedArgs p, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cu_q) {
    using L = Bf16Geo<D>;    // K tiles
    using LV = Bf16Geo<DV>;  // V tiles (the slice)
    // Two K stages then two V stages.  K runs one tile ahead of V: while the
    // weights of tile j are formed, the scores of tile j+1 are computed.
    // (Paged: then the validity of each K stage's four 16-key groups.)
    constexpr int VBASE = 2 * L::TILE;  // first V stage
    __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * L::TILE + 2 * LV::TILE + (PAGED ? 16 : 0)];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hg = lane >> 5;  // which half of the wave

    const TileInfo ti = decode_tile(a);
    // Head dim in memory: DR (GEN: a multiple of 8 below D; else D).  Rows are
    // DR wide in HBM and D wide on chip; the 16-byte chunks at or past DR are
    // read as zeros (their offsets lie outside the buffer) and never stored.
    const int DR = GEN ? a.D : D;
    // Value head dim in memory: DVM (GEN: a.Dv, which may differ from D; else
    // D).  Output slice: dims dv0 .. dv0 + DRV - 1 of the DVM (one slice of DV
    // dims per blockIdx.y).
    const int DVM = GEN ? a.Dv : DR;
    const int dv0 = DV * (int)blockIdx.y;
    const int DRV = min(DV, DVM - dv0);
    constexpr uint32_t kOut = 0x80000000u;  // past any num_records (<= INT_MAX)
    const uint16_t* kp;
    const uint16_t* vp;
    const uint16_t* qbase;
    uint16_t* op;
    int nrows, qoff, kv_lim, kv_end;
    int r0 = 0;        // paged: first packed row of the chunk
    uint32_t qstride;  // bytes between consecutive query rows
    uint32_t ostride;  // bytes between consecutive output rows
    if (PAGED) {
        // This workgroup's rows of sequence b's chunk (bounds clamped to the
        // packed rows so no store can leave out).
        r0 = min(max(cu_q[ti.b], 0), p.total_q);
        const int r1 = min(max(cu_q[ti.b + 1], r0), p.total_q);
        nrows = r1 - r0;
        if (ti.q0 >= nrows) return;  // the whole workgroup: no barrier reached yet
        kv_lim = min(seq_lens[ti.b], a.Sk);
        qoff = kv_lim - nrows;  // absolute position of the chunk's first row
        kv_end = kv_lim;
        if (a.causal) kv_end = min(kv_end, qoff + ti.q0 + kBr);
        const int64_t rb = (int64_t)r0 * a.Hq + ti.h;
        qbase = static_cast<const uint16_t*>(a.q) + rb * DR;
        op = static_cast<uint16_t*>(a.out) + rb * DVM;
        qstride = (uint32_t)a.Hq * DR * 2;
        ostride = (uint32_t)a.Hq * DVM * 2;
        kp = static_cast<const uint16_t*>(a.k);
        vp = static_cast<const uint16_t*>(a.v);
    } else {
        const int64_t bh = (int64_t)ti.b * a.Hq + ti.h;
        const int64_t kvh = ((int64_t)ti.b * a.Hkv + ti.gk) * a.Sk;
        kp = static_cast<const uint16_t*>(a.k) + kvh * DR;
        vp = static_cast<const uint16_t*>(a.v) + kvh * DVM;
        qbase = static_cast<const uint16_t*>(a.q) + bh * a.Sq * DR;
        op = static_cast<uint16_t*>(a.out) + bh * a.Sq * DVM;
        qstride = (uint32_t)DR * 2;
        ostride = (uint32_t)DVM * 2;
        nrows = a.Sq;
        qoff = 0;
        key_extent(a, ti.b, ti.q0, kv_lim, kv_end);
    }

    const int qw = ti.q0 + wave * 32;  // first query row of this wave
    const int qi = qw + l32;           // this lane's query row
    const int ntiles = kv_end > 0 ? (kv_end + kBc - 1) / kBc : 0;
    // Under a causal mask a wave stops taking part once a tile starts past
    // its last row (and never resumes: tiles only move forward).
    const int wave_tiles = a.causal ? max(0, min(ntiles, (qoff + qw + 31) / kBc + 1)) : ntiles;

    // Q fragment for the B operand of S^T = K Q^T: lane holds Q[qi][16t + 8hg .. +7]
    // (rows >= nrows read as zeros).
    // Without a causal mask (dense) Q is read non-temporally: it is read once,
    // and the XCD's L2 is better spent keeping the K/V rows the next
    // workgroups sweep (see decode_tile).
    const bool stream_q_o = !PAGED && !a.causal && !ELEM;
    u32x4 qr[D / 16];
    {
        const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qbase, (uint32_t)nrows * qstride);
        if constexpr (ELEM) {
#pragma unroll
            for (int t = 0; t < D / 16; ++t) {
                const int d0 = 16 * t + 8 * hg;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const int e0 = d0 + 2 * w;
                    const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(
                        qrs, e0 < DR ? qi * qstride + e0 * 2 : kOut, 0, 0);
                    const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(
                        qrs, e0 + 1 < DR ? qi * qstride + e0 * 2 + 2 : kOut, 0, 0);
                    qr[t][w] = lo | (hi << 16);
                }
            }
        } else if (stream_q_o) {
#pragma unroll
            for (int t = 0; t < D / 16; ++t) {
                const int d0 = 16 * t + 8 * hg;
                qr[t] = __builtin_amdgcn_raw_buffer_load_b128(qrs, d0 < DR ? qi * qstride + d0 * 2 : kOut,
                                                              0, kNonTemporal);
            }
        } else {
#pragma unroll
            for (int t = 0; t < D / 16; ++t) {
                const int d0 = 16 * t + 8 * hg;
                qr[t] = __builtin_amdgcn_raw_buffer_load_b128(qrs, d0 < DR ? qi * qstride + d0 * 2 : kOut,
                                                              0, 0);
            }
        }
    }

    // Bias: a resource over this (batch, head)'s [Sq, Sk] slice (rows >= Sq
    // and keys >= Sk read as 0); bq holds the four 16-byte runs of the next
    // tile to be masked.
    u32x4 bq[4];
    const __amdgpu_buffer_rsrc_t brs = make_rsrc(
        BIAS ? static_cast<const uint16_t*>(a.bias) + ti.b * a.bias_sb + ti.h * a.bias_sh : qbase,
        BIAS ? (uint32_t)a.Sq * a.Sk * 2 : 0u);
    const uint32_t brow = BIAS ? (uint32_t)qi * a.Sk * 2 + 16 * hg : 0u;
    auto load_bias = [&](int j0) __attribute__((always_inline)) {
        if constexpr (BIAS) {
#pragma unroll
            for (int g = 0; g < 4; ++g)
                bq[g] = __builtin_amdgcn_raw_buffer_load_b128(brs, brow + (uint32_t)(j0 + 16 * g) * 2, 0, 0);
        }
    };

    // DMA source offsets (bytes, relative to the tile's first key).  DMA load i
    // of this wave fills LDS bytes [1024*(DMA*wave + i), +1024) of a tile;
    // lane l's 16 B land at 16-byte slot p = 64*(DMA*wave + i) + l.
    // (Paged: relative to the wave's 16-key group, rows Hkv*D*2 bytes apart.)
    // The wave's LDS rows are 16*wave .. 16*wave+15, i.e. keys of the same group.
    const uint32_t row_bytes = PAGED ? (uint32_t)a.Hkv * DR * 2 : (uint32_t)DR * 2;
    const uint32_t vrow_bytes = PAGED ? (uint32_t)a.Hkv * DVM * 2 : (uint32_t)DVM * 2;
    const int row_base = PAGED ? 16 * wave : 0;
    uint32_t koff[L::DMA], voff[LV::DMA];
    int kvn[ELEM ? L::DMA : 1], vvn[ELEM ? LV::DMA : 1];  // ELEM: elements of the slot inside the row
#pragma unroll
    for (int i = 0; i < L::DMA; ++i) {
        const int q = 64 * (L::DMA * wave + i) + lane;
        const int row = q / L::CPR, pc = q % L::CPR;
        const int ck = pc ^ L::fk(row);  // logical chunk
        koff[i] = 8 * ck < DR ? (k_lds_row(row) - row_base) * row_bytes + ck * 16 : kOut;
        if constexpr (ELEM) kvn[i] = min(8, max(0, DR - 8 * ck));
    }
#pragma unroll
    for (int i = 0; i < LV::DMA; ++i) {
        const int q = 64 * (LV::DMA * wave + i) + lane;
        const int row = q / LV::CPR, pc = q % LV::CPR;
        const int cv = pc ^ LV::fv(row);  // logical chunk of the slice
        voff[i] = 8 * cv < DRV ? (row - row_base) * vrow_bytes + (dv0 + 8 * cv) * 2 : kOut;
        if constexpr (ELEM) vvn[i] = min(8, max(0, DRV - 8 * cv));
    }
    // ELEM: the 16 bytes of one slot from 2-byte loads (elements past the row,
    // and whole slots at kOut, read as zeros).
    auto elem_slot = [&](__amdgpu_buffer_rsrc_t r, uint32_t off, int valid, uint32_t soff) -> u32x4 {
        u32x4 v;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(r, 2 * w < valid ? off + 4 * w : kOut, soff, 0);
            const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(r, 2 * w + 1 < valid ? off + 4 * w + 2 : kOut, soff, 0);
            v[w] = lo | (hi << 16);
        }
        return v;
    };
    // Paged: resource over the page of keys j0 + 16*wave .. +15 (zero records
    // when the table entry is outside the cache) and the group's scalar
    // offset inside it; the validity goes to LDS for the mask.
    int* const kvalid = reinterpret_cast<int*>(smem + VBASE + 2 * LV::TILE);  // [K stage][group]
    // The lookup for a tile is made when its K is issued and kept (per K
    // stage) for its V, issued one step later.
    int64_t pg_off[2] = {0, 0}, vpg_off[2] = {0, 0};
    uint32_t pg_bytes[2] = {0u, 0u}, pg_soff[2] = {0u, 0u};
    uint32_t vpg_bytes[2] = {0u, 0u}, vpg_soff[2] = {0u, 0u};
    auto page_of = [&](int j0, int stage) -> bool {
        const int key = j0 + 16 * wave;
        const int lp = key / p.page_size;
        const int pg = lp < p.max_pages ? tables[(int64_t)ti.b * p.max_pages + lp] : -1;
        const bool ok = pg >= 0 && pg < p.pages;
        pg_off[stage] = ok ? (int64_t)pg * p.page_size * a.Hkv * DR : 0;
        pg_bytes[stage] = ok ? (uint32_t)p.page_size * row_bytes : 0u;
        pg_soff[stage] = ((uint32_t)(key % p.page_size) * a.Hkv + ti.gk) * DR * 2;
        vpg_off[stage] = ok ? (int64_t)pg * p.page_size * a.Hkv * DVM : 0;
        vpg_bytes[stage] = ok ? (uint32_t)p.page_size * vrow_bytes : 0u;
        vpg_soff[stage] = ((uint32_t)(key % p.page_size) * a.Hkv + ti.gk) * DVM * 2;
        return ok;
    };
    // Dense: resources start at the tile's first key; num_records ends at key Sk.
    auto issue_k = [&](int j0, int stage) {
        uint16_t* dst = smem + stage * L::TILE + 512 * L::DMA * wave;
        if (PAGED) {
            const bool ok = page_of(j0, stage);
            const __amdgpu_buffer_rsrc_t rk = make_rsrc(kp + pg_off[stage], pg_bytes[stage]);
            if constexpr (ELEM) {
#pragma unroll
                for (int i = 0; i < L::DMA; ++i)
                    *reinterpret_cast<u32x4*>(dst + 512 * i + 8 * lane) =
                        elem_slot(rk, koff[i], kvn[i], pg_soff[stage]);
            } else {
#pragma unroll
                for (int i = 0; i < L::DMA; ++i) dma16s(rk, dst + 512 * i, koff[i], pg_soff[stage]);
            }
            if (lane == 0) lds_store_i32(kvalid + 4 * stage + wave, ok ? 1 : 0);
        } else {
            const __amdgpu_buffer_rsrc_t rs =
                make_rsrc(kp + (int64_t)j0 * DR, (uint32_t)(a.Sk - j0) * DR * 2);
            if constexpr (ELEM) {
#pragma unroll
                for (int i = 0; i < L::DMA; ++i)
                    *reinterpret_cast<u32x4*>(dst + 512 * i + 8 * lane) = elem_slot(rs, koff[i], kvn[i], 0u);
            } else {
#pragma unroll
                for (int i = 0; i < L::DMA; ++i) dma16(rs, dst + 512 * i, koff[i]);
            }
        }
    };
    auto issue_v = [&](int j0, int stage) {
        uint16_t* dst = smem + VBASE + stage * LV::TILE + 512 * LV::DMA * wave;
        if (PAGED) {
            // K of this tile went to K stage (j0 / kBc) % 2 with the lookup.
            const int ks = (j0 / kBc) & 1;
            const __amdgpu_buffer_rsrc_t rv = make_rsrc(vp + vpg_off[ks], vpg_bytes[ks]);
            if constexpr (ELEM) {
#pragma unroll
                for (int i = 0; i < LV::DMA; ++i)
                    *reinterpret_cast<u32x4*>(dst + 512 * i + 8 * lane) =
                        elem_slot(rv, voff[i], vvn[i], vpg_soff[ks]);
            } else {
#pragma unroll
                for (int i = 0; i < LV::DMA; ++i) dma16s(rv, dst + 512 * i, voff[i], vpg_soff[ks]);
            }
        } else {
            const __amdgpu_buffer_rsrc_t rs =
                make_rsrc(vp + (int64_t)j0 * DVM, (uint32_t)(a.Sk - j0) * DVM * 2);
            if constexpr (ELEM) {
#pragma unroll
                for (int i = 0; i < LV::DMA; ++i)
                    *reinterpret_cast<u32x4*>(dst + 512 * i + 8 * lane) = elem_slot(rs, voff[i], vvn[i], 0u);
            } else {
#pragma unroll
                for (int i = 0; i < LV::DMA; ++i) dma16(rs, dst + 512 * i, voff[i]);
            }
        }
    };

    // Lane-constant LDS read offsets (bf16 elements).
    // K operand: LDS row 32*kb2 + l32, logical chunk 2t + hg.
    int krd[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) krd[t] = l32 * D + (((2 * t + hg) ^ L::fk(l32)) * 8);
    // V^T operand: row 16*kk + tr_row (+4), element column 32*db + tr_col.
    const int g16 = lane >> 4, j16 = lane & 15;
    const int tr_row = 8 * hg + (j16 >> 2);
    const int tr_col = 16 * (g16 & 1) + 4 * (j16 & 3);
    int vrd[DV / 32];
#pragma unroll
    for (int db = 0; db < DV / 32; ++db) {
        const int col = 32 * db + tr_col;
        vrd[db] = tr_row * DV + (((col >> 3) ^ LV::fv(tr_row)) * 8) + (col & 7);
    }

    f32x16 oacc[DV / 32];
#pragma unroll
    for (int db = 0; db < DV / 32; ++db) oacc[db] = f32x16{};
    float m_run = -INFINITY;  // reference max of row qi (raw score units)
    float l_run = 0.f;        // this lane's share of the running denominator
    const float c = a.scale * kLog2e;
    // The reference max moves only when a row's tile max exceeds it by more
    // than 8 in log2 units; weights then stay <= 2^8 and O / l is unchanged.
    const float tau = 8.0f / c;

    // S^T tile of the K stage at ks: register r of s[kb2] holds key
    // 32*kb2 + 16*(r/8) + 8*hg + r%8 of the tile.
    auto scores = [&](const uint16_t* ks, f32x16 (&sacc)[2]) __attribute__((always_inline)) {
        // K fragments are read two k-steps ahead of the MFMAs that use them.
        constexpr int NK = D / 16;  // contraction steps
        u32x4 kf[3][2];
        auto rd = [&](int t, int slot) __attribute__((always_inline)) {
            kf[slot][0] = *reinterpret_cast<const u32x4*>(ks + krd[t]);
            kf[slot][1] = *reinterpret_cast<const u32x4*>(ks + 32 * D + krd[t]);
        };
        rd(0, 0);
        rd(1, 1);
        sacc[0] = f32x16{};
        sacc[1] = f32x16{};
#pragma unroll
        for (int t = 0; t < NK; ++t) {
            if (t + 2 < NK) rd(t + 2, (t + 2) % 3);
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
                sacc[kb2] = mfma_32x32x16<T>(kf[t % 3][kb2], qr[t], sacc[kb2]);
        }
        // Keep the read-ahead: 4 reads, then (2 MFMAs, 2 reads) per k-step.
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
        for (int t = 0; t < NK; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
            if (t + 2 < NK) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
        }
    };

    // Hide keys of tile j0 that a row may not see (causal / key limit).
    // Row qi sits at absolute position qoff + qi (dense: qoff = 0).  Paged:
    // keys of a 16-key group whose table entry is invalid are hidden too.
    // Paged: bit g of a tile's validity word says keys 16g .. 16g+15 come from
    // a valid page; read once the tile's K issue is behind a barrier.
    auto tile_validity = [&](int j0) -> int {
        if (!PAGED) return 15;
        const i32x4 vg = lds_load_i32x4(kvalid + 4 * ((j0 / kBc) & 1));
        return __builtin_amdgcn_readfirstlane((vg[0] ? 1 : 0) | (vg[1] ? 2 : 0) | (vg[2] ? 4 : 0) |
                                              (vg[3] ? 8 : 0));
    };
    auto mask_tile = [&](int j0, f32x16 (&sacc)[2], int vmask) __attribute__((always_inline)) {
        bool need_mask = (a.causal && j0 + kBc - 1 > qoff + qw) || (j0 + kBc > kv_lim);
        if (PAGED) need_mask = need_mask || vmask != 15;
        if constexpr (BIAS) {
            // score + bias / scale, then the causal / key-limit hiding on
            // every element: one per-lane limit per tile (first hidden key
            // offset) against the element's constant key offset.
            const float inv_scale = 1.f / a.scale;
            const int lim = (a.causal ? min(kv_lim, qi + 1) : kv_lim) - j0 - 8 * hg;
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int g = 2 * kb2 + (r >> 3), e = r & 7;
                    const float bv = fmaf(bias_elem<T>(bq[g][e >> 1], e & 1), inv_scale, sacc[kb2][r]);
                    sacc[kb2][r] = (32 * kb2 + 16 * (r >> 3) + (r & 7) >= lim) ? -INFINITY : bv;
                }
        } else if (need_mask) {
            if constexpr (PAGED) {
                // A group on an invalid page gets a -inf bias (wave-uniform, so
                // this stays straight-line code: an add and a select per score).
                float gbias[4];
#pragma unroll
                for (int g = 0; g < 4; ++g) gbias[g] = ((vmask >> g) & 1) ? 0.f : -INFINITY;
#pragma unroll
                for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = j0 + 32 * kb2 + 16 * (r >> 3) + 8 * hg + (r & 7);
                        const bool hide = key >= kv_lim || (a.causal && key > qoff + qi);
                        const float v = sacc[kb2][r] + gbias[2 * kb2 + (r >> 3)];
                        sacc[kb2][r] = hide ? -INFINITY : v;
                    }
            } else {
#pragma unroll
                for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = j0 + 32 * kb2 + 16 * (r >> 3) + 8 * hg + (r & 7);
                        const bool hide = key >= kv_lim || (a.causal && key > qi);
                        if (hide) sacc[kb2][r] = -INFINITY;
                    }
            }
        }
    };
    // Row max of a (masked) score tile; moves the reference max when needed.
    auto update_max = [&](const f32x16 (&sacc)[2]) __attribute__((always_inline)) {
        // A tree of 3-input maxima (32 -> 11 -> 4 -> 1), then the partner half-wave.
        const float* sv = reinterpret_cast<const float*>(sacc);
        float m11[11];
#pragma unroll
        for (int g = 0; g < 10; ++g) m11[g] = max3f(sv[3 * g], sv[3 * g + 1], sv[3 * g + 2]);
        m11[10] = fmaxf(sv[30], sv[31]);
        const float m4a = max3f(m11[0], m11[1], m11[2]), m4b = max3f(m11[3], m11[4], m11[5]);
        const float m4c = max3f(m11[6], m11[7], m11[8]), m4d = fmaxf(m11[9], m11[10]);
        float mx = max3f(m4a, m4b, fmaxf(m4c, m4d));
        mx = max_half_waves(mx);
        if (__any(mx > m_run + tau)) {  // wave-uniform: move the reference max
            const float m_new = fmaxf(m_run, mx);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = fast_exp2((m_run - m_use) * c);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DV / 32; ++db) oacc[db] *= alpha;
        }
    };
    // bf16 weights of a score tile against the reference max; the denominator
    // sums the rounded weights (v_dot2 with (1, 1)), i.e. exactly the weights
    // multiplied into V.  Straight-line code.
    auto weights = [&](const f32x16 (&sacc)[2], uint32_t (&pk)[2][8]) __attribute__((always_inline)) -> float {
        const float neg = -((m_run == -INFINITY) ? 0.f : m_run) * c;
        float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = fast_exp2(fmaf(sacc[kb2][r], c, neg));
                const float p1 = fast_exp2(fmaf(sacc[kb2][r + 1], c, neg));
                pk[kb2][r >> 1] = pack2<T>(p0, p1);
                if (r & 2) ps1 = sum2<T>(pk[kb2][r >> 1], ps1);
                else ps0 = sum2<T>(pk[kb2][r >> 1], ps0);
            }
        return ps0 + ps1;
    };

    // O^T += V^T P^T over the four 16-key slices of the V stage at vs.
    auto accumulate = [&](const uint16_t* vs, const uint32_t (&pk)[2][8]) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int kb2 = kk >> 1, half = kk & 1;
            const u32x4 pw = {pk[kb2][4 * half], pk[kb2][4 * half + 1], pk[kb2][4 * half + 2],
                              pk[kb2][4 * half + 3]};
            // all of a 16-key slice's V^T fragments are read before its MFMAs
            // (each pair read right before its MFMA exposed the read latency)
            u32x4 vf[DV / 32];
#pragma unroll
            for (int db = 0; db < DV / 32; ++db) {
                const uint16_t* vb = vs + 16 * kk * DV + vrd[db];
                const u32x2 lo = lds_read_tr16x4(vb);
                const u32x2 hi = lds_read_tr16x4(vb + 4 * DV);
                vf[db] = u32x4{lo[0], lo[1], hi[0], hi[1]};
            }
#pragma unroll
            for (int db = 0; db < DV / 32; ++db) oacc[db] = mfma_32x32x16<T>(vf[db], pw, oacc[db]);
            __builtin_amdgcn_sched_group_barrier(0x100, DV / 16, 4);
            __builtin_amdgcn_sched_group_barrier(0x008, DV / 32, 4);
        }
    };

    // First key of the jt-th tile visited: tiles in order, or last first
    // when this workgroup sweeps backwards (dense, no causal mask: every
    // tile is visited, and the softmax does not depend on the order).
    const bool rev = !PAGED && ti.rev;
    auto tkey = [&](int jt) __attribute__((always_inline)) {
        return (rev ? ntiles - 1 - jt : jt) * kBc;
    };

    // Prologue: K(0), V(0), K(1) resident; scores of tile 0.
    if (ntiles > 0) {
        issue_k(tkey(0), 0);
        issue_v(tkey(0), 0);
    }
    if (ntiles > 1) issue_k(tkey(1), 1);
    if (ntiles > 0) load_bias(tkey(0));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    f32x16 sA[2], sB[2];
    if (wave_tiles > 0) {
        scores(smem, sA);
        mask_tile(tkey(0), sA, tile_validity(tkey(0)));
    }
    __syncthreads();  // K stage 0 is refilled with K(2) by the first step

    // Tile jt: K(jt+1) sits in K stage cur^1, V(jt) in V stage cur.  Issue
    // K(jt+2) into K stage cur and V(jt+1) into V stage cur^1, compute the
    // scores of tile jt+1 next to the weights of tile jt, then P V.  Both
    // calls below pass literal stages, so after inlining every LDS read
    // carries its stage base as an instruction offset and the two score
    // tiles swap roles without copies.
    auto step = [&](int jt, const int cur, f32x16 (&scur)[2], f32x16 (&snext)[2]) __attribute__((always_inline)) {
        // Tile jt+1's validity (written when its K was issued, a barrier ago);
        // K(jt+2)'s goes to the other slot.
        const int vnext = tile_validity(tkey(jt + 1));
        if (jt + 2 < ntiles) issue_k(tkey(jt + 2), cur);
        if (jt + 1 < ntiles) issue_v(tkey(jt + 1), cur ^ 1);
        if (BIAS && jt + 1 < wave_tiles) load_bias(tkey(jt + 1));
        if (jt < wave_tiles) {
            uint32_t pk[2][8];
            if (jt + 1 < wave_tiles) scores(smem + (cur ^ 1) * L::TILE, snext);
            // Weights against the current reference max.  They are >= 0, so a
            // lane sum <= 2^8 bounds every weight by 2^8, the lazy-rescale
            // bound; only otherwise (or before the first max) look at the
            // tile max and maybe move the reference.
            float ps = weights(scur, pk);
            if (__any(ps > 256.f || m_run == -INFINITY)) {
                update_max(scur);
                ps = weights(scur, pk);
            }
            l_run += ps;
            accumulate(smem + VBASE + cur * LV::TILE, pk);
            if (jt + 1 < wave_tiles) mask_tile(tkey(jt + 1), snext, vnext);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's DMA landed
        __syncthreads();
    };
    for (int jt = 0; jt < ntiles; jt += 2) {
        step(jt, 0, sA, sB);
        if (jt + 1 < ntiles) step(jt + 1, 1, sB, sA);
    }

    // Epilogue: O = O_acc / l, rounded to bf16.  Register r of d-block db holds
    // dim 32*db + 8*(r/4) + 4*hg + r%4 of row qi.
    const float lt = l_run + swap_half_wave(l_run);
    const float inv = 1.f / lt;
    // Optional log-sum-exp of the row (natural log, scaled-score units) for
    // the backward: the reference max plus ln of the denominator; -inf for a
    // row with no visible key.
    // (Dense: lse [B, Hq, Sq]; paged: [packed rows, Hq].)
    if (a.lse && hg == 0 && qi < nrows && dv0 == 0)
        a.lse[PAGED ? (int64_t)(r0 + qi) * a.Hq + ti.h : ((int64_t)ti.b * a.Hq + ti.h) * a.Sq + qi] =
            m_run == -INFINITY ? -INFINITY : m_run * a.scale + __logf(lt);
    if (stream_q_o) {
        // The wave's 32 output rows go through LDS (free: every wave has passed
        // the last tile's barrier) and out as whole 16-byte runs, a row's DV
        // dims by consecutive lanes, with non-temporal stores: whole lines,
        // kept from displacing K/V rows in the L2.  16-byte chunk c of LDS
        // row r sits at c ^ (r % CPR).
        constexpr int CPR = DV / 8;  // 16-byte chunks per row
        uint16_t* stage = smem + wave * 32 * DV;
#pragma unroll
        for (int db = 0; db < DV / 32; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const u32x2 w = {pack2<T>(oacc[db][4 * r4] * inv, oacc[db][4 * r4 + 1] * inv),
                                 pack2<T>(oacc[db][4 * r4 + 2] * inv, oacc[db][4 * r4 + 3] * inv)};
                const int pc = (4 * db + r4) ^ (l32 % CPR);
                *reinterpret_cast<u32x2*>(stage + l32 * DV + 8 * pc + 4 * hg) = w;
            }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's own rows are in LDS
#pragma unroll
        for (int it = 0; it < 32 * CPR / 64; ++it) {
            const int idx = 64 * it + lane;
            const int row = idx / CPR, cc = idx % CPR;
            const u32x4 v = *reinterpret_cast<const u32x4*>(stage + row * DV + 8 * (cc ^ (row % CPR)));
            if (qw + row < nrows && 8 * cc < DRV)  // 8 dims of the slice, all < DRV or none
                __builtin_nontemporal_store(
                    v, reinterpret_cast<u32x4*>(op + (int64_t)(qw + row) * (ostride / 2) + dv0 + 8 * cc));
        }
    } else if (qi < nrows) {
        uint16_t* orow = op + (int64_t)qi * (ostride / 2) + dv0;
#pragma unroll
        for (int db = 0; db < DV / 32; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const u32x2 w = {pack2<T>(oacc[db][4 * r4] * inv, oacc[db][4 * r4 + 1] * inv),
                                 pack2<T>(oacc[db][4 * r4 + 2] * inv, oacc[db][4 * r4 + 3] * inv)};
                const int d0 = 32 * db + 8 * r4 + 4 * hg;  // 4 dims of the slice, all < DRV or none
                if constexpr (ELEM) {  // element by element: the row need not be 8-byte aligned
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (d0 + e < DRV) orow[d0 + e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
                } else if (d0 < DRV) {
                    *reinterpret_cast<u32x2*>(orow + d0) = w;
                }
            }
    }
}

// ---------------------------------------------------------------------------
// Head dims above 128 and up to 256 (16-bit, dense, no bias) on paired waves.
// A workgroup of 8 waves owns 128 query rows of one (batch, head); waves w
// and w + 4 share rows 32*(w%4) .. +31 and split the head dim: wave w owns
// dims 0..127, wave w + 4 dims 128..255 (of both Q.K and the output).  Per
// 32-key tile each wave forms the partial scores S^T over its dims (the
// layout of forward_bf16_kernel, K rows from LDS), hands them to its partner
// through LDS, adds the partner's, and both waves of a pair then run the
// same online softmax on the full scores (the fp32 sum a + b is the same
// in either order) and form their own 128 output dims, O^T += V^T P^T.
// Every product is thus computed once (the two-slice form recomputes the
// scores in each slice), each wave holds a 128-dim Q and O like the 128-wide
// kernel (two waves per SIMD), and K and V tiles (all 256 dims) are shared
// by the 8 waves.  The partial scores run one tile ahead: step j forms the
// partial scores of tile j + 1 beside tile j's softmax and P.V, so the
// MFMA and exponential work of one wave overlap; the hand-over slots
// alternate between two buffers by tile, and one barrier per step covers
// both the hand-over and the K/V tiles (two LDS stages each, loaded a step
// ahead).
// ---------------------------------------------------------------------------
constexpr int kPairThreads = 512;
constexpr int kPairKeys = 32;

template <class T, bool GEN = false>
__global__ __launch_bounds__(kPairThreads, 1) void forward_pair_kernel(ForwardArgs a) {
    constexpr int D = 256;
    constexpr int KT = kPairKeys;
    using L = Bf16Geo<D>;
    constexpr int TILE = KT * D;                   // 16-bit elements per K or V tile
    constexpr int DMA = TILE * 2 / 1024 / 8;       // 1-KB DMA loads per wave per tensor
    constexpr int XF = 64 * 16;                    // floats of one wave's partial scores
    static_assert(DMA == 2, "tile geometry");
    // K stage s at s*TILE, V stage s at (2+s)*TILE, then two hand-over buffers.
    __shared__ __attribute__((aligned(1024))) uint16_t smem[4 * TILE + 2 * 8 * XF * 2];
    float* const xch = reinterpret_cast<float*>(smem + 4 * TILE);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hg = lane >> 5;
    const int rb = wave & 3, dh = wave >> 2;  // row block, head-dim half
    const TileInfo ti = decode_tile(a);
    const int DR = GEN ? a.D : D;  // head dim in memory
    constexpr uint32_t kOut = 0x80000000u;
    const int64_t bh = (int64_t)ti.b * a.Hq + ti.h;
    const int64_t kvh = ((int64_t)ti.b * a.Hkv + ti.gk) * a.Sk * DR;
    const uint16_t* kp = static_cast<const uint16_t*>(a.k) + kvh;
    const uint16_t* vp = static_cast<const uint16_t*>(a.v) + kvh;
    const uint16_t* qbase = static_cast<const uint16_t*>(a.q) + bh * a.Sq * DR;
    uint16_t* op = static_cast<uint16_t*>(a.out) + bh * a.Sq * DR;
    int kv_lim, kv_end;
    key_extent(a, ti.b, ti.q0, kv_lim, kv_end);
    const int qw = ti.q0 + 32 * rb;  // first row of this wave (and its partner)
    const int qi = qw + l32;
    const int ntiles = kv_end > 0 ? (kv_end + KT - 1) / KT : 0;
    const int wave_tiles = a.causal ? max(0, min(ntiles, (qw + 31) / KT + 1)) : ntiles;

    // Q of this wave's dims as B operands: lane holds Q[qi][128*dh + 16t + 8hg .. +7]
    // (rows past Sq, dims past DR read as zeros).
    u32x4 qr[8];
    {
        const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qbase, (uint32_t)a.Sq * DR * 2);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int d0 = 128 * dh + 16 * t + 8 * hg;
            qr[t] = __builtin_amdgcn_raw_buffer_load_b128(qrs, d0 < DR ? ((uint32_t)qi * DR + d0) * 2 : kOut, 0, 0);
        }
    }
    // DMA: load i of this wave fills 16-byte slot 64*(2*wave + i) + lane of a
    // tile, i.e. LDS row slot / 32, stored chunk slot % 32 (K rows in the
    // permuted key order of k_lds_row).
    uint32_t koff[DMA], voff[DMA];
#pragma unroll
    for (int i = 0; i < DMA; ++i) {
        const int s = 64 * (DMA * wave + i) + lane;
        const int row = s / L::CPR, pc = s % L::CPR;
        const int ck = pc ^ L::fk(row), cv = pc ^ L::fv(row);
        koff[i] = 8 * ck < DR ? (uint32_t)k_lds_row(row) * DR * 2 + ck * 16 : kOut;
        voff[i] = 8 * cv < DR ? (uint32_t)row * DR * 2 + cv * 16 : kOut;
    }
    // K operand: LDS row l32, logical chunk 16*dh + 2t + hg (dims of this wave).
    int krd[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) krd[t] = l32 * D + (((16 * dh + 2 * t + hg) ^ L::fk(l32)) * 8);
    // V^T operand: row 16*kk + tr_row (+4), column 128*dh + 32*db + tr_col.
    const int g16 = lane >> 4, j16 = lane & 15;
    const int tr_row = 8 * hg + (j16 >> 2);
    const int tr_col = 16 * (g16 & 1) + 4 * (j16 & 3);
    int vrd[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const int col = 128 * dh + 32 * db + tr_col;
        vrd[db] = tr_row * D + (((col >> 3) ^ L::fv(tr_row)) * 8) + (col & 7);
    }
    // Hand-over slots: 16 floats per lane as 4 chunks, chunk i at slot
    // (i + lane/4) % 4, so 16 lanes of one 16-byte access touch 16 bank groups.
    float* const xmine = xch + (wave * 64 + lane) * 16;  // + buffer * 8 * XF
    const float* const xpart = xch + ((wave ^ 4) * 64 + lane) * 16;
    auto xslot = [&](int i) { return 4 * ((i + (lane >> 2)) & 3); };

    f32x16 oacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
    float m_run = -INFINITY;  // reference max of row qi (raw score units)
    float l_run = 0.f;        // this lane's share of the denominator
    const float c = a.scale * kLog2e;
    const float tau = 8.0f / c;
    const bool rev = ti.rev;
    auto tkey = [&](int jt) { return (rev ? ntiles - 1 - jt : jt) * KT; };

    // This lane's hand-over slot addresses (its own 4 chunks, the partner's).
    float* xw[4];
    const float* xr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        xw[i] = xmine + xslot(i);
        xr[i] = xpart + xslot(i);
    }
    // Partial S^T over this wave's dims of the tile in K stage st: register r
    // holds key j0 + 16*(r/8) + 8*hg + r%8 of query qi.
    auto partial = [&](const int st, f32x16& s) __attribute__((always_inline)) {
        const uint16_t* ks = smem + st * TILE;
        u32x4 kf[3];
        kf[0] = *reinterpret_cast<const u32x4*>(ks + krd[0]);
        kf[1] = *reinterpret_cast<const u32x4*>(ks + krd[1]);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            if (t + 2 < 8) kf[(t + 2) % 3] = *reinterpret_cast<const u32x4*>(ks + krd[t + 2]);
            s = mfma_32x32x16<T>(kf[t % 3], qr[t], t == 0 ? f32x16{} : s);
        }
    };
    auto hand_over = [&](const int buf, const f32x16& s) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<f32x4*>(xw[i] + buf * 8 * XF) = f32x4{s[4 * i], s[4 * i + 1], s[4 * i + 2], s[4 * i + 3]};
    };
    auto add_partner = [&](const int buf, f32x16& s) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4 o = *reinterpret_cast<const f32x4*>(xr[i] + buf * 8 * XF);
            s[4 * i] += o[0];
            s[4 * i + 1] += o[1];
            s[4 * i + 2] += o[2];
            s[4 * i + 3] += o[3];
        }
    };
    auto issue_k = [&](int jt, const int st) __attribute__((always_inline)) {
        const int j0 = tkey(jt);
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kp + (int64_t)j0 * DR, (uint32_t)(a.Sk - j0) * DR * 2);
#pragma unroll
        for (int i = 0; i < DMA; ++i) dma16(rk, smem + st * TILE + 512 * (DMA * wave + i), koff[i]);
    };
    auto issue_v = [&](int jt, const int st) __attribute__((always_inline)) {
        const int j0 = tkey(jt);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vp + (int64_t)j0 * DR, (uint32_t)(a.Sk - j0) * DR * 2);
#pragma unroll
        for (int i = 0; i < DMA; ++i) dma16(rv, smem + (2 + st) * TILE + 512 * (DMA * wave + i), voff[i]);
    };

    // K of tile jt sits in K stage jt % 2, V of tile jt in V stage jt % 2,
    // the partial scores of tile jt go to hand-over buffer jt % 2.  Step jt
    // (cur = jt % 2, a literal in each call, so every LDS address is a
    // constant offset and the two score tiles swap roles without copies):
    // the full scores of tile jt are in scur, K of tile jt + 1 and V of tile
    // jt have landed; it issues K of jt + 2 and V of jt + 1, forms the partial
    // scores of tile jt + 1 into snext (MFMA) beside the softmax of tile jt
    // (VALU), accumulates P.V of tile jt, hands the partial over and, after
    // the barrier, adds the partner's.
    auto step = [&](int jt, const int cur, f32x16& scur, f32x16& snext) __attribute__((always_inline)) {
        const int j0 = tkey(jt);
        // K stage cur was last read for tile jt's partial, V stage cur ^ 1
        // for tile jt-1's P.V: both before the previous barrier
        if (jt + 2 < ntiles) issue_k(jt + 2, cur);
        if (jt + 1 < ntiles) issue_v(jt + 1, cur ^ 1);
        const bool act = jt < wave_tiles, act_next = jt + 1 < wave_tiles;  // the same for both waves of a pair
        if (act_next) partial(cur ^ 1, snext);
        if (act) {
            if ((a.causal && j0 + KT - 1 > qw) || j0 + KT > kv_lim) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = j0 + 16 * (r >> 3) + 8 * hg + (r & 7);
                    if (key >= kv_lim || (a.causal && key > qi)) scur[r] = -INFINITY;
                }
            }
            uint32_t pk[8];
            auto weights = [&]() -> float {
                const float neg = -((m_run == -INFINITY) ? 0.f : m_run) * c;
                float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    pk[r >> 1] = pack2<T>(fast_exp2(fmaf(scur[r], c, neg)), fast_exp2(fmaf(scur[r + 1], c, neg)));
                    if (r & 2) ps1 = sum2<T>(pk[r >> 1], ps1);
                    else ps0 = sum2<T>(pk[r >> 1], ps0);
                }
                return ps0 + ps1;
            };
            float ps = weights();
            if (__any(ps > 256.f || m_run == -INFINITY)) {
                float mx = scur[0];
#pragma unroll
                for (int r = 1; r < 16; ++r) mx = fmaxf(mx, scur[r]);
                mx = max_half_waves(mx);
                if (__any(mx > m_run + tau)) {
                    const float m_new = fmaxf(m_run, mx);
                    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
                    const float alpha = fast_exp2((m_run - m_use) * c);
                    m_run = m_new;
                    l_run *= alpha;
#pragma unroll
                    for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
                }
                ps = weights();
            }
            l_run += ps;
            // O^T += V^T P^T over the tile's two 16-key slices (this wave's dims)
            const uint16_t* vs = smem + (2 + cur) * TILE;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const u32x4 pw = {pk[4 * kk], pk[4 * kk + 1], pk[4 * kk + 2], pk[4 * kk + 3]};
                u32x4 vf[4];
#pragma unroll
                for (int db = 0; db < 4; ++db) {
                    const uint16_t* vb = vs + 16 * kk * D + vrd[db];
                    const u32x2 lo = lds_read_tr16x4(vb);
                    const u32x2 hi = lds_read_tr16x4(vb + 4 * D);
                    vf[db] = u32x4{lo[0], lo[1], hi[0], hi[1]};
                }
#pragma unroll
                for (int db = 0; db < 4; ++db) oacc[db] = mfma_32x32x16<T>(vf[db], pw, oacc[db]);
            }
        }
        if (act_next) hand_over(cur ^ 1, snext);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // K of jt+2 and V of jt+1 landed
        __syncthreads();
        if (act_next) add_partner(cur ^ 1, snext);
    };

    f32x16 sA = {}, sB = {};
    if (ntiles > 0) {
        issue_k(0, 0);
        issue_v(0, 0);
        if (ntiles > 1) issue_k(1, 1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (wave_tiles > 0) {
            partial(0, sA);
            hand_over(0, sA);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (wave_tiles > 0) add_partner(0, sA);
    }
    for (int jt = 0; jt < ntiles; jt += 2) {
        step(jt, 0, sA, sB);
        if (jt + 1 < ntiles) step(jt + 1, 1, sB, sA);
    }

    const float lt = l_run + swap_half_wave(l_run);
    const float inv = 1.f / lt;
    if (a.lse && dh == 0 && hg == 0 && qi < a.Sq)
        a.lse[bh * a.Sq + qi] = m_run == -INFINITY ? -INFINITY : m_run * a.scale + __logf(lt);
    if (qi < a.Sq) {
        uint16_t* orow = op + (int64_t)qi * DR;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const u32x2 w = {pack2<T>(oacc[db][4 * r4] * inv, oacc[db][4 * r4 + 1] * inv),
                                 pack2<T>(oacc[db][4 * r4 + 2] * inv, oacc[db][4 * r4 + 3] * inv)};
                const int d0 = 128 * dh + 32 * db + 8 * r4 + 4 * hg;  // 4 dims, all < DR or none
                if (d0 < DR) *reinterpret_cast<u32x2*>(orow + d0) = w;
            }
    }
}

// ---------------------------------------------------------------------------
// fp32 inputs, fp32 MFMA (v_mfma_f32_32x32x2_f32): every product exact in fp32.
// ---------------------------------------------------------------------------
// GEN: rows are DR = a.D floats in memory (a multiple of 4 below D); the
// 16-byte chunks past DR load as zeros and are never stored.
// PAGED: prefill chunks over fp32 page caches, with the row, position and
// page-table conventions of the 16-bit paged prefill above (each key row of a
// tile looks up its page; a table entry outside the cache is never read and
// its keys are hidden).
// SPLIT (dense, for grids that leave CUs idle): a workgroup owns 32 query
// rows instead of 128 and its 4 waves split the keys, wave w taking the
// 32-key blocks w, w + 4, w + 8, ... with its own running (max, sum, O), so
// each wave does a quarter of the serial work of a row block; at the end
// waves 1..3 hand their state to wave 0 through LDS, which rescales all four
// to the largest max and adds them (the merge of partial softmax states).
template <int D, bool GEN = false, bool PAGED = false, bool SPLIT = false>
__global__ __launch_bounds__(kThreads, 1) void forward_f32_kernel(
    ForwardArgs a, PagedArgs p, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cu_q) {
    static_assert(!(SPLIT && PAGED), "key-split waves: dense only");
    constexpr int RS = D + 4;                 // row stride in LDS (floats), 16 B of padding
    constexpr int KT = SPLIT ? 32 : kBc;      // keys per tile (SPLIT: per wave's block)
    constexpr int NH = KT / 32;               // 32-key halves per tile
    constexpr int NG = SPLIT ? 4 : 1;         // key groups (one tile each per round)
    constexpr int LT = SPLIT ? 64 : kThreads; // threads loading one tile
    __shared__ __attribute__((aligned(16))) float ks[NG * KT * RS];
    __shared__ __attribute__((aligned(16))) float vs[NG * KT * RS];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hg = lane >> 5;
    const int grp = SPLIT ? wave : 0;   // key group
    const int rwave = SPLIT ? 0 : wave; // 32-row block of the workgroup

    TileInfo ti;
    if constexpr (SPLIT) {
        // 32-row blocks; a grid this small needs no XCD ordering
        const int nqb = (a.Sq + 31) / 32;
        int t = blockIdx.x;
        const int qb = t % nqb;
        t /= nqb;
        ti.h = t % a.Hq;
        ti.b = t / a.Hq;
        ti.gk = ti.h / (a.Hq / a.Hkv);
        ti.q0 = 32 * qb;
        ti.rev = false;
    } else {
        ti = decode_tile(a);
    }
    const int DR = GEN ? a.D : D;
    const float* qp;
    const float* kp;
    const float* vp;
    float* op;
    int64_t rstride;  // floats between consecutive query (and output) rows
    int nrows, qoff, kv_lim, kv_end;
    int r0 = 0;  // paged: first packed row of the chunk
    if (PAGED) {
        r0 = min(max(cu_q[ti.b], 0), p.total_q);
        const int r1 = min(max(cu_q[ti.b + 1], r0), p.total_q);
        nrows = r1 - r0;
        if (ti.q0 >= nrows) return;  // the whole workgroup: no barrier reached yet
        kv_lim = min(seq_lens[ti.b], a.Sk);
        qoff = kv_lim - nrows;
        kv_end = kv_lim;
        if (a.causal) kv_end = min(kv_end, qoff + ti.q0 + kBr);
        const int64_t rb = ((int64_t)r0 * a.Hq + ti.h) * DR;
        qp = static_cast<const float*>(a.q) + rb;
        op = static_cast<float*>(a.out) + rb;
        rstride = (int64_t)a.Hq * DR;
        kp = static_cast<const float*>(a.k);
        vp = static_cast<const float*>(a.v);
    } else {
        const int64_t bh = (int64_t)ti.b * a.Hq + ti.h;
        qp = static_cast<const float*>(a.q) + bh * a.Sq * DR;
        const int64_t kvh = ((int64_t)ti.b * a.Hkv + ti.gk) * a.Sk * DR;
        kp = static_cast<const float*>(a.k) + kvh;
        vp = static_cast<const float*>(a.v) + kvh;
        op = static_cast<float*>(a.out) + bh * a.Sq * DR;
        rstride = DR;
        nrows = a.Sq;
        qoff = 0;
        key_extent(a, ti.b, ti.q0, kv_lim, kv_end);
        if (SPLIT && a.causal) kv_end = min(kv_end, ti.q0 + 32);
    }

    const int qw = ti.q0 + rwave * 32;
    const int qi = qw + l32;
    const int ntiles = kv_end > 0 ? (kv_end + KT - 1) / KT : 0;

    // Contraction slot (step t, lane half hg) <-> dim 8*(t/4) + 4*hg + t%4, so a
    // lane's operands for 4 consecutive steps are 4 consecutive floats.
    f32x4 qf[D / 8];
#pragma unroll
    for (int T = 0; T < D / 8; ++T) {
        qf[T] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (qi < nrows && 8 * T + 4 * hg < DR)
            qf[T] = *reinterpret_cast<const f32x4*>(qp + (int64_t)qi * rstride + 8 * T + 4 * hg);
    }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
    float m_run = -INFINITY;  // running max, log2-scaled units
    float l_run = 0.f;
    const float c = a.scale * kLog2e;

    float* const kg = ks + grp * KT * RS;  // this group's K and V tile
    float* const vg = vs + grp * KT * RS;
    // Every wave runs the same number of rounds (one barrier pair each);
    // group g takes tile NG * round + g.
    const int rounds = (ntiles + NG - 1) / NG;
    for (int rr = 0; rr < rounds; ++rr) {
        const int jt = rr * NG + grp;
        const int j0 = jt * KT;
        __syncthreads();
        static_assert(KT * (D / 4) % LT == 0, "whole load rounds");
#pragma unroll
        for (int li = 0; li < KT * (D / 4) / LT; ++li) {
            const int cidx = (SPLIT ? lane : tid) + li * LT;
            const int row = cidx / (D / 4), cc = cidx % (D / 4);
            const int key = j0 + row;
            f32x4 wk = {0.f, 0.f, 0.f, 0.f}, wv = {0.f, 0.f, 0.f, 0.f};
            if (PAGED) {
                // Key rows of invalid pages load zeros; the mask below hides them.
                const int lp = key / p.page_size;
                const int pg = (key < kv_lim && lp < p.max_pages)
                                   ? tables[(int64_t)ti.b * p.max_pages + lp] : -1;
                if (pg >= 0 && pg < p.pages && 4 * cc < DR) {
                    const int64_t off =
                        (((int64_t)pg * p.page_size + key % p.page_size) * a.Hkv + ti.gk) * DR + cc * 4;
                    wk = *reinterpret_cast<const f32x4*>(kp + off);
                    wv = *reinterpret_cast<const f32x4*>(vp + off);
                }
            } else if (key < a.Sk && 4 * cc < DR) {
                wk = *reinterpret_cast<const f32x4*>(kp + (int64_t)key * DR + cc * 4);
                wv = *reinterpret_cast<const f32x4*>(vp + (int64_t)key * DR + cc * 4);
            }
            *reinterpret_cast<f32x4*>(kg + row * RS + cc * 4) = wk;
            *reinterpret_cast<f32x4*>(vg + row * RS + cc * 4) = wv;
        }
        __syncthreads();
        if (jt >= ntiles) continue;  // (SPLIT) this wave has no block this round
        if (a.causal && j0 > qoff + qw + 31) continue;

        // S^T: register r of sacc[kb2] holds key j0 + 32*kb2 + 8*(r/4) + 4*hg + r%4.
        f32x16 sacc[NH];
#pragma unroll
        for (int kb2 = 0; kb2 < NH; ++kb2) {
            sacc[kb2] = f32x16{};
            const float* krow = kg + (32 * kb2 + l32) * RS + 4 * hg;
#pragma unroll
            for (int T = 0; T < D / 8; ++T) {
                const f32x4 kv = *reinterpret_cast<const f32x4*>(krow + 8 * T);
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    sacc[kb2] = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[u], qf[T][u], sacc[kb2], 0, 0, 0);
            }
        }

        // Paged: bit g says keys j0 + 16g .. +15 (one page: page sizes are
        // multiples of 16) come from a valid page.
        int vmask = 15;
        if (PAGED) {
            vmask = 0;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int key = j0 + 16 * g, lp = key / p.page_size;
                const int pg = (key < kv_lim && lp < p.max_pages) ? tables[(int64_t)ti.b * p.max_pages + lp] : -1;
                vmask |= (pg >= 0 && pg < p.pages) ? (1 << g) : 0;
            }
        }
        const bool need_mask = (a.causal && j0 + KT - 1 > qoff + qw) || (j0 + KT > kv_lim) || vmask != 15;
        if (need_mask) {
#pragma unroll
            for (int kb2 = 0; kb2 < NH; ++kb2)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int kt = 32 * kb2 + 8 * (r >> 2) + 4 * hg + (r & 3), key = j0 + kt;
                    const bool hide = key >= kv_lim || (a.causal && key > qoff + qi) ||
                                      !((vmask >> (kt >> 4)) & 1);
                    if (hide) sacc[kb2][r] = -INFINITY;
                }
        }
        // Work in log2-scaled units t = s * scale * log2(e): the row maximum
        // then gets weight exp2(t - m) = exp2(0) = 1 exactly.  Contraction is
        // off so the product is rounded on its own and never fused into the
        // later subtraction of m.
        {
#pragma clang fp contract(off)
#pragma unroll
            for (int kb2 = 0; kb2 < NH; ++kb2)
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kb2][r] = sacc[kb2][r] * c;
        }

        float mx = sacc[0][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[0][r]);
#pragma unroll
        for (int kb2 = 1; kb2 < NH; ++kb2)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb2][r]);
        mx = fmaxf(mx, swap_half_wave(mx));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        m_run = m_new;

        float psum = 0.f;
#pragma unroll
        for (int kb2 = 0; kb2 < NH; ++kb2)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
#pragma clang fp contract(off)
                const float p = fast_exp2(sacc[kb2][r] - m_use);
                sacc[kb2][r] = p;
                psum += p;
            }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;

        // O^T += V^T P^T: step u of block kb2 contracts the key held in register u.
#pragma unroll
        for (int kb2 = 0; kb2 < NH; ++kb2)
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int key = 32 * kb2 + 8 * (u >> 2) + 4 * hg + (u & 3);
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const float vv = vg[key * RS + 32 * db + l32];
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv, sacc[kb2][u], oacc[db], 0, 0, 0);
                }
            }
    }

    if constexpr (SPLIT) {
        // Waves 1..3 hand (O^T registers, m, lane sum) to wave 0 through the
        // K area, laid out [wave - 1][value][lane].
        constexpr int NF = (D / 32) * 16 + 2;
        static_assert(3 * NF * 64 <= NG * KT * RS, "hand-over fits the K area");
        __syncthreads();  // every tile read is done
        if (wave > 0) {
            float* const xw = ks + (wave - 1) * NF * 64 + lane;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) xw[(16 * db + r) * 64] = oacc[db][r];
            xw[(NF - 2) * 64] = m_run;
            xw[(NF - 1) * 64] = l_run;
        }
        __syncthreads();
        if (wave > 0) return;
        float m = m_run;
#pragma unroll
        for (int w = 0; w < 3; ++w) m = fmaxf(m, ks[(w * NF + NF - 2) * 64 + lane]);
        const float mu = m == -INFINITY ? 0.f : m;
        const float f0 = fast_exp2(m_run - mu);  // 1 for the wave holding the max
        l_run *= f0;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] *= f0;
#pragma unroll
        for (int w = 0; w < 3; ++w) {
            const float* xw = ks + w * NF * 64 + lane;
            const float f = fast_exp2(xw[(NF - 2) * 64] - mu);
            l_run = fmaf(xw[(NF - 1) * 64], f, l_run);
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] = fmaf(xw[(16 * db + r) * 64], f, oacc[db][r]);
        }
        m_run = m;
    }

    const float lt = l_run + swap_half_wave(l_run);
    const float inv = 1.f / lt;
    // Optional log-sum-exp (natural log; -inf for a row with no visible key):
    // dense [B, Hq, Sq], paged [packed rows, Hq].  m_run is in log2 units.
    if (a.lse && hg == 0 && qi < nrows)
        a.lse[PAGED ? (int64_t)(r0 + qi) * a.Hq + ti.h : ((int64_t)ti.b * a.Hq + ti.h) * a.Sq + qi] =
            m_run == -INFINITY ? -INFINITY : (m_run + __log2f(lt)) * 0.69314718055994531f;
    if (qi < nrows) {
        float* orow = op + (int64_t)qi * rstride;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f32x4 w = {oacc[db][4 * r4] * inv, oacc[db][4 * r4 + 1] * inv,
                                 oacc[db][4 * r4 + 2] * inv, oacc[db][4 * r4 + 3] * inv};
                const int d0 = 32 * db + 8 * r4 + 4 * hg;  // 4 dims, all < DR or none
                if (d0 < DR) *reinterpret_cast<f32x4*>(orow + d0) = w;
            }
    }
}

inline dim3 forward_grid(const ForwardArgs& a) {
    const int nqb = (a.Sq + kBr - 1) / kBr;
    // y: output slice of 128 dims when the value head dim is above 128
    return dim3((unsigned)(nqb * a.B * a.Hq), a.Dv > 128 ? 2u : 1u);
}

// Workgroups of this kernel one XCD holds at once (resident per CU times
// the CUs of one of the 8 XCDs); 0 when the runtime cannot say.  Looked up
// once per kernel (the instantiations share one pointer type, so the cache
// is keyed by address).
template <class Kernel>
int xcd_resident(Kernel kernel, int threads) {
    static std::mutex mu;
    static std::vector<std::pair<const void*, int>> cache;
    const void* key = reinterpret_cast<const void*>(kernel);
    std::lock_guard<std::mutex> lock(mu);
    for (const auto& e : cache)
        if (e.first == key) return e.second;
    int dev = 0, cus = 0, per_cu = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) == hipSuccess)
        n = per_cu * (cus / 8);
    cache.emplace_back(key, n);
    return n;
}

// Head dims that are multiples of 8 run on the 64-, 128- or 256-wide kernel
// (the general-width instantiation unless D is exactly 64, 128 or 256).  Above
// 128 the dense forward without a bias runs on paired waves; the paged and
// biased ones compute the output in two 128-dim slices.
template <bool PAGED, class T, bool BIAS = false>
hipError_t launch_16bit(const ForwardArgs& a, const PagedArgs& p, hipStream_t s) {
    if (a.D < 1 || a.D > 256) return hipErrorInvalidValue;
    const dim3 g = forward_grid(a), t(kThreads);
    auto go = [&](auto kernel) {
        ForwardArgs b = a;
        b.sweep_group = (!PAGED && !a.causal) ? xcd_resident(kernel, kThreads) : 0;
        hipLaunchKernelGGL(kernel, g, t, 0, s, b, p, p.block_tables, p.seq_lens, p.cu_seqlens_q);
    };
    if (a.D % 8 != 0 || a.Dv % 8 != 0) {
        // Head dims that are not multiples of 8 (up to 256): the element-wise
        // load path on the padded widths (no bias).
        if constexpr (!BIAS) {
            if (a.D < 1 || a.Dv < 1 || a.D > 256 || a.Dv > 256) return hipErrorInvalidValue;
            const bool v64 = a.Dv <= 64;
            if (a.D <= 64)
                v64 ? go(forward_bf16_kernel<64, PAGED, T, false, true, 64, true>)
                    : go(forward_bf16_kernel<64, PAGED, T, false, true, 128, true>);
            else if (a.D <= 128)
                v64 ? go(forward_bf16_kernel<128, PAGED, T, false, true, 64, true>)
                    : go(forward_bf16_kernel<128, PAGED, T, false, true, 128, true>);
            else
                v64 ? go(forward_bf16_kernel<256, PAGED, T, false, true, 64, true>)
                    : go(forward_bf16_kernel<256, PAGED, T, false, true, 128, true>);
            return hipGetLastError();
        }
        return hipErrorInvalidValue;
    }
    if (a.Dv != a.D) {
        // A value head dim of its own (paged prefill): general-width kernels
        // on the padded K width, V in one 64- or 128-dim pass or two 128-dim
        // slices.
        if constexpr (PAGED && !BIAS) {
            if (a.Dv % 8 != 0 || a.Dv < 8 || a.Dv > 256) return hipErrorInvalidValue;
            const bool v64 = a.Dv <= 64;
            if (a.D <= 64)
                v64 ? go(forward_bf16_kernel<64, PAGED, T, false, true, 64>)
                    : go(forward_bf16_kernel<64, PAGED, T, false, true, 128>);
            else if (a.D <= 128)
                v64 ? go(forward_bf16_kernel<128, PAGED, T, false, true, 64>)
                    : go(forward_bf16_kernel<128, PAGED, T, false, true, 128>);
            else
                v64 ? go(forward_bf16_kernel<256, PAGED, T, false, true, 64>)
                    : go(forward_bf16_kernel<256, PAGED, T, false, true, 128>);
            return hipGetLastError();
        }
        return hipErrorInvalidValue;
    }
    auto pair = [&](auto kernel) {
        ForwardArgs b = a;
        b.sweep_group = !a.causal ? xcd_resident(kernel, kPairThreads) : 0;
        hipLaunchKernelGGL(kernel, dim3(g.x, 1), dim3(kPairThreads), 0, s, b);
    };
    if (a.D == 64)
        go(forward_bf16_kernel<64, PAGED, T, BIAS>);
    else if (a.D == 128)
        go(forward_bf16_kernel<128, PAGED, T, BIAS>);
    else if (a.D > 128 && !PAGED && !BIAS)
        a.D == 256 ? pair(forward_pair_kernel<T>) : pair(forward_pair_kernel<T, true>);
    else if (a.D == 256)
        go(forward_bf16_kernel<256, PAGED, T, BIAS, false, 128>);
    else if (a.D < 64)
        go(forward_bf16_kernel<64, PAGED, T, BIAS, true>);
    else if (a.D < 128)
        go(forward_bf16_kernel<128, PAGED, T, BIAS, true>);
    else
        go(forward_bf16_kernel<256, PAGED, T, BIAS, true, 128>);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_forward_bf16(const ForwardArgs& a, hipStream_t s) {
    if (a.D > 256) return launch_forward_wide(a, false, s);
    return a.bias ? launch_16bit<false, Bf16T, true>(a, PagedArgs{}, s)
                  : launch_16bit<false, Bf16T>(a, PagedArgs{}, s);
}

hipError_t launch_forward_f16(const ForwardArgs& a, hipStream_t s) {
    if (a.D > 256) return launch_forward_wide(a, true, s);
    return a.bias ? launch_16bit<false, F16T, true>(a, PagedArgs{}, s)
                  : launch_16bit<false, F16T>(a, PagedArgs{}, s);
}

hipError_t launch_paged_prefill_16bit(const ForwardArgs& a, const PagedArgs& p, bool f16,
                                      hipStream_t s) {
    if (a.D > 256 || a.Dv > 256) return launch_paged_prefill_wide(a, p, f16, s);
    return f16 ? launch_16bit<true, F16T>(a, p, s) : launch_16bit<true, Bf16T>(a, p, s);
}

template <bool PAGED>
hipError_t launch_f32(const ForwardArgs& a, const PagedArgs& p, hipStream_t s) {
    if (a.D % 4 != 0 || a.D < 4 || a.D > 128 || a.Dv != a.D) return hipErrorInvalidValue;
    const dim3 g = forward_grid(a), t(kThreads);
    const int32_t *bt = p.block_tables, *sl = p.seq_lens, *cu = p.cu_seqlens_q;
    const int64_t g32 = (int64_t)a.B * a.Hq * ((a.Sq + 31) / 32);
    if (!PAGED && g32 <= 256) {
        // Grid of 32-row blocks fits the 256 CUs at one workgroup each: split
        // each block's keys over its 4 waves.
        const dim3 g2((unsigned)g32);
        if (a.D == 64)
            hipLaunchKernelGGL((forward_f32_kernel<64, false, false, true>), g2, t, 0, s, a, p, bt, sl, cu);
        else if (a.D == 128)
            hipLaunchKernelGGL((forward_f32_kernel<128, false, false, true>), g2, t, 0, s, a, p, bt, sl, cu);
        else if (a.D < 64)
            hipLaunchKernelGGL((forward_f32_kernel<64, true, false, true>), g2, t, 0, s, a, p, bt, sl, cu);
        else
            hipLaunchKernelGGL((forward_f32_kernel<128, true, false, true>), g2, t, 0, s, a, p, bt, sl, cu);
        return hipGetLastError();
    }
    if (a.D == 64)
        hipLaunchKernelGGL((forward_f32_kernel<64, false, PAGED>), g, t, 0, s, a, p, bt, sl, cu);
    else if (a.D == 128)
        hipLaunchKernelGGL((forward_f32_kernel<128, false, PAGED>), g, t, 0, s, a, p, bt, sl, cu);
    else if (a.D < 64)
        hipLaunchKernelGGL((forward_f32_kernel<64, true, PAGED>), g, t, 0, s, a, p, bt, sl, cu);
    else
        hipLaunchKernelGGL((forward_f32_kernel<128, true, PAGED>), g, t, 0, s, a, p, bt, sl, cu);
    return hipGetLastError();
}

hipError_t launch_forward_f32(const ForwardArgs& a, hipStream_t s) {
    return launch_f32<false>(a, PagedArgs{}, s);
}

hipError_t launch_paged_prefill_f32(const ForwardArgs& a, const PagedArgs& p, hipStream_t s) {
    return launch_f32<true>(a, p, s);
}

}  // namespace sdpa
