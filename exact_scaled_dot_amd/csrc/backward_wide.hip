// Attention backward for head dims above 128, up to 512, of any width (ruDNN user guide
// section 11: dq, dk, dv recomputed from the forward's log-sum-exp, ordered
// reductions; section 9 for the head-dim range).  The same three passes as
// the narrow backward (row statistics, a query-parallel dQ pass, a
// key-parallel dK/dV pass) with the head dim split across the waves of a
// workgroup, as in the head-dim-split forward: NW = 2 or 4 waves, wave w
// owning dims 128w .. 128w+127 (dims past D load as zeros, are never stored).
//
// dQ pass (workgroup = 32 query rows of one (batch, query head)); per 16-key
// tile (K and V tiles of the wave's dims by DMA, two stages):
//   every wave: partial S^T = K_w Q_w^T and dP^T = V_w dO_w^T
//     (v_mfma_f32_16x16x32, Q and dO rows in registers, K and V rows read
//     from LDS), both to LDS in fp32 (one buffer: a barrier before the
//     partials are written and one after, before they are read);
//   every lane: sums the partials of its query (lane%32) at keys
//     8*(lane/32) .. +7, P = exp2(S scale log2e - lse2), dS = P o (dP - delta),
//     exactly the B operand of dQ^T += K_w^T dS^T (v_mfma_f32_32x32x16, K^T
//     by transposed LDS reads).
// dK/dV pass (workgroup = 32 keys of one (batch, K/V head), walking the query
// tiles of every query head of the group); per 16-query step (Q and dO
// tiles and the tile's row statistics by DMA):
//   every wave: partial S = Q_w K_w^T and dP = dO_w V_w^T (K and V rows in
//     registers), to LDS; a barrier;
//   every lane: its key (lane%32) at queries 8*(lane/32) .. +7: P and dS,
//     then dV^T += dO_w^T P and dK^T += Q_w^T dS (transposed reads of the dO
//     and Q tiles).
// P and dS enter their products rounded to the input type; dS is formed from
// the unrounded P; accumulation is fp32.
// ELEM (head dims that are not multiples of 8): rows are not 16-byte
// aligned, so Q, dO, O, K and V are read element by element (into the same
// registers and LDS slots the 16-byte loads and the DMA fill) and dQ, dK, dV
// are stored element by element.
#include "device_common.hpp"
#include "launch.hpp"

namespace sdpa {
namespace {

constexpr int kXRows = 32;    // rows a workgroup owns (queries, or keys)
constexpr int kXTile = 16;    // rows streamed per step (keys, or queries)
constexpr int kXChunk = 128;  // head dims per wave
constexpr int kXStages = 3;    // dK/dV pass: Q/dO ring depth
constexpr int kXStagesQ = 2;   // dQ pass: K/V ring depth (40 KB per 2-wave workgroup: 4 per CU)
constexpr int kXTileEl = kXTile * kXChunk;  // 16-bit elements of one wave's tile
constexpr uint32_t kXOut = 0x80000000u;     // buffer offset past any num_records
constexpr float kXLog2e = 1.4426950408889634f;

typedef short x_i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void x_lds_void;

// LDS accessors (a __restrict__ parameter per access: no vmcnt(0) drain of the
// in-flight DMA in front of it).
__device__ __forceinline__ u32x2 x_lds_tr(const uint16_t* __restrict__ p) {
    typedef __attribute__((address_space(3))) x_i16x4 lds_i16x4;
    return __builtin_bit_cast(
        u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((__attribute__((address_space(3))) char*)p)));
}
__device__ __forceinline__ u32x4 x_lds_row(const uint16_t* __restrict__ p) {
    return *(const __attribute__((address_space(3))) u32x4*)((const __attribute__((address_space(3))) char*)p);
}
__device__ __forceinline__ void x_lds_st_f4(float* __restrict__ p, f32x4 v) {
    *(__attribute__((address_space(3))) f32x4*)((__attribute__((address_space(3))) char*)p) = v;
}
__device__ __forceinline__ f32x4 x_lds_ld_f4(const float* __restrict__ p) {
    return *(const __attribute__((address_space(3))) f32x4*)((const __attribute__((address_space(3))) char*)p);
}
__device__ __forceinline__ void x_lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t x_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void x_lds_st4(uint16_t* __restrict__ p, u32x4 v) {
    *(__attribute__((address_space(3))) u32x4*)((__attribute__((address_space(3))) char*)p) = v;
}
// 16 bytes (8 elements) of a row from 2-byte loads: element e from byte
// offset off + 2e when e < valid, else zero.
__device__ __forceinline__ u32x4 x_elem16(__amdgpu_buffer_rsrc_t r, uint32_t off, int valid) {
    u32x4 v;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(r, 2 * w < valid ? off + 4 * w : kXOut, 0, 0);
        const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(r, 2 * w + 1 < valid ? off + 4 * w + 2 : kXOut, 0, 0);
        v[w] = lo | (hi << 16);
    }
    return v;
}
// Four 16-bit values stored element by element (e < valid).
__device__ __forceinline__ void x_store4(uint16_t* p, u32x2 w, int valid) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (e < valid) p[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
}
__device__ __forceinline__ void x_dma(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (x_lds_void*)((__attribute__((address_space(3))) char*)lds), 16,
                                             voff, 0, 0, 0);
}
// Waits for a step's DMA when `newer` later steps (0..2) have been issued
// since, N loads each: vmcnt counts in issue order, so at most N * newer
// may stay in flight.
template <int N>
__device__ __forceinline__ void x_wait(int newer) {
    if (newer >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * N) : "memory");
    else if (newer == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}
__device__ __forceinline__ int x_xcd_order(int total) {
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    const int nx = total >> 3, rem = total & 7;
    return xcd * nx + min(xcd, rem) + local;
}

// A wave's [16 rows][128 dims] 16-bit tile: logical 16-byte chunk c of row r
// sits at chunk c ^ f(r), f(r) = 4*(r%4) + (r/4)%4: a row read (16 rows, one
// chunk) and a transposed read (4 rows x 4 chunks) each touch 16 distinct
// bank groups.
__device__ __forceinline__ int x_f(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }
__device__ __forceinline__ int x_at(int r, int c) { return r * kXChunk + ((c ^ x_f(r)) * 8); }

// Partial scores: [32 rows][16 columns] fp32 per (buffer, kind, wave); row r
// keeps its 4-column chunk g at chunk (g + r/4) % 4 (16-byte writes of 16
// rows and reads of 4 rows, conflict-free).
__device__ __forceinline__ int x_part(int r, int g) { return r * kXTile + (((g + (r >> 2)) & 3) * 4); }

// Transposed-read offsets of a tile for d-block db (32x32x16 A operand: row
// l%32 of the operand = dim 32db + l%32, contraction 8*(l/32) + e = tile rows).
struct XTr {
    int lo[4], hi[4];
    __device__ XTr(int lane) {
        const int g16 = lane >> 4, j16 = lane & 15;
        const int rl = 8 * (g16 >> 1) + (j16 >> 2), rh = rl + 4;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const int col = 32 * db + 16 * (g16 & 1) + 4 * (j16 & 3);
            lo[db] = rl * kXChunk + (((col >> 3) ^ x_f(rl)) * 8) + (col & 7);
            hi[db] = rh * kXChunk + (((col >> 3) ^ x_f(rh)) * 8) + (col & 7);
        }
    }
};

// Row statistics for both passes: (lse * log2e, rowsum(dO o O)) per query row,
// (+inf, 0) for a row with no visible key (lse = -inf).  One wave per row,
// 8 dims per lane.
template <class T, bool ELEM = false>
__global__ __launch_bounds__(256) void bwd_wide_stats_kernel(BackwardArgs a) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= (int64_t)a.B * a.Hq * a.Sq) return;
    float part = 0.f;
    if (8 * lane < a.D) {
        u32x4 o, d;
        if constexpr (ELEM) {  // rows not 16-byte aligned: element by element, zeros past D
            const uint16_t* orow = static_cast<const uint16_t*>(a.out) + row * a.D + 8 * lane;
            const uint16_t* drow = static_cast<const uint16_t*>(a.dout) + row * a.D + 8 * lane;
            const int n = min(8, a.D - 8 * lane);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t o0 = 2 * w < n ? orow[2 * w] : 0u, o1 = 2 * w + 1 < n ? orow[2 * w + 1] : 0u;
                const uint32_t d0 = 2 * w < n ? drow[2 * w] : 0u, d1 = 2 * w + 1 < n ? drow[2 * w + 1] : 0u;
                o[w] = o0 | (o1 << 16);
                d[w] = d0 | (d1 << 16);
            }
        } else {
            o = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.out) + row * a.D + 8 * lane);
            d = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.dout) + row * a.D + 8 * lane);
        }
        const uint32_t os[4] = {o[0], o[1], o[2], o[3]}, ds[4] = {d[0], d[1], d[2], d[3]};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (T::kF16)
                part = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, ds[i]), __builtin_bit_cast(f16x2, os[i]),
                                              part, false);
            else
                part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ds[i]),
                                                       __builtin_bit_cast(bf16x2, os[i]), part, false);
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) part += __shfl_xor(part, m);
    if (lane == 0) {
        const int64_t bh = row / a.Sq, i = row % a.Sq;
        const float l = a.lse[row];
        float2* st = reinterpret_cast<float2*>(a.delta) + bh * ((a.Sq + 1) & ~1) + i;
        *st = l == -INFINITY ? make_float2(INFINITY, 0.f) : make_float2(l * kXLog2e, part);
    }
}

template <int NW>
struct XLds {
    static constexpr int PKIND = NW * kXRows * kXTile;  // floats per (buffer, kind)
    static constexpr int PBUF = 2 * PKIND;
    static constexpr int TFL = 2 * PBUF;                // tiles start (floats)
    // per wave and stage: two tiles (+ the dK/dV pass's 1-KB statistics slot)
    static constexpr int STAGE_DQ = 2 * kXTileEl;       // 16-bit elements
    static constexpr int STAGE_KV = 2 * kXTileEl + 512;
};

// ---------------------------------------------------------------- dQ pass
template <int NW, class T, bool ELEM = false>
__global__ __launch_bounds__(NW * 64, 1) void bwd_wide_dq_kernel(BackwardArgs a, const int32_t* __restrict__ key_lens) {
    using LY = XLds<NW>;
    // one partial buffer (a second barrier per tile): 40 KB at NW = 2, four
    // workgroups per CU
    __shared__ __attribute__((aligned(1024))) float smem[LY::PBUF + NW * kXStagesQ * LY::STAGE_DQ / 2];
    uint16_t* const tiles = reinterpret_cast<uint16_t*>(smem + LY::PBUF);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l16 = lane & 15, g4 = lane >> 4, qr = lane & 31, kh = lane >> 5;
    const int D = a.D;
    const int d0 = kXChunk * wave;

    const int G = a.Hq / a.Hkv;
    const int nqb = (a.Sq + kXRows - 1) / kXRows;
    int t = x_xcd_order(a.B * a.Hkv * nqb * G);
    const int hsub = t % G;
    t /= G;
    const int qord = t % nqb;
    const int unit = t / nqb;
    const int b = unit / a.Hkv, gk = unit % a.Hkv, h = gk * G + hsub;
    const int q0 = (a.causal ? nqb - 1 - qord : qord) * kXRows;
    const int64_t bh = (int64_t)b * a.Hq + h;

    int kv_lim = a.Sk;
    if (a.padded) kv_lim = max(0, min(kv_lim, key_lens[b]));
    int kv_end = kv_lim;
    if (a.causal) kv_end = min(kv_end, q0 + kXRows);
    const int ntiles = kv_end > 0 ? (kv_end + kXTile - 1) / kXTile : 0;

    // Q and dO rows (B operands): query q0 + 16qb + lane%16, dims d0 + 32s + 8*(lane/16).
    u32x4 qf[2][4], df[2][4];
    {
        const int64_t qoff = bh * a.Sq * D;
        const __amdgpu_buffer_rsrc_t rq = x_rsrc(static_cast<const uint16_t*>(a.q) + qoff, (uint32_t)a.Sq * D * 2);
        const __amdgpu_buffer_rsrc_t rd = x_rsrc(static_cast<const uint16_t*>(a.dout) + qoff, (uint32_t)a.Sq * D * 2);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int row = q0 + 16 * qb + l16, dim = d0 + 32 * s + 8 * g4;
                const uint32_t o = (row < a.Sq && dim < D) ? ((uint32_t)row * D + dim) * 2 : kXOut;
                if constexpr (ELEM) {
                    qf[qb][s] = x_elem16(rq, o, D - dim);
                    df[qb][s] = x_elem16(rd, o, D - dim);
                } else {
                    qf[qb][s] = __builtin_amdgcn_raw_buffer_load_b128(rq, o, 0, 0);
                    df[qb][s] = __builtin_amdgcn_raw_buffer_load_b128(rd, o, 0, 0);
                }
            }
    }
    // this lane's query: (lse2, delta)
    const int qa = q0 + qr;
    float lse2 = INFINITY, delta = 0.f;
    if (qa < a.Sq) {
        const float2 st = reinterpret_cast<const float2*>(a.delta)[bh * ((a.Sq + 1) & ~1) + qa];
        lse2 = st.x;
        delta = st.y;
    }

    const int64_t kvh = ((int64_t)b * a.Hkv + gk) * a.Sk * D;
    const __amdgpu_buffer_rsrc_t rk = x_rsrc(static_cast<const uint16_t*>(a.k) + kvh, (uint32_t)a.Sk * D * 2);
    const __amdgpu_buffer_rsrc_t rv = x_rsrc(static_cast<const uint16_t*>(a.v) + kvh, (uint32_t)a.Sk * D * 2);
    uint16_t* const wt = tiles + wave * kXStagesQ * LY::STAGE_DQ;
    // DMA i fills tile rows 4i + lane/16, stored chunk lane%16
    auto load_tiles = [&](int kt, int st) {
        uint16_t* base = wt + st * LY::STAGE_DQ;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * i + g4, c = (lane & 15) ^ x_f(r);
            const uint32_t o = d0 + 8 * c < D ? ((uint32_t)(kt + r) * D + d0 + 8 * c) * 2 : kXOut;
            if constexpr (ELEM) {  // the slots the DMA would fill: 16 bytes at lane * 16
                x_lds_st4(base + 512 * i + 8 * lane, x_elem16(rk, o, D - d0 - 8 * c));
                x_lds_st4(base + kXTileEl + 512 * i + 8 * lane, x_elem16(rv, o, D - d0 - 8 * c));
            } else {
                x_dma(rk, base + 512 * i, o);
                x_dma(rv, base + kXTileEl + 512 * i, o);
            }
        }
    };
    const XTr tr(lane);

    f32x16 acc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[db] = f32x16{};
    const float c = a.scale * kXLog2e;
    const int poff0 = x_part(qr, 2 * kh), poff1 = x_part(qr, 2 * kh + 1);

    if (ntiles > 0) load_tiles(0, 0);
    for (int j = 0; j < ntiles; ++j) {
        const int kt = j * kXTile;
        // the stage refilled here was last read by this wave in tile j - 1
        if (j + 1 < ntiles) load_tiles(kt + kXTile, (j + 1) & 1);
        x_wait<8>(min(1, ntiles - 1 - j));  // this tile's 8 DMA loads have landed
        const uint16_t* kt_l = wt + (j & 1) * LY::STAGE_DQ;
        const uint16_t* vt_l = kt_l + kXTileEl;
        float* const pb = smem;

        // partial S^T and dP^T: register i of block qb = key 4*(lane/16) + i of
        // the tile, query 16qb + lane%16
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            f32x4 sa = {0.f, 0.f, 0.f, 0.f}, pa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                sa = mfma_16x16x32<T>(x_lds_row(kt_l + x_at(l16, 4 * s + g4)), qf[qb][s], sa);
                pa = mfma_16x16x32<T>(x_lds_row(vt_l + x_at(l16, 4 * s + g4)), df[qb][s], pa);
            }
            const int q = 16 * qb + l16;
            x_lds_st_f4(pb + wave * (kXRows * kXTile) + x_part(q, g4), sa);
            x_lds_st_f4(pb + LY::PKIND + wave * (kXRows * kXTile) + x_part(q, g4), pa);
        }
        x_lds_barrier();

        f32x4 s0 = x_lds_ld_f4(pb + poff0), s1 = x_lds_ld_f4(pb + poff1);
        f32x4 p0 = x_lds_ld_f4(pb + LY::PKIND + poff0), p1 = x_lds_ld_f4(pb + LY::PKIND + poff1);
#pragma unroll
        for (int w = 1; w < NW; ++w) {
            s0 += x_lds_ld_f4(pb + w * (kXRows * kXTile) + poff0);
            s1 += x_lds_ld_f4(pb + w * (kXRows * kXTile) + poff1);
            p0 += x_lds_ld_f4(pb + LY::PKIND + w * (kXRows * kXTile) + poff0);
            p1 += x_lds_ld_f4(pb + LY::PKIND + w * (kXRows * kXTile) + poff1);
        }
        // every wave has read the partials before any wave writes the next
        // tile's into the same buffer
        x_lds_barrier();
        const float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
        const float dv[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
        const int key0 = kt + 8 * kh;
        u32x4 ds;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float pe[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int key = key0 + 2 * e + u;
                const bool live = key < kv_lim && !(a.causal && key > qa);
                pe[u] = live ? fast_exp2(fmaf(sv[2 * e + u], c, -lse2)) * (dv[2 * e + u] - delta) : 0.f;
            }
            ds[e] = pack2<T>(pe[0], pe[1]);
        }
        // dQ^T += K_w^T dS^T
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const u32x2 lo = x_lds_tr(kt_l + tr.lo[db]), hi = x_lds_tr(kt_l + tr.hi[db]);
            acc[db] = mfma_32x32x16<T>(u32x4{lo[0], lo[1], hi[0], hi[1]}, ds, acc[db]);
        }
    }

    // dQ = scale * acc: register r of d-block db = dim d0 + 32db + 8*(r/4) +
    // 4*(lane/32) + r%4 of query q0 + lane%32
    if (qa < a.Sq) {
        uint16_t* row = static_cast<uint16_t*>(a.dq) + (bh * a.Sq + qa) * D;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int dim = d0 + 32 * db + 8 * r4 + 4 * kh;
                const f32x16& x = acc[db];
                const u32x2 w = {pack2<T>(x[4 * r4] * a.scale, x[4 * r4 + 1] * a.scale),
                                 pack2<T>(x[4 * r4 + 2] * a.scale, x[4 * r4 + 3] * a.scale)};
                if constexpr (ELEM) x_store4(row + dim, w, D - dim);
                else if (dim < D) *reinterpret_cast<u32x2*>(row + dim) = w;
            }
    }
}

// ---------------------------------------------------------------- dK/dV pass
template <int NW, class T, bool ELEM = false>
__global__ __launch_bounds__(NW * 64, 1) void bwd_wide_dkdv_kernel(BackwardArgs a,
                                                                   const int32_t* __restrict__ key_lens) {
    using LY = XLds<NW>;
    __shared__ __attribute__((aligned(1024))) float smem[LY::TFL + NW * kXStages * LY::STAGE_KV / 2];
    uint16_t* const tiles = reinterpret_cast<uint16_t*>(smem + LY::TFL);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l16 = lane & 15, g4 = lane >> 4, kr = lane & 31, kh = lane >> 5;
    const int D = a.D;
    const int d0 = kXChunk * wave;

    const int G = a.Hq / a.Hkv;
    const int nkb = (a.Sk + kXRows - 1) / kXRows;
    const int t = x_xcd_order(a.B * a.Hkv * nkb);
    const int unit = t / nkb;
    const int k0 = (t % nkb) * kXRows;
    const int b = unit / a.Hkv, gk = unit % a.Hkv;

    int kv_lim = a.Sk;
    if (a.padded) kv_lim = max(0, min(kv_lim, key_lens[b]));
    const int ka = k0 + kr;  // this lane's key

    // K and V rows (B operands): key k0 + 16kb + lane%16, dims d0 + 32s + 8*(lane/16).
    const int64_t kvh = ((int64_t)b * a.Hkv + gk) * a.Sk * D;
    u32x4 kf[2][4], vf[2][4];
    {
        const __amdgpu_buffer_rsrc_t rk = x_rsrc(static_cast<const uint16_t*>(a.k) + kvh, (uint32_t)a.Sk * D * 2);
        const __amdgpu_buffer_rsrc_t rv = x_rsrc(static_cast<const uint16_t*>(a.v) + kvh, (uint32_t)a.Sk * D * 2);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int row = k0 + 16 * kb + l16, dim = d0 + 32 * s + 8 * g4;
                const uint32_t o = (row < a.Sk && dim < D) ? ((uint32_t)row * D + dim) * 2 : kXOut;
                if constexpr (ELEM) {
                    kf[kb][s] = x_elem16(rk, o, D - dim);
                    vf[kb][s] = x_elem16(rv, o, D - dim);
                } else {
                    kf[kb][s] = __builtin_amdgcn_raw_buffer_load_b128(rk, o, 0, 0);
                    vf[kb][s] = __builtin_amdgcn_raw_buffer_load_b128(rv, o, 0, 0);
                }
            }
    }

    // Query tiles: all, or (causal) those holding a query >= k0; none when the
    // block's keys are all past the key limit.
    const int qt0 = a.causal ? k0 / kXTile : 0;
    const int nqt = k0 < kv_lim ? max(0, (a.Sq + kXTile - 1) / kXTile - qt0) : 0;
    const int steps = G * nqt;

    uint16_t* const wt = tiles + wave * kXStages * LY::STAGE_KV;
    // step st: head gk*G + st/nqt, queries q0 .. q0+15; Q and dO tiles (DMA i:
    // rows 4i + lane/16, stored chunk lane%16) and the 16 rows' (lse2, delta)
    // pairs (lanes 0..7 carry 16 bytes each; the rest read past the head)
    auto load_step = [&](int st, int stage) {
        const int h = gk * G + st / nqt;
        const int q0 = (qt0 + st % nqt) * kXTile;
        const int64_t bh = (int64_t)b * a.Hq + h;
        const __amdgpu_buffer_rsrc_t rq =
            x_rsrc(static_cast<const uint16_t*>(a.q) + bh * a.Sq * D, (uint32_t)a.Sq * D * 2);
        const __amdgpu_buffer_rsrc_t rd =
            x_rsrc(static_cast<const uint16_t*>(a.dout) + bh * a.Sq * D, (uint32_t)a.Sq * D * 2);
        uint16_t* base = wt + stage * LY::STAGE_KV;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * i + g4, c = (lane & 15) ^ x_f(r);
            const uint32_t o = (q0 + r < a.Sq && d0 + 8 * c < D) ? ((uint32_t)(q0 + r) * D + d0 + 8 * c) * 2 : kXOut;
            if constexpr (ELEM) {  // the slots the DMA would fill: 16 bytes at lane * 16
                x_lds_st4(base + 512 * i + 8 * lane, x_elem16(rq, o, D - d0 - 8 * c));
                x_lds_st4(base + kXTileEl + 512 * i + 8 * lane, x_elem16(rd, o, D - d0 - 8 * c));
            } else {
                x_dma(rq, base + 512 * i, o);
                x_dma(rd, base + kXTileEl + 512 * i, o);
            }
        }
        const int64_t srow = bh * ((a.Sq + 1) & ~1);
        const __amdgpu_buffer_rsrc_t rs =
            x_rsrc(reinterpret_cast<const float2*>(a.delta) + srow, (uint32_t)((a.Sq + 1) & ~1) * 8);
        x_dma(rs, base + 2 * kXTileEl, lane < 8 ? (uint32_t)(q0 * 8 + 16 * lane) : kXOut);
    };
    const XTr tr(lane);

    f32x16 acck[4], accv[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) acck[db] = accv[db] = f32x16{};
    const float c = a.scale * kXLog2e;
    const int poff0 = x_part(kr, 2 * kh), poff1 = x_part(kr, 2 * kh + 1);

    if (steps > 0) load_step(0, 0);
    if (steps > 1) load_step(1, 1);
    for (int st = 0; st < steps; ++st) {
        if (st + 2 < steps) load_step(st + 2, (st + 2) % kXStages);
        x_wait<9>(min(2, steps - 1 - st));  // this step's 9 DMA loads have landed
        const uint16_t* qt_l = wt + (st % kXStages) * LY::STAGE_KV;
        const uint16_t* dt_l = qt_l + kXTileEl;
        const float* stl = reinterpret_cast<const float*>(qt_l + 2 * kXTileEl);
        const int q0 = (qt0 + st % nqt) * kXTile;
        float* const pb = smem + (st & 1) * LY::PBUF;

        // partial S and dP (queries x keys): register i of block kb = query
        // 4*(lane/16) + i of the tile, key 16kb + lane%16
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            f32x4 sa = {0.f, 0.f, 0.f, 0.f}, pa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                sa = mfma_16x16x32<T>(x_lds_row(qt_l + x_at(l16, 4 * s + g4)), kf[kb][s], sa);
                pa = mfma_16x16x32<T>(x_lds_row(dt_l + x_at(l16, 4 * s + g4)), vf[kb][s], pa);
            }
            const int k = 16 * kb + l16;
            x_lds_st_f4(pb + wave * (kXRows * kXTile) + x_part(k, g4), sa);
            x_lds_st_f4(pb + LY::PKIND + wave * (kXRows * kXTile) + x_part(k, g4), pa);
        }
        x_lds_barrier();

        f32x4 s0 = x_lds_ld_f4(pb + poff0), s1 = x_lds_ld_f4(pb + poff1);
        f32x4 p0 = x_lds_ld_f4(pb + LY::PKIND + poff0), p1 = x_lds_ld_f4(pb + LY::PKIND + poff1);
#pragma unroll
        for (int w = 1; w < NW; ++w) {
            s0 += x_lds_ld_f4(pb + w * (kXRows * kXTile) + poff0);
            s1 += x_lds_ld_f4(pb + w * (kXRows * kXTile) + poff1);
            p0 += x_lds_ld_f4(pb + LY::PKIND + w * (kXRows * kXTile) + poff0);
            p1 += x_lds_ld_f4(pb + LY::PKIND + w * (kXRows * kXTile) + poff1);
        }
        const float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
        const float dv[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
        // this lane's queries q0 + 8kh + e: (lse2, delta) from the step's slot
        u32x4 pp, ds;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float pv[2], dsv[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int qi = 8 * kh + 2 * e + u, q = q0 + qi;
                const float l2 = stl[2 * qi], dl = stl[2 * qi + 1];
                // a query past Sq may read the unwritten padding slot of the
                // statistics: select, never multiply, its terms away
                const bool live = q < a.Sq && ka < kv_lim && !(a.causal && q < ka);
                const float p = fast_exp2(fmaf(sv[2 * e + u], c, -l2));
                pv[u] = live ? p : 0.f;
                dsv[u] = live ? p * (dv[2 * e + u] - dl) : 0.f;
            }
            pp[e] = pack2<T>(pv[0], pv[1]);
            ds[e] = pack2<T>(dsv[0], dsv[1]);
        }
        // dV^T += dO_w^T P, dK^T += Q_w^T dS
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const u32x2 dlo = x_lds_tr(dt_l + tr.lo[db]), dhi = x_lds_tr(dt_l + tr.hi[db]);
            accv[db] = mfma_32x32x16<T>(u32x4{dlo[0], dlo[1], dhi[0], dhi[1]}, pp, accv[db]);
            const u32x2 qlo = x_lds_tr(qt_l + tr.lo[db]), qhi = x_lds_tr(qt_l + tr.hi[db]);
            acck[db] = mfma_32x32x16<T>(u32x4{qlo[0], qlo[1], qhi[0], qhi[1]}, ds, acck[db]);
        }
    }

    // dK = scale * acck, dV = accv (0 for keys past the limit): register r of
    // d-block db = dim d0 + 32db + 8*(r/4) + 4*(lane/32) + r%4 of key k0 + lane%32
    if (ka < a.Sk) {
        const bool keep = ka < kv_lim;
        uint16_t* krow = static_cast<uint16_t*>(a.dk) + kvh + (int64_t)ka * D;
        uint16_t* vrow = static_cast<uint16_t*>(a.dv) + kvh + (int64_t)ka * D;
        const float sk = keep ? a.scale : 0.f, sv1 = keep ? 1.f : 0.f;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int dim = d0 + 32 * db + 8 * r4 + 4 * kh;
                const f32x16& xk = acck[db];
                const f32x16& xv = accv[db];
                const u32x2 wk = {pack2<T>(xk[4 * r4] * sk, xk[4 * r4 + 1] * sk),
                                  pack2<T>(xk[4 * r4 + 2] * sk, xk[4 * r4 + 3] * sk)};
                const u32x2 wv = {pack2<T>(xv[4 * r4] * sv1, xv[4 * r4 + 1] * sv1),
                                  pack2<T>(xv[4 * r4 + 2] * sv1, xv[4 * r4 + 3] * sv1)};
                if constexpr (ELEM) {
                    x_store4(krow + dim, wk, D - dim);
                    x_store4(vrow + dim, wv, D - dim);
                } else if (dim < D) {
                    *reinterpret_cast<u32x2*>(krow + dim) = wk;
                    *reinterpret_cast<u32x2*>(vrow + dim) = wv;
                }
            }
    }
}

template <int NW, class T, bool ELEM>
hipError_t launch_bw_wide_nw(const BackwardArgs& a, hipStream_t s) {
    const int64_t rows = (int64_t)a.B * a.Hq * a.Sq;
    hipLaunchKernelGGL((bwd_wide_stats_kernel<T, ELEM>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nqb = (a.Sq + kXRows - 1) / kXRows;
    hipLaunchKernelGGL((bwd_wide_dq_kernel<NW, T, ELEM>), dim3((unsigned)(a.B * a.Hq * nqb)), dim3(NW * 64), 0, s,
                       a, a.key_lens);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nkb = (a.Sk + kXRows - 1) / kXRows;
    hipLaunchKernelGGL((bwd_wide_dkdv_kernel<NW, T, ELEM>), dim3((unsigned)(a.B * a.Hkv * nkb)), dim3(NW * 64), 0,
                       s, a, a.key_lens);
    return hipGetLastError();
}

template <class T>
hipError_t launch_bw_wide_t(const BackwardArgs& a, hipStream_t s) {
    if (a.D % 8 != 0)
        return a.D <= 2 * kXChunk ? launch_bw_wide_nw<2, T, true>(a, s) : launch_bw_wide_nw<4, T, true>(a, s);
    return a.D <= 2 * kXChunk ? launch_bw_wide_nw<2, T, false>(a, s) : launch_bw_wide_nw<4, T, false>(a, s);
}

}  // namespace

hipError_t launch_backward_wide(const BackwardArgs& a, bool f16, hipStream_t s) {
    if (a.D <= 128 || a.D > 4 * kXChunk || a.bias || a.dq_acc) return hipErrorInvalidValue;
    return f16 ? launch_bw_wide_t<F16T>(a, s) : launch_bw_wide_t<Bf16T>(a, s);
}

}  // namespace sdpa
