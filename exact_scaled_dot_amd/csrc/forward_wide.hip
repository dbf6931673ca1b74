// Exact attention forward for wide heads: 16-bit Q, K, V with a head dim D
// above 256 and up to 1024 (any width), the range the ruDNN user guide
// allows for attention (section 9: D and Dv in 1..=1024).  Same definition
// and options as the narrow forward: softmax over the keys of
// Q K^T * scale (+ bias) under the causal / key-padding masks, grouped K/V
// heads, optional log-sum-exp output (tensai autograd guide, "Attention の
// 組み立て"; HOF essay section 4, the exact kernel with the n x n scores kept
// out of HBM).
//
// A 32-row query block of D = 1024 has 64 KB of Q and 128 KB of fp32 output:
// more than a wave's registers, so the head dim is split across the waves of
// a workgroup.  Workgroup = NW waves (NW = 4, 6 or 8) and one 32-row block of
// one (batch, query head); wave w owns dims 128w .. 128w+127: its Q rows
// (B operands) and its slice of O^T stay in registers.  Per 16-key tile:
//   A  every wave: partial S^T = K_w Q_w^T over its dims
//      (v_mfma_f32_16x16x32; K fragments straight from HBM into registers,
//      two tiles ahead), written to LDS in fp32 (two buffers, alternating);
//   -  one barrier;
//   B  every wave: each lane sums the NW partials of exactly the scores it
//      feeds to the P.V product (query lane%32, keys 8*(lane/32) .. +7),
//      scales, adds the bias, masks, and runs the online softmax for that
//      row (the row max across the two half-waves by v_permlane32_swap).
//      Every wave computes the same row statistics, so P never leaves the
//      registers and no second barrier is needed;
//   C  every wave: rescale its O^T if a row's max moved, then
//      O^T += V_w^T P^T (v_mfma_f32_32x32x16; V^T by transposed LDS reads
//      from the wave's own V tiles, which arrive by buffer-load DMA two
//      tiles ahead into a 3-stage ring per wave).
// The V tile of step j is issued right before the K fragments of step j, and
// vmcnt counts in issue order, so the compiler's wait for those K fragments
// also covers the V tile: no explicit wait is needed for V.
//
// PAGED: V rows may be Dv wide (Dv != D, the paged plan's value head dim):
// wave w then owns dims 128w .. 128w+127 of both, i.e. the waves cover the
// larger of D and Dv; a wave past D adds zero partial scores, a wave past Dv
// has no output dims.
//
// ELEM (head dims that are not multiples of 8): rows of such a width are not
// 16-byte aligned, so Q, K and V are read one element at a time (2-byte
// buffer loads; elements past the row at out-of-range offsets read as
// zeros) into the same registers and V ring slots the 16-byte loads and the
// DMA would fill, and the output is stored element by element; the decode
// partials' rows are padded to a multiple of 4 floats.
#include "device_common.hpp"
#include "launch.hpp"

namespace sdpa {
namespace {

constexpr int kWRows = 32;       // query rows per workgroup
constexpr int kWKeys = 16;       // keys per tile
constexpr int kWChunk = 128;     // head dims per wave
constexpr int kWVStages = 3;     // V tiles in flight per wave
constexpr uint32_t kWOutside = 0x80000000u;  // buffer offset past any num_records
constexpr float kWLog2e = 1.4426950408889634f;

typedef short w_i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void w_lds_void;

// LDS accessors; the __restrict__ parameters give each inlined access an alias
// scope of its own, so the compiler does not drain the in-flight LDS DMA
// (vmcnt(0)) in front of it.
__device__ __forceinline__ u32x2 w_lds_tr(const uint16_t* __restrict__ p) {
    typedef __attribute__((address_space(3))) w_i16x4 lds_i16x4;
    return __builtin_bit_cast(
        u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((__attribute__((address_space(3))) char*)p)));
}
__device__ __forceinline__ void w_lds_st_f4(float* __restrict__ p, f32x4 v) {
    *(__attribute__((address_space(3))) f32x4*)((__attribute__((address_space(3))) char*)p) = v;
}
__device__ __forceinline__ f32x4 w_lds_ld_f4(const float* __restrict__ p) {
    return *(const __attribute__((address_space(3))) f32x4*)((const __attribute__((address_space(3))) char*)p);
}
__device__ __forceinline__ void w_lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t w_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// 16 bytes (8 elements) of a row from 2-byte loads: element e at byte
// offset off + 2e when e < valid, else zero.
template <int AUX>
__device__ __forceinline__ u32x4 w_elem16(__amdgpu_buffer_rsrc_t r, uint32_t off, int valid) {
    u32x4 v;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(r, 2 * w < valid ? off + 4 * w : kWOutside, 0, AUX);
        const uint32_t hi =
            __builtin_amdgcn_raw_buffer_load_b16(r, 2 * w + 1 < valid ? off + 4 * w + 2 : kWOutside, 0, AUX);
        v[w] = lo | (hi << 16);
    }
    return v;
}

template <int AUX>
__device__ __forceinline__ void w_dma(__amdgpu_buffer_rsrc_t r, uint16_t* lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (w_lds_void*)((__attribute__((address_space(3))) char*)lds), 16,
                                             voff, 0, 0, AUX);
}

// LDS layout (floats / 16-bit elements):
//   partial S: 2 buffers x NW x [32 rows][16 keys] fp32; row q keeps its
//     4-key chunk g at chunk (g + q/4) % 4, so both the 16-byte writes and
//     the 16-byte reads (16 rows, one chunk each) are free of bank conflicts;
//   V: NW x kWVStages x [16 keys][128 dims] 16-bit; row r keeps its 16-byte
//     chunk c at c ^ 4*(r % 4), so a transposed read (4 rows x 64 bytes per
//     32 lanes) touches 16 distinct bank groups.
template <int NW>
struct WideLds {
    static constexpr int PBUF = NW * kWRows * kWKeys;                // floats per partial buffer
    static constexpr int VFL = 2 * PBUF;                             // V, in floats (16-byte aligned)
    static constexpr int VST = kWKeys * kWChunk;                     // 16-bit elements per V stage
    static constexpr int FLOATS = VFL + NW * kWVStages * VST / 2;
};

// x[l] + x[l^32] in every lane (v_permlane32_swap; see max_half_waves).
__device__ __forceinline__ float w_sum_half_waves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                   __builtin_bit_cast(unsigned, x), false, false);
    const unsigned r0 = r[0], r1 = r[1];
    return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
}

__device__ __forceinline__ int w_xcd_order(int total) {
    // workgroup id -> logical index such that each of the 8 XCDs (ids dealt
    // round-robin) owns one contiguous run
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    const int nx = total >> 3, rem = total & 7;
    return xcd * nx + min(xcd, rem) + local;
}

// Extra arguments of the decode form (DEC): a workgroup takes one key range
// (split) of one (batch, K/V head) for up to 32 query heads of its group
// (the rows), Sq = 1, and writes its normalised fp32 partial output and
// natural-log lse into the split-KV workspace for the merge pass.
//
// PAGED: K and V come from page caches [pages, page_size, Hkv, D] through a
// sequence's page table.  A 16-key tile lies in one page (page sizes are
// multiples of 16), found with one table lookup; an entry outside
// [0, pages) is never dereferenced (no records: zeros) and its keys are
// masked.  With DEC (paged attention, B = queries): a query sees the keys
// below its sequence's length and, under the causal flag, up to its
// absolute position; split lengths are multiples of 16.  Without DEC
// (prefill chunks, B = sequences, Sq = the longest chunk): the workgroup's
// rows are rows q0 .. q0+31 of sequence b's chunk, packed rows
// cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 of q / out ([rows, Hq, D]), and row i
// sits at absolute position seq_lens[b] - n_b + i.
struct WideDec {
    float* o_part;    // [B, Hq, splits, D]
    float* lse_part;  // [B, Hq, splits]
    int splits;
    const int32_t* tables;     // [num_seqs, max_pages]   (PAGED)
    const int32_t* seq_lens;   // [num_seqs]
    const int32_t* query_seq;  // [queries]
    const int32_t* query_pos;  // [queries]
    int num_seqs, max_pages, pages, page_size;
    bool causal;
    const int32_t* cu_q;  // [num_seqs + 1]  (PAGED prefill chunks)
    int total_q;
};

template <int NW, class T, bool BIAS, bool DEC, bool PAGED = false, bool ELEM = false>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 2 : 1) void forward_wide_kernel(
    ForwardArgs a, const int32_t* __restrict__ key_lens, WideDec dec, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ query_seq,
    const int32_t* __restrict__ query_pos) {

    using LY = WideLds<NW>;
    // K/V cache policy: the decode forms read each K/V byte once (streamed,
    // non-temporal); the prefill forms re-read a head's K/V from L2.
    constexpr int kKVPolicy = DEC ? 2 : 0;
    __shared__ __attribute__((aligned(1024))) float smem[LY::FLOATS];
    float* const part = smem;
    uint16_t* const vring = reinterpret_cast<uint16_t*>(smem + LY::VFL);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int D = a.D;
    const int Dv = a.Dv > 0 ? a.Dv : D;  // value / output head dim

    // Logical order: (batch, K/V head) outermost, then query blocks (under a
    // causal mask the longest first), then the query heads of the group.
    // DEC: (batch, K/V head), then splits, then blocks of 32 query heads.
    const int G = a.Hq / a.Hkv;
    int b, gk, h, q0, split = 0, hb = 0;
    if constexpr (DEC) {
        const int nhb = (G + kWRows - 1) / kWRows;
        int t = w_xcd_order(a.B * a.Hkv * dec.splits * nhb);
        hb = t % nhb;
        t /= nhb;
        split = t % dec.splits;
        const int unit = t / dec.splits;
        b = unit / a.Hkv;
        gk = unit % a.Hkv;
        h = gk * G + kWRows * hb;  // head of row 0
        q0 = 0;
    } else {
        const int nqb = (a.Sq + kWRows - 1) / kWRows;
        int t = w_xcd_order(a.B * a.Hkv * nqb * G);
        const int hsub = t % G;
        t /= G;
        const int qord = t % nqb;
        const int unit = t / nqb;
        b = unit / a.Hkv;
        gk = unit % a.Hkv;
        h = gk * G + hsub;
        q0 = (a.causal ? nqb - 1 - qord : qord) * kWRows;
    }
    const int64_t bh = (int64_t)b * a.Hq + h;

    // Visible keys [k_lo, kv_lim): DEC takes its split's range.  PAGED
    // prefill: this sequence's chunk rows (qbase, qstride) and the absolute
    // position qpos0 of its first row.
    int kv_lim = a.Sk, k_lo = 0, seq = 0, nrows = a.Sq, qpos0 = 0;
    int r0 = 0;  // PAGED prefill: the chunk's first packed row
    const uint16_t* qbase = static_cast<const uint16_t*>(a.q) + bh * a.Sq * D;
    uint16_t* obase = static_cast<uint16_t*>(a.out) + bh * a.Sq * Dv;
    int64_t qstride = D, ostride = Dv;
    if (a.padded) kv_lim = max(0, min(kv_lim, key_lens[b]));
    if constexpr (PAGED && !DEC) {
        r0 = min(max(dec.cu_q[b], 0), dec.total_q);
        const int r1 = min(max(dec.cu_q[b + 1], r0), dec.total_q);
        nrows = r1 - r0;
        if (q0 >= nrows) return;  // the whole workgroup, before any barrier
        seq = b;
        kv_lim = min(seq_lens[b], a.Sk);
        qpos0 = kv_lim - nrows;
        const int64_t rb = (int64_t)r0 * a.Hq + h;
        qbase = static_cast<const uint16_t*>(a.q) + rb * D;
        obase = static_cast<uint16_t*>(a.out) + rb * Dv;
        qstride = (int64_t)a.Hq * D;
        ostride = (int64_t)a.Hq * Dv;
    }
    if constexpr (PAGED && DEC) {
        seq = query_seq[b];
        if (seq >= 0 && seq < dec.num_seqs) {
            kv_lim = min(kv_lim, seq_lens[seq]);
            if (dec.causal) kv_lim = min(kv_lim, query_pos[b] + 1);
        } else {
            kv_lim = 0;
        }
    }
    if constexpr (DEC) {
        int chunk = (a.Sk + dec.splits - 1) / dec.splits;
        if (PAGED) chunk = (chunk + kWKeys - 1) / kWKeys * kWKeys;  // whole tiles per split
        k_lo = split * chunk;
        kv_lim = min(kv_lim, k_lo + chunk);
    }
    int kv_end = kv_lim;
    if (a.causal) kv_end = min(kv_end, qpos0 + q0 + kWRows);
    const int ntiles = kv_end > k_lo ? (kv_end - k_lo + kWKeys - 1) / kWKeys : 0;

    const int d0 = kWChunk * wave;  // this wave's first dim
    const int64_t kvh = ((int64_t)b * a.Hkv + gk) * a.Sk;
    const __amdgpu_buffer_rsrc_t rk = w_rsrc(static_cast<const uint16_t*>(a.k) + kvh * D, (uint32_t)a.Sk * D * 2);
    const __amdgpu_buffer_rsrc_t rv =
        w_rsrc(static_cast<const uint16_t*>(a.v) + kvh * Dv, (uint32_t)a.Sk * Dv * 2);
    // Where the 16 keys from kt live: dense, rows of D (V: Dv) from the head's
    // start; PAGED, rows of Hkv*D (V: Hkv*Dv) in the tile's page (head gk's
    // columns), or no records at all for an invalid table entry.
    struct Src {
        __amdgpu_buffer_rsrc_t k, v;
        uint32_t row0, rstride, col0, vrstride, vcol0;
        bool ok;
    };
    auto src = [&](int kt) -> Src {
        if constexpr (PAGED) {
            const int lp = kt / dec.page_size;
            const int pg = lp < dec.max_pages ? tables[(int64_t)seq * dec.max_pages + lp] : -1;
            const bool ok = pg >= 0 && pg < dec.pages;
            const int64_t off = ok ? (int64_t)pg * dec.page_size * a.Hkv : 0;
            return Src{w_rsrc(static_cast<const uint16_t*>(a.k) + off * D,
                              ok ? (uint32_t)dec.page_size * a.Hkv * D * 2 : 0u),
                       w_rsrc(static_cast<const uint16_t*>(a.v) + off * Dv,
                              ok ? (uint32_t)dec.page_size * a.Hkv * Dv * 2 : 0u),
                       (uint32_t)(kt % dec.page_size), (uint32_t)(a.Hkv * D), (uint32_t)(gk * D),
                       (uint32_t)(a.Hkv * Dv), (uint32_t)(gk * Dv), ok};
        } else {
            return Src{rk, rv, (uint32_t)kt, (uint32_t)D, 0u, (uint32_t)Dv, 0u, true};
        }
    };

    // Q^T as B operands of the 16x16x32 products: column 16qb + lane%16 (a
    // query), dims d0 + 32s + 8*(lane/16) .. +7 (rows past Sq and dims past D
    // read as zeros).
    const int l16 = lane & 15, g4 = lane >> 4;
    u32x4 qf[2][4];
    {
        // DEC: row r is query head h + r (one query each; heads past the group
        // read as zeros), so the rows form [G - 32hb, D] from head h on.
        const int nq = DEC ? G - kWRows * hb : nrows;
        const __amdgpu_buffer_rsrc_t rq = w_rsrc(qbase, (uint32_t)((nq - 1) * qstride + D) * 2);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int row = q0 + 16 * qb + l16, dim = d0 + 32 * s + 8 * g4;
                const uint32_t off = (row < nq && dim < D) ? ((uint32_t)(row * qstride) + dim) * 2 : kWOutside;
                if constexpr (ELEM)
                    qf[qb][s] = w_elem16<0>(rq, off, D - dim);
                else
                    qf[qb][s] = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
            }
    }
    // K fragments (A operands): key kt + lane%16, dims d0 + 32s + 8*(lane/16).
    auto load_k = [&](int kt, u32x4* kf) {
        const Src sr = src(kt);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int dim = d0 + 32 * s + 8 * g4;
            const uint32_t off = dim < D ? ((sr.row0 + l16) * sr.rstride + sr.col0 + dim) * 2 : kWOutside;
            if constexpr (ELEM)
                kf[s] = w_elem16<kKVPolicy>(sr.k, off, D - dim);
            else
                kf[s] = __builtin_amdgcn_raw_buffer_load_b128(sr.k, off, 0, kKVPolicy);
        }
    };
    // V tile of keys kt .. kt+15, this wave's dims, into ring stage st: DMA i
    // fills rows 4i + lane/16, stored chunk lane%16 (logical chunk
    // (lane%16) ^ 4*(lane/16)); keys past Sk read as zeros.
    uint16_t* const vw = vring + wave * kWVStages * LY::VST;
    const int vchunk = (lane & 15) ^ (4 * g4);
    const bool vdim_ok = d0 + 8 * vchunk < Dv;
    auto load_v = [&](int kt, int st) {
        const Src sr = src(kt);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t off =
                vdim_ok ? ((sr.row0 + 4 * i + g4) * sr.vrstride + sr.vcol0 + d0 + 8 * vchunk) * 2 : kWOutside;
            if constexpr (ELEM)  // the slot the DMA would fill: 16 bytes at lane * 16
                *reinterpret_cast<u32x4*>(vw + st * LY::VST + 512 * i + 8 * lane) =
                    w_elem16<kKVPolicy>(sr.v, off, Dv - (d0 + 8 * vchunk));
            else
                w_dma<kKVPolicy>(sr.v, vw + st * LY::VST + 512 * i, off);
        }
    };
    // Transposed-read offsets (32x32x16 A operand = V^T): lane reads rows
    // (keys) 8*(lane/32) + (lane%16)/4 (+4 for the upper half), dims
    // 32db + 16*((lane/16)%2) + 4*(lane%4).
    int vtr[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const int row = 8 * (g4 >> 1) + (l16 >> 2);
        const int col = 32 * db + 16 * (g4 & 1) + 4 * (l16 & 3);
        vtr[db] = row * kWChunk + (((col >> 3) ^ (4 * (row & 3))) * 8) + (col & 7);
    }
    // (row + 4 has the same swizzle term as row: (row + 4) % 4 == row % 4)

    f32x16 acc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[db] = f32x16{};

    // Softmax state of this lane's row: query qr = lane%32, keys 8*kh .. +7 of
    // each tile (the lane's P^T operand); m_run is the same in both halves.
    const int qr = lane & 31, kh = lane >> 5;
    const int qa = q0 + qr;
    float m_run = -INFINITY, l_part = 0.f;
    const float c = a.scale * kWLog2e;
    const __amdgpu_buffer_rsrc_t rb =
        w_rsrc(BIAS ? static_cast<const uint16_t*>(a.bias) + b * a.bias_sb + h * a.bias_sh
                    : static_cast<const uint16_t*>(a.q),
               BIAS ? (uint32_t)a.Sq * a.Sk * 2 : 0u);
    // this lane's two 4-key chunks (2kh, 2kh+1) of a partial row
    const int poff0 = qr * kWKeys + (((2 * kh + (qr >> 2)) & 3) * 4);
    const int poff1 = qr * kWKeys + (((2 * kh + 1 + (qr >> 2)) & 3) * 4);

    // K fragments: a ring of three tiles (this one and the next two).
    u32x4 kr0[4], kr1[4], kr2[4];
    if (ntiles > 0) load_v(k_lo, 0);
    asm volatile("" ::: "memory");
    if (ntiles > 0) load_k(k_lo, kr0);
    asm volatile("" ::: "memory");
    if (ntiles > 1) load_v(k_lo + kWKeys, 1);
    asm volatile("" ::: "memory");
    if (ntiles > 1) load_k(k_lo + kWKeys, kr1);

    auto tile = [&](int j, u32x4* kc, u32x4* kn2) __attribute__((always_inline)) {
        const int kt = k_lo + j * kWKeys;
        float* const pb = part + (j & 1) * LY::PBUF;
        // (BIAS) this lane's 8 bias values first, so that waiting for them
        // does not wait for the loads issued below
        u32x4 bw = {0u, 0u, 0u, 0u};
        if constexpr (BIAS) {
            const int key = kt + 8 * kh;
            bw = __builtin_amdgcn_raw_buffer_load_b128(
                rb, (qa < a.Sq && key < a.Sk) ? ((uint32_t)qa * a.Sk + key) * 2 : kWOutside, 0, 0);
        }
        // V and K two tiles ahead, V first: the wait for K(j+2) two tiles
        // from now then also covers V(j+2)
        if (j + 2 < ntiles) load_v(kt + 2 * kWKeys, (j + 2) % kWVStages);
        asm volatile("" ::: "memory");
        if (j + 2 < ntiles) load_k(kt + 2 * kWKeys, kn2);

        // A: partial S^T over this wave's dims; register i of block qb holds
        // key kt + 4*(lane/16) + i of query 16qb + lane%16.
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 4; ++st) sacc = mfma_16x16x32<T>(kc[st], qf[qb][st], sacc);
            const int q = 16 * qb + l16;
            w_lds_st_f4(pb + wave * (kWRows * kWKeys) + q * kWKeys + (((g4 + (q >> 2)) & 3) * 4), sacc);
        }
        // The buffer written here was last read in tile j-2, and every wave
        // finished those reads before the previous tile's barrier: one
        // barrier per tile suffices.
        w_lds_barrier();

        // B: this lane's 8 scores, keys kt + 8kh + e.
        float x[8];
        {
            f32x4 s0 = w_lds_ld_f4(pb + poff0), s1 = w_lds_ld_f4(pb + poff1);
#pragma unroll
            for (int w = 1; w < NW; ++w) {
                s0 += w_lds_ld_f4(pb + w * (kWRows * kWKeys) + poff0);
                s1 += w_lds_ld_f4(pb + w * (kWRows * kWKeys) + poff1);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[e] = s0[e] * c;
                x[4 + e] = s1[e] * c;
            }
        }
        if constexpr (BIAS) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t wv = bw[e >> 1];
                x[e] = fmaf(bias_elem<T>(wv, e & 1), kWLog2e, x[e]);
            }
        }
        const int key0 = kt + 8 * kh;
        if constexpr (PAGED) {
            if (!src(kt).ok) {  // the tile's page is invalid: its keys are hidden
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = -INFINITY;
            }
        }
        const int qp = qpos0 + qa;  // this row's absolute position
        const bool edge = key0 + 8 > kv_lim || (a.causal && key0 + 7 > qp);
        if (edge) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (key0 + e >= kv_lim || (a.causal && key0 + e > qp)) x[e] = -INFINITY;
        }
        // Weights against the current reference max; the reference moves only
        // when a tile max exceeds it by 2^8 (log2 units), so O and l, which
        // share the stale reference, rarely need rescaling.  A lane sum of at
        // most 2^8 proves each of its (non-negative) weights is at most 2^8,
        // so the tile max is only taken when a sum is larger or before the
        // row has a reference.  Every wave holds the same summed scores and
        // takes the same decisions.
        u32x4 pf;
        auto weights = [&]() -> float {
            const float mu = m_run == -INFINITY ? 0.f : m_run;
            float ws = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pf[e] = pack2<T>(fast_exp2(x[2 * e] - mu), fast_exp2(x[2 * e + 1] - mu));
                ws = sum2<T>(pf[e], ws);
            }
            return ws;
        };
        float ls = weights();
        if (__any(ls > 256.f || m_run == -INFINITY)) {
            float tmax = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                               fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
            tmax = max_half_waves(tmax);
            if (__any(tmax > m_run + 8.f)) {
                const float m_new = fmaxf(m_run, tmax);
                const float m_use = m_new == -INFINITY ? 0.f : m_new;
                const float alpha = fast_exp2(m_run - m_use);  // 0 while the row had no key
                m_run = m_new;
                l_part *= alpha;
                // C (first part): rescale O^T to the new reference
#pragma unroll
                for (int db = 0; db < 4; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
            }
            ls = weights();
        }
        l_part += ls;

        // C: O^T += V^T P^T over this wave's dims (column = query lane%32).
        const uint16_t* vs = vw + (j % kWVStages) * LY::VST;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const u32x2 lo = w_lds_tr(vs + vtr[db]);
            const u32x2 hi = w_lds_tr(vs + vtr[db] + 4 * kWChunk);
            acc[db] = mfma_32x32x16<T>(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf, acc[db]);
        }
    };
    for (int j = 0; j < ntiles; j += 3) {
        tile(j, kr0, kr2);
        if (j + 1 < ntiles) tile(j + 1, kr1, kr0);
        if (j + 2 < ntiles) tile(j + 2, kr2, kr1);
    }

    // Row sum (both halves) and log-sum-exp.
    const float l = w_sum_half_waves(l_part);
    if constexpr (DEC) {
        // normalised partial (0 for a split with no visible key, whose lse
        // is -inf and weight 0 in the merge)
        const int hr = kWRows * hb + qr;  // head within the group
        if (hr >= G) return;
        const int64_t prow = (bh + qr) * dec.splits + split;
        const float invd = l > 0.f ? 1.f / l : 0.f;
        if (wave == 0 && kh == 0) {
            const float m_use = m_run == -INFINITY ? 0.f : m_run;
            dec.lse_part[prow] = l > 0.f ? (m_use + __log2f(l)) * 0.69314718055994531f : -INFINITY;
        }
        const int DP = ELEM ? (Dv + 3) & ~3 : Dv;  // floats per partial row
        float* orow = dec.o_part + prow * DP;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int dim = d0 + 32 * db + 8 * r4 + 4 * kh;
                const f32x16& xo = acc[db];
                if (dim < Dv)
                    *reinterpret_cast<f32x4*>(orow + dim) =
                        f32x4{xo[4 * r4] * invd, xo[4 * r4 + 1] * invd, xo[4 * r4 + 2] * invd,
                              xo[4 * r4 + 3] * invd};
            }
        return;
    }
    const float inv = 1.f / l;  // a row with no visible key: 0 * inf = NaN
    // log-sum-exp of the row (natural log; -inf with no visible key): dense
    // [B, Hq, Sq], paged prefill [packed rows, Hq]
    if (wave == 0 && kh == 0 && a.lse && qa < nrows) {
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
        a.lse[PAGED ? (int64_t)(r0 + qa) * a.Hq + h : bh * a.Sq + qa] = (m_use + __log2f(l)) * 0.69314718055994531f;
    }

    // O: register r of d-block db holds dim d0 + 32db + 8*(r/4) + 4*(lane/32)
    // + r%4 of query q0 + lane%32.
    if (qa < nrows) {
        uint16_t* row = obase + qa * ostride;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int dim = d0 + 32 * db + 8 * r4 + 4 * kh;
                const f32x16& xo = acc[db];
                const u32x2 w = {pack2<T>(xo[4 * r4] * inv, xo[4 * r4 + 1] * inv),
                                 pack2<T>(xo[4 * r4 + 2] * inv, xo[4 * r4 + 3] * inv)};
                if constexpr (ELEM) {  // element by element: the row need not be 8-byte aligned
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (dim + e < Dv) row[dim + e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
                } else if (dim < Dv) {
                    *reinterpret_cast<u32x2*>(row + dim) = w;
                }
            }
    }
}

// The waves cover the larger of the key and value head dims.
inline int wide_dims(const ForwardArgs& a) { return a.Dv > a.D ? a.Dv : a.D; }
inline bool wide_elem(const ForwardArgs& a) { return a.D % 8 != 0 || (a.Dv > 0 && a.Dv % 8 != 0); }

template <int NW, class T>
hipError_t launch_wide_nw(const ForwardArgs& a, hipStream_t s) {
    const int nqb = (a.Sq + kWRows - 1) / kWRows;
    const dim3 grid((unsigned)(a.B * a.Hq * nqb));
    const int32_t* none = nullptr;
    if (a.D % 8 != 0) {
        if (a.bias) return hipErrorInvalidValue;
        hipLaunchKernelGGL((forward_wide_kernel<NW, T, false, false, false, true>), grid, dim3(NW * 64), 0, s, a,
                           a.key_lens, WideDec{}, none, none, none, none);
    } else if (a.bias)
        hipLaunchKernelGGL((forward_wide_kernel<NW, T, true, false>), grid, dim3(NW * 64), 0, s, a, a.key_lens,
                           WideDec{}, none, none, none, none);
    else
        hipLaunchKernelGGL((forward_wide_kernel<NW, T, false, false>), grid, dim3(NW * 64), 0, s, a, a.key_lens,
                           WideDec{}, none, none, none, none);
    return hipGetLastError();
}

template <int NW, class T, bool PAGED>
hipError_t launch_wide_dec_nw(const ForwardArgs& a, const WideDec& d, hipStream_t s) {
    const int nhb = (a.Hq / a.Hkv + kWRows - 1) / kWRows;
    const dim3 grid((unsigned)(a.B * a.Hkv * d.splits * nhb));
    if (wide_elem(a))
        hipLaunchKernelGGL((forward_wide_kernel<NW, T, false, true, PAGED, true>), grid, dim3(NW * 64), 0, s, a,
                           a.key_lens, d, d.tables, d.seq_lens, d.query_seq, d.query_pos);
    else
        hipLaunchKernelGGL((forward_wide_kernel<NW, T, false, true, PAGED>), grid, dim3(NW * 64), 0, s, a,
                           a.key_lens, d, d.tables, d.seq_lens, d.query_seq, d.query_pos);
    return hipGetLastError();
}

template <class T, bool PAGED>
hipError_t launch_wide_dec_t(const ForwardArgs& a, const WideDec& d, hipStream_t s) {
    if (wide_dims(a) <= 4 * kWChunk) return launch_wide_dec_nw<4, T, PAGED>(a, d, s);
    if (wide_dims(a) <= 6 * kWChunk) return launch_wide_dec_nw<6, T, PAGED>(a, d, s);
    return launch_wide_dec_nw<8, T, PAGED>(a, d, s);
}

template <class T>
hipError_t launch_wide_t(const ForwardArgs& a, hipStream_t s) {
    if (a.D <= 4 * kWChunk) return launch_wide_nw<4, T>(a, s);
    if (a.D <= 6 * kWChunk) return launch_wide_nw<6, T>(a, s);
    return launch_wide_nw<8, T>(a, s);
}

}  // namespace

hipError_t launch_forward_wide(const ForwardArgs& a, bool f16, hipStream_t s) {
    if (a.D <= 256 || a.D > 1024) return hipErrorInvalidValue;
    return f16 ? launch_wide_t<F16T>(a, s) : launch_wide_t<Bf16T>(a, s);
}

template <int NW, class T>
hipError_t launch_wide_paged_nw(const ForwardArgs& a, const WideDec& d, hipStream_t s) {
    const int nqb = (a.Sq + kWRows - 1) / kWRows;
    const dim3 grid((unsigned)(a.B * a.Hq * nqb));
    if (wide_elem(a))
        hipLaunchKernelGGL((forward_wide_kernel<NW, T, false, false, true, true>), grid, dim3(NW * 64), 0, s, a,
                           nullptr, d, d.tables, d.seq_lens, nullptr, nullptr);
    else
        hipLaunchKernelGGL((forward_wide_kernel<NW, T, false, false, true>), grid, dim3(NW * 64), 0, s, a, nullptr,
                           d, d.tables, d.seq_lens, nullptr, nullptr);
    return hipGetLastError();
}

template <class T>
hipError_t launch_wide_paged_t(const ForwardArgs& a, const WideDec& d, hipStream_t s) {
    if (wide_dims(a) <= 4 * kWChunk) return launch_wide_paged_nw<4, T>(a, d, s);
    if (wide_dims(a) <= 6 * kWChunk) return launch_wide_paged_nw<6, T>(a, d, s);
    return launch_wide_paged_nw<8, T>(a, d, s);
}

hipError_t launch_paged_prefill_wide(const ForwardArgs& a, const PagedArgs& p, bool f16, hipStream_t s) {
    if (wide_dims(a) <= 256 || wide_dims(a) > 1024 || a.D < 1 || a.Dv < 1) return hipErrorInvalidValue;
    WideDec w{};
    w.tables = p.block_tables;
    w.seq_lens = p.seq_lens;
    w.num_seqs = p.num_seqs;
    w.max_pages = p.max_pages;
    w.pages = p.pages;
    w.page_size = p.page_size;
    w.cu_q = p.cu_seqlens_q;
    w.total_q = p.total_q;
    ForwardArgs b = a;
    b.bias = nullptr;
    b.padded = false;
    return f16 ? launch_wide_paged_t<F16T>(b, w, s) : launch_wide_paged_t<Bf16T>(b, w, s);
}

hipError_t launch_decode_wide_split(const DecodeArgs& d, const PagedArgs* p, bool f16, hipStream_t s) {
    const int dv = d.Dv > 0 ? d.Dv : d.D;
    if ((d.D <= 256 && dv <= 256) || d.D > 1024 || dv > 1024 || (!p && dv != d.D)) return hipErrorInvalidValue;
    ForwardArgs a;
    a.q = d.q;
    a.k = d.k;
    a.v = d.v;
    a.out = nullptr;
    a.key_lens = d.key_lens;
    a.B = d.B;
    a.Hq = d.Hq;
    a.Hkv = d.Hkv;
    a.Sq = 1;
    a.Sk = d.Sk;
    a.D = d.D;
    a.Dv = dv;
    a.scale = d.scale;
    a.causal = false;
    a.padded = d.key_lens != nullptr;
    WideDec w{};
    w.o_part = d.o_part;
    w.lse_part = d.lse_part;
    w.splits = d.splits;
    if (p) {
        w.tables = p->block_tables;
        w.seq_lens = p->seq_lens;
        w.query_seq = p->query_seq;
        w.query_pos = p->query_pos;
        w.num_seqs = p->num_seqs;
        w.max_pages = p->max_pages;
        w.pages = p->pages;
        w.page_size = p->page_size;
        w.causal = p->causal;
        return f16 ? launch_wide_dec_t<F16T, true>(a, w, s) : launch_wide_dec_t<Bf16T, true>(a, w, s);
    }
    return f16 ? launch_wide_dec_t<F16T, false>(a, w, s) : launch_wide_dec_t<Bf16T, false>(a, w, s);
}

}  // namespace sdpa
