// Single-query decode with split-KV and a log-sum-exp merge (ruDNN user guide,
// section 9: the history is split into 2..=32 pieces whose partial statistics
// and merge are kept in FP32).  The split pass is memory bound: every byte of
// K and V of a (batch, K/V head) is read once for up to 16 query heads that
// share it.
//
// Split pass: a persistent grid, one workgroup of 4 independent waves per
// compute unit.  A work item is (batch, K/V head, block of <= 16 query heads,
// split).  A workgroup owns a contiguous run of items and its waves take them
// in turn (wave w: items w, w+4, ...), so at any time the 4 waves stream 4
// neighbouring splits of one head.  A wave computes each of its items whole
// and writes its normalised partial output and log-sum-exp; its K/V loads
// form one stream across items, so the prefetch never drains at a split
// boundary.  K and V are loaded non-temporally: each byte is read once.
//
// Merge pass: O = sum_s exp(lse_s - M) O_s / sum_s exp(lse_s - M), with
// M = max_s lse_s, one thread per (batch, query head, 4 dims).
#include <atomic>

#include "device_common.hpp"
#include "launch.hpp"

namespace sdpa {
namespace {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = 4;
constexpr int kQ = 16;              // query heads per item (the 16 MFMA columns)
constexpr int kStep = 16;           // keys per step
constexpr float kTau = 8.0f;        // lazy-rescale threshold, log2 units
constexpr int kRingBytes = 32768;   // LDS ring per wave
constexpr int kNonTemporal = 2;     // buffer-load cache policy: nt (streamed once)

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

// Transposed read of 4 bf16.  The __restrict__ parameter gives the inlined load
// its own alias scope, which keeps the compiler from putting a vmcnt(0) drain
// of the in-flight LDS-DMA writes in front of it (those are ordered by the
// explicit waits instead).
__device__ __forceinline__ u32x2 lds_read_tr(const uint16_t* __restrict__ p) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    lds_i16x4* lp = (lds_i16x4*)((__attribute__((address_space(3))) char*)p);
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(lp));
}
__device__ __forceinline__ u32x4 lds_read128(const uint16_t* __restrict__ p) {
    return *(lds_u32x4*)((__attribute__((address_space(3))) char*)p);
}
// fp32x4 LDS store / load of the cross-wave merge (same alias-scope reason).
__device__ __forceinline__ void lds_store_f32x4(float* __restrict__ p, f32x4 v) {
    typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
    *(lds_f32x4*)((__attribute__((address_space(3))) char*)p) = v;
}
__device__ __forceinline__ f32x4 lds_load_f32x4(const float* __restrict__ p) {
    typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
    return *(lds_f32x4*)((__attribute__((address_space(3))) char*)p);
}
template <typename T>
__device__ __forceinline__ void lds_store(T* __restrict__ p, T v) {
    *(__attribute__((address_space(3))) T*)((__attribute__((address_space(3))) char*)p) = v;
}
template <typename T>
__device__ __forceinline__ T lds_load(const T* __restrict__ p) {
    return *(const __attribute__((address_space(3))) T*)((const __attribute__((address_space(3))) char*)p);
}
// Workgroup barrier for LDS traffic only: this wave's LDS accesses complete,
// then s_barrier.  (__syncthreads() also waits for every outstanding global
// access, which would drain the K/V loads in flight.)  The memory clobbers keep
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}
// 16 bytes per lane from a buffer straight into LDS (lane l's bytes land at
// lds + 16*l); voff is per lane, soff wave-uniform.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint16_t* lds, uint32_t voff,
                                      uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (lds_void*)((__attribute__((address_space(3))) char*)lds), 16, voff, soff, 0, kNonTemporal);
}

template <int D>
struct DecGeo {
    static constexpr int CPR = D / 8;                  // 16-byte chunks per row
    static constexpr int RPW = D > 128 ? 1 : 256 / (2 * D);  // rows per 256-byte bank window (1: a row spans two)
    static constexpr int TILE = kStep * D;             // bf16 elements of one K or V step
    static constexpr int STAGE = 2 * TILE;             // K tile, then V tile
    static constexpr int DMA = TILE * 2 / 1024;        // 1-KB DMA loads per tile
    static constexpr int OPS = 2 * DMA;                // vector memory ops per step
    static constexpr int KSTEPS = D / 32;              // MFMA contraction steps of S
    // K chunk swizzle: the 16 rows one 16-lane ds_read_b128 touches (same
    // logical chunk) land on 16 distinct 16-byte bank groups.
    __device__ static int fk(int r) { return (r / RPW) % CPR; }
    // V chunk swizzle: the 8 rows x 32 B one 32-lane transposed read touches
    // fall on 16 distinct 16-byte bank groups.
    __device__ static int fv(int r) { return 2 * ((r / RPW) % (8 / RPW)); }
};

// Per-launch metadata pointers, each read with scalar loads (hence separate
// __restrict__ kernel arguments rather than struct members).
struct Meta {
    const int32_t* __restrict__ key_lens;   // dense: [B] or null
    const int32_t* __restrict__ tables;     // paged: [num_seqs, max_pages]
    const int32_t* __restrict__ seq_lens;   // paged: [num_seqs]
    const int32_t* __restrict__ query_seq;  // paged: [queries]
    const int32_t* __restrict__ query_pos;  // paged: [queries]
};

// Geometry of one work item.  b is the batch (dense) or the query (paged); seq
// the query's sequence (paged, -1 if out of range).
struct Item {
    int b, gk, h0, nh, split, lo, hi, nst, seq;
};

template <bool PAGED>
__device__ __forceinline__ Item item_geo(const DecodeArgs& a, const PagedArgs& p, const Meta& m,
                                         int it, int G, int nqc, int chunk) {
    Item g;
    g.split = it % a.splits;
    int r = it / a.splits;
    const int qc = r % nqc;
    r /= nqc;
    g.gk = r % a.Hkv;
    g.b = r / a.Hkv;
    g.h0 = g.gk * G + qc * kQ;
    g.nh = min(kQ, G - qc * kQ);
    int len = a.Sk;
    g.seq = -1;
    if (PAGED) {
        // Visible keys of query b: j < seq_lens[seq] (capped at max_seq_len)
        // and, under the causal flag, j <= its absolute position.  A sequence
        // id outside [0, num_seqs) leaves nothing visible.
        const int s = m.query_seq[g.b];
        if (s >= 0 && s < p.num_seqs) {
            g.seq = s;
            len = min(len, m.seq_lens[s]);
            if (p.causal) len = min(len, m.query_pos[g.b] + 1);
        } else {
            len = 0;
        }
    } else if (m.key_lens) {
        len = min(len, m.key_lens[g.b]);
    }
    g.lo = g.split * chunk;
    g.hi = min(g.lo + chunk, len);
    g.nst = g.hi > g.lo ? (g.hi - g.lo + kStep - 1) / kStep : 0;
    return g;
}

// Split pass.  Per 16-key step of an item, in one wave:
//   S^T[16 keys x 16 queries] = K Q^T   D/32 v_mfma_f32_16x16x32_bf16
//   O^T[D x 16 queries]      += V^T P^T  D/16 v_mfma_f32_16x16x16_bf16
// K and V of a step go HBM -> LDS by buffer-load DMA into the wave's private
// ring of NS stages, NS-1 steps ahead; K comes back with ds_read_b128 (the A
// operand), V transposed with ds_read_b64_tr_b16.  Lane l owns query column
// l % 16; its 4 scores per step are keys 4*(l/16) + i, exactly the 4
// contraction slots it feeds to the P.V product.  The kernel has no
// workgroup barrier: every wave runs its own items start to end.
//
// DV: on-chip width of V and of the partial output (the value head dim Dv,
// which may differ from D: ruDNN user guide section 9); K tiles are D wide,
// V tiles DV wide, each with its own swizzle and DMA count.
//
// PAGED: K and V come from page caches [pages, page_size, Hkv, D] and
// [.., Dv]; a step's
// 16 keys lie in one page (page_size and the split length are multiples of
// 16), found through the sequence's page table when the step enters a new
// page.  A table entry outside [0, pages) is never dereferenced: its keys
// load as zeros and are masked out.
// ELEM (with GEN; head dims that are not multiples of 8): Q, K and V are
// read one element at a time (2-byte buffer loads into the lanes' 16-byte
// slots, elements past a row reading as zeros), loaded and written to the
// ring at issue time; the partials' rows are padded to a multiple of 4
// floats (DVP) so their 16-byte stores stay aligned.
template <int D, bool PAGED, class T, bool GEN = false, int DV = D, bool ELEM = false>
__global__ __launch_bounds__(kDecThreads, 1) void decode_split_bf16_kernel(
    DecodeArgs a, PagedArgs p, const int32_t* __restrict__ key_lens,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ query_seq, const int32_t* __restrict__ query_pos, int items) {
    using L = DecGeo<D>;    // K
    using LV = DecGeo<DV>;  // V
    constexpr int STAGE = L::TILE + LV::TILE;          // K tile, then V tile
    // Parked partials (kPark): items with at most 4 query heads leave their
    // partial and lse in LDS, behind the rings, and a wave writes them out
    // KPARK items at a time.  The ring loads issued after a store cannot
    // retire before it (vmcnt retires in issue order), so one flush every
    // KPARK items holds the stream back once instead of KPARK times (the
    // flush after a wave's last item holds nothing back).  The 128-wide form
    // gives up a ring stage (24 KB per wave) for 7 slots.
    constexpr bool kPark = !GEN && !ELEM && DV == 128;
    constexpr bool kDeep = kPark && D == 128;
    constexpr int NS = (kDeep ? 24576 : kRingBytes) / (2 * STAGE);  // ring stages per wave
    constexpr int OPS = L::DMA + LV::DMA;              // vector memory ops per step
    static_assert(NS >= 2, "ring depth");
    const Meta meta{key_lens, tables, seq_lens, query_seq, query_pos};
    constexpr int KPARK = kDeep ? 7 : 3;
    constexpr int PSLOT = 4 * DV + 4;  // floats: 4 rows of DV, then 4 lse values
    constexpr int PARK = kPark ? kDecWaves * KPARK * PSLOT * 2 : 0;  // 16-bit units
    __shared__ __attribute__((aligned(1024))) uint16_t smem[kDecWaves * NS * STAGE + PARK];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int col = lane & 15;  // query column (and key row of the S^T tile)
    const int grp = lane >> 4;  // lane group

    // The workgroup owns items [wg0, it1); wave w takes wg0 + w, wg0 + w + 4, ...
    // so the 4 waves stream 4 neighbouring splits at a time.
    const int wg0 = (int)((int64_t)blockIdx.x * items / gridDim.x);
    const int it1 = (int)((int64_t)(blockIdx.x + 1) * items / gridDim.x);
    const int it0 = wg0 + wave;
    if (it0 >= it1) return;

    const int G = a.Hq / a.Hkv;
    const int nqc = (G + kQ - 1) / kQ;
    // Split length: ceil(Sk / splits) keys (paged: rounded up to a multiple of
    // the 16-key step, so no step crosses a page).
    int chunk = (a.Sk + a.splits - 1) / a.splits;
    if (PAGED) chunk = (chunk + kStep - 1) / kStep * kStep;
    const float c = a.scale * kLog2e;
    const float tau = kTau / c;
    // Head dim in memory: DR (GEN: a multiple of 8 below D; else D).  Rows
    // are DR wide in HBM and D wide on chip; chunks at or past DR read as
    // zeros (offsets outside the buffer) and are never stored.
    const int DR = GEN ? a.D : D;
    const int DVR = GEN ? a.Dv : DV;  // value head dim in memory
    const int DVP = ELEM ? (DVR + 3) & ~3 : DVR;  // floats per partial row
    constexpr uint32_t kOut = 0x80000000u;  // past any num_records (<= INT_MAX)
    const uint32_t head_bytes = (uint32_t)a.Sk * DR * 2;
    const uint32_t vhead_bytes = (uint32_t)a.Sk * DVR * 2;
    // Bytes between consecutive keys of one K/V head: DR*2 in a dense head,
    // Hkv*DR*2 inside a page (DVR for V).
    const uint32_t row_bytes = PAGED ? (uint32_t)a.Hkv * DR * 2 : (uint32_t)DR * 2;
    const uint32_t vrow_bytes = PAGED ? (uint32_t)a.Hkv * DVR * 2 : (uint32_t)DVR * 2;
    const uint32_t page_bytes = PAGED ? (uint32_t)p.page_size * row_bytes : 0u;
    const uint32_t vpage_bytes = PAGED ? (uint32_t)p.page_size * vrow_bytes : 0u;

    // Lane-constant DMA offsets (bytes from the step's first key) and LDS read
    // offsets (elements from the stage start).
    uint32_t koff[L::DMA], voff[LV::DMA];
    int kvn[ELEM ? L::DMA : 1], vvn[ELEM ? LV::DMA : 1];  // ELEM: elements of the slot inside the row
#pragma unroll
    for (int i = 0; i < L::DMA; ++i) {
        const int q = 64 * i + lane, row = q / L::CPR, pc = q % L::CPR;
        const int ck = pc ^ L::fk(row);  // logical chunk
        koff[i] = 8 * ck < DR ? row * row_bytes + ck * 16 : kOut;
        if constexpr (ELEM) kvn[i] = min(8, max(0, DR - 8 * ck));
    }
#pragma unroll
    for (int i = 0; i < LV::DMA; ++i) {
        const int q = 64 * i + lane, row = q / LV::CPR, pc = q % LV::CPR;
        const int cv = pc ^ LV::fv(row);  // logical chunk
        voff[i] = 8 * cv < DVR ? row * vrow_bytes + cv * 16 : kOut;
        if constexpr (ELEM) vvn[i] = min(8, max(0, DVR - 8 * cv));
    }
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
    // K fragment of kstep t: key row col, dims (D/4)*grp + 8t .. +7 (contraction
    // slot (t, grp, e) <-> dim (D/4)*grp + 8t + e, matching qb below).
    int krd[L::KSTEPS];
#pragma unroll
    for (int t = 0; t < L::KSTEPS; ++t)
        krd[t] = col * D + ((((D / 32) * grp + t) ^ L::fk(col)) * 8);
    // Transposed V read: lane j of group grp points at row 4*grp + j/4, dims
    // 16*dt + 4*(j%4); it receives V[4*grp .. 4*grp+3][16*dt + col].
    const int tr_row = 4 * grp + (col >> 2);
    int vrd[DV / 16];
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) {
        const int e = 16 * dt + 4 * (col & 3);
        vrd[dt] = L::TILE + tr_row * DV + (((e >> 3) ^ LV::fv(tr_row)) * 8) + (e & 7);
    }

    uint16_t* ring = smem + wave * NS * STAGE;

    // Issue cursor: the next step to load, running NS-1 steps ahead of compute
    // across item boundaries.  Empty items (no visible key) are skipped.
    int i_it = it0, i_st = 0, i_nst = 0, i_k0 = 0, i_seq = 0, i_gk = 0, i_page = -1;
    __amdgpu_buffer_rsrc_t ikrs = make_rsrc(a.k, 0), ivrs = make_rsrc(a.v, 0);
    // Bit (n % 32): step n's keys come from a valid page (paged; at most NS-1
    // steps are ahead of compute, so 32 bits never wrap onto a live step).
    uint32_t valid_bits = 0xffffffffu;
    auto seek = [&](int from) {
        for (i_it = from; i_it < it1; i_it += kDecWaves) {
            const Item g = item_geo<PAGED>(a, p, meta, i_it, G, nqc, chunk);
            if (g.nst > 0) {
                i_st = 0;
                i_nst = g.nst;
                i_k0 = g.lo;
                i_seq = g.seq;
                i_gk = g.gk;
                i_page = -1;
                if (!PAGED) {
                    const int64_t kvh = ((int64_t)g.b * a.Hkv + g.gk) * a.Sk;
                    ikrs = make_rsrc(static_cast<const uint16_t*>(a.k) + kvh * DR, head_bytes);
                    ivrs = make_rsrc(static_cast<const uint16_t*>(a.v) + kvh * DVR, vhead_bytes);
                }
                return;
            }
        }
    };
    int issued = 0;
    auto issue_next = [&]() {
        uint16_t* st = ring + (issued % NS) * STAGE;
        uint32_t base, vbase;
        if (PAGED) {
            const int lp = i_k0 / p.page_size;
            if (lp != i_page) {  // entering a new page: look it up
                i_page = lp;
                const int pg = lp < p.max_pages ? meta.tables[(int64_t)i_seq * p.max_pages + lp] : -1;
                const bool ok = pg >= 0 && pg < p.pages;
                const int64_t off = ok ? (int64_t)pg * p.page_size * a.Hkv : 0;
                ikrs = make_rsrc(static_cast<const uint16_t*>(a.k) + off * DR, ok ? page_bytes : 0u);
                ivrs = make_rsrc(static_cast<const uint16_t*>(a.v) + off * DVR, ok ? vpage_bytes : 0u);
                valid_bits = ok ? (valid_bits | (1u << (issued & 31))) : (valid_bits & ~(1u << (issued & 31)));
            } else {
                // same page as the previous step: same validity
                const uint32_t prev = (valid_bits >> ((issued - 1) & 31)) & 1u;
                valid_bits = (valid_bits & ~(1u << (issued & 31))) | (prev << (issued & 31));
            }
            base = ((uint32_t)(i_k0 % p.page_size) * a.Hkv + i_gk) * DR * 2;
            vbase = ((uint32_t)(i_k0 % p.page_size) * a.Hkv + i_gk) * DVR * 2;
        } else {
            base = (uint32_t)i_k0 * DR * 2;
            vbase = (uint32_t)i_k0 * DVR * 2;
        }
        // The buffer range check covers the per-lane offset but not the scalar
        // one.  Dense: the step offset goes into the per-lane offset, so rows
        // past Sk read zeros.  Paged: a step never leaves its page (and an
        // invalid page has no records at all), so it can ride in the scalar
        // offset.
        const uint32_t kb = PAGED ? 0u : base, ksb = PAGED ? base : 0u;
        const uint32_t vb = PAGED ? 0u : vbase, vsb = PAGED ? vbase : 0u;
        if constexpr (ELEM) {
            // (an out-of-range slot stays out of range: kOut plus a step offset
            // still exceeds every num_records)
#pragma unroll
            for (int i = 0; i < L::DMA; ++i)
                lds_store(reinterpret_cast<u32x4*>(st + 512 * i) + lane, elem_slot(ikrs, koff[i] + kb, kvn[i], ksb));
#pragma unroll
            for (int i = 0; i < LV::DMA; ++i)
                lds_store(reinterpret_cast<u32x4*>(st + L::TILE + 512 * i) + lane,
                          elem_slot(ivrs, voff[i] + vb, vvn[i], vsb));
        } else {
#pragma unroll
            for (int i = 0; i < L::DMA; ++i) dma16(ikrs, st + 512 * i, koff[i] + kb, ksb);
#pragma unroll
            for (int i = 0; i < LV::DMA; ++i) dma16(ivrs, st + L::TILE + 512 * i, voff[i] + vb, vsb);
        }
        ++issued;
        if (++i_st < i_nst)
            i_k0 += kStep;
        else
            seek(i_it + kDecWaves);
    };
    seek(it0);
    for (int j = 0; j < NS - 1 && i_it < it1; ++j) issue_next();

    float* const park = reinterpret_cast<float*>(smem + kDecWaves * NS * STAGE) + wave * KPARK * PSLOT;
    int nparked = 0;
    int pnh[KPARK];         // query heads of each parked item
    int64_t prw[KPARK];     // its first partial row
    // Write out the parked partials: each lane its own values, as parked.
    auto flush = [&]() {
#pragma unroll
        for (int k = 0; k < KPARK; ++k) {
            if (k >= nparked) break;
            const int nh = pnh[k];
            const int64_t pr = prw[k];
            if (col < nh) {
                const float* sl = park + k * PSLOT;
                const int64_t prow = pr + (int64_t)col * a.splits;
                float* op = a.o_part + prow * DVP + 4 * grp;
#pragma unroll
                for (int dt = 0; dt < DV / 16; ++dt)
                    __builtin_nontemporal_store(lds_load_f32x4(sl + col * DV + 16 * dt + 4 * grp),
                                                reinterpret_cast<f32x4*>(op + 16 * dt));
                if (grp == 0) __builtin_nontemporal_store(lds_load(sl + 4 * DV + col), a.lse_part + prow);
            }
        }
        nparked = 0;
    };

    u32x4 qb[L::KSTEPS];
    int q_head = -1;
    int done = 0;  // steps computed
    for (int it = it0; it < it1; it += kDecWaves) {
        const Item g = item_geo<PAGED>(a, p, meta, it, G, nqc, chunk);
        const int64_t prow0 = ((int64_t)g.b * a.Hq + g.h0) * a.splits + g.split;
        if (g.nst == 0) {  // no visible key in this split
            if (col < g.nh) {
                float* op = a.o_part + (prow0 + (int64_t)col * a.splits) * DVP + 4 * grp;
#pragma unroll
                for (int dt = 0; dt < DV / 16; ++dt)
                    if (16 * dt + 4 * grp < DVR)
                        __builtin_nontemporal_store(f32x4{0.f, 0.f, 0.f, 0.f}, reinterpret_cast<f32x4*>(op + 16 * dt));
                if (grp == 0) __builtin_nontemporal_store(-INFINITY, a.lse_part + prow0 + (int64_t)col * a.splits);
            }
            continue;
        }
        const int head = g.b * a.Hq + g.h0;
        if (head != q_head) {
            // Q^T B operand: column col = query head h0 + col (reads beyond the
            // block's nh heads return 0), slots as in krd.
            const __amdgpu_buffer_rsrc_t qrs = make_rsrc(
                static_cast<const uint16_t*>(a.q) + (int64_t)head * DR, (uint32_t)g.nh * DR * 2);
#pragma unroll
            for (int t = 0; t < L::KSTEPS; ++t) {
                const int d0 = (D / 4) * grp + 8 * t;
                if constexpr (ELEM)
                    qb[t] = elem_slot(qrs, d0 < DR ? (col * DR + d0) * 2 : kOut, min(8, max(0, DR - d0)), 0u);
                else
                    qb[t] = __builtin_amdgcn_raw_buffer_load_b128(
                        qrs, d0 < DR ? (col * DR + d0) * 2 : kOut, 0, 0);
            }
            // Take the wait for the Q loads here, once per head, not inside the
            // step loop.
#pragma unroll
            for (int t = 0; t < L::KSTEPS; ++t) asm volatile("" ::"v"(qb[t]));
            q_head = head;
        }

        f32x4 oacc[DV / 16];
#pragma unroll
        for (int dt = 0; dt < DV / 16; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        float m_run = -INFINITY, l_run = 0.f;

        for (int st = 0; st < g.nst; ++st, ++done) {
            if (i_it < it1) issue_next();
            // Every load but those of the steps issued after this one has landed.
            const int ahead = issued - done - 1;
            if (NS == 8 && ahead >= 7)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(7 * OPS) : "memory");
            else if (NS == 8 && ahead == 6)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(6 * OPS) : "memory");
            else if (NS == 8 && ahead == 5)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(5 * OPS) : "memory");
            else if (NS == 8 && ahead == 4)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * OPS) : "memory");
            else if (NS >= 4 && ahead >= 3)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * OPS) : "memory");
            else if (ahead >= 2)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * OPS) : "memory");
            else if (ahead == 1)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(OPS) : "memory");
            else
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

            const uint16_t* stg = ring + (done % NS) * STAGE;
            f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < L::KSTEPS; ++t)
                s = mfma_16x16x32<T>(lds_read128(stg + krd[t]), qb[t], s);
            const int k0 = g.lo + kStep * st;
            if (k0 + kStep > g.hi) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (k0 + 4 * grp + i >= g.hi) s[i] = -INFINITY;
            }
            if (PAGED && !((valid_bits >> (done & 31)) & 1u)) s = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            // Weights against the current reference max.  They are >= 0, so a
            // lane sum <= 2^8 bounds each by 2^8, the lazy-rescale bound; only
            // otherwise (or before the first max) take the tile max and maybe
            // move the reference.
            uint32_t p01, p23;
            auto weights = [&]() -> float {
                const float neg = -((m_run == -INFINITY) ? 0.f : m_run) * c;
                p01 = pack2<T>(fast_exp2(fmaf(s[0], c, neg)), fast_exp2(fmaf(s[1], c, neg)));
                p23 = pack2<T>(fast_exp2(fmaf(s[2], c, neg)), fast_exp2(fmaf(s[3], c, neg)));
                return sum2<T>(p23, sum2<T>(p01, 0.f));
            };
            float ps = weights();
            if (__any(ps > 256.f || m_run == -INFINITY)) {
                float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
                mx = fmaxf(mx, __shfl_xor(mx, 16));
                mx = max_half_waves(mx);  // all four lanes of a column agree
                if (__any(mx > m_run + tau)) {
                    const float m_new = fmaxf(m_run, mx);
                    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
                    const float alpha = fast_exp2((m_run - m_use) * c);
                    m_run = m_new;
                    l_run *= alpha;
#pragma unroll
                    for (int dt = 0; dt < DV / 16; ++dt) oacc[dt] *= alpha;
                }
                ps = weights();
            }
            l_run += ps;
            const u32x2 pb = u32x2{p01, p23};
            u32x2 vf[DV / 16];
#pragma unroll
            for (int dt = 0; dt < DV / 16; ++dt) vf[dt] = lds_read_tr(stg + vrd[dt]);
#pragma unroll
            for (int dt = 0; dt < DV / 16; ++dt)
                oacc[dt] = mfma_16x16x16<T>(vf[dt], pb, oacc[dt]);
        }

        // Column totals: the denominator is spread over the 4 lane groups.
        l_run += __shfl_xor(l_run, 16);
        l_run += __shfl_xor(l_run, 32);
        // The partial and its lse go out with non-temporal stores (read once,
        // by the merge pass).  vmcnt retires in issue order, so the ring
        // loads issued after an item's stores wait for the stores too; with
        // the default policy that cost the 128-wide decode 6% of its time.
        if (kPark && g.nh <= 4) {
            float* sl = park + nparked * PSLOT;
            if (col < g.nh) {
                const bool none = m_run == -INFINITY;  // every key masked (paged: invalid pages only)
#pragma unroll
                for (int dt = 0; dt < DV / 16; ++dt)
                    lds_store_f32x4(sl + col * DV + 16 * dt + 4 * grp,
                                    none ? f32x4{0.f, 0.f, 0.f, 0.f}
                                         : f32x4{oacc[dt][0] / l_run, oacc[dt][1] / l_run, oacc[dt][2] / l_run,
                                                 oacc[dt][3] / l_run});
                if (grp == 0) lds_store(sl + 4 * DV + col, none ? -INFINITY : m_run * a.scale + __logf(l_run));
            }
#pragma unroll
            for (int k = 0; k < KPARK; ++k)  // constant indices: the slots stay in registers
                if (k == nparked) {
                    prw[k] = prow0;
                    pnh[k] = g.nh;
                }
            if (++nparked == KPARK) flush();
        } else if (col < g.nh) {
            const int64_t prow = prow0 + (int64_t)col * a.splits;
            float* op = a.o_part + prow * DVP + 4 * grp;
            if (m_run == -INFINITY) {  // every key masked (paged: invalid pages only)
#pragma unroll
                for (int dt = 0; dt < DV / 16; ++dt)
                    if (16 * dt + 4 * grp < DVR)
                        __builtin_nontemporal_store(f32x4{0.f, 0.f, 0.f, 0.f}, reinterpret_cast<f32x4*>(op + 16 * dt));
                if (grp == 0) __builtin_nontemporal_store(-INFINITY, a.lse_part + prow);
            } else {
#pragma unroll
                for (int dt = 0; dt < DV / 16; ++dt)  // O^T register i of tile dt: dim 16*dt + 4*grp + i
                    if (16 * dt + 4 * grp < DVR)
                        __builtin_nontemporal_store(
                            f32x4{oacc[dt][0] / l_run, oacc[dt][1] / l_run, oacc[dt][2] / l_run,
                                  oacc[dt][3] / l_run},
                            reinterpret_cast<f32x4*>(op + 16 * dt));
                if (grp == 0) __builtin_nontemporal_store(m_run * a.scale + __logf(l_run), a.lse_part + prow);
            }
        }
    }
    if (kPark && nparked > 0) flush();
}

template <int D, class T, bool GEN = false, bool ELEM = false>
__global__ __launch_bounds__(256) void decode_merge_bf16_kernel(DecodeArgs a) {
    constexpr int TPR = D / 4;       // threads per row, 4 dims each
    constexpr int RPB = 256 / TPR;   // rows (batch, query head) per block
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
    const int d4 = threadIdx.x % TPR;
    const int DR = GEN ? a.Dv : D;  // value head dim in memory (<= D; a multiple of 8 unless ELEM)
    const int DP = ELEM ? (DR + 3) & ~3 : DR;  // floats per partial row
    if (row >= (int64_t)a.B * a.Hq || 4 * d4 >= DR) return;
    const float* lse = a.lse_part + row * a.splits;
    const f32x4* op = reinterpret_cast<const f32x4*>(a.o_part + row * a.splits * DP) + d4;
    float M = -INFINITY;
    for (int s = 0; s < a.splits; ++s) M = fmaxf(M, lse[s]);
    float den = 0.f;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int s = 0; s < a.splits; ++s) {
        const float w = fast_exp2((lse[s] - M) * kLog2e);  // empty split: exp(-inf) = 0
        den += w;
        const f32x4 o = op[(int64_t)s * (DP / 4)];
        acc[0] = fmaf(w, o[0], acc[0]);
        acc[1] = fmaf(w, o[1], acc[1]);
        acc[2] = fmaf(w, o[2], acc[2]);
        acc[3] = fmaf(w, o[3], acc[3]);
    }
    // Every split empty (no visible key): M = -inf, w = NaN, and the row is NaN.
    uint16_t* orow = static_cast<uint16_t*>(a.out) + row * DR + 4 * d4;
    if constexpr (ELEM) {  // element by element: the row need not be 8-byte aligned
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (4 * d4 + e < DR) orow[e] = (uint16_t)to16<T>(acc[e] / den);
    } else {
        const uint32_t lo = pack_lo16(to16<T>(acc[0] / den), to16<T>(acc[1] / den));
        const uint32_t hi = pack_lo16(to16<T>(acc[2] / den), to16<T>(acc[3] / den));
        *reinterpret_cast<u32x2*>(orow) = u32x2{lo, hi};
    }
}

// fp32 inputs (the ruDNN user guide's F32 Q/K/V, section 9): the same items,
// persistent grid, per-wave DMA ring and page lookup as the 16-bit split
// pass, with fp32 MFMAs (v_mfma_f32_16x16x4_f32) and no rounding of the
// weights.  Per 16-key step of an item, in one wave:
//   S^T[16 keys x 16 queries] = K Q^T   D/4 MFMAs; lane group g (lanes
//     16g .. 16g+15) contracts dims (D/4) g .. (D/4) g + D/4 - 1, so one
//     16-byte LDS read of K feeds four MFMAs;
//   O^T[D x 16 queries] += V^T P^T      4 x D/16 MFMAs; MFMA i takes key
//     4g + i in contraction slot g, which is exactly the score register i of
//     the lanes of group g: the weights never leave their lanes.
// Row r of the A operand of O^T tile dt is dim 4r + dt%4 + 64 (dt/4), so a
// lane's V^T operands of four tiles are one 16-byte run of its V row.
template <int D>
struct DecGeoF32 {
    static constexpr int CPR = D / 4;                    // 16-byte chunks per row
    static constexpr int TILE = kStep * D;               // floats of one K or V step
    static constexpr int STAGE = 2 * TILE;               // K tile, then V tile
    static constexpr int NS = kRingBytes / (4 * STAGE);  // ring stages per wave
    static constexpr int DMA = TILE * 4 / 1024;          // 1-KB DMA loads per tile
    static constexpr int OPS = 2 * DMA;                  // vector memory ops per step
    static constexpr int CG = CPR / 4;                   // K chunks per lane group
    // K chunk swizzle: the 16 rows a lane group reads at one logical chunk
    // fall on 16 distinct 16-byte bank groups.
    __device__ static int fk(int r) { return r % 16; }
};
static_assert(DecGeoF32<128>::NS == 2 && DecGeoF32<64>::NS == 4, "fp32 ring depth");

template <int D, bool PAGED, bool GEN = false>
__global__ __launch_bounds__(kDecThreads, 1) void decode_split_f32_kernel(
    DecodeArgs a, PagedArgs p, const int32_t* __restrict__ key_lens,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ query_seq, const int32_t* __restrict__ query_pos, int items) {
    using L = DecGeoF32<D>;
    constexpr int DT = D / 16;  // O^T tiles
    const Meta meta{key_lens, tables, seq_lens, query_seq, query_pos};
    __shared__ __attribute__((aligned(1024))) float smem[kDecWaves * L::NS * L::STAGE];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int col = lane & 15;  // query column (and key row of the S^T tile)
    const int grp = lane >> 4;  // lane group

    const int wg0 = (int)((int64_t)blockIdx.x * items / gridDim.x);
    const int it1 = (int)((int64_t)(blockIdx.x + 1) * items / gridDim.x);
    const int it0 = wg0 + wave;
    if (it0 >= it1) return;

    const int G = a.Hq / a.Hkv;
    const int nqc = (G + kQ - 1) / kQ;
    int chunk = (a.Sk + a.splits - 1) / a.splits;
    if (PAGED) chunk = (chunk + kStep - 1) / kStep * kStep;
    const float c = a.scale * kLog2e;
    const float tau = kTau / c;
    // Head dim in memory: DR floats (GEN: a multiple of 4 below D; else D).
    const int DR = GEN ? a.D : D;
    constexpr uint32_t kOut = 0x80000000u;
    const uint32_t head_bytes = (uint32_t)a.Sk * DR * 4;
    const uint32_t row_bytes = PAGED ? (uint32_t)a.Hkv * DR * 4 : (uint32_t)DR * 4;
    const uint32_t page_bytes = PAGED ? (uint32_t)p.page_size * row_bytes : 0u;

    // DMA slot s = 64 i + lane of a tile holds row s / CPR, physical chunk
    // s % CPR; K's logical chunk is swizzled, V's is not.
    uint32_t koff[L::DMA], voff[L::DMA];
#pragma unroll
    for (int i = 0; i < L::DMA; ++i) {
        const int q = 64 * i + lane, row = q / L::CPR, pc = q % L::CPR;
        const int ck = pc ^ L::fk(row);
        koff[i] = 4 * ck < DR ? row * row_bytes + ck * 16 : kOut;
        voff[i] = 4 * pc < DR ? row * row_bytes + pc * 16 : kOut;
    }

    float* ring = smem + wave * L::NS * L::STAGE;

    int i_it = it0, i_st = 0, i_nst = 0, i_k0 = 0, i_seq = 0, i_gk = 0, i_page = -1;
    __amdgpu_buffer_rsrc_t ikrs = make_rsrc(a.k, 0), ivrs = make_rsrc(a.v, 0);
    uint32_t valid_bits = 0xffffffffu;
    auto seek = [&](int from) {
        for (i_it = from; i_it < it1; i_it += kDecWaves) {
            const Item g = item_geo<PAGED>(a, p, meta, i_it, G, nqc, chunk);
            if (g.nst > 0) {
                i_st = 0;
                i_nst = g.nst;
                i_k0 = g.lo;
                i_seq = g.seq;
                i_gk = g.gk;
                i_page = -1;
                if (!PAGED) {
                    const int64_t kvh = ((int64_t)g.b * a.Hkv + g.gk) * a.Sk * DR;
                    ikrs = make_rsrc(static_cast<const float*>(a.k) + kvh, head_bytes);
                    ivrs = make_rsrc(static_cast<const float*>(a.v) + kvh, head_bytes);
                }
                return;
            }
        }
    };
    int issued = 0;
    auto issue_next = [&]() {
        uint16_t* st = reinterpret_cast<uint16_t*>(ring + (issued % L::NS) * L::STAGE);
        uint32_t base;
        if (PAGED) {
            const int lp = i_k0 / p.page_size;
            if (lp != i_page) {
                i_page = lp;
                const int pg = lp < p.max_pages ? meta.tables[(int64_t)i_seq * p.max_pages + lp] : -1;
                const bool ok = pg >= 0 && pg < p.pages;
                const int64_t off = ok ? (int64_t)pg * p.page_size * a.Hkv * DR : 0;
                ikrs = make_rsrc(static_cast<const float*>(a.k) + off, ok ? page_bytes : 0u);
                ivrs = make_rsrc(static_cast<const float*>(a.v) + off, ok ? page_bytes : 0u);
                valid_bits = ok ? (valid_bits | (1u << (issued & 31))) : (valid_bits & ~(1u << (issued & 31)));
            } else {
                const uint32_t prev = (valid_bits >> ((issued - 1) & 31)) & 1u;
                valid_bits = (valid_bits & ~(1u << (issued & 31))) | (prev << (issued & 31));
            }
            base = ((uint32_t)(i_k0 % p.page_size) * a.Hkv + i_gk) * DR * 4;
        } else {
            base = (uint32_t)i_k0 * DR * 4;
        }
        const uint32_t vb = PAGED ? 0u : base, sb = PAGED ? base : 0u;
#pragma unroll
        for (int i = 0; i < L::DMA; ++i) dma16(ikrs, st + 512 * i, koff[i] + vb, sb);
#pragma unroll
        for (int i = 0; i < L::DMA; ++i) dma16(ivrs, st + 2 * L::TILE + 512 * i, voff[i] + vb, sb);
        ++issued;
        if (++i_st < i_nst)
            i_k0 += kStep;
        else
            seek(i_it + kDecWaves);
    };
    seek(it0);
    for (int j = 0; j < L::NS - 1 && i_it < it1; ++j) issue_next();

    // K operand reads: row col, logical chunk CG*grp + u (dims (D/4) grp + 4u ..).
    int krd[L::CG];
#pragma unroll
    for (int u = 0; u < L::CG; ++u) krd[u] = col * D + (((L::CG * grp + u) ^ L::fk(col)) * 4);

    f32x4 qf[L::CG];
    int q_head = -1;
    int done = 0;
    for (int it = it0; it < it1; it += kDecWaves) {
        const Item g = item_geo<PAGED>(a, p, meta, it, G, nqc, chunk);
        const int64_t prow0 = ((int64_t)g.b * a.Hq + g.h0) * a.splits + g.split;
        if (g.nst == 0) {
            if (col < g.nh) {
                float* op = a.o_part + (prow0 + (int64_t)col * a.splits) * DR;
#pragma unroll
                for (int dh = 0; dh < D / 64; ++dh)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int d0 = 16 * grp + 4 * j + 64 * dh;
                        if (d0 < DR)
                            __builtin_nontemporal_store(f32x4{0.f, 0.f, 0.f, 0.f}, reinterpret_cast<f32x4*>(op + d0));
                    }
                if (grp == 0) __builtin_nontemporal_store(-INFINITY, a.lse_part + prow0 + (int64_t)col * a.splits);
            }
            continue;
        }
        const int head = g.b * a.Hq + g.h0;
        if (head != q_head) {
            const __amdgpu_buffer_rsrc_t qrs = make_rsrc(
                static_cast<const float*>(a.q) + (int64_t)head * DR, (uint32_t)g.nh * DR * 4);
#pragma unroll
            for (int u = 0; u < L::CG; ++u) {
                const int d0 = (D / 4) * grp + 4 * u;
                qf[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      qrs, d0 < DR ? (col * DR + d0) * 4 : kOut, 0, 0));
            }
#pragma unroll
            for (int u = 0; u < L::CG; ++u) asm volatile("" ::"v"(qf[u]));
            q_head = head;
        }

        f32x4 oacc[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        float m_run = -INFINITY, l_run = 0.f;

        for (int st = 0; st < g.nst; ++st, ++done) {
            if (i_it < it1) issue_next();
            const int ahead = issued - done - 1;
            if (L::NS == 4 && ahead >= 3)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * L::OPS) : "memory");
            else if (L::NS == 4 && ahead == 2)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * L::OPS) : "memory");
            else if (ahead >= 1)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(L::OPS) : "memory");
            else
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

            const float* stg = ring + (done % L::NS) * L::STAGE;
            f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < L::CG; ++u) {
                const f32x4 kv = __builtin_bit_cast(
                    f32x4, lds_read128(reinterpret_cast<const uint16_t*>(stg + krd[u])));
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    s = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[e], qf[u][e], s, 0, 0, 0);
            }
            const int k0 = g.lo + kStep * st;
            if (k0 + kStep > g.hi) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (k0 + 4 * grp + i >= g.hi) s[i] = -INFINITY;
            }
            if (PAGED && !((valid_bits >> (done & 31)) & 1u)) s = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            f32x4 pw;
            auto weights = [&]() -> float {
                const float neg = -((m_run == -INFINITY) ? 0.f : m_run) * c;
#pragma unroll
                for (int i = 0; i < 4; ++i) pw[i] = fast_exp2(fmaf(s[i], c, neg));
                return (pw[0] + pw[1]) + (pw[2] + pw[3]);
            };
            float ps = weights();
            if (__any(ps > 256.f || m_run == -INFINITY)) {
                float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
                mx = fmaxf(mx, __shfl_xor(mx, 16));
                mx = max_half_waves(mx);
                if (__any(mx > m_run + tau)) {
                    const float m_new = fmaxf(m_run, mx);
                    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
                    const float alpha = fast_exp2((m_run - m_use) * c);
                    m_run = m_new;
                    l_run *= alpha;
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
                }
                ps = weights();
            }
            l_run += ps;
            // V row of key 4*grp + i, runs 16h + col (dims 64h + 4col ..).
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float* vrow = stg + L::TILE + (4 * grp + i) * D + 4 * col;
#pragma unroll
                for (int dh = 0; dh < D / 64; ++dh) {
                    const f32x4 vv = __builtin_bit_cast(
                        f32x4, lds_read128(reinterpret_cast<const uint16_t*>(vrow + 64 * dh)));
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        oacc[4 * dh + e] =
                            __builtin_amdgcn_mfma_f32_16x16x4f32(vv[e], pw[i], oacc[4 * dh + e], 0, 0, 0);
                }
            }
        }

        l_run += __shfl_xor(l_run, 16);
        l_run += __shfl_xor(l_run, 32);
        if (col < g.nh) {
            const int64_t prow = prow0 + (int64_t)col * a.splits;
            float* op = a.o_part + prow * DR;
            const bool empty = m_run == -INFINITY;  // every key masked (paged: invalid pages only)
            const float inv = empty ? 0.f : 1.f / l_run;
            // O^T register j of tile 4 dh + e: dim 16 grp + 4 j + e + 64 dh.
#pragma unroll
            for (int dh = 0; dh < D / 64; ++dh)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int d0 = 16 * grp + 4 * j + 64 * dh;
                    if (d0 < DR)
                        __builtin_nontemporal_store(
                            f32x4{oacc[4 * dh][j] * inv, oacc[4 * dh + 1][j] * inv,
                                  oacc[4 * dh + 2][j] * inv, oacc[4 * dh + 3][j] * inv},
                            reinterpret_cast<f32x4*>(op + d0));
                }
            if (grp == 0)
                __builtin_nontemporal_store(empty ? -INFINITY : m_run * a.scale + __logf(l_run), a.lse_part + prow);
        }
    }
}

// Merge of fp32 partials into an fp32 output (4 dims per thread).
template <int D, bool GEN = false>
__global__ __launch_bounds__(256) void decode_merge_f32_kernel(DecodeArgs a) {
    constexpr int TPR = D / 4;
    constexpr int RPB = 256 / TPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
    const int d4 = threadIdx.x % TPR;
    const int DR = GEN ? a.Dv : D;
    if (row >= (int64_t)a.B * a.Hq || 4 * d4 >= DR) return;
    const float* lse = a.lse_part + row * a.splits;
    const f32x4* op = reinterpret_cast<const f32x4*>(a.o_part + row * a.splits * DR) + d4;
    float M = -INFINITY;
    for (int s = 0; s < a.splits; ++s) M = fmaxf(M, lse[s]);
    float den = 0.f;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < a.splits; ++s) {
        const float w = fast_exp2((lse[s] - M) * kLog2e);
        den += w;
        const f32x4 o = op[(int64_t)s * (DR / 4)];
        acc[0] = fmaf(w, o[0], acc[0]);
        acc[1] = fmaf(w, o[1], acc[1]);
        acc[2] = fmaf(w, o[2], acc[2]);
        acc[3] = fmaf(w, o[3], acc[3]);
    }
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + row * DR + 4 * d4) =
        f32x4{acc[0] / den, acc[1] / den, acc[2] / den, acc[3] / den};
}

// Compute units of the current device (cached per device).
hipError_t compute_units(int* n) {
    static std::atomic<int> cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64 && (*n = cache[dev].load(std::memory_order_relaxed)) > 0)
        return hipSuccess;
    e = hipDeviceGetAttribute(n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (*n < 1) *n = 1;
    if (dev >= 0 && dev < 64) cache[dev].store(*n, std::memory_order_relaxed);
    return hipSuccess;
}

// Split and merge for a value head dim Dv other than D (both multiples of 8
// up to 256), or (ELEM) head dims that are not multiples of 8 (up to 256):
// general-width kernels on the padded widths DP (K) and VP (V).
template <int DP, int VP, bool PAGED, class T, bool ELEM>
void launch_dv(const DecodeArgs& a, const PagedArgs& p, int wgs, int items, hipStream_t s) {
    const dim3 mgrid((unsigned)(((int64_t)a.B * a.Hq * VP / 4 + 255) / 256));
    hipLaunchKernelGGL((decode_split_bf16_kernel<DP, PAGED, T, true, VP, ELEM>), dim3(wgs), dim3(kDecThreads),
                       0, s, a, p, a.key_lens, p.block_tables, p.seq_lens, p.query_seq, p.query_pos, items);
    hipLaunchKernelGGL((decode_merge_bf16_kernel<VP, T, true, ELEM>), mgrid, dim3(256), 0, s, a);
}

template <int DP, bool PAGED, class T, bool ELEM = false>
void launch_dv_v(const DecodeArgs& a, const PagedArgs& p, int wgs, int items, hipStream_t s) {
    if (a.Dv <= 64)
        launch_dv<DP, 64, PAGED, T, ELEM>(a, p, wgs, items, s);
    else if (a.Dv <= 128)
        launch_dv<DP, 128, PAGED, T, ELEM>(a, p, wgs, items, s);
    else
        launch_dv<DP, 256, PAGED, T, ELEM>(a, p, wgs, items, s);
}

template <bool PAGED, class T>
hipError_t launch_split_and_merge(const DecodeArgs& a, const PagedArgs& p, hipStream_t s) {
    const int items = (int)decode_work_items(a.B, a.Hq, a.Hkv, a.splits);
    int cus = 0;
    const hipError_t e = compute_units(&cus);
    if (e != hipSuccess) return e;
    // One workgroup per compute unit (the LDS rings admit no second one), or
    // fewer when there are fewer items.
    const int wgs = std::min(cus, (items + kDecWaves - 1) / kDecWaves);
    if (a.D > 256 || a.Dv > 256) {
        // Wider heads (key or value): the head-dim-split kernel writes the
        // same partials (Dv wide), then the same merge (Dv/4 threads per row).
        if (a.D > 1024 || a.Dv > 1024 || a.D < 1 || a.Dv < 1 || (!PAGED && a.Dv != a.D))
            return hipErrorInvalidValue;
        const hipError_t ew = launch_decode_wide_split(a, PAGED ? &p : nullptr, T::kF16, s);
        if (ew != hipSuccess) return ew;
        const int dw = a.Dv <= 512 ? 512 : 1024;
        const bool elem = a.D % 8 != 0 || a.Dv % 8 != 0;  // partial rows padded to a multiple of 4 floats
        const dim3 mg((unsigned)(((int64_t)a.B * a.Hq * dw / 4 + 255) / 256));
        if (elem && dw == 512)
            hipLaunchKernelGGL((decode_merge_bf16_kernel<512, T, true, true>), mg, dim3(256), 0, s, a);
        else if (elem)
            hipLaunchKernelGGL((decode_merge_bf16_kernel<1024, T, true, true>), mg, dim3(256), 0, s, a);
        else if (a.Dv == 512)
            hipLaunchKernelGGL((decode_merge_bf16_kernel<512, T>), mg, dim3(256), 0, s, a);
        else if (a.Dv == 1024)
            hipLaunchKernelGGL((decode_merge_bf16_kernel<1024, T>), mg, dim3(256), 0, s, a);
        else if (dw == 512)
            hipLaunchKernelGGL((decode_merge_bf16_kernel<512, T, true>), mg, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((decode_merge_bf16_kernel<1024, T, true>), mg, dim3(256), 0, s, a);
        return hipGetLastError();
    }
    if ((a.D % 8 != 0 || a.Dv % 8 != 0) && a.D <= 256) {
        if (a.D < 1 || a.Dv < 1 || a.Dv > 256) return hipErrorInvalidValue;
        if constexpr (PAGED) {
            if (a.D <= 64)
                launch_dv_v<64, PAGED, T, true>(a, p, wgs, items, s);
            else if (a.D <= 128)
                launch_dv_v<128, PAGED, T, true>(a, p, wgs, items, s);
            else
                launch_dv_v<256, PAGED, T, true>(a, p, wgs, items, s);
        } else {  // the dense decode has Dv = D
            if (a.Dv != a.D) return hipErrorInvalidValue;
            if (a.D <= 64)
                launch_dv<64, 64, PAGED, T, true>(a, p, wgs, items, s);
            else if (a.D <= 128)
                launch_dv<128, 128, PAGED, T, true>(a, p, wgs, items, s);
            else
                launch_dv<256, 256, PAGED, T, true>(a, p, wgs, items, s);
        }
        return hipGetLastError();
    }
    if (a.Dv != a.D) {
        if constexpr (PAGED) {
            if (a.D % 8 != 0 || a.Dv % 8 != 0 || a.D < 8 || a.Dv < 8 || a.D > 256 || a.Dv > 256)
                return hipErrorInvalidValue;
            if (a.D <= 64)
                launch_dv_v<64, PAGED, T>(a, p, wgs, items, s);
            else if (a.D <= 128)
                launch_dv_v<128, PAGED, T>(a, p, wgs, items, s);
            else
                launch_dv_v<256, PAGED, T>(a, p, wgs, items, s);
            return hipGetLastError();
        }
        return hipErrorInvalidValue;  // the dense decode has Dv = D
    }
    if (a.D % 8 != 0 || a.D < 8 || a.D > 256) return hipErrorInvalidValue;
    // Head dims that are multiples of 8 run on the 64-, 128- or 256-wide
    // kernels (the 256-wide ring holds two steps per wave: one step ahead).
    const int dpad = a.D <= 64 ? 64 : (a.D <= 128 ? 128 : 256);
    const dim3 mgrid((unsigned)(((int64_t)a.B * a.Hq * dpad / 4 + 255) / 256));
    const dim3 sg(wgs), st(kDecThreads), mt(256);
    const int32_t *kl = a.key_lens, *bt = p.block_tables, *sl = p.seq_lens, *qs = p.query_seq,
                  *qp = p.query_pos;
    if (a.D == 64) {
        hipLaunchKernelGGL((decode_split_bf16_kernel<64, PAGED, T>), sg, st, 0, s, a, p, kl, bt, sl, qs,
                           qp, items);
        hipLaunchKernelGGL((decode_merge_bf16_kernel<64, T>), mgrid, mt, 0, s, a);
    } else if (a.D == 128) {
        hipLaunchKernelGGL((decode_split_bf16_kernel<128, PAGED, T>), sg, st, 0, s, a, p, kl, bt, sl, qs,
                           qp, items);
        hipLaunchKernelGGL((decode_merge_bf16_kernel<128, T>), mgrid, mt, 0, s, a);
    } else if (a.D == 256) {
        hipLaunchKernelGGL((decode_split_bf16_kernel<256, PAGED, T>), sg, st, 0, s, a, p, kl, bt, sl, qs,
                           qp, items);
        hipLaunchKernelGGL((decode_merge_bf16_kernel<256, T>), mgrid, mt, 0, s, a);
    } else if (dpad == 64) {
        hipLaunchKernelGGL((decode_split_bf16_kernel<64, PAGED, T, true>), sg, st, 0, s, a, p, kl, bt, sl,
                           qs, qp, items);
        hipLaunchKernelGGL((decode_merge_bf16_kernel<64, T, true>), mgrid, mt, 0, s, a);
    } else if (dpad == 256) {
        hipLaunchKernelGGL((decode_split_bf16_kernel<256, PAGED, T, true>), sg, st, 0, s, a, p, kl, bt,
                           sl, qs, qp, items);
        hipLaunchKernelGGL((decode_merge_bf16_kernel<256, T, true>), mgrid, mt, 0, s, a);
    } else {
        hipLaunchKernelGGL((decode_split_bf16_kernel<128, PAGED, T, true>), sg, st, 0, s, a, p, kl, bt,
                           sl, qs, qp, items);
        hipLaunchKernelGGL((decode_merge_bf16_kernel<128, T, true>), mgrid, mt, 0, s, a);
    }
    return hipGetLastError();
}

template <bool PAGED>
hipError_t launch_split_and_merge_f32(const DecodeArgs& a, const PagedArgs& p, hipStream_t s) {
    if (a.D % 4 != 0 || a.D < 4 || a.D > 128 || a.Dv != a.D) return hipErrorInvalidValue;
    const int items = (int)decode_work_items(a.B, a.Hq, a.Hkv, a.splits);
    int cus = 0;
    const hipError_t e = compute_units(&cus);
    if (e != hipSuccess) return e;
    const int wgs = std::min(cus, (items + kDecWaves - 1) / kDecWaves);
    const dim3 sg(wgs), st(kDecThreads), mt(256);
    const int dpad = a.D <= 64 ? 64 : 128;
    const dim3 mgrid((unsigned)(((int64_t)a.B * a.Hq * dpad / 4 + 255) / 256));
    const int32_t *kl = a.key_lens, *bt = p.block_tables, *sl = p.seq_lens, *qs = p.query_seq,
                  *qp = p.query_pos;
    if (a.D == 64) {
        hipLaunchKernelGGL((decode_split_f32_kernel<64, PAGED>), sg, st, 0, s, a, p, kl, bt, sl, qs, qp, items);
        hipLaunchKernelGGL((decode_merge_f32_kernel<64>), mgrid, mt, 0, s, a);
    } else if (a.D == 128) {
        hipLaunchKernelGGL((decode_split_f32_kernel<128, PAGED>), sg, st, 0, s, a, p, kl, bt, sl, qs, qp, items);
        hipLaunchKernelGGL((decode_merge_f32_kernel<128>), mgrid, mt, 0, s, a);
    } else if (dpad == 64) {
        hipLaunchKernelGGL((decode_split_f32_kernel<64, PAGED, true>), sg, st, 0, s, a, p, kl, bt, sl, qs, qp,
                           items);
        hipLaunchKernelGGL((decode_merge_f32_kernel<64, true>), mgrid, mt, 0, s, a);
    } else {
        hipLaunchKernelGGL((decode_split_f32_kernel<128, PAGED, true>), sg, st, 0, s, a, p, kl, bt, sl, qs, qp,
                           items);
        hipLaunchKernelGGL((decode_merge_f32_kernel<128, true>), mgrid, mt, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace

int64_t decode_work_items(int64_t B, int64_t Hq, int64_t Hkv, int splits) {
    const int64_t G = Hq / Hkv;
    return B * Hkv * ((G + kQ - 1) / kQ) * splits;
}

hipError_t launch_decode_16bit(const DecodeArgs& a, bool f16, hipStream_t s) {
    return f16 ? launch_split_and_merge<false, F16T>(a, PagedArgs{}, s)
               : launch_split_and_merge<false, Bf16T>(a, PagedArgs{}, s);
}

hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t s) {
    return launch_split_and_merge_f32<false>(a, PagedArgs{}, s);
}

hipError_t launch_paged_f32(const DecodeArgs& a, const PagedArgs& p, hipStream_t s) {
    return launch_split_and_merge_f32<true>(a, p, s);
}

hipError_t launch_paged_16bit(const DecodeArgs& a, const PagedArgs& p, bool f16, hipStream_t s) {
    return f16 ? launch_split_and_merge<true, F16T>(a, p, s) : launch_split_and_merge<true, Bf16T>(a, p, s);
}

}  // namespace sdpa
