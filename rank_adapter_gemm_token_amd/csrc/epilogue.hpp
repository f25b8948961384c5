// epilogue.hpp -- device pieces shared by the base-GEMM, shrink and expand
// kernels:
//   * shrink_role: one k part of h = x_tile . A_slot^T for a 16-row bucket
//     tile, the part's k range split over the workgroup's waves and reduced
//     in LDS in a fixed order (consumers add the parts in order: load_h8);
//   * lora_expand_mfma: y_acc += s * h_bucket . B_slot^T on MFMA for the rows
//     of one wave tile, one bucket at a time (rows are sorted by adapter, so a
//     16-row block meets only the few buckets that overlap it);
//   * store_rows: round to the pool dtype and scatter sorted rows back to
//     token order, NaN for invalid tokens.
//
// Accumulator layout (MFMA 16x16x32, wave64): for a 16x16 block, lane l holds
// rows 4*(l/16) + i, i = 0..3, of column l % 16.  Operand fragments: lane l
// holds row (or column) l % 16 and k = 8*(l/16) .. +7 of a 32-wide k step.
#pragma once

#include "dtype.hpp"
#include "internal.hpp"

namespace lora {

constexpr int SEG_NONE = 0;
constexpr int SEG_FUSED = 1;
constexpr int SEG_SEPARATE = 2;

// Sorted row -> token, clamped so that a logic error cannot leave x / y.
__device__ __forceinline__ int token_of(const ApplyArgs &a, int p) {
    return min(max(a.rv.perm[p], 0), a.T - 1);
}

// Partial h = x_tile . A_slot^T over k part `part` (of h_parts) for one
// 16-row tile of an adapter bucket: slot `key` of true rank `rank`, sorted
// rows row0 .. row0 + rows - 1, whose tokens are perm[row0 ..] (perm may
// live in LDS or global memory).  RB rank blocks of 16 are computed: the
// caller picks RB to cover the slot's true rank; h's columns past them (A
// rows that are zero) are stored as exact zeros.  RB also sets how many k
// steps a wave keeps in flight (U).  One workgroup of NWV waves; the part's k steps are split over the
// waves and the waves' sums are added in LDS in a fixed order.  `lds` holds
// >= NWV * RB * 64 16-byte words.  The part is written to h + part * T * R;
// consumers add the parts in order.
// h element store: plain, or (SC1) coherent at agent scope, for parts that
// another workgroup of the same launch adds up.
template <bool SC1>
__device__ __forceinline__ void store_h(float *p, float v) {
    if constexpr (SC1)
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        *p = v;
}

// UO (when > 0) sets U, the k steps a wave keeps in flight, to UO / RB in
// place of the default for RB (the same registers for every RB).
template <int DT, int RB, int NWV, bool SC1 = false, int UO = 0>
__device__ __forceinline__ void shrink_unit(const ApplyArgs &a, int key, int row0, int rows,
                                            const int32_t *perm, int part, u32x4_t *lds) {
    using E = Elem<DT>;
    using V = typename E::vec8;
    key = uniform(key);
    row0 = uniform(row0);
    rows = uniform(rows);
    part = uniform(part);
    const int Rp = a.R;
    const int wave = uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;
    const int kq = lane >> 4;
    const int kst = a.d_in / 32;
    const int split = part * NWV + wave;  // this wave's share of K
    const int nsplit = a.shrink_parts * NWV;
    const int kb = split * kst / nsplit;
    const int ke = (split + 1) * kst / nsplit;

    const bool xv = r < rows;
    const int tok = min(max(perm[row0 + min(r, rows - 1)], 0), a.T - 1);
    const uint16_t *xp = static_cast<const uint16_t *>(a.x) + static_cast<size_t>(tok) * a.d_in + 8 * kq;
    const uint16_t *ap[RB];
    bool av[RB];
#pragma unroll
    for (int cb = 0; cb < RB; ++cb) {
        const int j = cb * 16 + r;
        av[cb] = j < Rp;
        ap[cb] = static_cast<const uint16_t *>(a.A_slab) +
                 (static_cast<size_t>(key) * Rp + (av[cb] ? j : 0)) * a.d_in + 8 * kq;
    }
    f32x4_t acc[RB];
#pragma unroll
    for (int cb = 0; cb < RB; ++cb) acc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    constexpr int U = UO > 0 ? (UO / RB > 0 ? UO / RB : 1) : RB == 1 ? 16 : RB == 2 ? 8 : 4;  // k steps in flight together
    for (int k0 = kb; k0 < ke; k0 += U) {
        V xa[U];
        V b[U][RB];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kk = min(k0 + u, ke - 1);  // clamped: loads stay unconditional
            xa[u] = load8<V>(xp + kk * 32);
#pragma unroll
            for (int cb = 0; cb < RB; ++cb) b[u][cb] = load8<V>(ap[cb] + kk * 32);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const V xm = (k0 + u < ke && xv) ? xa[u] : zero8<V>();
#pragma unroll
            for (int cb = 0; cb < RB; ++cb) acc[cb] = E::mfma(xm, av[cb] ? b[u][cb] : zero8<V>(), acc[cb]);
        }
    }
    // Fixed-order reduction of the waves' partial sums.
    f32x4_t *red = reinterpret_cast<f32x4_t *>(lds);
#pragma unroll
    for (int cb = 0; cb < RB; ++cb) red[(wave * RB + cb) * 64 + lane] = acc[cb];
    __syncthreads();
    if (wave != 0) return;
    float *hout = a.h + static_cast<size_t>(part) * a.T * Rp;
#pragma unroll
    for (int cb = 0; cb < RB; ++cb) {
        f32x4_t s = red[cb * 64 + lane];
        for (int w = 1; w < NWV; ++w) s += red[(w * RB + cb) * 64 + lane];
        const int j = cb * 16 + r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = kq * 4 + i;
            if (row < rows && j < Rp) store_h<SC1>(&hout[static_cast<size_t>(row0 + row) * Rp + j], s[i]);
        }
    }
    for (int j = RB * 16 + r; j < Rp; j += 16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = kq * 4 + i;
            if (row < rows) store_h<SC1>(&hout[static_cast<size_t>(row0 + row) * Rp + j], 0.0f);
        }
    }
}

// shrink_unit for tile `tile` of the routing in global memory.
template <int DT, int RB, int NWV, bool SC1 = false, int UO = 0>
__device__ __forceinline__ void shrink_role(const ApplyArgs &a, int tile, int part, u32x4_t *lds) {
    if (tile >= uniform(*a.rv.n_tiles)) return;
    const int tw = a.rv.tiles[2 * tile];
    const int seg = tile_seg(tw);
    const int row0 = a.rv.tiles[2 * tile + 1];
    const int key = a.rv.segs[4 * seg];
    const int end = a.rv.segs[4 * seg + 1] + a.rv.segs[4 * seg + 2];
    const int rows = min(TILE_ROWS, end - row0);
    // Rank blocks that hold the slot's true rank (the tile carries it).
    const int nrb = uniform(min(RB, (tile_rank(tw) + 15) / 16));
    if (RB >= 4 && nrb == 4) shrink_unit<DT, (RB >= 4 ? 4 : 1), NWV, SC1, UO>(a, key, row0, rows, a.rv.perm, part, lds);
    else if (RB >= 3 && nrb == 3) shrink_unit<DT, (RB >= 3 ? 3 : 1), NWV, SC1, UO>(a, key, row0, rows, a.rv.perm, part, lds);
    else if (RB >= 2 && nrb == 2) shrink_unit<DT, (RB >= 2 ? 2 : 1), NWV, SC1, UO>(a, key, row0, rows, a.rv.perm, part, lds);
    else shrink_unit<DT, 1, NWV, SC1, UO>(a, key, row0, rows, a.rv.perm, part, lds);
}

// h[p][j .. j+7] summed over the shrink's k parts in order (p: the h row,
// a sorted position or a token).  The first HP parts' loads are all in flight
// before the first add; parts beyond HP (if any) are added one at a time.
// COH: h was written by other workgroups of the same launch (agent-coherent
// stores), so it is read with agent-coherent loads, which no stale line of
// this XCD's L2 can serve.
template <int HP, bool COH = false>
__device__ __forceinline__ void load_h8(const ApplyArgs &a, int p, int j, float (&hv)[8]) {
    const size_t stride = static_cast<size_t>(a.T) * a.R;
    const float *hp = a.h + static_cast<size_t>(p) * a.R + j;
    const int np = uniform(a.h_parts);
    float4 v[HP][2];
    if constexpr (COH) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.h, static_cast<uint32_t>(np * stride * 4));
        const uint32_t off = static_cast<uint32_t>((static_cast<size_t>(p) * a.R + j) * 4);
#pragma unroll
        for (int q = 0; q < HP; ++q) {
            if (q < np) {
                const uint32_t qo = static_cast<uint32_t>(q * stride * 4);
                v[q][0] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, qo, CPOL_SC1));
                v[q][1] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16, qo, CPOL_SC1));
            }
        }
    } else {
#pragma unroll
        for (int q = 0; q < HP; ++q) {
            if (q < np) {
                const float4 *hq = reinterpret_cast<const float4 *>(hp + q * stride);
                v[q][0] = hq[0];
                v[q][1] = hq[1];
            }
        }
    }
    float4 h0 = v[0][0], h1 = v[0][1];
    auto add = [&](const float4 &u0, const float4 &u1) {
        h0.x += u0.x; h0.y += u0.y; h0.z += u0.z; h0.w += u0.w;
        h1.x += u1.x; h1.y += u1.y; h1.z += u1.z; h1.w += u1.w;
    };
#pragma unroll
    for (int q = 1; q < HP; ++q)
        if (q < np) add(v[q][0], v[q][1]);
    static_assert(!COH || HP == MAX_HPARTS, "coherent h reads keep every part in flight");
    for (int q = HP; q < np; ++q) {
        const float4 *hq = reinterpret_cast<const float4 *>(hp + q * stride);
        add(hq[0], hq[1]);
    }
    hv[0] = h0.x; hv[1] = h0.y; hv[2] = h0.z; hv[3] = h0.w;
    hv[4] = h1.x; hv[5] = h1.y; hv[6] = h1.z; hv[7] = h1.w;
}

// Routing facts of a wave tile's rows, one row per lane: lane r holds row
// p0 + 16 tb + r of each of the TB row blocks (lanes 16..63 repeat lanes
// 0..15).  g is the bucket record (-1 for rows past rows_end), tok the token,
// key / mode the bucket's slot and mode, s the slot's scale.  Three batched
// rounds of loads for all TB blocks at once.
template <int TB>
struct RowFacts {
    int g[TB];
    int tok[TB];
    int key[TB];
    int mode[TB];
    int rank[TB];  // the slot's true rank (rank steps past it are skipped)
    float s[TB];
};

// row_facts in two stages, so that a caller can put other independent loads
// between them: the first issues the rows' bucket and token loads, the second
// (which waits for them) the bucket records and slot entries.
template <int TB>
__device__ __forceinline__ void row_facts_begin(const ApplyArgs &a, int p0, int rows_end, RowFacts<TB> &f) {
    const int r = threadIdx.x & 15;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
        const int pc = min(p0 + tb * 16 + r, rows_end - 1);
        f.g[tb] = a.rv.pos_seg[pc];
        f.tok[tb] = a.rv.perm[pc];
    }
}

template <int TB>
__device__ __forceinline__ void row_facts_end(const ApplyArgs &a, int p0, int rows_end, RowFacts<TB> &f) {
    const int r = threadIdx.x & 15;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) f.tok[tb] = min(max(f.tok[tb], 0), a.T - 1);
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
        f.key[tb] = a.rv.segs[4 * f.g[tb]];
        f.mode[tb] = a.rv.segs[4 * f.g[tb] + 3];
    }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
        const SlotDev *sd = a.slots + min(f.key[tb], a.S - 1);
        f.s[tb] = sd->scale;
        f.rank[tb] = sd->rank;
    }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
        if (p0 + tb * 16 + r >= rows_end) f.g[tb] = -1;
}

template <int TB>
__device__ __forceinline__ void row_facts(const ApplyArgs &a, int p0, int rows_end, RowFacts<TB> &f) {
    row_facts_begin<TB>(a, p0, rows_end, f);
    row_facts_end<TB>(a, p0, rows_end, f);
}

// Raw h of 16 sorted rows p0 .. (clamped to rows_end) for every 32-wide rank
// step, parts added in order: lane (r, kq) holds row p0 + r, ranks js * 32 +
// 8 kq .. +7 -- what lora_expand_mfma loads for a one-block tile, fetched
// early by a caller that has the rows before their routing facts.
template <int HP = MAX_HPARTS>
__device__ __forceinline__ void prefetch_h1(const ApplyArgs &a, int p0, int rows_end, float (&hv)[2][8]) {
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;
    const int kq = lane >> 4;
    const int row = min(p0 + r, rows_end - 1);
#pragma unroll
    for (int js = 0; js < 2; ++js) load_h8<HP>(a, row, min(js * 32 + 8 * kq, a.R - 8), hv[js]);
}

// Adds s_g * h[p][:] . B_g[n][:] to acc for every row p of the wave tile whose
// bucket g has mode `want` (FUSED inside the base GEMM, SEPARATE in the
// residual kernel).  The wave tile is TB blocks of 16 sorted rows starting at
// row p0, and WC blocks of 16 columns starting at column n0; rows_end bounds
// the rows considered (T, or the end of one bucket tile); f holds the rows'
// routing facts.  A block's H operand is s * h rounded to the pool dtype
// (zero for other rows); the h rows of the next block are requested while
// the current one is multiplied.  When one bucket covers the whole tile (the
// usual case for long buckets) its B fragments are loaded once; otherwise
// each block meets its buckets one at a time (rows are sorted, so a bucket
// is a run of lanes), one round of B loads per bucket.
template <int DT, int TB, int WC, int HP = MAX_HPARTS, bool COH = false>
__device__ __forceinline__ void lora_expand_mfma(const ApplyArgs &a, int p0, int rows_end, int n0, int want,
                                                 const RowFacts<TB> &f, f32x4_t (&acc)[TB][WC],
                                                 const float (*hpre)[8] = nullptr) {
    using E = Elem<DT>;
    using V = typename E::vec8;
    using raw = typename E::raw;
    constexpr int JM = 2;  // 32-wide rank steps (Rp <= 64)
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;
    const int kq = lane >> 4;
    const int Rp = a.R;
    p0 = uniform(p0);
    rows_end = uniform(rows_end);
    n0 = uniform(n0);

    bool any_row = false;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) any_row = any_row || (f.g[tb] >= 0 && f.key[tb] < a.S && f.mode[tb] == want);
    if (__ballot(any_row) == 0) return;

    // Raw h of block tb's rows for rank step js (unconditional loads:
    // clamped row and rank).
    // (hpre: the one block's h, prefetched by the caller with prefetch_h1.)
    auto load_h = [&](int tb, int js, float (&hv)[8]) {
        if (TB == 1 && hpre != nullptr) {
#pragma unroll
            for (int e = 0; e < 8; ++e) hv[e] = hpre[js][e];
            return;
        }
        const int hrow = a.h_by_token ? f.tok[tb] : min(p0 + tb * 16 + r, rows_end - 1);
        load_h8<HP, COH>(a, hrow, min(js * 32 + 8 * kq, Rp - 8), hv);
    };
    // H operand of block tb, rank step js, for bucket gg (-1: any bucket of
    // mode `want`).
    auto make_h = [&](int tb, int js, int gg, const float (&hv)[8]) {
        const bool lr = f.g[tb] >= 0 && f.key[tb] < a.S && f.mode[tb] == want && (gg < 0 || f.g[tb] == gg);
        raw hr[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) hr[e] = E::from_f(f.s[tb] * hv[e]);
        return (lr && js * 32 + 8 * kq < Rp) ? __builtin_bit_cast(V, hr) : zero8<V>();
    };
    auto load_b = [&](int key, int js, V (&bf)[WC]) {
        const int j = min(js * 32 + 8 * kq, Rp - 8);
        const uint16_t *bp =
            static_cast<const uint16_t *>(a.B_slab) + (static_cast<size_t>(key) * a.d_out + n0 + r) * Rp + j;
#pragma unroll
        for (int wc = 0; wc < WC; ++wc) bf[wc] = load8<V>(bp + static_cast<size_t>(wc) * 16 * Rp);
    };

    // One bucket over the whole tile?
    const int g_first = uniform(f.g[0]);
    bool other = false;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) other = other || (f.g[tb] >= 0 && f.g[tb] != g_first);
    if (__ballot(other) == 0) {
        const int key = uniform(f.key[0]);
        // Rank steps holding the true rank (B columns past it are zero).
        const int njs = uniform(min((Rp + 31) / 32, (f.rank[0] + 31) / 32));
#pragma unroll
        for (int js = 0; js < JM; ++js) {
            if (js >= njs) break;
            V bf[WC];
            load_b(key, js, bf);
            float hv[2][8];
            load_h(0, js, hv[0]);
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                if (p0 + tb * 16 >= rows_end) break;
                if (tb + 1 < TB) load_h(tb + 1, js, hv[(tb + 1) & 1]);  // next block's rows in flight
                const V h = make_h(tb, js, -1, hv[tb & 1]);
#pragma unroll
                for (int wc = 0; wc < WC; ++wc) acc[tb][wc] = E::mfma(h, bf[wc], acc[tb][wc]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        return;
    }
    // One row block (the split-sum and residual kernels): the block's buckets
    // NBB at a time, the B fragments of a batch requested together, so that a
    // block of many short buckets waits for ceil(buckets / NBB) rounds of B
    // loads instead of one per bucket.
    if constexpr (TB == 1) {
        constexpr int NBB = 4;
        float hv[JM][8];
#pragma unroll
        for (int js = 0; js < JM; ++js) load_h(0, js, hv[js]);
        const int last = min(15, rows_end - 1 - p0);
        const int g0 = uniform(f.g[0]);
        const int g1 = __builtin_amdgcn_readlane(f.g[0], last);
        for (int gb = g0; gb <= g1; gb += NBB) {
            int keys[NBB], rks[NBB];
            bool use[NBB];
#pragma unroll
            for (int b = 0; b < NBB; ++b) {
                const unsigned long long m = __ballot(f.g[0] == gb + b) & 0xFFFFull;
                const int l0 = m ? __ffsll(static_cast<long long>(m)) - 1 : 0;
                const int key = __builtin_amdgcn_readlane(f.key[0], l0);
                const int mode = __builtin_amdgcn_readlane(f.mode[0], l0);
                rks[b] = __builtin_amdgcn_readlane(f.rank[0], l0);
                use[b] = gb + b <= g1 && m != 0 && key < a.S && mode == want;
                keys[b] = key;
            }
#pragma unroll
            for (int js = 0; js < JM; ++js) {
                if (js * 32 >= Rp) break;
                V bf[NBB][WC];
#pragma unroll
                for (int b = 0; b < NBB; ++b) load_b(use[b] && js * 32 < rks[b] ? keys[b] : 0, js, bf[b]);
#pragma unroll
                for (int b = 0; b < NBB; ++b) {
                    if (use[b] && js * 32 < rks[b]) {
                        const V h = make_h(0, js, gb + b, hv[js]);
#pragma unroll
                        for (int wc = 0; wc < WC; ++wc) acc[0][wc] = E::mfma(h, bf[b][wc], acc[0][wc]);
                    }
                }
            }
        }
        return;
    }
    if constexpr (TB * WC <= 8) {
        // Several row blocks meeting several buckets: the wave's buckets (a
        // run of bucket records, since rows are sorted) NBB at a time, each
        // batch's B fragments requested together and multiplied into every
        // block that holds rows of the batch's buckets.  A block's H operand
        // (s * h of its rows of mode `want`) is formed once per rank step and
        // masked to one bucket's rows per product; a bucket's slot, mode and
        // rank come from the row facts of one of its rows (a ballot per
        // block).  Two batches are in flight: batch k + 1's B loads are
        // issued before batch k's products, so a wave of many short buckets
        // waits for about one round of loads instead of one per batch.  The B
        // loads are unconditional (a bucket left out, or a batch past the
        // run, reads slot 0's B and is not multiplied): the wait before a
        // batch's products then always counts the next batch's loads alone.
        // The loops over rank steps and batch pairs stay rolled (their code
        // is fetched once).
        constexpr int NBB = 4;
        const int last_row = min(rows_end, p0 + TB * 16) - 1 - p0;  // >= 0: p0 < rows_end
        const int g_lo = uniform(f.g[0]);
        int g_hi = g_lo;
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
            if (tb == last_row / 16) g_hi = __builtin_amdgcn_readlane(f.g[tb], last_row % 16);
        struct Batch {
            int keys[NBB];
            bool use[NBB];
            uint32_t blocks[NBB];  // bit tb: block tb holds rows of the bucket
        };
        auto describe = [&](int gb, int js, Batch &bt) {
#pragma unroll
            for (int b = 0; b < NBB; ++b) {
                const int gg = gb + b;
                uint32_t bl = 0;
                int key = a.S, mode = SEG_NONE, rk = 0;
#pragma unroll
                for (int tb = TB - 1; tb >= 0; --tb) {
                    const unsigned long long m = __ballot(f.g[tb] == gg) & 0xFFFFull;
                    if (m != 0) {
                        const int l0 = __ffsll(static_cast<long long>(m)) - 1;
                        bl |= 1u << tb;
                        key = __builtin_amdgcn_readlane(f.key[tb], l0);
                        mode = __builtin_amdgcn_readlane(f.mode[tb], l0);
                        rk = __builtin_amdgcn_readlane(f.rank[tb], l0);
                    }
                }
                bt.use[b] = gg <= g_hi && bl != 0 && key < a.S && mode == want && js * 32 < rk;
                bt.keys[b] = key;
                bt.blocks[b] = bl;
            }
        };
        auto issue = [&](const Batch &bt, int js, V (&bf)[NBB][WC]) {
#pragma unroll
            for (int b = 0; b < NBB; ++b) load_b(bt.use[b] ? bt.keys[b] : 0, js, bf[b]);
        };
        auto multiply = [&](int gb, const Batch &bt, const V (&hq)[TB], const V (&bf)[NBB][WC]) {
#pragma unroll
            for (int b = 0; b < NBB; ++b) {
                if (!bt.use[b]) continue;
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    if ((bt.blocks[b] >> tb) & 1u) {
                        const V h = f.g[tb] == gb + b ? hq[tb] : zero8<V>();
#pragma unroll
                        for (int wc = 0; wc < WC; ++wc) acc[tb][wc] = E::mfma(h, bf[b][wc], acc[tb][wc]);
                    }
                }
            }
        };
#pragma nounroll
        for (int js = 0; js < JM; ++js) {
            if (js * 32 >= Rp) break;
            V hq[TB];
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                float hv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                if (p0 + tb * 16 < rows_end) load_h(tb, js, hv);
                hq[tb] = make_h(tb, js, -1, hv);
            }
            Batch ba, bb;
            V fa[NBB][WC], fb[NBB][WC];
            describe(g_lo, js, ba);
            issue(ba, js, fa);
#pragma nounroll
            for (int gb = g_lo; gb <= g_hi; gb += 2 * NBB) {
                describe(gb + NBB, js, bb);
                issue(bb, js, fb);
                multiply(gb, ba, hq, fa);
                if (gb + NBB > g_hi) break;
                describe(gb + 2 * NBB, js, ba);
                issue(ba, js, fa);
                multiply(gb + NBB, bb, hq, fb);
            }
        }
        return;
    }
    // Wide wave tiles (registers for batches would not fit beside the
    // accumulators): block by block, bucket by bucket.
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
        const int pb = p0 + tb * 16;
        if (pb >= rows_end) break;
        float hv[JM][8];
#pragma unroll
        for (int js = 0; js < JM; ++js) load_h(tb, js, hv[js]);
        const int last = min(15, rows_end - 1 - pb);
        const int g0 = uniform(f.g[tb]);
        const int g1 = __builtin_amdgcn_readlane(f.g[tb], last);
        for (int gg = g0; gg <= g1; ++gg) {
            const unsigned long long m = __ballot(f.g[tb] == gg) & 0xFFFFull;
            if (m == 0) continue;
            const int l0 = __ffsll(static_cast<long long>(m)) - 1;
            const int key = __builtin_amdgcn_readlane(f.key[tb], l0);
            const int mode = __builtin_amdgcn_readlane(f.mode[tb], l0);
            const int rk = __builtin_amdgcn_readlane(f.rank[tb], l0);
            if (key >= a.S || mode != want) continue;
#pragma unroll
            for (int js = 0; js < JM; ++js) {
                if (js * 32 >= Rp || js * 32 >= rk) break;
                V bf[WC];
                load_b(key, js, bf);
                const V h = make_h(tb, js, gg, hv[js]);
#pragma unroll
                for (int wc = 0; wc < WC; ++wc) acc[tb][wc] = E::mfma(h, bf[wc], acc[tb][wc]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Round and store the wave tile's rows (sorted rows p0 + ...) to y in token
// order; invalid tokens get NaN.  The accumulator row 16 tb + 4 kq + i of a
// lane is row 4 kq + i of block tb, whose facts lane 4 kq + i holds.
template <int DT, int TB, int WC>
__device__ __forceinline__ void store_rows(const ApplyArgs &a, int p0, int rows_end, int n0, const RowFacts<TB> &f,
                                           const f32x4_t (&acc)[TB][WC]) {
    using E = Elem<DT>;
    using raw = typename E::raw;
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;
    const int kq = lane >> 4;
    raw *y = static_cast<raw *>(a.y);
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = __shfl(f.key[tb], kq * 4 + i, 64);
            const int tok = __shfl(f.tok[tb], kq * 4 + i, 64);
            const int p = p0 + tb * 16 + kq * 4 + i;
            if (p >= rows_end) continue;
            const size_t base = static_cast<size_t>(tok) * a.d_out + n0 + r;
#pragma unroll
            for (int wc = 0; wc < WC; ++wc)
                y[base + wc * 16] = (key == a.S + 1) ? E::qnan : E::from_f(acc[tb][wc][i]);
        }
    }
}

// store_rows with each row's token read from `rowtok` (row p0 + i at
// rowtok[i], in LDS; the bitwise NOT of the token marks a row of the invalid
// bucket, stored as NaN).
template <int DT, int TB, int WC>
__device__ __forceinline__ void store_rows_tok(const ApplyArgs &a, int p0, int rows_end, int n0, const int *rowtok,
                                               const f32x4_t (&acc)[TB][WC]) {
    using E = Elem<DT>;
    using raw = typename E::raw;
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;
    const int kq = lane >> 4;
    raw *y = static_cast<raw *>(a.y);
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = p0 + tb * 16 + kq * 4 + i;
            if (p >= rows_end) continue;
            const int v = rowtok[tb * 16 + kq * 4 + i];
            const size_t base = static_cast<size_t>(v < 0 ? ~v : v) * a.d_out + n0 + r;
#pragma unroll
            for (int wc = 0; wc < WC; ++wc) y[base + wc * 16] = v < 0 ? E::qnan : E::from_f(acc[tb][wc][i]);
        }
    }
}

}  // namespace lora
