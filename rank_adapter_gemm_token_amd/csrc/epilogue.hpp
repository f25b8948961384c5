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
// 16-row tile of an adapter bucket: slot `key`, sorted rows row0 .. row0 +
// rows - 1, whose tokens are perm[row0 ..] (perm may live in LDS or global
// memory).  One workgroup of NWV waves; the part's k steps are split over the
// waves and the waves' sums are added in LDS in a fixed order.  `lds` holds
// >= NWV * RB * 64 16-byte words.  The part is written to h + part * T * R;
// consumers add the parts in order.
template <int DT, int RB, int NWV>
__device__ __forceinline__ void shrink_unit(const ApplyArgs &a, int key, int row0, int rows, const int32_t *perm,
                                            int part, u32x4_t *lds) {
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
    const int nsplit = a.h_parts * NWV;
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

    constexpr int U = RB == 1 ? 16 : RB == 2 ? 8 : 4;  // k steps whose loads are all in flight together
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
            if (row < rows && j < Rp) hout[static_cast<size_t>(row0 + row) * Rp + j] = s[i];
        }
    }
}

// shrink_unit for tile `tile` of the routing in global memory.
template <int DT, int RB, int NWV>
__device__ __forceinline__ void shrink_role(const ApplyArgs &a, int tile, int part, u32x4_t *lds) {
    if (tile >= uniform(*a.rv.n_tiles)) return;
    const int seg = a.rv.tiles[2 * tile];
    const int row0 = a.rv.tiles[2 * tile + 1];
    const int key = a.rv.segs[4 * seg];
    const int end = a.rv.segs[4 * seg + 1] + a.rv.segs[4 * seg + 2];
    shrink_unit<DT, RB, NWV>(a, key, row0, min(TILE_ROWS, end - row0), a.rv.perm, part, lds);
}

// h[p][j .. j+7] summed over the shrink's k parts in order (p: the h row,
// a sorted position or a token).
__device__ __forceinline__ void load_h8(const ApplyArgs &a, int p, int j, float (&hv)[8]) {
    const size_t stride = static_cast<size_t>(a.T) * a.R;
    const float4 *hp = reinterpret_cast<const float4 *>(a.h + static_cast<size_t>(p) * a.R + j);
    float4 h0 = hp[0], h1 = hp[1];
    for (int q = 1; q < a.h_parts; ++q) {
        const float4 *hq = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(hp) + q * stride);
        const float4 g0 = hq[0], g1 = hq[1];
        h0.x += g0.x; h0.y += g0.y; h0.z += g0.z; h0.w += g0.w;
        h1.x += g1.x; h1.y += g1.y; h1.z += g1.z; h1.w += g1.w;
    }
    hv[0] = h0.x; hv[1] = h0.y; hv[2] = h0.z; hv[3] = h0.w;
    hv[4] = h1.x; hv[5] = h1.y; hv[6] = h1.z; hv[7] = h1.w;
}

// Adds s_g * h[p][:] . B_g[n][:] to acc for every row p of the wave tile whose
// bucket g has mode `want` (FUSED inside the base GEMM, SEPARATE in the
// residual kernel).  The wave tile is TB blocks of 16 sorted rows starting at
// row p0, and WC blocks of 16 columns starting at column n0.  rows_end bounds
// the rows considered (T, or the end of one bucket tile).
template <int DT, int TB, int WC>
__device__ __forceinline__ void lora_expand_mfma(const ApplyArgs &a, int p0, int rows_end, int n0, int want,
                                                 f32x4_t (&acc)[TB][WC]) {
    using E = Elem<DT>;
    using V = typename E::vec8;
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;
    const int kq = lane >> 4;
    const int Rp = a.R;
    p0 = uniform(p0);
    rows_end = uniform(rows_end);
    n0 = uniform(n0);
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
        const int pb = p0 + tb * 16;
        if (pb >= rows_end) break;
        const int g0 = uniform(a.rv.pos_seg[pb]);
        const int g1 = uniform(a.rv.pos_seg[min(pb + 15, rows_end - 1)]);
        const int ph = pb + r;  // this lane's row in the H operand
        const int gh = (ph < rows_end) ? a.rv.pos_seg[ph] : -1;
        for (int g = g0; g <= g1; ++g) {
            const int key = uniform(a.rv.segs[4 * g]);
            const int mode = uniform(a.rv.segs[4 * g + 3]);
            if (key >= a.S || mode != want) continue;
            const float s = a.slots[key].scale;
            for (int js = 0; js < Rp; js += 32) {
                const int j = js + 8 * kq;
                const bool jv = j < Rp;
                V hf = zero8<V>();
                if (jv && gh == g) {
                    float hv[8];
                    load_h8(a, a.h_by_token ? token_of(a, ph) : ph, j, hv);
                    typename E::raw hr[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) hr[e] = E::from_f(s * hv[e]);
                    hf = __builtin_bit_cast(V, hr);
                }
                const uint16_t *bp = static_cast<const uint16_t *>(a.B_slab) +
                                     (static_cast<size_t>(key) * a.d_out + n0 + r) * Rp + j;
#pragma unroll
                for (int wc = 0; wc < WC; ++wc) {
                    const V bf = jv ? load8<V>(bp + static_cast<size_t>(wc) * 16 * Rp) : zero8<V>();
                    acc[tb][wc] = E::mfma(hf, bf, acc[tb][wc]);
                }
            }
        }
    }
}

// Round and store the wave tile's rows (sorted rows p0 + ...) to y in token
// order; invalid tokens get NaN.
template <int DT, int TB, int WC>
__device__ __forceinline__ void store_rows(const ApplyArgs &a, int p0, int rows_end, int n0,
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
            const int key = a.rv.segs[4 * a.rv.pos_seg[p]];
            const size_t base = static_cast<size_t>(token_of(a, p)) * a.d_out + n0 + r;
#pragma unroll
            for (int wc = 0; wc < WC; ++wc)
                y[base + wc * 16] = (key == a.S + 1) ? E::qnan : E::from_f(acc[tb][wc][i]);
        }
    }
}

}  // namespace lora
