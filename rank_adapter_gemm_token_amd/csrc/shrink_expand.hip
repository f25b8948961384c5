// shrink_expand.hip -- the LoRA shrink h = x A_slot^T and the separate
// residual expand y += s h B_slot^T, for fp16/bf16 pools.
//
// A maps hidden size to rank and B maps rank to hidden size ("LLM 多 LoRA 推理服务
// 工程 2026", routing layer, zero-pad paragraph).  The separate school runs the
// LoRA product after the base linear as a residual add, at the price of one
// more launch and one more round trip of y (same page, execution-unit
// paragraph).
//
// Shrink: one workgroup of 4 waves per 16-row tile of one adapter bucket
// (shrink_role): the tile's x rows are the MFMA A operand, the slot's
// rank-padded A rows the B operand; K is split over the waves and the
// partial sums are added in LDS in a fixed order: h (fp32, by sorted row).
// The decode path runs the same role inside its main kernel.  Calls of many
// tokens (long buckets) group SHRINK_G consecutive tiles per workgroup: when
// they belong to one bucket, each A fragment is loaded once for all of them
// (A is read once per 16 G rows instead of once per 16), otherwise the tiles
// go one at a time.
//
// Separate expand: one workgroup of 4 waves per (tile of a SEPARATE bucket,
// 64 columns); acc = s * h . B on MFMA, then y = round(y + acc).
#include <algorithm>

#include "epilogue.hpp"

namespace lora {

namespace {

template <int DT, int RB>
__global__ __launch_bounds__(256) void k_shrink(ApplyArgs a) {
    __shared__ u32x4_t lds[4 * RB * 64];
    // Unit (tile, k part): part-major within a tile.
    shrink_role<DT, RB, 4>(a, blockIdx.x / a.shrink_parts, blockIdx.x % a.shrink_parts, lds);
}

// Partial h over k part `part` for G row blocks (16 rows each) of one bucket:
// slot `key`, sorted rows row0 .. row0 + rows - 1 (rows > 16 (G - 1)).  As
// shrink_unit, with the A fragments of each k step shared by the G blocks;
// the 4 waves split the part's k steps, their sums are added in LDS in a
// fixed order (wave 0, 1, 2, 3, the same order as shrink_unit's, so a row's
// h does not depend on the grouping).
template <int DT, int RB, int G>
__device__ __forceinline__ void shrink_group_unit(const ApplyArgs &a, int key, int row0, int rows, int part,
                                                  u32x4_t *lds) {
    using E = Elem<DT>;
    using V = typename E::vec8;
    constexpr int NWV = 4;
    key = uniform(key);
    row0 = uniform(row0);
    rows = uniform(rows);
    const int Rp = a.R;
    const int wave = uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;
    const int kq = lane >> 4;
    const int kst = a.d_in / 32;
    const int split = part * NWV + wave;
    const int nsplit = a.shrink_parts * NWV;
    const int kb = split * kst / nsplit;
    const int ke = (split + 1) * kst / nsplit;

    const uint16_t *xp[G];
    bool xv[G];
#pragma unroll
    for (int gb = 0; gb < G; ++gb) {
        xv[gb] = gb * 16 + r < rows;
        const int tok = min(max(a.rv.perm[row0 + min(gb * 16 + r, rows - 1)], 0), a.T - 1);
        xp[gb] = static_cast<const uint16_t *>(a.x) + static_cast<size_t>(tok) * a.d_in + 8 * kq;
    }
    const uint16_t *ap[RB];
    bool av[RB];
#pragma unroll
    for (int cb = 0; cb < RB; ++cb) {
        const int j = cb * 16 + r;
        av[cb] = j < Rp;
        ap[cb] = static_cast<const uint16_t *>(a.A_slab) +
                 (static_cast<size_t>(key) * Rp + (av[cb] ? j : 0)) * a.d_in + 8 * kq;
    }
    f32x4_t acc[G][RB];
#pragma unroll
    for (int gb = 0; gb < G; ++gb)
#pragma unroll
        for (int cb = 0; cb < RB; ++cb) acc[gb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    constexpr int U = 32 / (G + RB);  // k steps whose loads are in flight together (32 loads)
    for (int k0 = kb; k0 < ke; k0 += U) {
        V xa[U][G];
        V b[U][RB];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kk = min(k0 + u, ke - 1);  // clamped: loads stay unconditional
#pragma unroll
            for (int gb = 0; gb < G; ++gb) xa[u][gb] = load8<V>(xp[gb] + kk * 32);
#pragma unroll
            for (int cb = 0; cb < RB; ++cb) b[u][cb] = load8<V>(ap[cb] + kk * 32);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int gb = 0; gb < G; ++gb) {
                const V xm = (k0 + u < ke && xv[gb]) ? xa[u][gb] : zero8<V>();
#pragma unroll
                for (int cb = 0; cb < RB; ++cb)
                    acc[gb][cb] = E::mfma(xm, av[cb] ? b[u][cb] : zero8<V>(), acc[gb][cb]);
            }
        }
    }
    f32x4_t *red = reinterpret_cast<f32x4_t *>(lds);
#pragma unroll
    for (int gb = 0; gb < G; ++gb)
#pragma unroll
        for (int cb = 0; cb < RB; ++cb) red[((wave * G + gb) * RB + cb) * 64 + lane] = acc[gb][cb];
    __syncthreads();
    // Wave w adds and stores row block w (G = 4 blocks over 4 waves).
    float *hout = a.h + static_cast<size_t>(part) * a.T * Rp;
    for (int gb = wave; gb < G; gb += NWV) {
#pragma unroll
        for (int cb = 0; cb < RB; ++cb) {
            f32x4_t sm = red[((0 * G + gb) * RB + cb) * 64 + lane];
            for (int w = 1; w < NWV; ++w) sm += red[((w * G + gb) * RB + cb) * 64 + lane];
            const int j = cb * 16 + r;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = gb * 16 + kq * 4 + i;
                if (row < rows && j < Rp) store_h<true>(&hout[static_cast<size_t>(row0 + row) * Rp + j], sm[i]);
            }
        }
        for (int j = RB * 16 + r; j < Rp; j += 16) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = gb * 16 + kq * 4 + i;
                if (row < rows) store_h<true>(&hout[static_cast<size_t>(row0 + row) * Rp + j], 0.0f);
            }
        }
    }
}

// G consecutive tiles of the routing's tile list (group blockIdx.x / parts,
// k part blockIdx.x % parts): one pass with shared A fragments over the rank
// blocks that hold the slot's true rank when they are consecutive tiles of
// one bucket, else shrink_role tile by tile.  Each part stores its share of
// the group's h rows with agent-coherent stores into part slot `part`, then
// counts itself on the group's counter; the part that completes the count
// resets it and adds the parts in order 0, 1, .. (the order in which the
// consumers would add them) into part 0, which is all the consumers read.
template <int DT, int RB, int G>
__global__ __launch_bounds__(256) void k_shrink_grouped(ApplyArgs a) {
    constexpr int MAXP = 4;  // tiled_h_parts' bound for grouped calls
    __shared__ u32x4_t lds[4 * G * RB * 64];
    __shared__ int last;
    const int P = a.shrink_parts;
    const int grp = blockIdx.x / P;
    const int part = blockIdx.x % P;
    const int n_tiles = uniform(*a.rv.n_tiles);
    const int t0 = grp * G;
    if (t0 >= n_tiles) return;
    const int tw0 = uniform(a.rv.tiles[2 * t0]);
    const int seg = tile_seg(tw0);
    const int row0 = uniform(a.rv.tiles[2 * t0 + 1]);
    const int end = uniform(a.rv.segs[4 * seg + 1] + a.rv.segs[4 * seg + 2]);
    // The group is one bucket's run of G tiles when its last tile exists and
    // belongs to the same bucket (tiles of a bucket are consecutive, 16 rows
    // apart).
    bool one = t0 + G - 1 < n_tiles;
    if (one) one = tile_seg(uniform(a.rv.tiles[2 * (t0 + G - 1)])) == seg;
    if (one) {
        // Rank blocks that hold the slot's true rank (as shrink_role).
        const int nrb = uniform(min(RB, (tile_rank(tw0) + 15) / 16));
        const int key = a.rv.segs[4 * seg];
        const int rows = min(16 * G, end - row0);
        if (RB >= 4 && nrb == 4) shrink_group_unit<DT, (RB >= 4 ? 4 : 1), G>(a, key, row0, rows, part, lds);
        else if (RB >= 3 && nrb == 3) shrink_group_unit<DT, (RB >= 3 ? 3 : 1), G>(a, key, row0, rows, part, lds);
        else if (RB >= 2 && nrb == 2) shrink_group_unit<DT, (RB >= 2 ? 2 : 1), G>(a, key, row0, rows, part, lds);
        else shrink_group_unit<DT, 1, G>(a, key, row0, rows, part, lds);
    } else {
        for (int t = t0; t < min(t0 + G, n_tiles); ++t) {
            shrink_role<DT, RB, 4, true>(a, t, part, lds);
            __syncthreads();
        }
    }
    if (P == 1) return;
    // The stores are complete (at the agent's coherence point) before the
    // part is counted.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned old = __hip_atomic_fetch_add(a.cnt + grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int l = old == static_cast<unsigned>(P - 1);
        if (l) __hip_atomic_store(a.cnt + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = l;
    }
    __syncthreads();
    if (!last) return;
    // The group's rows: each tile's 16 rows (fewer at the end of a bucket),
    // Rp floats each, contiguous in every part (rows are h rows by sorted
    // position): at most 16 Rp / 4 <= 256 float4 a tile, one per thread.
    // Every tile's and every part's loads are issued before the first add
    // (clamped offsets keep them unconditional); a run of one bucket's tiles
    // needs no tile records (16 rows apart from row0).
    const int Rp = a.R;
    const uint32_t pstride = static_cast<uint32_t>(a.T) * Rp * 4;
    const __amdgpu_buffer_rsrc_t hrs = make_rsrc(a.h, static_cast<uint32_t>(P) * pstride);
    uint32_t off[G];
    bool ok[G];
#pragma unroll
    for (int ti = 0; ti < G; ++ti) {
        const int t = t0 + ti;
        int r0, e;
        if (one) {
            r0 = row0 + ti * 16;
            e = end;
        } else {
            const int tc = min(t, n_tiles - 1);
            r0 = a.rv.tiles[2 * tc + 1];
            const int sg = tile_seg(a.rv.tiles[2 * tc]);
            e = a.rv.segs[4 * sg + 1] + a.rv.segs[4 * sg + 2];
        }
        const int n4 = min(16, e - r0) * Rp / 4;  // float4 of the tile (Rp is a multiple of 8)
        ok[ti] = t < n_tiles && static_cast<int>(threadIdx.x) < n4;
        off[ti] = ok[ti] ? static_cast<uint32_t>(r0) * Rp * 4 + threadIdx.x * 16 : 0u;
    }
    f32x4_t v[G][MAXP];
#pragma unroll
    for (int ti = 0; ti < G; ++ti)
#pragma unroll
        for (int pp = 0; pp < MAXP; ++pp)
            if (pp < P)
                v[ti][pp] = __builtin_bit_cast(
                    f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(hrs, off[ti], pp * pstride, CPOL_SC1));
#pragma unroll
    for (int ti = 0; ti < G; ++ti) {
        if (!ok[ti]) continue;
        f32x4_t sm = v[ti][0];
#pragma unroll
        for (int pp = 1; pp < MAXP; ++pp)
            if (pp < P) sm += v[ti][pp];
        *reinterpret_cast<f32x4_t *>(reinterpret_cast<char *>(a.h) + off[ti]) = sm;
    }
}

template <int DT>
__global__ __launch_bounds__(256) void k_expand_sep(ApplyArgs a) {
    using E = Elem<DT>;
    using raw = typename E::raw;
    const int tile = blockIdx.x;
    if (tile >= uniform(*a.rv.n_tiles)) return;
    const int seg = uniform(tile_seg(a.rv.tiles[2 * tile]));
    if (uniform(a.rv.segs[4 * seg + 3]) != SEG_SEPARATE) return;
    const int row0 = uniform(a.rv.tiles[2 * tile + 1]);
    const int end = uniform(a.rv.segs[4 * seg + 1] + a.rv.segs[4 * seg + 2]);
    const int rows_end = min(row0 + TILE_ROWS, end);
    const int wave = uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;
    const int kq = lane >> 4;
    const int n0 = blockIdx.y * 64 + wave * 16;
    f32x4_t acc[1][1] = {{f32x4_t{0.f, 0.f, 0.f, 0.f}}};
    RowFacts<1> f;
    row_facts<1>(a, row0, rows_end, f);
    lora_expand_mfma<DT, 1, 1>(a, row0, rows_end, n0, SEG_SEPARATE, f, acc);
    raw *y = static_cast<raw *>(a.y);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int tok = __shfl(f.tok[0], kq * 4 + i, 64);
        const int p = row0 + kq * 4 + i;
        if (p >= rows_end) continue;
        raw *yp = y + static_cast<size_t>(tok) * a.d_out + n0 + r;
        *yp = E::from_f(E::to_f(*yp) + acc[0][0][i]);
    }
}

template <int DT>
hipError_t shrink_rb(const ApplyArgs &a, hipStream_t st) {
    if (a.shrink_g > 1) {
        if (a.shrink_parts > 4 || (a.shrink_parts > 1 && a.cnt == nullptr)) return hipErrorInvalidValue;
        const dim3 grid((a.tiles_bound + SHRINK_G - 1) / SHRINK_G * a.shrink_parts);
        switch ((a.R + 15) / 16) {
            case 1: hipLaunchKernelGGL((k_shrink_grouped<DT, 1, SHRINK_G>), grid, dim3(256), 0, st, a); break;
            case 2: hipLaunchKernelGGL((k_shrink_grouped<DT, 2, SHRINK_G>), grid, dim3(256), 0, st, a); break;
            case 3: hipLaunchKernelGGL((k_shrink_grouped<DT, 3, SHRINK_G>), grid, dim3(256), 0, st, a); break;
            default: hipLaunchKernelGGL((k_shrink_grouped<DT, 4, SHRINK_G>), grid, dim3(256), 0, st, a); break;
        }
        return hipGetLastError();
    }
    const dim3 grid(a.tiles_bound * a.shrink_parts);
    switch ((a.R + 15) / 16) {
        case 1: hipLaunchKernelGGL((k_shrink<DT, 1>), grid, dim3(256), 0, st, a); break;
        case 2: hipLaunchKernelGGL((k_shrink<DT, 2>), grid, dim3(256), 0, st, a); break;
        case 3: hipLaunchKernelGGL((k_shrink<DT, 3>), grid, dim3(256), 0, st, a); break;
        default: hipLaunchKernelGGL((k_shrink<DT, 4>), grid, dim3(256), 0, st, a); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_shrink16(const ApplyArgs &a, hipStream_t st) {
    return (a.dtype == DT_F16) ? shrink_rb<DT_F16>(a, st) : shrink_rb<DT_BF16>(a, st);
}

int shrink_group(int T, int tiles, int counters) {
    return T >= SHRINK_G_MIN_T && (tiles + SHRINK_G - 1) / SHRINK_G <= counters ? SHRINK_G : 1;
}

int tiled_h_parts(int d_in, int R, int tiles, int T) {
    if (T >= SHRINK_G_MIN_T) {
        // Grouped shrink: ~288 .. 512 workgroups over the groups, at most 4
        // parts (added into part 0 by the shrink itself).
        const int units = (tiles + SHRINK_G - 1) / SHRINK_G;
        return std::max(1, std::min(4, (512 + units - 1) / units));
    }
    // With few tiles (a few workgroups per CU at most) each wave's chain of
    // dependent load rounds sets the time: split k until each wave has about
    // one round (U k steps as in shrink_unit: 16, 8 or 4 for 1, 2, 3-4 rank
    // blocks) or the grid reaches ~512 workgroups.  With many tiles the
    // chip is full already and extra parts only add h traffic.
    if (tiles >= 256) return 1;
    const int rb = (R + 15) / 16;
    const int u = rb == 1 ? 16 : rb == 2 ? 8 : 4;
    const int kst = d_in / 32;
    int p = (kst + 4 * u - 1) / (4 * u);
    p = std::min(p, (512 + tiles - 1) / tiles);
    return std::max(1, std::min(p, MAX_HPARTS));
}

hipError_t launch_expand_sep16(const ApplyArgs &a, hipStream_t st) {
    const dim3 grid(a.tiles_bound, a.d_out / 64);
    if (a.dtype == DT_F16)
        hipLaunchKernelGGL(k_expand_sep<DT_F16>, grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(k_expand_sep<DT_BF16>, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace lora
