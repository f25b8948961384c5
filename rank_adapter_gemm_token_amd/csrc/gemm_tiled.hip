// gemm_tiled.hip -- base projection for calls of more than 64 tokens
// (fp16/bf16) with the fused LoRA term.  Three kernels:
//   * k_gemm_lds<256> (>= 2048 tokens): 256 x 256 tiles staged into LDS by
//     direct loads, the LoRA term computed into the accumulators before the
//     main loop (described at its definition);
//   * k_gemm_lds<64, split> (65 .. 2047 tokens): the same staging
//     over k ranges; the splits of a tile add up inside the launch (the last
//     one to finish sums them in split order) and apply the fused expand;
//   * k_gemm_tiled (shapes off the 128 grid), described here.
//
// Here the projection is a dense contraction with enough rows to be bound by
// the matrix cores, not by HBM, so both operands are reused from LDS:
//   * a workgroup of 4 waves owns a BM x BN output tile (sorted rows x
//     columns); each wave a (BM/2) x (BN/2) quadrant of 16x16 MFMA blocks;
//   * K advances in stages of BK = 64: the next stage's x and W fragments are
//     loaded from global memory into registers while the current stage is
//     multiplied from LDS, then stored to the other LDS buffer (double
//     buffering, one barrier per stage);
//   * LDS holds operands in MFMA fragment order (16 rows x 32 k per 1 KiB
//     fragment, lane-contiguous), so every operand read is a conflict-free
//     16-byte LDS read, and every global load moves 16 rows x 64 B;
//   * x rows are gathered in sorted order (row p = token perm[p]), so the
//     epilogue adds the LoRA term of FUSED buckets with MFMA over contiguous
//     buckets, rounds once, and scatters rows back to token order.
// The tile shape depends on (T, d_out) only.
#include "epilogue.hpp"

namespace lora {

namespace {

constexpr int BK = 64;  // k per stage: two 32-wide MFMA steps

template <int BM, int BN>
struct TileShape {
    static constexpr int TB = BM / 32;          // 16-row blocks per wave
    static constexpr int WC = BN / 32;          // 16-column blocks per wave
    static constexpr int FA = BM / 16 * 2;      // A fragments per stage
    static constexpr int FB = BN / 16 * 2;      // B fragments per stage
    static constexpr int LA = FA / 4;           // A fragments each wave loads
    static constexpr int LB = FB / 4;           // B fragments each wave loads
    static constexpr int STAGE = FA + FB;       // fragments (1 KiB) per stage
};

template <int DT, int BM, int BN>
__global__ __launch_bounds__(256) void k_gemm_tiled(ApplyArgs a) {
    using E = Elem<DT>;
    using V = typename E::vec8;
    using Sh = TileShape<BM, BN>;
    constexpr int TB = Sh::TB;
    constexpr int WC = Sh::WC;
    __shared__ u32x4_t lds[2][Sh::STAGE * 64];

    const int wave = uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;
    const int kq = lane >> 4;
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const int m0 = blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;
    const int ksel = wave & 1;  // the k half (of a 64-k stage) this wave loads

    // Fragments this wave loads each stage: A (rb, ksel) for rb = (wave + 4j) / 2,
    // B (cb, ksel) for cb = (wave + 4j) / 2.  32-bit element offsets from the
    // (uniform) x and W bases keep the per-lane address state small.
    const uint16_t *xg = static_cast<const uint16_t *>(a.x) + ksel * 32 + 8 * kq;
    const uint16_t *wg = static_cast<const uint16_t *>(a.W) + ksel * 32 + 8 * kq;
    uint32_t xo[Sh::LA];
    uint32_t xmask = 0;  // bit j: row of A fragment j is a real token
#pragma unroll
    for (int j = 0; j < Sh::LA; ++j) {
        const int p = m0 + ((wave + 4 * j) >> 1) * 16 + r;
        xmask |= (p < a.T ? 1u : 0u) << j;
        xo[j] = static_cast<uint32_t>(token_of(a, min(p, a.T - 1))) * static_cast<uint32_t>(a.d_in);
    }
    uint32_t wo[Sh::LB];
#pragma unroll
    for (int j = 0; j < Sh::LB; ++j)
        wo[j] = static_cast<uint32_t>(n0 + ((wave + 4 * j) >> 1) * 16 + r) * static_cast<uint32_t>(a.d_in);

    u32x4_t ra[Sh::LA], rbv[Sh::LB];
    auto load_stage = [&](int k0) {
#pragma unroll
        for (int j = 0; j < Sh::LA; ++j) {
            const u32x4_t v = *reinterpret_cast<const u32x4_t *>(xg + xo[j] + k0);
            ra[j] = ((xmask >> j) & 1u) ? v : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < Sh::LB; ++j) rbv[j] = *reinterpret_cast<const u32x4_t *>(wg + wo[j] + k0);
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int j = 0; j < Sh::LA; ++j) lds[buf][(wave + 4 * j) * 64 + lane] = ra[j];
#pragma unroll
        for (int j = 0; j < Sh::LB; ++j) lds[buf][(Sh::FA + wave + 4 * j) * 64 + lane] = rbv[j];
    };

    f32x4_t acc[TB][WC];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int wc = 0; wc < WC; ++wc) acc[tb][wc] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int nst = a.d_in / BK;
    load_stage(0);
    store_stage(0);
    __syncthreads();
    for (int s = 0; s < nst; ++s) {
        const int buf = s & 1;
        if (s + 1 < nst) load_stage((s + 1) * BK);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            // B fragments of the step once; A fragments one row block at a time.
            V bf[WC];
#pragma unroll
            for (int wc = 0; wc < WC; ++wc)
                bf[wc] = __builtin_bit_cast(V, lds[buf][(Sh::FA + (wn * WC + wc) * 2 + ks) * 64 + lane]);
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                const V af = __builtin_bit_cast(V, lds[buf][((wm * TB + tb) * 2 + ks) * 64 + lane]);
#pragma unroll
                for (int wc = 0; wc < WC; ++wc) acc[tb][wc] = E::mfma(af, bf[wc], acc[tb][wc]);
            }
        }
        if (s + 1 < nst) store_stage(buf ^ 1);
        __syncthreads();
    }

    const int pw = m0 + wm * TB * 16;
    const int nw = n0 + wn * WC * 16;
    RowFacts<TB> f;
    row_facts<TB>(a, pw, a.T, f);
    lora_expand_mfma<DT, TB, WC>(a, pw, a.T, nw, SEG_FUSED, f, acc);
    store_rows<DT, TB, WC>(a, pw, a.T, nw, f, acc);
}

// 256-row tiles, operands straight into LDS.  A workgroup of 8 waves computes
// a 256 x BN output tile over a range of k stages: 2 x 4 waves of 128 rows x
// BN/4 columns for BN = 256 and 128, 4 x 2 waves of 64 rows x 32 columns for
// BN = 64 (fewer LDS operand reads per MFMA than 128 x 16).  A 64-wide k stage
// is 16 row blocks of x and BN/16 of W, each 16 rows x 128 bytes (2 KiB) in
// LDS.  Operands go from global memory into LDS directly (buffer_load_dwordx4
// ... lds: lane l's 16 bytes land at instruction base + 16 l), one
// instruction per 8 rows, 8 lanes covering each row's whole 128-byte line.
// Which 16-byte chunk a lane fetches is XOR-swizzled by row, so the chunk in
// position m of row rho is chunk m ^ sw(rho), sw(rho) = rho & 7.  An MFMA
// operand read (lane 16 g + r: row r, chunk 4 ks + g) is then free of bank
// conflicts on gfx950: its 64 banks serve a ds_read_b128 16 lanes a cycle,
// lanes 8 j .. 8 j + 7 together with lanes 8 (j ^ 3) .. (lanes 0-7 with
// 24-31, 8-15 with 16-23: the grouping that timed read patterns agree
// with), here rows 0-7 of chunk c with rows 8-15
// of chunk c ^ 1, whose positions sw(rho) ^ c and sw(rho) ^ c ^ 1 differ in
// the last bit.  The swizzle (rho & 7) ^ (rho >> 3) made those two octets
// collide: a 2-way conflict on every read.  Two or three LDS buffers (separate arrays, so the compiler
// can tell a stage's reads from the next stages' loads): stages s + 1 (and s
// + 2) are loaded while stage s is multiplied, one barrier a stage.
//
// SPLIT = false (calls of >= 2048 tokens): all of d_in, then the fused
// expand and the scatter to token order in the epilogue.
// SPLIT = true (calls of 65 .. 2047 tokens, too few 256-row tiles to fill
// the chip): the grid is tiles x splits workgroups; split z of a tile takes
// the z-th of `splits` k ranges.  With one split the workgroup finishes its
// tile as the unsplit kernel does.  Otherwise each split stores its fp32
// partial sums (MFMA fragment order, agent-coherent stores that reach the
// memory side before the split is counted), then adds one to the tile's
// counter; the split that brings it to `splits` resets it to 0 for the next
// call, loads the other splits' partial sums (agent-coherent loads), adds
// all of them in split order z = 0, 1, .. (so the sum does not depend on
// which split finished last), adds the fused expand and stores y.  No
// workgroup waits for another, except (FS, below) an h consumer's bounded
// wait for the in-launch shrink.  The splits of a tile are numbered so that the
// hardware's round-robin dealing of workgroups to the 8 XCDs puts them on one
// XCD when 8 divides the grid.
using lds_ptr = __attribute__((address_space(3))) void *;

// Byte offset of an LDS object.
__device__ __forceinline__ uint32_t lds_offset(const void *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)(p)));
}

// 16-byte LDS read at byte offset `addr`, issued as inline assembly: its
// result is usable only after an lgkmcnt wait (lgkm_wait) and pin().
__device__ __forceinline__ u32x4_t ds_read16(uint32_t addr) {
    u32x4_t v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
    return v;
}

// Waits until at most N LDS reads of this wave are outstanding.
template <int N>
__device__ __forceinline__ void lgkm_wait() {
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N));
}

// Orders every use of v after the preceding lgkm_wait (both are volatile
// statements, which keep their order).
__device__ __forceinline__ void pin(u32x4_t &v) { asm volatile("" : "+v"(v)); }

// Output tile of workgroup `id` (of nx x ny): workgroups are dealt to the 8
// XCDs round-robin (id mod 8), so XCD k takes the k-th eighth of a grouped
// order -- 4 row tiles at a time, column by column -- and its workgroups share
// x rows and W columns in that XCD's L2 instead of each XCD fetching most of
// both.  A bijection for any nx, ny (without the XCD split when 8 does not
// divide the tile count).
__device__ __forceinline__ void xcd_tile_order(int nx, int ny, int id, int &tm, int &tn) {
    constexpr int G = 4;
    const int n = nx * ny;
    const int ord = (n % 8 == 0) ? (id % 8) * (n / 8) + id / 8 : id;
    const int group = ord / (G * nx);
    const int first = group * G;
    const int rows = min(G, ny - first);
    const int r = ord - first * nx;
    tm = first + r % rows;
    tn = r / rows;
}

// FS (split calls whose tiles leave CUs idle): the LoRA shrink runs inside
// this launch instead of a launch of its own, on the `shrink_wgs` workgroups
// after the tiles' contributors.  h is cut into units u = (bucket tile u / P,
// k part u % P), P = a.h_parts; the shrink workgroups take units round-robin,
// each an 8-wave shrink_role with agent-coherent h stores, and count the
// units they finished on sp.sync[0] once those stores are complete.  The
// consumers of h (the LoRA workgroups before their expand, else the last
// contributor of a tile before its tail expand) wait until the count reaches
// n_tiles x P, then read h with agent-coherent loads.  The wait is bounded: a
// consumer that does not see the count in time (only possible when the grid
// is not all resident at once) computes every unit itself with the same code
// -- the same h bits -- and goes on.  Every workgroup counts itself on
// sp.sync[1] when it is done with h; the last one resets both counters to 0
// for the next call.  Shrink workgroups never wait, so the grid drains in any
// residency.
constexpr int FS_U = 8;                 // k steps a shrink wave keeps in flight
constexpr int FS_SPIN_MAX = 1 << 17;    // polls of the unit count (~0.1-0.3 s)

template <int DT, int BN, bool SPLIT, bool FS = false>
__global__ __launch_bounds__(512) void k_gemm_lds(ApplyArgs a, SplitArgs sp) {
    static_assert(!FS || SPLIT, "the fused shrink serves split calls");
    using E = Elem<DT>;
    using V = typename E::vec8;
    constexpr int BM = 256;
    constexpr int WM = BN == 64 ? 4 : 2;  // waves along the rows
    constexpr int WN = 8 / WM;            // waves along the columns
    constexpr int TB = BM / 16 / WM;      // 16-row blocks per wave
    constexpr int WC = BN / 16 / WN;      // 16-column blocks per wave
    constexpr int RBU = 128;             // 16-byte units per row block (16 rows x 128 B)
    constexpr int BOFF = 16 * RBU;       // W row blocks follow the 16 x row blocks
    constexpr int NBW = BN / 16;         // W row blocks per stage
    constexpr int BLD = NBW / 2;         // W load instructions per W wave (4 waves)
    // Stage buffers: three at BN = 64 (two stages in flight while one is
    // multiplied, 120 KiB), two at BN = 256 (128 KiB).
    constexpr int NBUF = BN <= 128 ? 3 : 2;
    __shared__ u32x4_t lds0[(16 + NBW) * RBU];
    __shared__ u32x4_t lds1[(16 + NBW) * RBU];
    __shared__ u32x4_t lds2[NBUF == 3 ? (16 + NBW) * RBU : 1];
    // Output token of each sorted row of the tile (bitwise NOT of it for rows
    // of the invalid bucket), for the epilogue's stores.
    __shared__ int rowtok[SPLIT ? 1 : BM];
    __shared__ int last_split;
    __shared__ int h_late;

    const int wave = uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;
    const int g = lane >> 4;
    const int wm = wave / WN;  // rows wm * TB * 16
    const int wn = wave % WN;  // columns wn * WC * 16
    int tm, tn, z = 0, tile = 0;
    // Contributors per tile: the k splits, and the LoRA workgroup if the
    // plan has one (contributor 0 of the tile, numbered z = splits).
    const int nc = SPLIT ? sp.splits + sp.lora_wg : 1;
    bool lora_role = false;

    // Fused shrink (FS): this workgroup's units, then their count.
    auto produce = [&](int j, int np, u32x4_t *scratch) __attribute__((always_inline)) {
        const int P = uniform(a.h_parts);
        const int need = uniform(*a.rv.n_tiles) * P;
        int done = 0;
        for (int u = j; u < need; u += np) {
            const int t = u / P;
            shrink_role<DT, 4, 8, true, FS_U>(a, t, u - t * P, scratch);
            __syncthreads();  // wave 0's reads of the scratch are done before the next unit's writes
            ++done;
        }
        if (done > 0 && threadIdx.x == 0) {
            // (Thread 0 is in wave 0, which made the h stores.)
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __hip_atomic_fetch_add(sp.sync, static_cast<unsigned>(done), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
    };
    // Fused shrink: wait (bounded) until every unit is counted; past the
    // bound, compute them all here.  Every wave of the workgroup calls it.
    auto wait_h = [&](u32x4_t *scratch) __attribute__((always_inline)) {
        const int P = uniform(a.h_parts);
        const int need = uniform(*a.rv.n_tiles) * P;
        if (threadIdx.x == 0) {
            // (wait_polls 0: never wait, compute h here.)
            int spins = 0;
            bool short_count = sp.wait_polls == 0 ||
                               __hip_atomic_load(sp.sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                                   static_cast<unsigned>(need);
            while (short_count && spins < sp.wait_polls) {
                __builtin_amdgcn_s_sleep(2);
                ++spins;
                short_count = __hip_atomic_load(sp.sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                              static_cast<unsigned>(need);
            }
            h_late = short_count;
        }
        __syncthreads();
        if (uniform(h_late)) {
            for (int u = 0; u < need; ++u) {
                const int t = u / P;
                shrink_role<DT, 4, 8, true, FS_U>(a, t, u - t * P, scratch);
                __syncthreads();
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }
    };
    // Fused shrink: this workgroup is done with h (thread 0, once).
    auto depart = [&]() __attribute__((always_inline)) {
        if (threadIdx.x == 0) {
            const unsigned old =
                __hip_atomic_fetch_add(sp.sync + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (old == gridDim.x - 1) {
                __hip_atomic_store(sp.sync, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(sp.sync + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    };

    if constexpr (SPLIT) {
        // Workgroup id -> (tile, contributor): ids are dealt to the XCDs
        // round-robin (id mod 8), so when 8 divides the grid, XCD k takes the
        // k-th eighth of the (tile, contributor) sequence, in which a tile's
        // contributors follow one another.
        const int n = sp.tiles * nc;
        const int id = static_cast<int>(blockIdx.x);
        if constexpr (FS) {
            if (id >= n) {
                // A shrink workgroup (after the tiles' contributors).
                produce(id - n, sp.shrink_wgs, lds0);
                depart();
                return;
            }
        }
        const int q = uniform((n % 8 == 0) ? (id % 8) * (n / 8) + id / 8 : id);
        tile = uniform(q / nc);
        const int j = uniform(q - tile * nc);
        lora_role = sp.lora_wg && j == 0;
        z = lora_role ? sp.splits : j - sp.lora_wg;
        tm = tile / sp.tiles_x;
        tn = tile - tm * sp.tiles_x;
    } else {
        xcd_tile_order(gridDim.x, gridDim.y, blockIdx.x + gridDim.x * blockIdx.y, tm, tn);
    }
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int nst_all = a.d_in / 64;
    // The LoRA workgroup multiplies no k stage.
    const int s_beg = SPLIT ? (lora_role ? 0 : uniform(z * nst_all / sp.splits)) : 0;
    const int s_end = SPLIT ? (lora_role ? 0 : uniform((z + 1) * nst_all / sp.splits)) : nst_all;

    // Loads: wave w < 4 fetches x row blocks 4w .. 4w+3 (8 instructions),
    // wave w >= 4 W row blocks (BLD instructions); instruction i covers row
    // block (first + i/2), rows 8 (i&1) + lane/8, chunk (lane&7) ^ sw(row).
    // Buffer loads into LDS: the operand's resource in SGPRs, the stage's k
    // offset as the scalar offset, one 32-bit lane offset per instruction;
    // the row permutation is read once, in one batch.
    const bool xw = wave < 4;
    // Split calls (T < 2048, so a tile is often mostly past T): an x wave
    // whose 64 rows all lie past T loads nothing (its stage waits then have
    // nothing to wait for), and the waves computing those rows skip their
    // MFMAs (rows past T are never stored).  Not in the unsplit kernel: the
    // branch around its MFMAs makes the compiler spill the accumulators.
    const int nld = xw ? ((SPLIT && m0 + (wave & 3) * 64 >= a.T) ? 0 : 8) : BLD;
    const bool rows_live = !SPLIT || uniform(m0 + wm * TB * 16) < a.T;
    const __amdgpu_buffer_rsrc_t rs =
        xw ? make_rsrc(a.x, static_cast<uint32_t>(a.T) * a.d_in * 2)
           : make_rsrc(a.W, static_cast<uint32_t>(a.d_out) * a.d_in * 2);
    const int lrow = lane >> 3;  // row within the 8-row half
    const int rb0 = (wave & 3) * (xw ? 4 : BLD / 2);  // first row block this wave fills
    uint32_t off[8];
    int rowi[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) rowi[i] = (rb0 + (i >> 1)) * 16 + 8 * (i & 1) + lrow;  // row in tile
    if (xw) {
        int tok[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) tok[i] = a.rv.perm[min(m0 + rowi[i], a.T - 1)];
#pragma unroll
        for (int i = 0; i < 8; ++i) rowi[i] = min(max(tok[i], 0), a.T - 1);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) rowi[i] = min(n0 + rowi[i], a.d_out - 1);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int rho = 8 * (i & 1) + lrow;  // row within its block
        const int chunk = (lane & 7) ^ (rho & 7);
        off[i] = static_cast<uint32_t>(rowi[i]) * (a.d_in * 2) + chunk * 16;
    }
    const int ldsbase = (xw ? 0 : BOFF) + rb0 * RBU;
    auto issue = [&](int s, u32x4_t *buf) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i < nld)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)(buf + ldsbase + (i >> 1) * RBU + (i & 1) * 64),
                                                         16, off[i], s * 128, 0, 0);
    };

    // Operand reads: lane (r, g) of k step ks takes row r, chunk 4 ks + g,
    // stored at position (4 ks + g) ^ sw(r) of the row.
    const int sw = r & 7;
    const int lo0 = r * 8 + ((0 + g) ^ sw);
    const int lo1 = r * 8 + ((4 + g) ^ sw);

    f32x4_t acc[TB][WC];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int wc = 0; wc < WC; ++wc) acc[tb][wc] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // The operand reads are inline ds_read_b128, ordered after their own
    // lgkmcnt wait: the compiler then sees no LDS read that could alias the
    // buffer loads into LDS still in flight, and adds no wait for them of its
    // own (it would wait for every outstanding load -- the next stages' too).
    auto compute = [&](const u32x4_t *buf) {
        const uint32_t base = lds_offset(buf);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int lo = ks ? lo1 : lo0;
            const uint32_t xa = base + static_cast<uint32_t>((wm * TB) * RBU + lo) * 16;
            const uint32_t wa = base + static_cast<uint32_t>(BOFF + (wn * WC) * RBU + lo) * 16;
            // W fragments of the step, then x fragments two row blocks at a
            // time: the next pair's reads are issued before this pair's MFMAs.
            u32x4_t bq[WC], aq[TB];
#pragma unroll
            for (int wc = 0; wc < WC; ++wc) bq[wc] = ds_read16(wa + wc * RBU * 16);
            aq[0] = ds_read16(xa);
            aq[1] = ds_read16(xa + RBU * 16);
#pragma unroll
            for (int tp = 0; tp < TB; tp += 2) {
                lgkm_wait<0>();
                if (tp == 0) {
#pragma unroll
                    for (int wc = 0; wc < WC; ++wc) pin(bq[wc]);
                }
                pin(aq[tp]);
                pin(aq[tp + 1]);
                if (tp + 2 < TB) {
                    aq[tp + 2] = ds_read16(xa + (tp + 2) * RBU * 16);
                    aq[tp + 3] = ds_read16(xa + (tp + 3) * RBU * 16);
                }
#pragma unroll
                for (int tb = tp; tb < tp + 2; ++tb)
#pragma unroll
                    for (int wc = 0; wc < WC; ++wc)
                        acc[tb][wc] = E::mfma(__builtin_bit_cast(V, aq[tb]), __builtin_bit_cast(V, bq[wc]), acc[tb][wc]);
                // The pair's MFMAs are issued before the next wait.
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    // Waits for this wave's loads of the stage about to be multiplied (all
    // of them, or all but the next stage's when that one is in flight), then
    // for every wave's; the barrier also means that the buffer the next
    // issue writes is no longer read.
    auto sync_stage = [&](bool next_in_flight) {
        if (!next_in_flight) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        } else if (xw) {
            asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        } else {
            static_assert(BLD == 2 || BLD == 4 || BLD == 8, "W-wave load count");
            if (BLD == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
            else if (BLD == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
            else asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        }
        // A bare barrier: __syncthreads() adds a workgroup fence, for which
        // the compiler waits on every outstanding load, the next stage's too.
        // This wave's reads of the buffer the next issue overwrites returned
        // before its last MFMAs were issued.
        __builtin_amdgcn_s_barrier();
    };

    // SPLIT = false: the LoRA term s * h * B of the tile's FUSED rows is the
    // accumulators' starting value, computed while the first stage loads (the
    // main loop then adds x W^T to it; one rounding at the end either way).
    // Done here, the expand's registers are not live across the main loop.
    auto lora_prologue = [&]() {
        const int pw0 = m0 + wm * TB * 16;
        RowFacts<TB> f;
        row_facts<TB>(a, pw0, a.T, f);
        // Calls this large take one shrink part (tiled_h_parts).
        lora_expand_mfma<DT, TB, WC, 1>(a, pw0, a.T, n0 + wn * WC * 16, SEG_FUSED, f, acc);
        if (wn == 0 && g == 0) {
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
                rowtok[wm * TB * 16 + tb * 16 + r] = f.key[tb] == a.S + 1 ? ~f.tok[tb] : f.tok[tb];
        }
        __syncthreads();
    };

    const int nst = s_end - s_beg;
    if (nst == 0) {
        // (The LoRA workgroup of a split tile.)
        if constexpr (FS) wait_h(lds0);
    } else if (NBUF == 2) {
        issue(s_beg, lds0);
        if constexpr (!SPLIT) lora_prologue();
        for (int j = 0; j < nst; j += 2) {
            sync_stage(false);
            if (j + 1 < nst) issue(s_beg + j + 1, lds1);
            if (rows_live) compute(lds0);
            if (j + 1 < nst) {
                sync_stage(false);
                if (j + 2 < nst) issue(s_beg + j + 2, lds0);
                if (rows_live) compute(lds1);
            }
        }
    } else {
        issue(s_beg, lds0);
        if (nst > 1) issue(s_beg + 1, lds1);
        for (int j = 0; j < nst; j += 3) {
            sync_stage(j + 1 < nst);
            if (j + 2 < nst) issue(s_beg + j + 2, lds2);
            if (rows_live) compute(lds0);
            if (j + 1 >= nst) break;
            sync_stage(j + 2 < nst);
            if (j + 3 < nst) issue(s_beg + j + 3, lds0);
            if (rows_live) compute(lds1);
            if (j + 2 >= nst) break;
            sync_stage(j + 3 < nst);
            if (j + 4 < nst) issue(s_beg + j + 4, lds1);
            if (rows_live) compute(lds2);
        }
    }

    // The epilogue's addresses depend on pw, which the compiler may not
    // compute before the loop (keeps them from being hoisted and held in
    // registers across it).
    int pw = uniform(m0 + wm * TB * 16);
    asm volatile("" : "+s"(pw));
    const int nw = n0 + wn * WC * 16;
    if constexpr (!SPLIT) {
        static_assert(NBUF == 2, "the LoRA prologue runs in the two-buffer loop");
        store_rows_tok<DT, TB, WC>(a, pw, a.T, nw, rowtok + wm * TB * 16, acc);
    } else {
        // The tile's sum: this workgroup's own with one contributor;
        // otherwise the contributors' partial sums, added by the last one to
        // finish: the k splits in split order z = 0, 1, .., then the LoRA
        // workgroup's term if the plan has one (else the last contributor
        // adds the fused expand itself).
        f32x4_t sum[TB][WC];
        RowFacts<TB> f;
        if (lora_role && rows_live) {
            // The LoRA workgroup: the tile's fused expand, s * h . B^T, from
            // zero (its main loop took no k stage).
            row_facts<TB>(a, pw, a.T, f);
            lora_expand_mfma<DT, TB, WC, MAX_HPARTS, FS>(a, pw, a.T, nw, SEG_FUSED, f, acc);
        }
        if (nc == 1) {
            if constexpr (FS) wait_h(lds0);  // the tile's expand follows (no LoRA workgroup)
            if (!rows_live) return;  // (never wave 0, which departs at the end)
            row_facts_begin<TB>(a, pw, a.T, f);
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int wc = 0; wc < WC; ++wc) sum[tb][wc] = acc[tb][wc];
        } else {
            // This contributor's partial sums: wave w's TB x WC fragments at
            // [z][tile][w][tb][wc][lane], the waves whose rows all lie past T
            // left out (nobody reads them).
            constexpr uint32_t FRB = TB * WC * 64 * 16;  // bytes per wave
            const uint32_t zstride = static_cast<uint32_t>(sp.tiles) * 8 * FRB;
            const __amdgpu_buffer_rsrc_t prs = make_rsrc(sp.part, static_cast<uint32_t>(nc) * zstride);
            const uint32_t wbase = static_cast<uint32_t>(tile * 8 + wave) * FRB + lane * 16;
            if (rows_live) {
#pragma unroll
                for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                    for (int wc = 0; wc < WC; ++wc)
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, acc[tb][wc]), prs,
                                                               wbase + (tb * WC + wc) * 1024, z * zstride, CPOL_SC1);
            }
            // The stores are complete (at the agent's coherence point) before
            // the contributor is counted.
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (threadIdx.x == 0) {
                const unsigned old =
                    __hip_atomic_fetch_add(sp.cnt + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const int last = old == static_cast<unsigned>(nc - 1);
                if (last) __hip_atomic_store(sp.cnt + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                last_split = last;
            }
            __syncthreads();
            if constexpr (FS) {
                if (!uniform(last_split)) depart();
                else if (!sp.lora_wg) wait_h(lds0);
            }
            if (!last_split || !rows_live) return;
            // The last contributor of the tile: the rows' routing facts and
            // the other contributors' fragments requested together, NZ a
            // round, then the sum in order (its own from registers).
            if (!lora_role) row_facts_begin<TB>(a, pw, a.T, f);
            constexpr int NZ = 2;
#pragma unroll
            for (int zb = 0; zb < MAX_TSPLIT + 1; zb += NZ) {
                if (zb >= nc) break;
                f32x4_t v[NZ][TB][WC];
#pragma unroll
                for (int jz = 0; jz < NZ; ++jz) {
                    const int zz = zb + jz;
                    if (zz < nc && zz != z) {
#pragma unroll
                        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                            for (int wc = 0; wc < WC; ++wc)
                                v[jz][tb][wc] = __builtin_bit_cast(
                                    f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                 prs, wbase + (tb * WC + wc) * 1024, zz * zstride, CPOL_SC1));
                    }
                }
#pragma unroll
                for (int jz = 0; jz < NZ; ++jz) {
                    const int zz = zb + jz;
                    if (zz < nc) {
#pragma unroll
                        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                            for (int wc = 0; wc < WC; ++wc) {
                                const f32x4_t u = zz == z ? acc[tb][wc] : v[jz][tb][wc];
                                sum[tb][wc] = zz == 0 ? u : sum[tb][wc] + u;
                            }
                    }
                }
            }
        }
        if (!lora_role) row_facts_end<TB>(a, pw, a.T, f);
        if (!sp.lora_wg) lora_expand_mfma<DT, TB, WC, MAX_HPARTS, FS>(a, pw, a.T, nw, SEG_FUSED, f, sum);
        store_rows<DT, TB, WC>(a, pw, a.T, nw, f, sum);
        if constexpr (FS) depart();
    }
}

template <int DT, int BM, int BN>
hipError_t launch_shape(const ApplyArgs &a, hipStream_t st, LaunchEvents ev) {
    const dim3 grid(a.d_out / BN, (a.T + BM - 1) / BM);
    LORA_LAUNCH(ev, (k_gemm_tiled<DT, BM, BN>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const ApplyArgs &a, const SplitSpace &ws, hipStream_t st, LaunchEvents ev) {
    // One kernel per call: the completion event, when asked for, is that
    // kernel's stop event (callers that time the kernel record it themselves).
    if (ev.done != nullptr && ev.stop == nullptr) ev.stop = ev.done;
    if (a.T >= 2048 && a.d_out % 256 == 0 && a.d_in % 128 == 0) {
        const dim3 grid(a.d_out / 256, (a.T + 255) / 256);
        LORA_LAUNCH(ev, (k_gemm_lds<DT, 256, false>), grid, dim3(512), 0, st, a, SplitArgs{});
        return hipGetLastError();
    }
    const TiledPlan tp = tiled_plan(a.T, a.d_in, a.d_out);
    if (tp.splits > 0) {
        SplitArgs sp{};
        sp.splits = tp.splits;
        sp.lora_wg = tp.lora_wg;
        sp.tiles_x = a.d_out / tp.bn;
        sp.tiles = sp.tiles_x * ((a.T + 255) / 256);
        sp.part = ws.part;
        sp.cnt = ws.cnt;
        sp.shrink_wgs = tp.shrink_wgs;
        sp.sync = ws.sync;
        sp.wait_polls = ws.wait_polls < 0 ? FS_SPIN_MAX : ws.wait_polls;
        // The workspace was sized with tiled_part_bytes / tiled_split_tiles.
        const int nc = tp.splits + tp.lora_wg;
        if (nc > 1 && (ws.part == nullptr || ws.cnt == nullptr || sp.tiles > ws.max_tiles))
            return hipErrorInvalidValue;
        if (tp.bn != 64 || tp.splits > MAX_TSPLIT || tp.lora_wg > 1) return hipErrorInvalidValue;
        if (tp.fuse_parts > 0) {
            // The caller set h_parts to the plan's and launched no shrink.
            if (ws.sync == nullptr || tp.shrink_wgs <= 0 || a.h_parts != tp.fuse_parts ||
                a.shrink_parts != tp.fuse_parts || a.h_by_token != 0 || a.R > 64)
                return hipErrorInvalidValue;
            const dim3 grid(sp.tiles * nc + tp.shrink_wgs);
            LORA_LAUNCH(ev, (k_gemm_lds<DT, 64, true, true>), grid, dim3(512), 0, st, a, sp);
            return hipGetLastError();
        }
        const dim3 grid(sp.tiles * nc);
        LORA_LAUNCH(ev, (k_gemm_lds<DT, 64, true>), grid, dim3(512), 0, st, a, sp);
        return hipGetLastError();
    }
    if (a.T >= 512 && a.d_out % 128 == 0) return launch_shape<DT, 128, 128>(a, st, ev);
    return launch_shape<DT, 64, 64>(a, st, ev);
}

}  // namespace

TiledPlan tiled_plan(int T, int d_in, int d_out) {
    // Calls of 65 .. 2047 tokens with d_in a multiple of 128 and d_out of 64:
    // 256 x 64 tiles, k split `splits` ways, plus (lora_wg = 1) a LoRA
    // workgroup per tile that computes the fused expand beside the splits.
    // The choice minimises a rough time model of one launch (per-CU rates
    // measured on MI355X, rounded down): a workgroup streams its x rows and W
    // rows through LDS at ~100 GB/s and multiplies at ~60% of a CU's MFMA
    // peak; W streams from HBM at ~5 TB/s; with more than one contributor
    // the fp32 partial sums make a round trip at ~5 TB/s and the last
    // contributor reads the others' at ~100 GB/s; without a LoRA workgroup
    // the last contributor's expand adds ~6 us (a few rounds of dependent
    // loads).  A grid of more than 256 workgroups (one per CU) pays a round
    // per 256; LoRA workgroups are taken only when the grid stays within one
    // round.  (The same model prefers 64- over 128-column tiles at every T
    // here: the wider tile needs more splits for the same grid.)  splits 0:
    // not this path.
    if (T <= DECODE_MAX_T || T >= 2048 || d_out % 64 != 0 || d_in % 128 != 0) return TiledPlan{0, 0, 0, 0, 0};
    const int bn = 64;
    const int row_tiles = (T + 255) / 256;
    const double rows = T < 256 ? static_cast<double>((T + 63) / 64 * 64) : 256.0;  // x rows a tile loads
    const int nst = d_in / 64;
    const double w_s = static_cast<double>(d_in) * d_out * 2 / 5e12;
    const double cu_mfma = 2.5e15 / 256 * 0.6;
    const int tiles = d_out / bn * row_tiles;
    TiledPlan best{0, 0, 0, 0, 0};
    double best_t = 0.0;
    int best_wgs = 0;
    for (int s = 1; s <= MAX_TSPLIT; ++s) {
        if (s > 1 && nst / s < 4) break;
        for (int lw = 0; lw <= 1; ++lw) {
            const int nc = s + lw;
            if (nc > 1 && (tiles > MAX_SPLIT_TILES ||
                           static_cast<double>(nc) * tiles * 256 * bn * 4 >= 4294967296.0))
                continue;
            if (lw && tiles * nc > 256) continue;
            const int rounds = (tiles * s + 255) / 256;
            const int kst = (nst + s - 1) / s;
            const double ingest = rounds * (rows + bn) * kst * 128 / 100e9;
            const double mfma = rounds * rows * bn * kst * 64 * 2 / cu_mfma;
            double t = std::max(std::max(ingest, mfma), w_s);
            if (nc > 1) {
                t += 2.0 * nc * tiles * rows * bn * 4 / 5e12;
                t += (nc - 1) * rows * bn * 4 / 100e9;
            }
            if (!lw) t += 6e-6;
            // Plans within 1% of each other are a tie for this model (where W
            // streaming bounds both): the one with more workgroups wins, its
            // W requests spread over more CUs (128 tokens on 4096 x 4096:
            // 3 splits + LoRA workgroup, 22.0 us, against 2 + 1, 23.9 us).
            const int wgs = tiles * nc;
            const bool better = best.splits == 0 || (wgs > best_wgs ? t <= best_t * 1.01 : t < best_t * 0.99) ||
                                (wgs == best_wgs && t < best_t);
            if (better) {
                best = TiledPlan{bn, s, lw, 0, 0};
                best_t = t;
                best_wgs = wgs;
            }
        }
    }
    // The shrink joins the launch on the CUs the tiles leave idle (at least
    // 64): its k parts give each shrink wave at most FS_U k steps (one round
    // of loads).  With every CU taken by a tile, the shrink stays a launch of
    // its own: measured on MI355X, shrink units in the tile workgroups'
    // prologues delayed their main loops and the LoRA workgroups' expand by
    // more than the launch they saved (256 tokens, 4096 x 4096: GEMM 27 ->
    // 39 us, call 38.2 -> 43.6 us).
    const int wgs = tiles * (best.splits + best.lora_wg);
    if (best.splits > 0 && 256 - wgs >= 64) {
        best.fuse_parts = std::min(MAX_HPARTS, std::max(1, (d_in / 32 + 8 * FS_U - 1) / (8 * FS_U)));
        best.shrink_wgs = 256 - wgs;
    }
    return best;
}

int tiled_call_h_parts(int T, int d_in, int d_out, int R, int tiles) {
    const TiledPlan tp = tiled_plan(T, d_in, d_out);
    return tp.fuse_parts > 0 ? tp.fuse_parts : tiled_h_parts(d_in, R, tiles, T);
}

size_t tiled_part_bytes(int T, int d_in, int d_out) {
    const TiledPlan tp = tiled_plan(T, d_in, d_out);
    const int nc = tp.splits + tp.lora_wg;
    if (nc <= 1) return 0;
    return static_cast<size_t>(nc) * (d_out / tp.bn) * ((T + 255) / 256) * 256 * tp.bn * 4;
}

int tiled_split_tiles(int T, int d_in, int d_out) {
    const TiledPlan tp = tiled_plan(T, d_in, d_out);
    if (tp.splits + tp.lora_wg <= 1) return 0;
    return (d_out / tp.bn) * ((T + 255) / 256);
}

hipError_t launch_gemm_tiled(const ApplyArgs &a, const SplitSpace &ws, hipStream_t st, LaunchEvents ev) {
    return (a.dtype == DT_F16) ? launch_dt<DT_F16>(a, ws, st, ev) : launch_dt<DT_BF16>(a, ws, st, ev);
}

}  // namespace lora
