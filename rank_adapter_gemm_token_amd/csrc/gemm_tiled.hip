// gemm_tiled.hip -- base projection for calls of more than 64 tokens
// (fp16/bf16) with the fused LoRA term.  Three kernels:
//   * k_gemm_lds<256> (>= 2048 tokens): 256 x 256 tiles staged into LDS by
//     direct loads, the LoRA term computed into the accumulators before the
//     main loop (described at its definition);
//   * k_gemm_lds<128, split> + k_split_epilogue (65 .. 2047 tokens): the same
//     staging over k ranges, fp32 partial sums, then sum + fused expand;
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

// 256-row tiles, operands straight into LDS.  A workgroup of 8 waves (2 x
// 4) computes a 256 x BN output tile (BN = 256: each wave 128 rows x 64
// columns; BN = 128: 128 x 32) over a range of k stages.  A 64-wide k stage
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
// the chip): workgroup z of the grid's third dimension takes the z-th of
// gridDim.z k ranges and stores fp32 partial sums in MFMA fragment order;
// k_split_epilogue adds them.
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

template <int DT, int BN, bool SPLIT>
__global__ __launch_bounds__(512) void k_gemm_lds(ApplyArgs a, float *part) {
    using E = Elem<DT>;
    using V = typename E::vec8;
    constexpr int BM = 256, TB = 8, WC = BN / 64;
    constexpr int RBU = 128;             // 16-byte units per row block (16 rows x 128 B)
    constexpr int BOFF = 16 * RBU;       // W row blocks follow the 16 x row blocks
    constexpr int NBW = BN / 16;         // W row blocks per stage
    constexpr int BLD = NBW / 2;         // W load instructions per W wave (4 waves)
    // Stage buffers: three at BN = 128 (two stages in flight while one is
    // multiplied, 144 KiB), two at BN = 256 (128 KiB).
    constexpr int NBUF = BN == 128 ? 3 : 2;
    __shared__ u32x4_t lds0[(16 + NBW) * RBU];
    __shared__ u32x4_t lds1[(16 + NBW) * RBU];
    __shared__ u32x4_t lds2[NBUF == 3 ? (16 + NBW) * RBU : 1];
    // Output token of each sorted row of the tile (bitwise NOT of it for rows
    // of the invalid bucket), for the epilogue's stores.
    __shared__ int rowtok[SPLIT ? 1 : BM];

    const int wave = uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;
    const int g = lane >> 4;
    const int wm = wave >> 2;  // rows wm * 128
    const int wn = wave & 3;   // columns wn * BN / 4
    int tm = blockIdx.y, tn = blockIdx.x;
    if (!SPLIT) xcd_tile_order(gridDim.x, gridDim.y, blockIdx.x + gridDim.x * blockIdx.y, tm, tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int nst_all = a.d_in / 64;
    const int s_beg = SPLIT ? uniform(static_cast<int>(blockIdx.z) * nst_all / static_cast<int>(gridDim.z)) : 0;
    const int s_end = SPLIT ? uniform((static_cast<int>(blockIdx.z) + 1) * nst_all / static_cast<int>(gridDim.z))
                            : nst_all;

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
    const bool rows_live = !SPLIT || m0 + wm * TB * 16 < a.T;
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
            static_assert(BLD == 4 || BLD == 8, "W-wave load count");
            if (BLD == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
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
    if (NBUF == 2) {
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
    int pw = m0 + wm * TB * 16;
    asm volatile("" : "+s"(pw));
    const int nw = n0 + wn * WC * 16;
    if constexpr (!SPLIT) {
        static_assert(NBUF == 2, "the LoRA prologue runs in the two-buffer loop");
        store_rows_tok<DT, TB, WC>(a, pw, a.T, nw, rowtok + wm * TB * 16, acc);
    } else {
        // Partial sums [z][16-row block][16-column block][lane], row blocks
        // of sorted rows below T only; streaming stores (read once, by the
        // split epilogue).
        const int nrb = (a.T + 15) / 16, ncb = a.d_out / 16;
        f32x4_t *pz = reinterpret_cast<f32x4_t *>(part) + static_cast<size_t>(blockIdx.z) * nrb * ncb * 64;
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const int rb = pw / 16 + tb;
            if (rb < nrb) {
#pragma unroll
                for (int wc = 0; wc < WC; ++wc)
                    __builtin_nontemporal_store(acc[tb][wc], &pz[(static_cast<size_t>(rb) * ncb + nw / 16 + wc) * 64 + lane]);
            }
        }
    }
}

// Split sums of k_gemm_lds<.., true>: workgroup of 4 waves over 64 sorted rows
// x 16 WC columns, wave w = rows (4 blockIdx.y + w) * 16 .. +15.  Adds the
// splits' partial sums in a fixed order, then the fused expand and the
// scatter to token order, as the unsplit kernel's epilogue does.  WC = 2 for
// calls of at most 256 tokens (twice the waves in flight for the same work),
// else 4.
template <int DT, int WC>
__global__ __launch_bounds__(256) void k_split_epilogue(ApplyArgs a, const float *part, int splits) {
    const int wave = uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int rb = static_cast<int>(blockIdx.y) * 4 + wave;
    const int nrb = (a.T + 15) / 16, ncb = a.d_out / 16;
    if (rb >= nrb) return;
    const int cb0 = static_cast<int>(blockIdx.x) * WC;
    const f32x4_t *p = reinterpret_cast<const f32x4_t *>(part) + (static_cast<size_t>(rb) * ncb + cb0) * 64 + lane;
    const size_t zs = static_cast<size_t>(nrb) * ncb * 64;
    // Everything that does not depend on the routing facts is requested
    // before them, behind their first round: the rows' buckets and tokens,
    // then every split's partials (split index clamped, repeats not added, so
    // the wait counts stay exact) and the rows' h.
    RowFacts<1> f;
    row_facts_begin<1>(a, rb * 16, a.T, f);
    f32x4_t v[MAX_TSPLIT][WC];
#pragma unroll
    for (int z = 0; z < MAX_TSPLIT; ++z)
#pragma unroll
        for (int wc = 0; wc < WC; ++wc) v[z][wc] = p[min(z, splits - 1) * zs + wc * 64];
    float hpre[2][8];
    prefetch_h1(a, rb * 16, a.T, hpre);
    row_facts_end<1>(a, rb * 16, a.T, f);
    f32x4_t acc[1][WC];
#pragma unroll
    for (int wc = 0; wc < WC; ++wc) {
        acc[0][wc] = v[0][wc];
#pragma unroll
        for (int z = 1; z < MAX_TSPLIT; ++z)
            if (z < splits) acc[0][wc] += v[z][wc];
    }
    lora_expand_mfma<DT, 1, WC>(a, rb * 16, a.T, cb0 * 16, SEG_FUSED, f, acc, hpre);
    store_rows<DT, 1, WC>(a, rb * 16, a.T, cb0 * 16, f, acc);
}

template <int DT, int BM, int BN>
hipError_t launch_shape(const ApplyArgs &a, hipStream_t st, LaunchEvents ev) {
    const dim3 grid(a.d_out / BN, (a.T + BM - 1) / BM);
    LORA_LAUNCH(ev, (k_gemm_tiled<DT, BM, BN>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const ApplyArgs &a, float *part, hipStream_t st, LaunchEvents ev) {
    if (a.T >= 2048 && a.d_out % 256 == 0 && a.d_in % 128 == 0) {
        const dim3 grid(a.d_out / 256, (a.T + 255) / 256);
        LORA_LAUNCH(ev, (k_gemm_lds<DT, 256, false>), grid, dim3(512), 0, st, a, nullptr);
        return hipGetLastError();
    }
    const int splits = tiled_splits(a.T, a.d_in, a.d_out);
    if (splits > 0) {
        const dim3 grid(a.d_out / 128, (a.T + 255) / 256, splits);
        LORA_LAUNCH(ev, (k_gemm_lds<DT, 128, true>), grid, dim3(512), 0, st, a, part);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (a.T <= 256) {
            const dim3 egrid(a.d_out / 32, (a.T + 63) / 64);
            hipLaunchKernelGGL((k_split_epilogue<DT, 2>), egrid, dim3(256), 0, st, a, part, splits);
        } else {
            const dim3 egrid(a.d_out / 64, (a.T + 63) / 64);
            hipLaunchKernelGGL((k_split_epilogue<DT, 4>), egrid, dim3(256), 0, st, a, part, splits);
        }
        return hipGetLastError();
    }
    if (a.T >= 512 && a.d_out % 128 == 0) return launch_shape<DT, 128, 128>(a, st, ev);
    return launch_shape<DT, 64, 64>(a, st, ev);
}

}  // namespace

int tiled_splits(int T, int d_in, int d_out) {
    // Split-K for calls of 65 .. 2047 tokens: 256 x 128 tiles, the smallest
    // power-of-two split (<= MAX_TSPLIT) that gives >= 256 workgroups with
    // at least 4 k stages each; 0 when the shape does not fit the kernel
    // (then the register-staged tiles run unsplit).
    if (T <= DECODE_MAX_T || T >= 2048 || d_out % 128 != 0 || d_in % 128 != 0) return 0;
    const int tiles = (d_out / 128) * ((T + 255) / 256);
    int s = 1;
    while (s < MAX_TSPLIT && tiles * s < 256 && d_in / 64 >= 8 * s) s *= 2;
    return s;
}

hipError_t launch_gemm_tiled(const ApplyArgs &a, float *part, hipStream_t st, LaunchEvents ev) {
    return (a.dtype == DT_F16) ? launch_dt<DT_F16>(a, part, st, ev) : launch_dt<DT_BF16>(a, part, st, ev);
}

}  // namespace lora
