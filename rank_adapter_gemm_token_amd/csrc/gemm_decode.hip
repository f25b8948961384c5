// gemm_decode.hip -- the decode path (T <= 64 tokens per call, fp16/bf16):
// base projection, LoRA shrink, routing and the fused LoRA expand in two
// launches.
//
// At decode sizes a call is bound by streaming W (d_out x d_in, read once)
// from HBM.  The next cost is x: every output column needs all of x, so a
// layout in which each CU covers a few columns over the whole of d_in reads
// x from L2 once per CU (128 MiB at d_in = 4096, T = 64, 256 CUs).  Here a
// workgroup covers 64 columns over one k split of d_in (x traffic / 4), and
// the splits' fp32 partial sums are added by a second, small kernel, which
// also routes the tokens and applies the LoRA term.  Nothing in the first
// kernel waits for routing:
//
// k_decode_gemm -- workgroup (column group c of 64 columns, k split q), 4
//   waves (one per SIMD, 512 registers each); wave w takes the split's k
//   step pairs p = w, w+4, w+8, w+12 (64 k each) for all 64 columns and all
//   T rows.
//   * Operands go from global memory straight into LDS (buffer_load ... lds),
//     one instruction per 8 rows with 8 lanes covering each row's 128-byte
//     line, into a per-wave ring of 2-4 pair slots (up to 160 KiB); the
//     MFMA operands are read back from XOR-swizzled rows without bank
//     conflicts.  Each wave waits only for its own loads (no barrier in the
//     loop).  The A rows of slot c are requested first, into registers
//     (before the token indices are known -- a slot is named by few tokens
//     if any).
//   * GEMM: fp32 MFMA accumulators over the wave's pairs; the 4 waves' sums
//     are added in LDS in a fixed order and stored as the split's partial
//     sums in MFMA fragment order (16 bytes a lane, coalesced).
//   * Shrink: in the same loop, this split's part of h = x . A_c^T for all T
//     rows, rows of slot c's tokens kept (fp32, by token, part q); slots c +
//     groups, ... (pools with more slots than column groups) read x again.
// k_decode_epilogue -- one 16-column block per workgroup, thread (row block,
//   lane) = 4 rows of one column.  The splits' partial sums and the h parts
//   are requested first; meanwhile wave 0 routes the (at most 64) tokens in
//   LDS (each token's sorted position by comparing keys, then buckets,
//   modes and tiles from ballots -- the same stable order as the routing
//   kernel of larger calls) and workgroup 0 publishes the routing.  Then it
//   adds the parts in a fixed order, adds s * h . B for FUSED buckets (fp32
//   VALU), rounds once and stores; invalid tokens get NaN.  SEPARATE rows
//   keep the rounded base for the residual kernel.
//
// The fused/separate choice of "LLM 多 LoRA 推理服务工程 2026" (four-layer runtime,
// execution-unit paragraph) maps to: FUSED = the LoRA term enters the fp32
// accumulator before the single rounding; SEPARATE = the base is rounded and
// stored, and the residual kernel adds the LoRA term to y afterwards.
// The variant (TB, splits) depends on (T, d_in) only, so a token's result
// never depends on the rest of the batch.
#include "epilogue.hpp"

namespace lora {

namespace {

constexpr int NWK = 4;               // waves per workgroup (one per SIMD)
constexpr int DCB = 4;               // 16-column blocks per GEMM workgroup
constexpr int DCOLS = DCB * 16;      // columns per GEMM workgroup
constexpr int DPAIRS_PER_WAVE = 4;   // k step pairs per GEMM wave
constexpr int SMAX_SEG = DECODE_MAX_T + 2;

// ------------------------------------------------------ small-call routing --

// Orders one wave's LDS accesses: earlier writes are complete and visible to
// the wave's later reads, and the compiler moves no memory access across it.
__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// The routing of one call of T <= 64 tokens, in LDS.
struct SmallRoute {
    int perm[DECODE_MAX_T];     // sorted position -> token
    int pos_seg[DECODE_MAX_T];  // sorted position -> bucket record
    int tok_pos[DECODE_MAX_T];  // token -> sorted position
    int tok_seg[DECODE_MAX_T];  // token -> bucket record
    alignas(16) int key[DECODE_MAX_T];  // token -> key (lanes >= T: past every key)
    int rank[DECODE_MAX_T];     // token -> true rank (LoRA tokens)
    int segs[SMAX_SEG][4];      // {key, start, len, mode}
    int tiles[DECODE_MAX_T + SMAX_SEG][2];  // {bucket | rank << 16 (tile_pack), first row}
    int n_seg;
    int n_lora;                 // LoRA buckets (records 0 .. n_lora-1)
    int n_tiles;
    int stat[6];                // fused, separate, base_only, invalid, rows padded, rows true
};

// One wave: key = slot (active), S (base_only) or S + 1 (invalid) of the
// token of each lane (lanes >= T: S + 2, after every token), then each
// token's sorted position = #(smaller keys) + #(same key, smaller index),
// counted from one ballot per key bit; buckets, modes, tiles and statistics
// from ballots.  `v` is the lane's adapter index and `state`, `rank` the
// entry of slot v (any values when v is not a slot).
__device__ __forceinline__ void small_route(int v, int state, int rank_in, int T, int S, int max_rank, int policy,
                                            int theta, SmallRoute &sr) {
    const int lane = threadIdx.x & 63;
    const bool tv = lane < T;
    int key = S, rank = 0;
    if (v != -1) {
        key = S + 1;
        if (v >= 0 && v < S && state == SLOT_ACTIVE) {
            key = v;
            rank = rank_in;
        }
    }
    if (!tv) key = S + 2;
    sr.key[lane] = key;
    sr.rank[lane] = rank;
    // Rank by key, most significant bit first: `eq` holds the lanes whose
    // key agrees with this lane's on the bits seen so far.
    const int nbits = 32 - __clz(S + 2);
    unsigned long long eq = ~0ull;
    int pos = 0;
    for (int b = nbits - 1; b >= 0; --b) {
        const unsigned long long m = __ballot((key >> b) & 1);
        if ((key >> b) & 1) {
            pos += __popcll(eq & ~m);
            eq &= m;
        } else {
            eq &= ~m;
        }
    }
    pos += __popcll(eq & ((1ull << lane) - 1ull));
    lds_fence();
    if (tv) sr.perm[pos] = lane;
    lds_fence();
    // Lane p: the token at sorted position p.
    const int p = lane;
    const bool pv = p < T;
    const int ptok = pv ? sr.perm[p] : 0;
    const int pkey = pv ? sr.key[ptok] : S + 2;
    const int prev = (p > 0 && pv) ? sr.key[sr.perm[p - 1]] : -1;
    const bool start = pv && prev != pkey;
    const unsigned long long starts = __ballot(start);
    const unsigned long long upto = (p == 63) ? ~0ull : ((2ull << p) - 1ull);
    const int seg = __popcll(starts & upto) - 1;
    const unsigned long long later = starts & ~upto;
    const int next = later ? __ffsll(static_cast<long long>(later)) - 1 : T;
    const int len = next - p;  // meaningful at start lanes
    const bool lora = start && pkey < S;
    int mode = 0;
    if (lora) mode = (policy == 1) ? 1 : (policy == 2) ? 2 : (len > theta ? 1 : 2);
    // Tiles of LoRA buckets: exclusive prefix of ceil(len / 16) (1..4) over
    // start lanes, from one ballot per bit.
    const int nt = lora ? (len + TILE_ROWS - 1) / TILE_ROWS : 0;
    const unsigned long long below = upto >> 1;  // lanes < p
    int tile0 = 0, n_tiles = 0;
#pragma unroll
    for (int b = 0; b < 3; ++b) {
        const unsigned long long m = __ballot((nt >> b) & 1);
        tile0 += __popcll(m & below) << b;
        n_tiles += __popcll(m) << b;
    }
    if (pv) {
        sr.pos_seg[p] = seg;
        sr.tok_pos[ptok] = p;
        sr.tok_seg[ptok] = seg;
    }
    if (start) {
        sr.segs[seg][0] = pkey;
        sr.segs[seg][1] = p;
        sr.segs[seg][2] = len;
        sr.segs[seg][3] = mode;
        for (int j = 0; j < nt; ++j) {
            sr.tiles[tile0 + j][0] = tile_pack(seg, sr.rank[ptok]);
            sr.tiles[tile0 + j][1] = p + j * TILE_ROWS;
        }
    }
    // Statistics from ballots over tokens (sorted lanes) and bucket starts
    // (every lane takes part in each ballot).
    const bool lt = pv && pkey < S;
    const int prank = sr.rank[ptok];
    int rows_true = 0;
#pragma unroll
    for (int b = 0; b < 7; ++b) rows_true += __popcll(__ballot(lt && ((prank >> b) & 1))) << b;
    const int n_lora = __popcll(__ballot(lora));
    const int st0 = __popcll(__ballot(mode == 1));
    const int st1 = __popcll(__ballot(mode == 2));
    const int st2 = __popcll(__ballot(pv && pkey == S));
    const int st3 = __popcll(__ballot(pv && pkey == S + 1));
    const int n_lt = __popcll(__ballot(lt));
    if (lane == 0) {
        sr.n_seg = __popcll(starts);
        sr.n_lora = n_lora;
        sr.n_tiles = n_tiles;
        sr.stat[0] = st0;
        sr.stat[1] = st1;
        sr.stat[2] = st2;
        sr.stat[3] = st3;
        sr.stat[4] = n_lt * max_rank;
        sr.stat[5] = rows_true;
    }
}

// The routing wave of workgroup 0: publish the routing for the residual
// kernel and the caller, the statistics and the invalid-token count.
__device__ __forceinline__ void publish_route(const SmallRoute &sr, int T, const RouteOut &out) {
    const int lane = threadIdx.x & 63;
    if (lane < T) {
        out.perm[lane] = sr.perm[lane];
        out.pos_seg[lane] = sr.pos_seg[lane];
        out.tok_pos[lane] = sr.tok_pos[lane];
        out.tok_seg[lane] = sr.tok_seg[lane];
    }
    for (int i = lane; i < 4 * sr.n_seg; i += 64) out.segs[i] = sr.segs[i >> 2][i & 3];
    for (int i = lane; i < 2 * sr.n_tiles; i += 64) out.tiles[i] = sr.tiles[i >> 1][i & 1];
    if (lane == 0) {
        *out.n_seg = sr.n_seg;
        *out.n_tiles = sr.n_tiles;
        DevStats st;
        st.tokens = T;
        st.lora_buckets = sr.stat[0] + sr.stat[1];
        st.fused_buckets = sr.stat[0];
        st.separate_buckets = sr.stat[1];
        st.base_only_tokens = sr.stat[2];
        st.invalid_tokens = sr.stat[3];
        st.rows_padded = sr.stat[4];
        st.rows_true = sr.stat[5];
        if (out.stats) *out.stats = st;
        if (out.err && sr.stat[3] > 0) atomicAdd(out.err, static_cast<unsigned long long>(sr.stat[3]));
    }
}

// Routing alone of a call of 1 .. 64 tokens (lora_route on an fp16/bf16
// pool): the small_route that the decode epilogue runs, published the same
// way, plus the per-key counts and offsets the epilogue has no use for.  One
// wave.  A key's count is the length of its bucket (0 without one); its
// offset is where the first bucket of a key not below it starts (T past the
// last), i.e. the exclusive prefix sum of the counts.
__global__ __launch_bounds__(64) void k_route_small(const int32_t *__restrict__ idx, int T, int S,
                                                    const SlotDev *__restrict__ slots, int max_rank, int policy,
                                                    int theta, RouteOut out) {
    __shared__ SmallRoute sr;
    const int lane = threadIdx.x & 63;
    const int v = lane < T ? idx[lane] : -1;
    const int2 e = reinterpret_cast<const int2 *>(slots)[2 * min(max(v, 0), S - 1)];
    small_route(v, e.x, e.y, T, S, max_rank, policy, theta, sr);
    lds_fence();
    publish_route(sr, T, out);
    const int ns = sr.n_seg;
    for (int k = lane; k < S + 3; k += 64) {
        int lo = 0, hi = ns;  // first record whose key is >= k
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (sr.segs[mid][0] < k) lo = mid + 1;
            else hi = mid;
        }
        out.offsets[k] = lo < ns ? sr.segs[lo][1] : T;
        if (k < S + 2) out.counts[k] = (lo < ns && sr.segs[lo][0] == k) ? sr.segs[lo][2] : 0;
    }
}

// ------------------------------------------------------------------ GEMM --

using lds_ptr = __attribute__((address_space(3))) void *;

// Cache policy of the W loads: non-temporal.  W is read once per call;
// streamed through L2 with the default policy it evicts the x tile that
// every column group of a split reads.
constexpr int CPOL_NT = 2;

// Waits until at most N vector-memory operations of this wave are
// outstanding (they complete in order), and keeps the compiler from moving
// memory accesses across the wait.
template <int N>
__device__ __forceinline__ void vm_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Waits until at most later * L + extra loads are outstanding (later <= 3;
// the branches fold away when the arguments are constants).
template <int L>
__device__ __forceinline__ void wait_loads(int later, int extra) {
    static_assert(3 * L + 1 < 64, "vmcnt is 6 bits");
    if (later == 0) {
        if (extra) vm_wait<1>(); else vm_wait<0>();
    } else if (later == 1) {
        if (extra) vm_wait<L + 1>(); else vm_wait<L>();
    } else if (later == 2) {
        if (extra) vm_wait<2 * L + 1>(); else vm_wait<2 * L>();
    } else {
        if (extra) vm_wait<3 * L + 1>(); else vm_wait<3 * L>();
    }
}

// One step pair into a ring slot: nx x-row instructions then W-row ones up
// to nl, instruction g filling the slot's 16-byte units 64 g .. 64 g + 63.
__device__ __forceinline__ void issue_pair(const __amdgpu_buffer_rsrc_t &xrs, const __amdgpu_buffer_rsrc_t &wrs,
                                           u32x4_t *slot, const uint32_t *loff, int nx, int nl, uint32_t soff) {
#pragma unroll
    for (int g = 0; g < nx; ++g)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (lds_ptr)(slot + g * 64), 16, loff[g], soff, 0, 0);
#pragma unroll
    for (int g = nx; g < nl; ++g)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (lds_ptr)(slot + g * 64), 16, loff[g], soff, 0, CPOL_NT);
    __builtin_amdgcn_sched_barrier(0);
}

// Ring slots per wave for TB token blocks: a slot holds one step pair of x
// (16 TB rows) and W (64 rows), 128 bytes a row; the ring of the 4 waves
// stays within the 160 KiB of LDS.
template <int TB>
struct DecRing {
    static constexpr int XROWS = TB * 16;
    static constexpr int UNITS = (XROWS + DCOLS) * 8;          // 16-byte units per slot
    static constexpr int LOADS = (XROWS + DCOLS) / 8;          // load instructions per slot
    static constexpr int FIT = (160 * 1024 / 16) / (NWK * UNITS);
    static constexpr int SLOTS = FIT < DPAIRS_PER_WAVE ? FIT : DPAIRS_PER_WAVE;
};

// The A fragments of `slot` for a wave's k step pairs (pair i of the wave is
// split pair wave + NWK i, clamped to the split's pn pairs from pa): lane
// (r, kq) holds rank row jb * 16 + r (clamped), k 8 kq .. 8 kq + 7 of each
// 32-wide step.
template <typename V, int PPW, int RB>
__device__ __forceinline__ void load_a_frags(const ApplyArgs &a, int slot, int pa, int pn, int wave,
                                             V (&f)[PPW][2][RB]) {
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;
    const int kq = lane >> 4;
    const int Rp = a.R;
    const uint32_t rowb = static_cast<uint32_t>(a.d_in) * 2;
    const __amdgpu_buffer_rsrc_t ars =
        make_rsrc(static_cast<const uint16_t *>(a.A_slab) + static_cast<size_t>(slot) * Rp * a.d_in, Rp * rowb);
#pragma unroll
    for (int i = 0; i < PPW; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int jb = 0; jb < RB; ++jb)
                f[i][h][jb] = bload8<V>(ars, static_cast<uint32_t>(min(jb * 16 + r, Rp - 1)) * rowb + 16 * kq,
                                        static_cast<uint32_t>(2 * (pa + min(wave + NWK * i, pn - 1)) + h) * 64);
}

template <int DT, int TB, int RB>
__global__ __launch_bounds__(NWK * 64) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_decode_gemm(
    ApplyArgs a, DecodeArgs d, const int32_t *__restrict__ idx) {
    using E = Elem<DT>;
    using V = typename E::vec8;
    using Ring = DecRing<TB>;
    constexpr int NB = TB * DCB;  // 16x16 output blocks per wave
    constexpr int PPW = DPAIRS_PER_WAVE;
    constexpr int RS = Ring::SLOTS;
    constexpr int L = Ring::LOADS;
    static_assert(RS >= 1 && RS <= 4, "ring");
    static_assert(NWK * (NB + (RB <= 2 ? 2 : 1) * TB * RB) * 64 <= NWK * RS * Ring::UNITS,
                  "cross-wave sums fit in the ring");
    // Per-wave rings of step pairs; after the main loop, the cross-wave sums.
    __shared__ u32x4_t smem[NWK * RS * Ring::UNITS];

    const int tid = threadIdx.x;
    const int wave = uniform(tid >> 6);
    const int lane = tid & 63;
    const int r = lane & 15;
    const int kq = lane >> 4;
    const int T = a.T;
    const int Rp = a.R;
    const int ncg = a.d_out / DCOLS;
    const int cg = uniform(blockIdx.x % ncg);
    const int q = uniform(blockIdx.x / ncg);
    const int c0 = cg * DCOLS;
    const int kst = a.d_in >> 5;
    const int kp = kst >> 1;  // step pairs (d_in % 64 == 0)
    const int pa = uniform(q * kp / d.splits);
    const int pn = uniform((q + 1) * kp / d.splits - pa);  // pairs of this split (1 .. NWK * PPW)
    const uint32_t rowb = static_cast<uint32_t>(a.d_in) * 2;  // bytes per row
    // Pair i of this wave: split pair wave + NWK i (valid when < pn); its two
    // k steps are 2 (pa + p) and 2 (pa + p) + 1.
    auto pair_of = [&](int i) { return wave + NWK * i; };

    // 1. The A fragments of slot cg for this wave's steps (requested before
    //    the token indices are known: a slot is named by few tokens if any).
    //    Pools of more slots than column groups take slot cg + ncg in the
    //    main loop as well (HS = 2, ranks up to 32: the sums' LDS round has
    //    room for both); slots past those are added after it.
    constexpr int HS = RB <= 2 ? 2 : 1;
    V af[HS][PPW][2][RB];
    const bool shrink0 = cg < a.S;
    const bool shrink1 = HS == 2 && cg + ncg < a.S;
    if (shrink0) load_a_frags<V, PPW, RB>(a, cg, pa, pn, wave, af[0]);
    if (shrink1) load_a_frags<V, PPW, RB>(a, cg + ncg, pa, pn, wave, af[HS - 1]);
    // The states of those slots, used by the shrink's stores at the end
    // (vector loads, older than the ring's: no wait count changes).
    const __amdgpu_buffer_rsrc_t srs = make_rsrc(a.slots, static_cast<uint32_t>(a.S) * sizeof(SlotDev));
    const int state0 = shrink0 ? __builtin_amdgcn_raw_buffer_load_b32(srs, static_cast<uint32_t>(cg) * sizeof(SlotDev), 0, 0)
                               : SLOT_FREE;
    const int state1 =
        shrink1 ? __builtin_amdgcn_raw_buffer_load_b32(srs, static_cast<uint32_t>(cg + ncg) * sizeof(SlotDev), 0, 0)
                : SLOT_FREE;

    // 2. Step pairs straight into this wave's ring slots: one instruction per
    //    8 rows, 8 lanes a row covering its 128-byte line; the chunk a lane
    //    fetches is XOR-swizzled by the row within its 16-row block, so the
    //    chunk at position m of row rho is chunk m ^ sw(rho), sw(rho) =
    //    rho & 7, which keeps the operand reads free of bank conflicts (the
    //    same layout as the LDS-staged tiled GEMM).  x rows past T repeat row
    //    T - 1 (their outputs are never used).
    const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.x, static_cast<uint32_t>(T) * rowb);
    const __amdgpu_buffer_rsrc_t wrs =
        make_rsrc(static_cast<const uint16_t *>(a.W) + static_cast<size_t>(c0) * a.d_in, DCOLS * rowb);
    uint32_t loff[L];
#pragma unroll
    for (int g = 0; g < L; ++g) {
        const int rho = 8 * (g & 1) + (lane >> 3);   // row within its 16-row block
        const int chunk = (lane & 7) ^ (rho & 7);
        const int row = 8 * g + (lane >> 3);         // row of the slot: x rows first, then W
        const int src = row < Ring::XROWS ? min(row, T - 1) : row - Ring::XROWS;
        loff[g] = static_cast<uint32_t>(src) * rowb + chunk * 16;
    }
    u32x4_t *ring = smem + wave * RS * Ring::UNITS;
    // Byte offset of pair i of this wave within a row (clamped to the split).
    auto pair_off = [&](int i) { return static_cast<uint32_t>(pa + min(pair_of(i), pn - 1)) * 128; };
#pragma unroll
    for (int i = 0; i < RS; ++i)
        issue_pair(xrs, wrs, ring + (i % RS) * Ring::UNITS, loff, Ring::XROWS / 8, L, pair_off(i));
    // Adapter index of token `lane` (every wave holds all T of them), used
    // by the shrink at the end.
    const int my_idx = idx[min(lane, T - 1)];

    // 3. Base GEMM (and the shrink of slot cg) pair by pair.  Operand reads:
    //    lane (r, kq) of half h takes row r of a block, chunk 4 h + kq, at
    //    position (4 h + kq) ^ sw(r).
    const int sw = r & 7;
    const int lo[2] = {r * 8 + ((0 + kq) ^ sw), r * 8 + ((4 + kq) ^ sw)};
    f32x4_t acc[TB][DCB];
    f32x4_t hacc[HS][TB][RB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
#pragma unroll
        for (int c = 0; c < DCB; ++c) acc[tb][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int hs = 0; hs < HS; ++hs)
#pragma unroll
            for (int jb = 0; jb < RB; ++jb) hacc[hs][tb][jb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
        // Loads issued after pair i so far: pairs i + 1 .. min(i + RS - 1,
        // PPW - 1), and the token-index load (issued after pair RS - 1).
        const int later = (i + RS - 1 < PPW - 1 ? i + RS - 1 : PPW - 1) - i;
        wait_loads<L>(later, i < RS ? 1 : 0);
        const u32x4_t *slot = ring + (i % RS) * Ring::UNITS;
        V xf[2][TB], wf[2][DCB];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) xf[h][tb] = __builtin_bit_cast(V, slot[tb * 128 + lo[h]]);
#pragma unroll
            for (int c = 0; c < DCB; ++c) wf[h][c] = __builtin_bit_cast(V, slot[(TB + c) * 128 + lo[h]]);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (i + RS < PPW)
            issue_pair(xrs, wrs, ring + (i % RS) * Ring::UNITS, loff, Ring::XROWS / 8, L, pair_off(i + RS));
        if (pair_of(i) < pn) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                    for (int c = 0; c < DCB; ++c) acc[tb][c] = E::mfma(xf[h][tb], wf[h][c], acc[tb][c]);
#pragma unroll
                for (int hs = 0; hs < HS; ++hs) {
                    if (hs == 0 ? shrink0 : shrink1) {
#pragma unroll
                        for (int jb = 0; jb < RB; ++jb) {
                            const V am = (jb * 16 + r < Rp) ? af[hs][i][h][jb] : zero8<V>();
#pragma unroll
                            for (int tb = 0; tb < TB; ++tb)
                                hacc[hs][tb][jb] = E::mfma(xf[h][tb], am, hacc[hs][tb][jb]);
                        }
                    }
                }
            }
        }
    }

    // 4. The 4 waves' sums in LDS (the ring is free once every wave is past
    //    its last pair), added in a fixed order (wave 0 + 1 + 2 + 3), stored
    //    as this split's partial sums, fragment order [q][16-column
    //    block][tb][lane] (16 bytes a lane).  The shrink's sums (slots cg
    //    and cg + ncg) take the same LDS round, after the GEMM's.
    f32x4_t *red = reinterpret_cast<f32x4_t *>(smem);
    f32x4_t *hred = red + NWK * NB * 64;  // slot hs at hred + hs * NWK * TB * RB * 64
    __syncthreads();
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int c = 0; c < DCB; ++c) red[((wave * TB + tb) * DCB + c) * 64 + lane] = acc[tb][c];
#pragma unroll
    for (int hs = 0; hs < HS; ++hs) {
        if (hs == 0 ? shrink0 : shrink1) {
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int jb = 0; jb < RB; ++jb)
                    hred[((hs * NWK + wave) * TB + tb) * RB * 64 + jb * 64 + lane] = hacc[hs][tb][jb];
        }
    }
    __syncthreads();
    f32x4_t *part = reinterpret_cast<f32x4_t *>(d.part);
#pragma unroll
    for (int f0 = 0; f0 < NB; f0 += NWK) {
        const int f = f0 + wave;  // fragment (tb, c) = (f / DCB, f % DCB)
        f32x4_t v = red[f * 64 + lane];
#pragma unroll
        for (int w = 1; w < NWK; ++w) v += red[(w * NB + f) * 64 + lane];
        const int tb = f / DCB, c = f % DCB;
        // Streaming store: the epilogue reads the partials once, on other XCDs.
        __builtin_nontemporal_store(v, &part[((static_cast<size_t>(q) * (a.d_out / 16) + c0 / 16 + c) * TB + tb) * 64 + lane]);
    }

    // 5. Shrink results: this split's part of h = x . A_s^T for the rows of
    //    the tokens of slot s (fp32, by token, part q); the 4 waves' sums
    //    added in order.
    float *hout = a.h + static_cast<size_t>(q) * T * Rp;
    // Adds the 4 waves' h fragments at `hr` in order and stores the rows of
    // `mask`'s tokens.
    auto sum_store_h = [&](unsigned long long mask, const f32x4_t *hr) {
        for (int f = wave; f < TB * RB; f += NWK) {
            f32x4_t v = hr[f * 64 + lane];
#pragma unroll
            for (int w = 1; w < NWK; ++w) v += hr[(w * TB * RB + f) * 64 + lane];
            const int tb = f / RB, j = (f % RB) * 16 + r;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = tb * 16 + kq * 4 + e;
                if (j < Rp && t < T && ((mask >> t) & 1ull)) hout[static_cast<size_t>(t) * Rp + j] = v[e];
            }
        }
    };
    auto store_h = [&](unsigned long long mask, const f32x4_t (&hc)[TB][RB]) {
        __syncthreads();  // red free
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int jb = 0; jb < RB; ++jb) red[((wave * TB + tb) * RB + jb) * 64 + lane] = hc[tb][jb];
        __syncthreads();
        sum_store_h(mask, red);
    };
    if (shrink0) {
        const unsigned long long mask = __ballot(lane < T && my_idx == cg);
        if (mask != 0 && uniform(state0) == SLOT_ACTIVE) sum_store_h(mask, hred);
    }
    if (shrink1) {
        const unsigned long long mask = __ballot(lane < T && my_idx == cg + ncg);
        if (mask != 0 && uniform(state1) == SLOT_ACTIVE) sum_store_h(mask, hred + NWK * TB * RB * 64);
    }
    // Slots cg + HS ncg, ... (pools of more slots than HS column groups):
    // x fragments read again, straight from global memory.
    for (int s = cg + HS * ncg; s < a.S; s += ncg) {
        const unsigned long long mask = __ballot(lane < T && my_idx == s);
        if (mask == 0) continue;
        if (uniform(a.slots[s].state) != SLOT_ACTIVE) continue;
        const __amdgpu_buffer_rsrc_t ars =
            make_rsrc(static_cast<const uint16_t *>(a.A_slab) + static_cast<size_t>(s) * Rp * a.d_in, Rp * rowb);
        f32x4_t hc[TB][RB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int jb = 0; jb < RB; ++jb) hc[tb][jb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int i = 0; i < PPW; ++i) {
            if (pair_of(i) >= pn) break;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t sb = static_cast<uint32_t>(2 * (pa + pair_of(i)) + h) * 64;
                V xv[TB], av[RB];
#pragma unroll
                for (int tb = 0; tb < TB; ++tb)
                    xv[tb] = bload8<V>(xrs, static_cast<uint32_t>(min(tb * 16 + r, T - 1)) * rowb + 16 * kq, sb);
#pragma unroll
                for (int jb = 0; jb < RB; ++jb)
                    av[jb] = bload8<V>(ars, static_cast<uint32_t>(min(jb * 16 + r, Rp - 1)) * rowb + 16 * kq, sb);
#pragma unroll
                for (int jb = 0; jb < RB; ++jb) {
                    const V am = (jb * 16 + r < Rp) ? av[jb] : zero8<V>();
#pragma unroll
                    for (int tb = 0; tb < TB; ++tb) hc[tb][jb] = E::mfma(xv[tb], am, hc[tb][jb]);
                }
            }
        }
        store_h(mask, hc);
    }
}

// -------------------------------------------------------------- epilogue --

// Workgroup: NWK waves for one 16-column block, thread (tb = wave < TB,
// lane) holding rows tb*16 + 4*(lane/16) + i of column lane % 16, plus one
// routing wave.  The routing wave loads only the token indices and their slot
// entries, so its waits never include the row waves' loads.
template <int DT, int TB, int RB>
__global__ __launch_bounds__((NWK + 1) * 64) void k_decode_epilogue(ApplyArgs a, DecodeArgs d,
                                                                    const int32_t *__restrict__ idx, RouteOut out) {
    using E = Elem<DT>;
    using raw = typename E::raw;
    constexpr int HR = RB * 16;
    constexpr int TP = TB * 16;
    constexpr int HQ = (TP * HR / 4 + NWK * 64 - 1) / (NWK * 64);  // h float4s per row-wave thread
    __shared__ float hs[TP][HR + 1];
    __shared__ SmallRoute sr;
    const int tid = threadIdx.x;
    const int wave = uniform(tid >> 6);
    const int lane = tid & 63;
    const int T = a.T;
    const int Rp = a.R;
    const int nb = blockIdx.x;  // 16-column block
    const int n = nb * 16 + (lane & 15);

    // Every LoRA bucket runs fused under the FUSED policy and under AUTO with
    // a threshold below 1 (a bucket holds at least one token).  Then a row's
    // treatment follows from its own slot entry, and the row waves do not
    // wait for the routing, which only workgroup 0 computes (to publish it).
    const bool all_fused = a.policy == 1 || (a.policy == 0 && d.theta < 1);
    if (wave == NWK) {
        // Routing wave: token index, then its slot entry; the routing in LDS,
        // published by workgroup 0.  With all buckets fused it meets the row
        // waves' barrier first and routes afterwards.
        if (all_fused) {
            __syncthreads();
            if (blockIdx.x != 0) return;
        }
        const int v = lane < T ? idx[min(lane, T - 1)] : -1;
        const int2 e = reinterpret_cast<const int2 *>(a.slots)[2 * min(max(v, 0), a.S - 1)];
        small_route(v, e.x, e.y, T, a.S, d.max_rank, a.policy, d.theta, sr);
        if (blockIdx.x == 0) publish_route(sr, T, out);
        if (!all_fused) __syncthreads();
        return;
    }

    // Row waves: the adapter index of this thread's 4 rows; the first group
    // of splits' partial sums and h parts (which do not depend on it); then,
    // as soon as the indices arrive, the B rows and slot entries of their
    // slots (clamped: used only for FUSED rows, whose key is that index).
    const int tb = min(wave, TB - 1);
    int vi[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) vi[i] = idx[min(tb * 16 + (lane >> 4) * 4 + i, T - 1)];
    // Splits are taken SQ at a time (4: all of them at once for d_in <=
    // 4096; 2 at ranks above 32, for registers), each group's loads in
    // flight together, and added in split order.
    constexpr int SQ = RB >= 3 ? 2 : 4;
    const f32x4_t *part = reinterpret_cast<const f32x4_t *>(d.part) + (static_cast<size_t>(nb) * TB + tb) * 64 + lane;
    const size_t qstride = static_cast<size_t>(a.d_out / 16) * TB * 64;
    const int hq_n = T * Rp / 4;
    const size_t pstride = static_cast<size_t>(T) * Rp / 4;
    const float4 *hp = reinterpret_cast<const float4 *>(a.h);
    f32x4_t pv[SQ];
    float4 hv[HQ][SQ];
    // Unconditional loads (split index clamped; the repeats are not added),
    // so the wait counts stay exact.
    auto load_group = [&](int q0) {
#pragma unroll
        for (int u = 0; u < SQ; ++u) pv[u] = part[min(q0 + u, d.splits - 1) * qstride];
#pragma unroll
        for (int m = 0; m < HQ; ++m)
#pragma unroll
            for (int u = 0; u < SQ; ++u)
                hv[m][u] = hp[min(q0 + u, d.splits - 1) * pstride + min(tid + m * NWK * 64, hq_n - 1)];
    };
    load_group(0);
    u32x4_t bw[4][2 * RB];
    float sc[4];
    int st[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int kc = min(max(vi[i], 0), a.S - 1);
        const uint16_t *bp = static_cast<const uint16_t *>(a.B_slab) + (static_cast<size_t>(kc) * a.d_out + n) * Rp;
#pragma unroll
        for (int qb = 0; qb < 2 * RB; ++qb) bw[i][qb] = *reinterpret_cast<const u32x4_t *>(bp + min(8 * qb, Rp - 8));
        sc[i] = a.slots[kc].scale;
        st[i] = a.slots[kc].state;
    }
    f32x4_t acc;
    float4 hsum[HQ];
    for (int q0 = 0; q0 < d.splits; q0 += SQ) {
        if (q0 > 0) load_group(q0);
        asm volatile("" ::: "memory");  // every load of the group is issued before the first add
        if (q0 == 0) {
            acc = pv[0];
#pragma unroll
            for (int m = 0; m < HQ; ++m) hsum[m] = hv[m][0];
        }
#pragma unroll
        for (int u = 0; u < SQ; ++u) {
            if ((q0 > 0 || u > 0) && q0 + u < d.splits) {
                acc += pv[u];
#pragma unroll
                for (int m = 0; m < HQ; ++m) {
                    hsum[m].x += hv[m][u].x;
                    hsum[m].y += hv[m][u].y;
                    hsum[m].z += hv[m][u].z;
                    hsum[m].w += hv[m][u].w;
                }
            }
        }
    }
    // h by token, to LDS.
#pragma unroll
    for (int m = 0; m < HQ; ++m) {
        const int e = tid + m * NWK * 64;
        if (e < hq_n) {
            const int t = (e * 4) / Rp, j = (e * 4) % Rp;
            hs[t][j] = hsum[m].x;
            hs[t][j + 1] = hsum[m].y;
            hs[t][j + 2] = hsum[m].z;
            hs[t][j + 3] = hsum[m].w;
        }
    }
    __syncthreads();
    if (wave >= TB) return;

    // FUSED rows: the key of a LoRA token is its adapter index, so the B
    // rows loaded above are its slot's.  With every bucket fused the key
    // follows from the token's own index and slot entry (as the routing
    // defines it); otherwise from the routing's bucket records.
    int key[4];
    bool fused[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = tb * 16 + (lane >> 4) * 4 + i;
        if (all_fused) {
            const int v = vi[i];
            key[i] = v == -1 ? a.S : (v >= 0 && v < a.S && st[i] == SLOT_ACTIVE) ? v : a.S + 1;
            fused[i] = t < T && key[i] < a.S;
        } else {
            const int sg = sr.tok_seg[min(t, T - 1)];
            key[i] = sr.segs[sg][0];
            fused[i] = t < T && key[i] < a.S && sr.segs[sg][3] == SEG_FUSED;
        }
    }
    raw *y = static_cast<raw *>(a.y);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = tb * 16 + (lane >> 4) * 4 + i;
        if (t >= T) continue;
        float o = acc[i];
        if (fused[i]) {
            const float *hrow = hs[t];
            float dsum = 0.0f;
#pragma unroll
            for (int qb = 0; qb < 2 * RB; ++qb) {
                if (8 * qb < Rp) {
                    const u32x4_t bq = bw[i][qb];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        dsum += hrow[8 * qb + 2 * e] * E::to_f(static_cast<raw>(bq[e] & 0xFFFFu));
                        dsum += hrow[8 * qb + 2 * e + 1] * E::to_f(static_cast<raw>(bq[e] >> 16));
                    }
                }
            }
            o += sc[i] * dsum;
        }
        y[static_cast<size_t>(t) * a.d_out + n] = (key[i] == a.S + 1) ? E::qnan : E::from_f(o);
    }
}

template <int DT, int TB>
hipError_t launch_tb(const ApplyArgs &a, const DecodeArgs &d, const int32_t *idx, const RouteOut &out,
                     hipStream_t st, LaunchEvents ev) {
    const dim3 grid((a.d_out / DCOLS) * d.splits);
    const dim3 egrid(a.d_out / 16);
    const dim3 block(NWK * 64);
    const dim3 eblock((NWK + 1) * 64);
    switch ((a.R + 15) / 16) {
        case 1: LORA_LAUNCH(ev, (k_decode_gemm<DT, TB, 1>), grid, block, 0, st, a, d, idx); break;
        case 2: LORA_LAUNCH(ev, (k_decode_gemm<DT, TB, 2>), grid, block, 0, st, a, d, idx); break;
        case 3: LORA_LAUNCH(ev, (k_decode_gemm<DT, TB, 3>), grid, block, 0, st, a, d, idx); break;
        default: LORA_LAUNCH(ev, (k_decode_gemm<DT, TB, 4>), grid, block, 0, st, a, d, idx); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const LaunchEvents eev{nullptr, ev.done, nullptr};  // the epilogue ends the call
    switch ((a.R + 15) / 16) {
        case 1: LORA_LAUNCH(eev, (k_decode_epilogue<DT, TB, 1>), egrid, eblock, 0, st, a, d, idx, out); break;
        case 2: LORA_LAUNCH(eev, (k_decode_epilogue<DT, TB, 2>), egrid, eblock, 0, st, a, d, idx, out); break;
        case 3: LORA_LAUNCH(eev, (k_decode_epilogue<DT, TB, 3>), egrid, eblock, 0, st, a, d, idx, out); break;
        default: LORA_LAUNCH(eev, (k_decode_epilogue<DT, TB, 4>), egrid, eblock, 0, st, a, d, idx, out); break;
    }
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const ApplyArgs &a, const DecodeArgs &d, const int32_t *idx, const RouteOut &out,
                     hipStream_t st, LaunchEvents ev) {
    switch (decode_token_blocks(a.T)) {
        case 1: return launch_tb<DT, 1>(a, d, idx, out, st, ev);
        case 2: return launch_tb<DT, 2>(a, d, idx, out, st, ev);
        default: return launch_tb<DT, 4>(a, d, idx, out, st, ev);
    }
}

}  // namespace

int decode_token_blocks(int T) {
    int tb = 1;
    while (tb * 16 < T) tb *= 2;
    return tb;
}

int decode_splits(int T, int d_in, int d_out) {
    // Each GEMM wave takes at most DPAIRS_PER_WAVE step pairs (64 k each):
    // at least ceil(pairs / (NWK x DPAIRS_PER_WAVE)) splits, and at least 4.
    // Narrow outputs (d_out / 64 column groups, fewer than 64 of them) take
    // more splits, up to MAX_DSPLIT, so that the launch still spreads over
    // the 256 CUs: a 512-wide shard runs 8 groups x 16 splits.  Every split
    // keeps at least one pair; 0 beyond MAX_DSPLIT splits.  d_in and d_out
    // are multiples of 64.
    (void)T;
    const int kp = d_in / 64;
    const int per = NWK * DPAIRS_PER_WAVE;
    const int ncg = d_out / DCOLS;
    int s = (kp + per - 1) / per;
    if (s < 4) s = 4;
    if (s > MAX_DSPLIT) return 0;
    const int fill = (256 + ncg - 1) / ncg;
    if (s < fill) s = fill < MAX_DSPLIT ? fill : MAX_DSPLIT;
    if (s > kp) s = kp;
    return s;
}

hipError_t launch_decode(const ApplyArgs &a, const DecodeArgs &d, const int32_t *idx, const RouteOut &out,
                         hipStream_t st, LaunchEvents ev) {
    return (a.dtype == DT_F16) ? launch_dt<DT_F16>(a, d, idx, out, st, ev)
                               : launch_dt<DT_BF16>(a, d, idx, out, st, ev);
}

hipError_t launch_route_small(const int32_t *idx, int T, int S, const SlotDev *slots, int max_rank, int policy,
                              int theta, const RouteOut &out, hipStream_t st) {
    if (T < 1 || T > DECODE_MAX_T) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_route_small, dim3(1), dim3(64), 0, st, idx, T, S, slots, max_rank, policy, theta, out);
    return hipGetLastError();
}

}  // namespace lora
