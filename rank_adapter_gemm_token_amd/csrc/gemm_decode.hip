// gemm_decode.hip -- the decode path (T <= 64 tokens per call, fp16/bf16):
// routing, LoRA shrink, base projection and the fused LoRA expand in two
// launches.
//
// At decode sizes a call is bound by streaming W (d_out x d_in, read once)
// from HBM.  The next cost is x: every output column needs all of x, so a
// layout in which each CU covers a few columns over the whole of d_in reads
// x from L2 once per CU (128 MiB at d_in = 4096, T = 64, 256 CUs).  Here a
// workgroup covers 64 columns over one k split of d_in (x traffic / 4), and
// the splits' fp32 partial sums are added by a second, small kernel that
// also applies the LoRA term:
//
// k_decode_gemm -- workgroup (column group of 64, k split q), 4 waves (one
//   per SIMD, 512 registers each); wave w holds the split's k steps w, w+4,
//   ..., w+28 for all 64 columns and all T rows.
//   * Loads are issued in the order they are needed and all at once, through
//     buffer resources (uniform column-block and step offsets): the adapter
//     indices and the slot table (routing workgroups), then every x and W
//     fragment of the wave -- the whole of the workgroup's W tile is in
//     flight from the start.
//   * Routing workgroups sort the (at most 64) tokens by adapter in LDS, in
//     one wave: each token's sorted position by comparing keys, then
//     buckets, modes and tiles from ballots -- the same stable order as the
//     routing kernel of larger calls.  Workgroup 0 publishes it (permutation,
//     bucket records, tiles, statistics, invalid-token count).  The A rows of
//     the workgroup's first LoRA bucket are requested right after.
//   * GEMM: fp32 MFMA accumulators over the wave's steps; the 4 waves' sums
//     are added in LDS in a fixed order and the split's partial sums stored,
//     coalesced.
//   * Shrink: the workgroups of column group c also compute, for LoRA
//     buckets c, c + groups, ..., this split's part of h = x . A_slot^T for
//     all T rows from the x fragments they hold, keeping the bucket's rows
//     (fp32, by sorted row, part q).
// k_decode_epilogue -- 16 columns per workgroup, rows in token order: adds
//   the splits' partial sums in a fixed order, adds s * h . B for FUSED
//   buckets (h = the parts summed in order, fp32 VALU), rounds once and
//   stores; invalid tokens get NaN.  SEPARATE rows keep the rounded base for
//   the residual kernel.
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

constexpr int NWK = 4;            // waves per workgroup of the GEMM kernel (one per SIMD)
constexpr int DCB = 4;            // 16-column blocks per GEMM workgroup
constexpr int DCOLS = DCB * 16;   // columns per GEMM workgroup
constexpr int DSTEPS_PER_WAVE = 8;  // k steps a wave holds at once (per group)
constexpr int SMAX_SEG = DECODE_MAX_T + 2;
constexpr int SLOT_CAP = MAX_KEYS - 2;
constexpr int SLOT_LD = SLOT_CAP / (NWK * 64);  // slot-table loads per thread

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
    int tiles[DECODE_MAX_T + SMAX_SEG][2];  // {bucket, first row}
    int n_seg;
    int n_lora;                 // LoRA buckets (records 0 .. n_lora-1)
    int n_tiles;
    int stat[6];                // fused, separate, base_only, invalid, rows padded, rows true
};

// Wave 0: key = slot (active), S (base_only) or S + 1 (invalid) of each
// token, then each token's sorted position = #(smaller keys) + #(same key,
// smaller index); buckets, modes, tiles and statistics from ballots.
// `slot_sr` holds {state, rank} of every slot (LDS).  Other waves return.
__device__ void small_route(int v, int T, int S, const int2 *slot_sr, int max_rank, int policy, int theta,
                            SmallRoute &sr) {
    const int lane = threadIdx.x & 63;
    if (threadIdx.x >= 64) return;
    const bool tv = lane < T;
    int key = S, rank = 0;
    if (v != -1) {
        key = S + 1;
        if (v >= 0 && v < S) {
            const int2 e = slot_sr[v];
            if (e.x == SLOT_ACTIVE) {
                key = v;
                rank = e.y;
            }
        }
    }
    if (!tv) key = 0x7FFF;
    sr.key[lane] = key;
    sr.rank[lane] = rank;
    lds_fence();
    int pos = 0;
#pragma unroll
    for (int j4 = 0; j4 < DECODE_MAX_T; j4 += 4) {
        const int4 k4 = *reinterpret_cast<const int4 *>(&sr.key[j4]);
        const int kk[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) pos += (kk[u] < key || (kk[u] == key && j4 + u < lane)) ? 1 : 0;
    }
    if (tv) sr.perm[pos] = lane;
    lds_fence();
    // Lane p: the token at sorted position p.
    const int p = lane;
    const bool pv = p < T;
    const int ptok = pv ? sr.perm[p] : 0;
    const int pkey = pv ? sr.key[ptok] : 0x7FFF;
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
            sr.tiles[tile0 + j][0] = seg;
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

// Workgroup 0: publish the routing for the epilogue and residual kernels, the
// statistics and the invalid-token count.
__device__ void publish_route(const SmallRoute &sr, int T, const RouteOut &out) {
    const int tid = threadIdx.x;
    for (int i = tid; i < T; i += blockDim.x) {
        out.perm[i] = sr.perm[i];
        out.pos_seg[i] = sr.pos_seg[i];
        out.tok_pos[i] = sr.tok_pos[i];
        out.tok_seg[i] = sr.tok_seg[i];
    }
    for (int i = tid; i < 4 * sr.n_seg; i += blockDim.x) out.segs[i] = sr.segs[i >> 2][i & 3];
    for (int i = tid; i < 2 * sr.n_tiles; i += blockDim.x) out.tiles[i] = sr.tiles[i >> 1][i & 1];
    if (tid == 0) {
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
        *out.stats = st;
        if (sr.stat[3] > 0) atomicAdd(out.err, static_cast<unsigned long long>(sr.stat[3]));
    }
}

// ------------------------------------------------------------------ GEMM --

template <int DT, int TB, int RB>
__global__ __launch_bounds__(NWK * 64) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_decode_gemm(
    ApplyArgs a, DecodeArgs d, const int32_t *__restrict__ idx, RouteOut out) {
    using E = Elem<DT>;
    using V = typename E::vec8;
    constexpr int NB = TB * DCB;  // 16x16 output blocks per wave
    __shared__ f32x4_t red[NWK * NB * 64];  // cross-wave sums (64 KiB at TB = 4)
    __shared__ int2 s_slot[SLOT_CAP];       // {state, rank} per slot (routing workgroups)
    __shared__ SmallRoute sr;

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
    const int qa = q * kst / d.splits;
    const int nsq = (q + 1) * kst / d.splits - qa;  // k steps of this split
    const bool routes = cg < d.route_groups;

    // 1. Routing inputs first (they return first): the adapter indices and
    //    every slot's {state, rank}.
    int v_idx = -1;
    int2 sl[SLOT_LD];
    if (routes) {
        if (tid < T) v_idx = idx[tid];
#pragma unroll
        for (int u = 0; u < SLOT_LD; ++u)
            sl[u] = reinterpret_cast<const int2 *>(a.slots)[2 * min(tid + u * NWK * 64, a.S - 1)];
    }

    // 2. Wave w takes the split's k steps w, w + 4, ..., w + 28: x fragments
    //    for all T rows (rows past T repeat row T-1) and W fragments for all
    //    64 columns, every load unconditional (clamped step).  One wave per
    //    SIMD holds them all.
    constexpr int GS = DSTEPS_PER_WAVE;
    // Buffer loads: one per-lane byte offset per operand row; column blocks,
    // the wave's first step and the per-step stride are uniform (SGPR or
    // immediate offsets), so addressing costs few registers.
    const uint32_t rowb = static_cast<uint32_t>(a.d_in) * 2;  // bytes per row
    const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.x, static_cast<uint32_t>(T) * rowb);
    const __amdgpu_buffer_rsrc_t wrs =
        make_rsrc(static_cast<const uint16_t *>(a.W) + static_cast<size_t>(c0) * a.d_in, DCOLS * rowb);
    const uint32_t kb = static_cast<uint32_t>(qa) * 64 + 16 * kq;  // byte offset of the lane's k
    uint32_t xo[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) xo[tb] = static_cast<uint32_t>(min(tb * 16 + r, T - 1)) * rowb + kb;
    const uint32_t wo = static_cast<uint32_t>(r) * rowb + kb;

    // All of this wave's operands in flight at once (decode_splits keeps a
    // split at <= NWK * GS k steps).
    V xf[GS][TB];
    V wf[GS][DCB];
#pragma unroll
    for (int i = 0; i < GS; ++i) {
        const uint32_t sb = static_cast<uint32_t>(min(wave + NWK * i, nsq - 1)) * 64;  // uniform
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) xf[i][tb] = bload8<V>(xrs, xo[tb], sb);
#pragma unroll
        for (int c = 0; c < DCB; ++c) wf[i][c] = bload8<V>(wrs, wo, sb + c * 16 * rowb);
    }

    // 3. Routing in LDS (wave 0), published by workgroup 0.  This
    //    workgroup's LoRA buckets are g = cg, cg + groups, ...
    int n_lora = 0;
    if (routes) {
#pragma unroll
        for (int u = 0; u < SLOT_LD; ++u)
            if (tid + u * NWK * 64 < a.S) s_slot[tid + u * NWK * 64] = sl[u];
        __syncthreads();
        small_route(v_idx, T, a.S, s_slot, d.max_rank, a.policy, d.theta, sr);
        __syncthreads();
        if (blockIdx.x == 0) publish_route(sr, T, out);
        n_lora = uniform(sr.n_lora);
    }

    // 4. A fragments of the first bucket's slot for these steps, issued
    //    behind x and W so they never delay them.
    V af[GS][RB];
    auto load_a = [&](int g) {
        const int key = uniform(sr.segs[g][0]);
        const __amdgpu_buffer_rsrc_t ars =
            make_rsrc(static_cast<const uint16_t *>(a.A_slab) + static_cast<size_t>(key) * Rp * a.d_in, Rp * rowb);
#pragma unroll
        for (int i = 0; i < GS; ++i) {
            const uint32_t sb = static_cast<uint32_t>(min(wave + NWK * i, nsq - 1)) * 64;
#pragma unroll
            for (int jb = 0; jb < RB; ++jb)
                af[i][jb] = bload8<V>(ars, static_cast<uint32_t>(min(jb * 16 + r, Rp - 1)) * rowb + kb, sb);
        }
    };
    if (cg < n_lora) load_a(cg);

    // 5. Base GEMM on the steps this wave holds.
    f32x4_t acc[TB][DCB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int c = 0; c < DCB; ++c) acc[tb][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < GS; ++i) {
        if (wave + NWK * i < nsq) {
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int c = 0; c < DCB; ++c) acc[tb][c] = E::mfma(xf[i][tb], wf[i][c], acc[tb][c]);
        }
    }

    // 6. Cross-wave sums in LDS, fixed order (wave 0 + 1 + 2 + 3), stored
    //    as this split's partial sums [q][t][c0 .. c0+63], 16 bytes a thread.
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int c = 0; c < DCB; ++c) red[((wave * TB + tb) * DCB + c) * 64 + lane] = acc[tb][c];
    __syncthreads();
    float *part = d.part + static_cast<size_t>(q) * T * a.d_out;
    const float *redf = reinterpret_cast<const float *>(red);
    for (int e = tid; e < T * (DCOLS / 4); e += NWK * 64) {
        const int t = e / (DCOLS / 4), c4 = (e % (DCOLS / 4)) * 4;
        const int tb = t / 16, ii = t % 4, kq2 = (t % 16) / 4;
        float o[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int col = c4 + u, c = col / 16, ln = kq2 * 16 + col % 16;
            float sum = 0.0f;
#pragma unroll
            for (int w = 0; w < NWK; ++w) sum += redf[(((w * TB + tb) * DCB + c) * 64 + ln) * 4 + ii];
            o[u] = sum;
        }
        *reinterpret_cast<float4 *>(part + static_cast<size_t>(t) * a.d_out + c0 + c4) =
            float4{o[0], o[1], o[2], o[3]};
    }

    // 7. Shrink, bucket by bucket: this split's part of h = x . A_slot^T for
    //    all T rows from the x fragments already held, cross-wave sums in
    //    LDS, rows of the bucket kept (by sorted row, part q).
    float *hout = a.h + static_cast<size_t>(q) * T * Rp;
    for (int g = cg; g < n_lora; g += ncg) {
        if (g != cg) load_a(g);
        f32x4_t hacc[TB][RB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int jb = 0; jb < RB; ++jb) hacc[tb][jb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < GS; ++i) {
            if (wave + NWK * i < nsq) {
#pragma unroll
                for (int jb = 0; jb < RB; ++jb) {
                    const V am = (jb * 16 + r < Rp) ? af[i][jb] : zero8<V>();
#pragma unroll
                    for (int tb = 0; tb < TB; ++tb) hacc[tb][jb] = E::mfma(xf[i][tb], am, hacc[tb][jb]);
                }
            }
        }
        __syncthreads();  // red free
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int jb = 0; jb < RB; ++jb) red[((wave * TB + tb) * RB + jb) * 64 + lane] = hacc[tb][jb];
        __syncthreads();
        for (int e = tid; e < T * Rp; e += NWK * 64) {
            const int t = e / Rp, j = e % Rp;
            if (sr.tok_seg[t] != g) continue;
            const int tb = t / 16, ii = t % 4, ln = ((t % 16) / 4) * 16 + (j % 16), jb = j / 16;
            float sum = 0.0f;
#pragma unroll
            for (int w = 0; w < NWK; ++w) sum += redf[(((w * TB + tb) * RB + jb) * 64 + ln) * 4 + ii];
            hout[static_cast<size_t>(sr.tok_pos[t]) * Rp + j] = sum;
        }
    }
}

// -------------------------------------------------------------- epilogue --

// Workgroup: 256 threads, 16 columns; thread (t, 4 columns).
template <int DT, int RB>
__global__ __launch_bounds__(256) void k_decode_epilogue(ApplyArgs a, DecodeArgs d) {
    using E = Elem<DT>;
    using raw = typename E::raw;
    constexpr int HR = RB * 16;
    __shared__ float hs[DECODE_MAX_T][HR + 1];
    __shared__ int s_rec[SMAX_SEG][4];
    const int tid = threadIdx.x;
    const int T = a.T;
    const int Rp = a.R;
    const int n0 = blockIdx.x * 16;
    const int t = tid >> 2;
    const int c4 = (tid & 3) * 4;
    const int tc = min(t, T - 1);

    // Round 1: the splits' partial sums, routing records, h parts.
    float4 pv[MAX_DSPLIT];
#pragma unroll
    for (int qq = 0; qq < MAX_DSPLIT; ++qq)
        if (qq < d.splits)
            pv[qq] = *reinterpret_cast<const float4 *>(d.part + (static_cast<size_t>(qq) * T + tc) * a.d_out + n0 + c4);
    const int seg = a.rv.tok_seg[tc];
    const int pos = a.rv.tok_pos[tc];
    const int n_rec = min(T, a.S) + 2;
    for (int i = tid; i < 4 * n_rec; i += 256) s_rec[i >> 2][i & 3] = a.rv.segs[i];
    const size_t pstride = static_cast<size_t>(T) * Rp;
    for (int e = tid; e < T * Rp / 4; e += 256) {
        float4 hv = reinterpret_cast<const float4 *>(a.h)[e];
        for (int qq = 1; qq < d.splits; ++qq) {
            const float4 g = reinterpret_cast<const float4 *>(a.h + qq * pstride)[e];
            hv.x += g.x;
            hv.y += g.y;
            hv.z += g.z;
            hv.w += g.w;
        }
        const int p = (e * 4) / Rp, j = (e * 4) % Rp;
        hs[p][j] = hv.x;
        hs[p][j + 1] = hv.y;
        hs[p][j + 2] = hv.z;
        hs[p][j + 3] = hv.w;
    }
    __syncthreads();
    if (t >= T) return;
    float4 acc = pv[0];
#pragma unroll
    for (int qq = 1; qq < MAX_DSPLIT; ++qq) {
        if (qq < d.splits) {
            acc.x += pv[qq].x;
            acc.y += pv[qq].y;
            acc.z += pv[qq].z;
            acc.w += pv[qq].w;
        }
    }
    float o[4] = {acc.x, acc.y, acc.z, acc.w};
    const int key = s_rec[seg][0];
    // Round 2, FUSED rows: s * h . B for the thread's 4 columns.
    if (key < a.S && s_rec[seg][3] == SEG_FUSED) {
        u32x4_t bw[4][2 * RB];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint16_t *bp =
                static_cast<const uint16_t *>(a.B_slab) + (static_cast<size_t>(key) * a.d_out + n0 + c4 + u) * Rp;
#pragma unroll
            for (int qb = 0; qb < 2 * RB; ++qb) bw[u][qb] = *reinterpret_cast<const u32x4_t *>(bp + min(8 * qb, Rp - 8));
        }
        const float s = a.slots[key].scale;
        const float *hrow = hs[pos];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float dsum = 0.0f;
#pragma unroll
            for (int qb = 0; qb < 2 * RB; ++qb) {
                if (8 * qb < Rp) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        dsum += hrow[8 * qb + 2 * e] * E::to_f(static_cast<raw>(bw[u][qb][e] & 0xFFFFu));
                        dsum += hrow[8 * qb + 2 * e + 1] * E::to_f(static_cast<raw>(bw[u][qb][e] >> 16));
                    }
                }
            }
            o[u] += s * dsum;
        }
    }
    raw ov[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) ov[u] = (key == a.S + 1) ? E::qnan : E::from_f(o[u]);
    *reinterpret_cast<uint2 *>(static_cast<raw *>(a.y) + static_cast<size_t>(t) * a.d_out + n0 + c4) =
        uint2{static_cast<uint32_t>(ov[0]) | (static_cast<uint32_t>(ov[1]) << 16),
              static_cast<uint32_t>(ov[2]) | (static_cast<uint32_t>(ov[3]) << 16)};
}

template <int DT, int TB>
hipError_t launch_gemm_tb(const ApplyArgs &a, const DecodeArgs &d, const int32_t *idx, const RouteOut &out,
                          hipStream_t st, LaunchEvents ev) {
    const dim3 grid((a.d_out / DCOLS) * d.splits);
    const dim3 block(NWK * 64);
    switch ((a.R + 15) / 16) {
        case 1: LORA_LAUNCH(ev, (k_decode_gemm<DT, TB, 1>), grid, block, 0, st, a, d, idx, out); break;
        case 2: LORA_LAUNCH(ev, (k_decode_gemm<DT, TB, 2>), grid, block, 0, st, a, d, idx, out); break;
        case 3: LORA_LAUNCH(ev, (k_decode_gemm<DT, TB, 3>), grid, block, 0, st, a, d, idx, out); break;
        default: LORA_LAUNCH(ev, (k_decode_gemm<DT, TB, 4>), grid, block, 0, st, a, d, idx, out); break;
    }
    return hipGetLastError();
}

template <int DT>
hipError_t launch_gemm_dt(const ApplyArgs &a, const DecodeArgs &d, const int32_t *idx, const RouteOut &out,
                          hipStream_t st, LaunchEvents ev) {
    switch (decode_token_blocks(a.T)) {
        case 1: return launch_gemm_tb<DT, 1>(a, d, idx, out, st, ev);
        case 2: return launch_gemm_tb<DT, 2>(a, d, idx, out, st, ev);
        default: return launch_gemm_tb<DT, 4>(a, d, idx, out, st, ev);
    }
}

template <int DT>
hipError_t launch_epi_dt(const ApplyArgs &a, const DecodeArgs &d, hipStream_t st) {
    const dim3 grid(a.d_out / 16);
    switch ((a.R + 15) / 16) {
        case 1: hipLaunchKernelGGL((k_decode_epilogue<DT, 1>), grid, dim3(256), 0, st, a, d); break;
        case 2: hipLaunchKernelGGL((k_decode_epilogue<DT, 2>), grid, dim3(256), 0, st, a, d); break;
        case 3: hipLaunchKernelGGL((k_decode_epilogue<DT, 3>), grid, dim3(256), 0, st, a, d); break;
        default: hipLaunchKernelGGL((k_decode_epilogue<DT, 4>), grid, dim3(256), 0, st, a, d); break;
    }
    return hipGetLastError();
}

}  // namespace

int decode_token_blocks(int T) {
    int tb = 1;
    while (tb * 16 < T) tb *= 2;
    return tb;
}

int decode_splits(int T, int d_in) {
    // Every wave holds all its steps: at most NWK x DSTEPS_PER_WAVE k steps
    // per split, at least 4 splits (64-column workgroups: d_out / 16 of them
    // at d_out = 4096, one per CU); 0 beyond MAX_DSPLIT splits.
    (void)T;
    const int kst = d_in / 32;
    const int per = NWK * DSTEPS_PER_WAVE;
    int s = (kst + per - 1) / per;
    if (s < 4) s = 4;
    if (s > kst) s = kst;  // every split keeps at least one k step
    return s <= MAX_DSPLIT ? s : 0;
}

hipError_t launch_decode_gemm(const ApplyArgs &a, const DecodeArgs &d, const int32_t *idx, const RouteOut &out,
                              hipStream_t st, LaunchEvents ev) {
    return (a.dtype == DT_F16) ? launch_gemm_dt<DT_F16>(a, d, idx, out, st, ev)
                               : launch_gemm_dt<DT_BF16>(a, d, idx, out, st, ev);
}

hipError_t launch_decode_epilogue(const ApplyArgs &a, const DecodeArgs &d, hipStream_t st) {
    return (a.dtype == DT_F16) ? launch_epi_dt<DT_F16>(a, d, st) : launch_epi_dt<DT_BF16>(a, d, st);
}

}  // namespace lora
