// route.hip -- routing pass of the adapter execution unit: per-token key
// histogram, exclusive scan and stable scatter (a counting sort by adapter),
// then one bucket record per non-empty key and the tile list of the LoRA
// buckets.  Integer-only, bit-exact.
//
// Bucketing by adapter within one call is the adapter-level bucket of the
// two-level bucketing in "LLM 多 LoRA 推理服务工程 2026", routing layer; a bucket
// above the threshold runs fused, otherwise separate (same paragraph).  A token
// with a missing mapping goes to an error bucket, never to another adapter
// ("Multi-LoRA 在线服务隔离", request identity section).
//
// One workgroup of 1024 threads (16 wave64s) handles any T.  A wave finds the
// lanes that share its key with one ballot per key bit (wave64 has no
// match-any) and ranks a lane among its peers with a popcount of the
// lower-lane mask.
//
// Calls of at most 4096 tokens take one pass: wave w owns the contiguous
// token range [w n, (w + 1) n), n = 64 ceil(T / 1024), walks it 64 tokens at
// a time and keeps a running count per key in LDS, so a token's rank within
// its wave's range is the count before its group plus its rank among its
// peers.  One prefix over the 16 waves per key then gives the histogram and
// each wave's start within the key, one scan over keys the offsets, and a
// token's sorted position is
//   offset[key] + (tokens of key in earlier waves) + (rank within its wave).
// Three barriers in all.  Longer calls take chunks of 1024 tokens after a
// histogram over all of them:
//   offset[key] + (tokens of key in earlier chunks) + (in earlier waves) + rank.
// Either way ties keep ascending token order, which makes the result unique.
//
// Calls of at most 1024 tokens that route in the call and shrink in a launch
// of their own (fp16/bf16, one bucket tile a workgroup, at most 512
// workgroups) route inside the shrink launch instead (k_route_shrink): every
// shrink workgroup of 256 threads derives the whole routing into its own LDS
// with the same one-pass code at 4 waves, reads its bucket tile from it and
// runs the shrink unit; workgroup 0 also writes the routing arrays for the
// later kernels.  No workgroup waits for another, and the arrays are the
// ones k_route writes (the order is unique).
#include "epilogue.hpp"
#include "internal.hpp"

namespace lora {

namespace {

constexpr int RT = 1024;          // threads of k_route
constexpr int KEY_CAP = 32768;   // tokens whose keys stay in LDS (2 bytes each)
constexpr int IDX_UNROLL = 4;    // index loads per thread in flight
constexpr int RS_T = 256;        // threads of k_route_shrink
constexpr int RS_MAX_T = RS_T * IDX_UNROLL;  // its calls (one pass)
static_assert(RS_MAX_T == ROUTE_SHRINK_MAX_T, "k_route_shrink routes its calls in one pass");

// Global-memory views of the output pointers.  Stores through a generic
// pointer may alias LDS in the compiler's eyes, so every later LDS read would
// wait for them to complete; through these they need not.
template <typename T>
using gptr = __attribute__((address_space(1))) T *;
template <typename T>
__device__ __forceinline__ gptr<T> global(T *p) { return (gptr<T>)p; }

// Inclusive prefix sum across the 64 lanes of a wave in DPP steps: shifts by
// 1, 2, 4 and 8 lanes within each row of 16, then row 0's last lane into
// rows 1 and 3, then lane 31 into rows 2 and 3.  Lanes a step has no source
// for add 0.
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}

// The lanes of this wave whose key equals this lane's: one ballot when the
// whole wave holds one key (a sequence's tokens), else one ballot per key bit.
__device__ __forceinline__ unsigned long long key_peers(int key, int nbits) {
    const int k0 = __builtin_amdgcn_readfirstlane(key);
    if (__ballot(key != k0) == 0) return ~0ull;
    unsigned long long peers = ~0ull;
    for (int b = 0; b < nbits; ++b) {
        const int bit = (key >> b) & 1;
        const unsigned long long m = __ballot(bit);
        peers &= bit ? m : ~m;
    }
    return peers;
}

__device__ __forceinline__ int key_of(int32_t v, int S, const SlotDev *__restrict__ slots) {
    if (v == -1) return S;
    if (v >= 0 && v < S && slots[v].state == SLOT_ACTIVE) return v;
    return S + 1;
}

// Routing state in LDS for NT threads; the per-token key store only when
// calls longer than one pass are routed (MULTI).
template <int NT, bool MULTI>
struct RouteLds {
    int cnt[MAX_KEYS];
    int off[MAX_KEYS];
    int run[MAX_KEYS];
    int seg[MAX_KEYS];
    int tile[MAX_KEYS];
    unsigned short wc[NT / 64][MAX_KEYS];
    int tot[4];   // buckets, tiles, fused buckets, separate buckets
    int rows[2];  // padded rows, true rows
    unsigned char act[MAX_KEYS];    // slot k is ACTIVE
    unsigned short rank[MAX_KEYS];  // slot k's true rank
    unsigned short key[MULTI ? KEY_CAP : 1];  // token -> key (T <= KEY_CAP)
};

// The routing of one call by one workgroup of NT threads.  publish: write the
// arrays of `out` (else only L is filled); perm_lds (when not null): the
// sorted position -> token map also in LDS.  Without MULTI, T <= NT *
// IDX_UNROLL (one pass).  Ends with a barrier: L (and perm_lds) are complete.
template <int NT, bool MULTI>
__device__ __forceinline__ void route_body(const int32_t *__restrict__ idx, int T, int S,
                                           const SlotDev *__restrict__ slots, int R, int policy, int theta,
                                           const RouteOut &out, RouteLds<NT, MULTI> &L, bool publish,
                                           int *perm_lds) {
    constexpr int RW = NT / 64;
    constexpr int ONE_PASS_T = NT * IDX_UNROLL;  // calls routed in one pass
    auto &s_cnt = L.cnt;
    auto &s_off = L.off;
    auto &s_run = L.run;
    auto &s_seg = L.seg;
    auto &s_tile = L.tile;
    auto &s_wc = L.wc;
    auto &s_tot = L.tot;
    auto &s_rows = L.rows;
    auto &s_act = L.act;
    auto &s_rank = L.rank;
    auto &s_key = L.key;
    const int K = S + 2;
    const gptr<int32_t> o_counts = global(out.counts), o_offsets = global(out.offsets), o_perm = global(out.perm),
                        o_segs = global(out.segs), o_pos_seg = global(out.pos_seg), o_tok_pos = global(out.tok_pos),
                        o_tok_seg = global(out.tok_seg), o_tiles = global(out.tiles);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    const bool one_pass = !MULTI || T <= ONE_PASS_T;
    // Tokens per wave in one pass (a multiple of 64), and this lane's tokens:
    // wave w's range, 64 at a time (one pass), or chunk-strided (chunks).
    const int nsub = (T + NT - 1) / NT;  // 0 .. IDX_UNROLL in one pass
    auto tok = [&](int u) { return one_pass ? wave * 64 * nsub + u * 64 + lane : u * NT + tid; };

    // The first round of token indices and every slot's state and rank are
    // requested together, before the LDS set-up, in one round trip.  (T = 0:
    // no index is read.)
    int vi[IDX_UNROLL] = {};
    if (T > 0) {
#pragma unroll
        for (int u = 0; u < IDX_UNROLL; ++u) vi[u] = idx[min(tok(u), T - 1)];
        if (publish && out.idx_copy != nullptr) {
#pragma unroll
            for (int u = 0; u < IDX_UNROLL; ++u)
                if ((!one_pass || u < nsub) && tok(u) < T) out.idx_copy[tok(u)] = vi[u];
        }
    }
    for (int k = tid; k < S; k += NT) {
        const SlotDev sd = slots[k];
        s_act[k] = sd.state == SLOT_ACTIVE;
        s_rank[k] = static_cast<unsigned short>(sd.rank);
    }
    for (int k = tid; k < K; k += NT) {
        s_cnt[k] = 0;
        s_run[k] = 0;
        for (int w = 0; w < RW; ++w) s_wc[w][k] = 0;
    }
    if (tid < 4) s_tot[tid] = 0;
    if (tid < 2) s_rows[tid] = 0;
    __syncthreads();

    const bool keep = T <= KEY_CAP;
    const int nbits = 32 - __clz(K);  // enough bits for keys 0..K (K = pad lanes)
    const unsigned long long below = (1ull << lane) - 1ull;
    // One pass: this lane's keys and ranks within its wave's range.
    int okey[IDX_UNROLL] = {};
    int orank[IDX_UNROLL] = {};
    if (one_pass) {
        // Each group of 64 tokens in order: a token's rank is the wave's
        // running count of its key so far plus its rank among its peers;
        // the lowest of the peers then advances the count.  The count is
        // read by every peer before it is written (the LDS wait between).
#pragma unroll
        for (int u = 0; u < IDX_UNROLL; ++u) {
            if (u >= nsub) break;  // (uniform)
            const int t = tok(u);
            const bool v = t < T;
            const int key = !v ? K
                               : ((vi[u] == -1) ? S : ((vi[u] >= 0 && vi[u] < S && s_act[vi[u]]) ? vi[u] : S + 1));
            const unsigned long long peers = key_peers(key, nbits);
            const int rk = __popcll(peers & below);
            const int run = v ? static_cast<int>(s_wc[wave][key]) : 0;
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (v && rk == 0) s_wc[wave][key] = static_cast<unsigned short>(run + __popcll(peers));
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            okey[u] = key;
            orank[u] = run + rk;
        }
        __syncthreads();
        // Per key: the waves' counts become each wave's start within the key
        // (exclusive prefix in wave order), their sum the key's count.
        for (int k = tid; k < K; k += NT) {
            int c[RW];
#pragma unroll
            for (int w = 0; w < RW; ++w) c[w] = s_wc[w][k];
            int run = 0;
#pragma unroll
            for (int w = 0; w < RW; ++w) {
                s_wc[w][k] = static_cast<unsigned short>(run);
                run += c[w];
            }
            s_cnt[k] = run;
        }
    } else if constexpr (MULTI) {
        // Keys.  Every index is read once (IDX_UNROLL per thread in flight); a
        // token's key is an LDS lookup of its slot's state, kept in LDS for the
        // scatter when T <= KEY_CAP.  The histogram adds one count per distinct
        // key per wave: the lanes that share a key are found with one ballot per
        // key bit and the lowest of them adds their number (one LDS atomic per
        // key, instead of one per token: a wave of one adapter's tokens would
        // otherwise serialise 64 atomics on one address).
        for (int t0 = 0; t0 < T; t0 += NT * IDX_UNROLL) {
            if (t0 > 0) {
#pragma unroll
                for (int u = 0; u < IDX_UNROLL; ++u) vi[u] = idx[min(t0 + u * NT + tid, T - 1)];
                if (out.idx_copy != nullptr) {
#pragma unroll
                    for (int u = 0; u < IDX_UNROLL; ++u)
                        if (t0 + u * NT + tid < T) out.idx_copy[t0 + u * NT + tid] = vi[u];
                }
            }
#pragma unroll
            for (int u = 0; u < IDX_UNROLL; ++u) {
                if (t0 + u * NT >= T) break;  // (uniform) no token in this round
                const int t = t0 + u * NT + tid;
                const bool v = t < T;
                const int key = !v ? K
                                   : ((vi[u] == -1) ? S : ((vi[u] >= 0 && vi[u] < S && s_act[vi[u]]) ? vi[u] : S + 1));
                if (v && keep) s_key[t] = static_cast<unsigned short>(key);
                const unsigned long long peers = key_peers(key, nbits);
                // integer LDS atomics: counts do not depend on order
                if (v && (peers & below) == 0) atomicAdd(&s_cnt[key], __popcll(peers));
            }
        }
    }
    __syncthreads();

    // Exclusive scans over keys of: counts, non-empty flags, LoRA tiles; and
    // the statistics (fused and separate buckets, padded and true rows).
    // Wave 0; each lane owns a contiguous run of keys.
    if (wave == 0) {
        const int per = (K + 63) / 64;
        const int k0 = min(lane * per, K);
        const int k1 = min(k0 + per, K);
        int c = 0, z = 0, tl = 0, nf = 0, ns = 0, rp = 0, rt = 0;
        for (int k = k0; k < k1; ++k) {
            const int n = s_cnt[k];
            c += n;
            z += (n > 0);
            if (k < S && n > 0) {
                tl += (n + TILE_ROWS - 1) / TILE_ROWS;
                const int mode = (policy == 1) ? 1 : (policy == 2) ? 2 : (n > theta ? 1 : 2);
                nf += mode == 1;
                ns += mode == 2;
                rp += n * R;
                rt += n * s_rank[k];
            }
        }
        // Inclusive scans across the wave (the statistics' totals end in
        // lane 63).
        const int ic = wave_incl_scan(c), iz = wave_incl_scan(z), it = wave_incl_scan(tl);
        nf = wave_incl_scan(nf);
        ns = wave_incl_scan(ns);
        rp = wave_incl_scan(rp);
        rt = wave_incl_scan(rt);
        int ec = ic - c, ez = iz - z, et = it - tl;
        for (int k = k0; k < k1; ++k) {
            const int n = s_cnt[k];
            s_off[k] = ec;
            s_seg[k] = (n > 0) ? ez : -1;
            s_tile[k] = et;
            ec += n;
            ez += (n > 0);
            et += (k < S) ? (n + TILE_ROWS - 1) / TILE_ROWS : 0;
        }
        if (lane == 63) {
            s_tot[0] = iz;
            s_tot[1] = it;
            s_tot[2] = nf;
            s_tot[3] = ns;
            s_rows[0] = rp;
            s_rows[1] = rt;
        }
    }
    __syncthreads();

    // Per-key outputs: counts, offsets, bucket records.
    for (int k = tid; publish && k < K; k += NT) {
        const int n = s_cnt[k];
        o_counts[k] = n;
        o_offsets[k] = s_off[k];
        if (k == K - 1) o_offsets[K] = s_off[k] + n;
        if (n > 0) {
            int mode = 0;  // LORA_SEG_NONE
            if (k < S) mode = (policy == 1) ? 1 : (policy == 2) ? 2 : (n > theta ? 1 : 2);
            const gptr<int32_t> rec = o_segs + 4 * s_seg[k];
            rec[0] = k;
            rec[1] = s_off[k];
            rec[2] = n;
            rec[3] = mode;
        }
    }

    // Tiles of the LoRA buckets, one thread each (numbered from the last
    // wave down, so that the waves writing the per-key outputs above are
    // mostly others): tile j belongs to the last key k < S whose first tile
    // index s_tile[k] is at most j (keys without tiles share their
    // successor's index and are passed over).
    if (publish && out.tiles != nullptr) {
        for (int j = NT - 1 - tid; j < s_tot[1]; j += NT) {
            int lo = 0, hi = S;  // the first key whose first tile is past j
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (s_tile[mid] <= j) lo = mid + 1;
                else hi = mid;
            }
            const int k = lo - 1;
            o_tiles[2 * j] = tile_pack(s_seg[k], s_rank[k]);
            o_tiles[2 * j + 1] = s_off[k] + (j - s_tile[k]) * TILE_ROWS;
        }
    }

    // One pass: every token's sorted position from its wave's start within
    // the key and its rank within the wave.
    if (one_pass) {
#pragma unroll
        for (int u = 0; u < IDX_UNROLL; ++u) {
            if (u >= nsub) break;  // (uniform)
            const int t = tok(u);
            if (t >= T) continue;
            const int key = okey[u];
            const int pos = s_off[key] + s_wc[wave][key] + orank[u];
            if (pos >= 0 && pos < T) {  // always true; keeps a logic error in bounds
                if (perm_lds != nullptr) perm_lds[pos] = t;
                if (publish) {
                    o_perm[pos] = t;
                    if (out.pos_seg != nullptr) o_pos_seg[pos] = s_seg[key];
                    if (out.tok_pos != nullptr) o_tok_pos[t] = pos;
                    if (out.tok_seg != nullptr) o_tok_seg[t] = s_seg[key];
                }
            }
        }
    }

    // Stable scatter, one chunk of NT tokens at a time (k_route only).
    for (int c0 = 0; MULTI && !one_pass && c0 < T; c0 += NT) {
        const int t = c0 + tid;
        const bool v = t < T;
        const int key = !v ? K : (keep ? static_cast<int>(s_key[t]) : key_of(idx[t], S, slots));
        const unsigned long long peers = key_peers(key, nbits);
        const int rk = __popcll(peers & below);
        if (v && rk == 0) s_wc[wave][key] = static_cast<unsigned short>(__popcll(peers));
        __syncthreads();
        if (v) {
            int prior = s_run[key];
            for (int w = 0; w < wave; ++w) prior += s_wc[w][key];
            const int pos = s_off[key] + prior + rk;
            if (pos >= 0 && pos < T) {  // always true; keeps a logic error in bounds
                o_perm[pos] = t;
                if (out.pos_seg != nullptr) o_pos_seg[pos] = s_seg[key];
                if (out.tok_pos != nullptr) o_tok_pos[t] = pos;
                if (out.tok_seg != nullptr) o_tok_seg[t] = s_seg[key];
            }
        }
        __syncthreads();
        for (int k = tid; k < K; k += NT) {
            int add = 0;
            for (int w = 0; w < RW; ++w) {
                add += s_wc[w][k];
                s_wc[w][k] = 0;
            }
            s_run[k] += add;
        }
        __syncthreads();
    }

    __syncthreads();
    if (publish && tid == 0) {
        *global(out.n_seg) = s_tot[0];
        if (out.n_tiles != nullptr) *global(out.n_tiles) = s_tot[1];
        if (out.stats != nullptr) {
            DevStats st;
            st.tokens = T;
            st.lora_buckets = s_tot[2] + s_tot[3];
            st.fused_buckets = s_tot[2];
            st.separate_buckets = s_tot[3];
            st.base_only_tokens = s_cnt[S];
            st.invalid_tokens = s_cnt[S + 1];
            st.rows_padded = s_rows[0];
            st.rows_true = s_rows[1];
            *out.stats = st;
        }
        if (out.err != nullptr && s_cnt[S + 1] > 0)
            atomicAdd(out.err, static_cast<unsigned long long>(s_cnt[S + 1]));
    }
}

__global__ __launch_bounds__(RT) void k_route(const int32_t *__restrict__ idx, int T, int S,
                                               const SlotDev *__restrict__ slots, int R,
                                               int policy, int theta, RouteOut out) {
    __shared__ RouteLds<RT, true> L;
    route_body<RT, true>(idx, T, S, slots, R, policy, theta, out, L, true, nullptr);
}

// Routing and shrink in one launch, for calls of at most RS_MAX_T tokens:
// unit (tile, k part) per workgroup as k_shrink, each workgroup routing the
// whole call first (route_body into its own LDS, workgroup 0 publishing the
// arrays), then finding its tile there as the routing's tile list does.
template <int DT, int RB>
__global__ __launch_bounds__(RS_T) void k_route_shrink(const int32_t *__restrict__ idx, int R, int theta,
                                                       RouteOut out, ApplyArgs a) {
    __shared__ RouteLds<RS_T, false> L;
    __shared__ int s_perm[RS_MAX_T];
    __shared__ u32x4_t lds[4 * RB * 64];
    const int S = a.S;
    route_body<RS_T, false>(idx, a.T, S, a.slots, R, a.policy, theta, out, L, blockIdx.x == 0, s_perm);
    const int tile = blockIdx.x / a.shrink_parts;
    const int part = blockIdx.x % a.shrink_parts;
    if (tile >= L.tot[1]) return;
    // The last key k < S whose first tile index is at most `tile`.
    int lo = 0, hi = S;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (L.tile[mid] <= tile) lo = mid + 1;
        else hi = mid;
    }
    const int key = lo - 1;
    const int row0 = L.off[key] + (tile - L.tile[key]) * TILE_ROWS;
    const int rows = min(TILE_ROWS, L.off[key] + L.cnt[key] - row0);
    // Rank blocks that hold the slot's true rank.
    const int nrb = uniform(min(RB, (static_cast<int>(L.rank[key]) + 15) / 16));
    if (RB >= 4 && nrb == 4) shrink_unit<DT, (RB >= 4 ? 4 : 1), 4>(a, key, row0, rows, s_perm, part, lds);
    else if (RB >= 3 && nrb == 3) shrink_unit<DT, (RB >= 3 ? 3 : 1), 4>(a, key, row0, rows, s_perm, part, lds);
    else if (RB >= 2 && nrb == 2) shrink_unit<DT, (RB >= 2 ? 2 : 1), 4>(a, key, row0, rows, s_perm, part, lds);
    else shrink_unit<DT, 1, 4>(a, key, row0, rows, s_perm, part, lds);
}

template <int DT>
hipError_t route_shrink_rb(const ApplyArgs &a, dim3 grid, const int32_t *idx, int R, int theta, const RouteOut &out,
                           hipStream_t st) {
    switch ((a.R + 15) / 16) {
        case 1: hipLaunchKernelGGL((k_route_shrink<DT, 1>), grid, dim3(RS_T), 0, st, idx, R, theta, out, a); break;
        case 2: hipLaunchKernelGGL((k_route_shrink<DT, 2>), grid, dim3(RS_T), 0, st, idx, R, theta, out, a); break;
        case 3: hipLaunchKernelGGL((k_route_shrink<DT, 3>), grid, dim3(RS_T), 0, st, idx, R, theta, out, a); break;
        default: hipLaunchKernelGGL((k_route_shrink<DT, 4>), grid, dim3(RS_T), 0, st, idx, R, theta, out, a); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const int32_t *idx, int T, int S, const SlotDev *slots, int R, int policy,
                        int theta, const RouteOut &out, hipStream_t st, hipEvent_t done) {
    LORA_LAUNCH((LaunchEvents{nullptr, done}), k_route, dim3(1), dim3(RT), 0, st, idx, T, S, slots, R, policy, theta,
                out);
    return hipGetLastError();
}

hipError_t launch_route_shrink16(const ApplyArgs &a, const int32_t *idx, int R, int theta, const RouteOut &out,
                                 hipStream_t st) {
    const long wgs = static_cast<long>(a.tiles_bound) * a.shrink_parts;
    if (a.T < 1 || a.T > RS_MAX_T || a.S < 1 || a.S > MAX_KEYS - 2 || a.shrink_g != 1 || a.shrink_parts < 1 ||
        a.h_by_token != 0 || a.d_in % 32 != 0 || a.tiles_bound != max_tiles(a.T, a.S) || wgs > ROUTE_SHRINK_MAX_WGS)
        return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(wgs));
    return a.dtype == DT_F16 ? route_shrink_rb<DT_F16>(a, grid, idx, R, theta, out, st)
                             : route_shrink_rb<DT_BF16>(a, grid, idx, R, theta, out, st);
}

}  // namespace lora
