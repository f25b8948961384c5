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
#include "internal.hpp"

namespace lora {

namespace {

constexpr int RT = 1024;
constexpr int RW = RT / 64;
constexpr int KEY_CAP = 32768;   // tokens whose keys stay in LDS (2 bytes each)
constexpr int IDX_UNROLL = 4;    // index loads per thread in flight
constexpr int ONE_PASS_T = RT * IDX_UNROLL;  // calls routed in one pass

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

__global__ __launch_bounds__(RT) void k_route(const int32_t *__restrict__ idx, int T, int S,
                                               const SlotDev *__restrict__ slots, int R,
                                               int policy, int theta, RouteOut out) {
    __shared__ int s_cnt[MAX_KEYS];
    __shared__ int s_off[MAX_KEYS];
    __shared__ int s_run[MAX_KEYS];
    __shared__ int s_seg[MAX_KEYS];
    __shared__ int s_tile[MAX_KEYS];
    __shared__ unsigned short s_wc[RW][MAX_KEYS];
    __shared__ int s_tot[4];  // buckets, tiles, fused buckets, separate buckets
    __shared__ int s_rows[2]; // padded rows, true rows
    __shared__ unsigned char s_act[MAX_KEYS];     // slot k is ACTIVE
    __shared__ unsigned short s_rank[MAX_KEYS];   // slot k's true rank
    __shared__ unsigned short s_key[KEY_CAP];     // token -> key (T <= KEY_CAP)

    const int K = S + 2;
    const gptr<int32_t> o_counts = global(out.counts), o_offsets = global(out.offsets), o_perm = global(out.perm),
                        o_segs = global(out.segs), o_pos_seg = global(out.pos_seg), o_tok_pos = global(out.tok_pos),
                        o_tok_seg = global(out.tok_seg), o_tiles = global(out.tiles);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    const bool one_pass = T <= ONE_PASS_T;
    // Tokens per wave in one pass (a multiple of 64), and this lane's tokens:
    // wave w's range, 64 at a time (one pass), or chunk-strided (chunks).
    const int nsub = (T + RT - 1) / RT;  // 0 .. IDX_UNROLL in one pass
    auto tok = [&](int u) { return one_pass ? wave * 64 * nsub + u * 64 + lane : u * RT + tid; };

    // The first round of token indices and every slot's state and rank are
    // requested together, before the LDS set-up, in one round trip.  (T = 0:
    // no index is read.)
    int vi[IDX_UNROLL] = {};
    if (T > 0) {
#pragma unroll
        for (int u = 0; u < IDX_UNROLL; ++u) vi[u] = idx[min(tok(u), T - 1)];
        if (out.idx_copy != nullptr) {
#pragma unroll
            for (int u = 0; u < IDX_UNROLL; ++u)
                if ((!one_pass || u < nsub) && tok(u) < T) out.idx_copy[tok(u)] = vi[u];
        }
    }
    for (int k = tid; k < S; k += RT) {
        const SlotDev sd = slots[k];
        s_act[k] = sd.state == SLOT_ACTIVE;
        s_rank[k] = static_cast<unsigned short>(sd.rank);
    }
    for (int k = tid; k < K; k += RT) {
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
        for (int k = tid; k < K; k += RT) {
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
    } else {
        // Keys.  Every index is read once (IDX_UNROLL per thread in flight); a
        // token's key is an LDS lookup of its slot's state, kept in LDS for the
        // scatter when T <= KEY_CAP.  The histogram adds one count per distinct
        // key per wave: the lanes that share a key are found with one ballot per
        // key bit and the lowest of them adds their number (one LDS atomic per
        // key, instead of one per token: a wave of one adapter's tokens would
        // otherwise serialise 64 atomics on one address).
        for (int t0 = 0; t0 < T; t0 += RT * IDX_UNROLL) {
            if (t0 > 0) {
#pragma unroll
                for (int u = 0; u < IDX_UNROLL; ++u) vi[u] = idx[min(t0 + u * RT + tid, T - 1)];
                if (out.idx_copy != nullptr) {
#pragma unroll
                    for (int u = 0; u < IDX_UNROLL; ++u)
                        if (t0 + u * RT + tid < T) out.idx_copy[t0 + u * RT + tid] = vi[u];
                }
            }
#pragma unroll
            for (int u = 0; u < IDX_UNROLL; ++u) {
                if (t0 + u * RT >= T) break;  // (uniform) no token in this round
                const int t = t0 + u * RT + tid;
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
    for (int k = tid; k < K; k += RT) {
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
    if (out.tiles != nullptr) {
        for (int j = RT - 1 - tid; j < s_tot[1]; j += RT) {
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
                o_perm[pos] = t;
                if (out.pos_seg != nullptr) o_pos_seg[pos] = s_seg[key];
                if (out.tok_pos != nullptr) o_tok_pos[t] = pos;
                if (out.tok_seg != nullptr) o_tok_seg[t] = s_seg[key];
            }
        }
    }

    // Stable scatter, one chunk of RT tokens at a time.
    for (int c0 = 0; !one_pass && c0 < T; c0 += RT) {
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
        for (int k = tid; k < K; k += RT) {
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
    if (tid == 0) {
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

}  // namespace

hipError_t launch_route(const int32_t *idx, int T, int S, const SlotDev *slots, int R, int policy,
                        int theta, const RouteOut &out, hipStream_t st, hipEvent_t done) {
    LORA_LAUNCH((LaunchEvents{nullptr, done}), k_route, dim3(1), dim3(RT), 0, st, idx, T, S, slots, R, policy, theta,
                out);
    return hipGetLastError();
}

}  // namespace lora
