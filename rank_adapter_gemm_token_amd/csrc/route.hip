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
// One workgroup of 1024 threads (16 wave64s) handles any T: the tokens are
// processed in chunks of 1024.  Within a chunk, each wave finds the lanes that
// share its key with one ballot per key bit (wave64 has no match-any), ranks
// a lane among its peers with a popcount of the lower-lane mask, and
// publishes per-wave key counts in LDS; a lane's sorted position is
//   offset[key] + (tokens of key in earlier chunks) + (in earlier waves) + rank.
// Ties therefore keep ascending token order, which makes the result unique.
#include "internal.hpp"

namespace lora {

namespace {

constexpr int RT = 1024;
constexpr int RW = RT / 64;
constexpr int KEY_CAP = 32768;   // tokens whose keys stay in LDS (2 bytes each)
constexpr int IDX_UNROLL = 4;    // index loads per thread in flight

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
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // The first round of token indices and every slot's state and rank are
    // requested together, before the LDS set-up, in one round trip.  (T = 0:
    // no index is read.)
    int vi[IDX_UNROLL] = {};
    if (T > 0) {
#pragma unroll
        for (int u = 0; u < IDX_UNROLL; ++u) vi[u] = idx[min(u * RT + tid, T - 1)];
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

    // Keys.  Every index is read once (IDX_UNROLL per thread in flight); a
    // token's key is an LDS lookup of its slot's state, kept in LDS for the
    // scatter when T <= KEY_CAP.  The histogram adds one count per distinct
    // key per wave: the lanes that share a key are found with one ballot per
    // key bit and the lowest of them adds their number (one LDS atomic per
    // key, instead of one per token: a wave of one adapter's tokens would
    // otherwise serialise 64 atomics on one address).
    const bool keep = T <= KEY_CAP;
    const int nbits = 32 - __clz(K);  // enough bits for keys 0..K (K = pad lanes)
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int t0 = 0; t0 < T; t0 += RT * IDX_UNROLL) {
        if (t0 > 0) {
#pragma unroll
            for (int u = 0; u < IDX_UNROLL; ++u) vi[u] = idx[min(t0 + u * RT + tid, T - 1)];
        }
#pragma unroll
        for (int u = 0; u < IDX_UNROLL; ++u) {
            if (t0 + u * RT >= T) break;  // (uniform) no token in this round
            const int t = t0 + u * RT + tid;
            const bool v = t < T;
            const int key = !v ? K
                               : ((vi[u] == -1) ? S : ((vi[u] >= 0 && vi[u] < S && s_act[vi[u]]) ? vi[u] : S + 1));
            if (v && keep) s_key[t] = static_cast<unsigned short>(key);
            unsigned long long peers = ~0ull;
            for (int b = 0; b < nbits; ++b) {
                const int bit = (key >> b) & 1;
                const unsigned long long m = __ballot(bit);
                peers &= bit ? m : ~m;
            }
            // integer LDS atomics: counts do not depend on order
            if (v && (peers & below) == 0) atomicAdd(&s_cnt[key], __popcll(peers));
        }
    }
    __syncthreads();

    // Exclusive scans over keys of: counts, non-empty flags, LoRA tiles.
    // Wave 0; each lane owns a contiguous run of keys.
    if (wave == 0) {
        const int per = (K + 63) / 64;
        const int k0 = min(lane * per, K);
        const int k1 = min(k0 + per, K);
        int c = 0, z = 0, tl = 0;
        for (int k = k0; k < k1; ++k) {
            const int n = s_cnt[k];
            c += n;
            z += (n > 0);
            tl += (k < S) ? (n + TILE_ROWS - 1) / TILE_ROWS : 0;
        }
        int ic = c, iz = z, it = tl;
        for (int d = 1; d < 64; d <<= 1) {
            const int a = __shfl_up(ic, d, 64);
            const int b = __shfl_up(iz, d, 64);
            const int e = __shfl_up(it, d, 64);
            if (lane >= d) {
                ic += a;
                iz += b;
                it += e;
            }
        }
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
        }
    }
    __syncthreads();

    // Per-key outputs: counts, offsets, bucket records, tiles.
    for (int k = tid; k < K; k += RT) {
        const int n = s_cnt[k];
        out.counts[k] = n;
        out.offsets[k] = s_off[k];
        if (k == K - 1) out.offsets[K] = s_off[k] + n;
        if (n > 0) {
            int mode = 0;  // LORA_SEG_NONE
            if (k < S) {
                mode = (policy == 1) ? 1 : (policy == 2) ? 2 : (n > theta ? 1 : 2);
                atomicAdd(&s_tot[mode == 1 ? 2 : 3], 1);
                atomicAdd(&s_rows[0], n * R);
                atomicAdd(&s_rows[1], n * s_rank[k]);
                if (out.tiles != nullptr) {
                    const int nt = (n + TILE_ROWS - 1) / TILE_ROWS;
                    for (int j = 0; j < nt; ++j) {
                        out.tiles[2 * (s_tile[k] + j)] = tile_pack(s_seg[k], s_rank[k]);
                        out.tiles[2 * (s_tile[k] + j) + 1] = s_off[k] + j * TILE_ROWS;
                    }
                }
            }
            int32_t *rec = out.segs + 4 * s_seg[k];
            rec[0] = k;
            rec[1] = s_off[k];
            rec[2] = n;
            rec[3] = mode;
        }
    }

    // Stable scatter, one chunk of RT tokens at a time.
    for (int c0 = 0; c0 < T; c0 += RT) {
        const int t = c0 + tid;
        const bool v = t < T;
        const int key = !v ? K : (keep ? static_cast<int>(s_key[t]) : key_of(idx[t], S, slots));
        unsigned long long peers = ~0ull;
        for (int b = 0; b < nbits; ++b) {
            const int bit = (key >> b) & 1;
            const unsigned long long m = __ballot(bit);
            peers &= bit ? m : ~m;
        }
        const int rk = __popcll(peers & below);
        if (v && rk == 0) s_wc[wave][key] = static_cast<unsigned short>(__popcll(peers));
        __syncthreads();
        if (v) {
            int prior = s_run[key];
            for (int w = 0; w < wave; ++w) prior += s_wc[w][key];
            const int pos = s_off[key] + prior + rk;
            if (pos >= 0 && pos < T) {  // always true; keeps a logic error in bounds
                out.perm[pos] = t;
                if (out.pos_seg != nullptr) out.pos_seg[pos] = s_seg[key];
                if (out.tok_pos != nullptr) out.tok_pos[t] = pos;
                if (out.tok_seg != nullptr) out.tok_seg[t] = s_seg[key];
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
        *out.n_seg = s_tot[0];
        if (out.n_tiles != nullptr) *out.n_tiles = s_tot[1];
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
                        int theta, const RouteOut &out, hipStream_t st) {
    hipLaunchKernelGGL(k_route, dim3(1), dim3(RT), 0, st, idx, T, S, slots, R, policy, theta, out);
    return hipGetLastError();
}

}  // namespace lora
