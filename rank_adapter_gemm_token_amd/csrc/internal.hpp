// internal.hpp -- device-side records and kernel launchers shared by api.cpp
// and the .hip kernel files of liblora.so.  Not part of the public ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

namespace lora {

// Device slot entry, written by the host at register / unregister time and
// read by the routing kernel.  state: SLOT_FREE or SLOT_ACTIVE.
enum : int32_t { SLOT_FREE = 0, SLOT_ACTIVE = 1 };
struct SlotDev {
    int32_t state;
    int32_t rank;   // the adapter's true rank
    float scale;    // alpha / rank, fp32
    int32_t pad;
};

// Statistics of the last routed call, written by the routing kernel.
struct DevStats {
    int32_t tokens;
    int32_t lora_buckets;
    int32_t fused_buckets;
    int32_t separate_buckets;
    int32_t base_only_tokens;
    int32_t invalid_tokens;
    int32_t rows_padded;   // sum over LoRA tokens of R
    int32_t rows_true;     // sum over LoRA tokens of r_i
};

// Rows per routing tile: LoRA buckets are cut into tiles of this many sorted
// rows for the shrink and separate-expand kernels.
constexpr int TILE_ROWS = 16;
constexpr int MAX_KEYS = 1024 + 2;

// Where routing writes.  The first five arrays are the public routing outputs
// (lora_route); the rest are internal to lora_apply.
struct RouteOut {
    int32_t *counts;    // [S+2]
    int32_t *offsets;   // [S+3]
    int32_t *perm;      // [T]   sorted position -> token
    int32_t *segs;      // [(S+2)*4] {key, start, len, mode}
    int32_t *n_seg;     // [1]
    int32_t *pos_seg;   // [T]   sorted position -> bucket record index
    int32_t *tok_pos;   // [T]   token -> sorted position (may be null)
    int32_t *tok_seg;   // [T]   token -> bucket record index (may be null)
    int32_t *tiles;     // [max_tiles*2] {bucket, first row} of LoRA-bucket tiles
    int32_t *n_tiles;   // [1]
    DevStats *stats;    // [1]   may be null
    unsigned long long *err;  // invalid-token counter, may be null
    int32_t *idx_copy;  // [T]   copy of the token indices as read (may be null)
};

// Routing inputs and the epilogue's view of it.
struct RouteView {
    const int32_t *perm;
    const int32_t *pos_seg;
    const int32_t *tok_pos;
    const int32_t *tok_seg;
    const int32_t *segs;
    const int32_t *tiles;
    const int32_t *n_tiles;
};

// Upper bound of the number of LoRA-bucket tiles of a T-token call.
// A bucket tile's first word: its bucket record in the low 16 bits, the
// slot's true rank above them (shrink and expand skip the rank blocks past
// it: those A rows and B columns are zero).
__host__ __device__ inline int tile_pack(int seg, int rank) { return seg | (rank << 16); }
__host__ __device__ inline int tile_seg(int v) { return v & 0xFFFF; }
__host__ __device__ inline int tile_rank(int v) { return v >> 16; }

inline int max_tiles(int T, int S) {
    return (T + TILE_ROWS - 1) / TILE_ROWS + (S < T ? S : T);
}

// ---- launchers (return the launch's hipError_t) ----

hipError_t launch_route(const int32_t *idx, int T, int S, const SlotDev *slots, int R,
                        int policy, int theta, const RouteOut &out, hipStream_t st, hipEvent_t done = nullptr);

// Copy a user adapter into slot `slot` of the slabs, zero-padding rank..R-1.
// A_user [rank][d_in], B_user [d_out][rank]; slab A [S][R][d_in], slab B
// [S][d_out][R].  esz = element bytes (2 or 4); the copy is bitwise.
hipError_t launch_pad_copy(const void *A_user, const void *B_user, void *A_slab, void *B_slab,
                           int slot, int rank, int R, int d_in, int d_out, int esz,
                           hipStream_t st);

// Write slot-table entry `slot` (one thread, on stream st).
hipError_t launch_set_slot(SlotDev *slots, int slot, SlotDev ent, hipStream_t st);

struct ApplyArgs {
    int dtype;          // lora_dtype
    int T, d_in, d_out, S;
    int R;              // slab rank: the pool's max_rank rounded up to a multiple of 8
    const void *x;      // [T][d_in]
    const void *W;      // [d_out][d_in]
    void *y;            // [T][d_out]
    const void *A_slab; // [S][R][d_in]
    const void *B_slab; // [S][d_out][R]
    const SlotDev *slots;
    float *h;           // h_parts x [T][R] fp32; h = sum of the parts
    int h_parts;        // k parts of h the consumers read and add in order
    int shrink_parts;   // k parts the shrink computes (= h_parts, or more when
                        // the grouped shrink adds its parts into part 0 itself)
    int shrink_g;       // bucket tiles per shrink workgroup (1 or SHRINK_G)
    unsigned *cnt;      // per-group counters of the grouped shrink (0 between calls)
    int h_by_token;     // 1: h rows are indexed by token; 0: by sorted position
    RouteView rv;
    int tiles_bound;    // grid bound for tile-parallel kernels
    int policy;         // lora_mode
};

hipError_t launch_shrink(const ApplyArgs &a, hipStream_t st);
hipError_t launch_shrink16(const ApplyArgs &a, hipStream_t st);
// The routing and the fp16/bf16 shrink (one bucket tile a workgroup) in one
// launch: every workgroup routes the call into its own LDS, workgroup 0
// writes `out` as launch_route does (R, theta as there).  For calls of at
// most ROUTE_SHRINK_MAX_T tokens whose shrink grid (a.tiles_bound x
// a.shrink_parts) is at most ROUTE_SHRINK_MAX_WGS workgroups: each of them
// repeats the routing, so a larger grid would repeat it over more rounds.
constexpr int ROUTE_SHRINK_MAX_T = 1024;
constexpr int ROUTE_SHRINK_MAX_WGS = 512;
hipError_t launch_route_shrink16(const ApplyArgs &a, const int32_t *idx, int R, int theta, const RouteOut &out,
                                 hipStream_t st);
// k parts of the fp16/bf16 shrink on the tiled path (h_parts) for a call of
// at most `tiles` bucket tiles; consumers add the parts in order.
constexpr int MAX_HPARTS = 8;
// Calls of at least SHRINK_G_MIN_T tokens group SHRINK_G bucket tiles per
// shrink workgroup (shrink_group(T) = SHRINK_G, else 1).
constexpr int SHRINK_G = 4;
constexpr int SHRINK_G_MIN_T = 1024;
// Calls of at least SHRINK_G_MIN_T tokens whose tile groups fit `counters`
// use the grouped shrink: its k parts (tiled_h_parts) are added into part 0
// by the shrink itself, and the consumers read one part.
int shrink_group(int T, int tiles, int counters);
int tiled_h_parts(int d_in, int R, int tiles, int T);
hipError_t launch_expand_sep16(const ApplyArgs &a, hipStream_t st);
// Optional timing events of one launch: when `start` is set, the kernel is
// launched with hipExtLaunchKernelGGL, which records both events from the
// dispatch itself (the kernel's own device time, no inter-launch gap).
// Events bound to a launch's dispatch (hipExtLaunchKernelGGL): start and stop
// time one kernel; `done`, when set, is recorded by the completion of the
// launcher's last kernel, in place of a separate event record after it (a
// record is one more packet for the command processor, about 1 us of device
// time between calls on MI355X).
struct LaunchEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
    hipEvent_t done = nullptr;
};

#define LORA_LAUNCH(ev, kernel, grid, block, shmem, st, ...)                                             \
    do {                                                                                                \
        if ((ev).start || (ev).stop)                                                                    \
            hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, (ev).start, (ev).stop, 0u, __VA_ARGS__); \
        else                                                                                            \
            hipLaunchKernelGGL(kernel, grid, block, shmem, st, __VA_ARGS__);                            \
    } while (0)

// Calls of at most DECODE_MAX_T tokens (fp16/bf16), two launches: the
// split-K base GEMM with the shrink (partial sums and h parts, h by token),
// then the epilogue, which routes (writes `out`), sums the splits, adds the
// fused expand, rounds and stores.
constexpr int DECODE_MAX_T = 64;
constexpr int MAX_DSPLIT = 16;
struct DecodeArgs {
    int splits;         // k splits = h parts (decode_splits)
    int max_rank;       // the pool's rank, for the padded-row statistic
    int theta;          // fused threshold
    float *part;        // fp32 partial sums, [splits][d_out/16][TB][64 lanes] fragments
};
// ev (optional) times the GEMM launch.
hipError_t launch_decode(const ApplyArgs &a, const DecodeArgs &d, const int32_t *idx, const RouteOut &out,
                         hipStream_t st, LaunchEvents ev = {});
// The decode epilogue's routing alone (1 <= T <= DECODE_MAX_T): writes every
// array of `out` that launch_route writes, counts and offsets included, and
// the same values (both are the stable counting sort of the keys).
hipError_t launch_route_small(const int32_t *idx, int T, int S, const SlotDev *slots, int max_rank, int policy,
                              int theta, const RouteOut &out, hipStream_t st);
// k splits of the decode GEMM for (T, d_in); 0 if d_in is too large for it.
int decode_splits(int T, int d_in, int d_out);
int decode_token_blocks(int T);
// Larger calls (fp16/bf16): LDS-tiled MFMA GEMM with the fused expand.
// Calls of 65 .. 2047 tokens run 256-row tiles of `bn` columns with k split
// `splits` ways, plus a LoRA workgroup per tile when lora_wg (tiled_plan;
// splits 0: another kernel).  Tiles of more than one contributor keep their
// fp32 partial sums in `part` (tiled_part_bytes) and one counter per tile in
// `cnt` (tiled_split_tiles of them, 0 between calls: the last contributor of
// a tile resets its counter).
constexpr int MAX_TSPLIT = 8;
constexpr int MAX_SPLIT_TILES = 16384;
// When the tiles leave at least 64 CUs idle, the split GEMM also runs the
// shrink, on `shrink_wgs` extra workgroups (fuse_parts = the k parts P of h
// it computes; 0: a shrink launch precedes the GEMM).
struct TiledPlan {
    int bn;
    int splits;
    int lora_wg;         // 1: a LoRA workgroup per tile computes the fused expand
    int fuse_parts;
    int shrink_wgs;
};
TiledPlan tiled_plan(int T, int d_in, int d_out);
size_t tiled_part_bytes(int T, int d_in, int d_out);
int tiled_split_tiles(int T, int d_in, int d_out);
// k parts of h for a call of T tokens on the tiled path: the fused shrink's,
// or tiled_h_parts (tiles: the call's bound of bucket tiles).
int tiled_call_h_parts(int T, int d_in, int d_out, int R, int tiles);
struct SplitSpace {
    float *part = nullptr;
    unsigned *cnt = nullptr;
    int max_tiles = 0;   // counters available at cnt
    unsigned *sync = nullptr;  // [2] the fused shrink's counters (0 between calls)
    int wait_polls = -1;       // the fused shrink's consumer poll bound (-1: the default)
};
struct SplitArgs {
    int splits;
    int lora_wg;
    int tiles;           // output tiles (row tiles x tiles_x)
    int tiles_x;         // column tiles
    float *part;
    unsigned *cnt;
    int shrink_wgs;      // fused shrink: shrink workgroups after the tiles' contributors
    unsigned *sync;      // fused shrink: [units counted, workgroups done]
    int wait_polls;      // fused shrink: polls of the count before a consumer computes h itself
};
hipError_t launch_gemm_tiled(const ApplyArgs &a, const SplitSpace &ws, hipStream_t st, LaunchEvents ev = {});
// The static per-device workspace of lora_apply_noalloc (scratch.hip):
// scratch_setup resolves its device address once per device (call with that
// device current); scratch_device_ptr returns it (nullptr before set-up).
// The array's first SCRATCH_COUNTER_BYTES hold the split tiles' counters
// (zeroed at set-up, 0 between calls): scratch_split_counters; the per-call
// workspace is carved from scratch_device_ptr, the rest.
// The two counters after the split tiles' are the fused shrink's
// (SplitSpace::sync); the block stays a multiple of 256 bytes.
constexpr size_t SCRATCH_COUNTER_BYTES = static_cast<size_t>(MAX_SPLIT_TILES + 64) * 4;
hipError_t scratch_setup(int device);
char *scratch_device_ptr(int device);
unsigned *scratch_split_counters(int device);
// fp32 pools: VALU base GEMM and residual expand.
hipError_t launch_base_gemm(const ApplyArgs &a, hipStream_t st);
hipError_t launch_expand_separate(const ApplyArgs &a, hipStream_t st);

}  // namespace lora
