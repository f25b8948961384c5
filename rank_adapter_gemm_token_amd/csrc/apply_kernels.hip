// apply_kernels.hip -- the fp32 pools' path (VALU, one thread per output):
// LoRA shrink, base projection with the fused LoRA expand in its epilogue, and
// the separate residual expand.  fp16/bf16 pools use the MFMA kernels of
// gemm_decode.hip, gemm_tiled.hip and shrink_expand.hip.
//
// "LLM 多 LoRA 推理服务工程 2026", four-layer runtime, execution-unit paragraph:
// the base linear and the LoRA A/B products either run in one launch (fused)
// or the base runs alone and the LoRA term is added afterwards as a residual
// (separate: one more launch and one more round trip of y through memory).
// Routing (route.hip) sorts the tokens by adapter first, so every kernel here
// works on sorted rows: row p is token perm[p], and rows of one adapter are
// contiguous.
//
//   shrink   h[p][j] = sum_k x[perm[p]][k] * A_slot[j][k]         (fp32, by row)
//   base     acc[p][n] = sum_k x[perm[p]][k] * W[n][k]            (fp32 accum)
//            FUSED bucket:    y = round(acc + s * sum_j h[p][j] B_slot[n][j])
//            SEPARATE bucket: y = round(acc), later y = round(y + s * ...)
//            base_only:       y = round(acc);  invalid: y = NaN
//
// The scale s = alpha / r (true rank) is applied in fp32.  Every reduction runs
// in a fixed order that depends only on (T, d_in, d_out, dtype), never on the
// batch's composition or a row's position, so a token's row is bitwise
// independent of the other tokens under a forced fused/separate policy.
#include "dtype.hpp"
#include "internal.hpp"

namespace lora {

namespace {

constexpr int SEG_FUSED = 1;
constexpr int SEG_SEPARATE = 2;

// Token of sorted row p.  Routing writes every perm[p], p < T, with a token
// < T; the clamp only keeps a logic error from addressing outside x and y.
__device__ __forceinline__ int token_at(const ApplyArgs &a, int p) {
    return min(max(a.rv.perm[p], 0), a.T - 1);
}

// Epilogue for one output element of sorted row `row`, column `col`.
template <int DT>
__device__ __forceinline__ void finish(const ApplyArgs &a, int row, int col, float v) {
    using E = Elem<DT>;
    using raw = typename E::raw;
    const int seg = a.rv.pos_seg[row];
    const int key = a.rv.segs[4 * seg];
    const int mode = a.rv.segs[4 * seg + 3];
    const int t = token_at(a, row);
    raw *yp = static_cast<raw *>(a.y) + static_cast<size_t>(t) * a.d_out + col;
    if (key == a.S + 1) {
        *yp = E::qnan;
        return;
    }
    if (key < a.S && mode == SEG_FUSED) {
        const float *hr = a.h + static_cast<size_t>(row) * a.R;
        const raw *br = static_cast<const raw *>(a.B_slab) +
                        (static_cast<size_t>(key) * a.d_out + col) * a.R;
        float d = 0.0f;
        for (int j = 0; j < a.R; ++j) d += hr[j] * E::to_f(br[j]);
        v += a.slots[key].scale * d;
    }
    *yp = E::from_f(v);
}

// ---------------------------------------------------------------- shrink --

// fp32 pools: one thread per (row, rank index) of the tile, sequential k.
__global__ __launch_bounds__(256) void k_shrink_f32(ApplyArgs a) {
    const int tile = blockIdx.x;
    if (tile >= *a.rv.n_tiles) return;
    const int seg = tile_seg(a.rv.tiles[2 * tile]);
    const int row0 = a.rv.tiles[2 * tile + 1];
    const int key = a.rv.segs[4 * seg];
    const int end = a.rv.segs[4 * seg + 1] + a.rv.segs[4 * seg + 2];
    const int rows = min(TILE_ROWS, end - row0);
    const float *x = static_cast<const float *>(a.x);
    const float *A = static_cast<const float *>(a.A_slab);
    for (int q = threadIdx.x; q < TILE_ROWS * a.R; q += blockDim.x) {
        const int row = q / a.R;
        const int j = q - row * a.R;
        if (row >= rows) continue;
        const int t = token_at(a, row0 + row);
        const float *xr = x + static_cast<size_t>(t) * a.d_in;
        const float *ar = A + (static_cast<size_t>(key) * a.R + j) * a.d_in;
        float acc = 0.0f;
        for (int k = 0; k < a.d_in; ++k) acc = fmaf(xr[k], ar[k], acc);
        a.h[static_cast<size_t>(row0 + row) * a.R + j] = acc;
    }
}

// ------------------------------------------------------------- base GEMM --

// fp32 pools: one thread per output element, sequential k.
__global__ __launch_bounds__(256) void k_gemm_f32(ApplyArgs a) {
    const int col = blockIdx.x * 256 + threadIdx.x;
    const int row = blockIdx.y;
    if (col >= a.d_out) return;
    const int t = token_at(a, row);
    const float *xr = static_cast<const float *>(a.x) + static_cast<size_t>(t) * a.d_in;
    const float *wr = static_cast<const float *>(a.W) + static_cast<size_t>(col) * a.d_in;
    float acc = 0.0f;
    for (int k = 0; k < a.d_in; ++k) acc = fmaf(xr[k], wr[k], acc);
    finish<DT_F32>(a, row, col, acc);
}

// ------------------------------------------------------ separate expand --

// One workgroup per (LoRA tile, 256 columns); only SEPARATE buckets work:
// y = round(y + s * sum_j h[p][j] * B_slot[n][j]).
template <int DT>
__global__ __launch_bounds__(256) void k_expand_separate(ApplyArgs a) {
    using E = Elem<DT>;
    using raw = typename E::raw;
    const int tile = blockIdx.x;
    if (tile >= *a.rv.n_tiles) return;
    const int seg = tile_seg(a.rv.tiles[2 * tile]);
    const int row0 = a.rv.tiles[2 * tile + 1];
    const int key = a.rv.segs[4 * seg];
    const int end = a.rv.segs[4 * seg + 1] + a.rv.segs[4 * seg + 2];
    const int mode = a.rv.segs[4 * seg + 3];
    if (mode != SEG_SEPARATE) return;
    const int col = blockIdx.y * 256 + threadIdx.x;
    if (col >= a.d_out) return;
    const int row1 = min(row0 + TILE_ROWS, end);
    const raw *br = static_cast<const raw *>(a.B_slab) + (static_cast<size_t>(key) * a.d_out + col) * a.R;
    const float s = a.slots[key].scale;
    for (int row = row0; row < row1; ++row) {
        const int t = token_at(a, row);
        const float *hr = a.h + static_cast<size_t>(row) * a.R;
        float d = 0.0f;
        for (int j = 0; j < a.R; ++j) d += hr[j] * E::to_f(br[j]);
        raw *yp = static_cast<raw *>(a.y) + static_cast<size_t>(t) * a.d_out + col;
        *yp = E::from_f(E::to_f(*yp) + s * d);
    }
}

}  // namespace

hipError_t launch_shrink(const ApplyArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(k_shrink_f32, dim3(a.tiles_bound), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_base_gemm(const ApplyArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(k_gemm_f32, dim3((a.d_out + 255) / 256, a.T), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_expand_separate(const ApplyArgs &a, hipStream_t st) {
    const dim3 grid(a.tiles_bound, (a.d_out + 255) / 256);
    hipLaunchKernelGGL(k_expand_separate<DT_F32>, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace lora
