// apply_kernels.hip -- LoRA shrink, base projection with the fused LoRA expand
// in its epilogue, and the separate residual expand.
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

// One wave per 16-row tile of one LoRA bucket; MFMA 16x16x32 with the tile's
// x rows as the A operand and the slot's A rows (rank index j) as the B
// operand.  RB = ceil(R / 16) blocks of 16 rank columns.
template <int DT, int RB>
__global__ __launch_bounds__(64) void k_shrink_mfma(ApplyArgs a) {
    using E = Elem<DT>;
    using V = typename E::vec8;
    const int tile = blockIdx.x;
    if (tile >= *a.rv.n_tiles) return;
    const int seg = a.rv.tiles[2 * tile];
    const int row0 = a.rv.tiles[2 * tile + 1];
    const int key = a.rv.segs[4 * seg];
    const int end = a.rv.segs[4 * seg + 1] + a.rv.segs[4 * seg + 2];
    const int rows = min(TILE_ROWS, end - row0);

    const int lane = threadIdx.x & 63;
    const int r = lane & 15;
    const int kq = lane >> 4;
    const bool xv = r < rows;
    const int t = xv ? token_at(a, row0 + r) : 0;
    const uint16_t *xp = static_cast<const uint16_t *>(a.x) + static_cast<size_t>(t) * a.d_in + kq * 8;
    const uint16_t *ap[RB];
    bool av[RB];
#pragma unroll
    for (int cb = 0; cb < RB; ++cb) {
        const int j = cb * 16 + r;
        av[cb] = j < a.R;
        ap[cb] = static_cast<const uint16_t *>(a.A_slab) +
                 (static_cast<size_t>(key) * a.R + (av[cb] ? j : 0)) * a.d_in + kq * 8;
    }
    f32x4_t acc[RB];
#pragma unroll
    for (int cb = 0; cb < RB; ++cb) acc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int k0 = 0; k0 < a.d_in; k0 += 32) {
        const V xa = xv ? load8<V>(xp + k0) : zero8<V>();
#pragma unroll
        for (int cb = 0; cb < RB; ++cb) {
            const V b = av[cb] ? load8<V>(ap[cb] + k0) : zero8<V>();
            acc[cb] = E::mfma(xa, b, acc[cb]);
        }
    }
#pragma unroll
    for (int cb = 0; cb < RB; ++cb) {
        const int j = cb * 16 + r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = kq * 4 + i;
            if (row < rows && j < a.R) a.h[static_cast<size_t>(row0 + row) * a.R + j] = acc[cb][i];
        }
    }
}

// fp32 pools: one thread per (row, rank index) of the tile, sequential k.
__global__ __launch_bounds__(256) void k_shrink_f32(ApplyArgs a) {
    const int tile = blockIdx.x;
    if (tile >= *a.rv.n_tiles) return;
    const int seg = a.rv.tiles[2 * tile];
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

// 64 sorted rows x 64 columns per workgroup of 4 waves; wave w owns columns
// n0 + 16w .. +15 for all four 16-row blocks.  MFMA 16x16x32: x rows are the
// A operand, W rows (output columns) the B operand; both are K-contiguous.
template <int DT>
__global__ __launch_bounds__(256) void k_gemm_mfma(ApplyArgs a) {
    using E = Elem<DT>;
    using V = typename E::vec8;
    const int n0 = blockIdx.x * 64;
    const int m0 = blockIdx.y * 64;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;
    const int kq = lane >> 4;
    const int n = n0 + wave * 16 + r;
    const uint16_t *wp = static_cast<const uint16_t *>(a.W) + static_cast<size_t>(n) * a.d_in + kq * 8;
    const uint16_t *xp[4];
    bool xv[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        const int pos = m0 + rb * 16 + r;
        xv[rb] = pos < a.T;
        const int t = xv[rb] ? token_at(a, pos) : 0;
        xp[rb] = static_cast<const uint16_t *>(a.x) + static_cast<size_t>(t) * a.d_in + kq * 8;
    }
    f32x4_t acc[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) acc[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int k0 = 0; k0 < a.d_in; k0 += 32) {
        const V b = load8<V>(wp + k0);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            const V xa = xv[rb] ? load8<V>(xp[rb] + k0) : zero8<V>();
            acc[rb] = E::mfma(xa, b, acc[rb]);
        }
    }
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = m0 + rb * 16 + kq * 4 + i;
            if (row < a.T) finish<DT>(a, row, n, acc[rb][i]);
        }
    }
}

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
    const int seg = a.rv.tiles[2 * tile];
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

template <int DT>
hipError_t shrink_16(const ApplyArgs &a, hipStream_t st) {
    const dim3 grid(a.tiles_bound);
    const int rb = (a.R + 15) / 16;
    switch (rb) {
        case 1: hipLaunchKernelGGL((k_shrink_mfma<DT, 1>), grid, dim3(64), 0, st, a); break;
        case 2: hipLaunchKernelGGL((k_shrink_mfma<DT, 2>), grid, dim3(64), 0, st, a); break;
        case 3: hipLaunchKernelGGL((k_shrink_mfma<DT, 3>), grid, dim3(64), 0, st, a); break;
        default: hipLaunchKernelGGL((k_shrink_mfma<DT, 4>), grid, dim3(64), 0, st, a); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_shrink(const ApplyArgs &a, hipStream_t st) {
    switch (a.dtype) {
        case DT_F16: return shrink_16<DT_F16>(a, st);
        case DT_BF16: return shrink_16<DT_BF16>(a, st);
        default:
            hipLaunchKernelGGL(k_shrink_f32, dim3(a.tiles_bound), dim3(256), 0, st, a);
            return hipGetLastError();
    }
}

hipError_t launch_base_gemm(const ApplyArgs &a, hipStream_t st) {
    switch (a.dtype) {
        case DT_F16:
            hipLaunchKernelGGL(k_gemm_mfma<DT_F16>, dim3(a.d_out / 64, (a.T + 63) / 64), dim3(256), 0, st, a);
            break;
        case DT_BF16:
            hipLaunchKernelGGL(k_gemm_mfma<DT_BF16>, dim3(a.d_out / 64, (a.T + 63) / 64), dim3(256), 0, st, a);
            break;
        default:
            hipLaunchKernelGGL(k_gemm_f32, dim3((a.d_out + 255) / 256, a.T), dim3(256), 0, st, a);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_expand_separate(const ApplyArgs &a, hipStream_t st) {
    const dim3 grid(a.tiles_bound, (a.d_out + 255) / 256);
    switch (a.dtype) {
        case DT_F16: hipLaunchKernelGGL(k_expand_separate<DT_F16>, grid, dim3(256), 0, st, a); break;
        case DT_BF16: hipLaunchKernelGGL(k_expand_separate<DT_BF16>, grid, dim3(256), 0, st, a); break;
        default: hipLaunchKernelGGL(k_expand_separate<DT_F32>, grid, dim3(256), 0, st, a); break;
    }
    return hipGetLastError();
}

}  // namespace lora
