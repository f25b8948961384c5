// shrink_expand.hip -- the LoRA shrink h = x A_slot^T and the separate
// residual expand y += s h B_slot^T, for fp16/bf16 pools.
//
// A maps hidden size to rank and B maps rank to hidden size ("LLM 多 LoRA 推理服务
// 工程 2026", routing layer, zero-pad paragraph).  The separate school runs the
// LoRA product after the base linear as a residual add, at the price of one
// more launch and one more round trip of y (same page, execution-unit
// paragraph).
//
// Shrink: one workgroup of 4 waves per 16-row tile of one adapter bucket
// (shrink_role): the tile's x rows are the MFMA A operand, the slot's
// rank-padded A rows the B operand; K is split over the waves and the
// partial sums are added in LDS in a fixed order: h (fp32, by sorted row).
// The decode path runs the same role inside its main kernel.
//
// Separate expand: one workgroup of 4 waves per (tile of a SEPARATE bucket,
// 64 columns); acc = s * h . B on MFMA, then y = round(y + acc).
#include <algorithm>

#include "epilogue.hpp"

namespace lora {

namespace {

template <int DT, int RB>
__global__ __launch_bounds__(256) void k_shrink(ApplyArgs a) {
    __shared__ u32x4_t lds[4 * RB * 64];
    // Unit (tile, k part): part-major within a tile.
    shrink_role<DT, RB, 4>(a, blockIdx.x / a.h_parts, blockIdx.x % a.h_parts, lds);
}

template <int DT>
__global__ __launch_bounds__(256) void k_expand_sep(ApplyArgs a) {
    using E = Elem<DT>;
    using raw = typename E::raw;
    const int tile = blockIdx.x;
    if (tile >= uniform(*a.rv.n_tiles)) return;
    const int seg = uniform(tile_seg(a.rv.tiles[2 * tile]));
    if (uniform(a.rv.segs[4 * seg + 3]) != SEG_SEPARATE) return;
    const int row0 = uniform(a.rv.tiles[2 * tile + 1]);
    const int end = uniform(a.rv.segs[4 * seg + 1] + a.rv.segs[4 * seg + 2]);
    const int rows_end = min(row0 + TILE_ROWS, end);
    const int wave = uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;
    const int kq = lane >> 4;
    const int n0 = blockIdx.y * 64 + wave * 16;
    f32x4_t acc[1][1] = {{f32x4_t{0.f, 0.f, 0.f, 0.f}}};
    RowFacts<1> f;
    row_facts<1>(a, row0, rows_end, f);
    lora_expand_mfma<DT, 1, 1>(a, row0, rows_end, n0, SEG_SEPARATE, f, acc);
    raw *y = static_cast<raw *>(a.y);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int tok = __shfl(f.tok[0], kq * 4 + i, 64);
        const int p = row0 + kq * 4 + i;
        if (p >= rows_end) continue;
        raw *yp = y + static_cast<size_t>(tok) * a.d_out + n0 + r;
        *yp = E::from_f(E::to_f(*yp) + acc[0][0][i]);
    }
}

template <int DT>
hipError_t shrink_rb(const ApplyArgs &a, hipStream_t st) {
    const dim3 grid(a.tiles_bound * a.h_parts);
    switch ((a.R + 15) / 16) {
        case 1: hipLaunchKernelGGL((k_shrink<DT, 1>), grid, dim3(256), 0, st, a); break;
        case 2: hipLaunchKernelGGL((k_shrink<DT, 2>), grid, dim3(256), 0, st, a); break;
        case 3: hipLaunchKernelGGL((k_shrink<DT, 3>), grid, dim3(256), 0, st, a); break;
        default: hipLaunchKernelGGL((k_shrink<DT, 4>), grid, dim3(256), 0, st, a); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_shrink16(const ApplyArgs &a, hipStream_t st) {
    return (a.dtype == DT_F16) ? shrink_rb<DT_F16>(a, st) : shrink_rb<DT_BF16>(a, st);
}

int tiled_h_parts(int d_in, int R, int tiles) {
    // With few tiles (a few workgroups per CU at most) each wave's chain of
    // dependent load rounds sets the time: split k until each wave has about
    // one round (U k steps as in shrink_unit: 16, 8 or 4 for 1, 2, 3-4 rank
    // blocks) or the grid reaches ~512 workgroups.  With many tiles the
    // chip is full already and extra parts only add h traffic.
    if (tiles >= 256) return 1;
    const int rb = (R + 15) / 16;
    const int u = rb == 1 ? 16 : rb == 2 ? 8 : 4;
    const int kst = d_in / 32;
    int p = (kst + 4 * u - 1) / (4 * u);
    p = std::min(p, (512 + tiles - 1) / tiles);
    return std::max(1, std::min(p, MAX_HPARTS));
}

hipError_t launch_expand_sep16(const ApplyArgs &a, hipStream_t st) {
    const dim3 grid(a.tiles_bound, a.d_out / 64);
    if (a.dtype == DT_F16)
        hipLaunchKernelGGL(k_expand_sep<DT_F16>, grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(k_expand_sep<DT_BF16>, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace lora
