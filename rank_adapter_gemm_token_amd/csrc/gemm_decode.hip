// gemm_decode.hip -- the decode path (T <= 64 tokens per call, fp16/bf16):
// base projection, LoRA shrink, and the fused LoRA expand.
//
// At decode sizes a call is bound by streaming W (d_out x d_in, read once)
// from HBM; x (T x d_in) is small and reused by every column tile.  Two
// launches after routing:
//
// k_decode_main -- workgroups independent of each other (no cross-workgroup
//   synchronization anywhere), each doing two jobs:
//   * shrink units first, while its GEMM loads are already in flight: a unit
//     is (16-row tile of an adapter bucket, k part); the 8 waves split the
//     part's k steps, each MFMAs its share of x_tile . A_slot^T, and the
//     waves' sums are added in LDS in a fixed order: one part of h (fp32, by
//     sorted row);
//   * the GEMM: 128 output columns (16 per wave, 8 waves) x one k chunk of
//     d_in / splits.  W goes straight from global memory into MFMA operand
//     registers with PF k steps of loads in flight per wave; x rows (token
//     order) are staged in LDS in MFMA fragment order, the next stage loaded
//     while the current one is used.  The fp32 partial sums of the k chunk
//     are stored as MFMA fragments (coalesced) for the epilogue.
// k_decode_epilogue -- 64 columns per workgroup, rows in token order: sums the
//   splits' partials in a fixed order, adds s * h . B for FUSED buckets in
//   fp32 on the VALU (h stays fp32; at T <= 64 this is a few hundred FMAs per
//   lane, and every load is issued in one of three rounds), rounds once, and
//   stores whole 128-byte row segments of y (NaN rows for invalid tokens).
//
// The fused/separate choice of "LLM 多 LoRA 推理服务工程 2026" (four-layer runtime,
// execution-unit paragraph) maps to: FUSED = the LoRA term enters the fp32
// accumulator before the single rounding; SEPARATE = the base is rounded and
// stored, and the residual kernel adds the LoRA term to y afterwards.
// The variant (TB, splits) depends on (T, d_in, d_out) only, so a token's
// result never depends on the rest of the batch.
#include "epilogue.hpp"

namespace lora {

namespace {

constexpr int NW = 8;          // waves per workgroup of the main kernel
constexpr int MAX_SPLITS = 8;  // k chunks of the split-K (decode_splits)
constexpr int MAX_HPARTS = 8;  // k parts of the shrink (decode_h_parts)

template <int TB>
struct DecodeShape {
    // k steps of x staged in LDS per stage (64 KiB of fragments).
    static constexpr int KSS = 64 / TB;
    // W k steps in flight per wave (divides KSS).
    static constexpr int PF = KSS < 16 ? KSS : 16;
    // x fragments each wave stages per stage.
    static constexpr int FPW = TB * KSS / NW;
};

// ------------------------------------------------------------- GEMM role --

template <int DT, int TB, int RB>
__device__ __forceinline__ void gemm_role(const ApplyArgs &a, const DecodeArgs &d, int wg, u32x4_t *xs) {
    using E = Elem<DT>;
    using V = typename E::vec8;
    using Sh = DecodeShape<TB>;
    constexpr int KSS = Sh::KSS;
    constexpr int PF = Sh::PF;
    const int tiles = (a.d_out + 16 * NW - 1) / (16 * NW);
    const int tile = wg % tiles;
    const int c = wg / tiles;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;
    const int kq = lane >> 4;
    const int n0 = tile * 16 * NW + wave * 16;
    const bool wave_on = n0 < a.d_out;  // the last tile may be half used
    const int kbeg = c * d.KC;
    const int ksteps = d.KC / 32;
    const uint16_t *x = static_cast<const uint16_t *>(a.x);

    // This lane's x rows when staging: token tb*16 + r.
    const uint16_t *xr[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
        xr[tb] = (tb * 16 + r < a.T) ? x + static_cast<size_t>(tb * 16 + r) * a.d_in + kbeg + 8 * kq : nullptr;

    // x fragments (tb, ks) of one stage: wave w takes ks = NW*i % KSS + w of
    // token block tb = NW*i / KSS (KSS is a multiple of NW, so tb is known at
    // compile time); fragments past the chunk end are zeros.
    u32x4_t v[Sh::FPW];
    auto load_x = [&](int s0) {
        const int ns = min(KSS, ksteps - s0);
#pragma unroll
        for (int i = 0; i < Sh::FPW; ++i) {
            const int tb = (NW * i) / KSS;
            const int ks = (NW * i) % KSS + wave;
            v[i] = u32x4_t{0u, 0u, 0u, 0u};
            if (ks < ns && xr[tb] != nullptr) v[i] = *reinterpret_cast<const u32x4_t *>(xr[tb] + (s0 + ks) * 32);
        }
    };
    load_x(0);

    // Stream W, PF k steps ahead.  Ring loads are unconditional (the address
    // is clamped to the chunk's last k step; those extra values meet zero x
    // fragments), so no load ever has to complete early to be merged.
    const int nl = wave_on ? n0 : a.d_out - 16;
    const uint16_t *wp = static_cast<const uint16_t *>(a.W) + static_cast<size_t>(nl + r) * a.d_in + kbeg + 8 * kq;
    u32x4_t wr[PF];
#pragma unroll
    for (int u = 0; u < PF; ++u) wr[u] = *reinterpret_cast<const u32x4_t *>(wp + min(u, ksteps - 1) * 32);

    // While those loads are in flight: this workgroup's share of the shrink,
    // units (tile, k part) u = blockIdx.x, blockIdx.x + gridDim.x, ...
    // (LDS xs is free until the x stage is stored.)
    {
        const int n_tiles = *a.rv.n_tiles;
        const int n_units = n_tiles * a.h_parts;
        for (int u = blockIdx.x; u < n_units; u += gridDim.x) {
            shrink_role<DT, RB, NW>(a, u % n_tiles, u / n_tiles, xs);
            __syncthreads();  // the reduction's LDS reads are done
        }
    }

    f32x4_t acc[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int s0 = 0; s0 < ksteps; s0 += KSS) {
        const int ns = min(KSS, ksteps - s0);
#pragma unroll
        for (int i = 0; i < Sh::FPW; ++i) {
            const int tb = (NW * i) / KSS;
            const int ks = (NW * i) % KSS + wave;
            xs[(tb * KSS + ks) * 64 + lane] = v[i];
        }
        __syncthreads();
        if (s0 + KSS < ksteps) load_x(s0 + KSS);  // next stage, in flight during this one
        for (int k0 = 0; k0 < ns; k0 += PF) {
#pragma unroll
            for (int u = 0; u < PF; ++u) {
                const int ks = k0 + u;   // < KSS; steps past ns meet zero x fragments
                const int gk = s0 + ks;  // gk % PF == u: KSS and k0 are multiples of PF
                const V b = __builtin_bit_cast(V, wr[u]);
                wr[u] = *reinterpret_cast<const u32x4_t *>(wp + min(gk + PF, ksteps - 1) * 32);
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    const V xa = __builtin_bit_cast(V, xs[(tb * KSS + ks) * 64 + lane]);
                    acc[tb] = E::mfma(xa, b, acc[tb]);
                }
            }
        }
        __syncthreads();
    }

    // fp32 partial sums of this k chunk as MFMA fragments: [c][n0/16][tb][lane].
    if (!wave_on) return;
    f32x4_t *part = static_cast<f32x4_t *>(d.part) +
                    ((static_cast<size_t>(c) * (a.d_out / 16) + n0 / 16) * TB) * 64 + lane;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) part[tb * 64] = acc[tb];
}

template <int DT, int TB, int RB>
__global__ __launch_bounds__(NW * 64) void k_decode_main(ApplyArgs a, DecodeArgs d) {
    __shared__ u32x4_t lds[TB * DecodeShape<TB>::KSS * 64];
    static_assert(TB * DecodeShape<TB>::KSS >= NW * RB, "shrink reduction must fit");
    gemm_role<DT, TB, RB>(a, d, blockIdx.x, lds);
}

// -------------------------------------------------------------- epilogue --

// Workgroup: 4 waves, 64 columns (16 per wave), all T rows in token order.
template <int DT, int TB, int RB>
__global__ __launch_bounds__(256) void k_decode_epilogue(ApplyArgs a, DecodeArgs d) {
    using E = Elem<DT>;
    using raw = typename E::raw;
    constexpr int TP = TB * 16;     // padded rows
    constexpr int HR = RB * 16;     // padded rank (>= R)
    __shared__ float hs[TP][HR + 1];         // h by sorted row, parts summed
    __shared__ raw ys[TP][64 + 8];           // rounded output tile
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int r = lane & 15;
    const int kq = lane >> 4;
    const int c0 = blockIdx.x * 64;
    const int n = c0 + wave * 16 + r;  // this lane's column
    const int Rp = a.R;
    const f32x4_t *part = static_cast<const f32x4_t *>(d.part) + static_cast<size_t>(n / 16) * TB * 64 + lane;
    const size_t cstride = static_cast<size_t>(a.d_out / 16) * TB * 64;

    // Round 1 (all independent): every split's partial sums, each row's bucket
    // and sorted position, and h (summed over its k parts) into LDS.
    int seg[TB][4], pos[TB][4];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = min(tb * 16 + kq * 4 + i, a.T - 1);
            seg[tb][i] = a.rv.tok_seg[t];
            pos[tb][i] = a.rv.tok_pos[t];
        }
    f32x4_t pv[MAX_SPLITS][TB];
#pragma unroll
    for (int c = 0; c < MAX_SPLITS; ++c)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) pv[c][tb] = part[min(c, d.splits - 1) * cstride + tb * 64];
    {
        // Unrolled over entries and parts with clamped addresses, so every
        // load is issued before the first add.
        const size_t pstride = static_cast<size_t>(a.T) * Rp;
        float hv[TP * HR / 256][MAX_HPARTS];
#pragma unroll
        for (int m = 0; m < TP * HR / 256; ++m) {
            const int e = tid + 256 * m;
            const int p = min(e / HR, a.T - 1), j = min(e % HR, Rp - 1);
            const float *hp = a.h + static_cast<size_t>(p) * Rp + j;
#pragma unroll
            for (int q = 0; q < MAX_HPARTS; ++q) hv[m][q] = hp[min(q, a.h_parts - 1) * pstride];
        }
#pragma unroll
        for (int m = 0; m < TP * HR / 256; ++m) {
            const int e = tid + 256 * m;
            const int p = e / HR, j = e % HR;
            float v = hv[m][0];
#pragma unroll
            for (int q = 1; q < MAX_HPARTS; ++q)
                if (q < a.h_parts) v += hv[m][q];
            hs[p][j] = (p < a.T && j < Rp) ? v : 0.0f;
        }
    }
    f32x4_t acc[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
        acc[tb] = pv[0][tb];
#pragma unroll
        for (int c = 1; c < MAX_SPLITS; ++c)
            if (c < d.splits) acc[tb] += pv[c][tb];
    }
    // Round 2: bucket key and mode of each row.
    int key[TB][4], fused[TB][4];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            key[tb][i] = a.rv.segs[4 * seg[tb][i]];
            fused[tb][i] = key[tb][i] < a.S && a.rv.segs[4 * seg[tb][i] + 3] == SEG_FUSED;
        }
    __syncthreads();  // hs complete

    // Round 3, FUSED rows: acc += s * sum_j h[p][j] * B[key][n][j] in fp32.
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (!fused[tb][i]) continue;
            const int k = key[tb][i];
            const uint16_t *bp = static_cast<const uint16_t *>(a.B_slab) + (static_cast<size_t>(k) * a.d_out + n) * Rp;
            u32x4_t bw[2 * RB];
#pragma unroll
            for (int q = 0; q < 2 * RB; ++q)
                bw[q] = (8 * q < Rp) ? *reinterpret_cast<const u32x4_t *>(bp + 8 * q) : u32x4_t{0u, 0u, 0u, 0u};
            const float s = a.slots[k].scale;
            const float *hrow = hs[pos[tb][i]];
            float dsum = 0.0f;
#pragma unroll
            for (int q = 0; q < 2 * RB; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dsum += hrow[8 * q + 2 * e] * E::to_f(static_cast<raw>(bw[q][e] & 0xFFFFu));
                    dsum += hrow[8 * q + 2 * e + 1] * E::to_f(static_cast<raw>(bw[q][e] >> 16));
                }
            acc[tb][i] += s * dsum;
        }
    }
    // Round once; invalid tokens get NaN; stage the tile for whole-row stores.
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            ys[tb * 16 + kq * 4 + i][wave * 16 + r] = (key[tb][i] == a.S + 1) ? E::qnan : E::from_f(acc[tb][i]);
    __syncthreads();
    // 64 columns x 2 B = 128 B per row: 8 threads x 16 B.
    raw *y = static_cast<raw *>(a.y);
    for (int e = tid; e < a.T * 8; e += 256) {
        const int t = e >> 3, q = e & 7;
        const uint32_t *src = reinterpret_cast<const uint32_t *>(&ys[t][q * 8]);
        *reinterpret_cast<u32x4_t *>(y + static_cast<size_t>(t) * a.d_out + c0 + q * 8) =
            u32x4_t{src[0], src[1], src[2], src[3]};
    }
}

template <int DT, int TB>
hipError_t launch_tb(const ApplyArgs &a, const DecodeArgs &d, hipStream_t st) {
    const int tiles = (a.d_out + 16 * NW - 1) / (16 * NW);
    const dim3 grid(tiles * d.splits);
    const dim3 block(NW * 64);
    switch ((a.R + 15) / 16) {
        case 1: hipLaunchKernelGGL((k_decode_main<DT, TB, 1>), grid, block, 0, st, a, d); break;
        case 2: hipLaunchKernelGGL((k_decode_main<DT, TB, 2>), grid, block, 0, st, a, d); break;
        case 3: hipLaunchKernelGGL((k_decode_main<DT, TB, 3>), grid, block, 0, st, a, d); break;
        default: hipLaunchKernelGGL((k_decode_main<DT, TB, 4>), grid, block, 0, st, a, d); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    switch ((a.R + 15) / 16) {
        case 1: hipLaunchKernelGGL((k_decode_epilogue<DT, TB, 1>), dim3(a.d_out / 64), dim3(256), 0, st, a, d); break;
        case 2: hipLaunchKernelGGL((k_decode_epilogue<DT, TB, 2>), dim3(a.d_out / 64), dim3(256), 0, st, a, d); break;
        case 3: hipLaunchKernelGGL((k_decode_epilogue<DT, TB, 3>), dim3(a.d_out / 64), dim3(256), 0, st, a, d); break;
        default: hipLaunchKernelGGL((k_decode_epilogue<DT, TB, 4>), dim3(a.d_out / 64), dim3(256), 0, st, a, d); break;
    }
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const ApplyArgs &a, const DecodeArgs &d, hipStream_t st) {
    switch (decode_token_blocks(a.T)) {
        case 1: return launch_tb<DT, 1>(a, d, st);
        case 2: return launch_tb<DT, 2>(a, d, st);
        default: return launch_tb<DT, 4>(a, d, st);
    }
}

}  // namespace

int decode_token_blocks(int T) {
    int tb = 1;
    while (tb * 16 < T) tb *= 2;
    return tb;
}

int decode_splits(int T, int d_in, int d_out) {
    (void)T;
    // Enough k chunks for >= 256 workgroups (one per CU), never more than 8.
    const int tiles = (d_out + 16 * NW - 1) / (16 * NW);
    const int kst = d_in / 32;
    int s = 1;
    while (s < MAX_SPLITS && s * tiles < 256 && kst % (2 * s) == 0) s *= 2;
    return s;
}

int decode_h_parts(int d_in) {
    // About 2 k steps per shrink wave (8 waves per part), at most 8 parts.
    const int p = d_in / 32 / 16;
    return p < 1 ? 1 : (p > MAX_HPARTS ? MAX_HPARTS : p);
}

hipError_t launch_gemm_decode(const ApplyArgs &a, const DecodeArgs &d, hipStream_t st) {
    return (a.dtype == DT_F16) ? launch_dt<DT_F16>(a, d, st) : launch_dt<DT_BF16>(a, d, st);
}

}  // namespace lora
