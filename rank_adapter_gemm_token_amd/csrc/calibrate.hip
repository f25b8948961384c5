// calibrate.hip -- achievable-peak probes for the measurement harness.
//
// Not part of the library's call path: libcalibrate.so holds two plain
// kernels that set what this GPU reaches outside the method, so that a
// kernel's roofline fraction can be read against the spec peak and against
// what the part actually delivers.
//
//   calib_read  streams a device buffer once (16-byte non-temporal loads,
//               four in flight per lane, grid-stride); the bytes it reads
//               over its time are the achievable HBM read rate.
//   calib_mfma  runs a register-only loop of v_mfma_f32_16x16x32_{f16,bf16}
//               (eight independent accumulators per wave); its FLOPs over
//               its time are the achievable dense 16-bit MFMA rate.
//   calib_l2read  has every workgroup stream the same small window (a few
//               MiB, resident in each XCD's L2 after the first pass) with
//               16-byte loads, the way a GEMM's column tiles all re-read one
//               activation block; the bytes the CUs take in over its time
//               are the achievable L2-to-CU rate.
//
// Both write one word only when their data-dependent result hits a value it
// never takes, so the work cannot be dropped and nothing else is written.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <type_traits>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int kChains = 8;

__global__ __launch_bounds__(kThreads) void k_read(const u32x4 *__restrict__ p, size_t n16, uint32_t *sink) {
    const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
    size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
    const uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (r == 0x9e3779b9u) sink[0] = r;
}

// Workgroup b reads the window `reps` times, starting b * 64 KiB in (mod the
// window) so that the workgroups spread over the L2 channels; each pass is
// grid-stride over the workgroup's lanes, four loads in flight per lane.
__global__ __launch_bounds__(kThreads) void k_l2read(const u32x4 *__restrict__ p, size_t win16, int reps,
                                                     uint32_t *sink) {
    const size_t start = (static_cast<size_t>(blockIdx.x) * 4096) % win16;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int rep = 0; rep < reps; ++rep) {
        for (size_t i = threadIdx.x; i < win16; i += kUnroll * kThreads) {
            u32x4 v[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                size_t j = start + i + u * kThreads;
                j = j >= win16 ? j - win16 : j;
                j = j >= win16 ? j - win16 : j;
                v[u] = p[j];
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
        }
    }
    const uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (r == 0x9e3779b9u) sink[0] = r;
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_mfma(int iters, float *sink) {
    using V = typename std::conditional<BF16, bf16x8, f16x8>::type;
    using S = typename std::conditional<BF16, __bf16, _Float16>::type;
    const int lane = threadIdx.x & 63;
    V a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = static_cast<S>(static_cast<float>((lane + e) & 7) * 0.125f);
        b[e] = static_cast<S>(static_cast<float>((lane * 3 + e) & 7) * 0.0625f);
    }
    f32x4 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) {
            if constexpr (BF16)
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
            else
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += acc[c].x + acc[c].y + acc[c].z + acc[c].w;
    if (s == -1.0f) sink[0] = s;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) at `buf` once with `blocks` workgroups of
// 256 lanes on `stream`.  Returns the HIP status of the launch.
int calib_read(const void *buf, size_t bytes, uint32_t *sink, int blocks, void *stream) {
    if (buf == nullptr || sink == nullptr || blocks < 1 || bytes % 16 != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_read, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4 *>(buf), bytes / 16, sink);
    return hipGetLastError();
}

// `blocks` workgroups each read the `bytes` (a multiple of 16 * 1024) at `buf`
// `reps` times: blocks * reps * bytes bytes taken in by the CUs.
int calib_l2read(const void *buf, size_t bytes, int reps, uint32_t *sink, int blocks, void *stream) {
    if (buf == nullptr || sink == nullptr || blocks < 1 || reps < 1 || bytes % (16 * 1024) != 0)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_l2read, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4 *>(buf), bytes / 16, reps, sink);
    return hipGetLastError();
}

// `blocks` workgroups of 4 waves, each wave `iters` x 8 MFMAs of 16x16x32
// (fp16 when bf16 == 0, else bf16): 16384 FLOPs each.
int calib_mfma(int bf16, int iters, float *sink, int blocks, void *stream) {
    if (sink == nullptr || blocks < 1 || iters < 1) return hipErrorInvalidValue;
    if (bf16)
        hipLaunchKernelGGL(k_mfma<true>, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream), iters,
                           sink);
    else
        hipLaunchKernelGGL(k_mfma<false>, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream), iters,
                           sink);
    return hipGetLastError();
}

// FLOPs of one calib_mfma launch.
double calib_mfma_flops(int iters, int blocks) {
    return static_cast<double>(blocks) * (kThreads / 64) * iters * kChains * (2.0 * 16 * 16 * 32);
}

}  // extern "C"
