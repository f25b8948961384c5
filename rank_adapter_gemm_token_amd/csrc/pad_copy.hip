// pad_copy.hip -- register-time copy of one adapter into its slot of the
// rank-padded slabs.  A lower-rank adapter is zero-padded to the pool's common
// rank ("LLM 多 LoRA 推理服务工程 2026", routing layer, zero-pad paragraph), so
// every slot has the same shape and one launch serves mixed ranks.
//
//   A_user [rank][d_in]  -> slab A [slot][R][d_in]   rows rank..R-1 = 0
//   B_user [d_out][rank] -> slab B [slot][d_out][R]  cols rank..R-1 = 0
//
// The copy is bitwise (elements moved as raw 2- or 4-byte words).
#include "internal.hpp"

namespace lora {

namespace {

template <typename E>
__global__ __launch_bounds__(256) void k_pad_copy(const E *__restrict__ A_user,
                                                  const E *__restrict__ B_user,
                                                  E *__restrict__ A_slot, E *__restrict__ B_slot,
                                                  int rank, int R, int d_in, int d_out) {
    const size_t nA = static_cast<size_t>(R) * d_in;
    const size_t nB = static_cast<size_t>(d_out) * R;
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < nA + nB;
         i += stride) {
        if (i < nA) {
            const int j = static_cast<int>(i / d_in);
            const size_t k = i - static_cast<size_t>(j) * d_in;
            A_slot[i] = (j < rank) ? A_user[static_cast<size_t>(j) * d_in + k] : E(0);
        } else {
            const size_t q = i - nA;
            const size_t n = q / R;
            const int j = static_cast<int>(q - n * R);
            B_slot[q] = (j < rank) ? B_user[n * rank + j] : E(0);
        }
    }
}

// One slot-table entry, written by a kernel on the pool's internal stream so
// that the write is ordered by stream events like any other pool work.
__global__ void k_set_slot(SlotDev *slots, int slot, SlotDev ent) {
    if (threadIdx.x == 0) slots[slot] = ent;
}

}  // namespace

hipError_t launch_set_slot(SlotDev *slots, int slot, SlotDev ent, hipStream_t st) {
    hipLaunchKernelGGL(k_set_slot, dim3(1), dim3(64), 0, st, slots, slot, ent);
    return hipGetLastError();
}

hipError_t launch_pad_copy(const void *A_user, const void *B_user, void *A_slab, void *B_slab,
                           int slot, int rank, int R, int d_in, int d_out, int esz,
                           hipStream_t st) {
    const size_t total = static_cast<size_t>(R) * (d_in + d_out);
    int blocks = static_cast<int>((total + 255) / 256);
    if (blocks > 4096) blocks = 4096;
    const size_t a_off = static_cast<size_t>(slot) * R * d_in;
    const size_t b_off = static_cast<size_t>(slot) * d_out * R;
    if (esz == 2) {
        hipLaunchKernelGGL(k_pad_copy<uint16_t>, dim3(blocks), dim3(256), 0, st,
                           static_cast<const uint16_t *>(A_user), static_cast<const uint16_t *>(B_user),
                           static_cast<uint16_t *>(A_slab) + a_off, static_cast<uint16_t *>(B_slab) + b_off,
                           rank, R, d_in, d_out);
    } else {
        hipLaunchKernelGGL(k_pad_copy<uint32_t>, dim3(blocks), dim3(256), 0, st,
                           static_cast<const uint32_t *>(A_user), static_cast<const uint32_t *>(B_user),
                           static_cast<uint32_t *>(A_slab) + a_off, static_cast<uint32_t *>(B_slab) + b_off,
                           rank, R, d_in, d_out);
    }
    return hipGetLastError();
}

}  // namespace lora
