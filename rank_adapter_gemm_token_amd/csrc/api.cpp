// api.cpp -- host runtime behind include/lora.h: pool creation, the register /
// unregister control plane with its tenant ledger and drain, and the
// asynchronous lora_apply that enqueues routing, shrink, base GEMM and expand.
//
// No device allocation and no host synchronization happen on the hot path:
// every buffer lora_apply touches is carved out of the pool at creation.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "../../include/lora.h"
#include "internal.hpp"
#include "ledger.hpp"
#include "residency.hpp"

namespace {

thread_local std::string g_last_hip;

int hip_fail(hipError_t e) {
    g_last_hip = hipGetErrorString(e);
    return LORA_EHIP;
}

#define HIP_TRY(expr)                               \
    do {                                            \
        hipError_t e_ = (expr);                     \
        if (e_ != hipSuccess) return hip_fail(e_);  \
    } while (0)

// Make the pool's device current for the duration of a call.
class DeviceGuard {
public:
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev_) != hipSuccess) {
            prev_ = -1;
            return;
        }
        if (prev_ != dev) err_ = hipSetDevice(dev);
    }
    ~DeviceGuard() {
        int cur = -1;
        if (prev_ >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev_) (void)hipSetDevice(prev_);
    }
    hipError_t error() const { return err_; }

private:
    int prev_ = -1;
    hipError_t err_ = hipSuccess;
};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Default fused/separate threshold of gfx950.  The threshold is tuned per GPU
// model ("LLM 多 LoRA 推理服务工程 2026", SRE list item 11; the routing-layer
// paragraph gives 16 for other GPUs).  On MI355X the sweep over the
// 100-adapter workload at T = 1 .. 64 puts every AUTO threshold above 0
// about 20% below all-fused: the fused expand adds little to the base GEMM's
// epilogue, a separate bucket costs one more launch and a y round trip.  So:
// every LoRA bucket fused.
constexpr int kDefaultTheta = 0;

}  // namespace

struct lora_pool_s {
    int device = 0;
    int d_in = 0, d_out = 0, R = 0, S = 0, max_T = 0;
    int Rp = 0;  // slab rank: R rounded up to a multiple of 8 (16-byte rows of B)
    lora_dtype dtype = LORA_F32;
    int esz = 4;
    lora::SlotBook book;

    void *A_slab = nullptr;
    void *B_slab = nullptr;
    lora::SlotDev *slots_dev = nullptr;
    char *ws = nullptr;
    size_t device_bytes = 0;

    lora::RouteOut ro{};
    float *h = nullptr;
    float *part = nullptr;  // split-K partial sums (decode and split tiles)
    unsigned *split_cnt = nullptr;  // per-tile split counters of the split tiles (0 between calls)
    int split_tiles = 0;            // counters at split_cnt

    hipStream_t internal = nullptr;
    std::mutex mu;
    std::vector<std::pair<hipStream_t, hipEvent_t>> inflight;
    int policy = LORA_MODE_AUTO;
    int theta = kDefaultTheta;
    int shrink_wait_polls = -1;  // lora_set_shrink_wait_polls (-1: the kernel's bound)

    // Slot-entry publication (register, loader commit): `gate` is recorded on
    // `internal` after the last entry write; until it has completed, every
    // call that reads the slot table waits for it on its own stream.
    hipEvent_t gate = nullptr;
    bool gate_pending = false;
    hipEvent_t data_ev = nullptr;  // a register's copies, on the caller's stream
    // Completion of the last lora_apply_noalloc (created with the pool: that
    // call creates nothing); drains wait for it too once it has been recorded.
    hipEvent_t noalloc_done = nullptr;
    bool noalloc_used = false;

    // The routing the pool's own arrays hold: tokens of the call that wrote
    // it (0: none yet) and its stream (lora_last_routing).
    int last_route_T = 0;
    hipStream_t last_route_stream = nullptr;

    // Opt-in stage timing (lora_profile_enable).
    struct ProfSet {
        hipEvent_t e[7];  // stage marks 0..4; 5, 6: the base-GEMM kernel's own start / stop
        bool staged;      // marks 1..3 recorded (paths with separate stage launches)
    };
    std::vector<ProfSet> prof;
    size_t prof_used = 0;

    lora_pool_s(int n_slots, int max_rank, uint64_t slot_bytes) : book(n_slots, max_rank, slot_bytes) {}
};

struct lora_plan_s {
    int device = 0;
    int max_T = 0, S = 0;
    char *mem = nullptr;        // one device allocation: the index copy and the routing arrays
    int32_t *idx = nullptr;     // [max_T] copy of the routed batch's token indices
    lora::RouteOut ro{};
    hipStream_t internal = nullptr;
    // The routed batch and what its routing depended on (pool state at
    // lora_plan_route).
    int T = -1;
    int policy = 0, theta = 0;
    std::vector<int> rank;        // [S] the slot's rank if ACTIVE, else 0 (tiles carry ranks)
    hipEvent_t done = nullptr;    // after the routing was enqueued
    hipStream_t done_stream = nullptr;
};

struct lora_loader_s {
    int device = 0;
    uint64_t cap = 0;              // bytes of A + B one staging buffer holds
    hipStream_t copy = nullptr;    // the loader's copy stream
    void *host[2] = {nullptr, nullptr};  // pinned staging
    void *dev[2] = {nullptr, nullptr};   // device staging
    hipEvent_t done[2] = {nullptr, nullptr};
    uint64_t owner[2] = {0, 0};    // ticket whose copies a buffer holds (0: none pending)
    int next = 0;
    struct Pending {
        lora_pool pool;
        int slot;
        int rank;
        float alpha;
        int buf;
    };
    std::map<uint64_t, Pending> pending;
    uint64_t last_ticket = 0;
    std::mutex mu;
};

struct lora_residency_s {
    lora_pool pool = nullptr;
    lora_loader loader = nullptr;
    lora::Residency cache;
    std::vector<uint64_t> ticket;  // [S] the last load's ticket per slot
    int managed = 0;
    std::mutex mu;
    lora_residency_s(int n_slots, int k) : cache(n_slots, k), ticket(static_cast<size_t>(n_slots), 0) {}
};

namespace {

void free_profile(lora_pool p) {
    for (auto &ps : p->prof)
        for (hipEvent_t e : ps.e)
            if (e) (void)hipEventDestroy(e);
    p->prof.clear();
    p->prof_used = 0;
}

void free_pool_memory(lora_pool p) {
    free_profile(p);
    if (p->gate) (void)hipEventDestroy(p->gate);
    if (p->data_ev) (void)hipEventDestroy(p->data_ev);
    if (p->noalloc_done) (void)hipEventDestroy(p->noalloc_done);
    p->gate = p->data_ev = p->noalloc_done = nullptr;
    if (p->A_slab) (void)hipFree(p->A_slab);
    if (p->B_slab) (void)hipFree(p->B_slab);
    if (p->slots_dev) (void)hipFree(p->slots_dev);
    if (p->ws) (void)hipFree(p->ws);
    for (auto &se : p->inflight) (void)hipEventDestroy(se.second);
    p->inflight.clear();
    if (p->internal) (void)hipStreamDestroy(p->internal);
    p->A_slab = p->B_slab = nullptr;
    p->slots_dev = nullptr;
    p->ws = nullptr;
    p->internal = nullptr;
}

// Flags of the completion events recorded on the hot path.  They tell drains
// that earlier kernels have finished; no host read of device memory relies on
// them (reads go through HIP copies), so they skip the system-scope cache
// fence that an event record otherwise adds: about 2 us of device time per
// call on MI355X (one record per lora_apply).
constexpr unsigned kCompletionEventFlags = hipEventDisableTiming | hipEventDisableSystemFence;

// The completion event of the pool's work on `st` (created on first use, not
// recorded here).
hipError_t inflight_event(lora_pool p, hipStream_t st, hipEvent_t *out) {
    for (auto &se : p->inflight) {
        if (se.first == st) {
            *out = se.second;
            return hipSuccess;
        }
    }
    hipEvent_t ev = nullptr;
    hipError_t e = hipEventCreateWithFlags(&ev, kCompletionEventFlags);
    if (e != hipSuccess) return e;
    p->inflight.emplace_back(st, ev);
    *out = ev;
    return hipSuccess;
}

// Record completion of the work just enqueued on `st`.
hipError_t record_inflight(lora_pool p, hipStream_t st) {
    hipEvent_t ev = nullptr;
    hipError_t e = inflight_event(p, st, &ev);
    return e == hipSuccess ? hipEventRecord(ev, st) : e;
}

// Wait for everything recorded so far.
hipError_t drain_inflight(lora_pool p) {
    for (auto &se : p->inflight) {
        hipError_t e = hipEventSynchronize(se.second);
        if (e != hipSuccess) return e;
    }
    if (p->noalloc_used) return hipEventSynchronize(p->noalloc_done);
    return hipSuccess;
}

bool aligned(const void *ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

// Publish slot entry `ent` so that every apply sees either the old entry in
// all of its kernels or the new one in all of them (the decode path reads the
// slot table in both of its launches): the write runs on the pool's internal
// stream after every piece of work enqueued on the pool so far (and after the
// work enqueued on `after`, which wrote the slot's slabs, when has_after), and
// every later call that reads the slot table is ordered after it
// (order_after_publish).  Asynchronous: nothing here waits on the host.
// Pool mutex held, pool device current.
hipError_t publish_entry(lora_pool p, int slot, const lora::SlotDev &ent, bool has_after, hipStream_t after) {
    hipError_t e = hipSuccess;
    if (has_after && after != p->internal) {
        e = hipEventRecord(p->data_ev, after);
        if (e == hipSuccess) e = hipStreamWaitEvent(p->internal, p->data_ev, 0);
    }
    for (auto &se : p->inflight)
        if (e == hipSuccess && se.first != p->internal) e = hipStreamWaitEvent(p->internal, se.second, 0);
    if (e == hipSuccess && p->noalloc_used) e = hipStreamWaitEvent(p->internal, p->noalloc_done, 0);
    if (e == hipSuccess) e = lora::launch_set_slot(p->slots_dev, slot, ent, p->internal);
    if (e == hipSuccess) e = hipEventRecord(p->gate, p->internal);
    if (e == hipSuccess) {
        p->gate_pending = true;
        e = record_inflight(p, p->internal);
    }
    return e;
}

// Order the work about to be enqueued on `st` after the last slot-entry
// publication, if it may still be in flight.
hipError_t order_after_publish(lora_pool p, hipStream_t st) {
    if (!p->gate_pending) return hipSuccess;
    const hipError_t q = hipEventQuery(p->gate);
    if (q == hipSuccess) {
        p->gate_pending = false;
        return hipSuccess;
    }
    if (q != hipErrorNotReady) return q;
    return hipStreamWaitEvent(st, p->gate, 0);
}

}  // namespace

namespace {

// k splits of the decode path (two launches, routing in the epilogue) for a
// call of n_tokens on pool p, or 0: the path of fp16/bf16 calls of 1 ..
// DECODE_MAX_T tokens.
int decode_splits_for(lora_pool p, int n_tokens) {
    if (p->esz != 2 || n_tokens < 1 || n_tokens > lora::DECODE_MAX_T) return 0;
    return lora::decode_splits(n_tokens, p->d_in, p->d_out);
}

// The device workspace one call's kernels use: the routing arrays (stats and
// the error counter are always the pool's), h and the split-K partial sums.
struct CallSpace {
    lora::RouteOut ro;
    float *h;
    float *part;
    lora::SplitSpace split;  // partial sums and counters of the split tiles
};

// Lay out the workspace of one lora_apply_noalloc call of n_tokens (>= 1) on
// pool p in the static scratch at `base` (256-byte aligned pieces, sized for
// this call only) and return its bytes; base == nullptr only measures.
size_t carve_call(lora_pool p, int n_tokens, char *base, CallSpace *cs) {
    const size_t T = static_cast<size_t>(n_tokens), S = static_cast<size_t>(p->S);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    const size_t o_counts = take((S + 2) * 4);
    const size_t o_offsets = take((S + 3) * 4);
    const size_t o_perm = take(T * 4);
    const size_t o_segs = take((S + 2) * 16);
    const size_t o_nseg = take(4);
    const size_t o_posseg = take(T * 4);
    const size_t o_tokpos = take(T * 4);
    const size_t o_tokseg = take(T * 4);
    const size_t o_tiles = take(static_cast<size_t>(lora::max_tiles(n_tokens, p->S)) * 8);
    const size_t o_ntiles = take(4);
    // h parts and partial sums, as the launchers lay them out for this call.
    const int dsplits = decode_splits_for(p, n_tokens);
    size_t h_parts = 1, part_floats = 0;
    if (dsplits > 0) {
        h_parts = static_cast<size_t>(dsplits);
        part_floats = static_cast<size_t>(dsplits) * lora::decode_token_blocks(n_tokens) * 16 * p->d_out;
    } else if (p->esz == 2) {
        h_parts = static_cast<size_t>(
            lora::tiled_call_h_parts(n_tokens, p->d_in, p->d_out, p->Rp, lora::max_tiles(n_tokens, p->S)));
        part_floats = lora::tiled_part_bytes(n_tokens, p->d_in, p->d_out) / 4;
    }
    const size_t o_h = take(h_parts * T * p->Rp * 4);
    const size_t o_part = take(part_floats * 4);
    if (base != nullptr) {
        cs->ro.counts = reinterpret_cast<int32_t *>(base + o_counts);
        cs->ro.offsets = reinterpret_cast<int32_t *>(base + o_offsets);
        cs->ro.perm = reinterpret_cast<int32_t *>(base + o_perm);
        cs->ro.segs = reinterpret_cast<int32_t *>(base + o_segs);
        cs->ro.n_seg = reinterpret_cast<int32_t *>(base + o_nseg);
        cs->ro.pos_seg = reinterpret_cast<int32_t *>(base + o_posseg);
        cs->ro.tok_pos = reinterpret_cast<int32_t *>(base + o_tokpos);
        cs->ro.tok_seg = reinterpret_cast<int32_t *>(base + o_tokseg);
        cs->ro.tiles = reinterpret_cast<int32_t *>(base + o_tiles);
        cs->ro.n_tiles = reinterpret_cast<int32_t *>(base + o_ntiles);
        cs->ro.stats = p->ro.stats;
        cs->ro.err = p->ro.err;
        cs->h = reinterpret_cast<float *>(base + o_h);
        cs->part = reinterpret_cast<float *>(base + o_part);
        // The split counters sit in the scratch's own zeroed block (they are
        // back at 0 after every call).
        unsigned *cnt = lora::scratch_split_counters(p->device);
        cs->split = lora::SplitSpace{cs->part, cnt, lora::MAX_SPLIT_TILES, cnt + lora::MAX_SPLIT_TILES,
                                     p->shrink_wait_polls};
    }
    return off;
}

// The body of lora_apply and lora_apply_routed: pool mutex held, pool device
// current, arguments checked.  `pre`: routing already in place (a plan's), or
// nullptr to route here.
int apply_locked(lora_pool p, const void *x, const void *W_base, const int32_t *token_adapter_idx, int n_tokens,
                 void *y, hipStream_t st, const lora::RouteOut *pre, const CallSpace &cs, bool noalloc) {
    lora_pool_s::ProfSet *ps = (p->prof_used < p->prof.size()) ? &p->prof[p->prof_used++] : nullptr;
    auto mark = [&](int i) { return ps ? hipEventRecord(ps->e[i], st) : hipSuccess; };
    if (ps) ps->staged = false;
    lora::LaunchEvents kev{};
    if (ps) kev = lora::LaunchEvents{ps->e[5], ps->e[6]};

    lora::ApplyArgs a{};
    a.dtype = p->dtype;
    a.T = n_tokens;
    a.d_in = p->d_in;
    a.d_out = p->d_out;
    a.S = p->S;
    a.R = p->Rp;
    a.x = x;
    a.W = W_base;
    a.y = y;
    a.A_slab = p->A_slab;
    a.B_slab = p->B_slab;
    a.slots = p->slots_dev;
    a.h = cs.h;
    a.h_parts = 1;
    a.shrink_parts = 1;
    a.shrink_g = 1;
    a.cnt = cs.split.cnt;
    // Routing arrays: the plan's (routed already), or the pool's own.
    const lora::RouteOut &rsrc = pre ? *pre : cs.ro;
    a.rv = lora::RouteView{rsrc.perm, rsrc.pos_seg, rsrc.tok_pos, rsrc.tok_seg, rsrc.segs, rsrc.tiles, rsrc.n_tiles};
    a.tiles_bound = lora::max_tiles(n_tokens, p->S);
    a.policy = p->policy;
    const bool half = p->esz == 2;
    // Every LoRA bucket is FUSED under the FUSED policy, and under AUTO with
    // threshold 0 (a bucket holds at least one token): no residual launch then.
    const bool any_separate = !(p->policy == LORA_MODE_FUSED || (p->policy == LORA_MODE_AUTO && p->theta == 0));

    HIP_TRY(order_after_publish(p, st));
    HIP_TRY(mark(0));
    // The call's completion event: bound to the dispatch of the call's last
    // kernel where the launcher can (`bound`), else recorded after it.
    hipEvent_t done_ev = p->noalloc_done;
    if (!noalloc) HIP_TRY(inflight_event(p, st, &done_ev));
    bool bound = false;
    const int dsplits = decode_splits_for(p, n_tokens);
    if (dsplits > 0) {
        // Split-K GEMM with the shrink, then the epilogue, which routes,
        // sums the splits and adds the fused expand.
        lora::DecodeArgs d{};
        d.splits = dsplits;
        d.max_rank = p->R;
        d.theta = p->theta;
        d.part = cs.part;
        a.h_parts = dsplits;
        a.shrink_parts = dsplits;
        a.h_by_token = 1;
        // A routed call publishes into the pool's arrays (nobody reads them)
        // and leaves its statistics and error counter alone.
        lora::RouteOut out = cs.ro;
        if (pre) out.stats = nullptr, out.err = nullptr;
        if (!any_separate) {
            kev.done = done_ev;
            bound = true;
        }
        HIP_TRY(lora::launch_decode(a, d, token_adapter_idx, out, st, kev));
        if (!noalloc) {
            p->last_route_T = n_tokens;
            p->last_route_stream = st;
        }
    } else {
        if (ps) ps->staged = true;
        // Split calls whose GEMM grid is one round run the shrink inside the
        // GEMM launch (its k parts are the plan's).
        const int fused_parts = half ? lora::tiled_plan(n_tokens, p->d_in, p->d_out).fuse_parts : 0;
        if (fused_parts > 0) {
            a.shrink_parts = fused_parts;
            a.h_parts = fused_parts;
        } else if (half) {
            // k parts of the shrink; the grouped shrink adds them into part 0
            // itself (on the counters the split tiles also use, in stream
            // order, each kernel leaving them at 0), so its consumers read one.
            const int parts = lora::tiled_h_parts(p->d_in, p->Rp, a.tiles_bound, n_tokens);
            a.shrink_g = lora::shrink_group(n_tokens, a.tiles_bound, cs.split.max_tiles);
            a.shrink_parts = parts;
            a.h_parts = a.shrink_g > 1 ? 1 : parts;
        }
        // A call routed here whose shrink has a launch of its own, one tile a
        // workgroup, routes inside that launch when the call and the grid are
        // small enough (one launch fewer).
        const bool route_in_shrink =
            !pre && half && fused_parts == 0 && a.shrink_g == 1 && n_tokens <= lora::ROUTE_SHRINK_MAX_T &&
            static_cast<long>(a.tiles_bound) * a.shrink_parts <= lora::ROUTE_SHRINK_MAX_WGS;
        if (!pre) {
            if (!route_in_shrink)
                HIP_TRY(lora::launch_route(token_adapter_idx, n_tokens, p->S, p->slots_dev, p->R, p->policy,
                                           p->theta, cs.ro, st));
            if (!noalloc) {
                p->last_route_T = n_tokens;
                p->last_route_stream = st;
            }
        }
        HIP_TRY(mark(1));
        if (route_in_shrink)
            HIP_TRY(lora::launch_route_shrink16(a, token_adapter_idx, p->R, p->theta, cs.ro, st));
        else if (fused_parts == 0)
            HIP_TRY(half ? lora::launch_shrink16(a, st) : lora::launch_shrink(a, st));
        HIP_TRY(mark(2));
        if (half) {
            if (!any_separate && kev.stop == nullptr) {
                kev.done = done_ev;
                bound = true;
            }
            HIP_TRY(lora::launch_gemm_tiled(a, cs.split, st, kev));
        } else {
            HIP_TRY(lora::launch_base_gemm(a, st));
            HIP_TRY(mark(5));
            HIP_TRY(mark(6));
        }
    }
    if (ps && ps->staged) HIP_TRY(mark(3));
    if (any_separate) HIP_TRY(half ? lora::launch_expand_sep16(a, st) : lora::launch_expand_separate(a, st));
    HIP_TRY(mark(4));
    if (!bound) HIP_TRY(hipEventRecord(done_ev, st));
    if (noalloc) p->noalloc_used = true;
    return LORA_OK;
}

// The pool's own workspace.
CallSpace pool_space(lora_pool p) {
    return CallSpace{p->ro, p->h, p->part,
                     lora::SplitSpace{p->part, p->split_cnt, p->split_tiles, p->split_cnt + p->split_tiles,
                                      p->shrink_wait_polls}};
}

// Host-side checks shared by lora_apply and lora_apply_noalloc.
int check_apply_args(lora_pool p, const void *x, const void *W_base, const int32_t *token_adapter_idx,
                     int n_tokens, void *y) {
    if (p == nullptr || n_tokens < 0) return LORA_EINVAL;
    if (n_tokens == 0) return LORA_OK;
    if (n_tokens > p->max_T) return LORA_ETOKENS;
    if (x == nullptr || W_base == nullptr || token_adapter_idx == nullptr || y == nullptr) return LORA_EINVAL;
    const size_t al = (p->esz == 2) ? 16 : 4;
    if (!aligned(x, al) || !aligned(W_base, al) || !aligned(y, al) || !aligned(token_adapter_idx, 4))
        return LORA_EINVAL;
    if (x == y) return LORA_EINVAL;
    return LORA_OK;
}


}  // namespace

extern "C" {

const char *lora_strerror(int status) {
    switch (status) {
        case LORA_OK: return "ok";
        case LORA_EINVAL: return "invalid argument";
        case LORA_ETOKENS: return "n_tokens exceeds the pool's max_tokens";
        case LORA_ESLOT_BUSY: return "slot is not free";
        case LORA_ESLOT_EMPTY: return "slot holds no adapter";
        case LORA_ERANK: return "rank out of range";
        case LORA_EALPHA: return "alpha is not finite";
        case LORA_EQUOTA: return "tenant quota exceeded";
        case LORA_EMISMATCH: return "shape or dtype does not match the pool";
        case LORA_ENOMEM: return "out of memory";
        case LORA_EHIP: return "HIP runtime error";
        case LORA_ESCRATCH: return "call needs more workspace than the static scratch holds";
        default: return "unknown status";
    }
}

const char *lora_last_hip_error(void) { return g_last_hip.c_str(); }

int lora_pool_create(int d_in, int d_out, int max_rank, int n_slots, int max_tokens, lora_dtype dtype,
                     lora_pool *out) {
    if (out == nullptr) return LORA_EINVAL;
    *out = nullptr;
    if (d_in < 1 || d_out < 1 || max_tokens < 1) return LORA_EINVAL;
    if (max_rank < 1 || max_rank > LORA_MAX_RANK) return LORA_EINVAL;
    if (n_slots < 1 || n_slots > LORA_MAX_SLOTS) return LORA_EINVAL;
    int esz = 0;
    switch (dtype) {
        case LORA_F32: esz = 4; break;
        case LORA_F16:
        case LORA_BF16: esz = 2; break;
        default: return LORA_EINVAL;
    }
    if (esz == 2 && (d_in % 64 != 0 || d_out % 64 != 0)) return LORA_EINVAL;
    // The kernels address x, W and y of one call through 32-bit byte offsets
    // (buffer resources): each must stay below 4 GiB.
    constexpr uint64_t kMaxOperand = 0xFFFFFFFFull;
    if (static_cast<uint64_t>(max_tokens) * d_in * esz > kMaxOperand ||
        static_cast<uint64_t>(d_out) * d_in * esz > kMaxOperand ||
        static_cast<uint64_t>(max_tokens) * d_out * esz > kMaxOperand)
        return LORA_EINVAL;

    const int Rp = (max_rank + 7) / 8 * 8;
    const uint64_t slot_bytes = static_cast<uint64_t>(Rp) * (d_in + d_out) * esz;
    lora_pool p = new (std::nothrow) lora_pool_s(n_slots, max_rank, slot_bytes);
    if (p == nullptr) return LORA_ENOMEM;
    p->d_in = d_in;
    p->d_out = d_out;
    p->R = max_rank;
    p->Rp = Rp;
    p->S = n_slots;
    p->max_T = max_tokens;
    p->dtype = dtype;
    p->esz = esz;

    auto fail = [&](int rc) {
        free_pool_memory(p);
        delete p;
        return rc;
    };
    hipError_t e = hipGetDevice(&p->device);
    // The device address of the static workspace (lora_apply_noalloc), once
    // per device, with the device current.
    if (e == hipSuccess) e = lora::scratch_setup(p->device);
    if (e != hipSuccess) return fail(hip_fail(e));

    const size_t S = static_cast<size_t>(n_slots);
    const size_t T = static_cast<size_t>(max_tokens);
    const size_t a_bytes = S * Rp * d_in * esz;
    const size_t b_bytes = S * d_out * Rp * esz;
    const size_t dec_T = static_cast<size_t>(max_tokens < lora::DECODE_MAX_T ? max_tokens : lora::DECODE_MAX_T);

    // Workspace layout, each piece 256-byte aligned.
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    const size_t o_counts = take((S + 2) * 4);
    const size_t o_offsets = take((S + 3) * 4);
    const size_t o_perm = take(T * 4);
    const size_t o_segs = take((S + 2) * 16);
    const size_t o_nseg = take(4);
    const size_t o_posseg = take(T * 4);
    const size_t o_tokpos = take(T * 4);
    const size_t o_tokseg = take(T * 4);
    const size_t o_tiles = take(static_cast<size_t>(lora::max_tiles(max_tokens, n_slots)) * 8);
    const size_t o_ntiles = take(4);
    const size_t o_stats = take(sizeof(lora::DevStats));
    const size_t o_err = take(8);
    // h: fp32, [T][Rp]; calls of at most 64 tokens (fp16/bf16) keep one part
    // per k split of their GEMM, [splits][T][Rp], and the splits' partial
    // sums [splits][T rounded up to 16 .. 64][d_out].
    const int dec_splits = (esz == 2) ? lora::decode_splits(static_cast<int>(dec_T), d_in, d_out) : 0;
    // Calls on the tiled path keep tiled_call_h_parts parts, [parts][T][Rp].
    size_t h_rows = std::max(T, static_cast<size_t>(dec_splits) * dec_T);
    if (esz == 2)
        for (int t = 1; t <= max_tokens; ++t)
            h_rows = std::max(h_rows, static_cast<size_t>(t) *
                                          lora::tiled_call_h_parts(t, d_in, d_out, Rp, lora::max_tiles(t, n_slots)));
    const size_t o_h = take(h_rows * Rp * 4);
    const size_t dec_rows = static_cast<size_t>(lora::decode_token_blocks(static_cast<int>(dec_T))) * 16;
    // Split tiles of calls of 65 .. 2047 tokens: the largest partial-sum
    // buffer and counter count over the token counts the pool accepts.
    size_t tiled_part = 0;
    int split_tiles = 0;
    if (esz == 2) {
        for (int t = lora::DECODE_MAX_T + 1; t <= max_tokens && t < 2048; ++t) {
            tiled_part = std::max(tiled_part, lora::tiled_part_bytes(t, d_in, d_out));
            split_tiles = std::max(split_tiles, lora::tiled_split_tiles(t, d_in, d_out));
        }
        // The grouped shrink's per-group counters share the array (calls of
        // SHRINK_G_MIN_T tokens or more; the group count grows with T).
        if (max_tokens >= lora::SHRINK_G_MIN_T)
            split_tiles = std::max(split_tiles, (lora::max_tiles(max_tokens, n_slots) + lora::SHRINK_G - 1) /
                                                    lora::SHRINK_G);
    }
    const size_t o_part = take(std::max(static_cast<size_t>(dec_splits) * dec_rows * d_out * 4, tiled_part));
    // ... and the fused shrink's two counters after them.
    const size_t o_cnt = take(static_cast<size_t>(split_tiles + 2) * 4);
    const size_t ws_bytes = off;

    e = hipMalloc(&p->A_slab, a_bytes);
    if (e == hipSuccess) e = hipMalloc(&p->B_slab, b_bytes);
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void **>(&p->slots_dev), S * sizeof(lora::SlotDev));
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void **>(&p->ws), ws_bytes);
    if (e == hipErrorOutOfMemory) return fail(LORA_ENOMEM);
    if (e != hipSuccess) return fail(hip_fail(e));
    p->device_bytes = a_bytes + b_bytes + S * sizeof(lora::SlotDev) + ws_bytes;

    e = hipStreamCreateWithFlags(&p->internal, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&p->gate, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&p->data_ev, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&p->noalloc_done, kCompletionEventFlags);
    if (e == hipSuccess) e = hipMemsetAsync(p->A_slab, 0, a_bytes, p->internal);
    if (e == hipSuccess) e = hipMemsetAsync(p->B_slab, 0, b_bytes, p->internal);
    if (e == hipSuccess) e = hipMemsetAsync(p->slots_dev, 0, S * sizeof(lora::SlotDev), p->internal);
    if (e == hipSuccess) e = hipMemsetAsync(p->ws, 0, ws_bytes, p->internal);
    if (e == hipSuccess) e = hipStreamSynchronize(p->internal);
    if (e != hipSuccess) return fail(hip_fail(e));

    char *w = p->ws;
    p->ro.counts = reinterpret_cast<int32_t *>(w + o_counts);
    p->ro.offsets = reinterpret_cast<int32_t *>(w + o_offsets);
    p->ro.perm = reinterpret_cast<int32_t *>(w + o_perm);
    p->ro.segs = reinterpret_cast<int32_t *>(w + o_segs);
    p->ro.n_seg = reinterpret_cast<int32_t *>(w + o_nseg);
    p->ro.pos_seg = reinterpret_cast<int32_t *>(w + o_posseg);
    p->ro.tok_pos = reinterpret_cast<int32_t *>(w + o_tokpos);
    p->ro.tok_seg = reinterpret_cast<int32_t *>(w + o_tokseg);
    p->ro.tiles = reinterpret_cast<int32_t *>(w + o_tiles);
    p->ro.n_tiles = reinterpret_cast<int32_t *>(w + o_ntiles);
    p->ro.stats = reinterpret_cast<lora::DevStats *>(w + o_stats);
    p->ro.err = reinterpret_cast<unsigned long long *>(w + o_err);
    p->h = reinterpret_cast<float *>(w + o_h);
    p->part = reinterpret_cast<float *>(w + o_part);
    p->split_cnt = reinterpret_cast<unsigned *>(w + o_cnt);  // zeroed with the workspace
    p->split_tiles = split_tiles;
    *out = p;
    return LORA_OK;
}

int lora_pool_destroy(lora_pool p) {
    if (p == nullptr) return LORA_OK;
    int rc = LORA_OK;
    {
        std::lock_guard<std::mutex> lk(p->mu);
        DeviceGuard g(p->device);
        hipError_t e = drain_inflight(p);
        if (e != hipSuccess) rc = hip_fail(e);
        free_pool_memory(p);
    }
    delete p;
    return rc;
}

int lora_set_tenant_quota(lora_pool p, int32_t tenant, uint64_t bytes) {
    if (p == nullptr) return LORA_EINVAL;
    std::lock_guard<std::mutex> lk(p->mu);
    return p->book.set_quota(tenant, bytes);
}

int lora_register(lora_pool p, int slot, int32_t tenant, const void *A, const void *B, int rank,
                  float alpha, void *stream) {
    if (p == nullptr || A == nullptr || B == nullptr) return LORA_EINVAL;
    std::lock_guard<std::mutex> lk(p->mu);
    int rc = p->book.begin_register(slot, tenant, rank, alpha);
    if (rc != LORA_OK) return rc;
    DeviceGuard g(p->device);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = g.error();
    if (e == hipSuccess)
        e = lora::launch_pad_copy(A, B, p->A_slab, p->B_slab, slot, rank, p->Rp, p->d_in, p->d_out, p->esz, st);
    // The entry turns ACTIVE after the copies and after every apply already
    // enqueued on the pool; later calls wait for it (publish_entry).
    const lora::SlotDev ent{lora::SLOT_ACTIVE, rank, alpha / static_cast<float>(rank), 0};
    if (e == hipSuccess) e = publish_entry(p, slot, ent, true, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);  // A and B may be freed on return
    if (e != hipSuccess) {
        p->book.abort_register(slot);
        return hip_fail(e);
    }
    p->book.commit_register(slot);
    return LORA_OK;
}

int lora_unregister(lora_pool p, int slot) {
    if (p == nullptr) return LORA_EINVAL;
    std::lock_guard<std::mutex> lk(p->mu);
    int rc = p->book.begin_unregister(slot);
    if (rc != LORA_OK) return rc;
    DeviceGuard g(p->device);
    hipError_t e = g.error();
    // Drain: every apply enqueued before this call completes first.
    if (e == hipSuccess) e = drain_inflight(p);
    lora::SlotDev ent{lora::SLOT_FREE, 0, 0.0f, 0};
    if (e == hipSuccess)
        e = hipMemcpyAsync(p->slots_dev + slot, &ent, sizeof ent, hipMemcpyHostToDevice, p->internal);
    if (e == hipSuccess) e = hipStreamSynchronize(p->internal);
    if (e != hipSuccess) {
        p->book.cancel_unregister(slot);
        return hip_fail(e);
    }
    p->book.finish_unregister(slot);
    return LORA_OK;
}

int lora_set_shrink_wait_polls(lora_pool p, int polls) {
    if (p == nullptr || polls < -1) return LORA_EINVAL;
    std::lock_guard<std::mutex> lk(p->mu);
    p->shrink_wait_polls = polls;
    return LORA_OK;
}

int lora_set_policy(lora_pool p, lora_mode mode, int threshold) {
    if (p == nullptr || threshold < 0) return LORA_EINVAL;
    if (mode != LORA_MODE_AUTO && mode != LORA_MODE_FUSED && mode != LORA_MODE_SEPARATE) return LORA_EINVAL;
    std::lock_guard<std::mutex> lk(p->mu);
    p->policy = mode;
    p->theta = threshold;
    return LORA_OK;
}

int lora_get_policy(lora_pool p, lora_mode *mode, int *threshold) {
    if (p == nullptr || mode == nullptr || threshold == nullptr) return LORA_EINVAL;
    std::lock_guard<std::mutex> lk(p->mu);
    *mode = static_cast<lora_mode>(p->policy);
    *threshold = p->theta;
    return LORA_OK;
}

int lora_apply(lora_pool p, const void *x, const void *W_base, const int32_t *token_adapter_idx,
               int n_tokens, void *y, void *stream) {
    const int rc = check_apply_args(p, x, W_base, token_adapter_idx, n_tokens, y);
    if (rc != LORA_OK || n_tokens == 0) return rc;
    std::lock_guard<std::mutex> lk(p->mu);
    DeviceGuard g(p->device);
    HIP_TRY(g.error());
    return apply_locked(p, x, W_base, token_adapter_idx, n_tokens, y, static_cast<hipStream_t>(stream), nullptr,
                        pool_space(p), false);
}

int lora_apply_noalloc(lora_pool p, const void *x, const void *W_base, const int32_t *token_adapter_idx,
                       int n_tokens, void *y, void *stream) {
    const int rc = check_apply_args(p, x, W_base, token_adapter_idx, n_tokens, y);
    if (rc != LORA_OK || n_tokens == 0) return rc;
    std::lock_guard<std::mutex> lk(p->mu);
    // The static workspace's device address, resolved when the first pool
    // was created on this device.
    char *base = lora::scratch_device_ptr(p->device);
    if (base == nullptr) return LORA_EHIP;
    if (carve_call(p, n_tokens, nullptr, nullptr) > LORA_NOALLOC_SCRATCH_BYTES - lora::SCRATCH_COUNTER_BYTES)
        return LORA_ESCRATCH;
    CallSpace cs{};
    carve_call(p, n_tokens, base, &cs);
    DeviceGuard g(p->device);
    HIP_TRY(g.error());
    return apply_locked(p, x, W_base, token_adapter_idx, n_tokens, y, static_cast<hipStream_t>(stream), nullptr, cs,
                        true);
}

int lora_route(lora_pool p, const int32_t *token_adapter_idx, int n_tokens, int32_t *counts, int32_t *offsets,
               int32_t *perm, int32_t *segs, int32_t *n_seg, void *stream) {
    if (p == nullptr || n_tokens < 0) return LORA_EINVAL;
    if (n_tokens > p->max_T) return LORA_ETOKENS;
    if (counts == nullptr || offsets == nullptr || segs == nullptr || n_seg == nullptr) return LORA_EINVAL;
    if (n_tokens > 0 && (token_adapter_idx == nullptr || perm == nullptr)) return LORA_EINVAL;
    std::lock_guard<std::mutex> lk(p->mu);
    DeviceGuard g(p->device);
    HIP_TRY(g.error());
    hipStream_t st = static_cast<hipStream_t>(stream);
    lora::RouteOut ro = p->ro;
    ro.counts = counts;
    ro.offsets = offsets;
    ro.perm = perm;
    ro.segs = segs;
    ro.n_seg = n_seg;
    ro.stats = nullptr;
    ro.err = nullptr;
    HIP_TRY(order_after_publish(p, st));
    // The routing lora_apply would run for this call: the decode epilogue's
    // small-call routing on the decode path, the routing kernel otherwise.
    if (decode_splits_for(p, n_tokens) > 0)
        HIP_TRY(lora::launch_route_small(token_adapter_idx, n_tokens, p->S, p->slots_dev, p->R, p->policy, p->theta,
                                         ro, st));
    else
        HIP_TRY(lora::launch_route(token_adapter_idx, n_tokens, p->S, p->slots_dev, p->R, p->policy, p->theta, ro,
                                   st));
    HIP_TRY(record_inflight(p, st));
    return LORA_OK;
}

int lora_last_routing(lora_pool p, int *n_tokens, int32_t *perm, int32_t *segs, int32_t *n_seg, void *stream) {
    if (p == nullptr || n_tokens == nullptr || segs == nullptr || n_seg == nullptr) return LORA_EINVAL;
    std::lock_guard<std::mutex> lk(p->mu);
    const int T = p->last_route_T;
    if (T > 0 && perm == nullptr) return LORA_EINVAL;
    DeviceGuard g(p->device);
    HIP_TRY(g.error());
    hipStream_t st = static_cast<hipStream_t>(stream);
    // After the call that wrote the arrays, when it ran on another stream.
    if (T > 0 && p->last_route_stream != st)
        for (auto &se : p->inflight)
            if (se.first == p->last_route_stream) HIP_TRY(hipStreamWaitEvent(st, se.second, 0));
    if (T > 0)
        HIP_TRY(hipMemcpyAsync(perm, p->ro.perm, static_cast<size_t>(T) * 4, hipMemcpyDeviceToDevice, st));
    HIP_TRY(hipMemcpyAsync(segs, p->ro.segs, static_cast<size_t>(p->S + 2) * 16, hipMemcpyDeviceToDevice, st));
    HIP_TRY(hipMemcpyAsync(n_seg, p->ro.n_seg, 4, hipMemcpyDeviceToDevice, st));
    HIP_TRY(record_inflight(p, st));
    *n_tokens = T;
    return LORA_OK;
}

int lora_plan_create(int max_tokens, int n_slots, lora_plan *out) {
    if (out == nullptr) return LORA_EINVAL;
    *out = nullptr;
    if (max_tokens < 1 || n_slots < 1 || n_slots > LORA_MAX_SLOTS) return LORA_EINVAL;
    lora_plan pl = new (std::nothrow) lora_plan_s;
    if (pl == nullptr) return LORA_ENOMEM;
    pl->max_T = max_tokens;
    pl->S = n_slots;
    hipError_t e = hipGetDevice(&pl->device);
    // Carve the index copy and the routing arrays out of one allocation.
    const size_t T = static_cast<size_t>(max_tokens), S = static_cast<size_t>(n_slots);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    const size_t o_idx = take(T * 4);
    const size_t o_counts = take((S + 2) * 4);
    const size_t o_offsets = take((S + 3) * 4);
    const size_t o_perm = take(T * 4);
    const size_t o_segs = take((S + 2) * 16);
    const size_t o_nseg = take(4);
    const size_t o_posseg = take(T * 4);
    const size_t o_tokpos = take(T * 4);
    const size_t o_tokseg = take(T * 4);
    const size_t o_tiles = take(static_cast<size_t>(lora::max_tiles(max_tokens, n_slots)) * 8);
    const size_t o_ntiles = take(4);
    const size_t o_stats = take(sizeof(lora::DevStats));
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void **>(&pl->mem), off);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&pl->internal, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipMemsetAsync(pl->mem, 0, off, pl->internal);
    if (e == hipSuccess) e = hipStreamSynchronize(pl->internal);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&pl->done, kCompletionEventFlags);
    if (e != hipSuccess) {
        const int rc = (e == hipErrorOutOfMemory) ? LORA_ENOMEM : hip_fail(e);
        lora_plan_destroy(pl);
        return rc;
    }
    char *m = pl->mem;
    pl->idx = reinterpret_cast<int32_t *>(m + o_idx);
    pl->ro.counts = reinterpret_cast<int32_t *>(m + o_counts);
    pl->ro.offsets = reinterpret_cast<int32_t *>(m + o_offsets);
    pl->ro.perm = reinterpret_cast<int32_t *>(m + o_perm);
    pl->ro.segs = reinterpret_cast<int32_t *>(m + o_segs);
    pl->ro.n_seg = reinterpret_cast<int32_t *>(m + o_nseg);
    pl->ro.pos_seg = reinterpret_cast<int32_t *>(m + o_posseg);
    pl->ro.tok_pos = reinterpret_cast<int32_t *>(m + o_tokpos);
    pl->ro.tok_seg = reinterpret_cast<int32_t *>(m + o_tokseg);
    pl->ro.tiles = reinterpret_cast<int32_t *>(m + o_tiles);
    pl->ro.n_tiles = reinterpret_cast<int32_t *>(m + o_ntiles);
    pl->ro.stats = reinterpret_cast<lora::DevStats *>(m + o_stats);
    pl->ro.err = nullptr;  // set to the routing pool's counter per route
    *out = pl;
    return LORA_OK;
}

int lora_plan_destroy(lora_plan plan) {
    if (plan == nullptr) return LORA_OK;
    int rc = LORA_OK;
    DeviceGuard g(plan->device);
    if (plan->done_stream != nullptr) {
        const hipError_t e = hipEventSynchronize(plan->done);
        if (e != hipSuccess) rc = hip_fail(e);
    }
    if (plan->done) (void)hipEventDestroy(plan->done);
    if (plan->mem) (void)hipFree(plan->mem);
    if (plan->internal) (void)hipStreamDestroy(plan->internal);
    delete plan;
    return rc;
}

int lora_plan_route(lora_plan plan, lora_pool p, const int32_t *token_adapter_idx, int n_tokens, void *stream) {
    if (plan == nullptr || p == nullptr || n_tokens < 0) return LORA_EINVAL;
    if (n_tokens > plan->max_T || n_tokens > p->max_T) return LORA_ETOKENS;
    if (n_tokens > 0 && (token_adapter_idx == nullptr || !aligned(token_adapter_idx, 4))) return LORA_EINVAL;
    if (p->S != plan->S || p->device != plan->device) return LORA_EMISMATCH;
    std::lock_guard<std::mutex> lk(p->mu);
    DeviceGuard g(p->device);
    HIP_TRY(g.error());
    hipStream_t st = static_cast<hipStream_t>(stream);
    plan->T = -1;
    HIP_TRY(order_after_publish(p, st));
    if (n_tokens > 0) {
        // The routing kernel also keeps the plan's copy of the indices (the
        // small-call path reads them again at every apply).
        lora::RouteOut ro = plan->ro;
        ro.err = p->ro.err;  // invalid tokens counted once, on the routing pool
        ro.idx_copy = plan->idx;
        hipEvent_t pool_ev = nullptr;
        HIP_TRY(inflight_event(p, st, &pool_ev));
        HIP_TRY(lora::launch_route(token_adapter_idx, n_tokens, p->S, p->slots_dev, p->R, p->policy, p->theta, ro,
                                   st, pool_ev));
    }
    HIP_TRY(hipEventRecord(plan->done, st));
    plan->done_stream = st;
    plan->policy = p->policy;
    plan->theta = p->theta;
    plan->rank.assign(static_cast<size_t>(p->S), 0);
    for (int i = 0; i < p->S; ++i)
        if (p->book.slot(i).state == lora::SlotState::Active) plan->rank[i] = p->book.slot(i).rank;
    plan->T = n_tokens;
    return LORA_OK;
}

int lora_apply_routed(lora_pool p, lora_plan plan, const void *x, const void *W_base, void *y, void *stream) {
    if (p == nullptr || plan == nullptr || plan->T < 0) return LORA_EINVAL;
    const int n_tokens = plan->T;
    if (n_tokens == 0) return LORA_OK;
    if (n_tokens > p->max_T) return LORA_ETOKENS;
    if (x == nullptr || W_base == nullptr || y == nullptr) return LORA_EINVAL;
    const size_t al = (p->esz == 2) ? 16 : 4;
    if (!aligned(x, al) || !aligned(W_base, al) || !aligned(y, al)) return LORA_EINVAL;
    if (x == y) return LORA_EINVAL;

    std::lock_guard<std::mutex> lk(p->mu);
    // The plan's routing holds for this pool only if every input of the
    // routing matches: slot count, which slots are ACTIVE and their ranks
    // (the bucket tiles carry them), policy, threshold.
    if (p->S != plan->S || p->device != plan->device || p->policy != plan->policy || p->theta != plan->theta)
        return LORA_EMISMATCH;
    for (int i = 0; i < p->S; ++i) {
        const lora::SlotRecord &rec = p->book.slot(i);
        if ((rec.state == lora::SlotState::Active ? rec.rank : 0) != plan->rank[i]) return LORA_EMISMATCH;
    }
    DeviceGuard g(p->device);
    HIP_TRY(g.error());
    return apply_locked(p, x, W_base, plan->idx, n_tokens, y, static_cast<hipStream_t>(stream), &plan->ro,
                        pool_space(p), false);
}

int lora_loader_create(uint64_t capacity_bytes, lora_loader *out) {
    if (out == nullptr) return LORA_EINVAL;
    *out = nullptr;
    if (capacity_bytes == 0) return LORA_EINVAL;
    lora_loader l = new (std::nothrow) lora_loader_s;
    if (l == nullptr) return LORA_ENOMEM;
    l->cap = capacity_bytes;
    hipError_t e = hipGetDevice(&l->device);
    // Staging: A, then B at the next 256-byte boundary.
    const size_t bytes = align_up(static_cast<size_t>(capacity_bytes), 256) + 256;
    for (int b = 0; b < 2 && e == hipSuccess; ++b) {
        e = hipHostMalloc(&l->host[b], bytes, hipHostMallocDefault);
        if (e == hipSuccess) e = hipMalloc(&l->dev[b], bytes);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&l->done[b], hipEventDisableTiming);
    }
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&l->copy, hipStreamNonBlocking);
    if (e != hipSuccess) {
        const int rc = (e == hipErrorOutOfMemory) ? LORA_ENOMEM : hip_fail(e);
        lora_loader_destroy(l);
        return rc;
    }
    *out = l;
    return LORA_OK;
}

namespace {

// Make a finished load's slot ACTIVE: write its device slot entry, then the
// host state (pool mutex taken here).  The loader's mutex is held.
int commit_load(lora_loader l, uint64_t ticket) {
    auto it = l->pending.find(ticket);
    if (it == l->pending.end()) return LORA_OK;  // committed already
    const lora_loader_s::Pending pd = it->second;
    l->pending.erase(it);
    if (l->owner[pd.buf] == ticket) l->owner[pd.buf] = 0;
    lora_pool p = pd.pool;
    std::lock_guard<std::mutex> lk(p->mu);
    DeviceGuard g(p->device);
    hipError_t e = g.error();
    // The slot's copies have completed (the caller waited for them); the
    // entry turns ACTIVE after every apply already enqueued on the pool, and
    // later calls wait for it.  Nothing here blocks (lora_load_poll).
    const lora::SlotDev ent{lora::SLOT_ACTIVE, pd.rank, pd.alpha / static_cast<float>(pd.rank), 0};
    if (e == hipSuccess) e = publish_entry(p, pd.slot, ent, false, nullptr);
    if (e != hipSuccess) {
        p->book.abort_register(pd.slot);
        return hip_fail(e);
    }
    p->book.commit_register(pd.slot);
    return LORA_OK;
}

// Wait for staging buffer b's copies and commit the load that owns it.
int retire_buffer(lora_loader l, int b) {
    const uint64_t t = l->owner[b];
    if (t == 0) return LORA_OK;
    const hipError_t e = hipEventSynchronize(l->done[b]);
    if (e != hipSuccess) return hip_fail(e);
    return commit_load(l, t);
}

}  // namespace

int lora_loader_destroy(lora_loader l) {
    if (l == nullptr) return LORA_OK;
    int rc = LORA_OK;
    {
        std::lock_guard<std::mutex> lk(l->mu);
        DeviceGuard g(l->device);
        for (int b = 0; b < 2; ++b) {
            const int r = retire_buffer(l, b);
            if (r != LORA_OK && rc == LORA_OK) rc = r;
        }
        for (int b = 0; b < 2; ++b) {
            if (l->done[b]) (void)hipEventDestroy(l->done[b]);
            if (l->dev[b]) (void)hipFree(l->dev[b]);
            if (l->host[b]) (void)hipHostFree(l->host[b]);
        }
        if (l->copy) (void)hipStreamDestroy(l->copy);
    }
    delete l;
    return rc;
}

int lora_load_async(lora_loader l, lora_pool p, int slot, int32_t tenant, const void *A_host, const void *B_host,
                    int rank, float alpha, uint64_t *ticket) {
    if (l == nullptr || p == nullptr || A_host == nullptr || B_host == nullptr || ticket == nullptr)
        return LORA_EINVAL;
    if (p->device != l->device) return LORA_EINVAL;
    if (rank >= 1 && rank <= p->R) {
        const uint64_t need = static_cast<uint64_t>(rank) * (p->d_in + p->d_out) * p->esz;
        if (need > l->cap) return LORA_EINVAL;
    }
    std::lock_guard<std::mutex> lk(l->mu);
    DeviceGuard g(l->device);
    HIP_TRY(g.error());
    // Take the older staging buffer; if its copies are still in flight, wait
    // for them (and commit that load) first.
    const int b = l->next;
    const int rr = retire_buffer(l, b);
    if (rr != LORA_OK) return rr;
    {
        std::lock_guard<std::mutex> pk(p->mu);
        const int rc = p->book.begin_register(slot, tenant, rank, alpha);  // reserve: slot LOADING
        if (rc != LORA_OK) return rc;
    }
    const size_t a_bytes = static_cast<size_t>(rank) * p->d_in * p->esz;
    const size_t b_bytes = static_cast<size_t>(p->d_out) * rank * p->esz;
    const size_t b_off = align_up(a_bytes, 256);
    char *hs = static_cast<char *>(l->host[b]);
    char *ds = static_cast<char *>(l->dev[b]);
    std::memcpy(hs, A_host, a_bytes);
    std::memcpy(hs + b_off, B_host, b_bytes);
    hipError_t e = hipMemcpyAsync(ds, hs, b_off + b_bytes, hipMemcpyHostToDevice, l->copy);
    if (e == hipSuccess)
        e = lora::launch_pad_copy(ds, ds + b_off, p->A_slab, p->B_slab, slot, rank, p->Rp, p->d_in, p->d_out, p->esz,
                                  l->copy);
    if (e == hipSuccess) e = hipEventRecord(l->done[b], l->copy);
    if (e == hipSuccess) {
        std::lock_guard<std::mutex> pk(p->mu);
        e = record_inflight(p, l->copy);  // unregister / destroy drain these copies
    }
    if (e != hipSuccess) {
        std::lock_guard<std::mutex> pk(p->mu);
        p->book.abort_register(slot);
        return hip_fail(e);
    }
    const uint64_t t = ++l->last_ticket;
    l->pending[t] = lora_loader_s::Pending{p, slot, rank, alpha, b};
    l->owner[b] = t;
    l->next = b ^ 1;
    *ticket = t;
    return LORA_OK;
}

int lora_load_poll(lora_loader l, uint64_t ticket, int *done) {
    if (l == nullptr || done == nullptr) return LORA_EINVAL;
    std::lock_guard<std::mutex> lk(l->mu);
    if (ticket == 0 || ticket > l->last_ticket) return LORA_EINVAL;
    auto it = l->pending.find(ticket);
    if (it == l->pending.end()) {
        *done = 1;
        return LORA_OK;
    }
    DeviceGuard g(l->device);
    HIP_TRY(g.error());
    const hipError_t e = hipEventQuery(l->done[it->second.buf]);
    if (e == hipErrorNotReady) {
        *done = 0;
        return LORA_OK;
    }
    if (e != hipSuccess) return hip_fail(e);
    const int rc = commit_load(l, ticket);
    *done = (rc == LORA_OK) ? 1 : 0;
    return rc;
}

int lora_load_wait(lora_loader l, uint64_t ticket) {
    if (l == nullptr) return LORA_EINVAL;
    std::lock_guard<std::mutex> lk(l->mu);
    if (ticket == 0 || ticket > l->last_ticket) return LORA_EINVAL;
    auto it = l->pending.find(ticket);
    if (it == l->pending.end()) return LORA_OK;
    DeviceGuard g(l->device);
    HIP_TRY(g.error());
    const hipError_t e = hipEventSynchronize(l->done[it->second.buf]);
    if (e != hipSuccess) return hip_fail(e);
    return commit_load(l, ticket);
}

int lora_residency_create(lora_pool p, lora_loader l, int k, lora_residency *out) {
    if (out == nullptr) return LORA_EINVAL;
    *out = nullptr;
    if (p == nullptr || l == nullptr || k < 1) return LORA_EINVAL;
    lora_residency r = new (std::nothrow) lora_residency_s(p->S, k);
    if (r == nullptr) return LORA_ENOMEM;
    r->pool = p;
    r->loader = l;
    std::lock_guard<std::mutex> lk(p->mu);
    for (int s = 0; s < p->S; ++s) {
        const bool free_now = p->book.slot(s).state == lora::SlotState::Free;
        r->cache.set_usable(s, free_now);
        r->managed += free_now ? 1 : 0;
    }
    *out = r;
    return LORA_OK;
}

int lora_residency_destroy(lora_residency r) {
    delete r;
    return LORA_OK;
}

int lora_residency_set_share(lora_residency r, int32_t tenant, int max_slots) {
    if (r == nullptr) return LORA_EINVAL;
    std::lock_guard<std::mutex> lk(r->mu);
    return r->cache.set_share(tenant, max_slots);
}

int lora_residency_acquire(lora_residency r, uint64_t adapter_id, int32_t tenant, const void *A_host,
                           const void *B_host, int rank, float alpha, int *slot, uint64_t *ticket) {
    if (r == nullptr || slot == nullptr || ticket == nullptr) return LORA_EINVAL;
    std::lock_guard<std::mutex> lk(r->mu);
    lora::Residency::Decision d;
    const int rc = r->cache.acquire(adapter_id, tenant, &d);
    if (rc != LORA_OK) return rc;
    if (d.hit) {
        *slot = d.slot;
        *ticket = r->ticket[d.slot];
        return LORA_OK;
    }
    if (A_host == nullptr || B_host == nullptr) {
        r->cache.abandon(d.slot);
        return LORA_EINVAL;
    }
    if (d.evict) {
        // No holder references the victim.  Its load may still be pending:
        // finish it, then unload (the unregister drains every apply already
        // enqueued that might still read it).
        if (r->ticket[d.slot] != 0) {
            const int rw = lora_load_wait(r->loader, r->ticket[d.slot]);
            if (rw != LORA_OK) {
                r->cache.abandon(d.slot);
                return rw;
            }
        }
        const int ru = lora_unregister(r->pool, d.slot);
        if (ru != LORA_OK) {
            r->cache.abandon(d.slot);
            return ru;
        }
    }
    uint64_t t = 0;
    const int rl = lora_load_async(r->loader, r->pool, d.slot, tenant, A_host, B_host, rank, alpha, &t);
    if (rl != LORA_OK) {
        r->cache.abandon(d.slot);
        return rl;
    }
    r->ticket[d.slot] = t;
    *slot = d.slot;
    *ticket = t;
    return LORA_OK;
}

int lora_residency_release(lora_residency r, uint64_t adapter_id) {
    if (r == nullptr) return LORA_EINVAL;
    std::lock_guard<std::mutex> lk(r->mu);
    return r->cache.release(adapter_id);
}

int lora_residency_stats_read(lora_residency r, lora_residency_stats *out) {
    if (r == nullptr || out == nullptr) return LORA_EINVAL;
    std::lock_guard<std::mutex> lk(r->mu);
    out->hits = r->cache.hits;
    out->misses = r->cache.misses;
    out->evictions = r->cache.evictions;
    out->resident = r->cache.occupied();
    out->managed = r->managed;
    return LORA_OK;
}

int lora_pool_stats(lora_pool p, lora_stats *out) {
    if (p == nullptr || out == nullptr) return LORA_EINVAL;
    std::lock_guard<std::mutex> lk(p->mu);
    DeviceGuard g(p->device);
    HIP_TRY(g.error());
    HIP_TRY(drain_inflight(p));
    lora::DevStats ds{};
    HIP_TRY(hipMemcpyAsync(&ds, p->ro.stats, sizeof ds, hipMemcpyDeviceToHost, p->internal));
    HIP_TRY(hipStreamSynchronize(p->internal));
    std::memset(out, 0, sizeof *out);
    out->d_in = p->d_in;
    out->d_out = p->d_out;
    out->max_rank = p->R;
    out->n_slots = p->S;
    out->max_tokens = p->max_T;
    out->dtype = p->dtype;
    out->active_slots = p->book.count(lora::SlotState::Active);
    out->draining_slots = p->book.count(lora::SlotState::Draining);
    out->slot_bytes = p->book.slot_bytes();
    out->resident_bytes = p->book.resident_bytes();
    out->device_bytes = p->device_bytes;
    out->last_tokens = ds.tokens;
    out->last_adapters = ds.lora_buckets;
    out->last_fused_buckets = ds.fused_buckets;
    out->last_separate_buckets = ds.separate_buckets;
    out->last_base_only_tokens = ds.base_only_tokens;
    out->last_invalid_tokens = ds.invalid_tokens;
    out->last_lora_rows_padded = ds.rows_padded;
    out->last_lora_rows_true = ds.rows_true;
    out->last_zero_pad_fraction =
        ds.rows_padded > 0 ? 1.0 - static_cast<double>(ds.rows_true) / static_cast<double>(ds.rows_padded) : 0.0;
    return LORA_OK;
}

int lora_tenant_bytes(lora_pool p, int32_t tenant, uint64_t *out) {
    if (p == nullptr || out == nullptr) return LORA_EINVAL;
    std::lock_guard<std::mutex> lk(p->mu);
    *out = p->book.tenant_used(tenant);
    return LORA_OK;
}

int lora_poll_errors(lora_pool p, uint64_t *n_invalid_tokens) {
    if (p == nullptr || n_invalid_tokens == nullptr) return LORA_EINVAL;
    std::lock_guard<std::mutex> lk(p->mu);
    DeviceGuard g(p->device);
    HIP_TRY(g.error());
    HIP_TRY(drain_inflight(p));
    unsigned long long v = 0, zero = 0;
    HIP_TRY(hipMemcpyAsync(&v, p->ro.err, sizeof v, hipMemcpyDeviceToHost, p->internal));
    HIP_TRY(hipMemcpyAsync(p->ro.err, &zero, sizeof zero, hipMemcpyHostToDevice, p->internal));
    HIP_TRY(hipStreamSynchronize(p->internal));
    *n_invalid_tokens = v;
    return LORA_OK;
}

int lora_profile_enable(lora_pool p, int enable, int max_calls) {
    if (p == nullptr || (enable && max_calls < 1)) return LORA_EINVAL;
    std::lock_guard<std::mutex> lk(p->mu);
    DeviceGuard g(p->device);
    HIP_TRY(g.error());
    HIP_TRY(drain_inflight(p));
    free_profile(p);
    if (!enable) return LORA_OK;
    try {
        p->prof.resize(static_cast<size_t>(max_calls));
    } catch (...) {
        return LORA_ENOMEM;
    }
    for (auto &ps : p->prof)
        for (hipEvent_t &e : ps.e) e = nullptr;
    for (auto &ps : p->prof) {
        for (hipEvent_t &e : ps.e) {
            hipError_t err = hipEventCreate(&e);
            if (err != hipSuccess) {
                free_profile(p);
                return hip_fail(err);
            }
        }
    }
    return LORA_OK;
}

int lora_profile_read(lora_pool p, lora_profile *out) {
    if (p == nullptr || out == nullptr) return LORA_EINVAL;
    std::lock_guard<std::mutex> lk(p->mu);
    DeviceGuard g(p->device);
    HIP_TRY(g.error());
    std::memset(out, 0, sizeof *out);
    double *acc[4] = {&out->route_ms, &out->shrink_ms, &out->gemm_ms, &out->expand_ms};
    for (size_t c = 0; c < p->prof_used; ++c) {
        lora_pool_s::ProfSet &ps = p->prof[c];
        HIP_TRY(hipEventSynchronize(ps.e[4]));
        if (ps.staged) {
            for (int i = 0; i < 4; ++i) {
                float ms = 0.0f;
                HIP_TRY(hipEventElapsedTime(&ms, ps.e[i], ps.e[i + 1]));
                *acc[i] += ms;
            }
        } else {
            // One marked interval: the decode path's two launches and, when
            // some bucket runs SEPARATE, the residual expand.
            float ms = 0.0f;
            HIP_TRY(hipEventElapsedTime(&ms, ps.e[0], ps.e[4]));
            out->gemm_ms += ms;
        }
        float ms = 0.0f;
        HIP_TRY(hipEventElapsedTime(&ms, ps.e[5], ps.e[6]));
        out->kernel_ms += ms;
    }
    out->calls = static_cast<int64_t>(p->prof_used);
    p->prof_used = 0;
    return LORA_OK;
}

}  // extern "C"
