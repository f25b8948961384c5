/*
 * lora.h -- C ABI of liblora.so, the MI355X (gfx950) multi-LoRA adapter
 * execution unit.
 *
 * For a batch of T tokens, each tagged with an adapter slot or with
 * LORA_BASE_ONLY, one lora_apply call computes, per token t,
 *
 *     y[t] = x[t] W^T                                   (base_only)
 *     y[t] = x[t] W^T + (alpha_i / r_i) (x[t] A_i^T) B_i^T   (slot i)
 *
 * over an HBM-resident pool of adapters zero-padded to a common rank.
 *
 * Sources (page title and section):
 *  [P1] xpshop.cn article 492 (multi-tenant LoRA on one private base), sections
 *       二 and 三: one resident base shared by tenants, per-tenant memory quota
 *       as a hard boundary (over-quota mounts are refused, nothing is
 *       evicted), the tenant is mapped to an adapter handle once at request
 *       entry, hot-plug after weight validation, draining unload, refusal on a
 *       base-version mismatch, routing default base_only.
 *  [P3] "Multi-LoRA 在线服务隔离", sections on the request identity (default
 *       deny: a missing mapping is an explicit error, never a fallback; mixed
 *       adapters may share one batch with per-request index mapping) and on
 *       memory accounting (reserve memory before loading; never unload
 *       weights a request still holds).
 *  [P4] "LLM 多 LoRA 推理服务工程 2026": four-layer runtime, the adapter
 *       execution unit paragraph (base linear plus LoRA A/B, fused in one
 *       launch or separate with a residual add); routing layer, the
 *       two-level bucketing paragraph (bucket by adapter; a bucket above a
 *       threshold runs fused, otherwise separate) and the zero-pad paragraph
 *       (A maps hidden to rank, B maps rank to hidden; lower ranks are
 *       zero-padded to the common rank; report the zero-pad share); SRE list
 *       item 11 (the fused/separate threshold is tuned per GPU model).
 *
 * Conventions for every call:
 *  - Every function returns an int status: LORA_OK (0) or a negative LORA_E*
 *    code; lora_strerror() gives its text.  No call aborts the process.
 *  - Matrices are row-major and contiguous, in the nn.Linear [out][in]
 *    convention: W_base is [d_out][d_in], A is [rank][d_in], B is
 *    [d_out][rank].  x is [T][d_in] and y is [T][d_out].
 *  - One element type per pool (lora_dtype) for x, W_base, A, B and y.
 *  - "device" pointers are HIP device memory on the pool's device, 16-byte
 *    aligned.  The caller owns x, W_base, the index array and y, and keeps them
 *    alive until the stream work that uses them completes.
 *  - `stream` is a hipStream_t passed as void*; NULL is the legacy default
 *    stream.
 *  - Control-plane calls (create/destroy/quota/register/unregister/policy/
 *    stats/poll) and lora_apply/lora_route are serialized by a per-pool mutex.
 *    lora_apply and lora_route share the pool's workspace: calls on
 *    different streams must be ordered by the caller (one stream per pool is
 *    the simple contract).
 */
#ifndef LORA_H
#define LORA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- types -- */

typedef struct lora_pool_s *lora_pool; /* opaque; owned by the library */
typedef struct lora_plan_s *lora_plan; /* opaque routing plan; owned by the library */
typedef struct lora_loader_s *lora_loader; /* opaque host-to-slot loader; owned by the library */
typedef struct lora_residency_s *lora_residency; /* opaque slot residency manager */

typedef enum { LORA_F32 = 0, LORA_F16 = 1, LORA_BF16 = 2 } lora_dtype;

/* Fused/separate policy.  AUTO: a bucket (the tokens of one adapter in one
 * call) with more than `threshold` tokens runs FUSED, otherwise SEPARATE
 * [P4 two-level bucketing].  FUSED / SEPARATE force every bucket. */
typedef enum { LORA_MODE_AUTO = 0, LORA_MODE_FUSED = 1, LORA_MODE_SEPARATE = 2 } lora_mode;

/* Mode recorded per bucket by routing. */
#define LORA_SEG_NONE 0     /* base_only or invalid bucket: no LoRA term */
#define LORA_SEG_FUSED 1    /* LoRA expand added in the base GEMM's epilogue */
#define LORA_SEG_SEPARATE 2 /* base stored first, LoRA added by a residual kernel */

/* token_adapter_idx value for a token that uses the base model only [P1 三]. */
#define LORA_BASE_ONLY (-1)

/* Limits of this build. */
#define LORA_MAX_SLOTS 1024  /* n_slots per pool */
#define LORA_MAX_RANK 64     /* max_rank per pool */

/* Status codes. */
#define LORA_OK 0
#define LORA_EINVAL (-1)      /* null pointer, bad size, slot out of range, misalignment */
#define LORA_ETOKENS (-2)     /* n_tokens > the pool's max_tokens */
#define LORA_ESLOT_BUSY (-3)  /* register into a slot that is not FREE */
#define LORA_ESLOT_EMPTY (-4) /* unregister a slot that holds no adapter */
#define LORA_ERANK (-5)       /* rank < 1 or rank > the pool's max_rank */
#define LORA_EALPHA (-6)      /* alpha not finite */
#define LORA_EQUOTA (-7)      /* tenant's used + slot bytes > its quota [P1 三; P3 accounting] */
#define LORA_EMISMATCH (-8)   /* shape or dtype does not match the pool's base [P1 三] */
#define LORA_ENOMEM (-9)      /* device or host allocation failed */
#define LORA_EHIP (-10)       /* a HIP runtime call failed; lora_strerror has no detail,
                                 lora_last_hip_error() has the HIP text */
#define LORA_ESCRATCH (-11)   /* lora_apply_noalloc: the call's workspace exceeds
                                 LORA_NOALLOC_SCRATCH_BYTES */

/* Size of the library's static per-device workspace (lora_apply_noalloc). */
#define LORA_NOALLOC_SCRATCH_BYTES (32u << 20)

/* Pool statistics.  The `last_*` fields describe the most recent lora_apply
 * on the pool and are read back from the device (lora_pool_stats
 * synchronizes).  The three concatenation figures of [P4 zero-pad paragraph]
 * are: LoRA rows at the padded rank (last_lora_rows_padded), the launch extent
 * (last_tokens x d_out), and the zero-pad share (last_zero_pad_fraction). */
typedef struct {
    int32_t d_in, d_out, max_rank, n_slots, max_tokens, dtype;
    int32_t active_slots;            /* slots holding a registered adapter */
    int32_t draining_slots;          /* slots being unregistered */
    uint64_t slot_bytes;             /* bytes one slot occupies (and is charged) */
    uint64_t resident_bytes;         /* bytes charged to tenants, all slots */
    uint64_t device_bytes;           /* device memory the pool holds in total */
    int32_t last_tokens;
    int32_t last_adapters;           /* distinct adapters (LoRA buckets) */
    int32_t last_fused_buckets;
    int32_t last_separate_buckets;
    int32_t last_base_only_tokens;
    int32_t last_invalid_tokens;
    int64_t last_lora_rows_padded;   /* sum over LoRA tokens of max_rank */
    int64_t last_lora_rows_true;     /* sum over LoRA tokens of the adapter's rank */
    double last_zero_pad_fraction;   /* 1 - true / padded (0 if no LoRA token) */
} lora_stats;

/* ------------------------------------------------------------ lifecycle -- */

/* Create a pool for one linear layer on the current HIP device: n_slots
 * adapter slots of rank up to max_rank, zero-padded to max_rank [P4 zero-pad],
 * and a workspace for up to max_tokens tokens per call.  Allocates all device
 * memory now; lora_apply never allocates.
 *   d_in, d_out   the base linear's input and output widths.  For LORA_F16 /
 *                 LORA_BF16 both must be multiples of 64; LORA_F32 takes any.
 *   max_rank      1..LORA_MAX_RANK;  n_slots 1..LORA_MAX_SLOTS;
 *   max_tokens    >= 1.
 * The kernels address x, W_base and y through 32-bit byte offsets: each of
 * max_tokens*d_in, d_out*d_in and max_tokens*d_out elements must fit in
 * 4 GiB - 1 bytes, else LORA_EINVAL.
 * Errors: LORA_EINVAL (bad sizes, out == NULL), LORA_ENOMEM, LORA_EHIP. */
int lora_pool_create(int d_in, int d_out, int max_rank, int n_slots, int max_tokens,
                     lora_dtype dtype, lora_pool *out);

/* Wait for every lora_apply / lora_route enqueued on the pool, then free all
 * of its device memory and the handle.  p == NULL is a no-op. */
int lora_pool_destroy(lora_pool p);

/* ------------------------------------------------------- control plane -- */

/* Set a tenant's hard byte quota on this pool [P1 三: vram_quota].  A tenant
 * whose quota was never set has quota 0: every register is refused (default
 * deny, [P3 request identity]).  Lowering a quota below the tenant's current
 * use evicts nothing; later registers are refused.  tenant >= 0. */
int lora_set_tenant_quota(lora_pool p, int32_t tenant, uint64_t bytes);

/* Register an adapter into a FREE slot [P1 三: validate, then attach].
 *   A       device, [rank][d_in], pool dtype
 *   B       device, [d_out][rank], pool dtype
 *   rank    the adapter's true rank, 1..max_rank; rows/columns rank..max_rank-1
 *           of the slot are zero-filled [P4 zero-pad]
 *   alpha   finite; the slot's scale is alpha / rank (the true rank)
 *   stream  the copies are ordered after earlier work on `stream` (so A and B
 *           may have been written there) and complete before the call returns;
 *           A and B may be freed afterwards.
 * The slot turns ACTIVE on the device after every lora_apply / lora_route /
 * lora_plan_route enqueued on the pool before this call (on any stream) and
 * before every one enqueued after it: each call sees the slot either FREE in
 * all of its kernels (its tokens are invalid) or ACTIVE in all of them, never
 * a mix.  The call does not wait for those earlier applies.
 * The slot's bytes (lora_stats.slot_bytes) are reserved against the tenant's
 * quota before anything is copied [P3 accounting]; over quota the call fails
 * with LORA_EQUOTA and nothing else changes [P1 三: never evict another].
 * Errors: LORA_EINVAL (slot out of range, NULL A/B, tenant < 0), LORA_ESLOT_BUSY,
 * LORA_ERANK, LORA_EALPHA, LORA_EQUOTA, LORA_EHIP. */
int lora_register(lora_pool p, int slot, int32_t tenant, const void *A, const void *B,
                  int rank, float alpha, void *stream);

/* Unregister by draining [P1 二/三; P3 accounting: never unload weights a
 * request still holds]: mark the slot DRAINING, wait until every lora_apply
 * enqueued on the pool before this call has completed, then free the slot
 * and return its bytes to its tenant.  Blocks the calling thread; applies
 * from other threads wait on the pool mutex meanwhile.  A token that names
 * the slot in a later call is invalid (see lora_apply).
 * Errors: LORA_EINVAL, LORA_ESLOT_EMPTY, LORA_EHIP. */
int lora_unregister(lora_pool p, int slot);

/* Fused/separate policy [P4 two-level bucketing; SRE item 11].  threshold >= 0
 * is the bucket size above which AUTO runs FUSED.  Default: AUTO with the
 * per-device threshold this build ships for gfx950 (lora_get_policy). */
int lora_set_policy(lora_pool p, lora_mode mode, int threshold);
int lora_get_policy(lora_pool p, lora_mode *mode, int *threshold);

/* For tests of the in-launch shrink.  Calls of 65 .. 2047 tokens whose GEMM
 * tiles leave CUs idle compute h on those CUs inside the GEMM launch; the h
 * consumers of that launch poll a count of finished h units at most `polls`
 * times and, if it is still short, compute every unit themselves (the same
 * code, so the same bits).  polls = 0: they never wait and always compute h
 * themselves; polls = -1: the library's bound (about 0.1-0.3 s).  The
 * outputs do not depend on it.  LORA_EINVAL for a null pool or polls < -1. */
int lora_set_shrink_wait_polls(lora_pool p, int polls);

/* ------------------------------------------------------------ hot path -- */

/* y = x W_base^T + per-token LoRA term, asynchronously on `stream`
 * [P4 execution unit].  Routing, shrink, base GEMM and expand all run on the
 * device; the call neither allocates nor synchronizes.
 *   x                  device, [n_tokens][d_in]
 *   W_base             device, [d_out][d_in]; never retained by the pool
 *   token_adapter_idx  device int32 [n_tokens]: a slot, or LORA_BASE_ONLY
 *   y                  device, [n_tokens][d_out]; must not alias x
 * A token whose index is neither LORA_BASE_ONLY nor a registered slot (at the
 * time the call's routing kernel runs) is invalid: its y row is filled with
 * quiet NaN and the pool's device error counter grows by one; it never falls
 * back to the base or to another adapter [P3 request identity].
 * n_tokens == 0 is a no-op.
 * Errors (host-side, nothing enqueued): LORA_EINVAL, LORA_ETOKENS, LORA_EHIP. */
int lora_apply(lora_pool p, const void *x, const void *W_base,
               const int32_t *token_adapter_idx, int n_tokens, void *y, void *stream);

/* lora_apply for callers that cannot allocate device memory at call time
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and the same result, bit for bit, but the
 * call's workspace (routing arrays, h parts, split-K partial sums) lives in
 * the library's static per-device array of LORA_NOALLOC_SCRATCH_BYTES,
 * resolved when the first pool was created on the device; the call allocates
 * nothing and creates no HIP object.  Arguments, ordering and errors as
 * lora_apply, plus LORA_ESCRATCH (nothing enqueued) when the call needs more
 * workspace than the array holds: about 4 * splits * T * d_out bytes of
 * split-K partial sums plus the routing arrays and h -- every 7B-shaped
 * projection fits at up to 64 tokens, 4096-wide ones at up to 192, calls of
 * 2048 tokens and more (no split) at any width.  The array is shared by every pool and stream of the
 * device: two lora_apply_noalloc calls that may overlap in time race, so the
 * caller orders them (one stream, or events).  Nothing in it needs to start
 * at zero (every word a kernel reads was written earlier in the same call).
 * The pool's own workspace, the routing lora_last_routing reads and the
 * statistics are unaffected, except the last-call statistics and the error
 * counter, which the call updates as lora_apply does. */
int lora_apply_noalloc(lora_pool p, const void *x, const void *W_base,
                       const int32_t *token_adapter_idx, int n_tokens, void *y, void *stream);

/* Routing alone, asynchronously on `stream` [P4 two-level bucketing]: the
 * per-token histogram and stable segment sort, computed by the same device
 * code lora_apply routes with for this call size (fp16/bf16 calls of at most
 * 64 tokens route inside the decode path's epilogue; this call then runs
 * that routing in a one-wave kernel, others the routing kernel).
 * All outputs are device int32 arrays:
 *   counts[n_slots+2]     tokens per key; key = slot, n_slots = base_only,
 *                         n_slots+1 = invalid
 *   offsets[n_slots+3]    exclusive prefix sum of counts
 *   perm[n_tokens]        perm[p] = token at sorted position p, keys
 *                         ascending, ties in ascending token order
 *   segs[(n_slots+2)*4]   {key, start, len, mode} per non-empty key, keys
 *                         ascending; mode is a LORA_SEG_* value
 *   n_seg[1]              number of records
 * Does not touch the error counter.  Errors: LORA_EINVAL, LORA_ETOKENS, LORA_EHIP. */
int lora_route(lora_pool p, const int32_t *token_adapter_idx, int n_tokens,
               int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *segs,
               int32_t *n_seg, void *stream);

/* The routing the pool's kernels last used [P4 two-level bucketing; "Multi-
 * LoRA 在线服务隔离", request identity: per-request index mapping kept intact
 * in a mixed batch]: copies, asynchronously on `stream` (after the call that
 * built it, also when that ran on another stream), the stable permutation and
 * the bucket records of the last lora_apply on the pool -- or of the last
 * lora_apply_routed of at most 64 fp16/bf16 tokens, which routes in its
 * epilogue; a routed call of more tokens uses its plan's routing and leaves
 * these arrays alone.
 *   *n_tokens  host: tokens of that call (0 if no call has routed yet)
 *   perm       device int32 [*n_tokens] (may be NULL when *n_tokens is 0)
 *   segs       device int32 [(n_slots+2)*4], the first *n_seg records valid
 *   n_seg      device int32 [1]
 * Errors: LORA_EINVAL (NULL pointers), LORA_EHIP. */
int lora_last_routing(lora_pool p, int *n_tokens, int32_t *perm, int32_t *segs, int32_t *n_seg,
                      void *stream);

/* ------------------------------------------------- route once per step -- */

/* A routing plan: the tenant-to-adapter mapping of one batch resolved once,
 * at entry, and reused by every linear of the step instead of being looked
 * up again on the hot path ["xpshop.cn article 492", 二/三: the handle is
 * resolved at request entry; "LLM 多 LoRA 推理服务工程 2026", routing layer:
 * bucketing per batch].  The plan holds a device copy of the token indices
 * and the routing arrays (the same ones lora_apply builds), sized for
 * max_tokens and n_slots.  Allocates once, here.
 * Errors: LORA_EINVAL (sizes out of range, out == NULL), LORA_ENOMEM, LORA_EHIP. */
int lora_plan_create(int max_tokens, int n_slots, lora_plan *out);

/* Waits for the plan's enqueued routing, then frees it.  The caller must not
 * destroy a plan that applies still to run on another stream read. */
int lora_plan_destroy(lora_plan plan);

/* Route a batch into the plan, asynchronously on `stream`, with pool p's slot
 * table and fused/separate policy (p->n_slots must equal the plan's).  Copies
 * token_adapter_idx (device int32 [n_tokens]) into the plan, then runs the
 * routing kernel.  Invalid tokens are counted once, here, on p's error
 * counter.  The plan records p's active slots with their ranks, policy and
 * threshold at this call; lora_apply_routed checks them.
 * Errors: LORA_EINVAL, LORA_ETOKENS (n_tokens > the plan's max_tokens),
 * LORA_EMISMATCH (slot count differs), LORA_EHIP. */
int lora_plan_route(lora_plan plan, lora_pool p, const int32_t *token_adapter_idx, int n_tokens,
                    void *stream);

/* lora_apply for the plan's batch (n_tokens = the plan's), without the
 * routing pass: the plan's routing and token indices are used.  Must follow
 * the lora_plan_route on the same stream (or an event that orders them).
 * The result equals lora_apply's with the same indices bit for bit.  Pool p
 * must match the routing pool in slot count, active slots and their ranks,
 * policy and threshold (as of the route call), else LORA_EMISMATCH and
 * nothing is enqueued: its adapters' values (A, B, alpha) may differ -- one
 * plan serves the pools of every linear of a model.  Leaves p's last-call statistics and
 * error counter unchanged.
 * Errors (host-side, nothing enqueued): LORA_EINVAL (no routed batch,
 * pointers), LORA_ETOKENS, LORA_EMISMATCH, LORA_EHIP. */
int lora_apply_routed(lora_pool p, lora_plan plan, const void *x, const void *W_base, void *y,
                      void *stream);

/* ------------------------------------------------------- async loading -- */

/* The adapter loader ["LLM 多 LoRA 推理服务工程 2026", four-layer runtime,
 * loader paragraph]: moves an adapter from host memory into a pool slot
 * without blocking the hot path -- two pinned host staging buffers and two
 * device staging buffers (double buffering: one copy in flight while the
 * next adapter is staged), a copy stream of its own, and the register-time
 * pad kernel on that stream.  One loader serves any pools of its device.
 * capacity_bytes bounds one adapter's A and B together
 * (rank * (d_in + d_out) * element size).  Allocates once, here.
 * Errors: LORA_EINVAL (capacity 0, out == NULL), LORA_ENOMEM, LORA_EHIP. */
int lora_loader_create(uint64_t capacity_bytes, lora_loader *out);

/* Waits for and commits every pending load, then frees the loader. */
int lora_loader_destroy(lora_loader l);

/* Start loading an adapter into `slot` of pool p from host memory:
 *   A_host  [rank][d_in], B_host [d_out][rank], the pool's dtype, any host
 *           memory (copied into pinned staging before this call returns; the
 *           caller may reuse it at once)
 * The slot is reserved against the tenant's quota at once (the same checks
 * and errors as lora_register, nothing changes on error) and stays LOADING
 * -- tokens naming it are invalid -- until the load is committed by
 * lora_load_poll / lora_load_wait (or by a later load reusing its staging
 * buffer), which makes it ACTIVE -- ordered on the device, as for
 * lora_register, after every call already enqueued on the pool and before
 * every later one, without waiting for them on the host.  When both staging buffers are in flight
 * the call first waits for the older one.  *ticket identifies the load.
 * The caller must wait for its loads before destroying the pool.
 * Errors: LORA_EINVAL (NULL pointers, slot out of range, adapter larger than
 * the loader's capacity), LORA_ESLOT_BUSY, LORA_ERANK, LORA_EALPHA,
 * LORA_EQUOTA, LORA_EHIP. */
int lora_load_async(lora_loader l, lora_pool p, int slot, int32_t tenant, const void *A_host,
                    const void *B_host, int rank, float alpha, uint64_t *ticket);

/* Non-blocking: *done = 1 (and the slot committed, ACTIVE) once the load's
 * copies finished, else 0.  Errors: LORA_EINVAL (unknown ticket), LORA_EHIP. */
int lora_load_poll(lora_loader l, uint64_t ticket, int *done);

/* Blocking: wait for the load's copies, then commit it.  A ticket that was
 * committed already returns LORA_OK.  Errors: LORA_EINVAL, LORA_EHIP. */
int lora_load_wait(lora_loader l, uint64_t ticket);

/* ----------------------------------------------------------- residency -- */

/* Which adapters stay resident when a pool's slots run out
 * ["LLM 多 LoRA 推理服务工程 2026", four-layer runtime, storage-pool
 * paragraph: LRU-K between the HBM tier and the tiers below; "Multi-LoRA 在线
 * 服务隔离", memory-accounting section: evict only versions with no live
 * reference, least recently used first, never weights a request holds, per-
 * tenant resident shares].  The manager takes the slots of pool p that are
 * FREE now (slots registered outside it are never touched) and loads through
 * loader l.  k: accesses of history (LRU-K; 2 is the usual choice).
 * Errors: LORA_EINVAL, LORA_ENOMEM. */
int lora_residency_create(lora_pool p, lora_loader l, int k, lora_residency *out);

/* Frees the manager; resident adapters stay registered in the pool. */
int lora_residency_destroy(lora_residency r);

/* Cap on the slots tenant's adapters may hold at once (unset: no cap).
 * Errors: LORA_EINVAL (tenant < 0, max_slots < 0). */
int lora_residency_set_share(lora_residency r, int32_t tenant, int max_slots);

/* One more holder of adapter `adapter_id` (the caller's identity of a
 * version, e.g. a digest) of `tenant`.  Resident: *slot is its slot,
 * *ticket its load's ticket (0 if committed long ago; lora_load_wait on it
 * returns at once when done).  Not resident: a slot is chosen (a free one
 * within the tenant's share, else the LRU-K victim among unreferenced slots,
 * only the tenant's own when it is at its share), the victim is unloaded
 * (lora_unregister: drains the applies that may read it) and the adapter is
 * loaded there with lora_load_async from A_host / B_host (as there); wait on
 * *ticket before routing tokens to *slot.
 * Errors: LORA_ESLOT_BUSY (every candidate slot is referenced, or the
 * tenant's share is 0; nothing changes), LORA_EINVAL (NULL pointers, id
 * resident for another tenant), and lora_load_async's errors (then the
 * chosen slot is left empty). */
int lora_residency_acquire(lora_residency r, uint64_t adapter_id, int32_t tenant, const void *A_host,
                           const void *B_host, int rank, float alpha, int *slot, uint64_t *ticket);

/* One holder fewer.  Errors: LORA_EINVAL (not resident, or no holder). */
int lora_residency_release(lora_residency r, uint64_t adapter_id);

/* Counters since creation. */
typedef struct {
    uint64_t hits, misses, evictions;
    int32_t resident;  /* slots holding an adapter of the manager */
    int32_t managed;   /* slots the manager may use */
} lora_residency_stats;

int lora_residency_stats_read(lora_residency r, lora_residency_stats *out);

/* ---------------------------------------------------------- observation -- */

/* Fill *out (synchronizes with every apply enqueued on the pool). */
int lora_pool_stats(lora_pool p, lora_stats *out);

/* Bytes currently charged to `tenant` on this pool ["Multi-LoRA 在线服务隔离",
 * memory-accounting section: resident bytes are accounted per adapter and
 * tenant, and the release gate bounds the accounting error]: the padded slot
 * bytes of the tenant's registered or loading slots.  Host-side; no device
 * call.  Errors: LORA_EINVAL (NULL pointers). */
int lora_tenant_bytes(lora_pool p, int32_t tenant, uint64_t *out);

/* Read and clear the device count of tokens lora_apply / lora_plan_route found
 * invalid ["Multi-LoRA 在线服务隔离", request identity: a missing mapping is an
 * explicit error, never a fallback; their y rows are NaN].  Synchronizes with
 * every call enqueued on the pool.  Errors: LORA_EINVAL, LORA_EHIP. */
int lora_poll_errors(lora_pool p, uint64_t *n_invalid_tokens);

/* Per-stage device time of lora_apply, for measurement.  When enabled, each
 * lora_apply (up to max_calls of them between two reads) records HIP timing
 * events on its own stream before routing and after the routing, shrink,
 * base-GEMM and separate-expand launches; a stage's time is the interval
 * between its two events.  The base-GEMM kernel is also launched with a pair
 * of events that its dispatch records itself (kernel_ms: the kernel's own
 * device time, no launch gaps).  Events are created by lora_profile_enable,
 * not on the hot path.  enable = 0 turns it off and frees the events. */
typedef struct {
    int64_t calls;      /* timed lora_apply calls since the last read */
    double route_ms;    /* summed over those calls */
    double shrink_ms;
    double gemm_ms;     /* base projection with the fused expand.  fp16/bf16
                           calls of at most 64 tokens route and shrink inside
                           their two launches and record no stage marks
                           between them: route_ms, shrink_ms and expand_ms are
                           0 and gemm_ms is the whole call (with the residual
                           expand when a bucket runs SEPARATE).  Longer fp16/
                           bf16 calls may route inside the shrink launch
                           (route_ms 0, shrink_ms both) or shrink inside the
                           GEMM launch (shrink_ms 0, gemm_ms both) */
    double expand_ms;   /* separate residual expand */
    double kernel_ms;   /* device time of the base-GEMM kernel itself (fp16/
                           bf16 pools; 0 for fp32) */
} lora_profile;

int lora_profile_enable(lora_pool p, int enable, int max_calls);

/* Synchronize with the timed calls, fill *out and start a new interval. */
int lora_profile_read(lora_pool p, lora_profile *out);

/* Static text for a status code. */
const char *lora_strerror(int status);

/* Text of the last HIP error seen by this thread inside the library ("" if
 * none). */
const char *lora_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LORA_H */
