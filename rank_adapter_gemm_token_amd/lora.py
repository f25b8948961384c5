"""Thin ctypes binding of liblora.so (include/lora.h), same names as the C ABI.

Argument marshalling only: tensors become device pointers, streams become raw
hipStream_t handles, non-zero status codes become LoraError.  Every step of
the computation runs in liblora.so's HIP kernels; nothing here computes, and
there is no fallback: importing this module fails if liblora.so is missing.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblora.so")
if not os.path.exists(LIB_PATH):
    raise ImportError("liblora.so is not built (%s); run `python -m rank_adapter_gemm_token_amd.build` "
                      "or __graft_entry__.build()" % LIB_PATH)
_lib = ctypes.CDLL(LIB_PATH)

LORA_F32, LORA_F16, LORA_BF16 = 0, 1, 2
LORA_MODE_AUTO, LORA_MODE_FUSED, LORA_MODE_SEPARATE = 0, 1, 2
LORA_SEG_NONE, LORA_SEG_FUSED, LORA_SEG_SEPARATE = 0, 1, 2
LORA_BASE_ONLY = -1
LORA_MAX_SLOTS = 1024
LORA_MAX_RANK = 64

LORA_OK = 0
LORA_EINVAL = -1
LORA_ETOKENS = -2
LORA_ESLOT_BUSY = -3
LORA_ESLOT_EMPTY = -4
LORA_ERANK = -5
LORA_EALPHA = -6
LORA_EQUOTA = -7
LORA_EMISMATCH = -8
LORA_ENOMEM = -9
LORA_EHIP = -10
LORA_ESCRATCH = -11
LORA_NOALLOC_SCRATCH_BYTES = 32 << 20

DTYPE_OF = {torch.float32: LORA_F32, torch.float16: LORA_F16, torch.bfloat16: LORA_BF16}
TORCH_DTYPE = {v: k for k, v in DTYPE_OF.items()}

# Every symbol include/lora.h declares, in declaration order.
EXPORTS = ["lora_pool_create", "lora_pool_destroy", "lora_set_tenant_quota", "lora_register",
           "lora_unregister", "lora_set_policy", "lora_get_policy", "lora_set_shrink_wait_polls", "lora_apply",
           "lora_apply_noalloc", "lora_route",
           "lora_last_routing",
           "lora_plan_create", "lora_plan_destroy", "lora_plan_route", "lora_apply_routed",
           "lora_loader_create", "lora_loader_destroy", "lora_load_async", "lora_load_poll", "lora_load_wait",
           "lora_residency_create", "lora_residency_destroy", "lora_residency_set_share",
           "lora_residency_acquire", "lora_residency_release", "lora_residency_stats_read",
           "lora_pool_stats", "lora_tenant_bytes", "lora_poll_errors", "lora_profile_enable",
           "lora_profile_read", "lora_strerror", "lora_last_hip_error"]


class lora_stats(ctypes.Structure):
    _fields_ = [("d_in", ctypes.c_int32), ("d_out", ctypes.c_int32), ("max_rank", ctypes.c_int32),
                ("n_slots", ctypes.c_int32), ("max_tokens", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("active_slots", ctypes.c_int32), ("draining_slots", ctypes.c_int32),
                ("slot_bytes", ctypes.c_uint64), ("resident_bytes", ctypes.c_uint64),
                ("device_bytes", ctypes.c_uint64),
                ("last_tokens", ctypes.c_int32), ("last_adapters", ctypes.c_int32),
                ("last_fused_buckets", ctypes.c_int32), ("last_separate_buckets", ctypes.c_int32),
                ("last_base_only_tokens", ctypes.c_int32), ("last_invalid_tokens", ctypes.c_int32),
                ("last_lora_rows_padded", ctypes.c_int64), ("last_lora_rows_true", ctypes.c_int64),
                ("last_zero_pad_fraction", ctypes.c_double)]


class lora_residency_stats(ctypes.Structure):
    _fields_ = [("hits", ctypes.c_uint64), ("misses", ctypes.c_uint64), ("evictions", ctypes.c_uint64),
                ("resident", ctypes.c_int32), ("managed", ctypes.c_int32)]


class lora_profile(ctypes.Structure):
    _fields_ = [("calls", ctypes.c_int64), ("route_ms", ctypes.c_double), ("shrink_ms", ctypes.c_double),
                ("gemm_ms", ctypes.c_double), ("expand_ms", ctypes.c_double),
                ("kernel_ms", ctypes.c_double)]


_vp = ctypes.c_void_p
_i = ctypes.c_int
_lib.lora_pool_create.argtypes = [_i, _i, _i, _i, _i, _i, ctypes.POINTER(_vp)]
_lib.lora_pool_destroy.argtypes = [_vp]
_lib.lora_set_tenant_quota.argtypes = [_vp, ctypes.c_int32, ctypes.c_uint64]
_lib.lora_register.argtypes = [_vp, _i, ctypes.c_int32, _vp, _vp, _i, ctypes.c_float, _vp]
_lib.lora_unregister.argtypes = [_vp, _i]
_lib.lora_set_policy.argtypes = [_vp, _i, _i]
_lib.lora_set_shrink_wait_polls.argtypes = [_vp, _i]
_lib.lora_get_policy.argtypes = [_vp, ctypes.POINTER(_i), ctypes.POINTER(_i)]
_lib.lora_apply.argtypes = [_vp, _vp, _vp, _vp, _i, _vp, _vp]
_lib.lora_apply_noalloc.argtypes = [_vp, _vp, _vp, _vp, _i, _vp, _vp]
_lib.lora_route.argtypes = [_vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.lora_last_routing.argtypes = [_vp, ctypes.POINTER(_i), _vp, _vp, _vp, _vp]
_lib.lora_plan_create.argtypes = [_i, _i, ctypes.POINTER(_vp)]
_lib.lora_plan_destroy.argtypes = [_vp]
_lib.lora_plan_route.argtypes = [_vp, _vp, _vp, _i, _vp]
_lib.lora_apply_routed.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp]
_lib.lora_loader_create.argtypes = [ctypes.c_uint64, ctypes.POINTER(_vp)]
_lib.lora_loader_destroy.argtypes = [_vp]
_lib.lora_load_async.argtypes = [_vp, _vp, _i, ctypes.c_int32, _vp, _vp, _i, ctypes.c_float,
                                 ctypes.POINTER(ctypes.c_uint64)]
_lib.lora_load_poll.argtypes = [_vp, ctypes.c_uint64, ctypes.POINTER(_i)]
_lib.lora_load_wait.argtypes = [_vp, ctypes.c_uint64]
_lib.lora_residency_create.argtypes = [_vp, _vp, _i, ctypes.POINTER(_vp)]
_lib.lora_residency_destroy.argtypes = [_vp]
_lib.lora_residency_set_share.argtypes = [_vp, ctypes.c_int32, _i]
_lib.lora_residency_acquire.argtypes = [_vp, ctypes.c_uint64, ctypes.c_int32, _vp, _vp, _i, ctypes.c_float,
                                        ctypes.POINTER(_i), ctypes.POINTER(ctypes.c_uint64)]
_lib.lora_residency_release.argtypes = [_vp, ctypes.c_uint64]
_lib.lora_residency_stats_read.argtypes = [_vp, ctypes.POINTER(lora_residency_stats)]
_lib.lora_pool_stats.argtypes = [_vp, ctypes.POINTER(lora_stats)]
_lib.lora_tenant_bytes.argtypes = [_vp, ctypes.c_int32, ctypes.POINTER(ctypes.c_uint64)]
_lib.lora_poll_errors.argtypes = [_vp, ctypes.POINTER(ctypes.c_uint64)]
_lib.lora_profile_enable.argtypes = [_vp, _i, _i]
_lib.lora_profile_read.argtypes = [_vp, ctypes.POINTER(lora_profile)]
_lib.lora_strerror.argtypes = [_i]
_lib.lora_strerror.restype = ctypes.c_char_p
_lib.lora_last_hip_error.argtypes = []
_lib.lora_last_hip_error.restype = ctypes.c_char_p
for _n in EXPORTS:
    if _n not in ("lora_strerror", "lora_last_hip_error"):
        getattr(_lib, _n).restype = ctypes.c_int


class LoraError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        text = lora_strerror(status)
        if status == LORA_EHIP:
            text += ": " + _lib.lora_last_hip_error().decode()
        super().__init__("%s failed: %s (%d)" % (where, text, status))


def _check(rc, where):
    if rc != LORA_OK:
        raise LoraError(rc, where)


def _ptr(t):
    """Device pointer of a contiguous CUDA tensor (or a raw int / None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(s):
    if s is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def lora_strerror(status):
    return _lib.lora_strerror(int(status)).decode()


# Shapes of the pools created through this binding, so that a tensor of the
# wrong size or dtype is refused here instead of reaching a kernel.
_shapes = {}


def _need(t, numel, dtype, what):
    if isinstance(t, torch.Tensor):
        if t.dtype != dtype:
            raise ValueError("%s: expected %s, got %s" % (what, dtype, t.dtype))
        if t.numel() < numel:
            raise ValueError("%s: expected at least %d elements, got %d" % (what, numel, t.numel()))


def lora_pool_create(d_in, d_out, max_rank, n_slots, max_tokens, dtype):
    """Returns the pool handle (an int).  dtype: torch dtype or LORA_F32/F16/BF16."""
    if isinstance(dtype, torch.dtype):
        dtype = DTYPE_OF[dtype]
    h = _vp()
    _check(_lib.lora_pool_create(d_in, d_out, max_rank, n_slots, max_tokens, int(dtype), ctypes.byref(h)),
           "lora_pool_create")
    _shapes[h.value] = dict(d_in=d_in, d_out=d_out, R=max_rank, S=n_slots, max_T=max_tokens,
                            dtype=TORCH_DTYPE[int(dtype)])
    return h.value


def lora_pool_destroy(pool):
    _check(_lib.lora_pool_destroy(pool), "lora_pool_destroy")
    _shapes.pop(pool, None)


def lora_set_tenant_quota(pool, tenant, nbytes):
    _check(_lib.lora_set_tenant_quota(pool, tenant, nbytes), "lora_set_tenant_quota")


def lora_register(pool, slot, tenant, A, B, rank, alpha, stream=None):
    sh = _shapes.get(pool)
    if sh is not None and 0 < rank:
        _need(A, rank * sh["d_in"], sh["dtype"], "A")
        _need(B, sh["d_out"] * rank, sh["dtype"], "B")
    _check(_lib.lora_register(pool, slot, tenant, _ptr(A), _ptr(B), rank, float(alpha), _stream(stream)),
           "lora_register")


def lora_unregister(pool, slot):
    _check(_lib.lora_unregister(pool, slot), "lora_unregister")


def lora_set_policy(pool, mode, threshold):
    _check(_lib.lora_set_policy(pool, int(mode), int(threshold)), "lora_set_policy")


def lora_set_shrink_wait_polls(pool, polls):
    _check(_lib.lora_set_shrink_wait_polls(pool, int(polls)), "lora_set_shrink_wait_polls")


def lora_get_policy(pool):
    m, t = _i(), _i()
    _check(_lib.lora_get_policy(pool, ctypes.byref(m), ctypes.byref(t)), "lora_get_policy")
    return m.value, t.value


def lora_apply(pool, x, W_base, token_adapter_idx, n_tokens, y, stream=None):
    sh = _shapes.get(pool)
    if sh is not None and 0 < n_tokens <= sh["max_T"]:
        _need(x, n_tokens * sh["d_in"], sh["dtype"], "x")
        _need(W_base, sh["d_out"] * sh["d_in"], sh["dtype"], "W_base")
        _need(token_adapter_idx, n_tokens, torch.int32, "token_adapter_idx")
        _need(y, n_tokens * sh["d_out"], sh["dtype"], "y")
    _check(_lib.lora_apply(pool, _ptr(x), _ptr(W_base), _ptr(token_adapter_idx), int(n_tokens), _ptr(y),
                           _stream(stream)), "lora_apply")


def lora_apply_noalloc(pool, x, W_base, token_adapter_idx, n_tokens, y, stream=None):
    sh = _shapes.get(pool)
    if sh is not None and 0 < n_tokens <= sh["max_T"]:
        _need(x, n_tokens * sh["d_in"], sh["dtype"], "x")
        _need(W_base, sh["d_out"] * sh["d_in"], sh["dtype"], "W_base")
        _need(token_adapter_idx, n_tokens, torch.int32, "token_adapter_idx")
        _need(y, n_tokens * sh["d_out"], sh["dtype"], "y")
    _check(_lib.lora_apply_noalloc(pool, _ptr(x), _ptr(W_base), _ptr(token_adapter_idx), int(n_tokens), _ptr(y),
                                   _stream(stream)), "lora_apply_noalloc")


def lora_route(pool, token_adapter_idx, n_tokens, counts, offsets, perm, segs, n_seg, stream=None):
    sh = _shapes.get(pool)
    if sh is not None and 0 <= n_tokens <= sh["max_T"]:
        S = sh["S"]
        _need(token_adapter_idx, n_tokens, torch.int32, "token_adapter_idx")
        _need(counts, S + 2, torch.int32, "counts")
        _need(offsets, S + 3, torch.int32, "offsets")
        _need(perm, n_tokens, torch.int32, "perm")
        _need(segs, (S + 2) * 4, torch.int32, "segs")
        _need(n_seg, 1, torch.int32, "n_seg")
    _check(_lib.lora_route(pool, _ptr(token_adapter_idx), int(n_tokens), _ptr(counts), _ptr(offsets),
                           _ptr(perm), _ptr(segs), _ptr(n_seg), _stream(stream)), "lora_route")


def lora_last_routing(pool, perm, segs, n_seg, stream=None):
    """Copies the routing the pool's kernels last used into perm / segs / n_seg
    (device int32 tensors); returns that call's token count."""
    sh = _shapes.get(pool)
    if sh is not None:
        _need(segs, (sh["S"] + 2) * 4, torch.int32, "segs")
        _need(n_seg, 1, torch.int32, "n_seg")
        _need(perm, 0, torch.int32, "perm")  # the call's token count is known after it
    n = _i()
    _check(_lib.lora_last_routing(pool, ctypes.byref(n), _ptr(perm), _ptr(segs), _ptr(n_seg), _stream(stream)),
           "lora_last_routing")
    return n.value


# Plans created through this binding: capacity and the last routed batch size.
_plans = {}


def lora_plan_create(max_tokens, n_slots):
    """Returns the plan handle (an int)."""
    h = _vp()
    _check(_lib.lora_plan_create(int(max_tokens), int(n_slots), ctypes.byref(h)), "lora_plan_create")
    _plans[h.value] = dict(max_T=max_tokens, S=n_slots, T=None)
    return h.value


def lora_plan_destroy(plan):
    _check(_lib.lora_plan_destroy(plan), "lora_plan_destroy")
    _plans.pop(plan, None)


def lora_plan_route(plan, pool, token_adapter_idx, n_tokens, stream=None):
    pl = _plans.get(plan)
    if pl is not None and 0 <= n_tokens <= pl["max_T"]:
        _need(token_adapter_idx, n_tokens, torch.int32, "token_adapter_idx")
    _check(_lib.lora_plan_route(plan, pool, _ptr(token_adapter_idx), int(n_tokens), _stream(stream)),
           "lora_plan_route")
    if pl is not None:
        pl["T"] = int(n_tokens)


def lora_apply_routed(pool, plan, x, W_base, y, stream=None):
    sh, pl = _shapes.get(pool), _plans.get(plan)
    if sh is not None and pl is not None and pl["T"] is not None and 0 < pl["T"] <= sh["max_T"]:
        T = pl["T"]
        _need(x, T * sh["d_in"], sh["dtype"], "x")
        _need(W_base, sh["d_out"] * sh["d_in"], sh["dtype"], "W_base")
        _need(y, T * sh["d_out"], sh["dtype"], "y")
    _check(_lib.lora_apply_routed(pool, plan, _ptr(x), _ptr(W_base), _ptr(y), _stream(stream)),
           "lora_apply_routed")


def lora_loader_create(capacity_bytes):
    """Returns the loader handle (an int)."""
    h = _vp()
    _check(_lib.lora_loader_create(int(capacity_bytes), ctypes.byref(h)), "lora_loader_create")
    return h.value


def lora_loader_destroy(loader):
    _check(_lib.lora_loader_destroy(loader), "lora_loader_destroy")


def _host_ptr(t):
    """Host pointer of a contiguous CPU tensor (or a raw int)."""
    if isinstance(t, int):
        return t
    if t.is_cuda:
        raise ValueError("expected a host tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def lora_load_async(loader, pool, slot, tenant, A_host, B_host, rank, alpha):
    """Start loading host A [rank][d_in], B [d_out][rank] into `slot`; returns the ticket."""
    sh = _shapes.get(pool)
    if sh is not None and 0 < rank:
        _need(A_host, rank * sh["d_in"], sh["dtype"], "A")
        _need(B_host, sh["d_out"] * rank, sh["dtype"], "B")
    t = ctypes.c_uint64()
    _check(_lib.lora_load_async(loader, pool, int(slot), int(tenant), _host_ptr(A_host), _host_ptr(B_host),
                                int(rank), float(alpha), ctypes.byref(t)), "lora_load_async")
    return t.value


def lora_load_poll(loader, ticket):
    d = _i()
    _check(_lib.lora_load_poll(loader, int(ticket), ctypes.byref(d)), "lora_load_poll")
    return bool(d.value)


def lora_load_wait(loader, ticket):
    _check(_lib.lora_load_wait(loader, int(ticket)), "lora_load_wait")


def lora_residency_create(pool, loader, k=2):
    h = _vp()
    _check(_lib.lora_residency_create(pool, loader, int(k), ctypes.byref(h)), "lora_residency_create")
    return h.value


def lora_residency_destroy(res):
    _check(_lib.lora_residency_destroy(res), "lora_residency_destroy")


def lora_residency_set_share(res, tenant, max_slots):
    _check(_lib.lora_residency_set_share(res, int(tenant), int(max_slots)), "lora_residency_set_share")


def lora_residency_acquire(res, adapter_id, tenant, A_host, B_host, rank, alpha):
    """Returns (slot, ticket); ticket 0 for an adapter resident and committed."""
    s, t = _i(), ctypes.c_uint64()
    _check(_lib.lora_residency_acquire(res, int(adapter_id), int(tenant),
                                       None if A_host is None else _host_ptr(A_host),
                                       None if B_host is None else _host_ptr(B_host), int(rank), float(alpha),
                                       ctypes.byref(s), ctypes.byref(t)), "lora_residency_acquire")
    return s.value, t.value


def lora_residency_release(res, adapter_id):
    _check(_lib.lora_residency_release(res, int(adapter_id)), "lora_residency_release")


def lora_residency_stats_read(res):
    st = lora_residency_stats()
    _check(_lib.lora_residency_stats_read(res, ctypes.byref(st)), "lora_residency_stats_read")
    return {name: getattr(st, name) for name, _ in lora_residency_stats._fields_}


def lora_pool_stats(pool):
    s = lora_stats()
    _check(_lib.lora_pool_stats(pool, ctypes.byref(s)), "lora_pool_stats")
    return {name: getattr(s, name) for name, _ in lora_stats._fields_}


def lora_tenant_bytes(pool, tenant):
    v = ctypes.c_uint64()
    _check(_lib.lora_tenant_bytes(pool, tenant, ctypes.byref(v)), "lora_tenant_bytes")
    return v.value


def lora_poll_errors(pool):
    v = ctypes.c_uint64()
    _check(_lib.lora_poll_errors(pool, ctypes.byref(v)), "lora_poll_errors")
    return v.value


def lora_profile_enable(pool, enable, max_calls=1):
    _check(_lib.lora_profile_enable(pool, int(bool(enable)), int(max_calls)), "lora_profile_enable")


def lora_profile_read(pool):
    v = lora_profile()
    _check(_lib.lora_profile_read(pool, ctypes.byref(v)), "lora_profile_read")
    return {name: getattr(v, name) for name, _ in lora_profile._fields_}


def raw_lib():
    """The loaded CDLL, for tests that call the C ABI directly."""
    return _lib
