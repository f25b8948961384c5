"""Control plane through the C ABI on the GPU: errors never fall back, quotas
are hard, unregister drains, and the resident-byte ledger is exact.

Sources: xpshop.cn article 492, sections 二/三 (hard per-tenant quota, refusal
instead of eviction, validate then attach, draining unload) and "Multi-LoRA
在线服务隔离", request identity (default deny, explicit error) and accounting
(reserve before load; resident memory error under 5% as a release gate)."""
import threading

import numpy as np
import pytest
import torch

from gpu_helpers import Pool, dev
from rank_adapter_gemm_token_amd import lora

pytestmark = pytest.mark.gpu


def _adapter(d_in, d_out, r, seed=0, dtype=torch.float16):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn((r, d_in), generator=g).to(dtype) / 16,
            torch.randn((d_out, r), generator=g).to(dtype) / 10)


def test_invalid_tokens_are_nan_and_counted_never_fallback():
    p = Pool(128, 128, 8, 4, 64, "f16")
    try:
        A, B = _adapter(128, 128, 8)
        p.register(0, A, B, 8, 16.0)
        p.register(1, A, B, 8, 16.0)
        x = dev(torch.randn(10, 128).to(torch.float16))
        W = dev(torch.randn(128, 128).to(torch.float16) / 11)
        idx = torch.tensor([0, 2, -1, 1, 4, 99, -2, 3, 0, -1], dtype=torch.int32)
        y = p.apply(x, W, dev(idx)).cpu().float()
        bad = torch.tensor([False, True, False, False, True, True, True, True, False, False])
        assert torch.isnan(y[bad]).all()
        assert torch.isfinite(y[~bad]).all()
        assert p.poll_errors() == 5
        assert p.poll_errors() == 0  # read and clear
        st = p.stats()
        assert st["last_invalid_tokens"] == 5 and st["last_base_only_tokens"] == 2
        # After unregister, the slot's tokens are invalid too (no stale adapter, no base).
        p.unregister(1)
        y2 = p.apply(x, W, dev(torch.full((10,), 1, dtype=torch.int32))).cpu().float()
        assert torch.isnan(y2).all()
        assert p.poll_errors() == 10
    finally:
        p.close()


def test_argument_errors():
    p = Pool(64, 64, 8, 4, 16, "f16")
    try:
        A, B = _adapter(64, 64, 8)
        x = dev(torch.randn(32, 64).to(torch.float16))
        W = dev(torch.randn(64, 64).to(torch.float16))
        y = torch.full((32, 64), 7.0, dtype=torch.float16, device="cuda")
        idx = dev(torch.zeros(32, dtype=torch.int32))
        lib = lora.raw_lib()
        st = torch.cuda.current_stream().cuda_stream
        assert lib.lora_apply(p.h, x.data_ptr(), W.data_ptr(), idx.data_ptr(), 17, y.data_ptr(), st) \
            == lora.LORA_ETOKENS
        assert lib.lora_apply(p.h, x.data_ptr(), W.data_ptr(), idx.data_ptr(), -1, y.data_ptr(), st) \
            == lora.LORA_EINVAL
        assert lib.lora_apply(p.h, x.data_ptr() + 2, W.data_ptr(), idx.data_ptr(), 4, y.data_ptr(), st) \
            == lora.LORA_EINVAL  # misaligned
        assert lib.lora_apply(p.h, x.data_ptr(), W.data_ptr(), idx.data_ptr(), 0, y.data_ptr(), st) == 0
        torch.cuda.synchronize()
        assert (y.cpu() == 7.0).all()  # T = 0 wrote nothing
        lora.lora_set_tenant_quota(p.h, 0, 1 << 40)
        for rank, alpha, want in [(0, 1.0, lora.LORA_ERANK), (9, 1.0, lora.LORA_ERANK),
                                  (8, float("nan"), lora.LORA_EALPHA), (8, float("inf"), lora.LORA_EALPHA)]:
            rc = lib.lora_register(p.h, 0, 0, A.cuda().data_ptr(), B.cuda().data_ptr(), rank,
                                   lora.ctypes.c_float(alpha), st)
            assert rc == want
        assert lib.lora_register(p.h, 4, 0, A.cuda().data_ptr(), B.cuda().data_ptr(), 8,
                                 lora.ctypes.c_float(1.0), st) == lora.LORA_EINVAL
        p.register(0, A, B, 8, 16.0, tenant=0)
        with pytest.raises(lora.LoraError) as e:
            p.register(0, A, B, 8, 16.0, tenant=0)
        assert e.value.status == lora.LORA_ESLOT_BUSY
        with pytest.raises(lora.LoraError) as e:
            p.unregister(3)
        assert e.value.status == lora.LORA_ESLOT_EMPTY
    finally:
        p.close()


def test_quota_is_a_hard_boundary():
    p = Pool(256, 256, 16, 8, 16, "bf16")
    try:
        A, B = _adapter(256, 256, 16, dtype=torch.bfloat16)
        slot_bytes = 16 * (256 + 256) * 2
        assert p.stats()["slot_bytes"] == slot_bytes
        lib = lora.raw_lib()
        # Default deny: no quota set.
        with pytest.raises(lora.LoraError) as e:
            lora.lora_register(p.h, 0, 5, dev(A), dev(B), 16, 32.0)
        assert e.value.status == lora.LORA_EQUOTA
        lora.lora_set_tenant_quota(p.h, 5, 2 * slot_bytes)
        lora.lora_set_tenant_quota(p.h, 6, 10 * slot_bytes)
        lora.lora_register(p.h, 0, 5, dev(A), dev(B), 16, 32.0)
        lora.lora_register(p.h, 1, 6, dev(A), dev(B), 16, 32.0)
        lora.lora_register(p.h, 2, 5, dev(A), dev(B), 16, 32.0)
        with pytest.raises(lora.LoraError) as e:
            lora.lora_register(p.h, 3, 5, dev(A), dev(B), 16, 32.0)
        assert e.value.status == lora.LORA_EQUOTA
        # Nothing was evicted, the other tenant is untouched, bytes are exact.
        st = p.stats()
        assert st["active_slots"] == 3
        assert lora.lora_tenant_bytes(p.h, 5) == 2 * slot_bytes
        assert lora.lora_tenant_bytes(p.h, 6) == slot_bytes
        assert st["resident_bytes"] == 3 * slot_bytes
        lora.lora_unregister(p.h, 0)
        assert lora.lora_tenant_bytes(p.h, 5) == slot_bytes
        lora.lora_register(p.h, 3, 5, dev(A), dev(B), 16, 32.0)
        assert p.stats()["resident_bytes"] == 3 * slot_bytes
    finally:
        p.close()


def test_resident_bytes_match_device_memory():
    # The ledger charges slot_bytes per slot; the slabs occupy exactly S slots.
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    # Large enough (256 MiB of slabs) that the runtime's fixed per-pool
    # overhead (stream, allocation granularity) stays far below 5%.
    S, R, d_in, d_out = 1024, 16, 4096, 4096
    p = Pool(d_in, d_out, R, S, 64, "f16")
    try:
        free1, _ = torch.cuda.mem_get_info()
        st = p.stats()
        slabs = S * st["slot_bytes"]
        assert st["slot_bytes"] == R * (d_in + d_out) * 2
        used = free0 - free1
        # Device memory the pool holds matches what it reports within 5% ...
        assert abs(used - st["device_bytes"]) <= 0.05 * st["device_bytes"]
        # ... and the adapter slabs it charges to tenants are exactly S slots.
        assert st["device_bytes"] >= slabs
        for s in range(4):
            A, B = _adapter(d_in, d_out, R, s)
            p.register(s, A, B, R, 2.0 * R, tenant=s % 2)
        st = p.stats()
        assert st["resident_bytes"] == 4 * st["slot_bytes"]
        assert lora.lora_tenant_bytes(p.h, 0) + lora.lora_tenant_bytes(p.h, 1) == st["resident_bytes"]
    finally:
        p.close()


def test_unregister_drains_in_flight_work():
    d, T = 4096, 64
    p = Pool(d, d, 16, 2, T, "f16")
    try:
        A, B = _adapter(d, d, 16)
        p.register(0, A, B, 16, 32.0)
        x = dev(torch.randn(T, d).to(torch.float16))
        W = dev(torch.randn(d, d).to(torch.float16) / 64)
        idx = dev(torch.zeros(T, dtype=torch.int32))
        y = torch.empty((T, d), dtype=torch.float16, device="cuda")
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            for _ in range(300):
                p.apply(x, W, idx, y, stream=s)
            done = torch.cuda.Event()
            done.record(s)
        p.unregister(0)  # must not return before the 300 applies have finished
        assert done.query()
        assert not torch.isnan(y.float()).any()  # they ran with the adapter, not freed memory
    finally:
        p.close()


def test_apply_from_second_thread_waits_for_unregister():
    d, T = 1024, 32
    p = Pool(d, d, 16, 2, T, "f16")
    try:
        A, B = _adapter(d, d, 16)
        p.register(0, A, B, 16, 32.0)
        x = dev(torch.randn(T, d).to(torch.float16))
        W = dev(torch.randn(d, d).to(torch.float16) / 32)
        idx = dev(torch.zeros(T, dtype=torch.int32))
        outs = []

        def worker():
            for _ in range(50):
                outs.append(p.apply(x, W, idx))
            torch.cuda.synchronize()

        th = threading.Thread(target=worker)
        th.start()
        p.unregister(0)
        th.join()
        # Each call either ran entirely before the drain (finite) or entirely
        # after it (slot free -> all NaN); never a mixture inside one call.
        for y in outs:
            yf = y.float()
            nan = torch.isnan(yf)
            assert bool(nan.all()) or not bool(nan.any())
    finally:
        p.close()


def test_stats_zero_pad_fraction():
    # Two LoRA tokens of rank 8 and one of rank 32 in an R = 64 pool.
    p = Pool(64, 64, 64, 3, 8, "bf16")
    try:
        for s, r in enumerate([8, 32, 64]):
            A, B = _adapter(64, 64, r, s, torch.bfloat16)
            p.register(s, A, B, r, 2.0 * r)
        x = dev(torch.randn(5, 64).to(torch.bfloat16))
        W = dev(torch.randn(64, 64).to(torch.bfloat16))
        p.apply(x, W, dev(torch.tensor([0, 0, 1, -1, 7], dtype=torch.int32)))
        st = p.stats()
        assert st["last_tokens"] == 5 and st["last_adapters"] == 2
        assert st["last_lora_rows_padded"] == 3 * 64
        assert st["last_lora_rows_true"] == 8 + 8 + 32
        assert abs(st["last_zero_pad_fraction"] - (1 - 48 / 192)) < 1e-12
        assert p.poll_errors() == 1
        # 130 tokens on 64 x 64 route inside the shrink launch (workgroup 0
        # writes the statistics and the error count): the same figures.
        p.close()
        p = Pool(64, 64, 64, 3, 130, "bf16")
        for s, r in enumerate([8, 32, 64]):
            A, B = _adapter(64, 64, r, s, torch.bfloat16)
            p.register(s, A, B, r, 2.0 * r)
        idx = torch.tensor([0, 0, 1, -1, 7] * 26, dtype=torch.int32)
        p.apply(dev(torch.randn(130, 64).to(torch.bfloat16)), dev(torch.randn(64, 64).to(torch.bfloat16)), dev(idx))
        st = p.stats()
        assert st["last_tokens"] == 130 and st["last_adapters"] == 2
        assert st["last_lora_rows_padded"] == 3 * 26 * 64
        assert st["last_lora_rows_true"] == (8 + 8 + 32) * 26
        assert p.poll_errors() == 26
    finally:
        p.close()


def test_stage_profile_counts_calls_and_stages():
    # Opt-in stage timing: one event set per call, every stage non-negative.
    d = 1024
    p = Pool(d, d, 16, 2, 128, "f16")
    try:
        A, B = _adapter(d, d, 16)
        p.register(0, A, B, 16, 32.0)
        W = dev(torch.randn(d, d).to(torch.float16) / 32)
        lora.lora_profile_enable(p.h, 1, 8)
        for T in (64, 64, 64):
            p.apply(dev(torch.randn(T, d).to(torch.float16)), W, dev(torch.zeros(T, dtype=torch.int32)))
        r = lora.lora_profile_read(p.h)
        assert r["calls"] == 3
        # Calls of at most 64 tokens: no separate route, shrink or expand
        # launch, so those stages read exactly 0 and gemm_ms is the call.
        assert r["gemm_ms"] > 0 and r["route_ms"] == 0 and r["shrink_ms"] == 0 and r["expand_ms"] == 0
        # The main kernel's own dispatch time lies inside its stage interval.
        assert 0 < r["kernel_ms"] <= r["gemm_ms"] + 1e-3
        assert min(r[k] for k in r if k.endswith("_ms")) >= 0
        for T in (128, 128):
            p.apply(dev(torch.randn(T, d).to(torch.float16)), W, dev(torch.zeros(T, dtype=torch.int32)))
        r = lora.lora_profile_read(p.h)
        assert r["calls"] == 2 and r["gemm_ms"] > 0 and r["shrink_ms"] > 0 and r["route_ms"] > 0
        assert 0 < r["kernel_ms"] <= r["gemm_ms"] + 1e-3
        lora.lora_profile_enable(p.h, 0)
        p.apply(dev(torch.randn(8, d).to(torch.float16)), W, dev(torch.zeros(8, dtype=torch.int32)))
        assert lora.lora_profile_read(p.h)["calls"] == 0
    finally:
        p.close()
    # 300 tokens on 4096 -> 2048 route inside the shrink launch: the route
    # stage holds no launch, the shrink stage both.
    p = Pool(4096, 2048, 16, 2, 300, "f16")
    try:
        A, B = _adapter(4096, 2048, 16)
        p.register(1, A, B, 16, 32.0)
        W = dev(torch.randn(2048, 4096).to(torch.float16) / 64)
        lora.lora_profile_enable(p.h, 1, 8)
        for _ in range(2):
            p.apply(dev(torch.randn(300, 4096).to(torch.float16)), W, dev(torch.ones(300, dtype=torch.int32)))
        r = lora.lora_profile_read(p.h)
        assert r["calls"] == 2 and r["gemm_ms"] > 0 and r["shrink_ms"] > r["route_ms"] >= 0
        assert 0 < r["kernel_ms"] <= r["gemm_ms"] + 1e-3
    finally:
        p.close()


def test_default_policy_is_the_gfx950_threshold():
    # AUTO with the threshold the library ships for gfx950 (every LoRA bucket
    # fused, from the fused/separate sweep).
    p = Pool(64, 64, 8, 2, 4, "f16")
    try:
        assert lora.lora_get_policy(p.h) == (lora.LORA_MODE_AUTO, 0)
    finally:
        p.close()
