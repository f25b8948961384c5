"""Route once per step (lora_plan_route + lora_apply_routed) on the GPU,
through the C ABI.

A routed apply runs the same kernels on the same routing as lora_apply, so
its output must equal lora_apply's bit for bit -- on the routing pool and on
any other pool with the same slot count, active slots, ranks and policy
(other adapter values, other weights): one plan serves every linear of a
step.  A pool
whose routing inputs differ is refused (LORA_EMISMATCH) before anything is
enqueued.  lora_apply itself is compared with the oracle elsewhere
(test_apply_gpu.py)."""
import numpy as np
import pytest
import torch

from gpu_helpers import Pool, assert_close, dev, reference
from rank_adapter_gemm_token_amd import lora
from rank_adapter_gemm_token_amd import workloads as wl
from test_apply_gpu import _small_case

pytestmark = pytest.mark.gpu


def _pool_with(dtype, T, d_in, d_out, S, R, seed, policy=0, ranks=None):
    """A pool of S adapters; `ranks` (slot -> rank) fixes the ranks (the
    adapters' values still come from `seed`)."""
    x, W, ads, idx = _small_case(dtype, T, d_in, d_out, S, R, seed)
    if ranks is not None:
        rng = np.random.default_rng(seed + 1000)
        tdt = x.dtype
        ads = [wl.Adapter(a.slot, a.tenant, ranks[a.slot], float(2 * ranks[a.slot]),
                          torch.from_numpy(rng.standard_normal((ranks[a.slot], d_in)) / np.sqrt(d_in)).to(tdt),
                          torch.from_numpy(rng.standard_normal((d_out, ranks[a.slot])) * 0.1).to(tdt))
               for a in ads]
    p = Pool(d_in, d_out, R, S, T, dtype, policy, 4)
    p.register_all(ads)
    return p, x, W, idx


def _ranks(p):
    return {s: v[2] for s, v in p.adapters.items()}


def _routed(p, plan, x, W, T):
    y = torch.full((T, p.d_out), 7.0, dtype=x.dtype, device="cuda")
    lora.lora_apply_routed(p.h, plan, dev(x), dev(W), y)
    return y


# Shapes reach the decode path (T <= 64), the split-K 256-row tiles (65 ..
# 2047), the register-staged tiles (d_out off the 128 grid) and fp32.
@pytest.mark.parametrize("dtype,T,d_in,d_out,S,R", [("f16", 37, 128, 192, 5, 8), ("bf16", 64, 256, 128, 20, 64),
                                                    ("bf16", 300, 256, 256, 17, 16), ("f16", 200, 128, 192, 9, 32),
                                                    ("f32", 77, 64, 64, 6, 8)])
@pytest.mark.parametrize("policy", [0, 2])
def test_routed_equals_apply_across_pools(dtype, T, d_in, d_out, S, R, policy):
    pa, xa, Wa, idx = _pool_with(dtype, T, d_in, d_out, S, R, seed=T + 1, policy=policy)
    # A second linear: same slot count, active slots and ranks; other adapter
    # values and W.
    pb, xb, Wb, _ = _pool_with(dtype, T, d_in, d_out, S, R, seed=T + 2, policy=policy, ranks=_ranks(pa))
    plan = lora.lora_plan_create(T, S)
    try:
        ya = pa.apply(dev(xa), dev(Wa), dev(idx))
        yb = pb.apply(dev(xb), dev(Wb), dev(idx))
        lora.lora_plan_route(plan, pa.h, dev(idx), T)
        ra = _routed(pa, plan, xa, Wa, T)
        rb = _routed(pb, plan, xb, Wb, T)
        torch.cuda.synchronize()
        for got, want in ((ra, ya), (rb, yb)):
            g, w = got.cpu(), want.cpu()
            assert torch.equal(torch.isnan(g), torch.isnan(w))
            assert torch.equal(torch.nan_to_num(g, nan=0.0), torch.nan_to_num(w, nan=0.0))
        # And against the oracle, for the second pool (routing from the first).
        y_ref, inv = reference(pb, xb, Wb, idx)
        assert_close(rb.cpu(), y_ref, inv, dtype)
    finally:
        lora.lora_plan_destroy(plan)
        pa.close()
        pb.close()


def test_plan_reused_for_many_calls_and_errors_counted_once():
    T, S = 130, 9
    pa, xa, Wa, idx = _pool_with("bf16", T, 256, 128, S, 16, seed=5)
    pb, xb, Wb, _ = _pool_with("bf16", T, 256, 128, S, 16, seed=6, ranks=_ranks(pa))
    n_inv = int(((idx < -1) | (idx >= S)).sum())
    assert n_inv > 0
    plan = lora.lora_plan_create(T + 10, S)
    try:
        pa.poll_errors()
        pb.poll_errors()
        lora.lora_plan_route(plan, pa.h, dev(idx), T)
        outs = [_routed(pb, plan, xb, Wb, T) for _ in range(3)]
        torch.cuda.synchronize()
        for o in outs[1:]:
            assert torch.equal(torch.nan_to_num(o.cpu(), nan=0.0), torch.nan_to_num(outs[0].cpu(), nan=0.0))
        y_ref, inv = reference(pb, xb, Wb, idx)
        assert_close(outs[0].cpu(), y_ref, inv, "bf16")
        assert pa.poll_errors() == n_inv   # counted once, at routing
        assert pb.poll_errors() == 0       # routed applies do not count again
    finally:
        lora.lora_plan_destroy(plan)
        pa.close()
        pb.close()


def test_mismatched_pools_are_refused():
    T, S = 40, 6
    pa, xa, Wa, idx = _pool_with("f16", T, 128, 128, S, 8, seed=11)
    plan = lora.lora_plan_create(T, S)
    others = []
    try:
        lora.lora_plan_route(plan, pa.h, dev(idx), T)
        rk = _ranks(pa)
        # Fewer active slots.
        pc, xc, Wc, _ = _pool_with("f16", T, 128, 128, S, 8, seed=12, ranks=rk)
        others.append(pc)
        pc.unregister(3)
        # Other policy.
        pd, xd, Wd, _ = _pool_with("f16", T, 128, 128, S, 8, seed=13, policy=2, ranks=rk)
        others.append(pd)
        # Other slot count (routing into it is refused too).
        pe, xe, We, _ = _pool_with("f16", T, 128, 128, S + 1, 8, seed=14)
        others.append(pe)
        # Same active slots, one of another rank.
        rk2 = dict(rk)
        rk2[2] = 1 if rk[2] != 1 else 2
        pf, xf, Wf, _ = _pool_with("f16", T, 128, 128, S, 8, seed=15, ranks=rk2)
        others.append(pf)
        for p, x, W in ((pc, xc, Wc), (pd, xd, Wd), (pe, xe, We), (pf, xf, Wf)):
            y = torch.full((T, p.d_out), 3.0, dtype=torch.float16, device="cuda")
            with pytest.raises(lora.LoraError) as ei:
                lora.lora_apply_routed(p.h, plan, dev(x), dev(W), y)
            assert ei.value.status == lora.LORA_EMISMATCH
            torch.cuda.synchronize()
            assert bool((y == 3.0).all())  # nothing was enqueued
        with pytest.raises(lora.LoraError) as ei:
            lora.lora_plan_route(plan, pe.h, dev(idx), T)
        assert ei.value.status == lora.LORA_EMISMATCH
        # The routing pool itself, after one of its slots is unregistered.
        pa.unregister(0)
        y = torch.empty((T, pa.d_out), dtype=torch.float16, device="cuda")
        with pytest.raises(lora.LoraError) as ei:
            lora.lora_apply_routed(pa.h, plan, dev(xa), dev(Wa), y)
        assert ei.value.status == lora.LORA_EMISMATCH
        # Too many tokens for the plan.
        with pytest.raises(lora.LoraError) as ei:
            lora.lora_plan_route(plan, pa.h, dev(torch.zeros(T + 1, dtype=torch.int32)), T + 1)
        assert ei.value.status == lora.LORA_ETOKENS
    finally:
        lora.lora_plan_destroy(plan)
        pa.close()
        for p in others:
            p.close()


def test_unrouted_plan_and_empty_batch():
    S = 4
    pa, xa, Wa, idx = _pool_with("f16", 16, 64, 64, S, 8, seed=21)
    plan = lora.lora_plan_create(16, S)
    try:
        y = torch.empty((16, 64), dtype=torch.float16, device="cuda")
        with pytest.raises(lora.LoraError) as ei:
            lora.lora_apply_routed(pa.h, plan, dev(xa), dev(Wa), y)
        assert ei.value.status == lora.LORA_EINVAL
        lora.lora_plan_route(plan, pa.h, dev(idx), 0)
        lora.lora_apply_routed(pa.h, plan, dev(xa), dev(Wa), y)  # no-op
        torch.cuda.synchronize()
    finally:
        lora.lora_plan_destroy(plan)
        pa.close()
