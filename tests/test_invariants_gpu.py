"""Properties the pages fix, checked on the GPU path (lora_apply via the C ABI):

  * base_only tokens get exactly the base output, as floats, whatever else is
    in the batch (xpshop.cn article 492, section 三: routing default base_only);
  * an adapter with B = 0 is a no-op;
  * a rank-8 adapter zero-padded in the pool equals the same adapter given as
    rank 64 with zero rows/columns and the same alpha/r ("LLM 多 LoRA 推理服务工程
    2026", routing layer, zero-pad paragraph: padding keeps results correct);
  * each token's row is invariant to batch order and to which other adapters
    share the batch -- no cross-tenant bleed ("Multi-LoRA 在线服务隔离", request
    identity section), and 32 distinct adapters in one batch have zero
    attribution errors (same page, release-gate section);
  * integer-valued inputs give results exactly equal to the oracle;
  * repeated calls are bitwise identical.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import Pool, assert_close, dev, reference
from rank_adapter_gemm_token_amd import lora
from rank_adapter_gemm_token_amd import workloads as wl

pytestmark = pytest.mark.gpu

FORCED = [lora.LORA_MODE_FUSED, lora.LORA_MODE_SEPARATE]
ALL = [lora.LORA_MODE_AUTO] + FORCED


def _decode_pool(policy, dtype="f16", T=64):
    w = wl.decode(T=T)
    lin = w.linears[0]
    if dtype != "f16":
        tdt = torch.bfloat16
        lin = wl.Linear(lin.name, lin.d_in, lin.d_out, lin.W.to(tdt),
                        [wl.Adapter(a.slot, a.tenant, a.rank, a.alpha, a.A.to(tdt), a.B.to(tdt))
                         for a in lin.adapters])
        w.x = {k: v.to(tdt) for k, v in w.x.items()}
    p = Pool(lin.d_in, lin.d_out, w.R, w.S, 256, dtype, policy, 16)
    p.register_all(lin.adapters)
    return p, w, lin


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("policy", ALL)
def test_base_only_rows_are_exactly_base(dtype, policy):
    p, w, lin = _decode_pool(policy, dtype)
    try:
        x, W, idx = dev(w.x[4096]), dev(lin.W), dev(w.idx)
        y_mixed = p.apply(x, W, idx)
        y_base = p.apply(x, W, torch.full_like(idx, -1))
        torch.cuda.synchronize()
        b = (w.idx == -1).numpy()
        assert b.any()
        assert torch.equal(y_mixed.cpu()[b], y_base.cpu()[b])
        # and the all-base_only call is the plain product x W^T
        ref, inv = reference(p, w.x[4096], lin.W, torch.full_like(w.idx, -1))
        assert_close(y_base.cpu(), ref, inv, dtype)
    finally:
        p.close()


@pytest.mark.parametrize("policy", ALL)
def test_zero_B_is_noop(policy):
    p, w, lin = _decode_pool(policy)
    try:
        a = lin.adapters[2]
        p.unregister(2)
        p.register(2, a.A, torch.zeros_like(a.B), a.rank, a.alpha)
        x, W = dev(w.x[4096]), dev(lin.W)
        idx = torch.full((64,), 2, dtype=torch.int32)
        y = p.apply(x, W, dev(idx))
        y_base = p.apply(x, W, dev(torch.full_like(idx, -1)))
        torch.cuda.synchronize()
        assert torch.equal(y.cpu(), y_base.cpu())
    finally:
        p.close()


@pytest.mark.parametrize("policy", ALL)
def test_zero_padding_is_exact(policy):
    # Same pool (R = 64): rank 8 alpha 16 vs rank 64 zero-extended alpha 128.
    rng = np.random.default_rng(7)
    d, T = 256, 40
    A = torch.from_numpy(rng.standard_normal((8, d)) / 16).to(torch.bfloat16)
    B = torch.from_numpy(rng.standard_normal((d, 8)) * 0.1).to(torch.bfloat16)
    A64 = torch.zeros((64, d), dtype=torch.bfloat16)
    A64[:8] = A
    B64 = torch.zeros((d, 64), dtype=torch.bfloat16)
    B64[:, :8] = B
    x = torch.from_numpy(rng.standard_normal((T, d))).to(torch.bfloat16)
    W = torch.from_numpy(rng.standard_normal((d, d)) / 16).to(torch.bfloat16)
    p = Pool(d, d, 64, 2, T, "bf16", policy, 16)
    try:
        p.register(0, A, B, 8, 16.0)
        p.register(1, A64, B64, 64, 128.0)
        y0 = p.apply(dev(x), dev(W), dev(torch.zeros(T, dtype=torch.int32)))
        y1 = p.apply(dev(x), dev(W), dev(torch.ones(T, dtype=torch.int32)))
        torch.cuda.synchronize()
        assert torch.equal(y0.cpu(), y1.cpu())
        ref, inv = reference(p, x, W, torch.zeros(T, dtype=torch.int32))
        assert_close(y0.cpu(), ref, inv, "bf16")
    finally:
        p.close()


@pytest.mark.parametrize("policy", ALL)
def test_batch_order_invariance(policy):
    p, w, lin = _decode_pool(policy)
    try:
        x, W, idx = w.x[4096], lin.W, w.idx
        perm = torch.from_numpy(np.random.default_rng(3).permutation(64))
        y = p.apply(dev(x), dev(W), dev(idx))
        yp = p.apply(dev(x[perm]), dev(W), dev(idx[perm]))
        torch.cuda.synchronize()
        assert torch.equal(yp.cpu(), y.cpu()[perm])
    finally:
        p.close()


@pytest.mark.parametrize("policy", FORCED)
def test_no_cross_tenant_bleed(policy):
    # Token t's row does not change when every other token switches adapter.
    p, w, lin = _decode_pool(policy)
    try:
        x, W = dev(w.x[4096]), dev(lin.W)
        base_idx = w.idx.clone()
        y0 = p.apply(x, W, dev(base_idx)).cpu()
        rng = np.random.default_rng(11)
        for trial in range(4):
            other = torch.from_numpy(rng.integers(-1, 6, size=64).astype(np.int32))
            keep = torch.from_numpy(rng.random(64) < 0.25)
            mixed = torch.where(keep, base_idx, other)
            y1 = p.apply(x, W, dev(mixed)).cpu()
            assert torch.equal(y1[keep], y0[keep])
    finally:
        p.close()


@pytest.mark.parametrize("policy", ALL)
def test_32_adapters_zero_attribution_errors(policy):
    rng = np.random.default_rng(32)
    d, S, r, T = 256, 32, 16, 96
    ads = [wl.Adapter(s, s, r, 32.0,
                      torch.from_numpy(rng.standard_normal((r, d)) / 16).to(torch.float16),
                      torch.from_numpy(rng.standard_normal((d, r)) * 0.1).to(torch.float16))
           for s in range(S)]
    x = torch.from_numpy(rng.standard_normal((T, d))).to(torch.float16)
    W = torch.from_numpy(rng.standard_normal((d, d)) / 16).to(torch.float16)
    idx = torch.from_numpy(np.concatenate([np.arange(S), rng.integers(0, S, size=T - S)]).astype(np.int32))
    p = Pool(d, d, r, S, T, "f16", policy, 2)
    try:
        p.register_all(ads)
        y = p.apply(dev(x), dev(W), dev(idx)).cpu()
        torch.cuda.synchronize()
        ref, inv = reference(p, x, W, idx)
        assert_close(y, ref, inv, "f16")
        # Attribution: each row is nearest to its own adapter's output.
        g = oracle.to_f64(y)
        errs = np.zeros((T, S))
        for s in range(S):
            ref_s, _ = reference(p, x, W, torch.full_like(idx, s))
            errs[:, s] = np.abs(g - ref_s).max(axis=1)
        assert np.array_equal(errs.argmin(axis=1), idx.numpy())
    finally:
        p.close()


@pytest.mark.parametrize("dtype,limit", [("f16", 2048), ("bf16", 256)])
@pytest.mark.parametrize("policy", ALL)
def test_integer_inputs_exact(dtype, limit, policy):
    # Small-integer x, W, A, B and power-of-two scales keep every partial sum an
    # integer within the dtype's exact range, so any correct accumulation order
    # and either fused or separate path must equal the oracle exactly.
    rng = np.random.default_rng(5)
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    T, d_in, d_out, S, R = 70, 128, 192, 6, 16
    x = rng.integers(-2, 3, size=(T, d_in))
    W = (rng.random((d_out, d_in)) < 0.2) * rng.integers(-1, 2, size=(d_out, d_in))
    ads = []
    for s in range(S):
        rk = int(rng.choice([1, 2, 4, 8, 16]))
        A = (rng.random((rk, d_in)) < 0.1) * rng.integers(-1, 2, size=(rk, d_in))
        B = (rng.random((d_out, rk)) < 0.3) * rng.integers(-1, 2, size=(d_out, rk))
        alpha = float(rk * int(rng.integers(1, 3)))  # s in {1, 2}: integers stay integers
        ads.append(wl.Adapter(s, s, rk, alpha, torch.from_numpy(A).to(tdt), torch.from_numpy(B).to(tdt)))
    idx = torch.from_numpy(rng.integers(-1, S, size=T).astype(np.int32))
    xt, Wt = torch.from_numpy(x).to(tdt), torch.from_numpy(W).to(tdt)
    p = Pool(d_in, d_out, R, S, T, dtype, policy, 8)
    try:
        p.register_all(ads)
        y = p.apply(dev(xt), dev(Wt), dev(idx)).cpu()
        ref, inv = reference(p, xt, Wt, idx)
        assert not inv.any()
        assert np.abs(ref).max() <= limit
        assert np.array_equal(oracle.to_f64(y), ref)
    finally:
        p.close()


def test_repeat_calls_bitwise_identical():
    p, w, lin = _decode_pool(lora.LORA_MODE_AUTO)
    try:
        x, W, idx = dev(w.x[4096]), dev(lin.W), dev(w.idx)
        first = p.apply(x, W, idx).cpu()
        for _ in range(20):
            assert torch.equal(p.apply(x, W, idx).cpu(), first)
    finally:
        p.close()
