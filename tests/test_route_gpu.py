"""Routing on the GPU (lora_route through the C ABI) vs the oracle: every array
bit-exact -- counts, offsets, the stable permutation and the bucket records."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import Pool, dev
from rank_adapter_gemm_token_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _pool_with_slots(S, active, max_T, policy=0, theta=16):
    p = Pool(64, 64, 8, S, max_T, "f16", policy=policy, theta=theta)
    g = torch.Generator().manual_seed(S)
    for s in np.flatnonzero(active):
        A = torch.randn((4, 64), generator=g).to(torch.float16)
        B = torch.randn((64, 4), generator=g).to(torch.float16)
        p.register(int(s), A, B, 4, 8.0)
    return p


def _compare(p, idx_np, active, policy=0, theta=16):
    idx = dev(torch.from_numpy(np.asarray(idx_np, np.int32)))
    got = p.route(idx)
    ref = oracle.route(idx_np, p.S, active, policy, theta)
    assert got["counts"].tolist() == ref["counts"].tolist()
    assert got["offsets"].tolist() == ref["offsets"].tolist()
    assert got["perm"].tolist() == ref["perm"].tolist()
    assert got["n_seg"] == ref["n_seg"]
    assert got["segs"].tolist() == ref["segs"].tolist()


def _edge(T, S, rng):
    return {
        "all_same": np.full(T, S // 2),
        "all_base_only": np.full(T, -1),
        "sorted": np.sort(rng.integers(-1, S, size=T)),
        "reversed": np.sort(rng.integers(-1, S, size=T))[::-1].copy(),
        "all_invalid": rng.integers(S, S + 50, size=T),
        "mixed_invalid": rng.integers(-5, S + 5, size=T),
    }


@pytest.mark.parametrize("T", [1, 63, 64, 65, 1023, 1024, 1025, 3001, 4096])
def test_route_edge_cases(T):
    S = 12
    active = np.ones(S, np.int32)
    active[[3, 7]] = 0  # registered nowhere: tokens naming them are invalid
    p = _pool_with_slots(S, active, 4096)
    try:
        rng = np.random.default_rng(T)
        for name, idx in _edge(T, S, rng).items():
            _compare(p, idx, active)
    finally:
        p.close()


@pytest.mark.parametrize("policy,theta", [(0, 0), (0, 3), (0, 16), (0, 1000), (1, 16), (2, 16)])
def test_route_policies(policy, theta):
    S = 20
    active = np.ones(S, np.int32)
    p = _pool_with_slots(S, active, 512, policy, theta)
    try:
        rng = np.random.default_rng(99)
        idx = rng.choice(np.arange(-1, S), size=500, p=None)
        _compare(p, idx, active, policy, theta)
    finally:
        p.close()


def test_route_workload_indices():
    cases = [("tiny", wl.tiny().idx, 4), ("decode", wl.decode().idx, 6),
             ("prefill", wl.prefill().idx, 32), ("stack", wl.stack_idx(), 64)]
    cases += [("sweep%d" % T, wl.sweep(T).idx, 100) for T in wl.SWEEP_T]
    for name, idx, S in cases:
        active = np.ones(S, np.int32)
        p = _pool_with_slots(S, active, max(idx.numel(), 1))
        try:
            _compare(p, idx.numpy(), active)
        finally:
            p.close()


def test_route_max_slots():
    S = 1024
    rng = np.random.default_rng(5)
    active = (rng.random(S) < 0.5).astype(np.int32)
    p = _pool_with_slots(S, active, 4096)
    try:
        _compare(p, rng.integers(-1, S + 2, size=4096), active)
        _compare(p, rng.integers(-1, S + 2, size=777), active)
    finally:
        p.close()


def test_route_empty():
    p = _pool_with_slots(4, np.ones(4, np.int32), 16)
    try:
        got = p.route(torch.zeros(0, dtype=torch.int32, device="cuda"))
        assert got["counts"].tolist() == [0] * 6
        assert got["offsets"].tolist() == [0] * 7
        assert got["n_seg"] == 0
    finally:
        p.close()
