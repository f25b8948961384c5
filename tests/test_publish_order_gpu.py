"""A slot that is registered (or whose load is committed) while applies run on
another stream: every apply sees the slot either absent in all of its kernels
or present in all of them.  Each output row of a token naming the slot is then
either all NaN (the slot was not registered yet: an explicit error, never a
fallback -- "Multi-LoRA 在线服务隔离", request identity section) or the
adapter's correct row; and since the slot entry is published after the
applies enqueued before the register and before those enqueued after it
("xpshop.cn article 492", section 三: validate, then attach to the handle
table), the outputs of one stream switch from NaN to correct once, never
back."""
import threading
import time

import numpy as np
import pytest
import torch

from gpu_helpers import Pool, TOL, dev, reference, row_errors
from rank_adapter_gemm_token_amd import lora

pytestmark = pytest.mark.gpu

S, R = 4, 16
# (D, T): a decode call on 1024 x 1024, and 300 tokens on 192 x 192, which
# route inside the shrink launch (every workgroup reading the slot table).
SHAPES = [(1024, 64), (192, 300)]


def _setup(seed, D=1024, T=64):
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(rng.standard_normal((T, D))).to(torch.float16)
    W = torch.from_numpy(rng.standard_normal((D, D)) / np.sqrt(D)).to(torch.float16)
    ads = [(torch.from_numpy(rng.standard_normal((R, D)) / np.sqrt(D)).to(torch.float16),
            torch.from_numpy(rng.standard_normal((D, R)) * 0.1).to(torch.float16)) for _ in range(S)]
    idx = torch.from_numpy(rng.integers(-1, S, size=T).astype(np.int32))
    idx[::3] = 2  # the slot registered during the run
    return x, W, ads, idx


def _check_outputs(p, x, W, idx, ys):
    """Each output: slot-2 rows all NaN (not yet registered) or correct; the
    switch from NaN to correct happens once."""
    T = idx.numel()
    ref, _ = reference(p, x, W, idx)  # slot 2 registered in p.adapters
    two = (idx == 2).numpy()
    other_inv = np.zeros(T, bool)
    seen_active = False
    n_nan = 0
    for y in ys:
        g = y.cpu()
        nan_rows = torch.isnan(g.float()).all(dim=1).numpy()
        if nan_rows[two].all():
            assert not seen_active, "an apply after the slot turned active saw it absent"
            n_nan += 1
            inv = two
        else:
            seen_active = True
            inv = other_inv
        err = row_errors(g, ref, inv)
        assert err.max() <= TOL["f16"], "row error %.3e" % err.max()
    return n_nan


@pytest.mark.parametrize("D,T", SHAPES)
@pytest.mark.parametrize("seed", [0, 1])
def test_register_during_applies(seed, D, T):
    x, W, ads, idx = _setup(seed, D, T)
    p = Pool(D, D, R, S, T, "f16")
    try:
        for s in (0, 1, 3):
            p.register(s, ads[s][0], ads[s][1], R, 2.0 * R)
        lora.lora_set_tenant_quota(p.h, 2, 1 << 40)
        xd, Wd, idd = dev(x), dev(W), dev(idx)
        A2, B2 = dev(ads[2][0]), dev(ads[2][1])
        sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
        N = 300
        ys = [torch.empty((T, D), dtype=torch.float16, device="cuda") for _ in range(N)]
        torch.cuda.synchronize()
        go, started = threading.Event(), threading.Event()

        def applier():
            for i in range(N):
                lora.lora_apply(p.h, xd, Wd, idd, T, ys[i], sa.cuda_stream)
                if i == 40:
                    # Let the register take the pool mutex while applies are
                    # still in flight, and enqueue the rest after it.
                    go.set()
                    started.wait()
                    time.sleep(0.005)

        def registrar():
            go.wait()
            started.set()
            lora.lora_register(p.h, 2, 2, A2, B2, R, 2.0 * R, sb.cuda_stream)

        th = [threading.Thread(target=applier), threading.Thread(target=registrar)]
        for t in th:
            t.start()
        for t in th:
            t.join()
        torch.cuda.synchronize()
        p.adapters[2] = (ads[2][0], ads[2][1], R, 2.0 * R)
        n_nan = _check_outputs(p, x, W, idx, ys)
        assert 41 <= n_nan < N
    finally:
        p.close()


@pytest.mark.parametrize("D,T", SHAPES)
def test_loader_commit_during_applies(D, T):
    x, W, ads, idx = _setup(5, D, T)
    p = Pool(D, D, R, S, T, "f16")
    ld = lora.lora_loader_create(R * 2 * D * 2)
    try:
        for s in (0, 1, 3):
            p.register(s, ads[s][0], ads[s][1], R, 2.0 * R)
        lora.lora_set_tenant_quota(p.h, 2, 1 << 40)
        xd, Wd, idd = dev(x), dev(W), dev(idx)
        sa = torch.cuda.Stream()
        N = 300
        ys = [torch.empty((T, D), dtype=torch.float16, device="cuda") for _ in range(N)]
        torch.cuda.synchronize()
        go = threading.Event()

        def applier():
            for i in range(N):
                lora.lora_apply(p.h, xd, Wd, idd, T, ys[i], sa.cuda_stream)
                if i == 40:
                    go.set()

        def loader():
            go.wait()
            t = lora.lora_load_async(ld, p.h, 2, 2, ads[2][0].contiguous(), ads[2][1].contiguous(), R, 2.0 * R)
            while not lora.lora_load_poll(ld, t):  # commit by polling (never blocks on the applies)
                pass

        th = [threading.Thread(target=applier), threading.Thread(target=loader)]
        for t in th:
            t.start()
        for t in th:
            t.join()
        torch.cuda.synchronize()
        p.adapters[2] = (ads[2][0], ads[2][1], R, 2.0 * R)
        n_nan = _check_outputs(p, x, W, idx, ys)
        assert n_nan >= 41
    finally:
        lora.lora_loader_destroy(ld)
        p.close()
