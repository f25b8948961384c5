"""lora_apply_noalloc (the entry point for callers that cannot allocate: its
workspace is the library's static per-device array) against lora_apply, the
entry point it is a variant of: the same kernels, so the outputs must agree
bit for bit.  Two calls in a row on one stream, the second smaller, with no
synchronization between them (the array keeps the first call's contents);
every base-GEMM path; the size limit; and the oracle on one case."""
import numpy as np
import pytest
import torch

from gpu_helpers import Pool, assert_close, dev, reference
from rank_adapter_gemm_token_amd import lora
from rank_adapter_gemm_token_amd import workloads as wl

pytestmark = pytest.mark.gpu

TDT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def _case(dtype, T, d_in, d_out, S, R, seed):
    rng = np.random.default_rng(seed)
    tdt = TDT[dtype]
    x = torch.from_numpy(rng.standard_normal((T, d_in))).to(tdt)
    W = torch.from_numpy(rng.standard_normal((d_out, d_in)) / np.sqrt(d_in)).to(tdt)
    ads = []
    for s in range(S):
        r = int(rng.integers(1, R + 1))
        ads.append(wl.Adapter(s, s, r, float(2 * r),
                              torch.from_numpy(rng.standard_normal((r, d_in)) / np.sqrt(d_in)).to(tdt),
                              torch.from_numpy(rng.standard_normal((d_out, r)) * 0.1).to(tdt)))
    idx = rng.integers(-1, S, size=T)
    idx[rng.random(T) < 0.05] = S + 1  # invalid: NaN rows
    return x, W, ads, torch.from_numpy(idx.astype(np.int32))


def _bits(y):
    return y.cpu().view(torch.int16) if y.element_size() == 2 else y.cpu().view(torch.int32)


# (dtype, d_in, d_out, S, R, first T, second T): decode, split (WC 4 then 2),
# the unsplit 256-row tiles then the split path, off-grid tiles then decode,
# fp32; the routing inside the shrink launch ahead of split tiles and ahead of
# off-grid tiles.
CASES = [("f16", 4096, 1024, 6, 16, 64, 16), ("bf16", 1024, 512, 9, 32, 300, 100),
         ("bf16", 256, 256, 12, 64, 2048, 2000), ("f16", 128, 192, 6, 16, 70, 33),
         ("f32", 256, 256, 4, 8, 16, 5), ("f16", 4096, 2048, 9, 16, 300, 80),
         ("bf16", 192, 128, 40, 24, 513, 100)]


@pytest.mark.parametrize("dtype,d_in,d_out,S,R,T1,T2", CASES)
def test_noalloc_matches_apply(dtype, d_in, d_out, S, R, T1, T2):
    x, W, ads, idx = _case(dtype, T1, d_in, d_out, S, R, seed=T1 + d_out)
    p = Pool(d_in, d_out, R, S, T1, dtype, lora.LORA_MODE_AUTO, 0)
    try:
        p.register_all(ads)
        xd, Wd, idd = dev(x), dev(W), dev(idx)
        st = torch.cuda.current_stream()
        y1 = torch.full((T1, d_out), 7.0, dtype=TDT[dtype], device="cuda")
        y2 = torch.full((T2, d_out), 7.0, dtype=TDT[dtype], device="cuda")
        # Two calls in a row, the second on the first T2 tokens.
        lora.lora_apply_noalloc(p.h, xd, Wd, idd, T1, y1, st.cuda_stream)
        lora.lora_apply_noalloc(p.h, xd[:T2].contiguous(), Wd, idd[:T2].contiguous(), T2, y2, st.cuda_stream)
        r1 = p.apply(xd, Wd, idd)
        r2 = p.apply(xd[:T2].contiguous(), Wd, idd[:T2].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(_bits(y1), _bits(r1))
        assert torch.equal(_bits(y2), _bits(r2))
        # The error counter saw both noalloc calls and both lora_apply calls.
        n_inv = int((idx == S + 1).sum()) + int((idx[:T2] == S + 1).sum())
        assert p.poll_errors() == 2 * n_inv
    finally:
        p.close()


def test_noalloc_against_oracle_separate_policy():
    x, W, ads, idx = _case("f16", 40, 512, 256, 5, 16, seed=3)
    p = Pool(512, 256, 16, 5, 40, "f16", lora.LORA_MODE_SEPARATE, 16)
    try:
        p.register_all(ads)
        y = torch.empty((40, 256), dtype=torch.float16, device="cuda")
        lora.lora_apply_noalloc(p.h, dev(x), dev(W), dev(idx), 40, y)
        torch.cuda.synchronize()
        ref, inv = reference(p, x, W, idx)
        assert_close(y.cpu(), ref, inv, "f16")
    finally:
        p.close()


def test_noalloc_refuses_calls_beyond_the_scratch():
    # 512 tokens through an 8192 -> 11008 projection take 2 k splits of 344
    # tiles: 43 MiB of fp32 partial sums, beyond the 32 MiB array.  Refused
    # before anything runs.
    d_in, d_out, T = 8192, 11008, 512
    p = Pool(d_in, d_out, 16, 2, T, "bf16")
    try:
        x = torch.zeros((T, d_in), dtype=torch.bfloat16, device="cuda")
        W = torch.zeros((d_out, d_in), dtype=torch.bfloat16, device="cuda")
        idx = torch.full((T,), -1, dtype=torch.int32, device="cuda")
        y = torch.full((T, d_out), 3.0, dtype=torch.bfloat16, device="cuda")
        with pytest.raises(lora.LoraError) as ei:
            lora.lora_apply_noalloc(p.h, x, W, idx, T, y)
        assert ei.value.status == lora.LORA_ESCRATCH
        torch.cuda.synchronize()
        assert bool((y == 3.0).all())
        # 64 tokens of the same projection fit.
        lora.lora_apply_noalloc(p.h, x[:64].contiguous(), W, idx[:64].contiguous(), 64, y[:64])
        torch.cuda.synchronize()
        assert bool((y[:64] == 0).all())
    finally:
        p.close()
