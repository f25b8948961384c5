"""The exact properties the pages fix, on every base-GEMM kernel of lora_apply.

Each shape below is chosen so that the library takes one kernel (the variant
depends on (T, d_in, d_out, dtype) only):

  decode64    k_decode_gemm, 4 token blocks, + k_decode_epilogue (T <= 64)
  decode5     the same with 1 token block
  decodeS70   the same, 70 slots over 4 column groups (second shrink pass)
  decode_col  the same, 8 column groups x 16 k splits (narrow output)
  split4      k_gemm_lds<64, split> (65 .. 2047 tokens), 4 tiles x 4 k
              splits summed by the last split of each tile, a 64-row x
              group past T; the shrink in the same launch, on workgroups
              after the tiles' (the grid leaves CUs idle)
  split2_rows2  the same, two 256-row tiles, 2 k splits
  split_xcd   the same, 3 tiles x 4 splits (a grid 8 does not divide: a
              tile's splits run on different XCDs)
  split_tail1 128 tiles x 1 split + 128 shrink workgroups: each tile waits
              for the shrink before its tail expand
  split_tail2 96 tiles x 2 splits + 64 shrink workgroups, no LoRA
              workgroup: the last split of a tile waits before the expand
  split_r64   4 tiles x (6 splits + LoRA workgroup) + 228 shrink
              workgroups, ranks up to 64 (shrink units of 3-4 rank blocks)
              and two k parts of h
  split_lora_nofuse  56 tiles x (3 splits + LoRA workgroup) = 224
              workgroups: too few idle CUs, the shrink in a launch of its own
  split_nofuse  384 tiles x 1 split (more than one round of the CUs): the
              shrink in a launch of its own (grouped tiles, >= 1024 tokens)
  big         k_gemm_lds<256> (>= 2048 tokens, 256-row tiles)
  tiled       k_gemm_tiled (shapes off the 128 grid)

Properties (each exact, compared as values; NaN rows compare equal):
  * base_only rows equal the rows of an all-base_only call ("xpshop.cn
    article 492", section 三: routing default base_only, the base is shared);
  * permuting the batch permutes the rows ("Multi-LoRA 在线服务隔离", request
    identity section: per-request index mapping in a mixed batch);
  * a token's row does not change when every other token changes adapter,
    under a forced mode (same section: no cross-tenant bleed; release-gate
    section: zero attribution errors);
  * an adapter whose B is zero is a no-op ("LLM 多 LoRA 推理服务工程 2026",
    four-layer runtime, execution-unit paragraph: the LoRA product is a
    residual added to the base);
  * repeated calls are bitwise identical;
  * small-integer inputs give exactly the oracle's values (every partial sum
    is an integer the accumulator and the pool dtype hold exactly, so any
    correct summation order, fused or separate, must agree).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import Pool, assert_close, dev, reference
from rank_adapter_gemm_token_amd import lora
from rank_adapter_gemm_token_amd import workloads as wl

pytestmark = pytest.mark.gpu

# name -> (T, d_in, d_out, S, R)
SHAPES = {
    "decode64": (64, 4096, 1024, 6, 16),
    "decode5": (5, 2048, 256, 4, 16),
    "decodeS70": (64, 512, 256, 70, 16),
    "decode_col": (64, 4096, 512, 6, 16),   # 16 k splits over 8 column groups
    "split4": (130, 1024, 256, 9, 16),      # 4 tiles x 4 splits
    "split2_rows2": (300, 1024, 512, 9, 32),  # 16 tiles (2 rows) x 2 splits
    "split_xcd": (70, 1024, 192, 6, 16),     # 3 tiles x 4 splits: splits on different XCDs
    "split_tail1": (300, 1024, 4096, 9, 16),     # 128 tiles x 1 split + 128 shrink workgroups
    "split_tail2": (700, 2048, 2048, 9, 16),     # 96 tiles x 2 splits + 64 shrink workgroups
    "split_r64": (130, 4096, 256, 9, 64),        # in-launch shrink at ranks up to 64, 2 k parts
    "split_lora_nofuse": (1600, 2048, 512, 9, 16),  # 56 tiles x (3 + 1), separate shrink
    "split_nofuse": (1300, 256, 4096, 6, 16),    # 384 tiles: separate (grouped) shrink
    "split_route_shrink": (300, 4096, 2048, 9, 16),  # 64 tiles x (3 + 1), routing in the shrink launch
    "tiled_route_shrink": (513, 192, 128, 40, 24),   # unsplit tiles, routing in the shrink launch
    "big": (2048, 256, 256, 12, 64),
    "tiled": (70, 128, 192, 6, 16),
}
TDT = {"f16": torch.float16, "bf16": torch.bfloat16}
POLICIES = [lora.LORA_MODE_AUTO, lora.LORA_MODE_FUSED, lora.LORA_MODE_SEPARATE]
FORCED = [lora.LORA_MODE_FUSED, lora.LORA_MODE_SEPARATE]


def _same(a, b):
    """Equal as values, NaN == NaN (invalid rows are all NaN)."""
    a, b = a.float(), b.float()
    return bool(((a == b) | (torch.isnan(a) & torch.isnan(b))).all())


def _normal_case(shape, dtype, seed):
    T, d_in, d_out, S, R = SHAPES[shape]
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
    # Every slot, base_only and a few invalid indices.
    idx = rng.integers(-1, S, size=T)
    idx[rng.random(T) < 0.03] = S + 3
    return x, W, ads, torch.from_numpy(idx.astype(np.int32))


def _pool(shape, dtype, policy, ads, theta=16):
    T, d_in, d_out, S, R = SHAPES[shape]
    p = Pool(d_in, d_out, R, S, T, dtype, policy, theta)
    p.register_all(ads)
    return p


@pytest.mark.parametrize("shape", list(SHAPES))
@pytest.mark.parametrize("policy", POLICIES)
def test_base_only_rows_exact(shape, policy):
    x, W, ads, idx = _normal_case(shape, "bf16", 1)
    p = _pool(shape, "bf16", policy, ads)
    try:
        y_mixed = p.apply(dev(x), dev(W), dev(idx)).cpu()
        y_base = p.apply(dev(x), dev(W), dev(torch.full_like(idx, -1))).cpu()
        b = (idx == -1).numpy()
        assert b.any()
        assert _same(y_mixed[b], y_base[b])
        ref, inv = reference(p, x, W, torch.full_like(idx, -1))
        assert_close(y_base, ref, inv, "bf16")
    finally:
        p.close()


@pytest.mark.parametrize("shape", list(SHAPES))
@pytest.mark.parametrize("policy", POLICIES)
def test_batch_order_invariance(shape, policy):
    x, W, ads, idx = _normal_case(shape, "f16", 2)
    p = _pool(shape, "f16", policy, ads)
    try:
        perm = torch.from_numpy(np.random.default_rng(3).permutation(idx.numel()))
        y = p.apply(dev(x), dev(W), dev(idx)).cpu()
        yp = p.apply(dev(x[perm]), dev(W), dev(idx[perm])).cpu()
        assert _same(yp, y[perm])
        ref, inv = reference(p, x, W, idx)
        assert_close(y, ref, inv, "f16")
    finally:
        p.close()


@pytest.mark.parametrize("shape", list(SHAPES))
@pytest.mark.parametrize("policy", FORCED)
def test_no_cross_tenant_bleed(shape, policy):
    T, d_in, d_out, S, R = SHAPES[shape]
    x, W, ads, idx = _normal_case(shape, "bf16", 4)
    p = _pool(shape, "bf16", policy, ads)
    try:
        y0 = p.apply(dev(x), dev(W), dev(idx)).cpu()
        rng = np.random.default_rng(11)
        for trial in range(3):
            other = torch.from_numpy(rng.integers(-1, S + 1, size=T).astype(np.int32))
            keep = torch.from_numpy(rng.random(T) < 0.25)
            mixed = torch.where(keep, idx, other)
            y1 = p.apply(dev(x), dev(W), dev(mixed)).cpu()
            assert _same(y1[keep], y0[keep])
    finally:
        p.close()


@pytest.mark.parametrize("shape", list(SHAPES))
@pytest.mark.parametrize("policy", POLICIES)
def test_zero_B_is_noop(shape, policy):
    x, W, ads, idx = _normal_case(shape, "f16", 5)
    a = ads[1]
    ads[1] = wl.Adapter(a.slot, a.tenant, a.rank, a.alpha, a.A, torch.zeros_like(a.B))
    p = _pool(shape, "f16", policy, ads)
    try:
        one = torch.full_like(idx, 1)
        y = p.apply(dev(x), dev(W), dev(one)).cpu()
        y_base = p.apply(dev(x), dev(W), dev(torch.full_like(idx, -1))).cpu()
        assert _same(y, y_base)
    finally:
        p.close()


@pytest.mark.parametrize("shape", list(SHAPES))
def test_repeat_calls_bitwise(shape):
    x, W, ads, idx = _normal_case(shape, "bf16", 6)
    p = _pool(shape, "bf16", lora.LORA_MODE_AUTO, ads, theta=0)
    try:
        xd, Wd, idd = dev(x), dev(W), dev(idx)
        first = p.apply(xd, Wd, idd).cpu().view(torch.int16)
        for _ in range(5):
            assert torch.equal(p.apply(xd, Wd, idd).cpu().view(torch.int16), first)
    finally:
        p.close()


def _integer_case(shape, dtype, seed):
    """x in {-1, 0, 1} (fp16: {-2 .. 2}), sparse +-1 W, A and B, true ranks
    of 1 .. 16 with alpha / rank in {1, 2}: every product and partial sum is
    a small integer."""
    T, d_in, d_out, S, R = SHAPES[shape]
    rng = np.random.default_rng(seed)
    tdt = TDT[dtype]
    amp = 2 if dtype == "f16" else 1
    dens = min(0.25, 24.0 / d_in)
    x = rng.integers(-amp, amp + 1, size=(T, d_in))
    W = (rng.random((d_out, d_in)) < dens) * rng.integers(-1, 2, size=(d_out, d_in))
    ads = []
    for s in range(S):
        rk = int(rng.choice([r for r in (1, 2, 4, 8, 16) if r <= R]))
        A = (rng.random((rk, d_in)) < dens) * rng.integers(-1, 2, size=(rk, d_in))
        B = (rng.random((d_out, rk)) < 0.15) * rng.integers(-1, 2, size=(d_out, rk))
        alpha = float(rk * int(rng.integers(1, 3)))
        ads.append(wl.Adapter(s, s, rk, alpha, torch.from_numpy(A).to(tdt), torch.from_numpy(B).to(tdt)))
    idx = torch.from_numpy(rng.integers(-1, S, size=T).astype(np.int32))
    return torch.from_numpy(x).to(tdt), torch.from_numpy(W).to(tdt), ads, idx


@pytest.mark.parametrize("shape", list(SHAPES))
@pytest.mark.parametrize("dtype,limit", [("f16", 2048), ("bf16", 256)])
@pytest.mark.parametrize("policy", POLICIES)
def test_integer_inputs_exact(shape, dtype, limit, policy):
    x, W, ads, idx = _integer_case(shape, dtype, 7)
    # The scaled h (an MFMA operand in the pool dtype on the tiled paths) and
    # every output stay within the dtype's exact-integer range.
    xs = x.double().numpy()
    for a in ads:
        h = (a.alpha / a.rank) * (xs @ a.A.double().numpy().T)
        assert np.abs(h).max() <= limit
    p = _pool(shape, dtype, policy, ads, theta=8)
    try:
        y = p.apply(dev(x), dev(W), dev(idx)).cpu()
        ref, inv = reference(p, x, W, idx)
        assert not inv.any()
        assert np.abs(ref).max() <= limit
        assert np.array_equal(oracle.to_f64(y), ref)
    finally:
        p.close()


# Decode calls keep partial sums and h in the pool's workspace between the
# GEMM and its epilogue launch; split calls with the shrink in the GEMM
# launch count its units on counters that every call leaves at 0.
DECODE_SHAPES = ["decode64", "decode5", "decodeS70", "split4", "split_tail1", "split_tail2",
                 "split_route_shrink", "tiled_route_shrink"]


@pytest.mark.parametrize("shape", DECODE_SHAPES)
def test_decode_alternating_inputs(shape):
    # Two different batches, one after the other many times on one stream: an
    # epilogue that read another call's (stale) partial sums or h would break
    # the equality with each batch's own first result.
    x0, W, ads, idx0 = _normal_case(shape, "f16", 10)
    x1, _, _, idx1 = _normal_case(shape, "f16", 11)
    p = _pool(shape, "f16", lora.LORA_MODE_AUTO, ads, theta=0)
    try:
        Wd = dev(W)
        ins = [(dev(x0), dev(idx0)), (dev(x1), dev(idx1))]
        ref = [p.apply(x, Wd, i).cpu().view(torch.int16) for x, i in ins]
        outs = []
        for k in range(40):
            x, i = ins[k % 2]
            outs.append(p.apply(x, Wd, i))
        torch.cuda.synchronize()
        for k, y in enumerate(outs):
            assert torch.equal(y.cpu().view(torch.int16), ref[k % 2]), k
        r0, inv0 = reference(p, x0, W, idx0)
        assert_close(outs[0].cpu(), r0, inv0, "f16")
    finally:
        p.close()


def test_split_calls_of_every_plan_on_one_pool():
    # One pool, calls whose plans differ (shrink on extra workgroups, on the
    # tile workgroups with LoRA workgroups or tail consumers, or in its own
    # launch), in a repeating order on one stream: each call's output equals
    # its own first result bitwise (a counter left non-zero by one plan would
    # let the next call's consumers read h before it is complete) and the
    # oracle within tolerance.
    d_in, d_out, S, R = 256, 4096, 6, 16
    rng = np.random.default_rng(21)
    Ts = [130, 1024, 1300, 300, 1024, 70]
    p = Pool(d_in, d_out, R, S, max(Ts), "bf16", lora.LORA_MODE_AUTO, 0)
    try:
        ads = []
        for s in range(S):
            r = int(rng.integers(1, R + 1))
            ads.append(wl.Adapter(s, s, r, float(2 * r),
                                  torch.from_numpy(rng.standard_normal((r, d_in)) / np.sqrt(d_in)).bfloat16(),
                                  torch.from_numpy(rng.standard_normal((d_out, r)) * 0.1).bfloat16()))
        p.register_all(ads)
        W = torch.from_numpy(rng.standard_normal((d_out, d_in)) / np.sqrt(d_in)).bfloat16()
        Wd = dev(W)
        cases = []
        for T in Ts:
            x = torch.from_numpy(rng.standard_normal((T, d_in))).bfloat16()
            idx = torch.from_numpy(rng.integers(-1, S, size=T).astype(np.int32))
            cases.append((x, idx, dev(x), dev(idx)))
        first = [p.apply(xd, Wd, idd).cpu().view(torch.int16) for _, _, xd, idd in cases]
        outs = []
        for k in range(3 * len(cases)):
            _, _, xd, idd = cases[k % len(cases)]
            outs.append(p.apply(xd, Wd, idd))
        torch.cuda.synchronize()
        for k, y in enumerate(outs):
            assert torch.equal(y.cpu().view(torch.int16), first[k % len(cases)]), k
        for (x, idx, _, _), y in zip(cases, first):
            ref, inv = reference(p, x, W, idx)
            assert_close(y.view(torch.bfloat16), ref, inv, "bf16")
    finally:
        p.close()


@pytest.mark.parametrize("shape", ["split4", "split_tail1", "split_tail2", "split_r64"])
def test_in_launch_shrink_fallback_same_bits(shape):
    # Shapes whose GEMM runs the shrink on idle CUs in the same launch.  With
    # the poll bound at 0 every h consumer computes all of h itself instead of
    # waiting for the shrink workgroups: the output must be the same bits, and
    # the calls after it (default bound) must still agree (the counters end
    # each call at 0 whichever way h was obtained).
    x, W, ads, idx = _normal_case(shape, "bf16", 12)
    p = _pool(shape, "bf16", lora.LORA_MODE_AUTO, ads, theta=0)
    try:
        xd, Wd, idd = dev(x), dev(W), dev(idx)
        base = p.apply(xd, Wd, idd).cpu().view(torch.int16)
        lora.lora_set_shrink_wait_polls(p.h, 0)
        for _ in range(2):
            assert torch.equal(p.apply(xd, Wd, idd).cpu().view(torch.int16), base)
        lora.lora_set_shrink_wait_polls(p.h, -1)
        for _ in range(2):
            assert torch.equal(p.apply(xd, Wd, idd).cpu().view(torch.int16), base)
        ref, inv = reference(p, x, W, idx)
        assert_close(base.view(torch.bfloat16), ref, inv, "bf16")
    finally:
        p.close()
