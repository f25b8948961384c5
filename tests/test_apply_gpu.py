"""lora_apply on the GPU (through the C ABI) vs the CPU fp64 oracle, on the five
workloads and on small ragged shapes, under every fused/separate policy."""
import numpy as np
import pytest
import torch

from gpu_helpers import Pool, assert_close, dev, reference, sample_rows
from rank_adapter_gemm_token_amd import lora
from rank_adapter_gemm_token_amd import workloads as wl

pytestmark = pytest.mark.gpu

POLICIES = [(lora.LORA_MODE_AUTO, 16), (lora.LORA_MODE_FUSED, 16), (lora.LORA_MODE_SEPARATE, 16),
            (lora.LORA_MODE_AUTO, 0), (lora.LORA_MODE_AUTO, 3)]


def _run_full(w, lin, policy, theta, rows=None):
    p = Pool(lin.d_in, lin.d_out, w.R, w.S, w.T, w.dtype, policy, theta)
    try:
        p.register_all(lin.adapters)
        x, W, idx = dev(w.x[lin.d_in]), dev(lin.W), dev(w.idx)
        y = p.apply(x, W, idx)
        torch.cuda.synchronize()
        y_ref, inv = reference(p, w.x[lin.d_in], lin.W, w.idx, rows=rows)
        got = y.cpu() if rows is None else y.cpu()[torch.as_tensor(rows)]
        return assert_close(got, y_ref, inv, w.dtype)
    finally:
        p.close()


@pytest.mark.parametrize("policy,theta", POLICIES)
def test_tiny_fp32_full(policy, theta):
    w = wl.tiny()
    _run_full(w, w.linears[0], policy, theta)


@pytest.mark.parametrize("policy,theta", POLICIES[:3])
def test_decode_fp16_full(policy, theta):
    w = wl.decode()
    _run_full(w, w.linears[0], policy, theta)


@pytest.mark.parametrize("T", wl.SWEEP_T)
def test_sweep_fp16_full(T):
    w = wl.sweep(T)
    _run_full(w, w.linears[0], lora.LORA_MODE_AUTO, 16)


@pytest.mark.parametrize("kind", ["col", "row"])
@pytest.mark.parametrize("policy,theta", POLICIES[:3])
def test_shard_fp16_full(kind, policy, theta):
    # One GPU's 4096x512 / 512x4096 share of the decode q_proj (the narrow
    # one runs 16 k splits to spread over the CUs).
    w = wl.shard(kind)
    _run_full(w, w.linears[0], policy, theta)


@pytest.mark.parametrize("proj", [0, 1])
def test_prefill_bf16_sampled(proj):
    w = wl.prefill()
    ends = [s * 512 for s in range(8)] + [s * 512 + 511 for s in range(8)]
    rows = sample_rows(w.T, 48, seed=proj, must=ends)
    _run_full(w, w.linears[proj], lora.LORA_MODE_AUTO, 16, rows=rows)


@pytest.mark.parametrize("layer,proj", [(0, p) for p in range(7)] + [(31, 6)])
def test_stack_bf16_sampled(layer, proj):
    idx = wl.stack_idx()
    lin = wl.stack_linear(layer, proj, "cuda")
    x = wl.stack_x(lin.d_in, device="cpu")
    w = wl.Workload("stack", "bf16", 256, 64, 16, idx, {lin.d_in: x}, [lin], 5)
    rows = sample_rows(256, 24, seed=layer * 7 + proj)
    _run_full(w, lin, lora.LORA_MODE_AUTO, 16, rows=rows)


def _small_case(dtype, T, d_in, d_out, S, R, seed):
    rng = np.random.default_rng(seed)
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    x = torch.from_numpy(rng.standard_normal((T, d_in))).to(tdt)
    W = torch.from_numpy(rng.standard_normal((d_out, d_in)) / np.sqrt(d_in)).to(tdt)
    ads = []
    for s in range(S):
        r = int(rng.integers(1, R + 1))
        ads.append(wl.Adapter(s, s, r, float(2 * r),
                              torch.from_numpy(rng.standard_normal((r, d_in)) / np.sqrt(d_in)).to(tdt),
                              torch.from_numpy(rng.standard_normal((d_out, r)) * 0.1).to(tdt)))
    idx = torch.from_numpy(rng.integers(-1, S + 2, size=T).astype(np.int32))  # incl. invalid
    return x, W, ads, idx


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
# Shapes reach every base-GEMM variant: split-K decode (T <= 64), the
# register-staged tiles (ragged d_in / d_out), the split-K 256-row tiles
# (T 65 .. 2047 with d_in, d_out multiples of 128; 4 and 2 splits here) and
# the unsplit 256 x 256 tiles (T >= 2048), each with a ragged last tile; the
# 2200- and 2300-token cases hold many adapter buckets in every 256-row tile;
# the 4100- and 4096-token cases have >= 256 16-row bucket tiles (one shrink
# k part) and long and short buckets.
# 96, 130 and 190 tokens take the split path with 64-row groups of the tile
# wholly past T (their loads and MFMAs skipped).
# Split tiles whose grid 8 does not divide (70 x 1024 -> 192: 3 tiles x 4
# splits and a LoRA workgroup each; 100 x 2048 -> 960) put a tile's
# contributors on different XCDs; 300 x 1024 -> 512 splits two rows of tiles;
# 70 x 256 -> 64 is one split plus the LoRA workgroup, 300 x 256 -> 4096 one
# split with the expand in the tile's own tail.
# Narrow decode outputs take extra k splits (48 x 2048 -> 256: 16 splits of
# 2 step pairs; 20 x 1024 -> 128: 16 splits of 1 pair).
# Decode calls also cover pools beyond the epilogue's small-pool B tile (S R
# > 1024) and beyond 64 slots (routing loads each token's slot entry; the GEMM
# takes slots past its column groups in a second pass).
@pytest.mark.parametrize("T,d_in,d_out,S,R", [(1, 64, 64, 1, 1), (37, 128, 192, 5, 8),
                                               (50, 256, 128, 20, 64), (64, 128, 64, 70, 16),
                                               (77, 192, 128, 9, 16), (300, 256, 320, 17, 64),
                                               (513, 64, 128, 40, 24), (200, 1024, 384, 7, 16),
                                               (1000, 512, 512, 11, 32), (2100, 256, 256, 3, 8),
                                               (2200, 256, 256, 40, 16), (2300, 512, 256, 60, 64),
                                               (4100, 256, 256, 7, 64), (4096, 128, 128, 30, 24),
                                               (96, 256, 256, 9, 16), (130, 256, 384, 12, 32),
                                               (190, 512, 256, 5, 64), (48, 2048, 256, 6, 16),
                                               (20, 1024, 128, 3, 32), (70, 1024, 192, 6, 16),
                                               (100, 2048, 960, 9, 32), (300, 1024, 512, 13, 16),
                                               (70, 256, 64, 5, 16), (300, 256, 4096, 7, 16)])
@pytest.mark.parametrize("policy", [0, 1, 2])
def test_small_ragged_full(dtype, T, d_in, d_out, S, R, policy):
    x, W, ads, idx = _small_case(dtype, T, d_in, d_out, S, R, seed=T * 31 + S)
    p = Pool(d_in, d_out, R, S, T, dtype, policy, 4)
    try:
        p.register_all(ads)
        y = p.apply(dev(x), dev(W), dev(idx))
        torch.cuda.synchronize()
        y_ref, inv = reference(p, x, W, idx)
        assert_close(y.cpu(), y_ref, inv, dtype)
        assert p.poll_errors() == int(inv.sum())
    finally:
        p.close()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("policy", [0, 1, 2])
def test_split_without_lora_workgroup_sampled(dtype, policy):
    # 520 x 2048 -> 2048: 64 tiles (two rows of 256-row tiles) x 2 k splits
    # and no LoRA workgroup (the grid would exceed one round of the CUs), so
    # the last split of a tile adds the fused expand itself.
    T, d_in, d_out, S, R = 520, 2048, 2048, 23, 32
    x, W, ads, idx = _small_case(dtype, T, d_in, d_out, S, R, seed=520)
    p = Pool(d_in, d_out, R, S, T, dtype, policy, 4)
    try:
        p.register_all(ads)
        y = p.apply(dev(x), dev(W), dev(idx))
        torch.cuda.synchronize()
        rows = sample_rows(T, 96, seed=policy, must=[0, 255, 256, 511, 512, 519])
        y_ref, inv = reference(p, x, W, idx, rows=rows)
        assert_close(y.cpu()[torch.as_tensor(rows)], y_ref, inv, dtype)
    finally:
        p.close()


def _max_case(dtype, T, d_in, d_out, S, R, used, seed):
    """S slots of which only `used` (spread over the whole range, up to slot
    S - 1) hold adapters; tokens name those, base_only and invalid slots."""
    rng = np.random.default_rng(seed)
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    x = torch.from_numpy(rng.standard_normal((T, d_in))).to(tdt)
    W = torch.from_numpy(rng.standard_normal((d_out, d_in)) / np.sqrt(d_in)).to(tdt)
    slots = sorted(set([S - 1, 0] + rng.choice(S, size=used - 2, replace=False).tolist()))
    ads = []
    for s in slots:
        r = int(rng.integers(1, R + 1))
        ads.append(wl.Adapter(s, s % 3, r, float(2 * r),
                              torch.from_numpy(rng.standard_normal((r, d_in)) / np.sqrt(d_in)).to(tdt),
                              torch.from_numpy(rng.standard_normal((d_out, r)) * 0.1).to(tdt)))
    choice = np.array(slots + [-1, S + 5, 1 if 1 not in slots else S])  # incl. base_only and invalid
    idx = torch.from_numpy(choice[rng.integers(0, len(choice), size=T)].astype(np.int32))
    return x, W, ads, idx


# The largest pool (LORA_MAX_SLOTS slots, LORA_MAX_RANK rank) on every path:
# decode (d_out = 128: two column groups take slots 0..1023 in turn), the split
# 256-row tiles (at 256 x 4096 -> 4096 routed inside the shrink launch, rows
# sampled) and the unsplit ones (a call of 4100 tokens, rows sampled).
@pytest.mark.parametrize("dtype,T,d_in,d_out", [("f16", 64, 256, 128), ("bf16", 700, 256, 256),
                                                ("f16", 256, 4096, 4096),
                                                ("bf16", 4100, 256, 256), ("f32", 33, 64, 64)])
def test_max_slots_and_rank(dtype, T, d_in, d_out):
    S, R = lora.LORA_MAX_SLOTS, lora.LORA_MAX_RANK
    x, W, ads, idx = _max_case(dtype, T, d_in, d_out, S, R, used=40, seed=T)
    p = Pool(d_in, d_out, R, S, T, dtype)
    try:
        p.register_all(ads)
        y = p.apply(dev(x), dev(W), dev(idx))
        torch.cuda.synchronize()
        big = T > 1024 or d_in * d_out > 1 << 20
        rows = None if not big else sample_rows(T, 64, seed=1, must=[0, T - 1])
        y_ref, inv = reference(p, x, W, idx, rows=rows)
        got = y.cpu() if rows is None else y.cpu()[torch.as_tensor(rows)]
        assert_close(got, y_ref, inv, dtype)
    finally:
        p.close()
