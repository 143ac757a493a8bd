"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Small layers are compared on every output element; the full-size layers
in the launch configuration the benchmark times: every token's routing,
and every output row at the GPT-2, Mixtral and gpt-oss decode shapes, a
sample holding a token of every expert group at the DeepSeek-V3 shape.  Routing and counts must be bit-exact; outputs within
2e-2 (bf16) / 1e-4 (fp32) max-relative error; kept weights within 2e-6.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_common import (check_outputs, check_routing, covering_tokens, require_gpu,
                        run_forward, sample_tokens, to_f64)
from helpers import BF16, F32, GELU, SWIGLU, random_layer
from sparse_mixture_experts_07_amd import binding as B
from sparse_mixture_experts_07_amd.device import DeviceLayer, Forward

pytestmark = pytest.mark.gpu

SMALL = {
    "tiny-gelu-bias-bf16": dict(T=37, d=64, h=128, E=5, k=2, act=GELU, dtype=BF16, expert_bias=True),
    "ntail-swiglu-bf16": dict(T=300, d=192, h=320, E=7, k=3, act=SWIGLU, dtype=BF16, bias=True),
    "shared-swiglu-bf16": dict(T=129, d=128, h=256, E=16, k=4, act=SWIGLU, dtype=BF16, S=1),
    "one-token-f32": dict(T=1, d=64, h=64, E=4, k=1, act=GELU, dtype=F32),
    "k-eq-E-shared-f32": dict(T=50, d=64, h=192, E=8, k=8, act=SWIGLU, dtype=F32, S=1),
    "single-expert-bf16": dict(T=77, d=128, h=128, E=1, k=1, act=GELU, dtype=BF16, expert_bias=True),
    "big-groups-swiglu-bf16": dict(T=1000, d=256, h=512, E=3, k=2, act=SWIGLU, dtype=BF16),
    "e256-swiglu-bf16": dict(T=600, d=64, h=64, E=256, k=8, act=SWIGLU, dtype=BF16, bias=True),
    "gelu-f32-bias": dict(T=200, d=128, h=256, E=6, k=2, act=GELU, dtype=F32, expert_bias=True),
    "mid-groups-gelu-bf16": dict(T=700, d=128, h=192, E=4, k=2, act=GELU, dtype=BF16, expert_bias=True),
    "mid-groups-swiglu-shared-bf16": dict(T=520, d=192, h=320, E=3, k=2, act=SWIGLU, dtype=BF16, S=1),
    # router kernel selection: one chain per lane for decode-size batches
    # (32 and 64 expert lanes), four-wave workgroups for large batches, the
    # staged kernel for more experts on large batches
    "e48-decode-swiglu-bf16": dict(T=40, d=192, h=128, E=48, k=6, act=SWIGLU, dtype=BF16),
    "e32-decode-swiglu-f32": dict(T=64, d=128, h=128, E=32, k=4, act=SWIGLU, dtype=F32),
    "e24-bias-bf16": dict(T=900, d=128, h=128, E=24, k=3, act=SWIGLU, dtype=BF16, bias=True),
    "e16-bigT-bf16": dict(T=4200, d=64, h=64, E=16, k=2, act=GELU, dtype=BF16),
    "e20-bigT-bf16": dict(T=1500, d=64, h=64, E=20, k=2, act=SWIGLU, dtype=BF16),
    "f32-lane-router": dict(T=2100, d=64, h=64, E=8, k=2, act=GELU, dtype=F32),
    # more than 16384 assignments: the multi-workgroup grouping kernels
    "many-assignments-bf16": dict(T=3000, d=64, h=64, E=64, k=6, act=SWIGLU, dtype=BF16),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def test_tiny_fp32_layer_every_element():
    """The tiny fp32 layer (T=64, d=64, h=256, 8 experts, top-2, GELU)."""
    L = synthetic.make_inputs(synthetic.TINY)
    res, _, _ = run_forward(L)
    check_routing(L, res["idx"], res["w"], res["counts"])
    check_outputs(L, res["y"], range(L.cfg.T))


@pytest.mark.parametrize("name", list(SMALL))
def test_small_layers_every_element(name):
    kw = dict(SMALL[name])
    L = random_layer(zlib.crc32(name.encode()) % 1000, wstd=0.1, **kw)
    res, _, _ = run_forward(L)
    ridx, rw = check_routing(L, res["idx"], res["w"], res["counts"])
    check_outputs(L, res["y"], range(L.cfg.T))
    rc, rimp = oracle.counts(L.cfg, ridx, rw)
    np.testing.assert_allclose(res["importance"], rimp, rtol=1e-5)
    cvi, cvl, lb = oracle.load_stats(rc, rimp)
    np.testing.assert_allclose(res["stats"], [cvi, cvl, lb], rtol=1e-4, atol=1e-9)


def test_group_size_classes_in_one_layer():
    """Skewed router biases give groups of <= 64, 65..384 and > 384 rows in
    the same layer, so every tile class of the grouped GEMM runs; the
    shared expert (T rows) lands in the largest class."""
    L = random_layer(21, T=1000, d=128, h=256, E=8, k=2, act=SWIGLU, dtype=BF16,
                     S=1, bias=True, wstd=0.1)
    L.b_gate = np.float32([4, 3, 2, 1, 0, -1, -2, -3]) * np.float32(0.6)
    res, _, _ = run_forward(L)
    c = res["counts"]
    assert (c <= 64).any() and ((c > 64) & (c <= 384)).any() and (c > 384).any(), c
    check_routing(L, res["idx"], res["w"], res["counts"])
    check_outputs(L, res["y"], range(1000))


# Shapes that steer the large-group GEMM to each of its kernels and row
# tiles: the DMA-fed kernel (K <= 8192) and the ping-pong kernel (longer K),
# each with 256- and 192-row tiles (the 256-row tile wins when the 192-row
# tiling needs an extra round over the CUs).
LARGE_TILES = {
    "dma-bm256-down": dict(T=3200, d=2048, h=128, E=2, k=2, act=SWIGLU, dtype=BF16),
    "pp-bm192-down": dict(T=300, d=128, h=8256, E=4, k=2, act=SWIGLU, dtype=BF16),
    "pp-bm256-down": dict(T=3200, d=2048, h=8256, E=2, k=2, act=SWIGLU, dtype=BF16),
}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", list(LARGE_TILES))
def test_large_group_kernels(name):
    L = random_layer(zlib.crc32(name.encode()) % 1000, wstd=0.05, **LARGE_TILES[name])
    res, _, _ = run_forward(L)
    check_routing(L, res["idx"], res["w"], res["counts"])
    check_outputs(L, res["y"], sample_tokens(L.cfg.T, 40))


def test_single_class_with_a_small_group():
    """Groups averaging 512 rows or more all go to the large-tile kernel,
    including a group of a few rows (skewed router bias)."""
    L = random_layer(33, T=3000, d=64, h=128, E=4, k=2, act=SWIGLU, dtype=BF16,
                     bias=True, wstd=0.1)
    L.b_gate = np.float32([1.5, 1.0, 0.0, -1.2])
    res, _, _ = run_forward(L)
    c = res["counts"]
    assert c.sum() >= 512 * 4 and (c <= 64).any(), c
    check_routing(L, res["idx"], res["w"], res["counts"])
    check_outputs(L, res["y"], range(3000))


def test_stage_calls_equal_forward_and_are_deterministic():
    """route -> permute -> expert_ffn -> combine through the separate entry
    points gives bitwise the moe_forward output; two runs agree bitwise."""
    L = random_layer(5, T=257, d=128, h=192, E=9, k=3, act=SWIGLU, dtype=BF16, S=1)
    res, dl, fw = run_forward(L)
    y1 = fw.y.clone()
    fw()
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), fw.y.view(torch.int16))
    c = dl.cfg
    T, k, E, d = c.num_tokens, c.top_k, c.num_experts, c.d_model
    dev = dl.x.device
    R = B.moe_grouped_rows(c)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    B.moe_route(c, dl.x, dl.w_gate, dl.b_gate, idx, w, counts)
    ws = torch.empty(B.moe_workspace_bytes(c), dtype=torch.uint8, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm_src = torch.empty(T * k, dtype=torch.int32, device=dev)
    pos = torch.empty(T * k, dtype=torch.int32, device=dev)
    imp = torch.empty(E, dtype=torch.float32, device=dev)
    x_perm = torch.empty((T * k, d), dtype=torch.bfloat16, device=dev)
    B.moe_permute(c, idx, w, dl.x, offsets, perm_src, pos, imp, None, x_perm, ws)
    y_perm = torch.empty((R, d), dtype=torch.bfloat16, device=dev)
    B.moe_expert_ffn(c, dl.weights(), x_perm, dl.x, offsets, y_perm, ws)
    y = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    B.moe_combine(c, y_perm, pos, w, y)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y1.view(torch.int16))
    assert torch.equal(counts, fw.counts) and torch.equal(idx, fw.topk_idx)


def test_token_permutation_equivariance():
    """Shuffling the tokens shuffles the outputs bitwise: a row's result
    does not depend on where its token lands in the grouped tiles."""
    L = random_layer(6, T=300, d=128, h=256, E=6, k=2, act=SWIGLU, dtype=BF16)
    res, _, _ = run_forward(L)
    perm = np.random.default_rng(0).permutation(300)
    L.x = np.ascontiguousarray(L.x[perm])
    res2, _, _ = run_forward(L)
    assert np.array_equal(res2["y"], res["y"][perm])
    assert np.array_equal(res2["idx"], res["idx"][perm])


def test_ties_and_collapse_to_one_expert():
    """x = 0 rows tie every score: experts 0..k-1 with weight 1/k.  A huge
    bias on expert 3 sends every token there first (others may be empty)."""
    L = random_layer(7, T=130, d=64, h=128, E=8, k=3, act=SWIGLU, dtype=BF16, bias=True)
    L.x[::7] = 0
    L.b_gate = np.zeros(8, np.float32)
    res, _, _ = run_forward(L)
    zero_rows = np.arange(0, 130, 7)
    assert np.all(res["idx"][zero_rows] == [0, 1, 2])
    assert np.all(res["w"][zero_rows] == np.float32(1 / 3))
    check_routing(L, res["idx"], res["w"], res["counts"])
    check_outputs(L, res["y"], range(130))
    L.b_gate = np.zeros(8, np.float32)
    L.b_gate[3] = 1e4
    res, _, _ = run_forward(L)
    assert np.all(res["idx"][:, 0] == 3) and res["counts"][3] == 130
    check_routing(L, res["idx"], res["w"], res["counts"])
    check_outputs(L, res["y"], range(130))


def test_zero_tokens():
    L = random_layer(8, T=1, d=64, h=64, E=4, k=2, act=SWIGLU, dtype=BF16)
    L.cfg = L.cfg.with_(T=0)
    L.x = np.zeros((0, 64), np.uint16)
    dl = DeviceLayer.upload(L)
    fw = Forward(dl)
    fw.counts.fill_(7)
    fw.importance.fill_(7)
    fw.stats.fill_(7)
    fw()
    torch.cuda.synchronize()
    assert fw.counts.eq(0).all() and fw.importance.eq(0).all() and fw.stats.eq(0).all()


# ------------------------------------------------------------- full size --

ROUTE_CFGS = ["tiny-fp32", "gpt2-moe", "mixtral-8x7b", "gpt-oss-20b-decode", "deepseek-v3"]


@pytest.mark.parametrize("name", ROUTE_CFGS)
def test_full_size_routing_and_permutation(name):
    """Every token: router scores, indices and counts bit-exact; grouping
    (offsets, sources, positions) bit-exact against the oracle's, x_perm a
    bit-exact gather of x; Importance and the load statistics."""
    cfg = synthetic.BY_NAME[name]
    L = synthetic.make_inputs(cfg, experts=False)
    dl = DeviceLayer.upload(L)
    c = dl.cfg
    T, k, E, d = cfg.T, cfg.k, cfg.E, cfg.d
    dev = dl.x.device
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    B.moe_route(c, dl.x, dl.w_gate, dl.b_gate, idx, w, counts, logits)
    torch.cuda.synchronize()
    ridx, rw, rsc = oracle.route(L, want_scores=True)
    assert np.array_equal(logits.cpu().numpy().view(np.uint32), rsc.view(np.uint32))
    assert np.array_equal(idx.cpu().numpy(), ridx)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=2e-6, atol=1e-7)
    rc, rimp = oracle.counts(cfg, ridx, rw)
    assert np.array_equal(counts.cpu().numpy(), rc)

    # permutation on the oracle's routing (inputs never come from the GPU)
    gidx = torch.from_numpy(ridx).to(dev)
    gw = torch.from_numpy(rw.astype(np.float32)).to(dev)
    ws = torch.empty(B.moe_workspace_bytes(c), dtype=torch.uint8, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm_src = torch.empty(T * k, dtype=torch.int32, device=dev)
    pos = torch.empty(T * k, dtype=torch.int32, device=dev)
    imp = torch.empty(E, dtype=torch.float32, device=dev)
    stats = torch.empty(3, dtype=torch.float64, device=dev)
    x_perm = torch.empty((T * k, d), dtype=dl.x.dtype, device=dev)
    pcounts = torch.full((E,), -1, dtype=torch.int32, device=dev)
    B.moe_permute(c, gidx, gw, dl.x, offsets, perm_src, pos, imp, stats, x_perm, ws,
                  counts=pcounts)
    torch.cuda.synchronize()
    assert np.array_equal(pcounts.cpu().numpy(), rc)   # the grouping's counts
    roff, rsrc, rpos = oracle.permute(cfg, ridx)
    assert np.array_equal(offsets.cpu().numpy(), roff)
    assert np.array_equal(perm_src.cpu().numpy(), rsrc)
    assert np.array_equal(pos.cpu().numpy(), rpos)
    xp = x_perm.view(torch.int16 if cfg.dtype == 1 else torch.int32).cpu().numpy()
    assert np.array_equal(xp.view(L.x.dtype), L.x[rsrc])
    np.testing.assert_allclose(imp.cpu().numpy(), rimp, rtol=1e-5)
    np.testing.assert_allclose(stats.cpu().numpy(), oracle.load_stats(rc, rimp),
                               rtol=1e-4, atol=1e-9)


# Every output row is compared at the GPT-2, Mixtral and decode shapes (the
# oracle runs the whole batch: about 40 s of CPU for the Mixtral shape on 16
# cores); at the DeepSeek-V3 shape (about 80 s for all 8192 tokens) a sample
# that holds a token of every expert group the batch touches, so that every
# group and every group-size class of the grouped GEMM is compared, plus
# first, middle and last tokens.
FWD_ROWS = {"gpt2-moe": None, "mixtral-8x7b": None, "gpt-oss-20b-decode": None,
            "deepseek-v3": 512}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(FWD_ROWS))
def test_full_size_forward(name):
    """The benchmarked layer: routing of every token bit-exact; the
    max-relative error over the whole compared output (every row, or the
    covering sample) within tolerance."""
    cfg = synthetic.BY_NAME[name]
    L = synthetic.make_inputs(cfg)
    res, dl, fw = run_forward(L)
    del fw, dl
    torch.cuda.empty_cache()
    ridx, _ = check_routing(L, res["idx"], res["w"], res["counts"])
    n = FWD_ROWS[name]
    toks = range(cfg.T) if n is None else covering_tokens(ridx, n)
    err = check_outputs(L, res["y"], toks)
    print(f"{name}: max-relative error {err:.3e} over {len(toks)} of {cfg.T} rows")


GATHER_CASES = {
    "small-groups": dict(T=100, d=128, h=128, E=16, k=2, act=SWIGLU, dtype=BF16),
    "three-classes-shared": dict(T=1000, d=128, h=256, E=8, k=2, act=SWIGLU, dtype=BF16, S=1,
                                 bias=True),
    "dma-large-groups": dict(T=1200, d=256, h=512, E=3, k=2, act=SWIGLU, dtype=BF16),
    "pp-long-k": dict(T=300, d=8256, h=128, E=4, k=2, act=SWIGLU, dtype=BF16),
    "gelu-bias": dict(T=700, d=128, h=192, E=4, k=2, act=GELU, dtype=BF16, expert_bias=True),
    "f32-gelu-bias": dict(T=200, d=128, h=256, E=6, k=2, act=GELU, dtype=F32, expert_bias=True),
}


@pytest.mark.parametrize("name", list(GATHER_CASES))
@pytest.mark.parametrize("capacity", [0, 70])
def test_gathered_rows_equal_grouped_copy(name, capacity):
    """The up projection reading the token rows of x in place (perm_src)
    gives bitwise the result of reading the grouped copy x_perm, for every
    GEMM kernel and tile class, with and without dropped slots; so does the
    training up projection (hidden and pre-activations)."""
    kw = dict(GATHER_CASES[name])
    L = random_layer(zlib.crc32(name.encode()) % 1000, wstd=0.1, **kw)
    if name == "three-classes-shared":
        L.b_gate = np.float32([4, 3, 2, 1, 0, -1, -2, -3]) * np.float32(0.6)
    dl = DeviceLayer.upload(L, capacity=capacity)
    c = dl.cfg
    T, k, E, d, h = L.cfg.T, L.cfg.k, L.cfg.E, L.cfg.d, L.cfg.h
    dev = dl.x.device
    dt = dl.act_dtype
    R = B.moe_grouped_rows(c)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    B.moe_route(c, dl.x, dl.w_gate, dl.b_gate, idx, w, None)
    ws = torch.empty(B.moe_workspace_bytes(c), dtype=torch.uint8, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm_src = torch.empty(T * k, dtype=torch.int32, device=dev)
    pos = torch.empty(T * k, dtype=torch.int32, device=dev)
    imp = torch.empty(E, dtype=torch.float32, device=dev)
    x_perm = torch.empty((T * k, d), dtype=dt, device=dev)
    B.moe_permute(c, idx, w, dl.x, offsets, perm_src, pos, imp, None, x_perm, ws)
    h_copy = torch.full((R, h), 7, dtype=dt, device=dev)
    h_gath = torch.full((R, h), 7, dtype=dt, device=dev)
    B.moe_expert_up(c, dl.weights(), x_perm, dl.x, offsets, h_copy)
    B.moe_expert_up(c, dl.weights(), None, dl.x, offsets, h_gath, perm_src=perm_src)
    torch.cuda.synchronize()
    n = int(offsets[E].item())
    rows = list(range(n)) + list(range(T * k, R))   # computed rows (kept, then shared)
    iv = torch.int16 if dt == torch.bfloat16 else torch.int32
    assert torch.equal(h_copy.view(iv)[rows], h_gath.view(iv)[rows])
    if dt == torch.bfloat16:
        nup = 2 * h if L.cfg.act == SWIGLU else h
        p_copy = torch.empty((R, nup), dtype=dt, device=dev)
        p_gath = torch.empty((R, nup), dtype=dt, device=dev)
        t_copy = torch.empty_like(h_copy)
        t_gath = torch.empty_like(h_gath)
        B.moe_expert_up_train(c, dl.weights(), x_perm, dl.x, offsets, t_copy, p_copy)
        B.moe_expert_up_train(c, dl.weights(), None, dl.x, offsets, t_gath, p_gath,
                              perm_src=perm_src)
        torch.cuda.synchronize()
        assert torch.equal(t_copy.view(iv)[rows], t_gath.view(iv)[rows])
        assert torch.equal(p_copy.view(iv)[rows], p_gath.view(iv)[rows])
        assert torch.equal(t_gath.view(iv)[rows], h_gath.view(iv)[rows])
