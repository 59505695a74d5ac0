"""mla_decode_step (the whole step behind one call) against the CPU oracle, on the GPU.

For one bf16 sequence at the V3 head sizes with at most 4096 cached tokens the call is a single
kernel launch whose workgroups hand the folded query and the split partials to each other inside
the launch; other shapes take the three-call form.  Every compared (sequence, head) pair must meet
the tolerance on its own (relative L2 1e-2 for bf16/fp8, 1e-5 for fp32).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from mla_latent_kv_attn_amd import ops
from workloads import make_inputs
from workloads.configs import WORKLOADS
from workloads.device import device_cache, to_device

from tests.test_parity_gpu import compare, all_finite

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    ops._lib.lib()


def flag_region_bytes():
    # the error word (256 bytes) and the two flag arrays of the one-launch form
    return 256 + (4 * 32 * 4 * 64 + 128 * 32) * 4


def run_step(inp, workspace=None, cache=None, dev=None, calls=1):
    wl = inp.wl
    print(f"[gpu] decode_step {wl.name} B={wl.B} H={wl.H} layout={wl.layout} dtype={wl.dtype} "
          f"lens[:8]={inp.lens[:8].tolist()} calls={calls}", flush=True)
    dev = dev if dev is not None else to_device(inp)
    cache = cache if cache is not None else device_cache(inp, dev)
    if workspace is None:
        workspace = ops.mla_decode_step_workspace(wl.B, wl.H, wl.d_c, wl.n_max, "cuda")
    q_dtype = dev["q_C"].dtype
    outs = []
    for _ in range(calls):
        q_abs = torch.full((wl.B, wl.H, wl.d_c), float("nan"), dtype=q_dtype, device="cuda")
        o_lat = torch.full((wl.B, wl.H, wl.d_c), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((wl.B, wl.H), float("nan"), dtype=torch.float32, device="cuda")
        o = ops.mla_decode_step(dev["q_C"], dev["q_R"], dev["W_UK"], dev["W_UV"], cache, dev["lens"], wl.n_max,
                                workspace, q_abs=q_abs, o_latent=o_lat, lse=lse)
        torch.cuda.synchronize()
        outs.append({"q_abs": q_abs.float().cpu().numpy().astype(np.float64),
                     "o_lat": o_lat.cpu().numpy().astype(np.float64),
                     "lse": lse.cpu().numpy().astype(np.float64),
                     "o": o.cpu().numpy().astype(np.float64)})
    return outs, workspace


def check_workspace_clean(ws):
    head = ws[:flag_region_bytes()].cpu()
    err = int(head[:4].view(torch.int32)[0])
    assert err == 0, f"a wait inside the one-launch step gave up (error word {err})"
    assert int(torch.count_nonzero(head)) == 0, "flags left set after the step"


def v3_b1(lens, name="step-b1", layout="split", n_max=4096, **kw):
    wl = WORKLOADS[2].with_(name=name, n_max=n_max, len_lo=0, len_hi=n_max, layout=layout, **kw)
    return make_inputs(wl, lens=np.array(lens))


def test_step_cfg2_full():
    inp = make_inputs(2)
    (got,), ws = run_step(inp)
    check_workspace_clean(ws)
    all_finite(got, inp)
    compare(inp, got, oracle.decode(inp))


@pytest.mark.parametrize("L", [1, 2, 31, 32, 33, 100, 1000, 2049, 4064, 4095])
def test_step_b1_lengths(L):
    """Ragged lengths: fewer tiles than splits (empty splits), one partial tile, and the longest
    sequences (4 tiles per split).  n_max 4096 keeps the one-launch form."""
    inp = v3_b1([L], name=f"step-b1-L{L}")
    (got,), ws = run_step(inp)
    check_workspace_clean(ws)
    all_finite(got, inp)
    compare(inp, got, oracle.decode(inp))


def test_step_b1_empty_sequence():
    inp = v3_b1([0], name="step-b1-empty")
    (got,), ws = run_step(inp)
    check_workspace_clean(ws)
    assert np.all(got["o"] == 0.0) and np.all(got["o_lat"] == 0.0) and np.all(np.isneginf(got["lse"]))
    ref = oracle.decode(inp)
    np.testing.assert_allclose(got["q_abs"], ref["q_abs"], rtol=1e-2, atol=1e-2)


@pytest.mark.parametrize("page", [32, 64, 256])
def test_step_b1_paged(page):
    wl = WORKLOADS[4].with_(name=f"step-b1-paged{page}", B=1, n_max=4096, len_lo=0, len_hi=4096, page_size=page)
    inp = make_inputs(wl, lens=np.array([3001]))
    (got,), ws = run_step(inp)
    check_workspace_clean(ws)
    all_finite(got, inp)
    compare(inp, got, oracle.decode(inp))


def test_step_b1_packed_rows():
    inp = v3_b1([777], name="step-b1-packed", layout="packed")
    (got,), ws = run_step(inp)
    all_finite(got, inp)
    compare(inp, got, oracle.decode(inp))


def test_step_repeated_calls_bitwise_and_flags_reset():
    """Consecutive calls on one workspace: every call sees its own hand-overs (the flags start at
    zero and end at zero), results identical bit for bit, no wait gave up."""
    inp = v3_b1([4096], name="step-repeat")
    outs, ws = run_step(inp, calls=4)
    check_workspace_clean(ws)
    for o in outs[1:]:
        for k in ("q_abs", "o_lat", "lse", "o"):
            np.testing.assert_array_equal(o[k], outs[0][k])
    compare(inp, outs[-1], oracle.decode(inp))


def test_step_changing_lengths_on_one_workspace():
    """The same workspace and buffers with the sequence length changing between calls (4096, 5,
    0, 1500): every call matches the oracle for its own length."""
    import dataclasses
    ws = ops.mla_decode_step_workspace(1, 128, 512, 4096, "cuda")
    base = v3_b1([4096], name="step-varlen")
    dev = to_device(base)
    cache = device_cache(base, dev)
    for L in (4096, 5, 0, 1500):
        # the same stored rows and queries; only the length changes
        inp = dataclasses.replace(base, lens=np.array([L], dtype=np.int32))
        dev["lens"].fill_(L)
        (got,), _ = run_step(inp, workspace=ws, cache=cache, dev=dev)
        check_workspace_clean(ws)
        if L:
            compare(inp, got, oracle.decode(inp))
        else:
            assert np.all(got["o"] == 0.0) and np.all(np.isneginf(got["lse"]))


def test_step_padded_row_strides():
    wl = WORKLOADS[2].with_(name="step-padded", n_max=4096, len_lo=0, len_hi=4096)
    inp = make_inputs(wl, lens=np.array([2500]))
    dev = to_device(inp)
    N = wl.n_max
    lat = torch.zeros((1, N + 3, wl.d_c + 64), dtype=dev["latent"].dtype, device="cuda")
    lat[:, :N, :wl.d_c] = dev["latent"]
    rope = torch.zeros((1, N + 5, wl.d_R + 8), dtype=dev["rope"].dtype, device="cuda")
    rope[:, :N, :wl.d_R] = dev["rope"]
    cache = ops.Cache.split(lat[:, :N, :wl.d_c], rope[:, :N, :wl.d_R])
    (got,), _ = run_step(inp, cache=cache, dev=dev)
    compare(inp, got, oracle.decode(inp))


def test_step_graph_replays_match_eager():
    """The one-launch step captured in a HIP graph and replayed several times, with unrelated eager
    work between replays: every replay gives the eager result bit for bit and leaves the flags
    clear."""
    from mla_latent_kv_attn_amd.step import DecodeStep
    inp = v3_b1([4000], name="step-graph")
    dev = to_device(inp)
    cache = device_cache(inp, dev)
    print("[gpu] decode_step graph capture", flush=True)
    step = DecodeStep(1, 128, 128, 512, 64, 4096, torch.bfloat16, "cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        eager = step(dev["q_C"], dev["q_R"], dev["W_UK"], dev["W_UV"], cache, dev["lens"]).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(dev["q_C"], dev["q_R"], dev["W_UK"], dev["W_UV"], cache, dev["lens"])
    for _ in range(4):
        step.out.zero_()
        _ = torch.randn(1000, device="cuda").sum().item()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.out, eager)
    check_workspace_clean(step.workspace)
    got = {"q_abs": step.q_abs.float().cpu().numpy().astype(np.float64),
           "o_lat": step.o_latent.cpu().numpy().astype(np.float64),
           "lse": step.lse.cpu().numpy().astype(np.float64), "o": step.out.cpu().numpy().astype(np.float64)}
    compare(inp, got, oracle.decode(inp))


@pytest.mark.parametrize("name", ["b3-split", "f32", "fp8", "b1-long"])
def test_step_multi_kernel_form(name):
    """Shapes outside the one-launch form go through the three calls inside mla_decode_step."""
    if name == "b3-split":
        inp = make_inputs(WORKLOADS[2].with_(name="step-b3", B=3, n_max=300, len_lo=1, len_hi=300),
                          lens=np.array([300, 97, 2]))
    elif name == "f32":
        inp = make_inputs(1)
    elif name == "fp8":
        inp = make_inputs(WORKLOADS[5].with_(name="step-fp8", B=2, n_max=160, len_lo=1, len_hi=160),
                          lens=np.array([160, 7]))
    else:
        inp = v3_b1([5000], name="step-b1-5000", n_max=5000)
    (got,), _ = run_step(inp)
    all_finite(got, inp)
    compare(inp, got, oracle.decode(inp))
