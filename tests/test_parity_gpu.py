"""Parity of the HIP path (through the C ABI) against the CPU oracle, on the GPU.

Tolerance (relative L2 of each compared (sequence, head) pair on its own): 1e-5 for the fp32
path, 1e-2 for bf16/fp8, against the float64 oracle.  Full-size workloads compare sampled (sequence, head) pairs, which
the oracle computes one by one, plus properties that hold at any size.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from mla_latent_kv_attn_amd import ops
from workloads import make_inputs
from workloads.configs import WORKLOADS
from workloads.device import device_cache, to_device
from workloads.gen import bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 1e-2, "fp8": 1e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    ops._lib.lib()


def run_gpu(inp, num_splits=0):
    print(f"[gpu] {inp.wl.name} B={inp.wl.B} H={inp.wl.H} layout={inp.wl.layout} dtype={inp.wl.dtype} "
          f"splits={num_splits} lens[:8]={inp.lens[:8].tolist()}", flush=True)
    dev = to_device(inp)
    cache = device_cache(inp, dev)
    q_abs = ops.mla_absorb_q(dev["q_C"], dev["W_UK"])
    o_lat, lse = ops.mla_decode_attn(q_abs, dev["q_R"], cache, dev["lens"], inp.wl.n_max, d_h=inp.wl.d_h,
                                     num_splits=num_splits)
    o = ops.mla_uv_out(o_lat, dev["W_UV"])
    torch.cuda.synchronize()
    return {"q_abs": q_abs.float().cpu().numpy().astype(np.float64),
            "o_lat": o_lat.cpu().numpy().astype(np.float64),
            "lse": lse.cpu().numpy().astype(np.float64),
            "o": o.cpu().numpy().astype(np.float64)}


def per_pair_errors(got, ref, mask):
    """Relative L2 of every compared (sequence, head) pair on its own, per output.

    Returns {key: (max error, (b, h) of the max, global error over all pairs)}.  A pair whose
    reference row is all zero (an empty sequence's o_lat / o) is checked exactly elsewhere."""
    out = {}
    for key in ("q_abs", "o_lat", "o"):
        worst, where = 0.0, None
        for b, h in zip(*np.nonzero(mask)):
            r = ref[key][b, h]
            if not np.any(r):
                continue
            e = oracle.relative_l2(got[key][b, h], r)
            if not e <= worst:     # NaN errors are the worst of all
                worst, where = e, (int(b), int(h))
        out[key] = (worst, where, oracle.relative_l2(got[key][mask], ref[key][mask]))
    return out


def compare(inp, got, ref, pairs=None, tol=None):
    """Every compared (sequence, head) pair must meet the tolerance on its own: relative L2 of
    its q_abs, o_lat and o rows against the oracle's.  A global norm would let one head's error
    hide among the rest (one head 5 % off among 128 moves the global figure by 0.44 %)."""
    tol = TOL[inp.wl.dtype] if tol is None else tol
    B, H = inp.wl.B, inp.wl.H
    mask = np.zeros((B, H), dtype=bool)
    if pairs is None:
        mask[:] = True
    else:
        for b, h in pairs:
            mask[b, h] = True
    nonempty = mask & (inp.lens[:, None] > 0)
    per = per_pair_errors(got, ref, mask)
    errs = {k: v[2] for k, v in per.items()}
    errs.update({f"{k}_max_pair": v[0] for k, v in per.items()})
    if nonempty.any():
        errs["lse_abs"] = float(np.max(np.abs(got["lse"][nonempty] - ref["lse"][nonempty])))
    empty = mask & (inp.lens[:, None] == 0)
    if empty.any():
        assert np.all(got["o_lat"][empty] == 0.0) and np.all(got["o"][empty] == 0.0)
        assert np.all(np.isneginf(got["lse"][empty]))
    worst = {k: v[1] for k, v in per.items()}
    print(f"[parity] {inp.wl.name}: {errs} worst pairs {worst}", flush=True)
    for key in ("q_abs", "o_lat", "o"):
        assert per[key][0] <= tol, (key, "pair", per[key][1], per[key][0])
    if "lse_abs" in errs:
        assert errs["lse_abs"] <= (1e-4 if inp.wl.dtype == "f32" else 2e-2), errs
    return errs


def all_finite(got, inp):
    ne = inp.lens > 0
    for key in ("o_lat", "o"):
        assert np.all(np.isfinite(got[key])), key
    assert np.all(np.isfinite(got["lse"][ne]))


# ------------------------------------------------------------------------------------------------
# the five workloads
# ------------------------------------------------------------------------------------------------
def test_cfg1_tiny_f32_full():
    inp = make_inputs(1)
    got = run_gpu(inp)
    compare(inp, got, oracle.decode(inp))


def test_cfg2_v3_b1_full():
    inp = make_inputs(2)
    got = run_gpu(inp)
    all_finite(got, inp)
    compare(inp, got, oracle.decode(inp))


def _sample_pairs(inp, n_b=6, seed=0):
    rng = np.random.default_rng(seed)
    B, H = inp.wl.B, inp.wl.H
    bs = {int(np.argmin(inp.lens)), int(np.argmax(inp.lens)), 0, B - 1}
    bs |= set(int(x) for x in rng.choice(B, size=min(B, n_b), replace=False))
    pairs = []
    for b in sorted(bs):
        for h in {0, H - 1, int(rng.integers(H))}:
            pairs.append((b, h))
    return pairs


@pytest.mark.parametrize("cfg", [3, 4, 5])
def test_full_size_sampled(cfg):
    inp = make_inputs(cfg)
    got = run_gpu(inp)
    all_finite(got, inp)
    pairs = _sample_pairs(inp)
    ref = oracle.decode(inp, pairs=pairs)
    compare(inp, got, ref, pairs=pairs)


# ------------------------------------------------------------------------------------------------
# small shapes that span several tiles, ragged tails and empty sequences (full comparison)
# ------------------------------------------------------------------------------------------------
def mini(cfg, **kw):
    return WORKLOADS[cfg].with_(**kw)


MINI = {
    "packed": (mini(3, name="mini-packed", B=6, n_max=200, len_lo=1, len_hi=200), [1, 31, 32, 33, 0, 200]),
    "paged": (mini(4, name="mini-paged", B=4, n_max=256, len_lo=1, len_hi=256), [256, 65, 1, 0]),
    "fp8": (mini(5, name="mini-fp8", B=4, n_max=160, len_lo=1, len_hi=160), [160, 7, 64, 0]),
    "split": (mini(2, name="mini-split", B=3, n_max=300, len_lo=1, len_hi=300), [300, 97, 2]),
    "h64": (mini(2, name="mini-h64", B=2, H=64, n_max=130, len_lo=1, len_hi=130), [130, 40]),
    "h32": (mini(2, name="mini-h32", B=2, H=32, n_max=130, len_lo=1, len_hi=130), [77, 130]),
    "f32-var": (mini(1, name="mini-f32", B=4, n_max=100, len_lo=1, len_hi=100), [100, 1, 0, 33]),
    "fp8-h32": (mini(5, name="mini-fp8-h32", B=3, H=32, n_max=200, len_lo=1, len_hi=200), [200, 33, 0]),
    "fp8-h64": (mini(5, name="mini-fp8-h64", B=2, H=64, n_max=130, len_lo=1, len_hi=130), [1, 130]),
    "paged-h64": (mini(4, name="mini-paged-h64", B=3, H=64, n_max=192, len_lo=1, len_hi=192), [192, 64, 65]),
}


@pytest.mark.parametrize("name", sorted(MINI))
def test_mini_full_compare(name):
    wl, lens = MINI[name]
    inp = make_inputs(wl, lens=np.array(lens))
    got = run_gpu(inp)
    all_finite(got, inp)
    compare(inp, got, oracle.decode(inp))


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 1000])
def test_split_count_sweep(splits):
    wl, lens = MINI["packed"]
    inp = make_inputs(wl, lens=np.array(lens))
    got = run_gpu(inp, num_splits=splits)
    compare(inp, got, oracle.decode(inp))


def test_split_count_changes_only_rounding():
    inp = make_inputs(2)
    a = run_gpu(inp, num_splits=1)
    b = run_gpu(inp, num_splits=64)
    assert oracle.relative_l2(a["o"], b["o"]) <= 2e-3


def test_paged_equals_packed_bitwise():
    wl_pk = mini(3, name="pk", B=3, n_max=256, len_lo=1, len_hi=256, seed=21)
    wl_pg = mini(4, name="pg", B=3, n_max=256, len_lo=1, len_hi=256, seed=21)
    lens = np.array([256, 100, 37])
    a = run_gpu(make_inputs(wl_pk, lens=lens), num_splits=5)
    b = run_gpu(make_inputs(wl_pg, lens=lens), num_splits=5)
    for k in ("o_lat", "lse", "o"):
        np.testing.assert_array_equal(a[k], b[k])


def test_run_to_run_deterministic():
    wl, lens = MINI["fp8"]
    inp = make_inputs(wl, lens=np.array(lens))
    a = run_gpu(inp)
    b = run_gpu(inp)
    for k in ("q_abs", "o_lat", "lse", "o"):
        np.testing.assert_array_equal(a[k], b[k])


def test_rising_scores_force_rescales():
    """Rope keys grow with the token index, so the running maximum of the scores keeps rising
    within one segment and the accumulator is rescaled many times.  The growing term is the
    rope product, whose bf16 inputs are exact, so the check is not dominated by the bf16
    rounding of the folded query."""
    wl = mini(2, name="rising", B=2, n_max=1024, len_lo=1024, len_hi=1024)
    inp = make_inputs(wl)
    rope = bf16_bits_to_f32(inp.rope).reshape(2, 1024, 64)
    grow = (1.0 + np.arange(1024, dtype=np.float32) / 32.0)[None, :, None]
    inp.rope = f32_to_bf16_bits(rope * grow).reshape(inp.rope.shape)
    got = run_gpu(inp, num_splits=1)
    all_finite(got, inp)
    ref = oracle.decode(inp)
    # the scores must rise by several rescale thresholds (2^8, i.e. 5.5 in natural-log units)
    # over the sequence for the test to exercise the rescale path
    assert float(np.median(ref["lse"])) > 25.0
    compare(inp, got, ref)


def test_nan_padding_does_not_leak():
    wl, lens = MINI["split"]
    inp = make_inputs(wl, lens=np.array(lens), poison=True)
    assert np.any(inp.latent[1, 97:] == 0x7FC0)
    got = run_gpu(inp)
    all_finite(got, inp)


def test_graph_capture_replays_match_eager():
    """The whole step captured in a HIP graph, replayed several times with eager work in between,
    gives the eager result bit for bit on every replay."""
    from mla_latent_kv_attn_amd.step import DecodeStep
    wl, lens = MINI["packed"]
    inp = make_inputs(wl, lens=np.array(lens))
    dev = to_device(inp)
    cache = device_cache(inp, dev)
    print("[gpu] graph capture", flush=True)
    step = DecodeStep(wl.B, wl.H, wl.d_h, wl.d_c, wl.d_R, wl.n_max, torch.bfloat16, "cuda", num_splits=3)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        eager = step(dev["q_C"], dev["q_R"], dev["W_UK"], dev["W_UV"], cache, dev["lens"]).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(dev["q_C"], dev["q_R"], dev["W_UK"], dev["W_UV"], cache, dev["lens"])
    for _ in range(3):
        step.out.zero_()
        _ = torch.randn(1000, device="cuda").sum().item()     # unrelated eager work + sync
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.out, eager)


@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 33, 70, 129, 200])
def test_projections_batch_sweep(B):
    """The two projections alone at batch sizes on both sides of the small-batch switch (B <= 4
    streams the weights, larger batches use MFMA tiles of 128 / 32 rows), fed the oracle's o_lat.
    The MFMA absorb meets one to four 32-row blocks per workgroup (three at B = 70 and in the
    second workgroup row of B = 200); W_UV splits a head's rows over two workgroups when the grid
    would not fill the chip (B = 5, and the 32-head cases)."""
    wl = WORKLOADS[2].with_(name=f"proj-b{B}", B=B, H=128 if B <= 33 else 32, n_max=40, len_lo=1, len_hi=40)
    inp = make_inputs(wl)
    ref = oracle.decode(inp)
    print(f"[gpu] projections B={B}", flush=True)
    dev = to_device(inp)
    q_abs = ops.mla_absorb_q(dev["q_C"], dev["W_UK"])
    o_lat = torch.from_numpy(ref["o_lat"].astype(np.float32)).to("cuda")
    o = ops.mla_uv_out(o_lat, dev["W_UV"])
    torch.cuda.synchronize()
    got = {"q_abs": q_abs.float().cpu().numpy().astype(np.float64), "o_lat": ref["o_lat"],
           "o": o.cpu().numpy().astype(np.float64)}
    per = per_pair_errors(got, ref, np.ones((B, wl.H), dtype=bool))
    e_q, e_o = per["q_abs"][0], per["o"][0]
    print(f"[parity] projections B={B}: worst pair q_abs {e_q:.3e} {per['q_abs'][1]} o {e_o:.3e} {per['o'][1]}",
          flush=True)
    # per (sequence, head): q_abs is rounded once to bf16 (2^-9 relative); o is an fp32 product of
    # exact inputs
    assert e_q <= 4e-3 and e_o <= 1e-4


@pytest.mark.parametrize("B", [5, 70])
def test_absorb_output_alignment(B):
    """The MFMA absorb writes 16-byte pieces of whole output rows when q_abs is 16-byte aligned and
    single bf16 values otherwise: a q_abs that starts 4 bytes into its buffer gets the same bits."""
    wl = WORKLOADS[2].with_(name=f"absorb-align-b{B}", B=B, n_max=40, len_lo=1, len_hi=40)
    inp = make_inputs(wl)
    dev = to_device(inp)
    print(f"[gpu] absorb alignment B={B}", flush=True)
    aligned = ops.mla_absorb_q(dev["q_C"], dev["W_UK"])
    buf = torch.zeros(B * wl.H * wl.d_c + 8, dtype=torch.bfloat16, device="cuda")
    shifted = buf[2:2 + B * wl.H * wl.d_c].view(B, wl.H, wl.d_c)
    assert shifted.data_ptr() % 16 == 4
    ops.mla_absorb_q(dev["q_C"], dev["W_UK"], out=shifted)
    torch.cuda.synchronize()
    assert torch.equal(aligned.view(torch.int16), shifted.view(torch.int16))
    assert torch.count_nonzero(buf[:2].view(torch.int16)) == 0 and torch.count_nonzero(buf[-6:].view(torch.int16)) == 0


@pytest.mark.parametrize("H,B,splits", [(128, 64, 0), (128, 64, 200), (64, 128, 300)])
def test_wide_batch_combine(H, B, splits):
    """Batches wide enough (H/32 * B >= 256) for the combine pass to take one workgroup per
    (32-head block, sequence): full comparison, with empty sequences and several segments per
    sequence."""
    wl = WORKLOADS[3].with_(name=f"wide-h{H}-b{B}", B=B, H=H, n_max=96, len_lo=0, len_hi=96)
    rng = np.random.default_rng(7)
    lens = rng.integers(0, 97, size=B)
    lens[:3] = [0, 1, 96]
    inp = make_inputs(wl, lens=lens)
    got = run_gpu(inp, num_splits=splits)
    all_finite(got, inp)
    compare(inp, got, oracle.decode(inp))


def run_step(inp, num_splits=0):
    """The whole step through DecodeStep: absorb -> partial -> combine + W_UV (one fused kernel at
    batch <= 4 with bf16 weights, otherwise the two passes)."""
    from mla_latent_kv_attn_amd.step import DecodeStep
    print(f"[gpu] step {inp.wl.name} B={inp.wl.B} H={inp.wl.H} dtype={inp.wl.dtype} splits={num_splits}", flush=True)
    dev = to_device(inp)
    cache = device_cache(inp, dev)
    q_dtype = torch.float32 if inp.wl.dtype == "f32" else torch.bfloat16
    step = DecodeStep(inp.wl.B, inp.wl.H, inp.wl.d_h, inp.wl.d_c, inp.wl.d_R, inp.wl.n_max, q_dtype, "cuda",
                      num_splits=num_splits)
    step(dev["q_C"], dev["q_R"], dev["W_UK"], dev["W_UV"], cache, dev["lens"])
    torch.cuda.synchronize()
    return {"q_abs": step.q_abs.float().cpu().numpy().astype(np.float64),
            "o_lat": step.o_latent.cpu().numpy().astype(np.float64),
            "lse": step.lse.cpu().numpy().astype(np.float64),
            "o": step.out.cpu().numpy().astype(np.float64)}


@pytest.mark.parametrize("name,splits", [("split", 0), ("split", 1), ("split", 37), ("h64", 0), ("h32", 5),
                                         ("fp8", 0), ("paged", 9), ("f32-var", 0), ("packed", 4)])
def test_step_with_fused_combine_uv(name, splits):
    wl, lens = MINI[name]
    inp = make_inputs(wl, lens=np.array(lens))
    got = run_step(inp, num_splits=splits)
    all_finite(got, inp)
    compare(inp, got, oracle.decode(inp))


WIDE_STEP = {
    # large-batch partial pass (bf16 sums), packed cache, 40 sequences
    "packed-40": (mini(3, name="wide-packed", B=40, n_max=1100, len_lo=1, len_hi=1100), 0, 1),
    # paged cache, 20 sequences (W_UV over two workgroups per head)
    "paged-20": (mini(4, name="wide-paged", B=20, n_max=1856, len_lo=1, len_hi=1856), 0, 2),
    # E4M3 cache (large-batch partial at any batch), 6 sequences
    "fp8-6": (mini(5, name="wide-fp8", B=6, n_max=300, len_lo=1, len_hi=300), 0, 3),
    # about 200 segments per sequence (more than the combines keep weights for in LDS)
    "many-segments": (mini(2, name="wide-segs", B=5, n_max=8192, len_lo=1, len_hi=8192), 1000, 4),
    # small-batch partial pass (float sums) at B > 4
    "small-f32-sums": (mini(2, name="wide-small", B=12, n_max=640, len_lo=1, len_hi=640), 0, 5),
}


@pytest.mark.parametrize("name", list(WIDE_STEP))
def test_step_wide_batch(name):
    """The decode step at B > 4 (absorb, partial, combine, W_UV): bf16 and float partial sums,
    packed, paged and E4M3 caches, empty sequences, a sequence of one token, and many segments
    per sequence.  Sampled comparison (all pairs for the small cases)."""
    wl, splits, seed = WIDE_STEP[name]
    rng = np.random.default_rng(100 + seed)
    lens = rng.integers(1, wl.n_max + 1, size=wl.B)
    lens[:3] = [0, wl.n_max, 1]
    if name == "many-segments":
        lens[:] = wl.n_max
        lens[0] = 0
    inp = make_inputs(wl, lens=lens)
    got = run_step(inp, num_splits=splits)
    all_finite(got, inp)
    if wl.B * wl.n_max <= 4096:
        compare(inp, got, oracle.decode(inp))
    else:
        pairs = _sample_pairs(inp)
        compare(inp, got, oracle.decode(inp, pairs=pairs), pairs=pairs)


@pytest.mark.parametrize("cfg", [3, 4, 5])
def test_full_size_step_sampled(cfg):
    """The full-size batched workloads through the decode step, as the benchmark runs them."""
    inp = make_inputs(cfg)
    got = run_step(inp)
    all_finite(got, inp)
    pairs = _sample_pairs(inp)
    compare(inp, got, oracle.decode(inp, pairs=pairs), pairs=pairs)


def test_step_v3_b1_full():
    inp = make_inputs(2)
    got = run_step(inp)
    all_finite(got, inp)
    compare(inp, got, oracle.decode(inp))


@pytest.mark.parametrize("name", ["split", "fp8", "paged"])
def test_partial_warm_changes_nothing(name):
    """mla_decode_partial_warm (spare workgroups pull a buffer into the cache) leaves exactly the
    workspace contents of mla_decode_partial."""
    wl, lens = MINI[name]
    inp = make_inputs(wl, lens=np.array(lens))
    print(f"[gpu] partial warm {inp.wl.name}", flush=True)
    dev = to_device(inp)
    cache = device_cache(inp, dev)
    q_abs = ops.mla_absorb_q(dev["q_C"], dev["W_UK"])
    nbytes = ops.mla_decode_workspace_bytes(wl.B, wl.H, wl.d_c, wl.n_max, 5)
    ws = [torch.zeros(nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    ops.mla_decode_partial(q_abs, dev["q_R"], cache, dev["lens"], wl.n_max, wl.scale, ws[0], num_splits=5)
    ops.mla_decode_partial_warm(q_abs, dev["q_R"], cache, dev["lens"], wl.n_max, wl.scale, ws[1], dev["W_UV"],
                                num_splits=5)
    torch.cuda.synchronize()
    assert torch.equal(ws[0], ws[1])


@pytest.mark.parametrize("page", [32, 128, 256])
def test_page_sizes(page):
    """Paged caches with pages of 32, 128 and 256 tokens (a tile never straddles a page)."""
    wl = WORKLOADS[4].with_(name=f"paged-p{page}", B=3, n_max=512, len_lo=1, len_hi=512, page_size=page)
    inp = make_inputs(wl, lens=np.array([512, 100, 33]))
    got = run_gpu(inp, num_splits=7)
    all_finite(got, inp)
    compare(inp, got, oracle.decode(inp))


@pytest.mark.parametrize("cfg", [2, 5])
def test_padded_row_strides(cfg):
    """Split caches whose rows and sequences are padded in memory (token stride 512 + 64 latent
    elements, rope rows of 72, scales with a padded sequence stride): the strides come from the
    cache descriptor, not from the widths."""
    wl = WORKLOADS[cfg].with_(name=f"padded-{cfg}", B=3, n_max=160, len_lo=1, len_hi=160)
    inp = make_inputs(wl, lens=np.array([160, 45, 0]))
    print(f"[gpu] padded strides {wl.name}", flush=True)
    dev = to_device(inp)
    B, N = wl.B, wl.n_max
    lat = torch.zeros((B, N + 3, wl.d_c + 64), dtype=dev["latent"].dtype, device="cuda")
    lat[:, :N, :wl.d_c] = dev["latent"]
    rope = torch.zeros((B, N + 5, wl.d_R + 8), dtype=dev["rope"].dtype, device="cuda")
    rope[:, :N, :wl.d_R] = dev["rope"]
    scale = None
    if dev["scale"] is not None:
        scale = torch.ones((B, N + 16), dtype=torch.float32, device="cuda")
        scale[:, :N] = dev["scale"]
        scale = scale[:, :N]
    cache = ops.Cache.split(lat[:, :N, :wl.d_c], rope[:, :N, :wl.d_R], scale)
    q_abs = ops.mla_absorb_q(dev["q_C"], dev["W_UK"])
    o_lat, lse = ops.mla_decode_attn(q_abs, dev["q_R"], cache, dev["lens"], N, d_h=wl.d_h, num_splits=5)
    o = ops.mla_uv_out(o_lat, dev["W_UV"])
    torch.cuda.synchronize()
    got = {"q_abs": q_abs.float().cpu().numpy().astype(np.float64), "o_lat": o_lat.cpu().numpy().astype(np.float64),
           "lse": lse.cpu().numpy().astype(np.float64), "o": o.cpu().numpy().astype(np.float64)}
    compare(inp, got, oracle.decode(inp))


@pytest.mark.parametrize("H,splits", [(128, 100), (128, 0), (128, 129), (128, 1000), (64, 0), (32, 0)])
def test_large_batch_kernel_variants(H, splits):
    """Batches past the small-batch switch (more than 1024 tiles of 32 tokens) take the
    large-batch kernel: 128 heads in one workgroup (4 waves) with more than 128 splits (129 and
    1000 requested: more splits than tiles leave workgroups idle), in two head groups when there
    are at most 128, and the 64- and 32-head variants.  Sampled comparison."""
    B, n_max = 40, 1100
    wl = WORKLOADS[3].with_(name=f"large-h{H}-s{splits}", B=B, H=H, n_max=n_max, len_lo=1, len_hi=n_max)
    rng = np.random.default_rng(11)
    lens = rng.integers(1, n_max + 1, size=B)
    lens[:4] = [n_max, 0, 1, 33]
    inp = make_inputs(wl, lens=lens)
    got = run_gpu(inp, num_splits=splits)
    all_finite(got, inp)
    pairs = _sample_pairs(inp)
    ref = oracle.decode(inp, pairs=pairs)
    compare(inp, got, ref, pairs=pairs)


def test_rising_scores_force_rescales_large_batch():
    """As test_rising_scores_force_rescales, on a batch past the small-batch switch (the
    large-batch kernel, 128 heads per workgroup): the rope keys grow with the token index, so
    every segment's running maximum keeps rising and its accumulator is rescaled many times.
    Sampled comparison."""
    B, n_max = 40, 1100
    wl = WORKLOADS[3].with_(name="large-rising", B=B, n_max=n_max, len_lo=1, len_hi=n_max, layout="split")
    rng = np.random.default_rng(12)
    lens = rng.integers(600, n_max + 1, size=B)
    lens[:3] = [n_max, 1, 65]
    inp = make_inputs(wl, lens=lens)
    rope = bf16_bits_to_f32(inp.rope).reshape(B, n_max, 64)
    grow = (1.0 + np.arange(n_max, dtype=np.float32) / 32.0)[None, :, None]
    inp.rope = f32_to_bf16_bits(rope * grow).reshape(inp.rope.shape)
    got = run_gpu(inp)
    all_finite(got, inp)
    pairs = _sample_pairs(inp)
    ref = oracle.decode(inp, pairs=pairs)
    nonempty = [(b, h) for b, h in pairs if lens[b] > 64]
    assert float(np.median([ref["lse"][b, h] for b, h in nonempty])) > 25.0
    compare(inp, got, ref, pairs=pairs)


def test_max_batch_sampled():
    """The library's batch limit (2048 sequences) with short ragged lengths, empty sequences among
    them: the large-batch kernel's tile prefix and the combine at their widest.  Sampled pairs."""
    B, n_max = 2048, 40
    wl = WORKLOADS[2].with_(name="max-batch", B=B, n_max=n_max, len_lo=0, len_hi=n_max)
    rng = np.random.default_rng(21)
    lens = rng.integers(0, n_max + 1, size=B)
    lens[:3] = [n_max, 0, 1]
    inp = make_inputs(wl, lens=lens)
    got = run_gpu(inp)
    all_finite(got, inp)
    pairs = _sample_pairs(inp, n_b=10)
    ref = oracle.decode(inp, pairs=pairs)
    compare(inp, got, ref, pairs=pairs)


def test_long_sequence_sampled():
    """One sequence of 131072 tokens: past the small-batch switch at one sequence (the large-batch
    kernel over 256 splits), through the separate combine and through the decode step's fused
    combine + W_UV (256 segments per head).  Sampled heads."""
    n = 131072
    wl = WORKLOADS[2].with_(name="long-131k", B=1, n_max=n, len_lo=n, len_hi=n)
    inp = make_inputs(wl)
    pairs = [(0, 0), (0, 77), (0, 127)]
    ref = oracle.decode(inp, pairs=pairs)
    for got in (run_gpu(inp), run_step(inp)):
        all_finite(got, inp)
        compare(inp, got, ref, pairs=pairs)
