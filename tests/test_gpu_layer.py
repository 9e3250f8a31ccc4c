"""GPU parity of the reversible layer (dense maps on the matrix cores around
the LSH attention) against the fp64 oracle of oracle/layer.py.

Every step is checked with the GPU's own inputs to that step, so that the
bucket decisions are compared on identical qk values:
  - qk, v projections: within one bf16 rounding step of the oracle's value
    (the GPU sums in fp32 before rounding to bf16, the oracle in fp64);
  - bucket ids on the GPU's qk: bit-exact; per-head outputs: 2e-2;
  - output map + residual on the GPU's per-head outputs: 1e-4;
  - FFN + residual on the GPU's y1: 2e-3 (a hidden activation near a bf16
    rounding midpoint may round the other way: one bf16 step, about 2^-8 of
    the value, times one weight);
  - the one-call layer equals the composition of its ABI calls bit for bit;
  - FFN chunking does not change a single bit;
  - the inverse returns x2 within one fp32 rounding, and x1 within one
    rounding wherever bf16(x2) comes back bit for bit (else within 1e-2).
"""
import sys

import numpy as np
import pytest
import torch

from lsh_sparse_attention_hash_amd import synth
from oracle import layer as olayer
from oracle import oracle

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lsh_sparse_attention_hash_amd import binding
    return binding


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


CASES = {
    "small": synth.LayerWorkload("l_small", 2, 1024, 128, 256, 16, 2, True, True, 0, 61),
    "ragged": synth.LayerWorkload("l_ragged", 1, 192, 64, 64, 4, 1, False, True, 100, 62),
    "wide": synth.LayerWorkload("l_wide", 1, 2048, 512, 2048, 64, 4, True, True, 1000, 63),
}


class Run:
    """One GPU forward of the layer plus the same steps through the
    individual calls (qk, v, the LSH attention, y_att)."""

    def __init__(self, B, w):
        self.w = w
        self.inp = synth.make_layer_inputs(w)
        self.lc = B.make_layer_config(w)
        self.wd = B.layer_weights_to_device(self.inp)
        self.x1 = torch.from_numpy(self.inp["x1"]).cuda()
        self.x2 = torch.from_numpy(self.inp["x2"]).cuda()
        self.layer = B.Layer(self.lc, self.wd)
        self.y1 = torch.empty_like(self.x1)
        self.y2 = torch.empty_like(self.x2)
        self.layer.forward(self.x1, self.x2, self.y1, self.y2)
        # the same steps, call by call
        H, L, b = w.heads, w.seq_len, w.batch
        self.qk = torch.empty((b, H, L, 64), dtype=torch.bfloat16, device="cuda")
        self.v = torch.empty_like(self.qk)
        B.lsh_project_qkv(self.lc, self.x2, self.wd["w_qk"], self.wd["w_v"], self.qk, self.v)
        self.att = B.Forward(B.attention_config(self.lc))
        self.att.run(self.qk, self.v, self.wd["rot"] if w.n_buckets > 1 else None)
        self.y1c = torch.empty_like(self.x1)
        B.lsh_project_out(self.lc, self.att.y, self.wd["w_o"], self.x1, 0, self.y1c)
        self.ffn_ws = torch.empty(max(16, B.lsh_ffn_workspace_bytes(self.lc)), dtype=torch.uint8,
                                  device="cuda")
        self.y2c = torch.empty_like(self.x2)
        B.lsh_ffn(self.lc, self.y1c, self.wd["w_1"], self.wd["b_1"], self.wd["w_2"],
                  self.wd["b_2"], self.x2, 0, self.y2c, self.ffn_ws)
        torch.cuda.synchronize()

    def weights64(self):
        f = {k: synth.to_f64(self.inp[k], "bf16") for k in ("w_qk", "w_v", "w_o", "rot", "w_1",
                                                             "w_2")}
        f.update({k: self.inp[k].astype(np.float64) for k in ("b_1", "b_2")})
        return f


@pytest.fixture(scope="module")
def runs(B):
    return {}


def get_run(B, runs, name):
    if name not in runs:
        say(f"[layer] {CASES[name]}")
        runs[name] = Run(B, CASES[name])
    return runs[name]


@pytest.mark.parametrize("name", sorted(CASES))
def test_layer_is_the_composition_of_its_calls(B, runs, name):
    r = get_run(B, runs, name)
    assert torch.equal(r.y1, r.y1c)
    assert torch.equal(r.y2, r.y2c)


@pytest.mark.parametrize("name", sorted(CASES))
def test_projection_qkv(B, runs, name):
    r = get_run(B, runs, name)
    w = r.weights64()
    x = r.inp["x2"].astype(np.float64)
    qk_ref, v_ref = olayer.project_qkv(x, w["w_qk"], w["w_v"])
    xb = np.abs(olayer.bf16_round(x))
    K = r.w.d_model
    for got, ref, wm, what in ((host(r.qk), qk_ref, w["w_qk"], "qk"),
                               (host(r.v), v_ref, w["w_v"], "v")):
        # the GPU rounds its fp32 sum to bf16, the oracle its fp64 sum: apart
        # by at most one bf16 step plus the fp32 accumulation error
        # K * 2^-23 * sum_k |x_k w_k| (which dominates near cancellations)
        acc = olayer.split_heads(K * 2.0 ** -23 * (xb @ np.abs(wm).T), r.w.heads)
        step = np.maximum(np.ldexp(1.0, np.frexp(np.abs(ref))[1] - 8),
                          np.ldexp(1.0, np.frexp(np.abs(got))[1] - 8))
        bad = np.abs(got - ref) > step + acc
        assert not bad.any(), f"{what}: {int(bad.sum())} values beyond one bf16 step + fp32 error"
        frac = float((got != ref).mean())
        assert frac < 0.01, f"{what}: {frac:.3%} of values differ from the oracle's rounding"
        say(f"[layer] {name} {what}: {frac:.4%} of values one bf16 step away")


@pytest.mark.parametrize("name", sorted(CASES))
def test_attention_on_the_gpu_projections(B, runs, name):
    r = get_run(B, runs, name)
    w = r.weights64()
    qk, v = host(r.qk), host(r.v)
    ref = oracle.forward(qk, v, w["rot"] if r.w.n_buckets > 1 else np.zeros((r.w.heads, r.w.n_rounds, 0, 64)),
                         r.w.n_buckets, r.w.n_rounds, 64, r.w.causal, r.w.self_mask)
    assert np.array_equal(r.att.buckets.cpu().numpy(), ref["buckets"])
    assert np.abs(host(r.att.y) - ref["y"]).max() <= 2e-2


@pytest.mark.parametrize("name", sorted(CASES))
def test_output_map_and_ffn_on_gpu_inputs(B, runs, name):
    r = get_run(B, runs, name)
    w = r.weights64()
    y1_ref = r.inp["x1"] + olayer.project_out(host(r.att.y), w["w_o"])
    e1 = np.abs(host(r.y1) - y1_ref).max()
    assert e1 <= 1e-4, f"y1 err {e1}"
    y2_ref = r.inp["x2"] + olayer.ffn(host(r.y1), w, r.w.ffn_chunk or None)
    e2 = np.abs(host(r.y2) - y2_ref).max()
    assert e2 <= 2e-3, f"y2 err {e2}"
    say(f"[layer] {name}: y1 err {e1:.3g}, y2 err {e2:.3g}")


def test_ffn_chunking_changes_no_bit(B, runs):
    r = get_run(B, runs, "wide")
    outs = []
    for chunk in (0, 1000, 64, 2048):
        lc = B.make_layer_config(r.w)
        lc.ffn_chunk = chunk
        ws = torch.empty(max(16, B.lsh_ffn_workspace_bytes(lc)), dtype=torch.uint8, device="cuda")
        out = torch.empty_like(r.x2)
        B.lsh_ffn(lc, r.y1, r.wd["w_1"], r.wd["b_1"], r.wd["w_2"], r.wd["b_2"], r.x2, 0, out, ws)
        outs.append(out)
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


@pytest.mark.parametrize("name", sorted(CASES))
def test_inverse_reconstructs_the_inputs(B, runs, name):
    r = get_run(B, runs, name)
    x1 = torch.empty_like(r.x1)
    x2 = torch.empty_like(r.x2)
    r.layer.inverse(r.y1, r.y2, x1, x2)
    torch.cuda.synchronize()
    # x2 = fl(fl(x2 + g) - g): within one rounding of |y2|
    e2 = (x2 - r.x2).abs()
    assert bool((e2 <= 2.0 ** -23 * (r.y2.abs() + 1e-30) * 2).all()), f"x2 err {float(e2.max())}"
    # F sees bf16(x2): where the rounded values all come back, F is recomputed
    # bit for bit and x1 = fl(fl(x1 + f) - f) is within one rounding of |y1|;
    # an element of x2 within an fp32 rounding of a bf16 midpoint may round
    # the other way and move F (and so x1) by about one bf16 step of qk / v
    flips = int((olayer.bf16_round(host(x2)) != olayer.bf16_round(r.inp["x2"])).sum())
    e1 = (x1 - r.x1).abs()
    if flips == 0:
        assert bool((e1 <= 2.0 ** -23 * (r.y1.abs() + 1e-30) * 2).all()), f"x1 err {float(e1.max())}"
    else:
        assert float(e1.max()) <= 1e-2, f"x1 err {float(e1.max())} with {flips} bf16 flips in x2"
    say(f"[layer] {name}: inverse x1 err {float(e1.max()):.3g} ({flips} bf16 flips of x2), "
        f"x2 err {float(e2.max()):.3g}")


def test_layer_long_full_size_sampled(B):
    """The headline attention shape inside one layer (8 x 64 features,
    65,536 tokens, d_ff 2,048, FFN in chunks of 32,768): the one-call layer
    equals its calls, buckets and rows are sampled against the oracle."""
    w = synth.LAYER_WORKLOADS["layer_long"]
    r = Run(B, w)
    say(f"[layer-full] {w}")
    assert torch.equal(r.y1, r.y1c) and torch.equal(r.y2, r.y2c)
    wf = r.weights64()
    g = np.random.default_rng(64)
    qk = host(r.qk)
    idx = g.integers(0, w.heads * w.n_rounds * w.seq_len, 3000)
    assert np.array_equal(r.att.buckets.cpu().numpy().ravel()[idx],
                          oracle.hash_rows(qk, wf["rot"], w.n_buckets, w.n_rounds, idx))
    rows = g.integers(0, w.seq_len, 400)
    x2 = r.inp["x2"][0]
    xb = olayer.bf16_round(x2[rows].astype(np.float64))
    q_ref = olayer.bf16_round(oracle.linear(xb, wf["w_qk"]))
    q_got = host(r.qk)[0].transpose(1, 0, 2).reshape(w.seq_len, -1)[rows]
    assert np.abs(q_got - q_ref).max() <= np.abs(q_ref).max() * 2.0 ** -7
    y_att = host(r.att.y)[0].transpose(1, 0, 2).reshape(w.seq_len, -1)
    y1_ref = r.inp["x1"][0][rows] + oracle.linear(olayer.bf16_round(y_att[rows]), wf["w_o"])
    assert np.abs(host(r.y1)[0][rows] - y1_ref).max() <= 1e-4
    y2_ref = x2[rows] + olayer.ffn(host(r.y1)[:, rows], wf)[0]
    assert np.abs(host(r.y2)[0][rows] - y2_ref).max() <= 2e-3
    say("[layer-full] layer_long: composition exact; 3000 buckets, 400 rows of qk, y1, y2 within tolerance")
