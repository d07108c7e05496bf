"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle on
the same seeded inputs. Sizes the oracle finishes in seconds run the whole
layer element by element; the full-size workloads compare routing and
dispatch on every token and the outputs of sampled tokens."""
import sys

import numpy as np
import pytest
import torch

from oracle import moe_oracle as mo
from top_routing_expert_02_amd import synth
from top_routing_expert_02_amd.synth import WORKLOADS

from tests import parity as P

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from top_routing_expert_02_amd import moe
    moe.lib()  # fails loudly when libmoe.so is missing
    torch.manual_seed(0)
    yield


def moe():
    return P.moe_mod()


def cap(w):
    if w.dropless:
        return w.T  # a token holds an expert at most once, so count_e <= T
    C = moe().capacity(w.T, w.k, w.E, w.c)
    assert C == mo.capacity(w.T, w.k, w.E, w.c)
    return C


# Workloads at sizes the oracle finishes in seconds: same recipes, several
# GEMM tiles per expert, ragged token counts (not multiples of 64).
MINI = {
    "tiny_f32": WORKLOADS["tiny_f32"],
    "f32_mid": WORKLOADS["tiny_f32"].scaled(name="f32_mid", T=301, d=48, d_ff=80, E=4, k=2,
                                            act="gelu_tanh", renormalize=True, c=1.1),
    "small_bf16_mini": WORKLOADS["small_bf16"].scaled(name="small_bf16_mini", T=2000, d=256, d_ff=512),
    "mid_bf16_mini": WORKLOADS["mid_bf16"].scaled(name="mid_bf16_mini", T=777, d=512, d_ff=1024),
    "skewed_bf16_mini": WORKLOADS["skewed_bf16"].scaled(name="skewed_bf16_mini", T=1500, d=256, d_ff=256),
    "large_e_bf16_mini": WORKLOADS["large_e_bf16"].scaled(name="large_e_bf16_mini", T=600, d=256, d_ff=192),
    "max_e_k_bf16": WORKLOADS["large_e_bf16"].scaled(name="max_e_k_bf16", T=300, d=64, d_ff=64, E=1024, k=16),
    # an expert count that does not divide 256 (the per-expert histogram sums
    # take the strided path)
    "e12_bf16": WORKLOADS["skewed_bf16"].scaled(name="e12_bf16", T=900, d=64, d_ff=128, E=12, k=3),
    # capacity 400: at most 512 rows per expert, so the short-tile kernel
    # (192-, 128- and 64-row tiles) runs, with several M tiles per expert
    "mid_cap400_bf16": WORKLOADS["mid_bf16"].scaled(name="mid_cap400_bf16", T=1280, d=512, d_ff=1024),
    "skewed_cap400_bf16": WORKLOADS["skewed_bf16"].scaled(name="skewed_cap400_bf16", T=6400, d=256,
                                                          d_ff=256),
    # K stage counts one past a multiple of the weight ring (3 buffers for
    # 192-row tiles, 4 for 64-row tiles) in the short-tile kernel: the K
    # loop's last refill then loads a stage past the last one into weight
    # slot 1, and the epilogue's LDS staging must take slot 2 (d = 320, 448,
    # 832: 5, 7, 13 stages; d_ff = 576, 256, 320: 9, 4, 5 stages)
    "ring_wrap_decode_bf16": WORKLOADS["small_bf16"].scaled(name="ring_wrap_decode_bf16", T=40, d=320,
                                                            d_ff=576, dropless=True),
    "ring_wrap_c1_bf16": WORKLOADS["small_bf16"].scaled(name="ring_wrap_c1_bf16", T=900, d=448, d_ff=256,
                                                        c=1.0),
    "ring_wrap_k13_bf16": WORKLOADS["small_bf16"].scaled(name="ring_wrap_k13_bf16", T=1100, d=832,
                                                         d_ff=320, c=1.0),
    # more than 16384 tokens with at most 8 experts (over a thousand route
    # blocks, a ragged last one; with 5 experts the logits tile has columns
    # past E)
    "many_tokens_bf16": WORKLOADS["small_bf16"].scaled(name="many_tokens_bf16", T=16500, d=256, d_ff=256),
    "many_tokens_e5_bf16": WORKLOADS["small_bf16"].scaled(name="many_tokens_e5_bf16", T=16421, d=512,
                                                         d_ff=128, E=5, k=2),
    # 33 tiles x 1024 experts: above the single-launch scan limit, so the
    # separate scan kernel runs
    "scan_split_bf16": WORKLOADS["large_e_bf16"].scaled(name="scan_split_bf16", T=2100, d=64, d_ff=64,
                                                        E=1024, k=4),
}


@pytest.mark.parametrize("name", list(MINI))
def test_layer_parity_mini(name):
    w = MINI[name]
    say(f"[gpu] layer parity {name} T={w.T} d={w.d} d_ff={w.d_ff} E={w.E} k={w.k}")
    inp = synth.make_inputs(w, "cuda", seed=0)
    P.full_parity(w, inp, cap(w), report=say)


@pytest.mark.parametrize("T", [1, 2, 17, 64, 65])
@pytest.mark.parametrize("base", ["skewed_bf16", "mid_bf16"])
def test_dropless_decode_sizes(base, T):
    """Dropless (C = T) at decode batch sizes: every assignment is kept, the
    hottest expert may take every token."""
    w = WORKLOADS[base].scaled(name=f"dropless_{base}_T{T}", T=T, d=256, d_ff=512, dropless=True)
    say(f"[gpu] dropless decode {w.name}")
    inp = synth.make_inputs(w, "cuda", seed=1)
    _, _, o, stats = P.full_parity(w, inp, cap(w), report=say)
    assert stats["dropped"] == 0 and o["rows"] == T * w.k


# Priority order and overflow re-routing (the general capacity rule), on the
# mini workloads: drops are frequent in the skewed and capped ones.
REROUTE = {
    "skewed_rank": MINI["skewed_bf16_mini"].scaled(name="skewed_rank", priority="rank"),
    "skewed_reroute1": MINI["skewed_bf16_mini"].scaled(name="skewed_reroute1", reroute=1),
    "skewed_rank_reroute2": MINI["skewed_bf16_mini"].scaled(name="skewed_rank_reroute2",
                                                            priority="rank", reroute=2),
    "skewed_reroute3": MINI["skewed_bf16_mini"].scaled(name="skewed_reroute3", reroute=3),
    "small_capped_rank": MINI["small_bf16_mini"].scaled(name="small_capped_rank", c=0.8,
                                                        priority="rank"),
    "small_capped_reroute2": MINI["small_bf16_mini"].scaled(name="small_capped_reroute2", c=0.8,
                                                            reroute=2),
    "large_e_reroute1": MINI["large_e_bf16_mini"].scaled(name="large_e_reroute1", reroute=1),
    "tiny_f32_reroute1": MINI["tiny_f32"].scaled(name="tiny_f32_reroute1", reroute=1),
    "f32_mid_rank_reroute1": MINI["f32_mid"].scaled(name="f32_mid_rank_reroute1", c=0.7,
                                                    priority="rank", reroute=1),
    "e12_rank_reroute4": MINI["e12_bf16"].scaled(name="e12_rank_reroute4", priority="rank",
                                                 reroute=4),
}


@pytest.mark.parametrize("name", list(REROUTE))
def test_layer_parity_reroute(name):
    w = REROUTE[name]
    say(f"[gpu] reroute parity {name} priority={w.priority} rounds={w.reroute}")
    inp = synth.make_inputs(w, "cuda", seed=0)
    P.full_parity(w, inp, cap(w), report=say)


def test_reroute_golden_on_gpu():
    """The hand-worked re-routing and priority examples on the page's routing,
    through moe_dispatch_reroute with the candidate lists given."""
    import json
    import os
    cases = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                        "reroute_examples.json")))["cases"]
    m = moe()
    dev = "cuda"
    for c in cases:
        cand = torch.tensor(c["cand"], dtype=torch.int32, device=dev)
        T, n = cand.shape
        k, E = c["k"], c["E"]
        cg = (torch.arange(T * n, dtype=torch.float32, device=dev).reshape(T, n) + 1) / 64
        cfg = m.config(T, 64, 64, E, k, c["C"], True, "f32", "relu", priority=c["priority"],
                       reroute=c["rounds"])
        assert m.candidates(cfg) == n
        i32 = dict(dtype=torch.int32, device=dev)
        counts = torch.full((E,), -7, **i32)
        offs = torch.full((E + 1,), -7, **i32)
        slot = torch.full((T, k), -7, **i32)
        row_of = torch.full((T, k), -7, **i32)
        row_token = torch.full((m.max_rows(cfg),), -7, **i32)
        served = torch.full((T, k), -7, **i32)
        gates = torch.full((T, k), -7.0, dtype=torch.float32, device=dev)
        m.dispatch_reroute(cfg, None, cand, cg, counts, offs, slot, row_of, row_token, served, gates)
        torch.cuda.synchronize()
        rows = c["expert_offsets"][-1]
        assert counts.tolist() == c["expert_counts"], c["name"]
        assert offs.tolist() == c["expert_offsets"], c["name"]
        assert slot.tolist() == c["slot"], c["name"]
        assert row_of.tolist() == c["row_of"], c["name"]
        assert row_token[:rows].tolist() == c["row_token"], c["name"]
        assert served.tolist() == c["served_ids"], c["name"]
        col = torch.tensor(c["served_col"], dtype=torch.int64, device=dev)
        want = torch.where(col >= 0, torch.gather(cg, 1, col.clamp(min=0)), torch.zeros_like(gates))
        assert torch.equal(gates, want), c["name"]


def test_dispatch_entry_point_rank_priority():
    """moe_dispatch under rank-major priority equals the oracle's rule."""
    w = MINI["skewed_bf16_mini"].scaled(name="dispatch_rank", priority="rank")
    inp = synth.make_inputs(w, "cuda", seed=3)
    C = cap(w)
    m = moe()
    cfg = P.make_cfg(w, C)
    dev = "cuda"
    h = P.host_inputs(inp, w.dtype)
    ids = torch.from_numpy(mo.route(h["x"], h["W_r"], h["b_r"], w.k, w.renormalize)["topk_ids"]).to(dev)
    i32 = dict(dtype=torch.int32, device=dev)
    R = m.max_rows(cfg)
    out = {"expert_counts": torch.empty(w.E, **i32), "expert_offsets": torch.empty(w.E + 1, **i32),
           "slot": torch.empty((w.T, w.k), **i32), "row_of": torch.empty((w.T, w.k), **i32),
           "row_token": torch.full((R,), -1, **i32)}
    x_perm = torch.empty((R, w.d), dtype=w.torch_dtype, device=dev)
    m.dispatch(cfg, inp["x"], ids, out["expert_counts"], out["expert_offsets"], out["slot"],
               out["row_of"], out["row_token"], x_perm)
    torch.cuda.synchronize()
    o = mo.dispatch_rerouted(ids.cpu().numpy(), w.k, w.E, C, "rank", 0)
    P.check_dispatch({k: v.cpu().numpy() for k, v in out.items()}, o)
    rows = o["rows"]
    np.testing.assert_array_equal(synth.to_numpy_bits(x_perm[:rows]),
                                  synth.to_numpy_bits(inp["x"])[o["row_token"]])


def test_layer_parity_uncapped_hot_expert():
    """All tokens prefer one expert; with C >= T nothing drops and that
    expert's group spans several 256-row tiles."""
    w = WORKLOADS["small_bf16"].scaled(name="hot_uncapped", T=1100, d=128, d_ff=256, E=8, k=2)
    inp = synth.make_inputs(w, "cuda", seed=1)
    inp["b_r"][3] += 40.0
    say("[gpu] hot expert, C >= T")
    _, g, o, st = P.full_parity(w, inp, w.T, report=say)
    assert g["expert_counts"][3] == w.T and st["dropped"] == 0


def test_layer_parity_hot_expert_capped():
    w = WORKLOADS["small_bf16"].scaled(name="hot_capped", T=700, d=128, d_ff=128, E=8, k=2, c=1.0)
    inp = synth.make_inputs(w, "cuda", seed=2)
    inp["b_r"][5] += 40.0
    say("[gpu] hot expert, capped")
    _, g, o, st = P.full_parity(w, inp, cap(w), report=say)
    assert st["dropped"] == w.T - cap(w)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_token(dtype):
    base = WORKLOADS["tiny_f32"] if dtype == "f32" else WORKLOADS["small_bf16"]
    w = base.scaled(name=f"one_token_{dtype}", T=1, d=64, d_ff=128, E=4, k=2, renormalize=True)
    inp = synth.make_inputs(w, "cuda", seed=3)
    say(f"[gpu] T=1 {dtype}")
    P.full_parity(w, inp, cap(w), report=say)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_expert(dtype):
    base = WORKLOADS["tiny_f32"] if dtype == "f32" else WORKLOADS["small_bf16"]
    w = base.scaled(name=f"one_expert_{dtype}", T=130, d=64, d_ff=128, E=1, k=1, c=1.0)
    inp = synth.make_inputs(w, "cuda", seed=4)
    say(f"[gpu] E=1 {dtype}")
    y, g, o, st = P.full_parity(w, inp, cap(w), report=say)
    np.testing.assert_array_equal(g["topk_gates"], 1.0)  # softmax of one logit


def test_k_equals_E():
    w = WORKLOADS["small_bf16"].scaled(name="k_eq_E", T=200, d=64, d_ff=64, E=4, k=4, c=1.0)
    inp = synth.make_inputs(w, "cuda", seed=5)
    say("[gpu] k = E")
    y, g, o, st = P.full_parity(w, inp, cap(w), report=say)
    assert st["dropped"] == 0


def test_empty_batch_is_noop():
    w = WORKLOADS["small_bf16"].scaled(name="empty", T=0, d=64, d_ff=64)
    m = moe()
    cfg = P.make_cfg(w, 1)
    x = torch.empty((0, w.d), dtype=torch.bfloat16, device="cuda")
    inp = synth.make_inputs(w.scaled(name="empty_w", T=1), "cuda")
    y = torch.empty((0, w.d), dtype=torch.bfloat16, device="cuda")
    m.layer_forward(cfg, x, inp["W_r"], inp["b_r"], inp["W1"], inp["b1"], inp["W2"], inp["b2"], y)
    torch.cuda.synchronize()


def test_exact_ties_lowest_index():
    """Integer-valued inputs make the fp32 and fp64 logits exact, so ties are
    real ties on both sides and must go to the lower index on both."""
    w = WORKLOADS["small_bf16"].scaled(name="ties", T=500, d=64, d_ff=64, E=8, k=3,
                                       router_bias="zero", ffn_bias_var=0.0)
    inp = synth.make_inputs(w, "cuda", seed=6)
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    inp["x"] = torch.randint(-2, 3, (w.T, w.d), device="cuda", generator=g).to(torch.bfloat16)
    inp["W_r"] = torch.randint(-1, 2, (w.E, w.d), device="cuda", generator=g).to(torch.bfloat16)
    inp["W_r"][1] = inp["W_r"][0]      # experts 0 and 1 always tie
    inp["W_r"][6] = inp["W_r"][2]      # experts 2 and 6 always tie
    y, gi, cfg = P.gpu_layer(w, inp, cap(w))
    h = P.host_inputs(inp, w.dtype)
    o = mo.route(h["x"], h["W_r"], h["b_r"], w.k, w.renormalize)
    n_ties = int(o["near_tie"].sum())
    say(f"[gpu] exact ties: {n_ties} tokens with tied decisions")
    assert n_ties > 50
    np.testing.assert_array_equal(gi["topk_ids"], o["topk_ids"])


def test_page_drop_example_on_gpu():
    """The page's T=8, E=2 routing [1,1,1,1,1,1,2,2] (0-based [0*6, 1*2]) as a
    layer input: at C=4 tokens 4 and 5 overflow and output zero."""
    import json, os
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "drop_rule_example.json")))
    w = WORKLOADS["tiny_f32"]
    inp = synth.make_inputs(w, "cuda", seed=7)
    x = inp["x"]
    x[:, 0] = torch.tensor([1, 1, 1, 1, 1, 1, -1, -1], dtype=torch.float32, device="cuda") * 3.0
    inp["W_r"].zero_()
    inp["W_r"][0, 0] = 1.0
    inp["W_r"][1, 0] = -1.0
    for key in ("C4", "C6"):
        exp = gold[key]
        y, g, o, st = P.full_parity(w, inp, exp["C"], report=say)
        assert g["topk_ids"][:, 0].tolist() == [0] * 6 + [1] * 2
        assert g["expert_counts"].tolist() == exp["expert_counts"]
        assert g["expert_offsets"].tolist() == exp["expert_offsets"]
        assert g["row_token"][:sum(exp["kept_per_expert"])].tolist() == exp["row_token"]
        yh = y.cpu().numpy()
        for t in exp["overflow_tokens"]:
            assert np.all(yh[t] == 0.0)


def test_deterministic_reruns():
    w = MINI["skewed_bf16_mini"]
    inp = synth.make_inputs(w, "cuda", seed=8)
    C = cap(w)
    y1, g1, _ = P.gpu_layer(w, inp, C)
    y2, g2, _ = P.gpu_layer(w, inp, C)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    for k in g1:
        np.testing.assert_array_equal(g1[k], g2[k], err_msg=k)


# ------------------------------------------------------------------ stage entry points

@pytest.mark.parametrize("name", ["f32_mid", "small_bf16_mini", "skewed_bf16_mini"])
def test_stages_separately(name):
    """Each C-ABI stage against the oracle, fed with the oracle's own inputs."""
    w = MINI[name]
    m = moe()
    inp = synth.make_inputs(w, "cuda", seed=9)
    C = cap(w)
    cfg = P.make_cfg(w, C)
    R = m.max_rows(cfg)
    ws = m.alloc_workspace(cfg, "cuda")
    h = P.host_inputs(inp, w.dtype)
    o = mo.layer_forward(h["x"], h["W_r"], h["b_r"], h["W1"], h["b1"], h["W2"], h["b2"], k=w.k,
                         C=C, renormalize=w.renormalize, act=w.act)
    dev = "cuda"
    say(f"[gpu] stages {name}")
    # route
    ids = torch.empty((w.T, w.k), dtype=torch.int32, device=dev)
    gates = torch.empty((w.T, w.k), dtype=torch.float32, device=dev)
    psum = torch.empty(w.E, dtype=torch.float32, device=dev)
    logits = torch.empty((w.T, w.E), dtype=torch.float32, device=dev)
    m.route(cfg, inp["x"], inp["W_r"], inp["b_r"], ids, gates, psum, logits, ws=ws)
    torch.cuda.synchronize()
    P.check_routing(o, ids.cpu().numpy())
    P.check_gates(o, ids.cpu().numpy(), gates.cpu().numpy(), w.renormalize)
    np.testing.assert_allclose(logits.cpu().numpy(), o["logits"], rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(psum.cpu().numpy(), o["prob_sum"], rtol=1e-5, atol=1e-4)
    # dispatch, from the oracle's ids
    ids_o = torch.from_numpy(o["topk_ids"]).to(dev)
    counts = torch.empty(w.E, dtype=torch.int32, device=dev)
    offs = torch.empty(w.E + 1, dtype=torch.int32, device=dev)
    slot = torch.empty((w.T, w.k), dtype=torch.int32, device=dev)
    row_of = torch.empty((w.T, w.k), dtype=torch.int32, device=dev)
    row_token = torch.full((R,), -1, dtype=torch.int32, device=dev)
    x_perm = torch.zeros((R, w.d), dtype=w.torch_dtype, device=dev)
    m.dispatch(cfg, inp["x"], ids_o, counts, offs, slot, row_of, row_token, x_perm, ws=ws)
    torch.cuda.synchronize()
    P.check_dispatch({"expert_counts": counts.cpu().numpy(), "expert_offsets": offs.cpu().numpy(),
                      "slot": slot.cpu().numpy(), "row_of": row_of.cpu().numpy(),
                      "row_token": row_token.cpu().numpy()}, o)
    rows = o["rows"]
    xb = synth.to_numpy_bits(inp["x"])
    np.testing.assert_array_equal(synth.to_numpy_bits(x_perm)[:rows], xb[o["row_token"]])
    # expert FFN on the oracle's layout
    hbuf = torch.zeros((R, w.d_ff), dtype=w.torch_dtype, device=dev)
    yperm = torch.zeros((R, w.d), dtype=w.torch_dtype, device=dev)
    m.expert_ffn(cfg, x_perm, offs, inp["W1"], inp["b1"], inp["W2"], inp["b2"], hbuf, yperm, ws=ws)
    torch.cuda.synchronize()
    P.compare_outputs(P.host64(hbuf, w.dtype)[:rows], o["h"], w.dtype)
    P.compare_outputs(P.host64(yperm, w.dtype)[:rows], o["y_perm"], w.dtype)
    # combine, from the oracle's rows (rounded to the layer's dtype as the ABI
    # takes them) and gates (rounded to fp32)
    yp = torch.from_numpy(o["y_perm"].astype(np.float32)).to(dev).to(w.torch_dtype)
    if rows == 0:
        yp = torch.zeros((1, w.d), dtype=w.torch_dtype, device=dev)
    g32 = torch.from_numpy(o["topk_gates"].astype(np.float32)).to(dev)
    rof = torch.from_numpy(o["row_of"]).to(dev)
    y = torch.empty((w.T, w.d), dtype=w.torch_dtype, device=dev)
    m.combine(cfg, yp, rof, g32, y)
    torch.cuda.synchronize()
    P.compare_outputs(P.host64(y, w.dtype), o["y"], w.dtype)


# ------------------------------------------------------------------ full sizes

@pytest.mark.parametrize("name", ["small_bf16", "mid_bf16", "skewed_bf16", "large_e_bf16",
                                  "skewed_dropless_bf16", "decode_bf16", "skewed_reroute_bf16"])
def test_full_size_workload(name):
    """Full-size workload in the launch configuration the benchmark times:
    routing and dispatch on every token, x_perm on every row, the first
    GEMM's h on every kept row and the layer's y on every token against the
    oracle (its expert FFN batched expert by expert; under a minute on 16
    host cores for the largest layer)."""
    w = WORKLOADS[name]
    say(f"[gpu] full size {name}: generating inputs")
    inp = synth.make_inputs(w, "cuda", seed=0)
    C = cap(w)
    m = moe()
    cfg = P.make_cfg(w, C)
    R = m.max_rows(cfg)
    dev = "cuda"
    say(f"[gpu] full size {name}: layer forward (C={C})")
    info = P.info_tensors(w, R, dev)
    info["h"] = torch.empty((max(R, 1), w.d_ff), dtype=w.torch_dtype, device=dev)
    y = torch.full((w.T, w.d), float("nan"), dtype=w.torch_dtype, device=dev)
    ws = m.alloc_workspace(cfg, dev)
    m.layer_forward(cfg, inp["x"], inp["W_r"], inp["b_r"], inp["W1"], inp["b1"], inp["W2"],
                    inp["b2"], y, info=info, ws=ws)
    torch.cuda.synchronize()
    h_gpu = info.pop("h")
    g = {k: v.cpu().numpy() for k, v in info.items()}
    x64 = P.host64(inp["x"], w.dtype)
    o_route = mo.route(x64, P.host64(inp["W_r"], w.dtype), P.host64(inp["b_r"], "f32"),
                       P.n_cand(w), w.renormalize)
    stats = P.check_routing(o_route, g["topk_ids"])
    P.check_gates(o_route, g["topk_ids"], g["topk_gates"], w.renormalize, k=w.k)
    general = P.general_rule(w)
    if general:
        o_disp = mo.dispatch_rerouted(g["topk_ids"], w.k, w.E, C, w.priority, w.reroute)
        np.testing.assert_array_equal(g["served_ids"], o_disp["served_ids"])
        gates_ref = mo.served_gates(mo.candidate_gates(o_route["probs"], g["topk_ids"], w.k,
                                                       w.renormalize), o_disp["served_col"])
    else:
        o_disp = mo.dispatch(g["topk_ids"], w.E, C)
        gates_ref = mo.gates(o_route["probs"], g["topk_ids"], w.renormalize)
    P.check_dispatch(g, o_disp)
    # x_perm of the same call, through the dispatch entry point
    t = {k: torch.empty_like(torch.from_numpy(v)).to(dev) for k, v in g.items()
         if k in ("expert_counts", "expert_offsets", "slot", "row_of")}
    row_token = torch.full((R,), -1, dtype=torch.int32, device=dev)
    x_perm = torch.empty((R, w.d), dtype=w.torch_dtype, device=dev)
    if general:
        m.dispatch_reroute(cfg, inp["x"], torch.from_numpy(g["topk_ids"]).to(dev),
                           torch.from_numpy(g["topk_gates"]).to(dev), t["expert_counts"],
                           t["expert_offsets"], t["slot"], t["row_of"], row_token,
                           torch.empty((w.T, w.k), dtype=torch.int32, device=dev),
                           torch.empty((w.T, w.k), dtype=torch.float32, device=dev), x_perm, ws=ws)
    else:
        m.dispatch(cfg, inp["x"], torch.from_numpy(g["topk_ids"]).to(dev), t["expert_counts"],
                   t["expert_offsets"], t["slot"], t["row_of"], row_token, x_perm, ws=ws)
    torch.cuda.synchronize()
    rows = o_disp["rows"]
    xb = synth.to_numpy_bits(inp["x"])
    np.testing.assert_array_equal(synth.to_numpy_bits(x_perm[:rows]), xb[o_disp["row_token"]])
    del x_perm, ws
    # every token and every kept row
    offsets = o_disp["expert_offsets"]
    row_of = o_disp["row_of"]
    tokens = np.arange(w.T)
    need = np.unique(row_of[row_of >= 0])
    assert need.size == rows

    def expert_weights(e):
        return (P.host64(inp["W1"][e], w.dtype), P.host64(inp["b1"][e], "f32"),
                P.host64(inp["W2"][e], w.dtype), P.host64(inp["b2"][e], "f32"))

    say(f"[gpu] full size {name}: oracle on {need.size} rows of {rows}, {tokens.size} tokens")
    h_ref, Y_ref = P.oracle_rows(need, x64, o_disp["row_token"], offsets, expert_weights, w.act)
    h_sel = P.host64(h_gpu[torch.from_numpy(need).to(dev)], w.dtype)
    hs = P.compare_outputs(h_sel, h_ref, w.dtype)
    y_ref = P.oracle_tokens_y(tokens, need, Y_ref, row_of, gates_ref)
    stats.update(P.compare_outputs(P.host64(y[torch.from_numpy(tokens).to(dev)], w.dtype), y_ref,
                                   w.dtype))
    stats.update(rows=rows, dropped=int((~o_disp["kept"]).sum()), C=C, checked_rows=int(need.size),
                 checked_tokens=int(tokens.size), h_max_abs=hs["max_abs"], h_rel_l2=hs["rel_l2"])
    say(f"[gpu] full size {name}: {stats}")
    # fully dropped tokens output exact zeros
    dropped_tok = np.flatnonzero(~o_disp["kept"].any(axis=1))
    if dropped_tok.size:
        assert torch.all(y[torch.from_numpy(dropped_tok).to(dev)] == 0)
    if w.dropless:
        assert o_disp["kept"].all() and o_disp["rows"] == w.T * w.k


# One expert holds every token, in more than 12 M tiles with a partial last
# group of 6, so both GEMMs run the grouped tile order inside an expert
# (experts past 12 M tiles: groups of 6 M tiles swept over the N tiles).
# With 256 CUs the schedule picks 192-row tiles for the first case (16 M
# tiles, groups 6+6+4) and 256-row tiles for the first GEMM of the second
# (14 M tiles x 18 N tiles fill one round; groups 6+6+2); both split the
# second GEMM's K. The stage entry point runs the same problem unsplit.
MANY_MTILES = {
    "hot_mtiles_192": dict(T=3000, d=512, d_ff=512),
    "hot_mtiles_256": dict(T=3400, d=512, d_ff=4608),
}


@pytest.mark.parametrize("name", list(MANY_MTILES))
def test_grouped_order_many_m_tiles(name):
    w = WORKLOADS["small_bf16"].scaled(name=name, E=2, k=1, dropless=True, **MANY_MTILES[name])
    dev = "cuda"
    inp = synth.make_inputs(w, dev, seed=4)
    inp["b_r"][0] += 40.0  # every token chooses expert 0
    m = moe()
    C = cap(w)
    cfg = P.make_cfg(w, C)
    R = m.max_rows(cfg)
    say(f"[gpu] grouped order {name}: one expert with {w.T} rows, d={w.d} d_ff={w.d_ff}")
    info = P.info_tensors(w, R, dev)
    info["h"] = torch.full((R, w.d_ff), float("nan"), dtype=w.torch_dtype, device=dev)
    y = torch.full((w.T, w.d), float("nan"), dtype=w.torch_dtype, device=dev)
    m.layer_forward(cfg, inp["x"], inp["W_r"], inp["b_r"], inp["W1"], inp["b1"], inp["W2"],
                    inp["b2"], y, info=info)
    torch.cuda.synchronize()
    h = P.host_inputs(inp, w.dtype)
    o = mo.layer_forward(h["x"], h["W_r"], h["b_r"], h["W1"], h["b1"], h["W2"], h["b2"], k=w.k,
                         C=C, renormalize=w.renormalize, act=w.act)
    assert o["expert_counts"].tolist() == [w.T, 0]
    g = {k: v.cpu().numpy() for k, v in info.items() if k != "h"}
    P.check_dispatch(g, o)
    st = {"h": P.compare_outputs(P.host64(info["h"], w.dtype), o["h"], w.dtype),
          "y": P.compare_outputs(P.host64(y, w.dtype), o["y"], w.dtype)}
    # the stage entry points on the oracle's permuted rows (no gather, no split)
    xp = inp["x"][torch.from_numpy(o["row_token"]).to(dev)].contiguous()
    hb = torch.full((R, w.d_ff), float("nan"), dtype=w.torch_dtype, device=dev)
    yp = torch.full((R, w.d), float("nan"), dtype=w.torch_dtype, device=dev)
    m.expert_ffn(cfg, xp, torch.from_numpy(o["expert_offsets"]).to(dev), inp["W1"], inp["b1"],
                 inp["W2"], inp["b2"], hb, yp)
    torch.cuda.synchronize()
    st["stage_h"] = P.compare_outputs(P.host64(hb, w.dtype), o["h"], w.dtype)
    st["stage_y_perm"] = P.compare_outputs(P.host64(yp, w.dtype), o["y_perm"], w.dtype)
    say(f"[gpu] grouped order {name}: {st}")


# The second GEMM's tail parts (the M tiles of a last, partly filled round
# of whole tiles run as K parts, which the combine adds) at sizes the oracle
# finishes in seconds: the GEMMs' grid is capped at 16 blocks, so two full
# rounds take 32 tiles. d = 512 (two feature panels), d_ff = 1024 (16 K
# stages); the schedule's costs pick (by its arithmetic, which the sizes
# were chosen with):
#  * one expert of 3100 rows: 17 M tiles of 192 rows, 34 tiles; two rounds
#    and the last M tile's 2 tiles (28 rows) left, run as 4 K parts each;
#  * experts of 6200, 0 and 40 rows: 26 M tiles of 256 rows, 52 tiles;
#    three rounds and 4 tiles left: expert 0's last M tile (56 rows) and,
#    past the empty expert 1, expert 2's only one, run as 4 K parts each.
TAIL_CASES = {
    "tail_one_expert": dict(T=3100, E=2, last=None, counts=[3100, 0]),
    "tail_across_experts": dict(T=6240, E=3, last=40, counts=[6200, 0, 40]),
}


@pytest.mark.parametrize("name", list(TAIL_CASES))
def test_gemm2_tail_parts(name):
    spec = TAIL_CASES[name]
    w = WORKLOADS["small_bf16"].scaled(name=name, T=spec["T"], E=spec["E"], k=1, d=512, d_ff=1024,
                                       dropless=True)
    inp = synth.make_inputs(w, "cuda", seed=5)
    if spec["last"] is None:
        inp["b_r"][0] += 40.0  # every token chooses expert 0
    else:
        inp["b_r"][1] -= 40.0  # expert 1 is never chosen
        # exactly `last` tokens prefer expert 2: expert 0's bias moves to the
        # middle of the gap between the last-th and next largest margins
        h = P.host_inputs(inp, w.dtype)
        s = mo.router_logits(h["x"], h["W_r"], h["b_r"])
        gap = np.sort(s[:, 2] - s[:, 0])[::-1]
        inp["b_r"][0] += float((gap[spec["last"] - 1] + gap[spec["last"]]) / 2)
    m = moe()
    say(f"[gpu] tail parts {name}: GEMM grid capped at 16 blocks")
    m.set_gemm_max_blocks(16)
    try:
        _, _, o, _ = P.full_parity(w, inp, cap(w), report=say)
    finally:
        m.set_gemm_max_blocks(0)
    assert o["expert_counts"].tolist() == spec["counts"]


# The same layers on other grids: the tile plan (heights, K parts of a last
# partial round, XCD windows; a grid that is not a multiple of 8 takes the
# plain order) follows the grid the GEMMs get.
@pytest.mark.parametrize("blocks", [8, 60, 248])
@pytest.mark.parametrize("name", ["small_bf16_mini", "mid_bf16_mini", "mid_cap400_bf16"])
def test_layer_parity_capped_grid(name, blocks):
    w = MINI[name]
    inp = synth.make_inputs(w, "cuda", seed=3)
    m = moe()
    say(f"[gpu] capped grid {name}: {blocks} blocks")
    m.set_gemm_max_blocks(blocks)
    try:
        P.full_parity(w, inp, cap(w), report=say)
    finally:
        m.set_gemm_max_blocks(0)


# K stage counts 1, 2, 3 and 5 in both expert GEMMs, around the depths of the
# token and weight stage rings (2 to 4 buffers): the short-tile kernel
# (every expert under 256 rows: 64- and 128-row tiles) and the tall one
# (256- and 192-row tiles).
STAGE_EDGES = [(64, 320), (128, 192), (192, 128), (320, 64)]


@pytest.mark.parametrize("kernel", ["short", "tall"])
@pytest.mark.parametrize("d,d_ff", STAGE_EDGES, ids=[f"d{a}_f{b}" for a, b in STAGE_EDGES])
def test_gemm_stage_counts(kernel, d, d_ff):
    shape = dict(T=150, E=4, k=2) if kernel == "short" else dict(T=700, E=2, k=1)
    w = WORKLOADS["small_bf16"].scaled(name=f"stages_{kernel}_d{d}_f{d_ff}", d=d, d_ff=d_ff,
                                       dropless=True, **shape)
    inp = synth.make_inputs(w, "cuda", seed=7)
    say(f"[gpu] stage counts {w.name}")
    P.full_parity(w, inp, cap(w), report=say)


@pytest.mark.parametrize("name", ["tiny_f32", "f32_mid", "small_bf16_mini", "skewed_bf16_mini",
                                  "large_e_bf16_mini"])
def test_load_stats_on_gpu(name):
    """moe_load_stats on the layer's own counts and probability sums against
    the oracle's load_stats (pinned by hand-worked examples)."""
    w = MINI[name]
    dev = "cuda"
    inp = synth.make_inputs(w, dev, seed=2)
    C = cap(w)
    y, g, cfg = P.gpu_layer(w, inp, C)
    m = moe()
    counts = torch.from_numpy(g["expert_counts"]).to(dev)
    offsets = torch.from_numpy(g["expert_offsets"]).to(dev)
    psum = torch.from_numpy(g["prob_sum"]).to(dev)
    stats = torch.full((len(m.STAT_NAMES),), float("nan"), dtype=torch.float64, device=dev)
    kept = torch.full((w.E,), -7, dtype=torch.int32, device=dev)
    dropped = torch.full((w.E,), -7, dtype=torch.int32, device=dev)
    alpha = 0.01
    m.load_stats(cfg, counts, offsets, psum, alpha, stats, kept=kept, dropped=dropped)
    torch.cuda.synchronize()
    got = dict(zip(m.STAT_NAMES, stats.cpu().tolist()))
    h = P.host_inputs(inp, w.dtype)
    ref = mo.load_stats(g["expert_counts"], C, w.T, w.k,
                        prob_sum=mo.route(h["x"], h["W_r"], h["b_r"], w.k, w.renormalize)["prob_sum"],
                        alpha=alpha)
    say(f"[gpu] load stats {name}: {got}")
    assert kept.cpu().tolist() == ref["kept_per_expert"]
    assert dropped.cpu().tolist() == ref["dropped_per_expert"]
    assert got["dropped"] == ref["dropped"] and got["kept_rows"] == sum(ref["kept_per_expert"])
    for key in ("overflow_ratio", "max_over_mean_load", "padding_ratio", "load_entropy",
                "kept_variance"):
        assert got[key] == pytest.approx(ref[key], rel=1e-12, abs=1e-12), key
    assert got["aux_loss"] == pytest.approx(ref["aux_loss"], rel=1e-5)


def test_f32_layer_ignores_stale_split_word():
    """An fp32 layer has no K split: its combine must not read the split
    word or partial buffer of the workspace, whatever they hold (here int32
    2 everywhere, the value that means "split")."""
    w = MINI["f32_mid"]
    dev = "cuda"
    inp = synth.make_inputs(w, dev, seed=6)
    C = cap(w)
    m = moe()
    cfg = P.make_cfg(w, C)
    ws = m.alloc_workspace(cfg, dev)
    ws.view(torch.int32)[: ws.numel() // 4].fill_(2)
    y, g, _ = P.gpu_layer(w, inp, C, ws=ws)
    h = P.host_inputs(inp, w.dtype)
    o = mo.layer_forward(h["x"], h["W_r"], h["b_r"], h["W1"], h["b1"], h["W2"], h["b2"], k=w.k,
                         C=C, renormalize=w.renormalize, act=w.act, ids=g["topk_ids"])
    P.compare_outputs(P.host64(y, w.dtype), o["y"], w.dtype)


def test_graph_replay_matches_eager():
    """The layer captured once in a HIP graph and replayed gives the eager
    result bit for bit, on every replay, with eager work and synchronisation
    between replays (the benchmark times such replays)."""
    w = WORKLOADS["small_bf16"].scaled(name="graph_replay", T=1000, d=256, d_ff=512)
    dev = "cuda"
    inp = synth.make_inputs(w, dev, seed=5)
    other = synth.make_inputs(w, dev, seed=6)
    C = cap(w)
    m = moe()
    cfg = P.make_cfg(w, C)
    ws = m.alloc_workspace(cfg, dev)
    i32 = dict(dtype=torch.int32, device=dev)
    info = {"topk_ids": torch.empty((w.T, w.k), **i32),
            "expert_offsets": torch.empty(w.E + 1, **i32),
            "row_of": torch.empty((w.T, w.k), **i32)}
    y = torch.empty((w.T, w.d), dtype=w.torch_dtype, device=dev)

    def call(src, out, inf):
        m.layer_forward(cfg, src["x"], src["W_r"], src["b_r"], src["W1"], src["b1"], src["W2"],
                        src["b2"], out, info=inf, ws=ws)

    y_ref = torch.empty_like(y)
    info_ref = {k: torch.empty_like(v) for k, v in info.items()}
    call(inp, y_ref, info_ref)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(inp, y, info)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(inp, y, info)
    y_other = torch.empty_like(y)
    for rep in range(3):
        y.fill_(0)
        for v in info.values():
            v.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"replay {rep}: y differs"
        for k in info:
            assert torch.equal(info[k], info_ref[k]), f"replay {rep}: {k} differs"
        # eager work on the same workspace between replays
        call(other, y_other, {k: torch.empty_like(v) for k, v in info.items()})
        torch.cuda.synchronize()


# Router logits kernel shapes: every tile instantiation (E <= 16, <= 32,
# <= 64 with few and with many tokens, > 64) and K step counts that leave
# some of the four waves with no step (d = 64, 192) or with step counts that
# are not a multiple of the operand ring's depth (d = 704, 1344).
LOGIT_CASES = [
    ("e8_d64", dict(T=37, d=64, E=8, k=2)),
    ("e24_d192", dict(T=130, d=192, E=24, k=3)),
    ("e64_d1344_few", dict(T=300, d=1344, E=64, k=4)),
    ("e64_d1344_many", dict(T=8199, d=1344, E=64, k=4)),
    ("e200_d704", dict(T=130, d=704, E=200, k=8)),
]


@pytest.mark.parametrize("name,shape", LOGIT_CASES, ids=[c[0] for c in LOGIT_CASES])
def test_router_logits_shapes(name, shape):
    w = WORKLOADS["skewed_bf16"].scaled(name=name, d_ff=64, **shape)
    m = moe()
    inp = synth.make_inputs(w, "cuda", seed=5)
    C = cap(w)
    cfg = P.make_cfg(w, C)
    ws = m.alloc_workspace(cfg, "cuda")
    h = P.host_inputs(inp, w.dtype)
    say(f"[gpu] router logits {name} T={w.T} d={w.d} E={w.E}")
    ids = torch.empty((w.T, w.k), dtype=torch.int32, device="cuda")
    gates = torch.empty((w.T, w.k), dtype=torch.float32, device="cuda")
    psum = torch.empty(w.E, dtype=torch.float32, device="cuda")
    logits = torch.empty((w.T, w.E), dtype=torch.float32, device="cuda")
    m.route(cfg, inp["x"], inp["W_r"], inp["b_r"], ids, gates, psum, logits, ws=ws)
    torch.cuda.synchronize()
    s = mo.router_logits(h["x"], h["W_r"], h["b_r"])
    np.testing.assert_allclose(logits.cpu().numpy(), s, rtol=1e-5, atol=1e-5)
    o = mo.route(h["x"], h["W_r"], h["b_r"], w.k, w.renormalize)
    P.check_routing(o, ids.cpu().numpy())
