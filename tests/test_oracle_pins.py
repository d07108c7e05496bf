"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each check below ties one oracle function to something other than itself: a
value the pages print for a worked example (tests/golden/, each with its
citation), a closed form, an invariant, a special case that reduces to a
library routine, or brute force on tiny inputs. The mutation tests at the end
plant plausible mistakes in the oracle (on the CPU) and show that a pin fails
for each.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as mo

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------ capacity

def check_capacity_pages():
    for case in golden("capacity_examples.json")["cases"]:
        assert mo.capacity(case["T"], case["k"], case["E"], case["c"]) == case["C"], case


def check_capacity_closed_form():
    # ceil of a non-integer quotient: 1.0*10*1/4 = 2.5 -> 3; 1.25*7*2/3 = 5.833 -> 6
    assert mo.capacity(10, 1, 4, 1.0) == 3
    assert mo.capacity(7, 2, 3, 1.25) == 6
    # exact integer quotients stay put
    assert mo.capacity(12, 2, 8, 1.0) == 3
    # the five workloads
    assert mo.capacity(8, 1, 2, 1.0) == 4
    assert mo.capacity(4096, 2, 8, 1.25) == 1280
    assert mo.capacity(16384, 2, 8, 1.25) == 5120
    assert mo.capacity(8192, 4, 64, 1.0) == 512
    assert mo.capacity(4096, 8, 256, 1.25) == 160


def test_capacity_pages():
    check_capacity_pages()


def test_capacity_closed_form():
    check_capacity_closed_form()


# ------------------------------------------------------------------ dispatch

def check_drop_rule():
    g = golden("drop_rule_example.json")
    ids = np.array(g["topk_ids"], dtype=np.int32)
    for key in ("C4", "C6"):
        exp = g[key]
        out = mo.dispatch(ids, g["E"], exp["C"])
        assert out["expert_counts"].tolist() == exp["expert_counts"]
        assert out["n"].tolist() == exp["kept_per_expert"]
        assert np.flatnonzero(~out["kept"][:, 0]).tolist() == exp["overflow_tokens"]
        assert out["expert_offsets"].tolist() == exp["expert_offsets"]
        assert out["row_token"].tolist() == exp["row_token"]
        if "slot" in exp:
            assert out["slot"].tolist() == exp["slot"]
            assert out["row_of"].tolist() == exp["row_of"]


def test_drop_rule_pages():
    check_drop_rule()


def overflow_routing(seed=3):
    g = golden("overflow_example.json")
    T, E, hot, n_hot = g["T"], g["E"], g["hot_expert"], g["hot_tokens"]
    r = rng(seed)
    hot_pos = np.sort(r.choice(T, size=n_hot, replace=False))
    ids = np.empty((T, 1), dtype=np.int32)
    others = [e for e in range(E) if e != hot]
    ids[:, 0] = np.array(others)[np.arange(T) % len(others)]
    ids[hot_pos, 0] = hot
    return g, ids, hot_pos


def test_overflow_pages():
    g, ids, hot_pos = overflow_routing()
    for case in g["cases"]:
        C = mo.capacity(g["T"], g["k"], g["E"], case["c"])
        assert C == case["C"]
        out = mo.dispatch(ids, g["E"], C)
        dropped = int((~out["kept"]).sum())
        assert dropped == case["dropped"]
        # the hot expert keeps its earliest C tokens, in token order
        e = g["hot_expert"]
        a, b = out["expert_offsets"][e], out["expert_offsets"][e + 1]
        assert out["row_token"][a:b].tolist() == hot_pos[:C].tolist()
        # every other expert stays within capacity
        assert all(out["expert_counts"][i] <= C for i in range(g["E"]) if i != e)


def brute_dispatch(ids, E, k):
    """Token-by-token first-come assignment, pure Python."""
    T = len(ids)
    used = [0] * E
    slot = [[0] * k for _ in range(T)]
    for t in range(T):
        for j in range(k):
            e = ids[t][j]
            slot[t][j] = used[e]
            used[e] += 1
    return used, slot


def test_dispatch_bruteforce_and_invariants():
    r = rng(11)
    for trial in range(200):
        E = int(r.integers(1, 9))
        k = int(r.integers(1, E + 1))
        T = int(r.integers(0, 40))
        C = int(r.integers(1, max(2, T)))
        ids = np.stack([r.permutation(E)[:k] for _ in range(T)]) if T else np.zeros((0, k), np.int32)
        ids = ids.astype(np.int32).reshape(T, k)
        out = mo.dispatch(ids, E, C)
        used, slot = brute_dispatch(ids.tolist(), E, k)
        assert out["expert_counts"].tolist() == used
        assert out["slot"].tolist() == (slot if T else [])
        n = np.minimum(np.array(used), C)
        assert out["rows"] == int(n.sum()) == int(out["kept"].sum())
        assert out["expert_offsets"].tolist() == [0] + np.cumsum(n).tolist()
        for e in range(E):
            seg = out["row_token"][out["expert_offsets"][e]:out["expert_offsets"][e + 1]]
            assert np.all(np.diff(seg) > 0)              # token order inside an expert
            assert all(e in ids[t] for t in seg)
        for t in range(T):
            for j in range(k):
                row = out["row_of"][t, j]
                if row >= 0:
                    assert out["row_token"][row] == t
        if C >= T:
            assert out["rows"] == T * k


# ------------------------------------------------------------------ routing

def brute_topk(s32_row, k):
    """rank_i = |{j : s_j > s_i}| + |{j < i : s_j = s_i}| by counting pairs."""
    E = len(s32_row)
    rank = [sum(1 for j in range(E) if s32_row[j] > s32_row[i]) +
            sum(1 for j in range(i) if s32_row[j] == s32_row[i]) for i in range(E)]
    return [rank.index(r) for r in range(k)]


def check_topk_bruteforce():
    r = rng(5)
    for trial in range(300):
        E = int(r.integers(1, 9))
        k = int(r.integers(1, E + 1))
        T = int(r.integers(1, 6))
        d = int(r.integers(1, 5))
        if trial % 2 == 0:
            # integer-valued inputs: exact sums, frequent exact ties
            x = r.integers(-2, 3, size=(T, d)).astype(np.float64)
            W = r.integers(-2, 3, size=(E, d)).astype(np.float64)
            b = r.integers(-1, 2, size=E).astype(np.float64)
        else:
            x = r.standard_normal((T, d))
            W = r.standard_normal((E, d))
            b = r.standard_normal(E)
        s = mo.router_logits(x, W, b)
        ids = mo.topk_ids(s, k)
        s32 = mo.round_f32(s)
        for t in range(T):
            assert ids[t].tolist() == brute_topk(s32[t].tolist(), k), (s32[t], k)


def test_topk_bruteforce():
    check_topk_bruteforce()


def test_router_logits_bruteforce():
    r = rng(6)
    x = r.standard_normal((3, 5))
    W = r.standard_normal((4, 5))
    b = r.standard_normal(4)
    s = mo.router_logits(x, W, b)
    for t in range(3):
        for i in range(4):
            assert s[t, i] == pytest.approx(b[i] + sum(W[i, m] * x[t, m] for m in range(5)), abs=1e-12)


def check_gates():
    r = rng(8)
    s = r.standard_normal((50, 6)) * 3
    p = mo.softmax(s)
    # softmax against the library routine
    np.testing.assert_allclose(p, torch.softmax(torch.from_numpy(s), dim=1).numpy(), rtol=1e-13)
    for k in (1, 2, 6):
        ids = mo.topk_ids(s, k)
        g = mo.gates(p, ids, True)
        np.testing.assert_allclose(g.sum(axis=1), 1.0, atol=1e-14)
        chosen = np.take_along_axis(p, ids.astype(np.int64), axis=1)
        np.testing.assert_allclose(g, chosen / chosen.sum(axis=1, keepdims=True), rtol=1e-14)
        raw = mo.gates(p, ids, False)
        np.testing.assert_array_equal(raw, chosen)
        if k == 1:
            np.testing.assert_allclose(g, 1.0, atol=0)
            np.testing.assert_array_equal(raw[:, 0], p.max(axis=1))
        # descending order of the chosen probabilities
        assert np.all(np.diff(raw, axis=1) <= 0)


def test_gates():
    check_gates()


def test_near_ties():
    s = np.array([[1.0, 1.0 + 1e-9, -3.0], [2.0, 1.0, 0.0], [5.0, 4.0, 4.0 + 1e-12]])
    assert mo.near_ties(s, 1).tolist() == [True, False, False]
    assert mo.near_ties(s, 2).tolist() == [True, False, True]


# ------------------------------------------------------------------ aux loss

def check_aux_loss():
    g = golden("aux_loss_example.json")
    w = g["worked"]
    T, E = w["T"], w["E"]
    counts = np.array(w["f"]) * T
    prob_sum = np.array(w["pbar"]) * T
    assert mo.aux_loss(counts, prob_sum, T, E, 1.0) == pytest.approx(w["loss_over_alpha"], abs=1e-12)
    # realised by a real routing: rows with p = (0.6, 0.4) six times, (0.4, 0.6) twice
    a = math.log(1.5) / 2
    x = np.array([[1.0]] * 6 + [[-1.0]] * 2)
    W = np.array([[a], [-a]])
    r = mo.route(x, W, np.zeros(2), 1, False)
    np.testing.assert_allclose(r["probs"][0], [0.6, 0.4], rtol=1e-14)
    d = mo.dispatch(r["topk_ids"], E, 4)
    assert d["expert_counts"].tolist() == [6, 2]
    alpha = golden("aux_loss_example.json")["alpha_typical"]["alpha"]
    assert mo.aux_loss(d["expert_counts"], r["prob_sum"], T, E, alpha) == pytest.approx(1.05 * alpha, rel=1e-12)
    # uniform f (or uniform pbar) at k = 1 gives exactly alpha
    for E in (2, 8, 64):
        T = 4 * E
        assert mo.aux_loss(np.full(E, T // E), r_sum(E, T), T, E, 0.01) == pytest.approx(0.01, rel=1e-12)
        skew = rng(E).dirichlet(np.ones(E)) * T
        assert mo.aux_loss(np.full(E, T // E), skew, T, E, 0.01) == pytest.approx(0.01, rel=1e-12)


def r_sum(E, T):
    return np.full(E, T / E)


def test_aux_loss_pages():
    check_aux_loss()


# ------------------------------------------------------------------ experts

def test_gelu_against_library_and_exact():
    u = np.linspace(-8, 8, 4001)
    ref = torch.nn.functional.gelu(torch.from_numpy(u), approximate="tanh").numpy()
    np.testing.assert_allclose(mo.gelu_tanh(u), ref, rtol=1e-12, atol=1e-15)
    exact = u * 0.5 * (1 + np.array([math.erf(v / math.sqrt(2)) for v in u]))
    assert np.max(np.abs(mo.gelu_tanh(u) - exact)) < 1e-3
    np.testing.assert_array_equal(mo.relu(np.array([-1.0, 0.0, 2.5])), [0.0, 0.0, 2.5])


def dense_ffn_torch(x, W1, b1, W2, b2, act):
    F = torch.nn.functional
    u = F.linear(torch.from_numpy(x), torch.from_numpy(W1), torch.from_numpy(b1))
    h = F.gelu(u, approximate="tanh") if act == "gelu_tanh" else F.relu(u)
    return F.linear(h, torch.from_numpy(W2), torch.from_numpy(b2)).numpy()


def random_layer(r, T, d, d_ff, E):
    x = r.standard_normal((T, d))
    W_r = r.standard_normal((E, d)) / math.sqrt(d)
    b_r = r.standard_normal(E) * 0.1
    W1 = r.standard_normal((E, d_ff, d)) / math.sqrt(d)
    b1 = r.standard_normal((E, d_ff)) * 0.1
    W2 = r.standard_normal((E, d, d_ff)) / math.sqrt(d_ff)
    b2 = r.standard_normal((E, d)) * 0.1
    return x, W_r, b_r, W1, b1, W2, b2


def check_single_expert_is_dense_ffn():
    r = rng(21)
    x, W_r, b_r, W1, b1, W2, b2 = random_layer(r, 37, 12, 20, 1)
    for act in ("relu", "gelu_tanh"):
        out = mo.layer_forward(x, W_r, b_r, W1, b1, W2, b2, k=1, C=37, renormalize=True, act=act)
        np.testing.assert_allclose(out["y"], dense_ffn_torch(x, W1[0], b1[0], W2[0], b2[0], act),
                                   rtol=1e-12, atol=1e-12)


def test_single_expert_is_dense_ffn():
    check_single_expert_is_dense_ffn()


def check_identical_experts():
    r = rng(22)
    x, W_r, b_r, W1, b1, W2, b2 = random_layer(r, 41, 10, 16, 5)
    W1[:] = W1[0]
    b1[:] = b1[0]
    W2[:] = W2[0]
    b2[:] = b2[0]
    out = mo.layer_forward(x, W_r, b_r, W1, b1, W2, b2, k=3, C=41, renormalize=True, act="gelu_tanh")
    np.testing.assert_allclose(out["y"], dense_ffn_torch(x, W1[0], b1[0], W2[0], b2[0], "gelu_tanh"),
                               rtol=1e-12, atol=1e-12)


def test_identical_experts_give_dense_ffn():
    check_identical_experts()


def check_dense_soft_mixture():
    """k = E, renormalised, no drops: y = sum_i p_i E_i(x) over every expert."""
    r = rng(23)
    T, d, d_ff, E = 29, 9, 14, 4
    x, W_r, b_r, W1, b1, W2, b2 = random_layer(r, T, d, d_ff, E)
    out = mo.layer_forward(x, W_r, b_r, W1, b1, W2, b2, k=E, C=T, renormalize=True, act="relu")
    p = torch.softmax(torch.from_numpy(x @ W_r.T + b_r), dim=1).numpy()
    ref = sum(p[:, [i]] * dense_ffn_torch(x, W1[i], b1[i], W2[i], b2[i], "relu") for i in range(E))
    np.testing.assert_allclose(out["y"], ref, rtol=1e-11, atol=1e-12)


def test_dense_soft_mixture():
    check_dense_soft_mixture()


def test_layer_permutation_invariants():
    r = rng(24)
    T, d, d_ff, E, k = 53, 8, 12, 6, 2
    x, W_r, b_r, W1, b1, W2, b2 = random_layer(r, T, d, d_ff, E)
    b_r[2] += 3.0  # a hot expert so that drops happen
    C = mo.capacity(T, k, E, 1.0)
    out = mo.layer_forward(x, W_r, b_r, W1, b1, W2, b2, k=k, C=C, renormalize=True, act="gelu_tanh")
    assert (~out["kept"]).sum() > 0
    np.testing.assert_array_equal(out["x_perm"], x[out["row_token"]])
    dropped_all = ~out["kept"].any(axis=1)
    np.testing.assert_array_equal(out["y"][dropped_all], 0.0)
    # a token's output: its kept assignments, computed one by one
    for t in range(T):
        ref = np.zeros(d)
        for j in range(k):
            if out["kept"][t, j]:
                e = out["topk_ids"][t, j]
                _, Y = mo.expert_ffn(x[t:t + 1], W1[e], b1[e], W2[e], b2[e], "gelu_tanh")
                ref += out["topk_gates"][t, j] * Y[0]
        np.testing.assert_allclose(out["y"][t], ref, rtol=1e-12, atol=1e-13)


def test_sampled_outputs_match_full_layer():
    r = rng(25)
    T, d, d_ff, E, k = 40, 8, 12, 5, 2
    x, W_r, b_r, W1, b1, W2, b2 = random_layer(r, T, d, d_ff, E)
    out = mo.layer_forward(x, W_r, b_r, W1, b1, W2, b2, k=k, C=10, renormalize=True, act="relu")
    tok = [0, 7, 39]
    ys = mo.sampled_outputs(tok, x, out["topk_ids"], out["row_of"], out["topk_gates"],
                            lambda e: (W1[e], b1[e], W2[e], b2[e]), "relu")
    np.testing.assert_allclose(ys, out["y"][tok], rtol=1e-12, atol=1e-13)


def check_constructed_drop_layer():
    """The page's [1,1,1,1,1,1,2,2] routing realised as a layer input."""
    d, T = 16, 8
    x = np.zeros((T, d))
    x[:, 0] = [1, 1, 1, 1, 1, 1, -1, -1]
    x[:, 1:] = rng(9).standard_normal((T, d - 1))
    W_r = np.zeros((2, d))
    W_r[:, 0] = [0.5, -0.5]
    r = rng(10)
    W1 = r.standard_normal((2, 64, d)) / 4
    W2 = r.standard_normal((2, d, 64)) / 8
    b1 = np.zeros((2, 64))
    b2 = np.zeros((2, d))
    out = mo.layer_forward(x, W_r, np.zeros(2), W1, b1, W2, b2, k=1,
                           C=mo.capacity(T, 1, 2, 1.0), renormalize=False, act="relu")
    assert out["topk_ids"][:, 0].tolist() == [0] * 6 + [1] * 2
    assert out["n"].tolist() == [4, 2]
    np.testing.assert_array_equal(out["y"][4:6], 0.0)
    assert np.all(np.abs(out["y"][:4]).sum(axis=1) > 0)
    out6 = mo.layer_forward(x, W_r, np.zeros(2), W1, b1, W2, b2, k=1,
                            C=mo.capacity(T, 1, 2, 1.5), renormalize=False, act="relu")
    assert out6["rows"] == 8


def test_constructed_drop_layer():
    check_constructed_drop_layer()


def test_toy_top1_semantics():
    """The page's top-1 example: kept per expert <= C, overflow tokens output
    zero, the gate is the top softmax probability  [MoE Principles §7]."""
    r = rng(12)
    T, d, d_ff, E = 64, 4, 8, 2
    x, W_r, b_r, W1, b1, W2, b2 = random_layer(r, T, d, d_ff, E)
    b_r[:] = [0.8, 0.0]
    C = mo.capacity(T, 1, E, 1.0)
    out = mo.layer_forward(x, W_r, b_r, W1, b1, W2, b2, k=1, C=C, renormalize=False, act="relu")
    assert np.all(out["n"] <= C)
    overflow = ~out["kept"][:, 0]
    assert overflow.sum() == max(0, out["expert_counts"].max() - C)
    np.testing.assert_array_equal(out["y"][overflow], 0.0)
    np.testing.assert_array_equal(out["topk_gates"][:, 0], out["probs"].max(axis=1))


def test_flops_formula():
    # 2 x (2 d d_ff) per (token, expert)  [MoE Principles §8.3]
    assert mo.ffn_flops(1, 4096, 14336) == 2 * (2 * 4096 * 14336)


def test_load_stats():
    s = mo.load_stats([6, 2], 4, 8, 1)
    assert s["dropped"] == 2 and s["dropped_per_expert"] == [2, 0]
    assert s["padding_ratio"] == pytest.approx(2 * 4 / 6)


def test_load_stats_worked_example():
    """The page's §3.3 routing at C = 4 (§4.2), every figure worked by hand
    (tests/golden/load_stats_example.json)."""
    g = golden("load_stats_example.json")["worked"]
    s = mo.load_stats(g["counts"], g["C"], g["T"], g["k"], prob_sum=g["prob_sum"], alpha=1.0)
    assert s["kept_per_expert"] == [4, 2] and s["dropped_per_expert"] == [2, 0] and s["dropped"] == 2
    assert s["overflow_ratio"] == pytest.approx(0.25, abs=1e-15)
    assert s["max_over_mean_load"] == pytest.approx(1.5, abs=1e-15)
    assert s["padding_ratio"] == pytest.approx(4.0 / 3.0, abs=1e-15)
    assert s["load_entropy"] == pytest.approx(math.log(4.0) - 0.75 * math.log(3.0), abs=1e-15)
    assert s["kept_variance"] == pytest.approx(1.0, abs=1e-15)
    assert s["aux_loss"] == pytest.approx(1.05, abs=1e-12)


def test_load_stats_overflow_example():
    g = golden("load_stats_example.json")["overflow"]
    s = mo.load_stats(g["counts"], g["C"], g["T"], g["k"])
    assert s["dropped"] == 659
    assert s["overflow_ratio"] == pytest.approx(659 / 1024, abs=1e-15)
    assert s["max_over_mean_load"] == pytest.approx(819 / 128, abs=1e-15)
    assert s["padding_ratio"] == pytest.approx(1280 / 365, abs=1e-15)


@pytest.mark.parametrize("E,n", [(1, 7), (8, 100), (64, 3)])
def test_load_stats_uniform(E, n):
    """Equal loads: the entropy is ln E (its maximum), max/mean 1, no spread,
    and nothing overflows when C holds each expert's share."""
    s = mo.load_stats([n] * E, n, n * E, 1)
    assert s["load_entropy"] == pytest.approx(math.log(E), abs=1e-12)
    assert s["max_over_mean_load"] == 1.0 and s["kept_variance"] == 0.0
    assert s["overflow_ratio"] == 0.0 and s["padding_ratio"] == 1.0


def test_load_stats_one_hot_expert():
    """Every assignment on one expert: zero entropy, max/mean E, and C caps it."""
    s = mo.load_stats([0, 0, 40, 0], 10, 40, 1)
    assert s["load_entropy"] == 0.0 and s["max_over_mean_load"] == 4.0
    assert s["dropped"] == 30 and s["overflow_ratio"] == 0.75
    assert s["kept_variance"] == pytest.approx(np.var([0, 0, 10, 0]), abs=1e-15)


def test_widen_bf16_exact():
    vals = np.array([1.0, -2.5, 3.140625, 1e-3, 65504.0], dtype=np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    back = mo.widen(bits, "bf16")
    ref = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float64).numpy()
    # truncation equals RNE for these values (their low halves are zero or tiny)
    np.testing.assert_array_equal(back[:3], ref[:3])


# ------------------------------------------------------------------ planted mistakes

def _expect_fail(fn):
    with pytest.raises(AssertionError):
        fn()


def test_planted_tie_break_is_caught(monkeypatch):
    def highest_index_first(s, k):
        s32 = mo.round_f32(s)
        E = s32.shape[1]
        order = np.argsort(-s32[:, ::-1], axis=1, kind="stable")
        return (E - 1 - order[:, :k]).astype(np.int32)
    monkeypatch.setattr(mo, "topk_ids", highest_index_first)
    _expect_fail(check_topk_bruteforce)


def test_planted_ascending_topk_is_caught(monkeypatch):
    monkeypatch.setattr(mo, "topk_ids", lambda s, k: np.argsort(mo.round_f32(s), axis=1,
                                                                kind="stable")[:, :k].astype(np.int32))
    _expect_fail(check_topk_bruteforce)


def test_planted_missing_renormalisation_is_caught(monkeypatch):
    orig = mo.gates
    monkeypatch.setattr(mo, "gates", lambda p, ids, renormalize: orig(p, ids, False))
    _expect_fail(check_gates)
    _expect_fail(check_identical_experts)


def test_planted_last_come_slots_are_caught(monkeypatch):
    orig = mo.dispatch

    def last_come(ids, E, C):
        ids = np.asarray(ids)
        out = orig(ids[::-1], E, C)
        for key in ("slot", "kept", "row_of"):
            out[key] = out[key][::-1]
        return out
    monkeypatch.setattr(mo, "dispatch", last_come)
    _expect_fail(check_drop_rule)


def test_planted_floor_capacity_is_caught(monkeypatch):
    monkeypatch.setattr(mo, "capacity", lambda T, k, E, c: int(c * T * k // E))
    _expect_fail(check_capacity_closed_form)


def test_planted_capacity_without_k_is_caught(monkeypatch):
    monkeypatch.setattr(mo, "capacity", lambda T, k, E, c: math.ceil(c * T / E))
    _expect_fail(check_capacity_closed_form)


def test_planted_gelu_constant_is_caught(monkeypatch):
    monkeypatch.setattr(mo, "gelu_tanh", lambda u: 0.5 * u * (1.0 + np.tanh(
        math.sqrt(2.0 / math.pi) * (u + 0.44715 * u ** 3))))
    monkeypatch.setitem(mo.ACTS, "gelu_tanh", mo.gelu_tanh)
    _expect_fail(test_gelu_against_library_and_exact)
    _expect_fail(check_identical_experts)


def test_planted_transposed_w1_is_caught(monkeypatch):
    def transposed(x_rows, W1_e, b1_e, W2_e, b2_e, act):
        h = mo.ACTS[act](x_rows @ W1_e.reshape(W1_e.shape[1], W1_e.shape[0]) + b1_e[None, :])
        return h, h @ W2_e.T + b2_e[None, :]
    monkeypatch.setattr(mo, "expert_ffn", transposed)
    _expect_fail(check_single_expert_is_dense_ffn)


def test_planted_missing_bias_is_caught(monkeypatch):
    def no_b2(x_rows, W1_e, b1_e, W2_e, b2_e, act):
        h = mo.ACTS[act](x_rows @ W1_e.T + b1_e[None, :])
        return h, h @ W2_e.T
    monkeypatch.setattr(mo, "expert_ffn", no_b2)
    _expect_fail(check_single_expert_is_dense_ffn)


def test_planted_dropped_tokens_kept_is_caught(monkeypatch):
    def combine_all(Y_rows, row_of, g):
        return mo_combine_orig(Y_rows, np.where(row_of >= 0, row_of, 0), g)
    mo_combine_orig = mo.combine
    monkeypatch.setattr(mo, "combine", combine_all)
    _expect_fail(check_constructed_drop_layer)


def test_planted_aux_loss_without_E_is_caught(monkeypatch):
    monkeypatch.setattr(mo, "aux_loss", lambda counts, prob_sum, T, E, alpha: alpha * float(
        np.sum(np.asarray(counts) / T * np.asarray(prob_sum) / T)))
    _expect_fail(check_aux_loss)


def test_planted_softmax_sign_is_caught(monkeypatch):
    monkeypatch.setattr(mo, "softmax", lambda s: np.exp(-s) / np.exp(-s).sum(axis=1, keepdims=True))
    _expect_fail(check_gates)
    _expect_fail(check_dense_soft_mixture)


# ------------------------------------------------------------------ re-routing and priority

REROUTE_KEYS = ("expert_counts", "served_col", "served_ids", "slot", "expert_offsets", "row_of",
                "row_token")


def check_reroute_pages():
    for c in golden("reroute_examples.json")["cases"]:
        o = mo.dispatch_rerouted(np.array(c["cand"]), c["k"], c["E"], c["C"], c["priority"],
                                 c["rounds"])
        for key in REROUTE_KEYS:
            assert o[key].tolist() == c[key], (c["name"], key, o[key].tolist())


def test_reroute_pages():
    check_reroute_pages()


def random_candidates(r, T, E, n):
    return (np.stack([r.permutation(E)[:n] for _ in range(T)]).astype(np.int32).reshape(T, n)
            if T else np.zeros((0, n), np.int32))


def counting_slots(cand, k, E, C, priority, rounds):
    """The same rule as a count per round instead of a running simulation:
    the slot of arrival (t, r) in round j is fill_j[e] plus the number of
    arrivals at e before it in priority order in that round."""
    T, n = cand.shape
    pos = (lambda t, r: t * k + r) if priority == "token" else (lambda t, r: r * T + t)
    col = np.tile(np.arange(k), (T, 1))
    served = np.full((T, k), -1)
    dead = np.zeros((T, k), bool)
    slot = np.zeros((T, k), int)
    fill = np.zeros(E, int)
    used = np.full(T, k)
    for rnd in range(rounds + 1):
        if rnd:
            for t in range(T):
                for r in range(k):
                    if served[t, r] < 0 and not dead[t, r]:
                        if used[t] < n:
                            col[t, r] = used[t]
                            used[t] += 1
                        else:
                            dead[t, r] = True
        live = [(t, r) for t in range(T) for r in range(k) if served[t, r] < 0 and not dead[t, r]]
        exp = {(t, r): int(cand[t, col[t, r]]) for t, r in live}
        arrivals = np.zeros(E, int)
        for t, r in live:
            e = exp[(t, r)]
            before = sum(1 for (u, q) in live if exp[(u, q)] == e and pos(u, q) < pos(t, r))
            slot[t, r] = fill[e] + before
            arrivals[e] += 1
        for t, r in live:
            if slot[t, r] < C:
                served[t, r] = col[t, r]
        fill = np.minimum(fill + arrivals, C)
    return served, slot, fill


def check_reroute_properties(trials=150):
    r = rng(21)
    for trial in range(trials):
        E = int(r.integers(1, 7))
        k = int(r.integers(1, E + 1))
        T = int(r.integers(0, 24))
        C = int(r.integers(1, max(2, T)))
        rounds = int(r.integers(0, 4))
        n = min(E, k * (1 + rounds))
        cand = random_candidates(r, T, E, n)
        for priority in ("token", "rank"):
            o = mo.dispatch_rerouted(cand, k, E, C, priority, rounds)
            served, slot, fill = counting_slots(cand, k, E, C, priority, rounds)
            assert o["served_col"].tolist() == served.tolist()
            assert o["slot"].tolist() == slot.tolist()
            assert o["n"].tolist() == fill.tolist()
            # capacity and layout
            assert np.all(o["n"] <= C)
            assert o["rows"] == int(o["kept"].sum()) == int(o["n"].sum())
            assert o["expert_offsets"].tolist() == [0] + np.cumsum(o["n"]).tolist()
            for t in range(T):
                ids_t = [e for e in o["served_ids"][t] if e >= 0]
                assert len(ids_t) == len(set(ids_t))          # an expert serves a token once
                for q in range(k):
                    row = o["row_of"][t, q]
                    if row >= 0:
                        e = o["served_ids"][t, q]
                        assert o["row_token"][row] == t
                        assert o["expert_offsets"][e] <= row < o["expert_offsets"][e + 1]
                        assert row - o["expert_offsets"][e] == o["slot"][t, q]
            # the first round's demand is the top-k count
            assert o["expert_counts"].tolist() == np.bincount(cand[:, :k].ravel(),
                                                              minlength=E).tolist()
            if rounds == 0 and priority == "token":
                d = mo.dispatch(cand[:, :k], E, C)
                for key in ("expert_counts", "expert_offsets", "slot", "row_of", "row_token"):
                    assert o[key].tolist() == d[key].tolist(), key
            if rounds > 0:
                # more rounds never undo a placement
                prev = mo.dispatch_rerouted(cand, k, E, C, priority, rounds - 1)
                assert np.all(o["kept"][prev["kept"]])
        if k == 1:
            a = mo.dispatch_rerouted(cand, 1, E, C, "token", rounds)
            b = mo.dispatch_rerouted(cand, 1, E, C, "rank", rounds)
            for key in REROUTE_KEYS:
                assert a[key].tolist() == b[key].tolist()


def test_reroute_properties():
    check_reroute_properties()


def check_candidate_gates():
    p = np.array([[0.5, 0.2, 0.2, 0.1], [0.1, 0.3, 0.4, 0.2]])
    cand = mo.candidate_ids(np.log(p), 3)
    assert cand.tolist() == [[0, 1, 2], [2, 1, 3]]     # equal scores: lower index first
    g = mo.candidate_gates(p, cand, 2, True)
    np.testing.assert_allclose(g, [[0.5 / 0.7, 0.2 / 0.7, 0.2 / 0.7],
                                   [0.4 / 0.7, 0.3 / 0.7, 0.2 / 0.7]], rtol=1e-15)
    np.testing.assert_allclose(mo.candidate_gates(p, cand, 2, False),
                               [[0.5, 0.2, 0.2], [0.4, 0.3, 0.2]], rtol=1e-15)
    # the first k columns are the top-k gates
    np.testing.assert_allclose(g[:, :2], mo.gates(p, cand[:, :2], True), rtol=1e-15)
    sg = mo.served_gates(g, np.array([[0, -1], [2, 1]]))
    np.testing.assert_allclose(sg, [[0.5 / 0.7, 0.0], [0.2 / 0.7, 0.3 / 0.7]], rtol=1e-15)


def test_candidate_gates():
    check_candidate_gates()


def test_rerouted_layer_reduces_to_plain_layer():
    """rounds = 0 with token priority is the plain layer; with rounds > 0 an
    assignment served by its next candidate adds that expert's FFN with the
    candidate's weight (checked token by token)."""
    r = rng(31)
    T, d, d_ff, E, k, C = 40, 6, 10, 4, 2, 12
    x = r.standard_normal((T, d))
    W_r = r.standard_normal((E, d))
    b_r = np.array([2.0, 0.0, 0.0, 0.0])      # expert 0 is hot: it overflows
    W1 = r.standard_normal((E, d_ff, d))
    b1 = r.standard_normal((E, d_ff))
    W2 = r.standard_normal((E, d, d_ff))
    b2 = r.standard_normal((E, d))
    kw = dict(k=k, C=C, renormalize=True, act="relu")
    plain = mo.layer_forward(x, W_r, b_r, W1, b1, W2, b2, **kw)
    same = mo.layer_forward(x, W_r, b_r, W1, b1, W2, b2, priority="token", rounds=0, **kw)
    np.testing.assert_array_equal(plain["y"], same["y"])
    o = mo.layer_forward(x, W_r, b_r, W1, b1, W2, b2, rounds=1, **kw)
    assert o["kept"].sum() > plain["kept"].sum()
    p = mo.softmax(mo.router_logits(x, W_r, b_r))
    for t in range(T):
        top = np.sort(p[t])[::-1][:k].sum()
        want = np.zeros(d)
        for q in range(k):
            e = o["served_ids"][t, q]
            if e >= 0:
                _, Y = mo.expert_ffn(x[t:t + 1], W1[e], b1[e], W2[e], b2[e], "relu")
                want += p[t, e] / top * Y[0]
        np.testing.assert_allclose(o["y"][t], want, rtol=1e-12, atol=1e-12)


def test_planted_reroute_same_column_is_caught(monkeypatch):
    """A re-route that offers the same expert again must fail the pins."""
    orig = mo.dispatch_rerouted

    def no_advance(cand, k, E, C, priority="token", rounds=0):
        return orig(np.concatenate([cand[:, :k]] * (cand.shape[1] // k + 1), axis=1)[:, :cand.shape[1]],
                    k, E, C, priority, rounds)
    monkeypatch.setattr(mo, "dispatch_rerouted", no_advance)
    _expect_fail(check_reroute_pages)


def test_planted_priority_ignored_is_caught(monkeypatch):
    orig = mo.dispatch_rerouted
    monkeypatch.setattr(mo, "dispatch_rerouted",
                        lambda cand, k, E, C, priority="token", rounds=0: orig(cand, k, E, C, "token", rounds))
    _expect_fail(check_reroute_pages)


def test_planted_candidate_gate_denominator_is_caught(monkeypatch):
    orig = mo.candidate_gates
    monkeypatch.setattr(mo, "candidate_gates",
                        lambda p, cand, k, renormalize: orig(p, cand, cand.shape[1], renormalize))
    _expect_fail(check_candidate_gates)


# ------------------------------------------------------------------ backward

def small_layer(seed, T=24, d=6, d_ff=10, E=4, k=2, hot=1.5):
    r = rng(seed)
    x = r.standard_normal((T, d))
    W_r = r.standard_normal((E, d))
    b_r = np.zeros(E)
    b_r[0] = hot                      # expert 0 overflows at small C
    W1 = r.standard_normal((E, d_ff, d)) / math.sqrt(d)
    b1 = 0.1 * r.standard_normal((E, d_ff))
    W2 = r.standard_normal((E, d, d_ff)) / math.sqrt(d_ff)
    b2 = 0.1 * r.standard_normal((E, d))
    dy = r.standard_normal((T, d))
    return dict(x=x, W_r=W_r, b_r=b_r, W1=W1, b1=b1, W2=W2, b2=b2), dy


def check_backward_finite_differences(act="gelu_tanh", renormalize=True, alpha=0.3, C=9,
                                      priority="token", seed=41):
    """<grad, v> against a central difference of the forward's scalar loss
    along a random direction v, for every input and parameter tensor; the
    routing and capacity decisions do not change within +-eps."""
    P, dy = small_layer(seed)
    kw = dict(k=2, C=C, renormalize=renormalize, act=act, alpha=alpha, priority=priority)
    g = mo.layer_backward(P["x"], P["W_r"], P["b_r"], P["W1"], P["b1"], P["W2"], P["b2"], dy, **kw)
    assert 0 < g["fwd"]["rows"] < 24 * 2          # some drops, some kept
    names = {"x": "dx", "W_r": "dW_r", "b_r": "db_r", "W1": "dW1", "b1": "db1", "W2": "dW2",
             "b2": "db2"}
    r = rng(seed + 1)
    eps = 1e-6
    for name, gname in names.items():
        v = r.standard_normal(P[name].shape)
        plus, minus = dict(P), dict(P)
        plus[name] = P[name] + eps * v
        minus[name] = P[name] - eps * v
        args_p = [plus[n] for n in ("x", "W_r", "b_r", "W1", "b1", "W2", "b2")]
        args_m = [minus[n] for n in ("x", "W_r", "b_r", "W1", "b1", "W2", "b2")]
        fp = mo.layer_forward(*args_p, k=2, C=C, renormalize=renormalize, act=act, priority=priority)
        fm = mo.layer_forward(*args_m, k=2, C=C, renormalize=renormalize, act=act, priority=priority)
        assert np.array_equal(fp["row_of"], g["fwd"]["row_of"]) and np.array_equal(fm["row_of"], g["fwd"]["row_of"])
        fd = (mo.layer_loss(*args_p, dy, **kw) - mo.layer_loss(*args_m, dy, **kw)) / (2 * eps)
        an = float(np.sum(g[gname] * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_backward_finite_differences():
    check_backward_finite_differences()


@pytest.mark.parametrize("act,renormalize,alpha,priority", [
    ("relu", False, 0.0, "token"), ("gelu_tanh", True, 0.0, "rank"), ("relu", True, 1.0, "token")])
def test_backward_finite_differences_variants(act, renormalize, alpha, priority):
    check_backward_finite_differences(act=act, renormalize=renormalize, alpha=alpha,
                                      priority=priority, seed=43)


def torch_layer_loss(P, dy, ids, row_kept, k, renormalize, act, alpha, counts):
    """The same scalar loss written with torch ops (fp64) from the layer's
    definition, for autograd: the routing decisions are given."""
    x, W_r, b_r = P["x"], P["W_r"], P["b_r"]
    s = x @ W_r.T + b_r
    p = torch.softmax(s, dim=1)
    chosen = torch.gather(p, 1, ids)
    g = chosen / chosen.sum(dim=1, keepdim=True) if renormalize else chosen
    y = torch.zeros_like(x)
    T = x.shape[0]
    for j in range(k):
        e_j = ids[:, j]
        u = torch.einsum("tfd,td->tf", P["W1"][e_j], x) + P["b1"][e_j]
        hh = torch.nn.functional.gelu(u, approximate="tanh") if act == "gelu_tanh" else torch.relu(u)
        Y = torch.einsum("tdf,tf->td", P["W2"][e_j], hh) + P["b2"][e_j]
        y = y + (g[:, j] * row_kept[:, j])[:, None] * Y
    E = W_r.shape[0]
    aux = alpha * E * torch.sum((counts / T) * (p.sum(dim=0) / T))
    return torch.sum(dy * y) + aux


def test_backward_against_autograd():
    P, dy = small_layer(47, T=30, E=5)
    for act, renorm, alpha in [("gelu_tanh", True, 0.5), ("relu", False, 0.0)]:
        g = mo.layer_backward(P["x"], P["W_r"], P["b_r"], P["W1"], P["b1"], P["W2"], P["b2"], dy,
                              k=2, C=8, renormalize=renorm, act=act, alpha=alpha)
        f = g["fwd"]
        tp = {n: torch.tensor(v, dtype=torch.float64, requires_grad=True) for n, v in P.items()}
        ids = torch.tensor(f["used_ids"], dtype=torch.int64)
        kept = torch.tensor(f["row_of"] >= 0, dtype=torch.float64)
        counts = torch.tensor(f["expert_counts"], dtype=torch.float64)
        L = torch_layer_loss(tp, torch.tensor(dy), ids, kept, 2, renorm, act, alpha, counts)
        L.backward()
        for n, gn in [("x", "dx"), ("W_r", "dW_r"), ("b_r", "db_r"), ("W1", "dW1"), ("b1", "db1"),
                      ("W2", "dW2"), ("b2", "db2")]:
            np.testing.assert_allclose(g[gn], tp[n].grad.numpy(), rtol=1e-10, atol=1e-12,
                                       err_msg=f"{act} {n}")


def test_backward_single_expert_is_dense_mlp():
    """E = 1, k = 1, C >= T: the layer is a dense MLP; its router sees a
    softmax over one expert (constant 1), so the router gradients vanish."""
    P, dy = small_layer(53, T=12, E=1, k=1, hot=0.0)
    g = mo.layer_backward(P["x"], P["W_r"], P["b_r"], P["W1"], P["b1"], P["W2"], P["b2"], dy,
                          k=1, C=12, renormalize=True, act="gelu_tanh", alpha=0.7)
    x = torch.tensor(P["x"], requires_grad=True)
    W1 = torch.tensor(P["W1"][0], requires_grad=True)
    b1 = torch.tensor(P["b1"][0], requires_grad=True)
    W2 = torch.tensor(P["W2"][0], requires_grad=True)
    b2 = torch.tensor(P["b2"][0], requires_grad=True)
    F = torch.nn.functional
    y = F.linear(F.gelu(F.linear(x, W1, b1), approximate="tanh"), W2, b2)
    torch.sum(torch.tensor(dy) * y).backward()
    np.testing.assert_allclose(g["dx"], x.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dW1"][0], W1.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["db1"][0], b1.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dW2"][0], W2.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["db2"][0], b2.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.abs(g["dW_r"]).max() < 1e-14 and np.abs(g["db_r"]).max() < 1e-14


def test_planted_missing_activation_grad_is_caught(monkeypatch):
    monkeypatch.setitem(mo.ACT_GRADS, "gelu_tanh", lambda u: np.ones_like(u))
    _expect_fail(check_backward_finite_differences)


def test_planted_renorm_grad_sign_is_caught(monkeypatch):
    orig = mo.layer_backward

    def flipped(*a, **kw):
        out = orig(*a, **kw)
        out["db_r"] = -out["db_r"]
        return out
    monkeypatch.setattr(mo, "layer_backward", flipped)
    _expect_fail(check_backward_finite_differences)


def test_planted_missing_aux_grad_is_caught(monkeypatch):
    orig = mo.layer_backward
    monkeypatch.setattr(mo, "layer_backward", lambda *a, **kw: orig(*a, **{**kw, "alpha": 0.0}))
    _expect_fail(check_backward_finite_differences)


def test_load_stats_counts_assignments():
    """Top-2 over 2 experts: every token holds both, so the 4 tokens make 8
    assignments; C = 3 drops one per expert, 2 of the 8 (a ratio over tokens
    would read 2 / 4)."""
    s = mo.load_stats([4, 4], 3, 4, 2)
    assert s["dropped"] == 2 and s["overflow_ratio"] == 0.25
    assert s["padding_ratio"] == 1.0 and s["max_over_mean_load"] == 1.0
