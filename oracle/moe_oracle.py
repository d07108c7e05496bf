"""Plain fp64 CPU oracle for the MoE layer forward pass.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. It shares no code with the HIP
library and never imports it.

Every function follows one passage of the pages and is written to be read
against it, not to be fast. Floating point is fp64 throughout; stored bf16
values are widened exactly (a bf16 bit pattern is the top half of an fp32).
Nothing is rounded in between, except the one place where floating point
decides an integer (the top-k choice), which is taken on logits rounded to
fp32, the precision the GPU kernel decides in.

Sources, cited by short name:
  [MoE Principles]   wrblog.cn, "MoE 模型原理：路由、专家负载、容量、通信与推理成本"
                     (MoE principles: routing, expert load, capacity,
                     communication and inference cost), sections 1-14.
  [EP Token->Expert] 111qqz.com, "Expert Parallelism：为什么让 Token 去找 Expert，
                     而不是搬运参数？", cited by section heading.
  [Gate&Comm]        mianshidashi.cn, MiniMax interview answer on MoE gate
                     outputs and distributed communication, "深入解析" items 01-06.
  [EP 001]           ai-master.cc, interview answer "moe-expert-parallelism-
                     engineering-001", section 一 (load balance: capacity factor).

Readings where the pages leave a step open (each one is also listed with its
reason in the design notes):
  R1  top-k selects on the logits s (softmax is strictly increasing, so the
      chosen set equals TopK(p)); ids come in descending-score order and
      equal scores go to the lower expert index.
  R2  gate = renormalised top-k probability when `renormalize`, else the
      plain softmax probability (the page's top-1 toy).
  R3  gates are not renormalised again after capacity drops; a dropped
      assignment contributes zero and a token with every assignment dropped
      outputs exactly zero (the residual lies outside the layer).
  R4  capacity C = ceil(c*T*k/E) of the exact value of c (a binary float), for
      the whole call as one routing group.
  R5  capacity is granted first-come in token order; a token's own k choices
      never compete (they go to distinct experts).
  R6  f_i counts assignments before capacity.
  R7  dispatch layout: expert-major, token order within an expert, rows
      packed from 0 (no padding to C).
  R8  tanh-GELU is 0.5*u*(1 + tanh(sqrt(2/pi)*(u + 0.044715*u^3))) (Hendrycks &
      Gimpel's published approximation; the pages do not define sigma). Its
      constants are "parity unpinned" by the pages: they are pinned only
      against an independent library implementation and the exact GELU.
  R9  overflow re-routing ([MoE Principles §4.3], second option; [EP 001]
      section 一, overflow may go to the next-best expert): an assignment that overflows moves
      to the token's next candidate, the best-scoring expert the token has
      not yet been offered; it is served with that expert's probability as
      its weight (divided by the same top-k sum when renormalising).
  R10 capacity is allocated candidate by candidate, in rounds: round 0
      offers every top-k assignment and truncates each expert at C; round j
      offers the assignments still unplaced to their next candidates, which
      take what capacity round j-1 left. Inside a round, arrivals are served
      in priority order: token order (t, then rank r) or, GShard-style, rank
      order (every token's first choice before any second choice).
  R11 backward: the top-k choice and the capacity decisions are held fixed
      (a discrete choice has no gradient, [MoE Principles §2.4]); gradients
      reach the router through the combine weights of the kept assignments
      and, when alpha > 0, through pbar in L_aux (f_i is a count, constant)
      [MoE Principles §3.2]. The scalar differentiated is
      L = <dy, y> + L_aux.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

ORACLE_VERSION = 1

NEAR_TIE_REL = 1e-6


# ---------------------------------------------------------------- storage

def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values -> exact fp64. `a` is uint16 bit patterns for bf16,
    float32 for f32."""
    if dtype == "bf16":
        a = np.ascontiguousarray(a, dtype=np.uint16)
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def round_f32(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float32)


# ---------------------------------------------------------------- capacity

def capacity(T: int, k: int, E: int, c: float) -> int:
    """C = ceil(c * T * k / E)  [MoE Principles §4.1, capacity formula;
    EP Token->Expert, "Expert Capacity 和 Token Dropping"].

    Fraction(c) is the exact value of the float c (reading R4)."""
    return math.ceil(Fraction(c) * T * k / E)


# ---------------------------------------------------------------- routing

def router_logits(x: np.ndarray, W_r: np.ndarray, b_r: np.ndarray) -> np.ndarray:
    """s_t = W_r x_t + b_r for every token  [MoE Principles §2.1].

    x [T, d], W_r [E, d], b_r [E], all fp64 -> s [T, E]."""
    return x @ W_r.T + b_r[None, :]


def softmax(s: np.ndarray) -> np.ndarray:
    """p_{t,i} = exp(s_{t,i}) / sum_j exp(s_{t,j})  [MoE Principles §2.1].

    The row maximum is subtracted first; the quotient is unchanged."""
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)


def topk_ids(s: np.ndarray, k: int) -> np.ndarray:
    """S_t = TopK(p_t, k)  [MoE Principles §2.2], reading R1.

    The decision is taken on the logits rounded to fp32. A stable sort of the
    negated scores lists higher scores first and, among equal scores, lower
    expert indices first. Returns int32 [T, k]."""
    s32 = round_f32(s)
    order = np.argsort(-s32, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def gates(p: np.ndarray, ids: np.ndarray, renormalize: bool) -> np.ndarray:
    """Combine weights of the chosen experts  [MoE Principles §2.2]:
    p~_{t,i} = p_{t,i} / sum_{j in S_t} p_{t,j} when renormalising (reading R2),
    else p_{t,i} as the page's top-1 example uses it  [MoE Principles §7]."""
    chosen = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    if renormalize:
        return chosen / chosen.sum(axis=1, keepdims=True)
    return chosen


def near_ties(s: np.ndarray, k: int, rel: float = NEAR_TIE_REL) -> np.ndarray:
    """Tokens whose top-k decision is fragile: some gap between neighbouring
    sorted logits at ranks (r, r+1), r < k, is below rel * max_i |s_{t,i}|.
    Returns bool [T]."""
    T, E = s.shape
    srt = -np.sort(-s, axis=1)
    scale = np.abs(s).max(axis=1)
    fragile = np.zeros(T, dtype=bool)
    for r in range(min(k, E - 1)):
        fragile |= (srt[:, r] - srt[:, r + 1]) < rel * scale
    return fragile


def route(x, W_r, b_r, k: int, renormalize: bool) -> dict:
    """Router, softmax, top-k and gates on fp64 inputs."""
    s = router_logits(x, W_r, b_r)
    p = softmax(s)
    ids = topk_ids(s, k)
    return {"logits": s, "probs": p, "topk_ids": ids,
            "topk_gates": gates(p, ids, renormalize),
            "prob_sum": p.sum(axis=0), "near_tie": near_ties(s, k)}


# ---------------------------------------------------------------- dispatch

def dispatch(ids: np.ndarray, E: int, C: int) -> dict:
    """Capacity assignment and the expert-contiguous layout.

    count_e   = |{t : e in S_t}|                       [MoE Principles §3.2, f_i]
    slot(t,e) = |{t' < t : e in S_t'}|  (first come, token order)
    kept      = slot < C        [MoE Principles §4.2 worked example; reading R5]
    n_e       = min(count_e, C);  offset_e = sum_{e' < e} n_e'   (reading R7)
    row_of    = offset_e + slot if kept else -1
    row_token[offset_e + s] = the token holding slot s of expert e
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    member = np.zeros((T, E), dtype=np.int64)          # member[t, e] = [e in S_t]
    np.put_along_axis(member, ids, 1, axis=1)
    before = np.cumsum(member, axis=0) - member         # tokens t' < t holding e
    counts = member.sum(axis=0)
    slot = np.take_along_axis(before, ids, axis=1)
    kept = slot < C
    n = np.minimum(counts, C)
    offsets = np.concatenate([[0], np.cumsum(n)])
    row_of = np.where(kept, offsets[ids] + slot, -1)
    rows = int(offsets[-1])
    row_token = np.full(rows, -1, dtype=np.int64)
    tt = np.broadcast_to(np.arange(T)[:, None], (T, k))
    row_token[row_of[kept]] = tt[kept]
    return {"expert_counts": counts.astype(np.int32), "n": n.astype(np.int32),
            "expert_offsets": offsets.astype(np.int32), "slot": slot.astype(np.int32),
            "kept": kept, "row_of": row_of.astype(np.int32),
            "row_token": row_token.astype(np.int32), "rows": rows}


def candidate_ids(s: np.ndarray, n: int) -> np.ndarray:
    """Each token's n best experts in descending score order: the top-k list
    followed by the next candidates an overflowing assignment may move to
    [MoE Principles §4.3]; same decision rule as top-k (reading R1)."""
    return topk_ids(s, n)


def candidate_gates(p: np.ndarray, cand: np.ndarray, k: int, renormalize: bool) -> np.ndarray:
    """Weight of every candidate column (reading R9): p_{t,c} divided by the
    sum over the token's top-k when renormalising, else p_{t,c}. The first k
    columns equal `gates`."""
    chosen = np.take_along_axis(p, cand.astype(np.int64), axis=1)
    if renormalize:
        return chosen / chosen[:, :k].sum(axis=1, keepdims=True)
    return chosen


def dispatch_rerouted(cand: np.ndarray, k: int, E: int, C: int, priority: str = "token",
                      rounds: int = 0) -> dict:
    """Capacity assignment with a priority order and overflow re-routing,
    readings R9 and R10, written as the sequential process it describes.

    cand [T, n] holds each token's candidates (columns 0..k-1 = S_t). Round 0
    offers assignment (t, r) to cand[t, r]. Before round j >= 1, each
    still-unplaced assignment of token t, in rank order, takes the token's
    next unused candidate column (columns k, k+1, ...; with none left the
    assignment is dropped for good). In every round, arrivals at an expert
    are served in priority order while its capacity lasts:
      priority "token": (t, r) in token order, ranks inside a token;
      priority "rank":  (r, t): all first choices, then all second choices...
    An arrival's slot is its position in the expert's arrival order: the
    expert's fill at the start of the round plus the arrivals before it in
    this round; it is placed iff slot < C. Placed rows are laid out expert
    by expert in slot order (round 0 arrivals first).

    With rounds = 0 and priority "token" this is exactly `dispatch`.
    Returns the fields of `dispatch` (slot = slot at the expert last tried)
    plus served_col [T, k] (candidate column serving each assignment, -1 if
    dropped) and served_ids [T, k] (its expert, -1 if dropped)."""
    cand = np.asarray(cand, dtype=np.int64)
    T, n = cand.shape
    assert priority in ("token", "rank") and rounds >= 0 and n >= k
    if priority == "token":
        order = [(t, r) for t in range(T) for r in range(k)]
    else:
        order = [(t, r) for r in range(k) for t in range(T)]
    col = [[r for r in range(k)] for _ in range(T)]   # column each assignment tries
    next_col = [k] * T
    served = [[-1] * k for _ in range(T)]
    alive = [[True] * k for _ in range(T)]
    slot = [[0] * k for _ in range(T)]
    fill = [0] * E
    counts = [0] * E
    for rnd in range(rounds + 1):
        if rnd > 0:
            for t in range(T):
                for r in range(k):
                    if served[t][r] < 0 and alive[t][r]:
                        if next_col[t] < n:
                            col[t][r] = next_col[t]
                            next_col[t] += 1
                        else:
                            alive[t][r] = False
        arrived = list(fill)
        for t, r in order:
            if served[t][r] >= 0 or not alive[t][r]:
                continue
            e = int(cand[t, col[t][r]])
            if rnd == 0:
                counts[e] += 1
            slot[t][r] = arrived[e]
            arrived[e] += 1
            if slot[t][r] < C:
                served[t][r] = col[t][r]
        fill = [min(a, C) for a in arrived]
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + fill[e])
    rows = offsets[-1]
    row_of = np.full((T, k), -1, dtype=np.int64)
    served_ids = np.full((T, k), -1, dtype=np.int64)
    row_token = np.full(rows, -1, dtype=np.int64)
    for t in range(T):
        for r in range(k):
            if served[t][r] >= 0:
                e = int(cand[t, served[t][r]])
                served_ids[t, r] = e
                row_of[t, r] = offsets[e] + slot[t][r]
                row_token[row_of[t, r]] = t
    served_col = np.array(served, dtype=np.int64).reshape(T, k)
    return {"expert_counts": np.array(counts, dtype=np.int32),
            "n": np.array(fill, dtype=np.int32),
            "expert_offsets": np.array(offsets, dtype=np.int32),
            "slot": np.array(slot, dtype=np.int32).reshape(T, k), "kept": served_col >= 0,
            "row_of": row_of.astype(np.int32), "row_token": row_token.astype(np.int32),
            "rows": rows, "served_col": served_col.astype(np.int32),
            "served_ids": served_ids.astype(np.int32)}


def served_gates(cand_gates: np.ndarray, served_col: np.ndarray) -> np.ndarray:
    """Combine weight of each assignment: the weight of the candidate that
    serves it (reading R9), 0 for a dropped one."""
    col = np.maximum(served_col, 0).astype(np.int64)
    g = np.take_along_axis(cand_gates, col, axis=1)
    return np.where(served_col >= 0, g, 0.0)


def permute(x: np.ndarray, row_token: np.ndarray) -> np.ndarray:
    """x_perm[r] = x[row_token[r]]: tokens gathered expert by expert
    [MoE Principles §5; Gate&Comm 02, 06]. Works on stored values (a copy)."""
    return x[np.asarray(row_token, dtype=np.int64)]


# ---------------------------------------------------------------- experts

def gelu_tanh(u: np.ndarray) -> np.ndarray:
    """Reading R8 (parity unpinned by the pages)."""
    return 0.5 * u * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (u + 0.044715 * u ** 3)))


def relu(u: np.ndarray) -> np.ndarray:
    return np.maximum(u, 0.0)


ACTS = {"relu": relu, "gelu_tanh": gelu_tanh}


def expert_ffn(x_rows, W1_e, b1_e, W2_e, b2_e, act: str):
    """FFN(x) = W2 sigma(W1 x + b1) + b2  [MoE Principles §1], row by row.

    x_rows [n, d]; W1_e [d_ff, d] maps d -> d_ff; W2_e [d, d_ff] maps back.
    Returns (h [n, d_ff], Y [n, d])."""
    h = ACTS[act](x_rows @ W1_e.T + b1_e[None, :])
    return h, h @ W2_e.T + b2_e[None, :]


def combine(Y_rows: np.ndarray, row_of: np.ndarray, g: np.ndarray) -> np.ndarray:
    """y_t = sum_{i in S_t, kept} p~_{t,i} E_i(x_t)  [MoE Principles §2.2, §5];
    dropped assignments add nothing (reading R3). Y_rows is indexed by row."""
    T, k = row_of.shape
    y = np.zeros((T, Y_rows.shape[1]), dtype=np.float64)
    for j in range(k):
        keep = row_of[:, j] >= 0
        y[keep] += g[keep, j][:, None] * Y_rows[row_of[keep, j]]
    return y


# ---------------------------------------------------------------- whole layer

def layer_forward(x, W_r, b_r, W1, b1, W2, b2, *, k: int, C: int, renormalize: bool,
                  act: str, ids=None, priority: str = "token", rounds: int = 0) -> dict:
    """The whole hot path on fp64 inputs  [MoE Principles §5 flowchart]:
    router -> probabilities -> top-k -> capacity assignment -> dispatch ->
    expert FFNs -> combine.

    W1 [E, d_ff, d], W2 [E, d, d_ff], b1 [E, d_ff], b2 [E, d]. When `ids` is
    given, dispatch and everything after it use those expert ids (with
    re-routing: those candidate lists) instead of the oracle's own choice
    (used when the GPU took the other side of a near-tie). `priority` and
    `rounds` select the capacity rule of readings R9 and R10; the defaults
    are the plain first-come, drop-on-overflow rule."""
    E = W_r.shape[0]
    general = priority != "token" or rounds > 0
    n_cand = min(E, k * (1 + rounds)) if rounds > 0 else k
    r = route(x, W_r, b_r, n_cand, renormalize) if general else route(x, W_r, b_r, k, renormalize)
    use_ids = r["topk_ids"] if ids is None else np.asarray(ids, dtype=np.int32)
    if general:
        cg = candidate_gates(r["probs"], use_ids, k, renormalize)
        dsp = dispatch_rerouted(use_ids, k, E, C, priority, rounds)
        g = served_gates(cg, dsp["served_col"])
        r["topk_gates"] = cg
    else:
        g = r["topk_gates"] if ids is None else gates(r["probs"], use_ids, renormalize)
        dsp = dispatch(use_ids, E, C)
    rows = dsp["rows"]
    x_perm = permute(x, dsp["row_token"])
    h = np.zeros((rows, W1.shape[1]), dtype=np.float64)
    Y = np.zeros((rows, x.shape[1]), dtype=np.float64)
    off = dsp["expert_offsets"]
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if b > a:
            h[a:b], Y[a:b] = expert_ffn(x_perm[a:b], W1[e], b1[e], W2[e], b2[e], act)
    y = combine(Y, dsp["row_of"], g)
    out = dict(r)
    out.update(dsp)
    out.update({"used_ids": use_ids, "used_gates": g, "x_perm": x_perm, "h": h,
                "y_perm": Y, "y": y})
    return out


def sampled_outputs(tokens, x, ids, row_of, g, expert_weights, act: str) -> np.ndarray:
    """y_t for a few tokens only, one token and one expert at a time, for the
    full-size workloads where the oracle cannot afford every row: for each
    kept assignment (t, j) the FFN of expert ids[t, j] on x_t, weighted by
    g[t, j]  [MoE Principles §2.2 output formula].

    `expert_weights(e)` returns (W1_e, b1_e, W2_e, b2_e) in fp64; each expert's
    weights are fetched once (the pairs are visited expert by expert)."""
    out = np.zeros((len(tokens), x.shape[1]), dtype=np.float64)
    pairs = {}
    for n, t in enumerate(tokens):
        for j in range(ids.shape[1]):
            if row_of[t, j] >= 0:
                pairs.setdefault(int(ids[t, j]), []).append((n, t, j))
    for e in sorted(pairs):
        W1e, b1e, W2e, b2e = expert_weights(e)
        for n, t, j in pairs[e]:
            _, Y = expert_ffn(x[t:t + 1], W1e, b1e, W2e, b2e, act)
            out[n] += g[t, j] * Y[0]
    return out


# ---------------------------------------------------------------- backward

def gelu_tanh_grad(u: np.ndarray) -> np.ndarray:
    """d/du of gelu_tanh: 0.5 (1 + tanh z) + 0.5 u (1 - tanh^2 z) dz/du with
    z = a (u + b u^3), dz/du = a (1 + 3 b u^2)  (reading R8's function)."""
    a = math.sqrt(2.0 / math.pi)
    b = 0.044715
    th = np.tanh(a * (u + b * u ** 3))
    return 0.5 * (1.0 + th) + 0.5 * u * (1.0 - th * th) * a * (1.0 + 3.0 * b * u * u)


def relu_grad(u: np.ndarray) -> np.ndarray:
    return (u > 0).astype(np.float64)


ACT_GRADS = {"relu": relu_grad, "gelu_tanh": gelu_tanh_grad}


def layer_backward(x, W_r, b_r, W1, b1, W2, b2, dy, *, k: int, C: int, renormalize: bool,
                   act: str, alpha: float = 0.0, ids=None, priority: str = "token") -> dict:
    """Gradients of L = <dy, y> + L_aux with respect to x and every parameter,
    by the chain rule through the forward's steps (reading R11):

      dY_r   = g_{t,j} dy_t                    for each kept row r = row_of[t, j]
      dg_tj  = <dy_t, Y_r>                     (0 for a dropped assignment)
      dh     = dY W2_e;  du = dh * sigma'(u)   u = x_perm W1_e^T + b1_e
      dW2_e  = dY_e^T h_e, db2_e = sum_r dY_r; dW1_e = du_e^T x_perm_e, db1_e = sum_r du_r
      dx_t  += sum_j du_{row_of[t,j]} W1_e
      router: gates g = p_i / P (renormalised, P = sum over S_t) or p_i, so
        dp_i = (dg_i - sum_j dg_j g_j) / P  or  dg_i  for i in S_t;
        L_aux adds alpha E f_i / T to dp_{t,i} for every t, i;
        ds = p * (dp - sum_j p_j dp_j)  (softmax);
        dW_r = ds^T x, db_r = sum_t ds_t, dx_t += ds_t W_r.

    Works for the plain and rank-priority rules (both keep the top-k gates).
    Returns fp64 arrays dx [T,d], dW_r, db_r, dW1, db1, dW2, db2 and the
    forward dict under "fwd"."""
    T, d = x.shape
    E = W_r.shape[0]
    fwd = layer_forward(x, W_r, b_r, W1, b1, W2, b2, k=k, C=C, renormalize=renormalize,
                        act=act, ids=ids, priority=priority)
    use_ids = np.asarray(fwd["used_ids"], dtype=np.int64)[:, :k]
    g = fwd["used_gates"]
    row_of = fwd["row_of"]
    off = fwd["expert_offsets"]
    x_perm, h, Y = fwd["x_perm"], fwd["h"], fwd["y_perm"]
    rows = fwd["rows"]
    dY = np.zeros((rows, d))
    dg = np.zeros((T, k))
    for t in range(T):
        for j in range(k):
            r = row_of[t, j]
            if r >= 0:
                dY[r] = g[t, j] * dy[t]
                dg[t, j] = float(np.dot(dy[t], Y[r]))
    dx = np.zeros((T, d))
    dW1, db1 = np.zeros_like(W1), np.zeros_like(b1)
    dW2, db2 = np.zeros_like(W2), np.zeros_like(b2)
    dx_perm = np.zeros((rows, d))
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if b == a:
            continue
        u = x_perm[a:b] @ W1[e].T + b1[e][None, :]
        dh = dY[a:b] @ W2[e]
        du = dh * ACT_GRADS[act](u)
        dW2[e] = dY[a:b].T @ h[a:b]
        db2[e] = dY[a:b].sum(axis=0)
        dW1[e] = du.T @ x_perm[a:b]
        db1[e] = du.sum(axis=0)
        dx_perm[a:b] = du @ W1[e]
    for t in range(T):
        for j in range(k):
            r = row_of[t, j]
            if r >= 0:
                dx[t] += dx_perm[r]
    # router
    p = fwd["probs"]
    dp = np.zeros((T, E))
    chosen = np.take_along_axis(p, use_ids, axis=1)
    if renormalize:
        P = chosen.sum(axis=1, keepdims=True)
        gg = chosen / P
        inner = (dg * gg).sum(axis=1, keepdims=True)
        np.put_along_axis(dp, use_ids, (dg - inner) / P, axis=1)
    else:
        np.put_along_axis(dp, use_ids, dg, axis=1)
    if alpha != 0.0:
        f = np.asarray(fwd["expert_counts"], dtype=np.float64) / T
        dp += alpha * E * f[None, :] / T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dW_r = ds.T @ x
    db_r = ds.sum(axis=0)
    dx += ds @ W_r
    return {"dx": dx, "dW_r": dW_r, "db_r": db_r, "dW1": dW1, "db1": db1, "dW2": dW2,
            "db2": db2, "dg": dg, "ds": ds, "fwd": fwd}


def layer_loss(x, W_r, b_r, W1, b1, W2, b2, dy, *, k: int, C: int, renormalize: bool, act: str,
               alpha: float = 0.0, ids=None, priority: str = "token") -> float:
    """The scalar L = <dy, y> + L_aux that layer_backward differentiates."""
    o = layer_forward(x, W_r, b_r, W1, b1, W2, b2, k=k, C=C, renormalize=renormalize, act=act,
                      ids=ids, priority=priority)
    T, E = x.shape[0], W_r.shape[0]
    return float(np.sum(dy * o["y"])) + aux_loss(o["expert_counts"], o["prob_sum"], T, E, alpha)


# ---------------------------------------------------------------- statistics

def aux_loss(counts, prob_sum, T: int, E: int, alpha: float) -> float:
    """L_aux = alpha * E * sum_i f_i * pbar_i with f_i = count_i / T and
    pbar_i = (1/T) sum_t p_{t,i}  [MoE Principles §3.2; reading R6]."""
    f = np.asarray(counts, dtype=np.float64) / T
    pbar = np.asarray(prob_sum, dtype=np.float64) / T
    return alpha * E * float(np.sum(f * pbar))


def load_stats(counts, C: int, T: int, k: int, prob_sum=None, alpha: float = 1.0) -> dict:
    """What the pages ask to log per routing step  [MoE Principles §3.3: tokens
    and drops per expert, max/mean load; §13: tokens per expert, overflow
    ratio, padding ratio; EP 001, follow-up 2: entropy of the expert
    activation distribution and the variance of the tokens each expert
    actually processes].

    overflow_ratio = dropped assignments / (T k); max_over_mean_load = max /
    mean of the routed counts; padding_ratio = E C / kept rows (a padded
    [E, C] layout against the rows kept); load_entropy = -sum_i f_i ln f_i
    over the routed shares f_i = count_i / sum(count); kept_variance = the
    population variance of min(count_i, C). With prob_sum, aux_loss is
    L_aux of §3.2 (aux_loss below) with the given alpha."""
    counts = np.asarray(counts, dtype=np.int64)
    E = counts.size
    kept = np.minimum(counts, C)
    dropped = counts - kept
    frac = counts / max(1, counts.sum())
    nz = frac[frac > 0]
    out = {
        "tokens_per_expert": counts.tolist(),
        "kept_per_expert": kept.tolist(),
        "dropped_per_expert": dropped.tolist(),
        "dropped": int(dropped.sum()),
        "overflow_ratio": float(dropped.sum() / max(1, T * k)),
        "max_over_mean_load": float(counts.max() / max(1e-300, counts.mean())) if E else 0.0,
        "padding_ratio": float(E * C / max(1, kept.sum())),
        "load_entropy": float(-(nz * np.log(nz)).sum()),
        "kept_variance": float(np.mean((kept - kept.mean()) ** 2)) if E else 0.0,
    }
    if prob_sum is not None:
        out["aux_loss"] = aux_loss(counts, prob_sum, T, E, alpha)
    return out


def ffn_flops(rows: int, d: int, d_ff: int) -> int:
    """4 * d * d_ff per kept (token, expert) pair  [MoE Principles §8.3]."""
    return 4 * d * d_ff * rows
