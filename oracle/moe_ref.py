"""Plain fp64 CPU oracle of the dropless MoE layer, forward and backward.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
use this module; the GPU library never imports or calls it, and it shares no code with the GPU
path.  It is written for clarity, not speed: one Python loop over experts, the shape of the
per-expert Python-loop baseline described on the TE page (below), with numpy matmuls in fp64.

Pages cited (title as published; section headings translated in brackets):
  [Prime]  "Prime Mega MoE: tanításra is jó a DeepSeek MoE kernele" (neuraldaily.news)
  [JAX]    "Az NVIDIA szerint tízszer gyorsabb lett a dropless MoE tanítása JAX-ban" (aihirek.info)
  [TE]     "NVIDIA מציגה דרך יעילה לאמן מודלי MoE בביולוגיה" (sitech.ge)
  [Mega]   the DeepGEMM "Mega MoE" announcement on itsolotime.com (Thai)

What is computed, and where the pages state it:
  route    a learned router sends each token to its top-k experts ([JAX] "A dropless MoE minden
           tokent feldolgoz" [dropless MoE processes every token]).  The pages give no formula:
           slot j holds the j-th largest logit, ties go to the lower expert id, and the routing
           weights are the softmax over the k kept logits.
  plan     ragged per-expert groups ([JAX] "Az egyenetlen terhelés lassítja a tanítást" [uneven
           load slows training]; per-expert token counts given as split sizes, [TE] "מומחים
           מקובצים במקום לולאת Python" [grouped experts instead of a Python loop]): counts,
           exclusive offsets, and a stable counting sort of the (token, slot) pairs by expert.
  forward  dispatch, the first linear with a SwiGLU scaled by the routing weight, the second
           linear, combine ([Mega] "Mega MoE คืออะไร?" [what is Mega MoE?]; [TE] "צמצום הזיכרון
           ותקורות הכימות" [reducing memory and quantisation overheads]: GroupedLinear ->
           ScaledSwiGLU -> GroupedLinear).  Every routed pair is computed at its real count:
           no capacity, dropping or padding ([JAX] "A dropless MoE minden tokent feldolgoz";
           "Csoportosított mátrixszorzás és összevont adatmozgatás" [grouped GEMM and fused
           data movement]).
  backward the gradient of that forward pass ([Prime] "Mit csinált a Prime Intellect?" [what
           did Prime Intellect do?]: a backward for the fused MoE kernel): dx, dW1, dW2,
           d(routing weights) and d(logits) through the top-k softmax.
  router   the learned router's scores, logits = x Wg with the gate weight Wg [d, E] ([JAX] "A
           dropless MoE minden tokent feldolgoz"), and their gradients dWg and the part of dx
           that flows through the logits.

Conventions: W1[e] is [d, 2f] with gate columns [0, f) and up columns [f, 2f);
SwiGLU(g, u) = silu(g) * u with silu(g) = g * sigmoid(g).  A pair p = t*k + j is slot j of
token t.  Expert id -1 marks a slot that is not routed here (owned by another rank); such a
pair is skipped everywhere.  All inputs must be finite.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


# ------------------------------------------------------------------------------- routing
def route(logits: np.ndarray, k: int):
    """Top-k selection and softmax over the selected logits.

    Returns (ids int32 [T, k], w fp64 [T, k]).  Slot 0 is the largest logit; among equal
    logits the lower expert id comes first.  Selection is k rounds of "take the largest
    remaining value" (np.argmax returns the first maximum, i.e. the lowest id on ties)."""
    L = np.asarray(logits, dtype=np.float64)
    T, E = L.shape
    assert 1 <= k <= E
    assert np.all(np.isfinite(L)), "logits must be finite"
    taken = np.zeros((T, E), dtype=bool)
    ids = np.empty((T, k), dtype=np.int32)
    rows = np.arange(T)
    for j in range(k):
        cand = np.where(taken, -np.inf, L)
        best = np.argmax(cand, axis=1)
        ids[:, j] = best
        taken[rows, best] = True
    sel = L[rows[:, None], ids]                      # descending
    z = np.exp(sel - sel[:, :1])
    w = z / z.sum(axis=1, keepdims=True)
    return ids, w


# ---------------------------------------------------------------------------------- plan
@dataclass
class Plan:
    counts: np.ndarray    # int32 [E]        routed pairs per expert
    offsets: np.ndarray   # int32 [E+1]      exclusive prefix sum of counts
    perm: np.ndarray      # int32 [A]        sorted position -> pair index p
    inv_perm: np.ndarray  # int32 [T*k]      pair index p -> sorted position, -1 if not routed


def plan(ids: np.ndarray, E: int) -> Plan:
    """Counting sort of pairs by expert.  Within an expert, pairs keep ascending pair index
    (hence ascending token), which makes the order unique."""
    flat = np.asarray(ids, dtype=np.int64).ravel()
    assert np.all((flat >= -1) & (flat < E)), "expert ids must be in [-1, E)"
    counts = np.zeros(E, dtype=np.int64)
    for e in range(E):
        counts[e] = np.count_nonzero(flat == e)
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    perm = np.empty(offsets[E], dtype=np.int64)
    for e in range(E):
        perm[offsets[e]:offsets[e + 1]] = np.flatnonzero(flat == e)
    inv_perm = np.full(flat.size, -1, dtype=np.int64)
    inv_perm[perm] = np.arange(offsets[E])
    return Plan(counts.astype(np.int32), offsets.astype(np.int32), perm.astype(np.int32),
                inv_perm.astype(np.int32))


def _expert_rows(pl: Plan, e: int, k: int):
    P = pl.perm[pl.offsets[e]:pl.offsets[e + 1]].astype(np.int64)
    return P, P // k            # pair indices, token rows


# ------------------------------------------------------------------------------- forward
def forward(x, W1, W2, ids, w, E=None, return_saved=False):
    """y[t] = sum over routed slots j of w[t,j] * SwiGLU(x[t] W1[e]) W2[e], e = ids[t,j].

    Inputs fp64 (already decoded): x [T,d], W1 [E,d,2f], W2 [E,f,d], ids [T,k], w [T,k]."""
    x = np.asarray(x, np.float64)
    T, d = x.shape
    E = W1.shape[0] if E is None else E
    f = W2.shape[1]
    k = ids.shape[1]
    wf = np.asarray(w, np.float64).ravel()
    pl = plan(ids, E)
    y = np.zeros((T, d))
    saved = {}
    for e in range(E):
        if pl.counts[e] == 0:
            continue
        P, R = _expert_rows(pl, e, k)
        Xe = x[R]
        He = Xe @ W1[e]
        G, U = He[:, :f], He[:, f:]
        a = G * _sigmoid(G) * U
        Oe = a @ W2[e]
        np.add.at(y, R, wf[P][:, None] * Oe)
        if return_saved:
            saved[e] = (G, U, a, Oe)
    return (y, pl, saved) if return_saved else y


# ------------------------------------------------------------------------------ backward
def backward(x, W1, W2, ids, w, dy, logits_routed=True, W1_dx=None, W2_da=None, dy_da=None, x_dw=None, q_dw=None):
    """Gradients of L = sum(dy * y) for the forward above.

    Returns dict with dx [T,d], dW1 [E,d,2f], dW2 [E,f,d], d_topk_w [T,k] (0 on unrouted
    slots) and, when the weights came from route() (logits_routed=True), d_logits [T,E]
    through the softmax over the k selected logits (0 off the selected set).

    The optional operands name a different copy of a tensor for one product, as a quantised
    layer has when each GEMM quantises along its own K (MXFP8): dy_da and W2_da for
    da = (w dy) W2^T and the routing-weight gradient, W1_dx for dx = dH W1^T, x_dw for
    dW1 = x^T dH.  Left as None they are dy, W2, W1 and x.

    q_dw, when given, is applied to the layer inputs that enter the two weight-gradient
    products, one expert at a time with its rows in the expert's sorted order: dW2[e] =
    As_e^T q(dy_e) with As_e = w * a (the routing-scaled activation the down projection
    consumes) and dW1[e] = q(x_e)^T dH_e.  The intermediates As and dH stay exact, as they do
    everywhere in this oracle.  A layer that quantises the inputs along the token axis, in blocks
    that stay inside one expert, is modelled by q_dw = mx_roundtrip_rows."""
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    W1_dx = W1 if W1_dx is None else W1_dx
    W2_da = W2 if W2_da is None else W2_da
    dy_da = dy if dy_da is None else np.asarray(dy_da, np.float64)
    x_dw = x if x_dw is None else np.asarray(x_dw, np.float64)
    T, d = x.shape
    E = W1.shape[0]
    f = W2.shape[1]
    k = ids.shape[1]
    wf = np.asarray(w, np.float64).ravel()
    pl = plan(ids, E)
    dx = np.zeros((T, d))
    dW1 = np.zeros(W1.shape)
    dW2 = np.zeros(W2.shape)
    dw = np.zeros(T * k)
    for e in range(E):
        if pl.counts[e] == 0:
            continue                                   # an empty expert has zero gradient
        P, R = _expert_rows(pl, e, k)
        Xe = x[R]
        He = Xe @ W1[e]
        G, U = He[:, :f], He[:, f:]
        sg = _sigmoid(G)
        S = G * sg                                     # silu(g)
        a = S * U
        dYa = dy_da[R]
        dw[P] = np.sum(dYa * (a @ W2_da[e]), axis=1)   # y is linear in each routing weight
        if q_dw is None:
            dW2[e] = a.T @ (wf[P][:, None] * dy[R])
        else:
            dW2[e] = (wf[P][:, None] * a).T @ q_dw(dy[R])
        da = (wf[P][:, None] * dYa) @ W2_da[e].T
        dG = da * U * sg * (1.0 + G * (1.0 - sg))      # d silu / dg = sig * (1 + g (1 - sig))
        dU = da * S
        dH = np.concatenate([dG, dU], axis=1)
        dW1[e] = (x_dw[R] if q_dw is None else q_dw(x_dw[R])).T @ dH
        np.add.at(dx, R, dH @ W1_dx[e].T)
    out = dict(dx=dx, dW1=dW1, dW2=dW2, d_topk_w=dw.reshape(T, k), plan=pl)
    if logits_routed:
        wm = np.asarray(w, np.float64)
        dwm = dw.reshape(T, k)
        inner = np.sum(wm * dwm, axis=1, keepdims=True)
        dl = np.zeros((T, E))
        rows = np.arange(T)[:, None]
        dl[rows, ids] = wm * (dwm - inner)             # softmax Jacobian over the kept logits
        out["d_logits"] = dl
    return out


# --------------------------------------------------------- per-entry forms (large inputs)
# At full size the tests compare sampled outputs.  These functions compute single rows or
# single gradient entries from the same definitions, touching only the rows they need.
def token_forward(x_row, W1, W2, ids_row, w_row):
    """y[t] for one token: sum_j w_j * SwiGLU(x_t W1[e_j]) W2[e_j] over routed slots."""
    f = W2.shape[1]
    y = np.zeros(x_row.shape[0])
    for e, wj in zip(ids_row, w_row):
        if e < 0:
            continue
        h = x_row @ W1[e]
        g, u = h[:f], h[f:]
        y += wj * ((g * _sigmoid(g) * u) @ W2[e])
    return y


def token_backward(x_row, W1, W2, ids_row, w_row, dy_row, W1_dx=None, W2_da=None, dy_da=None):
    """(dx[t], d_topk_w[t, :]) for one token.  W1_dx, W2_da and dy_da name other copies of
    W1, W2 and dy for the products dx = dH W1^T and da = w dy W2^T, as in backward()."""
    f = W2.shape[1]
    W1_dx = W1 if W1_dx is None else W1_dx
    W2_da = W2 if W2_da is None else W2_da
    dy_da = dy_row if dy_da is None else dy_da
    dx = np.zeros(x_row.shape[0])
    dw = np.zeros(len(ids_row))
    for j, (e, wj) in enumerate(zip(ids_row, w_row)):
        if e < 0:
            continue
        h = x_row @ W1[e]
        g, u = h[:f], h[f:]
        sg = _sigmoid(g)
        s = g * sg
        a = s * u
        dw[j] = dy_da @ (a @ W2_da[e])
        da = wj * (W2_da[e] @ dy_da)
        dg = da * u * sg * (1.0 + g * (1.0 - sg))
        du = da * s
        dx += W1_dx[e] @ np.concatenate([dg, du])
    return dx, dw


def weight_grad_entries(x, W1, W2, ids, w, dy, e, rows_i, cols_j, which, q_dw=None):
    """Selected entries of dW1[e] (which='dW1', i over d, j over 2f) or dW2[e] (which='dW2',
    i over f, j over d), computed from the expert's token rows only.  q_dw as in backward(): it
    acts on the expert's rows of one input column at a time (x column i for dW1, dy column j
    for dW2), which is all an entry needs because its blocks run down that column."""
    k = ids.shape[1]
    f = W2.shape[1]
    flat = np.asarray(ids).ravel()
    P = np.flatnonzero(flat == e)
    if P.size == 0:
        return np.zeros(len(rows_i))
    R = P // k
    wv = np.asarray(w, np.float64).ravel()[P]
    Xe = np.asarray(x, np.float64)[R]
    dYe = np.asarray(dy, np.float64)[R]
    out = np.empty(len(rows_i))
    for n, (i, j) in enumerate(zip(rows_i, cols_j)):
        if which == "dW2":
            g = Xe @ W1[e][:, i]
            u = Xe @ W1[e][:, f + i]
            a_i = g * _sigmoid(g) * u
            dcol = dYe[:, j] if q_dw is None else q_dw(dYe[:, [j]])[:, 0]
            out[n] = np.sum(wv * a_i * dcol)
        else:
            c = j % f                                   # column pair (gate c, up f + c)
            g = Xe @ W1[e][:, c]
            u = Xe @ W1[e][:, f + c]
            sg = _sigmoid(g)
            da = wv * (dYe @ W2[e][c, :])
            dh = da * u * sg * (1.0 + g * (1.0 - sg)) if j < f else da * g * sg
            xcol = Xe[:, i] if q_dw is None else q_dw(Xe[:, [i]])[:, 0]
            out[n] = np.sum(xcol * dh)
    return out


def expert_weight_grads(x, W1, W2, ids, w, dy, e, W2_da=None, dy_da=None, x_dw=None, q_dw=None):
    """(dW1[e], dW2[e]) of backward() for one expert, from that expert's rows only (same
    arguments; the full-size checks use it where the whole backward would not fit)."""
    k = ids.shape[1]
    E = W1.shape[0]
    sel = np.asarray(ids) == e
    toks = np.flatnonzero(sel.any(axis=1))
    sub_ids = np.where(sel[toks], 0, -1)             # the expert becomes expert 0 of a 1-expert layer
    pick = lambda v: None if v is None else np.asarray(v, np.float64)[toks]
    one = lambda Wt: None if Wt is None else np.asarray(Wt[e], np.float64)[None]
    sub_w = np.where(sel[toks], np.asarray(w, np.float64)[toks], 0.0)
    out = backward(pick(x), one(W1), one(W2), sub_ids, sub_w, pick(dy), logits_routed=False,
                   W2_da=one(W2_da), dy_da=pick(dy_da), x_dw=pick(x_dw), q_dw=q_dw)
    return out["dW1"][0], out["dW2"][0]


def d_logits_from_dw(w, dw, ids, E):
    """d_logits[t, ids[t,j]] = w[t,j] * (dw[t,j] - sum_i w[t,i] dw[t,i]); zero elsewhere."""
    w = np.asarray(w, np.float64)
    dw = np.asarray(dw, np.float64)
    T = w.shape[0]
    inner = np.sum(w * dw, axis=1, keepdims=True)
    dl = np.zeros((T, E))
    dl[np.arange(T)[:, None], ids] = w * (dw - inner)
    return dl


# --------------------------------------------------------------------------- router front end
def router_logits(x, Wg):
    """Router scores logits[t, e] = sum_i x[t, i] Wg[i, e] for the gate weight Wg [d, E]."""
    return np.asarray(x, np.float64) @ np.asarray(Wg, np.float64)


def router_backward(x, Wg, d_logits):
    """Gradients through logits = x Wg for an upstream d_logits [T, E]: returns
    (dx_router [T, d], dWg [d, E]) with dx_router[t, i] = sum_e d_logits[t, e] Wg[i, e] (the part of
    dx that flows through the router, to be added to the expert path's dx) and
    dWg[i, e] = sum_t x[t, i] d_logits[t, e]."""
    x = np.asarray(x, np.float64)
    Wg = np.asarray(Wg, np.float64)
    dl = np.asarray(d_logits, np.float64)
    return dl @ Wg.T, x.T @ dl
