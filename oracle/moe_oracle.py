"""Plain, slow, obviously-correct CPU definition of the MoE layer hot path.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code with the
HIP path.  Arithmetic is NumPy float64 throughout, except the per-token int8
quantisation, which is done in fp32 exactly as the LightOP page writes it so
that its integer codes are a reproducible, exact target.

Sources, cited below by short name and section:

[FA-MoE]  "MoE 模型的 FlashAttention 跟普通模型有什么不一样？",
          http://www.framerc.cn/news/2508843/
[Router]  the MoE Router page on Ascend CANN,
          https://2048ai.net/6a1268d0662f9a54cb76af71.html
[LightOP] "大模型推理加速200%+？这套国产融合算子库把CUDA/Triton全替换了",
          https://adg.csdn.net/6a3a2e8f10ee7a33f281154b.html

The layer, in the order of [FA-MoE] section "FlashAttention 在 MoE 模型里的位置"
(steps 2-5): route every token to its top-k experts, group tokens by expert,
run each expert's FFN on its own tokens, merge the expert outputs weighted by
the route weights.

Readings where the pages are silent, ambiguous or disagree (each is used below):

R1  capacity C = ceil(factor * T * k / E): [Router] section "昇腾NPU的通信计算重叠"
    writes C = (total tokens / experts) * 1.25; the load it divides is the
    number of (token, expert) assignments, T*k, as the same page counts
    "expert accesses" in its dispatch estimate.  factor <= 0 means no limit.
R2  the assignments an expert drops are the ones beyond the first C in token
    order (first come, first served); they are not re-routed and the surviving
    weights are not renormalised.
R3  the layer returns the MoE branch only; a dropped assignment contributes 0
    (the residual connection belongs to the caller).
R4  top-k order is descending probability, equal probabilities go to the lower
    expert id.
R5  the gate is Linear(H, E) stored [E, H]; a per-expert bias is added to the
    logits only where a workload supplies one (the skewed workload's prior).
R6  expert FFN is SwiGLU: W2 (silu(W1 x) * W3 x), no biases, silu(z)=z/(1+e^-z);
    W13[e] stacks W1 (rows 0..I-1) over W3 (rows I..2I-1), W2[e] is [H, I].
R7  W8A8: activations quantised per token with the LightOP rule, int8 weights
    carry one fp32 scale per output channel, the int GEMM result is scaled by
    (activation scale of the row) * (weight scale of the column); the FFN's
    second GEMM quantises h the same way, one scale per row of h.  The page
    fixes no precision for h between the two GEMMs; h is taken in bf16, the
    layer's activation dtype (formed in fp32, rounded to nearest even), and
    the codes and row scale are those of the rounded values.
R8  MoE Sum's fused shared-expert factor and bias ([LightOP] section 3.2) add
    shared_factor * S[t] (the shared expert's output for token t) and a
    per-column bias b to the routed sum; the page names the fusion only.
R9  group-limited routing ([LightOP] section 3.1, Moe Fuse Gate: groups are
    chosen first, with each group's Top1/Top2 kept): the E experts form
    n_group contiguous groups of E/n_group; a group scores the sum of its two
    largest softmax probabilities (its only one for groups of one); the
    topk_group best groups (equal scores: lower group index first) are the
    only candidates for the usual top-k, whose weights are renormalised as
    in route.  The probabilities are those of the plain router's softmax.
    parity of this reading against the page is unpinned: the page gives no
    formula; the pins below fix the oracle to the reading itself.
R10 W4A16 ([LightOP] section 4.3, the quantisation matrix: INT4 weights with
    16-bit activations): integer weight codes in [-8, 7] with one fp32 scale
    per output channel (per row of W13 and of W2, as R7), so each expert
    weight is code * scale; activations stay in their 16-bit storage type and
    the FFN is the R6 SwiGLU on those weights.  How the codes are made from
    real weights is offline and outside the hot path.
R11 W4A8 ([LightOP] section 4.3, INT4 weights with INT8 activations): R7 with
    the weight codes of R10, i.e. per-token int8 activations, int4 codes with
    per-output-channel scales, integer accumulation, h re-quantised per row.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

__all__ = [
    "to_f64", "gate_logits", "softmax_rows", "topk_rows", "renormalise", "route",
    "quant_per_token_int8", "capacity", "align", "tiles", "silu", "swiglu_ffn",
    "layer", "layer_from_inputs", "layer_token_major", "combine", "combine_shared",
    "group_scores", "route_grouped", "dequant_rows", "round_bf16",
]


# ----------------------------------------------------------------------------
# storage decoding (the oracle's own; bf16 arrives as uint16 bit patterns)
# ----------------------------------------------------------------------------
def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored values exactly to float64 ("f32", "bf16" bits, "i8")."""
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype in ("f32", "i8"):
        return np.asarray(a).astype(np.float64)
    raise ValueError(dtype)


def _to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32)
    return np.asarray(a, dtype=np.float32)


# ----------------------------------------------------------------------------
# route: gate -> softmax -> top-k -> renormalise
# ----------------------------------------------------------------------------
def gate_logits(x: np.ndarray, wg: np.ndarray, bias: np.ndarray | None = None) -> np.ndarray:
    """logits[t, e] = sum_h x[t, h] * Wg[e, h] (+ bias[e]).

    [Router] section "Router 就是一个小型网络": the gate is a bias-free linear
    layer from the hidden size to the expert count; bias per R5.
    """
    logits = x @ wg.T
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float64)[None, :]
    return logits


def softmax_rows(logits: np.ndarray) -> np.ndarray:
    """Softmax over the experts of each token ([Router], same section)."""
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    return e / e.sum(axis=1, keepdims=True)


def topk_rows(p: np.ndarray, k: int) -> np.ndarray:
    """The k most probable experts of each row, most probable first.

    [Router] same section (top-k of the softmax scores); ties per R4: a stable
    sort of -p keeps equal probabilities in ascending expert order.
    """
    order = np.argsort(-p, axis=1, kind="stable")
    return order[:, :k]


def renormalise(p_sel: np.ndarray) -> np.ndarray:
    """Selected probabilities divided by their sum, so each row sums to 1
    ([Router], same section)."""
    return p_sel / p_sel.sum(axis=1, keepdims=True)


def route(x: np.ndarray, wg: np.ndarray, k: int, bias: np.ndarray | None = None) -> dict:
    """Full router on float64 inputs.  Returns ids (int32 [T,k]), w and p_sel
    (float64 [T,k]), the full logits/p, and the k-th/(k+1)-th gaps used to
    exempt near-ties from id parity."""
    logits = gate_logits(x, wg, bias)
    p = softmax_rows(logits)
    ids = topk_rows(p, k)
    p_sel = np.take_along_axis(p, ids, axis=1)
    w = renormalise(p_sel)
    T, E = p.shape
    if k < E:
        order = np.argsort(-p, axis=1, kind="stable")
        pk = np.take_along_axis(p, order[:, k - 1:k + 1], axis=1)
        lk = np.take_along_axis(logits, order[:, k - 1:k + 1], axis=1)
        gap_p = pk[:, 0] - pk[:, 1]
        gap_l = lk[:, 0] - lk[:, 1]
    else:
        gap_p = np.full(T, np.inf)
        gap_l = np.full(T, np.inf)
    return {"logits": logits, "p": p, "ids": ids.astype(np.int32), "w": w, "p_sel": p_sel,
            "gap_p": gap_p, "gap_logit": gap_l}


def group_scores(p: np.ndarray, n_group: int) -> np.ndarray:
    """Score of each contiguous expert group (R9): the sum of the group's two
    largest probabilities, or its single probability for groups of one."""
    T, E = p.shape
    gsz = E // n_group
    grouped = p.reshape(T, n_group, gsz)
    desc = -np.sort(-grouped, axis=2)
    return desc[:, :, :min(2, gsz)].sum(axis=2)


def route_grouped(x: np.ndarray, wg: np.ndarray, k: int, n_group: int, topk_group: int,
                  bias: np.ndarray | None = None) -> dict:
    """Group-limited router (R9) on float64 inputs: softmax as in route, the
    topk_group best groups by group_scores, then top-k (R4 order) among their
    experts only, renormalised.  Returns the keys of route plus the group
    scores, the chosen groups and the topk_group-th/next group-score gap."""
    T = x.shape[0]
    E = wg.shape[0]
    if E % n_group != 0 or not 1 <= topk_group <= n_group or k > topk_group * (E // n_group):
        raise ValueError("need E % n_group == 0, 1 <= topk_group <= n_group, k <= topk_group * E / n_group")
    logits = gate_logits(x, wg, bias)
    p = softmax_rows(logits)
    gsc = group_scores(p, n_group)
    gorder = np.argsort(-gsc, axis=1, kind="stable")
    chosen = gorder[:, :topk_group]
    allowed = np.zeros((T, n_group), dtype=bool)
    np.put_along_axis(allowed, chosen, True, axis=1)
    candidate = np.repeat(allowed, E // n_group, axis=1)
    p_cand = np.where(candidate, p, -1.0)     # below every probability
    ids = topk_rows(p_cand, k)
    p_sel = np.take_along_axis(p, ids, axis=1)
    w = renormalise(p_sel)
    n_cand = topk_group * (E // n_group)
    if k < n_cand:
        order = np.argsort(-p_cand, axis=1, kind="stable")
        pk = np.take_along_axis(p_cand, order[:, k - 1:k + 1], axis=1)
        gap_p = pk[:, 0] - pk[:, 1]
    else:
        gap_p = np.full(T, np.inf)
    if topk_group < n_group:
        gk = np.take_along_axis(gsc, gorder[:, topk_group - 1:topk_group + 1], axis=1)
        gap_group = gk[:, 0] - gk[:, 1]
    else:
        gap_group = np.full(T, np.inf)
    return {"logits": logits, "p": p, "ids": ids.astype(np.int32), "w": w, "p_sel": p_sel,
            "gap_p": gap_p, "group_scores": gsc, "groups": np.sort(chosen, axis=1),
            "gap_group": gap_group}


# ----------------------------------------------------------------------------
# per-token int8 quantisation, fp32 arithmetic as the page writes it
# ----------------------------------------------------------------------------
def quant_per_token_int8(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """[LightOP] section 4.1 (per_token_quant_int8): per row, scale = absmax/127
    (1 where the row is all zero), codes = round-half-even(x / scale) clamped
    to [-128, 127].  Every operation is an fp32 IEEE operation."""
    x32 = np.asarray(x, dtype=np.float32)
    absmax = np.abs(x32).max(axis=1, keepdims=True)
    scale = absmax / np.float32(127.0)
    scale = np.where(absmax == 0, np.float32(1.0), scale).astype(np.float32)
    q = np.clip(np.rint(x32 / scale), -128, 127).astype(np.int8)
    return q, scale[:, 0]


# ----------------------------------------------------------------------------
# align / dispatch
# ----------------------------------------------------------------------------
def capacity(T: int, k: int, E: int, factor: float) -> int | None:
    """Per-expert capacity C = ceil(factor * T * k / E) (R1); None = no limit."""
    if factor is None or factor <= 0:
        return None
    q = Fraction(factor).limit_denominator(1 << 20) * Fraction(T * k, E)
    return int(math.ceil(q))


def align(ids: np.ndarray, E: int, C: int | None) -> dict:
    """Group the T*k assignments by expert.

    [Router] "Token 分发的通信瓶颈": count the assignments per destination;
    [Router] "昇腾NPU的通信计算重叠": at most C per expert, the rest dropped (R1, R2);
    [LightOP] section 3.2 (MoE Align): histogram, prefix sum, expert-sorted ids.

    Slot s = t*k + j is token t's j-th choice.  rank[s] = number of earlier
    slots (in slot order) routed to the same expert; kept iff rank < C.
    """
    ids = np.asarray(ids)
    T, k = ids.shape
    flat = ids.reshape(-1).astype(np.int64)
    n = flat.size
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    order = np.argsort(flat, kind="stable")               # slots grouped by expert, slot order kept
    first = np.concatenate([[0], np.cumsum(counts)])[:-1]  # first sorted index of each expert
    rank = np.empty(n, dtype=np.int64)
    rank[order] = np.arange(n) - first[flat[order]]
    kept_e = counts if C is None else np.minimum(counts, C)
    offsets = np.concatenate([[0], np.cumsum(kept_e)]).astype(np.int64)
    keep = np.ones(n, dtype=bool) if C is None else rank < C
    pos = np.where(keep, offsets[flat] + rank, -1)
    sorted_slot = np.full(n, -1, dtype=np.int64)
    sorted_slot[pos[keep]] = np.nonzero(keep)[0]
    return {
        "counts": counts.astype(np.int32),
        "kept": kept_e.astype(np.int32),
        "offsets": offsets.astype(np.int32),
        "rank": rank.reshape(T, k),
        "pos": pos.reshape(T, k).astype(np.int32),
        "sorted_slot": sorted_slot.astype(np.int32),
        "num_dropped": int(n - offsets[-1]),
    }


def tiles(offsets: np.ndarray, block_m: int) -> list[tuple[int, int, int]]:
    """Row tiles of at most block_m rows, one expert each, in expert order:
    (expert, first sorted row, row count)."""
    out = []
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        for r in range(lo, hi, block_m):
            out.append((e, r, min(block_m, hi - r)))
    return out


# ----------------------------------------------------------------------------
# expert FFN (SwiGLU) and combine
# ----------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z * sigmoid(z) (R6)."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_ffn(a: np.ndarray, w1: np.ndarray, w3: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """W2 (silu(W1 a) * W3 a) for row vectors a [M, H]; W1, W3 [I, H]; W2 [H, I].

    [FA-MoE] section "手动编译 MoE 融合算子": the fused MoE call takes stacked expert
    weights and activation="silu"; the gated form is R6.
    """
    g = a @ w1.T
    u = a @ w3.T
    return (silu(g) * u) @ w2.T


def _w8a8_ffn(xq: np.ndarray, xs: np.ndarray, w13q: np.ndarray, s13: np.ndarray,
              w2q: np.ndarray, s2: np.ndarray, I: int) -> np.ndarray:
    """One expert's SwiGLU in W8A8 (R7, [LightOP] section 4.1 w8a8_gemm_smooth).

    The integer products are exact in float64 (|acc| < 2^53); h is formed in
    float64, rounded to fp32, then to bf16 (R7), and re-quantised per row
    with the same rule.
    """
    acc1 = xq.astype(np.float64) @ w13q.astype(np.float64).T          # exact integers
    deq = acc1 * xs.astype(np.float64)[:, None] * s13.astype(np.float64)[None, :]
    g, u = deq[:, :I], deq[:, I:]
    h16 = round_bf16((silu(g) * u).astype(np.float32))
    hq, hs = quant_per_token_int8(h16)
    acc2 = hq.astype(np.float64) @ w2q.astype(np.float64).T           # exact integers
    return acc2 * hs.astype(np.float64)[:, None] * s2.astype(np.float64)[None, :]


def round_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 (ties to even), as fp32: keep
    the top 16 bits after adding half an ulp of bf16 plus the kept lsb.
    Finite inputs only."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32)


def dequant_rows(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Weight of integer codes with one scale per output row (R7, R10):
    W[n, k] = q[n, k] * s[n]."""
    return np.asarray(q).astype(np.float64) * np.asarray(s, dtype=np.float64)[:, None]


def combine(y_rows: np.ndarray, pos: np.ndarray, w: np.ndarray) -> np.ndarray:
    """out[t] = sum over kept slots j of w[t,j] * Y[pos[t,j]] (R3).

    [FA-MoE] step 5 of the layer and its fusion two (weighted accumulation);
    [LightOP] section 3.2 (MoE Sum).  ``y_rows`` holds the unweighted expert
    output of every kept sorted row.
    """
    T, k = pos.shape
    out = np.zeros((T, y_rows.shape[1]), dtype=np.float64)
    for j in range(k):
        kept = pos[:, j] >= 0
        out[kept] += w[kept, j][:, None] * y_rows[pos[kept, j]]
    return out


def combine_shared(y_rows: np.ndarray, pos: np.ndarray, w: np.ndarray, shared: np.ndarray | None,
                   shared_factor: float, bias: np.ndarray | None) -> np.ndarray:
    """MoE Sum with the shared-expert term and a bias (R8):
    out[t] = sum over kept slots j of w[t,j] * Y[pos[t,j]] + shared_factor * S[t] + b.

    [LightOP] section 3.2 (MoE Sum) fuses the shared-expert factor and a bias
    add into the merge without giving the formula; the reading here adds the
    shared expert's output S [T,H], scaled by one scalar, and a per-column
    bias [H] to the routed sum.  Either term may be absent.
    """
    out = combine(y_rows, pos, w)
    if shared is not None:
        out = out + float(shared_factor) * np.asarray(shared, dtype=np.float64)
    if bias is not None:
        out = out + np.asarray(bias, dtype=np.float64)[None, :]
    return out


def layer(x, x_dtype, wg, wg_dtype, bias, w13, w2, w_dtype, k, capacity_factor,
          s13=None, s2=None, sample_tokens=None, n_group=0, topk_group=0, shared=None, shared_factor=1.0,
          out_bias=None) -> dict:
    """The whole layer, expert-major (the method's grouping).

    Routing and alignment always run over all T tokens (drops depend on every
    earlier token); the expert FFN and combine run for ``sample_tokens`` only
    when given (all tokens otherwise).  Returns intermediates and ``out``
    (float64, [len(sample), H]).  With ``n_group`` > 0 the routing is
    group-limited (R9); ``shared`` [T, H] (values), ``shared_factor`` and
    ``out_bias`` [H] enter the merge as in combine_shared (R8).
    """
    T, H = x.shape
    E = wg.shape[0]
    I = w2.shape[2]
    x64 = to_f64(x, x_dtype)
    if n_group:
        r = route_grouped(x64, to_f64(wg, wg_dtype), k, n_group, topk_group, bias)
    else:
        r = route(x64, to_f64(wg, wg_dtype), k, bias)
    C = capacity(T, k, E, capacity_factor)
    a = align(r["ids"], E, C)
    tok = np.arange(T) if sample_tokens is None else np.asarray(sample_tokens)
    res = {"route": r, "align": a, "capacity": C, "tokens": tok}

    xq = xs = None
    if w_dtype in ("i8", "i4a8"):
        xq, xs = quant_per_token_int8(_to_f32(x, x_dtype))
        res["xq"], res["xs"] = xq, xs

    # rows needed: kept slots of the sampled tokens, grouped by expert
    pos_s = a["pos"][tok]
    ids_s = r["ids"][tok]
    y_rows = np.zeros((T * k, H), dtype=np.float64)
    for e in range(E):
        sel = (ids_s == e) & (pos_s >= 0)
        if not sel.any():
            continue
        rows = pos_s[sel]
        tokens_e = tok[np.nonzero(sel)[0]]
        if w_dtype in ("i8", "i4a8"):
            y_rows[rows] = _w8a8_ffn(xq[tokens_e], xs[tokens_e], w13[e], s13[e], w2[e], s2[e], I)
        elif w_dtype == "i4":
            w13e = dequant_rows(w13[e], s13[e])
            y_rows[rows] = swiglu_ffn(x64[tokens_e], w13e[:I], w13e[I:], dequant_rows(w2[e], s2[e]))
        else:
            w13e = to_f64(w13[e], w_dtype)
            y_rows[rows] = swiglu_ffn(x64[tokens_e], w13e[:I], w13e[I:], to_f64(w2[e], w_dtype))
    if shared is not None or out_bias is not None:
        sh = None if shared is None else np.asarray(shared, dtype=np.float64)[tok]
        res["out"] = combine_shared(y_rows, pos_s, r["w"][tok], sh, shared_factor, out_bias)
    else:
        res["out"] = combine(y_rows, pos_s, r["w"][tok])
    return res


def layer_from_inputs(inp, sample_tokens=None) -> dict:
    """``layer`` on a generated input bundle (attributes as in moe_synth.Inputs)."""
    s = inp.spec
    return layer(inp.x, s.x_dtype, inp.wg, s.wg_dtype, inp.bias, inp.w13, inp.w2, s.w_dtype,
                 s.k, s.capacity_factor, inp.s13, inp.s2, sample_tokens)


def layer_token_major(x, x_dtype, wg, wg_dtype, bias, w13, w2, w_dtype, k, capacity_factor,
                      s13=None, s2=None) -> np.ndarray:
    """The same layer evaluated one token at a time with no grouping:
    out[t] = sum over kept j of w[t,j] * FFN_{ids[t,j]}(x[t]).  Small sizes only."""
    T, H = x.shape
    E = wg.shape[0]
    I = w2.shape[2]
    x64 = to_f64(x, x_dtype)
    r = route(x64, to_f64(wg, wg_dtype), k, bias)
    C = capacity(T, k, E, capacity_factor)
    seen = [0] * E
    out = np.zeros((T, H), dtype=np.float64)
    if w_dtype in ("i8", "i4a8"):
        xq, xs = quant_per_token_int8(_to_f32(x, x_dtype))
    for t in range(T):
        for j in range(k):
            e = int(r["ids"][t, j])
            kept = C is None or seen[e] < C
            seen[e] += 1
            if not kept:
                continue
            if w_dtype in ("i8", "i4a8"):
                y = _w8a8_ffn(xq[t:t + 1], xs[t:t + 1], w13[e], s13[e], w2[e], s2[e], I)[0]
            elif w_dtype == "i4":
                # element by element in Python floats (binary64)
                w1 = np.array([[float(q) * float(s13[e][n]) for q in w13[e][n]] for n in range(I)])
                w3 = np.array([[float(q) * float(s13[e][I + n]) for q in w13[e][I + n]] for n in range(I)])
                w2e = np.array([[float(q) * float(s2[e][n]) for q in w2[e][n]] for n in range(H)])
                y = swiglu_ffn(x64[t:t + 1], w1, w3, w2e)[0]
            else:
                w13e = to_f64(w13[e], w_dtype)
                y = swiglu_ffn(x64[t:t + 1], w13e[:I], w13e[I:], to_f64(w2[e], w_dtype))[0]
            out[t] += r["w"][t, j] * y
    return out
