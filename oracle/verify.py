"""fp64 oracle of the speculative-decoding verification step.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Every function is the
plain definition written out in numpy float64; matmul, cumsum and argmax are the
only library primitives used, with no blocking or fusion of the steps.

Notation, per request: K draft tokens x_1..x_K, target rows j = 0..K (row j
scores the token at draft position j+1, row K gives the bonus position), draft
rows j = 0..K-1 (the drafter's distribution for position j+1).

Sources (page titles, sections):
* [WB] "Speculative decoding in production: comparing methods in the Wildberries
  shopping assistant", sections "Where speculative decoding came from" (one
  target pass scores all draft tokens; accept the longest correct prefix and
  put the target's own token at the first error) and "A bit of theory"
  (Statement 1: accept with probability min(1, p(x)/q(x)), otherwise sample the
  normalised remainder max(0, p - q); p is the target distribution *after
  temperature*).
* [MISHA] "Let's start over, Misha: speculative decoding from draft to
  verification", sections "How it works" (left-to-right check; when every
  draft token is accepted the same pass yields one more token) and "Why isn't
  the answer spoiled?" (greedy verification reduces to an argmax match; the
  residual distribution on rejection).
* [DSPARK] "DSpark: speculative decoding with confidence-scheduled verification
  and semi-autoregressive generation": the verify length of each request is
  chosen from the estimated survival probability of the draft prefix under the
  engine's capacity.

Readings where the pages are silent (also listed with the design notes):
R1 the verified tail is a residual SwiGLU MLP followed by the LM head, the LM
   head shared with the drafter; R2 the intermediate ``a`` and the MLP output
   ``y`` are rounded to bf16 (the GPU stores them as bf16); R3 draft row j pairs
   with target row j; R4 the draft distribution uses the same temperature; R5
   an all-zero residual (impossible in exact arithmetic) falls back to p;
   R6 argmax ties go to the lowest index; R7 confidence = the draft's top-1
   probability, survival = running product, budget filled by descending
   floor(1024 * survival), then request, then position.

R13 FP8 weights (the pages serve FP8 targets: [WB] production model and the
   table of off-the-shelf drafters; [VLLM26] "Frequently asked questions";
   [MISHA] "Why is generation slow?" on weight bytes per token) are read as the
   OCP 8-bit E4M3 format with one fp32 scale per output channel (weight row);
   activations stay bf16, so an FP8 weight matrix is exactly decode(q) * scale.

Parity unpinned: the MLP weight scale and the 1/1024 key grid of the scheduler
are readings, not values the pages fix.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


# ----------------------------------------------------------------------------- numbers

def from_bf16_bits(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) exactly to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_rne(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even (reading R2).

    bfloat16 keeps 8 significant bits: write x = f * 2**e with 0.5 <= |f| < 1,
    round f * 2**8 to the nearest integer (half to even) and scale back.
    """
    x = np.asarray(x, dtype=np.float64)
    f, e = np.frexp(x)
    return np.ldexp(np.rint(np.ldexp(f, 8)), e - 8)


def from_e4m3_bits(codes) -> np.ndarray:
    """Decode 8-bit E4M3 codes (uint8) exactly to float64 (reading R13).

    Bit layout s eeee mmm with exponent bias 7: exponent field e > 0 gives
    (-1)^s * (1 + m/8) * 2**(e - 7); e = 0 gives the subnormal (-1)^s * m/8 * 2**-6.
    There is no infinity; s 1111 111 is NaN.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def silu(x) -> np.ndarray:
    """x * sigmoid(x) = x / (1 + exp(-x))."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


# ----------------------------------------------------------------------------- model tail

@dataclass
class Weights:
    """fp64 values of the weights (bf16, or FP8 times its row scales), row-major ``[out, in]``."""

    w_lm: np.ndarray                   # [V, d]
    w_gate: np.ndarray | None = None   # [d_ff, d]
    w_up: np.ndarray | None = None     # [d_ff, d]
    w_down: np.ndarray | None = None   # [d, d_ff]

    @classmethod
    def from_bits(cls, data: dict) -> "Weights":
        g = data.get("w_gate")
        return cls(from_bf16_bits(data["w_lm"]),
                   None if g is None else from_bf16_bits(g),
                   None if g is None else from_bf16_bits(data["w_up"]),
                   None if g is None else from_bf16_bits(data["w_down"]))

    @classmethod
    def from_fp8(cls, data: dict) -> "Weights":
        """FP8 weights (reading R13): W = decode(q_*) * s_*[:, None] for every matrix."""
        def mat(name):
            q = data.get("q_" + name)
            if q is None:
                return None
            return from_e4m3_bits(q) * np.asarray(data["s_" + name], dtype=np.float64)[:, None]
        return cls(mat("lm"), mat("gate"), mat("up"), mat("down"))


def target_hidden(h, w: Weights) -> np.ndarray:
    """Final hidden state of the target rows (readings R1, R2).

    a = bf16(silu(h W_gate^T) * (h W_up^T));  y = bf16(h + a W_down^T).
    Without an MLP (no gate weights) y = h.
    """
    h = np.asarray(h, dtype=np.float64)
    if w.w_gate is None:
        return h
    g = h @ w.w_gate.T
    u = h @ w.w_up.T
    a = bf16_rne(silu(g) * u)
    return bf16_rne(h + a @ w.w_down.T)


def lm_logits(w_lm, x) -> np.ndarray:
    """Logits of the shared LM head: z = x W_lm^T (the drafter uses the same head)."""
    return np.asarray(x, dtype=np.float64) @ w_lm.T


def softmax_t(z, T: float) -> np.ndarray:
    """Distribution after temperature T over the last axis: softmax(z / T) ([WB] "A bit of theory")."""
    s = np.asarray(z, dtype=np.float64) / T
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=-1, keepdims=True)


def row_stats(z, T: float = 1.0, tokens=None) -> dict:
    """Per-row diagnostics: log-sum-exp of z/T, argmax (lowest index), top-1 minus top-2
    logit gap (in z units, reading R6), and z at ``tokens`` when given."""
    z = np.asarray(z, dtype=np.float64)
    s = z / T
    m = s.max(axis=-1)
    lse = m + np.log(np.exp(s - m[..., None]).sum(axis=-1))
    top2 = -np.sort(-z, axis=-1)[..., :2]
    # one token: no second logit, so the margin is unbounded (no near tie can occur)
    gap = top2[..., 0] - top2[..., 1] if z.shape[-1] > 1 else np.full(z.shape[:-1], np.inf)
    out = {"lse": lse, "argmax": z.argmax(axis=-1), "gap": gap, "zmax": top2[..., 0]}
    if tokens is not None:
        out["z_x"] = np.take_along_axis(z, np.asarray(tokens)[..., None], axis=-1)[..., 0]
    return out


# ----------------------------------------------------------------------------- sampling

def inverse_cdf(w, u) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Sample index v* = min{v : C_v > u * C_last} with C the running sum of ``w`` in
    ascending index order, row-wise.  Returns (v*, C_{v*-1}/C_last, C_{v*}/C_last); the
    last two are the CDF boundaries around the coin, used to classify near-ties."""
    w = np.asarray(w, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    C = np.cumsum(w, axis=-1)
    S = C[..., -1]
    t = u * S
    v = (C <= t[..., None]).sum(axis=-1)
    v = np.minimum(v, w.shape[-1] - 1)
    hi = np.take_along_axis(C, v[..., None], axis=-1)[..., 0]
    lo = hi - np.take_along_axis(w, v[..., None], axis=-1)[..., 0]
    with np.errstate(invalid="ignore", divide="ignore"):
        return v, lo / S, hi / S


def _leading_true(ok) -> np.ndarray:
    """Number of leading True entries per row (the accepted prefix length)."""
    ok = np.asarray(ok, dtype=bool)
    if ok.shape[-1] == 0:
        return np.zeros(ok.shape[:-1], dtype=np.int64)
    return np.cumprod(ok, axis=-1).sum(axis=-1).astype(np.int64)


def accept_sample(p, q, draft, coins) -> dict:
    """Rejection-sampling verification of a batch of requests with the same K.

    p: [B, K+1, V] target distributions after temperature; q: [B, K, V] draft
    distributions; draft: [B, K] proposed ids; coins: [B, K+1] uniforms in [0,1).

    Left to right, draft token x_j (j = 1..K) is accepted when
    coins[j-1] < min(1, p_j(x_j) / q_j(x_j)).  At the first rejection the emitted
    token is drawn from the normalised max(0, p_j - q_j) with coins[K]; if every
    token is accepted the bonus token is drawn from p_{K+1} with coins[K]
    ([WB] Statement 1; [MISHA] "How it works", "Why isn't the answer spoiled?").
    """
    p = np.asarray(p, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    draft = np.asarray(draft, dtype=np.int64)
    coins = np.asarray(coins, dtype=np.float64)
    B, K = draft.shape
    bi = np.arange(B)
    if K:
        jj = np.arange(K)[None, :]
        px = p[bi[:, None], jj, draft]
        qx = q[bi[:, None], jj, draft]
        with np.errstate(divide="ignore", invalid="ignore"):
            ratio = np.where(qx > 0, px / qx, np.inf)
        ok = coins[:, :K] < np.minimum(1.0, ratio)
    else:
        px = qx = ratio = np.zeros((B, 0))
        ok = np.zeros((B, 0), dtype=bool)
    A = _leading_true(ok)
    rejected = A < K
    rowA = np.minimum(A, K)
    p_row = p[bi, rowA]
    if K:
        q_row = q[bi, np.minimum(A, K - 1)]
        resid = np.maximum(0.0, p_row - q_row)
    else:
        resid = p_row.copy()
    resid_mass = resid.sum(axis=-1)
    fallback = rejected & (resid_mass == 0.0)
    w = np.where((rejected & ~fallback)[:, None], resid, p_row)
    v, cdf_lo, cdf_hi = inverse_cdf(w, coins[:, K])
    emitted = np.full((B, K + 1), -1, dtype=np.int64)
    for b in range(B):
        emitted[b, :A[b]] = draft[b, :A[b]]
        emitted[b, A[b]] = v[b]
    return {"accepted": A, "emitted": emitted, "final": v, "p_x": px, "q_x": qx, "ratio": ratio,
            "resid_mass": np.where(rejected, resid_mass, 0.0), "fallback": fallback,
            "cdf_lo": cdf_lo, "cdf_hi": cdf_hi}


def accept_greedy(z_t, draft) -> dict:
    """Greedy verification: accept while x_j equals the target argmax of row j-1, then emit
    the argmax of the first mismatching row (or of the bonus row) ([MISHA] "Why isn't the
    answer spoiled?": at temperature 0 the check is an argmax comparison)."""
    z_t = np.asarray(z_t, dtype=np.float64)
    draft = np.asarray(draft, dtype=np.int64)
    B, K = draft.shape
    amax = z_t.argmax(axis=-1)
    A = _leading_true(draft == amax[:, :K])
    v = amax[np.arange(B), A]
    emitted = np.full((B, K + 1), -1, dtype=np.int64)
    for b in range(B):
        emitted[b, :A[b]] = draft[b, :A[b]]
        emitted[b, A[b]] = v[b]
    return {"accepted": A, "emitted": emitted, "final": v, "argmax": amax}


def propose(w: Weights, h_draft, T: float, draft_coins) -> dict:
    """The drafter's own step on the shared LM head (used to make test inputs).

    q = softmax(h_draft W_lm^T / T); x ~ q by inverse CDF with ``draft_coins``, or the
    argmax when T == 0 (greedy drafting).  ``conf`` = max_v q(v), the top-1 probability.
    """
    z = lm_logits(w.w_lm, h_draft)
    if T == 0:
        return {"draft": z.argmax(axis=-1), "conf": None, "logits": z}
    q = softmax_t(z, T)
    x, _, _ = inverse_cdf(q, draft_coins)
    return {"draft": x, "conf": q.max(axis=-1), "logits": z}


# ----------------------------------------------------------------------------- scheduling

def survival_schedule(conf, threshold: float, budget_rows: int) -> dict:
    """Confidence-scheduled verify lengths ([DSPARK]; reading R7).

    conf: [B, Kmax] draft top-1 probabilities.  Survival s_b(k) = prod_{i<=k} conf[b, i-1].
    Positions with s_b(k) >= threshold are eligible.  Every request keeps its one target
    row; if all eligible positions fit in ``budget_rows`` they are all verified, otherwise
    the budget_rows - B positions with the largest floor(1024 * s) are kept (ties: lower
    request index, then lower position).  k_b = number kept for request b (a prefix,
    since s is non-increasing in k).
    """
    conf = np.asarray(conf, dtype=np.float64)
    B, Kmax = conf.shape
    s = np.cumprod(conf, axis=1)
    elig = s >= threshold
    n_elig = int(elig.sum())
    key = np.floor(1024.0 * s)
    if B + n_elig <= budget_rows:
        k = _leading_true(elig)
        bound = False
    else:
        cand = [(-key[b, j], b, j) for b in range(B) for j in range(Kmax) if elig[b, j]]
        cand.sort()
        keep = cand[: max(0, budget_rows - B)]
        k = np.zeros(B, dtype=np.int64)
        for _, b, _j in keep:
            k[b] += 1
        bound = True
    return {"verify_len": k, "survival": s, "eligible": elig, "key": key, "budget_bound": bound}


# ----------------------------------------------------------------------------- verify calls

def _counters(A, k) -> np.ndarray:
    A = np.asarray(A, dtype=np.int64)
    return np.array([A.sum(), np.asarray(k, dtype=np.int64).sum(), (A + 1).sum()], dtype=np.int64)


def verify_greedy(w: Weights, h, draft) -> dict:
    """Greedy verification of B requests: h [B, K+1, d] target hidden rows, draft [B, K]."""
    draft = np.asarray(draft, dtype=np.int64)
    B, K = draft.shape
    y = target_hidden(h, w)
    z_t = lm_logits(w.w_lm, y)
    res = accept_greedy(z_t, draft)
    st = row_stats(z_t, 1.0)
    res.update({"logits_t": z_t, "y": y, "gap_t": st["gap"], "tau": float(np.mean(res["accepted"] + 1)),
                "counters": _counters(res["accepted"], np.full(B, K))})
    return res


def verify_sample(w: Weights, h, h_draft, draft, coins, T: float) -> dict:
    """Sampled verification of B requests at temperature T.

    h [B, K+1, d] target hidden rows, h_draft [B, K, d] draft hidden rows (same shared
    LM head, reading R3), draft [B, K], coins [B, K+1].
    """
    draft = np.asarray(draft, dtype=np.int64)
    B, K = draft.shape
    y = target_hidden(h, w)
    z_t = lm_logits(w.w_lm, y)
    z_d = lm_logits(w.w_lm, h_draft)
    p = softmax_t(z_t, T)
    q = softmax_t(z_d, T)
    res = accept_sample(p, q, draft, coins)
    st_t = row_stats(z_t, T)
    st_d = row_stats(z_d, T)
    res.update({"logits_t": z_t, "logits_d": z_d, "y": y, "lse_t": st_t["lse"], "lse_d": st_d["lse"],
                "argmax_t": st_t["argmax"], "gap_t": st_t["gap"], "conf": q.max(axis=-1),
                "alpha": np.minimum(p[:, :K], q).sum(axis=-1),
                "tau": float(np.mean(res["accepted"] + 1)),
                "counters": _counters(res["accepted"], np.full(B, K))})
    return res


def verify_scheduled(w: Weights, h, h_draft, draft, coins, T: float, threshold: float,
                     budget_rows: int) -> dict:
    """Confidence-scheduled verification ([DSPARK]; reading R7).

    h [B, Kmax+1, d], h_draft [B, Kmax, d], draft [B, Kmax], coins [B, Kmax+1].  The
    draft confidences come from the shared LM head over all Kmax draft rows; request b
    then verifies its first k_b drafts with coins[b, :k_b] and takes its final sample
    with coins[b, Kmax].  A request with k_b = 0 emits one token drawn from p_1.
    """
    draft = np.asarray(draft, dtype=np.int64)
    coins = np.asarray(coins, dtype=np.float64)
    B, Kmax = draft.shape
    z_d = lm_logits(w.w_lm, h_draft)
    q_all = softmax_t(z_d, T)
    conf = q_all.max(axis=-1)
    sch = survival_schedule(conf, threshold, budget_rows)
    k = sch["verify_len"]
    V = w.w_lm.shape[0]
    A = np.zeros(B, dtype=np.int64)
    emitted = np.full((B, Kmax + 1), -1, dtype=np.int64)
    ratio = np.full((B, Kmax), np.nan)
    p_x = np.full((B, Kmax), np.nan)
    q_x = np.full((B, Kmax), np.nan)
    cdf_lo = np.zeros(B)
    cdf_hi = np.zeros(B)
    fallback = np.zeros(B, dtype=bool)
    logits_t = np.full((B, Kmax + 1, V), np.nan)
    for b in range(B):
        kb = int(k[b])
        y = target_hidden(np.asarray(h[b, : kb + 1], dtype=np.float64), w)
        z_t = lm_logits(w.w_lm, y)
        logits_t[b, : kb + 1] = z_t
        p = softmax_t(z_t, T)[None]
        q = q_all[b, :kb][None]
        cb = np.concatenate([coins[b, :kb], coins[b, Kmax:]])[None]
        r = accept_sample(p, q, draft[b : b + 1, :kb], cb)
        A[b] = r["accepted"][0]
        emitted[b, : kb + 1] = r["emitted"][0]
        ratio[b, :kb] = r["ratio"][0]
        p_x[b, :kb] = r["p_x"][0]
        q_x[b, :kb] = r["q_x"][0]
        cdf_lo[b], cdf_hi[b] = r["cdf_lo"][0], r["cdf_hi"][0]
        fallback[b] = r["fallback"][0]
    return {"accepted": A, "emitted": emitted, "verify_len": k, "conf": conf,
            "survival": sch["survival"], "key": sch["key"], "eligible": sch["eligible"],
            "budget_bound": sch["budget_bound"], "ratio": ratio, "p_x": p_x, "q_x": q_x,
            "cdf_lo": cdf_lo, "cdf_hi": cdf_hi, "fallback": fallback, "logits_d": z_d,
            "logits_t": logits_t, "tau": float(np.mean(A + 1)), "counters": _counters(A, k)}
