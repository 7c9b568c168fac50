"""Plain fp64 CPU oracle for Fibonacci-spaced sparse attention (test infrastructure).

This module is TEST INFRASTRUCTURE. Only the test suite, the package's smoke
check and the benchmark's CPU-baseline leg may import or call it. The product
path (the HIP library and its Python binding) never routes through it, and it
shares no code with that path: it imports nothing but numpy and the standard
library.

Source of every definition below: the page "Depth-Staggered Fibonacci Spacing
for Sparse Attention: Static Schedules Beat Learned Dilation and Extrapolate
Where Dense Attention Fails" (C. A. Capps; gist.science technical summary),
cited as [DSFS: <section>]. Sections used:

* Methodology > Architecture and attention > Attended set: a query at
  position i sees a dense local window of W keys plus keys at distances taken
  from the Fibonacci list 1, 2, 3, 5, ..., 987.
* Methodology > Architecture and attention > Scaling: each Fibonacci distance
  f_k is multiplied by one per-layer scalar alpha in [0.5, 1.5], d_k = alpha*f_k.
* Methodology > Architecture and attention > Implementation: fractional
  distances are realised by linear interpolation between neighbouring key rows
  and neighbouring value rows, so the gradient reaches alpha; RoPE is applied
  to queries and keys before the gather (the oracle therefore receives
  post-RoPE q and k).
* Methodology > Experimental variables: the fixed (alpha = 1 everywhere),
  linear-stagger (alpha from 0.5 at layer 0 to 1.5 at the last layer) and
  coprime (the linear multiset re-assigned by l -> 7l mod L) schedules.

Readings taken where the page leaves a step open:

* R1 window: offsets 0..W-1, the query itself included, cut at position 0.
* R2 a tap with d_k < W lies inside the window and is dropped for every query.
* R3 a tap whose target position i - d_k is negative is dropped for that query.
* R4 lower row floor(i - d_k) = i - ceil(d_k); the upper row takes weight
  t_k = ceil(d_k) - d_k.
* R5 one softmax over the union of window entries and tap entries, each tap its
  own entry (no de-duplication).
* R6 score scale 1/sqrt(D).
* R7 alpha is an fp32 value; d_k is the exact fp64 product alpha*f_k.
* R8 d(alpha) at an integer d_k uses the right-hand slope K[a+1] - K[a].
* R9 the schedule for L layers: linear alpha_l = a_min + (a_max-a_min)*l/(L-1)
  evaluated in fp64 and rounded once to fp32; coprime out[(s*l) mod L] = lin[l].
* R12 RoPE (rope below): the page says only that RoPE is applied before the
  gather and that it is native, unscaled RoPE [DSFS: Significance and
  claims]. Reading: rotate-half pairs (m, m + D/2) for m < D/2, frequency
  theta_m = base^(-2m/D), row t at position pos0 + t, the pair turned by the
  angle position * theta_m.
* R14 the power-of-two control base (Methodology > Control variables) is the
  fifteen terms 1, 2, 4, ..., 16384: the page's examples of offsets first met at
  4096 tokens (1024, 2048; Core contributions and results > 3. Length
  extrapolation, base sensitivity) need a ladder past 987, and fifteen terms
  match the Fibonacci list's count.
* R16 learned alpha (Methodology > Experimental variables, Learned): one free
  parameter theta per layer, initialised so that alpha = 1, trained by
  gradient descent, alpha held in [0.5, 1.5] (Architecture and attention >
  Scaling). The page names neither the map from theta to alpha nor the
  optimizer. Two maps are provided: "clamp", alpha = clip(theta, 0.5, 1.5)
  with theta projected back into [0.5, 1.5] after every update (projected
  gradient descent; theta starts at 1), and "tanh", alpha = 1 + tanh(theta)/2
  with theta unconstrained (theta starts at 0). alpha is evaluated in fp64 and
  rounded once to fp32 (reading R7); the chain rule takes the rounding as the
  identity, dL/dtheta = dL/dalpha * dalpha/dtheta. Optimizers: plain gradient
  descent, theta <- theta - lr * g, and Adam with bias correction.
* R15 the rounded (mask) mode of the static runs (Core contributions and
  results > 2. Learned dilation is inert, efficiency) attends row i - round(d_k)
  with round to nearest, ties to even; a term is kept under the same rule
  d_k >= W and applies to query i when i >= round(d_k). The attended rows do
  not depend on alpha there, so d(loss)/d(alpha) = 0.

Every array argument is float64 (the caller up-casts the dtype-rounded inputs
exactly). Shapes are [B, H, T, D] (or a single [T, D] slab for the *_slab
helpers).
"""

from __future__ import annotations

import math
from typing import NamedTuple

import numpy as np

# [DSFS: Methodology > Architecture and attention > Attended set] -- the fifteen
# Fibonacci distances, 1 through 987, the leading 1 taken once.
FIB = (1, 2, 3, 5, 8, 13, 21, 34, 55, 89, 144, 233, 377, 610, 987)

# [DSFS: Methodology > Control variables] -- the power-of-two base, reading R14.
POW2 = tuple(2 ** n for n in range(15))

BASES = {"fib": FIB, "pow2": POW2}
MODES = ("lerp", "round")


class TapTable(NamedTuple):
    """Per base term k: distance d, lower-row distance c, upper-row weight t,
    kept flag, and the slope d(sample position)/d(alpha) of the term."""
    d: np.ndarray
    c: np.ndarray
    t: np.ndarray
    keep: np.ndarray
    slope: np.ndarray

SCHEDULE_FIXED = 0
SCHEDULE_LINEAR = 1
SCHEDULE_COPRIME = 2


# ---------------------------------------------------------------------------
# schedules  [DSFS: Methodology > Experimental variables]
# ---------------------------------------------------------------------------
def schedule(kind: int, num_layers: int = 16, a_min: float = 0.5,
             a_max: float = 1.5, stride: int = 7) -> np.ndarray:
    """Per-layer alpha table (float32), reading R9.

    fixed   -- alpha = 1 for every layer (Experimental variables, Fixed).
    linear  -- alpha rises linearly from a_min at layer 0 to a_max at the last
               layer (Experimental variables, Staggered (linear)).
    coprime -- the linear values, layer l's value moved to layer (stride*l) mod L
               (Experimental variables, Staggered (coprime/HDC)).
    """
    L = int(num_layers)
    if L < 1:
        raise ValueError("num_layers must be >= 1")
    if kind == SCHEDULE_FIXED:
        return np.ones(L, dtype=np.float32)
    if L == 1:
        lin = [a_min]
    else:
        lin = [a_min + (a_max - a_min) * (l / (L - 1)) for l in range(L)]
    lin32 = np.array(lin, dtype=np.float64).astype(np.float32)
    if kind == SCHEDULE_LINEAR:
        return lin32
    if kind == SCHEDULE_COPRIME:
        if math.gcd(stride, L) != 1:
            raise ValueError("stride must be coprime to num_layers")
        out = np.empty(L, dtype=np.float32)
        for l in range(L):
            out[(stride * l) % L] = lin32[l]
        return out
    raise ValueError("unknown schedule kind")


# ---------------------------------------------------------------------------
# offset table  [DSFS: Methodology > Architecture and attention > Scaling]
# ---------------------------------------------------------------------------
def offset_table(alpha: float, window: int, round_alpha_to_fp32: bool = True,
                 base: str = "fib", mode: str = "lerp") -> TapTable:
    """Return the TapTable of the fifteen base terms.

    d_k = alpha*f_k (exact in fp64 when alpha is an fp32 value, reading R7),
    keep_k = d_k >= W (reading R2), and
      lerp:  c_k = ceil(d_k) (distance to the lower interpolation row),
             t_k = c_k - d_k in [0, 1) (weight of the upper row, reading R4),
             slope_k = -f_k (the sample position i - alpha*f_k moves with alpha);
      round: c_k = round(d_k), ties to even, t_k = 0, slope_k = 0 (reading R15).

    `round_alpha_to_fp32=False` keeps alpha in fp64; only finite-difference
    tests use it, to step alpha by less than an fp32 ulp.
    """
    if base not in BASES or mode not in MODES:
        raise ValueError("unknown base or mode")
    a = float(np.float32(alpha)) if round_alpha_to_fp32 else float(alpha)
    f = np.array(BASES[base], dtype=np.float64)
    d = a * f
    if mode == "lerp":
        c = np.ceil(d).astype(np.int64)
        t = c.astype(np.float64) - d
        slope = -f
    else:
        # Python's round() on a float is round-half-even and exact
        c = np.array([round(float(x)) for x in d], dtype=np.int64)
        t = np.zeros_like(d)
        slope = np.zeros_like(d)
    keep = d >= float(window)
    return TapTable(d, c, t, keep, slope)


# ---------------------------------------------------------------------------
# attended entries of one (b, h) slab
# ---------------------------------------------------------------------------
def _entries(T: int, window: int, table):
    """List the attended entries as (kind, info) records.

    ("win", w): window entry at key j = i - w, valid for i >= w (reading R1).
    ("tap", k, c_k, t_k, slope_k): tap entry with lower row a = i - c_k and
    upper row a + 1, valid for i >= c_k (reading R3).
    """
    ents = []
    for w in range(min(window, T)):
        ents.append(("win", w))
    for k in range(len(table.c)):
        if table.keep[k] and table.c[k] <= T - 1:
            ents.append(("tap", k, int(table.c[k]), float(table.t[k]),
                         float(table.slope[k])))
    return ents


def _entry_rows(e, T):
    """For entry e return (first valid query i0, lower row offset, weights)."""
    if e[0] == "win":
        w = e[1]
        return w, w, 1.0, 0.0
    ck, tk = e[2], e[3]
    return ck, ck, 1.0 - tk, tk


def _gathered(X: np.ndarray, e, T: int):
    """Rows of X that entry e contributes to queries i0..T-1 (interpolated).

    Window: X[i - w]. Tap: (1 - t) X[i - c] + t X[i - c + 1] [DSFS: Methodology >
    Architecture and attention > Implementation]. Returns (i0, rows[T - i0, D]).
    """
    i0, off, w_lo, w_hi = _entry_rows(e, T)
    lo = X[i0 - off: T - off]
    if e[0] == "win":
        return i0, lo
    hi = X[i0 - off + 1: T - off + 1]
    return i0, w_lo * lo + w_hi * hi


def _scores_slab(q, k, ents, scale):
    """Score matrix S[T, E] (minus infinity where an entry is absent)."""
    T = q.shape[0]
    S = np.full((T, len(ents)), -np.inf, dtype=np.float64)
    for n, e in enumerate(ents):
        i0, key = _gathered(k, e, T)
        if i0 < T:
            S[i0:, n] = scale * np.einsum("td,td->t", q[i0:], key)
    return S


def forward_slab(q, k, v, alpha, window, table=None, base="fib", mode="lerp"):
    """Forward pass on one [T, D] slab; returns (out[T, D], lse[T]).

    One softmax over the union of window and tap entries (reading R5), scaled by
    1/sqrt(D) (reading R6): lse_i = log sum_e exp(s_ie), p_ie = exp(s_ie - lse_i),
    out_i = sum_e p_ie * value_ie [DSFS: Methodology > Architecture and
    attention > Attended set, Implementation].
    """
    T, D = q.shape
    if table is None:
        table = offset_table(alpha, window, base=base, mode=mode)
    scale = 1.0 / math.sqrt(D)
    ents = _entries(T, window, table)
    S = _scores_slab(q, k, ents, scale)
    m = S.max(axis=1)
    lse = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
    P = np.exp(S - lse[:, None])
    out = np.zeros_like(q)
    for n, e in enumerate(ents):
        i0, val = _gathered(v, e, T)
        if i0 < T:
            out[i0:] += P[i0:, n, None] * val
    return out, lse


def backward_slab(q, k, v, dout, alpha, window, table=None, base="fib",
                  mode="lerp"):
    """Backward pass on one slab; returns (dq, dk, dv, dalpha, lse).

    With p and the entry values from the forward definition:
      dP_ie = dout_i . value_ie,  Delta_i = sum_e p_ie dP_ie,
      dS_ie = p_ie (dP_ie - Delta_i),
      dq_i  = scale * sum_e dS_ie key_ie,
    and each entry hands its key/value gradient back to the rows it was
    gathered from, with the interpolation weights (1 - t) on the lower row and t
    on the upper row. Moving alpha moves the sample position i - alpha*f_k, so
      dalpha = sum over taps and queries of slope_k * [ scale*dS * q_i.(K[a+1]-K[a])
                                                        + p * dout_i.(V[a+1]-V[a]) ]
    with slope_k = -f_k when the distance interpolates and 0 in the rounded
    mode (reading R15)
    [DSFS: Methodology > Architecture and attention > Implementation (gradient
    to alpha); Experimental variables > Learned]. Reading R8 fixes the slope at
    integer distances.
    """
    T, D = q.shape
    if table is None:
        table = offset_table(alpha, window, base=base, mode=mode)
    scale = 1.0 / math.sqrt(D)
    ents = _entries(T, window, table)
    S = _scores_slab(q, k, ents, scale)
    m = S.max(axis=1)
    lse = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
    P = np.exp(S - lse[:, None])
    dP = np.zeros_like(S)
    for n, e in enumerate(ents):
        i0, val = _gathered(v, e, T)
        if i0 < T:
            dP[i0:, n] = np.einsum("td,td->t", dout[i0:], val)
    delta = (P * dP).sum(axis=1)
    dS = P * (dP - delta[:, None])
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dalpha = 0.0
    for n, e in enumerate(ents):
        i0, off, w_lo, w_hi = _entry_rows(e, T)
        if i0 >= T:
            continue
        _, key = _gathered(k, e, T)
        gs = dS[i0:, n, None]
        gp = P[i0:, n, None]
        dq[i0:] += gs * key
        # lower row a = i - off receives weight w_lo, upper row a + 1 weight w_hi
        dk[i0 - off: T - off] += w_lo * scale * gs * q[i0:]
        dv[i0 - off: T - off] += w_lo * gp * dout[i0:]
        if e[0] == "tap":
            dk[i0 - off + 1: T - off + 1] += w_hi * scale * gs * q[i0:]
            dv[i0 - off + 1: T - off + 1] += w_hi * gp * dout[i0:]
            slope = e[4]
            if slope != 0.0:
                dK = k[i0 - off + 1: T - off + 1] - k[i0 - off: T - off]
                dV = v[i0 - off + 1: T - off + 1] - v[i0 - off: T - off]
                term = (scale * dS[i0:, n] * np.einsum("td,td->t", q[i0:], dK)
                        + P[i0:, n] * np.einsum("td,td->t", dout[i0:], dV))
                dalpha += slope * float(term.sum())
    dq *= scale
    return dq, dk, dv, dalpha, lse


# ---------------------------------------------------------------------------
# batched entry points over [B, H, T, D]
# ---------------------------------------------------------------------------
def forward(q, k, v, alpha, window, base="fib", mode="lerp"):
    """Forward over [B, H, T, D] fp64 arrays; returns (out, lse)."""
    B, H, T, D = q.shape
    table = offset_table(alpha, window, base=base, mode=mode)
    out = np.empty_like(q)
    lse = np.empty((B, H, T), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            out[b, h], lse[b, h] = forward_slab(q[b, h], k[b, h], v[b, h],
                                                alpha, window, table)
    return out, lse


def backward(q, k, v, dout, alpha, window, base="fib", mode="lerp"):
    """Backward over [B, H, T, D]; returns (dq, dk, dv, dalpha) with dalpha
    summed over every batch entry, head and position."""
    B, H, T, D = q.shape
    table = offset_table(alpha, window, base=base, mode=mode)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    dalpha = 0.0
    for b in range(B):
        for h in range(H):
            g = backward_slab(q[b, h], k[b, h], v[b, h], dout[b, h], alpha,
                              window, table)
            dq[b, h], dk[b, h], dv[b, h] = g[0], g[1], g[2]
            dalpha += g[3]
    return dq, dk, dv, dalpha


# ---------------------------------------------------------------------------
# single rows, for spot checks at sizes where whole slabs are too costly
# ---------------------------------------------------------------------------
def forward_rows(q, k, v, alpha, window, rows, base="fib", mode="lerp"):
    """out[i], lse[i] of one slab for the listed query rows only."""
    T, D = q.shape
    table = offset_table(alpha, window, base=base, mode=mode)
    scale = 1.0 / math.sqrt(D)
    ents = _entries(T, window, table)
    outs, lses = [], []
    for i in rows:
        s_list, v_list = _row_entries(q, k, v, ents, int(i), scale)
        s = np.array(s_list)
        mx = s.max()
        l = mx + math.log(float(np.exp(s - mx).sum()))
        p = np.exp(s - l)
        outs.append((p[:, None] * np.array(v_list)).sum(axis=0))
        lses.append(l)
    return np.array(outs), np.array(lses)


def _row_entries(q, k, v, ents, i, scale):
    s_list, v_list = [], []
    for e in ents:
        i0, off, w_lo, w_hi = _entry_rows(e, q.shape[0])
        if i < i0:
            continue
        a = i - off
        if e[0] == "win":
            key, val = k[a], v[a]
        else:
            key = w_lo * k[a] + w_hi * k[a + 1]
            val = w_lo * v[a] + w_hi * v[a + 1]
        s_list.append(scale * float(q[i] @ key))
        v_list.append(val)
    return s_list, v_list


def dq_rows(q, k, v, dout, alpha, window, rows, base="fib", mode="lerp"):
    """dq[i] and Delta_i of one slab for the listed query rows only."""
    T, D = q.shape
    table = offset_table(alpha, window, base=base, mode=mode)
    scale = 1.0 / math.sqrt(D)
    ents = _entries(T, window, table)
    res, deltas = [], []
    for i in rows:
        i = int(i)
        s_list, v_list = _row_entries(q, k, v, ents, i, scale)
        keys = []
        for e in ents:
            i0, off, w_lo, w_hi = _entry_rows(e, T)
            if i < i0:
                continue
            a = i - off
            keys.append(k[a] if e[0] == "win" else w_lo * k[a] + w_hi * k[a + 1])
        s = np.array(s_list)
        mx = s.max()
        p = np.exp(s - (mx + math.log(float(np.exp(s - mx).sum()))))
        dp = np.array(v_list) @ dout[i]
        delta = float(p @ dp)
        ds = p * (dp - delta)
        res.append(scale * (ds[:, None] * np.array(keys)).sum(axis=0))
        deltas.append(delta)
    return np.array(res), np.array(deltas)


def dkdv_rows(q, k, v, dout, alpha, window, rows, base="fib", mode="lerp"):
    """dk[j], dv[j] of one slab for the listed key rows only, by enumerating
    every (query, entry) pair that gathers row j."""
    T, D = q.shape
    table = offset_table(alpha, window, base=base, mode=mode)
    scale = 1.0 / math.sqrt(D)
    ents = _entries(T, window, table)
    cache = {}

    def query_state(i):
        if i not in cache:
            s_list, v_list = _row_entries(q, k, v, ents, i, scale)
            s = np.array(s_list)
            mx = s.max()
            lse = mx + math.log(float(np.exp(s - mx).sum()))
            p = np.exp(s - lse)
            delta = float(p @ (np.array(v_list) @ dout[i]))
            cache[i] = (lse, delta)
        return cache[i]

    dks, dvs = [], []
    for j in rows:
        j = int(j)
        gk = np.zeros(D)
        gv = np.zeros(D)
        for e in ents:
            i0, off, w_lo, w_hi = _entry_rows(e, T)
            # row j as the lower row (weight w_lo): query i = j + off
            # row j as the upper row (weight w_hi): query i = j + off - 1
            cands = [(j + off, w_lo)]
            if e[0] == "tap":
                cands.append((j + off - 1, w_hi))
            for i, wgt in cands:
                if i < i0 or i >= T or wgt == 0.0:
                    continue
                a = i - off
                if e[0] == "win":
                    key, val = k[a], v[a]
                else:
                    key = w_lo * k[a] + w_hi * k[a + 1]
                    val = w_lo * v[a] + w_hi * v[a + 1]
                lse, delta = query_state(i)
                p = math.exp(scale * float(q[i] @ key) - lse)
                ds = p * (float(dout[i] @ val) - delta)
                gk += wgt * scale * ds * q[i]
                gv += wgt * p * dout[i]
        dks.append(gk)
        dvs.append(gv)
    return np.array(dks), np.array(dvs)


# ---------------------------------------------------------------------------
# decode: one new query per (b, h) against cached rows
# ---------------------------------------------------------------------------
def decode(q, k_cache, v_cache, pos, alpha, window, base="fib", mode="lerp"):
    """One decoding step: out[b, h] and lse[b, h] of the query q[b, h] at
    position i = pos[b], which attends the cached key and value rows 0..i of
    its (b, h) slab under the same rules as every other position: the window
    rows i-W+1..i (from row 0 on) and the kept taps with i >= c_k, each tap
    interpolating rows i-c_k and i-c_k+1 [DSFS: Methodology > Architecture and
    attention > Attended set, Scaling, Implementation]. This is the step whose
    latency the page compares between learned and static spacing [DSFS: Core
    contributions and results > 2. Learned dilation is inert, efficiency].

    q: [B, H, D]; k_cache, v_cache: [B, H, T_cap, D]; pos: B integers in
    [0, T_cap). Rows past pos[b] are never read.
    """
    B, H, D = q.shape
    table = offset_table(alpha, window, base=base, mode=mode)
    scale = 1.0 / math.sqrt(D)
    out = np.empty((B, H, D), dtype=np.float64)
    lse = np.empty((B, H), dtype=np.float64)
    for b in range(B):
        i = int(pos[b])
        if not 0 <= i < k_cache.shape[2]:
            raise ValueError("position outside the cache")
        for h in range(H):
            qi, K, V = q[b, h], k_cache[b, h], v_cache[b, h]
            scores, values = [], []
            for w in range(window):              # window rows, newest first
                j = i - w
                if j < 0:
                    break
                scores.append(scale * float(qi @ K[j]))
                values.append(V[j])
            for n in range(len(table.c)):        # kept taps that reach a row
                c = int(table.c[n])
                if not table.keep[n] or i < c:
                    continue
                a, t = i - c, float(table.t[n])
                key = (1.0 - t) * K[a] + t * K[a + 1]
                val = (1.0 - t) * V[a] + t * V[a + 1]
                scores.append(scale * float(qi @ key))
                values.append(val)
            s = np.array(scores)
            mx = s.max()
            lse[b, h] = mx + math.log(float(np.exp(s - mx).sum()))
            p = np.exp(s - lse[b, h])
            out[b, h] = (p[:, None] * np.array(values)).sum(axis=0)
    return out, lse


# ---------------------------------------------------------------------------
# rope: the rotation applied to queries and keys before the gather
# ---------------------------------------------------------------------------
def rope(x, base, pos0=None, inverse=False):
    """Rotary position embedding of rows x [B, H, T, D] in fp64 (reading R12):
    RoPE is applied to queries and keys before the gather [DSFS: Methodology >
    Architecture and attention > Implementation], native and unscaled [DSFS:
    Significance and claims]. Row t of batch entry b stands at position
    pos0[b] + t (pos0 None: t). For each m < D/2 the pair (x[m], x[m + D/2])
    turns by the angle position * base**(-2m/D); inverse=True turns by the
    negated angle, the transpose of the rotation (what maps a gradient with
    respect to rotated rows back to the rows before rotation)."""
    x = np.asarray(x, dtype=np.float64)
    B, H, T, D = x.shape
    if D % 2:
        raise ValueError("RoPE pairs need an even D")
    half = D // 2
    theta = np.array([float(base) ** (-2.0 * m / D) for m in range(half)])
    start = np.zeros(B, dtype=np.int64) if pos0 is None else np.asarray(pos0, dtype=np.int64)
    sign = -1.0 if inverse else 1.0
    y = np.empty_like(x)
    for b in range(B):
        position = (start[b] + np.arange(T)).astype(np.float64)
        angle = position[:, None] * theta[None, :]          # [T, D/2]
        c, s = np.cos(angle), sign * np.sin(angle)
        lo, hi = x[b, :, :, :half], x[b, :, :, half:]
        y[b, :, :, :half] = lo * c - hi * s
        y[b, :, :, half:] = lo * s + hi * c
    return y


# ---------------------------------------------------------------------------
# learned alpha: theta -> alpha, its slope, and the optimizer step (reading R16)
# [DSFS: Methodology > Experimental variables, Learned; Architecture and
# attention > Scaling (alpha in [0.5, 1.5])]
# ---------------------------------------------------------------------------
THETA_CLAMP = 0
THETA_TANH = 1
OPT_SGD = 0
OPT_ADAM = 1
ALPHA_MIN, ALPHA_MAX = 0.5, 1.5


def theta_init(theta_map: int) -> float:
    """The theta at which alpha = 1 (the page initialises the learned scalar
    there)."""
    return 1.0 if theta_map == THETA_CLAMP else 0.0


def theta_to_alpha(theta: float, theta_map: int) -> float:
    """alpha(theta) in fp64: clip(theta, 0.5, 1.5), or 1 + tanh(theta)/2."""
    t = float(theta)
    if theta_map == THETA_CLAMP:
        return min(max(t, ALPHA_MIN), ALPHA_MAX)
    if theta_map == THETA_TANH:
        return 1.0 + 0.5 * math.tanh(t)
    raise ValueError("unknown theta map")


def alpha_of_theta(theta: float, theta_map: int) -> float:
    """The fp32 alpha the attention layer uses: alpha(theta) rounded once."""
    return float(np.float32(theta_to_alpha(theta, theta_map)))


def dalpha_dtheta(theta: float, theta_map: int) -> float:
    """Slope of the map: 1 on the closed interval [0.5, 1.5] and 0 outside it
    for the clip; (1 - tanh(theta)^2) / 2 for the tanh map."""
    t = float(theta)
    if theta_map == THETA_CLAMP:
        return 1.0 if ALPHA_MIN <= t <= ALPHA_MAX else 0.0
    if theta_map == THETA_TANH:
        th = math.tanh(t)
        return 0.5 * (1.0 - th * th)
    raise ValueError("unknown theta map")


def theta_step(theta, dalpha, m, v, step, theta_map, optimizer, lr,
               beta1=0.9, beta2=0.999, eps=1e-8):
    """One optimizer update of every layer's theta from the layers' dL/dalpha.

    g_l = dalpha_l * dalpha/dtheta(theta_l) (chain rule, reading R16);
      gradient descent:  theta_l <- theta_l - lr * g_l;
      Adam (1-based step t = step + 1):
        m_l <- beta1 m_l + (1 - beta1) g_l,  v_l <- beta2 v_l + (1 - beta2) g_l^2,
        theta_l <- theta_l - lr * (m_l / (1 - beta1^t)) / (sqrt(v_l / (1 - beta2^t)) + eps);
    with the clip map theta is then projected onto [0.5, 1.5].
    Arguments are sequences over layers (fp32 values), step the number of
    updates already made. Returns (theta, m, v, g) as fp64 arrays; the
    library stores theta, m and v in fp32.
    """
    th = np.asarray(theta, dtype=np.float64).copy()
    da = np.asarray(dalpha, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64).copy()
    v = np.asarray(v, dtype=np.float64).copy()
    g = np.array([da[l] * dalpha_dtheta(th[l], theta_map) for l in range(len(th))])
    if optimizer == OPT_SGD:
        th = th - lr * g
    elif optimizer == OPT_ADAM:
        t = int(step) + 1
        m = beta1 * m + (1.0 - beta1) * g
        v = beta2 * v + (1.0 - beta2) * g * g
        mh = m / (1.0 - beta1 ** t)
        vh = v / (1.0 - beta2 ** t)
        th = th - lr * mh / (np.sqrt(vh) + eps)
    else:
        raise ValueError("unknown optimizer")
    if theta_map == THETA_CLAMP:
        th = np.clip(th, ALPHA_MIN, ALPHA_MAX)
    return th, m, v, g
