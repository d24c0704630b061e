"""Plain, slow, fp64 CPU oracle of the Sparse Delta Memory (SDM) hot path: the
forward pass, and the training pass (write log and reverse walk).

TEST INFRASTRUCTURE.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import or run this module.  It shares no code
with the HIP path: it takes plain numpy arrays, converts them to fp64 exactly,
and follows the method's steps one at a time.  It is never tuned for speed.

Sources (the method has no published code; these web pages define it):
  [rainbus]  "稀疏增量记忆：通过稀疏性扩展线性RNN的状态 / Sparse Delta Memory:
             Scaling the State of Linear RNNs through Sparsity",
             paper.rainbus.top/paper/2607.07386 -- the method paragraph, which
             states the four steps (sparse key selection, gated delta write,
             sparse read, normalisation + gating + head mixing) in formulas.
  [analysis] "用稀疏内存把线性RNN的状态放大1000倍：Meta SDM 在 8B 规模反超 Full
             Attention", ai-paper-analysis.pages.dev -- sections "步骤 1" to
             "步骤 4" and Figure 2 (layer diagram).
  [163]      m.163.com article on arXiv 2607.07386 -- section 二 (product-key
             "outer sum" addressing; write = forget gate + delta rule; read =
             weighted sum; unselected slots untouched).

Readings taken where the pages are silent (each listed in the design notes):
  * outer SUM of the two half-scores, slot id = i*n + j with i from the first
    half and j from the second;
  * the selection order is (score descending, slot id ascending); returned ids
    are ascending, weights aligned with them;
  * sparse key/query values k^(i), q^(i) = softmax over the selected scores;
  * alpha and beta are one scalar per (token, head); the write happens before
    the read of the same token; unselected slots are never touched;
  * RMSNorm over d_v with epsilon eps and weight gamma, then the gate
    activation (sigmoid unless stated) multiplies element-wise;
  * the output projection W_o is not part of this path.

Variant (not the pages' printed rule): scan_gdn uses Gated DeltaNet's
key-weighted error term on the write set; it is pinned against a dense
matrix-form gated delta recurrence with every slot selected.

Selection-pass backward (training): softmax_backward and pass_a_backward take the
gradients of the selection products (weights, value, gate, forget and input gates)
back to the projection output Y = x W_proj^T, to A and b_dt, and through the linear
projection to x and W_proj; the selected sets carry no gradient.

Chunkwise form ([163] section 八): scan_chunkwise computes scan / scan_gdn chunk by
chunk from the chunk-start state and the tokens' pairwise sparse inner products
(sparse_inner, a two-pointer merge over ascending slot ids); it is pinned against
the sequential scans, which define the result, and sparse_inner by brute force.
scan_backward_chunkwise is the reverse walk in the same chunks (the key-weighted
rule's de from the transposed triangular system, then each touched slot walked back
on its own); it is pinned against scan_backward.

Storage variant: scan(..., store=round_bf16) keeps a bf16 state (every written
row rounded to nearest-even bf16 from the exact value); round_bf16 is pinned
against torch's float32 -> bfloat16 conversion and hand-worked halfway cases.

Training (the [163] article, section 八: the sparse update applied in place and
undone in backward from the rows it overwrote): scan(..., record=True) keeps those
rows; scan_backward walks the tokens in reverse; quantize_rows / e4m3_encode keep
them in fp8 (OCP E4M3) or int4 with one absmax per row (the pages' fp8/int4
training checkpoints; the format details are a reading).

Pins (every function is checked against something other than itself):
  tests/test_oracle_pins.py            selection, gates, scan, norm, whole layer:
                                       hand-worked fixtures (tests/golden/, the
                                       layer's wiring from x in layer_wiring.json),
                                       closed forms, exact rationals, brute force,
                                       invariants
  tests/test_oracle_mutations.py       planted mistakes, each caught by a pin
  tests/test_oracle_gdn_pins.py        scan_gdn against a dense matrix recurrence
  tests/test_oracle_bf16_pins.py       round_bf16 and the bf16-storage scan
  tests/test_oracle_fp8_state_pins.py  the fp8 state format (block exponent, E4M3
                                       rounding against torch's float8_e4m3fn, a
                                       hand-worked row) and the fp8-storage scan
  tests/test_oracle_histogram_pins.py  slot_update_counts by brute force
  tests/test_oracle_shared_m0_pins.py  forward_walk_shared against plain walks
  tests/test_oracle_gdn_backward_pins.py
                                       scan_backward(rule="gdn") against central
                                       differences of scan_gdn
  tests/test_oracle_backward_pins.py   scan_backward against central differences
  tests/test_oracle_select_backward_pins.py
                                       pass_a_backward chained after scan_backward
                                       against central differences of the whole
                                       layer from x (x, W_proj, A, b_dt)
  tests/test_oracle_chunk_pins.py      scan_chunkwise against scan / scan_gdn for
                                       many chunk sizes, sparse_inner by brute force
  tests/test_oracle_chunk_backward_pins.py
                                       scan_backward_chunkwise against scan_backward
                                       for many chunk sizes, identity gates
  tests/test_oracle_quant_pins.py      E4M3 against torch's float8_e4m3fn, int4
                                       packing by hand, error bounds
No function of this module is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

F64 = np.float64

# gate activations for the output gate vector
GATE_NONE, GATE_SIGMOID, GATE_SILU = 0, 1, 2


# ----------------------------------------------------------------------------
# Step 1a: input projections.  [rainbus] method paragraph, step 1: W_k and W_q
# map x_t in R^d to R^{2 sqrt(N)}; [analysis] "步骤 1" and the isoFLOP section
# (W_v).  One dense product Y = x W_proj^T covers every projection of a head;
# per head its P = 4n + 2 d_v + 2 columns are, in order,
#   [write half 1 (n) | write half 2 (n) | read half 1 (n) | read half 2 (n) |
#    value v (d_v) | output-gate pre-activation (d_v) | forget pre-gate a |
#    input pre-gate b].
# ----------------------------------------------------------------------------
def project(x, w_proj):
    """Y = x @ W_proj^T in fp64.  x [..., d], w_proj [H*P, d] -> [..., H*P]."""
    return np.asarray(x, F64) @ np.asarray(w_proj, F64).T


def split_heads(Y, H: int, n: int, d_v: int):
    """Split Y [..., H*P] into the per-head pieces listed above."""
    P = 4 * n + 2 * d_v + 2
    Y = np.asarray(Y, F64)
    Yh = Y.reshape(Y.shape[:-1] + (H, P))
    o = 4 * n
    return dict(
        kw1=Yh[..., 0:n], kw2=Yh[..., n:2 * n],
        kr1=Yh[..., 2 * n:3 * n], kr2=Yh[..., 3 * n:4 * n],
        v=Yh[..., o:o + d_v], g=Yh[..., o + d_v:o + 2 * d_v],
        a=Yh[..., o + 2 * d_v], b=Yh[..., o + 2 * d_v + 1],
    )


# ----------------------------------------------------------------------------
# Step 2 gates.  [rainbus] step 2 and [analysis] "步骤 2":
#   alpha_t = exp(-A * softplus(W_a x_t + b_dt))   (per-head forget gate)
#   beta_t  = sigma(W_b x_t)                        (input gate)
# ----------------------------------------------------------------------------
def softplus(z):
    z = np.asarray(z, F64)
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def sigmoid(z):
    z = np.asarray(z, F64)
    return 1.0 / (1.0 + np.exp(-z))


def forget_gate(a, A, b_dt):
    """alpha = exp(-A * softplus(a + b_dt)); A and b_dt broadcast over heads."""
    return np.exp(-np.asarray(A, F64) * softplus(np.asarray(a, F64) + np.asarray(b_dt, F64)))


def input_gate(b):
    return sigmoid(b)


def gate_activation(g, kind: int = GATE_SIGMOID):
    g = np.asarray(g, F64)
    if kind == GATE_NONE:
        return g
    if kind == GATE_SIGMOID:
        return sigmoid(g)
    if kind == GATE_SILU:
        return g * sigmoid(g)
    raise ValueError(f"unknown gate activation {kind}")


# ----------------------------------------------------------------------------
# Step 1b: sparse slot selection.  [rainbus] step 1: the two halves of a
# pre-index vector form N = n*n scores by an outer sum, one per memory slot;
# top-W of the write scores and top-R of the read scores pick the slots.
# [analysis] "步骤 1" and [163] section 二 state the same outer-sum addressing.
# The product-key shortcut reaches exactly this set, so the oracle uses the
# plain definition: score every slot and take the best `count`.
# ----------------------------------------------------------------------------
def slot_scores(half1, half2):
    """All N outer-sum scores, slot id = i*n + j."""
    h1 = np.asarray(half1, F64)
    h2 = np.asarray(half2, F64)
    return (h1[:, None] + h2[None, :]).reshape(-1)


def top_slots(half1, half2, count: int):
    """Best `count` slots by (score desc, id asc).

    Returns (ids ascending [count] int64, their scores fp64, gap) where gap is
    the difference between the count-th and (count+1)-th largest scores
    (inf when every slot is selected).
    """
    S = slot_scores(half1, half2)
    N = S.shape[0]
    if not 1 <= count <= N:
        raise ValueError("count must be in [1, N]")
    if count < N:
        part = np.partition(S, [N - count - 1, N - count])
        kth, nxt = part[N - count], part[N - count - 1]
        gap = float(kth - nxt)
    else:
        kth = S.min()
        gap = float("inf")
    above = np.flatnonzero(S > kth)
    ties = np.flatnonzero(S == kth)           # ascending ids: lowest ids win
    ids = np.concatenate([above, ties[:count - above.size]])
    ids.sort()
    return ids.astype(np.int64), S[ids], gap


def softmax(s):
    """Sparse key/query values over the selected scores (temperature 1)."""
    s = np.asarray(s, F64)
    e = np.exp(s - s.max())
    return e / e.sum()


def select(half1, half2, count: int):
    """(ids ascending, softmax weights aligned with ids, gap)."""
    ids, sc, gap = top_slots(half1, half2, count)
    return ids, softmax(sc), gap


# ----------------------------------------------------------------------------
# Steps 2-3: the recurrent sparse scan of one (batch, head) memory.
# [rainbus] step 2: for each selected write slot i, first the forget gate
#   Mtilde[i] = alpha_t * M_{t-1}[i], then the delta update
#   M_t[i] = Mtilde[i] + beta_t * k^(i) * (v_t - Mtilde[i]);
# [analysis] "步骤 2": slots that are not selected keep M_t[i] = M_{t-1}[i].
# [rainbus] step 3: y_t = sum_{i in I_r} q^(i) M_t[i]  (reads the state after
# this token's write).
# ----------------------------------------------------------------------------
def scan(state0, idx_w, wt_w, idx_r, wt_r, v, alpha, beta, store=None, record=False):
    """Walk tokens in order over one memory.

    state0 [N, d_v]; idx_w/wt_w [T, W]; idx_r/wt_r [T, R]; v [T, d_v];
    alpha, beta [T].  Returns (y_raw [T, d_v], final state [N, d_v]) in fp64.
    store: None (the state holds the exact values), or a rounding function applied
    to every written row, the state then holding only its results (round_bf16 for
    a bf16 state); state0 must then be representable already.
    record: also return the rows each token overwrote, log [T, W, d_v] (the values
    of M[idx_w[t]] just before token t's write), as a third result.
    """
    M = np.array(state0, dtype=F64, copy=True)
    keep = store if store is not None else (lambda z: z)
    assert np.array_equal(keep(M), M), "state0 is not representable in the state's format"
    idx_w = np.asarray(idx_w)
    idx_r = np.asarray(idx_r)
    wt_w = np.asarray(wt_w, F64)
    wt_r = np.asarray(wt_r, F64)
    v = np.asarray(v, F64)
    alpha = np.asarray(alpha, F64)
    beta = np.asarray(beta, F64)
    T = idx_w.shape[0]
    y = np.zeros((T, M.shape[1]), F64)
    log = np.zeros((T, idx_w.shape[1], M.shape[1]), F64) if record else None
    for t in range(T):
        rows = idx_w[t]
        assert np.unique(rows).size == rows.size, "write slots of one token must be distinct"
        if record:
            log[t] = M[rows]
        m_tilde = alpha[t] * M[rows]                                   # forget gate
        M[rows] = keep(m_tilde + (beta[t] * wt_w[t])[:, None] * (v[t][None, :] - m_tilde))
        y[t] = wt_r[t] @ M[idx_r[t]]                                   # sparse read
    return (y, M, log) if record else (y, M)


# ----------------------------------------------------------------------------
# Variant: the gated delta rule of Gated DeltaNet restricted to the write set.
# [analysis] section "与 GDN 的关系" and [163] section 二 state that with every
# slot selected (W = R = N = d_qk) and a dense key the layer becomes Gated
# DeltaNet's update.  GDN's rule S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T)
# + beta_t v_t k_t^T is not printed on the pages; written per key row i it is
#   Mtilde = alpha_t * M_{t-1}            (forget gate, on the write set)
#   M_t[i] = Mtilde[i] + beta_t k^(i) (v_t - sum_j k^(j) Mtilde[j])
# i.e. the error term subtracts the key-weighted prediction of the whole write
# set instead of the slot's own value.  Reads are unchanged.
# ----------------------------------------------------------------------------
def scan_gdn(state0, idx_w, wt_w, idx_r, wt_r, v, alpha, beta, store=None, record=False):
    """Like scan(), with the key-weighted error term above (record: also the rows each
    token overwrote, as scan() keeps them)."""
    M = np.array(state0, dtype=F64, copy=True)
    keep = store if store is not None else (lambda z: z)
    assert np.array_equal(keep(M), M), "state0 is not representable in the state's format"
    idx_w = np.asarray(idx_w)
    idx_r = np.asarray(idx_r)
    wt_w = np.asarray(wt_w, F64)
    wt_r = np.asarray(wt_r, F64)
    v = np.asarray(v, F64)
    alpha = np.asarray(alpha, F64)
    beta = np.asarray(beta, F64)
    T = idx_w.shape[0]
    y = np.zeros((T, M.shape[1]), F64)
    log = np.zeros((T, idx_w.shape[1], M.shape[1]), F64) if record else None
    for t in range(T):
        rows = idx_w[t]
        assert np.unique(rows).size == rows.size, "write slots of one token must be distinct"
        if record:
            log[t] = M[rows]
        k = wt_w[t]
        m_tilde = alpha[t] * M[rows]                                   # forget gate
        pred = k @ m_tilde                                             # key-weighted prediction
        M[rows] = keep(m_tilde + (beta[t] * k)[:, None] * (v[t] - pred)[None, :])
        y[t] = wt_r[t] @ M[idx_r[t]]                                   # sparse read
    return (y, M, log) if record else (y, M)


# ----------------------------------------------------------------------------
# Chunkwise-parallel form of the same recurrences ([163] section 八, training
# paragraph; [rainbus] the paragraph on novelty, chunk-wise parallelism through
# the WY representation).  The sequence is cut into fixed-size chunks; inside a
# chunk the tokens' mutual influence is a sparse inner product of their sorted
# slot lists, found by a two-pointer merge; across chunks the state is carried
# serially.  Derivation (exact, a reordering of the same arithmetic):
#   every written slot j of token u evolves as M[j] <- a_{u,j} M[j] + k_{u,j} x_u,
#   with a_{u,j} = alpha_u (1 - beta_u k_{u,j}), x_u = beta_u v_u   (scan), or
#        a_{u,j} = alpha_u,
#        x_u = beta_u (v_u - alpha_u sum_{j in W_u} k_{u,j} M_{u-1}[j])   (scan_gdn).
#   With G_j(s, t] = product of a_{u,j} over chunk tokens s < u <= t writing j
#   (1 if none) and M0 the state at the chunk start (token c0 - 1):
#     M_t[j] = G_j(c0-1, t] M0[j] + sum_{s <= t, j in W_s} G_j(s, t] k_{s,j} x_s
#     y_t    = sum_{j in R_t} q_{t,j} G_j(c0-1, t] M0[j] + sum_{s <= t} A_{t,s} x_s,
#              A_{t,s} = sum_{j in R_t and W_s} q_{t,j} G_j(s, t] k_{s,j}
#   and for scan_gdn, since alpha_t G_j(s, t-1] = G_j(s, t] on j in W_t,
#     x_t = beta_t (v_t - sum_{j in W_t} k_{t,j} G_j(c0-1, t] M0[j]
#                        - sum_{s < t} B_{t,s} x_s),
#              B_{t,s} = sum_{j in W_t and W_s} k_{t,j} G_j(s, t] k_{s,j},
#   a unit lower-triangular system in the chunk's x (the WY/UT form), solved by
#   forward substitution.  The chunk-end state follows from M_t at the last token.
# ----------------------------------------------------------------------------
def sparse_inner(ids_a, ids_b, term):
    """Two-pointer merge of two ascending id lists: the sum of term(p, q) over the
    positions p, q with ids_a[p] == ids_b[q] (each common id once)."""
    p = q = 0
    acc = 0.0
    while p < len(ids_a) and q < len(ids_b):
        if ids_a[p] < ids_b[q]:
            p += 1
        elif ids_a[p] > ids_b[q]:
            q += 1
        else:
            acc += term(p, q)
            p += 1
            q += 1
    return acc


def scan_chunkwise(state0, idx_w, wt_w, idx_r, wt_r, v, alpha, beta, C: int, rule: str = "slot"):
    """scan() (rule "slot") or scan_gdn() (rule "gdn") in the chunkwise form above,
    with chunks of C tokens (the last one ragged).  Returns (y_raw, final state)."""
    M = np.array(state0, dtype=F64, copy=True)
    idx_w = np.asarray(idx_w)
    idx_r = np.asarray(idx_r)
    wt_w = np.asarray(wt_w, F64)
    wt_r = np.asarray(wt_r, F64)
    v = np.asarray(v, F64)
    alpha = np.asarray(alpha, F64)
    beta = np.asarray(beta, F64)
    T = idx_w.shape[0]
    y = np.zeros((T, M.shape[1]), F64)
    for c0 in range(0, T, C):
        toks = range(c0, min(c0 + C, T))
        pos = {u: {int(j): k for k, j in enumerate(idx_w[u])} for u in toks}   # slot -> k

        def a(u, j):                       # decay of slot j by token u, if u writes j
            k = pos[u].get(j)
            if k is None:
                return 1.0
            return alpha[u] * (1.0 - beta[u] * wt_w[u, k]) if rule == "slot" else alpha[u]

        def G(j, s, t):                    # product of a(u, j) over s < u <= t
            g = 1.0
            for u in range(s + 1, t + 1):
                g *= a(u, j)
            return g

        M0 = M.copy()
        x = {}
        for t in toks:
            if rule == "slot":
                x[t] = beta[t] * v[t]
            else:
                rhs = v[t].copy()
                for k, j in enumerate(idx_w[t]):
                    rhs -= wt_w[t, k] * G(int(j), c0 - 1, t) * M0[j]
                for s in range(c0, t):
                    b_ts = sparse_inner(idx_w[t], idx_w[s], lambda p, q, t=t, s=s:
                                        wt_w[t, p] * G(int(idx_w[t, p]), s, t) * wt_w[s, q])
                    rhs -= b_ts * x[s]
                x[t] = beta[t] * rhs
        for t in toks:
            for k, j in enumerate(idx_r[t]):
                y[t] += wt_r[t, k] * G(int(j), c0 - 1, t) * M0[j]
            for s in range(c0, t + 1):
                a_ts = sparse_inner(idx_r[t], idx_w[s], lambda p, q, t=t, s=s:
                                    wt_r[t, p] * G(int(idx_r[t, p]), s, t) * wt_w[s, q])
                y[t] += a_ts * x[s]
        end = toks[-1]
        for j in sorted({int(j) for u in toks for j in idx_w[u]}):
            row = G(j, c0 - 1, end) * M0[j]
            for s in toks:
                k = pos[s].get(j)
                if k is not None:
                    row = row + G(j, s, end) * wt_w[s, k] * x[s]
            M[j] = row
    return y, M


# ----------------------------------------------------------------------------
# Reduced-precision state storage (not a step of the pages, which keep the live
# state in full precision and quantise only training checkpoints: [analysis]
# section "训练效率", [163] section 八).  bf16 is IEEE binary32 with the low 16
# fraction bits dropped: 8 significant bits, the same exponent range (normal
# numbers down to 2^-126, subnormals spaced 2^-133).  Round to nearest, ties to
# the even significand, from the exact fp64 value (one rounding).
# ----------------------------------------------------------------------------
def round_bf16(x):
    """Nearest bf16 value of each element of x (ties to even), as fp64."""
    x = np.asarray(x, F64)
    with np.errstate(over="ignore", invalid="ignore"):
        _, e = np.frexp(x)                   # x = m 2^e, 0.5 <= |m| < 1
        e = np.maximum(e, -125)              # below 2^-126: the subnormal spacing 2^-133
        q = np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)   # 8 significant bits
        q = np.where(np.abs(q) >= 2.0 ** 128, np.copysign(np.inf, x), q)
    return np.where(np.isfinite(x), q, x)


# fp8 state storage (also not a step of the pages; the same caveat as bf16).  Each
# row of d_v values is cut into blocks of 32 columns; a block keeps one power-of-two
# scale 2^e (an E8M0 byte, s = e + 127) and each element an OCP E4M3 value c, the
# element being c 2^e.  e is the least integer >= -127 with absmax <= 448 2^e, so
# x 2^-e is exact and never beyond E4M3's largest value 448; c is the E4M3 value
# nearest to x 2^-e (ties to the even significand).  Rounded once from the exact
# value, as round_bf16.
# ----------------------------------------------------------------------------
FP8_BLOCK = 32


def fp8_block_exponent(amax):
    """Least integer e >= -127 with amax <= 448 * 2^e (amax >= 0)."""
    a = np.asarray(amax, F64)
    m, k = np.frexp(a)                        # a = m 2^k, 0.5 <= m < 1 (m = 0 for a = 0)
    e = (k - 1) - 8 + (2.0 * m > 1.75)        # a = (2m) 2^(k-1): 1.75 2^8 = 448
    return np.where(a > 0, np.maximum(e, -127), -127).astype(np.int64)


def round_e4m3(x):
    """Nearest OCP E4M3 value of each element (|x| <= 448), ties to even, as fp64.
    E4M3: 3 fraction bits, exponents -6 to 8, subnormals spaced 2^-9."""
    x = np.asarray(x, F64)
    a = np.abs(x)
    _, k = np.frexp(np.where(a > 0, a, 1.0))   # a in [2^(k-1), 2^k)
    step = np.ldexp(1.0, np.maximum(k - 1, -6) - 3)
    q = np.rint(a / step) * step               # a / step is exact (a power-of-two step)
    assert np.all(q <= 448.0), "beyond E4M3's range"
    return np.copysign(q, x)


def round_fp8_blocks(x):
    """Rows [..., d] (d a multiple of 32) as the fp8 state stores them, fp64."""
    x = np.asarray(x, F64)
    blk = x.reshape(x.shape[:-1] + (x.shape[-1] // FP8_BLOCK, FP8_BLOCK))
    e = fp8_block_exponent(np.max(np.abs(blk), axis=-1))[..., None]
    return (round_e4m3(np.ldexp(blk, -e)) * np.ldexp(1.0, e)).reshape(x.shape)


def fp8_state_encode(x):
    """Rows [..., d] -> (E4M3 codes [..., d] uint8, E8M0 exponents [..., d/32] uint8)
    of round_fp8_blocks(x)."""
    x = np.asarray(x, F64)
    blk = x.reshape(x.shape[:-1] + (x.shape[-1] // FP8_BLOCK, FP8_BLOCK))
    e = fp8_block_exponent(np.max(np.abs(blk), axis=-1))
    c = round_e4m3(np.ldexp(blk, -e[..., None])).astype(np.float32)
    return e4m3_encode(c).reshape(x.shape), (e + 127).astype(np.uint8)


def fp8_state_decode(codes, exps):
    codes = np.asarray(codes, np.uint8)
    e = np.asarray(exps, np.int64) - 127
    c = e4m3_decode(codes).reshape(codes.shape[:-1] + (codes.shape[-1] // FP8_BLOCK, FP8_BLOCK))
    return (c * np.ldexp(1.0, e)[..., None]).reshape(codes.shape)


# ----------------------------------------------------------------------------
# Slot-update histogram: the collapse monitor of the papers.ananclaw.com summary
# (engineering-risks section, risk 3 "寻址坍缩"): how often each slot of each
# head's memory is written, so that updates piling onto a few slots show up.
# ----------------------------------------------------------------------------
def slot_update_counts(idx_w, N: int):
    """idx_w [B, T, H, W] write ids -> counts [H, N]: for each head and slot, the
    number of (b, t) whose write set contains the slot."""
    idx_w = np.asarray(idx_w)
    B, T, H, W = idx_w.shape
    counts = np.zeros((H, N), np.int64)
    for h in range(H):
        ids = idx_w[:, :, h, :].reshape(-1)
        counts[h] = np.bincount(ids, minlength=N)[:N]
    return counts


# ----------------------------------------------------------------------------
# Step 4 (without the head-mixing projection): [rainbus] step 4 and
# [analysis] "步骤 4": RMS-Norm of the read vector, then element-wise gating.
# ----------------------------------------------------------------------------
def rms_norm_gate(y, gamma, gate, eps: float):
    y = np.asarray(y, F64)
    r = 1.0 / np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + eps)
    return y * r * np.asarray(gamma, F64) * np.asarray(gate, F64)


# ----------------------------------------------------------------------------
# Whole path.
# ----------------------------------------------------------------------------
def pass_a(x, w_proj, A, b_dt, H, n, d_v, W, R, gate_act=GATE_SIGMOID):
    """Projections, gates and selections for tokens x [..., d].

    Returns a dict of arrays shaped [..., H, *]: idx_w, wt_w, gap_w, idx_r, wt_r,
    gap_r, v, g (activated), alpha, beta, and the four half-score blocks.
    """
    parts = split_heads(project(x, w_proj), H, n, d_v)
    lead = parts["a"].shape            # [..., H]
    out = dict(
        v=parts["v"], g=gate_activation(parts["g"], gate_act),
        alpha=forget_gate(parts["a"], np.asarray(A, F64), np.asarray(b_dt, F64)),
        beta=input_gate(parts["b"]),
        scores=np.concatenate([parts["kw1"], parts["kw2"], parts["kr1"], parts["kr2"]], axis=-1),
        a_pre=parts["a"], b_pre=parts["b"], g_pre=parts["g"],
    )
    out.update(select_from_scores(out["scores"], n, W, R))
    assert out["idx_w"].shape[:-1] == lead
    return out


def select_from_scores(scores, n, W, R):
    """Selections from half-scores [..., 4n] (write half 1|2, read half 1|2)."""
    scores = np.asarray(scores, F64)
    lead = scores.shape[:-1]
    flat = scores.reshape(-1, 4 * n)
    res = {k: [] for k in ("idx_w", "wt_w", "gap_w", "idx_r", "wt_r", "gap_r")}
    for s in flat:
        i, w, gp = select(s[0:n], s[n:2 * n], W)
        res["idx_w"].append(i); res["wt_w"].append(w); res["gap_w"].append(gp)
        i, w, gp = select(s[2 * n:3 * n], s[3 * n:4 * n], R)
        res["idx_r"].append(i); res["wt_r"].append(w); res["gap_r"].append(gp)
    shp = {"idx_w": (W,), "wt_w": (W,), "gap_w": (), "idx_r": (R,), "wt_r": (R,), "gap_r": ()}
    return {k: np.array(v).reshape(lead + shp[k]) for k, v in res.items()}


def forward_walk(state0, sel, gamma_h, eps, rule: str = "slot", state: str = "exact"):
    """Scan + norm/gate for one (batch, head) walk given its pass-(a) products.

    sel holds [T, *] arrays for that walk: idx_w, wt_w, idx_r, wt_r, v, g,
    alpha, beta.  rule "slot" is the pages' per-slot error term (scan), "gdn"
    the key-weighted one (scan_gdn).  state "exact" keeps the state in fp64,
    "bf16" stores every written row rounded to bf16, "fp8" in 32-column blocks of
    E4M3 values with a power-of-two scale (round_fp8_blocks).  Returns (out [T, d_v],
    y_raw [T, d_v], final state).
    """
    walk = {"slot": scan, "gdn": scan_gdn}[rule]
    store = {"exact": None, "bf16": round_bf16, "fp8": round_fp8_blocks}[state]
    y, M = walk(state0, sel["idx_w"], sel["wt_w"], sel["idx_r"], sel["wt_r"],
                sel["v"], sel["alpha"], sel["beta"], store=store)
    return rms_norm_gate(y, gamma_h, sel["g"], eps), y, M


# ----------------------------------------------------------------------------
# Backward of the scan and the norm/gate (steps 2-4), reverse-mode by the chain
# rule.  The training scheme of [163] section 八 (memory-efficiency paragraph):
# the sparse update is applied in place and undone in backward, which needs the
# N x d state plus the T x W x d rows the writes overwrote.  So the forward
# records, per token, the rows before its write (scan(..., record=True)), and
# the backward walks tokens in reverse: the read of token t first (it saw the
# state after t's write), then the write, restoring the overwritten rows.
# For one written row, with c = beta k and m the row before the write,
#   M' = m~ + c (v - m~),  m~ = alpha m:
#   dM'/dm = alpha (1 - c),  dM'/dv = c,  dM'/dc = v - alpha m,
#   dM'/dalpha = (1 - c) m,  dc/dbeta = k,  dc/dk = beta.
# The key-weighted write (scan_gdn), for the write set's rows m_i before the write,
# m~ = alpha m, e = v - sum_i k_i m~_i, M'_i = m~_i + beta k_i e, and G_i = dL/dM'_i:
#   de = beta sum_i k_i G_i  (= d_v),   dm~_i = G_i - k_i de,
#   dk_i = beta <G_i, e> - <de, m~_i>,  dbeta = sum_i k_i <G_i, e>,
#   dalpha = sum_i <dm~_i, m_i>,        dL/dm_i = alpha dm~_i.
# For the read y = sum_r q_r M[r]: dq_r = <dy, M[r]>, dM[r] += q_r dy.
# For out = y s gamma g with s = (mean(y^2) + eps)^(-1/2), u = d_out gamma g:
#   dy = s (u - yhat mean(u yhat)),  yhat = y s;  d_gate = d_out yhat gamma;
#   d_gamma = sum over tokens of d_out yhat g.
# ----------------------------------------------------------------------------
def scan_backward(state_T, log, idx_w, wt_w, idx_r, wt_r, v, alpha, beta, y, gate,
                  gamma_h, eps, d_out, d_state, rule: str = "slot"):
    """Gradients of one walk.

    state_T [N, d_v] the state after the forward; log [T, W, d_v] from
    scan(..., record=True) (rule "slot") or scan_gdn(..., record=True) (rule "gdn");
    y [T, d_v] the forward's read vectors; d_out [T, d_v]
    and d_state [N, d_v] (gradient of the final state) are the incoming gradients.
    Returns (grads, state_0, d_state_0) with grads holding d_v, d_gate [T, d_v],
    d_alpha, d_beta [T], d_wt_w [T, W], d_wt_r [T, R], d_gamma [d_v]; state_0 is the
    restored initial state and d_state_0 the gradient of the initial state.
    """
    M = np.array(state_T, F64, copy=True)
    dM = np.array(d_state, F64, copy=True)
    idx_w, idx_r = np.asarray(idx_w), np.asarray(idx_r)
    wt_w, wt_r = np.asarray(wt_w, F64), np.asarray(wt_r, F64)
    v, y, gate = np.asarray(v, F64), np.asarray(y, F64), np.asarray(gate, F64)
    alpha, beta = np.asarray(alpha, F64), np.asarray(beta, F64)
    gamma_h, d_out, log = np.asarray(gamma_h, F64), np.asarray(d_out, F64), np.asarray(log, F64)
    T, d_v = y.shape
    g = dict(d_v=np.zeros((T, d_v)), d_gate=np.zeros((T, d_v)), d_alpha=np.zeros(T),
             d_beta=np.zeros(T), d_wt_w=np.zeros(idx_w.shape), d_wt_r=np.zeros(idx_r.shape),
             d_gamma=np.zeros(d_v))
    for t in range(T - 1, -1, -1):
        s = 1.0 / np.sqrt(np.mean(y[t] * y[t]) + eps)                # step 4
        yhat = y[t] * s
        g["d_gate"][t] = d_out[t] * yhat * gamma_h
        g["d_gamma"] += d_out[t] * yhat * gate[t]
        u = d_out[t] * gamma_h * gate[t]
        dy = s * (u - yhat * np.mean(u * yhat))
        rows = idx_r[t]                                              # step 3
        g["d_wt_r"][t] = M[rows] @ dy
        dM[rows] += wt_r[t][:, None] * dy[None, :]
        rows = idx_w[t]                                              # step 2, undone
        m = log[t]
        G = dM[rows]
        if rule == "gdn":
            k = wt_w[t]
            mt = alpha[t] * m
            e = v[t] - k @ mt
            de = beta[t] * (k @ G)
            dmt = G - np.outer(k, de)
            g["d_v"][t] = de
            g["d_wt_w"][t] = beta[t] * (G @ e) - mt @ de
            g["d_beta"][t] = k @ (G @ e)
            g["d_alpha"][t] = np.sum(dmt * m)
            dM[rows] = alpha[t] * dmt
            M[rows] = m
            continue
        c = beta[t] * wt_w[t]
        g["d_v"][t] = c @ G
        dc = np.sum(G * (v[t][None, :] - alpha[t] * m), axis=1)
        g["d_alpha"][t] = np.sum((1.0 - c)[:, None] * G * m)
        g["d_beta"][t] = wt_w[t] @ dc
        g["d_wt_w"][t] = beta[t] * dc
        dM[rows] = (alpha[t] * (1.0 - c))[:, None] * G
        M[rows] = m
    return g, M, dM


# ----------------------------------------------------------------------------
# The same backward in the chunkwise form ([163] section 八: fixed-size chunks,
# parallel inside a chunk, serial across chunks; the in-place update undone from
# the log).  In the reverse walk above the only coupling between different slots
# of one chunk is the key-weighted rule's de_u = beta_u sum_{j in W_u} k_{u,j} G_{u,j},
# where G_{u,j} is dL/dM[j] just after token u's write.  Following slot j back from
# the chunk end (writers u' of j after u, reads (t, j) at tokens t >= u):
#   G_{u,j} = G_j(u, end] dM_end[j] + sum_t q_{t,j} G_j(u, t] dy_t
#             - sum_{u'} k_{u',j} G_j(u, u'] de_{u'}          (key-weighted rule only)
# so, with the forward's A and B (chunkwise form above),
#   de_u = beta_u (h_u - sum_{t > u} B_{t,u} de_t),
#   h_u  = sum_{t >= u} A_{t,u} dy_t + sum_{j in W_u} k_{u,j} G_j(u, end] dM_end[j]:
# the transposed unit triangular system, solved by back substitution.  With de
# known, every slot touched in the chunk is walked back on its own (reads, then
# the write, of each token): the read gradients, the G of each write, the restored
# row and the chunk-start gradient, the same per-entry steps as the reverse walk.
# ----------------------------------------------------------------------------
def _norm_gate_backward(y, gate, gamma_h, eps, d_out):
    """dy, d_gate and the d_gamma terms of out = RMSNorm(y) gamma gate, per token."""
    s = 1.0 / np.sqrt(np.mean(y * y, axis=1, keepdims=True) + eps)
    yhat = y * s
    u = d_out * gamma_h * gate
    dy = s * (u - yhat * np.mean(u * yhat, axis=1, keepdims=True))
    return dy, d_out * yhat * gamma_h, d_out * yhat * gate


def scan_backward_chunkwise(state_T, log, idx_w, wt_w, idx_r, wt_r, v, alpha, beta, y, gate,
                            gamma_h, eps, d_out, d_state, C: int, rule: str = "slot"):
    """scan_backward() in the chunkwise form above, chunks of C tokens (the last one
    ragged), walked from the last chunk to the first.  Same arguments and results."""
    M = np.array(state_T, F64, copy=True)
    dM = np.array(d_state, F64, copy=True)
    idx_w, idx_r = np.asarray(idx_w), np.asarray(idx_r)
    wt_w, wt_r = np.asarray(wt_w, F64), np.asarray(wt_r, F64)
    v, y, gate = np.asarray(v, F64), np.asarray(y, F64), np.asarray(gate, F64)
    alpha, beta = np.asarray(alpha, F64), np.asarray(beta, F64)
    gamma_h, d_out, log = np.asarray(gamma_h, F64), np.asarray(d_out, F64), np.asarray(log, F64)
    T, d_v = y.shape
    gdn = rule == "gdn"
    g = dict(d_v=np.zeros((T, d_v)), d_gate=np.zeros((T, d_v)), d_alpha=np.zeros(T),
             d_beta=np.zeros(T), d_wt_w=np.zeros(idx_w.shape), d_wt_r=np.zeros(idx_r.shape),
             d_gamma=np.zeros(d_v))
    dy, g["d_gate"], dgam = _norm_gate_backward(y, gate, gamma_h, eps, d_out)
    g["d_gamma"] = dgam.sum(axis=0)
    starts = list(range(0, T, C))
    for c0 in reversed(starts):
        toks = range(c0, min(c0 + C, T))
        end = toks[-1]
        pos = {u: {int(j): k for k, j in enumerate(idx_w[u])} for u in toks}
        rpos = {u: {int(j): k for k, j in enumerate(idx_r[u])} for u in toks}

        def a(u, j):
            k = pos[u].get(j)
            if k is None:
                return 1.0
            return alpha[u] if gdn else alpha[u] * (1.0 - beta[u] * wt_w[u, k])

        def G(j, s, t):                    # product of a(u, j) over s < u <= t
            out = 1.0
            for u in range(s + 1, t + 1):
                out *= a(u, j)
            return out

        de = {u: np.zeros(d_v) for u in toks}
        if gdn:
            h = {}
            for u in toks:
                hu = np.zeros(d_v)
                for t in range(u, end + 1):
                    a_tu = sparse_inner(idx_r[t], idx_w[u], lambda p, q, t=t, u=u:
                                        wt_r[t, p] * G(int(idx_r[t, p]), u, t) * wt_w[u, q])
                    hu += a_tu * dy[t]
                for k, j in enumerate(idx_w[u]):
                    hu += wt_w[u, k] * G(int(j), u, end) * dM[j]
                h[u] = hu
            for u in reversed(toks):       # back substitution, B transposed
                rhs = h[u].copy()
                for t in range(u + 1, end + 1):
                    b_tu = sparse_inner(idx_w[t], idx_w[u], lambda p, q, t=t, u=u:
                                        wt_w[t, p] * G(int(idx_w[t, p]), u, t) * wt_w[u, q])
                    rhs -= b_tu * de[t]
                de[u] = beta[u] * rhs
        # every slot the chunk touches, walked back on its own
        Gw = {}
        for j in sorted({int(j) for u in toks for j in idx_w[u]} |
                        {int(j) for u in toks for j in idx_r[u]}):
            D, F = dM[j].copy(), M[j].copy()
            for t in reversed(toks):
                k = rpos[t].get(j)
                if k is not None:          # the read saw the row after t's write
                    g["d_wt_r"][t, k] = F @ dy[t]
                    D += wt_r[t, k] * dy[t]
                k = pos[t].get(j)
                if k is not None:
                    Gw[t, k] = D.copy()
                    F = log[t, k]
                    if gdn:
                        D = alpha[t] * (D - wt_w[t, k] * de[t])
                    else:
                        D = alpha[t] * (1.0 - beta[t] * wt_w[t, k]) * D
            dM[j], M[j] = D, F
        for u in toks:                     # per-token gradients from the G of each write
            m = log[u]
            Gu = np.array([Gw[u, k] for k in range(idx_w.shape[1])])
            if gdn:
                k = wt_w[u]
                e = v[u] - alpha[u] * (k @ m)
                g["d_v"][u] = de[u]
                g["d_wt_w"][u] = beta[u] * (Gu @ e) - alpha[u] * (m @ de[u])
                g["d_beta"][u] = k @ (Gu @ e)
                g["d_alpha"][u] = np.sum((Gu - np.outer(k, de[u])) * m)
            else:
                c = beta[u] * wt_w[u]
                g["d_v"][u] = c @ Gu
                dc = np.sum(Gu * (v[u][None, :] - alpha[u] * m), axis=1)
                g["d_alpha"][u] = np.sum((1.0 - c)[:, None] * Gu * m)
                g["d_beta"][u] = wt_w[u] @ dc
                g["d_wt_w"][u] = beta[u] * dc
    return g, M, dM


# ----------------------------------------------------------------------------
# Backward of the selection pass (steps 1-2 and the gate of step 4), reverse mode
# by the chain rule, down to the gradient of the projection output Y = x W_proj^T.
# The selected slot sets are piecewise constant in the scores, so the gradient
# reaches the half-scores only through the softmax weights of the selected slots
# ([rainbus] step 1; [analysis] "步骤 2": k^(i) and q^(i) are softmax-normalised
# scores of the selected slots).  For weights w = softmax(s) over the selected
# scores s_k = h1[i_k] + h2[j_k] (slot id i_k n + j_k):
#   ds_k = w_k (dw_k - sum_l w_l dw_l),   dh1[i] += sum_{k: i_k = i} ds_k,
#   dh2[j] += sum_{k: j_k = j} ds_k.
# Gates ([rainbus] step 2): alpha = exp(-A softplus(z)), z = a + b_dt:
#   dalpha/dz = -A alpha sigma(z),  dalpha/dA = -softplus(z) alpha,  dz/db_dt = 1;
#   beta = sigma(b): dbeta/db = beta (1 - beta).
# Output gate (step 4): sigmoid g = sigma(p): dg/dp = g (1 - g); SiLU g = p sigma(p):
#   dg/dp = sigma(p) (1 + p (1 - sigma(p))); none: 1.
# The value columns pass their gradient through.  Then dx = dY W_proj and
# dW_proj = dY^T x (the projection is linear).
# ----------------------------------------------------------------------------
def softmax_backward(w, dw):
    """Gradient of the scores of w = softmax(s) given dL/dw."""
    w = np.asarray(w, F64)
    dw = np.asarray(dw, F64)
    return w * (dw - np.sum(w * dw, axis=-1, keepdims=True))


def pass_a_backward(a, grads, A, b_dt, H, n, d_v, gate_act=GATE_SIGMOID, x=None, w_proj=None):
    """Gradients of pass_a's products back to the projection output.

    a: pass_a's result for tokens [..]; grads: dL/d of its products, [.., H, *]:
    d_wt_w, d_wt_r, d_v, d_g (of the activated gate), d_alpha, d_beta.
    Returns dY [.., H*P] (the gradient of Y = x W_proj^T, per head in the column
    order of split_heads), dA [H], db_dt [H], and, when x and w_proj are given,
    dx [.., d] and dW_proj [H*P, d].
    """
    A = np.asarray(A, F64)
    b_dt = np.asarray(b_dt, F64)
    lead = np.shape(a["alpha"])[:-1]                    # [..]
    P = 4 * n + 2 * d_v + 2
    dY = np.zeros(lead + (H, P))
    blocks = {"w": (0, n), "r": (2 * n, 3 * n)}          # offsets of the two halves
    for role, (o1, o2) in blocks.items():
        ids = np.asarray(a[f"idx_{role}"])
        ds = softmax_backward(a[f"wt_{role}"], grads[f"d_wt_{role}"])
        for idx in np.ndindex(*(lead + (H,))):
            for k in range(ids.shape[-1]):
                i, j = divmod(int(ids[idx][k]), n)
                dY[idx + (o1 + i,)] += ds[idx][k]
                dY[idx + (o2 + j,)] += ds[idx][k]
    o = 4 * n
    dY[..., o:o + d_v] = np.asarray(grads["d_v"], F64)
    p = np.asarray(a["g_pre"], F64)
    if gate_act == GATE_SIGMOID:
        g = sigmoid(p)
        dgp = g * (1.0 - g)
    elif gate_act == GATE_SILU:
        sg = sigmoid(p)
        dgp = sg * (1.0 + p * (1.0 - sg))
    else:
        dgp = np.ones_like(p)
    dY[..., o + d_v:o + 2 * d_v] = np.asarray(grads["d_g"], F64) * dgp
    z = np.asarray(a["a_pre"], F64) + b_dt
    alpha = forget_gate(a["a_pre"], A, b_dt)
    d_alpha = np.asarray(grads["d_alpha"], F64)
    dz = d_alpha * (-A * alpha * sigmoid(z))
    dY[..., o + 2 * d_v] = dz
    beta = input_gate(a["b_pre"])
    dY[..., o + 2 * d_v + 1] = np.asarray(grads["d_beta"], F64) * beta * (1.0 - beta)
    red = tuple(range(len(lead)))
    res = dict(dY=dY.reshape(lead + (H * P,)),
               dA=np.sum(d_alpha * (-softplus(z) * alpha), axis=red),
               db_dt=np.sum(dz, axis=red))
    if x is not None and w_proj is not None:
        dYf = res["dY"].reshape(-1, H * P)
        xf = np.asarray(x, F64).reshape(dYf.shape[0], -1)
        res["dx"] = (dYf @ np.asarray(w_proj, F64)).reshape(lead + (xf.shape[1],))
        res["dW_proj"] = dYf.T @ xf
    return res


# ----------------------------------------------------------------------------
# Quantised write log.  For long fine-tuning the pages store the state
# checkpoints of training in fp8 or int4 and report no harm to the loss ([163]
# section 八, memory-efficiency paragraph; [analysis] section "训练效率").  Here
# the checkpoint is the write log, quantised per logged row of d_v values with one
# absmax scale.  The code of each element is decided in fp32, as the kernels do:
#   fp8:  v = x * (448 / absmax) in fp32, then the nearest OCP E4M3 value (1 sign,
#         4 exponent bits with bias 7, 3 fraction bits; largest 448, subnormals
#         spaced 2^-9; ties to even), saturating at 448;
#   int4: v = x * (7 / absmax) in fp32, rounded to nearest even, in [-7, 7].
# Decoding: value(code) * (absmax / 448) or code * (absmax / 7), in fp32.
# ----------------------------------------------------------------------------
F32 = np.float32


def e4m3_encode(v):
    """fp32 values (|v| <= 448 up to rounding) -> E4M3 byte codes, ties to even,
    saturating at 448."""
    v = np.asarray(v, F32)
    a = np.abs(v).astype(np.float64)
    sign = np.signbit(v).astype(np.uint8) << 7
    code = np.zeros(v.shape, np.int64)
    sub = a < 2.0 ** -6
    code[sub] = np.rint(a[sub] * 512.0).astype(np.int64)       # 2^-9 steps; 8 -> 2^-6
    _, e = np.frexp(a[~sub])                                    # a = m 2^e, m in [0.5, 1)
    e = e - 1                                                   # a in [2^e, 2^(e+1))
    q = np.rint(np.ldexp(a[~sub], 3 - e)).astype(np.int64)      # in [8, 16]
    up = q == 16
    e = np.where(up, e + 1, e)
    q = np.where(up, 8, q)
    field = e + 7
    big = (field > 15) | ((field == 15) & (q - 8 == 7))         # above 448: saturate
    code[~sub] = np.where(big, (15 << 3) | 6, (field << 3) | (q - 8))
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def e4m3_decode(code):
    code = np.asarray(code, np.uint8).astype(np.int64)
    field, frac = (code >> 3) & 15, code & 7
    mag = np.where(field == 0, np.ldexp(frac.astype(np.float64), -9),
                   np.ldexp((8 + frac).astype(np.float64), field - 10))
    return np.where(code >> 7, -mag, mag)


def quantize_rows(rows, fmt: str):
    """rows [..., d] fp32 -> (codes, absmax [...] fp32); fmt "fp8" (one byte per
    element) or "int4" (signed codes -7..7, two per byte, low nibble first)."""
    x = np.asarray(rows, F32)
    amax = np.max(np.abs(x), axis=-1).astype(F32)
    top = F32(448.0) if fmt == "fp8" else F32(7.0)
    with np.errstate(divide="ignore"):
        inv = np.where(amax > 0, top / np.where(amax > 0, amax, F32(1)), F32(0)).astype(F32)
    v = (x * inv[..., None]).astype(F32)                        # fp32, as the kernels
    if fmt == "fp8":
        return e4m3_encode(v), amax
    q = np.clip(np.rint(v), -7, 7).astype(np.int64) & 15
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8), amax


def dequantize_rows(codes, amax, fmt: str):
    amax = np.asarray(amax, F32)
    if fmt == "fp8":
        unit = (amax / F32(448.0)).astype(F32)
        return (e4m3_decode(codes).astype(F32) * unit[..., None]).astype(F32)
    c = np.asarray(codes, np.uint8).astype(np.int64)
    lo, hi = c & 15, c >> 4
    q = np.stack([lo, hi], axis=-1).reshape(c.shape[:-1] + (2 * c.shape[-1],))
    q = np.where(q >= 8, q - 16, q).astype(F32)
    unit = (amax / F32(7.0)).astype(F32)
    return (q * unit[..., None]).astype(F32)


# ----------------------------------------------------------------------------
# Shared learned initial state ([analysis] section on the learned M0: M0 is a
# parameter of the layer, the same for every sequence; [163] section 三).  A
# sequence's memory starts as M0; a per-sequence store keeps only the rows that
# have been touched.  Effective state of slot i: store[i] if touched[i] else
# M0[i].  A call touches every slot it reads or writes.
# ----------------------------------------------------------------------------
def forward_walk_shared(m0_h, store_h, touched_h, sel, gamma_h, eps, rule="slot",
                        state="exact"):
    """forward_walk on the effective state of one walk.  Returns (out, y_raw,
    final effective state [N, d_v], touched after the call [N] bool)."""
    touched_h = np.asarray(touched_h, bool)
    m_init = np.where(touched_h[:, None], np.asarray(store_h, F64), np.asarray(m0_h, F64))
    out, y, M = forward_walk(m_init, sel, gamma_h, eps, rule, state)
    touched = touched_h.copy()
    touched[np.asarray(sel["idx_w"]).ravel()] = True
    touched[np.asarray(sel["idx_r"]).ravel()] = True
    return out, y, M, touched


def forward(x, w_proj, A, b_dt, gamma, state0, H, n, d_v, W, R, eps=1e-6,
            gate_act=GATE_SIGMOID):
    """Full path from x [B, T, d] and state0 [B, H, N, d_v].

    Returns (out [B, T, H, d_v], final state [B, H, N, d_v], pass-(a) dict).
    """
    x = np.asarray(x, F64)
    B, T = x.shape[:2]
    a = pass_a(x, w_proj, A, b_dt, H, n, d_v, W, R, gate_act)
    out = np.zeros((B, T, H, d_v), F64)
    st = np.zeros(np.shape(state0), F64)
    for b in range(B):
        for h in range(H):
            walk = {k: a[k][b, :, h] for k in ("idx_w", "wt_w", "idx_r", "wt_r", "v", "g",
                                               "alpha", "beta")}
            o, _, M = forward_walk(state0[b][h], walk, np.asarray(gamma, F64)[h], eps)
            out[b, :, h] = o
            st[b, h] = M
    return out, st, a
