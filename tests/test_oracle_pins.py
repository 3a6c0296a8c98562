"""Pins of the fp64 oracle against results the method and the mathematics fix.

None of these re-types the oracle's recurrence. Each checks it against a
different statement of the same layer:

* the semiseparable (quadratic) form y = M x with
  M_ij = C_i^T abar_{i:j} B_j for i >= j (youngju.dev "Mamba / selective SSM",
  section "State Space Dualityの発見", the M_ij equation), evaluated by brute
  force on tiny inputs with every decay product summed out explicitly;
* causal linear attention when A = 0 (Qiita "Mamba-2" article, section 3.3:
  SSM and linear attention share the same semiseparable matrix);
* closed forms for T = 1 and for a constant step size (the decay matrix
  gamma^(i-j) of RetNet's retention, waylandz LLM book ch. 32, section 32.6.2);
* dt = 0 tokens leave the state untouched (youngju.dev page, "デバッグチェックリスト":
  padding tokens get dt forced to zero to block the state update);
* a very large step resets the state (youngju.dev page, selection section:
  large dt drives exp(dt A) to 0);
* carrying the final state into the next call equals one long call
  (youngju.dev page, "状態初期化とシーケンス境界");
* the recurrent (decode) mode chained over T steps equals the forward
  (Qiita article, section 3.3: parallel for training, recurrent for inference).
"""
import math

import numpy as np
import pytest

import oracle

RTOL = 1e-12


def _close(got, ref, rtol=RTOL):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = max(1.0, float(np.max(np.abs(ref))))
    err = float(np.max(np.abs(got - ref))) / scale
    assert err <= rtol, f"max err {err:.3e} > {rtol:.1e}"


def _rand_problem(rng, b, T, H, P, N, G, A_scale=1.0, with_init=True, with_D=True):
    x = rng.standard_normal((b, T, H, P)).astype(np.float32)
    dt = rng.uniform(0.01, 0.5, size=(b, T, H)).astype(np.float32)
    A = (-rng.uniform(0.2, 3.0, size=H) * A_scale).astype(np.float32)
    B = rng.standard_normal((b, T, G, N)).astype(np.float32)
    C = rng.standard_normal((b, T, G, N)).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32) if with_D else None
    init = rng.standard_normal((b, H, N, P)) if with_init else None
    return x, dt, A, B, C, D, init


def _quadratic_form(x, dt, A, B, C, D, init):
    """y = M x + (decayed initial state read-out) + D x, brute force.

    M[i, j] = (C_i . B_j) * exp(sum_{k=j+1..i} dt_k A) * dt_j   for i >= j.
    The initial state enters as if it were the state before token 0, so token
    i sees it decayed by exp(sum_{k=0..i} dt_k A).
    """
    x, dt, A, B, C = (np.asarray(v, np.float64) for v in (x, dt, A, B, C))
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    y = np.zeros((b, T, H, P))
    fin = np.zeros((b, H, N, P))
    for bb in range(b):
        for h in range(H):
            g = h // (H // G)
            a = dt[bb, :, h] * A[h]
            M = np.zeros((T, T))
            for i in range(T):
                for j in range(i + 1):
                    decay = math.exp(sum(a[k] for k in range(j + 1, i + 1)))
                    M[i, j] = float(C[bb, i, g] @ B[bb, j, g]) * decay * dt[bb, j, h]
            y[bb, :, h, :] = M @ x[bb, :, h, :]
            if init is not None:
                for i in range(T):
                    decay0 = math.exp(sum(a[k] for k in range(0, i + 1)))
                    y[bb, i, h, :] += decay0 * (C[bb, i, g] @ init[bb, h])
            if D is not None:
                y[bb, :, h, :] += float(D[h]) * x[bb, :, h, :]
            # final state: sum_j exp(sum_{k>j} a_k) dt_j B_j x_j^T + exp(sum_k a_k) init
            for j in range(T):
                decay = math.exp(sum(a[k] for k in range(j + 1, T)))
                fin[bb, h] += decay * dt[bb, j, h] * np.outer(B[bb, j, g], x[bb, j, h])
            if init is not None:
                fin[bb, h] += math.exp(sum(a)) * init[bb, h]
    return y, fin


@pytest.mark.parametrize("T,H,P,N,G", [(1, 2, 3, 2, 1), (5, 2, 4, 3, 2), (16, 2, 4, 4, 1),
                                       (16, 4, 3, 4, 2), (11, 2, 10, 3, 1)])
def test_quadratic_semiseparable_form(T, H, P, N, G):
    rng = np.random.default_rng(100 + T * 7 + G)
    args = _rand_problem(rng, 2, T, H, P, N, G)
    y, fin = oracle.ssd_fwd(*args)
    y_ref, fin_ref = _quadratic_form(*args)
    _close(y, y_ref)
    _close(fin, fin_ref)


def test_quadratic_form_no_init_no_D():
    rng = np.random.default_rng(7)
    args = _rand_problem(rng, 1, 9, 2, 4, 3, 1, with_init=False, with_D=False)
    y, fin = oracle.ssd_fwd(*args)
    y_ref, fin_ref = _quadratic_form(*args)
    _close(y, y_ref)
    _close(fin, fin_ref)


def test_group_mapping_is_contiguous_blocks():
    """Heads h use group h // (H/G): with G = 2, H = 4, swapping the two groups'
    B/C must swap the outputs of heads {0,1} and {2,3} computed with swapped A, D."""
    rng = np.random.default_rng(11)
    x, dt, A, B, C, D, init = _rand_problem(rng, 1, 12, 4, 3, 5, 2)
    y, _ = oracle.ssd_fwd(x, dt, A, B, C, D, init)
    perm = np.array([2, 3, 0, 1])
    y2, _ = oracle.ssd_fwd(x[:, :, perm], dt[:, :, perm], A[perm], B[:, :, ::-1], C[:, :, ::-1],
                           D[perm], init[:, perm])
    np.testing.assert_array_equal(y2, y[:, :, perm])


def test_A_zero_is_causal_linear_attention():
    """A = 0: the state is a running sum, y_i = C_i^T (h0 + sum_{j<=i} dt_j B_j x_j^T) + D x_i,
    i.e. softmax-free causal attention with Q=C, K=B, V=dt*x."""
    rng = np.random.default_rng(3)
    b, T, H, P, N, G = 2, 40, 3, 5, 6, 1
    x, dt, A, B, C, D, init = _rand_problem(rng, b, T, H, P, N, G)
    A = np.zeros_like(A)
    y, fin = oracle.ssd_fwd(x, dt, A, B, C, D, init)
    x64, dt64, B64, C64 = (v.astype(np.float64) for v in (x, dt, B, C))
    for h in range(H):
        kv = np.einsum("btn,btp->btnp", B64[:, :, 0], dt64[:, :, h, None] * x64[:, :, h])
        S = np.cumsum(kv, axis=1) + init[:, None, h]
        y_ref = np.einsum("btn,btnp->btp", C64[:, :, 0], S) + D[h] * x64[:, :, h]
        _close(y[:, :, h], y_ref)
        _close(fin[:, h], S[:, -1])
    # the attention form itself: scores (C_i . B_j) dt_j on the lower triangle
    scores = np.einsum("in,jn->ij", C64[0, :, 0], B64[0, :, 0]) * np.tril(np.ones((T, T)))
    y_att = (scores * dt64[0, None, :, 1]) @ x64[0, :, 1] + C64[0, :, 0] @ init[0, 1] + D[1] * x64[0, :, 1]
    _close(y[0, :, 1], y_att)


def test_single_token_closed_form():
    rng = np.random.default_rng(5)
    b, H, P, N, G = 3, 4, 6, 5, 2
    x, dt, A, B, C, D, init = _rand_problem(rng, b, 1, H, P, N, G)
    y, fin = oracle.ssd_fwd(x, dt, A, B, C, D, init)
    for bb in range(b):
        for h in range(H):
            g = h // (H // G)
            d = float(dt[bb, 0, h])
            h1 = math.exp(d * float(A[h])) * init[bb, h] + d * np.outer(B[bb, 0, g].astype(np.float64),
                                                                         x[bb, 0, h].astype(np.float64))
            _close(fin[bb, h], h1)
            _close(y[bb, 0, h], C[bb, 0, g].astype(np.float64) @ h1 + float(D[h]) * x[bb, 0, h].astype(np.float64))


def test_constant_step_geometric_closed_form():
    """dt = delta, B = b, C = c, x = u constant: h_t = r^(t+1) h0 + delta b u^T (1 - r^(t+1)) / (1 - r)."""
    T, H, P, N = 50, 2, 3, 4
    rng = np.random.default_rng(9)
    delta = np.float32(0.125)
    A = np.array([-0.5, -2.0], np.float32)
    bv = rng.standard_normal(N).astype(np.float32)
    cv = rng.standard_normal(N).astype(np.float32)
    u = rng.standard_normal((H, P)).astype(np.float32)
    x = np.broadcast_to(u, (1, T, H, P)).copy()
    dt = np.full((1, T, H), delta, np.float32)
    B = np.broadcast_to(bv, (1, T, 1, N)).copy()
    C = np.broadcast_to(cv, (1, T, 1, N)).copy()
    D = np.array([0.3, -1.1], np.float32)
    h0 = rng.standard_normal((1, H, N, P))
    y, fin = oracle.ssd_fwd(x, dt, A, B, C, D, h0)
    for h in range(H):
        r = math.exp(float(delta) * float(A[h]))
        drive = float(delta) * np.outer(bv.astype(np.float64), u[h].astype(np.float64))
        for t in range(T):
            ht = r ** (t + 1) * h0[0, h] + drive * (1 - r ** (t + 1)) / (1 - r)
            _close(y[0, t, h], cv.astype(np.float64) @ ht + float(D[h]) * u[h].astype(np.float64))
        _close(fin[0, h], r ** T * h0[0, h] + drive * (1 - r ** T) / (1 - r))


def test_constant_step_is_retention_decay_matrix():
    """dt = delta constant, B, C, x random: M_ij = delta * r^(i-j) * (C_i . B_j) (RetNet's gamma^(i-j))."""
    rng = np.random.default_rng(13)
    T, H, P, N = 24, 2, 4, 3
    x, _, A, B, C, _, _ = _rand_problem(rng, 1, T, H, P, N, 1, with_init=False, with_D=False)
    delta = np.float32(0.0625)
    dt = np.full((1, T, H), delta, np.float32)
    y, _ = oracle.ssd_fwd(x, dt, A, B, C)
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    for h in range(H):
        r = math.exp(float(delta) * float(A[h]))
        gamma = np.where(i >= j, r ** np.maximum(i - j, 0), 0.0)
        qk = C[0, :, 0].astype(np.float64) @ B[0, :, 0].astype(np.float64).T
        _close(y[0, :, h], (float(delta) * gamma * qk) @ x[0, :, h].astype(np.float64))


def test_zero_step_tokens_are_identity():
    """Inserting dt = 0 tokens changes nothing for the other tokens nor the final state;
    at an inserted token the read-out is C_t^T h_{t-1} + D x_t."""
    rng = np.random.default_rng(17)
    b, T, H, P, N, G = 2, 20, 2, 4, 5, 1
    x, dt, A, B, C, D, init = _rand_problem(rng, b, T, H, P, N, G)
    y, fin = oracle.ssd_fwd(x, dt, A, B, C, D, init)
    pad = [0, 7, 8, 20]        # insert before these original positions (20 = at the end)
    ins = np.array(sorted(pad))
    keep_idx = np.arange(T) + np.searchsorted(ins, np.arange(T), side="right")
    T2 = T + len(pad)
    mask = np.ones(T2, bool)
    mask[ins + np.arange(len(ins))] = False
    assert np.array_equal(np.nonzero(mask)[0], keep_idx)

    def spread(a):
        out = rng.standard_normal((a.shape[0], T2) + a.shape[2:]).astype(np.float32)
        out[:, mask] = a
        return out

    x2, B2, C2 = spread(x), spread(B), spread(C)
    dt2 = np.zeros((b, T2, H), np.float32)
    dt2[:, mask] = dt
    y2, fin2 = oracle.ssd_fwd(x2, dt2, A, B2, C2, D, init)
    np.testing.assert_array_equal(y2[:, mask], y)
    np.testing.assert_array_equal(fin2, fin)
    # read-out at the inserted token placed before original position 7
    t_pad = int(np.nonzero(~mask)[0][1])
    _, fin_prefix = oracle.ssd_fwd(x[:, :7], dt[:, :7], A, B[:, :7], C[:, :7], D, init)
    for h in range(H):
        ref = np.einsum("bn,bnp->bp", C2[:, t_pad, 0].astype(np.float64), fin_prefix[:, h]) \
            + float(D[h]) * x2[:, t_pad, h].astype(np.float64)
        _close(y2[:, t_pad, h], ref, 1e-13)


def test_large_step_resets_state():
    """exp(dt A) underflows to 0: h_t = dt_t B_t x_t^T and y_t = dt_t (C_t . B_t) x_t + D x_t."""
    rng = np.random.default_rng(19)
    b, T, H, P, N, G = 1, 12, 2, 3, 4, 1
    x, _, _, B, C, D, init = _rand_problem(rng, b, T, H, P, N, G)
    dt = np.full((b, T, H), 0.1, np.float32)
    A = np.full(H, -1e4, np.float32)
    y, fin = oracle.ssd_fwd(x, dt, A, B, C, D, init)
    x64, B64, C64 = (v.astype(np.float64) for v in (x, B, C))
    d = float(np.float32(0.1))
    for h in range(H):
        cb = np.einsum("btn,btn->bt", C64[:, :, 0], B64[:, :, 0])
        _close(y[:, :, h], d * cb[..., None] * x64[:, :, h] + float(D[h]) * x64[:, :, h])
        _close(fin[:, h], d * np.einsum("bn,bp->bnp", B64[:, -1, 0], x64[:, -1, h]))


def test_split_and_resume_equals_one_call():
    rng = np.random.default_rng(23)
    b, T, H, P, N, G = 2, 37, 2, 5, 3, 1
    x, dt, A, B, C, D, init = _rand_problem(rng, b, T, H, P, N, G)
    y, fin = oracle.ssd_fwd(x, dt, A, B, C, D, init)
    for T1 in (1, 16, 36):
        ya, fa = oracle.ssd_fwd(x[:, :T1], dt[:, :T1], A, B[:, :T1], C[:, :T1], D, init)
        yb, fb = oracle.ssd_fwd(x[:, T1:], dt[:, T1:], A, B[:, T1:], C[:, T1:], D, fa)
        np.testing.assert_array_equal(np.concatenate([ya, yb], axis=1), y)
        np.testing.assert_array_equal(fb, fin)


def test_decode_chain_equals_forward_and_columns():
    rng = np.random.default_rng(29)
    b, T, H, P, N, G = 3, 15, 4, 9, 5, 2
    x, dt, A, B, C, D, init = _rand_problem(rng, b, T, H, P, N, G)
    y, fin = oracle.ssd_fwd(x, dt, A, B, C, D, init)
    # recurrent mode: step axis first
    ys, st = oracle.ssd_decode(init, x.transpose(1, 0, 2, 3), dt.transpose(1, 0, 2), A,
                               B.transpose(1, 0, 2, 3), C.transpose(1, 0, 2, 3), D)
    np.testing.assert_array_equal(ys.transpose(1, 0, 2, 3), y)
    np.testing.assert_array_equal(st, fin)
    # one step at a time through the single-step entry
    state = init
    for t in range(T):
        yt, state = oracle.ssd_state_update(state, x[:, t], dt[:, t], A, B[:, t], C[:, t], D)
        np.testing.assert_array_equal(yt, y[:, t])
    np.testing.assert_array_equal(state, fin)
    # selected heads
    heads = [(0, 3), (2, 1)]
    ysel, ssel = oracle.ssd_decode(init, x.transpose(1, 0, 2, 3), dt.transpose(1, 0, 2), A,
                                   B.transpose(1, 0, 2, 3), C.transpose(1, 0, 2, 3), D, heads=heads)
    for k, (bb, h) in enumerate(heads):
        np.testing.assert_array_equal(ysel[k], y[bb, :, h])
        np.testing.assert_array_equal(ssel[k], fin[bb, h])
    # selected columns of the forward
    cols = [(0, 0, 0), (1, 3, 8), (2, 2, 4)]
    yc, fc = oracle.ssd_fwd_columns(x, dt, A, B, C, D, init, cols)
    for k, (bb, h, p) in enumerate(cols):
        np.testing.assert_array_equal(yc[k], y[bb, :, h, p])
        np.testing.assert_array_equal(fc[k], fin[bb, h, :, p])


def test_threads_do_not_change_results():
    rng = np.random.default_rng(31)
    args = _rand_problem(rng, 2, 30, 3, 17, 6, 1)
    y1, f1 = oracle.ssd_fwd(*args, nthreads=1)
    y4, f4 = oracle.ssd_fwd(*args, nthreads=4)
    np.testing.assert_array_equal(y1, y4)
    np.testing.assert_array_equal(f1, f4)


def test_rejects_bad_shapes():
    rng = np.random.default_rng(37)
    x, dt, A, B, C, D, init = _rand_problem(rng, 1, 4, 3, 2, 2, 1)
    B2 = np.concatenate([B, B], axis=2)
    with pytest.raises(RuntimeError):
        oracle.ssd_fwd(x, dt, A, B2, B2, D, init)   # H=3 not divisible by G=2


# ------------------------------------------------------------ packed variable-length sequences

def _quadratic_form_varlen(x, dt, A, B, C, D, cu, init):
    """Brute force over one token axis with sequence boundaries cu: the
    semiseparable M restricted to pairs of tokens in the same sequence, each
    sequence's initial state entering before its first token."""
    x, dt, A, B, C = (np.asarray(v, np.float64) for v in (x, dt, A, B, C))
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    seq = np.zeros(T, dtype=int)
    for i in range(len(cu) - 1):
        seq[cu[i]:cu[i + 1]] = i
    y = np.zeros((T, H, P))
    fin = np.zeros((len(cu) - 1, H, N, P))
    for h in range(H):
        g = h // (H // G)
        a = dt[:, h] * A[h]
        for i in range(T):
            s0 = cu[seq[i]]
            for j in range(s0, i + 1):
                decay = math.exp(sum(a[k] for k in range(j + 1, i + 1)))
                y[i, h] += float(C[i, g] @ B[j, g]) * decay * dt[j, h] * x[j, h]
            if init is not None:
                y[i, h] += math.exp(sum(a[k] for k in range(s0, i + 1))) * (C[i, g] @ init[seq[i], h])
            if D is not None:
                y[i, h] += float(D[h]) * x[i, h]
        for q in range(len(cu) - 1):
            for j in range(cu[q], cu[q + 1]):
                decay = math.exp(sum(a[k] for k in range(j + 1, cu[q + 1])))
                fin[q, h] += decay * dt[j, h] * np.outer(B[j, g], x[j, h])
            if init is not None:
                fin[q, h] += math.exp(sum(a[k] for k in range(cu[q], cu[q + 1]))) * init[q, h]
    return y, fin


@pytest.mark.parametrize("cu", [[0, 9], [0, 3, 9], [0, 1, 5, 5, 12], [0, 0, 4, 11, 12]])
def test_varlen_quadratic_form(cu):
    rng = np.random.default_rng(400 + sum(cu))
    T, H, P, N, G = cu[-1], 2, 3, 4, 1
    x, dt, A, B, C, D, _ = (v[0] if isinstance(v, np.ndarray) and v.ndim > 1 else v
                            for v in _rand_problem(rng, 1, T, H, P, N, G))
    init = rng.standard_normal((len(cu) - 1, H, N, P))
    y, fin = oracle.ssd_fwd_varlen(x, dt, A, B, C, D, cu, init)
    y_ref, fin_ref = _quadratic_form_varlen(x, dt, A, B, C, D, cu, init)
    _close(y, y_ref)
    _close(fin, fin_ref)


def test_varlen_matches_independent_sequences_and_single_sequence():
    rng = np.random.default_rng(410)
    cu = [0, 7, 7, 20, 41]
    T, H, P, N, G = cu[-1], 4, 5, 3, 2
    x, dt, A, B, C, D, _ = _rand_problem(rng, 1, T, H, P, N, G)
    x, dt, B, C = x[0], dt[0], B[0], C[0]
    init = rng.standard_normal((len(cu) - 1, H, N, P))
    y, fin = oracle.ssd_fwd_varlen(x, dt, A, B, C, D, cu, init)
    for i in range(len(cu) - 1):
        s, e = cu[i], cu[i + 1]
        if e > s:   # each sequence run alone from its own initial state
            yi, fi = oracle.ssd_fwd(x[None, s:e], dt[None, s:e], A, B[None, s:e], C[None, s:e], D,
                                    init[i:i + 1])
            np.testing.assert_array_equal(y[s:e], yi[0])
            np.testing.assert_array_equal(fin[i], fi[0])
        else:       # an empty sequence keeps its initial state
            np.testing.assert_array_equal(fin[i], init[i])
    # what precedes a sequence does not matter: change everything before sequence 3
    x2, dt2 = x.copy(), dt.copy()
    x2[:20] = rng.standard_normal((20, H, P)).astype(np.float32)
    dt2[:20] *= np.float32(0.5)
    y2, fin2 = oracle.ssd_fwd_varlen(x2, dt2, A, B, C, D, cu, init)
    np.testing.assert_array_equal(y2[20:], y[20:])
    np.testing.assert_array_equal(fin2[3], fin[3])
    # one sequence is the plain forward
    y1, f1 = oracle.ssd_fwd_varlen(x, dt, A, B, C, D, [0, T], init[:1])
    yr, fr = oracle.ssd_fwd(x[None], dt[None], A, B[None], C[None], D, init[:1])
    np.testing.assert_array_equal(y1, yr[0])
    np.testing.assert_array_equal(f1, fr)


def test_varlen_rejects_bad_offsets():
    rng = np.random.default_rng(420)
    x, dt, A, B, C, D, _ = _rand_problem(rng, 1, 6, 2, 2, 2, 1)
    for cu in ([0, 3], [1, 6], [0, 4, 3, 6]):
        with pytest.raises(ValueError):
            oracle.ssd_fwd_varlen(x[0], dt[0], A, B[0], C[0], D, cu)
