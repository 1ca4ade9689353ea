"""Pins of the CPU oracle against facts that do not come from the oracle.

The pages print no worked example, so the oracle is pinned by: a hand-worked
two-token case and a sigmoid-table case (tests/golden), the matrix product
form of the recurrence, exact rational arithmetic, closed forms of special
cases (identity, plain delta rule, reset, retrieval, pure decay), and
invariants (chaining, slot skipping, permutation, head sharing, strided
views).  Each pin is chosen so that a plausible slip in the oracle (a dropped
term, a wrong sign, a transposed state, a stale state in the readout, a wrong
head map, sum instead of mean in the norm) fails at least one of them.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import kda_inputs as ki
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_fixture(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                key, *rest = line.split()
                vals[key] = [float(x) for x in rest]
    return vals


def _bf(x):
    return ki.to_bf16_bits(np.asarray(x, dtype=np.float64))


def _small(seed, N=3, H=2, HV=2, K=4, V=4, T=2, num_slots=6, **kw):
    return ki.make_problem("small", seed, N=N, H=H, HV=HV, K=K, V=V, num_slots=num_slots, T=T, **kw)


def _run(p, state64, **kw):
    extra = {}
    if p.gate is not None:
        extra = dict(gate=p.gate, norm_weight=p.norm_weight, eps=p.eps)
    if p.raw:
        extra.update(raw_gate=p.raw_gate, raw_beta=p.raw_beta, A_log=p.A_log, dt_bias=p.dt_bias)
    extra.update(kw)
    return oracle.decode_packed(p.q, p.k, p.v, p.g, p.beta, state64, p.slot_idx, p.cu_seqlens, p.scale, **extra)


def _f(bits):
    return ki.bf16_bits_to_f32(bits).astype(np.float64)


# ------------------------------------------------------------ hand-worked
def test_hand_worked_two_tokens_exact():
    fx = _read_fixture("hand_two_tokens.txt")
    K, V = int(fx["K"][0]), int(fx["V"][0])
    q = np.stack([_bf(fx["q0"]), _bf(fx["q1"])]).reshape(2, 1, K)
    k = np.stack([_bf(fx["k0"]), _bf(fx["k1"])]).reshape(2, 1, K)
    v = np.stack([_bf(fx["v0"]), _bf(fx["v1"])]).reshape(2, 1, V)
    g = np.array([fx["g0"], fx["g1"]], dtype=np.float32).reshape(2, 1, K)
    beta = np.array([fx["beta0"], fx["beta1"]], dtype=np.float32).reshape(2, 1)
    state = np.array(fx["S0"], dtype=np.float64).reshape(1, 1, K, V)
    out = oracle.decode_step(q, k, v, g, beta, state, np.array([0], np.int32), 2, fx["scale"][0])
    assert np.array_equal(out[0, 0], fx["o0"])
    assert np.array_equal(out[1, 0], fx["o1"])
    assert np.array_equal(state.reshape(-1), fx["S2"])


def test_gated_rmsnorm_sigmoid_table():
    fx = _read_fixture("gated_rmsnorm_sigmoid_table.txt")
    V = int(fx["V"][0])
    y = oracle.gated_rmsnorm(_bf(fx["x"]).reshape(1, V), _bf(fx["z"]).reshape(1, V), _bf(fx["w"]), fx["eps"][0])
    np.testing.assert_allclose(y[0], fx["y"], rtol=1e-15, atol=0)


# ------------------------------------------------------------ matrix form
def _matrix_form(p, state64):
    """(I - beta k k^T) diag(exp g) S + beta k v^T and o = scale S^T q, with
    numpy matrix products, for every live (request, head)."""
    S_all = state64.copy()
    out = np.full((p.tokens, p.HV, p.V), np.nan)
    rep = p.HV // p.H
    for n in range(p.N):
        s = int(p.slot_idx[n])
        if s < 0 or s >= p.num_slots:
            continue
        for hv in range(p.HV):
            h = hv // rep
            S = S_all[s, hv]
            for t in range(p.cu_seqlens[n], p.cu_seqlens[n + 1]):
                kk = _f(p.k[t, h])[:, None]
                qq = _f(p.q[t, h])[:, None]
                vv = _f(p.v[t, hv])[:, None]
                b = float(p.beta[t, hv])
                A = np.diag(np.exp(p.g[t, hv].astype(np.float64)))
                S = (np.eye(p.K) - b * kk @ kk.T) @ A @ S + b * kk @ vv.T
                out[t, hv] = p.scale * (S.T @ qq)[:, 0]
            S_all[s, hv] = S
    return out, S_all


@pytest.mark.parametrize("seed", range(6))
def test_matrix_form_brute_force_k4(seed):
    p = _small(100 + seed, N=3, H=2, HV=4, K=4, V=4, T=None, n_pad=1, num_slots=5)
    st = p.state_pool().astype(np.float64)
    ref_out, ref_state = _matrix_form(p, st)
    out = _run(p, st)
    live = np.isfinite(ref_out)
    assert np.array_equal(live, np.isfinite(out))
    np.testing.assert_allclose(out[live], ref_out[live], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(st, ref_state, rtol=1e-12, atol=1e-14)


def test_exact_rational_k3():
    """Exact rational evaluation of the product form (decay factors taken as
    the doubles exp(g) rounds to) against the oracle."""
    p = _small(7, N=1, H=1, HV=1, K=3, V=3, T=3, num_slots=1)
    st = p.state_pool().astype(np.float64)
    S = [[Fraction(float(st[0, 0, i, j])) for j in range(3)] for i in range(3)]
    outs = []
    for t in range(3):
        a = [Fraction(math.exp(float(x))) for x in p.g[t, 0]]
        kk = [Fraction(float(x)) for x in _f(p.k[t, 0])]
        qq = [Fraction(float(x)) for x in _f(p.q[t, 0])]
        vv = [Fraction(float(x)) for x in _f(p.v[t, 0])]
        b = Fraction(float(p.beta[t, 0]))
        D = [[a[i] * S[i][j] for j in range(3)] for i in range(3)]
        kD = [sum(kk[i] * D[i][j] for i in range(3)) for j in range(3)]     # k^T D
        S = [[D[i][j] - b * kk[i] * kD[j] + b * kk[i] * vv[j] for j in range(3)] for i in range(3)]
        outs.append([Fraction(p.scale) * sum(S[i][j] * qq[i] for i in range(3)) for j in range(3)])
    out = _run(p, st)
    for t in range(3):
        np.testing.assert_allclose(out[t, 0], [float(x) for x in outs[t]], rtol=1e-14, atol=1e-16)
    np.testing.assert_allclose(st[0, 0], [[float(x) for x in r] for r in S], rtol=1e-14, atol=1e-16)


# ------------------------------------------------------------ special cases
def test_identity_g0_beta0():
    p = ki.make_problem("id", 11, N=2, H=2, HV=2, K=128, V=128, num_slots=3, T=1)
    p.g[:] = 0.0
    p.beta[:] = 0.0
    st0 = p.state_pool().astype(np.float64)
    st = st0.copy()
    out = _run(p, st)
    assert np.array_equal(st, st0)                          # state unchanged
    for n in range(p.N):
        s = p.slot_idx[n]
        for hv in range(p.HV):
            ref = p.scale * (st0[s, hv].T @ _f(p.q[n, hv]))    # library GEMV
            np.testing.assert_allclose(out[n, hv], ref, rtol=1e-12, atol=1e-15)


def test_plain_delta_rule_g0():
    p = ki.make_problem("delta", 12, N=2, H=1, HV=2, K=128, V=128, num_slots=2, T=1)
    p.g[:] = 0.0
    st0 = p.state_pool().astype(np.float64)
    st = st0.copy()
    _run(p, st)
    for n in range(p.N):
        s = p.slot_idx[n]
        for hv in range(p.HV):
            kk = _f(p.k[n, 0])
            b = float(p.beta[n, hv])
            ref = (np.eye(128) - b * np.outer(kk, kk)) @ st0[s, hv] + b * np.outer(kk, _f(p.v[n, hv]))
            np.testing.assert_allclose(st[s, hv], ref, rtol=1e-10, atol=1e-13)


def test_reset_all_channels():
    p = ki.make_problem("reset", 13, N=1, H=1, HV=1, K=128, V=128, num_slots=1, T=1)
    p.g[:] = -np.inf
    st = p.state_pool().astype(np.float64)
    out = _run(p, st)
    kk, vv, qq = _f(p.k[0, 0]), _f(p.v[0, 0]), _f(p.q[0, 0])
    b = float(p.beta[0, 0])
    assert np.array_equal(st[0, 0], np.outer(kk, b * vv))       # S' = k (beta v)^T exactly
    np.testing.assert_allclose(out[0, 0], p.scale * b * float(kk @ qq) * vv, rtol=1e-12, atol=1e-15)


def test_reset_subset_of_channels():
    p = ki.make_problem("reset2", 14, N=1, H=1, HV=1, K=128, V=128, num_slots=1, T=1)
    R = np.arange(0, 128, 3)
    p.g[0, 0, R] = -np.inf
    st0 = p.state_pool().astype(np.float64)
    st = st0.copy()
    _run(p, st)
    a = np.exp(p.g[0, 0].astype(np.float64))
    kk, vv = _f(p.k[0, 0]), _f(p.v[0, 0])
    b = float(p.beta[0, 0])
    vp = b * (vv - (a[:, None] * st0[0, 0]).T @ kk)
    ref = a[:, None] * st0[0, 0] + np.outer(kk, vp)
    np.testing.assert_allclose(st[0, 0], ref, rtol=1e-11, atol=1e-14)
    # reset rows forget the old state: other old values there change nothing
    st_c = st0.copy()
    st_c[0, 0, R] = 7.0
    _run(p, st_c)
    assert np.array_equal(st_c, st)


def test_retrieval_unit_key():
    K = V = 128
    p = ki.make_problem("ret", 15, N=1, H=1, HV=1, K=K, V=V, num_slots=1, T=1)
    i = 37
    e = np.zeros(K)
    e[i] = 1.0
    p.k[0, 0] = _bf(e)
    p.q[0, 0] = _bf(e)
    p.beta[:] = 1.0
    p.g[:] = 0.0
    st0 = p.state_pool().astype(np.float64)
    st = st0.copy()
    out = _run(p, st)
    vv = _f(p.v[0, 0])
    np.testing.assert_allclose(st[0, 0, i], vv, rtol=4e-16, atol=1e-17)        # row i now holds v
    others = np.delete(np.arange(K), i)
    assert np.array_equal(st[0, 0, others], st0[0, 0, others])                  # other rows untouched
    np.testing.assert_allclose(out[0, 0], p.scale * vv, rtol=1e-15, atol=1e-17)


def test_pure_decay_beta0():
    p = ki.make_problem("decay", 16, N=1, H=1, HV=1, K=128, V=128, num_slots=1, T=1)
    p.beta[:] = 0.0
    st0 = p.state_pool().astype(np.float64)
    st = st0.copy()
    out = _run(p, st)
    ref = np.exp(p.g[0, 0].astype(np.float64))[:, None] * st0[0, 0]
    np.testing.assert_allclose(st[0, 0], ref, rtol=5e-16, atol=0)   # exp may differ by an ulp
    np.testing.assert_allclose(out[0, 0], p.scale * ref.T @ _f(p.q[0, 0]), rtol=1e-12, atol=1e-15)


# ------------------------------------------------------------ invariants
def test_chained_single_tokens_equal_one_multi_token_call():
    p = ki.make_problem("chain", 17, N=4, H=2, HV=4, K=16, V=8, num_slots=9, T=4)
    st_a = p.state_pool().astype(np.float64)
    st_b = st_a.copy()
    out_a = _run(p, st_a)
    out_b = np.full_like(out_a, np.nan)
    for t in range(4):
        rows = np.arange(p.N) * 4 + t
        o = oracle.decode_step(p.q[rows], p.k[rows], p.v[rows], p.g[rows], p.beta[rows],
                               st_b, p.slot_idx, 1, p.scale)
        out_b[rows] = o
    assert np.array_equal(out_a, out_b)
    assert np.array_equal(st_a, st_b)


def test_intermediate_states_are_the_chained_states():
    """The state after token t of a multi-token call is the final state of the
    chain of single-token calls that stops at t (pinned by the chaining pin)."""
    p = ki.make_problem("inter", 24, N=3, H=1, HV=2, K=8, V=8, num_slots=5, T=3, n_pad=1)
    st = p.state_pool().astype(np.float64)
    chain = st.copy()
    inter = np.full((p.tokens, p.HV, p.K, p.V), np.nan)
    _run(p, st.copy(), inter_state=inter)
    for t in range(3):
        rows = np.arange(p.N) * 3 + t
        oracle.decode_step(p.q[rows], p.k[rows], p.v[rows], p.g[rows], p.beta[rows], chain, p.slot_idx, 1, p.scale)
        for n in range(p.N):
            s_ = p.slot_idx[n]
            if s_ < 0:
                assert np.all(np.isnan(inter[n * 3 + t]))          # skipped: never written
            else:
                assert np.array_equal(inter[n * 3 + t], chain[s_])


def test_skipped_rows_and_untouched_slots():
    p = ki.make_problem("skip", 18, N=6, H=1, HV=2, K=8, V=8, num_slots=10, T=None, n_pad=2)
    p.slot_idx[np.nonzero(p.slot_idx >= 0)[0][0]] = 10          # out of range: skipped too
    st0 = p.state_pool().astype(np.float64)
    st = st0.copy()
    sentinel = np.full((p.tokens, p.HV, p.V), 12345.0)
    out = _run(p, st, out=sentinel)
    live = [n for n in range(p.N) if 0 <= p.slot_idx[n] < p.num_slots]
    dead = [n for n in range(p.N) if n not in live]
    assert len(dead) == 3
    for n in dead:
        assert np.all(out[p.cu_seqlens[n]:p.cu_seqlens[n + 1]] == 12345.0)
    for n in live:
        assert np.all(out[p.cu_seqlens[n]:p.cu_seqlens[n + 1]] != 12345.0)
    used = set(int(p.slot_idx[n]) for n in live)
    for s in range(p.num_slots):
        if s not in used:
            assert np.array_equal(st[s], st0[s])
        else:
            assert not np.array_equal(st[s], st0[s])


def test_request_permutation_invariance():
    p = ki.make_problem("perm", 19, N=5, H=2, HV=2, K=8, V=8, num_slots=7, T=None)
    st_a = p.state_pool().astype(np.float64)
    st_b = st_a.copy()
    out_a = _run(p, st_a)
    perm = np.array([3, 0, 4, 2, 1])
    rows = np.concatenate([np.arange(p.cu_seqlens[n], p.cu_seqlens[n + 1]) for n in perm])
    lens = np.diff(p.cu_seqlens)[perm]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    out_b = oracle.decode_packed(p.q[rows], p.k[rows], p.v[rows], p.g[rows], p.beta[rows],
                                 st_b, p.slot_idx[perm], cu, p.scale)
    assert np.array_equal(out_b, out_a[rows])
    assert np.array_equal(st_a, st_b)


def test_value_heads_share_qk_heads():
    """HV = 2H equals the same call with every q/k head duplicated (H' = HV)."""
    p = ki.make_problem("gqa", 20, N=3, H=2, HV=4, K=8, V=8, num_slots=4, T=2)
    st_a = p.state_pool().astype(np.float64)
    st_b = st_a.copy()
    out_a = _run(p, st_a)
    qd = np.ascontiguousarray(np.repeat(p.q, 2, axis=1))
    kd = np.ascontiguousarray(np.repeat(p.k, 2, axis=1))
    out_b = oracle.decode_packed(qd, kd, p.v, p.g, p.beta, st_b, p.slot_idx, p.cu_seqlens, p.scale)
    assert np.array_equal(out_a, out_b)
    assert np.array_equal(st_a, st_b)


def test_strided_views_of_a_fused_projection():
    p = ki.make_problem("fused", 21, N=3, H=2, HV=2, K=8, V=8, num_slots=4, T=2)
    T, HK, HVV = p.tokens, p.H * p.K, p.HV * p.V
    fused = np.zeros((T, 2 * HK + HVV + 8), dtype=np.uint16)
    fused[:, :HK] = p.q.reshape(T, HK)
    fused[:, HK:2 * HK] = p.k.reshape(T, HK)
    fused[:, 2 * HK:2 * HK + HVV] = p.v.reshape(T, HVV)
    qv = fused[:, :HK].reshape(T, p.H, p.K)
    kv = fused[:, HK:2 * HK].reshape(T, p.H, p.K)
    vv = fused[:, 2 * HK:2 * HK + HVV].reshape(T, p.HV, p.V)
    bw = np.zeros((T, 3), dtype=np.float32)
    bw[:, :2] = p.beta
    st_a = p.state_pool().astype(np.float64)
    st_b = st_a.copy()
    out_a = _run(p, st_a)
    out_b = oracle.decode_packed(qv, kv, vv, p.g, bw[:, :2], st_b, p.slot_idx, p.cu_seqlens, p.scale)
    assert np.array_equal(out_a, out_b)
    assert np.array_equal(st_a, st_b)


def test_zero_length_request_is_a_no_op():
    p = ki.make_problem("empty", 22, N=3, H=1, HV=1, K=8, V=8, num_slots=3, T=1)
    cu = np.array([0, 1, 1, 2], dtype=np.int32)        # request 1 has no tokens
    st0 = p.state_pool().astype(np.float64)
    st = st0.copy()
    oracle.decode_packed(p.q[:2], p.k[:2], p.v[:2], p.g[:2], p.beta[:2], st, p.slot_idx, cu, p.scale)
    assert np.array_equal(st[p.slot_idx[1]], st0[p.slot_idx[1]])


# ------------------------------------------------------------ gated RMSNorm
def test_norm_constant_row_closed_form():
    V = 16
    for c, eps in ((0.25, 1e-2), (3.0, 1e-6), (1e-3, 1e-6)):
        x = _bf(np.full(V, c))
        cval = _f(x)[0]
        z = _bf(np.full(V, 2.0))
        w = _bf(np.linspace(0.5, 2.0, V))
        y = oracle.gated_rmsnorm(x.reshape(1, V), z.reshape(1, V), w, eps)
        sig2 = 0.8807970779778823                      # sigmoid(2), textbook value
        ref = cval / math.sqrt(cval * cval + eps) * _f(w) * (2.0 * sig2)
        np.testing.assert_allclose(y[0], ref, rtol=1e-14)


def test_norm_scale_invariance_and_gate_symmetry():
    V = 128
    x = _bf(ki.normal(5, 1, V))
    z = _bf(ki.normal(5, 2, V))
    w = _bf(1.0 + 0.02 * ki.normal(5, 3, V))
    y1 = oracle.gated_rmsnorm(x.reshape(1, V), z.reshape(1, V), w, 0.0)
    x2 = _bf(2.0 * _f(x))                              # exact doubling in bf16
    y2 = oracle.gated_rmsnorm(x2.reshape(1, V), z.reshape(1, V), w, 0.0)
    np.testing.assert_allclose(y1, y2, rtol=1e-14)
    # silu(z) - silu(-z) = z
    zn = _bf(-_f(z))
    yn = oracle.gated_rmsnorm(x.reshape(1, V), zn.reshape(1, V), w, 0.0)
    xv = _f(x)
    r = 1.0 / math.sqrt(np.mean(xv * xv))
    np.testing.assert_allclose(y1[0] - yn[0], xv * r * _f(w) * _f(z), rtol=1e-12, atol=1e-14)


def test_norm_epilogue_wiring_in_decode():
    """silu(z) - silu(-z) = z, so decoding once with gate z and once with -z
    gives y(z) - y(-z) = z * w * o / sqrt(mean(o^2) + eps) with o the
    un-normed output: this pins which gate row and weight each output reads
    and that the norm sees the decoded o of its own (token, head)."""
    p = ki.make_problem("normwire", 23, N=3, H=2, HV=4, K=16, V=16, num_slots=5, T=2, norm=True)
    st0 = p.state_pool().astype(np.float64)
    st_a, st_b, st_c = st0.copy(), st0.copy(), st0.copy()
    y_pos = _run(p, st_a)
    neg = _bf(-_f(p.gate))
    y_neg = _run(p, st_b, gate=neg)
    o = oracle.decode_packed(p.q, p.k, p.v, p.g, p.beta, st_c, p.slot_idx, p.cu_seqlens, p.scale)
    assert np.array_equal(st_a, st_c) and np.array_equal(st_b, st_c)   # the norm never touches the state
    ms = np.mean(o * o, axis=-1, keepdims=True)
    ref = _f(p.gate) * _f(p.norm_weight) * o / np.sqrt(ms + p.eps)
    np.testing.assert_allclose(y_pos - y_neg, ref, rtol=1e-10, atol=1e-13)


def test_bf16_widening_is_exact():
    """k = e_0, g = 0, beta = 1 on a zero state writes v into row 0 unchanged,
    so row 0 shows how the bf16 bit patterns of v were widened."""
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x4049], dtype=np.uint16)
    q = np.zeros((1, 1, 5), np.uint16)
    k = np.zeros((1, 1, 5), np.uint16)
    k[0, 0, 0] = 0x3F80
    v = bits.reshape(1, 1, 5)
    g = np.zeros((1, 1, 5), np.float32)
    beta = np.ones((1, 1), np.float32)
    st = np.zeros((1, 1, 5, 5))
    oracle.decode_step(q, k, v, g, beta, st, np.array([0], np.int32), 1, 1.0)
    assert list(st[0, 0, 0]) == [1.0, -2.0, 2.0 ** -133, (2.0 - 2.0 ** -7) * 2.0 ** 127, 3.140625]


# ------------------------------------------------------------ gate activation
# Raw-projection inputs (FlashInfer PR 4562, inline review of the binding:
# raw_gate, raw_beta, A_log, dt_bias).  The activation is not printed on the
# pages; the oracle takes the Kimi Delta Attention gate.  These pins fix it
# through facts that do not evaluate that formula: the logistic closed form
# of exp(-softplus(x)), the odd part of softplus, the shift by dt_bias, the
# scaling by exp(A_log), the logistic function's symmetry and saturation.
def _raw_inputs(seed, tokens=3, HV=3, K=16, bias=None):
    """raw gate values in +/- pairs (channel i and i + K/2), A_log exact in
    fp32, optional dt_bias."""
    half = ki.normal(seed, 31, tokens * HV * (K // 2)).reshape(tokens, HV, K // 2) * 3.0
    half[0, 0, :4] = [0.0, 40.0, -40.0, 0.5]
    raw_gate = _bf(np.concatenate([half, -half], axis=-1))
    raw_beta = _bf(ki.normal(seed, 32, tokens * HV).reshape(tokens, HV) * 3.0)
    A_log = np.array([0.0, 0.75, -1.25, 1.5, -0.5][:HV], dtype=np.float32)
    dt_bias = np.zeros((HV, K), np.float32) if bias is None else bias
    return raw_gate, raw_beta, A_log, dt_bias


def test_gate_activation_logistic_closed_form():
    """exp(-softplus(x)) = 1 / (1 + e^x), so with A = exp(A_log) the decay
    factor is (1 + e^x)^-A: head by head, token by token, channel by channel."""
    raw_gate, raw_beta, A_log, dt_bias = _raw_inputs(7)
    g, _ = oracle.gate_activation(raw_gate, raw_beta, A_log, dt_bias)
    x = _f(raw_gate)
    logistic = 1.0 / (1.0 + np.exp(x))
    A = np.array([1.0, math.exp(0.75), math.exp(-1.25)])
    np.testing.assert_allclose(np.exp(g), logistic ** A[None, :, None], rtol=1e-12, atol=0)
    assert np.all(g <= 0)
    # A_log = 0: softplus(0) = ln 2
    assert abs(g[0, 0, 0] + math.log(2.0)) <= 1e-16


def test_gate_activation_odd_part_and_scaling():
    """softplus(x) - softplus(-x) = x, so g(x) - g(-x) = -exp(A_log) x; and
    g scales with exp(A_log) head by head."""
    raw_gate, raw_beta, A_log, dt_bias = _raw_inputs(8)
    g, _ = oracle.gate_activation(raw_gate, raw_beta, A_log, dt_bias)
    x = _f(raw_gate)
    K2 = raw_gate.shape[-1] // 2
    A = np.exp(A_log.astype(np.float64))
    diff = g[..., :K2] - g[..., K2:]
    np.testing.assert_allclose(diff, -A[None, :, None] * x[..., :K2], rtol=1e-13, atol=1e-300)
    # same raw values on every head: the heads differ by the factor exp(A_log[hv]) alone
    same = np.repeat(raw_gate[:, :1], 3, axis=1)
    gs, _ = oracle.gate_activation(same, raw_beta, A_log, dt_bias)
    for hv, a in enumerate((0.0, 0.75, -1.25)):
        np.testing.assert_allclose(gs[:, hv], gs[:, 0] * math.exp(a), rtol=1e-15)


def test_gate_activation_bias_shift():
    """dt_bias[hv][i] is added to the raw value of channel i of head hv:
    raw r with bias b gives exactly the g of raw r + b with no bias (values
    chosen so that r, b and r + b are exact)."""
    tokens, HV, K = 2, 3, 16
    r = (np.arange(tokens * HV * K).reshape(tokens, HV, K) % 29 - 14) * 0.25
    b = ((np.arange(HV * K).reshape(HV, K) * 7) % 17 - 8) * 0.125
    raw_beta = _bf(np.zeros((tokens, HV)))
    A_log = np.array([0.0, 0.75, -1.25], np.float32)
    g_bias, _ = oracle.gate_activation(_bf(r), raw_beta, A_log, b.astype(np.float32))
    g_shift, _ = oracle.gate_activation(_bf(r + b[None]), raw_beta, A_log, np.zeros((HV, K), np.float32))
    assert np.array_equal(g_bias, g_shift)
    g_none, _ = oracle.gate_activation(_bf(r), raw_beta, A_log, np.zeros((HV, K), np.float32))
    assert not np.array_equal(g_bias, g_none)


def test_gate_activation_beta_logistic():
    """beta = sigmoid(raw_beta): 1/2 at 0, beta(r) + beta(-r) = 1,
    beta(r) = e^r / (1 + e^r), and the infinities saturate to 0 and 1."""
    raw_gate, raw_beta, A_log, dt_bias = _raw_inputs(9)
    raw_beta[0, :3] = _bf([0.0, -np.inf, np.inf])
    _, beta = oracle.gate_activation(raw_gate, raw_beta, A_log, dt_bias)
    r = _f(raw_beta)
    assert beta[0, 0] == 0.5 and beta[0, 1] == 0.0 and beta[0, 2] == 1.0
    fin = np.isfinite(r)
    np.testing.assert_allclose(beta[fin], np.exp(r[fin]) / (1.0 + np.exp(r[fin])), rtol=1e-15)
    neg = raw_beta ^ np.uint16(0x8000)
    _, beta_neg = oracle.gate_activation(raw_gate, neg, A_log, dt_bias)
    np.testing.assert_allclose(beta + beta_neg, 1.0, rtol=0, atol=2e-16)


def test_gate_activation_saturates_at_infinity():
    """A raw gate of +inf clears the key channel (g = -inf, decay 0), -inf
    keeps it (g = 0, decay 1), for every A_log."""
    raw_gate, raw_beta, A_log, dt_bias = _raw_inputs(10)
    raw_gate[:, :, 0] = _bf(np.inf)
    raw_gate[:, :, 1] = _bf(-np.inf)
    g, _ = oracle.gate_activation(raw_gate, raw_beta, A_log, dt_bias)
    assert np.all(g[:, :, 0] == -np.inf)
    assert np.all(g[:, :, 1] == 0.0)


def test_fused_gate_decode_equals_exact_activated_inputs():
    """Raw values whose activation is exact (raw gate +/-inf: g = -inf or 0;
    raw beta 0, +inf, -inf: beta = 1/2, 1, 0) give bit for bit the decode of
    the activated inputs, per token, head and channel."""
    p = _small(21, N=3, H=2, HV=4, K=8, V=4, T=3, num_slots=5)
    tokens = p.tokens
    pick = ki.draws(77, 1, np.arange(tokens * p.HV * p.K, dtype=np.uint64)).reshape(tokens, p.HV, p.K)
    clear = (pick % np.uint64(5)) == 0                   # about one channel in five cleared
    raw_gate = np.where(clear, _bf(np.inf), _bf(-np.inf)).astype(np.uint16)
    g = np.where(clear, -np.inf, 0.0).astype(np.float32)
    choice = ki.draws(77, 2, np.arange(tokens * p.HV, dtype=np.uint64)).reshape(tokens, p.HV) % np.uint64(3)
    raw_beta = _bf(np.choose(choice.astype(np.int64), [0.0, np.inf, -np.inf]))
    beta = np.choose(choice.astype(np.int64), [0.5, 1.0, 0.0]).astype(np.float32)
    A_log = (0.5 * ki.normal(77, 3, p.HV)).astype(np.float32)
    dt_bias = (0.5 * ki.normal(77, 4, p.HV * p.K)).astype(np.float32).reshape(p.HV, p.K)
    s_raw = p.state_pool().astype(np.float64)
    s_act = s_raw.copy()
    out_raw = oracle.decode_packed(p.q, p.k, p.v, None, None, s_raw, p.slot_idx, p.cu_seqlens, p.scale,
                                   raw_gate=raw_gate, raw_beta=raw_beta, A_log=A_log, dt_bias=dt_bias)
    out_act = oracle.decode_packed(p.q, p.k, p.v, g, beta, s_act, p.slot_idx, p.cu_seqlens, p.scale)
    assert np.array_equal(out_raw, out_act, equal_nan=True)
    assert np.array_equal(s_raw, s_act)


def test_fused_gate_pure_decay_closed_form():
    """raw beta = -inf (beta = 0): T tokens only decay the state, each key row
    by prod_t (1 + e^(raw_t + bias))^(-exp(A_log))."""
    p = _small(22, N=2, H=1, HV=3, K=8, V=4, T=3, num_slots=4, raw_gates=True)
    raw_beta = np.full_like(p.raw_beta, _bf(-np.inf))
    s = p.state_pool().astype(np.float64)
    s0 = s.copy()
    oracle.decode_packed(p.q, p.k, p.v, None, None, s, p.slot_idx, p.cu_seqlens, p.scale,
                         raw_gate=p.raw_gate, raw_beta=raw_beta, A_log=p.A_log, dt_bias=p.dt_bias)
    A = np.exp(p.A_log.astype(np.float64))
    for n in range(p.N):
        slot = p.slot_idx[n]
        x = _f(p.raw_gate[p.cu_seqlens[n]:p.cu_seqlens[n + 1]]) + p.dt_bias.astype(np.float64)[None]
        factor = np.prod((1.0 + np.exp(x)) ** -A[None, :, None], axis=0)     # [HV, K]
        np.testing.assert_allclose(s[slot], s0[slot] * factor[:, :, None], rtol=1e-13, atol=0)


def test_fused_gate_with_zero_parameters_is_the_activated_recipe():
    """A_log = 0 and dt_bias = 0 give g = -softplus(x), beta = sigmoid(x):
    the activated workloads' recipe, drawn from the same raw values, agrees to
    the float32 rounding of its g and beta."""
    raw = _small(23, N=2, H=2, HV=2, K=8, V=4, T=2, num_slots=4, raw_gates=True, a_log_std=0.0, dt_bias_std=0.0)
    act = _small(23, N=2, H=2, HV=2, K=8, V=4, T=2, num_slots=4)
    g, beta = oracle.gate_activation(raw.raw_gate, raw.raw_beta, raw.A_log, raw.dt_bias)
    # the activated recipe evaluates the same draws before the bf16 rounding of
    # the raw values: |d softplus / dx| <= 1 and a bf16 rounding moves x by at
    # most 2^-9 |x|
    x, xb = _f(raw.raw_gate), _f(raw.raw_beta)
    assert np.all(np.abs(g - act.g) <= 2.0 ** -8 * np.abs(x) + 1e-6)
    assert np.all(np.abs(beta - act.beta) <= 2.0 ** -10 * np.abs(xb) + 1e-6)
