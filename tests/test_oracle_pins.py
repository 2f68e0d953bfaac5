"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every check here runs on the CPU.  Each one is chosen so that a plausible
mistake in the oracle (a dropped term, a wrong sign, a swapped index or
transposed operand) fails at least one of them:

* the 4-token decay table of weigao.cc ("递推公式如何展开成块内计算");
* the flat chunk table of weigao.cc ("chunked prefill 有两层含义");
* the checkpoint-count example of gitcode ("中间状态检查点");
* exact rational arithmetic at L = 8, D = 8 (0539edu section 3.1's first run)
  against the fp64 token form, the chunked form and the page-3 partial
  transitions (0539edu section 3.2);
* closed forms: beta = 0 (pure decay of the initial state), alpha = beta = 1
  with unit keys (S_t^T k_t = v_t), orthogonal keys with alpha = 1 (linear
  attention, 0539edu section 1.1);
* invariants: chunk-size independence, varlen = separate runs, GVA = head
  expansion, dv-column independence, linearity, checkpoints = prefix runs,
  split-run continuation, state orientation [V, K].
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle
from tests.conftest import read_golden


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    d = np.linalg.norm((a - b).ravel())
    n = np.linalg.norm(b.ravel())
    return d / n if n > 0 else d


def rand_problem(seed, lengths, hq=2, hk=2, hv=2, D=8, l2=True, init=False,
                 alpha=(0.7, 1.0), scale=None):
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    H = max(hq, hv)
    q = rng.standard_normal((T, hq, D))
    k = rng.standard_normal((T, hk, D))
    v = rng.standard_normal((T, hv, D))
    g = rng.uniform(alpha[0], alpha[1], (T, H))
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, H))))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    S0 = rng.standard_normal((len(lengths), H, D, D)) * 0.3 if init else None
    return oracle.Problem(q=q, k=k, v=v, cu=cu, g=g, beta=beta, l2norm=l2,
                          init_state=S0, scale=scale)


# ---------------------------------------------------------------- page values

def test_decay_table_weigao():
    """Orthonormal keys k_t = e_t and a zero start reduce the recurrence to
    S_t = alpha_t S_{t-1} + u_t with u_t = beta_t e_t v_t^T, the page's scalar
    unrolling; row j of S_t must be table(t, j) * beta_j v_j."""
    rows = read_golden("weigao_decay_table.txt")
    D, L = 6, 4
    alpha = np.array([0.9, 0.55, 0.8, 0.35])
    beta = np.array([0.7, 0.25, 0.6, 0.95])
    rng = np.random.default_rng(7)
    v = rng.standard_normal((L, 1, D))
    k = np.zeros((L, 1, D))
    for t in range(L):
        k[t, 0, t] = 1.0
    q = rng.standard_normal((L, 1, D))
    cu = np.array([0, L])
    p = oracle.Problem(q=q, k=k, v=v, cu=cu, g=alpha[:, None],
                       beta=beta[:, None], ckpt_every=1,
                       ckpt_cu_starts=np.array([0, L]))
    res = oracle.token(p)
    ck = res["ckpt"]  # [L, 1, D(v), D(k)] = S_t^T
    gate = {"g%d" % (i + 1): alpha[i] for i in range(L)}
    expect = np.zeros((L, L))
    s0_factor = None
    for st, up, fac in rows:
        val = 1.0
        if fac != "1":
            for name in fac.split("*"):
                val *= gate[name]
        if up == "S0":
            s0_factor = (int(st[1:]) - 1, val)
            continue
        expect[int(st[1:]) - 1, int(up[1:]) - 1] = val
    for t in range(L):
        S_t = ck[t, 0].T  # keys x values
        for j in range(L):
            want = expect[t, j] * beta[j] * v[j, 0]
            np.testing.assert_allclose(S_t[j], want, rtol=1e-14, atol=1e-15)
        for j in range(L, D):
            np.testing.assert_allclose(S_t[j], 0.0, atol=1e-15)
    # S0 coefficient: beta = 0 leaves g4 g3 g2 g1 S0
    t_idx, fac = s0_factor
    assert t_idx == 3
    S0 = rng.standard_normal((1, 1, D, D))
    p0 = oracle.Problem(q=q, k=rng.standard_normal((L, 1, D)), v=v, cu=cu,
                        g=alpha[:, None], beta=np.zeros((L, 1)),
                        init_state=S0)
    for form in (oracle.token(p0), oracle.chunked(p0, 4),
                 oracle.chunked(p0, 3)):
        np.testing.assert_allclose(form["final"][0, 0], fac * S0[0, 0],
                                   rtol=1e-14, atol=1e-15)
    # the chunked form reproduces the whole table too (chunk sizes 4, 3, 2)
    for C in (4, 3, 2):
        pc = oracle.Problem(q=q, k=k, v=v, cu=np.array([0, t_idx + 1]),
                            g=alpha[:, None], beta=beta[:, None])
        fin = oracle.chunked(pc, C)["final"][0, 0].T
        for j in range(L):
            np.testing.assert_allclose(fin[j], expect[3, j] * beta[j] * v[j, 0],
                                       rtol=1e-13, atol=1e-15)


def test_chunk_table_weigao():
    rows = read_golden("weigao_chunk_table.txt")
    lengths = [int(x) for x in rows[0][1:]]
    per = [int(x) for x in rows[1][1:]]
    flat = [tuple(int(x) for x in r[1:]) for r in rows if r[0] == "flat"]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    table, cu_chunks, n = oracle.chunk_table(cu, 64)
    assert n == sum(per)
    assert list(np.diff(cu_chunks)) == per
    for f, s, c in flat:
        assert tuple(table[f]) == (s, c)
    # the rest of the listing continues sequence-major, chunk-minor
    assert [tuple(x) for x in table] == [(i, c) for i in range(3)
                                         for c in range(per[i])]


def test_checkpoint_starts_gitcode():
    rows = dict((r[0], r[1:]) for r in read_golden("gitcode_checkpoints.txt"))
    every = int(rows["every"][0])
    lengths = [int(x) for x in rows["lengths"]]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    cs = oracle.checkpoint_starts(cu, every)
    assert int(cs[-1]) == int(rows["total"][0])
    assert list(cs) == [int(x) for x in rows["cu_starts"]]


def test_chunk_table_edge_cases():
    # empty sequences, exact multiples, single tokens
    cu = np.array([0, 0, 64, 64, 65, 193])
    table, cc, n = oracle.chunk_table(cu, 64)
    assert list(cc) == [0, 0, 1, 1, 2, 4]
    assert [tuple(x) for x in table] == [(1, 0), (3, 0), (4, 0), (4, 1)]
    _, cc, n = oracle.chunk_table(np.array([0, 0, 0]), 64)
    assert n == 0 and list(cc) == [0, 0, 0]


# ---------------------------------------------------------- exact arithmetic

def _rational_case(seed, L=8, D=8, with_s0=True):
    rng = np.random.default_rng(seed)

    def fr(lo, hi, den):
        return Fraction(int(rng.integers(lo, hi)), den)

    q = [[fr(-9, 10, 8) for _ in range(D)] for _ in range(L)]
    k = [[fr(-9, 10, 16) for _ in range(D)] for _ in range(L)]
    v = [[fr(-9, 10, 4) for _ in range(D)] for _ in range(L)]
    alpha = [fr(5, 17, 16) for _ in range(L)]
    beta = [fr(1, 9, 8) for _ in range(L)]
    S0 = [[fr(-5, 6, 8) for _ in range(D)] for _ in range(D)] if with_s0 else None
    return q, k, v, alpha, beta, S0


@pytest.mark.parametrize("with_s0", [False, True])
def test_exact_rational_L8_D8(with_s0):
    q, k, v, alpha, beta, S0 = _rational_case(11 + with_s0, with_s0=with_s0)
    scale = Fraction(3, 7)
    outs, states = oracle.exact_token(q, k, v, alpha, beta, scale, S0)
    L, D = len(q), len(q[0])
    exact_o = np.array([[float(x) for x in r] for r in outs])
    exact_S = np.array([[float(x) for x in r] for r in states[-1]])
    f = lambda m: np.array([[float(x) for x in r] for r in m])
    init = None if S0 is None else f(S0).T[None, None]
    p = oracle.Problem(q=f(q)[:, None], k=f(k)[:, None], v=f(v)[:, None],
                       cu=np.array([0, L]),
                       g=np.array([float(a) for a in alpha])[:, None],
                       beta=np.array([float(b) for b in beta])[:, None],
                       scale=float(scale), init_state=init)
    forms = [oracle.token(p)] + [oracle.chunked(p, C) for C in (1, 3, 8, 64)]
    for r in forms:
        assert rel(r["out"][:, 0], exact_o) < 1e-12
        assert rel(r["final"][0, 0].T, exact_S) < 1e-12
    y, S = oracle.partial_transition(
        f(q), f(k), f(v), [float(a) for a in alpha], [float(b) for b in beta],
        float(scale), 3, None if S0 is None else f(S0))
    assert rel(y, exact_o) < 1e-12
    assert rel(S, exact_S) < 1e-12


def test_pair_composition_matches_recurrence():
    """(M, N) pairs of adjacent ranges compose as M_R M_L, M_R N_L + N_R
    (0539edu section 2.1); folding all tokens gives the final state."""
    q, k, v, alpha, beta, S0 = _rational_case(5)
    f = lambda m: np.array([[float(x) for x in r] for r in m])
    K, V, S0f = f(k), f(v), f(S0)
    D = K.shape[1]
    pairs = []
    for i in range(len(K)):
        A = float(alpha[i]) * (np.eye(D) - float(beta[i]) * np.outer(K[i], K[i]))
        B = float(beta[i]) * np.outer(K[i], V[i])
        pairs.append((A, B))
    acc = pairs[0]
    for pr in pairs[1:]:
        acc = oracle.combine_pairs(acc, pr)
    # tree order gives the same
    left = oracle.combine_pairs(oracle.combine_pairs(pairs[0], pairs[1]),
                                oracle.combine_pairs(pairs[2], pairs[3]))
    right = oracle.combine_pairs(oracle.combine_pairs(pairs[4], pairs[5]),
                                 oracle.combine_pairs(pairs[6], pairs[7]))
    tree = oracle.combine_pairs(left, right)
    _, states = oracle.exact_token(q, k, v, alpha, beta, Fraction(1), S0)
    exact_S = f(states[-1])
    assert rel(acc[0] @ S0f + acc[1], exact_S) < 1e-12
    assert rel(tree[0] @ S0f + tree[1], exact_S) < 1e-12


# ----------------------------------------------------------------- closed forms

def test_beta_zero_pure_decay_and_orientation():
    """beta = 0: S_T = (prod alpha) S_0 and o_t = scale gamma_t S_0^T q_t.
    The stored state is [V, K], so o_t = scale gamma_t (st @ q_t) with st the
    stored matrix; a non-symmetric S_0 tells this from the transposed
    reading."""
    rng = np.random.default_rng(3)
    L, D = 37, 5
    st = rng.standard_normal((1, 1, D, D))
    assert not np.allclose(st[0, 0], st[0, 0].T)
    q = rng.standard_normal((L, 1, D))
    g = rng.uniform(0.6, 1.0, (L, 1))
    p = oracle.Problem(q=q, k=rng.standard_normal((L, 1, D)),
                       v=rng.standard_normal((L, 1, D)), cu=np.array([0, L]),
                       g=g, beta=np.zeros((L, 1)), init_state=st, scale=0.5)
    gamma = np.cumprod(g[:, 0])
    want_o = 0.5 * gamma[:, None] * (q[:, 0] @ st[0, 0].T)
    wrong_o = 0.5 * gamma[:, None] * (q[:, 0] @ st[0, 0])
    for r in (oracle.token(p), oracle.chunked(p, 16)):
        np.testing.assert_allclose(r["final"][0, 0], gamma[-1] * st[0, 0],
                                   rtol=1e-13)
        np.testing.assert_allclose(r["out"][:, 0], want_o, rtol=1e-12,
                                   atol=1e-14)
        assert rel(r["out"][:, 0], wrong_o) > 0.1


def test_unit_key_delta_rule_writes_value():
    """alpha = beta = 1 and |k_t| = 1: k_t^T S_t = v_t^T exactly.  Reading it
    through o_t with q_t = k_t and scale 1 gives o_t = v_t."""
    rng = np.random.default_rng(4)
    L, D = 90, 16
    k = rng.standard_normal((L, 1, D))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((L, 1, D))
    S0 = rng.standard_normal((1, 1, D, D))
    p = oracle.Problem(q=k.copy(), k=k, v=v, cu=np.array([0, L]),
                       g=np.ones((L, 1)), beta=np.ones((L, 1)), scale=1.0,
                       init_state=S0)
    for r in (oracle.token(p), oracle.chunked(p, 64), oracle.chunked(p, 7)):
        np.testing.assert_allclose(r["out"][:, 0], v[:, 0], atol=1e-11)


def test_orthogonal_keys_alpha_one_is_linear_attention():
    """Orthonormal keys, alpha = 1, zero start: the delta-rule erase term
    vanishes and o_t = scale sum_{j<=t} beta_j (q_t . k_j) v_j."""
    rng = np.random.default_rng(5)
    L, D = 12, 12
    Q, _ = np.linalg.qr(rng.standard_normal((D, D)))
    k = Q[:L][:, None, :]
    q = rng.standard_normal((L, 1, D))
    v = rng.standard_normal((L, 1, D))
    beta = rng.uniform(0.1, 1.0, (L, 1))
    p = oracle.Problem(q=q, k=k, v=v, cu=np.array([0, L]), g=np.ones((L, 1)),
                       beta=beta, scale=0.25)
    want = np.zeros((L, D))
    for t in range(L):
        for j in range(t + 1):
            want[t] += beta[j, 0] * (q[t, 0] @ k[j, 0]) * v[j, 0]
    want *= 0.25
    for r in (oracle.token(p), oracle.chunked(p, 5)):
        np.testing.assert_allclose(r["out"][:, 0], want, atol=1e-12)


def test_defaults_gate_and_scale():
    """g = beta = None means all ones; scale = None means 1/sqrt(D)."""
    p = rand_problem(8, [40], hq=1, hk=1, hv=1, D=9)
    p_def = oracle.Problem(q=p.q, k=p.k, v=p.v, cu=p.cu, l2norm=True)
    p_exp = oracle.Problem(q=p.q, k=p.k, v=p.v, cu=p.cu, l2norm=True,
                           g=np.ones((40, 1)), beta=np.ones((40, 1)),
                           scale=1 / 3.0)
    a, b = oracle.token(p_def), oracle.token(p_exp)
    np.testing.assert_array_equal(a["out"], b["out"])
    np.testing.assert_array_equal(a["final"], b["final"])


def test_l2norm_scale_invariance():
    """With in-kernel normalisation, rescaling q and k changes the result only
    through epsilon, and equals the run on unit vectors to ~1e-6."""
    p = rand_problem(9, [50], hq=1, hk=1, hv=1, D=16, l2=True)
    ref = oracle.token(p)
    p2 = oracle.Problem(q=p.q * 7.0, k=p.k * 0.5, v=p.v, cu=p.cu, g=p.g,
                        beta=p.beta, l2norm=True)
    r2 = oracle.token(p2)
    assert rel(r2["out"], ref["out"]) < 1e-5
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    p3 = oracle.Problem(q=unit(p.q), k=unit(p.k), v=p.v, cu=p.cu, g=p.g,
                        beta=p.beta, l2norm=False)
    assert rel(oracle.token(p3)["out"], ref["out"]) < 1e-5
    # and without normalisation the (divergent-scale) result differs
    p4 = oracle.Problem(q=p.q, k=p.k, v=p.v, cu=p.cu, g=p.g, beta=p.beta,
                        l2norm=False)
    assert rel(oracle.token(p4)["out"], ref["out"]) > 1e-2


# ------------------------------------------------------------------ invariants

@pytest.mark.parametrize("C", [1, 2, 3, 4, 8, 16, 64, 128])
def test_chunk_size_independence(C):
    p = rand_problem(21, [70, 0, 129, 1, 64], hq=2, hk=2, hv=4, D=8,
                     init=True)
    tok = oracle.token(p)
    ch = oracle.chunked(p, C)
    assert rel(ch["out"], tok["out"]) < 1e-12
    assert rel(ch["final"], tok["final"]) < 1e-12


def test_varlen_equals_separate_runs():
    lengths = [33, 0, 100, 5]
    p = rand_problem(22, lengths, init=True)
    full = oracle.token(p)
    cu = p.cu
    for i, L in enumerate(lengths):
        s, e = int(cu[i]), int(cu[i + 1])
        pi = oracle.Problem(q=p.q[s:e], k=p.k[s:e], v=p.v[s:e],
                            cu=np.array([0, L]), g=p.g[s:e], beta=p.beta[s:e],
                            l2norm=True, init_state=p.init_state[i:i + 1])
        r = oracle.token(pi)
        np.testing.assert_array_equal(r["out"], full["out"][s:e])
        np.testing.assert_array_equal(r["final"][0], full["final"][i])
    # an empty sequence's final state is its initial state
    np.testing.assert_array_equal(full["final"][1], p.init_state[1])


@pytest.mark.parametrize("hq,hk,hv", [(2, 2, 6), (6, 3, 3)])
def test_head_sharing_equals_expansion(hq, hk, hv):
    """GVA (hv > hq = hk) / GQA (hq > hk = hv): the same as expanding the
    shared heads block-wise (sab head h reads source head h / (H / h_src))."""
    p = rand_problem(23, [40, 27], hq=hq, hk=hk, hv=hv, D=6)
    H = max(hq, hv)
    ex = lambda x: np.repeat(x, H // x.shape[1], axis=1)
    pe = oracle.Problem(q=ex(p.q), k=ex(p.k), v=ex(p.v), cu=p.cu, g=p.g,
                        beta=p.beta, l2norm=True)
    a, b = oracle.token(p), oracle.token(pe)
    np.testing.assert_array_equal(a["out"], b["out"])
    np.testing.assert_array_equal(a["final"], b["final"])


def test_value_columns_independent_and_linear():
    p = rand_problem(24, [45, 20], hq=1, hk=1, hv=1, D=8, init=True)
    base = oracle.token(p)
    perm = np.random.default_rng(0).permutation(8)
    pp = oracle.Problem(q=p.q, k=p.k, v=p.v[..., perm], cu=p.cu, g=p.g,
                        beta=p.beta, l2norm=True,
                        init_state=p.init_state[:, :, perm, :])
    r = oracle.token(pp)
    np.testing.assert_allclose(r["out"], base["out"][..., perm], rtol=1e-13,
                               atol=1e-14)
    np.testing.assert_allclose(r["final"], base["final"][:, :, perm, :],
                               rtol=1e-13, atol=1e-14)
    # joint linearity in (V, S0)
    p2 = oracle.Problem(q=p.q, k=p.k, v=p.v * 2.5, cu=p.cu, g=p.g,
                        beta=p.beta, l2norm=True, init_state=p.init_state * 2.5)
    r2 = oracle.token(p2)
    np.testing.assert_allclose(r2["out"], 2.5 * base["out"], rtol=1e-12,
                               atol=1e-13)


def test_checkpoints_are_prefix_runs_and_continuation():
    lengths = [300, 64, 130]
    every = 64
    p = rand_problem(25, lengths, init=True)
    cs = oracle.checkpoint_starts(p.cu, every)
    p.ckpt_every, p.ckpt_cu_starts = every, cs
    full = oracle.token(p)
    ch = oracle.chunked(p, 64)
    assert rel(ch["ckpt"], full["ckpt"]) < 1e-12
    for i, L in enumerate(lengths):
        s = int(p.cu[i])
        for j in range(1, L // every + 1):
            e = s + j * every
            pi = oracle.Problem(q=p.q[s:e], k=p.k[s:e], v=p.v[s:e],
                                cu=np.array([0, e - s]), g=p.g[s:e],
                                beta=p.beta[s:e], l2norm=True,
                                init_state=p.init_state[i:i + 1])
            np.testing.assert_array_equal(
                oracle.token(pi)["final"][0], full["ckpt"][cs[i] + j - 1])
    # continuation: run(a + b) == run(b, init = run(a).final), any split
    s, e = int(p.cu[0]), int(p.cu[1])
    for cut in (1, 63, 64, 200):
        pa = oracle.Problem(q=p.q[s:s + cut], k=p.k[s:s + cut],
                            v=p.v[s:s + cut], cu=np.array([0, cut]),
                            g=p.g[s:s + cut], beta=p.beta[s:s + cut],
                            l2norm=True, init_state=p.init_state[0:1])
        ra = oracle.token(pa)
        pb = oracle.Problem(q=p.q[s + cut:e], k=p.k[s + cut:e],
                            v=p.v[s + cut:e], cu=np.array([0, e - s - cut]),
                            g=p.g[s + cut:e], beta=p.beta[s + cut:e],
                            l2norm=True, init_state=ra["final"])
        rb = oracle.chunked(pb, 64)
        assert rel(rb["final"][0], full["final"][0]) < 1e-12
        assert rel(np.concatenate([ra["out"], rb["out"]]),
                   full["out"][s:e]) < 1e-12


def test_pool_indices_read_and_write_rows():
    p = rand_problem(26, [20, 35, 9], init=False)
    rng = np.random.default_rng(1)
    pool = rng.standard_normal((10, 2, 8, 8))
    idx = np.array([7, 2, 5])
    pp = oracle.Problem(q=p.q, k=p.k, v=p.v, cu=p.cu, g=p.g, beta=p.beta,
                        l2norm=True, init_state=pool, state_indices=idx)
    ps = oracle.Problem(q=p.q, k=p.k, v=p.v, cu=p.cu, g=p.g, beta=p.beta,
                        l2norm=True, init_state=pool[idx])
    a, b = oracle.token(pp), oracle.token(ps)
    np.testing.assert_array_equal(a["out"], b["out"])
    np.testing.assert_array_equal(a["final"], b["final"])


def test_intermediates_chunk_states_and_new_values():
    """Chunk-start states equal the token recurrence's state at every 64th
    token; the new values are nu_t = beta_t (v_t - alpha_t S_{t-1}^T k_t)."""
    lengths = [150, 64, 10]
    p = rand_problem(27, lengths, D=8, init=True)
    ch = oracle.chunked(p, 64, dump=True)
    table, cc, n = oracle.chunk_table(p.cu, 64)
    # states at every token via 1-token checkpoints
    cs1 = oracle.checkpoint_starts(p.cu, 1)
    p1 = oracle.Problem(q=p.q, k=p.k, v=p.v, cu=p.cu, g=p.g, beta=p.beta,
                        l2norm=True, init_state=p.init_state, ckpt_every=1,
                        ckpt_cu_starts=cs1)
    tok = oracle.token(p1)
    H, D = p.H, p.D
    for f in range(n):
        i, c = table[f]
        if c == 0:
            want = p.init_state[i]
        else:
            want = tok["ckpt"][cs1[i] + 64 * c - 1]
        assert rel(ch["chunk_states"][f], want) < 1e-12
    # nu_t from the token states
    unit = lambda x: x / np.sqrt(np.sum(x * x, -1, keepdims=True) + 1e-6)
    K = unit(p.k)
    for i, L in enumerate(lengths):
        for tt in range(L):
            t = int(p.cu[i]) + tt
            for h in range(H):
                Sprev = (p.init_state[i, h] if tt == 0
                         else tok["ckpt"][cs1[i] + tt - 1, h]).T
                nu = p.beta[t, h] * (p.v[t, h] - p.g[t, h] * Sprev.T @ K[t, h])
                np.testing.assert_allclose(ch["vnew"][t, h], nu, rtol=1e-10,
                                           atol=1e-12)


def test_chunk_factors_reproduce_the_chunked_new_values():
    """oracle.chunk_factors (numpy, T = (I + A)^-1 by matrix inverse) against
    the C chunked form (a unit-lower-triangular solve): for every chunk and
    head, U - W S_chunkstart equals the dumped new values, and T (I + A) = I
    with T unit lower triangular."""
    lengths = [150, 64, 10, 129]
    p = rand_problem(31, lengths, D=8, init=True)
    ch = oracle.chunked(p, 64, dump=True)
    table, cc, n = oracle.chunk_table(p.cu, 64)
    for f in range(n):
        i, c = (int(x) for x in table[f])
        t0 = int(p.cu[i]) + 64 * c
        m = min(64, int(p.cu[i + 1]) - t0)
        for h in range(p.H):
            fa = oracle.chunk_factors(p, h, t0, m)
            S = ch["chunk_states"][f, h].T          # [k][v]
            np.testing.assert_allclose(fa["U"] - fa["W"] @ S, ch["vnew"][t0:t0 + m, h],
                                       rtol=1e-9, atol=1e-11)
            T = fa["T"]
            assert np.allclose(np.triu(T, 1), 0) and np.allclose(np.diag(T), 1)
    # a plausible slip (the decay on the wrong side of A) breaks the match
    p2 = rand_problem(32, [64], D=8, init=True)
    ch2 = oracle.chunked(p2, 64, dump=True)
    fa = oracle.chunk_factors(p2, 0, 0, 64)
    G, beta = fa["G"], fa["beta"]
    K = p2.k[0:64, 0] / np.sqrt(np.sum(p2.k[0:64, 0] ** 2, 1) + 1e-6)[:, None]
    A_bad = np.tril(beta[:, None] * np.exp(G[None, :] - G[:, None]) * (K @ K.T), -1)
    T_bad = np.linalg.inv(np.eye(64) + A_bad)
    W_bad = T_bad @ ((beta * np.exp(G))[:, None] * K)
    U_bad = T_bad @ (beta[:, None] * p2.v[0:64, 0])
    S = ch2["chunk_states"][0, 0].T
    assert not np.allclose(U_bad - W_bad @ S, ch2["vnew"][0:64, 0], rtol=1e-6)
