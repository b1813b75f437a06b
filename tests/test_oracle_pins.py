"""Pins for the fp64 oracle: checks against what the pages and the
mathematics fix, not against the oracle's own formula.

Sources (Kimi K3 explainer, SemiAnalysis, Chinese translation):
  * linear-attention section: online-learning view, S_t = S_{t-1} + beta v k^T;
  * DeltaNet section: S_t = S_{t-1} - beta_t (S_{t-1} k_t - v_t) k_t^T,
    one SGD step on 0.5 ||S k - v||^2;
  * GDN/KDA paragraph: a forget gate on S (scalar in GDN, one value per key
    channel in KDA);
  * FlashKDA paragraph: D_t / u_t recurrence, chunk unrolling, UT transform.
Each pin is also run against deliberately broken variants of the
recurrence (at the bottom) to show that the pins can fail.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import chunked_naive

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")
RNG = np.random.default_rng(12345)


def _rand_problem(T, H, D, *, seed, S0=True, gate="softplus", unit_k=True, Dv=None):
    r = np.random.default_rng(seed)
    Dv = Dv or D
    q = r.standard_normal((T, H, D))
    k = r.standard_normal((T, H, D))
    if unit_k:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((T, H, Dv))
    if gate == "softplus":
        g = -np.logaddexp(0.0, r.standard_normal((T, H, D)) + 2.0)
    elif gate == "zero":
        g = np.zeros((T, H, D))
    elif gate == "strong":
        g = -np.logaddexp(0.0, r.standard_normal((T, H, D)) + 6.0)
    else:
        raise ValueError(gate)
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal((T, H))))
    s0 = r.standard_normal((1, H, D, Dv)) * 0.5 if S0 else None
    return q, k, v, g, beta, s0


def _orc(q, k, v, g, beta, S0=None, cu=None):
    return oracle.recurrent(q, k, v, g, beta, S0=S0, cu_seqlens=cu)


# ----------------------------------------------------------------------------------------
# pin functions: each takes a runner with the oracle's signature and returns an error
# ----------------------------------------------------------------------------------------

def pin_deltanet(run):
    """alpha == 1: the DeltaNet update of the DeltaNet section, in S orientation."""
    q, k, v, g, beta, s0 = _rand_problem(23, 2, 6, seed=1, gate="zero")
    o, S = run(q, k, v, g, beta, s0)
    err = 0.0
    for h in range(2):
        Smat = s0[0, h].T.copy()                       # S = M^T, [Dv, Dk]
        for t in range(23):
            kt, vt = k[t, h], v[t, h]
            Smat = Smat - beta[t, h] * np.outer(Smat @ kt - vt, kt)
            err = max(err, np.abs(Smat @ q[t, h] - o[t, h]).max())
        err = max(err, np.abs(Smat.T - S[0, h]).max())
    return err


def pin_gdn(run):
    """Channel-uniform decay: GDN written as S_t = a_t S_{t-1}(I - b k k^T) + b v k^T."""
    q, k, v, g, beta, s0 = _rand_problem(19, 2, 5, seed=2)
    g = np.repeat(g[..., :1], 5, axis=-1)
    o, S = run(q, k, v, g, beta, s0)
    err = 0.0
    for h in range(2):
        Smat = s0[0, h].T.copy()
        for t in range(19):
            kt, vt, b = k[t, h], v[t, h], beta[t, h]
            a = np.exp(g[t, h, 0])
            Smat = a * Smat @ (np.eye(5) - b * np.outer(kt, kt)) + b * np.outer(vt, kt)
            err = max(err, np.abs(Smat @ q[t, h] - o[t, h]).max())
        err = max(err, np.abs(Smat.T - S[0, h]).max())
    return err


def pin_zero_beta(run):
    """beta == 0: the state only decays; M_T = Diag(exp(sum g)) M_0 and
    o_t = M_0^T (q_t * exp(sum_{s<=t} g_s))."""
    q, k, v, g, beta, s0 = _rand_problem(17, 2, 6, seed=3)
    beta = np.zeros_like(beta)
    o, S = run(q, k, v, g, beta, s0)
    cum = np.cumsum(g, axis=0)                          # [T, H, D]
    err = 0.0
    for h in range(2):
        for t in range(17):
            ref = s0[0, h].T @ (q[t, h] * np.exp(cum[t, h]))
            err = max(err, np.abs(ref - o[t, h]).max())
        err = max(err, np.abs(np.exp(cum[-1, h])[:, None] * s0[0, h] - S[0, h]).max())
    return err


def pin_deltanet_zero_beta_identity(run):
    """alpha == 1 and beta == 0: state unchanged, o_t = S0 q_t."""
    q, k, v, g, beta, s0 = _rand_problem(9, 1, 4, seed=4, gate="zero")
    beta = np.zeros_like(beta)
    o, S = run(q, k, v, g, beta, s0)
    ref_o = np.einsum("kv,tk->tv", s0[0, 0], q[:, 0])
    return max(np.abs(S - s0).max(), np.abs(o[:, 0] - ref_o).max())


def pin_full_forget(run):
    """alpha == 0 (g = -inf): M_t = beta_t k_t v_t^T, o_t = beta_t (k_t . q_t) v_t."""
    q, k, v, g, beta, s0 = _rand_problem(11, 2, 4, seed=5)
    g = np.full_like(g, -np.inf)
    o, S = run(q, k, v, g, beta, s0)
    ref_o = beta[..., None] * np.einsum("thc,thc->th", k, q)[..., None] * v
    ref_S = beta[-1][:, None, None] * np.einsum("hc,hv->hcv", k[-1], v[-1])
    return max(np.abs(o - ref_o).max(), np.abs(S[0] - ref_S).max())


def pin_retrieval(run):
    """beta == 1 and |k| == 1: after the step the memory returns v_t for key k_t
    exactly (the delta-rule objective 0.5||S k - v||^2 is zeroed), whatever the
    decay, because the decay is applied before the prediction. With q_t = k_t
    the read-out o_t must equal v_t."""
    q, k, v, g, beta, s0 = _rand_problem(21, 2, 7, seed=6)
    beta = np.ones_like(beta)
    o, _ = run(k.copy(), k, v, g, beta, s0)
    return np.abs(o - v).max()


def pin_linear_attention(run):
    """Orthonormal keys, alpha == 1, S0 = 0: S_{t-1} k_t = 0, so the delta rule
    reduces to linear attention's online update and o_t = sum_{s<=t} beta_s (k_s.q_t) v_s."""
    T, D = 6, 8
    r = np.random.default_rng(7)
    Qm, _ = np.linalg.qr(r.standard_normal((D, D)))
    k = Qm[:, :T].T[:, None, :].copy()                  # [T, 1, D], orthonormal rows
    q = r.standard_normal((T, 1, D))
    v = r.standard_normal((T, 1, 3))
    beta = r.uniform(0.1, 0.9, (T, 1))
    g = np.zeros((T, 1, D))
    o, _ = run(q, k, v, g, beta, None)
    err = 0.0
    for t in range(T):
        ref = sum(beta[s, 0] * (k[s, 0] @ q[t, 0]) * v[s, 0] for s in range(t + 1))
        err = max(err, np.abs(ref - o[t, 0]).max())
    return err


def pin_hand_fixtures(run):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    err = 0.0
    for c in cases:
        a = np.array(c["alpha"])
        with np.errstate(divide="ignore"):
            g = np.log(a)[:, None, :]
        q = np.array(c["q"])[:, None, :]
        k = np.array(c["k"])[:, None, :]
        v = np.array(c["v"])[:, None, :]
        beta = np.array(c["beta"])[:, None]
        s0 = np.array(c["S0"])[None, None]
        o, S = run(q, k, v, g, beta, s0)
        err = max(err, np.abs(o[:, 0] - np.array(c["o"])).max(),
                  np.abs(S[0, 0] - np.array(c["S_out"])).max())
    return err


PINS = [
    (pin_deltanet, 1e-12), (pin_gdn, 1e-12), (pin_zero_beta, 1e-13),
    (pin_deltanet_zero_beta_identity, 1e-14), (pin_full_forget, 1e-14),
    (pin_retrieval, 1e-12), (pin_linear_attention, 1e-12), (pin_hand_fixtures, 1e-14),
]


@pytest.mark.parametrize("pin,tol", PINS, ids=[p.__name__ for p, _ in PINS])
def test_oracle_pin(pin, tol):
    assert pin(_orc) <= tol


# ----------------------------------------------------------------------------------------
# the separately written chunked form (FlashKDA matrix form) against the recurrence
# ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("C", [1, 2, 3, 4, 8, 16, 64])
@pytest.mark.parametrize("gate", ["softplus", "strong", "zero"])
def test_chunked_matches_recurrent(C, gate):
    q, k, v, g, beta, s0 = _rand_problem(37, 2, 8, seed=100 + C, gate=gate)
    o1, S1 = _orc(q, k, v, g, beta, s0)
    o2, S2 = chunked_naive.chunked(q, k, v, g, beta, S0=s0, C=C)
    scale = max(1.0, np.abs(o1).max())
    assert np.abs(o1 - o2).max() <= 1e-12 * scale
    assert np.abs(S1 - S2).max() <= 1e-12 * max(1.0, np.abs(S1).max())


def test_chunked_matches_recurrent_varlen():
    lengths = [5, 0, 1, 33, 16, 17]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T = int(cu[-1])
    q, k, v, g, beta, _ = _rand_problem(T, 2, 6, seed=9)
    s0 = np.random.default_rng(10).standard_normal((len(lengths), 2, 6, 6))
    o1, S1 = _orc(q, k, v, g, beta, s0, cu)
    o2, S2 = chunked_naive.chunked(q, k, v, g, beta, S0=s0, cu_seqlens=cu, C=16)
    assert np.abs(o1 - o2).max() <= 1e-12
    assert np.abs(S1 - S2).max() <= 1e-12
    # a zero-length sequence hands its initial state through unchanged
    assert np.array_equal(S1[1], s0[1])


# ----------------------------------------------------------------------------------------
# structural properties of the method
# ----------------------------------------------------------------------------------------

def test_superposition_in_v_and_state():
    """For fixed q, k, g, beta the outputs are jointly linear in (V, S0)."""
    q, k, v, g, beta, s0 = _rand_problem(29, 2, 6, seed=11)
    v2 = np.random.default_rng(12).standard_normal(v.shape)
    s2 = np.random.default_rng(13).standard_normal(s0.shape)
    a, b = 0.7, -1.3
    oa, Sa = _orc(q, k, v, g, beta, s0)
    ob, Sb = _orc(q, k, v2, g, beta, s2)
    oc, Sc = _orc(q, k, a * v + b * v2, g, beta, a * s0 + b * s2)
    assert np.abs(a * oa + b * ob - oc).max() <= 1e-12
    assert np.abs(a * Sa + b * Sb - Sc).max() <= 1e-12
    # V = 0: outputs driven by the initial state alone
    o0, S0_out = _orc(q, k, np.zeros_like(v), g, beta, s0)
    assert np.abs(o0).max() > 0 and np.abs(S0_out).max() > 0


def test_varlen_equals_separate_runs():
    lengths = [7, 12, 1, 20]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    q, k, v, g, beta, _ = _rand_problem(int(cu[-1]), 3, 5, seed=14)
    s0 = np.random.default_rng(15).standard_normal((4, 3, 5, 5))
    o, S = _orc(q, k, v, g, beta, s0, cu)
    for n in range(4):
        a, b = cu[n], cu[n + 1]
        on, Sn = _orc(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], s0[n:n + 1])
        assert np.array_equal(on, o[a:b])
        assert np.array_equal(Sn[0], S[n])


def test_append_prefill_split():
    """prefill(x) == prefill(x[T1:], S0 = state after prefill(x[:T1]))."""
    q, k, v, g, beta, s0 = _rand_problem(40, 2, 6, seed=16)
    o, S = _orc(q, k, v, g, beta, s0)
    for T1 in (1, 13, 39):
        oa, Sa = _orc(q[:T1], k[:T1], v[:T1], g[:T1], beta[:T1], s0)
        ob, Sb = _orc(q[T1:], k[T1:], v[T1:], g[T1:], beta[T1:], Sa)
        assert np.abs(np.concatenate([oa, ob]) - o).max() <= 1e-13
        assert np.abs(Sb - S).max() <= 1e-13


def test_decode_steps_equal_prefill():
    """Repeated single-token decode steps reproduce a prefill of the same tokens."""
    N, H, D, steps = 3, 2, 5, 16
    r = np.random.default_rng(17)
    q, k, v, g, beta, _ = _rand_problem(steps * N, H, D, seed=18)
    q, k, v, g = (x.reshape(steps, N, H, D) for x in (q, k, v, g))
    beta = beta.reshape(steps, N, H)
    S = r.standard_normal((N, H, D, D))
    Sd = S.copy()
    outs = []
    for s in range(steps):
        o_s, Sd = oracle.decode_step(q[s], k[s], v[s], g[s], beta[s], Sd)
        outs.append(o_s)
    outs = np.stack(outs)                                   # [steps, N, H, D]
    # the same tokens as N packed sequences of length `steps`
    perm = lambda x: np.ascontiguousarray(np.swapaxes(x, 0, 1)).reshape(N * steps, *x.shape[2:])
    cu = np.arange(N + 1) * steps
    o, Sp = _orc(perm(q), perm(k), perm(v), perm(g), perm(beta), S, cu)
    assert np.abs(perm(outs) - o).max() <= 1e-13
    assert np.abs(Sp - Sd).max() <= 1e-13


def test_threads_do_not_change_results():
    q, k, v, g, beta, s0 = _rand_problem(50, 4, 6, seed=19)
    o1, S1 = oracle.recurrent(q, k, v, g, beta, S0=s0, nthreads=1)
    o4, S4 = oracle.recurrent(q, k, v, g, beta, S0=s0, nthreads=4)
    assert np.array_equal(o1, o4) and np.array_equal(S1, S4)


# ----------------------------------------------------------------------------------------
# the pins must be able to fail: broken variants of the recurrence (CPU only)
# ----------------------------------------------------------------------------------------

def _mutant(kind):
    def run(q, k, v, g, beta, S0=None, cu=None):
        T, H, Dk = q.shape
        Dv = v.shape[-1]
        o = np.zeros((T, H, Dv))
        S = np.zeros((1, H, Dk, Dv))
        for h in range(H):
            M = np.zeros((Dk, Dv)) if S0 is None else S0[0, h].copy()
            for t in range(T):
                a = np.exp(g[t, h])
                kt, qt, vt, b = k[t, h], q[t, h], v[t, h], beta[t, h]
                if kind == "predict_before_decay":
                    p = M.T @ kt
                    M = a[:, None] * M
                elif kind == "no_decay":
                    p = M.T @ kt
                elif kind == "decay_value_axis" and Dk == Dv:
                    M = M * a[None, :]
                    p = M.T @ kt
                else:
                    M = a[:, None] * M
                    p = M.T @ kt
                u = b * vt - p if kind == "beta_on_v_only" else b * (vt - p)
                Mprev = M
                M = M + np.outer(kt, u)
                if kind == "readout_before_write":
                    o[t, h] = Mprev.T @ qt
                elif kind == "transposed_readout" and Dk == Dv:
                    o[t, h] = M @ qt
                else:
                    o[t, h] = M.T @ qt
            S[0, h] = M
        return o, S
    return run


MUTANTS = ["predict_before_decay", "no_decay", "decay_value_axis", "beta_on_v_only",
           "readout_before_write", "transposed_readout"]


def test_reference_mutant_is_faithful():
    """The unmodified python variant passes every pin (so failures below are the mutation's)."""
    for pin, tol in PINS:
        assert pin(_mutant("none")) <= max(tol, 1e-12), pin.__name__


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_catch_mutant(kind):
    failed = [pin.__name__ for pin, tol in PINS if not pin(_mutant(kind)) <= max(tol, 1e-12)]
    assert failed, f"no pin detects mutant {kind}"


def test_l2norm_pins():
    """oracle.l2norm against values fixed by its definition: a 3-4-5 triangle,
    the eps term, scale invariance (eps = 0) and unit norms."""
    np.testing.assert_allclose(oracle.l2norm([3.0, 4.0], 0.0), [0.6, 0.8], rtol=0, atol=1e-15)
    np.testing.assert_allclose(oracle.l2norm([3.0, 4.0], 11.0), [0.5, 2.0 / 3.0], rtol=0, atol=1e-15)
    r = np.random.default_rng(5)
    x = r.normal(size=(7, 3, 64))
    np.testing.assert_allclose(oracle.l2norm(2.5 * x, 0.0), oracle.l2norm(x, 0.0), rtol=1e-14)
    np.testing.assert_allclose(np.linalg.norm(oracle.l2norm(x, 0.0), axis=-1), 1.0, rtol=1e-14)
    assert oracle.l2norm(x, 1e-6).shape == x.shape


# ---------------------------------------------------------------- output norm and gate
OUTPUT_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "output_gate_hand.json")


def _output_gate_mutants():
    """Plausible mistakes in the output side, each of which a pin below must reject."""
    def sum_not_mean(o, gate, weight=None, eps=1e-6):
        o = np.asarray(o, float)
        return o / np.sqrt(np.sum(o * o, -1, keepdims=True) + eps) * (1 if weight is None else weight) / (1 + np.exp(-np.asarray(gate)))

    def eps_outside(o, gate, weight=None, eps=1e-6):
        o = np.asarray(o, float)
        return o / (np.sqrt(np.mean(o * o, -1, keepdims=True)) + eps) * (1 if weight is None else weight) / (1 + np.exp(-np.asarray(gate)))

    def gate_sign(o, gate, weight=None, eps=1e-6):
        o = np.asarray(o, float)
        return o / np.sqrt(np.mean(o * o, -1, keepdims=True) + eps) * (1 if weight is None else weight) / (1 + np.exp(np.asarray(gate)))

    def norm_over_heads(o, gate, weight=None, eps=1e-6):
        o = np.asarray(o, float)
        return o / np.sqrt(np.mean(o * o, axis=(-2, -1), keepdims=True) + eps) * (1 if weight is None else weight) / (1 + np.exp(-np.asarray(gate)))
    return dict(sum_not_mean=sum_not_mean, eps_outside=eps_outside, gate_sign=gate_sign,
                norm_over_heads=norm_over_heads)


def _output_gate_pins(fn):
    """True when fn satisfies every output-side pin: the hand-worked cases, and the
    invariants an RMS norm with a sigmoid gate must have."""
    ok = True
    for c in json.load(open(OUTPUT_GOLDEN))["cases"]:
        w = None if c["weight"] is None else np.array(c["weight"])
        got = fn(np.array(c["o"]), np.array(c["gate"]), w, eps=c["eps"])
        ok &= np.allclose(got, np.array(c["out"]), rtol=1e-14, atol=1e-15)
    rng = np.random.default_rng(7)
    o = rng.normal(size=(5, 3, 16))
    z = rng.normal(size=(5, 3, 16))
    base = fn(o, z, None, eps=0.0)
    # scale invariance of the norm (eps = 0) and oddness in o
    ok &= np.allclose(fn(7.5 * o, z, None, eps=0.0), base, rtol=1e-13)
    ok &= np.allclose(fn(-o, z, None, eps=0.0), -base, rtol=1e-13)
    # an open gate (z -> +inf) leaves unit RMS per head; a closed one gives 0
    opened = fn(o, np.full_like(z, 60.0), None, eps=0.0)
    ok &= np.allclose(np.sqrt(np.mean(opened ** 2, -1)), 1.0, rtol=1e-12)
    ok &= np.allclose(fn(o, np.full_like(z, -60.0), None, eps=0.0), 0.0, atol=1e-20)
    # with eps the RMS becomes sqrt(ms / (ms + eps))
    ms = np.mean(o * o, -1)
    ok &= np.allclose(np.sqrt(np.mean(fn(o, np.full_like(z, 60.0), None, eps=0.5) ** 2, -1)),
                      np.sqrt(ms / (ms + 0.5)), rtol=1e-12)
    return bool(ok)


def test_output_gate_pins():
    assert _output_gate_pins(oracle.output_gate)


@pytest.mark.parametrize("kind", sorted(_output_gate_mutants()))
def test_output_gate_pins_catch_mutant(kind):
    assert not _output_gate_pins(_output_gate_mutants()[kind])
