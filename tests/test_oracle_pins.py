"""Pins of the fp64 oracle to facts the pages and mathematics fix.

None of these tests retypes an oracle formula: they use closed forms, limit
cases the pages state, exact rational arithmetic on a different formulation
(explicit transition matrices), the affine (KCP) structure, the chunkwise
reorganisation and numbers printed on the pages (tests/golden).
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import kda_oracle as ora

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))

BF16_MAX = float((2 - 2 ** -7) * 2 ** 127)
F32_MAX = float(np.finfo(np.float32).max)
F16_MAX = 65504.0
F64_MAX = float(np.finfo(np.float64).max)


def rand_problem(rng, B=2, T=37, H=3, Dk=8, Dv=6, s0=True):
    q = ora.l2_normalize(rng.standard_normal((B, T, H, Dk)))
    k = ora.l2_normalize(rng.standard_normal((B, T, H, Dk)))
    v = rng.standard_normal((B, T, H, Dv))
    g = ora.bounded_log_decay(rng.standard_normal((B, T, H, Dk)), rng.normal(0, 0.5, H))
    beta = ora.sigmoid(rng.standard_normal((B, T, H)))
    S0 = rng.normal(0, 0.3, (B, H, Dk, Dv)) if s0 else None
    return q, k, v, g, beta, S0


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# --------------------------------------------------------------------- gates

class TestGate:
    """Bounded log-decay, [LinAttn-demo] Eq. 8 / [Impl-KDA] 'La décroissance bornée'."""

    def test_zero_logit_gives_half_bound(self):
        # sigmoid(0) = 1/2 for every head scale: g = g_min / 2 exactly.
        z = np.zeros((1, 4, 3, 5))
        for A in ([0.0, 1.0, -2.0], [3.0, 0.3, -0.7]):
            g = ora.bounded_log_decay(z, np.array(A), -5.0)
            assert np.all(g == -2.5)

    def test_strict_bounds_and_alpha_range(self):
        rng = np.random.default_rng(0)
        z = rng.normal(0, 6, (2, 50, 4, 16))
        g = ora.bounded_log_decay(z, rng.normal(0, 0.5, 4), -5.0)
        assert np.all(g < 0) and np.all(g > -5.0)
        a = np.exp(g)
        assert np.all(a < 1) and np.all(a > math.exp(-5.0))

    def test_inverse_saturation_monotone(self):
        # [LinAttn-demo] Tab 2: larger z forgets more (alpha decreases in z).
        z = np.linspace(-8, 8, 401).reshape(1, -1, 1, 1)
        a = np.exp(ora.bounded_log_decay(z, np.array([0.4]), -5.0)).ravel()
        assert np.all(np.diff(a) < 0)
        # saturation limits: alpha -> 1 as z -> -inf, alpha -> exp(g_min) as z -> +inf
        ends = np.exp(ora.bounded_log_decay(np.array([[[[-60.0]], [[60.0]]]]), np.array([0.0]), -5.0)).ravel()
        assert abs(ends[0] - 1.0) < 1e-15 and abs(ends[1] - math.exp(-5.0)) < 1e-15

    def test_head_scale_multiplies_logit(self):
        # exp(A_log) scales z: A_log = ln 2 at z equals A_log = 0 at 2z.
        z = np.linspace(-3, 3, 13).reshape(1, -1, 1, 1)
        g1 = ora.bounded_log_decay(z, np.array([math.log(2.0)]), -5.0)
        g2 = ora.bounded_log_decay(2 * z, np.array([0.0]), -5.0)
        assert np.max(np.abs(g1 - g2)) < 1e-15

    def test_gate_derivative_minimum_matches_page(self):
        # [LinAttn-demo] Tab 3: alpha floor 0.01 (g_min = ln 0.01), A_log = 0:
        # d alpha / dz has its minimum about -0.29 near z = -1.5.
        gold = GOLD["gate_v2_dalpha_dz_min"]
        gmin = math.log(gold["alpha_floor"])
        z = np.linspace(-6, 6, 120001)
        h = 1e-5
        ap = np.exp(ora.bounded_log_decay((z + h).reshape(1, -1, 1, 1), np.array([gold["A_log"]]), gmin)).ravel()
        am = np.exp(ora.bounded_log_decay((z - h).reshape(1, -1, 1, 1), np.array([gold["A_log"]]), gmin)).ravel()
        d = (ap - am) / (2 * h)
        i = int(np.argmin(d))
        assert abs(d[i] - gold["value"]) <= gold["abs_tol"]
        assert abs(z[i] - gold["at_z"]) <= gold["z_tol"]

    def test_sigmoid_closed_values(self):
        x = np.array([0.0, math.log(3.0), -math.log(3.0), 800.0, -800.0])
        s = ora.sigmoid(x)
        assert s[0] == 0.5
        assert abs(s[1] - 0.75) < 1e-16 and abs(s[2] - 0.25) < 1e-16
        assert s[3] == 1.0 and s[4] == 0.0


class TestSoftplusGate:
    """The unbounded KDA v1 gate g = -exp(A_log) softplus(z) ([Impl-KDA] 'La
    décroissance bornée' states it as the form being replaced; [LinAttn-demo] Tab 3)."""

    def test_closed_values(self):
        # softplus(0) = ln 2; softplus(ln 3) = ln 4; A_log = ln 2 doubles g
        z = np.array([0.0, math.log(3.0), -math.log(3.0)]).reshape(1, -1, 1, 1)
        g = ora.softplus_log_decay(z, np.array([0.0])).ravel()
        assert abs(g[0] + math.log(2.0)) < 1e-15 and abs(g[1] + math.log(4.0)) < 1e-15
        assert abs(g[2] + math.log(4.0 / 3.0)) < 1e-15
        g2 = ora.softplus_log_decay(z, np.array([math.log(2.0)])).ravel()
        assert np.max(np.abs(g2 - 2 * g)) < 1e-15

    def test_retention_is_logistic_at_unit_scale(self):
        # A_log = 0: alpha = exp(-softplus(z)) = 1 / (1 + e^z) = sigmoid(-z)
        z = np.linspace(-30, 30, 601).reshape(1, -1, 1, 1)
        a = np.exp(ora.softplus_log_decay(z, np.array([0.0])))
        assert np.max(np.abs(a - 1.0 / (1.0 + np.exp(z)))) < 1e-15

    def test_unbounded_below_and_stable_tails(self):
        # z -> +inf: g ~ -exp(A) z (no floor, unlike the bounded gate); z -> -inf: g -> 0-
        z = np.array([800.0, 60.0, -60.0, -800.0]).reshape(1, -1, 1, 1)
        g = ora.softplus_log_decay(z, np.array([0.5])).ravel()
        assert np.all(np.isfinite(g)) and np.all(g <= 0.0)
        assert abs(g[0] + math.exp(0.5) * 800.0) < 1e-9 and abs(g[1] + math.exp(0.5) * 60.0) < 1e-9
        assert 0 > g[2] > -1e-25 and g[3] <= 0.0 and g[3] > -1e-300
        assert g[0] < -5.0 * 100  # far below any bounded gate's floor

    def test_gate_derivative_minimum_matches_page(self):
        # [LinAttn-demo] Tab 3 (v1 curve): d alpha / dz has its minimum about -0.25 at z = 0
        gold = GOLD["gate_v1_dalpha_dz_min"]
        z = np.linspace(-6, 6, 120001)
        h = 1e-5
        ap = np.exp(ora.softplus_log_decay((z + h).reshape(1, -1, 1, 1), np.array([gold["A_log"]]))).ravel()
        am = np.exp(ora.softplus_log_decay((z - h).reshape(1, -1, 1, 1), np.array([gold["A_log"]]))).ravel()
        d = (ap - am) / (2 * h)
        i = int(np.argmin(d))
        assert abs(d[i] - gold["value"]) <= gold["abs_tol"]
        assert abs(z[i] - gold["at_z"]) <= gold["z_tol"]

    def test_prepare_selects_the_v1_gate(self):
        rng = np.random.default_rng(41)
        q, k, z = (rng.standard_normal((1, 5, 2, 4)) for _ in range(3))
        br = rng.standard_normal((1, 5, 2))
        A = np.array([0.3, -0.2])
        _, _, g1, _ = ora.prepare(q, k, z, br, A, flags=ora.FLAGS_DEFAULT | ora.GATE_SOFTPLUS)
        _, _, g2, _ = ora.prepare(q, k, z, br, A, flags=ora.FLAGS_DEFAULT)
        assert np.max(np.abs(g1 - ora.softplus_log_decay(z, A))) == 0.0
        assert np.max(np.abs(g2 - ora.bounded_log_decay(z, A))) == 0.0
        # the bias of the grouped path is added before either gate
        _, _, g3, _ = ora.prepare(q, k, ora.biased_logit(z, np.full((2, 4), 1.5)), br, A,
                                  flags=ora.FLAGS_DEFAULT | ora.GATE_SOFTPLUS)
        assert np.max(np.abs(g3 - ora.softplus_log_decay(z + 1.5, A))) < 1e-15


class TestL2Norm:
    def test_unit_norm_and_scale_invariance(self):
        rng = np.random.default_rng(1)
        x = rng.standard_normal((5, 7, 128))
        y = ora.l2_normalize(x, eps=0.0)
        assert np.max(np.abs(np.linalg.norm(y, axis=-1) - 1)) < 1e-14
        assert np.max(np.abs(ora.l2_normalize(37.5 * x, eps=0.0) - y)) < 1e-15

    def test_epsilon_is_inside_the_root(self):
        # a vector of squared norm 3e-6 with eps 1e-6 has norm sqrt(3/4) after scaling
        x = np.full((1, 3), 1e-3)
        y = ora.l2_normalize(x, eps=1e-6)
        assert abs(np.linalg.norm(y) - math.sqrt(0.75)) < 1e-12


# ------------------------------------------------------------ limit behaviours

class TestLimits:
    """[Impl-KDA] 'Vérifier votre implémentation', Test 1."""

    def test_beta_zero_is_pure_decay_bitwise(self):
        rng = np.random.default_rng(2)
        q, k, v, g, beta, S0 = rand_problem(rng, T=1)
        _, S1 = ora.recurrent(q, k, v, g, np.zeros_like(beta), S0)
        expect = np.exp(g[:, 0])[..., None] * S0
        assert np.array_equal(S1, expect)

    def test_unit_gates_recall_value_exactly(self):
        rng = np.random.default_rng(3)
        B, H, Dk, Dv = 2, 3, 16, 9
        k = ora.l2_normalize(rng.standard_normal((B, 1, H, Dk)), eps=0.0)
        v = rng.standard_normal((B, 1, H, Dv))
        _, S1 = ora.recurrent(k, k, v, np.zeros((B, 1, H, Dk)), np.ones((B, 1, H)), None)
        readout = np.einsum("bhk,bhkv->bhv", k[:, 0], S1)
        assert np.max(np.abs(readout - v[:, 0])) < 1e-15 * 16

    def test_repeated_key_closed_form(self):
        # same key written n times with the same value, alpha = 1:
        # the retrieved value is (1 - (1 - beta)^n) v.
        rng = np.random.default_rng(4)
        Dk, Dv, n, b = 8, 5, 9, 0.35
        kk = ora.l2_normalize(rng.standard_normal(Dk), eps=0.0)
        vv = rng.standard_normal(Dv)
        k = np.tile(kk, (1, n, 1, 1))
        v = np.tile(vv, (1, n, 1, 1))
        o, S = ora.recurrent(k, k, v, np.zeros((1, n, 1, Dk)), np.full((1, n, 1), b), None)
        for t in range(n):
            expect = (1 - (1 - b) ** (t + 1)) * vv
            assert np.max(np.abs(o[0, t, 0] - expect)) < 1e-14

    def test_latest_value_wins_for_unit_beta(self):
        # [KDA-demo] §1.3: with the same key and changing values, retrieval
        # follows the newest value (beta = 1, alpha = 1 overwrites exactly).
        rng = np.random.default_rng(5)
        Dk, Dv, n = 6, 4, 7
        kk = ora.l2_normalize(rng.standard_normal(Dk), eps=0.0)
        k = np.tile(kk, (1, n, 1, 1))
        v = rng.standard_normal((1, n, 1, Dv))
        o, _ = ora.recurrent(k, k, v, np.zeros((1, n, 1, Dk)), np.ones((1, n, 1)), None)
        assert np.max(np.abs(o - v)) < 1e-14

    def test_orthonormal_keys_textbook_delta_rule(self):
        # DeltaNet special case (alpha = beta = 1): S = sum_i k_i v_i^T for
        # orthonormal keys, so key k_j retrieves v_j.
        rng = np.random.default_rng(6)
        Dk, Dv = 12, 7
        Qm, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
        k = Qm.T.reshape(1, Dk, 1, Dk)
        v = rng.standard_normal((1, Dk, 1, Dv))
        _, S = ora.recurrent(k, k, v, np.zeros((1, Dk, 1, Dk)), np.ones((1, Dk, 1)), None)
        assert np.max(np.abs(S[0, 0] - Qm @ v[0, :, 0])) < 1e-14
        assert np.max(np.abs(Qm.T @ S[0, 0] - v[0, :, 0])) < 1e-14


# ------------------------------------------------- exact rational brute force

def _frac_transition_run(ks, vs, qs, alphas, betas, S0):
    """Exact arithmetic on the transition-matrix form S_t = M_t S_{t-1} + beta k v^T,
    M_t = (I - beta k k^T) Diag(alpha): a different formulation from the oracle's
    rank-1 update sequence."""
    Dk = len(ks[0])
    Dv = len(vs[0])
    S = [[Fraction(x) for x in row] for row in S0]
    outs = []
    for k, v, q, a, b in zip(ks, vs, qs, alphas, betas):
        M = [[((1 if i == j else 0) - b * k[i] * k[j]) * a[j] for j in range(Dk)] for i in range(Dk)]
        S = [[sum(M[i][m] * S[m][c] for m in range(Dk)) + b * k[i] * v[c] for c in range(Dv)]
             for i in range(Dk)]
        outs.append([sum(S[i][c] * q[i] for i in range(Dk)) for c in range(Dv)])
    return outs, S


def test_exact_rational_recurrence():
    F = Fraction
    ks = [(F(3, 5), F(4, 5)), (F(-4, 5), F(3, 5)), (F(5, 13), F(12, 13)),
          (F(1), F(0)), (F(8, 17), F(-15, 17))]
    vs = [(F(1, 2), F(-3)), (F(2), F(1, 7)), (F(-5, 4), F(3, 8)), (F(1, 3), F(1)), (F(0), F(-2))]
    qs = [(F(1), F(2)), (F(-1, 2), F(1, 4)), (F(3), F(-1)), (F(2, 3), F(5, 6)), (F(1, 9), F(-7, 3))]
    alphas = [(F(1, 2), F(3, 4)), (F(7, 8), F(1, 4)), (F(1), F(2, 3)), (F(5, 6), F(9, 10)), (F(1, 5), F(1))]
    betas = [F(1, 3), F(1, 2), F(9, 10), F(1), F(1, 4)]
    S0 = [(F(1, 2), F(-1)), (F(3, 2), F(2, 5))]
    o_ex, S_ex = _frac_transition_run(ks, vs, qs, alphas, betas, S0)

    f = lambda rows: np.array([[float(x) for x in r] for r in rows])
    k = f(ks).reshape(1, 5, 1, 2)
    v = f(vs).reshape(1, 5, 1, 2)
    q = f(qs).reshape(1, 5, 1, 2)
    g = np.log(f(alphas)).reshape(1, 5, 1, 2)
    beta = np.array([float(b) for b in betas]).reshape(1, 5, 1)
    o, S = ora.recurrent(q, k, v, g, beta, f(S0).reshape(1, 1, 2, 2))
    assert np.max(np.abs(o[0, :, 0] - f(o_ex))) < 1e-14
    assert np.max(np.abs(S[0, 0] - f(S_ex))) < 1e-14
    # the erase-before-decay reading of the other pages gives a different model
    S_alt = f(S0)
    for t in range(5):
        kt = k[0, t, 0]
        S_alt = np.exp(g[0, t, 0])[:, None] * S_alt + beta[0, t, 0] * np.outer(kt, v[0, t, 0] - S_alt.T @ kt)
    assert np.max(np.abs(S_alt - f(S_ex))) > 1e-3


# --------------------------------------------------- affine structure (KCP)

class TestAffine:
    def test_kcp_identity(self):
        # [Impl-KDA] Test 2: run(S0) = run(0) + (prod M_t) S0.
        gold = GOLD["kcp_identity_max_err"]
        rng = np.random.default_rng(7)
        q, k, v, g, beta, S0 = rand_problem(rng, T=53)
        _, S_direct = ora.recurrent(q, k, v, g, beta, S0)
        M, S_tilde = ora.segment_fragment(k, v, g, beta)
        err = np.max(np.abs(S_direct - (S_tilde + M @ S0)))
        assert err < min(gold["bar"], 1e-12)

    @pytest.mark.parametrize("nseg", [2, 4, 8])
    def test_prefix_scan_equals_full_run(self, nseg):
        # [Impl-KDA] Test 3 with 2, 4 and 8 simulated ranks (uneven cuts).
        gold = GOLD["prefix_scan_4_ranks_max_err"]
        rng = np.random.default_rng(8 + nseg)
        q, k, v, g, beta, _ = rand_problem(rng, T=61, s0=False)
        cuts = np.sort(rng.choice(np.arange(1, 61), nseg - 1, replace=False))
        bounds = [0, *cuts.tolist(), 61]
        frags = [ora.segment_fragment(k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b])
                 for a, b in zip(bounds[:-1], bounds[1:])]
        states = ora.compose(frags)
        _, S_full = ora.recurrent(q, k, v, g, beta, None)
        assert np.max(np.abs(states[-1] - S_full)) < min(gold["bar"], 1e-12)
        for s, b in enumerate(bounds[1:]):
            _, S_pref = ora.recurrent(q[:, :b], k[:, :b], v[:, :b], g[:, :b], beta[:, :b], None)
            assert np.max(np.abs(states[s] - S_pref)) < 1e-12

    def test_composition_is_associative(self):
        rng = np.random.default_rng(9)
        q, k, v, g, beta, _ = rand_problem(rng, T=30, s0=False)
        a, b, c = [ora.segment_fragment(k[:, i:j], v[:, i:j], g[:, i:j], beta[:, i:j])
                   for i, j in ((0, 9), (9, 20), (20, 30))]
        left = ora.compose_pair(ora.compose_pair(c, b), a)
        right = ora.compose_pair(c, ora.compose_pair(b, a))
        whole = ora.segment_fragment(k, v, g, beta)
        for x, y, w in zip(left, right, whole):
            assert np.max(np.abs(x - y)) < 1e-12 and np.max(np.abs(x - w)) < 1e-12

    def test_linear_in_values_and_state(self):
        # [Impl-KDA] 'Que teste réellement le test 2': the recurrence is affine,
        # so (o, S_T) is linear in (V, S0) jointly.
        rng = np.random.default_rng(10)
        q, k, v1, g, beta, S1 = rand_problem(rng, T=25)
        v2 = rng.standard_normal(v1.shape)
        S2 = rng.standard_normal(S1.shape)
        a, b = 0.7, -1.9
        o1, T1 = ora.recurrent(q, k, v1, g, beta, S1)
        o2, T2 = ora.recurrent(q, k, v2, g, beta, S2)
        o3, T3 = ora.recurrent(q, k, a * v1 + b * v2, g, beta, a * S1 + b * S2)
        assert rel(o3, a * o1 + b * o2) < 1e-12 and rel(T3, a * T1 + b * T2) < 1e-12

    def test_resume_from_state(self):
        rng = np.random.default_rng(11)
        q, k, v, g, beta, S0 = rand_problem(rng, T=40)
        o, S = ora.recurrent(q, k, v, g, beta, S0)
        oa, Sa = ora.recurrent(q[:, :17], k[:, :17], v[:, :17], g[:, :17], beta[:, :17], S0)
        ob, Sb = ora.recurrent(q[:, 17:], k[:, 17:], v[:, 17:], g[:, 17:], beta[:, 17:], Sa)
        assert rel(np.concatenate([oa, ob], 1), o) < 1e-13 and rel(Sb, S) < 1e-13

    def test_transition_matches_one_token(self):
        rng = np.random.default_rng(12)
        q, k, v, g, beta, S0 = rand_problem(rng, T=1)
        _, S1 = ora.recurrent(q, k, v, g, beta, S0)
        M = ora.transition(k[:, 0], beta[:, 0], np.exp(g[:, 0]))
        expect = M @ S0 + beta[:, 0][..., None, None] * np.einsum("bhk,bhv->bhkv", k[:, 0], v[:, 0])
        assert np.max(np.abs(S1 - expect)) < 1e-14


    def test_readout_map_is_the_state_part_of_the_output(self):
        # affine in S0: o(S0) - o(0) = P S0, for any S0 (two random ones)
        rng = np.random.default_rng(13)
        q, k, v, g, beta, _ = rand_problem(rng, T=23)
        P = ora.readout_map(q, k, g, beta)
        o0, _ = ora.recurrent(q, k, v, g, beta, None)
        for seed in (1, 2):
            S0 = np.random.default_rng(seed).standard_normal((q.shape[0], q.shape[2], q.shape[3], v.shape[3]))
            oS, _ = ora.recurrent(q, k, v, g, beta, S0)
            assert rel(oS - o0, np.einsum("bthk,bhkv->bthv", P, S0)) < 1e-12

    def test_readout_map_first_token(self):
        # one token: P_1 = q_1^T M_1 with M_1 from the transition alone
        rng = np.random.default_rng(14)
        q, k, _, g, beta, _ = rand_problem(rng, T=1)
        M = ora.transition(k[:, 0], beta[:, 0], np.exp(g[:, 0]))
        expect = np.einsum("bhi,bhij->bhj", q[:, 0], M)
        assert np.max(np.abs(ora.readout_map(q, k, g, beta)[:, 0] - expect)) < 1e-14

    @pytest.mark.parametrize("with_state", [False, True])
    def test_segment_fixup_rebuilds_the_full_run(self, with_state):
        # KCP end to end: every segment from a zero state, its fragment and
        # readout map, the prefix scan, then the fix-up = the full recurrence.
        n, Tseg = 4, 11
        rng = np.random.default_rng(15 + with_state)
        q, k, v, g, beta, S0 = rand_problem(rng, T=n * Tseg, s0=with_state)
        parts = [slice(s * Tseg, (s + 1) * Tseg) for s in range(n)]
        o_zero = np.stack([ora.recurrent(q[:, p], k[:, p], v[:, p], g[:, p], beta[:, p], None)[0]
                           for p in parts])
        P = np.stack([ora.readout_map(q[:, p], k[:, p], g[:, p], beta[:, p]) for p in parts])
        S_pref = np.stack(ora.compose([ora.segment_fragment(k[:, p], v[:, p], g[:, p], beta[:, p])
                                       for p in parts], S0))
        o = ora.segment_fixup(o_zero, P, S_pref, S0)
        o_full, _ = ora.recurrent(q, k, v, g, beta, S0)
        assert rel(np.concatenate(list(o), axis=1), o_full) < 1e-12


# ----------------------------------------------------------- chunkwise form

@pytest.mark.parametrize("chunk", [8, 16, 32, 64])
def test_chunkwise_equals_recurrence(chunk):
    # [KDA-demo] Tab 8: the two forms agree to fp64 precision (bar 1e-10).
    gold = GOLD["recurrent_vs_chunk_fp64"]
    rng = np.random.default_rng(20 + chunk)
    q, k, v, g, beta, S0 = rand_problem(rng, B=2, T=141, H=2, Dk=16, Dv=12)
    o_r, S_r = ora.recurrent(q, k, v, g, beta, S0)
    o_c, S_c = ora.chunkwise(q, k, v, g, beta, S0, chunk=chunk)
    assert rel(o_c, o_r) < min(gold["bar"], 1e-12)
    assert rel(S_c, S_r) < min(gold["bar"], 1e-12)


def test_chunkwise_survives_strongest_decay():
    # worst-case gate (g = g_min on every token) over a 64-token chunk: the
    # element-wise factors stay finite and the forms still agree.
    rng = np.random.default_rng(30)
    q, k, v, _, beta, S0 = rand_problem(rng, B=1, T=128, H=1, Dk=8, Dv=8)
    g = np.full(q.shape, -5.0 + 1e-9)
    o_r, S_r = ora.recurrent(q, k, v, g, beta, S0)
    o_c, S_c = ora.chunkwise(q, k, v, g, beta, S0, chunk=64)
    assert np.all(np.isfinite(o_c)) and rel(o_c, o_r) < 1e-12 and rel(S_c, S_r) < 1e-12


def test_step_matches_sequence():
    # [KDA-demo] Tab 13: stepping token by token equals the sequence form.
    rng = np.random.default_rng(31)
    B, T, H, Dk, Dv = 2, 9, 3, 8, 5
    q, k, z = (rng.standard_normal((B, T, H, Dk)) for _ in range(3))
    v = rng.standard_normal((B, T, H, Dv))
    br = rng.standard_normal((B, T, H))
    A = rng.normal(0, 0.5, H)
    S0 = rng.standard_normal((B, H, Dk, Dv))
    o, S = ora.forward(q, k, v, z, br, A, S0)
    St = S0
    for t in range(T):
        ot, St = ora.step(St, q[:, t], k[:, t], v[:, t], z[:, t], br[:, t], A)
        assert np.max(np.abs(ot - o[:, t])) < 1e-13
    assert np.max(np.abs(St - S)) < 1e-13


def test_switches_off_take_activated_inputs():
    # [KDA-layer] 'three in_kernel switches': with a switch off the caller has
    # already applied the activation.
    rng = np.random.default_rng(32)
    B, T, H, Dk, Dv = 1, 6, 2, 4, 3
    q, k, z = (rng.standard_normal((B, T, H, Dk)) for _ in range(3))
    v = rng.standard_normal((B, T, H, Dv))
    br = rng.standard_normal((B, T, H))
    A = rng.normal(0, 0.5, H)
    o_on, S_on = ora.forward(q, k, v, z, br, A, flags=ora.FLAGS_DEFAULT)
    o_off, S_off = ora.forward(q / np.linalg.norm(q, axis=-1, keepdims=True),
                               k / np.linalg.norm(k, axis=-1, keepdims=True), v,
                               -5.0 / (1 + np.exp(-np.exp(A)[:, None] * z)),
                               1 / (1 + np.exp(-br)), A, flags=0)
    # eps = 1e-6 inside the root makes the only difference (relative ~1e-7)
    assert rel(o_off, o_on) < 1e-5 and rel(S_off, S_on) < 1e-5


# --------------------------------------------------------- safe chunk size

class TestSafeChunk:
    """[KDA-demo] §1.4 and Tab 9; [Impl-KDA] 'La décroissance bornée'."""

    def test_page_values(self):
        s_bf = ora.safe_chunk_size(-5.0, BF16_MAX)
        s_32 = ora.safe_chunk_size(-5.0, F32_MAX)
        assert s_bf == GOLD["safe_tile_g_min_5"]["value"] == s_32
        assert s_bf < GOLD["unsafe_tile_g_min_5"]["value"]
        assert ora.safe_chunk_size(GOLD["g_min_10_overflows_at_16"]["value"], BF16_MAX) < 16
        assert ora.safe_chunk_size(-10.0, BF16_MAX) == 8
        assert ora.safe_chunk_size(-5.0, F16_MAX) == 0
        assert ora.safe_chunk_size(-5.0, F64_MAX) == 140
        gold = GOLD["exp80"]
        assert abs(math.exp(80) - gold["value"]) <= gold["rel_tol"] * gold["value"]
        assert abs(BF16_MAX - GOLD["bf16_max"]["value"]) <= GOLD["bf16_max"]["rel_tol"] * BF16_MAX
        assert abs(F32_MAX - GOLD["fp32_max"]["value"]) <= GOLD["fp32_max"]["rel_tol"] * F32_MAX

    def test_bf16_and_fp32_curves_coincide(self):
        for gm in np.linspace(-12, -0.5, 200):
            assert ora.safe_chunk_size(gm, BF16_MAX) == ora.safe_chunk_size(gm, F32_MAX)

    def test_fp32_inverse_retention_overflow_edge(self):
        # worst case alpha = exp(g_min): 1/gamma over n tokens is exp(5 n);
        # finite in fp32 at 17 tokens, inf at 18 (headroom 1 gives 17).
        with np.errstate(over="ignore"):
            assert np.isfinite(np.float32(math.exp(5 * 17)))
            assert np.isinf(np.float32(math.exp(5 * 18)))
        assert ora.safe_chunk_size(-5.0, F32_MAX, headroom=1.0) == 17

    def test_rejects_bad_bound(self):
        for bad in (0.0, 1.0, float("nan"), float("-inf")):
            with pytest.raises(ValueError):
                ora.safe_chunk_size(bad, F32_MAX)


# ---------------------------------------------------------------------------
# Input side: short convolution and SiLU ([KDA-demo] §1.1, §1.7;
# [Impl-KDA] "La paramétrisation")
# ---------------------------------------------------------------------------

class TestShortConv:
    def test_identity_initialisation_is_a_no_op(self):
        # [KDA-demo] §1.1: last tap 1, the others 0 -> the layer is a no-op
        rng = np.random.default_rng(11)
        x = rng.standard_normal((2, 9, 6))
        w = np.zeros((6, 4))
        w[:, -1] = 1.0
        y, st = ora.short_conv(x, w)
        assert np.array_equal(y, x)
        assert np.array_equal(st, x[:, -3:])

    def test_matches_numpy_convolution(self):
        # causal correlation = full convolution with the reversed kernel,
        # truncated to T (np.convolve zero-pads the past, as the pages do)
        rng = np.random.default_rng(12)
        B, T, C = 2, 13, 5
        x = rng.standard_normal((B, T, C))
        w = rng.standard_normal((C, 4))
        bias = rng.standard_normal(C)
        y, _ = ora.short_conv(x, w, bias)
        for b in range(B):
            for c in range(C):
                ref = np.convolve(x[b, :, c], w[c, ::-1])[:T] + bias[c]
                assert np.allclose(y[b, :, c], ref, rtol=0, atol=1e-12)

    def test_shift_kernel_delays_by_three(self):
        # only the first tap: y[t] = x[t - 3], zero for t < 3 (left zero padding)
        rng = np.random.default_rng(13)
        x = rng.standard_normal((1, 8, 3))
        w = np.zeros((3, 4))
        w[:, 0] = 1.0
        y, _ = ora.short_conv(x, w)
        assert np.array_equal(y[:, 3:], x[:, :-3])
        assert np.array_equal(y[:, :3], np.zeros((1, 3, 3)))

    @pytest.mark.parametrize("split", [1, 2, 3, 5, 9])
    def test_state_continues_a_sequence(self, split):
        # [KDA-demo] §1.1 单步 decode: the K - 1 input window carries the sequence
        rng = np.random.default_rng(14 + split)
        x = rng.standard_normal((2, 10, 4))
        w = rng.standard_normal((4, 4))
        s0 = rng.standard_normal((2, 3, 4))
        y_full, st_full = ora.short_conv(x, w, None, s0)
        y1, st1 = ora.short_conv(x[:, :split], w, None, s0)
        y2, st2 = ora.short_conv(x[:, split:], w, None, st1)
        assert np.allclose(np.concatenate([y1, y2], axis=1), y_full, rtol=0, atol=1e-13)
        assert np.array_equal(st2, st_full)
        # the window is the last three inputs of (state, x)
        assert np.array_equal(st_full, np.concatenate([s0, x], axis=1)[:, -3:])

    def test_token_by_token_window_equals_sequence(self):
        rng = np.random.default_rng(21)
        x = rng.standard_normal((1, 6, 2))
        w = rng.standard_normal((2, 4))
        y_full, _ = ora.short_conv(x, w)
        st = None
        for t in range(6):
            y_t, st = ora.short_conv(x[:, t:t + 1], w, None, st)
            assert np.allclose(y_t[:, 0], y_full[:, t], rtol=0, atol=1e-13)


class TestSilu:
    def test_odd_part_is_identity(self):
        # x sigmoid(x) - (-x) sigmoid(-x) = x (sigmoid(x) + sigmoid(-x) = 1)
        x = np.linspace(-30, 30, 601)
        assert np.allclose(ora.silu(x) - ora.silu(-x), x, rtol=0, atol=1e-12)

    def test_limits_and_zero(self):
        assert ora.silu(np.array([0.0]))[0] == 0.0
        assert abs(ora.silu(np.array([40.0]))[0] - 40.0) < 1e-12
        assert abs(ora.silu(np.array([-40.0]))[0]) < 1e-15
        # the minimum of x sigmoid(x) is at x* with x* = -(1 + e^{x*}) (d/dx = 0),
        # about -1.2785: check against a dense grid
        xs = np.linspace(-3, 0, 30001)
        i = int(np.argmin(ora.silu(xs)))
        assert abs(xs[i] + 1 + math.exp(xs[i])) < 2e-4

    def test_conv_silu_composes_in_the_pages_order(self):
        # [KDA-demo] §1.7: ShortConv first, then SiLU; with identity taps the
        # composition is SiLU alone
        rng = np.random.default_rng(22)
        x = rng.standard_normal((1, 5, 3))
        w = np.zeros((3, 4))
        w[:, -1] = 1.0
        y, _ = ora.conv_silu(x, w)
        assert np.allclose(y, x / (1 + np.exp(-x)), rtol=1e-14, atol=0)


# ---------------------------------------------------------------------------
# Output side: per-head RMS normalisation and sigmoid gate ([KDA-demo] §1.7;
# [Impl-KDA] kda_output)
# ---------------------------------------------------------------------------

class TestOutputGate:
    def test_rms_of_normalised_head_is_one(self):
        rng = np.random.default_rng(31)
        o = rng.standard_normal((2, 5, 3, 64)) * 7.0
        y = ora.head_rms_norm(o, eps=0.0)
        assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=0, atol=1e-13)

    def test_scale_invariance_and_constant_head(self):
        rng = np.random.default_rng(32)
        o = rng.standard_normal((1, 4, 2, 32))
        assert np.allclose(ora.head_rms_norm(5.0 * o, eps=0.0), ora.head_rms_norm(o, eps=0.0), rtol=0, atol=1e-13)
        # a head of equal entries c normalises to sign(c) * 1 (eps -> 0)
        c = np.full((1, 1, 1, 16), -3.0)
        assert np.allclose(ora.head_rms_norm(c, eps=0.0), -1.0, rtol=0, atol=1e-15)
        # eps keeps a zero head at zero
        assert np.array_equal(ora.head_rms_norm(np.zeros((1, 1, 1, 8))), np.zeros((1, 1, 1, 8)))

    def test_gate_limits_and_weight(self):
        rng = np.random.default_rng(33)
        o = rng.standard_normal((1, 3, 2, 16))
        w = rng.standard_normal(16)
        n = ora.head_rms_norm(o, w, eps=0.0)
        # gate logit 0 halves, large positive passes, large negative closes
        assert np.allclose(ora.output_gate(o, np.zeros_like(o), w, eps=0.0), 0.5 * n, rtol=0, atol=1e-14)
        assert np.allclose(ora.output_gate(o, np.full_like(o, 60.0), w, eps=0.0), n, rtol=0, atol=1e-13)
        assert np.max(np.abs(ora.output_gate(o, np.full_like(o, -60.0), w, eps=0.0))) < 1e-24
        # the weight multiplies channels after the normalisation
        assert np.allclose(n, ora.head_rms_norm(o, eps=0.0) * w, rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# Variants: grouped value heads and the gate bias ([KDA-layer] 完整数据流 and
# its parameter table)
# ---------------------------------------------------------------------------

class TestGroupedHeads:
    def _problem(self, rng, B=2, T=19, H=2, HV=6, Dk=8, Dv=5):
        q = rng.standard_normal((B, T, H, Dk))
        k = rng.standard_normal((B, T, H, Dk))
        v = rng.standard_normal((B, T, HV, Dv))
        z = rng.standard_normal((B, T, HV, Dk))
        br = rng.standard_normal((B, T, HV))
        A = rng.normal(0, 0.5, HV)
        S0 = rng.normal(0, 0.3, (B, HV, Dk, Dv))
        return q, k, v, z, br, A, S0

    def test_equal_head_counts_is_the_plain_core(self):
        rng = np.random.default_rng(51)
        q, k, v, z, br, A, S0 = self._problem(rng, H=3, HV=3)
        o1, S1 = ora.forward_grouped(q, k, v, z, br, A, None, S0)
        o2, S2 = ora.forward(q, k, v, z, br, A, S0)
        assert np.array_equal(o1, o2) and np.array_equal(S1, S2)

    def test_each_value_head_runs_with_its_groups_qk(self):
        # a loop over value heads, each an independent plain core on one head
        rng = np.random.default_rng(52)
        q, k, v, z, br, A, S0 = self._problem(rng)
        o, S = ora.forward_grouped(q, k, v, z, br, A, None, S0)
        G = v.shape[2] // q.shape[2]
        for hv in range(v.shape[2]):
            h = hv // G
            oh, Sh = ora.forward(q[:, :, [h]], k[:, :, [h]], v[:, :, [hv]], z[:, :, [hv]], br[:, :, [hv]],
                                 A[[hv]], S0[:, [hv]])
            assert np.allclose(o[:, :, [hv]], oh, rtol=0, atol=1e-12)
            assert np.allclose(S[:, [hv]], Sh, rtol=0, atol=1e-12)

    def test_gate_bias_limits(self):
        # with beta = 0 the state only decays: a large positive bias saturates
        # the gate at g_min (S_T = e^{T g_min} S0), a large negative one opens it
        # (S_T = S0)
        rng = np.random.default_rng(53)
        q, k, v, z, br, A, S0 = self._problem(rng, T=7, H=1, HV=2)
        beta0 = np.zeros_like(br)
        flags = ora.QK_L2NORM | ora.GATE_IN_KERNEL  # beta taken as given
        Dk = z.shape[-1]
        big = np.full((2, Dk), 80.0)
        _, S_hi = ora.forward_grouped(q, k, v, z * 0.01, beta0, np.zeros(2), big, S0, flags=flags)
        assert np.allclose(S_hi, math.exp(7 * ora.G_MIN_DEFAULT) * S0, rtol=1e-12, atol=0)
        _, S_lo = ora.forward_grouped(q, k, v, z * 0.01, beta0, np.zeros(2), -big, S0, flags=flags)
        assert np.allclose(S_lo, S0, rtol=1e-12, atol=0)

    def test_gate_bias_needs_the_in_kernel_gate(self):
        rng = np.random.default_rng(54)
        q, k, v, z, br, A, S0 = self._problem(rng, H=1, HV=1)
        with pytest.raises(ValueError):
            ora.forward_grouped(q, k, v, z, br, A, np.zeros((1, z.shape[-1])), S0, flags=ora.QK_L2NORM)

    def test_grouped_step_follows_the_sequence(self):
        rng = np.random.default_rng(55)
        q, k, v, z, br, A, S0 = self._problem(rng, T=5)
        db = rng.normal(0, 0.5, (v.shape[2], z.shape[-1]))
        o, S = ora.forward_grouped(q, k, v, z, br, A, db, S0)
        St = S0.copy()
        for t in range(5):
            ot, St = ora.step_grouped(St, q[:, t], k[:, t], v[:, t], z[:, t], br[:, t], A, db)
            assert np.allclose(ot, o[:, t], rtol=0, atol=1e-12)
        assert np.allclose(St, S, rtol=0, atol=1e-12)


# ------------------------------------------------------------------ backward

class TestBackward:
    """The adjoint of the recurrence (oracle.backward): reverse-mode
    differentiation of `forward`, which the pages do not derive."""

    @staticmethod
    def problem(rng, flags, B=1, T=6, H=2, Dk=3, Dv=2):
        q, k, z = (rng.standard_normal((B, T, H, Dk)) for _ in range(3))
        if not flags & ora.GATE_IN_KERNEL:
            z = -np.abs(z) * 2.0          # the caller's log-decay itself
        v = rng.standard_normal((B, T, H, Dv))
        br = rng.standard_normal((B, T, H))
        if not flags & ora.BETA_SIGMOID:
            br = ora.sigmoid(br)
        A = rng.normal(0, 0.5, H)
        S0 = rng.normal(0, 0.3, (B, H, Dk, Dv))
        do = rng.standard_normal((B, T, H, Dv))
        dST = rng.standard_normal((B, H, Dk, Dv))
        return dict(q=q, k=k, v=v, z=z, beta_raw=br, A_log=A, S0=S0), do, dST

    @pytest.mark.parametrize("flags", [ora.FLAGS_DEFAULT, ora.FLAGS_DEFAULT | ora.GATE_SOFTPLUS, 0,
                                       ora.QK_L2NORM | ora.BETA_SIGMOID])
    def test_matches_central_differences(self, flags):
        # L = sum(do * o) + sum(dS_T * S_T); every input element perturbed by +-1e-6
        rng = np.random.default_rng(50 + flags)
        args, do, dST = self.problem(rng, flags)
        grads = ora.backward(args["q"], args["k"], args["v"], args["z"], args["beta_raw"], args["A_log"], do,
                             dST, args["S0"], flags=flags)

        def loss(a):
            o, S = ora.forward(a["q"], a["k"], a["v"], a["z"], a["beta_raw"], a["A_log"], a["S0"], flags=flags)
            return float(np.sum(do * o) + np.sum(dST * S))

        names = {"q": "dq", "k": "dk", "v": "dv", "z": "dz", "beta_raw": "dbeta_raw", "A_log": "dA_log",
                 "S0": "dS0"}
        h = 1e-6
        for n, gname in names.items():
            x = args[n]
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                ap, am = dict(args), dict(args)
                ap[n] = x.copy(); ap[n][idx] += h
                am[n] = x.copy(); am[n][idx] -= h
                fd[idx] = (loss(ap) - loss(am)) / (2 * h)
            if not np.any(fd):
                assert not np.any(grads[gname]), n       # A_log with the gate switch off
                continue
            assert rel(grads[gname], fd) < 1e-6, (n, rel(grads[gname], fd))

    def test_state_gradient_is_the_transposed_linear_map(self):
        # o_t = o_t(0) + P_t S0 and S_T = S_T(0) + M S0 (readout map, segment
        # transition), so dS0 = sum_t P_t^T do_t + M^T dS_T exactly
        rng = np.random.default_rng(60)
        q, k, v, g, beta, S0 = rand_problem(rng, T=19)
        do = rng.standard_normal(v.shape)
        dST = rng.standard_normal(S0.shape)
        grads = ora.backward(q, k, v, g, beta, np.zeros(q.shape[2]), do, dST, S0, flags=0)
        P = ora.readout_map(q, k, g, beta)
        M, _ = ora.segment_fragment(k, v, g, beta)
        expect = np.einsum("bthk,bthv->bhkv", P, do) + np.einsum("bhjk,bhjv->bhkv", M, dST)
        assert rel(grads["dS0"], expect) < 1e-12

    def test_value_gradient_of_an_isolated_token(self):
        # one token from a zero state: o = q^T k beta v, so dv = beta (q . k) do
        # and dbeta = (q . k) (v . do) (alpha drops out: the state starts empty)
        rng = np.random.default_rng(61)
        q, k, v, g, beta, _ = rand_problem(rng, T=1, s0=False)
        do = rng.standard_normal(v.shape)
        grads = ora.backward(q, k, v, g, beta, np.zeros(q.shape[2]), do, None, None, flags=0)
        qk = np.sum(q[:, 0] * k[:, 0], axis=-1)
        assert rel(grads["dv"][:, 0], (beta[:, 0] * qk)[..., None] * do[:, 0]) < 1e-14
        assert rel(grads["dbeta_raw"][:, 0], qk * np.sum(v[:, 0] * do[:, 0], axis=-1)) < 1e-14
        assert np.max(np.abs(grads["dz"])) == 0.0


class TestBackwardGrouped:
    def test_matches_central_differences(self):
        # two q/k heads read by four value heads, with a gate bias
        rng = np.random.default_rng(70)
        B, T, H, HV, Dk, Dv = 1, 5, 2, 4, 3, 2
        q, k = (rng.standard_normal((B, T, H, Dk)) for _ in range(2))
        v = rng.standard_normal((B, T, HV, Dv))
        z = rng.standard_normal((B, T, HV, Dk))
        br = rng.standard_normal((B, T, HV))
        A = rng.normal(0, 0.5, HV)
        db = rng.normal(0, 1.0, (HV, Dk))
        S0 = rng.normal(0, 0.3, (B, HV, Dk, Dv))
        do = rng.standard_normal((B, T, HV, Dv))
        dST = rng.standard_normal((B, HV, Dk, Dv))
        args = dict(q=q, k=k, z=z, dt_bias=db)
        grads = ora.backward_grouped(q, k, v, z, br, A, do, db, dST, S0)

        def loss(a):
            o, S = ora.forward_grouped(a["q"], a["k"], v, a["z"], br, A, a["dt_bias"], S0)
            return float(np.sum(do * o) + np.sum(dST * S))

        h = 1e-6
        for n, gname in (("q", "dq"), ("k", "dk"), ("z", "dz"), ("dt_bias", "ddt_bias")):
            x = args[n]
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                ap, am = dict(args), dict(args)
                ap[n] = x.copy(); ap[n][idx] += h
                am[n] = x.copy(); am[n][idx] -= h
                fd[idx] = (loss(ap) - loss(am)) / (2 * h)
            assert rel(grads[gname], fd) < 1e-6, (n, rel(grads[gname], fd))

    def test_equal_heads_without_bias_is_the_plain_backward(self):
        rng = np.random.default_rng(71)
        q, k, v, g, beta, S0 = rand_problem(rng, T=11)
        do = rng.standard_normal(v.shape)
        a = ora.backward(q, k, v, g, beta, np.zeros(q.shape[2]), do, None, S0, flags=0)
        b = ora.backward_grouped(q, k, v, g, beta, np.zeros(q.shape[2]), do, None, None, S0, flags=0)
        for n in ("dq", "dk", "dv", "dz", "dbeta_raw", "dS0"):
            assert np.array_equal(a[n], b[n]), n
        assert "ddt_bias" not in b
