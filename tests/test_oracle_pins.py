"""Pins of the float64 oracle against what the pages and the mathematics fix.

None of these tests compares the oracle with itself: each checks it against a
hand-worked example, a closed form, a special case of the recurrence, an
independent formulation (dense matrices, the fused single-pass form of the
"Module gdn" page, "The fusion"), an invariant, or a library routine.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import gdn_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _rand(seed, B=2, T=5, Hk=2, Hv=4, Dk=8, Dv=6, gated=False, s0_scale=0.5):
    r = np.random.default_rng(seed)
    d = dict(
        q=r.standard_normal((B, T, Hk, Dk)),
        k=r.standard_normal((B, T, Hk, Dk)),
        v=r.standard_normal((B, T, Hv, Dv)),
        log_decay=-np.logaddexp(0, r.standard_normal((B, T, Hv))),
        beta=1 / (1 + np.exp(-r.standard_normal((B, T, Hv)))),
        s0=r.standard_normal((B, Hv, Dv, Dk)) * s0_scale,
    )
    if gated:
        d["z"] = r.standard_normal((B, T, Hv, Dv))
        d["w"] = 1 + 0.1 * r.standard_normal((Dv,))
    return d


def _unit(x, axis=-1):
    return x / np.linalg.norm(x, axis=axis, keepdims=True)


# ---------------------------------------------------------------- worked examples
def test_hand_worked_examples():
    """Hand-derived examples ("Module gdn" page, module description)."""
    spec = json.load(open(GOLDEN))
    for ex in spec["examples"]:
        Dk, Dv, toks = ex["Dk"], ex["Dv"], ex["tokens"]
        T = len(toks)
        q = np.array([[t["q"] for t in toks]], dtype=float)[:, :, None, :]
        k = np.array([[t["k"] for t in toks]], dtype=float)[:, :, None, :]
        v = np.array([[t["v"] for t in toks]], dtype=float)[:, :, None, :]
        with np.errstate(divide="ignore"):
            g = np.log(np.array([[t["alpha"] for t in toks]], dtype=float))[:, :, None]
        b = np.array([[t["beta"] for t in toks]], dtype=float)[:, :, None]
        s0 = np.array(ex["s0"], dtype=float)[None, None]
        y, s = orc.scan(q, k, v, g, b, s0, fold_qk_l2norm=False, fold_q_scale=False)
        assert y.shape == (1, T, 1, Dv) and s.shape == (1, 1, Dv, Dk)
        np.testing.assert_allclose(y[0, :, 0], np.array(ex["y"], dtype=float), rtol=0, atol=1e-12,
                                   err_msg=ex["name"])
        np.testing.assert_allclose(s[0, 0], np.array(ex["s_final"], dtype=float), rtol=0,
                                   atol=1e-12, err_msg=ex["name"])


# ---------------------------------------------------------------- the fusion identity
def _fused_reference(d, fold=True, eps=1e-6):
    """Single-pass form of the "Module gdn" page, "The fusion":
    o[a] = alpha*(S_old.q)[a] + coef[a]*(k.q), coef[a] = beta*(v[a] - alpha*u[a]),
    S_new = alpha*S_old + coef k^T."""
    q, k, v, g, bt, s0 = (d[n] for n in ("q", "k", "v", "log_decay", "beta", "s0"))
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2:]
    G = Hv // Hk
    y = np.zeros((B, T, Hv, Dv))
    S = s0.copy()
    for b in range(B):
        for hv in range(Hv):
            St = S[b, hv]
            for t in range(T):
                qq, kk = q[b, t, hv // G].copy(), k[b, t, hv // G].copy()
                if fold:
                    qq = qq / math.sqrt((qq * qq).sum() + eps) / math.sqrt(Dk)
                    kk = kk / math.sqrt((kk * kk).sum() + eps)
                al, be = math.exp(g[b, t, hv]), bt[b, t, hv]
                u = St @ kk
                wq = St @ qq
                coef = be * (v[b, t, hv] - al * u)
                y[b, t, hv] = al * wq + coef * (kk @ qq)
                St = al * St + np.outer(coef, kk)
            S[b, hv] = St
    return y, S


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_fused_form_equals_three_pass(seed):
    d = _rand(seed)
    y, s = orc.scan(**d)
    yf, sf = _fused_reference(d)
    np.testing.assert_allclose(y, yf, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s, sf, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- special cases
def test_alpha1_beta0_leaves_memory_unchanged():
    d = _rand(3)
    d["log_decay"][:] = 0.0
    d["beta"][:] = 0.0
    d["q"] = _unit(d["q"])
    y, s = orc.scan(**d, fold_qk_l2norm=False, fold_q_scale=False)
    np.testing.assert_array_equal(s, d["s0"])
    G = d["v"].shape[2] // d["q"].shape[2]
    for hv in range(d["v"].shape[2]):
        ref = np.einsum("bac,btc->bta", d["s0"][:, hv], d["q"][:, :, hv // G])
        np.testing.assert_allclose(y[:, :, hv], ref, rtol=1e-13, atol=1e-14)


def test_alpha0_gives_beta_v_kT():
    d = _rand(4, T=1)
    d["log_decay"][:] = -np.inf
    d["k"], d["q"] = _unit(d["k"]), _unit(d["q"])
    y, s = orc.scan(**d, fold_qk_l2norm=False, fold_q_scale=False)
    G = d["v"].shape[2] // d["q"].shape[2]
    for b in range(2):
        for hv in range(d["v"].shape[2]):
            kk, qq = d["k"][b, 0, hv // G], d["q"][b, 0, hv // G]
            be, vv = d["beta"][b, 0, hv], d["v"][b, 0, hv]
            np.testing.assert_allclose(s[b, hv], be * np.outer(vv, kk), rtol=1e-14, atol=1e-15)
            np.testing.assert_allclose(y[b, 0, hv], be * vv * (kk @ qq), rtol=1e-13, atol=1e-14)


def test_update_along_and_across_the_key():
    """From S_new = alpha*S + beta*(v - alpha*S.k) k^T:
    S_new.k = alpha*(1 - beta*|k|^2)*S.k + beta*|k|^2*v, and S_new.x = alpha*S.x for x _|_ k.
    With alpha = beta = 1 and |k| = 1 this is S_new.k = v."""
    r = np.random.default_rng(5)
    Dk = Dv = 7
    s0 = r.standard_normal((1, 1, Dv, Dk))
    k = r.standard_normal((1, 1, 1, Dk)) * 1.7
    v = r.standard_normal((1, 1, 1, Dv))
    q = r.standard_normal((1, 1, 1, Dk))
    al, be = 0.7, 0.35
    y, s = orc.scan(q, k, v, np.log([[[al]]]), np.array([[[be]]]), s0,
                    fold_qk_l2norm=False, fold_q_scale=False)
    kk, S0, S1 = k[0, 0, 0], s0[0, 0], s[0, 0]
    n2 = kk @ kk
    np.testing.assert_allclose(S1 @ kk, al * (1 - be * n2) * (S0 @ kk) + be * n2 * v[0, 0, 0],
                               rtol=1e-12, atol=1e-12)
    x = r.standard_normal(Dk)
    x -= (x @ kk) / n2 * kk
    np.testing.assert_allclose(S1 @ x, al * (S0 @ x), rtol=1e-12, atol=1e-12)
    # alpha = beta = 1, unit key: the memory now returns v for k (any alpha in fact)
    ku = kk / math.sqrt(n2)
    for al2 in (1.0, 0.3):
        _, s2 = orc.scan(q, ku[None, None, None], v, np.log([[[al2]]]), np.ones((1, 1, 1)), s0,
                         fold_qk_l2norm=False, fold_q_scale=False)
        np.testing.assert_allclose(s2[0, 0] @ ku, v[0, 0, 0], rtol=1e-12, atol=1e-12)


def test_dense_matrix_brute_force():
    """S_t = S_{t-1} M_t + N_t with M_t = alpha_t (I - beta_t k_t k_t^T), N_t = beta_t v_t k_t^T,
    o_t = S_t q_t, multiplied out as dense matrices (T = 2 and T = 4)."""
    for T in (2, 4):
        d = _rand(6 + T, B=1, T=T, Hk=1, Hv=1, Dk=5, Dv=4)
        y, s = orc.scan(**d, fold_qk_l2norm=False, fold_q_scale=False)
        S = d["s0"][0, 0]
        for t in range(T):
            al, be = math.exp(d["log_decay"][0, t, 0]), d["beta"][0, t, 0]
            kk, vv, qq = d["k"][0, t, 0], d["v"][0, t, 0], d["q"][0, t, 0]
            M = al * (np.eye(5) - be * np.outer(kk, kk))
            N = be * np.outer(vv, kk)
            S = S @ M + N
            np.testing.assert_allclose(y[0, t, 0], S @ qq, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(s[0, 0], S, rtol=1e-12, atol=1e-12)


def test_decay_only_accumulates_product_of_alphas():
    d = _rand(9, T=6)
    d["beta"][:] = 0.0
    d["q"] = _unit(d["q"])
    y, s = orc.scan(**d, fold_qk_l2norm=False, fold_q_scale=False)
    G = d["v"].shape[2] // d["q"].shape[2]
    cum = np.exp(np.cumsum(d["log_decay"], axis=1))  # [B,T,Hv]
    for b in range(2):
        for hv in range(4):
            np.testing.assert_allclose(s[b, hv], cum[b, -1, hv] * d["s0"][b, hv], rtol=1e-12)
            for t in range(6):
                ref = cum[b, t, hv] * d["s0"][b, hv] @ d["q"][b, t, hv // G]
                np.testing.assert_allclose(y[b, t, hv], ref, rtol=1e-12, atol=1e-14)


def test_associative_recall_with_orthonormal_keys():
    r = np.random.default_rng(10)
    D, T = 8, 6
    Qm, _ = np.linalg.qr(r.standard_normal((D, D)))
    keys = Qm[:, :T].T  # T orthonormal keys
    vals = r.standard_normal((T, D))
    y, s = orc.scan(keys[None, :, None], keys[None, :, None], vals[None, :, None],
                    np.zeros((1, T, 1)), np.ones((1, T, 1)), np.zeros((1, 1, D, D)),
                    fold_qk_l2norm=False, fold_q_scale=False)
    for j in range(T):
        np.testing.assert_allclose(s[0, 0] @ keys[j], vals[j], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(y[0, j, 0], vals[j], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- invariants
def test_time_chaining():
    d = _rand(11, T=7, gated=True)
    y, s = orc.scan(**d)
    a = {n: (x[:, :3] if n not in ("s0", "w") else x) for n, x in d.items()}
    b = {n: (x[:, 3:] if n not in ("s0", "w") else x) for n, x in d.items()}
    y1, s1 = orc.scan(**a)
    b["s0"] = s1
    y2, s2 = orc.scan(**b)
    np.testing.assert_array_equal(np.concatenate([y1, y2], axis=1), y)
    np.testing.assert_array_equal(s2, s)
    # T single steps chained equal the scan
    st = d["s0"]
    for t in range(7):
        one = {n: (x[:, t:t + 1] if n not in ("s0", "w") else x) for n, x in d.items()}
        one["s0"] = st
        yt, st = orc.step(**one)
        np.testing.assert_array_equal(yt[:, 0], y[:, t])
    np.testing.assert_array_equal(st, s)


def test_head_major_is_a_transpose():
    d = _rand(12, gated=True)
    y, s = orc.scan(**d)
    hm = dict(d)
    for n in ("q", "k", "v", "z"):
        hm[n] = d[n].transpose(0, 2, 1, 3)
    for n in ("log_decay", "beta"):
        hm[n] = d[n].transpose(0, 2, 1)
    yh, sh = orc.scan(**hm, head_major=True)
    np.testing.assert_array_equal(yh, y.transpose(0, 2, 1, 3))
    np.testing.assert_array_equal(sh, s)


def test_grouped_heads_equal_repeated_keys():
    d = _rand(13, Hk=2, Hv=6, gated=True)
    y, s = orc.scan(**d)
    rep = dict(d)
    rep["q"] = np.repeat(d["q"], 3, axis=2)
    rep["k"] = np.repeat(d["k"], 3, axis=2)
    yr, sr = orc.scan(**rep)
    np.testing.assert_array_equal(y, yr)
    np.testing.assert_array_equal(s, sr)


def test_function_preserving_permutations():
    """Permuting value lanes permutes y and the state rows; permuting key lanes
    leaves y unchanged and permutes the state columns (GDNPermutation page)."""
    d = _rand(14, gated=True)
    y, s = orc.scan(**d)
    r = np.random.default_rng(15)
    pv = r.permutation(d["v"].shape[3])
    pk = r.permutation(d["q"].shape[3])
    e = dict(d)
    e["v"], e["z"], e["w"] = d["v"][..., pv], d["z"][..., pv], d["w"][pv]
    e["s0"] = d["s0"][:, :, pv, :]
    ye, se = orc.scan(**e)
    np.testing.assert_allclose(ye, y[..., pv], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(se, s[:, :, pv, :], rtol=1e-12, atol=1e-13)
    f = dict(d)
    f["q"], f["k"] = d["q"][..., pk], d["k"][..., pk]
    f["s0"] = d["s0"][..., pk]
    yf, sf = orc.scan(**f)
    np.testing.assert_allclose(yf, y, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sf, s[..., pk], rtol=1e-12, atol=1e-13)


def test_fold_equals_prenormalised_inputs():
    """Folding the L2 norm and q scale equals feeding q/sqrt(|q|^2+eps)/sqrt(Dk) and
    k/sqrt(|k|^2+eps) with the folds off ("gated_delta" page, native_gdn_reject_reason)."""
    d = _rand(16)
    y, s = orc.scan(**d)
    e = dict(d)
    eps, Dk = 1e-6, d["q"].shape[-1]
    e["q"] = d["q"] / np.sqrt((d["q"] ** 2).sum(-1, keepdims=True) + eps) / math.sqrt(Dk)
    e["k"] = d["k"] / np.sqrt((d["k"] ** 2).sum(-1, keepdims=True) + eps)
    ye, se = orc.scan(**e, fold_qk_l2norm=False, fold_q_scale=False)
    np.testing.assert_allclose(ye, y, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(se, s, rtol=1e-12, atol=1e-13)


def test_zero_length_and_zero_vectors():
    d = _rand(17, T=0)
    y, s = orc.scan(**d)
    assert y.shape[1] == 0
    np.testing.assert_array_equal(s, d["s0"])
    # zero q and k normalise to zero: u = w = k.q = 0, so S = alpha*S + beta*v*0 and o = 0
    d = _rand(18, T=1)
    d["q"][:] = 0.0
    d["k"][:] = 0.0
    y, s = orc.scan(**d)
    np.testing.assert_array_equal(y, 0.0)
    np.testing.assert_allclose(s, np.exp(d["log_decay"][:, 0, :, None, None]) * d["s0"], rtol=1e-15)


# ---------------------------------------------------------------- l2 norm and gated norm
def test_l2norm_closed_form():
    for c, n in ((0.5, 4), (-3.0, 16), (1e-4, 128)):
        x = np.full((n,), c)
        np.testing.assert_allclose(orc.l2norm(x), c / math.sqrt(n * c * c + 1e-6), rtol=1e-14)
    np.testing.assert_array_equal(orc.l2norm(np.zeros(5)), 0.0)


def test_l2norm_matches_hf_routine():
    hf = pytest.importorskip("transformers.models.qwen3_next.modeling_qwen3_next")
    import torch
    x = np.random.default_rng(19).standard_normal((6, 32))
    ref = hf.l2norm(torch.from_numpy(x), dim=-1, eps=1e-6).numpy()
    np.testing.assert_allclose(orc.l2norm(x), ref, rtol=1e-13, atol=1e-15)


def test_gated_norm_closed_forms():
    n = 8
    w = 1 + 0.1 * np.random.default_rng(20).standard_normal(n)
    o = np.random.default_rng(21).standard_normal(n)
    # z = 0 kills the gate: y = 0
    np.testing.assert_array_equal(orc.gated_rmsnorm(o, np.zeros(n), w), 0.0)
    # constant gated input x = c: y = c / sqrt(c^2 + eps) * w
    zc = 1.3
    silu = zc / (1 + math.exp(-zc))
    for c in (0.7, -2.0):
        x = c * silu
        y = orc.gated_rmsnorm(np.full(n, c), np.full(n, zc), w)
        np.testing.assert_allclose(y, x / math.sqrt(x * x + 1e-6) * w, rtol=1e-14)
    # scale invariance of the normalisation (eps aside)
    z = np.random.default_rng(22).standard_normal(n)
    np.testing.assert_allclose(orc.gated_rmsnorm(1000 * o, z, w, eps=0.0),
                               orc.gated_rmsnorm(o, z, w, eps=0.0), rtol=1e-13)


def test_gate_first_is_distinguished_from_norm_first():
    """The page multiplies the gate in before normalising.  With o = [1, 1] and z = [0, 10]:
    gate-first gives y = [0, sqrt(2)*x/sqrt(x^2 + 2eps)]*w with x = silu(10), while
    normalising first would give [0, x/sqrt(1 + eps)]*w."""
    w = np.array([1.0, 2.0])
    x = 10 / (1 + math.exp(-10))
    y = orc.gated_rmsnorm(np.ones(2), np.array([0.0, 10.0]), w)
    want = np.array([0.0, x / math.sqrt(x * x / 2 + 1e-6) * 2.0])
    np.testing.assert_allclose(y, want, rtol=1e-14)
    assert abs(y[1] - x / math.sqrt(1 + 1e-6) * 2.0) > 1.0


def test_gated_output_uses_gate_first_norm():
    d = _rand(23, gated=True)
    y, _ = orc.scan(**d)
    d2 = {n: x for n, x in d.items() if n not in ("z", "w")}
    o, _ = orc.scan(**d2)
    x = o * d["z"] / (1 + np.exp(-d["z"]))
    ref = x / np.sqrt((x * x).mean(-1, keepdims=True) + 1e-6) * d["w"]
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- library routine
def test_matches_hf_recurrent_rule():
    """Installed HF torch_recurrent_gated_delta_rule (named on the "gated_delta" page as
    the reference the pure-torch recurrence matches) with the in-kernel q/k L2 norm: same
    recurrence, state stored transposed ([B,H,Dk,Dv]), float32 inside."""
    hf = pytest.importorskip("transformers.models.qwen3_next.modeling_qwen3_next")
    import torch
    d = _rand(24, B=2, T=9, Hk=3, Hv=3, Dk=16, Dv=16)
    y, s = orc.scan(**d)
    t = {n: torch.from_numpy(x) for n, x in d.items()}
    out, fin = hf.torch_recurrent_gated_delta_rule(
        t["q"], t["k"], t["v"], t["log_decay"], t["beta"],
        initial_state=t["s0"].transpose(-1, -2).contiguous(), output_final_state=True,
        use_qk_l2norm_in_kernel=True)
    np.testing.assert_allclose(out.double().numpy(), y, rtol=0, atol=2e-5)
    np.testing.assert_allclose(fin.double().transpose(-1, -2).numpy(), s, rtol=0, atol=2e-5)


# ---------------------------------------------------------------- gate producer
def test_gate_producer_closed_forms():
    """softplus(0) = ln 2, sigmoid(0) = 1/2; softplus(x) -> x and -> e^x in the tails;
    sigmoid(-x) = 1 - sigmoid(x); the scale multiplies log_decay only."""
    a = np.array([0.0, 40.0, -40.0, 1.0])
    b = np.array([0.0, 3.0, -3.0, 50.0])
    ld, be = orc.gates(a, b, decay_scale=0.5)
    np.testing.assert_allclose(ld[0], -0.5 * math.log(2.0), rtol=1e-15)
    np.testing.assert_allclose(ld[1], -0.5 * 40.0, rtol=1e-15)
    np.testing.assert_allclose(ld[2], -0.5 * math.exp(-40.0), rtol=1e-12)
    np.testing.assert_allclose(ld[3], -0.5 * math.log1p(math.e), rtol=1e-15)
    np.testing.assert_allclose(be[0], 0.5, rtol=0)
    np.testing.assert_allclose(be[1] + be[2], 1.0, rtol=1e-15)
    np.testing.assert_allclose(be[3], 1.0, rtol=1e-15)


def test_gate_producer_matches_library_routines():
    r = np.random.default_rng(30)
    a, b = r.standard_normal(1000) * 5, r.standard_normal(1000) * 5
    ld, be = orc.gates(a, b, decay_scale=0.01)
    np.testing.assert_allclose(ld, -0.01 * np.logaddexp(0.0, a), rtol=1e-14)
    from scipy.special import expit
    np.testing.assert_allclose(be, expit(b), rtol=1e-14)


# ---------------------------------------------------------------- conv + silu producer
def _conv_operands(seed, B=2, T=9, C=5, W=4, state=True, bias=True):
    r = np.random.default_rng(seed)
    x = r.standard_normal((B, T, C))
    w = r.standard_normal((C, W))
    b = r.standard_normal(C) if bias else None
    s = r.standard_normal((B, C, W - 1)) if state else None
    return x, w, b, s


@pytest.mark.parametrize("W", [1, 2, 4, 6])
def test_conv_linear_part_matches_numpy_correlate(W):
    """Without the silu, each channel is a cross-correlation of its carried
    context followed by its inputs with the channel's taps (numpy.correlate,
    'valid' mode), plus the bias."""
    x, w, b, s = _conv_operands(40 + W, W=W)
    pre, _ = orc.conv_silu(x, w, b, s, apply_silu=False)
    B, T, C = x.shape
    for bb in range(B):
        for c in range(C):
            xx = np.concatenate([s[bb, c], x[bb, :, c]])
            ref = np.correlate(xx, w[c], mode="valid") + b[c]
            np.testing.assert_allclose(pre[bb, :, c], ref, rtol=1e-13, atol=1e-13)


def test_conv_silu_is_pre_times_sigmoid():
    from scipy.special import expit
    x, w, b, s = _conv_operands(50, T=12, C=7)
    pre, _ = orc.conv_silu(x, w, b, s, apply_silu=False)
    y, _ = orc.conv_silu(x, w, b, s)
    np.testing.assert_allclose(y, pre * expit(pre), rtol=1e-13, atol=1e-15)


def test_conv_impulse_response():
    """A unit impulse at (t0, c0) with no bias and no context gives
    silu(w[c0, W-1-i]) at t0 + i for i < W, and exactly zero elsewhere."""
    B, T, C, W = 1, 11, 3, 4
    w = np.random.default_rng(51).standard_normal((C, W))
    x = np.zeros((B, T, C))
    x[0, 4, 1] = 1.0
    y, st = orc.conv_silu(x, w)
    silu = lambda v: v / (1.0 + math.exp(-v))  # noqa: E731
    expect = np.zeros((B, T, C))
    for i in range(W):
        expect[0, 4 + i, 1] = silu(w[1, W - 1 - i])
    np.testing.assert_allclose(y, expect, rtol=1e-15, atol=0)
    assert np.all(st == 0.0)


def test_conv_width_one_is_elementwise():
    x, w, b, _ = _conv_operands(52, W=1, state=False)
    y, st = orc.conv_silu(x, w, b)
    pre = x * w[:, 0] + b
    np.testing.assert_allclose(y, pre / (1.0 + np.exp(-pre)), rtol=1e-14)
    assert st.shape == (x.shape[0], x.shape[2], 0)


def test_conv_time_chaining_through_the_state():
    """Splitting the time axis and carrying the last W-1 inputs as the state
    reproduces the whole sequence exactly; with fewer than W-1 new tokens the
    state is a shift register over the old state and the new inputs."""
    x, w, b, s = _conv_operands(53, T=10, C=6, W=4)
    y, st = orc.conv_silu(x, w, b, s)
    for T1 in (1, 2, 3, 7):
        y1, s1 = orc.conv_silu(x[:, :T1], w, b, s)
        y2, s2 = orc.conv_silu(x[:, T1:], w, b, s1)
        assert np.array_equal(np.concatenate([y1, y2], axis=1), y)
        assert np.array_equal(s2, st)
    # state after two tokens: the last old entry, then the two inputs
    _, s2 = orc.conv_silu(x[:, :2], w, b, s)
    np.testing.assert_array_equal(s2[:, :, 0], s[:, :, 2])
    np.testing.assert_array_equal(s2[:, :, 1:], x[:, :2].transpose(0, 2, 1))
    # no context is the same as a zero context; T = 0 returns the context
    y0, _ = orc.conv_silu(x, w, b, np.zeros_like(s))
    yn, _ = orc.conv_silu(x, w, b, None)
    assert np.array_equal(y0, yn)
    ye, se = orc.conv_silu(x[:, :0], w, b, s)
    assert ye.shape == (2, 0, 6) and np.array_equal(se, s)
