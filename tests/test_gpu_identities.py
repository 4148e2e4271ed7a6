"""The recurrence's own identities on the GPU block form, through the C ABI.

The update S = alpha*S + beta*(v - alpha*S.k^) k^T of the "Module gdn" page
(module description) fixes, for special gates and keys, results that need no
oracle:
  - alpha = 1, beta = 0 leaves S unchanged, and o_t = S_0 . q^_t;
  - alpha = 0 at one token restarts the memory at S = beta v k^T, whatever came
    before (here a token in the middle of a 16-token block);
  - alpha = beta = 1 with orthonormal keys from S_0 = 0 stores every pair:
    S_T . k^_j = v_j (associative recall), and a query equal to a stored key
    reads its value back;
  - beta = 1 and a unit key overwrite: S_new . k^ = v for any alpha, so a key
    repeated on consecutive tokens of one block keeps only the latest value.
Each case runs at head dim 128 on both block-form kernels (fewer than 256
value heads: the kernel with a workgroup per 16 state rows; 256 and more: a
workgroup per head) in both layouts and all three operand dtypes, at head dims
32 and 64 with float32 and bfloat16 operands, and at 256 with all three (where
both head counts take the kernel with a workgroup per 16 rows);
each is also compared with the float64 oracle at the usual bar.  The closed
forms are evaluated in float64 from the exact operand values.
"""
import sys

import numpy as np
import pytest
import scipy.linalg
import torch

from linear_attention_recurrence_recurrent_amd import scan, synth
from oracle import gdn_oracle as orc

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"f32": 1e-4, "f16": 3e-3, "bf16": 3e-3}
CLOSED = 1e-4  # closed forms: f32 arithmetic on exact inputs
SHAPES = {"few_heads": (1, 2, 4), "many_heads": (8, 16, 32)}  # (B, Hk, Hv)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _unit(x):
    """k^ as the op forms it (L2 norm with eps 1e-6 inside the root), float64."""
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + 1e-6)


def _cast(a, dt):
    return synth._cast(np.asarray(a, dtype=np.float64), dt).double().numpy()


def _ops(B, T, Hk, Hv, dt, seed, D):
    """Random operands, token-major, float64 arrays holding values exact in dt."""
    r = np.random.default_rng(seed)
    ops = dict(q=_cast(r.standard_normal((B, T, Hk, D)), dt),
               k=_cast(r.standard_normal((B, T, Hk, D)), dt),
               v=_cast(r.standard_normal((B, T, Hv, D)), dt),
               z=_cast(r.standard_normal((B, T, Hv, D)), dt),
               log_decay=_cast(-np.logaddexp(0.0, r.standard_normal((B, T, Hv))), dt),
               beta=_cast(1.0 / (1.0 + np.exp(-r.standard_normal((B, T, Hv)))), dt),
               s0=_cast(0.02 * r.standard_normal((B, Hv, D, D)), "f32"),
               w=_cast(1.0 + 0.1 * r.standard_normal(D), dt))
    return ops


def _run(ops, dt, head_major, gated, exact=False):
    """GPU scan (the default form, which is the block form at these head dims) and the
    oracle on the same values."""
    tdt = synth.DTYPES[dt]

    def dev(name):
        a = ops[name]
        if head_major and name in ("q", "k", "v", "z"):
            a = a.transpose(0, 2, 1, 3)
        elif head_major and name in ("log_decay", "beta"):
            a = a.transpose(0, 2, 1)
        t = torch.from_numpy(np.ascontiguousarray(a))
        return t.to(torch.float32 if name == "s0" else tdt).to(DEV)

    d = {n: dev(n) for n in ops}
    y, s = scan(d["q"], d["k"], d["v"], d["log_decay"], d["beta"], d["s0"],
                d["z"] if gated else None, d["w"] if gated else None, head_major=head_major,
                exact=exact)
    torch.cuda.synchronize()
    y = y.double().cpu().numpy()
    if head_major:
        y = y.transpose(0, 2, 1, 3)
    s = s.double().cpu().numpy()
    yr, sr = orc.scan(ops["q"], ops["k"], ops["v"], ops["log_decay"], ops["beta"], ops["s0"],
                      ops["z"] if gated else None, ops["w"] if gated else None)
    _close(y, yr, TOL[dt], "y vs oracle")
    _close(s, sr, TOL[dt], "state vs oracle")
    return y, s


def _close(got, ref, tol, what):
    err = np.abs(got - ref) / (1.0 + np.abs(ref))
    assert np.all(np.isfinite(got)), what + ": non-finite"
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, "%s: max rel err %.3e > %.1e at %s" % (
        what, worst, tol, np.unravel_index(int(err.argmax()), err.shape))


CASES = ([(kind, dt, hm, 128) for kind in SHAPES for dt in ("f32", "bf16", "f16")
          for hm in (False, True)]
         + [(kind, dt, False, d) for d in (32, 64) for kind in SHAPES for dt in ("f32", "bf16")]
         + [(kind, dt, False, 256) for kind in SHAPES for dt in ("f32", "bf16", "f16")])
IDS = ["%s-%s-%s-d%d" % (c[0], c[1], "hm" if c[2] else "tm", c[3]) for c in CASES]


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_decay_one_beta_zero_leaves_state(case):
    kind, dt, hm, D = case
    B, Hk, Hv = SHAPES[kind]
    T = 45  # two full blocks and a ragged one
    say("identity alpha=1 beta=0 %s" % (case,))
    ops = _ops(B, T, Hk, Hv, dt, seed=1, D=D)
    ops["log_decay"][:] = 0.0
    ops["beta"][:] = 0.0
    y, s = _run(ops, dt, hm, gated=False)
    _close(s, ops["s0"], 1e-6, "state unchanged")
    G = Hv // Hk
    qh = _unit(np.repeat(ops["q"], G, axis=2)) / np.sqrt(D)        # [B, T, Hv, D]
    o = np.einsum("bhac,bthc->btha", ops["s0"], qh)
    _close(y, o, CLOSED, "o = S0 q^")


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_zero_decay_mid_block_restarts_memory(case):
    kind, dt, hm, D = case
    B, Hk, Hv = SHAPES[kind]
    say("identity alpha=0 mid-block %s" % (case,))
    G = Hv // Hk
    for j in (5, 23):  # row 5 of block 0, row 7 of block 1
        ops = _ops(B, j + 1, Hk, Hv, dt, seed=2 + j, D=D)
        ops["log_decay"][:, j] = -np.inf
        y, s = _run(ops, dt, hm, gated=False)
        kh = _unit(np.repeat(ops["k"][:, j], G, axis=1))          # [B, Hv, D]
        qh = _unit(np.repeat(ops["q"][:, j], G, axis=1)) / np.sqrt(D)
        be = ops["beta"][:, j][..., None]                          # [B, Hv, 1]
        want = be[..., None] * ops["v"][:, j][..., :, None] * kh[..., None, :]
        _close(s, want, CLOSED, "S = beta v k^T after alpha = 0 (token %d)" % j)
        o = be * ops["v"][:, j] * (kh * qh).sum(-1, keepdims=True)
        _close(y[:, j], o, CLOSED, "o = beta v (k^.q^) at the restart")
    # the restart in the middle of a longer scan, gated, against the oracle only
    ops = _ops(B, 70, Hk, Hv, dt, seed=9, D=D)
    ops["log_decay"][:, 37] = -np.inf
    _run(ops, dt, hm, gated=True)


def _hadamard_keys(B, T, Hk, seed, D):
    """Rows of a D x D +-1 Hadamard matrix with random signs, a random subset
    per (batch, key head): exactly orthogonal, exact in every dtype."""
    r = np.random.default_rng(seed)
    H = scipy.linalg.hadamard(D).astype(np.float64)
    k = np.empty((B, T, Hk, D))
    for b in range(B):
        for h in range(Hk):
            rows = r.permutation(D)[:T]
            k[b, :, h] = H[rows] * r.choice([-1.0, 1.0], size=(T, 1))
    return k


# f32 operands take f32 products in both modes, so only 16-bit cases run exact
RECALL = [(c, False) for c in CASES] + [(c, True) for c in CASES if c[1] != "f32"]


RECALL_IDS = ["%s-%s-%s-d%d-%s" % (c[0], c[1], "hm" if c[2] else "tm", c[3],
                                   "exact" if e else "default") for c, e in RECALL]
# at most D orthonormal keys: a whole number of blocks and a ragged count per head dim
RECALL_T = {32: (32, 27), 64: (64, 50), 128: (128, 100), 256: (128, 100)}


@pytest.mark.parametrize("case,exact", RECALL, ids=RECALL_IDS)
@pytest.mark.parametrize("which", [0, 1], ids=["whole-blocks", "ragged"])
def test_associative_recall_orthonormal_keys(case, exact, which):
    kind, dt, hm, D = case
    T = RECALL_T[D][which]
    B, Hk, Hv = SHAPES[kind]
    say("identity associative recall T=%d %s" % (T, case))
    G = Hv // Hk
    r = np.random.default_rng(T)
    ops = _ops(B, T, Hk, Hv, dt, seed=3, D=D)
    ops["k"] = _hadamard_keys(B, T, Hk, seed=4, D=D)
    ops["s0"][:] = 0.0
    ops["log_decay"][:] = 0.0
    ops["beta"][:] = 1.0
    # each query repeats the key of an earlier (or the same) token
    src = np.array([r.integers(0, t + 1) for t in range(T)])
    ops["q"] = ops["k"][:, src].copy()
    y, s = _run(ops, dt, hm, gated=False, exact=exact)
    kh = _unit(np.repeat(ops["k"], G, axis=2))                     # [B, T, Hv, D]
    recall = np.einsum("bhac,bthc->btha", s, kh)
    _close(recall, ops["v"], CLOSED, "S_T k^_j = v_j")
    want = ops["v"][:, src] * (kh[:, src] * kh[:, src]).sum(-1, keepdims=True) / np.sqrt(D)
    _close(y, want, CLOSED, "o_t reads back the value of its key")


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_repeated_key_in_block_keeps_latest_value(case):
    kind, dt, hm, D = case
    B, Hk, Hv = SHAPES[kind]
    say("identity repeated key %s" % (case,))
    G = Hv // Hk
    T = 26  # the run covers rows 3..9 of block 1 (tokens 19..25)
    ops = _ops(B, T, Hk, Hv, dt, seed=5, D=D)
    run = slice(19, 26)
    ops["k"][:, run] = ops["k"][:, 19:20]
    ops["q"][:, run] = ops["k"][:, 19:20]
    ops["beta"][:, run] = 1.0
    y, s = _run(ops, dt, hm, gated=False)
    kh = _unit(np.repeat(ops["k"][:, 19], G, axis=1))              # [B, Hv, D]
    _close(np.einsum("bhac,bhc->bha", s, kh), ops["v"][:, 25], CLOSED, "S k^ = latest v")
    # every token of the run reads its own value back through q = k
    scale = (kh * kh).sum(-1, keepdims=True) / np.sqrt(D)
    for t in range(19, 26):
        _close(y[:, t], ops["v"][:, t] * scale, CLOSED, "o at token %d" % t)
