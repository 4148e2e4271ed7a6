"""Properties of the C ABI's validation over random descriptors (hypothesis;
on the CPU, no device work: the addresses below are never dereferenced).

For every drawn descriptor:
  - the status is a documented gdn_status, and a refusal leaves a reason;
  - gdn_scan_workspace_size and gdn_check agree on whether the shape is
    accepted;
  - an accepted shape's workspace is exactly what include/gdn.h states: 2560
    bytes per (value head, 16-token block), plus 3072 per (key head, block)
    when the few-head kernel runs (fewer than 256 value heads, or D = 256),
    and nothing when the block form is not used (D = 16, the token-by-token
    flag, one token, an empty batch, or offsets past the block form's bounds);
  - gdn_check accepts disjoint aligned buffers with that workspace, and when a
    workspace is needed refuses one byte less (GDN_EWORKSPACE) and no
    workspace at all;
  - the status follows the rules it depends on alone, in the order they are
    checked: Hv not a multiple of Hk is GDN_EGROUP, then both form flags
    GDN_EINVAL, then a head dim outside {16, 32, 64, 128, 256} or Dk != Dv
    GDN_EUNSUPPORTED.
"""
import ctypes

from hypothesis import given, settings, strategies as st

from linear_attention_recurrence_recurrent_amd import _native as nat
from linear_attention_recurrence_recurrent_amd import GdnDesc, check

STATUSES = set(range(10))
GAP = 1 << 40  # between fake buffers: more than any drawn operand's bytes
BASE = 1 << 44

descs = st.fixed_dictionaries(dict(
    B=st.integers(0, 48), T=st.integers(0, 3000), Hk=st.integers(1, 24),
    G=st.sampled_from([1, 1, 2, 3, 4, 8]),
    Dk=st.sampled_from([16, 32, 64, 128, 256, 256, 96]),
    same_dv=st.sampled_from([True, True, True, False]),
    head_major=st.integers(0, 1), dtype=st.integers(0, 2), gate_dtype=st.integers(0, 2),
    fold=st.integers(0, 3), form=st.sampled_from([0, 0, 4, 8, 12]),
    exact=st.booleans(), ungrouped=st.integers(0, 9)))


def _desc(p):
    Hv = p["Hk"] * p["G"] + (1 if p["ungrouped"] == 0 and p["Hk"] > 1 else 0)
    Dv = p["Dk"] if p["same_dv"] or p["Dk"] == 96 else 64
    flags = p["fold"] | p["form"] | (16 if p["exact"] else 0)
    return GdnDesc(B=p["B"], T=p["T"], Hk=p["Hk"], Hv=Hv, Dk=p["Dk"], Dv=Dv,
                   head_major=p["head_major"], dtype=p["dtype"], gate_dtype=p["gate_dtype"],
                   flags=flags, qk_eps=1e-6, norm_eps=1e-6)


def _expected_workspace(d):
    D = d.Dk
    if d.Dv != D or D not in (32, 64, 128, 256) or d.Hk * D >= 1 << 27 or d.Hv * D >= 1 << 27:
        return 0
    if d.T >= 1 << 29 or d.flags & 4 or d.T < 2 or d.B == 0:
        return 0
    nblk = (d.T + 15) // 16
    ws = d.B * d.Hv * nblk * 2560
    if d.B * d.Hv < 256 or D > 128:
        ws += d.B * d.Hk * nblk * 3072
    return ws


def _ws(d):
    n = ctypes.c_uint64(0)
    rc = nat.lib().gdn_scan_workspace_size(ctypes.byref(d), ctypes.byref(n))
    return rc, n.value


def _buffers(z=True):
    names = ("q", "k", "v", "log_decay", "beta", "s0", "z", "w", "y", "s_out")
    ops = {n: BASE + i * GAP for i, n in enumerate(names)}
    if not z:
        ops["z"] = ops["w"] = None
    return ops, BASE + len(names) * GAP


@settings(max_examples=400, deadline=None)
@given(descs, st.booleans())
def test_validation_properties(p, gated):
    d = _desc(p)
    rc, ws = _ws(d)
    assert rc in STATUSES
    if rc:
        assert nat.last_error(), "a refusal without a reason"
    # rules that decide the status on their own
    if d.Hv % d.Hk:
        assert rc == 4
    elif (d.flags & 12) == 12:
        assert rc == 1
    elif d.Dk not in (16, 32, 64, 128, 256) or d.Dk != d.Dv:
        assert rc == 5
    ops, ws_addr = _buffers(gated)
    if rc:
        assert check(d, **ops, workspace=ws_addr, workspace_bytes=1 << 40)[0] == rc
        return
    assert ws == _expected_workspace(d), (d.B, d.T, d.Hk, d.Hv, d.Dk, d.flags, ws)
    if ws:
        assert check(d, **ops, workspace=ws_addr, workspace_bytes=ws)[0] == 0
        assert check(d, **ops, workspace=ws_addr, workspace_bytes=ws - 1)[0] == 9
        assert check(d, **ops)[0] == 9
    else:
        assert check(d, **ops)[0] == 0
