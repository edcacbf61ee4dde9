"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins in test_oracle.py catch every one of them."""
import importlib.util
import os
import types

import pytest

import tests.test_oracle as pins
from oracle import attention as orc

SRC = open(orc.__file__).read()

MUTATIONS = {
    "top_left_causal": ("vis = j[None, :] <= i[:, None] + (lk - lq)", "vis = j[None, :] <= i[:, None]"),
    "gqa_modulo_map": ("o, l = attend(q[qa:qb, h], k[ka:kb, g]", "o, l = attend(q[qa:qb, h], k[ka:kb, h % Hkv]"),
    "dense_gqa_modulo": ("o, l = attend(q[b, h], k[b, h // G], v[b, h // G]", "o, l = attend(q[b, h], k[b, h % Hkv], v[b, h % Hkv]"),
    "scale_dropped_fwd": ("        s = scale * (q[r0:r1] @ k.T)\n        s = capped(s, softcap)", "        s = (q[r0:r1] @ k.T)\n        s = capped(s, softcap)"),
    "lse_base2": ("mx + np.log(np.where(live, tot, 1.0))", "mx + np.log2(np.where(live, tot, 1.0))"),
    "delta_dropped": ("ds = p * (dp - delta[r0:r1, None])", "ds = p * dp"),
    "dk_scale_dropped": ("dk += scale * (ds.T @ q[r0:r1])", "dk += (ds.T @ q[r0:r1])"),
    "dq_transposed_operand": ("dq[r0:r1] = scale * (ds @ k)", "dq[r0:r1] = scale * (ds @ k[::-1])"),
    "dv_uses_dp": ("dv += p.T @ do[r0:r1]", "dv += (p * 0.5).T @ do[r0:r1]"),
    "merge_wrong_weight": ("wb = np.where(live, np.exp(lse_b - safe), 0.0)", "wb = np.where(live, np.exp(lse_a - safe), 0.0)"),
    "doc_ignores_pad": ("& (q_doc[:, None] > 0)", "& (q_doc[:, None] >= 0)"),
    "doc_fwd_gqa_modulo": ("o, l = attend(q[:, h], k[:, h // G], v[:, h // G], vis, scale)", "o, l = attend(q[:, h], k[:, h % k.shape[1]], v[:, h % k.shape[1]], vis, scale)"),
    "doc_bwd_gqa_modulo": ("a, b, c = attend_backward(do[:, h], q[:, h], k[:, h // G], v[:, h // G], o[:, h],", "a, b, c = attend_backward(do[:, h], q[:, h], k[:, h % k.shape[1]], v[:, h % k.shape[1]], o[:, h],"),
    "doc_bwd_group_sum": ("        dk[:, h // G] += b\n", "        dk[:, h % k.shape[1]] += b\n"),
    "ring_gather_wrong_axes": ("return x.transpose(0, 2, 1, 3).reshape(B * S, H, D)[idx]", "return x.transpose(0, 1, 2, 3).reshape(B * S, H, D)[idx]"),
    "ring_merge_rows_keeps_old_out": ("    flat_o[idx] = mo\n", "    flat_o[idx] = flat_o[idx]\n"),
    "window_off_by_one": ("vis = vis & (j[None, :] > i[:, None] + (lk - lq) - window)", "vis = vis & (j[None, :] >= i[:, None] + (lk - lq) - window)"),
    "softcap_not_applied": ("    return softcap * np.tanh(s / softcap)", "    return s"),
    "softcap_grad_factor_dropped": ("            ds = ds * (1.0 - np.tanh(x / softcap) ** 2)", "            ds = ds * 1.0"),
    "doc_future_keys": ("(np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None])", "(np.asarray(k_pos)[None, :] >= 0)"),
}


def _mutant(old, new):
    assert SRC.count(old) == 1, old
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = orc.__file__
    exec(compile(SRC.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _pin_cases():
    for name in dir(pins):
        fn = getattr(pins, name)
        if not name.startswith("test_") or not callable(fn):
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not marks:
            yield name, fn, {}
            continue
        argnames, argvalues = marks[0].args[0], marks[0].args[1]
        names = [a.strip() for a in argnames.split(",")]
        for vals in argvalues:
            vals = vals if isinstance(vals, tuple) else (vals,)
            yield name, fn, dict(zip(names, vals))


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_mistake_is_caught(mutation, monkeypatch):
    mutant = _mutant(*MUTATIONS[mutation])
    monkeypatch.setattr(pins, "orc", mutant)
    caught = []
    for name, fn, kw in _pin_cases():
        try:
            fn(**kw)
        except Exception:  # noqa: BLE001 - any failure counts as caught
            caught.append(name)
    assert caught, f"no pin caught mutation {mutation}"


def test_unmutated_copy_passes_every_pin(monkeypatch):
    """Control: the copy mechanism itself breaks nothing."""
    monkeypatch.setattr(pins, "orc", _mutant("NEG_INF = -np.inf", "NEG_INF = -np.inf"))
    for name, fn, kw in _pin_cases():
        fn(**kw)
