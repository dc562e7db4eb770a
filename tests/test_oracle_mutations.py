"""CPU tests: a plausible mistake planted anywhere in the oracle fails at least one pin.

Each case copies the source of oracle/ref.py (or oracle/online.py), applies one textual
mutation, loads the copy as a fresh module and runs every pin against it.  Nothing here
touches a GPU.
"""

import os
import types

import pytest

import oracle
from tests.oracle_pins import failing_pins

ORACLE_DIR = os.path.dirname(os.path.abspath(oracle.__file__))

REF_MUTATIONS = {
    "causal_off_by_one": ("keys[None, :] <= rows[:, None]", "keys[None, :] < rows[:, None]"),
    "padding_off_by_one": ("keys[None, :] < int(kv_len_b)", "keys[None, :] <= int(kv_len_b)"),
    "lse_base2": ("m + np.log(safe_l)", "m + np.log2(safe_l)"),
    "lse_without_max": ("m + np.log(safe_l)", "np.log(safe_l)"),
    "unnormalised_p": ("p = e / safe_l[:, None]", "p = e"),
    "scores_transposed": ("s = scale * (q[rows] @ k.T)\n    ok", "s = scale * (k[rows] @ q.T)\n    ok"),
    "scale_dropped_in_scores": ("s = scale * (q[rows] @ k.T)\n    ok", "s = (q[rows] @ k.T)\n    ok"),
    "ds_sign_flipped": ("ds = p * (dp - dsum[:, None])\n        dq", "ds = p * (dsum[:, None] - dp)\n        dq"),
    "ds_dropped_d_term": ("ds = p * (dp - dsum[:, None])\n        dq", "ds = p * dp\n        dq"),
    "dsum_wrong_axis": ("dsum = (p * dp).sum(axis=1)\n        ds", "dsum = (p * dp).sum(axis=0)\n        ds"),
    "dq_missing_scale": ("dq[rows] = scale * (ds @ k)", "dq[rows] = (ds @ k)"),
    "dk_wrong_operand": ("dk += scale * (ds.T @ q[rows])", "dk += scale * (ds.T @ k[rows])"),
    "dv_p_not_transposed": ("dv += p.T @ dor", "dv += p @ dor"),
    "dp_uses_k": ("dp = dor @ v.T", "dp = dor @ k.T"),
    "dk_chunk_overwrites": ("dk += scale * (ds.T @ q[rows])", "dk = scale * (ds.T @ q[rows])"),
    "dv_chunk_overwrites": ("dv += p.T @ dor", "dv = p.T @ dor"),
    "chunk_rows_not_offset": ("rows = np.arange(r0, min(N, r0 + _ROW_CHUNK))",
                              "rows = np.arange(0, min(N, _ROW_CHUNK))"),
    "chunk_last_rows_dropped": ("rows = np.arange(r0, min(n, r0 + _ROW_CHUNK))",
                                "rows = np.arange(r0, min(n - 1, r0 + _ROW_CHUNK))"),
    "cols_dv_p_not_transposed": ("dv += p_c.T @ dor", "dv += p_c @ dor"),
    "cols_d_over_selected_keys_only": ("dsum = (p * dp).sum(axis=1)\n        p_c",
                                       "dsum = (p[:, cols] * dp[:, cols]).sum(axis=1)\n        p_c"),
    "cols_dk_chunk_overwrites": ("dk += scale * (ds_c.T @ q[rows])", "dk = scale * (ds_c.T @ q[rows])"),
    "cols_dk_missing_scale": ("dk += scale * (ds_c.T @ q[rows])", "dk += (ds_c.T @ q[rows])"),
    "gqa_interleaved_heads": ("return attention_forward(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)",
                              "return attention_forward(q, np.tile(k, (1, G, 1, 1)), np.tile(v, (1, G, 1, 1))"),
    "gqa_dk_not_summed": ("return dq, dk.reshape(B, Hkv, G, N, d).sum(axis=2)",
                          "return dq, dk.reshape(B, Hkv, G, N, d)[:, :, 0]"),
    "gqa_dv_mean": ("dv.reshape(B, Hkv, G, N, d).sum(axis=2)", "dv.reshape(B, Hkv, G, N, d).mean(axis=2)"),
    "gqa_dk_summed_over_wrong_axis": ("dk.reshape(B, Hkv, G, N, d).sum(axis=2)",
                                      "dk.reshape(B, G, Hkv, N, d).sum(axis=1)"),
}

ONLINE_MUTATIONS = {
    "no_rescale_of_sum": ("l = alpha * l + p.sum(axis=1)", "l = l + p.sum(axis=1)"),
    "no_rescale_of_acc": ("acc = alpha[:, None] * acc + p @ v[keys]", "acc = acc + p @ v[keys]"),
    "rescale_sign": ("np.exp(m - np.where(np.isfinite(new_m), new_m, 0.0))", "np.exp(np.where(np.isfinite(new_m), new_m, 0.0) - m)"),
}


def _load(name, old, new):
    path = os.path.join(ORACLE_DIR, name + ".py")
    with open(path) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor not found in {name}.py: {old!r}"
    mod = types.ModuleType(f"oracle_{name}_mutant")
    exec(compile(src.replace(old, new), path, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("case", sorted(REF_MUTATIONS))
def test_ref_mutation_is_caught(case):
    old, new = REF_MUTATIONS[case]
    mutant = _load("ref", old, new)
    assert failing_pins(mutant, oracle.online), f"no pin caught mutation {case}"


@pytest.mark.parametrize("case", sorted(ONLINE_MUTATIONS))
def test_online_mutation_is_caught(case):
    old, new = ONLINE_MUTATIONS[case]
    mutant = _load("online", old, new)
    assert failing_pins(oracle.ref, mutant), f"no pin caught mutation {case}"
