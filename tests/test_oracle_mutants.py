"""Plant plausible mistakes in a copy of the oracle and check the pins catch each one.

The mutants are built on the CPU from the oracle's source text; the real
oracle is never modified.  Each mutation must apply exactly once, so a change
to the oracle's text that silently disables a mutant fails this test too.
"""
import inspect
import types

import pytest

import oracle.recurrence as rec
import pins

MUTATIONS = {
    "phi_drops_plus_one": ("x + 1.0, np.exp", "x, np.exp"),
    "phi_wrong_branch": ("np.where(x > 0", "np.where(x < 0"),
    "phi_exp_of_raw_x_times_two": ("np.exp(np.minimum(x, 0.0))", "np.exp(2 * np.minimum(x, 0.0))"),
    "eps_added_not_clamped": ("np.maximum(den, eps)", "(den + eps)"),
    "no_eps_guard": ("np.maximum(den, eps)", "den"),
    "read_before_update": ("        S = S + fk[..., :, None] * v[..., t, None, :]\n        z = z + fk\n"
                           "        num = np.einsum(\"...d,...de->...e\", fq, S)\n"
                           "        den = np.einsum(\"...d,...d->...\", fq, z)\n",
                           "        num = np.einsum(\"...d,...de->...e\", fq, S)\n"
                           "        den = np.einsum(\"...d,...d->...\", fq, z)\n"
                           "        S = S + fk[..., :, None] * v[..., t, None, :]\n        z = z + fk\n"),
    "state_transposed": ("np.einsum(\"...d,...de->...e\", fq, S)", "np.einsum(\"...e,...de->...d\", fq, S)"),
    "key_query_swapped": ("fq = fmap(q[..., t, :])\n        fk = fmap(k[..., t, :])",
                          "fq = fmap(k[..., t, :])\n        fk = fmap(q[..., t, :])"),
    "z_not_updated": ("        z = z + fk\n", "        z = z\n"),
    "z_not_gated": ("            z = gt[..., None] * z\n", "            z = z\n"),
    "gate_after_update": ("            S = gt[..., None, None] * S\n", "            S = S\n"),
    "phi_on_values": ("S = S + fk[..., :, None] * v[..., t, None, :]",
                      "S = S + fk[..., :, None] * phi(v[..., t, None, :])"),
    "initial_state_ignored": ("S = np.array(s0, dtype=np.float64, copy=True)", "S = np.zeros(lead + (d, dv))"),
    "value_index_lag": ("v[..., t, None, :]", "v[..., max(t - 1, 0), None, :]"),
    "gate_index_lag": ("gt = g[..., t]", "gt = g[..., max(t - 1, 0)]"),
    "numerator_mode_still_divides": ("if normalize else num", "if normalize or True else num"),
    "numerator_mode_divides_by_raw_den": ("if normalize else num", "if normalize else num / den[..., None]"),
    "decode_drops_output_mode": ("eps=eps, normalize=normalize, a=aa,", "eps=eps, a=aa,"),
    "vector_decay_on_value_dim": ("S = at[..., :, None] * S", "S = at[..., :1, None] * S"),
    "vector_decay_skips_z": ("            z = at * z\n", "            z = z\n"),
    "vector_decay_index_lag": ("at = a[..., t, :]", "at = a[..., max(t - 1, 0), :]"),
    "relu_shift_dropped": ("return np.maximum(x, 0.0) + shift", "return np.maximum(x, 0.0) + 0.0"),
    "favor_no_norm_term": ("np.exp(proj - 0.5 * np.sum(x * x, axis=-1, keepdims=True))", "np.exp(proj)"),
    "favor_no_sqrt_m": ("/ np.sqrt(W.shape[-2])", "/ 1.0"),
}


def _mutant(name):
    old, new = MUTATIONS[name]
    src = inspect.getsource(rec)
    assert src.count(old) == 1, f"mutation {name} does not apply exactly once"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    mod.__dict__["__name__"] = mod.__name__
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


def test_unmutated_copy_passes_every_pin():
    src = inspect.getsource(rec)
    mod = types.ModuleType("oracle_copy")
    exec(compile(src, "<copy>", "exec"), mod.__dict__)
    for pin in pins.ALL_PINS:
        pin(mod)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutant_is_caught(name):
    mod = _mutant(name)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(mod)
        except Exception:                                  # noqa: BLE001 - any failure counts
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
