"""The backward oracle against its pins, and planted mistakes in copies of it (CPU only)."""
import inspect
import types

import pytest

import oracle.backward as bwd
import pins_bwd

MUTATIONS = {
    "dden_sign_flipped": ("-np.einsum(\"...e,...e->...\", do[..., t, :], num)", "np.einsum(\"...e,...e->...\", do[..., t, :], num)"),
    "dnum_not_divided": ("dnum = do[..., t, :] / dd[..., None]", "dnum = do[..., t, :]"),
    "clamp_mask_inverted": ("np.where(den >= eps,", "np.where(den < eps,"),
    "no_feature_map_derivative": ("\"dq\": dfq * dphi(q)", "\"dq\": dfq"),
    "dphi_wrong_branch": ("np.where(x > 0, 1.0,", "np.where(x < 0, 1.0,"),
    "dk_misses_z_adjoint": ("v[..., t, :]) + dz", "v[..., t, :])"),
    "dv_uses_query_features": ("dS, fk[..., t, :])", "dS, fq[..., t, :])"),
    "dg_uses_state_after_update": ("dS, S_prev)", "dS, S_t)"),
    "dg_misses_z_term": (" + np.einsum(\"...d,...d->...\", dz, z_prev)", ""),
    "adjoint_not_decayed": ("dS = g[..., t, None, None] * dS", "dS = dS"),
    "dq_from_previous_state": ("\"...de,...e->...d\", S_t, dnum)", "\"...de,...e->...d\", S_prev, dnum)"),
    "numerator_mode_keeps_dden": ("dden = np.zeros(den.shape)", "dden = -np.einsum(\"...e,...e->...\", do[..., t, :], num)"),
}


@pytest.mark.parametrize("pin", pins_bwd.ALL_PINS, ids=lambda p: p.__name__)
def test_backward_oracle_pin(pin):
    pin(bwd)


def _mutant(name):
    old, new = MUTATIONS[name]
    src = inspect.getsource(bwd)
    assert src.count(old) == 1, f"mutation {name} does not apply exactly once"
    src = src.replace("from .recurrence import", "from oracle.recurrence import")
    mod = types.ModuleType(f"oracle_bwd_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_backward_mutant_is_caught(name):
    mod = _mutant(name)
    caught = []
    for pin in pins_bwd.ALL_PINS:
        try:
            pin(mod)
        except Exception:                                  # noqa: BLE001 - any failure counts
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
