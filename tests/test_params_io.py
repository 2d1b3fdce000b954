"""Saving and loading a processor's parameters (structured_rotations_amd.params):
exact round trip, no unpickling, size checks against the schedule; the
parameter counts are the oracle's."""
import numpy as np
import pytest

from oracle import harp_oracle as O
from structured_rotations_amd import inputs as I
from structured_rotations_amd import params as P


@pytest.mark.parametrize("sch", [(8, 8, 8, 8), (8, 8, 8, 5, 2), (3, 7, 16, 2)])
def test_round_trip(tmp_path, sch):
    d = int(np.prod(sch))
    g_sign, g_theta, g_gauss, _ = I.streams(I.BASE_SEED + 7)
    theta = I.theta_params(g_theta, sch, d, 0.05, 0.1)
    gauss = I.gauss_mats(g_gauss, sch)
    signs = I.rademacher(g_sign, d)
    assert theta.size == sum(O.theta_counts(sch, d))
    codes, scales = O.quantize_theta(sch, d, theta)
    f = tmp_path / "p.npz"
    P.save_params(f, sch, d, signs, theta=theta, gauss=gauss, theta_codes=codes, theta_scales=scales,
                  seeds=[I.BASE_SEED + 7])
    back = P.load_params(f)
    assert back["schedule"] == tuple(sch) and back["d"] == d
    assert np.array_equal(back["theta"], theta) and np.array_equal(back["gauss"], np.ravel(gauss))
    assert np.array_equal(back["signs"], signs) and np.array_equal(back["theta_codes"], codes)
    assert np.array_equal(back["theta_scales"], np.asarray(scales, dtype=np.float32))
    # the reloaded parameters give the same blocks
    b0 = O.materialize_blocks(sch, d, theta, gauss)
    b1 = O.materialize_blocks(back["schedule"], back["d"], back["theta"], back["gauss"])
    assert all(np.array_equal(x, y) for x, y in zip(b0, b1))


def test_size_checks(tmp_path):
    sch, d = (8, 5, 2), 80
    signs = np.ones(d, dtype=np.int8)
    n = sum(O.theta_counts(sch, d))
    with pytest.raises(ValueError):
        P.save_params(tmp_path / "a.npz", sch, d, signs, theta=np.zeros(n + 1), gauss=np.zeros(25))
    with pytest.raises(ValueError):
        P.save_params(tmp_path / "b.npz", sch, d, signs, theta=np.zeros(n), gauss=np.zeros(24))
    with pytest.raises(ValueError):
        P.save_params(tmp_path / "c.npz", sch, 81, signs, theta=np.zeros(n), gauss=np.zeros(25))
    with pytest.raises(ValueError):
        P.save_params(tmp_path / "d.npz", sch, d, np.zeros(d, dtype=np.int8), theta=np.zeros(n), gauss=np.zeros(25))


def test_load_refuses_pickles(tmp_path):
    f = tmp_path / "obj.npz"
    np.savez(f, format=np.array(1, dtype=np.int32), schedule=np.array([2, 2], dtype=np.int32),
             d=np.array(4, dtype=np.int64), signs=np.ones(4, dtype=np.int8), gauss=np.zeros(0),
             theta=np.array([{"a": 1}], dtype=object))
    with pytest.raises(ValueError):
        P.load_params(f)
