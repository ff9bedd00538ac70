"""The parity statistics that the full-shape GPU tests print, checked on
hand-made arrays whose statistics are known."""
import numpy as np

from parity import ParityStats


def test_stats_on_known_errors():
    ref = np.array([[1.0, -2.0, 0.0], [0.5, 100.0, 1e-4]])
    got = ref.copy()
    got[0, 1] += 0.03     # |ref| = 2 -> bound 0.022: a failure, ratio 0.03 / 0.022
    got[1, 1] -= 0.5      # |ref| = 100 -> bound 1.002: within, relative error 5e-3
    got[1, 2] += 1e-3     # tiny |ref|: within (bound ~2e-3), excluded from the relative error
    s = ParityStats("t", rtol=1e-2, atol=2e-3)
    s.add(got[:1], ref[:1], where=(7,))
    s.add(got[1:], ref[1:], where=(8,))
    assert s.n == 6 and s.bad == 1 and s.n_rel == 4
    assert np.isclose(s.max_abs, 0.5)
    assert np.isclose(s.max_rel, 0.03 / 2.0)
    assert np.isclose(s.max_ratio, 0.03 / 0.022)
    assert s.worst == (7, 0, 1)
    assert "failures=1" in s.line() and "within=83.3333%" in s.line()


def test_stats_absolute_only():
    ref = np.linspace(-3.0, 3.0, 7)
    got = ref + np.array([0, 0, 5e-5, 0, -2e-4, 0, 0])
    s = ParityStats("lse", rtol=0.0, atol=1e-4)
    s.add(got, ref)
    assert s.bad == 1 and s.worst == (4,)
    assert np.isclose(s.max_ratio, 2.0)
    assert np.isclose(s.max_rel, 2e-4 / 1.0)  # over |ref| > 1e-2: 0 is left out
