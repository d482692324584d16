import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (generates hundreds of MB of input)")


@pytest.fixture(scope="session")
def oracle():
    import oracle as _oracle

    _oracle.set_threads(min(8, len(os.sched_getaffinity(0))))
    return _oracle


def pytest_terminal_summary(terminalreporter):
    """Report how close to their rounding midpoints the admitted code mismatches were."""
    try:
        from tiecheck import tie_window_stats
    except ImportError:
        return
    st = tie_window_stats()
    if st["admitted"]:
        terminalreporter.write_line(
            f"tie mismatches admitted: {st['admitted']}; largest distance from the midpoint "
            f"{st['max_distance']:.3e} code units, {100 * st['max_window_frac']:.1f}% of the "
            f"window; {st['over_half_window']} beyond half the window; largest distance at "
            f"|mid| <= 8: {st['max_distance_small_mid']:.3e} code units; largest relative distance "
            f"at |mid| > 8: {st['max_rel_distance_large_mid']:.3e}; window-fraction histogram "
            f"[0,1/64) [1/64,1/16) [1/16,1/4) [1/4,1/2) [1/2,1]: {st['window_frac_hist']}")
