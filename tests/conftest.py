import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


NAMED_WORKLOADS = ("tiny_fp32", "mixtral_like", "switch_skew", "decode", "gumbel_longtail")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """After a GPU session: the output error of the five named workloads against the oracle
    (tests/parity.py records every comparison), and the worst case over all other ones."""
    parity = sys.modules.get("tests.parity")
    table = getattr(parity, "PARITY_TABLE", None)
    if not table:
        return
    tr = terminalreporter
    tr.write_sep("-", "output parity against the oracle: max|err| <= 2e-2 rms where |y_ref| <= 2.56 rms, "
                      "err - ulp/2 <= 2e-2 rms above; mean_rel <= 5e-3")
    tr.write_line(f"{'workload':<16}{'max|err|/rms':>13}{'at |y|/rms':>11}{'<=2.56rms':>10}{'-ulp/2':>8}"
                  f"{'vs bf16(ref)':>13}{'mean_rel':>10}{'n_big':>7}{'credited':>9}{'elements':>10}")
    for name in NAMED_WORKLOADS:
        st = table.get(name)
        if st is None:
            continue
        if st["dtype"] == "f32":
            tr.write_line(f"{name:<16}  max|err|/max|y_ref| = {st['max_err_over_max_ref']:.2e} (bound 1e-5)"
                          f"{st['elements']:>20}")
            continue
        tr.write_line(f"{name:<16}{st['max_err_over_rms']:>13.4f}{st['at_abs_y_over_rms']:>11.2f}"
                      f"{st['max_err_small_over_rms']:>10.4f}{st['beyond_half_ulp_over_rms']:>8.4f}"
                      f"{st['err_vs_bf16_ref_over_rms']:>13.4f}{st['mean_rel']:>10.2e}{st['n_big']:>7}"
                      f"{st['n_credited']:>9}{st['elements']:>10}")
    others = {k: v for k, v in table.items() if k not in NAMED_WORKLOADS and v["dtype"] == "bf16"}
    if others:
        worst = max(others, key=lambda k: others[k]["max_err_over_rms"])
        st = others[worst]
        tr.write_line(f"other bf16 cases: {len(others)}, worst max|err|/rms {st['max_err_over_rms']:.4f} ({worst}), "
                      f"worst mean_rel {max(v['mean_rel'] for v in others.values()):.2e}, "
                      f"credited elements {sum(v['n_credited'] for v in others.values())}")
    raised = {k: v["bf16_h_bound_rms"] for k, v in others.items() if "bf16_h_bound_rms" in v}
    for name, b in sorted(raised.items()):
        tr.write_line(f"  {name}: the bf16 rounding of H alone is beyond 1e-2 rms; bound {b:.4f} rms "
                      f"(max|err|/rms {others[name]['max_err_over_rms']:.4f})")


@pytest.fixture(scope="session")
def repo_root():
    return ROOT
