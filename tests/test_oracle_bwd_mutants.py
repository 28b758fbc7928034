"""Plant plausible mistakes in the oracle's backward (copies of oracle.c,
compiled on the CPU) and show that the backward pins catch each one."""
import os
import tempfile

import pytest

from oracle import Oracle, _build
from tests.test_oracle_bwd_pins import ALL_CHECKS

MUTANTS = {
    "delta_dropped_dq": ("double ds = a * (da - delta[v * H + h]);\n                for (int d = 0; d < D; ++d) o[d]",
                         "double ds = a * da;\n                for (int d = 0; d < D; ++d) o[d]"),
    "delta_sign": ("double ds = a * (da - delta[v * H + h]);\n                for (int d = 0; d < D; ++d) {",
                   "double ds = a * (da + delta[v * H + h]);\n                for (int d = 0; d < D; ++d) {"),
    "dq_no_scale": ("o[d] += ds * elem(K, dtype, uo + d) * rs;", "o[d] += ds * elem(K, dtype, uo + d);"),
    "dq_uses_value": ("o[d] += ds * elem(K, dtype, uo + d) * rs;", "o[d] += ds * elem(V, dtype, uo + d) * rs;"),
    "dk_uses_key": ("ok[d] += ds * elem(Q, dtype, vo + d) * rs;", "ok[d] += ds * elem(K, dtype, vo + d) * rs;"),
    "dv_missing_alpha": ("ov[d] += a * elem(dO, dtype, vo + d);", "ov[d] += elem(dO, dtype, vo + d);"),
    "da_from_query": ("for (int d = 0; d < D; ++d) da += elem(dO, dtype, vo + d) * elem(V, dtype, uo + d);",
                      "for (int d = 0; d < D; ++d) da += elem(dO, dtype, vo + d) * elem(Q, dtype, uo + d);"),
    "lse_of_source": ("double a = exp(edge_score(Q, K, dtype, H, D, v, u, h) - lse[v * H + h]);\n                double da = 0.0;\n                for (int d = 0; d < D; ++d) da += elem(dO, dtype, vo + d)",
                      "double a = exp(edge_score(Q, K, dtype, H, D, v, u, h) - lse[u * H + h]);\n                double da = 0.0;\n                for (int d = 0; d < D; ++d) da += elem(dO, dtype, vo + d)"),
    "lse_without_max": ("double l = deg > 0 ? m + log(z) : -INFINITY;", "double l = deg > 0 ? log(z) : -INFINITY;"),
    "delta_unweighted": ("dl += a * da;", "dl += da;"),
}


@pytest.fixture(scope="module")
def workdir():
    with tempfile.TemporaryDirectory() as d:
        yield d


@pytest.mark.filterwarnings("ignore::RuntimeWarning")  # a planted mistake may make non-finite values
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_bwd_mutant_is_caught(name, workdir):
    old, new = MUTANTS[name]
    src = open(_build.SRC).read()
    # the plain backward precedes the variants' copy of some of its lines: the
    # first occurrence is the one in the plain backward
    assert src.count(old) >= 1, "mutation target not found: %r" % old
    path_c = os.path.join(workdir, "oracle_%s.c" % name)
    path_so = os.path.join(workdir, "liboracle_%s.so" % name)
    open(path_c, "w").write(src.replace(old, new, 1))
    _build.build(src=path_c, out=path_so, extra_flags=("-w",))
    orc = Oracle(path_so)
    failed = []
    for check in ALL_CHECKS:
        try:
            check(orc)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(check.__name__)
    assert failed, "mutant %s passed every backward pin" % name
