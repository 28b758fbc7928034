"""Plant plausible mistakes in copies of oracle.c and show that the pins catch each.

Every mutant is a text edit of the oracle source, compiled with gcc into a
temporary library on the CPU; the pins of test_oracle_pins.py then run
against it and at least one must fail.  Nothing here touches the GPU.
"""
import os
import tempfile

import pytest

from oracle import Oracle, _build
from tests.test_oracle_pins import ALL_CHECKS

MUTANTS = {
    # SDDMM
    "no_scale": ("return dot / sqrt((double)D);", "return dot;"),
    "scale_by_D": ("return dot / sqrt((double)D);", "return dot / (double)D;"),
    "query_from_source": ("int64_t qo = (v * H + h) * (int64_t)D, ko = (u * H + h) * (int64_t)D;",
                          "int64_t qo = (u * H + h) * (int64_t)D, ko = (u * H + h) * (int64_t)D;"),
    "key_from_destination": ("int64_t qo = (v * H + h) * (int64_t)D, ko = (u * H + h) * (int64_t)D;",
                             "int64_t qo = (v * H + h) * (int64_t)D, ko = (v * H + h) * (int64_t)D;"),
    "head_dropped": ("int64_t qo = (v * H + h) * (int64_t)D, ko = (u * H + h) * (int64_t)D;",
                     "int64_t qo = (v * H) * (int64_t)D, ko = (u * H) * (int64_t)D;"),
    "dot_skips_last": ("for (int d = 0; d < D; ++d) dot +=", "for (int d = 0; d < D - 1; ++d) dot +="),
    # softmax
    "no_normalise": ("for (int64_t i = 0; i < deg; ++i) a[i] /= z;", "(void)z;"),
    "no_max_shift": ("a[i] = exp(s[i] - m);", "a[i] = exp(s[i]);"),
    "sign_flip": ("a[i] = exp(s[i] - m);", "a[i] = exp(m - s[i]);"),
    "max_is_first": ("if (s[i] > m) m = s[i];", "if (i == 0) m = s[i];"),
    # SpMM / whole path
    "value_from_destination_fwd": ("int64_t vo = ((int64_t)indices[b + i] * H + h) * (int64_t)D;",
                                   "int64_t vo = (v * H + h) * (int64_t)D;"),
    "value_from_destination_spmm": ("int64_t vo = ((int64_t)indices[e] * H + h) * (int64_t)D;",
                                    "int64_t vo = (v * H + h) * (int64_t)D;"),
    "spmm_wrong_head_weight": ("double a = alpha[e * H + h];", "double a = alpha[e * H];"),
    "fwd_drops_last_edge": ("for (int64_t i = 0; i < deg; ++i) s[i] = edge_score",
                            "if (deg > 1) --deg; for (int64_t i = 0; i < deg; ++i) s[i] = edge_score"),
    "bf16_wrong_shift": ("uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;",
                         "uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 15;"),
    "sddmm_edge_offset": ("scores[e * H + h] = edge_score(Q, K, dtype, H, D, v, indices[e], h);",
                          "scores[e * H + h] = edge_score(Q, K, dtype, H, D, v, indices[e > 0 ? e - 1 : e], h);"),
}


@pytest.fixture(scope="module")
def workdir():
    with tempfile.TemporaryDirectory() as d:
        yield d


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, workdir):
    old, new = MUTANTS[name]
    src = open(_build.SRC).read()
    assert src.count(old) >= 1, "mutation target not found: %r" % old
    mutated = src.replace(old, new)
    path_c = os.path.join(workdir, "oracle_%s.c" % name)
    path_so = os.path.join(workdir, "liboracle_%s.so" % name)
    open(path_c, "w").write(mutated)
    _build.build(src=path_c, out=path_so, extra_flags=("-w",))
    orc = Oracle(path_so)
    failed = []
    for check in ALL_CHECKS:
        try:
            check(orc)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(check.__name__)
    assert failed, "mutant %s passed every pin" % name
