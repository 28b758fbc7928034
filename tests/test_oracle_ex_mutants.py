"""Plant plausible mistakes in the oracle's logit variants and dropout (copies
of oracle.c, compiled on the CPU) and show that the variant pins catch each."""
import os
import tempfile

import pytest

from oracle import Oracle, _build
from tests.test_oracle_ex_pins import ALL_CHECKS

MUTANTS = {
    "bias_sign": ("if (bias) s += (double)bias[e * H + h];", "if (bias) s -= (double)bias[e * H + h];"),
    "bias_head_dropped": ("if (bias) s += (double)bias[e * H + h];", "if (bias) s += (double)bias[e * H];"),
    "weight_scales_bias": ("    if (ew) s *= (double)ew[e];\n    if (bias) s += (double)bias[e * H + h];",
                           "    if (bias) s += (double)bias[e * H + h];\n    if (ew) s *= (double)ew[e];"),
    "no_inverse_keep": ("return hi >= thresh ? 1.0 / (1.0 - p) : 0.0;", "return hi >= thresh ? 1.0 : 0.0;"),
    "keep_inverted": ("return hi >= thresh ? 1.0 / (1.0 - p) : 0.0;", "return hi < thresh ? 1.0 / (1.0 - p) : 0.0;"),
    "word_index_head_dropped": ("philox_word(seed, (uint64_t)e * (uint64_t)H + (uint64_t)h)",
                                "philox_word(seed, (uint64_t)e * (uint64_t)H)"),
    "low_bits": ("(uint32_t)(philox_word(seed, (uint64_t)e * (uint64_t)H + (uint64_t)h) >> 32)",
                 "(uint32_t)(philox_word(seed, (uint64_t)e * (uint64_t)H + (uint64_t)h))"),
    "philox_counter_from_zero": ("uint64_t c0 = i / 4 + 1, c1 = 0", "uint64_t c0 = i / 4, c1 = 0"),
    "philox_key_not_bumped": ("        k0 += W0;\n        k1 += W1;", "        k1 += W1;"),
    "dq_without_weight": ("for (int d = 0; d < D; ++d) o[d] += ds * w * elem(K, dtype, uo + d) * rs;",
                          "for (int d = 0; d < D; ++d) o[d] += ds * elem(K, dtype, uo + d) * rs;"),
    "dk_without_weight": ("ok[d] += ds * w * elem(Q, dtype, vo + d) * rs;", "ok[d] += ds * elem(Q, dtype, vo + d) * rs;"),
    "dv_without_dropout": ("ov[d] += a * c * elem(dO, dtype, vo + d);", "ov[d] += a * elem(dO, dtype, vo + d);"),
    "dw_unscaled_dot": ("if (dw) dw[e] += ds * dot;", "if (dw) dw[e] += ds;"),
    "delta_without_dropout": ("double a = exp(s[i] - l) * drop_scale(drop_p, seed, b + i, H, h);",
                              "double a = exp(s[i] - l);"),
    "ds_dropout_on_delta": ("double ds = a * (drop_scale(drop_p, seed, e, H, h) * da - delta[v * H + h]);",
                            "double ds = a * drop_scale(drop_p, seed, e, H, h) * (da - delta[v * H + h]);"),
}


@pytest.fixture(scope="module")
def workdir():
    with tempfile.TemporaryDirectory() as d:
        yield d


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_ex_mutant_is_caught(name, workdir):
    old, new = MUTANTS[name]
    src = open(_build.SRC).read()
    assert src.count(old) == 1, "mutation target must occur once: %r" % old
    path_c = os.path.join(workdir, "oracle_%s.c" % name)
    path_so = os.path.join(workdir, "liboracle_%s.so" % name)
    open(path_c, "w").write(src.replace(old, new))
    _build.build(src=path_c, out=path_so, extra_flags=("-w",))
    orc = Oracle(path_so)
    failed = []
    for check in ALL_CHECKS:
        try:
            check(orc)
        except (AssertionError, ValueError, IndexError):
            failed.append(check.__name__)
    assert failed, "mutant %s passed every variant pin" % name
