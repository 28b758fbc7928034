"""Plant plausible mistakes in the oracle's graph construction (copies of
oracle.c, compiled on the CPU) and show that the graph pins catch each one.
Some mistakes write outside the arrays, so each mutant runs its pins in a
forked child process: a crash of the child, or pins that do not finish
within a minute (corrupted offsets can make a check loop nearly forever),
counts as caught."""
import multiprocessing
import os
import tempfile

import pytest

from oracle import Oracle, _build
from tests.test_oracle_graph_pins import ALL_CHECKS

MUTANTS = {
    # rows filled from their end: reverses the order of a row's edges
    "unstable_fill": ("for (int64_t v = 0; v < n_dst; ++v) next[v] = indptr[v];\n",
                      "for (int64_t v = 0; v < n_dst; ++v) next[v] = indptr[v + 1];\n"),
    "unstable_fill_step": ("int64_t p = next[dst[e]]++;", "int64_t p = --next[dst[e]];"),
    "grouped_by_source": ("indptr[dst[e] + 1] += 1;", "indptr[src[e] + 1] += 1;"),
    "counts_not_shifted": ("indptr[dst[e] + 1] += 1;", "indptr[dst[e]] += 1;"),
    "indices_hold_destination": ("indices[p] = src[e];", "indices[p] = dst[e];"),
    "prefix_skips_last": ("for (int64_t v = 0; v < n_dst; ++v) indptr[v + 1] += indptr[v];",
                          "for (int64_t v = 0; v + 1 < n_dst; ++v) indptr[v + 1] += indptr[v];"),
}


@pytest.fixture(scope="module")
def workdir():
    with tempfile.TemporaryDirectory() as d:
        yield d


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_graph_mutant_is_caught(name, workdir):
    old, new = MUTANTS[name]
    src = open(_build.SRC).read()
    assert src.count(old) == 1, "mutation target must occur once: %r" % old
    path_c = os.path.join(workdir, "oracle_%s.c" % name)
    path_so = os.path.join(workdir, "liboracle_%s.so" % name)
    open(path_c, "w").write(src.replace(old, new))
    _build.build(src=path_c, out=path_so, extra_flags=("-w",))
    child = multiprocessing.get_context("fork").Process(target=_run_pins, args=(path_so,), daemon=True)
    child.start()
    child.join(60)
    if child.exitcode is None:
        # the pins never finished: a mutant that corrupts the row offsets can
        # send a check into a near-endless loop.  Not passing is what counts.
        child.kill()
        child.join()
        return
    assert child.exitcode != 0, "mutant %s passed every graph pin" % name


def _run_pins(path_so):
    import faulthandler

    faulthandler.disable()  # a crash here is an expected outcome, not a report
    orc = Oracle(path_so)
    failed = 0
    for check in ALL_CHECKS:
        try:
            check(orc)
        except (AssertionError, ValueError, IndexError):
            failed += 1
    os._exit(1 if failed else 0)
