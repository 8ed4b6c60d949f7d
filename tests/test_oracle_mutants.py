"""CPU tests: the pins are sharp enough to catch plausible mistakes in the oracle.

Each mutant is a copy of oracle/kda_oracle.c with one plausible mistake planted
(a dropped term, a wrong sign, a wrong operand or axis, an off-by-one). The
copy is compiled into a temporary library and must fail at least one pin.
"""
import ctypes
import functools
import os
import shutil

import pytest

import oracle
from oracle import build as obuild

from oracle_pins import ALL_CHECKS

MUTANTS = {
    "no_decay": ("row[j] *= a;", "row[j] *= 1.0;"),
    "no_clamp": ("double gi = gt[i] < J->lower_bound ? J->lower_bound : gt[i];", "double gi = gt[i];"),
    "delta_sign": ("kv[j] = bt * (vt[j] - kv[j]);", "kv[j] = bt * (vt[j] + kv[j]);"),
    "no_beta": ("kv[j] = bt * (vt[j] - kv[j]);", "kv[j] = (vt[j] - kv[j]);"),
    "read_with_k": ("const double qi = qt[i];", "const double qi = kt[i];"),
    "no_scale": ("ot[j] *= J->scale;", "ot[j] *= 1.0;"),
    "ignore_initial_state": ("if (J->s0)", "if (0)"),
    "skip_first_token": ("for (int64_t t = bos; t < eos; ++t)", "for (int64_t t = bos + 1; t < eos; ++t)"),
    "half_write": ("row[j] += ki * kv[j];", "row[j] += 0.5 * ki * kv[j];"),
    "decay_exp_of_neg": ("double a = exp(gi);", "double a = exp(-gi);"),
    "beta_head_index": ("const double bt = J->beta[t * H + h];", "const double bt = J->beta[t * H];"),
    "gate_head_index": ("const double *gt = J->g + (t * H + h) * dk;", "const double *gt = J->g + (t * H) * dk;"),
}


@functools.lru_cache(maxsize=None)
def _mutant_lib(name, tmpdir):
    src = open(obuild.SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutant anchor not unique: {old!r}"
    path = os.path.join(tmpdir, f"mut_{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = obuild.compile_oracle(path, os.path.join(tmpdir, f"libmut_{name}.so"), strict=False)
    return oracle._bind(ctypes.CDLL(lib))


@pytest.fixture(scope="module")
def tmpdir_mod(tmp_path_factory):
    d = tmp_path_factory.mktemp("mutants")
    yield str(d)
    shutil.rmtree(str(d), ignore_errors=True)


@pytest.mark.skipif(shutil.which(os.environ.get("CC", "gcc")) is None, reason="no C compiler")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmpdir_mod):
    lib = _mutant_lib(name, tmpdir_mod)
    fwd = functools.partial(oracle.kda_forward, lib=lib)
    failed = []
    for check in ALL_CHECKS:
        try:
            check(fwd)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(check.__name__)
    assert failed, f"mutant {name} passed every pin"
