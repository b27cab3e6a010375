"""Sensitivity of the refit pins: plausible mistakes planted in copies of the
oracle's refit must each fail a hand-derived golden.

Every mutant is the oracle source with one textual change, compiled with the
oracle's own flags into a temporary library (nothing under oracle/ is
modified).  The unmutated copy must pass every golden, so a failure of a
mutant is the planted mistake and not the harness.  Pages: qingkeai STEPQuant
talk preview, "STEPQuant 核心设计…" (row scale from the row's magnitude and its
measured impact); e-cogni STEPQuant analysis, "Como funciona" (square-root
smoothing, geometric-mean normalisation of the row factors)."""
import ctypes
import hashlib
import os
import subprocess

import numpy as np
import pytest

from oracle import oracle as orc_mod
from test_oracle_refit import REFIT_GOLDENS, check_refit_golden

SRC = os.path.join(os.path.dirname(orc_mod.__file__), "stq_oracle.c")

# name -> [(text in the refit, replacement), ...]; each text must occur as
# often as listed (all occurrences are replaced)
MUTANTS = {
    "row-impact weight dropped": [("float p = m * w[i];", "float p = m; (void)w;", 1)],
    "row factor truncated to bf16": [("s0[i] = bf16_rne(rho);", "s0[i] = (uint16_t)(bits_of_f32(rho) >> 16);", 1)],
    "row factor rounded half away from zero": [
        ("s0[i] = bf16_rne(rho);", "s0[i] = (uint16_t)((bits_of_f32(rho) + 0x8000u) >> 16);", 1)],
    "X = S / sigma instead of S * fl(1/sigma)": [
        ("float X = S[(size_t)i * dv + j] * rs[i];", "float X = S[(size_t)i * dv + j] / bf16_val(s0[i]);", 1),
        ("float X = S[ix] * rs[i];", "float X = S[ix] / bf16_val(s0[i]);", 1)],
    "|X| / qmax instead of |X| * fl(1/qmax)": [
        ("float t = fabsf(X) * rq;", "float t = fabsf(X) / (float)qmax_of(nb[i]); (void)rq;", 1)],
    "code from the binary32 product": [
        ("double prod = (double)X * (double)rc;", "double prod = (double)(float)(X * rc);", 1)],
    "code from X / t": [
        ("double prod = (double)X * (double)rc;", "double prod = (double)(float)(X / bf16_val(t0)); (void)rc;", 1)],
    "column scale rounded to nearest": [("t0 = bf16_ru(M);", "t0 = bf16_rne(M);", 1)],
}


def _build(tmp, name, edits):
    src = open(SRC).read()
    for old, new, count in edits:
        assert src.count(old) == count, (name, old)
        src = src.replace(old, new)
    tag = "m" + hashlib.md5(name.encode()).hexdigest()[:10]
    c_path = os.path.join(tmp, tag + ".c")
    so_path = os.path.join(tmp, tag + ".so")
    with open(c_path, "w") as fh:
        fh.write(src)
    subprocess.check_call(["gcc"] + orc_mod._CFLAGS + ["-w", "-o", so_path, c_path, "-lm"])
    L = ctypes.CDLL(so_path)
    L.orc_refit.argtypes = [ctypes.c_int] * 2 + [ctypes.c_void_p] * 7
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)

    def refit(S, w, nb):
        S = np.ascontiguousarray(S, np.float32)
        dk, dv = S.shape
        w = np.ascontiguousarray(w, np.float32)
        nb = np.ascontiguousarray(nb, np.int32)
        sig = np.zeros(dk, np.uint16)
        cst = np.zeros(dv, np.uint16)
        Q = np.zeros((dk, dv), np.int32)
        E = np.zeros(1, np.int32)
        L.orc_refit(dk, dv, p(S), p(w), p(nb), p(sig), p(cst), p(Q), p(E))
        return sig, cst, Q, int(E[0])
    return refit


@pytest.fixture(scope="module")
def tmpdir_mut(tmp_path_factory):
    return str(tmp_path_factory.mktemp("oracle_mutants"))


def test_unmutated_copy_passes(tmpdir_mut):
    refit = _build(tmpdir_mut, "none", [])
    for g in REFIT_GOLDENS:
        assert check_refit_golden(refit, g) == [], g


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_golden(tmpdir_mut, name):
    refit = _build(tmpdir_mut, name, MUTANTS[name])
    failed = {g: check_refit_golden(refit, g) for g in REFIT_GOLDENS}
    print(name, failed)
    assert any(failed.values()), "planted mistake not caught: " + name
