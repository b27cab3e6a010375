"""Sensitivity of the refit pins: plausible mistakes planted in copies of the
oracle's refit must each fail a hand-derived golden.

Every mutant is the oracle source with one textual change, compiled with the
oracle's own flags into a temporary library (nothing under oracle/ is
modified).  The unmutated copy must pass every golden, so a failure of a
mutant is the planted mistake and not the harness.  Pages: qingkeai STEPQuant
talk preview, "STEPQuant 核心设计…" (row scale from the row's magnitude and its
measured impact); e-cogni STEPQuant analysis, "Como funciona" (square-root
smoothing, geometric-mean normalisation of the row factors)."""
import concurrent.futures
import ctypes
import hashlib
import os
import subprocess
import sys

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


# ---------------------------------------------------------------------------
# The other oracle functions: a planted mistake in the update, the window
# path, the tile layouts, the pool rules or the prefill must make one of the
# oracle's own pin files fail.  Each mutant is compiled on its own and the pin
# files run against it in a child pytest (STQ_ORACLE_LIB names the library the
# oracle loads); the unmutated copy must pass them all.  Pages: e-cogni
# STEPQuant analysis, "Contexto" (GDN and KDA gated delta update and readout);
# wink.run LeapQuant post, per-window quantization (window cache, gate
# products) and the section on decode cost under prefix caching (prefill).

PIN_FILES = ["tests/test_oracle_update.py", "tests/test_oracle_pool.py", "tests/test_oracle_window.py",
             "tests/test_oracle_layout.py", "tests/test_oracle_rows.py", "tests/test_oracle_prefill.py"]

WIDE_MUTANTS = {
    # A = Diag(a) S, u = A^T k, delta = b (v - u), S' = A + k delta^T, o = S'^T q
    "prediction from the ungated state": [
        ("u += Sp[(size_t)i * dv + j] * k[i];", "u += S[(size_t)i * dv + j] * k[i];", 1)],
    "delta with its sign flipped": [("delta[j] = b * (v[j] - u);", "delta[j] = b * (u - v[j]);", 1)],
    "write strength b dropped": [("delta[j] = b * (v[j] - u);", "delta[j] = (v[j] - u); (void)b;", 1)],
    "readout from the state before the update": [
        ("s += Sp[(size_t)i * dv + j] * q[i];", "s += S[(size_t)i * dv + j] * q[i];", 1)],
    "per-channel gate read as a scalar": [
        ("double ai = per_row_gate ? a[i] : a[0];", "double ai = a[0]; (void)per_row_gate;", 1)],
    # window: S_t = G_t S_0 + sum_s (G_t / G_s) k_s u_s^T
    "fold with the gate ratio inverted": [
        ("s += (Gt / (double)G[m]) * (double)K[", "s += ((double)G[m] / Gt) * (double)K[", 1)],
    "fold base not scaled by the gate product": [
        ("double s = Gt * (double)t->S[(size_t)i * dv + j];", "double s = (double)t->S[(size_t)i * dv + j];", 1)],
    "window readout with the gate ratio inverted": [
        ("ck[m] = ((double)Gt / (double)G[m]) * sk;", "ck[m] = ((double)G[m] / (double)Gt) * sk;", 1)],
    "window gate product not accumulated": [
        ("float Gt = (cnt == 0) ? a : G[cnt - 1] * a;", "float Gt = a;", 1)],
    # layouts
    "4-bit nibbles swapped": [
        ("bytes[0] = (uint8_t)(f[0] | (f[1] << 4));", "bytes[0] = (uint8_t)(f[1] | (f[0] << 4));", 1)],
    "two's complement fields instead of offset binary": [
        ("f[c] = (n == 16) ? q : q + (1 << (n - 1));", "f[c] = (n == 16) ? q : (q & ((1 << n) - 1));", 1)],
    "6-bit fields in reverse order": [
        ("uint32_t g = (uint32_t)f[0] | ((uint32_t)f[1] << 6) | ((uint32_t)f[2] << 12) | ((uint32_t)f[3] << 18);",
         "uint32_t g = (uint32_t)f[3] | ((uint32_t)f[2] << 6) | ((uint32_t)f[1] << 12) | ((uint32_t)f[0] << 18);", 2)],
    "lane rows interleaved the other way": [
        ("*i = 32 * rc + 16 * (t / 4) + 4 * (l / 16) + (t % 4);", "*i = 32 * rc + 16 * (t / 4) + (l / 16) + 4 * (t % 4);", 1)],
    "row-record scales big-endian": [
        ("for (int i = 0; i < dk; i++) { tile[off + 2 * i] = sig[i] & 0xFF; tile[off + 2 * i + 1] = sig[i] >> 8; }",
         "for (int i = 0; i < dk; i++) { tile[off + 2 * i] = sig[i] >> 8; tile[off + 2 * i + 1] = sig[i] & 0xFF; }", 1)],
    # pool rules and prefill
    "identity token re-encodes the tile": [
        ("if (identity) return;   /* the identity update leaves the encoding as it is */", "(void)identity;", 1)],
    "prefill drops the prompt's last token": [
        ("for (int tok = ss[c]; tok < ss[c + 1]; tok++) {", "for (int tok = ss[c]; tok < ss[c + 1] - 1; tok++) {", 1)],
    "prefill of a window pool without the fold": [
        ("if (cp) window_fold(&d, h, tp, cp, row_w(&d, img, h), &t);", "(void)0;", 1)],
}


def _build_lib(tmp, name, edits):
    src = open(SRC).read()
    for old, new, count in edits:
        assert src.count(old) == count, (name, old)
        src = src.replace(old, new)
    tag = "w" + hashlib.md5(name.encode()).hexdigest()[:10]
    c_path = os.path.join(tmp, tag + ".c")
    so_path = os.path.join(tmp, tag + ".so")
    with open(c_path, "w") as fh:
        fh.write(src)
    subprocess.check_call(["gcc"] + orc_mod._CFLAGS + ["-w", "-o", so_path, c_path, "-lm"])
    return so_path


def _run_pins(so_path):
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, STQ_ORACLE_LIB=so_path, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"]
                       + PIN_FILES, cwd=root, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


@pytest.fixture(scope="module")
def wide_results(tmpdir_mut):
    names = ["none"] + sorted(WIDE_MUTANTS)
    libs = {n: _build_lib(tmpdir_mut, n, WIDE_MUTANTS.get(n, [])) for n in names}
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        futs = {n: ex.submit(_run_pins, libs[n]) for n in names}
        return {n: f.result() for n, f in futs.items()}


def test_unmutated_copy_passes_every_pin(wide_results):
    rc, out = wide_results["none"]
    assert rc == 0, out


@pytest.mark.parametrize("name", sorted(WIDE_MUTANTS))
def test_mutant_fails_a_pin(wide_results, name):
    rc, out = wide_results[name]
    print(name, "->", out.strip().splitlines()[-1] if out.strip() else "")
    assert rc == 1, "planted mistake not caught (rc %d): %s\n%s" % (rc, name, out)
