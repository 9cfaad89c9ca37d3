"""The oracle's pins catch planted mistakes.

Each case below copies oracle/kgref.c, plants one plausible mistake (a wrong bias,
index, sign or rounding rule, a dropped term, a transposed operand or layout),
compiles the copy with gcc into a temporary library and runs the oracle's pin files
against it in a fresh interpreter (KGREF_LIB selects the library): at least one pin
must fail. The unchanged copy, built the same way, must pass them all. Two more
cases plant mistakes in the Python layer of the K-major entry the same way, by
replacing kgref.token_major before the pins run. Every planted mistake keeps the
oracle's memory accesses in bounds, so a failing pin is a detection, not a crash.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kgref.c")
PINS = ["tests/test_oracle.py", "tests/test_oracle_dgrad.py", "tests/test_oracle_nt.py",
        "tests/test_oracle_requant.py"]

# name -> [(text in kgref.c, replacement)]; every text must occur (all occurrences
# are replaced)
C_MUTANTS = {
    "e4m3 exponent bias 8": [("mag = ldexp((double)(8 + m), e - 10);",
                              "mag = ldexp((double)(8 + m), e - 11);")],
    "e4m3 subnormal scale": [("mag = ldexp((double)m, -9);", "mag = ldexp((double)m, -10);")],
    "e4m3 exponent 15 all NaN": [("if (e == 15 && m == 7)", "if (e == 15)")],
    "e4m3 sign dropped": [("g_e4m3[x] = s ? -mag : mag;", "g_e4m3[x] = mag;")],
    "e8m0 bias 128": [("ldexp(1.0, (int)byte - 127)", "ldexp(1.0, (int)byte - 128)")],
    "scale rows floor": [("boff[g + 1] = boff[g] + (ks[g] + gran_k - 1) / gran_k;",
                          "boff[g + 1] = boff[g] + ks[g] / gran_k;")],
    "blocks from token 0, not the expert start": [
        ("const int64_t srow = (int64_t)p->boff[g] + kb;", "const int64_t srow = t0 / L;")],
    "sb replaced by sa (transposed scale)": [
        ("const double s = s_a * scale_of(p, p->sb, srow, n, p->N);", "const double s = s_a * s_a;"),
        ("const double s = scale_of(p, p->sa, srow, m, p->M) * scale_of(p, p->sb, srow, n, p->N);",
         "const double s = scale_of(p, p->sa, srow, m, p->M) * scale_of(p, p->sa, srow, m, p->M);")],
    "C dropped": [("d_row[n] = (t_end > t_begin) ? c + acc[n] : c;",
                   "d_row[n] = (t_end > t_begin) ? acc[n] : c;"),
                  ("*d = (t_end > t_begin) ? c + acc : c;", "*d = (t_end > t_begin) ? acc : c;")],
    "empty expert zeroed": [("d_row[n] = (t_end > t_begin) ? c + acc[n] : c;",
                             "d_row[n] = (t_end > t_begin) ? c + acc[n] : 0.0;"),
                            ("*d = (t_end > t_begin) ? c + acc : c;",
                             "*d = (t_end > t_begin) ? c + acc : 0.0;")],
    "last token of an expert dropped": [("const int64_t t1 = (t0 + L < t_end) ? t0 + L : t_end;",
                                         "const int64_t t1 = (t0 + L < t_end) ? t0 + L : t_end - 1;")],
    "bound without |b|": [("part_abs[n] += aa * fabs(b);", "part_abs[n] += aa * b;"),
                          ("part_abs += fabs(a) * fabs(b);", "part_abs += fabs(a) * b;")],
    "bf16 ties away from zero": [("if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;",
                                  "if (frac >= 0.5) r += 1.0;")],
    "e4m3 encode ties up": [("c = (lo % 2 == 0) ? lo : hi;", "c = hi;")],
    "e4m3 encode overflow to NaN": [("if (a >= 448.0) return sign | 0x7E;",
                                     "if (a >= 448.0) return sign | 0x7F;")],
    "fp32 scale amax / 447": [("const float s = amax == 0.0f ? 1.0f : amax / 448.0f;",
                               "const float s = amax == 0.0f ? 1.0f : amax / 447.0f;")],
    "ue8m0 exponent not exact at powers of two": [("if (f == 0.5) k -= 1;", "(void)f;")],
    "ue8m0 infinite maximum not clamped": [("  if (isinf(r)) return 254;\n", "")],
    "ue8m0 underflowed quotient not clamped": [("  if (r == 0.0f) return 0;\n", "")],
    "requant amax takes NaNs": [("if (fabsf(x) > amax) amax = fabsf(x);",
                                 "if (!(fabsf(x) <= amax)) amax = fabsf(x);")],
    "e4m3 encode NaN keeps its sign": [("if (isnan(v)) return 0x7F;",
                                        "if (isnan(v)) return signbit(v) ? 0xFF : 0x7F;")],
    "ue8m0 zero block exponent 0": [("const uint8_t e = amax == 0.0f ? 127 : e8m0_ceil(amax / 448.0f);",
                                     "const uint8_t e = amax == 0.0f ? 0 : e8m0_ceil(amax / 448.0f);")],
    "dgrad activation scales token-major": [
        ("(double)p->sa[(int64_t)kb * p->M_total + t]",
         "(double)p->sa[t * (int64_t)(p->K / 128) + kb]")],
    "dgrad weight scale of block column 0": [
        ("(double)p->sw[((int64_t)g * nkb + kb) * (p->N / 128) + n / 128]",
         "(double)p->sw[((int64_t)g * nkb + kb) * (p->N / 128)]")],
    "dgrad weights read as [G][N][K]": [
        ("y = g_e4m3[w[(int64_t)k * p->N + n]]", "y = g_e4m3[w[(int64_t)n * p->K + k]]")],
    "dgrad expert of the previous token range": [
        ("const uint8_t* w = p->W + (int64_t)g * p->K * p->N;",
         "const uint8_t* w = p->W + (int64_t)(g > 0 ? g - 1 : 0) * p->K * p->N;")],
    "token sum not checked": [("if (sum != K_total) return KGREF_ERR_KSUM;\n  return KGREF_OK;",
                               "return KGREF_OK;")],
    "gran_k 64 accepted": [("if (dtype != KGREF_BF16 && gran_k != 32 && gran_k != 128) return KGREF_ERR_GRAN;",
                            "if (dtype != KGREF_BF16 && gran_k != 32 && gran_k != 64 && gran_k != 128)"
                            " return KGREF_ERR_GRAN;")],
}

# mistakes in the K-major entry's Python layer: replacements of kgref.token_major
PY_MUTANTS = {
    "K-major operand read from the row's end": (
        "lambda Xt, K_total: __import__('numpy').ascontiguousarray("
        "__import__('numpy').asarray(Xt)[:, Xt.shape[1] - K_total:].T)"),
    "K-major operand not transposed back": (
        "lambda Xt, K_total: __import__('numpy').ascontiguousarray("
        "__import__('numpy').asarray(Xt)[:, :K_total].reshape(K_total, -1))"),
}


def _compile(src_text, out_dir, name):
    c = os.path.join(out_dir, name + ".c")
    so = os.path.join(out_dir, name + ".so")
    with open(c, "w") as f:
        f.write(src_text)
    r = subprocess.run(["gcc", "-std=c11", "-O1", "-fPIC", "-shared", "-pthread",
                        "-I" + os.path.join(ROOT, "oracle"), c, "-o", so, "-lm"],
                       capture_output=True, text=True)
    assert r.returncode == 0, f"{name}: {r.stderr[-2000:]}"
    return so


def _run_pins(lib_path=None, token_major=None, timeout=600):
    env = dict(os.environ, KGREF_LIB=lib_path or "", OMP_NUM_THREADS="2")
    code = ("import sys, pytest\n"
            f"sys.path.insert(0, {ROOT!r})\n")
    if token_major:
        code += f"from oracle import kgref\nkgref.token_major = {token_major}\n"
    code += ("sys.exit(pytest.main(['-x', '-q', '-p', 'no:cacheprovider', '-m', 'not gpu', "
             + ", ".join(repr(os.path.join(ROOT, p)) for p in PINS) + "]))\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=timeout)
    return r.returncode, r.stdout[-3000:] + r.stderr[-1000:]


def test_pins_catch_every_planted_mistake():
    src = open(SRC).read()
    with tempfile.TemporaryDirectory() as d:
        jobs = [("control", _compile(src, d, "control"), None)]
        for i, (name, edits) in enumerate(C_MUTANTS.items()):
            text = src
            for old, new in edits:
                assert old in text, f"{name}: planted text not found in kgref.c"
                text = text.replace(old, new)
            jobs.append((name, _compile(text, d, f"m{i}"), None))
        for name, fn in PY_MUTANTS.items():
            jobs.append((name, None, fn))
        with ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda j: (j[0],) + _run_pins(j[1], j[2]), jobs))
    rc0, out0 = results[0][1], results[0][2]
    assert rc0 == 0, f"the unchanged oracle fails its pins:\n{out0}"
    missed = [name for name, rc, out in results[1:] if rc != 1 or "failed" not in out]
    assert not missed, f"pins did not catch: {missed}"
