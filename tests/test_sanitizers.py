"""The CPU code under the address and undefined-behaviour sanitizers.

- The oracle (``oracle/adacomp_oracle.c``) with the command-line driver
  ``tests/cpu/oracle_driver.c``, built twice -- plainly and with
  ``-fsanitize=address,undefined -fno-sanitize-recover=all`` -- runs the
  hand-worked cases of ``tests/golden/hand_worked.json``, random tiny tables
  (8- and 16-bit words, ragged last bins, local-selection segments, several
  learners and steps), every decode entry point (sum, accumulate, SGD, Adam),
  a refused corrupt message and refused tables.  The sanitized build must
  report nothing and print exactly what the plain build prints; the worked
  cases must give their printed residues and bin maxima.
- The host geometry check of the HIP library's tiling
  (``tests/cpu/geometry_check.cpp``) runs sanitized in ``test_capi_host.py``.
"""
import json
import os
import pathlib
import subprocess

import numpy as np

import oracle

ROOT = pathlib.Path(__file__).resolve().parents[1]
GOLDEN = ROOT / "tests" / "golden" / "hand_worked.json"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def build_driver(out: pathlib.Path, sanitize: bool) -> pathlib.Path:
    flags = [f for f in oracle.CFLAGS if f not in ("-fPIC", "-shared")]
    if sanitize:
        flags = [f if f != "-O2" else "-O1" for f in flags] + SAN
    subprocess.run(["gcc", *flags, "-o", str(out), str(ROOT / "tests" / "cpu" / "oracle_driver.c"),
                    str(ROOT / "oracle" / "adacomp_oracle.c"), "-lm"], check=True)
    return out


def hexs(a):
    return " ".join(f"{x:08x}" for x in np.asarray(a, np.float32).view(np.uint32))


def case_text(segs, K, T, span, residues, dws, w, m, v, params, step):
    """segs: (offset, numel, bin_len, flags); residues[k]; dws[k][t]."""
    lines = [f"{len(segs)} {K} {T} {span}"]
    lines += [f"{o} {n} {lt} {fl}" for (o, n, lt, fl) in segs]
    for k in range(K):
        lines.append(hexs(residues[k]))
        lines += [hexs(dws[k][t]) for t in range(T)]
    lines += [hexs(w), hexs(m), hexs(v), hexs(np.array(params, np.float32)), str(step)]
    return "\n".join(lines)


def golden_cases():
    out = []
    for c in json.loads(GOLDEN.read_text())["cases"]:
        if "residue" in c:
            r = np.array(c["residue"], np.float32)
            d = np.array(c["dW"], np.float32)
            want_r = np.array(c["residue_new"], np.float32)
        else:
            n = c["numel"]
            r, d, want_r = (np.zeros(n, np.float32) for _ in range(3))
            for src, dst in (("residue_sparse", r), ("dW_sparse", d), ("residue_new_sparse", want_r)):
                for k, x in c[src].items():
                    dst[int(k)] = x
        out.append((c, r, d, want_r))
    return out


def random_cases(rng, count):
    out = []
    for _ in range(count):
        segs, off = [], int(rng.integers(0, 3)) * 4
        for _ in range(int(rng.integers(1, 4))):
            n = int(rng.integers(1, 200))
            lt = int(rng.choice([1, 3, 7, 50, 63, 64, 65, 500, n]))
            segs.append((off, n, lt, int(rng.random() < 0.3)))
            off += (n + 3) // 4 * 4 + int(rng.integers(0, 2)) * 4
        span = off + 4
        K, T = int(rng.integers(1, 5)), int(rng.integers(1, 4))
        res = [(rng.standard_normal(span) * 1e-3).astype(np.float32) * (k % 2) for k in range(K)]
        dws = [[(rng.standard_normal(span) * 1e-3).astype(np.float32) for _ in range(T)]
               for _ in range(K)]
        w = (rng.standard_normal(span) * 0.05).astype(np.float32)
        m = (rng.standard_normal(span) * 1e-3).astype(np.float32)
        v = (rng.random(span) * 1e-6).astype(np.float32)
        params = [0.01, 0.9, float(rng.choice([0.0, 1e-4])), 1.0 / K, 0.9, 0.999, 1e-8]
        out.append((segs, K, T, span, res, dws, w, m, v, params, int(rng.integers(1, 10))))
    return out


def test_oracle_under_sanitizers(tmp_path):
    plain = build_driver(tmp_path / "driver_plain", False)
    san = build_driver(tmp_path / "driver_san", True)
    cases = []
    gold = golden_cases()
    for c, r, d, _ in gold:
        n = r.size
        z = np.zeros(n, np.float32)
        cases.append(case_text([(0, n, c["bin_len"], 0)], 1, 1, n, [r], [[d]], z + 0.5, z, z + 1e-6,
                               [0.1, 0.9, 0.0, 1.0, 0.9, 0.999, 1e-8], 1))
    rng = np.random.default_rng(4242)
    cases += [case_text(*rc) for rc in random_cases(rng, 24)]
    z4 = np.zeros(4, np.float32)
    for bad in ([(0, 0, 50, 0)], [(0, 4, 0, 0)], [(0, 4, 32769, 0)], [(0, 4, 8, 2)]):
        cases.append(case_text(bad, 1, 1, 4, [z4], [[z4]], z4, z4, z4, [0.0] * 7, 1))
    inp = tmp_path / "cases.txt"
    inp.write_text(f"{len(cases)}\n" + "\n".join(cases) + "\n")

    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    a = subprocess.run([str(plain), str(inp)], capture_output=True, text=True, timeout=300)
    b = subprocess.run([str(san), str(inp)], capture_output=True, text=True, timeout=600, env=env)
    assert a.returncode == 0, a.stderr[-2000:]
    assert b.returncode == 0, b.stderr[-4000:]
    assert "Sanitizer" not in b.stderr and "runtime error" not in b.stderr, b.stderr[-4000:]
    assert a.stdout == b.stdout

    lines = b.stdout.splitlines()
    # every call ran: one decode, SGD, Adam and refused corrupt message per valid case
    n_valid = len(cases) - 4
    for tag in ("decode 0", "decode_acc 0", "sgd 0", "adam 0", "corrupt -3"):
        assert sum(1 for l in lines if l == tag) == n_valid, tag
    assert sum(1 for l in lines if l.startswith("capacity -1")) == 4
    # the worked cases' printed residues and bin maxima
    res = [l for l in lines if l.startswith("residue")]
    gm = [l for l in lines if l.startswith("gmax")]
    for i, (c, _, _, want_r) in enumerate(gold):
        assert res[i] == "residue " + hexs(want_r), c["name"]
        assert gm[i] == "gmax " + hexs(np.array(c["gmax"], np.float32)), c["name"]
