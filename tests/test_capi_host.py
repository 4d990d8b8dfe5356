"""Host-side tests of the C ABI (no GPU needed): the library loads and exports
every function include/adacomp.h declares, segment-table validation, the plan
sizes, and a CPU check of the tile geometry every kernel launch relies on."""
import ctypes
import pathlib
import random
import re
import subprocess

import pytest

import adaptive_residual_gradient_amd as A
import msgparse as mp
import oracle
import workloads as W

ROOT = pathlib.Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "adacomp.h"


@pytest.fixture(scope="module", autouse=True)
def _lib_built():
    if not A.LIB_PATH.exists():
        from adaptive_residual_gradient_amd import _build
        _build.build()


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(adacomp_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 13
    h = ctypes.CDLL(str(A.LIB_PATH))
    for n in names:
        assert hasattr(h, n), f"{n} not exported"
    assert set(names) == set(A.SIGNATURES), "binding and header disagree"
    out = subprocess.run(["nm", "-D", "--defined-only", str(A.LIB_PATH)],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (adacomp_\w+)", out))
    assert set(names) <= exported


def test_binding_constants_match_the_header():
    text = HEADER.read_text()

    def macro(name):   # "N", "Nu" or "(Au << B)"
        m = re.search(r"#define\s+" + name + r"\s+(?:\((\d+)u?\s*<<\s*(\d+)\)|(\d+)u?\b)", text)
        assert m, name
        return int(m.group(1)) << int(m.group(2)) if m.group(1) else int(m.group(3))

    assert macro("ADACOMP_SEG_LS") == A.SEG_LS
    assert macro("ADACOMP_PLAN_SEPARATE_FINISH") == A.PLAN_SEPARATE_FINISH
    assert macro("ADACOMP_PLAN_SINGLE_LAUNCH") == A.PLAN_SINGLE_LAUNCH
    assert macro("ADACOMP_SMALL_TABLE_MAX_SPAN") == A.SMALL_TABLE_MAX_SPAN
    assert macro("ADACOMP_SMALL_TABLE_MAX_SEGMENTS") == A.SMALL_TABLE_MAX_SEGMENTS
    assert macro("ADACOMP_CHUNK_FINISH_MAX_TILES") == A.CHUNK_FINISH_MAX_TILES
    assert macro("ADACOMP_MAX_MESSAGES") == A.MAX_MESSAGES
    assert macro("ADACOMP_MAX_BIN_LEN") == A.MAX_BIN_LEN
    assert macro("ADACOMP_NUM_STAGES") == A.NUM_STAGES == len(A.STAGES)
    assert ctypes.sizeof(A.PlanInfo) == 8 + 10 * 8


def test_status_strings():
    for st in range(0, -8, -1):
        assert A.status_str(st) != "unknown status"
    assert A.status_str(-99) == "unknown status"


@pytest.mark.parametrize("segs,status", [
    ([], -1),
    ([(0, 0, 50)], -1),
    ([(0, 100, 0)], -2),
    ([(0, 100, 32769)], -2),
    ([(2, 100, 50)], -3),
    ([(0, 100, 50), (96, 10, 50)], -4),
    ([(100, 10, 50), (0, 101, 50)], -4),
    ([(0, 1 << 32, 500)], -7),
    ([(0, 100, 50, 2)], -1),
    ([(0, 100, 50, 3)], -1),
])
def test_plan_query_rejects(segs, status):
    with pytest.raises(A.AdaCompError) as e:
        A.plan_query(segs)
    assert e.value.status == status


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_plan_info_matches_format(name):
    wl = W.workload(name)
    info = A.plan_query(wl.segments)
    assert info.nseg == len(wl.segments)
    assert info.total_numel == wl.numel and info.span == W.alloc_len(wl)
    assert info.total_bins == wl.bins
    assert info.header_bytes == 32 + 16 * len(wl.segments)
    assert info.plan_hash == mp.table_hash(wl.segments) == oracle.plan_hash(wl.segments)
    assert info.message_capacity == oracle.message_capacity(wl.segments)


def test_ls_flag_enters_plan_hash():
    """The hard-local-selection flag is part of the segment table, so it enters
    the header hash; capacity is unchanged."""
    segs = [(0, 1000, 50, A.SEG_LS), (1000, 500, 500)]
    info = A.plan_query(segs)
    assert info.plan_hash == mp.table_hash(segs) == oracle.plan_hash(segs)
    assert info.plan_hash != A.plan_query([(0, 1000, 50), (1000, 500, 500)]).plan_hash
    assert info.message_capacity == oracle.message_capacity(segs)


def test_compress_launches_rule():
    """After one tile-pass launch per tile shape: tables of span <= 2^21 and
    <= 256 segments finish in one launch; other tables of <= 256 segments and
    <= 2^20 tiles in two; the rest in three."""
    launches = {name: A.plan_query(W.workload(name).segments).compress_launches
                for name in W.WORKLOADS}
    assert launches == {"fc": 2, "conv": 3, "fc_lstm": 3, "resnet50": 3, "large": 3}
    assert A.plan_query([(0, 1 << 21, 500)]).compress_launches == 2
    assert A.plan_query([(0, (1 << 21) + 4, 500)]).compress_launches == 3
    assert A.plan_query([(4 * i, 4, 4) for i in range(256)]).compress_launches == 2
    assert A.plan_query([(4 * i, 4, 4) for i in range(257)]).compress_launches == 4
    big = [(4 * i, 4, 4) for i in range(255)] + [(1020, 1 << 22, 500)]
    assert A.plan_query(big).compress_launches == 3
    assert A.plan_query(big + [(1020 + (1 << 22), 4, 4)]).compress_launches == 4
    # L_T 1: 2048 bins of one element per tile, so 2^20 tiles are 2^31 elements
    # (planned on the host only).
    assert A.plan_query([(0, 1 << 31, 1)]).ntiles == A.CHUNK_FINISH_MAX_TILES
    assert A.plan_query([(0, 1 << 31, 1)]).compress_launches == 3
    assert A.plan_query([(0, (1 << 31) + 4, 1)]).compress_launches == 4
    # three tile shapes (L_T 50, 4093, 5000): three tile-pass launches
    assert A.plan_query([(0, 1000, 50), (1000, 8186, 4093), (9188, 10000, 5000)]).compress_launches == 4


def test_plan_flags_rejected_before_any_device_call():
    L = A.lib()
    arr, n = A._segments([(0, 1000, 50)])
    h = ctypes.c_void_p()
    # both finish flags together, with or without the decode flag; unknown bits
    for flags in (3, 7, 8, 12, 0x80000000):
        assert L.adacomp_plan_create_ex(arr, n, flags, ctypes.byref(h)) == -1
        assert h.value is None


def test_null_plan_calls_fail_cleanly():
    L = A.lib()
    assert L.adacomp_compress(None, None, None, 0, None, 0, None, 0, None, None) == -1
    assert L.adacomp_decode_accumulate(None, None, 0, None, 0, 0, None, 0, None) == -1
    assert L.adacomp_plan_destroy(None) == -1
    assert L.adacomp_plan_get_info(None, None) == -1


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(A, "LIB_PATH", ROOT / "nonexistent" / "libadacomp.so")
    monkeypatch.setattr(A, "_lib", None)
    with pytest.raises(A.HipLibraryMissing):
        A.plan_query([(0, 100, 50)])


# --------------------------------------------------------------------------
# Tile geometry, checked on the CPU with the library's own layout code.
# --------------------------------------------------------------------------

EDGE_BINS = [1, 2, 3, 4, 5, 7, 8, 50, 63, 64, 65, 127, 500, 1000, 1021, 1022, 1023, 4093, 4094, 4095,
             4096, 5000, 8191, 32765, 32766, 32767, 32768]
EDGE_NUMEL = [1, 2, 3, 4, 5, 7, 63, 64, 65, 4093, 4096, 4097, 36861, 65537, 100003]


def geometry_tables():
    tables = [(wl.segments, 0) for wl in (W.workload(n) for n in W.WORKLOADS)]
    for lt in EDGE_BINS:
        segs, off = [], 0
        for n in EDGE_NUMEL:
            segs.append((off, n, lt))
            off += (n + 3) // 4 * 4 + 4
        tables.append((segs, 0))
    rng = random.Random(5)
    for _ in range(40):
        segs, off = [], 0
        for _ in range(rng.randint(1, 12)):
            n = rng.choice([rng.randint(1, 80), rng.randint(1, 20000), rng.randint(1, 300000)])
            lt = rng.choice([rng.randint(1, 70), rng.randint(1, 5000), rng.randint(4000, 32768)])
            segs.append((off, n, lt))
            off += (n + 3) // 4 * 4 + 4 * rng.randint(0, 3)
        tables.append((segs, 0))
    tables.append(([(0, 100, 0)], -2))
    tables.append(([(0, 10, 50), (4, 10, 50)], -4))
    return tables


def test_tile_geometry_on_cpu(tmp_path):
    exe = tmp_path / "geometry_check"
    # built with the address and undefined-behaviour sanitizers: any access
    # of the layout code outside its vectors, or an overflow, ends the run
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-o", str(exe),
                    str(ROOT / "tests" / "cpu" / "geometry_check.cpp")], check=True)
    tables = geometry_tables()
    lines = []
    for segs, expect in tables:
        lines.append(f"{len(segs)} {expect}")
        lines += [f"{o} {n} {lt}" for o, n, lt in segs]
    inp = tmp_path / "tables.txt"
    inp.write_text("\n".join(lines) + "\n")
    r = subprocess.run([str(exe), str(inp)], capture_output=True, text=True)
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    out = r.stdout.strip().splitlines()
    assert len(out) == len(tables), r.stderr
    fails = [(i, l) for i, l in enumerate(out) if not l.startswith("OK")]
    assert not fails, fails[:5]
    assert r.returncode == 0


def test_header_is_plain_c_and_host_calls_work(tmp_path):
    """include/adacomp.h compiles as C99 with warnings as errors, and a plain
    C program linked against the library makes the host-only calls (plan
    query, argument errors, status strings, an empty timer) without a GPU."""
    exe = tmp_path / "c_abi_check"
    lib_dir = ROOT / "adaptive_residual_gradient_amd"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-o", str(exe),
                    str(ROOT / "tests" / "cpu" / "c_abi_check.c"), f"-L{lib_dir}", "-ladacomp",
                    f"-Wl,-rpath,{lib_dir}"], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "OK host-only calls" in out.stdout


def test_bench_refuses_several_gpus():
    """The benchmark measures one GPU: asked for more it prints one JSON line
    saying so and exits with status 2, before touching any device."""
    import json
    import sys
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]
