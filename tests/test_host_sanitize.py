"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer,
on the CPU.

api.hip and host_layout.hip hold all of the host logic: argument
validation, the GEMM and attention planners, the workspace layout, COD
sampling and the sequence partition.  They are rebuilt with host-side
sanitizers (device code untouched), linked with the library's other objects
into tests/sanitize/host_driver.cpp, and fed the cases of test_host_layout
and test_abi_cpu plus seeded sweeps of shapes and of malformed row lists.
Every answer must equal the regular library's (and, for COD rows and
partitions, the oracle's), with no sanitizer report.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from drafting_eagle_draft_amd import binding as pe
from drafting_eagle_draft_amd import build as libbuild
from drafting_eagle_draft_amd import synth
from oracle import peagle_oracle as po

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "sanitize", "host_driver.cpp")
HOST_SOURCES = ("api.hip", "host_layout.hip")

pytestmark = pytest.mark.skipif(
    not (os.path.exists(pe.LIB_PATH) and os.path.isdir(libbuild.OBJDIR) and shutil.which(libbuild.HIPCC)),
    reason="library objects not built (run __graft_entry__.build())")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{cmd[0]} failed:\n{r.stdout}\n{r.stderr}"
    return r


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    out = tmp_path_factory.mktemp("sanitized")
    host_san = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer", "-g", "-O1"):
        host_san += ["-Xarch_host", f]
    objs = []
    for src in HOST_SOURCES:
        obj = str(out / (src + ".o"))
        _run([libbuild.HIPCC, *libbuild.DEVICE_FLAGS, *host_san, "-c", os.path.join(libbuild.CSRC, src), "-o", obj])
        objs.append(obj)
    others = sorted(os.path.join(libbuild.OBJDIR, f) for f in os.listdir(libbuild.OBJDIR)
                    if f.endswith(".hip.o") and f[:-2] not in HOST_SOURCES)
    dobj = str(out / "host_driver.o")
    _run([libbuild.HIPCC, "-x", "hip", "--offload-arch=" + libbuild.ARCH, "-std=c++17", *host_san,
          "-I", os.path.join(libbuild.ROOT, "include"), "-c", DRIVER, "-o", dobj])
    exe = str(out / "host_driver")
    # Link line: host sanitizer runtimes only (no -Xarch_ option here).
    _run([libbuild.HIPCC, "--offload-arch=" + libbuild.ARCH, "-fsanitize=address,undefined", "-fno-gpu-sanitize",
          dobj, *objs, *others, "-o", exe])
    return exe


def _drive(exe, script):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], input="\n".join(script) + "\n", capture_output=True, text=True, env=env,
                       timeout=300)
    report = [l for l in r.stderr.splitlines() if "AddressSanitizer" in l or "runtime error" in l
              or "LeakSanitizer" in l]
    assert r.returncode == 0 and not report, f"exit {r.returncode}\n{r.stderr[-4000:]}"
    lines = r.stdout.split("\n")
    answers = []
    for i in range(len(script)):
        vals = [int(x) for x in lines[2 * i].split()]
        answers.append((vals[0], vals[1:], lines[2 * i + 1]))
    return answers


def _expect(fn, *args):
    """(status, value, message) of the regular library."""
    try:
        return pe.PE_OK, fn(*args), ""
    except pe.PeagleError as e:
        return e.status, None, e.message


def _ints(a):
    return " ".join(str(int(x)) for x in a)


def test_cod_rows_and_partitions_sanitized(driver):
    script, want = [], []
    cfg = synth.config("tiny_f32")
    cod_cases = [(1, 1, 0.8, 0.2), (5, 8, 0.8, 0.2), (64, 8, 0.8, 0.2), (300, 6, 0.7, 0.2),
                 (257, 16, 0.8, 0.2), (97, 5, 0.5, 0.3), (40, 4, 1.0, 0.0), (4, 17, 0.8, 0.2),
                 (0, 4, 0.8, 0.2), (8192, 8, 0.8, 0.2)]
    kept = []
    for n, K, r, fl in cod_cases:
        U = synth.cod_uniforms(cfg, n, K, tag=f"san{n}_{K}") if n * K and K <= 16 else np.zeros(max(n * K, 0))
        script.append(f"cod {n} {K} {r!r} {fl!r} " + " ".join(repr(float(u)) for u in U.reshape(-1)))
        st, rows, msg = _expect(pe.pe_cod_rows, n, K, r, fl, U.reshape(-1))
        if st == pe.PE_OK:
            np.testing.assert_array_equal(rows, po.cod_rows(po.cod_keep(n, K, U.reshape(n, K), r=r, floor=fl)))
            kept.append((n, K, rows))
        want.append((st, None if rows is None else rows.tolist(), msg))
    # Valid partitions of the sampled rows, every chunk of each, and
    # malformed row lists (unsorted, repeated, out of range, negative,
    # missing parents or depth-0 cells).
    rng = np.random.default_rng(2024)
    part_inputs = []
    for n, K, rows in kept:
        if n > 400:
            continue
        for S in (1, 2, 3, max(1, n // 2), n, n + 1):
            part_inputs.append((n, K, S, rows))
    for _ in range(60):
        n, K = int(rng.integers(1, 12)), int(rng.integers(1, 6))
        L = int(rng.integers(1, 2 * n * K + 2))
        rows = rng.integers(-2, n * K + 3, L).astype(np.int32)
        if rng.random() < 0.5:
            rows = np.unique(rows)
        part_inputs.append((n, K, int(rng.integers(0, n + 2)), rows))
    for n, K, S, rows in part_inputs:
        script.append(f"part {n} {K} {S} {len(rows)} {_ints(rows)}")
        st, chunk, msg = _expect(pe.pe_partition, n, K, S, rows)
        if st == pe.PE_OK and S <= n and np.all(np.diff(rows) > 0) and rows.min() >= 0:
            want_chunk, _, _ = po.partition(n, K, S, rows)
            np.testing.assert_array_equal(chunk, want_chunk)
        want.append((st, None if chunk is None else chunk.tolist(), msg))
        for s in range(-1, min(S, 4) + 1):
            script.append(f"chunk {n} {K} {S} {s} {len(rows)} {_ints(rows)}")
            st, res, msg = _expect(pe.pe_partition_chunk, n, K, S, s, rows)
            if res is not None:
                cells, lead, out_rows, nc = res
                res = [len(cells), lead, nc, *cells.tolist(), *out_rows.tolist()]
            want.append((st, res, msg))
    got = _drive(driver, script)
    for i, ((gs, gv, gm), (ws, wv, wm)) in enumerate(zip(got, want)):
        assert gs == ws and gm == wm, (script[i][:80], gs, gm, ws, wm)
        if ws == pe.PE_OK:
            assert gv == wv, script[i][:80]


def test_shape_planning_and_validation_sanitized(driver):
    rng = np.random.default_rng(7)
    script, want = [], []
    shapes = [(4096, 1, 32, 8, 128, 14336, 128256, 1, B, K, 8192, cus)
              for B, K in [(1, 1), (2, 8), (4, 8), (8, 8), (4, 16), (63, 1), (8, 9)] for cus in (256, 80)]
    shapes += [(4096, 1, 32, 8, 128, 65536, 128256, 1, 8, 8, 4096, 256),
               (4096, 1, 32, 8, 128, 14336, 128256, 1, 2, 8, 1 << 22, 256),
               (4096, 1, 32, 8, 128, 14336, 128256, 1, 2, 8, 1 << 23, 256),
               (2880, 1, 64, 8, 64, 2880, 201088, 1, 2, 8, 4096, 256)]
    for _ in range(400):
        hd = int(rng.choice([64, 128, 96, 0]))
        nkv = int(rng.choice([1, 2, 4, 8, 0, -1]))
        nq = nkv * int(rng.choice([1, 2, 4, 8, 3])) if nkv > 0 else int(rng.integers(-1, 9))
        H = int(rng.choice([64, 128, 256, 1000, 2880, 4096, 8192, 16384, -16]))
        I = int(rng.choice([256, 1024, 2880, 14336, 28672, 65536, 1 << 20, 12]))
        V = int(rng.choice([4096, 32000, 128256, 201088, 1 << 24, 4095]))
        dtype = int(rng.choice([0, 1, 1, 3]))
        B = int(rng.choice([int(rng.integers(-1, 66)), 1 << 30, (1 << 31) - 1, -(1 << 31)]))
        K = int(rng.choice([int(rng.integers(-1, 18)), (1 << 31) - 1]))
        stride = int(rng.choice([-1, 0, 1, 63, 4096, 16384, 1 << 22, 1 << 23, 1 << 40, (1 << 62) + 1]))
        cus = int(rng.choice([-4, 0, 1, 8, 80, 256, 1 << 20]))
        shapes.append((H, 1, nq, nkv, hd, I, V, dtype, B, K, stride, cus))
    for s in shapes:
        script.append("shape " + " ".join(str(x) for x in s))
        H, nl, nq, nkv, hd, I, V, dt, B, K, stride, cus = s
        cfg = pe.PeConfig(hidden=H, n_layers=nl, n_q_heads=nq, n_kv_heads=nkv, head_dim=hd, intermediate=I,
                          vocab=V, rope_theta=5e5, rms_eps=1e-5, dtype=dt)
        st, _, msg = _expect(pe.pe_draft_shape_check, cfg, B, K, stride, cus)
        want.append((st, [], msg))
    # Model creation: every configuration is rejected before a weight is read.
    creates = [(256, 1, 6, 4, 64, 1024, 4096, 5e5, 0, 0), (256, 1, 4, 2, 96, 1024, 4096, 5e5, 0, 0),
               (256, 1, 4, 2, 64, 1024, 4096, 5e5, 7, 0), (256, 1, 4, 2, 64, 1024, 4095, 5e5, 0, 0),
               (64, 1, 4, 2, 64, 1024, 4096, 5e5, 0, 0), (256, 1, 4, 2, 128, 1024, 4096, 5e5, 0, 0),
               (256, 1, 4, 2, 64, 1024, 4096, 0.0, 0, 0), (256, 1, 4, 2, 64, 1024, 4096, 5e5, 0, 1 << 8),
               (256, 1, 4, 2, 64, 1024, 4096, 5e5, 0, 1 << 9), (256, 3, 4, 2, 64, 1024, 4096, 5e5, 0, 1 << 2),
               (256, 0, 4, 2, 64, 1024, 4096, 5e5, 0, 1 << 9), (256, -1, 4, 2, 64, 1024, 4096, 5e5, 0, 0)]
    for c in creates:
        script.append("create " + " ".join(repr(x) for x in c))
        H, nl, nq, nkv, hd, I, V, th, dt, bits = c
        cfg = pe.PeConfig(hidden=H, n_layers=nl, n_q_heads=nq, n_kv_heads=nkv, head_dim=hd, intermediate=I,
                          vocab=V, rope_theta=th, rms_eps=1e-5, dtype=dt)
        layers = (pe.PeLayerWeights * max(nl, 1))(
            *[pe.PeLayerWeights(*[0 if (bits >> i) & 1 else 16 for i in range(9)]) for _ in range(max(nl, 1))])
        w = pe.PeWeights(0 if (bits >> 9) & 1 else 16, 16, 16, 16, layers)
        st, _, msg = _expect(pe.pe_model_create, cfg, w, 0)
        assert st != pe.PE_OK
        want.append((st, [], msg))
    for B, K, nd in [(-1, 4, 0), (2, 0, 0), (2, 17, 0), (3, 4, 1), (0, 4, 1)]:
        script.append(f"accept {B} {K} {nd}")
        st, _, msg = _expect(pe.pe_accept, B, K, 0 if nd else 16, 16 if B else 0, 16 if B else 0, None, 0)
        want.append((st, [], msg))
    for n_max, K in [(0, 8), (16, 0), (16, 17), (1 << 22, 8), (-5, 4)]:
        script.append(f"mask {n_max} {K}")
        st, _, msg = _expect(pe.pe_mask_create, n_max, K, 0)
        assert st != pe.PE_OK
        want.append((st, [], msg))
    script += ["nullmodel", "version"]
    got = _drive(driver, script)
    for i, ((gs, gv, gm), (ws, wv, wm)) in enumerate(zip(got[:len(want)], want)):
        assert gs == ws and gm == wm, (script[i], gs, gm, ws, wm)
    nullmodel, version = got[len(want):]
    assert all(x == pe.PE_ERR_INVALID_ARGUMENT for x in nullmodel[1]), nullmodel
    assert version[1][0] == len(pe.pe_version())
