"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, CPU only): every entry point runs on the hand-worked cases, seeded
small sets and edge cases (empty input, one point, duplicates with eps = 0,
NaN and infinite coordinates, bad eps and MinPts, 64 dimensions, subnormal
scales, both distance forms).  The run must end without a sanitizer
report, and every value it writes must equal the regular oracle build's."""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
import pins
from all_pairs_distance_amd import datagen

ORACLE_DIR = os.path.dirname(os.path.abspath(oracle.__file__))
SAN_FLAGS = ["-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-Wall"]

OP_FIT, OP_GRAPH, OP_ROWS, OP_NEIGHBOURS, OP_DIST = 1, 2, 3, 4, 5
FORMS = ("direct", "expanded")


def _cases():
    out = []
    for cid, pts, eps, m, _, _ in pins.load_handworked():
        out.append((cid, pts, eps, m))
    for t, (x, eps, m) in enumerate(pins.small_cases(seed=41, count=24)):
        out.append((f"small{t}", x, eps, m))
    rng = np.random.default_rng(5)
    u = datagen.uniform_points(40, 3, 17)
    out.append(("empty", np.zeros((0, 2), np.float32), 0.1, 1))
    out.append(("one_point", np.array([[0.5, 0.5]], np.float32), 0.1, 1))
    dup = np.ascontiguousarray(u[rng.integers(0, 40, 120)])
    out.append(("duplicates_eps0", dup, 0.0, 2))
    nan = u.copy()
    nan[7, 1] = np.nan
    out.append(("nan_coordinate", nan, 0.2, 3))
    inf = u.copy()
    inf[3, 0] = np.inf
    out.append(("inf_coordinate", inf, 0.2, 3))
    out.append(("eps_nan", u, float("nan"), 3))
    out.append(("eps_negative", u, -0.5, 3))
    out.append(("minpts_zero", u, 0.2, 0))
    out.append(("d64", datagen.gaussian_blobs(150, 64, seed=3, n_blobs=3,
                                               sigma=0.05, noise_frac=0.1),
                0.4, 4))
    tiny = (datagen.uniform_points(60, 2, 6) * np.float32(1e-38)).astype(np.float32)
    out.append(("subnormal_scale", tiny, 2e-39, 2))
    return out


def _record(op, form, x, eps, m):
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x.reshape(-1, 1)
    n, d = x.shape
    head = np.zeros(1, dtype=[("op", "<i4"), ("form", "<i4"), ("n", "<i8"),
                              ("d", "<i4"), ("eps", "<f4"), ("m", "<i4"),
                              ("reserved", "<i4")])
    head[0] = (op, form, n, d, np.float32(eps), m, 0)
    return head.tobytes() + x.astype("<f4").tobytes()


class Reader:
    def __init__(self, data: bytes):
        self.b, self.o = data, 0

    def take(self, dtype, count):
        dt = np.dtype(dtype)
        a = np.frombuffer(self.b, dtype=dt, count=count, offset=self.o)
        self.o += dt.itemsize * count
        return a

    def i64(self):
        return int(self.take("<i8", 1)[0])


@pytest.fixture(scope="module")
def sanitized_binary():
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not available")
    tmp = tempfile.mkdtemp(prefix="oracle_san_")
    exe = os.path.join(tmp, "sanitize_check")
    cmd = ["gcc", *SAN_FLAGS, "-o", exe,
           os.path.join(ORACLE_DIR, "oracle.c"),
           os.path.join(ORACLE_DIR, "sanitize_check.c"), "-lm"]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0 and "sanitizer" in p.stderr.lower():
        pytest.skip("this gcc cannot build sanitizer binaries: " + p.stderr[-500:])
    assert p.returncode == 0, p.stderr
    yield exe, tmp
    shutil.rmtree(tmp, ignore_errors=True)


def test_oracle_clean_under_asan_and_ubsan(sanitized_binary, orc):
    exe, tmp = sanitized_binary
    cases = _cases()
    plan = []
    blob = bytearray()
    for cid, x, eps, m in cases:
        for form in (0, 1):
            for op in (OP_FIT, OP_GRAPH, OP_ROWS, OP_NEIGHBOURS):
                plan.append((cid, op, form, x, eps, m))
                blob += _record(op, form, x, eps, m)
        plan.append((cid, OP_DIST, 0, x, eps, m))
        blob += _record(OP_DIST, 0, x, eps, m)
    cases_path = os.path.join(tmp, "cases.bin")
    out_path = os.path.join(tmp, "results.bin")
    with open(cases_path, "wb") as f:
        f.write(bytes(blob))
    env = dict(os.environ, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="abort_on_error=0:halt_on_error=1:detect_leaks=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    p = subprocess.run([exe, cases_path, out_path], capture_output=True,
                       text=True, env=env, timeout=600)
    assert p.returncode == 0, p.stderr[-4000:]
    assert "runtime error" not in p.stderr, p.stderr[-4000:]
    assert "Sanitizer" not in p.stderr, p.stderr[-4000:]

    r = Reader(open(out_path, "rb").read())
    checked = 0
    for cid, op, form, x, eps, m in plan:
        x = np.ascontiguousarray(x, dtype=np.float32)
        if x.ndim == 1:
            x = x.reshape(-1, 1)
        n = x.shape[0]
        name = FORMS[form]
        if op == OP_FIT:
            st = r.i64()
            try:
                want_l, want_c, _ = orc.fit(x, eps, m, form=name)
            except oracle.OracleError as e:
                assert st == e.status, (cid, name, st)
                continue
            assert st == 0, (cid, name, st)
            assert np.array_equal(r.take("<i4", n), want_l), (cid, name)
            assert np.array_equal(r.take("<i4", n), want_c), (cid, name)
            k = r.i64()
            ids, sizes, want_k = orc.relabel(want_l)
            assert k == want_k, cid
            assert np.array_equal(r.take("<i4", n), ids), cid
            assert np.array_equal(r.take("<i4", k), sizes), cid
        elif op == OP_GRAPH:
            nnz = r.i64()
            try:
                want_rp, want_ci = orc.graph(x, eps, form=name)
            except oracle.OracleError as e:
                assert nnz == e.status, (cid, name, nnz)
                continue
            assert nnz == want_ci.size, (cid, name)
            assert np.array_equal(r.take("<i8", n + 1), want_rp), (cid, name)
            assert np.array_equal(r.take("<i4", nnz), want_ci), (cid, name)
        elif op == OP_ROWS:
            st = r.i64()
            try:
                want = orc.row_counts(x, eps, np.arange(n), form=name)
            except oracle.OracleError as e:
                assert st == e.status, (cid, name, st)
                continue
            assert st == 0, (cid, name, st)
            assert np.array_equal(r.take("<i4", n), want), (cid, name)
        elif op == OP_NEIGHBOURS:
            for i in range(min(n, 8)):
                c = r.i64()
                try:
                    want = orc.row_neighbours(x, eps, i, form=name)
                except oracle.OracleError as e:
                    assert c == e.status, (cid, name, i)
                    continue
                assert c == want.size, (cid, name, i)
                if c > 0:
                    got = r.take("<i8", min(c, 4))
                    assert np.array_equal(got, want[:4]), (cid, name, i)
        else:
            e2 = r.take("<f4", 1)[0]
            assert e2.tobytes() == orc.eps2(eps).tobytes(), cid
            for i in range(1, n):
                a, b = r.take("<f4", 2)
                assert a.tobytes() == orc.d2(x[0], x[i]).tobytes(), (cid, i)
                assert b.tobytes() == orc.d2_expanded(x[0], x[i]).tobytes(), (cid, i)
        checked += 1
    assert r.o == len(r.b), "unread results"
    assert checked > 200


def test_sanitizer_catches_a_planted_overflow(sanitized_binary, tmp_path):
    """A copy of the oracle whose core-flag array is one byte short must
    make the sanitized run fail: the check above is armed."""
    exe, _ = sanitized_binary
    src = open(os.path.join(ORACLE_DIR, "oracle.c")).read()
    needle = "uint8_t* core = (uint8_t*)malloc((size_t)n);"
    assert needle in src
    bad_src = tmp_path / "oracle.c"
    bad_src.write_text(src.replace(
        needle, "uint8_t* core = (uint8_t*)malloc((size_t)n - 1);"))
    shutil.copy(os.path.join(ORACLE_DIR, "oracle.h"), tmp_path / "oracle.h")
    bad_exe = str(tmp_path / "sanitize_check_bad")
    p = subprocess.run(["gcc", *SAN_FLAGS, "-o", bad_exe, str(bad_src),
                        os.path.join(ORACLE_DIR, "sanitize_check.c"),
                        f"-I{tmp_path}", "-lm"], capture_output=True, text=True)
    assert p.returncode == 0, p.stderr
    x = datagen.uniform_points(50, 2, 3)
    cases = tmp_path / "cases.bin"
    cases.write_bytes(_record(OP_FIT, 0, x, 0.2, 3))
    p = subprocess.run([bad_exe, str(cases), str(tmp_path / "out.bin")],
                       capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, OMP_NUM_THREADS="2"))
    assert p.returncode != 0
    assert "AddressSanitizer" in p.stderr
