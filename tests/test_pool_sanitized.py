"""The page allocator (pool.cpp) built for the host with AddressSanitizer and UndefinedBehaviorSanitizer,
driven through random grow/free traffic, exhaustion, double frees, repeated and foreign page ids; every
step's status, free count and block-table row must equal the oracle allocator's ("为什么要自己动手写一个LLM
推理引擎" §3.4: pages handed out from a free list and returned when a request ends), and the sanitizers
must report nothing."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import pages as op

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kv_cached_transformer_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no g++")
    out = str(tmp_path_factory.mktemp("pool_san") / "pool_driver")
    srcs = [os.path.join(CSRC, "pool.cpp"), os.path.join(CSRC, "errors.cpp"),
            os.path.join(ROOT, "tests", "native", "pool_driver.cpp")]
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-Wall", "-Werror", *SAN, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *srcs, "-o", out]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


def script_and_expected(seed):
    """A random script and the oracle's line for every step."""
    r = np.random.default_rng(seed)
    num_pages, max_pages, n_seq = int(r.integers(8, 48)), int(r.integers(2, 10)), int(r.integers(1, 7))
    order = r.permutation(num_pages).tolist()
    ref = op.PagePool(num_pages, order)
    lines = [f"create {num_pages} " + " ".join(map(str, order))]
    exp = [f"create 0 free {num_pages}"]
    rows = {}
    for _ in range(300):
        u = r.random()
        s = int(r.integers(n_seq))
        if s in rows and u < 0.15:                                   # a request ends
            row, npg, _ = rows.pop(s)
            lines.append(f"free {s}")
            exp.append(f"free {ref.free(row[:npg])} free {ref.n_free}")
        elif u < 0.25:                                               # error cases: nothing may change
            held = [p for row, npg, _ in rows.values() for p in row[:npg]]
            free_ids = [p for p in range(num_pages) if p not in held]
            kind = r.integers(4)
            if kind == 0:
                ids = [int(r.choice([-1, num_pages, num_pages + 7, -100]))]   # foreign ids
            elif kind == 1 and free_ids:
                ids = [int(r.choice(free_ids))]                                # already free (double free)
            elif kind == 2 and held:
                p = int(r.choice(held))
                ids = [p, p]                                                   # listed twice
            elif held:
                ids = [int(r.choice(held)), int(r.choice([num_pages, -1]))]   # valid id then a bad one
            else:
                ids = [-5]
            lines.append(f"raw {len(ids)} " + " ".join(map(str, ids)))
            st = ref.free(ids)
            assert st == op.E_INVALID
            exp.append(f"raw {st} free {ref.n_free}")
        else:                                                        # grow, sometimes past the row or the pool
            row, npg, toks = rows.get(s, ([-1] * max_pages, 0, 0))
            want = toks + int(r.integers(0, 60))
            st, n_new = ref.alloc(want, row, npg, max_pages)
            lines.append(f"alloc {s} {want} {max_pages}")
            exp.append(f"alloc {st} free {ref.n_free} row " + " ".join(map(str, row)))
            rows[s] = (row, n_new, want if st == op.OK else toks)
    lines.append("end")
    return "\n".join(lines) + "\n", exp


@pytest.mark.parametrize("seed", range(12))
def test_pool_under_sanitizers_matches_oracle(driver, seed):
    script, exp = script_and_expected(seed)
    res = subprocess.run([driver], input=script, capture_output=True, text=True, timeout=60,
                         env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0",
                              "UBSAN_OPTIONS": "print_stacktrace=1"})
    assert res.returncode == 0, res.stderr[-3000:]
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr[-3000:]
    got = res.stdout.strip().splitlines()
    assert len(got) == len(exp)
    for i, (g, e) in enumerate(zip(got, exp)):
        assert g == e, f"step {i}: allocator {g!r}, oracle {e!r}"
