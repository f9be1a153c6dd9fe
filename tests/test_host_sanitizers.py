"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer: the library's host-only source (the
deficit admission) is built with g++ -fsanitize=address,undefined together with a driver
(tests/native/admission_driver.cpp) and run over the golden trace and seeded random traces (decode
work above the budget included) and over calls with invalid arguments.  Any sanitizer report fails
the run; every output must equal the oracle's."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import admission
from tests.test_oracle_admission import random_case, read_trace

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path_factory.mktemp("san") / "admission_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", f"-I{ROOT}/include", f"{ROOT}/tests/native/admission_driver.cpp",
           f"{ROOT}/denoise_step_amd/csrc/admission.cpp", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr + r.stdout).lower():
        pytest.skip(f"sanitizer runtime unavailable: {r.stderr[-300:]}")
    assert r.returncode == 0, r.stderr
    return exe


def run(exe, traces):
    lines = [str(len(traces))]
    for budget, decode, arrivals in traces:
        lines.append(f"{budget} {len(decode)} {len(arrivals)}")
        lines.append(" ".join(str(int(x)) for x in decode))
        lines += [f"{int(t)} {int(s)}" for t, s in arrivals]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-2000:]
    return r.stdout.split("\n")


def test_admission_under_sanitizers_matches_oracle(driver):
    budget, arrivals, iters = read_trace()
    traces = [(budget, [it[0] for it in iters], arrivals)]
    rng = np.random.default_rng(900)
    traces += [random_case(rng, n_iter=120, n_pf=25) for _ in range(25)]
    traces.append((5, [9] * 30, [(0, 3), (2, 40), (2, 1)]))   # decode work above the budget every iteration
    out = run(driver, traces)
    i = 0
    for budget, decode, arrivals in traces:
        ref = admission.simulate(budget, decode, arrivals)
        for t in range(len(decode)):
            pid, d, tok = (int(x) for x in out[i].split())
            i += 1
            assert pid == (ref.admitted[t][0] if ref.admitted[t] else -1), (budget, t)
            assert (d, tok) == (ref.deficit[t], ref.tokens[t]), (budget, t)
    assert [out[i + k] for k in range(7)] == ["status -1"] * 7
    assert out[i + 7] == "untouched 7 11 9"
    assert out[i + 8] == f"null_tokens 0 1 0"
