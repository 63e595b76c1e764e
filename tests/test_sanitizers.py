"""The recurrent oracle and the host side of the C ABI built with
AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The oracle build runs the edge-case shapes under every merge and routing
metric, with the branch partials and two threads, and must give the same
bits as the regular build. The ABI build runs the host paths: parameter
derivation, sizes, the state layout, status strings and the argument
checks made before any device call. Any sanitizer report fails the run.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import rec

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _gcc_has_sanitizers(tmp):
    src = os.path.join(tmp, "probe.c")
    with open(src, "w") as f:
        f.write("int main(void){return 0;}\n")
    r = subprocess.run(["gcc"] + SAN + [src, "-o", os.path.join(tmp, "probe")],
                       capture_output=True)
    return r.returncode == 0


@pytest.fixture(scope="module")
def oracle_exe(tmp_path_factory):
    tmp = str(tmp_path_factory.mktemp("san_oracle"))
    if not _gcc_has_sanitizers(tmp):
        pytest.skip("gcc without the sanitizer runtimes")
    exe = os.path.join(tmp, "oracle_san")
    subprocess.run(["gcc", "-O1", "-g", "-ffp-contract=off", "-pthread"] + SAN +
                   [os.path.join(ROOT, "oracle", "still_oracle.c"),
                    os.path.join(HERE, "sanitize", "oracle_driver.c"), "-o", exe, "-lm"],
                   check=True)
    return exe


def _run_sanitized(exe, tmp, U, G, L, d, W, C, m, tm, merge, route, partials, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((U, G, L, d)).astype(np.float32)
    k = rng.standard_normal((U, L, d)).astype(np.float32)
    v = rng.standard_normal((U, L, d)).astype(np.float32)
    F = (rng.standard_normal((U, d, d)) / np.sqrt(d)).astype(np.float32)
    g = rng.uniform(0, 1, (U, G)).astype(np.float32)
    ext = rng.uniform(0, 1, (U, L)).astype(np.float32)
    eps, scale = 1e-6, 1 / np.sqrt(d)
    inp, out = os.path.join(tmp, "in.bin"), os.path.join(tmp, "out.bin")
    with open(inp, "wb") as f:
        np.array([U, L, d, G, W, C, m, tm, rec.MERGES[merge], rec.ROUTES[route], int(partials), 2],
                 np.int32).tofile(f)
        np.array([eps, scale], np.float64).tofile(f)
        for a in (q, k, v, F, g, ext):
            a.tofile(f)
    r = subprocess.run([exe, inp, out], capture_output=True, text=True, env=ENV)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    want = rec.run_units(q, k, v, F, g, window=W, chunk=C, budget=m, t_max=tm, eps=eps,
                         sm_scale=scale, n_threads=2, merge=merge, partials=partials,
                         route=route, ext=ext)
    lam, n_dec = want["lam"], want["n_dec"]
    buf = open(out, "rb").read()
    pos = 0

    def take(n, dt):
        nonlocal pos
        a = np.frombuffer(buf, dt, n, pos)
        pos += a.nbytes
        return a
    assert take(1, np.int32)[0] == 0
    names = [("y", U * G * L * d, np.float64), ("score", U * L, np.float64),
             ("S", U * d * d, np.float64), ("z", U * d, np.float64),
             ("pending", U * C, np.float64), ("sel", U * n_dec * lam, np.int32),
             ("n_pool", U, np.int32)]
    if partials:
        names += [("y_sa", U * G * L * d, np.float64), ("y_la", U * G * L * d, np.float64),
                  ("lse_sa", U * G * L, np.float64), ("lse_la", U * G * L, np.float64)]
    for name, n, dt in names:
        got = take(n, dt)
        np.testing.assert_array_equal(got, want[name].reshape(-1), err_msg=name)
    assert pos == len(buf)


CASES = [
    # (U, G, L, d, W, C, m, t_max)
    (2, 2, 61, 8, 8, 8, 8 + 14, 7),
    (1, 3, 77, 8, 6, 8, 6 + 8, 2),     # the budget fills
    (2, 1, 45, 16, 11, 4, 11 + 24, 6),  # W > C, lambda = C
    (1, 2, 1, 8, 4, 8, 12, 1),          # one token
    (1, 2, 9, 8, 2, 8, 12, 1),          # one decided chunk
]


@pytest.mark.parametrize("case", CASES)
def test_oracle_under_sanitizers(oracle_exe, tmp_path, case):
    U, G, L, d, W, C, m, tm = case
    for i, (merge, route) in enumerate([("one", "saliency"), ("sum", "diag"),
                                        ("softmax_only", "qk"), ("one", "keynorm"),
                                        ("sum", "uniform"), ("one", "external")]):
        _run_sanitized(oracle_exe, str(tmp_path), U, G, L, d, W, C, m, tm, merge, route,
                       partials=i % 2 == 0, seed=sum(case) + i)


def test_abi_host_paths_under_sanitizers(tmp_path):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    clangxx = "/opt/rocm/llvm/bin/clang++"
    if not (shutil.which(hipcc) and os.path.exists(clangxx)):
        pytest.skip("no hipcc")
    tmp = str(tmp_path)
    inc = ["-I", os.path.join(ROOT, "include")]
    csrc = os.path.join(ROOT, "linear_attention_still_amd", "csrc")
    # host code instrumented, device code built as usual (-Xarch_host keeps
    # the sanitizers off the gfx950 pass)
    host_san = []
    for flag in SAN:
        host_san += ["-Xarch_host", flag]
    subprocess.run([hipcc, "--offload-arch=gfx950", "-c", "-O1", "-g", "-std=c++17", "-fPIC",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + host_san +
                   inc + ["-I", csrc, os.path.join(csrc, "still_api.hip"), "-o",
                          os.path.join(tmp, "api.o")], check=True, capture_output=True)
    subprocess.run(["gcc", "-c", "-O1", "-g"] + SAN + inc +
                   [os.path.join(HERE, "sanitize", "abi_driver.c"), "-o",
                    os.path.join(tmp, "drv.o")], check=True)
    exe = os.path.join(tmp, "abi_san")
    subprocess.run([clangxx] + SAN + [os.path.join(tmp, "drv.o"), os.path.join(tmp, "api.o"),
                                      "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64",
                                      "-o", exe], check=True)
    # the HIP runtime keeps process-lifetime allocations of its own
    env = dict(ENV, ASAN_OPTIONS="detect_leaks=0")
    r = subprocess.run([exe], capture_output=True, text=True, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-4000:]
    assert "all checks passed" in r.stdout
