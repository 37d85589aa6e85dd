"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

1. oracle.c built with gcc -fsanitize=address,undefined: every oracle routine
   runs on small inputs in a subprocess with the sanitizer runtime preloaded,
   and must give the same values as the normal build.
2. The ABI layer's host code (tpshard_api.cpp) built with hipcc, -Xarch_host
   before each -fsanitize= so only the host side is instrumented, linked with
   the normal device objects: the ABI validation tests (tests/test_abi_cpu.py,
   which launch nothing) run against it in a subprocess with clang's
   sanitizer runtime preloaded.
Any sanitizer report aborts the subprocess (halt_on_error), failing the test.
"""
import glob
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.slow

ORACLE_CALLS = r"""
import numpy as np, sys
sys.path.insert(0, sys.argv[1])
import oracle as O
g = np.random.default_rng(0)
X, W1, W2, dY = g.standard_normal((9, 12)), g.standard_normal((12, 7)), g.standard_normal((7, 12)), g.standard_normal((9, 12))
out = {}
for a in ("relu", "gelu"):
    out["mlp_" + a] = np.concatenate([x.ravel() for x in O.mlp_fwd(a, X, W1, W2) + O.mlp_bwd(a, X, W1, W2, dY)])
Wg, Wu, Wd = g.standard_normal((12, 5)), g.standard_normal((12, 5)), g.standard_normal((5, 12))
out["swiglu"] = np.concatenate([x.ravel() for x in O.swiglu_fwd(X, Wg, Wu, Wd) + O.swiglu_bwd(X, Wg, Wu, Wd, dY)])
out["sampled"] = np.concatenate([x.ravel() for x in O.mlp_bwd_sampled("gelu", X, W1, W2, dY, [0, 8], [1, 6], [0, 3])])
z = g.standard_normal((6, 11)); t = np.array([0, 10, 3, -1, 11, 5])
m, se, tl = O.ce_stats(z, t, 0)
M, S = O.ce_global([m], [se])
out["ce"] = np.concatenate([m, se, tl, O.ce_combine([m], [se], [tl]), O.ce_bwd(z, t, 0, M, S, np.ones(6)).ravel()])
tab = (np.arange(44, dtype=np.uint16) + 1).reshape(11, 4)
out["embed"] = O.embed(np.array([3, -1, 12, 0]), tab, 2).astype(np.float64).ravel()
Q, K, V, dO = g.standard_normal((13, 32)), g.standard_normal((13, 16)), g.standard_normal((13, 16)), g.standard_normal((13, 32))
Oo, lse = O.attn_core_fwd(Q, K, V, 2, 1)
out["attn"] = np.concatenate([Oo.ravel(), lse.ravel()] + [x.ravel() for x in O.attn_core_bwd(Q, K, V, dO, 2, 1)])
y, x = g.standard_normal((5, 24)), g.standard_normal((5, 24))
mask = (g.random((5, 24)) > 0.2).astype(np.uint8)
u, zz, mu, rs = O.sp_ln_fwd(y, x, mask, np.ones(24), np.zeros(24), 0.2)
out["sp"] = np.concatenate([u.ravel(), zz.ravel(), mu, rs] + [a.ravel() for a in O.sp_ln_bwd(y, x, u, mu, rs, np.ones(24), mask, 0.2)])
np.savez(sys.argv[2], **out)
"""


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=timeout)
    assert r.returncode == 0, r.stdout[-4000:]
    return r.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    lib = str(tmp_path / "liboracle_san.so")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
          "-D_GNU_SOURCE", "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all",
          os.path.join(ROOT, "oracle", "oracle.c"), "-o", lib, "-lm"])
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], stdout=subprocess.PIPE, text=True).stdout.strip()
    ubsan = subprocess.run(["gcc", "-print-file-name=libubsan.so"], stdout=subprocess.PIPE, text=True).stdout.strip()
    script = str(tmp_path / "calls.py")
    with open(script, "w") as f:
        f.write(ORACLE_CALLS)
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}", ORACLE_LIB=lib, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    _run([sys.executable, script, ROOT, str(tmp_path / "san.npz")], env=env)
    env_plain = {k: v for k, v in os.environ.items() if k not in ("LD_PRELOAD", "ORACLE_LIB")}
    _run([sys.executable, script, ROOT, str(tmp_path / "plain.npz")], env=env_plain)
    a, b = np.load(tmp_path / "san.npz"), np.load(tmp_path / "plain.npz")
    assert set(a.files) == set(b.files)
    for k in a.files:
        assert np.array_equal(a[k], b[k]), k


ABI_RUNNER = r"""
import sys
sys.path.insert(0, sys.argv[1])
from megatron_tensor_layer_tp_amd import tpshard as T
T.LIB_PATH = sys.argv[2]
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", sys.argv[1] + "/tests/test_abi_cpu.py"]))
"""


def test_abi_validation_under_asan_ubsan(tmp_path):
    from megatron_tensor_layer_tp_amd import build as B
    objs = sorted(glob.glob(os.path.join(ROOT, "_build", "*.o")))
    need = [os.path.join(ROOT, "_build", s + ".o") for s in B.SOURCES if s != "tpshard_api.cpp"]
    if not all(os.path.exists(o) for o in need):
        B.build(verbose=False)
    hipcc = B._hipcc()
    api = str(tmp_path / "tpshard_api_san.o")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    _run([hipcc, *B.COMMON, *san, "-g", "-x", "hip", "-c", os.path.join(B.CSRC, "tpshard_api.cpp"), "-o", api],
         timeout=900)
    lib = str(tmp_path / "libtpshard_san.so")
    _run([hipcc, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-shared-libsan", *need, api, "-o", lib], timeout=900)
    clang_rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not clang_rt:
        pytest.skip("clang's AddressSanitizer runtime not found")
    runner = str(tmp_path / "abi_runner.py")
    with open(runner, "w") as f:
        f.write(ABI_RUNNER)
    env = dict(os.environ, LD_PRELOAD=clang_rt[0], ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    out = _run([sys.executable, runner, ROOT, lib], env=env, timeout=900)
    assert " passed" in out
