"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

- The oracle's C library, rebuilt with gcc -fsanitize=address,undefined, runs
  full and row-sampled attention (causal and not, GQA, bf16 inputs) and the
  merge in a subprocess with the sanitizer runtimes preloaded.
- Opt-in (RA_SANITIZE_HOST=1, about a minute): libra.so's host code (argument
  validation, planning, error messages) rebuilt with host-only sanitizers and
  the C-ABI tests run against it.  No GPU code is instrumented and no kernel
  runs.
"""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gcc_runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_under_asan_ubsan(tmp_path):
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
                    "-ffp-contract=off", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                    os.path.join(ROOT, "oracle", "attn_oracle.c"), "-o", str(lib), "-lm"], check=True)
    script = textwrap.dedent(f"""
        import sys
        sys.path.insert(0, {ROOT!r})
        import numpy as np
        import oracle
        from long_context_exact_amd import synthetic
        oracle._lib = None
        oracle._LIB_PATH = {str(lib)!r}
        Q = synthetic.normal_tensor((2, 37, 4, 16), (7, 0), "bf16")
        K = synthetic.normal_tensor((2, 37, 2, 16), (7, 1), "bf16")
        V = synthetic.normal_tensor((2, 37, 2, 16), (7, 2), "bf16")
        for causal in (False, True):
            O, L = oracle.attention(Q, K, V, causal)
            oracle.attention_rows(Q, K, V, causal, np.array([0, 1, 1]), np.array([0, 36, 5]))
        parts_O = np.random.default_rng(0).standard_normal((3, 8, 16))
        parts_l = np.array([[0.0] * 8, [-np.inf] * 8, [1.0] * 8])
        oracle.merge(parts_O, parts_l)
        print("clean")
    """)
    env = dict(os.environ, LD_PRELOAD=f"{asan} {ubsan}", ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True, env=env,
                       timeout=300)
    assert r.returncode == 0 and "clean" in r.stdout, r.stderr[-3000:]


@pytest.mark.skipif(os.environ.get("RA_SANITIZE_HOST") != "1", reason="opt-in: RA_SANITIZE_HOST=1")
def test_library_host_code_under_asan_ubsan(tmp_path):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    asan = subprocess.run([hipcc, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.exists(asan):
        pytest.skip("clang ASan runtime not found")
    build = os.path.join(ROOT, "long_context_exact_amd", "_build")
    objs = [os.path.join(build, f) for f in sorted(os.listdir(build))
            if f.endswith(".hip.o") and f != "api.hip.o"]
    if not objs:
        pytest.skip("build the library first")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    api_o = tmp_path / "api_san.o"
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang",
                    "-target-feature", "-Xclang", "-packed-fp32-ops", *san, "-c",
                    os.path.join(ROOT, "long_context_exact_amd", "csrc", "api.hip"), "-o", str(api_o)],
                   check=True, capture_output=True)
    lib = tmp_path / "libra_san.so"
    subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *san, *objs, str(api_o), "-o",
                    str(lib)], check=True, capture_output=True)
    plugin = tmp_path / "swap_lib.py"
    plugin.write_text("import long_context_exact_amd as ra\nra._lib = None\n"
                      f"ra.LIB_PATH = {str(lib)!r}\n")
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               PYTHONPATH=f"{tmp_path}:{os.environ.get('PYTHONPATH', '')}")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "swap_lib",
                        os.path.join(ROOT, "tests", "test_abi.py")], capture_output=True, text=True,
                       env=env, cwd=ROOT, timeout=900)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
