"""Host AddressSanitizer over the C ABI's host code (CPU only).

The library is rebuilt with the sanitizer on its host code (device code as usual)
and a C++ driver walks the validation paths, which read the caller's host arrays
(chunk_lens, seq_lens, head_lens) and format error text. The kernels use no
atomics and are deterministic; on the host side this is the memory-safety check.
A second run makes one deliberate caller error (a lengths array one short) to
show the sanitizer really instruments the library."""
import os
import shlex
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "context_attention_diffusion_non_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"


@pytest.fixture(scope="module")
def asan_driver(tmp_path_factory):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)):
        pytest.skip("ROCm compilers not available")
    d = tmp_path_factory.mktemp("asan")
    lib = d / "libcpattn_asan.so"
    srcs = " ".join(os.path.join(CSRC, s) for s in ("attn_fwd.hip", "lse_merge.hip", "permute.hip", "api.cpp", "noalloc.hip"))
    build = (f"{HIPCC} --offload-arch=gfx950 -O1 -g -std=c++17 -fPIC -shared "
             f"-Xclang -target-feature -Xclang -packed-fp32-ops -Xarch_device -fno-honor-nans "
             f"-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer "
             f"-I{os.path.join(ROOT, 'include')} -I{CSRC} {srcs} -o {lib}")
    r = subprocess.run(shlex.split(build), stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-4000:]
    exe = d / "driver"
    link = (f"{CLANGXX} -O1 -g -std=c++17 -fsanitize=address -fno-omit-frame-pointer "
            f"-I{os.path.join(ROOT, 'include')} {os.path.join(ROOT, 'tests', 'host_asan_driver.cpp')} "
            f"-L{d} -lcpattn_asan -Wl,-rpath,{d} -o {exe}")
    r = subprocess.run(shlex.split(link), stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-4000:]
    yield str(exe)
    shutil.rmtree(d, ignore_errors=True)


def _run(exe, *args):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    return subprocess.run([exe, *args], stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, env=env,
                          timeout=120)


def test_validation_paths_are_memory_safe(asan_driver):
    r = _run(asan_driver)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, r.stdout + r.stderr[-2000:]
    assert "0 failure(s)" in r.stdout


def test_sanitizer_catches_a_short_lengths_array(asan_driver):
    r = _run(asan_driver, "overread")
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr, r.stderr[-4000:]
    assert "ring_fwd" in r.stderr  # reported inside the library's chunk loop
