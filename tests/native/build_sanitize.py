"""Builds tests/native/abi_sanitize.cpp against the library's C-ABI layer with
the address and undefined-behaviour sanitizers on the host code (the device
code of the kernels is compiled as usual; no sanitizer reaches the GPU).
Used by tests/test_sanitize.py; returns the path of the executable."""
import concurrent.futures
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "hashed_gram_embedding_amd", "csrc")
INC = os.path.join(ROOT, "include")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
# host-only sanitizer options: on a hipcc line each one follows -Xarch_host
SAN = ["address", "undefined"]
HOST_SAN = [f for s in SAN for f in ("-Xarch_host", f"-fsanitize={s}")] + \
    ["-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(" ".join(cmd) + "\n" + r.stdout + r.stderr)


def build(out_dir: str) -> str:
    from hashed_gram_embedding_amd import build as bld
    os.makedirs(out_dir, exist_ok=True)
    hipcc = bld.hipcc()
    flags = bld.common_flags()
    objs = []
    jobs = []
    for f in sorted(os.listdir(CSRC)):
        if not f.endswith((".hip", ".cpp")):
            continue
        o = os.path.join(out_dir, f + ".o")
        extra = HOST_SAN if f == "api.cpp" else []
        jobs.append([hipcc] + flags + extra + ["-c", os.path.join(CSRC, f), "-o", o])
        objs.append(o)
    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(_run, jobs))
    clang = os.path.join(ROCM, "llvm", "bin", "clang++")
    drv = os.path.join(out_dir, "abi_sanitize.o")
    _run([clang, "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I", INC, "-I", os.path.join(ROCM, "include"),
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
          "-c", os.path.join(HERE, "abi_sanitize.cpp"), "-o", drv])
    exe = os.path.join(out_dir, "abi_sanitize")
    _run([clang, "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-o", exe, drv] + objs +
         ["-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"])
    return exe
