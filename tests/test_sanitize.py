"""The C-ABI layer under the address and undefined-behaviour sanitizers, on
the host: tests/native/abi_sanitize.cpp calls every entry point with
arguments the host checks must reject and builds the hot tier's minimal
perfect hash on 50,000 keys, linked against api.cpp compiled with
-fsanitize=address,undefined (host code only).  The driver passes fake
device pointers that validation must reject, so it runs only where no GPU is
visible, with HIP's device list emptied for good measure."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs hipcc")
@pytest.mark.skipif(_gpu_visible(), reason="host-only check: its fake device pointers must never reach a GPU")
def test_abi_layer_under_address_and_ub_sanitizers(tmp_path):
    sys.path.insert(0, os.path.join(ROOT, "tests", "native"))
    try:
        import build_sanitize
    finally:
        sys.path.pop(0)
    exe = build_sanitize.build(str(tmp_path))
    env = dict(os.environ, HIP_VISIBLE_DEVICES="", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "all passed" in r.stdout
    assert "AddressSanitizer" not in out and "runtime error" not in out and "LeakSanitizer" not in out
