"""Host-side logic of bench.py: the one-GPU contract, the algorithmic units
the roofline divides by, and the HBM byte counter scaling (no GPU needed)."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from hashed_gram_embedding_amd import inputs  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def test_kernel_units_of_the_single_branch_layer():
    lay = inputs.make_config(1, T=8, rows_per_table=997).layers[0]
    u = bench.kernel_units(4096, lay, "bf16")
    # 4 B of token id, then 16 rows of 128 B in and 128 B out per token
    assert u["gather_kernel<hashed>"] == ("hbm", 4096 * (4 + 16 * 256))
    assert u["proj_gate_kernel"] == ("mfma", 2.0 * 4096 * 2048 * 1024)
    # v (fp32) and 16 statistics tiles in; H in and out; alpha and gamma out
    assert u["conv_kernel"] == ("hbm", 4096 * (4096 + 16 * 16 + 2 * 2048 + 8))
    # MXFP8 rows: a code per element and a scale byte per 32
    assert bench.kernel_units(4096, lay, "bf16", mx=True)["gather_kernel<hashed>"][1] == 4096 * (4 + 16 * (128 + 66))
    # hot tier: every order adds a pilot and a 32-byte slot; a hit reads its 1 KiB row, a miss 8 cold rows
    hot = bench.kernel_units(4096, lay, "bf16", hot_hit=[1.0, 0.0])["gather_kernel<hashed,hot>"][1]
    assert hot == 4096 * (4 + 16 * 128 + 2 * 36 + 1024 + 8 * 128)
    # decode: below the ridge the projection is priced by the bytes it moves
    small = bench.kernel_units(256, lay, "bf16")["proj_gate_kernel"]
    assert small[0] == "hbm" and small[1] > 2048 * 1024 * 2
    # the FP8 small-batch product moves W as one byte per value plus a scale byte per 32
    small_mx = bench.kernel_units(256, lay, "bf16", mx=True)["proj_gate_kernel"]
    assert small_mx[0] == "hbm" and 2048 * 1024 * 33 / 32 < small_mx[1] < small[1]
    # past the switch the FP8 product is priced by its flops
    assert bench.kernel_units(4096, lay, "bf16", mx=True)["proj_gate_kernel"] == ("mfma", 2.0 * 4096 * 2048 * 1024)


def test_hbm_summary_scales_counters_by_the_calibration_copy(tmp_path, capsys):
    def write(path, rows):
        with open(path, "w") as f:
            f.write("Kernel_Name,Counter_Name,Counter_Value\n")
            for k, c, v in rows:
                f.write(f'"{k}",{c},{v}\n')
    n = 1 << 30
    gather = "void engram::(anonymous namespace)::hashed_gather_kernel<1, 1, false, 2>(unsigned int)"
    fetch = [(gather, "FETCH_SIZE", 4000.0), (gather, "FETCH_SIZE", 6000.0),
             ("__amd_rocclr_copyBuffer", "FETCH_SIZE", n / 1024 / 2)]          # the counter reads half
    write_ = [(gather, "WRITE_SIZE", 8192.0), ("__amd_rocclr_copyBuffer", "WRITE_SIZE", n / 1024)]
    write(tmp_path / "f.csv", fetch)
    write(tmp_path / "w.csv", write_)
    bench.hbm_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "wl", n)
    out = capsys.readouterr().out
    row = next(l for l in out.splitlines() if "`gather_kernel<hashed>`" in l)
    cells = [c.strip() for c in row.strip().strip("|").split("|")]
    assert cells[0] == "wl" and int(cells[2]) == 2 * 5000 * 1024 and int(cells[3]) == 8192 * 1024
    assert cells[4] == "2" and cells[5] == bench.kernel_source_hash("gather_kernel<hashed>")



def test_hbm_summary_takes_the_most_dispatched_instantiation(tmp_path, capsys):
    """A kernel with several instantiations in one run (a decode prefill and
    its single-token steps; the small-batch and the large projection) is
    summarised by the one dispatched most often."""
    def write(path, rows):
        with open(path, "w") as f:
            f.write("Kernel_Name,Counter_Name,Counter_Value\n")
            for k, c, v in rows:
                f.write(f'"{k}",{c},{v}\n')
    n = 1 << 30
    prefill = "void engram::(anonymous namespace)::proj_gate_kernel<128, false, 4, 3, true>(engram::ProjGateArgs)"
    steps = "void engram::(anonymous namespace)::proj_gate_small_kernel<false>(engram::ProjGateArgs)"
    copy = "__amd_rocclr_copyBuffer"
    fetch = [(prefill, "FETCH_SIZE", 90000.0)] * 2 + [(steps, "FETCH_SIZE", 4000.0)] * 5 + \
            [(copy, "FETCH_SIZE", n / 1024)]
    write_ = [(prefill, "WRITE_SIZE", 70000.0)] * 2 + [(steps, "WRITE_SIZE", 1000.0)] * 5 + \
             [(copy, "WRITE_SIZE", n / 1024)]
    write(tmp_path / "f.csv", fetch)
    write(tmp_path / "w.csv", write_)
    bench.hbm_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "wl", n)
    row = next(l for l in capsys.readouterr().out.splitlines() if "`proj_gate_kernel`" in l)
    cells = [c.strip() for c in row.strip().strip("|").split("|")]
    assert int(cells[2]) == 4000 * 1024 and int(cells[3]) == 1000 * 1024 and cells[4] == "5"

def test_rotation_touches_twice_the_infinity_cache():
    """The timed rotation holds whole graphs of batches and enough batches that
    their table rows add up to 512 MiB: 70 single-branch batches (8 MiB of
    rows each), 10 four-branch batches (64 MiB each)."""
    lay = inputs.make_config(1, T=8, rows_per_table=997).layers[0]
    assert bench.rows_per_batch([lay], 4096) == 4096 * 16 * 128
    assert bench.rotation_size(bench.rows_per_batch([lay], 4096), 10) == 70
    assert bench.rotation_size(bench.rows_per_batch([lay], 32768), 10) == 10
    assert bench.rotation_size(bench.rows_per_batch([lay], 32768), 10, override=1) == 10
    assert bench.rotation_size(123, 5, override=7) == 10
    # batches of the rotation are seeded: the same draw twice, different batches differ
    a, b = inputs.token_batch(1, 3, (1, 64)), inputs.token_batch(1, 3, (1, 64))
    assert np.array_equal(a, b) and not np.array_equal(a, inputs.token_batch(1, 4, (1, 64)))
    assert np.array_equal(inputs.hidden_batch(1, 2, (1, 4, 1, 8)), inputs.hidden_batch(1, 2, (1, 4, 1, 8)))


def test_cpu_baseline_covers_the_whole_batch_on_every_core():
    w = inputs.make_config(1, B=2, T=100, rows_per_table=997)
    r = bench.cpu_baseline(w, 0.3)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s" and r["value"] > 0
    assert 1 <= r["cores"] <= 16 and r["single_core"]["cores"] == 1 and r["single_core"]["value"] > 0
    assert "2 x 100 tokens" in r["sample"]


def test_chunked_oracle_with_halo_equals_the_whole_batch():
    """The CPU baseline's chunks (each with the 11 positions before it) give
    exactly the outputs of the oracle over the whole batch."""
    from oracle import engram_oracle as orc
    w = inputs.make_config(1, B=2, T=60, rows_per_table=997)
    full = orc.forward(w.tokens, w.H, w.layers[0], "bf16")
    for lo, hi in ((0, 13), (13, 30), (30, 60)):
        s = max(0, lo - bench.CPU_HALO)
        part = orc.forward(w.tokens[:, s:hi], w.H[:, s:hi], w.layers[0], "bf16")
        assert np.array_equal(part["Y"][:, lo - s:], full["Y"][:, lo:hi])
