"""Host logic of the benchmark (no GPU): the visible-pair count behind every
TFLOPS figure, the one-GPU rule, the HBM-traffic arithmetic of the profile
summaries and the CPU baseline's record."""
import math
import os
import sqlite3
import subprocess
import sys

import pytest
import torch

import block_diffusion_lm_amd as bd
import oracle
from block_diffusion_lm_amd import profiling

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402  (the repository root holds bench.py)


@pytest.mark.parametrize("n", [1, 7, 100, 129, 300])
@pytest.mark.parametrize("b", [1, 3, 4, 48, 128, 256])
def test_visible_pairs_match_the_mask(n, b):
    """bench counts n^2 + sum of squared block sizes (Fast Diffusion
    Attention, "The right yardstick"); the explicit mask of the oracle and the
    library's own count agree."""
    want = int(oracle.block_diffusion_mask(n, b).sum())
    assert bench.visible_pairs(n, b) == want
    assert bd.bdattn_visible_pairs(bd.MODE_DIFFUSION, n, b) == want


def test_visible_pairs_closed_form_at_the_workloads():
    """b dividing n gives exactly n^2 + n b; the stated workloads' counts."""
    for n, b in ((128, 4), (1024, 4), (2048, 16), (8192, 32), (4096, 128), (4096, 256)):
        assert bench.visible_pairs(n, b) == n * n + n * b
    # b = 3 and b = 48 do not divide 4096: the last block is shorter
    assert bench.visible_pairs(4096, 3) == 4096 ** 2 + 1365 * 9 + 1
    assert bench.visible_pairs(4096, 48) == 4096 ** 2 + 85 * 48 ** 2 + 16 ** 2


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv, capture_output=True, text=True,
                       env={**os.environ, **env}, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


def _db(path, kernels=(), counters=()):
    con = sqlite3.connect(path)
    con.execute("create table kernels (name text, duration real)")
    con.execute("create table counters_collection (kernel_name text, counter_name text, value real)")
    con.executemany("insert into kernels values (?, ?)", kernels)
    con.executemany("insert into counters_collection values (?, ?, ?)", counters)
    con.commit()
    con.close()


def test_traffic_summary_arithmetic(tmp_path):
    """Each counter is scaled by what it reads for the calibration copy of
    known size; the dominant kernel is the longest of the library's."""
    dkdv = "void bd::bwd_dkdv_kernel<128, false, false>(bd::AttnArgs, int)"
    dq = "void bd::bwd_dq_kernel<128, false>(bd::AttnArgs, int)"
    copy = "__amd_rocclr_copyBuffer"
    trace, fetch, write = (str(tmp_path / f"{x}.db") for x in ("trace", "fetch", "write"))
    _db(trace, kernels=[(dkdv, 4.0e6), (dkdv, 4.2e6), (dq, 2.9e6), ("other", 9e9)])
    # FETCH_SIZE reads half of the copy's 1 GiB: a scale of 2; WRITE_SIZE reads all of it
    _db(fetch, counters=[(dkdv, "FETCH_SIZE", 1000.0), (dkdv, "FETCH_SIZE", 1200.0), (copy, "FETCH_SIZE", 512.0 * 1024)])
    _db(write, counters=[(dkdv, "WRITE_SIZE", 300.0), (copy, "WRITE_SIZE", 1024.0 * 1024)])
    out = tmp_path / "profiles"
    profiling.summarize("t1", trace, fetch, write, "cmd-trace", str(out), copy_mib=1024,
                        fetch_command="cmd-fetch", write_command="cmd-write")
    lines = (out / "kernels_t1.txt").read_text().splitlines()
    body = [ln for ln in lines if ln.startswith("bd::")]
    assert body[0].startswith("bd::bwd_dkdv") and body[1].startswith("bd::bwd_dq")  # longest first
    assert "4100.0" in body[0]                                                       # average in us
    tr = profiling.read_traffic(str(out / "traffic_bwd_dkdv_t1.txt"))
    assert tr["kernel"] == "bwd_dkdv"
    assert float(tr["fetch_scale"]) == pytest.approx(2.0)
    assert float(tr["write_scale"]) == pytest.approx(1.0)
    assert float(tr["bytes_per_launch"]) == pytest.approx((1100.0 * 2.0 + 300.0 * 1.0) * 1024)
    assert tr["source_sha256"] == profiling.source_hash("bwd_dkdv")


def test_committed_traffic_figure_names_its_kernel_sources():
    """The figure bench.py reports is tied to the sources it was taken on."""
    tr = profiling.read_traffic(os.path.join(ROOT, "profiles", "traffic_bwd_dkdv_c4.txt"))
    assert tr is not None and tr["kernel"] == "bwd_dkdv" and tr["workload"] == "c4"
    assert len(tr["source_sha256"]) == 64
    assert float(tr["bytes_per_launch"]) > 0


def test_cpu_baseline_record():
    """The oracle timed on a bounded sample: the record's fields, and the
    visible pairs it counted (n^2 + n b for one tiny head)."""
    g = torch.Generator().manual_seed(5)
    n, D, b = 16, 8, 4
    head = [torch.randn(2 * n, D, generator=g).to(torch.bfloat16) for _ in range(4)]
    rec = bench.cpu_baseline([(*head, n, b)], "tiny", target_s=0.0, chunk=10)
    assert set(rec) == {"value", "unit", "cores", "kind", "sample"}
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOPS"
    assert rec["value"] > 0 and rec["cores"] >= 1
    assert f"{n * n + n * b} visible pairs" in rec["sample"]
    assert "4 chunks" in rec["sample"]  # 32 rows in chunks of 10
    assert math.isfinite(rec["value"])


def test_roofline_at_the_sampled_clock():
    """The peak scales with the engine clock: at 1.2 GHz half of it."""
    r = bench.at_clock({"achieved": 1000.0, "peak": 2500.0}, {"median_mhz": 1200.0})
    assert r["peak_at_median_sclk"] == pytest.approx(1250.0)
    assert r["frac_at_median_sclk"] == pytest.approx(0.8)
    assert set(bench.at_clock({"achieved": 1.0, "peak": 2.0}, None)) == {"achieved", "peak"}


def test_committed_counters_parse():
    """profiles/counters_c4.txt: every kernel has MFMA- and vector-busy
    shares in (0, 1] and a clock; the file names the sources it was taken on."""
    c = profiling.read_counters(os.path.join(ROOT, "profiles", "counters_c4.txt"))
    assert c is not None and len(c["source_sha256"]) == 64
    kernels = {k: v for k, v in c.items() if isinstance(v, dict)}
    assert set(kernels) == {"fwd", "bwd_dq", "bwd_dkdv"}
    for v in kernels.values():
        assert 0 < v["mfma_busy"] <= 1 and 0 < v["valu_busy"] <= 1 and 1000 < v["clock_mhz"] < 2600
        assert v["SQ_LDS_BANK_CONFLICT"] >= 0 and v["hbm_gbs"] > 0
