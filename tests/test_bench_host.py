"""Host-side logic of bench.py (CPU only): the one-GPU refusal, the mirror of
the library's launch rules that names the kernels a call runs (and so picks
the rocprofv3 counter summary a bench line quotes), the algorithmic byte
counts, and the source digest that ties a counter summary to the kernel
sources it was taken from."""
import importlib.util
import os
import shutil
import subprocess
import sys

import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NCU = 256  # MI355X


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("cid,call,comb", [
    (1, "layout_dispatch_small_kernel", "combine_kernel"),
    (2, "layout_dispatch_small_kernel", "combine_kernel"),
    (3, "layout_dispatch_persistent_kernel", "combine_persistent_kernel"),
    (4, "layout_whole_kernel+dispatch_fp8_kernel", "combine_persistent_kernel"),
    (5, "layout_hist_kernel+layout_dispatch_ranked_kernel", "combine_persistent_kernel"),
])
def test_launch_rule_mirror_on_the_five_workloads(cid, call, comb):
    """The kernels each workload's calls run on 256 CUs, as the kernel traces
    in profiles/ show them."""
    b = _bench()
    wl = workloads.make(cid)
    assert b.fused_call_name(wl, NCU) == call
    assert b.combine_kernel_name(wl, NCU) == comb
    assert call in b.FUSED_SOURCES


@pytest.mark.parametrize("over,call", [
    # FP8 rows up to 32768 entries: the one-launch form (any k)
    (dict(fp8=True, T=3000), "layout_dispatch_persistent_fp8_kernel"),
    (dict(fp8=True, T=4096, k=6), "layout_dispatch_persistent_fp8_kernel"),
    # more than 14 chunks per wave of bf16 rows, or more than 32768 entries
    (dict(T=8192), "layout_hist_kernel+layout_dispatch_ranked_kernel"),
    # FP8 with k < 8 past 32768 entries: whole-table layout from 32 experts,
    # the two layout kernels below
    (dict(fp8=True, T=8192, k=6), "layout_whole_kernel+dispatch_fp8_kernel"),
    (dict(fp8=True, T=8192, k=6, E=16), "layout_hist_kernel+layout_rank_kernel+dispatch_fp8_kernel"),
    (dict(fp8=True, T=16384, k=6), "layout_hist_kernel+layout_rank_kernel+dispatch_fp8_kernel"),
    # table length not a multiple of 4 stays off the one-launch form
    (dict(T=4095, k=7), "layout_hist_kernel+layout_dispatch_ranked_kernel"),
    # a small table whose one-kernel form would visit too many ids (64 column
    # tiles per token): FP8 with k < 8 takes the small-table layout kernel,
    # bf16 the ranking dispatch
    (dict(fp8=True, T=300, H=65536, k=4, E=64), "layout_small_kernel+dispatch_fp8_kernel"),
    (dict(T=300, H=65536, k=4, E=64), "layout_hist_kernel+layout_dispatch_ranked_kernel"),
])
def test_launch_rule_mirror_on_other_shapes(over, call):
    b = _bench()
    wl = workloads.make(3, **over)
    assert b.fused_call_name(wl, NCU) == call


def test_algorithmic_bytes_of_the_prefill_step():
    """The per-call byte counts quoted for the 4096-token prefill: dispatch
    kernel 528.6 MB, one ep_layout_dispatch call 528.9 MB, combine 528.7 MB."""
    b = _bench()
    wl = workloads.make(3)
    nb = b.algorithmic_bytes(wl)
    T, H, k, E = 4096, 7168, 8, 256
    assert nb["V"] == T * k
    assert nb["dispatch_kernel"] == 2 * T * H + 4 * T * k + T * k * H * 2 == 528613376
    assert nb["dispatch_total"] == 528877572
    assert nb["combine_kernel"] == 528744448
    assert nb["dispatch_total"] + nb["combine_total"] == 1057622020


def test_algorithmic_bytes_count_only_rows_that_get_a_slot():
    """With fixed capacity V counts min(count, cap) per expert, and FP8
    payloads are 1 byte per channel plus one scale per 128 channels."""
    b = _bench()
    wl = workloads.make(2)
    count = [200] * 10 + [50] * (wl.E - 10)  # 10 experts over the capacity of 128
    nb = b.algorithmic_bytes(wl, count)
    V = 10 * 128 + (wl.E - 10) * 50
    assert nb["V"] == V
    assert nb["dispatch_kernel"] == 2 * wl.T * wl.H + 4 * wl.T * wl.k + V * wl.H + 4 * V * (wl.H // 128)
    assert b.algorithmic_bytes(wl, count, scale_bytes=1)["dispatch_kernel"] == \
        nb["dispatch_kernel"] - 3 * V * (wl.H // 128)


def test_source_digest_follows_included_headers(tmp_path, monkeypatch):
    """A counter summary is quoted only while its digest matches: the digest
    covers the code of the kernel file and of every csrc header it includes,
    not their comments."""
    b = _bench()
    src = os.path.join(ROOT, "combine_ep_layout_09_amd", "csrc")
    fake_root = tmp_path / "root"
    shutil.copytree(src, fake_root / "combine_ep_layout_09_amd" / "csrc")
    monkeypatch.setattr(b, "ROOT", str(fake_root))
    d0 = b.kernel_source_digest("ep_fused_persist.hip")
    assert d0 == b.kernel_source_digest("ep_fused_persist.hip")
    hdr = fake_root / "combine_ep_layout_09_amd" / "csrc" / "ep_dispatch_dev.h"  # included by it
    hdr.write_text(hdr.read_text() + "\n// a comment\n/* and\n another */\n")
    assert b.kernel_source_digest("ep_fused_persist.hip") == d0
    hdr.write_text(hdr.read_text() + "\nconstexpr int kChanged = 1;\n")
    assert b.kernel_source_digest("ep_fused_persist.hip") != d0
    other = fake_root / "combine_ep_layout_09_amd" / "csrc" / "ep_combine.hip"  # not included
    d1 = b.kernel_source_digest("ep_fused_persist.hip")
    other.write_text(other.read_text() + "\nconstexpr int kChanged = 1;\n")
    assert b.kernel_source_digest("ep_fused_persist.hip") == d1
