"""Host-side logic of bench.py that runs without a GPU: the refusal of more
than one GPU, and the lookup of rocprofv3 traffic records (a record counts
only for the kernel, the decode workload and the kernel sources it was taken
on)."""

import hashlib
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _tree(tmp_path, source, records):
    csrc = tmp_path / "paged_kv_cache_inject_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "pkv_kernels.hip").write_bytes(source)
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "a.md").write_text("# summary\n\n" + "".join(r + "\n" for r in records))
    return str(tmp_path)


def test_traffic_record_matches_kernel_workload_and_sources(tmp_path):
    src = b"// kernels\n"
    sha = hashlib.sha256(src).hexdigest()[:16]
    root = _tree(tmp_path, src, [
        "traffic-record: kernel=decode_mfma_kernel workload=70b sources_sha256=%s "
        "bytes_per_launch=1000 fetch_bytes=900 write_bytes=100" % sha,
        "traffic-record: kernel=decode_mfma_kernel workload=mqa sources_sha256=%s "
        "bytes_per_launch=2000 fetch_bytes=1900 write_bytes=100" % sha,
        "traffic-record: kernel=decode_mfma_kernel workload=8b sources_sha256=0123456789abcdef "
        "bytes_per_launch=3000 fetch_bytes=2900 write_bytes=100",
    ])
    assert bench.recorded_traffic(workload="70b", root=root) == 1000
    assert bench.recorded_traffic(workload="mqa", root=root) == 2000
    # a record taken on other kernel sources is stale
    assert bench.recorded_traffic(workload="8b", root=root) is None
    # no record for this workload or kernel
    assert bench.recorded_traffic(workload="ragged", root=root) is None
    assert bench.recorded_traffic(kernel="inject_rope_kernel", workload="70b", root=root) is None


def test_committed_traffic_records_are_well_formed():
    import glob
    n = 0
    for path in glob.glob(os.path.join(ROOT, "profiles", "*.md")):
        for line in open(path):
            if line.startswith("traffic-record:"):
                f = dict(kv.split("=", 1) for kv in line.split()[1:])
                assert set(f) >= {"kernel", "workload", "sources_sha256", "bytes_per_launch",
                                  "fetch_bytes", "write_bytes"}, line
                assert len(f["sources_sha256"]) == 16
                # each figure is rounded from the scaled counter averages on its own
                total = int(f["fetch_bytes"]) + int(f["write_bytes"])
                assert abs(int(f["bytes_per_launch"]) - total) <= 1, line
                n += 1
    assert n >= 1


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_item_balance_load_model():
    """The balance figure of the ragged batch: items follow the plan's split
    rule, and the longest-first load model's finish over the even share is
    1 for equal items and the largest item's share for one dominant item."""
    even = bench.item_balance([32] * 256, 1 << 20, 1, n_cus=256)
    assert even["items"] == 256 and even["lpt_makespan_over_mean"] == 1.0
    one = bench.item_balance([1000] + [10] * 255, 1 << 20, 1, n_cus=256)
    assert abs(one["lpt_makespan_over_mean"] - 1000 / (3550 / 256)) < 1e-3
    split = bench.item_balance([1000] + [10] * 255, 100, 1, n_cus=256)
    assert split["items"] == 10 + 255
    assert abs(split["lpt_makespan_over_mean"] - 100 / (3550 / 256)) < 1e-3
    assert sum(split["tokens_per_item_histogram"].values()) == split["items"]
    # every KV head of an item is one workgroup
    assert bench.item_balance([64] * 4, 1 << 20, 8, n_cus=256)["workgroups"] == 32


def test_host_store_dma_comparison_is_opt_in():
    """The per-run DMA comparison of the host-store workload runs only when
    asked for (--dma-compare): the default bench run and the profiled runs
    leave it out."""
    import inspect
    assert inspect.signature(bench.run_inject_host).parameters["dma_compare"].default is False
    src = inspect.getsource(bench.main)
    assert "dma_compare=args.dma_compare" in src
    assert '"--dma-compare", action="store_true"' in src


def test_pool_layouts_tile_the_buffer():
    """Every layout bench.py offers places the K and V planes of every
    (layer, block, KV head) inside the pool buffer without overlap, and
    together they cover it exactly."""
    import numpy as np
    plane, nl, nb, h = 64, 2, 5, 3
    for layout in ("block", "head", "plane"):
        ls, bs, hs, v_off = bench.layout_strides(layout, nb, h, plane)
        used = np.zeros(nl * ls, dtype=np.int32)
        for layer in range(nl):
            for b in range(nb):
                for hh in range(h):
                    for base in (0, v_off):
                        at = base + layer * ls + b * bs + hh * hs
                        assert 0 <= at and at + plane <= used.size, (layout, layer, b, hh)
                        used[at:at + plane] += 1
        assert np.all(used == 1), layout
    # the plane layout keeps one head's planes of consecutive blocks adjacent
    ls, bs, hs, v_off = bench.layout_strides("plane", nb, h, plane)
    assert bs == plane and hs == nb * plane
