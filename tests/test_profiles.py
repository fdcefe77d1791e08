"""The committed HBM-traffic summaries (profiles/*_pmc.json) describe the
kernel sources as they stand.

bench.py puts a summary's calibrated HBM bytes into its roofline line only
when the summary's kernel-source hash matches the current sources, so a
summary left behind by a kernel change would silently turn the line's
traffic into null.  Each summary must also be self-consistent: its measured
bytes per call close to the algorithmic bytes it states (every K/V byte read
once; the calibration of FETCH_SIZE / WRITE_SIZE against a copy of known
size is in the file)."""
import glob
import importlib.util
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUMMARIES = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_pmc.json")))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_for_profiles", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _key(path):
    name = os.path.basename(path)[: -len("_pmc.json")]
    return name[len("decode_"):] if name.startswith("decode_") else name


def test_there_are_summaries():
    keys = {_key(p) for p in SUMMARIES}
    assert {"llama7b", "long", "gqa", "prefill"} <= keys, keys


@pytest.mark.parametrize("path", SUMMARIES, ids=[_key(p) for p in SUMMARIES])
def test_summary_was_taken_on_the_current_kernel_sources(path):
    d = json.load(open(path))
    assert d["kernel_source_sha256_16"] == _bench().kernel_source_hash(_key(path)), (
        f"{os.path.basename(path)} was taken on other kernel sources: retake its FETCH_SIZE / WRITE_SIZE passes")


@pytest.mark.parametrize("path", SUMMARIES, ids=[_key(p) for p in SUMMARIES])
def test_summary_traffic_is_close_to_its_algorithmic_bytes(path):
    d = json.load(open(path))
    cal = d["calibration"]
    assert cal["bytes_read"] > 0 and cal["FETCH_SIZE_KiB"] > 0 and cal["WRITE_SIZE_KiB"] > 0
    if "by_block_size" in d:
        ratios = [v["traffic_over_algorithmic"] for v in d["by_block_size"].values()]
        for v in d["by_block_size"].values():
            assert v["traffic_over_algorithmic"] == pytest.approx(
                v["hbm_bytes_per_call"] / v["algorithmic_bytes_per_call"], abs=1e-4)
    else:
        hbm = d.get("hbm_bytes_per_call", d.get("hbm_bytes_per_decode_call"))
        alg = d.get("algorithmic_total_bytes_per_call", d.get("algorithmic_bytes_per_call"))
        ratios = [d["traffic_over_algorithmic"]]
        assert ratios[0] == pytest.approx(hbm / alg, abs=1e-4)
        if "append_traffic_over_algorithmic" in d:
            ratios.append(d["append_traffic_over_algorithmic"])
            assert ratios[1] == pytest.approx(
                d["append_hbm_bytes_per_call"] / d["append_algorithmic_bytes_per_call"], abs=1e-4)
    # the counters see every algorithmic byte once, give or take the
    # calibration and a few re-read lines: far from 2x (a re-read of K/V)
    for r in ratios:
        assert 0.97 < r < 1.06, (os.path.basename(path), r)
