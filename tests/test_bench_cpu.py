"""bench.py's contract, checked without a GPU: the multi-GPU refusal, the
workload table (every row a configuration the library accepts, on the
shards the names promise) and the profiled traffic records it reads."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from communication_compressed_optimizer_elt_amd import binding as L  # noqa: E402
from communication_compressed_optimizer_elt_amd import synth  # noqa: E402

@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from communication_compressed_optimizer_elt_amd import build

        build.build()
    return L.lib()


SCHEMES = {"dct": L.SCHEME_DCT, "random": L.SCHEME_RANDOM, "stride": L.SCHEME_STRIDE, "diloco": L.SCHEME_DILOCO}
FORMATS = {"ternary": L.VAL_TERNARY, "f16": L.VAL_F16, "f32": L.VAL_F32}


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus 1" in r.stderr and r.stdout == ""


def test_default_workload_is_the_headline():
    assert bench.WORKLOADS["olmo2-1b-half-shard-demo-k1"] == bench.Workload("olmo2", "dct", 1, "ternary", 2)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0 and "olmo2-1b-half-shard-demo-k1" in r.stdout


def _config(w):
    return L.Config(scheme=SCHEMES[w.scheme], k=w.k, value_fmt=FORMATS[w.fmt], sign=w.sign,
                    period=bench.DILOCO_PERIOD)


@pytest.mark.parametrize("name", sorted(bench.WORKLOADS))
def test_every_workload_is_a_valid_configuration(lib, name):
    w = bench.WORKLOADS[name]
    cfg = _config(w)
    n = 4096 if w.shard == "tensor4096" else 2048 * 3 + 5
    lay = L.demo_payload_layout(cfg, n)  # raises on an invalid configuration
    assert lay["total_bytes"] > 0
    if w.adamw:  # Decoupled AdamW carries values: the sign-on form is refused
        assert w.sign == 0 and w.fmt != "ternary"
    if w.sign == 0:
        assert w.fmt != "ternary"
    assert w.mode in ("step", "decode") and w.R >= 1
    if w.mode == "decode":
        assert w.R == 64 and "decode-r64" in name
    # the name states the scheme and, for Random / Striding, n
    if w.scheme in ("random", "stride"):
        assert f"{w.scheme}-n{w.k}" in name
    if w.scheme == "dct":
        assert f"demo-k{w.k}" in name
    assert (w.shard == "vit") == name.startswith("vit-b-set")
    assert (w.shard == "olmo2-full") == name.startswith("olmo2-1b-full")


def test_shard_sizes():
    assert synth.shard_numel(synth.olmo2_half_shard()) == 639_697_920
    assert synth.shard_numel(synth.olmo2_full()) == 1_279_395_840
    assert synth.shard_numel(synth.vit_b_set()) == 85_017_600


def test_traffic_records_match_the_benchmark_accounting(lib):
    """Each profiled traffic record names its workload and kernel kind, and its
    algorithmic bytes per launch are what bench.py counts for that launch."""
    pdir = os.path.join(ROOT, "profiles")
    recs = [f for f in os.listdir(pdir) if f.startswith("traffic_") and f.endswith(".json")]
    assert recs
    for f in recs:
        kind, wl = f[len("traffic_"):-len(".json")].split("_", 1)
        assert kind in ("encode", "decode") and wl in bench.WORKLOADS, f
        rec = json.load(open(os.path.join(pdir, f)))
        assert rec["workload"] == wl
        w = bench.WORKLOADS[wl]
        n = synth.shard_numel({"olmo2": synth.olmo2_half_shard, "olmo2-full": synth.olmo2_full,
                               "vit": synth.vit_b_set}[w.shard]())
        lay = L.demo_payload_layout(_config(w), n)
        pb = lay["idx_bytes"] + 2 * lay["plane_bytes"] + lay["val_bytes"]
        if kind == "encode":
            # DiLoCo: the default run's 20 timed steps (3..22) hold one synchronisation
            # (step 15); the encode kind averages 19 momentum passes and that step's encode
            sends = 1 / 20 if w.scheme == "diloco" else 1
            expect = (20 if w.adamw else 12) * n + sends * pb
        else:
            expect = (12 if w.adamw else 8) * n + w.R * pb
        assert abs(rec["algorithmic_bytes_per_launch"] - expect) <= 1e-9 * expect, (f, expect)
        assert 0.99 <= rec["hbm_bytes_per_launch"] / rec["algorithmic_bytes_per_launch"] <= 1.01, f
