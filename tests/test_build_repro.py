"""The build is reproducible: compiling one translation unit twice, into two
different directories, gives byte-identical objects. The measured HBM bytes
of the sum kernel are tied to the sha256 of its object, so a fresh build of
the same sources must give the same hash."""
import hashlib
import os

from reduction_libred_amd import build


def _sha(path):
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def test_objects_are_byte_identical(tmp_path):
    a = tmp_path / "a"
    b = tmp_path / "b"
    a.mkdir()
    b.mkdir()
    oa = build.compile_unit("probe.hip", str(a / "probe.o"))
    ob = build.compile_unit("probe.hip", str(b / "probe.o"))
    assert os.path.getsize(oa) > 0
    assert _sha(oa) == _sha(ob)


def test_traffic_record_matches_the_built_sum_kernel():
    # profiles/traffic.json holds the HBM bytes per launch of the float32 sum
    # kernel, measured with FETCH_SIZE / WRITE_SIZE, under the identity of
    # the object it was measured on (sha256 of flat_sum_f32.hip's object and
    # the launch shape). A change to that kernel's code must come with a new
    # counter run, or the benchmark reports no traffic.
    import json
    import pytest

    import bench
    if not os.path.exists(bench.OBJECT_MANIFEST):
        pytest.skip("library not built")
    with open(bench.TRAFFIC_FILE) as fh:
        rec = json.load(fh)
    assert bench.kernel_identity(rec["launch_shape"]) == rec["kernel_identity"]
    assert bench.recorded_traffic(rec["launch_shape"]) == rec["flat_reduce_kernel_sum_f32_2p28_bytes_per_launch"]
    ratio = rec["flat_reduce_kernel_sum_f32_2p28_bytes_per_launch"] / rec["algorithmic_bytes_per_launch"]
    assert 1.0 <= ratio < 1.001
