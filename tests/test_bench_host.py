"""bench.py's host logic on the CPU: the HBM traffic record is built from
rocprofv3 counter files exactly as documented (FETCH_SIZE / WRITE_SIZE in KiB
per dispatch, each scaled by what the counter reads for a plain copy of known
size), kernels are matched to m by their template arguments, and a record
taken on other kernel sources is not reported."""
import csv
import json
import os

import pytest

import bench

HDR = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write(folder, name, rows):
    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, name), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(HDR)
        w.writerows(rows)


def _kernel(m, nr, unc):
    return f"void rex::mv_kernel<1, {m}, {nr}, false, false, {str(unc).lower()}>(rex::MvArgs)"


@pytest.fixture
def counters(tmp_path):
    d = tmp_path
    # two dispatches per kernel (mean taken), an unrelated kernel that must be ignored
    _write(d / "f" / "host", "bench_counter_collection.csv", [
        [1, _kernel(1, 1, False), "FETCH_SIZE", 8800.0], [2, _kernel(1, 1, False), "FETCH_SIZE", 8900.0],
        [3, _kernel(8, 2, False), "FETCH_SIZE", 9330.0], [4, _kernel(8, 2, False), "FETCH_SIZE", 9330.0],
        [5, "void stream_read_kernel<4>(...)", "FETCH_SIZE", 1e9]])
    _write(d / "w", "bench_counter_collection.csv", [
        [1, _kernel(1, 1, False), "WRITE_SIZE", 16.0], [2, _kernel(1, 1, False), "WRITE_SIZE", 16.0],
        [3, _kernel(8, 2, False), "WRITE_SIZE", 128.0], [4, _kernel(8, 2, False), "WRITE_SIZE", 128.0]])
    # calibration: a fill (reads nothing) and copies of 256 MiB; the copy reads half its bytes
    _write(d / "cf", "copy_counter_collection.csv", [
        [1, "FillFunctor", "FETCH_SIZE", 16.0], [2, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 131072.0],
        [3, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 131072.0]])
    _write(d / "cw", "copy_counter_collection.csv", [
        [1, "FillFunctor", "WRITE_SIZE", 262144.0], [2, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 262144.0]])
    return d


def test_write_traffic_scales_counters_by_the_copy(counters, monkeypatch, tmp_path):
    out_root = tmp_path / "root"
    os.makedirs(out_root / "profiles")
    monkeypatch.setattr(bench, "ROOT", str(out_root))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abc")
    d = counters
    bench.write_traffic(str(d / "f"), str(d / "w"), str(d / "cf"), str(d / "cw"), bench.copy_calibration_bytes(256))
    rec = json.load(open(out_root / "profiles" / "traffic.json"))
    assert all(e["kernel_source_hash"] == "abc" for e in rec["launches"].values())
    assert rec["copy_calibration"]["fetch_factor"] == pytest.approx(0.5)
    assert rec["copy_calibration"]["write_factor"] == pytest.approx(1.0)
    l1, l8 = rec["launches"]["q8_0_4096x4096:m1"], rec["launches"]["q8_0_4096x4096:m8"]
    assert l1["dispatches"] == 2 and l8["dispatches"] == 2
    assert l1["fetch_bytes"] == round(8850.0 * 1024 / 0.5)          # mean KiB, / fetch factor
    assert l1["write_bytes"] == 16 * 1024
    assert l8["hbm_bytes"] == round(9330.0 * 1024 / 0.5) + 128 * 1024
    # algorithmic bytes: weights + x (m rows of k floats) + y (m rows of n floats)
    assert l1["algorithmic_bytes"] == 4096 * 4096 // 32 * 34 + 4 * 4096 + 4 * 4096
    assert l8["algorithmic_bytes"] == 4096 * 4096 // 32 * 34 + 8 * 4 * 4096 + 8 * 4 * 4096
    # the record is reported only for the sources it was taken on
    assert bench.measured_traffic("q8_0_4096x4096", 8) == l8["hbm_bytes"]
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "other")
    assert bench.measured_traffic("q8_0_4096x4096", 8) is None
    # a record for another workload, taken later on other sources, leaves the
    # first workload's entries in place with their own hash
    bench.write_traffic(str(d / "f"), str(d / "w"), str(d / "cf"), str(d / "cw"), bench.copy_calibration_bytes(256),
                        workload="q8_0_4096x4096_add_rmsnorm")
    rec = json.load(open(out_root / "profiles" / "traffic.json"))
    assert rec["launches"]["q8_0_4096x4096:m8"]["kernel_source_hash"] == "abc"
    assert rec["launches"]["q8_0_4096x4096_add_rmsnorm:m8"]["kernel_source_hash"] == "other"
    assert bench.measured_traffic("q8_0_4096x4096_add_rmsnorm", 8) is not None
    assert bench.measured_traffic("q8_0_4096x4096", 8) is None


def test_host_threads_stay_within_one_gpu_share():
    threads, avail = bench.host_threads()
    assert 1 <= threads <= bench.HOST_THREADS_PER_GPU and threads <= avail
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()


def test_copy_calibration_size_is_whole_vectors():
    assert bench.copy_calibration_bytes(256) == 256 << 20
    assert bench.copy_calibration_bytes(0.001) % 16 == 0


def test_kernel_source_hash_ignores_comments_not_code(tmp_path, monkeypatch):
    """Counters stay attached to the kernel code: comment and whitespace
    edits keep the hash, a code edit (even inside a string) changes it."""
    csrc = tmp_path / "quantized_few_row_amd" / "csrc"
    csrc.mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    src = 'int f(int a) { // one\n  return a + 1; /* two */ }\nconst char *s = "x // y";\n'
    (csrc / "k.hip").write_text(src)
    h0 = bench.kernel_source_hash()
    (csrc / "k.hip").write_text(src.replace("// one", "// another comment").replace("  return", "\treturn"))
    assert bench.kernel_source_hash() == h0
    (csrc / "k.hip").write_text(src.replace("a + 1", "a + 2"))
    assert bench.kernel_source_hash() != h0
    (csrc / "k.hip").write_text(src.replace('"x // y"', '"x // z"'))
    assert bench.kernel_source_hash() != h0


def test_variant_build_needs_its_own_output_path():
    """A macro override never replaces the product library."""
    import subprocess
    import sys
    res = subprocess.run([sys.executable, "-m", "quantized_few_row_amd._build", "-D", "REX_HALF_STEP_LANES=0"],
                         cwd=bench.ROOT, capture_output=True, text=True)
    assert res.returncode != 0 and "own --out" in res.stderr


def test_variant_objects_stay_apart_from_the_product_build(monkeypatch, tmp_path):
    """A variant build compiles into its own object folder under the build
    folder and links to the path it is given (compiler calls recorded, not run)."""
    from quantized_few_row_amd import _build
    calls = []

    class Done:
        returncode = 0
        stderr = ""

    def fake_run(cmd, **kw):
        calls.append(cmd)
        if "-shared" in cmd:
            open(cmd[cmd.index("-o") + 1], "w").close()
        return Done()

    monkeypatch.setattr(_build.subprocess, "run", fake_run)
    monkeypatch.setattr(_build, "hipcc", lambda: "hipcc")
    monkeypatch.setattr(_build, "BUILD", str(tmp_path / "_build"))
    out = str(tmp_path / "v" / "x.so")
    assert _build.build(jobs=1, out=out, defines=("REX_HALF_STEP_LANES=0",)) == out
    assert os.path.exists(out)
    compiles = [c for c in calls if "-c" in c]
    assert len(compiles) == len(_build.SOURCES)
    for c in compiles:
        assert "-DREX_HALF_STEP_LANES=0" in c
        assert os.path.dirname(c[c.index("-o") + 1]) == str(tmp_path / "_build" / "x.so.objs")


def test_missing_variant_is_refused():
    import quantized_few_row_amd as qfr
    with pytest.raises(qfr.LibraryMissing):
        qfr.load_variant("/nonexistent/variant.so")
