"""The C ABI from plain C: tests/c_consumer/consumer.c includes
include/segattn.h, is compiled as C99 with every warning an error, links
against the in-tree libsegattn.so and calls the host planners and two
error paths that return before any device work (so it runs without a GPU).
Its printed results must equal the float64 / integer oracle's."""

import os
import shutil
import subprocess

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "segmented_causal_attention_amd")
SEGATTN_E_INVALID, SEGATTN_E_CAPACITY, SEGATTN_E_WORKSPACE = 1, 4, 5


@pytest.fixture(scope="module")
def output(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    if not os.path.exists(os.path.join(PKG, "libsegattn.so")):
        pytest.skip("libsegattn.so not built")
    exe = str(tmp_path_factory.mktemp("c_consumer") / "consumer")
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "c_consumer", "consumer.c"), "-L", PKG, "-lsegattn", f"-Wl,-rpath,{PKG}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    out = {}
    for line in r.stdout.splitlines():
        key, _, val = line.partition(": ")
        out.setdefault(key, []).append(val)
    return out


def ints(s):
    return [int(x) for x in s.split()]


def test_partition(output):
    assert output["partition_status"] == ["0"]
    assert ints(output["partition"][0]) == oracle.partition(1024, 4)


def test_varlen_capacity_query_then_items(output):
    cu = [0, 5000, 5001, 45001]
    ref = [list(map(int, it)) for it in oracle.partition_varlen(cu, 16384)]
    assert ints(output["varlen_query"][0]) == [SEGATTN_E_CAPACITY, len(ref)]
    assert ints(output["varlen_status"][0]) == [0, len(ref)]
    assert [ints(s) for s in output["varlen_item"]] == ref


def test_ring_items(output):
    ref = [list(map(int, it)) for it in oracle.ring_items([0, 512, 1024], 256)]
    assert ints(output["ring_status"][0]) == [0, len(ref)]
    assert [ints(s) for s in output["ring_item"]] == ref


def test_offload_plan_exact(output):
    rows, row_bytes, th = [3765, 3765, 2116], [16512] * 3, 30000000.0
    alpha, mem, peak = oracle.plan_offload([r * b for r, b in zip(rows, row_bytes)], th)
    assert output["offload_status"] == ["0"]
    assert [float(x) for x in output["offload_alpha"][0].split()] == alpha
    assert ints(output["offload_moved"][0]) == [oracle.offload_rows(a, r) for a, r in zip(alpha, rows)]
    assert float(output["offload_peak"][0]) == peak


def test_error_paths_return_before_device_work(output):
    st, rest = output["fwd_null_shape"][0].split(" ", 1)
    assert int(st) == SEGATTN_E_INVALID and rest.startswith("SEGATTN_E_INVALID | segattn_fwd: shape")
    assert output["fwd_workspace"] == ["0 positive"]
    assert output["fwd_small_workspace"] == [f"{SEGATTN_E_WORKSPACE} SEGATTN_E_WORKSPACE"]
