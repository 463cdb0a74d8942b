"""The rocprofv3 summariser on a small committed sample of its own CSV output (two
dispatches of the 4096^3 FP32 kernel and two of the 64 MiB device copy per counter
pass), against figures derived by hand from those rows; and the committed counter
summaries against the current sources (a summary taken before a kernel or the
configuration choice changed would make the benchmark report no traffic figure)."""
import glob
import os

import pytest

from linear_algebra_sgemm_amd import cost, profile_summary as ps

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FIX = os.path.join(ROOT, "tests", "fixtures", "rocprof")
KERNEL = ("void lasg::sgemm_dma_kernel<lasg::SDmaTile<256, 256, 4, 2, 2, 4, false>, false, "
          "false>(lasg::SgemmArgs)")


def _summary():
    passes = [os.path.join(FIX, "sgemm_4096_%s.csv" % t) for t in ("FETCH", "WRITE", "MFMA",
                                                                     "MOPS", "CLK")]
    return ps.counters_markdown("sgemm_4096", "sgemm", cost.gemm_flops(4096, 4096, 4096),
                                cost.sgemm_bytes(4096, 4096, 4096, 0.5), 4096 * 4096 * 4, passes,
                                ["cmd %d" % i for i in range(5)])


def test_counter_summary_figures():
    text = _summary()
    # fetch scale 65536 / median(32786.0625, 32779.5) KiB; write scale 65536 / 65536;
    # kernel: mean FETCH 229521.9375 KiB, mean WRITE 65536 KiB
    fs = 65536 / ((32786.0625 + 32779.5) / 2)
    want = 229521.9375 * 1024 * fs + 65536 * 1024
    got = float(text.split("hbm_bytes_per_launch:")[1].split()[0])
    assert abs(got - want) <= 1.0
    # MOPS_F32 268435456 per dispatch x 512 = 2 * 4096^3 exactly
    assert "ratio useful / executed = 1.0000" in text
    # GRBM_GUI_ACTIVE mean 18208199 over the CLK pass's mean duration 1081998 ns, 8 XCDs
    assert "= 2.104 GHz" in text
    assert "0 of 3.369e+07 active LDS cycles (0.00 %)" in text
    assert "| `%s` | 2 | MfmaUtil | 88.4137 |" % KERNEL in text
    assert "kernel_source_sha256: %s" % ps.source_digest("sgemm") in text
    assert "effective_clock_ghz: 2.104" in text and "mfma_util_pct: 88.41" in text


def test_trace_summary_table():
    text = ps.trace_markdown("sgemm_4096", os.path.join(FIX, "sgemm_4096_kernel_stats.csv"), "cmd")
    rows = [l for l in text.splitlines() if l.startswith("| `")]
    assert rows[0].startswith("| `%s` | 200 | 946508 |" % KERNEL)
    assert "__amd_rocclr_copyBuffer" in rows[1]


def test_calibration_needs_the_known_copy():
    w = ps.dispatches(os.path.join(FIX, "sgemm_4096_WRITE.csv"))
    f = ps.dispatches(os.path.join(FIX, "sgemm_4096_FETCH.csv"))
    with pytest.raises(ValueError):
        ps.copy_scale(w, f, 12345 * 1024)


COUNTER_FILES = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_counters.md")))


def test_every_workload_has_a_counter_summary():
    from linear_algebra_sgemm_amd import inputs
    names = {os.path.basename(p)[:-len("_counters.md")] for p in COUNTER_FILES}
    assert set(inputs.WORKLOADS) <= names


@pytest.mark.parametrize("path", COUNTER_FILES, ids=os.path.basename)
def test_counter_summaries_belong_to_the_current_sources(path):
    import bench
    from linear_algebra_sgemm_amd import inputs
    name = os.path.basename(path)[:-len("_counters.md")]
    w = inputs.WORKLOADS[name]
    traffic = bench.profiled_traffic(name, w.op)
    assert traffic is not None, "%s is stale: re-profile this workload" % path
    assert traffic > 0


def test_digest_ignores_comments_but_not_code():
    src = "int f(int x) {  // add one\n  return x + 1; /* the\n result */\n}\n"
    same = "int f(int x) {\n  return x + 1;   // a different comment\n}\n"
    other = "int f(int x) {  // add one\n  return x + 2;\n}\n"
    assert ps.code_only(src) == ps.code_only(same)
    assert ps.code_only(src) != ps.code_only(other)
