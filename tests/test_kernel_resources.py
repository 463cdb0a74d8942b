"""Every kernel instance of the library fits its register file without spilling.

Register arrays that do not fit are spilled to scratch memory in HBM ("local
memory"), the trap the register-array and register-accounting sections of
"SGEMM优化，从naive到warptiling" (kernels k5 and k10) warn against.  Each HIP
source is compiled here for gfx950 with the library's own flags and the
compiler's kernel-resource-usage remarks; every instance must report zero
scratch bytes and zero spilled VGPRs, registers within what its occupancy
allows, and LDS within 160 KiB.  No instance is exempt.  (Compiling both large
sources takes about a minute.)"""
import pytest

from linear_algebra_sgemm_amd import resource_usage


@pytest.fixture(scope="module")
def kernels():
    return resource_usage.all_kernels()


def test_every_source_has_kernels(kernels):
    srcs = {src for src, _ in kernels}
    assert {"sgemm_kernels.hip", "hgemm_kernels.hip", "pack_kernels.hip"} <= srcs
    # the headline FP32 kernel and both FFN kernels are among them
    names = " ".join(r["demangled"] for _, r in kernels)
    assert "sgemm_dma_kernel<lasg::SDmaTile<256, 256, 4, 2, 2, 4" in names
    assert "hgemm_dma_kernel<lasg::HDmaTile<lasg::EltBF16, 256, 256, 32, 4, 2, 2, 4>" in names


def test_no_instance_spills_or_exceeds_its_budget(kernels):
    bad = ["%s: %s (%s)" % (src, r["demangled"], "; ".join(resource_usage.over_budget(r)))
           for src, r in kernels if resource_usage.over_budget(r)]
    assert not bad, "\n".join(bad)


def test_the_remark_parser_reads_every_field(kernels):
    for _, r in kernels:
        for key in ("vgprs", "agprs", "sgprs", "scratch", "vgpr_spill", "lds", "occupancy"):
            assert key in r, (key, r["demangled"])
