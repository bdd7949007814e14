"""The build's guard on the compiler's per-kernel report: a kernel that uses
scratch (private) memory, or a requested unroll that did not happen, fails
the build (both once turned a quantizer's register array into scratch
traffic with only a warning)."""

import pytest

from fp8_fine_grained_quant_amd.build import check_resource_report

SRC = "x.hip:10:1: "
TAG = " [-Rpass-analysis=kernel-resource-usage]"


def _report(scratch):
    return "\n".join([
        SRC + "remark: Function Name: _Z1kv" + TAG,
        SRC + "remark:     VGPRs: 91" + TAG,
        SRC + f"remark:     ScratchSize [bytes/lane]: {scratch}" + TAG,
        "some other warning",
    ])


def test_clean_report_passes_other_lines_through():
    assert check_resource_report("x.hip", _report(0)) == "some other warning"


def test_scratch_use_fails_the_build():
    with pytest.raises(RuntimeError, match="_Z1kv"):
        check_resource_report("x.hip", _report(272))


def test_missed_unroll_fails_the_build():
    rep = _report(0) + "\nx.hip:207:3: warning: loop not unrolled: the optimizer was unable to perform"
    with pytest.raises(RuntimeError, match="loop not unrolled"):
        check_resource_report("x.hip", rep)
