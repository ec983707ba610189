"""Host-side checks of the build script (no GPU, no compiler): the parser of hipcc's resource-usage remarks
that rejects kernels with scratch memory."""
import pytest

from gaussian_mixture_token_amd import build

# the two forms hipcc prints the remarks in: location first (a plain compile) and "remark:" first (under
# -save-temps, which the build uses to check the assembly)
PLAIN = """\
/src/k.hip:10:1: remark: Function Name: _Z3fooPf [-Rpass-analysis=kernel-resource-usage]
/src/k.hip:10:1: remark:     VGPRs: 64 [-Rpass-analysis=kernel-resource-usage]
/src/k.hip:10:1: remark:     ScratchSize [bytes/lane]: {scratch} [-Rpass-analysis=kernel-resource-usage]
/src/k.hip:10:1: remark:     VGPRs Spill: {spill} [-Rpass-analysis=kernel-resource-usage]
"""
SAVE_TEMPS = """\
remark: /src/k.hip:10:0: Function Name: _Z3fooPf [-Rpass-analysis=kernel-resource-usage]
remark: /src/k.hip:10:0:     VGPRs: 64 [-Rpass-analysis=kernel-resource-usage]
remark: /src/k.hip:10:0:     ScratchSize [bytes/lane]: {scratch} [-Rpass-analysis=kernel-resource-usage]
remark: /src/k.hip:10:0:     VGPRs Spill: {spill} [-Rpass-analysis=kernel-resource-usage]
"""


@pytest.mark.parametrize("form", [PLAIN, SAVE_TEMPS], ids=["plain", "save-temps"])
def test_clean_kernel_passes(form):
    build._check_resources("k.hip", form.format(scratch=0, spill=0))


@pytest.mark.parametrize("form", [PLAIN, SAVE_TEMPS], ids=["plain", "save-temps"])
@pytest.mark.parametrize("scratch,spill", [(80, 0), (12, 2)])
def test_scratch_or_spill_is_rejected(form, scratch, spill):
    with pytest.raises(RuntimeError, match="_Z3fooPf"):
        build._check_resources("k.hip", form.format(scratch=scratch, spill=spill))


def test_listed_kernel_is_allowed():
    name = sorted(build.SCRATCH_ALLOWED)[0]
    build._check_resources("k.hip", SAVE_TEMPS.replace("_Z3fooPf", name).format(scratch=28, spill=6))
