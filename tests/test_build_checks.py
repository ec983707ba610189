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


ASM = """\
{name}:
\tbuffer_load_dwordx4 v0, s[0:3], 0 offen lds
\ts_barrier
\tbuffer_load_dwordx4 v0, s[0:3], 0 offen lds
\t{op}
\tbuffer_store_dwordx4 v[0:3], v4, s[0:3], 0 offen
\ts_endpgm
"""
TOK = "_ZN3gma10tok_kernelILi128ELi128ELi128ELi5ELi1EEEvNS_8MainArgsE"
DMA_MAIN = "_ZN3gma11main_kernelILb0ELi128ELi64ELi128ELi4ELi32ELi0ELb1ELi2EEEvNS_8MainArgsE"
PLAIN_MAIN = "_ZN3gma11main_kernelILb0ELi128ELi64ELi128ELi4ELi32ELi0ELb0ELi2EEEvNS_8MainArgsE"


@pytest.mark.parametrize("name", [TOK, DMA_MAIN])
def test_dma_loop_with_only_dma_loads_and_stores_passes(tmp_path, name):
    f = tmp_path / "k.s"
    f.write_text(ASM.format(name=name, op="s_nop 0"))
    assert build._check_vmem_in_loops(str(f)) == 1


@pytest.mark.parametrize("op", ["global_load_dword v1, v[2:3], off", "scratch_store_dword off, v1, s0",
                                "buffer_load_dword v1, v2, s[0:3], 0 offen"])
@pytest.mark.parametrize("name", [TOK, DMA_MAIN])
def test_dma_loop_with_another_load_is_rejected(tmp_path, name, op):
    f = tmp_path / "k.s"
    f.write_text(ASM.format(name=name, op=op))
    with pytest.raises(RuntimeError, match="unexpected vector-memory"):
        build._check_vmem_in_loops(str(f))


def test_register_staged_kernel_is_not_an_exact_count_kernel(tmp_path):
    f = tmp_path / "k.s"
    f.write_text(ASM.format(name=PLAIN_MAIN, op="global_load_dword v1, v[2:3], off"))
    assert build._check_vmem_in_loops(str(f)) == 0
