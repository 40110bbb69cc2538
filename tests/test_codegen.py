"""Properties of the generated gfx950 code, checked on the CPU from hipcc's assembly.

* No kernel spills to scratch.
* No compiler-generated instruction touches a register that an inline-asm LDS
  read is still filling (the kernels wait for those reads explicitly; a copy,
  spill or use placed by the compiler before the wait would see data that has
  not arrived). Checked by a dataflow walk over each kernel's control-flow graph.
* Kernels that read LDS from inline asm and are compiled with MFMA results in
  arch VGPRs use no AGPRs at all.
* No packed fp32 instructions (v_pk_fma_f32, v_pk_mul_f32, v_pk_add_f32)
  anywhere in the device code.
"""
import re
import shutil

import pytest

from _lds_hazards import asm_lds_reads, check_kernel
from io_aware_tiled_07_amd import build as fabuild

HIP_SOURCES = [s for s in fabuild.SOURCES if s.endswith(".hip")]


@pytest.fixture(scope="module", params=HIP_SOURCES)
def asm(request):
    try:
        fabuild.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    return request.param, fabuild.device_asm(request.param)


def kernels(text):
    """(name, body) of every kernel function in the assembly."""
    funcs = set(re.findall(r"^\s*\.type\s+(_Z\w+),@function", text, flags=re.M))
    names = [n for n in re.findall(r"^(_Z\w+):\s", text, flags=re.M) if n in funcs]  # not data (e.g. __device__ arrays)
    out = []
    for n in names:
        start = text.index(f"\n{n}:")
        end = text.index(".Lfunc_end", start)
        out.append((n, text[start:end]))
    return out


def test_no_spills(asm):
    src, text = asm
    ks = kernels(text)
    assert ks, f"no kernels found in {src}"
    for name, body in ks:
        assert "scratch_" not in body and "buffer_store_dword" not in body, f"{src}: {name} spills to scratch"
        if src not in fabuild.AGPR_SOURCES and asm_lds_reads(body):
            assert "v_accvgpr" not in body, f"{src}: {name} uses AGPRs"
    for m in re.finditer(r"; ScratchSize: (\d+)", text):
        assert m.group(1) == "0", f"{src}: scratch in use"


def test_asm_lds_reads_are_waited_for(asm):
    src, text = asm
    for name, body in kernels(text):
        bad = check_kernel(body)
        assert not bad, f"{src}: {name} touches in-flight LDS data: {bad[:4]}"


def test_backward_kernels_read_lds_from_asm(asm):
    """The hazard check above has something to check in the backward kernels."""
    src, text = asm
    if src not in ("fa_bwd.hip", "fa_bwd128.hip"):
        pytest.skip("forward / other files")
    for name, body in kernels(text):
        if "fused" in name:
            assert asm_lds_reads(body) > 50, name


SYNTH = """
_Zk:
  s_load_dwordx2 s[0:1], s[4:5], 0x0
  ;;#ASMSTART
  ds_read_b128 v[4:7], v1 offset:16
  ;;#ASMEND
  ;;#ASMSTART
  ds_read_b64_tr_b16 v[8:9], v1 offset:32
  ;;#ASMEND
  {early}
  ;;#ASMSTART
  s_waitcnt lgkmcnt(1)
  ;;#ASMEND
  v_mov_b32 v20, v5
  {middle}
  s_cbranch_scc0 .LBB0_2
  ;;#ASMSTART
  s_waitcnt lgkmcnt(0)
  ;;#ASMEND
.LBB0_2:
  {late}
  s_endpgm
.Lfunc_end0:
"""


@pytest.mark.parametrize("early,middle,late,flagged", [
    ("", "", "", 0),
    ("v_accvgpr_write_b32 a0, v6", "", "", 1),   # copy of a read before any wait
    ("", "v_add_f32_e32 v21, v8, v20", "", 1),   # second read not retired by lgkmcnt(1)
    ("", "", "v_mov_b32 v22, v9", 1),            # waited on one path only
    ("", "", "v_mov_b32 v22, v7", 0),            # first read retired on every path
    ("", "v_mov_b32 v9, 0", "", 1),              # overwrite of an in-flight destination
])
def test_hazard_check_on_synthetic_code(early, middle, late, flagged):
    body = SYNTH.format(early=early, middle=middle, late=late)
    assert len(check_kernel(body)) == flagged


def test_no_packed_fp32(asm):
    src, text = asm
    for op in ("v_pk_fma_f32", "v_pk_mul_f32", "v_pk_add_f32"):
        assert op not in text, f"{src} contains {op}"
