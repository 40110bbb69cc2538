"""Properties of the generated gfx950 code, checked on the CPU from hipcc's assembly.

* No kernel spills to scratch, and no kernel that reads LDS from inline asm
  (and waits for the data explicitly) copies registers through AGPRs: a spill
  or copy placed by the compiler between such a read and its wait would copy
  data that has not arrived yet. (MFMA results live in arch VGPRs.)
* No packed fp32 instructions (v_pk_fma_f32, v_pk_mul_f32, v_pk_add_f32)
  anywhere in the device code.
"""
import re
import shutil

import pytest

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
    names = re.findall(r"^(_Z\w+):\s", text, flags=re.M)
    out = []
    for n in names:
        start = text.index(f"\n{n}:")
        end = text.index(".Lfunc_end", start)
        out.append((n, text[start:end]))
    return out


def test_no_spills_or_agpr_copies(asm):
    src, text = asm
    ks = kernels(text)
    assert ks, f"no kernels found in {src}"
    for name, body in ks:
        asm_lds = re.search(r";;#ASMSTART\s*\n\s*ds_read", body) is not None
        if asm_lds:
            assert "v_accvgpr_write" not in body and "v_accvgpr_read" not in body, \
                f"{src}: {name} copies through AGPRs"
        assert "scratch_" not in body and "buffer_store_dword" not in body, f"{src}: {name} spills to scratch"
    for m in re.finditer(r"; ScratchSize: (\d+)", text):
        assert m.group(1) == "0", f"{src}: scratch in use"


def test_no_packed_fp32(asm):
    src, text = asm
    for op in ("v_pk_fma_f32", "v_pk_mul_f32", "v_pk_add_f32"):
        assert op not in text, f"{src} contains {op}"
