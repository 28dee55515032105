"""Every DPP lane exchange in the compiled kernels runs with a full exec mask
(CPU: compiles the kernel sources to gfx950 assembly with the library's flags)."""
import os
import shutil
import subprocess

import pytest

from dpp_exec import scan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

BAD = """_Zbad:
	v_cmp_eq_u32_e32 vcc, 0, v1
	s_and_saveexec_b64 s[0:1], vcc
	v_mov_b32_dpp v2, v3 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1
	s_or_b64 exec, exec, s[0:1]
	s_endpgm
.Lfunc_end0:
"""
GOOD = """_Zgood:
	v_cmp_eq_u32_e32 vcc, 0, v1
	s_and_saveexec_b64 s[0:1], vcc
	s_cbranch_execz .LBB0_2
	v_add_u32_e32 v2, 1, v2
.LBB0_2:
	s_or_b64 exec, exec, s[0:1]
	v_mov_b32_dpp v2, v3 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1
	s_endpgm
.Lfunc_end0:
"""


def test_scanner_on_small_programs():
    assert scan(BAD) == {"_Zbad": (1, 1)}
    assert scan(GOOD) == {"_Zgood": (1, 0)}


@pytest.mark.parametrize("src", ["quantize.hip", "misc.hip"])
def test_compiled_kernels_exchange_with_full_exec(src, tmp_path):
    from precision_rl_amd import build
    if not os.path.exists(build.HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    out = tmp_path / (src + ".s")
    subprocess.run([build.HIPCC, *build.FLAGS, "--cuda-device-only", "-S",
                    os.path.join(build.CSRC, src), "-o", str(out)], check=True, capture_output=True)
    res = scan(out.read_text())
    assert res, "no kernels found"
    bad = {k: v for k, v in res.items() if v[1]}
    assert not bad, bad
    if src == "quantize.hip":
        assert sum(v[0] for v in res.values()) > 0   # the exchanges are there
