"""The build's check that the compiler leaves M0 to the copy asm of the GEMM
kernels (which writes it without saving it), on hand-written assembly."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from structured_sparse_gemm_nm_amd import build  # noqa: E402

OK = """\
kernel:
\t;;#ASMSTART
\ts_mov_b32 m0, s38
\ts_nop 0
\tglobal_load_lds_dwordx4 v[138:139], off
\t;;#ASMEND
\tds_read_b128 v[0:3], v4 offset:16 ; reads LDS, no m0
\ts_endpgm
"""


def _check(tmp_path, text):
    p = tmp_path / "k.s"
    p.write_text(text)
    return build.check_m0_unused(str(p))


def test_copy_asm_alone_passes(tmp_path):
    assert _check(tmp_path, OK) == []


def test_compiler_uses_of_m0_are_reported(tmp_path):
    for line in ["\ts_mov_b32 m0, -1", "\tv_movrel_b32 v0, v1", "\tglobal_load_lds_dword v[0:1], off",
                 "\tbuffer_load_dword v1, off, s[0:3], 0 lds", "\ts_sendmsg sendmsg(MSG_DEALLOC_VGPRS)",
                 "\tv_readlane_b32 s0, v1, m0"]:
        assert _check(tmp_path, OK.replace("\ts_endpgm", line + "\n\ts_endpgm")) == [line.strip()], line


def test_the_built_gemm_unit_passes():
    asm = os.path.join(build.BUILD, "m0_check.s")
    if not os.path.exists(asm):
        import pytest
        pytest.skip("library not built here")
    assert build.check_m0_unused(asm) == []
