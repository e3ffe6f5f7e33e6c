"""The MFMA kernels' device assembly keeps the rules of tests/asm_hazards.py
(no use of a register while an asm LDS read into it is in flight; two wait
states between a VALU write and an MFMA read of a VGPR; a wait state
between a wide store and a write of its data registers), and no kernel uses
scratch memory. Host only: the kernels are compiled for gfx950 to assembly
with the library's own flags. The checker itself is first shown to catch
planted violations in small hand-written sequences."""
import importlib.util
import os
import re
import subprocess

import pytest

from asm_hazards import check

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "_tpmlp_build", os.path.join(ROOT, "tensor_transformer_mlp_rank_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    return b


TOY = """
_Ztoy:
\tds_read_b128 v[4:7], v1 offset:0
\tv_mov_b32 v5, 0
\ts_waitcnt lgkmcnt(0)
\tv_mov_b64_e32 v[8:9], v[4:5]
\tv_mfma_f32_16x16x32_bf16 a[0:3], v[8:11], v[12:15], a[0:3]
\ts_endpgm
.Lfunc_end0:
_Zclean:
\tds_read_b128 v[4:7], v1 offset:0
\tds_read_b128 v[8:11], v1 offset:16
\ts_waitcnt lgkmcnt(1)
\tv_add_u32_e32 v20, v4, v5
\ts_waitcnt lgkmcnt(0)
\tv_mov_b32 v12, 0
\ts_nop 1
\tv_mov_b32 v13, 0
\ts_nop 0
\ts_nop 0
\tv_mfma_f32_16x16x32_bf16 a[0:3], v[8:11], v[12:15], a[0:3]
\ts_endpgm
.Lfunc_end1:
_Zloop:
\tds_read_b128 v[4:7], v1 offset:0
.LBB2_1:
\tv_add_u32_e32 v4, 1, v4
\ts_waitcnt lgkmcnt(0)
\tds_read_b128 v[4:7], v1 offset:0
\ts_cbranch_scc1 .LBB2_1
\ts_endpgm
.Lfunc_end2:
_Zstore:
\tglobal_store_dwordx4 v[8:9], a[0:3], off
\tv_accvgpr_write_b32 a1, v250
\tglobal_store_dwordx4 v[8:9], a[0:3], off
\ts_nop 0
\tv_accvgpr_write_b32 a1, v250
\tbuffer_store_dwordx4 v[4:7], v1, s[0:3], 0 offen
\tv_mov_b32_e32 v5, 0
\tglobal_store_dwordx2 v[8:9], v[2:3], off
\tv_mov_b32_e32 v2, 0
\ts_endpgm
.Lfunc_end3:
"""


def test_checker_catches_planted_violations():
    r = check(TOY)
    assert r["_Ztoy"]["inflight"] == ["v_mov_b32 v5, 0"]
    assert r["_Ztoy"]["valu_mfma"] == [
        "v_mfma_f32_16x16x32_bf16 a[0:3], v[8:11], v[12:15], a[0:3]"]
    assert r["_Zclean"] == {"inflight": [], "valu_mfma": [], "store_data": []}
    # a 16-byte store's data registers written by the next instruction (twice);
    # after a wait state, or for an 8-byte store, no finding
    assert r["_Zstore"]["store_data"] == ["v_accvgpr_write_b32 a1, v250",
                                          "v_mov_b32_e32 v5, 0"]
    # the read at the bottom of the loop is still in flight at the top
    assert r["_Zloop"]["inflight"] == ["v_add_u32_e32 v4, 1, v4"]


@pytest.fixture(scope="module")
def mfma_asm(tmp_path_factory):
    b = _build_module()
    out = tmp_path_factory.mktemp("asm") / "kernels_mfma.s"
    cmd = [b.HIPCC, *b.CFLAGS, "--cuda-device-only", "-S",
           os.path.join(b.CSRC, "kernels_mfma.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def test_mfma_kernels_keep_the_asm_rules(mfma_asm):
    res = check(mfma_asm, prefix="_ZN5tpmlp16gemm_mfma_kernel")
    assert len(res) >= 20
    bad = {k[:90]: v for k, v in res.items()
           if v["inflight"] or v["valu_mfma"] or v["store_data"]}
    assert not bad, bad


def test_mfma_kernels_use_no_scratch(mfma_asm):
    sizes = re.findall(r'\.private_segment_fixed_size:\s+(\d+)', mfma_asm)
    assert sizes and all(int(v) == 0 for v in sizes), sorted(set(sizes))
