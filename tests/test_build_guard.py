"""The build's spill guard for kernels whose inline-asm LDS reads are waited on
later: its remark parser flags scratch and spills and finds the kernels."""
import pytest

from sparse_attention_04_amd.build import check_no_spills

R = "x.hip:1:1: remark: {} [-Rpass-analysis=kernel-resource-usage]"


def _remarks(name, scratch=0, vspill=0, sspill=0):
    return "\n".join(R.format(t) for t in [f"Function Name: {name}", "VGPRs: 256",
                                            f"ScratchSize [bytes/lane]: {scratch}", f"SGPRs Spill: {sspill}",
                                            f"VGPRs Spill: {vspill}"])


def test_clean_kernel_passes():
    assert check_no_spills(_remarks("_ZN3dsa15sfa_bf16_kernelI"), ("sfa_bf16_kernel",)) == []


@pytest.mark.parametrize("kw", [dict(scratch=16), dict(vspill=3)])
def test_spills_are_reported(kw):
    assert check_no_spills(_remarks("_ZN3dsa15sfa_bf16_kernelI", **kw), ("sfa_bf16_kernel",))


def test_sgpr_spills_to_vgpr_lanes_pass():
    # SGPR spills without scratch land in lanes of reserved VGPRs
    assert check_no_spills(_remarks("_ZN3dsa15sfa_bf16_kernelI", sspill=40), ("sfa_bf16_kernel",)) == []
    assert check_no_spills(_remarks("_ZN3dsa15sfa_bf16_kernelI", sspill=40, scratch=8), ("sfa_bf16_kernel",))


def test_other_kernels_are_ignored_but_some_must_be_seen():
    assert check_no_spills(_remarks("_ZN3dsa15sfa_bf16_kernelI") + "\n" + _remarks("other", scratch=8),
                           ("sfa_bf16_kernel",)) == []
    with pytest.raises(RuntimeError):
        check_no_spills(_remarks("other"), ("sfa_bf16_kernel",))


# ---- the device-assembly check for registers used before their LDS wait ----

from sparse_attention_04_amd.build import check_deferred_lds_waits  # noqa: E402


def _fn(body, name="_ZN3dsa15sfa_bf16_kernelI"):
    return f"{name}:                  ; @{name}\n" + "\n".join("\t" + l for l in body.strip().splitlines()) + "\n\ts_endpgm\n"


def _asm(ins):
    return f";;#ASMSTART\n{ins}\n;;#ASMEND"


def _check(body):
    return check_deferred_lds_waits(_fn(body), ("sfa_bf16_kernel",))


def test_copy_before_the_wait_is_flagged():
    bad = _check(_asm("ds_read_b128 v[2:5], v1 offset:64") + "\nv_mov_b64_e32 v[10:11], v[4:5]\ns_waitcnt lgkmcnt(0)")
    assert len(bad) == 1 and "v_mov_b64_e32" in bad[0]


def test_use_after_a_covering_wait_passes():
    assert _check(_asm("ds_read_b128 v[2:5], v1") + "\n" + _asm("s_waitcnt lgkmcnt(0)") +
                  "\nv_mfma_f32_16x16x32_bf16 a[0:3], v[2:5], v[6:9], a[0:3]") == []


def test_partial_wait_retires_the_older_reads_only():
    body = _asm("ds_read_b128 v[2:5], v1") + "\n" + _asm("ds_read_b128 v[12:15], v1 offset:16") + \
        "\n" + _asm("s_waitcnt lgkmcnt(1)")
    assert _check(body + "\nv_mov_b32_e32 v20, v3") == []
    assert len(_check(body + "\nv_mov_b32_e32 v20, v13")) == 1


def test_younger_compiler_reads_count_in_the_wait():
    body = _asm("ds_read_b128 v[2:5], v1") + "\nds_read_b32 v30, v31\ns_waitcnt lgkmcnt(1)\nv_mov_b32_e32 v20, v3"
    assert _check(body) == []


def test_outstanding_scalar_load_makes_partial_waits_unreliable():
    body = _asm("ds_read_b128 v[2:5], v1") + "\ns_load_dword s4, s[0:1], 0x10\ns_waitcnt lgkmcnt(1)\nv_mov_b32_e32 v20, v3"
    assert len(_check(body)) == 1


def test_overwriting_a_pending_register_is_flagged():
    assert len(_check(_asm("ds_read_b64_tr_b16 v[2:3], v1") + "\nv_mov_b32_e32 v3, 0\ns_waitcnt lgkmcnt(0)")) == 1


def test_stores_and_compiler_reads_are_not_checked_themselves():
    body = "ds_read_b32 v5, v1\nv_mov_b32_e32 v6, v5\n" + _asm("ds_read_b128 v[8:11], v1") + \
        "\nds_write_b32 v1, v7\ns_waitcnt lgkmcnt(0)\nv_add_u32_e32 v12, v8, v9"
    assert _check(body) == []


def test_other_functions_are_skipped_but_one_must_be_found():
    other = _fn(_asm("ds_read_b128 v[2:5], v1") + "\nv_mov_b32_e32 v9, v2", name="other_kernel")
    assert check_deferred_lds_waits(other + _fn("s_nop 0"), ("sfa_bf16_kernel",)) == []
    with pytest.raises(RuntimeError):
        check_deferred_lds_waits(other, ("sfa_bf16_kernel",))
