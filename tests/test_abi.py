"""The C-ABI library on the CPU: it loads, exports every function include/fa.h
declares, and rejects bad arguments before any HIP call (no kernel is launched
in these tests)."""
import ctypes
import os
import re

import pytest

import io_aware_exact_07_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "fa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"fa_fwd", "fa_bwd", "fa_bwd_workspace_bytes", "fa_status_string"} <= set(names)
    lib = ctypes.CDLL(fa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


FAKE = 0x100000  # 16-byte aligned, never dereferenced: every call below fails validation first


def fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, N=128, d=64, scale=0.125, causal=0, seqlens=None,
             dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.fa_fwd(*a.values())


def bwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, dO=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1, H=1, N=128, d=64,
             scale=0.125, causal=0, seqlens=None, workspace=FAKE, workspace_bytes=1 << 40, dtype=fa.FA_BF16,
             stream=None)
    a.update(kw)
    return fa.fa_bwd(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(lse=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=FAKE + 2), fa.FA_ERR_INVALID_ARG),          # misaligned
    (dict(seqlens=FAKE + 2), fa.FA_ERR_INVALID_ARG),
    (dict(d=80), fa.FA_ERR_UNSUPPORTED),
    (dict(d=32), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=7), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=-1.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(B=-1), fa.FA_ERR_INVALID_ARG),
    (dict(N=-5), fa.FA_ERR_INVALID_ARG),
    (dict(N=(1 << 24) + 1), fa.FA_ERR_INVALID_ARG),
    (dict(B=1 << 16, H=1 << 16), fa.FA_ERR_INVALID_ARG),   # B*H beyond 2^31 - 1
    (dict(H=1 << 15, N=1 << 24), fa.FA_ERR_INVALID_ARG),   # 2*B*H*ceil(N/128) = 2^33 workgroups
    (dict(B=0), fa.FA_OK),                              # empty: nothing to do, nothing launched
    (dict(N=0, q=None), fa.FA_OK),
])
def test_forward_validation(kw, status):
    assert fwd(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(dO=None), fa.FA_ERR_INVALID_ARG),
    (dict(dq=FAKE + 4), fa.FA_ERR_INVALID_ARG),
    (dict(workspace=None), fa.FA_ERR_WORKSPACE),
    (dict(workspace_bytes=100), fa.FA_ERR_WORKSPACE),
    (dict(workspace=FAKE + 8), fa.FA_ERR_WORKSPACE),
    (dict(d=256), fa.FA_ERR_UNSUPPORTED),
    (dict(H=1 << 15, N=1 << 24), fa.FA_ERR_INVALID_ARG),   # launch grid beyond 32 bits
    (dict(H=0), fa.FA_OK),
])
def test_backward_validation(kw, status):
    assert bwd(**kw) == status


def test_stage_validation():
    ws = fa.fa_bwd_workspace_bytes(1, 1, 128, 64, fa.FA_BF16)
    assert fa.fa_bwd_prepare(None, FAKE, FAKE, 1, 1, 128, 64, None, FAKE, ws, fa.FA_BF16, None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_bwd_prepare(FAKE, FAKE, None, 1, 1, 128, 64, None, FAKE, ws, fa.FA_BF16, None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_bwd_prepare(FAKE, FAKE, FAKE, 1, 1, 128, 64, None, FAKE, ws - 1, fa.FA_BF16, None) == fa.FA_ERR_WORKSPACE
    assert fa.fa_bwd_dkdv(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 1, 1, 128, 64, 0.1, 1, None, FAKE, ws,
                          fa.FA_BF16, None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_bwd_dkdv(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 1, 128, 64, 0.1, 1, None, FAKE, ws,
                          fa.FA_BF16, None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_bwd_dq(FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 1, 128, 64, 0.1, 1, None, FAKE, ws, fa.FA_BF16,
                        None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_bwd_dq(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 128, 64, 0.1, 1, None, FAKE, ws, 3,
                        None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_bwd_dq(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 128, 64, 0.1, 1, None, None, ws, fa.FA_BF16,
                        None) == fa.FA_ERR_WORKSPACE
    assert fa.fa_bwd_dkdv_dq(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 1, 128, 64, 0.1, 1, None, FAKE, ws,
                             fa.FA_BF16, None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_bwd_dkdv_dq(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 128, 64, 0.1, 1, None, FAKE, 8,
                             fa.FA_BF16, None) == fa.FA_ERR_WORKSPACE


def test_noalloc_validation_and_size_limit():
    """The allocation-free backward validates like fa_bwd and rejects problems
    whose row vectors exceed its static array before any HIP call."""
    def na(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, dO=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1, H=1, N=128, d=64,
                 scale=0.125, causal=0, seqlens=None, dtype=fa.FA_BF16, stream=None)
        a.update(kw)
        return fa.fa_bwd_noalloc(*a.values())
    assert na(dq=None) == fa.FA_ERR_INVALID_ARG
    assert na(lse=FAKE + 2) == fa.FA_ERR_INVALID_ARG
    assert na(d=80) == fa.FA_ERR_UNSUPPORTED
    assert na(B=0) == fa.FA_OK
    limit = fa.FA_NOALLOC_SCRATCH_BYTES
    # 2^21 padded rows fill the array exactly; one more 128-row block does not fit
    assert fa.fa_bwd_workspace_bytes(1, 16, 1 << 17, 64, fa.FA_BF16) == limit
    assert fa.fa_bwd_workspace_bytes(1, 16, (1 << 17) + 1, 64, fa.FA_BF16) > limit
    assert na(H=16, N=(1 << 17) + 1) == fa.FA_ERR_SCRATCH
    assert na(B=64, H=64, N=1024) == fa.FA_ERR_SCRATCH
    assert "scratch" in fa.fa_status_string(fa.FA_ERR_SCRATCH)


def test_workspace_is_linear_in_N_and_holds_row_vectors():
    for dt in (fa.FA_BF16, fa.FA_FP32):
        for d in (64, 96, 128):
            ws = [fa.fa_bwd_workspace_bytes(2, 3, n, d, dt) for n in (512, 1024, 2048, 4096)]
            assert all(b == 2 * a for a, b in zip(ws, ws[1:]))
            assert ws[0] == 2 * (2 * 3 * 512 * 4)   # D and lse2: one float32 each per row
            # rows are padded to whole 128-row blocks per head
            assert fa.fa_bwd_workspace_bytes(1, 1, 129, d, dt) == 2 * 256 * 4
    assert fa.fa_bwd_workspace_bytes(1, 1, 128, 80, fa.FA_BF16) == 0
    assert fa.fa_bwd_workspace_bytes(0, 1, 128, 64, fa.FA_BF16) == 0


def test_status_strings():
    for s in (fa.FA_OK, fa.FA_ERR_INVALID_ARG, fa.FA_ERR_UNSUPPORTED, fa.FA_ERR_WORKSPACE, fa.FA_ERR_HIP,
              fa.FA_ERR_SCRATCH):
        assert fa.fa_status_string(s) and fa.fa_status_string(s) != "unknown status"
    assert fa.fa_status_string(12345) == "unknown status"
