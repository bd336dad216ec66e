"""Host-side checks of libvit.so that need no GPU.

* the library loads and exports every function include/vit.h declares, and the
  binding's signature table covers exactly those;
* argument validation rejects bad calls with the documented status before any
  HIP runtime call (null pointers are never dereferenced);
* pure host queries (block size, work-list capacity) return the documented values.
"""
import ctypes
import os
import re

import pytest

from vision_encoder_varlen_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vit.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(vit_[a-z0-9_]+)\s*\(", text,
                       flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("vit_qk_norm_rope", "vit_varlen_attn", "vit_varlen_attn_f32",
                     "vit_varlen_worklist", "vit_varlen_attn_planned", "vit_attn_block_m",
                     "vit_worklist_capacity", "vit_device_error", "vit_last_error", "vit_release",
                     "vit_time_next_kernel", "vit_qk_norm_rope_worklist",
                     "vit_varlen_attn_lse", "vit_varlen_attn_strided",
                     "vit_qk_norm_rope_strided", "vit_dense_batch_attn", "vit_qk_norm_rope_ex",
                     "vit_varlen_attn_ex", "vit_varlen_attn_planned_qnorm_rope",
                     "vit_varlen_attn_planned_qk_norm_rope"):
        assert required in names
    assert sorted(_lib.SIGNATURES) == names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_block_m_and_capacity(lib):
    assert lib.vit_attn_block_m(16, 80, _lib.VIT_BF16) == 256
    assert lib.vit_attn_block_m(16, 128, _lib.VIT_BF16) == 128
    assert lib.vit_attn_block_m(2, 32, _lib.VIT_F32) == 32
    assert lib.vit_attn_block_m(16, 72, _lib.VIT_BF16) == -_lib.VIT_ERR_UNSUPPORTED
    assert lib.vit_attn_block_m(0, 64, _lib.VIT_BF16) == -_lib.VIT_ERR_INVALID_ARG
    assert lib.vit_worklist_capacity(24, 3100, 128) == 24 * 25
    assert lib.vit_worklist_capacity(2048, 64, 128) == 2048
    assert lib.vit_worklist_capacity(3, 0, 64) == 0
    assert lib.vit_worklist_capacity(-1, 5, 64) == -1


def _err(lib):
    return lib.vit_last_error().decode()


FAKE = 0x10000  # aligned non-null address; never dereferenced because validation fails first


@pytest.mark.parametrize("args,code,needle", [
    ((None, FAKE, FAKE, FAKE, 1, 8, 2, 64, 0.125, FAKE + 0x100, None), 1, "null"),
    ((FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 72, 0.125, FAKE + 0x100, None), 2, "head_dim"),
    ((FAKE, FAKE, FAKE, FAKE, 1, 8, 0, 64, 0.125, FAKE + 0x100, None), 1, "num_heads"),
    ((FAKE, FAKE, FAKE, FAKE, -1, 8, 2, 64, 0.125, FAKE + 0x100, None), 1, "num_seqs"),
    ((FAKE, FAKE, FAKE, FAKE, 9000, 8, 2, 64, 0.125, FAKE + 0x100, None), 2, "num_seqs"),
    ((FAKE, FAKE, FAKE, FAKE, 1, -3, 2, 64, 0.125, FAKE + 0x100, None), 1, "max_seqlen"),
    ((FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 64, float("nan"), FAKE + 0x100, None), 1, "scale"),
    ((FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 64, float("inf"), FAKE + 0x100, None), 1, "scale"),
    ((FAKE + 2, FAKE, FAKE, FAKE, 1, 8, 2, 64, 0.125, FAKE + 0x100, None), 1, "aligned"),
    ((FAKE, FAKE, FAKE, FAKE + 1, 1, 8, 2, 64, 0.125, FAKE + 0x100, None), 1, "aligned"),
    ((FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 64, 0.125, FAKE, None), 1, "alias"),
])
def test_attention_argument_errors(lib, args, code, needle):
    for fn in (lib.vit_varlen_attn, lib.vit_varlen_attn_f32):
        assert fn(*args) == code
        assert needle in _err(lib)


def test_prepass_argument_errors(lib):
    f = lib.vit_qk_norm_rope
    assert f(FAKE, None, 4, 2, 64, 1, FAKE, 10000.0, None, None, 1e-6, None) == 1
    assert "null k" in _err(lib)
    # q may be null (k only), but then q_weight must be null too
    assert f(None, FAKE, 4, 2, 64, 1, FAKE, 10000.0, FAKE, FAKE, 1e-6, None) == 1
    assert "q_weight given without q" in _err(lib)
    assert f(None, FAKE, 0, 2, 64, 1, FAKE, 10000.0, None, FAKE, 1e-6, None) == 0
    assert f(FAKE, FAKE + 0x100, 4, 2, 60, 1, FAKE, 10000.0, None, None, 1e-6, None) == 2
    assert f(FAKE, FAKE + 0x100, 4, 2, 64, 7, FAKE, 10000.0, None, None, 1e-6, None) == 1
    assert f(FAKE, FAKE + 0x100, 4, 2, 64, 1, FAKE, 10000.0, FAKE, None, 1e-6, None) == 1
    assert "both" in _err(lib)
    assert f(FAKE, FAKE + 0x100, 4, 2, 64, 1, FAKE, -1.0, None, None, 1e-6, None) == 1
    assert "theta" in _err(lib)
    assert f(FAKE, FAKE + 0x100, 4, 2, 64, 1, None, 0.0, FAKE, FAKE, -1.0, None) == 1
    assert "eps" in _err(lib)
    assert f(FAKE, FAKE, 4, 2, 64, 1, FAKE, 10000.0, None, None, 1e-6, None) == 1
    assert f(FAKE, FAKE + 0x100, -4, 2, 64, 1, FAKE, 10000.0, None, None, 1e-6, None) == 1
    # nothing to do: no positions and no weights, or no tokens -> OK without touching memory
    assert f(FAKE, FAKE + 0x100, 4, 2, 64, 1, None, 10000.0, None, None, 1e-6, None) == 0
    assert f(FAKE, FAKE + 0x100, 0, 2, 64, 1, FAKE, 10000.0, None, None, 1e-6, None) == 0


def test_prepass_into_argument_errors(lib):
    """The out-of-place pre-pass: every rejection happens before any launch.
    T = 4 tokens of H = 2, D = 64 bf16 span 1 KiB per tensor."""
    import ctypes
    f = lib.vit_qk_norm_rope_into
    qs, ks, q, k = FAKE, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000
    none_list = (None, 0, 0, 0, None, 0, None, None)

    def call(q_src, k_src, qq, kk, T=4, src_strides=None, strides=None, pos=FAKE, lst=none_list):
        return f(q_src, k_src, src_strides, qq, kk, T, 2, 64, 1, pos, 10000.0, None, None, 1e-6, 0,
                 strides, *lst)

    assert call(None, ks, q, k) == 1 and "both" in _err(lib)
    assert call(qs, ks, None, k) == 1
    assert call(qs, None, q, k) == 1 and "k_src" in _err(lib)
    assert call(qs + 8, ks, q, k) == 1 and "aligned" in _err(lib)
    # an output overlapping a source it is not
    assert call(qs, ks, qs + 0x200, k) == 1 and "overlaps" in _err(lib)
    assert call(qs, ks, q, ks + 0x3f0) == 1 and "overlaps" in _err(lib)
    assert call(qs, ks, ks, k) == 1 and "overlaps" in _err(lib)
    # in place with a different stride for the source and the output
    wide = (ctypes.c_int64 * 2)(256, 128)
    assert call(qs, ks, qs, k, src_strides=wide) == 1 and "stride" in _err(lib)
    # work-list arguments: all or none
    assert call(qs, ks, q, k, lst=(FAKE + 0x4000, 1, 4, 64, None, 1, FAKE + 0x5000, None)) == 1
    assert call(qs, ks, q, k, lst=(None, 1, 4, 64, FAKE + 0x4000, 1, None, None)) == 1
    # nothing to do: no tokens, or in place with neither norm nor rotary
    assert call(qs, ks, q, k, T=0) == 0
    assert call(qs, ks, qs, ks, pos=None) == 0


def test_worklist_argument_errors(lib):
    f = lib.vit_varlen_worklist
    meta = FAKE + 0x40
    assert f(None, 3, 10, 64, FAKE, 3, meta, None) == 1
    assert f(FAKE, 3, 10, 0, FAKE, 3, meta, None) == 1
    assert f(FAKE, 3, 200, 64, FAKE, 3, meta, None) == 1      # needs 3 * 4 = 12 items
    assert "capacity" in _err(lib)
    assert f(FAKE, 9000, 10, 64, FAKE, 9000, meta, None) == 2
    assert f(FAKE, 3, 10, 64, FAKE + 4, 3, meta, None) == 1     # items hold 16-byte records
    assert "16-byte" in _err(lib)


def test_planned_argument_errors(lib):
    f = lib.vit_varlen_attn_planned
    assert f(FAKE, FAKE, FAKE, FAKE, None, 4, FAKE, 2, 64, 0.1, 1, 0, FAKE + 0x100, None, None, None) == 1
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 2, 64, 0.1, 5, 0, FAKE + 0x100, None, None, None) == 1
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, -4, FAKE, 2, 64, 0.1, 1, 0, FAKE + 0x100, None, None, None) == 1
    # lse must be aligned and must not alias the tensors
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 2, 64, 0.1, 1, 0, FAKE + 0x100, FAKE + 2, None, None) == 1
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 2, 64, 0.1, 1, 0, FAKE + 0x100, FAKE + 0x100, None, None) == 1
    assert "alias" in _err(lib)
    # an empty plan is a no-op
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 2, 64, 0.1, 1, 0, FAKE + 0x100, None, None, None) == 0


def test_empty_batch_is_a_no_op(lib):
    assert lib.vit_varlen_attn(FAKE, FAKE, FAKE, FAKE, 0, 0, 2, 64, 0.1, FAKE + 0x100, None) == 0
    assert lib.vit_varlen_attn(FAKE, FAKE, FAKE, FAKE, 5, 0, 2, 64, 0.1, FAKE + 0x100, None) == 0
    assert _err(lib) == ""


def test_error_message_is_thread_local(lib):
    import threading
    assert lib.vit_varlen_attn(None, FAKE, FAKE, FAKE, 1, 8, 2, 64, 0.1, FAKE + 0x100, None) == 1
    seen = []
    t = threading.Thread(target=lambda: seen.append(_err(lib)))
    t.start()
    t.join()
    assert seen == [""] and "null" in _err(lib)


def test_timing_hook_needs_both_events_or_neither(lib):
    assert lib.vit_time_next_kernel(FAKE, None) == _lib.VIT_ERR_INVALID_ARG
    assert "both" in _err(lib)
    assert lib.vit_time_next_kernel(None, FAKE) == _lib.VIT_ERR_INVALID_ARG
    assert lib.vit_time_next_kernel(None, None) == _lib.VIT_OK


def test_probe_library_is_separate_and_checks_arguments(lib):
    """The MFMA-rate probe (measurement support) is in libvit_probe.so, which
    exports what include/vit_probe.h declares; libvit.so does not export it."""
    import re
    assert not hasattr(lib, "vit_probe_mfma")
    probe = _lib.load_probe()
    header = open(os.path.join(ROOT, "include", "vit_probe.h")).read()
    declared = set(re.findall(r"^(?:int|const char\*)\s+(vit_\w+)\(", header, re.M))
    assert declared == {"vit_probe_mfma", "vit_probe_last_error"}
    for name in declared:
        assert hasattr(probe, name), name
    f = probe.vit_probe_mfma
    big = 4 << 20
    assert f(None, big, 8, 10, FAKE, None) == _lib.VIT_ERR_INVALID_ARG
    assert f(FAKE, big - 16, 8, 10, FAKE, None) == _lib.VIT_ERR_INVALID_ARG
    assert "bytes" in probe.vit_probe_last_error().decode()
    assert f(FAKE, big, 0, 10, FAKE, None) == _lib.VIT_ERR_INVALID_ARG
    assert f(FAKE, big, 8, 0, FAKE, None) == _lib.VIT_ERR_INVALID_ARG
    assert f(FAKE + 8, big, 8, 10, FAKE, None) == _lib.VIT_ERR_INVALID_ARG


def test_fused_prepass_worklist_checks_both_argument_sets(lib):
    f = lib.vit_qk_norm_rope_worklist
    meta = FAKE + 0x40
    ok_pre = (FAKE, FAKE + 0x1000, 16, 2, 64, 1, None, 1e4, None, None, 1e-6, 0, None)
    ok_wl = (FAKE, 3, 10, 64, FAKE, 3, meta, None)
    assert f(ok_pre[0], None, *ok_pre[2:], *ok_wl) == _lib.VIT_ERR_INVALID_ARG  # pre-pass check
    assert "null k" in _err(lib)
    bad_dim = ok_pre[:4] + (60,) + ok_pre[5:]
    assert f(*bad_dim, *ok_wl) == _lib.VIT_ERR_UNSUPPORTED
    assert f(*ok_pre, FAKE, 3, 200, 64, FAKE, 3, meta, None) == _lib.VIT_ERR_INVALID_ARG  # capacity
    assert "capacity" in _err(lib)
    assert f(*ok_pre, FAKE, 9000, 10, 64, FAKE, 9000, meta, None) == _lib.VIT_ERR_UNSUPPORTED


def _i64(*v):
    return (ctypes.c_int64 * len(v))(*v)


def test_token_stride_errors(lib):
    """Strides below H * D, not a whole number of 16-byte units, or >= 2^26 are rejected."""
    f = lib.vit_varlen_attn_strided
    base = (FAKE, FAKE + 0x100, FAKE + 0x200, FAKE, 1, 8, 2, 64, 0.125)
    out = FAKE + 0x1000
    for dtype, bad in ((1, (100, 128, 128, 128)),       # below H * D = 128
                       (1, (132, 128, 128, 128)),       # bf16: 132 elements is not 16-byte units
                       (0, (128, 130, 128, 128)),       # f32: 130 elements is not 16-byte units
                       (1, (128, 128, 128, 1 << 26))):  # too large
        assert f(*base, dtype, out, None, _i64(*bad), None) == _lib.VIT_ERR_INVALID_ARG
        assert "token stride" in _err(lib)
    # packed [T, 3, H, D]: stride 3 * H * D on q, k, v and a dense output -> valid (empty batch)
    assert f(FAKE, FAKE + 0x100, FAKE + 0x200, FAKE, 0, 0, 2, 64, 0.125, 1, out, None,
             _i64(384, 384, 384, 128), None) == _lib.VIT_OK
    # a segment that would not fit the 32-bit buffer range at this stride is unsupported
    assert f(*base[:5], 1 << 16, 2, 64, 0.125, 1, out, None, _i64(8208, 8208, 8208, 128),
             None) == _lib.VIT_ERR_UNSUPPORTED
    # the bound counts the last tile's key padding: (max_seqlen + 64) * stride * 2 <= 2^30
    assert f(*base[:5], (1 << 16) - 63, 2, 64, 0.125, 1, out, None,
             _i64(8192, 8192, 8192, 128), None) == _lib.VIT_ERR_UNSUPPORTED
    assert "max_seqlen + 64" in _err(lib)
    p = lib.vit_qk_norm_rope_strided
    assert p(FAKE, FAKE + 0x100, 4, 2, 64, 1, FAKE, 1e4, None, None, 1e-6, _i64(120, 128),
             None) == _lib.VIT_ERR_INVALID_ARG
    # no tokens: nothing to do, valid packed strides accepted without touching memory
    assert p(FAKE, FAKE + 0x100, 0, 2, 64, 1, FAKE, 1e4, None, None, 1e-6, _i64(384, 384),
             None) == _lib.VIT_OK
    planned = lib.vit_varlen_attn_planned
    assert planned(FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 2, 64, 0.1, 1, 0, out, None,
                   _i64(128, 64, 128, 128), None) == _lib.VIT_ERR_INVALID_ARG
    fused = lib.vit_qk_norm_rope_worklist
    assert fused(FAKE, FAKE + 0x1000, 16, 2, 64, 1, None, 1e4, None, None, 1e-6, 0, _i64(128, 8),
                 FAKE, 3, 10, 64, FAKE, 3, FAKE + 0x40, None) == _lib.VIT_ERR_INVALID_ARG


def test_dense_batch_argument_errors(lib):
    f = lib.vit_dense_batch_attn
    out = FAKE + 0x1000
    args = [FAKE, FAKE + 0x100, FAKE + 0x200, 4, 64, 2, 64, 0.125, 1, 0, out, None, None, None]
    assert f(*args[:3], -1, *args[4:]) == _lib.VIT_ERR_INVALID_ARG
    assert "batch" in _err(lib)
    assert f(*args[:4], -2, *args[5:]) == _lib.VIT_ERR_INVALID_ARG
    assert f(*args[:3], 1 << 20, 1 << 12, *args[5:]) == _lib.VIT_ERR_UNSUPPORTED   # > int32 tokens
    assert f(*args[:8], 7, *args[9:]) == _lib.VIT_ERR_INVALID_ARG                    # dtype
    assert f(None, *args[1:]) == _lib.VIT_ERR_INVALID_ARG
    assert f(*args[:6], 72, *args[7:]) == _lib.VIT_ERR_UNSUPPORTED                   # head dim
    assert f(*args[:10], FAKE, *args[11:]) == _lib.VIT_ERR_INVALID_ARG               # out aliases q
    assert f(*args[:9], 2, *args[10:]) == _lib.VIT_ERR_INVALID_ARG                   # unknown flag
    assert "flags" in _err(lib)
    assert f(*args[:3], 2, 1 << 22, *args[5:]) == _lib.VIT_ERR_UNSUPPORTED           # offset span
    # empty batches are no-ops that touch no memory
    assert f(*args[:3], 0, 64, *args[5:]) == _lib.VIT_OK
    assert f(*args[:3], 5, 0, *args[5:]) == _lib.VIT_OK


def test_rope_mode_is_checked(lib):
    f = lib.vit_qk_norm_rope_ex
    for mode in (-1, 2, 7):
        assert f(FAKE, FAKE + 0x100, 4, 2, 64, 1, FAKE, 1e4, None, None, 1e-6, mode, None,
                 None) == _lib.VIT_ERR_INVALID_ARG
        assert "rope_mode" in _err(lib)
    # valid modes with no tokens: a no-op
    for mode in (_lib.VIT_ROPE_NEOX, _lib.VIT_ROPE_COMPLEX):
        assert f(FAKE, FAKE + 0x100, 0, 2, 64, 1, FAKE, 1e4, None, None, 1e-6, mode, None,
                 None) == _lib.VIT_OK
    fused = lib.vit_qk_norm_rope_worklist
    assert fused(FAKE, FAKE + 0x1000, 16, 2, 64, 1, None, 1e4, None, None, 1e-6, 3, None,
                 FAKE, 3, 10, 64, FAKE, 3, FAKE + 0x40, None) == _lib.VIT_ERR_INVALID_ARG


def test_attention_flags_are_checked(lib):
    f = lib.vit_varlen_attn_ex
    base = (FAKE, FAKE + 0x100, FAKE + 0x200, FAKE, 1, 8, 2, 64, 0.125, 1)
    for flags in (2, 4, -1):
        assert f(*base, flags, FAKE + 0x1000, None, None, None) == _lib.VIT_ERR_INVALID_ARG
        assert "flags" in _err(lib)
    # causal with an empty batch: a no-op
    assert f(FAKE, FAKE + 0x100, FAKE + 0x200, FAKE, 0, 0, 2, 64, 0.125, 1, _lib.VIT_ATTN_CAUSAL,
             FAKE + 0x1000, None, None, None) == _lib.VIT_OK
    planned = lib.vit_varlen_attn_planned
    assert planned(FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 2, 64, 0.1, 1, 8, FAKE + 0x100, None,
                   None, None) == _lib.VIT_ERR_INVALID_ARG


def test_qnorm_rope_attention_argument_errors(lib):
    f = lib.vit_varlen_attn_planned_qnorm_rope
    head = (FAKE, FAKE + 0x100, FAKE + 0x200, FAKE, FAKE, 4, FAKE + 0x40, 2, 64, 0.1, 1, 0)
    out = FAKE + 0x1000
    ok_q = (FAKE, 1e4, FAKE, 1e-6, 0)     # pos, theta, q_weight, eps, rope_mode
    bad = [((FAKE, 1e4, FAKE, 1e-6, 2), "rope_mode"),
           ((FAKE + 4, 1e4, FAKE, 1e-6, 0), "pos must be 8-byte aligned"),
           ((FAKE, 1e4, FAKE + 4, 1e-6, 0), "q_weight must be 16-byte aligned"),
           ((FAKE, -1.0, FAKE, 1e-6, 0), "theta"),
           ((FAKE, 1e4, FAKE, -1.0, 0), "eps")]
    for qa, needle in bad:
        assert f(*head, *qa, out, None, None, None) == _lib.VIT_ERR_INVALID_ARG
        assert needle in _err(lib), needle
    # the attention's own checks still apply
    assert f(*head[:10], 7, *head[11:], *ok_q, out, None, None, None) == _lib.VIT_ERR_INVALID_ARG
    # an empty plan is a no-op
    assert f(*head[:5], 0, *head[6:], *ok_q, out, None, None, None) == _lib.VIT_OK


def test_qk_norm_rope_attention_argument_errors(lib):
    """vit_varlen_attn_planned_qk_norm_rope: the q-side checks, plus the pairing
    and alignment of k_weight, all before any launch."""
    f = lib.vit_varlen_attn_planned_qk_norm_rope
    head = (FAKE, FAKE + 0x100, FAKE + 0x200, FAKE, FAKE, 4, FAKE + 0x40, 2, 64, 0.1, 1, 0)
    out = FAKE + 0x1000
    ok = (FAKE, 1e4, FAKE, FAKE + 0x80, 1e-6, 0)  # pos, theta, q_weight, k_weight, eps, rope_mode
    bad = [((FAKE, 1e4, FAKE, FAKE + 0x80, 1e-6, 2), "rope_mode"),
           ((FAKE + 4, 1e4, FAKE, FAKE + 0x80, 1e-6, 0), "pos must be 8-byte aligned"),
           ((FAKE, 1e4, FAKE + 4, FAKE + 0x80, 1e-6, 0), "q_weight must be 16-byte aligned"),
           ((FAKE, 1e4, FAKE, FAKE + 0x84, 1e-6, 0), "k_weight must be 16-byte aligned"),
           ((FAKE, 1e4, FAKE, None, 1e-6, 0), "both"),
           ((FAKE, 1e4, None, FAKE + 0x80, 1e-6, 0), "both"),
           ((FAKE, -1.0, FAKE, FAKE + 0x80, 1e-6, 0), "theta"),
           ((FAKE, 1e4, FAKE, FAKE + 0x80, -1.0, 0), "eps")]
    for a, needle in bad:
        assert f(*head, *a, out, None, None, None) == _lib.VIT_ERR_INVALID_ARG
        assert needle in _err(lib), needle
    assert f(*head[:10], 7, *head[11:], *ok, out, None, None, None) == _lib.VIT_ERR_INVALID_ARG
    assert f(*head[:11], 2, *ok, out, None, None, None) == _lib.VIT_ERR_INVALID_ARG
    assert "flags" in _err(lib)
    # an empty plan is a no-op, with or without the norm
    assert f(*head[:5], 0, *head[6:], *ok, out, None, None, None) == _lib.VIT_OK
    assert f(*head[:5], 0, *head[6:], None, 1e4, None, None, 1e-6, 1, out, None, None,
             None) == _lib.VIT_OK


def test_noalloc_limits_and_errors_before_any_launch(lib):
    """vit_varlen_attn_noalloc: the no-allocation scratch holds 2^18 work items;
    a larger list is refused before anything is enqueued, and the argument
    checks of vit_varlen_attn_ex apply unchanged."""
    f = lib.vit_varlen_attn_noalloc
    out = FAKE + 0x1000
    base = (FAKE, FAKE + 0x100, FAKE + 0x200, FAKE)
    # 8192 segments of up to 8192 tokens at 128 query rows per item: 2^19 items
    assert f(*base, 8192, 8192, 2, 64, 0.125, _lib.VIT_BF16, 0, out, None, None, None) == \
        _lib.VIT_ERR_UNSUPPORTED
    assert "no-allocation" in _err(lib)
    # fp32 items cover 32 rows: 2048 segments of 4097 tokens need 2048 * 129 > 2^18 items
    assert f(*base, 2048, 4097, 2, 64, 0.125, _lib.VIT_F32, 0, out, None, None, None) == \
        _lib.VIT_ERR_UNSUPPORTED
    assert f(None, *base[1:], 4, 64, 2, 64, 0.125, 1, 0, out, None, None, None) == \
        _lib.VIT_ERR_INVALID_ARG
    assert f(*base, 4, 64, 2, 64, 0.125, 7, 0, out, None, None, None) == _lib.VIT_ERR_INVALID_ARG
    assert f(*base, 4, 64, 2, 64, 0.125, 1, 2, out, None, None, None) == _lib.VIT_ERR_INVALID_ARG
    assert "flags" in _err(lib)
    # an empty batch is a no-op that touches no device state
    assert f(*base, 0, 0, 2, 64, 0.125, 1, 0, out, None, None, None) == _lib.VIT_OK
