"""C ABI checks that need no GPU: the library loads, exports every function
declared in include/t2va.h, and rejects bad arguments on the host before
launching anything."""
import ctypes
import math
import os
import re

import pytest

from joint_video_audio_trigflow_amd import _lib, inputs

HEADER = _lib.HEADER_PATH


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(t2va_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libt2va.so is not built (run __graft_entry__.build())")
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"t2va_scm_target", "t2va_joint_attn_fwd_jvp", "t2va_joint_attn_fwd_jvp_split",
            "t2va_trigflow_field", "t2va_scm_workspace_bytes", "t2va_last_error", "t2va_dmd_target",
            "t2va_dmd_workspace_bytes", "t2va_stage3_mix"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.t2va_abi_version() == 3


def test_struct_sizes_match_header(lib):
    # the binding's structs mirror the header: field counts and natural packing
    assert ctypes.sizeof(_lib.AttnDesc) == 5 * 4 + 4 + 9 * 8 + 3 * 4 + 4
    assert ctypes.sizeof(_lib.ScmDesc) == 10 * 4 + 5 * 8 + 2 * 4   # + int param, int precision
    assert ctypes.sizeof(_lib.BlockWeights) == 6 * 8
    assert ctypes.sizeof(_lib.DmdDesc) == 10 * 4 + 5 * 8 + 2 * 4
    assert _lib.ScmDesc.precision.offset == 10 * 4 + 5 * 8 + 4
    assert _lib.DmdDesc.precision.offset == 10 * 4 + 5 * 8 + 4


def err(lib):
    return lib.t2va_last_error().decode()


def test_workspace_bytes_validation(lib):
    cfg = inputs.CONFIGS["high-res"]
    d = _lib.scm_desc(cfg, _lib.DTYPE_BF16, _lib.DTYPE_BF16)
    n = lib.t2va_scm_workspace_bytes(ctypes.byref(d))
    assert n > 0 and n % 256 == 0
    # the big buffers: X, fused QK, V^T and O for primal and tangent
    assert n > 2 * cfg.N_all * cfg.d * 2 * 4
    assert n < 8 * 2**30
    bad = _lib.scm_desc(cfg.replace(H=5), _lib.DTYPE_BF16, _lib.DTYPE_BF16)
    assert lib.t2va_scm_workspace_bytes(ctypes.byref(bad)) == 0
    assert "multiple" in err(lib)
    bad = _lib.scm_desc(cfg.replace(H=32), _lib.DTYPE_BF16, _lib.DTYPE_BF16)  # dh = 64 ok
    assert lib.t2va_scm_workspace_bytes(ctypes.byref(bad)) > 0
    bad = _lib.scm_desc(cfg.replace(H=64), _lib.DTYPE_BF16, _lib.DTYPE_BF16)  # dh = 32
    assert lib.t2va_scm_workspace_bytes(ctypes.byref(bad)) == 0
    bad = _lib.scm_desc(cfg.replace(B=65), _lib.DTYPE_BF16, _lib.DTYPE_BF16)
    assert lib.t2va_scm_workspace_bytes(ctypes.byref(bad)) == 0
    bad = _lib.scm_desc(cfg.replace(Cv=100), _lib.DTYPE_BF16, _lib.DTYPE_BF16)
    assert lib.t2va_scm_workspace_bytes(ctypes.byref(bad)) == 0
    # one sample's rows must fit 32-bit offsets: (tokens + 128) * 3d * 2 < 2^31
    limit = 2**31 // (3 * cfg.d * 2) - 128 - cfg.Na - cfg.Nt   # largest Nv that fits, exclusive
    ok = _lib.scm_desc(cfg.replace(Nv=limit - 1), _lib.DTYPE_BF16, _lib.DTYPE_BF16)
    assert lib.t2va_scm_workspace_bytes(ctypes.byref(ok)) > 0
    bad = _lib.scm_desc(cfg.replace(Nv=limit + 1), _lib.DTYPE_BF16, _lib.DTYPE_BF16)
    assert lib.t2va_scm_workspace_bytes(ctypes.byref(bad)) == 0
    assert "2 GiB" in err(lib)
    bad = _lib.scm_desc(cfg.replace(gamma=1.5), _lib.DTYPE_BF16, _lib.DTYPE_BF16)
    assert lib.t2va_scm_workspace_bytes(ctypes.byref(bad)) == 0
    assert "gamma" in err(lib)


def fake_ptr(i=1):
    return ctypes.c_void_p(0x10000 * i)


def test_scm_target_rejects_before_launch(lib):
    cfg = inputs.CONFIGS["tiny"]
    d = _lib.scm_desc(cfg, _lib.DTYPE_FP32, _lib.DTYPE_FP32)
    w = _lib.BlockWeights(*[0x10000 * (i + 1) for i in range(6)])
    t = (ctypes.c_double * 1)(0.5)
    ptrs = [fake_ptr(i + 10) for i in range(6)]
    outs = [fake_ptr(i + 20) for i in range(8)]
    ws_bytes = lib.t2va_scm_workspace_bytes(ctypes.byref(d))

    def call(t_arr=t, ws=fake_ptr(100), nbytes=ws_bytes, weights=w, o=outs):
        return lib.t2va_scm_target(ctypes.byref(d), ctypes.byref(weights), ctypes.byref(w), *ptrs,
                                   t_arr, *o, ws, nbytes, None)

    assert call(t_arr=(ctypes.c_double * 1)(0.0)) == 1 and "t[0]" in err(lib)
    assert call(t_arr=(ctypes.c_double * 1)(math.pi / 2)) == 1
    assert call(t_arr=(ctypes.c_double * 1)(float("nan"))) == 1
    assert call(nbytes=ws_bytes - 1) == 3 and "workspace" in err(lib)
    assert call(ws=ctypes.c_void_p(0x10010)) == 1 and "aligned" in err(lib)
    o2 = list(outs)
    o2[7] = None  # loss is required
    assert call(o=o2) == 1
    w2 = _lib.BlockWeights(*([0] + [0x10000 * (i + 1) for i in range(5)]))
    assert call(weights=w2) == 1 and "teacher" in err(lib)
    w3 = _lib.BlockWeights(*[0x10008 * (i + 1) for i in range(6)])
    assert call(weights=w3) == 1 and "aligned" in err(lib)


def test_attention_rejects_before_launch(lib):
    d = _lib.AttnDesc()
    d.B, d.H, d.dh, d.Nq, d.Nk = 1, 2, 128, 10, 20
    d.q_batch_stride = d.k_batch_stride = 20 * 256
    d.q_row_stride = d.k_row_stride = d.o_row_stride = 256
    d.o_batch_stride = 10 * 256
    d.vt_row_stride, d.vt_head_stride, d.vt_batch_stride = 64, 64 * 128, 2 * 64 * 128
    d.has_tangent, d.out_dtype = 0, 1
    p = [fake_ptr(i + 1) for i in range(10)]

    def call(desc=d, tangents=(None, None, None), od=None):
        return lib.t2va_joint_attn_fwd_jvp(ctypes.byref(desc), p[0], p[1], p[2], *tangents, p[6], p[7],
                                           od, None, None)

    d.dh = 96
    assert call() == 2
    d.dh = 128
    assert call(tangents=(p[3], p[4], p[5])) == 1          # tangents with has_tangent = 0
    d.has_tangent = 1
    assert call() == 1                                      # has_tangent without tangents
    d.has_tangent = 0
    d.vt_row_stride = 24                                    # < round_up(Nk, 64)
    assert call() == 1 and "vt_row_stride" in err(lib)
    d.vt_row_stride = 64
    d.q_row_stride = 250                                    # not a multiple of 8
    assert call() == 1


def test_trigflow_rejects_before_launch(lib):
    t = (ctypes.c_double * 2)(0.3, 2.0)
    assert lib.t2va_trigflow_field(0, 2, 16, 0, 0, 1, t, fake_ptr(1), fake_ptr(2), fake_ptr(3), None) == 1
    t = (ctypes.c_double * 2)(0.3, 0.4)
    assert lib.t2va_trigflow_field(5, 2, 16, 0, 0, 1, t, fake_ptr(1), fake_ptr(2), fake_ptr(3), None) == 1
    assert lib.t2va_trigflow_field(0, 0, 16, 0, 0, 1, t, fake_ptr(1), fake_ptr(2), fake_ptr(3), None) == 2
    assert lib.t2va_trigflow_field(0, 2, 16, 0, 0, 1, t, ctypes.c_void_p(0x10004), fake_ptr(2),
                                   fake_ptr(3), None) == 1
    # zero elements: nothing to launch, success
    assert lib.t2va_trigflow_field(0, 2, 0, 0, 0, 1, t, None, None, None, None) == 0


def test_dmd_workspace_and_rejections(lib):
    cfg = inputs.CONFIGS["high-res"]
    d = _lib.dmd_desc(cfg, _lib.DTYPE_BF16, _lib.DTYPE_BF16)
    n = lib.t2va_dmd_workspace_bytes(ctypes.byref(d))
    # forward-only: X, QK and V^T for one batch, O for the two teacher passes
    assert n > cfg.N_all * cfg.d * 2 * 4 and n < 4 * 2**30 and n % 256 == 0
    for bad in (dict(eps_dmd=0.0), dict(cfg_v=float("inf")), dict(H=5), dict(Ca=96)):
        dd = _lib.dmd_desc(cfg.replace(**bad), _lib.DTYPE_BF16, _lib.DTYPE_BF16)
        assert lib.t2va_dmd_workspace_bytes(ctypes.byref(dd)) == 0, bad

    tiny = inputs.CONFIGS["tiny"]
    d = _lib.dmd_desc(tiny, _lib.DTYPE_FP32, _lib.DTYPE_FP32)
    w = _lib.BlockWeights(*[0x10000 * (i + 1) for i in range(6)])
    t = (ctypes.c_double * 1)(0.5)
    ptrs = [fake_ptr(i + 10) for i in range(6)]
    outs = [fake_ptr(i + 20) for i in range(4)]
    ws_bytes = lib.t2va_dmd_workspace_bytes(ctypes.byref(d))

    def call(t_arr=t, ws=fake_ptr(100), nbytes=ws_bytes, fake=w, o=outs):
        return lib.t2va_dmd_target(ctypes.byref(d), ctypes.byref(w), ctypes.byref(fake), *ptrs,
                                   t_arr, *o, ws, nbytes, None)

    assert call(t_arr=(ctypes.c_double * 1)(-0.1)) == 1 and "t[0]" in err(lib)
    assert call(nbytes=ws_bytes - 1) == 3
    assert call(ws=ctypes.c_void_p(0x10040)) == 1 and "aligned" in err(lib)
    o2 = list(outs)
    o2[3] = None  # loss is required
    assert call(o=o2) == 1
    o3 = list(outs)
    o3[2] = None  # scales are optional: passes validation (not launched: fake pointers)
    w2 = _lib.BlockWeights(*([0x10000] * 5 + [0]))
    assert call(fake=w2) == 1 and "fake" in err(lib)


def test_stage3_mix_rejections(lib):
    assert lib.t2va_stage3_mix(0, 1.0, 1.0, fake_ptr(1), fake_ptr(2), fake_ptr(3), None) == 2
    assert lib.t2va_stage3_mix(2, float("nan"), 1.0, fake_ptr(1), fake_ptr(2), fake_ptr(3), None) == 1
    assert lib.t2va_stage3_mix(2, 1.0, 1.0, None, fake_ptr(2), fake_ptr(3), None) == 1


def test_param_validation(lib):
    cfg = inputs.CONFIGS["standard"]
    d = _lib.scm_desc(cfg, _lib.DTYPE_BF16, _lib.DTYPE_BF16)
    d.param = 2
    assert lib.t2va_scm_workspace_bytes(ctypes.byref(d)) == 0 and "param" in err(lib)
    d.param = _lib.PARAM_RF
    assert lib.t2va_scm_workspace_bytes(ctypes.byref(d)) > 0
    dd = _lib.dmd_desc(cfg, _lib.DTYPE_BF16, _lib.DTYPE_BF16)
    dd.param = -1
    assert lib.t2va_dmd_workspace_bytes(ctypes.byref(dd)) == 0 and "param" in err(lib)


def test_precision_validation(lib):
    cfg = inputs.CONFIGS["stress"]
    assert cfg.precision == "split"
    d = _lib.scm_desc(cfg, _lib.DTYPE_BF16, _lib.DTYPE_BF16)
    assert d.precision == _lib.PREC_SPLIT
    n_split = lib.t2va_scm_workspace_bytes(ctypes.byref(d))
    d.precision = _lib.PREC_BF16
    n_bf16 = lib.t2va_scm_workspace_bytes(ctypes.byref(d))
    # split rows double the latent, token-row and Q|K buffers and add the fp32 latents and weight pairs
    assert n_split > n_bf16 > 0
    d.precision = 2
    assert lib.t2va_scm_workspace_bytes(ctypes.byref(d)) == 0 and "precision" in err(lib)
    # the training backward runs in bf16 precision only
    d.precision = _lib.PREC_SPLIT
    assert lib.t2va_scm_grad_workspace_bytes(ctypes.byref(d)) == 0 and "precision" in err(lib)
    d.precision = _lib.PREC_BF16
    assert lib.t2va_scm_grad_workspace_bytes(ctypes.byref(d)) > 0
    dd = _lib.dmd_desc(cfg, _lib.DTYPE_BF16, _lib.DTYPE_BF16)
    assert dd.precision == _lib.PREC_SPLIT and lib.t2va_dmd_workspace_bytes(ctypes.byref(dd)) > 0
    dd.precision = -1
    assert lib.t2va_dmd_workspace_bytes(ctypes.byref(dd)) == 0 and "precision" in err(lib)


def test_split_attention_rejects_before_launch(lib):
    d = _lib.AttnDesc()
    d.B, d.H, d.dh, d.Nq, d.Nk = 1, 2, 128, 10, 20
    d.q_batch_stride = d.k_batch_stride = 20 * 256
    d.q_row_stride = d.k_row_stride = d.o_row_stride = 256
    d.o_batch_stride = 10 * 256
    d.vt_row_stride, d.vt_head_stride, d.vt_batch_stride = 64, 64 * 128, 2 * 64 * 128
    d.has_tangent, d.out_dtype = 0, 1
    p = [fake_ptr(i + 1) for i in range(12)]

    def call(q_lo=p[1], k_lo=p[3]):
        return lib.t2va_joint_attn_fwd_jvp_split(ctypes.byref(d), p[0], q_lo, p[2], k_lo, p[4], None, None, None,
                                                 p[8], p[9], None, None, None)

    assert call(q_lo=None) == 1 and "q_lo" in err(lib)
    assert call(k_lo=None) == 1
    assert call(k_lo=ctypes.c_void_p(0x30008)) == 1 and "aligned" in err(lib)
    d.dh = 96
    assert call() == 2


def test_attention_offset_bound_covers_a_stage_past_the_keys(lib):
    """The kernels address K rows up to one 128-key stage past the last key
    with 32-bit offsets: the host bound uses (Nk + 128) rows."""
    d = _lib.AttnDesc()
    d.B, d.H, d.dh = 1, 1, 128
    d.Nq = 16
    d.q_row_stride = d.o_row_stride = 128
    d.q_batch_stride = d.o_batch_stride = 16 * 128
    d.k_row_stride = 3 * 2048   # the fused QKV row stride of a 2048-wide block
    d.k_batch_stride = 0
    d.has_tangent, d.out_dtype = 0, 1
    p = [fake_ptr(i + 1) for i in range(10)]
    limit = 2**31 // (d.k_row_stride * 2)   # rows whose byte offsets stay below 2^31
    d.Nk = limit - 127                      # Nk + 128 rows pass it (Nk + 64 would not): rejected
    ldv = (d.Nk + 63) // 64 * 64
    d.vt_row_stride, d.vt_head_stride, d.vt_batch_stride = ldv, 128 * ldv, 128 * ldv
    assert lib.t2va_joint_attn_fwd_jvp(ctypes.byref(d), p[0], p[1], p[2], None, None, None, p[6], p[7],
                                       None, None, None) == 2 and "2 GiB" in err(lib)


def test_noalloc_rejects_shapes_beyond_its_scratch(lib):
    """The allocation-free entry point refuses, before touching the GPU, any
    shape whose workspace (without split attention tails) exceeds its static
    scratch."""
    assert hasattr(lib, "t2va_scm_target_noalloc")
    cfg = inputs.CONFIGS["standard"]
    d = _lib.scm_desc(cfg, _lib.DTYPE_BF16, _lib.DTYPE_BF16)
    w = _lib.BlockWeights(*[0x10000 * (i + 1) for i in range(6)])
    t = (ctypes.c_double * 1)(0.5)
    ptrs = [fake_ptr(i + 10) for i in range(6)]
    outs = [fake_ptr(i + 20) for i in range(8)]
    st = lib.t2va_scm_target_noalloc(ctypes.byref(d), ctypes.byref(w), ctypes.byref(w), *ptrs, t, *outs, None)
    assert st == 3 and "static scratch" in err(lib)
    d.gamma = 2.0   # descriptor errors come first
    st = lib.t2va_scm_target_noalloc(ctypes.byref(d), ctypes.byref(w), ctypes.byref(w), *ptrs, t, *outs, None)
    assert st == 1 and "gamma" in err(lib)


def test_v_transpose_rejects_before_launch(lib):
    """The dh-major V layout of the attention entry points: t2va_v_transpose
    converts a sequence-major V and rejects what it cannot convert."""
    v, vt = fake_ptr(1), fake_ptr(2)
    call = lambda B=1, N=100, H=2, dh=128, vrs=256, vtrs=128, vp=v: lib.t2va_v_transpose(
        B, N, H, dh, vp, N * vrs, vrs, vt, 2 * 128 * vtrs, 128 * vtrs, vtrs, None)
    assert call(dh=96) == 2
    assert call(N=0) == 2
    assert call(vtrs=64) == 1 and "round_up" in err(lib)      # 100 keys need 128 columns
    assert call(vrs=200) == 1                                  # below H * dh
    assert call(vrs=260) == 1                                  # not a multiple of 8
    assert call(vp=ctypes.c_void_p(0x10008)) == 1 and "aligned" in err(lib)
    assert call(vp=None) == 1


def test_profile_phase_mask(lib):
    """t2va_profile_set_phases selects the phases later calls record; with no
    events recorded (none here: no GPU call runs) it always succeeds, and the
    binding maps phase names to mask bits in the header's order."""
    assert lib.t2va_profile_set_phases(1 << 2) == 0          # T2VA_PHASE_STUDENT_ATTN only
    _lib.profile_set_phases(["student_attn", "bwd_attn"])
    _lib.profile_set_phases(None)                            # every phase again
    src = open(HEADER).read()
    for i, name in enumerate(_lib.PHASES):
        assert re.search(rf"#define T2VA_PHASE_{name.upper()} {i}\b", src), name
