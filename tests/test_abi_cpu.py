"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/comba.h declares, and rejects bad arguments with the
documented status codes before enqueuing anything."""
import ctypes
import os
import re
import subprocess

import pytest

import bilinear_rnn_amd as comba
from bilinear_rnn_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "comba.h")

FAKE = ctypes.c_void_p(4096)   # never dereferenced: every call below fails validation first


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(comba_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    declared = header_functions()
    assert declared == sorted(api.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", comba.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (comba_\w+)", out))
    assert set(declared) <= exported
    L = comba.lib()
    for name in declared:
        assert hasattr(L, name)


def test_version_and_status_strings():
    L = comba.lib()
    assert L.comba_abi_version() == 6
    assert api.status_string(0) == "COMBA_OK"
    assert api.status_string(-1) == "COMBA_ERR_INVALID_ARG"
    assert api.status_string(-2) == "COMBA_ERR_UNSUPPORTED"
    assert api.status_string(-3) == "COMBA_ERR_WORKSPACE"
    assert api.status_string(-4) == "COMBA_ERR_HIP"
    assert api.status_string(7) == "COMBA_ERR_UNKNOWN"


def chunk(fusion=None, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, alpha=FAKE, beta=FAKE, d=FAKE, s0=None, cu=None, n=0,
                B=1, T=16, H=2, K=64, V=64, idt=0, odt=0, o=FAKE, sf=None, ws=None, wsb=0)
    args.update(kw)
    L = comba.lib()
    a = (args["q"], args["k"], args["v"], args["alpha"], args["beta"], args["d"], args["s0"], args["cu"],
         args["n"], args["B"], args["T"], args["H"], args["K"], args["V"], args["idt"], args["odt"],
         args["o"], args["sf"], args["ws"], args["wsb"])
    if fusion is None:
        return L.comba_chunk_fwd(*a, None)
    return L.comba_chunk_fwd_fused(*a, fusion, None)


def step(fusion=None, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, alpha=FAKE, beta=FAKE, d=FAKE, s0=None, cu=None, n=0,
                B=1, T=1, H=2, K=64, V=64, idt=0, odt=0, o=FAKE, sf=None)
    args.update(kw)
    L = comba.lib()
    a = (args["q"], args["k"], args["v"], args["alpha"], args["beta"], args["d"], args["s0"], args["cu"],
         args["n"], args["B"], args["T"], args["H"], args["K"], args["V"], args["idt"], args["odt"],
         args["o"], args["sf"])
    if fusion is None:
        return L.comba_recurrent_step(*a, None)
    return L.comba_recurrent_step_fused(*a, fusion, None)


def segmented(fusion=0, nseg=4, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, alpha=FAKE, beta=FAKE, d=FAKE, s0=None, B=1, T=1000, H=2, K=64, V=64,
                idt=0, odt=0, o=FAKE, sf=None, ws=FAKE, wsb=1 << 40)
    args.update({k2: v2 for k2, v2 in kw.items() if k2 not in ("cu", "n")})
    if "cu" in kw:  # no packed batches on this entry point: map the case onto an equivalent invalid one
        args["B"] = 0
    L = comba.lib()
    return L.comba_chunk_fwd_segmented(args["q"], args["k"], args["v"], args["alpha"], args["beta"], args["d"],
                                       args["s0"], args["B"], args["T"], args["H"], args.get("Hk", args["H"]),
                                       args["K"], args["V"], args["idt"], args["odt"], args["o"], args["sf"],
                                       nseg, args["ws"],
                                       args["wsb"], fusion, None)


def chunk_noalloc(fusion=None, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, alpha=FAKE, beta=FAKE, d=FAKE, s0=None, cu=None, n=0,
                B=1, T=1, H=2, K=64, V=64, idt=0, odt=0, o=FAKE, sf=None)
    args.update(kw)
    if fusion is not None:  # no fusion argument on this entry point: map onto an invalid call
        args["q"] = None
    return comba.lib().comba_chunk_fwd_noalloc(
        args["q"], args["k"], args["v"], args["alpha"], args["beta"], args["d"], args["s0"], args["cu"], args["n"],
        args["B"], args["T"], args["H"], args["K"], args["V"], args["idt"], args["odt"], args["o"], args["sf"], None)


def chunk_fused(**kw):
    return chunk(fusion=api.COMBA_FUSE_GATE_LOGITS | api.COMBA_FUSE_QK_L2NORM, **kw)


def step_fused(**kw):
    return step(fusion=api.COMBA_FUSE_QK_L2NORM, **kw)


@pytest.mark.parametrize("fn", [chunk, step, chunk_fused, step_fused, segmented, chunk_noalloc])
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(alpha=None), -1),
    (dict(beta=None), -1), (dict(d=None), -1), (dict(o=None), -1),
    (dict(B=0), -1), (dict(H=0), -1), (dict(T=0), -1), (dict(K=0), -1), (dict(V=-3), -1),
    (dict(idt=2), -1), (dict(odt=-1), -1),
    (dict(K=96), -2), (dict(V=32), -2), (dict(K=256), -2),
    (dict(H=32769, K=128, V=128), -2), (dict(H=65537), -2), (dict(H=32769, K=64, V=128), -2),
    (dict(cu=FAKE, n=3, B=2), -1), (dict(cu=FAKE, n=0), -1), (dict(cu=FAKE, n=2, T=-1), -1),
    (dict(s0=ctypes.c_void_p(4096), sf=ctypes.c_void_p(4096 + 64)), -1),
])
def test_invalid_arguments_are_rejected_before_launch(fn, kw, code):
    assert fn(**kw) == code
    assert api.last_error() != ""


@pytest.mark.parametrize("fn", [chunk, step, segmented])
@pytest.mark.parametrize("fusion", [4, 8, 1 << 16, 1 << 17, 1 << 18, 0x80000000, 0xFFFFFFFF])
def test_unknown_fusion_bits_are_rejected(fn, fusion):
    assert fn(fusion=fusion) == api.COMBA_ERR_INVALID_ARG
    assert "fusion" in api.last_error()


def test_segmented_plan_and_workspace():
    ws = comba.segmented_workspace_size
    # one 64K-token sequence of 16 heads: 32 workgroups, so 8 segments of 8192 tokens
    assert ws(1, 65536, 16, 128, 128, 0) == 256 + 3 * 8 * 16 * 128 * 128 * 4
    # the 1.3B layer already fills the chip: no segmentation, no workspace
    assert ws(8, 4096, 16, 128, 128, 0) == 0
    # explicit counts are capped at one chunk per segment: T = 100 allows 2
    assert ws(1, 100, 2, 64, 64, 5) == ws(1, 100, 2, 64, 64, 2) > 0
    assert ws(1, 100, 2, 64, 64, 1) == 0
    # K != V: Phi is K x K, the states V x K
    S = 4
    assert ws(2, 4096, 3, 64, 128, S) == 256 + 2 * S * 3 * (2 * 128 * 64 + 64 * 64) * 4
    # too small a workspace, negative counts, packed batches are not accepted
    assert segmented(nseg=4, ws=FAKE, wsb=ws(1, 1000, 2, 64, 64, 4) - 1) == -3
    assert segmented(nseg=4, ws=None, wsb=0) == -3
    assert segmented(nseg=-1) == -1
    assert segmented(B=2, T=(1 << 30)) == -2


def _ex(fn_name, Hk, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, alpha=FAKE, beta=FAKE, d=FAKE, s0=None, cu=None, n=0,
                B=1, T=16, H=4, K=64, V=64, idt=0, odt=0, o=FAKE, sf=None)
    args.update(kw)
    a = (args["q"], args["k"], args["v"], args["alpha"], args["beta"], args["d"], args["s0"], args["cu"],
         args["n"], args["B"], args["T"], args["H"], Hk, args["K"], args["V"], args["idt"], args["odt"],
         args["o"], args["sf"])
    L = comba.lib()
    if fn_name == "chunk":
        return L.comba_chunk_fwd_ex(*a, None, 0, 0, None)
    return L.comba_recurrent_step_ex(*a, 0, None)


@pytest.mark.parametrize("fn_name", ["chunk", "step"])
@pytest.mark.parametrize("Hk", [0, -1, 3, 8])
def test_qk_heads_must_divide_value_heads(fn_name, Hk):
    assert _ex(fn_name, Hk) == api.COMBA_ERR_INVALID_ARG
    assert "num_qk_heads" in api.last_error()


@pytest.mark.parametrize("fn_name", ["chunk", "step"])
def test_qk_heads_other_errors_still_reported(fn_name):
    assert _ex(fn_name, 2, q=None) == api.COMBA_ERR_INVALID_ARG
    assert _ex(fn_name, 2, K=96) == api.COMBA_ERR_UNSUPPORTED


def test_segmented_qk_heads_checked():
    assert segmented(Hk=3, H=4) == api.COMBA_ERR_INVALID_ARG


def bwd(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, alpha=FAKE, beta=FAKE, d=FAKE, s0=None, cu=None, n=0,
                B=1, T=16, H=2, K=64, V=64, idt=0, do=FAKE, dsf=None, dq=FAKE, dk=FAKE, dv=FAKE, da=FAKE,
                db=FAKE, dd=FAKE, ds0=None, ws=FAKE, wsb=1 << 40)
    args.update(kw)
    return comba.lib().comba_chunk_bwd(
        args["q"], args["k"], args["v"], args["alpha"], args["beta"], args["d"], args["s0"], args["cu"], args["n"],
        args["B"], args["T"], args["H"], args["K"], args["V"], args["idt"], args["do"], args["dsf"], args["dq"],
        args["dk"], args["dv"], args["da"], args["db"], args["dd"], args["ds0"], args["ws"], args["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(do=None), -1), (dict(dq=None), -1), (dict(dk=None), -1), (dict(dv=None), -1), (dict(da=None), -1),
    (dict(db=None), -1), (dict(dd=None), -1), (dict(q=None), -1), (dict(T=0), -1), (dict(idt=3), -1),
    (dict(K=96), -2), (dict(H=32769, K=128, V=128), -2), (dict(cu=FAKE, n=0), -1), (dict(ws=None, wsb=0), -3),
    (dict(wsb=100), -3),
])
def test_backward_rejects_bad_arguments(kw, code):
    assert bwd(**kw) == code
    assert api.last_error() != ""


@pytest.mark.parametrize("sink,blocks,iters,code", [
    (None, 1, 1, -1), (FAKE, 0, 1, -1), (FAKE, 1, 0, -1), (FAKE, -3, 5, -1), (FAKE, 1 << 30, 1, -2),
])
def test_mfma_peak_probe_rejects_bad_arguments(sink, blocks, iters, code):
    assert comba.lib().comba_mfma_peak_probe(sink, blocks, iters, None) == code
    assert api.last_error() != ""


def fwd_keep(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, alpha=FAKE, beta=FAKE, d=FAKE, s0=None, cu=None, n=0,
                B=1, T=100, H=2, K=64, V=64, idt=0, odt=0, o=FAKE, sf=None, ws=None, wsb=0, cs=FAKE, csb=1 << 40)
    args.update(kw)
    a = args
    return comba.lib().comba_chunk_fwd_keep_states(
        a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["d"], a["s0"], a["cu"], a["n"], a["B"], a["T"], a["H"],
        a["K"], a["V"], a["idt"], a["odt"], a["o"], a["sf"], a["ws"], a["wsb"], a["cs"], a["csb"], None)


def bwd_cached(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, alpha=FAKE, beta=FAKE, d=FAKE, s0=None, cu=None, n=0,
                B=1, T=100, H=2, K=64, V=64, idt=0, do=FAKE, dsf=None, cs=FAKE, csb=1 << 40, dq=FAKE, dk=FAKE,
                dv=FAKE, da=FAKE, db=FAKE, dd=FAKE, ds0=None, ws=FAKE, wsb=1 << 40)
    args.update(kw)
    a = args
    return comba.lib().comba_chunk_bwd_cached(
        a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["d"], a["s0"], a["cu"], a["n"], a["B"], a["T"], a["H"],
        a["K"], a["V"], a["idt"], a["do"], a["dsf"], a["cs"], a["csb"], a["dq"], a["dk"], a["dv"], a["da"], a["db"],
        a["dd"], a["ds0"], a["ws"], a["wsb"], None)


def test_chunk_state_sizes():
    # one fp32 V x K state per 64-token chunk and head
    assert comba.chunk_states_size(1, 100, 2, 64, 64) == 2 * 2 * 64 * 64 * 4
    assert comba.chunk_states_size(8, 4096, 16, 128, 128) == 8 * 64 * 16 * 128 * 128 * 4
    # packed: T / 64 + N + 1 slots
    assert comba.chunk_states_size(1, 1000, 2, 64, 64, 5) == (1000 // 64 + 5 + 1) * 2 * 64 * 64 * 4
    # the cached backward needs the plain backward's workspace less its own copy of the states
    for args in [(8, 4096, 16, 128, 128), (1, 1000, 2, 64, 64, 5), (3, 65, 4, 64, 128)]:
        assert comba.bwd_workspace_size(*args) - comba.bwd_cached_workspace_size(*args) == comba.chunk_states_size(*args)


@pytest.mark.parametrize("kw,code", [
    (dict(cs=None), -1), (dict(csb=2 * 2 * 64 * 64 * 4 - 1), -3), (dict(q=None), -1), (dict(K=96), -2),
    (dict(H=32769, K=128, V=128), -2),
])
def test_keep_states_forward_rejects_bad_arguments(kw, code):
    assert fwd_keep(**kw) == code
    assert api.last_error() != ""


@pytest.mark.parametrize("kw,code", [
    (dict(cs=None), -1), (dict(csb=100), -3), (dict(do=None), -1), (dict(dq=None), -1), (dict(K=96), -2),
    (dict(ws=None, wsb=0), -3), (dict(wsb=comba.api.lib().comba_chunk_bwd_cached_workspace_size(1, 100, 2, 64, 64, 0) - 1), -3),
])
def test_cached_backward_rejects_bad_arguments(kw, code):
    assert bwd_cached(**kw) == code
    assert api.last_error() != ""


def test_backward_workspace_size():
    ws = comba.bwd_workspace_size
    # per chunk and head: two fp32 states, three fp32 64 x 64 matrices, seven
    # rows of 64 gate values, one float
    pairs = 8 * 64 * 16
    assert ws(8, 4096, 16, 128, 128) == pairs * (2 * 128 * 128 * 4 + 3 * 64 * 64 * 4 + 7 * 64 * 4 + 4)
    # packed: T / 64 + N + 1 slots
    pairs = (1000 // 64 + 5 + 1) * 2
    assert ws(1, 1000, 2, 64, 64, 5) == (pairs * (2 * 64 * 64 * 4 + 3 * 64 * 64 * 4 + 7 * 64 * 4)
                                         + ((pairs * 4 + 255) // 256) * 256)


def test_workspace_rules():
    assert comba.workspace_size(1, 100, 4, 64, 64, 0) == 0
    ws = comba.workspace_size(1, 100, 4, 64, 64, 10)
    assert ws >= 40 and ws % 256 == 0
    # packed batch with no workspace
    assert chunk(cu=FAKE, n=10, T=100) == -3
    assert chunk(cu=FAKE, n=10, T=100, ws=FAKE, wsb=ws - 1) == -3


def test_python_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16)
    a = torch.ones(1, 4, 2)
    with pytest.raises(ValueError):
        comba.chunk_fwd(x, x, x, a, a, torch.zeros(2))


def test_noalloc_rejects_more_packed_sequences_than_its_scratch():
    """The allocation-free forward keeps the packed-sequence order in a device
    array of 16384 entries: more sequences are refused on the host."""
    assert chunk_noalloc(cu=FAKE, n=16385, T=16385) == api.COMBA_ERR_UNSUPPORTED
    assert "16384" in api.last_error()


LDS_OFFS = (ctypes.c_int32 * 64)(*[16 * i for i in range(64)])


@pytest.mark.parametrize("kind,offs,iters,sink,blocks,code", [
    (0, None, 1, FAKE, 1, -1), (0, LDS_OFFS, 1, None, 1, -1), (8, LDS_OFFS, 1, FAKE, 1, -1),
    (-1, LDS_OFFS, 1, FAKE, 1, -1), (0, LDS_OFFS, 0, FAKE, 1, -1), (0, LDS_OFFS, 1, FAKE, 0, -1),
    (0, (ctypes.c_int32 * 64)(*([8] + [0] * 63)), 1, FAKE, 1, -1),        # 16-byte access at an 8-byte offset
    (0, (ctypes.c_int32 * 64)(*([65536 - 8] + [0] * 63)), 1, FAKE, 1, -1),  # past 64 KiB
    (7, (ctypes.c_int32 * 64)(*([-2] + [0] * 63)), 1, FAKE, 1, -1),
    (0, LDS_OFFS, 1, FAKE, 1 << 30, -2),
])
def test_lds_probe_rejects_bad_arguments(kind, offs, iters, sink, blocks, code):
    assert comba.lib().comba_lds_probe(kind, offs, iters, sink, blocks, None) == code
    assert api.last_error() != ""


def test_lds_patterns_are_aligned_and_inside_the_probe_array():
    from bilinear_rnn_amd import lds_patterns
    width = {"read16": 16, "read8": 8, "read4": 4, "read8_tr": 8, "write16": 16, "write8": 8, "write4": 4, "write2": 2}
    pats = lds_patterns.patterns()
    assert len(pats) > 100
    for name, kind, offs in pats:
        assert len(offs) == 64, name
        assert all(o % width[kind] == 0 and 0 <= o <= 65536 - width[kind] for o in offs), name


def test_lds_pattern_layouts_cover_each_tile_once():
    # the q / k swizzles and staging rows address every 16-byte piece of a tile exactly once
    from bilinear_rnn_amd import lds_patterns as lp
    for K in (128, 64):
        for sw in lp.QK_ALTERNATIVES.values():
            pieces = sorted(lp.qk_off(K, sw, r, 8 * c) // 8 for r in range(64) for c in range(K // 8))
            assert pieces == list(range(64 * K // 8))
        kp = K // 8
        for spread in (True, False):
            rows = sorted((lp.qk_row(K, p, j, spread), lp.qk_col(K, p, spread))
                          for p in range(256) for j in range(64 * kp // 256))
            assert rows == [(r, c) for r in range(64) for c in range(kp)]



@pytest.mark.parametrize("alpha,n_alpha,cu,nseq,T,flags", [
    (None, 16, None, 0, 0, FAKE),      # NULL alpha
    (FAKE, 16, None, 0, 0, None),      # NULL flags
    (FAKE, -1, None, 0, 0, FAKE),      # negative count
    (FAKE, 16, FAKE, 0, 16, FAKE),     # cu_seqlens with no sequence
    (FAKE, 16, FAKE, 2, -1, FAKE),     # cu_seqlens with T < 0
])
def test_check_inputs_rejects_bad_arguments(alpha, n_alpha, cu, nseq, T, flags):
    assert comba.lib().comba_check_inputs(alpha, n_alpha, cu, nseq, T, flags, None) == api.COMBA_ERR_INVALID_ARG
    assert api.last_error() != ""


def test_check_flags_match_the_header():
    text = open(os.path.join(ROOT, "include", "comba.h")).read()
    for name in ("COMBA_CHECK_ALPHA_RANGE", "COMBA_CHECK_CU_ORDER", "COMBA_CHECK_CU_BOUNDS"):
        m = re.search(rf"#define {name} (\d+)u", text)
        assert m and int(m.group(1)) == getattr(api, name), name
