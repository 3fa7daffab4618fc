"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function
``include/kda.h`` declares, and rejects bad arguments before any device work."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_78_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIP = 0, -1, -2, -3, -4
FAKE = 0x7F0000000000  # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.LIB_PATH):
        from gated_delta_rule_78_amd import build
        build.build()
    return kda.library()


def test_header_declares_the_boundary():
    assert declared_functions() == ["kda_chunk_bwd", "kda_chunk_bwd_workspace_bytes", "kda_chunk_fwd",
                                    "kda_chunk_fwd_noalloc", "kda_chunk_fwd_varlen", "kda_chunk_fwd_varlen_workspace_bytes",
                                    "kda_chunk_fwd_workspace_bytes", "kda_decode_step", "kda_decode_step_gated",
                                    "kda_status_string", "kda_version"]


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version(lib):
    for code in (OK, INVALID, UNSUPPORTED, WORKSPACE, HIP):
        s = lib.kda_status_string(code).decode()
        assert s.startswith("KDA_")
    assert lib.kda_status_string(12345).decode() == "unknown kda_status"
    assert lib.kda_version().decode().startswith("kda-gfx950")


def _desc(B=1, H=2, T=128, dk=128, dv=128, chunk=64, ind=1, outd=1, seg=0):
    return kda.ChunkDesc(B, H, T, dk, dv, chunk, ind, outd, seg)


def _chunk(lib, d, q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), la=FAKE + (3 << 30), beta=FAKE + (4 << 30),
           S0=None, o=FAKE + (5 << 30), ST=None, ws=None, ws_bytes=0):
    P = ctypes.c_void_p
    return lib.kda_chunk_fwd(None if d is None else ctypes.byref(d), P(q), P(k), P(v), P(la), P(beta), P(S0), P(o),
                             P(ST), P(ws), ws_bytes, None)


def test_chunk_rejects_bad_descriptors(lib):
    assert _chunk(lib, None) == INVALID
    assert _chunk(lib, _desc(B=0)) == INVALID
    assert _chunk(lib, _desc(T=-1)) == INVALID
    assert _chunk(lib, _desc(seg=-2)) == INVALID
    assert _chunk(lib, _desc(ind=7)) == INVALID
    assert _chunk(lib, _desc(chunk=32)) == UNSUPPORTED
    assert _chunk(lib, _desc(dk=96)) == UNSUPPORTED
    assert _chunk(lib, _desc(dv=256)) == UNSUPPORTED
    assert _chunk(lib, _desc(ind=0, dk=128)) == UNSUPPORTED   # the fp32 path is dk = 64 only


def test_chunk_rejects_bad_pointers(lib):
    assert _chunk(lib, _desc(), q=0) == INVALID
    assert _chunk(lib, _desc(), o=0) == INVALID
    assert _chunk(lib, _desc(), q=FAKE + 8) == INVALID               # misaligned
    assert _chunk(lib, _desc(), S0=FAKE + (6 << 30) + 4) == INVALID  # misaligned state
    assert _chunk(lib, _desc(), o=FAKE + 64) == INVALID              # o overlaps q
    S = FAKE + (6 << 30)
    assert _chunk(lib, _desc(), S0=S, ST=S + 1024) == INVALID        # partial state overlap
    assert _chunk(lib, _desc(), S0=S, ST=S + (1 << 28), o=S + 16) == INVALID  # o overlaps S0


def record_bytes(dk, dv):
    """Bytes of one chunk record as include/kda.h documents them: W, Q~ and K- blocks (dk/32 * 4
    KiB each), six A_qk blocks, U (dv/16 * 2 KiB) and one block of gamma_C."""
    return (12 * (dk // 32) + 7 + 2 * (dv // 16)) * 1024


def test_workspace_query_and_check(lib):
    lanes, dk, dv, nchunks, nseg = 2, 128, 128, 40, 4
    d = _desc(B=1, H=lanes, T=64 * nchunks, seg=nseg)
    need = lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(d))
    # records, then per (lane, segment) an affine pair [dk x (dv + dk)], an entry state [dk x dv]
    # and a 4-byte window flag
    assert need == lanes * nchunks * record_bytes(dk, dv) + lanes * nseg * (dk * (2 * dv + dk) + 1) * 4
    assert _chunk(lib, d) == WORKSPACE
    assert _chunk(lib, d, ws=FAKE + (7 << 30), ws_bytes=need - 1) == WORKSPACE
    assert _chunk(lib, d, ws=FAKE + (7 << 30) + 8, ws_bytes=need) == INVALID   # misaligned workspace
    assert _chunk(lib, d, ws=FAKE + 32, ws_bytes=need) == INVALID              # workspace overlaps q
    # one segment: records only; a ragged tail counts as a whole chunk
    one = _desc(B=2, H=3, T=64 * 5 + 1, dk=64, dv=128, seg=1)
    assert lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(one)) == 6 * 6 * record_bytes(64, 128)
    assert lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(_desc(ind=0, dk=64, dv=64))) == 0   # fp32 path
    assert lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(_desc(T=0))) == 0
    assert lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(_desc(dk=96))) == 0
    assert lib.kda_chunk_fwd_workspace_bytes(None) == 0


def _decode(lib, d, q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), la=FAKE + (3 << 30), beta=FAKE + (4 << 30),
            S=FAKE + (5 << 30), o=FAKE + (6 << 30)):
    P = ctypes.c_void_p
    return lib.kda_decode_step(None if d is None else ctypes.byref(d), P(q), P(k), P(v), P(la), P(beta), P(S),
                               P(o), None)


def test_decode_rejects_bad_arguments(lib):
    d = kda.DecodeDesc(4, 2, 128, 128, 1, 1)
    assert _decode(lib, None) == INVALID
    assert _decode(lib, kda.DecodeDesc(0, 2, 128, 128, 1, 1)) == INVALID
    assert _decode(lib, kda.DecodeDesc(4, 2, 80, 128, 1, 1)) == UNSUPPORTED
    assert _decode(lib, kda.DecodeDesc(4, 2, 128, 128, 3, 1)) == INVALID
    assert _decode(lib, d, S=0) == INVALID
    assert _decode(lib, d, S=FAKE + (5 << 30) + 4) == INVALID           # misaligned state
    assert _decode(lib, d, o=FAKE + (5 << 30) + 64) == INVALID          # o overlaps S
    assert _decode(lib, d, q=FAKE + (5 << 30) + 256) == INVALID         # input overlaps S


# ---- packed variable-length batches with checkpoints (kda_chunk_fwd_varlen) ----

def _vdesc(N=3, H=2, T=640, max_len=512, dk=128, dv=128, chunk=64, ind=1, outd=1, seg=0, ck=0, packed=1):
    return kda.VarlenDesc(N, H, T, max_len, dk, dv, chunk, ind, outd, seg, ck, packed)


def _varlen(lib, d, cu=FAKE + (6 << 30), S0=None, ST=None, ckpt=None, ckoff=None, ws=FAKE + (8 << 30),
            ws_bytes=1 << 40, q=FAKE, o=FAKE + (5 << 30), la=FAKE + (3 << 30), gating=None):
    P = ctypes.c_void_p
    return lib.kda_chunk_fwd_varlen(None if d is None else ctypes.byref(d), P(q), P(FAKE + (1 << 30)),
                                    P(FAKE + (2 << 30)), P(la), P(FAKE + (4 << 30)), P(cu), P(S0),
                                    P(o), P(ST), P(ckpt), P(ckoff), None if gating is None else ctypes.byref(gating),
                                    P(ws), ws_bytes, None)


def test_varlen_rejects_bad_arguments(lib):
    assert _varlen(lib, None) == INVALID
    assert _varlen(lib, _vdesc(), cu=None) == INVALID                      # packed needs cu_seqlens
    assert _varlen(lib, _vdesc(packed=0)) == INVALID                       # equal lengths take no cu_seqlens
    assert _varlen(lib, _vdesc(packed=2)) == INVALID
    assert _varlen(lib, _vdesc(ck=100)) == INVALID                         # not a multiple of 64
    assert _varlen(lib, _vdesc(ck=-64)) == INVALID
    assert _varlen(lib, _vdesc(ind=0)) == UNSUPPORTED                      # bf16 inputs only
    assert _varlen(lib, _vdesc(chunk=32)) == UNSUPPORTED
    assert _varlen(lib, _vdesc(dk=96)) == UNSUPPORTED
    assert _varlen(lib, _vdesc(max_len=1 << 22)) == UNSUPPORTED            # 32-bit output offsets
    assert _varlen(lib, _vdesc(N=0)) == INVALID
    assert _varlen(lib, _vdesc(ck=512)) == INVALID                         # checkpoints need S_ckpt ...
    assert _varlen(lib, _vdesc(ck=512), ckpt=FAKE + (9 << 30)) == INVALID  # ... and (packed) the offsets
    assert _varlen(lib, _vdesc(), cu=FAKE + (6 << 30) + 2) == INVALID      # misaligned cu_seqlens
    assert _varlen(lib, _vdesc(), o=FAKE + 64) == INVALID                  # o overlaps q
    assert _varlen(lib, _vdesc(ck=512), ckpt=FAKE + (9 << 30), ckoff=FAKE + (9 << 30) + 64) == INVALID  # overlap


def test_varlen_workspace_query_and_check(lib):
    N, H, T, dk, dv = 3, 2, 640, 128, 128
    d = _vdesc(N=N, H=H, T=T, max_len=512, seg=1)
    need = lib.kda_chunk_fwd_varlen_workspace_bytes(ctypes.byref(d))
    slots = T // 64 + N   # chunk slots per head: sequence s's chunk c sits in slot cu[s]/64 + s + c
    assert need == H * slots * record_bytes(dk, dv) + slots * 8
    # with a split of the longest sequence (8 chunks) into 4 segments: affine pairs, entries and
    # window flags per lane
    d4 = _vdesc(N=N, H=H, T=T, max_len=512, seg=4)
    assert lib.kda_chunk_fwd_varlen_workspace_bytes(ctypes.byref(d4)) == need + N * H * 4 * (dk * (2 * dv + dk) + 1) * 4
    assert _varlen(lib, d, ws=None, ws_bytes=0) == WORKSPACE
    assert _varlen(lib, d, ws_bytes=need - 1) == WORKSPACE
    assert _varlen(lib, d, ws=FAKE + (8 << 30) + 8, ws_bytes=need) == INVALID
    # equal lengths: the fixed-length call's workspace with B = N
    e = _vdesc(N=N, H=H, T=T, seg=1, packed=0)
    assert lib.kda_chunk_fwd_varlen_workspace_bytes(ctypes.byref(e)) == N * H * (T // 64) * record_bytes(dk, dv)
    assert lib.kda_chunk_fwd_varlen_workspace_bytes(ctypes.byref(_vdesc(ind=0))) == 0


def test_gating_rejects_bad_arguments(lib):
    G = kda.Gating
    z, A, gate, w = FAKE + (10 << 30), FAKE + (11 << 30), FAKE + (12 << 30), FAKE + (13 << 30)
    d = _vdesc()
    assert _varlen(lib, d, la=None) == INVALID                                        # no decay input at all
    assert _varlen(lib, d, la=None, gating=G(z, None, -5.0, 0.0, None, None)) == INVALID   # z without A_log
    assert _varlen(lib, d, la=None, gating=G(z, A, 0.0, 0.0, None, None)) == INVALID       # g_min must be < 0
    assert _varlen(lib, d, la=None, gating=G(z, A, float("nan"), 0.0, None, None)) == INVALID
    assert _varlen(lib, d, la=None, gating=G(z + 8, A, -5.0, 0.0, None, None)) == INVALID  # misaligned z
    assert _varlen(lib, d, gating=G(None, None, 0.0, 0.0, gate, None)) == INVALID          # eps must be > 0
    assert _varlen(lib, d, gating=G(None, None, 0.0, 1e-6, gate, w + 4)) == INVALID        # misaligned weight
    assert _varlen(lib, d, gating=G(None, None, 0.0, 1e-6, FAKE + (5 << 30), None)) == INVALID  # gate overlaps o
    # a valid gating passes validation and stops at the missing workspace
    assert _varlen(lib, d, la=None, ws=None, ws_bytes=0, gating=G(z, A, -5.0, 1e-6, gate, w)) == WORKSPACE
    dd = kda.DecodeDesc(4, 2, 128, 128, 1, 1)
    P = ctypes.c_void_p
    call = lambda la, g: lib.kda_decode_step_gated(ctypes.byref(dd), P(FAKE), P(FAKE + (1 << 30)), P(FAKE + (2 << 30)),
                                                   P(la), P(FAKE + (4 << 30)), None if g is None else ctypes.byref(g),
                                                   P(FAKE + (5 << 30)), P(FAKE + (6 << 30)), None)
    assert call(None, None) == INVALID
    assert call(None, G(z, None, -5.0, 0.0, None, None)) == INVALID
    assert call(FAKE + (3 << 30), G(None, None, 0.0, -1.0, gate, None)) == INVALID
    assert call(FAKE + (3 << 30), G(None, None, 0.0, 1e-6, FAKE + (6 << 30), None)) == INVALID   # gate overlaps o


def test_backward_rejects_bad_arguments(lib):
    d = _desc(B=1, H=2, T=256)
    P = ctypes.c_void_p
    base = [FAKE + (i << 30) for i in range(14)]   # q k v la beta S0 dO dS_T dq dk dv dla dbeta dS0

    def call(desc, ptrs, ws=FAKE + (20 << 30), ws_bytes=1 << 40):
        return lib.kda_chunk_bwd(None if desc is None else ctypes.byref(desc), *[P(p) for p in ptrs], P(ws), ws_bytes,
                                 None)
    assert call(None, base) == INVALID
    assert call(_desc(ind=0, dk=64, dv=64), base) == UNSUPPORTED        # bf16 inputs only
    assert call(d, base[:8] + [None] + base[9:]) == INVALID             # dq missing
    bad = list(base)
    bad[9] = base[8] + 64                                                # dk overlaps dq
    assert call(d, bad) == INVALID
    bad = list(base)
    bad[10] = base[2]                                                    # dv overlaps v
    assert call(d, bad) == INVALID
    assert call(d, base, ws=None, ws_bytes=0) == WORKSPACE
    need = lib.kda_chunk_bwd_workspace_bytes(ctypes.byref(d))
    assert need > lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(d))
    assert call(d, base, ws_bytes=need - 1) == WORKSPACE
    assert call(d, base, ws=FAKE + (20 << 30) + 16, ws_bytes=need) == INVALID   # 256-byte alignment
    assert lib.kda_chunk_bwd_workspace_bytes(ctypes.byref(_desc(T=0))) == 0


def test_final_state_must_not_overlap_inputs(lib):
    """S_T is written by the state pass's last segment while other workgroups may still read the
    inputs: an S_T range that overlaps any input is rejected (S_T == S0 stays allowed)."""
    d = _desc(B=1, H=2, T=128)
    need = lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(d))
    ws = FAKE + (7 << 30)
    assert _chunk(lib, d, ST=FAKE + 256, ws=ws, ws_bytes=need) == INVALID              # S_T inside q
    assert _chunk(lib, d, ST=FAKE + (4 << 30), ws=ws, ws_bytes=need) == INVALID        # S_T on beta
    vd = _vdesc()
    assert _varlen(lib, vd, ST=FAKE + (2 << 30) + 512) == INVALID                      # S_T inside v
    assert _varlen(lib, vd, ST=FAKE + (3 << 30)) == INVALID                            # S_T on log_alpha


def test_backward_needs_the_forward_alignment(lib):
    """The backward reruns the forward's 16-byte loads on q, k, v, log_alpha (and reads dO the same
    way): 4-byte aligned inputs that kda_chunk_fwd refuses are refused here too."""
    d = _desc(B=1, H=2, T=256)
    P = ctypes.c_void_p
    base = [FAKE + (i << 30) for i in range(14)]

    def call(ptrs):
        return lib.kda_chunk_bwd(ctypes.byref(d), *[P(p) for p in ptrs], P(FAKE + (20 << 30)), 1 << 40, None)
    for i in (0, 1, 2, 3, 6):   # q k v log_alpha dO
        bad = list(base)
        bad[i] = base[i] + 4
        assert call(bad) == INVALID, i
    bad = list(base)
    bad[4] = base[4] + 1          # beta at an odd byte address
    assert call(bad) == INVALID
    bad = list(base)
    bad[4] = base[4] + 2          # beta only needs its element alignment
    assert call(bad) != INVALID


def test_binding_checks_caller_buffers():
    """The binding checks caller-supplied outputs and workspace like the inputs (shape, dtype,
    contiguity) before any device work; with CPU tensors the checks run and only then the call
    refuses to run off the GPU."""
    import torch
    B, H, T, d = 1, 2, 70, 64
    bf = torch.bfloat16
    q = torch.zeros(B, H, T, d, dtype=bf)
    beta = torch.zeros(B, H, T, dtype=bf)
    with pytest.raises(ValueError, match="S_T"):
        kda.chunk_fwd(q, q, q, q, beta, S_T=torch.zeros(B, H, d, d + 1))
    with pytest.raises(ValueError, match="S_T"):
        kda.chunk_fwd(q, q, q, q, beta, S_T=torch.zeros(B, H, d, d, dtype=torch.float64))
    with pytest.raises(ValueError, match="o must"):
        kda.chunk_fwd(q, q, q, q, beta, o=torch.zeros(B, H, T, d + 2, dtype=bf)[..., :d])   # strided view
    with pytest.raises(ValueError, match="workspace"):
        kda.chunk_fwd(q, q, q, q, beta, workspace=torch.zeros(64, 64, dtype=torch.uint8)[:, ::2])
    with pytest.raises(ValueError, match="runs on the GPU"):
        kda.chunk_fwd(q, q, q, q, beta, S_T=torch.zeros(B, H, d, d))
    # packed batch: S_ckpt with a wrong head count, ckpt_offsets with a wrong length, S_T shape
    pq = torch.zeros(H, 256, d, dtype=bf)
    pb = torch.zeros(H, 256, dtype=bf)
    cu = torch.tensor([0, 100, 256], dtype=torch.int32)
    with pytest.raises(ValueError, match="S_ckpt"):
        kda.chunk_fwd_varlen(pq, pq, pq, pq, pb, cu, ckpt_every=64, S_ckpt=torch.zeros(4, H + 1, d, d))
    with pytest.raises(ValueError, match="S_ckpt"):
        kda.chunk_fwd_varlen(pq, pq, pq, pq, pb, cu, ckpt_every=64, S_ckpt=torch.zeros(2, H, d, d))
    with pytest.raises(ValueError, match="ckpt_offsets"):
        kda.chunk_fwd_varlen(pq, pq, pq, pq, pb, cu, ckpt_every=64, ckpt_offsets=torch.zeros(2, dtype=torch.int32))
    with pytest.raises(ValueError, match="S_T"):
        kda.chunk_fwd_varlen(pq, pq, pq, pq, pb, cu, S_T=torch.zeros(1, H, d, d))
    with pytest.raises(ValueError, match="runs on the GPU"):
        kda.chunk_fwd_varlen(pq, pq, pq, pq, pb, cu, ckpt_every=64, S_ckpt=torch.zeros(4, H, d, d))
    with pytest.raises(ValueError, match="workspace"):
        kda.chunk_bwd(q, q, q, q, beta, None, q, workspace=torch.zeros(8, 8, dtype=torch.uint8).t())


def test_noalloc_rejects_calls_beyond_its_scratch(lib):
    """kda_chunk_fwd_noalloc refuses, before any device work, a call whose workspace would not fit
    the library's fixed scratch, and validates its arguments like kda_chunk_fwd."""
    P = ctypes.c_void_p
    call = lambda d, q=FAKE, o=FAKE + (5 << 30): lib.kda_chunk_fwd_noalloc(
        None if d is None else ctypes.byref(d), P(q), P(FAKE + (1 << 30)), P(FAKE + (2 << 30)), P(FAKE + (3 << 30)),
        P(FAKE + (4 << 30)), None, P(o), None, None)
    SCRATCH_ERR = -5
    assert kda.SCRATCH_BYTES == 192 << 20
    big = _desc(B=1, H=32, T=8192)
    assert lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(big)) > kda.SCRATCH_BYTES
    assert call(big) == SCRATCH_ERR
    assert lib.kda_status_string(SCRATCH_ERR).decode().startswith("KDA_ERR_SCRATCH")
    assert call(None) == INVALID
    assert call(_desc(dk=96)) == UNSUPPORTED
    assert call(_desc(), q=0) == INVALID
    assert call(_desc(), o=FAKE + 64) == INVALID   # o overlaps q
