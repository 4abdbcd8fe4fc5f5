"""Host-only checks of libdr's C ABI: the library loads, exports every symbol include/dr.h
declares, and rejects invalid arguments synchronously.  No call here reaches a kernel: every
call either fails validation (pointers are fake, never dereferenced) or only queries sizes."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_dr_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dr.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_abi.LIB_PATH), reason="libdr.so not built")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(dr_\w+)\s*\(", src, re.M)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == set(_abi.EXPORTS)
    lib = ctypes.CDLL(_abi.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    L = _abi.lib()
    assert L.dr_abi_version() == 1
    for code in range(-9, 1):
        assert _abi.status_str(code)
    assert _abi.status_str(-99) == "unknown status"
    assert _abi.status_str(0) == "ok"


def _good_desc(**kw):
    d = _abi.DrDesc()
    vals = dict(B=2, T=100, H=4, dk=128, dv=128, chunk=0, qkv_dtype=_abi.DR_BF16, o_dtype=_abi.DR_F32,
                decay_kind=_abi.DR_GATE_HEAD, erase_kind=_abi.DR_GATE_HEAD, write_kind=_abi.DR_GATE_HEAD,
                write_is_erase=1)
    vals.update(kw)
    for k, v in vals.items():
        setattr(d, k, v)
    return d


GB = 1 << 30
# Fake, 16-byte aligned, widely separated addresses: validation never dereferences them.
P = {name: (i + 1) * 64 * GB for i, name in enumerate(["q", "k", "v", "ld", "e", "w", "S0", "o", "ST", "ws"])}


def _fwd(desc, **over):
    ptr = dict(P)
    ptr.update(over)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return _abi.lib().dr_chunk_fwd(ctypes.byref(desc) if desc is not None else None,
                                   vp(ptr["q"]), vp(ptr["k"]), vp(ptr["v"]), vp(ptr["ld"]), vp(ptr["e"]),
                                   vp(ptr["w"]), vp(ptr["S0"]), vp(ptr["o"]), vp(ptr["ST"]),
                                   vp(ptr["ws"]), ptr.get("wsn", 1 << 30), None)


def _dec(desc, **over):
    ptr = dict(P)
    ptr.update(over)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return _abi.lib().dr_decode_step(ctypes.byref(desc), vp(ptr["q"]), vp(ptr["k"]), vp(ptr["v"]),
                                     vp(ptr["ld"]), vp(ptr["e"]), vp(ptr["w"]), vp(ptr["S0"]), vp(ptr["o"]), None)


def test_null_arguments():
    assert _fwd(None) == _abi.DR_E_NULL
    d = _good_desc()
    for name in ("q", "k", "v", "ld", "e", "o"):
        assert _fwd(d, **{name: None}) == _abi.DR_E_NULL, name
    assert _fwd(_good_desc(write_is_erase=0), w=None) == _abi.DR_E_NULL
    assert _dec(_good_desc(T=1), S0=None) == _abi.DR_E_NULL


def test_shape_errors():
    for kw in (dict(B=0), dict(H=0), dict(T=-1), dict(dk=0), dict(dv=-4)):
        assert _fwd(_good_desc(**kw)) == _abi.DR_E_SHAPE, kw
    # per-channel erase reused as the write gate needs dk == dv
    assert _fwd(_good_desc(dk=64, dv=128, erase_kind=_abi.DR_GATE_CHANNEL)) == _abi.DR_E_SHAPE
    # decode is exactly one token
    assert _dec(_good_desc(T=2)) == _abi.DR_E_SHAPE
    # element counts that overflow
    assert _fwd(_good_desc(B=2**30, T=2**30, H=2**30)) == _abi.DR_E_SHAPE


def test_dtype_and_kind_errors():
    assert _fwd(_good_desc(qkv_dtype=7)) == _abi.DR_E_DTYPE
    assert _fwd(_good_desc(o_dtype=-1)) == _abi.DR_E_DTYPE
    assert _fwd(_good_desc(decay_kind=2)) == _abi.DR_E_DTYPE
    assert _fwd(_good_desc(erase_kind=5)) == _abi.DR_E_DTYPE
    assert _fwd(_good_desc(write_is_erase=0, write_kind=3)) == _abi.DR_E_DTYPE


def test_unsupported():
    assert _fwd(_good_desc(dk=96)) == _abi.DR_E_UNSUPPORTED
    assert _fwd(_good_desc(dv=256)) == _abi.DR_E_UNSUPPORTED
    assert _fwd(_good_desc(chunk=32)) == _abi.DR_E_UNSUPPORTED


def test_alignment():
    d = _good_desc()
    for name in ("q", "k", "v", "ld", "e", "S0", "o", "ST"):
        assert _fwd(d, **{name: P[name] + 4}) == _abi.DR_E_ALIGN, name


def test_aliasing():
    d = _good_desc()
    assert _fwd(d, o=P["q"]) == _abi.DR_E_ALIAS
    assert _fwd(d, o=P["v"] + 1024) == _abi.DR_E_ALIAS  # partial overlap
    assert _fwd(d, ST=P["k"]) == _abi.DR_E_ALIAS
    assert _fwd(d, ST=P["o"]) == _abi.DR_E_ALIAS
    assert _fwd(d, ST=P["S0"] + 4096) == _abi.DR_E_ALIAS  # overlapping but not identical
    assert _dec(_good_desc(T=1), o=P["S0"]) == _abi.DR_E_ALIAS
    assert _dec(_good_desc(T=1), S0=P["e"]) == _abi.DR_E_ALIAS


def test_workspace_query_and_errors():
    L = _abi.lib()
    # matrix-core path: one packet per chunk of every (b, h) -- the six nonzero 16 x 32 blocks of
    # each lower-triangular fp16 64 x 64 matrix (2 or 4), fp16 operand tiles, fp32 gate vector
    # (256 floats for a per-head decay with symmetric gates, else 512)
    scal = 2 * 6 * 16 * 32 * 2 + 2 * 64 * 128 * 2 + 256 * 4
    kda = 2 * 6 * 16 * 32 * 2 + 3 * 64 * 128 * 2 + 512 * 4
    gen = 4 * 6 * 16 * 32 * 2 + 4 * 64 * 128 * 2 + 512 * 4
    assert L.dr_chunk_fwd_workspace_bytes(ctypes.byref(_good_desc())) == 2 * 4 * 2 * scal
    assert L.dr_chunk_fwd_workspace_bytes(ctypes.byref(_good_desc(T=64))) == 2 * 4 * 1 * scal
    ch = _good_desc(decay_kind=_abi.DR_GATE_CHANNEL)
    assert L.dr_chunk_fwd_workspace_bytes(ctypes.byref(ch)) == 2 * 4 * 2 * kda
    g1 = _good_desc(erase_kind=_abi.DR_GATE_CHANNEL)
    assert L.dr_chunk_fwd_workspace_bytes(ctypes.byref(g1)) == 2 * 4 * 2 * gen
    g2 = _good_desc(write_is_erase=0)
    assert L.dr_chunk_fwd_workspace_bytes(ctypes.byref(g2)) == 2 * 4 * 2 * gen
    g3 = _good_desc(write_is_erase=0, decay_kind=_abi.DR_GATE_CHANNEL, erase_kind=_abi.DR_GATE_CHANNEL)
    assert L.dr_chunk_fwd_workspace_bytes(ctypes.byref(g3)) == 2 * 4 * 2 * gen
    # separate erase and write gates: the packets, rounded up to 256 bytes, then the segmented
    # scan's maps (fp32 F, H and entering state per segment, 3 x 64 KiB) for S segments,
    # S = 1 + min(256 / (B * H), 8) and at most half the chunks: 2 x 4 heads of 10 chunks -> S = 5;
    # 1 x 32 heads of 1,024 chunks -> S = 9; 4 x 64 heads -> S = 1 (no maps)
    maps = 3 * 128 * 128 * 4
    up = lambda n: (n + 255) // 256 * 256
    g4 = _good_desc(write_is_erase=0, T=640)
    assert L.dr_chunk_fwd_workspace_bytes(ctypes.byref(g4)) == up(2 * 4 * 10 * gen) + 2 * 4 * 5 * maps
    g5 = _good_desc(write_is_erase=0, B=1, H=32, T=65536)
    assert L.dr_chunk_fwd_workspace_bytes(ctypes.byref(g5)) == up(32 * 1024 * gen) + 32 * 9 * maps
    g6 = _good_desc(write_is_erase=0, B=4, H=64, T=640)
    assert L.dr_chunk_fwd_workspace_bytes(ctypes.byref(g6)) == 4 * 64 * 10 * gen
    # token path and empty sequences need none
    assert L.dr_chunk_fwd_workspace_bytes(ctypes.byref(_good_desc(chunk=1))) == 0
    assert L.dr_chunk_fwd_workspace_bytes(ctypes.byref(_good_desc(qkv_dtype=_abi.DR_F32))) == 0
    assert L.dr_chunk_fwd_workspace_bytes(ctypes.byref(_good_desc(T=0))) == 0
    assert L.dr_chunk_fwd_workspace_bytes(None) == 0
    assert L.dr_chunk_fwd_workspace_bytes(ctypes.byref(_good_desc(B=0))) == 0
    need = L.dr_chunk_fwd_workspace_bytes(ctypes.byref(_good_desc()))
    assert _fwd(_good_desc(), wsn=need - 1) == _abi.DR_E_WORKSPACE
    assert _fwd(_good_desc(), ws=None, wsn=0) == _abi.DR_E_WORKSPACE
    assert _fwd(_good_desc(), ws=P["ws"] + 8, wsn=need) == _abi.DR_E_ALIGN
    assert _fwd(_good_desc(), ws=P["q"], wsn=need) == _abi.DR_E_ALIAS
    assert _fwd(_good_desc(), ws=P["o"] + 4096, wsn=need) == _abi.DR_E_ALIAS


def test_descriptor_layout():
    assert ctypes.sizeof(_abi.DrDesc) == 48
    src = open(HEADER).read()
    body = re.search(r"typedef struct \{(.*?)\} dr_desc;", src, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"(\w+)\s*[,;]", body)
    assert fields == [f[0] for f in _abi.DrDesc._fields_]


# ---- packed sequences of different lengths ---------------------------------------------------
P_CU = 2 * 1024 * GB  # fake device address of the offsets (4-byte aligned)


def _vfwd(desc, nseq=3, **over):
    ptr = dict(P)
    ptr.update(over)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return _abi.lib().dr_chunk_fwd_varlen(ctypes.byref(desc) if desc is not None else None,
                                          vp(ptr.get("cu", P_CU)), nseq,
                                          vp(ptr["q"]), vp(ptr["k"]), vp(ptr["v"]), vp(ptr["ld"]), vp(ptr["e"]),
                                          vp(ptr["w"]), vp(ptr["S0"]), vp(ptr["o"]), vp(ptr["ST"]),
                                          vp(ptr["ws"]), ptr.get("wsn", 1 << 30), None)


def test_varlen_workspace_query():
    L = _abi.lib()
    scal = 2 * 6 * 16 * 32 * 2 + 2 * 64 * 128 * 2 + 256 * 4
    gen = 4 * 6 * 16 * 32 * 2 + 4 * 64 * 128 * 2 + 512 * 4
    r256 = lambda n: (n + 255) // 256 * 256
    # T = 1000 packed tokens in 5 sequences: at most (1000 + 63 * 5) // 64 = 20 chunks per head
    d = _good_desc(B=1, T=1000)
    maxc = (1000 + 63 * 5) // 64
    tables = r256(16 * maxc) + r256(16 * 5) + r256(4 * 5) + 256
    assert L.dr_chunk_fwd_varlen_workspace_bytes(ctypes.byref(d), 5) == 4 * maxc * scal + tables
    g = _good_desc(B=1, T=1000, write_is_erase=0)
    assert L.dr_chunk_fwd_varlen_workspace_bytes(ctypes.byref(g), 5) == 4 * maxc * gen + tables
    # the token path keeps only the sequence table
    t = _good_desc(B=1, T=1000, chunk=1)
    assert L.dr_chunk_fwd_varlen_workspace_bytes(ctypes.byref(t), 5) == r256(16 * 5) + 256
    # invalid: B != 1, no sequences, too many
    assert L.dr_chunk_fwd_varlen_workspace_bytes(ctypes.byref(_good_desc(B=2)), 5) == 0
    assert L.dr_chunk_fwd_varlen_workspace_bytes(ctypes.byref(d), 0) == 0
    assert L.dr_chunk_fwd_varlen_workspace_bytes(ctypes.byref(d), -1) == 0
    assert L.dr_chunk_fwd_varlen_workspace_bytes(None, 5) == 0


def test_varlen_argument_errors():
    d = _good_desc(B=1, T=1000)
    assert _vfwd(None) == _abi.DR_E_NULL
    assert _vfwd(_good_desc(B=2)) == _abi.DR_E_SHAPE
    assert _vfwd(d, nseq=-1) == _abi.DR_E_SHAPE
    assert _vfwd(d, nseq=2**30 + 1) == _abi.DR_E_SHAPE
    assert _vfwd(d, cu=None) == _abi.DR_E_NULL
    assert _vfwd(d, cu=P_CU + 2) == _abi.DR_E_ALIGN
    for name in ("q", "k", "v", "ld", "e", "o"):
        assert _vfwd(d, **{name: None}) == _abi.DR_E_NULL, name
    # the states are [nseq, H, dk, dv]: S_T overlapping S0 partially, o or the offsets
    assert _vfwd(d, ST=P["S0"] + 4096) == _abi.DR_E_ALIAS
    assert _vfwd(d, o=P_CU) == _abi.DR_E_ALIAS
    assert _vfwd(d, ST=P_CU - 16) == _abi.DR_E_ALIAS
    assert _vfwd(d, ws=P_CU - 4096, wsn=1 << 30) == _abi.DR_E_ALIAS
    need = _abi.lib().dr_chunk_fwd_varlen_workspace_bytes(ctypes.byref(d), 3)
    assert _vfwd(d, wsn=need - 1) == _abi.DR_E_WORKSPACE
    assert _vfwd(d, ws=None, wsn=0) == _abi.DR_E_WORKSPACE
    # the per-sequence state is the extent that is checked: an S_T right after S0's 3 states is fine
    # to validate but one inside them is not
    state = 3 * 4 * 128 * 128 * 4
    assert _vfwd(d, ST=P["S0"] + state - 16) == _abi.DR_E_ALIAS


# ---- FG2's per-channel rate (erase kind DR_GATE_RATE_SQRT) ----------------------------------------
def test_rate_sqrt_kind():
    L = _abi.lib()
    R = _abi.DR_GATE_RATE_SQRT
    # symmetric packets plus the scaled values v~ as fp16 [64][128]
    scal = 2 * 6 * 16 * 32 * 2 + 2 * 64 * 128 * 2 + 256 * 4 + 64 * 128 * 2
    kda = 2 * 6 * 16 * 32 * 2 + 3 * 64 * 128 * 2 + 512 * 4 + 64 * 128 * 2
    assert (scal, kda) == (62464, 79872)
    d = _good_desc(erase_kind=R)
    assert L.dr_chunk_fwd_workspace_bytes(ctypes.byref(d)) == 2 * 4 * 2 * scal
    dc = _good_desc(erase_kind=R, decay_kind=_abi.DR_GATE_CHANNEL)
    assert L.dr_chunk_fwd_workspace_bytes(ctypes.byref(dc)) == 2 * 4 * 2 * kda
    assert L.dr_chunk_fwd_workspace_bytes(ctypes.byref(_good_desc(erase_kind=R, chunk=1))) == 0
    # the rate is read per channel of dk: passes validation of the extents (fake pointers fail later)
    assert _fwd(_good_desc(erase_kind=R), e=P["e"] + 8) == _abi.DR_E_ALIGN
    # needs write == erase and dk == dv; only the erase gate takes this kind
    assert _fwd(_good_desc(erase_kind=R, write_is_erase=0)) == _abi.DR_E_DTYPE
    assert _fwd(_good_desc(erase_kind=R, dk=64)) == _abi.DR_E_SHAPE
    assert _fwd(_good_desc(decay_kind=R)) == _abi.DR_E_DTYPE
    assert _fwd(_good_desc(write_is_erase=0, write_kind=R)) == _abi.DR_E_DTYPE
    # a per-channel extent: the rate array overlapping o by one channel row is an alias
    rate_bytes = 2 * 100 * 4 * 128 * 4
    assert _fwd(_good_desc(erase_kind=R), o=P["e"] + rate_bytes - 512) == _abi.DR_E_ALIAS


# ---- gradients ---------------------------------------------------------------------------------
PG = {name: (20 + i) * 64 * GB for i, name in enumerate(["dO", "dST", "dq", "dk", "dv", "dla", "de", "dw", "dS0"])}


def _bwd(desc, **over):
    ptr = dict(P)
    ptr.update(PG)
    ptr.update(over)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    names = ["q", "k", "v", "ld", "e", "w", "S0", "dO", "dST", "dq", "dk", "dv", "dla", "de", "dw", "dS0", "ws"]
    return _abi.lib().dr_chunk_bwd(ctypes.byref(desc), *[vp(ptr[n]) for n in names], ptr.get("wsn", 1 << 40), None)


def test_bwd_workspace_and_errors():
    L = _abi.lib()
    d = _good_desc(B=2, T=100, H=4, dk=128, dv=128)
    waves, nck, bth = 2 * 4 * 64, 2, 2 * 100 * 4
    # the token path (chunk = 1): one wave per (b, h, 256 / dk = 2 value columns), 64 column
    # groups; a checkpoint per chunk and one chunk of states per wave; row parts per workgroup of
    # 32 columns; v * dv~
    token = 4 * (waves * nck * 128 * 2 + waves * 64 * 128 * 2 + 4 * 4 * bth * 128 + bth * 128)
    assert L.dr_chunk_bwd_workspace_bytes(ctypes.byref(_good_desc(B=2, T=100, H=4, chunk=1))) == token
    # the chunk path (one per-head gate): the forward's packets (46,080 B per chunk), a bf16 o
    # buffer, the state at every chunk start and its adjoint at every chunk end (fp16), delta and
    # Z (fp16 [64][128] per chunk), the prep's A_kk (6 KB per chunk), then the per-token sums of
    # the per-head gates over each half of the channels (2 x (3 x 64 + 4) fp32 per chunk)
    r256 = lambda n: (n + 255) // 256 * 256
    chunks = 2 * 4 * nck
    need = (r256(chunks * 46080) + r256(bth * 128 * 2) + 2 * r256(chunks * 128 * 128 * 2) +
            2 * r256(chunks * 64 * 128 * 2) + r256(chunks * 6 * 1024) + r256(chunks * 2 * 196 * 4))
    assert L.dr_chunk_bwd_workspace_bytes(ctypes.byref(d)) == need
    assert L.dr_chunk_bwd_workspace_bytes(ctypes.byref(_good_desc(T=0))) == 0
    assert L.dr_chunk_bwd_workspace_bytes(ctypes.byref(_good_desc(erase_kind=_abi.DR_GATE_RATE_SQRT))) > 0
    for name in ("dO", "dq", "dk", "dv", "dla", "de"):
        assert _bwd(d, **{name: None}) == _abi.DR_E_NULL, name
    assert _bwd(_good_desc(write_is_erase=0), dw=None) == _abi.DR_E_NULL
    assert _bwd(d, dq=PG["dq"] + 8) == _abi.DR_E_ALIGN
    assert _bwd(d, dk=PG["dq"] + 4096) == _abi.DR_E_ALIAS  # two outputs overlap
    assert _bwd(d, dv=P["v"]) == _abi.DR_E_ALIAS  # output on an input
    assert _bwd(d, ws=PG["dO"], wsn=need) == _abi.DR_E_ALIAS
    assert _bwd(d, wsn=need - 1) == _abi.DR_E_WORKSPACE



def test_bwd_varlen_workspace_and_errors():
    L = _abi.lib()
    d = _good_desc(B=1, T=1000, H=4, dk=128, dv=128)
    nseq = 5
    maxc = (1000 + 63 * nseq) // 64
    nslice, waves, bth = 64, nseq * 4 * 64, 1000 * 4
    # the token path (chunk = 1): the sequence table, checkpoints, states, row parts, v * dv~
    tables = (16 * nseq + 255) // 256 * 256 + 256
    layout = 4 * (nslice * 4 * maxc * 128 * 2 + waves * 64 * 128 * 2 + 4 * (nslice // 16) * bth * 128 + bth * 128)
    assert L.dr_chunk_bwd_varlen_workspace_bytes(ctypes.byref(_good_desc(B=1, T=1000, H=4, chunk=1)), nseq) == \
        tables + layout
    # the chunk path: the packed forward's workspace (packets of H x maxc chunks, the chunk,
    # sequence and order tables, the count), then the dense path's buffers for H x maxc chunks
    r256 = lambda n: (n + 255) // 256 * 256
    chunks = 4 * maxc
    fwd = chunks * 46080 + r256(maxc * 16) + r256(nseq * 16) + r256(nseq * 4) + 256
    need = (r256(fwd) + r256(bth * 128 * 2) + 2 * r256(chunks * 128 * 128 * 2) + 2 * r256(chunks * 64 * 128 * 2) +
            r256(chunks * 6 * 1024) + r256(chunks * 2 * 196 * 4))
    assert L.dr_chunk_bwd_varlen_workspace_bytes(ctypes.byref(d), nseq) == need
    assert L.dr_chunk_bwd_varlen_workspace_bytes(ctypes.byref(_good_desc(B=2)), nseq) == 0
    assert L.dr_chunk_bwd_varlen_workspace_bytes(ctypes.byref(d), 0) == 0
    ptr = dict(P)
    ptr.update(PG)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    names = ["q", "k", "v", "ld", "e", "w", "S0", "dO", "dST", "dq", "dk", "dv", "dla", "de", "dw", "dS0", "ws"]

    def call(desc, cu=P_CU, n=nseq, **over):
        pp = dict(ptr)
        pp.update(over)
        return L.dr_chunk_bwd_varlen(ctypes.byref(desc), vp(cu), n, *[vp(pp[x]) for x in names], 1 << 40, None)

    assert call(_good_desc(B=2)) == _abi.DR_E_SHAPE
    assert call(d, cu=None) == _abi.DR_E_NULL
    assert call(d, cu=P_CU + 2) == _abi.DR_E_ALIGN
    assert call(d, dq=P_CU) == _abi.DR_E_ALIAS  # an output on the offsets
    assert call(d, n=-1) == _abi.DR_E_SHAPE


def _fwd_noalloc(desc, **over):
    ptr = dict(P)
    ptr.update(over)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return _abi.lib().dr_chunk_fwd_noalloc(ctypes.byref(desc) if desc is not None else None,
                                           vp(ptr["q"]), vp(ptr["k"]), vp(ptr["v"]), vp(ptr["ld"]), vp(ptr["e"]),
                                           vp(ptr["w"]), vp(ptr["S0"]), vp(ptr["o"]), vp(ptr["ST"]), None)


def test_noalloc_validates_before_any_device_work():
    # the allocation-free forward checks every argument as dr_chunk_fwd does, and refuses a
    # problem beyond its fixed scratch, all before it touches the device
    L = _abi.lib()
    assert L.dr_chunk_fwd_noalloc_max_bytes() == 64 << 20
    assert _abi.status_str(_abi.DR_E_SCRATCH) != "unknown status"
    assert _fwd_noalloc(None) == _abi.DR_E_NULL
    assert _fwd_noalloc(_good_desc(), q=None) == _abi.DR_E_NULL
    assert _fwd_noalloc(_good_desc(), o=P["q"]) == _abi.DR_E_ALIAS
    assert _fwd_noalloc(_good_desc(qkv_dtype=7)) == _abi.DR_E_DTYPE
    assert _fwd_noalloc(_good_desc(), k=P["k"] + 8) == _abi.DR_E_ALIGN
    # 2 x 4 heads x 100 tokens fit; 64 heads x 1,600 tokens of separate gates do not
    big = _good_desc(B=1, T=1600, H=64, decay_kind=_abi.DR_GATE_CHANNEL, erase_kind=_abi.DR_GATE_CHANNEL,
                     write_kind=_abi.DR_GATE_CHANNEL, write_is_erase=0)
    assert L.dr_chunk_fwd_workspace_bytes(ctypes.byref(big)) > 64 << 20
    assert _fwd_noalloc(big) == _abi.DR_E_SCRATCH
