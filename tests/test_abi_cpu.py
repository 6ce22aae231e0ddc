"""The C-ABI library loads, exports every entry point include/fa2.h declares,
and rejects bad arguments on the host before any HIP call (so these run
without a GPU: the pointers below are never dereferenced)."""
import ctypes
import os
import re

import pytest

import exact_attention_85_amd as fa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa2.h")

OK, NULLPTR, BAD_SHAPE, HEAD_DIM, BAD_SCALE, WORKSPACE, ALIAS, HIP, SPLITS, WINDOW, ALIGN, SCRATCH, CONFIG = (
    0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10, -11, -12)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa2_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["fa2_bwd", "fa2_bwd_workspace_bytes", "fa2_decode_fp8", "fa2_fp8_vt_stride", "fa2_fwd",
                                    "fa2_fwd_blocksparse",
                                    "fa2_fwd_config", "fa2_fwd_config_name", "fa2_fwd_default_config",
                                    "fa2_fwd_fp8", "fa2_fwd_num_configs", "fa2_fwd_splitkv",
                                    "fa2_fwd_splitkv_noalloc", "fa2_fwd_window", "fa2_num_splits",
                                    "fa2_probe_xcc", "fa2_quantize_fp8", "fa2_splitkv_workspace_bytes",
                                    "fa2_status_string"]


def test_status_codes_pinned():
    # the seven codes of the boundary's contract keep their values (FA2_ERR_HIP is -7);
    # the codes added for later entry points follow them
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef enum fa2_status \{(.*?)\} fa2_status;", text, flags=re.S).group(1)
    codes = {name: int(val) for name, val in re.findall(r"(FA2_[A-Z_]+)\s*=\s*(-?\d+)", body)}
    assert codes == {"FA2_OK": 0, "FA2_ERR_NULLPTR": -1, "FA2_ERR_BAD_SHAPE": -2, "FA2_ERR_HEAD_DIM": -3,
                     "FA2_ERR_BAD_SCALE": -4, "FA2_ERR_WORKSPACE": -5, "FA2_ERR_ALIAS": -6, "FA2_ERR_HIP": -7,
                     "FA2_ERR_SPLITS": -8, "FA2_ERR_WINDOW": -9, "FA2_ERR_ALIGN": -10, "FA2_ERR_SCRATCH": -11,
                     "FA2_ERR_CONFIG": -12}
    for name, val in codes.items():
        assert fa2.status_string(val).startswith(name + ":"), name


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fa2.lib_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for code in (OK, NULLPTR, BAD_SHAPE, HEAD_DIM, BAD_SCALE, WORKSPACE, ALIAS, SPLITS, HIP, WINDOW, ALIGN, SCRATCH, CONFIG):
        s = fa2.status_string(code)
        assert s and "unknown" not in s
    assert "unknown" in fa2.status_string(12345)


# fake, well separated device addresses: validation must fail before any use
GB = 1 << 30
Q, K, V, O, L, W = (0x10000000000 + i * 64 * GB for i in range(6))


def fwd(q=Q, k=K, v=V, o=O, l=L, B=1, H=2, nq=256, nk=256, d=64, causal=0, scale=0.125):
    lib = fa2.load_library()
    return lib.fa2_fwd(q, k, v, o, l, B, H, nq, nk, d, causal, scale, None)


def split(q=Q, k=K, v=V, o=O, l=L, B=1, H=2, nq=1, nk=256, d=64, causal=0, scale=0.125, s=4, ws=W,
          ws_bytes=None):
    lib = fa2.load_library()
    if ws_bytes is None:
        ws_bytes = lib.fa2_splitkv_workspace_bytes(B, H, nq, d, s)
    return lib.fa2_fwd_splitkv(q, k, v, o, l, B, H, nq, nk, d, causal, scale, s, ws, ws_bytes, None)


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "l"])
def test_null_pointers(which):
    assert fwd(**{which: None}) == NULLPTR
    assert split(**{which: None}) == NULLPTR


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(nq=0), dict(nk=0), dict(B=-1), dict(nk=-5),
                                dict(nk=(1 << 30) // 64 + 1), dict(nq=(1 << 30) // 64 + 1)])
def test_bad_shapes(kw):
    assert fwd(**kw) == BAD_SHAPE


@pytest.mark.parametrize("d", [0, 32, 96, 127, 256])
def test_head_dim(d):
    assert fwd(d=d) == HEAD_DIM
    assert split(d=d) == HEAD_DIM


@pytest.mark.parametrize("scale", [float("nan"), float("inf"), float("-inf"), 3e38])
def test_bad_scale(scale):
    assert fwd(scale=scale) == BAD_SCALE


def test_alias():
    # O overlapping Q, K, V or LSE; LSE overlapping an input
    assert fwd(o=Q) == ALIAS
    assert fwd(o=K + 100) == ALIAS
    assert fwd(o=V) == ALIAS
    assert fwd(o=L) == ALIAS
    assert fwd(l=Q + 2) == ALIAS
    assert split(ws=O) == ALIAS


def test_splits_and_workspace():
    lib = fa2.load_library()
    # S * B * H * N_q * (d + 2) * 4: per chunk and row, d accumulators, the reference m and the sum l
    for B, H, nq, d, S in ((64, 32, 1, 128, 16), (2, 3, 5, 64, 7), (1, 1, 1, 64, 1), (3, 1, 1000, 128, 256)):
        assert lib.fa2_splitkv_workspace_bytes(B, H, nq, d, S) == S * B * H * nq * (d + 2) * 4
    assert split(ws_bytes=lib.fa2_splitkv_workspace_bytes(1, 2, 1, 64, 4) - 1) == WORKSPACE
    assert lib.fa2_splitkv_workspace_bytes(1, 1, 1, 64, 0) == 0
    assert lib.fa2_splitkv_workspace_bytes(1, 1, 1, 64, 257) == 0
    assert split(s=0) == SPLITS
    assert split(s=257, nk=1000) == SPLITS
    assert split(s=300, nk=256) == SPLITS     # more splits than keys
    assert split(ws=None) == WORKSPACE
    assert split(ws_bytes=100) == WORKSPACE


# --- split-count heuristic (pure host arithmetic when num_cus > 0) ---
CUS = 256


# Shapes whose best split count was measured on MI355X (key-chunk sweep over
# S in {1, 2, 4, ..., 128}): the heuristic must land on the measured best or on a
# count within 5% of it.
@pytest.mark.parametrize("shape,allowed", [
    ((64, 32, 1, 8192, 128), {1}),          # decode, B*H = 2048 fills the chip
    ((1, 32, 1, 65536, 128), {8}),          # decode, B*H = 32
    ((1, 8, 1, 131072, 128), {16, 32}),     # decode, B*H = 8
    ((32, 8, 1, 4096, 128), {1, 2}),        # decode, B*H = 256
    ((1, 8, 2048, 2048, 128), {2, 4}),      # prefill, 128 query blocks
    ((1, 4, 4096, 4096, 128), {2, 4}),
    ((1, 2, 1024, 32768, 128), {16}),       # 16 query blocks, long keys
    ((2, 8, 512, 16384, 64), {8}),
    ((1, 16, 256, 8192, 128), {8}),
    ((1, 32, 128, 4096, 128), {8}),
    ((4, 16, 4096, 4096, 128), {1}),        # 2048 query blocks: no split
])
def test_num_splits_measured_shapes(shape, allowed):
    assert fa2.num_splits(*shape, num_cus=CUS) in allowed


def test_num_splits_properties():
    for B, H in ((1, 1), (1, 3), (2, 8), (4, 32), (64, 32)):
        for n_q in (1, 100, 128, 4096):
            for n_k in (1, 7, 512, 5000, 1 << 20):
                for d in (64, 128):
                    s = fa2.num_splits(B, H, n_q, n_k, d, num_cus=CUS)
                    units = B * H * (1 if n_q == 1 else -(-n_q // 128))
                    assert 1 <= s <= min(fa2.FA2_MAX_SPLITS, max(1, n_k // 512))
                    if units >= CUS:
                        assert s == 1
                    else:
                        # enough workgroups to cover the chip unless the chunk floor binds
                        assert units * s >= CUS or s == min(fa2.FA2_MAX_SPLITS, max(1, n_k // 512))
    # more units never asks for more splits
    prev = 10 ** 9
    for H in range(1, 300):
        s = fa2.num_splits(1, H, 1, 1 << 16, 128, num_cus=CUS)
        assert s <= prev
        prev = s


def test_num_splits_errors():
    with pytest.raises(fa2.Fa2Error) as e:
        fa2.num_splits(0, 1, 1, 1, 64, num_cus=CUS)
    assert e.value.status == BAD_SHAPE
    with pytest.raises(fa2.Fa2Error) as e:
        fa2.num_splits(1, 1, 1, 1, 96, num_cus=CUS)
    assert e.value.status == HEAD_DIM


def window(q=Q, k=K, v=V, o=O, l=L, B=1, H=2, nq=256, nk=256, d=64, wl=16, wr=0, scale=0.125):
    lib = fa2.load_library()
    return lib.fa2_fwd_window(q, k, v, o, l, B, H, nq, nk, d, wl, wr, scale, None)


def test_window_validation():
    for wl, wr in ((-2, 0), (0, -2), ((1 << 30) + 1, 0), (0, (1 << 30) + 1), (-7, -7)):
        assert window(wl=wl, wr=wr) == WINDOW
    assert window(q=None) == NULLPTR
    assert window(d=96) == HEAD_DIM
    assert window(nk=0) == BAD_SHAPE
    assert window(scale=float("nan")) == BAD_SCALE
    assert window(o=Q) == ALIAS


DO, DQ, DK, DV = (0x20000000000 + i * 64 * GB for i in range(4))


def bwd(q=Q, k=K, v=V, o=O, do=DO, l=L, dq=DQ, dk=DK, dv=DV, B=1, H=2, nq=256, nk=200, d=64, causal=0, scale=0.125,
        ws=W, ws_bytes=None):
    lib = fa2.load_library()
    if ws_bytes is None:
        ws_bytes = lib.fa2_bwd_workspace_bytes(B, H, nq, nk, d)
    return lib.fa2_bwd(q, k, v, o, do, l, dq, dk, dv, B, H, nq, nk, d, causal, scale, ws, ws_bytes, None)


def test_bwd_validation():
    lib = fa2.load_library()
    R = 1 * 2 * 256
    # LSE * log2(e) and D for every query row: 2 * B * H * N_q floats, whatever N_k and d
    for (B, H, nq, nk, d) in ((1, 2, 256, 200, 64), (1, 2, 256, 300, 128), (4, 16, 4096, 4096, 128),
                              (1, 32, 16384, 16384, 128), (8, 16, 2048, 2048, 64)):
        assert lib.fa2_bwd_workspace_bytes(B, H, nq, nk, d) == 2 * B * H * nq * 4
    assert lib.fa2_bwd_workspace_bytes(0, 2, 256, 200, 64) == 0
    for name in ("q", "k", "v", "o", "do", "l", "dq", "dk", "dv"):
        assert bwd(**{name: None}) == NULLPTR, name
    assert bwd(d=96) == HEAD_DIM
    assert bwd(nk=0) == BAD_SHAPE
    assert bwd(scale=float("inf")) == BAD_SCALE
    assert bwd(ws=None) == WORKSPACE
    assert bwd(ws_bytes=2 * 2 * 256 * 4 - 4) == WORKSPACE
    assert bwd(dq=Q) == ALIAS
    assert bwd(dk=DO + 10) == ALIAS
    assert bwd(dv=DQ) == ALIAS
    assert bwd(ws=DK) == ALIAS


# ---- FP8 entry points ----
SQ, SK, SV = (0x10000000000 + (6 + i) * 64 * GB for i in range(3))  # descale arrays


def fwd8(q=Q, k=K, v=V, dq=SQ, dk=SK, dv=SV, o=O, l=L, B=1, H=2, nq=256, nk=256, d=64, causal=0, scale=0.125):
    lib = fa2.load_library()
    return lib.fa2_fwd_fp8(q, k, v, dq, dk, dv, o, l, B, H, nq, nk, d, causal, scale, None)


def quant8(x=Q, c=K, s=L, B=1, H=2, n=256, d=64, t=0):
    return fa2.load_library().fa2_quantize_fp8(x, c, s, B, H, n, d, t, None)


def test_fp8_vt_stride():
    lib = fa2.load_library()
    assert [lib.fa2_fp8_vt_stride(n) for n in (1, 15, 16, 17, 100, 4096)] == [16, 16, 16, 32, 112, 4096]
    assert lib.fa2_fp8_vt_stride(0) == BAD_SHAPE and lib.fa2_fp8_vt_stride((1 << 30) + 1) == BAD_SHAPE


@pytest.mark.parametrize("which", ["q", "k", "v", "dq", "dk", "dv", "o", "l"])
def test_fp8_null_pointers(which):
    assert fwd8(**{which: None}) == NULLPTR


@pytest.mark.parametrize("which", ["x", "c", "s"])
def test_quant8_null_pointers(which):
    assert quant8(**{which: None}) == NULLPTR


def test_fp8_shapes_and_scale():
    assert fwd8(nq=0) == BAD_SHAPE and fwd8(nk=0) == BAD_SHAPE and fwd8(B=0) == BAD_SHAPE
    assert fwd8(d=96) == HEAD_DIM and quant8(d=32) == HEAD_DIM
    assert quant8(n=0) == BAD_SHAPE and quant8(B=256, H=256) == BAD_SHAPE
    assert fwd8(scale=float("nan")) == BAD_SCALE


@pytest.mark.parametrize("which", ["q", "k", "v", "dq", "o", "l"])
def test_fp8_alignment(which):
    base = dict(q=Q, k=K, v=V, dq=SQ, o=O, l=L)
    assert fwd8(**{which: base[which] + 8}) == ALIGN


def test_quant8_alignment_and_alias():
    assert quant8(x=Q + 2) == ALIGN and quant8(c=K + 4) == ALIGN
    # codes overlapping X, descale overlapping codes
    assert quant8(c=Q + 256) == ALIAS
    assert quant8(s=K + 16) == ALIAS
    # transposed codes are d * stride per head: a descale right after the row-layout size overlaps
    assert quant8(n=100, s=K + 2 * 100 * 64, t=1) == ALIAS


def test_fp8_alias():
    # O over the transposed V codes (d * stride bytes per head), LSE over a descale
    assert fwd8(o=V + 64 * 256 * 2 - 16) == ALIAS
    assert fwd8(l=SK) == ALIAS
    assert fwd8(o=L) == ALIAS


def dec8(q=Q, k=K, v=V, dq=SQ, dk=SK, dv=SV, o=O, l=L, B=2, H=3, nk=500, d=128, scale=0.1):
    return fa2.load_library().fa2_decode_fp8(q, k, v, dq, dk, dv, o, l, B, H, nk, d, scale, None)


def test_decode_fp8_validation():
    for name in ("q", "k", "v", "dq", "dk", "dv", "o", "l"):
        assert dec8(**{name: None}) == NULLPTR, name
    assert dec8(nk=0) == BAD_SHAPE and dec8(B=0) == BAD_SHAPE
    assert dec8(d=96) == HEAD_DIM
    assert dec8(scale=float("inf")) == BAD_SCALE
    assert dec8(v=V + 4) == ALIGN
    assert dec8(o=K + 64) == ALIAS
    assert dec8(l=SV) == ALIAS


def test_work_item_limits():
    # a dispatch counts at most 2^32 - 1 work-items: 2^20 heads of one query row in 16 chunks
    # need 2^24 decode workgroups of 256 work-items, one past it; nothing is enqueued
    lib = fa2.load_library()
    need = lib.fa2_splitkv_workspace_bytes(1 << 10, 1 << 10, 1, 128, 16)
    assert split(B=1 << 10, H=1 << 10, nq=1, nk=16, d=128, s=16, ws_bytes=need) == BAD_SHAPE
    # the tile kernel: ceil(N_q / 128) * B * H workgroups of 256 work-items
    assert fwd(B=1 << 12, H=1 << 12, nq=128, nk=16, d=64) == BAD_SHAPE
    assert window(B=1 << 12, H=1 << 12, nq=128, nk=16, d=64) == BAD_SHAPE
    assert fwd8(B=1 << 12, H=1 << 12, nq=128, nk=16, d=64) == BAD_SHAPE
    assert dec8(B=1 << 12, H=1 << 12, nk=16, d=64) == BAD_SHAPE
    # the backward: the key pass takes 512 work-items per 128-key block, the dQ pass 256 per
    # 128-row block (or 512 per 256 rows); 2^22 heads reach 2^32 at 2 key blocks or 512 rows
    assert bwd(B=1 << 11, H=1 << 11, nq=128, nk=256, d=128) == BAD_SHAPE
    assert bwd(B=1 << 11, H=1 << 11, nq=512, nk=128, d=128) == BAD_SHAPE
    assert bwd(B=1 << 11, H=1 << 11, nq=256, nk=128, d=128) != BAD_SHAPE  # 2^22 * 512 < 2^32


def noalloc(q=Q, k=K, v=V, o=O, l=L, B=1, H=2, nq=1, nk=256, d=64, causal=0, scale=0.125, s=4):
    return fa2.load_library().fa2_fwd_splitkv_noalloc(q, k, v, o, l, B, H, nq, nk, d, causal, scale, s, None)


def test_noalloc_validation():
    # the checks of fa2_fwd_splitkv, then the fixed array's size, all before any HIP call
    text = open(HEADER).read()
    assert "#define FA2_NOALLOC_SCRATCH_BYTES (32u << 20)" in text
    assert fa2.NOALLOC_SCRATCH_BYTES == 32 << 20
    assert noalloc(q=None) == NULLPTR
    assert noalloc(d=96) == HEAD_DIM
    assert noalloc(s=0) == SPLITS and noalloc(s=300, nk=256) == SPLITS
    assert noalloc(o=Q) == ALIAS
    assert noalloc(scale=float("nan")) == BAD_SCALE
    # partials of S * B * H * N_q * (d + 2) * 4 bytes: one chunk-row more than fits is refused
    S, d = 16, 128
    rows_fit = (32 << 20) // (S * (d + 2) * 4)
    assert noalloc(B=1, H=rows_fit + 1, nq=1, nk=64, d=d, s=S) == SCRATCH
    assert noalloc(B=4, H=64, nq=1024, nk=8192, d=d, s=S) == SCRATCH


def cfg(q=Q, k=K, v=V, o=O, l=L, B=1, H=2, nq=256, nk=256, d=64, wl=-1, wr=0, scale=0.125, c=0):
    return fa2.load_library().fa2_fwd_config(q, k, v, o, l, B, H, nq, nk, d, wl, wr, scale, c, None)


def test_config_validation():
    n = fa2.num_configs()
    assert n == 10 and len({fa2.config_name(c) for c in range(n)}) == n
    assert cfg(c=-1) == CONFIG and cfg(c=n) == CONFIG
    assert cfg(q=None) == NULLPTR and cfg(d=96) == HEAD_DIM and cfg(wl=-5) == WINDOW and cfg(o=Q) == ALIAS
    assert fa2.load_library().fa2_fwd_config_name(n) is None
    with pytest.raises(ValueError):
        fa2.config_name(n)
    with pytest.raises(fa2.Fa2Error):
        fa2.default_config(96, False, 100)
    assert fa2.load_library().fa2_probe_xcc(None, 10, None) == NULLPTR
    assert fa2.load_library().fa2_probe_xcc(Q, 0, None) == BAD_SHAPE


MASK = 0x10000000000 + 9 * 64 * GB


def bsp(q=Q, k=K, v=V, o=O, l=L, B=2, H=3, nq=300, nk=700, d=64, m=MASK, Mb=1, Mh=1, wl=-1, wr=-1, scale=0.125):
    return fa2.load_library().fa2_fwd_blocksparse(q, k, v, o, l, B, H, nq, nk, d, m, Mb, Mh, wl, wr, scale, None)


def test_blocksparse_validation():
    assert bsp(m=None) == NULLPTR and bsp(q=None) == NULLPTR
    assert bsp(Mb=3) == BAD_SHAPE and bsp(Mh=2) == BAD_SHAPE and bsp(Mb=0) == BAD_SHAPE
    assert bsp(d=96) == HEAD_DIM and bsp(wl=-2) == WINDOW and bsp(scale=float("inf")) == BAD_SCALE
    assert bsp(o=Q) == ALIAS
    # O or LSE over the mask: [Mb][Mh][3][11] bytes at MASK
    assert bsp(o=MASK + 16) == ALIAS and bsp(l=MASK + 2 * 3 * 3 * 11 - 1, Mb=2, Mh=3) == ALIAS
    assert bsp(B=1 << 12, H=1 << 12, nq=128, nk=16) == BAD_SHAPE  # launch limits
