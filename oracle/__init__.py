"""Exact-attention oracle (fp64, CPU).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the bench's
CPU-baseline leg may import this package; the product path never does.  It
shares no code with the HIP library.

The arithmetic lives in ``attn_oracle.c`` (plain C, fp64, textbook two-pass
softmax); this module only marshals numpy arrays through ctypes.  What is
computed follows the FlashAttention-2 walkthrough page, "kernel main loop"
section (online-softmax pseudocode; v1 and v2 compute the same mathematics):
for each query row i,

    s_ij  = scale * q_i . k_j          over allowed j (j < N_k, and j <= i if causal)
    O_i   = sum_j exp(s_ij - m_i) v_j / sum_j exp(s_ij - m_i),   m_i = max_j s_ij
    LSE_i = m_i + ln sum_j exp(s_ij - m_i)

Arrays are contiguous [B, H, N, d]; LSE is [B, H, N_q].
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i64p = ctypes.POINTER(ctypes.c_int64)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_i = ctypes.c_int


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_attention_f64.argtypes = [_dp, _dp, _dp, _dp, _dp, _i, _i, _i, _i, _i, _i, ctypes.c_double]
    lib.oracle_attention_rows_bf16.argtypes = [_u16p, _u16p, _u16p, _i64p, ctypes.c_int64, _dp, _dp,
                                               _i, _i, _i, _i, _i, _i, ctypes.c_double]
    lib.oracle_partial_f64.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _i, _i, _i, _i, _i, _i, ctypes.c_double,
                                       _i, _i]
    lib.oracle_merge_f64.argtypes = [_dp, _dp, _dp, _dp, _dp, _i, ctypes.c_int64, _i]
    lib.oracle_probs_f64.argtypes = [_dp, _dp, _dp, _i, _i, _i, _i, _i, _i, ctypes.c_double]
    lib.oracle_bf16_to_f64.argtypes = [_u16p, _dp, ctypes.c_int64]
    lib.oracle_attention_window_f64.argtypes = [_dp, _dp, _dp, _dp, _dp, _i, _i, _i, _i, _i, _i, _i,
                                                ctypes.c_double]
    lib.oracle_attention_window_rows_bf16.argtypes = [_u16p, _u16p, _u16p, _i64p, ctypes.c_int64, _dp, _dp,
                                                      _i, _i, _i, _i, _i, _i, _i, ctypes.c_double]
    lib.oracle_window_pairs.argtypes = [_i, _i, _i, _i]
    lib.oracle_window_pairs.restype = ctypes.c_int64
    lib.oracle_backward_f64.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _i, _i, _i, _i, _i, _i,
                                        ctypes.c_double]
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_decode.restype = ctypes.c_double
    lib.oracle_quantize_fp8.argtypes = [_u16p, ctypes.POINTER(ctypes.c_uint8), ctypes.POINTER(ctypes.c_float),
                                        _i, _i, _i, _i]
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    _fp = ctypes.POINTER(ctypes.c_float)
    lib.oracle_attention_fp8_rows.argtypes = [_u8p, _u8p, _u8p, _fp, _fp, _fp, _i64p, ctypes.c_int64, _dp, _dp,
                                              _i, _i, _i, _i, _i, _i, ctypes.c_double]
    lib.oracle_attention_blockmask_f64.argtypes = [_dp, _dp, _dp, _dp, _dp, _i, _i, _i, _i, _i, _u8p, _i, _i, _i,
                                                   _i, _i, _i, ctypes.c_double]
    lib.oracle_attention_blockmask_rows_bf16.argtypes = [_u16p, _u16p, _u16p, _i64p, ctypes.c_int64, _dp, _dp, _i,
                                                         _i, _i, _i, _i, _u8p, _i, _i, _i, _i, _i, _i,
                                                         ctypes.c_double]
    lib.oracle_blockmask_pairs.argtypes = [_i, _i, _u8p, _i, _i, _i, _i, _i, _i, _i, _i]
    lib.oracle_blockmask_pairs.restype = ctypes.c_int64
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a, typ):
    return a.ctypes.data_as(typ)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle: {what} rejected its arguments")


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact fp64 values of bf16 numbers given as uint16 bit patterns."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float64)
    _load().oracle_bf16_to_f64(_ptr(bits, _u16p), _ptr(out, _dp), bits.size)
    return out


def attention(q, k, v, causal: bool, scale: float):
    """O [B,H,N_q,d] and LSE [B,H,N_q] in fp64 from fp64 inputs."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, n_q, d = q.shape
    n_k = k.shape[2]
    assert k.shape == (B, H, n_k, d) and v.shape == (B, H, n_k, d)
    o = np.empty((B, H, n_q, d), dtype=np.float64)
    lse = np.empty((B, H, n_q), dtype=np.float64)
    rc = _load().oracle_attention_f64(_ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), _ptr(o, _dp), _ptr(lse, _dp),
                                      B, H, n_q, n_k, d, int(bool(causal)), float(scale))
    _check(rc, "attention")
    return o, lse


def attention_rows_bf16(q_bits, k_bits, v_bits, rows, causal: bool, scale: float):
    """O and LSE for selected flat rows ((b*H + h)*N_q + i) of bf16 inputs given as uint16 bit arrays."""
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    k_bits = np.ascontiguousarray(k_bits, dtype=np.uint16)
    v_bits = np.ascontiguousarray(v_bits, dtype=np.uint16)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    B, H, n_q, d = q_bits.shape
    n_k = k_bits.shape[2]
    assert k_bits.shape == (B, H, n_k, d) and v_bits.shape == (B, H, n_k, d)
    o = np.empty((rows.size, d), dtype=np.float64)
    lse = np.empty((rows.size,), dtype=np.float64)
    rc = _load().oracle_attention_rows_bf16(_ptr(q_bits, _u16p), _ptr(k_bits, _u16p), _ptr(v_bits, _u16p),
                                            _ptr(rows, _i64p), rows.size, _ptr(o, _dp), _ptr(lse, _dp),
                                            B, H, n_q, n_k, d, int(bool(causal)), float(scale))
    _check(rc, "attention_rows_bf16")
    return o, lse


def partial(q, k, v, causal: bool, scale: float, key_begin: int, key_end: int):
    """Unnormalised (acc [B,H,N_q,d], m [B,H,N_q], l [B,H,N_q]) over keys [key_begin, key_end)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, n_q, d = q.shape
    n_k = k.shape[2]
    acc = np.empty((B, H, n_q, d), dtype=np.float64)
    m = np.empty((B, H, n_q), dtype=np.float64)
    l_ = np.empty((B, H, n_q), dtype=np.float64)
    rc = _load().oracle_partial_f64(_ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), _ptr(acc, _dp), _ptr(m, _dp),
                                    _ptr(l_, _dp), B, H, n_q, n_k, d, int(bool(causal)), float(scale),
                                    int(key_begin), int(key_end))
    _check(rc, "partial")
    return acc, m, l_


def merge(acc, m, l_):
    """Merge partials stacked on axis 0: acc [S, ..., d], m and l [S, ...] -> (O [..., d], LSE [...])."""
    acc, m, l_ = _f64(acc), _f64(m), _f64(l_)
    n_parts = acc.shape[0]
    d = acc.shape[-1]
    row_shape = acc.shape[1:-1]
    n_rows = int(np.prod(row_shape)) if row_shape else 1
    assert m.shape == (n_parts,) + row_shape and l_.shape == m.shape
    o = np.empty(row_shape + (d,), dtype=np.float64)
    lse = np.empty(row_shape, dtype=np.float64)
    rc = _load().oracle_merge_f64(_ptr(acc, _dp), _ptr(m, _dp), _ptr(l_, _dp), _ptr(o, _dp), _ptr(lse, _dp),
                                  n_parts, n_rows, d)
    _check(rc, "merge")
    return o, lse


def probs(q, k, causal: bool, scale: float):
    """The attention probability matrix P [B,H,N_q,N_k] (zeros where masked)."""
    q, k = _f64(q), _f64(k)
    B, H, n_q, d = q.shape
    n_k = k.shape[2]
    p = np.empty((B, H, n_q, n_k), dtype=np.float64)
    rc = _load().oracle_probs_f64(_ptr(q, _dp), _ptr(k, _dp), _ptr(p, _dp), B, H, n_q, n_k, d,
                                  int(bool(causal)), float(scale))
    _check(rc, "probs")
    return p


def attention_window(q, k, v, window_left: int, window_right: int, scale: float):
    """Sliding-window attention in fp64: key j is visible to query i iff j < N_k,
    (window_left < 0 or j >= i - window_left) and (window_right < 0 or j <= i + window_right).
    Rows that see no key get O = 0 and LSE = -inf."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, n_q, d = q.shape
    n_k = k.shape[2]
    assert k.shape == (B, H, n_k, d) and v.shape == (B, H, n_k, d)
    o = np.empty((B, H, n_q, d), dtype=np.float64)
    lse = np.empty((B, H, n_q), dtype=np.float64)
    rc = _load().oracle_attention_window_f64(_ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), _ptr(o, _dp),
                                             _ptr(lse, _dp), B, H, n_q, n_k, d, int(window_left),
                                             int(window_right), float(scale))
    _check(rc, "attention_window")
    return o, lse


def attention_window_rows_bf16(q_bits, k_bits, v_bits, rows, window_left: int, window_right: int, scale: float):
    """attention_window for selected flat rows of bf16 inputs given as uint16 bit arrays."""
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    k_bits = np.ascontiguousarray(k_bits, dtype=np.uint16)
    v_bits = np.ascontiguousarray(v_bits, dtype=np.uint16)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    B, H, n_q, d = q_bits.shape
    n_k = k_bits.shape[2]
    o = np.empty((rows.size, d), dtype=np.float64)
    lse = np.empty((rows.size,), dtype=np.float64)
    rc = _load().oracle_attention_window_rows_bf16(_ptr(q_bits, _u16p), _ptr(k_bits, _u16p), _ptr(v_bits, _u16p),
                                                   _ptr(rows, _i64p), rows.size, _ptr(o, _dp), _ptr(lse, _dp),
                                                   B, H, n_q, n_k, d, int(window_left), int(window_right),
                                                   float(scale))
    _check(rc, "attention_window_rows_bf16")
    return o, lse


def window_pairs(n_q: int, n_k: int, window_left: int, window_right: int) -> int:
    """Visible (query, key) pairs of one head under the window."""
    return int(_load().oracle_window_pairs(int(n_q), int(n_k), int(window_left), int(window_right)))


def backward(q, k, v, do, causal: bool, scale: float):
    """Gradients (dQ, dK, dV) of exact attention for upstream gradient dO, in fp64:
    P = softmax(scale Q K^T [+ causal mask]), dV = P^T dO, dS = P * (dO V^T - rowsum(dO * O)),
    dQ = scale dS K, dK = scale dS^T Q."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, n_q, d = q.shape
    n_k = k.shape[2]
    assert k.shape == (B, H, n_k, d) and v.shape == (B, H, n_k, d) and do.shape == q.shape
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    rc = _load().oracle_backward_f64(_ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), _ptr(do, _dp), _ptr(dq, _dp),
                                     _ptr(dk, _dp), _ptr(dv, _dp), B, H, n_q, n_k, d, int(bool(causal)),
                                     float(scale))
    _check(rc, "backward")
    return dq, dk, dv


def e4m3_decode_table() -> np.ndarray:
    """fp64 value of every e4m3fn code 0..255.  Codes 0x7f and 0xff are NaN in the format; the table
    holds their bit pattern's arithmetic value, which no quantised code ever takes."""
    lib = _load()
    return np.array([lib.oracle_e4m3_decode(c) for c in range(256)], dtype=np.float64)


def e4m3_encode(y: float) -> int:
    """Round-to-nearest-even e4m3fn code of the fp32 value y (|y| <= 448)."""
    return int(_load().oracle_e4m3_encode(float(np.float32(y))))


def quantize_fp8(x_bits):
    """Per-(batch, head) e4m3 quantisation of bf16 X (uint16 bit array [B, H, N, d]):
    returns (codes uint8 [B, H, N, d], descale fp32 [B, H])."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    B, H, n, d = x_bits.shape
    codes = np.empty((B, H, n, d), dtype=np.uint8)
    descale = np.empty((B, H), dtype=np.float32)
    rc = _load().oracle_quantize_fp8(_ptr(x_bits, _u16p), codes.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
                                     descale.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), B, H, n, d)
    _check(rc, "quantize_fp8")
    return codes, descale


def dequantize_fp8(codes, descale):
    """decode(code) * descale of each (batch, head) slice, in fp64."""
    table = e4m3_decode_table()
    return table[np.asarray(codes)] * np.asarray(descale, dtype=np.float64)[..., None, None]


def attention_fp8(qc, kc, vc, dq, dk, dv, causal: bool, scale: float):
    """Exact attention (fp64) of the dequantised FP8 inputs; codes [B, H, N, d] with V in row layout,
    descales [B, H].  Returns (O, LSE)."""
    return attention(dequantize_fp8(qc, dq), dequantize_fp8(kc, dk), dequantize_fp8(vc, dv), causal, scale)


def attention_fp8_rows(qc, kc, vc, dq, dk, dv, rows, causal: bool, scale: float):
    """attention_fp8 for the flattened rows (b*H + h)*N_q + i listed in `rows`: (O [n, d], LSE [n])."""
    u8 = ctypes.POINTER(ctypes.c_uint8)
    fp = ctypes.POINTER(ctypes.c_float)
    qc, kc, vc = (np.ascontiguousarray(a, dtype=np.uint8) for a in (qc, kc, vc))
    dq, dk, dv = (np.ascontiguousarray(a, dtype=np.float32) for a in (dq, dk, dv))
    B, H, n_q, d = qc.shape
    n_k = kc.shape[2]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    O = np.empty((len(rows), d), dtype=np.float64)
    L = np.empty(len(rows), dtype=np.float64)
    rc = _load().oracle_attention_fp8_rows(qc.ctypes.data_as(u8), kc.ctypes.data_as(u8), vc.ctypes.data_as(u8),
                                           dq.ctypes.data_as(fp), dk.ctypes.data_as(fp), dv.ctypes.data_as(fp),
                                           _ptr(rows, _i64p), len(rows), _ptr(O, _dp), _ptr(L, _dp),
                                           B, H, n_q, n_k, d, int(causal), float(scale))
    _check(rc, "attention_fp8_rows")
    return O, L


def _mask4(mask, B, H):
    """A block mask as a contiguous uint8 [Mb, Mh, n_qb, n_kb] array with Mb in {1, B}, Mh in {1, H}."""
    m = np.ascontiguousarray(mask, dtype=np.uint8)
    if m.ndim == 2:
        m = m[None, None]
    elif m.ndim == 3:
        m = m[None]
    assert m.ndim == 4 and m.shape[0] in (1, B) and m.shape[1] in (1, H), m.shape
    return np.ascontiguousarray(m)


def attention_blockmask(q, k, v, mask, block_q: int, block_k: int, scale: float, window_left: int = -1,
                        window_right: int = -1):
    """Block-sparse attention in fp64 (the synthesis page, section 5 item 4).

    mask: uint8 [n_qb, n_kb], [Mh, n_qb, n_kb] or [Mb, Mh, n_qb, n_kb] (Mb in {1, B}, Mh in {1, H};
    n_qb = ceil(N_q / block_q), n_kb = ceil(N_k / block_k)).  Key j is visible to query i of
    (b, h) iff mask[b][h][i // block_q][j // block_k] != 0 and the band (window_left,
    window_right) admits it (as attention_window).  Rows that see no key get O = 0, LSE = -inf."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, n_q, d = q.shape
    n_k = k.shape[2]
    m = _mask4(mask, B, H)
    assert m.shape[2:] == (-(-n_q // block_q), -(-n_k // block_k)), m.shape
    o = np.empty((B, H, n_q, d), dtype=np.float64)
    lse = np.empty((B, H, n_q), dtype=np.float64)
    rc = _load().oracle_attention_blockmask_f64(_ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), _ptr(o, _dp),
                                                _ptr(lse, _dp), B, H, n_q, n_k, d, _ptr(m, _u8p), m.shape[0],
                                                m.shape[1], int(block_q), int(block_k), int(window_left),
                                                int(window_right), float(scale))
    _check(rc, "attention_blockmask")
    return o, lse


def attention_blockmask_rows_bf16(q_bits, k_bits, v_bits, rows, mask, block_q: int, block_k: int, scale: float,
                                  window_left: int = -1, window_right: int = -1):
    """attention_blockmask for selected flat rows ((b*H + h)*N_q + i) of bf16 inputs given as uint16 bits."""
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    k_bits = np.ascontiguousarray(k_bits, dtype=np.uint16)
    v_bits = np.ascontiguousarray(v_bits, dtype=np.uint16)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    B, H, n_q, d = q_bits.shape
    n_k = k_bits.shape[2]
    m = _mask4(mask, B, H)
    assert m.shape[2:] == (-(-n_q // block_q), -(-n_k // block_k)), m.shape
    o = np.empty((rows.size, d), dtype=np.float64)
    lse = np.empty((rows.size,), dtype=np.float64)
    rc = _load().oracle_attention_blockmask_rows_bf16(_ptr(q_bits, _u16p), _ptr(k_bits, _u16p), _ptr(v_bits, _u16p),
                                                      _ptr(rows, _i64p), rows.size, _ptr(o, _dp), _ptr(lse, _dp),
                                                      B, H, n_q, n_k, d, _ptr(m, _u8p), m.shape[0], m.shape[1],
                                                      int(block_q), int(block_k), int(window_left),
                                                      int(window_right), float(scale))
    _check(rc, "attention_blockmask_rows_bf16")
    return o, lse


def blockmask_pairs(n_q: int, n_k: int, mask, b: int, h: int, block_q: int, block_k: int, window_left: int = -1,
                    window_right: int = -1) -> int:
    """Visible (query, key) pairs of one (b, h) under the block mask and band."""
    m = np.ascontiguousarray(mask, dtype=np.uint8)
    while m.ndim < 4:
        m = m[None]
    m = np.ascontiguousarray(m)
    return int(_load().oracle_blockmask_pairs(int(n_q), int(n_k), _ptr(m, _u8p), m.shape[0], m.shape[1], int(b),
                                              int(h), int(block_q), int(block_k), int(window_left),
                                              int(window_right)))
