"""GPU parity of the FP8 path (fa2_quantize_fp8, fa2_fwd_fp8) against the fp64 oracle.

Quantisation is integer work: codes and descales must match the oracle bit for bit.
The forward is compared with exact attention of the dequantised inputs under bounds
derived from the arithmetic (tests/gpu_util.fp8_head_bounds): an element-wise bound and
an RMS check against the expected error of independent roundings."""
import math

import numpy as np
import pytest
import torch

import exact_attention_85_amd as fa2
import oracle
import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _vt(vc):
    """[B, H, n_k, d] codes -> the transposed, zero-padded V layout [B, H, d, stride]."""
    B, H, n_k, d = vc.shape
    out = np.zeros((B, H, d, fa2.fp8_vt_stride(n_k)), dtype=np.uint8)
    out[:, :, :, :n_k] = np.transpose(vc, (0, 1, 3, 2))
    return out


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _check_against_oracle(o_gpu, lse_gpu, qc, kc, vc, dq, dk, dv, causal, scale, rows, what):
    """rows: list of (b, h, i).  Oracle rows + bounds per head, then one combined assertion."""
    table = oracle.e4m3_decode_table()
    B, H, n_q, d = qc.shape
    flat = np.array([(b * H + h) * n_q + i for b, h, i in rows], dtype=np.int64)
    o_ref, lse_ref = oracle.attention_fp8_rows(qc, kc, vc, dq, dk, dv, flat, causal, scale)
    bound = np.empty_like(o_ref)
    var = np.empty_like(o_ref)
    blse = np.empty_like(lse_ref)
    by_head = {}
    for n, (b, h, i) in enumerate(rows):
        by_head.setdefault((b, h), []).append((n, i))
    for (b, h), items in by_head.items():
        idx = np.array([n for n, _ in items])
        ii = np.array([i for _, i in items])
        qh = table[qc[b, h, ii]] * np.float64(dq[b, h])
        kh = table[kc[b, h]] * np.float64(dk[b, h])
        vh = table[vc[b, h]] * np.float64(dv[b, h])
        bo, va, bl = gu.fp8_head_bounds(qh, kh, vh, ii, causal, scale, o_ref[idx], lse_ref[idx])
        bound[idx], var[idx], blse[idx] = bo, va, bl
    o_g, l_g = gu.gpu_rows(o_gpu, lse_gpu, rows)
    return gu.assert_fp8_close(o_g, l_g, o_ref, lse_ref, bound, var, blse, what=what)


def _all_rows(B, H, n_q):
    return [(b, h, i) for b in range(B) for h in range(H) for i in range(n_q)]


def _codes_case(B, H, n_q, n_k, d, seed, exp_lo=9, exp_hi=14):
    qc = workloads.make_fp8_codes((B, H, n_q, d), seed * 8 + 0, exp_lo, exp_hi)
    kc = workloads.make_fp8_codes((B, H, n_k, d), seed * 8 + 1, exp_lo, exp_hi)
    vc = workloads.make_fp8_codes((B, H, n_k, d), seed * 8 + 2, exp_lo, exp_hi)
    dq = workloads.make_fp8_descales(B, H, seed * 8 + 3)
    dk = workloads.make_fp8_descales(B, H, seed * 8 + 4)
    dv = workloads.make_fp8_descales(B, H, seed * 8 + 5)
    return qc, kc, vc, dq, dk, dv


def _run_codes(qc, kc, vc, dq, dk, dv, causal, scale):
    o, lse = fa2.forward_fp8(_dev(qc), _dev(kc), _dev(_vt(vc)), _dev(dq), _dev(dk), _dev(dv),
                             causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


# ---------------------------------------------------------------- quantiser
QUANT_SHAPES = [(1, 1, 1, 64), (1, 1, 17, 128), (2, 3, 100, 64), (2, 2, 1000, 128), (1, 2, 4095, 128),
                (1, 1, 64, 64), (3, 1, 129, 128)]


@pytest.mark.parametrize("shape", QUANT_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("sigma", [1.0, 1e-3, 300.0])
def test_quantize_parity(shape, sigma):
    B, H, n, d = shape
    print(f"case quantize shape={shape} sigma={sigma}", flush=True)
    x = workloads.make_qkv_shape(B, H, n, n, d, seed=sum(shape) + int(sigma * 7), device=DEV, sigma=sigma)[0]
    if B * H > 1:
        x[-1, -1].zero_()  # an all-zero slice: descale 1, codes 0
    codes_ref, ds_ref = oracle.quantize_fp8(workloads.bf16_bits(x))
    codes, ds = fa2.quantize_fp8(x)
    vt, ds_t = fa2.quantize_fp8(x, transposed=True)
    torch.cuda.synchronize()
    codes, ds, vt, ds_t = (t.cpu().numpy() for t in (codes, ds, vt, ds_t))
    assert np.array_equal(ds, ds_ref) and np.array_equal(ds_t, ds_ref)
    bad = np.argwhere(codes != codes_ref)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[0]}"
    assert np.array_equal(vt[:, :, :, :n], np.transpose(codes_ref, (0, 1, 3, 2)))
    assert np.all(vt[:, :, :, n:] == 0)


# ---------------------------------------------------------------- forward on codes
RAGGED = [(1, 1), (17, 17), (100, 100), (255, 255), (600, 600), (17, 100), (100, 17), (255, 1000),
          (1000, 255), (129, 64), (64, 129), (300, 1)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", RAGGED)
def test_fwd_fp8_ragged(nq, nk, causal, d):
    scale = [0.5, 1.0 / math.sqrt(d), 2.0 / math.sqrt(d)][(nq + nk + d) % 3]
    seed = nq * 7919 + nk * 31 + d + int(causal)
    print(f"case fp8 ragged nq={nq} nk={nk} d={d} causal={causal} scale={scale}", flush=True)
    case = _codes_case(2, 2, nq, nk, d, seed)
    o, lse = _run_codes(*case, causal, scale)
    _check_against_oracle(o, lse, *case, causal, scale, _all_rows(2, 2, nq),
                          what=f"nq={nq} nk={nk} d={d} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("scale", [4.0, -2.0])
def test_fwd_fp8_peaked_and_negative_scale(d, scale):
    """Large |scale|: few keys carry each row (the bound is tight there); a negative scale
    flips the scores' sign."""
    print(f"case fp8 peaked d={d} scale={scale}", flush=True)
    case = _codes_case(1, 3, 333, 517, d, seed=d + int(scale * 10))
    for causal in (False, True):
        o, lse = _run_codes(*case, causal, scale / math.sqrt(d))
        _check_against_oracle(o, lse, *case, causal, scale / math.sqrt(d), _all_rows(1, 3, 333),
                              what=f"peaked d={d} scale={scale} causal={causal}")


def test_fwd_fp8_wide_exponents():
    """Codes of every exponent (subnormals included): wide dynamic range in both products."""
    print("case fp8 wide exponents", flush=True)
    case = _codes_case(1, 2, 200, 300, 128, seed=77, exp_lo=0, exp_hi=14)
    o, lse = _run_codes(*case, True, 0.02)
    _check_against_oracle(o, lse, *case, True, 0.02, _all_rows(1, 2, 200), what="wide exponents")


def test_fwd_fp8_deterministic():
    case = _codes_case(2, 4, 700, 700, 128, seed=5)
    o1, l1 = _run_codes(*case, True, 0.1)
    o2, l2 = _run_codes(*case, True, 0.1)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ---------------------------------------------------------------- end to end from bf16
def _end_to_end(q, k, v, causal, scale, rows, what):
    qc, dq = fa2.quantize_fp8(q)
    kc, dk = fa2.quantize_fp8(k)
    vt, dv = fa2.quantize_fp8(v, transposed=True)
    o, lse = fa2.forward_fp8(qc, kc, vt, dq, dk, dv, causal=causal, scale=scale)
    torch.cuda.synchronize()
    # the oracle quantises the same bf16 inputs itself (per head: only the heads the rows touch)
    B, H = q.shape[:2]
    heads = sorted({(b, h) for b, h, _ in rows})
    codes = {}
    for name, t in (("q", q), ("k", k), ("v", v)):
        c = np.zeros(tuple(t.shape), dtype=np.uint8)
        ds = np.ones((B, H), dtype=np.float32)
        for b, h in heads:
            cb, db = oracle.quantize_fp8(workloads.bf16_bits(t[b, h][None, None]))
            c[b, h], ds[b, h] = cb[0, 0], db[0, 0]
        codes[name] = (c, ds)
    (qc_r, dq_r), (kc_r, dk_r), (vc_r, dv_r) = codes["q"], codes["k"], codes["v"]
    return _check_against_oracle(o, lse, qc_r, kc_r, vc_r, dq_r, dk_r, dv_r, causal, scale, rows, what)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_fp8_end_to_end_small(d, causal):
    print(f"case fp8 end-to-end small d={d} causal={causal}", flush=True)
    q, k, v = workloads.make_qkv_shape(2, 3, 450, 390, d, seed=31 + d + int(causal), device=DEV)
    _end_to_end(q, k, v, causal, 1.0 / math.sqrt(d), _all_rows(2, 3, 450), f"e2e d={d} causal={causal}")


@pytest.mark.parametrize("w,causal", [(workloads.C3, False), (workloads.C3, True), (workloads.C4, False),
                                      (workloads.C4, True)], ids=["c3", "c3_causal", "c4", "c4_causal"])
def test_fwd_fp8_full_size_sampled(w, causal):
    """The named workloads' inputs, quantised on the GPU, at full size; sampled rows."""
    print(f"case fp8 {w.name} causal={causal}", flush=True)
    q, k, v = workloads.make_qkv(w, DEV)
    rows = gu.sample_rows(w.B, w.H, w.n_q, 48, seed=w.index * 10 + int(causal) + 500)
    _end_to_end(q, k, v, causal, w.scale, rows, f"{w.name} causal={causal}")


# ---------------------------------------------------------------- FP8 decode (one query row)
# The probabilities stay fp32 here, so the bf16 path's tolerance applies: |dO| <= 1e-2 plus half a bf16
# ulp of the reference (outputs reach |O| > 4 with these codes) and |dLSE| <= 1e-3.
DECODE_SHAPES = [(2, 3, 1, 64), (2, 3, 17, 128), (1, 4, 1000, 64), (3, 2, 4097, 128), (2, 2, 300, 128),
                 (1, 1, 8192, 128)]


@pytest.mark.parametrize("shape", DECODE_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("scale", [0.09, -0.3])
def test_decode_fp8_parity(shape, scale):
    B, H, n_k, d = shape
    print(f"case fp8 decode shape={shape} scale={scale}", flush=True)
    qc, kc, vc, dq, dk, dv = _codes_case(B, H, 1, n_k, d, seed=n_k + d + B)
    o, lse = fa2.decode_fp8(_dev(qc), _dev(kc), _dev(vc), _dev(dq), _dev(dk), _dev(dv), scale=scale)
    torch.cuda.synchronize()
    rows = np.arange(B * H, dtype=np.int64)
    o_ref, lse_ref = oracle.attention_fp8_rows(qc, kc, vc, dq, dk, dv, rows, False, scale)
    gu.assert_close(o.float().reshape(B * H, d).cpu().double().numpy(), lse.reshape(-1).cpu().double().numpy(),
                    o_ref, lse_ref, what=f"fp8 decode {shape} scale={scale}", out_grid=True)


def test_decode_fp8_full_size_sampled():
    """The decode workload's shape (B64 H32 N_k 8192 d128), bf16 inputs quantised on both sides."""
    w = workloads.C5
    print(f"case fp8 decode {w.name}", flush=True)
    q, k, v = workloads.make_qkv(w, DEV)
    qc, dq = fa2.quantize_fp8(q)
    kc, dk = fa2.quantize_fp8(k)
    vc, dv = fa2.quantize_fp8(v)
    o, lse = fa2.decode_fp8(qc, kc, vc, dq, dk, dv, scale=w.scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(55)
    heads = sorted(set(map(tuple, rng.integers(0, [w.B, w.H], (24, 2)).tolist())) | {(0, 0), (w.B - 1, w.H - 1)})
    o_ref = np.empty((len(heads), w.d))
    lse_ref = np.empty(len(heads))
    for n, (b, h) in enumerate(heads):
        codes = [oracle.quantize_fp8(workloads.bf16_bits(t[b, h][None, None])) for t in (q, k, v)]
        orow, lrow = oracle.attention_fp8_rows(codes[0][0], codes[1][0], codes[2][0], codes[0][1], codes[1][1],
                                               codes[2][1], np.array([0]), False, w.scale)
        o_ref[n], lse_ref[n] = orow[0], lrow[0]
    idx = torch.tensor([b * w.H + h for b, h in heads], device=DEV)
    og = o.float().reshape(w.B * w.H, w.d)[idx].cpu().double().numpy()
    lg = lse.reshape(-1)[idx].cpu().double().numpy()
    gu.assert_close(og, lg, o_ref, lse_ref, what="fp8 decode C5", out_grid=True)
