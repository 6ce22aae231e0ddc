"""GPU parity of fa2_fwd_window (sliding-window / banded attention) against the
oracle's windowed attention: small and ragged shapes over many bands, rows that
see no key, equality with fa2_fwd for the plain and causal bands, full-size
sampled rows, and the single-row (decode) route."""
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

SHAPES = [(1, 1), (17, 100), (100, 17), (255, 255), (300, 1000), (513, 513), (129, 64), (64, 129)]
WINDOWS = [(0, 0), (1, 0), (7, 3), (63, 0), (64, 64), (200, -1), (-1, 5), (1000, 1000), (0, -1), (31, 33),
           (127, 0), (5, 130)]


def _oracle_window(q, k, v, wl, wr, scale):
    return oracle.attention_window(workloads.bf16_to_f64(q), workloads.bf16_to_f64(k), workloads.bf16_to_f64(v),
                                   wl, wr, scale)


def _check(o, lse, o_ref, lse_ref, what, out_grid=True):
    og = o.float().cpu().double().numpy()
    lg = lse.cpu().double().numpy()
    empty = np.isneginf(lse_ref)
    # rows that see no key: exactly zero output and -inf log-sum-exp
    assert np.all(og[empty] == 0.0), what
    assert np.all(np.isneginf(lg[empty])), what
    seen = ~empty
    gu.assert_close(og[seen], lg[seen], o_ref[seen], lse_ref[seen], what=what, out_grid=out_grid)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("nq,nk", SHAPES)
def test_window_parity(nq, nk, d):
    scale = 1.0 / math.sqrt(d)
    q, k, v = workloads.make_qkv_shape(2, 3, nq, nk, d, 7 * nq + 13 * nk + d, DEV)
    # three bands per shape, chosen so that every band meets every head dim over the sweep
    picks = [WINDOWS[(nq + nk + d + 5 * t) % len(WINDOWS)] for t in range(3)]
    for wl, wr in picks:
        print(f"case window nq={nq} nk={nk} d={d} wl={wl} wr={wr}", flush=True)
        o, lse = fa2.forward_window(q, k, v, wl, wr, scale=scale)
        torch.cuda.synchronize()
        o_ref, lse_ref = _oracle_window(q, k, v, wl, wr, scale)
        _check(o, lse, o_ref, lse_ref, f"nq={nq} nk={nk} d={d} window=({wl},{wr})")


@pytest.mark.parametrize("d", [64, 128])
def test_window_all_bands_one_shape(d):
    scale = 0.9 / math.sqrt(d)
    q, k, v = workloads.make_qkv_shape(1, 2, 333, 270, d, 91 + d, DEV)
    for wl, wr in WINDOWS:
        print(f"case window sweep d={d} wl={wl} wr={wr}", flush=True)
        o, lse = fa2.forward_window(q, k, v, wl, wr, scale=scale)
        torch.cuda.synchronize()
        o_ref, lse_ref = _oracle_window(q, k, v, wl, wr, scale)
        _check(o, lse, o_ref, lse_ref, f"d={d} window=({wl},{wr})")


def test_plain_and_causal_bands_equal_fwd():
    for d in (64, 128):
        q, k, v = workloads.make_qkv_shape(2, 2, 700, 650, d, 5 + d, DEV)
        for causal, (wl, wr) in ((False, (-1, -1)), (True, (-1, 0))):
            o1, l1 = fa2.forward(q, k, v, causal=causal, scale=0.1)
            o2, l2 = fa2.forward_window(q, k, v, wl, wr, scale=0.1)
            torch.cuda.synchronize()
            assert torch.equal(o1, o2) and torch.equal(l1, l2), (d, causal)


@pytest.mark.parametrize("wl,wr", [(4095, 0), (1023, 1024)])
def test_window_full_size_sampled(wl, wr):
    w = workloads.C4
    print(f"case {w.name} window=({wl},{wr})", flush=True)
    q, k, v = workloads.make_qkv(w, DEV)
    o, lse = fa2.forward_window(q, k, v, wl, wr, scale=w.scale)
    torch.cuda.synchronize()
    rows = gu.sample_rows(w.B, w.H, w.n_q, 160, seed=wl + wr)
    flat = np.array([(b * w.H + h) * w.n_q + i for (b, h, i) in rows], dtype=np.int64)
    o_ref, lse_ref = oracle.attention_window_rows_bf16(workloads.bf16_bits(q), workloads.bf16_bits(k),
                                                       workloads.bf16_bits(v), flat, wl, wr, w.scale)
    o_g, l_g = gu.gpu_rows(o, lse, rows)
    gu.assert_close(o_g, l_g, o_ref, lse_ref, what=f"C4 window=({wl},{wr})")
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("wr", [0, 3, 700, -1])
def test_window_single_row(wr):
    q, k, v = workloads.make_qkv_shape(4, 8, 1, 2000, 128, 17 + wr, DEV)
    o, lse = fa2.forward_window(q, k, v, 50, wr, scale=0.088)
    torch.cuda.synchronize()
    o_ref, lse_ref = _oracle_window(q, k, v, 50, wr, 0.088)
    _check(o, lse, o_ref, lse_ref, f"single row wr={wr}")
