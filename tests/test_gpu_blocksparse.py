"""GPU parity of fa2_fwd_blocksparse (a byte mask over 128-row query blocks and 64-key
blocks, with a band) against the fp64 block-mask oracle, through the C ABI."""
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
BQ, BK = 128, 64


def _check_full(q, k, v, mask, wl, wr, scale, what):
    o, lse = fa2.forward_blocksparse(q, k, v, torch.from_numpy(mask).to(DEV), wl, wr, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_blockmask(*(workloads.bf16_to_f64(t) for t in (q, k, v)), mask, BQ, BK, scale,
                                                wl, wr)
    lg = lse.cpu().double().numpy()
    og = o.float().cpu().double().numpy()
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lg), empty), what
    assert np.all(og[empty] == 0), what
    gu.assert_close(og, np.where(empty, 0.0, lg), o_ref, np.where(empty, 0.0, lse_ref), what=what, out_grid=True)
    return o, lse


CASES = [  # B, H, N_q, N_k, d, mask shape (Mb, Mh), density, window
    (2, 3, 300, 700, 64, (1, 1), 0.5, (-1, -1)),
    (2, 3, 300, 700, 128, (2, 3), 0.3, (-1, -1)),
    (1, 4, 1000, 1000, 128, (1, 4), 0.6, (-1, 0)),
    (2, 2, 777, 500, 64, (2, 1), 0.4, (200, 50)),
    (1, 2, 129, 1500, 128, (1, 1), 0.1, (-1, -1)),
    (1, 2, 256, 256, 64, (1, 2), 0.0, (-1, -1)),   # nothing visible
    (1, 2, 640, 640, 128, (1, 1), 1.0, (-1, 0)),   # the all-ones mask
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}q{c[2]}k{c[3]}d{c[4]}m{c[5][0]}x{c[5][1]}p{c[6]}"
                                              f"w{c[7][0]}_{c[7][1]}" for c in CASES])
def test_random_masks(case):
    B, H, nq, nk, d, (Mb, Mh), dens, (wl, wr) = case
    print(f"case blocksparse {case}", flush=True)
    q, k, v = workloads.make_qkv_shape(B, H, nq, nk, d, nq + nk + d, DEV)
    mask = workloads.random_block_mask((Mb, Mh, -(-nq // BQ), -(-nk // BK)), dens, nq * 3 + nk)
    _check_full(q, k, v, mask, wl, wr, 1.0 / math.sqrt(d), f"blocksparse {case}")


def test_all_ones_mask_is_the_tile_kernel_bit_for_bit():
    q, k, v = workloads.make_qkv_shape(2, 2, 900, 1100, 128, 41, DEV)
    ones = torch.ones((-(-900 // BQ), -(-1100 // BK)), dtype=torch.uint8, device=DEV)
    for wl, wr in ((-1, -1), (-1, 0), (300, 20)):
        o1, l1 = fa2.forward_blocksparse(q, k, v, ones, wl, wr)
        o2, l2 = fa2.forward_config(q, k, v, 0, wl, wr)  # the 4-wave kernel on the dense loop
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), (wl, wr)


@pytest.mark.parametrize("causal", [True, False])
def test_dilated_mask(causal):
    n, d = 3000, 128
    q, k, v = workloads.make_qkv_shape(1, 4, n, n, d, 43 + causal, DEV)
    mask = workloads.dilated_block_mask(n, n, 3, 4, causal)
    print(f"case dilated N{n} r3 w4 causal={causal}: {int(mask.sum())} of {mask.size} blocks", flush=True)
    _check_full(q, k, v, mask, -1, 0 if causal else -1, 1.0 / math.sqrt(d), f"dilated causal={causal}")


def test_dilated_long_sequence_all_rows():
    # the long-sequence shape (B1 H32 N16384 d128), causal, dilation 2 over 64 key blocks per side:
    # every row against the oracle
    w = workloads.C4
    q, k, v = workloads.make_qkv(w, DEV)
    mask = workloads.dilated_block_mask(w.n_q, w.n_k, 2, 64, True)
    print(f"case dilated {w.name}: {int(mask.sum())} of {mask.size} blocks", flush=True)
    o, lse = fa2.forward_blocksparse(q, k, v, torch.from_numpy(mask).to(DEV), -1, 0, scale=w.scale)
    torch.cuda.synchronize()

    def rows_oracle(qb, kb, vb, rows, b):
        return oracle.attention_blockmask_rows_bf16(qb, kb, vb, rows, mask, BQ, BK, w.scale, -1, 0)

    gu.assert_all_rows(q, k, v, o, lse, True, w.scale, what=f"dilated {w.name}", rows_oracle=rows_oracle)


def test_mask_errors():
    q, k, v = workloads.make_qkv_shape(1, 2, 200, 300, 64, 5, DEV)
    good = torch.ones((2, 5), dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        fa2.forward_blocksparse(q, k, v, torch.ones((2, 4), dtype=torch.uint8, device=DEV))
    with pytest.raises(ValueError):
        fa2.forward_blocksparse(q, k, v, torch.ones((3, 2, 5), dtype=torch.uint8, device=DEV))
    with pytest.raises(ValueError):
        fa2.forward_blocksparse(q, k, v, good.cpu())
    with pytest.raises(TypeError):
        fa2.forward_blocksparse(q, k, v, good.float())
    with pytest.raises(fa2.Fa2Error):
        fa2.forward_blocksparse(q, k, v, good, -5, 0)
    o, lse = fa2.forward_blocksparse(q, k, v, good)
    torch.cuda.synchronize()
    assert torch.isfinite(lse).all()
