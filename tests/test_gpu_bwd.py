"""GPU parity of fa2_bwd (deterministic attention backward) against the fp64
oracle's gradients: small and ragged shapes with both masks, bit-exact
repeatability, a side stream, and full-size workloads checked on sampled heads."""
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


def _run(q, k, v, do, causal, scale):
    o, lse = fa2.forward(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa2.backward(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, dq, dk, dv


def _check_heads(q, k, v, do, o, dq, dk, dv, causal, scale, heads, what):
    """Gradients of the listed (b, h) heads against the oracle (heads gathered into one batch)."""
    pick = lambda t: workloads.bf16_to_f64(torch.stack([t[b, h] for (b, h) in heads])[:, None])  # noqa: E731
    qd, kd, vd, dod, od = (pick(t) for t in (q, k, v, do, o))
    ref = oracle.backward(qd, kd, vd, dod, causal, scale)
    bounds = gu.bwd_bounds(qd, kd, vd, od, dod, causal, scale)
    got = tuple(pick(t) for t in (dq, dk, dv))
    gu.assert_grads_close(got, ref, bounds, what=f"{what} heads {heads}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(1, 1), (17, 100), (100, 17), (64, 128), (129, 257), (300, 300), (513, 200)])
def test_bwd_parity(nq, nk, causal, d):
    print(f"case bwd nq={nq} nk={nk} d={d} causal={causal}", flush=True)
    scale = 1.0 / math.sqrt(d)
    q, k, v = workloads.make_qkv_shape(2, 2, nq, nk, d, 3 * nq + nk + d + int(causal), DEV)
    do = workloads.make_qkv_shape(2, 2, nq, 1, d, 999 + nq, DEV)[0]
    o, dq, dk, dv = _run(q, k, v, do, causal, scale)
    _check_heads(q, k, v, do, o, dq, dk, dv, causal, scale, [(0, 0), (0, 1), (1, 0), (1, 1)],
                 f"nq={nq} nk={nk} d={d} causal={causal}")


# Many heads (many workgroups in both passes), ragged key counts and N_q < N_k or N_q > N_k
# (under the causal mask most key blocks then see no row, or rows see few keys); checked on
# sampled heads.
@pytest.mark.parametrize("B,H,nq,nk,d,causal", [
    (16, 16, 600, 600, 64, True), (16, 16, 64, 1000, 64, True), (8, 8, 200, 1900, 128, False),
    (8, 8, 300, 1900, 64, True), (4, 8, 150, 2000, 128, False), (4, 8, 1000, 2000, 64, True),
    (4, 8, 1900, 300, 128, True)])
def test_bwd_many_heads(B, H, nq, nk, d, causal):
    print(f"case bwd many heads B={B} H={H} nq={nq} nk={nk} d={d} causal={causal}", flush=True)
    assert fa2.bwd_workspace_bytes(B, H, nq, nk, d) == 2 * B * H * nq * 4
    scale = 1.0 / math.sqrt(d)
    q, k, v = workloads.make_qkv_shape(B, H, nq, nk, d, 31 * H + nq + int(causal), DEV)
    do = workloads.make_qkv_shape(B, H, nq, 1, d, 777 + nq, DEV)[0]
    o, dq, dk, dv = _run(q, k, v, do, causal, scale)
    _check_heads(q, k, v, do, o, dq, dk, dv, causal, scale, [(0, 0), (B // 2, 1), (B - 1, H - 1)],
                 f"many heads nq={nq} nk={nk} d={d} causal={causal}")


# From 2048 query rows at d = 128 (4096 under the causal mask) the dQ pass takes the 8-wave
# ping-pong kernel: ragged row and key counts around its 256-row blocks and 64-key tiles, both
# masks, and the causal 4-wave kernel just below its threshold
@pytest.mark.parametrize("nq,nk,causal", [(4101, 4101, True), (2053, 2053, False), (2100, 1, False),
                                          (4096, 100, True), (2300, 333, False), (4097, 4100, True),
                                          (4095, 4095, True)])
def test_bwd_pingpong_dq(nq, nk, causal):
    print(f"case bwd ping-pong dQ nq={nq} nk={nk} causal={causal}", flush=True)
    d, scale = 128, 1.0 / math.sqrt(128)
    q, k, v = workloads.make_qkv_shape(1, 2, nq, nk, d, 5 * nq + nk + int(causal), DEV)
    do = workloads.make_qkv_shape(1, 2, nq, 1, d, 55 + nq, DEV)[0]
    o, dq, dk, dv = _run(q, k, v, do, causal, scale)
    _check_heads(q, k, v, do, o, dq, dk, dv, causal, scale, [(0, 0), (0, 1)], f"pp nq={nq} nk={nk} causal={causal}")


def test_bwd_deterministic_and_stream():
    q, k, v = workloads.make_qkv_shape(2, 3, 700, 900, 128, 21, DEV)
    do = workloads.make_qkv_shape(2, 3, 700, 1, 128, 22, DEV)[0]
    for causal in (False, True):
        o, lse = fa2.forward(q, k, v, causal=causal, scale=0.09)
        g1 = fa2.backward(q, k, v, o, lse, do, causal=causal, scale=0.09)
        g2 = fa2.backward(q, k, v, o, lse, do, causal=causal, scale=0.09)
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            g3 = fa2.backward(q, k, v, o, lse, do, causal=causal, scale=0.09)
        s.synchronize()
        torch.cuda.synchronize()
        for a, b, c in zip(g1, g2, g3):
            assert torch.equal(a, b) and torch.equal(a, c)


@pytest.mark.parametrize("w,causal", [(workloads.C2, False), (workloads.C2, True), (workloads.C3, False),
                                      (workloads.C3, True)], ids=["c2", "c2_causal", "c3", "c3_causal"])
def test_bwd_full_size_sampled_heads(w, causal):
    print(f"case bwd {w.name} causal={causal}", flush=True)
    q, k, v = workloads.make_qkv(w, DEV)
    do = workloads.make_tensor(w.index, 3, w.B, w.H, w.n_q, w.d, DEV)
    o, dq, dk, dv = _run(q, k, v, do, causal, w.scale)
    assert all(torch.isfinite(t.float()).all() for t in (dq, dk, dv))
    _check_heads(q, k, v, do, o, dq, dk, dv, causal, w.scale, [(0, 0), (w.B - 1, w.H - 1)],
                 f"{w.name} causal={causal}")
