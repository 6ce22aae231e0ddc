"""GPU parity of fa2_fwd against the fp64 oracle (called through the C ABI via
the thin binding).  Tolerances: max|O - O_ref| <= 1e-2, max|LSE - LSE_ref| <= 1e-3."""
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


def _run(q, k, v, causal, scale):
    o, lse = fa2.forward(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def test_c1_full_parity():
    w = workloads.C1
    q, k, v = (t.to(DEV) for t in workloads.make_qkv(w))
    print(f"case C1 {w.name}", flush=True)
    o, lse = _run(q, k, v, False, w.scale)
    o_ref, lse_ref = gu.oracle_full(q, k, v, False, w.scale)
    gu.assert_close(o.float().cpu().double().numpy(), lse.cpu().double().numpy(), o_ref, lse_ref, what="C1")


RAGGED = [(1, 1), (17, 17), (100, 100), (255, 255), (1000, 1000), (17, 100), (100, 17), (255, 1000),
          (1000, 255), (129, 64), (64, 129)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", RAGGED)
def test_ragged_full_parity(nq, nk, causal, d):
    scale = [0.5, 1.0 / math.sqrt(d), 2.0][(nq + nk + d) % 3]
    seed = nq * 7919 + nk * 31 + d + int(causal)
    print(f"case ragged nq={nq} nk={nk} d={d} causal={causal} scale={scale}", flush=True)
    q, k, v = workloads.make_qkv_shape(2, 3, nq, nk, d, seed, DEV)
    o, lse = _run(q, k, v, causal, scale)
    o_ref, lse_ref = gu.oracle_full(q, k, v, causal, scale)
    gu.assert_close(o.float().cpu().double().numpy(), lse.cpu().double().numpy(), o_ref, lse_ref,
                    what=f"nq={nq} nk={nk} d={d} causal={causal}", out_grid=True)


@pytest.mark.parametrize("w,causal", [(workloads.C2, False), (workloads.C2, True), (workloads.C3, False),
                                      (workloads.C3, True), (workloads.C4, True), (workloads.C4, False)],
                         ids=["c2", "c2_causal", "c3", "c3_causal", "c4_causal", "c4"])
def test_full_size_all_rows(w, causal):
    # every row of the named workload against the oracle (C4 non-causal: 4.4 TFLOP of fp64 host
    # work, about 45 s on 16 cores)
    print(f"case {w.name} causal={causal}: all rows", flush=True)
    q, k, v = workloads.make_qkv(w, DEV)
    o, lse = _run(q, k, v, causal, w.scale)
    gu.assert_all_rows(q, k, v, o, lse, causal, w.scale, what=f"{w.name} causal={causal}")


@pytest.mark.parametrize("sigma", [2.0, 3.0])
def test_peaky_scores(sigma):
    # Q and K with sigma > 1 make the softmax sharply peaked (large maxima, many
    # underflowing probabilities); V stays N(0, 1)
    for causal in (False, True):
        q, k, v = workloads.make_qkv_shape(1, 4, 300, 300, 128, 77, DEV)
        q = (q.float() * sigma).to(torch.bfloat16)
        k = (k.float() * sigma).to(torch.bfloat16)
        o, lse = _run(q, k, v, causal, 1.0 / math.sqrt(128))
        o_ref, lse_ref = gu.oracle_full(q, k, v, causal, 1.0 / math.sqrt(128))
        gu.assert_close(o.float().cpu().double().numpy(), lse.cpu().double().numpy(), o_ref, lse_ref,
                        what=f"sigma={sigma} causal={causal}", out_grid=True)


@pytest.mark.parametrize("scale", [-0.25, 0.0, 1e-3])
def test_negative_and_zero_scale(scale):
    q, k, v = workloads.make_qkv_shape(1, 2, 150, 200, 64, 5, DEV)
    for causal in (False, True):
        o, lse = _run(q, k, v, causal, scale)
        o_ref, lse_ref = gu.oracle_full(q, k, v, causal, scale)
        gu.assert_close(o.float().cpu().double().numpy(), lse.cpu().double().numpy(), o_ref, lse_ref,
                        what=f"scale={scale} causal={causal}", out_grid=True)


def test_constant_v_causal_row0_uniform_q():
    d = 128
    q, k, v = workloads.make_qkv_shape(2, 2, 333, 333, d, 11, DEV)
    # constant V returns that constant for every row and mask
    c = torch.linspace(-2, 2, d, device=DEV).to(torch.bfloat16)
    vc = c.expand(2, 2, 333, d).contiguous()
    for causal in (False, True):
        o, _ = _run(q, k, vc, causal, 0.1)
        assert (o.float() - c.float()).abs().max().item() <= 1e-2
    # causal row 0 returns V[0] exactly and LSE = s_00
    o, lse = _run(q, k, v, True, 0.1)
    assert torch.equal(o[:, :, 0], v[:, :, 0])
    s00 = (q[:, :, 0].double() * k[:, :, 0].double()).sum(-1) * 0.1
    assert (lse[:, :, 0].double() - s00).abs().max().item() <= 1e-4
    # Q = 0: the mean of the visible values, LSE = ln(#visible)
    qz = torch.zeros_like(q)
    for causal in (False, True):
        o, lse = _run(qz, k, v, causal, 0.1)
        n = torch.arange(1, 334, device=DEV, dtype=torch.float64) if causal else torch.full((333,), 333.0,
                                                                                              device=DEV,
                                                                                              dtype=torch.float64)
        mean = v.double().cumsum(2) / n[None, None, :, None] if causal else v.double().mean(2, keepdim=True)
        assert (o.double() - mean).abs().max().item() <= 1e-2
        assert (lse.double() - n.log()).abs().max().item() <= 1e-3


def test_deterministic_and_stream():
    q, k, v = workloads.make_qkv_shape(2, 4, 777, 777, 128, 3, DEV)
    o1, l1 = _run(q, k, v, True, 0.09)
    o2, l2 = _run(q, k, v, True, 0.09)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o3, l3 = fa2.forward(q, k, v, causal=True, scale=0.09)
    s.synchronize()
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_many_heads_small_rows():
    # B*H large, N small: many tiny workgroups, one partial tile each
    q, k, v = workloads.make_qkv_shape(16, 40, 33, 47, 64, 9, DEV)
    for causal in (False, True):
        o, lse = _run(q, k, v, causal, 0.125)
        o_ref, lse_ref = gu.oracle_full(q, k, v, causal, 0.125)
        gu.assert_close(o.float().cpu().double().numpy(), lse.cpu().double().numpy(), o_ref, lse_ref,
                        what=f"many heads causal={causal}")


def test_errors_raise():
    q, k, v = workloads.make_qkv_shape(1, 1, 8, 8, 96, 1, DEV)
    with pytest.raises(fa2.Fa2Error) as e:
        fa2.forward(q, k, v)
    assert e.value.status == -3
    q, k, v = workloads.make_qkv_shape(1, 1, 8, 8, 64, 1, DEV)
    with pytest.raises(fa2.Fa2Error):
        fa2.forward(q, k, v, scale=float("nan"))


# Shapes at d = 128 that take the 8-wave ping-pong kernel (256-row blocks): unbanded attention
# from N_q = 2048, causal or windowed from N_q = 8192.  Ragged query and key tails included.
PINGPONG_FULL = [(2048, 2048), (2049, 777), (2300, 3001), (2111, 64), (2048, 1)]


@pytest.mark.parametrize("nq,nk", PINGPONG_FULL)
def test_pingpong_full_parity(nq, nk):
    print(f"case pingpong nq={nq} nk={nk}", flush=True)
    q, k, v = workloads.make_qkv_shape(1, 2, nq, nk, 128, seed=nq + 3 * nk, device=DEV)
    o, lse = _run(q, k, v, False, 1.0 / math.sqrt(128))
    o_ref, lse_ref = gu.oracle_full(q, k, v, False, 1.0 / math.sqrt(128))
    gu.assert_close(o.float().cpu().double().numpy(), lse.cpu().double().numpy(), o_ref, lse_ref,
                    what=f"pingpong nq={nq} nk={nk}")


@pytest.mark.parametrize("nq,nk,window", [(8192, 8192, None), (8300, 8300, None), (8200, 5000, None),
                                          (8450, 8450, (1000, 0)), (8192, 9000, (300, 300))])
def test_pingpong_banded_sampled(nq, nk, window):
    print(f"case pingpong banded nq={nq} nk={nk} window={window}", flush=True)
    q, k, v = workloads.make_qkv_shape(1, 2, nq, nk, 128, seed=nq + nk, device=DEV)
    scale = 1.0 / math.sqrt(128)
    if window is None:
        o, lse = _run(q, k, v, True, scale)
        wl, wr = -1, 0
    else:
        wl, wr = window
        o, lse = fa2.forward_window(q, k, v, wl, wr, scale=scale)
        torch.cuda.synchronize()
    rows = gu.sample_rows(1, 2, nq, 120, seed=nq, block=256)
    flat = np.array([h * nq + i for (_, h, i) in rows], dtype=np.int64)
    o_ref, lse_ref = oracle.attention_window_rows_bf16(workloads.bf16_bits(q), workloads.bf16_bits(k),
                                                       workloads.bf16_bits(v), flat, wl, wr, scale)
    o_g, l_g = gu.gpu_rows(o, lse, rows)
    gu.assert_close(o_g, l_g, o_ref, lse_ref, what=f"pingpong banded nq={nq} nk={nk} window={window}")


def test_bad_outputs_rejected():
    # caller-supplied outputs of the wrong shape, dtype or device are refused before any launch
    q, k, v = workloads.make_qkv_shape(1, 2, 100, 120, 64, 2, DEV)
    bf, f32 = torch.bfloat16, torch.float32
    with pytest.raises(ValueError):
        fa2.forward(q, k, v, out=torch.empty((1, 2, 99, 64), dtype=bf, device=DEV))
    with pytest.raises(ValueError):
        fa2.forward(q, k, v, out=torch.empty((1, 2, 100, 64), dtype=bf))  # host memory
    with pytest.raises(ValueError):
        fa2.forward(q, k, v, lse=torch.empty((1, 2, 100), dtype=torch.float64, device=DEV))
    with pytest.raises(ValueError):
        fa2.forward_window(q, k, v, 5, 0, out=torch.empty((1, 2, 100, 64), dtype=f32, device=DEV))
    with pytest.raises(ValueError):
        fa2.forward_splitkv(q, k, v, num_splits=2, workspace=torch.empty(1 << 20, dtype=f32))
    with pytest.raises(fa2.Fa2Error) as e:  # a workspace one element short
        need = fa2.splitkv_workspace_bytes(1, 2, 100, 64, 2) // 4
        fa2.forward_splitkv(q, k, v, num_splits=2, workspace=torch.empty(need - 1, dtype=f32, device=DEV))
    assert e.value.status == -5
    o, lse = fa2.forward(q, k, v)
    do = torch.randn_like(q)
    with pytest.raises(ValueError):
        fa2.backward(q, k, v, o, lse, do, dk=torch.empty((1, 2, 100, 64), dtype=bf, device=DEV))
    torch.cuda.synchronize()
