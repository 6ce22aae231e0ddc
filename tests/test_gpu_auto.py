"""GPU parity of the two automatic routes: fa2_fwd with a single query row
(the streaming decode kernel writing O and LSE directly) and attention(),
which takes the split count from fa2_num_splits."""
import math

import pytest
import torch

import exact_attention_85_amd as fa2
import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,nk", [(2, 3, 1), (2, 3, 5), (4, 8, 1000), (3, 5, 4097), (1, 2, 70000)])
def test_single_row_forward_parity(B, H, nk, causal, d):
    scale = [1.0 / math.sqrt(d), -0.3, 0.0][(nk + d) % 3]
    print(f"case single-row fwd B={B} H={H} nk={nk} d={d} causal={causal} scale={scale}", flush=True)
    q, k, v = workloads.make_qkv_shape(B, H, 1, nk, d, nk * 3 + d + B, DEV)
    o, lse = fa2.forward(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = gu.oracle_full(q, k, v, causal, scale)
    gu.assert_close(o.float().cpu().double().numpy(), lse.cpu().double().numpy(), o_ref, lse_ref,
                    what=f"single row B={B} H={H} nk={nk}", out_grid=True)
    # the split path over the same keys agrees
    o2, l2 = fa2.forward_splitkv(q, k, v, num_splits=min(nk, 7), causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert (o.float() - o2.float()).abs().max().item() <= 1e-2
    assert (lse - l2).abs().max().item() <= 1e-3


def test_decode_full_size_direct():
    w = workloads.C5
    print(f"case {w.name} direct", flush=True)
    q, k, v = workloads.make_qkv(w, DEV)
    o, lse = fa2.forward(q, k, v, scale=w.scale)
    torch.cuda.synchronize()
    gu.assert_all_rows(q, k, v, o, lse, False, w.scale, what="decode C5 direct", heads_per_call=w.H)
    o2, l2 = fa2.forward(q, k, v, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2)


def test_num_splits_queries_the_device():
    cus = torch.cuda.get_device_properties(DEV).multi_processor_count
    for shape in ((1, 8, 1, 131072, 128), (1, 4, 4096, 4096, 128), (64, 32, 1, 8192, 128), (1, 1, 300, 5000, 64)):
        assert fa2.num_splits(*shape) == fa2.num_splits(*shape, num_cus=cus)


@pytest.mark.parametrize("B,H,nq,nk,d,causal", [(1, 4, 300, 5000, 64, False), (1, 4, 300, 5000, 64, True),
                                                 (1, 2, 1, 20000, 128, False), (1, 2, 640, 9000, 128, True),
                                                 (2, 3, 129, 257, 128, False)])
def test_attention_auto_split_parity(B, H, nq, nk, d, causal):
    scale = 1.0 / math.sqrt(d)
    s = fa2.num_splits(B, H, nq, nk, d)
    print(f"case auto B={B} H={H} nq={nq} nk={nk} d={d} causal={causal} splits={s}", flush=True)
    q, k, v = workloads.make_qkv_shape(B, H, nq, nk, d, nq + 5 * nk + d, DEV)
    o, lse = fa2.attention(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = gu.oracle_full(q, k, v, causal, scale)
    gu.assert_close(o.float().cpu().double().numpy(), lse.cpu().double().numpy(), o_ref, lse_ref,
                    what=f"auto splits={s}", out_grid=True)
