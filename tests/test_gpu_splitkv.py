"""GPU parity of fa2_fwd_splitkv (split-KV partials + merge) against the
oracle: the merged result, the per-chunk partials, and equality with the
unsplit forward."""
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


def _partials(ws, S, R, d):
    """acc [S][R][d], then m and l, each [S][R]: the workspace layout of fa2_fwd_splitkv."""
    acc = ws[: S * R * d].view(S, R, d)
    m = ws[S * R * d: S * R * (d + 1)].view(S, R)
    l_ = ws[S * R * (d + 1): S * R * (d + 2)].view(S, R)
    return acc, m, l_


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk,S", [(1, 1, 1), (1, 100, 7), (1, 1000, 16), (1, 5, 4), (3, 200, 5),
                                     (130, 300, 4), (64, 64, 64), (257, 1000, 3)])
def test_splitkv_parity_and_partials(nq, nk, S, causal, d):
    print(f"case splitkv nq={nq} nk={nk} S={S} d={d} causal={causal}", flush=True)
    _check_splitkv(2, 3, nq, nk, S, causal, d, nq * 131 + nk + S)


# thousands of single-query chunks at once: ragged chunk lengths, an empty last
# chunk, and under the causal mask every chunk but the first empty
@pytest.mark.parametrize("B,H,nk,S,d,causal", [(64, 32, 1000, 5, 128, False), (64, 32, 1000, 5, 128, True),
                                               (64, 32, 9, 4, 64, False), (128, 16, 333, 4, 64, False)])
def test_splitkv_decode_many_chunks(B, H, nk, S, d, causal):
    print(f"case splitkv decode many chunks B={B} H={H} nk={nk} S={S} d={d} causal={causal}", flush=True)
    _check_splitkv(B, H, 1, nk, S, causal, d, B * 7 + nk + S)


def _check_splitkv(B, H, nq, nk, S, causal, d, seed):
    scale = 1.0 / math.sqrt(d)
    q, k, v = workloads.make_qkv_shape(B, H, nq, nk, d, seed, DEV)
    R = B * H * nq
    # the workspace is exactly the documented size, with a canary word after it
    ws = torch.full((S * R * (d + 2) + 1,), 12345.0, dtype=torch.float32, device=DEV)
    assert fa2.splitkv_workspace_bytes(B, H, nq, d, S) == S * R * (d + 2) * 4
    o, lse = fa2.forward_splitkv(q, k, v, num_splits=S, causal=causal, scale=scale, workspace=ws)
    torch.cuda.synchronize()
    assert ws[-1].item() == 12345.0
    o_ref, lse_ref = gu.oracle_full(q, k, v, causal, scale)
    gu.assert_close(o.float().cpu().double().numpy(), lse.cpu().double().numpy(), o_ref, lse_ref,
                    what="merged", out_grid=True)
    # per-chunk partials: compare the chunk's normalised output acc / l and its log-sum-exp m + ln l
    acc, m, l_ = (t.cpu().double().numpy() for t in _partials(ws, S, R, d))
    qd, kd, vd = (workloads.bf16_to_f64(t) for t in (q, k, v))
    L = -(-nk // S)
    for c in range(S):
        a_ref, m_ref, l_ref = oracle.partial(qd, kd, vd, causal, scale, min(c * L, nk), min((c + 1) * L, nk))
        a_ref, m_ref, l_ref = a_ref.reshape(R, d), m_ref.reshape(R), l_ref.reshape(R)
        empty = np.isneginf(m_ref)
        assert np.array_equal(np.isneginf(m[c]), empty), c
        assert np.all(l_[c][empty] == 0) and np.all(acc[c][empty] == 0)
        ne = ~empty
        if ne.any():
            o_c = acc[c][ne] / l_[c][ne][:, None]
            o_c_ref = a_ref[ne] / l_ref[ne][:, None]
            assert np.max(np.abs(o_c - o_c_ref)) <= 1e-2, c
            lse_c = m[c][ne] + np.log(l_[c][ne])
            lse_c_ref = m_ref[ne] + np.log(l_ref[ne])
            assert np.max(np.abs(lse_c - lse_c_ref)) <= 1e-3, c


def test_decode_full_size():
    w = workloads.C5
    print(f"case {w.name}", flush=True)
    q, k, v = workloads.make_qkv(w, DEV)
    o, lse = fa2.forward_splitkv(q, k, v, num_splits=w.num_splits, scale=w.scale)
    torch.cuda.synchronize()
    # every one of the 2048 query rows against the oracle
    gu.assert_all_rows(q, k, v, o, lse, False, w.scale, what="decode C5, 16 splits", heads_per_call=w.H)
    # split equals unsplit on every row, within the same tolerance
    o1, l1 = fa2.forward(q, k, v, scale=w.scale)
    torch.cuda.synchronize()
    assert (o1.float() - o.float()).abs().max().item() <= 1e-2
    assert (l1 - lse).abs().max().item() <= 1e-3
    # deterministic
    o2, l2 = fa2.forward_splitkv(q, k, v, num_splits=w.num_splits, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2)


def test_splitkv_matches_fwd_causal_square():
    q, k, v = workloads.make_qkv_shape(2, 4, 500, 500, 128, 21, DEV)
    for S in (2, 5, 16):
        o, lse = fa2.forward_splitkv(q, k, v, num_splits=S, causal=True, scale=0.088)
        o1, l1 = fa2.forward(q, k, v, causal=True, scale=0.088)
        torch.cuda.synchronize()
        assert (o1.float() - o.float()).abs().max().item() <= 1e-2
        assert (l1 - lse).abs().max().item() <= 1e-3
