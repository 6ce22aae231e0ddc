"""GPU parity at the size limits of the boundary.

* One head holding the largest K and V the API accepts (N_k * d = 2^30 - 1
  elements, byte offsets up to just under 2^31), through the tile kernel
  (N_q = 130), the single-row decode kernel (N_q = 1, fa2_fwd) and the split
  path (fa2_fwd_splitkv).  Random inputs over millions of keys give outputs
  near zero, which would hide a wrong far-key read, so each checked row gets
  one planted key (a scaled copy of its own query) that carries almost all of
  its weight; the planted positions include the last key and the key at byte
  offset 2^30.  The reference is the oracle's split into key chunks (partial
  and merge), which holds fp64 copies of one chunk of K and V at a time.
* A long sequence, N_q = N_k = 131072 at d = 128, through the 8-wave kernel:
  non-causal, causal and a sliding window, on sampled rows.
"""
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
MAX_HEAD_ELEMS = (1 << 30) - 1  # the per-head limit fa2_fwd validates
CHUNK = 1 << 20                 # keys per oracle partial


def chunked_reference(q_rows, k, v, scale):
    """Non-causal O [R, d] and LSE [R] of fp64 query rows q_rows [R, d] against every key
    of one head (k, v: [N_k, d] bf16 on the GPU), as merged oracle partials over key chunks."""
    n_k = k.shape[0]
    accs, ms, ls = [], [], []
    for c0 in range(0, n_k, CHUNK):
        c1 = min(n_k, c0 + CHUNK)
        kc = workloads.bf16_to_f64(k[c0:c1])[None, None]
        vc = workloads.bf16_to_f64(v[c0:c1])[None, None]
        acc, m, l_ = oracle.partial(q_rows[None, None], kc, vc, False, scale, 0, c1 - c0)
        accs.append(acc[0, 0])
        ms.append(m[0, 0])
        ls.append(l_[0, 0])
    return oracle.merge(np.stack(accs), np.stack(ms), np.stack(ls))


@pytest.mark.parametrize("d", [64, 128])
def test_largest_head(d):
    n_k = MAX_HEAD_ELEMS // d
    n_q = 130
    scale = 1.0 / math.sqrt(d)
    print(f"case largest head n_q={n_q} n_k={n_k} d={d}", flush=True)
    q, k, v = workloads.make_qkv_shape(1, 1, n_q, n_k, d, 97 + d, DEV)
    rows = [0, 1, 63, 64, 127, 128, 129]
    planted = [n_k - 1, (1 << 29) // d, n_k - 64, 12345, n_k // 2 + 17, n_k - 65, 0]
    for r, j in zip(rows, planted):
        k[0, 0, j] = (q[0, 0, r].float() * 8.0).to(torch.bfloat16)
    o_ref, lse_ref = chunked_reference(workloads.bf16_to_f64(q[0, 0, rows]), k[0, 0], v[0, 0], scale)
    # the planted key dominates each row, so O is close to that key's V row
    v_planted = workloads.bf16_to_f64(v[0, 0, planted])
    assert np.max(np.abs(o_ref - v_planted)) < 1e-3

    o, lse = fa2.forward(q, k, v, causal=False, scale=scale)
    torch.cuda.synchronize()
    og = o[0, 0, rows].float().cpu().double().numpy()
    lg = lse[0, 0, rows].cpu().double().numpy()
    gu.assert_close(og, lg, o_ref, lse_ref, what=f"largest head, tile kernel, d={d}")

    # row 0 alone: the streaming decode kernel, directly and split in 16 chunks
    q0 = q[:, :, :1].contiguous()
    o1, l1 = fa2.forward(q0, k, v, causal=False, scale=scale)
    o2, l2 = fa2.forward_splitkv(q0, k, v, num_splits=16, causal=False, scale=scale)
    torch.cuda.synchronize()
    for oo, ll, what in ((o1, l1, "decode"), (o2, l2, "split 16")):
        gu.assert_close(oo[0, 0].float().cpu().double().numpy(), ll[0, 0].cpu().double().numpy(),
                        o_ref[:1], lse_ref[:1], what=f"largest head, {what}, d={d}")


@pytest.mark.parametrize("mode", ["plain", "causal", "window"])
def test_long_sequence_pingpong(mode):
    n = 131072
    d = 128
    scale = 1.0 / math.sqrt(d)
    print(f"case long sequence n={n} d={d} {mode}", flush=True)
    q, k, v = workloads.make_qkv_shape(1, 2, n, n, d, 131 + len(mode), DEV)
    wl, wr = (4095, 0) if mode == "window" else (-1, 0 if mode == "causal" else -1)
    if mode == "window":
        o, lse = fa2.forward_window(q, k, v, wl, wr, scale=scale)
    else:
        o, lse = fa2.forward(q, k, v, causal=mode == "causal", scale=scale)
    torch.cuda.synchronize()
    rows = gu.sample_rows(1, 2, n, 40, seed=n + len(mode), block=256)
    og, lg = gu.gpu_rows(o, lse, rows)
    if mode == "window":
        o_ref, lse_ref = np.empty_like(og), np.empty_like(lg)
        for h in range(2):
            sel = [i for i, r in enumerate(rows) if r[1] == h]
            idx = np.array([rows[i][2] for i in sel], dtype=np.int64)
            a, b = oracle.attention_window_rows_bf16(
                workloads.bf16_bits(q[0, h][None, None]), workloads.bf16_bits(k[0, h][None, None]),
                workloads.bf16_bits(v[0, h][None, None]), idx, wl, wr, scale)
            o_ref[sel], lse_ref[sel] = a, b
    else:
        o_ref, lse_ref = gu.oracle_rows(q, k, v, rows, mode == "causal", scale)
    gu.assert_close(og, lg, o_ref, lse_ref, what=f"long sequence {mode}")
