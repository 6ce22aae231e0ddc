"""Every forward configuration (kernel x workgroup order, fa2_fwd_config) against
the oracle, called through the C ABI; the workgroup order must not change a
single bit of the result; fa2_fwd takes the tuned table's configuration; and
the dispatch-order probe behind the XCD-aware order."""
import math

import numpy as np
import pytest
import torch

import exact_attention_85_amd as fa2
import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
CONFIGS = list(range(fa2.num_configs()))

# (B, H, N_q, N_k, d, window): ragged tails, both head dims, plain, causal and banded, and a
# B*H that is not a multiple of the 8 XCDs
SHAPES = [
    (2, 3, 300, 300, 64, (-1, -1)),
    (2, 3, 300, 300, 64, (-1, 0)),
    (1, 5, 777, 640, 128, (-1, -1)),
    (1, 5, 777, 777, 128, (-1, 0)),
    (2, 4, 1100, 900, 128, (200, 30)),
    (1, 8, 520, 520, 64, (100, 0)),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"B{s[0]}H{s[1]}q{s[2]}k{s[3]}d{s[4]}w{s[5][0]}_{s[5][1]}"
                                                for s in SHAPES])
def test_every_config_against_oracle(shape):
    B, H, nq, nk, d, (wl, wr) = shape
    scale = 1.0 / math.sqrt(d)
    q, k, v = workloads.make_qkv_shape(B, H, nq, nk, d, nq + 7 * nk + d, DEV)
    if (wl, wr) == (-1, -1):
        o_ref, lse_ref = gu.oracle_full(q, k, v, False, scale)
    elif (wl, wr) == (-1, 0):
        o_ref, lse_ref = gu.oracle_full(q, k, v, True, scale)
    else:
        import oracle
        o_ref, lse_ref = oracle.attention_window(*(workloads.bf16_to_f64(t) for t in (q, k, v)), wl, wr, scale)
    by_kernel = {}
    for c in CONFIGS:
        print(f"case config {c} {fa2.config_name(c)} shape {shape}", flush=True)
        o, lse = fa2.forward_config(q, k, v, c, wl, wr, scale=scale)
        torch.cuda.synchronize()
        fin = np.isfinite(lse_ref)
        lg = lse.cpu().double().numpy()
        assert np.array_equal(np.isfinite(lg), fin)
        gu.assert_close(o.float().cpu().double().numpy(), np.where(fin, lg, 0.0), o_ref, np.where(fin, lse_ref, 0.0),
                        what=f"config {fa2.config_name(c)}", out_grid=True)
        # the workgroup order moves work between compute units, never the arithmetic
        kernel = fa2.config_name(c).split("_")[0]
        if kernel in by_kernel:
            o0, l0 = by_kernel[kernel]
            assert torch.equal(o, o0) and torch.equal(lse, l0), fa2.config_name(c)
        else:
            by_kernel[kernel] = (o, lse)


# key lengths of one to four 64-key tiles (and one past): the first and last tiles of a
# kernel's load ring, for query blocks of one and of several waves' rows
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_short_key_ranges_every_config(d, causal):
    scale = 1.0 / math.sqrt(d)
    for nk in (1, 63, 64, 65, 128, 129, 192, 193, 256, 257):
        nq = nk if causal else 300
        q, k, v = workloads.make_qkv_shape(1, 3, nq, nk, d, 5 * nk + d + int(causal), DEV)
        o_ref, lse_ref = gu.oracle_full(q, k, v, causal, scale)
        by_kernel = {}
        for c in CONFIGS:
            print(f"case config {fa2.config_name(c)} d={d} causal={causal} nq={nq} nk={nk}", flush=True)
            o, lse = fa2.forward_config(q, k, v, c, -1, 0 if causal else -1, scale=scale)
            torch.cuda.synchronize()
            gu.assert_close(o.float().cpu().double().numpy(), lse.cpu().double().numpy(), o_ref, lse_ref,
                            what=f"config {fa2.config_name(c)} nk={nk}", out_grid=True)
            kernel = fa2.config_name(c).split("_")[0]
            if kernel in by_kernel:
                assert torch.equal(o, by_kernel[kernel][0]) and torch.equal(lse, by_kernel[kernel][1])
            else:
                by_kernel[kernel] = (o, lse)


def test_named_workload_every_config():
    # the C3 shape (B4 H16 N4096 d128), causal: every configuration on all rows of two heads
    w = workloads.C3
    q, k, v = workloads.make_qkv(w, DEV)
    for c in CONFIGS:
        print(f"case config {fa2.config_name(c)} on {w.name} causal", flush=True)
        o, lse = fa2.forward_config(q, k, v, c, -1, 0, scale=w.scale)
        torch.cuda.synchronize()
        gu.assert_all_rows(q[:1, :2].contiguous(), k[:1, :2].contiguous(), v[:1, :2].contiguous(),
                           o[:1, :2], lse[:1, :2], True, w.scale, what=f"{w.name} {fa2.config_name(c)}")


def test_fwd_takes_the_table_config():
    q, k, v = workloads.make_qkv_shape(1, 4, 2100, 2100, 128, 31, DEV)
    for causal in (False, True):
        c = fa2.default_config(128, causal, 2100, 1, 4)
        o1, l1 = fa2.forward(q, k, v, causal=causal)
        o2, l2 = fa2.forward_config(q, k, v, c, -1, 0 if causal else -1)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_dispatch_order_probe():
    # workgroup -> XCD as the hardware deals them.  The XCD-aware order needs the ids of one
    # residue class mod 8 to share an XCD: id i on XCD (i + o) mod 8 for some offset o
    n = 4096
    for _ in range(3):
        xcd, hw = fa2.probe_xcc(n)
        xcd = xcd.numpy()
        assert xcd.min() >= 0 and xcd.max() <= 7 and len(set(xcd.tolist())) == 8
        off = np.bincount((xcd - np.arange(n)) % 8, minlength=8)
        o = int(np.argmax(off))
        print(f"dispatch order: {100 * off[o] / n:.1f} % of {n} workgroups ran on XCD (id + {o}) mod 8; "
              f"per-XCD counts {np.bincount(xcd, minlength=8).tolist()}", flush=True)
        assert np.bincount(xcd, minlength=8).min() >= n // 16  # every XCD takes a share
