"""Race check of the LDS pipelines: the normal build against the race-check build.

The race-check build (libfa2_poison.so, FA2_POISON_LDS) fills every LDS slot
with a NaN pattern right before its asynchronous buffer->LDS load.  When every
read of a slot is ordered after that load's wait and the barrier that
publishes it, and every load after the barrier that retires the slot's last
reader, the poison is never seen and the outputs are bit-identical to the
normal build's.  A missing wait or barrier shows up as NaN or as a changed
bit.  Each case runs both builds on the same inputs through the C ABI and
compares every output bit for bit, over the paths that stream through LDS:
the 4-wave and 8-wave forward kernels (plain, causal, windowed, ragged), the
split-KV partials, the backward pass (one key block or a group of them per
workgroup) and the FP8 forward.
"""
import pytest
import torch

import exact_attention_85_amd as fa2
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def both(fn):
    """fn() with the normal build, then with the race-check build."""
    a = fn()
    torch.cuda.synchronize()
    with fa2.library_at(fa2.poison_lib_path()):
        b = fn()
        torch.cuda.synchronize()
    return a, b


def same(a, b, what):
    for x, y in zip(a, b):
        assert not torch.isnan(x.float()).any(), f"{what}: NaN in the normal build's output"
        assert torch.equal(x, y), f"{what}: race-check build differs (max |d| {(x.float() - y.float()).abs().max()})"


FWD = [  # B, H, N_q, N_k, d, causal: 4-wave kernel below N_q = 2048 (d = 128), 8-wave from there
    (1, 2, 1000, 1000, 128, 0),
    (1, 2, 1000, 1000, 128, 1),
    (2, 3, 777, 500, 64, 0),
    (2, 3, 777, 777, 64, 1),
    (1, 2, 2100, 2100, 128, 0),
    (1, 1, 8200, 8200, 128, 1),
]


@pytest.mark.parametrize("B,H,nq,nk,d,causal", FWD)
def test_forward(B, H, nq, nk, d, causal):
    print(f"race check fa2_fwd B{B} H{H} N_q{nq} N_k{nk} d{d} causal={causal}", flush=True)
    q, k, v = workloads.make_qkv_shape(B, H, nq, nk, d, 71, DEV)
    a, b = both(lambda: fa2.forward(q, k, v, causal=bool(causal)))
    same(a, b, "forward")


@pytest.mark.parametrize("nq,wl,wr", [(1000, 37, 5), (8200, 300, 40)])
def test_window(nq, wl, wr):
    print(f"race check fa2_fwd_window N{nq} window ({wl}, {wr})", flush=True)
    q, k, v = workloads.make_qkv_shape(1, 2, nq, nq, 128, 72, DEV)
    a, b = both(lambda: fa2.forward_window(q, k, v, wl, wr))
    same(a, b, "window")


def test_splitkv_partials():
    print("race check fa2_fwd_splitkv B2 H2 N_q300 N_k1000 d128 S3", flush=True)
    q, k, v = workloads.make_qkv_shape(2, 2, 300, 1000, 128, 73, DEV)

    def run():
        ws = torch.empty(fa2.splitkv_workspace_bytes(2, 2, 300, 128, 3) // 4, dtype=torch.float32, device=DEV)
        o, lse = fa2.forward_splitkv(q, k, v, num_splits=3, causal=False, workspace=ws)
        return o, lse, ws

    a, b = both(run)
    same(a, b, "split-KV")


# B*H = 2: few workgroups; B*H = 256: many workgroups per compute unit in turn, which refill
# the same LDS buffers; from 2048 rows at d = 128 the dQ pass is the ping-pong kernel
@pytest.mark.parametrize("B,H,nq,d,causal", [(1, 2, 700, 128, 0), (1, 2, 700, 128, 1), (1, 2, 450, 64, 0),
                                             (16, 16, 600, 128, 1), (16, 16, 1000, 64, 0), (2, 2, 2100, 128, 0),
                                             (2, 2, 2100, 128, 1)])
def test_backward(B, H, nq, d, causal):
    print(f"race check fa2_bwd B{B} H{H} N{nq} d{d} causal={causal}", flush=True)
    q, k, v = workloads.make_qkv_shape(B, H, nq, nq, d, 74, DEV)
    do = workloads.make_qkv_shape(B, H, nq, nq, d, 75, DEV)[0]
    o, lse = fa2.forward(q, k, v, causal=bool(causal))
    a, b = both(lambda: fa2.backward(q, k, v, o, lse, do, causal=bool(causal)))
    same(a, b, "backward")


@pytest.mark.parametrize("causal", [0, 1])
def test_fp8_forward(causal):
    print(f"race check fa2_fwd_fp8 B1 H2 N1000 d128 causal={causal}", flush=True)
    q, k, v = workloads.make_qkv_shape(1, 2, 1000, 1000, 128, 76, DEV)
    (qc, sq), (kc, sk), (vt, sv) = fa2.quantize_fp8(q), fa2.quantize_fp8(k), fa2.quantize_fp8(v, transposed=True)
    a, b = both(lambda: fa2.forward_fp8(qc, kc, vt, sq, sk, sv, causal=bool(causal)))
    same(a, b, "FP8 forward")
