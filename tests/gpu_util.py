"""Helpers for GPU parity tests: oracle values for chosen rows and the comparison."""
import numpy as np
import torch

import oracle
import workloads

TOL_O = 1e-2     # max |O - O_ref| for bf16 inputs
TOL_LSE = 1e-3   # max |LSE - LSE_ref|


def oracle_rows(q, k, v, rows, causal, scale):
    """Oracle O [n, d] and LSE [n] for rows = [(b, h, i), ...] of (GPU or CPU) bf16 tensors.
    Only the heads the rows touch are copied to the host."""
    d = q.shape[-1]
    o_ref = np.empty((len(rows), d))
    lse_ref = np.empty((len(rows),))
    by_head = {}
    for n, (b, h, i) in enumerate(rows):
        by_head.setdefault((b, h), []).append((n, i))
    for (b, h), items in by_head.items():
        qb = workloads.bf16_bits(q[b, h][None, None])
        kb = workloads.bf16_bits(k[b, h][None, None])
        vb = workloads.bf16_bits(v[b, h][None, None])
        idx = np.array([i for _, i in items], dtype=np.int64)
        o, lse = oracle.attention_rows_bf16(qb, kb, vb, idx, causal, scale)
        for (n, _), orow, lrow in zip(items, o, lse):
            o_ref[n] = orow
            lse_ref[n] = lrow
    return o_ref, lse_ref


def oracle_full(q, k, v, causal, scale):
    """Oracle O, LSE for every row (small shapes)."""
    return oracle.attention(workloads.bf16_to_f64(q), workloads.bf16_to_f64(k), workloads.bf16_to_f64(v),
                            causal, scale)


def gpu_rows(o, lse, rows):
    idx = torch.tensor(rows, dtype=torch.long)
    b, h, i = idx[:, 0], idx[:, 1], idx[:, 2]
    o_rows = o[b.to(o.device), h.to(o.device), i.to(o.device)].float().cpu().double().numpy()
    l_rows = lse[b.to(o.device), h.to(o.device), i.to(o.device)].cpu().double().numpy()
    return o_rows, l_rows


def bf16_half_ulp(x):
    """Half the spacing of the bf16 grid at |x| (8 significant bits): the
    largest error that storing an exact value as bf16 can make."""
    ax = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(ax)) - 8)


def assert_close(o_gpu, lse_gpu, o_ref, lse_ref, tol_o=TOL_O, tol_lse=TOL_LSE, what="", out_grid=False):
    """Element-wise parity; reports the worst element and its reference value.

    out_grid=False: |O - O_ref| <= tol_o everywhere (the named workloads).
    out_grid=True: |O - O_ref| <= tol_o + half a bf16 ulp of O_ref.  Used for
    stress inputs (large scale or sigma) whose outputs reach |O| >= 4, where the
    bf16 output format alone rounds by up to 2^-6 > 1e-2; the compute part of
    the error is still held to tol_o."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    assert o_gpu.shape == o_ref.shape and lse_gpu.shape == lse_ref.shape
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite O"
    assert np.all(np.isfinite(lse_gpu)), f"{what}: non-finite LSE"
    do = np.abs(o_gpu - o_ref)
    dl = np.abs(lse_gpu - lse_ref)
    bound = tol_o + (bf16_half_ulp(o_ref) if out_grid else 0.0)
    excess = do - bound
    io = np.unravel_index(np.argmax(excess), do.shape)
    il = np.unravel_index(np.argmax(dl), dl.shape)
    msg = (f"{what}: max|dO|={do.max():.3e}, worst vs bound {do[io]:.3e} at {io} (ref {o_ref[io]:.4f}, "
           f"bound {np.broadcast_to(bound, do.shape)[io]:.3e}), mean {do.mean():.2e}, over {int((excess > 0).sum())}; "
           f"max|dLSE|={dl[il]:.3e} at {il} (ref {lse_ref[il]:.4f})")
    print(msg, flush=True)
    assert excess[io] <= 0 and dl[il] <= tol_lse, msg
    return float(do.max()), float(dl[il])


def sample_rows(B, H, n_q, n, seed, block=128):
    """Rows (b, h, i): every head's first and last row, rows at query-block
    boundaries, and n random rows."""
    rng = np.random.default_rng(seed)
    rows = set()
    for b in {0, B - 1}:
        for h in {0, H - 1}:
            for i in (0, 1, n_q - 1, block - 1, block, n_q // 2):
                rows.add((b, h, min(i, n_q - 1)))
    while len(rows) < min(n + 24, B * H * n_q):
        rows.add((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(n_q))))
    return sorted(rows)


def bwd_bounds(q, k, v, o, do, causal, scale):
    """Element-wise error bounds for bf16 backward outputs against the fp64
    oracle's gradients, derived from the operand roundings of the GPU path:
    P and dS are rounded to bf16 (relative error <= 2^-9) before their
    products, O reaches D_i = sum dO_i O_i as bf16 (relative <= 2^-9), and the
    outputs are stored as bf16.  With magnitudes
        MV = P^T |dO|,   MK = scale (|dS|^T + P^T |Dabs|) |Q|,   MQ = scale (|dS| + P |Dabs|) |K|,
    (Dabs_i = sum_c |dO_ic O_ic|), each bound is 2^-7 M + 2^-8 |ref| + 1e-6, a
    factor 2 above the first-order sum of those roundings.  Inputs are fp64
    arrays [B, H, N, d]; returns (bound_dq, bound_dk, bound_dv) and needs the
    reference gradients only through |ref|, which the caller adds."""
    p = oracle.probs(q, k, causal, scale)
    dp = np.matmul(do, np.swapaxes(v, -1, -2))
    dsum = np.sum(do * o, axis=-1, keepdims=True)
    ds = np.abs(p * (dp - dsum))
    dabs = np.sum(np.abs(do * o), axis=-1, keepdims=True)
    mv = np.matmul(np.swapaxes(p, -1, -2), np.abs(do))
    mk = scale * np.matmul(np.swapaxes(ds + p * dabs, -1, -2), np.abs(q))
    mq = scale * np.matmul(ds + p * dabs, np.abs(k))
    return 2.0 ** -7 * mq, 2.0 ** -7 * mk, 2.0 ** -7 * mv


def assert_grads_close(got, ref, bounds, what=""):
    for name, g, r, b in zip(("dQ", "dK", "dV"), got, ref, bounds):
        tol = b + 2.0 ** -8 * np.abs(r) + 1e-6
        err = np.abs(g - r)
        bad = err > tol
        if bad.any():
            idx = np.unravel_index(np.argmax(err - tol), err.shape)
            raise AssertionError(f"{what} {name}: {int(bad.sum())} elements out of bound; worst at {idx}: "
                                 f"got {g[idx]:.6g} ref {r[idx]:.6g} err {err[idx]:.3g} tol {tol[idx]:.3g}")
