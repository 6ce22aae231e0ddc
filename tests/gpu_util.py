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


def balanced_order(n):
    """0, n-1, 1, n-2, ...: under the causal mask row i costs i+1 keys, so consecutive pairs cost
    the same and the oracle's static split of the row list over its threads stays even."""
    i = np.arange(n, dtype=np.int64)
    out = np.empty(n, dtype=np.int64)
    out[0::2] = i[: (n + 1) // 2]
    out[1::2] = (n - 1 - i)[: n // 2]
    return out


def assert_all_rows(q, k, v, o, lse, causal, scale, what, heads_per_call=4, tol_o=TOL_O, tol_lse=TOL_LSE,
                    rows_oracle=None):
    """Every row of a GPU result (o [B,H,N_q,d] bf16, lse [B,H,N_q] fp32) against the oracle.

    The oracle runs on the bf16 bits of q, k, v, a few heads per call, so host memory stays
    bounded; each call takes all rows of its heads.  Reports max|dO| and max|dLSE| with their
    (b, h, i, c) locations, the reference value there, the mean error and the count over the
    tolerance, and asserts max|dO| <= tol_o, max|dLSE| <= tol_lse and no NaN.  rows_oracle(qb, kb,
    vb, rows, b) replaces the plain oracle (qb, kb, vb: bf16 bits of batch b, [1, H, N, d]); rows
    whose reference LSE is -inf (no visible key) must have LSE = -inf and O = 0."""
    B, H, n_q, d = q.shape
    worst_o = (-1.0, None, 0.0)
    worst_l = (-1.0, None, 0.0)
    sum_o, n_el, over_o, over_l = 0.0, 0, 0, 0
    order = balanced_order(n_q)
    for b in range(B):
        kb = workloads.bf16_bits(k[b][None])
        vb = workloads.bf16_bits(v[b][None])
        qb = workloads.bf16_bits(q[b][None])
        og = o[b].float().cpu().double().numpy()
        lg = lse[b].cpu().double().numpy()
        for h0 in range(0, H, heads_per_call):
            h1 = min(H, h0 + heads_per_call)
            rows = (np.arange(h0, h1, dtype=np.int64)[:, None] * n_q + order[None, :]).reshape(-1)
            if rows_oracle is None:
                o_ref, l_ref = oracle.attention_rows_bf16(qb, kb, vb, rows, causal, scale)
            else:
                o_ref, l_ref = rows_oracle(qb, kb, vb, rows, b)
            hh, ii = rows // n_q, rows % n_q
            o_g, l_g = og[hh, ii], lg[hh, ii]
            empty = np.isneginf(l_ref)
            if empty.any():
                if not (np.all(np.isneginf(l_g[empty])) and np.all(o_g[empty] == 0)):
                    raise AssertionError(f"{what}: a row with no visible key is not O = 0, LSE = -inf")
                l_ref, l_g = np.where(empty, 0.0, l_ref), np.where(empty, 0.0, l_g)
            if not (np.all(np.isfinite(o_g)) and np.all(np.isfinite(l_g))):
                raise AssertionError(f"{what}: non-finite output in batch {b}, heads {h0}..{h1 - 1}")
            do = np.abs(o_g - o_ref)
            dl = np.abs(l_g - l_ref)
            sum_o += float(do.sum())
            n_el += do.size
            over_o += int((do > tol_o).sum())
            over_l += int((dl > tol_lse).sum())
            r, c = np.unravel_index(np.argmax(do), do.shape)
            if do[r, c] > worst_o[0]:
                worst_o = (float(do[r, c]), (b, int(hh[r]), int(ii[r]), int(c)), float(o_ref[r, c]))
            r = int(np.argmax(dl))
            if dl[r] > worst_l[0]:
                worst_l = (float(dl[r]), (b, int(hh[r]), int(ii[r])), float(l_ref[r]))
    msg = (f"{what}: all {B * H * n_q} rows: max|dO|={worst_o[0]:.3e} at (b,h,i,c)={worst_o[1]} "
           f"(ref {worst_o[2]:.4f}), mean|dO|={sum_o / n_el:.2e}, over {tol_o}: {over_o}; "
           f"max|dLSE|={worst_l[0]:.3e} at (b,h,i)={worst_l[1]} (ref {worst_l[2]:.4f}), over {tol_lse}: {over_l}")
    print(msg, flush=True)
    assert worst_o[0] <= tol_o and worst_l[0] <= tol_lse, msg
    return worst_o[0], worst_l[0]


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


# ---- FP8 forward ----
# Error of the 8-bit matrix product relative to sum |a_k b_k| of its terms, with margin over
# the worst case seen on the hardware (2^-11.7 over random codes of every exponent); the
# probabilities are scaled by 2^7 before rounding to e4m3 (3 mantissa bits: relative error
# 2^-4, subnormal spacing 2^-9 below 2^-6).
FP8_EPS_MMA = 2.0 ** -10
FP8_U = 2.0 ** -4
FP8_PSCALE = 2.0 ** 7


def fp8_head_bounds(qh, kh, vh, rows_i, causal, scale, o_ref, lse_ref):
    """Error bounds for the FP8 forward of one head's rows against the fp64 oracle.

    qh [n, d]: dequantised Q rows (indices rows_i); kh, vh [n_k, d] dequantised K, V; o_ref,
    lse_ref: the oracle's result for those rows.  Returns (bound_o [n, d], var_o [n, d],
    bound_lse [n]):
      * each probability p_j reaches the P.V product with relative error t_j = u_j + 2 E_j:
        u_j from rounding to e4m3 (2^-4, or the subnormal floor) and E_j the score error of
        the 8-bit product; the output row is a convex combination of V rows, so
        |O - O_ref| <= sum_j p_j (t_j + tbar) |v_j - O_ref| / (1 - tbar), tbar = sum_j p_j t_j,
        plus the product error of P.V and of the row sum, and the bf16 output rounding;
      * var_o: the expected squared error if the rounding errors are independent (used by an
        RMS check that a systematic mistake would fail);
      * |LSE - LSE_ref| <= sum_j p_j E_j plus fp32 summation and logarithm rounding."""
    n_k = kh.shape[0]
    s = scale * (qh @ kh.T)
    if causal:
        s = np.where(np.arange(n_k)[None, :] > np.asarray(rows_i)[:, None], -np.inf, s)
    p = np.exp(s - lse_ref[:, None])
    E = FP8_EPS_MMA * abs(scale) * (np.abs(qh) @ np.abs(kh).T) + 2.0 ** -20 * np.abs(np.where(np.isfinite(s), s, 0))
    E = np.where(p > 0, E, 0.0)
    smax = np.max(s, axis=1)
    Z = np.exp(lse_ref - smax - E.max(axis=1))  # lower bound of the kernel's final sum of exp(s - m)
    normal = FP8_PSCALE * p * Z[:, None] >= 2.0 ** -6
    pu = np.where(normal, FP8_U * p, np.minimum(p, 2.0 ** -10 / (FP8_PSCALE * Z[:, None])))
    pt = pu + p * (2 * E + 2.0 ** -20)
    tbar = pt.sum(axis=1)
    assert np.all(tbar < 0.5), "bound derivation assumes small perturbations"
    vabs = np.abs(vh)
    n, d = o_ref.shape
    bound = np.empty((n, d))
    var = np.empty((n, d))
    for r in range(n):
        dev = np.abs(vh - o_ref[r][None, :])
        b1 = (pt[r] + p[r] * tbar[r]) @ dev / (1 - tbar[r])
        b2 = 2.5 * FP8_EPS_MMA * (p[r] @ vabs) / (1 - tbar[r])
        bound[r] = b1 + b2 + 2.0 ** -8 * np.abs(o_ref[r]) + 1e-6 * vabs.max()
        var[r] = (pu[r] ** 2 / 3 + (2 * p[r] * E[r]) ** 2) @ dev ** 2 + (2.0 ** -7 * o_ref[r]) ** 2 / 12
    bound_lse = (p * E).sum(axis=1) + 2.0 ** -20 * (1 + np.abs(lse_ref)) + n_k * 2.0 ** -23
    return bound, var, bound_lse


def assert_fp8_close(o_gpu, lse_gpu, o_ref, lse_ref, bound, var, bound_lse, what=""):
    """Element-wise |O - O_ref| <= bound and |LSE - LSE_ref| <= bound_lse, and the RMS check
    sum (O - O_ref)^2 <= 4 sum var (the expected squared error of independent roundings,
    with margin)."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    assert np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(lse_gpu)), f"{what}: non-finite output"
    err = np.abs(o_gpu - o_ref)
    el = np.abs(lse_gpu - lse_ref)
    ratio = err / bound
    io = np.unravel_index(np.argmax(ratio), err.shape)
    il = int(np.argmax(el / bound_lse))
    rms = float(np.sum(err ** 2) / np.sum(var))
    msg = (f"{what}: max|dO|={err.max():.3e}, worst/bound {ratio[io]:.3f} at {io} (ref {o_ref[io]:.4f}, "
           f"bound {bound[io]:.3e}); mean|dO| {err.mean():.2e}; sum dO^2 / sum var = {rms:.3f}; "
           f"max|dLSE|={el.max():.3e}, worst/bound {el[il] / bound_lse[il]:.3f}")
    print(msg, flush=True)
    assert ratio[io] <= 1 and el[il] <= bound_lse[il] and rms <= 4.0, msg
    return rms
