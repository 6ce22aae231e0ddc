"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function takes an oracle module (the real one, or a mutated
copy built by the mutation test) and raises AssertionError when the oracle
disagrees with:

  P1  brute force at 50 significant digits (mpmath), without the max shift;
  P2  rows of P summing to 1 and P vanishing where masked;
  P3  constant V returning that constant;
  P4  causal row 0 returning v_0 with LSE = s_00;
  P5  Q = 0: O = mean of the allowed values, LSE = ln(#allowed);
  P6  one-hot scores: a closed form in e^a;
  P7  LSE = ln sum exp(s) (exact summation) and max s <= LSE <= max s + ln n;
  P8  torch's fp64 CPU scaled_dot_product_attention (a library special case);
  P9  invariants: joint key/value permutation, query permutation, linearity
      in V, and split-then-merge equal to the unsplit result;
  P10 a float64 transcription of the pages' tiled online recurrence
      (FlashAttention-2 walkthrough page, main-loop pseudocode) with random
      tile sizes.

Sliding-window pins (the synthesis page, section 5 item 4), for key j visible
to query i iff j < N_k, j >= i - wl (wl >= 0) and j <= i + wr (wr >= 0):

  P11 brute force at 50 digits over the band, empty rows O = 0, LSE = -inf;
  P12 special windows: (-1, -1) is plain attention, (-1, 0) the causal mask,
      (0, 0) returns v_i with LSE = s_ii, and a window wider than the
      sequence changes nothing;
  P13 torch's fp64 CPU scaled_dot_product_attention with the band written
      out as a boolean mask, and the visible-pair count against that mask;
  P14 the tiled online recurrence of P10 with the band mask applied per tile.

Backward pins (gradients of exact attention for an upstream gradient dO):

  P15 central finite differences of L = sum(dO * O(Q, K, V)) through the
      pinned forward oracle, for every element of Q, K and V on tiny shapes;
  P16 torch's fp64 CPU autograd through scaled_dot_product_attention;
  P17 identities: sum_j dK_j = 0 (softmax is invariant to a shift of all
      keys' scores of a row), sum_j dV_j = sum_i dO_i (rows of P sum to 1),
      dV linear in dO, and all gradients zero for dO = 0.

The definition pinned is exact attention with top-left causal masking
(key j allowed for query i iff j <= i), scale applied to q.k before the
softmax, and LSE the natural log of sum exp of the scaled, masked scores.

FP8 pins (OCP e4m3fn codes with per-(batch, head) scaling; the improvements
page, section 四 point ③, asks for scaling without giving a recipe):

  P18 the decode table against torch's float8_e4m3fn and the format's
      published landmarks (1.0, largest finite 448, smallest normal 2^-6,
      smallest subnormal 2^-9), monotone over the positive codes;
  P19 the round-to-nearest-even encoder: every finite code round-trips,
      midpoints go to the even code and one fp32 step either side to the
      nearer code, and random values agree with torch's cast;
  P20 the quantiser: the slice's amax maps to +-448, every dequantised value
      lies within half a code step of its input, an all-zero slice gets
      descale 1, and the codes equal torch's cast of fp32(x) * fp32(448/amax);
  P21 attention on FP8 inputs: with power-of-two descales the dequantised
      values are bf16 numbers, and the result equals the pinned bf16 row
      oracle on them; the row function equals the full composition for
      arbitrary descales; O scales with descale_v and the scores with
      descale_q * descale_k.

Block-sparse pins (the synthesis page, section 5 item 4: one block-skip mechanism for windows
and dilated patterns), for key j visible to query i of (b, h) iff M[b][h][i // bq][j // bk] != 0
and the band admits it:

  P22 brute force at 50 digits, without the max shift, over random masks (shared or per batch
      and head), block sizes and bands; rows that see no key give O = 0, LSE = -inf;
  P23 an all-ones mask is the pinned window oracle (and so plain and causal attention);
  P24 torch's fp64 CPU scaled_dot_product_attention with the mask expanded to keys and
      queries by repetition, and the visible-pair count against that expansion;
  P25 with no band, the rows of a query block equal plain attention over the keys of its
      visible key blocks only (the others deleted), and a mask shared over heads equals its
      per-head copy.
"""
import math

import mpmath
import numpy as np
import torch

RNG = np.random.default_rng


def _allowed(i, n_k, causal):
    return min(i + 1, n_k) if causal else n_k


def pin_p1_bruteforce(orc):
    mpmath.mp.dps = 50
    rng = RNG(101)
    cases = [(1, 2, 5, 7, 3, False), (1, 2, 5, 7, 3, True), (2, 1, 8, 4, 4, True), (1, 1, 6, 6, 2, True),
             (1, 1, 1, 8, 4, False), (1, 1, 8, 1, 4, True)]
    for B, H, n_q, n_k, d, causal in cases:
        q = rng.normal(size=(B, H, n_q, d)) * 1.5
        k = rng.normal(size=(B, H, n_k, d)) * 1.5
        v = rng.normal(size=(B, H, n_k, d))
        scale = 0.7
        o, lse = orc.attention(q, k, v, causal, scale)
        for b in range(B):
            for h in range(H):
                for i in range(n_q):
                    n = _allowed(i, n_k, causal)
                    ex = []
                    for j in range(n):
                        s = mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[b, h, i, c]) * mpmath.mpf(k[b, h, j, c])
                                                            for c in range(d))
                        ex.append(mpmath.e ** s)
                    z = mpmath.fsum(ex)
                    for c in range(d):
                        ref = mpmath.fsum(ex[j] * mpmath.mpf(v[b, h, j, c]) for j in range(n)) / z
                        assert abs(float(ref) - o[b, h, i, c]) <= 1e-13 * (1 + abs(float(ref))), (b, h, i, c)
                    ref_lse = mpmath.log(z)
                    assert abs(float(ref_lse) - lse[b, h, i]) <= 1e-13 * (1 + abs(float(ref_lse))), (b, h, i)


def pin_p2_rows_sum_to_one(orc):
    rng = RNG(202)
    for causal in (False, True):
        q = rng.normal(size=(2, 3, 9, 5)) * 2
        k = rng.normal(size=(2, 3, 11, 5)) * 2
        p = orc.probs(q, k, causal, 0.9)
        assert np.all(p >= 0)
        assert np.max(np.abs(p.sum(-1) - 1.0)) <= 1e-14
        if causal:
            for i in range(9):
                assert np.all(p[:, :, i, i + 1:] == 0.0)
        # P agrees with the O the oracle returns: O = P V
        v = rng.normal(size=(2, 3, 11, 5))
        o, _ = orc.attention(q, k, v, causal, 0.9)
        assert np.max(np.abs(np.einsum("bhij,bhjc->bhic", p, v) - o)) <= 1e-13


def pin_p3_constant_v(orc):
    rng = RNG(303)
    for causal in (False, True):
        q = rng.normal(size=(1, 2, 13, 8)) * 3
        k = rng.normal(size=(1, 2, 17, 8)) * 3
        c = rng.normal(size=(8,))
        v = np.broadcast_to(c, (1, 2, 17, 8)).copy()
        o, _ = orc.attention(q, k, v, causal, 0.5)
        assert np.max(np.abs(o - c)) <= 1e-14 * (1 + np.max(np.abs(c)))


def pin_p4_causal_row0(orc):
    rng = RNG(404)
    q = rng.normal(size=(2, 2, 6, 4))
    k = rng.normal(size=(2, 2, 9, 4))
    v = rng.normal(size=(2, 2, 9, 4))
    scale = 1.3
    o, lse = orc.attention(q, k, v, True, scale)
    assert np.max(np.abs(o[:, :, 0, :] - v[:, :, 0, :])) <= 1e-15
    s00 = scale * np.sum(q[:, :, 0, :] * k[:, :, 0, :], axis=-1)
    assert np.max(np.abs(lse[:, :, 0] - s00)) <= 1e-14


def pin_p5_uniform_scores(orc):
    rng = RNG(505)
    n_q, n_k, d = 10, 7, 6
    q = np.zeros((1, 2, n_q, d))
    k = rng.normal(size=(1, 2, n_k, d))
    v = rng.normal(size=(1, 2, n_k, d))
    for causal in (False, True):
        o, lse = orc.attention(q, k, v, causal, 0.8)
        for i in range(n_q):
            n = _allowed(i, n_k, causal)
            assert np.max(np.abs(o[:, :, i, :] - v[:, :, :n, :].mean(axis=2))) <= 1e-14
            assert np.max(np.abs(lse[:, :, i] - math.log(n))) <= 1e-14


def pin_p6_one_hot(orc):
    # q_i = k_i = c e_i (N <= d) so s_ij = a * delta_ij with a = scale * c^2.
    n, d, c, scale = 6, 8, 4.0, 0.125   # a = 2
    a = scale * c * c
    q = np.zeros((1, 1, n, d))
    for i in range(n):
        q[0, 0, i, i] = c
    k = q.copy()
    v = RNG(606).normal(size=(1, 1, n, d))
    for causal in (False, True):
        o, lse = orc.attention(q, k, v, causal, scale)
        for i in range(n):
            na = i + 1 if causal else n
            z = math.exp(a) + (na - 1)
            ref = (math.exp(a) * v[0, 0, i] + (v[0, 0, :na].sum(axis=0) - v[0, 0, i])) / z
            assert np.max(np.abs(o[0, 0, i] - ref)) <= 1e-14
            assert abs(lse[0, 0, i] - math.log(z)) <= 1e-14


def pin_p7_lse_identity(orc):
    rng = RNG(707)
    n_q, n_k, d = 7, 12, 5
    q = rng.normal(size=(1, 1, n_q, d)) * 4
    k = rng.normal(size=(1, 1, n_k, d)) * 4
    v = rng.normal(size=(1, 1, n_k, d))
    scale = 0.6
    for causal in (False, True):
        _, lse = orc.attention(q, k, v, causal, scale)
        for i in range(n_q):
            n = _allowed(i, n_k, causal)
            s = [scale * math.fsum(q[0, 0, i, c] * k[0, 0, j, c] for c in range(d)) for j in range(n)]
            smax = max(s)
            ref = smax + math.log(math.fsum(math.exp(x - smax) for x in s))
            assert abs(lse[0, 0, i] - ref) <= 1e-13 * (1 + abs(ref))
            assert smax - 1e-13 <= lse[0, 0, i] <= smax + math.log(n) + 1e-13


def pin_p8_torch_sdpa(orc):
    rng = RNG(808)
    for (n_q, n_k, d, causal) in [(33, 33, 16, False), (33, 33, 16, True), (20, 45, 8, True), (45, 20, 8, True),
                                  (64, 70, 32, False)]:
        q = rng.normal(size=(2, 3, n_q, d))
        k = rng.normal(size=(2, 3, n_k, d))
        v = rng.normal(size=(2, 3, n_k, d))
        scale = 1.0 / math.sqrt(d)
        o, lse = orc.attention(q, k, v, causal, scale)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        if causal:
            # top-left alignment written out: key j visible to query i iff j <= i
            mask = torch.ones(n_q, n_k, dtype=torch.bool).tril()
            ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
        else:
            ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
        assert np.max(np.abs(ref.numpy() - o)) <= 1e-12
        scores = torch.matmul(tq, tk.transpose(-1, -2)) * scale
        if causal:
            scores = scores.masked_fill(~mask, float("-inf"))
        assert np.max(np.abs(torch.logsumexp(scores, dim=-1).numpy() - lse)) <= 1e-12


def pin_p9_invariants(orc):
    rng = RNG(909)
    n_q, n_k, d = 14, 19, 6
    q = rng.normal(size=(1, 2, n_q, d))
    k = rng.normal(size=(1, 2, n_k, d))
    v = rng.normal(size=(1, 2, n_k, d))
    v2 = rng.normal(size=(1, 2, n_k, d))
    scale = 0.45
    o, lse = orc.attention(q, k, v, False, scale)
    # joint key/value permutation (non-causal) changes nothing
    perm = rng.permutation(n_k)
    o_p, lse_p = orc.attention(q, k[:, :, perm], v[:, :, perm], False, scale)
    assert np.max(np.abs(o_p - o)) <= 1e-13 and np.max(np.abs(lse_p - lse)) <= 1e-13
    # query permutation permutes output rows
    qp = rng.permutation(n_q)
    o_q, lse_q = orc.attention(q[:, :, qp], k, v, False, scale)
    assert np.max(np.abs(o_q - o[:, :, qp])) <= 1e-13 and np.max(np.abs(lse_q - lse[:, :, qp])) <= 1e-13
    # linear in V
    for causal in (False, True):
        oa, _ = orc.attention(q, k, v, causal, scale)
        ob, _ = orc.attention(q, k, v2, causal, scale)
        oc, _ = orc.attention(q, k, 2.0 * v - 3.0 * v2, causal, scale)
        assert np.max(np.abs(oc - (2.0 * oa - 3.0 * ob))) <= 1e-12
    # split the keys into chunks, merge the partials: equals the unsplit result
    for causal in (False, True):
        o_full, lse_full = orc.attention(q, k, v, causal, scale)
        for n_splits in (1, 2, 3, 7, n_k):
            L = -(-n_k // n_splits)
            parts = [orc.partial(q, k, v, causal, scale, c * L, min((c + 1) * L, n_k)) for c in range(n_splits)]
            acc = np.stack([p[0] for p in parts])
            m = np.stack([p[1] for p in parts])
            l_ = np.stack([p[2] for p in parts])
            o_m, lse_m = orc.merge(acc, m, l_)
            assert np.max(np.abs(o_m - o_full)) <= 1e-13, (causal, n_splits)
            assert np.max(np.abs(lse_m - lse_full)) <= 1e-13, (causal, n_splits)
        # an empty chunk is (acc 0, m -inf, l 0)
        acc, m, l_ = orc.partial(q, k, v, True, scale, n_k, n_k)
        assert np.all(acc == 0) and np.all(np.isneginf(m)) and np.all(l_ == 0)
    # row-selected bf16 entry point equals the full one on bf16-exact values
    qb = torch.from_numpy(q).to(torch.bfloat16)
    kb = torch.from_numpy(k).to(torch.bfloat16)
    vb = torch.from_numpy(v).to(torch.bfloat16)
    bits = [t.contiguous().view(torch.int16).numpy().view(np.uint16) for t in (qb, kb, vb)]
    vals = [t.to(torch.float64).numpy() for t in (qb, kb, vb)]
    assert np.array_equal(orc.bf16_bits_to_f64(bits[0]), vals[0])
    for causal in (False, True):
        o_full, lse_full = orc.attention(*vals, causal, scale)
        rows = np.array([0, 5, n_q - 1, n_q, 2 * n_q - 1], dtype=np.int64)
        o_r, lse_r = orc.attention_rows_bf16(*bits, rows, causal, scale)
        assert np.array_equal(o_r, o_full.reshape(-1, d)[rows])
        assert np.array_equal(lse_r, lse_full.reshape(-1)[rows])


def _block_state(s, vb):
    """Softmax state (m, l, a) of one block of scores s [rows, keys] (-inf where not visible)
    and its values vb [keys, d]: m = row maximum, l = sum exp(s - m), a = sum exp(s - m) v.
    A row with no visible key is the empty state (-inf, 0, 0)."""
    m = s.max(axis=1)
    shift = np.where(np.isneginf(m), 0.0, m)
    e = np.exp(s - shift[:, None])
    return m, e.sum(axis=1), e @ vb


def _combine(x, y):
    """The associative combination of two softmax states over disjoint key sets: both are
    brought to the larger maximum.  The empty state is its identity."""
    (m1, l1, a1), (m2, l2, a2) = x, y
    m = np.maximum(m1, m2)
    shift = np.where(np.isneginf(m), 0.0, m)
    w1, w2 = np.exp(m1 - shift), np.exp(m2 - shift)
    return m, w1 * l1 + w2 * l2, w1[:, None] * a1 + w2[:, None] * a2


def blockwise_model(q, k, v, visible, scale, block_r, block_c):
    """Attention assembled from tiles, the decomposition the kernels rely on (FlashAttention-2
    walkthrough page, kernel main loop section: per query block, key/value blocks are folded into a
    running maximum, sum and accumulator, and O and the log-sum-exp come out at the end).  Here
    every (query block, key block) tile yields its own state, and the states of a query block are
    combined pairwise as a balanced tree rather than left to right, so the check rests on the
    associativity of the combination rather than on one order of it.  visible(rows, cols) is the
    boolean mask of a tile.  Rows that see no key get O = 0 and LSE = -inf."""
    B, H, n_q, d = q.shape
    n_k = k.shape[2]
    o = np.zeros((B, H, n_q, d))
    lse = np.zeros((B, H, n_q))
    for b in range(B):
        for h in range(H):
            for r0 in range(0, n_q, block_r):
                r1 = min(r0 + block_r, n_q)
                rows = np.arange(r0, r1)[:, None]
                states = []
                for c0 in range(0, n_k, block_c):
                    c1 = min(c0 + block_c, n_k)
                    s = scale * (q[b, h, r0:r1] @ k[b, h, c0:c1].T)
                    s = np.where(visible(rows, np.arange(c0, c1)[None, :]), s, -np.inf)
                    states.append(_block_state(s, v[b, h, c0:c1]))
                while len(states) > 1:
                    states = [_combine(states[i], states[i + 1]) if i + 1 < len(states) else states[i]
                              for i in range(0, len(states), 2)]
                m, l_, a = states[0]
                seen = l_ > 0
                o[b, h, r0:r1] = np.where(seen[:, None], a / np.where(seen, l_, 1.0)[:, None], 0.0)
                lse[b, h, r0:r1] = np.where(seen, m + np.log(np.where(seen, l_, 1.0)), -np.inf)
    return o, lse


def recurrence_model(q, k, v, causal, scale, block_r, block_c):
    """blockwise_model under the causal (top-left) mask, or none."""
    return blockwise_model(q, k, v, (lambda r, c: c <= r) if causal else (lambda r, c: np.ones(
        np.broadcast_shapes(r.shape, c.shape), dtype=bool)), scale, block_r, block_c)


def pin_p10_recurrence(orc):
    rng = RNG(1010)
    for causal in (False, True):
        q = rng.normal(size=(1, 2, 37, 8))
        k = rng.normal(size=(1, 2, 37, 8))
        v = rng.normal(size=(1, 2, 37, 8))
        o, lse = orc.attention(q, k, v, causal, 0.35)
        for block_r, block_c in [(1, 1), (4, 7), (16, 5), (37, 37), (64, 64)]:
            o_r, lse_r = recurrence_model(q, k, v, causal, 0.35, block_r, block_c)
            assert np.max(np.abs(o_r - o)) <= 1e-12
            assert np.max(np.abs(lse_r - lse)) <= 1e-12


def _band(i, n_k, wl, wr):
    lo = max(0, i - wl) if wl >= 0 else 0
    hi = min(n_k, i + wr + 1) if wr >= 0 else n_k
    return lo, max(lo, hi)


def pin_p11_window_bruteforce(orc):
    mpmath.mp.dps = 50
    rng = RNG(1111)
    for (n_q, n_k, d, wl, wr) in [(6, 6, 3, 1, 0), (7, 5, 2, 2, 1), (5, 8, 3, 0, 2), (8, 4, 2, 1, -1),
                                  (4, 9, 3, -1, 3), (9, 3, 2, 0, 0)]:
        q = rng.normal(size=(1, 1, n_q, d)) * 1.5
        k = rng.normal(size=(1, 1, n_k, d)) * 1.5
        v = rng.normal(size=(1, 1, n_k, d))
        scale = 0.8
        o, lse = orc.attention_window(q, k, v, wl, wr, scale)
        for i in range(n_q):
            lo, hi = _band(i, n_k, wl, wr)
            if hi == lo:
                assert np.all(o[0, 0, i] == 0) and np.isneginf(lse[0, 0, i]), (i, wl, wr)
                continue
            ex = []
            for j in range(lo, hi):
                s_ = mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[0, 0, i, c]) * mpmath.mpf(k[0, 0, j, c])
                                                     for c in range(d))
                ex.append(mpmath.e ** s_)
            z = mpmath.fsum(ex)
            for c in range(d):
                ref = mpmath.fsum(ex[j - lo] * mpmath.mpf(v[0, 0, j, c]) for j in range(lo, hi)) / z
                assert abs(o[0, 0, i, c] - float(ref)) <= 1e-13 * (1 + abs(float(ref))), (i, c, wl, wr)
            assert abs(lse[0, 0, i] - float(mpmath.log(z))) <= 1e-13 * (1 + abs(float(mpmath.log(z))))


def pin_p12_window_special(orc):
    rng = RNG(1212)
    q = rng.normal(size=(2, 2, 23, 5))
    k = rng.normal(size=(2, 2, 19, 5))
    v = rng.normal(size=(2, 2, 19, 5))
    for causal, (wl, wr) in ((False, (-1, -1)), (True, (-1, 0))):
        o_ref, lse_ref = orc.attention(q, k, v, causal, 0.6)
        o, lse = orc.attention_window(q, k, v, wl, wr, 0.6)
        assert np.array_equal(o, o_ref) and np.array_equal(lse, lse_ref)
    o_ref, lse_ref = orc.attention(q, k, v, False, 0.6)
    o, lse = orc.attention_window(q, k, v, 40, 40, 0.6)
    assert np.array_equal(o, o_ref) and np.array_equal(lse, lse_ref)
    o, lse = orc.attention_window(q, k, v, 0, 0, 0.6)
    n = 19
    assert np.array_equal(o[:, :, :n], v)
    s_ii = 0.6 * np.einsum("bhid,bhid->bhi", q[:, :, :n], k)
    assert np.max(np.abs(lse[:, :, :n] - s_ii)) <= 1e-14
    assert np.all(o[:, :, n:] == 0) and np.all(np.isneginf(lse[:, :, n:]))
    # the row-selected bf16 entry point equals the full one on bf16-exact values
    tb = [torch.from_numpy(x).to(torch.bfloat16) for x in (q, k, v)]
    bits = [t.contiguous().view(torch.int16).numpy().view(np.uint16) for t in tb]
    vals = [t.to(torch.float64).numpy() for t in tb]
    rows = np.array([0, 7, 22, 23, 60, 91], dtype=np.int64)
    for wl, wr in ((4, 0), (2, 3), (0, 0)):
        o_full, lse_full = orc.attention_window(*vals, wl, wr, 0.6)
        o_r, lse_r = orc.attention_window_rows_bf16(*bits, rows, wl, wr, 0.6)
        assert np.array_equal(o_r, o_full.reshape(-1, 5)[rows])
        assert np.array_equal(lse_r, lse_full.reshape(-1)[rows])


def pin_p13_window_torch(orc):
    rng = RNG(1313)
    for (n_q, n_k, d, wl, wr) in [(40, 40, 8, 7, 0), (40, 40, 8, 5, 3), (33, 50, 16, 10, -1), (50, 33, 16, -1, 4),
                                  (31, 31, 8, 0, 6)]:
        q = rng.normal(size=(2, 2, n_q, d))
        k = rng.normal(size=(2, 2, n_k, d))
        v = rng.normal(size=(2, 2, n_k, d))
        scale = 1.0 / math.sqrt(d)
        o, lse = orc.attention_window(q, k, v, wl, wr, scale)
        ii = torch.arange(n_q)[:, None]
        jj = torch.arange(n_k)[None, :]
        mask = torch.ones(n_q, n_k, dtype=torch.bool)
        if wl >= 0:
            mask &= jj >= ii - wl
        if wr >= 0:
            mask &= jj <= ii + wr
        assert orc.window_pairs(n_q, n_k, wl, wr) == int(mask.sum())
        rows = mask.any(dim=1).numpy()
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale).numpy()
        assert np.max(np.abs(ref[:, :, rows] - o[:, :, rows])) <= 1e-12
        scores = (torch.matmul(tq, tk.transpose(-1, -2)) * scale).masked_fill(~mask, float("-inf"))
        lse_ref = torch.logsumexp(scores, dim=-1).numpy()
        assert np.max(np.abs(lse_ref[:, :, rows] - lse[:, :, rows])) <= 1e-12
        assert np.all(np.isneginf(lse[:, :, ~rows])) and np.all(o[:, :, ~rows] == 0)


def window_recurrence_model(q, k, v, wl, wr, scale, block_r, block_c):
    """blockwise_model under the band mask: key j visible to query i iff (wl < 0 or j >= i - wl)
    and (wr < 0 or j <= i + wr)."""
    def visible(r, c):
        vis = np.ones(np.broadcast_shapes(r.shape, c.shape), dtype=bool)
        if wl >= 0:
            vis &= c >= r - wl
        if wr >= 0:
            vis &= c <= r + wr
        return vis
    return blockwise_model(q, k, v, visible, scale, block_r, block_c)


def pin_p14_window_recurrence(orc):
    rng = RNG(1414)
    q = rng.normal(size=(1, 2, 41, 8))
    k = rng.normal(size=(1, 2, 37, 8))
    v = rng.normal(size=(1, 2, 37, 8))
    for wl, wr in [(9, 0), (3, 5), (0, 0), (-1, 2), (12, -1)]:
        o, lse = orc.attention_window(q, k, v, wl, wr, 0.35)
        for block_r, block_c in [(1, 1), (4, 7), (16, 5), (64, 64)]:
            o_r, lse_r = window_recurrence_model(q, k, v, wl, wr, 0.35, block_r, block_c)
            assert np.max(np.abs(o_r - o)) <= 1e-12
            fin = np.isfinite(lse)
            assert np.array_equal(fin, np.isfinite(lse_r))
            assert np.max(np.abs(lse_r[fin] - lse[fin])) <= 1e-12


def pin_p15_backward_finite_differences(orc):
    rng = RNG(1515)
    for (n_q, n_k, d, causal) in [(4, 5, 3, False), (5, 5, 3, True), (3, 6, 2, True)]:
        q = rng.normal(size=(1, 1, n_q, d))
        k = rng.normal(size=(1, 1, n_k, d))
        v = rng.normal(size=(1, 1, n_k, d))
        do = rng.normal(size=(1, 1, n_q, d))
        scale = 0.7
        dq, dk, dv = orc.backward(q, k, v, do, causal, scale)

        def loss(qq, kk, vv):
            o, _ = orc.attention(qq, kk, vv, causal, scale)
            return float(np.sum(do * o))

        h = 1e-6
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = [xp if name == n else a for n, a in (("q", q), ("k", k), ("v", v))]
                args_m = [xm if name == n else a for n, a in (("q", q), ("k", k), ("v", v))]
                fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
                assert abs(fd - g[idx]) <= 1e-7 * (1 + abs(fd)), (name, idx, causal, fd, g[idx])


def pin_p16_backward_torch(orc):
    rng = RNG(1616)
    for (n_q, n_k, d, causal) in [(21, 21, 8, False), (21, 21, 8, True), (13, 30, 16, True), (30, 13, 16, True),
                                  (17, 40, 8, False)]:
        q, k, v = (rng.normal(size=(2, 2, n, d)) for n in (n_q, n_k, n_k))
        do = rng.normal(size=(2, 2, n_q, d))
        scale = 1.0 / math.sqrt(d)
        dq, dk, dv = orc.backward(q, k, v, do, causal, scale)
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        mask = torch.ones(n_q, n_k, dtype=torch.bool).tril() if causal else None
        o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
        o.backward(torch.from_numpy(do))
        for ref, got in ((tq.grad, dq), (tk.grad, dk), (tv.grad, dv)):
            assert np.max(np.abs(ref.numpy() - got)) <= 1e-12


def pin_p17_backward_identities(orc):
    rng = RNG(1717)
    q, k, v = (rng.normal(size=(1, 2, n, 6)) for n in (11, 14, 14))
    do = rng.normal(size=(1, 2, 11, 6))
    do2 = rng.normal(size=(1, 2, 11, 6))
    for causal in (False, True):
        dq, dk, dv = orc.backward(q, k, v, do, causal, 0.5)
        assert np.max(np.abs(dk.sum(axis=2))) <= 1e-12
        assert np.max(np.abs(dv.sum(axis=2) - do.sum(axis=2))) <= 1e-12
        _, _, dv2 = orc.backward(q, k, v, do2, causal, 0.5)
        _, _, dv3 = orc.backward(q, k, v, 2.0 * do - 0.5 * do2, causal, 0.5)
        assert np.max(np.abs(dv3 - (2.0 * dv - 0.5 * dv2))) <= 1e-12
        z = orc.backward(q, k, v, np.zeros_like(do), causal, 0.5)
        assert all(np.all(g == 0) for g in z)



def _torch_e4m3(values_f32):
    return torch.from_numpy(np.asarray(values_f32, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def pin_p18_e4m3_decode(orc):
    t = orc.e4m3_decode_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    finite = np.isfinite(ref)
    assert list(np.where(~finite)[0]) == [0x7F, 0xFF]
    assert np.array_equal(t[finite], ref[finite])
    assert t[0x38] == 1.0 and t[0x7E] == 448.0 and t[0x08] == 2.0 ** -6 and t[0x01] == 2.0 ** -9
    assert t[0x07] == 7 * 2.0 ** -9 and t[0xB8] == -1.0 and t[0x00] == 0.0
    assert np.all(np.diff(t[:0x7F]) > 0)
    assert np.array_equal(t[0x80:0xFF], -t[0x00:0x7F])


def pin_p19_e4m3_encode(orc):
    t = orc.e4m3_decode_table()
    for c in list(range(0x7F)) + list(range(0x80, 0xFF)):
        if c == 0x80:
            continue  # -0 encodes to 0x80 as well; checked below
        assert orc.e4m3_encode(t[c]) == c, hex(c)
    assert orc.e4m3_encode(-0.0) == 0x80 and orc.e4m3_encode(0.0) == 0x00
    for c in range(0x7E):
        lo, hi = t[c], t[c + 1]
        mid = np.float32((lo + hi) / 2)  # exact: codes have 4 significant bits
        even = c if c % 2 == 0 else c + 1
        assert orc.e4m3_encode(mid) == even, hex(c)
        assert orc.e4m3_encode(np.nextafter(mid, np.float32(np.inf))) == c + 1
        assert orc.e4m3_encode(np.nextafter(mid, np.float32(0))) == c
        assert orc.e4m3_encode(-mid) == 0x80 | even
    assert orc.e4m3_encode(np.float32(448.0) * np.float32(1 + 2.0 ** -20)) == 0x7E
    rng = RNG(1919)
    vals = (rng.standard_normal(4000) * 2.0 ** rng.integers(-12, 8, 4000)).astype(np.float32)
    vals = vals[np.abs(vals) <= 448]
    got = np.array([orc.e4m3_encode(v) for v in vals], dtype=np.uint8)
    assert np.array_equal(got, _torch_e4m3(vals))


def pin_p20_quantize(orc):
    rng = RNG(2020)
    t = orc.e4m3_decode_table()
    x = torch.from_numpy(rng.standard_normal((2, 3, 37, 16)) * np.array([0.5, 3.0, 40.0])[None, :, None, None])
    x[1, 2] = 0.0
    xb = x.to(torch.bfloat16)
    bits = xb.view(torch.int16).numpy().view(np.uint16)
    codes, ds = orc.quantize_fp8(bits)
    xf = xb.to(torch.float32).numpy()
    amax = np.abs(xf).max(axis=(2, 3))
    assert ds[1, 2] == 1.0 and np.all(codes[1, 2] == 0)
    for b in range(2):
        for h in range(3):
            if amax[b, h] == 0:
                continue
            assert ds[b, h] == np.float32(amax[b, h] / np.float32(448.0))
            at = np.abs(xf[b, h]) == amax[b, h]
            assert np.all(np.isin(codes[b, h][at], [0x7E, 0xFE]))
            inv = np.float32(448.0) / np.float32(amax[b, h])
            y = xf[b, h] * inv
            assert np.array_equal(codes[b, h], _torch_e4m3(y))
            xh = t[codes[b, h]] * np.float64(ds[b, h])
            err = np.abs(xh - xf[b, h].astype(np.float64))
            step = np.maximum(2.0 ** -4 * np.abs(xf[b, h]), 2.0 ** -10 * np.float64(ds[b, h]) * 1.01)
            assert np.all(err <= step * (1 + 2.0 ** -18)), float(np.max(err / step))
    assert not np.any((codes & 0x7F) == 0x7F)


def pin_p21_fp8_attention(orc):
    rng = RNG(2121)
    B, H, n_q, n_k, d = 2, 2, 23, 31, 16

    def codes(n):
        c = rng.integers(0x20, 0x7E, (B, H, n, d)).astype(np.uint8)
        return c | (rng.integers(0, 2, c.shape).astype(np.uint8) << 7)

    qc, kc, vc = codes(n_q), codes(n_k), codes(n_k)
    rows = np.arange(B * H * n_q)
    # power-of-two descales: the dequantised values are bf16 numbers
    dq = np.float32(2.0 ** rng.integers(-9, -5, (B, H)))
    dk = np.float32(2.0 ** rng.integers(-9, -5, (B, H)))
    dv = np.float32(2.0 ** rng.integers(-8, -2, (B, H)))
    for causal in (False, True):
        o8, l8 = orc.attention_fp8_rows(qc, kc, vc, dq, dk, dv, rows, causal, 0.3)
        deq = [orc.dequantize_fp8(c, s) for c, s in ((qc, dq), (kc, dk), (vc, dv))]
        bits = []
        for a in deq:
            tb = torch.from_numpy(a).to(torch.bfloat16)
            assert np.array_equal(tb.to(torch.float64).numpy(), a)
            bits.append(tb.view(torch.int16).numpy().view(np.uint16))
        o16, l16 = orc.attention_rows_bf16(bits[0], bits[1], bits[2], rows, causal, 0.3)
        assert np.max(np.abs(o8 - o16)) <= 1e-13 and np.max(np.abs(l8 - l16)) <= 1e-13
    # arbitrary descales: the row function against the composition
    dq, dk, dv = (np.float32(rng.uniform(0.001, 0.02, (B, H))) for _ in range(3))
    for causal in (False, True):
        O, L = orc.attention_fp8(qc, kc, vc, dq, dk, dv, causal, 0.7)
        sel = rng.choice(B * H * n_q, 20, replace=False)
        o8, l8 = orc.attention_fp8_rows(qc, kc, vc, dq, dk, dv, sel, causal, 0.7)
        assert np.max(np.abs(O.reshape(-1, d)[sel] - o8)) <= 1e-12
        assert np.max(np.abs(L.reshape(-1)[sel] - l8)) <= 1e-12
        # O is linear in descale_v; descale_q * descale_k only scales the scores
        o2, l2 = orc.attention_fp8_rows(qc, kc, vc, dq, dk, 2 * dv, sel, causal, 0.7)
        assert np.max(np.abs(o2 - 2 * o8)) <= 1e-12 and np.max(np.abs(l2 - l8)) <= 1e-12
        o3, l3 = orc.attention_fp8_rows(qc, kc, vc, 2 * dq, dk, dv, sel, causal, 0.35)
        assert np.max(np.abs(o3 - o8)) <= 1e-12 and np.max(np.abs(l3 - l8)) <= 1e-12


def _expand_mask(mask4, B, H, n_q, n_k, bq, bk, wl, wr):
    """Element mask [B, H, N_q, N_k] from a block mask by repeating each block entry over its
    rows and keys (numpy broadcasting and repetition), with the band applied."""
    m = np.broadcast_to(mask4, (B, H) + mask4.shape[2:]).astype(bool)
    e = np.repeat(np.repeat(m, bq, axis=2), bk, axis=3)[:, :, :n_q, :n_k]
    i = np.arange(n_q)[:, None]
    j = np.arange(n_k)[None, :]
    band = np.ones((n_q, n_k), dtype=bool)
    if wl >= 0:
        band &= j >= i - wl
    if wr >= 0:
        band &= j <= i + wr
    return e & band


def _random_blockmask(rng, B, H, n_q, n_k, bq, bk, density):
    Mb = B if rng.random() < 0.5 else 1
    Mh = H if rng.random() < 0.5 else 1
    shape = (Mb, Mh, -(-n_q // bq), -(-n_k // bk))
    return (rng.random(shape) < density).astype(np.uint8)


def pin_p22_blockmask_bruteforce(orc):
    mpmath.mp.dps = 50
    rng = RNG(2222)
    for trial in range(10):
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        n_q, n_k, d = int(rng.integers(1, 8)), int(rng.integers(1, 9)), int(rng.integers(1, 4))
        bq, bk = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        wl, wr = [(-1, -1), (-1, 0), (2, 1), (0, 3)][trial % 4]
        mask = _random_blockmask(rng, B, H, n_q, n_k, bq, bk, 0.6)
        q, k, v = (rng.normal(size=(B, H, n, d)) for n in (n_q, n_k, n_k))
        scale = 0.7
        o, lse = orc.attention_blockmask(q, k, v, mask, bq, bk, scale, wl, wr)
        for b in range(B):
            for h in range(H):
                for i in range(n_q):
                    vis = [j for j in range(n_k) if mask[b % mask.shape[0], h % mask.shape[1], i // bq, j // bk]
                           and (wl < 0 or j >= i - wl) and (wr < 0 or j <= i + wr)]
                    if not vis:
                        assert np.all(o[b, h, i] == 0) and np.isneginf(lse[b, h, i]), (trial, b, h, i)
                        continue
                    e = {j: mpmath.exp(scale * mpmath.fsum(mpmath.mpf(float(q[b, h, i, c])) * float(k[b, h, j, c])
                                                           for c in range(d))) for j in vis}
                    z = mpmath.fsum(e.values())
                    for c in range(d):
                        ref = mpmath.fsum(e[j] * float(v[b, h, j, c]) for j in vis) / z
                        assert abs(float(ref) - o[b, h, i, c]) <= 1e-13 * (1 + abs(float(ref))), (trial, b, h, i)
                    assert abs(float(mpmath.log(z)) - lse[b, h, i]) <= 1e-13 * (1 + abs(lse[b, h, i]))


def pin_p23_blockmask_all_ones(orc):
    rng = RNG(2323)
    q, k, v = (rng.normal(size=(2, 2, n, 6)) for n in (21, 17, 17))
    for bq, bk in ((1, 1), (4, 5), (32, 64)):
        ones = np.ones((-(-21 // bq), -(-17 // bk)), dtype=np.uint8)
        for wl, wr in ((-1, -1), (-1, 0), (3, 2), (0, 0)):
            o, lse = orc.attention_blockmask(q, k, v, ones, bq, bk, 0.4, wl, wr)
            o_w, lse_w = orc.attention_window(q, k, v, wl, wr, 0.4)
            assert np.max(np.abs(o - o_w)) <= 1e-14
            fin = np.isfinite(lse_w)
            assert np.array_equal(fin, np.isfinite(lse)) and np.max(np.abs(lse[fin] - lse_w[fin])) <= 1e-14


def pin_p24_blockmask_torch(orc):
    rng = RNG(2424)
    for (B, H, n_q, n_k, bq, bk, wl, wr) in [(2, 3, 40, 50, 8, 16, -1, -1), (1, 2, 33, 33, 4, 8, -1, 0),
                                             (2, 2, 30, 45, 5, 3, 10, 4), (1, 4, 64, 64, 16, 16, 20, 0)]:
        mask = _random_blockmask(rng, B, H, n_q, n_k, bq, bk, 0.5)
        q, k, v = (rng.normal(size=(B, H, n, 8)) for n in (n_q, n_k, n_k))
        o, lse = orc.attention_blockmask(q, k, v, mask, bq, bk, 0.3, wl, wr)
        em = _expand_mask(mask, B, H, n_q, n_k, bq, bk, wl, wr)
        rows = em.any(-1)
        qt, kt, vt = (torch.from_numpy(x) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(em), scale=0.3)
        ref = ref.numpy()
        assert np.max(np.abs(np.where(rows[..., None], o - ref, 0.0))) <= 1e-12
        assert np.all(o[~rows] == 0) and np.all(np.isneginf(lse[~rows]))
        scores = (qt @ kt.transpose(-1, -2)) * 0.3
        lse_ref = torch.logsumexp(scores.masked_fill(~torch.from_numpy(em), float("-inf")), dim=-1).numpy()
        assert np.max(np.abs(lse[rows] - lse_ref[rows])) <= 1e-12
        for b in range(B):
            for h in range(H):
                assert orc.blockmask_pairs(n_q, n_k, mask, b, h, bq, bk, wl, wr) == int(em[b, h].sum())


def pin_p25_blockmask_deletion(orc):
    rng = RNG(2525)
    B, H, n_q, n_k, d, bq, bk = 2, 3, 24, 40, 5, 8, 5
    mask = _random_blockmask(rng, B, H, n_q, n_k, bq, bk, 0.5)
    mask = np.broadcast_to(mask, (B, H) + mask.shape[2:]).copy()
    mask[0, 0, 0] = 0  # a query block that sees nothing
    q, k, v = (rng.normal(size=(B, H, n, d)) for n in (n_q, n_k, n_k))
    o, lse = orc.attention_blockmask(q, k, v, mask, bq, bk, 0.6)
    for b in range(B):
        for h in range(H):
            for qb in range(mask.shape[2]):
                keep = np.repeat(mask[b, h, qb].astype(bool), bk)[:n_k]
                rows = slice(qb * bq, min(n_q, (qb + 1) * bq))
                if not keep.any():
                    assert np.all(o[b, h, rows] == 0) and np.all(np.isneginf(lse[b, h, rows]))
                    continue
                o_r, lse_r = orc.attention(q[b:b + 1, h:h + 1, rows], k[b:b + 1, h:h + 1, keep],
                                           v[b:b + 1, h:h + 1, keep], False, 0.6)
                assert np.max(np.abs(o_r[0, 0] - o[b, h, rows])) <= 1e-13
                assert np.max(np.abs(lse_r[0, 0] - lse[b, h, rows])) <= 1e-13
    # a mask shared over heads and batches equals its explicit copy
    shared = (rng.random((1, 1, 3, 8)) < 0.5).astype(np.uint8)
    o1, l1 = orc.attention_blockmask(q, k, v, shared, bq, bk, 0.6, 5, 1)
    o2, l2 = orc.attention_blockmask(q, k, v, np.broadcast_to(shared, (B, H, 3, 8)).copy(), bq, bk, 0.6, 5, 1)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


ALL_PINS = [pin_p22_blockmask_bruteforce, pin_p23_blockmask_all_ones, pin_p24_blockmask_torch,
            pin_p25_blockmask_deletion, pin_p1_bruteforce, pin_p2_rows_sum_to_one, pin_p3_constant_v, pin_p4_causal_row0,
            pin_p5_uniform_scores, pin_p6_one_hot, pin_p7_lse_identity, pin_p8_torch_sdpa,
            pin_p9_invariants, pin_p10_recurrence, pin_p11_window_bruteforce, pin_p12_window_special,
            pin_p13_window_torch, pin_p14_window_recurrence, pin_p15_backward_finite_differences,
            pin_p16_backward_torch, pin_p17_backward_identities, pin_p18_e4m3_decode, pin_p19_e4m3_encode,
            pin_p20_quantize, pin_p21_fp8_attention]
