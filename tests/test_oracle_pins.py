"""The float64 oracle against brute force, closed forms, worked examples,
scipy, invariants and an independent online-softmax tiled implementation."""
import numpy as np
import pytest

import oracle
import pins


def _impl(q, k, v, causal):
    return oracle.attention_forward(q, k, v, causal)


def _impl_chunked(q, k, v, causal):
    # row chunks smaller than the shapes, so that chunk edges are exercised
    return oracle.attention_forward(q, k, v, causal, row_chunk=3)


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pinned(check):
    check(_impl)


@pytest.mark.parametrize("check", [pins.check_brute_force, pins.check_online_tiled,
                                   pins.check_causal_row0_and_last], ids=lambda f: f.__name__)
def test_oracle_row_chunking(check):
    check(_impl_chunked)


def test_attention_rows_matches_forward():
    r = np.random.default_rng(3)
    q = r.standard_normal((2, 3, 37, 16))
    k = r.standard_normal((2, 3, 53, 16))
    v = r.standard_normal((2, 3, 53, 16))
    for causal in (False, True):
        O, L = oracle.attention_forward(q, k, v, causal)
        rows = [(1, 2, 0), (0, 0, 36), (1, 1, 17), (0, 2, 5), (1, 2, 36)]
        Or, Lr = oracle.attention_rows(q, k, v, causal, rows)
        for n, (b, h, i) in enumerate(rows):
            assert np.max(np.abs(Or[n] - O[b, h, i])) <= 1e-13
            assert abs(Lr[n] - L[b, h, i]) <= 1e-13


def test_attention_rows_torch_inputs():
    torch = pytest.importorskip("torch")
    r = np.random.default_rng(4)
    q = r.standard_normal((1, 2, 20, 8)).astype(np.float32)
    k = r.standard_normal((1, 2, 30, 8)).astype(np.float32)
    v = r.standard_normal((1, 2, 30, 8)).astype(np.float32)
    O, L = oracle.attention_forward(q, k, v, True)
    Or, Lr = oracle.attention_rows(torch.from_numpy(q).to(torch.bfloat16).float(),
                                   torch.from_numpy(k), torch.from_numpy(v), True, [(0, 1, 19)])
    assert Or.shape == (1, 8) and np.isfinite(Lr).all()
    Or, Lr = oracle.attention_rows(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                   True, [(0, 1, 19), (0, 0, 3)])
    assert np.max(np.abs(Or[0] - O[0, 1, 19])) <= 1e-13
    assert abs(Lr[1] - L[0, 0, 3]) <= 1e-13


def test_empty_is_rejected():
    with pytest.raises(ValueError):
        oracle.attention_forward(np.zeros((1, 1, 0, 4)), np.zeros((1, 1, 3, 4)), np.zeros((1, 1, 3, 4)), False)
    with pytest.raises(ValueError):
        oracle.attention_forward(np.zeros((1, 1, 2, 4)), np.zeros((1, 1, 0, 4)), np.zeros((1, 1, 0, 4)), False)


def test_online_reference_matches_page_grid_dtype_free():
    # The online recurrence is tile-size invariant: two very different tilings
    # agree to rounding (a pin of the reference itself, independent of the oracle).
    from online_reference import online_tiled_attention

    r = np.random.default_rng(11)
    q = r.standard_normal((1, 2, 90, 32))
    k = r.standard_normal((1, 2, 70, 32))
    v = r.standard_normal((1, 2, 70, 32))
    for causal in (False, True):
        a = online_tiled_attention(q, k, v, causal, 1, 1)
        b = online_tiled_attention(q, k, v, causal, 90, 70)
        c = online_tiled_attention(q, k, v, causal, 7, 13, skip_masked_tiles=False)
        for x, y in ((a, b), (a, c)):
            assert np.max(np.abs(x[0] - y[0])) <= 1e-12
            assert np.max(np.abs(x[1] - y[1])) <= 1e-12


def test_oracle_explicit_scale():
    pins.check_explicit_scale(lambda q, k, v, causal, scale: oracle.attention_forward(q, k, v, causal, scale=scale))
    # attention_rows and scores_row honour the same scale
    r = np.random.default_rng(8)
    q = r.standard_normal((1, 2, 11, 8))
    k = r.standard_normal((1, 2, 13, 8))
    v = r.standard_normal((1, 2, 13, 8))
    O, L = oracle.attention_forward(q, k, v, True, scale=0.3)
    Or, Lr = oracle.attention_rows(q, k, v, True, [(0, 1, 7)], scale=0.3)
    assert np.max(np.abs(Or[0] - O[0, 1, 7])) <= 1e-13 and abs(Lr[0] - L[0, 1, 7]) <= 1e-13
    s = oracle.scores_row(q, k, 0, 1, 7, True, scale=0.3)
    from scipy.special import logsumexp

    assert abs(logsumexp(s) - L[0, 1, 7]) <= 1e-12


def test_partials_merge_to_the_full_result():
    # The associative update: exact partials over disjoint key ranges merge
    # into the exact result over all keys (any split, causal ranges that some
    # rows cannot see included), and one range is the whole computation.
    r = np.random.default_rng(12)
    q = r.standard_normal((2, 2, 13, 8)) * 2.0
    k = r.standard_normal((2, 2, 37, 8))
    v = r.standard_normal((2, 2, 37, 8))
    for causal in (False, True):
        O, L = oracle.attention_forward(q, k, v, causal)
        for cuts in ([0, 37], [0, 5, 37], [0, 1, 2, 20, 36, 37], [0, 12, 13, 14, 37]):
            parts = [oracle.attention_partial(q, k, v, causal, a, b) for a, b in zip(cuts, cuts[1:])]
            Om, Lm = oracle.merge_partials(parts)
            assert np.max(np.abs(Om - O)) <= 1e-12 and np.max(np.abs(Lm - L)) <= 1e-12
        # a range past every row's last key (causal) is empty
        if causal:
            Oe, Le = oracle.attention_partial(q, k, v, True, 13, 37)
            assert np.all(Le == -np.inf) and np.all(Oe == 0.0)
    # one range equals the partial over all keys
    Op, Lp = oracle.attention_partial(q, k, v, False, 0, 37)
    O, L = oracle.attention_forward(q, k, v, False)
    assert np.max(np.abs(Op - O)) <= 1e-13 and np.max(np.abs(Lp - L)) <= 1e-13


def test_partial_against_brute_force_on_the_range():
    # a non-causal partial is the plain definition on the sliced keys
    r = np.random.default_rng(13)
    q = r.standard_normal((1, 2, 4, 3))
    k = r.standard_normal((1, 2, 9, 3))
    v = r.standard_normal((1, 2, 9, 3))
    Op, Lp = oracle.attention_partial(q, k, v, False, 2, 7)
    Ob, Lb = pins.brute_force(q, k[:, :, 2:7], v[:, :, 2:7], False)
    assert np.max(np.abs(Op - Ob)) <= 1e-12 and np.max(np.abs(Lp - Lb)) <= 1e-12


def test_varlen_oracle_against_brute_force_and_padding():
    # Each packed sequence is the plain definition on its own slices (brute
    # force), and the whole batch equals dense attention over the padded
    # batch with the padded keys masked out, on the real rows ("use padding
    # with an attention mask"), which the varlen path skips.
    from scipy.special import logsumexp, softmax

    r = np.random.default_rng(21)
    lens_q = [3, 0, 5, 1, 4]
    lens_k = [4, 3, 5, 2, 0]
    cu_q = np.concatenate([[0], np.cumsum(lens_q)])
    cu_k = np.concatenate([[0], np.cumsum(lens_k)])
    H, D = 2, 4
    q = r.standard_normal((H, cu_q[-1], D))
    k = r.standard_normal((H, cu_k[-1], D))
    v = r.standard_normal((H, cu_k[-1], D))
    for causal in (False, True):
        O, L = oracle.attention_varlen(q, k, v, cu_q, cu_k, causal)
        for b in range(len(lens_q)):
            q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
            if q1 == q0:
                continue
            if k1 == k0:
                assert np.all(O[:, q0:q1] == 0) and np.all(L[:, q0:q1] == -np.inf)
                continue
            Ob, Lb = pins.brute_force(q[None, :, q0:q1], k[None, :, k0:k1], v[None, :, k0:k1], causal)
            assert np.max(np.abs(O[:, q0:q1] - Ob[0])) <= 1e-12
            assert np.max(np.abs(L[:, q0:q1] - Lb[0])) <= 1e-12
            # padded to the longest key count, padded keys masked
            mk = max(lens_k)
            kp = np.concatenate([k[:, k0:k1], 7.0 * np.ones((H, mk - (k1 - k0), D))], axis=1)
            vp = np.concatenate([v[:, k0:k1], 9.0 * np.ones((H, mk - (k1 - k0), D))], axis=1)
            s = np.einsum("hid,hjd->hij", q[:, q0:q1], kp) / np.sqrt(D)
            keep = np.arange(mk)[None, :] < (k1 - k0)
            if causal:
                keep = keep & (np.arange(mk)[None, :] <= np.arange(q1 - q0)[:, None])
            s = np.where(keep, s, -np.inf)
            assert np.max(np.abs(np.matmul(softmax(s, -1), vp) - O[:, q0:q1])) <= 1e-12
            assert np.max(np.abs(logsumexp(s, -1) - L[:, q0:q1])) <= 1e-12
