"""Pins for the sliding-window rows of oracle.attention (window w: the row at
position p sees keys max(0, p-w+1) .. p).  Each pin comes from outside the
windowed code path:

  * a window at least as long as the sequence changes nothing (reduces to the
    causal oracle, itself pinned against torch's SDPA);
  * closed forms: w = 1 returns V_p exactly; w = 2 returns
    V_{p-1} + sigmoid(s_p - s_{p-1}) (V_p - V_{p-1}); q = 0 returns the mean
    of the w visible V rows;
  * translation: with no positional encoding a windowed row equals the last
    row of a causal prefill over just its w visible keys;
  * torch SDPA (fp64) with an explicit band mask, and brute force with
    math.fsum on tiny inputs.
The last test plants window mistakes in a copy of the oracle and checks that
the pins catch each.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import expit

from oracle import attention as A


def rnd(rng, *shape):
    return rng.standard_normal(shape)


def case(seed, n=9, ctx=14, Hq=4, Hkv=2, d=16):
    rng = np.random.default_rng(seed)
    return rnd(rng, n, Hq, d), rnd(rng, ctx + n, Hkv, d), rnd(rng, ctx + n, Hkv, d), ctx


@pytest.mark.parametrize("w", [23, 24, 1000])
def test_long_window_is_no_window(w):
    q, k, v, ctx = case(1)
    assert np.array_equal(A.causal_rows(q, k, v, ctx, 0.3, w), A.causal_rows(q, k, v, ctx, 0.3))


def test_shorter_window_changes_the_rows_it_cuts():
    q, k, v, ctx = case(2)
    full, win = A.causal_rows(q, k, v, ctx, 0.3), A.causal_rows(q, k, v, ctx, 0.3, 20)
    # rows at p <= 19 see all keys 0..p either way; rows p >= 20 lose key 0 .. p-20
    for i in range(q.shape[0]):
        same = ctx + i <= 19
        assert np.array_equal(full[i], win[i]) == same


def test_window_one_returns_own_value():
    q, k, v, ctx = case(3)
    out = A.causal_rows(q, k, v, ctx, 0.5, 1)
    for i in range(q.shape[0]):
        for h in range(4):
            assert np.array_equal(out[i, h], v[ctx + i, h // 2])


def test_window_two_closed_form():
    q, k, v, ctx = case(4, ctx=0)
    scale = 0.6
    out = A.causal_rows(q, k, v, ctx, scale, 2)
    for i in range(q.shape[0]):
        for h in range(4):
            kh = h // 2
            if i == 0:
                want = v[0, kh]
            else:
                s0, s1 = scale * q[i, h] @ k[i - 1, kh], scale * q[i, h] @ k[i, kh]
                want = v[i - 1, kh] + expit(s1 - s0) * (v[i, kh] - v[i - 1, kh])
            np.testing.assert_allclose(out[i, h], want, rtol=0, atol=1e-14)


def test_zero_query_mean_over_window():
    _, k, v, ctx = case(5)
    q = np.zeros((9, 4, 16))
    w = 6
    out = A.causal_rows(q, k, v, ctx, 0.3, w)
    for i in range(9):
        p = ctx + i
        for h in range(4):
            np.testing.assert_allclose(out[i, h], v[p - w + 1:p + 1, h // 2].mean(axis=0), atol=1e-14)


@pytest.mark.parametrize("w", [3, 7, 16])
def test_translation_to_a_short_prefill(w):
    q, k, v, ctx = case(6)
    out = A.causal_rows(q, k, v, ctx, 0.3, w)
    for i in range(q.shape[0]):
        p = ctx + i
        a = max(0, p - w + 1)
        want = A.causal_rows(q[i:i + 1], k[a:p + 1], v[a:p + 1], p - a, 0.3)[0]
        np.testing.assert_allclose(out[i], want, rtol=0, atol=1e-13)


@pytest.mark.parametrize("w", [1, 5, 12])
def test_matches_torch_sdpa_with_band_mask(w):
    q, k, v, ctx = case(7, n=11, ctx=9, Hq=6, Hkv=3, d=8)
    n, total = q.shape[0], ctx + q.shape[0]
    pos = ctx + np.arange(n)[:, None]
    j = np.arange(total)[None, :]
    band = torch.from_numpy((j <= pos) & (j > pos - w))
    g = 2
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(k).repeat_interleave(g, dim=1).permute(1, 0, 2)
    tv = torch.from_numpy(v).repeat_interleave(g, dim=1).permute(1, 0, 2)
    want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=band, scale=0.4)
    np.testing.assert_allclose(A.causal_rows(q, k, v, ctx, 0.4, w), want.permute(1, 0, 2).numpy(), atol=1e-12)


def brute(q, k, v, ctx, scale, w):
    n, Hq, d = q.shape
    g = Hq // k.shape[1]
    out = np.zeros_like(q)
    for i in range(n):
        p = ctx + i
        keys = [j for j in range(p + 1) if p - j < w]
        for h in range(Hq):
            kh = h // g
            s = [scale * math.fsum(q[i, h, e] * k[j, kh, e] for e in range(d)) for j in keys]
            m = max(s)
            e_ = [math.exp(x - m) for x in s]
            z = math.fsum(e_)
            for e in range(d):
                out[i, h, e] = math.fsum(wt * v[j, kh, e] for wt, j in zip(e_, keys)) / z
    return out


@pytest.mark.parametrize("seed", range(3))
def test_brute_force_tiny(seed):
    rng = np.random.default_rng(300 + seed)
    w = int(rng.integers(1, 10))
    seqs, qs, kvs = [], [], []
    for _ in range(int(rng.integers(1, 4))):
        ctx, n = int(rng.integers(0, 14)), int(rng.integers(1, 6))
        seqs.append((ctx, n))
        qs.append(rnd(rng, n, 4, 8))
        kvs.append((rnd(rng, ctx + n, 2, 8), rnd(rng, ctx + n, 2, 8)))
    got = A.attend(seqs, np.concatenate(qs), kvs, 0.35, w)
    want = np.concatenate([brute(qq, k, v, ctx, 0.35, w) for qq, (k, v), (ctx, n) in zip(qs, kvs, seqs)])
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


def test_negative_window_rejected():
    q, k, v, ctx = case(8)
    with pytest.raises(ValueError):
        A.causal_rows(q, k, v, ctx, 0.3, -1)


# ----------------------------------------------------------- planted mistakes
def _mutant(kind):
    orig = A.causal_rows

    def f(q, k, v, ctx, scale, window=0):
        if not window:
            return orig(q, k, v, ctx, scale)
        n, Hq, d = q.shape
        total, Hkv, _ = k.shape
        g = Hq // Hkv
        pos = ctx + np.arange(n)[:, None]
        j = np.arange(total)[None, :]
        if kind == "wide":          # w + 1 keys
            vis = (j <= pos) & (j >= pos - window)
        elif kind == "narrow":      # w - 1 keys (own key kept)
            vis = (j <= pos) & (j > pos - window + 1)
        elif kind == "ignored":
            vis = j <= pos
        else:                       # "absolute": window counted from key 0 instead of from p
            vis = (j <= pos) & (j < window)
        out = np.empty((n, Hq, d))
        with np.errstate(invalid="ignore"):     # a row left with no key gives NaN
            for h in range(Hq):
                kh = h // g
                s = np.where(vis, scale * (q[:, h] @ k[:, kh].T), -np.inf)
                e = np.exp(s - s.max(axis=1, keepdims=True))
                out[:, h] = (e @ v[:, kh]) / e.sum(axis=1, keepdims=True)
        return out
    return f


@pytest.mark.parametrize("kind", ["wide", "narrow", "ignored", "absolute"])
def test_pins_catch_planted_window_mistakes(kind, monkeypatch):
    monkeypatch.setattr(A, "causal_rows", _mutant(kind))
    pins = [test_window_one_returns_own_value, test_window_two_closed_form, test_zero_query_mean_over_window]
    caught = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, f"mutant {kind} passed every pin"
