"""Pins for oracle.attention: the oracle is checked against facts that do not
come from the oracle itself.

  * library special case: with no cached prefix, a prefill is textbook causal
    attention, so it must equal torch's scaled_dot_product_attention (fp64,
    is_causal, enable_gqa for grouped heads);
  * chunked == unchunked ("Sarathi-Serve: Chunked Prefills for Stall-Free LLM
    Inference", intro: chunking changes the schedule, not the math);
  * a decode row == the last row of a prefill over the same prefix;
  * grouped-query == multi-head attention on kv heads repeated g times;
  * closed forms: one visible key returns V0 exactly; constant V rows return
    that row; q = 0 returns the mean of the visible V rows; two visible keys
    give V0 + sigmoid(s1 - s0) * (V1 - V0);
  * brute force with math.fsum on tiny inputs.
A last test plants mistakes in a copy of the oracle and checks that the pins
catch each of them.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import expit

from oracle import attention as A


def rnd(rng, *shape):
    return rng.standard_normal(shape)


def sdpa_causal(q, k, v, scale):
    """q [n, Hq, d], k/v [n, Hkv, d] -> torch SDPA (fp64, causal, GQA) as [n, Hq, d]."""
    Hq, Hkv = q.shape[1], k.shape[1]
    tq = torch.from_numpy(q).permute(1, 0, 2).unsqueeze(0)
    tk = torch.from_numpy(k).permute(1, 0, 2).unsqueeze(0)
    tv = torch.from_numpy(v).permute(1, 0, 2).unsqueeze(0)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=True, scale=scale, enable_gqa=(Hq != Hkv))
    return o.squeeze(0).permute(1, 0, 2).numpy()


@pytest.mark.parametrize("n,Hq,Hkv,d", [(1, 1, 1, 8), (7, 4, 1, 16), (33, 8, 2, 32), (64, 6, 3, 64), (50, 7, 7, 16)])
def test_prefill_matches_torch_sdpa(n, Hq, Hkv, d):
    rng = np.random.default_rng(n * 100 + Hq)
    q, k, v = rnd(rng, n, Hq, d), rnd(rng, n, Hkv, d), rnd(rng, n, Hkv, d)
    scale = 1 / math.sqrt(d)
    got = A.causal_rows(q, k, v, 0, scale)
    want = sdpa_causal(q, k, v, scale)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_scale_is_applied():
    rng = np.random.default_rng(5)
    q, k, v = rnd(rng, 9, 2, 8), rnd(rng, 9, 2, 8), rnd(rng, 9, 2, 8)
    got = A.causal_rows(q, k, v, 0, 0.37)
    np.testing.assert_allclose(got, sdpa_causal(q, k, v, 0.37), atol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_chunked_equals_unchunked(seed):
    rng = np.random.default_rng(seed)
    L, Hq, Hkv, d = int(rng.integers(2, 90)), 4, 2, 16
    q, k, v = rnd(rng, L, Hq, d), rnd(rng, L, Hkv, d), rnd(rng, L, Hkv, d)
    whole = A.causal_rows(q, k, v, 0, 0.25)
    cuts = sorted(set(rng.integers(1, L, size=int(rng.integers(1, 6))).tolist()))
    bounds = [0] + cuts + [L]
    parts = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        parts.append(A.causal_rows(q[a:b], k[:b], v[:b], a, 0.25))
    np.testing.assert_allclose(np.concatenate(parts), whole, rtol=0, atol=1e-12)


def test_decode_is_last_prefill_row():
    rng = np.random.default_rng(11)
    ctx, Hq, Hkv, d = 45, 8, 2, 32
    q, k, v = rnd(rng, ctx + 1, Hq, d), rnd(rng, ctx + 1, Hkv, d), rnd(rng, ctx + 1, Hkv, d)
    full = A.causal_rows(q, k, v, 0, 0.2)
    dec = A.causal_rows(q[ctx:], k, v, ctx, 0.2)
    np.testing.assert_allclose(dec[0], full[-1], rtol=0, atol=1e-12)


def test_gqa_equals_mha_on_repeated_kv_heads():
    rng = np.random.default_rng(12)
    n, ctx, Hq, Hkv, d = 10, 13, 12, 3, 16
    q = rnd(rng, n, Hq, d)
    k, v = rnd(rng, ctx + n, Hkv, d), rnd(rng, ctx + n, Hkv, d)
    g = Hq // Hkv
    k_rep = torch.from_numpy(k).repeat_interleave(g, dim=1).numpy()
    v_rep = torch.from_numpy(v).repeat_interleave(g, dim=1).numpy()
    np.testing.assert_allclose(A.causal_rows(q, k, v, ctx, 0.3), A.causal_rows(q, k_rep, v_rep, ctx, 0.3),
                               rtol=0, atol=1e-13)


def test_first_prompt_token_returns_v0_exactly():
    rng = np.random.default_rng(13)
    q, k, v = rnd(rng, 1, 4, 8), rnd(rng, 1, 2, 8), rnd(rng, 1, 2, 8)
    out = A.causal_rows(q, k, v, 0, 0.5)
    for h in range(4):
        assert np.array_equal(out[0, h], v[0, h // 2])


def test_constant_v_rows_return_that_row():
    rng = np.random.default_rng(14)
    n, ctx, d = 6, 20, 16
    q, k = rnd(rng, n, 2, d), rnd(rng, ctx + n, 1, d)
    row = rnd(rng, d)
    v = np.broadcast_to(row, (ctx + n, 1, d)).copy()
    out = A.causal_rows(q, k, v, ctx, 0.25)
    np.testing.assert_allclose(out, np.broadcast_to(row, out.shape), rtol=0, atol=1e-14)


def test_zero_query_gives_mean_of_visible_values():
    rng = np.random.default_rng(15)
    n, ctx, d = 5, 7, 8
    q = np.zeros((n, 1, d))
    k, v = rnd(rng, ctx + n, 1, d), rnd(rng, ctx + n, 1, d)
    out = A.causal_rows(q, k, v, ctx, 0.25)
    for i in range(n):
        np.testing.assert_allclose(out[i, 0], v[:ctx + i + 1, 0].mean(axis=0), atol=1e-14)


def test_two_keys_closed_form():
    rng = np.random.default_rng(16)
    d, scale = 8, 0.7
    q, k, v = rnd(rng, 1, 1, d), rnd(rng, 2, 1, d), rnd(rng, 2, 1, d)
    out = A.causal_rows(q, k, v, 1, scale)[0, 0]
    s0, s1 = scale * q[0, 0] @ k[0, 0], scale * q[0, 0] @ k[1, 0]
    want = v[0, 0] + expit(s1 - s0) * (v[1, 0] - v[0, 0])
    np.testing.assert_allclose(out, want, atol=1e-14)


def brute(q, k, v, ctx, scale):
    n, Hq, d = q.shape
    g = Hq // k.shape[1]
    out = np.zeros_like(q)
    for i in range(n):
        p = ctx + i
        for h in range(Hq):
            kh = h // g
            s = [scale * math.fsum(q[i, h, e] * k[j, kh, e] for e in range(d)) for j in range(p + 1)]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = math.fsum(w)
            for e in range(d):
                out[i, h, e] = math.fsum(w[j] * v[j, kh, e] for j in range(p + 1)) / z
    return out


@pytest.mark.parametrize("seed", range(4))
def test_brute_force_tiny(seed):
    rng = np.random.default_rng(100 + seed)
    seqs, qs, kvs = [], [], []
    for _ in range(int(rng.integers(1, 4))):
        ctx, n = int(rng.integers(0, 12)), int(rng.integers(1, 6))
        seqs.append((ctx, n))
        qs.append(rnd(rng, n, 4, 8))
        kvs.append((rnd(rng, ctx + n, 2, 8), rnd(rng, ctx + n, 2, 8)))
    q = np.concatenate(qs)
    got = A.attend(seqs, q, kvs, 0.35)
    want = np.concatenate([brute(qq, k, v, ctx, 0.35) for qq, (k, v), (ctx, n) in zip(qs, kvs, seqs)])
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


def test_bf16_widening_is_exact():
    x = torch.randn(1000, dtype=torch.float32).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(A.bf16_bits_to_f64(bits), x.to(torch.float64).numpy())


# ----------------------------------------------------------- planted mistakes
def _mutant(kind):
    def f(q, k, v, ctx, scale):
        n, Hq, d = q.shape
        total, Hkv, _ = k.shape
        g = Hq // Hkv
        pos = ctx + np.arange(n)
        lim = pos if kind != "offbyone" else pos - 1
        vis = np.arange(total)[None, :] <= lim[:, None]
        if kind == "offbyone":
            vis[:, 0] = True
        out = np.empty((n, Hq, d))
        for h in range(Hq):
            kh = (h % Hkv) if kind == "headmap" else h // g
            sc = 1.0 if kind == "noscale" else scale
            s = sc * (q[:, h] @ k[:, kh].T)
            if kind == "sign":
                s = -s
            s = np.where(vis, s, -np.inf)
            w = np.exp(s - s.max(axis=1, keepdims=True))
            vv = k[:, kh] if kind == "kforv" else v[:, kh]
            out[:, h] = (w @ vv) / w.sum(axis=1, keepdims=True)
        return out
    return f


@pytest.mark.parametrize("kind", ["offbyone", "headmap", "noscale", "sign", "kforv"])
def test_pins_catch_planted_mistakes(kind, monkeypatch):
    monkeypatch.setattr(A, "causal_rows", _mutant(kind))
    pins = [
        lambda: test_prefill_matches_torch_sdpa(33, 8, 2, 32),
        lambda: test_gqa_equals_mha_on_repeated_kv_heads(),
        lambda: test_two_keys_closed_form(),
        lambda: test_first_prompt_token_returns_v0_exactly(),
    ]
    caught = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, f"mutant {kind} passed every pin"
