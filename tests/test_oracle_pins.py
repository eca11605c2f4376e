"""Pins of the CPU oracle: each check ties a function to something other than itself.

Brute-force loops on tiny inputs, closed forms, invariants of the method,
library routines and hand-derived fixtures (tests/golden/).  These run on the CPU.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import policy as opol
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------- brute-force helpers
# Scalar loops over plain Python lists: a second, independent way of computing
# the same definitions, used only on tiny inputs.

def bf_linear(x, W):
    return [[sum(row[k] * W[n][k] for k in range(len(row))) for n in range(len(W))] for row in x]


def bf_rms(x, w, eps):
    out = []
    for row in x:
        r = 1.0 / math.sqrt(sum(v * v for v in row) / len(row) + eps)
        out.append([row[k] * r * (1.0 + w[k]) for k in range(len(row))])
    return out


def bf_gelu(v):
    return 0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0)))


def bf_attention(q, k, v, Hq, Hkv, hd, mask=None):
    nq, nk = len(q), len(k)
    out = [[0.0] * (Hq * hd) for _ in range(nq)]
    for j in range(Hq):
        g = j * Hkv // Hq
        for i in range(nq):
            s = []
            for t in range(nk):
                dot = sum(q[i][j * hd + d] * k[t][g * hd + d] for d in range(hd))
                s.append(dot / math.sqrt(hd) + (0.0 if mask is None else mask[i][t]))
            m = max(s)
            lse = m + math.log(sum(math.exp(x - m) for x in s))
            p = [math.exp(x - lse) for x in s]
            for d in range(hd):
                out[i][j * hd + d] = sum(p[t] * v[t][g * hd + d] for t in range(nk))
    return out


def bf_add(a, b):
    return [[x + y for x, y in zip(r, s)] for r, s in zip(a, b)]


def L(a):
    return np.asarray(a, dtype=np.float64).tolist()


def tiny_cfg(**kw):
    base = dict(d_p=8, L_p=1, Hq=2, Hkv=1, hd=4, F_p=6, d_e=8, L_e=1, Hq_e=2, Hkv_e=1,
                hd_e=4, F_e=6, H=3, d_a=2, steps=2, n_prefix=5)
    base.update(kw)
    return synth.config(0, **base)


def big_weights(cfg, seed=0, scale=25.0):
    """Synthetic weights with linear layers scaled up so every term is visible."""
    w, b = synth.make_weights(cfg, seed)
    kinds = {n: k for n, _, k in synth.weight_specs(cfg)}
    return {n: (a * scale if kinds[n] == "linear" else a) for n, a in w.items()}, b


# ------------------------------------------------------------------- attention

def test_attention_golden_eq2():
    g = golden("attention_eq2.json")
    ln3 = math.log(3.0)
    q = np.array([[ln3, -ln3]])
    k, v = np.array(g["k"]), np.array(g["v"])
    out = oracle.attention(q, k, v, g["n_heads"], g["n_kv_heads"], g["head_dim"])
    np.testing.assert_allclose(out, g["out"], rtol=0, atol=1e-13)
    mask = np.array([[0.0, -np.inf]])
    out = oracle.attention(q, k, v, 2, 1, 1, mask=mask)
    np.testing.assert_allclose(out, g["masked_second_key_out"], rtol=0, atol=1e-13)


@pytest.mark.parametrize("Hq,Hkv", [(2, 1), (4, 4), (4, 2), (3, 1)])
def test_attention_brute_force(Hq, Hkv):
    rng = np.random.default_rng(1)
    hd, nq, nk = 3, 5, 7
    q = rng.standard_normal((nq, Hq * hd)) * 2
    k = rng.standard_normal((nk, Hkv * hd)) * 2
    v = rng.standard_normal((nk, Hkv * hd))
    ref = bf_attention(L(q), L(k), L(v), Hq, Hkv, hd)
    np.testing.assert_allclose(oracle.attention(q, k, v, Hq, Hkv, hd), ref, rtol=1e-12, atol=1e-13)


def test_attention_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(2)
    Hq, Hkv, hd, nq, nk = 8, 2, 16, 11, 13
    q = rng.standard_normal((nq, Hq * hd))
    k = rng.standard_normal((nk, Hkv * hd))
    v = rng.standard_normal((nk, Hkv * hd))
    tq = torch.from_numpy(q).view(nq, Hq, hd).transpose(0, 1)
    tk = torch.from_numpy(k).view(nk, Hkv, hd).transpose(0, 1).repeat_interleave(Hq // Hkv, 0)
    tv = torch.from_numpy(v).view(nk, Hkv, hd).transpose(0, 1).repeat_interleave(Hq // Hkv, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)
    ref = ref.transpose(0, 1).reshape(nq, Hq * hd).numpy()
    np.testing.assert_allclose(oracle.attention(q, k, v, Hq, Hkv, hd), ref, rtol=1e-12, atol=1e-12)


def test_attention_rows_sum_to_one_and_key_permutation_invariance():
    rng = np.random.default_rng(3)
    hd, n = 4, 9
    q = rng.standard_normal((n, hd))
    k = rng.standard_normal((n, hd))
    v = np.ones((n, hd))  # with V = 1 the output is the row sum of P
    np.testing.assert_allclose(oracle.attention(q, k, v, 1, 1, hd), 1.0, atol=1e-14)
    v = rng.standard_normal((n, hd))
    perm = rng.permutation(n)
    a = oracle.attention(q, k, v, 1, 1, hd)
    b = oracle.attention(q, k[perm], v[perm], 1, 1, hd)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)


# ------------------------------------------------------ norms, activations, time

def test_rms_norm_library_and_scale_invariance():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 16))
    w = rng.standard_normal(16) * 0.1
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (16,), torch.from_numpy(1.0 + w), eps=1e-6)
    np.testing.assert_allclose(oracle.rms_norm(x, w, 1e-6), ref.numpy(), rtol=1e-13)
    np.testing.assert_allclose(oracle.rms_norm(x, w, 0.0), oracle.rms_norm(7.5 * x, w, 0.0), rtol=1e-13)
    np.testing.assert_allclose(oracle.rms_norm(L(x), w, 1e-6), bf_rms(L(x), L(w), 1e-6), rtol=1e-13)


def test_gelu_library_and_erf():
    x = np.linspace(-6, 6, 101)
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="none").numpy()
    np.testing.assert_allclose(oracle.gelu(x), ref, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(oracle.gelu(x), [bf_gelu(t) for t in x], rtol=1e-14, atol=1e-16)
    assert oracle.gelu(np.array([0.0]))[0] == 0.0


def test_time_embedding_golden_and_norm():
    g = golden("time_embedding.json")
    for c in g["cases"]:
        np.testing.assert_allclose(oracle.time_embedding(c["tau"], g["d"]), c["phi"], rtol=0, atol=1e-15)
    for tau in (0.0, 0.1, 0.37, 1.0):
        phi = oracle.time_embedding(tau, 1024)
        assert abs(float(phi @ phi) - 512.0) < 1e-9
    phi0 = oracle.time_embedding(0.0, 10)
    assert list(phi0) == [0.0, 1.0] * 5


# ----------------------------------------------------------------- Euler solver

def test_euler_linear_field_closed_form():
    rng = np.random.default_rng(5)
    x0 = rng.standard_normal((4, 3))
    for a, b, T in [(0.7, 0.3, 10), (-1.3, 2.0, 4), (0.0, 0.5, 7), (2.0, -1.0, 1)]:
        sched = oracle.uniform_schedule(T)
        dt = 1.0 / T
        got = oracle.euler_integrate(x0, sched, lambda x, tau: a * x + b)
        g = (1 + a * dt) ** T
        want = x0 + T * dt * b if a == 0 else g * x0 + b * (g - 1) / a
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_euler_uses_left_endpoint_time_and_step_sizes():
    # v depends only on tau: X^T - X^0 = sum_k (tau_{k+1} - tau_k) f(tau_k)
    sched = np.array([0.0, 0.1, 0.35, 0.8, 1.0])
    got = oracle.euler_integrate(np.zeros(1), sched, lambda x, tau: np.full_like(x, tau ** 2 + 1))
    want = sum((sched[k + 1] - sched[k]) * (sched[k] ** 2 + 1) for k in range(4))
    assert abs(got[0] - want) < 1e-15
    # reversed schedule 1 -> 0 flips the sign of every step
    rev = oracle.uniform_schedule(4, 1.0, 0.0)
    np.testing.assert_allclose(rev, [1.0, 0.75, 0.5, 0.25, 0.0])


def test_uniform_schedule():
    s = oracle.uniform_schedule(10)
    assert s[0] == 0.0 and abs(s[-1] - 1.0) < 1e-15 and len(s) == 11
    np.testing.assert_allclose(np.diff(s), 0.1, rtol=1e-12)


# ------------------------------------------------------ prefix layer and expert

def pad_mask(nq, nk, n):
    """Additive key-padding mask as lists: keys t >= n get -inf for every query."""
    return [[0.0 if t < n else -math.inf for t in range(nk)] for _ in range(nq)]


def bf_prefix_layer(W, h, l, c, n_valid=None):
    p = f"prefix.{l}."
    u = bf_rms(h, L(W[p + "w1"]), c.rms_eps)
    q, k, v = bf_linear(u, L(W[p + "wq"])), bf_linear(u, L(W[p + "wk"])), bf_linear(u, L(W[p + "wv"]))
    mask = None if n_valid is None else pad_mask(len(h), len(h), n_valid)
    h = bf_add(h, bf_linear(bf_attention(q, k, v, c.Hq, c.Hkv, c.hd, mask), L(W[p + "wo"])))
    u = bf_rms(h, L(W[p + "w2"]), c.rms_eps)
    g, up = bf_linear(u, L(W[p + "wg"])), bf_linear(u, L(W[p + "wu"]))
    m = [[bf_gelu(a) * b for a, b in zip(r, s)] for r, s in zip(g, up)]
    return bf_add(h, bf_linear(m, L(W[p + "wd"])))


def bf_velocity(W, x, tau, cache, c):
    d = c.d_e
    phi = []
    for i in range(d // 2):
        f = 10000.0 ** (-2.0 * i / d)
        phi += [math.sin(tau * f), math.cos(tau * f)]
    e = [[a + b for a, b in zip(r, phi)] for r in bf_linear(x, L(W["expert.w_in"]))]
    for l in range(c.L_e):
        p = f"expert.{l}."
        u = bf_rms(e, L(W[p + "a1"]), c.rms_eps)
        q, k, v = bf_linear(u, L(W[p + "wqs"])), bf_linear(u, L(W[p + "wks"])), bf_linear(u, L(W[p + "wvs"]))
        e = bf_add(e, bf_linear(bf_attention(q, k, v, c.Hq_e, c.Hkv_e, c.hd_e), L(W[p + "wos"])))
        u = bf_rms(e, L(W[p + "a2"]), c.rms_eps)
        qc = bf_linear(u, L(W[p + "wqc"]))
        kc, vc = cache[l]
        e = bf_add(e, bf_linear(bf_attention(qc, L(kc), L(vc), c.Hq_e, c.Hkv_e, c.hd_e), L(W[p + "woc"])))
        u = bf_rms(e, L(W[p + "a3"]), c.rms_eps)
        g, up = bf_linear(u, L(W[p + "wg"])), bf_linear(u, L(W[p + "wu"]))
        m = [[bf_gelu(a) * b for a, b in zip(r, s)] for r, s in zip(g, up)]
        e = bf_add(e, bf_linear(m, L(W[p + "wd"])))
    return bf_linear(bf_rms(e, L(W["expert.norm"]), c.rms_eps), L(W["expert.w_out"]))


@pytest.mark.parametrize("Hq,Hkv", [(2, 1), (2, 2)])
def test_prefix_layer_brute_force(Hq, Hkv):
    c = tiny_cfg(Hq=Hq, Hkv=Hkv)
    W, _ = big_weights(c, seed=11)
    h = synth.make_prefix(c, 11)[0].astype(np.float64)
    got = oracle.Oracle(c, W).prefix_layer(h, 0)
    np.testing.assert_allclose(got, bf_prefix_layer(W, L(h), 0, c), rtol=1e-11, atol=1e-12)


def test_cache_projection_brute_force():
    c = tiny_cfg(L_e=2)
    W, _ = big_weights(c, seed=12)
    z = np.random.default_rng(12).standard_normal((c.n_prefix, c.d_p))
    cache = oracle.Oracle(c, W).cache_project(z)
    for e in range(2):
        np.testing.assert_allclose(cache[e][0], bf_linear(L(z), L(W[f"cache.{e}.wk"])), rtol=1e-12)
        np.testing.assert_allclose(cache[e][1], bf_linear(L(z), L(W[f"cache.{e}.wv"])), rtol=1e-12)


@pytest.mark.parametrize("Hkv_e", [1, 2])
def test_velocity_brute_force(Hkv_e):
    c = tiny_cfg(L_e=2, Hkv_e=Hkv_e)
    W, _ = big_weights(c, seed=13)
    o = oracle.Oracle(c, W)
    z = o.encode_prefix(synth.make_prefix(c, 13)[0])
    cache = o.cache_project(z)
    x = synth.make_noise(c, 13)[0].astype(np.float64)
    for tau in (0.0, 0.4):
        np.testing.assert_allclose(o.velocity(x, tau, cache), bf_velocity(W, L(x), tau, cache, c),
                                   rtol=1e-10, atol=1e-12)


# ------------------------------------------------ key padding (Eq. 2 masks, §III-B)

@pytest.mark.parametrize("n", [1, 3, 5])
def test_masked_attention_brute_force_and_exact_zero_weights(n):
    """Keys past n get M = -inf: the brute-force softmax with that mask agrees, masked keys carry
    weight exactly 0 (any finite keys and values there leave the output bit for bit the same),
    and the visible keys alone give the same output."""
    rng = np.random.default_rng(40 + n)
    Nq, Nk, Hq, Hkv, hd = 4, 5, 2, 1, 4
    q, k, v = rng.standard_normal((Nq, Hq * hd)), rng.standard_normal((Nk, Hkv * hd)), rng.standard_normal((Nk, Hkv * hd))
    mask = opol.key_mask(n, Nk)
    got = oracle.attention(q, k, v, Hq, Hkv, hd, mask)
    np.testing.assert_allclose(got, bf_attention(L(q), L(k), L(v), Hq, Hkv, hd, pad_mask(Nq, Nk, n)),
                               rtol=1e-12, atol=1e-14)
    k2, v2 = k.copy(), v.copy()
    k2[n:] = 1e3 * rng.standard_normal(k2[n:].shape)
    v2[n:] = 1e300
    np.testing.assert_array_equal(oracle.attention(q, k2, v2, Hq, Hkv, hd, mask), got)
    np.testing.assert_allclose(oracle.attention(q, k[:n], v[:n], Hq, Hkv, hd), got, rtol=1e-13, atol=1e-15)
    with pytest.raises(ValueError):
        opol.key_mask(0, Nk)


def test_masked_prefix_layer_brute_force():
    c = tiny_cfg(n_prefix=6)
    W, _ = big_weights(c, seed=41)
    h = synth.make_prefix(c, 41)[0].astype(np.float64)
    got = oracle.Oracle(c, W).prefix_layer(h, 0, n_valid=4)
    np.testing.assert_allclose(got, bf_prefix_layer(W, L(h), 0, c, n_valid=4), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("attn", ["cross", "joint"])
def test_padded_observation_equals_true_length_and_ignores_padding(attn):
    """An observation filling 4 of 9 prefix positions gives the chunk (and the valid cache rows)
    of the same observation run at length 4; two different paddings give the same bits; and a
    length equal to N is the unmasked computation bit for bit."""
    c = tiny_cfg(L_p=2, L_e=2, n_prefix=9, attn=attn)
    W, _ = big_weights(c, seed=42, scale=5.0)
    o = oracle.Oracle(c, W)
    rng = np.random.default_rng(42)
    n = 4
    z = synth.make_prefix(c, 42)[0].astype(np.float64)
    x0 = synth.make_noise(c, 42)
    pad1, pad2 = z.copy(), z.copy()
    pad1[n:] = 7.0 * rng.standard_normal((c.n_prefix - n, c.d_p))
    pad2[n:] = -3.0 * rng.standard_normal((c.n_prefix - n, c.d_p))
    out1, caches1 = o.run(pad1[None], x0, keep_cache=True, lengths=[n])
    out2, caches2 = o.run(pad2[None], x0, keep_cache=True, lengths=[n])
    np.testing.assert_array_equal(out1, out2)
    short, caches_s = o.run(z[None, :n], x0, keep_cache=True)
    np.testing.assert_allclose(out1, short, rtol=1e-11, atol=1e-12)
    for (k1, v1), (k2, v2), (ks, vs) in zip(caches1[0], caches2[0], caches_s[0]):
        np.testing.assert_array_equal(k1[:n], k2[:n])
        np.testing.assert_array_equal(v1[:n], v2[:n])
        np.testing.assert_allclose(k1[:n], ks, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(v1[:n], vs, rtol=1e-11, atol=1e-12)
    np.testing.assert_array_equal(o.run(z[None], x0, lengths=[c.n_prefix]), o.run(z[None], x0))


def test_encode_prefix_is_layers_then_final_norm():
    c = tiny_cfg(L_p=3)
    W, _ = big_weights(c, seed=14)
    z0 = synth.make_prefix(c, 14)[0].astype(np.float64)
    h = L(z0)
    for l in range(3):
        h = bf_prefix_layer(W, h, l, c)
    want = bf_rms(h, L(W["prefix.norm"]), c.rms_eps)
    np.testing.assert_allclose(oracle.Oracle(c, W).encode_prefix(z0), want, rtol=1e-10, atol=1e-12)


# ------------------------------------------------------------ structural invariants

def test_bidirectional_prefix_first_token_sees_last():
    c = synth.config(0)
    W, _ = synth.make_weights(c, 0)
    o = oracle.Oracle(c, W)
    z0 = synth.make_prefix(c, 0)[0].astype(np.float64)
    z1 = z0.copy()
    z1[-1] += 1.0
    delta = np.abs(o.prefix_layer(z1, 0)[0] - o.prefix_layer(z0, 0)[0]).max()
    assert delta > 1e-8
    # the attention weight of token 0 on token N-1 is positive
    u = oracle.rms_norm(z0, W["prefix.0.w1"], c.rms_eps)
    q = u @ W["prefix.0.wq"].T.astype(np.float64)
    k = u @ W["prefix.0.wk"].T.astype(np.float64)
    s = q[0, :c.hd] @ k[:, :c.hd].T / math.sqrt(c.hd)
    p = np.exp(s - s.max()) / np.exp(s - s.max()).sum()
    assert p[-1] > 0


def test_bidirectional_check_detects_a_planted_causal_mask(monkeypatch):
    """Plant a causal mask in the oracle: the check above must then see no change."""
    real = opol.attention

    def causal(q, k, v, n_heads, n_kv_heads, head_dim, mask=None):
        n = q.shape[0]
        m = np.triu(np.full((n, k.shape[0]), -np.inf), 1)
        return real(q, k, v, n_heads, n_kv_heads, head_dim, mask=m)

    monkeypatch.setattr(opol, "attention", causal)
    c = synth.config(0)
    W, _ = synth.make_weights(c, 0)
    o = oracle.Oracle(c, W)
    z0 = synth.make_prefix(c, 0)[0].astype(np.float64)
    z1 = z0.copy()
    z1[-1] += 1.0
    assert np.abs(o.prefix_layer(z1, 0)[0] - o.prefix_layer(z0, 0)[0]).max() == 0.0


def test_prefix_token_permutation_equivariance():
    c = synth.config(0)
    W, _ = synth.make_weights(c, 1)
    o = oracle.Oracle(c, W)
    z0 = synth.make_prefix(c, 1)[0].astype(np.float64)
    perm = np.random.default_rng(0).permutation(c.n_prefix)
    np.testing.assert_allclose(o.encode_prefix(z0[perm]), o.encode_prefix(z0)[perm], rtol=1e-11, atol=1e-12)


def test_action_invariant_to_prefix_order_and_equivariant_to_chunk_order():
    c = synth.config(0)
    W, _ = synth.make_weights(c, 2)
    o = oracle.Oracle(c, W)
    z0 = synth.make_prefix(c, 2)
    x0 = synth.make_noise(c, 2)
    base = o.run(z0, x0)
    pz = np.random.default_rng(1).permutation(c.n_prefix)
    np.testing.assert_allclose(o.run(z0[:, pz], x0), base, rtol=1e-11, atol=1e-12)
    px = np.random.default_rng(2).permutation(c.H)
    np.testing.assert_allclose(o.run(z0, x0[:, px]), base[:, px], rtol=1e-11, atol=1e-12)


def test_zero_linear_prefix_is_identity_plus_final_norm():
    c = synth.config(0)
    W, _ = synth.make_weights(c, 3)
    for n, _, kind in synth.weight_specs(c):
        if n.startswith("prefix.") and kind == "linear":
            W[n] = np.zeros_like(W[n])
    z0 = synth.make_prefix(c, 3)[0].astype(np.float64)
    want = oracle.rms_norm(z0, W["prefix.norm"], c.rms_eps)
    np.testing.assert_array_equal(oracle.Oracle(c, W).encode_prefix(z0), want)


def test_zero_sublayer_expert_is_embedding_head():
    c = synth.config(0)
    W, _ = synth.make_weights(c, 4)
    for e in range(c.L_e):
        for n in ("wos", "woc", "wd"):
            W[f"expert.{e}.{n}"] = np.zeros_like(W[f"expert.{e}.{n}"])
    o = oracle.Oracle(c, W)
    x = synth.make_noise(c, 4)[0].astype(np.float64)
    cache = o.cache_project(o.encode_prefix(synth.make_prefix(c, 4)[0]))
    e = x @ W["expert.w_in"].T.astype(np.float64) + oracle.time_embedding(0.3, c.d_e)
    want = oracle.rms_norm(e, W["expert.norm"], c.rms_eps) @ W["expert.w_out"].T.astype(np.float64)
    np.testing.assert_allclose(o.velocity(x, 0.3, cache), want, rtol=1e-13, atol=1e-15)


def test_zero_velocity_leaves_noise_unchanged_bitwise():
    c = synth.config(0)
    W, _ = synth.make_weights(c, 5)
    W["expert.w_out"] = np.zeros_like(W["expert.w_out"])
    z0, x0 = synth.make_prefix(c, 5), synth.make_noise(c, 5)
    np.testing.assert_array_equal(oracle.Oracle(c, W).run(z0, x0), x0.astype(np.float64))


def test_cached_equals_recompute_bitwise():
    c = synth.config(0)
    W, _ = synth.make_weights(c, 6)
    o = oracle.Oracle(c, W)
    z0, x0 = synth.make_prefix(c, 6)[0], synth.make_noise(c, 6)[0]
    sched = oracle.uniform_schedule(c.steps)
    cached = o.denoise(o.cache_project(o.encode_prefix(z0)), x0, sched)
    np.testing.assert_array_equal(cached, o.denoise_recompute(z0, x0, sched))


# ---------------------------------------------------------------- joint attention (pi0 form, §III-B)

JOINT = synth.config(0, name="tiny_joint_fp32", attn="joint", n_prefix=20, H=6)


def _masked_sequence_velocity(c, W, z0, x, tau):
    """v(x, tau) from ONE transformer pass over the joint sequence [prefix; chunk]: prefix
    rows use the backbone's weights, chunk rows the expert's, every layer attends over all
    N + H keys with the block mask (prefix queries see no chunk key), then the head.  Written
    out from the page's description of joint attention, independently of the oracle's cached
    form (which keeps per-layer prefix K/V and appends the chunk's)."""
    N, H = z0.shape[0], x.shape[0]
    mask = np.zeros((N + H, N + H))
    mask[:N, N:] = -np.inf
    f = lambda n: W[n].astype(np.float64)
    hp = z0.astype(np.float64)
    he = x @ f("expert.w_in").T + oracle.time_embedding(tau, c.d_e)
    for l in range(c.L_p):
        p, e = f"prefix.{l}.", f"expert.{l}."
        up, ue = oracle.rms_norm(hp, f(p + "w1"), c.rms_eps), oracle.rms_norm(he, f(e + "a1"), c.rms_eps)
        q = np.concatenate([up @ f(p + "wq").T, ue @ f(e + "wqs").T])
        k = np.concatenate([up @ f(p + "wk").T, ue @ f(e + "wks").T])
        v = np.concatenate([up @ f(p + "wv").T, ue @ f(e + "wvs").T])
        o = oracle.attention(q, k, v, c.Hq, c.Hkv, c.hd, mask=mask)
        hp = hp + o[:N] @ f(p + "wo").T
        he = he + o[N:] @ f(e + "wos").T
        up, ue = oracle.rms_norm(hp, f(p + "w2"), c.rms_eps), oracle.rms_norm(he, f(e + "a3"), c.rms_eps)
        hp = hp + (oracle.gelu(up @ f(p + "wg").T) * (up @ f(p + "wu").T)) @ f(p + "wd").T
        he = he + (oracle.gelu(ue @ f(e + "wg").T) * (ue @ f(e + "wu").T)) @ f(e + "wd").T
    return oracle.rms_norm(he, f("expert.norm"), c.rms_eps) @ f("expert.w_out").T


def test_joint_cache_equals_block_masked_sequence():
    """The cached joint form (per-layer prefix K/V, chunk keys appended) equals one masked pass
    over the whole sequence, for every solver time: pins the cache contents (each layer's own
    pre-attention keys and values), the concatenation and the joint layer's structure."""
    c = JOINT
    W, _ = synth.make_weights(c, 11)
    z0, x = synth.make_prefix(c, 11)[0], synth.make_noise(c, 11)[0].astype(np.float64)
    o = oracle.Oracle(c, W)
    cache = o.conditioning(z0)
    assert len(cache) == c.L_p and cache[0][0].shape == (c.n_prefix, c.Hkv * c.hd)
    for tau in (0.0, 0.37, 1.0):
        np.testing.assert_allclose(o.velocity(x, tau, cache), _masked_sequence_velocity(c, W, z0, x, tau),
                                   rtol=1e-11, atol=1e-13)


def test_joint_cache_is_each_layers_own_keys_and_values():
    c = JOINT
    W, _ = synth.make_weights(c, 12)
    o = oracle.Oracle(c, W)
    z0 = synth.make_prefix(c, 12)[0].astype(np.float64)
    cache = o.prefix_kv(z0)
    h = z0
    for l in range(c.L_p):
        u = oracle.rms_norm(h, W[f"prefix.{l}.w1"], c.rms_eps)
        np.testing.assert_array_equal(cache[l][0], u @ W[f"prefix.{l}.wk"].astype(np.float64).T)
        np.testing.assert_array_equal(cache[l][1], u @ W[f"prefix.{l}.wv"].astype(np.float64).T)
        h = o.prefix_layer(h, l)


def test_joint_attention_merges_prefix_and_chunk_softmaxes():
    """Attention over [prefix keys; chunk keys] is the log-sum-exp merge of the two separate
    attentions (one softmax over both sets, not two)."""
    rng = np.random.default_rng(13)
    hd, n, h = 32, 9, 5
    q = rng.standard_normal((4, 2 * hd))
    kp, vp = rng.standard_normal((n, hd)), rng.standard_normal((n, hd))
    ks, vs = rng.standard_normal((h, hd)), rng.standard_normal((h, hd))
    joint = oracle.attention(q, np.concatenate([kp, ks]), np.concatenate([vp, vs]), 2, 1, hd)
    for j in range(2):
        qj = q[:, j * hd:(j + 1) * hd] / math.sqrt(hd)
        sp, ss = qj @ kp.T, qj @ ks.T
        m = np.maximum(sp.max(1), ss.max(1))[:, None]
        ap, as_ = np.exp(sp - m), np.exp(ss - m)
        want = (ap @ vp + as_ @ vs) / (ap.sum(1) + as_.sum(1))[:, None]
        np.testing.assert_allclose(joint[:, j * hd:(j + 1) * hd], want, rtol=1e-12, atol=1e-14)


def test_joint_cached_equals_recompute_and_zero_velocity():
    c = JOINT
    W, _ = synth.make_weights(c, 14)
    o = oracle.Oracle(c, W)
    z0, x0 = synth.make_prefix(c, 14)[0], synth.make_noise(c, 14)[0]
    sched = oracle.uniform_schedule(c.steps)
    np.testing.assert_array_equal(o.denoise(o.conditioning(z0), x0, sched), o.denoise_recompute(z0, x0, sched))
    W["expert.w_out"] = np.zeros_like(W["expert.w_out"])
    np.testing.assert_array_equal(oracle.Oracle(c, W).run(z0[None], x0[None])[0], x0.astype(np.float64))


def test_joint_weight_order_has_no_cross_attention_or_projection():
    names = [n for n, _, _ in synth.weight_specs(JOINT)]
    assert not any(n.startswith("cache.") or n == "prefix.norm" for n in names)
    assert not any(n.endswith((".a2", ".wqc", ".woc")) for n in names)
    assert len(names) == len(synth.weight_specs(synth.config(0))) - 1 - 2 * JOINT.L_e - 3 * JOINT.L_e


def test_float32_vs_float64_self_consistency():
    c = synth.config(0)
    W, _ = synth.make_weights(c, 7)
    z0, x0 = synth.make_prefix(c, 7), synth.make_noise(c, 7)
    a64 = oracle.Oracle(c, W, dtype=np.float64).run(z0, x0)
    a32 = oracle.Oracle(c, W, dtype=np.float32).run(z0, x0)
    assert oracle.e_rel(a32, a64) < 1e-5
    d64, d32 = a64 - x0, a32 - x0
    assert oracle.e_rel(d32, d64) < 1e-4


# ---------------------------------------------------------------- ternary, Eq. 4

def test_quantizer_golden():
    g = golden("quantizer_eq4.json")
    for c in g["cases"]:
        a, alpha = oracle.quantize_rows(np.array([c["x"]], dtype=np.float32))
        want_alpha = (np.float32(1e-5) / np.float32(127)) if isinstance(c["alpha"], str) else c["alpha"]
        assert alpha.dtype == np.float32 and alpha[0] == np.float32(want_alpha)
        assert a.dtype == np.int8 and a[0].tolist() == c["a"]


def test_quantizer_invariants():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((64, 96)) * rng.uniform(1e-4, 50, (64, 1))).astype(np.float32)
    x[3] = 0.0
    a, alpha = oracle.quantize_rows(x)
    assert np.abs(a.astype(int)).max() <= 127
    big = np.abs(x).max(axis=1) >= 1e-5
    assert np.all(np.abs(a[big].astype(int)).max(axis=1) == 127)
    assert np.all(a[3] == 0)
    # reconstruction error at most half a step per entry
    assert np.all(np.abs(a * alpha[:, None] - x) <= 0.5 * alpha[:, None] * (1 + 1e-6))


def test_quantizer_ties_to_even():
    x = np.array([[127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5]], dtype=np.float32)
    a, _ = oracle.quantize_rows(x)
    assert a[0].tolist() == [127, 0, 2, 2, 0, -2, -2, 126]


def test_int32_accumulator_brute_force_and_special_cases():
    rng = np.random.default_rng(9)
    a = rng.integers(-128, 128, (5, 12), dtype=np.int8)
    q = rng.integers(-1, 2, (7, 12), dtype=np.int8)
    want = [[sum(int(a[m, j]) * int(q[n, j]) for j in range(12)) for n in range(7)] for m in range(5)]
    got = oracle.w2a8_accumulate(a, q)
    assert got.dtype == np.int32 and got.tolist() == want
    ones = np.ones((3, 12), dtype=np.int8)
    assert oracle.w2a8_accumulate(a, ones).tolist() == [[int(r.astype(int).sum())] * 3 for r in a]
    eye = np.eye(12, dtype=np.int8)
    assert oracle.w2a8_accumulate(a, eye).tolist() == a.astype(int).tolist()


def test_int32_accumulator_exact_at_large_k():
    rng = np.random.default_rng(10)
    K = 6912
    a = rng.integers(-127, 128, (4, K), dtype=np.int8)
    a[0] = 127
    q = rng.integers(-1, 2, (5, K), dtype=np.int8)
    q[0] = 1
    want = a.astype(np.int64) @ q.astype(np.int64).T
    np.testing.assert_array_equal(oracle.w2a8_accumulate(a, q), want)


def test_w2a8_linear_composition():
    rng = np.random.default_rng(15)
    x = rng.standard_normal((6, 16)).astype(np.float32)
    q = rng.integers(-1, 2, (5, 16), dtype=np.int8)
    beta = 0.0137
    y = oracle.w2a8_linear(x, q, beta)
    for m in range(6):
        am = float(np.max(np.abs(x[m])))
        alpha = np.float32(max(am, np.float32(1e-5))) / np.float32(127)
        codes = [max(-128, min(127, int(np.rint(np.float32(v) / alpha)))) for v in x[m]]
        for n in range(5):
            acc = sum(cd * int(qq) for cd, qq in zip(codes, q[n]))
            s = np.float32(alpha * np.float32(beta))
            ref = torch.tensor(float(np.float32(np.float32(acc) * s))).to(torch.bfloat16).item()
            assert y[m, n] == np.float32(ref)


def test_w2a8_grouped_scales():
    """Group-wise beta_g(n): element by element in plain Python, torch's bf16 cast as the rounding
    reference; one group over all channels is the per-tensor form."""
    rng = np.random.default_rng(16)
    x = rng.standard_normal((5, 32)).astype(np.float32)
    q = rng.integers(-1, 2, (8, 32), dtype=np.int8)
    betas = np.array([0.011, 0.023, 0.0071, 0.05], dtype=np.float32)
    y = oracle.w2a8_linear_grouped(x, q, betas, 2)
    a, alpha = oracle.quantize_rows(x)
    for m in range(5):
        for n in range(8):
            acc = int(sum(int(u) * int(v) for u, v in zip(a[m], q[n])))
            s = np.float32(alpha[m] * betas[n // 2])
            ref = torch.tensor(float(np.float32(np.float32(acc) * s))).to(torch.bfloat16).item()
            assert y[m, n] == np.float32(ref)
    np.testing.assert_array_equal(oracle.w2a8_linear_grouped(x, q, betas[:1], 8), oracle.w2a8_linear(x, q, betas[0]))


def test_pack_golden_roundtrip_and_invalid_code():
    g = golden("ternary_pack.json")
    q = np.array(g["q"], dtype=np.int8)
    assert oracle.pack_ternary(q).tolist() == g["packed"]
    rng = np.random.default_rng(16)
    q = rng.integers(-1, 2, (9, 40), dtype=np.int8)
    np.testing.assert_array_equal(oracle.unpack_ternary(oracle.pack_ternary(q)), q)
    with pytest.raises(ValueError):
        oracle.unpack_ternary(np.array([[0b11000000]], dtype=np.uint8))
    with pytest.raises(ValueError):
        oracle.pack_ternary(np.zeros((1, 6), dtype=np.int8))


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(17)
    x = (rng.standard_normal(100000) * 10.0 ** rng.uniform(-30, 30, 100000)).astype(np.float32)
    # exact ties: halfway between two bfloat16 values
    ties = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 3.0e38, 1e-40], dtype=np.float32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(oracle.bf16_round(x), ref)


# ------------------------------------------------------------------ metrics, Eq. 5

def test_metrics_golden():
    for c in golden("metrics_eq5.json")["cases"]:
        assert oracle.e_inf(c["a"], c["ref"]) == c["e_inf"]
        assert abs(oracle.e_rel(c["a"], c["ref"]) - c["e_rel"]) < 1e-15


# ---------------------------------------------------------------- ternary workload

def test_ternary_prefix_layer_uses_w2a8_every_linear():
    c = tiny_cfg(precision="w2a8", d_p=8, Hq=2, Hkv=2, hd=4, F_p=8)
    W, betas = synth.make_weights(c, 18)
    assert W["prefix.0.wq"].dtype == np.int8
    o = oracle.Oracle(c, W, betas)
    h = synth.make_prefix(c, 18)[0].astype(np.float64)
    # brute force with the Eq. 4 linear written out per element
    def lin(x, name):
        return oracle.w2a8_linear(np.asarray(x, np.float32), W[name], betas[name]).astype(np.float64).tolist()
    p = "prefix.0."
    u = bf_rms(L(h), L(W[p + "w1"]), c.rms_eps)
    q, k, v = lin(u, p + "wq"), lin(u, p + "wk"), lin(u, p + "wv")
    hh = bf_add(L(h), lin(bf_attention(q, k, v, c.Hq, c.Hkv, c.hd), p + "wo"))
    u = bf_rms(hh, L(W[p + "w2"]), c.rms_eps)
    g, up = lin(u, p + "wg"), lin(u, p + "wu")
    m = [[bf_gelu(a) * b for a, b in zip(r, s)] for r, s in zip(g, up)]
    want = bf_add(hh, lin(m, p + "wd"))
    np.testing.assert_allclose(o.prefix_layer(h, 0), want, rtol=1e-6, atol=1e-6)


# ------------------------------------------------------------ seeded generator

def test_generator_is_deterministic_and_per_tensor():
    c = synth.config(0)
    w1, _ = synth.make_weights(c, 3)
    w2, _ = synth.make_weights(c, 3, workers=1)
    for n in w1:
        np.testing.assert_array_equal(w1[n], w2[n])
    np.testing.assert_array_equal(synth.make_noise(c, 3), synth.make_noise(c, 3))
    assert not np.array_equal(synth.make_noise(c, 3), synth.make_noise(c, 4))
    cb = synth.config(1)
    names = [s[0] for s in synth.weight_specs(cb)]
    assert len(names) == len(set(names)) == 18 * 9 + 1 + 36 + 1 + 18 * 12 + 2
