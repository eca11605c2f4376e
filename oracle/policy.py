"""Dual-phase policy step, written out plainly in numpy -- test infrastructure only.

"The paper" is *vla.cpp: A Unified Inference Runtime for Vision-Language-Action
Models* (arXiv 2606.08094); "the reading notes" are the paper.gecl.asia notes on it.

One observation at a time:

1. Prefix (the reading notes, Method points 1-2: image, text and state tokens
   attend to each other freely, and the action head reads the final hidden
   states taken before any LM output projection).  h <- Z0; for every layer:
       u = RMS(h; w1);  Q, K, V = u Wq^T, u Wk^T, u Wv^T
       h = h + Attn(Q, K, V; M = 0) Wo^T
       u = RMS(h; w2);  h = h + (GELU(u Wg^T) * (u Wu^T)) Wd^T
   and Z = RMS(h; w_final).
2. Cache (the paper, §III-B, Eq. 2): for every expert layer e,
   K_C^e = Z Wk_e^T and V_C^e = Z Wv_e^T, computed once per observation.
3. Denoise (the paper, §III-A, Eq. 1): X^{k+1} = X^k + (tau_{k+1} - tau_k) v(X^k, tau_k)
   for k = 0..T-1, with v(X, tau) the action expert:
       E = X W_in^T + phi(tau)                    (phi added to every chunk token)
       for every expert layer:
           E = E + SelfAttn(RMS(E; a1)) over the H chunk tokens (M = 0)
           E = E + Attn(RMS(E; a2) Wqc^T, K_C^e, V_C^e; M = 0) Woc^T
           E = E + GeGLU(RMS(E; a3))
       v = RMS(E; w_final) W_out^T

Joint attention (the paper, §III-B: pi0 caches every layer's prefix keys and
values, and joint-attention layers append the suffix's keys and values) is the
other cache form.  The cache is the keys and values each prefix layer computes
for itself, [(K_l, V_l)], with no final norm and no projection; expert layer l
has one attention sublayer, whose keys are prefix layer l's followed by the
chunk's own, in one softmax, then the MLP:
           u = RMS(E; a1);  Q, K, V = u Wqs^T, u Wks^T, u Wvs^T
           E = E + Attn(Q, [K_l; K], [V_l; V]; M = 0) Wos^T
           E = E + GeGLU(RMS(E; a3))
Prefix tokens never see the chunk (their keys and values come from the prefix
pass alone): the block mask of the joint sequence.

Key padding (the paper, §III-B, Eq. 2: M is 0 for visible keys and -inf for
masked ones, and adapters keep each model's masks): an observation may fill
only its first n of the N prefix positions.  Its keys past n then get M = -inf
in every softmax that reads prefix keys -- the prefix's own attention, the
cross-attention into its cache and the prefix part of joint attention -- so a
padded observation gives the same chunk as the same observation run at length
n, whatever the (finite) padding holds.  Padded query rows are computed and
never read.

Readings where the pages are silent (the pages name none of these pieces):
  * RMS(x; w) = x / sqrt(mean(x^2) + eps) * (1 + w), pre-norm before every
    sublayer, eps = 1e-6;
  * GELU is the exact erf form, 0.5 x (1 + erf(x / sqrt 2));
  * phi is the sinusoidal embedding with position tau: phi_{2i} =
    sin(tau / 10000^(2i/d)), phi_{2i+1} = cos(tau / 10000^(2i/d));
  * no positional encoding anywhere, no biases, all masks M = 0;
  * query head j reads key/value head floor(j * Hkv / Hq);
  * linear weights are [out, in]: y = x W^T;
  * default schedule: uniform from tau = 0 to tau = 1 (the paper's GR00T-style
    direction), tau_k = tau_start + k (tau_end - tau_start) / T.

In the ternary workload every prefix linear is the W2A8 linear of §III-D (see
ternary.py); attention, norms, the cache projection and the expert stay dense.
"""
from __future__ import annotations

import math
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np
from scipy.special import erf

from .ternary import w2a8_linear


# --------------------------------------------------------------------------- parts

def rms_norm(x, w, eps):
    """x / sqrt(mean(x^2) + eps) * (1 + w), over the last axis."""
    x = np.asarray(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * (1.0 + np.asarray(w, dtype=x.dtype))


def gelu(x):
    """Exact GELU: 0.5 x (1 + erf(x / sqrt(2)))."""
    x = np.asarray(x)
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def linear(x, w):
    """y = x W^T with W stored [out, in]."""
    return x @ np.asarray(w, dtype=x.dtype).T


def attention(q, k, v, n_heads: int, n_kv_heads: int, head_dim: int, mask=None):
    """Multi-head softmax(Q K^T / sqrt(d_k) + M) V -- the paper, §III-B, Eq. 2.

    q: [Nq, n_heads * head_dim]; k, v: [Nk, n_kv_heads * head_dim]; query head j
    uses key/value head floor(j * n_kv_heads / n_heads).  mask, if given, is an
    additive [Nq, Nk] array (0 for visible keys, -inf for masked ones).  Softmax
    runs over the keys.  Returns [Nq, n_heads * head_dim].
    """
    q = np.asarray(q)
    out = np.empty((q.shape[0], n_heads * head_dim), dtype=q.dtype)
    scale = 1.0 / math.sqrt(head_dim)
    for j in range(n_heads):
        g = (j * n_kv_heads) // n_heads
        qj = q[:, j * head_dim:(j + 1) * head_dim]
        kj = k[:, g * head_dim:(g + 1) * head_dim]
        vj = v[:, g * head_dim:(g + 1) * head_dim]
        s = (qj @ kj.T) * scale
        if mask is not None:
            s = s + mask
        s = s - np.max(s, axis=-1, keepdims=True)
        p = np.exp(s)
        p = p / np.sum(p, axis=-1, keepdims=True)
        out[:, j * head_dim:(j + 1) * head_dim] = p @ vj
    return out


def key_mask(n_valid: Optional[int], n_keys: int, n_extra: int = 0):
    """Additive key mask of Eq. 2 for an observation whose first n_valid of n_keys prefix keys are
    real: a [1, n_keys + n_extra] row, 0 for visible keys and -inf past n_valid; the n_extra keys
    appended after the prefix's (the chunk's own, in joint attention) stay visible.  None when
    every key is visible (n_valid is None or n_keys)."""
    if n_valid is None or n_valid >= n_keys:
        return None
    if n_valid < 1:
        raise ValueError("an observation needs at least one visible prefix key")
    m = np.zeros((1, n_keys + n_extra), dtype=np.float64)
    m[0, n_valid:n_keys] = -np.inf
    return m


def time_embedding(tau: float, d: int, dtype=np.float64):
    """Sinusoidal embedding of the solver time tau, interleaved (sin, cos) pairs."""
    i = np.arange(d // 2, dtype=np.float64)
    freq = 10000.0 ** (-2.0 * i / d)
    phi = np.empty(d, dtype=np.float64)
    phi[0::2] = np.sin(tau * freq)
    phi[1::2] = np.cos(tau * freq)
    return phi.astype(dtype)


def uniform_schedule(steps: int, tau_start: float = 0.0, tau_end: float = 1.0):
    """tau_0..tau_T with tau_k = tau_start + k (tau_end - tau_start) / T."""
    dt = (tau_end - tau_start) / steps
    return np.array([tau_start + k * dt for k in range(steps + 1)], dtype=np.float64)


def euler_integrate(x0, schedule: Sequence[float],
                    vfield: Callable[[np.ndarray, float], np.ndarray]):
    """Eq. 1 of the paper's §III-A: X^{k+1} = X^k + (tau_{k+1} - tau_k) v(X^k, tau_k)."""
    x = np.array(x0, copy=True)
    for k in range(len(schedule) - 1):
        x = x + (schedule[k + 1] - schedule[k]) * vfield(x, schedule[k])
    return x


# --------------------------------------------------------------------------- model

class Oracle:
    """The policy of one workload, evaluated in `dtype` (float64 by default).

    cfg is any object with the workload's fields (precision, d_p, L_p, Hq, Hkv,
    hd, d_e, L_e, Hq_e, Hkv_e, hd_e, rms_eps, ...).  weights maps tensor names to
    arrays (linear weights [out, in]; ternary tensors as codes in {-1, 0, 1});
    betas maps each ternary tensor to its fp32 scale.
    """

    def __init__(self, cfg, weights: Dict[str, np.ndarray],
                 betas: Optional[Dict[str, float]] = None, dtype=np.float64):
        self.cfg = cfg
        self.W = weights
        self.betas = betas or {}
        self.dtype = dtype
        self._expert_cache: Dict[str, np.ndarray] = {}

    # weights converted to the working precision
    def _w(self, name):
        return np.asarray(self.W[name], dtype=self.dtype)

    def _we(self, name):  # expert weights are reused every step: convert once
        w = self._expert_cache.get(name)
        if w is None:
            w = self._expert_cache[name] = np.asarray(self.W[name], dtype=self.dtype)
        return w

    def _plin(self, x, name):
        """A prefix linear: dense, or W2A8 (the paper, §III-D, Eq. 4) when ternary."""
        if self.cfg.precision == "w2a8":
            y = w2a8_linear(np.asarray(x, dtype=np.float32), self.W[name], self.betas[name])
            return y.astype(self.dtype)
        return x @ self._w(name).T

    def is_joint(self) -> bool:
        return getattr(self.cfg, "attn", "cross") == "joint"

    # ---- phase 1: prefix
    def prefix_layer_kv(self, h, l: int, n_valid: Optional[int] = None):
        """One prefix layer: (its output, its keys K, its values V); keys past n_valid are masked."""
        c, p = self.cfg, f"prefix.{l}."
        u = rms_norm(h, self._w(p + "w1"), c.rms_eps)
        q = self._plin(u, p + "wq")
        k = self._plin(u, p + "wk")
        v = self._plin(u, p + "wv")
        mask = key_mask(n_valid, np.shape(h)[0])
        h = h + self._plin(attention(q, k, v, c.Hq, c.Hkv, c.hd, mask), p + "wo")
        u = rms_norm(h, self._w(p + "w2"), c.rms_eps)
        m = gelu(self._plin(u, p + "wg")) * self._plin(u, p + "wu")
        return h + self._plin(m, p + "wd"), k, v

    def prefix_layer(self, h, l: int, n_valid: Optional[int] = None):
        return self.prefix_layer_kv(h, l, n_valid)[0]

    def prefix_kv(self, z0, n_valid: Optional[int] = None) -> List[Tuple[np.ndarray, np.ndarray]]:
        """Joint-attention cache: [(K_l, V_l)] of every prefix layer, each [N, Hkv * hd]."""
        h = np.asarray(z0, dtype=self.dtype)
        kv = []
        for l in range(self.cfg.L_p):
            h, k, v = self.prefix_layer_kv(h, l, n_valid)
            kv.append((k, v))
        return kv

    def encode_prefix(self, z0, n_valid: Optional[int] = None):
        """Z = RMS(h_L; w_final) for one observation's prefix z0 [N, d_p] (first n_valid rows real)."""
        h = np.asarray(z0, dtype=self.dtype)
        for l in range(self.cfg.L_p):
            h = self.prefix_layer(h, l, n_valid)
        return rms_norm(h, self._w("prefix.norm"), self.cfg.rms_eps)

    # ---- phase 2: cache
    def cache_project(self, z) -> List[Tuple[np.ndarray, np.ndarray]]:
        """[(K_C^e, V_C^e)] for every expert layer e, each [N, Hkv_e * hd_e]."""
        return [(z @ self._w(f"cache.{e}.wk").T, z @ self._w(f"cache.{e}.wv").T)
                for e in range(self.cfg.L_e)]

    def conditioning(self, z0, n_valid: Optional[int] = None):
        """The cached collection for one observation: projected final states, or per-layer prefix K/V."""
        if self.is_joint():
            return self.prefix_kv(z0, n_valid)
        return self.cache_project(self.encode_prefix(z0, n_valid))

    # ---- phase 3: expert and solver
    def velocity(self, x, tau: float, cache, n_valid: Optional[int] = None):
        """v(X, tau); cached prefix keys past n_valid are masked."""
        c = self.cfg
        W = self._we
        e_ = x @ W("expert.w_in").T + time_embedding(tau, c.d_e, self.dtype)[None, :]
        for e in range(c.L_e):
            p = f"expert.{e}."
            u = rms_norm(e_, W(p + "a1"), c.rms_eps)
            q, k, v = u @ W(p + "wqs").T, u @ W(p + "wks").T, u @ W(p + "wvs").T
            mask = None
            if self.is_joint():
                kp, vp = cache[e]  # prefix layer e's keys and values, then the chunk's
                mask = key_mask(n_valid, kp.shape[0], k.shape[0])
                k, v = np.concatenate([kp, k]), np.concatenate([vp, v])
            e_ = e_ + attention(q, k, v, c.Hq_e, c.Hkv_e, c.hd_e, mask) @ W(p + "wos").T
            if not self.is_joint():
                u = rms_norm(e_, W(p + "a2"), c.rms_eps)
                kc, vc = cache[e]
                e_ = e_ + attention(u @ W(p + "wqc").T, kc, vc, c.Hq_e, c.Hkv_e,
                                    c.hd_e, key_mask(n_valid, kc.shape[0])) @ W(p + "woc").T
            u = rms_norm(e_, W(p + "a3"), c.rms_eps)
            e_ = e_ + (gelu(u @ W(p + "wg").T) * (u @ W(p + "wu").T)) @ W(p + "wd").T
        return rms_norm(e_, W("expert.norm"), c.rms_eps) @ W("expert.w_out").T

    def denoise(self, cache, x0, schedule, n_valid: Optional[int] = None):
        """X^T from X^0 [H, d_a] with the cache computed once (the cached mode)."""
        return euler_integrate(np.asarray(x0, dtype=self.dtype), schedule,
                               lambda x, tau: self.velocity(x, tau, cache, n_valid))

    def denoise_recompute(self, z0, x0, schedule, n_valid: Optional[int] = None):
        """Same result, re-encoding the prefix and re-projecting the cache every step."""
        def v(x, tau):
            return self.velocity(x, tau, self.conditioning(z0, n_valid), n_valid)
        return euler_integrate(np.asarray(x0, dtype=self.dtype), schedule, v)

    def run(self, z0, x0, schedule=None, keep_cache: bool = False, lengths=None):
        """Whole step for a batch: z0 [B, N, d_p], x0 [B, H, d_a] -> X^T [B, H, d_a].

        lengths (optional, [B]): observation b fills its first lengths[b] prefix positions."""
        if schedule is None:
            schedule = uniform_schedule(self.cfg.steps)
        outs, caches = [], []
        for b in range(np.shape(z0)[0]):
            n = None if lengths is None else int(lengths[b])
            cache = self.conditioning(z0[b], n)
            outs.append(self.denoise(cache, x0[b], schedule, n))
            if keep_cache:
                caches.append(cache)
        out = np.stack(outs)
        return (out, caches) if keep_cache else out


# --------------------------------------------------------------- functional forms

def prefix_layer(cfg, weights, h, l, betas=None, dtype=np.float64):
    return Oracle(cfg, weights, betas, dtype).prefix_layer(np.asarray(h, dtype=dtype), l)


def encode_prefix(cfg, weights, z0, betas=None, dtype=np.float64):
    return Oracle(cfg, weights, betas, dtype).encode_prefix(z0)


def cache_project(cfg, weights, z, dtype=np.float64):
    return Oracle(cfg, weights, None, dtype).cache_project(np.asarray(z, dtype=dtype))


def velocity(cfg, weights, x, tau, cache, dtype=np.float64):
    return Oracle(cfg, weights, None, dtype).velocity(np.asarray(x, dtype=dtype), tau, cache)


def denoise(cfg, weights, cache, x0, schedule=None, dtype=np.float64):
    if schedule is None:
        schedule = uniform_schedule(cfg.steps)
    return Oracle(cfg, weights, None, dtype).denoise(cache, x0, schedule)


def denoise_recompute(cfg, weights, z0, x0, schedule=None, betas=None, dtype=np.float64):
    if schedule is None:
        schedule = uniform_schedule(cfg.steps)
    return Oracle(cfg, weights, betas, dtype).denoise_recompute(z0, x0, schedule)


def run_policy(cfg, weights, z0, x0, betas=None, schedule=None, dtype=np.float64):
    return Oracle(cfg, weights, betas, dtype).run(z0, x0, schedule)
