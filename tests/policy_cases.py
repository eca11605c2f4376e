"""Shared helpers of the GPU parity tests: workloads, device inputs, oracle runs."""
from __future__ import annotations

import functools
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

# Small workloads that still span several tiles and ragged tails of every kernel.
SMALL_BF16 = synth.config(1, name="small_bf16", n_prefix=100, d_p=256, L_p=2, Hq=4, Hkv=1, hd=64, F_p=512,
                          d_e=128, L_e=2, Hq_e=2, Hkv_e=1, hd_e=64, F_e=256, H=20, d_a=7, steps=3)
SMALL_BF16_B3 = synth.config(1, name="small_bf16_b3", batch=3, n_prefix=70, d_p=256, L_p=2, Hq=8, Hkv=1, hd=128,
                             F_p=512, d_e=128, L_e=2, Hq_e=8, Hkv_e=1, hd_e=128, F_e=256, H=33, d_a=5, steps=2)
# Grouped heads on both sides (two KV heads per layer), a prefix that is not a
# whole number of 32-key tiles, and a chunk of three 16-row blocks.
SMALL_GQA = synth.config(1, name="small_gqa", n_prefix=90, d_p=256, L_p=2, Hq=4, Hkv=2, hd=64, F_p=512,
                         d_e=192, L_e=2, Hq_e=4, Hkv_e=2, hd_e=64, F_e=256, H=40, d_a=16, steps=2)
# Joint attention (per-layer prefix K/V, the pi0 form) at the same small shapes.
JOINT_F32 = synth.config(0, name="tiny_joint_fp32", attn="joint", n_prefix=40, H=6)
SMALL_JOINT = synth.config(1, name="small_joint_bf16", attn="joint", n_prefix=100, d_p=256, L_p=2, Hq=4, Hkv=1,
                           hd=64, F_p=512, d_e=128, L_e=2, Hq_e=2, Hkv_e=1, hd_e=64, F_e=256, H=20, d_a=7, steps=3)
SMALL_JOINT_GQA = synth.config(1, name="small_joint_gqa", attn="joint", n_prefix=90, d_p=256, L_p=2, Hq=4, Hkv=2,
                               hd=64, F_p=512, d_e=192, L_e=2, Hq_e=4, Hkv_e=2, hd_e=64, F_e=256, H=40, d_a=16, steps=2)
SMALL_JOINT_B3 = synth.config(1, name="small_joint_b3", attn="joint", batch=3, n_prefix=70, d_p=256, L_p=2, Hq=8,
                              Hkv=1, hd=128, F_p=512, d_e=128, L_e=2, Hq_e=8, Hkv_e=1, hd_e=128, F_e=256, H=33, d_a=5,
                              steps=2)
# Enough query rows (8 observations x 8 heads x 260 tokens: 1040 16-row blocks) and keys (9 tiles, the last
# ragged) for the prefix attention's 64-row workgroups sharing key tiles through LDS.
SMALL_ROWS = synth.config(1, name="small_rows_b8", batch=8, n_prefix=260, d_p=256, L_p=2, Hq=8, Hkv=1, hd=64,
                          F_p=512, d_e=128, L_e=2, Hq_e=2, Hkv_e=1, hd_e=64, F_e=256, H=20, d_a=7, steps=2)
SMALL_W2A8 = synth.config(4, name="small_w2a8", n_prefix=100, d_p=256, L_p=2, Hq=2, Hkv=2, hd=128, F_p=384,
                          d_e=128, L_e=2, Hq_e=2, Hkv_e=1, hd_e=64, F_e=256, H=8, d_a=7, steps=3)


def ordered(cfg, weights):
    return [weights[name] for name, _, _ in synth.weight_specs(cfg)]


def ordered_betas(cfg, betas):
    return [betas[name] for name, _, kind in synth.weight_specs(cfg) if kind == "ternary"] or None


@functools.lru_cache(maxsize=4)
def host_inputs(cfg, seed):
    w, b = synth.make_weights(cfg, seed)
    return w, b, synth.make_prefix(cfg, seed), synth.make_noise(cfg, seed)


def build_model(cfg, weights, betas, env=None):
    """A model on the GPU; `env` ({name: value}) is set in the environment while it is created (the
    library reads VLA_FUSED and VLA_FOLD there)."""
    from prefix_cache_flow_amd import vla
    old = {k: os.environ.get(k) for k in (env or {})}
    os.environ.update(env or {})
    try:
        tensors = vla.upload_weights(cfg.to_dict(), ordered(cfg, weights))
        model = vla.vla_model_create(cfg.to_dict(), tensors, ordered_betas(cfg, betas))
        del tensors
    finally:
        for k, v in old.items():
            if v is None:
                del os.environ[k]
            else:
                os.environ[k] = v
    return model


def gpu_run(cfg, model, z0, x0, steps=None, out_dtype=None, schedule=None):
    """Encode + denoise on the GPU; returns (X^T as float64 numpy, cache storage tensor)."""
    import torch
    from prefix_cache_flow_amd import vla
    zt = torch.from_numpy(np.ascontiguousarray(z0)).cuda()
    xt = torch.from_numpy(np.ascontiguousarray(x0)).cuda()
    kv = vla.vla_prefix_encode(model, zt)
    out = vla.vla_denoise_chunk(model, kv, xt, steps or cfg.steps, schedule=schedule,
                                out_dtype=out_dtype or torch.float32)
    torch.cuda.synchronize()
    res = out.float().cpu().numpy().astype(np.float64)
    storage = kv.storage
    kv.close()
    return res, storage


def _cache_index_maps(N, hd):
    """Positions of (t, d) inside one bf16 K block and one V block (the layout vla.h states)."""
    t = np.arange(N)[:, None]
    d = np.arange(hd)[None, :]
    kpos = ((((t // 16) * (hd // 32) + d // 32) * 64 + t % 16 + 16 * ((d // 8) % 4)) * 8 + d % 8)
    u = t % 32
    vpos = ((((t // 32) * (hd // 16) + d // 16) * 64 + d % 16 + 16 * ((u % 16) // 4)) * 8 + 4 * (u // 16) + u % 4)
    return kpos, vpos


def cache_from_storage(cfg, storage, B, N):
    """Cache storage -> per observation list of (K_C, V_C), each [N, Hkv_e*hd_e] float64.

    fp32 caches are plain rows; bf16 caches hold 32-row-padded blocks in the MFMA operand orders.
    """
    import torch
    f32 = cfg.precision == "f32"
    dt = torch.float32 if f32 else torch.bfloat16
    Np = N if f32 else (N + 31) // 32 * 32
    t = storage.view(dt)[: B * cfg.L_e * 2 * cfg.Hkv_e * Np * cfg.hd_e].float().cpu().numpy()
    t = t.reshape(B, cfg.L_e, 2, cfg.Hkv_e, Np * cfg.hd_e)
    if f32:
        kpos = vpos = (np.arange(N)[:, None] * cfg.hd_e + np.arange(cfg.hd_e)[None, :])
    else:
        kpos, vpos = _cache_index_maps(N, cfg.hd_e)
    out = []
    for b in range(B):
        layers = []
        for e in range(cfg.L_e):
            k = t[b, e, 0][:, kpos].transpose(1, 0, 2).reshape(N, cfg.Hkv_e * cfg.hd_e)
            v = t[b, e, 1][:, vpos].transpose(1, 0, 2).reshape(N, cfg.Hkv_e * cfg.hd_e)
            layers.append((k.astype(np.float64), v.astype(np.float64)))
        out.append(layers)
    return out