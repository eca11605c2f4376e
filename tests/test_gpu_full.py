"""Parity at the full workload sizes, through the same library calls the benchmark times.

Each test builds the workload's seeded weights and inputs, runs the prefix
encode and the denoise on the GPU, and compares with the float64 oracle on the
same inputs: Eq. 5's relative error (the paper, §III-E) on the bf16 action chunk
within 2e-2, plus bounds on the displacement X^T - X^0 and on the K/V cache.
The batched workload runs all 16 observations on the GPU and checks a sample of
them against the oracle (observations are independent); every batched case is
also run with its observations in reverse order, which must give the same
chunks and caches bit for bit, reversed (no observation's result depends on
its position or its neighbours).
"""
import gc
import time

import numpy as np
import pytest

import oracle
import synth
from policy_cases import build_model, cache_from_storage

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from prefix_cache_flow_amd import vla  # noqa: E402

# (workload index, bound on e_rel(D), bound on the cache's e_rel, observations the oracle checks)
# A CPU emulation of this library's bf16 rounding points at the single-camera
# shapes gives e_rel(X^T) 1.3e-3, e_rel(D) 2.6e-3 and a cache e_rel of 1.08e-2
# (bf16 activations through 18 layers); the bounds leave about 2x-4x margin.
# The ternary prefix is far more sensitive: its int8 codes flip when the last
# bits of an activation move across a rounding boundary, and the flips compound
# over 30 layers.  The oracle evaluated in float32 departs from its own float64
# evaluation by e_rel(X^T) 8.4e-3, e_rel(D) 1.8e-2 and a cache e_rel of 5.1e-2;
# its bounds are about twice that (X^T keeps the stated 2e-2).
# "joint" is the single-camera workload with joint attention (per-layer prefix
# K/V as the cache, the pi0 form); its cache is the 18 layers' own keys and values.
CASES = [
    (1, 1e-2, 2e-2, None),
    (2, 1e-2, 2e-2, None),
    (3, 1e-2, 2e-2, (0, 5, 10, 15)),
    (4, 4e-2, 1e-1, None),
    ("joint", 1e-2, 2e-2, None),
]


def workload(idx):
    if idx == "joint":
        return synth.config(1, name="single_camera_joint_bf16", attn="joint"), 5
    return synth.config(idx), idx


def log(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("idx,dtol,ctol,sample", CASES, ids=lambda v: str(v))
def test_full_size_against_oracle(idx, dtol, ctol, sample):
    cfg, seed = workload(idx)
    t0 = time.time()
    log(f"case {cfg.name}: generating seeded inputs")
    w, b = synth.make_weights(cfg, seed)
    z0, x0 = synth.make_prefix(cfg, seed), synth.make_noise(cfg, seed)
    model = build_model(cfg, w, b)
    zt, xt = torch.from_numpy(z0).cuda(), torch.from_numpy(x0).cuda()
    kv = vla.vla_prefix_encode(model, zt)
    out16 = vla.vla_denoise_chunk(model, kv, xt, cfg.steps, out_dtype=torch.bfloat16)
    out32 = vla.vla_denoise_chunk(model, kv, xt, cfg.steps)
    torch.cuda.synchronize()
    got16 = out16.float().cpu().numpy().astype(np.float64)
    got32 = out32.cpu().numpy().astype(np.float64)
    gcache = cache_from_storage(cfg, kv.storage, cfg.batch, cfg.n_prefix)
    kv.close()
    if cfg.batch > 1:
        rev = list(range(cfg.batch))[::-1]
        zr, xr = torch.from_numpy(z0[rev].copy()).cuda(), torch.from_numpy(x0[rev].copy()).cuda()
        kvr = vla.vla_prefix_encode(model, zr)
        outr = vla.vla_denoise_chunk(model, kvr, xr, cfg.steps)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(outr.cpu().numpy()[rev], got32.astype(np.float32))
        rcache = cache_from_storage(cfg, kvr.storage, cfg.batch, cfg.n_prefix)
        for bo in range(cfg.batch):
            for l in range(cfg.L_e):
                for i in range(2):
                    np.testing.assert_array_equal(rcache[rev[bo]][l][i], gcache[bo][l][i])
        kvr.close()
        del zr, xr, outr
        log(f"case {cfg.name}: reversed batch identical at {time.time() - t0:.1f}s")
    model.close()
    del zt, xt, out16, out32
    torch.cuda.empty_cache()
    log(f"case {cfg.name}: GPU done at {time.time() - t0:.1f}s, running the oracle")
    obs = list(sample) if sample else list(range(cfg.batch))
    o = oracle.Oracle(cfg, w, b)
    ref, caches = o.run(z0[obs], x0[obs], keep_cache=True)
    log(f"case {cfg.name}: oracle done at {time.time() - t0:.1f}s")
    x0o = x0[obs].astype(np.float64)
    e16 = oracle.e_rel(got16[obs], ref)
    e32 = oracle.e_rel(got32[obs], ref)
    ed = oracle.e_rel(got32[obs] - x0o, ref - x0o)
    ec = max(oracle.e_rel(gcache[bo][l][i], caches[k][l][i])
             for k, bo in enumerate(obs) for l in range(cfg.L_e) for i in range(2))
    log(f"[{cfg.name}] e_rel(bf16 X^T)={e16:.3e} e_rel(X^T)={e32:.3e} e_rel(X^T-X^0)={ed:.3e} "
        f"e_inf={oracle.e_inf(got32[obs], ref):.3e} max cache e_rel={ec:.3e}")
    del w, o
    gc.collect()
    assert e16 <= 2e-2
    assert ed <= dtol
    assert ec <= ctol


@pytest.mark.parametrize("attn", ["cross", "joint"])
def test_degenerate_sizes(attn):
    """One prefix token, one chunk row, one step."""
    cfg = synth.config(1, name="degenerate", n_prefix=1, d_p=128, L_p=1, Hq=2, Hkv=1, hd=64, F_p=128, d_e=128, L_e=1,
                       Hq_e=2, Hkv_e=1, hd_e=64, F_e=128, H=1, d_a=1, steps=1, attn=attn)
    w, b = synth.make_weights(cfg, 9)
    z0, x0 = synth.make_prefix(cfg, 9), synth.make_noise(cfg, 9)
    model = build_model(cfg, w, b)
    kv = vla.vla_prefix_encode(model, torch.from_numpy(z0).cuda())
    got = vla.vla_denoise_chunk(model, kv, torch.from_numpy(x0).cuda(), 1).cpu().numpy().astype(np.float64)
    ref = oracle.Oracle(cfg, w, b).run(z0, x0)
    assert oracle.e_rel(got - x0, ref - x0) <= 5e-3
    # empty requests are rejected, and leave no handle behind
    for bad in ((0, 1), (1, 0)):
        with pytest.raises(vla.VlaError) as ei:
            vla.vla_prefix_encode(model, torch.zeros((bad[0], bad[1], cfg.d_p), device="cuda"))
        assert ei.value.status == 1
    kv.close()
    model.close()
