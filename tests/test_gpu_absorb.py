"""The absorbed cross sublayer against the three-kernel one and the oracle.

For one observation the encode also forms, per expert layer, Wq_j^T K^T and
V Wo_j^T from the cached keys and values (the paper's §III-B: they stay fixed
while the solver runs), and each solver step runs a cross sublayer as two
products: the scores with each 32-key block's max and weight sum, then the
normalised weights times Wvo into the residual.  That is the same attention
with other rounding points, so a model created with VLA_ABSORB=0 (query
product, attention over the cache, output product) is its comparison; both
are held to the end-to-end oracle bounds (§III-E, Eq. 5), masked keys
(Eq. 2, M = -inf) included.
"""

import numpy as np
import pytest

import oracle
import synth
from policy_cases import SMALL_BF16, SMALL_W2A8, build_model, host_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from prefix_cache_flow_amd import vla  # noqa: E402

# grouped heads (two query heads per key/value head) and a prefix that is not whole 32-key tiles
SMALL_GQA_ABS = synth.config(1, name="small_gqa_absorbed", n_prefix=90, d_p=256, L_p=2, Hq=4, Hkv=2, hd=64, F_p=512,
                             d_e=128, L_e=2, Hq_e=4, Hkv_e=2, hd_e=64, F_e=256, H=40, d_a=16, steps=2)
# the ternary prefix with a chunk of two row blocks (one block keeps the three-kernel form)
SMALL_W2A8_H20 = synth.config(4, name="small_w2a8_h20", n_prefix=100, d_p=256, L_p=2, Hq=2, Hkv=2, hd=128, F_p=384,
                              d_e=128, L_e=2, Hq_e=2, Hkv_e=1, hd_e=64, F_e=256, H=20, d_a=7, steps=3)
# head width 256 with 16 key tiles per head (the most the absorbed products take) and a 50-row chunk
SMALL_HD256_ABS = synth.config(1, name="small_hd256_absorbed", n_prefix=500, d_p=256, L_p=2, Hq=4, Hkv=1, hd=64,
                               F_p=512, d_e=256, L_e=3, Hq_e=4, Hkv_e=1, hd_e=256, F_e=512, H=50, d_a=32, steps=3)


def _run(cfg, model, z0, x0, lengths=None):
    zt = torch.from_numpy(np.ascontiguousarray(z0)).cuda()
    xt = torch.from_numpy(np.ascontiguousarray(x0)).cuda()
    kv = vla.vla_prefix_encode(model, zt, lengths=lengths)
    out = vla.vla_denoise_chunk(model, kv, xt, cfg.steps, out_dtype=torch.float32)
    torch.cuda.synchronize()
    res = out.cpu().numpy().astype(np.float64)
    kv.close()
    return res


CASES = [(SMALL_BF16, None), (SMALL_GQA_ABS, None), (SMALL_HD256_ABS, None), (SMALL_W2A8_H20, None),
         (SMALL_BF16, [37]), (SMALL_HD256_ABS, [300])]


@pytest.mark.parametrize("cfg,lengths", CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_absorbed_cross_sublayer_matches_three_kernels_and_oracle(cfg, lengths):
    print(f"case {cfg.name} lengths {lengths}", flush=True)
    w, b, z0, x0 = host_inputs(cfg, 0)
    absorbed = build_model(cfg, w, b)
    plain = build_model(cfg, w, b, env={"VLA_ABSORB": "0"})
    # the absorbed products live in the cache storage after the keys, values and lengths
    assert vla.vla_kv_cache_bytes(absorbed, 1, cfg.n_prefix) > vla.vla_kv_cache_bytes(plain, 1, cfg.n_prefix)
    got = _run(cfg, absorbed, z0, x0, lengths)
    ref3 = _run(cfg, plain, z0, x0, lengths)
    assert not np.array_equal(got, ref3), "the absorbed path did not run"
    x0d = x0.astype(np.float64)
    e_pair = oracle.e_rel(got - x0d, ref3 - x0d)
    ref = oracle.Oracle(cfg, w, b).run(z0, x0, lengths=lengths)
    e, ed = oracle.e_rel(got, ref), oracle.e_rel(got - x0d, ref - x0d)
    ed3 = oracle.e_rel(ref3 - x0d, ref - x0d)
    print(f"[{cfg.name}] e_rel(D, absorbed vs three kernels)={e_pair:.3e} oracle: e_rel(X^T)={e:.3e} "
          f"e_rel(D)={ed:.3e} (three kernels {ed3:.3e})", flush=True)
    tol_d = 4e-2 if cfg.precision == "w2a8" else 1e-2
    assert e <= 2e-2 and ed <= tol_d
    # bf16 rounding of the products in place of the query and the attention output: the same order
    # of error as the three-kernel path's own distance to the oracle
    assert e_pair <= max(3 * ed3, 2e-3)


def test_absorbed_padding_content_does_not_reach_the_chunk():
    """Tokens past the length hold junk (NaN included); the chunk is the same bits either way."""
    cfg, n = SMALL_BF16, 37
    w, b, z0, x0 = host_inputs(cfg, 1)
    model = build_model(cfg, w, b)
    z1 = z0.copy()
    z1[0, n:] = 1e4
    z2 = z0.copy()
    z2[0, n:] = np.nan
    a = _run(cfg, model, z1, x0, [n])
    c = _run(cfg, model, z2, x0, [n])
    np.testing.assert_array_equal(a.view(np.int64), c.view(np.int64))
    assert np.isfinite(a).all()


def test_absorbed_repeats_and_graph_replays_are_bitwise():
    cfg = SMALL_GQA_ABS
    w, b, z0, x0 = host_inputs(cfg, 2)
    model = build_model(cfg, w, b)
    first = _run(cfg, model, z0, x0)
    for _ in range(3):
        np.testing.assert_array_equal(_run(cfg, model, z0, x0).view(np.int64), first.view(np.int64))
    import os
    os.environ["VLA_NO_GRAPH"] = "1"  # eager launches, read at each call
    try:
        eager = _run(cfg, model, z0, x0)
    finally:
        del os.environ["VLA_NO_GRAPH"]
    np.testing.assert_array_equal(eager.view(np.int64), first.view(np.int64))


def test_one_row_block_keeps_the_three_kernel_form():
    """A chunk of at most 16 rows gets no absorbed products: the cache is only keys, values and lengths."""
    cfg = SMALL_W2A8
    w, b, z0, x0 = host_inputs(cfg, 0)
    a = build_model(cfg, w, b)
    p = build_model(cfg, w, b, env={"VLA_ABSORB": "0"})
    assert vla.vla_kv_cache_bytes(a, 1, cfg.n_prefix) == vla.vla_kv_cache_bytes(p, 1, cfg.n_prefix)
    np.testing.assert_array_equal(_run(cfg, a, z0, x0).view(np.int64), _run(cfg, p, z0, x0).view(np.int64))
