"""Key padding (the paper, §III-B, Eq. 2: M = -inf on masked keys) on the GPU against the oracle.

A batch of observations with different prefix lengths, padded to one N, is
encoded with vla_prefix_encode_masked and denoised; the chunk must match the
oracle run with the same lengths (Eq. 5 of §III-E, the end-to-end bounds), the
padding's content must not change a single bit of the outputs (the library
zeroes padded rows and gives padded keys weight 0), and each observation must
match the same observation encoded alone at its own length.
"""

import numpy as np
import pytest

import oracle
import synth
from policy_cases import JOINT_F32, SMALL_BF16, SMALL_JOINT, SMALL_W2A8, build_model, cache_from_storage

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from prefix_cache_flow_amd import vla  # noqa: E402

# ragged batches: lengths that are not whole 32-key tiles, one observation at full length
RAGGED = [
    (synth.config(0, name="tiny_fp32_ragged", batch=3, n_prefix=40), [40, 23, 9], 1e-3, 1e-3),
    (synth.config(1, name="small_bf16_ragged", batch=3, n_prefix=100, d_p=256, L_p=2, Hq=4, Hkv=1, hd=64, F_p=512,
                  d_e=128, L_e=2, Hq_e=2, Hkv_e=1, hd_e=64, F_e=256, H=20, d_a=7, steps=3),
     [100, 69, 17], 2e-2, 5e-3),
    # 80 chunk rows: the expert runs on the wide tiles
    (synth.config(1, name="small_bf16_ragged_b4", batch=4, n_prefix=70, d_p=256, L_p=2, Hq=8, Hkv=1, hd=128,
                  F_p=512, d_e=128, L_e=2, Hq_e=8, Hkv_e=1, hd_e=128, F_e=256, H=20, d_a=5, steps=2),
     [33, 70, 1, 64], 2e-2, 5e-3),
    (synth.config(1, name="small_joint_ragged", attn="joint", batch=3, n_prefix=100, d_p=256, L_p=2, Hq=4, Hkv=1,
                  hd=64, F_p=512, d_e=128, L_e=2, Hq_e=2, Hkv_e=1, hd_e=64, F_e=256, H=20, d_a=7, steps=3),
     [100, 47, 5], 2e-2, 5e-3),
    (synth.config(0, name="tiny_joint_fp32_ragged", attn="joint", batch=2, n_prefix=40, H=6), [40, 13], 1e-3, 1e-3),
    (synth.config(4, name="small_w2a8_ragged", batch=3, n_prefix=100, d_p=256, L_p=2, Hq=2, Hkv=2, hd=128, F_p=384,
                  d_e=128, L_e=2, Hq_e=2, Hkv_e=1, hd_e=64, F_e=256, H=8, d_a=7, steps=3),
     [100, 61, 30], 2e-2, 1e-2),
    # 1040 16-row blocks of prefix queries: the 64-row attention workgroups sharing key tiles through LDS
    (synth.config(1, name="small_rows_ragged_b8", batch=8, n_prefix=260, d_p=256, L_p=2, Hq=8, Hkv=1, hd=64,
                  F_p=512, d_e=128, L_e=2, Hq_e=2, Hkv_e=1, hd_e=64, F_e=256, H=20, d_a=7, steps=2),
     [260, 33, 1, 200, 129, 64, 259, 96], 2e-2, 5e-3),
]


def _inputs(cfg, seed, lengths, junk_scale):
    w, b = synth.make_weights(cfg, seed)
    z0, x0 = synth.make_prefix(cfg, seed), synth.make_noise(cfg, seed)
    rng = np.random.default_rng(1000 + seed)
    z = z0.copy()
    for i, n in enumerate(lengths):
        z[i, n:] = junk_scale * rng.standard_normal(z[i, n:].shape).astype(np.float32)
    return w, b, z, x0


def _run(cfg, model, z, x0, lengths):
    B, N = z.shape[0], z.shape[1]
    storage = torch.zeros(vla.vla_kv_cache_bytes(model, B, N), dtype=torch.uint8, device="cuda")
    kv = vla.vla_prefix_encode(model, torch.from_numpy(z).cuda(), kv_storage=storage, lengths=lengths)
    out = vla.vla_denoise_chunk(model, kv, torch.from_numpy(x0).cuda(), cfg.steps)
    torch.cuda.synchronize()
    res = out.cpu().numpy()
    storage = kv.storage.clone()
    kv.close()
    return res, storage


@pytest.mark.parametrize("cfg,lengths,tol,dtol", RAGGED, ids=lambda v: getattr(v, "name", ""))
def test_ragged_batch_matches_oracle_and_ignores_padding(cfg, lengths, tol, dtol):
    print(f"case {cfg.name} lengths {lengths}", flush=True)
    w, b, z, x0 = _inputs(cfg, 3, lengths, 5.0)
    model = build_model(cfg, w, b)
    got, storage = _run(cfg, model, z, x0, lengths)
    ref = oracle.Oracle(cfg, w, b).run(z, x0, lengths=lengths)
    x0d = x0.astype(np.float64)
    e, ed = oracle.e_rel(got, ref), oracle.e_rel(got - x0d, ref - x0d)
    print(f"[{cfg.name}] e_rel(X^T)={e:.3e} e_rel(D)={ed:.3e}", flush=True)
    assert e <= tol and ed <= dtol
    # other padding, including non-finite values: the same bits everywhere
    z2 = z.copy()
    for i, n in enumerate(lengths):
        if n < cfg.n_prefix:
            z2[i, n:] = -3.0
            z2[i, -1, 0] = np.nan
    got2, storage2 = _run(cfg, model, z2, x0, lengths)
    np.testing.assert_array_equal(got2.view(np.int32), got.view(np.int32))
    np.testing.assert_array_equal(storage2.cpu().numpy(), storage.cpu().numpy())
    model.close()


def test_padded_observation_matches_its_own_length_and_full_length_is_unmasked():
    cfg, lengths = RAGGED[1][0], RAGGED[1][1]
    w, b, z, x0 = _inputs(cfg, 4, lengths, 2.0)
    model = build_model(cfg, w, b)
    got, _ = _run(cfg, model, z, x0, lengths)
    x0d = x0.astype(np.float64)
    for i, n in enumerate(lengths):
        one = synth.config(1, **{**cfg.to_dict(), "name": "one", "batch": 1, "n_prefix": n})
        alone, _ = _run(one, model, np.ascontiguousarray(z[i:i + 1, :n]), np.ascontiguousarray(x0[i:i + 1]), None)
        ed = oracle.e_rel(got[i:i + 1] - x0d[i:i + 1], alone.astype(np.float64) - x0d[i:i + 1])
        print(f"observation {i} (length {n}): e_rel(D, padded batch vs alone) = {ed:.3e}", flush=True)
        assert ed <= 2e-3
    # every length equal to N is the unmasked encode, bit for bit
    full = [cfg.n_prefix] * cfg.batch
    a, sa = _run(cfg, model, z, x0, full)
    u, su = _run(cfg, model, z, x0, None)
    np.testing.assert_array_equal(a.view(np.int32), u.view(np.int32))
    # the K/V blocks agree; only the masked encode writes the lengths tail after them
    core = cfg.batch * cfg.L_e * 2 * cfg.Hkv_e * ((cfg.n_prefix + 31) // 32 * 32) * cfg.hd_e * 2
    np.testing.assert_array_equal(sa.cpu().numpy()[:core], su.cpu().numpy()[:core])
    assert sa.cpu().numpy()[core:].view(np.int32)[:cfg.batch].tolist() == full
    for bad in ([0, 50, 50], [101, 50, 50], [-1, 1, 1]):
        with pytest.raises(vla.VlaError) as ei:
            vla.vla_prefix_encode(model, torch.from_numpy(z).cuda(), lengths=bad)
        assert ei.value.status == 1
    model.close()


def test_ragged_batch_on_the_persistent_step():
    """The opt-in persistent solver step masks the cached keys like the kernel chain (with the expert's
    norms as row kernels, the persistent step's summation order): same bits."""
    cfg, lengths = RAGGED[1][0], RAGGED[1][1]
    w, b, z, x0 = _inputs(cfg, 5, lengths, 2.0)
    fused_model = build_model(cfg, w, b, env={"VLA_FUSED": "1"})
    chain_model = build_model(cfg, w, b, env={"VLA_FOLD": "0"})
    f, _ = _run(cfg, fused_model, z, x0, lengths)
    c, _ = _run(cfg, chain_model, z, x0, lengths)
    np.testing.assert_array_equal(f.view(np.int32), c.view(np.int32))
