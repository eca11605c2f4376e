"""The allocation-free ternary GEMM entry point against the allocating one (needs a gfx950 GPU).

vla_w2a8_gemm_noalloc keeps its repacked weights and flag in the library's
fixed per-device scratch array.  Two calls in a row, the second smaller, must
each give the int32 accumulators and bf16 outputs of vla_w2a8_gemm bit for bit
(the second call must not see the first call's leftovers), and a shape beyond
the scratch is refused with a clear error.
"""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from prefix_cache_flow_amd import vla  # noqa: E402


def _case(M, N, K, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((M, K)) * rng.uniform(0.5, 3.0, (M, 1))).astype(np.float32)
    a, alpha = oracle.quantize_rows(x)
    q = rng.integers(-1, 2, (N, K), dtype=np.int8)
    beta = float(np.float32(rng.uniform(0.005, 0.05)))
    return (torch.from_numpy(a).cuda(), torch.from_numpy(alpha).cuda(),
            torch.from_numpy(oracle.pack_ternary(q)).cuda(), beta, oracle.w2a8_accumulate(a, q))


def test_noalloc_matches_allocating_entry_point_twice():
    # the ternary workload's largest shape first, then a smaller one in the same scratch
    for (M, N, K), seed in (((320, 13824, 2560), 11), ((37, 96, 384), 12)):
        print(f"noalloc M={M} N={N} K={K} seed={seed}", flush=True)
        a, alpha, packed, beta, acc_ref = _case(M, N, K, seed)
        acc0, y0 = vla.vla_w2a8_gemm(a, alpha, packed, beta)
        acc = torch.full((M, N), -7, dtype=torch.int32, device="cuda")
        y = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
        vla.vla_w2a8_gemm_noalloc(a, alpha, packed, beta, acc, y)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(acc.cpu().numpy(), acc0.cpu().numpy())
        np.testing.assert_array_equal(acc.cpu().numpy(), acc_ref)
        np.testing.assert_array_equal(y.view(torch.int16).cpu().numpy(), y0.view(torch.int16).cpu().numpy())


def test_noalloc_rejects_code_3_then_recovers():
    a = torch.zeros((32, 128), dtype=torch.int8, device="cuda")
    al = torch.ones(32, dtype=torch.float32, device="cuda")
    bad = np.zeros((32, 32), dtype=np.uint8)
    bad[5, 7] = 0b11 << 4
    acc = torch.empty((32, 32), dtype=torch.int32, device="cuda")
    with pytest.raises(vla.VlaError) as ei:
        vla.vla_w2a8_gemm_noalloc(a, al, torch.from_numpy(bad).cuda(), 1.0, acc, None)
    assert ei.value.status == 1
    # the flag left set by that call is cleared by the next one
    good = np.full((32, 32), 0b01010101, dtype=np.uint8)  # every code 1: q = 0
    vla.vla_w2a8_gemm_noalloc(a, al, torch.from_numpy(good).cuda(), 1.0, acc, None)
    assert int(acc.abs().sum()) == 0


def test_noalloc_rejects_shapes_beyond_the_scratch():
    M, N, K = 1, 32768, 2048 + 128  # N * K / 4 > 16 MiB - 256
    a = torch.zeros((M, K), dtype=torch.int8, device="cuda")
    al = torch.ones(M, dtype=torch.float32, device="cuda")
    packed = torch.zeros((N, K // 4), dtype=torch.uint8, device="cuda")
    with pytest.raises(vla.VlaError) as ei:
        vla.vla_w2a8_gemm_noalloc(a, al, packed, 1.0, None, None)
    assert ei.value.status == 4 and "scratch" in str(ei.value)
