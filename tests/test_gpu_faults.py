"""Every device allocation of the library failing in turn (needs a gfx950 GPU).

With VLA_FAIL_ALLOC=n the library's n-th allocation fails as if memory were
exhausted.  For n = 1, 2, ... the whole request -- model creation, prefix
encode, denoise, and a ternary GEMM through the unit entry point -- must stop
with VLA_ERR_OUT_OF_MEMORY (never a crash, never a handle left behind), until
n passes the number of allocations and the request succeeds; afterwards the
library gives the same bits as before the sweep and device memory is back
where it started.  (The paper, §III-C: a response carries the chunk "or an
error".)
"""
import os

import numpy as np
import pytest

import oracle
from policy_cases import SMALL_BF16, SMALL_W2A8, host_inputs, ordered, ordered_betas

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from prefix_cache_flow_amd import vla  # noqa: E402


def _request(cfg, tensors, betas, zt, xt):
    model = vla.vla_model_create(cfg.to_dict(), tensors, betas)
    try:
        kv = vla.vla_prefix_encode(model, zt)
        try:
            out = vla.vla_denoise_chunk(model, kv, xt, cfg.steps, timing=True)[0]
            torch.cuda.synchronize()
            return out.cpu().numpy()
        finally:
            kv.close()
    finally:
        model.close()


@pytest.mark.parametrize("cfg", [SMALL_BF16, SMALL_W2A8], ids=lambda c: c.name)
def test_each_allocation_failure_is_reported_and_recovered(cfg):
    w, b, z0, x0 = host_inputs(cfg, 0)
    tensors = vla.upload_weights(cfg.to_dict(), ordered(cfg, w))
    betas = ordered_betas(cfg, b)
    zt, xt = torch.from_numpy(z0).cuda(), torch.from_numpy(x0).cuda()
    reference = _request(cfg, tensors, betas, zt, xt)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    failures = 0
    try:
        for n in range(1, 400):
            os.environ["VLA_FAIL_ALLOC"] = str(n)
            try:
                got = _request(cfg, tensors, betas, zt, xt)
            except vla.VlaError as e:
                assert e.status == 5, f"allocation {n}: {e}"
                failures += 1
                continue
            print(f"[{cfg.name}] {failures} allocation sites each reported VLA_ERR_OUT_OF_MEMORY", flush=True)
            np.testing.assert_array_equal(got.view(np.int32), reference.view(np.int32))
            break
        else:
            pytest.fail("the request never succeeded")
    finally:
        del os.environ["VLA_FAIL_ALLOC"]
    assert failures >= 10
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    assert abs(free1 - free0) < (64 << 20), f"device memory moved by {free0 - free1} bytes"
    np.testing.assert_array_equal(_request(cfg, tensors, betas, zt, xt).view(np.int32), reference.view(np.int32))


def test_ternary_unit_entry_point_reports_allocation_failures():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    a, al = oracle.quantize_rows(x)
    q = rng.integers(-1, 2, (64, 256), dtype=np.int8)
    at, alt = torch.from_numpy(a).cuda(), torch.from_numpy(al).cuda()
    packed = torch.from_numpy(oracle.pack_ternary(q)).cuda()
    try:
        for n in (1, 2):
            os.environ["VLA_FAIL_ALLOC"] = str(n)
            with pytest.raises(vla.VlaError) as ei:
                vla.vla_w2a8_gemm(at, alt, packed, 0.5)
            assert ei.value.status == 5
    finally:
        del os.environ["VLA_FAIL_ALLOC"]
    acc, _ = vla.vla_w2a8_gemm(at, alt, packed, 0.5)
    np.testing.assert_array_equal(acc.cpu().numpy(), oracle.w2a8_accumulate(a, q))
