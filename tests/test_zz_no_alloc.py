"""The decode step's no-allocation entry point (its workspace in the library's static device
scratch) against the workspace entry point: two calls in a row, the second with a smaller batch,
each compared bit for bit with pkv_paged_decode_step on the same inputs and with the oracle."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests.helpers import DeviceWorkload, assert_parity, log, to_device, to_f64, to_numpy_storage
from tests.test_gpu_step import with_new_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import paged_kv_cache_203_amd as lib
    return lib


def test_no_alloc_step_matches_workspace_step(pkv):
    for batch, lens in ((48, ("uniform", 300, 3000)), (7, ("uniform", 1, 500))):
        w = W.make_workload(W.config(2).scaled(batch=batch, lengths=lens))
        log(f"case no-alloc batch={batch} lens={w.context_lens.tolist()[:8]}")
        k_new, v_new, alens = with_new_rows(w)
        lens_d = torch.from_numpy(alens).cuda()
        outs, pools = [], []
        for noalloc in (False, True):
            d = DeviceWorkload(w)   # each call appends into its own copy of the pools
            kn, vn = to_device(k_new, w.dtype), to_device(v_new, w.dtype)
            out = torch.empty_like(d.q)
            lse = torch.empty(d.q.shape[:2], dtype=torch.float32, device="cuda")
            if noalloc:
                pkv.paged_decode_step_noalloc(d.q, d.k_pool, d.v_pool, d.page_table, lens_d, out,
                                              d.scale, k_new=kn, v_new=vn, lse_out=lse)
            else:
                pkv.paged_decode_step(d.q, d.k_pool, d.v_pool, d.page_table, lens_d, d.scale,
                                      k_new=kn, v_new=vn, out=out, lse_out=lse)
            torch.cuda.synchronize()
            outs.append((out, lse))
            pools.append((to_numpy_storage(d.k_pool, w.dtype), to_numpy_storage(d.v_pool, w.dtype)))
        assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
        assert torch.equal(outs[0][1], outs[1][1])
        kp, vp = O.paged_kv_append(w.k_pool, w.v_pool, k_new, v_new, w.page_table, alens)
        for got in pools:
            assert np.array_equal(got[0].view(np.uint8), kp.view(np.uint8))
            assert np.array_equal(got[1].view(np.uint8), vp.view(np.uint8))
        ref, ref_lse = O.paged_decode_attention(w.q, kp, vp, w.page_table, w.context_lens, w.scale,
                                                w.dtype)
        assert_parity(to_f64(outs[1][0]), ref, w.dtype, f"no-alloc step batch={batch}")
        assert np.abs(outs[1][1].double().cpu().numpy() - ref_lse).max() <= 1e-4


def test_no_alloc_step_rejects_oversized_shapes(pkv):
    # 4096 sequences of 128 query heads need more step workspace than the 64 MiB scratch holds
    s = pkv.make_shape(4096, 128, 8, 128, 16, 64, 4, 1)
    import ctypes
    rc = pkv.lib.pkv_paged_decode_step_noalloc(16, None, None, 16, 16, 16, 16, ctypes.c_float(0.1),
                                               16, None, ctypes.byref(s), None)
    assert rc == -4, (rc, pkv.last_error())
    assert "scratch" in pkv.last_error()
