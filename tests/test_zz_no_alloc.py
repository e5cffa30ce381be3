"""kvs_token_confidence_static (the entry point for callers that cannot allocate: it
keeps its partial results in the library's own static device buffer) against
kvs_token_confidence with a caller workspace, through the C ABI: the same kernels on
the same inputs, so the confidences must be equal bit for bit.  Two calls in a row,
the second smaller (the buffer keeps the first call's contents, which must not leak
into the second), on bf16 and fp32 logits; and the rejection of a call whose partial
results exceed the buffer."""
import ctypes as C

import numpy as np
import pytest

from workloads import logits as LG

pytestmark = pytest.mark.gpu


def _ws_call(L, x, dtype, rows, V, k, conf):
    import torch
    need = int(L.kvs_token_confidence_workspace_size(rows, V, k))
    ws = torch.empty(max(need, 4), dtype=torch.uint8, device="cuda")
    st = L.kvs_token_confidence(C.c_void_p(x.data_ptr()), dtype, rows, V, int(x.stride(0)), k,
                                C.c_void_p(conf.data_ptr()), C.c_void_p(ws.data_ptr()), need, None)
    assert st == 0, L.kvs_last_error()
    return need


def _static_call(L, x, dtype, rows, V, k, conf):
    return L.kvs_token_confidence_static(C.c_void_p(x.data_ptr()), dtype, rows, V, int(x.stride(0)), k,
                                         C.c_void_p(conf.data_ptr()), None)


@pytest.mark.parametrize("bf16", [True, False])
def test_static_buffer_matches_workspace_call(bf16):
    import torch
    import kv_cache_eviction_lse_amd as K
    L = K.lib()
    dtype = K.KVS_DTYPE_BF16 if bf16 else K.KVS_DTYPE_F32
    tdt = torch.bfloat16 if bf16 else torch.float32
    # first a large call (many chunks per row), then a smaller one: fewer rows, a
    # shorter vocabulary and another k, so it reads partial slots the first call wrote
    for seed, rows, V, k in ((11, 600, 151936, 20), (12, 37, 70000, 7)):
        x = LG.lm_rows_device(seed, rows, V, torch.device("cuda", 0), tdt)
        want = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
        got = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
        print(f"static confidence: bf16={bf16} rows={rows} vocab={V} k={k}", flush=True)
        need = _ws_call(L, x, dtype, rows, V, k, want)
        assert need > 0
        assert _static_call(L, x, dtype, rows, V, k, got) == 0, L.kvs_last_error()
        torch.cuda.synchronize()
        w, g = want.cpu().numpy(), got.cpu().numpy()
        assert np.all(np.isfinite(w))
        np.testing.assert_array_equal(g.view(np.uint32), w.view(np.uint32))


def test_static_buffer_limit():
    import torch
    import kv_cache_eviction_lse_amd as K
    L = K.lib()
    rows, V, k = 4096, 1 << 20, 20
    assert L.kvs_token_confidence_workspace_size(rows, V, k) > (16 << 20)
    x = torch.zeros((1, 8), dtype=torch.float32, device="cuda")       # never read
    conf = torch.zeros(1, dtype=torch.float32, device="cuda")
    st = L.kvs_token_confidence_static(C.c_void_p(x.data_ptr()), K.KVS_DTYPE_F32, rows, V, V, k,
                                       C.c_void_p(conf.data_ptr()), None)
    from kv_cache_eviction_lse_amd._lib import STATUS
    assert STATUS[st] == "KVS_ERR_UNSUPPORTED" and b"static buffer" in L.kvs_last_error()
