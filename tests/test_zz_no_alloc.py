"""gq_attn_decode_noalloc (the allocation-free variant of gq_attn_decode,
through the C ABI) against gq_attn_decode with a caller workspace: the same
kernels, so bit-identical results, and within the attention bound of the
oracle; two calls in a row, the second smaller, so the shared device array
is reused with a different layout."""
import sys

import numpy as np
import pytest
import torch

import gguf_quant_matmul_amd as gq
from test_gpu_attn import make_cache, reference

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("first,second", [
    (("q8_0", 3000, 4, 20, 128), ("q4_0", 700, 2, 8, 64)),
    (("q4_0", 32768, 8, 40, 128), ("q8_0", 37, 1, 16, 256)),
])
def test_noalloc_matches_workspace_variant(first, second):
    dev = torch.device("cuda:0")
    for i, (t, kv_len, n_kv, n_heads, hd) in enumerate((first, second)):
        say(f"noalloc call {i}: {t} kv_len={kv_len} n_kv={n_kv} heads={n_heads} hd={hd}")
        kb, vb = make_cache(t, kv_len, n_kv, hd, seed=900 + 10 * i)
        q = np.random.default_rng(901 + i).standard_normal((n_heads, hd)).astype(np.float32)
        kd, vd = torch.from_numpy(kb).to(dev), torch.from_numpy(vb).to(dev)
        qd = torch.from_numpy(q).to(dev)
        ref_ws = gq.attn_decode(kd, vd, t, kv_len, n_kv, hd, qd)
        out = torch.full((n_heads, hd), float("nan"), dtype=torch.float32, device=dev)
        gq.attn_decode_noalloc(kd, vd, t, kv_len, n_kv, hd, qd, out)
        torch.cuda.synchronize()
        a, b = out.cpu().numpy(), ref_ws.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"call {i}: differs from the workspace variant"
        if kv_len <= 4000:
            ref, tol = reference(kb, vb, t, kv_len, n_kv, hd, q.astype(np.float64))
            err = np.abs(a.astype(np.float64) - ref)
            say(f"  max err / bound = {float(np.max(err / np.maximum(tol, 1e-300))):.3e}")
            assert np.all(err <= tol)
