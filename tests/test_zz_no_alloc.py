"""moe_forward_static_scratch (the forward for callers that cannot allocate:
its scratch is a static device array) against moe_forward through the C ABI:
two contexts set up alike, the same inputs, two calls in a row (a grouped
16-token batch, then a smaller 3-token batch on the fused path), outputs,
routing and the cache step's decisions identical, outputs within 2e-3 of the
oracle; and a request larger than the array is refused."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import moe_expert_offload_gemv_amd as moe  # noqa: E402
import oracle  # noqa: E402
from tests._gpu import TOL, Decode, token_rel_err  # noqa: E402
from workload import Workload, activations, zipf_logits  # noqa: E402

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def test_static_scratch_forward_matches_the_allocating_one():
    wl = Workload("decode-e64k8-h2048f1024-l2-b16-static", 119, 2, 64, 8, 2048, 1024, tokens=16, steps=2,
                  zipf_s=1.1, slots=24)
    a = Decode(wl, max_batch=256)
    b = Decode(wl, max_batch=256)
    try:
        k, H = wl.top_k, wl.hidden
        for step, T in enumerate((16, 3)):  # the second call is smaller
            z = zipf_logits(wl, steps=step + 1, tokens=T)[step]
            for layer in range(wl.n_layers):
                x32 = activations(wl, step, tokens=T, layer=layer)
                x, zl = _dev(x32), _dev(z[layer])
                outs = []
                for d, fwd in ((a, moe.moe_forward), (b, moe.moe_forward_static_scratch)):
                    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
                    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
                    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
                    fwd(d.ctx, layer, T, x, zl, y, ids, w)
                    outs.append((y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()))
                (ya, ia, wa), (yb, ib, wb) = outs
                assert np.array_equal(ia, ib) and np.array_equal(wa, wb), (step, layer)
                assert np.array_equal(ya, yb), (step, layer, np.abs(ya - yb).max())
                y_ref, ids_ref, _ = oracle.moe_layer(wl.n_experts, k, H, wl.ffn, a.experts(layer, ia),
                                                     x32.astype(np.float64), logits=z[layer])
                assert np.array_equal(ib, ids_ref)
                assert token_rel_err(yb, y_ref) < TOL
            sa, sb = moe.moe_cache_step(a.ctx), moe.moe_cache_step(b.ctx)
            assert sa == sb, (sa, sb)
            for layer in range(wl.n_layers):
                assert np.array_equal(moe.moe_get_slot_table(a.ctx, layer, wl.n_experts),
                                      moe.moe_get_slot_table(b.ctx, layer, wl.n_experts))
            assert np.array_equal(moe.moe_get_miss_log(a.ctx), moe.moe_get_miss_log(b.ctx))
        # 256 tokens x top-8 at H = 2048, F = 1024 need 25 MB of scratch, more than the 16 MiB array
        T = 256
        x = torch.zeros((T, H), dtype=torch.float32, device="cuda")
        zl = torch.zeros((T, wl.n_experts), dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_forward_static_scratch(b.ctx, 0, T, x, zl, y)
        assert ei.value.code == moe.MOE_E_INVAL
    finally:
        a.close()
        b.close()
