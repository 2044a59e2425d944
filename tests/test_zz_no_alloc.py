"""moe_permute_noalloc (the permute with the library's own static scratch,
for callers that cannot allocate) against moe_permute with a workspace:
every output bit-identical, on consecutive calls of decreasing size so the
second call reuses the scratch the first one left behind (needs MI355X)."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_fp32_amd as moe

pytestmark = pytest.mark.gpu


def _routing(T, E, k, seed):
    g = np.random.default_rng(seed)
    # distinct experts per token, skewed towards low ids
    p = 1.0 / np.arange(1, E + 1)
    p /= p.sum()
    return np.stack([g.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)


def _outputs(d, T, k, n, cap, D, dev):
    return dict(counts=torch.full((n,), -3, dtype=torch.int32, device=dev),
                offsets=torch.full((n + 1,), -3, dtype=torch.int32, device=dev),
                split=torch.full((d.ep_size,), -3, dtype=torch.int32, device=dev),
                perm_src=torch.full((cap,), -7, dtype=torch.int32, device=dev),
                pos=torch.full((T, k), -9, dtype=torch.int32, device=dev),
                x_perm=torch.zeros(cap, D, dtype=torch.bfloat16, device=dev))


def test_permute_noalloc_matches_permute():
    assert torch.cuda.is_available(), "no GPU visible"
    moe.load_library()
    dev = "cuda"
    # (T, D, E, k, ep_size, expert range): 400k pairs over 256 experts (2048-token
    # count blocks, 6400 block counts), then 12000 pairs (count kernel), then
    # 2800 pairs (the scan counts them itself), then a sub-range of experts
    cases = [(50000, 128, 256, 8, 8, (0, 256)), (3000, 256, 64, 4, 4, (0, 64)),
             (700, 256, 64, 4, 4, (0, 64)), (1500, 128, 64, 4, 4, (16, 48))]
    for i, (T, D, E, k, R, (eb, ee)) in enumerate(cases):
        print(f"[no_alloc] call {i}: T={T} D={D} E={E} k={k} range=[{eb},{ee})", flush=True)
        d = moe.make_desc(T=T, D=D, E=E, top_k=k, I=64, ep_size=R)
        n = ee - eb
        cap = T * min(k, n)
        idx = torch.from_numpy(_routing(T, E, k, 100 + i)).to(dev)
        x = torch.randn(T, D, generator=torch.Generator().manual_seed(i)).to(torch.bfloat16)
        x = x.to(dev)
        a = _outputs(d, T, k, n, cap, D, dev)
        b = _outputs(d, T, k, n, cap, D, dev)
        ws = moe.workspace(moe.moe_permute_workspace_size(d, eb, ee))
        assert ws.numel() <= 2 * 12288 * 4
        moe.moe_permute(d, x, idx, eb, ee, cap, a["counts"], a["offsets"], a["split"],
                        a["perm_src"], a["pos"], a["x_perm"], ws)
        moe.moe_permute_noalloc(d, x, idx, eb, ee, cap, b["counts"], b["offsets"], b["split"],
                                b["perm_src"], b["pos"], b["x_perm"])
        torch.cuda.synchronize()
        M = int(a["offsets"][-1].item())
        for key in ("counts", "offsets", "split", "pos"):
            assert torch.equal(a[key], b[key]), (i, key)
        assert torch.equal(a["perm_src"][:M], b["perm_src"][:M]), (i, "perm_src")
        assert torch.all(b["perm_src"][M:] == -7)
        assert torch.equal(a["x_perm"][:M].view(torch.int16), b["x_perm"][:M].view(torch.int16))
        assert int(a["counts"].sum().item()) == M
