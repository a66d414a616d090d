"""moe_dispatch_noalloc (the dispatch whose workspace is the library's own
device array) against moe_dispatch with a caller workspace, through the C ABI:
bit-identical counts, offsets, tile offsets, perm, inv and x_perm on calls in
a row, each later call smaller than the one before it, over every metadata
path; and a request larger than the array is rejected before any launch."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _B():
    import combine_dual_overlap_amd as C
    C.binding.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return C.binding


def _outputs(B, T, k, E_loc, H, dt):
    cap = max(T * k, 1)
    mk = lambda n: torch.full((n,), -7, dtype=torch.int32, device="cuda")
    return dict(counts=mk(E_loc), offsets=mk(E_loc + 1), tile_offsets=mk(E_loc + 1), perm=mk(cap), inv=mk(cap),
                x_perm=torch.zeros(cap, H, dtype=dt, device="cuda"))


def _run(B, x, ids, E, lo, hi, tile_m, noalloc):
    T, H = x.shape
    k = ids.shape[1]
    o = _outputs(B, T, k, hi - lo, H, x.dtype)
    if noalloc:
        B.moe_dispatch_noalloc(x, ids, E, lo, hi, o["counts"], o["offsets"], o["perm"], o["inv"], o["x_perm"],
                               tile_m=tile_m, tile_offsets=o["tile_offsets"])
    else:
        ws = torch.empty(B.moe_dispatch_workspace_size(T, k, hi - lo), dtype=torch.uint8, device="cuda")
        B.moe_dispatch(x, ids, E, lo, hi, o["counts"], o["offsets"], o["perm"], o["inv"], o["x_perm"], ws,
                       tile_m=tile_m, tile_offsets=o["tile_offsets"])
    torch.cuda.synchronize()
    return {n: t.cpu() for n, t in o.items()}


# (T, k, E, local range): count + rank-with-scan path (32768 pairs), the
# one-workgroup path, the count / scan / rank path (300 local experts), and
# a last, smaller call on the first path again.
CALLS = [(4096, 8, 128, 0, 128), (300, 6, 64, 0, 64), (1000, 3, 300, 0, 300), (2500, 8, 256, 32, 64)]


def test_noalloc_dispatch_equals_dispatch_on_calls_in_a_row():
    B = _B()
    assert B.moe_dispatch_noalloc_max_workspace() == 8 << 20
    rng = np.random.default_rng(7)
    for T, k, E, lo, hi in CALLS:
        print(f"noalloc dispatch T={T} k={k} E={E} local=[{lo},{hi})", flush=True)
        ids = torch.from_numpy(np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)).cuda()
        x = torch.randn(T, 256, device="cuda").to(torch.bfloat16)
        want = _run(B, x, ids, E, lo, hi, 64, noalloc=False)
        got = _run(B, x, ids, E, lo, hi, 64, noalloc=True)
        M = int(want["offsets"][-1])
        for name in ("counts", "offsets", "tile_offsets", "inv"):
            assert torch.equal(got[name], want[name]), name
        assert torch.equal(got["perm"][:M], want["perm"][:M])
        assert torch.equal(got["x_perm"][:M].view(torch.int16), want["x_perm"][:M].view(torch.int16))


def test_noalloc_dispatch_rejects_requests_beyond_its_array():
    B = _B()
    T, k, E = 131072, 8, 1024          # 4096 pair blocks x 1024 experts x 4 bytes = 16 MiB of histograms
    assert B.moe_dispatch_workspace_size(T, k, E) > B.moe_dispatch_noalloc_max_workspace()
    x = torch.zeros(T, 128, dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros(T, k, dtype=torch.int32, device="cuda")
    o = _outputs(B, 1, 1, E, 128, x.dtype)
    with pytest.raises(B.MoEError) as e:
        B.moe_dispatch_noalloc(x, ids, E, 0, E, o["counts"], o["offsets"], o["perm"], o["inv"], o["x_perm"])
    assert e.value.status == B.MOE_ERR_WORKSPACE
