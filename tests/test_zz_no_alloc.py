"""GPU check of moe_permute_noalloc, the permute entry point that allocates
nothing: its per-block counts live in the library's static device scratch
instead of a caller workspace.  Called through the C ABI, its outputs must be
bit-identical to moe_permute's (same inputs, a caller workspace) -- rows,
E4M3 codes and scales, counts, offsets and both index maps -- on calls in a
row that reuse the scratch, each later one smaller than the one before, up to
the largest size the scratch allows.  The scratch holds the block counts of
the three-launch path (T k above the one-launch limit of 32768 entries);
the last calls take the one-launch path, which needs no scratch."""
import pytest
import torch

from grouped_gemm_router_amd import api, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def routing(T, k, E, seed):
    """Random valid top-k ids: k distinct experts per token."""
    g = torch.Generator().manual_seed(seed)
    return torch.rand((T, E), generator=g).argsort(dim=1)[:, :k].to(torch.int32).to(DEV)


def buffers(T, d, E, k, ns, fp8):
    rows = T * k + ns * T
    i32 = torch.int32
    return {
        "x_perm": torch.full((rows, d), 0x7F if fp8 else -1,
                             dtype=torch.uint8 if fp8 else torch.int16, device=DEV),
        "scale": torch.full((d // 128, rows), -1.0, device=DEV) if fp8 else None,
        "counts": torch.full((E,), -7, dtype=i32, device=DEV),
        "offsets": torch.full((E + ns + 1,), -7, dtype=i32, device=DEV),
        "perm_src": torch.full((T * k,), -7, dtype=i32, device=DEV),
        "flat_to_row": torch.full((T * k + ns * T,), -7, dtype=i32, device=DEV),
    }


def call_pair(T, d, E, k, ns, fp8, seed):
    print("noalloc permute: T %d d %d E %d k %d shared %d fp8 %s" % (T, d, E, k, ns, fp8),
          flush=True)
    x = synth.randn((T, d), 1.0, seed, DEV, torch.bfloat16)
    idx = routing(T, k, E, seed + 1)
    a, b = buffers(T, d, E, k, ns, fp8), buffers(T, d, E, k, ns, fp8)
    xp = lambda o: o["x_perm"] if fp8 else o["x_perm"].view(torch.bfloat16)  # noqa: E731
    ws = torch.empty((max(api.moe_permute_workspace_size(T, k, E), 4),), dtype=torch.uint8,
                     device=DEV)
    api.moe_permute(x, idx, E, ns, xp(a), a["counts"], a["offsets"], a["perm_src"],
                    a["flat_to_row"], ws, x_perm_scale=a["scale"])
    api.moe_permute_noalloc(x, idx, E, ns, xp(b), b["counts"], b["offsets"], b["perm_src"],
                            b["flat_to_row"], x_perm_scale=b["scale"])
    torch.cuda.synchronize()
    for name in a:
        if a[name] is None:
            continue
        u, v = a[name], b[name]
        if u.dtype == torch.float32:
            u, v = u.view(torch.int32), v.view(torch.int32)
        assert torch.equal(u, v), "%s differs from moe_permute's (T %d)" % (name, T)
    assert int(b["offsets"][E]) == T * k


@pytest.mark.parametrize("fp8", [False, True])
def test_noalloc_matches_permute_on_calls_in_a_row(fp8):
    # the first call needs the largest scratch the limit allows at E = 256
    # ((T/64 + 1) * E * 4 bytes of block counts and overflow starts)
    assert api.moe_permute_workspace_size(65472, 8, 256) <= api.PERMUTE_NOALLOC_SCRATCH_BYTES
    call_pair(65472, 128, 256, 8, 1, fp8, 11)
    # smaller, still three launches: the scratch left by the first call is reused
    call_pair(20000, 128, 64, 4, 0, fp8, 14)
    call_pair(4096, 7168 if fp8 else 4096, 256 if fp8 else 8, 8 if fp8 else 2, 1 if fp8 else 0,
              fp8, 12)
    call_pair(300, 1024, 64, 4, 1, fp8, 13)


def test_noalloc_refuses_sizes_beyond_its_scratch():
    T, d, E, k = 65536, 128, 256, 8
    assert api.moe_permute_workspace_size(T, k, E) > api.PERMUTE_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, d), dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros((T, k), dtype=torch.int32, device=DEV)
    b = buffers(T, d, E, k, 0, False)
    with pytest.raises(api.MoEError) as e:
        api.moe_permute_noalloc(x, idx, E, 0, b["x_perm"].view(torch.bfloat16), b["counts"],
                                b["offsets"], b["perm_src"], b["flat_to_row"])
    assert e.value.status == api.MOE_ERR_WORKSPACE
