"""GPU: lamp_decode_fwd_noalloc (split partials in the library's fixed
per-GPU scratch, nothing allocated) against lamp_decode_fwd (partials in a
workspace the caller passes), through the C ABI, on the same inputs: the
outputs and LSE must be equal bit for bit (same kernels, same splits), on
two calls in a row, the second with a smaller input, so that the scratch
holds the first call's partials when the second starts."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def L():
    import mixed_precision_tiled_amd as m
    return m


def run_pair(B, Hq, Hkv, S_q, S_k, D, causal, dtype, seed):
    m = L()
    dev = torch.device("cuda:0")
    print(f"[no-alloc] B{B} Hq{Hq} Hkv{Hkv} S_q{S_q} S_k{S_k} D{D} causal{causal} {dtype}",
          flush=True)
    g = torch.Generator(device=dev).manual_seed(seed)
    q = torch.randn((B, Hq, S_q, D), generator=g, device=dev).to(dtype)
    k = torch.randn((B, Hkv, S_k, D), generator=g, device=dev).to(dtype)
    v = torch.randn((B, Hkv, S_k, D), generator=g, device=dev).to(dtype)
    q8, sq = m.lamp_quantize_blocks(q, 64, "i8")
    k8, sk = m.lamp_quantize_blocks(k, 64, "i8")
    v8, sv = m.lamp_quantize_blocks(v, 64, "i8")
    assert m.lamp_decode_workspace_bytes(B, Hkv, S_k, D) <= m.LAMP_DECODE_SCRATCH_BYTES
    out_ref = torch.full((B, Hq, S_q, D), float("nan"), dtype=dtype, device=dev)
    lse_ref = torch.full((B, Hq, S_q), float("nan"), device=dev)
    m.lamp_decode_fwd(q8, sq, k8, sk, v8, sv, causal=causal, tile_m=64, dtype=dtype,
                      out=out_ref, lse=lse_ref)
    out = torch.full_like(out_ref, float("nan"))
    lse = torch.full_like(lse_ref, float("nan"))
    m.lamp_decode_fwd_noalloc(q8, sq, k8, sk, v8, sv, causal=causal, tile_m=64, out=out, lse=lse)
    torch.cuda.synchronize()
    a, b = out_ref.view(torch.int16).cpu().numpy(), out.view(torch.int16).cpu().numpy()
    assert np.isfinite(out.float().cpu().numpy()).all()
    assert (a == b).all()
    assert np.array_equal(lse_ref.cpu().numpy(), lse.cpu().numpy())


def test_noalloc_matches_workspace_entry_point_twice():
    # the benchmarked decode step (17 MB of partials), then a smaller one
    run_pair(8, 32, 8, 1, 32768, 128, True, torch.bfloat16, 1)
    run_pair(2, 8, 2, 3, 4097, 64, True, torch.float16, 2)
