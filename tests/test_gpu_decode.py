"""GPU parity of lamp_decode_fwd (attention over an int8 key/value cache)
against oracle.decode, element by element."""
import numpy as np
import pytest
import torch

from oracle import compare, decode
from gpu_util import record_path

pytestmark = pytest.mark.gpu


def L():
    import mixed_precision_tiled_amd as m
    return m


def dev():
    return torch.device("cuda:0")


def rand16(shape, seed, dtype):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g).to(dtype)


DT = {"bf16": torch.bfloat16, "f16": torch.float16}

CASES = [
    # D, dtype, B, Hq, Hkv, S_q, S_k, causal, tile_m
    (128, "bf16", 2, 32, 8, 1, 5000, True, 64),      # one new token, Qwen3-8B-like heads
    (128, "bf16", 1, 8, 2, 4, 777, True, 64),        # a few new tokens, ragged cache
    (64, "f16", 2, 4, 4, 8, 300, False, 64),
    (128, "bf16", 1, 4, 1, 8, 64, True, 128),        # 32 columns, one tile
    (128, "f16", 1, 2, 2, 3, 1, False, 64),          # a one-key cache
    (64, "bf16", 3, 16, 2, 2, 4097, True, 64),       # more than one split, ragged last split
    # the benchmarked step: batch 8, Qwen3-8B heads, one new token over a
    # 32768-token cache (32-tile splits, 16 per (batch, KV head))
    (128, "bf16", 8, 32, 8, 1, 32768, True, 64),
    # the longest supported cache, 2^20 keys: 16-tile splits, 1024 of them;
    # Q times 6 (logits of standard deviation 6), so that each query's few
    # largest keys, wherever they lie, dominate its output
    (128, "bf16", 1, 8, 1, 1, 1 << 20, True, 64, 6.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "d{}_{}_b{}_h{}x{}_q{}_k{}_{}".format(
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], "causal" if c[7] else "full"))
def test_decode_parity(case):
    D, dt, B, Hq, Hkv, S_q, S_k, causal, tm, *qmul = case
    print(f"[decode] {case}", flush=True)
    q = rand16((B, Hq, S_q, D), 1, DT[dt])
    if qmul:
        q = q * qmul[0]
    k = rand16((B, Hkv, S_k, D), 2, DT[dt])
    v = rand16((B, Hkv, S_k, D), 3, DT[dt])
    qd, kd, vd = q.to(dev()), k.to(dev()), v.to(dev())
    q8, sq = L().lamp_quantize_blocks(qd, tm, "i8")
    k8, sk = L().lamp_quantize_blocks(kd, 64, "i8")
    v8, sv = L().lamp_quantize_blocks(vd, 64, "i8")
    lse = torch.full((B, Hq, S_q), float("nan"), device=dev())
    out = L().lamp_decode_fwd(q8, sq, k8, sk, v8, sv, causal=causal, tile_m=tm, dtype=DT[dt],
                              lse=lse)
    torch.cuda.synchronize()
    P, (vc, vs) = decode.decode_problem(q.double().numpy(), k.double().numpy(),
                                        v.double().numpy(), causal=causal, tile_m=tm)
    assert (q8.cpu().numpy() == P.q_codes).all() and (k8.cpu().numpy() == P.k_codes).all()
    assert (v8.cpu().numpy() == vc).all() and (sv.cpu().numpy() == vs).all()
    got, glse = out.float().cpu().numpy(), lse.cpu().numpy()
    for b in range(B):
        for h in range(Hq):
            O, lse_ref = decode.decode_attention(P, b, h, np.arange(S_q))
            if qmul:
                assert np.abs(O).max() > 0.5
            st = compare.check(got[b, h], O, dt)
            assert st["ok"], f"({b},{h}): {st}"
            lse_tol = 2e-3 + 1e-5 * np.abs(lse_ref).max()
            lse_dev = np.abs(glse[b, h] - lse_ref)
            assert lse_dev.max() <= lse_tol
            record_path("decode", st, got[b, h], O, dt, None, lse_dev, np.full(lse_dev.shape, lse_tol))


def test_decode_graph_replay_matches_eager():
    # a decode step captured in a HIP graph (split and merge kernels, no
    # memset nodes) and replayed: every replay equals the eager call bit for
    # bit, also after new query codes are written into the captured buffer
    m = L()
    B, Hq, Hkv, S_k, D = 2, 32, 8, 5000, 128
    print("[decode] graph replay", flush=True)
    q = rand16((B, Hq, 1, D), 11, torch.bfloat16).to(dev())
    k = rand16((B, Hkv, S_k, D), 12, torch.bfloat16).to(dev())
    v = rand16((B, Hkv, S_k, D), 13, torch.bfloat16).to(dev())
    q8, sq = m.lamp_quantize_blocks(q, 64, "i8")
    k8, sk = m.lamp_quantize_blocks(k, 64, "i8")
    v8, sv = m.lamp_quantize_blocks(v, 64, "i8")
    out = torch.empty((B, Hq, 1, D), dtype=torch.bfloat16, device=dev())
    ws = torch.empty(m.lamp_decode_workspace_bytes(B, Hkv, S_k, D), dtype=torch.uint8,
                     device=dev())

    def run():
        m.lamp_decode_fwd(q8, sq, k8, sk, v8, sv, causal=True, tile_m=64, dtype=torch.bfloat16,
                          out=out, workspace=ws)

    run()
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        run()
    for _ in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
    q2 = rand16((B, Hq, 1, D), 14, torch.bfloat16).to(dev())
    q8b, sqb = m.lamp_quantize_blocks(q2, 64, "i8")
    q8.copy_(q8b)
    sq.copy_(sqb)
    run()
    torch.cuda.synchronize()
    ref2 = out.clone()
    assert not torch.equal(ref2, ref)
    for _ in range(2):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref2)


def test_decode_workspace_and_errors():
    m = L()
    # 79 tiles x 16 (b, KV head) groups -> 8-tile splits (the minimum), 10 of them
    assert m.lamp_decode_workspace_bytes(2, 8, 5000, 128) == 2 * 8 * 10 * 32 * 130 * 4
    # the Qwen3-8B-like step: 512 tiles x 64 groups -> 32-tile splits (the maximum)
    assert m.lamp_decode_workspace_bytes(8, 8, 32768, 128) == 8 * 8 * 16 * 32 * 130 * 4
    x = torch.zeros((1, 40, 2, 128), dtype=torch.uint8, device=dev())
    s = torch.zeros((1, 40, 1), dtype=torch.float32, device=dev())
    kx = torch.zeros((1, 1, 64, 128), dtype=torch.uint8, device=dev())
    ks = torch.zeros((1, 1, 1), dtype=torch.float32, device=dev())
    with pytest.raises(m.LampError):          # (Hq / Hkv) * S_q = 80 > 32
        m.lamp_decode_fwd(x, s, kx, ks, kx, ks, causal=True, tile_m=64, dtype=torch.bfloat16)
    small = torch.empty(16, dtype=torch.uint8, device=dev())
    with pytest.raises(m.LampError):          # workspace too small
        m.lamp_decode_fwd(x[:, :8], s[:, :8], kx, ks, kx, ks, causal=True, tile_m=64,
                          dtype=torch.bfloat16, workspace=small)
