"""Needle-in-a-haystack proxy (riverfrot "TurboQuant" post, section 5.6) on the GPU.

One key per (sequence, KV head) is planted among random keys, aimed at the
group's first query head; the question is whether the top-scoring token is
still the needle after compression. The pages give no needle construction,
so the preservation rates themselves are unpinned; what is checked here is
parity: libtq's score argmax (its own quantiser, its own decode through the
C ABI) must be the oracle's argmax on the same codes, except where the
oracle's two best scores lie within the score tolerance of each other.
"""
import math

import numpy as np
import pytest

import synth
from oracle import tq as otq
from parity import REL_TOL, torch_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import decode_tq_quantize_amd as tq
    tq.lib()


@pytest.mark.parametrize("T", [1024, 4096, 16384])
@pytest.mark.parametrize("kb,kprod", [(3, True), (2, True), (4, False)])
def test_needle_argmax_matches_oracle(T, kb, kprod):
    print(f"needle T={T} keys {kb}{'+1' if kprod else ''}", flush=True)
    B, Hq, Hkv, d = 2, 32, 8, 128
    G = Hq // Hkv
    K = synth.kv_with_outliers(B, Hkv, T, d, 4, 10.0, T, synth.STREAM_DATA, synth.STREAM_OUTLIER)
    V = synth.kv_with_outliers(B, Hkv, T, d, 4, 10.0, T, synth.STREAM_NORM, synth.STREAM_R_V)
    qry = synth.bf16_bits_to_f32(synth.to_bf16_bits(synth.rng(T, 40).standard_normal((B, Hq, d)).astype(np.float32)))
    K, pos = synth.plant_needles(K, qry[:, ::G], 0.4, T)
    R = synth.haar_orthogonal(d, 7)
    S = synth.gaussian_matrix(d, d, 7) if kprod else None
    Rv = synth.haar_orthogonal(d, 7, synth.STREAM_R_V)
    Rt, Rvt = torch_dev(R), torch_dev(Rv)
    St = torch_dev(S) if kprod else None
    qk = tq.tq_quantizer_init(d, kb, tq.TQ_PROD if kprod else tq.TQ_MSE, Rt, St)
    SR = None
    if kprod:
        SR = torch.empty(tq.tq_fold_bytes(d) // 4, dtype=torch.float32, device="cuda")
        tq.tq_quantizer_fold(qk, SR)
    qv = tq.tq_quantizer_init(d, 3, tq.TQ_MSE, Rvt)
    n = B * Hkv * T
    var = tq.TQ_PROD if kprod else tq.TQ_MSE
    kp = torch.empty(tq.tq_packed_bytes(d, kb, var, tq.TQ_LAYOUT_KEYS, n) // 4, dtype=torch.int32, device="cuda")
    kn = torch.empty(n, dtype=torch.int16, device="cuda")
    kr = torch.empty(n, dtype=torch.int16, device="cuda") if kprod else None
    vp = torch.empty(tq.tq_packed_bytes(d, 3, tq.TQ_MSE, tq.TQ_LAYOUT_VALUES, n) // 4, dtype=torch.int32,
                     device="cuda")
    vn = torch.empty(n, dtype=torch.int16, device="cuda")
    tq.tq_quantize_kv(qk, tq.TQ_LAYOUT_KEYS, tq.TQ_BF16, torch_dev(K.reshape(n, d), torch.bfloat16), n, d, kp, kn, kr)
    tq.tq_quantize_kv(qv, tq.TQ_LAYOUT_VALUES, tq.TQ_BF16, torch_dev(V.reshape(n, d), torch.bfloat16), n, d, vp, vn)
    kd = tq.make_desc([tq.make_group(qk, 0, kp, kn, kr, T)])
    vd = tq.make_desc([tq.make_group(qv, 0, vp, vn, None, T)])
    wsb = tq.tq_decode_workspace_bytes(kd, vd, B, Hq, Hkv, T)
    ws = torch.empty(wsb // 4 + 4, dtype=torch.float32, device="cuda")
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    sc = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
    tq.tq_decode_attn(kd, vd, torch_dev(qry, torch.bfloat16), tq.TQ_BF16, B, Hq, Hkv, T, None, 1 / math.sqrt(d),
                      out, sc, ws, wsb)
    torch.cuda.synchronize()
    got = sc.cpu().numpy()[:, ::G]  # [B, Hkv, T]: each group's first query head
    # the oracle scores the GPU's own codes
    ki, kz = otq.unpack(kp.cpu().numpy().view(np.uint32), n, d, kb, kprod, "keys")
    shp = (B, Hkv, T)
    codes = otq.Codes(ki.reshape(shp + (d,)), None if kz is None else kz.reshape(shp + (d,)), None, None,
                      kn.cpu().numpy().view(np.float16).reshape(shp),
                      kr.cpu().numpy().view(np.float16).reshape(shp) if kprod else np.zeros(shp, np.float16),
                      None, None)
    oq = otq.make_quantizer(d, kb, kprod, R, S)
    want = otq.decode_scores(qry.astype(np.float64), [otq.Group(0, oq, codes)], Hkv)[:, ::G]
    hits_gpu = hits_oracle = 0
    for b in range(B):
        for g in range(Hkv):
            s = want[b, g]
            top2 = np.sort(s)[-2:]
            a_gpu, a_or = int(np.argmax(got[b, g])), int(np.argmax(s))
            if top2[1] - top2[0] > REL_TOL * np.max(np.abs(s)):
                assert a_gpu == a_or, (b, g, a_gpu, a_or)
            else:  # a near-tie: libtq's pick must be one of the tied tokens
                assert s[a_gpu] >= top2[1] - REL_TOL * np.max(np.abs(s))
            hits_gpu += a_gpu == pos[b, g]
            hits_oracle += a_or == pos[b, g]
    print(f"needle preserved: libtq {hits_gpu}/{B * Hkv}, oracle {hits_oracle}/{B * Hkv}", flush=True)
