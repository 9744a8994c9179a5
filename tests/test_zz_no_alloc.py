"""tq_decode_attn_noalloc (workspace in the library's fixed per-GPU scratch
array) against tq_decode_attn with a caller workspace.

Both entry points run the same kernels with the same launch plan, so their
outputs and scores must agree bit for bit. The calls come two in a row, the
second on a smaller cache, so the second runs over the first one's leftovers
in the scratch array.
"""
import math

import numpy as np
import pytest

import synth
from synth import device as sdev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import decode_tq_quantize_amd as tq
    tq.lib()  # fail loudly if the library is missing


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class _Cache:
    """A [B, Hkv, T_cap] cache quantised on the device, keys and values each in
    channel groups given as (first channel, channels, bits)."""

    def __init__(self, B, Hkv, T_cap, kspec, vspec, seed):
        d = sum(g[1] for g in kspec)
        n = B * Hkv * T_cap
        K = sdev.kv_with_outliers(B, Hkv, T_cap, d, 4, 10.0, seed, 1).view(n, d)
        V = sdev.kv_with_outliers(B, Hkv, T_cap, d, 4, 10.0, seed, 2).view(n, d)
        self.keep = []
        self.k = self._groups(K, n, d, kspec, tq.TQ_PROD, tq.TQ_LAYOUT_KEYS, T_cap, seed)
        self.v = self._groups(V, n, d, vspec, tq.TQ_MSE, tq.TQ_LAYOUT_VALUES, T_cap, seed + 50)
        self.B, self.Hkv, self.T_cap, self.d = B, Hkv, T_cap, d

    def _groups(self, X, n, d, spec, variant, layout, T_cap, seed):
        groups = []
        for i, (ch, gd, bits) in enumerate(spec):
            R = _dev(synth.haar_orthogonal(gd, seed + i))
            S = _dev(synth.gaussian_matrix(gd, gd, seed + i)) if variant == tq.TQ_PROD else None
            q = tq.tq_quantizer_init(gd, bits, variant, R, S)
            nb = tq.tq_packed_bytes(gd, bits, variant, layout, n)
            pk = torch.empty(nb // 4, dtype=torch.int32, device="cuda")
            nr = torch.empty(n, dtype=torch.int16, device="cuda")
            rr = torch.empty(n, dtype=torch.int16, device="cuda") if variant == tq.TQ_PROD else None
            tq.tq_quantize_kv(q, layout, tq.TQ_BF16, X[:, ch:], n, d, pk, nr, rr)
            self.keep += [R, S, pk, nr, rr]
            groups.append(tq.make_group(q, ch, pk, nr, rr, T_cap))
        return tq.make_desc(groups)


def _both(cache, Hq, lens, seed):
    B, Hkv, T, d = cache.B, cache.Hkv, cache.T_cap, cache.d
    q = torch.randn((B, Hq, d), generator=sdev.generator(seed, 9), device="cuda").to(torch.bfloat16)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(d)
    ws_bytes = tq.tq_decode_workspace_bytes(cache.k, cache.v, B, Hq, Hkv, T)
    assert 0 < ws_bytes <= tq.TQ_DECODE_SCRATCH_BYTES
    ws = torch.empty(ws_bytes // 4 + 4, dtype=torch.float32, device="cuda")
    out_ws = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    sc_ws = torch.full((B, Hq, T), float("nan"), dtype=torch.float32, device="cuda")
    tq.tq_decode_attn(cache.k, cache.v, q, tq.TQ_BF16, B, Hq, Hkv, T, sl, scale, out_ws, sc_ws, ws, ws_bytes)
    out_na = torch.full_like(out_ws, float("nan"))
    sc_na = torch.full_like(sc_ws, float("nan"))
    tq.tq_decode_attn_noalloc(cache.k, cache.v, q, tq.TQ_BF16, B, Hq, Hkv, T, sl, scale, out_na, sc_na)
    torch.cuda.synchronize()
    assert torch.isfinite(out_na).all()
    assert torch.equal(out_na, out_ws)
    for b, L in enumerate(lens):  # scores are written for t < len only
        assert torch.equal(sc_na[b, :, :L], sc_ws[b, :, :L])
    print(f"noalloc: B={B} Hq={Hq} T={T} lens={lens} workspace {ws_bytes} bytes: identical", flush=True)


# 2.5 bits per channel: 32 outlier channels (keys 2+1 bits, values 3 bits) and
# 96 others (keys 1+1, values 2)
SPLIT_K = [(0, 32, 2), (32, 96, 1)]
SPLIT_V = [(0, 32, 3), (32, 96, 2)]


def test_noalloc_decode_equals_workspace_decode_twice():
    print("noalloc: call 1 (B=4, T=4096) then call 2 (B=2, T=1024)", flush=True)
    big = _Cache(4, 8, 4096, SPLIT_K, SPLIT_V, seed=21)
    _both(big, 32, [4096, 3001, 1, 2500], seed=21)
    small = _Cache(2, 8, 1024, SPLIT_K, SPLIT_V, seed=22)
    _both(small, 32, [1000, 17], seed=22)


def test_noalloc_decode_general_head_size():
    # 64-channel heads take the general decode kernel (a different workspace plan)
    print("noalloc: 64-channel heads (B=3, T=512)", flush=True)
    c = _Cache(3, 2, 512, [(0, 64, 3)], [(0, 64, 2)], seed=23)
    _both(c, 8, [512, 300, 0], seed=23)


def test_noalloc_rejects_requests_beyond_the_scratch():
    # 1024 sequences x 64 query heads need more than the fixed array: the call
    # returns TQ_ERR_SCRATCH before any device work
    c = _Cache(1, 8, 1024, SPLIT_K, SPLIT_V, seed=24)
    B, Hq = 1024, 64
    need = tq.tq_decode_workspace_bytes(c.k, c.v, B, Hq, 8, 1024)
    assert need > tq.TQ_DECODE_SCRATCH_BYTES
    fake = 1 << 20  # never dereferenced: the size check comes first
    rc = tq.lib().tq_decode_attn_noalloc(c.k, c.v, fake, tq.TQ_BF16, B, Hq, 8, 1024, None, 0.088, fake, None, None)
    assert rc == tq.TQ_ERR_SCRATCH
