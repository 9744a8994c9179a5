"""tq_decode_step (append the new token's key and value, then decode) against the oracle.

Each case builds a cache on the device, then runs one step with new key and
value rows for every (sequence, KV head). Checked:
  * the appended rows' codes, signs and norms against the oracle's quantiser
    applied to the new rows (outside the threshold windows, as every
    quantiser test);
  * every other row of the cache unchanged, bit for bit;
  * the attention output and scores against the oracle's decode over the
    GPU cache after the step, at the new lengths;
  * the same outputs and cache words as the two-call sequence (tq_append_kv
    per group, then tq_decode_attn).
Paths: head_dim 128 with S R folded (the appends run inside the decode's
query-transform launch; small and large launches), one and two channel
groups; head_dim 128 without S R (appends launched on their own); head_dim
64 (the general decode).
"""
import math

import numpy as np
import pytest

import synth
from oracle import tq as otq
from parity import REL_TOL, assert_codes_match, normwise_rel_err, rowmax_rel_err, torch_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import decode_tq_quantize_amd as tq
    from synth import device as sdev
    tq.lib()  # fail loudly if the library is missing


class _Group:
    """One channel group of a [B, Hkv, T_cap] cache on the device."""

    def __init__(self, ch, d, bits, prod, layout, seed, fold):
        self.ch, self.d, self.bits, self.prod, self.layout = ch, d, bits, prod, layout
        self.R = synth.haar_orthogonal(d, seed)
        self.S = synth.gaussian_matrix(d, d, seed) if prod else None
        self.Rt = torch_dev(self.R)
        self.St = torch_dev(self.S) if prod else None
        var = tq.TQ_PROD if prod else tq.TQ_MSE
        self.q = tq.tq_quantizer_init(d, bits, var, self.Rt, self.St)
        self.SRt = None
        if fold and prod:
            self.SRt = torch.empty(tq.tq_fold_bytes(d) // 4, dtype=torch.float32, device="cuda")
            tq.tq_quantizer_fold(self.q, self.SRt)
        self.oq = otq.make_quantizer(d, bits, prod, self.R, self.S)

    def alloc(self, n):
        var = tq.TQ_PROD if self.prod else tq.TQ_MSE
        nb = tq.tq_packed_bytes(self.d, self.bits, var, self.layout, n)
        self.pk = torch.empty(nb // 4, dtype=torch.int32, device="cuda")
        self.nr = torch.empty(n, dtype=torch.int16, device="cuda")
        self.rr = torch.empty(n, dtype=torch.int16, device="cuda") if self.prod else None

    def lay(self):
        return "keys" if self.layout == tq.TQ_LAYOUT_KEYS else "values"

    def unpack(self, n):
        words = self.pk.cpu().numpy().view(np.uint32)
        idx, z = otq.unpack(words, n, self.d, self.bits, self.prod, self.lay())
        n16 = self.nr.cpu().numpy().view(np.float16)
        r16 = self.rr.cpu().numpy().view(np.float16) if self.prod else np.zeros(n, np.float16)
        return idx, z, n16, r16


def _build(B, Hkv, T_cap, kspec, vspec, fold, seed):
    """Cache of B x Hkv x T_cap rows (quantised on the device) and its groups."""
    n = B * Hkv * T_cap
    caches = {}
    for name, spec, layout, stream in (("k", kspec, tq.TQ_LAYOUT_KEYS, 1), ("v", vspec, tq.TQ_LAYOUT_VALUES, 2)):
        D = sum(s[1] for s in spec)
        X = sdev.kv_with_outliers(B, Hkv, T_cap, D, 4, 10.0, seed, stream).view(n, D)
        groups = []
        for i, (ch, d, bits, prod) in enumerate(spec):
            g = _Group(ch, d, bits, prod, layout, seed + 10 * stream + i, fold)
            g.alloc(n)
            tq.tq_quantize_kv(g.q, layout, tq.TQ_BF16, X[:, ch:], n, D, g.pk, g.nr, g.rr)
            groups.append(g)
        caches[name] = groups
    torch.cuda.synchronize()
    return caches


def _desc(groups, T_cap):
    return tq.make_desc([tq.make_group(g.q, g.ch, g.pk, g.nr, g.rr, T_cap) for g in groups])


def _snapshot(caches):
    return {name: [(g.pk.clone(), g.nr.clone(), None if g.rr is None else g.rr.clone()) for g in gl]
            for name, gl in caches.items()}


def _restore(caches, snap):
    for name, gl in caches.items():
        for g, (pk, nr, rr) in zip(gl, snap[name]):
            g.pk.copy_(pk)
            g.nr.copy_(nr)
            if rr is not None:
                g.rr.copy_(rr)


CASES = [
    # B, Hq, Hkv, T_cap, lens before the step (-1: the sequence stays empty),
    # key groups, value groups, S R folded
    (3, 8, 2, 640, [300, 639, -1], [(0, 128, 3, True)], [(0, 128, 3, False)], True),
    (2, 32, 8, 512, [0, 511], [(0, 32, 2, True), (32, 96, 1, True)], [(0, 32, 3, False), (32, 96, 2, False)],
     True),
    (2, 8, 2, 384, [100, 257], [(0, 128, 2, True)], [(0, 128, 2, False)], False),
    (2, 8, 2, 256, [17, 255], [(0, 64, 3, True)], [(0, 64, 2, False)], True),
    # a large launch (4096 transform workgroups, 2048 append tiles)
    (64, 32, 8, 128, [int(x) for x in synth.rng(3, 9).integers(0, 127, 64)], [(0, 128, 3, True)],
     [(0, 128, 3, False)], True),
]


@pytest.mark.parametrize("B,Hq,Hkv,T_cap,lens0,kspec,vspec,fold", CASES)
def test_decode_step_matches_oracle(B, Hq, Hkv, T_cap, lens0, kspec, vspec, fold):
    print(f"decode step B={B} Hq={Hq} Hkv={Hkv} T_cap={T_cap} lens={lens0} k={kspec} v={vspec} fold={fold}",
          flush=True)
    seed = 7 + T_cap
    caches = _build(B, Hkv, T_cap, kspec, vspec, fold, seed)
    D = sum(s[1] for s in kspec)
    Dv = sum(s[1] for s in vspec)
    lens1 = [0 if L < 0 else L + 1 for L in lens0]
    rng = synth.rng(seed, 5)
    k_new = synth.bf16_bits_to_f32(synth.to_bf16_bits(rng.standard_normal((B, Hkv, D)).astype(np.float32)))
    v_new = synth.bf16_bits_to_f32(synth.to_bf16_bits(rng.standard_normal((B, Hkv, Dv)).astype(np.float32)))
    qry = synth.bf16_bits_to_f32(synth.to_bf16_bits(rng.standard_normal((B, Hq, D)).astype(np.float32)))
    kn_t = torch_dev(k_new, torch.bfloat16)
    vn_t = torch_dev(v_new, torch.bfloat16)
    q_t = torch_dev(qry, torch.bfloat16)
    sl = torch_dev(np.asarray(lens1, np.int32))
    kd, vd = _desc(caches["k"], T_cap), _desc(caches["v"], T_cap)
    wsb = tq.tq_decode_workspace_bytes(kd, vd, B, Hq, Hkv, T_cap)
    ws = torch.empty(wsb // 4 + 4, dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(D)
    before = _snapshot(caches)

    # the step
    out = torch.full((B, Hq, Dv), float("nan"), dtype=torch.float32, device="cuda")
    sc = torch.full((B, Hq, T_cap), float("nan"), dtype=torch.float32, device="cuda")
    tq.tq_decode_step(kd, vd, kn_t, vn_t, tq.TQ_BF16, q_t, tq.TQ_BF16, B, Hq, Hkv, T_cap, sl, scale, out, sc,
                      ws, wsb)
    torch.cuda.synchronize()
    after = _snapshot(caches)

    # the two-call sequence from the same starting cache
    _restore(caches, before)
    n = B * Hkv
    rows = np.array([(b * Hkv + g) * T_cap + lens1[b] - 1 if lens1[b] > 0 else -1
                     for b in range(B) for g in range(Hkv)], np.int64)
    rows_t = torch_dev(rows)
    for name, x_t, width in (("k", kn_t, D), ("v", vn_t, Dv)):
        for g in caches[name]:
            tq.tq_append_kv(g.q, g.layout, tq.TQ_BF16, x_t.view(n, width)[:, g.ch:], n, width, rows_t,
                            B * Hkv * T_cap, g.pk, g.nr, g.rr)
    out2 = torch.full_like(out, float("nan"))
    sc2 = torch.full_like(sc, float("nan"))
    tq.tq_decode_attn(kd, vd, q_t, tq.TQ_BF16, B, Hq, Hkv, T_cap, sl, scale, out2, sc2, ws, wsb)
    torch.cuda.synchronize()
    for name, gl in caches.items():
        for g, (pk, nr, rr) in zip(gl, after[name]):
            assert torch.equal(g.pk, pk) and torch.equal(g.nr, nr) and (rr is None or torch.equal(g.rr, rr)), \
                f"{name} group at channel {g.ch}: step and two-call caches differ"
    assert torch.equal(out, out2)
    for b, L in enumerate(lens1):
        assert torch.equal(sc[b, :, :L], sc2[b, :, :L])

    # the appended rows against the oracle's quantiser; every other row unchanged
    _restore(caches, after)
    N = B * Hkv * T_cap
    live = rows >= 0
    kgroups, vgroups = [], []
    for name, x, gl_out in (("k", k_new, kgroups), ("v", v_new, vgroups)):
        for g, (pk0, nr0, rr0) in zip(caches[name], before[name]):
            idx, z, n16, r16 = g.unpack(N)
            i0, z0 = otq.unpack(pk0.cpu().numpy().view(np.uint32), N, g.d, g.bits, g.prod, g.lay())
            other = np.ones(N, bool)
            other[rows[live]] = False
            assert np.array_equal(idx[other], i0[other]), f"{name}@{g.ch}: codes of other rows changed"
            if g.prod:
                assert np.array_equal(z[other], z0[other]), f"{name}@{g.ch}: signs of other rows changed"
            assert np.array_equal(n16.view(np.uint16)[other], nr0.cpu().numpy()[other].view(np.uint16))
            xs = x.reshape(n, -1)[live][:, g.ch:g.ch + g.d].astype(np.float64)
            want = otq.quantize(xs, g.oq)
            assert_codes_match(idx[rows[live]], None if z is None else z[rows[live]], n16[rows[live]],
                               r16[rows[live]] if g.prod else None, want, g.oq)
            shp = (B, Hkv, T_cap)
            c = otq.Codes(idx.reshape(shp + (g.d,)), None if z is None else z.reshape(shp + (g.d,)), None, None,
                          n16.reshape(shp), r16.reshape(shp), None, None)
            gl_out.append(otq.Group(g.ch, g.oq, c))

    # the attention at the new lengths, over the cache after the step
    o_out, o_sc = otq.decode_attention(qry.astype(np.float64), kgroups, vgroups, Hkv, lens1, scale)
    o = out.cpu().numpy()
    s = sc.cpu().numpy()
    worst = 0.0
    for b, L in enumerate(lens1):
        if L == 0:
            assert np.all(o[b] == 0)
            continue
        e_out = normwise_rel_err(o[b], o_out[b])
        e_sc = rowmax_rel_err(s[b, :, :L], o_sc[b, :, :L])
        worst = max(worst, e_out, e_sc)
        assert e_out <= REL_TOL and e_sc <= REL_TOL, f"batch {b}: output {e_out}, scores {e_sc}"
    print(f"decode step margin: {worst:.2e} (tolerance {REL_TOL:.0e})", flush=True)
