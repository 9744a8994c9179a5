"""GPU parity at the full benchmark sizes, in the launch configurations bench.py times.

Every workload is built with the same seeded generators and the same calls
as the benchmark. The oracle then checks all outputs where it finishes in
seconds (the single-layer decode and both of its caches' quantisation) and
sampled outputs elsewhere: one layer of the prefill quantiser on sampled
vectors, the long-context decode on two (sequence, KV head) pairs, and the
vector search on sampled queries against their returned top-k and random
other database vectors.
"""
import math

import numpy as np
import pytest

import synth
from oracle import tq as otq
from parity import REL_TOL, assert_codes_match, assert_topk_match, normwise_rel_err, rowmax_rel_err, torch_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import decode_tq_quantize_amd as tq
    from synth import device as sdev
    from test_gpu_parity import GpuQuantizer, check_decode, gpu_quantize, run_decode, to_np_f16, to_np_u32
    tq.lib()


def _bf16_exact(x):
    return synth.bf16_bits_to_f32(synth.to_bf16_bits(x))


def _key_rows(words, rows, d, mse_bits, prod):
    """Codes of the given rows of a key-layout array (their whole 16-vector tiles unpacked)."""
    P = mse_bits + (1 if prod else 0)
    per_tile = (d // 32) * 16 * P
    tiles = np.unique(rows // 16)
    sub = words.reshape(-1, per_tile)[tiles].reshape(-1)
    idx, z = otq.unpack(sub, len(tiles) * 16, d, mse_bits, prod, "keys")
    pos = np.searchsorted(tiles, rows // 16) * 16 + rows % 16
    return idx[pos], (z[pos] if z is not None else None)


def _value_rows(words, rows, d, mse_bits, prod):
    """Codes of the given rows of a value-layout array (their whole 64-vector blocks unpacked)."""
    P = mse_bits + (1 if prod else 0)
    B = otq.VALUES_BLOCK
    per_block = B * d * P // 32
    blocks = np.unique(rows // B)
    sub = words.reshape(-1, per_block)[blocks].reshape(-1)
    idx, z = otq.unpack(sub, len(blocks) * B, d, mse_bits, prod, "values")
    pos = np.searchsorted(blocks, rows // B) * B + rows % B
    return idx[pos], (z[pos] if z is not None else None)


def _slice_words(words, r0, T, d, mse_bits, prod, layout):
    """Packed words of rows r0 .. r0 + T (r0 and T multiples of the layout's packing unit)."""
    P = mse_bits + (1 if prod else 0)
    unit = otq.KEYS_TILE if layout == "keys" else otq.VALUES_BLOCK
    per_row = d * P // 32  # words per vector, whole units
    return words[r0 // unit * unit * per_row:(r0 + T) // unit * unit * per_row]


def test_single_layer_decode_full_size():
    # batch 1, 32 query / 8 KV heads, head_dim 128, 32768 tokens; K 3 + 1
    # bits, V 3 bits; bf16 K, V with 4 of 128 channels x10, bf16 query
    B, Hq, Hkv, T, d = 1, 32, 8, 32768, 128
    n = B * Hkv * T
    print("full-size single-layer decode", flush=True)
    K = _bf16_exact(synth.kv_with_outliers(B, Hkv, T, d, 4, 10.0, 2, synth.STREAM_DATA, synth.STREAM_OUTLIER))
    V = _bf16_exact(synth.kv_with_outliers(B, Hkv, T, d, 4, 10.0, 2, synth.STREAM_NORM, synth.STREAM_R_V))
    qry = _bf16_exact(synth.rng(2, synth.STREAM_QUERY).standard_normal((B, Hq, d)).astype(np.float32))
    gk = GpuQuantizer(d, 3, True, seed=2, fold=True)
    gv = GpuQuantizer(d, 3, False, seed=2, r_stream=synth.STREAM_R_V)
    kp, kn, kr = gpu_quantize(gk, torch_dev(K.reshape(n, d), torch.bfloat16), n, d, tq.TQ_LAYOUT_KEYS, tq.TQ_BF16)
    vp, vn, _ = gpu_quantize(gv, torch_dev(V.reshape(n, d), torch.bfloat16), n, d, tq.TQ_LAYOUT_VALUES, tq.TQ_BF16)
    torch.cuda.synchronize()
    # the whole layer's codes against the oracle's quantiser
    ki, kz = otq.unpack(to_np_u32(kp), n, d, 3, True, "keys")
    vi, _ = otq.unpack(to_np_u32(vp), n, d, 3, False, "values")
    kn16, kr16, vn16 = to_np_f16(kn), to_np_f16(kr), to_np_f16(vn)
    assert_codes_match(ki, kz, kn16, kr16, otq.quantize(K.reshape(n, d).astype(np.float64), gk.oq), gk.oq)
    assert_codes_match(vi, None, vn16, None, otq.quantize(V.reshape(n, d).astype(np.float64), gv.oq), gv.oq)
    del K, V

    class _C:
        pass

    kc, vc = _C(), _C()
    kc.group = tq.make_group(gk.q, 0, kp, kn, kr, T)
    vc.group = tq.make_group(gv.q, 0, vp, vn, None, T)
    shp = (B, Hkv, T)
    ck = otq.Codes(ki.reshape(shp + (d,)), kz.reshape(shp + (d,)), None, None, kn16.reshape(shp), kr16.reshape(shp),
                   None, None)
    cv = otq.Codes(vi.reshape(shp + (d,)), None, None, None, vn16.reshape(shp), np.zeros(shp, np.float16), None, None)
    kg, vg = [otq.Group(0, gk.oq, ck)], [otq.Group(0, gv.oq, cv)]
    # the timed call (no score output), then once more with the raw scores
    out, _ = run_decode([kc], [vc], qry, Hkv, T, None, "bf16", scores=False)
    o_out, _ = check_decode(out, None, kg, vg, qry, Hkv, None)
    out2, sc = run_decode([kc], [vc], qry, Hkv, T, None, "bf16")
    check_decode(out2, sc, kg, vg, qry, Hkv, None)
    assert np.array_equal(out, out2)


@pytest.mark.parametrize("keys", [True, False])
def test_prefill_quantize_full_layer(keys):
    # one layer of the prefill workload per call, as the benchmark issues it:
    # 16 x 8192 tokens x 8 KV heads = 1,048,576 bf16 vectors with
    # LogNormal(0, 0.5) norms; keys 2 + 1 bits, values 3 bits
    L_seed, d, n = 1000 + (0 if keys else 1), 128, 16 * 8192 * 8
    print(f"full-size prefill quantise keys={keys}", flush=True)
    X = sdev.lognormal_norm_vectors(n, d, seed=L_seed)
    if keys:
        gq = GpuQuantizer(d, 2, True, seed=3)
        layout = tq.TQ_LAYOUT_KEYS
    else:
        gq = GpuQuantizer(d, 3, False, seed=3, r_stream=synth.STREAM_R_V)
        layout = tq.TQ_LAYOUT_VALUES
    packed, norm, rnorm = gpu_quantize(gq, X, n, d, layout, tq.TQ_BF16)
    torch.cuda.synchronize()
    rows = np.sort(synth.rng(L_seed, 7).choice(n, 16384, replace=False))
    # every tile's last vectors and the final rows are in the sample
    rows = np.unique(np.concatenate([rows, np.arange(n - 40, n), np.arange(31, n, n // 64)]))
    xs = X[torch_dev(rows.astype(np.int64))].float().cpu().numpy().astype(np.float64)
    idx, z = otq.unpack(to_np_u32(packed), n, d, gq.B, gq.prod, "keys" if keys else "values")
    want = otq.quantize(xs, gq.oq)
    assert_codes_match(idx[rows], None if z is None else z[rows], to_np_f16(norm)[rows],
                       None if rnorm is None else to_np_f16(rnorm)[rows], want, gq.oq)


@pytest.mark.parametrize("keys", [True, False])
def test_channel_group_quantize_large(keys):
    # the long-context cache's channel groups (32 outlier channels, 96 others;
    # keys 2 + 1 and 1 + 1 bits, values 3 and 2 bits) quantised as the
    # benchmark quantises them, strided out of 128-channel bf16 rows, for 8 of
    # its 64 sequences: 8 x 8 KV heads x 131072 tokens = 8,388,608 vectors per
    # call; sampled rows against the oracle
    n, d = 8 * 8 * 131072, 128
    stream = 11 if keys else 12
    print(f"channel-group quantise keys={keys} n={n}", flush=True)
    X = sdev.kv_with_outliers(8, 8, 131072, d, 0, 1.0, seed=4, stream=stream)
    X[..., :32] *= 10
    X = X.view(n, d)
    rows = np.sort(synth.rng(stream, 7).choice(n, 8192, replace=False))
    rows = np.unique(np.concatenate([rows, np.arange(n - 40, n), np.arange(31, n, n // 64)]))
    xs = X[torch_dev(rows.astype(np.int64))].float().cpu().numpy().astype(np.float64)
    groups = [(0, 32, 2, True), (32, 96, 1, True)] if keys else [(0, 32, 3, False), (32, 96, 2, False)]
    layout = tq.TQ_LAYOUT_KEYS if keys else tq.TQ_LAYOUT_VALUES
    for gi, (ch, gd, bits, prod) in enumerate(groups):
        seed = 40 + gi + 10 * stream
        R = synth.haar_orthogonal(gd, seed)
        S = synth.gaussian_matrix(gd, gd, seed) if prod else None
        R_t, S_t = torch_dev(R), (torch_dev(S) if prod else None)
        var = tq.TQ_PROD if prod else tq.TQ_MSE
        q = tq.tq_quantizer_init(gd, bits, var, R_t, S_t)
        pk = torch.empty(tq.tq_packed_bytes(gd, bits, var, layout, n) // 4, dtype=torch.int32, device="cuda")
        nr = torch.empty(n, dtype=torch.int16, device="cuda")
        rr = torch.empty(n, dtype=torch.int16, device="cuda") if prod else None
        tq.tq_quantize_kv(q, layout, tq.TQ_BF16, X[:, ch:], n, d, pk, nr, rr)
        torch.cuda.synchronize()
        words = to_np_u32(pk)
        idx, z = (_key_rows if keys else _value_rows)(words, rows, gd, bits, prod)
        oq = otq.make_quantizer(gd, bits, prod, R, S)
        want = otq.quantize(xs[:, ch:ch + gd], oq)
        assert_codes_match(idx, z, to_np_f16(nr)[rows], None if rr is None else to_np_f16(rr)[rows], want, oq)
        del pk, nr, rr


def test_long_context_decode_full_size():
    # batch 64 x 131072 tokens, 32 query / 8 KV heads, head_dim 128; keys in
    # two groups (32 outlier channels 2 + 1 bits, 96 channels 1 + 1 bits),
    # values 3 / 2 bits; checked on two (sequence, KV head) pairs
    B, Hq, Hkv, T, d = 64, 32, 8, 131072, 128
    G = Hq // Hkv
    n = B * Hkv * T
    print("full-size long-context decode", flush=True)
    groups_k = [(0, 32, 2, tq.TQ_PROD), (32, 96, 1, tq.TQ_PROD)]
    groups_v = [(0, 32, 3, tq.TQ_MSE), (32, 96, 2, tq.TQ_MSE)]
    pairs = [(0, 0), (63, 7)]
    keep, descs, host = [], {}, {}
    for name, groups, layout, stream in (("k", groups_k, tq.TQ_LAYOUT_KEYS, 11),
                                         ("v", groups_v, tq.TQ_LAYOUT_VALUES, 12)):
        X = sdev.kv_with_outliers(B, Hkv, T, d, 0, 1.0, seed=4, stream=stream)
        X[..., :32] *= 10
        X = X.view(n, d)
        gl = []
        for gi, (ch, gd, bits, var) in enumerate(groups):
            seed = 40 + gi + 10 * stream
            R = synth.haar_orthogonal(gd, seed)
            S = synth.gaussian_matrix(gd, gd, seed) if var == tq.TQ_PROD else None
            R_t, S_t = torch_dev(R), (torch_dev(S) if S is not None else None)
            q = tq.tq_quantizer_init(gd, bits, var, R_t, S_t)
            if var == tq.TQ_PROD:
                SR_t = torch.empty(tq.tq_fold_bytes(gd) // 4, dtype=torch.float32, device="cuda")
                tq.tq_quantizer_fold(q, SR_t)
                keep.append(SR_t)
            pk = torch.empty(tq.tq_packed_bytes(gd, bits, var, layout, n) // 4, dtype=torch.int32, device="cuda")
            nr = torch.empty(n, dtype=torch.int16, device="cuda")
            rr = torch.empty(n, dtype=torch.int16, device="cuda") if var == tq.TQ_PROD else None
            tq.tq_quantize_kv(q, layout, tq.TQ_BF16, X[:, ch:], n, d, pk, nr, rr)
            keep += [R_t, S_t, pk, nr, rr]
            gl.append(tq.make_group(q, ch, pk, nr, rr, T))
            oq = otq.make_quantizer(gd, bits, var == tq.TQ_PROD, R, S)
            torch.cuda.synchronize()
            for (b, g) in pairs:
                r0 = (b * Hkv + g) * T
                lay = "keys" if layout == tq.TQ_LAYOUT_KEYS else "values"
                words = _slice_words(pk, r0, T, gd, bits, var == tq.TQ_PROD, lay).cpu().numpy().view(np.uint32)
                idx, z = otq.unpack(words, T, gd, bits, var == tq.TQ_PROD, lay)
                n16 = nr[r0:r0 + T].cpu().numpy().view(np.float16)
                r16 = rr[r0:r0 + T].cpu().numpy().view(np.float16) if rr is not None else np.zeros(T, np.float16)
                c = otq.Codes(idx[None, None], None if z is None else z[None, None], None, None,
                              n16[None, None], r16[None, None], None, None)
                host.setdefault((name, b, g), []).append(otq.Group(ch, oq, c))
        del X
        torch.cuda.empty_cache()
        descs[name] = tq.make_desc(gl)
    q_t = torch.randn((B, Hq, d), generator=sdev.generator(4, 13), device="cuda").to(torch.bfloat16)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    wsb = tq.tq_decode_workspace_bytes(descs["k"], descs["v"], B, Hq, Hkv, T)
    ws = torch.empty(wsb // 4 + 4, dtype=torch.float32, device="cuda")
    tq.tq_decode_attn(descs["k"], descs["v"], q_t, tq.TQ_BF16, B, Hq, Hkv, T, None, 1 / math.sqrt(d), out,
                      None, ws, wsb)
    scores = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
    out2 = torch.empty_like(out)
    tq.tq_decode_attn(descs["k"], descs["v"], q_t, tq.TQ_BF16, B, Hq, Hkv, T, None, 1 / math.sqrt(d), out2,
                      scores, ws, wsb)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    qf = q_t.float().cpu().numpy()
    for (b, g) in pairs:
        qry = qf[b, g * G:(g + 1) * G][None].astype(np.float64)
        o_out, o_sc = otq.decode_attention(qry, host[("k", b, g)], host[("v", b, g)], 1, None, 1 / math.sqrt(d))
        got = out[b, g * G:(g + 1) * G].cpu().numpy()
        e_out = normwise_rel_err(got, o_out[0])
        assert e_out <= REL_TOL, f"(b={b}, g={g}) output error {e_out}"
        e_sc = rowmax_rel_err(scores[b, g * G:(g + 1) * G].cpu().numpy(), o_sc[0])
        assert e_sc <= REL_TOL, f"(b={b}, g={g}) score error {e_sc}"
        print(f"long-context decode margin (b={b}, g={g}): output {e_out:.2e}, scores {e_sc:.2e}", flush=True)


def test_vector_search_full_size():
    # 1M x 1536 unit-normalised Gaussian-mixture database, 1024 queries,
    # 3 + 1-bit codes, top-10 (the benchmark's call); four sampled queries
    # are checked against the oracle's scores of the whole database
    N, d, Q, k = 1 << 20, 1536, 1024, 10
    print("full-size vector search", flush=True)
    db, means = sdev.gaussian_mixture(N, d, 256, seed=5, stream=0)
    qs, _ = sdev.gaussian_mixture(Q, d, 256, seed=5, stream=1, means=means)
    gq = GpuQuantizer(d, 3, True, seed=5)
    pk, nr, rr = gpu_quantize(gq, db, N, d, tq.TQ_LAYOUT_KEYS, tq.TQ_F32)
    g = tq.make_group(gq.q, 0, pk, nr, rr, 0)
    wsb = tq.tq_search_workspace_bytes(g, N, Q, k)
    ws = torch.empty(wsb // 4 + 4, dtype=torch.float32, device="cuda")
    oi = torch.full((Q, k), -7, dtype=torch.int64, device="cuda")
    osc = torch.empty((Q, k), dtype=torch.float32, device="cuda")
    tq.tq_search_topk(g, N, qs, Q, k, oi, osc, ws, wsb)
    torch.cuda.synchronize()
    gi, gs = oi.cpu().numpy(), osc.cpu().numpy()
    words = to_np_u32(pk)
    n16, r16 = to_np_f16(nr), to_np_f16(rr)
    others = np.sort(synth.rng(5, 8).choice(N, 6000, replace=False))
    # the GPU's quantisation of sampled database vectors against the oracle's
    qrows = others[:1024]
    idx_q, z_q = _key_rows(words, qrows, d, 3, True)
    xs = db[torch_dev(qrows.astype(np.int64))].cpu().numpy().astype(np.float64)
    assert_codes_match(idx_q, z_q, n16[qrows], r16[qrows], otq.quantize(xs, gq.oq), gq.oq)
    # the oracle scores every one of the 1,048,576 database vectors (the
    # GPU's own codes, unpacked chunk by chunk) for four sampled queries, and
    # the returned lists must be its exact top-k up to ties within 1e-6
    sampled = [0, 341, 682, 1023]
    yq = qs[sampled].cpu().numpy().astype(np.float64)
    full = np.empty((len(sampled), N))
    chunk = 1 << 16
    per_row = d * 4 // 32
    for lo in range(0, N, chunk):
        idx, z = otq.unpack(words[lo * per_row:(lo + chunk) * per_row], chunk, d, 3, True, "keys")
        c = otq.Codes(idx, z, None, None, n16[lo:lo + chunk], r16[lo:lo + chunk], None, None)
        full[:, lo:lo + chunk] = otq.estimate_ip(yq, c, gq.oq)
    print("search: oracle scored the whole database for 4 queries", flush=True)
    for row, qi in enumerate(sampled):
        got = gi[qi]
        assert len(set(got.tolist())) == k and got.min() >= 0 and got.max() < N
        assert np.all(np.diff(gs[qi]) <= 1e-6)
        assert_topk_match(got[None], gs[qi][None], full[row][None], k)
