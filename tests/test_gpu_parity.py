"""GPU parity of libtq against the fp64 oracle (calls go through the C ABI).

Each kernel is checked element by element on seeded inputs at sizes that
span several tiles and a ragged tail; decode and search are run both on
oracle-packed inputs and on GPU-packed inputs decoded by the oracle's own
unpacker, so a quantiser mismatch cannot hide a decode or search bug.
"""
import math

import numpy as np
import pytest

import synth
from oracle import tq as otq
from parity import (REL_TOL, assert_codes_match, assert_topk_match, normwise_rel_err, rowmax_rel_err,
                          torch_dev)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import decode_tq_quantize_amd as tq
    tq.lib()  # fail loudly if the library is missing


def _variant(prod):
    return tq.TQ_PROD if prod else tq.TQ_MSE


class GpuQuantizer:
    """Device copies of R and S plus the library quantiser that points at them."""

    def __init__(self, d, B, prod, seed, r_stream=synth.STREAM_R, s_stream=synth.STREAM_S, fold=False):
        self.R32 = synth.haar_orthogonal(d, seed, r_stream)
        self.S32 = synth.gaussian_matrix(d, d, seed, s_stream) if prod else None
        self.Rt = torch_dev(self.R32)
        self.St = torch_dev(self.S32) if prod else None
        self.q = tq.tq_quantizer_init(d, B, _variant(prod), self.Rt, self.St)
        self.SRt = None
        if fold and prod:  # S R precomputed: decode takes the one-pass query transform
            self.SRt = torch.empty(tq.tq_fold_bytes(d) // 4, dtype=torch.float32, device="cuda")
            tq.tq_quantizer_fold(self.q, self.SRt)
        self.d, self.B, self.prod = d, B, prod
        self.oq = otq.make_quantizer(d, B, prod, self.R32, self.S32)


def gpu_quantize(gq: GpuQuantizer, x_t, n, stride, layout, dtype):
    nbytes = tq.tq_packed_bytes(gq.d, gq.B, _variant(gq.prod), layout, n)
    packed = torch.full((nbytes // 4,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    norm = torch.zeros(n, dtype=torch.int16, device="cuda")
    rnorm = torch.zeros(n, dtype=torch.int16, device="cuda") if gq.prod else None
    tq.tq_quantize_kv(gq.q, layout, dtype, x_t, n, stride, packed, norm, rnorm)
    return packed, norm, rnorm


def to_np_u32(t):
    return t.cpu().numpy().view(np.uint32)


def to_np_f16(t):
    return None if t is None else t.cpu().numpy().view(np.float16)


def lay_name(layout):
    return "keys" if layout == tq.TQ_LAYOUT_KEYS else "values"


# --------------------------------------------------------------------------
# quantize
# --------------------------------------------------------------------------

QUANT_CASES = [
    (128, 3, True, "keys", 1000, "bf16"),
    (128, 2, True, "keys", 37, "f32"),
    (128, 3, False, "values", 1000, "bf16"),
    (128, 4, True, "keys", 333, "bf16"),
    (128, 2, True, "values", 100, "bf16"),
    (128, 1, True, "values", 70, "f32"),
    (128, 4, False, "values", 129, "f32"),
    (128, 1, False, "keys", 45, "bf16"),
    (32, 2, True, "keys", 100, "f32"),
    (96, 1, True, "keys", 100, "bf16"),
    (96, 2, False, "values", 77, "f32"),
    (256, 4, True, "keys", 50, "f32"),
    (64, 4, False, "values", 64, "bf16"),
    (1536, 3, True, "keys", 40, "f32"),
    (2048, 1, True, "keys", 5, "f32"),
    # channel groups on the matrix cores (d = 32, 64, 96): several tiles and a
    # ragged tail
    (32, 3, False, "values", 1000, "bf16"),
    (32, 1, True, "keys", 777, "bf16"),
    (64, 3, True, "keys", 333, "f32"),
    (64, 2, True, "values", 513, "bf16"),
    (96, 2, True, "keys", 1000, "bf16"),
    (96, 3, False, "values", 999, "bf16"),
    (96, 4, True, "values", 301, "bf16"),
    # wide vectors (more than 128 channels, key layout) on the GEMM-shaped
    # matrix-core passes: several 128-vector tiles and a ragged tail,
    # partial 128-channel tiles (160, 320), both input types
    (256, 2, True, "keys", 300, "bf16"),
    (1536, 3, True, "keys", 700, "f32"),
    (320, 1, False, "keys", 257, "f32"),
    (160, 4, True, "keys", 130, "bf16"),
    (384, 3, False, "keys", 129, "bf16"),
]


@pytest.mark.parametrize("d,B,prod,lay,N,dt", QUANT_CASES)
def test_quantize_matches_oracle(d, B, prod, lay, N, dt):
    print(f"quantize d={d} B={B} prod={prod} {lay} N={N} {dt}", flush=True)
    gq = GpuQuantizer(d, B, prod, seed=d + B)
    x = synth.unit_gaussian(N, d, 11) * synth.rng(12, 0).lognormal(0, 0.5, (N, 1)).astype(np.float32)
    x[min(3, N - 1)] = 0.0  # the zero-vector convention
    if dt == "bf16":
        x = synth.bf16_bits_to_f32(synth.to_bf16_bits(x))
    layout = tq.TQ_LAYOUT_KEYS if lay == "keys" else tq.TQ_LAYOUT_VALUES
    x_t = torch_dev(x, torch.bfloat16 if dt == "bf16" else torch.float32)
    packed, norm, rnorm = gpu_quantize(gq, x_t, N, d, layout, tq.TQ_BF16 if dt == "bf16" else tq.TQ_F32)
    torch.cuda.synchronize()
    words = to_np_u32(packed)
    idx, z = otq.unpack(words, N, d, B, prod, lay)
    codes = otq.quantize(x.astype(np.float64), gq.oq)
    assert_codes_match(idx, z, to_np_f16(norm), to_np_f16(rnorm), codes, gq.oq)
    # padding vectors of the last tile (64-vector block for values) are zero bits
    tile = otq.KEYS_TILE if lay == "keys" else otq.VALUES_BLOCK
    n_round = -(-N // tile) * tile
    pidx, pz = otq.unpack(words, n_round, d, B, prod, lay)
    assert not pidx[N:].any() and (pz is None or not pz[N:].any())


@pytest.mark.parametrize("d,B,prod,lay,N,dt", [
    (128, 2, True, "keys", 300, "bf16"),
    (128, 3, False, "values", 200, "bf16"),
    (64, 3, True, "keys", 97, "f32"),
    (256, 2, True, "keys", 150, "bf16"),
    (256, 3, False, "values", 70, "f32"),
])
def test_quantize_asymmetric_codebook(d, B, prod, lay, N, dt):
    """A codebook whose middle threshold is not 0 (sorted, as the library
    accepts): zero vectors still get index L / 2 (and rho 0, signs +),
    padding still all-zero bits, every path (narrow and wide matrix-core
    kernels, the vector-unit kernel)."""
    print(f"asymmetric codebook d={d} B={B} prod={prod} {lay} N={N} {dt}", flush=True)
    gq = GpuQuantizer(d, B, prod, seed=d + 7 * B)
    L = 1 << B
    cent = np.array(gq.q.centroids[:L], np.float64) + 0.35 / np.sqrt(d)
    thr = 0.5 * (cent[:-1] + cent[1:])
    assert thr[L // 2 - 1] > 0.0  # the middle threshold is off zero
    cent32, thr32 = cent.astype(np.float32), thr.astype(np.float32)
    for i in range(L):
        gq.q.centroids[i] = float(cent32[i])
    for i in range(L - 1):
        gq.q.thresholds[i] = float(thr32[i])
    gq.oq = otq.make_quantizer(d, B, prod, gq.R32, gq.S32, cent32.astype(np.float64), thr32.astype(np.float64))
    x = synth.unit_gaussian(N, d, 21) * synth.rng(22, 0).lognormal(0, 0.5, (N, 1)).astype(np.float32)
    for z in (0, 5, 40, N - 1):  # zero vectors in the first tile, later tiles and the ragged tail
        x[z] = 0.0
    if dt == "bf16":
        x = synth.bf16_bits_to_f32(synth.to_bf16_bits(x))
    layout = tq.TQ_LAYOUT_KEYS if lay == "keys" else tq.TQ_LAYOUT_VALUES
    x_t = torch_dev(x, torch.bfloat16 if dt == "bf16" else torch.float32)
    packed, norm, rnorm = gpu_quantize(gq, x_t, N, d, layout, tq.TQ_BF16 if dt == "bf16" else tq.TQ_F32)
    torch.cuda.synchronize()
    words = to_np_u32(packed)
    idx, z = otq.unpack(words, N, d, B, prod, lay)
    codes = otq.quantize(x.astype(np.float64), gq.oq)
    assert (codes.idx[[0, 5, 40, N - 1]] == L // 2).all()
    assert_codes_match(idx, z, to_np_f16(norm), to_np_f16(rnorm), codes, gq.oq)
    tile = otq.KEYS_TILE if lay == "keys" else otq.VALUES_BLOCK
    n_round = -(-N // tile) * tile
    pidx, pz = otq.unpack(words, n_round, d, B, prod, lay)
    assert not pidx[N:].any() and (pz is None or not pz[N:].any())


def test_quantize_wide_across_batches():
    # wide vectors are quantised in batches of 65536 (the residual workspace
    # holds one batch): 65536 + 300 vectors of 256 channels cross a batch
    # boundary mid-key-tile free (65536 is a multiple of 128); every code,
    # sign and norm against the oracle
    d, B, N = 256, 2, 65536 + 300
    print(f"quantize wide d={d} B={B} N={N} across batches", flush=True)
    gq = GpuQuantizer(d, B, True, seed=29)
    x = synth.unit_gaussian(N, d, 31) * synth.rng(32, 0).lognormal(0, 0.5, (N, 1)).astype(np.float32)
    x[65535] = 0.0  # a zero vector at the end of the first batch
    packed, norm, rnorm = gpu_quantize(gq, torch_dev(x), N, d, tq.TQ_LAYOUT_KEYS, tq.TQ_F32)
    torch.cuda.synchronize()
    idx, z = otq.unpack(to_np_u32(packed), N, d, B, True, "keys")
    codes = otq.quantize(x.astype(np.float64), gq.oq)
    assert_codes_match(idx, z, to_np_f16(norm), to_np_f16(rnorm), codes, gq.oq)


APPEND_CASES = [
    # d, B, prod, layout, dtype, cache rows, appended rows (the count picks the
    # kernel's tile: 2 vectors per workgroup below 1024 (matrices straight to
    # registers up to 64 vectors of d <= 128, staged through LDS above), 4
    # below 2048, 8 below 4096, 16 below 8192, 32 from 8192)
    (128, 3, True, "keys", "bf16", 2000, 500),
    (128, 3, False, "values", "bf16", 2000, 65),
    (128, 3, True, "keys", "bf16", 203, 61),
    (128, 3, False, "values", "bf16", 203, 61),
    (128, 2, True, "values", "f32", 203, 61),
    (96, 1, True, "keys", "f32", 203, 61),
    (32, 2, False, "values", "bf16", 203, 61),
    (256, 4, True, "keys", "f32", 203, 61),
    (128, 3, True, "keys", "bf16", 4000, 1500),
    (128, 3, False, "values", "bf16", 6000, 2500),
    (128, 3, True, "keys", "bf16", 6000, 4300),
    (128, 3, False, "values", "f32", 12000, 9000),
    (1536, 3, True, "keys", "f32", 700, 300),
]


@pytest.mark.parametrize("d,B,prod,lay,dt,C,n_in", APPEND_CASES)
def test_append_writes_only_its_rows(d, B, prod, lay, dt, C, n_in):
    # vectors appended into rows of an existing cache (unsorted, not tile
    # aligned, sharing tiles, the first and last row, two rows outside the
    # cache): the appended rows decode to the oracle's codes, every other
    # bit and norm of the cache is unchanged
    print(f"append d={d} B={B} prod={prod} {lay} {dt} C={C} n={n_in}", flush=True)
    gq = GpuQuantizer(d, B, prod, seed=d + 3 * B)
    layout = tq.TQ_LAYOUT_KEYS if lay == "keys" else tq.TQ_LAYOUT_VALUES
    g = synth.rng(d + B, 9)
    rows = np.concatenate([[C - 1, 0], g.choice(np.arange(1, C - 1), n_in - 2, replace=False)]).astype(np.int64)
    g.shuffle(rows)
    rows_all = np.concatenate([rows[:n_in // 2], [-1], rows[n_in // 2:], [C]]).astype(np.int64)  # two outside
    n = rows_all.size
    x = synth.unit_gaussian(n, d, 21) * g.lognormal(0, 0.5, (n, 1)).astype(np.float32)
    x[5] = 0.0
    if dt == "bf16":
        x = synth.bf16_bits_to_f32(synth.to_bf16_bits(x))
    nbytes = tq.tq_packed_bytes(d, B, _variant(prod), layout, C)
    w0 = g.integers(0, 2**32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    n0 = g.integers(0, 2**16, C, dtype=np.uint64).astype(np.uint16)
    r0 = g.integers(0, 2**16, C, dtype=np.uint64).astype(np.uint16)
    packed = torch_dev(w0.view(np.int32))
    norm = torch_dev(n0.view(np.int16))
    rnorm = torch_dev(r0.view(np.int16)) if prod else None
    x_t = torch_dev(x, torch.bfloat16 if dt == "bf16" else torch.float32)
    tq.tq_append_kv(gq.q, layout, tq.TQ_BF16 if dt == "bf16" else tq.TQ_F32, x_t, n, d, torch_dev(rows_all), C,
                    packed, norm, rnorm)
    torch.cuda.synchronize()
    tile = otq.KEYS_TILE if lay == "keys" else otq.VALUES_BLOCK
    n_round = -(-C // tile) * tile
    w1 = to_np_u32(packed)
    idx0, z0 = otq.unpack(w0, n_round, d, B, prod, lay)
    idx1, z1 = otq.unpack(w1, n_round, d, B, prod, lay)
    other = np.ones(n_round, bool)
    other[rows] = False
    assert np.array_equal(idx1[other], idx0[other])
    if prod:
        assert np.array_equal(z1[other], z0[other])
    n1 = to_np_f16(norm).view(np.uint16)
    assert np.array_equal(n1[other[:C]], n0[other[:C]])
    r1 = to_np_f16(rnorm).view(np.uint16) if prod else None
    if prod:
        assert np.array_equal(r1[other[:C]], r0[other[:C]])
    keep = (rows_all >= 0) & (rows_all < C)
    codes = otq.quantize(x[keep].astype(np.float64), gq.oq)
    rk = rows_all[keep]
    assert_codes_match(idx1[rk], None if not prod else z1[rk], n1[rk].view(np.float16),
                       None if not prod else r1[rk].view(np.float16), codes, gq.oq)


@pytest.mark.parametrize("dk,dv", [(128, 128), (128, 64)])
def test_append_pair_equals_two_appends(dk, dv):
    # one launch for keys and values writes exactly what two appends write
    print(f"append pair dk={dk} dv={dv}", flush=True)
    C, n = 4096, 700
    gk = GpuQuantizer(dk, 3, True, seed=7, fold=True)
    gv = GpuQuantizer(dv, 3, False, seed=8, r_stream=synth.STREAM_R_V)
    g = synth.rng(dk + dv, 10)
    rows = torch_dev(g.choice(C, n, replace=False).astype(np.int64))
    xk = torch_dev(synth.unit_gaussian(n, dk, 1) * 3, torch.bfloat16)
    xv = torch_dev(synth.unit_gaussian(n, dv, 2) * 2, torch.bfloat16)

    def cache(gq, lay):
        nbytes = tq.tq_packed_bytes(gq.d, 3, _variant(gq.prod), lay, C)
        w = torch_dev(g.integers(0, 2**32, nbytes // 4, dtype=np.uint64).astype(np.uint32).view(np.int32))
        nrm = torch_dev(g.integers(0, 2**16, C, dtype=np.uint64).astype(np.uint16).view(np.int16))
        rn = torch_dev(g.integers(0, 2**16, C, dtype=np.uint64).astype(np.uint16).view(np.int16)) if gq.prod else None
        return w, nrm, rn

    kA, vA = cache(gk, tq.TQ_LAYOUT_KEYS), cache(gv, tq.TQ_LAYOUT_VALUES)
    kB = tuple(None if t is None else t.clone() for t in kA)
    vB = tuple(None if t is None else t.clone() for t in vA)
    tq.tq_append_kv_pair(gk.q, gv.q, tq.TQ_BF16, xk, xv, n, dk, dv, rows, C, kA[0], kA[1], kA[2], vA[0], vA[1])
    tq.tq_append_kv(gk.q, tq.TQ_LAYOUT_KEYS, tq.TQ_BF16, xk, n, dk, rows, C, kB[0], kB[1], kB[2])
    tq.tq_append_kv(gv.q, tq.TQ_LAYOUT_VALUES, tq.TQ_BF16, xv, n, dv, rows, C, vB[0], vB[1])
    torch.cuda.synchronize()
    for a_, b_ in zip(kA + vA, kB + vB):
        if a_ is not None:
            assert torch.equal(a_, b_)


def test_quantize_strided_channel_group():
    # quantise channels 32..127 of 128-channel rows (a channel group)
    N, D = 200, 128
    gq = GpuQuantizer(96, 1, True, seed=5)
    x = synth.bf16_bits_to_f32(synth.to_bf16_bits(synth.rng(3, 0).standard_normal((N, D)).astype(np.float32)))
    x_t = torch_dev(x, torch.bfloat16)
    packed, norm, rnorm = gpu_quantize(gq, x_t[:, 32:], N, D, tq.TQ_LAYOUT_KEYS, tq.TQ_BF16)
    torch.cuda.synchronize()
    idx, z = otq.unpack(to_np_u32(packed), N, 96, 1, True, "keys")
    assert_codes_match(idx, z, to_np_f16(norm), to_np_f16(rnorm), otq.quantize(x[:, 32:].astype(np.float64), gq.oq),
                       gq.oq)


def test_quantize_is_deterministic():
    gq = GpuQuantizer(128, 3, True, seed=1)
    x_t = torch_dev(synth.unit_gaussian(4096, 128, 2))
    a = gpu_quantize(gq, x_t, 4096, 128, tq.TQ_LAYOUT_KEYS, tq.TQ_F32)
    b = gpu_quantize(gq, x_t, 4096, 128, tq.TQ_LAYOUT_KEYS, tq.TQ_F32)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


# --------------------------------------------------------------------------
# decode attention
# --------------------------------------------------------------------------

class Cache:
    """One compressed K or V channel group of a [B, Hkv, T_cap] cache, on the device."""

    def __init__(self, gq: GpuQuantizer, ch, codes: otq.Codes, T_cap, layout):
        B, H, T, d = codes.idx.shape
        n_all = B * H * T_cap
        idx = np.zeros((B, H, T_cap, d), np.uint8)
        idx[:, :, :T] = codes.idx
        z = None
        if gq.prod:
            z = np.zeros((B, H, T_cap, d), bool)
            z[:, :, :T] = codes.z
        n16 = np.zeros((B, H, T_cap), np.float16)
        n16[:, :, :T] = codes.n16
        r16 = np.zeros((B, H, T_cap), np.float16)
        r16[:, :, :T] = codes.rho16
        words = otq.pack(idx.reshape(n_all, d), None if z is None else z.reshape(n_all, d), gq.B, layout)
        self.packed = torch_dev(words.view(np.int32))
        self.norm = torch_dev(n16.reshape(-1).view(np.int16))
        self.rnorm = torch_dev(r16.reshape(-1).view(np.int16)) if gq.prod else None
        self.group = tq.make_group(gq.q, ch, self.packed, self.norm, self.rnorm, T_cap)


def run_decode(kcaches, vcaches, qry, Hkv, T_cap, seq_lens, qdt, scores=True):
    B, Hq, D = qry.shape
    Dv = sum(c.group.q.d for c in vcaches)
    kd = tq.make_desc([c.group for c in kcaches])
    vd = tq.make_desc([c.group for c in vcaches])
    ws_bytes = tq.tq_decode_workspace_bytes(kd, vd, B, Hq, Hkv, T_cap)
    ws = torch.empty(ws_bytes // 4 + 4, dtype=torch.float32, device="cuda")
    q_t = torch_dev(qry.astype(np.float32), torch.bfloat16 if qdt == "bf16" else torch.float32)
    out = torch.full((B, Hq, Dv), float("nan"), dtype=torch.float32, device="cuda")
    sc = torch.full((B, Hq, T_cap), float("nan"), dtype=torch.float32, device="cuda") if scores else None
    sl = torch_dev(np.asarray(seq_lens, np.int32)) if seq_lens is not None else None
    tq.tq_decode_attn(kd, vd, q_t, tq.TQ_BF16 if qdt == "bf16" else tq.TQ_F32, B, Hq, Hkv, T_cap, sl,
                      1.0 / math.sqrt(D), out, sc, ws, ws_bytes)
    torch.cuda.synchronize()
    return out.cpu().numpy(), None if sc is None else sc.cpu().numpy()


def check_decode(out, sc, kgroups, vgroups, qry, Hkv, seq_lens):
    B, Hq, D = qry.shape
    o_out, o_sc = otq.decode_attention(qry.astype(np.float64), kgroups, vgroups, Hkv, seq_lens,
                                       1.0 / math.sqrt(D))
    lens = seq_lens if seq_lens is not None else [o_sc.shape[2]] * B
    worst_out = worst_sc = 0.0
    for b in range(B):
        L = int(lens[b])
        if L == 0:
            assert np.all(out[b] == 0)
            continue
        e_out = normwise_rel_err(out[b], o_out[b])
        worst_out = max(worst_out, e_out)
        assert e_out <= REL_TOL, f"batch {b}: output error {e_out}"
        if sc is not None:
            e_sc = rowmax_rel_err(sc[b, :, :L], o_sc[b, :, :L])
            worst_sc = max(worst_sc, e_sc)
            assert e_sc <= REL_TOL, f"batch {b}: score error {e_sc}"
    # the margin against the 2e-3 tolerance, for the record
    print(f"decode margin: output {worst_out:.2e}, scores {worst_sc:.2e} (tolerance {REL_TOL:.0e})", flush=True)
    return o_out, o_sc


def make_kv(B, Hkv, T, d, seed):
    K = synth.kv_with_outliers(B, Hkv, T, d, 4, 10.0, seed, synth.STREAM_DATA, synth.STREAM_OUTLIER)
    V = synth.kv_with_outliers(B, Hkv, T, d, 4, 10.0, seed, synth.STREAM_NORM, synth.STREAM_R_V)
    return K, V


DECODE_CASES = [
    # B, Hq, Hkv, T, T_cap, seq_lens, kB, vB, qdt
    (2, 8, 2, 300, 320, [300, 123], 3, 3, "bf16"),
    (1, 32, 8, 1024, 1024, None, 3, 3, "bf16"),
    (3, 4, 1, 65, 128, [1, 64, 65], 2, 2, "f32"),
    (2, 4, 2, 63, 64, [0, 63], 1, 1, "f32"),
]


@pytest.mark.parametrize("fold", [False, True])
@pytest.mark.parametrize("B,Hq,Hkv,T,T_cap,seq_lens,kB,vB,qdt", DECODE_CASES)
def test_decode_matches_oracle_on_oracle_packed_cache(B, Hq, Hkv, T, T_cap, seq_lens, kB, vB, qdt, fold):
    print(f"decode B={B} Hq={Hq} Hkv={Hkv} T={T} lens={seq_lens} fold={fold}", flush=True)
    _decode_case(B, Hq, Hkv, T, T_cap, seq_lens, kB, vB, qdt, 128, fold)


@pytest.mark.parametrize("d,Hq,Hkv,kB,vB", [(64, 8, 2, 3, 2), (256, 4, 2, 2, 3), (128, 16, 2, 4, 4), (128, 6, 2, 1, 1)])
def test_decode_other_head_sizes_and_tiles(d, Hq, Hkv, kB, vB):
    # head sizes other than 128 (general kernel), GQA groups of 8 (two
    # head tiles), groups of 3 (a partial tile) and 4-bit codebooks
    print(f"decode d={d} Hq={Hq} Hkv={Hkv} kB={kB} vB={vB}", flush=True)
    _decode_case(2, Hq, Hkv, 700, 768, [700, 333], kB, vB, "bf16", d)


def _decode_case(B, Hq, Hkv, T, T_cap, seq_lens, kB, vB, qdt, d, fold=False, kprod=True):
    K, V = make_kv(B, Hkv, T, d, seed=T)
    gk = GpuQuantizer(d, kB, kprod, seed=1, fold=fold)
    gv = GpuQuantizer(d, vB, False, seed=2, r_stream=synth.STREAM_R_V)
    ck, cv = otq.quantize(K, gk.oq), otq.quantize(V, gv.oq)
    qry = synth.rng(T, 30).standard_normal((B, Hq, d)).astype(np.float32)
    if qdt == "bf16":
        qry = synth.bf16_bits_to_f32(synth.to_bf16_bits(qry))
    kc = Cache(gk, 0, ck, T_cap, "keys")
    vc = Cache(gv, 0, cv, T_cap, "values")
    out, sc = run_decode([kc], [vc], qry, Hkv, T_cap, seq_lens, qdt)
    check_decode(out, sc, [otq.Group(0, gk.oq, ck)], [otq.Group(0, gv.oq, cv)], qry, Hkv, seq_lens)


@pytest.mark.parametrize("d,kB,kprod,vB", [
    (128, 4, False, 3), (128, 3, False, 3), (128, 2, False, 2), (128, 4, False, 2),  # MSE-only keys
    (128, 3, True, 2), (128, 1, True, 4),  # asymmetric key / value widths
    (64, 3, False, 2),  # MSE-only keys on the general kernel
])
def test_decode_key_value_bit_allocations(d, kB, kprod, vB):
    # keys without the QJL sketch (TurboQuant_mse: no sign plane, no residual
    # norm, no S R q) and keys and values at different widths
    print(f"decode d={d} keys {kB}{'+1' if kprod else ''} values {vB}", flush=True)
    _decode_case(2, 8, 2, 600, 640, [600, 257], kB, vB, "bf16", d, fold=kprod, kprod=kprod)


@pytest.mark.parametrize("b_total", [2, 3, 4])
def test_score_matrix_tiny_workload(b_total):
    # 4096 unit keys, 64 unit queries, d = 128, TurboQuant_prod at b = 2, 3, 4
    # (b - 1 MSE bits + 1 QJL bit), 64 x 4096 score matrix, seed 0.
    d, N, Q = 128, 4096, 64
    keys = synth.unit_gaussian(N, d, 0, synth.STREAM_DATA)
    qry = synth.unit_gaussian(Q, d, 0, synth.STREAM_QUERY)
    gk = GpuQuantizer(d, b_total - 1, True, seed=0)
    gv = GpuQuantizer(d, 2, False, seed=0, r_stream=synth.STREAM_R_V)
    ck = otq.quantize(keys[None, None], gk.oq)
    cv = otq.quantize(keys[None, None], gv.oq)
    kc = Cache(gk, 0, ck, N, "keys")
    vc = Cache(gv, 0, cv, N, "values")
    out, sc = run_decode([kc], [vc], qry[None], 1, N, None, "f32")
    check_decode(out, sc, [otq.Group(0, gk.oq, ck)], [otq.Group(0, gv.oq, cv)], qry[None], 1, None)


@pytest.mark.parametrize("fold", [False, True])
def test_decode_two_channel_groups(fold):
    # 2.5 bits per channel: 32 outlier channels (keys 2+1 bits, values 3 bits)
    # and 96 others (keys 1+1, values 2), each group with its own norms.
    B, Hq, Hkv, T, T_cap = 2, 8, 2, 200, 256
    K, V = make_kv(B, Hkv, T, 128, seed=4)
    ka, kb = GpuQuantizer(32, 2, True, 1, fold=fold), GpuQuantizer(96, 1, True, 2, fold=fold)
    va, vb = GpuQuantizer(32, 3, False, 3), GpuQuantizer(96, 2, False, 4)
    cka, ckb = otq.quantize(K[..., :32], ka.oq), otq.quantize(K[..., 32:], kb.oq)
    cva, cvb = otq.quantize(V[..., :32], va.oq), otq.quantize(V[..., 32:], vb.oq)
    qry = synth.bf16_bits_to_f32(synth.to_bf16_bits(synth.rng(9, 0).standard_normal((B, Hq, 128)).astype(np.float32)))
    kcs = [Cache(ka, 0, cka, T_cap, "keys"), Cache(kb, 32, ckb, T_cap, "keys")]
    vcs = [Cache(va, 0, cva, T_cap, "values"), Cache(vb, 32, cvb, T_cap, "values")]
    out, sc = run_decode(kcs, vcs, qry, Hkv, T_cap, [200, 150], "bf16")
    check_decode(out, sc, [otq.Group(0, ka.oq, cka), otq.Group(32, kb.oq, ckb)],
                 [otq.Group(0, va.oq, cva), otq.Group(32, vb.oq, cvb)], qry, Hkv, [200, 150])


def paged_group(gq: GpuQuantizer, ch, codes: otq.Codes, table, bt, num_blocks, layout, rng, lens=None,
                garbage=None):
    """One channel group of a paged cache: a pool of num_blocks blocks of bt
    rows per KV head holding every (sequence, head, token) at row
    (table[b, t // bt] * H + g) * bt + t % bt; the other rows hold random
    codes and finite random norms (never to be read as the cache's). With
    `garbage` (IEEE half bits), every row that is not a token t < lens[b] of
    its sequence holds those bits as its norms instead."""
    B, H, T, d = codes.idx.shape
    rows = num_blocks * H * bt
    idx = rng.integers(0, 1 << gq.B, (rows, d)).astype(np.uint8)
    z = (rng.random((rows, d)) < 0.5) if gq.prod else None
    n16 = np.abs(rng.standard_normal(rows)).astype(np.float16)
    r16 = np.abs(rng.standard_normal(rows)).astype(np.float16)
    if garbage is not None:
        n16[:] = np.uint16(garbage).view(np.float16)
        r16[:] = np.uint16(garbage).view(np.float16)
    for b in range(B):
        for g in range(H):
            for t0 in range(0, T, bt):
                r0 = (int(table[b, t0 // bt]) * H + g) * bt
                nt = min(bt, T - t0)
                if garbage is not None:
                    nt = max(0, min(nt, int(lens[b]) - t0))
                idx[r0:r0 + nt] = codes.idx[b, g, t0:t0 + nt]
                if gq.prod:
                    z[r0:r0 + nt] = codes.z[b, g, t0:t0 + nt]
                    r16[r0:r0 + nt] = codes.rho16[b, g, t0:t0 + nt]
                n16[r0:r0 + nt] = codes.n16[b, g, t0:t0 + nt]
    words = otq.pack(idx, z, gq.B, layout)
    c = Cache.__new__(Cache)
    c.packed = torch_dev(words.view(np.int32))
    c.norm = torch_dev(n16.view(np.int16))
    c.rnorm = torch_dev(r16.view(np.int16)) if gq.prod else None
    c.group = tq.make_group(gq.q, ch, c.packed, c.norm, c.rnorm, bt)
    c.gq = gq  # keeps R, S and S R (which the group points at) alive
    return c


@pytest.mark.parametrize("bt,split", [(256, False), (1024, False), (512, True)])
def test_decode_paged_cache(bt, split):
    # the cache in a shuffled pool of blocks with spare (garbage) blocks; one
    # or two channel groups; sequences ending inside a block
    print(f"paged decode block={bt} groups={2 if split else 1}", flush=True)
    B, Hq, Hkv, T, d = 2, 8, 2, 1500, 128
    lens = [1500, 700]
    K, V = make_kv(B, Hkv, T, d, seed=bt)
    rng = synth.rng(bt, 5)
    nbs = -(-T // bt)
    max_blocks = nbs + 1
    num_blocks = B * nbs + 3
    table = np.full((B, max_blocks), -1, np.int32)
    table[:, :nbs] = rng.permutation(num_blocks)[:B * nbs].reshape(B, nbs)
    if split:
        specs_k = [(0, 32, 2, True, 1), (32, 96, 1, True, 2)]
        specs_v = [(0, 32, 3, False, 3), (32, 96, 2, False, 4)]
    else:
        specs_k = [(0, 128, 3, True, 1)]
        specs_v = [(0, 128, 3, False, 2)]
    kcs, vcs, kgs, vgs = [], [], [], []
    for specs, X, caches, ogs, lay in ((specs_k, K, kcs, kgs, "keys"), (specs_v, V, vcs, vgs, "values")):
        for ch, gd, bits, prod, seed in specs:
            gq = GpuQuantizer(gd, bits, prod, seed, fold=prod,
                              r_stream=synth.STREAM_R if lay == "keys" else synth.STREAM_R_V)
            codes = otq.quantize(X[..., ch:ch + gd], gq.oq)
            caches.append(paged_group(gq, ch, codes, table, bt, num_blocks, lay, rng))
            ogs.append(otq.Group(ch, gq.oq, codes))
    qry = synth.bf16_bits_to_f32(synth.to_bf16_bits(synth.rng(bt, 31).standard_normal((B, Hq, d)).astype(np.float32)))
    kd = tq.make_desc([c.group for c in kcs])
    vd = tq.make_desc([c.group for c in vcs])
    wsb = tq.tq_decode_paged_workspace_bytes(kd, vd, B, Hq, Hkv, T, bt)
    assert wsb > 0
    ws = torch.empty(wsb // 4 + 4, dtype=torch.float32, device="cuda")
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    sc = torch.full((B, Hq, T), float("nan"), dtype=torch.float32, device="cuda")
    tq.tq_decode_attn_paged(kd, vd, torch_dev(qry, torch.bfloat16), tq.TQ_BF16, B, Hq, Hkv, T,
                            torch_dev(np.asarray(lens, np.int32)), torch_dev(table), max_blocks, bt, num_blocks,
                            1.0 / math.sqrt(d), out, sc, ws, wsb)
    torch.cuda.synchronize()
    check_decode(out.cpu().numpy(), sc.cpu().numpy(), kgs, vgs, qry, Hkv, lens)


GARBAGE_HALF_BITS = [0x7E00, 0xFC00, 0x8001, 0x7BFF]  # NaN, -inf, a negative subnormal, the largest half
SPECS_ONE = ([(0, 128, 3, True, 1)], [(0, 128, 3, False, 2)])
SPECS_SPLIT = ([(0, 32, 2, True, 1), (32, 96, 1, True, 2)], [(0, 32, 3, False, 3), (32, 96, 2, False, 4)])


def _groups(specs, X, lay):
    gqs, codes = [], []
    for ch, gd, bits, prod, seed in specs:
        gq = GpuQuantizer(gd, bits, prod, seed, fold=prod,
                          r_stream=synth.STREAM_R if lay == "keys" else synth.STREAM_R_V)
        gqs.append(gq)
        codes.append(otq.quantize(X[..., ch:ch + gd], gq.oq))
    return gqs, codes


@pytest.mark.parametrize("bits", GARBAGE_HALF_BITS)
@pytest.mark.parametrize("split", [False, True])
def test_decode_ignores_rows_past_the_length(bits, split):
    # rows at or past a sequence's length hold norm bits no quantiser writes
    # (a cache allocated uninitialised and filled by appends): the decode must
    # not let them into any result; lengths 1 and 300 leave whole splits empty
    print(f"decode rows past the length: norm bits {bits:#06x}, groups {2 if split else 1}", flush=True)
    B, Hq, Hkv, T, d = 3, 16, 2, 1024, 128
    lens = [1000, 1, 300]
    K, V = make_kv(B, Hkv, T, d, seed=bits & 0xff)
    specs_k, specs_v = SPECS_SPLIT if split else SPECS_ONE
    kq, kcodes = _groups(specs_k, K, "keys")
    vq, vcodes = _groups(specs_v, V, "values")
    gbits = np.uint16(bits).view(np.float16)
    for c in kcodes + vcodes:
        for b, L in enumerate(lens):
            c.n16[b, :, L:] = gbits
            c.rho16[b, :, L:] = gbits
    kcs = [Cache(gq, specs_k[i][0], kcodes[i], T, "keys") for i, gq in enumerate(kq)]
    vcs = [Cache(gq, specs_v[i][0], vcodes[i], T, "values") for i, gq in enumerate(vq)]
    qry = synth.rng(bits, 31).standard_normal((B, Hq, d)).astype(np.float32)
    out, sc = run_decode(kcs, vcs, qry, Hkv, T, lens, "f32")
    assert np.isfinite(out).all()
    with np.errstate(invalid="ignore", over="ignore"):
        check_decode(out, sc, [otq.Group(s[0], gq.oq, c) for s, gq, c in zip(specs_k, kq, kcodes)],
                     [otq.Group(s[0], gq.oq, c) for s, gq, c in zip(specs_v, vq, vcodes)], qry, Hkv, lens)


@pytest.mark.parametrize("split", [False, True])
def test_decode_query_dynamic_range(split):
    # the score operands carry one power-of-two scale per 32-channel block of
    # each query head: a head of zeros, a zero block beside normal ones, a
    # block whose largest entry is 1e4 times the rest, and heads scaled by
    # 2^-100 and 2^100 must all score like the oracle
    print(f"decode query dynamic range: groups {2 if split else 1}", flush=True)
    B, Hq, Hkv, T, d = 2, 8, 2, 512, 128
    lens = [512, 77]
    K, V = make_kv(B, Hkv, T, d, seed=41)
    specs_k, specs_v = SPECS_SPLIT if split else SPECS_ONE
    kq, kcodes = _groups(specs_k, K, "keys")
    vq, vcodes = _groups(specs_v, V, "values")
    kcs = [Cache(gq, specs_k[i][0], kcodes[i], T, "keys") for i, gq in enumerate(kq)]
    vcs = [Cache(gq, specs_v[i][0], vcodes[i], T, "values") for i, gq in enumerate(vq)]
    qry = synth.rng(41, 32).standard_normal((B, Hq, d)).astype(np.float32)
    qry[0, 0] = 0.0
    qry[0, 1, 32:64] = 0.0
    qry[0, 2, 64:96] *= 1e-4
    qry[0, 2, 70] = 3.0
    qry[1, 3] *= np.float32(2.0 ** -100)
    qry[1, 5] *= np.float32(2.0 ** 100)
    out, sc = run_decode(kcs, vcs, qry, Hkv, T, lens, "f32")
    assert np.isfinite(out).all()
    assert np.all(sc[0, 0, :lens[0]] == 0.0)
    check_decode(out, sc, [otq.Group(s[0], gq.oq, c) for s, gq, c in zip(specs_k, kq, kcodes)],
                 [otq.Group(s[0], gq.oq, c) for s, gq, c in zip(specs_v, vq, vcodes)], qry, Hkv, lens)


@pytest.mark.parametrize("bits", [0x7E00, 0x8001])
def test_paged_decode_ignores_rows_past_the_length(bits):
    print(f"paged decode rows past the length: norm bits {bits:#06x}", flush=True)
    B, Hq, Hkv, T, d, bt = 2, 8, 2, 1500, 128, 512
    lens = [1500, 300]
    K, V = make_kv(B, Hkv, T, d, seed=7)
    rng = synth.rng(7, 5)
    nbs = -(-T // bt)
    num_blocks = B * nbs + 2
    table = np.full((B, nbs + 1), -1, np.int32)
    table[:, :nbs] = rng.permutation(num_blocks)[:B * nbs].reshape(B, nbs)
    kcs, vcs, kgs, vgs = [], [], [], []
    for specs, X, caches, ogs, lay in ((SPECS_SPLIT[0], K, kcs, kgs, "keys"), (SPECS_SPLIT[1], V, vcs, vgs, "values")):
        gqs, codes = _groups(specs, X, lay)
        for (ch, *_), gq, c in zip(specs, gqs, codes):
            caches.append(paged_group(gq, ch, c, table, bt, num_blocks, lay, rng, lens, bits))
            ogs.append(otq.Group(ch, gq.oq, c))
    qry = synth.rng(3, 31).standard_normal((B, Hq, d)).astype(np.float32)
    kd = tq.make_desc([c.group for c in kcs])
    vd = tq.make_desc([c.group for c in vcs])
    wsb = tq.tq_decode_paged_workspace_bytes(kd, vd, B, Hq, Hkv, T, bt)
    ws = torch.empty(wsb // 4 + 4, dtype=torch.float32, device="cuda")
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    sc = torch.full((B, Hq, T), float("nan"), dtype=torch.float32, device="cuda")
    tq.tq_decode_attn_paged(kd, vd, torch_dev(qry), tq.TQ_F32, B, Hq, Hkv, T,
                            torch_dev(np.asarray(lens, np.int32)), torch_dev(table), nbs + 1, bt, num_blocks,
                            1.0 / math.sqrt(d), out, sc, ws, wsb)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.isfinite(o).all()
    check_decode(o, sc.cpu().numpy(), kgs, vgs, qry, Hkv, lens)


@pytest.mark.parametrize("fold", [False, True])
def test_decode_on_gpu_quantized_cache(fold):
    # stage isolation: the GPU quantiser writes the cache, the oracle decodes
    # the GPU's own codes, and the GPU decode must agree with that.
    B, Hq, Hkv, T = 1, 8, 2, 512
    d = 128
    K, V = make_kv(B, Hkv, T, d, seed=8)
    gk = GpuQuantizer(d, 3, True, seed=1, fold=fold)
    gv = GpuQuantizer(d, 3, False, seed=2, r_stream=synth.STREAM_R_V)
    n = B * Hkv * T
    kp, kn, kr = gpu_quantize(gk, torch_dev(K.reshape(n, d), torch.bfloat16), n, d, tq.TQ_LAYOUT_KEYS, tq.TQ_BF16)
    vp, vn, _ = gpu_quantize(gv, torch_dev(V.reshape(n, d), torch.bfloat16), n, d, tq.TQ_LAYOUT_VALUES, tq.TQ_BF16)
    torch.cuda.synchronize()
    ki, kz = otq.unpack(to_np_u32(kp), n, d, 3, True, "keys")
    vi, _ = otq.unpack(to_np_u32(vp), n, d, 3, False, "values")
    shp = (B, Hkv, T)
    ck = otq.Codes(ki.reshape(shp + (d,)), kz.reshape(shp + (d,)), None, None, to_np_f16(kn).reshape(shp),
                   to_np_f16(kr).reshape(shp), None, None)
    cv = otq.Codes(vi.reshape(shp + (d,)), None, None, None, to_np_f16(vn).reshape(shp), np.zeros(shp, np.float16),
                   None, None)
    qry = synth.rng(1, 31).standard_normal((B, Hq, d)).astype(np.float32)
    kd = tq.make_group(gk.q, 0, kp, kn, kr, T)
    vd = tq.make_group(gv.q, 0, vp, vn, None, T)

    class _C:
        pass

    kc, vc = _C(), _C()
    kc.group, vc.group = kd, vd
    out, sc = run_decode([kc], [vc], qry, Hkv, T, None, "f32")
    check_decode(out, sc, [otq.Group(0, gk.oq, ck)], [otq.Group(0, gv.oq, cv)], qry, Hkv, None)


def test_decode_is_deterministic():
    B, Hq, Hkv, T = 1, 32, 8, 2048
    K, V = make_kv(B, Hkv, T, 128, seed=3)
    gk = GpuQuantizer(128, 3, True, seed=1)
    gv = GpuQuantizer(128, 3, False, seed=2, r_stream=synth.STREAM_R_V)
    kc = Cache(gk, 0, otq.quantize(K, gk.oq), T, "keys")
    vc = Cache(gv, 0, otq.quantize(V, gv.oq), T, "values")
    qry = synth.rng(2, 0).standard_normal((B, Hq, 128)).astype(np.float32)
    a = run_decode([kc], [vc], qry, Hkv, T, None, "f32")
    b = run_decode([kc], [vc], qry, Hkv, T, None, "f32")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_decode_across_split_counts(monkeypatch):
    # the same cache decoded with the sequence cut into splits of 256, 1024
    # and 4096 tokens (and the shape's own choice): each run repeats bit for
    # bit, each matches the oracle, and the runs agree within the tolerance
    # (a missing barrier or a split-boundary error shows up as a difference)
    B, Hq, Hkv, T = 2, 32, 8, 4096
    lens = [4096, 2500]
    K, V = make_kv(B, Hkv, T, 128, seed=5)
    gk = GpuQuantizer(128, 3, True, seed=1, fold=True)
    gv = GpuQuantizer(128, 3, False, seed=2, r_stream=synth.STREAM_R_V)
    ck, cv = otq.quantize(K, gk.oq), otq.quantize(V, gv.oq)
    kc = Cache(gk, 0, ck, T, "keys")
    vc = Cache(gv, 0, cv, T, "values")
    qry = synth.rng(5, 0).standard_normal((B, Hq, 128)).astype(np.float32)
    kd = tq.make_desc([kc.group])
    vd = tq.make_desc([vc.group])
    outs, sizes = [], set()
    for sl in ("256", "1024", "4096", None):
        if sl is None:
            monkeypatch.delenv("TQ_DECODE_SPLIT_TOKENS", raising=False)
        else:
            monkeypatch.setenv("TQ_DECODE_SPLIT_TOKENS", sl)
        print(f"decode split tokens {sl}", flush=True)
        sizes.add(tq.tq_decode_workspace_bytes(kd, vd, B, Hq, Hkv, T))
        a = run_decode([kc], [vc], qry, Hkv, T, lens, "f32")
        b = run_decode([kc], [vc], qry, Hkv, T, lens, "f32")
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1], equal_nan=True)
        check_decode(a[0], a[1], [otq.Group(0, gk.oq, ck)], [otq.Group(0, gv.oq, cv)], qry, Hkv, lens)
        outs.append(a[0])
    assert len(sizes) >= 3  # the partials' workspace follows the split count
    for o in outs[1:]:
        for bb in range(B):
            assert normwise_rel_err(o[bb], outs[0][bb].astype(np.float64)) <= REL_TOL


@pytest.mark.parametrize("d", [32, 96, 128, 1536])
def test_fold_matches_matrix_product(d):
    # S R and its largest row norm against a float64 product of the same
    # fp32 matrices; the norm must bound every row (it is rounded up).
    print(f"fold d={d}", flush=True)
    gq = GpuQuantizer(d, 2, True, seed=d, fold=True)
    sr = gq.SRt.cpu().numpy()
    want = gq.S32.astype(np.float64) @ gq.R32.astype(np.float64)
    got = sr[:d * d].reshape(d, d)
    assert np.max(np.abs(got - want)) <= 2e-5 * np.max(np.abs(want))
    rn = np.sqrt((got.astype(np.float64) ** 2).sum(axis=1))
    assert sr[d * d] >= rn.max() and sr[d * d] <= rn.max() * (1 + 1e-5)
    assert np.all(sr[d * d + 1:d * d + 4] == 0)


# --------------------------------------------------------------------------
# search
# --------------------------------------------------------------------------

def run_search(gq, packed, norm, rnorm, N, queries, k, want_ws=False):
    db = tq.make_group(gq.q, 0, packed, norm, rnorm, 0)
    Q = queries.shape[0]
    ws_bytes = tq.tq_search_workspace_bytes(db, N, Q, k)
    ws = torch.empty(ws_bytes // 4 + 4, dtype=torch.float32, device="cuda")
    oi = torch.full((Q, k), -7, dtype=torch.int64, device="cuda")
    osc = torch.empty((Q, k), dtype=torch.float32, device="cuda")
    tq.tq_search_topk(db, N, torch_dev(queries.astype(np.float32)), Q, k, oi, osc, ws, ws_bytes)
    torch.cuda.synchronize()
    if want_ws:
        return oi.cpu().numpy(), osc.cpu().numpy(), ws.cpu().numpy()
    return oi.cpu().numpy(), osc.cpu().numpy()


@pytest.mark.parametrize("d,B,N,Q,k", [(128, 3, 3001, 16, 10), (256, 2, 777, 5, 64), (96, 1, 100, 3, 100 // 2)])
def test_search_matches_oracle_on_oracle_packed_db(d, B, N, Q, k):
    gq = GpuQuantizer(d, B, True, seed=d)
    db, means = synth.gaussian_mixture(N, d, 16, seed=d)
    qs, _ = synth.gaussian_mixture(Q, d, 16, seed=d, stream=synth.STREAM_QUERY, means=means)
    codes = otq.quantize(db.astype(np.float64), gq.oq)
    words = otq.pack(codes.idx, codes.z, B, "keys")
    gi, gs = run_search(gq, torch_dev(words.view(np.int32)), torch_dev(codes.n16.view(np.int16)),
                        torch_dev(codes.rho16.view(np.int16)), N, qs, k)
    full = otq.estimate_ip(qs.astype(np.float64), codes, gq.oq)
    assert_topk_match(gi, gs, full, k)


def test_search_on_gpu_quantized_db_d1536():
    d, N, Q, k = 1536, 2000, 8, 10
    gq = GpuQuantizer(d, 3, True, seed=7)
    db, means = synth.gaussian_mixture(N, d, 32, seed=7)
    qs, _ = synth.gaussian_mixture(Q, d, 32, seed=7, stream=synth.STREAM_QUERY, means=means)
    packed, norm, rnorm = gpu_quantize(gq, torch_dev(db), N, d, tq.TQ_LAYOUT_KEYS, tq.TQ_F32)
    torch.cuda.synchronize()
    idx, z = otq.unpack(to_np_u32(packed), N, d, 3, True, "keys")
    codes = otq.Codes(idx, z, None, None, to_np_f16(norm), to_np_f16(rnorm), None, None)
    gi, gs = run_search(gq, packed, norm, rnorm, N, qs, k)
    full = otq.estimate_ip(qs.astype(np.float64), codes, gq.oq)
    assert_topk_match(gi, gs, full, k)
    # recall against exact inner products is reported, not pinned
    truth, _ = otq.exact_topk(qs, db, k)
    print("recall@10", otq.recall_at_k(gi, truth))


@pytest.mark.parametrize("k", [1, 10, 64])
def test_search_topk_selects_exactly_from_the_score_rows(k):
    # The selection is exact on the fp32 scores the scan produced (the
    # workspace holds them as [Q, N] after the [Q, 2 d] query transforms):
    # the same indices in the same order, equal scores by ascending index.
    # Every database vector appears about ten times, so the rows are full of
    # exact ties; N = 50001 leaves rows that start off a 16-byte boundary and
    # gives each wave of the selection several chunks.
    d, B, N, Q = 128, 3, 50001, 7
    print(f"topk selection k={k} N={N}", flush=True)
    gq = GpuQuantizer(d, B, True, seed=11)
    base, means = synth.gaussian_mixture(5000, d, 16, seed=11)
    pick = synth.rng(11, synth.STREAM_QUERY + 7).integers(0, 5000, size=N)
    db = base[pick]
    qs, _ = synth.gaussian_mixture(Q, d, 16, seed=12, stream=synth.STREAM_QUERY, means=means)
    packed, norm, rnorm = gpu_quantize(gq, torch_dev(db), N, d, tq.TQ_LAYOUT_KEYS, tq.TQ_F32)
    torch.cuda.synchronize()
    gi, gs, ws = run_search(gq, packed, norm, rnorm, N, qs, k, want_ws=True)
    sc = ws[Q * 2 * d:Q * 2 * d + Q * N].reshape(Q, N)
    ties = 0
    for i in range(Q):
        order = np.lexsort((np.arange(N), -sc[i].astype(np.float64)))[:k]
        assert np.array_equal(gi[i], order), (i, gi[i], order)
        assert np.array_equal(gs[i], sc[i][order])
        ties += int(np.sum(sc[i][order][1:] == sc[i][order][:-1]))
    if k > 1:
        assert ties > 0  # the case the index order decides was exercised
