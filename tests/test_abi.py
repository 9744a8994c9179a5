"""C-ABI contract of libtq, checked on the CPU (no kernel is launched).

* the library loads and exports every function include/tq.h declares;
* the ctypes mirrors of the structs have the C layout (a gcc-compiled probe
  prints sizeof/offsetof from the header itself);
* the host codebook equals the oracle's Lloyd-Max codebook;
* every validation path returns its status before touching the device.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import decode_tq_quantize_amd as tq
from oracle import tq as otq
from oracle import codebook as ocb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tq.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(tq.EXPORTS)
    L = tq.lib()
    for n in names:
        assert hasattr(L, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", tq.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}\b", nm), f"{n} not exported"


def test_struct_layout_matches_header(tmp_path):
    probe = tmp_path / "probe.c"
    probe.write_text(r'''
#include <stdio.h>
#include <stddef.h>
#include "tq.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu %zu\n", sizeof(tq_quantizer), offsetof(tq_quantizer, R),
         offsetof(tq_quantizer, SR), offsetof(tq_quantizer, centroids), offsetof(tq_quantizer, thresholds),
         sizeof(tq_group), offsetof(tq_group, packed), offsetof(tq_group, seq_stride), sizeof(tq_kv_desc),
         offsetof(tq_kv_desc, g));
  return 0;
}
''')
    exe = tmp_path / "probe"
    subprocess.run(["gcc", "-I", os.path.dirname(HEADER), str(probe), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    want = [ctypes.sizeof(tq.tq_quantizer), tq.tq_quantizer.R.offset, tq.tq_quantizer.SR.offset,
            tq.tq_quantizer.centroids.offset, tq.tq_quantizer.thresholds.offset, ctypes.sizeof(tq.tq_group),
            tq.tq_group.packed.offset,
            tq.tq_group.seq_stride.offset, ctypes.sizeof(tq.tq_kv_desc), tq.tq_kv_desc.g.offset]
    assert got == want


@pytest.mark.parametrize("d,B", [(3, 2), (32, 2), (96, 1), (128, 2), (128, 3), (128, 4), (1536, 4), (2048, 3)])
def test_host_codebook_equals_oracle(d, B):
    c, t, D = tq.tq_build_codebook(d, B)
    co, to = otq.symmetric_codebook(d, B)
    np.testing.assert_allclose(c, co, atol=5e-12, rtol=0)
    np.testing.assert_allclose(t, to, atol=5e-12, rtol=0)
    _, _, Do, _ = ocb.lloyd_max(d, B)
    assert abs(D - Do) < 1e-8
    assert np.array_equal(np.array(c), -np.array(c)[::-1])
    assert t[len(t) // 2] == 0.0


def test_codebook_errors():
    assert tq.lib().tq_build_codebook(2, 2, None, None, None, 0) == tq.TQ_ERR_INVALID_ARG
    c = (ctypes.c_double * 16)()
    t = (ctypes.c_double * 15)()
    assert tq.lib().tq_build_codebook(2, 2, c, t, None, 0) == tq.TQ_ERR_UNSUPPORTED
    assert tq.lib().tq_build_codebook(128, 5, c, t, None, 0) == tq.TQ_ERR_UNSUPPORTED
    assert tq.lib().tq_build_codebook(128, 0, c, t, None, 0) == tq.TQ_ERR_UNSUPPORTED
    assert tq.lib().tq_build_codebook(128, 4, c, t, None, 1) == tq.TQ_ERR_NO_CONVERGE
    assert "converge" in tq.tq_status_string(tq.TQ_ERR_NO_CONVERGE)


def test_quantizer_init_rounds_codebook_to_fp32():
    q = tq.tq_quantizer_init(128, 3, tq.TQ_PROD, 0x1000, 0x2000)
    co, to = otq.symmetric_codebook(128, 3)
    assert np.array_equal(np.array(q.centroids[:8], np.float32), co.astype(np.float32))
    assert np.array_equal(np.array(q.thresholds[:7], np.float32), to.astype(np.float32))
    assert q.S == 0x2000
    qm = tq.tq_quantizer_init(128, 3, tq.TQ_MSE, 0x1000, 0x2000)
    assert qm.S is None
    with pytest.raises(tq.TQError):
        tq.tq_quantizer_init(100, 3, tq.TQ_MSE, 0x1000)


def test_packed_bytes():
    assert tq.tq_packed_bytes(128, 3, tq.TQ_PROD, tq.TQ_LAYOUT_KEYS, 1) == 16 * 64
    assert tq.tq_packed_bytes(128, 3, tq.TQ_PROD, tq.TQ_LAYOUT_KEYS, 32768) == 32768 * 64
    assert tq.tq_packed_bytes(128, 3, tq.TQ_MSE, tq.TQ_LAYOUT_VALUES, 33) == 64 * 48
    assert tq.tq_packed_bytes(32, 2, tq.TQ_PROD, tq.TQ_LAYOUT_KEYS, 0) == 0
    assert tq.tq_packed_bytes(100, 2, tq.TQ_PROD, tq.TQ_LAYOUT_KEYS, 5) == 0
    # the oracle's word count agrees
    for d, B, prod, n, lay in [(96, 2, True, 45, "keys"), (96, 2, False, 45, "values")]:
        want = otq.packed_words(d, B, prod, n, lay) * 4
        assert tq.tq_packed_bytes(d, B, int(prod), 0 if lay == "keys" else 1, n) == want


FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced (validation fails first)


def _q(d=128, B=3, variant=tq.TQ_PROD):
    return tq.tq_quantizer_init(d, B, variant, FAKE, FAKE)


def test_quantize_validation_paths():
    L = tq.lib()

    def call(q, layout=tq.TQ_LAYOUT_KEYS, dt=tq.TQ_F32, x=FAKE, n=10, stride=128, p=FAKE, nrm=FAKE, rn=FAKE):
        return L.tq_quantize_kv(ctypes.byref(q), layout, dt, x, n, stride, p, nrm, rn, None)

    q = _q()
    assert call(q, x=None) == tq.TQ_ERR_INVALID_ARG
    assert call(q, rn=None) == tq.TQ_ERR_INVALID_ARG
    assert call(q, n=-1) == tq.TQ_ERR_INVALID_ARG
    assert call(q, stride=64) == tq.TQ_ERR_INVALID_ARG
    assert call(q, x=FAKE + 4) == tq.TQ_ERR_MISALIGNED
    assert call(q, dt=7) == tq.TQ_ERR_INVALID_ARG
    assert call(q, layout=5) == tq.TQ_ERR_INVALID_ARG
    assert call(q, n=0) == tq.TQ_OK  # nothing to do, nothing launched
    bad = _q()
    bad.d = 100
    assert call(bad) == tq.TQ_ERR_UNSUPPORTED
    bad = _q()
    bad.mse_bits = 5
    assert call(bad) == tq.TQ_ERR_UNSUPPORTED
    bad = _q()
    bad.S = None
    assert call(bad) == tq.TQ_ERR_INVALID_ARG
    bad = _q()
    bad.centroids[1] = bad.centroids[0]
    assert call(bad) == tq.TQ_ERR_INVALID_ARG
    big = _q(d=512, B=2, variant=tq.TQ_MSE)
    assert call(big, layout=tq.TQ_LAYOUT_VALUES, stride=512) == tq.TQ_ERR_UNSUPPORTED


def test_append_validation_paths():
    L = tq.lib()

    def call(q, layout=tq.TQ_LAYOUT_KEYS, dt=tq.TQ_F32, x=FAKE, n=10, stride=128, rows=FAKE, cache_rows=64,
             p=FAKE, nrm=FAKE, rn=FAKE):
        return L.tq_append_kv(ctypes.byref(q), layout, dt, x, n, stride, rows, cache_rows, p, nrm, rn, None)

    q = _q()
    assert call(q, rows=None) == tq.TQ_ERR_INVALID_ARG
    assert call(q, x=None) == tq.TQ_ERR_INVALID_ARG
    assert call(q, rn=None) == tq.TQ_ERR_INVALID_ARG
    assert call(q, cache_rows=0) == tq.TQ_ERR_INVALID_ARG
    assert call(q, n=-1) == tq.TQ_ERR_INVALID_ARG
    assert call(q, stride=64) == tq.TQ_ERR_INVALID_ARG
    assert call(q, rows=FAKE + 4) == tq.TQ_ERR_MISALIGNED
    assert call(q, p=FAKE + 4) == tq.TQ_ERR_MISALIGNED
    assert call(q, layout=5) == tq.TQ_ERR_INVALID_ARG
    assert call(q, dt=7) == tq.TQ_ERR_INVALID_ARG
    assert call(q, n=0) == tq.TQ_OK  # nothing to do, nothing launched
    big = _q(d=512, B=2, variant=tq.TQ_MSE)
    assert call(big, layout=tq.TQ_LAYOUT_VALUES, stride=512, rn=None) == tq.TQ_ERR_UNSUPPORTED


def test_kv_bit_allocation_matches_oracle():
    for r in np.concatenate([np.geomspace(0.01, 1e4, 400), [9.999, 10.0, 60.0, 60.001, 100.0, 100.001]]):
        for v in (0.5, 3.0, 1000.0):
            assert tq.tq_kv_bit_allocation(r * v, v) == otq.kv_bit_allocation(r * v, v), (r, v)
    L = tq.lib()
    kb, vb = ctypes.c_int(-7), ctypes.c_int(-7)
    for k, v in [(0.0, 1.0), (1.0, 0.0), (-2.0, 1.0), (float("inf"), 1.0), (1.0, float("nan"))]:
        assert L.tq_kv_bit_allocation(k, v, ctypes.byref(kb), ctypes.byref(vb)) == tq.TQ_ERR_INVALID_ARG
    assert (kb.value, vb.value) == (-7, -7)  # nothing written on error
    assert L.tq_kv_bit_allocation(1.0, 1.0, None, ctypes.byref(vb)) == tq.TQ_ERR_INVALID_ARG


def test_append_pair_validation_paths():
    L = tq.lib()

    def call(qk, qv, xk=FAKE, xv=FAKE, n=10, rows=FAKE, cache_rows=64, kr=FAKE, vr=None, sk=128, sv=128):
        return L.tq_append_kv_pair(ctypes.byref(qk), ctypes.byref(qv), tq.TQ_F32, xk, xv, n, sk, sv, rows,
                                   cache_rows, FAKE, FAKE, kr, FAKE, FAKE, vr, None)

    qk, qv = _q(), _q(128, 3, tq.TQ_MSE)
    assert call(qk, qv, rows=None) == tq.TQ_ERR_INVALID_ARG
    assert call(qk, qv, xv=None) == tq.TQ_ERR_INVALID_ARG
    assert call(qk, qv, kr=None) == tq.TQ_ERR_INVALID_ARG   # PROD keys need their residual norms
    assert call(qk, qv, cache_rows=0) == tq.TQ_ERR_INVALID_ARG
    assert call(qk, qv, sv=64) == tq.TQ_ERR_INVALID_ARG
    assert call(qk, qv, xk=FAKE + 4) == tq.TQ_ERR_MISALIGNED
    assert call(qk, qv, n=0) == tq.TQ_OK
    assert call(qk, _q(512, 2, tq.TQ_MSE), sv=512) == tq.TQ_ERR_UNSUPPORTED  # values layout needs d <= 256


def _desc(groups):
    return tq.make_desc(groups)


def _kv(T=1024, kd=128, vd=128):
    k = _desc([tq.make_group(_q(kd, 3, tq.TQ_PROD), 0, FAKE, FAKE, FAKE, T)])
    v = _desc([tq.make_group(_q(vd, 3, tq.TQ_MSE), 0, FAKE, FAKE, None, T)])
    return k, v


def test_decode_validation_paths():
    L = tq.lib()
    k, v = _kv()
    ws = tq.tq_decode_workspace_bytes(k, v, 1, 32, 8, 1024)
    assert ws > 0

    def call(k=k, v=v, q=FAKE, B=1, Hq=32, Hkv=8, T=1024, out=FAKE, wsp=FAKE, wsb=ws, scale=0.088):
        return L.tq_decode_attn(ctypes.byref(k), ctypes.byref(v), q, tq.TQ_BF16, B, Hq, Hkv, T, None, scale,
                                out, None, wsp, wsb, None)

    assert call(Hq=30) == tq.TQ_ERR_INVALID_ARG
    assert call(T=2048) == tq.TQ_ERR_INVALID_ARG         # longer than the cache stride
    assert call(wsb=ws - 1) == tq.TQ_ERR_WORKSPACE
    assert call(wsp=None) == tq.TQ_ERR_WORKSPACE
    assert call(out=None) == tq.TQ_ERR_INVALID_ARG
    assert call(q=FAKE + 2) == tq.TQ_ERR_MISALIGNED
    assert call(scale=float("nan")) == tq.TQ_ERR_INVALID_ARG
    kp, vp = _kv(kd=512, vd=512)
    assert call(k=kp, v=vp) == tq.TQ_ERR_UNSUPPORTED
    # values must be MSE-only
    vprod = _desc([tq.make_group(_q(128, 3, tq.TQ_PROD), 0, FAKE, FAKE, FAKE, 1024)])
    assert call(v=vprod) == tq.TQ_ERR_UNSUPPORTED
    # groups must tile the channels in order
    g1 = tq.make_group(_q(32, 2, tq.TQ_PROD), 0, FAKE, FAKE, FAKE, 1024)
    g2 = tq.make_group(_q(96, 1, tq.TQ_PROD), 40, FAKE, FAKE, FAKE, 1024)
    assert call(k=_desc([g1, g2])) == tq.TQ_ERR_INVALID_ARG
    # the cache stride must be a multiple of the value tile
    k2, v2 = _kv(T=1000)
    assert call(k=k2, v=v2, T=1000) == tq.TQ_ERR_INVALID_ARG
    assert tq.tq_decode_workspace_bytes(k, v, 1, 30, 8, 1024) == 0


def test_decode_step_validation_paths():
    L = tq.lib()
    k, v = _kv()
    ws = tq.tq_decode_workspace_bytes(k, v, 1, 32, 8, 1024)

    def call(kn=FAKE, vn=FAKE, kvdt=tq.TQ_BF16, sl=FAKE, Hq=32, wsp=FAKE, wsb=ws, out=FAKE):
        return L.tq_decode_step(ctypes.byref(k), ctypes.byref(v), kn, vn, kvdt, FAKE, tq.TQ_BF16, 1, Hq, 8, 1024, sl,
                                0.088, out, None, wsp, wsb, None)

    assert call(Hq=30) == tq.TQ_ERR_INVALID_ARG
    assert call(kn=None) == tq.TQ_ERR_INVALID_ARG
    assert call(vn=None) == tq.TQ_ERR_INVALID_ARG
    assert call(sl=None) == tq.TQ_ERR_INVALID_ARG     # the lengths say where the new rows go
    assert call(kvdt=7) == tq.TQ_ERR_INVALID_ARG
    assert call(kn=FAKE + 8) == tq.TQ_ERR_MISALIGNED
    assert call(out=None) == tq.TQ_ERR_INVALID_ARG
    assert call(wsb=ws - 1) == tq.TQ_ERR_WORKSPACE
    assert call(wsp=None) == tq.TQ_ERR_WORKSPACE


def test_noalloc_decode_validation_paths():
    # the allocation-free entry point validates like tq_decode_attn and refuses
    # requests beyond its fixed scratch array, all before any device call
    L = tq.lib()
    k, v = _kv()

    def call(k=k, v=v, q=FAKE, B=1, Hq=32, Hkv=8, T=1024, out=FAKE, scale=0.088):
        return L.tq_decode_attn_noalloc(ctypes.byref(k), ctypes.byref(v), q, tq.TQ_BF16, B, Hq, Hkv, T, None,
                                        scale, out, None, None)

    assert call(Hq=30) == tq.TQ_ERR_INVALID_ARG
    assert call(T=2048) == tq.TQ_ERR_INVALID_ARG
    assert call(out=None) == tq.TQ_ERR_INVALID_ARG
    assert call(q=FAKE + 2) == tq.TQ_ERR_MISALIGNED
    assert call(scale=float("nan")) == tq.TQ_ERR_INVALID_ARG
    kp, vp = _kv(kd=512, vd=512)
    assert call(k=kp, v=vp) == tq.TQ_ERR_UNSUPPORTED
    need = tq.tq_decode_workspace_bytes(k, v, 1024, 64, 8, 1024)
    assert need > tq.TQ_DECODE_SCRATCH_BYTES
    assert call(B=1024, Hq=64) == tq.TQ_ERR_SCRATCH
    assert "TQ_DECODE_SCRATCH_BYTES" in L.tq_status_string(tq.TQ_ERR_SCRATCH).decode()


def test_paged_decode_validation_paths():
    L = tq.lib()
    bt = 512
    k, v = _kv(T=bt)  # every group's rows per (block, KV head) = the block size
    ws = tq.tq_decode_paged_workspace_bytes(k, v, 2, 32, 8, 4000, bt)
    assert ws > 0
    assert tq.tq_decode_paged_workspace_bytes(k, v, 2, 32, 8, 4000, 300) == 0   # not a multiple of 256
    assert tq.tq_decode_paged_workspace_bytes(k, v, 2, 32, 8, 4000, 1024) == 0  # seq_stride != block size

    def call(k=k, v=v, table=FAKE, max_blocks=8, bt=bt, nblk=64, T=4000, out=FAKE, wsp=FAKE, wsb=ws):
        return L.tq_decode_attn_paged(ctypes.byref(k), ctypes.byref(v), FAKE, tq.TQ_BF16, 2, 32, 8, T, None, table,
                                      max_blocks, bt, nblk, 0.088, out, None, wsp, wsb, None)

    assert call(table=None) == tq.TQ_ERR_INVALID_ARG
    assert call(max_blocks=7) == tq.TQ_ERR_INVALID_ARG      # 7 x 512 < 4000 tokens
    assert call(nblk=0) == tq.TQ_ERR_INVALID_ARG
    assert call(bt=384) == tq.TQ_ERR_UNSUPPORTED            # not a multiple of 256
    assert call(table=FAKE + 2) == tq.TQ_ERR_MISALIGNED
    assert call(wsb=ws - 1) == tq.TQ_ERR_WORKSPACE
    assert call(out=None) == tq.TQ_ERR_INVALID_ARG
    k2, v2 = _kv(T=1024)
    assert call(k=k2, v=v2) == tq.TQ_ERR_INVALID_ARG        # rows per block differ from the block size
    kp, vp = _kv(T=bt, kd=64, vd=64)
    assert call(k=kp, v=vp) == tq.TQ_ERR_UNSUPPORTED        # head size without the matrix-core decode


def test_search_validation_paths():
    L = tq.lib()
    db = tq.make_group(_q(1536, 3, tq.TQ_PROD), 0, FAKE, FAKE, FAKE, 0)
    ws = tq.tq_search_workspace_bytes(db, 1000, 4, 10)
    assert ws > 0

    def call(N=1000, Q=4, k=10, wsb=ws, qp=FAKE):
        return L.tq_search_topk(ctypes.byref(db), N, qp, Q, k, FAKE, FAKE, FAKE, wsb, None)

    assert call(k=0) == tq.TQ_ERR_INVALID_ARG
    assert call(k=65) == tq.TQ_ERR_INVALID_ARG
    assert call(N=5) == tq.TQ_ERR_INVALID_ARG
    assert call(N=1 << 29) == tq.TQ_ERR_INVALID_ARG
    assert tq.tq_search_workspace_bytes(db, 1 << 29, 4, 10) == 0
    assert call(wsb=ws - 8) == tq.TQ_ERR_WORKSPACE
    assert call(qp=None) == tq.TQ_ERR_INVALID_ARG
    assert tq.tq_search_workspace_bytes(db, 1000, 4, 0) == 0


def test_fold_validation_paths():
    L = tq.lib()
    assert tq.tq_fold_bytes(128) == (128 * 128 + 4) * 4
    assert tq.tq_fold_bytes(100) == 0
    qp = _q(128, 3, tq.TQ_PROD)
    qm = _q(128, 3, tq.TQ_MSE)
    assert L.tq_fold_qjl(ctypes.byref(qm), FAKE, None) == tq.TQ_ERR_INVALID_ARG   # no sketch to fold
    assert L.tq_fold_qjl(ctypes.byref(qp), None, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_fold_qjl(ctypes.byref(qp), FAKE + 4, None) == tq.TQ_ERR_MISALIGNED
    # a quantiser carrying SR must be PROD and SR aligned
    bad = _q(128, 3, tq.TQ_MSE)
    bad.SR = FAKE
    g = tq.make_group(bad, 0, FAKE, FAKE, None, 64)
    assert L.tq_quantize_kv(ctypes.byref(bad), tq.TQ_LAYOUT_VALUES, tq.TQ_F32, FAKE, 4, 128, FAKE, FAKE, None,
                            None) == tq.TQ_ERR_INVALID_ARG
    mis = _q(128, 3, tq.TQ_PROD)
    mis.SR = FAKE + 8
    assert L.tq_quantize_kv(ctypes.byref(mis), tq.TQ_LAYOUT_KEYS, tq.TQ_F32, FAKE, 4, 128, FAKE, FAKE, FAKE,
                            None) == tq.TQ_ERR_MISALIGNED
    del g
