"""The C ABI on the host: the library loads, exports what include/rmm.h declares,
computes k like the oracle, and rejects bad arguments before enqueuing anything.

No test here launches a kernel; the error paths return during host-side
validation, so they run without a GPU.
"""
import ctypes
import json
import math
import os
import re

import numpy as np
import pytest

import oracle
from input_adaptive_reduced_rmm_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rmm.h")
FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: validation rejects the call first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.lib_path):
        pytest.fail("librmm.so is not built (run __graft_entry__.build())")
    return B.load()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rmm_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_five_entry_points():
    syms = declared_symbols()
    for name in ("rmm_colnorm", "rmm_topk", "rmm_gemm", "rmm_qk", "rmm_pv"):
        assert name in syms


def test_every_declared_symbol_is_exported(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name
    # and the binding wraps each entry point under the same name
    for name in ("rmm_colnorm", "rmm_topk", "rmm_gemm", "rmm_qk", "rmm_pv", "rmm_k_from_rho", "rmm_k_pad"):
        assert callable(getattr(B, name))


def test_status_strings(lib):
    assert lib.rmm_status_string(0) == b"RMM_OK"
    assert lib.rmm_status_string(3) == b"RMM_ERR_WORKSPACE"
    assert lib.rmm_version() >= 100


def test_k_from_rho_matches_oracle_table(lib):
    rows = json.load(open(os.path.join(ROOT, "tests", "golden", "retained_counts.json")))
    for r in rows["rows"] + rows["decimal_traps"]:
        assert B.rmm_k_from_rho(r["rho"], r["d"]) == r["k"], r


def test_k_from_rho_matches_oracle_on_random_decimals(lib):
    rng = np.random.default_rng(21)
    for _ in range(3000):
        q = int(rng.integers(1, 5))
        p = int(rng.integers(1, 10 ** q + 1))
        rho = float(f"{p}e-{q}")
        d = int(rng.integers(1, 200000))
        assert B.rmm_k_from_rho(rho, d) == oracle.retained_count(rho, d), (rho, d)


def _adversarial_ratios(rng, n):
    """Doubles in (0, 1] whose shortest decimal strings are long: random bit
    patterns, sums of short decimals, the binary neighbours of short decimals,
    and every power of two down to the smallest subnormal."""
    out = [0.1 + 0.2, 0.7 + 0.1, 0.1 * 3, 1.0 - 1e-16, 5e-324, 2.2250738585072014e-308,
           math.nextafter(0.5, 1.0), math.nextafter(0.7, 1.0), math.nextafter(0.7, 0.0),
           math.nextafter(1.0, 0.0), math.nextafter(0.3, 1.0), math.nextafter(0.55, 0.0)]
    out += [math.ldexp(1.0, -e) for e in range(0, 1075)]
    bits = rng.integers(1, 0x3FF0000000000000, size=n // 3, dtype=np.int64)
    out += [float(x) for x in bits.view(np.float64)]
    u = rng.random(n // 3)
    out += [float(x) for x in u if x > 0.0]
    for _ in range(n // 3):
        q = int(rng.integers(1, 9))
        p = int(rng.integers(1, 10 ** q + 1))
        r = float(f"{p}e-{q}")
        step = int(rng.integers(-3, 4))
        for _ in range(abs(step)):
            r = math.nextafter(r, 1.0 if step > 0 else 0.0)
        if 0.0 < r <= 1.0:
            out.append(r)
    return out


def test_k_from_rho_matches_oracle_on_long_decimals(lib):
    """Integer result: bit-exact against the oracle's exact rational ceiling for
    ratios whose shortest decimal strings run to 15-17 digits, with d up to 2^31 - 1."""
    rng = np.random.default_rng(22)
    ratios = _adversarial_ratios(rng, 100000)
    ds = rng.integers(1, 2 ** 31 - 1, size=len(ratios))
    small = rng.integers(1, 1000, size=len(ratios))
    bad = []
    for rho, d, ds_ in zip(ratios, ds, small):
        for dd in (int(d), int(ds_), 10, 100):
            if B.rmm_k_from_rho(rho, dd) != oracle.retained_count(rho, dd):
                bad.append((repr(rho), dd))
    assert not bad, bad[:10]


def test_k_from_rho_long_decimal_examples(lib):
    # worked by hand from the shortest decimal strings
    assert B.rmm_k_from_rho(0.1 + 0.2, 10) == 4          # 0.30000000000000004 * 10 = 3.0000000000000004
    assert B.rmm_k_from_rho(0.1 + 0.2, 100) == 31
    assert B.rmm_k_from_rho(math.nextafter(0.5, 1.0), 2) == 2    # 0.5000000000000001 * 2
    assert B.rmm_k_from_rho(math.nextafter(0.7, 1.0), 10) == 8   # 0.7000000000000001 * 10
    assert B.rmm_k_from_rho(math.nextafter(0.7, 0.0), 10) == 7   # 0.6999999999999998 * 10
    assert B.rmm_k_from_rho(5e-324, 2 ** 31 - 1) == 1
    assert B.rmm_k_from_rho(1.0, 2 ** 31 - 1) == 2 ** 31 - 1


@pytest.mark.parametrize("rho,d", [(0.0, 10), (-0.5, 10), (1.5, 10), (float("nan"), 10), (0.5, 0)])
def test_k_from_rho_rejects(lib, rho, d):
    with pytest.raises(B.RMMError) as e:
        B.rmm_k_from_rho(rho, d)
    assert e.value.status == 1


def test_k_pad(lib):
    assert [B.rmm_k_pad(k) for k in (0, 1, 63, 64, 65, 1434, 11469)] == [0, 64, 64, 64, 128, 1472, 11520]


def _st(x):
    return int(x)


def test_colnorm_rejects(lib):
    f = lib.rmm_colnorm
    assert f(0, None, 4, 4, 4, 1, 0, FAKE, None, 0, None) == 1          # NULL A
    assert f(0, FAKE, 4, 8, 4, 1, 0, FAKE, None, 0, None) == 1          # lda < d
    assert f(0, FAKE, 0, 8, 8, 1, 0, FAKE, None, 0, None) == 1          # m = 0
    assert f(7, FAKE, 4, 8, 8, 1, 0, FAKE, None, 0, None) == 1          # unknown dtype
    assert f(0, FAKE, 4, 8, 8, 70000, 8, FAKE, None, 0, None) == 1      # batch too large
    assert f(1, ctypes.c_void_p(0x10002), 4, 8, 8, 1, 0, FAKE, None, 0, None) == 1   # f32 misaligned
    need = lib.rmm_colnorm_workspace_bytes(0, 65536, 4096, 1)
    assert need > 0
    assert f(0, FAKE, 65536, 4096, 4096, 1, 0, FAKE, FAKE, need - 1, None) == 3
    assert b"workspace" in lib.rmm_last_error()


def test_topk_rejects(lib):
    f = lib.rmm_topk
    assert f(FAKE, 1, 10, 0, FAKE, None, 0, None) == 1
    assert f(FAKE, 1, 10, 11, FAKE, None, 0, None) == 1
    assert f(None, 1, 10, 5, FAKE, None, 0, None) == 1
    assert f(FAKE, 0, 10, 5, FAKE, None, 0, None) == 1
    assert lib.rmm_topk_workspace_bytes(4, 1000) == 0


def test_gemm_rejects(lib):
    f = lib.rmm_gemm
    args = dict(dt=0, A=FAKE, lda=64, B=FAKE, ldb=32, idx=FAKE, m=16, d=64, n=32, k=8, Y=FAKE, ldy=32)
    def call(ws=FAKE, wsb=1 << 30, **kw):
        a = {**args, **kw}
        return f(a["dt"], a["A"], a["lda"], a["B"], a["ldb"], a["idx"], a["m"], a["d"], a["n"], a["k"], a["Y"],
                 a["ldy"], ws, wsb, None)
    assert call(k=0) == 1
    assert call(k=65) == 1
    assert call(lda=63) == 1
    assert call(ldb=31) == 1
    assert call(ldy=31) == 1
    assert call(idx=None) == 1
    assert call(dt=5) == 1
    need = lib.rmm_gemm_workspace_bytes(0, 16, 32, 8)
    assert need == 16 * 64 * 2 + 256      # packed A + cleaned index list
    assert call(wsb=need - 1) == 3
    assert call(ws=None) == 3


def test_qk_pv_reject(lib):
    q = lib.rmm_qk
    # Hq % Hkv != 0
    assert q(FAKE, 64, 6, 128, 768, 128, FAKE, 64, 4, 8192, 64, 32, 0, FAKE, 4096, 64, FAKE, None, FAKE, 1 << 30, None) == 1
    # k > dh
    assert q(FAKE, 64, 4, 128, 512, 128, FAKE, 64, 2, 8192, 64, 129, 0, FAKE, 4096, 64, FAKE, None, FAKE, 1 << 30, None) == 1
    # q_tok_stride < dh
    assert q(FAKE, 64, 4, 128, 100, 128, FAKE, 64, 2, 8192, 64, 64, 1, FAKE, 4096, 64, FAKE, None, FAKE, 1 << 30, None) == 1
    need = lib.rmm_qk_workspace_bytes(64, 4, 128, 64)
    assert q(FAKE, 64, 4, 128, 512, 128, FAKE, 64, 2, 8192, 64, 64, 0, FAKE, 4096, 64, FAKE, None, FAKE, need - 1, None) == 3
    p = lib.rmm_pv
    assert p(FAKE, 4, 64, 64, 4096, 64, FAKE, 2, 128, 256, 128, 65, 0, FAKE, 512, 128, FAKE, None, FAKE, 1 << 30, None) == 1
    assert p(FAKE, 4, 64, 64, 4096, 63, FAKE, 2, 128, 256, 128, 32, 1, FAKE, 512, 128, FAKE, None, FAKE, 1 << 30, None) == 1
    need = lib.rmm_pv_workspace_bytes(4, 64, 64, 32)
    assert need > 0
    assert p(FAKE, 4, 64, 64, 4096, 64, FAKE, 2, 128, 256, 128, 32, 0, FAKE, 512, 128, FAKE, None, FAKE, need - 1, None) == 3


def test_gemm_w8_rejects(lib):
    f = lib.rmm_gemm_w8
    args = dict(A=FAKE, lda=64, Bq=FAKE, ldb=32, scale=FAKE, idx=FAKE, m=16, d=64, n=32, k=8, Y=FAKE, ldy=32)
    def call(ws=FAKE, wsb=1 << 30, **kw):
        a = {**args, **kw}
        return f(a["A"], a["lda"], a["Bq"], a["ldb"], a["scale"], a["idx"], a["m"], a["d"], a["n"], a["k"], a["Y"],
                 a["ldy"], ws, wsb, None)
    assert call(scale=None) == 1
    assert call(k=0) == 1
    assert call(k=65) == 1
    assert call(ldb=31) == 1
    assert call(lda=63) == 1
    assert call(ldb=40) == 2                     # decode rows must be 16-byte aligned
    assert call(Bq=ctypes.c_void_p(0x10008)) == 2
    need = lib.rmm_gemm_w8_workspace_bytes(16, 32, 8)
    assert need >= 16 * 64 * 2 + 256
    assert call(wsb=need - 1) == 3
    # more rows: the dequantized kept rows are part of the workspace
    assert lib.rmm_gemm_w8_workspace_bytes(2048, 1024, 300) >= 2048 * 320 * 2 + 320 * 1024 * 2
    assert lib.rmm_gemm_w8_workspace_bytes(0, 32, 8) == 0


def test_swiglu_scored_rejects(lib):
    f = lib.rmm_swiglu_scored
    def call(G=FAKE, ldg=64, U=FAKE, ldu=64, m=100, n=64, H=FAKE, ldh=64, s=FAKE, ws=FAKE, wsb=1 << 30):
        return f(G, ldg, U, ldu, m, n, H, ldh, s, ws, wsb, None)
    assert call(s=None) == 1
    assert call(m=0) == 1
    assert call(ldg=63) == 1
    assert call(n=60, ldg=64, ldu=64, ldh=64) == 2          # n % 8 != 0
    assert call(ldu=68) == 2                                 # unaligned rows
    assert call(G=ctypes.c_void_p(0x10002)) == 2
    need = lib.rmm_swiglu_scored_workspace_bytes(100000, 4096)
    assert need > 0
    assert call(m=100000, n=4096, ldg=4096, ldu=4096, ldh=4096, wsb=need - 1) == 3
    assert lib.rmm_swiglu_scored_workspace_bytes(1, 0) == 0


def test_rmsnorm_scored_rejects(lib):
    f = lib.rmm_rmsnorm_scored
    def call(X=FAKE, ldx=1024, w=FAKE, eps=1e-5, m=100, d=1024, Y=FAKE, ldy=1024, s=FAKE, ws=FAKE, wsb=1 << 30):
        return f(X, ldx, w, eps, m, d, Y, ldy, s, ws, wsb, None)
    assert call(w=None) == 1
    assert call(m=0) == 1
    assert call(eps=-1e-6) == 1
    assert call(eps=float("nan")) == 1
    assert call(eps=float("inf")) == 1
    assert call(ldy=1000) == 1
    assert call(d=1000, ldx=1000, ldy=1000) == 2             # d % 512 != 0
    assert call(d=512 * 17, ldx=512 * 17, ldy=512 * 17) == 2  # wider than 8192
    assert call(ldx=1028) == 2                                 # unaligned rows
    assert call(w=ctypes.c_void_p(0x10008)) == 2
    need = lib.rmm_rmsnorm_scored_workspace_bytes(100000, 4096)
    assert need > 0
    assert call(m=100000, d=4096, ldx=4096, ldy=4096, wsb=need - 1) == 3
    assert lib.rmm_rmsnorm_scored_workspace_bytes(0, 4096) == 0


def test_attention_decode_batch_rejects(lib):
    f = lib.rmm_attention_decode_batch
    def call(Q=FAKE, Kt=FAKE, V=FAKE, lens=FAKE, ktok=FAKE, nseq=4, Hq=8, Hkv=2, dh=128, Lmax=1000, kf=64,
             ktm=500, vts=256, ws=FAKE, wsb=1 << 30, O=FAKE):
        return f(Q, 8 * 128, 128, Kt, 2 * 128 * 1000, 128 * 1000, 1000, V, 1000 * 256, vts, 128,
                 lens, ktok, nseq, Hq, Hkv, dh, Lmax, kf, ktm, O, 8 * 128, 128, FAKE, FAKE, None, ws, wsb, None)
    assert call(lens=None) == 1
    assert call(O=None) == 1
    assert call(nseq=0) == 1
    assert call(Hkv=3) == 1                   # Hq % Hkv != 0
    assert call(nseq=9000) == 1               # nseq * Hq > 65535
    assert call(kf=0) == 1
    assert call(ktm=1001) == 1                # kt_max > Lmax
    assert call(dh=64) == 2
    assert call(vts=252) == 2                 # value rows not 16-byte aligned
    assert call(V=ctypes.c_void_p(0x10008)) == 2
    need = lib.rmm_attention_decode_batch_workspace_bytes(4, 8, 128, 1000, 500)
    assert need > 0
    assert call(wsb=need - 1) == 3
    assert lib.rmm_attention_decode_batch_workspace_bytes(4, 8, 64, 1000, 500) == 0


def test_attention_rejects(lib):
    f = lib.rmm_attention
    def call(Lq=64, Hq=4, dh=128, qts=512, qhs=128, Lk=64, Hkv=2, kths=8192, ldkt=64, vts=256, vhs=128,
             kf=32, kt=32, causal=1, ots=512, ohs=128, ws=FAKE, wsb=1 << 30, O=FAKE):
        return f(FAKE, Lq, Hq, dh, qts, qhs, FAKE, Lk, Hkv, kths, ldkt, FAKE, vts, vhs, kf, kt, causal, O, ots, ohs,
                 FAKE, FAKE, None, None, ws, wsb, None)
    assert call(O=None) == 1
    assert call(Hq=6, Hkv=4) == 1                 # Hq % Hkv != 0
    assert call(kf=129) == 1                      # more features than dh
    assert call(kt=65) == 1                       # more tokens than Lk
    assert call(Lq=65) == 1                       # causal queries beyond the keys
    assert call(ldkt=63) == 1
    assert call(dh=64, qts=256, qhs=64, vts=128, vhs=64, ots=256, ohs=64) == 2   # head size not served
    for Lq in (1, 16, 64):
        need = lib.rmm_attention_workspace_bytes(Lq, 64, 4, 128, 32, 32)
        assert need > 0
        assert call(Lq=Lq, wsb=need - 1) == 3
    assert lib.rmm_attention_workspace_bytes(0, 64, 4, 128, 32, 32) == 0
