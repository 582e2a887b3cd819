"""The C-ABI library without a GPU: it loads, exports exactly the entry
points include/*.h declare, its host-side codebook equals the oracle's,
and every invalid argument is rejected on the host before any launch (the
pointers below are never dereferenced)."""

import os
import re
import subprocess

import numpy as np
import pytest

import dequant_gemm_nf4_amd as bnbx
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


def header_functions():
    text = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"BNBX_API\s+[\w\s\*]*?\b(bnbx_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return bnbx.lib()


def test_exports_every_declared_symbol(lib):
    declared = header_functions()
    assert len(declared) == 18
    assert sorted(bnbx.EXPORTED_SYMBOLS) == declared
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", bnbx.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = sorted(re.findall(r"\sT\s(\w+)$", out, flags=re.M))
    assert exported == declared


def test_codebook_equals_oracle_bit_for_bit():
    ours = np.array(bnbx.bnbx_nf4_codebook(), dtype=np.float32)
    assert np.array_equal(ours.view(np.uint32), oracle.codebook().view(np.uint32))


def test_fp4_codebook_equals_oracle_bit_for_bit():
    ours = np.array(bnbx.bnbx_fp4_codebook(), dtype=np.float32)
    assert np.array_equal(ours.view(np.uint32), oracle.fp4_codebook().view(np.uint32))


def test_dynamic_map_equals_oracle_bit_for_bit():
    """The library's compile-time dynamic 8-bit map against the oracle's
    (two independent constructions of the same definition)."""
    ours = np.array(bnbx.bnbx_dynamic_map(), dtype=np.float32)
    assert ours.shape == (256,)
    assert np.array_equal(ours.view(np.uint32), oracle.dynamic_map().view(np.uint32))


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5):
        assert bnbx.bnbx_status_str(code).startswith("BNBX")
    assert "unknown" in bnbx.bnbx_status_str(7)


def test_workspace_queries():
    n = 4096 * 4096
    nb = n // 64
    assert bnbx.bnbx_quantize_nf4_workspace_bytes(n, 64, 0) == 0
    ws = bnbx.bnbx_quantize_nf4_workspace_bytes(n, 64, 1)
    assert ws >= 256 * 8 + 4 * nb and ws % 256 == 0
    assert bnbx.bnbx_quantize_nf4_workspace_bytes(n + 1, 64, 1) == 0
    assert bnbx.bnbx_quantize_nf4_workspace_bytes(n, 32, 1) == 0
    assert bnbx.bnbx_gemm_nf4_workspace_bytes(2048, 8192, 8192) == 0
    # split K for shapes whose 256 x 256 tiles fill at most half of the CUs
    # (256 on MI355X, also the count assumed without a device), and for the
    # tail beyond one full round of tiles: fp32 partial tiles of 256 x 256
    tile = 256 * 256 * 4
    assert bnbx.bnbx_gemm_nf4_workspace_bytes(2048, 4096, 4096) == 2 * 128 * tile
    assert bnbx.bnbx_gemm_nf4_workspace_bytes(300, 500, 4096) == 4 * 4 * tile
    assert bnbx.bnbx_gemm_nf4_workspace_bytes(2048, 11008, 4096) == 2 * 88 * tile   # 344 tiles
    assert bnbx.bnbx_gemm_nf4_workspace_bytes(2304, 8192, 4096) == 4 * 32 * tile    # 288 tiles
    assert bnbx.bnbx_gemm_nf4_workspace_bytes(4096, 8192, 4096) == 0   # 512 tiles: two rounds
    assert bnbx.bnbx_gemm_nf4_workspace_bytes(2048, 4096, 1024) == 0   # K too short
    assert bnbx.bnbx_gemm_nf4_workspace_bytes(0, 4096, 4096) == 0
    assert bnbx.bnbx_gemm_nf4_workspace_bytes(2048, 4096, 100) == 0
    # grouped: one tensor needs what the single call needs; more add their
    # slots and fp32 absmax arrays
    g = bnbx.bnbx_quantize_nf4_grouped_workspace_bytes
    assert g([n], 64, 1) == ws
    n2 = 11008 * 4096
    both = g([n, n2], 64, 1)
    assert both >= ws + bnbx.bnbx_quantize_nf4_workspace_bytes(n2, 64, 1) and both % 256 == 0
    assert g([n, n2], 64, 0) == 0
    assert g([], 64, 1) == 0
    assert g([n] * 9, 64, 1) == 0
    assert g([n, n + 1], 64, 1) == 0
    assert g([n], 32, 1) == 0


A = 1 << 20          # fake, 256-byte aligned "device" addresses: never touched
B = 2 << 20
C = 3 << 20
D = 4 << 20


def state(n=4096, dq=1, blocksize=64, absmax=C, absmax2=D, mean=D + 4096, qt=0, dt=0):
    return bnbx.Nf4State(n=n, blocksize=blocksize, double_quant=dq, quant_type=qt,
                         compute_dtype=dt, absmax=absmax,
                         absmax2=absmax2 if dq else None, absmax_mean=mean if dq else None)


def status_of(fn, *args):
    try:
        fn(*args)
    except bnbx.BnbxError as e:
        return e.status
    raise AssertionError("call was accepted (it would have launched)")


@pytest.mark.parametrize("case,expect", [
    ("null_w", bnbx.BNBX_E_INVAL),
    ("odd_n", bnbx.BNBX_E_INVAL),
    ("tiny_n", bnbx.BNBX_E_INVAL),
    ("blocksize", bnbx.BNBX_E_UNSUPPORTED),
    ("dq_flag", bnbx.BNBX_E_INVAL),
    ("quant_type", bnbx.BNBX_E_INVAL),
    ("compute_dtype", bnbx.BNBX_E_INVAL),
    ("null_absmax", bnbx.BNBX_E_INVAL),
    ("null_absmax2", bnbx.BNBX_E_INVAL),
    ("misaligned_w", bnbx.BNBX_E_ALIGN),
    ("misaligned_packed", bnbx.BNBX_E_ALIGN),
    ("no_workspace", bnbx.BNBX_E_WORKSPACE),
    ("small_workspace", bnbx.BNBX_E_WORKSPACE),
    ("misaligned_workspace", bnbx.BNBX_E_ALIGN),
])
def test_quantize_rejects(case, expect):
    n = 4096
    ws_need = bnbx.bnbx_quantize_nf4_workspace_bytes(n, 64, 1)
    w, p, st, ws, wsb = A, B, state(n), C + (1 << 16), ws_need
    if case == "null_w":
        w = None
    elif case == "odd_n":
        st = state(n + 1)
    elif case == "tiny_n":
        st = state(0)
    elif case == "blocksize":
        st = state(n, blocksize=128)
    elif case == "dq_flag":
        st = state(n, dq=3)
    elif case == "quant_type":
        st = state(n, qt=2)
    elif case == "compute_dtype":
        st = state(n, dt=-1)
    elif case == "null_absmax":
        st = state(n, absmax=None)
    elif case == "null_absmax2":
        st = state(n)
        st.absmax2 = None
    elif case == "misaligned_w":
        w = A + 2
    elif case == "misaligned_packed":
        p = B + 8
    elif case == "no_workspace":
        ws = None
    elif case == "small_workspace":
        wsb = ws_need - 1
    elif case == "misaligned_workspace":
        ws = C + 128
    assert status_of(bnbx.bnbx_quantize_nf4, w, p, st, ws, wsb, 0) == expect


def test_quantize_grouped_rejects():
    """Checked on the host before any launch: item count, states that differ,
    each item's own checks and the workspace."""
    f = bnbx.bnbx_quantize_nf4_grouped
    n = 4096
    need = bnbx.bnbx_quantize_nf4_grouped_workspace_bytes([n, n], 64, 1)
    ws = C + (1 << 16)

    def item(st=None, w=A, p=B):
        return (w, p, st if st is not None else state(n))

    ok = [item(), item()]
    assert status_of(f, [], ws, need, None) == bnbx.BNBX_E_INVAL                  # count 0
    assert status_of(f, [item()] * 9, ws, need, None) == bnbx.BNBX_E_INVAL        # count 9
    assert status_of(f, [item(), item(state(n, qt=1))], ws, need, None) == bnbx.BNBX_E_INVAL
    assert status_of(f, [item(), item(state(n, dq=2))], ws, need, None) == bnbx.BNBX_E_INVAL
    assert status_of(f, [item(), item(state(n, dq=0))], ws, need, None) == bnbx.BNBX_E_INVAL
    assert status_of(f, [item(), item(w=None)], ws, need, None) == bnbx.BNBX_E_INVAL
    assert status_of(f, [item(), item(state(n + 1))], ws, need, None) == bnbx.BNBX_E_INVAL
    assert status_of(f, [item(), item(state(n, blocksize=32))], ws, need, None) == \
        bnbx.BNBX_E_UNSUPPORTED
    assert status_of(f, [item(), item(w=A + 2)], ws, need, None) == bnbx.BNBX_E_ALIGN
    assert status_of(f, [item(), item(p=B + 8)], ws, need, None) == bnbx.BNBX_E_ALIGN
    assert status_of(f, ok, None, need, None) == bnbx.BNBX_E_WORKSPACE
    assert status_of(f, ok, ws, need - 1, None) == bnbx.BNBX_E_WORKSPACE
    assert status_of(f, ok, ws + 128, need, None) == bnbx.BNBX_E_ALIGN


def test_dequantize_rejects():
    assert status_of(bnbx.bnbx_dequantize_nf4, None, state(), B, 0) == bnbx.BNBX_E_INVAL
    assert status_of(bnbx.bnbx_dequantize_nf4, A, state(), None, 0) == bnbx.BNBX_E_INVAL
    assert status_of(bnbx.bnbx_dequantize_nf4, A + 1, state(), B, 0) == bnbx.BNBX_E_ALIGN
    assert status_of(bnbx.bnbx_dequantize_nf4, A, state(), B + 2, 0) == bnbx.BNBX_E_ALIGN
    assert status_of(bnbx.bnbx_dequantize_nf4, A, state(7), B, 0) == bnbx.BNBX_E_INVAL
    assert status_of(bnbx.bnbx_dequantize_nf4, A, state(blocksize=32), B, 0) == \
        bnbx.BNBX_E_UNSUPPORTED
    assert status_of(bnbx.bnbx_dequantize_nf4, A, state(qt=5), B, 0) == bnbx.BNBX_E_INVAL
    assert status_of(bnbx.bnbx_dequantize_nf4, A, state(dt=2), B, 0) == bnbx.BNBX_E_INVAL


def test_gemv_grouped_rejects():
    """Checked on the host before any launch: item count, NULL items, states
    that differ, and each item's own checks."""
    f = bnbx.bnbx_gemv_nf4_grouped
    K, N = 256, 64
    n = N * K

    def item(st=None, y=D, N_=N, ldy=N, packed=B):
        return (packed, st if st is not None else state(n), N_, y, ldy)

    ok = [item(), item()]
    # a valid call would launch: only invalid ones are made here
    assert status_of(f, A, K, [], 1, K, None) == bnbx.BNBX_E_INVAL                 # count 0
    assert status_of(f, A, K, [item()] * 5, 1, K, None) == bnbx.BNBX_E_INVAL       # count 5
    assert status_of(f, A, K, ok, 17, K, None) == bnbx.BNBX_E_INVAL                # M > 16
    assert status_of(f, A, K, ok, 0, K, None) == bnbx.BNBX_E_INVAL                 # M < 1
    assert status_of(f, A, K, [item(), item(state(n, qt=1))], 1, K, None) == bnbx.BNBX_E_INVAL
    assert status_of(f, A, K, [item(), item(state(n, dt=1))], 1, K, None) == bnbx.BNBX_E_INVAL
    assert status_of(f, A, K, [item(), item(state(n, dq=2))], 1, K, None) == bnbx.BNBX_E_INVAL
    assert status_of(f, A, K, [item(), item(N_=N + 1)], 1, K, None) == bnbx.BNBX_E_INVAL  # n != N*K
    assert status_of(f, A, K, [item(), item(ldy=N - 1)], 1, K, None) == bnbx.BNBX_E_INVAL
    assert status_of(f, A, K, [item(), item(packed=B + 8)], 1, K, None) == bnbx.BNBX_E_ALIGN
    assert status_of(f, A, K, [item(), item(y=None)], 1, K, None) == bnbx.BNBX_E_INVAL


def test_lora_down_rejects():
    f = bnbx.bnbx_lora_down
    K, r = 256, 16
    ok = dict(x=A, ldx=K, a=B, lda=K, M=4, K=K, r=r, s=1.0, dt=0, xa=C, ldxa=r)

    def call(**kw):
        a = {**ok, **kw}
        return status_of(f, a["x"], a["ldx"], a["a"], a["lda"], a["M"], a["K"], a["r"], a["s"],
                         a["dt"], a["xa"], a["ldxa"], None)

    assert call(x=None) == bnbx.BNBX_E_INVAL
    assert call(a=None) == bnbx.BNBX_E_INVAL
    assert call(xa=None) == bnbx.BNBX_E_INVAL
    assert call(dt=2) == bnbx.BNBX_E_INVAL
    assert call(M=0) == bnbx.BNBX_E_INVAL
    assert call(K=48, ldx=48, lda=48) == bnbx.BNBX_E_INVAL        # K % 32
    assert call(r=8) == bnbx.BNBX_E_INVAL
    assert call(r=24) == bnbx.BNBX_E_INVAL
    assert call(r=272, ldxa=272) == bnbx.BNBX_E_INVAL
    assert call(ldx=K - 8) == bnbx.BNBX_E_INVAL
    assert call(lda=K - 8) == bnbx.BNBX_E_INVAL
    assert call(ldxa=r - 1) == bnbx.BNBX_E_INVAL
    assert call(ldx=K + 4) == bnbx.BNBX_E_ALIGN
    assert call(x=A + 8) == bnbx.BNBX_E_ALIGN
    assert call(a=B + 2) == bnbx.BNBX_E_ALIGN
    assert call(xa=C + 1) == bnbx.BNBX_E_ALIGN


def test_probe_stream_read_rejects():
    f = bnbx.bnbx_probe_stream_read
    assert status_of(f, None, 16, None, 0, C, 0) == bnbx.BNBX_E_INVAL      # a NULL, a_bytes > 0
    assert status_of(f, A, 16, None, 16, C, 0) == bnbx.BNBX_E_INVAL       # b NULL, b_bytes > 0
    assert status_of(f, A, 16, None, 0, None, 0) == bnbx.BNBX_E_INVAL     # no sink
    assert status_of(f, A, 0, None, 0, C, 0) == bnbx.BNBX_E_INVAL         # nothing to read
    assert status_of(f, A, 24, None, 0, C, 0) == bnbx.BNBX_E_INVAL        # not whole 16 B units
    assert status_of(f, A + 8, 16, None, 0, C, 0) == bnbx.BNBX_E_ALIGN
    assert status_of(f, A, 16, B + 4, 16, C, 0) == bnbx.BNBX_E_ALIGN
    assert status_of(f, A, 16, None, 0, C + 2, 0) == bnbx.BNBX_E_ALIGN


def test_probe_binding_rejects_byte_counts_past_a_tensor():
    torch = pytest.importorskip("torch")
    a = torch.zeros(64, dtype=torch.uint8)          # never handed to the library
    sink = torch.zeros(bnbx.BNBX_PROBE_SINK_WORDS, dtype=torch.int32)
    with pytest.raises(bnbx.BnbxError) as e:
        bnbx.bnbx_probe_stream_read(a, 80, None, 0, sink, 0)
    assert e.value.status == bnbx.BNBX_E_INVAL
    with pytest.raises(bnbx.BnbxError):
        bnbx.bnbx_probe_stream_read(a, 32, a, 96, sink, 0)
    with pytest.raises(bnbx.BnbxError):
        bnbx.bnbx_probe_stream_read(a, 16, None, 0, sink[:10], 0)


@pytest.mark.parametrize("fn", ["gemv", "gemm"])
def test_matmul_rejects(fn):
    N, K = 256, 512

    def call(x=A, ldx=K, p=B, st=None, M=1, N_=N, K_=K, y=C, ldy=N):
        st = st if st is not None else state(N * K)
        if fn == "gemv":
            return status_of(bnbx.bnbx_gemv_nf4, x, ldx, p, st, M, N_, K_, y, ldy, 0)
        return status_of(bnbx.bnbx_gemm_nf4, x, ldx, p, st, M, N_, K_, y, ldy, None, 0, 0)

    assert call(x=None) == bnbx.BNBX_E_INVAL
    assert call(y=None) == bnbx.BNBX_E_INVAL
    assert call(p=None) == bnbx.BNBX_E_INVAL
    assert call(M=0) == bnbx.BNBX_E_INVAL
    assert call(N_=0) == bnbx.BNBX_E_INVAL
    assert call(K_=100, st=state(N * 100)) == bnbx.BNBX_E_INVAL      # K % 64 != 0
    assert call(st=state(N * K + 2)) == bnbx.BNBX_E_INVAL           # n != N*K
    assert call(ldx=K - 8) == bnbx.BNBX_E_INVAL
    assert call(ldy=N - 1) == bnbx.BNBX_E_INVAL
    assert call(ldx=K + 4) == bnbx.BNBX_E_ALIGN
    assert call(x=A + 8) == bnbx.BNBX_E_ALIGN
    assert call(p=B + 4) == bnbx.BNBX_E_ALIGN
    assert call(y=C + 1) == bnbx.BNBX_E_ALIGN
    assert call(st=state(N * K, blocksize=32)) == bnbx.BNBX_E_UNSUPPORTED
    if fn == "gemv":
        assert call(M=17) == bnbx.BNBX_E_INVAL
    else:
        assert status_of(bnbx.bnbx_gemm_nf4, A, K, B, state(N * K), 1, N, K, C, N, D + 8, 64,
                         0) == bnbx.BNBX_E_ALIGN      # workspace not 16-byte aligned


def test_binding_names_match_header():
    for name in header_functions():
        assert callable(getattr(bnbx, name)), name


def test_gemm_dx_rejects():
    st = state(n=128 * 256)
    f = bnbx.bnbx_gemm_nf4_dx
    assert status_of(f, None, 128, B, st, 4, 128, 256, C, 256, 0) == bnbx.BNBX_E_INVAL
    assert status_of(f, A, 128, B, st, 0, 128, 256, C, 256, 0) == bnbx.BNBX_E_INVAL
    assert status_of(f, A, 100, B, st, 4, 128, 256, C, 256, 0) == bnbx.BNBX_E_INVAL   # lddy < N
    assert status_of(f, A, 128, B, st, 4, 128, 256, C, 200, 0) == bnbx.BNBX_E_INVAL   # lddx < K
    assert status_of(f, A, 132, B, st, 4, 128, 256, C, 256, 0) == bnbx.BNBX_E_ALIGN   # lddy % 8
    assert status_of(f, A + 8, 128, B, st, 4, 128, 256, C, 256, 0) == bnbx.BNBX_E_ALIGN
    assert status_of(f, A, 128, B, state(n=96 * 256), 4, 96, 256, C, 256, 0) == \
        bnbx.BNBX_E_UNSUPPORTED                                                        # N % 64
    assert status_of(f, A, 128, B, state(n=128 * 250), 4, 128, 250, C, 256, 0) == \
        bnbx.BNBX_E_INVAL                                                              # K % 64


def test_gemm_lora_rejects():
    st = state(n=128 * 256)
    f = bnbx.bnbx_gemm_nf4_lora
    D2 = D + (1 << 16)
    ok = (A, 256, B, st, 4, 128, 256, C, 16, D2, 16, 16, D2 + 4096, 128, 0)
    def case(i, v):
        a = list(ok)
        a[i] = v
        return status_of(f, *a)
    assert case(7, None) == bnbx.BNBX_E_INVAL        # xa
    assert case(9, None) == bnbx.BNBX_E_INVAL        # lora_b
    assert case(11, 8) == bnbx.BNBX_E_INVAL          # r < 16
    assert case(11, 24) == bnbx.BNBX_E_INVAL         # r % 16
    assert case(8, 8) == bnbx.BNBX_E_INVAL           # ldxa < r
    assert case(10, 8) == bnbx.BNBX_E_INVAL          # ldb < r
    assert case(8, 20) == bnbx.BNBX_E_ALIGN          # ldxa % 8
    assert case(7, C + 8) == bnbx.BNBX_E_ALIGN       # xa alignment
    assert case(4, 0) == bnbx.BNBX_E_INVAL           # M


@pytest.mark.parametrize("case,expect", [
    ("null_w", bnbx.BNBX_E_INVAL),
    ("null_packed", bnbx.BNBX_E_INVAL),
    ("odd_n", bnbx.BNBX_E_INVAL),
    ("blocksize", bnbx.BNBX_E_UNSUPPORTED),
    ("null_absmax2", bnbx.BNBX_E_INVAL),
    ("misaligned_w", bnbx.BNBX_E_ALIGN),
    ("past_max", bnbx.BNBX_E_WORKSPACE),
])
def test_quantize_noalloc_rejects(case, expect):
    """The no-allocation quantize checks its arguments like bnbx_quantize_nf4
    and rejects double-quant sizes past its fixed scratch before any launch."""
    n = 4096
    w, p, st = A, B, state(n)
    if case == "null_w":
        w = None
    elif case == "null_packed":
        p = None
    elif case == "odd_n":
        st = state(n + 1)
    elif case == "blocksize":
        st = state(n, blocksize=128)
    elif case == "null_absmax2":
        st = state(n)
        st.absmax2 = None
    elif case == "misaligned_w":
        w = A + 2
    elif case == "past_max":
        st = state(bnbx.BNBX_NOALLOC_MAX_WEIGHTS + 2)
    assert status_of(bnbx.bnbx_quantize_nf4_noalloc, w, p, st, 0) == expect


def test_noalloc_limit_matches_header():
    text = open(os.path.join(ROOT, "include", "bnbx.h")).read()
    m = re.search(r"#define BNBX_NOALLOC_MAX_WEIGHTS \(\(int64_t\)1 << (\d+)\)", text)
    assert m and (1 << int(m.group(1))) == bnbx.BNBX_NOALLOC_MAX_WEIGHTS
