"""The C-ABI library on the host: it loads, exports every symbol the header
declares, and rejects bad arguments before any HIP call (no GPU needed)."""
import ctypes

import pytest

import gguf_quant_matmul_amd as gq
import oracle


def test_exports_every_declared_symbol():
    names = gq.header_symbols()
    assert {"gq_matmul", "gq_matmul_ex", "gq_matmul_decode", "gq_dequant", "gq_quantize",
            "gq_type_info", "gq_row_bytes", "gq_strerror"} <= set(names)
    L = gq.lib()
    for n in names:
        assert hasattr(L, n), n


def test_type_info_matches_oracle_and_pages():
    for t in gq.QUANT_TYPES:
        assert gq.type_info(t) == oracle.block_info(t)
    assert gq.type_info("q4_k") == (256, 144)      # Hitchhiker's Guide §11.2
    assert gq.row_bytes("q6_k", 11008) == 9030
    assert gq.row_bytes("q4_k", 4096) == 2304
    with pytest.raises(gq.GQError):
        gq.row_bytes("q4_k", 100)


def test_strerror_covers_codes():
    fallback = gq.strerror(-99)
    assert fallback == "unknown error code"
    msgs = [gq.strerror(c) for c in range(0, -7, -1)]
    assert all(m and m != fallback for m in msgs) and len(set(msgs)) == 7


A = 0x10000          # fake, 16-B aligned addresses: every call below must fail
B = 0x20000          # a check before touching them


@pytest.mark.parametrize("args,code", [
    ((A, 99, 16, 256, B, 0x30000, 1, None), -1),            # bad type
    ((A, gq.F32, 16, 256, B, 0x30000, 1, None), -1),        # F32 is not a weight type
    ((A, gq.Q4_K, 16, 100, B, 0x30000, 1, None), -2),       # cols % 256
    ((A, gq.Q4_K, 0, 256, B, 0x30000, 1, None), -2),        # rows < 1
    ((A, gq.Q4_K, 16, 256, B, 0x30000, -1, None), -2),      # n_tok < 0
    ((None, gq.Q4_K, 16, 256, B, 0x30000, 1, None), -3),    # null blob
    ((A, gq.Q4_K, 16, 256, None, 0x30000, 1, None), -3),    # null x
    ((A + 4, gq.Q4_K, 16, 256, B, 0x30000, 1, None), -4),   # misaligned blob
    ((A, gq.Q4_K, 16, 256, B + 8, 0x30000, 1, None), -4),   # misaligned x
    ((A, gq.Q4_K, 16, 256, B, B + 16, 1, None), -3),        # y overlaps x
    ((A, gq.Q4_K, 16, 256, B, A + 32, 1, None), -3),        # y overlaps blob
    ((A, gq.Q4_K, 1 << 31, 256, B, 0x30000, 1, None), -5),  # rows too large
    ((A, gq.Q4_K, 16, 32768, B, 0x30000, 1, None), -5),     # cols beyond GEMV LDS limit
])
def test_matmul_validation(args, code):
    assert gq.lib().gq_matmul(*args) == code


def test_matmul_zero_tokens_is_noop():
    # n_tok = 0 succeeds without touching any pointer
    assert gq.lib().gq_matmul(None, gq.Q4_K, 16, 256, None, None, 0, None) == 0


def test_matmul_ex_bad_x_type():
    assert gq.lib().gq_matmul_ex(A, gq.Q4_K, 16, 256, B, gq.Q8_0, 0x30000, 1, None) == -1


def test_dequant_and_quantize_validation():
    L = gq.lib()
    assert L.gq_dequant(A, gq.Q6_K, 4, 255, B, gq.F32, None) == -2
    assert L.gq_dequant(A, gq.Q6_K, 4, 256, B, gq.Q4_0, None) == -1
    assert L.gq_dequant(A, gq.Q6_K, 4, 256, A + 16, gq.F32, None) == -3
    assert L.gq_dequant(A, gq.Q6_K, 4, 256, B + 2, gq.F16, None) == -4
    assert L.gq_quantize(A, gq.Q4_K, 4, 200, B, None) == -2
    assert L.gq_quantize(None, gq.Q4_K, 4, 256, B, None) == -3
    assert L.gq_quantize(A, gq.Q4_K, 4, 256, A + 64, None) == -3


C = 0x30000
N = 0x40000          # fake norm weights
U = 0x50000          # fake up-projection blob


@pytest.mark.parametrize("args,code", [
    ((A, None, 99, 16, 256, B, gq.F32, None, 1e-5, C, None), -1),      # bad type
    ((A, None, gq.Q4_K, 16, 256, B, gq.Q8_0, None, 1e-5, C, None), -1),  # bad x_type
    ((A, None, gq.Q4_K, 16, 100, B, gq.F32, None, 1e-5, C, None), -2),   # cols % 256
    ((A, None, gq.Q4_K, 16, 256, B, gq.F32, N, -1.0, C, None), -2),      # eps < 0
    ((A, None, gq.Q4_K, 16, 256, B, gq.F32, N, float("nan"), C, None), -2),   # eps NaN
    ((A, None, gq.Q4_K, 16, 256, B, gq.F32, N, float("inf"), C, None), -2),   # eps inf
    ((None, U, gq.Q4_K, 16, 256, B, gq.F32, N, 1e-5, C, None), -3),      # null blob
    ((A, U, gq.Q4_K, 16, 256, None, gq.F32, N, 1e-5, C, None), -3),      # null x
    ((A, U, gq.Q4_K, 16, 256, B, gq.F32, N, 1e-5, None, None), -3),      # null y
    ((A, U + 4, gq.Q4_K, 16, 256, B, gq.F32, N, 1e-5, C, None), -4),     # misaligned up blob
    ((A, U, gq.Q4_K, 16, 256, B, gq.F32, N + 8, 1e-5, C, None), -4),     # misaligned norm weights
    ((A, U, gq.Q4_K, 16, 256, B, gq.F32, N, 1e-5, N + 16, None), -3),    # y overlaps norm weights
    ((A, U, gq.Q4_K, 16, 256, B, gq.F32, N, 1e-5, U + 32, None), -3),    # y overlaps up blob
    ((A, U, gq.Q4_K, 16, 256, B, gq.F32, N, 1e-5, B + 16, None), -3),    # y overlaps x
    ((A, U, gq.Q4_K, 16, 32768, B, gq.F32, N, 1e-5, C, None), -5),       # cols beyond the LDS limit
])
def test_matmul_decode_validation(args, code):
    assert gq.lib().gq_matmul_decode(*args) == code


def test_probe_validation():
    L = gq.lib()
    assert L.gq_probe_stream_read(A, 100, B, None) == -2           # not a multiple of 16
    assert L.gq_probe_stream_read(A, -16, B, None) == -2
    assert L.gq_probe_stream_read(A, (1 << 30) + 16, B, None) == -5
    assert L.gq_probe_stream_read(None, 64, B, None) == -3
    assert L.gq_probe_stream_read(None, 0, None, None) == -3
    assert L.gq_probe_stream_read(A, 64, None, None) == -3
    assert L.gq_probe_stream_read(A + 8, 64, B, None) == -4
    assert L.gq_probe_stream_read(A, 64, A + 32, None) == -3       # out overlaps buf


def test_attn_workspace_and_validation():
    L = gq.lib()
    # 32k positions, 8 KV heads, 40 query heads, head_dim 128: 128 chunks of 256
    assert L.gq_attn_decode_workspace_bytes(32768, 8, 40, 128) == 128 * 40 * 130 * 4
    assert L.gq_attn_decode_workspace_bytes(1, 1, 1, 64) == 1 * 1 * 66 * 4
    assert L.gq_attn_decode_workspace_bytes(10, 8, 44, 128) == -2     # heads not a multiple
    assert L.gq_attn_decode_workspace_bytes(10, 2, 34, 128) == -2     # 17 query heads per KV head
    assert L.gq_attn_decode_workspace_bytes(10, 2, 4, 96) == -2       # head_dim
    assert L.gq_attn_decode_workspace_bytes(0, 2, 4, 128) == -2       # no positions
    K, V, Q, O, WS = 0x100000, 0x200000, 0x300000, 0x310000, 0x400000
    ok = (K, V, gq.Q8_0, 100, 2, 128, Q, 8, O, WS, 1 << 20, None)

    def call(**kw):
        names = ["k", "v", "t", "n", "nkv", "hd", "q", "nh", "o", "ws", "wsb", "s"]
        a = dict(zip(names, ok))
        a.update(kw)
        return L.gq_attn_decode(*[a[n] for n in names])

    assert call(t=gq.Q4_K) == -1
    assert call(t=gq.F16) == -1
    assert call(hd=96) == -2
    assert call(nh=7) == -2 and call(nh=34, nkv=2) == -2
    assert call(wsb=100) == -2                                        # workspace too small
    assert call(k=None) == -3 and call(ws=None) == -3
    assert call(v=V + 4) == -4 and call(o=O + 8) == -4
    assert call(o=Q + 64) == -3                                       # out overlaps q
    assert call(ws=K + 256) == -3                                     # workspace overlaps the K cache
    assert call(n=1 << 28, nkv=8) == -5                               # cache beyond 2^31 bytes


def test_matmul_path_validation():
    L = gq.lib()
    args = (A, gq.Q4_K, 16, 256, B, gq.F32, 0x30000)
    assert L.gq_matmul_path(*args, 2, gq.PATH_GEMV, None) == -2          # GEMV needs one token
    assert L.gq_matmul_path(*args, 1, gq.PATH_TILED, None) == -2         # batched paths need two
    assert L.gq_matmul_path(*args, 1, gq.PATH_WEIGHT_STREAM, None) == -2
    assert L.gq_matmul_path(*args, 2, 7, None) == -2                     # unknown path
    assert L.gq_matmul_path(*args, 2, -1, None) == -2
    assert L.gq_matmul_path(A, gq.Q4_K, 16, 100, B, gq.F32, 0x30000, 2, gq.PATH_TILED, None) == -2
    assert L.gq_matmul_path(*args, 0, gq.PATH_TILED, None) == 0          # no tokens: no-op


def test_attn_kv_cache_bound():
    """Each KV cache stays within 0x7FFF0000 bytes: out-of-chunk loads go to
    that offset and must read as zero."""
    L = gq.lib()
    K, V, Q, O, WS = 0x100000, 0x200000, 0x300000, 0x310000, 0x400000
    rb = 136                                                          # q8_0, head_dim 128
    n_ok = 0x7FFF0000 // (8 * rb)
    assert L.gq_attn_decode(K, V, gq.Q8_0, n_ok + 1, 8, 128, Q, 8, O, WS, 1 << 40, None) == -5


def test_attn_noalloc_validation():
    """gq_attn_decode_noalloc: the same checks as gq_attn_decode, and a call
    whose workspace would exceed the fixed array is refused before any HIP
    call (so all of this runs without a GPU)."""
    L = gq.lib()
    K, V, Q, O = 0x100000, 0x200000, 0x300000, 0x310000
    ok = (K, V, gq.Q8_0, 100, 2, 128, Q, 8, O, None)

    def call(**kw):
        names = ["k", "v", "t", "n", "nkv", "hd", "q", "nh", "o", "s"]
        a = dict(zip(names, ok))
        a.update(kw)
        return L.gq_attn_decode_noalloc(*[a[n] for n in names])

    assert call(t=gq.Q4_K) == -1
    assert call(hd=96) == -2 and call(nh=7) == -2
    assert call(k=None) == -3 and call(o=None) == -3
    assert call(v=V + 4) == -4
    assert call(o=Q + 64) == -3
    # 2^22 positions, one KV head, 16 query heads of 128: 16384 chunks of 256,
    # 16384 * 16 * 130 * 4 bytes of statistics > the 32 MiB array
    big = L.gq_attn_decode_workspace_bytes(1 << 22, 1, 16, 128)
    assert big > (32 << 20)
    far = dict(k=1 << 40, v=2 << 40, q=3 << 40, o=4 << 40)          # ranges that do not overlap
    assert call(n=1 << 22, nkv=1, nh=16, **far) == -5
    assert "gq_attn_decode_noalloc" in gq.header_symbols()
