"""C-ABI checks that need no GPU: the library loads, exports every symbol the
public header declares, and rejects bad arguments on the host before any
launch (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import post_weight_quantization_04_amd as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gptq.h")
FAKE = ctypes.c_void_p(0x1000)      # never dereferenced: validation fails first


def declared_symbols():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"GPTQ_API\s+[\w\s\*]*?\b(gptq_\w+)\s*\(", src)))


def test_header_declares_the_two_entry_points():
    syms = declared_symbols()
    assert "gptq_hessian_accumulate" in syms and "gptq_quantize_layer" in syms
    assert len(syms) >= 10


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(P.LIB_PATH)
    for s in declared_symbols():
        assert hasattr(lib, s), s


def test_no_other_exported_symbols():
    # the library's dynamic symbol table holds the C ABI and nothing of ours besides
    out = os.popen(f"nm -D --defined-only {P.LIB_PATH}").read().split("\n")
    ours = sorted({l.split()[-1] for l in out if l.strip() and "gptq" in l.split()[-1]})
    assert set(ours) == set(declared_symbols()), ours


def test_host_helpers():
    assert P.packed_words(4096, 4) == 512
    assert P.packed_words(4096, 3) == 384
    assert P.packed_words(33, 3) == 4
    assert P.packed_words(10, 5) == -1
    assert P.num_groups(4096, 128) == 32
    assert P.num_groups(11008, 128) == 86
    assert P.num_groups(4096, -1) == 1
    assert P.num_groups(100, 200) == 1
    assert P.num_groups(100, 0) == -1
    lib = P.lib
    assert lib.gptq_status_string(2) == b"damped Hessian not positive definite"
    assert b"gfx950" in lib.gptq_version()


def test_workspace_sizes():
    ws = P.quantize_layer_workspace_size(4096, 4096, 4, 128, 128, 0)
    assert ws >= 4 * 4096 * 4096 + 4 * 4096 * 4096
    assert ws < 4 * 4096 * 4096 * 3
    assert P.quantize_layer_workspace_size(4096, 4096, 4, 100, 128, 0) == 0   # group not a multiple of 16
    assert P.quantize_layer_workspace_size(4096, 4096, 5, 128, 128, 0) == 0
    h = P.hessian_workspace_size(262144, 4096, P.BF16)
    assert h > 0 and h % 256 == 0
    assert P.hessian_workspace_size(0, 4096, P.BF16) == 0
    assert P.hessian_workspace_size(10, 0, P.BF16) == 0


def _q(**kw):
    a = dict(W=FAKE, dt=P.BF16, d_out=64, d_in=256, H=FAKE, bits=4, g=128, B=128, damp=0.01, act=0,
             Q=FAKE, S=FAKE, Z=FAKE, perm=FAKE, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return P.lib.gptq_quantize_layer(a["W"], a["dt"], a["d_out"], a["d_in"], a["H"], a["bits"], a["g"], a["B"],
                                     a["damp"], a["act"], a["Q"], a["S"], a["Z"], a["perm"], a["ws"], a["wsb"],
                                     a["stream"])


@pytest.mark.parametrize("kw,msg", [
    (dict(W=None), "NULL"), (dict(H=None), "NULL"), (dict(Q=None), "NULL"), (dict(perm=None), "NULL"),
    (dict(d_out=0), "d_out"), (dict(d_in=-3), "d_in"), (dict(bits=5), "bits"), (dict(bits=1), "bits"),
    (dict(g=100), "multiple of 16"), (dict(g=0), "group_size"), (dict(g=64, B=96), "multiple of group_size"),
    (dict(B=0), "block_size"), (dict(damp=float("nan")), "damp"), (dict(damp=-1.0), "damp"),
    (dict(act=2), "act_order"), (dict(dt=7), "w_dtype"),
])
def test_quantize_layer_rejects_bad_arguments(kw, msg):
    assert _q(**kw) == 1
    assert msg in P.lib.gptq_last_error().decode()


def test_quantize_layer_workspace_too_small():
    assert _q(wsb=1024) == 4
    assert _q(ws=None) == 4


def test_group_spanning_row_allows_any_block():
    # one group per row: any block size is accepted (check stops at the workspace)
    assert _q(g=-1, B=100, wsb=16) == 4
    assert _q(g=512, B=100, d_in=256, wsb=16) == 4


def test_hessian_rejects_bad_arguments():
    L = P.lib
    assert L.gptq_hessian_accumulate(FAKE, 5, 10, 10, FAKE, FAKE, 1 << 30, None) == 1
    assert L.gptq_hessian_accumulate(FAKE, P.BF16, -1, 10, FAKE, FAKE, 1 << 30, None) == 1
    assert L.gptq_hessian_accumulate(FAKE, P.BF16, 10, 0, FAKE, FAKE, 1 << 30, None) == 1
    assert L.gptq_hessian_accumulate(FAKE, P.BF16, 10, 10, None, FAKE, 1 << 30, None) == 1
    assert L.gptq_hessian_accumulate(None, P.BF16, 10, 10, FAKE, FAKE, 1 << 30, None) == 1
    assert L.gptq_hessian_accumulate(FAKE, P.BF16, 10, 10, FAKE, FAKE, 8, None) == 4
    # n == 0 is a no-op that touches nothing
    assert L.gptq_hessian_accumulate(None, P.BF16, 0, 10, FAKE, None, 0, None) == 0


def test_inverse_factor_rejects_bad_arguments():
    L = P.lib
    assert L.gptq_inverse_factor(None, 10, 0.01, 0, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert L.gptq_inverse_factor(FAKE, 0, 0.01, 0, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert L.gptq_inverse_factor(FAKE, 10, float("inf"), 0, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert L.gptq_inverse_factor(FAKE, 10, 0.01, 0, FAKE, FAKE, FAKE, 4, None) == 4


def test_hessian_noalloc_limits_and_rejections():
    L = P.lib
    # the static scratch holds 1024 partial 256x256 tiles (bf16) or 4096 of
    # 128x128 (fp32): one token split of every lower tile up to these d_in
    assert P.hessian_noalloc_max_d_in(P.BF16) == 44 * 256
    assert P.hessian_noalloc_max_d_in(P.F32) == 90 * 128
    assert P.hessian_noalloc_max_d_in(7) == -1
    big = P.hessian_noalloc_max_d_in(P.BF16) + 1
    assert L.gptq_hessian_accumulate_noalloc(FAKE, P.BF16, 100, big, FAKE, None) == 1
    assert b"static scratch" in L.gptq_last_error()
    assert L.gptq_hessian_accumulate_noalloc(FAKE, 5, 10, 10, FAKE, None) == 1
    assert L.gptq_hessian_accumulate_noalloc(FAKE, P.BF16, -1, 10, FAKE, None) == 1
    assert L.gptq_hessian_accumulate_noalloc(FAKE, P.BF16, 10, 0, FAKE, None) == 1
    assert L.gptq_hessian_accumulate_noalloc(FAKE, P.BF16, 10, 10, None, None) == 1
    assert L.gptq_hessian_accumulate_noalloc(None, P.BF16, 10, 10, FAKE, None) == 1
    # n == 0 is a no-op that touches nothing
    assert L.gptq_hessian_accumulate_noalloc(None, P.BF16, 0, 10, FAKE, None) == 0


def test_dequant_matmul_rejects_bad_arguments():
    L = P.lib
    ok = dict(A=FAKE, at=P.BF16, m=2, d_in=256, Q=FAKE, S=FAKE, Z=FAKE, perm=None, d_out=64, bits=4, g=128,
              Y=FAKE, yt=P.F32, ws=FAKE, wsb=1 << 30)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return L.gptq_dequant_matmul(a["A"], a["at"], a["m"], a["d_in"], a["Q"], a["S"], a["Z"], a["perm"],
                                     a["d_out"], a["bits"], a["g"], a["Y"], a["yt"], a["ws"], a["wsb"], None)

    for kw in (dict(A=None), dict(Q=None), dict(S=None), dict(Z=None), dict(Y=None), dict(m=-1), dict(d_in=0),
               dict(d_out=0), dict(bits=5), dict(g=100), dict(g=0), dict(at=7), dict(yt=7)):
        assert call(**kw) == 1, kw
    assert call(m=0, A=None, ws=None, wsb=0) == 0          # no-op
    # partial sums of the k-ranges (a multiple of one 4096-row fp32 vector),
    # then 16 tile counters in their own 256-byte block
    ws = P.dequant_matmul_workspace_size(1, 4096, 4096, 4, 128)
    assert ws > 4096 * 4 and (ws - 256) % (4096 * 4) == 0
    assert call(wsb=16) == 4
    assert P.dequant_matmul_workspace_size(0, 4096, 4096, 4, 128) == 0
    assert P.dequant_matmul_workspace_size(1, 4096, 4096, 5, 128) == 0


def test_quantize_layers_rejects_bad_arguments():
    L = P.lib
    n = 2
    arr = lambda: (ctypes.c_void_p * n)(FAKE.value, FAKE.value)
    dout = (ctypes.c_int64 * n)(64, 32)

    def call(**kw):
        a = dict(n=n, W=arr(), dt=P.BF16, dout=dout, d_in=256, H=FAKE, bits=4, g=128, B=128, damp=0.01, act=0,
                 Q=arr(), S=arr(), Z=arr(), perm=FAKE, ws=FAKE, wsb=1 << 40)
        a.update(kw)
        return L.gptq_quantize_layers(a["n"], a["W"], a["dt"], a["dout"], a["d_in"], a["H"], a["bits"], a["g"],
                                      a["B"], a["damp"], a["act"], a["Q"], a["S"], a["Z"], a["perm"], a["ws"],
                                      a["wsb"], None)

    assert call(n=0) == 1
    assert call(W=None) == 1
    assert call(W=(ctypes.c_void_p * n)(FAKE.value, None)) == 1
    assert call(dout=(ctypes.c_int64 * n)(64, 0)) == 1
    assert call(bits=5) == 1
    assert call(perm=None) == 1
    assert call(wsb=1024) == 4
    # the workspace is that of the widest layer
    assert L.gptq_quantize_layers_workspace_size(n, dout, 256, 4, 128, 128, 0) == \
        P.quantize_layer_workspace_size(64, 256, 4, 128, 128, 0)
