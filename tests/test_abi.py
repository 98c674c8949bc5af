"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")


@pytest.fixture(scope="module")
def pkg():
    import compressed_fp4_kv_amd as p
    return p


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(pkg):
    names = _declared()
    assert len(names) >= 13
    for n in names:
        assert hasattr(pkg.lib, n), n
    assert sorted(pkg.EXPORTED_SYMBOLS) == names


def test_status_strings(pkg):
    for s in range(6):
        assert pkg.lib.csa2_status_str(s).decode().startswith("CSA2")


NULL = None


def _idx(pkg, fn="csa2_index_full", **kw):
    a = dict(qI=1, kI=1, off=1, qseq=1, nvis=1, Q=1, Hi=4, Hk=4, Di=128, maxn=100, topk=8,
             out=1, P=0, bs=8, pool=NULL, ws=1, wsb=1 << 30)
    a.update(kw)
    v = lambda x: None if x is None else ctypes.c_void_p(16 * x)
    return getattr(pkg.lib, fn)(v(a["qI"]), v(a["kI"]), v(a["off"]), v(a["qseq"]), v(a["nvis"]),
                                   a["Q"], a["Hi"], a["Hk"], a["Di"], a["maxn"], a["topk"],
                                   v(a["out"]), a["P"], a["bs"], v(a["pool"]), v(a["ws"]), a["wsb"],
                                   None)


def test_index_full_argument_checks(pkg):
    assert _idx(pkg, qI=NULL) == 1
    assert _idx(pkg, out=NULL) == 1
    assert _idx(pkg, P=16, pool=NULL) == 1
    assert _idx(pkg, Q=-1) == 2
    assert _idx(pkg, topk=-3) == 2
    assert _idx(pkg, Hk=2) == 3            # neither 1 nor Hi
    assert _idx(pkg, Di=100) == 3          # row width not 256/512/1024
    assert _idx(pkg, topk=4096) == 3
    assert _idx(pkg, P=16, bs=3, pool=1) == 3
    assert _idx(pkg, P=16, bs=0, pool=1) == 2
    assert _idx(pkg, wsb=10) == 4
    assert _idx(pkg, Q=0) == 0             # nothing to do, nothing launched
    need = pkg.csa2_index_full_workspace_bytes(1, 100, 8, 0, 8)
    assert need > 0 and _idx(pkg, wsb=need - 1) == 4
    # the prefill form (q_seq NULL) also holds the bf16 row copies: a
    # workspace sized for the decode form is refused before any launch
    pre = pkg.csa2_index_prefill_workspace_bytes(1, 100, 8, 4, 128)
    assert pre > need
    assert _idx(pkg, qseq=NULL, wsb=need) == 4
    assert _idx(pkg, qseq=NULL, wsb=pre - 1) == 4
    # a pool in the prefill form needs the larger workspace of the _ex query
    pre_pool = pkg.csa2_index_prefill_workspace_bytes_ex(1, 100, 8, 16, 8, 4, 128)
    assert pre_pool > pre
    assert _idx(pkg, qseq=NULL, P=16, pool=1, wsb=pre) == 4
    assert pkg.csa2_index_prefill_workspace_bytes_ex(1, 100, 8, 0, 1, 4, 128) == pre
    assert pkg.csa2_index_prefill_workspace_bytes(-1, 100, 8, 4, 128) == 0


def test_index_full_e4m3_argument_checks(pkg):
    # the E4M3-key form shares the checks of csa2_index_full
    f = "csa2_index_full_e4m3"
    assert _idx(pkg, f, kI=NULL) == 1
    assert _idx(pkg, f, Q=-1) == 2
    assert _idx(pkg, f, Hk=2) == 3
    assert _idx(pkg, f, Di=100) == 3
    assert _idx(pkg, f, wsb=10) == 4
    assert _idx(pkg, f, Q=0) == 0
    pre = pkg.csa2_index_prefill_workspace_bytes(1, 100, 8, 4, 128)
    assert _idx(pkg, f, qseq=NULL, wsb=pre - 1) == 4
    assert _idx(pkg, f, qseq=NULL, P=16, pool=1, wsb=pre) == 4


@pytest.mark.parametrize("fn", ["csa2_reindex", "csa2_reindex_e4m3"])
def test_reindex_argument_checks(pkg, fn):
    v = lambda x: None if x is None else ctypes.c_void_p(16 * x)
    f = getattr(pkg.lib, fn)
    base = [v(1), v(1), v(1), v(1), v(1), v(1), 2048, 8, 4, 4, 4, 128, 512, v(1), v(1), 1 << 30, None]
    assert f(*base[:5], None, *base[6:]) == 1
    b = list(base); b[6] = 4096
    assert f(*b) == 3                       # 4096 x 8 > 16,384 candidates
    b = list(base); b[7] = 0
    assert f(*b) == 2
    b = list(base); b[15] = 8
    assert f(*b) == 4
    b = list(base); b[1] = None
    assert f(*b) == 1                       # no key cache


def test_attention_argument_checks(pkg):
    v = lambda x: None if x is None else ctypes.c_void_p(16 * x)
    f = pkg.lib.csa2_sparse_attn_decode
    base = [v(1), v(1), v(1), v(1), v(1), 512, v(1), v(1), v(1), 128, 4, 64, 512, 0.04, v(1), None,
            v(1), 1 << 30, None]
    b = list(base); b[12] = 256
    assert f(*b) == 3                       # D != 512
    b = list(base); b[11] = 24
    assert f(*b) == 3                       # H not a multiple of 16
    b = list(base); b[0] = None
    assert f(*b) == 1
    b = list(base); b[10] = -1
    assert f(*b) == 2
    b = list(base); b[17] = 0
    assert f(*b) == 4                       # needs split workspace at B=4
    g = pkg.lib.csa2_sparse_attn_prefill_chunk
    pb = [v(1), -5, v(1), v(1), v(1), 512, v(1), v(1), 128, 64, 64, 512, 0.04, v(1), None, v(1),
          1 << 30, None]
    assert g(*pb) == 2                      # negative position


def test_index_full_ex_refuses_unknown_rule_and_key_format(pkg):
    v = lambda x: ctypes.c_void_p(16 * x)
    f = pkg.lib.csa2_index_full_ex
    base = [v(1), v(1), 0, v(1), v(1), v(1), 1, 4, 4, 128, 100, 8, v(1), 16, 8, v(1), 0, v(1),
            1 << 30, None]
    b = list(base); b[16] = 2
    assert f(*b) == 3                       # unknown block rule
    b = list(base); b[2] = 7
    assert f(*b) == 3                       # unknown key format
    b = list(base); b[1] = None
    assert f(*b) == 1
    b = list(base); b[18] = 10
    assert f(*b) == 4


def test_decode_layers_argument_checks(pkg):
    arr = (ctypes.c_void_p * 2)(16, 32)
    v = lambda x: ctypes.c_void_p(16 * x)
    f = pkg.lib.csa2_sparse_attn_decode_layers
    base = [2, arr, v(1), v(1), v(1), v(1), 512, arr, arr, v(1), 128, 4, 64, 512, 0.04, arr, None,
            v(1), 1 << 30, None]
    b = list(base); b[0] = 0
    assert f(*b) == 2                       # no layer
    b = list(base); b[0] = 9
    assert f(*b) == 3                       # more than 8 layers
    b = list(base); b[1] = None
    assert f(*b) == 1
    b = list(base); b[12] = 24
    assert f(*b) == 3                       # H not a multiple of 16
    b = list(base); b[18] = 0
    assert f(*b) == 4                       # 2 layers x 4 queries need split partials
    # one layer is the per-layer call; 4 layers x 64 queries fill the chip unsplit
    assert (pkg.csa2_decode_layers_workspace_bytes(1, 32, 64, 512, 512, 128)
            == pkg.csa2_decode_workspace_bytes(32, 64, 512, 512, 128))
    assert pkg.csa2_decode_layers_workspace_bytes(4, 64, 64, 512, 512, 128) == 0
    assert pkg.csa2_decode_layers_workspace_bytes(9, 64, 64, 512, 512, 128) == 0


def test_kv_quantize_argument_checks(pkg):
    # every case below is refused (or is an empty call) on the host: nothing launches
    f = pkg.lib.csa2_kv_quantize_fp4
    p = lambda a: None if a is None else ctypes.c_void_p(a)
    ok = dict(x=0x10000, rows=4, D=512, codes=0x20000, scales=0x30000)

    def call(**kw):
        a = dict(ok, **kw)
        return f(p(a["x"]), a["rows"], a["D"], p(a["codes"]), p(a["scales"]), None)

    assert call(rows=-1) == 2
    assert call(D=0) == 2
    assert call(D=24) == 3                  # not a whole number of 16-channel groups
    assert call(rows=0, x=None, codes=None, scales=None) == 0
    assert call(x=None) == 1
    assert call(scales=None) == 1
    assert call(x=0x10008) == 3             # fp32 rows must be 16-byte aligned
    assert call(codes=0x20001) == 3         # code rows must be 2-byte aligned


def test_swa_append_argument_checks(pkg):
    f = pkg.lib.csa2_swa_append
    p = lambda a: None if a is None else ctypes.c_void_p(a)
    ok = dict(k=0x10000, v=0x20000, pos=0x30000, B=2, D=512, W=128, sk=0x40000, sv=0x50000)

    def call(**kw):
        a = dict(ok, **kw)
        return f(p(a["k"]), p(a["v"]), p(a["pos"]), a["B"], a["D"], a["W"], p(a["sk"]),
                 p(a["sv"]), None)

    assert call(B=-1) == 2
    assert call(W=0) == 2
    assert call(D=0) == 2
    assert call(D=12) == 3
    assert call(B=0, k=None, v=None, pos=None, sk=None, sv=None) == 0
    assert call(pos=None) == 1
    assert call(sv=None) == 1
    assert call(k=0x10008) == 3
    assert call(sk=0x40004) == 3


def test_reindex_noalloc_argument_checks(pkg):
    v = lambda x: ctypes.c_void_p(16 * x)

    def call(Q=1, P=2048, bs=8, topk=512):
        return pkg.lib.csa2_reindex_noalloc(v(1), v(1), v(1), v(1), v(1), v(1), P, bs, Q, 4, 4,
                                            128, topk, v(1), None)
    # more candidates than the static scratch holds: refused before anything is enqueued
    assert pkg.NOALLOC_MAX_CAND == 2097152
    assert call(Q=129) == 3
    assert call(Q=1, P=2048, bs=8 * 129) == 3
    assert call(Q=-1) == 2 and call(bs=0) == 2 and call(topk=-1) == 2 and call(P=-5) == 2
    assert call(Q=0) == 0             # nothing to do, nothing launched
