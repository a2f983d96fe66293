"""The C ABI library: it loads, exports what include/msa.h declares, and rejects
bad arguments before launching anything (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")


@pytest.fixture(scope="module")
def L():
    from learned_block_sparse_amd import msa
    if not os.path.exists(msa.LIB_PATH):
        from learned_block_sparse_amd import build
        build.build()
    return msa.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_three_entry_points():
    names = _declared_functions()
    for n in ("msa_index_topk", "msa_sparse_attn_prefill", "msa_sparse_attn_decode"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    names = _declared_functions()
    assert len(names) >= 7
    for n in names:
        assert hasattr(L, n), f"libmsa.so does not export {n}"


def test_no_torch_or_oracle_symbols_in_library():
    """The product library links neither torch nor the oracle."""
    from learned_block_sparse_amd import msa
    data = open(msa.LIB_PATH, "rb").read()
    assert b"oracle_index_topk" not in data and b"oracle_sparse_attn" not in data
    assert b"libtorch" not in data and b"libc10" not in data


def test_status_strings(L):
    for code, name in enumerate(["MSA_OK", "MSA_ERR_INVALID_ARG", "MSA_ERR_UNSUPPORTED",
                                 "MSA_ERR_WORKSPACE", "MSA_ERR_HIP"]):
        assert L.msa_status_string(code).decode() == name
    assert L.msa_status_string(99).decode() == "MSA_ERR_UNKNOWN"


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


def _index(L, **kw):
    a = dict(q=FAKE, k=FAKE, dtype=1, cuq=FAKE, cuk=FAKE, batch=1, mq=256, mk=256, G=4, DI=128,
             bk=128, topk=16, out=FAKE, ws=None, wsb=0, stream=None)
    a.update(kw)
    return L.msa_index_topk(a["q"], a["k"], a["dtype"], a["cuq"], a["cuk"], a["batch"], a["mq"], a["mk"],
                            a["G"], a["DI"], a["bk"], a["topk"], a["out"], a["ws"], a["wsb"], a["stream"])


def test_index_topk_argument_errors(L):
    assert _index(L, q=None) == 1
    assert _index(L, batch=0) == 1
    assert _index(L, dtype=7) == 1
    assert _index(L, topk=0) == 1
    assert _index(L, bk=64) == 2
    assert _index(L, DI=96) == 2
    assert _index(L, topk=17) == 2
    assert _index(L, G=17) == 2
    # prefill with more than one block needs a workspace
    assert L.msa_index_topk_workspace_size(1, 256, 256, 4, 128, 16) > 0
    assert _index(L) == 3
    assert _index(L, ws=FAKE, wsb=16) == 3


def test_index_topk_noalloc_argument_errors(L):
    """The allocation-free variant checks like msa_index_topk and refuses calls
    whose scratch would exceed its static array, all before any HIP call."""
    def call(**kw):
        a = dict(q=FAKE, k=FAKE, dtype=1, cuq=FAKE, cuk=FAKE, batch=1, mq=256, mk=256, G=4, DI=128,
                 bk=128, topk=16, out=FAKE, stream=None)
        a.update(kw)
        return L.msa_index_topk_noalloc(a["q"], a["k"], a["dtype"], a["cuq"], a["cuk"], a["batch"], a["mq"],
                                        a["mk"], a["G"], a["DI"], a["bk"], a["topk"], a["out"], a["stream"])
    assert call(out=None) == 1
    assert call(batch=0) == 1
    assert call(dtype=7) == 1
    assert call(bk=64) == 2
    assert call(topk=17) == 2
    limit = 32 << 20
    assert L.msa_index_topk_workspace_size(1, 32768, 32768, 4, 128, 16) > limit
    assert call(mq=32768, mk=32768) == 3
    assert L.msa_index_topk_workspace_size(32, 1, 1 << 20, 4, 128, 16) <= limit


def test_workspace_sizes(L):
    # a single block per sequence needs no candidate buffer
    assert L.msa_index_topk_workspace_size(1, 100, 100, 4, 128, 16) == 0
    # decode: one fp32 score per (sequence, group, block)
    assert L.msa_index_topk_workspace_size(3, 1, 1000, 4, 128, 16) >= 3 * 4 * 8 * 4
    # unsupported block size reports 0
    assert L.msa_index_topk_workspace_size(1, 256, 256, 4, 64, 16) == 0
    # one split: no workspace; more splits: partial outputs
    assert L.msa_sparse_attn_workspace_size(1, 8192, 8192, 64, 4, 128, 16, 1) == 0
    ws = L.msa_sparse_attn_workspace_size(2, 1, 4096, 64, 4, 128, 16, 4)
    assert ws >= 2 * 64 * 4 * (128 + 1) * 4
    # automatic schedule of a large prefill: KV-outer edge lists + bf16 partial slots
    kvo = L.msa_sparse_attn_workspace_size(1, 8192, 131072, 64, 4, 128, 16, 0)
    assert kvo >= 8192 * 4 * 16 * (16 * 128 * 2 + 16 * 4)


def _prefill(L, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=1, bi=FAKE, cuq=FAKE, cuk=FAKE, batch=1, mq=256, mk=256,
             Hq=64, Hkv=4, D=128, bk=128, topk=16, scale=0.0, ns=0, out=FAKE, lse=None, ws=None,
             wsb=0, stream=None)
    a.update(kw)
    return L.msa_sparse_attn_prefill(a["q"], a["k"], a["v"], a["dtype"], a["bi"], a["cuq"], a["cuk"],
                                     a["batch"], a["mq"], a["mk"], a["Hq"], a["Hkv"], a["D"], a["bk"],
                                     a["topk"], a["scale"], a["ns"], a["out"], a["lse"], a["ws"],
                                     a["wsb"], a["stream"])


def test_prefill_argument_errors(L):
    assert _prefill(L, out=None) == 1
    assert _prefill(L, Hq=63) == 1           # not a multiple of Hkv
    assert _prefill(L, ns=-1) == 1
    assert _prefill(L, D=64) == 2
    assert _prefill(L, Hq=68, Hkv=4) == 2    # 17 heads per group
    assert _prefill(L, bk=256) == 2
    assert _prefill(L, ns=4) == 3            # split partials need a workspace


def test_decode_argument_errors(L):
    args = [FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, 32, 1 << 20, 64, 4, 128, 128, 16, 0.0, 0, FAKE,
            None, None, 0, None]
    assert L.msa_sparse_attn_decode(*args) == 3      # automatic splits need a workspace
    bad = list(args)
    bad[5] = None                                    # cache_offsets
    assert L.msa_sparse_attn_decode(*bad) == 1
    bad = list(args)
    bad[11] = 96                                     # head_dim
    assert L.msa_sparse_attn_decode(*bad) == 2


def _frontend(L, **kw):
    a = dict(x=FAKE, wq=FAKE, wk=FAKE, dtype=1, gq=FAKE, gk=FAKE, cuq=FAKE, cuk=FAKE, batch=1, total=256,
             dm=3072, G=4, DI=128, rope=64, theta=10000.0, eps=1e-6, q=FAKE, k=FAKE, odt=1, stream=None)
    a.update(kw)
    return L.msa_index_frontend(a["x"], a["wq"], a["wk"], a["dtype"], a["gq"], a["gk"], a["cuq"], a["cuk"],
                                a["batch"], a["total"], a["dm"], a["G"], a["DI"], a["rope"], a["theta"], a["eps"],
                                a["q"], a["k"], a["odt"], a["stream"])


def test_frontend_argument_errors(L):
    assert _frontend(L, x=None) == 1
    assert _frontend(L, wq=None, total=0) == 1
    assert _frontend(L, gk=None) == 1
    assert _frontend(L, total=-1) == 1
    assert _frontend(L, rope=130) == 1       # wider than the head
    assert _frontend(L, theta=0.0) == 1
    assert _frontend(L, eps=-1.0) == 1
    assert _frontend(L, dtype=7) == 1
    assert _frontend(L, dtype=2) == 2        # fp8 hidden states
    assert _frontend(L, odt=2) == 2
    assert _frontend(L, DI=96) == 2
    assert _frontend(L, dm=3000) == 2        # not a multiple of 64
    assert _frontend(L, rope=32) == 2
    assert _frontend(L, DI=64, rope=128) == 1
    # no tokens: nothing to launch, and the token-indexed buffers may be null
    assert _frontend(L, total=0) == 0
    assert _frontend(L, total=0, x=None, q=None, k=None) == 0


def test_frontend_backward_argument_errors_and_workspace(L):
    def call(**kw):
        a = dict(x=FAKE, wq=FAKE, wk=FAKE, dtype=1, gq=FAKE, gk=FAKE, cuq=FAKE, cuk=FAKE, batch=1, total=256,
                 dm=3072, G=4, DI=128, rope=64, theta=10000.0, eps=1e-6, dq=FAKE, dk=FAKE, dwq=FAKE, dwk=FAKE,
                 dgq=FAKE, dgk=FAKE, ws=None, wsb=0, stream=None)
        a.update(kw)
        return L.msa_index_frontend_backward(*a.values())
    assert call(dq=None) == 1
    assert call(dgk=None) == 1
    assert call(theta=-1.0) == 1
    assert call(dtype=0) == 2                # fp32 hidden states
    assert call(DI=96) == 2
    assert call(rope=32) == 2
    assert call() == 3                       # needs a workspace
    ws = L.msa_index_frontend_backward_workspace_size(131072, 3072, 4, 128)
    # dy (bf16) + at least one fp32 slice of the weight gradient
    assert ws >= 131072 * 640 * 2 + 640 * 3072 * 4
    assert L.msa_index_frontend_backward_workspace_size(0, 3072, 4, 128) == 0
    assert L.msa_index_frontend_backward_workspace_size(10, 3000, 4, 128) == 0


def _backward(L, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, dout=FAKE, lse=FAKE, dtype=1, bi=FAKE, cuq=FAKE, cuk=FAKE, batch=1,
             mq=256, mk=256, Hq=64, Hkv=4, D=128, bk=128, topk=16, scale=0.0, dq=FAKE, dk=FAKE, dv=FAKE, ws=None,
             wsb=0, stream=None)
    a.update(kw)
    return L.msa_sparse_attn_backward(a["q"], a["k"], a["v"], a["out"], a["dout"], a["lse"], a["dtype"], a["bi"],
                                      a["cuq"], a["cuk"], a["batch"], a["mq"], a["mk"], a["Hq"], a["Hkv"], a["D"],
                                      a["bk"], a["topk"], a["scale"], a["dq"], a["dk"], a["dv"], a["ws"], a["wsb"],
                                      a["stream"])


def test_backward_argument_errors_and_workspace(L):
    assert _backward(L, dout=None) == 1
    assert _backward(L, lse=None) == 1
    assert _backward(L, dk=None) == 1
    assert _backward(L, Hq=63) == 1          # not a multiple of Hkv
    assert _backward(L, dtype=0) == 2        # the backward takes bf16 inputs only
    assert _backward(L, D=64) == 2
    assert _backward(L, topk=17) == 2
    assert _backward(L) == 3                 # edge lists and dq partials need a workspace
    # one window of at most 8192 rows: edge lists, delta per (row, head) and bf16 dq partials per slot
    ws = L.msa_sparse_attn_backward_workspace_size(1, 8192, 131072, 64, 4, 128, 16)
    assert ws >= 8192 * 4 * 16 * 16 * 128 * 2 + 8192 * 64 * 4
    # the window is capped: a longer call needs no more partial space than 8192 rows
    ws2 = L.msa_sparse_attn_backward_workspace_size(1, 65536, 131072, 64, 4, 128, 16)
    assert ws2 - ws < 65536 * 64 * 4 + (1 << 20)
    assert L.msa_sparse_attn_backward_workspace_size(0, 8192, 131072, 64, 4, 128, 16) == 0


def _kl(L, **kw):
    a = dict(qi=FAKE, ki=FAKE, dtype=1, bi=FAKE, lse=FAKE, blse=FAKE, cuq=FAKE, cuk=FAKE, batch=1, mq=256, mk=256,
             Hq=64, G=4, DI=128, bk=128, topk=16, loss=FAKE, dq=FAKE, dk=FAKE, ws=None, wsb=0, stream=None)
    a.update(kw)
    return L.msa_index_kl_backward(a["qi"], a["ki"], a["dtype"], a["bi"], a["lse"], a["blse"], a["cuq"], a["cuk"],
                                   a["batch"], a["mq"], a["mk"], a["Hq"], a["G"], a["DI"], a["bk"], a["topk"],
                                   a["loss"], a["dq"], a["dk"], a["ws"], a["wsb"], a["stream"])


def test_index_kl_argument_errors_and_workspace(L):
    assert _kl(L, blse=None) == 1            # the forward's per-slot block LSEs are required
    assert _kl(L, loss=None) == 1
    assert _kl(L, Hq=62) == 1                # not a multiple of the groups
    assert _kl(L, DI=96) == 2
    assert _kl(L, Hq=68, G=4) == 2           # 17 heads per group
    assert _kl(L, dtype=2) == 2              # E4M3 index tensors are not taken here
    assert _kl(L) == 3
    ws = L.msa_index_kl_workspace_size(1, 8192, 131072, 4, 16)
    assert ws >= 8192 * 4 * 16 * 4 * 3       # score, argmax and dS per attended slot of one window
    assert L.msa_index_kl_workspace_size(1, 8192, 131072, 0, 16) == 0


def test_attention_ex_element_types(L):
    # bf16 q/out with E4M3 K/V is the one mixed pair; E4M3 q, or E4M3 K/V under fp32 q, is unsupported
    # (the accepted pair itself is not called here: it would launch)
    args = [FAKE, FAKE, FAKE, 1, 2, FAKE, FAKE, FAKE, 1, 256, 256, 64, 4, 128, 128, 16, 0.0, 1, FAKE, None, None,
            None, 0, None]
    bad = list(args)
    bad[3], bad[4] = 0, 2
    assert L.msa_sparse_attn_prefill_ex(*bad) == 2
    bad = list(args)
    bad[3], bad[4] = 2, 2
    assert L.msa_sparse_attn_prefill_ex(*bad) == 2
    dec = [FAKE, FAKE, FAKE, 0, 2, FAKE, FAKE, FAKE, 4, 4096, 64, 4, 128, 128, 16, 0.0, 1, FAKE, None, None, None,
           0, None]
    assert L.msa_sparse_attn_decode_ex(*dec) == 2
