"""The C-ABI library loads on a CPU-only host, exports every symbol the header
declares, and rejects bad arguments before touching the GPU (CPU only)."""
import ctypes
import os
import re

import pytest

import split_kv_paged_amd as skv
from split_kv_paged_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "skv.h")
P = ctypes.c_void_p(4096)       # a non-NULL pointer value that is never dereferenced


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S.*?\b(skv_\w+)\(", text, flags=re.M)))


def test_header_declarations_are_exported():
    lib = skv.load()
    names = _declared()
    assert names == sorted(skv.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_sizes():
    assert skv.plan_words(16, 2, 256) == 129
    assert skv.plan_words(128, 8, 256) == 129
    assert skv.plan_words(2, 2, 256) == 129
    assert skv.plan_words(300, 1, 256) == 301
    assert skv.plan_words(0, 2, 256) == 0
    assert skv.workspace_bytes(64, 32, 128, 64) == 64 * 32 * 64 * (128 + 1) * 4
    assert skv.workspace_bytes(0, 32, 128, 64) == 0


def test_strerror():
    assert skv.strerror(0) == "ok"
    assert skv.strerror(1) == "invalid argument"
    assert skv.strerror(2) == "unsupported geometry or type"
    assert skv.strerror(3) == "kernel launch failed"
    assert skv.strerror(99) == "unknown status"


def _plan(**kw):
    a = dict(seq_lens=P, cu=P, bs=2, total_q=2, kv_heads=2, page_size=16, num_cus=256,
             seg_max=64, causal=1, plan=P, tok=P)
    a.update(kw)
    return skv.load().skv_plan_build(a["seq_lens"], a["cu"], a["bs"], a["total_q"],
                                     a["kv_heads"], a["page_size"], a["num_cus"],
                                     a["seg_max"], a["causal"], a["plan"], a["tok"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(seq_lens=None), 1), (dict(cu=None), 1), (dict(plan=None), 1), (dict(tok=None), 1),
    (dict(bs=0), 1), (dict(bs=32768), 1), (dict(total_q=0), 1), (dict(kv_heads=0), 1),
    (dict(num_cus=0), 1), (dict(seg_max=0), 1), (dict(seg_max=65536), 1),
    (dict(page_size=64), 2), (dict(page_size=8), 2),
])
def test_plan_build_errors(kw, code):
    assert _plan(**kw) == code


def _attn(**kw):
    a = dict(q=P, kv_a=P, kv_b=None, layout=0, kv_dtype=0, pt=P, pt_stride=8, seq_lens=P,
             cu=P, bs=2, total_q=2, max_q=1, q_heads=8, kv_heads=2, head_dim=128,
             page_size=16, k_scale=None, v_scale=None, causal=1, plan=P, tok=P,
             num_cus=256, seg_max=64, part_o=P, part_lse=P, out=P, out_lse=None, flags=0)
    a.update(kw)
    return skv.load().skv_paged_decode_attn(
        a["q"], a["kv_a"], a["kv_b"], a["layout"], a["kv_dtype"], a["pt"], a["pt_stride"],
        a["seq_lens"], a["cu"], a["bs"], a["total_q"], a["max_q"], a["q_heads"],
        a["kv_heads"], a["head_dim"], a["page_size"], a["k_scale"], a["v_scale"],
        a["causal"], a["plan"], a["tok"], a["num_cus"], a["seg_max"], a["part_o"],
        a["part_lse"], a["out"], a["out_lse"], a["flags"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(kv_a=None), 1), (dict(pt=None), 1),
    (dict(tok=None), 1), (dict(part_o=None), 1), (dict(part_lse=None), 1), (dict(out=None), 1),
    (dict(plan=None, tok=None), 1),                       # the fixed split writes tok_nseg
    (dict(plan=None, head_dim=96), 2),
    (dict(seq_lens=None), 1), (dict(cu=None), 1),
    (dict(layout=2), 1), (dict(kv_dtype=3), 1), (dict(kv_dtype=-1), 1),
    (dict(layout=1), 1),                                  # shuffled needs the V plane
    (dict(kv_b=P), 1),                                    # standard takes no V plane
    (dict(kv_dtype=1), 1),                                # fp8 needs scales
    (dict(k_scale=P, v_scale=P), 1),                      # bf16 takes none
    (dict(kv_dtype=1, k_scale=P), 1),
    (dict(kv_dtype=2, k_scale=P, v_scale=P), 1),          # fp16 takes none
    (dict(q_heads=12, kv_heads=8), 1), (dict(bs=0), 1), (dict(bs=40000), 1),
    (dict(total_q=0), 1), (dict(max_q=0), 1), (dict(seg_max=0), 1), (dict(seg_max=70000), 1),
    (dict(pt_stride=0), 1), (dict(num_cus=0), 1), (dict(kv_heads=0), 1),
    (dict(head_dim=96), 2), (dict(head_dim=512), 2), (dict(head_dim=32), 2),
    (dict(page_size=64), 2), (dict(page_size=24), 2), (dict(max_q=5), 2),
    (dict(q_heads=32, kv_heads=2, max_q=8), 2),           # rows 128 > 64 (max_q checked first)
    (dict(q_heads=64, kv_heads=2, max_q=3), 2),           # rows 96 > 64
    (dict(flags=4), 1), (dict(flags=-1), 1), (dict(flags=3), 1),   # 3: both flags at once
])
def test_attn_errors(kw, code):
    assert _attn(**kw) == code


@pytest.mark.parametrize("flags,code", [(3, 1), (-1, 1), (4, 1), (1 << 30, 1)])
def test_segment_attn_flag_errors(flags, code):
    st = skv.load().skv_segment_attn(P, P, None, 0, 0, P, 8, P, P, 2, 2, 1, 8, 2, 128, 16, None,
                                     None, 1, P, P, 256, 64, P, P, flags, None)
    assert st == code


def _reduce(**kw):
    a = dict(po=P, pl=P, tok=P, total_q=2, q_heads=8, head_dim=128, seg_max=64, odt=0, out=P)
    a.update(kw)
    return skv.load().skv_split_reduce(a["po"], a["pl"], a["tok"], a["total_q"], a["q_heads"],
                                       a["head_dim"], a["seg_max"], a["odt"], a["out"], None,
                                       None)


@pytest.mark.parametrize("kw,code", [
    (dict(po=None), 1), (dict(pl=None), 1), (dict(tok=None), 1), (dict(out=None), 1),
    (dict(total_q=0), 1), (dict(q_heads=0), 1), (dict(seg_max=0), 1), (dict(seg_max=65536), 1),
    (dict(head_dim=96), 2), (dict(head_dim=512), 2), (dict(odt=1), 1), (dict(odt=3), 1), (dict(odt=-1), 1),
])
def test_reduce_errors(kw, code):
    assert _reduce(**kw) == code


def _shuffle(**kw):
    a = dict(src=P, k=P, v=P, ids=None, nb=4, h=2, ps=16, hd=128, e=2)
    a.update(kw)
    return skv.load().skv_kv_page_shuffle(a["src"], a["k"], a["v"], a["ids"], a["nb"], a["h"],
                                          a["ps"], a["hd"], a["e"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(src=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(nb=0), 1), (dict(h=0), 1),
    (dict(hd=96), 2), (dict(hd=512), 2), (dict(ps=64), 2), (dict(ps=8), 2), (dict(e=4), 2),
])
def test_shuffle_errors(kw, code):
    assert _shuffle(**kw) == code


def _convert(**kw):
    a = dict(k=P, v=P, ids=None, nb=4, h=2, ps=16, hd=128, e=2, d=0)
    a.update(kw)
    return skv.load().skv_kv_page_convert(a["k"], a["v"], a["ids"], a["nb"], a["h"], a["ps"],
                                          a["hd"], a["e"], a["d"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(k=None), 1), (dict(v=None), 1), (dict(nb=0), 1), (dict(h=0), 1), (dict(d=2), 1),
    (dict(d=-1), 1), (dict(hd=96), 2), (dict(hd=512), 2), (dict(ps=64), 2), (dict(e=4), 2),
    (dict(h=17), 2), (dict(h=33, e=1), 2),               # block above 128 KiB
    (dict(h=9, ps=32), 2), (dict(h=17, ps=32, e=1), 2),
    (dict(h=9, hd=256), 2), (dict(h=33, hd=64), 2),      # the same bound at head dims 256 and 64
])
def test_convert_errors(kw, code):
    assert _convert(**kw) == code


def _unshuffle(**kw):
    a = dict(k=P, v=P, dst=P, ids=None, nb=4, h=2, ps=16, hd=128, e=2)
    a.update(kw)
    return skv.load().skv_kv_page_unshuffle(a["k"], a["v"], a["dst"], a["ids"], a["nb"], a["h"],
                                            a["ps"], a["hd"], a["e"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dst=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(nb=0), 1), (dict(h=0), 1),
    (dict(hd=96), 2), (dict(hd=512), 2), (dict(ps=64), 2), (dict(e=4), 2),
])
def test_unshuffle_errors(kw, code):
    assert _unshuffle(**kw) == code


def _write(**kw):
    a = dict(k=P, v=P, slots=P, T=4, ks=256, vs=256, kp=P, vp=P, nb=8, h=2, ps=16, hd=128, e=2,
             ksc=None, vsc=None)
    a.update(kw)
    return skv.load().skv_kv_cache_write(a["k"], a["v"], a["slots"], a["T"], a["ks"], a["vs"],
                                         a["kp"], a["vp"], a["nb"], a["h"], a["ps"], a["hd"],
                                         a["e"], a["ksc"], a["vsc"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(k=None), 1), (dict(v=None), 1), (dict(slots=None), 1), (dict(kp=None), 1),
    (dict(vp=None), 1), (dict(T=0), 1), (dict(nb=0), 1), (dict(h=0), 1),
    (dict(ks=255), 1), (dict(vs=128), 1), (dict(ks=260), 1),       # below H*D / not a multiple of x
    (dict(hd=96), 2), (dict(hd=512), 2), (dict(ps=64), 2), (dict(e=4), 2),
    (dict(ksc=P), 1), (dict(vsc=P), 1),                  # one scale without the other
    (dict(ksc=P, vsc=P), 1),                              # quantising needs an fp8 cache
    (dict(ksc=P, vsc=P, e=1, ks=260), 1),                 # bf16 input rows: multiple of 8
])
def test_cache_write_errors(kw, code):
    assert _write(**kw) == code


def test_python_binding_raises_on_error_status():
    with pytest.raises(_lib.SkvError) as ei:
        _lib._check(2, "x")
    assert ei.value.status == 2


def _static(**kw):
    a = dict(q=P, kv_a=P, kv_b=None, layout=0, dtype=0, pt=P, pt_stride=8, sl=P, cu=P, bs=2,
             total_q=2, max_q=1, q_heads=8, kv_heads=2, head_dim=128, page_size=16,
             ks=None, vs=None, causal=1, plan=P, tok=P, num_cus=256, seg_max=64, out=P,
             out_lse=None, flags=0)
    a.update(kw)
    return skv.load().skv_paged_decode_attn_static(
        a["q"], a["kv_a"], a["kv_b"], a["layout"], a["dtype"], a["pt"], a["pt_stride"], a["sl"],
        a["cu"], a["bs"], a["total_q"], a["max_q"], a["q_heads"], a["kv_heads"], a["head_dim"],
        a["page_size"], a["ks"], a["vs"], a["causal"], a["plan"], a["tok"], a["num_cus"],
        a["seg_max"], a["out"], a["out_lse"], a["flags"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(out=None), 1), (dict(tok=None), 1), (dict(kv_b=P), 1),
    (dict(flags=3), 1), (dict(head_dim=96), 2), (dict(max_q=5), 2),
    # partials beyond the library's 64 MiB array: 64 x 32 x 64 x (128 + 1) x 4 B
    (dict(total_q=64, q_heads=32, max_q=4, seg_max=64), 2),
    (dict(total_q=8, q_heads=16, head_dim=256, seg_max=65535), 2),
])
def test_static_attn_errors(kw, code):
    """Rejected on the host, before the device array is looked up."""
    assert _static(**kw) == code


def test_static_scratch_size_matches_header():
    text = open(HEADER).read()
    assert "#define SKV_STATIC_SCRATCH_BYTES (64u << 20)" in text
    assert skv.STATIC_SCRATCH_BYTES == 64 << 20


def _check_inputs(**kw):
    a = dict(pt=P, pt_stride=8, sl=P, cu=P, bs=2, total_q=2, max_q=4, page_size=16, nb=64,
             res=P)
    a.update(kw)
    return skv.load().skv_check_inputs(a["pt"], a["pt_stride"], a["sl"], a["cu"], a["bs"],
                                       a["total_q"], a["max_q"], a["page_size"], a["nb"],
                                       a["res"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(pt=None), 1), (dict(sl=None), 1), (dict(cu=None), 1), (dict(res=None), 1),
    (dict(bs=0), 1), (dict(bs=32768), 1), (dict(total_q=0), 1), (dict(max_q=0), 1),
    (dict(pt_stride=0), 1), (dict(nb=0), 1), (dict(page_size=64), 2),
])
def test_check_inputs_errors(kw, code):
    assert _check_inputs(**kw) == code


def test_contract_bits_match_header():
    text = open(HEADER).read()
    for name, bit in (("LEN_NEGATIVE", 1), ("LEN_TABLE", 2), ("CU", 4), ("QLEN", 8),
                      ("PAGE_ID", 16)):
        assert re.search(rf"SKV_BAD_{name} = {bit}\b", text), name
    assert sorted(skv.CONTRACT_BITS.values()) == [1, 2, 4, 8, 16]
