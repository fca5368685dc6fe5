"""CPU tests of the libgdn boundary: the library loads and exports every
entry point include/gdn.h declares, the ctypes mirror matches the C struct
layouts, page layouts follow their definition, and host-side validation
answers with the documented status codes before anything is launched
(no GPU is touched by any call made here)."""
import ctypes
import os
import re
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")
FAKE = 0x10000  # a non-null, 256-aligned address: validation never dereferences it


@pytest.fixture(scope="module")
def L():
    import linear_attention_ssm_gdn_amd._lib as lib
    if not os.path.exists(lib.LIB_PATH):
        pytest.skip("libgdn.so not built")
    return lib


@pytest.fixture(scope="module")
def so(L):
    return L.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


def test_header_compiles_as_plain_c(tmp_path):
    src = tmp_path / "h.c"
    src.write_text('#include "gdn.h"\nint main(void) { return GDN_ABI_VERSION == 2 ? 0 : 1; }\n')
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.dirname(HEADER),
                    str(src), "-o", str(tmp_path / "h")], check=True)
    subprocess.run([str(tmp_path / "h")], check=True)


def test_every_declared_symbol_is_exported(so):
    names = declared_functions()
    assert set(names) == {"gdn_abi_version", "gdn_status_str", "gdn_spec_page_layout",
                          "gdn_chunked_workspace_bytes", "gdn_conv_update", "gdn_recurrent_seq",
                          "gdn_chunked_prefill", "gdn_prefill_path", "gdn_prefill", "gdn_spec_verify",
                          "gdn_spec_verify_cached", "gdn_prefix_restore", "gdn_mixed_step",
                          "gdn_recurrent_seq_noalloc", "gdn_mixed_launches", "gdn_mixed_step_launches"}
    for n in names:
        assert hasattr(so, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", os.path.join(ROOT, "linear_attention_ssm_gdn_amd",
                                                                       "libgdn.so")],
                         capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.split()[-1].startswith("gdn_")}
    assert exported == set(names)


def test_struct_layouts_match_c(L, tmp_path):
    structs = {"gdn_dims": L.GdnDims, "gdn_params": L.GdnParams, "gdn_batch": L.GdnBatch,
               "gdn_conv_pool": L.GdnConvPool, "gdn_state_pool": L.GdnStatePool,
               "gdn_spec_layout": L.GdnSpecLayout, "gdn_seq_part": L.GdnSeqPart,
               "gdn_verify_part": L.GdnVerifyPart, "gdn_prefix_cache": L.GdnPrefixCache}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "gdn.h"', 'int main(void) {']
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'  printf("{cname}.{f} %zu\\n", offsetof({cname}, {f}));')
    lines.append('  printf("gdn_spec_header %zu\\n", sizeof(gdn_spec_header));')
    lines.append("  return 0; }")
    (tmp_path / "l.c").write_text("\n".join(lines))
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(tmp_path / "l.c"), "-o",
                    str(tmp_path / "l")], check=True)
    got = dict(l.rsplit(" ", 1) for l in subprocess.run([str(tmp_path / "l")], capture_output=True, text=True,
                                                          check=True).stdout.splitlines())
    for cname, py in structs.items():
        assert int(got[cname]) == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert int(got[f"{cname}.{f}"]) == getattr(py, f).offset, (cname, f)
    assert int(got["gdn_spec_header"]) == 256


def test_version_and_status_strings(so, L):
    assert so.gdn_abi_version() == L.ABI_VERSION == 2
    for code, text in ((0, b"ok"), (1, b"invalid argument"), (2, b"unsupported configuration"),
                       (3, b"kernel launch failed"), (99, b"unknown status")):
        assert so.gdn_status_str(code) == text


def _dims(L, **kw):
    d = dict(h_k=16, h_v=32, d_k=128, d_v=128, conv_w=4, n_spec=7, act_dtype=1, state_dtype=0, scale=1.0,
             l2_eps=1e-6)
    d.update(kw)
    return L.GdnDims(**d)


def test_spec_page_layout_definition(so, L):
    for sd, es in ((0, 4), (1, 2)):
        d = _dims(L, state_dtype=sd)
        one, slots = L.GdnSpecLayout(), L.GdnSpecLayout()
        assert so.gdn_spec_page_layout(ctypes.byref(d), 0, ctypes.byref(one)) == 0
        assert so.gdn_spec_page_layout(ctypes.byref(d), 1, ctypes.byref(slots)) == 0
        head = 128 * 128 * es
        C = 2 * 16 * 128 + 32 * 128
        assert one.header_off == 0 and one.state_off == 256
        assert one.record_row_bytes == (C + 2 * 32) * 4
        assert one.record_off == 256 + 32 * head
        assert one.page_bytes == ((one.record_off + 2 * 8 * one.record_row_bytes + 255) // 256) * 256
        assert slots.state_off == 256 and slots.page_bytes == 256 + 8 * 32 * head
        # the one-page layout is the smaller one (fp32: 2.5 MiB vs 16 MiB per request)
        assert slots.page_bytes / one.page_bytes > (5.0 if sd == 1 else 6.0)
    bad = _dims(L, n_spec=16)
    assert so.gdn_spec_page_layout(ctypes.byref(bad), 0, ctypes.byref(L.GdnSpecLayout())) == 2
    assert so.gdn_spec_page_layout(ctypes.byref(_dims(L)), 5, ctypes.byref(L.GdnSpecLayout())) == 1


def _seq_args(L, d, **over):
    C = 2 * d.h_k * d.d_k + d.h_v * d.d_v
    batch = L.GdnBatch(FAKE, FAKE, None, 2, 8, 16)
    conv = L.GdnConvPool(FAKE, 3 * C, 3, 4, FAKE)
    state = L.GdnStatePool(FAKE, d.h_v * d.d_k * d.d_v, 4)
    params = L.GdnParams(FAKE, FAKE, FAKE)
    a = dict(dims=d, params=params, x=FAKE, x_stride=C, a=FAKE, b=FAKE, ab_stride=d.h_v, batch=batch, conv=conv,
             state=state, o=FAKE)
    a.update(over)
    return a


def _call_seq(so, a):
    return so.gdn_recurrent_seq(ctypes.byref(a["dims"]), ctypes.byref(a["params"]) if a["params"] else None,
                                a["x"], a["x_stride"], a["a"], a["b"], a["ab_stride"],
                                ctypes.byref(a["batch"]) if a["batch"] else None, a["conv"], a["state"], a["o"],
                                None, None)


def test_recurrent_seq_validation(so, L):
    d = _dims(L)
    C = 2 * 16 * 128 + 32 * 128
    cases = [
        (dict(params=None), 1),
        (dict(batch=None), 1),
        (dict(x=None), 1),
        (dict(x_stride=C - 1), 1),
        (dict(ab_stride=31), 1),
        (dict(conv=L.GdnConvPool(FAKE, 3 * C, 2, 4, FAKE)), 1),      # fewer than W-1 window rows
        (dict(conv=L.GdnConvPool(FAKE, 3 * C, 3, 4, None)), 1),      # no sync words
        (dict(conv=L.GdnConvPool(FAKE, 3 * C - 1, 3, 4, FAKE)), 1),  # page stride too small
        (dict(state=L.GdnStatePool(FAKE + 4, 32 * 128 * 128, 4)), 1),  # misaligned state base
        (dict(state=L.GdnStatePool(FAKE, 32 * 128 * 128 - 1, 4)), 1),
        (dict(dims=_dims(L, h_v=24)), 1),                            # h_v % h_k != 0
        (dict(dims=_dims(L, l2_eps=-1.0)), 1),
        (dict(dims=_dims(L, act_dtype=7)), 1),
        (dict(dims=_dims(L, conv_w=3)), 2),
        (dict(dims=_dims(L, d_k=96)), 2),
        (dict(dims=_dims(L, d_v=100)), 2),
    ]
    for over, want in cases:
        assert _call_seq(so, _seq_args(L, d, **over)) == want, over
    # an empty batch is a no-op that returns OK without launching
    assert _call_seq(so, _seq_args(L, d, batch=L.GdnBatch(None, None, None, 0, 0, 0))) == 0


def test_recurrent_seq_noalloc_validation(so, L):
    """The entry point that keeps its sync words in the library's own array
    validates like gdn_recurrent_seq, needs no conv.sync, and refuses a conv
    pool whose sync words (n_pages * h_k + 1) exceed its maximum before
    touching the device."""
    d = _dims(L)
    C = 2 * 16 * 128 + 32 * 128

    def call(**over):
        a = _seq_args(L, d, **over)
        return so.gdn_recurrent_seq_noalloc(ctypes.byref(a["dims"]), ctypes.byref(a["params"]) if a["params"] else None,
                                            a["x"], a["x_stride"], a["a"], a["b"], a["ab_stride"],
                                            ctypes.byref(a["batch"]) if a["batch"] else None, a["conv"], a["state"],
                                            a["o"], None, None)
    assert call(x=None) == 1
    assert call(params=None) == 1
    assert call(conv=L.GdnConvPool(FAKE, 3 * C, 2, 4, None)) == 1
    max_pages = (L.GDN_NOALLOC_SYNC_WORDS - 1) // 16
    assert call(conv=L.GdnConvPool(FAKE, 3 * C, 3, max_pages + 1, None)) == 1
    assert call(conv=L.GdnConvPool(FAKE, 3 * C, 3, 1 << 20, None)) == 1
    assert call(batch=L.GdnBatch(None, None, None, 0, 0, 0)) == 0
    assert "#define GDN_NOALLOC_SYNC_WORDS %d" % L.GDN_NOALLOC_SYNC_WORDS in open(HEADER).read()


def test_chunked_validation(so, L):
    d = _dims(L)
    a = _seq_args(L, d)

    def call(chunk=64, ws=None, ws_bytes=0, dims=d, x=a["x"], x_stride=a["x_stride"], conv=a["conv"], o=a["o"]):
        return so.gdn_chunked_prefill(ctypes.byref(dims), ctypes.byref(a["params"]), x, x_stride, a["a"],
                                      a["b"], a["ab_stride"], ctypes.byref(a["batch"]), conv, a["state"],
                                      o, chunk, ws, ws_bytes, None, None)
    assert call(chunk=0) == 1
    assert call(chunk=32) == 2
    assert call(dims=_dims(L, d_k=64)) == 2
    # rows are read as 16-byte vectors: 8 bf16 (or 4 fp32) elements
    C = a["x_stride"]
    assert call(x=FAKE + 2) == 1
    assert call(x_stride=C + 4) == 1
    assert call(conv=L.GdnConvPool(FAKE + 8, 3 * C, 3, 4, FAKE)) == 1
    assert call(conv=L.GdnConvPool(FAKE, 3 * C + 4, 3, 4, FAKE)) == 1
    assert call(o=FAKE + 4) == 1
    assert call(x_stride=(1 << 24) + 8) == 1  # a chunk's rows are addressed with 32-bit offsets
    # the workspace: one slot of records per sequence plus one per 64 rows
    def ws(n_seqs, n_rows, dims=d):
        out = ctypes.c_size_t(123)
        assert so.gdn_chunked_workspace_bytes(ctypes.byref(dims), n_seqs, n_rows, 64, ctypes.byref(out)) == 0
        return out.value
    slot = ws(1, 0)
    assert slot > 0 and slot % 256 == 0
    assert ws(4, 32768) == (4 + 512) * slot
    assert ws(2, 16) == 3 * slot and ws(2, 129) == 5 * slot and ws(0, 0) == 0
    # key-head and value-head records both count
    assert ws(1, 0, _dims(L, h_v=16)) < slot and ws(1, 0, _dims(L, h_k=8)) < slot
    out = ctypes.c_size_t(0)
    assert so.gdn_chunked_workspace_bytes(ctypes.byref(d), -1, 16, 64, ctypes.byref(out)) == 1
    assert so.gdn_chunked_workspace_bytes(ctypes.byref(d), 2, 16, 32, ctypes.byref(out)) == 2
    # the batch of _seq_args (2 sequences, 16 rows) needs three slots: short,
    # missing or misaligned workspaces are argument errors
    need = ws(2, 16)
    assert call(ws=None, ws_bytes=need) == 1
    assert call(ws=FAKE, ws_bytes=need - 1) == 1
    assert call(ws=FAKE + 16, ws_bytes=need) == 1


def test_prefill_path_selection(so, L):
    """Host-side choice between the token-by-token and chunked paths: the
    measured default break-even (32 rows for 1-2 sequences, 16 for 3-8, 8 for
    more), an explicit token_max, max_seqlen unknown (n_rows stands in), and
    head dims the chunked kernel is not compiled for."""
    def path(dims, n_seqs, max_seqlen, token_max=-1, n_rows=None):
        b = L.GdnBatch(FAKE, FAKE, None, n_seqs, max_seqlen, n_rows if n_rows is not None else n_seqs * max_seqlen)
        out = ctypes.c_int32(-7)
        assert so.gdn_prefill_path(ctypes.byref(dims), ctypes.byref(b), token_max, ctypes.byref(out)) == 0
        return out.value
    d = _dims(L)
    T, K = L.GDN_PATH_TOKEN, L.GDN_PATH_CHUNKED
    for n in (1, 2):
        assert path(d, n, 1) == T and path(d, n, 32) == T and path(d, n, 33) == K
    for n in (3, 4, 5, 8):
        assert path(d, n, 16) == T and path(d, n, 17) == K and path(d, n, 8192) == K
    for n in (9, 16, 64):
        assert path(d, n, 8) == T and path(d, n, 9) == K and path(d, n, 8192) == K
    assert path(d, 8, 4096, token_max=2 ** 31 - 1) == T
    assert path(d, 1, 1, token_max=0) == K
    assert path(d, 1, 100, token_max=100) == T and path(d, 1, 101, token_max=100) == K
    assert path(d, 4, 0, n_rows=40) == K and path(d, 4, 0, n_rows=16) == T
    assert path(d, 0, 0, n_rows=0) == T
    assert path(_dims(L, d_k=64), 1, 4096) == T        # no chunked kernel for d_k = 64
    assert path(_dims(L, d_v=96), 1, 4096) == T        # nor for d_v % 64 != 0
    b = L.GdnBatch(FAKE, FAKE, None, 1, 8, 8)
    assert so.gdn_prefill_path(ctypes.byref(d), ctypes.byref(b), -1, None) == 1
    assert so.gdn_prefill_path(ctypes.byref(_dims(L, conv_w=3)), ctypes.byref(b), -1,
                               ctypes.byref(ctypes.c_int32())) == 2


def test_prefill_validation(so, L):
    """gdn_prefill validates as the path it selects: the chunked path's
    16-byte alignment applies only to batches that take it."""
    d = _dims(L)
    a = _seq_args(L, d)

    def call(max_seqlen, x=a["x"], token_max=-1, params=a["params"]):
        b = L.GdnBatch(FAKE, FAKE, None, 2, max_seqlen, 2 * max_seqlen)
        p = ctypes.c_int32(-7)
        st = so.gdn_prefill(ctypes.byref(d), ctypes.byref(params) if params is not None else None, x,
                            a["x_stride"], a["a"], a["b"], a["ab_stride"], ctypes.byref(b), a["conv"], a["state"],
                            a["o"], token_max, None, 0, ctypes.byref(p), None, None)
        return st, p.value
    assert call(4096, x=FAKE + 2)[0] == 1                     # chunked: x must be 16-byte aligned
    assert call(4096, x=None)[0] == 1
    assert call(8, params=None)[0] == 1
    assert call(4096, x=None, token_max=2 ** 31 - 1)[0] == 1       # token path: its own checks
    b0 = L.GdnBatch(None, None, None, 0, 0, 0)
    p = ctypes.c_int32(-7)
    assert so.gdn_prefill(ctypes.byref(d), ctypes.byref(a["params"]), None, a["x_stride"], None, None,
                          a["ab_stride"], ctypes.byref(b0), a["conv"], a["state"], None, -1, None, 0,
                          ctypes.byref(p), None, None) == 0
    assert p.value == L.GDN_PATH_TOKEN


def test_verify_validation(so, L):
    d = _dims(L)
    C = 2 * 16 * 128 + 32 * 128
    lay = L.GdnSpecLayout()
    assert so.gdn_spec_page_layout(ctypes.byref(d), 0, ctypes.byref(lay)) == 0
    params = L.GdnParams(FAKE, FAKE, FAKE)

    def call(layout=0, n_req=2, n_cand=8, pages=FAKE, page_bytes=None, conv_rows=10, x=FAKE, dims=d):
        conv = L.GdnConvPool(FAKE, conv_rows * C, conv_rows, 4, FAKE)
        return so.gdn_spec_verify(ctypes.byref(dims), ctypes.byref(params), layout, x, C, FAKE, FAKE, 32, n_req,
                                  n_cand, FAKE, FAKE, FAKE, pages, page_bytes or lay.page_bytes, 4, conv, FAKE, None,
                                  None)
    assert call(n_cand=9) == 1                       # more than n_spec + 1 candidates
    assert call(conv_rows=9) == 1                    # conv buffer narrower than W-1+n_spec rows
    assert call(page_bytes=lay.page_bytes - 256) == 1
    assert call(pages=FAKE + 16) == 1                # pages not 256-aligned
    assert call(layout=3) == 1
    assert call(x=None) == 1
    assert call(n_req=0) == 0                        # nothing to do


def test_mixed_step_validation(so, L):
    """Each part of a mixed step is validated as its stand-alone entry point;
    absent or empty parts are allowed and an empty step launches nothing."""
    d = _dims(L)
    C = 2 * 16 * 128 + 32 * 128
    lay = L.GdnSpecLayout()
    assert so.gdn_spec_page_layout(ctypes.byref(d), 0, ctypes.byref(lay)) == 0
    params = L.GdnParams(FAKE, FAKE, FAKE)
    sa = _seq_args(L, d)

    def seq_part(x=FAKE, batch=None, rows=3):
        b = batch or L.GdnBatch(FAKE, FAKE, None, 2, 8, 16)
        return L.GdnSeqPart(x, C, FAKE, FAKE, 32, ctypes.pointer(b), L.GdnConvPool(FAKE, rows * C, rows, 4, FAKE),
                            sa["state"], FAKE)

    def ver_part(n_req=2, n_cand=8, layout=0, rows=10, pages=FAKE):
        return L.GdnVerifyPart(layout, FAKE, C, FAKE, FAKE, 32, n_req, n_cand, FAKE, FAKE, FAKE, pages,
                               lay.page_bytes, 4, L.GdnConvPool(FAKE, rows * C, rows, 4, FAKE), FAKE)

    def call(seq=None, ver=None, p=params, dims=d):
        return so.gdn_mixed_step(ctypes.byref(dims), ctypes.byref(p) if p is not None else None,
                                 ctypes.byref(seq) if seq is not None else None,
                                 ctypes.byref(ver) if ver is not None else None, None, None)
    assert call() == 0                                           # nothing to do
    empty = L.GdnBatch(None, None, None, 0, 0, 0)
    assert call(seq=seq_part(batch=empty), ver=ver_part(n_req=0)) == 0
    assert call(seq=seq_part(), p=None) == 1
    assert call(seq=seq_part(x=None), ver=ver_part(n_req=0)) == 1
    assert call(seq=seq_part(rows=2), ver=ver_part(n_req=0)) == 1   # window narrower than W-1 rows
    assert call(seq=seq_part(batch=empty), ver=ver_part(rows=9)) == 1  # buffer narrower than W-1+n_spec
    assert call(seq=seq_part(batch=empty), ver=ver_part(n_cand=9)) == 1
    assert call(seq=seq_part(batch=empty), ver=ver_part(layout=2)) == 1
    assert call(ver=ver_part(pages=FAKE + 16)) == 1
    assert call(seq=seq_part(), dims=_dims(L, d_k=96)) == 2
    sp = seq_part(batch=empty)
    for pages, nbytes in ((FAKE + 64, 1024), (FAKE, 1000), (FAKE, 0)):
        sp.spec_pages, sp.spec_page_bytes, sp.spec_n_pages = pages, nbytes, 4
        assert call(seq=sp) == 1, (pages, nbytes)
    sp.spec_pages, sp.spec_page_bytes = FAKE, lay.page_bytes
    assert call(seq=sp) == 0                                     # empty batch: validated, nothing launched


def test_mixed_step_launch_count(so, L):
    """gdn_mixed_launches: two launches exactly when both parts are non-empty,
    every sequence has 1-4 rows, no speculative pages are written and d_v is
    a multiple of 64 (the short-sequence kernel's shapes); gdn_mixed_step_launches
    takes AUTO, ONE or TWO and rejects anything else before launching."""
    C = 2 * 16 * 128 + 32 * 128
    lay = L.GdnSpecLayout()
    d = _dims(L)
    assert so.gdn_spec_page_layout(ctypes.byref(d), 0, ctypes.byref(lay)) == 0
    sa = _seq_args(L, d)

    def seq_part(max_seqlen, n_seqs=2, spec=False):
        b = L.GdnBatch(FAKE, FAKE, None, n_seqs, max_seqlen, 4 * max(n_seqs, 1))
        sp = L.GdnSeqPart(FAKE, C, FAKE, FAKE, 32, ctypes.pointer(b), L.GdnConvPool(FAKE, 10 * C, 10, 4, FAKE),
                          sa["state"], FAKE)
        sp._batch = b
        if spec:
            sp.spec_pages, sp.spec_page_bytes, sp.spec_n_pages = FAKE, lay.page_bytes, 4
        return sp

    def ver_part(n_req=2):
        return L.GdnVerifyPart(0, FAKE, C, FAKE, FAKE, 32, n_req, 8, FAKE, FAKE, FAKE, FAKE, lay.page_bytes, 4,
                               L.GdnConvPool(FAKE, 10 * C, 10, 4, FAKE), FAKE)

    def launches(seq=None, ver=None, dims=d):
        out = ctypes.c_int32(-1)
        st = so.gdn_mixed_launches(ctypes.byref(dims), ctypes.byref(seq) if seq is not None else None,
                                   ctypes.byref(ver) if ver is not None else None, ctypes.byref(out))
        assert st == 0
        return out.value
    ONE, TWO = L.GDN_MIXED_ONE_LAUNCH, L.GDN_MIXED_TWO_LAUNCHES
    for m in (1, 2, 3, 4):
        assert launches(seq_part(m), ver_part()) == TWO, m
    assert launches(seq_part(5), ver_part()) == ONE
    assert launches(seq_part(0), ver_part()) == ONE                # longest length not given
    assert launches(seq_part(1, spec=True), ver_part()) == ONE     # the prefill writes page headers
    assert launches(seq_part(1), ver_part(n_req=0)) == ONE
    assert launches(seq_part(1, n_seqs=0), ver_part()) == ONE
    assert launches(seq_part(1)) == ONE
    assert launches(None, ver_part()) == ONE
    assert launches(seq_part(1), ver_part(), dims=_dims(L, d_v=96)) == ONE
    d96 = _dims(L)
    assert so.gdn_mixed_launches(ctypes.byref(d96), None, None, None) == 1
    params = L.GdnParams(FAKE, FAKE, FAKE)
    for bad in (-1, 3):
        assert so.gdn_mixed_step_launches(ctypes.byref(d), ctypes.byref(params), None, None, bad, None, None) == 1
    for ok in (0, 1, 2):
        assert so.gdn_mixed_step_launches(ctypes.byref(d), ctypes.byref(params), None, None, ok, None, None) == 0


def test_conv_update_validation(so, L):
    d = _dims(L)
    C = 2 * 16 * 128 + 32 * 128
    batch = L.GdnBatch(FAKE, FAKE, None, 2, 8, 16)

    def call(act=1, y_dtype=0, y_stride=C, rows=3):
        conv = L.GdnConvPool(FAKE, rows * C, rows, 4, None)
        return so.gdn_conv_update(ctypes.byref(d), FAKE, FAKE, C, ctypes.byref(batch), conv, act, FAKE, y_dtype,
                                  y_stride, None, None)
    assert call(act=2) == 1
    assert call(y_dtype=5) == 1
    assert call(y_stride=C - 8) == 1
    assert call(rows=2) == 1


def test_missing_library_fails_loudly(tmp_path):
    code = textwrap.dedent(f"""
        import sys; sys.path.insert(0, {ROOT!r})
        import linear_attention_ssm_gdn_amd._lib as L
        L.LIB_PATH = {str(tmp_path / 'absent.so')!r}
        try:
            L.load()
        except ImportError as e:
            print('raised', e)
            sys.exit(0)
        sys.exit(1)
    """)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "not built" in r.stdout
