"""The C-ABI library loads without a GPU, exports every entry point that
include/*.h declares, and rejects bad arguments on the host before any HIP
call (so no compute runs here)."""
import glob
import os
import re

import pytest

from gated_causal_attention_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
S = binding.Status
FAKE = 1 << 20  # a non-null, aligned address; never dereferenced by these calls


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)
    return sorted({n for n in names if n.startswith("resolvent_")})


def test_library_exports_every_declared_symbol():
    lib = binding._load()
    names = declared_functions()
    assert "resolvent_forward" in names and len(names) >= 3
    for name in names:
        assert hasattr(lib, name), name


def call(B=1, H=1, n=128, d=64, beta=1.0, qk=1.0, g=1.0, qdt=0, vdt=0, ws_bytes=None,
         ptr=FAKE, ws=FAKE, status=FAKE):
    lib = binding._load()
    if ws_bytes is None:
        ws_bytes = lib.resolvent_workspace_bytes(max(B, 1), max(H, 1), max(n, 1), max(d, 64),
                                                 qdt, vdt)
    return lib.resolvent_forward(ptr, ptr, ptr, ptr, ptr, beta, qk, g, B, H, n, d, qdt, vdt, ptr,
                                 ptr, ws, ws_bytes, status, None)


def test_shapes_and_empty():
    assert call(B=-1) == S.BAD_SHAPE
    assert call(n=-5) == S.BAD_SHAPE
    assert call(d=-1) == S.BAD_SHAPE
    assert call(n=0) == S.OK  # empty in, empty out: nothing enqueued
    assert call(B=0) == S.OK
    assert call(H=0, ptr=None) == S.OK
    assert call(d=0) == S.BAD_SHAPE  # head_dim = 0 with n > 0


def test_non_finite_switches():
    for bad in (float("nan"), float("inf"), -float("inf")):
        assert call(beta=bad) == S.NONFINITE
        assert call(qk=bad) == S.NONFINITE
        assert call(g=bad) == S.NONFINITE
    assert call(qk=1e300) == S.NONFINITE  # the float32 logit scale overflows


def test_unsupported():
    assert call(d=96) == S.UNSUPPORTED
    assert call(d=256) == S.UNSUPPORTED
    assert call(qdt=1, vdt=0) == S.UNSUPPORTED
    assert call(qdt=7) == S.UNSUPPORTED


def test_bad_pointers_and_workspace():
    assert call(ptr=None) == S.BAD_ARG
    assert call(ws=None) == S.BAD_ARG
    assert call(status=None) == S.BAD_ARG
    assert call(ptr=FAKE + 2) == S.BAD_ARG  # misaligned
    assert call(ws=FAKE + 16) == S.BAD_ARG
    assert call(ws_bytes=100) == S.BAD_ARG


def test_workspace_sizes():
    ws = binding.resolvent_workspace_bytes
    assert ws(0, 1, 10, 64) == 0 and ws(1, 1, 0, 64) == 0
    assert ws(1, 1, 10, 96) == 0
    bq, bk = binding.resolvent_tile_shape()
    assert bq % bk == 0 and bq % 32 == 0 and bk % 32 == 0
    a, b = ws(1, 1, bq, 64), ws(1, 1, bq + 1, 64)  # one more query tile
    assert 0 < a < b
    # values are read where they lie; only fp32 values on the bf16 path need
    # a bf16 copy (n x d_v x 2 bytes per key/value head)
    assert ws(1, 1, bq, 64, binding.F32, binding.F32) <= a
    assert ws(1, 1, bq, 64, binding.BF16, binding.F32) >= a + bq * 64 * 2
    off = binding.resolvent_counters_offset(4, 16, 8192, 128)
    assert 0 < off < ws(4, 16, 8192, 128)
    assert binding.resolvent_counters_offset(1, 1, 0, 64) == 2 ** 64 - 1
    # linear in n: the carried products of the visits are not stored per visit,
    # so a 4x longer sequence needs ~4x the workspace (not ~16x), and the
    # longest accepted sequence stays within a few GB
    s1, s4 = ws(1, 1, 1 << 18, 128), ws(1, 1, 1 << 20, 128)
    assert 3.9 < s4 / s1 < 4.1
    assert ws(1, 1, 1 << 22, 128) < 4 << 30


def test_noalloc_host_checks():
    lib = binding._load()
    assert lib.resolvent_noalloc_scratch_bytes() == 64 << 20

    def na(B=1, H=1, n=128, d=64):
        return lib.resolvent_forward_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 1.0, 1.0, 1.0, B, H,
                                             n, d, 0, 0, FAKE, FAKE, FAKE, None)

    # refused on the host before the scratch array is looked up
    assert lib.resolvent_workspace_bytes(4, 16, 65536, 128, 0, 0) > 64 << 20
    assert na(B=4, H=16, n=65536, d=128) == S.TOO_LARGE
    # fp32 values on the bf16 path add a bf16 copy of V to the workspace
    assert lib.resolvent_workspace_bytes(4, 16, 8192, 128, 0, 1) > 64 << 20
    assert na(B=-1) == S.BAD_SHAPE
    assert na(n=0) == S.OK
    assert na(d=0) == S.BAD_SHAPE
    assert na(d=96) == S.UNSUPPORTED


def test_status_strings():
    for s in S:
        text = binding.resolvent_status_str(int(s))
        assert text and text != "unknown status"
    assert binding.resolvent_status_str(99) == "unknown status"


def chain_call(B=1, H=1, n=128, dv=64, g=1.0, vdt=0, ws_bytes=None, ptr=FAKE, ws=FAKE,
               status=FAKE):
    lib = binding._load()
    if ws_bytes is None:
        ws_bytes = lib.resolvent_chain_workspace_bytes(max(B, 1), max(H, 1), max(n, 1),
                                                       max(dv, 64))
    return lib.resolvent_chain(ptr, ptr, ptr, g, B, H, n, dv, vdt, ptr, ptr, ws, ws_bytes,
                               status, None)


def test_chain_host_checks():
    assert chain_call(B=-1) == S.BAD_SHAPE
    assert chain_call(dv=-64) == S.BAD_SHAPE
    assert chain_call(n=0, ptr=None) == S.OK  # empty in, empty out
    assert chain_call(dv=0) == S.BAD_SHAPE
    for bad in (float("nan"), float("inf")):
        assert chain_call(g=bad) == S.NONFINITE
    assert chain_call(dv=96) == S.UNSUPPORTED
    assert chain_call(dv=8192) == S.UNSUPPORTED
    assert chain_call(vdt=5) == S.UNSUPPORTED
    assert chain_call(ptr=None) == S.BAD_ARG
    assert chain_call(ptr=FAKE + 1) == S.BAD_ARG  # v misaligned for bf16
    assert chain_call(ws=FAKE + 16) == S.BAD_ARG
    assert chain_call(ws_bytes=100) == S.BAD_ARG


def test_chain_workspace_sizes():
    ws = binding.resolvent_chain_workspace_bytes
    assert ws(0, 1, 10, 64) == 0 and ws(1, 1, 10, 96) == 0
    a, b = ws(1, 1, 64, 64), ws(1, 1, 64, 128)
    assert 0 < a < b  # the tile carries grow with the channels
    bq, _ = binding.resolvent_tile_shape()
    assert ws(1, 1, bq + 1, 64) > ws(1, 1, bq, 64)  # sized on n rounded up to bq


def grouped_call(B=1, H=4, Hkv=2, n=128, d=64, dv=128, qdt=0, vdt=0, ws_bytes=None, ptr=FAKE):
    lib = binding._load()
    if ws_bytes is None:
        ws_bytes = lib.resolvent_workspace_bytes_grouped(1, 4, 2, 128, 64, 128, qdt, vdt)
    return lib.resolvent_forward_grouped(ptr, ptr, ptr, ptr, ptr, 1.0, 1.0, 1.0, B, H, Hkv, n,
                                         d, dv, qdt, vdt, ptr, ptr, FAKE, ws_bytes, FAKE, None)


def test_grouped_host_checks():
    assert grouped_call(Hkv=3) == S.BAD_SHAPE  # 4 query heads cannot share 3 k/v heads
    assert grouped_call(Hkv=0) == S.BAD_SHAPE
    assert grouped_call(Hkv=-1) == S.BAD_SHAPE
    assert grouped_call(dv=0) == S.BAD_SHAPE
    assert grouped_call(dv=96) == S.UNSUPPORTED
    assert grouped_call(dv=256) == S.UNSUPPORTED
    assert grouped_call(n=0, ptr=None) == S.OK
    assert grouped_call(ptr=None) == S.BAD_ARG
    assert grouped_call(ws_bytes=64) == S.BAD_ARG
    ws = binding.resolvent_workspace_bytes_grouped
    assert ws(1, 4, 3, 128, 64, 64) == 0 and ws(1, 4, 2, 128, 64, 96) == 0
    # bf16 values are read where they lie: the workspace does not depend on Hkv or dv;
    # the same call as resolvent_forward at Hkv = H, dv = d
    assert ws(2, 8, 2, 512, 128, 128) == ws(2, 8, 8, 512, 128, 128)
    assert ws(2, 8, 8, 512, 128, 128) == binding.resolvent_workspace_bytes(2, 8, 512, 128)
    assert ws(1, 2, 2, 256, 64, 128) == ws(1, 2, 2, 256, 64, 64)
    # fp32 values on the bf16 path: a bf16 copy of V, Hkv x n x dv per sequence
    f = lambda Hkv, dv: ws(2, 8, Hkv, 512, 128, dv, binding.BF16, binding.F32)
    assert f(2, 128) < f(8, 128)
    assert f(8, 128) - f(2, 128) >= 2 * 6 * 512 * 128 * 2
    assert f(2, 128) > f(2, 64)


def decode_call(B=1, H=4, Hkv=2, n=130, cap=None, d=64, dv=128, beta=1.0, qk=1.0, g=1.0, qdt=0,
                vdt=0, ws_bytes=None, ptr=FAKE, ws=FAKE):
    lib = binding._load()
    if ws_bytes is None:
        ws_bytes = lib.resolvent_decode_workspace_bytes(1, 4, 2, 130, 64, 128, qdt, vdt)
    return lib.resolvent_decode(ptr, ptr, ptr, ptr, ptr, beta, qk, g, B, H, Hkv, n,
                                n if cap is None else cap, d, dv, qdt, vdt, ptr, ptr, ws,
                                ws_bytes, FAKE, None)


def test_decode_host_checks():
    assert decode_call(B=-1) == S.BAD_SHAPE
    assert decode_call(n=-1) == S.BAD_SHAPE
    assert decode_call(n=0, ptr=None) == S.OK  # no position, no readout
    assert decode_call(Hkv=3) == S.BAD_SHAPE
    assert decode_call(Hkv=0) == S.BAD_SHAPE
    assert decode_call(cap=129) == S.BAD_SHAPE  # the cache holds fewer positions than n
    assert decode_call(dv=0) == S.BAD_SHAPE
    for bad in (float("nan"), float("inf")):
        assert decode_call(beta=bad) == S.NONFINITE
        assert decode_call(qk=bad) == S.NONFINITE
        assert decode_call(g=bad) == S.NONFINITE
    assert decode_call(qk=1e308) == S.NONFINITE  # qk log2(e)/sqrt(d) beyond float32
    assert decode_call(d=96) == S.UNSUPPORTED
    assert decode_call(dv=256) == S.UNSUPPORTED
    assert decode_call(qdt=1, vdt=0) == S.UNSUPPORTED  # fp32 q,k with bf16 v
    assert decode_call(ptr=None) == S.BAD_ARG
    assert decode_call(ptr=FAKE + 8) == S.BAD_ARG  # q, k, v are 16-byte aligned
    assert decode_call(ws=FAKE + 16) == S.BAD_ARG
    assert decode_call(ws_bytes=64) == S.BAD_ARG


def test_decode_workspace_sizes():
    ws = binding.resolvent_decode_workspace_bytes
    assert ws(1, 4, 3, 128, 64, 64) == 0 and ws(1, 4, 2, 128, 64, 96) == 0
    assert ws(0, 4, 2, 128, 64, 64) == 0
    assert 0 < ws(1, 4, 2, 128, 64, 64) < ws(1, 4, 2, 128, 64, 128)  # partials grow with dv
    bq, _ = binding.resolvent_tile_shape()
    assert ws(1, 1, 1, bq + 1, 64, 64) > ws(1, 1, 1, bq, 64, 64)


def chain_step_call(B=2, H=3, dv=64, g=1.0, vdt=0, ptr=FAKE):
    lib = binding._load()
    return lib.resolvent_chain_step(ptr, ptr, ptr, ptr, ptr, g, B, H, dv, vdt, FAKE, None)


def test_chain_step_host_checks():
    assert chain_step_call(B=-1) == S.BAD_SHAPE
    assert chain_step_call(dv=-1) == S.BAD_SHAPE
    assert chain_step_call(dv=0, ptr=None) == S.OK
    assert chain_step_call(H=0, ptr=None) == S.OK
    for bad in (float("nan"), float("-inf")):
        assert chain_step_call(g=bad) == S.NONFINITE
    assert chain_step_call(vdt=7) == S.UNSUPPORTED
    assert chain_step_call(dv=8192) == S.UNSUPPORTED
    assert chain_step_call(ptr=None) == S.BAD_ARG
    assert chain_step_call(ptr=FAKE + 1) == S.BAD_ARG


def operator_call(B=1, H=2, n=130, d=64, beta=1.0, qk=1.0, g=1.0, qdt=0, ws_bytes=None,
                  ptr=FAKE, ws=FAKE):
    lib = binding._load()
    if ws_bytes is None:
        ws_bytes = lib.resolvent_operator_workspace_bytes(1, 2, 130, 64, qdt)
    return lib.resolvent_operator(ptr, ptr, ptr, ptr, beta, qk, g, B, H, n, d, qdt, ptr, ptr, ws,
                                  ws_bytes, FAKE, None)


def test_operator_host_checks():
    assert operator_call(B=-1) == S.BAD_SHAPE
    assert operator_call(n=0, ptr=None) == S.OK
    assert operator_call(d=0) == S.BAD_SHAPE
    for bad in (float("nan"), float("inf")):
        assert operator_call(beta=bad) == S.NONFINITE
        assert operator_call(g=bad) == S.NONFINITE
    assert operator_call(qk=1e308) == S.NONFINITE
    assert operator_call(d=96) == S.UNSUPPORTED
    assert operator_call(qdt=3) == S.UNSUPPORTED
    assert operator_call(n=65537) == S.UNSUPPORTED  # the [n, n] export is for small n
    assert operator_call(ptr=None) == S.BAD_ARG
    assert operator_call(ptr=FAKE + 8) == S.BAD_ARG
    assert operator_call(ws=FAKE + 64) == S.BAD_ARG
    assert operator_call(ws_bytes=16) == S.BAD_ARG
    ws = binding.resolvent_operator_workspace_bytes
    assert ws(1, 2, 130, 96) == 0 and ws(0, 2, 130, 64) == 0
    assert 0 < ws(1, 2, 130, 64) < ws(1, 2, 131 + 256, 64)


def test_path_product_host_checks():
    lib = binding._load()

    def call(batch=2, n=100, ptr=FAKE):
        return lib.resolvent_path_product(ptr, ptr, batch, n, ptr, ptr, None)

    assert call(batch=-1) == S.BAD_SHAPE
    assert call(n=-1) == S.BAD_SHAPE
    assert call(n=0, ptr=None) == S.OK
    assert call(batch=0, ptr=None) == S.OK
    assert call(n=65537) == S.UNSUPPORTED
    assert call(ptr=None) == S.BAD_ARG
    assert call(ptr=FAKE + 4) == S.BAD_ARG
