"""The C ABI on the host (no GPU needed): the library loads, exports every
function include/pkv.h declares, and rejects bad arguments before any launch."""
import ctypes
import os
import re

import pytest

import paged_kv_gqa_mapping_amd as pkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")

needs_lib = pytest.mark.skipif(not os.path.exists(pkv.library_path), reason="libpkv.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_three_operations():
    names = declared_functions()
    for n in ("pkv_kv_store", "pkv_paged_decode_attn", "pkv_paged_prefill_attn"):
        assert n in names


@needs_lib
def test_library_exports_every_declared_function():
    L = ctypes.CDLL(pkv.library_path)
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing


@needs_lib
def test_status_strings_and_version():
    L = pkv.lib()
    assert L.pkv_version() >= 100
    for code, name in [(0, "PKV_OK"), (-1, "PKV_ERR_INVALID_ARG"), (-2, "PKV_ERR_UNSUPPORTED"),
                       (-3, "PKV_ERR_WORKSPACE"), (-4, "PKV_ERR_HIP")]:
        assert L.pkv_status_string(code).decode() == name


def _dec(L, **kw):
    args = dict(q=1 << 20, k=1 << 20, v=1 << 20, bt=1 << 20, W=4, cl=1 << 20, maxL=1000, scale=0.1, out=1 << 20,
                B=2, Hq=32, Hkv=8, D=128, NB=10, bs=256, dtype=1, split=0, ws=None, ws_bytes=0)
    args.update(kw)
    a = args
    return L.pkv_paged_decode_attn(a["q"], a["k"], a["v"], a["bt"], a["W"], a["cl"], a["maxL"], a["scale"], a["out"],
                                   a["B"], a["Hq"], a["Hkv"], a["D"], a["NB"], a["bs"], a["dtype"], a["split"],
                                   a["ws"], a["ws_bytes"], None)


@needs_lib
def test_decode_argument_errors_before_launch():
    L = pkv.lib()
    assert _dec(L, D=96) == -2
    assert _dec(L, bs=48) == -2
    assert _dec(L, Hq=24) == -2            # group size 3
    assert _dec(L, Hq=30) == -1            # not a multiple of Hkv
    assert _dec(L, q=None) == -1
    assert _dec(L, q=(1 << 20) + 8) == -1  # misaligned
    assert _dec(L, maxL=2000) == -1        # beyond W * bs
    assert _dec(L, split=100) == -1        # not a multiple of 64
    assert _dec(L, maxL=1000, split=64) == -3   # needs a workspace
    assert "workspace" in L.pkv_last_error().decode()
    assert _dec(L, B=0) == 0               # nothing to do
    assert _dec(L, dtype=7) == -2


@needs_lib
def test_workspace_and_split_queries():
    L = pkv.lib()
    assert L.pkv_decode_workspace_bytes(4, 8, 128, 100, 128) == 0
    assert L.pkv_decode_workspace_bytes(4, 8, 128, 300, 128) == 4 * 8 * 3 * 130 * 4
    # the library's choice: token-balanced ranges above 256 tokens of context,
    # else one split per sequence (the context rounded up to 64)
    for B, Hkv, maxL in [(256, 8, 1024), (64, 8, 8192), (200, 8, 32768), (4096, 8, 2048), (1, 1, 257)]:
        assert L.pkv_decode_split_tokens(B, Hkv * 4, Hkv, 128, maxL, 256, 1) == pkv.SPLIT_BALANCED
    for B, Hkv, maxL, split in [(4, 2, 100, 128), (1, 1, 1, 64), (4096, 8, 256, 256)]:
        assert L.pkv_decode_split_tokens(B, Hkv * 4, Hkv, 128, maxL, 256, 1) == split
    # token-balanced ranges: state slots for 1024 waves plus one per sequence
    # (a wave's range can end inside a sequence), then two ints per sequence
    assert L.pkv_decode_workspace_bytes(4, 8, 128, 100, pkv.SPLIT_BALANCED) == (1024 + 4) * 8 * 130 * 4 + 4 * 8
    assert L.pkv_decode_workspace_bytes(1500, 4, 64, 9, pkv.SPLIT_BALANCED) == (1024 + 1500) * 4 * 66 * 4 + 1500 * 8
    # other negative splits are rejected before anything else is looked at
    assert _dec(L, maxL=1000, split=-2) == -1


@needs_lib
def test_kv_store_and_prefill_argument_errors():
    L = pkv.lib()
    P = 1 << 20
    assert L.pkv_kv_store(P, P, P, P, P, -1, 8, 128, 10, 256, 1, None) == -1
    assert L.pkv_kv_store(P, P, P, P, P, 0, 8, 128, 10, 256, 1, None) == 0
    assert L.pkv_kv_store(P, P, P, P, None, 4, 8, 128, 10, 256, 1, None) == -1
    assert L.pkv_kv_store(P, P, P, P, P, 4, 8, 128, 10, 100, 1, None) == -2
    # prefill: max_seqlen_q > max_seqlen_k, and a table too narrow for max_seqlen_k
    assert L.pkv_paged_prefill_attn(P, P, P, P, P, P, 4, P, 0.0, 2, 10, 9, 8, 32, 8, 128, 10, 256, 1, None, 0, None) == -1
    assert L.pkv_paged_prefill_attn(P, P, P, P, P, P, 1, P, 0.0, 2, 10, 9, 300, 32, 8, 128, 10, 256, 1, None, 0, None) == -1
    assert L.pkv_paged_prefill_attn(P, P, P, P, P, P, 4, P, 0.0, 0, 0, 0, 0, 32, 8, 128, 10, 256, 1, None, 0, None) == 0


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(pkv, "library_path", "/nonexistent/libpkv.so")
    monkeypatch.setattr(pkv, "_lib", None)
    with pytest.raises(pkv.PkvError):
        pkv.lib()


@needs_lib
def test_rope_kv_store_argument_errors_before_launch():
    L = pkv.lib()
    p = 1 << 20

    def call(**kw):
        a = dict(q=p, k=p, v=p, pos=p, kc=p, vc=p, sl=p, N=4, Hq=32, Hkv=8, D=128, NB=10, bs=16, theta=1e6,
                 inter=0, dtype=1)
        a.update(kw)
        return L.pkv_rope_kv_store(a["q"], a["k"], a["v"], a["pos"], a["kc"], a["vc"], a["sl"], a["N"], a["Hq"],
                                   a["Hkv"], a["D"], a["NB"], a["bs"], a["theta"], a["inter"], a["dtype"], None)
    assert call(D=96) == -2
    assert call(bs=48) == -2
    assert call(dtype=7) == -2
    assert call(N=-1) == -1
    assert call(Hq=0) == -1
    assert call(theta=0.5) == -1
    assert call(theta=float("nan")) == -1
    assert call(inter=2) == -1
    assert call(q=None) == -1
    assert call(k=p + 8) == -1           # misaligned
    assert call(N=0, q=None) == 0         # nothing to do: no launch, no pointer needed


@needs_lib
def test_cascade_argument_errors_before_launch():
    L = pkv.lib()
    p = 1 << 20

    def call(**kw):
        a = dict(q=p, k=p, v=p, bt=p, W=80, cl=p, maxL=17000, sh=p, go=p, gs=p, ng=1, gmax=64, smax=16384,
                 own=600, scale=0.1, out=p, B=64, Hq=32, Hkv=8, D=128, NB=200, bs=256, dtype=1, split=0, ws=p,
                 ws_bytes=1 << 40)
        a.update(kw)
        return L.pkv_cascade_decode_attn(a["q"], a["k"], a["v"], a["bt"], a["W"], a["cl"], a["maxL"], a["sh"],
                                         a["go"], a["gs"], a["ng"], a["gmax"], a["smax"], a["own"], a["scale"],
                                         a["out"], a["B"], a["Hq"], a["Hkv"], a["D"], a["NB"], a["bs"], a["dtype"],
                                         a["split"], a["ws"], a["ws_bytes"], None)
    assert call(dtype=0) == -2             # the group pass is bf16 only
    assert call(smax=16384 + 3) == -1      # not whole blocks
    assert call(smax=17000) == -1          # must leave every sequence a key of its own
    assert call(ng=-1) == -1
    assert call(own=-5) == -1
    assert call(gmax=0) == -1
    assert call(sh=None) == -1
    assert call(split=100) == -1
    assert call(ws=None) == -3             # workspace needed
    assert call(ws_bytes=16) == -3
    assert call(D=96) == -2


@needs_lib
def test_cascade_workspace_bytes():
    L = pkv.lib()
    # no groups: the plain decode workspace for the same split
    for maxL, split in ((1000, 256), (20000, 512), (300, 512)):
        assert L.pkv_cascade_workspace_bytes(64, 32, 8, 128, maxL, 0, split, 0, 0, 0) == \
            L.pkv_decode_workspace_bytes(64, 32, 128, maxL, split)
    # one group of 64 behind 16,384 shared keys with at most 512 keys of its own:
    # 2 split states of 256 keys plus the group-pass states (chunk doubled from 256 while
    # member tiles x 8 head groups x chunks > 256 workgroups; a group-pass workgroup
    # takes 64 members for 4 query heads per KV head, so 1 member tile: 512 keys -> 32 chunks)
    assert L.pkv_cascade_workspace_bytes(64, 32, 8, 128, 16896, 512, 256, 1, 64, 16384) == \
        64 * 32 * (2 + 32) * (128 + 2) * 4
    # twice the members: 2 member tiles x 8 head groups, so 1024-key chunks -> 16 chunks
    assert L.pkv_cascade_workspace_bytes(128, 32, 8, 128, 16896, 512, 256, 1, 128, 16384) == \
        128 * 32 * (2 + 16) * (128 + 2) * 4
    # token-balanced own keys (asked for): slots for 1024 waves plus one per
    # sequence, then the group-pass chunks in a region of their own, then two
    # ints per sequence
    assert L.pkv_cascade_workspace_bytes(64, 32, 8, 128, 16896, 512, pkv.SPLIT_BALANCED, 1, 64, 16384) == \
        ((1024 + 64) * 32 + 64 * 32 * 32) * (128 + 2) * 4 + 64 * 8
    # the library's choice: balanced when the own keys could give 1024 waves 256
    # each (200 x 28,672 here; the 64 x 512 above keep the 256-key split)
    ws = L.pkv_cascade_workspace_bytes(200, 32, 8, 128, 32768, 28672, 0, 1, 50, 4096)
    assert ws == L.pkv_cascade_workspace_bytes(200, 32, 8, 128, 32768, 28672, pkv.SPLIT_BALANCED, 1, 50, 4096)
    assert ws % 4 == 0 and ws > (1024 + 200) * 32 * 130 * 4


@needs_lib
def test_check_calls_reject_bad_arguments_on_the_host():
    L = pkv.lib()
    p = 1 << 20
    assert L.pkv_check_decode_inputs(p, 4, p, 100, 2, 10, 16, None, None) == -1          # no flags
    assert L.pkv_check_decode_inputs(p, 0, p, 100, 2, 10, 16, p, None) == -1             # empty table row
    assert L.pkv_check_decode_inputs(None, 4, p, 100, 2, 10, 16, p, None) == -1
    assert L.pkv_check_prefill_inputs(None, p, None, 0, 2, 10, 10, 10, 16, p, None) == -1
    assert L.pkv_check_slots(p, -1, 10, 16, None, p, None) == -1
    assert L.pkv_check_slots(p, 5, 1 << 30, 1 << 10, None, p, None) == -2                # more slots than int32
    assert L.pkv_check_cascade_inputs(p, 4, p, p, p, p, 1, 3, 2, 3, 64, 16, None, p, None) == -1  # no seen
    assert L.pkv_check_cascade_inputs(p, 4, p, p, None, p, 1, 3, 2, 3, 64, 16, p, p, None) == -1


def test_check_names_follow_the_header():
    text = open(HEADER).read()
    codes = dict((m.group(1).lower(), int(m.group(2)))
                 for m in re.finditer(r"PKV_CHECK_([A-Z_]+)\s*=\s*(\d+)", text))
    assert codes.pop("num_flags") == 8
    assert [codes[n] for n in pkv.CHECK_NAMES] == list(range(len(pkv.CHECK_NAMES)))
