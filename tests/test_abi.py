"""libfa.so loads, exports every symbol include/fa.h declares, and validates arguments.

These run without a GPU: every call below returns from host-side validation before the
library touches the HIP runtime (no kernel is launched, no pointer is dereferenced).
"""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


@pytest.fixture(scope="module")
def lib():
    from tiled_attention_causal_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libfa.so is not built; run `python -m tiled_attention_causal_amd.build`")
    return _lib.load()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"FA_API\s+[\w\s\*]+?\b(fa_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_symbols() == ["fa_backward", "fa_backward_atomic",
                                  "fa_backward_atomic_workspace_bytes",
                                  "fa_backward_kernel_name", "fa_backward_main",
                                  "fa_backward_noalloc",
                                  "fa_backward_preprocess", "fa_backward_workspace_bytes",
                                  "fa_forward", "fa_forward_kernel_name",
                                  "fa_forward_with_workspace", "fa_forward_workspace_bytes",
                                  "fa_status_string"]


def _prototype(name):
    """(return type, [(parameter type, name), ...]) of `name` as include/fa.h declares it,
    whitespace normalised."""
    text = open(HEADER).read()
    m = re.search(r"FA_API\s+([\w\s\*]+?)\s*\b" + name + r"\s*\(([^)]*)\)", text)
    assert m, name
    params = []
    for a in m.group(2).split(","):
        a = " ".join(a.split())
        t, n = re.match(r"(.*?)\s*\b(\w+)$", a).groups()
        params.append((t.replace(" *", "*"), n))
    return " ".join(m.group(1).split()), params


# The boundary's contract: the entry points, argument lists and types of the scope table
# (problems flash_forward / flash_backward: forward(Q, K, V, is_causal) -> O with L saved;
# the backward takes the forward's mask and scale with O, L and dO).
CONTRACT = {
    "fa_forward": ("fa_status", [
        ("fa_dtype", "dtype"), ("int64_t", "B"), ("int64_t", "H"), ("int64_t", "Nq"),
        ("int64_t", "Nk"), ("int64_t", "d"), ("const void*", "Q"), ("const void*", "K"),
        ("const void*", "V"), ("int", "is_causal"), ("float", "scale"), ("void*", "O"),
        ("float*", "L"), ("hipStream_t", "stream")]),
    "fa_backward_workspace_bytes": ("size_t", [
        ("fa_dtype", "dtype"), ("int64_t", "B"), ("int64_t", "H"), ("int64_t", "Nq"),
        ("int64_t", "Nk"), ("int64_t", "d")]),
    "fa_backward": ("fa_status", [
        ("fa_dtype", "dtype"), ("int64_t", "B"), ("int64_t", "H"), ("int64_t", "Nq"),
        ("int64_t", "Nk"), ("int64_t", "d"), ("const void*", "Q"), ("const void*", "K"),
        ("const void*", "V"), ("const void*", "O"), ("const float*", "L"),
        ("const void*", "dO"), ("int", "is_causal"), ("float", "scale"), ("void*", "dQ"),
        ("void*", "dK"), ("void*", "dV"), ("void*", "workspace"), ("size_t", "workspace_bytes"),
        ("hipStream_t", "stream")]),
    "fa_status_string": ("const char*", [("fa_status", "status")]),
}


@pytest.mark.parametrize("name", sorted(CONTRACT))
def test_header_matches_the_contract_signatures(name):
    assert _prototype(name) == CONTRACT[name]


def test_status_and_dtype_codes_match_the_contract():
    text = open(HEADER).read()
    for sym, val in (("FA_SUCCESS", 0), ("FA_ERROR_INVALID_VALUE", 1),
                     ("FA_ERROR_NOT_SUPPORTED", 2), ("FA_ERROR_LAUNCH_FAILED", 3),
                     ("FA_DTYPE_F32", 0), ("FA_DTYPE_BF16", 1)):
        assert re.search(r"\b" + sym + r"\s*=\s*" + str(val) + r"\b", text), sym


def test_every_declared_symbol_is_exported(lib):
    from tiled_attention_causal_amd import _lib
    for name in declared_symbols():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, name


def test_only_the_c_abi_is_exported():
    from tiled_attention_causal_amd import _lib
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], stdout=subprocess.PIPE,
                         text=True, check=True).stdout
    text_syms = sorted(ln.split()[-1] for ln in out.splitlines() if " T " in ln)
    assert text_syms == declared_symbols()


def test_status_strings(lib):
    names = {0: "FA_SUCCESS", 1: "FA_ERROR_INVALID_VALUE", 2: "FA_ERROR_NOT_SUPPORTED",
             3: "FA_ERROR_LAUNCH_FAILED", 4: "FA_ERROR_SCRATCH_TOO_SMALL"}
    for code, name in names.items():
        assert lib.fa_status_string(code).decode() == name
    assert lib.fa_status_string(77).decode() == "FA_UNKNOWN_STATUS"


def test_workspace_sizes(lib):
    # bf16: L log2(e) and -D per query row; fp32: none of those; rejected sizes report 0.
    assert lib.fa_backward_workspace_bytes(1, 8, 1, 4096, 4096, 64) == 8 * 4096 * 8
    # Small square grids add room for fp32 partial sums: 64-row tiles x ways x 48 * d/32
    # floats x 128 lanes (B*H = 1, N = 8192, d = 64: 128 tiles, 4 ways).
    assert lib.fa_backward_workspace_bytes(1, 1, 1, 8192, 8192, 64) == (
        8192 * 8 + 128 * 4 * 96 * 128 * 4)
    # N = 2048, d = 32: the causal paired kernel takes 4 ways, the non-causal bwd_kernel 8 (its
    # steps are 32 rows); the size covers either.
    assert lib.fa_backward_workspace_bytes(1, 1, 1, 2048, 2048, 32) == (
        2048 * 8 + 32 * 8 * 48 * 128 * 4)
    # d = 128 (bwd_kernel, two workgroups per CU): causal 8 ways, non-causal 4.
    assert lib.fa_backward_workspace_bytes(1, 1, 1, 8192, 8192, 128) == (
        8192 * 8 + 128 * 8 * 192 * 128 * 4)
    assert lib.fa_backward_workspace_bytes(1, 8, 1, 8192, 8192, 128) == 8 * 8192 * 8
    assert lib.fa_backward_workspace_bytes(1, 4, 25, 2048, 1024, 128) == 100 * 2048 * 8
    assert lib.fa_backward_workspace_bytes(1, 2, 3, 0, 64, 64) == 0
    # fp32: only the partial sums of small grids (8 heads of 4096 at d = 64: causal 2 ways).
    assert lib.fa_backward_workspace_bytes(0, 8, 1, 4096, 4096, 64) == 64 * 8 * 2 * 192 * 64 * 4
    assert lib.fa_backward_workspace_bytes(0, 16, 8, 4096, 4096, 64) == 0   # fills the CUs
    assert lib.fa_backward_workspace_bytes(0, 1, 1, 4000, 4000, 64) == 0    # not 128-aligned
    assert lib.fa_backward_workspace_bytes(1, 8, 1, 4096, 4096, 48) == 0
    assert lib.fa_backward_workspace_bytes(1, -1, 1, 4096, 4096, 64) == 0


def test_forward_workspace_sizes(lib):
    # Small causal bf16 grids (d = 32, 64) use one; everything else needs none.
    ws = lib.fa_forward_workspace_bytes
    # B*H = 1, N = 8192, d = 64: 64 tile pairs x 4 ways x 2 records x 34 x 128 floats
    assert ws(1, 1, 1, 8192, 8192, 64, 1) == 64 * 4 * 2 * 34 * 128 * 4
    # d = 32: 18 floats per lane in a record
    assert ws(1, 1, 1, 8192, 8192, 32, 1) == 64 * 4 * 2 * 18 * 128 * 4
    assert ws(1, 8, 1, 4096, 4096, 64, 1) == 0      # 256 tile pairs fill the CUs already
    assert ws(1, 1, 1, 8192, 8192, 64, 0) == 0      # not causal
    # d = 128 (the paired kernel): 64 tile pairs x 4 ways x 2 records x 66 x 128 floats
    assert ws(1, 1, 1, 8192, 8192, 128, 1) == 64 * 4 * 2 * 66 * 128 * 4
    assert ws(1, 1, 1, 8192, 8192, 16, 1) == 64 * 4 * 2 * 18 * 128 * 4  # split kernel, d = 16
    assert ws(1, 1, 1, 8192, 4096, 64, 1) == 0      # Nq != Nk
    # fp32: 64 query tiles x 8 ways x (16 * ceil(d/32) + 2) floats x 256 lanes
    assert ws(0, 1, 1, 8192, 8192, 64, 1) == 64 * 8 * 34 * 256 * 4
    assert ws(0, 16, 8, 8192, 8192, 64, 1) == 0     # fp32 grid that fills the CUs
    assert ws(1, 1, 1, 256, 256, 64, 1) == 0        # runs would be too short
    assert ws(1, -1, 1, 8192, 8192, 64, 1) == 0     # rejected arguments


# A fake, 16-byte aligned address. Only passed where validation must fail first (or where
# the call is a no-op), so it is never dereferenced.
P = 0x10000
BAD = 0x10002  # misaligned


def fwd(lib, dtype=1, B=1, H=1, Nq=128, Nk=128, d=64, q=P, k=P, v=P, causal=1, scale=0.125,
        o=P, lse=P, ws=None, ws_bytes=0):
    """fa_forward_with_workspace, and fa_forward (the same validation) when there is no
    workspace: both must agree."""
    code = lib.fa_forward_with_workspace(dtype, B, H, Nq, Nk, d, q, k, v, causal, scale, o,
                                         lse, ws, ws_bytes, None)
    if ws is None and ws_bytes == 0:
        assert lib.fa_forward(dtype, B, H, Nq, Nk, d, q, k, v, causal, scale, o, lse,
                              None) == code
    return code


def bwd(lib, dtype=1, B=1, H=1, Nq=128, Nk=128, d=64, q=P, k=P, v=P, o=P, lse=P, do=P,
        causal=1, scale=0.125, dq=P, dk=P, dv=P, ws=P, ws_bytes=1 << 30):
    return lib.fa_backward(dtype, B, H, Nq, Nk, d, q, k, v, o, lse, do, causal, scale, dq, dk,
                           dv, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), 2), (dict(dtype=-1), 2),
    (dict(d=48), 2), (dict(d=256), 2), (dict(d=0), 1), (dict(d=-64), 1),
    (dict(B=-1), 1), (dict(H=-1), 1), (dict(Nq=-1), 1), (dict(Nk=-5), 1),
    (dict(Nk=0), 1),
    (dict(Nq=(1 << 22) + 1), 2), (dict(Nk=(1 << 22) + 1), 2), (dict(B=1 << 20, H=1 << 12), 2),
    (dict(scale=math.inf), 1), (dict(scale=math.nan), 1),
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(o=None), 1),
    (dict(lse=None), 1), (dict(q=BAD), 1), (dict(o=BAD), 1),
    (dict(ws=None, ws_bytes=64), 1), (dict(ws=P + 8, ws_bytes=64), 1),
])
def test_forward_rejects(lib, kw, code):
    assert fwd(lib, **kw) == code


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(Nq=0), dict(Nq=0, Nk=0, q=None,
                                                                        k=None, v=None, o=None,
                                                                        lse=None)])
def test_forward_empty_is_a_noop(lib, kw):
    assert fwd(lib, **kw) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), 2), (dict(d=24), 2), (dict(Nq=-1), 1), (dict(Nk=0), 1),
    (dict(scale=-math.inf), 1),
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(o=None), 1),
    (dict(lse=None), 1), (dict(do=None), 1), (dict(dq=None), 1), (dict(dk=None), 1),
    (dict(dv=None), 1), (dict(dk=BAD), 1),
    (dict(Nq=0, dk=None), 1),  # Nq == 0 still writes dK and dV
    (dict(ws_bytes=128 * 8 - 1), 1), (dict(ws=None), 1), (dict(ws=P + 2), 1),
])
def test_backward_rejects(lib, kw, code):
    assert bwd(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), 2), (dict(d=24), 2), (dict(Nk=0), 1), (dict(q=None), 1), (dict(dk=BAD), 1),
    (dict(ws_bytes=128 * 8 - 1), 1), (dict(ws=None), 1), (dict(scale=math.nan), 1),
])
def test_backward_main_rejects_like_backward(lib, kw, code):
    args = dict(dtype=1, B=1, H=1, Nq=128, Nk=128, d=64, q=P, k=P, v=P, o=P, lse=P, do=P,
                causal=1, scale=0.125, dq=P, dk=P, dv=P, ws=P, ws_bytes=1 << 30)
    args.update(kw)
    a = args
    assert lib.fa_backward_main(a["dtype"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"], a["q"],
                                a["k"], a["v"], a["o"], a["lse"], a["do"], a["causal"],
                                a["scale"], a["dq"], a["dk"], a["dv"], a["ws"], a["ws_bytes"],
                                None) == code


def prep(lib, dtype=1, B=1, H=1, Nq=128, d=64, o=P, lse=P, do=P, ws=P, ws_bytes=1 << 30):
    return lib.fa_backward_preprocess(dtype, B, H, Nq, d, o, lse, do, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), 2), (dict(d=24), 2), (dict(Nq=-1), 1), (dict(Nq=(1 << 22) + 1), 2),
    (dict(o=None), 1), (dict(o=BAD), 1), (dict(do=None), 1), (dict(lse=None), 1),
    (dict(lse=P + 2), 1), (dict(ws=None), 1), (dict(ws=P + 2), 1),
    (dict(ws_bytes=128 * 8 - 1), 1),
])
def test_backward_preprocess_rejects(lib, kw, code):
    assert prep(lib, **kw) == code


def test_backward_preprocess_noops(lib):
    # fp32 has no preprocessing step, and there is nothing to do without query rows.
    assert prep(lib, dtype=0, o=None, lse=None, do=None, ws=None, ws_bytes=0) == 0
    assert prep(lib, B=0, o=None, lse=None, do=None, ws=None, ws_bytes=0) == 0
    assert prep(lib, Nq=0, o=None, lse=None, do=None, ws=None, ws_bytes=0) == 0


def test_backward_empty_is_a_noop(lib):
    assert bwd(lib, B=0) == 0
    assert bwd(lib, B=0, ws=None, ws_bytes=0) == 0
    assert bwd(lib, Nq=0, Nk=0, q=None, k=None, v=None, o=None, lse=None, do=None, dq=None,
               dk=None, dv=None) == 0


def test_python_binding_refuses_cpu_tensors():
    import torch
    from tiled_attention_causal_amd import fa_forward
    x = torch.zeros(1, 1, 16, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa_forward(x, x, x, True)


def test_signature_table_matches_header_argument_counts():
    from tiled_attention_causal_amd import _lib
    text = open(HEADER).read()
    for name in declared_symbols():
        m = re.search(r"FA_API[\w\s\*]+?\b" + name + r"\s*\(([^)]*)\)", text)
        nargs = len([a for a in m.group(1).split(",") if a.strip()])
        assert nargs == len(_lib.SIGNATURES[name][1]), name


def bwd_atomic(lib, dtype=1, B=1, H=1, Nq=128, Nk=128, d=64, q=P, k=P, v=P, o=P, lse=P, do=P,
               causal=1, scale=0.125, dq=P, dk=P, dv=P, ws=P, ws_bytes=1 << 30):
    return lib.fa_backward_atomic(dtype, B, H, Nq, Nk, d, q, k, v, o, lse, do, causal, scale,
                                  dq, dk, dv, ws, ws_bytes, None)


def test_atomic_workspace_sizes(lib):
    # Two per-row floats, then the fp32 dQ accumulator: B*H*Nq*(2 + d)*4 bytes; bf16 only.
    assert lib.fa_backward_atomic_workspace_bytes(1, 8, 1, 4096, 4096, 64) == 8 * 4096 * 66 * 4
    assert lib.fa_backward_atomic_workspace_bytes(1, 2, 3, 100, 300, 16) == 6 * 100 * 18 * 4
    assert lib.fa_backward_atomic_workspace_bytes(0, 8, 1, 4096, 4096, 64) == 0
    assert lib.fa_backward_atomic_workspace_bytes(1, 8, 1, 4096, 4096, 48) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=0), 2), (dict(dtype=5), 2), (dict(d=24), 2), (dict(Nk=0), 1),
    (dict(q=None), 1), (dict(dq=None), 1), (dict(dk=BAD), 1), (dict(scale=math.nan), 1),
    (dict(ws=None), 1),
    (dict(ws_bytes=128 * 8), 1),             # enough for fa_backward, not for the accumulator
    (dict(ws_bytes=128 * 66 * 4 - 1), 1),
])
def test_backward_atomic_rejects(lib, kw, code):
    assert bwd_atomic(lib, **kw) == code


def test_backward_atomic_empty_is_a_noop(lib):
    assert bwd_atomic(lib, B=0) == 0
    assert bwd_atomic(lib, Nq=0, Nk=0, q=None, k=None, v=None, o=None, lse=None, do=None,
                      dq=None, dk=None, dv=None) == 0


def test_kernel_names_follow_dispatch(lib):
    """The library names the kernels its dispatch picks (the launchers and the name queries
    share one plan per pass)."""
    def names(dtype, B, H, Nq, Nk, d, causal, fws=0, bws=1 << 40):
        return (lib.fa_forward_kernel_name(dtype, B, H, Nq, Nk, d, causal, fws).decode(),
                lib.fa_backward_kernel_name(dtype, B, H, Nq, Nk, d, causal, bws).decode())
    # 8 heads of 4096 at d = 64, causal: 256 tile pairs fill the CUs once
    assert names(1, 8, 1, 4096, 4096, 64, 1) == ("fwd_causal_wide_kernel<64>",
                                                 "bwd_causal_paired_kernel<64>")
    # 768 backward workgroups: the lean kernel runs them three per CU, all at once
    assert names(1, 4, 12, 1024, 1024, 64, 1) == ("fwd_causal_paired_kernel<64>",
                                                  "bwd_causal_paired_lean_kernel<64>")
    assert names(1, 1, 40, 1024, 1024, 32, 1)[1] == "bwd_causal_paired_lean_kernel<32>"
    assert names(1, 1, 32, 1024, 1024, 64, 1)[1] == "bwd_causal_paired_kernel<64>"  # 512
    assert names(1, 4, 25, 2048, 2048, 64, 1) == ("fwd_kernel<64, true>", "bwd_kernel<64, true>")
    assert names(1, 4, 25, 2048, 2048, 64, 0) == ("fwd_kernel<64, false>",
                                                  "bwd_kernel<64, false>")
    assert names(1, 8, 1, 16384, 16384, 128, 1) == ("fwd_kernel<128, true>",
                                                    "bwd_kernel<128, true>")
    assert names(1, 1, 2, 2048, 2048, 128, 1) == ("fwd_causal_paired_kernel<128>",
                                                  "bwd_kernel<128, true>")
    assert names(1, 1, 1, 512, 512, 16, 1) == ("fwd_causal_split_kernel<16>",
                                               "bwd_kernel<16, true>")
    assert names(1, 1, 1, 200, 300, 64, 1) == ("fwd_kernel<64, true>", "bwd_kernel<64, true>")
    assert names(0, 1, 1, 128, 128, 16, 1) == ("fwd_f32_kernel<16, true>",
                                               "bwd_f32_kernel<16, true>")
    assert names(1, 1, 1, 128, 128, 48, 1) == ("", "")     # rejected arguments


def bwd_noalloc(lib, dtype=1, B=1, H=1, Nq=128, Nk=128, d=64, q=P, k=P, v=P, o=P, lse=P, do=P,
                causal=1, scale=0.125, dq=P, dk=P, dv=P):
    return lib.fa_backward_noalloc(dtype, B, H, Nq, Nk, d, q, k, v, o, lse, do, causal, scale,
                                   dq, dk, dv, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), 2), (dict(d=24), 2), (dict(Nk=0), 1), (dict(q=None), 1), (dict(dk=BAD), 1),
    (dict(scale=math.nan), 1), (dict(lse=None), 1), (dict(do=None), 1),
    # bf16 needs B*H*Nq*8 bytes of the 32 MiB array: 2 * 2^22 rows need 64 MiB
    (dict(B=2, Nq=1 << 22, Nk=1 << 22), 4),
    (dict(B=1, H=3, Nq=1 << 21, Nk=64), 4),
])
def test_backward_noalloc_rejects_before_any_gpu_call(lib, kw, code):
    assert bwd_noalloc(lib, **kw) == code


def test_backward_noalloc_limit_and_empty(lib):
    from tiled_attention_causal_amd import _lib
    assert _lib.FA_BACKWARD_NOALLOC_MAX_BYTES == 32 << 20
    assert "FA_BACKWARD_NOALLOC_MAX_BYTES ((size_t)32 << 20)" in open(HEADER).read()
    assert lib.fa_status_string(4).decode() == "FA_ERROR_SCRATCH_TOO_SMALL"
    # exactly at the limit the sizes pass validation (the fake pointers then fail it)
    assert bwd_noalloc(lib, B=1, Nq=1 << 22, Nk=1 << 22, q=None) == 1
    # nothing to do returns before the array's address is looked up
    assert bwd_noalloc(lib, B=0) == 0
    assert bwd_noalloc(lib, Nq=0, Nk=0, q=None, k=None, v=None, o=None, lse=None, do=None,
                       dq=None, dk=None, dv=None) == 0
