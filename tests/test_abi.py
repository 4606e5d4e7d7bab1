"""CPU tests of the C ABI: the library loads, exports every symbol that
include/kda.h declares, and rejects invalid arguments on the host before any
HIP call (so these run without a GPU)."""

import ctypes
import os
import re

import pytest

from gated_delta_rule_10_amd import kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

A = 0x10000  # a 16-byte aligned stand-in address; never dereferenced on the host


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.LIB_PATH):
        pytest.skip("libkda.so not built")
    return kda.load_library()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted([
        "kda_abi_version", "kda_status_string", "kda_chunk_fwd_workspace_size",
        "kda_chunk_fwd", "kda_decode_step", "kda_chunk_fwd_ex", "kda_decode_step_ex",
        "kda_chunk_fwd_ex_noalloc"])


def test_options_struct_layout_matches_the_header(tmp_path):
    """kda_options_t as laid out by a C compiler equals the binding's ctypes mirror."""
    import subprocess
    fields = [f for f, _ in kda.KdaOptions._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "kda.h"\nint main(void) {\n'
                   '  printf("%zu\\n", sizeof(kda_options_t));\n'
                   + "".join(f'  printf("%zu\\n", offsetof(kda_options_t, {f}));\n' for f in fields)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    try:
        subprocess.check_call(["gcc", "-std=c99", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                               "-I", "/opt/rocm/include", str(src), "-o", str(exe)])
    except (OSError, subprocess.CalledProcessError):
        pytest.skip("no C compiler / ROCm headers for the layout probe")
    got = [int(x) for x in subprocess.check_output([str(exe)]).split()]
    assert got[0] == ctypes.sizeof(kda.KdaOptions)
    assert got[1:] == [getattr(kda.KdaOptions, f).offset for f in fields]


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert kda.kda_abi_version() == 1
    for s in range(5):
        assert kda.kda_status_string(s).startswith("KDA_")
    assert "unknown" in kda.kda_status_string(99)


def _prefill(lib, **over):
    args = dict(q=A, k=A, v=A, g=A, b=A, cu=A, N=2, T=100, H=4, dk=128, dv=128,
                din=kda.KDA_BF16, dout=kda.KDA_BF16, scale=1.0, s0=None, sT=None, o=A,
                chunk=64, ws=None, wsb=0)
    args.update(over)
    return lib.kda_chunk_fwd(args["q"], args["k"], args["v"], args["g"], args["b"],
                             args["cu"], args["N"], args["T"], args["H"], args["dk"],
                             args["dv"], args["din"], args["dout"], args["scale"],
                             args["s0"], args["sT"], args["o"], args["chunk"], args["ws"],
                             args["wsb"], None)


@pytest.mark.parametrize("over,status", [
    (dict(q=None), kda.KDA_ERR_INVALID_ARG),
    (dict(cu=None), kda.KDA_ERR_INVALID_ARG),
    (dict(o=None), kda.KDA_ERR_INVALID_ARG),
    (dict(v=A + 8), kda.KDA_ERR_INVALID_ARG),
    (dict(s0=A + 4), kda.KDA_ERR_INVALID_ARG),
    (dict(N=0), kda.KDA_ERR_INVALID_ARG),
    (dict(H=0), kda.KDA_ERR_INVALID_ARG),
    (dict(T=-1), kda.KDA_ERR_INVALID_ARG),
    (dict(T=2**31 - 64, H=1, dk=64, dv=64), kda.KDA_ERR_INVALID_ARG),  # whole chunks past int32
    (dict(N=2**26, H=2), kda.KDA_ERR_INVALID_ARG),                      # N H 16 past int32
    (dict(din=7), kda.KDA_ERR_INVALID_ARG),
    (dict(dk=96), kda.KDA_ERR_UNSUPPORTED),
    (dict(dv=256), kda.KDA_ERR_UNSUPPORTED),
    (dict(chunk=128), kda.KDA_ERR_UNSUPPORTED),
    (dict(din=kda.KDA_F32, dout=kda.KDA_BF16), kda.KDA_ERR_UNSUPPORTED),
])
def test_chunk_fwd_rejects(lib, over, status):
    assert _prefill(lib, **over) == status


def test_workspace_query(lib):
    import torch
    ws = kda.kda_chunk_fwd_workspace_size
    # the bf16 path stages one record per (chunk, head): at least 54 KB each at d_k = 128
    big = ws(16, 524288, 32, 128, 128, torch.bfloat16)
    assert big >= (524288 // 64) * 32 * 54 * 1024
    assert ws(1, 0, 4, 128, 128, torch.bfloat16) > 0          # offsets even without tokens
    # the fp32 path stages one fp32 record per (chunk, head): at least 128 KB each at d_k = 128
    assert ws(1, 4096, 4, 128, 128, torch.float32) >= (4096 // 64) * 4 * 128 * 1024
    assert ws(1, 0, 4, 128, 128, torch.float32) == 0          # no tokens, no records
    assert ws(1, 4096, 4, 96, 128, torch.bfloat16) == 0       # unsupported head dim
    assert ws(0, 4096, 4, 128, 128, torch.bfloat16) == 0      # invalid N
    assert ws(1, 2**31 - 64, 1, 64, 64, torch.bfloat16) == 0  # token count past the limit
    assert ws(1, 2**31 - 65, 1, 64, 64, torch.bfloat16) >= (2**31 // 64) * 24 * 1024  # the largest allowed
    # grows with the token count and the head count
    assert ws(1, 8192, 4, 128, 128, torch.bfloat16) > ws(1, 4096, 4, 128, 128, torch.bfloat16)
    assert ws(1, 4096, 8, 128, 128, torch.bfloat16) > ws(1, 4096, 4, 128, 128, torch.bfloat16)


def _prefill_ex(lib, opt, **over):
    args = dict(q=A, k=A, v=A, g=A, b=A, cu=A, N=2, T=100, H=4, dk=128, dv=128,
                din=kda.KDA_BF16, dout=kda.KDA_BF16, scale=1.0, s0=None, sT=None, o=A,
                chunk=64, ws=None, wsb=0)
    args.update(over)
    return lib.kda_chunk_fwd_ex(args["q"], args["k"], args["v"], args["g"], args["b"],
                                args["cu"], args["N"], args["T"], args["H"], args["dk"],
                                args["dv"], args["din"], args["dout"], args["scale"],
                                args["s0"], args["sT"], args["o"], args["chunk"], args["ws"],
                                args["wsb"], ctypes.byref(opt), None)


@pytest.mark.parametrize("opt_over,call_over", [
    (dict(num_k_heads=3), {}),                          # 4 value heads are not a multiple of 3
    (dict(num_k_heads=-1), {}),
    (dict(gate_x=A), {}),                               # both gate forms given
    (dict(gate_x=A, gate_scale=0.0), dict(g=None)),     # gate scale must be positive
    (dict(beta_y=A), {}),
    ({}, dict(g=None)),                                 # no gate at all
    (dict(out_gate=A, out_gate_act=7), {}),
    (dict(norm=1, norm_eps=-1.0), {}),
    (dict(norm_weight=A + 4, norm=1), {}),              # misaligned
    (dict(state_slots=A, num_slots=0), {}),
])
def test_chunk_fwd_ex_rejects_inconsistent_options(lib, opt_over, call_over):
    opt = kda.KdaOptions()
    for f, val in opt_over.items():
        setattr(opt, f, val)
    assert _prefill_ex(lib, opt, **call_over) == kda.KDA_ERR_INVALID_ARG


def test_no_tokens_needs_no_gates(lib):
    """With T_total = 0 no gate is read: missing gates pass validation (the call
    then fails on the unsupported head size, which is checked later, before any
    HIP call), while both forms of one gate are still rejected."""
    none = dict(T=0, q=None, k=None, v=None, o=None, g=None, b=None, dk=96)
    assert _prefill(lib, **none) == kda.KDA_ERR_UNSUPPORTED
    assert _prefill_ex(lib, kda.KdaOptions(), **none) == kda.KDA_ERR_UNSUPPORTED
    both = kda.KdaOptions()
    both.gate_x = A
    assert _prefill_ex(lib, both, T=0, g=A, dk=96) == kda.KDA_ERR_INVALID_ARG
    assert _prefill(lib, T=1, g=None, dk=96) == kda.KDA_ERR_INVALID_ARG


def test_plain_entry_point_needs_both_gates(lib):
    assert _prefill(lib, g=None) == kda.KDA_ERR_INVALID_ARG
    assert _decode(lib, b=None) == kda.KDA_ERR_INVALID_ARG


def _decode(lib, **over):
    args = dict(q=A, k=A, v=A, g=A, b=A, st=A, si=None, o=A, B=4, H=2, dk=128, dv=128,
                slots=4, din=kda.KDA_BF16, dout=kda.KDA_BF16, scale=1.0)
    args.update(over)
    return lib.kda_decode_step(args["q"], args["k"], args["v"], args["g"], args["b"],
                               args["st"], args["si"], args["o"], args["B"], args["H"],
                               args["dk"], args["dv"], args["slots"], args["din"],
                               args["dout"], args["scale"], None)


@pytest.mark.parametrize("over,status", [
    (dict(st=None), kda.KDA_ERR_INVALID_ARG),
    (dict(k=A + 2), kda.KDA_ERR_INVALID_ARG),
    (dict(B=0), kda.KDA_ERR_INVALID_ARG),
    (dict(B=5), kda.KDA_ERR_INVALID_ARG),  # identity slots need B <= num_slots
    (dict(slots=0), kda.KDA_ERR_INVALID_ARG),
    (dict(dk=32), kda.KDA_ERR_UNSUPPORTED),
    (dict(din=kda.KDA_F32, dout=kda.KDA_BF16), kda.KDA_ERR_UNSUPPORTED),
])
def test_decode_rejects(lib, over, status):
    assert _decode(lib, **over) == status


def test_binding_refuses_host_tensors(lib):
    import torch
    x = torch.zeros((4, 2, 64))
    with pytest.raises(ValueError):
        kda.kda_chunk_fwd(x, x, x, x, torch.zeros((4, 2)), torch.zeros(2, dtype=torch.int32))


def test_binding_helpers_refuse_mixed_devices_and_wrong_outputs():
    """Host-side checks of the Python binding, without a GPU: tensors on another
    device than the call's, and a caller's output of the wrong shape or dtype."""
    import torch
    from gated_delta_rule_10_amd import kda as kb
    dev = torch.device("cuda", 0)
    with pytest.raises(ValueError, match="all tensors must be on"):
        kb._one_device(dev, None, torch.empty(2))
    kb._one_device(torch.device("cpu"), None, torch.empty(2))  # same device: accepted
    with pytest.raises(ValueError, match=r"o must be torch.bfloat16 \(4, 2, 8\)"):
        kb._out(torch.empty((4, 2, 7), dtype=torch.bfloat16), (4, 2, 8), torch.bfloat16, dev)
    with pytest.raises(ValueError, match="o must be"):
        kb._out(torch.empty((4, 2, 8), dtype=torch.float32), (4, 2, 8), torch.bfloat16, dev)


def test_noalloc_rejects_on_the_host(lib):
    """kda_chunk_fwd_ex_noalloc: a call whose workspace would pass the static scratch
    is refused with KDA_ERR_WORKSPACE before any HIP call (this host has no GPU), and
    invalid arguments are refused as by kda_chunk_fwd_ex."""
    def call(**over):
        a = dict(q=A, k=A, v=A, g=A, b=A, cu=A, N=1, T=1 << 20, H=32, dk=128, dv=128,
                 din=kda.KDA_BF16, dout=kda.KDA_BF16, chunk=64)
        a.update(over)
        return lib.kda_chunk_fwd_ex_noalloc(a["q"], a["k"], a["v"], a["g"], a["b"], a["cu"], a["N"], a["T"],
                                            a["H"], a["dk"], a["dv"], a["din"], a["dout"], 1.0, None, None,
                                            a["q"], a["chunk"], None, None)
    import torch
    limit = 256 << 20
    assert kda.kda_chunk_fwd_workspace_size(1, 1 << 20, 32, 128, 128, torch.bfloat16) > limit
    assert call() == kda.KDA_ERR_WORKSPACE
    assert kda.kda_chunk_fwd_workspace_size(1, 4096, 32, 128, 128, torch.bfloat16) <= limit
    assert call(T=65536) == kda.KDA_ERR_WORKSPACE
    assert call(N=0, T=4096) == kda.KDA_ERR_INVALID_ARG
    assert call(T=4096, dk=96) == kda.KDA_ERR_UNSUPPORTED
    assert call(T=4096, chunk=32) == kda.KDA_ERR_UNSUPPORTED
