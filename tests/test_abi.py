"""The C ABI on the host: the library loads, exports what include/gdn.h declares,
and validates arguments (no GPU needed; no call here reaches a kernel launch)."""

import ctypes
import os
import re
import subprocess

import pytest

import linear_attention_recurrence_forward_amd as gdn
from linear_attention_recurrence_forward_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_binding.LIBRARY):
        from linear_attention_recurrence_forward_amd import build
        build.build()
    return _binding._load()


def header_text():
    with open(HEADER) as f:
        return f.read()


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", header_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(_binding.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _binding.LIBRARY],
                         capture_output=True, text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for name in declared_functions():
        assert name in exported, f"{name} declared in gdn.h but not exported"
        assert getattr(lib, name) is not None


def test_status_enum_matches_header():
    text = header_text()
    for code, name in _binding.STATUS.items():
        m = re.search(rf"\b{name}\s*=\s*(\d+)", text)
        assert m and int(m.group(1)) == code, name


def test_params_struct_is_nine_words():
    assert ctypes.sizeof(_binding.GdnParams) == 36
    assert [f[0] for f in _binding.GdnParams._fields_][-1] == "q_scale_bits"


def test_status_strings(lib):
    for code in _binding.STATUS:
        s = gdn.gdn_status_string(code)
        assert s and s != "unknown gdn_status"
    assert gdn.gdn_status_string(999) == "unknown gdn_status"


OK = dict(d_k=128, d_v=128, n_k_heads=16, n_v_heads=48, n_tokens=1, n_seqs=1)


@pytest.mark.parametrize("change,status", [
    ({}, "GDN_OK"),
    ({"d_k": 0}, "GDN_ERR_ZERO_DIM"),
    ({"d_v": 0}, "GDN_ERR_ZERO_DIM"),
    ({"n_k_heads": 0}, "GDN_ERR_ZERO_DIM"),
    ({"n_v_heads": 0}, "GDN_ERR_ZERO_DIM"),
    ({"n_tokens": 0}, "GDN_ERR_ZERO_EXTENT"),
    ({"n_seqs": 0}, "GDN_ERR_ZERO_EXTENT"),
    ({"n_v_heads": 40}, "GDN_ERR_GQA_RATIO"),
    ({"d_k": 96}, "GDN_ERR_UNSUPPORTED_DK"),
    ({"d_k": 16}, "GDN_ERR_UNSUPPORTED_DK"),
    ({"d_k": 256}, "GDN_ERR_UNSUPPORTED_DK"),
    ({"d_k": 33}, "GDN_ERR_UNSUPPORTED_DK"),
    ({"reserved6": 1}, "GDN_ERR_RESERVED_NONZERO"),
    ({"reserved7": 7}, "GDN_ERR_RESERVED_NONZERO"),
    ({"n_seqs": 2**32 - 1, "n_tokens": 2**32 - 1}, "GDN_ERR_SIZE_OVERFLOW"),
    ({"d_v": 2**23}, "GDN_ERR_SIZE_OVERFLOW"),
    ({"d_v": 2**23 - 1, "n_v_heads": 1, "n_k_heads": 1}, "GDN_OK"),
    ({"d_v": 2**17, "n_v_heads": 64, "n_k_heads": 1}, "GDN_ERR_SIZE_OVERFLOW"),
    ({"n_k_heads": 2**16, "n_v_heads": 2**16}, "GDN_ERR_SIZE_OVERFLOW"),
    ({"n_v_heads": 2**20, "n_k_heads": 1, "n_seqs": 2**12}, "GDN_ERR_SIZE_OVERFLOW"),
    ({"d_k": 32, "d_v": 1, "n_k_heads": 1, "n_v_heads": 1}, "GDN_OK"),
    ({"d_k": 64, "d_v": 1000, "n_tokens": 4096, "n_seqs": 3}, "GDN_OK"),
    ({"q_scale_bits": 0xFFFFFFFF}, "GDN_OK"),
])
def test_check_params(lib, change, status):
    p = gdn.make_params(**{**OK, **change})
    assert _binding.STATUS[gdn.gdn_check_params(p)] == status


def test_null_params(lib):
    assert _binding.STATUS[lib.gdn_check_params(None)] == "GDN_ERR_NULL_POINTER"


# Fake, never dereferenced device addresses: every case below fails validation
# before the library touches the runtime.
def fake(addr):
    return ctypes.cast(ctypes.c_void_p(addr), ctypes.POINTER(ctypes.c_float))


def layout(p, base=1 << 40, gap=1 << 30, **overrides):
    """Non-overlapping aligned fake addresses for every array."""
    names = ["q", "k", "v", "g", "beta", "state_in", "output", "state_out", "state_capture"]
    addrs = {n: base + i * gap for i, n in enumerate(names)}
    addrs.update(overrides)
    return addrs


def call(lib, p, addrs, capture=True, null=()):
    order = ["q", "k", "v", "g", "beta", "state_in", "output", "state_out"]
    ptrs = [None if n in null else fake(addrs[n]) for n in order]
    if capture:
        cap = None if "state_capture" in null else fake(addrs["state_capture"])
        st = lib.gdn_forward_capture(*ptrs, cap, ctypes.byref(p), None)
    else:
        st = lib.gdn_forward(*ptrs, ctypes.byref(p), None)
    return _binding.STATUS[st]


def test_forward_rejects_bad_params_first(lib):
    p = gdn.make_params(**{**OK, "n_tokens": 0})
    assert call(lib, p, layout(p), null=("q",)) == "GDN_ERR_ZERO_EXTENT"
    assert call(lib, p, layout(p), capture=False) == "GDN_ERR_ZERO_EXTENT"


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "state_in", "output",
                                  "state_out"])
def test_forward_null_pointer(lib, name):
    p = gdn.make_params(**OK)
    assert call(lib, p, layout(p), null=(name,)) == "GDN_ERR_NULL_POINTER"
    assert call(lib, p, layout(p), capture=False, null=(name,)) == "GDN_ERR_NULL_POINTER"


@pytest.mark.parametrize("name,offset", [
    ("q", 4), ("k", 8), ("state_in", 12), ("state_out", 4), ("state_capture", 8),
    ("v", 2), ("g", 1), ("beta", 3), ("output", 2),
])
def test_forward_misaligned(lib, name, offset):
    p = gdn.make_params(**OK)
    a = layout(p)
    a[name] += offset
    assert call(lib, p, a) == "GDN_ERR_MISALIGNED"


def test_forward_aliasing(lib):
    p = gdn.make_params(**{**OK, "n_tokens": 4})
    c = p.counts()
    a = layout(p)
    # output overlapping the tail of v
    b = dict(a, output=a["v"] + 4 * (c["v"] - 4))
    assert call(lib, p, b) == "GDN_ERR_ALIASING"
    # state_out shifted into state_in (partial overlap) is refused ...
    b = dict(a, state_out=a["state_in"] + 16)
    assert call(lib, p, b) == "GDN_ERR_ALIASING"
    # capture overlapping state_out
    b = dict(a, state_capture=a["state_out"] + 4 * c["state_out"] - 16)
    assert call(lib, p, b) == "GDN_ERR_ALIASING"
    # output overlapping q
    b = dict(a, output=a["q"])
    assert call(lib, p, b) == "GDN_ERR_ALIASING"
    # capture overlapping k
    b = dict(a, state_capture=a["k"] + 1024)
    assert call(lib, p, b) == "GDN_ERR_ALIASING"


def test_binding_checks_tensors_before_the_library():
    torch = pytest.importorskip("torch")
    p = gdn.make_params(32, 32, 1, 2, 8, 1)
    c = p.counts()
    cpu = {n: torch.zeros(c[n]) for n in ("q", "k", "v", "g", "beta", "state_in",
                                          "output", "state_out")}
    with pytest.raises(ValueError, match="must be on the GPU"):
        gdn.gdn_forward(**cpu, params=p)
    bad = dict(cpu, q=torch.zeros(c["q"], dtype=torch.float64))
    with pytest.raises(ValueError, match="must be f32"):
        gdn.gdn_forward(**bad, params=p)
    with pytest.raises(gdn.GdnError, match="GDN_ERR_ZERO_EXTENT"):
        gdn.gdn_forward(**cpu, params=gdn.make_params(32, 32, 1, 2, 0, 1))


def test_rollback_validation(lib):
    p = gdn.make_params(**{**OK, "n_tokens": 4, "n_seqs": 2})
    c = p.counts()
    fp = lambda a: fake(a)  # noqa: E731
    up = lambda a: ctypes.cast(ctypes.c_void_p(a), ctypes.POINTER(ctypes.c_uint32))  # noqa: E731
    cap, acc, st = 1 << 40, (1 << 40) + (1 << 32), (1 << 40) + (2 << 32)

    def rb(c_, a_, s_, params=p):
        return _binding.STATUS[lib.gdn_rollback(c_, a_, s_, ctypes.byref(params), None)]

    assert rb(fp(cap), up(acc), fp(st), gdn.make_params(**{**OK, "n_seqs": 0})) == \
        "GDN_ERR_ZERO_EXTENT"
    assert rb(None, up(acc), fp(st)) == "GDN_ERR_NULL_POINTER"
    assert rb(fp(cap), None, fp(st)) == "GDN_ERR_NULL_POINTER"
    assert rb(fp(cap), up(acc), None) == "GDN_ERR_NULL_POINTER"
    assert rb(fp(cap + 4), up(acc), fp(st)) == "GDN_ERR_MISALIGNED"
    assert rb(fp(cap), up(acc + 2), fp(st)) == "GDN_ERR_MISALIGNED"
    assert rb(fp(cap), up(acc), fp(st + 8)) == "GDN_ERR_MISALIGNED"
    # state inside the capture buffer, or over the index array
    assert rb(fp(cap), up(acc), fp(cap + 4 * c["state_capture"] - 64)) == "GDN_ERR_ALIASING"
    assert rb(fp(cap), up(st + 16), fp(st)) == "GDN_ERR_ALIASING"


def test_forward_bf16_alignment(lib):
    """bf16 q and k need 8-byte alignment, v and output 2-byte."""
    p = gdn.make_params(**OK)
    a = layout(p)
    vp = lambda n, off=0: ctypes.c_void_p(a[n] + off)  # noqa: E731

    def call16(**off):
        return _binding.STATUS[lib.gdn_forward_bf16(
            vp("q", off.get("q", 0)), vp("k", off.get("k", 0)), vp("v", off.get("v", 0)),
            fake(a["g"]), fake(a["beta"]), fake(a["state_in"]),
            vp("output", off.get("output", 0)), fake(a["state_out"]),
            fake(a["state_capture"]), ctypes.byref(p), None)]

    assert call16(q=4) == "GDN_ERR_MISALIGNED"
    assert call16(k=2) == "GDN_ERR_MISALIGNED"
    assert call16(v=1) == "GDN_ERR_MISALIGNED"
    assert call16(output=1) == "GDN_ERR_MISALIGNED"
    # bf16 output overlapping the bf16 v buffer's tail
    c = p.counts()
    b = dict(a, output=a["v"] + 2 * c["v"] - 2)
    assert _binding.STATUS[lib.gdn_forward_bf16(
        ctypes.c_void_p(b["q"]), ctypes.c_void_p(b["k"]), ctypes.c_void_p(b["v"]),
        fake(b["g"]), fake(b["beta"]), fake(b["state_in"]), ctypes.c_void_p(b["output"]),
        fake(b["state_out"]), None, ctypes.byref(p), None)] == "GDN_ERR_ALIASING"


def test_forward_ex_options(lib):
    """gdn_forward_ex: unknown option bits are refused first (after params);
    the known bits select the f32/bf16 rules of the other entry points."""
    p = gdn.make_params(**OK)
    a = layout(p)
    vp = lambda n, off=0: ctypes.c_void_p(a[n] + off)  # noqa: E731

    def ex(options, params=p, **off):
        return _binding.STATUS[lib.gdn_forward_ex(
            vp("q", off.get("q", 0)), vp("k", off.get("k", 0)), vp("v"), fake(a["g"]),
            fake(a["beta"]), fake(a["state_in"]), vp("output"), fake(a["state_out"]),
            None, ctypes.byref(params) if params is not None else None, options, None)]

    assert ex(0, params=None) == "GDN_ERR_NULL_POINTER"
    for bad in (4, 8, 1 << 31, 0xFFFFFFFF):
        assert ex(bad) == "GDN_ERR_OPTION"
        assert ex(bad | _binding.OPT_NORMALIZE_K) == "GDN_ERR_OPTION"
    assert ex(_binding.OPT_NORMALIZE_K, params=gdn.make_params(**{**OK, "d_k": 48})) == \
        "GDN_ERR_UNSUPPORTED_DK"
    # f32 rule (16-byte q) without the bf16 bit, 8-byte with it
    assert ex(_binding.OPT_NORMALIZE_K, q=8) == "GDN_ERR_MISALIGNED"
    assert ex(_binding.OPT_NORMALIZE_K | _binding.OPT_BF16_IO, k=4) == "GDN_ERR_MISALIGNED"


def test_q_scale_value_or_bits():
    """forward(q_scale=<float>) stores the value's binary32 bits in params word
    8; q_scale_bits passes them as they are; neither means q is pre-scaled
    (bits 0). +0.0 has bits 0, which read as "no scale", so it is refused;
    -0.0 is a literal scale. The checks run before any tensor is touched."""
    from linear_attention_recurrence_forward_amd import _binding as b
    assert b.scale_bits() == 0
    assert b.scale_bits(q_scale=1 / 128 ** 0.5) == 0x3DB504F3
    assert b.scale_bits(q_scale_bits=0x3E3504F3) == 0x3E3504F3
    assert b.scale_bits(q_scale=-0.0) == 0x80000000
    with pytest.raises(ValueError, match="cannot be expressed"):
        b.scale_bits(q_scale=0.0)
    with pytest.raises(ValueError, match="not both"):
        b.scale_bits(q_scale=0.5, q_scale_bits=0x3F000000)
    torch = pytest.importorskip("torch")
    z = torch.zeros(1, 1, 1, 32)
    with pytest.raises(ValueError, match="cannot be expressed"):
        b.forward(z, z, z, z[..., 0], z[..., 0], torch.zeros(1, 1, 32, 32), q_scale=0.0)
