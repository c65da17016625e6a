"""The C ABI on the host: the library loads, exports every symbol that
include/abg.h declares, and rejects every invalid argument with its status
code before any HIP call (so these run without a GPU; no kernel is launched).
"""

import ctypes
import os
import re

import pytest

import long_context_biased_amd as abg
from long_context_biased_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "abg.h")

OK, NULL, SHAPE, UNSUP, ALIGN, VALUE, DEVICE, ALIAS = range(8)

# Fake, distinct, 16-byte aligned "device" addresses: validation never
# dereferences them, and every call below fails validation.
Q, K, V, BIAS, OUT, WS = (0x100000000 * (i + 1) for i in range(6))
BF16, F32 = abg.ABG_BF16, abg.ABG_F32


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:abg_status|int64_t|int|const char\*)\s+(abg_\w+)\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    lib = abg.load()
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_version_and_status_strings():
    lib = abg.load()
    assert lib.abg_abi_version() == 1
    for code, name in _lib.STATUS.items():
        assert lib.abg_status_string(code).decode() == name
    assert lib.abg_status_string(99).decode() == "ABG_UNKNOWN_STATUS"


def attn(**kw):
    a = dict(q=Q, k=K, v=V, bias=BIAS, out=OUT, B=1, S=8192, Hq=8, Dk=128, Dv=128,
             bias_batch_stride=0, bias_group=1, scale=0.088, softcap=5.0, dtype=BF16)
    a.update(kw)
    return abg.raw_biased_mqa_fwd(a["q"], a["k"], a["v"], a["bias"], a["out"], a["B"], a["S"],
                                  a["Hq"], a["Dk"], a["Dv"], a["bias_batch_stride"],
                                  a["bias_group"], a["scale"], a["softcap"], a["dtype"], None)


ATTN_CASES = [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(v=None), NULL),
    (dict(bias=None), NULL), (dict(out=None), NULL),
    (dict(B=0), SHAPE), (dict(B=70000), SHAPE),
    (dict(S=0), SHAPE), (dict(S=-64), SHAPE), (dict(S=262144 + 64), SHAPE),
    # the generic kernel takes any length, but not value width 192
    (dict(S=8192 + 16, dtype=F32, Dv=192), UNSUP), (dict(S=100, softcap=0.0, Dv=192), UNSUP),
    (dict(S=32, dtype=F32, bias_batch_stride=4), SHAPE),
    (dict(Hq=4), UNSUP), (dict(Hq=16), UNSUP),
    # (every case here must stay invalid: the pointers are not device memory)
    (dict(Dk=64), UNSUP), (dict(Dv=64), UNSUP), (dict(Dv=256), UNSUP),
    (dict(Dv=192, dtype=F32), UNSUP), (dict(Dv=192, softcap=0.0), UNSUP),
    (dict(scale=float("nan")), VALUE), (dict(scale=float("inf")), VALUE),
    (dict(softcap=-1.0), VALUE), (dict(softcap=float("inf")), VALUE),
    (dict(softcap=float("nan")), VALUE),
    (dict(dtype=7), VALUE),
    (dict(bias_group=0), SHAPE), (dict(B=2, bias_group=3), SHAPE),
    (dict(B=2, bias_batch_stride=100), SHAPE), (dict(B=2, bias_batch_stride=(1 << 40) + 4), SHAPE),
    (dict(bias_batch_stride=-4), SHAPE),
    (dict(B=2, bias_batch_stride=8 * 512 * 512 + 2), ALIGN),
    (dict(q=Q + 8), ALIGN), (dict(k=K + 4), ALIGN), (dict(v=V + 2), ALIGN),
    (dict(bias=BIAS + 12), ALIGN), (dict(out=OUT + 8), ALIGN),
    (dict(out=Q), ALIAS), (dict(out=Q + 16 * 1024 * 1024 - 16), ALIAS),
    (dict(out=K), ALIAS), (dict(out=V), ALIAS), (dict(out=BIAS), ALIAS),
    (dict(out=K - 16 * 1024 * 1024 + 16), ALIAS),
]


@pytest.mark.parametrize("kw,code", ATTN_CASES, ids=lambda x: str(x))
def test_attention_rejects(kw, code):
    st = attn(**kw)
    assert st == code, (st, abg.load().abg_last_error())
    assert abg.load().abg_last_error().decode()


def attn_ex(**kw):
    a = dict(q=Q, k=K, v=V, bias=BIAS, out=OUT, ws=WS, ws_bytes=1 << 30, B=1, Sq=1024, Sk=8192,
             q_offset=1024, Hq=8, Dk=128, Dv=128, bias_batch_stride=0, bias_group=1,
             kv_splits=8, scale=0.088, softcap=5.0, dtype=BF16)
    a.update(kw)
    return abg.raw_biased_mqa_fwd_ex(a["q"], a["k"], a["v"], a["bias"], a["out"], a["ws"],
                                     a["ws_bytes"], a["B"], a["Sq"], a["Sk"], a["q_offset"],
                                     a["Hq"], a["Dk"], a["Dv"], a["bias_batch_stride"],
                                     a["bias_group"], a["kv_splits"], a["scale"], a["softcap"],
                                     a["dtype"], None)


# Every case must stay invalid: the pointers are not device memory.
ATTN_EX_CASES = [
    (dict(Sq=1000, dtype=F32, kv_splits=2, Dv=192), UNSUP), (dict(Sq=0), SHAPE), (dict(Sq=8192 + 32), SHAPE),
    (dict(q_offset=8), UNSUP), (dict(q_offset=-16), SHAPE), (dict(q_offset=8192 - 1024 + 16), SHAPE),
    (dict(kv_splits=0), SHAPE), (dict(kv_splits=65), SHAPE), (dict(kv_splits=3), SHAPE),
    # key ranges on the generic kernel (float32 or no cap): same workspace rules
    (dict(dtype=F32, ws=None), NULL), (dict(softcap=0.0, ws_bytes=1024), SHAPE),
    (dict(dtype=F32, kv_splits=3), SHAPE), (dict(softcap=0.0, ws=Q), ALIAS),
    (dict(ws=None), NULL), (dict(ws_bytes=1024), SHAPE), (dict(ws=WS + 8), ALIGN),
    (dict(ws=Q), ALIAS), (dict(ws=OUT - 1024), ALIAS),
    (dict(Sk=8192 + 64, dtype=F32, kv_splits=3, ws=None), NULL), (dict(Dv=192, dtype=F32, kv_splits=1), UNSUP),
    # 8192 + 16 keys make 129 tiles, which 8 ranges do not divide
    (dict(Sk=8192 + 16), SHAPE), (dict(Sk=100, Sq=64, q_offset=0, kv_splits=4), SHAPE),
    (dict(q=None), NULL), (dict(out=Q), ALIAS),
    # more partial rows than the merge grid takes (checked before the overlaps)
    (dict(B=65535, Sq=262144, Sk=262144, q_offset=0, kv_splits=2, ws_bytes=1 << 62), SHAPE),
]


@pytest.mark.parametrize("kw,code", ATTN_EX_CASES, ids=lambda x: str(x))
def test_attention_ex_rejects(kw, code):
    st = attn_ex(**kw)
    assert st == code, (st, abg.load().abg_last_error())
    assert abg.load().abg_last_error().decode()


def attn_noalloc(**kw):
    a = dict(q=Q, k=K, v=V, bias=BIAS, out=OUT, B=1, Sq=1024, Sk=8192, q_offset=3072, Hq=8,
             Dk=128, Dv=128, bias_batch_stride=0, bias_group=1, kv_splits=8, scale=0.088,
             softcap=5.0, dtype=BF16)
    a.update(kw)
    return abg.raw_biased_mqa_fwd_ex_noalloc(a["q"], a["k"], a["v"], a["bias"], a["out"], a["B"],
                                             a["Sq"], a["Sk"], a["q_offset"], a["Hq"], a["Dk"],
                                             a["Dv"], a["bias_batch_stride"], a["bias_group"],
                                             a["kv_splits"], a["scale"], a["softcap"], a["dtype"],
                                             None)


# The no-allocation entry point validates everything before its scratch
# lookup (the only HIP call before the launch), so these run without a GPU.
# Every case must stay invalid: the pointers are not device memory.
NOALLOC_CASES = [
    (dict(q=None), NULL), (dict(bias=None), NULL), (dict(out=None), NULL),
    (dict(out=Q), ALIAS), (dict(Hq=4), UNSUP), (dict(kv_splits=3), SHAPE),
    (dict(kv_splits=0), SHAPE), (dict(q_offset=8), UNSUP), (dict(scale=float("nan")), VALUE),
    # partials past the 64 MiB scratch: 8 ranges x 8192 rows x 8 heads x 129 x 4 B
    (dict(Sq=8192, q_offset=0), SHAPE),
    # just past: 2033 positions x 8 ranges need 67,141,888 B > 67,108,864 B
    (dict(Sq=2048 + 1, q_offset=0), SHAPE), (dict(B=2, Sq=1024 + 16, Sk=8192), SHAPE),
    (dict(Dv=192, Sq=1400, q_offset=0), SHAPE), (dict(softcap=0.0, Sq=4096, q_offset=0), SHAPE),
]


@pytest.mark.parametrize("kw,code", NOALLOC_CASES, ids=lambda x: str(x))
def test_noalloc_rejects(kw, code):
    st = attn_noalloc(**kw)
    assert st == code, (st, abg.load().abg_last_error())
    msg = abg.load().abg_last_error().decode()
    assert msg
    if code == SHAPE and "Sq" in kw and kw.get("q_offset") == 0 and kw.get("Sq", 0) > 2048:
        assert "no-allocation" in msg, msg


def test_noalloc_scratch_limit_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define ABG_NOALLOC_SCRATCH_BYTES \((\d+)LL << (\d+)\)", text)
    assert m, "ABG_NOALLOC_SCRATCH_BYTES not found"
    assert int(m.group(1)) << int(m.group(2)) == _lib.NOALLOC_SCRATCH_BYTES == 64 << 20
    # the largest request that fits: 8 ranges of 2032 query positions
    assert abg.workspace_bytes(1, 2032, 8, 128, 8) <= _lib.NOALLOC_SCRATCH_BYTES
    assert abg.workspace_bytes(1, 2033, 8, 128, 8) > _lib.NOALLOC_SCRATCH_BYTES


def pattn(**kw):
    a = dict(q=Q, k=K, v=V, pair=BIAS, weight=WS, out=OUT, ws=None, ws_bytes=0, B=1, Sq=8192,
             Sk=8192, q_offset=0, Hq=8, Dk=128, Dv=128, C=128, pair_batch_stride=0, pair_group=1,
             kv_splits=1, scale=0.088, softcap=5.0, dtype=BF16)
    a.update(kw)
    return abg.raw_pair_biased_mqa_fwd(a["q"], a["k"], a["v"], a["pair"], a["weight"], a["out"],
                                       a["ws"], a["ws_bytes"], a["B"], a["Sq"], a["Sk"],
                                       a["q_offset"], a["Hq"], a["Dk"], a["Dv"], a["C"],
                                       a["pair_batch_stride"], a["pair_group"], a["kv_splits"],
                                       a["scale"], a["softcap"], a["dtype"], None)


# The pair form (projection inside the attention kernel).  Every case must
# stay invalid: the pointers are not device memory.
PAIR_CASES = [
    (dict(pair=None), NULL), (dict(weight=None), NULL), (dict(q=None), NULL), (dict(out=None), NULL),
    (dict(dtype=F32), UNSUP), (dict(softcap=0.0), UNSUP), (dict(Dv=256), UNSUP),
    (dict(C=64), UNSUP), (dict(C=256), UNSUP), (dict(dtype=5), VALUE),
    (dict(Sk=0), SHAPE), (dict(Sq=0), SHAPE), (dict(kv_splits=3), SHAPE),
    (dict(kv_splits=8, ws=None), NULL),
    (dict(B=2, pair_batch_stride=100), SHAPE), (dict(B=2, pair_batch_stride=512 * 512 * 128 + 4), ALIGN),
    (dict(B=2, pair_batch_stride=1 << 41), SHAPE),
    (dict(pair_group=0), SHAPE), (dict(B=2, pair_group=3), SHAPE),
    (dict(pair=BIAS + 8), ALIGN), (dict(weight=WS + 2), ALIGN), (dict(out=OUT + 8), ALIGN),
    (dict(out=BIAS), ALIAS), (dict(out=WS - 1024), ALIAS), (dict(out=Q), ALIAS),
    (dict(kv_splits=8, ws=Q, ws_bytes=1 << 30), ALIAS),
    (dict(kv_splits=8, ws=WS + 1024, ws_bytes=1 << 30), ALIAS),  # onto the 2 KiB weight
]


@pytest.mark.parametrize("kw,code", PAIR_CASES, ids=lambda x: str(x))
def test_pair_attention_rejects(kw, code):
    st = pattn(**kw)
    assert st == code, (st, abg.load().abg_last_error())
    assert abg.load().abg_last_error().decode()


def test_workspace_bytes():
    assert abg.workspace_bytes(1, 2048, 8, 128, 1) == 0
    assert abg.workspace_bytes(2, 1024, 8, 128, 4) == 4 * 2 * 1024 * 8 * 129 * 4
    assert abg.workspace_bytes(1, 1024, 8, 192, 8) == 8 * 1024 * 8 * 193 * 4
    for bad in [(0, 1024, 8, 128, 2), (1, 1024, 8, 128, 0), (1, 1024, 8, 128, 65),
                (2**40, 2**20, 8, 128, 64), (1, 2**62, 8, 128, 2)]:
        assert abg.workspace_bytes(*bad) == -1
    assert abg.auto_kv_splits(1, 2048, 2048) == 4
    assert abg.auto_kv_splits(1, 8192, 8192) == 1
    assert abg.auto_kv_splits(1, 1024, 8192) == 8
    assert abg.auto_kv_splits(1, 64, 64) == 1
    # ragged lengths: tiles = ceil(Sk / 64), query blocks = ceil(Sq / 32)
    assert abg.auto_kv_splits(1, 1000, 1000) == 8  # 16 tiles, 32 query blocks: 8 x 32 = 256
    assert abg.auto_kv_splits(1, 100, 100) == 2    # 2 tiles cap it


def proj(**kw):
    a = dict(pair=Q, weight=K, bias=BIAS, Bp=1, P=512, C=128, H=8, dtype=BF16)
    a.update(kw)
    return abg.raw_pair_bias_project(a["pair"], a["weight"], a["bias"], a["Bp"], a["P"],
                                     a["C"], a["H"], a["dtype"], None)


PROJ_CASES = [
    (dict(pair=None), NULL), (dict(weight=None), NULL), (dict(bias=None), NULL),
    (dict(Bp=0), SHAPE), (dict(P=0), SHAPE), (dict(P=70000), SHAPE),
    (dict(C=0), UNSUP), (dict(C=12), UNSUP), (dict(C=1024), UNSUP),
    (dict(H=4), UNSUP), (dict(dtype=3), VALUE),
    (dict(pair=Q + 8), ALIGN), (dict(weight=K + 2), ALIGN), (dict(bias=BIAS + 4), ALIGN),
    (dict(bias=Q + 1024), ALIAS), (dict(bias=K), ALIAS),
]


@pytest.mark.parametrize("kw,code", PROJ_CASES, ids=lambda x: str(x))
def test_projection_rejects(kw, code):
    st = proj(**kw)
    assert st == code, (st, abg.load().abg_last_error())


def test_error_message_is_thread_local_and_cleared():
    import threading
    lib = abg.load()
    assert attn(q=None) == NULL
    msg = lib.abg_last_error().decode()
    assert "q" in msg
    seen = {}

    def other():
        seen["msg"] = lib.abg_last_error().decode()

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen["msg"] == ""
    assert attn(Dk=64) == UNSUP
    assert "Dk" in lib.abg_last_error().decode()


def test_python_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 64, 8, 128)
    with pytest.raises(ValueError):
        abg.biased_mqa_fwd(q, q[:, :, :1], q[:, :, :1], torch.zeros(8, 4, 4))
    with pytest.raises(ValueError):
        abg.pair_bias_project(torch.zeros(4, 4, 8), torch.zeros(8, 8))


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load(str(tmp_path / "nope.so"))


def test_plain_c_consumer(tmp_path):
    """The boundary is usable from C alone: a C99 program built with
    -pedantic -Werror against include/abg.h, linked to the library, gets the
    same host-side validation results as the Python binding."""
    import shutil
    import subprocess

    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not on PATH")
    abg.load()
    libdir = os.path.dirname(_lib.LIB_PATH)
    exe = str(tmp_path / "c_consumer")
    subprocess.run([gcc, "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
                    "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c_consumer.c"),
                    "-L", libdir, "-labg", "-Wl,-rpath," + libdir, "-o", exe],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert "c consumer ok" in r.stdout


def test_build_flags():
    """Every HIP source is compiled for gfx950 with packed FP32 VALU
    instructions disabled (the compiler would otherwise form them from
    ordinary float code)."""
    from long_context_biased_amd import _build
    f = _build.HIP_FLAGS
    assert "--offload-arch=gfx950" in f
    i = f.index("-packed-fp32-ops")
    assert f[i - 3:i] == ["-Xclang", "-target-feature", "-Xclang"]
    assert set(_build.SOURCES) == {"biased_mqa_fwd.hip", "pair_bias_project.hip", "scratch.hip",
                                   "abg_api.cpp"}
