"""The C-ABI library loads and exports what include/zha.h declares; host-side
validation rejects bad arguments before anything reaches a GPU.  CPU only:
nothing here launches a kernel."""
import ctypes
import os
import re

import pytest

from hierarchical_tree_indexed_02_amd import zha

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "zha.h"), encoding="utf-8") as f:
        src = f.read()
    return sorted(set(re.findall(r"^ZHA_API [^(]*?\b(zha_\w+)\(", src, flags=re.M)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 16
    lib = ctypes.CDLL(zha.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in zha.h but not exported"


def test_binding_covers_every_symbol():
    for n in _declared():
        assert callable(getattr(zha, n)), n


def test_status_strings():
    assert zha.zha_status_str(zha.ZHA_OK) == "ok"
    assert "capacity" in zha.zha_status_str(zha.ZHA_ERR_CAPACITY)
    assert "gave up" in zha.zha_status_str(zha.ZHA_ERR_DEVICE)
    assert zha.zha_status_str(99) == "unknown status"


def _desc(**kw):
    base = dict(batch=1, n_kv_heads=4, n_q_heads=32, head_dim=128, chunk=4, levels=6, n_refs=16, max_tokens=1 << 18,
                dtype=zha.ZHA_BF16, summary=zha.ZHA_SUMMARY_NATIVE, per_head_routes=0, max_queries=0)
    base.update(kw)
    return zha.zha_tree_desc(*[base[k] for k in ("batch", "n_kv_heads", "n_q_heads", "head_dim", "chunk", "levels",
                                                   "n_refs", "max_tokens", "dtype", "summary", "per_head_routes",
                                                   "max_queries")])


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), zha.ZHA_ERR_INVALID),
    (dict(chunk=1), zha.ZHA_ERR_INVALID),
    (dict(levels=0), zha.ZHA_ERR_INVALID),
    (dict(n_refs=0), zha.ZHA_ERR_INVALID),
    (dict(n_q_heads=30), zha.ZHA_ERR_INVALID),
    (dict(dtype=7), zha.ZHA_ERR_INVALID),
    (dict(max_tokens=0), zha.ZHA_ERR_INVALID),
    (dict(head_dim=96), zha.ZHA_ERR_UNSUPPORTED),
    (dict(n_refs=3), zha.ZHA_ERR_UNSUPPORTED),
    (dict(n_refs=32), zha.ZHA_ERR_UNSUPPORTED),
    (dict(n_q_heads=4 * 17), zha.ZHA_ERR_UNSUPPORTED),
    (dict(batch=65), zha.ZHA_ERR_UNSUPPORTED),
    (dict(chunk=4, levels=16), zha.ZHA_ERR_UNSUPPORTED),
    (dict(max_tokens=1 << 31), zha.ZHA_ERR_UNSUPPORTED),
    (dict(max_queries=-1), zha.ZHA_ERR_INVALID),
    # routing units of the largest route: 64 * 4 * 256 = 65536, one more than a grid dimension holds
    (dict(batch=64, max_queries=256), zha.ZHA_ERR_UNSUPPORTED),
    (dict(batch=64, max_queries=32, per_head_routes=1), zha.ZHA_ERR_UNSUPPORTED),
])
def test_create_rejects(kw, status):
    with pytest.raises(zha.ZhaError) as ei:
        zha.zha_tree_create(_desc(**kw))
    assert ei.value.status == status


def test_null_arguments_rejected():
    lib = zha.load()
    assert lib.zha_tree_create(None, None) == zha.ZHA_ERR_INVALID
    assert lib.zha_build(None, None, None, None, None) == zha.ZHA_ERR_INVALID
    assert lib.zha_append(None, None, None, None) == zha.ZHA_ERR_INVALID
    assert lib.zha_route(None, None, ctypes.c_float(0.9), ctypes.c_float(1.0), None, None) == zha.ZHA_ERR_INVALID
    assert lib.zha_attend(None, None, None, None, None, ctypes.c_float(1.0), None, None, None) == zha.ZHA_ERR_INVALID
    assert lib.zha_route_multi(None, None, 2, ctypes.c_float(0.9), ctypes.c_float(1.0), 0, None,
                               None) == zha.ZHA_ERR_INVALID
    assert lib.zha_attend_multi(None, None, 2, None, None, None, ctypes.c_float(1.0), None, None,
                                None) == zha.ZHA_ERR_INVALID
    assert lib.zha_tree_bytes(None, None) == zha.ZHA_ERR_INVALID
    assert lib.zha_tree_check(None, None) == zha.ZHA_ERR_INVALID
    assert lib.zha_timing_enable(None, 1, -1) == zha.ZHA_ERR_INVALID
    n = ctypes.c_int32()
    assert lib.zha_timing_read(None, None, None, None, 0, ctypes.byref(n)) == zha.ZHA_ERR_INVALID
    assert lib.zha_calibration_copy(None, None, 1, None) == zha.ZHA_ERR_INVALID
    assert lib.zha_calibration_copy(16, 24, 1, None) == zha.ZHA_ERR_INVALID  # misaligned


def test_dense_noalloc_rejects_oversized_shapes_on_host():
    """Shapes whose partials exceed the library's fixed array are refused before the device
    is touched (this runs without a GPU)."""
    fake = 1 << 40  # never dereferenced
    # 64 sequences x 64 KV heads x 16 query heads each: far beyond ZHA_DENSE_SCRATCH_BYTES
    need = zha.zha_dense_workspace_bytes(64, 1024, 64, 128, 1000)
    assert need > zha.ZHA_DENSE_SCRATCH_BYTES
    with pytest.raises(zha.ZhaError) as ei:
        zha.zha_dense_decode_noalloc(fake, fake, fake, [100] * 64, 64, 1024, 64, 128, 1000, zha.ZHA_BF16, 1.0, fake,
                                     fake, stream=0)
    assert ei.value.status == zha.ZHA_ERR_CAPACITY
    with pytest.raises(zha.ZhaError) as ei:  # ordinary validation first, as for zha_dense_decode
        zha.zha_dense_decode_noalloc(0, fake, fake, [100], 1, 32, 4, 128, 1000, zha.ZHA_BF16, 1.0, fake, fake,
                                     stream=0)
    assert ei.value.status == zha.ZHA_ERR_INVALID


def test_dense_validation_on_host():
    lens = [100]
    ws = zha.zha_dense_workspace_bytes(1, 32, 4, 128, 1000)
    assert ws > 0
    assert zha.zha_dense_workspace_bytes(0, 32, 4, 128, 1000) == 0
    fake = 1 << 40  # never dereferenced: every case fails validation first
    cases = [
        (dict(q=0), zha.ZHA_ERR_INVALID),
        (dict(n_q_heads=30), zha.ZHA_ERR_INVALID),
        (dict(lens=[0]), zha.ZHA_ERR_INVALID),
        (dict(lens=[1001]), zha.ZHA_ERR_CAPACITY),
        (dict(head_dim=80), zha.ZHA_ERR_UNSUPPORTED),
        (dict(ws_bytes=ws - 1), zha.ZHA_ERR_INVALID),
        (dict(dtype=5), zha.ZHA_ERR_INVALID),
    ]
    for kw, status in cases:
        a = dict(q=fake, lens=lens, n_q_heads=32, head_dim=128, ws_bytes=ws, dtype=zha.ZHA_BF16)
        a.update(kw)
        with pytest.raises(zha.ZhaError) as ei:
            zha.zha_dense_decode(a["q"], fake, fake, a["lens"], 1, a["n_q_heads"], 4, a["head_dim"], 1000, a["dtype"],
                                 1.0, fake, fake, fake, a["ws_bytes"], stream=0)
        assert ei.value.status == status, kw
