"""C-ABI surface on the CPU: the library loads, exports every function that
include/qk4v8.h declares, and rejects invalid arguments with the documented
status before touching the GPU (no compute calls here)."""
import ctypes
import os
import re

import pytest

from bit_quantized_attention_online_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "qk4v8.h")).read()
    return sorted(set(re.findall(r"\b(qk4v8_[a-z_]+)\s*\(", src)))


def test_header_declares_the_exported_api():
    assert _declared() == sorted(ops.EXPORTED)


def test_peaks_library_exports_its_header():
    from bit_quantized_attention_online_amd import peaks
    src = open(os.path.join(ROOT, "include", "qk4v8_peaks.h")).read()
    declared = sorted(set(re.findall(r"\b(qk4v8_peak_[a-z0-9_]+)\s*\(", src)))
    assert declared == sorted(peaks.EXPORTED)
    L = peaks.lib()
    for name in declared:
        assert hasattr(L, name), name
    d = ctypes.c_double(0)
    assert L.qk4v8_peak_hbm_read(None, 64, ctypes.c_void_p(4096), None) == 1
    assert L.qk4v8_peak_hbm_read(ctypes.c_void_p(4096), 60, ctypes.c_void_p(4096), None) == 2
    assert L.qk4v8_peak_mfma(3, 10, ctypes.c_void_p(4096), ctypes.byref(d), None) == 2
    assert L.qk4v8_peak_mfma(4, 0, ctypes.c_void_p(4096), ctypes.byref(d), None) == 2
    assert L.qk4v8_peak_exp2(1 << 25, ctypes.c_void_p(4096), ctypes.byref(d), None) == 2


def test_default_p_mode_matches_header():
    src = open(os.path.join(ROOT, "include", "qk4v8.h")).read()
    names = dict(re.findall(r"#define (QK4V8_P_[A-Z0-9_]+) (\w+)", src))
    value = lambda n: int(names[n]) if names[n].isdigit() else value(names[n])
    assert value("QK4V8_P_DEFAULT_MODE") == ops.P_DEFAULT_MODE
    assert [value(n) for n in ("QK4V8_P_DEFAULT", "QK4V8_P_FP8_SINGLE", "QK4V8_P_FP8_TWO_TERM", "QK4V8_P_BF16")] == \
        [ops.P_DEFAULT, ops.P_FP8_SINGLE, ops.P_FP8_TWO_TERM, ops.P_BF16]


def test_library_exports_every_declared_symbol():
    L = ops.lib()
    for name in _declared():
        assert hasattr(L, name), name
    assert L.qk4v8_abi_version() == 8
    for s in range(7):
        assert L.qk4v8_status_string(s)


def test_quantize_validation():
    L = ops.lib()
    p = ctypes.c_void_p(4096)
    assert L.qk4v8_quantize_qk(p, 10, 48, 48, p, p, None) == 2          # d % 32
    assert L.qk4v8_quantize_qk(p, -1, 64, 64, p, p, None) == 2
    assert L.qk4v8_quantize_qk(p, 10, 64, 60, p, p, None) == 3          # ld < d
    assert L.qk4v8_quantize_qk(p, 10, 64, 68, p, p, None) == 3          # ld % 8
    assert L.qk4v8_quantize_qk(None, 10, 64, 64, p, p, None) == 1
    assert L.qk4v8_quantize_qk(None, 0, 64, 64, None, None, None) == 0  # empty is a no-op
    assert L.qk4v8_quantize_qk(ctypes.c_void_p(4098), 10, 64, 64, p, p, None) == 3   # misaligned
    assert L.qk4v8_quantize_v(p, 2, 10, 64, 640, 64, 48, p, p, None) == 2            # tile rows
    assert L.qk4v8_quantize_v(p, 2, 10, 64, 644, 64, 64, p, p, None) == 3            # group stride % 8
    assert L.qk4v8_quantize_v(p, 2, 10, 64, 640, 60, 64, p, p, None) == 3            # row stride < d
    assert L.qk4v8_quantize_v(p, 0, 10, 64, 640, 64, 64, None, None, None) == 0


def _prefill(**kw):
    a = ops.PrefillArgs()
    a.q = a.k = a.v = a.o = 4096
    for f in ("q_stride", "k_stride", "v_stride", "o_stride"):
        getattr(a, f)[:] = [8 * 64 * 128, 64 * 128, 128]
    a.batch, a.q_heads, a.kv_heads, a.seq_q, a.seq_k, a.head_dim = 1, 8, 2, 64, 64, 128
    a.v_tile_rows, a.causal, a.softmax_scale = 64, 1, 0.088
    a.workspace, a.workspace_bytes = 1 << 20, 1 << 30
    for k, v in kw.items():
        if k.endswith("stride"):
            getattr(a, k)[:] = v
        else:
            setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(q_heads=6, kv_heads=4), 2), (dict(head_dim=96), 2), (dict(v_tile_rows=100), 2),
    (dict(causal=2), 2), (dict(seq_q=65), 2), (dict(softmax_scale=0.0), 2), (dict(softmax_scale=float("nan")), 2),
    (dict(q=None), 1), (dict(q_stride=[64 * 128, 128, 36]), 3), (dict(o_stride=[64 * 128, 128, 4]), 3),
    (dict(k=4100), 3), (dict(workspace=None), 5), (dict(workspace=1 << 20 | 8), 5), (dict(workspace_bytes=16), 5),
    (dict(p_mode=4), 2), (dict(p_mode=-1), 2), (dict(hadamard=2), 2), (dict(window=-1), 2), (dict(window=16, causal=0), 2),
])
def test_prefill_validation(kw, status):
    a = _prefill(**kw)
    assert ops.lib().qk4v8_attn_prefill(ctypes.byref(a), None) == status


def test_prefill_empty_and_workspace_query():
    L = ops.lib()
    assert L.qk4v8_attn_prefill(ctypes.byref(_prefill(batch=0, q=None)), None) == 0
    assert L.qk4v8_attn_prefill(ctypes.byref(_prefill(seq_q=0, causal=0)), None) == 0
    ws = L.qk4v8_prefill_workspace_bytes(ctypes.byref(_prefill()))
    # K codes + K scales + V codes + V tile-scale words + per-tile V scales, 256-B aligned
    assert ws >= 2 * 1 * 128 * (64 + 4 + 128)
    assert L.qk4v8_prefill_workspace_bytes(ctypes.byref(_prefill(head_dim=96))) == 0


def _decode(**kw):
    a = ops.DecodeArgs()
    a.q = a.k_codes = a.v_codes = a.o = 4096
    a.k_scales = a.v_scales = 4096
    a.q_stride[:] = [64 * 128, 64 * 128, 128]
    a.o_stride[:] = [64 * 128, 64 * 128, 128]
    a.batch, a.q_len, a.q_heads, a.kv_heads, a.kv_len, a.cap = 2, 1, 64, 8, 1000, 1024
    a.head_dim, a.v_tile_rows, a.num_splits, a.softmax_scale = 128, 256, 0, 0.088
    a.workspace, a.workspace_bytes = 1 << 20, 1 << 30
    for k, v in kw.items():
        if k.endswith("stride"):
            getattr(a, k)[:] = v
        else:
            setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(q_len=9), 2), (dict(kv_len=1025), 2), (dict(kv_len=0), 2), (dict(head_dim=256), 2),
    (dict(v_tile_rows=16), 2), (dict(num_splits=-1), 2), (dict(v_codes=None), 1),
    (dict(q_stride=[64 * 128, 64 * 128, 100]), 3), (dict(k_codes=4104), 3),
    (dict(workspace_bytes=0, num_splits=2), 5),
    (dict(window=-3), 2),
    (dict(block_table=4096, page_size=200, pages_per_seq=5, cap=1000), 2),       # not a multiple of 128
    (dict(block_table=4096, page_size=128, pages_per_seq=8), 2),                 # page < V tile (256)
    (dict(block_table=4096, page_size=256, pages_per_seq=3), 2),                 # cap != pages * page_size
    (dict(block_table=4098, page_size=512, pages_per_seq=2), 2),                 # misaligned table
])
def test_decode_validation(kw, status):
    assert ops.lib().qk4v8_attn_decode(ctypes.byref(_decode(**kw)), None) == status


def test_decode_workspace_query():
    L = ops.lib()
    a = _decode(num_splits=4)
    # partial outputs: batch * kv_heads * splits * (G * q_len) rows of head_dim fp32 + one lse each
    rows = 2 * 8 * 4 * 8
    assert L.qk4v8_decode_workspace_bytes(ctypes.byref(a)) >= rows * (128 * 4 + 4)
    assert L.qk4v8_decode_workspace_bytes(ctypes.byref(_decode(q_len=9))) == 0


def test_decode_paging_is_validated_by_the_workspace_query():
    L = ops.lib()
    ok = _decode(block_table=4096, page_size=512, pages_per_seq=2, num_splits=2)   # cap 1024 = 2 pages of 512
    assert L.qk4v8_decode_workspace_bytes(ctypes.byref(ok)) == L.qk4v8_decode_workspace_bytes(
        ctypes.byref(_decode(num_splits=2)))
    assert L.qk4v8_decode_workspace_bytes(ctypes.byref(_decode(block_table=4096, page_size=384, num_splits=2,
                                                                pages_per_seq=3, cap=1152, v_tile_rows=128))) > 0
    assert L.qk4v8_decode_workspace_bytes(ctypes.byref(_decode(block_table=4096, page_size=384, num_splits=2,
                                                                pages_per_seq=3, cap=1152))) == 0   # 384 % 256


def test_decode_auto_splits_need_a_device():
    # with num_splits = 0 the split count comes from the device's CU count
    # and occupancy: without a device the query reports 0 and the call
    # QK4V8_ERR_HIP instead of guessing a machine
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    L = ops.lib()
    assert L.qk4v8_decode_workspace_bytes(ctypes.byref(_decode())) == 0
    assert L.qk4v8_attn_decode(ctypes.byref(_decode()), None) == 6


@pytest.mark.parametrize("kw,status", [
    (dict(q_len=9), 2), (dict(kv_len=1025), 2), (dict(v_codes=None), 1), (dict(k_codes=4104), 3),
    (dict(workspace=None, workspace_bytes=0, num_splits=2, batch=0), 0),          # empty: no-op, no workspace
    # partials beyond the fixed array (64 x 8 x 8 splits x 64 rows x 516 B = 135 MB > 32 MiB)
    (dict(batch=64, q_len=8, kv_len=32768, cap=32768, num_splits=8), 5),
])
def test_decode_noalloc_validation(kw, status):
    a = _decode(**kw)
    a.workspace, a.workspace_bytes = None, 0     # ignored by this entry point
    assert ops.lib().qk4v8_attn_decode_noalloc(ctypes.byref(a), None) == status


def test_noalloc_scratch_size_matches_header():
    src = open(os.path.join(ROOT, "include", "qk4v8.h")).read()
    m = re.search(r"#define QK4V8_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == ops.NOALLOC_SCRATCH_BYTES


def test_append_paging_validation():
    L = ops.lib()
    assert L.qk4v8_kv_append(ctypes.byref(_append(block_table=4096, page_size=200, pages_per_seq=5,
                                                  cap=1000)), None) == 2
    assert L.qk4v8_kv_append(ctypes.byref(_append(block_table=4096, page_size=256, pages_per_seq=3)), None) == 2


def _append(**kw):
    a = ops.AppendArgs()
    a.k_new = a.v_new = a.k_codes = a.k_scales = a.v_codes = a.v_scales = a.v_tail = 4096
    a.k_stride[:] = [8 * 128, 8 * 128, 128]
    a.v_stride[:] = [8 * 128, 8 * 128, 128]
    a.batch, a.kv_heads, a.n_new, a.kv_len, a.cap = 2, 8, 1, 1000, 1024
    a.head_dim, a.v_tile_rows = 128, 256
    for k, v in kw.items():
        if k.endswith("stride"):
            getattr(a, k)[:] = v
        else:
            setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), 2),
    (dict(v_tile_rows=100), 2),
    (dict(n_new=-1), 2),
    (dict(kv_heads=0), 2),
    (dict(kv_len=1020, n_new=8), 2),           # does not fit the capacity
    (dict(kv_len=-1), 2),
    (dict(k_stride=[8 * 128, 8 * 128, 100]), 3),
    (dict(v_stride=[8 * 128, -8, 128]), 3),
    (dict(v_tail=0), 1),
    (dict(k_new=0), 1),
    (dict(v_codes=4100), 3),                   # not 8-byte aligned
    (dict(k_codes=4104), 3),                   # not 16-byte aligned
    (dict(hadamard=-1), 2),
    (dict(n_new=0), 0),                        # no-op
    (dict(batch=0), 0),
])
def test_append_validation(kw, status):
    assert ops.lib().qk4v8_kv_append(ctypes.byref(_append(**kw)), None) == status


C_CALLER = r'''
#include "qk4v8.h"
#include <stdio.h>
#include <string.h>
int main(void) {
  uint16_t x[32] = {0};
  uint8_t codes[16], scales[1];
  qk4v8_decode_args d;
  memset(&d, 0, sizeof d);
  if (qk4v8_abi_version() != QK4V8_ABI_VERSION) return 1;
  if (qk4v8_status_string(QK4V8_ERR_SHAPE) == NULL) return 2;
  if (qk4v8_quantize_qk(x, -1, 32, 32, codes, scales, NULL) != QK4V8_ERR_SHAPE) return 3;
  if (qk4v8_quantize_qk(x, 0, 32, 32, codes, scales, NULL) != QK4V8_OK) return 4;
  if (qk4v8_attn_decode(NULL, NULL) != QK4V8_ERR_NULL) return 5;
  if (qk4v8_attn_decode(&d, NULL) != QK4V8_ERR_SHAPE) return 6;
  printf("abi %d\n", qk4v8_abi_version());
  return 0;
}
'''


def test_header_is_plain_c_and_links(tmp_path):
    """The boundary is a C ABI: a C99 program (gcc, no C++) includes the
    header, links the library and gets the documented statuses back from
    calls that fail validation before any GPU work."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    lib_dir = os.path.dirname(ops._LIB_PATH)
    if not os.path.exists(ops._LIB_PATH):
        pytest.skip("libqk4v8.so not built")
    src, exe = tmp_path / "caller.c", tmp_path / "caller"
    src.write_text(C_CALLER)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
                    "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe), "-L", lib_dir, "-lqk4v8",
                    "-Wl,-rpath," + lib_dir], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert r.stdout.strip() == f"abi {ops.lib().qk4v8_abi_version()}"
