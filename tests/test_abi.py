"""The C-ABI library loads, exports what include/qtalk.h declares, agrees with
the binding's struct layouts, and rejects bad arguments before touching the
GPU (CPU only: no compute call is made)."""
import ctypes
import os
import re
import subprocess

import pytest

from qwen3_tts_talker_amd import qtalk as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qtalk.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qtalk_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = q.load_library()
    names = declared_functions()
    assert len(names) == 19, names
    assert sorted(q.EXPORTS) == names
    for n in names:
        assert hasattr(lib, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", q.LIB_PATH],
                        stdout=subprocess.PIPE, text=True, check=True).stdout
    exported = sorted(set(re.findall(r" T (qtalk_\w+)", nm)))
    assert exported == names


def test_struct_layouts_match_the_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text("""
#include <stddef.h>
#include <stdio.h>
#include "qtalk.h"
#define F(T, f) printf(#T "." #f " %zu\\n", offsetof(T, f))
int main(void) {
  printf("qtalk_config %zu\\n", sizeof(qtalk_config));
  printf("qtalk_layer_weights %zu\\n", sizeof(qtalk_layer_weights));
  printf("qtalk_weights %zu\\n", sizeof(qtalk_weights));
  F(qtalk_config, rms_eps); F(qtalk_config, rope_theta);
  F(qtalk_config, max_seq_len); F(qtalk_config, kv_dtype);
  F(qtalk_config, n_output_heads);
  F(qtalk_layer_weights, down_proj); F(qtalk_layer_weights, k_norm);
  F(qtalk_weights, final_norm); F(qtalk_weights, codec_head);
  printf("qtalk_gather %zu\\n", sizeof(qtalk_gather));
  F(qtalk_gather, tables); F(qtalk_gather, table_rows); F(qtalk_gather, ids);
  F(qtalk_gather, overlay);
  return 0;
}
""")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.dirname(HEADER), str(src), "-o",
                    str(exe)], check=True)
    got = dict(l.rsplit(" ", 1) for l in subprocess.run(
        [str(exe)], stdout=subprocess.PIPE, text=True, check=True
    ).stdout.splitlines())
    assert int(got["qtalk_config"]) == ctypes.sizeof(q.qtalk_config)
    assert int(got["qtalk_layer_weights"]) == ctypes.sizeof(q.qtalk_layer_weights)
    assert int(got["qtalk_weights"]) == ctypes.sizeof(q.qtalk_weights)
    assert int(got["qtalk_gather"]) == ctypes.sizeof(q.qtalk_gather)
    for key, val in got.items():
        if "." in key:
            st, f = key.split(".")
            assert getattr(getattr(q, st), f).offset == int(val), key


def _config(**kw):
    base = dict(n_layers=1, hidden=256, n_heads=4, n_kv_heads=2, head_dim=64,
                intermediate=768, vocab=3072, rms_eps=1e-6, rope_theta=1e6,
                max_seq_len=64, max_seqs=1, weight_dtype=q.QTALK_F32,
                kv_dtype=q.QTALK_F32)
    base.update(kw)
    return q.qtalk_config(**base)


@pytest.mark.parametrize("bad", [dict(head_dim=96), dict(n_kv_heads=3),
                                 dict(hidden=100), dict(max_seq_len=0),
                                 dict(weight_dtype=q.QTALK_F16),
                                 dict(kv_dtype=q.QTALK_BF16),
                                 dict(n_heads=12, n_kv_heads=4),
                                 dict(n_output_heads=-1),
                                 dict(n_output_heads=65),
                                 dict(hidden=8256), dict(intermediate=8256),
                                 dict(n_heads=130, n_kv_heads=2)])
def test_create_rejects_bad_config_before_any_device_call(bad):
    lib = q.load_library()
    w = q.qtalk_weights()
    out = ctypes.c_void_p(123)
    s = lib.qtalk_create(ctypes.byref(_config(**bad)), ctypes.byref(w), None,
                         ctypes.byref(out))
    assert s == q.QTALK_E_INVAL
    assert out.value is None


def test_null_context_calls_are_rejected():
    lib = q.load_library()
    assert lib.qtalk_kv_len(None, 0) == -1
    assert lib.qtalk_prefill(None, 0, None, 1, None, None) == q.QTALK_E_INVAL
    assert lib.qtalk_decode(None, 0, None, None, None) == q.QTALK_E_INVAL
    assert lib.qtalk_kv_rewind(None, 0, 0) == q.QTALK_E_INVAL
    assert lib.qtalk_sync(None) == q.QTALK_E_INVAL
    assert lib.qtalk_select_head(None, 0) == q.QTALK_E_INVAL
    assert lib.qtalk_set_wait_limit(None, 0) == q.QTALK_E_INVAL
    assert lib.qtalk_decode_noalloc(None, 0, None, None, None) == q.QTALK_E_INVAL
    assert lib.qtalk_decode_step(None, 0, None, None, None, None, 0, -1, None) == q.QTALK_E_INVAL
    assert lib.qtalk_embed_sum(None, 1, None, None, None, 1, None, None) == q.QTALK_E_INVAL
    assert lib.qtalk_argmax(None, None, 1, 8, 8, -1, None) == q.QTALK_E_INVAL
    assert lib.qtalk_argmax_embed(None, None, 1, 8, 8, -1, None, 4, None, None) == q.QTALK_E_INVAL
    assert lib.qtalk_last_error(None) == b"null context"
    lib.qtalk_destroy(None)
    # missing weights are rejected before any allocation
    s = lib.qtalk_create(ctypes.byref(_config()), None, None,
                         ctypes.byref(ctypes.c_void_p()))
    assert s == q.QTALK_E_INVAL
