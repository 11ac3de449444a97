"""MI355X-native KV-cached forward of the Qwen3-TTS Talker decoder stack.

The compute lives in ``libqtalk.so`` (HIP kernels for gfx950 behind the C ABI
of ``include/qtalk.h``); ``qwen3_tts_talker_amd.qtalk`` is its Python binding.
"""
from .qtalk import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    QtalkError,
    Talker,
    load_library,
    qtalk_argmax,
    qtalk_argmax_embed,
    qtalk_create,
    qtalk_decode,
    qtalk_decode_batch,
    qtalk_decode_noalloc,
    qtalk_decode_step,
    make_gather,
    qtalk_destroy,
    qtalk_embed_sum,
    qtalk_extend,
    qtalk_kv_len,
    qtalk_kv_read,
    qtalk_kv_rewind,
    qtalk_last_error,
    qtalk_prefill,
    qtalk_prefill_batch,
    qtalk_select_head,
    qtalk_set_wait_limit,
    qtalk_sync,
)
