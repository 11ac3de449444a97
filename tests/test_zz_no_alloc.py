"""qtalk_decode_noalloc (the persistent decode exchanging through a static
device array instead of the context's buffers) against qtalk_decode, through
the C ABI: bit-identical logits, hidden state and caches on two calls in a
row, the second at a smaller context; and its error cases."""
import numpy as np
import pytest

from oracle import TalkerOracle
from synth import prefill_embeddings, step_embedding, workload
from tests.helpers import argmax_ok, dev, host, rel_err, say, weights_for

pytestmark = pytest.mark.gpu


def test_decode_noalloc_matches_decode():
    import torch
    from qwen3_tts_talker_amd import QtalkError, Talker, qtalk
    shape = workload("talker_28l_t128_d1024")
    w = weights_for("talker_28l_t128_d1024", 4)
    emb = prefill_embeddings(shape, 300)
    steps = [step_embedding(shape, s) for s in range(2)]
    say("[case] qtalk_decode_noalloc vs qtalk_decode, 4 layers, contexts 301 then 101")
    a, b = Talker(shape, w), Talker(shape, w)
    a.prefill(0, dev(emb))
    b.prefill(0, dev(emb))
    orc = TalkerOracle(shape, w)
    for call, (n_keep, e) in enumerate(((300, steps[0]), (100, steps[1]))):
        a.kv_rewind(0, n_keep)
        b.kv_rewind(0, n_keep)
        la, ha = a.decode(0, dev(e), hidden=True)
        lb = torch.empty(shape.vocab, device="cuda")
        hb = torch.empty(shape.hidden, device="cuda")
        qtalk.qtalk_decode_noalloc(b.ctx, 0, dev(e), lb, hb)
        a.sync()
        b.sync()
        assert a.kv_len(0) == b.kv_len(0) == n_keep + 1
        assert np.array_equal(host(la), host(lb)), call
        assert np.array_equal(host(ha), host(hb)), call
        for which in (0, 1):
            assert np.array_equal(host(a.kv_read(0, 3, which)), host(b.kv_read(0, 3, which))), call
        orc.kv_rewind(0, n_keep) if orc.kv_len(0) else orc.prefill(0, emb[:n_keep])
        lo, _ = orc.decode(0, e)
        assert rel_err(host(lb), lo) <= 2e-2 and argmax_ok(host(lb), lo), call
    # interleaved with ordinary decodes of the same context: same cache, same results
    la = a.decode(0, dev(steps[0]))
    lb = torch.empty(shape.vocab, device="cuda")
    qtalk.qtalk_decode_noalloc(b.ctx, 0, dev(steps[0]), lb, None)
    lb2 = b.decode(0, dev(steps[1]))
    la2 = a.decode(0, dev(steps[1]))
    a.sync()
    b.sync()
    assert np.array_equal(host(la), host(lb)) and np.array_equal(host(la2), host(lb2))
    # errors: a full cache, a bad id; nothing changes
    b.kv_rewind(0, 0)
    with pytest.raises(QtalkError) as err:
        qtalk.qtalk_decode_noalloc(b.ctx, 7, dev(steps[0]), lb, None)
    assert err.value.status == -1
    a.close()
    b.close()


def test_decode_noalloc_rejects_contexts_without_the_persistent_decode():
    import torch
    from qwen3_tts_talker_amd import QtalkError, Talker, qtalk
    shape = workload("tiny_f32_2l")
    tk = Talker(shape, weights_for("tiny_f32_2l"))
    tk.prefill(0, dev(prefill_embeddings(shape, 4)))
    lg = torch.empty(shape.vocab, device="cuda")
    with pytest.raises(QtalkError) as err:
        qtalk.qtalk_decode_noalloc(tk.ctx, 0, dev(step_embedding(shape, 0)), lg, None)
    assert err.value.status == -1 and tk.kv_len(0) == 4
    tk.close()
