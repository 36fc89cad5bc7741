"""spd_prefill_static_scratch against spd_prefill, through the C ABI (needs an MI355X).

The allocation-free entry point runs the same prefill with its chunk buffers in the
library's static device array, so it processes the prompt in smaller chunks (144 rows at
d2560 instead of 512). Every output row's arithmetic is independent of the chunking, so
the two must agree bit for bit: first token, target logits, the target and PDM KV caches
over the prompt, the residual ring; and a few pipeline steps taken afterwards must commit
the same records. Two calls in a row on the same handles, the second with a shorter
prompt (the array keeps the first call's contents).
"""
import numpy as np
import pytest

from conftest import workload

pytestmark = pytest.mark.gpu

_dev = {}


def _weights(name):
    import torch
    from speculative_pipeline_decoding_amd import upload_weights
    if name not in _dev:
        _dev.clear()
        torch.cuda.empty_cache()
        cfg, W, _ = workload(name)
        _dev[name] = upload_weights(cfg, W)
    return _dev[name]


def _kv(gpu, what, cfg, layers, P):
    a = gpu.debug(what).reshape(layers, 2, cfg.n_kv_heads, cfg.max_ctx, cfg.head_dim)
    return a[:, :, :, :P, :]


def _state(gpu, cfg, P):
    nsoft = sum(1 for k in cfg.kinds if k == 0)
    return {"logits": gpu.debug("target_logits"), "target_kv": _kv(gpu, "target_kv", cfg, nsoft, P),
            "pdm_kv": _kv(gpu, "pdm_kv", cfg, cfg.pdm_layers, P)}


@pytest.mark.parametrize("name,T", [("tiny", 0.0), ("mid_bf16_L6_d384_n3", 1.0),
                                    ("dense_bf16_L32_d2560_n8_ctx2048", 1.0)])
def test_static_scratch_prefill_matches_prefill(name, T):
    from speculative_pipeline_decoding_amd import SPD
    cfg, _, prompt = workload(name)
    dW = _weights(name)
    ref = SPD(cfg, dW, temperature=T, seed=7)
    new = SPD(cfg, dW, temperature=T, seed=7)
    try:
        for call, plen in enumerate((len(prompt), len(prompt) // 3 + 1)):
            print(f"[no-alloc] {name} call {call + 1}: {plen}-token prompt", flush=True)
            if call:
                ref.reset()
                new.reset()
            p = prompt[:plen]
            t_ref = ref.prefill(p)
            t_new = new.prefill_static_scratch(p)
            assert t_new == t_ref
            a, b = _state(ref, cfg, plen), _state(new, cfg, plen)
            for k in a:
                assert np.array_equal(a[k], b[k]), f"call {call + 1}: {k} differs"
            for step in range(2 * cfg.n_stages + 2):
                ref.step()
                new.step()
                ca, cb = ref.verify_commit().as_dict(), new.verify_commit().as_dict()
                assert ca == cb, f"call {call + 1}, step {step}: {ca} != {cb}"
    finally:
        ref.close()
        new.close()
