"""GPU parity at the full sizes of the larger workloads, on sampled decode
steps: the Llama-3-8B shape (2048-token context) and the Llama-3.2-1B shape
with a 32768-token context; and the Llama-2/3-70B widths (hidden 8192, 64
query heads x 128, 8 KV heads, FFN 28672, vocab 128256, 4096-token context)
with 2 of the 80 layers (the per-layer code and geometry do not depend on the
layer count), weights loaded a layer at a time.  Both sides start from the same synthetic cache
prefix (an fp64 oracle prefill of thousands of positions is too slow for a
test); the step itself -- append, attention over the whole cache, every
layer, the LM head -- is compared element by element at the 2e-2 bar."""
import pytest

import synth

from test_gpu_parity import env, run_pair  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu


def test_llama8b_full_size(env):
    cfg = synth.CONFIGS["llama8b"]
    errs, agree = run_pair(env, cfg, seed=21, n_prompt=cfg.context, n_steps=2, gains="ones", use_prefill=False)
    assert max(errs) <= 2e-2 and agree == 2


def test_llama1b_32k_context(env):
    cfg = synth.CONFIGS["llama1b_32k"]
    errs, agree = run_pair(env, cfg, seed=22, n_prompt=cfg.context, n_steps=2, gains="ones", use_prefill=False)
    assert max(errs) <= 2e-2 and agree == 2


def test_llama70b_widths_two_layers(env):
    cfg = synth.CONFIGS["llama70b"].with_(n_layers=2)
    errs, agree = run_pair(env, cfg, seed=23, n_prompt=cfg.context, n_steps=2, gains="ones", use_prefill=False,
                           deferred=True)
    assert max(errs) <= 2e-2 and agree == 2
