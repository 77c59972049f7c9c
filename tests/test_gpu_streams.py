"""Calls on different streams, from different host threads, run
concurrently with distinct buffers and give the same bits as the same calls
made one after the other (the library keeps no device state between calls;
its host-side caches of device attributes are guarded by a lock)."""
import threading

import numpy as np
import pytest

from post_weight_quantization_layer_amd import inputs as I
from tests.gpu_harness import gpu_layer, log

pytestmark = pytest.mark.gpu

FIELDS = ("H", "hdiag", "U", "perm", "q", "g_idx", "W_hat")


def _cases():
    a = I.CONFIGS["down_proj_4096x11008_int4_g128_actorder"].with_(rows=96, cols=640,
                                                                  tokens=1500)
    b = I.CONFIGS["q4k_14336x4096"].with_(rows=64, cols=512, tokens=1200)
    c = I.CONFIGS["up_proj_28672x8192_int3_g128_actorder"].with_(rows=80, cols=384, tokens=900)
    out = []
    for cfg in (a, b, c):
        W = I.weight(cfg)
        store = [I.x_chunk_storage(cfg, 0, cfg.tokens)]
        out.append((cfg, W, store))
    return out


def test_layers_on_concurrent_streams_match_sequential():
    import torch
    cases = _cases()
    seq = [gpu_layer(cfg, W, store) for cfg, W, store in cases]
    for rep in range(2):
        results = [None] * len(cases)
        errors = []
        start = threading.Barrier(len(cases))

        def run(i):
            try:
                s = torch.cuda.Stream()            # default priority
                with torch.cuda.stream(s):
                    start.wait()
                    cfg, W, store = cases[i]
                    results[i] = gpu_layer(cfg, W, store)
            except Exception as exc:  # pragma: no cover - reported below
                errors.append(exc)

        threads = [threading.Thread(target=run, args=(i,)) for i in range(len(cases))]
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        assert not errors, errors
        for (cfg, _, _), a, b in zip(cases, seq, results):
            for f in FIELDS:
                np.testing.assert_array_equal(getattr(a, f), getattr(b, f),
                                              err_msg=f"{cfg.name} {f}")
            if cfg.grid == "affine":
                np.testing.assert_array_equal(a.scale, b.scale)
                np.testing.assert_array_equal(a.zero, b.zero)
            else:
                for f in ("D", "Dm", "sc", "mc"):
                    np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
        log(f"[streams] round {rep}: {len(cases)} layers on concurrent streams match")
