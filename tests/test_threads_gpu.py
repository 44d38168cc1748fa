"""Library calls from several host threads at once, each thread on its own
stream, each shape on a different tile kernel (256x256 8-wave, 128x128
8-wave, 128x128 at two blocks per CU, the general kernel): every thread's
output must equal, byte for byte, the same call made alone.  The first
calls of a kernel on a device set its dynamic-LDS limit and fill the
per-device caches, which the threads may race to do."""

import threading

import numpy as np
import pytest
import torch

import scaled_quantize_fp8_amd as F
from tests.gpu_util import DEV

pytestmark = pytest.mark.gpu

# (M, N, K): 2048x4096x1536 -> 256x256, 2048x1536x1536 -> 8-wave 128x128,
# 2048x1024x1024 -> 128x128 at two blocks per CU, 200x136x200 -> general
SHAPES = [(2048, 4096, 1536), (2048, 1536, 1536), (2048, 1024, 1024), (200, 136, 200)]


def _operands(M, N, K, seed):
    rng = np.random.default_rng(seed)
    ok = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    a = torch.from_numpy(rng.choice(ok, size=(M, K))).to(DEV)
    b = torch.from_numpy(rng.choice(ok, size=(N, K))).to(DEV)
    bias = torch.from_numpy(rng.standard_normal(N).astype(np.float32)).to(torch.bfloat16).to(DEV)
    return a, b, bias


def _call(a, b, bias, y, stream):
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    F.fp8_linear_fwd(F.Quantized(a, F.FP8_E4M3, one), F.Quantized(b, F.FP8_E4M3, one), bias,
                     F.FP8_E4M3, y, stream=stream)


def test_concurrent_host_threads_match_single_calls():
    ops = [_operands(M, N, K, 100 + i) for i, (M, N, K) in enumerate(SHAPES)]
    outs = [torch.empty(M, N, dtype=torch.bfloat16, device=DEV) for M, N, _ in SHAPES]
    refs = [torch.empty_like(o) for o in outs]
    streams = [torch.cuda.Stream() for _ in SHAPES]
    torch.cuda.synchronize()
    barrier = threading.Barrier(len(SHAPES))
    errors = []

    def work(i):
        try:
            torch.cuda.set_device(0)
            barrier.wait()
            for _ in range(3):
                _call(*ops[i], outs[i], streams[i])
            streams[i].synchronize()
        except Exception as exc:  # reported below, with the thread's shape
            errors.append((SHAPES[i], repr(exc)))

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(SHAPES))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    for i in range(len(SHAPES)):  # the same calls, one at a time
        _call(*ops[i], refs[i], streams[i])
        streams[i].synchronize()
        assert torch.equal(outs[i].view(torch.int16), refs[i].view(torch.int16)), SHAPES[i]
