"""The measured-ceiling kernels (awq_ceiling_mfma, awq_ceiling_stream) that
the bench reports every kernel against: the copy moves every byte, the write
kernel writes its documented pattern, and the matrix-core and read kernels
run and give positive rates."""

import numpy as np
import torch

import post_weight_quantization_stats_amd as awq
from gpu_util import announce, require_gpu

import pytest

pytestmark = pytest.mark.gpu


def test_stream_ceilings_move_the_bytes():
    dev = require_gpu()
    announce("ceiling kernels: copy, read, write")
    for nbytes, blocks in ((16, 1), (4096 + 16, 1024), ((1 << 24) + 48, 65536), ((1 << 24) + 48, 7),
                           ((1 << 24) + 48, (1 << 22) + 3)):
        src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=dev)
        dst = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        awq.ceiling_stream(awq.CEILING_COPY, src, dst, nbytes, blocks)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        awq.ceiling_stream(awq.CEILING_READ, src, sink, nbytes, blocks)
        out = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        awq.ceiling_stream(awq.CEILING_WRITE, None, out, nbytes, blocks)
        torch.cuda.synchronize()
        assert torch.equal(dst, src), nbytes
        words = out.cpu().numpy().view(np.uint32).reshape(-1, 4)
        i = np.arange(words.shape[0], dtype=np.uint32)
        want = np.stack([i, i ^ 1, i ^ 2, i ^ 3], axis=1)
        assert np.array_equal(words, want), nbytes


def test_mfma_ceiling_runs_and_counts_flops():
    dev = require_gpu()
    announce("ceiling kernel: matrix cores")
    sink = torch.zeros(4, dtype=torch.float32, device=dev)
    flops = awq.ceiling_mfma(sink, 8, 16)
    assert flops == 8 * 8 * 16 * 32 * 16 * 16 * 32 * 2
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    awq.ceiling_mfma(sink, 256, 200)
    awq.ceiling_mfma(sink, 256, 200, zero=True)
    end.record()
    end.synchronize()
    assert start.elapsed_time(end) > 0
    assert torch.all(sink == 0)
