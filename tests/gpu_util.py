"""Helpers shared by the GPU tests: device upload, one readout call through
the C-ABI, and the oracle's answer on the same host buffers."""
from __future__ import annotations

import os
import sys

import numpy as np

import oracle

ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))


def say(msg: str):
    """Name the GPU step about to run, flushed, so a crash still shows it."""
    sys.stdout.write("[gpu] %s\n" % msg)
    sys.stdout.flush()


def to_dev(a: np.ndarray):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(a).cuda()


def oracle_blk(base, bias, blk0, N, B, V, sb, sbi):
    """Expected blk: the oracle's per-row answers scattered into a copy of blk0."""
    rows = N * (B - 1)
    out = blk0.copy()
    if rows == 0:
        return out
    idx = oracle.add_argmax_rows_threaded(base, bias, rows, V, sb, sbi, ORACLE_THREADS)
    out[:, 1:] = idx.reshape(N, B - 1)
    return out


def gpu_blk(base_d, bias_d, blk0, N, B, V, sb, sbi, stream=None):
    """Run the readout on device copies and return blk on the host."""
    import torch
    from vocab_wide_add_amd import native
    blk_d = to_dev(blk0)
    native.xpress_add_argmax_to_blk(base_d, bias_d, blk_d, N, B, V, sb, sbi, stream=stream)
    torch.cuda.synchronize()
    return blk_d.cpu().numpy()


class Plan:
    """Context manager: force a combine / split count / block size."""

    def __init__(self, combine=0, splits=0, threads=0):
        self.args = (combine, splits, threads)

    def __enter__(self):
        from vocab_wide_add_amd import native
        native.xpress_set_plan(*self.args)
        return self

    def __exit__(self, *exc):
        from vocab_wide_add_amd import native
        native.xpress_set_plan(0, 0, 0)
        return False
