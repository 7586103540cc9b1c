"""The checked build (libbss_attn_checked.so: the forward kernels with range checks on their work items,
listed key tiles and pointers).  On valid launches it writes exactly what the normal build writes and
reports no violation; on a device image whose list entry or work item was overwritten with an
out-of-range value, the kernel's checks report the violation and the work-group returns without
using it."""

import contextlib
import ctypes
import gc
import os

import numpy as np
import pytest
import torch

from block_sparse_softmax_amd import _lib
from block_sparse_softmax_amd.build import LIB_CHECKED

pytestmark = pytest.mark.gpu

CASES = [
    # (mask, L, H, Hkv, D, B): one per forward kernel, batch 1 (split rows) and 2
    (dict(kind="full"), 700, 2, 2, 80, 2),
    (dict(kind="window", left=300, right=0, causal=True), 1800, 2, 2, 128, 1),
    (dict(kind="full"), 2200, 2, 2, 128, 1),
    (dict(kind="window", left=575, right=0, causal=True), 1500, 16, 4, 256, 1),
]


@contextlib.contextmanager
def _library(path):
    """Run the body against another build of the library (objects made inside must die inside)."""
    old = _lib._lib
    _lib._lib = None
    try:
        yield _lib.load_library(path)
    finally:
        gc.collect()
        _lib._lib = old


def _inputs(seed, B, H, Hkv, L, D):
    g = torch.Generator(device="cuda").manual_seed(seed)
    q = torch.randn((B, H, L, D), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((B, Hkv, L, D), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((B, Hkv, L, D), generator=g, device="cuda").to(torch.bfloat16)
    sink = torch.randn(H, generator=g, device="cuda")
    return q, k, v, sink


def _run(mask, q, k, v, sink):
    B, H, L, D = q.shape
    pm = _lib.PreparedMask(mask, L, H, D, q.device)
    o = torch.full_like(q, float("nan"))
    pm.launch(q, k, v, o, sink=sink, layout="bhld")
    torch.cuda.synchronize()
    kind = pm.plan.kernel()
    del pm
    return o, kind


def test_normal_build_has_no_checks():
    enabled, bits = _lib.checks()
    assert not enabled and bits == 0


@pytest.mark.skipif(not os.path.exists(LIB_CHECKED), reason="checked build missing")
@pytest.mark.parametrize("ci", range(len(CASES)))
def test_checked_build_matches_and_reports_nothing(ci):
    mask, L, H, Hkv, D, B = CASES[ci]
    q, k, v, sink = _inputs(40 + ci, B, H, Hkv, L, D)
    print(f"[case] checked {mask} L={L} H={H}/{Hkv} D={D} B={B}", flush=True)
    ref, kind = _run(mask, q, k, v, sink)
    with _library(LIB_CHECKED):
        assert _lib.checks(clear=True)[0]
        got, kind_c = _run(mask, q, k, v, sink)
        enabled, bits = _lib.checks()
    assert enabled and bits == 0, bits
    assert kind == kind_c
    assert torch.equal(got, ref), kind


def _find(hay: np.ndarray, needle: np.ndarray) -> list:
    """Byte offsets of needle's bytes inside hay's (at least one; the split and unsplit schedules are
    the same array when no row is split, and the image holds both)."""
    hb, nb = hay.tobytes(), needle.tobytes()
    found, at = [], hb.find(nb)
    while at >= 0:
        found.append(at)
        at = hb.find(nb, at + 1)
    assert found
    return found


@pytest.mark.skipif(not os.path.exists(LIB_CHECKED), reason="checked build missing")
def test_checked_build_reports_planted_violations():
    mask, L, H, D = dict(kind="window", left=300, right=0, causal=True), 1800, 2, 128
    q, k, v, sink = _inputs(77, 1, H, H, L, D)
    ref, _ = _run(mask, q, k, v, sink)
    with _library(LIB_CHECKED):
        _lib.checks(clear=True)
        pm = _lib.PreparedMask(mask, L, H, D, q.device)
        _, _, _, kv_tile, flags = pm.plan.tiles()
        entries = ((kv_tile.astype(np.int32) << 1) | flags.astype(np.int32)).astype(np.int32)
        items = pm.plan.schedule().astype(np.int32)
        image = pm.workspace.cpu().numpy()
        (off_kv,) = _find(image, entries)
        offs_items = _find(image, items)
        nk = -(-L // 64)
        o = torch.empty_like(q)
        print("[case] planted: key tile past the sequence", flush=True)
        j = len(entries) // 2
        bad = np.array([(nk + 3) << 1], np.int32).view(np.uint8)
        pm.workspace[off_kv + 4 * j: off_kv + 4 * j + 4] = torch.from_numpy(bad).cuda()
        pm.launch(q, k, v, o, sink=sink, layout="bhld")
        torch.cuda.synchronize()
        assert _lib.checks(clear=True)[1] == 16
        print("[case] planted: list range past the entries", flush=True)
        pm.plan.upload(pm.workspace)                     # the clean image again
        r = int(np.nonzero(items[:, 0] >= 0)[0][0])
        bad = np.array([len(entries) + 100], np.int32).view(np.uint8)
        for off_items in offs_items:
            at = off_items + 4 * (8 * r + 3)
            pm.workspace[at: at + 4] = torch.from_numpy(bad).cuda()
        pm.launch(q, k, v, o, sink=sink, layout="bhld")
        torch.cuda.synchronize()
        assert _lib.checks(clear=True)[1] == 4
        print("[case] clean image", flush=True)
        pm.plan.upload(pm.workspace)
        pm.launch(q, k, v, o, sink=sink, layout="bhld")
        torch.cuda.synchronize()
        assert _lib.checks(clear=True)[1] == 0
        assert torch.equal(o, ref)
        del pm
