"""The allocation-free forward (attn_masked_fwd_noalloc, through the C ABI) against the allocating
one-shot forward (attn_masked_fwd with a caller workspace): the same kernels over the same plan, so
the outputs must be bitwise equal.  Two calls in a row with different masks and shapes (the second
smaller, and on the batched, unsplit schedule), then the first again; plus the refusals (a plan
larger than the static scratch, a workspace passed in)."""

import ctypes

import numpy as np
import pytest
import torch

from block_sparse_softmax_amd import _lib as lib_mod
from block_sparse_softmax_amd import inputs as gen

pytestmark = pytest.mark.gpu


def _tensors(seed, B, H, L, D):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(3):
        bits = gen.f32_to_bf16_bits(rng.standard_normal((B, H, L, D), dtype=np.float32))
        out.append(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda())
    return out


def _call(entry, q, k, v, mask, sink, out, workspace=None):
    lib = lib_mod.load_library()
    qv, kv, vv, ov = (lib_mod.tensor_view(x, "bhld") for x in (q, k, v, out))
    desc, keep = lib_mod.build_desc(mask, qv.H)
    ln = lib_mod.Launch()
    ln.stream = torch.cuda.current_stream().cuda_stream
    if workspace is not None:
        ln.workspace = workspace.data_ptr()
        ln.workspace_bytes = workspace.numel()
    st = getattr(lib, entry)(ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), ctypes.byref(desc),
                             lib_mod._sink_ptr(sink, qv.H), ctypes.byref(ov), ctypes.byref(ln))
    del keep
    return st


def _reference(q, k, v, mask, sink):
    lib = lib_mod.load_library()
    B, H, L, D = q.shape
    desc, keep = lib_mod.build_desc(mask, H)
    n = ctypes.c_size_t()
    assert lib.attn_workspace_bytes(ctypes.byref(desc), L, H, D, ctypes.byref(n)) == 0
    ws = torch.empty(max(256, n.value), dtype=torch.uint8, device=q.device)
    out = torch.empty_like(q)
    assert _call("attn_masked_fwd", q, k, v, mask, sink, out, ws) == 0, lib.attn_last_error()
    torch.cuda.synchronize()
    lib.attn_workspace_release(ctypes.c_void_p(ws.data_ptr()))
    return out


CASES = [
    # (mask, B, H, L, D, sink): batch 1 with split rows, then a smaller batched launch
    (dict(kind="window", causal=True, left=0, right=0, head_left=[99, 699, 2999, 1999]), 1, 4, 3000, 128, True),
    (dict(kind="chunk", chunk=100), 2, 2, 1000, 80, False),
]


def test_noalloc_matches_the_allocating_entry_point():
    lib = lib_mod.load_library()
    results = []
    for i, (mask, B, H, L, D, with_sink) in enumerate(CASES + CASES[:1]):
        print(f"[case] noalloc {i} {mask['kind']} B={B} H={H} L={L} D={D}", flush=True)
        q, k, v = _tensors(10 + (i % len(CASES)), B, H, L, D)
        sink = torch.from_numpy(np.linspace(-1, 1, H).astype(np.float32)).cuda() if with_sink else None
        ref = _reference(q, k, v, mask, sink)
        out = torch.full_like(q, float("nan"))
        assert _call("attn_masked_fwd_noalloc", q, k, v, mask, sink, out) == 0, lib.attn_last_error()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"case {i}: outputs differ"
        results.append(out)
    assert torch.equal(results[0], results[2])          # the scratch switched back to the first plan


def test_noalloc_refusals():
    lib = lib_mod.load_library()
    q, k, v = _tensors(3, 1, 2, 512, 64)
    out = torch.empty_like(q)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=q.device)
    assert _call("attn_masked_fwd_noalloc", q, k, v, dict(kind="full"), None, out, ws) == lib_mod.ATTN_E_INVAL
    # 16 heads x 512 query tiles x 1024 key tiles of list entries: far above the 32 MiB scratch
    big = torch.empty((1, 16, 65536, 64), dtype=torch.bfloat16, device=q.device)
    st = _call("attn_masked_fwd_noalloc", big, big, big, dict(kind="full"), None, torch.empty_like(big))
    assert st == lib_mod.ATTN_E_WORKSPACE
    assert b"bytes of scratch" in lib.attn_last_error()
