"""GPU parity of one-query decode attention (attn_decode_fwd, through the C ABI) against the float64
decode oracle.

Caches hold NaN in every row a case does not fill (bf16 0x7FC0): a read of any key outside the query's
window / prefix set, or a wrong clamp of a ragged tile, would show up as NaN in the output.  Bar: the
forward's (max-abs <= 2e-2 and relative Frobenius <= 5e-3 over every compared row).  Small cases cover
head dims 64/128/256, 1/4/16 query heads per cache head, windows (none, 1, 64, 200), prefix tokens,
sinks, ragged lengths (1 .. Lmax), zero-length and over-long sequences, both cache layouts, and the
split path (keys of one sequence spread over many work-groups, merged by the second kernel); the decode
workloads of bench.py are compared on sampled sequences in the launch configuration bench.py times.
"""

import numpy as np
import pytest
import torch

from block_sparse_softmax_amd import inputs as gen
from oracle.decode import decode_attention

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
REL_FROB = 5e-3
NAN_BF16 = 0x7FC0


def _bits(t_u16, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(t_u16).view(np.int16)).view(torch.bfloat16).to(device)


def _host_caches(cfg, B, Hkv, Lmax, D, lens, head_rows, tail_rows):
    """Dense host caches [B, Hkv, Lmax, D] (bf16 bits): the generator's rows, NaN elsewhere."""
    k = np.full((B, Hkv, Lmax, D), NAN_BF16, np.uint16)
    v = np.full((B, Hkv, Lmax, D), NAN_BF16, np.uint16)
    for b in range(B):
        pos, kr, vr = gen.decode_cache_rows(0, cfg, b, min(int(lens[b]), Lmax), Hkv, D, head_rows, tail_rows)
        k[b][:, pos] = kr
        v[b][:, pos] = vr
    return k, v


def _run(q, k, v, lens, max_len, window, prefix, sink, layout="blhd"):
    from block_sparse_softmax_amd import decode_fwd
    qd = _bits(q)
    if layout == "blhd":
        kd, vd = _bits(k.transpose(0, 2, 1, 3)), _bits(v.transpose(0, 2, 1, 3))
    else:
        kd, vd = _bits(k), _bits(v)
    ld = torch.as_tensor(np.asarray(lens, np.int32)).cuda()
    sd = None if sink is None else torch.as_tensor(np.asarray(sink, np.float32)).cuda()
    out = decode_fwd(qd, kd, vd, ld, max_len, window=window, prefix=prefix, sink=sd, layout=layout)
    torch.cuda.synchronize()
    return out.float().cpu().double().numpy()


def _compare(got, ref, what):
    assert np.all(np.isfinite(got)), what
    err = np.abs(got - ref)
    max_abs = float(err.max())
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / nref) if nref > 0 else max_abs
    print(f"[decode parity] {what}: max_abs={max_abs:.3e} rel_frob={rel:.3e}", flush=True)
    assert max_abs <= MAX_ABS, (what, max_abs)
    assert rel <= REL_FROB, (what, rel)


CASES = [  # D, Hkv, G, window, prefix, sink
    (64, 2, 1, 0, 0, False),
    (64, 2, 16, 64, 4, True),
    (64, 1, 4, 1, 0, True),
    (128, 2, 4, 0, 0, True),
    (128, 2, 4, 200, 0, True),
    (128, 2, 4, 64, 4, False),
    (128, 3, 2, 1, 3, False),
    (256, 2, 4, 0, 0, False),
    (256, 2, 4, 200, 4, True),
]


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_small_cases(ci):
    D, Hkv, G, window, prefix, with_sink = CASES[ci]
    H, Lmax = Hkv * G, 700
    lens = np.array([1, 37, 333, 700, 64, 65], np.int32)
    B = len(lens)
    cfg = 100 + ci
    print(f"[decode] case {CASES[ci]}", flush=True)
    q = gen.decode_queries(0, cfg, B, H, D)
    tail = window if window > 0 else Lmax
    k, v = _host_caches(cfg, B, Hkv, Lmax, D, lens, prefix, tail)
    sink = gen.head_sinks(0, cfg, H) if with_sink else None
    for layout in ("blhd", "bhld"):
        got = _run(q, k, v, lens, Lmax, window, prefix, sink, layout)
        ref = decode_attention(q, k, v, lens, window, prefix, sink=sink)["out"]
        _compare(got, ref, f"{CASES[ci]} {layout}")


@pytest.mark.parametrize("window,prefix,B,Hkv,Lmax,D,G", [(0, 0, 1, 2, 20000, 128, 4), (5000, 4, 2, 1, 9000, 128, 4),
                                                       (0, 0, 1, 1, 12000, 256, 8), (3000, 2, 1, 2, 7000, 64, 2)])
def test_split_path(window, prefix, B, Hkv, Lmax, D, G):
    """Few sequences x heads: one sequence's keys spread over many work-groups, merged in split order."""
    H = Hkv * G
    cfg = 120 + Hkv + D
    lens = np.array([Lmax - 17, Lmax][:B], np.int32)
    print(f"[decode] split path window={window} prefix={prefix} B={B} Lmax={Lmax} D={D} G={G}", flush=True)
    q = gen.decode_queries(0, cfg, B, H, D)
    k, v = _host_caches(cfg, B, Hkv, Lmax, D, lens, prefix, window if window > 0 else Lmax)
    sink = gen.head_sinks(0, cfg, H)
    got = _run(q, k, v, lens, Lmax, window, prefix, sink)
    ref = decode_attention(q, k, v, lens, window, prefix, sink=sink)["out"]
    _compare(got, ref, f"split window={window}")


def test_zero_and_clamped_lengths():
    D, Hkv, G, Lmax, max_len = 128, 2, 4, 512, 300
    H = Hkv * G
    lens = np.array([0, 900, 300, 5], np.int32)      # 900 > max_len: treated as max_len
    eff = np.minimum(lens, max_len)
    q = gen.decode_queries(0, 130, len(lens), H, D)
    k, v = _host_caches(130, len(lens), Hkv, Lmax, D, eff, 2, 100)
    sink = gen.head_sinks(0, 130, H)
    got = _run(q, k, v, lens, max_len, 100, 2, sink)
    ref = decode_attention(q, k, v, eff, 100, 2, sink=sink)["out"]
    assert np.all(got[0] == 0)
    _compare(got, ref, "zero / clamped lengths")


def test_deterministic():
    D, Hkv, G, Lmax = 128, 1, 4, 6000
    H = Hkv * G
    lens = np.array([Lmax], np.int32)
    q = gen.decode_queries(0, 131, 1, H, D)
    k, v = _host_caches(131, 1, Hkv, Lmax, D, lens, 0, Lmax)
    a = _run(q, k, v, lens, Lmax, 0, 0, None)
    b = _run(q, k, v, lens, Lmax, 0, 0, None)
    assert np.array_equal(a, b)


def _device_caches(w, device):
    """The bench's caches: NaN everywhere, the generator's rows of every sequence scattered in."""
    B, Hkv, D, L = w["B"], w["Hkv"], w["D"], w["Lmax"]
    kc = torch.full((B, L, Hkv, D), float("nan"), dtype=torch.bfloat16, device=device)
    vc = torch.full((B, L, Hkv, D), float("nan"), dtype=torch.bfloat16, device=device)
    tail = w["window"] if w["window"] > 0 else L
    for b in range(B):
        pos, kr, vr = gen.decode_cache_rows(0, w["cfg"], b, int(w["lens"][b]), Hkv, D, w["prefix"], tail)
        idx = torch.as_tensor(pos, device=device)
        kc[b].index_copy_(0, idx, _bits(kr.transpose(1, 0, 2), device))
        vc[b].index_copy_(0, idx, _bits(vr.transpose(1, 0, 2), device))
    return kc, vc


@pytest.mark.parametrize("name", gen.DECODE_WORKLOADS)
def test_decode_workloads_sampled(name):
    from block_sparse_softmax_amd import PreparedDecode
    w = gen.decode_workload(name)
    B, H, Hkv, D, L = w["B"], w["H"], w["Hkv"], w["D"], w["Lmax"]
    print(f"[decode] workload {name}", flush=True)
    q = gen.decode_queries(0, w["cfg"], B, H, D)
    kc, vc = _device_caches(w, "cuda")
    qd = _bits(q)
    ld = torch.as_tensor(w["lens"]).cuda()
    sd = None if w["sink"] is None else torch.as_tensor(w["sink"]).cuda()
    out = torch.empty_like(qd)
    pd = PreparedDecode(qd, kc, L, w["window"], w["prefix"])
    pd.bind(qd, kc, vc, ld, out, sink=sd)()
    torch.cuda.synchronize()
    got = out.float().cpu().double().numpy()
    del kc, vc
    torch.cuda.empty_cache()
    pick = sorted(set(np.random.default_rng([0, w["cfg"], 99]).choice(B, size=min(B, 6), replace=False).tolist()))
    tail = w["window"] if w["window"] > 0 else L
    for b in pick:
        n = int(w["lens"][b])
        pos, kr, vr = gen.decode_cache_rows(0, w["cfg"], b, n, Hkv, D, w["prefix"], tail)
        kb = np.full((Hkv, n, D), NAN_BF16, np.uint16)
        vb = np.full((Hkv, n, D), NAN_BF16, np.uint16)
        kb[:, pos], vb[:, pos] = kr, vr
        ref = decode_attention(q, {b: kb}, {b: vb}, w["lens"], w["window"], w["prefix"], sink=w["sink"],
                               batches=[b])["out"]
        _compare(got[b], ref[b], f"{name} sequence {b} (n={n})")
