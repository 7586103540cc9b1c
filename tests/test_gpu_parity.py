"""GPU parity: the HIP kernel (through the C ABI) against the float64 oracle.

Bar (bf16 inputs, fp32 accumulation): max-abs error <= 2e-2 and relative
Frobenius error <= 5e-3 over the evaluated rows of all heads.  Small cases
compare every row and span several tiles plus a ragged tail; the 16K-token
and 128K-token workloads compare 512 seeded sampled rows per head of the
launch that bench.py times.
"""

import numpy as np
import pytest
import torch

from block_sparse_softmax_amd import inputs as gen
from oracle.attention import attention

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
REL_FROB = 5e-3


def _bits_to_bf16(u16: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).to(device)


def _to_blhd(t_bhld: torch.Tensor) -> torch.Tensor:
    return t_bhld.permute(0, 2, 1, 3).contiguous()


def _run_gpu(q, k, v, mask, sink=None, layout="blhd", oneshot=False):
    from block_sparse_softmax_amd import masked_fwd, masked_fwd_oneshot
    qt, kt, vt = (_bits_to_bf16(x) for x in (q, k, v))
    if layout == "blhd":
        qt, kt, vt = _to_blhd(qt), _to_blhd(kt), _to_blhd(vt)
    st = None if sink is None else torch.as_tensor(np.asarray(sink, np.float32)).cuda()
    fn = masked_fwd_oneshot if oneshot else masked_fwd
    o = fn(qt, kt, vt, mask, sink=st, layout=layout)
    torch.cuda.synchronize()
    if layout == "blhd":
        o = o.permute(0, 2, 1, 3)
    return o.float().cpu().double().numpy()     # [B, H, L, D]


def _compare(got_rows, ref_rows, what):
    err = np.abs(got_rows - ref_rows)
    max_abs = float(err.max()) if err.size else 0.0
    rel = float(np.linalg.norm(got_rows - ref_rows) / max(np.linalg.norm(ref_rows), 1e-300))
    print(f"[parity] {what}: max_abs={max_abs:.3e} rel_frob={rel:.3e}", flush=True)
    assert np.all(np.isfinite(got_rows)), what
    assert max_abs <= MAX_ABS, (what, max_abs)
    assert rel <= REL_FROB, (what, rel)
    return max_abs, rel


def _random_case(seed, B, H, L, D):
    rng = np.random.default_rng(seed)
    q, k, v = (gen.f32_to_bf16_bits(rng.standard_normal((B, H, L, D), dtype=np.float32)) for _ in range(3))
    return q, k, v


SMALL = [
    # (mask, L, H, D, sink)
    (dict(kind="full"), 300, 2, 64, False),
    (dict(kind="full"), 300, 2, 80, True),
    (dict(kind="full", causal=True), 517, 2, 128, False),
    (dict(kind="chunk", chunk=64), 256, 2, 64, False),
    (dict(kind="chunk", chunk=100), 450, 2, 80, True),
    (dict(kind="window", left=128, right=128), 1000, 2, 80, False),
    (dict(kind="window", left=40, right=7), 333, 3, 128, True),
    (dict(kind="window", left=0, right=0, causal=True, head_left=[0, 63, 200, 2000]), 777, 4, 128, True),
    (dict(kind="window", left=0, right=0), 200, 1, 64, False),
    (dict(kind="full"), 300, 2, 256, True),
    (dict(kind="chunk", chunk=100), 450, 2, 256, False),
]


@pytest.mark.parametrize("ci", range(len(SMALL)))
@pytest.mark.parametrize("layout", ["blhd", "bhld"])
def test_small_cases(ci, layout):
    mask, L, H, D, with_sink = SMALL[ci]
    print(f"[case] small {ci} {mask['kind']} L={L} H={H} D={D} sink={with_sink} {layout}", flush=True)
    q, k, v = _random_case(100 + ci, 2, H, L, D)
    sink = np.random.default_rng(200 + ci).standard_normal(H).astype(np.float32) if with_sink else None
    got = _run_gpu(q, k, v, mask, sink, layout)
    ref = attention(q, k, v, mask, sink=sink)["out"]
    _compare(got, ref, f"small{ci}-{layout}")


@pytest.mark.parametrize("bs,L", [(128, 1024), (128, 1000), (256, 1536)])
def test_block_masks(bs, L):
    H, D = 2, 128
    nb = -(-L // bs)
    bm = gen.block_matrix_top_half(3, 5, H, nb)
    bm[1, nb // 2, :] = 0                       # an empty block row: those queries see nothing
    mask = dict(kind="block", block=bs, block_mask=bm)
    print(f"[case] block bs={bs} L={L}", flush=True)
    q, k, v = _random_case(7, 1, H, L, D)
    got = _run_gpu(q, k, v, mask)
    ref = attention(q, k, v, mask)["out"]
    _compare(got, ref, f"block{bs}-{L}")
    empty = slice((nb // 2) * bs, min(L, (nb // 2 + 1) * bs))
    assert np.all(got[0, 1, empty] == 0.0)


def test_tiny_chunk_workload():
    w = gen.workload("tiny_chunk")
    q, k, v = gen.qkv_bf16(0, w["cfg"], w["B"], w["H"], w["L"], w["D"])
    mask = w["masks"]["chunk64"]
    got = _run_gpu(q, k, v, mask)
    ref = attention(q, k, v, mask)["out"]
    _compare(got, ref, "tiny_chunk")
    got1 = _run_gpu(q, k, v, mask, oneshot=True)
    assert np.array_equal(got, got1)


def test_vit896_workload_all_rows():
    w = gen.workload("vit896")
    q, k, v = gen.qkv_bf16(0, w["cfg"], w["B"], w["H"], w["L"], w["D"])
    for label, mask in w["masks"].items():
        print(f"[case] vit896 {label}", flush=True)
        got = _run_gpu(q, k, v, mask)
        ref = attention(q, k, v, mask)["out"]
        _compare(got, ref, f"vit896-{label}")


def test_lm_headwin_workload_all_rows():
    w = gen.workload("lm_headwin")
    q, k, v = gen.qkv_bf16(0, w["cfg"], w["B"], w["H"], w["L"], w["D"])
    mask = w["masks"]["headwin"]
    got = _run_gpu(q, k, v, mask, sink=w["sink"])
    r = attention(q, k, v, mask, sink=w["sink"])
    _compare(got, r["out"], "lm_headwin")


def test_vit1792_workload_sampled_rows():
    w = gen.workload("vit1792")
    q, k, v = gen.qkv_bf16(0, w["cfg"], w["B"], w["H"], w["L"], w["D"])
    rows = gen.sampled_rows(0, w["cfg"], w["H"], w["L"], w["rows"])
    for label, mask in w["masks"].items():
        print(f"[case] vit1792 {label}", flush=True)
        got = _run_gpu(q, k, v, mask)
        ref = attention(q, k, v, mask, rows=rows)["out"]
        sel = np.stack([got[:, h, rows[h]] for h in range(w["H"])], axis=1)
        _compare(sel, ref, f"vit1792-{label}")


def test_blocksparse128k_workload_sampled_rows():
    w = gen.workload("blocksparse128k")
    print("[case] blocksparse128k: generating inputs", flush=True)
    q, k, v = gen.qkv_bf16(0, w["cfg"], w["B"], w["H"], w["L"], w["D"])
    rows = gen.sampled_rows(0, w["cfg"], w["H"], w["L"], w["rows"])
    mask = w["masks"]["block50"]
    got = _run_gpu(q, k, v, mask)
    print("[case] blocksparse128k: oracle on sampled rows", flush=True)
    ref = attention(q, k, v, mask, rows=rows)["out"]
    sel = np.stack([got[:, h, rows[h]] for h in range(w["H"])], axis=1)
    _compare(sel, ref, "blocksparse128k")


def test_v_ones_probe_and_determinism():
    """V = 1 gives o_i = 1 - pi_i; two launches are bitwise identical."""
    mask = dict(kind="window", left=0, right=0, causal=True, head_left=[10, 500, 1000, 3000])
    H, L, D = 4, 1500, 128
    q, k, _ = _random_case(5, 1, H, L, D)
    v = np.full_like(q, 0x3F80)                     # bf16 1.0
    sink = np.array([0.5, -1.0, 2.0, -np.inf], np.float32)
    got = _run_gpu(q, k, v, mask, sink)
    r = attention(q, k, v, mask, sink=sink)
    exp = (1.0 - r["sink_mass"])[..., None]
    assert np.max(np.abs(got - exp)) <= 8e-3
    got2 = _run_gpu(q, k, v, mask, sink)
    assert np.array_equal(got, got2)


KERNELS_128 = [
    # (mask, L, kernel the plan picks at head dim 128)
    (dict(kind="full"), 2200, "pingpong"),
    (dict(kind="full", causal=True), 2500, "single"),
    (dict(kind="window", left=300, right=0, causal=True), 1800, "single"),
    (dict(kind="chunk", chunk=1024, causal=True), 3000, "single"),
    (dict(kind="window", left=2000, right=2000), 2600, "pingpong"),
]


@pytest.mark.parametrize("ci", range(len(KERNELS_128)))
def test_both_head_dim_128_kernels(ci):
    """Head dim 128 runs the single-group kernel for short rows and the ping-pong kernel for long
    ones (the plan decides); both against the oracle, with a sink, batch 2 (unsplit) and batch 1
    (split rows)."""
    from block_sparse_softmax_amd import _lib
    mask, L, kind = KERNELS_128[ci]
    H, D = 2, 128
    assert _lib.Plan(mask, L, H, D).kernel() == kind
    sink = np.random.default_rng(700 + ci).standard_normal(H).astype(np.float32)
    for B in (2, 1):
        print(f"[case] d128 {kind} {mask} L={L} B={B}", flush=True)
        q, k, v = _random_case(710 + ci, B, H, L, D)
        got = _run_gpu(q, k, v, mask, sink, layout="bhld")
        ref = attention(q, k, v, mask, sink=sink)["out"]
        _compare(got, ref, f"d128-{kind}-{ci}-B{B}")


def _offset_case(seed, H, L, D, first_sign):
    """Q, K with a shared direction u: the first 64 keys score about first_sign * 40 (log2 units) against
    every query, all other keys about -first_sign * 40, plus N(0, 1) noise in every element."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    a = np.sqrt(40.0 * np.sqrt(D) / np.log2(np.e))
    q = rng.standard_normal((1, H, L, D)) + a * u
    k = rng.standard_normal((1, H, L, D)) - first_sign * a * u
    k[:, :, :64] += 2 * first_sign * a * u
    v = rng.standard_normal((1, H, L, D))
    return tuple(gen.f32_to_bf16_bits(x.astype(np.float32)) for x in (q, k, v))


@pytest.mark.parametrize("D", [64, 80, 128, 256])
@pytest.mark.parametrize("first_sign", [-1, 1])
def test_wide_logit_range(D, first_sign):
    """Scores of later tiles far above (-1) or below (+1) those of the first listed tile: the first case
    makes the probabilities relative to the first tile's reference overflow the fast pass's bound, so the
    work-group redoes the item with a running max; the second underflows harmlessly."""
    L, H = 700, 2
    q, k, v = _offset_case(31 + D, H, L, D, first_sign)
    for mask in (dict(kind="full"), dict(kind="window", left=300, right=300)):
        print(f"[case] wide logit range D={D} sign={first_sign} {mask['kind']}", flush=True)
        got = _run_gpu(q, k, v, mask, layout="bhld")
        ref = attention(q, k, v, mask)["out"]
        _compare(got, ref, f"wide-range-d{D}-{first_sign}-{mask['kind']}")


def _far_below_case(seed, H, L, D):
    """Every score about 200 below zero (log2 units), spread about +-3 by the keys: q = n1 + a u,
    k = n2 / 2 - a u for one shared unit direction u (the rounding of the large shared part shifts
    all scores of a row alike, which the softmax ignores)."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    a = np.sqrt(200.0 * np.sqrt(D) / np.log2(np.e))
    q = rng.standard_normal((1, H, L, D)) + a * u
    k = 0.5 * rng.standard_normal((1, H, L, D)) - a * u
    v = rng.standard_normal((1, H, L, D))
    return tuple(gen.f32_to_bf16_bits(x.astype(np.float32)) for x in (q, k, v))


@pytest.mark.parametrize("D", [64, 80, 128, 256])
def test_scores_far_below_placeholder_reference(D):
    """Rows whose first listed tile holds none of their keys start from the placeholder reference 0;
    with every score about 2^-200 relative to it the probabilities underflow, and the work-group must
    still return the exact softmax (its rows are recomputed)."""
    L, H = 700, 2
    q, k, v = _far_below_case(57 + D, H, L, D)
    for mask in (dict(kind="window", left=300, right=300), dict(kind="chunk", chunk=100),
                 dict(kind="window", left=0, right=0, causal=True, head_left=[150, 333])):
        print(f"[case] far below reference D={D} {mask['kind']}", flush=True)
        got = _run_gpu(q, k, v, mask, layout="bhld")
        ref = attention(q, k, v, mask)["out"]
        _compare(got, ref, f"far-below-d{D}-{mask['kind']}")


SPLIT = [
    # (mask, L, sink): rows long enough that the batch-1 schedule cuts them into pieces
    (dict(kind="chunk", chunk=1000), 3000, False),    # pieces with rows that see none of their keys
    (dict(kind="full", causal=True), 2500, True),
    (dict(kind="window", left=700, right=50), 2200, True),
]


@pytest.mark.parametrize("D", [64, 80, 128, 256])
@pytest.mark.parametrize("ci", range(len(SPLIT)))
def test_split_rows_merge(D, ci):
    """Long rows split into pieces whose partial states the last piece merges (batch 1)."""
    from block_sparse_softmax_amd import _lib
    mask, L, with_sink = SPLIT[ci]
    H = 2
    items = _lib.Plan(mask, L, H, D).schedule()
    assert np.any(items[:, 6] > 1), "the schedule should split some rows"
    print(f"[case] split rows {mask['kind']} L={L} D={D} sink={with_sink}", flush=True)
    q, k, v = _random_case(300 + ci, 1, H, L, D)
    sink = np.random.default_rng(400 + ci).standard_normal(H).astype(np.float32) if with_sink else None
    got = _run_gpu(q, k, v, mask, sink)
    ref = attention(q, k, v, mask, sink=sink)["out"]
    _compare(got, ref, f"split-{ci}-d{D}")
    got2 = _run_gpu(q, k, v, mask, sink)   # a second launch on the same workspace: the same result
    assert np.array_equal(got, got2)


def test_launch_events_bracket_the_kernel():
    """Events handed to the launch are recorded at the kernel's start and end: their interval is
    positive and lies inside an interval bracketed by ordinary stream events around the launch."""
    from block_sparse_softmax_amd import prepare
    L, H, D = 2048, 4, 80
    q, k, v = (_bits_to_bf16(x) for x in _random_case(11, 1, H, L, D))
    o = torch.empty_like(q)
    pm = prepare(dict(kind="full"), L, H, D, q.device)
    run = pm.bind(q, k, v, o, layout="bhld")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    ev[0].record()
    run(ev[1], ev[2])
    ev[3].record()
    torch.cuda.synchronize()
    inner, outer = ev[1].elapsed_time(ev[2]), ev[0].elapsed_time(ev[3])
    print(f"[events] kernel {inner * 1e3:.1f} us inside {outer * 1e3:.1f} us", flush=True)
    assert 0.0 < inner <= outer + 1e-3
    assert torch.isfinite(o.float()).all()


def test_grouped_launch_matches_single_launches():
    """One grouped launch of several masks (split rows and a sink among them) writes exactly what
    the single launches write."""
    from block_sparse_softmax_amd import bind_group, prepare
    L, H, D = 2500, 2, 80
    q, k, v = (_bits_to_bf16(x) for x in _random_case(21, 1, H, L, D))
    sink = torch.as_tensor(np.random.default_rng(22).standard_normal(H).astype(np.float32)).cuda()
    masks = [dict(kind="full"), dict(kind="chunk", chunk=256), dict(kind="window", left=128, right=128),
             dict(kind="full", causal=True)]
    sinks = [None, None, None, sink]
    pms = [prepare(m, L, H, D, q.device) for m in masks]
    single = []
    for pm, s in zip(pms, sinks):
        o = torch.empty_like(q)
        pm.launch(q, k, v, o, sink=s, layout="bhld")
        single.append(o)
    outs = [torch.empty_like(q) for _ in masks]
    run = bind_group(pms, [q] * 4, [k] * 4, [v] * 4, outs, sinks=sinks, layout="bhld")
    for _ in range(2):  # twice on the same workspaces: the same result
        for o in outs:
            o.zero_()
        run()
        torch.cuda.synchronize()
        for j in range(len(masks)):
            assert torch.equal(outs[j], single[j]), masks[j]
    ref = attention(*(x for x in _random_case(21, 1, H, L, D)), masks[1])["out"]
    _compare(outs[1].float().cpu().double().numpy(), ref, "group-chunk")


GQA_PREFIX = [
    # (mask, L, H, Hkv, D, sink, B)
    (dict(kind="full", causal=True), 700, 8, 2, 128, False, 1),
    (dict(kind="window", left=300, right=0, causal=True), 1000, 4, 1, 80, True, 2),
    # the pages' SWA with 4 StreamingLLM sink tokens (572 + 4) and 32 query heads on 8 K/V heads, scaled down
    (dict(kind="window", left=571, right=0, causal=True, prefix=4), 2048, 8, 2, 128, True, 1),
    (dict(kind="chunk", chunk=256, prefix=16), 900, 4, 2, 64, False, 1),
    (dict(kind="window", left=64, right=64, prefix=100), 1500, 2, 2, 80, False, 1),   # prefix over 2 tiles
    (dict(kind="full", prefix=40), 333, 2, 1, 64, True, 2),                           # prefix inside full: no-op
    # head dim 256 with 16 query heads on 4 K/V heads (the SWA-vs-linear-attention article's speed-test
    # layer): its sliding window of 576 keys with a learned sink, and 572 window keys + 4 prefix tokens
    (dict(kind="window", left=575, right=0, causal=True), 1500, 16, 4, 256, True, 1),
    (dict(kind="window", left=571, right=0, causal=True, prefix=4), 1500, 16, 4, 256, True, 1),
    (dict(kind="full", causal=True), 777, 16, 4, 256, False, 2),
]


@pytest.mark.parametrize("ci", range(len(GQA_PREFIX)))
def test_grouped_query_heads_and_prefix_tokens(ci):
    mask, L, H, Hkv, D, with_sink, B = GQA_PREFIX[ci]
    print(f"[case] gqa/prefix {ci} {mask} L={L} H={H}/{Hkv} D={D} B={B}", flush=True)
    rng = np.random.default_rng(500 + ci)
    q = gen.f32_to_bf16_bits(rng.standard_normal((B, H, L, D), dtype=np.float32))
    k = gen.f32_to_bf16_bits(rng.standard_normal((B, Hkv, L, D), dtype=np.float32))
    v = gen.f32_to_bf16_bits(rng.standard_normal((B, Hkv, L, D), dtype=np.float32))
    sink = rng.standard_normal(H).astype(np.float32) if with_sink else None
    got = _run_gpu(q, k, v, mask, sink, layout="bhld")
    ref = attention(q, k, v, mask, sink=sink)["out"]
    _compare(got, ref, f"gqa-prefix{ci}")


@pytest.mark.parametrize("mask", [dict(kind="window", left=575, right=0, causal=True),
                                  dict(kind="window", left=571, right=0, causal=True, prefix=4)],
                         ids=["swa576-sink", "swa572-prefix4"])
def test_d256_grouped_query_sampled_rows(mask):
    """Head dim 256, 16 query heads on 4 K/V heads over 16384 tokens (batch 1): the windows of the
    SWA-vs-linear-attention article's speed test, with a learned sink; 512 seeded rows per head."""
    B, H, Hkv, L, D = 1, 16, 4, 16384, 256
    print(f"[case] d256 gqa sampled {mask}", flush=True)
    rng = np.random.default_rng(900 + mask.get("prefix", 0))
    q = gen.f32_to_bf16_bits(rng.standard_normal((B, H, L, D), dtype=np.float32))
    k = gen.f32_to_bf16_bits(rng.standard_normal((B, Hkv, L, D), dtype=np.float32))
    v = gen.f32_to_bf16_bits(rng.standard_normal((B, Hkv, L, D), dtype=np.float32))
    sink = rng.standard_normal(H).astype(np.float32)
    got = _run_gpu(q, k, v, mask, sink, layout="bhld")
    rows = np.sort(rng.choice(L, size=(H, 512), replace=True), axis=1)
    rows[:, :4] = [0, 575, 576, L - 1]          # the first row, both sides of the window edge, the last
    ref = attention(q, k, v, mask, sink=sink, rows=rows)["out"]
    sel = np.stack([got[:, h, rows[h]] for h in range(H)], axis=1)
    _compare(sel, ref, f"d256-sampled-{mask.get('prefix', 0)}")


def _grouped_as_bench(w, q, k, v):
    """Every mask of workload w in ONE grouped launch on [B, H, L, D] tensors: the launch bench.py times."""
    from block_sparse_softmax_amd import bind_group, prepare
    qt, kt, vt = (_bits_to_bf16(x) for x in (q, k, v))
    sink = None if w["sink"] is None else torch.as_tensor(w["sink"]).cuda()
    labels = list(w["masks"])
    pms = [prepare(w["masks"][m], w["L"], w["H"], w["D"], qt.device) for m in labels]
    outs = [torch.empty_like(qt) for _ in labels]
    n = len(labels)
    bind_group(pms, [qt] * n, [kt] * n, [vt] * n, outs, sinks=[sink] * n, layout="bhld")()
    torch.cuda.synchronize()
    return {m: o.float().cpu().double().numpy() for m, o in zip(labels, outs)}


@pytest.mark.parametrize("name", ["vit896", "vit1792", "lm_headwin", "blocksparse128k", "swa576_d256"])
def test_workloads_in_the_bench_launch(name):
    """The grouped [B, H, L, D] launch of each workload against the oracle: all rows up to 4096 tokens,
    512 seeded rows per head beyond."""
    w = gen.workload(name)
    print(f"[case] {name}: grouped launch as timed", flush=True)
    q, k, v = gen.qkv_bf16(0, w["cfg"], w["B"], w["H"], w["L"], w["D"], w["Hkv"])
    got = _grouped_as_bench(w, q, k, v)
    rows = None if w["rows"] is None else gen.sampled_rows(0, w["cfg"], w["H"], w["L"], w["rows"])
    for label, mask in w["masks"].items():
        ref = attention(q, k, v, mask, sink=w["sink"], rows=rows)["out"]
        g = got[label] if rows is None else np.stack([got[label][:, h, rows[h]] for h in range(w["H"])], axis=1)
        _compare(g, ref, f"{name}-{label} grouped")


def _spread_case(seed, H, L, D, spread_log2):
    """Q = N(0,1) + 8u and K = N(0,1) + b_j u with b_j uniform, so that a row's logits differ across
    its keys by about `spread_log2` log2 units (peaky heads), bf16."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    c = np.log2(np.e) / np.sqrt(D)
    alpha = 8.0
    b = spread_log2 / (2 * c * alpha)
    q = rng.standard_normal((1, H, L, D)) + alpha * u
    k = rng.standard_normal((1, H, L, D)) + rng.uniform(-b, b, (1, H, L, 1)) * u
    v = rng.standard_normal((1, H, L, D))
    return tuple(gen.f32_to_bf16_bits(x.astype(np.float32)) for x in (q, k, v))


@pytest.mark.parametrize("D", [64, 80, 128, 256])
@pytest.mark.parametrize("spread", [14.0, 32.0])
def test_large_logit_spread(D, spread):
    """Logits of a row spread over 20-40 log2 units across its keys (the key term b_j u gives
    `spread`, the Gaussian parts about 7 more): the softmax concentrates on a few keys and the
    kernel's score precision (bf16 operands, fp32 scores) decides the result."""
    from oracle.attention import bf16_to_f64
    L, H = 640, 2
    q, k, v = _spread_case(int(spread) + D, H, L, D, spread)
    s2 = (bf16_to_f64(q[0, 0]) @ bf16_to_f64(k[0, 0]).T) * (np.log2(np.e) / np.sqrt(D))
    observed = float(np.median(s2.max(axis=1) - s2.min(axis=1)))
    assert 18.0 <= observed <= 42.0, observed
    for mask in (dict(kind="full"), dict(kind="window", left=200, right=0, causal=True)):
        print(f"[case] spread {spread} D={D} {mask['kind']}", flush=True)
        got = _run_gpu(q, k, v, mask, layout="bhld")
        ref = attention(q, k, v, mask)["out"]
        _compare(got, ref, f"spread{spread:.0f}-D{D}-{mask['kind']}")


@pytest.mark.parametrize("D", [64, 80, 128, 256])
@pytest.mark.parametrize("L", [1, 2, 63, 65])
def test_sequences_shorter_than_a_tile(D, L):
    """Sequences of one token, two tokens and one either side of a 64-key tile: every key tile is the
    ragged last one and every query tile is mostly past the end (rows clamped on load, never stored)."""
    masks = [dict(kind="full"), dict(kind="full", causal=True),
             dict(kind="window", left=3, right=0, causal=True), dict(kind="chunk", chunk=32)]
    q, k, v = _random_case(900 + L + D, 2, 2, L, D)
    sink = np.random.default_rng(L + D).standard_normal(2).astype(np.float32)
    for mi, mask in enumerate(masks):
        for layout in ("bhld", "blhd"):
            print(f"[case] short L={L} D={D} {mask} {layout}", flush=True)
            s = sink if mi % 2 else None
            got = _run_gpu(q, k, v, mask, s, layout)
            ref = attention(q, k, v, mask, sink=s)["out"]
            _compare(got, ref, f"short-L{L}-D{D}-{mi}-{layout}")
