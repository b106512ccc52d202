"""The C ABI on the CPU: the library loads, exports every symbol the header
declares, rejects invalid arguments on the host before any HIP call, and
plans work lists that cover every (row, key) exactly once.  No kernel runs."""
import ctypes
import os
import re

import numpy as np
import pytest

from paged_kv_varlen_flash_amd import ops, workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedattn.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ops.LIB_PATH):
        from paged_kv_varlen_flash_amd import build
        build.build()
    return ops.lib()


def header_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    funcs = set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text))
    vars_ = set(re.findall(r"extern\s+const\s+\w+\s+(pa_[a-z0-9_]+)\s*\[", text))
    return funcs | vars_


def test_exports_every_declared_symbol(L):
    syms = header_symbols()
    assert {"pa_plan_varlen", "pa_reshape_and_cache", "pa_varlen_fwd",
            "pa_merge_attn_states"} <= syms
    for s in syms:
        assert hasattr(L, s), f"{s} declared in pagedattn.h but not exported"
    assert sorted(syms) == sorted(ops.EXPORTED)


def test_status_strings_and_version(L):
    assert ops.status_str(0) == "PA_OK"
    assert ops.status_str(3) == "PA_ERR_WORKSPACE_TOO_SMALL"
    assert ops.status_str(99) == "PA_ERR_UNKNOWN"
    assert L.pa_version() >> 16 == 5              # pa_attn_params.num_cus
    assert ops.supported_head_sizes() == [64, 128, 256]


def params(**kw):
    base = dict(batch=2, num_heads=4, num_kv_heads=2, head_size=64, block_size=16,
                num_blocks=16, max_blocks_per_seq=6, causal=True, scale=0.125)
    raw_causal = kw.pop("raw_causal", None)
    base.update(kw)
    p = ops.make_params(**base)
    if raw_causal is not None:
        p.causal = raw_causal
    return p


CU = [0, 37, 38]
SK = [37, 81]


@pytest.mark.parametrize("kw,status", [
    (dict(block_size=24), ops.PA_ERR_INVALID_ARGUMENT),      # not a multiple of 16
    (dict(block_size=0), ops.PA_ERR_INVALID_ARGUMENT),
    (dict(head_size=96), ops.PA_ERR_UNSUPPORTED),            # valid size, not compiled
    (dict(head_size=100), ops.PA_ERR_INVALID_ARGUMENT),      # not a multiple of 8
    (dict(head_size=512), ops.PA_ERR_INVALID_ARGUMENT),      # above 256
    (dict(num_heads=5), ops.PA_ERR_INVALID_ARGUMENT),        # H % Hkv != 0
    (dict(num_kv_heads=0), ops.PA_ERR_INVALID_ARGUMENT),
    (dict(batch=-1), ops.PA_ERR_INVALID_ARGUMENT),
    (dict(max_blocks_per_seq=5), ops.PA_ERR_INVALID_ARGUMENT),  # 81 keys need 6 blocks
    (dict(raw_causal=2), ops.PA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("nan")), ops.PA_ERR_INVALID_ARGUMENT),
    (dict(block_table_stride=3), ops.PA_ERR_INVALID_ARGUMENT),
])
def test_plan_rejects(L, kw, status):
    with pytest.raises(ops.PaError) as e:
        ops.pa_plan_varlen(params(**kw), CU, SK)
    assert e.value.status == status


def test_plan_rejects_bad_lengths(L):
    with pytest.raises(ops.PaError):
        ops.pa_plan_varlen(params(), [1, 37, 38], SK)          # cu[0] != 0
    with pytest.raises(ops.PaError):
        ops.pa_plan_varlen(params(), [0, 37, 30], SK)          # decreasing
    with pytest.raises(ops.PaError):
        ops.pa_plan_varlen(params(), CU, [37, -1])
    with pytest.raises(ops.PaError):
        ops.pa_plan_varlen(params(), CU, SK, force_splits=-2)


def test_plan_capacity_error(L):
    p = params()
    info = ops.PlanInfo()
    cu = np.array(CU, np.int32)
    sk = np.array(SK, np.int32)
    small = np.zeros(4, np.int32)
    st = L.pa_plan_varlen(ctypes.byref(p), cu.ctypes.data_as(ops._I32P),
                          sk.ctypes.data_as(ops._I32P), 0, small.ctypes.data_as(ops._I32P),
                          small.nbytes, ctypes.byref(info))
    assert st == ops.PA_ERR_WORKSPACE_TOO_SMALL
    assert info.worklist_bytes > small.nbytes


def _fwd_call(L, p, info, **override):
    """pa_varlen_fwd with fake (never dereferenced) pointers; only calls that
    fail host validation may be made on a machine without a GPU."""
    args = dict(worklist=0x1000, q=0x2000, kv=0x3000, cu=0x4000, sk=0x5000, bt=0x6000,
                T=info.num_tokens if info is not None else 38, out=0x7000, lse=0x8000, ws=0x10000, ws_bytes=1 << 30)
    args.update(override)
    P = ctypes.c_void_p
    return L.pa_varlen_fwd(ctypes.byref(p), ctypes.byref(info) if info is not None else None,
                           P(args["worklist"]), P(args["q"]), P(args["kv"]), P(args["cu"]),
                           P(args["sk"]), P(args["bt"]), args["T"], P(args["out"]),
                           P(args["lse"]), P(args["ws"]), args["ws_bytes"], None)


def test_fwd_validation_before_launch(L):
    p = params()
    _, info = ops.pa_plan_varlen(p, CU, SK, force_splits=3)
    assert info.workspace_bytes > 0
    E = ops.PA_ERR_INVALID_ARGUMENT
    assert _fwd_call(L, p, None) == E
    assert _fwd_call(L, p, info, q=0) == E
    assert _fwd_call(L, p, info, worklist=0) == E
    assert _fwd_call(L, p, info, out=0) == E
    assert _fwd_call(L, p, info, bt=0) == E
    assert _fwd_call(L, p, info, q=0x2008) == E              # misaligned
    assert _fwd_call(L, p, info, ws=0) == E
    assert _fwd_call(L, p, info, ws=0x10010) == E            # not 256-B aligned
    assert _fwd_call(L, p, info, T=info.num_tokens + 1) == E  # plan/params mismatch
    assert _fwd_call(L, p, info, ws_bytes=info.workspace_bytes - 1) == ops.PA_ERR_WORKSPACE_TOO_SMALL
    p2 = params(causal=False)
    assert _fwd_call(L, p2, info) == E                       # planned causal, called non-causal
    p3 = params(head_size=96)
    assert _fwd_call(L, p3, info) == ops.PA_ERR_UNSUPPORTED


def test_fp8_entry_points_validate_before_launch(L):
    P = ctypes.c_void_p
    E = ops.PA_ERR_INVALID_ARGUMENT
    p = params()
    _, info = ops.pa_plan_varlen(p, CU, SK, force_splits=3)

    def fwd8(ks=0x9000, vs=0x9100, **kw):
        a = dict(worklist=0x1000, q=0x2000, kv=0x3000, cu=0x4000, sk=0x5000, bt=0x6000,
                 out=0x7000, lse=0x8000, ws=0x10000)
        a.update(kw)
        return L.pa_varlen_fwd_fp8(ctypes.byref(p), ctypes.byref(info), P(a["worklist"]), P(a["q"]),
                                   P(a["kv"]), P(a["cu"]), P(a["sk"]), P(a["bt"]), P(ks), P(vs),
                                   info.num_tokens, P(a["out"]), P(a["lse"]), P(a["ws"]), 1 << 30, None)
    assert fwd8(ks=0) == E                       # a scale pointer is required
    assert fwd8(vs=0) == E
    assert fwd8(ks=0x9002) == E                  # misaligned scales
    assert fwd8(q=0) == E

    def rc8(**kw):
        a = dict(k=0x1000, v=0x2000, ks_=128, vs_=128, c=0x3000, s=0x4000, kscale=0x5000,
                 vscale=0x6000, T=4, Hkv=2, D=64, NB=4, BS=16)
        a.update(kw)
        return L.pa_reshape_and_cache_fp8(P(a["k"]), P(a["v"]), a["ks_"], a["vs_"], P(a["c"]),
                                          P(a["s"]), P(a["kscale"]), P(a["vscale"]), a["T"],
                                          a["Hkv"], a["D"], a["NB"], a["BS"], None)
    assert rc8(D=72, ks_=144, vs_=144) == E       # head size not a multiple of 16
    assert rc8(kscale=0) == E and rc8(vscale=0) == E
    assert rc8(BS=24) == E
    assert rc8(T=0, k=0, v=0, c=0, s=0, kscale=0, vscale=0) == ops.PA_OK   # no launch


def test_reshape_and_cache_validation(L):
    P = ctypes.c_void_p
    E = ops.PA_ERR_INVALID_ARGUMENT
    ok = dict(k=0x1000, v=0x2000, ks=128, vs=128, c=0x3000, s=0x4000, T=4, Hkv=2, D=64, NB=4, BS=16)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return L.pa_reshape_and_cache(P(a["k"]), P(a["v"]), a["ks"], a["vs"], P(a["c"]), P(a["s"]),
                                      a["T"], a["Hkv"], a["D"], a["NB"], a["BS"], None)
    assert call(BS=24) == E
    assert call(D=60) == E
    assert call(ks=64) == E          # stride below Hkv*D
    assert call(vs=130) == E         # stride not a multiple of 8
    assert call(k=0) == E
    assert call(s=0) == E
    assert call(c=0x3004) == E       # misaligned cache
    assert call(T=-1) == E
    assert call(T=0, k=0, v=0, c=0, s=0) == ops.PA_OK   # nothing to do: no launch


def test_merge_validation(L):
    P = ctypes.c_void_p
    E = ops.PA_ERR_INVALID_ARGUMENT
    f = L.pa_merge_attn_states
    assert f(P(0x1000), None, P(0x2000), P(0x3000), P(0x4000), P(0x5000), 4, 2, 60, None) == E
    assert f(P(0x1000), None, P(0), P(0x3000), P(0x4000), P(0x5000), 4, 2, 64, None) == E
    assert f(P(0x1008), None, P(0x2000), P(0x3000), P(0x4000), P(0x5000), 4, 2, 64, None) == E
    assert f(P(0), None, P(0), P(0), P(0), P(0), 0, 2, 64, None) == ops.PA_OK


def test_noalloc_rejects_plans_beyond_its_scratch(L):
    """pa_varlen_fwd_noalloc refuses a plan whose partials exceed
    PA_NOALLOC_SCRATCH_BYTES, on the host, before any HIP call (fake
    pointers are never touched)."""
    B, Lk = 512, 4096
    p = ops.make_params(B, 64, 8, 256, 16, B * Lk // 16, Lk // 16, True, 0.0625)
    cu = np.arange(B + 1, dtype=np.int32)
    sk = np.full(B, Lk, np.int32)
    _, info = ops.pa_plan_varlen(p, cu, sk, force_splits=64)
    assert info.workspace_bytes > ops.NOALLOC_SCRATCH_BYTES
    P = ctypes.c_void_p
    st = L.pa_varlen_fwd_noalloc(ctypes.byref(p), ctypes.byref(info), P(0x1000), P(0x2000),
                                 P(0x3000), P(0x4000), P(0x5000), P(0x6000), None, B, P(0x7000),
                                 P(0x8000), None)
    assert st == ops.PA_ERR_WORKSPACE_TOO_SMALL
    # an invalid cache format is refused as well
    opt = ops.FwdOptions(7, None, None, None)
    st = L.pa_varlen_fwd_noalloc(ctypes.byref(p), ctypes.byref(info), P(0x1000), P(0x2000),
                                 P(0x3000), P(0x4000), P(0x5000), P(0x6000), ctypes.byref(opt), B,
                                 P(0x7000), P(0x8000), None)
    assert st == ops.PA_ERR_INVALID_ARGUMENT


def test_merge_rejects_lse_aliasing(L):
    """out_lse may not overlap prefix_lse or suffix_lse (rows of 4 tokens x
    2 heads = 8 floats = 32 bytes); out may still alias either output."""
    P = ctypes.c_void_p
    E = ops.PA_ERR_INVALID_ARGUMENT
    f = L.pa_merge_attn_states
    assert f(P(0x1000), P(0x3000), P(0x1000), P(0x3000), P(0x4000), P(0x5000), 4, 2, 64, None) == E
    assert f(P(0x1000), P(0x5000), P(0x2000), P(0x3000), P(0x4000), P(0x5000), 4, 2, 64, None) == E
    assert f(P(0x1000), P(0x3010), P(0x2000), P(0x3000), P(0x4000), P(0x5000), 4, 2, 64, None) == E
    assert f(P(0x1000), P(0x2ff0), P(0x2000), P(0x3000), P(0x4000), P(0x5000), 4, 2, 64, None) == E


def test_cascade_split(L):
    wl = W.make("cascade_prefix", materialise=False)
    p = ops.make_params(wl.B, wl.H, wl.Hkv, wl.D, wl.BS, wl.num_blocks, wl.block_table.shape[1],
                        True, wl.scale)
    pp, sp, pcu, psk, ssk, col0 = ops.pa_cascade_split(p, 2048, wl.cu_seqlens_q, wl.k_lens)
    assert col0 == 2048 // 16 and list(pcu) == [0, wl.T] and list(psk) == [2048]
    assert np.array_equal(ssk, wl.k_lens - 2048)
    assert pp.batch == 1 and pp.causal == 0 and pp.max_blocks_per_seq == 128
    assert sp.causal == 1 and sp.block_table_stride == wl.block_table.shape[1]
    with pytest.raises(ops.PaError):
        ops.pa_cascade_split(p, 2040, wl.cu_seqlens_q, wl.k_lens)     # not block aligned
    with pytest.raises(ops.PaError):
        ops.pa_cascade_split(p, 4096, wl.cu_seqlens_q, wl.k_lens)     # longer than a context


# ---------------------------------------------------------------- plan coverage
def parse(wl_words, info):
    assert wl_words[0] == ops.PA_WORKLIST_MAGIC and wl_words[1] == 3
    n_att = info.num_small_items + info.num_tiled_items
    IW = ops.PA_ITEM_WORDS
    items = wl_words[16:16 + IW * n_att].reshape(-1, IW)
    red = wl_words[16 + IW * n_att:].reshape(-1, IW)
    assert len(red) == info.num_reduce_items
    return items, red


def check_plan_covers(H, Hkv, q_lens, k_lens, causal, force_splits=0, kv_cache_fp8=False):
    """Every visible (row, key) pair is covered by exactly one item; split
    units have a reduce item whose partial rows match their items."""
    G = H // Hkv
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    BS = 16
    MB = max(1, max((k + BS - 1) // BS for k in k_lens))
    p = ops.make_params(len(q_lens), H, Hkv, 64, BS, 4096, MB, causal, 0.1,
                        kv_cache_fp8=kv_cache_fp8)
    words, info = ops.pa_plan_varlen(p, cu, k_lens, force_splits)
    items, red = parse(words, info)
    cover = {}
    small_rows = PA_SMALL = 16
    assert (items[:, 7] == 0).sum() == info.num_small_items
    assert (items[:, 7] == 1).sum() == info.num_tiled_items
    # words 8, 9: the sequence's first token and Lk - Lq
    assert np.array_equal(items[:, 8], cu[items[:, 0]])
    assert np.array_equal(items[:, 9], np.asarray(k_lens)[items[:, 0]] - np.diff(cu)[items[:, 0]])
    # tiled items hold up to 256 rows in plans without small-row items at D <= 128
    assert info.tiled_rows in (ops.PA_TILED_ROWS, ops.PA_TILED_ROWS_WIDE)
    if info.num_small_items > 0:
        assert info.tiled_rows == ops.PA_TILED_ROWS
    tiled_max = info.tiled_rows
    for idx, (seq, kvh, row0, nrows, k0, k1, prow, kind, *_) in enumerate(items):
        is_small = kind == 0
        assert nrows <= (PA_SMALL if is_small else tiled_max) and nrows >= 1
        for r in range(row0, row0 + nrows):
            cover.setdefault((seq, kvh, r), []).append((k0, k1, prow))
    seen_prow = set()
    for b in range(len(q_lens)):
        Lq, Lk = int(q_lens[b]), int(k_lens[b])
        for kvh in range(Hkv):
            for r in range(Lq * G):
                ranges = sorted(cover.pop((b, kvh, r)))
                i = r // G
                vis_end = min(Lk, max(0, i + Lk - Lq + 1)) if causal else Lk
                # ranges tile [0, end) with end >= vis_end, and nothing past Lk
                pos = 0
                for k0, k1, _ in ranges:
                    assert k0 == pos
                    pos = k1
                assert pos >= vis_end and pos <= Lk
                if len(ranges) > 1:
                    for _, _, prow in ranges:
                        assert prow >= 0
                        seen_prow.add(prow)
                else:
                    assert ranges[0][2] == -1
    assert not cover, "items for rows that do not exist"
    # reduce items point at the split items' partial rows
    for seq, kvh, row0, nrows, prow0, nsplit, tok0, *_ in red:
        assert nsplit >= 2
        assert tok0 == cu[seq]                       # first token of the sequence
        assert row0 + nrows <= q_lens[seq] * G       # rows are clipped by the planner
        for s in range(nsplit):
            assert prow0 + s * nrows in seen_prow
    assert info.num_partial_rows == (max(seen_prow) + 1 if seen_prow else 0) or \
        info.num_partial_rows >= len(seen_prow)
    return info


@pytest.mark.parametrize("force", [0, 1, 3, 7])
def test_plan_covers_mixed(L, force):
    rng = np.random.default_rng(force)
    q_lens = np.array([37, 1, 1, 200, 3, 1, 0, 129], np.int32)
    k_lens = np.array([37, 81, 1, 250, 40, 0, 5, 129], np.int32)
    for causal in (True, False):
        check_plan_covers(8, 2, q_lens, k_lens, causal, force)
        check_plan_covers(4, 4, q_lens, k_lens, causal, force)
    q2 = rng.integers(1, 40, size=12).astype(np.int32)
    k2 = (q2 + rng.integers(0, 300, size=12)).astype(np.int32)
    check_plan_covers(32, 8, q2, k2, True, force)


@pytest.mark.parametrize("name", W.ORDER)
def test_plan_covers_workloads(L, name):
    wl = W.make(name, materialise=False)
    if wl.T * wl.H > 5000 * 32:
        # full coverage on the big mix is slow in Python; check the counts only
        p = ops.make_params(wl.B, wl.H, wl.Hkv, wl.D, wl.BS, wl.num_blocks,
                            wl.block_table.shape[1], wl.causal, wl.scale)
        words, info = ops.pa_plan_varlen(p, wl.cu_seqlens_q, wl.k_lens)
        items, red = parse(words, info)
        assert info.num_tiled_items > 0 and info.num_small_items > 0
        return
    check_plan_covers(wl.H, wl.Hkv, wl.q_lens, wl.k_lens, wl.causal)


def test_plan_is_deterministic(L):
    wl = W.make("decode_llama8b", materialise=False)
    p = ops.make_params(wl.B, wl.H, wl.Hkv, wl.D, wl.BS, wl.num_blocks, wl.block_table.shape[1],
                        True, wl.scale)
    a, _ = ops.pa_plan_varlen(p, wl.cu_seqlens_q, wl.k_lens)
    b, _ = ops.pa_plan_varlen(p, wl.cu_seqlens_q, wl.k_lens)
    assert np.array_equal(a, b)


def test_small_items_longest_first(L):
    """Small items (decode rows) are listed longest first, and the pieces of
    a split unit are a multiple of 64 keys (one step of each of the kernel's
    four waves) except the last one."""
    wl = W.make("decode_llama8b", materialise=False)
    p = ops.make_params(wl.B, wl.H, wl.Hkv, wl.D, wl.BS, wl.num_blocks, wl.block_table.shape[1],
                        True, wl.scale)
    words, info = ops.pa_plan_varlen(p, wl.cu_seqlens_q, wl.k_lens)
    items, red = parse(words, info)
    small = items[items[:, 7] == 0]
    cost = (small[:, 5] - small[:, 4]) * small[:, 3]
    assert np.all(np.diff(cost) <= 0)
    assert (small[:, 5] - small[:, 4]).sum() == int(wl.k_lens.sum()) * wl.Hkv
    for seq, kvh, row0, nrows, k0, k1, prow, *_ in small:
        if prow >= 0 and k1 != wl.k_lens[seq]:
            assert (k1 - k0) % 64 == 0 and k0 % 64 == 0



def test_fp8_cache_plan(L):
    """An E4M3 cache only changes how finely decode key ranges are cut: the
    plan still covers every (row, key) pair once, with no fewer items."""
    rng = np.random.default_rng(31)
    k_lens = rng.integers(512, 4097, 64).astype(np.int32)
    q_lens = np.ones(64, np.int32)
    check_plan_covers(32, 8, q_lens, k_lens, False, kv_cache_fp8=True)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    n = []
    for fp8 in (False, True):
        p = ops.make_params(64, 32, 8, 128, 16, 20000, 256, False, 0.1, kv_cache_fp8=fp8)
        n.append(ops.pa_plan_varlen(p, cu, k_lens)[1].num_small_items)
    assert n[1] > n[0]
    # beside tiled items (prefill rows) an E4M3 cache gets the plan of a bf16
    # cache that the LDS-DMA kernel does not run (block size 48); the DMA
    # kernel's mixed launch (bf16, power-of-two block size) cuts decode ranges
    # more finely (three workgroups per compute unit)
    q_mix = np.concatenate([np.ones(56, np.int32), np.full(8, 700, np.int32)])
    k_mix = np.concatenate([k_lens[:56], np.full(8, 900, np.int32)])
    cu_mix = np.concatenate([[0], np.cumsum(q_mix)]).astype(np.int32)
    words, small = [], []
    for fp8, bs in ((False, 48), (True, 16), (False, 16)):
        p = ops.make_params(64, 32, 8, 128, bs, 20000, 256, True, 0.1, kv_cache_fp8=fp8)
        w, info = ops.pa_plan_varlen(p, cu_mix, k_mix)
        assert info.num_tiled_items > 0
        words.append(w)
        small.append(info.num_small_items)
    assert np.array_equal(words[0], words[1])
    assert small[2] > small[1]
    p = params()
    p.kv_cache_fp8 = 2
    with pytest.raises(ops.PaError) as e:
        ops.pa_plan_varlen(p, CU, SK)
    assert e.value.status == ops.PA_ERR_INVALID_ARGUMENT

def test_mixed_launch_order(L):
    """A mixed launch keeps each (sequence, KV head)'s tiled row blocks on one
    XCD (workgroup i runs on XCD i % 8): every group's items share one
    position residue mod 8.  Within each residue class each kind is longest
    first and the two are merged in proportion to their counts (after m items
    the number of tiled items is within one of m * tiled / all); the XCDs'
    tiled work differs by less than the largest group."""
    wl = W.make("chunked_prefill_mix", materialise=False)
    p = ops.make_params(wl.B, wl.H, wl.Hkv, wl.D, wl.BS, wl.num_blocks, wl.block_table.shape[1],
                        True, wl.scale)
    words, info = ops.pa_plan_varlen(p, wl.cu_seqlens_q, wl.k_lens)
    items, _ = parse(words, info)
    pos = np.arange(len(items))
    tiled = items[:, 7] == 1
    groups = {}
    for i in np.where(tiled)[0]:
        groups.setdefault((items[i, 0], items[i, 1]), set()).add(i % 8)
    assert all(len(x) == 1 for x in groups.values())
    assert len(items) % 8 == 0       # equal queues: no slot is lent
    gwork = {}
    cost_all = (items[:, 5] - items[:, 4]).astype(np.int64) * np.where(tiled, items[:, 3], 128)
    for i in np.where(tiled)[0]:
        gwork[(items[i, 0], items[i, 1])] = gwork.get((items[i, 0], items[i, 1]), 0) + cost_all[i]
    xwork = [int(cost_all[(pos % 8 == x) & tiled].sum()) for x in range(8)]
    assert max(xwork) - min(xwork) <= max(gwork.values())
    for x in range(8):
        sub = items[pos % 8 == x]
        t = sub[:, 7] == 1
        for kind in (False, True):
            it = sub[t == kind]
            cost = (it[:, 5] - it[:, 4]).astype(np.int64) * (it[:, 3] if kind else 128)
            assert np.all(np.diff(cost) <= 0)
        n, nt = len(sub), int(t.sum())
        m = np.arange(1, n + 1)
        assert np.all(np.abs(np.cumsum(t) - m * nt / n) <= 1.0)


def test_large_plan_order_is_stable(L):
    """From 2048 items up the planner orders by a radix sort: costs are
    non-increasing and equal costs keep the units' order (sequence, KV head,
    first key)."""
    B, H, Hkv = 600, 32, 8
    rng = np.random.default_rng(5)
    k_lens = rng.integers(100, 3000, size=B).astype(np.int32)
    cu = np.arange(B + 1, dtype=np.int32)
    p = ops.make_params(B, H, Hkv, 128, 16, 200000, 256, True, 0.1)
    words, info = ops.pa_plan_varlen(p, cu, k_lens)
    items, _ = parse(words, info)
    assert len(items) >= 2048 and np.all(items[:, 7] == 0)
    cost = (items[:, 5] - items[:, 4]).astype(np.int64)
    assert np.all(np.diff(cost) <= 0)
    key = items[:, 0].astype(np.int64) * 1 << 40 | items[:, 1].astype(np.int64) << 32 | items[:, 4]
    same = np.diff(cost) == 0
    assert np.all(np.diff(key)[same] > 0)


# ---------------------------------------------------------------- cascade decision
def _brute_common_prefix(cu, sk, bt, BS, NB):
    B = len(sk)
    if B < 2:
        return 0
    limit = min(int(sk[b]) - int(cu[b + 1] - cu[b]) for b in range(B))
    n = 0
    while (n + 1) * BS <= limit:
        col = [int(bt[b][n]) for b in range(B)]
        if col[0] < 0 or col[0] >= NB or any(c != col[0] for c in col):
            break
        n += 1
    return n * BS


def test_cascade_decide_on_workloads(L):
    wl = W.make("cascade_prefix", materialise=False)
    p = ops.make_params(wl.B, wl.H, wl.Hkv, wl.D, wl.BS, wl.num_blocks, wl.block_table.shape[1],
                        True, wl.scale)
    # measured on MI355X: single pass 37.9 us, cascade 41.4 us (the 8.4 MB
    # prefix is re-read from the last-level cache): the model keeps the
    # single pass
    P, use = ops.pa_cascade_decide(p, wl.cu_seqlens_q, wl.k_lens, wl.block_table)
    assert P == wl.spec.shared_prefix and not use
    P8, use8 = ops.pa_cascade_decide(p, wl.cu_seqlens_q, wl.k_lens, wl.block_table, 1)
    assert P8 == P and not use8
    wl2 = W.make("decode_llama8b", materialise=False)
    p2 = ops.make_params(wl2.B, wl2.H, wl2.Hkv, wl2.D, wl2.BS, wl2.num_blocks,
                         wl2.block_table.shape[1], True, wl2.scale)
    assert ops.pa_cascade_decide(p2, wl2.cu_seqlens_q, wl2.k_lens, wl2.block_table) == (0, False)


@pytest.mark.parametrize("seed", range(12))
def test_cascade_common_prefix_brute_force(L, seed):
    rng = np.random.default_rng(300 + seed)
    B = int(rng.integers(1, 12))
    BS = int(rng.choice([16, 32]))
    shared = int(rng.integers(0, 20))
    q_lens = rng.integers(1, 40, B)
    k_lens = q_lens + rng.integers(0, 30 * BS, B)
    nblk = (k_lens + BS - 1) // BS
    MB = int(nblk.max()) + 2
    NB = shared + int(nblk.sum()) + 5
    bt = np.full((B, MB), -1, np.int32)
    prefix = rng.permutation(NB)[:shared]
    free = [x for x in rng.permutation(NB) if x not in set(prefix.tolist())]
    c = 0
    for b in range(B):
        for j in range(int(nblk[b])):
            if j < shared:
                bt[b, j] = prefix[j]
            else:
                bt[b, j] = free[c]
                c += 1
    if B > 1 and shared > 3 and seed % 3 == 0:
        bt[B - 1, shared - 2] = free[c]          # a row that diverges early
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    p = ops.make_params(B, 8, 2, 64, BS, NB, MB, True, 0.125)
    P, use = ops.pa_cascade_decide(p, cu, k_lens.astype(np.int32), bt)
    assert P == _brute_common_prefix(cu, k_lens, bt, BS, NB)
    assert (not use) or (P >= 256 and B >= 8)


def test_cascade_decide_thresholds(L):
    """The section's thresholds: prefix >= 256 tokens, >= 8 requests, causal;
    and the cost model declines a prefix that saves little against long
    private suffixes."""
    def case(B, P, suffix, causal=True, BS=16):
        nb_p, nb_s = P // BS, (suffix + BS - 1) // BS
        bt = np.zeros((B, nb_p + nb_s), np.int32)
        bt[:, :nb_p] = np.arange(nb_p)
        bt[:, nb_p:] = nb_p + np.arange(B * nb_s).reshape(B, nb_s)
        q_lens = np.ones(B, np.int32)
        k_lens = np.full(B, P + suffix, np.int32)
        cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
        p = ops.make_params(B, 32, 8, 128, BS, nb_p + B * nb_s, nb_p + nb_s, causal, 0.088)
        return ops.pa_cascade_decide(p, cu, k_lens, bt)
    assert case(64, 16384, 300) == (16384, True)        # 64 x 64 MB of prefix re-reads
    assert case(4, 16384, 300) == (16384, False)        # fewer than 8 requests
    assert case(64, 128, 300) == (128, False)           # prefix below 256
    assert case(64, 16384, 300, causal=False) == (16384, False)
    assert case(8, 256, 100000)[1] is False             # saves 0.2 % of the bytes
    assert case(32, 2048, 300)[1] is False              # the measured cascade_prefix shape


# ---------------------------------------------------------------- sliding window plans
@pytest.mark.parametrize("seed", range(6))
def test_plan_covers_sliding_window(L, seed):
    """With a window of W keys, each row block's ranges start at a multiple of
    16 at or below its first row's window start and still tile up to the
    block's causal end; every visible key of every row is covered."""
    rng = np.random.default_rng(900 + seed)
    G = int(rng.choice([1, 4, 8]))
    Hkv = 2
    B = 6
    q_lens = rng.integers(1, 300, B).astype(np.int32)
    q_lens[::2] = 1                                   # decode rows too
    k_lens = (q_lens + rng.integers(0, 2000, B)).astype(np.int32)
    W_ = int(rng.choice([1, 16, 100, 1000]))
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    BS = 16
    MB = int((k_lens.max() + BS - 1) // BS)
    force = int(rng.choice([0, 3]))
    p = ops.make_params(B, G * Hkv, Hkv, 64, BS, 40000, MB, True, 0.1, sliding_window=W_)
    words, info = ops.pa_plan_varlen(p, cu, k_lens, force)
    assert info.sliding_window == W_
    items, red = parse(words, info)
    cover = {}
    for seq, kvh, row0, nrows, k0, k1, prow, word7, *_ in items:
        assert k0 % 16 == 0
        for r in range(row0, row0 + nrows):
            cover.setdefault((seq, kvh, r), []).append((k0, k1))
    for b in range(B):
        Lq, Lk = int(q_lens[b]), int(k_lens[b])
        for kvh in range(Hkv):
            for r in range(Lq * G):
                ranges = sorted(cover[(b, kvh, r)])
                i = r // G
                hi = min(Lk - 1, i + Lk - Lq)
                lo = max(0, i + Lk - Lq - (W_ - 1))
                pos = ranges[0][0]
                assert pos <= max(lo, 0) or hi < lo
                for k0, k1 in ranges:
                    assert k0 == pos
                    pos = k1
                assert pos >= hi + 1 or hi < lo


def test_num_cus(L):
    """num_cus = 256 plans exactly as num_cus = 0 (PA_PLAN_TARGET_CUS); a
    smaller device gets fewer, longer decode pieces; out-of-range values are
    rejected."""
    wl = W.make("decode_llama8b", materialise=False)
    def plan(n):
        p = ops.make_params(wl.B, wl.H, wl.Hkv, wl.D, wl.BS, wl.num_blocks,
                            wl.block_table.shape[1], True, wl.scale, num_cus=n)
        return ops.pa_plan_varlen(p, wl.cu_seqlens_q, wl.k_lens)
    w0, i0 = plan(0)
    w256, i256 = plan(256)
    assert np.array_equal(w0, w256) and i0.as_dict() == i256.as_dict()
    w32, i32 = plan(32)
    assert i32.num_small_items < i0.num_small_items
    check = lambda n: ops.pa_plan_varlen(
        ops.make_params(2, 4, 2, 64, 16, 16, 6, True, 0.125, num_cus=n), CU, SK)
    for bad in (-1, 65537):
        with pytest.raises(ops.PaError):
            check(bad)


def test_wide_rows_rule(L):
    """Prefill-only plans use 256-row blocks at D = 64, or when the prefills
    average 2048 query tokens or more and the cache is one the DMA kernel
    does not run (E4M3, or a block size that is not a power of two); the 8
    prefills of chunked_prefill_mix (592-1811 tokens) keep 128-row blocks
    either way, and a plan with decode rows always does."""
    def rows(name, bs=None, fp8=False, d=None):
        wl = W.make(name, materialise=False)
        bs = bs or wl.BS
        p = ops.make_params(wl.B, wl.H, wl.Hkv, d or wl.D, bs, -(-wl.num_blocks * wl.BS // bs),
                            -(-wl.block_table.shape[1] * wl.BS // bs), True, wl.scale,
                            kv_cache_fp8=fp8)
        return ops.pa_plan_varlen(p, wl.cu_seqlens_q, wl.k_lens)[1].tiled_rows
    short, long_ = "chunked_prefill_mix_prefill", "prefill_causal_8k"
    for kw in ({}, {"bs": 64}, {"bs": 48}, {"fp8": True}):
        assert rows(short, **kw) == ops.PA_TILED_ROWS
    assert rows(long_) == ops.PA_TILED_ROWS                   # bf16, BS = 32: DMA kernel
    assert rows(long_, bs=64) == ops.PA_TILED_ROWS
    assert rows(long_, bs=48) == ops.PA_TILED_ROWS_WIDE
    assert rows(long_, fp8=True) == ops.PA_TILED_ROWS_WIDE
    assert rows(short, d=64) == ops.PA_TILED_ROWS_WIDE
    assert rows("chunked_prefill_mix") == ops.PA_TILED_ROWS


def test_binding_checks_fwd_shapes():
    """The forward bindings check shapes, strides and sizes against the params
    and the plan before any launch (CPU tensors: a call that passes the checks
    stops at the device-tensor check instead, with TypeError)."""
    import torch
    wl = W.make("tiny_mixed")
    T, H, D, Hkv = wl.T, wl.H, wl.D, wl.Hkv
    p = ops.make_params(wl.B, H, Hkv, D, wl.BS, wl.num_blocks, wl.block_table.shape[1], True,
                        wl.scale)
    words, info = ops.pa_plan_varlen(p, wl.cu_seqlens_q, wl.k_lens)
    good = dict(worklist=torch.from_numpy(words), q=torch.zeros(T, H, D, dtype=torch.bfloat16),
                kv_cache=torch.zeros(2, wl.num_blocks, wl.BS, Hkv, D, dtype=torch.bfloat16),
                cu_seqlens_q=torch.from_numpy(wl.cu_seqlens_q.astype(np.int32)),
                seqused_k=torch.from_numpy(wl.k_lens.astype(np.int32)),
                block_table=torch.from_numpy(wl.block_table.astype(np.int32)),
                out=torch.zeros(T, H, D, dtype=torch.bfloat16),
                lse=torch.zeros(T, H, dtype=torch.float32))

    def call(**bad):
        a = dict(good, **bad)
        ops.pa_varlen_fwd(p, info, a["worklist"], a["q"], a["kv_cache"], a["cu_seqlens_q"],
                          a["seqused_k"], a["block_table"], a["out"], a["lse"])

    with pytest.raises(TypeError):        # all checks pass; CPU tensors stop here
        call()
    bt = good["block_table"]
    wide = torch.zeros(bt.shape[0], bt.shape[1] + 3, dtype=torch.int32)
    for bad in (dict(out=torch.zeros(T + 1, H, D, dtype=torch.bfloat16)),
                dict(out=torch.zeros(T, H, D + 8, dtype=torch.bfloat16)),
                dict(out=torch.zeros(T, D, H, dtype=torch.bfloat16).transpose(1, 2)),
                dict(q=torch.zeros(T - 1, H, D, dtype=torch.bfloat16)),
                dict(lse=torch.zeros(T, H + 1, dtype=torch.float32)),
                dict(lse=torch.zeros(H, T, dtype=torch.float32).t()),
                dict(kv_cache=torch.zeros(2, wl.num_blocks - 1, wl.BS, Hkv, D,
                                          dtype=torch.bfloat16)),
                dict(kv_cache=torch.zeros(2, wl.num_blocks, wl.BS, Hkv, D, dtype=torch.uint8)),
                dict(block_table=bt[:1]),
                dict(block_table=bt[:, :-1]),
                dict(block_table=wide[:, :bt.shape[1]]),          # row stride differs from params
                dict(cu_seqlens_q=good["cu_seqlens_q"][:-1]),
                dict(seqused_k=good["seqused_k"][:1]),
                dict(worklist=good["worklist"][:-1])):
        with pytest.raises(ValueError):
            call(**bad)
    # the E4M3 entry point: the scales must cover every KV head
    kv8 = torch.zeros(2, wl.num_blocks, wl.BS, Hkv, D, dtype=torch.uint8)
    with pytest.raises(ValueError):
        ops.pa_varlen_fwd_fp8(p, info, good["worklist"], good["q"], kv8, good["cu_seqlens_q"],
                              good["seqused_k"], bt, torch.ones(Hkv - 1), torch.ones(Hkv),
                              good["out"], good["lse"])
    with pytest.raises(ValueError):
        ops.pa_varlen_fwd_ex(p, info, good["worklist"], good["q"], good["kv_cache"],
                             good["cu_seqlens_q"], good["seqused_k"], bt, good["out"],
                             good["lse"], s_aux=torch.zeros(H + 1))


def test_window_params_validation(L):
    E = ops.PA_ERR_INVALID_ARGUMENT
    cu = np.array(CU, np.int32)
    sk = np.array(SK, np.int32)
    info = ops.PlanInfo()
    for causal, W_ in ((False, 16), (True, -1)):
        p = ops.make_params(len(SK), 8, 2, 64, 16, 64, 8, causal, 0.1, sliding_window=W_)
        st = L.pa_plan_varlen(ctypes.byref(p), cu.ctypes.data_as(ops._I32P),
                              sk.ctypes.data_as(ops._I32P), 0, None, 0, ctypes.byref(info))
        assert st == E
    # a plan made without the window does not serve a call with one
    p = params()
    _, info = ops.pa_plan_varlen(p, CU, SK)
    pw = params()
    pw.sliding_window = 32
    assert _fwd_call(L, pw, info) == E
    # the extended entry point wants its options and a known cache format
    P = ctypes.c_void_p
    assert L.pa_varlen_fwd_ex(ctypes.byref(p), ctypes.byref(info), P(0x1000), P(0x2000), P(0x3000),
                              P(0x4000), P(0x5000), P(0x6000), None, info.num_tokens, P(0x7000),
                              P(0x8000), P(0x10000), 1 << 30, None) == E
    bad = ops.FwdOptions(7, None, None, None)
    assert L.pa_varlen_fwd_ex(ctypes.byref(p), ctypes.byref(info), P(0x1000), P(0x2000), P(0x3000),
                              P(0x4000), P(0x5000), P(0x6000), ctypes.byref(bad), info.num_tokens,
                              P(0x7000), P(0x8000), P(0x10000), 1 << 30, None) == E


def test_upload_words_rejects_bad_arguments_before_any_launch(L):
    P = ctypes.c_void_p
    buf = (ctypes.c_int32 * 8)()
    a = ctypes.addressof(buf)
    a16 = a + (-a) % 16 if (a % 16) else a
    bad = [(P(a16), P(a16), -1), (None, P(a16), 4), (P(a16), None, 4),
           (P(a16 + 4), P(a16), 4), (P(a16), P(a16 + 4), 4)]
    for src, dst, n in bad:
        assert L.pa_upload_words(src, dst, n, None) == 1     # PA_ERR_INVALID_ARGUMENT
    assert L.pa_upload_words(None, None, 0, None) == 0       # nothing to copy


def test_plan_with_no_query_tokens(L):
    """A batch whose sequences have no query tokens plans no work: the forward
    call then launches nothing and writes nothing."""
    p = params(batch=3, max_blocks_per_seq=4)
    words, info = ops.pa_plan_varlen(p, np.array([0, 0, 0, 0], np.int32),
                                     np.array([0, 30, 1], np.int32))
    assert info.num_tokens == 0
    assert info.num_small_items == info.num_tiled_items == info.num_reduce_items == 0
    assert info.workspace_bytes == 0 or info.num_partial_rows == 0
