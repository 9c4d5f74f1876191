"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/msa_nvfp4.h declares, sizes workspaces, and rejects
bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa_nvfp4.h")

nb = pytest.importorskip("nvfp4_kv_cache_amd")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(nb.LIB_PATH):
        pytest.skip("library not built")
    return nb.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert {"msa_nvfp4_quantize", "msa_indexer_decode", "msa_sparse_attn_decode"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
        assert n in nb.binding.SIGNATURES, f"binding lacks {n}"


def test_status_strings(L):
    for s in range(5):
        assert nb.msa_status_string(s).startswith("MSA_")
    assert "unknown" in nb.msa_status_string(99)


def _attn_splits(pairs, num_sel):
    # the launch plan: few (query token, KV head) pairs -> one workgroup per
    # selected block; otherwise one block per wavefront (4 per workgroup),
    # R slots per wavefront, the R whose grid fits the 512 workgroups the
    # chip holds at once with the shortest chain (R blocks at 3 units with
    # at most one workgroup per CU, 5 with two, + 1.5 for a split merge;
    # ties to fewer splits), else one split per pair
    if pairs * num_sel <= 384:
        return num_sel
    sp = lambda r: -(-num_sel // (4 * r))
    best = None
    for r in range(1, -(-num_sel // 4) + 1):
        wgs = pairs * sp(r)
        if wgs > 512:
            continue
        cost = r * (30 if wgs <= 256 else 50) + (15 if sp(r) > 1 else 0)
        if best is None or (cost, sp(r)) < best:
            best = (cost, sp(r))
    return best[1] if best else 1


@pytest.mark.parametrize("seqs,q,heads,sel", [(16, 8, 32, 17), (8, 1, 32, 17), (32, 1, 32, 17),
                                              (1, 1, 32, 17), (2, 1, 8, 64), (45, 1, 32, 17),
                                              (24, 1, 32, 17), (40, 1, 32, 17), (48, 1, 32, 17),
                                              (96, 1, 32, 17), (4, 1, 32, 64), (16, 1, 32, 33),
                                              (40, 1, 32, 64), (96, 1, 32, 64)])
def test_workspace_sizes(L, seqs, q, heads, sel):
    assert nb.msa_indexer_workspace_bytes(8, 1, 2048) == 8 * 2048 * 4
    assert nb.msa_indexer_workspace_bytes(0, 1, 10) == 0
    rows = seqs * q * heads
    splits = _attn_splits(seqs * q * heads // 8, sel)
    # partials (o, then m and l) and one arrival counter per (token, KV head)
    want = (rows * splits * 128 * 4 + rows * splits * 2 * 4 + seqs * q * heads // 8 * 4
            if splits > 1 else 0)
    got = nb.msa_attn_workspace_bytes(seqs, q, heads, sel)
    assert want <= got <= want + 3 * 255


def _desc(heads=4, d=128, bt=128, pages=10):
    return nb.PoolDesc(heads, d, bt, 0, pages)


def test_quantize_rejects_before_launch(L):
    f = L.msa_nvfp4_quantize
    assert f(None, None, None, 1, None, None, None) == 1
    assert f(ctypes.byref(_desc(d=64)), None, None, 1, None, None, None) == 2
    assert f(ctypes.byref(_desc(heads=9)), None, None, 1, None, None, None) == 2
    assert f(ctypes.byref(_desc()), None, None, -1, None, None, None) == 1
    assert f(ctypes.byref(_desc()), None, None, 0, None, None, None) == 0      # no-op
    assert f(ctypes.byref(_desc()), None, None, 5, None, None, None) == 1      # null buffers
    assert f(ctypes.byref(_desc()), 16, 8, 5, 3, 16, None) == 1                # misaligned codes


def test_indexer_rejects_before_launch(L):
    f = L.msa_indexer_decode
    d = ctypes.byref(_desc())
    ok = dict(q=32, mb=4, ns=1, qps=1, topk=16)

    def call(desc=d, q=32, mb=4, ns=1, qps=1, topk=16, ptr=256, ws=None, wsb=0):
        return f(desc, ptr, ptr, ptr, ptr, q, ptr, mb, ptr, ns, qps, topk, ptr, None,
                 ws, wsb, None)
    assert call(desc=None) == 1
    assert call(q=16) == 2                       # not 8 query heads per index head
    assert call(topk=8) == 2
    assert call(qps=9) == 2
    assert call(qps=0) == 1
    assert call(ns=0) == 0
    assert call(ptr=None) == 1
    assert call(ptr=4096 + 8) == 1               # misaligned
    assert call(ws=None) == 3                    # workspace missing
    assert call(ws=4096, wsb=16) == 3            # too small
    assert call(desc=ctypes.byref(_desc(bt=64))) == 2


def test_noalloc_indexer_rejects_before_launch(L):
    # the same argument checks as msa_indexer_decode, and more block scores
    # than the library's device array holds is refused (nothing launched)
    f = L.msa_indexer_decode_noalloc
    d = ctypes.byref(_desc())

    def call(desc=d, q=32, mb=4, ns=1, qps=1, topk=16, ptr=256):
        return f(desc, ptr, ptr, ptr, ptr, q, ptr, mb, ptr, ns, qps, topk, ptr, None, None)
    assert nb.NOALLOC_MAX_SCORES == 1 << 20
    assert call(desc=None) == 1
    assert call(q=16) == 2
    assert call(topk=8) == 2
    assert call(qps=9) == 2
    assert call(ns=0) == 0
    assert call(ptr=None) == 1
    assert call(ptr=4096 + 8) == 1
    assert call(ns=1025, mb=1024) == 3           # 1,049,600 scores > 2^20
    assert call(ns=128, qps=8, mb=1025) == 3     # 1,049,600 scores > 2^20


def test_attention_rejects_before_launch(L):
    f = L.msa_sparse_attn_decode
    d = ctypes.byref(_desc())

    def call(desc=d, q=32, mb=4, ns=1, qps=1, nsel=17, scale=0.088, ptr=256, ws=None, wsb=0):
        return f(desc, ptr, ptr, ptr, ptr, ptr, q, ptr, mb, ptr, ns, qps, ptr, nsel, scale,
                 ptr, ws, wsb, None)
    assert call(desc=None) == 1
    assert call(q=24) == 2
    assert call(nsel=0) == 2 and call(nsel=65) == 2
    assert call(scale=0.0) == 1 and call(scale=float("nan")) == 1
    assert call(ns=0) == 0
    assert call(ptr=None) == 1
    assert call(ptr=4096 + 4) == 1              # misaligned
    assert call(ws=None) == 3                    # 17 blocks need split partials


def test_select_attention_rejects_before_launch(L):
    f = L.msa_sparse_attn_select_decode
    d = ctypes.byref(_desc())

    def call(desc=d, q=32, mb=4, ns=1, qps=1, bs=256, topk=16, ids=None, scale=0.088, ptr=256,
             ws=None, wsb=0):
        return f(desc, ptr, ptr, ptr, ptr, ptr, q, ptr, mb, ptr, ns, qps, bs, topk, ids, scale,
                 ptr, ws, wsb, None)
    assert call(desc=None) == 1
    assert call(q=24) == 2
    assert call(topk=17) == 2
    assert call(qps=9) == 2
    assert call(scale=-1.0) == 1
    assert call(ns=0) == 0
    assert call(bs=None) == 1                    # no block scores
    assert call(bs=4096 + 2) == 1                # misaligned scores
    assert call(ids=4096 + 2) == 1               # misaligned ids
    assert call(ptr=None) == 1
    assert call(ws=None) == 3                    # 17 blocks need split partials
    assert call(ws=4096, wsb=64) == 3


def test_two_stage_indexer_rejects_before_launch(L):
    d = ctypes.byref(_desc())
    scan = L.msa_indexer_scan
    assert scan(None, 256, 256, 256, 256, 32, 256, 4, 256, 1, 1, 256, None) == 1
    assert scan(d, 256, 256, 256, 256, 24, 256, 4, 256, 1, 1, 256, None) == 2
    assert scan(d, 256, 256, 256, 256, 32, 256, 4, 256, 0, 1, None, None) == 0
    assert scan(d, 256, 256, 256, 256, 32, 256, 4, 256, 1, 1, None, None) == 1
    sel = L.msa_indexer_select
    assert sel(256, 256, 4, 1, 1, 15, 256, None, None) == 2
    assert sel(None, 256, 4, 1, 1, 16, 256, None, None) == 1
    assert sel(256, 256, 0, 1, 1, 16, 256, None, None) == 1
    assert sel(256, 256, 4, 0, 1, 16, None, None, None) == 0
    assert sel(256, 256, 4, 1, 9, 16, 256, None, None) == 2


def test_shared_prefix_scan_rejects_before_launch(L):
    f = L.msa_indexer_scan_shared
    d = ctypes.byref(_desc())

    def call(desc=d, q=32, mb=4, ns=1, qps=1, ng=1, gl=256, gb=256, mgb=2, sg=256, bs=256,
             ptr=256):
        return f(desc, ptr, ptr, ptr, ptr, q, ptr, mb, ptr, ns, qps, ng, gl, gb, mgb, sg, bs, None)
    assert call(desc=None) == 1
    assert call(q=24) == 2
    assert call(qps=9) == 2
    assert call(ng=-1) == 1
    assert call(ng=65536) == 1
    assert call(mgb=0) == 1                      # groups need shared blocks
    assert call(mgb=5) == 1                      # more than max_blocks
    assert call(ns=0) == 0
    assert call(gl=None) == 1
    assert call(gb=None) == 1
    assert call(sg=None) == 1
    assert call(gl=4096 + 2) == 1                # misaligned group arrays


def _groups_reference(bt, lens, q):
    """The grouping rule read directly: valid sequences keyed by their block-0
    page (>= 0), in order of first appearance; a key with two or more members
    shares the largest r such that every member has at least r blocks and
    the same non-negative pages in blocks 0..r-1 as the first member."""
    nb = [(int(L) + 127) // 128 for L in lens]
    valid = [q <= int(L) <= bt.shape[1] * 128 for L in lens]
    keys = []
    members = {}
    for b in range(len(lens)):
        if valid[b] and bt[b, 0] >= 0:
            k = int(bt[b, 0])
            if k not in members:
                keys.append(k)
                members[k] = []
            members[k].append(b)
    lead, blocks, group = [], [], [-1] * len(lens)
    for k in keys:
        m = members[k]
        if len(m) < 2:
            continue
        best = 0
        for r in range(1, bt.shape[1] + 1):
            if all(r <= nb[x] and all(bt[x, i] == bt[m[0], i] >= 0 for i in range(r)) for x in m):
                best = r
        if best == 0:
            continue
        for x in m:
            group[x] = len(lead)
        lead.append(m[0])
        blocks.append(best)
    return lead, blocks, group


def test_shared_prefix_groups_match_the_rule(L):
    import numpy as np
    import torch
    from msa_workloads import get_config, tiny_config
    cases = [get_config(4), get_config(2), get_config(0),
             tiny_config([1000, 700, 3000, 130, 2600, 900], 2, seed=72,
                         shared=[([0, 1, 3], 6), ([2, 4], 20)]),
             tiny_config([2300] * 9 + [500], 1, seed=71, shared=[(list(range(9)), 17)])]
    rng = np.random.default_rng(5)
    for t in range(30):                          # random aliasing, invalid lengths and pages
        ns, mb = int(rng.integers(1, 12)), int(rng.integers(1, 9))
        bt = rng.integers(-1, 4, size=(ns, mb)).astype(np.int32)
        bt[rng.random(ns) < 0.5, 0] = 1
        lens = rng.integers(-2, mb * 128 + 40, size=ns).astype(np.int32)
        cases.append((bt, lens, int(rng.integers(1, 3))))
    for c in cases:
        bt, lens, q = (c if isinstance(c, tuple) else
                       (c.block_table.astype(np.int32), np.asarray(c.seq_lens, np.int32), c.q_per_seq))
        lead, blocks, mgb, group = nb.msa_shared_prefix_groups(torch.from_numpy(bt),
                                                                torch.from_numpy(lens), q)
        want = _groups_reference(bt, lens, q)
        assert lead.tolist() == want[0] and blocks.tolist() == want[1], (bt, lens)
        assert group.tolist() == want[2]
        assert mgb == (max(want[1]) if want[1] else 0)
    # the ragged workload: one group of all 45 requests sharing 128 blocks
    w4 = get_config(4)
    lead, blocks, mgb, group = nb.msa_shared_prefix_groups(
        torch.from_numpy(w4.block_table.astype(np.int32)), torch.tensor(w4.seq_lens, dtype=torch.int32), 1)
    assert lead.tolist() == [0] and blocks.tolist() == [128] and mgb == 128
    assert group.tolist() == [0] * 45
    f = L.msa_shared_prefix_groups
    out = (ctypes.c_int32 * 4)()
    assert f(None, 4, None, 0, 1, None, None, None, ctypes.byref(out, 0), ctypes.byref(out, 4)) == 0
    assert f(None, 4, None, 2, 1, None, None, None, ctypes.byref(out, 0), ctypes.byref(out, 4)) == 1
    assert f(None, 0, None, 0, 1, None, None, None, ctypes.byref(out, 0), ctypes.byref(out, 4)) == 1


def test_scale_layout_view_matches_header_formula():
    import torch
    from nvfp4_kv_cache_amd import scales_rows
    p_, h_ = 2, 3
    phys = torch.arange(p_ * h_ * 1024, dtype=torch.int64).reshape(p_, h_, 1024)
    rows = scales_rows(phys)
    for r in range(128):
        for g in range(8):
            off = ((g // 2) * 16 + r % 16) * 16 + (r // 16) * 2 + g % 2
            assert int(rows[1, 2, r, g]) == (1 * h_ + 2) * 1024 + off


def test_qkv_rope_insert_rejects_before_launch(L):
    f = L.msa_qkv_rope_insert
    kv, idx = ctypes.byref(_desc(heads=4)), ctypes.byref(_desc(heads=4))
    fake = ctypes.c_void_p(1 << 20)   # never dereferenced: every call below fails a host check

    def call(n=1, kvd=kv, idxd=idx, qn=None, eps=1e-6, rot=128, theta=1e4, qkv=fake):
        return f(qkv, n, fake, fake, kvd, fake, fake, fake, fake, idxd, fake, fake, qn, None,
                 eps, rot, theta, fake, fake, None)

    assert call(n=-1) == 1
    assert call(kvd=None) == 1
    assert call(kvd=ctypes.byref(_desc(d=64))) == 2
    assert call(idxd=ctypes.byref(_desc(heads=9))) == 2
    assert call(idxd=ctypes.byref(_desc(pages=0))) == 1
    for bad_rot in (-32, 16, 48, 160):
        assert call(rot=bad_rot) == 2
    assert call(theta=0.5) == 1                 # rope needs theta > 1
    assert call(theta=float("nan")) == 1
    assert call(qn=fake, eps=-1.0) == 1         # negative eps with a norm
    assert call(n=0, qkv=None) == 0             # nothing to do
    assert call(qkv=None) == 1
    assert call(qkv=ctypes.c_void_p((1 << 20) + 8)) == 1   # qkv must be 16-byte aligned
    assert call(n=1 << 31) == 2


def test_mono_workspace_layout(L):
    # scores, partial o, partial (m, l), then the counters: every part
    # 256-byte aligned; the error word is the last 32-bit word
    def a256(x):
        return -(-x // 256) * 256
    for ns, q, mb in [(1, 1, 32), (4, 1, 33), (2, 8, 40), (3, 2, 1)]:
        tq, rows = ns * q, ns * q * 32
        want = (a256(tq * mb * 4) + a256(rows * mb * 128 * 4) + a256(rows * mb * 2 * 4)
                + a256(((ns + tq * 4) * 128 + ns * 16 + 1) * 4))
        assert nb.msa_decode_mono_workspace_bytes(ns, q, 32, mb) == want
    assert nb.msa_decode_mono_workspace_bytes(0, 1, 32, 4) == 0


def test_mono_rejects_before_launch(L):
    f = L.msa_decode_mono
    d4 = ctypes.byref(_desc())

    def call(idx=d4, kv=d4, q=32, mb=4, ns=1, qps=1, topk=16, ids=None, scale=0.088, ptr=256,
             ws=4096, wsb=None):
        if wsb is None:
            wsb = nb.msa_decode_mono_workspace_bytes(max(ns, 1), qps, 32, mb)
        return f(idx, ptr, ptr, ptr, ptr, kv, ptr, ptr, ptr, ptr, ptr, q, ptr, mb, ptr, ns, qps,
                 topk, ids, scale, ptr, ws, wsb, None)
    assert call(idx=None) == 1 and call(kv=None) == 1
    assert call(idx=ctypes.byref(_desc(heads=2))) == 2   # the scan's wavefronts: 4 index heads
    assert call(kv=ctypes.byref(_desc(heads=8))) == 2
    assert call(q=64) == 2
    assert call(topk=8) == 2
    assert call(qps=9) == 2
    assert call(idx=ctypes.byref(_desc(bt=64))) == 2
    assert call(mb=257) == 2                             # 4 x 257 block workgroups > 1024
    assert call(ns=2, qps=8, mb=17) == 2                 # 16 x 4 x 17 > 1024
    assert call(ns=2, qps=8, mb=16, ptr=None) == 1       # at the bound: reaches the null check
    assert call(mb=256, ptr=None) == 1                   # 1 x 32K tokens: at the bound
    assert call(scale=0.0) == 1
    assert call(ns=0) == 0
    assert call(ptr=None) == 1
    assert call(ptr=4096 + 8) == 1                       # misaligned
    assert call(ids=4096 + 2) == 1
    assert call(ws=None) == 3
    assert call(ws=4096 + 16) == 3                       # workspace not 256-byte aligned
    assert call(wsb=64) == 3


def test_host_checks_under_asan_and_ubsan():
    """The host tests above, again in a child process on the library built
    with host-side AddressSanitizer and UndefinedBehaviorSanitizer
    (python -m nvfp4_kv_cache_amd.build --sanitize; __graft_entry__.build()
    builds it): every argument check, the group derivation and the launch
    set-up run without a memory error or undefined behaviour. No GPU is
    touched (every call in those tests is rejected before a launch)."""
    import subprocess
    import sys
    from nvfp4_kv_cache_amd import build as B
    if os.environ.get("MSA_TEST_LIB"):
        pytest.skip("already running on another build of the library")
    if not os.path.exists(B.SAN_LIB):
        pytest.skip("host-sanitized library not built")
    r = subprocess.run([B.HIPCC, "--print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    asan = r.stdout.strip()
    if r.returncode != 0 or not os.path.exists(asan):
        pytest.skip("no AddressSanitizer runtime found")
    env = dict(os.environ, LD_PRELOAD=asan, MSA_TEST_LIB=B.SAN_LIB,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.abspath(__file__), "-q",
                        "-p", "no:cacheprovider", "-k", "not asan_and_ubsan"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:] + r.stderr[-3000:])
    assert " passed" in r.stdout
