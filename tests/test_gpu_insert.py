"""Parity of msa_qkv_rope_insert (through the C ABI) with oracle.insert.

Without normalisation and RoPE the kernel rounds the bf16 inputs themselves,
so every byte must match the oracle bit for bit (pools, FP8 queries, rows
that must stay untouched). With them, the kernel's fp32 values differ from
the oracle's fp64 values by rounding; each byte must then be the encoding of
a value within delta of the oracle's (oracle.acceptance), with delta = 2e-5
times the largest magnitude in the head row (fp32 RMSNorm and rotation error
is below 1e-6 of it), and the count of bytes that need delta must stay small.
"""
import numpy as np
import pytest
import torch

from msa_workloads import synth
from oracle import acceptance as A
from oracle import formats as F
from oracle import insert as I
from oracle import nvfp4 as N

pytestmark = pytest.mark.gpu

WINDOW = 2e-5


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def nb():
    import nvfp4_kv_cache_amd as m
    m.lib()
    return m


def _pools(nb, pages, hkv, hidx, fill):
    out = []
    for h in (hkv, hkv, hidx):
        c, s = nb.empty_pool(pages, h)
        c.fill_(fill)
        s.fill_(fill)
        out.append((c, s))
    return out


def _run(nb, rows, pos, slots, pages, hkv, hidx, qn=None, kn=None, eps=1e-6, rot=128, theta=1e4,
         fill=0x5A):
    t = rows.shape[0]
    dev = "cuda"
    pools = _pools(nb, pages, hkv, hidx, fill)
    q = torch.full((t, 8 * hkv, 128), 0xA5, dtype=torch.uint8, device=dev)
    qi = torch.full((t, 8 * hidx, 128), 0xA5, dtype=torch.uint8, device=dev)
    nb.msa_qkv_rope_insert(rows.to(dev), torch.as_tensor(pos, dtype=torch.int32, device=dev),
                           torch.as_tensor(slots, dtype=torch.int64, device=dev), *pools, q, qi,
                           q_norm_w=None if qn is None else qn.to(dev),
                           k_norm_w=None if kn is None else kn.to(dev), rms_eps=eps,
                           rotary_dim=rot, rope_theta=theta)
    torch.cuda.synchronize()
    host = [(c.cpu().numpy(), nb.scales_rows(s).cpu().numpy()) for c, s in pools]
    return host, q.cpu().numpy(), qi.cpu().numpy()


def _bits(rows):
    return rows.view(torch.int16).numpy().view(np.uint16)


def _special_rows(t, width):
    """bf16 rows holding every E4M3 midpoint and its two bf16 neighbours (both
    signs), values beyond 448, E4M3 subnormals and a subnormal tie, zeros and
    -0, over random rows; all in the query heads of token 0."""
    bits = _bits(synth.projection_rows(31, t, width)).copy()
    flat = bits.reshape(-1)
    mid = torch.from_numpy(F.E4M3_MID.astype(np.float32)).to(torch.bfloat16)
    mb = mid.view(torch.int16).numpy().view(np.uint16).astype(np.int64)
    assert np.array_equal(mid.double().numpy(), F.E4M3_MID)        # exact in bf16
    special = np.concatenate([mb, mb - 1, mb + 1])
    special = np.concatenate([special, special | 0x8000])
    extra = torch.tensor([448.0, 464.0, 1e4, -3e38, 2.0 ** -9, 3 * 2.0 ** -10, 0.0, -0.0],
                         dtype=torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    special = np.concatenate([special.astype(np.uint16), extra])
    flat[:special.size] = special
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)


@pytest.mark.parametrize("hkv,hidx,t", [(4, 4, 37), (2, 1, 9), (1, 3, 130)])
def test_insert_bit_exact_without_norm_and_rope(nb, hkv, hidx, t):
    say(f"[insert exact] hkv={hkv} hidx={hidx} T={t}")
    width = (8 * hkv + 8 * hidx + 2 * hkv + hidx) * 128
    rows = _special_rows(t, width)
    pages = (t + 127) // 128 + 2
    rng = np.random.default_rng(t)
    slots = rng.permutation(pages * 128)[:t].astype(np.int64)
    slots[::7] = -1                                      # not inserted
    slots[3] = pages * 128 + 5                           # past the pool: not inserted
    pos = rng.integers(0, 1 << 20, size=t)
    host, q, qi = _run(nb, rows, pos, slots, pages, hkv, hidx, rot=0)
    opools = [N.empty_pool(pages, h, fill=0x5A) for h in (hkv, hkv, hidx)]
    ok_slots = np.where(slots < pages * 128, slots, -1)
    oq, oqi = I.insert(_bits(rows), pos, ok_slots, *opools, rotary_dim=0)
    assert np.array_equal(q, oq) and np.array_equal(qi, oqi)
    for (gc, gs), (oc, os_) in zip(host, opools):
        assert np.array_equal(gc, oc)
        assert np.array_equal(gs, os_)


# norm: which heads carry RMSNorm weights ("qk" both, "q" / "k" one class).
# Head counts (1, 3) and (3, 1) put rows of several kinds (keys, values,
# index keys) into one wavefront pass of eight rows; (8, 8) is the largest.
@pytest.mark.parametrize("rot,theta,norm,hkv,hidx", [
    (128, 1e4, "qk", 4, 4), (64, 1e6, "qk", 4, 4), (96, 5e5, "", 4, 4), (32, 1e4, "qk", 4, 4),
    (0, 1e4, "qk", 4, 4), (128, 1e4, "", 4, 4), (128, 1e6, "q", 1, 3), (128, 1e4, "k", 3, 1),
    (64, 1e4, "qk", 1, 3), (0, 1e4, "k", 3, 1), (128, 1e4, "qk", 8, 8), (32, 5e5, "q", 2, 1)])
def test_insert_with_norm_and_rope_matches_oracle(nb, rot, theta, norm, hkv, hidx):
    t = 53
    say(f"[insert norm/rope] rot={rot} theta={theta} norm={norm!r} hkv={hkv} hidx={hidx}")
    width = (8 * hkv + 8 * hidx + 2 * hkv + hidx) * 128
    rows = synth.projection_rows(7 + rot + 10 * hkv + hidx, t, width)
    # token 0's first value head: signed zeros and every E2M1 midpoint of
    # scale 1 (amax 6), which the value path must pass through unchanged
    vrow = (8 * hkv + 8 * hidx + hkv) * 128
    rows[0, vrow:vrow + 16] = torch.tensor([-0.0, 0.0, 0.25, -0.75, 1.25, -1.75, 2.5, -3.5, 5.0,
                                            6.0, -0.0, 0.5, -1.0, 1.5, -2.0, 3.0])
    pages = 3
    slots = np.random.default_rng(rot).permutation(pages * 128)[:t].astype(np.int64)
    pos = np.concatenate([[0, 1, 2], np.random.default_rng(1).integers(0, 262144, size=t - 4),
                          [262143]])
    qn = synth.norm_weights(3, 0) if "q" in norm else None
    kn = synth.norm_weights(3, 1) if "k" in norm else None
    host, q, qi = _run(nb, rows, pos, slots, pages, hkv, hidx, qn, kn, 1e-6, rot, theta)
    oq, oqi, ok, ov, oki = I.transform(_bits(rows), pos, hkv, hidx,
                                       None if qn is None else qn.numpy(),
                                       None if kn is None else kn.numpy(), 1e-6, rot, theta)
    total, window = 0, 0
    for got, x in ((q, oq), (qi, oqi)):
        d = WINDOW * np.abs(x).max(axis=-1, keepdims=True)
        msg, n = A.check_e4m3_within(got, x, d)
        assert msg is None, msg
        total, window = total + got.size, window + n
    for (gc, gs), x in zip(host, (ok, ov, oki)):
        c = gc[slots // 128, :, slots % 128]
        s = gs[slots // 128, :, slots % 128]
        d = WINDOW * np.abs(x).max(axis=-1, keepdims=True)
        msg, n = A.check_nvfp4_within(c, s, x, d)
        assert msg is None, msg
        total, window = total + s.size, window + n
        # V is neither normalised nor rotated: exact
        if x is ov:
            assert n == 0
    say(f"  {window} of {total} bytes/groups needed the rounding window")
    assert window <= max(4, total // 500)


def test_insert_at_benchmark_shape_sampled(nb):
    """The benchmark's launch (16,384 tokens, 4 KV + 4 index heads, norm and
    RoPE at positions near 256K), checked on a sample of tokens."""
    hkv, hidx, t = 4, 4, 16384
    say("[insert bench shape] T=16384")
    width = (8 * hkv + 8 * hidx + 2 * hkv + hidx) * 128
    rows = synth.projection_rows(11, t, width, device="cuda")
    pos = np.tile(np.arange(262144 - 2048, 262144), 8)
    pages = t // 128
    slots = np.arange(t, dtype=np.int64)
    qn, kn = synth.norm_weights(5, 0), synth.norm_weights(5, 1)
    host, q, qi = _run(nb, rows, pos, slots, pages, hkv, hidx, qn, kn, 1e-6, 128, 1e4)
    sample = np.random.default_rng(0).choice(t, 48, replace=False)
    sample[:2] = [0, t - 1]
    oq, oqi, ok, ov, oki = I.transform(_bits(rows[sample].cpu()), pos[sample], hkv, hidx, qn.numpy(),
                                       kn.numpy(), 1e-6, 128, 1e4)
    for got, x in ((q[sample], oq), (qi[sample], oqi)):
        msg, _ = A.check_e4m3_within(got, x, WINDOW * np.abs(x).max(axis=-1, keepdims=True))
        assert msg is None, msg
    for (gc, gs), x in zip(host, (ok, ov, oki)):
        sl = slots[sample]
        msg, _ = A.check_nvfp4_within(gc[sl // 128, :, sl % 128], gs[sl // 128, :, sl % 128], x,
                                      WINDOW * np.abs(x).max(axis=-1, keepdims=True))
        assert msg is None, msg


def test_insert_empty_and_bad_shapes(nb):
    rows = torch.zeros((0, 76 * 128), dtype=torch.bfloat16, device="cuda")
    e = torch.zeros((0,), dtype=torch.int32, device="cuda")
    pools = _pools(nb, 1, 4, 4, 0)
    q = torch.zeros((0, 32, 128), dtype=torch.uint8, device="cuda")
    nb.msa_qkv_rope_insert(rows, e, e.long(), *pools, q, q.clone())   # no-op
    with pytest.raises(ValueError):
        nb.msa_qkv_rope_insert(torch.zeros((1, 75 * 128), dtype=torch.bfloat16, device="cuda"),
                               e[:1], e[:1].long(), *pools, q, q)
    with pytest.raises(nb.MsaError):
        bad = torch.zeros((1, 76 * 128), dtype=torch.bfloat16, device="cuda")
        one = torch.zeros((1,), dtype=torch.int32, device="cuda")
        qq = torch.zeros((1, 32, 128), dtype=torch.uint8, device="cuda")
        nb.msa_qkv_rope_insert(bad, one, one.long(), *pools, qq, qq.clone(), rotary_dim=48)
