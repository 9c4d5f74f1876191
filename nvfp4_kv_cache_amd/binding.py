"""ctypes binding of libmsa_nvfp4.so (include/msa_nvfp4.h).

Argument marshalling only: shapes and dtypes are checked, device pointers and
torch's current HIP stream are passed through, and a non-OK status raises
MsaError. Every step of the computation runs in the library's HIP kernels;
there is no fallback of any kind. If the library is not built, loading it
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmsa_nvfp4.so")

MSA_OK = 0
HEAD_DIM = 128
BLOCK_TOKENS = 128
TOPK = 16

_lib = None


class MsaError(RuntimeError):
    pass


class PoolDesc(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_tokens", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("num_pages", ctypes.c_int64)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F32 = ctypes.c_float
_DESC = ctypes.POINTER(PoolDesc)

SIGNATURES = {
    "msa_status_string": (ctypes.c_char_p, [_I32]),
    "msa_nvfp4_quantize": (ctypes.c_int, [_DESC, _P, _P, _I64, _P, _P, _P]),
    "msa_indexer_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
    "msa_indexer_decode": (ctypes.c_int, [_DESC, _P, _P, _P, _P, _I32, _P, _I32, _P, _I32, _I32,
                                          _I32, _P, _P, _P, _SZ, _P]),
    "msa_indexer_decode_noalloc": (ctypes.c_int, [_DESC, _P, _P, _P, _P, _I32, _P, _I32, _P, _I32,
                                                  _I32, _I32, _P, _P, _P]),
    "msa_indexer_scan": (ctypes.c_int, [_DESC, _P, _P, _P, _P, _I32, _P, _I32, _P, _I32, _I32,
                                        _P, _P]),
    "msa_indexer_scan_shared": (ctypes.c_int, [_DESC, _P, _P, _P, _P, _I32, _P, _I32, _P, _I32,
                                               _I32, _I32, _P, _P, _I32, _P, _P, _P]),
    "msa_shared_prefix_groups": (ctypes.c_int, [_P, _I32, _P, _I32, _I32, _P, _P, _P, _P, _P]),
    "msa_indexer_select": (ctypes.c_int, [_P, _P, _I32, _I32, _I32, _I32, _P, _P, _P]),
    "msa_attn_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
    "msa_sparse_attn_decode": (ctypes.c_int, [_DESC, _P, _P, _P, _P, _P, _I32, _P, _I32, _P,
                                              _I32, _I32, _P, _I32, _F32, _P, _P, _SZ, _P]),
    "msa_sparse_attn_select_decode": (ctypes.c_int, [_DESC, _P, _P, _P, _P, _P, _I32, _P, _I32,
                                                     _P, _I32, _I32, _P, _I32, _P, _F32, _P, _P,
                                                     _SZ, _P]),
    "msa_decode_mono_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
    "msa_decode_mono": (ctypes.c_int, [_DESC, _P, _P, _P, _P, _DESC, _P, _P, _P, _P, _P, _I32, _P,
                                       _I32, _P, _I32, _I32, _I32, _P, _F32, _P, _P, _SZ, _P]),
    "msa_read_probe": (ctypes.c_int, [_P, _I64, _I64, _P, _P]),
    "msa_stream_probe": (ctypes.c_int, [_P, _I64, _P, _I64, _I64, _P]),
    "msa_qkv_rope_insert": (ctypes.c_int, [_P, _I64, _P, _P, _DESC, _P, _P, _P, _P, _DESC, _P, _P,
                                           _P, _P, _F32, _I32, _F32, _P, _P, _P]),
}


def lib() -> ctypes.CDLL:
    """Load libmsa_nvfp4.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MsaError(f"{LIB_PATH} is not built: run `python -m nvfp4_kv_cache_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def msa_status_string(status: int) -> str:
    return lib().msa_status_string(status).decode()


def _check(status: int, what: str):
    if status != MSA_OK:
        raise MsaError(f"{what}: {msa_status_string(status)}")


class Prepared:
    """One library call with its arguments validated and marshalled once
    (device pointers, sizes, the stream that was current): calling it issues
    the same launch again, for loops that re-run a step on unchanged buffers.
    The tensors it was prepared from must stay alive and keep their shapes."""

    def __init__(self, name: str, args: tuple, keep: tuple):
        self._fn = getattr(lib(), name)
        self._args = args
        self._keep = keep
        self.name = name

    def __call__(self) -> None:
        status = self._fn(*self._args)
        if status != MSA_OK:
            raise MsaError(f"{self.name}: {msa_status_string(status)}")


def _issue(name: str, args: tuple, prepare: bool, keep: tuple = ()):
    """Call the library now, or (prepare=True) return the call as a Prepared."""
    if prepare:
        return Prepared(name, args, keep)
    _check(getattr(lib(), name)(*args), name)
    return None


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype, ndim=None, device=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if device and t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def pool_desc(codes: torch.Tensor) -> PoolDesc:
    """Pool shape from a codes tensor uint8 [num_pages, num_heads, 128, 64]."""
    if codes.dim() != 4 or codes.shape[2] != BLOCK_TOKENS or codes.shape[3] != HEAD_DIM // 2:
        raise ValueError(f"codes must be [pages, heads, 128, 64], got {tuple(codes.shape)}")
    return PoolDesc(codes.shape[1], HEAD_DIM, BLOCK_TOKENS, 0, codes.shape[0])


SCALE_PAGE = BLOCK_TOKENS * HEAD_DIM // 16   # 1 KiB of scales per (page, head)


def _check_pool(codes, scales, name):
    _need(codes, f"{name}_codes", torch.uint8, 4)
    _need(scales, f"{name}_scales", torch.uint8, 3)
    if tuple(scales.shape) != tuple(codes.shape[:2]) + (SCALE_PAGE,):
        raise ValueError(f"{name}_scales shape {tuple(scales.shape)} does not match codes")


def empty_pool(num_pages: int, num_heads: int, device="cuda"):
    """Uninitialised (codes, scales) pool tensors in the library's layout:
    codes [pages, heads, 128, 64], scales [pages, heads, 1024] (tile-major)."""
    codes = torch.empty((num_pages, num_heads, BLOCK_TOKENS, HEAD_DIM // 2), dtype=torch.uint8,
                        device=device)
    scales = torch.empty((num_pages, num_heads, SCALE_PAGE), dtype=torch.uint8, device=device)
    return codes, scales


def scales_rows(scales: torch.Tensor) -> torch.Tensor:
    """Row-major view [pages, heads, 128 rows, 8 groups] of tile-major scales.

    Byte ((g/2)*16 + r%16)*16 + (r/16)*2 + g%2 of a (page, head) holds the
    scale of row r, group g (include/msa_nvfp4.h)."""
    p, h = scales.shape[:2]
    x = scales.reshape(p, h, 4, 16, 8, 2)          # [slice c][row i][tile j][e]
    return x.permute(0, 1, 4, 3, 2, 5).reshape(p, h, BLOCK_TOKENS, HEAD_DIM // 16)


def msa_nvfp4_quantize(src, slot_mapping, codes, scales, prepare=False):
    """Quantise src float32 [T, H, 128] into the pool at slot_mapping int64 [T]."""
    _check_pool(codes, scales, "pool")
    _need(src, "src", torch.float32, 3)
    _need(slot_mapping, "slot_mapping", torch.int64, 1)
    desc = pool_desc(codes)
    if src.shape[1] != desc.num_heads or src.shape[2] != HEAD_DIM:
        raise ValueError(f"src must be [T, {desc.num_heads}, 128], got {tuple(src.shape)}")
    if slot_mapping.shape[0] != src.shape[0]:
        raise ValueError("slot_mapping length must equal the number of tokens")
    return _issue("msa_nvfp4_quantize", (
        ctypes.byref(desc), _ptr(src), _ptr(slot_mapping), src.shape[0], _ptr(codes),
        _ptr(scales), _stream()), prepare, keep=(desc,))


def msa_qkv_rope_insert(qkv, positions, slot_mapping, k_pool, v_pool, idx_pool, q_fp8, q_idx_fp8,
                        q_norm_w=None, k_norm_w=None, rms_eps=1e-6, rotary_dim=128,
                        rope_theta=10000.0, prepare=False):
    """The cache-insertion path after the QKV projection, in one launch.

    qkv bfloat16 [T, (8 Hkv + 8 Hidx + 2 Hkv + Hidx) * 128] (heads q, q_idx,
    k, v, k_idx), positions int32 [T], slot_mapping int64 [T]; pools are
    (codes, scales) pairs (K and V with Hkv heads, the index keys with Hidx);
    q_fp8 uint8 [T, 8 Hkv, 128] and q_idx_fp8 uint8 [T, 8 Hidx, 128] receive
    the FP8 queries. q_norm_w / k_norm_w float32 [128] or None (no RMSNorm)."""
    for (c, sc), nm in ((k_pool, "k"), (v_pool, "v"), (idx_pool, "idx")):
        _check_pool(c, sc, nm)
    _need(qkv, "qkv", torch.bfloat16, 2)
    _need(positions, "positions", torch.int32, 1)
    _need(slot_mapping, "slot_mapping", torch.int64, 1)
    _need(q_fp8, "q_fp8", torch.uint8, 3)
    _need(q_idx_fp8, "q_idx_fp8", torch.uint8, 3)
    kv, idx = pool_desc(k_pool[0]), pool_desc(idx_pool[0])
    if tuple(v_pool[0].shape) != tuple(k_pool[0].shape):
        raise ValueError("the K and V pools must have the same shape")
    hkv, hidx, t = kv.num_heads, idx.num_heads, qkv.shape[0]
    width = (8 * hkv + 8 * hidx + 2 * hkv + hidx) * HEAD_DIM
    if qkv.shape[1] != width:
        raise ValueError(f"qkv rows must hold {width} channels, got {qkv.shape[1]}")
    if positions.shape[0] != t or slot_mapping.shape[0] != t:
        raise ValueError("positions and slot_mapping need one entry per token")
    if tuple(q_fp8.shape) != (t, 8 * hkv, HEAD_DIM) or tuple(q_idx_fp8.shape) != (t, 8 * hidx, HEAD_DIM):
        raise ValueError("q_fp8 / q_idx_fp8 shapes do not match the pools' head counts")
    for w, nm in ((q_norm_w, "q_norm_w"), (k_norm_w, "k_norm_w")):
        if w is not None:
            _need(w, nm, torch.float32, 1)
            if w.shape[0] != HEAD_DIM:
                raise ValueError(f"{nm} must have {HEAD_DIM} entries")
    return _issue("msa_qkv_rope_insert", (
        _ptr(qkv), t, _ptr(positions), _ptr(slot_mapping), ctypes.byref(kv), _ptr(k_pool[0]),
        _ptr(k_pool[1]), _ptr(v_pool[0]), _ptr(v_pool[1]), ctypes.byref(idx), _ptr(idx_pool[0]),
        _ptr(idx_pool[1]), _ptr(q_norm_w), _ptr(k_norm_w), float(rms_eps), int(rotary_dim),
        float(rope_theta), _ptr(q_fp8), _ptr(q_idx_fp8), _stream()), prepare, keep=(kv, idx))


def msa_indexer_workspace_bytes(num_seqs: int, q_per_seq: int, max_blocks: int) -> int:
    return int(lib().msa_indexer_workspace_bytes(num_seqs, q_per_seq, max_blocks))


def msa_attn_workspace_bytes(num_seqs: int, q_per_seq: int, num_q_heads: int, num_sel: int) -> int:
    return int(lib().msa_attn_workspace_bytes(num_seqs, q_per_seq, num_q_heads, num_sel))


def attn_workspace(num_seqs, q_per_seq, num_q_heads, num_sel, device="cuda"):
    """Workspace for msa_sparse_attn_decode / msa_sparse_attn_select_decode,
    zero-filled once (its split-arrival counters start at zero, and every
    call leaves them zero)."""
    n = msa_attn_workspace_bytes(num_seqs, q_per_seq, num_q_heads, num_sel)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


def indexer_workspace(num_seqs, q_per_seq, max_blocks, device="cuda"):
    """Workspace for msa_indexer_decode (contents need no initialisation)."""
    n = msa_indexer_workspace_bytes(num_seqs, q_per_seq, max_blocks)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def msa_indexer_decode(idx_codes, idx_scales, q_fp8, head_w, block_table, seq_lens, q_per_seq,
                       out_ids, workspace, out_scores=None, topk=TOPK, prepare=False):
    """Top-16 + recent block ids per query token into out_ids int32 [B*Q, 17]."""
    _check_pool(idx_codes, idx_scales, "idx")
    _need(q_fp8, "q_fp8", torch.uint8, 3)
    _need(head_w, "head_w", torch.float32, 2)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    _need(out_ids, "out_ids", torch.int32, 2)
    _need(workspace, "workspace", torch.uint8, 1)
    if out_scores is not None:
        _need(out_scores, "out_scores", torch.float32, 2)
    num_seqs, max_blocks = block_table.shape
    tq = num_seqs * q_per_seq
    hq = q_fp8.shape[1]
    if seq_lens.shape[0] != num_seqs or q_fp8.shape != (tq, hq, HEAD_DIM):
        raise ValueError("q_fp8 must be [num_seqs*q_per_seq, Hq, 128] and seq_lens [num_seqs]")
    if head_w.shape != (tq, hq) or out_ids.shape != (tq, topk + 1):
        raise ValueError("head_w must be [T_q, Hq] and out_ids [T_q, topk+1]")
    if out_scores is not None and out_scores.shape != out_ids.shape:
        raise ValueError("out_scores must match out_ids")
    desc = pool_desc(idx_codes)
    return _issue("msa_indexer_decode", (
        ctypes.byref(desc), _ptr(idx_codes), _ptr(idx_scales), _ptr(q_fp8), _ptr(head_w), hq,
        _ptr(block_table), max_blocks, _ptr(seq_lens), num_seqs, q_per_seq, topk, _ptr(out_ids),
        _ptr(out_scores), _ptr(workspace), workspace.numel(), _stream()), prepare, keep=(desc,))


NOALLOC_MAX_SCORES = 1 << 20   # MSA_NOALLOC_MAX_SCORES


def msa_indexer_decode_noalloc(idx_codes, idx_scales, q_fp8, head_w, block_table, seq_lens,
                               q_per_seq, out_ids, out_scores=None, topk=TOPK, prepare=False):
    """msa_indexer_decode without a workspace: the block scores live in the
    library's own device array (at most NOALLOC_MAX_SCORES = T_q x max_blocks
    entries); calls on one GPU share it and must not overlap."""
    _check_pool(idx_codes, idx_scales, "idx")
    num_seqs, max_blocks, tq, hq = _check_indexer_inputs(q_fp8, head_w, block_table, seq_lens,
                                                         q_per_seq)
    _need(out_ids, "out_ids", torch.int32, 2)
    if out_ids.shape != (tq, topk + 1):
        raise ValueError("out_ids must be [T_q, topk+1]")
    if out_scores is not None:
        _need(out_scores, "out_scores", torch.float32, 2)
        if out_scores.shape != out_ids.shape:
            raise ValueError("out_scores must match out_ids")
    desc = pool_desc(idx_codes)
    return _issue("msa_indexer_decode_noalloc", (
        ctypes.byref(desc), _ptr(idx_codes), _ptr(idx_scales), _ptr(q_fp8), _ptr(head_w), hq,
        _ptr(block_table), max_blocks, _ptr(seq_lens), num_seqs, q_per_seq, topk, _ptr(out_ids),
        _ptr(out_scores), _stream()), prepare, keep=(desc,))


def _check_indexer_inputs(q_fp8, head_w, block_table, seq_lens, q_per_seq):
    _need(q_fp8, "q_fp8", torch.uint8, 3)
    _need(head_w, "head_w", torch.float32, 2)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    num_seqs, max_blocks = block_table.shape
    tq = num_seqs * q_per_seq
    hq = q_fp8.shape[1]
    if seq_lens.shape[0] != num_seqs or q_fp8.shape != (tq, hq, HEAD_DIM):
        raise ValueError("q_fp8 must be [num_seqs*q_per_seq, Hq, 128] and seq_lens [num_seqs]")
    if head_w.shape != (tq, hq):
        raise ValueError("head_w must be [T_q, Hq]")
    return num_seqs, max_blocks, tq, hq


def msa_indexer_scan(idx_codes, idx_scales, q_fp8, head_w, block_table, seq_lens, q_per_seq,
                     block_scores, prepare=False):
    """Block scores B(j) into block_scores float32 [B*Q, max_blocks]."""
    _check_pool(idx_codes, idx_scales, "idx")
    num_seqs, max_blocks, tq, hq = _check_indexer_inputs(q_fp8, head_w, block_table, seq_lens,
                                                         q_per_seq)
    _need(block_scores, "block_scores", torch.float32, 2)
    if block_scores.shape != (tq, max_blocks):
        raise ValueError("block_scores must be [T_q, max_blocks]")
    desc = pool_desc(idx_codes)
    return _issue("msa_indexer_scan", (
        ctypes.byref(desc), _ptr(idx_codes), _ptr(idx_scales), _ptr(q_fp8), _ptr(head_w), hq,
        _ptr(block_table), max_blocks, _ptr(seq_lens), num_seqs, q_per_seq, _ptr(block_scores),
        _stream()), prepare, keep=(desc,))


def msa_shared_prefix_groups(block_table, seq_lens, q_per_seq, device=None):
    """Shared-prefix groups of a batch, derived by the library on the host
    from a host copy of the block table int32 [B, max_blocks] and seq_lens
    int32 [B] (torch CPU tensors). Returns (group_lead, group_blocks,
    max_group_blocks, seq_group): int32 tensors (on `device` when given) and
    a host int, msa_indexer_scan_shared's group arguments."""
    for t, name in ((block_table, "block_table"), (seq_lens, "seq_lens")):
        _need(t, name, torch.int32, device=False)
        if t.device.type != "cpu":
            raise ValueError(f"{name} must be a host (CPU) tensor")
    if block_table.dim() != 2 or seq_lens.dim() != 1 or seq_lens.shape[0] != block_table.shape[0]:
        raise ValueError("block_table must be [B, max_blocks] and seq_lens [B]")
    num_seqs, max_blocks = block_table.shape
    n = max(num_seqs, 1)
    lead = torch.empty(n, dtype=torch.int32)
    blocks = torch.empty(n, dtype=torch.int32)
    group = torch.empty(n, dtype=torch.int32)
    ng, mgb = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib().msa_shared_prefix_groups(
        _ptr(block_table), max_blocks, _ptr(seq_lens), num_seqs, int(q_per_seq), _ptr(lead),
        _ptr(blocks), _ptr(group), ctypes.byref(ng), ctypes.byref(mgb)), "msa_shared_prefix_groups")
    out = (lead[:ng.value].clone(), blocks[:ng.value].clone(), group[:num_seqs].clone())
    if device is not None:
        out = tuple(t.to(device) for t in out)
    return out[0], out[1], int(mgb.value), out[2]


def msa_indexer_scan_shared(idx_codes, idx_scales, q_fp8, head_w, block_table, seq_lens, q_per_seq,
                            group_lead, group_blocks, max_group_blocks, seq_group, block_scores,
                            prepare=False):
    """msa_indexer_scan with the blocks of shared prefixes read and
    dequantised once per group, in the same launch: group_lead int32 [G],
    group_blocks int32 [G], seq_group int32 [B] (device; from
    msa_shared_prefix_groups), max_group_blocks >= every group_blocks entry
    (host int)."""
    _check_pool(idx_codes, idx_scales, "idx")
    num_seqs, max_blocks, tq, hq = _check_indexer_inputs(q_fp8, head_w, block_table, seq_lens,
                                                         q_per_seq)
    _need(block_scores, "block_scores", torch.float32, 2)
    if block_scores.shape != (tq, max_blocks):
        raise ValueError("block_scores must be [T_q, max_blocks]")
    for t, name in ((group_lead, "group_lead"), (group_blocks, "group_blocks"),
                    (seq_group, "seq_group")):
        _need(t, name, torch.int32, 1)
    num_groups = group_lead.shape[0]
    if group_blocks.shape[0] != num_groups:
        raise ValueError("group_lead and group_blocks must both be [G]")
    if seq_group.shape[0] != num_seqs:
        raise ValueError("seq_group must be [num_seqs]")
    desc = pool_desc(idx_codes)
    return _issue("msa_indexer_scan_shared", (
        ctypes.byref(desc), _ptr(idx_codes), _ptr(idx_scales), _ptr(q_fp8), _ptr(head_w), hq,
        _ptr(block_table), max_blocks, _ptr(seq_lens), num_seqs, q_per_seq, num_groups,
        _ptr(group_lead), _ptr(group_blocks), int(max_group_blocks), _ptr(seq_group),
        _ptr(block_scores), _stream()), prepare, keep=(desc,))


def msa_indexer_select(block_scores, seq_lens, q_per_seq, out_ids, out_scores=None, topk=TOPK,
                       prepare=False):
    """Top-16 + recent block ids from block scores float32 [B*Q, max_blocks]."""
    _need(block_scores, "block_scores", torch.float32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    _need(out_ids, "out_ids", torch.int32, 2)
    if out_scores is not None:
        _need(out_scores, "out_scores", torch.float32, 2)
    tq, max_blocks = block_scores.shape
    num_seqs = seq_lens.shape[0]
    if tq != num_seqs * q_per_seq or out_ids.shape != (tq, topk + 1):
        raise ValueError("block_scores must be [num_seqs*q_per_seq, max_blocks], out_ids [T_q, 17]")
    if out_scores is not None and out_scores.shape != out_ids.shape:
        raise ValueError("out_scores must match out_ids")
    return _issue("msa_indexer_select", (
        _ptr(block_scores), _ptr(seq_lens), max_blocks, num_seqs, q_per_seq, topk, _ptr(out_ids),
        _ptr(out_scores), _stream()), prepare)


def _check_attn_inputs(k_codes, k_scales, v_codes, v_scales, q_fp8, block_table, seq_lens,
                       q_per_seq, out, workspace):
    _check_pool(k_codes, k_scales, "k")
    _check_pool(v_codes, v_scales, "v")
    if k_codes.shape != v_codes.shape:
        raise ValueError("K and V pools must have the same shape")
    _need(q_fp8, "q_fp8", torch.uint8, 3)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    _need(out, "out", torch.float32, 3)
    _need(workspace, "workspace", torch.uint8, 1)
    num_seqs, max_blocks = block_table.shape
    tq = num_seqs * q_per_seq
    hq = q_fp8.shape[1]
    if q_fp8.shape != (tq, hq, HEAD_DIM) or out.shape != (tq, hq, HEAD_DIM):
        raise ValueError("q_fp8 and out must be [num_seqs*q_per_seq, Hq, 128]")
    if seq_lens.shape[0] != num_seqs:
        raise ValueError("seq_lens must be [num_seqs]")
    return num_seqs, max_blocks, tq, hq


def msa_sparse_attn_decode(k_codes, k_scales, v_codes, v_scales, q_fp8, block_table, seq_lens,
                           q_per_seq, sel_ids, softmax_scale, out, workspace, prepare=False):
    """Attention over the selected blocks into out float32 [B*Q, Hq, 128]."""
    num_seqs, max_blocks, tq, hq = _check_attn_inputs(k_codes, k_scales, v_codes, v_scales, q_fp8,
                                                      block_table, seq_lens, q_per_seq, out,
                                                      workspace)
    _need(sel_ids, "sel_ids", torch.int32, 2)
    if sel_ids.shape[0] != tq:
        raise ValueError("sel_ids must be [T_q, num_sel]")
    desc = pool_desc(k_codes)
    return _issue("msa_sparse_attn_decode", (
        ctypes.byref(desc), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes), _ptr(v_scales),
        _ptr(q_fp8), hq, _ptr(block_table), max_blocks, _ptr(seq_lens), num_seqs, q_per_seq,
        _ptr(sel_ids), sel_ids.shape[1], float(softmax_scale), _ptr(out), _ptr(workspace),
        workspace.numel(), _stream()), prepare, keep=(desc,))


def msa_sparse_attn_select_decode(k_codes, k_scales, v_codes, v_scales, q_fp8, block_table,
                                  seq_lens, q_per_seq, block_scores, softmax_scale, out, workspace,
                                  out_ids=None, topk=TOPK, prepare=False):
    """Selection from block scores [B*Q, max_blocks] and attention in one launch; the selected
    ids go to out_ids int32 [B*Q, 17] when given."""
    num_seqs, max_blocks, tq, hq = _check_attn_inputs(k_codes, k_scales, v_codes, v_scales, q_fp8,
                                                      block_table, seq_lens, q_per_seq, out,
                                                      workspace)
    _need(block_scores, "block_scores", torch.float32, 2)
    if block_scores.shape != (tq, max_blocks):
        raise ValueError("block_scores must be [T_q, max_blocks]")
    if out_ids is not None:
        _need(out_ids, "out_ids", torch.int32, 2)
        if out_ids.shape != (tq, topk + 1):
            raise ValueError("out_ids must be [T_q, topk + 1]")
    desc = pool_desc(k_codes)
    return _issue("msa_sparse_attn_select_decode", (
        ctypes.byref(desc), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes), _ptr(v_scales),
        _ptr(q_fp8), hq, _ptr(block_table), max_blocks, _ptr(seq_lens), num_seqs, q_per_seq,
        _ptr(block_scores), topk, _ptr(out_ids), float(softmax_scale), _ptr(out),
        _ptr(workspace), workspace.numel(), _stream()), prepare, keep=(desc,))


def msa_decode_mono_workspace_bytes(num_seqs: int, q_per_seq: int, num_q_heads: int,
                                    max_blocks: int) -> int:
    return int(lib().msa_decode_mono_workspace_bytes(num_seqs, q_per_seq, num_q_heads, max_blocks))


def mono_workspace(num_seqs, q_per_seq, num_q_heads, max_blocks, device="cuda"):
    """Workspace for msa_decode_mono, zero-filled (its counters must start at
    zero; a call whose waits all end in time leaves them zero)."""
    n = msa_decode_mono_workspace_bytes(num_seqs, q_per_seq, num_q_heads, max_blocks)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


def mono_check(workspace, num_seqs, q_per_seq, num_q_heads, max_blocks):
    """Read the error word msa_decode_mono leaves in the last 32 bits of its
    workspace (waits for the stream). If a bounded wait of an earlier call
    timed out (error word 1), the counters may hold stale arrivals: the whole
    counter region, error word included, is zeroed and MsaError is raised."""
    n = msa_decode_mono_workspace_bytes(num_seqs, q_per_seq, num_q_heads, max_blocks)
    err = int(workspace[n - 4:n].view(torch.int32).item())
    if err == 0:
        return
    # counters: (num_seqs + pairs) arrival counts of 8 x 16 words, num_seqs
    # reader counters of 16 words, the error word; 256-byte aligned at the end
    pairs = num_seqs * q_per_seq * (num_q_heads // 8)
    words = (num_seqs + pairs) * 128 + num_seqs * 16 + 1
    region = -(-words * 4 // 256) * 256
    torch.cuda.current_stream().synchronize()
    workspace[n - region:n].zero_()
    torch.cuda.current_stream().synchronize()
    raise MsaError("msa_decode_mono: a bounded wait timed out (the output of the affected query "
                   "tokens is zero and their ids -1); the workspace counters were reset")


class MonoPrepared(Prepared):
    """A prepared msa_decode_mono call; check() reads its error word."""

    def __init__(self, args, keep, shape):
        super().__init__("msa_decode_mono", args, keep)
        self._shape = shape

    def check(self):
        mono_check(*self._shape)


def mono_block_scores(workspace, num_seqs, q_per_seq, max_blocks):
    """The block scores [T_q, max_blocks] a msa_decode_mono call left at the
    start of its workspace (a view)."""
    tq = num_seqs * q_per_seq
    return workspace[: tq * max_blocks * 4].view(torch.float32).view(tq, max_blocks)


def msa_decode_mono(idx_codes, idx_scales, q_idx_fp8, head_w, k_codes, k_scales, v_codes,
                    v_scales, q_fp8, block_table, seq_lens, q_per_seq, softmax_scale, out,
                    workspace, out_ids=None, topk=TOPK, prepare=False, check=True):
    """The whole decode step (index scan, selection, sparse attention) in one
    launch: out float32 [B*Q, Hq, 128], ids into out_ids int32 [B*Q, 17] when
    given; workspace from mono_workspace().

    check=True (direct calls): wait for the stream and read the launch's
    error word (mono_check): a timed-out wait raises MsaError after the
    workspace counters are reset. prepare=True returns a MonoPrepared, whose
    check() does the same when the caller chooses to synchronise."""
    _check_pool(idx_codes, idx_scales, "idx")
    num_seqs, max_blocks, tq, hq = _check_attn_inputs(k_codes, k_scales, v_codes, v_scales, q_fp8,
                                                      block_table, seq_lens, q_per_seq, out,
                                                      workspace)
    _need(q_idx_fp8, "q_idx_fp8", torch.uint8, 3)
    _need(head_w, "head_w", torch.float32, 2)
    if q_idx_fp8.shape != q_fp8.shape or head_w.shape != (tq, hq):
        raise ValueError("q_idx_fp8 must match q_fp8 and head_w be [T_q, Hq]")
    if out_ids is not None:
        _need(out_ids, "out_ids", torch.int32, 2)
        if out_ids.shape != (tq, topk + 1):
            raise ValueError("out_ids must be [T_q, topk + 1]")
    idesc, kdesc = pool_desc(idx_codes), pool_desc(k_codes)
    args = (ctypes.byref(idesc), _ptr(idx_codes), _ptr(idx_scales), _ptr(q_idx_fp8), _ptr(head_w),
            ctypes.byref(kdesc), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes), _ptr(v_scales),
            _ptr(q_fp8), hq, _ptr(block_table), max_blocks, _ptr(seq_lens), num_seqs, q_per_seq,
            topk, _ptr(out_ids), float(softmax_scale), _ptr(out), _ptr(workspace),
            workspace.numel(), _stream())
    shape = (workspace, num_seqs, q_per_seq, hq, max_blocks)
    if prepare:
        return MonoPrepared(args, (idesc, kdesc), shape)
    _issue("msa_decode_mono", args, False)
    if check:
        mono_check(*shape)
    return None


def msa_read_probe(buf, chunk_bytes, sink, prepare=False):
    """Plain streaming read of the device tensor buf (its bytes, a multiple
    of 16) in chunks of chunk_bytes per workgroup; sink int32 with at least
    ceil(bytes / chunk_bytes) entries."""
    if not isinstance(buf, torch.Tensor) or buf.device.type != "cuda" or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    _need(sink, "sink", torch.int32, 1)
    n = buf.numel() * buf.element_size()
    if sink.numel() < -(-n // chunk_bytes):
        raise ValueError("sink needs one entry per chunk")
    return _issue("msa_read_probe", (_ptr(buf), n, int(chunk_bytes), _ptr(sink), _stream()),
                  prepare)


def msa_stream_probe(src, dst, chunk_bytes, prepare=False):
    """Plain streaming read of all of src and write of all of dst (contiguous
    GPU tensors, byte sizes multiples of 16) at once, src in chunks of
    chunk_bytes per workgroup and dst split evenly over the workgroups."""
    for t, nm in ((src, "src"), (dst, "dst")):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError(f"{nm} must be a contiguous GPU tensor")
    return _issue("msa_stream_probe", (
        _ptr(src), src.numel() * src.element_size(), _ptr(dst), dst.numel() * dst.element_size(),
        int(chunk_bytes), _stream()), prepare)
