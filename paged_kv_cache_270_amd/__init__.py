"""Python binding of libpkv (paged KV cache + decode PagedAttention for MI355X).

Argument marshalling only: every step of the hot path runs in the HIP kernels
of ``libpkv.so``; PyTorch supplies device memory and streams.  The function
names are those of the C ABI declared in ``include/pkv.h``.  If the library
has not been built the import of any entry point raises: there is no
fallback implementation.

Build with ``python -m paged_kv_cache_270_amd.build`` (or
``__graft_entry__.build()``).
"""
import ctypes
import os

__all__ = [
    "PKV_F16", "PKV_FP8_E4M3FN", "PKV_OK", "PkvError", "CacheLayout", "BlockPool", "lib_path",
    "load_library", "pkv_status_string", "pkv_bytes_per_token", "pkv_pool_bytes",
    "pkv_decode_partition_size", "pkv_decode_workspace_bytes", "pkv_reshape_and_cache",
    "pkv_paged_attention_decode", "pkv_decode_partitions", "pkv_decode_reduce",
    "pkv_paged_attention_decode_append", "pkv_decode_partitions_append",
    "pkv_copy_blocks", "pkv_reshape_dynamic_workspace_bytes", "pkv_reshape_and_cache_dynamic",
    "pkv_paged_attention_decode_dynamic", "pkv_copy_blocks_dynamic", "pkv_paged_prefill_attention",
    "pkv_paged_prefill_attention_dynamic", "pkv_swap_blocks", "pkv_validate_tables",
    "pkv_set_debug_checks", "pkv_get_debug_checks", "pkv_hbm_read_probe",
    "pkv_hbm_mix_probe", "pkv_tile_gather_probe", "pkv_paged_attention_decode_append_noalloc",
    "NOALLOC_SCRATCH_BYTES",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
# PKV_LIBRARY names another build of the library, e.g. the host half alone
# built with sanitizers for the CPU tests; functions it lacks then raise when
# called
_OVERRIDE = os.environ.get("PKV_LIBRARY", "")
lib_path = _OVERRIDE or os.path.join(_HERE, "libpkv.so")

PKV_OK = 0
PKV_ERR_INVALID_ARG = -1
PKV_ERR_UNSUPPORTED = -2
PKV_ERR_NO_FREE_BLOCKS = -3
PKV_ERR_HIP = -4
PKV_ERR_WORKSPACE = -5
PKV_ERR_BAD_HANDLE = -6
PKV_ERR_REFCOUNT = -7
PKV_F16 = 0
PKV_FP8_E4M3FN = 1
BLOCK_SIZE = 16
HEAD_DIM = 128
NOALLOC_SCRATCH_BYTES = 64 << 20   # PKV_NOALLOC_SCRATCH_BYTES


class CacheLayout(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]

    def __init__(self, num_blocks, num_kv_heads, dtype=PKV_F16, block_size=BLOCK_SIZE,
                 head_dim=HEAD_DIM):
        super().__init__(num_blocks, block_size, num_kv_heads, head_dim, dtype)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == PKV_F16 else 1


class PkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {pkv_status_string(status)} (status {status})")


_lib = None


def load_library():
    """Load libpkv.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise ImportError(f"libpkv.so not found at {lib_path}; build it with "
                          "`python -m paged_kv_cache_270_amd.build`")
    L = ctypes.CDLL(lib_path)
    P, i32, i64, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
    f32, f64 = ctypes.c_float, ctypes.c_double
    LP = ctypes.POINTER(CacheLayout)
    sig = {
        "pkv_status_string": ([i32], ctypes.c_char_p),
        "pkv_bytes_per_token": ([i32, i32, i32, i32], u64),
        "pkv_pool_bytes": ([LP], u64),
        "pkv_decode_partition_size": ([i32, i32, i32, i32, i32], i32),
        "pkv_decode_workspace_bytes": ([i32, i32, i32, i32, i32, i32], u64),
        "pkv_validate_tables": ([P, i32, P, i32, i32, i32, ctypes.POINTER(i32)], i32),
        "pkv_set_debug_checks": ([i32], i32),
        "pkv_hbm_read_probe": ([P, u64, i32, P, ctypes.c_uint32, P], i32),
        "pkv_hbm_mix_probe": ([P, P, u64, i32, i32, P], i32),
        "pkv_tile_gather_probe": ([P, P, P, i32, P, i32, i32, LP, P, ctypes.c_uint32, P], i32),
        "pkv_get_debug_checks": ([], i32),
        "pkv_reshape_and_cache": ([P, P, P, P, P, i32, LP, f32, f32, P], i32),
        "pkv_paged_attention_decode": ([P, P, P, P, P, i32, P, P, i32, i32, i32, LP, f32, f32,
                                        f32, i32, P, u64, P], i32),
        "pkv_decode_partitions": ([P, P, P, P, P, i32, P, P, i32, i32, i32, LP, f32, f32, f32,
                                   i32, P, u64, P], i32),
        "pkv_decode_reduce": ([P, P, i32, i32, i32, i32, LP, f32, i32, P, u64, P], i32),
        "pkv_paged_attention_decode_append": ([P, P, P, P, P, P, P, i32, P, P, i32, i32, i32,
                                               LP, f32, f32, f32, i32, P, u64, P], i32),
        "pkv_decode_partitions_append": ([P, P, P, P, P, P, P, i32, P, P, i32, i32, i32, LP,
                                          f32, f32, f32, i32, P, u64, P], i32),
        "pkv_paged_attention_decode_append_noalloc": ([P, P, P, P, P, P, P, i32, P, P, i32, i32,
                                                       i32, LP, f32, f32, f32, i32, P], i32),
        "pkv_paged_attention_decode_cascade": ([P, P, P, P, P, P, P, i32, P, P, P, P, i32, i32,
                                                i32, P, i32, P, i32, i32, i32, LP, f32, f32,
                                                f32, i32, P, u64, P], i32),
        "pkv_paged_attention_decode_cascade_dynamic": ([P, P, P, P, P, P, P, i32, P, P, P, P,
                                                        i32, i32, i32, P, i32, P, i32, i32,
                                                        i32, LP, f32, i32, P, u64, P], i32),
        "pkv_pool_cascade_tail_units": ([P, P, i32, P, i32, i32, ctypes.POINTER(i64)], i32),
        "pkv_pool_cascade_tail_map": ([P, P, i32, P, i32, i32, P, P, i64,
                                       ctypes.POINTER(i64)], i32),
        "pkv_decode_cascade_workspace_bytes": ([i32, i32, i32, i32, i32, i32, i32], u64),
        "pkv_pool_prefix_groups": ([P, P, i32, i32, i32, P, P, ctypes.POINTER(i32),
                                    ctypes.POINTER(i32), P], i32),
        "pkv_copy_blocks": ([P, P, LP, P, i32, P], i32),
        "pkv_reshape_dynamic_workspace_bytes": ([LP], u64),
        "pkv_reshape_and_cache_dynamic": ([P, P, P, P, P, P, P, i32, LP, P, u64, P], i32),
        "pkv_paged_attention_decode_dynamic": ([P, P, P, P, P, P, P, i32, P, P, i32, i32, i32,
                                                LP, f32, i32, P, u64, P], i32),
        "pkv_copy_blocks_dynamic": ([P, P, P, P, LP, P, i32, P], i32),
        "pkv_paged_prefill_attention": ([P, P, P, P, P, i32, P, P, i32, i32, i32, i32, LP, f32,
                                         f32, f32, P], i32),
        "pkv_paged_prefill_attention_dynamic": ([P, P, P, P, P, P, P, i32, P, P, i32, i32, i32,
                                                 i32, LP, f32, P], i32),
        "pkv_swap_blocks": ([P, P, P, P, i32, LP, P, i32, i32, P], i32),
        "pkv_pool_set_swap_space": ([P, i32], i32),
        "pkv_pool_num_free_host": ([P], i32),
        "pkv_seq_num_swapped": ([P, i32], i32),
        "pkv_seq_swap_out": ([P, i32, i32, i32, P], i32),
        "pkv_seq_swap_in": ([P, i32, P, i32, ctypes.POINTER(i32)], i32),
        "pkv_pool_create": ([i32, i32, u64, ctypes.POINTER(P)], i32),
        "pkv_pool_destroy": ([P], None),
        "pkv_pool_num_blocks": ([P], i32),
        "pkv_pool_num_free": ([P], i32),
        "pkv_pool_usage": ([P], f64),
        "pkv_pool_refcount": ([P, i32], i32),
        "pkv_pool_num_seqs": ([P], i32),
        "pkv_seq_create": ([P, ctypes.POINTER(i32)], i32),
        "pkv_seq_fork": ([P, i32, ctypes.POINTER(i32)], i32),
        "pkv_seq_append": ([P, i32, i32, P, P, ctypes.POINTER(i32)], i32),
        "pkv_seq_free": ([P, i32], i32),
        "pkv_seq_append_each": ([P, P, i32, P, P, ctypes.POINTER(i32), ctypes.POINTER(i32)],
                                i32),
        "pkv_seq_block_table": ([P, i32, P, i32, ctypes.POINTER(i32)], i32),
        "pkv_seq_len": ([P, i32], i64),
        "pkv_seq_shared_prefix_blocks": ([P, i32], i32),
        "pkv_seq_create_cached": ([P, P, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)], i32),
        "pkv_seq_cache_prefix": ([P, i32, P, i32], i32),
        "pkv_prefix_cache_stats": ([P, ctypes.POINTER(i64), ctypes.POINTER(i64),
                                    ctypes.POINTER(i32), ctypes.POINTER(i32)], i32),
        "pkv_prefix_cache_clear": ([P], None),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name, None)
        if fn is None and _OVERRIDE:
            continue
        if fn is None:
            raise ImportError(f"{lib_path} does not export {name}; rebuild it")
        fn.argtypes = args
        fn.restype = res
    _lib = L
    return L


def _check(status: int, where: str) -> None:
    if status != PKV_OK:
        raise PkvError(status, where)


def _ptr(x):
    """Device (or host) address of a tensor / int / None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_contiguous():
        raise ValueError("libpkv needs contiguous tensors")
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _require(t, dtype, name, device=True):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


# --------------------------------------------------------------- sizing

def pkv_status_string(status: int) -> str:
    return load_library().pkv_status_string(status).decode()


def pkv_bytes_per_token(n_layers: int, n_kv_heads: int, d_head: int, elem_bytes: int) -> int:
    return load_library().pkv_bytes_per_token(n_layers, n_kv_heads, d_head, elem_bytes)


def pkv_pool_bytes(layout: CacheLayout) -> int:
    return load_library().pkv_pool_bytes(ctypes.byref(layout))


def pkv_decode_partition_size(num_seqs, num_kv_heads, max_context_len, dtype=PKV_FP8_E4M3FN,
                              requested=0) -> int:
    return load_library().pkv_decode_partition_size(num_seqs, num_kv_heads, max_context_len,
                                                    dtype, requested)


def pkv_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, max_context_len,
                               dtype=PKV_FP8_E4M3FN, partition_size=0) -> int:
    return load_library().pkv_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads,
                                                     max_context_len, dtype, partition_size)


# --------------------------------------------------------- device calls

def pkv_validate_tables(block_tables, context_lens, max_context_len: int, num_blocks: int) -> int:
    """Host check of block tables and lengths (numpy int32 arrays): -1 if
    every length fits the table and every used entry names a pool block,
    else the first offending sequence.  Raises on bad sizes."""
    import numpy as np
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    if bt.ndim != 2 or lens.ndim != 1 or lens.shape[0] != bt.shape[0]:
        raise ValueError("block_tables [B][max_blocks] and context_lens [B] expected")
    bad = ctypes.c_int32(-1)
    st = load_library().pkv_validate_tables(bt.ctypes.data, bt.shape[1], lens.ctypes.data,
                                            lens.shape[0], max_context_len, num_blocks,
                                            ctypes.byref(bad))
    if st != PKV_OK and bad.value < 0:
        _check(st, "pkv_validate_tables")
    return bad.value


def pkv_set_debug_checks(on: bool) -> bool:
    """Turn the debug table checks of the device calls on or off; returns the
    previous setting."""
    return bool(load_library().pkv_set_debug_checks(1 if on else 0))


def pkv_get_debug_checks() -> bool:
    return bool(load_library().pkv_get_debug_checks())


_PROBE_KEY = 0x9E3779B9   # stored only if the folded data equals it


def pkv_hbm_read_probe(buf, sink, workgroups: int = 0, stream=None) -> None:
    """Stream the bytes of device tensor `buf` once (the streaming-read
    ceiling), each workgroup its own contiguous slab; `sink` is a device
    int32/uint32 tensor of at least one word."""
    _check(load_library().pkv_hbm_read_probe(_ptr(buf), buf.numel() * buf.element_size(),
                                             workgroups, _ptr(sink), _PROBE_KEY,
                                             _stream(stream)), "pkv_hbm_read_probe")


def pkv_hbm_mix_probe(src, dst, reads_per_write: int, workgroups: int = 0,
                      stream=None) -> None:
    """Stream `reads_per_write` planes of `dst`'s size from device tensor `src`
    into `dst` (their XOR), non-temporal both ways: the ceiling for a write
    with that mix of reads and writes."""
    nbytes = dst.numel() * dst.element_size()
    if src.numel() * src.element_size() < reads_per_write * nbytes:
        raise ValueError("pkv_hbm_mix_probe: src holds fewer than reads_per_write planes")
    _check(load_library().pkv_hbm_mix_probe(_ptr(src), _ptr(dst), nbytes, reads_per_write,
                                            workgroups, _stream(stream)), "pkv_hbm_mix_probe")


def pkv_tile_gather_probe(k_pool, v_pool, block_tables, context_lens, max_context_len: int,
                          layout: CacheLayout, sink, stream=None) -> None:
    """Read every K and V tile the decode of this batch reads, through the
    block table, without arithmetic (the gather ceiling)."""
    _check(load_library().pkv_tile_gather_probe(
        _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), block_tables.shape[1],
        _ptr(context_lens), context_lens.shape[0], max_context_len, ctypes.byref(layout),
        _ptr(sink), _PROBE_KEY, _stream(stream)), "pkv_tile_gather_probe")


def pkv_reshape_and_cache(key, value, k_pool, v_pool, slot_mapping, layout: CacheLayout,
                          k_scale: float = 1.0, v_scale: float = 1.0, stream=None) -> None:
    """key/value: fp16 [T][Hkv][128]; slot_mapping: int64 [T] (device)."""
    import torch
    _require(key, torch.float16, "key")
    _require(value, torch.float16, "value")
    _require(slot_mapping, torch.int64, "slot_mapping")
    T = key.shape[0]
    if key.shape != value.shape or tuple(key.shape[1:]) != (layout.num_kv_heads, layout.head_dim):
        raise ValueError("key/value must be [T][num_kv_heads][head_dim]")
    if slot_mapping.numel() != T:
        raise ValueError("slot_mapping must hold one slot per token")
    _check(load_library().pkv_reshape_and_cache(
        _ptr(key), _ptr(value), _ptr(k_pool), _ptr(v_pool), _ptr(slot_mapping), T,
        ctypes.byref(layout), k_scale, v_scale, _stream(stream)), "pkv_reshape_and_cache")


def _decode_args(out, q, block_tables, context_lens):
    import torch
    _require(out, torch.float32, "out")
    _require(q, torch.float16, "q")
    _require(block_tables, torch.int32, "block_tables")
    _require(context_lens, torch.int32, "context_lens")
    B, Hq, D = q.shape
    if tuple(out.shape) != (B, Hq, D):
        raise ValueError("out must match q's shape")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.numel() != B:
        raise ValueError("block_tables must be [B][max_blocks], context_lens [B]")
    return B, Hq, block_tables.shape[1]


def _workspace(workspace, B, Hq, layout, max_context_len, partition_size):
    need = pkv_decode_workspace_bytes(B, Hq, layout.num_kv_heads, max_context_len,
                                      layout.dtype, partition_size)
    if workspace is None and need > 0:
        import torch
        workspace = torch.empty(need, dtype=torch.uint8, device="cuda")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return workspace, nbytes


def _hint(shared_prefix_blocks, B):
    if shared_prefix_blocks is None:
        return None
    import torch
    _require(shared_prefix_blocks, torch.int32, "shared_prefix_blocks")
    if shared_prefix_blocks.numel() != B:
        raise ValueError("shared_prefix_blocks must hold one count per sequence")
    return _ptr(shared_prefix_blocks)


def pkv_paged_attention_decode(out, q, k_pool, v_pool, block_tables, context_lens,
                               max_context_len: int, layout: CacheLayout, sm_scale: float,
                               k_scale: float = 1.0, v_scale: float = 1.0,
                               partition_size: int = 0, workspace=None, stream=None,
                               shared_prefix_blocks=None) -> None:
    B, Hq, mb = _decode_args(out, q, block_tables, context_lens)
    workspace, nbytes = _workspace(workspace, B, Hq, layout, max_context_len, partition_size)
    _check(load_library().pkv_paged_attention_decode(
        _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), mb,
        _ptr(context_lens), _hint(shared_prefix_blocks, B), B, Hq, max_context_len,
        ctypes.byref(layout), sm_scale, k_scale, v_scale, partition_size, _ptr(workspace),
        nbytes, _stream(stream)), "pkv_paged_attention_decode")


def pkv_decode_partitions(out, q, k_pool, v_pool, block_tables, context_lens,
                          max_context_len: int, layout: CacheLayout, sm_scale: float,
                          k_scale: float = 1.0, v_scale: float = 1.0, partition_size: int = 0,
                          workspace=None, stream=None, shared_prefix_blocks=None) -> None:
    B, Hq, mb = _decode_args(out, q, block_tables, context_lens)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().pkv_decode_partitions(
        _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), mb,
        _ptr(context_lens), _hint(shared_prefix_blocks, B), B, Hq, max_context_len,
        ctypes.byref(layout), sm_scale, k_scale, v_scale, partition_size, _ptr(workspace),
        nbytes, _stream(stream)), "pkv_decode_partitions")


def pkv_decode_reduce(out, context_lens, max_context_len: int, max_blocks_per_seq: int,
                      layout: CacheLayout, v_scale: float = 1.0, partition_size: int = 0,
                      workspace=None, stream=None) -> None:
    B, Hq = out.shape[0], out.shape[1]
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().pkv_decode_reduce(
        _ptr(out), _ptr(context_lens), B, Hq, max_context_len, max_blocks_per_seq,
        ctypes.byref(layout), v_scale, partition_size, _ptr(workspace), nbytes,
        _stream(stream)), "pkv_decode_reduce")


def _new_rows(key, value, B, layout):
    import torch
    _require(key, torch.float16, "key")
    _require(value, torch.float16, "value")
    if key.shape != value.shape or tuple(key.shape) != (B, layout.num_kv_heads, layout.head_dim):
        raise ValueError("key/value must be [num_seqs][num_kv_heads][head_dim]")
    return _ptr(key), _ptr(value)


def pkv_paged_attention_decode_append(out, q, key, value, k_pool, v_pool, block_tables,
                                      context_lens, max_context_len: int, layout: CacheLayout,
                                      sm_scale: float, k_scale: float = 1.0,
                                      v_scale: float = 1.0, partition_size: int = 0,
                                      workspace=None, stream=None,
                                      shared_prefix_blocks=None) -> None:
    """One decode step: store each sequence's newest token (key/value fp16
    [B][Hkv][128], at position context_lens[b] - 1) and attend over all."""
    B, Hq, mb = _decode_args(out, q, block_tables, context_lens)
    kp, vp = _new_rows(key, value, B, layout)
    workspace, nbytes = _workspace(workspace, B, Hq, layout, max_context_len, partition_size)
    _check(load_library().pkv_paged_attention_decode_append(
        _ptr(out), _ptr(q), kp, vp, _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), mb,
        _ptr(context_lens), _hint(shared_prefix_blocks, B), B, Hq, max_context_len,
        ctypes.byref(layout), sm_scale, k_scale, v_scale, partition_size, _ptr(workspace),
        nbytes, _stream(stream)), "pkv_paged_attention_decode_append")


def pkv_decode_partitions_append(out, q, key, value, k_pool, v_pool, block_tables,
                                 context_lens, max_context_len: int, layout: CacheLayout,
                                 sm_scale: float, k_scale: float = 1.0, v_scale: float = 1.0,
                                 partition_size: int = 0, workspace=None, stream=None,
                                 shared_prefix_blocks=None) -> None:
    B, Hq, mb = _decode_args(out, q, block_tables, context_lens)
    kp, vp = _new_rows(key, value, B, layout)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().pkv_decode_partitions_append(
        _ptr(out), _ptr(q), kp, vp, _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), mb,
        _ptr(context_lens), _hint(shared_prefix_blocks, B), B, Hq, max_context_len,
        ctypes.byref(layout), sm_scale, k_scale, v_scale, partition_size, _ptr(workspace),
        nbytes, _stream(stream)), "pkv_decode_partitions_append")


def pkv_paged_attention_decode_append_noalloc(out, q, key, value, k_pool, v_pool, block_tables,
                                              context_lens, max_context_len: int,
                                              layout: CacheLayout, sm_scale: float,
                                              k_scale: float = 1.0, v_scale: float = 1.0,
                                              partition_size: int = 0, stream=None,
                                              shared_prefix_blocks=None) -> None:
    """pkv_paged_attention_decode_append with its split-KV partials in the
    library's own fixed array (NOALLOC_SCRATCH_BYTES per device): no
    workspace argument and no allocation.  Calls overlapping in time on one
    device race."""
    B, Hq, mb = _decode_args(out, q, block_tables, context_lens)
    kp, vp = _new_rows(key, value, B, layout)
    _check(load_library().pkv_paged_attention_decode_append_noalloc(
        _ptr(out), _ptr(q), kp, vp, _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), mb,
        _ptr(context_lens), _hint(shared_prefix_blocks, B), B, Hq, max_context_len,
        ctypes.byref(layout), sm_scale, k_scale, v_scale, partition_size, _stream(stream)),
        "pkv_paged_attention_decode_append_noalloc")


def pkv_decode_cascade_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, max_context_len,
                                       max_prefix_blocks, dtype=PKV_FP8_E4M3FN,
                                       partition_size=0) -> int:
    return load_library().pkv_decode_cascade_workspace_bytes(
        num_seqs, num_q_heads, num_kv_heads, max_context_len, max_prefix_blocks, dtype,
        partition_size)


def pkv_paged_attention_decode_cascade(out, q, key, value, k_pool, v_pool, block_tables,
                                       context_lens, max_context_len: int, layout: CacheLayout,
                                       sm_scale: float, prefix_blocks, prefix_groups,
                                       max_prefix_blocks: int, k_scale: float = 1.0,
                                       v_scale: float = 1.0, partition_size: int = 0,
                                       workspace=None, stream=None,
                                       shared_prefix_blocks=None, seq_order=None,
                                       tail_units: int = 0, tail_map=None) -> None:
    """Decode with each group's shared prefix attended once for the group.
    prefix_blocks: device int32 [B]; prefix_groups: device int32
    [n_groups][group_cap] (or None for no groups); key/value: the newest
    tokens' rows to write in the same launch, or both None; seq_order:
    optional device int32 [B], the order the tails are scheduled in;
    tail_units: the batch's tail work (BlockPool.cascade_tail_units), 0 =
    unknown; tail_map: optional device int32 [tail_units][2]
    (BlockPool.cascade_tail_map)."""
    import torch
    B, Hq, mb = _decode_args(out, q, block_tables, context_lens)
    if key is None and value is None:
        kp = vp = None
    else:
        kp, vp = _new_rows(key, value, B, layout)
    n_groups, cap, gp, pp = _cascade_groups(prefix_blocks, prefix_groups, B)
    _check_order(seq_order, tail_map, tail_units, B)
    need = pkv_decode_cascade_workspace_bytes(B, Hq, layout.num_kv_heads, max_context_len,
                                              max_prefix_blocks if n_groups else 0,
                                              layout.dtype, partition_size)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device="cuda")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().pkv_paged_attention_decode_cascade(
        _ptr(out), _ptr(q), kp, vp, _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), mb,
        _ptr(context_lens), _hint(shared_prefix_blocks, B), pp, gp, n_groups, cap,
        max_prefix_blocks, _ptr(seq_order), tail_units, _ptr(tail_map), B, Hq, max_context_len,
        ctypes.byref(layout), sm_scale, k_scale, v_scale, partition_size, _ptr(workspace), nbytes,
        _stream(stream)), "pkv_paged_attention_decode_cascade")


def _check_order(seq_order, tail_map, tail_units, B):
    import torch
    if seq_order is not None:
        _require(seq_order, torch.int32, "seq_order")
        if seq_order.numel() != B:
            raise ValueError("seq_order must hold one entry per sequence")
    if tail_map is not None:
        _require(tail_map, torch.int32, "tail_map")
        if tail_map.numel() != 2 * tail_units:
            raise ValueError("tail_map must hold tail_units (batch index, partition) pairs")


def _cascade_groups(prefix_blocks, prefix_groups, B):
    import torch
    if prefix_groups is None or prefix_groups.numel() == 0:
        return 0, 1, None, None
    _require(prefix_groups, torch.int32, "prefix_groups")
    _require(prefix_blocks, torch.int32, "prefix_blocks")
    if prefix_groups.dim() != 2 or prefix_blocks.numel() != B:
        raise ValueError("prefix_groups must be [n_groups][group_cap], prefix_blocks [B]")
    n_groups, cap = prefix_groups.shape
    return n_groups, cap, _ptr(prefix_groups), _ptr(prefix_blocks)


def pkv_paged_attention_decode_cascade_dynamic(out, q, k_pool, v_pool, k_block_scales,
                                               v_block_scales, block_tables, context_lens,
                                               max_context_len: int, layout: CacheLayout,
                                               sm_scale: float, prefix_blocks, prefix_groups,
                                               max_prefix_blocks: int, partition_size: int = 0,
                                               workspace=None, stream=None,
                                               shared_prefix_blocks=None,
                                               seq_order=None, tail_units: int = 0,
                                               tail_map=None) -> None:
    """The cascade decode over per-(block, KV head) scales (fp32
    [num_blocks][Hkv] device tensors); decode only."""
    import torch
    B, Hq, mb = _decode_args(out, q, block_tables, context_lens)
    _require(k_block_scales, torch.float32, "k_block_scales")
    _require(v_block_scales, torch.float32, "v_block_scales")
    n_groups, cap, gp, pp = _cascade_groups(prefix_blocks, prefix_groups, B)
    _check_order(seq_order, tail_map, tail_units, B)
    need = pkv_decode_cascade_workspace_bytes(B, Hq, layout.num_kv_heads, max_context_len,
                                              max_prefix_blocks if n_groups else 0,
                                              layout.dtype, partition_size)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device="cuda")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().pkv_paged_attention_decode_cascade_dynamic(
        _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_block_scales),
        _ptr(v_block_scales), _ptr(block_tables), mb, _ptr(context_lens),
        _hint(shared_prefix_blocks, B), pp, gp, n_groups, cap, max_prefix_blocks,
        _ptr(seq_order), tail_units, _ptr(tail_map), B, Hq, max_context_len,
        ctypes.byref(layout), sm_scale, partition_size, _ptr(workspace), nbytes,
        _stream(stream)),
        "pkv_paged_attention_decode_cascade_dynamic")


def pkv_copy_blocks(k_pool, v_pool, layout: CacheLayout, src_dst_pairs, stream=None) -> None:
    """src_dst_pairs: int32 [n][2] device tensor of (source, destination)."""
    import torch
    _require(src_dst_pairs, torch.int32, "src_dst_pairs")
    n = src_dst_pairs.shape[0] if src_dst_pairs.dim() == 2 else src_dst_pairs.numel() // 2
    _check(load_library().pkv_copy_blocks(_ptr(k_pool), _ptr(v_pool), ctypes.byref(layout),
                                          _ptr(src_dst_pairs), n, _stream(stream)),
           "pkv_copy_blocks")


# ------------------------------------------------------------------ swap

def pkv_swap_blocks(k_pool, v_pool, host_k, host_v, num_host_blocks: int, layout: CacheLayout,
                    pairs, to_host: bool, stream=None) -> None:
    """Copy blocks between the device pools and pinned host buffers."""
    import torch
    _require(pairs, torch.int32, "pairs")
    for t, name in ((host_k, "host_k"), (host_v, "host_v")):
        if t.is_cuda or not t.is_pinned():
            raise ValueError(f"{name} must be pinned host memory")
    _check(load_library().pkv_swap_blocks(
        _ptr(k_pool), _ptr(v_pool), _ptr(host_k), _ptr(host_v), num_host_blocks,
        ctypes.byref(layout), _ptr(pairs), pairs.numel() // 2, int(bool(to_host)),
        _stream(stream)), "pkv_swap_blocks")


# ------------------------------------------------------ chunked prefill

def _prefill_args(out, q, block_tables, context_lens, query_start):
    import torch
    _require(out, torch.float32, "out")
    _require(q, torch.float16, "q")
    _require(block_tables, torch.int32, "block_tables")
    _require(context_lens, torch.int32, "context_lens")
    _require(query_start, torch.int32, "query_start")
    B = context_lens.numel()
    if tuple(out.shape) != tuple(q.shape) or q.dim() != 3:
        raise ValueError("q and out must be [rows][num_q_heads][head_dim]")
    if query_start.numel() != B + 1 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("query_start must be [B + 1], block_tables [B][max_blocks]")
    return B


def pkv_paged_prefill_attention(out, q, k_pool, v_pool, block_tables, context_lens, query_start,
                                max_query_len: int, max_context_len: int, layout: CacheLayout,
                                sm_scale: float, k_scale: float = 1.0, v_scale: float = 1.0,
                                stream=None) -> None:
    """Causal attention of each sequence's last chunk of tokens (rows
    query_start[b] .. query_start[b+1]-1 of q) over the paged cache."""
    B = _prefill_args(out, q, block_tables, context_lens, query_start)
    _check(load_library().pkv_paged_prefill_attention(
        _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), _ptr(query_start), B, q.shape[1],
        max_query_len, max_context_len, ctypes.byref(layout), sm_scale, k_scale, v_scale,
        _stream(stream)), "pkv_paged_prefill_attention")


# ------------------------------------------- per-block dynamic FP8 scales

def pkv_reshape_dynamic_workspace_bytes(layout: CacheLayout) -> int:
    return load_library().pkv_reshape_dynamic_workspace_bytes(ctypes.byref(layout))


def _block_scales(k_block_scales, v_block_scales, layout):
    import torch
    for t, name in ((k_block_scales, "k_block_scales"), (v_block_scales, "v_block_scales")):
        _require(t, torch.float32, name)
        if t.numel() != layout.num_blocks * layout.num_kv_heads:
            raise ValueError(f"{name} must be [num_blocks][num_kv_heads]")


def pkv_reshape_and_cache_dynamic(key, value, k_pool, v_pool, k_block_scales, v_block_scales,
                                  slot_mapping, layout: CacheLayout, workspace=None,
                                  stream=None) -> None:
    """FP8 write with per-(block, KV head) scales, updated in place."""
    import torch
    _require(key, torch.float16, "key")
    _require(value, torch.float16, "value")
    _require(slot_mapping, torch.int64, "slot_mapping")
    _block_scales(k_block_scales, v_block_scales, layout)
    T = key.shape[0]
    if key.shape != value.shape or tuple(key.shape[1:]) != (layout.num_kv_heads, layout.head_dim):
        raise ValueError("key/value must be [T][num_kv_heads][head_dim]")
    if slot_mapping.numel() != T:
        raise ValueError("slot_mapping must hold one slot per token")
    if workspace is None:
        need = pkv_reshape_dynamic_workspace_bytes(layout)
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().pkv_reshape_and_cache_dynamic(
        _ptr(key), _ptr(value), _ptr(k_pool), _ptr(v_pool), _ptr(k_block_scales),
        _ptr(v_block_scales), _ptr(slot_mapping), T, ctypes.byref(layout), _ptr(workspace),
        nbytes, _stream(stream)), "pkv_reshape_and_cache_dynamic")


def pkv_paged_attention_decode_dynamic(out, q, k_pool, v_pool, k_block_scales, v_block_scales,
                                       block_tables, context_lens, max_context_len: int,
                                       layout: CacheLayout, sm_scale: float,
                                       partition_size: int = 0, workspace=None, stream=None,
                                       shared_prefix_blocks=None) -> None:
    B, Hq, mb = _decode_args(out, q, block_tables, context_lens)
    _block_scales(k_block_scales, v_block_scales, layout)
    workspace, nbytes = _workspace(workspace, B, Hq, layout, max_context_len, partition_size)
    _check(load_library().pkv_paged_attention_decode_dynamic(
        _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_block_scales),
        _ptr(v_block_scales), _ptr(block_tables), mb, _ptr(context_lens),
        _hint(shared_prefix_blocks, B), B, Hq, max_context_len, ctypes.byref(layout), sm_scale,
        partition_size, _ptr(workspace), nbytes, _stream(stream)),
        "pkv_paged_attention_decode_dynamic")


def pkv_paged_prefill_attention_dynamic(out, q, k_pool, v_pool, k_block_scales, v_block_scales,
                                        block_tables, context_lens, query_start,
                                        max_query_len: int, max_context_len: int,
                                        layout: CacheLayout, sm_scale: float,
                                        stream=None) -> None:
    """Chunked prefill over an FP8 pool with per-(block, head) scales."""
    B = _prefill_args(out, q, block_tables, context_lens, query_start)
    _block_scales(k_block_scales, v_block_scales, layout)
    _check(load_library().pkv_paged_prefill_attention_dynamic(
        _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_block_scales),
        _ptr(v_block_scales), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        _ptr(query_start), B, q.shape[1], max_query_len, max_context_len, ctypes.byref(layout),
        sm_scale, _stream(stream)), "pkv_paged_prefill_attention_dynamic")


def pkv_copy_blocks_dynamic(k_pool, v_pool, k_block_scales, v_block_scales, layout: CacheLayout,
                            src_dst_pairs, stream=None) -> None:
    import torch
    _require(src_dst_pairs, torch.int32, "src_dst_pairs")
    _block_scales(k_block_scales, v_block_scales, layout)
    n = src_dst_pairs.numel() // 2
    _check(load_library().pkv_copy_blocks_dynamic(
        _ptr(k_pool), _ptr(v_pool), _ptr(k_block_scales), _ptr(v_block_scales),
        ctypes.byref(layout), _ptr(src_dst_pairs), n, _stream(stream)),
        "pkv_copy_blocks_dynamic")


# ---------------------------------------------------------- block pool

class BlockPool:
    """Host block pool and sequence tables (pkv_pool_* / pkv_seq_*)."""

    def __init__(self, num_blocks: int, block_size: int = BLOCK_SIZE, shuffle_seed: int = 0):
        self._L = load_library()
        h = ctypes.c_void_p()
        _check(self._L.pkv_pool_create(num_blocks, block_size, shuffle_seed, ctypes.byref(h)),
               "pkv_pool_create")
        self._h = h

    def close(self):
        if self._h:
            self._L.pkv_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def num_blocks(self) -> int:
        return self._L.pkv_pool_num_blocks(self._h)

    def num_free(self) -> int:
        return self._L.pkv_pool_num_free(self._h)

    def usage(self) -> float:
        return self._L.pkv_pool_usage(self._h)

    def refcount(self, block: int) -> int:
        return self._L.pkv_pool_refcount(self._h, block)

    def num_seqs(self) -> int:
        return self._L.pkv_pool_num_seqs(self._h)

    def create(self) -> int:
        out = ctypes.c_int32()
        _check(self._L.pkv_seq_create(self._h, ctypes.byref(out)), "pkv_seq_create")
        return out.value

    def fork(self, parent: int) -> int:
        out = ctypes.c_int32()
        _check(self._L.pkv_seq_fork(self._h, parent, ctypes.byref(out)), "pkv_seq_fork")
        return out.value

    def append(self, seq: int, n_tokens: int):
        """Returns (slots: list[int], cow_pairs: list[(old, new)])."""
        slots = (ctypes.c_int64 * max(1, n_tokens))()
        pairs = (ctypes.c_int32 * 2)()
        n_cow = ctypes.c_int32()
        _check(self._L.pkv_seq_append(self._h, seq, n_tokens, slots, pairs, ctypes.byref(n_cow)),
               "pkv_seq_append")
        cow = [(pairs[0], pairs[1])] if n_cow.value else []
        return list(slots[:n_tokens]), cow

    def append_each(self, seqs):
        """One token for each sequence of `seqs`, in order.  Returns (slots
        int64 [n], cow_pairs list of (old, new)); raises on the first failing
        sequence (those before it are appended)."""
        import numpy as np
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        n = seqs.size
        slots = np.zeros(max(1, n), dtype=np.int64)
        pairs = np.zeros((max(1, n), 2), dtype=np.int32)
        n_cow, n_done = ctypes.c_int32(), ctypes.c_int32()
        _check(self._L.pkv_seq_append_each(self._h, seqs.ctypes.data, n, slots.ctypes.data,
                                           pairs.ctypes.data, ctypes.byref(n_cow),
                                           ctypes.byref(n_done)), "pkv_seq_append_each")
        return slots[:n].copy(), [tuple(int(x) for x in r) for r in pairs[:n_cow.value]]

    def free(self, seq: int) -> None:
        _check(self._L.pkv_seq_free(self._h, seq), "pkv_seq_free")

    def block_table(self, seq: int):
        n = ctypes.c_int32()
        st = self._L.pkv_seq_block_table(self._h, seq, None, 0, ctypes.byref(n))
        if st not in (PKV_OK, PKV_ERR_INVALID_ARG):
            _check(st, "pkv_seq_block_table")
        buf = (ctypes.c_int32 * max(1, n.value))()
        _check(self._L.pkv_seq_block_table(self._h, seq, buf, n.value, ctypes.byref(n)),
               "pkv_seq_block_table")
        return list(buf[:n.value])

    def seq_len(self, seq: int) -> int:
        return self._L.pkv_seq_len(self._h, seq)

    def shared_prefix_blocks(self, seq: int) -> int:
        return self._L.pkv_seq_shared_prefix_blocks(self._h, seq)

    def prefix_groups(self, seqs, group_cap: int = 8, with_order: bool = False):
        """Prefix groups of a batch for the cascade decode.  Returns
        (prefix_blocks int32 [n], groups int32 [n_groups][group_cap] with -1
        padding, max_prefix_blocks) as numpy arrays and an int, plus the batch
        order by decreasing tail (int32 [n]) if with_order."""
        import numpy as np
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        n = seqs.size
        prefix = np.zeros(max(1, n), dtype=np.int32)
        cap_groups = max(1, n)
        groups = np.full((cap_groups, group_cap), -1, dtype=np.int32)
        order = np.zeros(max(1, n), dtype=np.int32)
        ng, mx = ctypes.c_int32(), ctypes.c_int32()
        _check(self._L.pkv_pool_prefix_groups(
            self._h, seqs.ctypes.data, n, group_cap, cap_groups, prefix.ctypes.data,
            groups.ctypes.data, ctypes.byref(ng), ctypes.byref(mx), order.ctypes.data),
            "pkv_pool_prefix_groups")
        res = (prefix[:n].copy(), groups[:ng.value].copy(), mx.value)
        return res + (order[:n].copy(),) if with_order else res

    def cascade_tail_units(self, seqs, prefix_blocks, max_prefix_blocks: int,
                           partition_size: int) -> int:
        """The tail_units argument of the cascade decode for this batch and
        the prefix_groups result (prefix_blocks, max_prefix_blocks)."""
        import numpy as np
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        pre = np.ascontiguousarray(prefix_blocks, dtype=np.int32)
        if pre.size != seqs.size:
            raise ValueError("one prefix length per sequence")
        out = ctypes.c_int64()
        _check(self._L.pkv_pool_cascade_tail_units(self._h, seqs.ctypes.data, seqs.size,
                                                   pre.ctypes.data, max_prefix_blocks,
                                                   partition_size, ctypes.byref(out)),
               "pkv_pool_cascade_tail_units")
        return out.value

    def cascade_tail_map(self, seqs, prefix_blocks, max_prefix_blocks: int,
                         partition_size: int, order=None):
        """The tail_map argument of the cascade decode: an int32 array
        [units][2] of (batch index, tail partition) in the decode's schedule
        order (order: the seq_order it gets, or None for batch order)."""
        import numpy as np
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        pre = np.ascontiguousarray(prefix_blocks, dtype=np.int32)
        if pre.size != seqs.size:
            raise ValueError("one prefix length per sequence")
        if order is not None:
            order = np.ascontiguousarray(order, dtype=np.int32)
            if order.size != seqs.size:
                raise ValueError("order must hold one entry per sequence")
        cap = self.cascade_tail_units(seqs, pre, max_prefix_blocks, partition_size)
        out = np.zeros((max(cap, 1), 2), dtype=np.int32)
        units = ctypes.c_int64()
        _check(self._L.pkv_pool_cascade_tail_map(
            self._h, seqs.ctypes.data, seqs.size, pre.ctypes.data, max_prefix_blocks,
            partition_size, None if order is None else order.ctypes.data, out.ctypes.data,
            cap, ctypes.byref(units)), "pkv_pool_cascade_tail_map")
        return out[:units.value].copy()

    # ---- swap space (page-granular eviction to host memory)

    def set_swap_space(self, num_host_blocks: int) -> None:
        _check(self._L.pkv_pool_set_swap_space(self._h, num_host_blocks),
               "pkv_pool_set_swap_space")

    def num_free_host(self) -> int:
        return self._L.pkv_pool_num_free_host(self._h)

    def num_swapped(self, seq: int) -> int:
        return self._L.pkv_seq_num_swapped(self._h, seq)

    def swap_out(self, seq: int, first_block: int, n_blocks: int):
        """Returns [(device block, host slot)] in logical order."""
        buf = (ctypes.c_int32 * max(2, 2 * n_blocks))()
        _check(self._L.pkv_seq_swap_out(self._h, seq, first_block, n_blocks, buf),
               "pkv_seq_swap_out")
        return [(buf[2 * i], buf[2 * i + 1]) for i in range(n_blocks)]

    def swap_in(self, seq: int):
        """Returns [(host slot, device block)] in logical order."""
        n = ctypes.c_int32()
        st = self._L.pkv_seq_swap_in(self._h, seq, None, 0, ctypes.byref(n))
        if st not in (PKV_OK, PKV_ERR_INVALID_ARG):
            _check(st, "pkv_seq_swap_in")
        if n.value == 0:
            return []
        buf = (ctypes.c_int32 * (2 * n.value))()
        _check(self._L.pkv_seq_swap_in(self._h, seq, buf, n.value, ctypes.byref(n)),
               "pkv_seq_swap_in")
        return [(buf[2 * i], buf[2 * i + 1]) for i in range(n.value)]

    def create_cached(self, tokens):
        """New sequence whose leading cached chunks of `tokens` are mapped onto
        the cached blocks; returns (seq, n_cached_tokens)."""
        toks = _i32_array(tokens)
        seq, n_cached = ctypes.c_int32(), ctypes.c_int32()
        _check(self._L.pkv_seq_create_cached(self._h, toks, len(tokens), ctypes.byref(seq),
                                             ctypes.byref(n_cached)), "pkv_seq_create_cached")
        return seq.value, n_cached.value

    def cache_prefix(self, seq: int, tokens) -> None:
        """Register the filled full blocks of `seq`, whose token ids are `tokens`."""
        _check(self._L.pkv_seq_cache_prefix(self._h, seq, _i32_array(tokens), len(tokens)),
               "pkv_seq_cache_prefix")

    def prefix_cache_stats(self) -> dict:
        hit, miss = ctypes.c_int64(), ctypes.c_int64()
        cached, evictable = ctypes.c_int32(), ctypes.c_int32()
        _check(self._L.pkv_prefix_cache_stats(self._h, ctypes.byref(hit), ctypes.byref(miss),
                                              ctypes.byref(cached), ctypes.byref(evictable)),
               "pkv_prefix_cache_stats")
        return {"hit_blocks": hit.value, "miss_blocks": miss.value,
                "cached_blocks": cached.value, "evictable_blocks": evictable.value}

    def clear_prefix_cache(self) -> None:
        self._L.pkv_prefix_cache_clear(self._h)


def _i32_array(values):
    vals = [int(v) for v in values]
    return (ctypes.c_int32 * max(1, len(vals)))(*vals)

