"""CPU oracle for the paged KV cache hot path — TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does, and
this package never imports the product: the two share no code.

The arithmetic lives in ``pkv_oracle.c`` (fp64 C, built by ``oracle/build.py``);
this module only marshals numpy arrays, plus two plain-Python models that
need no arithmetic beyond counting:

* :func:`bytes_per_token` — the KV sizing formula of "Optimización de KV Cache
  con PagedAttention y Cuantización FP8 para Contextos Largos (128K)", §2.
* :class:`BlockPoolModel` — reference counts, free list, fork, copy-on-write
  and free-on-cancel of the block pool described in "LLM Primer VI, Capítulo 8
  — Gestión de caché KV", §8.1, "KV Cache y PagedAttention: por qué se reduce
  la velocidad de tu servidor LLM" (on-demand pages, copy-on-write) and
  "PagedAttention y Gestión de KV-Cache" §3.01, §4.02.

Every function is pinned by ``tests/test_oracle_*.py`` against something other
than itself (library routines, closed forms, the pages' worked numbers).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# PKV_ORACLE_LIBRARY names another build of pkv_oracle.c (the sanitizer
# build of the CPU tests)
_LIB_PATH = os.environ.get("PKV_ORACLE_LIBRARY") or os.path.join(_HERE, "libpkv_oracle.so")
_lib = None

BLOCK_SIZE = 16


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, f32, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double
    lib.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_double.restype = f64
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_decode.restype = f64
    lib.oracle_e4m3_encode.argtypes = [f32]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_e4m3_encode_array.argtypes = [P, i64, P]
    lib.oracle_e4m3_encode_array.restype = None
    lib.oracle_quotient.argtypes = [f64, f32]
    lib.oracle_quotient.restype = f32
    lib.oracle_quantize_f16.argtypes = [P, i64, f32, P]
    lib.oracle_quantize_f16.restype = None
    lib.oracle_k_offset.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.oracle_k_offset.restype = i64
    lib.oracle_v_offset.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.oracle_v_offset.restype = i64
    lib.oracle_slot.argtypes = [P, i64]
    lib.oracle_slot.restype = i64
    lib.oracle_reshape_and_cache.argtypes = [P, P, P, P, P, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_int, f32, f32]
    lib.oracle_reshape_and_cache.restype = None
    lib.oracle_paged_attention_decode.argtypes = [P, P, P, P, P, ctypes.c_int, P] + \
        [ctypes.c_int] * 5 + [f32, f32, f32, ctypes.c_int]
    lib.oracle_paged_attention_decode.restype = None
    lib.oracle_reshape_and_cache_dynamic.argtypes = [P] * 7 + [ctypes.c_int] * 4
    lib.oracle_reshape_and_cache_dynamic.restype = None
    lib.oracle_paged_attention_decode_dynamic.argtypes = [P] * 7 + [ctypes.c_int, P] + \
        [ctypes.c_int] * 4 + [f32, ctypes.c_int]
    lib.oracle_paged_attention_decode_dynamic.restype = None
    lib.oracle_paged_prefill_attention.argtypes = [P] * 5 + [ctypes.c_int, P, P] + \
        [ctypes.c_int] * 5 + [f32, f32, f32, ctypes.c_int]
    lib.oracle_paged_prefill_attention.restype = None
    lib.oracle_paged_prefill_attention_dynamic.argtypes = [P] * 7 + [ctypes.c_int, P, P] + \
        [ctypes.c_int] * 4 + [f32, ctypes.c_int]
    lib.oracle_paged_prefill_attention_dynamic.restype = None
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _swap_library(path: str):
    """Load the oracle from another build of pkv_oracle.c (used by the tests
    that plant mistakes in copies of the oracle to show its pins catch them);
    returns the previously loaded library so it can be restored."""
    global _lib
    prev = _load()
    _lib = None
    global _LIB_PATH
    saved, _LIB_PATH = _LIB_PATH, path
    try:
        _load()
    finally:
        _LIB_PATH = saved
    return prev


def _restore_library(lib) -> None:
    global _lib
    _lib = lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _f16_bits(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    assert a.dtype == np.uint16, a.dtype
    return a


# ------------------------------------------------------------------- numbers

def f16_to_double(bits: int) -> float:
    return _load().oracle_f16_to_double(int(bits))


def e4m3_decode(code: int) -> float:
    return _load().oracle_e4m3_decode(int(code))


def e4m3_decode_table() -> np.ndarray:
    """Value of each of the 256 E4M3FN codes (NaN for 0x7F and 0xFF)."""
    lib = _load()
    return np.array([lib.oracle_e4m3_decode(c) for c in range(256)], dtype=np.float64)


def e4m3_encode(u) -> np.ndarray:
    """Brute-force nearest E4M3FN code of each fp32 value (ties to even,
    saturating at +-448, NaN -> 0x7F|sign)."""
    u = np.asarray(u, dtype=np.float32)
    shape = u.shape
    u = np.ascontiguousarray(u.reshape(-1))
    out = np.empty(u.shape, dtype=np.uint8)
    _load().oracle_e4m3_encode_array(_ptr(u), u.size, _ptr(out))
    return out.reshape(shape)


def quotient(x: float, scale: float) -> np.float32:
    """Correctly rounded fp32 value of x / scale."""
    return np.float32(_load().oracle_quotient(float(x), float(np.float32(scale))))


def quantize_f16(x, scale: float) -> np.ndarray:
    """E4M3(x / scale) for an array of fp16 values."""
    bits = _f16_bits(x)
    out = np.empty(bits.shape, dtype=np.uint8)
    _load().oracle_quantize_f16(_ptr(bits), bits.size, float(np.float32(scale)), _ptr(out))
    return out


# -------------------------------------------------------------------- layout

def k_offset(t: int, d: int, elem_bytes: int) -> int:
    return _load().oracle_k_offset(t, d, elem_bytes)


def v_offset(t: int, d: int, elem_bytes: int) -> int:
    return _load().oracle_v_offset(t, d, elem_bytes)


def slot(table_row, pos: int) -> int:
    row = np.ascontiguousarray(np.asarray(table_row, dtype=np.int32))
    return _load().oracle_slot(_ptr(row), int(pos))


def slots_for(block_tables, seq_ids, positions) -> np.ndarray:
    """Slot of (sequence, logical position) pairs through their block tables."""
    bt = np.ascontiguousarray(np.asarray(block_tables, dtype=np.int32))
    return np.array([slot(bt[s], p) for s, p in zip(seq_ids, positions)], dtype=np.int64)


def bytes_per_token(n_layers: int, n_kv_heads: int, d_head: int, elem_bytes: int) -> int:
    """KV bytes one token occupies: 2 (K and V) x layers x KV heads x head dim
    x bytes per element ("Optimización de KV Cache con PagedAttention y
    Cuantización FP8 ...", §2)."""
    return 2 * n_layers * n_kv_heads * d_head * elem_bytes


# ---------------------------------------------------------------- hot path

def reshape_and_cache(key, value, k_pool: np.ndarray, v_pool: np.ndarray, slots,
                      num_kv_heads: int, fp8: bool, k_scale: float = 1.0,
                      v_scale: float = 1.0) -> None:
    """Write [T][Hkv][D] fp16 rows into the byte pools (in place)."""
    kb, vb = _f16_bits(key), _f16_bits(value)
    T = kb.shape[0] if kb.ndim else 0
    D = kb.shape[-1]
    assert kb.shape == vb.shape and kb.shape[1] == num_kv_heads
    sl = np.ascontiguousarray(np.asarray(slots, dtype=np.int64))
    assert sl.shape == (T,)
    assert k_pool.dtype == np.uint8 and v_pool.dtype == np.uint8
    e = 1 if fp8 else 2
    tile = BLOCK_SIZE * D * e * num_kv_heads
    assert k_pool.size % tile == 0 and v_pool.size == k_pool.size
    nb = k_pool.size // tile
    _load().oracle_reshape_and_cache(_ptr(kb), _ptr(vb), _ptr(k_pool), _ptr(v_pool), _ptr(sl),
                                     T, num_kv_heads, D, nb, int(bool(fp8)),
                                     float(np.float32(k_scale)), float(np.float32(v_scale)))


def paged_attention_decode(q, k_pool: np.ndarray, v_pool: np.ndarray, block_tables,
                           context_lens, num_kv_heads: int, fp8: bool, sm_scale: float,
                           k_scale: float = 1.0, v_scale: float = 1.0,
                           threads: int = 0) -> np.ndarray:
    """fp64 decode attention; q is fp16 [B][Hq][D]; returns fp64 [B][Hq][D]."""
    qb = _f16_bits(q)
    B, Hq, D = qb.shape
    assert Hq % num_kv_heads == 0
    bt = np.ascontiguousarray(np.asarray(block_tables, dtype=np.int32))
    cl = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    assert bt.ndim == 2 and bt.shape[0] == B and cl.shape == (B,)
    out = np.empty((B, Hq, D), dtype=np.float64)
    _load().oracle_paged_attention_decode(
        _ptr(out), _ptr(qb), _ptr(np.ascontiguousarray(k_pool)), _ptr(np.ascontiguousarray(v_pool)),
        _ptr(bt), bt.shape[1], _ptr(cl), B, Hq, num_kv_heads, D, int(bool(fp8)),
        float(np.float32(sm_scale)), float(np.float32(k_scale)), float(np.float32(v_scale)),
        int(threads))
    return out


def paged_prefill_attention(q, k_pool: np.ndarray, v_pool: np.ndarray, block_tables,
                            context_lens, query_start, num_kv_heads: int, fp8: bool,
                            sm_scale: float, k_scale: float = 1.0, v_scale: float = 1.0,
                            threads: int = 0) -> np.ndarray:
    """fp64 causal attention of each sequence's last chunk of tokens over the
    paged cache; q is fp16 [rows][Hq][D] with sequence b's chunk at rows
    query_start[b] .. query_start[b+1]-1; returns fp64 [rows][Hq][D]."""
    qb = _f16_bits(q)
    R, Hq, D = qb.shape
    assert Hq % num_kv_heads == 0
    bt = np.ascontiguousarray(np.asarray(block_tables, dtype=np.int32))
    cl = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    qs = np.ascontiguousarray(np.asarray(query_start, dtype=np.int32))
    B = cl.shape[0]
    assert bt.ndim == 2 and bt.shape[0] == B and qs.shape == (B + 1,) and qs[-1] == R
    out = np.empty((R, Hq, D), dtype=np.float64)
    _load().oracle_paged_prefill_attention(
        _ptr(out), _ptr(qb), _ptr(np.ascontiguousarray(k_pool)), _ptr(np.ascontiguousarray(v_pool)),
        _ptr(bt), bt.shape[1], _ptr(cl), _ptr(qs), B, Hq, num_kv_heads, D, int(bool(fp8)),
        float(np.float32(sm_scale)), float(np.float32(k_scale)), float(np.float32(v_scale)),
        int(threads))
    return out


def reshape_and_cache_dynamic(key, value, k_pool: np.ndarray, v_pool: np.ndarray,
                              k_scales: np.ndarray, v_scales: np.ndarray, slots,
                              num_kv_heads: int) -> None:
    """Write [T][Hkv][D] fp16 rows into FP8 byte pools whose (block, head)
    tiles carry their own fp32 scale ([NB][Hkv] arrays, updated in place):
    dynamic per-block scaling, "Optimización de KV Cache ... (128K)", §8."""
    kb, vb = _f16_bits(key), _f16_bits(value)
    T = kb.shape[0] if kb.ndim else 0
    D = kb.shape[-1]
    assert kb.shape == vb.shape and kb.shape[1] == num_kv_heads
    sl = np.ascontiguousarray(np.asarray(slots, dtype=np.int64))
    assert sl.shape == (T,)
    tile = BLOCK_SIZE * D * num_kv_heads
    assert k_pool.dtype == np.uint8 and v_pool.dtype == np.uint8
    assert k_pool.size % tile == 0 and v_pool.size == k_pool.size
    nb = k_pool.size // tile
    for a in (k_scales, v_scales):
        assert a.dtype == np.float32 and a.shape == (nb, num_kv_heads) and a.flags["C_CONTIGUOUS"]
    _load().oracle_reshape_and_cache_dynamic(_ptr(kb), _ptr(vb), _ptr(k_pool), _ptr(v_pool),
                                             _ptr(k_scales), _ptr(v_scales), _ptr(sl), T,
                                             num_kv_heads, D, nb)


def paged_attention_decode_dynamic(q, k_pool: np.ndarray, v_pool: np.ndarray,
                                   k_scales: np.ndarray, v_scales: np.ndarray, block_tables,
                                   context_lens, num_kv_heads: int, sm_scale: float,
                                   threads: int = 0) -> np.ndarray:
    """fp64 decode attention over an FP8 pool with per-(block, head) scales."""
    qb = _f16_bits(q)
    B, Hq, D = qb.shape
    assert Hq % num_kv_heads == 0
    bt = np.ascontiguousarray(np.asarray(block_tables, dtype=np.int32))
    cl = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    assert bt.ndim == 2 and bt.shape[0] == B and cl.shape == (B,)
    ks = np.ascontiguousarray(k_scales, dtype=np.float32)
    vs = np.ascontiguousarray(v_scales, dtype=np.float32)
    out = np.empty((B, Hq, D), dtype=np.float64)
    _load().oracle_paged_attention_decode_dynamic(
        _ptr(out), _ptr(qb), _ptr(np.ascontiguousarray(k_pool)), _ptr(np.ascontiguousarray(v_pool)),
        _ptr(ks), _ptr(vs), _ptr(bt), bt.shape[1], _ptr(cl), B, Hq, num_kv_heads, D,
        float(np.float32(sm_scale)), int(threads))
    return out


def paged_prefill_attention_dynamic(q, k_pool: np.ndarray, v_pool: np.ndarray,
                                    k_scales: np.ndarray, v_scales: np.ndarray, block_tables,
                                    context_lens, query_start, num_kv_heads: int,
                                    sm_scale: float, threads: int = 0) -> np.ndarray:
    """fp64 chunked-prefill attention over an FP8 pool with per-(block, head)
    scales; arguments as paged_prefill_attention, scales [NB][Hkv] fp32."""
    qb = _f16_bits(q)
    R, Hq, D = qb.shape
    assert Hq % num_kv_heads == 0
    bt = np.ascontiguousarray(np.asarray(block_tables, dtype=np.int32))
    cl = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    qs = np.ascontiguousarray(np.asarray(query_start, dtype=np.int32))
    B = cl.shape[0]
    assert bt.ndim == 2 and bt.shape[0] == B and qs.shape == (B + 1,) and qs[-1] == R
    ks = np.ascontiguousarray(k_scales, dtype=np.float32)
    vs = np.ascontiguousarray(v_scales, dtype=np.float32)
    out = np.empty((R, Hq, D), dtype=np.float64)
    _load().oracle_paged_prefill_attention_dynamic(
        _ptr(out), _ptr(qb), _ptr(np.ascontiguousarray(k_pool)), _ptr(np.ascontiguousarray(v_pool)),
        _ptr(ks), _ptr(vs), _ptr(bt), bt.shape[1], _ptr(cl), _ptr(qs), B, Hq, num_kv_heads, D,
        float(np.float32(sm_scale)), int(threads))
    return out


def max_threads() -> int:
    return _load().oracle_max_threads()


# ------------------------------------------------------------ pool model

class NoFreeBlocks(Exception):
    pass


class InvalidArg(Exception):
    pass


class SharedBlock(Exception):
    """A block other sequences also hold cannot leave the device."""


class BlockPoolModel:
    """Plain model of a refcounted block pool (host bookkeeping only).

    * blocks are handed out from a free list and only when a sequence's next
      token needs a new block (on-demand allocation);
    * fork shares every block of the parent (refcount + 1 each);
    * appending into a partially filled block that another sequence also
      holds first replaces it by a fresh block (copy-on-write) and reports the
      (old, new) pair;
    * freeing a sequence drops one reference per block; a block returns to the
      free list when its count reaches zero (no leak on cancel);
    * an append that cannot get all the blocks it needs changes nothing.

    Prefix cache ("LLM Primer VI, Capítulo 8", §8.3: a prompt is cut into
    block-sized chunks; a chunk already filled for the same preceding text is
    reused by pointing the new table at its block; otherwise it is prefilled and
    its block registered).  The model keys an entry by the exact token prefix up
    to the end of the chunk, so no hashing is involved:

    * only full blocks are cached; the cache's hold on a block is not a
      reference;
    * a cached block that no sequence holds is evictable; it counts as
      available, and when the free list is empty a new block comes from the
      evictable block whose entry was hit or registered longest ago;
    * registration keeps an entry that already exists for the same prefix and
      stops at the first chunk whose block already serves another prefix.

    Swap space ("KV Cache y PagedAttention: por qué se reduce la velocidad de
    tu servidor LLM": when memory runs out, single pages go to CPU memory
    instead of whole sequences):

    * host slots are handed out in ascending order and returned at the back;
    * a run of a sequence's blocks moves to host slots only if every block is
      on the device and held by that sequence alone; the device blocks are
      released (a cached one loses its cache entry);
    * swapping in takes device blocks as an append would, in logical order;
    * a sequence with swapped blocks cannot be appended to, forked or
      registered; its table shows -1 for them.
    """

    def __init__(self, free_order, block_size: int = BLOCK_SIZE):
        self.block_size = block_size
        self.num_blocks = len(free_order)
        # free list is popped from the front in the given order
        self.free = list(free_order)
        self.ref = [0] * self.num_blocks
        self.seqs = {}
        self._next = 0
        self.cache = {}         # token prefix (tuple) -> block
        self.prefix_of = {}     # block -> token prefix it is cached for
        self.last_use = {}      # token prefix -> tick of last hit or registration
        self._tick = 0
        self.hit_blocks = 0
        self.miss_blocks = 0
        self.num_host = 0
        self.host_free = []

    def num_free(self) -> int:
        return len(self.free)

    def evictable(self):
        """Cached blocks no sequence holds, least recently used first."""
        blocks = [b for b, pre in self.prefix_of.items() if self.ref[b] == 0]
        return sorted(blocks, key=lambda b: self.last_use[self.prefix_of[b]])

    def available(self) -> int:
        return len(self.free) + len(self.evictable())

    def usage(self) -> float:
        return (self.num_blocks - self.available()) / self.num_blocks

    def _take(self) -> int:
        if self.free:
            b = self.free.pop(0)
        else:
            b = self.evictable()[0]
            pre = self.prefix_of.pop(b)
            del self.cache[pre]
            del self.last_use[pre]
        self.ref[b] += 1
        return b

    def _release(self, b: int) -> None:
        self.ref[b] -= 1
        assert self.ref[b] >= 0
        if self.ref[b] == 0 and b not in self.prefix_of:
            self.free.append(b)

    def create(self) -> int:
        sid = self._next
        self._next += 1
        self.seqs[sid] = ([], 0)
        return sid

    def _swapped(self, sid) -> int:
        return sum(1 for b in self.seqs[sid][0] if isinstance(b, tuple))

    def fork(self, parent: int) -> int:
        blocks, n = self.seqs[parent]
        if self._swapped(parent):
            raise InvalidArg()
        for b in blocks:
            self.ref[b] += 1
        sid = self.create()
        self.seqs[sid] = (list(blocks), n)
        return sid

    def append(self, sid: int, n_tokens: int):
        blocks, n = self.seqs[sid]
        bs = self.block_size
        if n_tokens == 0:      # nothing is written, so nothing needs copying
            return [], []
        if self._swapped(sid):
            raise InvalidArg()
        cow = n % bs != 0 and self.ref[blocks[-1]] > 1
        have = -(-n // bs)
        need = -(-(n + n_tokens) // bs) - have + (1 if cow else 0)
        if need > self.available():
            raise NoFreeBlocks()
        blocks = list(blocks)
        pairs = []
        if cow:
            new = self._take()
            old = blocks[-1]
            self._release(old)
            blocks[-1] = new
            pairs.append((old, new))
        slots = []
        for pos in range(n, n + n_tokens):
            if pos // bs >= len(blocks):
                blocks.append(self._take())
            slots.append(blocks[pos // bs] * bs + pos % bs)
        self.seqs[sid] = (blocks, n + n_tokens)
        return slots, pairs

    def free_seq(self, sid: int) -> None:
        blocks, _ = self.seqs.pop(sid)
        for b in blocks:
            if isinstance(b, tuple):
                self.host_free.append(b[1])
            else:
                self._release(b)

    def create_cached(self, tokens):
        """New sequence mapped onto the cached blocks of the leading chunks of
        `tokens`, up to the first chunk not cached; returns (sid, n_cached)."""
        bs = self.block_size
        chunks = len(tokens) // bs
        blocks = []
        for i in range(chunks):
            pre = tuple(tokens[:bs * (i + 1)])
            if pre not in self.cache:
                break
            b = self.cache[pre]
            self.ref[b] += 1
            self._tick += 1
            self.last_use[pre] = self._tick
            blocks.append(b)
        self.hit_blocks += len(blocks)
        self.miss_blocks += chunks - len(blocks)
        sid = self.create()
        self.seqs[sid] = (blocks, len(blocks) * bs)
        return sid, len(blocks) * bs

    def cache_prefix(self, sid: int, tokens) -> None:
        """Register the full, filled blocks of `sid` under the prefixes of `tokens`."""
        blocks, n = self.seqs[sid]
        if self._swapped(sid):
            raise InvalidArg()
        bs = self.block_size
        for i in range(min(len(tokens), n) // bs):
            pre = tuple(tokens[:bs * (i + 1)])
            if pre in self.cache:
                continue
            b = blocks[i]
            if b in self.prefix_of:
                break
            self.cache[pre] = b
            self.prefix_of[b] = pre
            self._tick += 1
            self.last_use[pre] = self._tick

    def prefix_cache_stats(self) -> dict:
        return {"hit_blocks": self.hit_blocks, "miss_blocks": self.miss_blocks,
                "cached_blocks": len(self.cache), "evictable_blocks": len(self.evictable())}

    def clear_prefix_cache(self) -> None:
        self.free.extend(self.evictable())
        self.cache.clear()
        self.prefix_of.clear()
        self.last_use.clear()

    def table(self, sid: int):
        return [-1 if isinstance(b, tuple) else b for b in self.seqs[sid][0]]

    def num_free_host(self) -> int:
        return len(self.host_free)

    def num_swapped(self, sid: int) -> int:
        return self._swapped(sid)

    def set_swap_space(self, num_host_blocks: int) -> None:
        if len(self.host_free) != self.num_host:
            raise InvalidArg()
        self.num_host = num_host_blocks
        self.host_free = list(range(num_host_blocks))

    def swap_out(self, sid: int, first: int, n_blocks: int):
        blocks, n = self.seqs[sid]
        if first < 0 or n_blocks < 0 or first + n_blocks > len(blocks):
            raise InvalidArg()
        for b in blocks[first:first + n_blocks]:
            if isinstance(b, tuple):
                raise InvalidArg()
            if self.ref[b] != 1:
                raise SharedBlock()
        if n_blocks > len(self.host_free):
            raise NoFreeBlocks()
        blocks = list(blocks)
        pairs = []
        for i in range(first, first + n_blocks):
            b = blocks[i]
            slot = self.host_free.pop(0)
            if b in self.prefix_of:
                pre = self.prefix_of.pop(b)
                del self.cache[pre]
                del self.last_use[pre]
            self._release(b)
            blocks[i] = ("h", slot)
            pairs.append((b, slot))
        self.seqs[sid] = (blocks, n)
        return pairs

    def swap_in(self, sid: int):
        blocks, n = self.seqs[sid]
        k = self._swapped(sid)
        if k == 0:
            return []
        if k > self.available():
            raise NoFreeBlocks()
        blocks = list(blocks)
        pairs = []
        for i, b in enumerate(blocks):
            if isinstance(b, tuple):
                d = self._take()
                self.host_free.append(b[1])
                blocks[i] = d
                pairs.append((b[1], d))
        self.seqs[sid] = (blocks, n)
        return pairs

    def length(self, sid: int) -> int:
        return self.seqs[sid][1]
