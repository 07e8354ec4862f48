"""MI355X-native jagged flash attention: thin Python binding over libjfa.so.

Every step of the computation runs in the HIP kernels behind the C ABI declared
in include/jfa.h; this module only marshals arguments (torch tensors supply
device memory and the stream). If libjfa.so has not been built, every entry
point raises: there is no fallback path.

Low-level names mirror the C ABI (tile_rows, default_slots, schedule_count,
schedule, bwd_workspace_bytes, fwd, bwd, and the block-sparse sparse_lists,
schedule_sparse, fwd_sparse, bwd_sparse). `Plan` bundles the host schedule,
its device copy and the workspace for one problem.
"""
from __future__ import annotations

import ctypes
import functools
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libjfa.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
CAUSAL, BROADCAST_Q, BLOCK_DIAG64, ROTARY, BLOCK_DIAG, BLOCK_SPARSE = 1, 2, 4, 8, 16, 32
KIND_FWD, KIND_BWD = 0, 1
ORDER_INORDER, ORDER_ZIGZAG, ORDER_XCD_ZIGZAG, ORDER_FOLDED_ZIGZAG, ORDER_XCD_INORDER = 0, 1, 2, 3, 4
PASS_DQ, PASS_DKDV, PASS_ALL = 1, 2, 3


class JfaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"jfa status {status}: {message}")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("max_len", ctypes.c_int32),
                ("lq", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("total_kv", ctypes.c_int64), ("scale", ctypes.c_float),
                ("rope_base", ctypes.c_float), ("window", ctypes.c_int32),
                ("block", ctypes.c_int32)]


class SparseListsDev(ctypes.Structure):
    _fields_ = [("seq_base", ctypes.c_void_p), ("list_ptr", ctypes.c_void_p),
                ("entries", ctypes.c_void_p)]


_lib = None


def lib():
    """Load libjfa.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m variable_length_flash_jaggedfa_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(Problem)
        vp, i32, i64, u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
        L.jfa_tile_rows.argtypes = [i32, i32, u32]
        L.jfa_tile_rows.restype = i32
        L.jfa_default_slots.argtypes = [i32, i32, u32, i32, ctypes.POINTER(i32)]
        L.jfa_default_slots.restype = i32
        L.jfa_schedule_count.argtypes = [P, vp, i32, ctypes.POINTER(i64)]
        L.jfa_schedule_count.restype = i32
        L.jfa_schedule.argtypes = [P, vp, i32, i32, i32, vp, vp, i64]
        L.jfa_schedule.restype = i32
        L.jfa_bwd_workspace_bytes.argtypes = [P]
        L.jfa_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.jfa_fwd_workspace_bytes.argtypes = [P]
        L.jfa_fwd_workspace_bytes.restype = ctypes.c_size_t
        L.jfa_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, ctypes.c_size_t, vp]
        L.jfa_fwd.restype = i32
        L.jfa_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, i32, vp, vp,
                              vp, vp, ctypes.c_size_t, vp]
        L.jfa_bwd.restype = i32
        L.jfa_bwd_passes.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, i32, vp,
                                     vp, vp, vp, ctypes.c_size_t, ctypes.c_uint32, vp]
        L.jfa_bwd_passes.restype = i32
        L.jfa_bwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, i32,
                                      vp, vp, vp, vp]
        L.jfa_bwd_noalloc.restype = i32
        SL = ctypes.POINTER(SparseListsDev)
        L.jfa_sparse_lists_count.argtypes = [P, vp, vp, i64, i32, ctypes.POINTER(i64),
                                             ctypes.POINTER(i64)]
        L.jfa_sparse_lists_count.restype = i32
        L.jfa_sparse_lists.argtypes = [P, vp, vp, i64, i32, vp, vp, vp, i64]
        L.jfa_sparse_lists.restype = i32
        L.jfa_schedule_sparse.argtypes = [P, vp, vp, vp, i32, i32, i32, vp, vp, i64]
        L.jfa_schedule_sparse.restype = i32
        L.jfa_fwd_sparse.argtypes = [P, vp, vp, vp, vp, SL, vp, vp, i32, vp, vp, vp]
        L.jfa_fwd_sparse.restype = i32
        L.jfa_bwd_sparse.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, SL, vp, vp, i32, SL, vp, vp,
                                     i32, vp, vp, vp, vp, ctypes.c_size_t, ctypes.c_uint32, vp]
        L.jfa_bwd_sparse.restype = i32
        L.jfa_probe_copy.argtypes = [vp, vp, ctypes.c_uint64, i32, vp]
        L.jfa_probe_copy.restype = i32
        L.jfa_probe_mfma.argtypes = [i32, i32, vp, vp, vp]
        L.jfa_probe_mfma.restype = i32
        L.jfa_status_string.argtypes = [i32]
        L.jfa_status_string.restype = ctypes.c_char_p
        L.jfa_last_error.argtypes = []
        L.jfa_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int):
    if status != OK:
        raise JfaError(status, lib().jfa_last_error().decode())


def problem(num_seqs, num_heads, head_dim, max_len, total_kv, scale, flags=0, lq=0,
            rope_base=0.0, window=0, block=0) -> Problem:
    return Problem(int(num_seqs), int(num_heads), int(head_dim), int(max_len), int(lq),
                   int(flags), int(total_kv), float(scale), float(rope_base), int(window),
                   int(block))


def tile_rows(kind: int, head_dim: int, flags: int = 0) -> int:
    return int(lib().jfa_tile_rows(kind, head_dim, flags))


@functools.lru_cache(maxsize=None)
def default_slots(kind: int, head_dim: int, flags: int = 0, device: int = 0) -> int:
    """Persistent workgroups for a schedule of `kind` on `device` (the device's
    compute units times the kernel's resident workgroups per unit; fixed for the
    process, so kept once asked)."""
    n = ctypes.c_int32(0)
    _check(lib().jfa_default_slots(kind, head_dim, flags, device, ctypes.byref(n)))
    return int(n.value)


def _host_i32(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a


def schedule_count(p: Problem, offsets_host, kind: int) -> int:
    off = _host_i32(offsets_host)
    n = ctypes.c_int64(0)
    _check(lib().jfa_schedule_count(ctypes.byref(p), off.ctypes.data, kind, ctypes.byref(n)))
    return int(n.value)


def schedule(p: Problem, offsets_host, kind: int, order: int, num_slots: int):
    """Host tile schedule -> (slot_ptr int32 [S+1], tiles int32 [N,4])."""
    off = _host_i32(offsets_host)
    n = schedule_count(p, off, kind)
    slot_ptr = np.zeros(num_slots + 1, dtype=np.int32)
    tiles = np.zeros((max(n, 1), 4), dtype=np.int32)
    _check(lib().jfa_schedule(ctypes.byref(p), off.ctypes.data, kind, order, num_slots,
                              slot_ptr.ctypes.data, tiles.ctypes.data, n))
    return slot_ptr, tiles[:n]


def _host_u8(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.uint8).reshape(-1)


def sparse_lists(p: Problem, offsets_host, mask_host, kind: int):
    """Block-sparse step lists of `kind` -> (seq_base [B+1], list_ptr [units+1],
    entries), int32 host arrays."""
    off, m = _host_i32(offsets_host), _host_u8(mask_host)
    nu, ne = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(lib().jfa_sparse_lists_count(ctypes.byref(p), off.ctypes.data, m.ctypes.data, m.size,
                                        kind, ctypes.byref(nu), ctypes.byref(ne)))
    seq_base = np.zeros(p.num_seqs + 1, dtype=np.int32)
    list_ptr = np.zeros(nu.value + 1, dtype=np.int32)
    entries = np.zeros(max(ne.value, 1), dtype=np.int32)
    _check(lib().jfa_sparse_lists(ctypes.byref(p), off.ctypes.data, m.ctypes.data, m.size, kind,
                                  seq_base.ctypes.data, list_ptr.ctypes.data,
                                  entries.ctypes.data, ne.value))
    return seq_base, list_ptr, entries[:ne.value]


def schedule_sparse(p: Problem, offsets_host, list_ptr_host, entries_host, kind: int, order: int,
                    num_slots: int):
    """Block-sparse host tile schedule from the step lists of `kind` (list_ptr and
    entries of sparse_lists) -> (slot_ptr int32 [S+1], tiles int32 [N,4])."""
    off, lp = _host_i32(offsets_host), _host_i32(list_ptr_host)
    ent = _host_i32(entries_host if entries_host is not None and len(entries_host) else [0])
    n = schedule_count(p, off, kind)
    slot_ptr = np.zeros(num_slots + 1, dtype=np.int32)
    tiles = np.zeros((max(n, 1), 4), dtype=np.int32)
    _check(lib().jfa_schedule_sparse(ctypes.byref(p), off.ctypes.data, lp.ctypes.data,
                                     ent.ctypes.data, kind, order, num_slots,
                                     slot_ptr.ctypes.data, tiles.ctypes.data, n))
    return slot_ptr, tiles[:n]


def _lists(dev):
    """(seq_base, list_ptr, entries) device tensors -> jfa_sparse_lists_dev."""
    return SparseListsDev(*(_ptr(t) for t in dev))


def fwd_sparse(p: Problem, q, k, v, offsets_dev, lists_dev, slot_ptr_dev, tiles_dev, num_slots,
               out, lse, stream=None):
    sl = _lists(lists_dev)
    _check(lib().jfa_fwd_sparse(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(offsets_dev),
                                ctypes.byref(sl), _ptr(slot_ptr_dev), _ptr(tiles_dev),
                                int(num_slots), _ptr(out), _ptr(lse), _stream(stream)))


def bwd_sparse(p: Problem, q, k, v, out, dout, lse, offsets_dev, q_lists_dev, q_slot_ptr_dev,
               q_tiles_dev, q_num_slots, kv_lists_dev, kv_slot_ptr_dev, kv_tiles_dev,
               kv_num_slots, dq, dk, dv, workspace, passes=PASS_ALL, stream=None):
    ql, kl = _lists(q_lists_dev), _lists(kv_lists_dev)
    _check(lib().jfa_bwd_sparse(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                _ptr(dout), _ptr(lse), _ptr(offsets_dev), ctypes.byref(ql),
                                _ptr(q_slot_ptr_dev), _ptr(q_tiles_dev), int(q_num_slots),
                                ctypes.byref(kl), _ptr(kv_slot_ptr_dev), _ptr(kv_tiles_dev),
                                int(kv_num_slots), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                _ws_bytes(workspace), int(passes), _stream(stream)))


def bwd_workspace_bytes(p: Problem) -> int:
    return int(lib().jfa_bwd_workspace_bytes(ctypes.byref(p)))


def fwd_workspace_bytes(p: Problem) -> int:
    return int(lib().jfa_fwd_workspace_bytes(ctypes.byref(p)))


def _ws_bytes(workspace) -> int:
    return 0 if workspace is None else workspace.numel() * workspace.element_size()


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def fwd(p: Problem, q, k, v, offsets_dev, slot_ptr_dev, tiles_dev, num_slots, out, lse,
        workspace=None, stream=None):
    _check(lib().jfa_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(offsets_dev),
                         _ptr(slot_ptr_dev), _ptr(tiles_dev), int(num_slots), _ptr(out),
                         _ptr(lse), _ptr(workspace), _ws_bytes(workspace), _stream(stream)))


def bwd(p: Problem, q, k, v, out, dout, lse, offsets_dev, q_slot_ptr_dev, q_tiles_dev,
        q_num_slots, kv_slot_ptr_dev, kv_tiles_dev, kv_num_slots, dq, dk, dv, workspace,
        stream=None):
    ws_bytes = _ws_bytes(workspace)
    _check(lib().jfa_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout),
                         _ptr(lse), _ptr(offsets_dev), _ptr(q_slot_ptr_dev), _ptr(q_tiles_dev),
                         int(q_num_slots), _ptr(kv_slot_ptr_dev), _ptr(kv_tiles_dev),
                         int(kv_num_slots), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                         ws_bytes, _stream(stream)))


def bwd_passes(p: Problem, q, k, v, out, dout, lse, offsets_dev, q_slot_ptr_dev, q_tiles_dev,
               q_num_slots, kv_slot_ptr_dev, kv_tiles_dev, kv_num_slots, dq, dk, dv, workspace,
               passes, stream=None):
    ws_bytes = _ws_bytes(workspace)
    _check(lib().jfa_bwd_passes(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                _ptr(dout), _ptr(lse), _ptr(offsets_dev), _ptr(q_slot_ptr_dev),
                                _ptr(q_tiles_dev), int(q_num_slots), _ptr(kv_slot_ptr_dev),
                                _ptr(kv_tiles_dev), int(kv_num_slots), _ptr(dq), _ptr(dk),
                                _ptr(dv), _ptr(workspace), ws_bytes, int(passes),
                                _stream(stream)))


NOALLOC_SCRATCH_BYTES = 32 << 20  # JFA_NOALLOC_SCRATCH_BYTES


def bwd_noalloc(p: Problem, q, k, v, out, dout, lse, offsets_dev, q_slot_ptr_dev, q_tiles_dev,
                q_num_slots, kv_slot_ptr_dev, kv_tiles_dev, kv_num_slots, dq, dk, dv,
                stream=None):
    """jfa_bwd with the library's static scratch array as its workspace."""
    _check(lib().jfa_bwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                 _ptr(dout), _ptr(lse), _ptr(offsets_dev), _ptr(q_slot_ptr_dev),
                                 _ptr(q_tiles_dev), int(q_num_slots), _ptr(kv_slot_ptr_dev),
                                 _ptr(kv_tiles_dev), int(kv_num_slots), _ptr(dq), _ptr(dk),
                                 _ptr(dv), _stream(stream)))


def probe_copy(src, dst, workgroups: int, stream=None):
    """HBM copy probe (measurement only): src -> dst, equal-sized device tensors."""
    nbytes = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() == nbytes
    _check(lib().jfa_probe_copy(_ptr(src), _ptr(dst), nbytes, int(workgroups), _stream(stream)))


def probe_mfma(iters: int, workgroups: int, sink, clocks, stream=None):
    """Matrix-core throughput probe (measurement only): `sink` float32
    [workgroups*256] and `clocks` int64 [workgroups*4] device tensors."""
    _check(lib().jfa_probe_mfma(int(iters), int(workgroups), _ptr(sink), _ptr(clocks),
                                _stream(stream)))


@dataclass
class Schedule:
    slot_ptr: np.ndarray
    tiles: np.ndarray
    num_slots: int
    slot_ptr_dev: object = None
    tiles_dev: object = None
    lists: tuple = None       # BLOCK_SPARSE: host (seq_base, list_ptr, entries)
    lists_dev: tuple = None   # and their device copies


class Plan:
    """Everything one jagged problem needs on the device, built once.

    offsets_host: int32 [B+1] (numpy); H, D; flags; lq for broadcast-Q; rope_base
    for ROTARY; window (CAUSAL only) for a causal sliding window of that many keys;
    block (BLOCK_DIAG) for the tokens per diagonal block; block_mask (BLOCK_SPARSE)
    for the flat uint8 block masks of every sequence (row-major n_b x n_b each,
    n_b = ceil(L_b / 64)), from which the step lists of both kinds are built.
    Builds the FWD and BWD schedules on the host (by default the folded zigzag:
    the work-sorted zigzag deal, with the tiles of a causal (sequence, head) paired
    so that they run side by side; for BLOCK_SPARSE the balanced in-order deal,
    which keeps the tiles of one (sequence, head) together in time and on one XCD:
    their step lists differ, so a work-sorted deal scatters them and they share
    less K/V in L2), copies them and the offsets to the device, and allocates the
    dQ workspace.
    """

    def __init__(self, offsets_host, num_heads, head_dim, scale, flags=0, lq=0,
                 order=None, num_slots=None, device="cuda", rope_base=0.0,
                 window=0, block=0, block_mask=None):
        import torch
        off = _host_i32(offsets_host)
        L = np.diff(off.astype(np.int64))
        self.offsets_host = off
        self.sparse = bool(flags & BLOCK_SPARSE)
        if self.sparse:
            block = 64
        if order is None:
            order = ORDER_XCD_INORDER if self.sparse else ORDER_FOLDED_ZIGZAG
        self.order = order
        self.p = problem(len(L), num_heads, head_dim, int(L.max()) if len(L) else 0,
                         int(off[-1]), scale, flags, lq, rope_base, window, block)
        self.device = torch.device(device)
        # Every int32 array the kernels read (the offsets, the schedules and the
        # step lists) goes to the device in one copy, each array at a 256-byte
        # boundary of the packed buffer and at least one element long (an empty
        # array still needs a valid device pointer).
        packed, spans = [], []

        def put(a):
            a = np.ascontiguousarray(a, dtype=np.int32).ravel()
            if a.size == 0:
                a = np.zeros(1, np.int32)
            pos = sum(x.size for x in packed)
            packed.append(a)
            packed.append(np.zeros((-a.size) % 64, np.int32))
            spans.append((pos, a.size))
            return len(spans) - 1

        i_off = put(off)
        bs = 64 if flags & BLOCK_DIAG64 else (block if flags & BLOCK_DIAG else 0)
        # blocks of 32 or 64 tokens: single-tile kernels, no schedule and no lse;
        # blocks of 128 or 256 tokens are scheduled as jagged tiles over the blocks
        self.block = 0 < bs <= 64
        self.sched = {}
        if self.block:
            schedule_count(self.p, off, KIND_FWD)  # validates the offsets
        else:
            for kind in (KIND_FWD, KIND_BWD):
                S = num_slots or default_slots(kind, head_dim, flags, self.device.index or 0)
                lists = None
                if self.sparse:
                    lists = sparse_lists(self.p, off, block_mask, kind)
                    sp, tl = schedule_sparse(self.p, off, lists[1], lists[2], kind, order, S)
                else:
                    sp, tl = schedule(self.p, off, kind, order, S)
                sch = Schedule(sp, tl, S)
                if lists is not None:
                    sch.lists = lists
                    sch.lists_dev = tuple(put(a) for a in lists)
                sch.slot_ptr_dev = put(sp)
                sch.tiles_dev = put(tl if len(tl) else np.zeros((1, 4), np.int32))
                self.sched[kind] = sch
        dev = torch.from_numpy(np.concatenate(packed)).to(self.device)

        def view(i):
            pos, n = spans[i]
            return dev[pos:pos + n]

        self.offsets_dev = view(i_off)
        for sch in self.sched.values():
            if sch.lists_dev is not None:
                sch.lists_dev = tuple(view(i) for i in sch.lists_dev)
            sch.slot_ptr_dev = view(sch.slot_ptr_dev)
            sch.tiles_dev = view(sch.tiles_dev).view(-1, 4)
        nbytes = bwd_workspace_bytes(self.p)
        self.workspace = (torch.empty((nbytes + 3) // 4, dtype=torch.float32, device=self.device)
                          if nbytes else None)
        nbytes = fwd_workspace_bytes(self.p)
        self.fwd_workspace = (torch.empty((nbytes + 3) // 4, dtype=torch.float32,
                                          device=self.device) if nbytes else None)

    @property
    def num_q_rows(self):
        return self.p.lq if self.p.flags & BROADCAST_Q else self.p.total_kv

    def _out_shape(self):
        H, D = self.p.num_heads, self.p.head_dim
        if self.p.flags & BROADCAST_Q:
            return (self.p.num_seqs, self.p.lq, H, D)
        return (self.p.total_kv, H, D)

    def _lse_shape(self):
        H = self.p.num_heads
        if self.p.flags & BROADCAST_Q:
            return (self.p.num_seqs, H, self.p.lq)
        return (H, self.p.total_kv)

    def forward(self, q, k, v, out=None, lse=None, stream=None):
        import torch
        out = out if out is not None else torch.empty(self._out_shape(), dtype=torch.bfloat16,
                                                      device=self.device)
        if not self.block and lse is None:
            lse = torch.empty(self._lse_shape(), dtype=torch.float32, device=self.device)
        s = self.sched.get(KIND_FWD)
        if self.sparse:
            fwd_sparse(self.p, q, k, v, self.offsets_dev, s.lists_dev, s.slot_ptr_dev,
                       s.tiles_dev, s.num_slots, out, lse, stream)
            return out, lse
        fwd(self.p, q, k, v, self.offsets_dev, s.slot_ptr_dev if s else None,
            s.tiles_dev if s else None, s.num_slots if s else 0, out,
            None if self.block else lse, self.fwd_workspace, stream)
        return out, (None if self.block else lse)

    def backward(self, q, k, v, out, dout, lse=None, dq=None, dk=None, dv=None, stream=None,
                 passes=PASS_ALL):
        """dQ, dK, dV. `passes` selects the backward passes (PASS_DQ must run before
        PASS_DKDV on the same inputs: the second reads Di from the plan's workspace)."""
        import torch
        dq = dq if dq is not None else torch.empty_like(q)
        dk = dk if dk is not None else torch.empty_like(k)
        dv = dv if dv is not None else torch.empty_like(v)
        sq, skv = self.sched.get(KIND_FWD), self.sched.get(KIND_BWD)
        if self.sparse:
            bwd_sparse(self.p, q, k, v, out, dout, lse, self.offsets_dev, sq.lists_dev,
                       sq.slot_ptr_dev, sq.tiles_dev, sq.num_slots, skv.lists_dev,
                       skv.slot_ptr_dev, skv.tiles_dev, skv.num_slots, dq, dk, dv,
                       self.workspace, passes, stream)
            return dq, dk, dv
        args = (self.p, q, k, v, out, dout, None if self.block else lse, self.offsets_dev,
                sq.slot_ptr_dev if sq else None, sq.tiles_dev if sq else None,
                sq.num_slots if sq else 0, skv.slot_ptr_dev if skv else None,
                skv.tiles_dev if skv else None, skv.num_slots if skv else 0,
                dq, dk, dv, self.workspace)
        if passes == PASS_ALL:
            bwd(*args, stream)
        else:
            bwd_passes(*args, passes, stream)
        return dq, dk, dv

    def backward_noalloc(self, q, k, v, out, dout, lse=None, dq=None, dk=None, dv=None,
                         stream=None):
        """The backward through jfa_bwd_noalloc (the library's static scratch array
        instead of the plan's workspace); the outputs must be given to allocate
        nothing here either."""
        sq, skv = self.sched.get(KIND_FWD), self.sched.get(KIND_BWD)
        bwd_noalloc(self.p, q, k, v, out, dout, None if self.block else lse, self.offsets_dev,
                    sq.slot_ptr_dev if sq else None, sq.tiles_dev if sq else None,
                    sq.num_slots if sq else 0, skv.slot_ptr_dev if skv else None,
                    skv.tiles_dev if skv else None, skv.num_slots if skv else 0, dq, dk, dv,
                    stream)
        return dq, dk, dv
