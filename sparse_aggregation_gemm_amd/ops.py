"""Thin Python binding of the C ABI, with the same names as its entry points.

Argument marshalling only: tensors become device pointers, sizes and leading
dimensions; PyTorch supplies device memory and the current stream.  Every
step of the computation runs in libsag.so's HIP kernels.

Dense operands are 2-D tensors with unit column stride whose row stride is
the leading dimension (a multiple of 16 bytes); ``empty_dense`` allocates
such a tensor with the row padded.  bf16 tensors are torch.bfloat16.
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass, field

import torch

from . import _lib as L

_DT = {torch.float32: L.SAG_F32, torch.bfloat16: L.SAG_BF16}
_NORM = {"gcn": L.SAG_NORM_GCN, "mean": L.SAG_NORM_MEAN, "none": L.SAG_NORM_NONE}


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def dtype_code(dtype: torch.dtype) -> int:
    if dtype not in _DT:
        raise TypeError(f"unsupported dtype {dtype}")
    return _DT[dtype]


def padded_ld(d: int, dtype: torch.dtype) -> int:
    """Row pitch in elements: rows wider than 64 bytes span whole 128-byte
    cache lines (a gathered row then touches as few lines as possible),
    narrower rows are padded to 16 bytes."""
    es = torch.empty(0, dtype=dtype).element_size()
    nbytes = max(d, 1) * es
    line = 128 if nbytes > 64 else 16
    return (nbytes + line - 1) // line * line // es


def empty_dense(rows: int, d: int, dtype: torch.dtype, device, fill=None) -> torch.Tensor:
    """[rows, d] view of a [rows, ld] buffer with ld = padded_ld(d, dtype)."""
    buf = torch.empty((rows, padded_ld(d, dtype)), dtype=dtype, device=device)
    if fill is not None:
        buf.fill_(fill)
    return buf[:, :d]


def as_dense(x: torch.Tensor) -> torch.Tensor:
    """x with a 16-byte row pitch (copied into a padded buffer if needed)."""
    es = x.element_size()
    if x.dim() == 2 and x.stride(1) == 1 and (x.stride(0) * es) % 16 == 0 \
            and x.stride(0) >= x.shape[1] and x.data_ptr() % 16 == 0:
        return x
    out = empty_dense(x.shape[0], x.shape[1], x.dtype, x.device)
    out.copy_(x)
    return out


def _ld(x: torch.Tensor) -> int:
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("dense operands must be 2-D with unit column stride")
    return max(x.stride(0), x.shape[1]) if x.shape[0] <= 1 else x.stride(0)


def _need_rows(what: str, t, n: int) -> None:
    """ValueError unless t (when given) has at least n rows: the C ABI takes
    pointers and cannot see tensor sizes, so a short buffer would be read or
    written past its end on the GPU."""
    if t is not None and t.shape[0] < n:
        raise ValueError(f"{what} has {t.shape[0]} rows; the call reads or writes {n}")


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


@dataclass
class Csr:
    """A CSR matrix in device memory plus its optional schedule."""
    n_rows: int
    n_cols: int
    indptr: torch.Tensor
    indices: torch.Tensor
    values: torch.Tensor | None
    sched: torch.Tensor | None = None
    row_mean: bool = False     # every entry of row r is 1/len(r) (the build's mean-normalised A)
    raw: L.SagCsr = field(default_factory=L.SagCsr)
    hub_part: "Csr | None" = None    # hub split (csr_hub_split): entries in the hub columns
    cold_part: "Csr | None" = None   # and the rest
    col_slices: bool = False   # products gather X in 128-byte column slices (csr_set_col_slices)

    def __post_init__(self):
        self.raw.n_rows = self.n_rows
        self.raw.n_cols = self.n_cols
        self.raw.nnz = self.nnz
        self.raw.indptr = _ptr(self.indptr)
        self.raw.indices = _ptr(self.indices)
        self.raw.values = _ptr(self.values)
        self.raw.row_mean = int(bool(self.row_mean))
        self.raw.col_slices = int(bool(self.col_slices))

    @property
    def nnz(self) -> int:
        return int(self.indices.numel())

    @property
    def ref(self):
        return ctypes.byref(self.raw)

    @property
    def device(self):
        return self.indptr.device


@dataclass
class Built:
    A: Csr
    AT: Csr | None
    deg: torch.Tensor        # int32 [n_local + n_halo]
    halo_gid: torch.Tensor   # int32 [n_halo]

    @property
    def n_local(self) -> int:
        return self.A.n_rows

    @property
    def n_halo(self) -> int:
        return int(self.halo_gid.numel())


def csr_build_normalize_query(src: torch.Tensor, dst: torch.Tensor, n_global: int, lo: int, hi: int,
                              symmetrize: bool, self_loops: bool) -> tuple[int, int]:
    """sag_csr_build_normalize_query: (nnz, n_halo) of the build of rows
    [lo, hi), without its outputs.  Synchronises the current stream."""
    dev = src.device
    src = src.to(torch.int32).contiguous()
    dst = dst.to(torch.int32).contiguous()
    n_edges = src.numel()
    flags = (L.SAG_SYMMETRIZE if symmetrize else 0) | (L.SAG_SELF_LOOPS if self_loops else 0)
    lib = L.lib()
    ws = _ws(lib.sag_csr_build_workspace_bytes(n_edges, n_global, lo, hi, flags), dev)
    nnz, n_halo = ctypes.c_int64(0), ctypes.c_int64(0)
    st = lib.sag_csr_build_normalize_query(_ptr(src), _ptr(dst), n_edges, n_global, lo, hi, flags,
                                           ctypes.byref(nnz), ctypes.byref(n_halo), _ptr(ws), ws.numel(),
                                           _stream(dev))
    L.check("sag_csr_build_normalize_query", st)
    return nnz.value, n_halo.value


def csr_build_normalize(src: torch.Tensor, dst: torch.Tensor, n_global: int, lo: int, hi: int,
                        symmetrize: bool, self_loops: bool, norm: str = "gcn",
                        deg_global: torch.Tensor | None = None, transpose: bool = True,
                        max_halo: int | None = None) -> Built:
    """sag_csr_build_normalize: the normalised CSR of rows [lo, hi), its
    transpose, degrees and HALO list.  Synchronises the current stream."""
    dev = src.device
    src = src.to(torch.int32).contiguous()
    dst = dst.to(torch.int32).contiguous()
    n_edges = src.numel()
    flags = (L.SAG_SYMMETRIZE if symmetrize else 0) | (L.SAG_SELF_LOOPS if self_loops else 0)
    n_local = hi - lo
    cap_nnz = (2 if symmetrize else 1) * n_edges + (n_local if self_loops else 0)
    cap_halo = n_global - n_local if max_halo is None else int(max_halo)
    lib = L.lib()
    ws = _ws(lib.sag_csr_build_workspace_bytes(n_edges, n_global, lo, hi, flags), dev)
    indptr = torch.empty(n_local + 1, dtype=torch.int64, device=dev)
    indices = torch.empty(max(cap_nnz, 1), dtype=torch.int32, device=dev)
    values = torch.empty(max(cap_nnz, 1), dtype=torch.float32, device=dev)
    if transpose:
        indptr_t = torch.empty(n_local + cap_halo + 1, dtype=torch.int64, device=dev)
        indices_t = torch.empty(max(cap_nnz, 1), dtype=torch.int32, device=dev)
        values_t = torch.empty(max(cap_nnz, 1), dtype=torch.float32, device=dev)
    else:
        indptr_t = indices_t = values_t = None
    deg = torch.empty(max(n_local + cap_halo, 1), dtype=torch.int32, device=dev)
    halo = torch.empty(max(cap_halo, 1), dtype=torch.int32, device=dev)
    if deg_global is not None:
        deg_global = deg_global.to(device=dev, dtype=torch.int32).contiguous()
    nnz, n_halo = ctypes.c_int64(0), ctypes.c_int64(0)
    st = lib.sag_csr_build_normalize(
        _ptr(src), _ptr(dst), n_edges, n_global, lo, hi, flags, _NORM[norm], _ptr(deg_global),
        cap_nnz, cap_halo, _ptr(indptr), _ptr(indices), _ptr(values), _ptr(indptr_t),
        _ptr(indices_t), _ptr(values_t), _ptr(deg), _ptr(halo), ctypes.byref(nnz),
        ctypes.byref(n_halo), _ptr(ws), ws.numel(), _stream(dev))
    L.check("sag_csr_build_normalize", st)
    nnz, n_halo = nnz.value, n_halo.value
    n_ext = n_local + n_halo
    A = Csr(n_local, n_ext, indptr, indices[:nnz], values[:nnz], row_mean=(norm == "mean"))
    AT = None
    if transpose:
        AT = Csr(n_ext, n_local, indptr_t[:n_ext + 1], indices_t[:nnz], values_t[:nnz])
    return Built(A, AT, deg[:n_ext], halo[:n_halo])


# Long rows are cut into segments of seg_len entries, one wavefront each.
# Longer segments mean fewer fp32 partial rows and reduce steps, shorter ones
# a smaller last wavefront at the end of a launch.  Measured per product
# (2.45M-node graph 126M entries: 1024 -> 4096 saves 0.3 ms of the step's
# SpMMs; 100M-graph share 194M entries: 7.49 -> 7.26 ms; R-MAT partition
# 7.9M entries and the hub parts of the dense GCN graph, 2-42M entries each:
# 1024 best, 8192 up to 40% slower), so the length follows the entries a
# launch spreads over the chip's ~8,192 resident wavefronts: a quarter of
# each one's share, nnz / 32768, to the nearest power of two in [1024, 4096].
SEG_LEN_ENTRIES = 32768
SEG_LEN_MIN, SEG_LEN_MAX = 1024, 4096


def auto_seg_len(A: Csr) -> int:
    """The segment length csr_schedule uses for A when given none."""
    x = max(A.nnz, 1) / SEG_LEN_ENTRIES
    p = 1 << max(0, round(math.log2(x)))
    return min(max(p, SEG_LEN_MIN), SEG_LEN_MAX)


def csr_schedule(A: Csr, seg_len: int | None = None) -> Csr:
    """sag_csr_schedule: attach the degree-binned schedule to A (in place),
    with long rows cut into segments of seg_len entries (None:
    auto_seg_len(A)).  Synchronises the current stream."""
    if seg_len is None:
        seg_len = auto_seg_len(A)
    lib = L.lib()
    dev = A.device
    nb = lib.sag_csr_schedule_bytes(A.n_rows, A.nnz, seg_len)
    buf = torch.empty(max(int(nb), 16), dtype=torch.uint8, device=dev)
    ws = _ws(lib.sag_csr_schedule_workspace_bytes(A.n_rows), dev)
    st = lib.sag_csr_schedule(A.ref, seg_len, _ptr(buf), buf.numel(), _ptr(ws), ws.numel(), _stream(dev))
    L.check("sag_csr_schedule", st)
    A.sched = buf
    return A


# A hub split pays where rows hold many entries: the fp32 partial rows each
# pass writes and the next reads back then cost little next to the gathers
# they move into L2 (measured: 493 entries per row, products 35% faster over
# a chain of twelve 12,288-column groups; 51 entries per row, one 16,384-
# column group already 10% slower).  A group of 12,288 rows of X is 3-6 MB
# at the widths the workloads use, about one XCD's L2.  The chain goes on
# while the last group held at least 2% of the matrix's entries.
HUB_SPLIT_MIN_ENTRIES_PER_ROW = 128
HUB_COLS = 12288
HUB_MIN_SHARE = 0.02
HUB_MAX_LEVELS = 32


def hub_split_pays(A: Csr) -> bool:
    """Whether products over A gain from a hub split (the rule above)."""
    return A.n_rows > 0 and A.nnz >= HUB_SPLIT_MIN_ENTRIES_PER_ROW * A.n_rows and A.n_cols > 2 * HUB_COLS


def csr_hub_split(A: Csr, n_hub: int = HUB_COLS, seg_len: int | None = None, levels: int | None = None) -> Csr:
    """sag_csr_hub_split: split A's entries into those of the n_hub columns
    holding the most entries and the rest, schedule both parts (seg_len;
    None: each part's own auto_seg_len) and attach them to A (in
    place); then split the cold part the same way, and so on: `levels`
    times, or (None) while the last hub part held at least HUB_MIN_SHARE of
    A's entries (at most HUB_MAX_LEVELS).  Products over A take one pass per
    hub part plus one.  Synchronises the current stream."""
    if A.hub_part is not None:
        raise ValueError("the matrix already has a hub split")
    if levels is not None and levels < 1:
        raise ValueError("levels must be at least 1")
    M, k = A, 0
    while True:
        _split_once(M, n_hub, seg_len)
        k += 1
        if levels is not None:
            if k >= levels:
                break
        elif M.hub_part.nnz < HUB_MIN_SHARE * A.nnz or k >= HUB_MAX_LEVELS:
            break
        M = M.cold_part
        if M.nnz == 0:
            break
    return A


def hub_chain(A: Csr) -> list:
    """The entry counts of A's hub parts, first to last, and of its final
    cold part (empty when A has no split)."""
    out, M = [], A
    while M.hub_part is not None:
        out.append(M.hub_part.nnz)
        M = M.cold_part
    return out + [M.nnz] if out else []


def _split_once(A: Csr, n_hub: int, seg_len: int | None) -> None:
    lib = L.lib()
    dev = A.device
    cap = max(A.nnz, 1)
    parts = []
    bufs = []
    for _ in range(2):
        ip = torch.empty(A.n_rows + 1, dtype=torch.int64, device=dev)
        ix = torch.empty(cap, dtype=torch.int32, device=dev)
        vv = torch.empty(cap, dtype=torch.float32, device=dev) if A.values is not None else None
        bufs.append((ip, ix, vv))
    ws = _ws(lib.sag_csr_hub_split_workspace_bytes(A.n_rows, A.n_cols), dev)
    nh = ctypes.c_int64(0)
    (hp, hi, hv), (cp, ci, cv) = bufs
    st = lib.sag_csr_hub_split(A.ref, n_hub, cap, _ptr(hp), _ptr(hi), _ptr(hv), cap, _ptr(cp), _ptr(ci), _ptr(cv),
                               ctypes.byref(nh), _ptr(ws), ws.numel(), _stream(dev))
    L.check("sag_csr_hub_split", st)
    nh = nh.value
    for (ip, ix, vv), k in zip(bufs, (nh, A.nnz - nh)):
        # exact-size copies, so that the parts hold no spare capacity
        P = Csr(A.n_rows, A.n_cols, ip, ix[:k].clone(), vv[:k].clone() if vv is not None else None)
        csr_schedule(P, seg_len)
        parts.append(P)
    A.hub_part, A.cold_part = parts
    A.raw.hub_part = ctypes.addressof(parts[0].raw)
    A.raw.cold_part = ctypes.addressof(parts[1].raw)


COL_SLICE_BYTES = 128        # one cache line of each row of X per pass
COL_SLICE_MIN_ROW_BYTES = 257   # rows of at most two slices are gathered whole
COL_SLICE_MARGIN = 0.01     # slices are kept only when this much faster


def csr_set_col_slices(A: Csr, on: bool) -> Csr:
    """Set A's col_slices flag: products over A whose rows of X span more
    than 256 bytes run one pass per 128-byte column slice of X."""
    A.col_slices = bool(on)
    A.raw.col_slices = int(A.col_slices)
    return A


def col_slices_apply(A: Csr, d: int, dtype: torch.dtype) -> bool:
    """Whether a product of width d in dtype over A runs in column slices
    when A asks for them (no hub split, rows wider than two slices)."""
    es = torch.empty(0, dtype=dtype).element_size()
    return A.hub_part is None and d * es >= COL_SLICE_MIN_ROW_BYTES


def csr_tune_col_slices(A: Csr, d: int, dtype: torch.dtype, reps: int = 5,
                        margin: float = COL_SLICE_MARGIN) -> dict:
    """Time the product over A at width d both ways (random X, the library's
    own entry point, HIP events on the current stream, a warm round then
    `reps` rounds alternated, medians) and set A's col_slices when slices
    are faster by more than `margin`.  Whether slices pay depends on how much
    of the matrix its busiest columns carry, so it is measured on the matrix
    itself.  Returns {"on", "whole_ms", "sliced_ms"} (timings None where
    slices cannot apply)."""
    if not col_slices_apply(A, d, dtype) or A.nnz == 0:
        csr_set_col_slices(A, False)
        return {"on": False, "whole_ms": None, "sliced_ms": None}
    dev = A.device
    X = empty_dense(A.n_cols, d, dtype, dev)
    X.normal_()
    Y = empty_dense(A.n_rows, d, dtype, dev)
    times = {False: [], True: []}
    for r in range(reps + 1):
        for on in (False, True):
            csr_set_col_slices(A, on)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            spmm_csr(A, X, Y=Y)
            b.record()
            b.synchronize()
            if r > 0:   # the first round warms both
                times[on].append(a.elapsed_time(b))
    whole = sorted(times[False])[len(times[False]) // 2]
    sliced = sorted(times[True])[len(times[True]) // 2]
    on = sliced < (1.0 - margin) * whole
    csr_set_col_slices(A, on)
    return {"on": on, "whole_ms": whole, "sliced_ms": sliced}


def csr_info(A: Csr) -> dict:
    r = A.raw
    return {"n_short": r.n_short, "n_medium": r.n_medium, "n_long": r.n_long,
            "n_seg": r.n_seg, "seg_len": r.seg_len}


def halo_gather(src: torch.Tensor, rows: torch.Tensor, out: torch.Tensor, row_base: int = 0) -> torch.Tensor:
    """sag_halo_gather: out[k] = src[rows[k] - row_base] (bitwise).  The ids
    must lie in src's rows (the kernel does not check them)."""
    _need_rows("halo_gather out", out, rows.numel())
    rows = rows.to(torch.int32).contiguous()
    st = L.lib().sag_halo_gather(_ptr(src), _ld(src), _ptr(rows), row_base, rows.numel(), src.shape[1],
                                 dtype_code(src.dtype), _ptr(out), _ld(out) if out.shape[0] else src.shape[1],
                                 _stream(src.device))
    L.check("sag_halo_gather", st)
    return out


def halo_push(src: torch.Tensor, ids: torch.Tensor, dst: torch.Tensor, row_base: int = 0,
              accumulate: bool = False) -> torch.Tensor:
    """sag_halo_push: dst[ids[k] - row_base] = src[k] (or += for gradients);
    targets outside dst's rows are skipped."""
    _need_rows("halo_push src", src, ids.numel())
    ids = ids.to(torch.int32).contiguous()
    st = L.lib().sag_halo_push(_ptr(src), _ld(src), _ptr(ids), row_base, ids.numel(), src.shape[1],
                               dtype_code(src.dtype), int(bool(accumulate)), _ptr(dst), _ld(dst), dst.shape[0],
                               _stream(src.device))
    L.check("sag_halo_push", st)
    return dst


def code_row_bytes(d: int, bits: int) -> int:
    return int(L.lib().sag_code_row_bytes(d, bits))


def quantize_rows(src: torch.Tensor, bits: int, seed: int, epoch: int, rows: torch.Tensor | None = None,
                  nodes: torch.Tensor | None = None, n: int | None = None, out=None):
    """sag_quantize_rows: message row k = Sylvie's b-bit quantization of
    src[rows[k]] (rows None: src[k]) with stream id nodes[k] (None: k).
    Returns (codes uint8 [n, code_row_bytes], scale float32 [n], zero float32 [n])."""
    dev = src.device
    if rows is not None:
        rows = rows.to(torch.int32).contiguous()
        n = rows.numel()
    elif n is None:
        n = src.shape[0]
    if nodes is not None:
        nodes = nodes.to(torch.int32).contiguous()
        if nodes.numel() != n:
            raise ValueError("nodes must have one id per message row")
    d = src.shape[1]
    if out is None:
        codes = torch.empty((n, code_row_bytes(d, bits)), dtype=torch.uint8, device=dev)
        scale = torch.empty(n, dtype=torch.float32, device=dev)
        zero = torch.empty(n, dtype=torch.float32, device=dev)
    else:
        codes, scale, zero = out
    st = L.lib().sag_quantize_rows(_ptr(src), _ld(src), dtype_code(src.dtype), _ptr(rows),
                                   src.shape[0], _ptr(nodes), n, d, bits,
                                   seed & (2 ** 64 - 1), epoch & 0xFFFFFFFF, _ptr(codes), codes.stride(0),
                                   _ptr(scale), _ptr(zero), _stream(dev))
    L.check("sag_quantize_rows", st)
    return codes, scale, zero


def dequantize_rows(codes: torch.Tensor, scale: torch.Tensor, zero: torch.Tensor, d: int, bits: int,
                    dst: torch.Tensor, ids: torch.Tensor | None = None, row_base: int = 0,
                    accumulate: bool = False) -> torch.Tensor:
    """sag_dequantize_rows: dst[ids[k] - row_base] (ids None: dst[k]) =
    zero[k] + code * scale[k] (or += for gradients)."""
    if ids is not None:
        ids = ids.to(torch.int32).contiguous()
    st = L.lib().sag_dequantize_rows(_ptr(codes), codes.stride(0), _ptr(scale), _ptr(zero), codes.shape[0], d,
                                     bits, _ptr(ids), row_base,
                                     int(bool(accumulate)), dtype_code(dst.dtype), _ptr(dst), _ld(dst),
                                     dst.shape[0], _stream(codes.device))
    L.check("sag_dequantize_rows", st)
    return dst


def _spmm(name, A: Csr, X, out_dtype=None, Y=None, addend=None):
    _need_rows(f"{name} X", X, A.n_cols)
    _need_rows(f"{name} Y", Y, A.n_rows)
    lib = L.lib()
    d = X.shape[1]
    yt = out_dtype or X.dtype
    if Y is None:
        Y = empty_dense(A.n_rows, d, yt, X.device)
    n_add = addend.shape[0] if addend is not None else 0
    ws = _ws(lib.sag_spmm_workspace_bytes(A.ref, d), X.device)
    st = getattr(lib, name)(A.ref, _ptr(X), _ld(X), dtype_code(X.dtype), d, _ptr(Y), _ld(Y),
                            dtype_code(Y.dtype), _ptr(addend),
                            _ld(addend) if addend is not None else 0, n_add,
                            _ptr(ws), ws.numel(), _stream(X.device))
    L.check(name, st)
    return Y


def spmm_csr(A: Csr, X, out_dtype=None, Y=None, addend=None):
    """sag_spmm_csr: Y = A X (+ addend on its first rows)."""
    return _spmm("sag_spmm_csr", A, X, out_dtype, Y, addend)


def spmm_csr_t(AT: Csr, X, out_dtype=None, Y=None, addend=None):
    """sag_spmm_csr_t: the same product over a transposed CSR."""
    return _spmm("sag_spmm_csr_t", AT, X, out_dtype, Y, addend)


def spmm_csr_noalloc(A: Csr, X, Y, addend=None):
    """sag_spmm_csr_noalloc: Y = A X (+ addend) into the caller's Y, with
    the long rows' partials in the library's fixed device scratch (no
    workspace; nothing allocated by the call)."""
    _need_rows("spmm_csr_noalloc X", X, A.n_cols)
    _need_rows("spmm_csr_noalloc Y", Y, A.n_rows)
    n_add = addend.shape[0] if addend is not None else 0
    st = L.lib().sag_spmm_csr_noalloc(A.ref, _ptr(X), _ld(X), dtype_code(X.dtype), X.shape[1], _ptr(Y), _ld(Y),
                                      dtype_code(Y.dtype), _ptr(addend), _ld(addend) if addend is not None else 0,
                                      n_add, _stream(X.device))
    L.check("sag_spmm_csr_noalloc", st)
    return Y


def spmm_noalloc_scratch_bytes() -> int:
    return int(L.lib().sag_spmm_noalloc_scratch_bytes())


# ---- layers ------------------------------------------------------------------------

@dataclass
class LayerCtx:
    """What a layer's forward hands to its backward."""
    kind: str
    save: torch.Tensor
    H_ext: torch.Tensor
    W: torch.Tensor
    d_in: int
    d_out: int
    relu: bool


def _layer_forward(kind, A: Csr, H_ext, W, b, relu, want_pre, Out=None, Y_pre=None, ws=None, fused=False):
    _need_rows(f"{kind}_layer_forward H_ext (local + halo rows)", H_ext, A.n_cols)
    _need_rows(f"{kind}_layer_forward W", W, (2 if kind == "sage" else 1) * H_ext.shape[1])
    _need_rows(f"{kind}_layer_forward Out", Out, A.n_rows)
    _need_rows(f"{kind}_layer_forward Y_pre", Y_pre, A.n_rows)
    lib = L.lib()
    dt = dtype_code(H_ext.dtype)
    d_in = H_ext.shape[1]
    d_out = W.shape[1]
    dev = H_ext.device
    W = W.contiguous()
    if Out is None:
        Out = empty_dense(A.n_rows, d_out, H_ext.dtype, dev)
    if want_pre and Y_pre is None:
        Y_pre = empty_dense(A.n_rows, d_out, H_ext.dtype, dev)
    if want_pre and _ld(Y_pre) != _ld(Out):
        raise ValueError("Y_pre and Out must share their leading dimension")
    save_bytes = getattr(lib, f"sag_{kind}_save_bytes")(A.n_rows, d_in, d_out, dt)
    save = _ws(save_bytes, dev)
    nws = getattr(lib, f"sag_{kind}_forward_workspace_bytes")(A.ref, d_in, d_out, dt)
    if ws is None or ws.numel() < nws:
        ws = _ws(nws, dev)
    st = getattr(lib, f"sag_{kind}_layer_forward")(
        A.ref, _ptr(H_ext), _ld(H_ext), d_in, _ptr(W), _ptr(b), d_out, int(relu),
        L.SAG_LAYER_FUSED if fused else 0, dt, _ptr(Y_pre) if want_pre else None, _ptr(Out), _ld(Out), _ptr(save), save.numel(),
        _ptr(ws), ws.numel(), _stream(dev))
    L.check(f"sag_{kind}_layer_forward", st)
    ctx = LayerCtx(kind, save, H_ext, W, d_in, d_out, bool(relu))
    return Out, Y_pre, ctx


def _layer_backward(ctx: LayerCtx, AT: Csr | None, n_local: int, Y, G_out, want_dH=True,
                    want_db=True, dH=None, ws=None):
    _need_rows(f"{ctx.kind}_layer_backward G_out", G_out, n_local)
    if ctx.relu:
        _need_rows(f"{ctx.kind}_layer_backward Y", Y, n_local)
    if AT is not None:
        _need_rows(f"{ctx.kind}_layer_backward H_ext", ctx.H_ext, AT.n_rows)
        if want_dH:
            _need_rows(f"{ctx.kind}_layer_backward dH", dH, AT.n_rows)
    lib = L.lib()
    kind = ctx.kind
    dt = dtype_code(G_out.dtype)
    dev = G_out.device
    w_rows = ctx.W.shape[0]
    dW = torch.empty((w_rows, ctx.d_out), dtype=torch.float32, device=dev)
    db = torch.empty(ctx.d_out, dtype=torch.float32, device=dev) if want_db else None
    if want_dH and dH is None:
        dH = empty_dense(AT.n_rows, ctx.d_in, G_out.dtype, dev)
    if not want_dH:
        dH = None
    if ctx.relu and _ld(Y) != _ld(G_out):
        raise ValueError("Y and G_out must share their leading dimension")
    nws = getattr(lib, f"sag_{kind}_backward_workspace_bytes")(
        AT.ref if AT is not None else None, n_local, ctx.d_in, ctx.d_out, dt)
    if ws is None or ws.numel() < nws:
        ws = _ws(nws, dev)
    st = getattr(lib, f"sag_{kind}_layer_backward")(
        AT.ref if AT is not None else None, n_local, _ptr(ctx.H_ext), _ld(ctx.H_ext), ctx.d_in,
        _ptr(ctx.W), ctx.d_out, int(ctx.relu), _ptr(Y) if ctx.relu else None, _ptr(G_out),
        _ld(G_out), _ptr(dW), _ptr(db), _ptr(dH), _ld(dH) if dH is not None else 0, dt,
        _ptr(ctx.save), ctx.save.numel(), _ptr(ws), ws.numel(), _stream(dev))
    L.check(f"sag_{kind}_layer_backward", st)
    return dW, db, dH


def gcn_layer_forward(A: Csr, H_ext, W, b=None, relu=True, want_pre=False, **kw):
    """sag_gcn_layer_forward: Out = relu(A H_ext W + b).  Returns (Out, Y_pre, ctx).
    fused=True passes SAG_LAYER_FUSED (the fused aggregate -> transform
    kernel where it applies)."""
    return _layer_forward("gcn", A, H_ext, W, b, relu, want_pre, **kw)


def gcn_layer_backward(ctx, AT, n_local, Y, G_out, want_dH=True, want_db=True, **kw):
    """sag_gcn_layer_backward: returns (dW, db, dH_ext)."""
    return _layer_backward(ctx, AT, n_local, Y, G_out, want_dH, want_db, **kw)


def sage_layer_forward(A: Csr, H_ext, W, b=None, relu=True, want_pre=False, **kw):
    """sag_sage_layer_forward: Out = relu([H_local | A_mean H_ext] W + b)."""
    return _layer_forward("sage", A, H_ext, W, b, relu, want_pre, **kw)


def sage_layer_backward(ctx, AT, n_local, Y, G_out, want_dH=True, want_db=True, **kw):
    """sag_sage_layer_backward: returns (dW, db, dH_ext)."""
    return _layer_backward(ctx, AT, n_local, Y, G_out, want_dH, want_db, **kw)


def aggregate_transform(A: Csr, H_ext, W, b=None, self_rows=False, relu=True, want_pre=False, want_z=True,
                        Out=None, Z=None, ws=None):
    """sag_aggregate_transform: Out = act(Z W + b) or act([H_local | Z] W + b)
    with Z = A H_ext summed and multiplied in one kernel.  Returns
    (Out, Y_pre, Z)."""
    _need_rows("aggregate_transform H_ext (local + halo rows)", H_ext, A.n_cols)
    _need_rows("aggregate_transform Out", Out, A.n_rows)
    _need_rows("aggregate_transform Z", Z, A.n_rows)
    lib = L.lib()
    dt = dtype_code(H_ext.dtype)
    d_in = H_ext.shape[1]
    d_out = W.shape[1]
    dev = H_ext.device
    W = W.contiguous()
    if Out is None:
        Out = empty_dense(A.n_rows, d_out, H_ext.dtype, dev)
    Y_pre = empty_dense(A.n_rows, d_out, H_ext.dtype, dev) if want_pre else None
    if want_pre and _ld(Y_pre) != _ld(Out):
        raise ValueError("Y_pre and Out must share their leading dimension")
    if want_z and Z is None:
        Z = empty_dense(A.n_rows, d_in, H_ext.dtype, dev)
    if not want_z:
        Z = None
    nws = lib.sag_aggregate_transform_workspace_bytes(A.ref, d_in, d_out, int(bool(self_rows)), dt)
    if ws is None or ws.numel() < nws:
        ws = _ws(nws, dev)
    st = lib.sag_aggregate_transform(A.ref, _ptr(H_ext), _ld(H_ext), d_in, _ptr(W), _ptr(b), d_out,
                                     int(bool(self_rows)), int(relu), dt, _ptr(Y_pre), _ptr(Out), _ld(Out),
                                     _ptr(Z), _ld(Z) if Z is not None else 0, _ptr(ws), ws.numel(),
                                     _stream(dev))
    L.check("sag_aggregate_transform", st)
    return Out, Y_pre, Z


@dataclass
class GatCtx:
    """What the GAT forward hands to its backward."""
    save: torch.Tensor
    H_ext: torch.Tensor
    W: torch.Tensor
    a_src: torch.Tensor
    a_dst: torch.Tensor
    heads: int
    d_head: int
    slope: float
    relu: bool


def gat_layer_forward(A: Csr, H_ext, W, a_src, a_dst, b=None, heads=1, slope=0.2, relu=True,
                      Out=None, ws=None):
    """sag_gat_layer_forward: Out = act(concat_k sum_u alpha^k_vu (H_ext W)_k[u] + b).
    W [d_in, heads * d_head]; a_src, a_dst fp32 [heads, d_head].  Returns (Out, ctx)."""
    _need_rows("gat_layer_forward H_ext (local + halo rows)", H_ext, A.n_cols)
    _need_rows("gat_layer_forward Out", Out, A.n_rows)
    lib = L.lib()
    dt = dtype_code(H_ext.dtype)
    d_in = H_ext.shape[1]
    F = W.shape[1]
    if F % heads:
        raise ValueError("W's width must be heads * d_head")
    d_head = F // heads
    dev = H_ext.device
    W = W.contiguous()
    a_src = a_src.to(torch.float32).contiguous()
    a_dst = a_dst.to(torch.float32).contiguous()
    if Out is None:
        Out = empty_dense(A.n_rows, F, H_ext.dtype, dev)
    save = _ws(lib.sag_gat_save_bytes(A.n_rows, A.n_cols, heads, d_head, dt), dev)
    nws = lib.sag_gat_forward_workspace_bytes(A.ref, d_in, heads, d_head, dt)
    if ws is None or ws.numel() < nws:
        ws = _ws(nws, dev)
    st = lib.sag_gat_layer_forward(A.ref, _ptr(H_ext), _ld(H_ext), d_in, _ptr(W), _ptr(a_src), _ptr(a_dst),
                                   _ptr(b), heads, d_head, float(slope), int(relu), dt, _ptr(Out), _ld(Out),
                                   _ptr(save), save.numel(), _ptr(ws), ws.numel(), _stream(dev))
    L.check("sag_gat_layer_forward", st)
    return Out, GatCtx(save, H_ext, W, a_src, a_dst, heads, d_head, float(slope), bool(relu))


def gat_layer_backward(ctx: GatCtx, A: Csr, AT: Csr, Y, G_out, want_dH=True, dH=None, ws=None):
    """sag_gat_layer_backward: returns (dW, da_src, da_dst, db, dH_ext)."""
    _need_rows("gat_layer_backward G_out", G_out, A.n_rows)
    if ctx.relu:
        _need_rows("gat_layer_backward Y", Y, A.n_rows)
    if want_dH:
        _need_rows("gat_layer_backward dH", dH, AT.n_rows)
    lib = L.lib()
    dt = dtype_code(G_out.dtype)
    dev = G_out.device
    d_in = ctx.H_ext.shape[1]
    F = ctx.heads * ctx.d_head
    dW = torch.empty((d_in, F), dtype=torch.float32, device=dev)
    da_src = torch.empty((ctx.heads, ctx.d_head), dtype=torch.float32, device=dev)
    da_dst = torch.empty((ctx.heads, ctx.d_head), dtype=torch.float32, device=dev)
    db = torch.empty(F, dtype=torch.float32, device=dev)
    if want_dH and dH is None:
        dH = empty_dense(A.n_cols, d_in, G_out.dtype, dev)
    if not want_dH:
        dH = None
    if ctx.relu and _ld(Y) != _ld(G_out):
        raise ValueError("Y and G_out must share their leading dimension")
    nws = lib.sag_gat_backward_workspace_bytes(A.ref, AT.ref, d_in, ctx.heads, ctx.d_head, dt)
    if ws is None or ws.numel() < nws:
        ws = _ws(nws, dev)
    st = lib.sag_gat_layer_backward(
        A.ref, AT.ref, _ptr(ctx.H_ext), _ld(ctx.H_ext), d_in, _ptr(ctx.W), _ptr(ctx.a_src), _ptr(ctx.a_dst),
        ctx.heads, ctx.d_head, ctx.slope, int(ctx.relu), _ptr(Y) if ctx.relu else None, _ptr(G_out),
        _ld(G_out), _ptr(dW), _ptr(da_src), _ptr(da_dst), _ptr(db), _ptr(dH), _ld(dH) if dH is not None else 0,
        dt, _ptr(ctx.save), ctx.save.numel(), _ptr(ws), ws.numel(), _stream(dev))
    L.check("sag_gat_layer_backward", st)
    return dW, da_src, da_dst, db, dH


# ---- dense building blocks ------------------------------------------------------------

def gemm(A1, B, A2=None, mask=None, trans_b=False, bias=None, addend=None, relu=False,
         want_pre=False):
    """sag_gemm: C = [A1 | A2] B (+ bias) (+ addend), optional ReLU."""
    M = A1.shape[0]
    _need_rows("gemm A2", A2, M)
    _need_rows("gemm mask", mask, M)
    _need_rows("gemm B (rows = K)" if not trans_b else "gemm B (transposed: rows = N)", B,
               0 if trans_b else A1.shape[1] + (A2.shape[1] if A2 is not None else 0))
    _need_rows("gemm addend", addend, M)
    _need_rows("gemm bias", bias, B.shape[0] if trans_b else B.shape[1])
    lib = L.lib()
    dt = dtype_code(A1.dtype)
    M = A1.shape[0]
    K1 = A1.shape[1]
    K2 = A2.shape[1] if A2 is not None else 0
    B = B.contiguous()
    N = B.shape[0] if trans_b else B.shape[1]
    C = empty_dense(M, N, A1.dtype, A1.device)
    pre = empty_dense(M, N, A1.dtype, A1.device) if want_pre else None
    if pre is not None and _ld(pre) != _ld(C):
        raise AssertionError
    ws = _ws(lib.sag_gemm_workspace_bytes(M, K1 + K2, N, dt), A1.device)
    st = lib.sag_gemm(M, N, _ptr(A1), _ld(A1), K1, _ptr(A2), _ld(A2) if A2 is not None else 0, K2,
                      _ptr(mask), _ld(mask) if mask is not None else 0, _ptr(B), B.stride(0),
                      int(trans_b), _ptr(bias), _ptr(addend), _ld(addend) if addend is not None else 0,
                      int(relu), _ptr(C), _ptr(pre), _ld(C), dt, _ptr(ws), ws.numel(),
                      _stream(A1.device))
    L.check("sag_gemm", st)
    return (C, pre) if want_pre else C


def gemm_tn(A1, B, A2=None, mask=None, want_colsum=True):
    """sag_gemm_tn: C = [A1 | A2]^T (B * 1[mask > 0]) in fp32, and column sums."""
    M = A1.shape[0]
    _need_rows("gemm_tn A2", A2, M)
    _need_rows("gemm_tn B", B, M)
    _need_rows("gemm_tn mask", mask, M)
    lib = L.lib()
    dt = dtype_code(A1.dtype)
    M, K1 = A1.shape
    K2 = A2.shape[1] if A2 is not None else 0
    N = B.shape[1]
    C = torch.empty((K1 + K2, N), dtype=torch.float32, device=A1.device)
    cs = torch.empty(N, dtype=torch.float32, device=A1.device) if want_colsum else None
    ws = _ws(lib.sag_gemm_tn_workspace_bytes(M, K1 + K2, N, dt), A1.device)
    st = lib.sag_gemm_tn(M, N, _ptr(A1), _ld(A1), K1, _ptr(A2), _ld(A2) if A2 is not None else 0, K2,
                         _ptr(B), _ld(B), _ptr(mask), _ld(mask) if mask is not None else 0, _ptr(C),
                         N, _ptr(cs), dt, _ptr(ws), ws.numel(), _stream(A1.device))
    L.check("sag_gemm_tn", st)
    return (C, cs) if want_colsum else C


def trace_enable(on: bool = True) -> None:
    """sag_trace_enable: HIP-event timing of every internal operation."""
    L.check("sag_trace_enable", L.lib().sag_trace_enable(int(on)))


def trace_records(clear: bool = True) -> list:
    """All trace records as dicts {name, ms, bytes, flops} (synchronises)."""
    lib = L.lib()
    out = []
    buf = ctypes.create_string_buffer(256)
    ms, nb, nf = ctypes.c_float(), ctypes.c_int64(), ctypes.c_int64()
    for i in range(lib.sag_trace_count()):
        L.check("sag_trace_get", lib.sag_trace_get(i, buf, 256, ctypes.byref(ms), ctypes.byref(nb),
                                                   ctypes.byref(nf)))
        out.append({"name": buf.value.decode(), "ms": ms.value, "bytes": nb.value, "flops": nf.value})
    if clear:
        lib.sag_trace_clear()
    return out


def gather_probe(X: torch.Tensor, ids: torch.Tensor, sink: torch.Tensor | None = None) -> torch.Tensor:
    """sag_gather_probe: read rows ids of X (in order, the SpMM's lane layout)
    and fold them into the returned sink (uint8 bytes; viewed as int32 words,
    word k of the sum over its 16-byte entries is the wrapping sum of word k
    of every vector read).  A measurement helper: it times the row gather of
    an SpMM over the same ids without the product around it."""
    ids = ids.to(torch.int32).contiguous()
    lib = L.lib()
    if sink is None:
        sink = torch.empty(int(lib.sag_gather_probe_sink_bytes()), dtype=torch.uint8, device=X.device)
    st = lib.sag_gather_probe(_ptr(X), _ld(X), X.shape[1], dtype_code(X.dtype), _ptr(ids), ids.numel(),
                              _ptr(sink), sink.numel(), _stream(X.device))
    L.check("sag_gather_probe", st)
    return sink


def version() -> str:
    return L.lib().sag_version().decode()
