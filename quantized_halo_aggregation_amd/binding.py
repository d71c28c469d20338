"""Thin ctypes binding of libqha (include/qha.h): argument marshalling only.

Each function takes torch tensors that live on the GPU (or numpy arrays for the host helpers),
checks dtype / device / layout, passes raw pointers to the C entry point of the same name and
raises on a non-OK status.  All arithmetic happens in the HIP kernels behind the C ABI; there is
no fallback path -- importing this module fails loudly if libqha.so has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# QHA_LIB may name another build of the library (same ABI), e.g. one installed elsewhere
LIB_PATH = os.environ.get("QHA_LIB") or os.path.join(_HERE, "libqha.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m quantized_halo_aggregation_amd.build` "
                      "(or __graft_entry__.build()); there is no CPU fallback")

# libqha and torch must share one HIP runtime: torch ships its own libamdhip64 with the same soname,
# so torch is loaded first and libqha's dependency then resolves to the runtime already in the process.
import torch  # noqa: E402,F401

_lib = C.CDLL(LIB_PATH)


def _hip_runtimes():
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


if len(_hip_runtimes()) > 1:
    raise ImportError(f"two HIP runtimes are loaded in this process ({_hip_runtimes()}); import torch before "
                      "loading libqha so that both use the same one")

QHA_OK, QHA_ERR_INVALID_ARG, QHA_ERR_UNSUPPORTED, QHA_ERR_HIP, QHA_ERR_WORKSPACE = range(5)
NORM_GCN, NORM_MEAN = 0, 1
PRO_NONE, PRO_RELU_MASK = 0, 1
EPI_NONE, EPI_RELU = 0, 1
DEFAULT_CHUNK = 512
DEFAULT_GROUP_EDGES = 256
GROUP_ROWS = 15

_i32, _i64, _u32, _u64, _sz, _vp = C.c_int32, C.c_int64, C.c_uint32, C.c_uint64, C.c_size_t, C.c_void_p


class AggPlanStruct(C.Structure):
    _fields_ = [("n_rows", _i64), ("chunk", _i32), ("group_edges", _i32), ("skip_empty", _i32),
                ("reserved", _i32), ("n_items", _i64), ("n_split_items", _i64), ("n_split_rows", _i64),
                ("items", _vp), ("split_row", _vp), ("split_ptr", _vp)]


MAX_CLASSES = 8


class WidthClassesStruct(C.Structure):
    _fields_ = [("n", _i32), ("bits", _i32 * MAX_CLASSES), ("start", _i32 * (MAX_CLASSES + 1)),
                ("base", _u32 * MAX_CLASSES)]


class ReceivedStruct(C.Structure):
    _fields_ = [("copy_ptr", _vp), ("copy_idx", _vp), ("n_rows", _i64), ("codes", _vp), ("meta", _vp), ("bits", _vp),
                ("word_offset", _vp), ("classes", C.POINTER(WidthClassesStruct))]


MAX_LEVELS = 8
LDR_MAX_DELTA = 64


class CoordinatorStruct(C.Structure):
    _fields_ = [("lambda_", C.c_double), ("sign", C.c_double), ("f_prev", C.c_double), ("last_ldr", C.c_double),
                ("ldr", C.c_double * (LDR_MAX_DELTA + 1)), ("t", _i64), ("delta", _i32), ("b_min", _i32),
                ("b_max", _i32), ("bits", _i32), ("sync", _i32)]


def _sig(name, res, *args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_P = C.POINTER
_abi_version = _sig("qha_abi_version", _i32)
_status_string = _sig("qha_status_string", C.c_char_p, _i32)
_last_error = _sig("qha_last_error", C.c_char_p)
_pack_layout = _sig("qha_pack_layout", _i32, _vp, _i64, _i32, _vp, _P(_u64))
_pack_classes = _sig("qha_pack_classes", _i32, _vp, _i64, _i32, _P(WidthClassesStruct))
_mask_levels = _sig("qha_mask_levels", _i32, _vp, _i64, _i32, _vp, _vp)
_node_bits = _sig("qha_node_bits", _i32, _vp, _i64, _i32, _i32, _vp)
_level_order = _sig("qha_level_order", _i32, _vp, _i64, _vp)
_coord_init = _sig("qha_coordinator_init", _i32, _P(CoordinatorStruct), C.c_double, _i32, _i32, _i32, _i32)
_coord_step = _sig("qha_coordinator_step", _i32, _P(CoordinatorStruct), _vp, _i32, C.c_double, _P(_i32), _P(_i32))
_edge_weights = _sig("qha_edge_weights", _i32, _i64, _vp, _vp, _vp, _vp, _vp, _vp)
_validate_csr = _sig("qha_validate_csr", _i32, _i64, _i64, _vp, _vp, _i32)
_csr_transpose = _sig("qha_csr_transpose", _i32, _i64, _i64, _vp, _vp, _vp, _vp)
_plan_size = _sig("qha_agg_plan_size", _i32, _i64, _vp, _i32, _i32, _i32, _P(AggPlanStruct))
_plan_fill = _sig("qha_agg_plan_fill", _i32, _vp, _P(AggPlanStruct), _vp, _vp, _vp)
_plan_ws = _sig("qha_agg_workspace_bytes", _sz, _P(AggPlanStruct), _i32)
_degree_norm = _sig("qha_degree_norm", _i32, _vp, _i64, _i32, _vp, _vp)
_quantize_pack = _sig("qha_quantize_pack", _i32, _vp, _i64, _vp, _i64, _i32, _vp, _vp, _P(WidthClassesStruct), _u64,
                      _u32, _u32, _u32, _vp, _vp, _vp)
_dequant_aggregate_fwd = _sig("qha_dequant_aggregate_fwd", _i32, _i64, _vp, _vp, _vp, _vp, _P(AggPlanStruct), _vp,
                              _i64, _i64, _vp, _vp, _vp, _P(WidthClassesStruct), _vp, _i64, _i32, _i32, _vp, _i64, _vp,
                              _sz, _vp)
_dequant_aggregate_fwd_noalloc = _sig("qha_dequant_aggregate_fwd_noalloc", _i32, _i64, _vp, _vp, _vp, _vp,
                                      _P(AggPlanStruct), _vp, _i64, _i64, _vp, _vp, _vp, _P(WidthClassesStruct), _vp,
                                      _i64, _i32, _i32, _vp, _i64, _vp)
_aggregate_bwd = _sig("qha_aggregate_bwd", _i32, _i64, _vp, _vp, _vp, _P(AggPlanStruct), _vp, _i64, _i64, _i32, _i32,
                      _vp, _i64, _vp, _sz, _vp)
_aggregate_bwd_quantize = _sig("qha_aggregate_bwd_quantize", _i32, _i64, _vp, _vp, _vp, _P(AggPlanStruct), _vp, _i64,
                               _i64, _i32, _i64, _i32, _vp, _i64, _vp, _vp, _P(WidthClassesStruct), _u64, _u32, _u32,
                               _u32, _vp, _vp, _P(ReceivedStruct), _vp, _sz, _vp)
_dense_project = _sig("qha_dense_project", _i32, _i32, _i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _i32, _vp,
                      _i64, _i32, _vp, _i64, _i32, _vp, _sz, _vp)
_dense_ws = _sig("qha_dense_project_workspace", _sz, _i32, _i32, _i64, _i64, _i64)
_dense_bwd = _sig("qha_dense_backward", _i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                  _vp, _i64, _vp, _sz, _vp)
_dense_bwd_ws = _sig("qha_dense_backward_workspace", _sz, _i64, _i64, _i64)

EXPORTED = ["qha_abi_version", "qha_status_string", "qha_last_error", "qha_pack_layout", "qha_pack_classes",
            "qha_edge_weights", "qha_validate_csr",
            "qha_csr_transpose", "qha_agg_plan_size", "qha_agg_plan_fill", "qha_agg_workspace_bytes",
            "qha_degree_norm", "qha_quantize_pack", "qha_dequant_aggregate_fwd", "qha_dequant_aggregate_fwd_noalloc",
            "qha_aggregate_bwd",
            "qha_aggregate_bwd_quantize", "qha_dense_project", "qha_dense_project_workspace", "qha_dense_backward",
            "qha_dense_backward_workspace", "qha_mask_levels", "qha_node_bits", "qha_level_order",
            "qha_coordinator_init", "qha_coordinator_step"]


class QhaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _last_error().decode(errors="replace")
        super().__init__(f"{where}: {_status_string(status).decode()} ({msg})")


def _check(status: int, where: str):
    if status != QHA_OK:
        if status in (QHA_ERR_INVALID_ARG, QHA_ERR_UNSUPPORTED, QHA_ERR_WORKSPACE):
            raise ValueError(str(QhaError(status, where)))
        raise QhaError(status, where)


def abi_version() -> int:
    return int(_abi_version())


# ------------------------------------------------------------------------------------------------
# pointer helpers
# ------------------------------------------------------------------------------------------------

def _dev(t, dtype, name, allow_none=False):
    """Device pointer of a torch tensor after dtype / device checks (None -> NULL if allowed)."""
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} must not be None")
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    return t.data_ptr()


def _dev32(t, name):
    """Pointer of a 32-bit word array (int32 or uint32 tensor, reinterpreted as uint32)."""
    import torch
    if t is None or t.dtype not in (torch.int32, getattr(torch, "uint32", torch.int32)):
        raise TypeError(f"{name} must be an int32/uint32 tensor")
    return _dev(t, t.dtype, name)


def _rows(t, name):
    """(pointer, leading dimension) of a float32 matrix whose rows may be strided."""
    import torch
    if t is None:
        return None, 0
    _dev(t, torch.float32, name)
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with contiguous rows")
    return t.data_ptr(), t.stride(0)


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return int(stream)


def _host(a, dtype, name):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


# ------------------------------------------------------------------------------------------------
# host-side set-up helpers
# ------------------------------------------------------------------------------------------------

def pack_layout(bits, d: int):
    """Word offsets (uint32 [n+1]) and total words of a packed message buffer."""
    bits, pb = _host(bits, np.uint8, "bits")
    off = np.empty(bits.size + 1, dtype=np.uint32)
    total = _u64(0)
    _check(_pack_layout(pb, bits.size, int(d), off.ctypes.data, C.byref(total)), "qha_pack_layout")
    return off, int(total.value)


def pack_classes(bits, d: int):
    """Width classes of a width-grouped row order, or None if the rows form too many runs."""
    bits, pb = _host(bits, np.uint8, "bits")
    st = WidthClassesStruct()
    status = _pack_classes(pb, bits.size, int(d), C.byref(st))
    if status == QHA_ERR_UNSUPPORTED and bits.size > 0:
        return None
    _check(status, "qha_pack_classes")
    return st


def mask_levels(deg, n_levels: int = 4):
    """Graph Extractor: (levels uint8, importance float64) of a boundary pool's global degrees."""
    deg, pd = _host(deg, np.int32, "deg")
    level = np.empty(deg.size, np.uint8)
    imp = np.empty(deg.size, np.float64)
    _check(_mask_levels(pd, deg.size, int(n_levels), level.ctypes.data, imp.ctypes.data), "qha_mask_levels")
    return level, imp


def node_bits(level, base_bits: int, max_bits: int = 8):
    """Quant Orchestrator: the epoch's per-node widths (uint8)."""
    level, pl = _host(level, np.uint8, "level")
    bits = np.empty(level.size, np.uint8)
    _check(_node_bits(pl, level.size, int(base_bits), int(max_bits), bits.ctypes.data), "qha_node_bits")
    return bits


def level_order(level):
    level, pl = _host(level, np.uint8, "level")
    order = np.empty(level.size, np.int32)
    _check(_level_order(pl, level.size, order.ctypes.data), "qha_level_order")
    return order


class Coordinator:
    """The base width and execution mode per epoch (guide section 8); state lives in the C struct."""

    def __init__(self, lam: float = 0.9, delta: int = 5, b_min: int = 1, b_max: int = 8,
                 descent_magnitude: bool = False):
        self.state = CoordinatorStruct()
        _check(_coord_init(C.byref(self.state), float(lam), int(delta), int(b_min), int(b_max),
                           int(bool(descent_magnitude))), "qha_coordinator_init")

    def step(self, partition_losses, epoch_time: float):
        losses = np.ascontiguousarray(partition_losses, dtype=np.float64)
        bits, sync = _i32(), _i32()
        _check(_coord_step(C.byref(self.state), losses.ctypes.data, losses.size, float(epoch_time), C.byref(bits),
                           C.byref(sync)), "qha_coordinator_step")
        return int(bits.value), bool(sync.value)


def validate_csr(rowptr, colidx, n_cols: int, require_sorted: bool = True):
    rowptr, pr = _host(rowptr, np.int32, "rowptr")
    colidx, pc = _host(colidx, np.int32, "colidx")
    _check(_validate_csr(rowptr.size - 1, int(n_cols), pr, pc, int(require_sorted)), "qha_validate_csr")


def csr_transpose(rowptr, colidx, n_cols: int):
    rowptr, pr = _host(rowptr, np.int32, "rowptr")
    colidx, pc = _host(colidx, np.int32, "colidx")
    colptr = np.empty(int(n_cols) + 1, dtype=np.int32)
    rowidx = np.empty(colidx.size, dtype=np.int32)
    _check(_csr_transpose(rowptr.size - 1, int(n_cols), pr, pc, colptr.ctypes.data, rowidx.ctypes.data),
           "qha_csr_transpose")
    return colptr, rowidx


def plan_items(rowptr, chunk: int = DEFAULT_CHUNK, group_edges: int = DEFAULT_GROUP_EDGES,
               skip_empty: bool = False) -> int:
    """The number of work items qha_agg_plan_size gives for this CSR (host only)."""
    rowptr, pr = _host(rowptr, np.int32, "rowptr")
    st = AggPlanStruct()
    _check(_plan_size(rowptr.size - 1, pr, int(chunk), int(group_edges), int(skip_empty), C.byref(st)),
           "qha_agg_plan_size")
    return int(st.n_items)


class AggPlan:
    """A work plan for one CSR (host arrays built by the library, kept on the device)."""

    def __init__(self, rowptr, chunk: int = DEFAULT_CHUNK, group_edges: int = DEFAULT_GROUP_EDGES,
                 skip_empty: bool = False, device="cuda"):
        import torch
        rowptr, pr = _host(rowptr, np.int32, "rowptr")
        st = AggPlanStruct()
        _check(_plan_size(rowptr.size - 1, pr, int(chunk), int(group_edges), int(skip_empty), C.byref(st)),
               "qha_agg_plan_size")
        items = np.zeros(4 * max(st.n_items, 1), np.int32)
        split_row = np.zeros(max(st.n_split_rows, 1), np.int32)
        split_ptr = np.zeros(st.n_split_rows + 1, np.int32)
        _check(_plan_fill(pr, C.byref(st), items.ctypes.data, split_row.ctypes.data, split_ptr.ctypes.data),
               "qha_agg_plan_fill")
        self.host = {"items": items[:4 * st.n_items].reshape(-1, 4), "split_row": split_row[:st.n_split_rows],
                     "split_ptr": split_ptr}
        self.dev = {"items": torch.from_numpy(items).to(device), "split_row": torch.from_numpy(split_row).to(device),
                    "split_ptr": torch.from_numpy(split_ptr).to(device)}
        st.items = self.dev["items"].data_ptr()
        st.split_row = self.dev["split_row"].data_ptr()
        st.split_ptr = self.dev["split_ptr"].data_ptr()
        self.struct = st

    @property
    def n_items(self):
        return int(self.struct.n_items)

    @property
    def n_split_rows(self):
        return int(self.struct.n_split_rows)

    def workspace_bytes(self, d: int) -> int:
        return int(_plan_ws(C.byref(self.struct), int(d)))


def _plan_ref(plan):
    return None if plan is None else C.byref(plan.struct)


def _cls_ref(classes):
    return None if classes is None else C.byref(classes)


def dense_project_workspace(trans_a: int, trans_b: int, m: int, n: int, k: int) -> int:
    return int(_dense_ws(int(trans_a), int(trans_b), int(m), int(n), int(k)))


def dense_backward_workspace(m: int, n: int, k: int) -> int:
    return int(_dense_bwd_ws(int(m), int(n), int(k)))


# ------------------------------------------------------------------------------------------------
# device entry points
# ------------------------------------------------------------------------------------------------

def degree_norm(deg, kind: int, out, stream=None):
    import torch
    _check(_degree_norm(_dev(deg, torch.int32, "deg"), deg.numel(), int(kind), _dev(out, torch.float32, "out"),
                        _stream(stream)), "qha_degree_norm")


def edge_weights(rowptr, colidx, r, c, w, stream=None):
    import torch
    _check(_edge_weights(rowptr.numel() - 1, _dev(rowptr, torch.int32, "rowptr"), _dev(colidx, torch.int32, "colidx"),
                         _dev(r, torch.float32, "r", allow_none=True), _dev(c, torch.float32, "c", allow_none=True),
                         _dev(w, torch.float32, "w"), _stream(stream)), "qha_edge_weights")


def quantize_pack(x, row_index, n_rows: int, bits, word_offset, classes, seed: int, epoch: int, stream_id: int,
                  node_base: int, codes, meta, stream=None):
    """meta receives (min, scale) per row: a float32 tensor of n_rows * 2 elements.  classes (from
    pack_classes) describes a width-grouped layout; bits / word_offset may then be None."""
    import torch
    px, ldx = _rows(x, "x")
    d = x.shape[1]
    _check(_quantize_pack(px, ldx, _dev(row_index, torch.int32, "row_index", allow_none=True), int(n_rows), int(d),
                          _dev(bits, torch.uint8, "bits", allow_none=True),
                          None if word_offset is None else _dev32(word_offset, "word_offset"), _cls_ref(classes),
                          int(seed) & 0xFFFFFFFFFFFFFFFF, int(epoch), int(stream_id), int(node_base),
                          _dev32(codes, "codes"), _dev(meta, torch.float32, "meta"), _stream(stream)),
           "qha_quantize_pack")


def _dequant_aggregate_args(rowptr, colidx, w, plan, x_inner, n_inner, codes, word_offset, bits, classes, meta,
                            n_halo, beta, out, row_ids, n_rows):
    import torch
    n_rows = rowptr.numel() - 1 if n_rows is None else int(n_rows)
    px, ldx = _rows(x_inner, "x_inner")
    po, ldo = _rows(out, "out")
    d = out.shape[1]
    halo = n_halo > 0
    return (n_rows, _dev(rowptr, torch.int32, "rowptr"), _dev(colidx, torch.int32, "colidx"),
            _dev(w, torch.float32, "w", allow_none=True), _dev(row_ids, torch.int32, "row_ids", allow_none=True),
            _plan_ref(plan), px, ldx, int(n_inner),
            _dev32(codes, "codes") if halo else None,
            _dev32(word_offset, "word_offset") if (halo and word_offset is not None) else None,
            _dev(bits, torch.uint8, "bits") if (halo and bits is not None) else None,
            _cls_ref(classes) if halo else None,
            _dev(meta, torch.float32, "meta") if halo else None,
            int(n_halo), int(d), int(beta), po, ldo)


def dequant_aggregate_fwd(rowptr, colidx, w, plan, x_inner, n_inner: int, codes, word_offset, bits, classes, meta,
                          n_halo: int, beta: int, out, workspace=None, row_ids=None, n_rows=None, stream=None):
    args = _dequant_aggregate_args(rowptr, colidx, w, plan, x_inner, n_inner, codes, word_offset, bits, classes, meta,
                                   n_halo, beta, out, row_ids, n_rows)
    ws_ptr = None if workspace is None else _dev(workspace, workspace.dtype, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_dequant_aggregate_fwd(*args, ws_ptr, ws_bytes, _stream(stream)), "qha_dequant_aggregate_fwd")


NOALLOC_SCRATCH_BYTES = 128 << 20


def dequant_aggregate_fwd_noalloc(rowptr, colidx, w, plan, x_inner, n_inner: int, codes, word_offset, bits, classes,
                                  meta, n_halo: int, beta: int, out, row_ids=None, n_rows=None, stream=None):
    """dequant_aggregate_fwd without a workspace: split-row partials go to the library's device scratch
    (no allocation in the call; calls that overlap on one GPU race on the scratch)."""
    args = _dequant_aggregate_args(rowptr, colidx, w, plan, x_inner, n_inner, codes, word_offset, bits, classes, meta,
                                   n_halo, beta, out, row_ids, n_rows)
    _check(_dequant_aggregate_fwd_noalloc(*args, _stream(stream)), "qha_dequant_aggregate_fwd_noalloc")


def aggregate_bwd(colptr, rowidx, w, plan, grad_out, n_grad_rows: int, beta: int, grad_in, workspace=None,
                  n_rows=None, stream=None):
    import torch
    n_rows = colptr.numel() - 1 if n_rows is None else int(n_rows)
    pg, ldg = _rows(grad_out, "grad_out")
    pi, ldi = _rows(grad_in, "grad_in")
    d = grad_in.shape[1]
    ws_ptr = None if workspace is None else _dev(workspace, workspace.dtype, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_aggregate_bwd(n_rows, _dev(colptr, torch.int32, "colptr"), _dev(rowidx, torch.int32, "rowidx"),
                          _dev(w, torch.float32, "w", allow_none=True), _plan_ref(plan), pg, ldg, int(n_grad_rows),
                          int(d), int(beta), pi, ldi, ws_ptr, ws_bytes, _stream(stream)), "qha_aggregate_bwd")


def aggregate_bwd_quantize(colptr, rowidx, w, plan, grad_out, n_grad_rows: int, d: int, bits, word_offset, classes,
                           seed: int, epoch: int, stream_id: int, node_base: int, codes, meta, workspace=None,
                           n_rows=None, stream=None, grad_in=None, n_stored: int = 0, beta: int = 0,
                           received=None):
    """The transposed gather over colptr's rows: rows below n_stored are stored into grad_in (added
    to it when beta = 1), every later row is quantised into codes / meta as message row r - n_stored.
    received = (copy_ptr, copy_idx, n_rows, codes, meta, bits, word_offset, classes) adds those
    earlier messages to the stored rows (bits / word_offset may be None with classes)."""
    import torch
    rs = None
    if received is not None:
        c_ptr, c_idx, r_rows, r_codes, r_meta, r_bits, r_off, r_cls = received
        rs = ReceivedStruct(_dev(c_ptr, torch.int32, "copy_ptr"), _dev(c_idx, torch.int32, "copy_idx"), int(r_rows),
                            _dev32(r_codes, "received codes"), _dev(r_meta, torch.float32, "received meta"),
                            _dev(r_bits, torch.uint8, "received bits", allow_none=True),
                            None if r_off is None else _dev32(r_off, "received word_offset"),
                            None if r_cls is None else C.pointer(r_cls))
    n_rows = colptr.numel() - 1 if n_rows is None else int(n_rows)
    pg, ldg = _rows(grad_out, "grad_out")
    pi, ldi = _rows(grad_in, "grad_in") if grad_in is not None else (None, d)
    msgs = n_rows > n_stored
    ws_ptr = None if workspace is None else _dev(workspace, workspace.dtype, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_aggregate_bwd_quantize(n_rows, _dev(colptr, torch.int32, "colptr"), _dev(rowidx, torch.int32, "rowidx"),
                                   _dev(w, torch.float32, "w", allow_none=True), _plan_ref(plan), pg, ldg,
                                   int(n_grad_rows), int(d), int(n_stored), int(beta), pi, ldi,
                                   _dev(bits, torch.uint8, "bits", allow_none=True) if msgs else None,
                                   None if (word_offset is None or not msgs) else _dev32(word_offset, "word_offset"),
                                   _cls_ref(classes) if msgs else None, int(seed) & 0xFFFFFFFFFFFFFFFF, int(epoch),
                                   int(stream_id), int(node_base), _dev32(codes, "codes") if msgs else None,
                                   _dev(meta, torch.float32, "meta") if msgs else None,
                                   None if rs is None else C.byref(rs), ws_ptr, ws_bytes,
                                   _stream(stream)), "qha_aggregate_bwd_quantize")


def dense_project(trans_a: int, trans_b: int, a, b, beta: int, c, prologue: int = PRO_NONE, aux=None,
                  epilogue: int = EPI_NONE, workspace=None, stream=None):
    """C = (beta ? C : 0) + op(A) op(B); shapes are read from the tensors."""
    pa, lda = _rows(a, "a")
    pb, ldb = _rows(b, "b")
    pc, ldc = _rows(c, "c")
    m = a.shape[1] if trans_a else a.shape[0]
    k = a.shape[0] if trans_a else a.shape[1]
    kb = b.shape[1] if trans_b else b.shape[0]
    n = b.shape[0] if trans_b else b.shape[1]
    if kb != k or tuple(c.shape) != (m, n):
        raise ValueError(f"shape mismatch: op(A) {m}x{k}, op(B) {kb}x{n}, C {tuple(c.shape)}")
    paux, ldaux = (None, 0)
    if prologue == PRO_RELU_MASK:
        if aux is None or tuple(aux.shape) != tuple(a.shape):
            raise ValueError("aux must have A's shape")
        paux, ldaux = _rows(aux, "aux")
    ws_ptr = None if workspace is None else _dev(workspace, workspace.dtype, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_dense_project(int(trans_a), int(trans_b), m, n, k, pa, lda, pb, ldb, int(beta), pc, ldc, int(prologue),
                          paux, ldaux, int(epilogue), ws_ptr, ws_bytes, _stream(stream)), "qha_dense_project")


def dense_backward(dh, h, a, w, da, dw, workspace=None, stream=None):
    """dZ = dH * [H > 0]; dA = dZ W (into da), dW = dZ^T A (into dw); shapes are read from the tensors:
    dh, h [m x n], a [m x k], w [n x k], da [m x k], dw [n x k]."""
    m, n = dh.shape
    k = a.shape[1]
    if tuple(h.shape) != (m, n) or tuple(a.shape) != (m, k) or tuple(w.shape) != (n, k) \
            or tuple(da.shape) != (m, k) or tuple(dw.shape) != (n, k):
        raise ValueError(f"shape mismatch: dh {tuple(dh.shape)}, h {tuple(h.shape)}, a {tuple(a.shape)}, "
                         f"w {tuple(w.shape)}, da {tuple(da.shape)}, dw {tuple(dw.shape)}")
    pg, ldg = _rows(dh, "dh")
    ph, ldh = _rows(h, "h")
    pa, lda = _rows(a, "a")
    pw, ldw = _rows(w, "w")
    pda, ldda = _rows(da, "da")
    pdw, lddw = _rows(dw, "dw")
    ws_ptr = None if workspace is None else _dev(workspace, workspace.dtype, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_dense_bwd(int(m), int(n), int(k), pg, ldg, ph, ldh, pa, lda, pw, ldw, pda, ldda, pdw, lddw, ws_ptr,
                      ws_bytes, _stream(stream)), "qha_dense_backward")
