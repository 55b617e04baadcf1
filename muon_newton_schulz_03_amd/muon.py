"""Python binding of the gfx950 Muon step: marshals torch tensors into the C ABI.

Every step of the update runs in the HIP library; this module only builds
descriptor arrays, allocates the workspace with torch (device memory
plumbing) and passes the current torch stream.  There is no fallback: if the
library is missing, `_lib.load` raises.
"""
from __future__ import annotations

import ctypes
from typing import Dict, List, Optional, Sequence, Tuple

import torch

from . import _lib
from ._lib import MatrixDesc, Options, PlanInfo

DEFAULT_COEFFS = (3.4445, -4.7750, 2.0315)

_DTYPES = {torch.float32: _lib.MUON_DTYPE_F32, torch.bfloat16: _lib.MUON_DTYPE_BF16}
_PATHS = {"bf16": _lib.MUON_PATH_BF16, "f32": _lib.MUON_PATH_F32}


def version() -> str:
    return _lib.load().muon_version().decode()


def _options(path: str, x_master_iters: int, zero_momentum: bool, max_T: int, groups: int = 0,
             fused: bool = False) -> Options:
    if path not in _PATHS:
        raise ValueError(f"path must be one of {sorted(_PATHS)}")
    return Options(_PATHS[path], x_master_iters, int(zero_momentum), max_T, groups, int(bool(fused)))


def _desc_array(shapes_dtypes, ptrs=None, scales=None) -> ctypes.Array:
    n = len(shapes_dtypes)
    arr = (MatrixDesc * n)()
    for i, (rows, cols, w_dt, g_dt) in enumerate(shapes_dtypes):
        d = arr[i]
        d.rows, d.cols = rows, cols
        d.ld_w = d.ld_g = cols
        d.w_dtype, d.g_dtype = w_dt, g_dt
        d.scale = 0.0 if scales is None else float(scales[i])
        d.reserved = 0
        if ptrs is not None:
            d.weight, d.grad, d.momentum = ptrs[i]
    return arr


def _tensor_descs(weights, grads, moms, scales) -> ctypes.Array:
    if not (len(weights) == len(grads) == len(moms)):
        raise ValueError("weights, grads and moms must have the same length")
    items, ptrs = [], []
    for i, (w, g, m) in enumerate(zip(weights, grads, moms)):
        for name, t in (("weight", w), ("grad", g), ("momentum", m)):
            if not t.is_cuda:
                raise ValueError(f"matrix {i}: {name} is not a device tensor")
            if t.dim() != 2 or not t.is_contiguous():
                raise ValueError(f"matrix {i}: {name} must be a contiguous 2-D tensor")
        if not (w.shape == g.shape == m.shape):
            raise ValueError(f"matrix {i}: weight, grad and momentum shapes differ")
        if m.dtype != torch.float32:
            raise ValueError(f"matrix {i}: momentum must be float32")
        if w.dtype not in _DTYPES or g.dtype not in _DTYPES:
            raise ValueError(f"matrix {i}: weight/grad dtype must be float32 or bfloat16")
        items.append((w.shape[0], w.shape[1], _DTYPES[w.dtype], _DTYPES[g.dtype]))
        ptrs.append((w.data_ptr(), g.data_ptr(), m.data_ptr()))
    return _desc_array(items, ptrs, scales)


def describe(shapes: Sequence[Tuple[int, int]], path: str = "bf16", x_master_iters: int = -1,
             kind: Optional[int] = None, grad_dtype=torch.bfloat16, weight_dtype=torch.float32,
             groups: int = 0, fused: bool = False) -> Tuple[dict, list]:
    """Host-only plan description (no GPU needed): sizes, grids and one tile list
    ((matrix, tile_row, tile_col) triples; for KIND_FUSED (xcd, product, matrix,
    tile_row, tile_col) quintuples)."""
    lib = _lib.load()
    arr = _desc_array([(r, c, _DTYPES[weight_dtype], _DTYPES[grad_dtype]) for r, c in shapes])
    opts = _options(path, x_master_iters, False, 0, groups, fused)
    info = PlanInfo()
    count = ctypes.c_int32(0)
    k = -1 if kind is None else kind
    _lib.check(lib.muon_describe(arr, len(shapes), ctypes.byref(opts), ctypes.byref(info), k, None, 0,
                                 ctypes.byref(count)))
    tiles = []
    if kind is not None and count.value:
        width = 5 if k == _lib.KIND_FUSED else 3
        buf = (ctypes.c_int32 * (width * count.value))()
        _lib.check(lib.muon_describe(arr, len(shapes), ctypes.byref(opts), None, k, buf, count.value,
                                     ctypes.byref(count)))
        tiles = [tuple(buf[width * q:width * q + width]) for q in range(count.value)]
    d = dict(workspace_bytes=info.workspace_bytes, n_matrices=info.n_matrices, tile=info.tile,
             blocks=list(info.blocks), x_master_iters=info.x_master_iters, path=info.path,
             n_f32_matrices=info.n_f32_matrices, n_groups=info.n_groups,
             bf16_tile_rows=info.bf16_tile_rows, bf16_tile_cols=info.bf16_tile_cols, fused=info.fused)
    return d, tiles


def step_scratch(weights: Sequence[torch.Tensor], grads: Sequence[torch.Tensor], moms: Sequence[torch.Tensor], *,
                 a: float = DEFAULT_COEFFS[0], b: float = DEFAULT_COEFFS[1], c: float = DEFAULT_COEFFS[2],
                 T: int = 5, momentum: float = 0.95, nesterov: bool = True, lr: float = 0.05,
                 path: str = "bf16", x_master_iters: int = -1, max_T: int = 0,
                 scales: Optional[Sequence[float]] = None) -> None:
    """One Muon step over these matrices through muon_step_scratch: no plan and no
    workspace; the library's static device array holds the working memory, so
    nothing is allocated.  Enqueued on the current torch stream."""
    lib = _lib.load()
    descs = _tensor_descs(weights, grads, moms, None if scales is None else list(scales))
    opts = _options(path, x_master_iters, False, max_T, 1)
    stream = torch.cuda.current_stream(weights[0].device).cuda_stream
    _lib.check(lib.muon_step_scratch(descs, len(weights), ctypes.byref(opts), a, b, c, T, momentum,
                                     int(bool(nesterov)), lr, ctypes.c_void_p(stream)))


class MuonStep:
    """A Muon plan over a fixed list of hidden matrices.

    ``step()`` enqueues one Muon step (momentum, normalisation, T Newton-Schulz
    iterations, weight update) on the current torch stream of the tensors'
    device.  Momentum buffers and weights are updated in place.
    """

    def __init__(self, weights: Sequence[torch.Tensor], grads: Sequence[torch.Tensor],
                 moms: Sequence[torch.Tensor], *, path: str = "bf16", x_master_iters: int = -1,
                 zero_momentum: bool = False, max_T: int = 0, scales: Optional[Sequence[float]] = None,
                 groups: int = 0, fused: bool = False):
        self._lib = _lib.load()
        self.n = len(weights)
        if self.n == 0:
            raise ValueError("no matrices")
        self.device = weights[0].device
        self.scales = None if scales is None else list(scales)
        self._descs = _tensor_descs(weights, grads, moms, self.scales)
        self._keep = (list(weights), list(grads), list(moms))
        self._opts = _options(path, x_master_iters, zero_momentum, max_T, groups, fused)
        ws = self._lib.muon_workspace_size(self._descs, self.n, ctypes.byref(self._opts))
        if ws == 0:
            raise _lib.MuonError(_lib.MUON_E_INVAL, _lib.last_error())
        self.workspace = torch.empty(int(ws), dtype=torch.uint8, device=self.device)
        self._plan = ctypes.c_void_p()
        stream = torch.cuda.current_stream(self.device).cuda_stream
        _lib.check(self._lib.muon_init(self._descs, self.n, ctypes.byref(self._opts),
                                       ctypes.c_void_p(self.workspace.data_ptr()), ctypes.c_size_t(int(ws)),
                                       ctypes.c_void_p(stream), ctypes.byref(self._plan)))

    @property
    def workspace_bytes(self) -> int:
        return self.workspace.numel()

    def step(self, *, a: float = DEFAULT_COEFFS[0], b: float = DEFAULT_COEFFS[1], c: float = DEFAULT_COEFFS[2],
             T: int = 5, momentum: float = 0.95, nesterov: bool = True, lr: float = 0.05,
             weights=None, grads=None, moms=None, schedule: Optional[Sequence[Tuple[float, float, float]]] = None
             ) -> None:
        """Enqueue one step.  New tensors (same shapes/dtypes) may replace any of the lists.

        ``schedule`` (one (a, b, c) per iteration) replaces a, b, c and T.
        """
        descs = None
        if weights is not None or grads is not None or moms is not None:
            w, g, m = self._keep
            w = list(weights) if weights is not None else w
            g = list(grads) if grads is not None else g
            m = list(moms) if moms is not None else m
            descs = _tensor_descs(w, g, m, self.scales)
            self._keep = (w, g, m)
        stream = torch.cuda.current_stream(self.device).cuda_stream
        if schedule is not None:
            flat = [float(v) for triple in schedule for v in triple]
            if len(flat) != 3 * len(schedule):
                raise ValueError("schedule entries must be (a, b, c) triples")
            arr = (ctypes.c_float * max(len(flat), 1))(*flat)
            _lib.check(self._lib.muon_step_schedule(self._plan, descs, self.n, arr, len(schedule), momentum,
                                                    int(bool(nesterov)), lr, ctypes.c_void_p(stream)))
            return
        _lib.check(self._lib.muon_step(self._plan, descs, self.n, a, b, c, int(T), momentum, int(bool(nesterov)),
                                       lr, ctypes.c_void_p(stream)))

    def check(self) -> None:
        """Wait for the current stream; raise if a fused launch gave up a dependency wait."""
        stream = torch.cuda.current_stream(self.device).cuda_stream
        _lib.check(self._lib.muon_check(self._plan, ctypes.c_void_p(stream)))

    def fused_limits(self, spin_limit: int, dep_bias: int = 0) -> None:
        """Poll limit and target bias of the fused launch's dependency waits (tests of the give-up path)."""
        _lib.check(self._lib.muon_fused_limits(self._plan, int(spin_limit), int(dep_bias)))

    def profile(self, enable: bool = True, kinds: Optional[Sequence[str]] = None) -> None:
        """Time launches with HIP events; ``kinds`` (names from KIND_NAMES) limits which."""
        mask = 0xFFFFFFFF if kinds is None else sum(1 << _lib.KIND_NAMES.index(k) for k in kinds)
        _lib.check(self._lib.muon_profile_select(self._plan, mask))
        _lib.check(self._lib.muon_profile_enable(self._plan, int(enable)))

    def read_profile(self) -> Dict[str, Tuple[float, int]]:
        """{kind: (total milliseconds, launches)} since the last read."""
        ms = (ctypes.c_double * _lib.KIND_COUNT)()
        cnt = (ctypes.c_int64 * _lib.KIND_COUNT)()
        _lib.check(self._lib.muon_profile_read(self._plan, ms, cnt))
        return {name: (ms[k], cnt[k]) for k, name in enumerate(_lib.KIND_NAMES)}

    def close(self) -> None:
        if getattr(self, "_plan", None) is not None and self._plan.value:
            self._lib.muon_destroy(self._plan)
            self._plan = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
