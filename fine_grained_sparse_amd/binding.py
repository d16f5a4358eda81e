"""ctypes binding of the C ABI in include/fgs_moe.h (argument marshalling only).

Every step of the layer runs in the HIP library; this module only turns torch
tensors into device pointers and the current HIP stream.  It raises when the
library is missing: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# FGS_MOE_LIB may point at another build of the same sources
LIB_PATH = os.environ.get("FGS_MOE_LIB") or os.path.join(HERE, "libfgs_moe.so")

MOE_OK, MOE_ERR_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_DTYPE_F32, MOE_DTYPE_BF16, MOE_DTYPE_FP8_E4M3 = 0, 1, 2
MOE_FLAG_ACCUMULATE = 1
MOE_FLAG_RENORMALIZE = 2
MOE_FLAG_FP8_BLOCK128 = 4
MOE_FLAG_FP8_ACT_QUANT = 8
STAGES = ("router", "topk", "dispatch", "gate_up", "down", "combine")
MOE_NUM_STAGES = len(STAGES)

EXPORTED = ("moe_workspace_size", "moe_forward", "moe_status_string", "moe_last_hip_error",
            "moe_block_workspace_size", "moe_block_forward", "moe_quantize_groups", "moe_forward_noalloc")
MOE_NOALLOC_SCRATCH_BYTES = 32 << 20


class MoeDesc(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("d_ff_shared", ctypes.c_int32),
                ("x_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
                                               "ws_gate", "ws_up", "ws_down", "ss_gate", "ss_up", "ss_down")]


class MoeAux(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("logits", "topk_ids", "topk_w", "gap", "expert_offsets",
                                               "pair_of_row", "row_of_pair", "stage_events")]


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})"
                         + (f", hip error {last_hip_error()}" if status == MOE_ERR_HIP else ""))
        self.status = status


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with fine_grained_sparse_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_workspace_size.argtypes = [ctypes.POINTER(MoeDesc)]
        L.moe_workspace_size.restype = ctypes.c_size_t
        L.moe_forward.argtypes = [ctypes.POINTER(MoeDesc), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.POINTER(MoeWeights), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.POINTER(MoeAux), ctypes.c_void_p]
        L.moe_forward.restype = ctypes.c_int
        L.moe_forward_noalloc.argtypes = [ctypes.POINTER(MoeDesc), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.POINTER(MoeWeights), ctypes.c_void_p, ctypes.POINTER(MoeAux),
                                          ctypes.c_void_p]
        L.moe_forward_noalloc.restype = ctypes.c_int
        L.moe_block_workspace_size.argtypes = [ctypes.POINTER(MoeDesc)]
        L.moe_block_workspace_size.restype = ctypes.c_size_t
        L.moe_block_forward.argtypes = [ctypes.POINTER(MoeDesc), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(MoeWeights),
                                        ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(MoeAux), ctypes.c_void_p]
        L.moe_block_forward.restype = ctypes.c_int
        L.moe_quantize_groups.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int32,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.moe_quantize_groups.restype = ctypes.c_int
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_last_hip_error.argtypes = []
        L.moe_last_hip_error.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def last_hip_error() -> int:
    return lib().moe_last_hip_error()


_XDT = {torch.float32: MOE_DTYPE_F32, torch.bfloat16: MOE_DTYPE_BF16}


def make_desc(n_tokens: int, d_model: int, n_experts: int, top_k: int, d_ff: int, d_ff_shared: int,
              x_dtype: int, w_dtype: int, flags: int = 0) -> MoeDesc:
    return MoeDesc(n_tokens, d_model, n_experts, top_k, d_ff, d_ff_shared, x_dtype, w_dtype, flags)


def workspace_size(desc: MoeDesc) -> int:
    return int(lib().moe_workspace_size(ctypes.byref(desc)))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def quantize_groups(v: torch.Tensor, q: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None):
    """moe_quantize_groups on a [rows, cols] float32/bfloat16 device tensor -> (uint8 codes, float32 scales)."""
    rows, cols = v.shape
    if q is None:
        q = torch.empty(rows, cols, dtype=torch.uint8, device=v.device)
    if scales is None:
        scales = torch.empty(rows, max(cols // 128, 1), dtype=torch.float32, device=v.device)
    st = lib().moe_quantize_groups(_ptr(v), _XDT[v.dtype], rows, cols, _ptr(q), _ptr(scales),
                                   torch.cuda.current_stream(v.device).cuda_stream)
    if st != MOE_OK:
        raise MoeError(st, "moe_quantize_groups")
    return q, scales


def weights_struct(w: Dict[str, torch.Tensor]) -> MoeWeights:
    names = [f[0] for f in MoeWeights._fields_]
    return MoeWeights(*[_ptr(w.get(n)) for n in names])


def forward_raw(desc: MoeDesc, x: torch.Tensor, router_w: torch.Tensor, router_b: torch.Tensor,
                weights: MoeWeights, out: torch.Tensor, workspace: torch.Tensor,
                aux: Optional[MoeAux] = None, stream: Optional[int] = None) -> int:
    """Call moe_forward with already-built structs; returns the status code."""
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    return lib().moe_forward(ctypes.byref(desc), _ptr(x), _ptr(router_w), _ptr(router_b),
                             ctypes.byref(weights), _ptr(out), _ptr(workspace), workspace.numel(),
                             ctypes.byref(aux) if aux is not None else None, stream)


def forward_noalloc_raw(desc: MoeDesc, x: torch.Tensor, router_w: torch.Tensor, router_b: torch.Tensor,
                        weights: MoeWeights, out: torch.Tensor, aux: Optional[MoeAux] = None,
                        stream: Optional[int] = None) -> int:
    """Call moe_forward_noalloc (the library's own per-GPU scratch); returns the status code."""
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    return lib().moe_forward_noalloc(ctypes.byref(desc), _ptr(x), _ptr(router_w), _ptr(router_b),
                                     ctypes.byref(weights), _ptr(out), ctypes.byref(aux) if aux is not None else None,
                                     stream)


class MoeLayer:
    """Device tensors of one layer plus a workspace; calls the C ABI."""

    def __init__(self, top_k: int, inputs: Dict[str, torch.Tensor], n_tokens_max: int, x_dtype: torch.dtype):
        self.top_k = top_k
        self.w = inputs
        E, d = inputs["router_w"].shape
        self.E, self.d = E, d
        self.f = inputs["w_gate"].shape[1]
        self.fs = inputs["ws_gate"].shape[0]
        self.wdt = MOE_DTYPE_FP8_E4M3 if inputs["w_gate"].dtype == torch.uint8 else MOE_DTYPE_BF16
        self.xdt = _XDT[x_dtype]
        # FP8 scales of shape [E, f/128, d/128] are 128 x 128 block scales
        sg = inputs.get("s_gate")
        self.base_flags = MOE_FLAG_FP8_BLOCK128 if sg is not None and sg.dim() == 3 else 0
        self.weights = weights_struct(inputs)
        ws = workspace_size(self.desc(n_tokens_max))
        if ws == 0:
            raise MoeError(MOE_ERR_ARG, "moe_workspace_size")
        dev = inputs["router_w"].device
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=dev)

    def desc(self, n: int, flags: int = 0) -> MoeDesc:
        return make_desc(n, self.d, self.E, self.top_k, self.f, self.fs, self.xdt, self.wdt, flags | self.base_flags)

    def forward(self, x: torch.Tensor, out: Optional[torch.Tensor] = None, accumulate: bool = False,
                aux: Optional[MoeAux] = None, router_w: Optional[torch.Tensor] = None,
                router_b: Optional[torch.Tensor] = None, renormalize: bool = False,
                act_quant: bool = False) -> torch.Tensor:
        n = x.shape[0]
        if out is None:
            out = torch.empty_like(x)
        flags = ((MOE_FLAG_ACCUMULATE if accumulate else 0) | (MOE_FLAG_RENORMALIZE if renormalize else 0)
                 | (MOE_FLAG_FP8_ACT_QUANT if act_quant else 0))
        desc = self.desc(n, flags)
        need = workspace_size(desc)
        if need > self.workspace.numel():
            self.workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        st = forward_raw(desc, x, self.w["router_w"] if router_w is None else router_w,
                         self.w["router_b"] if router_b is None else router_b, self.weights, out,
                         self.workspace, aux)
        if st != MOE_OK:
            raise MoeError(st, "moe_forward")
        return out

    def block_forward(self, resid: torch.Tensor, norm_pre: torch.Tensor, norm_post: torch.Tensor, eps: float,
                      aux: Optional[MoeAux] = None, renormalize: bool = False,
                      act_quant: bool = False) -> torch.Tensor:
        """Sandwich-normalised MoE sublayer; updates `resid` in place and returns it."""
        n = resid.shape[0]
        desc = self.desc(n, (MOE_FLAG_RENORMALIZE if renormalize else 0) | (MOE_FLAG_FP8_ACT_QUANT if act_quant else 0))
        need = int(lib().moe_block_workspace_size(ctypes.byref(desc)))
        if need == 0:
            raise MoeError(MOE_ERR_ARG, "moe_block_workspace_size")
        if need > self.workspace.numel():
            self.workspace = torch.empty(need, dtype=torch.uint8, device=resid.device)
        stream = torch.cuda.current_stream(resid.device).cuda_stream
        st = lib().moe_block_forward(ctypes.byref(desc), _ptr(resid), _ptr(norm_pre), _ptr(norm_post), eps,
                                     _ptr(self.w["router_w"]), _ptr(self.w["router_b"]), ctypes.byref(self.weights),
                                     _ptr(self.workspace), self.workspace.numel(),
                                     ctypes.byref(aux) if aux is not None else None, stream)
        if st != MOE_OK:
            raise MoeError(st, "moe_block_forward")
        return resid


def route_outputs(n: int, E: int, k: int, device) -> Dict[str, torch.Tensor]:
    """Allocate every optional intermediate output of one call."""
    i32, f32 = torch.int32, torch.float32
    return dict(logits=torch.empty(n, E, dtype=f32, device=device),
                topk_ids=torch.empty(n, k, dtype=i32, device=device),
                topk_w=torch.empty(n, k, dtype=f32, device=device),
                gap=torch.empty(n, dtype=f32, device=device),
                expert_offsets=torch.empty(E + 1, dtype=i32, device=device),
                pair_of_row=torch.empty(n * k, dtype=i32, device=device),
                row_of_pair=torch.empty(n * k, dtype=i32, device=device))


def aux_struct(bufs: Dict[str, torch.Tensor], events_array=None) -> MoeAux:
    a = MoeAux(*[_ptr(bufs.get(f[0])) for f in MoeAux._fields_[:-1]], None)
    if events_array is not None:
        a.stage_events = ctypes.cast(events_array, ctypes.c_void_p)
    return a
