"""The C-ABI library on the host: it loads, exports what the header declares,
and rejects bad arguments before touching a device (no GPU needed)."""
import ctypes
import glob
import os
import re

import pytest

from fine_grained_sparse_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*([a-z_][a-z0-9_]*)\s*\(", src, re.M):
            names.add(m.group(1))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from fine_grained_sparse_amd.build import build
        build()
    return B.lib()


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert set(declared) == set(B.EXPORTED), declared
    for name in declared:
        assert hasattr(lib, name), name


def _desc(**kw):
    base = dict(n_tokens=32, d_model=2560, n_experts=384, top_k=6, d_ff=512, d_ff_shared=512,
                x_dtype=B.MOE_DTYPE_BF16, w_dtype=B.MOE_DTYPE_BF16, flags=0)
    base.update(kw)
    return B.MoeDesc(**base)


def test_workspace_size_host_only(lib):
    n = B.workspace_size(_desc())
    assert n > 0 and n % 256 == 0
    # grows with the token count
    assert B.workspace_size(_desc(n_tokens=64)) > n
    # invalid descriptions give 0
    for bad in (dict(top_k=0), dict(top_k=9), dict(n_experts=4, top_k=6), dict(d_model=100),
                dict(d_ff=0), dict(n_tokens=-1), dict(flags=8), dict(n_experts=2000),
                # block scales need FP8 weights and 128-multiples
                dict(flags=B.MOE_FLAG_FP8_BLOCK128),
                dict(flags=B.MOE_FLAG_FP8_BLOCK128, w_dtype=B.MOE_DTYPE_FP8_E4M3, d_ff=448),
                dict(flags=B.MOE_FLAG_FP8_BLOCK128, w_dtype=B.MOE_DTYPE_FP8_E4M3, d_model=2496)):
        assert B.workspace_size(_desc(**bad)) == 0, bad
    assert B.workspace_size(_desc(flags=B.MOE_FLAG_FP8_BLOCK128, w_dtype=B.MOE_DTYPE_FP8_E4M3)) == n


def test_status_strings(lib):
    for st in (B.MOE_OK, B.MOE_ERR_ARG, B.MOE_ERR_UNSUPPORTED, B.MOE_ERR_WORKSPACE, B.MOE_ERR_HIP):
        assert B.status_string(st)
    assert B.last_hip_error() == 0


def _call(lib, desc, x=1 << 20, rw=16, rb=16, w=None, out=1 << 32, ws=1 << 36, wsb=None, aux=None):
    weights = w or B.MoeWeights(*([16 * (i + 1) for i in range(3)] + [None] * 3 +
                                  [16 * (i + 5) for i in range(3)] + [None] * 3))
    size = B.workspace_size(desc) if wsb is None else wsb
    return lib.moe_forward(ctypes.byref(desc), x, rw, rb, ctypes.byref(weights), out, ws, size, aux, None)


def test_argument_errors_before_device(lib):
    d = _desc()
    assert _call(lib, _desc(top_k=0)) == B.MOE_ERR_ARG
    assert _call(lib, d, x=None) == B.MOE_ERR_ARG
    assert _call(lib, d, out=None) == B.MOE_ERR_ARG
    assert _call(lib, d, x=(1 << 20) + 8) == B.MOE_ERR_ARG  # misaligned
    assert _call(lib, d, ws=(1 << 36) + 16) == B.MOE_ERR_ARG  # workspace not 256-aligned
    assert _call(lib, d, wsb=100) == B.MOE_ERR_WORKSPACE
    # bfloat16 weights must not carry scales; FP8 weights need them
    w = B.MoeWeights(16, 32, 48, 64, None, None, 80, 96, 112, None, None, None)
    assert _call(lib, d, w=w) == B.MOE_ERR_ARG
    assert _call(lib, _desc(w_dtype=B.MOE_DTYPE_FP8_E4M3)) == B.MOE_ERR_ARG
    # x and out overlap without accumulate
    assert _call(lib, d, x=1 << 32, out=(1 << 32) + 4096) == B.MOE_ERR_ARG
    # unsupported dtypes
    assert _call(lib, _desc(x_dtype=7)) == B.MOE_ERR_UNSUPPORTED
    # zero tokens: a valid no-op even without buffers
    assert lib.moe_forward(ctypes.byref(_desc(n_tokens=0)), None, None, None, None, None, None, 0, None,
                           None) == B.MOE_OK


def test_noalloc_argument_errors_before_device(lib):
    """moe_forward_noalloc checks its arguments and the scratch size on the host, before any device call."""
    weights = B.MoeWeights(*([16 * (i + 1) for i in range(3)] + [None] * 3 +
                             [16 * (i + 5) for i in range(3)] + [None] * 3))

    def call(desc, x=1 << 20, out=1 << 32):
        return lib.moe_forward_noalloc(ctypes.byref(desc), x, 16, 16, ctypes.byref(weights), out, None, None)

    assert call(_desc(top_k=0)) == B.MOE_ERR_ARG
    assert call(_desc(), x=None) == B.MOE_ERR_ARG
    assert call(_desc(), x=(1 << 20) + 8) == B.MOE_ERR_ARG
    # the scratch array holds the full layer up to 256 tokens, not 320
    assert B.workspace_size(_desc(n_tokens=256)) <= B.MOE_NOALLOC_SCRATCH_BYTES
    assert B.workspace_size(_desc(n_tokens=320)) > B.MOE_NOALLOC_SCRATCH_BYTES
    assert call(_desc(n_tokens=320)) == B.MOE_ERR_WORKSPACE
    assert lib.moe_forward_noalloc(ctypes.byref(_desc(n_tokens=0)), None, None, None, None, None, None,
                                   None) == B.MOE_OK
