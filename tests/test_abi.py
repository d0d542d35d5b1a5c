"""Host-only checks of the C ABI: the library loads, exports every symbol moe.h declares, and
rejects invalid arguments before launching anything (no GPU needed for any of these calls)."""
import ctypes
import os
import re
import subprocess

import pytest

import sparse_mixture_experts_33_amd as moe
from sparse_mixture_experts_33_amd.moe import moe_dims, moe_opts

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

FAKE = 1 << 20           # an aligned, never dereferenced address: validation fails or T=0 returns first


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_header_declares_the_five_stage_calls():
    names = declared_functions()
    for n in ("moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_forward"):
        assert n in names
    assert set(names) == set(moe.moe.SYMBOLS)


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", moe.moe.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (moe_\w+)", out))
    assert set(declared_functions()) <= exported


def test_status_strings_and_version():
    assert moe.moe_abi_version() == 5
    assert [moe.moe_status_string(i) for i in range(5)] == list(moe.moe.STATUS.values())


def _route(dims, x=FAKE, wg=FAKE, idx=FAKE, w=FAKE, logits=None):
    return moe.lib().moe_route(ctypes.byref(dims), None, x, wg, idx, w, logits, None)


@pytest.mark.parametrize("dims,status,msg", [
    (moe_dims(-1, 128, 256, 8, 2, 0), 1, "negative"),
    (moe_dims(4, 0, 256, 8, 2, 0), 1, "d = 0"),
    (moe_dims(4, 128, 256, 8, 9, 0), 1, "exceeds"),
    (moe_dims(4, 128, 256, 0, 1, 0), 1, "positive"),
    (moe_dims(4, 128, 256, 8, 2, 7), 1, "dtype"),
    (moe_dims(4, 100, 256, 8, 2, 0), 2, "multiple of 64"),
    (moe_dims(4, 128, 256, 65, 2, 0), 2, "E = 65"),
    (moe_dims(4, 128, 256, 16, 9, 0), 2, "K = 9"),
    (moe_dims(1 << 30, 128, 256, 8, 2, 0), 2, "2^31"),
])
def test_route_validation(dims, status, msg):
    assert _route(dims) == status
    assert msg in moe.moe_last_error()


def test_null_and_misaligned_pointers():
    d = moe_dims(4, 128, 256, 8, 2, 1)
    assert _route(d, x=None) == 1 and "x is NULL" in moe.moe_last_error()
    assert _route(d, wg=FAKE + 8) == 1 and "aligned" in moe.moe_last_error()
    assert _route(d, logits=FAKE + 4) == 1
    assert moe.lib().moe_route(None, None, FAKE, FAKE, FAKE, FAKE, None, None) == 1


def test_zero_tokens_launch_nothing():
    d = moe_dims(0, 128, 256, 8, 2, 1)
    L = moe.lib()
    assert _route(d) == 0
    assert L.moe_permute(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 0
    assert L.moe_expert_ffn(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 0
    assert L.moe_combine(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, None) == 0
    assert L.moe_forward(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 0
    assert L.moe_rmsnorm(0, 128, ctypes.c_float(1e-5), FAKE, FAKE, None) == 0


def test_workspace_checks():
    L = moe.lib()
    d = moe_dims(32, 4096, 14336, 8, 2, 1)
    need = moe.moe_workspace_bytes(moe.Dims(32, 4096, 14336, 8, 2, 1))
    S = 32 * 2
    assert need >= S * 14336 * 2 + S * 4096 * 4 + S * 16      # hidden, expert outputs, maps
    assert moe.moe_workspace_bytes(moe.Dims(64, 4096, 14336, 8, 2, 1)) > need
    assert moe.moe_workspace_bytes(moe.Dims(32, 4096, 14336, 8, 9, 1)) == 0
    assert L.moe_forward(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == 3
    assert "needs" in moe.moe_last_error()
    assert L.moe_forward(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 16, need, None) == 1
    bad = moe_opts(None, 5, 0)
    assert L.moe_forward(ctypes.byref(d), ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need,
                         None) == 1
    acc = moe_opts(None, 0, 2)
    assert L.moe_combine(ctypes.byref(d), ctypes.byref(acc), FAKE, FAKE, FAKE, FAKE, None) == 1


def test_noalloc_rejects_sizes_beyond_its_scratch():
    """moe_forward_noalloc refuses, before any HIP call, sizes whose workspace exceeds the static
    scratch (64 MiB), and validates its dims like moe_forward."""
    L = moe.lib()
    assert moe.moe.MOE_NOALLOC_SCRATCH_BYTES == 64 << 20
    big = moe.Dims(4096, 4096, 14336, 8, 2, 1)
    assert moe.moe_workspace_bytes(big) > moe.moe.MOE_NOALLOC_SCRATCH_BYTES
    assert L.moe_forward_noalloc(ctypes.byref(big.c()), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 3
    assert "static scratch" in moe.moe_last_error()
    assert moe.moe_workspace_bytes(moe.Dims(32, 4096, 14336, 8, 2, 1)) <= moe.moe.MOE_NOALLOC_SCRATCH_BYTES
    bad = moe_dims(32, 4096, 14336, 8, 9, 1)
    assert L.moe_forward_noalloc(ctypes.byref(bad), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1


def test_saved_activations_validation():
    """moe_opts.activations: 16-byte aligned, bf16, d and F multiples of 256 (forward and backward)."""
    L = moe.lib()
    d = moe_dims(32, 4096, 14336, 8, 2, 1)
    need = moe.moe_workspace_bytes(moe.Dims(32, 4096, 14336, 8, 2, 1))
    fwd = lambda dims, o, nbytes: L.moe_forward(ctypes.byref(dims), ctypes.byref(o), FAKE, FAKE, FAKE, FAKE, FAKE,
                                                FAKE, FAKE, nbytes, None)
    ok = moe_opts(None, 1, 0, None, FAKE)
    assert fwd(d, ok, need - 1) == 3                                   # accepted, then the workspace check
    assert fwd(d, moe_opts(None, 1, 0, None, FAKE + 4), need) == 1     # misaligned
    assert "activations" in moe.moe_last_error()
    f32 = moe_dims(32, 4096, 14336, 8, 2, 0)
    assert fwd(f32, moe_opts(None, 0, 0, None, FAKE), moe.moe_workspace_bytes(moe.Dims(32, 4096, 14336, 8, 2, 0))) == 2
    d192 = moe_dims(32, 192, 512, 8, 2, 1)
    assert fwd(d192, ok, moe.moe_workspace_bytes(moe.Dims(32, 192, 512, 8, 2, 1))) == 2
    bwd = moe_dims(64, 256, 512, 8, 2, 1, 0)
    bad = moe_opts(None, 1, 0, None, FAKE + 4)
    assert L.moe_backward(ctypes.byref(bwd), ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                          FAKE, FAKE, None, FAKE, 1 << 40, None) == 1


def test_rmsnorm_validation():
    L = moe.lib()
    assert L.moe_rmsnorm(-1, 128, ctypes.c_float(1e-5), FAKE, FAKE, None) == 1
    assert L.moe_rmsnorm(4, 96, ctypes.c_float(1e-5), FAKE, FAKE, None) == 2
    assert L.moe_rmsnorm(4, 128, ctypes.c_float(-1.0), FAKE, FAKE, None) == 1
    assert L.moe_rmsnorm(4, 128, ctypes.c_float(1e-5), None, FAKE, None) == 1


def test_binding_raises_with_detail():
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_route(moe.Dims(4, 128, 256, 8, 9, 0), FAKE, FAKE, FAKE, FAKE, stream=0)
    assert ei.value.status == 1 and "exceeds" in str(ei.value)


def _backward(dims, ws=FAKE, nbytes=1 << 40, dy=FAKE, dlogits=None):
    return moe.lib().moe_backward(ctypes.byref(dims), None, FAKE, FAKE, FAKE, FAKE, FAKE, dy, FAKE, FAKE, FAKE, FAKE,
                                  FAKE, dlogits, ws, nbytes, None)


def test_backward_validation():
    L = moe.lib()
    ok = moe_dims(64, 256, 512, 8, 2, 1, 0)
    assert L.moe_backward_workspace_bytes(ctypes.byref(ok)) > 0
    # either weight layout (the packed one gives the same workspace)
    pk = moe_dims(64, 256, 512, 8, 2, 1, 1)
    assert L.moe_backward_workspace_bytes(ctypes.byref(pk)) == L.moe_backward_workspace_bytes(ctypes.byref(ok))
    assert _backward(moe_dims(64, 256, 512, 8, 2, 1, 2)) == 1        # not a layout
    # supported sizes only: bf16, d and F multiples of 256
    for bad in (moe_dims(64, 256, 512, 8, 2, 0, 0), moe_dims(64, 192, 512, 8, 2, 1, 0),
                moe_dims(64, 256, 448, 8, 2, 1, 0)):
        assert L.moe_backward_workspace_bytes(ctypes.byref(bad)) == 0
        assert _backward(bad) == 2
    assert _backward(moe_dims(64, 256, 512, 8, 9, 1, 0)) == 1       # K > E
    assert _backward(ok, dy=None) == 1 and "dy" in moe.moe_last_error()
    assert _backward(ok, dlogits=FAKE + 4) == 1                      # misaligned optional output
    assert _backward(ok, nbytes=16) == 3                             # workspace too small
    assert _backward(ok, ws=FAKE + 64) == 1                          # workspace not 256-byte aligned
    assert _backward(moe_dims(0, 256, 512, 8, 2, 1, 0), ws=None, nbytes=0) == 0   # T = 0: nothing to do
    # the workspace grows with the tokens
    big = moe_dims(4096, 256, 512, 8, 2, 1, 0)
    assert L.moe_backward_workspace_bytes(ctypes.byref(big)) > L.moe_backward_workspace_bytes(ctypes.byref(ok))


def test_attention_and_block_validation():
    from sparse_mixture_experts_33_amd.moe import moe_attn_dims
    L = moe.lib()
    ok = moe_attn_dims(64, 512, 8, 2, 128, 1e6, 1e-5)
    mdims = moe_dims(64, 512, 512, 8, 2, 1, 0)
    att = lambda a, q=FAKE, o=FAKE: L.moe_attention(ctypes.byref(a), q, FAKE, FAKE, o, None)
    blk = lambda m, a, h=FAKE, ws=FAKE, nbytes=1 << 40: L.moe_block_forward(
        ctypes.byref(m), ctypes.byref(a), None, h, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, nbytes, None)
    assert att(moe_attn_dims(-1, 512, 8, 2, 128, 1e6, 1e-5)) == 1
    assert att(moe_attn_dims(64, 512, 8, 3, 128, 1e6, 1e-5)) == 1      # heads not a multiple of kv heads
    assert att(moe_attn_dims(64, 512, 8, 2, 64, 1e6, 1e-5)) == 2       # head width other than 128
    assert att(moe_attn_dims(64, 512, 4, 2, 128, 1e6, 1e-5)) == 2      # group of 2 query heads
    assert att(moe_attn_dims(64, 512, 8, 2, 128, 1.0, 1e-5)) == 1      # rotary base must exceed 1
    assert att(ok, q=None) == 1 and "q" in moe.moe_last_error()
    assert att(ok, o=FAKE + 8) == 1                                     # misaligned
    assert att(moe_attn_dims(0, 512, 8, 2, 128, 1e6, 1e-5), q=None, o=None) == 1   # pointers checked first
    assert L.moe_block_workspace_bytes(ctypes.byref(mdims), ctypes.byref(ok)) > 0
    assert blk(moe_dims(64, 512, 512, 8, 2, 0, 0), ok) == 2                         # fp32 block
    assert blk(moe_dims(32, 512, 512, 8, 2, 1, 0), ok) == 1                         # T disagrees
    assert blk(moe_dims(64, 448, 512, 8, 2, 1, 0), moe_attn_dims(64, 448, 8, 2, 128, 1e6, 1e-5)) == 2  # d % 256
    assert blk(mdims, ok, h=None) == 1
    assert blk(mdims, ok, nbytes=16) == 3
    assert blk(mdims, ok, ws=FAKE + 64) == 1
    z = moe_attn_dims(0, 512, 8, 2, 128, 1e6, 1e-5)
    assert blk(moe_dims(0, 512, 512, 8, 2, 1, 0), z, ws=None, nbytes=0) == 0         # T = 0: nothing to do
