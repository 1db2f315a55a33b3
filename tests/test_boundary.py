"""The C ABI on the CPU: the library loads, exports every declared symbol, and
rejects invalid calls on the host before any HIP call (no GPU needed)."""
import ctypes
import json
import os
import re

import pytest

from linear_cross_entropy_bf16_amd import _lib
from linear_cross_entropy_bf16_amd.build import LIB_PATH, build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flce.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")

# Any 256-byte aligned, never-dereferenced address: every call below is
# rejected by host validation before a pointer is touched.
FAKE = 0x7f0000000000


@pytest.fixture(scope="module")
def lib():
    build(force=False)          # rebuild when any source is newer than the library
    return _lib.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(flce_[a-z_]+)\s*\(", src)))


def test_header_declares_the_documented_entry_points():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    names = {s: lib.flce_status_string(s).decode() for s in range(6)}
    assert names[0] == "ok"
    assert names[4] == "target out of range"
    assert len(set(names.values())) == 6
    assert lib.flce_status_string(99).decode() == "unknown status"
    assert _lib.version() >= 100


def P(**kw):
    base = dict(n=256, d=128, v=1024, dtype=_lib.DTYPE_F32)
    base.update(kw)
    return _lib.make_params(**base)


def test_workspace_size_rejects_bad_params(lib):
    assert _lib.workspace_size(P(), True) > 0
    for bad in (P(d=100), P(d=0), P(v=0), P(n=-1), P(dtype=7), P(label_smoothing=1.5),
                P(label_smoothing=-0.1), P(lse_square_scale=-1.0), P(softcap=-2.0),
                P(vocab_slice=-1), P(n=1 << 31)):
        assert _lib.workspace_size(bad, True) == 0
    assert lib.flce_workspace_size(None, 1) == 0


def test_workspace_never_holds_the_logits():
    g = json.load(open(os.path.join(GOLDEN, "logit_bottleneck_sizes.json")))
    n, d, v = g["n"], g["d"], g["v"]
    assert round(n * v / 1e9, 1) == g["logit_elements_billions"]
    assert round(2 * n * v / 1e9, 1) == g["logits_bf16_gb"]
    assert round(4 * n * v / 1e9, 1) == g["logits_fp32_gb"]
    p = _lib.make_params(n, d, v, _lib.DTYPE_BF16)
    ws = _lib.workspace_size(p, True)
    # under a third of one bf16 copy of the logits (the workspace holds one G
    # slice in both orientations, X^T, the fp32 dX sum and the packed valid rows of X)
    assert 0 < ws < 2 * n * v / 3
    assert _lib.workspace_size(p, False) < ws


def test_workspace_grows_with_slice_and_batch():
    a = _lib.workspace_size(_lib.make_params(8192, 4096, 128256, 0, vocab_slice=2048), True)
    b = _lib.workspace_size(_lib.make_params(8192, 4096, 128256, 0, vocab_slice=8192), True)
    c = _lib.workspace_size(_lib.make_params(16384, 4096, 128256, 0, vocab_slice=8192), True)
    assert a < b < c


def fwd(p, x=FAKE, w=FAKE, bias=None, t=FAKE, loss=FAKE, lse=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return _lib.forward(p, x, w, bias, t, loss, lse, None, ws, ws_bytes, None)


def bwd(p, x=FAKE, w=FAKE, bias=None, t=FAKE, lse=FAKE, dx=FAKE, dw=FAKE, db=None, ws=FAKE,
        ws_bytes=1 << 40):
    return _lib.backward(p, x, w, bias, t, lse, None, dx, dw, db, ws, ws_bytes, None)


def fused(p, ws_bytes=1 << 40, **kw):
    args = dict(x=FAKE, w=FAKE, bias=None, t=FAKE, loss=FAKE, lse=FAKE, dx=FAKE, dw=FAKE, db=None,
                ws=FAKE)
    args.update(kw)
    return _lib.fused_fwd_bwd(p, args["x"], args["w"], args["bias"], args["t"], args["loss"],
                              args["lse"], args["dx"], args["dw"], args["db"], args["ws"], ws_bytes,
                              None)


def stored(p, ws_bytes=1 << 40, **kw):
    args = dict(x=FAKE, w=FAKE, bias=None, t=FAKE, loss=FAKE, lse=FAKE, dx=FAKE, dw=FAKE, db=None,
                ws=FAKE)
    args.update(kw)
    return _lib.fused_fwd_bwd_stored(p, args["x"], args["w"], args["bias"], args["t"], args["loss"],
                                     args["lse"], args["dx"], args["dw"], args["db"], args["ws"],
                                     ws_bytes, None)


INVALID = _lib.FLCE_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("call", ["forward", "backward", "fused", "stored"])
def test_host_validation(lib, call):
    f = {"forward": fwd, "backward": bwd, "fused": fused, "stored": stored}[call]
    assert f(P(d=12)) == INVALID                    # D not a multiple of 8
    assert f(P(v=0)) == INVALID
    assert f(P(n=-5)) == INVALID
    assert f(P(dtype=3)) == INVALID
    assert f(P(label_smoothing=2.0)) == INVALID
    assert f(P(reduction=7)) == INVALID
    assert f(P(softcap=float("nan"))) == INVALID
    assert f(P(lse_square_scale=float("inf"))) == INVALID
    assert f(P(), w=None) == INVALID                # missing weight
    assert f(P(), x=None) == INVALID                # missing x with n > 0
    assert f(P(), t=None) == INVALID                # missing targets
    assert f(P(), w=FAKE + 8) == INVALID            # weight not 16-byte aligned
    assert f(P(), ws=FAKE + 64) == INVALID          # workspace not 256-byte aligned
    assert f(P(), ws=None) == INVALID
    assert f(P(), ws_bytes=16) == _lib.FLCE_ERR_WORKSPACE_TOO_SMALL
    need = (_lib.stored_workspace_size(P()) if call == "stored"
            else _lib.workspace_size(P(), call != "forward"))
    assert f(P(), ws_bytes=need - 1) == _lib.FLCE_ERR_WORKSPACE_TOO_SMALL
    if call == "forward":
        assert f(P(), loss=None) == INVALID
        assert f(P(), lse=None) == INVALID
    else:
        assert f(P(), dw=None) == INVALID
        assert f(P(), dx=FAKE + 4) == INVALID
        assert f(P(), bias=FAKE, db=None) == INVALID   # bias without a place for its gradient


def test_backward_refuses_reduction_none(lib):
    p = P(reduction=2)
    assert bwd(p) == _lib.FLCE_ERR_UNSUPPORTED
    assert fused(p) == _lib.FLCE_ERR_UNSUPPORTED
    assert stored(p) == _lib.FLCE_ERR_UNSUPPORTED


def test_null_params(lib):
    pp = ctypes.POINTER(_lib.Params)()
    assert lib.flce_forward(pp, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None) == INVALID
    assert lib.flce_check_status(None, None) == INVALID


# ------------------------------------------------- cross-entropy on logits

def ce_fwd(p, r=FAKE, t=FAKE, loss=FAKE, lse=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return _lib.ce_forward(p, r, t, loss, lse, None, ws, ws_bytes, None)


def ce_bwd(p, r=FAKE, t=FAKE, lse=FAKE, g=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return _lib.ce_backward(p, r, t, lse, None, g, ws, ws_bytes, None)


def ce_fused(p, r=FAKE, t=FAKE, loss=FAKE, lse=FAKE, g=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return _lib.ce_fused_fwd_bwd(p, r, t, loss, lse, g, ws, ws_bytes, None)


def test_ce_workspace_is_per_row_only(lib):
    p = _lib.make_params(65536, 8, 128256, _lib.DTYPE_BF16)
    ws = _lib.ce_workspace_size(p)
    # status word, row map, row losses, predicted tokens, hits and their block sums
    assert 0 < ws < 20 * 65536 + 8192
    # the hidden size and the slice width play no part
    assert _lib.ce_workspace_size(_lib.make_params(65536, 12, 128256, _lib.DTYPE_BF16,
                                                   vocab_slice=-3)) == ws
    for bad in (P(v=0), P(n=-1), P(dtype=7), P(label_smoothing=1.5), P(softcap=-1.0),
                P(lse_square_scale=float("nan")), P(reduction=5)):
        assert _lib.ce_workspace_size(bad) == 0
    assert lib.flce_ce_workspace_size(None) == 0


@pytest.mark.parametrize("call", ["forward", "backward", "fused"])
def test_ce_host_validation(lib, call):
    f = {"forward": ce_fwd, "backward": ce_bwd, "fused": ce_fused}[call]
    bf = dict(dtype=_lib.DTYPE_BF16)
    assert f(P(v=0)) == INVALID
    assert f(P(n=-5)) == INVALID
    assert f(P(dtype=3)) == INVALID
    assert f(P(label_smoothing=2.0)) == INVALID
    assert f(P(reduction=7)) == INVALID
    assert f(P(), r=None) == INVALID                 # missing logits with n > 0
    assert f(P(), t=None) == INVALID
    assert f(P(**bf), r=FAKE + 1) == INVALID         # bf16 logits not 2-byte aligned
    assert f(P(), r=FAKE + 2) == INVALID             # fp32 logits not 4-byte aligned
    assert f(P(), t=FAKE + 2) == INVALID
    assert f(P(), ws=FAKE + 64) == INVALID
    assert f(P(), ws=None) == INVALID
    need = _lib.ce_workspace_size(P())
    assert f(P(), ws_bytes=need - 1) == _lib.FLCE_ERR_WORKSPACE_TOO_SMALL
    assert f(P(), lse=None) == INVALID
    if call != "forward":
        assert f(P(), g=None) == INVALID             # nowhere to write dL/dlogits
        assert f(P(), g=FAKE + 8) == INVALID         # splits rows differently from the logits
        assert f(P(**bf), g=FAKE + 2) == INVALID
        assert f(P(reduction=2)) == _lib.FLCE_ERR_UNSUPPORTED
    if call != "backward":
        assert f(P(), loss=None) == INVALID


def test_token_chunk_and_dw_bf16_params(lib):
    assert _lib.workspace_size(P(token_chunk=-1), True) == 0
    assert _lib.workspace_size(P(dw_bf16=2), True) == 0
    assert fwd(P(token_chunk=-256)) == INVALID
    assert bwd(P(dw_bf16=-1)) == INVALID
    # the backward workspace is sized by the chunk, not by the batch
    full = _lib.workspace_size(_lib.make_params(65536, 4096, 128256, _lib.DTYPE_BF16), True)
    chunked = _lib.workspace_size(_lib.make_params(65536, 4096, 128256, _lib.DTYPE_BF16,
                                                   token_chunk=16384), True)
    assert chunked < full / 2
    a = _lib.workspace_size(_lib.make_params(32768, 4096, 128256, _lib.DTYPE_BF16,
                                             token_chunk=8192), True)
    b = _lib.workspace_size(_lib.make_params(65536, 4096, 128256, _lib.DTYPE_BF16,
                                             token_chunk=8192), True)
    # doubling N adds only the per-row and packed-row parts (forward partials, packed X)
    assert b - a < 32768 * (4096 * 2 + 4 * 600) * 1.1
    # a chunk larger than the batch is the whole batch
    assert (_lib.workspace_size(P(token_chunk=1 << 20), True) == _lib.workspace_size(P(), True))


def test_class_weight_params(lib):
    assert fwd(P(class_weight=FAKE + 2)) == INVALID            # weights not 4-byte aligned
    # the logits path has no class weights
    assert ce_fwd(P(class_weight=FAKE)) == _lib.FLCE_ERR_UNSUPPORTED
    assert ce_fused(P(class_weight=FAKE)) == _lib.FLCE_ERR_UNSUPPORTED
    assert _lib.ce_workspace_size(P(class_weight=FAKE)) == 0
    # weights change no buffer size
    assert _lib.workspace_size(P(class_weight=FAKE), True) == _lib.workspace_size(P(), True)


def test_size_limits(lib):
    """The documented limits (N <= 2^22, D <= 2^20, V < 2^31; slice and chunk
    widths) are accepted at the limit and refused one step beyond it."""
    def ws(**kw):
        return _lib.workspace_size(P(**kw), True)
    assert ws(n=1 << 22) > 0 and ws(n=(1 << 22) + 1) == 0
    assert ws(d=1 << 20) > 0 and ws(d=(1 << 20) + 8) == 0
    assert ws(v=(1 << 31) - 1) > 0 and ws(v=1 << 31) == 0
    assert ws(n=1 << 22, d=1 << 20, v=1 << 16) > 0
    assert ws(n=1 << 22, v=(1 << 31) - 1) == 0          # 2^37 forward tiles
    assert ws(vocab_slice=1 << 20) > 0 and ws(vocab_slice=(1 << 20) + 1) == 0
    assert ws(token_chunk=1 << 22) > 0 and ws(token_chunk=(1 << 22) + 1) == 0
    assert _lib.stored_workspace_size(P(n=1 << 22)) > 0
    assert _lib.stored_workspace_size(P(n=(1 << 22) + 1)) == 0
    assert _lib.ce_workspace_size(P(n=1 << 22, v=(1 << 31) - 1)) > 0
    assert _lib.ce_workspace_size(P(n=(1 << 22) + 1)) == 0
    # bf16 K-major pitches: the stored schedule's G rows span V (rounded up to
    # 256, + 128): 510 * pitch + 112 < 2^31 holds up to V = 4210432
    bf = _lib.DTYPE_BF16
    assert _lib.stored_workspace_size(P(dtype=bf, v=4210432)) > 0
    assert _lib.stored_workspace_size(P(dtype=bf, v=4210433)) == 0
    assert _lib.stored_workspace_size(P(v=4210561)) > 0            # fp32: 64-bit addressing
    assert ws(dtype=bf, n=1 << 22) > 0 and ws(dtype=bf, vocab_slice=1 << 20, v=1 << 21) > 0
    # the entry point refuses it on the host too, before any HIP call
    st = lib.flce_fused_fwd_bwd_stored(ctypes.byref(P(dtype=bf, v=4210433)), FAKE, FAKE, None, FAKE,
                                       FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None)
    assert st == _lib.FLCE_ERR_INVALID_ARGUMENT


def test_loss_module_options():
    """The module form validates its options on construction (no GPU)."""
    import torch
    from linear_cross_entropy_bf16_amd import LinearCrossEntropyLoss
    m = LinearCrossEntropyLoss(label_smoothing=0.1, softcap=30.0, reduction="sum",
                               class_weight=torch.ones(7))
    assert "softcap=30.0" in repr(m) and m.class_weight.shape == (7,)
    assert "class_weight" not in m.state_dict()      # not saved with a model
    with pytest.raises(ValueError):
        LinearCrossEntropyLoss(reduction="avg")
    with pytest.raises(ValueError):
        LinearCrossEntropyLoss(label_smoothing=1.5)


def test_binding_refuses_host_tensors():
    """Every entry point of the binding needs GPU tensors; host tensors are
    refused before the library is called."""
    import torch
    from linear_cross_entropy_bf16_amd import api
    x, w, t = torch.zeros(4, 8), torch.zeros(16, 8), torch.zeros(4, dtype=torch.int32)
    for call in (lambda: api.forward(x, w, t), lambda: api.fused_fwd_bwd(x, w, t),
                 lambda: api.linear_cross_entropy(x, w, t),
                 lambda: api.cross_entropy(torch.zeros(4, 16), t),
                 lambda: api.cross_entropy_fused_fwd_bwd(torch.zeros(4, 16), t)):
        with pytest.raises(ValueError):
            call()


def test_binding_checks_caller_buffers():
    """Caller-supplied output buffers and workspace must match what the
    library writes (shape, dtype, device, contiguity): a short or mistyped
    buffer is refused on the host instead of being overrun on the device."""
    import torch
    from linear_cross_entropy_bf16_amd import api
    cpu = torch.device("cpu")
    api._check_buffer(torch.zeros(4, 8), "dx", (4, 8), torch.float32, cpu)
    bad = [(torch.zeros(3, 8), (4, 8), torch.float32),               # short
           (torch.zeros(4, 8), (4, 8), torch.bfloat16),              # mistyped (bf16 dW requested)
           (torch.zeros(8, 4).t(), (4, 8), torch.float32),           # not contiguous
           (torch.zeros(32), (4, 8), torch.float32)]                 # flat
    for t, shape, dtype in bad:
        with pytest.raises(ValueError):
            api._check_buffer(t, "dx", shape, dtype, cpu)
    with pytest.raises(ValueError):
        api._check_buffer(torch.zeros(4, 8), "dx", (4, 8), torch.float32, torch.device("cuda", 0))


def test_noalloc_entry_point_validates_on_the_host(lib):
    """flce_fused_fwd_bwd_noalloc refuses, before any HIP call, what the
    workspace call refuses and any problem whose workspace exceeds the
    library's scratch array."""
    bf = _lib.DTYPE_BF16

    def call(p, **kw):
        a = dict(x=FAKE, w=FAKE, bias=None, t=FAKE, loss=FAKE, lse=FAKE, dx=FAKE, dw=FAKE, db=None)
        a.update(kw)
        return lib.flce_fused_fwd_bwd_noalloc(ctypes.byref(p), a["x"], a["w"], a["bias"], a["t"], a["loss"],
                                              a["lse"], a["dx"], a["dw"], a["db"], None)

    big = P(dtype=bf, n=4096, d=2048, v=32000)
    assert _lib.workspace_size(big, True) > _lib.NOALLOC_MAX_BYTES
    assert call(big) == _lib.FLCE_ERR_WORKSPACE_TOO_SMALL
    assert call(P(dtype=bf, reduction="none")) == _lib.FLCE_ERR_UNSUPPORTED
    assert call(P(dtype=bf, d=12)) == _lib.FLCE_ERR_INVALID_ARGUMENT
    assert call(P(dtype=bf), dx=FAKE + 4) == _lib.FLCE_ERR_INVALID_ARGUMENT      # misaligned dX
    assert call(P(dtype=bf), bias=FAKE) == _lib.FLCE_ERR_INVALID_ARGUMENT        # bias without dbias
