"""Host-side checks of the C ABI that need no GPU: the library loads, every
function include/fp8bl.h declares is exported, and argument errors come back
as status codes before anything touches a device."""

import ctypes

import pytest

from block_scaled_fp8_linear_amd import _lib as L


@pytest.fixture(scope="module")
def lib():
    return L.load()


def test_header_symbols_exported(lib):
    names = L.header_functions()
    assert set(names) == {
        "fp8_block_abi_version", "fp8_block_status_string", "fp8_block_device_supported",
        "fp8_block_dequant", "fp8_block_linear_workspace_size", "fp8_block_linear",
        "fp8_block_linear_ex", "fp8_block_quantize", "fp8_block_quantize_bf16",
        "fp8_block_mlp_gate_up", "fp8_block_mlp_gate_up_ex", "fp8_act_quantize", "fp8_block_linear_w8a8_workspace_size",
        "fp8_block_linear_w8a8", "fp8_block_linear_w8a8_ex", "fp8_block_linear_w8a8_bf16", "fp8_block_stream_read",
        "fp8_block_linear_noalloc",
    }
    for name in names:
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_version_and_status_strings(lib):
    assert L.abi_version() == 1
    for st in range(6):
        s = L.status_string(st)
        assert s.startswith("FP8BL_")
    assert L.status_string(99) == "FP8BL_UNKNOWN_STATUS"


def test_workspace_sizes():
    assert L.workspace_size(0, 10, 16) == 0
    assert L.workspace_size(4, 0, 16) == 0
    assert L.workspace_size(4, 8, 15) == 0          # invalid K -> 0, never fails
    for m, n, k in [(1, 8000, 8192), (16, 8000, 8192), (512, 5120, 5120), (64, 384, 256),
                    (16384, 3072, 3072), (3, 100, 4096), (512, 5120, 25600)]:
        ws = L.workspace_size(m, n, k)
        assert ws % 256 == 0
        assert ws <= 8 * (m * n + 64) * 4 + 256     # <= 8 splits, slabs padded to 64 floats


FAKE = 1 << 20  # a 16-byte aligned non-null address; never dereferenced here


@pytest.mark.parametrize("args,status", [
    # (x, q, s, y, m, n, k, ws, ws_bytes, path)
    ((FAKE, FAKE, FAKE, 4 * FAKE, 4, 8, 15, 0, 0, 0), L.FP8BL_INVALID_ARG),    # K % 16
    ((FAKE, FAKE, FAKE, 4 * FAKE, 4, 8, 0, 0, 0, 0), L.FP8BL_INVALID_ARG),     # K == 0
    ((FAKE, FAKE, FAKE, 4 * FAKE, -1, 8, 16, 0, 0, 0), L.FP8BL_INVALID_ARG),   # M < 0
    ((FAKE, FAKE, FAKE, 4 * FAKE, 4, -8, 16, 0, 0, 0), L.FP8BL_INVALID_ARG),   # N < 0
    ((0, FAKE, FAKE, 4 * FAKE, 4, 8, 16, 0, 0, 0), L.FP8BL_INVALID_ARG),       # null x
    ((FAKE, 0, FAKE, 4 * FAKE, 4, 8, 16, 0, 0, 0), L.FP8BL_INVALID_ARG),       # null q
    ((FAKE, FAKE, 0, 4 * FAKE, 4, 8, 16, 0, 0, 0), L.FP8BL_INVALID_ARG),       # null s
    ((FAKE, FAKE, FAKE, 0, 4, 8, 16, 0, 0, 0), L.FP8BL_INVALID_ARG),           # null y
    ((FAKE + 2, FAKE, FAKE, 4 * FAKE, 4, 8, 16, 0, 0, 0), L.FP8BL_ALIGNMENT),  # x misaligned
    ((FAKE, FAKE + 8, FAKE, 4 * FAKE, 4, 8, 16, 0, 0, 0), L.FP8BL_ALIGNMENT),  # q misaligned
    ((FAKE, FAKE, FAKE + 2, 4 * FAKE, 4, 8, 16, 0, 0, 0), L.FP8BL_ALIGNMENT),  # s misaligned
    ((FAKE, FAKE, FAKE, 4 * FAKE + 4, 4, 8, 16, 0, 0, 0), L.FP8BL_ALIGNMENT),  # y misaligned
    ((FAKE, FAKE, FAKE, FAKE, 4, 8, 16, 0, 0, 0), L.FP8BL_INVALID_ARG),        # y overlaps x
    ((FAKE, FAKE, FAKE, 4 * FAKE, 4, 8, 16, 0, 0, 7), L.FP8BL_INVALID_ARG),    # bad path
    ((FAKE, FAKE, FAKE, 4 * FAKE, 1 << 31, 8, 16, 0, 0, 0), L.FP8BL_INVALID_ARG),  # M too big
    ((FAKE, FAKE, FAKE, 4 * FAKE, 1, 8, (1 << 20) + 16, 0, 0, 0), L.FP8BL_INVALID_ARG),  # K too big
    ((FAKE, FAKE, FAKE, 4 * FAKE, 1 << 19, 1 << 16, 1 << 16, 0, 0, 0), L.FP8BL_INVALID_ARG),  # M*K = 2^35
    ((FAKE, FAKE, FAKE, 4 * FAKE, 0, 8, 16, 0, 0, 0), L.FP8BL_OK),             # empty M: no-op
    ((FAKE, FAKE, FAKE, 4 * FAKE, 4, 0, 16, 0, 0, 0), L.FP8BL_OK),             # empty N: no-op
    ((0, 0, 0, 0, 0, 0, 16, 0, 0, 0), L.FP8BL_OK),                             # empty, null ok
])
def test_linear_argument_errors(lib, args, status):
    x, q, s, y, m, n, k, ws, wsb, path = args
    assert L.linear_raw(x, q, s, y, m, n, k, ws, wsb, path) == status


@pytest.mark.parametrize("args,status", [
    # (x, q, s, y, m, n, k)
    ((FAKE, FAKE, FAKE, 4 * FAKE, 4, 8, 15), L.FP8BL_INVALID_ARG),        # K % 16
    ((0, FAKE, FAKE, 4 * FAKE, 4, 8, 16), L.FP8BL_INVALID_ARG),           # null x
    ((FAKE, FAKE, FAKE, 0, 4, 8, 16), L.FP8BL_INVALID_ARG),               # null y
    ((FAKE + 2, FAKE, FAKE, 4 * FAKE, 4, 8, 16), L.FP8BL_ALIGNMENT),      # x misaligned
    ((FAKE, FAKE, FAKE, FAKE, 4, 8, 16), L.FP8BL_INVALID_ARG),            # y overlaps x
    ((FAKE, FAKE, FAKE, 4 * FAKE, 0, 8, 16), L.FP8BL_OK),                 # empty M: no-op
    ((0, 0, 0, 0, 4, 0, 16), L.FP8BL_OK),                                 # empty N, null ok
    # partials of 768 x 8192 x 65536 (split K) exceed the 64 MiB scratch
    ((1 << 40, 1 << 41, 1 << 42, 1 << 43, 768, 8192, 65536), L.FP8BL_WORKSPACE),
])
def test_linear_noalloc_argument_errors(lib, args, status):
    """The allocation-free linear checks its arguments like fp8_block_linear and
    rejects a shape whose split-K partials exceed its scratch, all before any
    HIP call (none of these touches a device)."""
    assert L.linear_noalloc_raw(*args) == status


def test_noalloc_scratch_size_matches_header():
    text = open(L.HEADER_PATH).read()
    assert "#define FP8BL_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)" in text
    assert L.NOALLOC_SCRATCH_BYTES == 64 * 1024 * 1024


@pytest.mark.parametrize("args,status", [
    # (x, qg, sg, qu, su, h, m, n, k)
    ((FAKE, 2 * FAKE, 3 * FAKE, 4 * FAKE, 5 * FAKE, 8 * FAKE, 4, 8, 15), L.FP8BL_INVALID_ARG),
    ((FAKE, 2 * FAKE, 3 * FAKE, 0, 5 * FAKE, 8 * FAKE, 4, 8, 16), L.FP8BL_INVALID_ARG),       # null q_up
    ((FAKE, 2 * FAKE, 3 * FAKE, 4 * FAKE, 0, 8 * FAKE, 4, 8, 16), L.FP8BL_INVALID_ARG),       # null s_up
    ((FAKE, 0, 3 * FAKE, 4 * FAKE, 5 * FAKE, 8 * FAKE, 4, 8, 16), L.FP8BL_INVALID_ARG),       # null q_gate
    ((FAKE, 2 * FAKE, 3 * FAKE, 4 * FAKE + 8, 5 * FAKE, 8 * FAKE, 4, 8, 16), L.FP8BL_ALIGNMENT),
    ((FAKE, 2 * FAKE, 3 * FAKE, 4 * FAKE, 5 * FAKE + 2, 8 * FAKE, 4, 8, 16), L.FP8BL_ALIGNMENT),
    ((FAKE, 2 * FAKE, 3 * FAKE, 4 * FAKE, 5 * FAKE, 4 * FAKE, 4, 8, 16), L.FP8BL_INVALID_ARG),  # h over q_up
    ((FAKE, 2 * FAKE, 3 * FAKE, 4 * FAKE, 5 * FAKE, 5 * FAKE, 4, 8, 16), L.FP8BL_INVALID_ARG),  # h over s_up
    ((FAKE, 2 * FAKE, 3 * FAKE, 4 * FAKE, 5 * FAKE, 8 * FAKE, 1, 8, (1 << 20) + 16), L.FP8BL_INVALID_ARG),
    ((FAKE, 2 * FAKE, 3 * FAKE, 4 * FAKE, 5 * FAKE, 8 * FAKE, 0, 8, 16), L.FP8BL_OK),          # empty
    ((0, 0, 0, 0, 0, 0, 4, 0, 16), L.FP8BL_OK),                                               # empty N
])
def test_mlp_gate_up_argument_errors(lib, args, status):
    assert L.mlp_gate_up_raw(*args) == status
    # the kernel-choosing form checks the same way on each path that takes the shape
    for path in (L.PATH_AUTO, L.PATH_TILED) + ((L.PATH_LARGE,) if args[7] % 8 == 0 else ()):
        assert L.mlp_gate_up_ex_raw(*args, path) == status


@pytest.mark.parametrize("n,path,status", [
    (8, 2, L.FP8BL_INVALID_ARG),          # SKINNY is not a gate/up kernel
    (8, 4, L.FP8BL_INVALID_ARG),          # unknown path
    (8, -1, L.FP8BL_INVALID_ARG),
    (12, L.PATH_LARGE, L.FP8BL_INVALID_ARG),   # the large kernel needs N % 8 == 0
    (1 << 21, L.PATH_LARGE, L.FP8BL_INVALID_ARG),
    (12, L.PATH_TILED, L.FP8BL_OK),
])
def test_mlp_gate_up_ex_paths(lib, n, path, status):
    """Path checks come before any device work (M = 0 here: a valid call
    returns at once)."""
    args = (FAKE, 2 * FAKE, 3 * FAKE, 4 * FAKE, 5 * FAKE, 8 * FAKE, 0, n, 16)
    assert L.mlp_gate_up_ex_raw(*args, path) == status


@pytest.mark.parametrize("m,k,xoff,qoff,soff,status", [
    (4, 15, 0, 0, 0, L.FP8BL_INVALID_ARG),
    (-1, 16, 0, 0, 0, L.FP8BL_INVALID_ARG),
    (4, 0, 0, 0, 0, L.FP8BL_INVALID_ARG),
    (4, 16, 2, 0, 0, L.FP8BL_ALIGNMENT),
    (4, 16, 0, 8, 0, L.FP8BL_ALIGNMENT),
    (4, 16, 0, 0, 2, L.FP8BL_ALIGNMENT),
    (0, 16, 0, 0, 0, L.FP8BL_OK),
])
def test_act_quantize_argument_errors(lib, m, k, xoff, qoff, soff, status):
    assert L.act_quantize_raw(FAKE + xoff, 8 * FAKE + qoff, 16 * FAKE + soff, m, k) == status
    assert L.act_quantize_raw(FAKE, FAKE, 16 * FAKE, 4, 16) == L.FP8BL_INVALID_ARG   # xq over x
    assert L.act_quantize_raw(0, 8 * FAKE, 16 * FAKE, 4, 16) == L.FP8BL_INVALID_ARG


@pytest.mark.parametrize("args,status", [
    # (xq, xs, q, s, y, m, n, k, ws, ws_bytes)
    ((FAKE, 2 * FAKE, 3 * FAKE, 4 * FAKE, 8 * FAKE, 4, 8, 15, 0, 0), L.FP8BL_INVALID_ARG),
    ((0, 2 * FAKE, 3 * FAKE, 4 * FAKE, 8 * FAKE, 4, 8, 16, 0, 0), L.FP8BL_INVALID_ARG),
    ((FAKE, 0, 3 * FAKE, 4 * FAKE, 8 * FAKE, 4, 8, 16, 0, 0), L.FP8BL_INVALID_ARG),
    ((FAKE + 4, 2 * FAKE, 3 * FAKE, 4 * FAKE, 8 * FAKE, 4, 8, 16, 0, 0), L.FP8BL_ALIGNMENT),
    ((FAKE, 2 * FAKE + 2, 3 * FAKE, 4 * FAKE, 8 * FAKE, 4, 8, 16, 0, 0), L.FP8BL_ALIGNMENT),
    ((FAKE, 2 * FAKE, 3 * FAKE, 4 * FAKE, 2 * FAKE, 4, 8, 16, 0, 0), L.FP8BL_INVALID_ARG),   # y over xs
    ((FAKE, 2 * FAKE, 3 * FAKE, 4 * FAKE, 8 * FAKE, 1, 8, (1 << 20) + 16, 0, 0), L.FP8BL_INVALID_ARG),
    ((FAKE, 2 * FAKE, 3 * FAKE, 4 * FAKE, 8 * FAKE, 0, 8, 16, 0, 0), L.FP8BL_OK),
])
def test_w8a8_argument_errors(lib, args, status):
    assert L.linear_w8a8_raw(*args) == status


def test_w8a8_workspace_rules(lib):
    assert L.w8a8_workspace_size(0, 8, 16) == 0
    assert L.w8a8_workspace_size(4, 8, 15) == 0
    m, n, k = 512, 5120, 5120
    need = L.w8a8_workspace_size(m, n, k)
    act = -(-m * k // 256) * 256 + -(-(k // 128) * m * 4 // 256) * 256
    assert need >= act and need % 256 == 0
    assert need <= act + 8 * (m * n + 64) * 4 + 256
    x, q, s, y = FAKE, 64 * FAKE, 96 * FAKE, 128 * FAKE
    # the bf16 entry always needs the workspace (it holds the quantized x)
    assert L.linear_w8a8_bf16_raw(x, q, s, y, 4, 8, 16, 0, 0) == L.FP8BL_WORKSPACE
    assert L.linear_w8a8_bf16_raw(x, q, s, y, m, n, k, 256 * FAKE, need - 256) == L.FP8BL_WORKSPACE
    assert L.linear_w8a8_bf16_raw(x, q, s, y, m, n, k, 256 * FAKE + 16, need) == L.FP8BL_ALIGNMENT
    assert L.linear_w8a8_bf16_raw(x, q, s, y, m, n, k, y, need) == L.FP8BL_INVALID_ARG
    # the pre-quantized entry needs it only for split-K shapes
    assert L.linear_w8a8_raw(x, 32 * FAKE, q, s, y, m, n, k, 0, 0) == L.FP8BL_WORKSPACE


def test_linear_workspace_errors(lib):
    # a shape that needs a split-K workspace on the skinny path
    m, n, k = 16, 64, 8192
    need = L.workspace_size(m, n, k)
    assert need > 0
    x, q, s, y = FAKE, 8 * FAKE, 16 * FAKE, 24 * FAKE
    assert L.linear_raw(x, q, s, y, m, n, k, 0, 0, L.PATH_SKINNY) == L.FP8BL_WORKSPACE
    assert L.linear_raw(x, q, s, y, m, n, k, 32 * FAKE, 1024, L.PATH_SKINNY) == L.FP8BL_WORKSPACE
    assert L.linear_raw(x, q, s, y, m, n, k, 32 * FAKE, 1024, L.PATH_TILED) == L.FP8BL_WORKSPACE
    assert L.linear_raw(x, q, s, y, m, n, k, 32 * FAKE + 16, need, L.PATH_SKINNY) == L.FP8BL_ALIGNMENT
    assert L.linear_raw(x, q, s, y, m, n, k, y, need, L.PATH_SKINNY) == L.FP8BL_INVALID_ARG


def test_valid_call_without_gpu_reports_device_status(lib):
    """With valid arguments the gate runs; on a machine without a gfx950 it
    must answer with a status, not crash. (With a GPU present this test is
    not meaningful and is skipped.)"""
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st = L.linear_raw(FAKE, 8 * FAKE, 16 * FAKE, 24 * FAKE, 4, 8, 16, 0, 0, L.PATH_AUTO)
    assert st in (L.FP8BL_HIP_ERROR, L.FP8BL_UNSUPPORTED_DEVICE)
    assert L.device_supported(0) is False


@pytest.mark.parametrize("n,k,qoff,soff,woff,status", [
    (8, 15, 0, 0, 0, L.FP8BL_INVALID_ARG),
    (-1, 16, 0, 0, 0, L.FP8BL_INVALID_ARG),
    (8, 16, 8, 0, 0, L.FP8BL_ALIGNMENT),
    (8, 16, 0, 2, 0, L.FP8BL_ALIGNMENT),
    (8, 16, 0, 0, 4, L.FP8BL_ALIGNMENT),
    (0, 16, 0, 0, 0, L.FP8BL_OK),
])
def test_dequant_and_quantize_argument_errors(lib, n, k, qoff, soff, woff, status):
    q, s, w = FAKE + qoff, 8 * FAKE + soff, 16 * FAKE + woff
    assert L.dequant_raw(q, s, w, n, k) == status
    # quantize(w, q, s): w is the fp32 (or bf16) input
    assert L.quantize_raw(w, q, s, n, k) == status
    assert L.quantize_bf16_raw(w, q, s, n, k) == status
    # overlapping output
    assert L.dequant_raw(FAKE, 8 * FAKE, FAKE, 8, 16) == L.FP8BL_INVALID_ARG


def test_element_count_limit_is_strict(lib):
    # 2^35 elements would wrap the kernels' 32-bit 8-element chunk index
    n, k = 1 << 19, 1 << 16
    assert L.dequant_raw(FAKE, 8 * FAKE, 16 * FAKE, n, k) == L.FP8BL_INVALID_ARG
    assert L.quantize_raw(FAKE, 8 * FAKE, 16 * FAKE, n, k) == L.FP8BL_INVALID_ARG
    assert L.act_quantize_raw(FAKE, 8 * FAKE, 16 * FAKE, n, k) == L.FP8BL_INVALID_ARG


@pytest.mark.parametrize("args,status", [
    # (buf, bytes, sink, blocks)
    ((FAKE, 0, 0, 0), L.FP8BL_OK),                          # empty read: no-op
    ((0, 1 << 20, 64 * FAKE, 2048), L.FP8BL_INVALID_ARG),     # null buffer
    ((FAKE, 1 << 20, 0, 2048), L.FP8BL_INVALID_ARG),          # null sink
    ((FAKE, 1 << 20, 64 * FAKE, 0), L.FP8BL_INVALID_ARG),     # no workgroups
    ((FAKE, 1 << 20, 64 * FAKE, 65537), L.FP8BL_INVALID_ARG),
    ((FAKE, (1 << 20) + 8, 64 * FAKE, 2048), L.FP8BL_INVALID_ARG),   # not a multiple of 16
    ((FAKE + 8, 1 << 20, 64 * FAKE, 2048), L.FP8BL_ALIGNMENT),
    ((FAKE, 1 << 20, 64 * FAKE + 2, 2048), L.FP8BL_ALIGNMENT),
    ((FAKE, 1 << 20, FAKE + 4096, 2048), L.FP8BL_INVALID_ARG),       # sink inside the buffer
])
def test_stream_read_argument_errors(lib, args, status):
    assert L.stream_read_raw(*args) == status


@pytest.mark.parametrize("n,path,status", [
    (8, 2, L.FP8BL_INVALID_ARG),          # SKINNY is not a W8A8 kernel
    (8, 4, L.FP8BL_INVALID_ARG),
    (12, L.PATH_LARGE, L.FP8BL_INVALID_ARG),   # the 192x256-tile kernel needs N % 8 == 0
    (1 << 21, L.PATH_LARGE, L.FP8BL_INVALID_ARG),
    (12, L.PATH_TILED, L.FP8BL_OK),
    (16, L.PATH_LARGE, L.FP8BL_OK),
])
def test_w8a8_ex_paths(lib, n, path, status):
    """Path checks of the kernel-choosing W8A8 call come before any device
    work (M = 0: a valid call returns at once)."""
    assert L.linear_w8a8_ex_raw(FAKE, 2 * FAKE, 3 * FAKE, 4 * FAKE, 8 * FAKE, 0, n, 16, 0, 0,
                                path) == status


def test_w8a8_activation_scales_over_4gib_rejected(lib):
    """The W8A8 GEMMs address the activation scales with 32-bit buffer
    offsets: 4 * m * ceil(k/128) bytes must stay below 2^32. With k = 16 that
    is m < 2^30, a shape the other limits (m*k, m*n < 2^35) still allow."""
    m, n, k = 1 << 30, 8, 16
    for path in (L.PATH_AUTO, L.PATH_TILED, L.PATH_LARGE):
        assert L.linear_w8a8_ex_raw(FAKE, 2 * FAKE, 3 * FAKE, 4 * FAKE, 8 * FAKE, m, n, k, 0, 0,
                                    path) == L.FP8BL_INVALID_ARG
    assert L.linear_w8a8_bf16_raw(FAKE, 3 * FAKE, 4 * FAKE, 8 * FAKE, m, n, k, 0, 0) == \
        L.FP8BL_INVALID_ARG
