"""The C-ABI library loads, exports every function include/fa2.h declares, and
reports every argument error before any HIP call (so this runs without a GPU)."""
import os
import re

import pytest

import attention_forward_fa2_amd as fa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa2.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa2_\w+)\s*\(", text, flags=re.M)))


def header_status_codes():
    text = open(HEADER).read()
    return {int(v): k for k, v in re.findall(r"(FA2_\w+)\s*=\s*(\d+)", text)}


def test_library_loads_and_exports_all_declared_symbols():
    lib = fa2.load_library()
    declared = header_functions()
    assert declared == sorted(fa2.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), f"{name} not exported"
    # and the export table itself, read with nm
    out = os.popen(f"nm -D --defined-only {fa2.LIB_PATH}").read()
    for name in declared:
        assert re.search(rf"\bT {name}\b", out), f"{name} missing from the dynamic symbol table"


def test_status_codes_match_header():
    codes = header_status_codes()
    assert codes == fa2.STATUS_NAMES
    for code in codes:
        msg = fa2.fa2_strerror(code)
        assert isinstance(msg, str) and msg
    assert fa2.fa2_strerror(99) == "unknown status"


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


# The tests below hand fake device addresses to fa2_fwd and rely on the
# argument checks to stop before any launch. Where a GPU is visible a bug in
# those checks could launch a kernel on them, so the module runs only where none is.
pytestmark = pytest.mark.skipif(_gpu_visible(), reason="fake device pointers are passed only where no GPU exists")

# Fake, never-dereferenced device addresses: 16-byte aligned and far apart.
BASE = 1 << 40
GAP = 1 << 36
Q, K, V, O, L = (BASE + i * GAP for i in range(5))


def call(q=Q, k=K, v=V, o=O, lse=L, B=1, H=1, S=128, D=64, causal=0, scale=0.125):
    return fa2.fa2_fwd(q, k, v, o, lse, B, H, S, D, causal, scale, None)


@pytest.mark.parametrize("which", range(5))
def test_null_pointer(which):
    ptrs = [Q, K, V, O, L]
    ptrs[which] = None
    assert call(*ptrs) == 1


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(S=0), dict(B=-1), dict(D=32), dict(D=96),
                                dict(D=256), dict(causal=2), dict(causal=-1)])
def test_bad_shape(kw):
    assert call(**kw) == 2


@pytest.mark.parametrize("scale", [0.0, -0.125, float("inf"), float("nan"), -float("inf")])
def test_bad_scale(scale):
    assert call(scale=scale) == 3


@pytest.mark.parametrize("field,off", [("q", 8), ("k", 2), ("v", 4), ("o", 8), ("lse", 2)])
def test_misaligned(field, off):
    kw = {field: {"q": Q, "k": K, "v": V, "o": O, "lse": L}[field] + off}
    assert call(**kw) == 4


# Calls below always carry one error that is checked last (o aliasing q), so
# reaching FA2_ERR_ALIAS shows every earlier check passed, and no call here can
# ever reach a kernel launch with these fake pointers.
ALIAS, DEVICE, ARG = 8, 6, 9

def test_lse_needs_only_4_byte_alignment():
    assert call(lse=L + 4, o=Q) == ALIAS


def test_overflow():
    assert call(S=1 << 29, D=64) == 5          # row index plus a window side must stay below 2^31
    assert call(S=(1 << 29) - 1, D=128, o=Q) == ALIAS
    # tensors far beyond 2^31 elements are fine (64-bit addressing) ...
    assert call(B=64, H=64, S=1 << 20, D=128, o=Q) == ALIAS
    # ... but the grid must fit in 2^31 - 1 workgroups
    assert call(B=1 << 16, H=1 << 12, S=1 << 12, D=64) == 5


def test_valid_arguments_reach_the_alias_check():
    for D in (64, 128):
        for causal in (0, 1):
            assert call(D=D, causal=causal, o=Q) == ALIAS


def test_alias():
    assert call(o=Q) == ALIAS
    assert call(lse=V + 100 * 64 * 2 // 2 * 2) == ALIAS  # inside v
    assert call(o=K + 16) == ALIAS
    assert call(lse=O + 64) == ALIAS


def test_error_order():
    # null beats shape beats scale beats alignment beats overflow
    assert call(q=None, B=0, scale=-1.0) == 1
    assert call(B=0, scale=-1.0, q=Q + 2) == 2
    assert call(scale=-1.0, q=Q + 2) == 3
    assert call(q=Q + 2, S=1 << 29) == 4


def call_ex(q=Q, k=K, v=V, o=O, lse=L, B=1, H=4, H_kv=2, S=128, D=64, wl=-1, wr=-1, p=0.0, seed=0, offset=0,
            scale=0.125):
    return fa2.fa2_fwd_ex(q, k, v, o, lse, B, H, H_kv, S, D, wl, wr, p, seed, offset, scale, None)


CU = BASE + 5 * GAP


def call_varlen(q=Q, k=K, v=V, o=O, lse=L, cu=CU, nseq=3, total=300, max_seqlen=200, H=4, H_kv=1, D=128,
                wl=-1, wr=-1, p=0.0, seed=0, offset=0, scale=0.125):
    return fa2.fa2_fwd_varlen(q, k, v, o, lse, cu, nseq, total, max_seqlen, H, H_kv, D, wl, wr, p, seed, offset,
                              scale, None)


@pytest.mark.parametrize("which", range(5))
def test_ex_null_pointer(which):
    ptrs = [Q, K, V, O, L]
    ptrs[which] = None
    assert call_ex(*ptrs) == 1


@pytest.mark.parametrize("which", range(6))
def test_varlen_null_pointer(which):
    ptrs = [Q, K, V, O, L, CU]
    ptrs[which] = None
    assert call_varlen(*ptrs) == 1


@pytest.mark.parametrize("kw", [dict(H_kv=0), dict(H_kv=3), dict(H=2, H_kv=4), dict(B=0), dict(S=0), dict(D=96)])
def test_ex_bad_shape(kw):
    assert call_ex(**kw) == 2


@pytest.mark.parametrize("kw", [dict(nseq=0), dict(total=0), dict(max_seqlen=0), dict(H_kv=3), dict(D=32),
                                dict(H=0)])
def test_varlen_bad_shape(kw):
    assert call_varlen(**kw) == 2


@pytest.mark.parametrize("kw", [dict(wl=-2), dict(wr=-5), dict(p=-0.1), dict(p=1.0), dict(p=1.5),
                                dict(p=float("nan")), dict(p=float("inf"))])
def test_bad_window_or_dropout(kw):
    assert call_ex(**kw) == ARG
    assert call_varlen(**kw) == ARG


def test_ex_and_varlen_accept_valid_extras():
    # every call here also aliases o with q, the last check
    for kw in (dict(wl=0, wr=0), dict(wl=5, wr=-1), dict(wl=-1, wr=0), dict(p=0.0), dict(p=0.999, seed=2**64 - 1),
               dict(H=8, H_kv=1), dict(H=8, H_kv=8), dict(offset=2**32 - 1)):
        assert call_ex(o=Q, **kw) == ALIAS
        assert call_varlen(o=Q, **kw) == ALIAS


def test_varlen_alignment_and_alias():
    assert call_varlen(cu=CU + 2) == 4
    assert call_varlen(cu=CU + 4, o=Q) == ALIAS     # 4-byte alignment is enough
    assert call_varlen(cu=O + 64) == ALIAS          # the table inside o
    assert call_varlen(lse=CU) == ALIAS


def test_varlen_overflow():
    assert call_varlen(max_seqlen=1 << 29) == 5
    assert call_varlen(H=1 << 19, H_kv=1 << 19, D=64) == 5   # a K/V row stride too large for 32-bit lane offsets
    assert call_varlen(H=1 << 10, H_kv=1 << 10, D=128, o=Q) == ALIAS


def test_extended_error_order():
    # scale beats window/dropout beats alignment
    assert call_ex(scale=0.0, p=2.0, q=Q + 2) == 3
    assert call_ex(p=2.0, q=Q + 2) == ARG
    assert call_varlen(wl=-3, cu=CU + 1) == ARG
    assert call_ex(H_kv=3, p=2.0) == 2


def test_status_codes_follow_the_boundary_table():
    """The eight codes of the plain entry point keep their documented values;
    the two added for the extended entry points come after them."""
    assert fa2.STATUS_NAMES == {0: "FA2_OK", 1: "FA2_ERR_NULLPTR", 2: "FA2_ERR_SHAPE", 3: "FA2_ERR_SCALE",
                                4: "FA2_ERR_ALIGN", 5: "FA2_ERR_OVERFLOW", 6: "FA2_ERR_DEVICE",
                                7: "FA2_ERR_LAUNCH", 8: "FA2_ERR_ALIAS", 9: "FA2_ERR_ARG"}


def test_valid_arguments_without_a_gpu_report_device():
    """Arguments that pass every check reach the device check, which fails
    here (no HIP device): FA2_ERR_DEVICE, and nothing is launched."""
    assert call() == DEVICE
    assert call(D=128, causal=1) == DEVICE
    assert call_ex(wl=16, wr=0, p=0.25, seed=3) == DEVICE
    assert call_varlen() == DEVICE
    assert call_varlen(H=8, H_kv=2, D=64, wl=-1, wr=0) == DEVICE


def test_grid_bound_counts_half_height_workgroups():
    """Launches that pick the half-height (128-row) workgroups have twice the
    workgroups of the full-height shape; the grid limit is checked at that
    height. One packed sequence of one row with max_seqlen 2^29 - 1 and 127
    query heads per K/V head: 8 units x 2^22 tiles x 127 heads > 2^31 - 1."""
    assert call_varlen(nseq=1, total=1, max_seqlen=(1 << 29) - 1, H=127, H_kv=1, D=64, wl=-1, wr=0) == 5
    assert call_varlen(nseq=1, total=1, max_seqlen=(1 << 29) - 1, H=127, H_kv=1, D=64) == 5
    assert call_varlen(nseq=1, total=1, max_seqlen=(1 << 29) - 1, H=63, H_kv=1, D=64, wl=-1, wr=0, o=Q) == ALIAS
    # dense short causal sequences (half height): 3 * 2^25 heads of 4095 rows
    # are 3 * 2^29 workgroups at full height (below 2^31) but 3 * 2^30 at half
    assert call(B=3, H=1 << 25, S=4095, D=64, causal=1) == 5
    assert call(B=1, H=1 << 25, S=4095, D=64, causal=1, o=Q) == ALIAS


def test_kernel_config():
    cfg = fa2.fa2_kernel_config(4, 8, 4096, 64, 0)
    assert cfg["threads_per_block"] % 64 == 0
    assert cfg["blocks"] == 4 * 8 * -(-4096 // cfg["rows_per_block"])
    assert cfg["keys_per_tile"] % 32 == 0
    assert 0 < cfg["lds_bytes"] <= 160 * 1024
    cfg = fa2.fa2_kernel_config(16, 12, 1000, 64, 1)
    assert cfg["blocks"] == 16 * 12 * -(-1000 // cfg["rows_per_block"])
    with pytest.raises(fa2.FA2Error):
        fa2.fa2_kernel_config(1, 1, 128, 80, 0)


def test_kernel_config_shapes():
    """Causal grids that fit in one round of resident workgroups (2 per CU at
    D=64, 1 at D=128, 256 CUs), or whose sequences are short (S < 4096 at
    D=64, S <= 1024 at D=128), use half-height workgroups, and so do unmasked
    grids whose full-height grid is smaller than one round; other grids use the
    full height."""
    full64 = fa2.fa2_kernel_config(4, 8, 4096, 64, 0)
    assert (full64["rows_per_block"], full64["threads_per_block"], full64["blocks"]) == (256, 512, 512)
    half64 = fa2.fa2_kernel_config(4, 8, 4096, 64, 1)      # 512 full-height blocks: one round
    assert (half64["rows_per_block"], half64["threads_per_block"], half64["blocks"]) == (128, 256, 1024)
    assert half64["lds_bytes"] < full64["lds_bytes"]
    assert fa2.fa2_kernel_config(4, 8, 4100, 64, 1)["rows_per_block"] == 256   # 544 blocks: more than one round
    assert fa2.fa2_kernel_config(1, 32, 16384, 64, 1)["rows_per_block"] == 256
    assert fa2.fa2_kernel_config(1, 16, 4096, 128, 1)["rows_per_block"] == 128  # 256 blocks, 1 per CU
    assert fa2.fa2_kernel_config(2, 16, 8192, 128, 1)["rows_per_block"] == 256
    # short causal sequences: half height even when the grid needs several rounds
    short64 = fa2.fa2_kernel_config(16, 12, 1000, 64, 1)
    assert (short64["rows_per_block"], short64["blocks"]) == (128, 16 * 12 * 8)
    assert fa2.fa2_kernel_config(16, 12, 1000, 64, 0)["rows_per_block"] == 256   # non-causal: full height
    assert fa2.fa2_kernel_config(2, 32, 4095, 64, 1)["rows_per_block"] == 128
    assert fa2.fa2_kernel_config(2, 32, 4096, 64, 1)["rows_per_block"] == 256    # 1024 blocks, S not short
    assert fa2.fa2_kernel_config(8, 16, 1024, 128, 1)["rows_per_block"] == 128
    assert fa2.fa2_kernel_config(8, 16, 1025, 128, 1)["rows_per_block"] == 256
    # unmasked grids smaller than one round of full-height workgroups: half height
    assert fa2.fa2_kernel_config(1, 8, 4096, 64, 0)["rows_per_block"] == 128     # 128 < 512 full-height blocks
    assert fa2.fa2_kernel_config(3, 8, 4096, 64, 0)["rows_per_block"] == 128     # 384 < 512
    assert fa2.fa2_kernel_config(1, 8, 4096, 128, 0)["rows_per_block"] == 128    # 128 < 256
    assert fa2.fa2_kernel_config(1, 16, 4096, 128, 0)["rows_per_block"] == 256   # 256: one round


def test_forward_rejects_bad_tensors():
    import torch
    q = torch.zeros((1, 1, 8, 64), dtype=torch.float16)
    with pytest.raises(TypeError):
        fa2.forward(q.float(), q.float(), q.float())
    with pytest.raises(ValueError):
        fa2.forward(q, q[:, :, :4], q)
    with pytest.raises(ValueError):
        fa2.forward(q, q, q)  # CPU tensors: there is no CPU path
    with pytest.raises(ValueError):
        fa2.forward_ex(q, q, q, window=(2, 2))
    with pytest.raises(ValueError):
        fa2.forward_ex(q, q[:, :, :4], q[:, :, :4])
    p = torch.zeros((8, 1, 64), dtype=torch.float16)
    cu = torch.tensor([0, 8], dtype=torch.int32)
    with pytest.raises(ValueError):
        fa2.forward_varlen(p, p, p, cu)
    with pytest.raises(ValueError):
        fa2.forward_varlen(p, p, p, cu.long())


def test_inputs_on_different_devices_are_rejected():
    """The kernel reads every tensor from the device of q; stand-ins for GPU
    tensors on two devices (no second GPU is needed to check the host side)."""
    import types
    import torch

    def fake(dev):
        return types.SimpleNamespace(dtype=torch.float16, is_cuda=True, device=torch.device(dev),
                                     shape=(1, 1, 8, 64), is_contiguous=lambda: True)
    fa2._check_inputs(fake("cuda:0"), fake("cuda:0"), fake("cuda:0"))
    for k_dev, v_dev in (("cuda:1", "cuda:0"), ("cuda:0", "cuda:1")):
        with pytest.raises(ValueError, match="one device"):
            fa2._check_inputs(fake("cuda:0"), fake(k_dev), fake(v_dev))


def test_no_fallback_when_library_missing(tmp_path):
    with pytest.raises(ImportError):
        fa2.load_library(str(tmp_path / "libfa2.so"))
