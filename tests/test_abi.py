"""The C ABI on the host: exported symbols, argument checks, path choice.

Every check in attn_forward runs before any HIP call, so these calls use fake
(never dereferenced) addresses and need no GPU.
"""
import ctypes
import os
import re
import subprocess

import pytest

import exact_softmax_attention_bf16_amd as eab
from exact_softmax_attention_bf16_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

# These calls pass fake device addresses and rely on a host check refusing each
# one before any launch; where a GPU is visible a mistake in a test would send
# them to a kernel, so the module runs only on GPU-less hosts.
import torch  # noqa: E402
if torch.cuda.device_count() > 0:
    pytest.skip("host-side ABI checks with fake addresses run on GPU-less hosts",
                allow_module_level=True)

A = 0x7F0000000000          # fake, 16-byte aligned device addresses (never touched)
MB = 1 << 20


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(attn_[a-z_0-9]+)\s*\(", text, flags=re.M)))


def fwd(q=A, k=A + 64 * MB, v=A + 128 * MB, out=A + 192 * MB, B=1, H=1, L=16, d=64,
        scale=0.125, causal=0):
    return _lib.load().attn_forward(q, k, v, out, B, H, L, d, scale, causal, None)


def test_header_declares_the_boundary():
    names = declared_functions()
    assert names == sorted(["attn_forward", "attn_forward_ex", "attn_forward_varlen",
                            "attn_forward_noalloc",
                            "attn_status_string",
                            "attn_path_for_head_dim", "attn_workspace_bytes",
                            "attn_timing_enable", "attn_timing_collect"])
    assert set(names) == set(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True)
    exported = set(re.findall(r"\sT\s(attn_\w+)", out.stdout))
    assert set(declared_functions()) <= exported


def test_status_strings():
    for code in range(13):
        s = eab.status_string(code)
        assert s and s != "unknown status"
    assert eab.status_string(99) == "unknown status"


@pytest.mark.parametrize("d,path", [(32, 0), (64, 0), (128, 0), (192, 1), (256, 1), (320, 1),
                                    (1024, 1), (0, -1), (16, -1), (48, -1), (96, -1), (160, -1),
                                    (1088, -1), (2048, -1), (-64, -1)])
def test_path_for_head_dim(d, path):
    assert eab.path_for_head_dim(d) == path


def _values_narrow(n, L, d):
    """The values pass runs on 128 x 128 tiles when its 256 x 256 grid
    (n * T * ceil(d/256) workgroups) would fill at most half of 256 CUs and the
    narrow grid (n * ceil(L/128) * ceil(d/128)) fits on them in one round."""
    base = n * -(-L // 256) * -(-d // 256)
    return 2 * base <= 256 and n * -(-L // 128) * -(-d // 128) <= 256


def _values_split(n, L, d, causal):
    """Key splits of the values pass for n heads: 1 unless the unsplit grid
    would fill at most half of 256 CUs and the narrow tiles do not apply; then as
    many as fit in 256, at most 4, with at least 8 K steps (64 keys) per split in
    the query tile with the fewest; below 2, no split."""
    T = -(-L // 256)
    base = n * T * (-(-d // 256))
    if 2 * base > 256 or _values_narrow(n, L, d):
        return 1
    steps = -(-L // 64)
    fewest = min(4, steps) if causal else steps
    s = min(256 // base, 4, fewest // 8)
    return s if s >= 2 else 1


def test_values_tiles_choice():
    # one frame of 3432 x 1024: 56 wide tiles, 216 narrow ones -> narrow, no split
    assert _values_narrow(1, 3432, 1024) and _values_split(1, 3432, 1024, False) == 1
    # two frames: 112 wide tiles, 432 narrow ones -> wide, two splits
    assert not _values_narrow(2, 3432, 1024) and _values_split(2, 3432, 1024, False) == 2
    # 4096 x 1024: exactly 256 narrow tiles
    assert _values_narrow(1, 4096, 1024)
    assert not _values_narrow(1, 4097, 1024) and _values_split(1, 4097, 1024, False) == 3
    # 12 heads of 2048 x 256 (96 wide, 384 narrow) -> 2 splits; 10 of 1600 x 256 -> 3
    assert _values_split(12, 2048, 256, False) == 2 and _values_split(10, 1600, 256, False) == 3
    # enough heads: neither
    assert not _values_narrow(31, 3432, 1024) and _values_split(31, 3432, 1024, False) == 1


def test_workspace_bytes():
    # per head: E (1 KB blocks of 32 queries x 16 keys: ceil(L/32) x 16 T of them,
    # T = ceil(L/256)) and two fp32 [TK, L] tables (TK = ceil(L/128) score tiles of
    # 128 keys); plus split * n * L * d fp32 partial outputs when the values pass
    # splits the keys
    L, d, T, TK = 3432, 1024, 14, 27
    r = lambda x: (x + 255) // 256 * 256
    e_bytes = lambda n: ((n + 31) // 32) * 16 * ((n + 255) // 256) * 1024  # noqa: E731
    per_head = r(e_bytes(L)) + 2 * r(TK * L * 4)
    assert eab.workspace_bytes(1, 1, L, d) == per_head  # narrow tiles: no partials
    assert eab.workspace_bytes(2, 1, L, d) == 2 * per_head + r(2 * 2 * L * d * 4)
    assert eab.workspace_bytes(4, 1, L, d) == 4 * per_head
    assert eab.workspace_bytes(31, 1, L, d) == 31 * per_head
    # tiny: L = 286, d = 256
    Lt, dt = 286, 256
    pt = r(e_bytes(Lt)) + 2 * r(3 * Lt * 4)
    assert _values_split(1, Lt, dt, False) == 1
    assert eab.workspace_bytes(1, 1, Lt, dt) == pt
    assert eab.workspace_bytes(1, 1, 3432, 1024, True) == per_head
    # one head of L = 4097, d = 1024: 264 narrow tiles -> 3 splits of the 68 wide ones
    L4 = 4097
    T4, TK4 = 17, 33
    p4 = r(((L4 + 31) // 32) * 16 * T4 * 1024) + 2 * r(TK4 * L4 * 4)
    assert eab.workspace_bytes(1, 1, L4, 1024) == p4 + r(3 * L4 * 1024 * 4)
    # 12 heads of L = 2048, d = 256: 2 splits
    p12 = r(e_bytes(2048)) + 2 * r(16 * 2048 * 4)
    assert eab.workspace_bytes(12, 1, 2048, 256) == 12 * p12 + r(2 * 12 * 2048 * 256 * 4)
    assert eab.workspace_bytes(4, 8, 1024, 64) == 0       # online path, 256 workgroups: none
    assert eab.workspace_bytes(0, 1, L, d) == 0
    big = eab.workspace_bytes(1000, 1, L, d)              # chunked under ~2 GiB
    assert per_head <= big <= (2 << 30)


def test_valid_empty_problem_queues_nothing():
    assert fwd(q=None, k=None, v=None, out=None, L=0) == _lib.ATTN_OK
    assert fwd(B=0) == _lib.ATTN_OK
    assert fwd(H=0, d=1024) == _lib.ATTN_OK


@pytest.mark.parametrize("which", ["q", "k", "v", "out"])
def test_null_pointer(which):
    assert fwd(**{which: None}) == _lib.ATTN_ERR_NULL_PTR


@pytest.mark.parametrize("dims", [dict(B=-1), dict(H=-2), dict(L=-5), dict(d=-64),
                                  dict(B=1 << 40, H=1 << 20, L=1 << 10)])
def test_bad_shape(dims):
    assert fwd(**dims) == _lib.ATTN_ERR_BAD_SHAPE


@pytest.mark.parametrize("d", [0, 16, 48, 96, 100, 160, 1088, 2048])
def test_unsupported_head_dim(d):
    assert fwd(d=d) == _lib.ATTN_ERR_UNSUPPORTED_HEAD_DIM


@pytest.mark.parametrize("scale", [float("nan"), float("inf"), float("-inf")])
def test_bad_scale(scale):
    assert fwd(scale=scale) == _lib.ATTN_ERR_BAD_SCALE


@pytest.mark.parametrize("which", ["q", "k", "v", "out"])
def test_misaligned(which):
    base = {"q": A, "k": A + 64 * MB, "v": A + 128 * MB, "out": A + 192 * MB}[which]
    assert fwd(**{which: base + 8}) == _lib.ATTN_ERR_MISALIGNED


@pytest.mark.parametrize("which", ["q", "k", "v"])
def test_out_overlapping_an_input(which):
    base = {"q": A, "k": A + 64 * MB, "v": A + 128 * MB}[which]
    nbytes = 2 * 3 * 5 * 100 * 64 * 2
    assert fwd(out=base, B=2, H=3, L=500) == _lib.ATTN_ERR_ALIAS
    assert fwd(out=base + nbytes - 16, B=2, H=3, L=500) == _lib.ATTN_ERR_ALIAS


def test_adjacent_buffers_do_not_alias():
    # out starts exactly where q ends: allowed (checked, then it would launch, so
    # only the alias predicate is exercised through a too-large shape error path)
    L, d = 1 << 21, 1024  # one head of 4 GiB: rejected after the alias check
    nbytes = L * d * 2
    assert fwd(q=A, k=A + nbytes, v=A + 2 * nbytes, out=A + 3 * nbytes, L=L, d=d) == _lib.ATTN_ERR_TOO_LARGE


def test_too_large_two_pass_head():
    # E for one head would need more than 2^32 bytes of offsets
    L, d = 50000, 256
    n = L * d * 2
    assert fwd(q=A, k=A + n, v=A + 2 * n, out=A + 3 * n, L=L, d=d) == _lib.ATTN_ERR_TOO_LARGE


def test_two_pass_length_cap():
    # the values pass keeps a byte per (128-key tile, query) in LDS: L <= 124 * 128 when d > 128
    L, d = 124 * 128 + 1, 192
    n = L * d * 2
    assert fwd(q=A, k=A + n, v=A + 2 * n, out=A + 3 * n, L=L, d=d) == _lib.ATTN_ERR_TOO_LARGE


def test_check_order_is_documented():
    # shape before head dim before scale before emptiness before pointers
    assert fwd(B=-1, d=48) == _lib.ATTN_ERR_BAD_SHAPE
    assert fwd(d=48, scale=float("nan")) == _lib.ATTN_ERR_UNSUPPORTED_HEAD_DIM
    assert fwd(scale=float("nan"), q=None) == _lib.ATTN_ERR_BAD_SCALE
    assert fwd(q=None, out=A + 8) == _lib.ATTN_ERR_NULL_PTR
    assert fwd(out=A + 8, k=A) == _lib.ATTN_ERR_MISALIGNED


def test_timing_collect_without_records():
    lib = _lib.load()
    n = 4
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    assert lib.attn_timing_collect(ms, cnt, n) == _lib.ATTN_OK
    assert list(cnt) == [0] * n


def test_python_binding_rejects_bad_tensors():
    import torch
    from exact_softmax_attention_bf16_amd import attention
    x = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):          # CPU tensors never reach the library
        attention(x, x, x)
    with pytest.raises(TypeError):
        attention(x.float(), x, x)


# ---- attn_forward_ex: strides, grouped heads, log-sum-exp --------------------

def st(*x):
    return (ctypes.c_int64 * 3)(*x)


def fwd_ex(q=A, k=A + 64 * MB, v=A + 128 * MB, out=A + 192 * MB, lse=None, B=1, H=1, H_kv=1,
           L=16, d=64, qs=None, ks=None, vs=None, os_=None, scale=0.125, causal=0, wl=-1, wr=-1):
    return _lib.load().attn_forward_ex(q, k, v, out, lse, B, H, H_kv, L, d, qs, ks, vs, os_,
                                       scale, causal, wl, wr, None)


# A valid call would launch; these shapes pass every earlier check and are then
# refused as too large for the kernels' 32-bit offsets (q's row stride), which
# shows the layout itself was accepted.
BIG_L = 1 << 23


def test_ex_empty_and_shared_checks():
    assert fwd_ex(B=0) == _lib.ATTN_OK
    assert fwd_ex(L=0, q=None) == _lib.ATTN_OK
    assert fwd_ex(q=None) == _lib.ATTN_ERR_NULL_PTR
    assert fwd_ex(d=96) == _lib.ATTN_ERR_UNSUPPORTED_HEAD_DIM
    assert fwd_ex(scale=float("inf")) == _lib.ATTN_ERR_BAD_SCALE
    assert fwd_ex(out=A + 8) == _lib.ATTN_ERR_MISALIGNED


@pytest.mark.parametrize("H,H_kv", [(4, 0), (4, 3), (2, 4), (4, -1)])
def test_ex_key_value_heads_must_divide(H, H_kv):
    assert fwd_ex(H=H, H_kv=H_kv) == _lib.ATTN_ERR_BAD_SHAPE


@pytest.mark.parametrize("which", ["qs", "ks", "vs", "os_"])
@pytest.mark.parametrize("bad", [(4096, 1024, 60), (4096, 1028, 64), (-1024, 1024, 64),
                                 (1024, 1024, 32)])
def test_ex_bad_strides(which, bad):
    # a stride not a multiple of 8, a negative one, a row stride below d
    assert fwd_ex(**{which: st(*bad)}, d=64) == _lib.ATTN_ERR_BAD_STRIDE


def test_ex_out_elements_must_not_overlap():
    # two heads of out at the same address
    assert fwd_ex(H=2, H_kv=2, os_=st(2048, 0, 64)) == _lib.ATTN_ERR_BAD_STRIDE
    # rows 32 elements apart with d = 64
    assert fwd_ex(os_=st(4096, 4096, 32)) == _lib.ATTN_ERR_BAD_STRIDE


def test_ex_permuted_and_packed_layouts_are_accepted():
    L, d, H = BIG_L, 64, 2
    n = L * H * d * 2
    # out as [B, L, H, d] memory: head stride d, row stride H * d
    assert fwd_ex(q=A, k=A + n, v=A + 2 * n, out=A + 3 * n, B=1, H=H, H_kv=H, L=L, d=d,
                  qs=st(L * H * d, d, H * d), ks=st(L * H * d, d, H * d),
                  vs=st(L * H * d, d, H * d), os_=st(L * H * d, d, H * d)) == _lib.ATTN_ERR_TOO_LARGE
    # packed [T, 1, HW, 3C]: q, k, v overlap each other (they are only read)
    C = 64
    row = 3 * C
    span = 2 * BIG_L * row * 2
    ps = st(BIG_L * row, BIG_L * row, row)
    assert fwd_ex(q=A, k=A + 2 * C, v=A + 4 * C, out=A + span, B=2, H=1, H_kv=1, L=BIG_L, d=C,
                  qs=ps, ks=ps, vs=ps) == _lib.ATTN_ERR_TOO_LARGE


def test_ex_zero_strides_broadcast_inputs():
    # one key/value head broadcast over all batches and heads (strides 0)
    L, d = BIG_L, 64
    assert fwd_ex(q=A, k=A + (1 << 34), v=A + (1 << 35), out=A + (1 << 36), B=2, H=4, H_kv=4,
                  L=L, d=d, qs=st(4 * L * 2 * d, L * 2 * d, 2 * d), ks=st(0, 0, d),
                  vs=st(0, 0, d)) == _lib.ATTN_ERR_TOO_LARGE


def test_ex_out_must_not_overlap_a_strided_input():
    # out starts inside the span of a packed q (row stride 3d)
    L, d = 100, 64
    ps = st(L * 3 * d, L * 3 * d, 3 * d)
    assert fwd_ex(q=A, k=A + 2 * d, v=A + 4 * d, out=A + 2 * (L - 1) * 3 * d, L=L, d=d,
                  qs=ps, ks=ps, vs=ps) == _lib.ATTN_ERR_ALIAS


def test_ex_lse_checks():
    assert fwd_ex(lse=A + 256 * MB + 2) == _lib.ATTN_ERR_MISALIGNED
    assert fwd_ex(lse=A + 192 * MB + 64) == _lib.ATTN_ERR_ALIAS   # inside out
    assert fwd_ex(lse=A + 16) == _lib.ATTN_ERR_ALIAS              # inside q
    L = BIG_L
    n = L * 64 * 2
    assert fwd_ex(q=A, k=A + n, v=A + 2 * n, out=A + 3 * n, lse=A + 4 * n, L=L,
                  qs=st(L * 128, L * 128, 128)) == _lib.ATTN_ERR_TOO_LARGE


def test_ex_defaults_match_attn_forward_checks():
    # NULL strides and H_kv == H: the same verdicts as attn_forward
    for kw in [dict(B=-1), dict(d=48), dict(scale=float("nan")), dict(q=None), dict(out=A + 8)]:
        assert fwd_ex(**kw) == fwd(**kw)
    nbytes = 2 * 3 * 500 * 64 * 2
    assert fwd_ex(out=A + nbytes - 16, B=2, H=3, H_kv=3, L=500) == _lib.ATTN_ERR_ALIAS


def test_python_binding_rejects_bad_layouts():
    import torch
    from exact_softmax_attention_bf16_amd import attention, attention_packed_qkv
    x = torch.zeros(1, 2, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):   # CPU tensors never reach the library
        attention(x, x[:, :1], x[:, :1])
    with pytest.raises(ValueError):
        attention_packed_qkv(torch.zeros(1, 1, 4, 100, dtype=torch.bfloat16))


@pytest.mark.parametrize("wl,wr", [(-2, 0), (0, -2), (-5, -5)])
def test_ex_bad_window(wl, wr):
    assert fwd_ex(wl=wl, wr=wr) == _lib.ATTN_ERR_BAD_SHAPE


def test_ex_window_is_accepted():
    L = BIG_L
    n = L * 64 * 2
    for wl, wr in [(0, 0), (5, -1), (-1, 7), (L + 5, L + 5)]:
        assert fwd_ex(q=A, k=A + n, v=A + 2 * n, out=A + 3 * n, L=L, wl=wl, wr=wr,
                      qs=st(L * 128, L * 128, 128)) == _lib.ATTN_ERR_TOO_LARGE


# ---- attn_forward_varlen: token-packed sequences of different lengths ----------

def st2(*x):
    return (ctypes.c_int64 * 2)(*x)


def fwd_var(q=A, k=A + 64 * MB, v=A + 128 * MB, out=A + 192 * MB, lse=None, cu=A + 256 * MB,
            B=2, max_seqlen=16, total=32, H=1, H_kv=1, d=64, qs=None, ks=None, vs=None, os_=None,
            scale=0.125, causal=0, wl=-1, wr=-1, cuk=None, max_k=0, total_k=0):
    return _lib.load().attn_forward_varlen(q, k, v, out, lse, cu, B, max_seqlen, total, cuk, max_k,
                                           total_k, H, H_kv, d, qs, ks, vs, os_, scale, causal, wl,
                                           wr, None)


def test_varlen_nothing_to_do():
    for kw in [dict(B=0), dict(total=0), dict(max_seqlen=0), dict(H=0, H_kv=0)]:
        assert fwd_var(cu=None, **kw) == _lib.ATTN_OK


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), "BAD_SHAPE"), (dict(max_seqlen=-1), "BAD_SHAPE"), (dict(total=-3), "BAD_SHAPE"),
    (dict(H=4, H_kv=3), "BAD_SHAPE"), (dict(wl=-2), "BAD_SHAPE"),
    (dict(d=256), "UNSUPPORTED_HEAD_DIM"), (dict(d=48), "UNSUPPORTED_HEAD_DIM"),
    (dict(scale=float("nan")), "BAD_SCALE"), (dict(cu=None), "NULL_PTR"), (dict(q=None), "NULL_PTR"),
    (dict(qs=st2(60, 64)), "BAD_STRIDE"), (dict(ks=st2(32, 64)), "BAD_STRIDE"),
    (dict(H=2, H_kv=2, os_=st2(64, 0)), "BAD_STRIDE"),
    (dict(cu=A + 256 * MB + 2), "MISALIGNED"), (dict(lse=A + 300 * MB + 1), "MISALIGNED"),
    (dict(out=A + 8), "MISALIGNED"),
    (dict(cu=A + 192 * MB + 64), "ALIAS"), (dict(lse=A + 192 * MB), "ALIAS"),
    (dict(out=A + 64), "ALIAS"),
    (dict(causal=2, wl=5), "BAD_MASK"), (dict(causal=2, wr=0), "BAD_MASK"),
    (dict(causal=2, wl=0, wr=7, B=-1), "BAD_SHAPE"),
])
def test_varlen_checks(kw, code):
    assert fwd_var(**kw) == getattr(_lib, "ATTN_ERR_" + code)


def test_varlen_layouts_are_accepted():
    # [total, H, d] packed, and q/k/v inside one [total, 3, H, d] tensor; a row
    # stride too wide for 32-bit offsets shows every earlier check passed
    big, T = 1 << 22, 1 << 40
    assert fwd_var(q=A, k=A + T, v=A + 2 * T, out=A + 3 * T, cu=A + 4 * T, total=1024,
                   max_seqlen=1024, H=2, H_kv=2, qs=st2(big, 64), ks=st2(big, 64),
                   vs=st2(big, 64)) == _lib.ATTN_ERR_TOO_LARGE
    H, d = 2, 64
    row = 3 * H * d
    span = 1024 * row * 2
    assert fwd_var(q=A, k=A + H * d * 2, v=A + 2 * H * d * 2, out=A + span, cu=A + 2 * span,
                   total=1024, max_seqlen=1 << 22, H=H, H_kv=H, qs=st2(row, d), ks=st2(row, d),
                   vs=st2(row, d)) == _lib.ATTN_ERR_TOO_LARGE


def _online_split(n, L):
    """Key splits of the online kernel for n heads: 1 unless the unsplit grid
    (n * ceil(L/128) workgroups) would fill at most half of 256 CUs; then as many
    as fit in 256, at most 8, each share keeping >= 2 key blocks (64 keys) per
    group (two groups); below 2, no split."""
    base = n * -(-L // 128)
    if 2 * base > 256:
        return 1
    s = min(256 // base, 8, -(-L // 64) // 4)
    return s if s >= 2 else 1


@pytest.mark.parametrize("B,H,L,d,split", [(1, 1, 4096, 64, 8), (1, 2, 1000, 128, 4),
                                           (1, 1, 300, 32, 1), (4, 8, 1024, 64, 1),
                                           (2, 4, 1024, 64, 4), (1, 1, 128, 64, 1)])
def test_online_split_workspace(B, H, L, d, split):
    # split shares: fp32 O [split, heads, L, d] and (m, l) [split, heads, L, 2]
    assert _online_split(B * H, L) == split
    r = lambda x: (x + 255) // 256 * 256
    want = r(split * B * H * L * (d + 2) * 4) if split > 1 else 0
    assert eab.workspace_bytes(B, H, L, d) == want
    assert eab.workspace_bytes(B, H, L, d, True) == want


@pytest.mark.parametrize("kw,code", [
    (dict(cuk=A + 300 * MB, max_k=-1, total_k=10), "BAD_SHAPE"),
    (dict(cuk=A + 300 * MB, max_k=10, total_k=-1), "BAD_SHAPE"),
    (dict(cuk=A + 300 * MB + 2, max_k=10, total_k=10), "MISALIGNED"),
    (dict(cuk=A + 192 * MB + 16, max_k=10, total_k=10), "ALIAS"),
])
def test_varlen_key_offsets_checks(kw, code):
    assert fwd_var(**kw) == getattr(_lib, "ATTN_ERR_" + code)


def test_varlen_key_offsets_layout_accepted():
    # q: 8 tokens, keys: a long cache with a row stride too wide for 32-bit offsets
    T = 1 << 40
    assert fwd_var(q=A, k=A + T, v=A + 2 * T, out=A + 3 * T, cu=A + 4 * T, cuk=A + 5 * T,
                   B=1, max_seqlen=8, total=8, max_k=1 << 22, total_k=1 << 22,
                   ks=st2(1024, 64), vs=st2(1024, 64)) == _lib.ATTN_ERR_TOO_LARGE


def test_varlen_compressed_causal_is_accepted():
    # every check passes; a row stride too wide for 32-bit offsets shows it
    T = 1 << 40
    assert fwd_var(q=A, k=A + T, v=A + 2 * T, out=A + 3 * T, cu=A + 4 * T, cuk=A + 5 * T,
                   causal=_lib.ATTN_MASK_COMPRESSED_CAUSAL, B=1, max_seqlen=8, total=8,
                   max_k=1 << 22, total_k=1 << 22, ks=st2(1024, 64),
                   vs=st2(1024, 64)) == _lib.ATTN_ERR_TOO_LARGE


def test_python_varlen_rejects_unknown_mask_names():
    import torch
    t = torch.zeros(4, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="compressed"):
        eab.attention_varlen(t, t, t, torch.zeros(2, dtype=torch.int32), 4, causal="sliding")


def test_varlen_without_key_tokens_takes_null_keys():
    # total_k == 0: k and v are never read, NULL is accepted (the too-wide q row
    # stride shows every earlier check passed); with keys, NULL k is an error
    T = 1 << 40
    kw = dict(q=A, out=A + 3 * T, cu=A + 4 * T, cuk=A + 5 * T, B=1, max_seqlen=8, total=8,
              max_k=0, total_k=0, qs=st2(1 << 22, 64))
    assert fwd_var(k=None, v=None, **kw) == _lib.ATTN_ERR_TOO_LARGE
    kw.update(max_k=4, total_k=4)
    assert fwd_var(k=None, v=A + T, **kw) == _lib.ATTN_ERR_NULL_PTR


# ---- attn_forward_noalloc: the same checks as attn_forward, plus its scratch limit

def fwd_noalloc(q=A, k=A + 64 * MB, v=A + 128 * MB, out=A + 192 * MB, B=1, H=1, L=16, d=64,
                scale=0.125, causal=0):
    return _lib.load().attn_forward_noalloc(q, k, v, out, B, H, L, d, scale, causal, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), _lib.ATTN_ERR_NULL_PTR), (dict(B=-1), _lib.ATTN_ERR_BAD_SHAPE),
    (dict(d=96), _lib.ATTN_ERR_UNSUPPORTED_HEAD_DIM), (dict(scale=float("nan")), _lib.ATTN_ERR_BAD_SCALE),
    (dict(k=A + 8), _lib.ATTN_ERR_MISALIGNED), (dict(out=A), _lib.ATTN_ERR_ALIAS),
    (dict(B=0), _lib.ATTN_OK), (dict(L=0), _lib.ATTN_OK)])
def test_noalloc_shares_the_checks_of_attn_forward(kw, code):
    assert fwd_noalloc(**kw) == code
    assert fwd(**kw) == code


def _two_pass_head_bytes(L):
    """E (ceil(L/32) x 16 ceil(L/256) blocks of 1 KB) and two fp32 [ceil(L/128), L] tables."""
    r = lambda x: (x + 255) // 256 * 256  # noqa: E731
    T, TK, QB = (L + 255) // 256, (L + 127) // 128, (L + 31) // 32
    return r(QB * 16 * T * 1024) + 2 * r(4 * TK * L)


@pytest.mark.parametrize("L", [7937, 8000, 15000])
def test_noalloc_rejects_a_head_beyond_its_scratch(L):
    """d > 128: one head's staging must fit ATTN_NOALLOC_SCRATCH_BYTES; the call is
    refused before any HIP call."""
    assert _two_pass_head_bytes(L) > _lib.ATTN_NOALLOC_SCRATCH_BYTES
    big = 4 * L * 1024 * 2
    assert fwd_noalloc(q=A, k=A + big, v=A + 2 * big, out=A + 3 * big, L=L, d=1024) == \
        _lib.ATTN_ERR_SCRATCH_TOO_SMALL


def test_noalloc_largest_head_fits():
    """L = 7936 is the longest head at d > 128 whose staging fits the array."""
    assert _two_pass_head_bytes(7936) <= _lib.ATTN_NOALLOC_SCRATCH_BYTES


def test_noalloc_python_binding_needs_out():
    import torch
    with pytest.raises(TypeError):
        eab.attention_noalloc(torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16),
                              torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16),
                              torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16))


PROBE_HEADER = os.path.join(ROOT, "include", "attn_probe.h")
PROBE_LIB = os.path.join(ROOT, "exact_softmax_attention_bf16_amd", "libattn_probe.so")


def test_probe_library_exports_its_header_and_checks_arguments():
    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    names = set(re.findall(r"^\s*int\s+(attn_probe_[a-z_0-9]+)\s*\(", text, flags=re.M))
    assert names == {"attn_probe_split_columns"}
    out = subprocess.run(["nm", "-D", "--defined-only", PROBE_LIB], capture_output=True, text=True)
    assert names <= set(re.findall(r"\sT\s(attn_probe_\w+)", out.stdout))
    f = ctypes.CDLL(PROBE_LIB).attn_probe_split_columns
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64] * 4 + [ctypes.c_float, ctypes.c_void_p]
    assert f(None, A, A, A, 1, 1, 64, 1024, 0.03125, None) == 1
    assert f(A, A + 64 * MB, A + 128 * MB, A + 192 * MB, 1, 1, 64, 512, 0.03125, None) == 2
    assert f(A, A + 64 * MB, A + 128 * MB, A + 192 * MB, 1, 1, 0, 1024, 0.03125, None) == 2
    assert f(A, A + 64 * MB, A + 128 * MB, A + 192 * MB, 1, 1, 1 << 20, 1024, 0.03125, None) == 2
